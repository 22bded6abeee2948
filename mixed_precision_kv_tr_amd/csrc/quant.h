// Eq. (4) of the TriRoute review page (xllm-io.github.io): one token's K or V vector of one
// head quantized asymmetrically at its width b, shared by every kernel that writes the cache.
//
// A group is the D bf16 values of one (token, head, K or V); D/8 consecutive lanes hold it, 8
// values each (one 128-bit load).  In binary32, in this order: mx, mn exact; z = mn + 0 (no
// -0); R = fl(mx - mn); s = fl(R / (2^b - 1)) + 0 with a correctly rounded divide;
// code = rint(fl(fl(x - z) / s)), 0 for every value when s = 0.  b = 16 stores the bf16 input.
#pragma once

#include "common.h"

struct QPiece {
  uint4 raw;                  // this lane's 8 input values (bf16 bits)
  int cls;                    // width class; 3 = native bf16
  float s, z;                 // scale and zero point ((1, 0) for native storage)
  uint32_t code[8];           // codes (b < 16)
};

// Loads and quantizes this lane's piece.  Every lane of the group must call it (the min/max are
// reduced across the group's lanes); lanes with live = false contribute nothing.
template <int D>
__device__ __forceinline__ void eq4_piece(QPiece& qp, const uint16_t* src, int part, bool live, int bval) {
#pragma clang fp contract(off)
  constexpr int LPG = D / 8;
  qp.raw = live ? *reinterpret_cast<const uint4*>(src + part * 8) : make_uint4(0, 0, 0, 0);
  float x[8];
  x[0] = tr_bf16_lo(qp.raw.x); x[1] = tr_bf16_hi(qp.raw.x);
  x[2] = tr_bf16_lo(qp.raw.y); x[3] = tr_bf16_hi(qp.raw.y);
  x[4] = tr_bf16_lo(qp.raw.z); x[5] = tr_bf16_hi(qp.raw.z);
  x[6] = tr_bf16_lo(qp.raw.w); x[7] = tr_bf16_hi(qp.raw.w);
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) { mn = fminf(mn, x[e]); mx = fmaxf(mx, x[e]); }
#pragma unroll
  for (int off = 1; off < LPG; off <<= 1) {
    mn = fminf(mn, __shfl_xor(mn, off, 64));
    mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  }
  int cls = tr_class_of_bits(bval);
  if (cls < 0) cls = 3;                                // flagged by the slot assignment
  qp.cls = cls;
  if (cls == 3) {
    qp.s = 1.0f;
    qp.z = 0.0f;
    return;
  }
  const int b = 2 << cls;
  const float nlev = (float)((1 << b) - 1);
  const float z = mn + 0.0f;                           // -0 -> +0
  const float R = mx - mn;
  const float sc = R / nlev + 0.0f;                    // correctly rounded divide; -0 -> +0
  qp.s = sc;
  qp.z = z;
  if (sc == 0.0f) {
#pragma unroll
    for (int e = 0; e < 8; ++e) qp.code[e] = 0;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = x[e] - z;
      const float r = d / sc;
      float cf = rintf(r);
      cf = fminf(fmaxf(cf, 0.0f), nlev);
      qp.code[e] = (uint32_t)cf;
    }
  }
}

// Stores this lane's piece into its slot: position p of sequence s, head h, kv = 0 for K and 1 for
// V.  The slot assignment must have run (prefix counts and page tables of position p).
__device__ __forceinline__ void store_piece(const CacheLayout& c, int layer, int s, int p, int h, int kv, int part,
                                            const QPiece& qp) {
  const int cls = qp.cls;
  const int32_t slot = tr_prefix_row(c, layer, s, p)[cls];
  const int P = c.ptok[cls];
  const int32_t page = tr_ptab(c, layer, s, cls)[slot / P];
  if (page < 0) return;                                // pool exhausted (flagged)
  const int j = slot % P;
  uint8_t* base = c.pool + (int64_t)page * c.page_bytes;
  uint8_t* row = base + (kv ? c.v_off[cls] : c.k_off[cls]) + (int64_t)h * c.cb + (int64_t)j * c.rowb[cls];
  if (h == 0 && kv == 0 && part == 0) reinterpret_cast<int32_t*>(base)[j] = p;
  if (cls == 3) {                                      // b = 16: native bf16 storage
    reinterpret_cast<uint4*>(row)[part] = qp.raw;
    return;
  }
  if (part == 0) {
    float2* side = reinterpret_cast<float2*>(base + (kv ? c.sv_off[cls] : c.sk_off[cls]));
    side[(int64_t)h * P + j] = make_float2(qp.s, qp.z);
  }
  if (cls == 0) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) w |= qp.code[e] << (2 * e);
    reinterpret_cast<uint16_t*>(row)[part] = (uint16_t)w;
  } else if (cls == 1) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) w |= qp.code[e] << (4 * e);
    reinterpret_cast<uint32_t*>(row)[part] = w;
  } else {
    uint2 w;
    w.x = qp.code[0] | (qp.code[1] << 8) | (qp.code[2] << 16) | (qp.code[3] << 24);
    w.y = qp.code[4] | (qp.code[5] << 8) | (qp.code[6] << 16) | (qp.code[7] << 24);
    reinterpret_cast<uint2*>(row)[part] = w;
  }
}
