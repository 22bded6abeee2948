// The write path of the mixed-width cache (TriRoute review page, xllm-io.github.io: Eq. (4) and
// the inference paragraph after Algorithm 1), shared by every kernel that writes the cache:
// slot assignment of new positions, and the quantization and store of one group.
//
// Slot assignment (one workgroup of TR_ASSIGN_THREADS per sequence): a block-wide scan of the
// new positions' width classes gives the prefix counts (slot of each position in its class
// stream); the pages for the new slots come from the shared pool (one atomic per (sequence,
// class) that needs pages), pages kept from before a truncation being reused first.
//
// Eq. (4): one token's K or V vector of one head quantized asymmetrically at its width b.
// A group is the D bf16 values of one (token, head, K or V); D/8 consecutive lanes hold it, 8
// values each (one 128-bit load).  In binary32, in this order: mx, mn exact; z = mn + 0 (no
// -0); R = fl(mx - mn); s = fl(R / (2^b - 1)) + 0 with a correctly rounded divide;
// code = rint(fl(fl(x - z) / s)), 0 for every value when s = 0.  b = 16 stores the bf16 input.
#pragma once

#include "common.h"

#define TR_ASSIGN_THREADS 1024

// Slots and pages of positions [p0, p0 + n) of sequence s; blockDim.x must be TR_ASSIGN_THREADS.
// Classes are counted in two 32-bit words of 16-bit fields (classes 0|1 and 2|3); a chunk of
// TR_ASSIGN_THREADS positions adds at most that many to a field.
__device__ __forceinline__ void tr_assign_slots_seq(const CacheLayout& c, int layer, int p0, int n,
                                                    const uint8_t* __restrict__ bits, int s) {
  constexpr int NW = TR_ASSIGN_THREADS / 64;
  __shared__ uint32_t wsum[2][NW];
  __shared__ int32_t base[TR_NCLASS];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int32_t* pre0 = tr_prefix_row(c, layer, s, p0);
  if (tid < TR_NCLASS) base[tid] = pre0[tid];
  __syncthreads();
  int32_t n0[TR_NCLASS];
#pragma unroll
  for (int k = 0; k < TR_NCLASS; ++k) n0[k] = base[k];

  for (int chunk = 0; chunk < n; chunk += TR_ASSIGN_THREADS) {
    const int i = chunk + tid;
    uint32_t a = 0, b = 0;
    if (i < n) {
      int cls = tr_class_of_bits(bits[(int64_t)s * n + i]);
      if (cls < 0) {
        atomicOr(c.err, TR_ERRF_BAD_BITS);
        cls = 3;                                     // stored as native; output unspecified
      }
      if (cls == 0) a = 1u; else if (cls == 1) a = 1u << 16; else if (cls == 2) b = 1u; else b = 1u << 16;
    }
    uint32_t ia = tr_wave_incl_scan(a), ib = tr_wave_incl_scan(b);
    if (lane == 63) { wsum[0][wave] = ia; wsum[1][wave] = ib; }
    __syncthreads();
    uint32_t pa = 0, pb = 0, ta = 0, tb = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t xa = wsum[0][w], xb = wsum[1][w];
      if (w < wave) { pa += xa; pb += xb; }
      ta += xa; tb += xb;
    }
    ia += pa; ib += pb;
    if (i < n) {
      int32_t* row = const_cast<int32_t*>(tr_prefix_row(c, layer, s, p0 + i + 1));
      int4 v;
      v.x = base[0] + (int)(ia & 0xffffu);
      v.y = base[1] + (int)(ia >> 16);
      v.z = base[2] + (int)(ib & 0xffffu);
      v.w = base[3] + (int)(ib >> 16);
      *reinterpret_cast<int4*>(row) = v;
    }
    __syncthreads();
    if (tid == 0) {
      base[0] += (int)(ta & 0xffffu); base[1] += (int)(ta >> 16);
      base[2] += (int)(tb & 0xffffu); base[3] += (int)(tb >> 16);
    }
    __syncthreads();
  }
  // Pages for the slots [n0, n1) of class k = wave k.  Entries of the page table that are still
  // set (pages kept from before a truncation) are reused up to the first empty one; the rest
  // take new pages from the pool.
  if (wave < TR_NCLASS) {
    const int k = wave;
    const int P = c.ptok[k];
    const int first = (n0[k] + P - 1) / P, last = (base[k] + P - 1) / P;
    int32_t* pt = tr_ptab(c, layer, s, k);
    int reuse = last;
    for (int j0 = first; j0 < last; j0 += 64) {
      const int j = j0 + lane;
      const uint64_t empty = __ballot(j < last && pt[j] < 0);
      if (empty) {
        reuse = j0 + __ffsll((unsigned long long)empty) - 1;
        break;
      }
    }
    const int need = last - reuse;
    if (need > 0) {
      int id0 = 0;
      if (lane == 0) id0 = atomicAdd(c.next_page, need);
      id0 = __shfl(id0, 0, 64);
      const bool ok = (int64_t)id0 + need <= c.pool_pages;
      if (!ok && lane == 0) atomicOr(c.err, TR_ERRF_NO_PAGES);
      for (int j = lane; j < need; j += 64) pt[reuse + j] = ok ? id0 + j : -1;
    }
  }
}

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

// Stores this lane's piece into row j of a class page (base): head h, kv = 0 for K and 1 for V.
__device__ __forceinline__ void put_piece(const CacheLayout& c, uint8_t* base, int j, int h, int kv, int part,
                                          const QPiece& qp) {
  const int cls = qp.cls;
  uint8_t* row = base + (kv ? c.v_off[cls] : c.k_off[cls]) + (int64_t)h * c.cb + (int64_t)j * c.rowb[cls];
  if (cls == 3) {                                      // b = 16: native bf16 storage
    reinterpret_cast<uint4*>(row)[part] = qp.raw;
    return;
  }
  if (part == 0) {
    float2* side = reinterpret_cast<float2*>(base + (kv ? c.sv_off[cls] : c.sk_off[cls]));
    side[(int64_t)h * c.ptok[cls] + j] = make_float2(qp.s, qp.z);
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

// Page of slot `slot` of class cls (nullptr when the pool was exhausted, which is flagged) and the
// row within it.
__device__ __forceinline__ uint8_t* slot_page(const CacheLayout& c, int layer, int s, int cls, int32_t slot, int& j) {
  const int32_t page = tr_ptab(c, layer, s, cls)[slot >> c.ptok_log2[cls]];
  j = slot & (c.ptok[cls] - 1);
  return page < 0 ? nullptr : c.pool + (int64_t)page * c.page_bytes;
}

// Stores this lane's piece into its slot: position p of sequence s, head h, kv = 0 for K and 1 for
// V.  The slot assignment must have run (prefix counts and page tables of position p).
__device__ __forceinline__ void store_piece(const CacheLayout& c, int layer, int s, int p, int h, int kv, int part,
                                            const QPiece& qp) {
  int j;
  uint8_t* base = slot_page(c, layer, s, qp.cls, tr_prefix_row(c, layer, s, p)[qp.cls], j);
  if (!base) return;
  if (h == 0 && kv == 0 && part == 0) reinterpret_cast<int32_t*>(base)[j] = p;
  put_piece(c, base, j, h, kv, part, qp);
}

// Both pieces of position p, head h (K and V share the width class and so the slot), given the
// position's prefix-count row.
__device__ __forceinline__ void store_pair(const CacheLayout& c, int layer, int s, int p, int h, int part,
                                           const QPiece& qk, const QPiece& qv, int4 prefix) {
  const int cls = qk.cls;
  const int32_t slot = cls == 0 ? prefix.x : cls == 1 ? prefix.y : cls == 2 ? prefix.z : prefix.w;
  int j;
  uint8_t* base = slot_page(c, layer, s, cls, slot, j);
  if (!base) return;
  if (h == 0 && part == 0) reinterpret_cast<int32_t*>(base)[j] = p;
  put_piece(c, base, j, h, 0, part, qk);
  put_piece(c, base, j, h, 1, part, qv);
}
