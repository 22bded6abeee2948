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
// A group is the D bf16 values of one (token, head, K or V); D/NV consecutive lanes hold it, NV
// values each (8 or 16: one or two 128-bit loads).  In binary32, in this order: mx, mn exact; z = mn + 0 (no
// -0); R = fl(mx - mn); s = fl(R / (2^b - 1)) + 0 with a correctly rounded divide;
// code = rint(fl(fl(x - z) / s)), 0 for every value when s = 0.  b = 16 stores the bf16 input.
#pragma once

#include "common.h"

#define TR_ASSIGN_THREADS 1024

// Slots and pages of positions [p0, p0 + n) of sequence s; blockDim.x must be TR_ASSIGN_THREADS.
// Thread t takes the contiguous positions [t R, t R + R): it counts their classes, one block-wide
// scan of the four counts gives its slots, and a second pass writes the prefix rows.  The bits
// are loaded 4 positions at a time (addresses clamped into the row, so the loads go out
// together) and, for R <= 16, kept as 2-bit classes for the second pass.
__device__ __forceinline__ void tr_assign_slots_seq(const CacheLayout& c, int layer, int p0, int n,
                                                    const uint8_t* __restrict__ bits, int s) {
  constexpr int NT = TR_ASSIGN_THREADS;
  constexpr int NW = NT / 64;
  __shared__ int32_t wsum[TR_NCLASS][NW];
  __shared__ int32_t base[TR_NCLASS];
  if (n <= 0) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int32_t* pre0 = tr_prefix_row(c, layer, s, p0);
  const uint8_t* brow = bits + (int64_t)s * n;
  const int R = (n + NT - 1) / NT;
  const int i0 = min(n, tid * R), i1 = min(n, i0 + R);
  bool bad = false;
  auto load4 = [&](int r0, int (&k)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + r0 + u;
      const int cl = tr_class_of_bits(brow[min(i, n - 1)]);
      bad |= i < i1 && cl < 0;
      k[u] = cl < 0 ? 3 : cl;                        // stored as native; output unspecified
    }
  };
  const bool cached = R <= 16;
  uint32_t cp = 0;
  int cnt[TR_NCLASS] = {0, 0, 0, 0};
  for (int r0 = 0; r0 < R; r0 += 4) {
    int k[4];
    load4(r0, k);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (i0 + r0 + u >= i1) break;
#pragma unroll
      for (int x = 0; x < TR_NCLASS; ++x) cnt[x] += k[u] == x;
      if (cached) cp |= (uint32_t)k[u] << (2 * (r0 + u));
    }
  }
  if (bad) atomicOr(c.err, TR_ERRF_BAD_BITS);
  int excl[TR_NCLASS];
#pragma unroll
  for (int x = 0; x < TR_NCLASS; ++x) {
    const int incl = (int)tr_wave_incl_scan((uint32_t)cnt[x]);
    excl[x] = incl - cnt[x];
    if (lane == 63) wsum[x][wave] = incl;
  }
  if (tid < TR_NCLASS) base[tid] = pre0[tid];
  __syncthreads();
  int32_t n0[TR_NCLASS], run[TR_NCLASS], tot[TR_NCLASS];
#pragma unroll
  for (int x = 0; x < TR_NCLASS; ++x) {
    n0[x] = base[x];
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int v = wsum[x][w];
      before += w < wave ? v : 0;
      all += v;
    }
    run[x] = n0[x] + before + excl[x];
    tot[x] = n0[x] + all;
  }
  // prefix row of position p0 + i + 1 = slots used up to and including position p0 + i
  for (int r0 = 0; r0 < R; r0 += 4) {
    int k[4];
    if (cached) {
#pragma unroll
      for (int u = 0; u < 4; ++u) k[u] = (int)((cp >> (2 * (r0 + u))) & 3u);
    } else {
      load4(r0, k);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + r0 + u;
      if (i >= i1) break;
#pragma unroll
      for (int x = 0; x < TR_NCLASS; ++x) run[x] += k[u] == x;
      *reinterpret_cast<int4*>(const_cast<int32_t*>(tr_prefix_row(c, layer, s, p0 + i + 1))) =
          make_int4(run[0], run[1], run[2], run[3]);
    }
  }
  // Pages for the slots [n0, n1) of class k = wave k.  Entries of the page table that are still
  // set (pages kept from before a truncation) are reused up to the first empty one; the rest
  // take new pages from the pool.
  if (wave < TR_NCLASS) {
    const int k = wave;
    const int P = c.ptok[k];
    const int n0k = k == 0 ? n0[0] : k == 1 ? n0[1] : k == 2 ? n0[2] : n0[3];
    const int n1k = k == 0 ? tot[0] : k == 1 ? tot[1] : k == 2 ? tot[2] : tot[3];
    const int first = (n0k + P - 1) / P, last = (n1k + P - 1) / P;
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

// Value of lane (lane ^ 1), (lane ^ 2), or of the mirrored lane within 8 / 16 lanes (DPP, no
// LDS traffic).  After the two quad steps every lane holds its quad's result, and the mirror
// within 8 (16) lanes pairs it with the other quad (half-row), so a min / max over a group of 4,
// 8 or 16 lanes takes 2, 3 or 4 steps.
template <int CTRL>
__device__ __forceinline__ float tr_dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// min / max that do not quiet NaNs first (v_minimum / v_maximum): the same result as fminf /
// fmaxf for the finite values the cache stores, without a canonicalizing op per input.
__device__ __forceinline__ float tr_min(float a, float b) { return __builtin_elementwise_minimum(a, b); }
__device__ __forceinline__ float tr_max(float a, float b) { return __builtin_elementwise_maximum(a, b); }
template <int LPG>
__device__ __forceinline__ void tr_group_minmax(float& mn, float& mx) {
  static_assert(LPG == 4 || LPG == 8 || LPG == 16, "groups of 4, 8 or 16 lanes");
  mn = tr_min(mn, tr_dpp<0xB1>(mn)); mx = tr_max(mx, tr_dpp<0xB1>(mx));     // quad_perm 1,0,3,2
  mn = tr_min(mn, tr_dpp<0x4E>(mn)); mx = tr_max(mx, tr_dpp<0x4E>(mx));     // quad_perm 2,3,0,1
  if constexpr (LPG >= 8) {
    mn = tr_min(mn, tr_dpp<0x141>(mn)); mx = tr_max(mx, tr_dpp<0x141>(mx)); // row_half_mirror
  }
  if constexpr (LPG == 16) {
    mn = tr_min(mn, tr_dpp<0x140>(mn)); mx = tr_max(mx, tr_dpp<0x140>(mx)); // row_mirror
  }
}

// One of four per-class layout values for a lane's own class.  The values are pinned in
// registers first: a select between loads of the kernel-argument array would otherwise become
// one load with a lane-dependent index, a memory round trip on the store path.
__device__ __forceinline__ int tr_sel4(int cls, const int32_t (&a)[TR_NCLASS]) {
  int a0 = a[0], a1 = a[1], a2 = a[2], a3 = a[3];
  asm volatile("" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3));
  const int lo = (cls & 1) ? a1 : a0, hi = (cls & 1) ? a3 : a2;   // bit tests: selects, not a branch tree
  return (cls & 2) ? hi : lo;
}

// Width class of a position (a bits value outside {2, 4, 8, 16} is flagged by the slot
// assignment and stored natively).
__device__ __forceinline__ int eq4_class(int bval) {
  const int c = tr_class_of_bits(bval);
  return c < 0 ? 3 : c;
}

// NV values of one group held by one lane (the group's D values are spread over D / NV lanes).
template <int NV>
struct QVec {
  float f[NV];                // b < 16: the codes (exact small integers); b = 16: the input values
  float s, z;                 // scale and zero point ((1, 0) for native storage)
};

// Quantizes this lane's NV values (w: NV/2 words of bf16 pairs, in channel order) at width
// class cls.  Every lane of the group must call it (the min/max are reduced across the group's
// D / NV lanes).
//
// The codes are rint(fl(d / s)), d = fl(x - z).  Each quotient is first taken as q = fl(d * r)
// with r = v_rcp_f32(s) (1 ulp): |q - fl(d / s)| <= 2^-22 q, and q <= n = 2^b - 1 (up to
// rounding), so when q lies more than n * 2^-20 from the nearest half-integer, rint(q) =
// rint(fl(d / s)) exactly.  Values that miss this (or with s = 0, or s outside [2^-100, 2^100])
// are redone with the correctly rounded divide; the codes are the same either way.  Such values
// are common (bf16 inputs often put d / s on a half-integer exactly), so the fallback is taken
// per value rather than per lane.  On the fast path the codes already lie in [0, n]: 0 <= d <= R
// and r ~ n / R.
template <int D, int NV>
__device__ __forceinline__ void eq4_quant(QVec<NV>& q, const uint32_t* w, int cls) {
#pragma clang fp contract(off)
  constexpr int LPG = D / NV;
  float x[NV];
#pragma unroll
  for (int e = 0; e < NV / 2; ++e) {
    x[2 * e] = tr_bf16_lo(w[e]);
    x[2 * e + 1] = tr_bf16_hi(w[e]);
  }
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int e = 1; e < NV; ++e) {
    mn = tr_min(mn, x[e]);
    mx = tr_max(mx, x[e]);
  }
  tr_group_minmax<LPG>(mn, mx);
  q.s = 1.0f;
  q.z = 0.0f;
#pragma unroll
  for (int e = 0; e < NV; ++e) q.f[e] = x[e];
  if (cls == 3) return;
  const float nlev = (float)((1 << (2 << cls)) - 1);
  const float z = mn + 0.0f;                           // -0 -> +0
  const float R = mx - mn;
  const float sc = R / nlev + 0.0f;                    // correctly rounded divide; -0 -> +0
  q.s = sc;
  q.z = z;
  const float r = __builtin_amdgcn_rcpf(sc);
  const float lim = 0.5f - nlev * 0x1p-20f;
  const bool sc_ok = sc >= 0x1p-100f && sc <= 0x1p100f;
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const float d = x[e] - z;
    const float qq = d * r;
    const float cf = rintf(qq);
    q.f[e] = cf;
    // Per value, so that a wave runs the divide only for the elements some lane needs it for.
    if (!(fabsf(qq - cf) < lim && sc_ok))
      q.f[e] = sc == 0.0f ? 0.0f : __builtin_amdgcn_fmed3f(rintf(d / sc), 0.0f, nlev);
  }
}

// f as bf16 words (exact: codes are integers <= 255, b = 16 values were bf16): NV / 2 words.
template <int NV>
__device__ __forceinline__ void bf16_words(const QVec<NV>& q, uint32_t* out) {
#pragma unroll
  for (int e = 0; e < NV / 2; ++e)
    out[e] = __builtin_amdgcn_perm(__float_as_uint(q.f[2 * e + 1]), __float_as_uint(q.f[2 * e]), 0x07060302u);
}

// Codes packed from the low bit up (code e at bit e * b) for b = 2, 4, 8: NV * b / 32 words of
// out[NV / 4] are meaningful.  Branch-free over the three widths.
template <int NV>
__device__ __forceinline__ void code_words(const QVec<NV>& q, int cls, uint32_t* out) {
  const int b = 2 << cls;
  uint32_t A[NV / 4];                                  // 4 codes each, in the low 4b bits
#pragma unroll
  for (int k = 0; k < NV / 4; ++k) {
    const uint32_t u0 = (uint32_t)q.f[4 * k], u1 = (uint32_t)q.f[4 * k + 1];
    const uint32_t u2 = (uint32_t)q.f[4 * k + 2], u3 = (uint32_t)q.f[4 * k + 3];
    A[k] = u0 | (u1 << b) | (u2 << (2 * b)) | (u3 << (3 * b));
  }
#pragma unroll
  for (int k = 0; k < NV / 4; ++k) {
    uint32_t v = A[k];                                 // b = 8
    if (2 * k + 1 < NV / 4) {
      const uint32_t v4 = A[2 * k] | (A[2 * k + 1] << 16);
      v = cls == 1 ? v4 : v;
    }
    if (4 * k + 3 < NV / 4) {
      const uint32_t v2 = A[4 * k] | (A[4 * k + 1] << 8) | (A[4 * k + 2] << 16) | (A[4 * k + 3] << 24);
      v = cls == 0 ? v2 : v;
    } else if (NV == 8 && k == 0) {
      v = cls == 0 ? (A[0] | (A[1] << 8)) : v;         // b = 2, 8 codes: 16 bits
    }
    out[k] = v;
  }
}

// Stores this lane's share of a page row (row = the row's first byte): NV * b / 8 bytes at
// part * NV * b / 8.
template <int NV>
__device__ __forceinline__ void put_row(uint8_t* row, int part, int cls, const QVec<NV>& q) {
  if (cls == 3) {
    uint32_t w[NV / 2];
    bf16_words<NV>(q, w);
#pragma unroll
    for (int x = 0; x < NV / 8; ++x)
      reinterpret_cast<uint4*>(row)[part * (NV / 8) + x] = make_uint4(w[4 * x], w[4 * x + 1], w[4 * x + 2], w[4 * x + 3]);
    return;
  }
  uint32_t w[NV / 4];
  code_words<NV>(q, cls, w);
  if constexpr (NV == 8) {
    if (cls == 0) reinterpret_cast<uint16_t*>(row)[part] = (uint16_t)w[0];
    else if (cls == 1) reinterpret_cast<uint32_t*>(row)[part] = w[0];
    else reinterpret_cast<uint2*>(row)[part] = make_uint2(w[0], w[1]);
  } else {
    if (cls == 0) reinterpret_cast<uint32_t*>(row)[part] = w[0];
    else if (cls == 1) reinterpret_cast<uint2*>(row)[part] = make_uint2(w[0], w[1]);
    else reinterpret_cast<uint4*>(row)[part] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Row of position slot-index j, head h, kv = 0 for K and 1 for V, in a page of class cls, and
// its group's (s, z) entry (b < 16).
__device__ __forceinline__ uint8_t* page_row(const CacheLayout& c, uint8_t* base, int j, int h, int kv, int cls) {
  return base + tr_sel4(cls, kv ? c.v_off : c.k_off) + (int64_t)h * c.cb + (int64_t)j * tr_sel4(cls, c.rowb);
}
__device__ __forceinline__ float2* page_side(const CacheLayout& c, uint8_t* base, int j, int h, int kv, int cls) {
  return reinterpret_cast<float2*>(base + tr_sel4(cls, kv ? c.sv_off : c.sk_off)) + (int64_t)h * tr_sel4(cls, c.ptok) + j;
}

// Stores this lane's piece (and, from the group's first lane, its (s, z) for b < 16).
template <int NV>
__device__ __forceinline__ void put_piece(const CacheLayout& c, uint8_t* base, int j, int h, int kv, int part, int cls,
                                          const QVec<NV>& q) {
  put_row<NV>(page_row(c, base, j, h, kv, cls), part, cls, q);
  if (cls != 3 && part == 0) *page_side(c, base, j, h, kv, cls) = make_float2(q.s, q.z);
}

// Page of slot `slot` of class cls (nullptr when the pool was exhausted, which is flagged) and the
// row within it.
__device__ __forceinline__ uint8_t* slot_page(const CacheLayout& c, int layer, int s, int cls, int32_t slot, int& j) {
  const int32_t* pt = c.ptab + ((int64_t)layer * c.B + s) * c.pt_stride + tr_sel4(cls, c.pt_off);
  const int32_t page = pt[slot >> tr_sel4(cls, c.ptok_log2)];
  j = slot & (tr_sel4(cls, c.ptok) - 1);
  uint8_t* base = c.pool + (int64_t)max(page, 0) * c.page_bytes;
  return page < 0 ? nullptr : base;
}

// Stores this lane's piece into its slot: position p of sequence s, head h, kv = 0 for K and 1 for
// V.  The slot assignment must have run (prefix counts and page tables of position p).
template <int NV>
__device__ __forceinline__ void store_piece(const CacheLayout& c, int layer, int s, int p, int h, int kv, int part,
                                            int cls, const QVec<NV>& q) {
  int j;
  uint8_t* base = slot_page(c, layer, s, cls, tr_prefix_row(c, layer, s, p)[cls], j);
  if (!base) return;
  if (h == 0 && kv == 0 && part == 0) reinterpret_cast<int32_t*>(base)[j] = p;
  put_piece<NV>(c, base, j, h, kv, part, cls, q);
}

__device__ __forceinline__ int32_t slot_of(int cls, int4 prefix) {
  const int lo = (cls & 1) ? prefix.y : prefix.x, hi = (cls & 1) ? prefix.w : prefix.z;
  return (cls & 2) ? hi : lo;
}
