// Prefill routed attention over the mixed-width paged cache (TriRoute review page,
// xllm-io.github.io: Eq. (2) for every query of the prompt, reading the K/V that Eq. (4) has
// just written -- the inference paragraph after Algorithm 1).
//
// Heads: the cache holds H KV heads; the queries have HQ = G * H heads, and query head h reads
//   KV head h / G (grouped-query attention; G = 1 is multi-head).  Staging is per KV head; the
//   compaction, attention and merge are per query head.
// k_prefill_prep (one workgroup per (seq, query head), plus one per sequence for the slot
//   assignment of the call's positions): stable partition of the T query rows by mode -- full
//   rows, then local rows, then skip rows (and rows with an invalid mode) -- so that a 128-row
//   tile holds one mode and its key range is tight.  Then the attention work units of the
//   (seq, query head).
// Dense staging: the cache range the call's queries read, staged once in position order: K as
//   its code in bf16 (an exact integer <= 255, or the stored bf16 for b = 16) with per-key
//   (alpha, r) = (s_K * log2(e)/sqrt(D), z_K / s_K); V as v_hat = s * c + z (fp32) rounded to
//   fp16, channel-major.  Every 128-row tile of a (seq, head) then reads this
//   instead of re-unpacking the pages (a (seq, head) stays on one XCD, so the re-reads hit its
//   L2).  k_prefill_write (one workgroup per (seq, head, 32 positions)) quantizes the call's
//   own K/V into the pages and stages them from registers; k_prefill_dense stages the tiles
//   holding earlier calls' positions from the pages.
// k_prefill_attn (one workgroup = 4 waves = one 128-row tile), per 32-key tile:
//     staging   16-byte buffer loads of K rows and V^T rows (the tile offset in a scalar
//               register) into double-buffered LDS, the next tile's loads in flight in
//               registers while the current one is computed.
//     QK^T      S^T[32 keys x 32 queries] per wave = v_mfma_f32_32x32x16_bf16 over D/16 steps
//               on the exact codes, plus one k-step that adds r * sum(q) (r and sum(q) as bf16
//               hi + lo pairs); the exponent is then alpha * S - m_ref, one FMA per score.
//               This is Eq. (4)'s reconstruction folded out of the product:
//               q . (s c + z) = s (q . c + (z / s) sum(q)).
//     softmax   fp32 in registers, each lane holds 16 keys of one query; running reference
//               max with a lazy rescale (only when a row's max grows by more than 2^8);
//               masks only on tiles that cross a row's window edge; waves skip tiles outside
//               their own windows.
//     PV        O^T[D x 32 queries] += V^T P^T with v_mfma_f32_32x32x16_f16; P is the lane's
//               own scores; the dense V^T rows store keys in the S^T accumulator's order
//               (vt_pos), so each V^T operand is one 16-byte LDS read.
//   epilogue  O / l -> bf16, scattered back to the rows' original positions.
// k_prefill_merge combines the chunks of split tiles and writes the zeros of the skip rows.
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "common.h"
#include "kv_write.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBlock = 256;
constexpr int BM = 128;       // query rows per workgroup (4 waves x 32)
constexpr int BN = 32;        // keys per tile
constexpr float kRescale = 8.0f;
constexpr int kSlotsPerHead = TR_PREFILL_SLOTS;   // partial-result slots of one (seq, head)

// Max / sum of a value and its copy 32 lanes away, with v_permlane32_swap (no LDS traffic): the
// swap hands lanes 0-31 the upper half's value in its second result and lanes 32-63 the lower
// half's in its first, so max(first, second) is the pairwise max in every lane.
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Work units of the attention kernel for one (seq, head), after the row compaction: one per
// 128-row tile, except that a tile whose key range spans n > kch key tiles is cut into
// ceil(n / kch) near-equal chunks that run as separate units, write partial (max, sum, O) rows,
// and are merged by k_prefill_merge.  kch is the smallest of 16, 32, 64, ... key tiles for which the
// head's partial results fit its kSlotsPerHead slots (no split if none does).
//   unit  = (r0 | full << 31, rend | (partial slot + 1, or 0) << 25, kt0, kt1)   (rend < 2^25:
//           positions are below 2^24 for every cache tr_kv_cache_alloc accepts)
//   merge = (r0, rend, first slot, chunks)
// Units are listed heaviest first: full tiles from the last (longest key range), then local.
// Sum over the 64 lanes of a wave (the result in every lane).
__device__ __forceinline__ int wave_sum(int v) { return __builtin_amdgcn_readlane((int)tr_wave_incl_scan((uint32_t)v), 63); }

// Row tiles whose first and last positions the compaction leaves in LDS; calls with more row
// tiles read them back from the compacted row list instead.
#ifndef TR_PREFILL_TILE_CAP
#define TR_PREFILL_TILE_CAP 512
#endif
constexpr int kTileCap = TR_PREFILL_TILE_CAP;

// Run by one wave (the other waves of the workgroup do not take part): tiles in chunks of 64, one
// per lane, with wave-level sums and scans only -- no workgroup barriers.
__device__ __forceinline__ void build_units(int sh, int p0, int window, int nfull, int nl, const int32_t* rl,
                                            const int32_t* tpos, int32_t* counts, int4* units, int4* merges) {
  constexpr int NC = 8;                            // candidate chunk sizes 16 << j key tiles
  const int lane = threadIdx.x & 63;
  const int nft = (nfull + BM - 1) / BM, nlt = (nl + BM - 1) / BM, ntl = nft + nlt;
  auto tile_range = [&](int k, int& r0, int& rend, int& full, int& klo, int& khi) {
    full = k < nft;
    const int ft = nft - 1 - k;                    // full tiles from the last
    r0 = full ? ft * BM : nfull + (k - nft) * BM;
    rend = full ? min(r0 + BM, nfull) : min(r0 + BM, nfull + nl);
    // rows are in position order; row tile idx (full tiles in row order, then local) has its
    // first and last positions at tpos[2 idx], tpos[2 idx + 1]
    const int idx = full ? ft : k;
    const bool lds = ntl <= kTileCap;
    const int tmin = p0 + (lds ? tpos[2 * idx] : rl[r0]), tmax = p0 + (lds ? tpos[2 * idx + 1] : rl[rend - 1]);
    const int blo = full ? 0 : max(0, tmin - window);
    klo = blo >> 5;
    khi = (tmax + 1 + 31) >> 5;
  };
  // pass A: partial slots each candidate chunk size would need
  int want[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) want[j] = 0;
  for (int k = lane; k < ntl; k += 64) {
    int r0, rend, full, klo, khi;
    tile_range(k, r0, rend, full, klo, khi);
    const int nkt = khi - klo;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int kc = 16 << j;
      want[j] += (nkt > kc) ? (nkt + kc - 1) / kc : 0;
    }
  }
  int kch = 1 << 30;                               // no split
#pragma unroll
  for (int j = NC - 1; j >= 0; --j)
    if (wave_sum(want[j]) <= kSlotsPerHead) kch = 16 << j;
  // pass B: units, slots and merges in tile order (exclusive scans carried across chunks)
  int base[3] = {0, 0, 0};
  for (int k0 = 0; k0 < ntl; k0 += 64) {
    const int k = k0 + lane;
    int r0 = 0, rend = 0, full = 0, klo = 0, khi = 0, nch = 0;
    if (k < ntl) {
      tile_range(k, r0, rend, full, klo, khi);
      nch = (khi - klo > kch) ? (khi - klo + kch - 1) / kch : 1;
    }
    const int v[3] = {nch, nch > 1 ? nch : 0, nch > 1 ? 1 : 0};
    int pos[3];
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      const int incl = (int)tr_wave_incl_scan((uint32_t)v[x]);
      pos[x] = base[x] + incl - v[x];
      base[x] += __shfl(incl, 63, 64);
    }
    if (k < ntl) {
      for (int cc = 0; cc < nch; ++cc) {
        const int kt0 = klo + ((khi - klo) * cc) / nch, kt1 = klo + ((khi - klo) * (cc + 1)) / nch;
        units[pos[0] + cc] = make_int4(r0 | (full << 31), rend | ((nch > 1 ? pos[1] + cc + 1 : 0) << 25), kt0, kt1);
      }
      if (nch > 1) merges[pos[2]] = make_int4(r0, rend, pos[1], nch);
    }
  }
  if (lane == 0) {
    counts[sh * 4 + 0] = nfull;
    counts[sh * 4 + 1] = nl;
    counts[sh * 4 + 2] = base[0];
    counts[sh * 4 + 3] = base[2];
  }
}

// Stable partition of the query rows of one (seq, head) by mode, NT threads: thread t takes
// the contiguous rows [t R, t R + R), counts its full and local rows, one block-wide scan gives
// every thread its output offsets, and a second pass over its rows writes them.  The modes are
// loaded 4 rows at a time (addresses clamped into the column, so the loads go out together) and,
// for R <= 16, kept as 2-bit codes for the second pass.
template <int D, int NT>
__device__ __forceinline__ void compact_rows(const CacheLayout& c, int HQ, int sh, int p0, int T, int window,
                                             const uint8_t* __restrict__ mode, int32_t* __restrict__ rows,
                                             int32_t* __restrict__ counts, int4* __restrict__ units,
                                             int4* __restrict__ merges, int uph) {
  constexpr int NW = NT / 64;
  __shared__ uint32_t wf[NW], wl[NW];
  __shared__ int32_t tpos[2 * kTileCap];           // first / last position of each row tile
  const int s = sh / HQ, h = sh % HQ;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int32_t* rl = rows + (int64_t)sh * c.pfN;
  const uint8_t* mcol = mode + (int64_t)s * T * HQ + h;
  const int R = (T + NT - 1) / NT;
  const int i0 = min(T, tid * R), i1 = min(T, i0 + R);
  // 2-bit code of a row's mode: 0 skip, 1 local, 2 full, 3 invalid (flagged, treated as skip)
  auto load4 = [&](int r0, uint32_t (&m)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + r0 + u;
      const uint32_t x = mcol[(int64_t)min(i, T - 1) * HQ];
      m[u] = i < i1 ? (x > TR_MODE_FULL ? 3u : x) : 0u;
    }
  };
  const bool cached = R <= 16;
  uint32_t mp = 0;
  uint32_t nf = 0, nlc = 0;
  for (int r0 = 0; r0 < R; r0 += 4) {
    uint32_t m[4];
    load4(r0, m);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      nf += m[u] == TR_MODE_FULL;
      nlc += m[u] == TR_MODE_LOCAL;
      if (cached && r0 + u < 16) mp |= m[u] << (2 * (r0 + u));
    }
  }
  const uint32_t incf = tr_wave_incl_scan(nf), incl = tr_wave_incl_scan(nlc);
  if (lane == 63) {
    wf[wave] = incf;
    wl[wave] = incl;
  }
  __syncthreads();
  uint32_t bf = incf - nf, bl = incl - nlc, tf = 0, tl = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w < wave) {
      bf += wf[w];
      bl += wl[w];
    }
    tf += wf[w];
    tl += wl[w];
  }
  const int nfull = (int)tf, nl = (int)tl;
  const int nft = (nfull + BM - 1) / BM, ntl = nft + (nl + BM - 1) / BM;
  // row d of a mode's list ends or starts a row tile: its position goes to the tile's LDS slots
  auto mark = [&](int d, int nmode, int tile0, int i) {
    const int idx = tile0 + d / BM;
    if (idx < kTileCap) {
      if (d % BM == 0) tpos[2 * idx] = i;
      if (d % BM == BM - 1 || d == nmode - 1) tpos[2 * idx + 1] = i;
    }
  };
  uint32_t bs = (uint32_t)i0 - bf - bl;            // skip rows before this thread's
  for (int r0 = 0; r0 < R; r0 += 4) {
    uint32_t m[4];
    if (cached) {
#pragma unroll
      for (int u = 0; u < 4; ++u) m[u] = (mp >> (2 * (r0 + u))) & 3u;
    } else {
      load4(r0, m);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + r0 + u;
      if (i >= i1) break;
      if (m[u] == TR_MODE_FULL) {
        mark((int)bf, nfull, 0, i);
        rl[bf++] = i;
      } else if (m[u] == TR_MODE_LOCAL) {
        mark((int)bl, nl, nft, i);
        rl[nfull + bl++] = i;
      } else {
        if (m[u] == 3u) atomicOr(c.err, TR_ERRF_BAD_MODE);
        rl[nfull + nl + bs++] = i;                   // skip rows: zeroed by k_prefill_merge
      }
    }
  }
  if (ntl > kTileCap) __threadfence_block();      // the unit list then reads the row list back
  __syncthreads();
  if (wave == 0)
    build_units(sh, p0, window, nfull, nl, rl, tpos, counts, units + (int64_t)sh * uph,
                merges + (int64_t)sh * (kSlotsPerHead / 2));
}

// Preparation of a prefill call, one launch: workgroups [0, B*HQ) compact the query rows of one
// (seq, query head) each and list its attention work units; with assign set, workgroups
// [B*HQ, B*HQ + B)
// assign the slots and pages of the call's positions, one sequence each (independent work that
// the quantize-write needs, so it overlaps the compaction instead of taking a launch of its own).
template <int D>
__global__ __launch_bounds__(TR_ASSIGN_THREADS) void k_prefill_prep(CacheLayout c, int layer, int p0, int T,
                                                                    int window, const uint8_t* __restrict__ mode,
                                                                    const uint8_t* __restrict__ bits, int32_t* rows,
                                                                    int32_t* counts, int4* units, int4* merges,
                                                                    int uph, int HQ) {
  const int BH = c.B * HQ;
  if ((int)blockIdx.x >= BH) {
    tr_assign_slots_seq(c, layer, p0, T, bits, blockIdx.x - BH);
    return;
  }
  compact_rows<D, TR_ASSIGN_THREADS>(c, HQ, blockIdx.x, p0, T, window, mode, rows, counts, units, merges, uph);
}


template <int NB>
__device__ __forceinline__ uint32_t code_at(const uint32_t* w, int e) {
  return (w[(e * NB) >> 5] >> ((e * NB) & 31)) & ((1u << NB) - 1u);
}

template <int BYTES>
__device__ __forceinline__ void load_slice_c(const uint8_t* p, uint32_t* w) {
  if constexpr (BYTES == 2) {
    w[0] = *reinterpret_cast<const uint16_t*>(p);
  } else if constexpr (BYTES == 4) {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (BYTES == 8) {
    const uint2 t = *reinterpret_cast<const uint2*>(p);
    w[0] = t.x; w[1] = t.y;
  } else {
#pragma unroll
    for (int x = 0; x < BYTES / 16; ++x) {
      const uint4 t = reinterpret_cast<const uint4*>(p)[x];
      w[4 * x] = t.x; w[4 * x + 1] = t.y; w[4 * x + 2] = t.z; w[4 * x + 3] = t.w;
    }
  }
}

__device__ __forceinline__ uint16_t f16_bits(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }

// The attention's PV product takes v_hat in fp16: a stored value with |v_hat| >= 65504 (fp16's
// largest finite value) sets the sticky range flag instead of turning into an infinity silently.
// Every V input with |v| <= 65280 (the largest bf16 below 65504) stays inside: v_hat lies within
// its group's [min, max] up to 2^-22 relative.
constexpr float kF16Max = 65504.0f;

// Dequantize DPL channels of one (token, head) K/V pair of width class C into the dense
// scratch (K row slice) and the LDS V^T tile.
// Position of key k (0..31) of a tile inside a V^T row: bits 2 and 3 swapped within each group
// of 16, so that the 8 keys one lane of the PV product needs (4g .. 4g+3 and 8+4g .. 8+4g+3 of a
// 16-key step, the key order of the S^T accumulator) are contiguous.
__device__ __forceinline__ int vt_pos(int k) { return (k & ~15) | (k & 3) | ((k & 4) << 1) | ((k & 8) >> 1); }

__device__ __forceinline__ uint32_t f16_pair(float lo, float hi) {
  return (uint32_t)f16_bits(lo) | ((uint32_t)f16_bits(hi) << 16);
}

// Per-key factors of the QK^T product: alpha = s * kscale and r = z / s, so that
// kscale * q . (s c + z) = alpha * (q . c + r * sum(q)).  b = 16 keys (stored bf16 x, "codes" x)
// take (kscale, 0); a constant group (s = 0, codes 0) takes (kscale, z).
__device__ __forceinline__ float2 key_factors(bool native, float s, float z, float kscale) {
  if (native) return make_float2(kscale, 0.0f);
  if (s == 0.0f) return make_float2(kscale, z);
  return make_float2(s * kscale, z / s);
}

template <int D, int C>
__device__ __forceinline__ void dense_token(const uint8_t* pb, const CacheLayout& c, int h, int j, int part,
                                            uint16_t* krow, _Float16 (*vt)[40], int tk, float kscale,
                                            float2* kf_out) {
  constexpr int DPL = D / 8;
  constexpr int b = 2 << C;
  constexpr int SLB = DPL * b / 8;                 // slice bytes
  uint32_t wk[8], wv[8];
  const int64_t off = (int64_t)h * c.cb + (int64_t)j * (D * b / 8) + part * SLB;
  load_slice_c<SLB>(pb + c.k_off[C] + off, wk);
  load_slice_c<SLB>(pb + c.v_off[C] + off, wv);
  uint32_t ko[DPL / 2];
  if constexpr (C == 3) {
#pragma unroll
    for (int e = 0; e < DPL / 2; ++e) {
      ko[e] = wk[e];
      vt[part * DPL + 2 * e][vt_pos(tk)] = (_Float16)tr_bf16_lo(wv[e]);
      vt[part * DPL + 2 * e + 1][vt_pos(tk)] = (_Float16)tr_bf16_hi(wv[e]);
    }
    *kf_out = key_factors(true, 1.0f, 0.0f, kscale);
    float vmax = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL / 2; ++e) vmax = tr_max(vmax, tr_max(fabsf(tr_bf16_lo(wv[e])), fabsf(tr_bf16_hi(wv[e]))));
    if (vmax >= kF16Max) atomicOr(c.err, TR_ERRF_RANGE);
  } else {
    const int P = c.ptok[C];
    const float2 szk = reinterpret_cast<const float2*>(pb + c.sk_off[C])[(int64_t)h * P + j];
    const float2 szv = reinterpret_cast<const float2*>(pb + c.sv_off[C])[(int64_t)h * P + j];
    float vmax = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; e += 2) {
      const float k0 = (float)code_at<b>(wk, e), k1 = (float)code_at<b>(wk, e + 1);
      ko[e / 2] = (__float_as_uint(k0) >> 16) | (__float_as_uint(k1) & 0xffff0000u);
      const float v0 = fmaf(szv.x, (float)code_at<b>(wv, e), szv.y);
      const float v1 = fmaf(szv.x, (float)code_at<b>(wv, e + 1), szv.y);
      vmax = tr_max(vmax, tr_max(fabsf(v0), fabsf(v1)));
      vt[part * DPL + e][vt_pos(tk)] = (_Float16)v0;
      vt[part * DPL + e + 1][vt_pos(tk)] = (_Float16)v1;
    }
    if (vmax >= kF16Max) atomicOr(c.err, TR_ERRF_RANGE);
    *kf_out = key_factors(false, szk.x, szk.y, kscale);
  }
#pragma unroll
  for (int x = 0; x < DPL / 8; ++x)
    reinterpret_cast<uint4*>(krow)[x] = make_uint4(ko[4 * x], ko[4 * x + 1], ko[4 * x + 2], ko[4 * x + 3]);
}

// Positions [32 * tile0, 32 * tile0 + 32 * ntile) of every (seq, head); positions >= pend
// are written as zeros (they are only ever read masked).
template <int D>
__global__ __launch_bounds__(kBlock) void k_prefill_dense(CacheLayout c, int layer, int tile0, int ntile, int pend,
                                                          int np, float kscale, uint16_t* __restrict__ dk,
                                                          uint16_t* __restrict__ dv, float2* __restrict__ dkf) {
  constexpr int DPL = D / 8;
  __shared__ _Float16 vt[D][40];                   // v_hat tile, channel-major (row = 80 B)
  const int lin = tr_xcd_linear(c.B * c.H * ntile);
  if (lin < 0) return;
  const int tile = tile0 + lin % ntile, sh = lin / ntile;
  const int s = sh / c.H, h = sh % c.H;
  const int tid = threadIdx.x, tk = tid / 8, part = tid % 8;
  const int p = tile * 32 + tk;
  uint16_t* krow = dk + ((int64_t)sh * np + p) * D + part * DPL;
  float2 kf = make_float2(0.0f, 0.0f);
  if (p < pend) {
    const int32_t* pr0 = tr_prefix_row(c, layer, s, p);
    const int32_t* pr1 = tr_prefix_row(c, layer, s, p + 1);
    int cls = 3;
#pragma unroll
    for (int x = 0; x < TR_NCLASS; ++x)
      if (pr1[x] != pr0[x]) cls = x;
    const int32_t slot = pr0[cls];
    const int32_t page = tr_ptab(c, layer, s, cls)[slot >> c.ptok_log2[cls]];
    const int j = slot & (c.ptok[cls] - 1);
    const uint8_t* pb = c.pool + (int64_t)(page < 0 ? 0 : page) * c.page_bytes;
    switch (cls) {
      case 0: dense_token<D, 0>(pb, c, h, j, part, krow, vt, tk, kscale, &kf); break;
      case 1: dense_token<D, 1>(pb, c, h, j, part, krow, vt, tk, kscale, &kf); break;
      case 2: dense_token<D, 2>(pb, c, h, j, part, krow, vt, tk, kscale, &kf); break;
      default: dense_token<D, 3>(pb, c, h, j, part, krow, vt, tk, kscale, &kf); break;
    }
  } else {
#pragma unroll
    for (int x = 0; x < DPL / 8; ++x) reinterpret_cast<uint4*>(krow)[x] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < DPL; ++e) vt[part * DPL + e][vt_pos(tk)] = (_Float16)0.0f;
  }
  if (part == 0) dkf[(int64_t)sh * np + p] = kf;
  __syncthreads();
  // V^T rows: D rows x 32 positions (64 bytes each), 16 bytes per thread.
  for (int x = tid; x < D * 4; x += kBlock) {
    const int d = x >> 2, seg = x & 3;
    const uint4 v = *reinterpret_cast<const uint4*>(&vt[d][seg * 8]);
    *reinterpret_cast<uint4*>(dv + ((int64_t)sh * D + d) * np + tile * 32 + seg * 8) = v;
  }
}

// Eq. (4) quantize-write of a prefill call's positions [p0, p0 + T), fused with their dense
// staging: one workgroup of 4D threads per (seq, head, 64 positions) of tiles [tile0, tile0 +
// ntile); D/16 lanes per position, 16 channels of K and of V each.  A lane issues all its loads
// (bits, prefix counts, K, V), then the page-table lookup of its slot, and quantizes while that
// lookup is in flight.  Codes, scales and page stores are the plain write path's (the same Eq. (4)
// helpers); tiles from dense_from on also get their K rows, key factors and v_hat columns from
// the values in registers, without re-reading the pages, and zeros at positions >= p0 + T.  Runs after the
// slot assignment of the same positions.
constexpr int kWriteTile = 64;
constexpr int kWriteNV = 16;                       // channels per lane

template <int D>
__global__ __launch_bounds__(4 * D) void k_prefill_write(CacheLayout c, int layer, int p0, int T, int tile0,
                                                         int ntile, int dense_from, int np, float kscale,
                                                         const uint16_t* __restrict__ kin,
                                                         const uint16_t* __restrict__ vin,
                                                         const uint8_t* __restrict__ bits, uint16_t* __restrict__ dk,
                                                         uint16_t* __restrict__ dv, float2* __restrict__ dkf) {
  constexpr int NV = kWriteNV;
  constexpr int LPG = D / NV;
  constexpr int NT = 4 * D;
  constexpr int TP = kWriteTile;
  static_assert(NT / LPG == TP, "one position per lane group");
  __shared__ _Float16 vt[D][TP + 8];               // v_hat tile, channel-major (row = 144 B)
  const int lin = tr_xcd_linear(c.B * c.H * ntile);
  if (lin < 0) return;
  const int tile = tile0 + lin % ntile, sh = lin / ntile;
  const int s = sh / c.H, h = sh % c.H;
  const int tid = threadIdx.x, tk = tid / LPG, part = tid % LPG;
  const int p = tile * TP + tk, i = p - p0;
  const bool live = i >= 0 && i < T;
  // positions outside the call read the call's first position and store nothing
  const int64_t tok = (int64_t)s * T + (live ? i : 0);
  const int bval = bits[tok];
  const int4 prefix = *reinterpret_cast<const int4*>(tr_prefix_row(c, layer, s, live ? p : p0));
  const uint4* ksrc = reinterpret_cast<const uint4*>(kin + (tok * c.H + h) * D + part * NV);
  const uint4* vsrc = reinterpret_cast<const uint4*>(vin + (tok * c.H + h) * D + part * NV);
  const uint4 k0 = ksrc[0], k1 = ksrc[1], v0 = vsrc[0], v1 = vsrc[1];
  const int cls = eq4_class(bval);
  int j;
  uint8_t* base = slot_page(c, layer, s, cls, slot_of(cls, prefix), j);
  QVec<NV> qk, qv;
  {
    const uint32_t w[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
    eq4_quant<D, NV>(qk, w, cls);
  }
  {
    const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    eq4_quant<D, NV>(qv, w, cls);
  }
  const bool dense = tile >= dense_from;           // else the tile also holds earlier positions
  if (dense) {
    // K: the codes (or the b = 16 values) as bf16 plus the key's (alpha, r); v_hat =
    // fp16(s * f + z), where b = 16 takes z = -0 so that fma(1, x, -0) = x keeps a zero's sign.
    const float zv = cls == 3 ? -0.0f : qv.z;
    uint32_t kw[NV / 2];
    bf16_words<NV>(qk, kw);
    uint4* krow = reinterpret_cast<uint4*>(dk + ((int64_t)sh * np + p) * D + part * NV);
    krow[0] = live ? make_uint4(kw[0], kw[1], kw[2], kw[3]) : make_uint4(0, 0, 0, 0);
    krow[1] = live ? make_uint4(kw[4], kw[5], kw[6], kw[7]) : make_uint4(0, 0, 0, 0);
    if (part == 0)
      dkf[(int64_t)sh * np + p] = live ? key_factors(cls == 3, qk.s, qk.z, kscale) : make_float2(0.0f, 0.0f);
    // The V^T column is XOR-swizzled by 16 * (part & 3): the lanes of one store hold 16 positions
    // of 4 parts whose rows are 16 rows (a multiple of 64 banks) apart, so without it they collide.
    const int tpos = vt_pos(tk) ^ (16 * (part & 3));
    float vmax = 0.0f;
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      const float vh = fmaf(qv.s, qv.f[e], zv);
      vmax = tr_max(vmax, fabsf(vh));
      vt[part * NV + e][tpos] = live ? (_Float16)vh : (_Float16)0.0f;
    }
    if (live && vmax >= kF16Max) atomicOr(c.err, TR_ERRF_RANGE);
  }
  if (live && base) {
    if (h == 0 && part == 0) reinterpret_cast<int32_t*>(base)[j] = p;
    put_piece<NV>(c, base, j, h, 0, part, cls, qk);
    put_piece<NV>(c, base, j, h, 1, part, cls, qv);
  }
  if (!dense) return;
  __syncthreads();
  // V^T rows: D rows x TP positions (128 bytes each), 16 bytes per thread; row d was written by
  // part d / 16, so its segment seg sits at seg ^ 2 (part & 3).
  constexpr int SEGS = TP / 8;
  for (int x = tid; x < D * SEGS; x += NT) {
    const int d = x / SEGS, seg = x % SEGS;
    const uint4 v = *reinterpret_cast<const uint4*>(&vt[d][8 * (seg ^ (2 * ((d / NV) & 3)))]);
    *reinterpret_cast<uint4*>(dv + ((int64_t)sh * D + d) * np + tile * TP + seg * 8) = v;
  }
}

template <int D>
struct alignas(16) PrefillTile {
  uint16_t ks[BN][D + 8];      // K codes as bf16 integers / stored bf16, key-major; columns
                               // D .. D + 7 hold the key's (r_hi, r_hi, r_lo, 0, ...) in bf16
  uint16_t vt[D][BN + 8];      // v_hat fp16, channel-major, keys in vt_pos order
  alignas(16) float alpha[BN]; // s_K * log2(e) / sqrt(D) (or log2(e) / sqrt(D))
};

template <int D>
struct PrefillSmem {
  PrefillTile<D> tile[2];      // double buffer
};

// Buffer-resource loads: the base and size live in scalar registers, the tile's key offset is a
// scalar offset, so advancing a tile costs no vector instructions; reads past the size return 0.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRsrcWord3);
}

#ifndef TR_PREFILL_WAVES
#define TR_PREFILL_WAVES 4
#endif
template <int D>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(D == 64 ? TR_PREFILL_WAVES : 2))) void k_prefill_attn(
    CacheLayout c, int p0, int T, int window, int np, const uint16_t* __restrict__ q,
    const int32_t* __restrict__ rows, const int32_t* __restrict__ counts, const int4* __restrict__ units, int uph,
    const uint16_t* __restrict__ dk, const uint16_t* __restrict__ dv, const float2* __restrict__ dkf,
    float* __restrict__ part, uint16_t* __restrict__ out, int HQ, int QG) {
  constexpr int KS = D / 16;           // MFMA k-steps for QK^T
  constexpr int MT = D / 32;           // 32-channel tiles of O^T
  constexpr int KPT = D / 64;          // 16-byte K pieces per thread per tile
  constexpr int VPT = D / 64;          // 16-byte V^T pieces per thread per tile
  __shared__ PrefillSmem<D> sm;

  const int BH = c.B * HQ;
  const int u = blockIdx.x / BH, sh = blockIdx.x % BH;   // sh: (seq, query head)
  const int s = sh / HQ, h = sh % HQ;
  const int64_t skv = (int64_t)s * c.H + h / QG;         // its KV head's dense rows
  if (u >= counts[sh * 4 + 2]) return;
  const int4 unit = units[(int64_t)sh * uph + u];
  const bool full = unit.x < 0;
  const int r0 = unit.x & 0x7fffffff, rend = unit.y & 0x1ffffff;
  const int kt0 = unit.z, kt1 = unit.w, slot = (unit.y >> 25) - 1;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, g = lane >> 5;
  const int kb0 = kt0 * BN;                        // this unit's key tiles [kt0, kt1)
  const int ntiles = kt1 - kt0;

  // Staging: thread -> K row (tid / 8), 16-byte piece (tid % 8); V^T row (tid / 4), piece
  // (tid % 4); for D = 128 every thread moves two pieces of each.
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(dk + skv * np * D, (uint32_t)np * D * 2u);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(dv + skv * D * np, (uint32_t)np * D * 2u);
  const __amdgpu_buffer_rsrc_t frs = make_rsrc(dkf + skv * np, (uint32_t)np * 8u);
  uint32_t voff[VPT];
#pragma unroll
  for (int x = 0; x < VPT; ++x) {
    const int e = tid + x * kBlock;
    voff[x] = (uint32_t)(((e >> 2) * np + (e & 3) * 8) * 2);
  }
  u32x4 rk[KPT], rv[VPT];
  u32x2 rf = {0u, 0u};
  auto load_tile = [&](int kb) {
#pragma unroll
    for (int x = 0; x < KPT; ++x) rk[x] = __builtin_amdgcn_raw_buffer_load_b128(krs, (tid + x * kBlock) * 16, kb * D * 2, 0);
#pragma unroll
    for (int x = 0; x < VPT; ++x) rv[x] = __builtin_amdgcn_raw_buffer_load_b128(vrs, voff[x], kb * 2, 0);
    if (tid < BN) rf = __builtin_amdgcn_raw_buffer_load_b64(frs, tid * 8, kb * 8, 0);
  };
  auto store_tile = [&](PrefillTile<D>& tl) {
#pragma unroll
    for (int x = 0; x < KPT; ++x) {
      const int e = tid + x * kBlock;
      *reinterpret_cast<u32x4*>(&tl.ks[(e * 8) / D][(e * 8) % D]) = rk[x];
    }
#pragma unroll
    for (int x = 0; x < VPT; ++x) {
      const int e = tid + x * kBlock;
      *reinterpret_cast<u32x4*>(&tl.vt[e >> 2][(e & 3) * 8]) = rv[x];
    }
    if (tid < BN) {
      tl.alpha[tid] = __uint_as_float(rf.x);
      const float r = __uint_as_float(rf.y);
      const uint16_t hi = tr_f32_to_bf16(r);
      const uint16_t lo = tr_f32_to_bf16(r - tr_bf16_lo(hi));
      *reinterpret_cast<uint4*>(&tl.ks[tid][D]) = make_uint4((uint32_t)hi | ((uint32_t)hi << 16), lo, 0, 0);
    }
  };
  // The first tile's loads go out before the query rows', so the two round trips overlap.
  if (ntiles > 0) load_tile(kb0);

  const int ri = r0 + wave * 32 + n;
  const bool row_ok = ri < rend;
  const int i = row_ok ? rows[(int64_t)sh * c.pfN + ri] : 0;
  const int t = row_ok ? p0 + i : -1;
  const int lo = row_ok ? (full ? 0 : max(0, t - window)) : 0x7fffffff;

  // Q^T operand (B of the QK^T MFMA): column n = query, k = channels 16*ks + 8*g .. +7.
  bf16x8 qb[KS];
  float qsum = 0.0f;
  const uint16_t* qrow = q + (((int64_t)s * T + i) * HQ + h) * D;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint4 raw = row_ok ? *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * g) : make_uint4(0, 0, 0, 0);
    qb[ks] = __builtin_bit_cast(bf16x8, raw);
    qsum += (tr_bf16_lo(raw.x) + tr_bf16_hi(raw.x)) + (tr_bf16_lo(raw.y) + tr_bf16_hi(raw.y)) +
            (tr_bf16_lo(raw.z) + tr_bf16_hi(raw.z)) + (tr_bf16_lo(raw.w) + tr_bf16_hi(raw.w));
  }
  qsum = xor32_sum(qsum);
  // The zero-point k-step's B operand: (sq_hi, sq_lo, sq_hi, 0, ...) at k = 0 .. 7 (lanes g = 0),
  // zeros at k = 8 .. 15, against the keys' (r_hi, r_hi, r_lo, 0, ...): r * sum(q) to ~2^-16.
  bf16x8 qz;
  {
    const uint16_t hi = tr_f32_to_bf16(qsum);
    const uint16_t lo2 = tr_f32_to_bf16(qsum - tr_bf16_lo(hi));
    const uint4 w = g == 0 ? make_uint4((uint32_t)hi | ((uint32_t)lo2 << 16), hi, 0, 0) : make_uint4(0, 0, 0, 0);
    qz = __builtin_bit_cast(bf16x8, w);
  }

  // The wave's key-position range: [wlo, whi) holds every visible key of its rows; tiles at or
  // below tmin are causal for all of them, tiles at or above lomax inside every window.
  int wlo = lo, whi = row_ok ? t + 1 : -1, tmin = row_ok ? t : 0x7fffffff, lomax = row_ok ? lo : -1;
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) {
    wlo = min(wlo, __shfl_xor(wlo, o, 64));
    whi = max(whi, __shfl_xor(whi, o, 64));
    tmin = min(tmin, __shfl_xor(tmin, o, 64));
    lomax = max(lomax, __shfl_xor(lomax, o, 64));
  }
  wlo = __builtin_amdgcn_readfirstlane(wlo);
  whi = __builtin_amdgcn_readfirstlane(whi);
  tmin = __builtin_amdgcn_readfirstlane(tmin);
  lomax = __builtin_amdgcn_readfirstlane(lomax);
  const bool wave_live = whi > 0;

  f32x16 o[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[mt][r] = 0.0f;
  // Running reference m_ref of the row (log2 domain), with nm = -m_ref (0 before the row's first
  // visible key) and the threshold that triggers a rescale: any visible key before the first
  // one, then a tile maximum more than kRescale above m_ref.
  float mref = -INFINITY, lsum = 0.0f, nm = 0.0f, thr = -INFINITY;

  auto compute = [&](const PrefillTile<D>& tl, int kb) {
    // S = q . c + r * sum(q) (the zero-point k-step first, on a zero accumulator); then
    // x = score - mref = alpha * S - mref, one FMA per score.
    f32x16 sacc = {};
    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(&tl.ks[n][D]), qz, sacc, 0, 0, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&tl.ks[n][16 * ks + 8 * g]);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[ks], sacc, 0, 0, 0);
    }
    // Lane (n, g) holds keys kb + 4g + off, off = 8 * r4 + x.  Only tiles that cross a row's window
    // edge are masked, each with the cheapest test that suffices (a wave-uniform choice): key
    // visible iff off <= t - kb - 4g (causal edge) and off >= lo - kb - 4g (window's left edge).
    float sv[16];
    auto scores = [&](auto mask) {
      constexpr int M = decltype(mask)::value;     // 0 none, 1 causal edge, 2 left edge, 3 both
      const int dt = row_ok ? t - kb - 4 * g : -1;                // rows past the tile's end: all masked
      const int dl = row_ok ? lo - kb - 4 * g : 0x40000000;
      const uint32_t span = row_ok ? (uint32_t)(t - lo) : 0u;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float4 al = *reinterpret_cast<const float4*>(&tl.alpha[8 * r4 + 4 * g]);
        const float alv[4] = {al.x, al.y, al.z, al.w};
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int off = 8 * r4 + x;
          float v = fmaf(alv[x], sacc[4 * r4 + x], nm);
          if constexpr (M == 1) {
            if (off > dt) v = -INFINITY;
          } else if constexpr (M == 2) {
            if (off < dl) v = -INFINITY;
          } else if constexpr (M == 3) {
            if ((uint32_t)(off - dl) > span) v = -INFINITY;
          }
          sv[4 * r4 + x] = v;
        }
      }
    };
    const bool cross_t = kb + BN - 1 > tmin, cross_lo = kb < lomax;
    if (!cross_t && !cross_lo) scores(std::integral_constant<int, 0>());
    else scores(std::integral_constant<int, 3>());
    float tmax = tr_max(sv[0], sv[1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) tmax = tr_max(tmax, tr_max(sv[r], sv[r + 1]));   // v_maximum3, no quieting
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
      tmax = tr_max(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    // Lazy rescale: x is relative to the running reference mref; it moves only when some
    // row's maximum exceeds it by more than kRescale (so p <= 2^kRescale in fp16), or on the
    // first visible key of a row.
    if (__any(tmax > thr)) {
      // Rows past their threshold move the reference to the tile maximum (a row's first visible
      // keys set it); the others keep theirs.  O and the sum need scaling only in rows that
      // already hold weight, and that part is skipped when no row of the wave does.
      const bool move = tmax > thr, first = (mref == -INFINITY);
      const float shift = move ? tmax : 0.0f;
      if (__any(move && !first)) {
        const float corr = first ? 1.0f : exp2f(-shift);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[mt][r] *= corr;
        lsum *= corr;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[r] -= shift;
      if (move) mref = first ? tmax : mref + tmax;
      const bool none = (mref == -INFINITY);
      nm = none ? 0.0f : -mref;
      thr = none ? -INFINITY : kRescale;
    }
    // p in fp16 (the PV operand); the row sum adds those same fp16 weights, two per v_dot2 with
    // an fp32 accumulator, so numerator and denominator use identical weights.
    f16x8 pk[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) pk[r >> 3][r & 7] = (_Float16)__builtin_amdgcn_exp2f(sv[r]);
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 one2 = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const f16x2 pp = {pk[r >> 3][r & 7], pk[r >> 3][(r & 7) + 1]};
      lsum = __builtin_amdgcn_fdot2(pp, one2, lsum, false);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const f16x8 av = *reinterpret_cast<const f16x8*>(&tl.vt[32 * mt + n][16 * kh + 8 * g]);
        o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, pk[kh], o[mt], 0, 0, 0);
      }
    }
  };

  if (ntiles > 0) store_tile(sm.tile[0]);
  if (ntiles > 1) load_tile(kb0 + BN);
  __syncthreads();
  // Key tile it sits in buffer it & 1; the loop is unrolled by two so that every LDS address is
  // a loop-invariant base plus a constant.  While tile it is computed, tile it + 1 (loaded one
  // step earlier) goes into the other buffer and the loads of tile it + 2 are issued.
  auto step = [&](int it, auto buf) {
    constexpr int b = decltype(buf)::value;
    const int kb = kb0 + it * BN;
    if (wave_live && kb < whi && kb + BN - 1 >= wlo) compute(sm.tile[b], kb);
    if (it + 1 < ntiles) store_tile(sm.tile[b ^ 1]);
    if (it + 2 < ntiles) load_tile(kb + 2 * BN);
    __syncthreads();
  };
  for (int it = 0; it < ntiles; it += 2) {
    step(it, std::integral_constant<int, 0>());
    if (it + 1 < ntiles) step(it + 1, std::integral_constant<int, 1>());
  }
  const float ltot = xor32_sum(lsum);
  if (!row_ok) return;
  if (slot >= 0) {
    // one chunk of a split tile: unnormalized O, reference max and sum of this row
    float* pr = part + (((int64_t)sh * kSlotsPerHead + slot) * BM + (ri - r0)) * (D + 4);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = 32 * mt + 8 * j + 4 * g;
        *reinterpret_cast<float4*>(pr + d0) = make_float4(o[mt][4 * j], o[mt][4 * j + 1], o[mt][4 * j + 2],
                                                          o[mt][4 * j + 3]);
      }
    }
    if (g == 0) *reinterpret_cast<float2*>(pr + D) = make_float2(mref, ltot);
    return;
  }
  const float inv = 1.0f / ltot;
  uint16_t* orow = out + (((int64_t)s * T + i) * HQ + h) * D;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * mt + 8 * j + 4 * g;
      uint2 w;
      w.x = (uint32_t)tr_f32_to_bf16(o[mt][4 * j + 0] * inv) | ((uint32_t)tr_f32_to_bf16(o[mt][4 * j + 1] * inv) << 16);
      w.y = (uint32_t)tr_f32_to_bf16(o[mt][4 * j + 2] * inv) | ((uint32_t)tr_f32_to_bf16(o[mt][4 * j + 3] * inv) << 16);
      *reinterpret_cast<uint2*>(orow + d0) = w;
    }
  }
}

// Merge of the chunks of split tiles: per row, out = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c.
// A partial row is D + 4 floats: O[D], then the reference max and the sum (16-byte aligned rows).
// Chunks go in pairs: both chunks' loads are issued together (the second clamped to the last
// chunk and weighted 0 when past it), and pairs fold into a running (max, num, den).
template <int D>
__global__ __launch_bounds__(kBlock) void k_prefill_merge(CacheLayout c, int T, const int32_t* __restrict__ rows,
                                                          const int32_t* __restrict__ counts,
                                                          const int4* __restrict__ merges, const float* __restrict__ part,
                                                          uint16_t* __restrict__ out, int HQ) {
  constexpr int MPH = kSlotsPerHead / 2;
  constexpr int TPR = kBlock / BM;                 // threads per row
  constexpr int CPT = D / TPR;                     // channels per thread
  constexpr int64_t SLOT = (int64_t)BM * (D + 4);
  const int BH = c.B * HQ;
  const int mi = blockIdx.x / BH, sh = blockIdx.x % BH;
  const int s = sh / HQ, h = sh % HQ;
  {
    // The head's skip rows (listed after its full and local rows) get their zeros here: whole
    // 2D-byte output rows per group of D / 8 threads, the list split over the head's workgroups.
    constexpr int TPZ = D / 8, RPI = kBlock / TPZ;
    const int nfull = counts[sh * 4 + 0], nl = counts[sh * 4 + 1], nskip = T - nfull - nl;
    const int per = (nskip + MPH - 1) / MPH, k1 = min(nskip, (mi + 1) * per);
    const int32_t* sl = rows + (int64_t)sh * c.pfN + nfull + nl;
    for (int k = mi * per + (int)threadIdx.x / TPZ; k < k1; k += RPI)
      reinterpret_cast<uint4*>(out + (((int64_t)s * T + sl[k]) * HQ + h) * D)[threadIdx.x % TPZ] = make_uint4(0, 0, 0, 0);
  }
  if (mi >= counts[sh * 4 + 3]) return;
  const int4 mg = merges[(int64_t)sh * MPH + mi];
  const int r = threadIdx.x / TPR, d0 = (threadIdx.x % TPR) * CPT;
  const int ri = mg.x + r;
  if (ri >= mg.y) return;
  const float* base = part + ((int64_t)sh * kSlotsPerHead + mg.z) * SLOT + (int64_t)r * (D + 4);
  const int nch = mg.w;
  float M = -INFINITY, den = 0.0f;
  float acc[CPT];
#pragma unroll
  for (int x = 0; x < CPT; ++x) acc[x] = 0.0f;
  for (int k0 = 0; k0 < nch; k0 += 2) {
    const float* p0 = base + k0 * SLOT;
    const float* p1 = base + min(k0 + 1, nch - 1) * SLOT;
    float v0[CPT], v1[CPT];
#pragma unroll
    for (int x = 0; x < CPT; x += 4) {
      const float4 a0 = *reinterpret_cast<const float4*>(p0 + d0 + x);
      const float4 a1 = *reinterpret_cast<const float4*>(p1 + d0 + x);
      v0[x] = a0.x; v0[x + 1] = a0.y; v0[x + 2] = a0.z; v0[x + 3] = a0.w;
      v1[x] = a1.x; v1[x + 1] = a1.y; v1[x + 2] = a1.z; v1[x + 3] = a1.w;
    }
    const float2 ml0 = *reinterpret_cast<const float2*>(p0 + D);
    const float2 ml1 = *reinterpret_cast<const float2*>(p1 + D);
    const bool two = k0 + 1 < nch;
    const float m1 = two ? ml1.x : -INFINITY;
    const float Mn = fmaxf(M, fmaxf(ml0.x, m1));
    const float a = (M == -INFINITY) ? 0.0f : exp2f(M - Mn);
    const float w0 = (ml0.x == -INFINITY) ? 0.0f : exp2f(ml0.x - Mn);
    const float w1 = (m1 == -INFINITY) ? 0.0f : exp2f(m1 - Mn);
    den = den * a + fmaf(w0, ml0.y, w1 * ml1.y);
#pragma unroll
    for (int x = 0; x < CPT; ++x) acc[x] = acc[x] * a + fmaf(w0, v0[x], w1 * v1[x]);
    M = Mn;
  }
  const float inv = 1.0f / den;
  const int i = rows[(int64_t)sh * c.pfN + ri];
  uint16_t* orow = out + (((int64_t)s * T + i) * HQ + h) * D + d0;
#pragma unroll
  for (int x = 0; x < CPT; x += 4) {
    uint2 w;
    w.x = (uint32_t)tr_f32_to_bf16(acc[x] * inv) | ((uint32_t)tr_f32_to_bf16(acc[x + 1] * inv) << 16);
    w.y = (uint32_t)tr_f32_to_bf16(acc[x + 2] * inv) | ((uint32_t)tr_f32_to_bf16(acc[x + 3] * inv) << 16);
    *reinterpret_cast<uint2*>(orow + x) = w;
  }
}

}  // namespace

namespace {

// Quantize-write of positions [p0, p0 + T) in 64-position tiles (slots already assigned); tiles
// from dense_from on are also staged for the prefill attention.
template <int D>
tr_status launch_write_tiles(tr_kv_cache* c, int layer, int p0, const uint16_t* k, const uint16_t* v,
                             const uint8_t* bits, int T, int dense_from, hipStream_t stream) {
  const CacheLayout& L = c->lay;
  const float kscale = (float)(1.4426950408889634 / sqrt((double)D));
  const int tile0 = p0 / kWriteTile, ntile = (p0 + T + kWriteTile - 1) / kWriteTile - tile0;
  const int64_t blocks = (int64_t)L.B * L.H * ntile;
  if (blocks > (int64_t)1 << 30) return TR_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(k_prefill_write<D>, dim3(tr_xcd_grid((int)blocks)), dim3(4 * D), 0, stream, L, layer, p0, T, tile0,
                     ntile, dense_from, c->np, kscale, k, v, bits, c->dk, c->dv, c->dkf);
  TR_LAUNCH_CHECK();
  return TR_OK;
}

template <int D>
tr_status prefill_launch_d(tr_kv_cache* c, int layer, int p0, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const uint8_t* bits, const uint8_t* mode, int T, int window,
                           uint16_t* out, hipStream_t stream) {
  const CacheLayout& L = c->lay;
  const int BH = L.B * L.H;              // (seq, KV head): dense staging
  const int BQ = L.B * c->hq;            // (seq, query head): compaction, attention, merge
  const float kscale = (float)(1.4426950408889634 / sqrt((double)D));
  const int uph = tr_prefill_units_per_head(T);
  if (p0 + T > L.pfN || uph > c->pf_uph) return TR_ERR_UNSUPPORTED;
  const int pend = p0 + T;
  // Short calls take the one-launch append and stage every dense tile from the pages; longer
  // ones assign their slots beside the row compaction, then quantize and stage their own
  // positions in one pass (the dense pass keeps the tiles that hold earlier positions).
  const bool fused = T > 64;
  const int write_from = (p0 + kWriteTile - 1) / kWriteTile;      // first tile k_prefill_write stages
  const int dense_to = fused ? min((pend + 31) / 32, write_from * (kWriteTile / 32)) : (pend + 31) / 32;
  if (!fused) {
    const tr_status st = tr_write_launch(c, layer, p0, k, v, bits, T, stream);
    if (st != TR_OK) return st;
  }
  {
    TrProfScope prof(c, TR_PROF_PREFILL_COMPACT, stream);
    hipLaunchKernelGGL(k_prefill_prep<D>, dim3(BQ + (fused ? L.B : 0)), dim3(TR_ASSIGN_THREADS), 0, stream, L, layer,
                       p0, T, window, mode, bits, c->rows, c->row_counts, c->pf_units, c->pf_merges, c->pf_uph, c->hq);
    TR_LAUNCH_CHECK();
  }
  if (fused) {
    TrProfScope prof(c, TR_PROF_WRITE, stream);
    const tr_status st = launch_write_tiles<D>(c, layer, p0, k, v, bits, T, write_from, stream);
    if (st != TR_OK) return st;
  }
  if (dense_to > 0) {
    TrProfScope prof(c, TR_PROF_PREFILL_COMPACT, stream);
    hipLaunchKernelGGL(k_prefill_dense<D>, dim3(tr_xcd_grid(BH * dense_to)), dim3(kBlock), 0, stream, L, layer, 0, dense_to, pend,
                       c->np, kscale, c->dk, c->dv, c->dkf);
    TR_LAUNCH_CHECK();
  }
  {
    TrProfScope prof(c, TR_PROF_PREFILL_ATTN, stream);
    hipLaunchKernelGGL(k_prefill_attn<D>, dim3(BQ * uph), dim3(kBlock), 0,
                       stream, L, p0, T, window, c->np, q, c->rows, c->row_counts, c->pf_units, c->pf_uph, c->dk, c->dv,
                       c->dkf, c->pf_part, out, c->hq, c->grp);
    TR_LAUNCH_CHECK();
  }
  TrProfScope prof(c, TR_PROF_PREFILL_MERGE, stream);
  hipLaunchKernelGGL(k_prefill_merge<D>, dim3(BQ * (kSlotsPerHead / 2)), dim3(kBlock), 0, stream, L, T, c->rows,
                     c->row_counts, c->pf_merges, c->pf_part, out, c->hq);
  TR_LAUNCH_CHECK();
  return TR_OK;
}

}  // namespace

tr_status tr_prefill_launch(tr_kv_cache* c, int layer, int p0, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, const uint8_t* bits, const uint8_t* mode, int T, int window,
                            uint16_t* out, hipStream_t stream) {
  if (c->lay.D == 64) return prefill_launch_d<64>(c, layer, p0, q, k, v, bits, mode, T, window, out, stream);
  return prefill_launch_d<128>(c, layer, p0, q, k, v, bits, mode, T, window, out, stream);
}

tr_status tr_write_tiles_launch(tr_kv_cache* c, int layer, int p0, const uint16_t* k, const uint16_t* v,
                                const uint8_t* bits, int n, hipStream_t stream) {
  if (c->lay.D == 64) return launch_write_tiles<64>(c, layer, p0, k, v, bits, n, 1 << 30, stream);
  return launch_write_tiles<128>(c, layer, p0, k, v, bits, n, 1 << 30, stream);
}
