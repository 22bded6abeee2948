// Decode routed attention over the mixed-width paged cache (TriRoute review page,
// xllm-io.github.io: Eq. (2) modes read by a query; Eq. (4) codes written per token).
//
// One query per (sequence, query head) at position t, reading the K/V of its KV head
// (query head h reads KV head h / G with G query heads per KV head; G = 1 is plain multi-head
// attention).  Its key set is the position window
// [lo, t] (lo = 0 for full, max(0, t - w) for local; skip heads read nothing).  The window is
// split into position chunks (split-K); every chunk maps, through the per-position class
// prefix counts, to one contiguous slot range per width class, so out-of-window keys are
// never read and each inner loop runs over a single width (wave-uniform unpacking).
//
// k_decode: one wavefront = one workgroup = one (seq, query head, chunk) work item, with no
// cross-wave synchronization, so every wave streams independently.
//   prologue the chunk's page ids of every class and q -> LDS.
//   phase 1  K codes -> scores in LDS.  Each lane takes a 16/32-byte slice of a key row;
//            batches of keys are software-pipelined (the next batch is in flight while the
//            current one is computed).  2- and 4-bit codes become bf16 (128 + c) by an OR
//            into the mantissa and go through v_dot2_f32_bf16 with bf16 q pairs; 8-bit codes
//            use byte converts and fp32 FMA; bf16 keys use v_dot2 directly.  Partial dots are
//            reduced across the lanes of the key.  The zero point folds out as
//            s * (q . c) + z * sum(q) (an exact identity of Eq. (4)'s reconstruction); scores
//            are kept in the log2 domain.
//   softmax  chunk max m, p = 2^(score - m), l = sum p (fp32).
//   phase 2  V codes, pipelined the same way: each lane owns 32 fixed channels of a key, so
//            all width classes accumulate into the same 32 fp32 registers:
//            acc += (p * s_v) * c, plus sum(p * z_v) once per key.
//   epilogue a one-chunk window writes bf16 out directly; otherwise the chunk writes
//            (o[D], m, l).  Skip heads: chunk 0 writes zeros.
// k_decode_combine: log-sum-exp merge of multi-chunk windows -> bf16.
#include <math.h>

#include <mutex>

#include "common.h"

namespace {

constexpr int kWave = 64;
constexpr int kItemMax = TR_DECODE_ITEM_MAX;
constexpr int kPgMax = TR_DECODE_PG_MAX;
constexpr int kMinChunk = TR_DECODE_MIN_CHUNK;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// A constant hidden from the compiler in an SGPR / a VGPR, so that (x & m) | c is emitted as one
// v_and_or_b32 (gfx9 VOP3 takes no literal operands; left visible, the compiler splits it into
// an AND and an OR with literals).
__device__ __forceinline__ uint32_t opaque_s(uint32_t x) {
  __asm__("" : "+s"(x));
  return x;
}
__device__ __forceinline__ uint32_t opaque_v(uint32_t x) {
  __asm__("" : "+v"(x));
  return x;
}

// Class-0 (2-bit) keys as bf16 dot operands.  Pair k of a code word holds elements (k, k + 8) of
// its 16 (bits 2k and 16 + 2k).  Fields 0-2 are masked in place, fields 3-5 after w >> 6, fields
// 6-7 after w >> 12, and ORed into bf16 128.0's mantissa: pair k then reads 128 + c * 4^(k % 3),
// exactly, with two shifts per word.  The q pair k is scaled by 4^-(k % 3) to match (exact in
// bf16), so the dot is sum(c q) + 128 * sum(q 4^-(k % 3)).
__device__ __forceinline__ float q_scale_k2(int k) { return k % 3 == 0 ? 1.0f : k % 3 == 1 ? 0.25f : 0.0625f; }

template <int NP>
__device__ __forceinline__ float dot_k2_word(uint32_t w, const uint32_t* qp, float acc, uint32_t m0, uint32_t m1,
                                             uint32_t m2, uint32_t ob) {
  const uint32_t w6 = w >> 6, w12 = w >> 12;
  acc = dot2((w & m0) | ob, qp[0], acc);
  acc = dot2((w & m1) | ob, qp[1], acc);
  acc = dot2((w & m2) | ob, qp[2], acc);
  acc = dot2((w6 & m0) | ob, qp[3], acc);
  acc = dot2((w6 & m1) | ob, qp[4], acc);
  acc = dot2((w6 & m2) | ob, qp[5], acc);
  acc = dot2((w12 & m0) | ob, qp[6], acc);
  acc = dot2((w12 & m1) | ob, qp[7], acc);
  return acc;
}

// bf16 bit pattern of a float that holds a bf16 value (q is bf16 on input, so this is exact).
__device__ __forceinline__ uint32_t bf16_bits(float x) { return __float_as_uint(x) >> 16; }

// Cross-lane sums and maxima without LDS: DPP inside rows of 16 lanes (quad_perm 1,0,3,2 and
// 2,3,0,1; row_half_mirror; row_mirror; row_ror 4 and 8), v_permlane16_swap / v_permlane32_swap
// across rows and halves.  Each swap hands every lane its partner's value (l ^ 16, l ^ 32) in one
// of its two results, so combining both results gives the pairwise reduction in every lane.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float sum16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Sum over each group of N adjacent lanes (N = 1, 2, 4, 8, 16), result in every lane of it.
template <int N>
__device__ __forceinline__ float sum_adjacent(float v) {
  if constexpr (N >= 2) v += dpp_f<0xB1>(v);
  if constexpr (N >= 4) v += dpp_f<0x4E>(v);
  if constexpr (N >= 8) v += dpp_f<0x141>(v);
  if constexpr (N >= 16) v += dpp_f<0x140>(v);
  return v;
}
// Sum over the lanes l' = l mod S (S = 1, 2, 4, 8): all 64 / S lanes of one residue.
template <int S>
__device__ __forceinline__ float sum_strided(float v) {
  if constexpr (S == 1) v = sum_adjacent<2>(v);
  if constexpr (S <= 2) v += dpp_f<0x4E>(v);
  if constexpr (S <= 4) v += dpp_f<0x124>(v);
  v += dpp_f<0x128>(v);
  return sum32(sum16(v));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return max32(max16(v));
}

__device__ __forceinline__ float wave_sum(float v) { return sum_strided<1>(v); }

// Codes of b bits, element e of a little-endian packed slice, as floats, in groups that map to
// byte converts: for b = 2 the mask (w >> 2k) & 0x03030303 holds elements 4i + k in byte i;
// b = 4: (w >> 4k) & 0x0f0f0f0f holds 2i + k; b = 8: byte i is element i.
template <int B, int NW>
__device__ __forceinline__ void unpack_codes(const uint32_t* w, float* out) {
#pragma unroll
  for (int d = 0; d < NW; ++d) {
    if constexpr (B == 2) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t m = (w[d] >> (2 * k)) & 0x03030303u;
#pragma unroll
        for (int i = 0; i < 4; ++i) out[16 * d + 4 * i + k] = (float)((m >> (8 * i)) & 0xffu);
      }
    } else if constexpr (B == 4) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t m = (w[d] >> (4 * k)) & 0x0f0f0f0fu;
#pragma unroll
        for (int i = 0; i < 4; ++i) out[8 * d + 2 * i + k] = (float)((m >> (8 * i)) & 0xffu);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) out[4 * d + i] = (float)((w[d] >> (8 * i)) & 0xffu);
    }
  }
}

// Codes of b = 2 or 4 bits as floats c * 4^k (b = 2, element 4i + k of a word) or c * 16^k
// (b = 4, element 2i + k): each word is masked in place (one AND per field) and its bytes go
// through v_cvt_f32_ubyte0..3; the caller scales its weights by 4^-k / 16^-k (exact).  The
// masked word is hidden from the compiler, which would otherwise re-derive every element with
// a bit-field extract of its own.
template <int B, int NW>
__device__ __forceinline__ void unpack_codes_scaled(const uint32_t* w, float* out) {
#pragma unroll
  for (int d = 0; d < NW; ++d) {
    if constexpr (B == 2) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t m = w[d] & (0x03030303u << (2 * k));
        __asm__("" : "+v"(m));
#pragma unroll
        for (int i = 0; i < 4; ++i) out[16 * d + 4 * i + k] = (float)((m >> (8 * i)) & 0xffu);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        uint32_t m = w[d] & (0x0f0f0f0fu << (4 * k));
        __asm__("" : "+v"(m));
#pragma unroll
        for (int i = 0; i < 4; ++i) out[8 * d + 2 * i + k] = (float)((m >> (8 * i)) & 0xffu);
      }
    }
  }
}

// Weight factor of element e of a scaled unpack: 4^-(e % 4) (b = 2) or 16^-(e % 2) (b = 4).
template <int B>
__device__ __forceinline__ float unpack_scale(int e) {
  if constexpr (B == 2) return e % 4 == 0 ? 1.0f : e % 4 == 1 ? 0.25f : e % 4 == 2 ? 0.0625f : 0.015625f;
  else return e % 2 == 0 ? 1.0f : 0.0625f;
}

template <int NW>
__device__ __forceinline__ void load_words(const uint8_t* p, uint32_t* w) {
  if constexpr (NW == 1) {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (NW == 2) {
    const uint2 t = *reinterpret_cast<const uint2*>(p);
    w[0] = t.x; w[1] = t.y;
  } else {
#pragma unroll
    for (int x = 0; x < NW / 4; ++x) {
      const uint4 t = reinterpret_cast<const uint4*>(p)[x];
      w[4 * x] = t.x; w[4 * x + 1] = t.y; w[4 * x + 2] = t.z; w[4 * x + 3] = t.w;
    }
  }
}

// One batch of U keys (one sub-iteration of KPW keys per u) of class C: codes and (s, z).
template <int U, int NW, bool SIDE>
struct Batch {
  uint32_t w[U][NW];
  float2 sz[U];
};

template <int U, int NW, bool SIDE, int LPK>
__device__ __forceinline__ void load_batch(Batch<U, NW, SIDE>& bt, const CacheLayout& c, const int32_t* pg, int first,
                                           int lp, int pm, int base, int e, int kslot, int64_t code_off,
                                           int64_t side_off, int rowb) {
  constexpr int KPW = kWave / LPK;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = min(base + u * KPW + kslot, e - 1);    // clamped: loads never branch
    const int page = pg[(j >> lp) - first];
    const int slot = j & pm;
    const uint8_t* pb = c.pool + (int64_t)page * c.page_bytes;
    load_words<NW>(pb + code_off + (int64_t)slot * rowb, bt.w[u]);
    if constexpr (SIDE) bt.sz[u] = reinterpret_cast<const float2*>(pb + side_off)[slot];
  }
}

// Phase 1 for width class C over class slots [a, e): scores into sc[off + (j - a)].
// Lane slices: 16 bytes (b = 2, 4, 8) or 32 bytes (b = 16) of one key row.
//   b = 2, 4: code pairs are ORed into bf16 mantissas (value 128 + c, exact) and dotted with
//             bf16 q pairs by v_dot2_f32_bf16; the 128 * sum(q) offset is removed with the
//             zero point: score = s * dot + (z - 128 s) * sum(q).
//   b = 8:    byte converts and fp32 FMA.
//   b = 16:   native bf16 pairs straight into v_dot2_f32_bf16.
template <int D, int C>
__device__ __forceinline__ void score_phase(const CacheLayout& c, const int32_t* pg, int first, int h, int a, int e,
                                            int off, const float* qs, float sigma, float sig0, float kscale,
                                            float* sc) {
  constexpr int b = 2 << C;
  constexpr int SB = (C == 3) ? 32 : 16;           // slice bytes per lane per key
  constexpr int E = SB * 8 / b;                    // elements per lane
  constexpr int LPK = D * b / 8 / SB;              // lanes per key
  constexpr int KPW = kWave / LPK;                 // keys per wave sub-iteration
  constexpr int NW = SB / 4;
#ifndef TR_DECODE_U1
#define TR_DECODE_U1 2
#endif
#ifndef TR_DECODE_UK3
#define TR_DECODE_UK3 4                            // bf16 keys: 4 x 8 keys (8 KB) per batch
#endif
  constexpr int U = (C == 3) ? TR_DECODE_UK3 : TR_DECODE_U1;   // sub-iterations per batch
  constexpr int NQ = (C == 2) ? 1 : E / 2;
  const int lane = threadIdx.x;
  const int part = lane % LPK, kslot = lane / LPK;
  const float* qv = qs + part * E;
  uint32_t qp[NQ];
  float qf[(C == 2) ? E : 1];
  if constexpr (C == 0) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int k = 0; k < 8; ++k)
        qp[8 * d + k] = bf16_bits(qv[16 * d + k] * q_scale_k2(k)) | (bf16_bits(qv[16 * d + k + 8] * q_scale_k2(k)) << 16);
  } else if constexpr (C == 1) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int k = 0; k < 4; ++k) qp[4 * d + k] = bf16_bits(qv[8 * d + k]) | (bf16_bits(qv[8 * d + k + 4]) << 16);
  } else if constexpr (C == 2) {
#pragma unroll
    for (int k = 0; k < E; ++k) qf[k] = qv[k];
  } else {
#pragma unroll
    for (int k = 0; k < NQ; ++k) qp[k] = bf16_bits(qv[2 * k]) | (bf16_bits(qv[2 * k + 1]) << 16);
  }
  const int lp = c.ptok_log2[C], pm = c.ptok[C] - 1;
  const int64_t code_off = c.k_off[C] + (int64_t)h * c.cb + part * SB;
  const int64_t side_off = c.sk_off[C] + (int64_t)h * c.ptok[C] * 8;
  constexpr int RB = D * b / 8;
  constexpr int STEP = KPW * U;
  const uint32_t ob = opaque_v(0x43004300u);
  const uint32_t m0 = opaque_s(C == 0 ? 0x00030003u : 0x000f000fu), m1 = opaque_s(0x000c000cu),
                 m2 = opaque_s(0x00300030u);
  Batch<U, NW, (C < 3)> cur, nxt;
  load_batch<U, NW, (C < 3), LPK>(cur, c, pg, first, lp, pm, a, e, kslot, code_off, side_off, RB);
  for (int base = a; base < e; base += STEP) {
    if (base + STEP < e) load_batch<U, NW, (C < 3), LPK>(nxt, c, pg, first, lp, pm, base + STEP, e, kslot, code_off,
                                                        side_off, RB);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (base + u * KPW >= e) break;              // past the class's last key: nothing to compute
      float dot = 0.0f;
      if constexpr (C == 0) {
#pragma unroll
        for (int d = 0; d < 4; ++d) dot = dot_k2_word<8>(cur.w[u][d], qp + 8 * d, dot, m0, m1, m2, ob);
      } else if constexpr (C == 1) {
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int k = 0; k < 4; ++k) dot = dot2(((cur.w[u][d] >> (4 * k)) & m0) | ob, qp[4 * d + k], dot);
      } else if constexpr (C == 2) {
        float cf[E];
        unpack_codes<8, NW>(cur.w[u], cf);
#pragma unroll
        for (int k = 0; k < E; ++k) dot = fmaf(qf[k], cf[k], dot);
      } else {
#pragma unroll
        for (int k = 0; k < NW; ++k) dot = dot2(cur.w[u][k], qp[k], dot);
      }
      dot = sum_adjacent<LPK>(dot);
      const int j = base + u * KPW + kslot;
      if (j < e && part == 0) {
        float x;
        if constexpr (C == 0) x = fmaf(cur.sz[u].x, dot, fmaf(-128.0f * cur.sz[u].x, sig0, cur.sz[u].y * sigma));
        else if constexpr (C == 1) x = fmaf(cur.sz[u].x, dot, fmaf(-128.0f, cur.sz[u].x, cur.sz[u].y) * sigma);
        else if constexpr (C == 2) x = fmaf(cur.sz[u].x, dot, cur.sz[u].y * sigma);
        else x = dot;
        sc[off + (j - a)] = x * kscale;
      }
    }
    cur = nxt;
  }
}

// Phase 2 for width class C: acc[32] (channels 32*part ..) += p * v_hat.
template <int D, int C>
__device__ __forceinline__ void value_phase(const CacheLayout& c, const int32_t* pg, int first, int h, int a, int e,
                                            int off, const float* pw, float* acc, float& zacc) {
  constexpr int b = 2 << C;
  constexpr int VLPK = D / 32;                     // lanes per key
  constexpr int KPW = kWave / VLPK;
  constexpr int NW = b;                            // 32 codes of b bits = b words
#ifndef TR_DECODE_U2
#define TR_DECODE_U2 2
#endif
#ifndef TR_DECODE_UV
#define TR_DECODE_UV 1
#endif
#ifndef TR_DECODE_UV3
#define TR_DECODE_UV3 1
#endif
  constexpr int U = (C == 0) ? TR_DECODE_U2 : (C == 3) ? TR_DECODE_UV3 : TR_DECODE_UV;
  constexpr int RB = D * b / 8;
  constexpr int STEP = KPW * U;
  const int lane = threadIdx.x;
  const int part = lane % VLPK, kslot = lane / VLPK;
  const int lp = c.ptok_log2[C], pm = c.ptok[C] - 1;
  const int64_t code_off = c.v_off[C] + (int64_t)h * c.cb + part * (4 * b);
  const int64_t side_off = c.sv_off[C] + (int64_t)h * c.ptok[C] * 8;
  Batch<U, NW, (C < 3)> cur, nxt;
  load_batch<U, NW, (C < 3), VLPK>(cur, c, pg, first, lp, pm, a, e, kslot, code_off, side_off, RB);
  for (int base = a; base < e; base += STEP) {
    if (base + STEP < e) load_batch<U, NW, (C < 3), VLPK>(nxt, c, pg, first, lp, pm, base + STEP, e, kslot,
                                                         code_off, side_off, RB);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (base + u * KPW >= e) break;              // past the class's last key
      const int jr = base + u * KPW + kslot;
      const float p = (jr < e) ? pw[off + (min(jr, e - 1) - a)] : 0.0f;
      if constexpr (C < 2) {
        const float ps = p * cur.sz[u].x;
        if (part == 0) zacc = fmaf(p, cur.sz[u].y, zacc);
        float cf[32];
        unpack_codes_scaled<b, NW>(cur.w[u], cf);
#pragma unroll
        for (int k = 0; k < 32; ++k) acc[k] = fmaf(ps * unpack_scale<b>(k), cf[k], acc[k]);
      } else if constexpr (C == 2) {
        const float ps = p * cur.sz[u].x;
        if (part == 0) zacc = fmaf(p, cur.sz[u].y, zacc);
        float cf[32];
        unpack_codes<b, NW>(cur.w[u], cf);
#pragma unroll
        for (int k = 0; k < 32; ++k) acc[k] = fmaf(ps, cf[k], acc[k]);
      } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          acc[2 * k] = fmaf(p, tr_bf16_lo(cur.w[u][k]), acc[2 * k]);
          acc[2 * k + 1] = fmaf(p, tr_bf16_hi(cur.w[u][k]), acc[2 * k + 1]);
        }
      }
    }
    cur = nxt;
  }
}

// Occupancy floor handed to the compiler.  With 4 it settles at 96 VGPRs for D = 128 (5 waves per
// SIMD, no spills; a 1.3B-shaped decode has ~4100 items for 5120 wave slots) and at 120 for D = 64.
#ifndef TR_DECODE_WAVES
#define TR_DECODE_WAVES 4
#endif
template <int D>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(TR_DECODE_WAVES, 8))) void k_decode(CacheLayout c, int layer, int t, int window, int CH, int nch_grid,
                                                  int max_chunks, float kscale, const uint16_t* __restrict__ q,
                                                  const uint8_t* __restrict__ mode, float* __restrict__ part,
                                                  uint16_t* __restrict__ out, int HQ, int G) {
  __shared__ float qs[D];
  __shared__ float sc[kItemMax];
  __shared__ int32_t pg[TR_NCLASS][kPgMax];
  const int lane = threadIdx.x;
  const int k = blockIdx.x % nch_grid;
  const int sh = blockIdx.x / nch_grid;             // (seq, query head)
  const int s = sh / HQ, h = (sh % HQ) / G;         // sequence, KV head it reads
  const int m = mode[sh];
  uint16_t* o = out + (int64_t)sh * D;
  if (m != TR_MODE_LOCAL && m != TR_MODE_FULL) {
    if (k == 0) {
#pragma unroll
      for (int d = lane; d < D; d += kWave) o[d] = 0;
      if (lane == 0 && m != TR_MODE_SKIP) atomicOr(c.err, TR_ERRF_BAD_MODE);
    }
    return;
  }
  const int lo = (m == TR_MODE_FULL) ? 0 : max(0, t - window);
  const int L = t + 1 - lo;
  const int nch = (L + CH - 1) / CH;
  if (k >= nch) return;
  const int per = (L + nch - 1) / nch;
  const int p0 = lo + k * per, p1 = min(p0 + per, t + 1);

  const int32_t* pa = tr_prefix_row(c, layer, s, p0);
  const int32_t* pe = tr_prefix_row(c, layer, s, p1);
  int a[4], e[4], off[4], first[4];
  int nk = 0;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    a[x] = pa[x];
    e[x] = pe[x];
    off[x] = nk;
    nk += e[x] - a[x];
    first[x] = a[x] >> c.ptok_log2[x];
  }
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    if (e[x] > a[x]) {
      const int np = ((e[x] - 1) >> c.ptok_log2[x]) - first[x] + 1;
      const int32_t* pt = tr_ptab(c, layer, s, x) + first[x];
      for (int i = lane; i < np; i += kWave) pg[x][i] = pt[i];
    }
  }
  float qpart = 0.0f, qpart0 = 0.0f;
#pragma unroll
  for (int d = lane; d < D; d += kWave) {
    const float v = tr_bf16_lo((uint32_t)q[(int64_t)sh * D + d]);
    qs[d] = v;
    qpart += v;
    qpart0 += v * q_scale_k2(d & 7);              // channel d sits in pair (d & 7) of its 16
  }
  const float sigma = wave_sum(qpart), sig0 = wave_sum(qpart0);
  __syncthreads();

  if (e[0] > a[0]) score_phase<D, 0>(c, pg[0], first[0], h, a[0], e[0], off[0], qs, sigma, sig0, kscale, sc);
  if (e[1] > a[1]) score_phase<D, 1>(c, pg[1], first[1], h, a[1], e[1], off[1], qs, sigma, sig0, kscale, sc);
  if (e[2] > a[2]) score_phase<D, 2>(c, pg[2], first[2], h, a[2], e[2], off[2], qs, sigma, sig0, kscale, sc);
  if (e[3] > a[3]) score_phase<D, 3>(c, pg[3], first[3], h, a[3], e[3], off[3], qs, sigma, sig0, kscale, sc);
  __syncthreads();

  float mx = -INFINITY;
  for (int i = lane; i < nk; i += kWave) mx = fmaxf(mx, sc[i]);
  mx = wave_max(mx);
  float lsum = 0.0f;
  for (int i = lane; i < nk; i += kWave) {
    const float p = exp2f(sc[i] - mx);
    sc[i] = p;
    lsum += p;
  }
  lsum = wave_sum(lsum);
  __syncthreads();

  float acc[32];
#pragma unroll
  for (int x = 0; x < 32; ++x) acc[x] = 0.0f;
  float zacc = 0.0f;
  if (e[0] > a[0]) value_phase<D, 0>(c, pg[0], first[0], h, a[0], e[0], off[0], sc, acc, zacc);
  if (e[1] > a[1]) value_phase<D, 1>(c, pg[1], first[1], h, a[1], e[1], off[1], sc, acc, zacc);
  if (e[2] > a[2]) value_phase<D, 2>(c, pg[2], first[2], h, a[2], e[2], off[2], sc, acc, zacc);
  if (e[3] > a[3]) value_phase<D, 3>(c, pg[3], first[3], h, a[3], e[3], off[3], sc, acc, zacc);

  // Sum over the key slots (lanes with the same channel group); lane p < VLPK then holds
  // channels [32 p, 32 p + 32).
  constexpr int VLPK = D / 32;
#pragma unroll
  for (int x = 0; x < 32; ++x) acc[x] = sum_strided<VLPK>(acc[x]);
  zacc = wave_sum(zacc);
  if (nch == 1) {                                  // whole window in this chunk
    if (lane < VLPK) {
      const float inv = 1.0f / lsum;
      uint32_t pk[16];
#pragma unroll
      for (int x = 0; x < 16; ++x)
        pk[x] = (uint32_t)tr_f32_to_bf16((acc[2 * x] + zacc) * inv) |
                ((uint32_t)tr_f32_to_bf16((acc[2 * x + 1] + zacc) * inv) << 16);
      uint4* dst = reinterpret_cast<uint4*>(o + 32 * lane);
#pragma unroll
      for (int x = 0; x < 4; ++x) dst[x] = make_uint4(pk[4 * x], pk[4 * x + 1], pk[4 * x + 2], pk[4 * x + 3]);
    }
    return;
  }
  float* dst = part + ((int64_t)sh * max_chunks + k) * (D + 2);
  if (lane < VLPK) {
#pragma unroll
    for (int x = 0; x < 32; ++x) dst[32 * lane + x] = acc[x] + zacc;
  }
  if (lane == 0) {
    dst[D] = mx;
    dst[D + 1] = lsum;
  }
}

// Log-sum-exp merge of the chunks of windows that span more than one chunk: one workgroup per
// (seq, head), thread d = channel d.  Chunks go in batches of 32: every load of a batch -- the
// channel's 32 partial values and, in lane k of each wave, chunk k's (max, sum) -- is issued at
// once (indices clamped into the window), then the batch folds into a running (max, num, den)
// with the chunk weights broadcast from their lanes.
template <int D>
__global__ __launch_bounds__(D) void k_decode_combine(int t, int window, int CH, int max_chunks,
                                                      const uint8_t* __restrict__ mode,
                                                      const float* __restrict__ part, uint16_t* __restrict__ out) {
  constexpr int KB = 32;
  const int sh = blockIdx.x;
  const int d = threadIdx.x, lane = d & 63;
  const int m = mode[sh];
  if (m != TR_MODE_LOCAL && m != TR_MODE_FULL) return;
  const int lo = (m == TR_MODE_FULL) ? 0 : max(0, t - window);
  const int L = t + 1 - lo;
  const int nch = (L + CH - 1) / CH;
  if (nch == 1) return;                            // written by k_decode
  const float* base = part + (int64_t)sh * max_chunks * (D + 2);
  float M = -INFINITY, num = 0.0f, den = 0.0f;
  for (int k0 = 0; k0 < nch; k0 += KB) {
    float v[KB];
#pragma unroll
    for (int x = 0; x < KB; ++x) v[x] = base[(int64_t)min(k0 + x, nch - 1) * (D + 2) + d];
    const int kk = k0 + (lane & (KB - 1));
    const float* pk = base + (int64_t)min(kk, nch - 1) * (D + 2);
    const bool own = kk < nch && lane < KB;        // lanes KB..63 repeat lanes 0..KB-1
    const float mk = own ? pk[D] : -INFINITY;
    const float lk = pk[D + 1];
    const float Mn = fmaxf(M, wave_max(mk));
    const float a = (M == -INFINITY) ? 0.0f : exp2f(M - Mn);
    const float wk = own ? exp2f(mk - Mn) : 0.0f;
    den = den * a + wave_sum(wk * lk);
    float nb = 0.0f;
#pragma unroll
    for (int x = 0; x < KB; ++x)
      nb = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk), x)), v[x], nb);
    num = num * a + nb;
    M = Mn;
  }
  out[(int64_t)sh * D + d] = tr_f32_to_bf16(num / den);
}

}  // namespace

namespace {

// Chunks per window for a decode over n positions of BH (seq, query head) pairs with room for
// `limit` partial records per pair: about 8192 work items if every head were full (a few times
// the waves the chip holds at once), but no chunk below kMinChunk positions and none above the
// work item's limit; 0 if `limit` cannot hold the chunks a full window needs.
int decode_chunks(const tr_kv_cache* c, int n, int BH, int limit) {
  const int max_ch = tr_decode_max_chunk(c->lay);
  const int need = (n + max_ch - 1) / max_ch;      // fewest chunks a full window allows
  int nch = (8192 + BH - 1) / BH;
  if (nch > (n + kMinChunk - 1) / kMinChunk) nch = (n + kMinChunk - 1) / kMinChunk;
  if (nch < need) nch = need;
  if (nch > limit) nch = limit;
  if (nch < 1) nch = 1;
  if (c->force_chunks > 0) nch = c->force_chunks < n ? c->force_chunks : n;
  const int CH = (n + nch - 1) / nch;
  return (CH > max_ch || nch > limit) ? 0 : nch;
}

// The decode kernels with the split-K partial results in `part` (records of D + 2 floats,
// `stride` records per (seq, query head)).
tr_status decode_run(tr_kv_cache* c, int layer, const uint16_t* q, const uint8_t* mode, int window, uint16_t* out,
                     int nch, float* part, int stride, bool prof_ok, hipStream_t stream) {
  const CacheLayout& L = c->lay;
  const int t = c->len[layer] - 1;
  const int n = t + 1;
  const int BH = L.B * c->hq;                       // (seq, query head) pairs
  const int CH = (n + nch - 1) / nch;
  const float kscale = (float)(1.4426950408889634 / sqrt((double)L.D));
  const int grid = BH * nch;
  const bool prof_was = c->prof_on;
  c->prof_on = prof_was && prof_ok;
  tr_status st = TR_OK;
  {
    TrProfScope prof(c, TR_PROF_DECODE_SPLIT, stream);
    if (L.D == 64)
      hipLaunchKernelGGL(k_decode<64>, dim3(grid), dim3(kWave), 0, stream, L, layer, t, window, CH, nch, stride,
                         kscale, q, mode, part, out, c->hq, c->grp);
    else
      hipLaunchKernelGGL(k_decode<128>, dim3(grid), dim3(kWave), 0, stream, L, layer, t, window, CH, nch, stride,
                         kscale, q, mode, part, out, c->hq, c->grp);
    if (hipGetLastError() != hipSuccess) st = TR_ERR_HIP;
  }
  if (st == TR_OK && nch > 1) {
    TrProfScope prof(c, TR_PROF_DECODE_COMBINE, stream);
    if (L.D == 64)
      hipLaunchKernelGGL(k_decode_combine<64>, dim3(BH), dim3(64), 0, stream, t, window, CH, stride, mode, part, out);
    else
      hipLaunchKernelGGL(k_decode_combine<128>, dim3(BH), dim3(128), 0, stream, t, window, CH, stride, mode, part, out);
    if (hipGetLastError() != hipSuccess) st = TR_ERR_HIP;
  }
  c->prof_on = prof_was;
  return st;
}

}  // namespace

tr_status tr_decode_launch(tr_kv_cache* c, int layer, const uint16_t* q, const uint8_t* mode, int window,
                           uint16_t* out, hipStream_t stream) {
  const int n = c->len[layer];
  const int nch = decode_chunks(c, n, c->lay.B * c->hq, c->max_chunks);
  if (nch < 1) return TR_ERR_UNSUPPORTED;
  return decode_run(c, layer, q, mode, window, out, nch, c->partials, c->max_chunks, true, stream);
}

// ---------------------------------------------------------------------------------------------
// Decode without any allocation: the split-K partial results go to a file-scope device array
// instead of the cache's scratch.  Every device the library runs on holds its own copy of the
// array for the life of the process; host code reaches it only through the device address that
// hipGetSymbolAddress returns on that device (the array's name on the host is a stand-in, not a
// device address).

#define TR_NOALLOC_SCRATCH_BYTES (8u << 20)
static __device__ __align__(256) float scratch[TR_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices];                  // device address of `scratch` on each device

// Device address of this device's scratch, looked up once per device with it current.
tr_status scratch_of_current_device(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return TR_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return TR_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TR_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return TR_OK;
}

}  // namespace

tr_status tr_decode_noalloc_launch(tr_kv_cache* c, int layer, const uint16_t* q, const uint8_t* mode, int window,
                                   uint16_t* out, hipStream_t stream) {
  float* part = nullptr;
  const tr_status st = scratch_of_current_device(&part);
  if (st != TR_OK) return st;
  const int BH = c->lay.B * c->hq;
  const int64_t rec = (int64_t)(c->lay.D + 2) * sizeof(float);
  const int64_t limit = (int64_t)TR_NOALLOC_SCRATCH_BYTES / rec / BH;    // partial records per pair
  const int nch = decode_chunks(c, c->len[layer], BH, (int)(limit < (1 << 20) ? limit : (1 << 20)));
  if (nch < 1) return TR_ERR_SCRATCH;
  // every chunk writes its own record before the combine reads it: nothing needs clearing
  return decode_run(c, layer, q, mode, window, out, nch, part, nch, false, stream);
}
