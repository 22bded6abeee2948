// Decode routed attention over the mixed-width paged cache (TriRoute review page,
// xllm-io.github.io: Eq. (2) modes read by a query; Eq. (4) codes written per token).
//
// One query per (sequence, head) at position t.  Its key set is the position window
// [lo, t] (lo = 0 for full, max(0, t - w) for local; skip heads read nothing).  The window is
// split into position chunks (split-K); every chunk maps, through the per-position class
// prefix counts, to one contiguous slot range per width class, so out-of-window keys are
// never read and each inner loop runs over a single width (wave-uniform unpacking).
//
// k_decode_split (one workgroup per (seq, head, chunk)):
//   phase 1  K codes -> scores in LDS: 8/16-byte loads per lane, codes unpacked in
//            registers, dot with q in fp32, reduced across the lanes of a key; the zero
//            point folds in as s * (q . c) + z * sum(q) (exact identity of Eq. (4)'s
//            reconstruction), scaled into the log2 domain.
//   softmax  chunk max m, p = 2^(score - m), l = sum p (fp32).
//   phase 2  V codes: every lane owns 16 fixed channels of a key, so all width classes
//            accumulate into the same 16 fp32 registers: acc += (p * s_v) * c,
//            plus sum(p * z_v) once per key.
//   output   partial (o[D], m, l) per chunk.
// k_decode_combine: log-sum-exp merge of the chunks -> bf16; zeros for skip heads.
#include <math.h>
#include <stdlib.h>

#include "common.h"

namespace {

constexpr int kBlock = 256;
constexpr int kMaxChunkPositions = 4096;

template <int B>
__device__ __forceinline__ uint32_t code_at(const uint32_t* w, int k) {
  return (w[(k * B) >> 5] >> ((k * B) & 31)) & ((1u << B) - 1u);
}

__device__ __forceinline__ float block_reduce_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ float block_reduce_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Phase 1 for width class C over class slots [a, e): scores into sc[off + (j - a)].
template <int D, int C>
__device__ __forceinline__ void score_phase(const CacheLayout& c, int layer, int s, int h, int a, int e, int off,
                                            const float* qs, float sigma, float kscale, float* sc) {
  constexpr int b = 2 << C;
  constexpr int KBL = (C == 0) ? 8 : 16;           // bytes per lane per key
  constexpr int E = KBL * 8 / b;                   // elements per lane
  constexpr int LPK = D * b / 8 / KBL;             // lanes per key
  constexpr int KPI = kBlock / LPK;                // keys per block iteration
  constexpr int W = KBL / 4;
  const int tid = threadIdx.x;
  const int part = tid % LPK;
  float qr[E];
#pragma unroll
  for (int k = 0; k < E; ++k) qr[k] = qs[part * E + k];
  const int32_t* pt = tr_ptab(c, layer, s, C);
  const int P = c.ptok[C];
  const int64_t hoff = (int64_t)h * c.cb + part * KBL;
  for (int base = a; base < e; base += KPI) {
    const int j = base + tid / LPK;
    const bool valid = j < e;
    float dot = 0.0f, sK = 1.0f, zK = 0.0f;
    if (valid) {
      const int page = pt[j / P];
      const int slot = j % P;
      const uint8_t* pb = c.pool + (int64_t)page * c.page_bytes;
      const uint8_t* row = pb + c.k_off[C] + hoff + (int64_t)slot * (D * b / 8);
      uint32_t w[W];
      if constexpr (W == 2) {
        const uint2 t = *reinterpret_cast<const uint2*>(row);
        w[0] = t.x; w[1] = t.y;
      } else {
        const uint4 t = *reinterpret_cast<const uint4*>(row);
        w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
      }
      if constexpr (C < 3) {
        const float2 sz = reinterpret_cast<const float2*>(pb + c.sk_off[C])[(int64_t)h * P + slot];
        sK = sz.x;
        zK = sz.y;
#pragma unroll
        for (int k = 0; k < E; ++k) dot = fmaf(qr[k], (float)code_at<b>(w, k), dot);
      } else {
#pragma unroll
        for (int k = 0; k < E / 2; ++k) {
          dot = fmaf(qr[2 * k], tr_bf16_lo(w[k]), dot);
          dot = fmaf(qr[2 * k + 1], tr_bf16_hi(w[k]), dot);
        }
      }
    }
#pragma unroll
    for (int o = 1; o < LPK; o <<= 1) dot += __shfl_xor(dot, o, 64);
    if (valid && part == 0) sc[off + (j - a)] = fmaf(sK, dot, zK * sigma) * kscale;
  }
}

// Phase 2 for width class C: acc[16] (channels 16*part ..) += p * v_hat.
template <int D, int C>
__device__ __forceinline__ void value_phase(const CacheLayout& c, int layer, int s, int h, int a, int e, int off,
                                            const float* pw, float* acc, float& zacc) {
  constexpr int b = 2 << C;
  constexpr int VLPK = D / 16;
  constexpr int KPI = kBlock / VLPK;
  constexpr int BYTES = 2 * b;                     // 16 codes of b bits
  const int tid = threadIdx.x;
  const int part = tid % VLPK;
  const int32_t* pt = tr_ptab(c, layer, s, C);
  const int P = c.ptok[C];
  const int64_t hoff = (int64_t)h * c.cb + part * BYTES;
  for (int base = a; base < e; base += KPI) {
    const int j = base + tid / VLPK;
    if (j >= e) continue;
    const int page = pt[j / P];
    const int slot = j % P;
    const uint8_t* pb = c.pool + (int64_t)page * c.page_bytes;
    const uint8_t* row = pb + c.v_off[C] + hoff + (int64_t)slot * (D * b / 8);
    const float p = pw[off + (j - a)];
    if constexpr (C < 3) {
      const float2 sz = reinterpret_cast<const float2*>(pb + c.sv_off[C])[(int64_t)h * P + slot];
      const float ps = p * sz.x;
      if (part == 0) zacc = fmaf(p, sz.y, zacc);
      uint32_t w[4];
      if constexpr (b == 2) {
        w[0] = *reinterpret_cast<const uint32_t*>(row);
      } else if constexpr (b == 4) {
        const uint2 t = *reinterpret_cast<const uint2*>(row);
        w[0] = t.x; w[1] = t.y;
      } else {
        const uint4 t = *reinterpret_cast<const uint4*>(row);
        w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) acc[k] = fmaf(ps, (float)code_at<b>(w, k), acc[k]);
    } else {
      const uint4 t0 = reinterpret_cast<const uint4*>(row)[0];
      const uint4 t1 = reinterpret_cast<const uint4*>(row)[1];
      const uint32_t w[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        acc[2 * k] = fmaf(p, tr_bf16_lo(w[k]), acc[2 * k]);
        acc[2 * k + 1] = fmaf(p, tr_bf16_hi(w[k]), acc[2 * k + 1]);
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(kBlock) void k_decode_split(CacheLayout c, int layer, int t, int window, int CH, int nch_grid,
                                                         int max_chunks, float kscale,
                                                         const uint16_t* __restrict__ q,
                                                         const uint8_t* __restrict__ mode,
                                                         float* __restrict__ part) {
  extern __shared__ float sc[];                    // [CH] scores, then weights
  __shared__ float qs[D];
  __shared__ float red[4];
  __shared__ float ored[4][D + 1];
  const int tid = threadIdx.x;
  const int k = blockIdx.x % nch_grid;
  const int sh = blockIdx.x / nch_grid;
  const int h = sh % c.H, s = sh / c.H;
  const int m = mode[sh];
  if (m == TR_MODE_SKIP) return;
  if (m != TR_MODE_LOCAL && m != TR_MODE_FULL) {
    if (k == 0 && tid == 0) atomicOr(c.err, TR_ERRF_BAD_MODE);
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
  int a[4], e[4], off[4];
  int nk = 0;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    a[x] = pa[x];
    e[x] = pe[x];
    off[x] = nk;
    nk += e[x] - a[x];
  }
  if (tid < D) qs[tid] = tr_bf16_lo((uint32_t)q[(int64_t)sh * D + tid]);
  __syncthreads();
  float sigma = 0.0f;
  for (int d = 0; d < D; ++d) sigma += qs[d];      // same order in every thread

  if (e[0] > a[0]) score_phase<D, 0>(c, layer, s, h, a[0], e[0], off[0], qs, sigma, kscale, sc);
  if (e[1] > a[1]) score_phase<D, 1>(c, layer, s, h, a[1], e[1], off[1], qs, sigma, kscale, sc);
  if (e[2] > a[2]) score_phase<D, 2>(c, layer, s, h, a[2], e[2], off[2], qs, sigma, kscale, sc);
  if (e[3] > a[3]) score_phase<D, 3>(c, layer, s, h, a[3], e[3], off[3], qs, sigma, kscale, sc);
  __syncthreads();

  float mx = -INFINITY;
  for (int i = tid; i < nk; i += kBlock) mx = fmaxf(mx, sc[i]);
  mx = block_reduce_max(mx, red);
  float lsum = 0.0f;
  for (int i = tid; i < nk; i += kBlock) {
    const float p = exp2f(sc[i] - mx);
    sc[i] = p;
    lsum += p;
  }
  lsum = block_reduce_sum(lsum, red);              // contains the barrier before phase 2

  float acc[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) acc[x] = 0.0f;
  float zacc = 0.0f;
  if (e[0] > a[0]) value_phase<D, 0>(c, layer, s, h, a[0], e[0], off[0], sc, acc, zacc);
  if (e[1] > a[1]) value_phase<D, 1>(c, layer, s, h, a[1], e[1], off[1], sc, acc, zacc);
  if (e[2] > a[2]) value_phase<D, 2>(c, layer, s, h, a[2], e[2], off[2], sc, acc, zacc);
  if (e[3] > a[3]) value_phase<D, 3>(c, layer, s, h, a[3], e[3], off[3], sc, acc, zacc);

  // Reduce over the key slots of the wave (lanes with the same channel group), then waves.
  constexpr int VLPK = D / 16;
#pragma unroll
  for (int o = VLPK; o < 64; o <<= 1) {
#pragma unroll
    for (int x = 0; x < 16; ++x) acc[x] += __shfl_xor(acc[x], o, 64);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) zacc += __shfl_xor(zacc, o, 64);
  const int wave = tid >> 6, lane = tid & 63;
  if (lane < VLPK) {
#pragma unroll
    for (int x = 0; x < 16; ++x) ored[wave][lane * 16 + x] = acc[x];
  }
  if (lane == 0) ored[wave][D] = zacc;
  __syncthreads();
  float* dst = part + ((int64_t)sh * max_chunks + k) * (D + 2);
  if (tid < D) {
    const float z = (ored[0][D] + ored[1][D]) + (ored[2][D] + ored[3][D]);
    dst[tid] = (ored[0][tid] + ored[1][tid]) + (ored[2][tid] + ored[3][tid]) + z;
  }
  if (tid == 0) {
    dst[D] = mx;
    dst[D + 1] = lsum;
  }
}

template <int D>
__global__ __launch_bounds__(D) void k_decode_combine(int H, int t, int window, int CH, int max_chunks,
                                                      const uint8_t* __restrict__ mode,
                                                      const float* __restrict__ part, uint16_t* __restrict__ out) {
  const int sh = blockIdx.x;
  const int d = threadIdx.x;
  const int m = mode[sh];
  uint16_t* o = out + (int64_t)sh * D;
  if (m != TR_MODE_LOCAL && m != TR_MODE_FULL) {
    o[d] = 0;
    return;
  }
  const int lo = (m == TR_MODE_FULL) ? 0 : max(0, t - window);
  const int L = t + 1 - lo;
  const int nch = (L + CH - 1) / CH;
  const float* base = part + (int64_t)sh * max_chunks * (D + 2);
  float M = -INFINITY;
  for (int k = 0; k < nch; ++k) M = fmaxf(M, base[(int64_t)k * (D + 2) + D]);
  float num = 0.0f, den = 0.0f;
  for (int k = 0; k < nch; ++k) {
    const float* pk = base + (int64_t)k * (D + 2);
    const float wgt = exp2f(pk[D] - M);
    num = fmaf(wgt, pk[d], num);
    den = fmaf(wgt, pk[D + 1], den);
  }
  o[d] = tr_f32_to_bf16(num / den);
}

}  // namespace

tr_status tr_decode_launch(tr_kv_cache* c, int layer, const uint16_t* q, const uint8_t* mode, int window,
                           uint16_t* out, hipStream_t stream) {
  const CacheLayout& L = c->lay;
  const int t = c->len[layer] - 1;
  const int n = t + 1;
  const int BH = L.B * L.H;
  int nch = (4096 + BH - 1) / BH;
  if (const char* env = getenv("TR_DECODE_NCH")) nch = atoi(env);
  if (nch > (n + 63) / 64) nch = (n + 63) / 64;
  if (nch < (n + kMaxChunkPositions - 1) / kMaxChunkPositions) nch = (n + kMaxChunkPositions - 1) / kMaxChunkPositions;
  if (nch > c->max_chunks) nch = c->max_chunks;
  if (nch < 1) nch = 1;
  const int CH = (n + nch - 1) / nch;
  if (CH > kMaxChunkPositions) return TR_ERR_UNSUPPORTED;
  const float kscale = (float)(1.4426950408889634 / sqrt((double)L.D));
  const size_t lds = sizeof(float) * (size_t)CH;
  const int grid = BH * nch;
  {
    TrProfScope prof(c, TR_PROF_DECODE_SPLIT, stream);
    if (L.D == 64)
      hipLaunchKernelGGL(k_decode_split<64>, dim3(grid), dim3(kBlock), lds, stream, L, layer, t, window, CH, nch,
                         c->max_chunks, kscale, q, mode, c->partials);
    else
      hipLaunchKernelGGL(k_decode_split<128>, dim3(grid), dim3(kBlock), lds, stream, L, layer, t, window, CH, nch,
                         c->max_chunks, kscale, q, mode, c->partials);
    TR_LAUNCH_CHECK();
  }
  {
    TrProfScope prof(c, TR_PROF_DECODE_COMBINE, stream);
    if (L.D == 64)
      hipLaunchKernelGGL(k_decode_combine<64>, dim3(BH), dim3(64), 0, stream, L.H, t, window, CH, c->max_chunks,
                         mode, c->partials, out);
    else
      hipLaunchKernelGGL(k_decode_combine<128>, dim3(BH), dim3(128), 0, stream, L.H, t, window, CH, c->max_chunks,
                         mode, c->partials, out);
  }
  TR_LAUNCH_CHECK();
  return TR_OK;
}
