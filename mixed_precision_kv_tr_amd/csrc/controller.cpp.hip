// Routing controller at inference (TriRoute review page, xllm-io.github.io: "core formulas"
// item 5, Eq. (5), the shared controller; item 10, Eq. (11), per-axis whitening; the inference
// paragraph after Algorithm 1: the routers take the hard argmax).  For every token:
//
//   h     = W2 silu(W1 [RMSNorm(x); psi] + b1) + b2        trunk, d_r = 128
//   hhat  = RMSNorm(h);  hhat^ax = (hhat - mu_ax) / (sigma_ax + 1e-5)
//   mode  = argmax over each head's 3 logits of W_a hhat^a;  bits = (2,4,8,16)[argmax W_b hhat^b]
//
// One workgroup (16 waves) per 32 tokens:
//   layer 1   X[32 x d] . W1x^T on the matrix cores (v_mfma_f32_32x32x16_bf16): wave (ub, ks)
//             computes trunk units 32 ub .. 32 ub + 31 over the ks-th quarter of the channels,
//             with x and W1 as exact bf16 operands and fp32 accumulation, and the next 4
//             k-steps' operands in flight while the current 4 multiply; the quarters are summed
//             in LDS.  W1 comes pre-packed (tr_controller_pack_w1) so that each k-step of a
//             wave reads 1 KB contiguous, and each lane reads 64 contiguous bytes of its x row.  RMSNorm(x) is applied afterwards as a per-token scale (the sum of squares
//             comes from the same A operands), then the side-feature term, the bias and SiLU,
//             in fp32.  (Splitting the channels gives a 32-token decode step 16 waves instead of
//             4, and shortens each wave's chain of dependent loads 4x.)
//   layer 2   fp32 FMAs: thread (unit n, tokens n8 + 8 m) runs over the 128 inputs, weights from
//             LDS (W2's loads are issued at the start and overlap layer 1) and activations
//             broadcast from LDS.  The heads' weights then replace W2 in LDS (up to 40 heads;
//             beyond that they are read from global memory).
//   RMSNorm, whitening of both axes, the heads (fp32) and the argmaxes, all from LDS.
// The controller is < 1% of a layer's FLOPs on the page; the kernel streams x once (2 d bytes
// per token) and re-reads the 0.25-4 MB of weights from L2.
#include <math.h>
#include <stdint.h>

#include "common.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTok = 32;        // tokens per workgroup
constexpr int kDr = 128;        // trunk width
constexpr int kSplit = 4;       // k-splits of layer 1 (one per group of 4 waves)
constexpr int kThreads = 256 * kSplit;
constexpr int kMaxHeads = 64;
constexpr int kMaxSide = 32;
constexpr int kMaxOut = 3 * kMaxHeads + 4;
constexpr int kRow = kDr + 4;   // padded LDS row (16-byte aligned)

struct CtlArgs {
  int d, d_side, heads;
  const uint16_t* w1;
  const float* w1_side;
  const float* b1;
  const float* w2;
  const float* b2;
  const float* mu_a;
  const float* sigma_a;
  const float* mu_b;
  const float* sigma_b;
  const float* w_a;
  const float* w_b;
};

// 16-byte load through a global-address-space pointer (a pointer taken from a struct argument is
// otherwise generic, and its loads become flat loads that also wait on the LDS counter).
__device__ __forceinline__ uint4 gload16(const uint16_t* p) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  typedef const __attribute__((address_space(1))) v4u* gp;
  const v4u v = *(gp)(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float sq8(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = tr_bf16_lo(w[i]), hi = tr_bf16_hi(w[i]);
    s = fmaf(lo, lo, s);
    s = fmaf(hi, hi, s);
  }
  return s;
}

// LDS: layer 1's partial sums per k-split [kSplit][kTok][kRow]; after the reduction, split 0
// holds the trunk's first activation (then hhat^a), split 1 the second (then hhat^b), splits 2-3
// the logits.
// wts holds W2 (loaded while layer 1 runs), then the two heads' weights when they fit.
struct CtlSmem {
  float part[kSplit][kTok][kRow];
  float wts[kDr * kDr];
  float sd[kTok][kMaxSide];
  float ssp[kSplit][kTok];
  float inv2[kTok];
};
static_assert(2 * kTok * kRow >= kTok * (kMaxOut + 1), "logits fit two partial planes");

__global__ __launch_bounds__(kThreads) void k_controller(CtlArgs a, const uint16_t* __restrict__ x,
                                                         const float* __restrict__ side, int64_t M,
                                                         uint8_t* __restrict__ mode, uint8_t* __restrict__ bits) {
  __shared__ __align__(16) CtlSmem sm;
  float(*hs)[kRow] = sm.part[0];
  float(*h2s)[kRow] = sm.part[1];
  float(*zl)[kMaxOut + 1] = reinterpret_cast<float(*)[kMaxOut + 1]>(&sm.part[2][0][0]);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t tok0 = (int64_t)blockIdx.x * kTok;
  const int ntok = (int)min<int64_t>(kTok, M - tok0);
  // W2's 64 KB, 16 floats per thread: loads issued now, stored to LDS after layer 1
  static_assert(kDr * kDr == 16 * kThreads, "one 64-byte share of W2 per thread");
  float4 w2r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) w2r[j] = reinterpret_cast<const float4*>(a.w2)[tid + j * kThreads];
  for (int i = tid; i < kTok * a.d_side; i += kThreads) {
    const int t = i / a.d_side, s = i % a.d_side;
    sm.sd[t][s] = t < ntok ? side[(tok0 + t) * a.d_side + s] : 0.0f;
  }

  // ---- layer 1 on the matrix cores: wave (unit block ub, k-split ks) computes
  //      D[token][unit] over its quarter of the channel groups, unit = 32 ub + (lane & 31) ----
  // Channel order: group g holds channels 64 g .. 64 g + 63; in its 4 k-steps j, lane half kh
  // supplies channels 64 g + 32 kh + 8 j .. + 7, so a lane reads 64 contiguous bytes of its x
  // row per group, and the packed W1 (tr_controller_pack_w1) holds the same channels of 32 units
  // of one k-step in one contiguous 1 KB.
  {
    const int ub = wave & 3, ks = wave >> 2;
    const int r = lane & 31, kh = lane >> 5;
    const int ng = a.d / 64;                        // channel groups
    const int g0 = ks * ng / kSplit, g1 = (ks + 1) * ng / kSplit;
    // rows past the last token repeat it (their results are never written out)
    const uint16_t* xr = x + (tok0 + min(r, ntok - 1)) * a.d + 32 * kh;
    const uint16_t* wr = a.w1 + (int64_t)(32 * ub + r) * 16 + 8 * kh;
    const int64_t wstep = (int64_t)kDr * 16;        // packed W1: one k-step of all units
    f32x16 acc = {};
    float ss = 0.0f;
    if (g0 < g1) {
      uint4 xa[4], wb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xa[j] = gload16(xr + 64 * g0 + 8 * j);
        wb[j] = gload16(wr + (4 * g0 + j) * wstep);
      }
      for (int g = g0; g < g1; ++g) {
        const int gn = min(g + 1, g1 - 1);          // clamped: the loads never branch
        uint4 xn[4], wn[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xn[j] = gload16(xr + 64 * gn + 8 * j);
          wn[j] = gload16(wr + (4 * gn + j) * wstep);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xa[j]),
                                                        __builtin_bit_cast(bf16x8, wb[j]), acc, 0, 0, 0);
          ss += sq8(xa[j]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xa[j] = xn[j];
          wb[j] = wn[j];
        }
      }
    }
    // sum of squares of token r over this split: this lane's half of the channels plus the other's
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
    if (ub == 0 && lane < kTok) sm.ssp[ks][lane] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
#pragma unroll
    for (int reg = 0; reg < 16; ++reg) sm.part[ks][8 * (reg >> 2) + 4 * kh + (reg & 3)][32 * ub + r] = acc[reg];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) reinterpret_cast<float4*>(sm.wts)[tid + j * kThreads] = w2r[j];
  __syncthreads();
  // ---- reduce the splits, RMSNorm(x) as a per-token scale, side features, bias, SiLU ----
  {
    const int n = tid & (kDr - 1), p = tid >> 7;    // tokens p, p + 8, p + 16, p + 24
    const float b1 = a.b1[n];
#pragma unroll
    for (int m = 0; m < kTok / 8; ++m) {
      const int t = p + 8 * m;
      float sum = 0.0f, sq = 0.0f;
#pragma unroll
      for (int k = 0; k < kSplit; ++k) {
        sum += sm.part[k][t][n];
        sq += sm.ssp[k][t];
      }
      float v = fmaf(sum, 1.0f / sqrtf(sq / (float)a.d + 1e-6f), b1);
      for (int s = 0; s < a.d_side; ++s) v = fmaf(sm.sd[t][s], a.w1_side[n * a.d_side + s], v);
      hs[t][n] = v / (1.0f + expf(-v));
    }
  }
  __syncthreads();
  // ---- layer 2: h2 = h W2 + b2, thread (unit n, tokens p + 8 m) ----
  {
    const int n = tid & (kDr - 1), p = tid >> 7;
    float acc[kTok / 8];
    const float b2 = a.b2[n];
#pragma unroll
    for (int m = 0; m < kTok / 8; ++m) acc[m] = b2;
    for (int k = 0; k < kDr; k += 4) {
      const float w0 = sm.wts[(k + 0) * kDr + n], w1 = sm.wts[(k + 1) * kDr + n];
      const float w2 = sm.wts[(k + 2) * kDr + n], w3 = sm.wts[(k + 3) * kDr + n];
#pragma unroll
      for (int m = 0; m < kTok / 8; ++m) {
        const float4 hv = *reinterpret_cast<const float4*>(&hs[p + 8 * m][k]);
        acc[m] = fmaf(hv.x, w0, acc[m]);
        acc[m] = fmaf(hv.y, w1, acc[m]);
        acc[m] = fmaf(hv.z, w2, acc[m]);
        acc[m] = fmaf(hv.w, w3, acc[m]);
      }
    }
#pragma unroll
    for (int m = 0; m < kTok / 8; ++m) h2s[p + 8 * m][n] = acc[m];
  }
  __syncthreads();
  // the heads' weights replace W2 in LDS when they fit (up to 40 heads): one round of loads
  const int na = 3 * a.heads, no = na + 4;
  const bool wl = no * kDr <= kDr * kDr;
  if (wl) {
    for (int i = tid; i < kDr * na; i += kThreads) sm.wts[i] = a.w_a[i];
    for (int i = tid; i < kDr * 4; i += kThreads) sm.wts[kDr * na + i] = a.w_b[i];
  }
  if (tid < kTok) {
    float s = 0.0f;
    for (int k = 0; k < kDr; ++k) s = fmaf(h2s[tid][k], h2s[tid][k], s);
    sm.inv2[tid] = 1.0f / sqrtf(s / (float)kDr + 1e-6f);
  }
  __syncthreads();
  // ---- RMSNorm and Eq. (11) per axis: hhat^a -> hs, hhat^b -> h2s ----
  {
    const int n = tid & (kDr - 1), p = tid >> 7;
    const float mua = a.mu_a[n], sa = a.sigma_a[n] + 1e-5f, mub = a.mu_b[n], sb = a.sigma_b[n] + 1e-5f;
#pragma unroll
    for (int m = 0; m < kTok / 8; ++m) {
      const int t = p + 8 * m;
      const float hh = h2s[t][n] * sm.inv2[t];
      hs[t][n] = (hh - mua) / sa;
      h2s[t][n] = (hh - mub) / sb;
    }
  }
  __syncthreads();
  // ---- heads: column o of [W_a | W_b] for the tokens of thread group g ----
  {
    const int groups = kThreads / no;               // >= 5 since no <= 196
    const int o = tid % no, g = tid / no;
    if (g < groups) {
      const bool att = o < na;
      const float* wa = wl ? sm.wts : a.w_a;
      const float* wb = wl ? sm.wts + kDr * na : a.w_b;
      const float* wcol = att ? wa + o : wb + (o - na);
      const int ws = att ? na : 4;
      for (int t = g; t < kTok; t += groups) {
        const float* src = att ? &hs[t][0] : &h2s[t][0];
        float z[4] = {0.0f, 0.0f, 0.0f, 0.0f};       // four independent chains
#pragma unroll 4
        for (int k = 0; k < kDr; k += 4) {
          const float4 v = *reinterpret_cast<const float4*>(src + k);
          z[0] = fmaf(v.x, wcol[(k + 0) * ws], z[0]);
          z[1] = fmaf(v.y, wcol[(k + 1) * ws], z[1]);
          z[2] = fmaf(v.z, wcol[(k + 2) * ws], z[2]);
          z[3] = fmaf(v.w, wcol[(k + 3) * ws], z[3]);
        }
        zl[t][o] = (z[0] + z[1]) + (z[2] + z[3]);
      }
    }
  }
  __syncthreads();
  // ---- hard argmax (first maximum on ties) ----
  for (int i = tid; i < ntok * a.heads; i += kThreads) {
    const int t = i / a.heads, h = i % a.heads;   // (the heads' weights are no longer read)
    const float z0 = zl[t][3 * h], z1 = zl[t][3 * h + 1], z2 = zl[t][3 * h + 2];
    int idx = 0;
    float best = z0;
    if (z1 > best) { idx = 1; best = z1; }
    if (z2 > best) idx = 2;
    mode[(tok0 + t) * a.heads + h] = (uint8_t)idx;
  }
  if (tid < ntok) {
    int idx = 0;
    float best = zl[tid][na];
#pragma unroll
    for (int j = 1; j < 4; ++j) {
      if (zl[tid][na + j] > best) {
        idx = j;
        best = zl[tid][na + j];
      }
    }
    bits[tok0 + tid] = (uint8_t)(2 << idx);
  }
}

// Packed W1: element [s][n][16] for k-step s = 4 g + j and unit n holds channels
// 64 g + 8 j .. + 7 (first 8) and 64 g + 32 + 8 j .. + 7 (last 8) of row n.  One thread per
// (k-step, unit, half): a 16-byte copy.
__global__ __launch_bounds__(256) void k_pack_w1(const uint16_t* __restrict__ w1, uint16_t* __restrict__ wp, int d) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)(d / 16) * kDr * 2;
  if (i >= total) return;
  const int h = (int)(i & 1), n = (int)((i >> 1) % kDr), s = (int)((i >> 1) / kDr);
  const int g = s >> 2, j = s & 3;
  *reinterpret_cast<uint4*>(wp + ((int64_t)s * kDr + n) * 16 + 8 * h) =
      *reinterpret_cast<const uint4*>(w1 + (int64_t)n * d + 64 * g + 32 * h + 8 * j);
}

}  // namespace

extern "C" {

tr_status tr_controller_pack_w1(const void* w1, void* w1_packed, int32_t d, void* stream) {
  if (!w1 || !w1_packed || w1 == w1_packed || d < 64 || d > 16384 || d % 64 != 0) return TR_ERR_INVALID_ARG;
  const int64_t total = (int64_t)(d / 16) * kDr * 2;
  hipLaunchKernelGGL(k_pack_w1, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(w1), static_cast<uint16_t*>(w1_packed), d);
  TR_LAUNCH_CHECK();
  return TR_OK;
}

tr_status tr_controller_route(const tr_controller_weights* w, const void* x, const float* side, int64_t n_tokens,
                              uint8_t* mode, uint8_t* bits, void* stream) {
  if (!w || n_tokens < 0) return TR_ERR_INVALID_ARG;
  if (w->d_r != kDr || w->d < 64 || w->d > 16384 || w->d % 64 != 0 || w->d_side < 0 || w->d_side > kMaxSide ||
      w->heads < 1 || w->heads > kMaxHeads)
    return TR_ERR_INVALID_ARG;
  if (n_tokens == 0) return TR_OK;
  if (!x || !mode || !bits || !w->w1 || !w->b1 || !w->w2 || !w->b2 || !w->mu_a || !w->sigma_a || !w->mu_b ||
      !w->sigma_b || !w->w_a || !w->w_b || (w->d_side > 0 && (!side || !w->w1_side)))
    return TR_ERR_INVALID_ARG;
  const int64_t blocks = (n_tokens + kTok - 1) / kTok;
  if (blocks > 0x7fffffffLL) return TR_ERR_UNSUPPORTED;
  CtlArgs a{w->d, w->d_side, w->heads, static_cast<const uint16_t*>(w->w1), w->w1_side, w->b1, w->w2, w->b2,
            w->mu_a, w->sigma_a, w->mu_b, w->sigma_b, w->w_a, w->w_b};
  hipLaunchKernelGGL(k_controller, dim3((unsigned)blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), a,
                     static_cast<const uint16_t*>(x), side, n_tokens, mode, bits);
  TR_LAUNCH_CHECK();
  return TR_OK;
}

}  // extern "C"
