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
//   layer 2   on the matrix cores with fp32 operands (v_mfma_f32_16x16x4f32): wave w takes a
//             16-token x 16-unit block over the 128 inputs, weights from LDS (W2's loads are
//             issued at the start and overlap layer 1).  The heads' weights then replace W2 in
//             LDS (up to 40 heads; beyond that they are read from global memory).
//   RMSNorm (sums of squares over 32-lane groups), whitening of both axes, the heads (fp32
//   matrix cores again, 16 x 16 blocks of tokens x outputs) and the argmaxes, all from LDS.
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

// Every kernel argument in scalar registers at this point: the argument loads then go out
// together and are waited for once, instead of one wait per argument at its first use.
template <typename T>
__device__ __forceinline__ void pin_sreg(T& v) {
  asm volatile("" : "+s"(v));
}
__device__ __forceinline__ void pin_args(CtlArgs& a) {
  pin_sreg(a.d), pin_sreg(a.d_side), pin_sreg(a.heads), pin_sreg(a.w1), pin_sreg(a.w1_side), pin_sreg(a.b1);
  pin_sreg(a.w2), pin_sreg(a.b2), pin_sreg(a.mu_a), pin_sreg(a.sigma_a), pin_sreg(a.mu_b), pin_sreg(a.sigma_b);
  pin_sreg(a.w_a), pin_sreg(a.w_b);
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
  float w1s[kMaxSide][kDr];       // layer 1's side-feature weights, transposed (unit-contiguous)
  float pu[6][kDr];               // per unit: b1, b2, mu_a, sigma_a, mu_b, sigma_b
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
  // every other small parameter goes out now too, so that no later step waits on memory: the side
  // features and their weights, the per-unit vectors, and the heads' weights when they fit LDS
  // (held in registers until W2 is done)
  for (int i = tid; i < kTok * a.d_side; i += kThreads) {
    const int t = i / a.d_side, s = i % a.d_side;
    sm.sd[t][s] = t < ntok ? side[(tok0 + t) * a.d_side + s] : 0.0f;
  }
  for (int i = tid; i < kDr * a.d_side; i += kThreads) sm.w1s[i % a.d_side][i / a.d_side] = a.w1_side[i];
  if (tid < 6 * kDr) {
    const int v = tid / kDr, n = tid % kDr;
    const float* src = v == 0 ? a.b1 : v == 1 ? a.b2 : v == 2 ? a.mu_a : v == 3 ? a.sigma_a : v == 4 ? a.mu_b : a.sigma_b;
    sm.pu[v][n] = src[n];
  }
  const int na = 3 * a.heads, no = na + 4;
  const bool wl = no * kDr <= kDr * kDr;
  constexpr int kHW = (3 * 40 + 4) * kDr / kThreads + 1;   // head weights per thread (up to 40 heads)
  float hw[kHW];
  if (wl) {
#pragma unroll
    for (int q = 0; q < kHW; ++q) {
      const int i = tid + q * kThreads;
      hw[q] = i < kDr * na ? a.w_a[i] : i < kDr * no ? a.w_b[i - kDr * na] : 0.0f;
    }
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
    // The wave's channel groups in chunks of kCG: every load of a chunk is issued before any of
    // its products, so a split of up to kCG groups (d <= 2048) costs one memory round trip.
    // Indices are clamped (loads never branch); groups past the split's end are not multiplied.
    constexpr int kCG = 8;
    for (int c0 = g0; c0 < g1; c0 += kCG) {
      uint4 xa[kCG][4], wb[kCG][4];
#pragma unroll
      for (int q = 0; q < kCG; ++q) {
        const int g = min(c0 + q, g1 - 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xa[q][j] = gload16(xr + 64 * g + 8 * j);
          wb[q][j] = gload16(wr + (4 * g + j) * wstep);
        }
      }
#pragma unroll
      for (int q = 0; q < kCG; ++q) {
        if (c0 + q >= g1) break;                    // wave-uniform
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xa[q][j]),
                                                        __builtin_bit_cast(bf16x8, wb[q][j]), acc, 0, 0, 0);
          ss += sq8(xa[q][j]);
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
    const float b1 = sm.pu[0][n];
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
      for (int s = 0; s < a.d_side; ++s) v = fmaf(sm.sd[t][s], sm.w1s[s][n], v);
      hs[t][n] = v / (1.0f + expf(-v));
    }
  }
  __syncthreads();
  // ---- layer 2 on the matrix cores (v_mfma_f32_16x16x4f32, fp32 operands): wave w computes
  //      tokens 16 (w >> 3) .. + 15 x units 16 (w & 7) .. + 15 over all 128 inputs; lane l
  //      supplies h[row l % 16][k + l / 16] and W2[k + l / 16][col l % 16] and ends with
  //      D[4 (l / 16) + r][l % 16] ----
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int r16 = lane & 15, q16 = lane >> 4;
  {
    const int tb = wave >> 3, ub = wave & 7;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const float* arow = &hs[16 * tb + r16][q16];
    const float* bcol = &sm.wts[q16 * kDr + 16 * ub + r16];
#pragma unroll 8
    for (int k = 0; k < kDr; k += 4) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(arow[k], bcol[k * kDr], acc, 0, 0, 0);
    const float b2 = sm.pu[1][16 * ub + r16];
#pragma unroll
    for (int r = 0; r < 4; ++r) h2s[16 * tb + 4 * q16 + r][16 * ub + r16] = acc[r] + b2;
  }
  __syncthreads();
  // the heads' weights replace W2 in LDS when they fit (up to 40 heads), from registers
  if (wl) {
#pragma unroll
    for (int q = 0; q < kHW; ++q) {
      const int i = tid + q * kThreads;
      if (i < kDr * no) sm.wts[i] = hw[q];
    }
  }
  // sums of squares: thread (token tid / 32, units 4 (tid % 32) .. + 3), then over 32 lanes
  {
    const int t = tid >> 5, j4 = 4 * (tid & 31);
    const float4 v = *reinterpret_cast<const float4*>(&h2s[t][j4]);
    float e = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, v.w * v.w)));
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) e += __shfl_xor(e, off);
    if ((tid & 31) == 0) sm.inv2[t] = 1.0f / sqrtf(e / (float)kDr + 1e-6f);
  }
  __syncthreads();
  // ---- RMSNorm and Eq. (11) per axis: hhat^a -> hs, hhat^b -> h2s ----
  {
    const int n = tid & (kDr - 1), p = tid >> 7;
    const float mua = sm.pu[2][n], sa = sm.pu[3][n] + 1e-5f, mub = sm.pu[4][n], sb = sm.pu[5][n] + 1e-5f;
#pragma unroll
    for (int m = 0; m < kTok / 8; ++m) {
      const int t = p + 8 * m;
      const float hh = h2s[t][n] * sm.inv2[t];
      hs[t][n] = (hh - mua) / sa;
      h2s[t][n] = (hh - mub) / sb;
    }
  }
  __syncthreads();
  // ---- heads on the matrix cores: items (token block of 16, output block of 16) over the
  //      attention head's ceil(3 H / 16) blocks (inputs hhat^a) and the bit head's one block
  //      (inputs hhat^b); outputs past a head's columns multiply zeros ----
  {
    const int nab = (na + 15) / 16, items = 2 * (nab + 1);
    const float* wa = wl ? sm.wts : a.w_a;
    const float* wb = wl ? sm.wts + kDr * na : a.w_b;
    for (int it = wave; it < items; it += kThreads / 64) {
      const int tb = it & 1, ob = it >> 1;
      const bool att = ob < nab;
      const int o = att ? 16 * ob + r16 : r16;      // column within its head
      const bool live = att ? o < na : o < 4;
      const float* src = att ? &hs[16 * tb + r16][q16] : &h2s[16 * tb + r16][q16];
      const float* wcol = att ? wa + min(o, na - 1) : wb + min(o, 3);
      const int ws = att ? na : 4;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
      for (int k = 0; k < kDr; k += 4) {
        const float w = live ? wcol[(k + q16) * ws] : 0.0f;
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(src[k], w, acc, 0, 0, 0);
      }
      if (live) {
        const int col = att ? o : na + o;
#pragma unroll
        for (int r = 0; r < 4; ++r) zl[16 * tb + 4 * q16 + r][col] = acc[r];
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

// ---- split path for small calls (up to kSplitMaxTok tokens) ----
// A decode step routes a few dozen tokens: one workgroup per 32 tokens would leave the chip idle
// and pull all of W1 through one CU.  Instead two launches:
//   k_ctl_l1   workgroup (token block, channel slice ks, unit block us): 4 waves, wave w takes
//              channel group 4 ks + w (64 channels, 4 k-steps) for 32 tokens x 32 units on the
//              matrix cores; the 4 waves are summed in LDS and the partial goes to the workspace
//              (with the slice's sums of squares of x, from the us = 0 workgroups).
//   k_ctl_tok  one workgroup (8 waves) per token: sums the slices, and runs RMSNorm(x), the side
//              term, SiLU, layer 2, RMSNorm, Eq. (11) and the heads for that token, with every
//              weight it needs requested at its start.
constexpr int kSplitMaxTok = 256;
constexpr int kFinThreads = 512;

__host__ __device__ constexpr int ctl_slices(int d) { return (d / 64 + 3) / 4; }
int64_t ctl_ws_floats(int d) { return (int64_t)(kSplitMaxTok / kTok) * ctl_slices(d) * kTok * (kDr + 1); }

__global__ __launch_bounds__(256) void k_ctl_l1(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w1p, int d,
                                                int64_t M, int KS, float* __restrict__ part, float* __restrict__ ssp) {
  __shared__ float red[4][kTok][33];
  __shared__ float ssr[4][kTok];
  pin_sreg(x), pin_sreg(w1p), pin_sreg(d), pin_sreg(M), pin_sreg(KS), pin_sreg(part), pin_sreg(ssp);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int b = blockIdx.x, us = b & 3, ks = (b >> 2) % KS, blk = (b >> 2) / KS;
  const int64_t tok0 = (int64_t)blk * kTok;
  const int ntok = (int)min<int64_t>(kTok, M - tok0);
  const int g = 4 * ks + wave, r = lane & 31, kh = lane >> 5;
  f32x16 acc = {};
  float ss = 0.0f;
  if (g < d / 64) {                                 // wave-uniform
    // rows past the last token repeat it (their partials are never read)
    const uint16_t* xr = x + (tok0 + min(r, ntok - 1)) * d + 64 * g + 32 * kh;
    const uint16_t* wr = w1p + ((int64_t)(4 * g) * kDr + 32 * us + r) * 16 + 8 * kh;
    uint4 xa[4], wb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xa[j] = gload16(xr + 8 * j);
      wb[j] = gload16(wr + (int64_t)j * kDr * 16);
    }
    __builtin_amdgcn_sched_barrier(0);              // all eight loads issued before the first wait
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xa[j]), __builtin_bit_cast(bf16x8, wb[j]),
                                                    acc, 0, 0, 0);
      ss += sq8(xa[j]);
    }
  }
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
  if (lane < kTok) ssr[wave][lane] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
#pragma unroll
  for (int reg = 0; reg < 16; ++reg) red[wave][8 * (reg >> 2) + 4 * kh + (reg & 3)][r] = acc[reg];
  __syncthreads();
  float* dst = part + ((int64_t)blk * KS + ks) * kTok * kDr + 32 * us;
  const int u = tid & 31;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = (tid >> 5) + 8 * i;
    dst[t * kDr + u] = (red[0][t][u] + red[1][t][u]) + (red[2][t][u] + red[3][t][u]);
  }
  if (us == 0 && tid < kTok)
    ssp[((int64_t)blk * KS + ks) * kTok + tid] = (ssr[0][tid] + ssr[1][tid]) + (ssr[2][tid] + ssr[3][tid]);
}

__device__ __forceinline__ float gload_f(const float* p) { return *(const __attribute__((address_space(1))) float*)(p); }
__device__ __forceinline__ float4 gload_f4(const float* p) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  const v4f v = *(const __attribute__((address_space(1))) v4f*)(p);
  return make_float4(v.x, v.y, v.z, v.w);
}

// PER: layer-1 slices per thread (KS <= 4 PER); OPW: head outputs per row of threads (64, 128 or
// 256, >= 3 heads + 4).  Thread (output o = tid % OPW, input group hp = tid / OPW) holds the
// weights of o for inputs hp kper .. hp kper + kper - 1, kper = 128 OPW / 512: a wave's lanes
// are consecutive outputs of one input row, so every weight load is a contiguous row segment.
template <int PER, int OPW>
__global__ __launch_bounds__(kFinThreads) void k_ctl_tok(CtlArgs a, const float* __restrict__ side, int KS,
                                                          const float* __restrict__ part, const float* __restrict__ ssp,
                                                          uint8_t* __restrict__ mode, uint8_t* __restrict__ bits) {
  __shared__ float r1[4][kDr];
  __shared__ float w1s[kMaxSide][kDr];
  __shared__ float sds[kMaxSide];
  __shared__ float hs[kDr];
  __shared__ float r2[16][kDr];
  __shared__ float hab[2][kDr];
  __shared__ float zp[kFinThreads];
  __shared__ float sq[4];
  pin_args(a);
  pin_sreg(side), pin_sreg(KS), pin_sreg(part), pin_sreg(ssp), pin_sreg(mode), pin_sreg(bits);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t m = blockIdx.x;
  const int64_t blk = m / kTok;
  const int row = (int)(m % kTok);
  // ---- every load goes out first (none waits on another) ----
  const int n = tid & (kDr - 1), kq = tid >> 7;     // layer-1 slices kq, kq + 4, ...
  // side features: W1's side columns (at most 32 x 128 = 8 per thread) and the token's row
  float wsr[kMaxSide * kDr / kFinThreads];
#pragma unroll
  for (int j = 0; j < kMaxSide * kDr / kFinThreads; ++j) {
    const int i = tid + j * kFinThreads;
    wsr[j] = i < kDr * a.d_side ? gload_f(a.w1_side + i) : 0.0f;
  }
  const float sdv = tid < a.d_side ? gload_f(side + m * a.d_side + tid) : 0.0f;
  // W2 (in x out): thread (unit quad q, k-group kg) holds W2[8 kg .. 8 kg + 7][4 q .. 4 q + 3]
  const int q = tid & 31, kg = tid >> 5;
  float4 w2v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    w2v[i] = gload_f4(a.w2 + (8 * kg + i) * kDr + 4 * q);
  // heads
  const int na = 3 * a.heads, no = na + 4;
  constexpr int kper = kDr * OPW / kFinThreads;
  const int o = tid % OPW, hp = tid / OPW;
  float hw[kper];
  {
    // (threads past the last output read the last column; their sums are never used)
    const bool att = o < na;
    const float* wcol = att ? a.w_a + min(o, na - 1) : a.w_b + min(o - na, 3);
    const int ws = att ? na : 4;
#pragma unroll
    for (int j = 0; j < kper; ++j) hw[j] = gload_f(wcol + (hp * kper + j) * ws);
  }
  const float b1 = gload_f(a.b1 + n), b2 = gload_f(a.b2 + n);
  const float mua = gload_f(a.mu_a + n), sa = gload_f(a.sigma_a + n) + 1e-5f;
  const float mub = gload_f(a.mu_b + n), sb = gload_f(a.sigma_b + n) + 1e-5f;
  // the layer-1 partials of this token (at most 64 slices: 16 per thread) and the slices' sums
  // of squares of x (one per lane of wave 0).  The loads are unconditional, from indices clamped
  // to the last slice, and the extras multiplied by 0 afterwards (the partials are finite): a
  // load under a condition, or a select of it, ends up in a branch that waits for it (and for
  // every load before it) on the spot.
  const float* pp = part + (blk * KS * kTok + row) * kDr + n;
  float pv[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) pv[j] = gload_f(pp + (int64_t)min(kq + 4 * j, KS - 1) * kTok * kDr);
  float sqx = gload_f(ssp + (blk * KS + min(lane, KS - 1)) * kTok + row);
  float s1 = 0.0f;
#pragma unroll
  for (int j = 0; j < PER; ++j) s1 = fmaf(pv[j], kq + 4 * j < KS ? 1.0f : 0.0f, s1);
  sqx *= (wave == 0 && lane < KS) ? 1.0f : 0.0f;

  // ---- layer 1: sum of the slices, RMSNorm(x) as a scale, side term, bias, SiLU ----
  r1[kq][n] = s1;
  const int dsd = max(a.d_side, 1);
#pragma unroll
  for (int j = 0; j < kMaxSide * kDr / kFinThreads; ++j) {
    const int i = tid + j * kFinThreads;
    if (i < kDr * a.d_side) w1s[i % dsd][i / dsd] = wsr[j];
  }
  if (tid < a.d_side) sds[tid] = sdv;
  if (wave == 0) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sqx += __shfl_xor(sqx, off);
    if (lane == 0) sq[0] = sqx;
  }
  __syncthreads();
  if (tid < kDr) {
    const float sum = (r1[0][n] + r1[1][n]) + (r1[2][n] + r1[3][n]);
    float v = fmaf(sum, 1.0f / sqrtf(sq[0] / (float)a.d + 1e-6f), b1);
    for (int s = 0; s < a.d_side; ++s) v = fmaf(sds[s], w1s[s][n], v);
    hs[n] = v / (1.0f + expf(-v));
  }
  __syncthreads();
  // ---- layer 2 ----
  {
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float h = hs[8 * kg + i];
      acc.x = fmaf(h, w2v[i].x, acc.x);
      acc.y = fmaf(h, w2v[i].y, acc.y);
      acc.z = fmaf(h, w2v[i].z, acc.z);
      acc.w = fmaf(h, w2v[i].w, acc.w);
    }
    *reinterpret_cast<float4*>(&r2[kg][4 * q]) = acc;
  }
  __syncthreads();
  float h2 = 0.0f;
  if (tid < kDr) {
    float s = 0.0f;
#pragma unroll
    for (int g = 0; g < 16; ++g) s += r2[g][n];
    h2 = b2 + s;
    float e = h2 * h2;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) e += __shfl_xor(e, off);
    if (lane == 0) sq[1 + wave] = e;
  }
  __syncthreads();
  // ---- RMSNorm and Eq. (11) per axis ----
  if (tid < kDr) {
    const float hh = h2 * (1.0f / sqrtf((sq[1] + sq[2]) / (float)kDr + 1e-6f));
    hab[0][n] = (hh - mua) / sa;
    hab[1][n] = (hh - mub) / sb;
  }
  __syncthreads();
  // ---- heads: partial logits per input group, summed in a fixed order by the argmax ----
  {
    const float* src = &hab[o < na ? 0 : 1][hp * kper];
    float z = 0.0f;
#pragma unroll
    for (int j = 0; j < kper; ++j) z = fmaf(src[j], hw[j], z);
    zp[tid] = z;
  }
  __syncthreads();
  constexpr int kGroups = kFinThreads / OPW;
  const auto zl = [&](int oo) {
    float z = zp[oo];
#pragma unroll
    for (int g = 1; g < kGroups; ++g) z += zp[g * OPW + oo];
    return z;
  };
  // ---- hard argmax (first maximum on ties) ----
  if (tid < a.heads) {
    const float z0 = zl(3 * tid), z1 = zl(3 * tid + 1), z2 = zl(3 * tid + 2);
    int idx = 0;
    float best = z0;
    if (z1 > best) { idx = 1; best = z1; }
    if (z2 > best) idx = 2;
    mode[m * a.heads + tid] = (uint8_t)idx;
  } else if (tid == kFinThreads - 1) {
    int idx = 0;
    float best = zl(na);
#pragma unroll
    for (int j = 1; j < 4; ++j) {
      const float zj = zl(na + j);
      if (zj > best) {
        idx = j;
        best = zj;
      }
    }
    bits[m] = (uint8_t)(2 << idx);
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

int64_t tr_controller_workspace_bytes(int32_t d) {
  if (d < 64 || d > 16384 || d % 64 != 0) return -1;
  return (int64_t)sizeof(float) * ctl_ws_floats(d);
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
  if (w->workspace) {
    if (w->workspace_bytes < (int64_t)sizeof(float) * ctl_ws_floats(w->d) ||
        reinterpret_cast<uintptr_t>(w->workspace) % 16 != 0)
      return TR_ERR_INVALID_ARG;
    if (n_tokens <= kSplitMaxTok) {
      const int KS = ctl_slices(w->d);
      float* part = static_cast<float*>(w->workspace);
      float* ssp = part + (int64_t)(kSplitMaxTok / kTok) * KS * kTok * kDr;
      hipStream_t st = static_cast<hipStream_t>(stream);
      hipLaunchKernelGGL(k_ctl_l1, dim3((unsigned)(blocks * KS * 4)), dim3(256), 0, st, static_cast<const uint16_t*>(x),
                         static_cast<const uint16_t*>(w->w1), w->d, n_tokens, KS, part, ssp);
      TR_LAUNCH_CHECK();
      const int no = 3 * w->heads + 4;
      const int opw = no <= 64 ? 64 : no <= 128 ? 128 : 256;
      const float* cp = part;
      const float* cs = ssp;
      const dim3 grid((unsigned)n_tokens), blk(kFinThreads);
#define TR_CTL_TOK(PER, OPW) hipLaunchKernelGGL((k_ctl_tok<PER, OPW>), grid, blk, 0, st, a, side, KS, cp, cs, mode, bits)
#define TR_CTL_TOK_T(PER)                \
  switch (opw) {                         \
    case 64: TR_CTL_TOK(PER, 64); break;   \
    case 128: TR_CTL_TOK(PER, 128); break; \
    default: TR_CTL_TOK(PER, 256); break;  \
  }
      if (KS <= 8) {
        TR_CTL_TOK_T(2)
      } else {
        TR_CTL_TOK_T(16)
      }
#undef TR_CTL_TOK_T
#undef TR_CTL_TOK
      TR_LAUNCH_CHECK();
      return TR_OK;
    }
  }
  hipLaunchKernelGGL(k_controller, dim3((unsigned)blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), a,
                     static_cast<const uint16_t*>(x), side, n_tokens, mode, bits);
  TR_LAUNCH_CHECK();
  return TR_OK;
}

}  // extern "C"
