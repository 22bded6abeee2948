// Expert FFN with a null expert (TriRoute review page, xllm-io.github.io: "core formulas" item 3,
// Eq. (3)): FFN_t = sum_{j in S_t} p_tj / sum_{S_t} p * f_j(Norm(x_t)), p_t = softmax(z_t^e) over
// E experts plus the null expert f_0 = 0, S_t the top-k; each expert a SwiGLU FFN
// f(u) = W2 (silu(W1 u) * (W3 u)) with hidden width d_e.
//
// One call = four launches:
//   k_moe_route   one wave per token: 1 / rms(x_t), the top-k of the logits (ties to the lower
//                 index) and the renormalized weights exp(z_j - z_max) / sum over S_t.
//   k_moe_lists   one workgroup per (slot, expert, null included): the tokens whose slot-th
//                 choice is that expert, in token order (a block scan) -- the ragged batches.
//   k_moe_up      one workgroup per (slot, expert, 32 or 64 listed tokens, 128 hidden units): the gate
//                 and up products on the matrix cores (x rows gathered from the list, bf16 x and
//                 packed bf16 W1 / W3 as exact operands, fp32 accumulation), then the RMSNorm
//                 scale, silu(g) * u and bf16 rounding into the hidden buffer.
//   k_moe_down    per slot, in slot order: one workgroup per (expert, 32 or 64 listed tokens, 128 output
//                 channels): the down product of the gathered hidden rows, times the token's
//                 weight, stored (slot 0; the null expert stores zeros) or added (slot 1) into the
//                 fp32 output -- no atomics, so the result does not depend on scheduling.
// Weight matrices are packed once (tr_moe_set_weights) into the operand order of the matrix-core
// k-loop: for k-step s = 4 g + j and output unit n, 16 bf16 holding input channels 64 g + 8 j ..
// + 7 and 64 g + 32 + 8 j .. + 7, so that the 32 units of a wave read one contiguous 1 KB per
// k-step.  The gathered activation rows of a tile are shared by its four waves: each stage of
// k-steps is loaded once per workgroup into double-buffered LDS (16-byte-padded rows), while each
// wave's weight columns come straight from memory into registers, the next stage in flight.
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "common.h"

struct tr_moe {
  int d, de, E, k, max_tokens, device;
  uint16_t* wg;      // packed gate weights, per expert [d / 16][de][16]
  uint16_t* wu;      // packed up weights, per expert [d / 16][de][16]
  uint16_t* wd;      // packed down weights, per expert [de / 16][d][16]
  int32_t* sel;      // [max_tokens][k] chosen gate index (0 = null expert)
  float* wt;         // [max_tokens][k] renormalized weight
  float* inv_rms;    // [max_tokens]
  int32_t* lists;    // [k][E + 1][max_tokens] tokens per (slot, expert), in token order
  int32_t* counts;   // [k][E + 1]
  uint16_t* hbuf;    // [max_tokens * k][de] bf16 hidden rows (row t * k + slot)
  bool weights_set;
};

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Token tiles of 32 * MB listed tokens: each wave computes its 32 units for MB 32-token blocks,
// so a weight load feeds MB matrix-core products.  MB = 2 for calls of more than 512 tokens
// (weights re-read half as often), MB = 1 below (a decode step's few tokens per expert).
constexpr int kSmallCall = 512;
constexpr int kUnits = 128;       // output units per workgroup (4 waves x 32)
constexpr int kMaxExperts = 64;
constexpr int kMaxTopK = 2;

__device__ __forceinline__ uint4 gload16(const uint16_t* p) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  typedef const __attribute__((address_space(1))) v4u* gp;
  const v4u v = *(gp)(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ f32x16 mfma(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// Pack E matrices [units][K] (out x in) into the k-step operand order [K / 16][units][16].
__global__ __launch_bounds__(256) void k_moe_pack(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                  int units, int K, int E) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per = (int64_t)(K / 16) * units * 2;
  if (i >= per * E) return;
  const int e = (int)(i / per);
  const int64_t r = i % per;
  const int h = (int)(r & 1), n = (int)((r >> 1) % units), s = (int)((r >> 1) / units);
  const int g = s >> 2, j = s & 3;
  const int64_t mat = (int64_t)units * K;
  *reinterpret_cast<uint4*>(dst + e * mat + ((int64_t)s * units + n) * 16 + 8 * h) =
      *reinterpret_cast<const uint4*>(src + e * mat + (int64_t)n * K + 64 * g + 32 * h + 8 * j);
}

// One wave per token.
__global__ __launch_bounds__(256) void k_moe_route(const uint16_t* __restrict__ x, const float* __restrict__ z,
                                                   int M, int d, int E, int k, int32_t* __restrict__ sel,
                                                   float* __restrict__ wt, float* __restrict__ inv_rms) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (t >= M) return;
  float ss = 0.0f;
  const uint16_t* xr = x + (int64_t)t * d;
  for (int c = lane * 8; c < d; c += 64 * 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(xr + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = tr_bf16_lo(w[i]), hi = tr_bf16_hi(w[i]);
      ss = fmaf(lo, lo, ss);
      ss = fmaf(hi, hi, ss);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if (lane != 0) return;
  inv_rms[t] = 1.0f / sqrtf(ss / (float)d + 1e-6f);
  const float* zr = z + (int64_t)t * (E + 1);
  int idx[kMaxTopK];
  float zs[kMaxTopK];
  for (int j = 0; j < k; ++j) {                    // top-k, ties to the lower index
    int best = -1;
    float bz = -INFINITY;
    for (int e = 0; e <= E; ++e) {
      bool taken = false;
      for (int q = 0; q < j; ++q) taken |= idx[q] == e;
      const float v = zr[e];
      if (!taken && (best < 0 || v > bz)) {
        best = e;
        bz = v;
      }
    }
    idx[j] = best;
    zs[j] = bz;
  }
  float den = 0.0f, p[kMaxTopK];
  for (int j = 0; j < k; ++j) {                    // zs[0] is the largest selected logit
    p[j] = expf(zs[j] - zs[0]);
    den += p[j];
  }
  for (int j = 0; j < k; ++j) {
    sel[t * k + j] = idx[j];
    wt[t * k + j] = p[j] / den;
  }
}

// One workgroup (1024 threads) per (slot, expert): compaction of the tokens with that choice.
__global__ __launch_bounds__(1024) void k_moe_lists(const int32_t* __restrict__ sel, int M, int k, int E, int cap,
                                                    int32_t* __restrict__ lists, int32_t* __restrict__ counts) {
  __shared__ uint32_t wsum[16];
  const int slot = blockIdx.x / (E + 1), e = blockIdx.x % (E + 1);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int32_t* out = lists + (int64_t)blockIdx.x * cap;
  int base = 0;
  for (int t0 = 0; t0 < M; t0 += 1024) {
    const int t = t0 + tid;
    const uint32_t f = (t < M && sel[t * k + slot] == e) ? 1u : 0u;
    const uint32_t incl = tr_wave_incl_scan(f);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      before += w < wave ? wsum[w] : 0u;
      total += wsum[w];
    }
    if (f) out[base + before + incl - 1] = t;
    base += (int)total;
    __syncthreads();
  }
  if (tid == 0) counts[blockIdx.x] = base;
}

// The tile a workgroup takes: tiles of kTile listed tokens over the (slot, expert) lists in order,
// restricted to slots [s0, s1) and experts [e0, E]; returns false past the last tile.
template <int kTile>
__device__ __forceinline__ bool find_tile(const int32_t* counts, int E, int s0, int s1, int e0, int id, int& slot,
                                          int& e, int& tile, int& cnt) {
  for (int s = s0; s < s1; ++s) {
    for (int x = e0; x <= E; ++x) {
      const int c = counts[s * (E + 1) + x];
      const int nt = (c + kTile - 1) / kTile;
      if (id < nt) {
        slot = s;
        e = x;
        tile = id;
        cnt = c;
        return true;
      }
      id -= nt;
    }
  }
  return false;
}

// Gate and up products for 32 kMB tokens of one (slot, expert) list and 128 hidden units: each
// wave computes 32 units for kMB 32-token blocks.
template <int kMB>
__global__ __launch_bounds__(256) void k_moe_up(const uint16_t* __restrict__ x, const int32_t* __restrict__ lists,
                                                const int32_t* __restrict__ counts, const float* __restrict__ inv_rms,
                                                const uint16_t* __restrict__ wg, const uint16_t* __restrict__ wu,
                                                uint16_t* __restrict__ hbuf, int d, int de, int E, int k, int cap) {
  constexpr int kTile = 32 * kMB;
  __shared__ int32_t tok[kTile];
  __shared__ float inv[kTile];
  int slot, e, tile, cnt;
  if (!find_tile<kTile>(counts, E, 0, k, 1, blockIdx.x, slot, e, tile, cnt)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ntok = min(kTile, cnt - tile * kTile);
  const int32_t* lst = lists + (int64_t)(slot * (E + 1) + e) * cap + tile * kTile;
  if (tid < kTile) {
    const int t = lst[min(tid, ntok - 1)];         // rows past the list's end repeat its last token
    tok[tid] = t;
    inv[tid] = inv_rms[t];
  }
  __syncthreads();
  const int r = lane & 31, kh = lane >> 5;
  const int n = blockIdx.y * kUnits + 32 * wave + r;  // hidden unit of this lane's B column
  // The tile's token rows are shared by the four waves: each stage of kPS k-steps (kPS * 16
  // channels of every row) is loaded once per workgroup, one 16-byte piece per thread, into a
  // double-buffered LDS tile whose 16-byte-padded rows spread over the banks.  Each wave's own
  // weight columns stay in registers, the next stage's in flight.
  constexpr int kPS = 4 / kMB;                      // k-steps per stage
  constexpr int PR = 2 * kPS;                       // 16-byte pieces per row and stage
  static_assert(kTile * PR == 256, "one piece per thread per stage");
  __shared__ uint4 xs[2][kTile][PR + 1];
  const int prow = tid / PR, pp = tid % PR;        // this thread's piece of each stage
  const uint16_t* xrow = x + (int64_t)tok[prow] * d + 32 * (pp & 1);
  auto xaddr = [&](int st) {                        // piece pp of stage st: k-step st + pp / 2, half pp & 1
    const int s = st + (pp >> 1);
    return xrow + 64 * (s >> 2) + 8 * (s & 3);
  };
  const int64_t mat = (int64_t)de * d, wstep = (int64_t)de * 16;
  const uint16_t* gr = wg + (e - 1) * mat + (int64_t)n * 16 + 8 * kh;
  const uint16_t* ur = wu + (e - 1) * mat + (int64_t)n * 16 + 8 * kh;
  f32x16 ag[kMB] = {}, au[kMB] = {};
  const int ns = d / 16;                          // a multiple of 8
  uint4 ga[kPS], ua[kPS];
  auto wload = [&](int st, uint4 (&gv)[kPS], uint4 (&uv)[kPS]) {
#pragma unroll
    for (int q = 0; q < kPS; ++q) {
      gv[q] = gload16(gr + (st + q) * wstep);
      uv[q] = gload16(ur + (st + q) * wstep);
    }
  };
  xs[0][prow][pp] = gload16(xaddr(0));
  wload(0, ga, ua);
  __syncthreads();
  int buf = 0;
  for (int st = 0; st < ns; st += kPS) {
    const int nx = min(st + kPS, ns - kPS);       // clamped: the loads never branch
    const uint4 xn = gload16(xaddr(nx));
    uint4 gn[kPS], un[kPS];
    wload(nx, gn, un);
#pragma unroll
    for (int q = 0; q < kPS; ++q) {
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        const uint4 a = xs[buf][32 * mb + r][2 * q + kh];
        ag[mb] = mfma(a, ga[q], ag[mb]);
        au[mb] = mfma(a, ua[q], au[mb]);
      }
    }
    xs[buf ^ 1][prow][pp] = xn;
#pragma unroll
    for (int q = 0; q < kPS; ++q) {
      ga[q] = gn[q];
      ua[q] = un[q];
    }
    buf ^= 1;
    __syncthreads();
  }
  // D[row][unit]: this lane holds unit n for rows 32 mb + 8 (reg / 4) + 4 kh + reg % 4
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) {
#pragma unroll
    for (int reg = 0; reg < 16; ++reg) {
      const int row = 32 * mb + 8 * (reg >> 2) + 4 * kh + (reg & 3);
      if (row < ntok) {
        const float gv = ag[mb][reg] * inv[row], uv = au[mb][reg] * inv[row];
        const float h = gv / (1.0f + expf(-gv)) * uv;
        hbuf[((int64_t)tok[row] * k + slot) * de + n] = tr_f32_to_bf16(h);
      }
    }
  }
}

// Down product for one slot: 32 kMB tokens of one (slot, expert) list and 128 output channels.
template <int kMB>
__global__ __launch_bounds__(256) void k_moe_down(const uint16_t* __restrict__ hbuf, const int32_t* __restrict__ lists,
                                                  const int32_t* __restrict__ counts, const float* __restrict__ wt,
                                                  const uint16_t* __restrict__ wd, float* __restrict__ y, int d, int de,
                                                  int E, int k, int cap, int slot) {
  constexpr int kTile = 32 * kMB;
  __shared__ int32_t tok[kTile];
  __shared__ float wgt[kTile];
  int s_, e, tile, cnt;
  // slot 0 also takes the null expert's tiles (zeros); later slots skip it
  if (!find_tile<kTile>(counts, E, slot, slot + 1, slot == 0 ? 0 : 1, blockIdx.x, s_, e, tile, cnt)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ntok = min(kTile, cnt - tile * kTile);
  const int32_t* lst = lists + (int64_t)(slot * (E + 1) + e) * cap + tile * kTile;
  if (tid < kTile) {
    const int t = lst[min(tid, ntok - 1)];
    tok[tid] = t;
    wgt[tid] = wt[t * k + slot];
  }
  __syncthreads();
  const int r = lane & 31, kh = lane >> 5;
  const int n = blockIdx.y * kUnits + 32 * wave + r;  // output channel of this lane's B column
  f32x16 acc[kMB] = {};
  if (e > 0) {
    // hidden rows shared by the four waves through LDS, as in k_moe_up
    constexpr int kPS = 4 / kMB;
    constexpr int PR = 2 * kPS;
    static_assert(kTile * PR == 256, "one piece per thread per stage");
    __shared__ uint4 hs[2][kTile][PR + 1];
    const int prow = tid / PR, pp = tid % PR;
    const uint16_t* hrow = hbuf + ((int64_t)tok[prow] * k + slot) * de + 32 * (pp & 1);
    auto haddr = [&](int st) {
      const int s = st + (pp >> 1);
      return hrow + 64 * (s >> 2) + 8 * (s & 3);
    };
    const int64_t wstep = (int64_t)d * 16;
    const uint16_t* dr = wd + (int64_t)(e - 1) * d * de + (int64_t)n * 16 + 8 * kh;
    const int ns = de / 16;                       // a multiple of 8
    uint4 wa[kPS];
    auto wload = [&](int st, uint4 (&wv)[kPS]) {
#pragma unroll
      for (int q = 0; q < kPS; ++q) wv[q] = gload16(dr + (st + q) * wstep);
    };
    hs[0][prow][pp] = gload16(haddr(0));
    wload(0, wa);
    __syncthreads();
    int buf = 0;
    for (int st = 0; st < ns; st += kPS) {
      const int nx = min(st + kPS, ns - kPS);
      const uint4 hn = gload16(haddr(nx));
      uint4 wn[kPS];
      wload(nx, wn);
#pragma unroll
      for (int q = 0; q < kPS; ++q)
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) acc[mb] = mfma(hs[buf][32 * mb + r][2 * q + kh], wa[q], acc[mb]);
      hs[buf ^ 1][prow][pp] = hn;
#pragma unroll
      for (int q = 0; q < kPS; ++q) wa[q] = wn[q];
      buf ^= 1;
      __syncthreads();
    }
  }
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) {
#pragma unroll
    for (int reg = 0; reg < 16; ++reg) {
      const int row = 32 * mb + 8 * (reg >> 2) + 4 * kh + (reg & 3);
      if (row < ntok) {
        float* dst = y + (int64_t)tok[row] * d + n;
        const float v = e > 0 ? acc[mb][reg] * wgt[row] : 0.0f;
        if (slot == 0) *dst = v;
        else *dst += v;
      }
    }
  }
}

}  // namespace

extern "C" {

tr_status tr_moe_alloc(const tr_moe_desc* desc, tr_moe** out) {
  if (!desc || !out) return TR_ERR_INVALID_ARG;
  *out = nullptr;
  const tr_moe_desc& q = *desc;
  if (q.d < 128 || q.d > 16384 || q.d % 128 != 0 || q.d_expert < 128 || q.d_expert > 65536 ||
      q.d_expert % 128 != 0 || q.experts < 1 || q.experts > kMaxExperts || q.top_k < 1 || q.top_k > kMaxTopK ||
      q.max_tokens < 1 || q.max_tokens > (1 << 24))
    return TR_ERR_INVALID_ARG;
  tr_moe* m = new tr_moe();
  m->d = q.d;
  m->de = q.d_expert;
  m->E = q.experts;
  m->k = q.top_k;
  m->max_tokens = q.max_tokens;
  (void)hipGetDevice(&m->device);
  const size_t mat = (size_t)q.d * q.d_expert * q.experts;
  const size_t M = q.max_tokens, K = q.top_k, E1 = q.experts + 1;
  bool ok = hipMalloc((void**)&m->wg, 2 * mat) == hipSuccess;
  ok = ok && hipMalloc((void**)&m->wu, 2 * mat) == hipSuccess;
  ok = ok && hipMalloc((void**)&m->wd, 2 * mat) == hipSuccess;
  ok = ok && hipMalloc((void**)&m->sel, sizeof(int32_t) * M * K) == hipSuccess;
  ok = ok && hipMalloc((void**)&m->wt, sizeof(float) * M * K) == hipSuccess;
  ok = ok && hipMalloc((void**)&m->inv_rms, sizeof(float) * M) == hipSuccess;
  ok = ok && hipMalloc((void**)&m->lists, sizeof(int32_t) * K * E1 * M) == hipSuccess;
  ok = ok && hipMalloc((void**)&m->counts, sizeof(int32_t) * K * E1) == hipSuccess;
  ok = ok && hipMalloc((void**)&m->hbuf, 2 * M * K * q.d_expert) == hipSuccess;
  if (!ok) {
    tr_moe_free(m);
    return TR_ERR_HIP;
  }
  *out = m;
  return TR_OK;
}

tr_status tr_moe_free(tr_moe* m) {
  if (!m) return TR_OK;
  (void)hipDeviceSynchronize();
  for (void* p : {(void*)m->wg, (void*)m->wu, (void*)m->wd, (void*)m->sel, (void*)m->wt, (void*)m->inv_rms,
                  (void*)m->lists, (void*)m->counts, (void*)m->hbuf})
    if (p) (void)hipFree(p);
  delete m;
  return TR_OK;
}

tr_status tr_moe_set_weights(tr_moe* m, const void* w_gate, const void* w_up, const void* w_down, void* stream) {
  if (!m || !w_gate || !w_up || !w_down) return TR_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t per_up = (int64_t)(m->d / 16) * m->de * 2, per_dn = (int64_t)(m->de / 16) * m->d * 2;
  const unsigned gu = (unsigned)((per_up * m->E + 255) / 256), gd = (unsigned)((per_dn * m->E + 255) / 256);
  hipLaunchKernelGGL(k_moe_pack, dim3(gu), dim3(256), 0, st, static_cast<const uint16_t*>(w_gate), m->wg, m->de, m->d,
                     m->E);
  hipLaunchKernelGGL(k_moe_pack, dim3(gu), dim3(256), 0, st, static_cast<const uint16_t*>(w_up), m->wu, m->de, m->d,
                     m->E);
  hipLaunchKernelGGL(k_moe_pack, dim3(gd), dim3(256), 0, st, static_cast<const uint16_t*>(w_down), m->wd, m->d, m->de,
                     m->E);
  TR_LAUNCH_CHECK();
  m->weights_set = true;
  return TR_OK;
}

tr_status tr_moe_ffn(tr_moe* m, const void* x, const float* gate_logits, int32_t n_tokens, float* y, void* stream) {
  if (!m || n_tokens < 0 || n_tokens > m->max_tokens) return TR_ERR_INVALID_ARG;
  if (n_tokens == 0) return TR_OK;
  if (!x || !gate_logits || !y || !m->weights_set) return TR_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int M = n_tokens, E = m->E, K = m->k;
  hipLaunchKernelGGL(k_moe_route, dim3((M + 3) / 4), dim3(256), 0, st, static_cast<const uint16_t*>(x), gate_logits,
                     M, m->d, E, K, m->sel, m->wt, m->inv_rms);
  hipLaunchKernelGGL(k_moe_lists, dim3(K * (E + 1)), dim3(1024), 0, st, m->sel, M, K, E, m->max_tokens, m->lists,
                     m->counts);
  // upper bounds on the tile counts (the workgroups past the real count exit at once)
  auto run = [&](auto mb) {
    constexpr int MB = decltype(mb)::value, T = 32 * MB;
    const int tiles_up = K * ((M + T - 1) / T) + K * E;
    hipLaunchKernelGGL(k_moe_up<MB>, dim3(tiles_up, m->de / kUnits), dim3(256), 0, st, static_cast<const uint16_t*>(x),
                       m->lists, m->counts, m->inv_rms, m->wg, m->wu, m->hbuf, m->d, m->de, E, K, m->max_tokens);
    const int tiles_dn = (M + T - 1) / T + E + 1;
    for (int s = 0; s < K; ++s)
      hipLaunchKernelGGL(k_moe_down<MB>, dim3(tiles_dn, m->d / kUnits), dim3(256), 0, st, m->hbuf, m->lists,
                         m->counts, m->wt, m->wd, y, m->d, m->de, E, K, m->max_tokens, s);
  };
  if (M > kSmallCall) run(std::integral_constant<int, 2>());
  else run(std::integral_constant<int, 1>());
  TR_LAUNCH_CHECK();
  return TR_OK;
}

}  // extern "C"
