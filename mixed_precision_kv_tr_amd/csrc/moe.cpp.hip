// Expert FFN with a null expert (TriRoute review page, xllm-io.github.io: "core formulas" item 3,
// Eq. (3)): FFN_t = sum_{j in S_t} p_tj / sum_{S_t} p * f_j(Norm(x_t)), p_t = softmax(z_t^e) over
// E experts plus the null expert f_0 = 0, S_t the top-k; each expert a SwiGLU FFN
// f(u) = W2 (silu(W1 u) * (W3 u)) with hidden width d_e.
//
// One call = four launches (five for calls of at most kSmallCall tokens with top-2):
//   k_moe_route   one wave per token: 1 / rms(x_t), the top-k of the logits (ties to the lower
//                 index) and the renormalized weights exp(z_j - z_max) / sum over S_t.
//   k_moe_lists   one workgroup per (slot, expert, null included): the tokens whose slot-th
//                 choice is that expert, in token order (a block scan) -- the ragged batches.
//   k_moe_up      one workgroup per (slot, expert, 32 or 64 listed tokens, 128 hidden units): the gate
//                 and up products on the matrix cores (x rows gathered from the list, bf16 x and
//                 packed bf16 W1 / W3 as exact operands, fp32 accumulation), then the RMSNorm
//                 scale, silu(g) * u, stored into the hidden buffer in fp16 (11 significant bits;
//                 an |h| beyond fp16's range sets the sticky TR_ERRF_RANGE flag).
//   k_moe_down    per slot, in slot order: one workgroup per (expert, 32 or 64 listed tokens, 128 output
//                 channels): the down product of the gathered fp16 hidden rows against the fp16
//                 copy of W2 (packed once; exact for bf16 weights in fp16's range), times the token's
//                 weight, stored (slot 0; the null expert stores zeros) or added (slot 1) into the
//                 fp32 output -- no atomics, so the result does not depend on scheduling.  Calls of
//                 at most kSmallCall tokens with top-2 run every slot in one launch, each tile split
//                 into halves of the hidden channels, every (token, slot, half) row stored apart,
//                 and k_moe_ysum adds them in a fixed order.  Calls above kSmallCall tokens take
//                 the tiled forms k_moe_up_t / k_moe_down_t (below).
// Weight matrices are packed once (tr_moe_set_weights) into the operand order of the matrix-core
// k-loop: for k-step s = 4 g + j and output unit n, 16 values (bf16 for W1 / W3, fp16 for W2)
// holding input channels 64 g + 8 j .. + 7 and 64 g + 32 + 8 j .. + 7, so that the 32 units of a
// wave read one contiguous 1 KB per k-step.  The gathered activation rows of a tile are shared by its four waves: each stage of
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
  uint16_t* hbuf;    // [max_tokens * k][de] fp16 hidden rows (row t * k + slot)
  uint32_t* err;     // sticky TR_ERRF_* flags
  float* ys;         // [k][kDownSplit][kSmallCall][d] partial down-product rows of calls of <= kSmallCall tokens
  bool weights_set;
};

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
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

// fp16 bits of x (round to nearest even); an |x| beyond fp16's range (an infinity after rounding,
// or a NaN) sets TR_ERRF_RANGE in *err.
__device__ __forceinline__ uint16_t f16_checked(float x, uint32_t* err) {
  const _Float16 v = (_Float16)x;
  if (!(fabsf((float)v) <= 65504.0f)) atomicOr(err, TR_ERRF_RANGE);
  return __builtin_bit_cast(uint16_t, v);
}

__device__ __forceinline__ f32x16 mfma_f16(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                0);
}

__device__ __forceinline__ f32x16 mfma(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// Pack E matrices [units][K] (out x in) into the k-step operand order [K / 16][units][16].
// to_f16: the packed copy holds the fp16 rounding of each bf16 weight (exact in fp16's normal
// range; a weight beyond fp16's range sets TR_ERRF_RANGE).
__global__ __launch_bounds__(256) void k_moe_pack(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                  int units, int K, int E, int to_f16, uint32_t* __restrict__ err) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per = (int64_t)(K / 16) * units * 2;
  if (i >= per * E) return;
  const int e = (int)(i / per);
  const int64_t r = i % per;
  const int h = (int)(r & 1), n = (int)((r >> 1) % units), s = (int)((r >> 1) / units);
  const int g = s >> 2, j = s & 3;
  const int64_t mat = (int64_t)units * K;
  uint4 v = *reinterpret_cast<const uint4*>(src + e * mat + (int64_t)n * K + 64 * g + 32 * h + 8 * j);
  if (to_f16) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = (uint32_t)f16_checked(tr_bf16_lo(w[q]), err) | ((uint32_t)f16_checked(tr_bf16_hi(w[q]), err) << 16);
    v = make_uint4(w[0], w[1], w[2], w[3]);
  }
  *reinterpret_cast<uint4*>(dst + e * mat + ((int64_t)s * units + n) * 16 + 8 * h) = v;
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
// Work item of workgroup `b` of a 1-D grid of n: consecutive workgroups go to the eight XCDs in
// turn, so XCD x (= b % 8) gets the contiguous range of items [start_x, start_x + count_x) --
// items listed weight block by weight block then share their block in that XCD's L2 instead of
// every XCD fetching it.
__device__ __forceinline__ int xcd_item(int b, int n) {
  constexpr int kXcd = 8;
  const int x = b % kXcd, i = b / kXcd, q = n / kXcd, r = n % kXcd;
  return x * q + min(x, r) + i;
}

// Token tile `id` of the up products, expert by expert and, within an expert, slot by slot (so the
// tiles of both slots that read one expert's weights are listed together).
template <int kTile>
__device__ __forceinline__ bool find_tile_expert_major(const int32_t* counts, int E, int K, int id, int& slot, int& e,
                                                       int& tile, int& cnt) {
  for (int x = 1; x <= E; ++x) {
    for (int s = 0; s < K; ++s) {
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

constexpr int kDownSplit = 2;     // hidden-channel halves of the small calls' down product

// Tiles of every slot, expert by expert (the null expert first), the slots of an expert side by
// side, so that the workgroups reading one expert's weights run close together.
template <int kTile>
__device__ __forceinline__ bool find_tile_all(const int32_t* counts, int E, int K, int id, int& slot, int& e, int& tile,
                                              int& cnt) {
  for (int x = 0; x <= E; ++x) {
    for (int s = 0; s < K; ++s) {
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
                                                uint16_t* __restrict__ hbuf, int d, int de, int E, int k, int cap,
                                                int ntiles, uint32_t* __restrict__ err) {
  constexpr int kTile = 32 * kMB;
  __shared__ int32_t tok[kTile];
  __shared__ float inv[kTile];
  // work item: (block of 128 hidden units, token tile), unit block by unit block
  const int item = xcd_item(blockIdx.x, (int)gridDim.x);
  const int ublk = item / ntiles;
  int slot, e, tile, cnt;
  if (!find_tile_expert_major<kTile>(counts, E, k, item % ntiles, slot, e, tile, cnt)) return;
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
  const int n = ublk * kUnits + 32 * wave + r;      // hidden unit of this lane's B column
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
        hbuf[((int64_t)tok[row] * k + slot) * de + n] = f16_checked(h, err);
      }
    }
  }
}

// Gate and up products on a tile of 256 listed tokens x 128 hidden units (large calls): 8 waves,
// each 64 tokens x 64 units of both products.  Per stage of 64 input channels the workgroup loads
// the tile's x rows (A, 16-byte-padded rows) and the two weight blocks (B, in their packed k-step
// order) into double-buffered LDS, one 64-byte piece of each per thread, the next stage in
// registers while the current one multiplies: every weight byte brought in serves 256 tokens and
// every x byte 128 units, against 64 and 128 in k_moe_up.  Epilogue as in k_moe_up.
// Workgroup barrier for the stage pipelines that orders LDS only: the wave's LDS accesses
// complete, then s_barrier.  __syncthreads() also carries a workgroup-scope memory fence, which
// waits for every global load of the wave, including the next stage's, issued a stage earlier to
// stay in flight across the barrier.  The empty asm statements keep the compiler from moving
// memory accesses across (the barrier builtin itself does not).
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);              // lgkmcnt(0); vmcnt and expcnt untouched
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

constexpr int kTM = 256;                 // listed tokens per tile
constexpr int kGY = 4;                   // unit blocks per group in the work order

// Items of the tiled up products, expert by expert: for expert e with T_e token tiles (both slots)
// and NY unit blocks, groups of kGY unit blocks, within a group token tile by token tile, within
// a tile its kGY unit blocks.  The XCD ranges (xcd_item) then give each XCD about one expert, and
// the ~32 workgroups it runs at once share kGY weight blocks and a few token tiles in its L2.
// Returns the item count when id < 0.
__device__ __forceinline__ int up_item(const int32_t* counts, int E, int K, int NY, int id, int& slot, int& e, int& tile,
                                       int& cnt, int& y) {
  int base = 0;
  for (int x = 1; x <= E; ++x) {
    int te = 0;
    for (int s = 0; s < K; ++s) te += (counts[s * (E + 1) + x] + kTM - 1) / kTM;
    const int ne = te * NY;
    if (id >= base && id < base + ne) {
      const int i = id - base, nfull = NY / kGY;
      int t;
      if (i < nfull * te * kGY) {
        const int r2 = i % (te * kGY);
        t = r2 / kGY;
        y = (i / (te * kGY)) * kGY + r2 % kGY;
      } else {
        const int i2 = i - nfull * te * kGY, gs = NY - nfull * kGY;
        t = i2 / gs;
        y = nfull * kGY + i2 % gs;
      }
      for (int s = 0; s < K; ++s) {
        const int c = counts[s * (E + 1) + x];
        const int nt = (c + kTM - 1) / kTM;
        if (t < nt) {
          slot = s;
          e = x;
          tile = t;
          cnt = c;
          return 1;
        }
        t -= nt;
      }
      return 0;
    }
    base += ne;
  }
  return id < 0 ? base : 0;
}
constexpr int kTN = 128;                 // hidden units per tile
constexpr int kAP = 144;                 // LDS bytes per A row: 64 channels + 16 bytes
constexpr int kBS = 2 * 4 * kTN * 32;    // LDS bytes of one stage's B tiles: [gate, up][k-step][unit][16]

__global__ __launch_bounds__(512) void k_moe_up_t(const uint16_t* __restrict__ x, const int32_t* __restrict__ lists,
                                                  const int32_t* __restrict__ counts,
                                                  const float* __restrict__ inv_rms, const uint16_t* __restrict__ wg,
                                                  const uint16_t* __restrict__ wu, uint16_t* __restrict__ hbuf, int d,
                                                  int de, int E, int k, int cap, uint32_t* __restrict__ err) {
  __shared__ int32_t tok[kTM];
  __shared__ float inv[kTM];
  __shared__ __align__(16) uint8_t As[2][kTM * kAP];
  __shared__ __align__(16) uint8_t Bs[2][kBS];
  int slot = 0, e = 0, tile = 0, cnt = 0, ublk = 0;
  const int nitems = up_item(counts, E, k, de / kTN, -1, slot, e, tile, cnt, ublk);
  if ((int)blockIdx.x >= nitems) return;
  if (!up_item(counts, E, k, de / kTN, xcd_item(blockIdx.x, nitems), slot, e, tile, cnt, ublk)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ntok = min(kTM, cnt - tile * kTM);
  const int32_t* lst = lists + (int64_t)(slot * (E + 1) + e) * cap + tile * kTM;
  if (tid < kTM) {
    const int t = lst[min(tid, ntok - 1)];         // rows past the list's end repeat its last token
    tok[tid] = t;
    inv[tid] = inv_rms[t];
  }
  __syncthreads();
  // this thread's pieces of a stage g (channels 64 g .. 64 g + 63):
  //   A: row tid / 2, channels 32 (tid % 2) .. + 31 of the stage
  //   B: piece c = tid / 64 = (matrix c / 4, k-step 4 g + c % 4), units 2 (tid % 64) and + 1
  const int arow = tid >> 1, ahalf = tid & 1;
  const uint16_t* xa = x + (int64_t)tok[arow] * d + 32 * ahalf;
  const int bc = tid >> 6, bn = 2 * (tid & 63);
  const int64_t mat = (int64_t)de * d;
  const uint16_t* wb = ((bc >> 2) ? wu : wg) + (int64_t)(e - 1) * mat + ((int64_t)(bc & 3) * de + ublk * kTN + bn) * 16;
  const int64_t gstep = (int64_t)4 * de * 16;     // elements per stage of 4 k-steps
  // two register sets, one and two stages ahead of the stage being multiplied
  uint4 ra0[4], rb0[4], ra1[4], rb1[4];
  auto gl = [&](int g, uint4 (&ra)[4], uint4 (&rb)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ra[q] = gload16(xa + 64 * g + 8 * q);
      rb[q] = gload16(wb + g * gstep + 8 * q);
    }
  };
  auto st = [&](int b, const uint4 (&ra)[4], const uint4 (&rb)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<uint4*>(&As[b][arow * kAP + 64 * ahalf + 16 * q]) = ra[q];
      // unit u's two 16-byte halves swap places when bit 3 of u is set (see compute)
      const int u = bn + (q >> 1);
      *reinterpret_cast<uint4*>(&Bs[b][(bc * kTN + u) * 32 + 16 * ((q & 1) ^ ((u >> 3) & 1))]) = rb[q];
    }
  };
  const int r = lane & 31, kh = lane >> 5;
  const int tw = wave & 3, uw = wave >> 2;          // this wave: tokens 64 tw .., units 64 uw ..
  f32x16 acc[2][2][2] = {};                         // [gate, up][token block][unit block]
  // operands of k-step j of buffer b
  auto rd = [&](int b, int j, uint4 (&av)[2], uint4 (&bv)[2][2]) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
      av[tb] = *reinterpret_cast<const uint4*>(&As[b][(64 * tw + 32 * tb + r) * kAP + 16 * j + 64 * kh]);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int ub = 0; ub < 2; ++ub) {
        // units r and r + 8 of a 16-lane pass would share banks at a 32-byte pitch: the halves
        // of every unit with bit 3 set are stored swapped
        const int u = 64 * uw + 32 * ub + r;
        bv[m][ub] = *reinterpret_cast<const uint4*>(&Bs[b][((4 * m + j) * kTN + u) * 32 + 16 * (kh ^ ((u >> 3) & 1))]);
      }
  };
  // the 4 k-steps of a stage, each k-step's LDS reads issued before the previous one's products
  // (scheduling barriers keep the order), so the reads' latency hides behind 8 products
  auto compute = [&](int b) {
    uint4 av0[2], bv0[2][2], av1[2], bv1[2][2];
    rd(b, 0, av0, bv0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4(&av)[2] = (j & 1) ? av1 : av0;
      uint4(&bv)[2][2] = (j & 1) ? bv1 : bv0;
      if (j < 3) rd(b, j + 1, (j & 1) ? av0 : av1, (j & 1) ? bv0 : bv1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int ub = 0; ub < 2; ++ub) acc[m][tb][ub] = mfma(av[tb], bv[m][ub], acc[m][tb][ub]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const int ns = d / 64;                            // even: d is a multiple of 128
  gl(0, ra0, rb0);
  st(0, ra0, rb0);
  __syncthreads();
  // stage 1's loads strictly before stage 2's, as in the loop: the wait before each stage's LDS
  // stores then leaves the later stage's loads in flight (with the two sets issued the other way
  // round here, the compiler's wait at the loop head, valid for both orders, is a full drain)
  gl(min(1, ns - 1), ra0, rb0);
  __builtin_amdgcn_sched_barrier(0);
  gl(min(2, ns - 1), ra1, rb1);
  // stage g sits in LDS buffer g & 1; the loop is unrolled by two so that each register set keeps
  // its registers (set 0 holds the odd stages, set 1 the even ones); loads are clamped, never
  // branched around
  for (int g = 0; g < ns; g += 2) {
    compute(0);
    st(1, ra0, rb0);                                // stage g + 1
    lds_barrier();
    gl(min(g + 3, ns - 1), ra0, rb0);
    compute(1);
    st(0, ra1, rb1);                                // stage g + 2 (a repeat of the last one at the end)
    lds_barrier();
    gl(min(g + 4, ns - 1), ra1, rb1);
  }
  // D[token][unit]: lane (r, kh) holds unit r of its unit block for rows 8 (reg / 4) + 4 kh + reg % 4
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int ub = 0; ub < 2; ++ub)
#pragma unroll
      for (int reg = 0; reg < 16; ++reg) {
        const int row = 64 * tw + 32 * tb + 8 * (reg >> 2) + 4 * kh + (reg & 3);
        if (row < ntok) {
          const int n = ublk * kTN + 64 * uw + 32 * ub + r;
          const float gv = acc[0][tb][ub][reg] * inv[row], uv = acc[1][tb][ub][reg] * inv[row];
          const float h = gv / (1.0f + expf(-gv)) * uv;
          hbuf[((int64_t)tok[row] * k + slot) * de + n] = f16_checked(h, err);
        }
      }
}

// Down product: 32 kMB tokens of one (slot, expert) list and 128 output channels.  With ys null,
// the tiles of one slot, stored into y (slot 0) or added to it (later slots); otherwise the tiles
// of every slot in one launch, each also split into kDownSplit halves of the hidden channels,
// each (token, slot, half) row stored into ys[slot][half][token] (kSmallCall rows each), the null
// expert's as zeros, for k_moe_ysum to add in a fixed order.
template <int kMB>
__global__ __launch_bounds__(256) void k_moe_down(const uint16_t* __restrict__ hbuf, const int32_t* __restrict__ lists,
                                                  const int32_t* __restrict__ counts, const float* __restrict__ wt,
                                                  const uint16_t* __restrict__ wd, float* __restrict__ y, int d, int de,
                                                  int E, int k, int cap, int slot_arg, int ntiles,
                                                  float* __restrict__ ys) {
  constexpr int kTile = 32 * kMB;
  __shared__ int32_t tok[kTile];
  __shared__ float wgt[kTile];
  // work item: (block of 128 output channels, token tile), channel block by channel block
  const int item0 = xcd_item(blockIdx.x, (int)gridDim.x);
  const int half = ys ? item0 % kDownSplit : 0;    // the halves of a tile run side by side
  const int item = ys ? item0 / kDownSplit : item0;
  const int cblk = item / ntiles;
  int slot, e, tile, cnt;
  // slot 0 also takes the null expert's tiles (zeros); later slots skip it
  if (ys ? !find_tile_all<kTile>(counts, E, k, item % ntiles, slot, e, tile, cnt)
         : !find_tile<kTile>(counts, E, slot_arg, slot_arg + 1, slot_arg == 0 ? 0 : 1, item % ntiles, slot, e, tile,
                             cnt))
    return;
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
  const int n = cblk * kUnits + 32 * wave + r;      // output channel of this lane's B column
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
    // this workgroup's k-steps: all of them, or one half (ns is a multiple of 8, a half of 4)
    const int s0 = ys ? half * (ns / kDownSplit) : 0, s1 = ys ? s0 + ns / kDownSplit : ns;
    hs[0][prow][pp] = gload16(haddr(s0));
    wload(s0, wa);
    __syncthreads();
    int buf = 0;
    for (int st = s0; st < s1; st += kPS) {
      const int nx = min(st + kPS, s1 - kPS);
      const uint4 hn = gload16(haddr(nx));
      uint4 wn[kPS];
      wload(nx, wn);
#pragma unroll
      for (int q = 0; q < kPS; ++q)
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) {
          acc[mb] = mfma_f16(hs[buf][32 * mb + r][2 * q + kh], wa[q], acc[mb]);
        }
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
        const float v = e > 0 ? acc[mb][reg] * wgt[row] : 0.0f;
        if (ys) {
          ys[((int64_t)(slot * kDownSplit + half) * kSmallCall + tok[row]) * d + n] = v;
        } else {
          float* dst = y + (int64_t)tok[row] * d + n;
          if (slot == 0) *dst = v;
          else *dst += v;
        }
      }
    }
  }
}

// y = the sum of the (slot, half) rows k_moe_down stored in ys, slot by slot and half by half
// (a fixed order, so the result does not depend on scheduling).
__global__ __launch_bounds__(256) void k_moe_ysum(const float* __restrict__ ys, float* __restrict__ y, int M, int d,
                                                  int k) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;          // float4 index
  if (i >= (int64_t)M * d / 4) return;
  const int64_t t = i / (d / 4), c4 = i % (d / 4);
  float4 acc = reinterpret_cast<const float4*>(ys + t * d)[c4];
  for (int s = 1; s < k * kDownSplit; ++s) {
    const float4 v = reinterpret_cast<const float4*>(ys + ((int64_t)s * kSmallCall + t) * d)[c4];
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  reinterpret_cast<float4*>(y + t * d)[c4] = acc;
}

// Down product of one slot on a tile of 128 listed tokens x 256 output channels (large calls, d a
// multiple of 256): 8 waves, each 64 tokens x 64 channels.  Per stage of 64 hidden channels the
// workgroup loads the tile's fp16 hidden rows (16-byte-padded rows; 32 bytes per thread) and the
// fp16 weight block (in its packed k-step order; 64 bytes per thread) into double-buffered LDS,
// the next two stages in registers: every weight byte brought in serves 128 tokens and every
// hidden byte 256 channels, against 64 and 128 in k_moe_down.  Epilogue as in k_moe_down.
constexpr int kDM = 128;                 // listed tokens per tile
constexpr int kDN = 256;                 // output channels per tile
constexpr int kDBS = 4 * kDN * 32;       // LDS bytes of one stage's B tile: [k-step][channel][16]

// Items of the tiled down product of one slot, expert by expert (the null expert first in slot 0:
// its tiles only write zeros): for expert e with T_e token tiles and NY channel blocks, groups of
// kGY channel blocks, within a group token tile by token tile, within a tile its kGY blocks, as
// in up_item.  Returns the item count when id < 0.
__device__ __forceinline__ int down_item(const int32_t* counts, int E, int slot, int NY, int id, int& e, int& tile,
                                         int& cnt, int& y) {
  int base = 0;
  for (int x = slot == 0 ? 0 : 1; x <= E; ++x) {
    const int c = counts[slot * (E + 1) + x];
    const int te = (c + kDM - 1) / kDM;
    const int ne = te * NY;
    if (id >= base && id < base + ne) {
      const int i = id - base, nfull = NY / kGY;
      if (i < nfull * te * kGY) {
        const int r2 = i % (te * kGY);
        tile = r2 / kGY;
        y = (i / (te * kGY)) * kGY + r2 % kGY;
      } else {
        const int i2 = i - nfull * te * kGY, gs = NY - nfull * kGY;
        tile = i2 / gs;
        y = nfull * kGY + i2 % gs;
      }
      e = x;
      cnt = c;
      return 1;
    }
    base += ne;
  }
  return id < 0 ? base : 0;
}

__global__ __launch_bounds__(512) void k_moe_down_t(const uint16_t* __restrict__ hbuf, const int32_t* __restrict__ lists,
                                                    const int32_t* __restrict__ counts, const float* __restrict__ wt,
                                                    const uint16_t* __restrict__ wd, float* __restrict__ y, int d, int de,
                                                    int E, int k, int cap, int slot) {
  __shared__ int32_t tok[kDM];
  __shared__ float wgt[kDM];
  __shared__ __align__(16) uint8_t As[2][kDM * kAP];         // [buffer][row]
  __shared__ __align__(16) uint8_t Bs[2][kDBS];
  int e = 0, tile = 0, cnt = 0, cblk = 0;
  const int nitems = down_item(counts, E, slot, d / kDN, -1, e, tile, cnt, cblk);
  if ((int)blockIdx.x >= nitems) return;
  if (!down_item(counts, E, slot, d / kDN, xcd_item(blockIdx.x, nitems), e, tile, cnt, cblk)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ntok = min(kDM, cnt - tile * kDM);
  const int32_t* lst = lists + (int64_t)(slot * (E + 1) + e) * cap + tile * kDM;
  if (tid < kDM) {
    const int t = lst[min(tid, ntok - 1)];         // rows past the list's end repeat its last token
    tok[tid] = t;
    wgt[tid] = wt[t * k + slot];
  }
  __syncthreads();
  const int r = lane & 31, kh = lane >> 5;
  const int tw = wave & 1, uw = wave >> 1;          // this wave: tokens 64 tw .., channels 64 uw ..
  f32x16 acc[2][2] = {};                            // [token block][channel block]
  if (e > 0) {
    // this thread's pieces of a stage g (hidden channels 64 g .. 64 g + 63):
    //   A: row tid / 4, channels 16 (tid % 4) .. + 15 of the stage
    //   B: k-step 4 g + tid / 128, channels 2 (tid % 128) and + 1 of the block
    const int arow = tid >> 2, aq = tid & 3;
    const uint16_t* ha = hbuf + ((int64_t)tok[arow] * k + slot) * de + 16 * aq;
    const int bc = tid >> 7, bn = 2 * (tid & 127);
    const uint16_t* wb = wd + (int64_t)(e - 1) * d * de + ((int64_t)bc * d + cblk * kDN + bn) * 16;
    const int64_t gstep = (int64_t)4 * d * 16;      // elements per stage of 4 k-steps
    uint4 ra0[2], rb0[4], ra1[2], rb1[4];
    auto gl = [&](int g, uint4 (&ra)[2], uint4 (&rb)[4]) {
#pragma unroll
      for (int q = 0; q < 2; ++q) ra[q] = gload16(ha + 64 * g + 8 * q);
#pragma unroll
      for (int q = 0; q < 4; ++q) rb[q] = gload16(wb + g * gstep + 8 * q);
    };
    auto st = [&](int b, const uint4 (&ra)[2], const uint4 (&rb)[4]) {
#pragma unroll
      for (int q = 0; q < 2; ++q) *reinterpret_cast<uint4*>(&As[b][arow * kAP + 32 * aq + 16 * q]) = ra[q];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // channel u's two 16-byte halves swap places when bit 3 of u is set (see compute)
        const int u = bn + (q >> 1);
        *reinterpret_cast<uint4*>(&Bs[b][(bc * kDN + u) * 32 + 16 * ((q & 1) ^ ((u >> 3) & 1))]) = rb[q];
      }
    };
    auto rd = [&](int b, int j, uint4 (&av)[2], uint4 (&bv)[2]) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
        av[tb] = *reinterpret_cast<const uint4*>(&As[b][(64 * tw + 32 * tb + r) * kAP + 16 * j + 64 * kh]);
#pragma unroll
      for (int ub = 0; ub < 2; ++ub) {
        const int u = 64 * uw + 32 * ub + r;
        bv[ub] = *reinterpret_cast<const uint4*>(&Bs[b][(j * kDN + u) * 32 + 16 * (kh ^ ((u >> 3) & 1))]);
      }
    };
    // as in k_moe_up_t: each k-step's reads go out before the previous k-step's products
    auto compute = [&](int b) {
      uint4 av0[2], bv0[2], av1[2], bv1[2];
      rd(b, 0, av0, bv0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint4(&av)[2] = (j & 1) ? av1 : av0;
        uint4(&bv)[2] = (j & 1) ? bv1 : bv0;
        if (j < 3) rd(b, j + 1, (j & 1) ? av0 : av1, (j & 1) ? bv0 : bv1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int ub = 0; ub < 2; ++ub) acc[tb][ub] = mfma_f16(av[tb], bv[ub], acc[tb][ub]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    const int ns = de / 64;                         // even: de is a multiple of 128
    gl(0, ra0, rb0);
    st(0, ra0, rb0);
    __syncthreads();
    gl(min(1, ns - 1), ra0, rb0);                  // in order, as in k_moe_up_t
    __builtin_amdgcn_sched_barrier(0);
    gl(min(2, ns - 1), ra1, rb1);
    for (int g = 0; g < ns; g += 2) {
      compute(0);
      st(1, ra0, rb0);                              // stage g + 1
      lds_barrier();
      gl(min(g + 3, ns - 1), ra0, rb0);
      compute(1);
      st(0, ra1, rb1);                              // stage g + 2 (a repeat of the last one at the end)
      lds_barrier();
      gl(min(g + 4, ns - 1), ra1, rb1);
    }
  }
  // D[token][channel]: lane (r, kh) holds channel r of its block for rows 8 (reg / 4) + 4 kh + reg % 4
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int ub = 0; ub < 2; ++ub)
#pragma unroll
      for (int reg = 0; reg < 16; ++reg) {
        const int row = 64 * tw + 32 * tb + 8 * (reg >> 2) + 4 * kh + (reg & 3);
        if (row < ntok) {
          float* dst = y + (int64_t)tok[row] * d + cblk * kDN + 64 * uw + 32 * ub + r;
          const float v = e > 0 ? acc[tb][ub][reg] * wgt[row] : 0.0f;
          if (slot == 0) *dst = v;
          else *dst += v;
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
  ok = ok && hipMalloc((void**)&m->err, sizeof(uint32_t)) == hipSuccess;
  ok = ok && hipMalloc((void**)&m->ys, sizeof(float) * K * kDownSplit * kSmallCall * q.d) == hipSuccess;
  ok = ok && hipMemset(m->err, 0, sizeof(uint32_t)) == hipSuccess;
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
                  (void*)m->lists, (void*)m->counts, (void*)m->hbuf, (void*)m->err, (void*)m->ys})
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
                     m->E, 0, m->err);
  hipLaunchKernelGGL(k_moe_pack, dim3(gu), dim3(256), 0, st, static_cast<const uint16_t*>(w_up), m->wu, m->de, m->d,
                     m->E, 0, m->err);
  hipLaunchKernelGGL(k_moe_pack, dim3(gd), dim3(256), 0, st, static_cast<const uint16_t*>(w_down), m->wd, m->d, m->de,
                     m->E, 1, m->err);
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
    // 1-D grids of (unit block, token tile) items, see xcd_item
    if (MB == 2) {
      const int tiles_up = K * ((M + kTM - 1) / kTM) + K * E;
      hipLaunchKernelGGL(k_moe_up_t, dim3(tiles_up * (m->de / kTN)), dim3(512), 0, st, static_cast<const uint16_t*>(x),
                         m->lists, m->counts, m->inv_rms, m->wg, m->wu, m->hbuf, m->d, m->de, E, K, m->max_tokens,
                         m->err);
    } else {
      const int tiles_up = K * ((M + T - 1) / T) + K * E;
      hipLaunchKernelGGL(k_moe_up<MB>, dim3(tiles_up * (m->de / kUnits)), dim3(256), 0, st,
                         static_cast<const uint16_t*>(x), m->lists, m->counts, m->inv_rms, m->wg, m->wu, m->hbuf, m->d,
                         m->de, E, K, m->max_tokens, tiles_up, m->err);
    }
    if (MB == 2 && m->d % kDN == 0) {
      const int tiles_dn = (M + kDM - 1) / kDM + E + 1;
      for (int s = 0; s < K; ++s)
        hipLaunchKernelGGL(k_moe_down_t, dim3(tiles_dn * (m->d / kDN)), dim3(512), 0, st, m->hbuf, m->lists, m->counts,
                           m->wt, m->wd, y, m->d, m->de, E, K, m->max_tokens, s);
    } else if (MB == 1 && K > 1) {
      // small calls: every slot's tiles in one launch, each split into halves of the hidden
      // channels (four times the workgroups of a slot's launch, each expert's weights read by
      // its slots' tiles together), then the sum
      const int tiles_dn = K * ((M + T - 1) / T + E + 1);
      hipLaunchKernelGGL(k_moe_down<MB>, dim3(tiles_dn * (m->d / kUnits) * kDownSplit), dim3(256), 0, st, m->hbuf,
                         m->lists, m->counts, m->wt, m->wd, y, m->d, m->de, E, K, m->max_tokens, 0, tiles_dn, m->ys);
      hipLaunchKernelGGL(k_moe_ysum, dim3((unsigned)(((int64_t)M * m->d / 4 + 255) / 256)), dim3(256), 0, st, m->ys, y,
                         M, m->d, K);
    } else {
      const int tiles_dn = (M + T - 1) / T + E + 1;
      for (int s = 0; s < K; ++s)
        hipLaunchKernelGGL(k_moe_down<MB>, dim3(tiles_dn * (m->d / kUnits)), dim3(256), 0, st, m->hbuf, m->lists,
                           m->counts, m->wt, m->wd, y, m->d, m->de, E, K, m->max_tokens, s, tiles_dn,
                           static_cast<float*>(nullptr));
    }
  };
  if (M > kSmallCall) run(std::integral_constant<int, 2>());
  else run(std::integral_constant<int, 1>());
  TR_LAUNCH_CHECK();
  return TR_OK;
}

tr_status tr_moe_status(tr_moe* m, void* stream) {
  if (!m) return TR_ERR_INVALID_ARG;
  uint32_t flags = 0;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return TR_ERR_HIP;
  if (hipMemcpy(&flags, m->err, sizeof(flags), hipMemcpyDeviceToHost) != hipSuccess) return TR_ERR_HIP;
  return (flags & TR_ERRF_RANGE) ? TR_ERR_RANGE : TR_OK;
}

}  // extern "C"
