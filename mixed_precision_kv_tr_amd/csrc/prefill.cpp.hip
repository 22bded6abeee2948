// Prefill routed attention over the mixed-width paged cache (TriRoute review page,
// xllm-io.github.io: Eq. (2) for every query of the prompt, reading the K/V that Eq. (4) has
// just written -- the inference paragraph after Algorithm 1).
//
// k_prefill_compact (one workgroup per (seq, head)): stable partition of the T query rows
//   by mode -- full rows, then local rows -- so that a 128-row tile holds one mode and its
//   key range is tight; skip rows (and rows with an invalid mode) get zeros right here.
// k_prefill_attn (one workgroup = 4 waves = one 128-row tile):
//   key range of the tile = union of its rows' windows, mapped through the class prefix
//   counts to one slot range per width class; the four ranges are walked as one virtual
//   stream in 32-key tiles.  Per tile:
//     staging   K codes -> LDS as bf16 integers (exact; b = 16 keeps its bf16 bits), key-major;
//               V -> v_hat = s*c + z in fp32 -> fp16, channel-major (transposed);
//               per key alpha = s_K * log2(e)/sqrt(D), beta = z_K * log2(e)/sqrt(D), position.
//     QK^T      S^T[32 keys x 32 queries] per wave = v_mfma_f32_32x32x16_bf16 over D/16 steps;
//               the score is alpha * (q . c) + beta * sum(q) -- Eq. (4)'s reconstruction
//               folded out of the product, so K stays exact in the matrix cores.
//     softmax   fp32 in registers, each lane holds 16 keys of one query; running max with a
//               lazy rescale (only when the max grows by more than 2^8), mask only on tiles
//               that cross a row's window edge; waves skip tiles outside their own window.
//     PV        O^T[D x 32 queries] += V^T P^T with v_mfma_f32_32x32x16_f16; P is the lane's
//               own scores (the key order of the S^T layout is mirrored in the V^T read).
//   epilogue  O / l -> bf16, scattered back to the rows' original positions.
#include <math.h>
#include <stdint.h>

#include "common.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBlock = 256;
constexpr int BM = 128;       // query rows per workgroup (4 waves x 32)
constexpr int BN = 32;        // keys per tile
constexpr float kRescale = 8.0f;

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  return v;
}

// Stable partition of the query rows of one (seq, head) by mode.
template <int D>
__global__ __launch_bounds__(kBlock) void k_prefill_compact(CacheLayout c, int T, const uint8_t* __restrict__ mode,
                                                            int32_t* __restrict__ rows, int32_t* __restrict__ counts,
                                                            uint16_t* __restrict__ out) {
  __shared__ uint32_t wsum[kBlock / 64];
  __shared__ int32_t nfull_s, run_f, run_l;
  const int sh = blockIdx.x;
  const int s = sh / c.H, h = sh % c.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int32_t* rl = rows + (int64_t)sh * c.N;
  // pass 1: number of full rows
  uint32_t nf = 0;
  for (int i = tid; i < T; i += kBlock) nf += mode[((int64_t)s * T + i) * c.H + h] == TR_MODE_FULL;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) nf += __shfl_xor(nf, o, 64);
  if (lane == 0) wsum[wave] = nf;
  __syncthreads();
  if (tid == 0) {
    nfull_s = (int)(wsum[0] + wsum[1] + wsum[2] + wsum[3]);
    run_f = 0;
    run_l = 0;
  }
  __syncthreads();
  const int nfull = nfull_s;
  // pass 2: ordered positions; full and local counters packed in 16-bit halves
  for (int chunk = 0; chunk < T; chunk += kBlock) {
    const int i = chunk + tid;
    int m = TR_MODE_SKIP;
    if (i < T) {
      m = mode[((int64_t)s * T + i) * c.H + h];
      if (m > TR_MODE_FULL) {
        atomicOr(c.err, TR_ERRF_BAD_MODE);
        m = TR_MODE_SKIP;
      }
      if (m == TR_MODE_SKIP) {
        uint4* o = reinterpret_cast<uint4*>(out + (((int64_t)s * T + i) * c.H + h) * D);
#pragma unroll
        for (int x = 0; x < D / 8; ++x) o[x] = make_uint4(0, 0, 0, 0);
      }
    }
    const uint32_t one = (m == TR_MODE_FULL) ? 1u : (m == TR_MODE_LOCAL) ? (1u << 16) : 0u;
    uint32_t incl = wave_incl_scan(one);
    __syncthreads();
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kBlock / 64; ++w) {
      if (w < wave) before += wsum[w];
      total += wsum[w];
    }
    const uint32_t excl = incl - one + before;
    if (m == TR_MODE_FULL) rl[run_f + (int)(excl & 0xffffu)] = i;
    if (m == TR_MODE_LOCAL) rl[nfull + run_l + (int)(excl >> 16)] = i;
    __syncthreads();
    if (tid == 0) {
      run_f += (int)(total & 0xffffu);
      run_l += (int)(total >> 16);
    }
  }
  __syncthreads();
  if (tid == 0) {
    counts[sh * 4 + 0] = nfull;
    counts[sh * 4 + 1] = run_l;
  }
}

template <int NB>
__device__ __forceinline__ uint32_t code_at(const uint32_t* w, int e) {
  return (w[(e * NB) >> 5] >> ((e * NB) & 31)) & ((1u << NB) - 1u);
}

// Load the DPT codes (or bf16 values) of one thread's channel slice of a key row.
template <int DPT>
__device__ __forceinline__ void load_slice(const uint8_t* p, int b, uint32_t* w) {
  const int bytes = DPT * b / 8;
  if (bytes == 2) {
    w[0] = *reinterpret_cast<const uint16_t*>(p);
  } else if (bytes == 4) {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if (bytes == 8) {
    const uint2 t = *reinterpret_cast<const uint2*>(p);
    w[0] = t.x; w[1] = t.y;
  } else if (bytes == 16) {
    const uint4 t = *reinterpret_cast<const uint4*>(p);
    w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
  } else {
    const uint4 t0 = reinterpret_cast<const uint4*>(p)[0];
    const uint4 t1 = reinterpret_cast<const uint4*>(p)[1];
    w[0] = t0.x; w[1] = t0.y; w[2] = t0.z; w[3] = t0.w;
    w[4] = t1.x; w[5] = t1.y; w[6] = t1.z; w[7] = t1.w;
  }
}

template <int DPT>
__device__ __forceinline__ float code_f(const uint32_t* w, int b, int e) {
  switch (b) {
    case 2: return (float)code_at<2>(w, e);
    case 4: return (float)code_at<4>(w, e);
    default: return (float)code_at<8>(w, e);
  }
}

template <int D>
struct PrefillSmem {
  uint16_t ks[BN][D + 8];      // K codes / bf16 values, key-major
  _Float16 vt[D][BN + 8];      // v_hat, channel-major
  float alpha[BN];
  float beta[BN];
  int32_t kpos[BN];
  int32_t wrange[4][4];        // per wave: lo, hi, tmin, lomax
};

template <int D>
__global__ __launch_bounds__(kBlock) void k_prefill_attn(CacheLayout c, int layer, int p0, int T, int window,
                                                         float kscale, const uint16_t* __restrict__ q,
                                                         const int32_t* __restrict__ rows,
                                                         const int32_t* __restrict__ counts,
                                                         uint16_t* __restrict__ out) {
  constexpr int DPT = D / 8;           // channels per thread when staging a key
  constexpr int KS = D / 16;           // MFMA k-steps for QK^T
  constexpr int MT = D / 32;           // 32-channel tiles of O^T
  __shared__ PrefillSmem<D> sm;

  const int BH = c.B * c.H;
  const int rank = blockIdx.x / BH, sh = blockIdx.x % BH;
  const int s = sh / c.H, h = sh % c.H;
  const int nf = counts[sh * 4 + 0], nl = counts[sh * 4 + 1];
  const int ftiles = (nf + BM - 1) / BM, ltiles = (nl + BM - 1) / BM;
  if (rank >= ftiles + ltiles) return;
  const bool full = rank < ftiles;
  int r0, rend;
  if (full) {                                   // heaviest full tiles first
    const int ft = ftiles - 1 - rank;
    r0 = ft * BM;
    rend = min(r0 + BM, nf);
  } else {
    r0 = nf + (rank - ftiles) * BM;
    rend = min(r0 + BM, nf + nl);
  }
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, g = lane >> 5;
  const int ri = r0 + wave * 32 + n;
  const bool row_ok = ri < rend;
  const int i = row_ok ? rows[(int64_t)sh * c.N + ri] : 0;
  const int t = row_ok ? p0 + i : -1;
  const int lo = row_ok ? (full ? 0 : max(0, t - window)) : 0x7fffffff;

  // Q^T operand (B of the QK^T MFMA): column n = query, k = channels 16*ks + 8*g .. +7.
  bf16x8 qb[KS];
  float qsum = 0.0f;
  const uint16_t* qrow = q + (((int64_t)s * T + i) * c.H + h) * D;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    uint4 raw = row_ok ? *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * g) : make_uint4(0, 0, 0, 0);
    qb[ks] = __builtin_bit_cast(bf16x8, raw);
    qsum += (tr_bf16_lo(raw.x) + tr_bf16_hi(raw.x)) + (tr_bf16_lo(raw.y) + tr_bf16_hi(raw.y)) +
            (tr_bf16_lo(raw.z) + tr_bf16_hi(raw.z)) + (tr_bf16_lo(raw.w) + tr_bf16_hi(raw.w));
  }
  qsum += __shfl_xor(qsum, 32, 64);

  // Wave and workgroup key-position ranges.
  int wlo = lo, whi = row_ok ? t + 1 : -1, tmin = row_ok ? t : 0x7fffffff, lomax = row_ok ? lo : -1;
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) {
    wlo = min(wlo, __shfl_xor(wlo, o, 64));
    whi = max(whi, __shfl_xor(whi, o, 64));
    tmin = min(tmin, __shfl_xor(tmin, o, 64));
    lomax = max(lomax, __shfl_xor(lomax, o, 64));
  }
  if (lane == 0) {
    sm.wrange[wave][0] = wlo;
    sm.wrange[wave][1] = whi;
    sm.wrange[wave][2] = tmin;
    sm.wrange[wave][3] = lomax;
  }
  __syncthreads();
  int blo = 0x7fffffff, bhi = -1;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    blo = min(blo, sm.wrange[w][0]);
    bhi = max(bhi, sm.wrange[w][1]);
  }
  const bool wave_live = whi > 0;

  const int32_t* pa = tr_prefix_row(c, layer, s, blo);
  const int32_t* pe = tr_prefix_row(c, layer, s, bhi);
  int A[4], voff[5];
  voff[0] = 0;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    A[x] = pa[x];
    voff[x + 1] = voff[x] + (pe[x] - pa[x]);
  }
  const int total = voff[4];

  f32x16 o[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[mt][r] = 0.0f;
  float mref = -INFINITY, lsum = 0.0f;

  const int kk = tid / 8, sub = tid % 8;
  for (int tb = 0; tb < total; tb += BN) {
    __syncthreads();
    // ---- stage one 32-key tile ----
    {
      const int vi = tb + kk;
      if (vi < total) {
        int cls = 0;
        while (cls < 3 && vi >= voff[cls + 1]) ++cls;
        const int slot = A[cls] + (vi - voff[cls]);
        const int P = c.ptok[cls];
        const int page = tr_ptab(c, layer, s, cls)[slot / P];
        const int j = slot % P;
        const uint8_t* pb = c.pool + (int64_t)page * c.page_bytes;
        const int b = 2 << cls;
        const int rowb = D * b / 8;
        const int64_t hoff = (int64_t)h * c.cb + (int64_t)j * rowb + sub * (DPT * b / 8);
        uint32_t wk[8], wv[8];
        load_slice<DPT>(pb + c.k_off[cls] + hoff, b, wk);
        load_slice<DPT>(pb + c.v_off[cls] + hoff, b, wv);
        if (cls == 3) {
#pragma unroll
          for (int e = 0; e < DPT / 2; ++e) {
            sm.ks[kk][sub * DPT + 2 * e] = (uint16_t)(wk[e] & 0xffffu);
            sm.ks[kk][sub * DPT + 2 * e + 1] = (uint16_t)(wk[e] >> 16);
            sm.vt[sub * DPT + 2 * e][kk] = (_Float16)tr_bf16_lo(wv[e]);
            sm.vt[sub * DPT + 2 * e + 1][kk] = (_Float16)tr_bf16_hi(wv[e]);
          }
          if (sub == 0) {
            sm.alpha[kk] = kscale;
            sm.beta[kk] = 0.0f;
          }
        } else {
          const float2 szv = reinterpret_cast<const float2*>(pb + c.sv_off[cls])[(int64_t)h * P + j];
#pragma unroll
          for (int e = 0; e < DPT; ++e) {
            const float ck = code_f<DPT>(wk, b, e);
            sm.ks[kk][sub * DPT + e] = (uint16_t)(__float_as_uint(ck) >> 16);
            sm.vt[sub * DPT + e][kk] = (_Float16)fmaf(szv.x, code_f<DPT>(wv, b, e), szv.y);
          }
          if (sub == 0) {
            const float2 szk = reinterpret_cast<const float2*>(pb + c.sk_off[cls])[(int64_t)h * P + j];
            sm.alpha[kk] = szk.x * kscale;
            sm.beta[kk] = szk.y * kscale;
          }
        }
        if (sub == 0) sm.kpos[kk] = reinterpret_cast<const int32_t*>(pb)[j];
      } else {
#pragma unroll
        for (int e = 0; e < DPT; ++e) {
          sm.ks[kk][sub * DPT + e] = 0;
          sm.vt[sub * DPT + e][kk] = (_Float16)0.0f;
        }
        if (sub == 0) {
          sm.alpha[kk] = 0.0f;
          sm.beta[kk] = 0.0f;
          sm.kpos[kk] = 0x7fffffff;
        }
      }
    }
    __syncthreads();
    if (!wave_live) continue;
    // ---- does this tile touch the wave's windows? ----
    const int mypos = sm.kpos[n];
    int kmin = mypos, kmax_raw = mypos, kmax_real = (mypos == 0x7fffffff) ? -1 : mypos;
#pragma unroll
    for (int o2 = 16; o2 > 0; o2 >>= 1) {
      kmin = min(kmin, __shfl_xor(kmin, o2, 64));
      kmax_raw = max(kmax_raw, __shfl_xor(kmax_raw, o2, 64));
      kmax_real = max(kmax_real, __shfl_xor(kmax_real, o2, 64));
    }
    if (kmin >= whi || kmax_real < wlo) continue;
    const bool needmask = !(kmax_raw <= tmin && kmin >= lomax);

    // ---- S^T = K Q^T ----
    f32x16 sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.ks[n][16 * ks + 8 * g]);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[ks], sacc, 0, 0, 0);
    }
    // ---- scores, mask, running max ----
    float sv[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * g + (r & 3);
      float x = fmaf(sm.alpha[key], sacc[r], sm.beta[key] * qsum);
      if (needmask) {
        const int kp = sm.kpos[key];
        if (!(kp <= t && kp >= lo)) x = -INFINITY;
      }
      sv[r] = x;
      tmax = fmaxf(tmax, x);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    if (__any(tmax > mref + kRescale)) {
      const float mnew = fmaxf(mref, tmax);
      const float corr = (mref == -INFINITY) ? 0.0f : exp2f(mref - mnew);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[mt][r] *= corr;
      lsum *= corr;
      mref = mnew;
    }
    f16x8 pk[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = (sv[r] == -INFINITY) ? 0.0f : exp2f(sv[r] - mref);
      lsum += p;
      pk[r >> 3][r & 7] = (_Float16)p;
    }
    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const _Float16* vrow = &sm.vt[32 * mt + n][16 * kh + 4 * g];
        f16x8 a;
        const uint2 lo4 = *reinterpret_cast<const uint2*>(vrow);
        const uint2 hi4 = *reinterpret_cast<const uint2*>(vrow + 8);
        a = __builtin_bit_cast(f16x8, make_uint4(lo4.x, lo4.y, hi4.x, hi4.y));
        o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pk[kh], o[mt], 0, 0, 0);
      }
    }
  }
  if (!row_ok) return;
  const float ltot = lsum + __shfl_xor(lsum, 32, 64);
  const float inv = 1.0f / ltot;
  uint16_t* orow = out + (((int64_t)s * T + i) * c.H + h) * D;
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

}  // namespace

tr_status tr_prefill_launch(tr_kv_cache* c, int layer, int p0, const uint16_t* q, const uint8_t* mode, int T,
                            int window, uint16_t* out, hipStream_t stream) {
  const CacheLayout& L = c->lay;
  const int BH = L.B * L.H;
  const float kscale = (float)(1.4426950408889634 / sqrt((double)L.D));
  const int ranks = (T + BM - 1) / BM + 1;
  {
    TrProfScope prof(c, TR_PROF_PREFILL_COMPACT, stream);
    if (L.D == 64)
      hipLaunchKernelGGL(k_prefill_compact<64>, dim3(BH), dim3(kBlock), 0, stream, L, T, mode, c->rows,
                         c->row_counts, out);
    else
      hipLaunchKernelGGL(k_prefill_compact<128>, dim3(BH), dim3(kBlock), 0, stream, L, T, mode, c->rows,
                         c->row_counts, out);
    TR_LAUNCH_CHECK();
  }
  TrProfScope prof(c, TR_PROF_PREFILL_ATTN, stream);
  if (L.D == 64)
    hipLaunchKernelGGL(k_prefill_attn<64>, dim3(BH * ranks), dim3(kBlock), 0, stream, L, layer, p0, T, window,
                       kscale, q, c->rows, c->row_counts, out);
  else
    hipLaunchKernelGGL(k_prefill_attn<128>, dim3(BH * ranks), dim3(kBlock), 0, stream, L, layer, p0, T, window,
                       kscale, q, c->rows, c->row_counts, out);
  TR_LAUNCH_CHECK();
  return TR_OK;
}
