// Cache allocation, the Eq. (4) write path and diagnostics.
//
// Write path of one tr_kv_quantize_write call (TriRoute review page, xllm-io.github.io,
// Eq. (4) and the inference paragraph after Algorithm 1):
//   n <= 64 (decode steps): k_write_small, one workgroup per sequence -- slot assignment, page
//                    allocation and quantization in one launch.
//   n > 64:          k_assign_slots (one workgroup per sequence: prefix counts, the slot of
//                    each token in its class stream, and pages from the shared pool), then the
//                    64-position tile kernel of the prefill path without its dense staging
//                    (prefill.cpp.hip): 16 channels per lane, reciprocal fast path with an
//                    exact fallback, packed stores into the class pages.
// The Eq. (4) arithmetic is shared by both through kv_write.h.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "common.h"
#include "kv_write.h"

namespace {

constexpr int kBlock = 256;
constexpr int kAssignBlock = TR_ASSIGN_THREADS;

__global__ void k_fill_i32(int32_t* __restrict__ p, int64_t n, int32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// prefix[layer][seq][0][*] = 0 for every (layer, seq); allocator and flags reset.
__global__ void k_reset(CacheLayout c) {
  int64_t n = (int64_t)c.L * c.B;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    int32_t* row = c.prefix + i * (int64_t)(c.N + 1) * TR_NCLASS;
    row[0] = row[1] = row[2] = row[3] = 0;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *c.next_page = 0;
    *c.err = 0;
  }
}

__global__ __launch_bounds__(kAssignBlock) void k_assign_slots(CacheLayout c, int layer, int p0, int n,
                                                               const uint8_t* __restrict__ bits) {
  tr_assign_slots_seq(c, layer, p0, n, bits, blockIdx.x);
}

// Small appends (n <= 64 tokens per sequence, e.g. one decode step): slot assignment, page
// allocation and quantization of one sequence in one workgroup -- a single launch.  The inputs of
// the first two passes are loaded before anything else; wave 0 then assigns the slots and pages
// (keeping every new position's slot and the class pages it touches in LDS), and after one
// barrier the groups are quantized and stored without another global lookup.
template <int D>
__global__ __launch_bounds__(kBlock) void k_write_small(CacheLayout c, int layer, int p0, int n,
                                                        const uint16_t* __restrict__ kin,
                                                        const uint16_t* __restrict__ vin,
                                                        const uint8_t* __restrict__ bits) {
  constexpr int LPG = D / 8;
  constexpr int GPI = kBlock / LPG;                // groups per pass
  constexpr int NPF = 2;                           // passes loaded up front
  constexpr int kPg = 32;                          // pages per class one call can touch: n <= 64, >= 4 tokens a page
  __shared__ int32_t tslot[64], tcls[64];
  __shared__ int32_t pgs[TR_NCLASS][kPg];
  __shared__ int32_t fps[TR_NCLASS];
  const int s = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, part = tid % LPG;
  const int ngroups = n * c.H * 2;
  auto src_of = [&](int gid) {
    const int g = gid < ngroups ? gid : 0;
    const int kv = g & 1, th = g >> 1;
    const int h = th % c.H, i = th / c.H;
    return (kv ? vin : kin) + (((int64_t)s * n + i) * c.H + h) * D + part * 8;
  };
  uint4 raw[NPF];
#pragma unroll
  for (int x = 0; x < NPF; ++x) raw[x] = *reinterpret_cast<const uint4*>(src_of(x * GPI + tid / LPG));

  if (tid < 64) {
    // the widths and the prefix row go out together (the width load unconditional, clamped: a
    // load under a condition would be waited for on the spot, before the prefix row is issued)
    const int bw = bits[(int64_t)s * n + min(lane, n - 1)];
    const int4 pre0 = *reinterpret_cast<const int4*>(tr_prefix_row(c, layer, s, p0));
    asm volatile("" ::"v"(bw), "v"(pre0.x), "v"(pre0.y), "v"(pre0.z), "v"(pre0.w));
    int cls = 3;
    if (lane < n) {
      cls = tr_class_of_bits(bw);
      if (cls < 0) {
        atomicOr(c.err, TR_ERRF_BAD_BITS);
        cls = 3;
      }
    }
    uint32_t a = 0, b = 0;
    if (lane < n) {
      if (cls == 0) a = 1u; else if (cls == 1) a = 1u << 16; else if (cls == 2) b = 1u; else b = 1u << 16;
    }
    const uint32_t ia = tr_wave_incl_scan(a), ib = tr_wave_incl_scan(b);
    const int n0[4] = {pre0.x, pre0.y, pre0.z, pre0.w};
    const int inc[4] = {(int)(ia & 0xffffu), (int)(ia >> 16), (int)(ib & 0xffffu), (int)(ib >> 16)};
    if (lane < n) {
      *reinterpret_cast<int4*>(const_cast<int32_t*>(tr_prefix_row(c, layer, s, p0 + lane + 1))) =
          make_int4(n0[0] + inc[0], n0[1] + inc[1], n0[2] + inc[2], n0[3] + inc[3]);
      const int own = cls == 0 ? inc[0] : cls == 1 ? inc[1] : cls == 2 ? inc[2] : inc[3];
      const int nb = cls == 0 ? n0[0] : cls == 1 ? n0[1] : cls == 2 ? n0[2] : n0[3];
      tslot[lane] = nb + own - 1;                  // slots before it in its class, plus its own
      tcls[lane] = cls;
    }
    const uint32_t ta = __shfl(ia, 63, 64), tb = __shfl(ib, 63, 64);
    // Pages: lanes 16k .. 16k + 15 take class k, entries fp + (lane & 15) and fp + 16 + (lane & 15)
    // of its page table, fp = the page of its first new slot.  Entries from the first page no slot
    // used before are reused while set (pages kept from before a truncation); the rest are new.
    const int k = lane >> 4, jl = lane & 15;
    const int tot = k == 0 ? (int)(ta & 0xffffu) : k == 1 ? (int)(ta >> 16) : k == 2 ? (int)(tb & 0xffffu) : (int)(tb >> 16);
    const int n0k = k == 0 ? n0[0] : k == 1 ? n0[1] : k == 2 ? n0[2] : n0[3];
    const int P = c.ptok[0] >> k;                  // tokens per page halve with each doubling of b
    const int fp = n0k / P, first = (n0k + P - 1) / P, last = (n0k + tot + P - 1) / P;
    int32_t* pt = c.ptab + ((int64_t)layer * c.B + s) * c.pt_stride + tr_sel4(k, c.pt_off);
    const int e0 = fp + jl, e1 = fp + 16 + jl;
    int v0 = e0 < last ? pt[e0] : -1;
    int v1 = e1 < last ? pt[e1] : -1;
    const uint32_t sh16 = 16 * k;
    const uint32_t m0 = (uint32_t)(__ballot(e0 >= first && e0 < last && v0 < 0) >> sh16) & 0xffffu;
    const uint32_t m1 = (uint32_t)(__ballot(e1 >= first && e1 < last && v1 < 0) >> sh16) & 0xffffu;
    const int reuse = m0 ? fp + __ffs(m0) - 1 : m1 ? fp + 16 + __ffs(m1) - 1 : max(first, last);
    const int need = last - reuse;
    int id0 = 0;
    if (jl == 0 && need > 0) id0 = atomicAdd(c.next_page, need);
    id0 = __shfl(id0, 16 * k, 64);
    const bool ok = (int64_t)id0 + need <= c.pool_pages;
    if (jl == 0 && need > 0 && !ok) atomicOr(c.err, TR_ERRF_NO_PAGES);
    if (e0 >= reuse && e0 < last) {
      v0 = ok ? id0 + (e0 - reuse) : -1;
      pt[e0] = v0;
    }
    if (e1 >= reuse && e1 < last) {
      v1 = ok ? id0 + (e1 - reuse) : -1;
      pt[e1] = v1;
    }
    pgs[k][jl] = v0;
    pgs[k][jl + 16] = v1;
    if (jl == 0) fps[k] = fp;
  }
  __syncthreads();
  auto do_pass = [&](int x, uint4 w4) {
    const int gid = x * GPI + tid / LPG;
    const bool live = gid < ngroups;
    const int g = live ? gid : 0;
    const int kv = g & 1, th = g >> 1;
    const int h = th % c.H, i = th / c.H;
    const int cls = tcls[i];
    const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
    QVec<8> q;
    eq4_quant<D, 8>(q, w, cls);
    if (!live) return;
    const int slot = tslot[i];
    const int page = pgs[cls][(slot >> tr_sel4(cls, c.ptok_log2)) - fps[cls]];
    if (page < 0) return;                          // pool exhausted (flagged)
    const int j = slot & (tr_sel4(cls, c.ptok) - 1);
    uint8_t* base = c.pool + (int64_t)page * c.page_bytes;
    if (h == 0 && kv == 0 && part == 0) reinterpret_cast<int32_t*>(base)[j] = p0 + i;
    put_piece<8>(c, base, j, h, kv, part, cls, q);
  };
#pragma unroll
  for (int x = 0; x < NPF; ++x)
    if (x * GPI < ngroups) do_pass(x, raw[x]);
  for (int x = NPF; x * GPI < ngroups; ++x) do_pass(x, *reinterpret_cast<const uint4*>(src_of(x * GPI + tid / LPG)));
}

// Read back positions tok0 .. tok0+n-1 of every sequence (position order).
template <int D>
__global__ __launch_bounds__(kBlock) void k_export(CacheLayout c, int layer, int tok0, int n,
                                                   uint16_t* __restrict__ codes, float* __restrict__ scale,
                                                   float* __restrict__ zero, uint8_t* __restrict__ bits) {
  const int64_t total = (int64_t)c.B * n * 2 * c.H * D;
  for (int64_t e = blockIdx.x * (int64_t)kBlock + threadIdx.x; e < total; e += (int64_t)gridDim.x * kBlock) {
    const int d = (int)(e % D);
    int64_t r = e / D;
    const int h = (int)(r % c.H); r /= c.H;
    const int kv = (int)(r % 2); r /= 2;
    const int i = (int)(r % n);
    const int s = (int)(r / n);
    const int p = tok0 + i;
    const int32_t* pa = tr_prefix_row(c, layer, s, p);
    const int32_t* pb = tr_prefix_row(c, layer, s, p + 1);
    int cls = 3;
#pragma unroll
    for (int k = 0; k < TR_NCLASS; ++k)
      if (pb[k] != pa[k]) cls = k;
    const int32_t slot = pa[cls];
    const int P = c.ptok[cls];
    const int32_t page = tr_ptab(c, layer, s, cls)[slot / P];
    const int j = slot % P;
    uint16_t val = 0;
    float sv = 1.0f, zv = 0.0f;
    if (page >= 0) {
      const uint8_t* base = c.pool + (int64_t)page * c.page_bytes;
      const uint8_t* row = base + (kv ? c.v_off[cls] : c.k_off[cls]) + (int64_t)h * c.cb + (int64_t)j * c.rowb[cls];
      const int b = 2 << cls;
      if (cls == 3) {
        val = reinterpret_cast<const uint16_t*>(row)[d];
      } else {
        const int bit = d * b;
        val = (uint16_t)((row[bit >> 3] >> (bit & 7)) & ((1u << b) - 1u));
        const float2 sz = reinterpret_cast<const float2*>(base + (kv ? c.sv_off[cls] : c.sk_off[cls]))[(int64_t)h * P + j];
        sv = sz.x;
        zv = sz.y;
      }
    }
    codes[e] = val;
    if (d == 0) {
      const int64_t si = (((int64_t)s * n + i) * 2 + kv) * c.H + h;
      scale[si] = sv;
      zero[si] = zv;
      if (kv == 0 && h == 0) bits[(int64_t)s * n + i] = (uint8_t)(2 << cls);
    }
  }
}

int grid_for(int64_t items, int per_block) {
  int64_t g = (items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > (1 << 20)) g = 1 << 20;
  return (int)g;
}

int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

}  // namespace

tr_status tr_write_launch(tr_kv_cache* c, int layer, int p0, const uint16_t* k, const uint16_t* v,
                          const uint8_t* bits, int n, hipStream_t stream) {
  const CacheLayout& L = c->lay;
  TrProfScope prof(c, TR_PROF_WRITE, stream);
  if (n <= 64) {
    if (L.D == 64)
      hipLaunchKernelGGL(k_write_small<64>, dim3(L.B), dim3(kBlock), 0, stream, L, layer, p0, n, k, v, bits);
    else
      hipLaunchKernelGGL(k_write_small<128>, dim3(L.B), dim3(kBlock), 0, stream, L, layer, p0, n, k, v, bits);
    TR_LAUNCH_CHECK();
    return TR_OK;
  }
  hipLaunchKernelGGL(k_assign_slots, dim3(L.B), dim3(kAssignBlock), 0, stream, L, layer, p0, n, bits);
  TR_LAUNCH_CHECK();
  return tr_write_tiles_launch(c, layer, p0, k, v, bits, n, stream);
}

extern "C" {

const char* tr_status_str(tr_status s) {
  switch (s) {
    case TR_OK: return "ok";
    case TR_ERR_INVALID_ARG: return "invalid argument";
    case TR_ERR_CAPACITY: return "write exceeds the per-sequence capacity";
    case TR_ERR_OUT_OF_PAGES: return "page pool exhausted";
    case TR_ERR_HIP: return "HIP runtime error";
    case TR_ERR_UNSUPPORTED: return "unsupported shape";
    case TR_ERR_BAD_VALUE: return "a bits or mode element outside its domain";
    case TR_ERR_RANGE: return "a value outside the fp16 range of the prefill attention's V operand";
    case TR_ERR_SCRATCH: return "the call needs more scratch than the no-allocation entry point's fixed array";
  }
  return "unknown status";
}

static void free_all(tr_kv_cache* c) {
  if (!c) return;
  for (auto& r : c->prof) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  for (auto e : c->ev_free) (void)hipEventDestroy(e);
  (void)hipFree(c->lay.pool);
  (void)hipFree(c->lay.ptab);
  (void)hipFree(c->lay.prefix);
  (void)hipFree(c->lay.next_page);
  (void)hipFree(c->lay.err);
  (void)hipFree(c->partials);
  (void)hipFree(c->merge_cnt);
  (void)hipFree(c->rows);
  (void)hipFree(c->row_counts);
  (void)hipFree(c->dk);
  (void)hipFree(c->dv);
  (void)hipFree(c->dkf);
  (void)hipFree(c->pf_units);
  (void)hipFree(c->pf_merges);
  (void)hipFree(c->pf_part);
  delete c;
}

tr_status tr_kv_cache_alloc(const tr_kv_cache_desc* d, tr_kv_cache** out) {
  if (!d || !out) return TR_ERR_INVALID_ARG;
  *out = nullptr;
  if (d->num_layers < 1 || d->batch < 1 || d->num_heads < 1 || d->max_tokens < 1 || d->pool_pages < 0)
    return TR_ERR_INVALID_ARG;
  if (d->head_dim != 64 && d->head_dim != 128) return TR_ERR_UNSUPPORTED;
  // one (seq, head)'s dense prefill staging must stay addressable by a 32-bit buffer offset
  if ((int64_t)d->max_tokens * d->head_dim > (1LL << 30) - 64LL * d->head_dim) return TR_ERR_UNSUPPORTED;
  const int hq = d->num_query_heads ? d->num_query_heads : d->num_heads;
  if (hq < d->num_heads || hq % d->num_heads) return TR_ERR_INVALID_ARG;
  if (d->prefill_tokens < -1 || d->prefill_tokens > d->max_tokens) return TR_ERR_INVALID_ARG;
  const int cb = d->page_code_bytes ? d->page_code_bytes : 4096;
  if (cb < 1024 || cb > 65536 || (cb & (cb - 1))) return TR_ERR_INVALID_ARG;

  tr_kv_cache* c = new tr_kv_cache();
  memset(&c->lay, 0, sizeof(c->lay));
  c->partials = nullptr;
  c->merge_cnt = nullptr;
  c->rows = c->row_counts = nullptr;
  c->dk = c->dv = nullptr;
  c->dkf = nullptr;
  c->pf_units = c->pf_merges = nullptr;
  c->pf_part = nullptr;
  c->prof_on = false;
  CacheLayout& L = c->lay;
  L.L = d->num_layers; L.B = d->batch; L.H = d->num_heads; L.D = d->head_dim; L.N = d->max_tokens;
  L.pfN = d->prefill_tokens == 0 ? L.N : d->prefill_tokens < 0 ? 0 : d->prefill_tokens;
  c->hq = hq;
  c->grp = hq / L.H;
  L.cb = cb;
  int64_t page_bytes = 0;
  L.pt_stride = 0;
  for (int k = 0; k < TR_NCLASS; ++k) {
    const int b = 2 << k;
    L.rowb[k] = L.D * b / 8;
    L.ptok[k] = cb / L.rowb[k];
    L.ptok_log2[k] = 0;
    while ((1 << L.ptok_log2[k]) < L.ptok[k]) ++L.ptok_log2[k];
    int64_t off = align256(4LL * L.ptok[k]);
    L.k_off[k] = (int32_t)off; off += (int64_t)L.H * cb;
    L.v_off[k] = (int32_t)off; off += (int64_t)L.H * cb;
    if (k < 3) {
      L.sk_off[k] = (int32_t)off; off += align256((int64_t)L.H * L.ptok[k] * 8);
      L.sv_off[k] = (int32_t)off; off += align256((int64_t)L.H * L.ptok[k] * 8);
    } else {
      L.sk_off[k] = L.sv_off[k] = 0;
    }
    if (off > page_bytes) page_bytes = off;
    L.maxp[k] = (L.N + L.ptok[k] - 1) / L.ptok[k] + 1;
    L.pt_off[k] = L.pt_stride;
    L.pt_stride += L.maxp[k];
  }
  if (page_bytes > (1LL << 30)) { delete c; return TR_ERR_UNSUPPORTED; }
  L.page_bytes = (int32_t)page_bytes;
  // Worst case over any mix of widths: every token in the class with the fewest tokens per
  // page, plus one partial page for each other class.
  const int64_t worst = (int64_t)L.L * L.B * ((L.N + L.ptok[3] - 1) / L.ptok[3] + TR_NCLASS);
  L.pool_pages = d->pool_pages ? d->pool_pages : worst;
  if (L.pool_pages > 0x7fffffffLL) { delete c; return TR_ERR_UNSUPPORTED; }

  c->len.assign(L.L, 0);
  {
    const int min_chunk = tr_decode_max_chunk(L) < TR_DECODE_MIN_CHUNK ? tr_decode_max_chunk(L) : TR_DECODE_MIN_CHUNK;
    c->max_chunks = (L.N + min_chunk - 1) / min_chunk + 1;
    if (c->max_chunks < TR_DECODE_FORCE_MAX) c->max_chunks = TR_DECODE_FORCE_MAX;
  }
  c->force_chunks = 0;
  (void)hipGetDevice(&c->device);
  bool ok = true;
  ok = ok && hipMalloc((void**)&L.pool, (size_t)(L.pool_pages * L.page_bytes)) == hipSuccess;
  ok = ok && hipMalloc((void**)&L.ptab, sizeof(int32_t) * (size_t)L.L * L.B * L.pt_stride) == hipSuccess;
  ok = ok && hipMalloc((void**)&L.prefix, sizeof(int32_t) * TR_NCLASS * (size_t)L.L * L.B * (L.N + 1)) == hipSuccess;
  ok = ok && hipMalloc((void**)&L.next_page, sizeof(int32_t)) == hipSuccess;
  ok = ok && hipMalloc((void**)&L.err, sizeof(uint32_t)) == hipSuccess;
  ok = ok && hipMalloc((void**)&c->partials,
                       sizeof(float) * (size_t)L.B * hq * c->max_chunks * (L.D + 2)) == hipSuccess;
  ok = ok && hipMalloc((void**)&c->merge_cnt, sizeof(int32_t) * (size_t)L.B * hq) == hipSuccess;
  ok = ok && hipMemset(c->merge_cnt, 0, sizeof(int32_t) * (size_t)L.B * hq) == hipSuccess;
  c->np = (L.pfN + 63) / 64 * 64;
  c->pf_uph = L.pfN ? tr_prefill_units_per_head(L.pfN) : 0;
  if (L.pfN > 0) {                                 // prefill scratch, sized by its capacity
    ok = ok && hipMalloc((void**)&c->rows, sizeof(int32_t) * (size_t)L.B * hq * L.pfN) == hipSuccess;
    ok = ok && hipMalloc((void**)&c->row_counts, sizeof(int32_t) * (size_t)L.B * hq * 4) == hipSuccess;
    ok = ok && hipMalloc((void**)&c->dk, sizeof(uint16_t) * (size_t)L.B * L.H * c->np * L.D) == hipSuccess;
    ok = ok && hipMalloc((void**)&c->dv, sizeof(uint16_t) * (size_t)L.B * L.H * c->np * L.D) == hipSuccess;
    ok = ok && hipMalloc((void**)&c->dkf, sizeof(float2) * (size_t)L.B * L.H * c->np) == hipSuccess;
    ok = ok && hipMalloc((void**)&c->pf_units, sizeof(int4) * (size_t)L.B * hq * c->pf_uph) == hipSuccess;
    ok = ok && hipMalloc((void**)&c->pf_merges, sizeof(int4) * (size_t)L.B * hq * (TR_PREFILL_SLOTS / 2)) == hipSuccess;
    ok = ok && hipMalloc((void**)&c->pf_part,
                         sizeof(float) * (size_t)L.B * hq * TR_PREFILL_SLOTS * 128 * (L.D + 4)) == hipSuccess;
  }
  if (!ok) {
    hipGetLastError();
    free_all(c);
    return TR_ERR_HIP;
  }
  const int64_t npt = (int64_t)L.L * L.B * L.pt_stride;
  hipLaunchKernelGGL(k_fill_i32, dim3(grid_for(npt, kBlock)), dim3(kBlock), 0, 0, L.ptab, npt, -1);
  hipLaunchKernelGGL(k_reset, dim3(grid_for((int64_t)L.L * L.B, kBlock)), dim3(kBlock), 0, 0, L);
  if (hipGetLastError() != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    free_all(c);
    return TR_ERR_HIP;
  }
  *out = c;
  return TR_OK;
}

tr_status tr_kv_cache_free(tr_kv_cache* c) {
  if (!c) return TR_OK;
  hipDeviceSynchronize();
  free_all(c);
  return TR_OK;
}

tr_status tr_kv_cache_reset(tr_kv_cache* c, void* stream) {
  if (!c) return TR_ERR_INVALID_ARG;
  CacheLayout& L = c->lay;
  hipStream_t st = (hipStream_t)stream;
  const int64_t npt = (int64_t)L.L * L.B * L.pt_stride;
  hipLaunchKernelGGL(k_fill_i32, dim3(grid_for(npt, kBlock)), dim3(kBlock), 0, st, L.ptab, npt, -1);
  hipLaunchKernelGGL(k_reset, dim3(grid_for((int64_t)L.L * L.B, kBlock)), dim3(kBlock), 0, st, L);
  TR_LAUNCH_CHECK();
  for (auto& x : c->len) x = 0;
  return TR_OK;
}

tr_status tr_kv_cache_truncate(tr_kv_cache* c, int32_t layer, int32_t new_len) {
  if (!c || layer < 0 || layer >= c->lay.L || new_len < 0 || new_len > c->len[layer]) return TR_ERR_INVALID_ARG;
  c->len[layer] = new_len;
  return TR_OK;
}

int32_t tr_kv_cache_length(const tr_kv_cache* c, int32_t layer) {
  if (!c || layer < 0 || layer >= c->lay.L) return -1;
  return c->len[layer];
}

tr_status tr_kv_quantize_write(tr_kv_cache* c, int32_t layer, const void* k, const void* v,
                               const uint8_t* bits, int32_t n_new, void* stream) {
  if (!c || layer < 0 || layer >= c->lay.L || n_new < 0) return TR_ERR_INVALID_ARG;
  if (n_new == 0) return TR_OK;
  if (!k || !v || !bits) return TR_ERR_INVALID_ARG;
  if ((int64_t)c->len[layer] + n_new > c->lay.N) return TR_ERR_CAPACITY;
  tr_status st = tr_write_launch(c, layer, c->len[layer], (const uint16_t*)k, (const uint16_t*)v, bits, n_new,
                                 (hipStream_t)stream);
  if (st == TR_OK) c->len[layer] += n_new;
  return st;
}

tr_status tr_routed_attn_decode(tr_kv_cache* c, int32_t layer, const void* q, const uint8_t* mode,
                                int32_t window, void* out, void* stream) {
  if (!c || layer < 0 || layer >= c->lay.L || !q || !mode || !out || window < 0) return TR_ERR_INVALID_ARG;
  if (c->len[layer] < 1) return TR_ERR_INVALID_ARG;
  return tr_decode_launch(c, layer, (const uint16_t*)q, mode, window, (uint16_t*)out, (hipStream_t)stream);
}

tr_status tr_routed_attn_decode_noalloc(tr_kv_cache* c, int32_t layer, const void* q, const uint8_t* mode,
                                        int32_t window, void* out, void* stream) {
  if (!c || layer < 0 || layer >= c->lay.L || !q || !mode || !out || window < 0) return TR_ERR_INVALID_ARG;
  if (c->len[layer] < 1) return TR_ERR_INVALID_ARG;
  return tr_decode_noalloc_launch(c, layer, (const uint16_t*)q, mode, window, (uint16_t*)out, (hipStream_t)stream);
}

tr_status tr_routed_attn_prefill(tr_kv_cache* c, int32_t layer, const void* q, const void* k, const void* v,
                                 const uint8_t* bits, const uint8_t* mode, int32_t T, int32_t window, void* out,
                                 void* stream) {
  if (!c || layer < 0 || layer >= c->lay.L || T < 0 || window < 0) return TR_ERR_INVALID_ARG;
  if (T == 0) return TR_OK;
  if (!q || !k || !v || !bits || !mode || !out) return TR_ERR_INVALID_ARG;
  if ((int64_t)c->len[layer] + T > c->lay.N) return TR_ERR_CAPACITY;
  const int p0 = c->len[layer];
  hipStream_t st = (hipStream_t)stream;
  const tr_status s = tr_prefill_launch(c, layer, p0, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                                       bits, mode, T, window, (uint16_t*)out, st);
  if (s == TR_OK) c->len[layer] += T;
  return s;
}

tr_status tr_kv_cache_export(const tr_kv_cache* c, int32_t layer, int32_t tok0, int32_t n, uint16_t* codes,
                             float* scale, float* zero, uint8_t* bits, void* stream) {
  if (!c || layer < 0 || layer >= c->lay.L || tok0 < 0 || n < 0) return TR_ERR_INVALID_ARG;
  if ((int64_t)tok0 + n > c->len[layer]) return TR_ERR_INVALID_ARG;
  if (n == 0) return TR_OK;
  if (!codes || !scale || !zero || !bits) return TR_ERR_INVALID_ARG;
  const CacheLayout& L = c->lay;
  const int64_t total = (int64_t)L.B * n * 2 * L.H * L.D;
  const int grid = grid_for(total, kBlock);
  if (L.D == 64)
    hipLaunchKernelGGL(k_export<64>, dim3(grid), dim3(kBlock), 0, (hipStream_t)stream, L, layer, tok0, n, codes,
                       scale, zero, bits);
  else
    hipLaunchKernelGGL(k_export<128>, dim3(grid), dim3(kBlock), 0, (hipStream_t)stream, L, layer, tok0, n, codes,
                       scale, zero, bits);
  TR_LAUNCH_CHECK();
  return TR_OK;
}

tr_status tr_kv_cache_status(tr_kv_cache* c, void* stream) {
  if (!c) return TR_ERR_INVALID_ARG;
  uint32_t flags = 0;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return TR_ERR_HIP;
  if (hipMemcpy(&flags, c->lay.err, sizeof(flags), hipMemcpyDeviceToHost) != hipSuccess) return TR_ERR_HIP;
  if (flags & TR_ERRF_NO_PAGES) return TR_ERR_OUT_OF_PAGES;
  if (flags & (TR_ERRF_BAD_BITS | TR_ERRF_BAD_MODE)) return TR_ERR_BAD_VALUE;
  if (flags & TR_ERRF_RANGE) return TR_ERR_RANGE;
  return TR_OK;
}

tr_status tr_kv_cache_set_decode_chunks(tr_kv_cache* c, int32_t n) {
  if (!c || n < 0 || n > c->max_chunks) return TR_ERR_INVALID_ARG;
  c->force_chunks = n;
  return TR_OK;
}

tr_status tr_profile_enable(tr_kv_cache* c, int32_t enable) {
  if (!c) return TR_ERR_INVALID_ARG;
  c->prof_on = enable != 0;
  return TR_OK;
}

tr_status tr_profile_read(tr_kv_cache* c, int64_t* launches, double* total_ms) {
  if (!c || !launches || !total_ms) return TR_ERR_INVALID_ARG;
  for (int f = 0; f < TR_PROF_NFAM; ++f) {
    launches[f] = 0;
    total_ms[f] = 0.0;
  }
  tr_status st = TR_OK;
  for (auto& r : c->prof) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      st = TR_ERR_HIP;
    } else {
      launches[r.fam] += 1;
      total_ms[r.fam] += ms;
    }
    c->ev_free.push_back(r.a);
    c->ev_free.push_back(r.b);
  }
  c->prof.clear();
  return st;
}

int64_t tr_kv_cache_pages_used(tr_kv_cache* c, void* stream) {
  if (!c) return -1;
  int32_t used = 0;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return -1;
  if (hipMemcpy(&used, c->lay.next_page, sizeof(used), hipMemcpyDeviceToHost) != hipSuccess) return -1;
  return used < c->lay.pool_pages ? used : c->lay.pool_pages;
}

}  // extern "C"
