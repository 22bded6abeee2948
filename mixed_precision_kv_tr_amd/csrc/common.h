// Internal declarations shared by the translation units of libtriroute.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "layout.h"
#include "triroute.h"

struct tr_kv_cache {
  CacheLayout lay;                // lay.H = KV heads (what the cache stores)
  int32_t hq;                     // query heads of the attention calls (a multiple of lay.H)
  int32_t grp;                    // hq / lay.H: query heads per KV head (1 = multi-head)
  int device;
  std::vector<int32_t> len;       // host mirror: tokens written per layer (same for every sequence)
  // decode split-K partials: [B][HQ][max_chunks][D + 2] floats (o[D], m, l)
  float* partials;
  int32_t max_chunks;
  // decode merge counters, one per (seq, query head) (at least one per (seq, KV head, block)):
  // zero between calls
  int32_t* merge_cnt;
  int32_t force_chunks;           // tr_kv_cache_set_decode_chunks: 0 = automatic
  // prefill scratch: compacted query rows per (seq, query head) [B][HQ][N] and counts [B][HQ][4]
  int32_t* rows;
  int32_t* row_counts;
  // prefill scratch: the cache range a prefill call reads, staged once per KV head, position order
  //   dk [B][H][NP][D] uint16: K code as a bf16 integer (exact), or the stored bf16 (b = 16)
  //   dkf [B][H][NP] float2:   (alpha, r) = (s_K * log2(e) / sqrt(D), z_K / s_K) per key
  //   dv [B][H][D][NP] uint16: v_hat = s * c + z as fp16, channel-major; within each group of
  //                            16 positions, bits 2 and 3 of the position are swapped
  // prefill attention work, per (seq, query head): units (128-row tile, key-tile chunk)
  // [B][HQ][pf_uph] int4, merges of split tiles [B][HQ][TR_PREFILL_SLOTS / 2] int4, partial
  // results of split tiles [B][HQ][TR_PREFILL_SLOTS][128][D + 4] floats (O, max, sum, padding)
  int4* pf_units;
  int4* pf_merges;
  float* pf_part;
  int32_t pf_uph;
  int32_t np;                     // N rounded up to a multiple of 64 (the write tile)
  uint16_t* dk;
  float2* dkf;
  uint16_t* dv;
  // optional kernel timing (tr_profile_enable): HIP events around each kernel launch
  bool prof_on;
  struct ProfRec { int fam; hipEvent_t a, b; };
  std::vector<ProfRec> prof;
  std::vector<hipEvent_t> ev_free;
};

// Decode work items: at most TR_DECODE_ITEM_MAX positions (LDS score buffer) and at most
// TR_DECODE_PG_MAX page ids per width class (LDS page list); the host never picks chunks below
// TR_DECODE_MIN_CHUNK positions unless those limits force it.
#define TR_DECODE_ITEM_MAX 544
#define TR_DECODE_PG_MAX 36
#ifndef TR_DECODE_MIN_CHUNK
#define TR_DECODE_MIN_CHUNK 128
#endif

// Partial-result slots per (seq, query head) of the decode split-K are at least this many, so a
// forced chunk count (tr_kv_cache_set_decode_chunks) up to it is always available.
#define TR_DECODE_FORCE_MAX 64

// Largest decode chunk (positions) this layout allows.
inline int tr_decode_max_chunk(const CacheLayout& L) {
  const int by_pages = (TR_DECODE_PG_MAX - 2) * L.ptok[3];
  return by_pages < TR_DECODE_ITEM_MAX ? by_pages : TR_DECODE_ITEM_MAX;
}


// Prefill: partial-result slots per (seq, head) for key-split row tiles, and the work units of a
// prefill of T tokens per (seq, head): one per 128-row tile (full and local rows fill separate
// tiles) plus the extra chunks of split tiles.
#ifndef TR_PREFILL_SLOTS
#define TR_PREFILL_SLOTS 16
#endif
inline int tr_prefill_units_per_head(int T) { return (T + 127) / 128 + 1 + TR_PREFILL_SLOTS; }

// Workgroups are dealt to the 8 XCDs round-robin by id; this gives XCD x the contiguous run
// [x * per, (x + 1) * per) of the n work items (grid = 8 * per, per = ceil(n / 8)), so that
// neighbouring items -- which share cache lines -- go through the same L2.  -1 for the padding
// workgroups.
__device__ __forceinline__ int tr_xcd_linear(int n) {
  const int per = (n + 7) >> 3;
  const int lin = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  return lin < n ? lin : -1;
}
inline int tr_xcd_grid(int n) { return ((n + 7) >> 3) << 3; }

// Kernel families reported by tr_profile_read.
enum { TR_PROF_WRITE = 0, TR_PROF_DECODE_SPLIT = 1, TR_PROF_DECODE_COMBINE = 2, TR_PROF_PREFILL_COMPACT = 3,
       TR_PROF_PREFILL_ATTN = 4, TR_PROF_PREFILL_MERGE = 5, TR_PROF_NFAM = 6 };

// Brackets the kernel launches of its scope with events when timing is on.
struct TrProfScope {
  tr_kv_cache* c;
  int fam;
  hipStream_t st;
  hipEvent_t a = nullptr;
  static hipEvent_t take(tr_kv_cache* c) {
    if (!c->ev_free.empty()) {
      hipEvent_t e = c->ev_free.back();
      c->ev_free.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    // No system-scope fence: the events only timestamp the stream, and a fence would add the
    // write-back of the kernel's dirty L2 lines to the measured interval.
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    return e;
  }
  TrProfScope(tr_kv_cache* c_, int fam_, hipStream_t st_) : c(c_), fam(fam_), st(st_) {
    if (c->prof_on && (a = take(c))) (void)hipEventRecord(a, st);
  }
  ~TrProfScope() {
    if (!c->prof_on || !a) return;
    hipEvent_t b = take(c);
    if (!b) return;
    (void)hipEventRecord(b, st);
    c->prof.push_back({fam, a, b});
  }
};

// Every kernel launch goes through here so launch errors map to TR_ERR_HIP.
#define TR_LAUNCH_CHECK()                                     \
  do {                                                        \
    if (hipGetLastError() != hipSuccess) return TR_ERR_HIP;   \
  } while (0)

// bf16 bits -> float (exact) and float -> bf16 bits (round to nearest even, finite input).
__device__ __forceinline__ float tr_bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float tr_bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint16_t tr_f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Inclusive prefix sum over the 64 lanes of a wave (called with all 64 lanes active).
__device__ __forceinline__ uint32_t tr_wave_incl_scan(uint32_t v) {
  // DPP: shifts by 1, 2, 4, 8 inside each row of 16 lanes (lanes before the shift read 0), then
  // each row adds the total of the rows before it through the row_bcast:15 / row_bcast:31 moves.
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);   // rows 1, 3 += rows 0, 2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);   // rows 2, 3 += rows 0-1
  return v;
}

// Decode entry points implemented in decode.hip / prefill.hip.
tr_status tr_decode_launch(tr_kv_cache* c, int layer, const uint16_t* q, const uint8_t* mode, int window,
                           uint16_t* out, hipStream_t stream);
// The same with the split-K partials in the library's file-scope device scratch (no allocation).
tr_status tr_decode_noalloc_launch(tr_kv_cache* c, int layer, const uint16_t* q, const uint8_t* mode, int window,
                                   uint16_t* out, hipStream_t stream);
// The whole prefill call: Eq. (4) write of positions [p0, p0 + T), then routed attention of their
// queries over [0, p0 + T).
tr_status tr_prefill_launch(tr_kv_cache* c, int layer, int p0, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, const uint8_t* bits, const uint8_t* mode, int T, int window,
                            uint16_t* out, hipStream_t stream);
tr_status tr_write_launch(tr_kv_cache* c, int layer, int p0, const uint16_t* k, const uint16_t* v,
                          const uint8_t* bits, int n, hipStream_t stream);
// Quantize-write of positions [p0, p0 + n) whose slots are assigned, 64-position tiles per (seq,
// head) (the prefill write kernel without its dense staging).
tr_status tr_write_tiles_launch(tr_kv_cache* c, int layer, int p0, const uint16_t* k, const uint16_t* v,
                                const uint8_t* bits, int n, hipStream_t stream);
