// Decode routed attention over the mixed-width paged cache on the matrix cores (TriRoute review
// page, xllm-io.github.io: Eq. (2) modes read by a query; Eq. (4) codes written per token).
//
// Work item: one wavefront = one workgroup = (sequence, KV head, block of up to GB query heads of
// that KV head, position chunk).  The block's query heads are the columns of the matrix products:
// query head h reads KV head h / G, so with grouped-query attention (G > 1) the KV rows a block
// reads serve all of its query heads at once; G = 1 is multi-head attention, one column.  The item
// covers a chunk of the union of its columns' windows ([lo, t]: lo = 0 for full, max(0, t - w) for
// local; skip columns read nothing); every chunk maps, through the per-position class prefix
// counts, to one contiguous slot range per width class, so out-of-window keys are never read and
// each inner loop runs over a single width.  A local column of a block that also holds a full
// column sees only the slots at or after its window start (one more prefix row).
//
// phase 1  S^T = Q K^T per 16 keys on v_mfma_f32_16x16x32_f16 (_bf16 for b = 16 keys).  The lane
//          that owns a key's B column loads its slice of the key's code row and expands it in
//          registers to exact fp16 values 1024 + c 2^(kf): code fields are ORed into fp16 1024's
//          mantissa where they sit, and the field's power of two is folded into the query row (A),
//          which is prescaled into fp16 range per column.  Eq. (4)'s reconstruction folds out
//          exactly: q . (s c + z) = s (q . c) + z sum(q).  Scores (log2 domain) go to LDS, with
//          per-column running maxima and the chunk's largest V scale per class.
// phase 2  O^T = V^T P'^T per tile of keys.  The tile's raw V code rows are staged in LDS and read
//          back transposed (ds_read_b64_tr_b4 / _b8 / _b16), so each lane holds one channel of 8 or
//          16 keys, expanded to fp16 like the keys; P' = p s_V 2^-tau (p = 2^(score - max)) enters
//          as an fp16 hi + lo pair (bf16 for b = 16 keys, whose values are bf16), and the zero
//          points add sum(p z_V) per column.  2-bit tiles hold two channels per nibble: they
//          accumulate apart and are added through LDS.
// epilogue a one-chunk window writes bf16 out directly; otherwise the chunk writes (o[D], m, l)
//          per column.  Columns whose mode is skip get zeros from chunk 0.
// merge    with one column per item, the wave that finishes a window's last chunk merges the
//          window's chunk records (log-sum-exp) into bf16; with blocks of query heads,
//          k_decode_combine does it in a launch of its own.
#include <math.h>

#include <mutex>

#include "common.h"

namespace {

constexpr int kWave = 64;
constexpr int kPgMax = TR_DECODE_PG_MAX;
constexpr int kMinChunk = TR_DECODE_MIN_CHUNK;
constexpr int kMergeBatch = 32;                    // chunk records a merge folds per round trip
constexpr uint32_t kF16K = 0x64006400u;            // the fp16 pair (1024, 1024)
constexpr uint32_t kF16B = 0x64646464u;            // byte 0x64 (fp16 1024's high byte) everywhere

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Positions per chunk the LDS score buffer holds, by columns per item.
template <int GB>
constexpr int chunk_cap() { return GB == 1 ? TR_DECODE_ITEM_MAX : 352; }

// A constant hidden from the compiler in an SGPR / a VGPR, so that (x & m) | c is emitted as one
// v_and_or_b32 (VOP3 takes no literal operands; left visible, the compiler splits it in two).
__device__ __forceinline__ uint32_t opaque_s(uint32_t x) {
  __asm__("" : "+s"(x));
  return x;
}
__device__ __forceinline__ uint32_t opaque_v(uint32_t x) {
  __asm__("" : "+v"(x));
  return x;
}

// Address of row `row` (of `rb` bytes) of pool page `pg`, from `base` = the pool plus the offset of
// the row region inside a page: two unsigned 32 x 32 -> 64-bit multiply-adds (v_mad_u64_u32), with
// no sign extension and no zero-extended 64-bit operand.  `rb` goes through an SGPR so that a
// power of two stays a multiply (a 64-bit shift would need the row zero-extended first), and the
// result is a global-memory pointer (a generic one would make the loads flat loads, which also
// count against the LDS wait counter).
typedef const __attribute__((address_space(1))) uint8_t* gbytes_t;
__device__ __forceinline__ gbytes_t page_row(uint64_t base, uint32_t page_bytes, int32_t pg, int row, uint32_t rb) {
  return (gbytes_t)((uint64_t)(uint32_t)row * opaque_s(rb) + ((uint64_t)(uint32_t)pg * page_bytes + base));
}
// Page id of class slot j from the chunk's page list `pg` (whose entry 0 is page `first` of the class):
// the list's LDS byte address minus 4 * first is a wave-uniform base, so the lookup costs a shift
// and one v_lshl_add_u32 per lane.
__device__ __forceinline__ uint32_t pg_base(const int32_t* pg, int first) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) int32_t*)pg - 4u * (uint32_t)first;
}
__device__ __forceinline__ int32_t page_of(uint32_t pgb, int j, int lp) {
  return *(const __attribute__((address_space(3))) int32_t*)(uintptr_t)((((uint32_t)j >> lp) << 2) + pgb);
}
template <typename T>
__device__ __forceinline__ T gload(gbytes_t p) {
  return *(const __attribute__((address_space(1))) T*)p;
}

__device__ __forceinline__ f32x4 mma_f16(const uint32_t* a, const uint32_t* b, f32x4 acc) {
  const u32x4 av = {a[0], a[1], a[2], a[3]}, bv = {b[0], b[1], b[2], b[3]};
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av), __builtin_bit_cast(f16x8, bv), acc, 0,
                                                0, 0);
}
__device__ __forceinline__ f32x4 mma_bf16(const uint32_t* a, const uint32_t* b, f32x4 acc) {
  const u32x4 av = {a[0], a[1], a[2], a[3]}, bv = {b[0], b[1], b[2], b[3]};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), acc,
                                                 0, 0, 0);
}
// K = 16: A / B hold 4 bf16 each (two words).
__device__ __forceinline__ f32x4 mma_bf16_k16(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f32x4 acc) {
  const u32x2 av = {a0, a1}, bv = {b0, b1};
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, av), __builtin_bit_cast(s16x4, bv), acc,
                                                   0, 0, 0);
}

// Transposing LDS reads.  Each lane names 8 bytes; within every group of 16 lanes, lane L receives
//   tr4:  nibble L of the 16 lanes' reads, in lane order (16 values);
//   tr8:  byte L % 8 of the reads of lanes L / 8, L / 8 + 2, ..., L / 8 + 14 (8 values);
//   tr16: element L % 4 of the reads of lanes L / 4, L / 4 + 4, L / 4 + 8, L / 4 + 12 (4 values).
#define TR_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))
__device__ __forceinline__ void tr4(const uint8_t* p, uint32_t& x0, uint32_t& x1) {
  const i32x2 r = __builtin_amdgcn_ds_read_tr4_b64_v2i32(TR_LDS(i32x2, p));
  x0 = (uint32_t)r[0];
  x1 = (uint32_t)r[1];
}
__device__ __forceinline__ void tr8(const uint8_t* p, uint32_t& x0, uint32_t& x1) {
  const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(TR_LDS(i32x2, p));
  x0 = (uint32_t)r[0];
  x1 = (uint32_t)r[1];
}
__device__ __forceinline__ void tr16(const uint8_t* p, uint32_t& x0, uint32_t& x1) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(TR_LDS(s16x4, p));
  const u32x2 w = __builtin_bit_cast(u32x2, r);
  x0 = w[0];
  x1 = w[1];
}

// Orders this wave's LDS accesses around it.  A workgroup here is a single wave, and LDS
// instructions of a wave complete in the order they are issued, so no barrier is needed -- only
// that the compiler moves no memory access across, and that earlier LDS accesses are done.  The
// wave's global loads stay in flight (a barrier's workgroup fence would wait for them as well).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xc07f);              // lgkmcnt(0); vmcnt and expcnt untouched
  __asm__ volatile("" ::: "memory");
}

// Cross-lane sums and maxima without LDS: DPP inside rows of 16 lanes, v_permlane16_swap /
// v_permlane32_swap across rows and halves (each swap hands every lane its partner's value in one
// of its two results, so combining both results gives the pairwise reduction in every lane).
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
// Sum / max over the 16 lanes of each row (result in every lane of the row).
__device__ __forceinline__ float row_sum(float v) {
  v += dpp_f<0xB1>(v);                             // quad_perm 1,0,3,2
  v += dpp_f<0x4E>(v);                             // quad_perm 2,3,0,1
  v += dpp_f<0x141>(v);                            // row_half_mirror
  v += dpp_f<0x140>(v);                            // row_mirror
  return v;
}
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return v;
}
__device__ __forceinline__ float wave_max(float v) { return max32(max16(row_max(v))); }
__device__ __forceinline__ float wave_sum(float v) { return sum32(sum16(row_sum(v))); }

// ---- code expansion to fp16 operands ------------------------------------------------------------
// Every expansion writes pairs (lo, hi) of fp16 values 1024 + (code field in place); the other
// operand of the product carries the field's inverse power of two.

// 16 two-bit codes of a word (element e at bits 2e) as 8 pairs: pair f (f = 0..4) holds elements
// (f, 8 + f) times 4^f, pair 5 + f (f = 0..2) elements (5 + f, 13 + f) times 4^f.
__device__ __forceinline__ void exp_k2(uint32_t w, uint32_t* p, uint32_t K, const uint32_t* m) {
  p[0] = (w & m[0]) | K;
  p[1] = (w & m[1]) | K;
  p[2] = (w & m[2]) | K;
  p[3] = (w & m[3]) | K;
  p[4] = (w & m[4]) | K;
  const uint32_t w10 = w >> 10;
  p[5] = (w10 & m[0]) | K;
  p[6] = (w10 & m[1]) | K;
  p[7] = (w10 & m[2]) | K;
}
// 8 four-bit codes of a word (element e at bits 4e) as 4 pairs: (0, 4), (1, 5) x 16, (2, 6),
// (3, 7) x 16.  The same expansion serves V: a tr4 word holds one channel of 8 keys.
__device__ __forceinline__ void exp_k4(uint32_t w, uint32_t* p, uint32_t K, uint32_t m0, uint32_t m1) {
  p[0] = (w & m0) | K;
  p[1] = (w & m1) | K;
  const uint32_t w8 = w >> 8;
  p[2] = (w8 & m0) | K;
  p[3] = (w8 & m1) | K;
}
// 4 byte codes of a word as 2 pairs (0, 1), (2, 3): the bytes with 0x64 above them.
__device__ __forceinline__ void exp_k8(uint32_t w, uint32_t* p, uint32_t B) {
  p[0] = __builtin_amdgcn_perm(B, w, 0x04010400u);
  p[1] = __builtin_amdgcn_perm(B, w, 0x04030402u);
}
// A tr4 word of a 2-bit tile: nibble k = key k, the even channel's code in bits 0-1 and the odd
// channel's in bits 2-3 (the caller shifts the word right by 2 for the odd channel).  Pairs
// (k, k + 4): keys 0, 1, 2 in place (times 1, 16, 256), key 3 after a shift.
__device__ __forceinline__ void exp_v2(uint32_t x, uint32_t* p, uint32_t K, uint32_t m0, uint32_t m1, uint32_t m2) {
  p[0] = (x & m0) | K;
  p[1] = (x & m1) | K;
  p[2] = (x & m2) | K;
  p[3] = ((x >> 12) & m0) | K;
}

// 8 two-bit fields (element e at bits 2e of the low 16 bits, or of the high 16 bits for hi) into
// 8 four-bit slots (element e at bits 4e): a 2-bit code row restaged with the 4-bit row layout.
__device__ __forceinline__ uint32_t spread2(uint32_t w, bool hi) {
  uint32_t x = __builtin_amdgcn_perm(0u, w, hi ? 0x0c030c02u : 0x0c010c00u);   // bytes b, 0, b', 0
  x = (x | (x << 4)) & 0x0f0f0f0fu;
  x = (x | (x << 2)) & 0x33333333u;
  return x;
}

// Factor on the P' operand of key k (0..7) of a tr4 word, undoing the expansion's field scale.
template <int C>
__device__ __forceinline__ float pfield(int k) {
  if constexpr (C == 0) return (k & 3) == 1 ? 0.0625f : (k & 3) == 2 ? 0.00390625f : 1.0f;
  else if constexpr (C == 1) return (k & 1) ? 0.0625f : 1.0f;
  else return 1.0f;
}

// Per-class constants (D channels, class C: b = 2 << C).
template <int D, int C>
struct Cls {
  static constexpr int b = 2 << C;
  static constexpr int RB = D * b / 8;             // code row bytes of one (token, head)
  static constexpr int NWK = RB / 16;              // words per lane in phase 1 (a quarter row)
  static constexpr int TK = C <= 1 ? 64 : C == 2 ? 32 : 16;   // keys per phase-2 tile
  static constexpr int RS = RB + 16;               // LDS row stride of a staged tile
  static constexpr int PPR = RB / 16;              // 16-byte pieces per row
  static constexpr int NP = TK * PPR;              // pieces per tile
  static constexpr int NPL = (NP + 63) / 64;       // pieces per lane
  // phase-1 groups of 16 keys per batch: 4 KB of codes per wave (2 KB for D = 64's 2- and 4-bit
  // classes, whose chunks hold fewer bytes), and the side-data slots that cover them (64 keys each)
  static constexpr int U = (D == 128) ? (C == 0 ? 8 : C == 1 ? 4 : C == 2 ? 2 : 1) : (C <= 2 ? 4 : 2);
  static constexpr int NS = (16 * U + 63) / 64;
};

// Shared state of a work item.
template <int D, int GB>
struct Smem {
  static constexpr int SCAP = chunk_cap<GB>() + 32;   // per column: chunk + 8-padding per class
  static constexpr int VT = D == 128 ? 5120 : 3072;   // one staged V tile (largest class)
  // The 2-bit class's contribution waits in LDS (one column) or in registers (blocks of query
  // heads, whose LDS is the tighter budget; it passes through the dead score buffer at the end).
  static constexpr bool kOdLds = GB == 1;
  union {                                             // phase 1 reads qv, phase 2 stages vt
    alignas(16) uint8_t vt[VT];                       // one staged V tile
    alignas(16) uint16_t qv[4][GB][D];                // query rows as A operands, per class
  };
  alignas(16) float sc[GB * SCAP];                    // scores; q rows during the prologue
  alignas(16) uint16_t pb[GB + 1][2][64];             // P' hi / lo of a tile; column GB = zeros
  alignas(16) float od[kOdLds ? GB : 1][kOdLds ? D : 1];
  int32_t pg[TR_NCLASS][kPgMax];                      // page ids of the chunk, per class
  float qoff[4][GB];                                  // 1024 * sum of each class's A row
  float isig[GB], qsum[GB], cmax[GB];
  int32_t lb[TR_NCLASS][GB];                          // first visible slot per class and column
};

// The query operand's channel map.  Lane l builds 8 elements of the A operand of class
// cl = l / (D / 8) (classes 0, 1, 2 fp16, class 3 bf16) for MFMA step s and lane group g
// ((s, g) = ((l % (D / 8)) / 4, l % 4)): element j is channel ch[l][j] of the query row, times
// 2^-fx[l][j], the inverse of the power of two at which the key expansion leaves that channel's
// code field (D / 4 channels per lane group).  A compile-time table: every item reads its two
// 8-byte rows instead of recomputing the map.
struct QMap {
  uint8_t ch[kWave][8];
  uint8_t fx[kWave][8];
};
template <int D>
constexpr QMap make_qmap() {
  QMap t{};
  constexpr int GPC = (D / 32) * 4;
  for (int lane = 0; lane < kWave; ++lane) {
    const int cl = lane / GPC, sg = lane % GPC, s = sg / 4, g = sg % 4;
    const int base = (D / 4) * g;
    for (int j = 0; j < 8; ++j) {
      int ch = 0, fx = 0;
      if (cl == 0) {                               // 2-bit: pairs (f, 8 + f) of field f in 0..4
        const int fld = 4 * (s & 1) + (j >> 1);
        ch = base + 16 * (s >> 1) + fld + 8 * (j & 1);
        fx = 2 * (fld < 5 ? fld : fld - 5);
      } else if (cl == 1) {                        // 4-bit: pairs (0, 4), (1, 5) x 16, ...
        ch = base + 8 * s + (j >> 1) + 4 * (j & 1);
        fx = ((j >> 1) & 1) ? 4 : 0;
      } else if (cl < 4) {                         // 8-bit and bf16: in order
        ch = base + 8 * s + j;
      }
      t.ch[lane][j] = (uint8_t)ch;
      t.fx[lane][j] = (uint8_t)fx;
    }
  }
  return t;
}
__constant__ QMap kQmap64 = make_qmap<64>();
__constant__ QMap kQmap128 = make_qmap<128>();

// A phase-1 batch: the code words of U groups of 16 keys (lane: key kr of each group, quarter row g),
// and the K scale / zero and V scale of the batch's keys, one key per lane (key 64 i + lane in slot
// i), handed to the lanes that need them by a cross-lane permute.
template <int D, int C>
struct P1Batch {
  uint32_t w[Cls<D, C>::U][Cls<D, C>::NWK];
  float sk[Cls<D, C>::NS], zk[Cls<D, C>::NS], sv[Cls<D, C>::NS];
};

// Issues the loads of the phase-1 batch of class C that starts at class slot `base` (of the slots
// [., e) whose pages are listed in sm.pg[C] from page `first` on).  Indices are clamped into the
// range, so the loads never branch.
template <int D, int GB, int C>
__device__ __forceinline__ void p1_load(const CacheLayout& c, const Smem<D, GB>& sm, int first, int h, int e, int base,
                                        P1Batch<D, C>& bt) {
  using K = Cls<D, C>;
  const int lane = threadIdx.x, kr = lane & 15, g = lane >> 4;
  const int lp = c.ptok_log2[C], pm = c.ptok[C] - 1, P = c.ptok[C];
  const uint64_t pool = (uint64_t)c.pool;
  const uint32_t pbytes = (uint32_t)c.page_bytes;
  const uint64_t code_base = pool + (uint32_t)(c.k_off[C] + h * c.cb + g * (K::RB / 4));
  const uint64_t sk_base = pool + (uint32_t)(c.sk_off[C] + h * P * 8), sv_base = pool + (uint32_t)(c.sv_off[C] + h * P * 8);
  const uint32_t pgb = pg_base(sm.pg[C], first);
  if constexpr (C < 3) {
#pragma unroll
    for (int i = 0; i < K::NS; ++i) {
      const int j = min(base + 64 * i + lane, e - 1);
      const int32_t page = page_of(pgb, j, lp);
      const u32x2 kz = gload<u32x2>(page_row(sk_base, pbytes, page, j & pm, 8u));
      bt.sk[i] = __uint_as_float(kz[0]);
      bt.zk[i] = __uint_as_float(kz[1]);
      bt.sv[i] = gload<float>(page_row(sv_base, pbytes, page, j & pm, 8u));
    }
  }
#pragma unroll
  for (int u = 0; u < K::U; ++u) {
    const int j = min(base + 16 * u + kr, e - 1);
    const gbytes_t src = page_row(code_base, pbytes, page_of(pgb, j, lp), j & pm, (uint32_t)K::RB);
    if constexpr (K::NWK == 1) {
      bt.w[u][0] = gload<uint32_t>(src);
    } else if constexpr (K::NWK == 2) {
      const u32x2 v = gload<u32x2>(src);
      bt.w[u][0] = v[0]; bt.w[u][1] = v[1];
    } else {
#pragma unroll
      for (int x = 0; x < K::NWK / 4; ++x) {
        const u32x4 v = gload<u32x4>(src + 16 * x);
        bt.w[u][4 * x] = v[0]; bt.w[u][4 * x + 1] = v[1]; bt.w[u][4 * x + 2] = v[2]; bt.w[u][4 * x + 3] = v[3];
      }
    }
  }
}

// Phase 1 for width class C over class slots [a, e): scores into sc[n * SCAP + off + (j - a)].
// `cur` holds the loads of the first batch (slots from a), issued by the caller.
template <int D, int GB, int C, typename Next>
__device__ __forceinline__ void phase1(const CacheLayout& c, Smem<D, GB>& sm, int first, int h, int a, int e, int off,
                                       int ncol, float kscale, float (&mrun)[(GB + 3) / 4], float& vmax,
                                       P1Batch<D, C> cur, Next&& next) {
  using K = Cls<D, C>;
  constexpr int KS = D / 32;
  constexpr int NCL = (GB + 3) / 4;
  constexpr int SCAP = Smem<D, GB>::SCAP;
  constexpr int U = K::U;
  const int lane = threadIdx.x, kr = lane & 15, g = lane >> 4;
  // A operand: query row n at MFMA row 4 (n % 4) + n / 4, zeros for rows without a column
  uint32_t qa[KS][4];
  {
    const int n = 4 * (kr & 3) + (kr >> 2);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (n < ncol) v = *reinterpret_cast<const uint4*>(&sm.qv[C][n][(s * 4 + g) * 8]);
      qa[s][0] = v.x; qa[s][1] = v.y; qa[s][2] = v.z; qa[s][3] = v.w;
    }
  }
  // this lane's columns n = 4 i + g: score factors and first visible slot
  float fs[NCL], fz[NCL], fo[NCL];
  int lbn[NCL];
  bool act[NCL];
#pragma unroll
  for (int i = 0; i < NCL; ++i) {
    const int n = 4 * i + g;
    act[i] = n < ncol && sm.lb[C][min(n, GB - 1)] >= 0;
    const int nn = act[i] ? n : 0;
    fs[i] = (C < 3 ? sm.isig[nn] : 1.0f) * kscale;
    fz[i] = sm.qsum[nn] * kscale;
    fo[i] = sm.qoff[C][nn];
    lbn[i] = act[i] ? sm.lb[C][nn] : e;
  }
  const uint32_t KK = opaque_v(kF16K);
  uint32_t mk[5] = {0, 0, 0, 0, 0};
  if constexpr (C == 0) {
#pragma unroll
    for (int f = 0; f < 5; ++f) mk[f] = opaque_s(0x00030003u << (2 * f));
  } else if constexpr (C == 1) {
    mk[0] = opaque_s(0x000f000fu);
    mk[1] = opaque_s(0x00f000f0u);
  }
  const uint32_t BB = opaque_s(kF16B);

  // One batch: U groups of 16 keys from `base`; scores of the keys before e.
  auto compute = [&](const P1Batch<D, C>& cur, int base) {
    if constexpr (C < 3) {
#pragma unroll
      for (int i = 0; i < K::NS; ++i)
        if (base + 64 * i + lane < e) vmax = fmaxf(vmax, cur.sv[i]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (base + 16 * u >= e) break;               // past the class's last key (wave-uniform)
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        uint32_t bop[4];
        if constexpr (C == 0) {
          if ((s & 1) == 0) {
            uint32_t p8[8];
            exp_k2(cur.w[u][s >> 1], p8, KK, mk);
            bop[0] = p8[0]; bop[1] = p8[1]; bop[2] = p8[2]; bop[3] = p8[3];
            acc = mma_f16(qa[s], bop, acc);
            bop[0] = p8[4]; bop[1] = p8[5]; bop[2] = p8[6]; bop[3] = p8[7];
            acc = mma_f16(qa[s + 1], bop, acc);
          }
        } else if constexpr (C == 1) {
          exp_k4(cur.w[u][s], bop, KK, mk[0], mk[1]);
          acc = mma_f16(qa[s], bop, acc);
        } else if constexpr (C == 2) {
          exp_k8(cur.w[u][2 * s], bop, BB);
          exp_k8(cur.w[u][2 * s + 1], bop + 2, BB);
          acc = mma_f16(qa[s], bop, acc);
        } else {
          bop[0] = cur.w[u][4 * s]; bop[1] = cur.w[u][4 * s + 1];
          bop[2] = cur.w[u][4 * s + 2]; bop[3] = cur.w[u][4 * s + 3];
          acc = mma_bf16(qa[s], bop, acc);
        }
      }
      // lane (key kr, group g) holds rows 4 g + i: columns n = 4 i + g
      const int jr = base + 16 * u + kr;
      float sk = 0.0f, zk = 0.0f;
      if constexpr (C < 3) {                       // key 16 u + kr of the batch: slot u / 4
        const int src = 4 * (16 * (u & 3) + kr);
        sk = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(cur.sk[u >> 2])));
        zk = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(cur.zk[u >> 2])));
      }
#pragma unroll
      for (int i = 0; i < NCL; ++i) {
        if (!act[i] || jr >= e) continue;
        float x;
        if constexpr (C < 3) x = fmaf(sk * fs[i], acc[i] - fo[i], zk * fz[i]);
        else x = acc[i] * fs[i];
        x = jr >= lbn[i] ? x : -INFINITY;
        mrun[i] = fmaxf(mrun[i], x);
        sm.sc[(4 * i + g) * SCAP + off + (jr - a)] = x;
      }
    }
  };
  // The next batch's loads are issued before the current one is computed, so they stay in flight
  // during its products; the last batch is peeled off and runs with `next()`'s loads in flight (the
  // first loads of the next class or phase).  The batches rotate by value (see phase 2).
  P1Batch<D, C> nxt;
  int base = a;
  for (; base + 16 * U < e; base += 16 * U) {
    p1_load<D, GB, C>(c, sm, first, h, e, base + 16 * U, nxt);
    compute(cur, base);
    cur = nxt;
  }
  next();
  compute(cur, base);
}

// A phase-2 tile: the 16-byte code pieces of TK keys' V rows (NPL per lane) and, in lane j, key j's
// V scale and zero.
template <int D, int C>
struct P2Tile {
  u32x4 pc[Cls<D, C>::NPL];
  float sz[2];
};

// Issues the loads of the phase-2 tile of class C that starts at class slot tb (of the slots
// [., e) whose pages are listed in sm.pg[C] from page `first` on), indices clamped into the range.
template <int D, int GB, int C>
__device__ __forceinline__ void p2_load(const CacheLayout& c, const Smem<D, GB>& sm, int first, int h, int e, int tb,
                                        P2Tile<D, C>& tl) {
  using K = Cls<D, C>;
  constexpr int TK = K::TK;
  const int lane = threadIdx.x;
  const int lpg = c.ptok_log2[C], pm = c.ptok[C] - 1, P = c.ptok[C];
  const uint64_t pool = (uint64_t)c.pool;
  const uint32_t pbytes = (uint32_t)c.page_bytes;
  const uint32_t pgb = pg_base(sm.pg[C], first);
#pragma unroll
  for (int x = 0; x < K::NPL; ++x) {
    const int pcx = lane + 64 * x;
    const int key = min(pcx / K::PPR, TK - 1), part = pcx % K::PPR;
    const int j = min(tb + key, e - 1);
    const uint64_t code_base = pool + (uint32_t)(c.v_off[C] + h * c.cb + 16 * part);
    tl.pc[x] = gload<u32x4>(page_row(code_base, pbytes, page_of(pgb, j, lpg), j & pm, (uint32_t)K::RB));
  }
  if constexpr (C < 3) {
    const uint64_t sv_base = pool + (uint32_t)(c.sv_off[C] + h * P * 8);
    const int j = min(tb + min(lane, TK - 1), e - 1);
    const u32x2 w = gload<u32x2>(page_row(sv_base, pbytes, page_of(pgb, j, lpg), j & pm, 8u));
    tl.sz[0] = __uint_as_float(w[0]);
    tl.sz[1] = __uint_as_float(w[1]);
  } else {
    tl.sz[0] = 1.0f;
    tl.sz[1] = 0.0f;
  }
}

// Phase 2 for width class C over class slots [a, e): acc += V^T P'^T in units of 2^tau.  `cur` holds
// the loads of the first tile (slots from a), issued by the caller; the last tile's products run
// with `next()`'s loads in flight (the first tile of the next class) instead of another tile's.
template <int D, int GB, int C, typename Next>
__device__ __forceinline__ void phase2(const CacheLayout& c, Smem<D, GB>& sm, int first, int h, int a, int e, int off,
                                       int ncol, float tsc, f32x4 (&acc)[D / 16], float (&lp)[GB], float (&zp)[GB],
                                       float (&cp)[GB], P2Tile<D, C> cur, Next&& next) {
  using K = Cls<D, C>;
  constexpr int NT = D / 16;
  constexpr int SCAP = Smem<D, GB>::SCAP;
  // SP: the 2-bit class restaged with each code in a 4-bit slot (blocks of query heads), so that
  // its products land in the same accumulator layout as the other classes
  constexpr bool SP = C == 0 && !Smem<D, GB>::kOdLds;
  constexpr int TK = K::TK, RS = SP ? 2 * K::RB + 16 : K::RS;
  const int lane = threadIdx.x, r = lane & 15, g = lane >> 4;
  const uint32_t KK = opaque_v(kF16K);
  const uint32_t m40 = opaque_s(0x000f000fu), m41 = opaque_s(0x00f000f0u);
  const uint32_t m20 = opaque_s(0x00030003u), m21 = opaque_s(0x00300030u), m22 = opaque_s(0x03000300u);
  const uint32_t BB = opaque_s(kF16B);
  // this lane's B-operand column (P' rows of column n; the zero column for rows without one)
  const int ncolB = (r < ncol) ? r : GB;
  // tr read address of this lane within a tile (plus the channel-tile offset)
  int tro;
  if constexpr (C <= 1) tro = (16 * g + r) * RS;                            // tr4: row = key 16 g + r
  else if constexpr (C == 2) tro = (8 * g + (r >> 1)) * RS + 8 * (r & 1);   // tr8: key 8 g + r / 2
  else tro = (4 * g + (r >> 2)) * RS + 8 * (r & 3);                         // tr16: key 4 g + r / 4

  using Tile = P2Tile<D, C>;
  // One tile from tb, with its rows and V side data already in registers.
  auto run = [&](const Tile& cur, int tb) {
    // stage the tile's rows
#pragma unroll
    for (int x = 0; x < K::NPL; ++x) {
      const int pcx = lane + 64 * x;
      if (K::NP % 64 == 0 || pcx < K::NP) {
        if constexpr (SP) {
          const u32x4 v = cur.pc[x];
          const u32x4 lo = {spread2(v[0], false), spread2(v[0], true), spread2(v[1], false), spread2(v[1], true)};
          const u32x4 hi = {spread2(v[2], false), spread2(v[2], true), spread2(v[3], false), spread2(v[3], true)};
          uint8_t* dst = sm.vt + (pcx / K::PPR) * RS + 32 * (pcx % K::PPR);
          *reinterpret_cast<u32x4*>(dst) = lo;
          *reinterpret_cast<u32x4*>(dst + 16) = hi;
        } else {
          *reinterpret_cast<u32x4*>(sm.vt + (pcx / K::PPR) * RS + 16 * (pcx % K::PPR)) = cur.pc[x];
        }
      }
    }
    const float2 szv = make_float2(cur.sz[0], cur.sz[1]);
    // P' of the tile's keys for every column: key j = lane
    if (lane < TK) {
      const int jr = tb + lane;
      int pos;                                      // element position in the B operand
      float fld;
      if constexpr (C <= 1) {
        const int kk = lane & 7;
        pos = (lane & ~7) + 2 * (kk & 3) + (kk >> 2);
        fld = pfield<SP ? 1 : C>(kk);
      } else {
        pos = lane;
        fld = 1.0f;
      }
#pragma unroll
      for (int n = 0; n < GB; ++n) {
        if (n >= ncol) break;
        const float mx = sm.cmax[n];
        float p = 0.0f;
        if (jr < e && mx != -INFINITY) p = exp2f(sm.sc[n * SCAP + off + (jr - a)] - mx);
        lp[n] += p;
        uint16_t hi, lo;
        if constexpr (C < 3) {
          zp[n] = fmaf(p, szv.y, zp[n]);
          const float v = p * szv.x * tsc * fld;
          const _Float16 vh = (_Float16)v;
          const _Float16 vl = (_Float16)(v - (float)vh);
          cp[n] += 1024.0f * ((float)vh + (float)vl);   // the offset the fp16 codes carry
          hi = __builtin_bit_cast(uint16_t, vh);
          lo = __builtin_bit_cast(uint16_t, vl);
        } else {
          const float v = p * tsc;
          hi = tr_f32_to_bf16(v);
          lo = tr_f32_to_bf16(v - tr_bf16_lo(hi));
        }
        sm.pb[n][0][pos] = hi;
        sm.pb[n][1][pos] = lo;
      }
    }
    wave_lds_sync();
    if constexpr (C <= 1) {
      // B operands: keys 16 g + 8 hb .. + 7 (the two words of this lane group's tr4 rows)
      uint32_t bh[2][4], bl[2][4];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const uint4 vh = *reinterpret_cast<const uint4*>(&sm.pb[ncolB][0][(2 * g + hb) * 8]);
        const uint4 vl = *reinterpret_cast<const uint4*>(&sm.pb[ncolB][1][(2 * g + hb) * 8]);
        bh[hb][0] = vh.x; bh[hb][1] = vh.y; bh[hb][2] = vh.z; bh[hb][3] = vh.w;
        bl[hb][0] = vl.x; bl[hb][1] = vl.y; bl[hb][2] = vl.z; bl[hb][3] = vl.w;
      }
      if constexpr (C == 1 || SP) {
#pragma unroll
        for (int m = 0; m < NT; ++m) {
          uint32_t x0, x1, av[4];
          tr4(sm.vt + tro + 8 * m, x0, x1);
          exp_k4(x0, av, KK, m40, m41);
          acc[m] = mma_f16(av, bh[0], acc[m]);
          acc[m] = mma_f16(av, bl[0], acc[m]);
          exp_k4(x1, av, KK, m40, m41);
          acc[m] = mma_f16(av, bh[1], acc[m]);
          acc[m] = mma_f16(av, bl[1], acc[m]);
        }
      } else {
        // 32 channels per tr4 (two per nibble): even channels into tile 2 m, odd into 2 m + 1
#pragma unroll
        for (int m = 0; m < NT / 2; ++m) {
          uint32_t x0, x1, av[4];
          tr4(sm.vt + tro + 8 * m, x0, x1);
          exp_v2(x0, av, KK, m20, m21, m22);
          acc[2 * m] = mma_f16(av, bh[0], acc[2 * m]);
          acc[2 * m] = mma_f16(av, bl[0], acc[2 * m]);
          exp_v2(x0 >> 2, av, KK, m20, m21, m22);
          acc[2 * m + 1] = mma_f16(av, bh[0], acc[2 * m + 1]);
          acc[2 * m + 1] = mma_f16(av, bl[0], acc[2 * m + 1]);
          exp_v2(x1, av, KK, m20, m21, m22);
          acc[2 * m] = mma_f16(av, bh[1], acc[2 * m]);
          acc[2 * m] = mma_f16(av, bl[1], acc[2 * m]);
          exp_v2(x1 >> 2, av, KK, m20, m21, m22);
          acc[2 * m + 1] = mma_f16(av, bh[1], acc[2 * m + 1]);
          acc[2 * m + 1] = mma_f16(av, bl[1], acc[2 * m + 1]);
        }
      }
    } else if constexpr (C == 2) {
      uint32_t bh[4], bl[4];
      {
        const uint4 vh = *reinterpret_cast<const uint4*>(&sm.pb[ncolB][0][8 * g]);
        const uint4 vl = *reinterpret_cast<const uint4*>(&sm.pb[ncolB][1][8 * g]);
        bh[0] = vh.x; bh[1] = vh.y; bh[2] = vh.z; bh[3] = vh.w;
        bl[0] = vl.x; bl[1] = vl.y; bl[2] = vl.z; bl[3] = vl.w;
      }
#pragma unroll
      for (int m = 0; m < NT; ++m) {
        uint32_t x0, x1, av[4];
        tr8(sm.vt + tro + 16 * m, x0, x1);
        exp_k8(x0, av, BB);
        exp_k8(x1, av + 2, BB);
        acc[m] = mma_f16(av, bh, acc[m]);
        acc[m] = mma_f16(av, bl, acc[m]);
      }
    } else {
      const uint2 vh = *reinterpret_cast<const uint2*>(&sm.pb[ncolB][0][4 * g]);
      const uint2 vl = *reinterpret_cast<const uint2*>(&sm.pb[ncolB][1][4 * g]);
#pragma unroll
      for (int m = 0; m < NT; ++m) {
        uint32_t x0, x1;
        tr16(sm.vt + tro + 32 * m, x0, x1);
        acc[m] = mma_bf16_k16(x0, x1, vh.x, vh.y, acc[m]);
        acc[m] = mma_bf16_k16(x0, x1, vl.x, vl.y, acc[m]);
      }
    }
    wave_lds_sync();                               // the tile and P' are rewritten next
  };
  // The next tile's loads are issued before the current one is staged and computed, so they stay
  // in flight during its products; the last tile is peeled off, and the next class's first loads
  // go out in its place (a branch between the two kinds of loads in one body would make the wait
  // counts of every tile assume the smaller of the two).  The tiles rotate by value: two tiles
  // used in turn through one loop body would be addressed through a pointer, which keeps them out
  // of registers (in scratch memory, one more round trip per tile).
  Tile nxt;
  int tb = a;
  for (; tb + TK < e; tb += TK) {
    p2_load<D, GB, C>(c, sm, first, h, e, tb + TK, nxt);
    run(cur, tb);
    cur = nxt;
  }
  next();
  run(cur, tb);
}

// e with vmax <= 2^e (0 for vmax = 0): the P' normalization of a class set.
__device__ __forceinline__ int scale_exp(float vmax) { return vmax > 0.0f ? __builtin_amdgcn_frexp_expf(vmax) : 0; }

// Agent-coherent (sc1) vector memory accesses for the split-K records: a record written by a wave
// on one XCD is read by a wave of the same launch on another, so it must not wait in either XCD's
// L2.  The base and size of a (seq, query head)'s records sit in a buffer resource.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kSc1 = 16;                            // cache policy bits: sc1 (agent scope)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rec_rsrc(const float* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), (short)0, (int)bytes, kRsrcWord3);
}

// Log-sum-exp merge of one (seq, query head)'s nch chunk records (o[D], m, l) into bf16 `dst`, by a
// single wave: lane l holds channels D / 64 * l .. + D / 64 - 1.  Records go in batches of 32: every
// load of a batch (the lane's channels of 32 records and, in lane k, record k's (m, l)) is issued
// at once, indices clamped into the window, then the batch folds into a running (max, num, den)
// with the chunk weights broadcast from their lanes.
template <int D>
__device__ __forceinline__ void merge_records(__amdgpu_buffer_rsrc_t rs, int nch, uint16_t* __restrict__ dst) {
  constexpr int KB = kMergeBatch, CPL = D / 64, REC = (D + 2) * 4;
  const int lane = threadIdx.x;
  float M = -INFINITY, den = 0.0f, num[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) num[i] = 0.0f;
  for (int k0 = 0; k0 < nch; k0 += KB) {
    float v[KB][CPL];
#pragma unroll
    for (int x = 0; x < KB; ++x) {
      const int off = min(k0 + x, nch - 1) * REC + 4 * CPL * lane;
      if constexpr (CPL == 2) {
        const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kSc1));
        v[x][0] = __uint_as_float(w[0]);
        v[x][1] = __uint_as_float(w[1]);
      } else {
        v[x][0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, kSc1));
      }
    }
    const int kk = k0 + (lane & (KB - 1));
    const u32x2 ml =
        __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, min(kk, nch - 1) * REC + 4 * D, 0, kSc1));
    const bool own = kk < nch && lane < KB;         // lanes KB..63 repeat lanes 0..KB-1
    const float mk = own ? __uint_as_float(ml[0]) : -INFINITY;
    const float lk = __uint_as_float(ml[1]);
    const float Mn = fmaxf(M, wave_max(mk));
    const float a = (M == -INFINITY) ? 0.0f : exp2f(M - Mn);
    const float wk = (own && mk != -INFINITY) ? exp2f(mk - Mn) : 0.0f;
    den = den * a + wave_sum(wk * lk);
    float nb[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) nb[i] = 0.0f;
#pragma unroll
    for (int x = 0; x < KB; ++x) {
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk), x));
#pragma unroll
      for (int i = 0; i < CPL; ++i) nb[i] = fmaf(w, v[x][i], nb[i]);
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) num[i] = num[i] * a + nb[i];
    M = Mn;
  }
  if constexpr (CPL == 2) {
    const uint32_t w = (uint32_t)tr_f32_to_bf16(num[0] / den) | ((uint32_t)tr_f32_to_bf16(num[1] / den) << 16);
    *reinterpret_cast<uint32_t*>(dst + 2 * lane) = w;
  } else {
    dst[lane] = tr_f32_to_bf16(num[0] / den);
  }
}

// Occupancy floor handed to the compiler.
#ifndef TR_DECODE_WAVES
#define TR_DECODE_WAVES 4
#endif
// Work items in launch order.  Each item is one chunk of one group (seq, KV head, block of query
// heads); a group is "full" if any of its columns is, else "local" if any is, else "skip".  Rank r
// (the block index) takes, in turn: the chunks of the full groups (chunk-major: chunk 0 of every
// full group, then chunk 1, ...), the chunks of the local groups (chunk-major), one item per skip
// group (it writes the zero rows), and nothing for the ranks left over.  So every item that
// reads the cache is dispatched before any empty one -- mixed in, the short-lived empty waves make
// the dispatcher pile long ones onto a few compute units -- and consecutive ranks, which go to
// the XCDs in turn, spread each chunk index over all of them.
//
// Every wave ranks the groups itself: lane l holds groups [l P, l P + P) (P <= kRankPerLane; larger
// batches fall back to chunk-major order over all groups), one bit each in a full and a local
// mask; scans over the lanes place rank r.
constexpr int kRankPerLane = 32;

__device__ __forceinline__ bool item_of_rank(int r, const uint8_t* __restrict__ mode, int groups, int H, int HQ, int G,
                                             int GB, int NB, int nchf, int nchl, int& k, int& grp) {
  const int lane = threadIdx.x;
  const int P = (groups + kWave - 1) / kWave;
  if (P > kRankPerLane) {
    k = r / groups;
    grp = r % groups;
    return k < nchf;
  }
  uint32_t fb = 0, lb = 0, vb = 0;
  for (int i0 = 0; i0 < P; i0 += 8) {
    uint8_t m[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {                    // every load issued before any is used
      const int g = min(lane * P + i0 + i, groups - 1);
      if (NB == 1) {
        // one block per KV head: group g's G columns are query heads g G .. g G + G - 1
#pragma unroll
        for (int n = 0; n < 4; ++n) m[i][n] = n < GB ? mode[(int64_t)g * G + min(n, G - 1)] : 0;
      } else {
        const int s = g / (H * NB), hb = g % (H * NB);
        const int h0 = (hb / NB) * G + (hb % NB) * GB;
        const int nc = min(GB, G - (hb % NB) * GB);
#pragma unroll
        for (int n = 0; n < 4; ++n) m[i][n] = n < GB ? mode[(int64_t)s * HQ + h0 + min(n, nc - 1)] : 0;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int li = i0 + i;
      if (li >= P || lane * P + li >= groups) continue;
      bool full = false, loc = false;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        full = full || m[i][n] == TR_MODE_FULL;
        loc = loc || m[i][n] == TR_MODE_LOCAL;
      }
      vb |= 1u << li;
      fb |= (full ? 1u : 0u) << li;
      lb |= (!full && loc ? 1u : 0u) << li;
    }
  }
  const uint32_t sb = vb & ~(fb | lb);
  // inclusive scans over the lanes of the three counts, packed 21 bits apiece
  long long sc = (long long)__popc(fb) | ((long long)__popc(lb) << 21) | ((long long)__popc(sb) << 42);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const long long x = __shfl_up(sc, o);
    if (lane >= o) sc += x;
  }
  const long long tot = __shfl(sc, kWave - 1);
  const int NF = (int)__builtin_amdgcn_readfirstlane((int)(tot & 0x1fffff));
  const int NL = (int)__builtin_amdgcn_readfirstlane((int)((tot >> 21) & 0x1fffff));
  const int NS = (int)__builtin_amdgcn_readfirstlane((int)((tot >> 42) & 0x1fffff));
  int which, j;
  if (r < NF * nchf) {
    which = 0;
    k = r / NF;
    j = r % NF;
  } else if (r - NF * nchf < NL * nchl) {
    which = 1;
    k = (r - NF * nchf) / NL;
    j = (r - NF * nchf) % NL;
  } else if (r - NF * nchf - NL * nchl < NS) {
    which = 2;
    k = 0;
    j = r - NF * nchf - NL * nchl;
  } else {
    return false;
  }
  const uint32_t bits = which == 0 ? fb : which == 1 ? lb : sb;
  const int incl = (int)((sc >> (21 * which)) & 0x1fffff);
  const int excl = incl - __popc(bits);
  const uint64_t hit = __ballot(excl <= j && j < incl);
  const int L = __builtin_amdgcn_readfirstlane(hit ? (int)__builtin_ctzll(hit) : 0);
  // the (j - excl)-th set bit of this lane's mask (meaningful in lane L only)
  uint32_t b = bits;
  const int drop = min(max(j - excl, 0), 31);
  for (int x = 0; x < drop; ++x) b &= b - 1;
  const int pos = b ? __builtin_ctz(b) : 0;
  grp = __builtin_amdgcn_readlane(lane * P + pos, L);
  return true;
}

template <int D, int GB>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(TR_DECODE_WAVES, 8))) void k_decode(
    CacheLayout c, int layer, int t, int window, int CH, int stride, float kscale, const uint16_t* __restrict__ q,
    const uint8_t* __restrict__ mode, float* __restrict__ part, uint16_t* __restrict__ out, int HQ, int G, int NB,
    int32_t* __restrict__ cnt) {
  constexpr int NT = D / 16, KS = D / 32, NCL = (GB + 3) / 4;
  __shared__ Smem<D, GB> sm;
  // one column per item only without grouping (G = 1, so one block per KV head)
  if constexpr (GB == 1) {
    G = 1;
    NB = 1;
  }
  const int lane = threadIdx.x;
  const int groups = c.B * c.H * NB;
  int k, grp;
  {
    const int nchf = (t + 1 + CH - 1) / CH, nchl = (t + 1 - max(0, t - window) + CH - 1) / CH;
    if (!item_of_rank(blockIdx.x, mode, groups, c.H, HQ, G, GB, NB, nchf, nchl, k, grp)) return;
  }
  const int s = grp / (c.H * NB), hb = grp % (c.H * NB);
  const int hk = hb / NB, blk = hb % NB;
  const int h0 = hk * G + blk * GB;                  // the block's first query head
  const int ncol = min(GB, G - blk * GB);
  const int64_t row0 = (int64_t)s * HQ + h0;         // (seq, query head) index of column 0

  // Every load that needs nothing else goes out at once: the columns' modes, the query rows, and
  // the class prefix rows of the chunk under both possible windows (any full column: [0, t];
  // local columns only: [lo_loc, t]) plus that of lo_loc.  Page ids follow; phase 1 next.
  const int lo_loc = max(0, t - window);
  int cb[2][2];                                      // [window kind][p0, p1]; p0 > t: no chunk k
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const int lo = w == 0 ? 0 : lo_loc;
    const int L = t + 1 - lo;
    const int nch = (L + CH - 1) / CH;
    const int per = (L + nch - 1) / nch;
    cb[w][0] = k < nch ? lo + k * per : t + 1;
    cb[w][1] = k < nch ? min(cb[w][0] + per, t + 1) : t + 1;
  }
  const int mval = lane < ncol ? (int)mode[row0 + lane] : 0;
  const QMap& qmap = D == 128 ? kQmap128 : kQmap64;
  const u32x2 qch = *reinterpret_cast<const u32x2*>(&qmap.ch[lane][0]);
  const u32x2 qfx = *reinterpret_cast<const u32x2*>(&qmap.fx[lane][0]);
  constexpr int QPL = (GB * D + kWave - 1) / kWave;  // query values per lane
  uint16_t qraw[QPL];
#pragma unroll
  for (int i = 0; i < QPL; ++i) {
    const int x = lane + kWave * i;
    // unconditional (clamped) loads: one under a condition would wait on the spot; the values
    // past the block's columns are never used
    qraw[i] = q[row0 * D + min(x, ncol * D - 1)];
  }
  const int4 paf = *reinterpret_cast<const int4*>(tr_prefix_row(c, layer, s, cb[0][0]));
  const int4 pef = *reinterpret_cast<const int4*>(tr_prefix_row(c, layer, s, cb[0][1]));
  const int4 pal = *reinterpret_cast<const int4*>(tr_prefix_row(c, layer, s, cb[1][0]));
  const int4 pel = *reinterpret_cast<const int4*>(tr_prefix_row(c, layer, s, cb[1][1]));
  const int4 pl = *reinterpret_cast<const int4*>(tr_prefix_row(c, layer, s, lo_loc));
  // the prefix rows arrive here, together with the modes and query rows issued above (otherwise
  // the compiler issues them only after the modes are used, one more memory round trip)
  asm volatile("" ::"s"(paf.x), "s"(paf.y), "s"(paf.z), "s"(paf.w), "s"(pef.x), "s"(pef.y), "s"(pef.z), "s"(pef.w));
  asm volatile("" ::"s"(pal.x), "s"(pal.y), "s"(pal.z), "s"(pal.w), "s"(pel.x), "s"(pel.y), "s"(pel.z), "s"(pel.w));
  asm volatile("" ::"s"(pl.x), "s"(pl.y), "s"(pl.z), "s"(pl.w), "v"(qch[0]), "v"(qch[1]), "v"(qfx[0]), "v"(qfx[1]));

  // modes of the block's columns
  const bool bad = lane < ncol && mval > TR_MODE_FULL;
  const uint64_t fullm = __ballot(lane < ncol && mval == TR_MODE_FULL);
  const uint64_t locm = __ballot(lane < ncol && mval == TR_MODE_LOCAL);
  if (k == 0) {
    if (bad) atomicOr(c.err, TR_ERRF_BAD_MODE);
    // columns that attend to nothing get zeros
    for (int n = 0; n < ncol; ++n) {
      if (((fullm | locm) >> n) & 1) continue;
      for (int d = lane; d < D; d += kWave) out[(row0 + n) * D + d] = 0;
    }
  }
  if (!(fullm | locm)) return;
  const int wk = fullm ? 0 : 1;
  const int p0 = cb[wk][0];
  if (p0 > t) return;                                // the union window has fewer chunks
  const int lo = fullm ? 0 : lo_loc;
  const int nch = (t + 1 - lo + CH - 1) / CH;
  const bool mixed = fullm && locm;

  // slot ranges of the chunk, and the first slot a local column sees
  const int4 pa = fullm ? paf : pal, pe = fullm ? pef : pel;
  const int a[4] = {pa.x, pa.y, pa.z, pa.w}, e[4] = {pe.x, pe.y, pe.z, pe.w};
  const int4 plv = mixed ? pl : pa;
  const int al[4] = {max(pa.x, plv.x), max(pa.y, plv.y), max(pa.z, plv.z), max(pa.w, plv.w)};
  int first[4], off[4];
  {
    int o = 0;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      first[x] = a[x] >> c.ptok_log2[x];
      off[x] = o;
      o += (e[x] - a[x] + 7) & ~7;
    }
  }
  // page ids: at most kPgMax (< 64) per class, one per lane; the four classes' loads go out together
  // and land in LDS after the query rows' sums, so their round trip overlaps that work
  int32_t pv[4];
  {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int np = e[x] > a[x] ? ((e[x] - 1) >> c.ptok_log2[x]) - first[x] + 1 : 0;
      // unconditional (index clamped into the class's page table): a load under a condition
      // makes the compiler's wait counts conservative, and the query rows' wait below would then
      // wait for these too
      const int32_t v = tr_ptab(c, layer, s, x)[min(first[x] + min(lane, max(np - 1, 0)), c.maxp[x] - 1)];
      pv[x] = lane < np ? v : -1;
    }
  }
  // per column: first visible slot per class (-1: the column attends to nothing)
  if (lane < GB) {
    const bool on = lane < ncol && (mval == TR_MODE_FULL || mval == TR_MODE_LOCAL);
#pragma unroll
    for (int x = 0; x < 4; ++x) sm.lb[x][lane] = !on ? -1 : (mval == TR_MODE_LOCAL ? al[x] : a[x]);
  }
  // query rows in fp32 (in the score buffer), their sums and fp16 prescale
  float* qf = sm.sc;
#pragma unroll
  for (int i = 0; i < QPL; ++i) {
    const int x = lane + kWave * i;
    if (x < GB * D) qf[x] = x < ncol * D && (((fullm | locm) >> (x / D)) & 1) ? tr_bf16_lo((uint32_t)qraw[i]) : 0.0f;
  }
  wave_lds_sync();
  for (int n = 0; n < ncol; ++n) {
    float qs = 0.0f, qm = 0.0f;
    for (int d = lane; d < D; d += kWave) {
      const float v = qf[n * D + d];
      qs += v;
      qm = fmaxf(qm, fabsf(v));
    }
    qs = wave_sum(qs);
    qm = wave_max(qm);
    if (lane == 0) {
      const int ex = qm > 0.0f ? __builtin_amdgcn_frexp_expf(qm) : 0;   // qm < 2^ex
      sm.isig[n] = ldexpf(1.0f, ex - 15);                                // q' = q 2^(15 - ex) < 2^15
      sm.qsum[n] = qs;
    }
  }
  // The page ids land in LDS, and the first phase-1 batch of class 0 (and of class 1 with one
  // column, whose registers allow it) goes out: its round trip overlaps the rest of the query work,
  // so the cache reads start as early as the page ids allow.
  constexpr bool kEarly1 = GB == 1;
#pragma unroll
  for (int x = 0; x < 4; ++x)
    if (lane < kPgMax) sm.pg[x][lane] = pv[x];
  wave_lds_sync();
  P1Batch<D, 0> b0;
  P1Batch<D, 1> b1;
  if (e[0] > a[0]) p1_load<D, GB, 0>(c, sm, first[0], hk, e[0], a[0], b0);
  if (kEarly1 && e[1] > a[1]) p1_load<D, GB, 1>(c, sm, first[1], hk, e[1], a[1], b1);
  // A operands of every class: lane -> (class cl, step st, group gg), 8 values each; the fp16
  // classes' 1024-offset sums per (class, column)
  {
    constexpr int GPC = KS * 4;                    // (step, group) pairs per class
    const int cl = lane / GPC, sg = lane % GPC;
    for (int n = 0; n < ncol; ++n) {
      const float pre = 1.0f / sm.isig[n];
      float osum = 0.0f;
      if (cl < 4) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const int ch0 = (qch[j >> 2] >> (8 * (j & 3))) & 0xff, ch1 = (qch[j >> 2] >> (8 * (j & 3) + 8)) & 0xff;
          const int x0 = (qfx[j >> 2] >> (8 * (j & 3))) & 0xff, x1 = (qfx[j >> 2] >> (8 * (j & 3) + 8)) & 0xff;
          const float v0 = qf[n * D + ch0], v1 = qf[n * D + ch1];
          if (cl < 3) {
            const _Float16 h0v = (_Float16)ldexpf(v0 * pre, -x0), h1v = (_Float16)ldexpf(v1 * pre, -x1);
            osum += (float)h0v + (float)h1v;
            w[j / 2] = (uint32_t)__builtin_bit_cast(uint16_t, h0v) | ((uint32_t)__builtin_bit_cast(uint16_t, h1v) << 16);
          } else {
            w[j / 2] = (__float_as_uint(v0) >> 16) | (__float_as_uint(v1) & 0xffff0000u);   // exact: q is bf16
          }
        }
        *reinterpret_cast<uint4*>(&sm.qv[cl][n][sg * 8]) = make_uint4(w[0], w[1], w[2], w[3]);
      }
      // sum over the GPC lanes of each class (rows of 16 lanes for D = 128; half rows for 64)
      if constexpr (GPC == 16) {
        osum = row_sum(osum);
      } else {
        osum += dpp_f<0xB1>(osum);
        osum += dpp_f<0x4E>(osum);
        osum += dpp_f<0x141>(osum);
      }
      if (sg == 0 && cl < 3) sm.qoff[cl][n] = 1024.0f * osum;
    }
  }
  if constexpr (Smem<D, GB>::kOdLds)
    for (int i = lane; i < GB * D; i += kWave) (&sm.od[0][0])[i] = 0.0f;
  for (int i = lane; i < 128; i += kWave) (&sm.pb[GB][0][0])[i] = 0;
  wave_lds_sync();

  // Issue priority by progress: the items of a launch are alike in size and all resident at once,
  // and among waves of equal priority a SIMD issues for the oldest first, so the items would
  // finish in start order, several microseconds apart, the last ones alone at the end.  A wave
  // steps its priority down as it gets through its item (3, 2, 1, 0 at about a quarter, half and
  // three quarters of the work), so that waves behind are issued first and the items finish
  // together.
  __builtin_amdgcn_s_setprio(3);
  // phase 1
  float mrun[NCL];
#pragma unroll
  for (int i = 0; i < NCL; ++i) mrun[i] = -INFINITY;
  float vm[3] = {0.0f, 0.0f, 0.0f};
  float vdummy = 0.0f;
  // One load pipeline across the classes and the two phases (one column per item): the last batch
  // (tile) of a class is computed with the first loads of the next non-empty class in flight -- of
  // phase 2's first class after phase 1's last -- so only a class that follows an empty one starts
  // cold.  Blocks of query heads load each class's first batch on entry: their registers would
  // not hold both (184 instead of 164, two waves per SIMD instead of three).
  constexpr bool kChain = GB == 1;
  const bool nz[4] = {e[0] > a[0], e[1] > a[1], e[2] > a[2], e[3] > a[3]};
  const int lastnz = nz[3] ? 3 : nz[2] ? 2 : nz[1] ? 1 : 0;
  P1Batch<D, 2> b2;
  P1Batch<D, 3> b3;
  P2Tile<D, 0> t0;
  P2Tile<D, 1> t1;
  P2Tile<D, 2> t2;
  P2Tile<D, 3> t3;
  auto load_t0 = [&] {
    if (kChain && nz[0]) p2_load<D, GB, 0>(c, sm, first[0], hk, e[0], a[0], t0);
  };
  if (nz[0])
    phase1<D, GB, 0>(c, sm, first[0], hk, a[0], e[0], off[0], ncol, kscale, mrun, vm[0], b0, [&] {
      if (!nz[1] && lastnz == 0) load_t0();          // (class 1's first batch went out with class 0's)
    });
  if (nz[1]) {
    if (!kEarly1) p1_load<D, GB, 1>(c, sm, first[1], hk, e[1], a[1], b1);
    phase1<D, GB, 1>(c, sm, first[1], hk, a[1], e[1], off[1], ncol, kscale, mrun, vm[1], b1, [&] {
      if constexpr (kChain) {
        if (nz[2]) p1_load<D, GB, 2>(c, sm, first[2], hk, e[2], a[2], b2);
        else if (lastnz == 1) load_t0();
      }
    });
  }
  __builtin_amdgcn_s_setprio(2);
  if (nz[2]) {
    if (!(kChain && nz[1])) p1_load<D, GB, 2>(c, sm, first[2], hk, e[2], a[2], b2);
    phase1<D, GB, 2>(c, sm, first[2], hk, a[2], e[2], off[2], ncol, kscale, mrun, vm[2], b2, [&] {
      if constexpr (kChain) {
        if (nz[3]) p1_load<D, GB, 3>(c, sm, first[3], hk, e[3], a[3], b3);
        else load_t0();
      }
    });
  }
  if (nz[3]) {
    if (!(kChain && nz[2])) p1_load<D, GB, 3>(c, sm, first[3], hk, e[3], a[3], b3);
    phase1<D, GB, 3>(c, sm, first[3], hk, a[3], e[3], off[3], ncol, kscale, mrun, vdummy, b3, load_t0);
  }
  // column maxima: lanes of group g hold columns 4 i + g
#pragma unroll
  for (int i = 0; i < NCL; ++i) {
    const float mx = row_max(mrun[i]);
    if ((lane & 15) == 0 && 4 * i + (lane >> 4) < GB) sm.cmax[4 * i + (lane >> 4)] = mx;
  }
  // P' scales: class 0 alone, classes 1-3 together (b = 16 keys count as scale 1)
  const int e0 = scale_exp(wave_max(vm[0]));
  const int em = scale_exp(fmaxf(wave_max(fmaxf(vm[1], vm[2])), e[3] > a[3] ? 1.0f : 0.0f));
  wave_lds_sync();

  // phase 2
  __builtin_amdgcn_s_setprio(1);
  f32x4 acc[NT];
  float lp[GB], zp[GB], cp[GB];
#pragma unroll
  for (int n = 0; n < GB; ++n) lp[n] = zp[n] = cp[n] = 0.0f;
  const int r = lane & 15, g = lane >> 4;
  constexpr bool kOdLds = Smem<D, GB>::kOdLds;
  if (e[0] > a[0]) {
#pragma unroll
    for (int m = 0; m < NT; ++m) acc[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (!kChain) p2_load<D, GB, 0>(c, sm, first[0], hk, e[0], a[0], t0);
    phase2<D, GB, 0>(c, sm, first[0], hk, a[0], e[0], off[0], ncol, ldexpf(1.0f, -e0), acc, lp, zp, cp, t0, [&] {
      if (kChain && nz[1]) p2_load<D, GB, 1>(c, sm, first[1], hk, e[1], a[1], t1);
    });
    float cr = 0.0f;
#pragma unroll
    for (int n = 0; n < GB; ++n) {
      const float cs = wave_sum(cp[n]);
      cp[n] = 0.0f;
      cr = r == n ? cs : cr;
    }
    if constexpr (kOdLds) {
      // the 2-bit class into od: tile 2 m row L = channel 32 m + 2 L, tile 2 m + 1 the odd one
      const float s0 = ldexpf(1.0f, e0);
      if (r < ncol) {
#pragma unroll
        for (int m = 0; m < NT / 2; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int ch = 32 * m + 2 * (4 * g + i);
            sm.od[r][ch] = (acc[2 * m][i] - cr) * s0;
            sm.od[r][ch + 1] = (acc[2 * m + 1][i] - cr) * s0;
          }
      }
    } else {
      // same layout as the other classes: the offsets out, then rescaled (exactly, by a power of
      // two) to their P' scale, and the other classes accumulate on top
      const float s0 = ldexpf(1.0f, e0 - em);
#pragma unroll
      for (int m = 0; m < NT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[m][i] = (acc[m][i] - cr) * s0;
    }
  }
  if (kOdLds || !(e[0] > a[0])) {
#pragma unroll
    for (int m = 0; m < NT; ++m) acc[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  const float tm = ldexpf(1.0f, -em);
  if (nz[1]) {
    if (!(kChain && nz[0])) p2_load<D, GB, 1>(c, sm, first[1], hk, e[1], a[1], t1);
    phase2<D, GB, 1>(c, sm, first[1], hk, a[1], e[1], off[1], ncol, tm, acc, lp, zp, cp, t1, [&] {
      if (kChain && nz[2]) p2_load<D, GB, 2>(c, sm, first[2], hk, e[2], a[2], t2);
    });
  }
  __builtin_amdgcn_s_setprio(0);
  if (nz[2]) {
    if (!(kChain && nz[1])) p2_load<D, GB, 2>(c, sm, first[2], hk, e[2], a[2], t2);
    phase2<D, GB, 2>(c, sm, first[2], hk, a[2], e[2], off[2], ncol, tm, acc, lp, zp, cp, t2, [&] {
      if (kChain && nz[3]) p2_load<D, GB, 3>(c, sm, first[3], hk, e[3], a[3], t3);
    });
  }
  if (nz[3]) {
    if (!(kChain && nz[2])) p2_load<D, GB, 3>(c, sm, first[3], hk, e[3], a[3], t3);
    phase2<D, GB, 3>(c, sm, first[3], hk, a[3], e[3], off[3], ncol, tm, acc, lp, zp, cp, t3, [] {});
  }
  wave_lds_sync();

  // epilogue: lane (column r, group g) holds channels 16 m + 4 g + i of column r
  float lsum = 0.0f, zsum = 0.0f, corr = 0.0f;
#pragma unroll
  for (int n = 0; n < GB; ++n) {
    const float ls = wave_sum(lp[n]), zs = wave_sum(zp[n]), cs = wave_sum(cp[n]);
    if (r == n) {
      lsum = ls;
      zsum = zs;
      corr = cs;
    }
  }
  const bool own = r < ncol && (((fullm | locm) >> r) & 1);
  const int64_t orow = row0 + r;
  if (own) {
    const float sM = ldexpf(1.0f, em);
    const float mx = sm.cmax[r];
    float o[NT][4];
#pragma unroll
    for (int m = 0; m < NT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[m][i] = (acc[m][i] - corr) * sM + (kOdLds ? sm.od[r][16 * m + 4 * g + i] : 0.0f) + zsum;
    if (nch == 1) {
      const float inv = 1.0f / lsum;
#pragma unroll
      for (int m = 0; m < NT; ++m) {
        uint2 w;
        w.x = (uint32_t)tr_f32_to_bf16(o[m][0] * inv) | ((uint32_t)tr_f32_to_bf16(o[m][1] * inv) << 16);
        w.y = (uint32_t)tr_f32_to_bf16(o[m][2] * inv) | ((uint32_t)tr_f32_to_bf16(o[m][3] * inv) << 16);
        *reinterpret_cast<uint2*>(out + orow * D + 16 * m + 4 * g) = w;
      }
    } else if (GB == 1 && cnt) {
      // the chunk's record (o[D], m, l), agent-coherent: a wave of this launch merges it
      const __amdgpu_buffer_rsrc_t rs = rec_rsrc(part + orow * stride * (D + 2), (uint32_t)(stride * (D + 2) * 4));
      const int rec = k * (D + 2) * 4;
#pragma unroll
      for (int m = 0; m < NT; ++m) {
        const u32x4 w = {__float_as_uint(o[m][0]), __float_as_uint(o[m][1]), __float_as_uint(o[m][2]),
                         __float_as_uint(o[m][3])};
        __builtin_amdgcn_raw_buffer_store_b128(w, rs, rec + 4 * (16 * m + 4 * g), 0, kSc1);
      }
      if (g == 0) {
        const u32x2 w = {__float_as_uint(mx), __float_as_uint(lsum)};
        __builtin_amdgcn_raw_buffer_store_b64(w, rs, rec + 4 * D, 0, kSc1);
      }
    } else {
      // the chunk's record, merged by k_decode_combine
      float* dst = part + (orow * stride + k) * (D + 2);
#pragma unroll
      for (int m = 0; m < NT; ++m)
        *reinterpret_cast<float4*>(dst + 16 * m + 4 * g) = make_float4(o[m][0], o[m][1], o[m][2], o[m][3]);
      if (g == 0) {
        dst[D] = mx;
        dst[D + 1] = lsum;
      }
    }
  }
  if (nch == 1 || !cnt) return;
  // With one column per item, the wave that completes a group's last chunk merges the group's
  // records itself: each wave's records are performed at agent scope before it counts its chunk
  // in the group's counter, and the wave that brings the count to nch reads them all back with
  // agent-coherent loads and returns the counter to zero for the next call.  (Blocks of query
  // heads merge in a launch of their own: one wave merging a block's columns one after another
  // ended the launch later than that launch takes.)
  if constexpr (GB == 1) {
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    int prev = 0;
    if (lane == 0) prev = __hip_atomic_fetch_add(cnt + grp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev != nch - 1) return;
    if (lane == 0) __hip_atomic_store(cnt + grp, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    merge_records<D>(rec_rsrc(part + row0 * stride * (D + 2), (uint32_t)(stride * (D + 2) * 4)), nch, out + row0 * D);
  }
}

// Log-sum-exp merge of the chunks of windows that span more than one chunk: one workgroup per
// (seq, query head), thread d = channel d.  The chunks are those of the union window of the
// head's block of query heads (a chunk outside the head's own window carries max -inf, weight 0).
// Chunks go in batches of 32: every load of a batch -- the channel's 32 partial values and, in
// lane k of each wave, chunk k's (max, sum) -- is issued at once (indices clamped into the window),
// then the batch folds into a running (max, num, den) with the chunk weights broadcast from their
// lanes.
template <int D>
__global__ __launch_bounds__(D) void k_decode_combine(int t, int window, int CH, int stride,
                                                      const uint8_t* __restrict__ mode, const float* __restrict__ part,
                                                      uint16_t* __restrict__ out, int HQ, int G, int GB) {
  constexpr int KB = kMergeBatch;
  const int sh = blockIdx.x;
  const int d = threadIdx.x, lane = d & 63;
  const int m = mode[sh];
  if (m != TR_MODE_LOCAL && m != TR_MODE_FULL) return;
  // the union window of the head's block
  const int hq = sh % HQ;
  const int b0 = (hq / G) * G + ((hq % G) / GB) * GB;
  const int nb = min(GB, (hq / G) * G + G - b0);
  bool anyfull = false;
  for (int n = 0; n < nb; ++n) anyfull |= mode[sh - hq + b0 + n] == TR_MODE_FULL;
  const int lo = anyfull ? 0 : max(0, t - window);
  const int L = t + 1 - lo;
  const int nch = (L + CH - 1) / CH;
  if (nch == 1) return;                            // written by k_decode
  const float* base = part + (int64_t)sh * stride * (D + 2);
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
    const float wk = (own && mk != -INFINITY) ? exp2f(mk - Mn) : 0.0f;
    den = den * a + wave_sum(wk * lk);
    float nb2 = 0.0f;
#pragma unroll
    for (int x = 0; x < KB; ++x)
      nb2 = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk), x)), v[x], nb2);
    num = num * a + nb2;
    M = Mn;
  }
  out[(int64_t)sh * D + d] = tr_f32_to_bf16(num / den);
}

// Columns per item: the query heads of one KV head, up to 4 per item.
int block_cols(int G) { return G == 1 ? 1 : 4; }

// Waves of k_decode<D, GB> the device holds at once (occupancy x compute units), per device; 0 if
// the runtime cannot tell.
template <int D, int GB>
int resident_waves() {
  static std::mutex mu;
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (!cache[dev]) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(&k_decode<D, GB>), kWave,
                                                     0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || per_cu < 1 ||
        cus < 1) {
      (void)hipGetLastError();
      return 0;
    }
    cache[dev] = per_cu * cus;
  }
  return cache[dev];
}

// Chunks per window for a decode over n positions with room for `limit` partial records per
// (seq, query head).  The kernel dispatches the items that read the cache first, so the count
// aims at as many items as the chip holds waves at once if every group were full (fewer, longer
// items when the groups alone fill it), but no chunk below kMinChunk positions and none above
// the work item's limits, and no more merge batches (kMergeBatch records each, one round trip
// apiece at the end of the window's last chunk) than the fewest chunks need: on a 65537-position
// window of 16 heads, 256 chunks took 65 us per launch and 128 took 47.  0 if `limit` cannot
// hold the chunks a full window needs.
int decode_chunks(const tr_kv_cache* c, int n, int limit) {
  const int GB = block_cols(c->grp);
  const int NB = (c->grp + GB - 1) / GB;
  const int items = c->lay.B * c->lay.H * NB;       // (seq, KV head, block) groups
  int max_ch = tr_decode_max_chunk(c->lay);
  const int cap = GB == 1 ? chunk_cap<1>() : chunk_cap<4>();
  if (max_ch > cap) max_ch = cap;
  const int need = (n + max_ch - 1) / max_ch;      // fewest chunks a full window allows
  int waves = c->lay.D == 64 ? (GB == 1 ? resident_waves<64, 1>() : resident_waves<64, 4>())
                             : (GB == 1 ? resident_waves<128, 1>() : resident_waves<128, 4>());
  if (waves < 1) waves = 4096;
  int nch = waves / items;
  if (nch > (n + kMinChunk - 1) / kMinChunk) nch = (n + kMinChunk - 1) / kMinChunk;
  if (nch < need) nch = need;
  const int by_merge = (need + kMergeBatch - 1) / kMergeBatch * kMergeBatch;
  if (nch > by_merge) nch = by_merge;
  if (nch > limit) nch = limit;
  if (nch < 1) nch = 1;
  if (c->force_chunks > 0) nch = c->force_chunks < n ? c->force_chunks : n;
  const int CH = (n + nch - 1) / nch;
  return (CH > max_ch || nch > limit) ? 0 : nch;
}

// The decode kernels with the split-K partial results in `part` (records of D + 2 floats,
// `stride` records per (seq, query head)).
// With one column per item and a counter per (seq, KV head) in `cnt` (zero on entry, left zero),
// k_decode merges the chunks itself; otherwise (blocks of query heads, or no counters) the merge is
// a launch of its own.
tr_status decode_run(tr_kv_cache* c, int layer, const uint16_t* q, const uint8_t* mode, int window, uint16_t* out,
                     int nch, float* part, int stride, int32_t* cnt, bool prof_ok, hipStream_t stream) {
  const CacheLayout& L = c->lay;
  const int t = c->len[layer] - 1;
  const int n = t + 1;
  const int G = c->grp;
  const int GB = block_cols(G);
  const int NB = (G + GB - 1) / GB;
  const int BH = L.B * c->hq;                       // (seq, query head) pairs
  const int CH = (n + nch - 1) / nch;
  const float kscale = (float)(1.4426950408889634 / sqrt((double)L.D));
  const int grid = L.B * L.H * NB * nch;
  if (GB != 1) cnt = nullptr;
  const bool prof_was = c->prof_on;
  c->prof_on = prof_was && prof_ok;
  tr_status st = TR_OK;
  {
    TrProfScope prof(c, TR_PROF_DECODE_SPLIT, stream);
#define TR_DECODE_LAUNCH(DD, GG)                                                                             \
  hipLaunchKernelGGL((k_decode<DD, GG>), dim3(grid), dim3(kWave), 0, stream, L, layer, t, window, CH, stride, \
                     kscale, q, mode, part, out, c->hq, G, NB, cnt)
    if (L.D == 64) {
      if (GB == 1) TR_DECODE_LAUNCH(64, 1);
      else TR_DECODE_LAUNCH(64, 4);
    } else {
      if (GB == 1) TR_DECODE_LAUNCH(128, 1);
      else TR_DECODE_LAUNCH(128, 4);
    }
#undef TR_DECODE_LAUNCH
    if (hipGetLastError() != hipSuccess) st = TR_ERR_HIP;
  }
  if (st == TR_OK && nch > 1 && !cnt) {
    TrProfScope prof(c, TR_PROF_DECODE_COMBINE, stream);
    if (L.D == 64)
      hipLaunchKernelGGL(k_decode_combine<64>, dim3(BH), dim3(64), 0, stream, t, window, CH, stride, mode, part, out,
                         c->hq, G, GB);
    else
      hipLaunchKernelGGL(k_decode_combine<128>, dim3(BH), dim3(128), 0, stream, t, window, CH, stride, mode, part,
                         out, c->hq, G, GB);
    if (hipGetLastError() != hipSuccess) st = TR_ERR_HIP;
  }
  c->prof_on = prof_was;
  return st;
}

}  // namespace

tr_status tr_decode_launch(tr_kv_cache* c, int layer, const uint16_t* q, const uint8_t* mode, int window,
                           uint16_t* out, hipStream_t stream) {
  const int nch = decode_chunks(c, c->len[layer], c->max_chunks);
  if (nch < 1) return TR_ERR_UNSUPPORTED;
  return decode_run(c, layer, q, mode, window, out, nch, c->partials, c->max_chunks, c->merge_cnt, true, stream);
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
  const int nch = decode_chunks(c, c->len[layer], (int)(limit < (1 << 20) ? limit : (1 << 20)));
  if (nch < 1) return TR_ERR_SCRATCH;
  // every chunk writes its own record before the merge reads it, which here is always a launch of
  // its own (an in-kernel merge would need counters that start at zero): nothing needs clearing
  return decode_run(c, layer, q, mode, window, out, nch, part, nch, nullptr, false, stream);
}
