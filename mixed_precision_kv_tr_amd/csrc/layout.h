// Paged mixed-width KV cache layout, shared by the host code and the gfx950 kernels.
//
// TriRoute (xllm-io.github.io review page) stores each token's K/V at the width b its
// controller chose (Eq. 4) and keeps inference compatible with KV paging (the paragraph after
// Algorithm 1); the pages give no layout.  This one segregates tokens by width class:
//
//   class c = 0, 1, 2, 3  <->  b = 2, 4, 8, 16
//
//   per (layer, sequence, class): a stream of slots 0, 1, 2, ... in position order, held in
//   pages of one shared pool.  A page of class c holds P_c = page_code_bytes * 8 / (D * b)
//   tokens of all H heads:
//     [pos   : int32  P_c               ]  absolute position of each slot
//     [K     : H x page_code_bytes      ]  head h: P_c rows of D*b/8 bytes (codes or bf16)
//     [V     : H x page_code_bytes      ]
//     [sideK : H x P_c x float2 (s, z)  ]  b < 16 only
//     [sideV : H x P_c x float2 (s, z)  ]
//   every region 256-byte aligned; all classes share one page size (the largest).
//
//   prefix[layer][seq][p][c] = tokens of class c among positions < p (int32), so the slot of
//   position p is prefix[p][class(p)] and a position window [lo, hi) maps to the contiguous
//   slot range [prefix[lo][c], prefix[hi][c]) of every class.
//
//   codes: element e of a group sits at bits [e*b, e*b + b) of the row (little-endian).
#pragma once

#include <stdint.h>

#define TR_NCLASS 4
#define TR_ERRF_BAD_BITS 1u
#define TR_ERRF_BAD_MODE 2u
#define TR_ERRF_NO_PAGES 4u
#define TR_ERRF_RANGE 8u                // prefill: a stored V value outside fp16's range

struct CacheLayout {
  int32_t L, B, H, D, N;          // layers, batch, heads, head_dim, max_tokens
  int32_t pfN;                    // positions a prefill call may reach (0: no prefill scratch);
                                  // also the stride of the prefill row lists
  int32_t cb;                     // code bytes per head per page (K or V)
  int32_t page_bytes;
  int32_t ptok[TR_NCLASS];        // tokens per page (a power of two)
  int32_t ptok_log2[TR_NCLASS];
  int32_t rowb[TR_NCLASS];        // code bytes per (token, head): D * b / 8
  int32_t k_off[TR_NCLASS], v_off[TR_NCLASS], sk_off[TR_NCLASS], sv_off[TR_NCLASS];
  int32_t maxp[TR_NCLASS];        // page-table entries per (layer, seq, class)
  int32_t pt_off[TR_NCLASS];      // offset of class c inside a (layer, seq) page-table block
  int32_t pt_stride;              // entries per (layer, seq)
  int64_t pool_pages;
  uint8_t* pool;
  int32_t* ptab;                  // [L][B][pt_stride], -1 = no page
  int32_t* prefix;                // [L][B][N + 1][4]
  int32_t* next_page;             // bump allocator
  uint32_t* err;                  // sticky TR_ERRF_* flags
};

__host__ __device__ inline int tr_bits_of_class(int c) { return 2 << c; }

// Class of a width value; -1 if the value is not one of 2, 4, 8, 16.
__host__ __device__ inline int tr_class_of_bits(int b) {
  // b = 2^(c+1) for c in 0..3: a power of two in [2, 16] (branch-free: no compare tree on GPUs)
  const bool ok = b >= 2 && b <= 16 && (b & (b - 1)) == 0;
  return ok ? __builtin_ctz((unsigned)b) - 1 : -1;
}

__host__ __device__ inline const int32_t* tr_prefix_row(const CacheLayout& c, int layer, int seq, int p) {
  return c.prefix + (((int64_t)layer * c.B + seq) * (c.N + 1) + p) * TR_NCLASS;
}

__host__ __device__ inline int32_t* tr_ptab(const CacheLayout& c, int layer, int seq, int cls) {
  return c.ptab + ((int64_t)layer * c.B + seq) * c.pt_stride + c.pt_off[cls];
}
