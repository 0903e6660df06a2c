// Device helpers shared by the SGA kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sga.h"

namespace sga {

// ---------------------------------------------------------------------------
// vector types used as MFMA operands
// ---------------------------------------------------------------------------
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// radix-select digits of the order-preserving score key
//   level 0: key bits 31..20 (4096 bins), level 1: 19..10, level 2: 9..0
// ---------------------------------------------------------------------------
constexpr int kHist0Bins = 4096;
constexpr int kHist0Shift = 20;
constexpr int kHist12Bins = 1024;
constexpr int kTopkChunk = 4096;  // scores per top-k scan workgroup

// fp32 score -> uint32 key whose unsigned order is the numeric order of the
// scores; -0.0 maps to the key of +0.0, and every NaN (either sign, any
// payload) to the one top key, above +inf.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0xFFFFFFFFu;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// sequence metadata
// ---------------------------------------------------------------------------
struct SeqMeta {
  const int32_t *q_seq;
  const int32_t *q_pos;
  const int64_t *kv_start;
  const int32_t *kv_len;
  int32_t num_seqs;
  int32_t max_kv_len;
  int64_t num_kv_rows;
  // paged layout (page_shift > 0): position s of sequence b is row
  // block_table[b * max_pages + (s >> page_shift)] << page_shift | s & mask
  const int32_t *block_table;
  int32_t page_shift;  // 0: contiguous rows from kv_start
  int32_t max_pages;
};

// Cached length of sequence b clipped to the buffers (0 for a bad b). In the
// contiguous layout *start is its first row; in the paged layout it is 0.
__device__ __forceinline__ int32_t seq_len_clipped(const SeqMeta &m, int32_t b, int64_t *start) {
  if (b < 0 || b >= m.num_seqs) {
    *start = 0;
    return 0;
  }
  int64_t len = m.kv_len[b];
  if (m.page_shift) {
    *start = 0;
    if ((m.num_kv_rows >> m.page_shift) == 0) return 0;
    const int64_t cap = (int64_t)m.max_pages << m.page_shift;
    if (len > cap) len = cap;
  } else {
    const int64_t s = m.kv_start[b];
    if (s < 0 || s > m.num_kv_rows) {
      *start = 0;
      return 0;
    }
    if (len > m.num_kv_rows - s) len = m.num_kv_rows - s;
    *start = s;
  }
  if (len > m.max_kv_len) len = m.max_kv_len;
  if (len < 0) len = 0;
  return (int32_t)len;
}

// Candidate count n_t of query t (positions 0..q_pos that are cached).
__device__ __forceinline__ int32_t query_candidates(const SeqMeta &m, int32_t t, int64_t *start) {
  int32_t L = seq_len_clipped(m, m.q_seq[t], start);
  int64_t n = (int64_t)m.q_pos[t] + 1;
  if (n > L) n = L;
  if (n < 0) n = 0;
  return (int32_t)n;
}

// A page id as the kernels use it: ids outside the cache read page 0.
__device__ __forceinline__ int64_t checked_page(const SeqMeta &m, int32_t pg) {
  return (pg < 0 || (int64_t)pg >= (m.num_kv_rows >> m.page_shift)) ? 0 : pg;
}

// Cache row of position s (0 <= s < the clipped length) of sequence b; start
// comes from seq_len_clipped.
__device__ __forceinline__ int64_t kv_row(const SeqMeta &m, int32_t b, int64_t start, int32_t s) {
  if (!m.page_shift) return start + s;
  const int32_t pg = m.block_table[(int64_t)b * m.max_pages + (s >> m.page_shift)];
  return (checked_page(m, pg) << m.page_shift) | (s & ((1 << m.page_shift) - 1));
}

// The pages under a workgroup's key range, for kernels that copy 64-key
// tiles: lane l of ids[v] holds the checked page id of page first + 64 v + l
// of sequence b (pages at or past the sequence's last page read as 0). Pages
// hold at least 64 keys, so a tile that starts at a multiple of 64 lies in
// one page, and row() of its first key gives the tile's first row.
template <int kV>
struct PageWindow {
  int32_t ids[kV];
  int32_t first;

  __device__ __forceinline__ void load(const SeqMeta &m, int32_t b, int32_t key0, int32_t n) {
    first = key0 >> m.page_shift;
    const int32_t npages = n > 0 ? ((n - 1) >> m.page_shift) + 1 : 0;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int v = 0; v < kV; ++v) {
      const int32_t pg = first + 64 * v + lane;
      ids[v] = pg < npages ? (int32_t)checked_page(m, m.block_table[(int64_t)b * m.max_pages + pg]) : 0;
    }
  }
  // row of key (wave-uniform), which lies inside the window; keys outside
  // it read a row of page 0
  __device__ __forceinline__ int64_t row(const SeqMeta &m, int32_t key) const {
    const int rel = __builtin_amdgcn_readfirstlane((key >> m.page_shift) - first);
    int32_t id = 0;
#pragma unroll
    for (int v = 0; v < kV; ++v)
      if ((rel >> 6) == v) id = __builtin_amdgcn_readlane(ids[v], rel & 63);
    return ((int64_t)id << m.page_shift) | (key & ((1 << m.page_shift) - 1));
  }
};

// ---------------------------------------------------------------------------
// number formats
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);                                // round to nearest even
  return u >> 16;
}

// OCP E4M3FN byte -> fp32 (exact).
__device__ __forceinline__ float e4m3fn_to_f32(uint32_t code) {
  uint32_t e = (code >> 3) & 0xFu;
  uint32_t m = code & 0x7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  if ((code & 0x7fu) == 0x7fu) v = __builtin_nanf("");
  return (code & 0x80u) ? -v : v;
}

// E8M0 scale byte -> fp32 2^(e-127) (NaN for 0xFF).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  if (e == 255u) return __builtin_nanf("");
  if (e == 0u) return 0x1p-127f;
  return __uint_as_float(e << 23);
}

__device__ __forceinline__ float load_as_f32(const void *p, int dtype, size_t i) {
  if (dtype == SGA_BF16) return bf16_bits_to_f32(((const uint16_t *)p)[i]);
  return ((const float *)p)[i];
}

__device__ __forceinline__ void store_from_f32(void *p, int dtype, size_t i, float v) {
  if (dtype == SGA_BF16)
    ((uint16_t *)p)[i] = (uint16_t)f32_to_bf16_bits(v);
  else
    ((float *)p)[i] = v;
}

__device__ __forceinline__ float sigmoidf_exact_ends(float g) {
  // 1 / (1 + e^-g): +inf -> 1 exactly, -inf -> 0 exactly
  return 1.0f / (1.0f + __expf(-g));
}

// ---------------------------------------------------------------------------
// prefix sums
// ---------------------------------------------------------------------------
// Inclusive prefix sum over the 64 lanes of a wave: shifts within each row of
// 16 lanes (DPP row_shr 1, 2, 4, 8), then the row totals carried with the
// gfx9 row broadcasts (lane 15 into rows 1 and 3, lane 31 into rows 2 and 3).
// Lanes a DPP move has no source for add 0.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Block-wide exclusive scan of one uint32 per thread (blockDim a multiple of
// 64, at most 1024); *total receives the block sum. `scratch` needs
// blockDim / 64 words of LDS. Two barriers; the second lets the caller reuse
// `scratch` right away.
// Workgroup barrier for threads that communicate through LDS only: it waits
// for this wave's LDS operations, not for its outstanding global loads (a
// __syncthreads() drains those too, which stalls on loads whose results are
// not needed yet).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0) only
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// kLdsOnly: the barriers wait for LDS operations only (lds_barrier).
template <bool kLdsOnly = false>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *scratch,
                                                         uint32_t *total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const uint32_t inc = wave_inclusive_scan(v);
  if (lane == 63) scratch[wave] = inc;
  if (kLdsOnly) lds_barrier(); else __syncthreads();
  uint32_t base = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    const uint32_t x = scratch[i];
    base += i < wave ? x : 0u;
    tot += x;
  }
  *total = tot;
  if (kLdsOnly) lds_barrier(); else __syncthreads();
  return base + inc - v;
}

}  // namespace sga
