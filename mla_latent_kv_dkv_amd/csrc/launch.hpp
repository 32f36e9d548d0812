// Host-side launchers of the MLA kernels (internal to libmla.so).
// Every launcher enqueues on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace mla {

// Epilogues of the projection GEMM Y[m, n] = sum_k X(m, k) W(n, k).
enum GemmEpilogue : int {
  EPI_STORE = 0,   // y[z*y_bs + m*ldy + n]
  EPI_APPEND = 1,  // [c | RoPE(k^R, row_pos[m])] scattered into the paged pool
  EPI_QPROJ = 2,   // n < n_split -> y (q^C); n >= n_split -> RoPE per head -> y2 (q_pe)
  // EPI_QPROJ for n < n_append, and the latent append of the same rows for
  // n >= n_append: W rows from w3 (c^KV, n - n_append < n_split3) and w4 (k^R),
  // written as EPI_APPEND does into the pool y3 (or, with ld3 > 0, as fp32 rows)
  EPI_QPROJ_APPEND = 3,
};

struct GemmArgs {
  // X(m, k) = x[z*x_bs + m*ldx_m + k*ldx_k]
  const void* x;
  int64_t ldx_m, ldx_k, x_bs;
  // W(n, k) = w1[z*w_bs + n*ldw_n + k*ldw_k] for n < n_split, else the same on w2 at n - n_split
  const void* w1;
  const void* w2;
  int n_split;
  int64_t ldw_n, ldw_k, w_bs;
  int M, N, K, batch;
  int epi;
  int x_f32;        // X is fp32 (else the storage dtype of W)
  int y_f32;        // EPI_STORE output / EPI_QPROJ's q^C is fp32 (else the storage dtype)
  void* y;
  int64_t ldy, y_bs;
  void* y2;         // EPI_QPROJ: q_pe [M, N - n_split], fp32
  int d_rope;       // EPI_APPEND / EPI_QPROJ: rope width (pairs restart every d_rope columns)
  RopeSpec rope;    // RoPE frequencies (EPI_APPEND / EPI_QPROJ)
  float* rope_tab;  // optional cos/sin of the rows' RoPE angles, [M][d_rope/2][2] (else computed)
  const int32_t* pos;      // EPI_APPEND: row_pos; EPI_QPROJ: decode positions
  const int32_t* row_seq;  // EPI_APPEND
  const int32_t* block_table;
  int n_seqs, max_pages, page_size, row_width;
  int64_t num_pages;
  int* err;
  // EPI_QPROJ_APPEND only
  const void* w3;
  const void* w4;
  int n_append, n_split3;
  void* y3;
  // 0: the append columns go into the pool y3 as EPI_APPEND writes them; > 0:
  // they stay fp32 and unrotated, row m at y3 + m * ld3 (the rows an FP8 pool's
  // quantizer rotates, scales and scatters)
  int64_t ld3;
  // columns the weight stream's K-slice plan counts (0: N).  The query projection
  // counts the latent-append columns as well, so that it takes the slices of the
  // fused query/append product and gives the same queries bit for bit.
  int plan_cols;
};

hipError_t launch_gemm_generic(const GemmArgs& a, bool bf16, hipStream_t stream);

struct AttnArgs {
  const float* q_lat;   // [batch, n_h, d_c]
  const float* q_pe;    // [batch, n_h, d_R]
  const void* pool;
  int64_t num_pages;
  const int32_t* block_table;
  int max_pages;
  const int32_t* seq_lens;
  int batch, num_splits, n_heads, d_latent, d_rope, page_size;
  float scale;
  float* o_part;
  float* lse_part;
  int* err;
  // prefill: unit b is query token b at position q_pos[b] of sequence q_seq[b]
  // (block-table row q_seq[b], attended length q_pos[b] + 1); null for decode,
  // where unit b is sequence b with length seq_lens[b]
  const int32_t* q_seq;
  const int32_t* q_pos;
  int n_seqs;
  // work units: batch * num_splits uniform splits (plan null), or the entries
  // (b, t0, t1) of a length-proportional plan (decode only); partials of unit u
  // at head rows u * n_heads ..
  const int32_t* plan;
  int units;
};

// Work unit u: query row b, block-table row sq and token range [t0, t1).
// Uniform splits: split u mod S of query row u / S (split_range).  Plan: entry
// (b, t0, t1), checked against the batch and the table's length; a bad entry
// sets ERR_POS (when `flag`) and gives an empty range.
__device__ __forceinline__ void attn_unit(const AttnArgs& a, int u, bool flag, int* b, int* sq,
                                          int* t0, int* t1) {
  if (a.plan) {
    const int pb = a.plan[3 * u], p0 = a.plan[3 * u + 1], p1 = a.plan[3 * u + 2];
    if (pb < 0 || pb >= a.batch || p0 < 0 || p0 > p1 || p1 > a.max_pages * a.page_size) {
      if (flag) set_err(a.err, ERR_POS);
      *b = 0; *sq = 0; *t0 = 0; *t1 = 0;
    } else {
      *b = pb; *sq = pb; *t0 = p0; *t1 = p1;
    }
    return;
  }
  const int S = a.num_splits;
  *b = u / S;
  int L;
  unit_seq_len(a.seq_lens, a.q_seq, a.q_pos, a.n_seqs, a.max_pages * a.page_size, *b, flag, a.err,
               sq, &L);
  split_range(L, S, u - *b * S, a.page_size, t0, t1);
}

hipError_t launch_attention_generic(const AttnArgs& a, bool bf16, hipStream_t stream);
// FP8 pool: pages of page_size rows [d_c e4m3 | d_R bf16], then page_size fp32 row scales
hipError_t launch_attention_generic_fp8(const AttnArgs& a, hipStream_t stream);

// FP8 latent pool: quantize fp32 rows [n_rows, d_c + d_R] into their page slots.
struct QuantArgs {
  const float* rows;
  int64_t ld_rows;
  int n_rows, d_latent, d_rope;
  int rope;                 // rotate the k^R part at row_pos (rows straight from the projection)
  RopeSpec rs;
  const int32_t* row_seq;
  const int32_t* row_pos;
  const int32_t* block_table;
  int n_seqs, max_pages, page_size;
  int64_t num_pages, page_bytes, row_bytes;
  uint8_t* pool;
  int* err;
};

hipError_t launch_quantize_rows(const QuantArgs& a, hipStream_t stream);

struct MergeArgs {
  const float* o_part;
  const float* lse_part;
  int batch, num_splits, n_heads, d_latent;
  float* o_lat;
  float* lse;
  // plan: the partials of row b are units unit_start[b] .. unit_start[b+1]-1 of
  // `units` (else b * num_splits .. + num_splits - 1); a bad range sets ERR_POS
  const int32_t* unit_start;
  int units;
  int* err;
  // when set, k_merge_rows writes the merged rows here as bf16 (round to nearest
  // even, the W_UV product's input precision) instead of fp32 to o_lat
  void* o_lat_bf16;
};

// Partials of merge row b: first unit and count.
__device__ __forceinline__ void merge_units(const MergeArgs& a, int b, bool flag, int* first,
                                            int* count) {
  if (!a.unit_start) {
    *first = b * a.num_splits;
    *count = a.num_splits;
    return;
  }
  const int f = a.unit_start[b], e = a.unit_start[b + 1];
  if (f < 0 || f > e || e > a.units) {
    if (flag && a.err) set_err(a.err, ERR_POS);
    *first = 0;
    *count = 0;
    return;
  }
  *first = f;
  *count = e - f;
}

hipError_t launch_merge_generic(const MergeArgs& a, bool bf16, hipStream_t stream);

}  // namespace mla
