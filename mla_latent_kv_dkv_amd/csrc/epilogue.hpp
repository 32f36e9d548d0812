// Output stage shared by the projection GEMM kernels: plain stores, the
// RoPE'd query split (absorbed query) and the RoPE'd latent-row scatter into
// the paged pool (latent append).
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace mla {

// Element i of an activation that is fp32 or the storage type T.
template <typename T>
__device__ __forceinline__ float ld_act(const void* p, int64_t i, int f32) {
  return f32 ? static_cast<const float*>(p)[i] : ld(static_cast<const T*>(p) + i);
}
template <typename T>
__device__ __forceinline__ void st_act(void* p, int64_t i, float v, int f32) {
  if (f32) static_cast<float*>(p)[i] = v; else st(static_cast<T*>(p) + i, v);
}

// Latent-append columns (n even) of row m: [c | RoPE(k^R, row_pos[m])] into
// the pool slot of (row_seq[m], row_pos[m]); pool, c/k^R split given.
template <typename T>
__device__ __forceinline__ void append_pair(const GemmArgs& a, void* pool, int split, int m, int n,
                                            float v0, float v1) {
  const int seq = a.row_seq[m];
  const int pos = a.pos[m];
  if (seq < 0 || seq >= a.n_seqs) { if (n == 0) set_err(a.err, ERR_SEQ); return; }
  if (pos < 0 || pos >= a.max_pages * a.page_size) { if (n == 0) set_err(a.err, ERR_POS); return; }
  const int page = a.block_table[static_cast<int64_t>(seq) * a.max_pages + pos / a.page_size];
  if (page < 0 || page >= a.num_pages) { if (n == 0) set_err(a.err, ERR_PAGE); return; }
  T* row = static_cast<T*>(pool) +
           (static_cast<int64_t>(page) * a.page_size + pos % a.page_size) * a.row_width;
  if (n < split) {
    st(row + n, v0);
    st(row + n + 1, v1);
  } else {
    const int k = (n - split) >> 1;
    float c, s;
    rope_cs(pos, k, a.d_rope, a.log_base, &c, &s);
    st(row + n, v0 * c - v1 * s);
    st(row + n + 1, v0 * s + v1 * c);
  }
}

template <typename T>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& a, int z, int m, int n, float v0,
                                              float v1) {
  // columns n, n+1 (n even): a pair that never straddles n_split (n_split is even)
  if (a.epi == EPI_STORE) {
    const int64_t base = z * a.y_bs + static_cast<int64_t>(m) * a.ldy;
    if (n < a.N) st_act<T>(a.y, base + n, v0, a.y_f32);
    if (n + 1 < a.N) st_act<T>(a.y, base + n + 1, v1, a.y_f32);
    return;
  }
  if (a.epi == EPI_QPROJ_APPEND && n >= a.n_append) {
    append_pair<T>(a, a.y3, a.n_split3, m, n - a.n_append, v0, v1);
    return;
  }
  if (a.epi == EPI_QPROJ || a.epi == EPI_QPROJ_APPEND) {
    if (n < a.n_split) {
      T* y = static_cast<T*>(a.y) + static_cast<int64_t>(m) * a.ldy;
      st(y + n, v0);
      st(y + n + 1, v1);
    } else {
      const int r = n - a.n_split;              // column within q_pe row
      const int k = (r % a.d_rope) >> 1;       // pair index within the head
      float c, s;
      rope_cs(a.pos[m], k, a.d_rope, a.log_base, &c, &s);
      const int qpe_w = (a.epi == EPI_QPROJ_APPEND ? a.n_append : a.N) - a.n_split;
      float* y2 = static_cast<float*>(a.y2) + static_cast<int64_t>(m) * qpe_w;
      y2[r] = v0 * c - v1 * s;
      y2[r + 1] = v0 * s + v1 * c;
    }
    return;
  }
  // EPI_APPEND
  append_pair<T>(a, a.y, a.n_split, m, n, v0, v1);
}

}  // namespace mla
