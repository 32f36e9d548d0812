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

// cos/sin of the RoPE angle (pos, pair k) of output row m: from the table when
// the caller computed one, else evaluated here.
__device__ __forceinline__ void rope_row(const GemmArgs& a, int m, int pos, int k, float* c,
                                         float* s) {
  if (a.rope_tab) {
    const float2 t = *reinterpret_cast<const float2*>(a.rope_tab + 2 * (m * (a.d_rope / 2) + k));
    *c = t.x;
    *s = t.y;
  } else {
    rope_cs(pos, k, a.d_rope, a.rope, c, s);
  }
}

// Element offset of the pool row that appended row m goes to, the slot of
// (row_seq[m], row_pos[m]), or -1 when its sequence, position or page is out of
// range (flagged in the error word when `flag`).
__device__ __forceinline__ int64_t append_row_offset(const GemmArgs& a, int m, bool flag) {
  const int seq = a.row_seq[m];
  const int pos = a.pos[m];
  if (seq < 0 || seq >= a.n_seqs) { if (flag) set_err(a.err, ERR_SEQ); return -1; }
  if (pos < 0 || pos >= a.max_pages * a.page_size) { if (flag) set_err(a.err, ERR_POS); return -1; }
  const int page = a.block_table[static_cast<int64_t>(seq) * a.max_pages + pos / a.page_size];
  if (page < 0 || page >= a.num_pages) { if (flag) set_err(a.err, ERR_PAGE); return -1; }
  return (static_cast<int64_t>(page) * a.page_size + pos % a.page_size) * a.row_width;
}

// Latent-append columns n, n+1 (n even) of row m, at position pos, into the pool
// row at element offset `off` (nothing when off < 0): [c | RoPE(k^R, pos)];
// pool, c/k^R split given.
template <typename T>
__device__ __forceinline__ void append_pair_at(const GemmArgs& a, void* pool, int split,
                                               int64_t off, int m, int pos, int n, float v0,
                                               float v1) {
  if (off < 0) return;
  T* row = static_cast<T*>(pool) + off;
  if (n < split) {
    st(row + n, v0);
    st(row + n + 1, v1);
  } else {
    const int k = (n - split) >> 1;
    float c, s;
    rope_row(a, m, pos, k, &c, &s);
    st(row + n, v0 * c - v1 * s);
    st(row + n + 1, v0 * s + v1 * c);
  }
}

// Latent-append columns (n even) of row m: [c | RoPE(k^R, row_pos[m])] into
// the pool slot of (row_seq[m], row_pos[m]); pool, c/k^R split given.
template <typename T>
__device__ __forceinline__ void append_pair(const GemmArgs& a, void* pool, int split, int m, int n,
                                            float v0, float v1) {
  const int64_t off = append_row_offset(a, m, n == 0);
  if (off >= 0) append_pair_at<T>(a, pool, split, off, m, a.pos[m], n, v0, v1);
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
    if (a.ld3 > 0) {   // fp32 rows for a quantizer
      float* r = static_cast<float*>(a.y3) + m * a.ld3 + (n - a.n_append);
      r[0] = v0;
      r[1] = v1;
    } else {
      append_pair<T>(a, a.y3, a.n_split3, m, n - a.n_append, v0, v1);
    }
    return;
  }
  if (a.epi == EPI_QPROJ || a.epi == EPI_QPROJ_APPEND) {
    if (n < a.n_split) {   // q^C: fp32 (y_f32) or the storage type
      const int64_t base = static_cast<int64_t>(m) * a.ldy;
      st_act<T>(a.y, base + n, v0, a.y_f32);
      st_act<T>(a.y, base + n + 1, v1, a.y_f32);
    } else {
      const int r = n - a.n_split;              // column within q_pe row
      const int k = (r % a.d_rope) >> 1;       // pair index within the head
      float c, s;
      rope_row(a, m, a.pos[m], k, &c, &s);
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

// Columns n .. n+3 of row m (n a multiple of 4): one 16-byte store for an fp32
// plain output, for q^C and for q_pe when the four columns lie in one region and
// the destination is 16-byte aligned; the pair stages otherwise.
template <typename T>
__device__ __forceinline__ void gemm_epilogue4(const GemmArgs& a, int z, int m, int n, float4 v) {
  auto aligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  if (a.epi == EPI_STORE && a.y_f32 && n + 3 < a.N) {
    float* y = static_cast<float*>(a.y) + z * a.y_bs + static_cast<int64_t>(m) * a.ldy + n;
    if (aligned(y)) {
      *reinterpret_cast<float4*>(y) = v;
      return;
    }
  }
  const bool qproj = a.epi == EPI_QPROJ || a.epi == EPI_QPROJ_APPEND;
  const int n_q = a.epi == EPI_QPROJ_APPEND ? a.n_append : a.N;   // end of the query columns
  if (a.epi == EPI_QPROJ_APPEND && a.ld3 > 0 && n >= a.n_append && n + 3 < a.N) {
    float* r = static_cast<float*>(a.y3) + m * a.ld3 + (n - a.n_append);
    if (aligned(r)) {
      *reinterpret_cast<float4*>(r) = v;
      return;
    }
  }
  if (qproj && a.y_f32 && n + 3 < a.n_split) {
    float* y = static_cast<float*>(a.y) + static_cast<int64_t>(m) * a.ldy + n;
    if (aligned(y)) {
      *reinterpret_cast<float4*>(y) = v;
      return;
    }
  }
  if (qproj && n >= a.n_split && n + 3 < n_q && (a.d_rope & 3) == 0) {
    const int r = n - a.n_split;   // two pairs of one head
    const int k = (r % a.d_rope) >> 1;
    float* y2 = static_cast<float*>(a.y2) + static_cast<int64_t>(m) * (n_q - a.n_split) + r;
    if (aligned(y2)) {
      float c0, s0, c1, s1;
      rope_row(a, m, a.pos[m], k, &c0, &s0);
      rope_row(a, m, a.pos[m], k + 1, &c1, &s1);
      *reinterpret_cast<float4*>(y2) = make_float4(v.x * c0 - v.y * s0, v.x * s0 + v.y * c0,
                                                   v.z * c1 - v.w * s1, v.z * s1 + v.w * c1);
      return;
    }
  }
  gemm_epilogue<T>(a, z, m, n, v.x, v.y);
  gemm_epilogue<T>(a, z, m, n + 2, v.z, v.w);
}

}  // namespace mla
