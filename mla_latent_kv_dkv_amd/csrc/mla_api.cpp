// C ABI of libmla.so: argument checks, workspace layout and kernel selection.
// The operations themselves are described in include/mla.h.
#include "../../include/mla.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>
#include <atomic>
#include <cmath>
#include <cstring>

#include "launch.hpp"
#include "launch_fast.hpp"

namespace {

std::atomic<int32_t> g_path{0};

// Per-device address of the sticky error word (defined in errword.hip).
constexpr int kMaxDevices = 64;
int* g_err_ptr[kMaxDevices] = {};
std::atomic<int> g_err_ready[kMaxDevices] = {};

int* err_word() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  if (!g_err_ready[dev].load(std::memory_order_acquire)) {
    int* p = mla::error_word_address();
    if (!p) return nullptr;
    g_err_ptr[dev] = p;
    g_err_ready[dev].store(1, std::memory_order_release);
  }
  return g_err_ptr[dev];
}

// Scratch of mla_absorb_out_noalloc: one array per device, held for the life of
// the process.  In host code `scratch` names a host-side stand-in, never the
// device memory: every host use goes through the address hipGetSymbolAddress
// returns for the current device, cached per device below.
constexpr size_t kScratchBytes = size_t{32} << 20;
static __device__ __align__(256) char scratch[kScratchBytes];
void* g_scratch_ptr[kMaxDevices] = {};
std::atomic<int> g_scratch_ready[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per device),
// or nullptr when the runtime cannot say.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  if (!g_scratch_ready[dev].load(std::memory_order_acquire)) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_scratch_ptr[dev] = p;
    g_scratch_ready[dev].store(1, std::memory_order_release);
  }
  return g_scratch_ptr[dev];
}

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

mla_status check_dims(const mla_dims* d) {
  if (!d) return MLA_ERR_NULL;
  if (d->abi_version != MLA_ABI_VERSION) return MLA_ERR_UNSUPPORTED;
  if (d->dtype != MLA_F32 && d->dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  if (!is_pow2(d->page_size) || d->page_size > 1024) return MLA_ERR_UNSUPPORTED;
  if (d->hidden < 1 || d->n_heads < 1 || d->d_head < 2 || d->d_latent < 2 || d->d_rope < 2)
    return MLA_ERR_SHAPE;
  if ((d->d_head | d->d_latent | d->d_rope) & 1) return MLA_ERR_SHAPE;
  if (d->hidden > (1 << 20) || d->n_heads > 4096 || d->d_head > 4096 || d->d_latent > 4096 ||
      d->d_rope > 1024)
    return MLA_ERR_SHAPE;
  if (!(d->rope_base > 0.f) || !std::isfinite(d->rope_base)) return MLA_ERR_SHAPE;
  if (!std::isfinite(d->softmax_scale)) return MLA_ERR_SHAPE;
  if (!std::isfinite(d->rope_scale)) return MLA_ERR_SHAPE;
  if (d->rope_scale > 1.f &&
      !(d->rope_orig_len >= 1 && std::isfinite(d->yarn_alpha) && std::isfinite(d->yarn_beta) &&
        d->yarn_alpha >= 0.f && d->yarn_beta > d->yarn_alpha))
    return MLA_ERR_SHAPE;
  return MLA_OK;
}

bool yarn_on(const mla_dims* d) { return d->rope_scale > 1.f; }

// RoPE frequencies of the dims (YaRN-stretched when rope_scale > 1).
mla::RopeSpec rope_spec(const mla_dims* d) {
  mla::RopeSpec r{};
  r.log_base = std::log(static_cast<double>(d->rope_base));
  r.yarn_scale = yarn_on(d) ? static_cast<double>(d->rope_scale) : 1.0;
  r.orig_len = static_cast<double>(d->rope_orig_len);
  r.alpha = static_cast<double>(d->yarn_alpha);
  r.beta = static_cast<double>(d->yarn_beta);
  return r;
}

size_t elem_bytes(const mla_dims* d) { return d->dtype == MLA_BF16 ? 2 : 4; }

// tau: softmax_scale, or 1/sqrt(d_h + d_R); with YaRN times its logit factor
// (0.1 ln s + 1)^2
float softmax_scale(const mla_dims* d) {
  double tau = d->softmax_scale > 0.f ? d->softmax_scale
                                      : 1.0 / std::sqrt(static_cast<double>(d->d_head + d->d_rope));
  if (yarn_on(d)) {
    const double m = 0.1 * std::log(static_cast<double>(d->rope_scale)) + 1.0;
    tau *= m * m;
  }
  return static_cast<float>(tau);
}

bool use_fast() { return g_path.load(std::memory_order_relaxed) == 0; }

mla_status hip_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

// Shapes of the projection GEMMs (pointers filled in by the callers).
mla::GemmArgs qproj_args(const mla_dims* d, int batch) {
  const bool bf16 = d->dtype == MLA_BF16;
  const int64_t nhdh = static_cast<int64_t>(d->n_heads) * d->d_head;
  mla::GemmArgs a{};
  a.ldx_m = d->hidden; a.ldx_k = 1;
  a.n_split = static_cast<int>(nhdh);
  a.ldw_n = d->hidden; a.ldw_k = 1;
  a.M = batch; a.N = static_cast<int>(nhdh + static_cast<int64_t>(d->n_heads) * d->d_rope);
  a.K = d->hidden; a.batch = 1;
  // q^C is kept in fp32 for the W_UK product (which takes it as two bf16 terms)
  a.epi = mla::EPI_QPROJ; a.x_f32 = !bf16; a.y_f32 = 1;
  a.ldy = nhdh; a.d_rope = d->d_rope;
  a.rope = rope_spec(d);
  a.plan_cols = a.N + d->d_latent + d->d_rope;   // the fused product's columns
  return a;
}

// The query projection and the latent append of the same rows as one product:
// columns [q^C | q^R | c^KV | k^R] over [W_Q; W_QR; W_DKV; W_KR].
mla::GemmArgs qa_args(const mla_dims* d, int batch) {
  mla::GemmArgs a = qproj_args(d, batch);
  a.epi = mla::EPI_QPROJ_APPEND;
  a.n_append = a.N;
  a.n_split3 = d->d_latent;
  a.N += d->d_latent + d->d_rope;
  a.row_width = d->d_latent + d->d_rope;
  return a;
}

// Compressed query, first product: [c^Q | q^R] = h [W_DQ; W_QR]^T, RoPE on the
// q^R columns (the q^C split of EPI_QPROJ with n_split = d_cq); c^Q in dtype.
mla::GemmArgs cqproj_args(const mla_dims* d, int d_cq, int batch) {
  const bool bf16 = d->dtype == MLA_BF16;
  mla::GemmArgs a{};
  a.ldx_m = d->hidden; a.ldx_k = 1;
  a.n_split = d_cq;
  a.ldw_n = d->hidden; a.ldw_k = 1;
  a.M = batch; a.N = d_cq + d->n_heads * d->d_rope; a.K = d->hidden; a.batch = 1;
  a.epi = mla::EPI_QPROJ; a.x_f32 = !bf16; a.y_f32 = !bf16;
  a.ldy = d_cq; a.d_rope = d->d_rope;
  a.rope = rope_spec(d);
  return a;
}

// second product: q^C = W_UQ c^Q (c^Q in dtype, q^C in fp32 for the W_UK product)
mla::GemmArgs uq_args(const mla_dims* d, int d_cq, int batch) {
  const bool bf16 = d->dtype == MLA_BF16;
  const int64_t nhdh = static_cast<int64_t>(d->n_heads) * d->d_head;
  mla::GemmArgs a{};
  a.ldx_m = d_cq; a.ldx_k = 1;
  a.n_split = static_cast<int>(nhdh);
  a.ldw_n = d_cq; a.ldw_k = 1;
  a.M = batch; a.N = static_cast<int>(nhdh); a.K = d_cq; a.batch = 1;
  a.epi = mla::EPI_STORE; a.x_f32 = !bf16; a.y_f32 = 1;
  a.ldy = nhdh;
  return a;
}

// q_lat = W_UK^T q^C per head; q^C in fp32 (qc_f32) or the storage type
mla::GemmArgs uk_args(const mla_dims* d, int batch, bool qc_f32) {
  const int64_t nhdh = static_cast<int64_t>(d->n_heads) * d->d_head;
  mla::GemmArgs g{};
  g.ldx_m = nhdh; g.ldx_k = 1; g.x_bs = d->d_head;
  g.n_split = d->d_latent;
  g.ldw_n = 1; g.ldw_k = d->d_latent; g.w_bs = static_cast<int64_t>(d->d_head) * d->d_latent;
  g.M = batch; g.N = d->d_latent; g.K = d->d_head; g.batch = d->n_heads;
  g.epi = mla::EPI_STORE; g.x_f32 = qc_f32; g.y_f32 = 1;
  g.ldy = static_cast<int64_t>(d->n_heads) * d->d_latent; g.y_bs = d->d_latent;
  return g;
}

mla::GemmArgs uv_args(const mla_dims* d, int batch) {
  const bool bf16 = d->dtype == MLA_BF16;
  const int64_t nhdh = static_cast<int64_t>(d->n_heads) * d->d_head;
  mla::GemmArgs g{};
  g.ldx_m = static_cast<int64_t>(d->n_heads) * d->d_latent; g.ldx_k = 1; g.x_bs = d->d_latent;
  g.n_split = d->d_head;
  g.ldw_n = d->d_latent; g.ldw_k = 1; g.w_bs = static_cast<int64_t>(d->d_head) * d->d_latent;
  g.M = batch; g.N = d->d_head; g.K = d->d_latent; g.batch = d->n_heads;
  g.epi = mla::EPI_STORE; g.x_f32 = 1; g.y_f32 = !bf16;
  g.ldy = nhdh; g.y_bs = d->d_head;
  return g;
}

mla::GemmArgs oproj_args(const mla_dims* d, int batch) {
  const bool bf16 = d->dtype == MLA_BF16;
  const int64_t nhdh = static_cast<int64_t>(d->n_heads) * d->d_head;
  mla::GemmArgs a{};
  a.ldx_m = nhdh; a.ldx_k = 1;
  a.n_split = d->hidden;
  a.ldw_n = nhdh; a.ldw_k = 1;
  a.M = batch; a.N = d->hidden; a.K = static_cast<int>(nhdh); a.batch = 1;
  a.epi = mla::EPI_STORE; a.x_f32 = !bf16; a.y_f32 = 1;
  a.ldy = d->hidden;
  return a;
}

mla::GemmArgs append_args(const mla_dims* d, int n_rows) {
  const bool bf16 = d->dtype == MLA_BF16;
  mla::GemmArgs a{};
  a.ldx_m = d->hidden; a.ldx_k = 1; a.x_bs = 0;
  a.n_split = d->d_latent;
  a.ldw_n = d->hidden; a.ldw_k = 1; a.w_bs = 0;
  a.M = n_rows; a.N = d->d_latent + d->d_rope; a.K = d->hidden; a.batch = 1;
  a.epi = mla::EPI_APPEND; a.x_f32 = !bf16;
  a.d_rope = d->d_rope; a.rope = rope_spec(d);
  a.row_width = d->d_latent + d->d_rope;
  return a;
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

bool ws_aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255) == 0; }

// Bytes of the activation region (q^C, fp32, or the per-head outputs o in the
// storage type) at the front of the workspace: sized for fp32.
size_t act_bytes(const mla_dims* d, int batch) {
  return align256(static_cast<size_t>(batch) * d->n_heads * d->d_head * sizeof(float));
}

bool fast_for(const mla_dims* d, const mla::GemmArgs& a) {
  return use_fast() && d->dtype == MLA_BF16 && mla::fast_gemm_ok(a);
}

size_t partial_bytes(const mla_dims* d, const mla::GemmArgs& a) {
  return fast_for(d, a) ? align256(mla::gemm_partial_bytes(a)) : 0;
}

// Run one projection GEMM on the fast path when it applies, else the vector path.
hipError_t run_gemm(const mla_dims* d, const mla::GemmArgs& a, void* partial, size_t pbytes,
                    hipStream_t stream) {
  if (fast_for(d, a)) return mla::launch_gemm_fast(a, partial, pbytes, stream);
  return mla::launch_gemm_generic(a, d->dtype == MLA_BF16, stream);
}

bool cq_ok(int d_cq) { return d_cq >= 2 && d_cq <= 65536 && (d_cq & 1) == 0; }

size_t cq_bytes(const mla_dims* d, int d_cq, int batch) {
  return align256(static_cast<size_t>(batch) * static_cast<size_t>(d_cq) * elem_bytes(d));
}

// ---- FP8 pool: pages of page_size rows [d_c e4m3 | d_R bf16], then page_size fp32 scales
bool fp8_ok(const mla_dims* d) { return d->d_latent % 8 == 0; }

int64_t fp8_row_bytes(const mla_dims* d) { return d->d_latent + 2 * static_cast<int64_t>(d->d_rope); }

int64_t fp8_page_bytes(const mla_dims* d) {
  return static_cast<int64_t>(d->page_size) * (fp8_row_bytes(d) + 4);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// fp32 stride of the appended rows in the workspace: d_c + d_R rounded up to a
// multiple of 4, so every row starts 16-byte aligned for the quantizer's loads.
int64_t rows_ld(const mla_dims* d) { return (static_cast<int64_t>(d->d_latent) + d->d_rope + 3) / 4 * 4; }

// Projection of appended rows into fp32 [c | k^R] (k^R not yet rotated).
mla::GemmArgs append_rows_args(const mla_dims* d, int n_rows) {
  mla::GemmArgs a{};
  a.ldx_m = d->hidden; a.ldx_k = 1;
  a.n_split = d->d_latent;
  a.ldw_n = d->hidden; a.ldw_k = 1;
  a.M = n_rows; a.N = d->d_latent + d->d_rope; a.K = d->hidden; a.batch = 1;
  a.epi = mla::EPI_STORE; a.x_f32 = d->dtype != MLA_BF16; a.y_f32 = 1;
  a.ldy = rows_ld(d);
  return a;
}

size_t rows_bytes(const mla_dims* d, int n_rows) {
  return align256(static_cast<size_t>(n_rows) * static_cast<size_t>(rows_ld(d)) * sizeof(float));
}

// Appended fp32 rows [c | k^R] (k^R not yet rotated, stride rows_ld) of tokens
// (row_seq[i], row_pos[i]): RoPE on k^R, quantize, scatter into the FP8 pages.
hipError_t quantize_appended(const mla_dims* d, const float* rows, int n_rows,
                             const int32_t* row_seq, const int32_t* row_pos,
                             const int32_t* block_table, int n_seqs, int max_pages, void* pool,
                             int64_t num_pages, int* err, hipStream_t stream) {
  mla::QuantArgs q{};
  q.rows = rows; q.ld_rows = rows_ld(d); q.n_rows = n_rows;
  q.d_latent = d->d_latent; q.d_rope = d->d_rope; q.rope = 1;
  q.rs = rope_spec(d);
  q.row_seq = row_seq; q.row_pos = row_pos; q.block_table = block_table;
  q.n_seqs = n_seqs; q.max_pages = max_pages; q.page_size = d->page_size;
  q.num_pages = num_pages; q.page_bytes = fp8_page_bytes(d); q.row_bytes = fp8_row_bytes(d);
  q.pool = static_cast<uint8_t*>(pool); q.err = err;
  return mla::launch_quantize_rows(q, stream);
}

// Checks shared by the attention calls; fills `a` (pool format aside).  Decode
// units are sequences (seq_lens); prefill units are query tokens (q_seq, q_pos
// into n_seqs block-table rows).
mla_status attention_args(const mla_dims* d, bool prefill, const float* q_lat, const float* q_pe,
                          const void* pool, int64_t num_pages, const int32_t* block_table,
                          int32_t max_pages, const int32_t* seq_lens, const int32_t* q_seq,
                          const int32_t* q_pos, int32_t n_seqs, int32_t batch, int32_t num_splits,
                          float* o_part, float* lse_part, mla::AttnArgs* a) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (batch < 0 || batch > 65535 || num_splits < 1 || num_splits > 4096 || max_pages < 1 ||
      num_pages < 1)
    return MLA_ERR_SHAPE;
  if (static_cast<int64_t>(max_pages) * d->page_size > (int64_t{1} << 30)) return MLA_ERR_SHAPE;
  if (prefill && n_seqs < 1) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (!q_lat || !q_pe || !pool || !block_table || !o_part || !lse_part) return MLA_ERR_NULL;
  if (prefill ? (!q_seq || !q_pos) : !seq_lens) return MLA_ERR_NULL;
  int* err = err_word();
  if (!err) return MLA_ERR_HIP;
  *a = mla::AttnArgs{};
  a->q_lat = q_lat; a->q_pe = q_pe; a->pool = pool; a->num_pages = num_pages;
  a->block_table = block_table; a->max_pages = max_pages; a->seq_lens = prefill ? nullptr : seq_lens;
  a->batch = batch; a->num_splits = num_splits; a->n_heads = d->n_heads;
  a->d_latent = d->d_latent; a->d_rope = d->d_rope; a->page_size = d->page_size;
  a->scale = softmax_scale(d); a->o_part = o_part; a->lse_part = lse_part; a->err = err;
  a->q_seq = prefill ? q_seq : nullptr; a->q_pos = prefill ? q_pos : nullptr;
  a->n_seqs = prefill ? n_seqs : batch;
  a->units = batch * num_splits;
  return MLA_OK;
}

// Checks of the planned calls: the plan pointer and its unit count (a multiple
// of 8, as mla_decode_plan pads it).
mla_status plan_args(const int32_t* plan, int32_t n_units) {
  if (!plan) return MLA_ERR_NULL;
  if (n_units < 8 || n_units % 8 != 0 || n_units > (1 << 24)) return MLA_ERR_SHAPE;
  return MLA_OK;
}

hipError_t launch_attention_plain(const mla_dims* d, const mla::AttnArgs& a, hipStream_t stream) {
  const bool bf16 = d->dtype == MLA_BF16;
  if (use_fast() && bf16 && (mla::fast_attention_ok(a) || mla::fast_attention_h16_ok(a)))
    return mla::launch_attention_fast(a, stream);
  return mla::launch_attention_generic(a, bf16, stream);
}

hipError_t launch_attention_f8(const mla_dims* d, const mla::AttnArgs& a, hipStream_t stream) {
  if (use_fast() && d->dtype == MLA_BF16 &&
      (mla::fast_attention_ok(a) || mla::fast_attention_h16_ok(a)))
    return mla::launch_attention_fp8(a, stream);
  return mla::launch_attention_generic_fp8(a, stream);
}

// Bytes mla_absorb_out uses of its workspace: o in dtype, then the fp32 K-split
// partial sums of the larger of its two products.
size_t absorb_out_bytes(const mla_dims* d, int batch) {
  return act_bytes(d, batch) + std::max(partial_bytes(d, uv_args(d, batch)),
                                        partial_bytes(d, oproj_args(d, batch)));
}

// The two products of the absorbed output with `ws` (256-byte aligned, at least
// absorb_out_bytes) as their scratch.
mla_status absorb_out_run(const mla_dims* d, const void* o_lat, const void* w_uv, const void* w_o,
                          int32_t batch, float* u, void* ws, size_t ws_bytes, hipStream_t stream,
                          bool o_lat_bf16 = false) {
  char* part = static_cast<char*>(ws) + act_bytes(d, batch);
  const size_t pbytes = ws_bytes - act_bytes(d, batch);
  // 1) o[b, i*d_h + e] = sum_c W_UV[i*d_h + e, c] o_lat[b, i, c] per head i -> workspace
  //    (o_lat fp32, or already rounded to bf16, the product's input precision)
  mla::GemmArgs g = uv_args(d, batch);
  g.x = o_lat; g.w1 = w_uv; g.w2 = w_uv; g.y = ws;
  if (o_lat_bf16) g.x_f32 = 0;
  if (run_gemm(d, g, part, pbytes, stream) != hipSuccess) return MLA_ERR_HIP;
  // 2) u = o W_O^T
  mla::GemmArgs a = oproj_args(d, batch);
  a.x = ws; a.w1 = w_o; a.w2 = w_o; a.y = u;
  return hip_status(run_gemm(d, a, part, pbytes, stream));
}

}  // namespace

extern "C" {

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

int32_t mla_set_kernel_path(int32_t path) { return g_path.exchange(path == 1 ? 1 : 0); }

const char* mla_status_string(int32_t s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "null pointer argument";
    case MLA_ERR_SHAPE: return "dimension or count out of range";
    case MLA_ERR_UNSUPPORTED: return "unsupported dtype, abi version or page size";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_HIP: return "HIP runtime rejected a launch";
    default: return "unknown status";
  }
}

size_t mla_workspace_bytes_cq(const mla_dims* d, int32_t d_cq, int32_t batch) {
  if (check_dims(d) != MLA_OK || batch < 0 || !cq_ok(d_cq)) return 0;
  // [q^C, batch x n_h*d_h in dtype][c^Q, batch x d_cq in dtype][fp32 K-split partials]
  size_t part = 0;
  if (batch > 0) {
    for (const mla::GemmArgs& a : {cqproj_args(d, d_cq, batch), uq_args(d, d_cq, batch),
                                   uk_args(d, batch, true)})
      part = std::max(part, partial_bytes(d, a));
  }
  return act_bytes(d, batch) + cq_bytes(d, d_cq, batch) + part + 256;
}

size_t mla_workspace_bytes(const mla_dims* d, int32_t batch) {
  if (check_dims(d) != MLA_OK || batch < 0) return 0;
  // [activation region: q^C or o, batch x n_h*d_h in dtype][fp32 K-split partials]
  size_t part = 0;
  if (batch > 0) {
    for (const mla::GemmArgs& a : {qproj_args(d, batch), uk_args(d, batch, true), uv_args(d, batch),
                                   oproj_args(d, batch), append_args(d, batch), qa_args(d, batch)})
      part = std::max(part, partial_bytes(d, a));
  }
  return act_bytes(d, batch) + part + 256;
}

size_t mla_append_workspace_bytes(const mla_dims* d, int32_t n_rows) {
  if (check_dims(d) != MLA_OK || n_rows < 0) return 0;
  return n_rows > 0 ? partial_bytes(d, append_args(d, n_rows)) + 256 : 0;
}

mla_status mla_device_error(int32_t* out, int32_t clear, hipStream_t stream) {
  if (!out) return MLA_ERR_NULL;
  int* p = err_word();
  if (!p) return MLA_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return MLA_ERR_HIP;
  int v = 0;
  if (hipMemcpy(&v, p, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return MLA_ERR_HIP;
  *out = v;
  if (clear) {
    if (hipMemsetAsync(p, 0, sizeof(int), stream) != hipSuccess) return MLA_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return MLA_ERR_HIP;
  }
  return MLA_OK;
}

mla_status mla_append_latent(const mla_dims* d, const void* h, const void* w_dkv, const void* w_kr,
                             const int32_t* row_seq, const int32_t* row_pos, int32_t n_rows,
                             const int32_t* block_table, int32_t n_seqs, int32_t max_pages,
                             void* pool, int64_t num_pages, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (n_rows < 0 || n_seqs < 0 || max_pages < 0 || num_pages < 0) return MLA_ERR_SHAPE;
  if (n_rows == 0) return MLA_OK;
  if (n_seqs < 1 || max_pages < 1 || num_pages < 1) return MLA_ERR_SHAPE;
  if (static_cast<int64_t>(max_pages) * d->page_size > (int64_t{1} << 30)) return MLA_ERR_SHAPE;
  if (!h || !w_dkv || !w_kr || !row_seq || !row_pos || !block_table || !pool) return MLA_ERR_NULL;
  mla::GemmArgs a = append_args(d, n_rows);
  const size_t need = partial_bytes(d, a);
  if (need > 0 && (!ws || ws_bytes < need || !ws_aligned(ws))) return MLA_ERR_WORKSPACE;
  int* err = err_word();
  if (!err) return MLA_ERR_HIP;
  a.x = h; a.w1 = w_dkv; a.w2 = w_kr; a.y = pool;
  a.pos = row_pos; a.row_seq = row_seq; a.block_table = block_table;
  a.n_seqs = n_seqs; a.max_pages = max_pages; a.page_size = d->page_size;
  a.num_pages = num_pages; a.err = err;
  return hip_status(run_gemm(d, a, ws, ws_bytes, stream));
}

mla_status mla_absorb_q(const mla_dims* d, const void* h, const void* w_q, const void* w_qr,
                        const void* w_uk, const int32_t* pos, int32_t batch, float* q_lat,
                        float* q_pe, void* ws, size_t ws_bytes, hipStream_t stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (batch < 0 || batch > (1 << 20)) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (!h || !w_q || !w_qr || !w_uk || !pos || !q_lat || !q_pe) return MLA_ERR_NULL;
  if (!ws || ws_bytes < mla_workspace_bytes(d, batch) || !ws_aligned(ws)) return MLA_ERR_WORKSPACE;
  char* part = static_cast<char*>(ws) + act_bytes(d, batch);
  const size_t pbytes = ws_bytes - act_bytes(d, batch);
  // 1) [q^C | q^R] = h [W_Q; W_QR]^T, RoPE on the q^R columns; q^C -> workspace
  mla::GemmArgs a = qproj_args(d, batch);
  a.x = h; a.w1 = w_q; a.w2 = w_qr; a.y = ws; a.y2 = q_pe; a.pos = pos;
  if (run_gemm(d, a, part, pbytes, stream) != hipSuccess) return MLA_ERR_HIP;
  // 2) q_lat[b, i, :] = W_UK,i^T q^C[b, i, :] per head i (q^C in fp32)
  mla::GemmArgs g = uk_args(d, batch, true);
  g.x = ws; g.w1 = w_uk; g.w2 = w_uk; g.y = q_lat;
  return hip_status(run_gemm(d, g, part, pbytes, stream));
}

mla_status mla_absorb_q_append(const mla_dims* d, const void* h, const void* w_q,
                               const void* w_qr, const void* w_uk, const void* w_dkv,
                               const void* w_kr, const int32_t* pos, const int32_t* row_seq,
                               int32_t batch, const int32_t* block_table, int32_t n_seqs,
                               int32_t max_pages, void* pool, int64_t num_pages, float* q_lat,
                               float* q_pe, void* ws, size_t ws_bytes, hipStream_t stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (batch < 0 || batch > (1 << 20) || n_seqs < 0 || max_pages < 0 || num_pages < 0)
    return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (n_seqs < 1 || max_pages < 1 || num_pages < 1) return MLA_ERR_SHAPE;
  if (static_cast<int64_t>(max_pages) * d->page_size > (int64_t{1} << 30)) return MLA_ERR_SHAPE;
  if (!h || !w_q || !w_qr || !w_uk || !w_dkv || !w_kr || !pos || !row_seq || !block_table ||
      !pool || !q_lat || !q_pe)
    return MLA_ERR_NULL;
  if (!ws || ws_bytes < mla_workspace_bytes(d, batch) || !ws_aligned(ws)) return MLA_ERR_WORKSPACE;
  int* err = err_word();
  if (!err) return MLA_ERR_HIP;
  char* part = static_cast<char*>(ws) + act_bytes(d, batch);
  const size_t pbytes = ws_bytes - act_bytes(d, batch);
  // 1) [q^C | q^R | c^KV | k^R] = h [W_Q; W_QR; W_DKV; W_KR]^T: q^C -> workspace,
  //    RoPE'd q^R -> q_pe, [c^KV | RoPE(k^R)] -> the rows' pool slots.  The
  //    pointers are set before the shape check, which also tests their alignment.
  mla::GemmArgs a = qa_args(d, batch);
  a.x = h; a.w1 = w_q; a.w2 = w_qr; a.w3 = w_dkv; a.w4 = w_kr;
  a.y = ws; a.y2 = q_pe; a.y3 = pool; a.pos = pos; a.row_seq = row_seq;
  a.block_table = block_table; a.n_seqs = n_seqs; a.max_pages = max_pages;
  a.page_size = d->page_size; a.num_pages = num_pages; a.err = err;
  if (!(use_fast() && d->dtype == MLA_BF16 && mla::fused_qa_ok(a))) {
    // shapes the fused product does not take: the two calls one after the other
    st = mla_absorb_q(d, h, w_q, w_qr, w_uk, pos, batch, q_lat, q_pe, ws, ws_bytes, stream);
    if (st != MLA_OK) return st;
    return mla_append_latent(d, h, w_dkv, w_kr, row_seq, pos, batch, block_table, n_seqs,
                             max_pages, pool, num_pages, ws, ws_bytes, stream);
  }
  if (mla::launch_gemm_fast(a, part, pbytes, stream) != hipSuccess) return MLA_ERR_HIP;
  // 2) q_lat[b, i, :] = W_UK,i^T q^C[b, i, :] per head i (q^C in fp32)
  mla::GemmArgs g = uk_args(d, batch, true);
  g.x = ws; g.w1 = w_uk; g.w2 = w_uk; g.y = q_lat;
  return hip_status(run_gemm(d, g, part, pbytes, stream));
}

mla_status mla_absorb_q_cq(const mla_dims* d, int32_t d_cq, const void* h, const void* w_dq,
                           const void* w_uq, const void* w_qr, const void* w_uk,
                           const int32_t* pos, int32_t batch, float* q_lat, float* q_pe, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!cq_ok(d_cq) || batch < 0 || batch > (1 << 20)) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (!h || !w_dq || !w_uq || !w_qr || !w_uk || !pos || !q_lat || !q_pe) return MLA_ERR_NULL;
  if (!ws || ws_bytes < mla_workspace_bytes_cq(d, d_cq, batch) || !ws_aligned(ws))
    return MLA_ERR_WORKSPACE;
  char* qc = static_cast<char*>(ws);
  char* cq = qc + act_bytes(d, batch);
  char* part = cq + cq_bytes(d, d_cq, batch);
  const size_t pbytes = ws_bytes - act_bytes(d, batch) - cq_bytes(d, d_cq, batch);
  // 1) [c^Q | q^R] = h [W_DQ; W_QR]^T, RoPE on the q^R columns; c^Q -> workspace
  mla::GemmArgs a = cqproj_args(d, d_cq, batch);
  a.x = h; a.w1 = w_dq; a.w2 = w_qr; a.y = cq; a.y2 = q_pe; a.pos = pos;
  if (run_gemm(d, a, part, pbytes, stream) != hipSuccess) return MLA_ERR_HIP;
  // 2) q^C = W_UQ c^Q -> workspace
  mla::GemmArgs u = uq_args(d, d_cq, batch);
  u.x = cq; u.w1 = w_uq; u.w2 = w_uq; u.y = qc;
  if (run_gemm(d, u, part, pbytes, stream) != hipSuccess) return MLA_ERR_HIP;
  // 3) q_lat[b, i, :] = W_UK,i^T q^C[b, i, :] per head i (q^C in fp32)
  mla::GemmArgs g = uk_args(d, batch, true);
  g.x = qc; g.w1 = w_uk; g.w2 = w_uk; g.y = q_lat;
  return hip_status(run_gemm(d, g, part, pbytes, stream));
}

mla_status mla_decode_attention(const mla_dims* d, const float* q_lat, const float* q_pe,
                                const void* pool, int64_t num_pages, const int32_t* block_table,
                                int32_t max_pages, const int32_t* seq_lens, int32_t batch,
                                int32_t num_splits, float* o_part, float* lse_part,
                                hipStream_t stream) {
  mla::AttnArgs a{};
  mla_status st = attention_args(d, false, q_lat, q_pe, pool, num_pages, block_table, max_pages,
                                 seq_lens, nullptr, nullptr, batch, batch, num_splits, o_part,
                                 lse_part, &a);
  if (st != MLA_OK || batch == 0) return st;
  return hip_status(launch_attention_plain(d, a, stream));
}

mla_status mla_prefill_attention(const mla_dims* d, const float* q_lat, const float* q_pe,
                                 const void* pool, int64_t num_pages, const int32_t* block_table,
                                 int32_t n_seqs, int32_t max_pages, const int32_t* q_seq,
                                 const int32_t* q_pos, int32_t n_q, int32_t num_splits,
                                 float* o_part, float* lse_part, hipStream_t stream) {
  mla::AttnArgs a{};
  mla_status st = attention_args(d, true, q_lat, q_pe, pool, num_pages, block_table, max_pages,
                                 nullptr, q_seq, q_pos, n_seqs, n_q, num_splits, o_part, lse_part,
                                 &a);
  if (st != MLA_OK || n_q == 0) return st;
  return hip_status(launch_attention_plain(d, a, stream));
}

size_t mla_fp8_page_bytes(const mla_dims* d) {
  if (check_dims(d) != MLA_OK || !fp8_ok(d)) return 0;
  return static_cast<size_t>(fp8_page_bytes(d));
}

size_t mla_append_workspace_bytes_fp8(const mla_dims* d, int32_t n_rows) {
  if (check_dims(d) != MLA_OK || !fp8_ok(d) || n_rows <= 0) return 0;
  // [fp32 rows, n_rows x (d_c + d_R)][fp32 K-split partials]
  return rows_bytes(d, n_rows) + partial_bytes(d, append_rows_args(d, n_rows)) + 256;
}

mla_status mla_quantize_rows_fp8(const mla_dims* d, const float* rows, int64_t ld_rows,
                                 const int32_t* row_seq, const int32_t* row_pos, int32_t n_rows,
                                 const int32_t* block_table, int32_t n_seqs, int32_t max_pages,
                                 void* pool, int64_t num_pages, hipStream_t stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!fp8_ok(d)) return MLA_ERR_UNSUPPORTED;
  if (n_rows < 0 || n_seqs < 0 || max_pages < 0 || num_pages < 0) return MLA_ERR_SHAPE;
  if (ld_rows < d->d_latent + d->d_rope || ld_rows % 4 != 0 || ld_rows > (int64_t{1} << 32))
    return MLA_ERR_SHAPE;
  if (n_rows == 0) return MLA_OK;
  if (n_seqs < 1 || max_pages < 1 || num_pages < 1) return MLA_ERR_SHAPE;
  if (static_cast<int64_t>(max_pages) * d->page_size > (int64_t{1} << 30)) return MLA_ERR_SHAPE;
  if (!rows || !row_seq || !row_pos || !block_table || !pool) return MLA_ERR_NULL;
  if (!aligned16(rows) || !aligned16(pool)) return MLA_ERR_UNSUPPORTED;
  int* err = err_word();
  if (!err) return MLA_ERR_HIP;
  mla::QuantArgs q{};
  q.rows = rows; q.ld_rows = ld_rows; q.n_rows = n_rows;
  q.d_latent = d->d_latent; q.d_rope = d->d_rope; q.rope = 0;
  q.rs = rope_spec(d);
  q.row_seq = row_seq; q.row_pos = row_pos; q.block_table = block_table;
  q.n_seqs = n_seqs; q.max_pages = max_pages; q.page_size = d->page_size;
  q.num_pages = num_pages; q.page_bytes = fp8_page_bytes(d); q.row_bytes = fp8_row_bytes(d);
  q.pool = static_cast<uint8_t*>(pool); q.err = err;
  return hip_status(mla::launch_quantize_rows(q, stream));
}

mla_status mla_append_latent_fp8(const mla_dims* d, const void* h, const void* w_dkv,
                                 const void* w_kr, const int32_t* row_seq,
                                 const int32_t* row_pos, int32_t n_rows,
                                 const int32_t* block_table, int32_t n_seqs, int32_t max_pages,
                                 void* pool, int64_t num_pages, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!fp8_ok(d)) return MLA_ERR_UNSUPPORTED;
  if (n_rows < 0 || n_seqs < 0 || max_pages < 0 || num_pages < 0) return MLA_ERR_SHAPE;
  if (n_rows == 0) return MLA_OK;
  if (n_rows > (1 << 20) || n_seqs < 1 || max_pages < 1 || num_pages < 1) return MLA_ERR_SHAPE;
  if (static_cast<int64_t>(max_pages) * d->page_size > (int64_t{1} << 30)) return MLA_ERR_SHAPE;
  if (!h || !w_dkv || !w_kr || !row_seq || !row_pos || !block_table || !pool) return MLA_ERR_NULL;
  if (!aligned16(pool)) return MLA_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < mla_append_workspace_bytes_fp8(d, n_rows) || !ws_aligned(ws))
    return MLA_ERR_WORKSPACE;
  int* err = err_word();
  if (!err) return MLA_ERR_HIP;
  // 1) fp32 rows [c | W_KR h] = h [W_DKV; W_KR]^T -> workspace
  float* rows = static_cast<float*>(ws);
  char* part = static_cast<char*>(ws) + rows_bytes(d, n_rows);
  mla::GemmArgs a = append_rows_args(d, n_rows);
  a.x = h; a.w1 = w_dkv; a.w2 = w_kr; a.y = rows;
  if (run_gemm(d, a, part, ws_bytes - rows_bytes(d, n_rows), stream) != hipSuccess)
    return MLA_ERR_HIP;
  // 2) RoPE on k^R at row_pos, quantize, scatter into the pages
  return hip_status(quantize_appended(d, rows, n_rows, row_seq, row_pos, block_table, n_seqs,
                                      max_pages, pool, num_pages, err, stream));
}

size_t mla_absorb_q_append_fp8_workspace_bytes(const mla_dims* d, int32_t batch) {
  if (check_dims(d) != MLA_OK || batch < 0 || !fp8_ok(d)) return 0;
  // [q^C][fp32 rows [c^KV | k^R]][fp32 K-split partials]; no less than the two
  // separate calls take when the fused product does not apply
  return std::max(mla_workspace_bytes(d, batch) + rows_bytes(d, batch),
                  mla_append_workspace_bytes_fp8(d, batch));
}

mla_status mla_absorb_q_append_fp8(const mla_dims* d, const void* h, const void* w_q,
                                   const void* w_qr, const void* w_uk, const void* w_dkv,
                                   const void* w_kr, const int32_t* pos, const int32_t* row_seq,
                                   int32_t batch, const int32_t* block_table, int32_t n_seqs,
                                   int32_t max_pages, void* pool, int64_t num_pages, float* q_lat,
                                   float* q_pe, void* ws, size_t ws_bytes, hipStream_t stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!fp8_ok(d)) return MLA_ERR_UNSUPPORTED;
  if (batch < 0 || batch > (1 << 20) || n_seqs < 0 || max_pages < 0 || num_pages < 0)
    return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (n_seqs < 1 || max_pages < 1 || num_pages < 1) return MLA_ERR_SHAPE;
  if (static_cast<int64_t>(max_pages) * d->page_size > (int64_t{1} << 30)) return MLA_ERR_SHAPE;
  if (!h || !w_q || !w_qr || !w_uk || !w_dkv || !w_kr || !pos || !row_seq || !block_table ||
      !pool || !q_lat || !q_pe)
    return MLA_ERR_NULL;
  if (!aligned16(pool)) return MLA_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < mla_absorb_q_append_fp8_workspace_bytes(d, batch) || !ws_aligned(ws))
    return MLA_ERR_WORKSPACE;
  int* err = err_word();
  if (!err) return MLA_ERR_HIP;
  float* rows = reinterpret_cast<float*>(static_cast<char*>(ws) + act_bytes(d, batch));
  char* part = reinterpret_cast<char*>(rows) + rows_bytes(d, batch);
  const size_t pbytes = ws_bytes - act_bytes(d, batch) - rows_bytes(d, batch);
  // 1) [q^C | q^R | c^KV | k^R] = h [W_Q; W_QR; W_DKV; W_KR]^T: q^C -> workspace,
  //    RoPE'd q^R -> q_pe, the rows [c^KV | k^R] -> workspace in fp32
  mla::GemmArgs a = qa_args(d, batch);
  a.x = h; a.w1 = w_q; a.w2 = w_qr; a.w3 = w_dkv; a.w4 = w_kr;
  a.y = ws; a.y2 = q_pe; a.y3 = rows; a.ld3 = rows_ld(d); a.pos = pos;
  if (!(use_fast() && d->dtype == MLA_BF16 && mla::fused_qa_ok(a))) {
    // shapes the fused product does not take: the two calls one after the other
    st = mla_absorb_q(d, h, w_q, w_qr, w_uk, pos, batch, q_lat, q_pe, ws, ws_bytes, stream);
    if (st != MLA_OK) return st;
    return mla_append_latent_fp8(d, h, w_dkv, w_kr, row_seq, pos, batch, block_table, n_seqs,
                                 max_pages, pool, num_pages, ws, ws_bytes, stream);
  }
  if (mla::launch_gemm_fast(a, part, pbytes, stream) != hipSuccess) return MLA_ERR_HIP;
  // 2) RoPE on k^R at pos, quantize, scatter into the rows' pages
  if (quantize_appended(d, rows, batch, row_seq, pos, block_table, n_seqs, max_pages, pool,
                        num_pages, err, stream) != hipSuccess)
    return MLA_ERR_HIP;
  // 3) q_lat[b, i, :] = W_UK,i^T q^C[b, i, :] per head i (q^C in fp32)
  mla::GemmArgs g = uk_args(d, batch, true);
  g.x = ws; g.w1 = w_uk; g.w2 = w_uk; g.y = q_lat;
  return hip_status(run_gemm(d, g, part, pbytes, stream));
}

mla_status mla_decode_attention_fp8(const mla_dims* d, const float* q_lat, const float* q_pe,
                                    const void* pool, int64_t num_pages,
                                    const int32_t* block_table, int32_t max_pages,
                                    const int32_t* seq_lens, int32_t batch, int32_t num_splits,
                                    float* o_part, float* lse_part, hipStream_t stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!fp8_ok(d)) return MLA_ERR_UNSUPPORTED;
  mla::AttnArgs a{};
  st = attention_args(d, false, q_lat, q_pe, pool, num_pages, block_table, max_pages, seq_lens,
                      nullptr, nullptr, batch, batch, num_splits, o_part, lse_part, &a);
  if (st != MLA_OK || batch == 0) return st;
  if (!aligned16(pool)) return MLA_ERR_UNSUPPORTED;
  return hip_status(launch_attention_f8(d, a, stream));
}

mla_status mla_prefill_attention_fp8(const mla_dims* d, const float* q_lat, const float* q_pe,
                                     const void* pool, int64_t num_pages,
                                     const int32_t* block_table, int32_t n_seqs,
                                     int32_t max_pages, const int32_t* q_seq,
                                     const int32_t* q_pos, int32_t n_q, int32_t num_splits,
                                     float* o_part, float* lse_part, hipStream_t stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!fp8_ok(d)) return MLA_ERR_UNSUPPORTED;
  mla::AttnArgs a{};
  st = attention_args(d, true, q_lat, q_pe, pool, num_pages, block_table, max_pages, nullptr, q_seq,
                      q_pos, n_seqs, n_q, num_splits, o_part, lse_part, &a);
  if (st != MLA_OK || n_q == 0) return st;
  if (!aligned16(pool)) return MLA_ERR_UNSUPPORTED;
  return hip_status(launch_attention_f8(d, a, stream));
}

}  // extern "C"

namespace {
mla_status merge_run(const mla_dims* d, const float* o_part, const float* lse_part, int32_t batch,
                     int32_t num_splits, const int32_t* unit_start, int32_t n_units, float* o_lat,
                     float* lse, hipStream_t stream) {
  mla::MergeArgs a{};
  a.o_part = o_part; a.lse_part = lse_part; a.batch = batch; a.num_splits = num_splits;
  a.n_heads = d->n_heads; a.d_latent = d->d_latent; a.o_lat = o_lat; a.lse = lse;
  a.unit_start = unit_start; a.units = n_units;
  a.err = err_word();
  if (!a.err) return MLA_ERR_HIP;
  const bool bf16 = d->dtype == MLA_BF16;
  if (use_fast() && bf16 && mla::fast_merge_ok(a)) return hip_status(mla::launch_merge_fast(a, stream));
  return hip_status(mla::launch_merge_generic(a, bf16, stream));
}
}  // namespace

extern "C" {

mla_status mla_merge_lse(const mla_dims* d, const float* o_part, const float* lse_part,
                         int32_t batch, int32_t num_splits, float* o_lat, float* lse,
                         hipStream_t stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (batch < 0 || batch > 65535 || num_splits < 1 || num_splits > 4096) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (!o_part || !lse_part || !o_lat) return MLA_ERR_NULL;
  return merge_run(d, o_part, lse_part, batch, num_splits, nullptr, batch * num_splits, o_lat, lse,
                   stream);
}

int64_t mla_decode_plan_capacity(int32_t batch, int32_t target_units) {
  if (batch < 0 || batch > 65535 || target_units < 1 || target_units > (1 << 20)) return 0;
  return 3 * (static_cast<int64_t>(batch) + target_units + 8) + batch + 1;
}

int32_t mla_decode_plan(const int32_t* seq_lens, int32_t batch, int32_t page_size,
                        int32_t target_units, int32_t* plan, int64_t capacity) {
  if (!seq_lens || !plan) return MLA_ERR_NULL;
  if (batch < 1 || batch > 65535 || page_size < 1 || target_units < 1 ||
      target_units > (1 << 20))
    return MLA_ERR_SHAPE;
  if (capacity < mla_decode_plan_capacity(batch, target_units)) return MLA_ERR_WORKSPACE;
  for (int b = 0; b < batch; ++b)
    if (seq_lens[b] < 0) return MLA_ERR_SHAPE;
  // unit length: the fewest whole pages whose unit count stays within the target
  // (the count falls as the length grows, so a bisection over pages finds it); one
  // unit per sequence when even that is over the target
  int64_t max_len = 0;
  for (int b = 0; b < batch; ++b) max_len = std::max<int64_t>(max_len, seq_lens[b]);
  auto count = [&](int64_t u) {
    int64_t c = 0;
    for (int b = 0; b < batch; ++b) c += std::max<int64_t>(1, (seq_lens[b] + u - 1) / u);
    return c;
  };
  int64_t lo = 1, hi = std::max<int64_t>(1, (max_len + page_size - 1) / page_size);   // pages
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (count(mid * page_size) <= target_units) hi = mid; else lo = mid + 1;
  }
  const int64_t unit = lo * page_size;
  int32_t* units = plan;
  std::vector<int32_t> start(batch + 1);
  int64_t n = 0;
  for (int b = 0; b < batch; ++b) {
    const int64_t L = seq_lens[b];
    const int64_t parts = std::max<int64_t>(1, (L + unit - 1) / unit);
    // page-aligned equal chunks, as the uniform splits take them
    const int64_t per = (L + parts - 1) / parts;
    const int64_t chunk = std::max<int64_t>(page_size, (per + page_size - 1) / page_size * page_size);
    start[b] = static_cast<int32_t>(n);
    for (int64_t p = 0; p < parts; ++p) {
      const int64_t t0 = std::min(L, p * chunk), t1 = std::min(L, (p + 1) * chunk);
      if (t0 >= t1 && p > 0) break;   // one (empty) unit for an empty sequence
      units[3 * n] = b;
      units[3 * n + 1] = static_cast<int32_t>(t0);
      units[3 * n + 2] = static_cast<int32_t>(t1);
      ++n;
    }
  }
  start[batch] = static_cast<int32_t>(n);
  while (n % 8 != 0 || n < 8) {   // empty units of sequence 0 (no sequence's range holds them)
    units[3 * n] = 0;
    units[3 * n + 1] = 0;
    units[3 * n + 2] = 0;
    ++n;
  }
  std::copy(start.begin(), start.end(), plan + 3 * n);
  return static_cast<int32_t>(n);
}

mla_status mla_decode_attention_planned(const mla_dims* d, const float* q_lat, const float* q_pe,
                                        const void* pool, int64_t num_pages,
                                        const int32_t* block_table, int32_t max_pages,
                                        const int32_t* plan, int32_t n_units, int32_t batch,
                                        float* o_part, float* lse_part, hipStream_t stream) {
  mla::AttnArgs a{};
  // validated as decode with one split (the plan stands in for the lengths)
  mla_status st = attention_args(d, false, q_lat, q_pe, pool, num_pages, block_table, max_pages,
                                 plan, nullptr, nullptr, batch, batch, 1, o_part, lse_part, &a);
  if (st != MLA_OK || batch == 0) return st;
  if ((st = plan_args(plan, n_units)) != MLA_OK) return st;
  a.seq_lens = nullptr; a.plan = plan; a.units = n_units;
  return hip_status(launch_attention_plain(d, a, stream));
}

mla_status mla_decode_attention_fp8_planned(const mla_dims* d, const float* q_lat,
                                            const float* q_pe, const void* pool,
                                            int64_t num_pages, const int32_t* block_table,
                                            int32_t max_pages, const int32_t* plan,
                                            int32_t n_units, int32_t batch, float* o_part,
                                            float* lse_part, hipStream_t stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!fp8_ok(d)) return MLA_ERR_UNSUPPORTED;
  mla::AttnArgs a{};
  st = attention_args(d, false, q_lat, q_pe, pool, num_pages, block_table, max_pages, plan,
                      nullptr, nullptr, batch, batch, 1, o_part, lse_part, &a);
  if (st != MLA_OK || batch == 0) return st;
  if ((st = plan_args(plan, n_units)) != MLA_OK) return st;
  if (!aligned16(pool)) return MLA_ERR_UNSUPPORTED;
  a.seq_lens = nullptr; a.plan = plan; a.units = n_units;
  return hip_status(launch_attention_f8(d, a, stream));
}

mla_status mla_merge_lse_planned(const mla_dims* d, const float* o_part, const float* lse_part,
                                 const int32_t* plan, int32_t n_units, int32_t batch,
                                 float* o_lat, float* lse, hipStream_t stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (batch < 0 || batch > 65535) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (!o_part || !lse_part || !o_lat) return MLA_ERR_NULL;
  if ((st = plan_args(plan, n_units)) != MLA_OK) return st;
  return merge_run(d, o_part, lse_part, batch, 1, plan + 3 * static_cast<int64_t>(n_units),
                   n_units, o_lat, lse, stream);
}

mla_status mla_absorb_out(const mla_dims* d, const float* o_lat, const void* w_uv, const void* w_o,
                          int32_t batch, float* u, void* ws, size_t ws_bytes, hipStream_t stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (batch < 0 || batch > (1 << 20)) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (!o_lat || !w_uv || !w_o || !u) return MLA_ERR_NULL;
  if (!ws || ws_bytes < mla_workspace_bytes(d, batch) || !ws_aligned(ws)) return MLA_ERR_WORKSPACE;
  return absorb_out_run(d, o_lat, w_uv, w_o, batch, u, ws, ws_bytes, stream);
}

size_t mla_merge_absorb_out_workspace_bytes(const mla_dims* d, int32_t batch) {
  if (check_dims(d) != MLA_OK || batch < 0 || batch > 65535) return 0;
  return align256(mla_workspace_bytes(d, batch)) +
         align256(static_cast<size_t>(batch) * d->n_heads * d->d_latent * sizeof(float));
}

mla_status mla_merge_absorb_out(const mla_dims* d, const float* o_part, const float* lse_part,
                                int32_t batch, int32_t num_splits, const int32_t* plan,
                                int32_t n_units, const void* w_uv, const void* w_o, float* u,
                                float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (batch < 0 || batch > 65535) return MLA_ERR_SHAPE;
  if (plan) {
    if ((st = plan_args(plan, n_units)) != MLA_OK) return st;
  } else if (num_splits < 1 || num_splits > 4096) {
    return MLA_ERR_SHAPE;
  }
  if (batch == 0) return MLA_OK;
  if (!o_part || !lse_part || !w_uv || !w_o || !u) return MLA_ERR_NULL;
  if (!ws || ws_bytes < mla_merge_absorb_out_workspace_bytes(d, batch) || !ws_aligned(ws))
    return MLA_ERR_WORKSPACE;
  // workspace: [mla_absorb_out's region][o_lat, fp32: the merged rows where the
  // merge runs on its own]
  const size_t base = align256(mla_workspace_bytes(d, batch));
  float* o_lat = reinterpret_cast<float*>(static_cast<char*>(ws) + base);
  mla::MergeArgs m{};
  m.o_part = o_part; m.lse_part = lse_part; m.batch = batch;
  m.num_splits = plan ? 1 : num_splits;
  m.n_heads = d->n_heads; m.d_latent = d->d_latent; m.o_lat = o_lat; m.lse = lse;
  m.unit_start = plan ? plan + 3 * static_cast<int64_t>(n_units) : nullptr;
  m.units = plan ? n_units : batch * num_splits;
  m.err = err_word();
  if (!m.err) return MLA_ERR_HIP;
  if (!plan && num_splits == 1) {
    // one split: the merge is the identity (weight exp(0) = 1, sum 1), so the
    // partials are o_lat and lse_part is lse
    if (lse && lse != lse_part &&
        hipMemcpyAsync(lse, lse_part, sizeof(float) * batch * d->n_heads,
                       hipMemcpyDeviceToDevice, stream) != hipSuccess)
      return MLA_ERR_HIP;
    return absorb_out_run(d, o_part, w_uv, w_o, batch, u, ws, base, stream);
  }
  mla::GemmArgs g = uv_args(d, batch);
  g.x = o_part; g.w1 = w_uv; g.w2 = w_uv; g.y = ws;
  if (use_fast() && d->dtype == MLA_BF16 && mla::uv_merge_ok(g, m) && mla::uv_merge_pays(g, m)) {
    // 1) o = W_UV,i (merged partials) per head, the merge inside the product -> workspace
    if (mla::launch_uv_merge(g, m, stream) != hipSuccess) return MLA_ERR_HIP;
    // 2) u = o W_O^T
    mla::GemmArgs a = oproj_args(d, batch);
    a.x = ws; a.w1 = w_o; a.w2 = w_o; a.y = u;
    return hip_status(run_gemm(d, a, static_cast<char*>(ws) + act_bytes(d, batch),
                               base - act_bytes(d, batch), stream));
  }
  // Batches whose W_UV runs on the tiled product (>= 256 rows): the merge writes its
  // rows in bf16, the precision that product reads them in, and the product takes
  // them as such (half the bytes of an fp32 o_lat, each way; the same products)
  mla::GemmArgs gb = uv_args(d, batch);
  gb.x = o_lat; gb.w1 = w_uv; gb.w2 = w_uv; gb.y = ws; gb.x_f32 = 0;
  mla::MergeArgs mb = m;
  mb.o_lat_bf16 = o_lat;
  if (use_fast() && d->dtype == MLA_BF16 && mla::fast_merge_ok(mb) && mla::merge_bf16_ok(mb) &&
      mla::gemm_tiled_ok(gb)) {
    if (mla::launch_merge_fast(mb, stream) != hipSuccess) return MLA_ERR_HIP;
    return absorb_out_run(d, o_lat, w_uv, w_o, batch, u, ws, base, stream, true);
  }
  st = merge_run(d, o_part, lse_part, batch, m.num_splits, m.unit_start, m.units, o_lat, lse,
                 stream);
  if (st != MLA_OK) return st;
  return absorb_out_run(d, o_lat, w_uv, w_o, batch, u, ws, base, stream);
}

size_t mla_absorb_out_noalloc_max_bytes(void) { return kScratchBytes; }

mla_status mla_absorb_out_noalloc(const mla_dims* d, const float* o_lat, const void* w_uv,
                                  const void* w_o, int32_t batch, float* u, hipStream_t stream) {
  mla_status st = check_dims(d);
  if (st != MLA_OK) return st;
  if (batch < 0 || batch > (1 << 20)) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (!o_lat || !w_uv || !w_o || !u) return MLA_ERR_NULL;
  const size_t need = absorb_out_bytes(d, batch);
  if (need > kScratchBytes) return MLA_ERR_WORKSPACE;
  void* ws = scratch_address();
  if (!ws) return MLA_ERR_HIP;
  return absorb_out_run(d, o_lat, w_uv, w_o, batch, u, ws, kScratchBytes, stream);
}
}  // extern "C"
