/*
 * mla.h -- C ABI of the MLA latent-KV decode library (libmla.so, gfx950).
 *
 * One decode step of Multi-head Latent Attention: every token is cached only as
 * a latent row [c^KV (d_c) | k^R (d_R)], and attention runs with W_UK folded
 * into the query and W_UV folded into the output, so per-head keys and values
 * are never formed.  Sources (web pages, by title and section):
 *   [Report] "《DeepSeek-V2》深度解读报告": §2.2 low-rank joint KV compression
 *     (c^KV = W_DKV h; k^C = W_UK c, v^C = W_UV c), §2.3 absorption
 *     (W_UK into the query side, W_UV into W_O), §2.4 decoupled RoPE (per-head
 *     q^R, one k^R shared by all heads, score = content score + RoPE score),
 *     §3.1 data flow and cache accounting (d_c + d_R elements per token).
 *   [Digest] "DeepSeek-V2论文解读 ... KV缓存压93.3%": §2.1 (only the latent is cached),
 *     §3.1 (paged cache management).
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers, row-major, densely packed, owned
 *     by the caller.  The library never allocates, frees or synchronises; work
 *     is enqueued on the caller's stream and the call returns at once.
 *   - Storage type is mla_dims.dtype (fp32 or bf16) for h, the weights and the
 *     pool.  Activations handed from one call to the next (q_lat, q_pe,
 *     o_part, lse_part, o_lat, lse) and the output u are always fp32, so that
 *     no extra rounding enters between the calls.  Accumulation is fp32.
 *   - Weights (head i owns rows i*d_h..(i+1)*d_h-1, or i*d_R.. for W_QR):
 *       w_q  [n_h*d_h, H]   w_qr [n_h*d_R, H]   w_dkv [d_c, H]   w_kr [d_R, H]
 *       w_uk [n_h*d_h, d_c] w_uv [n_h*d_h, d_c] w_o   [H, n_h*d_h]
 *   - Paged latent pool: [num_pages, page_size, d_c + d_R]; logical position j
 *     of sequence b lives in row block_table[b*max_pages + j/page_size] *
 *     page_size + j%page_size.  block_table is int32 [batch, max_pages].
 *   - RoPE: adjacent pairs (x[2k], x[2k+1]) are turned by pos*theta_k,
 *     theta_k = rope_base^(-2k/d_R) (YaRN-stretched when rope_scale > 1, see
 *     mla_dims), angles evaluated in fp64.
 *   - Softmax scale tau = softmax_scale if > 0, else 1/sqrt(d_h + d_R); with
 *     YaRN times (0.1 ln rope_scale + 1)^2.
 *   - Errors: every argument the host can see is checked before anything is
 *     enqueued; a failing check returns a negative mla_status and enqueues
 *     nothing.  Device-side values the host cannot see (block-table entries,
 *     positions, sequence lengths) are range-checked inside the kernels: an
 *     out-of-range entry is skipped (never dereferenced) and sets a sticky
 *     device error word, read with mla_device_error().  No call aborts.
 *   - Thread safety: calls keep no state between invocations (apart from the
 *     sticky error word and the kernel-path switch below).
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 2

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = -1,        /* a required pointer is NULL */
  MLA_ERR_SHAPE = -2,       /* a dimension or count is out of range */
  MLA_ERR_UNSUPPORTED = -3, /* dtype / abi_version / page_size / alignment not supported */
  MLA_ERR_WORKSPACE = -4,   /* workspace missing, smaller than mla_workspace_bytes() or
                               not 256-byte aligned */
  MLA_ERR_HIP = -5          /* a kernel launch was rejected by the HIP runtime */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

/* Model dimensions; passed by host pointer to every call. */
typedef struct {
  int32_t abi_version;   /* must equal MLA_ABI_VERSION */
  int32_t hidden;        /* H */
  int32_t n_heads;       /* n_h */
  int32_t d_head;        /* d_h */
  int32_t d_latent;      /* d_c, even */
  int32_t d_rope;        /* d_R, even */
  int32_t page_size;     /* rows per pool page, a power of two in [1, 1024] */
  int32_t dtype;         /* mla_dtype */
  float rope_base;       /* > 0, e.g. 10000 */
  float softmax_scale;   /* <= 0 selects 1/sqrt(d_h + d_R) */
  /* YaRN-stretched RoPE ([Report] §3.3, long-context paragraph: 4K -> 128K with
   * scale 40, alpha 1, beta 32; the method as published by Peng et al., "YaRN:
   * Efficient Context Window Extension of Large Language Models", 2023).  With
   * rope_scale = s > 1, pair k's frequency theta_k = rope_base^(-2k/d_R) becomes
   * theta_k ((1 - g)/s + g), g = clamp((r - alpha)/(beta - alpha), 0, 1),
   * r = rope_orig_len theta_k / (2 pi) (the pair's turns over the original
   * window), and tau (as chosen above) is multiplied by (0.1 ln s + 1)^2, the
   * method's temperature, over the whole score.  rope_scale <= 1: plain RoPE
   * and the three fields below are ignored; else rope_orig_len >= 1 and
   * 0 <= yarn_alpha < yarn_beta (MLA_ERR_SHAPE otherwise). */
  float rope_scale;
  int32_t rope_orig_len;
  float yarn_alpha;
  float yarn_beta;
} mla_dims;

/*
 * Latent append ([Report] §2.2 down-projection, §2.4 shared RoPE key).
 * For each row r < n_rows: c = W_DKV h[r], k^R = RoPE(W_KR h[r], row_pos[r]);
 * the row [c | k^R] (rounded to dtype) is written to the pool at logical
 * position row_pos[r] of sequence row_seq[r].  Also the cache-fill path.
 *   h        [n_rows, H] dtype          row_seq, row_pos  [n_rows] int32
 *   block_table [n_seqs, max_pages] int32, pool [num_pages, page_size, d_c+d_R]
 * Workspace: mla_append_workspace_bytes(dims, n_rows) bytes of device memory,
 * 256-byte aligned (may be 0, then workspace may be NULL); scratch for the
 * duration of the call.
 * Rows whose (seq, pos) or table entry is out of range are not written and set
 * the device error word.  Rows must target distinct slots (else the last
 * writer is unspecified).  n_rows == 0 is a no-op.
 */
mla_status mla_append_latent(const mla_dims* dims, const void* h, const void* w_dkv,
                             const void* w_kr, const int32_t* row_seq, const int32_t* row_pos,
                             int32_t n_rows, const int32_t* block_table, int32_t n_seqs,
                             int32_t max_pages, void* pool, int64_t num_pages, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * Absorbed query ([Report] §2.3: q.(W_UK c) regrouped as (W_UK^T q).c; §3.1:
 * per-head RoPE query from h).  For each sequence b with decode position pos[b]:
 *   q^C_i = W_Q,i h_b,  q_lat[b,i,:] = W_UK,i^T q^C_i           (d_c)
 *   q_pe[b,i,:] = RoPE(W_QR,i h_b, pos[b])                        (d_R)
 *   h [batch, H] dtype; pos [batch] int32; q_lat [batch, n_h, d_c] fp32;
 *   q_pe [batch, n_h, d_R] fp32.
 * Workspace: at least mla_workspace_bytes(dims, batch) bytes of device memory,
 * 256-byte aligned, used for q^C; its contents are scratch for the duration of
 * the call.
 */
mla_status mla_absorb_q(const mla_dims* dims, const void* h, const void* w_q, const void* w_qr,
                        const void* w_uk, const int32_t* pos, int32_t batch, float* q_lat,
                        float* q_pe, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mla_absorb_q and mla_append_latent of the same rows in one call ([Report]
 * §2.2/§2.3/§3.1: the step's new token is both queried and cached from the same
 * h): row b is token (row_seq[b], pos[b]); its absorbed query goes to
 * q_lat / q_pe and its latent row [W_DKV h | RoPE(W_KR h, pos)] to the pool,
 * exactly as the two calls define them.  Both products read h once: on the
 * matrix-core path (bf16 dtype, batch <= 64) they run as one projection over
 * [W_Q; W_QR; W_DKV; W_KR]; other shapes make the two calls in turn.
 * Arguments as in those calls (pos serves as row_pos); workspace: at least
 * mla_workspace_bytes(dims, batch) bytes, 256-byte aligned.  Out-of-range rows
 * are not written to the pool and set the device error word, as in
 * mla_append_latent; their queries are still computed.
 */
mla_status mla_absorb_q_append(const mla_dims* dims, const void* h, const void* w_q,
                               const void* w_qr, const void* w_uk, const void* w_dkv,
                               const void* w_kr, const int32_t* pos, const int32_t* row_seq,
                               int32_t batch, const int32_t* block_table, int32_t n_seqs,
                               int32_t max_pages, void* pool, int64_t num_pages, float* q_lat,
                               float* q_pe, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * Split-KV latent attention ([Report] §2.3, §2.4: every head scores the same
 * cached latent rows, s_ij = tau (q_lat,i . c_j + q_pe,i . k^R_j)).  Sequence b has
 * seq_lens[b] = L tokens (positions 0..L-1, the decode token included).  With
 * S = num_splits, chunk = page_size * ceil(ceil(L/S)/page_size); split s covers
 * positions [s*chunk, min(L, (s+1)*chunk)).  For every (b, s, head i):
 *   lse_part[b,s,i]   = log sum_{j in split} exp(s_ij)         (-inf if empty)
 *   o_part[b,s,i,:]   = sum_j exp(s_ij - lse_part) c_j          (0 if empty)
 *   q_lat [batch, n_h, d_c], q_pe [batch, n_h, d_R] fp32 (the matrix-core path
 *   -- bf16 dtype, n_h = 128 or 16, d_c = 512, d_R = 64, page_size = 64,
 *   q_lat and q_pe 16-byte aligned -- rounds them to bf16 once per work unit,
 *   which bounds its score precision: a relative query error of up to 2^-8 per
 *   element); pool dtype;
 *   seq_lens [batch] int32 in [0, max_pages*page_size];
 *   o_part [batch, S, n_h, d_c] fp32; lse_part [batch, S, n_h] fp32.
 * num_splits in [1, 4096].
 */
mla_status mla_decode_attention(const mla_dims* dims, const float* q_lat, const float* q_pe,
                                const void* pool, int64_t num_pages, const int32_t* block_table,
                                int32_t max_pages, const int32_t* seq_lens, int32_t batch,
                                int32_t num_splits, float* o_part, float* lse_part,
                                hipStream_t stream);

/*
 * Length-proportional work list for the decode attention of a ragged batch
 * ([Report] §2.3: the work of one head group is a pass over its sequence's
 * cached rows, so equal work means equal token counts).  Host function: from
 * seq_lens [batch] (host memory), the unit length U is the smallest multiple of
 * page_size for which sum_b max(1, ceil(L_b / U)) <= target_units (the longest
 * length rounded up to a page when batch alone exceeds target_units), so a
 * target of k times the device's compute units gives at most k rounds of work
 * units; sequence b gets n_b = max(1, ceil(L_b / U)) units, the page-aligned chunks of
 * mla_decode_attention's split rule with S = n_b (trailing empty chunks dropped;
 * an empty sequence keeps one empty unit).  Writes to plan (host memory, at
 * least mla_decode_plan_capacity(batch, target_units) entries):
 *   plan[3u], plan[3u+1], plan[3u+2] = (b, t0, t1) for u < n_units, units of
 *     one sequence consecutive and in order; n_units padded to a multiple of 8
 *     with empty units (0, 0, 0);
 *   plan[3 n_units + b] = first unit of sequence b, b = 0..batch (the last entry
 *     is the number of units before the padding).
 * Returns n_units (>= 8), or a negative mla_status: null pointers, a negative
 * length, batch outside [1, 65535], page_size < 1, target_units outside
 * [1, 2^20], or a capacity below mla_decode_plan_capacity.  The plan is copied
 * to device memory by the caller for the *_planned calls.
 */
int64_t mla_decode_plan_capacity(int32_t batch, int32_t target_units);
int32_t mla_decode_plan(const int32_t* seq_lens, int32_t batch, int32_t page_size,
                        int32_t target_units, int32_t* plan, int64_t capacity);

/*
 * mla_decode_attention over the units of a plan (device copy of
 * mla_decode_plan's output, n_units as it returned): unit u = (b, t0, t1)
 * attends query row b to positions [t0, t1) of sequence b (block_table row b):
 *   o_part [n_units, n_h, d_c] fp32, lse_part [n_units, n_h] fp32 (unit u's
 *   partials, the padding units' empty).
 * A unit with b outside [0, batch) or a range outside [0, max_pages*page_size]
 * is treated as empty and sets bit 1 of the device error word.  Other
 * arguments as in mla_decode_attention; n_units a positive multiple of 8.
 */
mla_status mla_decode_attention_planned(const mla_dims* dims, const float* q_lat,
                                        const float* q_pe, const void* pool, int64_t num_pages,
                                        const int32_t* block_table, int32_t max_pages,
                                        const int32_t* plan, int32_t n_units, int32_t batch,
                                        float* o_part, float* lse_part, hipStream_t stream);

/*
 * Prefill (chunked-prefill) attention: many query tokens per sequence, each
 * attending causally to the latent cache of its own sequence ([Report] §3.1: the
 * same per-token MLA flow for every prompt token; the pages quote prompt
 * throughput for it).  Query token i is the token at position q_pos[i] of
 * sequence q_seq[i]; its row must already be in the pool (append the chunk
 * first).  It attends to positions 0..q_pos[i] of that sequence, split as in
 * mla_decode_attention with L = q_pos[i] + 1; outputs are indexed by query:
 *   q_lat [n_q, n_h, d_c], q_pe [n_q, n_h, d_R] fp32 (from mla_absorb_q with
 *   batch n_q and pos = q_pos); block_table [n_seqs, max_pages] int32;
 *   q_seq, q_pos [n_q] int32; o_part [n_q, S, n_h, d_c], lse_part [n_q, S, n_h].
 * n_q in [0, 65535].  A query whose sequence or position is out of range gets an
 * empty result (lse = -inf) and sets the device error word.  mla_merge_lse and
 * mla_absorb_out then run with batch = n_q.
 */
mla_status mla_prefill_attention(const mla_dims* dims, const float* q_lat, const float* q_pe,
                                 const void* pool, int64_t num_pages, const int32_t* block_table,
                                 int32_t n_seqs, int32_t max_pages, const int32_t* q_seq,
                                 const int32_t* q_pos, int32_t n_q, int32_t num_splits,
                                 float* o_part, float* lse_part, hipStream_t stream);

/*
 * Log-sum-exp merge of split partials: per (b, i), m = max_s lse_s,
 * w_s = exp(lse_s - m), o_lat = sum_s w_s o_s / sum_s w_s, lse = m + log sum_s w_s.
 * Splits with lse = -inf weigh 0; a row whose every split is empty gives
 * o_lat = 0 and lse = -inf.
 *   o_part [batch, S, n_h, d_c] fp32, lse_part [batch, S, n_h] fp32,
 *   o_lat [batch, n_h, d_c] fp32, lse [batch, n_h] fp32 (may be NULL).
 */
mla_status mla_merge_lse(const mla_dims* dims, const float* o_part, const float* lse_part,
                         int32_t batch, int32_t num_splits, float* o_lat, float* lse,
                         hipStream_t stream);

/*
 * mla_merge_lse over the partials of a plan: row b merges units
 * plan[3 n_units + b] .. plan[3 n_units + b + 1] - 1 (same rules; a range
 * outside [0, n_units] merges nothing and sets bit 1 of the device error word).
 *   o_part [n_units, n_h, d_c], lse_part [n_units, n_h]; o_lat, lse as in
 *   mla_merge_lse.
 */
mla_status mla_merge_lse_planned(const mla_dims* dims, const float* o_part, const float* lse_part,
                                 const int32_t* plan, int32_t n_units, int32_t batch,
                                 float* o_lat, float* lse, hipStream_t stream);

/*
 * Absorbed output ([Report] §2.3: W_UV folded into the output projection):
 *   o_i = W_UV,i o_lat[b,i,:] (d_h),  u[b,:] = W_O [o_1; ...; o_n_h]   (H)
 *   o_lat [batch, n_h, d_c] fp32; u [batch, H] fp32.
 * Workspace: at least mla_workspace_bytes(dims, batch) bytes, 256-byte aligned,
 * used for o.
 */
mla_status mla_absorb_out(const mla_dims* dims, const float* o_lat, const void* w_uv,
                          const void* w_o, int32_t batch, float* u, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/*
 * mla_merge_lse and mla_absorb_out as one call ([Report] §2.3: the merged
 * latent output o_lat is only the input of the W_UV product, so the merge is
 * folded into that product's operand loads and o_lat is never stored):
 *   u [batch, H] fp32 = mla_absorb_out of the o_lat that mla_merge_lse (plan
 *   NULL) or mla_merge_lse_planned (plan != NULL) forms from o_part / lse_part,
 *   lse [batch, n_h] fp32 (may be NULL) = that merge's lse.
 * plan NULL: uniform splits, o_part [batch, num_splits, n_h, d_c], lse_part
 * [batch, num_splits, n_h], n_units ignored.  plan != NULL: the plan of
 * mla_decode_plan, o_part [n_units, n_h, d_c], lse_part [n_units, n_h],
 * num_splits ignored; bad ranges as mla_merge_lse_planned.
 * Workspace: at least mla_merge_absorb_out_workspace_bytes(dims, batch) bytes,
 * 256-byte aligned.  bf16 decode batches (batch <= 64) at n_h % 8 = 0,
 * n_h * d_h / 64 >= 256, d_c = 512, with a plan or at most 16 splits take the
 * fused product, whose u and lse are bit-identical to the two calls; other
 * shapes run the two calls inside (same results).  One uniform split (and no
 * plan) merges nothing: o_part is taken as o_lat and lse_part copied to lse,
 * which is what the merge gives for partials as the attention calls write them
 * (an empty split has lse -inf and o 0).
 */
mla_status mla_merge_absorb_out(const mla_dims* dims, const float* o_part, const float* lse_part,
                                int32_t batch, int32_t num_splits, const int32_t* plan,
                                int32_t n_units, const void* w_uv, const void* w_o, float* u,
                                float* lse, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);
/* Workspace bytes of mla_merge_absorb_out (0 for bad dims or batch). */
size_t mla_merge_absorb_out_workspace_bytes(const mla_dims* dims, int32_t batch);

/*
 * mla_absorb_out for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same operation and arguments without the workspace.  Its scratch (the
 * per-head products o, then the fp32 partial sums of the projection) is a
 * static device array of mla_absorb_out_noalloc_max_bytes() bytes (32 MiB)
 * inside the library, one per device, allocated when the library's code is
 * loaded on that device and held until the process ends; no call allocates,
 * frees or synchronises.  A call whose scratch need (the part of
 * mla_workspace_bytes that mla_absorb_out uses: at the full shape H = 5120,
 * n_h = d_h = 128, bf16, about 25 MiB at batch 64) exceeds that returns
 * MLA_ERR_WORKSPACE and enqueues nothing.  Every call on one device shares the
 * one array: calls that may overlap on a device (two streams, two threads)
 * race and must be ordered by the caller.  Results equal mla_absorb_out's.
 */
mla_status mla_absorb_out_noalloc(const mla_dims* dims, const float* o_lat, const void* w_uv,
                                  const void* w_o, int32_t batch, float* u, hipStream_t stream);
/* Bytes of the static scratch array of mla_absorb_out_noalloc. */
size_t mla_absorb_out_noalloc_max_bytes(void);

/*
 * Absorbed query with the query's low-rank compression (the MLA information
 * flow of [Report] §3.1: h -> W_D^Q -> c^Q (d_c' = 1536 there) -> q^C, while the
 * RoPE query q^R is still taken from h).  For each sequence b:
 *   c^Q = W_DQ h_b (d_cq),  q^C_i = W_UQ,i c^Q,  q_lat[b,i,:] = W_UK,i^T q^C_i
 *   q_pe[b,i,:] = RoPE(W_QR,i h_b, pos[b])
 *   w_dq [d_cq, H] and w_uq [n_h*d_h, d_cq] in dtype (head i owns rows
 *   i*d_h..(i+1)*d_h-1 of W_UQ); the rest as mla_absorb_q.  d_cq is even, in
 *   [2, 65536]; inside the call c^Q is held in dtype and q^C in fp32 (as in
 *   mla_absorb_q).
 * Workspace: at least mla_workspace_bytes_cq(dims, d_cq, batch) bytes,
 * 256-byte aligned, used for c^Q and q^C (scratch for the duration of the call).
 */
mla_status mla_absorb_q_cq(const mla_dims* dims, int32_t d_cq, const void* h, const void* w_dq,
                           const void* w_uq, const void* w_qr, const void* w_uk,
                           const int32_t* pos, int32_t batch, float* q_lat, float* q_pe,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes needed by mla_absorb_q / mla_absorb_out for `batch` sequences
 * (0 if dims are invalid): the intermediate q^C or o (batch x n_h*d_h in dtype)
 * followed by fp32 partial sums of the projection GEMMs. */
size_t mla_workspace_bytes(const mla_dims* dims, int32_t batch);
/* Workspace bytes needed by mla_absorb_q_cq (0 if dims or d_cq are invalid):
 * q^C as above, then c^Q (batch x d_cq in dtype), then the GEMM partial sums. */
size_t mla_workspace_bytes_cq(const mla_dims* dims, int32_t d_cq, int32_t batch);

/* Workspace bytes needed by mla_append_latent for `n_rows` rows (0 if none is
 * needed or dims are invalid). */
size_t mla_append_workspace_bytes(const mla_dims* dims, int32_t n_rows);

/*
 * FP8 latent pool ([Report] §4.2: at inference the 576-wide cached latent is
 * further quantized, to about 6 bits per element on average; the pages do not
 * give the scheme).  The format used by the *_fp8 calls (8.9 bits per cached
 * element at d_c = 512, d_R = 64, scale included):
 *   - the pool is [num_pages, page_bytes] bytes, page_bytes =
 *     mla_fp8_page_bytes(dims) = page_size * (d_c + 2*d_R + 4), device memory
 *     owned by the caller, 16-byte aligned;
 *   - a page holds page_size rows of d_c + 2*d_R bytes, [c^KV as d_c e4m3 codes
 *     | k^R as d_R bf16 (little-endian)], followed by page_size fp32 row
 *     scales; logical position j of sequence b is row j%page_size of page
 *     block_table[b*max_pages + j/page_size], its scale the (j%page_size)-th;
 *   - e4m3 (OCP FP8): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits,
 *     largest finite 448, codes 0x7f/0xff are NaN and never written;
 *   - a row's scale is 2^e with e the smallest integer such that
 *     max_k |c_k| / 2^e <= 448 (e = 0 for an all-zero c), clamped to
 *     [-126, 127]; code_k = round-to-nearest-even of c_k / 2^e (exact
 *     division); the dequantized value is value(code_k) * 2^e.  k^R is rounded
 *     to bf16 (nearest even).
 * The *_fp8 calls need d_c a multiple of 8 (else MLA_ERR_UNSUPPORTED); dtype
 * still gives the storage type of h and the weights.
 */

/* Bytes of one FP8 page (0 if dims are invalid or d_c is not a multiple of 8). */
size_t mla_fp8_page_bytes(const mla_dims* dims);

/*
 * Quantize cache rows into the FP8 pool (the cache-fill path of the FP8 pool).
 * Row r < n_rows is rows[r*ld_rows .. r*ld_rows + d_c + d_R) = [c | k^R] in
 * fp32, k^R already rotated; it is written, as the format above fixes it, to
 * logical position row_pos[r] of sequence row_seq[r].
 *   rows fp32 device, 16-byte aligned, ld_rows >= d_c + d_R and a multiple
 *   of 4; row_seq, row_pos [n_rows] int32; block_table [n_seqs, max_pages].
 * Rows whose (seq, pos) or table entry is out of range are not written and set
 * the device error word; rows must target distinct slots.  n_rows == 0 is a
 * no-op.
 */
mla_status mla_quantize_rows_fp8(const mla_dims* dims, const float* rows, int64_t ld_rows,
                                 const int32_t* row_seq, const int32_t* row_pos, int32_t n_rows,
                                 const int32_t* block_table, int32_t n_seqs, int32_t max_pages,
                                 void* pool, int64_t num_pages, hipStream_t stream);

/*
 * Latent append into the FP8 pool: as mla_append_latent (c = W_DKV h[r],
 * k^R = RoPE(W_KR h[r], row_pos[r])), the row computed in fp32 and then
 * quantized as mla_quantize_rows_fp8 does.
 * Workspace: mla_append_workspace_bytes_fp8(dims, n_rows) bytes, 256-byte
 * aligned (the fp32 rows, then GEMM partial sums), scratch for the call.
 */
mla_status mla_append_latent_fp8(const mla_dims* dims, const void* h, const void* w_dkv,
                                 const void* w_kr, const int32_t* row_seq,
                                 const int32_t* row_pos, int32_t n_rows,
                                 const int32_t* block_table, int32_t n_seqs, int32_t max_pages,
                                 void* pool, int64_t num_pages, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);
/* Workspace bytes needed by mla_append_latent_fp8 (0 if n_rows is 0 or dims are
 * invalid). */
size_t mla_append_workspace_bytes_fp8(const mla_dims* dims, int32_t n_rows);

/*
 * mla_absorb_q and mla_append_latent_fp8 of the same rows in one call (the
 * FP8-pool form of mla_absorb_q_append, [Report] §2.2/§2.3/§3.1: the step's new
 * token is queried and cached from the same h).  Row b is token
 * (row_seq[b], pos[b]); its absorbed query goes to q_lat / q_pe and its latent
 * row, computed in fp32, rotated and quantized exactly as mla_append_latent_fp8
 * defines it, to the FP8 pool.  On the matrix-core path (bf16 dtype,
 * batch <= 64) one projection over [W_Q; W_QR; W_DKV; W_KR] reads h once and
 * leaves the fp32 rows in the workspace for the quantizer; other shapes make
 * the two calls in turn.  The queries are those of mla_absorb_q bit for bit;
 * the rows' fp32 sums may differ from mla_append_latent_fp8's in rounding order.
 * Arguments as in mla_absorb_q_append (pos serves as row_pos; pool is the FP8
 * pool, 16-byte aligned; d_c a multiple of 8).  Workspace: at least
 * mla_absorb_q_append_fp8_workspace_bytes(dims, batch) bytes, 256-byte aligned,
 * scratch for the call.  Out-of-range rows are not written to the pool and set
 * the device error word; their queries are still computed.
 */
mla_status mla_absorb_q_append_fp8(const mla_dims* dims, const void* h, const void* w_q,
                                   const void* w_qr, const void* w_uk, const void* w_dkv,
                                   const void* w_kr, const int32_t* pos, const int32_t* row_seq,
                                   int32_t batch, const int32_t* block_table, int32_t n_seqs,
                                   int32_t max_pages, void* pool, int64_t num_pages,
                                   float* q_lat, float* q_pe, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);
/* Workspace bytes needed by mla_absorb_q_append_fp8 (0 if dims are invalid or
 * d_c is not a multiple of 8). */
size_t mla_absorb_q_append_fp8_workspace_bytes(const mla_dims* dims, int32_t batch);

/*
 * Split-KV latent attention over the FP8 pool: mla_decode_attention with every
 * cached row replaced by its dequantized value [value(code) * 2^e | k^R].
 * The matrix-core path (bf16 dtype, n_h = 128, d_c = 512, d_R = 64,
 * page_size = 64) multiplies the stored e4m3 codes directly on the FP8 matrix
 * cores (the row scale applied exactly as a power of two); the queries and
 * the softmax weights enter those products as two e4m3 terms each (relative
 * error <= 2^-8, the order of bf16 rounding), accumulation in fp32.  Other
 * shapes use the plain vector kernel (fp32 arithmetic on the dequantized
 * rows).  Arguments and outputs as mla_decode_attention.
 */
mla_status mla_decode_attention_fp8(const mla_dims* dims, const float* q_lat, const float* q_pe,
                                    const void* pool, int64_t num_pages,
                                    const int32_t* block_table, int32_t max_pages,
                                    const int32_t* seq_lens, int32_t batch, int32_t num_splits,
                                    float* o_part, float* lse_part, hipStream_t stream);

/* mla_decode_attention_planned over the FP8 pool (rows as in
 * mla_decode_attention_fp8). */
mla_status mla_decode_attention_fp8_planned(const mla_dims* dims, const float* q_lat,
                                            const float* q_pe, const void* pool,
                                            int64_t num_pages, const int32_t* block_table,
                                            int32_t max_pages, const int32_t* plan,
                                            int32_t n_units, int32_t batch, float* o_part,
                                            float* lse_part, hipStream_t stream);

/* Prefill attention over the FP8 pool (as mla_prefill_attention, rows dequantized
 * as in mla_decode_attention_fp8). */
mla_status mla_prefill_attention_fp8(const mla_dims* dims, const float* q_lat, const float* q_pe,
                                     const void* pool, int64_t num_pages,
                                     const int32_t* block_table, int32_t n_seqs,
                                     int32_t max_pages, const int32_t* q_seq,
                                     const int32_t* q_pos, int32_t n_q, int32_t num_splits,
                                     float* o_part, float* lse_part, hipStream_t stream);

/* Static text for a status code. */
const char* mla_status_string(int32_t status);

/* Returns MLA_ABI_VERSION of the loaded library. */
int32_t mla_abi_version(void);

/*
 * Sticky device error word: bit 0 = a block-table entry outside [0, num_pages),
 * bit 1 = a position / length beyond max_pages*page_size or negative (also a bad
 * plan entry or unit range), bit 2 = a sequence index outside [0, n_seqs).
 * Synchronises `stream`, copies the word to *out and, if clear != 0, resets it.
 * Returns MLA_ERR_HIP on a runtime error.
 */
mla_status mla_device_error(int32_t* out, int32_t clear, hipStream_t stream);

/*
 * Kernel selection for the whole process: 0 = automatic (the MFMA kernels where
 * the shape allows, else the plain vector kernels), 1 = plain vector kernels
 * only.  Both compute the same quantities; the switch exists so both can be
 * checked (a test hook).  It is one process-wide setting, read when each call
 * is made: it changes the path for every caller in the process, and a call on
 * another thread concurrent with the switch may take either path.  Returns the
 * previous value.
 */
int32_t mla_set_kernel_path(int32_t path);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
