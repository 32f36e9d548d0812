// Plain vector-ALU kernels for every MLA step, any shape, fp32 or bf16 storage.
//
// They are the shape-general path (the 64-wide fp32 workload runs here) and a
// second implementation the MFMA kernels are checked against.  fp32
// accumulation throughout.
#include "common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"

namespace mla {

// ----------------------------------------------------------------- GEMM --
// Y[m, n] = sum_k X(m, k) W(n, k); tile 32 (m) x 64 (n) x 32 (k); each thread
// owns 2 rows x 4 adjacent columns, so RoPE pairs (even, odd) stay in-thread.
constexpr int GT_M = 32, GT_N = 64, GT_K = 32;

template <typename T>
__global__ __launch_bounds__(256) void k_gemm_generic(GemmArgs a) {
  __shared__ float xs[GT_M][GT_K + 1];
  __shared__ float ws[GT_N][GT_K + 1];
  const int z = blockIdx.z;
  const int m0 = blockIdx.y * GT_M, n0 = blockIdx.x * GT_N;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t xb = z * a.x_bs;
  float acc[2][4] = {};
  for (int k0 = 0; k0 < a.K; k0 += GT_K) {
    for (int e = tid; e < GT_M * GT_K; e += 256) {
      const int r = e / GT_K, kk = e % GT_K;
      const int m = m0 + r, k = k0 + kk;
      xs[r][kk] = (m < a.M && k < a.K) ? ld_act<T>(a.x, xb + m * a.ldx_m + k * a.ldx_k, a.x_f32)
                                       : 0.f;
    }
    for (int e = tid; e < GT_N * GT_K; e += 256) {
      const int r = e / GT_K, kk = e % GT_K;
      const int n = n0 + r, k = k0 + kk;
      float v = 0.f;
      if (n < a.N && k < a.K) {
        const T* w = n < a.n_split ? static_cast<const T*>(a.w1) + z * a.w_bs + n * a.ldw_n
                                   : static_cast<const T*>(a.w2) + z * a.w_bs +
                                         (n - a.n_split) * a.ldw_n;
        v = ld(w + k * a.ldw_k);
      }
      ws[r][kk] = v;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < GT_K; ++kk) {
      const float x0 = xs[ty * 2][kk], x1 = xs[ty * 2 + 1][kk];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float w = ws[tx * 4 + j][kk];
        acc[0][j] += x0 * w;
        acc[1][j] += x1 * w;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + ty * 2 + i;
    if (m >= a.M) continue;
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      const int n = n0 + tx * 4 + j;
      if (n < a.N) gemm_epilogue<T>(a, z, m, n, acc[i][j], acc[i][j + 1]);
    }
  }
}

hipError_t launch_gemm_generic(const GemmArgs& a, bool bf16, hipStream_t stream) {
  if (a.M == 0 || a.N == 0 || a.batch == 0) return hipSuccess;
  dim3 grid((a.N + GT_N - 1) / GT_N, (a.M + GT_M - 1) / GT_M, a.batch);
  if (bf16)
    hipLaunchKernelGGL(k_gemm_generic<bf16_t>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(k_gemm_generic<float>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ attention --
// Row readers of the two pool formats.  row() gives a handle of the row at
// (page, slot), scale() its multiplier and get() element e of it as fp32.
template <typename T>
struct PlainRows {   // pages of page_size rows of d_c + d_R values of T
  const T* pool;
  int row_w, page_size;
  __device__ PlainRows(const AttnArgs& a)
      : pool(static_cast<const T*>(a.pool)), row_w(a.d_latent + a.d_rope), page_size(a.page_size) {}
  __device__ int64_t row(int page, int slot) const {
    return (static_cast<int64_t>(page) * page_size + slot) * row_w;
  }
  __device__ float scale(int, int) const { return 1.f; }
  __device__ float get(int64_t r, int e, float) const { return ld(pool + r + e); }
};

struct Fp8Rows {     // pages of page_size rows [d_c e4m3 | d_R bf16], then page_size fp32 scales
  const uint8_t* pool;
  int d_c, row_bytes, page_size;
  int64_t page_bytes;
  __device__ Fp8Rows(const AttnArgs& a)
      : pool(static_cast<const uint8_t*>(a.pool)), d_c(a.d_latent),
        row_bytes(a.d_latent + 2 * a.d_rope), page_size(a.page_size),
        page_bytes(static_cast<int64_t>(a.page_size) * (a.d_latent + 2 * a.d_rope + 4)) {}
  __device__ int64_t row(int page, int slot) const {
    return static_cast<int64_t>(page) * page_bytes + static_cast<int64_t>(slot) * row_bytes;
  }
  __device__ float scale(int page, int slot) const {
    return *reinterpret_cast<const float*>(pool + static_cast<int64_t>(page) * page_bytes +
                                           static_cast<int64_t>(page_size) * row_bytes + 4 * slot);
  }
  __device__ float get(int64_t r, int e, float sc) const {
    if (e < d_c) return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(pool[r + e]), 0) * sc;
    return bf16_to_f32(*reinterpret_cast<const bf16_t*>(pool + r + d_c + 2 * (e - d_c)));
  }
};

// One workgroup per (head, split, sequence).  Tokens are taken 256 at a time:
// thread t scores token t (full d_c + d_R dot product), the chunk's weights
// go through an online softmax, then each thread accumulates latent columns.
template <typename Rows>
__global__ __launch_bounds__(256) void k_attention_generic(AttnArgs a) {
  extern __shared__ float smem[];
  const int row_w = a.d_latent + a.d_rope;
  float* qs = smem;                         // [row_w]
  float* acc = qs + row_w;                  // [d_latent]
  float* ps = acc + a.d_latent;             // [256]
  float* rsc = ps + 256;                    // [256] row scales
  float* red = rsc + 256;                   // [8]
  int64_t* rowoff = reinterpret_cast<int64_t*>(red + 8);  // [256]

  const int i = blockIdx.x;
  const int u = blockIdx.y + blockIdx.z * gridDim.y;   // work unit
  if (u >= a.units) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nh = a.n_heads;
  int b, sq, t0, t1;
  attn_unit(a, u, tid == 0 && i == 0, &b, &sq, &t0, &t1);

  const float* ql = a.q_lat + (static_cast<int64_t>(b) * nh + i) * a.d_latent;
  const float* qp = a.q_pe + (static_cast<int64_t>(b) * nh + i) * a.d_rope;
  for (int e = tid; e < a.d_latent; e += 256) { qs[e] = ql[e]; acc[e] = 0.f; }
  for (int e = tid; e < a.d_rope; e += 256) qs[a.d_latent + e] = qp[e];
  __syncthreads();

  const Rows rows(a);
  float m_run = -INFINITY, l_run = 0.f;
  for (int c0 = t0; c0 < t1; c0 += 256) {
    const int j = c0 + tid;
    float sc = -INFINITY, rs = 0.f;
    int64_t off = -1;
    if (j < t1) {
      const int page = a.block_table[static_cast<int64_t>(sq) * a.max_pages + j / a.page_size];
      if (page < 0 || page >= a.num_pages) {
        set_err(a.err, ERR_PAGE);
      } else {
        off = rows.row(page, j % a.page_size);
        rs = rows.scale(page, j % a.page_size);
        float d = 0.f;
        for (int e = 0; e < row_w; ++e) d += qs[e] * rows.get(off, e, rs);
        sc = d * a.scale;
      }
    }
    rowoff[tid] = off;
    rsc[tid] = rs;
    float cmax = wave_max(sc);
    if (lane == 0) red[wv] = cmax;
    __syncthreads();
    cmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : __expf(m_run - m_new);
    const float p = (off < 0 || m_new == -INFINITY) ? 0.f : __expf(sc - m_new);
    ps[tid] = p;
    float psum = wave_sum(p);
    __syncthreads();
    if (lane == 0) red[4 + wv] = psum;
    __syncthreads();
    psum = red[4] + red[5] + red[6] + red[7];
    l_run = l_run * alpha + psum;
    m_run = m_new;
    const int cnt = min(256, t1 - c0);
    for (int d = tid; d < a.d_latent; d += 256) {
      float v = acc[d] * alpha;
      for (int jj = 0; jj < cnt; ++jj) {
        const int64_t o = rowoff[jj];
        if (o >= 0) v += ps[jj] * rows.get(o, d, rsc[jj]);
      }
      acc[d] = v;
    }
    __syncthreads();
  }
  const int64_t ob = static_cast<int64_t>(u) * nh + i;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  for (int d = tid; d < a.d_latent; d += 256) a.o_part[ob * a.d_latent + d] = acc[d] * inv;
  if (tid == 0) a.lse_part[ob] = l_run > 0.f ? m_run + __logf(l_run) : -INFINITY;
}

// pool: 0 = fp32 rows, 1 = bf16 rows, 2 = FP8 pages
static hipError_t launch_attention_rows(const AttnArgs& a, int pool, hipStream_t stream) {
  if (a.units == 0) return hipSuccess;
  const size_t shm = (a.d_latent + a.d_rope + a.d_latent + 256 + 256 + 8) * sizeof(float) +
                     256 * sizeof(int64_t) + 16;
  const int gy = a.units < 32768 ? a.units : 32768;   // units over y and z
  dim3 grid(a.n_heads, gy, (a.units + gy - 1) / gy);
  if (pool == 2)
    hipLaunchKernelGGL(k_attention_generic<Fp8Rows>, grid, dim3(256), shm, stream, a);
  else if (pool == 1)
    hipLaunchKernelGGL(k_attention_generic<PlainRows<bf16_t>>, grid, dim3(256), shm, stream, a);
  else
    hipLaunchKernelGGL(k_attention_generic<PlainRows<float>>, grid, dim3(256), shm, stream, a);
  return hipGetLastError();
}

hipError_t launch_attention_generic(const AttnArgs& a, bool bf16, hipStream_t stream) {
  return launch_attention_rows(a, bf16 ? 1 : 0, stream);
}

hipError_t launch_attention_generic_fp8(const AttnArgs& a, hipStream_t stream) {
  return launch_attention_rows(a, 2, stream);
}

// ---------------------------------------------------------------- merge --
__global__ __launch_bounds__(256) void k_merge_generic(MergeArgs a) {
  const int d = blockIdx.x * 256 + threadIdx.x;
  const int i = blockIdx.y, b = blockIdx.z;
  const int nh = a.n_heads;
  int first, S;
  merge_units(a, b, d == 0 && i == 0, &first, &S);
  const float* lse = a.lse_part + static_cast<int64_t>(first) * nh + i;
  float m = -INFINITY;
  for (int s = 0; s < S; ++s) m = fmaxf(m, lse[static_cast<int64_t>(s) * nh]);
  float z = 0.f, o = 0.f;
  if (m != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float l = lse[static_cast<int64_t>(s) * nh];
      if (l == -INFINITY) continue;
      const float w = __expf(l - m);
      z += w;
      if (d < a.d_latent)
        o += w * a.o_part[((static_cast<int64_t>(first) + s) * nh + i) * a.d_latent + d];
    }
  }
  if (d < a.d_latent)
    a.o_lat[(static_cast<int64_t>(b) * nh + i) * a.d_latent + d] = z > 0.f ? o / z : 0.f;
  if (a.lse && d == 0) a.lse[static_cast<int64_t>(b) * nh + i] = z > 0.f ? m + __logf(z) : -INFINITY;
}

hipError_t launch_merge_generic(const MergeArgs& a, bool, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  dim3 grid((a.d_latent + 255) / 256, a.n_heads, a.batch);
  hipLaunchKernelGGL(k_merge_generic, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
