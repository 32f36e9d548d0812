// MFMA projection GEMMs for gfx950 (the absorbed query, latent append and
// absorbed output steps; [Report] §2.2/§2.3 of "《DeepSeek-V2》深度解读报告").
//
// All of them are weight-streaming at decode batch sizes: Y[m, n] = sum_k
// X[m, k] W[n, k] with M = batch (tens to hundreds), N and K in the thousands,
// so the time is the time to read W once from HBM.
//
// k_gemm_skinny (W row-major [N, K], K contiguous): a workgroup of 4 waves owns
// 64 rows of W and 64 rows of X; each wave takes a quarter of the workgroup's
// K slice.  W and X fragments go straight from memory into MFMA operand
// registers (no LDS on the way in): mfma_f32_32x32x16_bf16 with W rows as M and
// X rows as N.  Inside each group of 64 k the lanes of k-group g hold
// k = 32g + 8s + j for step s, so every lane reads 64 contiguous bytes per row.
// The 4 wave partials are summed through LDS; with a K split across
// workgroups the partial tiles go to an fp32 buffer that k_gemm_finish sums in
// a fixed order (deterministic), applying the output stage.
//
// k_gemm_uk (the per-head W_UK product, W row-major [K=d_h, N=d_c], N
// contiguous): the workgroup stages a 128 x 128 W tile in LDS and reads MFMA
// operands from it with ds_read_b64_tr_b16, the hardware transpose.
#include <algorithm>

#include "common.hpp"
#include "epilogue.hpp"
#include "launch_fast.hpp"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;        // W rows and X rows per workgroup
constexpr int kGroupK = 64;      // k per load group (4 MFMA k-steps)
constexpr int kWavesK = 4;       // waves splitting the workgroup's K slice

__device__ __forceinline__ unsigned cvt2(float lo, float hi) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// 8 consecutive k of one row as an MFMA operand (bf16 source).
__device__ __forceinline__ bf16x8_t ld8(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8_t*>(p);
}

// 8 consecutive k of one row as an MFMA operand (fp32 source, rounded to bf16).
__device__ __forceinline__ bf16x8_t ld8(const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  const u32x4_t u = {cvt2(a.x, a.y), cvt2(a.z, a.w), cvt2(b.x, b.y), cvt2(b.z, b.w)};
  return __builtin_bit_cast(bf16x8_t, u);
}

template <typename XT>
__global__ __launch_bounds__(256, 2) void k_gemm_skinny(GemmArgs a, int ntiles, int ksplit,
                                                        int kslice, float* partial) {
  __shared__ float red[kWavesK][kTile][kTile + 1];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 31, g = lane >> 5;
  const int zb = blockIdx.x / ntiles, nt = blockIdx.x - zb * ntiles;
  const int n0 = nt * kTile, ks = blockIdx.y, m0 = blockIdx.z * kTile;

  // W rows n0+r and n0+32+r (the tile never straddles n_split)
  const bf16_t* wbase = n0 < a.n_split
                            ? static_cast<const bf16_t*>(a.w1) + zb * a.w_bs +
                                  static_cast<int64_t>(n0) * a.ldw_n
                            : static_cast<const bf16_t*>(a.w2) + zb * a.w_bs +
                                  static_cast<int64_t>(n0 - a.n_split) * a.ldw_n;
  const bf16_t* wr[2] = {wbase + static_cast<int64_t>(r) * a.ldw_n,
                         wbase + static_cast<int64_t>(r + 32) * a.ldw_n};
  // X rows m0+r and m0+32+r; rows past M read row 0 (their products are dropped)
  const XT* xbase = static_cast<const XT*>(a.x) + zb * a.x_bs;
  const XT* xr[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int m = m0 + 32 * q + r;
    xr[q] = xbase + static_cast<int64_t>(m < a.M ? m : 0) * a.ldx_m;
  }

  const int kw = kslice / kWavesK;
  const int kbeg = ks * kslice + wv * kw;
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  bf16x8_t wf[2][2][4], xf[2][2][4];   // [buffer][block][step]
  auto load = [&](int buf, int k) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        wf[buf][q][s] = ld8(wr[q] + k + 32 * g + 8 * s);
        xf[buf][q][s] = ld8(xr[q] + k + 32 * g + 8 * s);
      }
  };
  load(0, kbeg);
  for (int k = kbeg; k < kbeg + kw; k += 2 * kGroupK) {
    if (k + kGroupK < kbeg + kw) load(1, k + kGroupK);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[0][i][s], xf[0][j][s], acc[i][j],
                                                              0, 0, 0);
    if (k + kGroupK >= kbeg + kw) break;
    if (k + 2 * kGroupK < kbeg + kw) load(0, k + 2 * kGroupK);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[1][i][s], xf[1][j][s], acc[i][j],
                                                              0, 0, 0);
  }

  // acc[i][j] lane (x row r, g) holds W rows 32i + 8(e/4) + 4g + (e%4), X row 32j + r
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        red[wv][32 * i + 8 * (e >> 2) + 4 * g + (e & 3)][32 * j + r] = acc[i][j][e];
  __syncthreads();

  // thread -> output pairs (W rows 2p, 2p+1; X row xr) so RoPE pairs stay together
  for (int p = tid; p < kTile * kTile / 2; p += 256) {
    const int xrow = p & (kTile - 1), wp = p >> 6;
    const int m = m0 + xrow;
    if (m >= a.M) continue;
    float v0 = 0.f, v1 = 0.f;
#pragma unroll
    for (int w = 0; w < kWavesK; ++w) {
      v0 += red[w][2 * wp][xrow];
      v1 += red[w][2 * wp + 1][xrow];
    }
    const int n = n0 + 2 * wp;
    if (ksplit == 1) {
      gemm_epilogue<bf16_t>(a, zb, m, n, v0, v1);
    } else {
      float* dst = partial + ((static_cast<int64_t>(ks) * a.batch + zb) * a.M + m) * a.N + n;
      dst[0] = v0;
      dst[1] = v1;
    }
  }
}

// Sum of the K-split partials (fixed order) followed by the output stage.
__global__ __launch_bounds__(256) void k_gemm_finish(GemmArgs a, int ksplit, const float* partial) {
  const int64_t pairs = static_cast<int64_t>(a.batch) * a.M * (a.N / 2);
  for (int64_t p = blockIdx.x * int64_t{256} + threadIdx.x; p < pairs;
       p += int64_t{256} * gridDim.x) {
    const int np = static_cast<int>(p % (a.N / 2));
    const int64_t rest = p / (a.N / 2);
    const int m = static_cast<int>(rest % a.M), zb = static_cast<int>(rest / a.M);
    const int n = 2 * np;
    float v0 = 0.f, v1 = 0.f;
    for (int s = 0; s < ksplit; ++s) {
      const float* src = partial + ((static_cast<int64_t>(s) * a.batch + zb) * a.M + m) * a.N + n;
      v0 += src[0];
      v1 += src[1];
    }
    gemm_epilogue<bf16_t>(a, zb, m, n, v0, v1);
  }
}

// ---- per-head q_lat[b, i, c] = sum_d X[b, i*d_h + d] W_UK[i*d_h + d, c] ----
// Workgroup = (head, 128 columns c, 64 rows b); K = d_h = 128.  The W tile
// [128 d x 128 c] is staged in LDS (rows padded by 16 bytes) and read as the
// MFMA A operand (M = c) with transposed reads; X rows are the B operand (N = b).
constexpr int kUkK = 128, kUkN = 128, kUkPad = kUkN * 2 + 16;   // LDS row bytes

__global__ __launch_bounds__(256) void k_gemm_uk(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) char wt[kUkK * kUkPad];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int head = blockIdx.x, c0 = blockIdx.y * kUkN, m0 = blockIdx.z * kTile;
  // stage W_UK rows head*d_h .. +128, columns c0 .. c0+127 (16 bytes per thread per step)
  const bf16_t* wsrc = static_cast<const bf16_t*>(a.w1) + head * a.w_bs + c0;
  for (int e = tid; e < kUkK * (kUkN / 8); e += 256) {
    const int row = e >> 4, ch = e & 15;
    *reinterpret_cast<u32x4_t*>(wt + row * kUkPad + ch * 16) =
        *reinterpret_cast<const u32x4_t*>(wsrc + static_cast<int64_t>(row) * a.ldw_k + ch * 8);
  }
  // X fragments: rows m0+r, m0+32+r, k = 16s + 8g + j
  const int r = lane & 31, g = lane >> 5;
  const bf16_t* xb = static_cast<const bf16_t*>(a.x) + head * a.x_bs;
  bf16x8_t xf[2][kUkK / 16];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int m = m0 + 32 * q + r;
    const bf16_t* row = xb + static_cast<int64_t>(m < a.M ? m : 0) * a.ldx_m;
#pragma unroll
    for (int s = 0; s < kUkK / 16; ++s) xf[q][s] = ld8(row + 16 * s + 8 * g);
  }
  __syncthreads();
  // wave wv owns columns c0 + 32wv .. +31 (A operand M index = column)
  const int i16 = lane & 15, G = lane >> 4;
  const int col = 32 * wv + 16 * (G & 1) + 4 * (i16 & 3);
  f32x16_t acc[2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[q][e] = 0.f;
#pragma unroll
  for (int s = 0; s < kUkK / 16; ++s) {
    const int krow = 16 * s + 8 * (G >> 1) + (i16 >> 2);
    const char* p = wt + krow * kUkPad + col * 2;
    const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(p));
    const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(p + 4 * kUkPad));
    const s16x4_t vv[2] = {v0, v1};
    const bf16x8_t af = __builtin_bit_cast(bf16x8_t, vv);
#pragma unroll
    for (int q = 0; q < 2; ++q)
      acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, xf[q][s], acc[q], 0, 0, 0);
  }
  // acc[q] lane (x row r, g): columns 32wv + 8(e/4) + 4g + (e%4), X row 32q + r
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int m = m0 + 32 * q + r;
    if (m >= a.M) continue;
    float* y = static_cast<float*>(a.y) + head * a.y_bs + static_cast<int64_t>(m) * a.ldy + c0 +
               32 * wv;
#pragma unroll
    for (int e = 0; e < 16; ++e) y[8 * (e >> 2) + 4 * g + (e & 3)] = acc[q][e];
  }
}

int divisor_plan(int tiles, int k_groups) {
  // smallest divisor d of k_groups with tiles*d >= 1024 workgroups (else the largest)
  int best = 1;
  for (int d = 1; d <= k_groups; ++d) {
    if (k_groups % d) continue;
    best = d;
    if (static_cast<int64_t>(tiles) * d >= 1024) break;
  }
  return best;
}

}  // namespace

// NT form: W K-contiguous, X K-contiguous, bf16 weights, tiles of 64 that do not
// straddle the W1/W2 boundary, K a multiple of 256.
static bool skinny_ok(const GemmArgs& a) {
  return a.ldw_k == 1 && a.ldx_k == 1 && a.N % kTile == 0 && a.n_split % kTile == 0 &&
         a.K % (kGroupK * kWavesK) == 0 && a.K > 0 && a.M > 0 && a.ldw_n % 8 == 0 &&
         a.ldx_m % 8 == 0 && a.x_bs % 8 == 0 && a.w_bs % 8 == 0;
}

// The per-head W_UK form: W is [K=128, N] N-contiguous, output fp32.
static bool uk_ok(const GemmArgs& a) {
  return a.ldw_n == 1 && a.ldw_k % 8 == 0 && a.K == kUkK && a.N % kUkN == 0 && a.ldx_k == 1 &&
         !a.x_f32 && a.y_f32 && a.epi == EPI_STORE && a.ldx_m % 8 == 0 && a.x_bs % 8 == 0 &&
         a.w1 == a.w2 && a.n_split >= a.N;
}

bool fast_gemm_ok(const GemmArgs& a) { return skinny_ok(a) || uk_ok(a); }

size_t gemm_partial_bytes(const GemmArgs& a) {
  if (!skinny_ok(a)) return 0;
  const int tiles = a.batch * (a.N / kTile) * ((a.M + kTile - 1) / kTile);
  const int d = divisor_plan(tiles, a.K / (kGroupK * kWavesK));
  return d > 1 ? static_cast<size_t>(d) * a.batch * a.M * a.N * sizeof(float) : 0;
}

hipError_t launch_gemm_fast(const GemmArgs& a, void* partial, size_t partial_bytes,
                            hipStream_t stream) {
  if (a.M == 0 || a.N == 0 || a.batch == 0) return hipSuccess;
  if (uk_ok(a) && !skinny_ok(a)) {
    dim3 grid(a.batch, a.N / kUkN, (a.M + kTile - 1) / kTile);
    hipLaunchKernelGGL(k_gemm_uk, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  const int ntiles = a.N / kTile;
  const int mtiles = (a.M + kTile - 1) / kTile;
  const int d = divisor_plan(a.batch * ntiles * mtiles, a.K / (kGroupK * kWavesK));
  if (d > 1 && (partial == nullptr || partial_bytes < gemm_partial_bytes(a)))
    return hipErrorInvalidValue;
  dim3 grid(a.batch * ntiles, d, mtiles);
  const int kslice = a.K / d;
  if (a.x_f32)
    hipLaunchKernelGGL(k_gemm_skinny<float>, grid, dim3(256), 0, stream, a, ntiles, d, kslice,
                       static_cast<float*>(partial));
  else
    hipLaunchKernelGGL(k_gemm_skinny<bf16_t>, grid, dim3(256), 0, stream, a, ntiles, d, kslice,
                       static_cast<float*>(partial));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || d == 1) return e;
  const int64_t pairs = static_cast<int64_t>(a.batch) * a.M * (a.N / 2);
  const int blocks = static_cast<int>(std::min<int64_t>((pairs + 255) / 256, 8192));
  hipLaunchKernelGGL(k_gemm_finish, dim3(blocks), dim3(256), 0, stream, a, d,
                     static_cast<const float*>(partial));
  return hipGetLastError();
}

}  // namespace mla
