// MFMA projection GEMMs for gfx950 (the absorbed query, latent append and
// absorbed output steps; [Report] §2.2/§2.3 of "《DeepSeek-V2》深度解读报告").
//
// All of them are weight-streaming at decode batch sizes: Y[m, n] = sum_k
// X[m, k] W[n, k] with M = batch (tens to hundreds), N and K in the thousands,
// so the time is the time to read W once from HBM.
//
// k_gemm_ws (W row-major [N, K], K contiguous): a workgroup of 4 waves owns 64
// rows of W, 16 per wave, and an M tile of up to 256 X rows.  Each wave
// streams its 16 W rows straight from memory into MFMA A operands
// (mfma_f32_16x16x32_bf16: lane l holds row l%16, k 8(l/16)..+7 of a 32-k
// step), keeping kWsRing steps in flight per lane.  The X rows of the current
// K chunk sit in LDS, shared by the 4 waves (B operands, one ds_read_b128 per
// 16-row block and step); chunk c + kWsXAhead is loaded into registers when
// chunk c starts and written to LDS one chunk before it is used, so that the
// in-order completion count a wave waits on for X still leaves kWsRing W
// steps in flight.  X is read once per workgroup (not once per wave),
// so the vector memory path carries little beyond the W stream.  When the
// W rows alone give too few workgroups to fill the chip, K is split across
// workgroups: each writes an fp32 partial tile and k_gemm_finish sums them in
// a fixed order (deterministic) and applies the output stage.
//
// k_gemm_uk (the per-head W_UK product, W row-major [K=d_h, N=d_c], N
// contiguous): the workgroup stages a 128 x 128 W tile in LDS and reads MFMA
// operands from it with ds_read_b64_tr_b16, the hardware transpose.
#include <algorithm>
#include <atomic>
#include <type_traits>

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

constexpr int kTile = 64;        // X rows per W_UK workgroup
constexpr int kWsWaves = 4;
constexpr int kWsRows = 16;                     // W rows per wave (MFMA M)
constexpr int kWsTile = kWsWaves * kWsRows;     // W rows per workgroup
constexpr int kWsChunkBytes = 16384;            // one LDS buffer of X rows
constexpr int kWsRing = 8;                      // W k-steps in flight per lane
constexpr int kWsXAhead = 2;                    // X chunks held in registers
constexpr int kWsMaxRows = 128;                 // X rows per workgroup at most

__device__ __forceinline__ unsigned cvt2(float lo, float hi) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// 8 consecutive k of one row as an MFMA operand (bf16 source).
__device__ __forceinline__ bf16x8_t ld8(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8_t*>(p);
}

// Shape of one k_gemm_ws instance: MB blocks of 16 X rows.
template <int MB>
struct WsShape {
  static constexpr int kRowsX = 16 * MB;
  static constexpr int kKC = kWsChunkBytes / (2 * kRowsX);   // k per X chunk
  static constexpr int kSPC = kKC / 32;                       // MFMA k-steps per chunk
  static constexpr int kUnroll =
      kSPC * kWsXAhead > kWsRing ? kSPC * kWsXAhead : kWsRing;   // powers of two: the lcm
  static constexpr int kPitch = 2 * kKC + 16;                 // LDS bytes per X row
  static constexpr int kVecRow = kKC / 8;                     // 16-byte vectors per row
  static constexpr int kVecThread = kRowsX * kVecRow / 256;   // per thread per chunk
  static_assert(kKC >= 32 && kKC % 32 == 0, "chunk");
  static_assert(kUnroll % (kSPC * kWsXAhead) == 0 && kUnroll % kWsRing == 0, "unroll");
  static_assert(kVecThread * 256 == kRowsX * kVecRow, "staging");
};

// k granule of one workgroup's K slice for an instance with MB row blocks
constexpr int ws_kunit(int mb) {
  return 32 * (kWsChunkBytes / (1024 * mb) * kWsXAhead > kWsRing
                   ? kWsChunkBytes / (1024 * mb) * kWsXAhead
                   : kWsRing);
}

// 16-row X blocks per workgroup for M rows (larger M takes several M tiles)
constexpr int ws_mb(int M) {
  return M <= 16 ? 1 : M <= 32 ? 2 : M <= 64 ? 4 : kWsMaxRows / 16;
}

// One 16-byte vector of X (8 values), loaded now and stored to LDS as bf16 later.
template <typename XT>
struct XVec;
template <>
struct XVec<bf16_t> {
  u32x4_t v;
  __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const u32x4_t*>(p); }
  __device__ __forceinline__ u32x4_t bits() const { return v; }
};
template <>
struct XVec<float> {
  float4 lo, hi;
  __device__ __forceinline__ void load(const float* p) {
    lo = *reinterpret_cast<const float4*>(p);
    hi = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ u32x4_t bits() const {
    return (u32x4_t){cvt2(lo.x, lo.y), cvt2(lo.z, lo.w), cvt2(hi.x, hi.y), cvt2(hi.z, hi.w)};
  }
};

template <typename XT, int MB>
__global__ __launch_bounds__(256) void k_gemm_ws(GemmArgs a, int ntiles, int ksplit, int kslice,
                                                 float* partial) {
  using S = WsShape<MB>;
  __shared__ __attribute__((aligned(16))) char xs[2][S::kRowsX * S::kPitch];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int zb = blockIdx.x / ntiles, nt = blockIdx.x - zb * ntiles;
  const int n0 = nt * kWsTile, ks = blockIdx.y, m0 = blockIdx.z * S::kRowsX;
  const int nw = n0 + kWsRows * wv;   // first W row of this wave
  const int64_t kbeg = static_cast<int64_t>(ks) * kslice;

  // this lane's W row (the 64-row tile never straddles n_split)
  const bf16_t* wrow =
      (n0 < a.n_split ? static_cast<const bf16_t*>(a.w1) + zb * a.w_bs +
                            static_cast<int64_t>(nw + r16) * a.ldw_n
                      : static_cast<const bf16_t*>(a.w2) + zb * a.w_bs +
                            static_cast<int64_t>(nw - a.n_split + r16) * a.ldw_n) +
      kbeg + 8 * g;

  // X staging: vector v = tid + 256 i covers row v / kVecRow, k 8 (v % kVecRow);
  // rows past M read row 0 (their outputs are never stored)
  const XT* xsrc[S::kVecThread];
  int xoff[S::kVecThread];
#pragma unroll
  for (int i = 0; i < S::kVecThread; ++i) {
    const int v = tid + 256 * i, row = v / S::kVecRow, kv = v - row * S::kVecRow;
    const int m = m0 + row;
    xsrc[i] = static_cast<const XT*>(a.x) + zb * a.x_bs +
              static_cast<int64_t>(m < a.M ? m : 0) * a.ldx_m + kbeg + 8 * kv;
    xoff[i] = row * S::kPitch + 16 * kv;
  }
  // The workgroup walks its K slice starting at chunk `rot` (wrapping), so at
  // any moment the workgroups read different X chunks instead of all asking the
  // same L2 lines for the same chunk.
  const int nsteps = kslice / 32, nchunks = kslice / S::kKC;
  const int rot = static_cast<int>(blockIdx.x % static_cast<unsigned>(nchunks));
  auto wstep = [&](int st) {   // logical step -> step within the slice
    const int p = st + rot * S::kSPC;
    return p >= nsteps ? p - nsteps : p;
  };
  XVec<XT> xv[kWsXAhead][S::kVecThread];
  auto xload = [&](int set, int c) {
    const int pc = c + rot >= nchunks ? c + rot - nchunks : c + rot;
#pragma unroll
    for (int i = 0; i < S::kVecThread; ++i) xv[set][i].load(xsrc[i] + pc * S::kKC);
  };
  auto xstore = [&](int set, int buf) {
#pragma unroll
    for (int i = 0; i < S::kVecThread; ++i)
      *reinterpret_cast<u32x4_t*>(&xs[buf][xoff[i]]) = xv[set][i].bits();
  };

  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  f32x4_t acc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) acc[i] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  bf16x8_t wr[kWsRing];
#pragma unroll
  for (int u = 0; u < kWsRing; ++u) wr[u] = ld8(wrow + 32 * wstep(u));
#pragma unroll
  for (int c = 0; c < kWsXAhead; ++c) xload(c, min(c, nchunks - 1));
  xstore(0, 0);
  __syncthreads();

  // B operand of block mb at step u of the chunk in buffer buf
  const int boff = r16 * S::kPitch + 16 * g;
  for (int s0 = 0; s0 < nsteps; s0 += S::kUnroll) {
#pragma unroll
    for (int u = 0; u < S::kUnroll; ++u) {
      // s0 is a multiple of kUnroll, so chunk parity and register set are static
      const int s = s0 + u, cu = u / S::kSPC, su = u % S::kSPC;
      const int c = s0 / S::kSPC + cu, buf = cu & 1, set = cu % kWsXAhead;
      // prefetches past the slice re-read its last chunk / step instead of
      // branching: the body stays branch-free, so every wait is exact
      if (su == 0) xload(set, min(c + kWsXAhead, nchunks - 1));
      const bf16x8_t wf = wr[u % kWsRing];
      wr[u % kWsRing] = ld8(wrow + 32 * wstep(min(s + kWsRing, nsteps - 1)));
      // keep every load at its own step: the scheduler would otherwise sink the
      // refills below the products and drain the ring
      __builtin_amdgcn_sched_barrier(0);
      bf16x8_t xf[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        xf[mb] = *reinterpret_cast<const bf16x8_t*>(&xs[buf][boff + 16 * mb * S::kPitch + 64 * su]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, xf[mb], acc[mb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (su == S::kSPC - 1) {
        xstore((cu + 1) % kWsXAhead, buf ^ 1);   // past the end: a buffer nobody reads
        __syncthreads();
      }
    }
  }

  // acc[mb] lane (r16, g) holds W rows nw + 4g + e (e = 0..3), X row m0 + 16 mb + r16
  const int n = nw + 4 * g;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = m0 + 16 * mb + r16;
    if (m >= a.M) continue;
    if (ksplit == 1) {
      gemm_epilogue<bf16_t>(a, zb, m, n, acc[mb][0], acc[mb][1]);
      gemm_epilogue<bf16_t>(a, zb, m, n + 2, acc[mb][2], acc[mb][3]);
    } else {
      float* dst = partial + ((static_cast<int64_t>(ks) * a.batch + zb) * a.M + m) * a.N + n;
      *reinterpret_cast<f32x4_t*>(dst) = acc[mb];
    }
  }
}

// ---- X-stationary weight stream (one K slice of X held in LDS per workgroup) ----
// For one activation matrix (batch 1, M <= 64) the grid is one workgroup per CU;
// workgroup w owns K slice w % d and keeps X[:, slice] in LDS for its whole
// life, so after a one-time load the loop issues only weight loads: no X
// traffic and no barriers.  Its kXsWaves waves walk 16-row weight strips (strip
// s of the slice goes to wave s mod (kXsWaves G/d)), one strip after another with a
// kXsRing-deep load ring that runs across strip boundaries, and write each
// strip's result (or fp32 partial when d > 1) as soon as it is done.
// X layout in LDS: row r at 2 kw r bytes, 16-byte chunk c at c ^ 2(r & 7): the
// 16-row B-operand reads are bank-conflict free.
constexpr int kXsLdsBytes = 128 * 1024;
constexpr int kXsRing = 16;
constexpr int kXsWaves = 4;                     // waves per workgroup

template <typename XT, int MB>
__global__ __launch_bounds__(64 * kXsWaves, 1) void k_gemm_xs(GemmArgs a, int d, int kw,
                                                               float* partial) {
  extern __shared__ __attribute__((aligned(16))) char xs[];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n16 = lane & 15, g = lane >> 4;
  const int ks = blockIdx.x % d, wg = blockIdx.x / d, wgs = gridDim.x / d;
  const int64_t kbeg = static_cast<int64_t>(ks) * kw;
  const int nsteps = kw / 32, nstrips = a.N / 16;
  const int wave = wg * kXsWaves + wv, nwaves = wgs * kXsWaves;
  const int my = wave < nstrips ? (nstrips - 1 - wave) / nwaves + 1 : 0;
  const int rowb = 2 * kw;   // LDS bytes per X row

  // this lane's weight row in the wave's i-th strip, at the start of the slice
  // (with the fused latent append, strips from n_append on come from w3 / w4)
  auto wrow = [&](int i) -> const bf16_t* {
    const int n0 = 16 * (wave + i * nwaves);
    const bf16_t* base;
    if (a.epi == EPI_QPROJ_APPEND && n0 >= a.n_append) {
      const int r = n0 - a.n_append;
      base = r < a.n_split3
                 ? static_cast<const bf16_t*>(a.w3) + static_cast<int64_t>(r) * a.ldw_n
                 : static_cast<const bf16_t*>(a.w4) + static_cast<int64_t>(r - a.n_split3) * a.ldw_n;
    } else {
      base = n0 < a.n_split
                 ? static_cast<const bf16_t*>(a.w1) + static_cast<int64_t>(n0) * a.ldw_n
                 : static_cast<const bf16_t*>(a.w2) + static_cast<int64_t>(n0 - a.n_split) * a.ldw_n;
    }
    return base + static_cast<int64_t>(n16) * a.ldw_n + kbeg + 8 * g;
  };
  const int total = my * nsteps;   // steps of this wave over all its strips
  bf16x8_t wr[kXsRing];
  if (my > 0) {
    const bf16_t* p0 = wrow(0);
#pragma unroll
    for (int u = 0; u < kXsRing; ++u) wr[u] = ld8(p0 + 32 * min(u, nsteps - 1));
  }

  // X slice -> LDS (rows past M repeat row 0; their outputs are never stored)
  {
    const int cpr = kw / 8;   // 16-byte chunks per row
    const XT* xb = static_cast<const XT*>(a.x) + kbeg;
#pragma unroll 4
    for (int v = tid; v < 16 * MB * cpr; v += 64 * kXsWaves) {
      const int r = v / cpr, c = v - r * cpr;
      XVec<XT> t;
      t.load(xb + static_cast<int64_t>(r < a.M ? r : 0) * a.ldx_m + 8 * c);
      *reinterpret_cast<u32x4_t*>(&xs[r * rowb + 16 * (c ^ (2 * (r & 7)))]) = t.bits();
    }
  }
  __syncthreads();
  if (my == 0) return;

  // B operand of block mb at step st: row 16mb + n16, chunk 4st + g (swizzled)
  uint32_t xoff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) xoff[q] = n16 * rowb + 16 * ((4 * q + g) ^ (2 * (n16 & 7)));
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  f32x4_t acc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) acc[i] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  // operands of step 4j + q (q static): xoff[q] + 256 j, block mb at +16 rowb mb
  auto ldx = [&](int q, int j, bf16x8_t (&dst)[MB]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      dst[mb] = *reinterpret_cast<const bf16x8_t*>(&xs[xoff[q] + 256 * j + 16 * rowb * mb]);
  };
  bf16x8_t xc[MB];   // B operands of the current step, read one step ahead
  ldx(0, 0, xc);
  for (int t0 = 0; t0 < total; t0 += kXsRing) {
    // the group t0..t0+R-1 lies in strip t0 / nsteps (nsteps is a multiple of R);
    // its refills target the next group, in strip (t0+R) / nsteps (the last strip
    // re-read past the end, so the body stays branch-free)
    const int st0 = t0 % nsteps;
    const int pt = min(t0 + kXsRing, total - 1);
    const bf16_t* pp = wrow(pt / nsteps) + 32 * (pt % nsteps);
    const int plim = total - 1 - pt;   // refills past this re-read pt
    // st0 is a multiple of kXsRing: step st0 + u has q = u & 3, j = st0/4 + u/4
    const int j0 = st0 >> 2;
    const int jn = st0 + kXsRing == nsteps ? 0 : j0 + kXsRing / 4;   // first step of the next group
#pragma unroll
    for (int u = 0; u < kXsRing; ++u) {
      bf16x8_t xn[MB];
      if (u + 1 < kXsRing) ldx((u + 1) & 3, j0 + ((u + 1) >> 2), xn);
      else ldx(0, jn, xn);
      __builtin_amdgcn_sched_barrier(0);   // the reads go out a whole step before their use
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wr[u], xc[mb], acc[mb], 0, 0, 0);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) xc[mb] = xn[mb];
      // the refill reuses the slot's registers once its products are issued (a
      // load into fresh registers would force copies, and waits, at the loop edge)
      wr[u] = ld8(pp + 32 * min(u, plim));
      __builtin_amdgcn_sched_barrier(0);
    }
    if (st0 + kXsRing == nsteps) {   // strip done: lane (n16, g) holds rows n0 + 4g + e, X row 16mb + n16
      const int n = 16 * (wave + (t0 / nsteps) * nwaves) + 4 * g;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int m = 16 * mb + n16;
        if (m < a.M) {
          if (d == 1) {
            gemm_epilogue<bf16_t>(a, 0, m, n, acc[mb][0], acc[mb][1]);
            gemm_epilogue<bf16_t>(a, 0, m, n + 2, acc[mb][2], acc[mb][3]);
          } else {
            *reinterpret_cast<f32x4_t*>(partial + (static_cast<int64_t>(ks) * a.M + m) * a.N + n) =
                acc[mb];
          }
        }
        acc[mb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
      }
    }
  }
}

// Sum of the K-split partials (fixed order) followed by the output stage; each
// thread takes 4 consecutive columns of one output row.
__global__ __launch_bounds__(256) void k_gemm_finish(GemmArgs a, int ksplit, const float* partial) {
  const uint32_t quads_row = static_cast<uint32_t>(a.N) / 4;
  const uint32_t quads = static_cast<uint32_t>(a.batch) * a.M * quads_row;
  const int64_t plane = static_cast<int64_t>(a.batch) * a.M * a.N;
  for (uint32_t q = blockIdx.x * blockDim.x + threadIdx.x; q < quads; q += blockDim.x * gridDim.x) {
    const float* src = partial + static_cast<int64_t>(q) * 4;
    float4 v = *reinterpret_cast<const float4*>(src);
    // eight partials in flight at a time, summed in split order
    for (int s0 = 1; s0 < ksplit; s0 += 8) {
      float4 t[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (s0 + j < ksplit) t[j] = *reinterpret_cast<const float4*>(src + (s0 + j) * plane);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (s0 + j < ksplit) { v.x += t[j].x; v.y += t[j].y; v.z += t[j].z; v.w += t[j].w; }
    }
    const uint32_t row = q / quads_row;
    const int n = static_cast<int>(q - row * quads_row) * 4;
    const int m = static_cast<int>(row % static_cast<uint32_t>(a.M));
    const int zb = static_cast<int>(row / static_cast<uint32_t>(a.M));
    gemm_epilogue<bf16_t>(a, zb, m, n, v.x, v.y);
    gemm_epilogue<bf16_t>(a, zb, m, n + 2, v.z, v.w);
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

// ---- large-M tiled product (prefill batch sizes) ---------------------------
// For M in the hundreds and more every weight tile is worth reusing across X
// rows: a workgroup owns a 128 (n) x 128 (m) output tile and walks K in chunks of
// 64 with both operand tiles in LDS (two buffers; chunk c + 1 is loaded into
// registers while chunk c is multiplied, every load a run of whole 128-byte
// lines).  4 waves, wave (wn, wm) a 64 x 64 block of 2 x 2 mfma_f32_32x32x16_bf16
// tiles.  Weight rows are the MFMA M side and X rows its N side, so a lane ends
// with column pairs (n, n + 1) of one output row m: the epilogue's unit.
constexpr int kTt = 128, kTk = 64;   // large tile; K chunk
constexpr int kTPitch = kTk * 2 + 16;   // LDS bytes per staged row (conflict-free 16-byte reads)

// TN x TM output tile (TN, TM multiples of 64): 4 waves in 2 x 2, each wave
// TN/64 x TM/64 blocks of 32 x 32.  TN = TM = 128 for prefill-sized X; 64 x 64 for
// the per-head batched products at decode sizes, whose 128-row outputs give 2
// tiles per head.
template <typename XT, int TN, int TM>
__global__ __launch_bounds__(256, 2) void k_gemm_tile(GemmArgs a) {
  constexpr int BN = TN / 64, BM = TM / 64;   // 32-row blocks per wave
  constexpr int CW = TN / 32, CX = TM / 32;   // 16-byte chunks per thread per K chunk
  // operand tiles, buffer b: W rows at tiles[b][0], X rows after them; one array,
  // so the output tile staged at the end may span both buffers
  __shared__ __attribute__((aligned(16))) char tiles[2][(TN + TM) * kTPitch];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int z = blockIdx.z, n0 = blockIdx.x * TN, m0 = blockIdx.y * TM;
  // staging: thread t moves 16-byte chunks c = t + 256 j of each tile: row c >> 3,
  // k 8 (c & 7); rows past N or M re-read the last row (never stored)
  const bf16_t* wp[CW];
  const XT* xp[CX];
#pragma unroll
  for (int j = 0; j < CW; ++j) {
    const int c = tid + 256 * j, r = c >> 3, kc = 8 * (c & 7);
    const int n = min(n0 + r, a.N - 1);
    wp[j] = (n < a.n_split ? static_cast<const bf16_t*>(a.w1) + static_cast<int64_t>(n) * a.ldw_n
                           : static_cast<const bf16_t*>(a.w2) +
                                 static_cast<int64_t>(n - a.n_split) * a.ldw_n) +
            static_cast<int64_t>(z) * a.w_bs + kc;
  }
#pragma unroll
  for (int j = 0; j < CX; ++j) {
    const int c = tid + 256 * j, r = c >> 3, kc = 8 * (c & 7);
    const int m = min(m0 + r, a.M - 1);
    xp[j] = static_cast<const XT*>(a.x) + static_cast<int64_t>(z) * a.x_bs +
            static_cast<int64_t>(m) * a.ldx_m + kc;
  }
  // two register sets of staged chunks: chunk c is loaded into set c & 1 two steps
  // before it is multiplied (so two chunks are in flight while one is multiplied)
  u32x4_t wreg[2][CW];
  XVec<XT> xreg[2][CX];
  auto gload = [&](auto set_c, int k0) {
    constexpr int st = decltype(set_c)::value;
#pragma unroll
    for (int j = 0; j < CW; ++j) wreg[st][j] = *reinterpret_cast<const u32x4_t*>(wp[j] + k0);
#pragma unroll
    for (int j = 0; j < CX; ++j) xreg[st][j].load(xp[j] + k0);
  };
  auto lstore = [&](auto set_c, int buf) {
    constexpr int st = decltype(set_c)::value;
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      const int c = tid + 256 * j;
      *reinterpret_cast<u32x4_t*>(&tiles[buf][(c >> 3) * kTPitch + 16 * (c & 7)]) = wreg[st][j];
    }
#pragma unroll
    for (int j = 0; j < CX; ++j) {
      const int c = tid + 256 * j;
      *reinterpret_cast<u32x4_t*>(&tiles[buf][(TN + (c >> 3)) * kTPitch + 16 * (c & 7)]) =
          xreg[st][j].bits();
    }
  };
  const int wn = wv & 1, wm = wv >> 1, r32 = lane & 31, h = lane >> 5;
  // operand of 32-row block i at k-step s: row 32i + r32 of the wave's half, k 16s + 8h
  const int aoff = (32 * BN * wn + r32) * kTPitch + 16 * h;
  const int boff = (TN + 32 * BM * wm + r32) * kTPitch + 16 * h;
  f32x16_t acc[BN][BM];
#pragma unroll
  for (int i = 0; i < BN; ++i)
#pragma unroll
    for (int j = 0; j < BM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  auto multiply = [&](int buf) {
#pragma unroll
    for (int s = 0; s < kTk / 16; ++s) {
      bf16x8_t af[BN], bf[BM];
#pragma unroll
      for (int i = 0; i < BN; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(&tiles[buf][aoff + 32 * i * kTPitch + 32 * s]);
#pragma unroll
      for (int j = 0; j < BM; ++j)
        bf[j] = *reinterpret_cast<const bf16x8_t*>(&tiles[buf][boff + 32 * j * kTPitch + 32 * s]);
#pragma unroll
      for (int i = 0; i < BN; ++i)
#pragma unroll
        for (int j = 0; j < BM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  const int nk = a.K / kTk;
  gload(S0{}, 0);
  if (nk > 1) gload(S1{}, kTk);
  lstore(S0{}, 0);
  __syncthreads();
  // step c multiplies buffer c & 1 (chunk c); before that, chunk c + 2 is loaded
  // into the register set chunk c came from, and after it chunk c + 1 goes from its
  // set into the other buffer (last read before the previous barrier)
  for (int kb = 0; kb < nk; kb += 2) {
    if (kb + 2 < nk) gload(S0{}, (kb + 2) * kTk);
    multiply(0);
    if (kb + 1 < nk) lstore(S1{}, 1);
    __syncthreads();
    if (kb + 1 >= nk) break;
    if (kb + 3 < nk) gload(S1{}, (kb + 3) * kTk);
    multiply(1);
    if (kb + 2 < nk) lstore(S0{}, 0);
    __syncthreads();
  }
  // acc[i][j] element e of lane (r32, h): row 32 BM wm + 32j + r32, column
  // 32 BN wn + 32i + 8(e >> 2) + 4h + (e & 3) of the tile.  The tile goes to LDS (the
  // operand buffers are free after the last barrier) and a compact loop applies the
  // epilogue to column pairs: unrolled over the accumulators, the epilogue's
  // registers made the compiler spill the accumulators on every K step.
  constexpr int kOPitch = TN + 4;   // floats per staged output row
  static_assert(TM * kOPitch * 4 <= static_cast<int>(sizeof(tiles)), "output tile fits the operand buffers");
  float* ot = reinterpret_cast<float*>(&tiles[0][0]);
#pragma unroll
  for (int j = 0; j < BM; ++j)
#pragma unroll
    for (int i = 0; i < BN; ++i)
#pragma unroll
      for (int e = 0; e < 16; e += 2)
        *reinterpret_cast<float2*>(&ot[(32 * BM * wm + 32 * j + r32) * kOPitch + 32 * BN * wn + 32 * i +
                                       8 * (e >> 2) + 4 * h + (e & 3)]) =
            make_float2(acc[i][j][e], acc[i][j][e + 1]);
  __syncthreads();
  for (int q = tid; q < TM * TN / 2; q += 256) {   // pair q: row q / (TN/2), columns 2 (q % (TN/2)), +1
    const int ml = q / (TN / 2), nl = 2 * (q % (TN / 2));
    const int m = m0 + ml, n = n0 + nl;
    if (m < a.M && n < a.N) {
      const float2 v = *reinterpret_cast<const float2*>(&ot[ml * kOPitch + nl]);
      gemm_epilogue<bf16_t>(a, z, m, n, v.x, v.y);
    }
  }
}

constexpr int kWsMinGroups = 512;   // workgroups wanted before K is split further

struct WsPlan {
  int mb, mtiles, ntiles, d;
};

WsPlan ws_plan(const GemmArgs& a) {
  WsPlan p{};
  p.mb = ws_mb(a.M);
  p.mtiles = (a.M + 16 * p.mb - 1) / (16 * p.mb);
  p.ntiles = a.N / kWsTile;
  const int64_t tiles = static_cast<int64_t>(a.batch) * p.ntiles * p.mtiles;
  const int groups = a.K / ws_kunit(p.mb);
  // smallest divisor of the K granules that reaches the workgroup target
  p.d = 1;
  for (int d = 1; d <= groups; ++d) {
    if (groups % d) continue;
    p.d = d;
    if (tiles * d >= kWsMinGroups) break;
  }
  return p;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <typename XT>
void launch_ws(const GemmArgs& a, const WsPlan& p, float* partial, hipStream_t stream) {
  const dim3 grid(a.batch * p.ntiles, p.d, p.mtiles);
  const int kslice = a.K / p.d;
  switch (p.mb) {
    case 1: hipLaunchKernelGGL((k_gemm_ws<XT, 1>), grid, dim3(256), 0, stream, a, p.ntiles, p.d, kslice, partial); break;
    case 2: hipLaunchKernelGGL((k_gemm_ws<XT, 2>), grid, dim3(256), 0, stream, a, p.ntiles, p.d, kslice, partial); break;
    case 4: hipLaunchKernelGGL((k_gemm_ws<XT, 4>), grid, dim3(256), 0, stream, a, p.ntiles, p.d, kslice, partial); break;
    default: hipLaunchKernelGGL((k_gemm_ws<XT, 8>), grid, dim3(256), 0, stream, a, p.ntiles, p.d, kslice, partial); break;
  }
}

// Sum of d fp32 partials + output stage; small outputs use 64-thread blocks so
// that the (latency-bound) sums spread over more CUs.
hipError_t launch_finish(const GemmArgs& a, int d, const float* partial, hipStream_t stream) {
  const int64_t quads = static_cast<int64_t>(a.batch) * a.M * (a.N / 4);
  const int threads = quads < 65536 ? 64 : 256;
  const int blocks = static_cast<int>(std::min<int64_t>((quads + threads - 1) / threads, 8192));
  hipLaunchKernelGGL(k_gemm_finish, dim3(blocks), dim3(threads), 0, stream, a, d, partial);
  return hipGetLastError();
}

struct XsPlan {
  int mb, d, kw;
};

XsPlan xs_plan(const GemmArgs& a) {
  XsPlan p{};
  p.mb = a.M <= 16 ? 1 : a.M <= 32 ? 2 : 4;
  // slices are whole groups of 32 * kXsRing k (a strip's steps fill whole ring turns)
  constexpr int kUnit = 32 * kXsRing;
  const int kw_max = kXsLdsBytes / (2 * 16 * p.mb) / kUnit * kUnit;
  const int groups = a.K / kUnit;
  p.d = groups;
  for (int d = 1; d <= groups; ++d)
    if (groups % d == 0 && a.K / d <= kw_max) { p.d = d; break; }
  p.kw = a.K / p.d;
  return p;
}

int cu_count() {
  static std::atomic<int> cached{0};
  int v = cached.load(std::memory_order_relaxed);
  if (v > 0) return v;
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess ||
      prop.multiProcessorCount < 1)
    return 256;
  cached.store(prop.multiProcessorCount, std::memory_order_relaxed);
  return prop.multiProcessorCount;
}

template <typename XT, int MB>
hipError_t launch_xs_inst(const GemmArgs& a, const XsPlan& p, float* partial, hipStream_t stream) {
  static std::atomic<int> attr_set{0};
  if (!attr_set.load(std::memory_order_acquire)) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_xs<XT, MB>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             kXsLdsBytes);
    if (e != hipSuccess) return e;
    attr_set.store(1, std::memory_order_release);
  }
  const int grid = std::max(1, cu_count() / p.d) * p.d;
  const size_t lds = static_cast<size_t>(16 * MB) * p.kw * 2;
  hipLaunchKernelGGL((k_gemm_xs<XT, MB>), dim3(grid), dim3(64 * kXsWaves), lds, stream, a, p.d, p.kw,
                     partial);
  return hipGetLastError();
}

hipError_t launch_xs(const GemmArgs& a, const XsPlan& p, float* partial, hipStream_t stream) {
  if (a.x_f32) {
    if (p.mb == 1) return launch_xs_inst<float, 1>(a, p, partial, stream);
    if (p.mb == 2) return launch_xs_inst<float, 2>(a, p, partial, stream);
    return launch_xs_inst<float, 4>(a, p, partial, stream);
  }
  if (p.mb == 1) return launch_xs_inst<bf16_t, 1>(a, p, partial, stream);
  if (p.mb == 2) return launch_xs_inst<bf16_t, 2>(a, p, partial, stream);
  return launch_xs_inst<bf16_t, 4>(a, p, partial, stream);
}

}  // namespace

// NT form: W and X K-contiguous, 16-byte aligned rows, 64-row W tiles that do
// not straddle the W1/W2 boundary, K a multiple of the instance's k granule.
static bool ws_ok(const GemmArgs& a) {
  if (!(a.ldw_k == 1 && a.ldx_k == 1 && a.K > 0 && a.M > 0 && a.N > 0 && a.batch > 0 &&
        a.N % kWsTile == 0 && (a.n_split % kWsTile == 0 || a.n_split >= a.N) &&
        a.ldw_n % 8 == 0 && a.ldx_m % 8 == 0 && a.x_bs % 8 == 0 && a.w_bs % 8 == 0 &&
        aligned16(a.x) && aligned16(a.w1) && aligned16(a.w2)))
    return false;
  if (static_cast<int64_t>(a.batch) * a.M * a.N >= (int64_t{1} << 31)) return false;
  return a.K % ws_kunit(ws_mb(a.M)) == 0;
}

// The per-head W_UK form: W is [K=128, N] N-contiguous, output fp32.
static bool uk_ok(const GemmArgs& a) {
  return a.ldw_n == 1 && a.ldw_k % 8 == 0 && a.K == kUkK && a.N % kUkN == 0 && a.ldx_k == 1 &&
         !a.x_f32 && a.y_f32 && a.epi == EPI_STORE && a.ldx_m % 8 == 0 && a.x_bs % 8 == 0 &&
         a.w1 == a.w2 && a.n_split >= a.N;
}

// One activation matrix of at most 64 rows and enough weight rows to give every
// wave of the grid strips to stream (narrow outputs, like the 576-wide latent
// append, leave most waves idle there and go to k_gemm_ws): the X-stationary kernel.
static bool xs_ok(const GemmArgs& a) {
  if (a.epi == EPI_QPROJ_APPEND &&
      !(a.n_append % 16 == 0 && a.n_split3 % 16 == 0 && a.n_split < a.n_append))
    return false;
  return ws_ok(a) && a.batch == 1 && a.M <= 64 && a.N >= 2048 && a.N % 16 == 0 &&
         (a.n_split % 16 == 0 || a.n_split >= a.N) && a.K % (32 * kXsRing) == 0;
}

// The fused query projection + latent append runs only on k_gemm_xs.
bool fused_qa_ok(const GemmArgs& a) { return a.epi == EPI_QPROJ_APPEND && xs_ok(a); }

// Prefill-sized activations (M >= 256): the tiled product.  Same operand forms as
// k_gemm_ws; K a multiple of the 64-wide chunk.
static bool tile_ok(const GemmArgs& a) {
  const int64_t groups = static_cast<int64_t>((a.N + kTt - 1) / kTt) * ((a.M + kTt - 1) / kTt) * a.batch;
  // grids of fewer than 256 output tiles (narrow outputs such as the latent append)
  // would leave most of the chip idle: those stay with the K-split weight stream
  return ws_ok(a) && a.epi != EPI_QPROJ_APPEND && a.M >= 256 && a.K % kTk == 0 &&
         a.n_split % 2 == 0 && groups >= 256;
}

// Per-head batched products at decode sizes (M <= 64, N a multiple of 64): one
// 64 x 64 tile per workgroup, no K split, when that gives at least 256 workgroups.
static bool small_tile_ok(const GemmArgs& a) {
  return ws_ok(a) && a.epi == EPI_STORE && a.batch > 1 && a.M <= 64 && a.N % 64 == 0 &&
         a.K % kTk == 0 && static_cast<int64_t>(a.N / 64) * a.batch >= 256;
}

bool fast_gemm_ok(const GemmArgs& a) { return ws_ok(a) || uk_ok(a); }

size_t gemm_partial_bytes(const GemmArgs& a) {
  if (!ws_ok(a) || tile_ok(a) || small_tile_ok(a)) return 0;
  if (xs_ok(a)) {
    const XsPlan q = xs_plan(a);
    return q.d > 1 ? static_cast<size_t>(q.d) * a.M * a.N * sizeof(float) : 0;
  }
  const WsPlan p = ws_plan(a);
  return p.d > 1 ? static_cast<size_t>(p.d) * a.batch * a.M * a.N * sizeof(float) : 0;
}

hipError_t launch_gemm_fast(const GemmArgs& a, void* partial, size_t partial_bytes,
                            hipStream_t stream) {
  if (a.M == 0 || a.N == 0 || a.batch == 0) return hipSuccess;
  if (a.epi == EPI_QPROJ_APPEND && !xs_ok(a)) return hipErrorInvalidValue;
  if (!ws_ok(a)) {
    if (!uk_ok(a)) return hipErrorInvalidValue;
    dim3 grid(a.batch, a.N / kUkN, (a.M + kTile - 1) / kTile);
    hipLaunchKernelGGL(k_gemm_uk, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  if (tile_ok(a)) {
    const dim3 grid((a.N + kTt - 1) / kTt, (a.M + kTt - 1) / kTt, a.batch);
    if (a.x_f32)
      hipLaunchKernelGGL((k_gemm_tile<float, kTt, kTt>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((k_gemm_tile<bf16_t, kTt, kTt>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  if (small_tile_ok(a)) {
    const dim3 grid(a.N / 64, 1, a.batch);
    if (a.x_f32)
      hipLaunchKernelGGL((k_gemm_tile<float, 64, 64>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((k_gemm_tile<bf16_t, 64, 64>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  if (xs_ok(a)) {
    const XsPlan q = xs_plan(a);
    if (q.d > 1 && (partial == nullptr || !aligned16(partial) ||
                    partial_bytes < gemm_partial_bytes(a)))
      return hipErrorInvalidValue;
    hipError_t e = launch_xs(a, q, static_cast<float*>(partial), stream);
    if (e != hipSuccess || q.d == 1) return e;
    return launch_finish(a, q.d, static_cast<const float*>(partial), stream);
  }
  const WsPlan p = ws_plan(a);
  if (p.d > 1 && (partial == nullptr || !aligned16(partial) ||
                  partial_bytes < gemm_partial_bytes(a)))
    return hipErrorInvalidValue;
  if (a.x_f32)
    launch_ws<float>(a, p, static_cast<float*>(partial), stream);
  else
    launch_ws<bf16_t>(a, p, static_cast<float*>(partial), stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.d == 1) return e;
  return launch_finish(a, p.d, static_cast<const float*>(partial), stream);
}

}  // namespace mla
