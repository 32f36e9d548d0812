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
#include "lds_copy.hpp"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

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

// cos/sin of the RoPE angles of the output rows, (pos[m], pair k) at
// rope_tab[2 (m d_R/2 + k)], computed once per call by the K-split weight stream
// (strided over the grid's threads) for its output stage in k_gemm_finish_xs,
// which would otherwise evaluate them once per head.
__device__ __forceinline__ void rope_table_fill(const GemmArgs& a, int e0, int stride) {
  if (a.rope_tab == nullptr) return;
  for (int e = e0; e < a.M * (a.d_rope / 2); e += stride) {
    const int m = e / (a.d_rope / 2), k = e - m * (a.d_rope / 2);
    float c, sn;
    rope_cs(a.pos[m], k, a.d_rope, a.rope, &c, &sn);
    a.rope_tab[2 * e] = c;
    a.rope_tab[2 * e + 1] = sn;
  }
}

// The same table as a kernel of its own, ahead of a tiled product whose output
// stage rotates (otherwise each of its RoPE tiles would evaluate the fp64 angles
// of every (row, pair) it holds).
__global__ __launch_bounds__(256) void k_rope_table(GemmArgs a) {
  rope_table_fill(a, blockIdx.x * blockDim.x + threadIdx.x, gridDim.x * blockDim.x);
}

// ---- X-stationary weight stream (one K slice of X held in LDS per workgroup) ----
// For one activation matrix (batch 1, M <= 64) the grid is one workgroup per CU;
// workgroup w owns K slice w % d and keeps X[:, slice] in LDS for its whole
// life, so after a one-time load the loop issues only weight loads: no X
// traffic and no barriers.  Its kXsWaves waves walk 16-row weight strips (strip
// s of the slice goes to wave s mod (kXsWaves G/d)), one strip after another with an
// R-deep load ring that runs across strip boundaries, and write each
// strip's result (or fp32 partial when d > 1) as soon as it is done.
// X layout in LDS: row r at 2 kw r bytes, 16-byte chunk c at c ^ 2(r & 7): the
// 16-row B-operand reads are bank-conflict free.  A bf16 X slice arrives by
// asynchronous copies (1 KB per wave instruction, all of them in flight at once);
// an fp32 X is converted in registers on the way.
constexpr int kXsLdsBytes = 128 * 1024;   // the largest X slice
constexpr int kXsWaves = 4;                     // waves per workgroup

// kSplit (d > 1): the strip results are fp32 partials, and the instance holds no
// output-stage code at all (the compiler would otherwise evaluate parts of it,
// such as the RoPE angles, on every strip end before testing d).
template <typename XT, int MB, int R, bool kSplit>
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
  bf16x8_t wr[R];
  if (my > 0) {
    const bf16_t* p0 = wrow(0);
#pragma unroll
    for (int u = 0; u < R; ++u) wr[u] = ld8(p0 + 32 * min(u, nsteps - 1));
  }

  // X slice -> LDS (rows past M repeat row 0; their outputs are never stored)
  if constexpr (std::is_same<XT, bf16_t>::value) {
    // LDS block j (1 KB) is one copy: lane l fills bytes 1024 j + 16 l, i.e. row
    // r, stored chunk cs, which holds source chunk cs ^ 2(r & 7)
    const int nblk = 16 * MB * rowb / 1024;
    const uint64_t xg = reinterpret_cast<uint64_t>(static_cast<const bf16_t*>(a.x) + kbeg);
    const uint32_t x0 = lds_addr(xs);
    for (int j = wv; j < nblk; j += kXsWaves) {
      const int byte = 1024 * j + 16 * lane;
      const int r = byte / rowb, cs = (byte - r * rowb) >> 4;
      const uint32_t voff = static_cast<uint32_t>(
          (static_cast<int64_t>(r < a.M ? r : 0) * a.ldx_m + 8 * (cs ^ (2 * (r & 7)))) * 2);
      dma_block(xg, voff, x0 + 1024 * j);
    }
    wait_vmcnt<0>();
    lds_barrier();
  } else {
    const int cpr = kw / 8;   // 16-byte chunks per row
    const XT* xb = static_cast<const XT*>(a.x) + kbeg;
#pragma unroll 8
    for (int v = tid; v < 16 * MB * cpr; v += 64 * kXsWaves) {
      const int r = v / cpr, c = v - r * cpr;
      XVec<XT> t;
      t.load(xb + static_cast<int64_t>(r < a.M ? r : 0) * a.ldx_m + 8 * c);
      *reinterpret_cast<u32x4_t*>(&xs[r * rowb + 16 * (c ^ (2 * (r & 7)))]) = t.bits();
    }
    __syncthreads();
  }
  // the RoPE table (split instances): entry blockIdx + grid * tid, once the
  // thread's strips are done (the fp64 angles would otherwise stall the stream)
  const int tab_e = blockIdx.x + gridDim.x * tid, tab_stride = gridDim.x * blockDim.x;
  if (my == 0) {
    if constexpr (kSplit) rope_table_fill(a, tab_e, tab_stride);
    return;
  }

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
  for (int t0 = 0; t0 < total; t0 += R) {
    // the group t0..t0+R-1 lies in strip t0 / nsteps (nsteps is a multiple of R);
    // its refills target the next group, in strip (t0+R) / nsteps (the last strip
    // re-read past the end, so the body stays branch-free)
    const int st0 = t0 % nsteps;
    const int pt = min(t0 + R, total - 1);
    const bf16_t* pp = wrow(pt / nsteps) + 32 * (pt % nsteps);
    const int plim = total - 1 - pt;   // refills past this re-read pt
    // st0 is a multiple of R: step st0 + u has q = u & 3, j = st0/4 + u/4
    const int j0 = st0 >> 2;
    const int jn = st0 + R == nsteps ? 0 : j0 + R / 4;   // first step of the next group
#pragma unroll
    for (int u = 0; u < R; ++u) {
      bf16x8_t xn[MB];
      if (u + 1 < R) ldx((u + 1) & 3, j0 + ((u + 1) >> 2), xn);
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
    if (st0 + R == nsteps) {   // strip done: lane (n16, g) holds rows n0 + 4g + e, X row 16mb + n16
      const int strip = wave + (t0 / nsteps) * nwaves;
      const int n = 16 * strip + 4 * g;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int m = 16 * mb + n16;
        if (m < a.M) {
          if constexpr (!kSplit) {
            gemm_epilogue<bf16_t>(a, 0, m, n, acc[mb][0], acc[mb][1]);
            gemm_epilogue<bf16_t>(a, 0, m, n + 2, acc[mb][2], acc[mb][3]);
          } else {
            // partial tile of (slice, strip): [16 MB rows m][16 columns], 1 KB per block
            float* tile = partial + (static_cast<int64_t>(ks) * nstrips + strip) * (256 * MB);
            *reinterpret_cast<f32x4_t*>(tile + 16 * m + 4 * g) = acc[mb];
          }
        }
        acc[mb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
      }
    }
  }
  if constexpr (kSplit) rope_table_fill(a, tab_e, tab_stride);
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

// Sum of the K-split partial tiles of k_gemm_xs (fixed order) followed by the
// output stage.  Thread q takes 4 columns of one row: strip q / (4 M) (rotated so
// that the latent-append strips, whose stores wait on a page lookup, go first),
// row (q / 4) mod M, columns 4 (q mod 4)..+3 of the strip, so that a wave reads
// whole 1 KB pieces of a tile.
__global__ __launch_bounds__(256) void k_gemm_finish_xs(GemmArgs a, int ksplit, int rows_pad,
                                                        const float* partial) {
  const uint32_t per_strip = static_cast<uint32_t>(a.M) * 4;
  const uint32_t nstrips = static_cast<uint32_t>(a.N) / 16;
  const uint32_t quads = nstrips * per_strip;
  const int64_t plane = static_cast<int64_t>(nstrips) * rows_pad * 16;   // one slice
  const uint32_t first = a.epi == EPI_QPROJ_APPEND ? static_cast<uint32_t>(a.n_append) / 16 : 0;
  for (uint32_t q = blockIdx.x * blockDim.x + threadIdx.x; q < quads; q += blockDim.x * gridDim.x) {
    const uint32_t qs = q / per_strip, r = q - qs * per_strip;
    const uint32_t strip = qs + first < nstrips ? qs + first : qs + first - nstrips;
    const int m = static_cast<int>(r >> 2), g = static_cast<int>(r & 3);
    const float* src = partial + static_cast<int64_t>(strip) * rows_pad * 16 + 16 * m + 4 * g;
    float4 v = *reinterpret_cast<const float4*>(src);
    for (int s0 = 1; s0 < ksplit; s0 += 8) {   // eight partials in flight, summed in slice order
      float4 t[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (s0 + j < ksplit) t[j] = *reinterpret_cast<const float4*>(src + (s0 + j) * plane);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (s0 + j < ksplit) { v.x += t[j].x; v.y += t[j].y; v.z += t[j].z; v.w += t[j].w; }
    }
    gemm_epilogue4<bf16_t>(a, 0, m, 16 * static_cast<int>(strip) + 4 * g, v);
  }
}

// ---- per-head q_lat[b, i, c] = sum_d X[b, i*d_h + d] W_UK[i*d_h + d, c] ----
// Workgroup = (head, 128 columns c, 64 rows b); K = d_h = 128.  The W tile
// [128 d x 128 c] is staged in LDS (rows padded by 16 bytes) and read as the
// MFMA A operand (M = c) with transposed reads; X rows are the B operand (N = b).
constexpr int kUkK = 128, kUkN = 128, kUkPad = kUkN * 2 + 16;   // LDS row bytes

// An fp32 X (the absorbed query's q^C) enters as two bf16 terms, hi = RNE(x) and
// lo = RNE(x - hi), each multiplied with the same W operand: the product is then
// exact to about 2^-16 of x instead of bf16's 2^-8.
template <typename XT>
__global__ __launch_bounds__(256) void k_gemm_uk(GemmArgs a) {
  constexpr bool kSplit = std::is_same<XT, float>::value;
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
  const XT* xb = static_cast<const XT*>(a.x) + head * a.x_bs;
  bf16x8_t xf[2][kUkK / 16];
  bf16x8_t xl[kSplit ? 2 : 1][kSplit ? kUkK / 16 : 1];   // lo terms of an fp32 X
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int m = m0 + 32 * q + r;
    const XT* row = xb + static_cast<int64_t>(m < a.M ? m : 0) * a.ldx_m;
#pragma unroll
    for (int s = 0; s < kUkK / 16; ++s) {
      if constexpr (kSplit) {
        const float4 v0 = *reinterpret_cast<const float4*>(row + 16 * s + 8 * g);
        const float4 v1 = *reinterpret_cast<const float4*>(row + 16 * s + 8 * g + 4);
        const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        const u32x4_t hi = {cvt2(v[0], v[1]), cvt2(v[2], v[3]), cvt2(v[4], v[5]), cvt2(v[6], v[7])};
        float rl[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          rl[2 * j] = v[2 * j] - __uint_as_float(hi[j] << 16);
          rl[2 * j + 1] = v[2 * j + 1] - __uint_as_float(hi[j] & 0xFFFF0000u);
        }
        const u32x4_t lo = {cvt2(rl[0], rl[1]), cvt2(rl[2], rl[3]), cvt2(rl[4], rl[5]),
                            cvt2(rl[6], rl[7])};
        xf[q][s] = __builtin_bit_cast(bf16x8_t, hi);
        xl[q][s] = __builtin_bit_cast(bf16x8_t, lo);
      } else {
        xf[q][s] = ld8(row + 16 * s + 8 * g);
      }
    }
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
    for (int q = 0; q < 2; ++q) {
      acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, xf[q][s], acc[q], 0, 0, 0);
      if constexpr (kSplit)
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, xl[q][s], acc[q], 0, 0, 0);
    }
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

// ---- the same product for an fp32 X, with asynchronous copies ---------------
// Workgroup = (head, NW columns c, 64 rows b): the W tile [128 d x NW c] and the
// fp32 X tile [64 b x 128 d] (32 KB) arrive by asynchronous copies of 1 KB, all
// in flight at once, and the output tile leaves through the same LDS as whole
// rows.  LDS layouts (16-byte chunks swizzled so that no read phase puts two
// addresses on one bank):
//   W: row d at 2 NW d, chunk q (8 columns) at q ^ 4(d & 3); A fragments by
//      transposed reads, four rows by four column quads per 16-lane group
//   X: row b at 512 b, chunk q (4 values) at q ^ (b & 15); B fragments as two
//      16-byte reads per lane, split into hi + lo bf16 terms
//   Y: row b at 4 NW b, chunk q (4 columns) at q ^ (b & 15)
// Wave w computes the NW / 128 column tiles (32 columns each) from 32 NW w / 128
// for both 32-row halves of b.  NW = 128 keeps two workgroups on a CU (64 KB of
// LDS each), so that one's copies overlap the other's products and stores.
constexpr int kUwM = 64;
__device__ __forceinline__ s16x4_t lds_tr16_u(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) s16x4_t*>(static_cast<uintptr_t>(addr)));
}
__device__ __forceinline__ u32x4_t lds_u128(uint32_t addr) {
  return *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(static_cast<uintptr_t>(addr));
}
__device__ __forceinline__ void lds_st128(uint32_t addr, u32x4_t v) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(static_cast<uintptr_t>(addr)) = v;
}

template <int NW>
__global__ __launch_bounds__(256, 2) void k_gemm_uk_wide(GemmArgs a) {
  constexpr int kWRow = 2 * NW, kWBytes = kUkK * kWRow, kCT = NW / 128;
  constexpr int kYRow = 4 * NW;
  static_assert(kUwM * kYRow <= kWBytes, "output staging fits the W region");
  __shared__ __attribute__((aligned(1024))) char lds[kWBytes + kUwM * 512];   // W, then X
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int head = blockIdx.x, c0 = blockIdx.y * NW, m0 = blockIdx.z * kUwM;
  const uint32_t wl = lds_addr(lds), xl = wl + kWBytes;

  // ---- copies: 1 KB blocks; W block j = rows (1024 / kWRow) j .., X block j = rows 2j, 2j+1
  {
    const uint64_t wg = reinterpret_cast<uint64_t>(static_cast<const bf16_t*>(a.w1) +
                                                   head * a.w_bs + c0);
    const uint64_t xg = reinterpret_cast<uint64_t>(static_cast<const float*>(a.x) +
                                                   head * a.x_bs + static_cast<int64_t>(m0) * a.ldx_m);
    constexpr int kQW = NW / 8;   // 16-byte chunks per W row
    for (int j = wv; j < kWBytes / 1024; j += 4) {
      const int byte = 1024 * j + 16 * lane;
      const int d = byte / kWRow, qs = (byte % kWRow) >> 4;
      const uint32_t voff = static_cast<uint32_t>((static_cast<int64_t>(d) * a.ldw_k +
                                                   8 * (qs ^ (4 * (d & 3)))) * 2);
      dma_block(wg, voff, wl + 1024 * j);
      static_assert(kQW % 16 == 0, "swizzle stays inside a row");
    }
    for (int j = wv; j < kUwM / 2; j += 4) {
      const int b = 2 * j + (lane >> 5), qs = lane & 31;
      const int br = m0 + b < a.M ? b : a.M - 1 - m0;   // rows past M repeat the last one
      const uint32_t voff = static_cast<uint32_t>((static_cast<int64_t>(br) * a.ldx_m +
                                                   4 * (qs ^ (b & 15))) * 4);
      dma_block(xg, voff, xl + 1024 * j);
    }
    wait_vmcnt<0>();
    lds_barrier();
  }

  // ---- products: acc[ct][mt], column tile kCT wv + ct, row half mt
  const int i16 = lane & 15, G = lane >> 4, j32 = lane & 31, g = lane >> 5;
  f32x16_t acc[kCT][2];
#pragma unroll
  for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[ct][mt][e] = 0.f;
#pragma unroll 2
  for (int s = 0; s < kUkK / 16; ++s) {
    // A (W^T): lane group G: columns +16(G & 1) + 4(i16 & 3), rows 16s + 8(G >> 1) + (i16 >> 2) (+4)
    bf16x8_t af[kCT];
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) {
      const int col = 32 * (kCT * wv + ct) + 16 * (G & 1) + 4 * (i16 & 3);
      const int d = 16 * s + 8 * (G >> 1) + (i16 >> 2);
      const int q = col >> 3, h8 = 8 * ((col >> 2) & 1);
      const s16x4_t v0 = lds_tr16_u(wl + kWRow * d + 16 * (q ^ (4 * (d & 3))) + h8);
      const s16x4_t v1 = lds_tr16_u(wl + kWRow * (d + 4) + 16 * (q ^ (4 * ((d + 4) & 3))) + h8);
      const s16x4_t vv[2] = {v0, v1};
      af[ct] = __builtin_bit_cast(bf16x8_t, vv);
    }
    // B (X^T): lane (row 32mt + j32, k group g): values 16s + 8g .. +7 as hi + lo
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int b = 32 * mt + j32;
      const int q = 4 * s + 2 * g;
      const u32x4_t x0 = lds_u128(xl + 512 * b + 16 * (q ^ (b & 15)));
      const u32x4_t x1 = lds_u128(xl + 512 * b + 16 * ((q + 1) ^ (b & 15)));
      float v[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = __uint_as_float(x0[e]);
        v[4 + e] = __uint_as_float(x1[e]);
      }
      const u32x4_t hi = {cvt2(v[0], v[1]), cvt2(v[2], v[3]), cvt2(v[4], v[5]), cvt2(v[6], v[7])};
      float rl[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rl[2 * e] = v[2 * e] - __uint_as_float(hi[e] << 16);
        rl[2 * e + 1] = v[2 * e + 1] - __uint_as_float(hi[e] & 0xFFFF0000u);
      }
      const u32x4_t lo = {cvt2(rl[0], rl[1]), cvt2(rl[2], rl[3]), cvt2(rl[4], rl[5]),
                          cvt2(rl[6], rl[7])};
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
        acc[ct][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ct], __builtin_bit_cast(bf16x8_t, hi),
                                                              acc[ct][mt], 0, 0, 0);
        acc[ct][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ct], __builtin_bit_cast(bf16x8_t, lo),
                                                              acc[ct][mt], 0, 0, 0);
      }
    }
  }

  // ---- output: stage in the W region (every wave done with it), then whole rows
  __syncthreads();
  // acc[ct][mt] lane (j32, g): columns 32(kCT wv + ct) + 8(e >> 2) + 4g + (e & 3), row 32mt + j32
#pragma unroll
  for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int b = 32 * mt + j32;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int q = (32 * (kCT * wv + ct) + 8 * e4 + 4 * g) >> 2;
        const u32x4_t v = {__float_as_uint(acc[ct][mt][4 * e4]), __float_as_uint(acc[ct][mt][4 * e4 + 1]),
                           __float_as_uint(acc[ct][mt][4 * e4 + 2]), __float_as_uint(acc[ct][mt][4 * e4 + 3])};
        lds_st128(wl + kYRow * b + 16 * (q ^ (b & 15)), v);
      }
    }
  __syncthreads();
  // one 1 KB store per wave instruction: rows 1024 / kYRow at a time
  float* y = static_cast<float*>(a.y) + head * a.y_bs + c0;
  constexpr int kRowsPer = 1024 / kYRow, kLanesRow = kYRow / 16;
  for (int r0 = kRowsPer * wv; r0 < kUwM; r0 += 4 * kRowsPer) {
    const int b = r0 + lane / kLanesRow, q = lane % kLanesRow;
    if (m0 + b < a.M) {
      const u32x4_t v = lds_u128(wl + kYRow * b + 16 * (q ^ (b & 15)));
      *reinterpret_cast<u32x4_t*>(y + static_cast<int64_t>(m0 + b) * a.ldy + 4 * q) = v;
    }
  }
}

constexpr int kUwN = 256;   // columns per workgroup of the fp32-X W_UK product

// ---- the same product for batches of several 64-row tiles ----------------------
// Workgroup = (head, NW columns c) for all the rows: the W tile is copied to LDS
// once and stays; the fp32 X tiles of the rows pass through two LDS buffers, the
// next tile's copies in flight during the current tile's products, and each lane
// stores its outputs straight from the accumulators (four columns, 16 bytes).  The
// products are k_gemm_uk_wide's, in the same order (bit-identical q_lat); one
// workgroup per (head, column tile) instead of one per row tile as well, so at 256
// and 1024 rows the W tiles are read once and the grid is one round.
template <int NW>
__global__ __launch_bounds__(256, 1) void k_gemm_uk_rows(GemmArgs a) {
  constexpr int kWRow = 2 * NW, kWBytes = kUkK * kWRow, kCT = NW / 128;
  constexpr int kXBytes = kUwM * 512;               // one fp32 X tile: 64 rows x 128 d
  constexpr int kXPerWave = kXBytes / 1024 / 4;     // copies of one X tile per wave
  __shared__ __attribute__((aligned(1024))) char lds[kWBytes + 2 * kXBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int head = blockIdx.x, c0 = blockIdx.y * NW;
  const uint32_t wl = lds_addr(lds), xl0 = wl + kWBytes;
  const int tiles = (a.M + kUwM - 1) / kUwM;
  const uint64_t xg = reinterpret_cast<uint64_t>(static_cast<const float*>(a.x) + head * a.x_bs);
  // X tile t -> buffer t & 1: block j = rows 2j, 2j + 1 of the tile, row b at 512 b,
  // 16-byte chunk q at q ^ (b & 15); rows past M repeat the last one (never stored)
  auto issue_x = [&](int t) {
    const uint32_t xl = xl0 + static_cast<uint32_t>(t & 1) * kXBytes;
    for (int j = wv; j < kUwM / 2; j += 4) {
      const int b = 2 * j + (lane >> 5), qs = lane & 31;
      const int br = t * kUwM + b < a.M ? t * kUwM + b : a.M - 1;
      const uint32_t voff =
          static_cast<uint32_t>((static_cast<int64_t>(br) * a.ldx_m + 4 * (qs ^ (b & 15))) * 4);
      dma_block(xg, voff, xl + 1024 * j);
    }
  };
  {  // the W tile, once: block j = rows (1024 / kWRow) j .., chunk q at q ^ 4(d & 3)
    const uint64_t wg = reinterpret_cast<uint64_t>(static_cast<const bf16_t*>(a.w1) +
                                                   head * a.w_bs + c0);
    for (int j = wv; j < kWBytes / 1024; j += 4) {
      const int byte = 1024 * j + 16 * lane;
      const int d = byte / kWRow, qs = (byte % kWRow) >> 4;
      const uint32_t voff = static_cast<uint32_t>((static_cast<int64_t>(d) * a.ldw_k +
                                                   8 * (qs ^ (4 * (d & 3)))) * 2);
      dma_block(wg, voff, wl + 1024 * j);
    }
  }
  issue_x(0);

  const int i16 = lane & 15, G = lane >> 4, j32 = lane & 31, g = lane >> 5;
  float* y = static_cast<float*>(a.y) + head * a.y_bs + c0;
  for (int t = 0; t < tiles; ++t) {
    if (t + 1 < tiles) {   // (buffer (t + 1) & 1 was freed by the barrier ending tile t - 1)
      issue_x(t + 1);
      wait_vmcnt<kXPerWave>();   // W and tile t have landed; tile t + 1 may fly
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();   // ... for every wave's copies
    const uint32_t xl = xl0 + static_cast<uint32_t>(t & 1) * kXBytes;
    f32x16_t acc[kCT][2];
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[ct][mt][e] = 0.f;
#pragma unroll 2
    for (int s = 0; s < kUkK / 16; ++s) {
      bf16x8_t af[kCT];
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
        const int col = 32 * (kCT * wv + ct) + 16 * (G & 1) + 4 * (i16 & 3);
        const int d = 16 * s + 8 * (G >> 1) + (i16 >> 2);
        const int q = col >> 3, h8 = 8 * ((col >> 2) & 1);
        const s16x4_t v0 = lds_tr16_u(wl + kWRow * d + 16 * (q ^ (4 * (d & 3))) + h8);
        const s16x4_t v1 = lds_tr16_u(wl + kWRow * (d + 4) + 16 * (q ^ (4 * ((d + 4) & 3))) + h8);
        const s16x4_t vv[2] = {v0, v1};
        af[ct] = __builtin_bit_cast(bf16x8_t, vv);
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int b = 32 * mt + j32;
        const int q = 4 * s + 2 * g;
        const u32x4_t x0 = lds_u128(xl + 512 * b + 16 * (q ^ (b & 15)));
        const u32x4_t x1 = lds_u128(xl + 512 * b + 16 * ((q + 1) ^ (b & 15)));
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = __uint_as_float(x0[e]);
          v[4 + e] = __uint_as_float(x1[e]);
        }
        const u32x4_t hi = {cvt2(v[0], v[1]), cvt2(v[2], v[3]), cvt2(v[4], v[5]), cvt2(v[6], v[7])};
        float rl[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          rl[2 * e] = v[2 * e] - __uint_as_float(hi[e] << 16);
          rl[2 * e + 1] = v[2 * e + 1] - __uint_as_float(hi[e] & 0xFFFF0000u);
        }
        const u32x4_t lo = {cvt2(rl[0], rl[1]), cvt2(rl[2], rl[3]), cvt2(rl[4], rl[5]),
                            cvt2(rl[6], rl[7])};
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) {
          acc[ct][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ct], __builtin_bit_cast(bf16x8_t, hi),
                                                                acc[ct][mt], 0, 0, 0);
          acc[ct][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ct], __builtin_bit_cast(bf16x8_t, lo),
                                                                acc[ct][mt], 0, 0, 0);
        }
      }
    }
    // acc[ct][mt] lane (j32, g): columns 32(kCT wv + ct) + 8 e4 + 4g + (0..3), row 32mt + j32
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int m = t * kUwM + 32 * mt + j32;
        if (m < a.M) {
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4)
            *reinterpret_cast<float4*>(y + static_cast<int64_t>(m) * a.ldy + 32 * (kCT * wv + ct) +
                                       8 * e4 + 4 * g) =
                make_float4(acc[ct][mt][4 * e4], acc[ct][mt][4 * e4 + 1], acc[ct][mt][4 * e4 + 2],
                            acc[ct][mt][4 * e4 + 3]);
        }
      }
    lds_barrier();   // every wave is done with buffer t & 1 before tile t + 2 goes there
  }
}

// ---- per-head o[b, i, d] = sum_c X[b, i, c] W_UV[i*d_h + d, c], fp32 X ---------
// (the absorbed output's first product: X = o_lat, K = d_c = 512, N = d_h.)
// Workgroup = (head, 64 rows d of W, 64 rows b).  The W rows (64 KB) arrive by
// asynchronous copies; the fp32 X rows (128 KB) are read into registers, all in
// flight at once, rounded to bf16 (the product's input precision) and stored to
// LDS.  Both are K-contiguous, so every fragment is one 16-byte read: row r at
// 1 KB r, chunk q (8 values) at q ^ (r & 15).  Wave w computes the 32 x 32 tile
// (d half w & 1, b half w >> 1) over the 32 k-steps.  The two d halves of a head
// run on one XCD (workgroups 8 apart), so the second reads X from its L2.
constexpr int kUvK = 512, kUvN = 64, kUvM = 64;
// merge: rows per pass, partials per load batch
constexpr int kUvMergeRows = 2, kUvMergeUnits = 4;

// kMerge: X(b, c) of head i is not read from o_lat but formed from the split
// partials of row b ([Report] §2.3 absorbs W_UV into the output side, so the
// merged latent output is only ever an operand of this product): per row, m =
// max lse_u, w_u = exp(lse_u - m), X = sum_u w_u o_u / sum_u w_u, in the order and
// arithmetic of k_merge_rows, so the bf16 operand is the one the same product
// takes from mla_merge_lse's o_lat.  Eight waves form X (twice the loads in
// flight of four); four of them then run the products as the plain form does.
// The first half's workgroups write the merged lse when asked for.
template <bool kMerge>
__global__ __launch_bounds__(kMerge ? 512 : 256, 1) void k_gemm_uv_wide(GemmArgs a, MergeArgs mg) {
  constexpr int kWaves = kMerge ? 8 : 4;
  __shared__ __attribute__((aligned(1024))) char lds[(kUvN + kUvM) * 1024];   // W rows, X rows
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int L = blockIdx.x, halves = a.N / kUvN;   // (head, half) pairs, XCD-paired
  const int pair = (L >> 3) / halves * 8 + (L & 7), half = (L >> 3) % halves;
  const int head = pair, n0 = half * kUvN, m0 = blockIdx.y * kUvM;
  const uint32_t wl = lds_addr(lds), xl = wl + kUvN * 1024;

  // ---- W rows n0 .. n0+63 of the head: one 1 KB copy each
  {
    const uint64_t wg = reinterpret_cast<uint64_t>(static_cast<const bf16_t*>(a.w1) +
                                                   head * a.w_bs + static_cast<int64_t>(n0) * a.ldw_n);
    for (int r = wv; r < kUvN; r += kWaves) {
      const uint32_t voff = static_cast<uint32_t>((static_cast<int64_t>(r) * a.ldw_n +
                                                   8 * (lane ^ (r & 15))) * 2);
      dma_block(wg, voff, wl + 1024 * r);
    }
  }
  // X element (b, c) at xl + 1024 b + 16 ((c >> 3) ^ (b & 15)) + 8 ((c >> 2) & 1), bf16
  auto x_store = [&](int b, int c, float4 v) {
    const uint32_t addr = xl + 1024 * b + 16 * ((c >> 3) ^ (b & 15)) + 8 * ((c >> 2) & 1);
    *reinterpret_cast<__attribute__((address_space(3))) u32x2_t*>(static_cast<uintptr_t>(addr)) =
        (u32x2_t){cvt2(v.x, v.y), cvt2(v.z, v.w)};
  };
  if constexpr (kMerge) {
    // ---- the partials of every row of the block: first unit and count (a bad range
    // is flagged once, by head 0)
    __shared__ int st_first[kUvM], st_count[kUvM];
    if (tid < kUvM) {
      const int bq = m0 + tid;
      int first = 0, count = 0;   // rows past M: no partials (zero X rows, never stored)
      if (bq < a.M) merge_units(mg, bq, head == 0 && half == 0, &first, &count);
      st_first[tid] = count > 0 ? first : 0;   // no partials: unit 0, weight 0
      st_count[tid] = count;
    }
    __syncthreads();
    // ---- thread: columns c..c+3 of rows 4i + rq (a wave's rows are uniform), in
    // passes of R rows (a pass whose rows are all past M reads nothing).  A pass
    // reads the partials in batches of U per row, each
    // batch one load per (row, partial) plus one lse load per wave (lane r U + k
    // fetches partial k of row r; the values are read back lane by lane).  A row of
    // at most U partials takes its reference from its one batch, else a first sweep
    // over its lse finds it.  (Small batches measured fastest: 2 rows x 4 partials
    // per pass beat 8 x 4, 4 x 4 and 1 x 4, and issuing the next pass's batch
    // before combining the current one gained nothing.)
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    constexpr int R = kUvMergeRows, U = kUvMergeUnits, P = kUvM / 4 / R;
    static_assert(R * U <= 64 && P * R * 4 == kUvM, "merge batch shape");
    const int nh = mg.n_heads;
    const int c = 4 * (tid & 127), rq = tid >> 7;
    const float* op = mg.o_part + static_cast<int64_t>(head) * kUvK + c;
    const float* lp = mg.lse_part + head;
    const int64_t ustride = static_cast<int64_t>(nh) * kUvK;   // floats between units
    const bool lead = (tid & 127) == 0 && half == 0;   // writes the rows' lse
    const int jr = min(lane / U, R - 1), jk = lane % U;   // lse lane: row jr, partial jk
    struct Batch {
      f32x4_t x[R][U];
      float lv;
    };
    auto row_of = [&](int p, int r) { return 4 * (R * p + r) + rq; };
    // lse of partial s0 + jk of the lse lane's row of pass p (-inf past its count)
    auto lse_lane = [&](int p, int s0) {
      const int row = row_of(p, jr), f = st_first[row];
      const bool in = s0 + jk < st_count[row];
      const float lv = lp[static_cast<int64_t>(in ? f + s0 + jk : f) * nh];
      return in ? lv : -INFINITY;
    };
    auto load = [&](int p, int s0, Batch& bt) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = row_of(p, r);
        const int f = __builtin_amdgcn_readfirstlane(st_first[row]);
        const int n = __builtin_amdgcn_readfirstlane(st_count[row]);
#pragma unroll
        for (int k = 0; k < U; ++k) {
          const int u = s0 + k < n ? f + s0 + k : f;
          bt.x[r][k] = *reinterpret_cast<const f32x4_t*>(op + u * ustride);
        }
      }
      bt.lv = lse_lane(p, s0);
    };
    // every load of a batch is issued before its first use (the weighted add below
    // is a select, which the compiler would otherwise turn into a branch around a
    // load of its own)
    auto settle = [&](Batch& bt) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int k = 0; k < U; ++k) asm volatile("" : "+v"(bt.x[r][k]));
    };
    auto lse_at = [&](float lv, int r, int k) {
      return __builtin_bit_cast(float,
                                __builtin_amdgcn_readlane(__builtin_bit_cast(int, lv), r * U + k));
    };
    Batch cur;
#pragma unroll 1
    for (int p = 0; p < P; ++p) {
      int cmax = 0;
#pragma unroll
      for (int r = 0; r < R; ++r)
        cmax = max(cmax, __builtin_amdgcn_readfirstlane(st_count[row_of(p, r)]));
      float m[R], zz[R];
      float4 acc[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        m[r] = -INFINITY;
        zz[r] = 0.f;
        acc[r] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      if (cmax > U) {   // the references first
        for (int s0 = 0; s0 < cmax; s0 += U) {
          const float lv = lse_lane(p, s0);
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int k = 0; k < U; ++k) m[r] = fmaxf(m[r], lse_at(lv, r, k));
        }
      }
      for (int s0 = 0; s0 < cmax; s0 += U) {
        load(p, s0, cur);
        settle(cur);
        float l[R][U];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int k = 0; k < U; ++k) l[r][k] = lse_at(cur.lv, r, k);
        if (cmax <= U) {
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int k = 0; k < U; ++k) m[r] = fmaxf(m[r], l[r][k]);
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int k = 0; k < U; ++k) {
            // partials past the row's count have l = -inf: weight 0, nothing added
            const float w = l[r][k] == -INFINITY ? 0.f : __expf(l[r][k] - m[r]);
            zz[r] += w;
            const bool on = w != 0.f;
            float n0 = acc[r].x, n1 = acc[r].y, n2 = acc[r].z, n3 = acc[r].w;
            n0 += w * cur.x[r][k][0]; n1 += w * cur.x[r][k][1];
            n2 += w * cur.x[r][k][2]; n3 += w * cur.x[r][k][3];
            acc[r].x = on ? n0 : acc[r].x;
            acc[r].y = on ? n1 : acc[r].y;
            acc[r].z = on ? n2 : acc[r].z;
            acc[r].w = on ? n3 : acc[r].w;
          }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = row_of(p, r), bq = m0 + row;
        const float inv = zz[r] > 0.f ? 1.f / zz[r] : 0.f;
        x_store(row, c, make_float4(acc[r].x * inv, acc[r].y * inv, acc[r].z * inv, acc[r].w * inv));
        if (lead && mg.lse && bq < a.M)
          mg.lse[static_cast<int64_t>(bq) * nh + head] =
              zz[r] > 0.f ? m[r] + __logf(zz[r]) : -INFINITY;
      }
    }
    wait_vmcnt<0>();   // the W copies
    __syncthreads();
  } else {
    // ---- X rows: 32 float4 per thread in flight, then bf16 into LDS
    const float* xb = static_cast<const float*>(a.x) + head * a.x_bs;
    float4 v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int e = 4 * (256 * i + tid);   // element of the 64 x 512 tile
      const int b = e >> 9, c = e & 511;
      const int br = m0 + b < a.M ? m0 + b : a.M - 1;   // rows past M repeat the last one
      v[i] = *reinterpret_cast<const float4*>(xb + static_cast<int64_t>(br) * a.ldx_m + c);
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int e = 4 * (256 * i + tid);
      x_store(e >> 9, e & 511, v[i]);
    }
    wait_vmcnt<0>();   // the W copies
    __syncthreads();
  }
  if (wv >= 4) return;   // (merge form) waves 4..7 only formed X

  // ---- products: wave tile (d rows 32(wv & 1) .., b rows 32(wv >> 1) ..)
  const int j32 = lane & 31, g = lane >> 5;
  const int dr = 32 * (wv & 1) + j32, br = 32 * (wv >> 1) + j32;
  f32x16_t acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll 8
  for (int s = 0; s < kUvK / 16; ++s) {
    const int q = 2 * s + g;
    const u32x4_t av = lds_u128(wl + 1024 * dr + 16 * (q ^ (dr & 15)));
    const u32x4_t bv = lds_u128(xl + 1024 * br + 16 * (q ^ (br & 15)));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                  __builtin_bit_cast(bf16x8_t, bv), acc, 0, 0, 0);
  }
  // acc lane (j32, g): d = n0 + 32(wv & 1) + 8(e >> 2) + 4g + (e & 3), b = m0 + 32(wv >> 1) + j32
  const int b = m0 + 32 * (wv >> 1) + j32;
  if (b < a.M) {
    bf16_t* y = static_cast<bf16_t*>(a.y) + head * a.y_bs + static_cast<int64_t>(b) * a.ldy + n0 +
                32 * (wv & 1) + 4 * g;
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4)
      *reinterpret_cast<u32x2_t*>(y + 8 * e4) =
          (u32x2_t){cvt2(acc[4 * e4], acc[4 * e4 + 1]), cvt2(acc[4 * e4 + 2], acc[4 * e4 + 3])};
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


// The tiled product for a bf16 X with both operand tiles staged by asynchronous
// global->LDS copies (no register staging, so no compiler-placed waits between a
// chunk's loads and its use): 2 stages of (TN + TM) rows x 64 k (128 bytes per row,
// 16-byte chunk c of row r at c ^ ((r >> 1) & 7): conflict-free fragment reads).  A
// copy instruction moves 8 rows; wave w issues instructions w, w + 4, ...  Chunk
// c + 1 is in flight while chunk c is multiplied.  Products and epilogue as
// k_gemm_tile.  The 8 weight rows of a copy never straddle w1 / w2 (n_split is a
// multiple of TN or past N).  With ksplit > 1 (grid z = batch x ksplit) a workgroup
// takes K slice ks and writes its fp32 tile to partial[ks][z][m][n] for
// k_gemm_finish instead of applying the epilogue.
template <int TN, int TM>
__global__ __launch_bounds__(256, 2) void k_gemm_tile_dma(GemmArgs a, int ksplit, float* partial) {
  constexpr int BN = TN / 64, BM = TM / 64;   // 32-row blocks per wave
  constexpr int kRows = TN + TM, kStage = kRows * kTk * 2;
  constexpr int kInstr = kRows / 8, kPerWave = kInstr / 4;   // copies per stage, per wave
  constexpr int kOPitch = TN + 4;   // floats per staged output row
  constexpr int kBytes = 2 * kStage > TM * kOPitch * 4 ? 2 * kStage : TM * kOPitch * 4;
  __shared__ __attribute__((aligned(1024))) char tiles[kBytes];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int z = blockIdx.z / ksplit, ks = blockIdx.z - z * ksplit;
  const int n0 = blockIdx.x * TN, m0 = blockIdx.y * TM;
  // a grid's x of more than 8 is padded to a multiple of 8 (the two row tiles of a
  // weight tile, blocks x and x + gridDim.x, then share an XCD and its L2): padding
  // exits here
  if (n0 >= a.N) return;
  const int kslice = a.K / ksplit;
  const int64_t kbeg = static_cast<int64_t>(ks) * kslice;
  const uint32_t lds0 = lds_addr(tiles);
  auto key = [](int r) { return (r >> 1) & 7; };
  // copy j of this wave: stage rows 8q .. 8q + 7 (q = wv + 4j); base of its first
  // row (uniform) and this lane's byte offset (row 8q + (lane >> 3), source chunk
  // (lane & 7) ^ key(row)); rows past N or M re-read the last row (never stored).
  // With the fused latent append, weight rows from n_append on come from w3 / w4
  // (an 8-row group never straddles them: n_append and n_split3 are multiples of 8)
  uint64_t gb[kPerWave];
  uint32_t vo[kPerWave];
#pragma unroll
  for (int j = 0; j < kPerWave; ++j) {
    const int q = wv + 4 * j, row = 8 * q + (lane >> 3), ch = (lane & 7) ^ key(row);
    if (8 * q < TN) {
      const int nb = min(n0 + 8 * q, a.N - 1), nr = min(n0 + row, a.N - 1);
      const bf16_t* w;
      if (a.epi == EPI_QPROJ_APPEND && nb >= a.n_append) {   // the fused latent append's rows
        const int r = nb - a.n_append;
        w = r < a.n_split3
                ? static_cast<const bf16_t*>(a.w3) + static_cast<int64_t>(r) * a.ldw_n
                : static_cast<const bf16_t*>(a.w4) + static_cast<int64_t>(r - a.n_split3) * a.ldw_n;
      } else {
        w = nb < a.n_split
                ? static_cast<const bf16_t*>(a.w1) + static_cast<int64_t>(nb) * a.ldw_n
                : static_cast<const bf16_t*>(a.w2) + static_cast<int64_t>(nb - a.n_split) * a.ldw_n;
      }
      gb[j] = reinterpret_cast<uint64_t>(w + static_cast<int64_t>(z) * a.w_bs + kbeg);
      vo[j] = static_cast<uint32_t>(((nr - nb) * a.ldw_n + 8 * ch) * 2);
    } else {
      const int mb = min(m0 + 8 * q - TN, a.M - 1), mr = min(m0 + row - TN, a.M - 1);
      gb[j] = reinterpret_cast<uint64_t>(static_cast<const bf16_t*>(a.x) +
                                         static_cast<int64_t>(z) * a.x_bs +
                                         static_cast<int64_t>(mb) * a.ldx_m + kbeg);
      vo[j] = static_cast<uint32_t>(((mr - mb) * a.ldx_m + 8 * ch) * 2);
    }
  }
  auto issue = [&](int stage, int k0) {
#pragma unroll
    for (int j = 0; j < kPerWave; ++j)
      dma_block(gb[j] + 2 * static_cast<uint64_t>(k0), vo[j],
                lds0 + stage * kStage + 1024 * (wv + 4 * j));
  };
  const int wn = wv & 1, wm = wv >> 1, r32 = lane & 31, h = lane >> 5;
  f32x16_t acc[BN][BM];
#pragma unroll
  for (int i = 0; i < BN; ++i)
#pragma unroll
    for (int j = 0; j < BM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  // operand of 32-row block i at k-step s: row 32i + r32 of the wave's half, chunk 2s + h
  auto frag = [&](uint32_t st, int row, int s) {
    return __builtin_bit_cast(bf16x8_t,
                              lds_u128(st + 128 * row + 16 * ((2 * s + h) ^ key(row))));
  };
  auto multiply = [&](int stage) {
    const uint32_t st = lds0 + stage * kStage;
#pragma unroll
    for (int s = 0; s < kTk / 16; ++s) {
      bf16x8_t af[BN], bfr[BM];
#pragma unroll
      for (int i = 0; i < BN; ++i) af[i] = frag(st, 32 * BN * wn + 32 * i + r32, s);
#pragma unroll
      for (int j = 0; j < BM; ++j) bfr[j] = frag(st, TN + 32 * BM * wm + 32 * j + r32, s);
#pragma unroll
      for (int i = 0; i < BN; ++i)
#pragma unroll
        for (int j = 0; j < BM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };
  const int nk = kslice / kTk;
  issue(0, 0);
  if (nk > 1) issue(1, kTk);
  for (int kb = 0; kb < nk; ++kb) {
    if (kb + 1 < nk) wait_vmcnt<kPerWave>();   // chunk kb has landed (kb + 1 may fly)
    else wait_vmcnt<0>();
    __syncthreads();   // ... for every wave's copies
    multiply(kb & 1);
    __syncthreads();   // every wave is done with this stage before it is refilled
    if (kb + 2 < nk) issue(kb & 1, (kb + 2) * kTk);
  }
  // acc[i][j] element e of lane (r32, h): row 32 BM wm + 32j + r32, column
  // 32 BN wn + 32i + 8(e >> 2) + 4h + (e & 3) of the tile; through LDS (the stages
  // are free after the last barrier) to the epilogue's column pairs
  float* ot = reinterpret_cast<float*>(tiles);
#pragma unroll
  for (int j = 0; j < BM; ++j)
#pragma unroll
    for (int i = 0; i < BN; ++i)
#pragma unroll
      for (int e = 0; e < 16; e += 2)
        *reinterpret_cast<float2*>(&ot[(32 * BM * wm + 32 * j + r32) * kOPitch + 32 * BN * wn + 32 * i +
                                       8 * (e >> 2) + 4 * h + (e & 3)]) =
            make_float2(acc[i][j][e], acc[i][j][e + 1]);
  // fused latent append into the pool: each output row's pool row and position,
  // looked up once per row instead of once per column pair
  __shared__ int64_t app_off[TM];
  __shared__ int app_pos[TM];
  const bool app = a.epi == EPI_QPROJ_APPEND && a.ld3 == 0 && n0 + TN > a.n_append;
  if (app)
    for (int r = tid; r < TM; r += 256) {
      const bool in = m0 + r < a.M;
      app_off[r] = in ? append_row_offset(a, m0 + r, n0 <= a.n_append) : -1;
      app_pos[r] = in ? a.pos[m0 + r] : 0;
    }
  __syncthreads();
  for (int q = tid; q < TM * TN / 2; q += 256) {   // pair q: row q / (TN/2), columns 2 (q % (TN/2)), +1
    const int ml = q / (TN / 2), nl = 2 * (q % (TN / 2));
    const int m = m0 + ml, n = n0 + nl;
    if (m < a.M && n < a.N) {
      const float2 v = *reinterpret_cast<const float2*>(&ot[ml * kOPitch + nl]);
      if (ksplit > 1)
        *reinterpret_cast<float2*>(partial + ((static_cast<int64_t>(ks) * a.batch + z) * a.M + m) *
                                                 a.N + n) = v;
      else if (app && n >= a.n_append)
        append_pair_at<bf16_t>(a, a.y3, a.n_split3, app_off[ml], m, app_pos[ml], n - a.n_append,
                               v.x, v.y);
      else
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

constexpr int kXsRing = 8;   // weight loads in flight per lane

struct XsPlan {
  int mb, d, kw;
};

// K slices d.  A slice is a whole number of ring turns (32 kXsRing k) whose X
// slice fits kXsLdsBytes; among those, d minimises a cost in weight-step units
// (one step: 1 KB per wave, ≈0.2 µs of the whole chip's stream): the busiest
// wave's (strip, slice) pairs times their steps plus the MB KB partial tile each
// writes, and for d > 1 the finish pass (≈12 steps of launch, plus reading every
// partial tile at the chip's rate).  The grid has cu_count() / d workgroups per
// slice.  A narrow weight (16 heads: 228 strips of the fused query product) gets
// slices that give its idle waves strips; a few rows (M <= 16) get more slices,
// whose partial tiles are small, to even out the busiest wave (the 4-row query
// projection: 8 against 3.07 strips per wave, 5 slices instead of 2).  The plan
// depends on M, K, the planned columns and the chip only, so the fused query
// projection + latent append takes the same slices, and produces the same
// queries bit for bit, as the query projection alone.  (At 64 rows: 5 slices of
// 1024 for K = 5120, where the 1572 strips of the fused call come to 7.7 per
// wave against a busiest wave's 8, and 16 slices for K = 16384.)
XsPlan xs_plan(const GemmArgs& a) {
  XsPlan p{};
  p.mb = a.M <= 16 ? 1 : a.M <= 32 ? 2 : 4;
  constexpr int kUnit = 32 * kXsRing;
  constexpr int64_t kFinishSteps = 12;
  const int kw_max = kXsLdsBytes / (2 * 16 * p.mb) / kUnit * kUnit;
  const int groups = a.K / kUnit;
  const int64_t strips = (a.plan_cols > 0 ? a.plan_cols : a.N) / 16;
  const int cus = cu_count();
  const int64_t waves = static_cast<int64_t>(cus) * kXsWaves;
  int64_t best = -1;
  p.d = groups;
  for (int d = 1; d <= groups; ++d) {
    if (groups % d != 0 || a.K / d > kw_max) continue;
    const int64_t nw = static_cast<int64_t>(std::max(1, cus / d)) * kXsWaves;
    const int64_t busiest = (strips + nw - 1) / nw;
    const int64_t steps = a.K / d / 32;
    const int64_t cost =
        d == 1 ? busiest * steps
               : busiest * (steps + p.mb) + kFinishSteps + d * strips * p.mb / waves;
    if (best < 0 || cost < best) {
      best = cost;
      p.d = d;
    }
  }
  p.kw = a.K / p.d;
  return p;
}

template <typename XT, int MB, bool kSplit>
hipError_t launch_xs_kernel(const GemmArgs& a, const XsPlan& p, float* partial, hipStream_t stream) {
  static std::atomic<int> attr_set{0};
  if (!attr_set.load(std::memory_order_acquire)) {
    const hipError_t e =
        hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_xs<XT, MB, kXsRing, kSplit>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kXsLdsBytes);
    if (e != hipSuccess) return e;
    attr_set.store(1, std::memory_order_release);
  }
  const int grid = std::max(1, cu_count() / p.d) * p.d;
  const size_t lds = static_cast<size_t>(16 * MB) * p.kw * 2;
  hipLaunchKernelGGL((k_gemm_xs<XT, MB, kXsRing, kSplit>), dim3(grid), dim3(64 * kXsWaves), lds,
                     stream, a, p.d, p.kw, partial);
  return hipGetLastError();
}

template <typename XT, int MB>
hipError_t launch_xs_inst(const GemmArgs& a, const XsPlan& p, float* partial, hipStream_t stream) {
  return p.d > 1 ? launch_xs_kernel<XT, MB, true>(a, p, partial, stream)
                 : launch_xs_kernel<XT, MB, false>(a, p, partial, stream);
}

// K-split partial tiles of k_gemm_xs: d slices x N/16 strips x [16 mb rows][16]
size_t xs_tiles_bytes(const GemmArgs& a, const XsPlan& p) {
  return static_cast<size_t>(p.d) * (a.N / 16) * (256 * p.mb) * sizeof(float);
}

// the RoPE cos/sin table behind the tiles (output stages that rotate)
bool epi_rotates(const GemmArgs& a) {
  return a.epi == EPI_QPROJ || a.epi == EPI_QPROJ_APPEND || a.epi == EPI_APPEND;
}
size_t xs_rope_bytes(const GemmArgs& a) {
  return epi_rotates(a) ? static_cast<size_t>(a.M) * a.d_rope * sizeof(float) : 0;
}

hipError_t launch_finish_xs(const GemmArgs& a, const XsPlan& p, const float* partial,
                            hipStream_t stream) {
  const int64_t quads = static_cast<int64_t>(a.N / 16) * a.M * 4;
  const int threads = quads < 65536 ? 64 : 256;
  const int blocks = static_cast<int>(std::min<int64_t>((quads + threads - 1) / threads, 8192));
  hipLaunchKernelGGL(k_gemm_finish_xs, dim3(blocks), dim3(threads), 0, stream, a, p.d, 16 * p.mb,
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

// The per-head W_UK form: W is [K=128, N] N-contiguous, output fp32; X bf16, or
// fp32 (taken as two bf16 terms).
static bool uk_ok(const GemmArgs& a) {
  return a.ldw_n == 1 && a.ldw_k % 8 == 0 && a.K == kUkK && a.N % kUkN == 0 && a.ldx_k == 1 &&
         a.y_f32 && a.epi == EPI_STORE && a.ldx_m % 8 == 0 && a.x_bs % 8 == 0 &&
         a.w1 == a.w2 && a.n_split >= a.N && aligned16(a.x) && aligned16(a.w1);
}

// The wide W_UK form: an fp32 X, 256-column tiles, every row and block start
// 16-byte aligned (asynchronous copies and 16-byte stores), copy offsets in 32 bits.
static bool uk_wide_ok(const GemmArgs& a) {
  return uk_ok(a) && a.x_f32 && a.N % kUwN == 0 && a.ldw_k % 8 == 0 && a.w_bs % 8 == 0 &&
         a.ldx_m % 4 == 0 && a.x_bs % 4 == 0 && a.ldy % 4 == 0 && a.y_bs % 4 == 0 &&
         aligned16(a.y) && static_cast<int64_t>(kUwM) * a.ldx_m * 4 < (int64_t{1} << 31);
}

// One activation matrix of at most 64 rows and enough weight rows to give every
// wave of the grid strips to stream (narrow outputs, like the 576-wide latent
// append, leave most waves idle there and go to k_gemm_ws): the X-stationary kernel.
static bool xs_ok(const GemmArgs& a) {
  // the fused append reads its two weights (w3, w4) with the same 16-byte loads
  if (a.epi == EPI_QPROJ_APPEND &&
      !(a.n_append % 16 == 0 && a.n_split3 % 16 == 0 && a.n_split < a.n_append &&
        aligned16(a.w3) && aligned16(a.w4)))
    return false;
  // (the asynchronous X copies address X with 32-bit byte offsets)
  return ws_ok(a) && a.batch == 1 && a.M <= 64 && a.N >= 2048 && a.N % 16 == 0 &&
         (a.n_split % 16 == 0 || a.n_split >= a.N) && a.K % (32 * kXsRing) == 0 &&
         (static_cast<int64_t>(a.M) * a.ldx_m + a.K) * 4 < (int64_t{1} << 31);
}

// Prefill-sized activations (M >= 256): the tiled product.  Same operand forms as
// k_gemm_ws; K a multiple of the 64-wide chunk.
static bool tile_ok(const GemmArgs& a) {
  const int64_t groups = static_cast<int64_t>((a.N + kTt - 1) / kTt) * ((a.M + kTt - 1) / kTt) * a.batch;
  // the fused query projection + latent append runs on the copy-staged form only
  // (bf16 X, the query split on a tile boundary), whose weight copies know w3 / w4
  if (a.epi == EPI_QPROJ_APPEND) {
    if (!(!a.x_f32 && a.batch == 1 && a.n_split % kTt == 0 && a.n_split < a.n_append &&
          a.n_append % 8 == 0 && a.n_split3 % 8 == 0 && aligned16(a.w3) && aligned16(a.w4)))
      return false;
    // ... and only where the appended rows' tiles fit the rounds of workgroups (two
    // per CU) that the query tiles take anyway: at M = 1024 the 1536 query tiles fill
    // three rounds exactly, and 40 more would add a fourth (the two calls are faster)
    const int64_t slots = 2 * static_cast<int64_t>(cu_count());
    const int64_t mt = (a.M + kTt - 1) / kTt;
    const int64_t tq = (a.n_append + kTt - 1) / kTt * mt, tf = (a.N + kTt - 1) / kTt * mt;
    if ((tf + slots - 1) / slots > (tq + slots - 1) / slots) return false;
  }
  // grids of fewer than 256 output tiles (narrow outputs such as the latent append)
  // would leave most of the chip idle: those stay with the K-split weight stream
  return ws_ok(a) && a.M >= 256 && a.K % kTk == 0 && a.n_split % 2 == 0 && groups >= 256;
}

bool gemm_tiled_ok(const GemmArgs& a) { return ws_ok(a) && tile_ok(a); }

// Column tiles of a tiled product's grid: more than 8 are padded to a multiple of 8
// (k_gemm_tile_dma), so that blocks x and x + gridDim.x share an XCD; fewer stay as
// they are (padding one column tile to 8 would put every real block on one XCD).
static unsigned xcd_pad(unsigned x) { return x > 8 ? (x + 7) / 8 * 8 : x; }

// The fused query projection + latent append runs on k_gemm_xs (decode batches)
// and on the copy-staged tiled product (M >= 256).
bool fused_qa_ok(const GemmArgs& a) {
  return a.epi == EPI_QPROJ_APPEND && (xs_ok(a) || tile_ok(a));
}

// Per-head batched products at decode sizes (M <= 64, N a multiple of 64): one
// 64 x 64 tile per workgroup, no K split, when that gives at least 256 workgroups.
static bool small_tile_ok(const GemmArgs& a) {
  return ws_ok(a) && a.epi == EPI_STORE && a.batch > 1 && a.M <= 64 && a.N % 64 == 0 &&
         a.K % kTk == 0 && static_cast<int64_t>(a.N / 64) * a.batch >= 256;
}

// The per-head W_UV form for an fp32 X and bf16 output: K = 512, N a multiple of
// 64, heads a multiple of 8 (XCD pairing), rows 16-byte aligned, bf16 stores of 8 bytes.
static bool uv_wide_ok(const GemmArgs& a) {
  return a.ldw_k == 1 && a.ldx_k == 1 && a.M > 0 && a.N > 0 && a.batch > 0 &&
         a.epi == EPI_STORE && a.x_f32 && !a.y_f32 && a.K == kUvK && a.N % kUvN == 0 &&
         a.batch % 8 == 0 && a.n_split >= a.N && a.ldw_n % 8 == 0 && a.w_bs % 8 == 0 &&
         a.x_bs % 4 == 0 && a.ldx_m % 4 == 0 && a.ldy % 4 == 0 && a.y_bs % 4 == 0 &&
         aligned16(a.x) && aligned16(a.w1) && (reinterpret_cast<uintptr_t>(a.y) & 7) == 0 &&
         static_cast<int64_t>(a.batch) * a.M * a.N < (int64_t{1} << 31) &&
         static_cast<int64_t>(a.batch) * (a.N / kUvN) < 65536;
}

bool fast_gemm_ok(const GemmArgs& a) { return ws_ok(a) || uk_ok(a) || uv_wide_ok(a); }

// Large-batch plain products whose 128 x 128 tiles would not cover the chip (W_O at
// 256 rows: 80 tiles): the copy-staged tiled product over d K slices, d the smallest
// divisor of K / 64 that gives 256 workgroups, then k_gemm_finish.  0 where it does
// not apply.
static int tile_split_d(const GemmArgs& a) {
  if (!(ws_ok(a) && a.epi == EPI_STORE && !a.x_f32 && a.M >= 256 && a.K % kTk == 0 &&
        a.N % 4 == 0 && (a.n_split % kTt == 0 || a.n_split >= a.N) && !tile_ok(a)))
    return 0;
  const int64_t groups = static_cast<int64_t>((a.N + kTt - 1) / kTt) * ((a.M + kTt - 1) / kTt) * a.batch;
  const int chunks = a.K / kTk;
  for (int d = 2; d <= chunks; ++d)
    if (chunks % d == 0 && groups * d >= 256) return static_cast<int64_t>(d) * a.batch < 65536 ? d : 0;
  return 0;
}

// W_UV with the merge folded in: the k_gemm_uv_wide form, the partials of every
// head at 512 latent columns (16-byte aligned rows), one merge row per product row.
bool uv_merge_ok(const GemmArgs& a, const MergeArgs& m) {
  return uv_wide_ok(a) && m.d_latent == kUvK && m.n_heads == a.batch && m.batch == a.M &&
         m.o_part != nullptr && m.lse_part != nullptr && aligned16(m.o_part) &&
         (m.unit_start != nullptr || m.num_splits >= 1);
}

// Where the fused form is the faster one (measured): decode batches (one 64-row
// block), a grid that covers the chip, and few partials per row.  Larger batches
// (a tiled W_UV, and many more merge rows) and small grids (16 heads) go faster as
// the two separate kernels, and so do long rows of uniform splits (64 per row),
// which a workgroup would merge serially.
bool uv_merge_pays(const GemmArgs& a, const MergeArgs& m) {
  return a.M <= kUvM && static_cast<int64_t>(a.batch) * (a.N / kUvN) >= 256 &&
         (m.unit_start != nullptr || m.num_splits <= 16);
}

hipError_t launch_uv_merge(const GemmArgs& a, const MergeArgs& m, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  if (!uv_merge_ok(a, m)) return hipErrorInvalidValue;
  const dim3 grid(a.batch * (a.N / kUvN), (a.M + kUvM - 1) / kUvM);
  hipLaunchKernelGGL(k_gemm_uv_wide<true>, grid, dim3(512), 0, stream, a, m);
  return hipGetLastError();
}

size_t gemm_partial_bytes(const GemmArgs& a) {
  if (ws_ok(a) && tile_ok(a)) return xs_rope_bytes(a);   // the RoPE table of a rotating output
  if (!ws_ok(a) || uv_wide_ok(a) || small_tile_ok(a)) return 0;
  if (const int d = tile_split_d(a))
    return static_cast<size_t>(d) * a.batch * a.M * a.N * sizeof(float);
  if (xs_ok(a)) {
    const XsPlan q = xs_plan(a);
    return q.d > 1 ? xs_tiles_bytes(a, q) + xs_rope_bytes(a) : 0;
  }
  const WsPlan p = ws_plan(a);
  return p.d > 1 ? static_cast<size_t>(p.d) * a.batch * a.M * a.N * sizeof(float) : 0;
}

hipError_t launch_gemm_fast(const GemmArgs& a, void* partial, size_t partial_bytes,
                            hipStream_t stream) {
  if (a.M == 0 || a.N == 0 || a.batch == 0) return hipSuccess;
  if (a.epi == EPI_QPROJ_APPEND && !fused_qa_ok(a)) return hipErrorInvalidValue;
  if (!ws_ok(a)) {
    if (uv_wide_ok(a)) {   // small batches, whose K granule the weight stream does not take
      const dim3 grid(a.batch * (a.N / kUvN), (a.M + kUvM - 1) / kUvM);
      hipLaunchKernelGGL(k_gemm_uv_wide<false>, grid, dim3(256), 0, stream, a, MergeArgs{});
      return hipGetLastError();
    }
    if (!uk_ok(a)) return hipErrorInvalidValue;
    if (uk_wide_ok(a)) {
      const int tiles_m = (a.M + kUwM - 1) / kUwM;
      // several row tiles and a grid of (head, 256 columns) that covers the chip:
      // one workgroup per (head, column tile) walks the row tiles
      if (tiles_m > 1 && static_cast<int64_t>(a.batch) * (a.N / kUwN) >= 256 &&
          static_cast<int64_t>(a.M) * a.ldx_m * 4 < (int64_t{1} << 32)) {
        hipLaunchKernelGGL(k_gemm_uk_rows<kUwN>, dim3(a.batch, a.N / kUwN), dim3(256), 0, stream, a);
        return hipGetLastError();
      }
      // grids of fewer than 256 workgroups (16 heads) take 128-column tiles: twice
      // the workgroups for the same products in the same order (bit-identical q_lat)
      if (static_cast<int64_t>(a.batch) * (a.N / kUwN) * tiles_m < 256) {
        dim3 grid(a.batch, a.N / (kUwN / 2), tiles_m);
        hipLaunchKernelGGL(k_gemm_uk_wide<kUwN / 2>, grid, dim3(256), 0, stream, a);
      } else {
        dim3 grid(a.batch, a.N / kUwN, tiles_m);
        hipLaunchKernelGGL(k_gemm_uk_wide<kUwN>, grid, dim3(256), 0, stream, a);
      }
      return hipGetLastError();
    }
    dim3 grid(a.batch, a.N / kUkN, (a.M + kTile - 1) / kTile);
    if (a.x_f32)
      hipLaunchKernelGGL(k_gemm_uk<float>, grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(k_gemm_uk<bf16_t>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  if (tile_ok(a)) {
    // a rotating output stage reads its cos/sin from a table made first (in the
    // partial region), once per (row, pair) of the call
    GemmArgs b = a;
    if (epi_rotates(a)) {
      if (partial == nullptr || !aligned16(partial) || partial_bytes < xs_rope_bytes(a))
        return hipErrorInvalidValue;
      b.rope_tab = static_cast<float*>(partial);
      const int entries = a.M * (a.d_rope / 2);
      hipLaunchKernelGGL(k_rope_table, dim3((entries + 255) / 256), dim3(256), 0, stream, b);
      if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    const dim3 grid((a.N + kTt - 1) / kTt, (a.M + kTt - 1) / kTt, a.batch);
    if (a.x_f32)
      hipLaunchKernelGGL((k_gemm_tile<float, kTt, kTt>), grid, dim3(256), 0, stream, b);
    else if (a.n_split % kTt == 0 || a.n_split >= a.N)
      hipLaunchKernelGGL((k_gemm_tile_dma<kTt, kTt>), dim3(xcd_pad(grid.x), grid.y, grid.z),
                         dim3(256), 0, stream, b, 1, nullptr);
    else
      hipLaunchKernelGGL((k_gemm_tile<bf16_t, kTt, kTt>), grid, dim3(256), 0, stream, b);
    return hipGetLastError();
  }
  if (uv_wide_ok(a)) {
    const dim3 grid(a.batch * (a.N / kUvN), (a.M + kUvM - 1) / kUvM);
    hipLaunchKernelGGL(k_gemm_uv_wide<false>, grid, dim3(256), 0, stream, a, MergeArgs{});
    return hipGetLastError();
  }
  if (const int d = tile_split_d(a)) {
    if (partial == nullptr || !aligned16(partial) || partial_bytes < gemm_partial_bytes(a))
      return hipErrorInvalidValue;
    const dim3 grid(xcd_pad((a.N + kTt - 1) / kTt), (a.M + kTt - 1) / kTt, a.batch * d);
    hipLaunchKernelGGL((k_gemm_tile_dma<kTt, kTt>), grid, dim3(256), 0, stream, a, d,
                       static_cast<float*>(partial));
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    return launch_finish(a, d, static_cast<float*>(partial), stream);
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
    if (q.d == 1) return launch_xs(a, q, nullptr, stream);
    // both kernels take the RoPE angles from the table behind the partial tiles
    GemmArgs b = a;
    b.rope_tab = epi_rotates(a) ? reinterpret_cast<float*>(static_cast<char*>(partial) +
                                                           xs_tiles_bytes(a, q))
                                : nullptr;
    hipError_t e = launch_xs(b, q, static_cast<float*>(partial), stream);
    if (e != hipSuccess) return e;
    return launch_finish_xs(b, q, static_cast<const float*>(partial), stream);
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
