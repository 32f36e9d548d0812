// MFMA kernels for gfx950 (CDNA4 matrix cores, wave64).
//
// Split-KV latent attention, the hot loop of the decode step
// ([Report] §2.3/§2.4 of "《DeepSeek-V2》深度解读报告": every head scores the
// same cached latent rows [c | k^R]; s = tau (q_lat . c + q_pe . k^R)).
//
// Work unit = (sequence b, split s).  A 512-thread workgroup (8 waves, two per
// SIMD so that one wave's softmax and LDS waits hide behind the other's matrix
// products) streams the split's rows in tiles of 32 tokens (32 rows x 1152
// bytes, contiguous inside one 64-row page) through a 3-slot LDS ring filled by
// asynchronous global->LDS copies (global_load_lds_dwordx4), two tiles ahead
// of the one consumed.  Wave w owns heads 16w..16w+15 (mfma_f32_16x16x32_bf16):
//   scores  S^T[t, h] = sum_k C[t, k] Q[h, k]   (M = 16 tokens, two blocks;
//           N = 16 heads; K = 576 in 18 steps; A = tile rows from LDS, B = the
//           wave's queries: 14 k-steps in VGPRs, 4 in LDS, for the whole unit)
//   softmax per head in the exp2 domain: in-lane over 8 tokens plus two
//           cross-lane steps.  The exponent reference of each head is fixed at
//           the maximum of its first scored tile, so the accumulator is never
//           rescaled; later scores may exceed it by up to 2^64 (no fp32/bf16
//           overflow).  A score beyond that headroom makes the whole unit run
//           again with the larger reference (at most once).
//   P.C     O[h, d] += sum_t P[h, t] C[t, d]   (M = 16 heads, N = 512 in 32
//           blocks, K = 32 tokens).  The score accumulator of a lane holds one
//           head and tokens 16 tb + 4 g + i; taking the contraction's k order
//           as t(g, j) = 16 (j >> 2) + 4 g + (j & 3) makes the packed
//           probabilities exactly the A operand, and the B operand (4 tokens
//           of one column per half) is one ds_read_b64_tr_b16 (hardware
//           transpose) per half from the same tile.
// LDS tile layout (36 KB): the 512 latent values of row r fill one 1 KB block
// (block r), chunk c (16 bytes) stored at c ^ 2(r & 7); the 64 RoPE values of
// rows 8j..8j+7 fill block 32 + j, row r at 128 (r & 7), chunk c' at
// c' ^ (r & 7).  Every copy fills one block.  LDS has 64 banks of 4 bytes; a
// ds_read_b128 is served in four 16-lane phases, the lanes of a phase being
// those with equal lane >> 5 and equal parity of bits 2..4 of the lane, and a
// ds_read_b64(_tr_b16) in two 32-lane phases (lane >> 5).  Under this layout
// no phase of a score read (16 rows, one chunk per lane group) or of a
// transposed read (8 rows, a chunk pair) puts two addresses on one bank.
#include "common.hpp"
#include "launch_fast.hpp"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const bf16x8_t lds_bf16x8;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

constexpr int kDc = 512, kDr = 64, kPage = 64;
constexpr int kTileTok = 32;
constexpr int kRowBytes = (kDc + kDr) * 2;            // 1152: one cached row
constexpr int kRopeOff = kTileTok * 1024;             // RoPE blocks follow the 32 latent blocks
constexpr int kTileBytes = kRopeOff + (kTileTok / 8) * 1024;   // 36864
constexpr int kThreads = 512, kWaves = 8;
constexpr int kKSteps = (kDc + kDr) / 32;             // 18
constexpr int kColBlocks = kDc / 16;                  // 32
constexpr int kStages = 3;                            // LDS ring depth
constexpr int kQReg = 14;                             // k-steps of Q held in VGPRs
constexpr int kQLds = kKSteps - kQReg;                // k-steps of Q held in LDS
constexpr int kPageWin = 2048;                        // page ids of the split held in LDS
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kHeadroom = 64.0f;                    // log2 units above the reference

__device__ __forceinline__ int ukey(int r) { return 2 * (r & 7); }
__device__ __forceinline__ int vkey(int r) { return r & 7; }

__device__ __forceinline__ unsigned cvt2(float lo, float hi) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

__device__ __forceinline__ bf16x8_t pack8(const float* v) {
  const u32x4_t u = {cvt2(v[0], v[1]), cvt2(v[2], v[3]), cvt2(v[4], v[5]), cvt2(v[6], v[7])};
  return __builtin_bit_cast(bf16x8_t, u);
}

__device__ __forceinline__ bf16x8_t lds_b128(uint32_t addr) {
  return *reinterpret_cast<lds_bf16x8*>(static_cast<uintptr_t>(addr));
}

__device__ __forceinline__ s16x4_t lds_tr16(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4*>(
      static_cast<uintptr_t>(addr)));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)(p)));
}

// Keep a value in a register as computed (no reassociation or hoisting).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Work-unit index of workgroup x: consecutive splits of a sequence go to the
// same XCD (workgroups are dealt to the 8 XCDs round robin).
__device__ __forceinline__ int unit_of(int x, int units) {
  if ((units & 7) != 0) return x;
  return (x & 7) * (units >> 3) + (x >> 3);
}

// vmcnt(n) with expcnt/lgkmcnt left alone (gfx9 encoding of s_waitcnt).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that neither waits for outstanding global->LDS copies nor
// lets the compiler move memory operations across it; completion of the
// copies is ordered explicitly with wait_vmcnt.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One wave-wide asynchronous copy global -> LDS: lane l's 16 bytes at
// gbase + voff land at LDS byte address lds + 16*l.  Written as inline asm so
// that the compiler does not track it (it would otherwise drain every
// outstanding copy before each LDS read it cannot prove disjoint); completion
// is ordered explicitly with wait_vmcnt + lds_barrier.  The block writes no
// VGPR; M0 (the LDS base) is saved and restored and gets one wait state.
__device__ __forceinline__ void dma_block(uint64_t gbase, uint32_t voff, uint32_t lds) {
  // both bases are wave-uniform by construction; make that explicit for the SGPR
  // operands (readfirstlane yields int: widen through uint32_t, never sign-extend)
  lds = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(lds)));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(gbase >> 32))));
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(gbase))));
  gbase = (static_cast<uint64_t>(hi) << 32) | static_cast<uint64_t>(lo);
  uint32_t save;
  // s_nop 4: five wait states between any VALU write of the base SGPRs and the
  // vector-memory read of them (a hazard the compiler does not see inside asm)
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 4\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(voff), "s"(gbase), "s"(lds)
      : "memory");
}

// Start the asynchronous copy of the tile at `tok0` (32 rows of one page) into
// the ring slot at LDS address `slot`.  Wave wv copies latent rows 4wv..4wv+3
// and, for wv < 4, RoPE block wv (5 or 4 copies).  In a partial tile, rows past
// the split's end re-read row 0 (finite data whose score is masked); a page
// outside the pool reads pool row 0 (and is flagged).
__device__ __forceinline__ void tile_issue(const char* __restrict__ pool, int page, bool ok,
                                           int tok0, int t1, uint32_t slot, int wv, int lane) {
  const int nvalid = ok ? min(kTileTok, t1 - tok0) : 0;
  const uint64_t tile = reinterpret_cast<uint64_t>(
      ok ? pool + (static_cast<int64_t>(page) * kPage + (tok0 & (kPage - 1))) * kRowBytes : pool);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 4 * wv + q;
    dma_block(tile + (r < nvalid ? r : 0) * kRowBytes, 16 * (lane ^ ukey(r)), slot + 1024 * r);
  }
  if (wv < 4) {
    const int rr = 8 * wv + (lane >> 3);
    const uint32_t voff =
        (rr < nvalid ? rr : 0) * kRowBytes + 2 * kDc + 16 * ((lane & 7) ^ vkey(rr));
    dma_block(tile, voff, slot + kRopeOff + 1024 * wv);
  }
}

// Wait until this wave's copies of the current tile have landed, `after` tiles
// (0..kStages-2) having been issued since; waves 0..3 issue 5 copies per tile,
// waves 4..7 issue 4.
__device__ __forceinline__ void wait_tile(int after, bool five) {
  if (after >= 3) {
    if (five) wait_vmcnt<15>(); else wait_vmcnt<12>();
  } else if (after == 2) {
    if (five) wait_vmcnt<10>(); else wait_vmcnt<8>();
  } else if (after == 1) {
    if (five) wait_vmcnt<5>(); else wait_vmcnt<4>();
  } else {
    wait_vmcnt<0>();
  }
}

__global__ __launch_bounds__(kThreads, 1) void k_attn_mfma_h128(
    AttnArgs a, const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    const char* __restrict__ pool) {
  __shared__ __attribute__((aligned(1024))) char ring[kStages * kTileBytes];
  __shared__ __attribute__((aligned(16))) float xch[kWaves][16];
  // k-steps kQReg.. of every wave's Q fragments: [wave][k-step][lane] x 16 B
  __shared__ __attribute__((aligned(16))) bf16x8_t qlds[kWaves][kQLds][64];
  // page ids of the split's pages [wbase, wbase + kPageWin): a copy in LDS, so
  // a tile's page costs a short LDS read instead of a scalar memory load whose
  // wait would also block every LDS wait behind it
  __shared__ int pwin[kPageWin];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4;            // k-group of the MFMA operands
  const int n16 = lane & 15;          // head (scores) / column (P.C output) of this lane
  const int S = a.num_splits;
  const int unit = unit_of(blockIdx.x, a.batch * S);
  const int b = unit / S, s = unit - b * S;
  const int nh = 128;

  int L = seq_lens[b];
  if (L < 0 || L > a.max_pages * kPage) {
    if (tid == 0) set_err(a.err, ERR_POS);
    L = 0;
  }
  int t0, t1;
  split_range(L, S, s, kPage, &t0, &t1);

  const int64_t ob = (static_cast<int64_t>(b) * S + s) * nh + 16 * wv;
  float* o_out = a.o_part + ob * kDc;
  float* lse_out = a.lse_part + ob;

  if (t0 >= t1) {  // empty split (uniform across the workgroup)
    for (int e = lane; e < 16 * kDc; e += 64) o_out[e] = 0.f;
    if (lane < 16) lse_out[lane] = -INFINITY;
    return;
  }
  const int32_t* bt = block_table + static_cast<int64_t>(b) * a.max_pages;
  const int p_first = t0 / kPage, p_end = (t1 - 1) / kPage + 1;
  int wbase = -1;
  // (uniform) make pwin hold pages [base, base + kPageWin); drains every copy
  auto load_window = [&](int base) {
    wait_vmcnt<0>();
    lds_barrier();                       // nobody still reads the old window
    for (int i = tid; i < kPageWin; i += kThreads) {
      const int pg = base + i;
      pwin[i] = pg < p_end ? bt[pg] : 0;
    }
    __syncthreads();
    wbase = base;
  };

  // ---- this wave's queries as MFMA B fragments: head 16wv + n16, k = 32ks + 8g + j
  bf16x8_t qf[kQReg];
  {
    const int h = 16 * wv + n16;
    const float* ql = a.q_lat + (static_cast<int64_t>(b) * nh + h) * kDc + 8 * g;
    const float* qp = a.q_pe + (static_cast<int64_t>(b) * nh + h) * kDr + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      const float* src = ks < kDc / 32 ? ql + 32 * ks : qp + 32 * (ks - kDc / 32);
      float v[8];
      const float4 lo = *reinterpret_cast<const float4*>(src);
      const float4 hi = *reinterpret_cast<const float4*>(src + 4);
      v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
      v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
      if (ks < kQReg) qf[ks] = pack8(v);
      else qlds[wv][ks - kQReg][lane] = pack8(v);
    }
  }
  const uint32_t qtail = lds_addr(&qlds[wv][0][lane]);

  // ---- per-lane constant offsets inside a tile
  // score A fragment, token row 16tb + n16, latent chunk 4ks + g:
  //   soff[ks & 3] + 256 (ks >> 2) + 16384 tb; RoPE chunk 4(ks-16) + g: roff[ks-16] + 2048 tb
  const int u = ukey(n16), v = vkey(n16);
  uint32_t soff[4], roff[2];
#pragma unroll
  for (int q = 0; q < 4; ++q) soff[q] = 1024 * n16 + 16 * ((4 * q + g) ^ u);
#pragma unroll
  for (int q = 0; q < 2; ++q)
    roff[q] = kRopeOff + 1024 * (n16 >> 3) + 128 * (n16 & 7) + 16 * ((4 * q + g) ^ v);
  // P.C B fragment, transposed read: this lane addresses token row rt (+16 for
  // the second half) and columns 16nb + 4(n16 & 3)..+3: toff[nb & 7] + 256 (nb >> 3)
  const int rt = 4 * g + (n16 >> 2);
  const int wt = ((n16 & 3) >> 1) ^ ukey(rt);
  uint32_t toff[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) toff[m] = 1024 * rt + 16 * ((2 * m) ^ wt) + 8 * (n16 & 1);
  const uint32_t ring0 = lds_addr(ring);
  const bool five = wv < 4;

  f32x4_t o[kColBlocks];
  float m_ref = -INFINITY;   // exponent reference (log2 units) of head n16
  float l_sum = 0.f;         // sum of exp2(x - m_ref) of head n16
  const float cs = a.scale * kLog2e;
  bool bad_page = false;
  const int ntiles = (t1 - t0 + kTileTok - 1) / kTileTok;

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int nb = 0; nb < kColBlocks; ++nb) o[nb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    l_sum = 0.f;
    float seen = m_ref;        // largest tile maximum met in this pass
    bool over = false;

    if (wbase != p_first) load_window(p_first);
    for (int j = 0; j < kStages - 1 && j < ntiles; ++j) {
      const int tok = t0 + j * kTileTok;
      const int pg = pwin[tok / kPage - wbase];
      tile_issue(pool, pg, pg >= 0 && pg < a.num_pages, tok, t1, ring0 + j * kTileBytes, wv, lane);
    }

    int cur = 0;                                       // slot of tile `it`
    for (int it = 0; it < ntiles; ++it) {
      const int tok0 = t0 + it * kTileTok;
      wait_tile(min(ntiles - 1 - it, kStages - 2), five);
      lds_barrier();   // tile `it` is in LDS for every wave; the slot of tile it-1 is free
      const int page = pwin[tok0 / kPage - wbase];
      const bool ok = page >= 0 && page < a.num_pages;
      bad_page |= !ok;
      const int nvalid = ok ? min(kTileTok, t1 - tok0) : 0;
      if (it + kStages - 1 < ntiles) {
        const int tok = tok0 + (kStages - 1) * kTileTok;
        if (tok / kPage - wbase >= kPageWin) load_window(tok / kPage);   // splits > 2048 pages
        const int pg = pwin[tok / kPage - wbase];
        const int nxt = cur == 0 ? kStages - 1 : cur - 1;
        tile_issue(pool, pg, pg >= 0 && pg < a.num_pages, tok, t1, ring0 + nxt * kTileBytes, wv,
                   lane);
      }
      const uint32_t T = ring0 + cur * kTileBytes;
      cur = cur == kStages - 1 ? 0 : cur + 1;

      // ---- scores S^T (tokens x heads): two 16-token blocks, independent chains
      f32x4_t sc[2] = {(f32x4_t){0.f, 0.f, 0.f, 0.f}, (f32x4_t){0.f, 0.f, 0.f, 0.f}};
      {
        uint32_t sa[4], ra[2];
#pragma unroll
        for (int q = 0; q < 4; ++q) sa[q] = opaque(T + soff[q]);
#pragma unroll
        for (int q = 0; q < 2; ++q) ra[q] = opaque(T + roff[q]);
        auto lda = [&](int ks, int tb) {
          return ks < kDc / 32 ? lds_b128(sa[ks & 3] + 256 * (ks >> 2) + 16384 * tb)
                               : lds_b128(ra[ks - kDc / 32] + 2048 * tb);
        };
        // operands of step ks: A for both token blocks and, past kQReg, B from LDS
        bf16x8_t af[2][3];
        auto ld_step = [&](int ks, bf16x8_t (&dst)[3]) {
          dst[0] = lda(ks, 0);
          dst[1] = lda(ks, 1);
          if (ks >= kQReg) dst[2] = lds_b128(qtail + (ks - kQReg) * 1024);
        };
        ld_step(0, af[0]);
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
          if (ks + 1 < kKSteps) ld_step(ks + 1, af[(ks + 1) & 1]);
          const bf16x8_t qb = ks < kQReg ? qf[ks < kQReg ? ks : 0] : af[ks & 1][2];
          sc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks & 1][0], qb, sc[0], 0, 0, 0);
          sc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks & 1][1], qb, sc[1], 0, 0, 0);
        }
      }

      // ---- softmax weights of head n16 for tokens 16tb + 4g + i
      if (nvalid < kTileTok) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * tb + 4 * g + i >= nvalid) sc[tb][i] = -INFINITY;
      }
      float tmax = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                         fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * cs;
      if (m_ref == -INFINITY) m_ref = tmax;      // first scored tile fixes the reference
      seen = fmaxf(seen, tmax);
      over |= tmax > m_ref + kHeadroom;
      const float mr = fmaxf(m_ref, -1e30f);
      float pv[8];
      float psum = 0.f;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[4 * tb + i] = __builtin_amdgcn_exp2f(fminf(fmaf(sc[tb][i], cs, -mr), kHeadroom));
          psum += pv[4 * tb + i];
        }
      psum += __shfl_xor(psum, 16, 64);
      psum += __shfl_xor(psum, 32, 64);
      l_sum += psum;
      const bf16x8_t pp = pack8(pv);   // k order t(g, j) = 16(j >> 2) + 4g + (j & 3)

      // ---- O += P . C  (B operand via transposed LDS reads), four products ahead
      {
        s16x4_t bv[2][2][2];
        auto load_grp = [&](int grp, s16x4_t (&dst)[2][2]) {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int nb = 2 * grp + q;
            const uint32_t p0 = T + toff[nb & 7] + 256 * (nb >> 3);
            dst[q][0] = lds_tr16(p0);
            dst[q][1] = lds_tr16(p0 + 16384);
          }
        };
        load_grp(0, bv[0]);
#pragma unroll
        for (int grp = 0; grp < kColBlocks / 2; ++grp) {
          if (grp + 1 < kColBlocks / 2) load_grp(grp + 1, bv[(grp + 1) & 1]);
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int nb = 2 * grp + q;
            const bf16x8_t bf = __builtin_bit_cast(bf16x8_t, bv[grp & 1][q]);
            o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pp, bf, o[nb], 0, 0, 0);
          }
        }
      }
    }
    // every copy has landed (the last iteration waited for all of them)
    if (!__syncthreads_or(over)) break;
    m_ref = seen;              // run the unit again with the largest maximum as reference
  }
  if (bad_page && tid == 0) set_err(a.err, ERR_PAGE);

  // ---- epilogue: o_part = O / l, lse = (m + log2 l) ln 2; lane holds heads 4g + i
  const float inv = l_sum > 0.f ? 1.f / l_sum : 0.f;
  if (g == 0) {
    xch[wv][n16] = inv;
    lse_out[n16] = l_sum > 0.f ? (m_ref + __log2f(l_sum)) * 0.6931471805599453f : -INFINITY;
  }
  __builtin_amdgcn_wave_barrier();
  const float4 il = *reinterpret_cast<const float4*>(&xch[wv][4 * g]);
  const float ilv[4] = {il.x, il.y, il.z, il.w};
#pragma unroll
  for (int nb = 0; nb < kColBlocks; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) o_out[(4 * g + i) * kDc + 16 * nb + n16] = o[nb][i] * ilv[i];
}

}  // namespace

bool fast_attention_ok(const AttnArgs& a) {
  return a.n_heads == 128 && a.d_latent == kDc && a.d_rope == kDr && a.page_size == kPage;
}

hipError_t launch_attention_fast(const AttnArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  const int units = a.batch * a.num_splits;
  hipLaunchKernelGGL(k_attn_mfma_h128, dim3(units), dim3(kThreads), 0, stream, a, a.block_table,
                     a.seq_lens, static_cast<const char*>(a.pool));
  return hipGetLastError();
}

// Log-sum-exp merge of split partials: one wave per (sequence, head) row, one
// float4 of the row per lane and split, so every byte of o_part is read once
// with 16-byte coalesced loads.  The split weights exp(lse_s - max) are
// wave-uniform and recomputed by every lane.
__global__ __launch_bounds__(256) void k_merge_rows(MergeArgs a, int rows) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int nh = a.n_heads, S = a.num_splits, dq = a.d_latent / 4;
  const int b = row / nh, i = row - b * nh;
  const float* lse = a.lse_part + static_cast<int64_t>(b) * S * nh + i;
  float m = -INFINITY;
  for (int s = lane; s < S; s += 64) m = fmaxf(m, lse[static_cast<int64_t>(s) * nh]);
  m = wave_max(m);
  const float4* src =
      reinterpret_cast<const float4*>(a.o_part) + (static_cast<int64_t>(b) * S * nh + i) * dq;
  const int64_t split_stride = static_cast<int64_t>(nh) * dq;   // float4s between splits
  float4* dst = reinterpret_cast<float4*>(a.o_lat) + static_cast<int64_t>(row) * dq;
  float z = 0.f;
  for (int v = lane; v < dq; v += 64) {   // lane 0 always runs: dq >= 1
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float zz = 0.f;
    if (m != -INFINITY) {
#pragma unroll 4
      for (int s = 0; s < S; ++s) {
        const float l = lse[static_cast<int64_t>(s) * nh];
        const float w = l == -INFINITY ? 0.f : __expf(l - m);
        zz += w;
        if (w != 0.f) {
          const float4 x = src[s * split_stride + v];
          acc.x += w * x.x; acc.y += w * x.y; acc.z += w * x.z; acc.w += w * x.w;
        }
      }
    }
    z = zz;
    const float inv = zz > 0.f ? 1.f / zz : 0.f;
    dst[v] = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
  if (a.lse && lane == 0) a.lse[row] = z > 0.f ? m + __logf(z) : -INFINITY;
}

bool fast_merge_ok(const MergeArgs& a) {
  return a.d_latent % 4 == 0 && (reinterpret_cast<uintptr_t>(a.o_part) & 15) == 0 &&
         (reinterpret_cast<uintptr_t>(a.o_lat) & 15) == 0 &&
         static_cast<int64_t>(a.batch) * a.n_heads < (int64_t{1} << 31) - 4;
}

hipError_t launch_merge_fast(const MergeArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  const int rows = a.batch * a.n_heads;
  hipLaunchKernelGGL(k_merge_rows, dim3((rows + 3) / 4), dim3(256), 0, stream, a, rows);
  return hipGetLastError();
}

}  // namespace mla
