// MFMA kernels for gfx950 (CDNA4 matrix cores, wave64).
//
// Split-KV latent attention, the hot loop of the decode step
// ([Report] §2.3/§2.4 of "《DeepSeek-V2》深度解读报告": every head scores the
// same cached latent rows [c | k^R]; s = tau (q_lat . c + q_pe . k^R)).
//
// Work unit = (sequence b, split s).  A 256-thread workgroup (4 waves) streams
// the split's rows in tiles of 32 tokens (32 rows x 1152 bytes, contiguous
// inside one 64-row page) through a 3-slot LDS ring filled by asynchronous
// global->LDS copies (global_load_lds_dwordx4), two tiles ahead of the one
// consumed.  Wave w owns heads 32w..32w+31:
//   scores  S^T[t, h] = sum_k C[t, k] Q[h, k]   (M = 32 tokens, N = 32 heads,
//           K = 576, 36 x mfma_f32_32x32x16_bf16; A = tile rows from LDS,
//           B = the wave's queries: 27 k-steps in VGPRs, 9 in LDS)
//   softmax per head in the exp2 domain, in-lane plus one cross-half
//           max/sum.  The exponent reference of each head is fixed at the
//           maximum of its first scored tile, so the accumulator is never
//           rescaled and stays in AGPRs; later scores may exceed it by up to
//           2^64 (no fp32/bf16 overflow).  A score beyond that headroom makes
//           the whole unit run again with the larger reference (at most once).
//   P.C     O[h, d] += sum_t P[h, t] C[t, d]   (M = 32 heads, N = 512 in 16
//           blocks, K = 32 tokens); the S^T accumulator registers are, after
//           conversion to bf16, exactly the A operand of this product, and the
//           B operand is read from the same tile with ds_read_b64_tr_b16
//           (hardware transpose), so no second copy exists.
// LDS tile layout: 4 row groups x 9 chunk groups of 1 KB blocks; a block holds
// 8 rows x 8 16-byte chunks (128 bytes per row), chunk c of row r stored at
// chunk c ^ key(r), key(r) = 2(r&3) + (r>>2).  One wave-wide copy fills one
// block, so every lane's global source offset is a per-lane constant, and both
// the row reads of the score product (8 rows, one chunk) and the transposed
// reads of the P.C product (4 rows, chunk pairs) hit distinct banks.  Row
// groups are padded by 128 bytes so consecutive groups alternate bank halves.
#include "common.hpp"
#include "launch_fast.hpp"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const bf16x8_t lds_bf16x8;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

constexpr int kDc = 512, kDr = 64, kPage = 64;
constexpr int kTileTok = 32;
constexpr int kRowBytes = (kDc + kDr) * 2;            // 1152
constexpr int kChunkGroups = kRowBytes / 128;         // 9
constexpr int kBlockBytes = 1024;                     // 8 rows x 128 bytes
constexpr int kRowGroupBytes = kChunkGroups * kBlockBytes + 128;  // 9344
constexpr int kTileBytes = 4 * kRowGroupBytes;        // 37376
constexpr int kThreads = 256, kWaves = 4;
constexpr int kBlocksPerTile = 4 * kChunkGroups;      // 36
constexpr int kDmaPerWave = kBlocksPerTile / kWaves;  // 9 copies per wave per tile
constexpr int kKSteps = (kDc + kDr) / 16;             // 36
constexpr int kQReg = 27;                             // k-steps of Q held in VGPRs
constexpr int kQLds = kKSteps - kQReg;                // k-steps of Q held in LDS
constexpr int kStages = 3;                            // LDS ring depth
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kHeadroom = 64.0f;                    // log2 units above the reference

__device__ __forceinline__ int rkey(int r8) { return 2 * (r8 & 3) + (r8 >> 2); }

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
// the ring slot at LDS address `slot`.  Wave wv copies blocks wv, wv+4, ...;
// `voff` is the lane's source offset inside a block of a full tile.  In a
// partial tile, rows past the split's end re-read row 0 (finite data whose
// score is masked); a page outside the pool reads pool row 0 (and is flagged).
__device__ __forceinline__ void tile_issue(const char* __restrict__ pool, int page, bool ok,
                                           int tok0, int t1, uint32_t slot, int wv, int lane,
                                           uint32_t voff) {
  const int nvalid = ok ? min(kTileTok, t1 - tok0) : 0;
  const uint64_t tile = reinterpret_cast<uint64_t>(
      ok ? pool + (static_cast<int64_t>(page) * kPage + (tok0 & (kPage - 1))) * kRowBytes : pool);
  if (nvalid == kTileTok) {
#pragma unroll
    for (int r = 0; r < kDmaPerWave; ++r) {
      const int bi = r * kWaves + wv, rg = bi / kChunkGroups, cg = bi - rg * kChunkGroups;
      dma_block(tile + rg * 8 * kRowBytes + cg * 128, voff,
                slot + rg * kRowGroupBytes + cg * kBlockBytes);
    }
  } else {
    const int r8 = lane >> 3, c8 = (lane & 7) ^ rkey(lane >> 3);
#pragma unroll
    for (int r = 0; r < kDmaPerWave; ++r) {
      const int bi = r * kWaves + wv, rg = bi / kChunkGroups, cg = bi - rg * kChunkGroups;
      const int row = rg * 8 + r8;
      const uint32_t off = (row < nvalid ? row : 0) * kRowBytes + (cg * 8 + c8) * 16;
      dma_block(tile, off, slot + rg * kRowGroupBytes + cg * kBlockBytes);
    }
  }
}

__global__ __launch_bounds__(kThreads, 1) void k_attn_mfma_h128(
    AttnArgs a, const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    const char* __restrict__ pool) {
  __shared__ __attribute__((aligned(1024))) char ring[kStages * kTileBytes];
  // k-steps kQReg.. of every wave's Q fragments: [wave][k-step][lane] x 16 B
  __shared__ __attribute__((aligned(16))) bf16x8_t qlds[kWaves][kQLds][64];
  __shared__ __attribute__((aligned(16))) float xch[kWaves][32];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 5;            // k-group of the MFMA operands
  const int hl = lane & 31;           // head (score N index / P.C M index) of this lane
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

  const int64_t ob = (static_cast<int64_t>(b) * S + s) * nh + 32 * wv;
  float* o_out = a.o_part + ob * kDc;
  float* lse_out = a.lse_part + ob;

  if (t0 >= t1) {  // empty split (uniform across the workgroup)
    for (int e = lane; e < 32 * kDc; e += 64) o_out[e] = 0.f;
    if (lane < 32) lse_out[lane] = -INFINITY;
    return;
  }
  const int32_t* bt = block_table + static_cast<int64_t>(b) * a.max_pages;

  // ---- this wave's queries as MFMA B fragments: head hl, k = 16kk + 8g + j
  bf16x8_t qf[kQReg];
  {
    const int h = 32 * wv + hl;
    const float* ql = a.q_lat + (static_cast<int64_t>(b) * nh + h) * kDc + 8 * g;
    const float* qp = a.q_pe + (static_cast<int64_t>(b) * nh + h) * kDr + 8 * g;
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk) {
      const float* src = kk < kDc / 16 ? ql + 16 * kk : qp + 16 * (kk - kDc / 16);
      float v[8];
      const float4 lo = *reinterpret_cast<const float4*>(src);
      const float4 hi = *reinterpret_cast<const float4*>(src + 4);
      v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
      v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
      if (kk < kQReg) qf[kk] = pack8(v);
      else qlds[wv][kk - kQReg][lane] = pack8(v);
    }
  }
  const uint32_t qtail = lds_addr(&qlds[wv][0][lane]);

  // ---- per-lane constant offsets inside a tile
  // copy: lane l of a block moves row l>>3, logical chunk (l&7)^key(l>>3)
  const uint32_t voff = (lane >> 3) * kRowBytes + (((lane & 7) ^ rkey(lane >> 3)) << 4);
  // score A fragment: row trow, chunk 2kk+g -> soff[kk&3] + 1024*(kk>>2)
  const int trow = lane & 31, tr8 = trow & 7;
  uint32_t soff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    soff[q] = (trow >> 3) * kRowGroupBytes + tr8 * 128 + (((2 * q + g) ^ rkey(tr8)) << 4);
  // P.C B fragment (transposed read): rows 16mi+8h+r8, chunk 4nb+2(G&1)+((i16&3)>>1)
  //   -> toff[nb&1] + kRowGroupBytes*(2mi+h) + 1024*(nb>>1)
  const int i16 = lane & 15, G = lane >> 4;
  const int r8t = 4 * (G >> 1) + (i16 >> 2);
  uint32_t toff[2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
    toff[q] = r8t * 128 + (((4 * q + 2 * (G & 1) + ((i16 & 3) >> 1)) ^ rkey(r8t)) << 4) +
              8 * (i16 & 1);
  const uint32_t ring0 = lds_addr(ring);

  f32x16_t o[kDc / 32];
  float m_ref = -INFINITY;   // exponent reference (log2 units) of head hl
  float l_sum = 0.f;         // sum of exp2(x - m_ref) of head hl
  const float cs = a.scale * kLog2e;
  bool bad_page = false;
  const int ntiles = (t1 - t0 + kTileTok - 1) / kTileTok;

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int nb = 0; nb < kDc / 32; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[nb][i] = 0.f;
    l_sum = 0.f;
    float seen = m_ref;        // largest tile maximum met in this pass
    bool over = false;

    for (int j = 0; j < kStages - 1 && j < ntiles; ++j) {
      const int tok = t0 + j * kTileTok;
      const int pg = bt[tok / kPage];
      tile_issue(pool, pg, pg >= 0 && pg < a.num_pages, tok, t1, ring0 + j * kTileBytes, wv, lane,
                 voff);
    }

    uint32_t cur = 0;                                  // slot offset of tile `it`
    for (int it = 0; it < ntiles; ++it) {
      const int tok0 = t0 + it * kTileTok;
      // copies issued after tile `it`: tile it+1 (if any)
      if (it + 1 < ntiles) wait_vmcnt<kDmaPerWave>();
      else wait_vmcnt<0>();
      lds_barrier();   // tile `it` is in LDS for every wave; the slot of tile it-1 is free
      const uint32_t nxt = cur == 0 ? (kStages - 1) * kTileBytes : cur - kTileBytes;
      if (it + kStages - 1 < ntiles) {
        const int tok = tok0 + (kStages - 1) * kTileTok;
        const int pg = bt[tok / kPage];
        tile_issue(pool, pg, pg >= 0 && pg < a.num_pages, tok, t1, ring0 + nxt, wv, lane, voff);
      }
      const int page = bt[tok0 / kPage];
      const bool ok = page >= 0 && page < a.num_pages;
      bad_page |= !ok;
      const int nvalid = ok ? min(kTileTok, t1 - tok0) : 0;
      const uint32_t T = ring0 + cur;
      cur = cur == (kStages - 1) * kTileBytes ? 0 : cur + kTileBytes;

      // ---- scores S^T (tokens x heads)
      uint32_t sa[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) sa[q] = opaque(T + soff[q]);
      f32x16_t sc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = 0.f;
      {
        bf16x8_t af[2][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) af[0][q] = lds_b128(sa[q]);
#pragma unroll
        for (int grp = 0; grp < kKSteps / 4; ++grp) {
          if (grp + 1 < kKSteps / 4) {
#pragma unroll
            for (int q = 0; q < 4; ++q) af[(grp + 1) & 1][q] = lds_b128(sa[q] + 1024 * (grp + 1));
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int kk = 4 * grp + q;
            const bf16x8_t qb = kk < kQReg ? qf[kk < kQReg ? kk : 0]
                                           : lds_b128(qtail + (kk - kQReg) * 1024);
            sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[grp & 1][q], qb, sc, 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // ---- softmax weights of head hl for the tile's tokens 8(i/4)+4g+(i%4)
      if (nvalid < kTileTok) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int tok = 8 * (i >> 2) + 4 * g + (i & 3);
          if (tok >= nvalid) sc[i] = -INFINITY;
        }
      }
      float tmax = sc[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) tmax = fmaxf(tmax, sc[i]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * cs;
      if (m_ref == -INFINITY) m_ref = tmax;      // first scored tile fixes the reference
      seen = fmaxf(seen, tmax);
      over |= tmax > m_ref + kHeadroom;
      const float mr = fmaxf(m_ref, -1e30f);
      float psum = 0.f;
      float pv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(fminf(fmaf(sc[i], cs, -mr), kHeadroom));
        psum += pv[i];
      }
      psum += __shfl_xor(psum, 32, 64);
      l_sum += psum;
      const bf16x8_t pp[2] = {pack8(pv), pack8(pv + 8)};   // tokens 0..15 / 16..31

      // ---- O += P . C  (B operand via transposed LDS reads), four MFMAs ahead
      {
        uint32_t ta[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) ta[q] = opaque(T + toff[q]);
        s16x4_t bv[2][4][2];
        auto load_grp = [&](int grp, s16x4_t (&dst)[4][2]) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int f = 4 * grp + q, mi = f >> 4, nb = f & 15;
            const uint32_t p0 = ta[nb & 1] + kRowGroupBytes * 2 * mi + 1024 * (nb >> 1);
            dst[q][0] = lds_tr16(p0);
            dst[q][1] = lds_tr16(p0 + kRowGroupBytes);
          }
        };
        load_grp(0, bv[0]);
#pragma unroll
        for (int grp = 0; grp < 8; ++grp) {
          if (grp + 1 < 8) load_grp(grp + 1, bv[(grp + 1) & 1]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int f = 4 * grp + q, mi = f >> 4, nb = f & 15;
            const bf16x8_t bf = __builtin_bit_cast(bf16x8_t, bv[grp & 1][q]);
            o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pp[mi], bf, o[nb], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // every copy has landed (the last iteration waited for all of them)
    if (!__syncthreads_or(over)) break;
    m_ref = seen;              // run the unit again with the largest maximum as reference
  }
  if (bad_page && tid == 0) set_err(a.err, ERR_PAGE);

  // ---- epilogue: o_part = O / l, lse = (m + log2 l) ln 2
  const float inv = l_sum > 0.f ? 1.f / l_sum : 0.f;
  if (g == 0) {
    xch[wv][hl] = inv;
    lse_out[hl] = l_sum > 0.f ? (m_ref + __log2f(l_sum)) * 0.6931471805599453f : -INFINITY;
  }
  __builtin_amdgcn_wave_barrier();
  float il[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v = *reinterpret_cast<const float4*>(&xch[wv][8 * q + 4 * g]);
    il[4 * q] = v.x; il[4 * q + 1] = v.y; il[4 * q + 2] = v.z; il[4 * q + 3] = v.w;
  }
#pragma unroll
  for (int nb = 0; nb < kDc / 32; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int hh = 8 * (i >> 2) + 4 * g + (i & 3);
      o_out[hh * kDc + 32 * nb + hl] = o[nb][i] * il[i];
    }
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

bool fast_merge_ok(const MergeArgs&) { return false; }
hipError_t launch_merge_fast(const MergeArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace mla
