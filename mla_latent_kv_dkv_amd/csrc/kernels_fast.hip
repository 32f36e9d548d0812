// MFMA kernels for gfx950 (CDNA4 matrix cores, wave64).
//
// Split-KV latent attention, the hot loop of the decode step
// ([Report] §2.3/§2.4 of "《DeepSeek-V2》深度解读报告": every head scores the
// same cached latent rows [c | k^R]; s = tau (q_lat . c + q_pe . k^R)).
//
// Two kernels share the structure below: k_attn_mfma_h128 for a bf16 pool and
// k_attn_f8mma_h128 for the FP8 pool (its own header further down: the codes go
// into the FP8 matrix instruction as stored).
//
// Work unit = (sequence b, split s).  A 256-thread workgroup (4 waves, one per
// SIMD) streams the split's rows in tiles of 32 tokens (32 rows x 1152 bytes,
// contiguous inside one 64-row page) through a 4-slot LDS ring filled by
// asynchronous global->LDS copies (global_load_lds_dwordx4), two tiles ahead.
// Wave w owns heads 32w..32w+31 and uses mfma_f32_32x32x16_bf16 throughout:
//   scores  S^T[t, h] = sum_k C[t, k] Q[h, k]   (M = the tile's 32 tokens,
//           N = the wave's 32 heads, K = 576 in 36 steps; A = tile rows from
//           LDS, B = the wave's queries, all 36 k-steps held in VGPRs for the
//           whole unit).  The accumulator stays in VGPRs (inline asm).
//   softmax per head in the exp2 domain.  The exponent reference of each head
//           is fixed at the maximum of the split's first tile, so the output
//           accumulator is never rescaled; a later score more than 2^64 above
//           it makes the whole unit run again with the split's maximum as
//           reference (at most once).  Row sums and maxima stay per lane and
//           are combined across the two lanes of a head at the end.
//   P.C     O[h, d] += sum_t P[h, t] C[t, d]   (M = 32 heads, N = 512 in 16
//           blocks, K = 32 tokens in 2 steps).  O (32 x 512 fp32 per wave)
//           lives in the 256 AGPRs.  A lane's score accumulator holds head
//           32w + (lane & 31) and tokens 8(i >> 2) + 4(lane >> 5) + (i & 3);
//           taking the contraction's k order as t = 16kk + 8(j >> 2) +
//           4(lane >> 5) + (j & 3) makes the packed weights exactly the A
//           operand, and the B operand (4 tokens of one column per half) is
//           one ds_read_b64_tr_b16 (hardware transpose) per half.
// Pipeline: iteration t computes the scores of tile t, then the products of
// tile t-1 with the weights of tile t computed between them, so the softmax
// arithmetic runs in the shadow of the matrix products; tiles t-1, t and the
// two in flight occupy the 4 slots.
// LDS tile layout (38 KB): latent row r at 1088 r (1 KB + 64 bytes of pad),
// its 16-byte chunk c at c ^ ((r >> 2) & 3); the 64 RoPE values of rows
// 8j..8j+7 fill the 1 KB block j after the latent rows, row r at 128 (r & 7),
// chunk c' at c' ^ ((r >> 1) & 7).  Every copy fills 1 KB.  LDS has 64 banks
// of 4 bytes; a ds_read_b128 is served in four 16-lane phases (lanes with
// equal lane >> 5 and equal parity of bits 2..4 of the lane), a
// ds_read_b64(_tr_b16) in two 32-lane phases (lane >> 5).  Under this layout
// no phase of a score read (16 rows, one chunk) or of a transposed read (4
// rows, 4 chunks) puts two addresses on one bank, and the per-step offsets of
// both reads are instruction immediates.
#include <type_traits>

#include "common.hpp"
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
typedef __attribute__((address_space(3))) const bf16x8_t lds_bf16x8;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

constexpr int kDc = 512, kDr = 64, kPage = 64;
constexpr int kTileTok = 32;
constexpr int kRowBytes = (kDc + kDr) * 2;            // 1152: one cached row
constexpr int kPitch = 1088;                          // LDS bytes per latent row (1 KB + pad)
constexpr int kRopeOff = kTileTok * kPitch;           // RoPE blocks follow the 32 latent rows
constexpr int kTileBytes = kRopeOff + (kTileTok / 8) * 1024;   // 38912
constexpr int kThreads = 256, kWaves = 4;             // one wave per SIMD
constexpr int kHeads = 32;                            // heads of one wave
constexpr int kKSteps = (kDc + kDr) / 16;             // 36 score k-steps
constexpr int kLatSteps = kDc / 16;                   // 32 of them over the latent part
constexpr int kColBlocks = kDc / 32;                  // 16 output column blocks
constexpr int kStages = 4;                            // LDS ring depth
constexpr int kCopies = 9;                            // copies per wave per tile
constexpr int kARing = 6;                             // score operands in flight
constexpr int kBRing = 4;                             // P.C operand pairs in flight
constexpr int kPageWin = 512;                         // page ids of the split held in LDS
constexpr float kLog2e = 1.4426950408889634f;
// FP8 pool: a page is 64 rows of [512 e4m3 | 64 bf16] (640 bytes), then 64 fp32
// row scales.  A tile is staged in LDS as its codes, its k^R block and its 32
// scales (k_attn_f8mma_h128 below).
constexpr int kF8Row = kDc + 2 * kDr;                  // 640
constexpr int kF8ScaleOff = kPage * kF8Row;             // 40960
constexpr int64_t kF8PageBytes = kF8ScaleOff + 4 * kPage;   // 41216
constexpr int kF8RopeOff = kTileTok * kDc;              // 16384: k^R block of a staged tile
constexpr int kF8ScaleLds = kF8RopeOff + kTileTok * 2 * kDr;   // 20480: its scales
constexpr int kF8Stage = kF8ScaleLds + 4 * kTileTok;    // 20608
constexpr int kF8Copies = 6;                            // copies per wave per tile
constexpr float kHeadroom = 64.0f;                    // log2 units above the reference

// 16-byte chunk c of latent row r sits at chunk c ^ lkey(r) of the row's
// 1 KB (at kPitch r); chunk c' of the RoPE part of row r at chunk c' ^ rkey(r)
// of its 128 bytes.
__device__ __forceinline__ int lkey(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int rkey(int r) { return (r >> 1) & 7; }

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

// Keep a value in a register as computed (no reassociation or hoisting).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Score products with the accumulator in VGPRs.  Written as inline asm
// because the builtin takes the AGPR-accumulator form in a kernel that may use
// more than 256 registers, and here the 256 AGPRs hold the P.C accumulators.
// Wait states: back-to-back products on the same accumulator need none; a
// VALU read of the result needs 12 after the last one (16 are given), and the
// first product keeps 2 after any VALU write of registers it takes over.
__device__ __forceinline__ f32x16_t mfma_v_first(const bf16x8_t& a, const bf16x8_t& b) {
  f32x16_t d;
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ void mfma_v(f32x16_t& d, const bf16x8_t& a, const bf16x8_t& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v_last(f32x16_t& d, const bf16x8_t& a, const bf16x8_t& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 15" : "+v"(d) : "v"(a), "v"(b));
}

// Work-unit index of workgroup x: consecutive splits of a sequence go to the
// same XCD (workgroups are dealt to the 8 XCDs round robin).
__device__ __forceinline__ int unit_of(int x, int units) {
  if ((units & 7) != 0) return x;
  return (x & 7) * (units >> 3) + (x >> 3);
}

// lgkmcnt(n) with vmcnt/expcnt left alone (gfx9 encoding of s_waitcnt; n <= 15).
__device__ __forceinline__ void wait_lgkm(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0xC07F); break;
    case 1: __builtin_amdgcn_s_waitcnt(0xC17F); break;
    case 2: __builtin_amdgcn_s_waitcnt(0xC27F); break;
    case 3: __builtin_amdgcn_s_waitcnt(0xC37F); break;
    case 4: __builtin_amdgcn_s_waitcnt(0xC47F); break;
    case 5: __builtin_amdgcn_s_waitcnt(0xC57F); break;
    case 6: __builtin_amdgcn_s_waitcnt(0xC67F); break;
    case 7: __builtin_amdgcn_s_waitcnt(0xC77F); break;
    case 8: __builtin_amdgcn_s_waitcnt(0xC87F); break;
    case 9: __builtin_amdgcn_s_waitcnt(0xC97F); break;
    case 10: __builtin_amdgcn_s_waitcnt(0xCA7F); break;
    default: __builtin_amdgcn_s_waitcnt(0xCB7F); break;
  }
}

// Start the asynchronous copy of the tile at `tok0` (32 rows of one page) into
// the ring slot at LDS address `slot`.  Wave wv copies latent rows
// 8wv..8wv+7 and RoPE block wv (rows 8wv..8wv+7): kCopies copies.  In a
// partial tile, rows past the split's end re-read row 0 (finite data whose
// score is masked); a page outside the pool reads pool row 0 (masked, and
// flagged by the caller).
template <bool kStream>
__device__ __forceinline__ void tile_issue(const char* __restrict__ pool, int page, bool ok,
                                           int tok0, int t1, uint32_t slot, int wv, int lane) {
  const int nvalid = ok ? min(kTileTok, t1 - tok0) : 0;
  const uint64_t tile = reinterpret_cast<uint64_t>(
      ok ? pool + (static_cast<int64_t>(page) * kPage + (tok0 & (kPage - 1))) * kRowBytes : pool);
  lane = static_cast<int>(opaque(static_cast<uint32_t>(lane)));   // per-copy offsets stay unhoisted
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int r = 8 * wv + q;
    dma_block<kStream>(tile + (r < nvalid ? r : 0) * kRowBytes, 16 * (lane ^ lkey(r)),
                       slot + kPitch * r);
  }
  const int rr = 8 * wv + (lane >> 3);
  const uint32_t voff =
      (rr < nvalid ? rr : 0) * kRowBytes + 2 * kDc + 16 * ((lane & 7) ^ rkey(rr));
  dma_block<kStream>(tile, voff, slot + kRopeOff + 1024 * wv);
}

// Text of the full-tile copies below; NT is the cache-policy suffix of each copy.
#define MLA_TILE_COPY_ASM(NT) \
  "s_mov_b32 %0, m0\n\t" \
  "s_mov_b32 m0, %6\n\t" \
  "s_nop 4\n\t" \
  "global_load_lds_dwordx4 %2, %5" NT "\n\t" \
  "v_add_u32 %1, 0x480, %2\n\t" \
  "s_add_u32 m0, m0, 0x440\n\t" \
  "s_nop 0\n\t" \
  "global_load_lds_dwordx4 %1, %5" NT "\n\t" \
  "v_add_u32 %1, 0x900, %2\n\t" \
  "s_add_u32 m0, m0, 0x440\n\t" \
  "s_nop 0\n\t" \
  "global_load_lds_dwordx4 %1, %5" NT "\n\t" \
  "v_add_u32 %1, 0xd80, %2\n\t" \
  "s_add_u32 m0, m0, 0x440\n\t" \
  "s_nop 0\n\t" \
  "global_load_lds_dwordx4 %1, %5" NT "\n\t" \
  "s_add_u32 m0, m0, 0x440\n\t" \
  "s_nop 0\n\t" \
  "global_load_lds_dwordx4 %3, %5" NT "\n\t" \
  "v_add_u32 %1, 0x480, %3\n\t" \
  "s_add_u32 m0, m0, 0x440\n\t" \
  "s_nop 0\n\t" \
  "global_load_lds_dwordx4 %1, %5" NT "\n\t" \
  "v_add_u32 %1, 0x900, %3\n\t" \
  "s_add_u32 m0, m0, 0x440\n\t" \
  "s_nop 0\n\t" \
  "global_load_lds_dwordx4 %1, %5" NT "\n\t" \
  "v_add_u32 %1, 0xd80, %3\n\t" \
  "s_add_u32 m0, m0, 0x440\n\t" \
  "s_nop 0\n\t" \
  "global_load_lds_dwordx4 %1, %5" NT "\n\t" \
  "s_mov_b32 m0, %7\n\t" \
  "s_nop 0\n\t" \
  "global_load_lds_dwordx4 %4, %5" NT "\n\t" \
  "s_mov_b32 m0, %0"
// The same copies for a full tile of a valid page, as one block: M0 steps by
// the LDS row pitch and the per-lane offset by the row stride, so the block
// needs one VGPR temporary and no 64-bit address arithmetic.  `voff` =
// 1152 (8 wv) + 16 (lane ^ lkey(8 wv)), `voff_hi` the same for row 8 wv + 4
// (the key changes every 4 rows), `voff_rope` the RoPE copy's offset, `lds` =
// slot + kPitch (8 wv).  Wait states: 5 after any VALU write of the SGPR
// operands, 1 after each M0 write before the copy that reads it.  kStream: the
// copies are non-temporal (decode, where each work unit reads its rows once).
template <bool kStream>
__device__ __forceinline__ void tile_issue_full(uint64_t tile, uint32_t voff, uint32_t voff_hi,
                                                uint32_t voff_rope, uint32_t lds,
                                                uint32_t lds_rope) {
  uint32_t save, tmp;
  if constexpr (kStream)
    asm volatile(MLA_TILE_COPY_ASM(" nt")
                 : "=&s"(save), "=&v"(tmp)
                 : "v"(voff), "v"(voff_hi), "v"(voff_rope), "s"(tile), "s"(lds), "s"(lds_rope)
                 : "memory");
  else
    asm volatile(MLA_TILE_COPY_ASM("")
                 : "=&s"(save), "=&v"(tmp)
                 : "v"(voff), "v"(voff_hi), "v"(voff_rope), "s"(tile), "s"(lds), "s"(lds_rope)
                 : "memory");
}
#undef MLA_TILE_COPY_ASM

// Wait until this wave's copies of a tile have landed, `after` tiles (0..2)
// having been issued since.
__device__ __forceinline__ void wait_tile(int after) {
  if (after >= 2) wait_vmcnt<2 * kCopies>();
  else if (after == 1) wait_vmcnt<kCopies>();
  else wait_vmcnt<0>();
}

// Staged FP8 tile (32 rows): the codes of row r at kDc r, its 16-byte chunk c at
// chunk c ^ f8key(r); the k^R block of row r at kF8RopeOff + 128 r, chunk c at
// c ^ rkey(r); the 32 row scales at kF8ScaleLds.  f8key puts the 16 rows that a
// 128-bit score read serves together, and the 8 rows of a transposed P.C read,
// on distinct banks.
__device__ __forceinline__ int f8key(int r) {
  return 2 * ((r & 3) | ((r >> 1) & 4)) + ((r >> 2) & 1);
}

// Start the copy of the FP8 tile at `tok0` into the staging slot at `stage`.
// Wave wv copies rows 8wv..8wv+7: their codes (four 1 KB copies of two rows
// each), their k^R (one copy) and their 8 scales (two lanes): kF8Copies
// copies.  Rows past the split's end re-read the tile's first row; a page
// outside the pool reads page 0 (the caller masks those rows and flags it).
__device__ __forceinline__ void tile_issue_f8(const char* __restrict__ pool, int page, bool ok,
                                              int tok0, int t1, uint32_t stage, int wv, int lane) {
  const int nvalid = ok ? min(kTileTok, t1 - tok0) : 0;
  const int64_t pbase = ok ? static_cast<int64_t>(page) * kF8PageBytes : 0;
  const uint64_t rows = reinterpret_cast<uint64_t>(pool + pbase + (tok0 & (kPage - 1)) * kF8Row);
  lane = static_cast<int>(opaque(static_cast<uint32_t>(lane)));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * wv + 2 * i + (lane >> 5);
    dma_block(rows, (r < nvalid ? r : 0) * kF8Row + 16 * ((lane & 31) ^ f8key(r)),
              stage + kDc * (8 * wv + 2 * i));
  }
  const int rr = 8 * wv + (lane >> 3);
  dma_block(rows, (rr < nvalid ? rr : 0) * kF8Row + kDc + 16 * ((lane & 7) ^ rkey(rr)),
            stage + kF8RopeOff + 1024 * wv);
  const uint64_t scales =
      reinterpret_cast<uint64_t>(pool + pbase + kF8ScaleOff + 4 * (tok0 & (kPage - 1)));
  if (lane < 2) dma_block(scales, 32 * wv + 16 * lane, stage + kF8ScaleLds + 32 * wv);
}

// Wait until this wave's copies of a staged tile have landed, `after` (0..3)
// tiles having been issued since.
__device__ __forceinline__ void wait_tile_f8(int after) {
  switch (after) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<kF8Copies>(); break;
    case 2: wait_vmcnt<2 * kF8Copies>(); break;
    default: wait_vmcnt<3 * kF8Copies>(); break;
  }
}

typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
__device__ __forceinline__ u32x4_t lds_ld128(uint32_t addr) {
  return *reinterpret_cast<lds_u32x4*>(static_cast<uintptr_t>(addr));
}
__device__ __forceinline__ void lds_st128(uint32_t addr, u32x4_t v) {
  *reinterpret_cast<lds_u32x4*>(static_cast<uintptr_t>(addr)) = v;
}
__device__ __forceinline__ void lds_st32(uint32_t addr, uint32_t v) {
  *reinterpret_cast<__attribute__((address_space(3))) uint32_t*>(static_cast<uintptr_t>(addr)) = v;
}
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float lds_f32(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) float*>(static_cast<uintptr_t>(addr));
}
// 8 bytes per lane, transposed across 16-lane groups: output lane i < 8 of a
// group gets byte i of the blocks of its lanes 0, 2, .., 14, lane 8 + i byte i
// of those of lanes 1, 3, .., 15
__device__ __forceinline__ u32x2_t lds_tr8(uint32_t addr) {
  typedef int i32x2_t __attribute__((ext_vector_type(2)));
  const i32x2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      reinterpret_cast<__attribute__((address_space(3))) i32x2_t*>(static_cast<uintptr_t>(addr)));
  return __builtin_bit_cast(u32x2_t, v);
}
__global__ __launch_bounds__(kThreads, 1) void k_attn_mfma_h128(
    AttnArgs a, const int32_t* __restrict__ block_table, const char* __restrict__ pool) {
  __shared__ __attribute__((aligned(1024))) char ring[kStages * kTileBytes];   // tile ring
  __shared__ __attribute__((aligned(16))) float xch[kWaves][kHeads];
  // page ids of the split's pages [wbase, wbase + kPageWin): a copy in LDS, so
  // a tile's page costs a short LDS read instead of a scalar memory load whose
  // wait would also block every LDS wait behind it
  __shared__ int pwin[kPageWin];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int g2 = lane >> 5;           // k-group of the 32x32 MFMA operands
  const int r32 = lane & 31;          // token row (scores A) / head (scores B, P.C A)
  const int unit = unit_of(blockIdx.x, a.units);
  const int nh = 128;
  // decode units read their rows once (non-temporal copies); prefill units share
  // a sequence's rows, which stay cacheable
  const bool stream = a.q_seq == nullptr;

  int b, sq, t0, t1;
  attn_unit(a, unit, tid == 0, &b, &sq, &t0, &t1);
  b = __builtin_amdgcn_readfirstlane(b);     // uniform by construction; say so for the
  sq = __builtin_amdgcn_readfirstlane(sq);   // scalar operands of the copies
  t0 = __builtin_amdgcn_readfirstlane(t0);
  t1 = __builtin_amdgcn_readfirstlane(t1);

  const int64_t ob = static_cast<int64_t>(unit) * nh + kHeads * wv;
  float* o_out = a.o_part + ob * kDc;
  float* lse_out = a.lse_part + ob;

  if (t0 >= t1) {  // empty split (uniform across the workgroup)
    for (int e = lane; e < kHeads * kDc; e += 64) o_out[e] = 0.f;
    if (lane < kHeads) lse_out[lane] = -INFINITY;
    return;
  }
  const int32_t* bt = block_table + static_cast<int64_t>(sq) * a.max_pages;
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

  // ---- this wave's queries as MFMA B fragments: head 32wv + r32, k = 16ks + 8g2 + j
  bf16x8_t qf[kKSteps];
  {
    // The wave's 32 latent query rows go into the still unused tile ring by
    // asynchronous copies, every copy of a half in flight at once (wave w at 32 KB w;
    // half hf: columns 256 hf .., row r at 1 KB r, fp32, 16-byte chunk c at
    // c ^ (r & 15), so a fragment read of 32 rows is conflict-free), and are read
    // back as bf16 fragments; the k^R part (64 columns) goes straight to registers
    // while the copies run.
    const uint32_t qst = lds_addr(ring) + 32768u * static_cast<uint32_t>(wv);
    const uint64_t qlb = reinterpret_cast<uint64_t>(
        a.q_lat + (static_cast<int64_t>(b) * nh + kHeads * wv) * kDc);
    const float* qpr = a.q_pe + (static_cast<int64_t>(b) * nh + kHeads * wv + r32) * kDr;
    float4 pe[8];   // k^R columns 16 q + 8 g2 .. + 7 of row r32
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      pe[2 * q] = *reinterpret_cast<const float4*>(qpr + 16 * q + 8 * g2);
      pe[2 * q + 1] = *reinterpret_cast<const float4*>(qpr + 16 * q + 8 * g2 + 4);
    }
    const int sw = r32 & 15;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int r = 0; r < kHeads; ++r)
        dma_block(qlb, static_cast<uint32_t>(r * kDc * 4 + hf * 1024 + 16 * (lane ^ (r & 15))),
                  qst + 1024 * r);
      wait_vmcnt<0>();   // this wave's half is in LDS (a wave reads only its own rows)
#pragma unroll
      for (int kl = 0; kl < 16; ++kl) {
        const int c0 = 4 * kl + 2 * g2;   // fp32 chunk of columns 16 kl + 8 g2 ..
        const u32x4_t x0 = lds_ld128(qst + 1024 * r32 + 16 * (c0 ^ sw));
        const u32x4_t x1 = lds_ld128(qst + 1024 * r32 + 16 * ((c0 + 1) ^ sw));
        const float v[8] = {__uint_as_float(x0[0]), __uint_as_float(x0[1]), __uint_as_float(x0[2]),
                            __uint_as_float(x0[3]), __uint_as_float(x1[0]), __uint_as_float(x1[1]),
                            __uint_as_float(x1[2]), __uint_as_float(x1[3])};
        qf[16 * hf + kl] = pack8(v);
      }
      wait_lgkm(0);   // read before the next half's copies land on the same rows
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float v[8] = {pe[2 * q].x, pe[2 * q].y, pe[2 * q].z, pe[2 * q].w,
                          pe[2 * q + 1].x, pe[2 * q + 1].y, pe[2 * q + 1].z, pe[2 * q + 1].w};
      qf[kLatSteps + q] = pack8(v);
    }
    lds_barrier();  // every wave is done with the ring before tiles are copied into it
  }

  // ---- per-lane constant offsets inside a tile
  // score A fragment, token row r32, latent chunk 2ks + g2: soff[ks & 1] + 64 (ks >> 1);
  // RoPE chunk 2q + g2 (q = ks - 32): roff[q]
  const int ky = lkey(r32), vy = rkey(r32);
  uint32_t soff[2], roff[4];
#pragma unroll
  for (int j = 0; j < 2; ++j) soff[j] = kPitch * r32 + 16 * ((2 * j + g2) ^ ky);
#pragma unroll
  for (int q = 0; q < 4; ++q) roff[q] = kRopeOff + 128 * r32 + 16 * ((2 * q + g2) ^ vy);
  // P.C B fragment of 16-lane group (ch, g2), lane s16: token row 16kk + 8jj + 4g2 + (s16 >> 2),
  // columns 32nb + 16ch + 4(s16 & 3)..+3: toff[jj] + 64 nb + 16 kPitch kk
  const int s16 = lane & 15, ch = (lane >> 4) & 1;
  const int cp = 2 * ch + ((s16 & 3) >> 1);
  uint32_t toff[2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
    toff[jj] = kPitch * (8 * jj + 4 * g2 + (s16 >> 2)) + 16 * (cp ^ (2 * jj + g2)) + 8 * (s16 & 1);
  const uint32_t ring0 = lds_addr(ring);

  // scores S^T[t, h] of the tile in slot T: lane holds head 32wv + r32 and
  // tokens 8(i >> 2) + 4g2 + (i & 3), i = 0..15
  // `hook` runs once, among the products (the next tile's copies go out there, in
  // their shadow): wave w at k-step 8w, so the four waves do not all push their
  // copies into the memory pipeline at the same moment
  auto scores = [&](uint32_t T, auto&& hook) {
    f32x16_t acc;
    const uint32_t sa0 = T + soff[0], sa1 = T + soff[1];
    auto lda = [&](int ks) {
      return ks < kLatSteps ? lds_b128((ks & 1 ? sa1 : sa0) + 64 * (ks >> 1))
                            : lds_b128(T + roff[ks < kLatSteps ? 0 : ks - kLatSteps]);
    };
    // operands of steps ks, ks+1 are awaited together; kARing - 2 steps are read ahead
    bf16x8_t ar[kARing];
#pragma unroll
    for (int d = 0; d < kARing - 2; ++d) ar[d] = lda(d);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ks += 2) {
#pragma unroll
      for (int e = 0; e < 2; ++e)
        if (ks + kARing - 2 + e < kKSteps) ar[(ks + kARing - 2 + e) % kARing] = lda(ks + kARing - 2 + e);
      const int ahead = min(kARing - 2, kKSteps - ks - 2);   // reads issued after step ks+1's
      wait_lgkm(ahead);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int k = ks + e;
        if (k == 0) acc = mfma_v_first(ar[0], qf[0]);
        else if (k == kKSteps - 1) mfma_v_last(acc, ar[k % kARing], qf[k]);
        else mfma_v(acc, ar[k % kARing], qf[k]);
      }
      if ((ks & 7) == 0 && (ks >> 3) == wv) hook();   // the waves issue their copies in turn
      __builtin_amdgcn_sched_barrier(0);
    }
    return acc;
  };
  auto mask = [&](f32x16_t& x, int nvalid) {
    if (nvalid < kTileTok) {   // partial tile only (a real branch: nvalid is uniform)
      asm volatile("");
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + 4 * g2 + (i & 3) >= nvalid) x[i] = -INFINITY;
    }
  };

  f32x16_t o[kColBlocks];
  float m_ref = -INFINITY;   // exponent reference (log2 units) of head 32wv + r32
  float l_part = 0.f;        // this lane's share of sum exp2(x - m_ref)
  const float cs = a.scale * kLog2e;
  bool bad_page = false;
  const int ntiles = (t1 - t0 + kTileTok - 1) / kTileTok;

  // per-lane offsets of the full-tile copies (rows 8wv.., 8wv+4.., RoPE block)
  const uint32_t voff_lo = kRowBytes * 8 * wv + 16 * (lane ^ lkey(8 * wv));
  const uint32_t voff_hi = kRowBytes * (8 * wv + 4) + 16 * (lane ^ lkey(8 * wv + 4));
  const uint32_t voff_rope = kRowBytes * (8 * wv + (lane >> 3)) + 2 * kDc +
                             16 * ((lane & 7) ^ rkey(8 * wv + (lane >> 3)));
  // page id of tile j, as loaded from the window (reloaded first when tile j is
  // past it; uniform), so that the wait for the read falls where the id is used
  auto page_load = [&](int j) {
    const int tok = t0 + j * kTileTok;
    if (tok / kPage - wbase >= kPageWin) load_window(tok / kPage);   // splits > kPageWin pages
    return pwin[tok / kPage - wbase];
  };
  // start the copy of tile j (page id pgv from page_load) into slot j & 3;
  // returns its count of valid rows
  auto issue_pg = [&](int j, int pgv) {
    const int tok = t0 + j * kTileTok;
    const int pg = __builtin_amdgcn_readfirstlane(pgv);   // uniform
    const bool ok = pg >= 0 && pg < a.num_pages;
    bad_page |= !ok;
    const uint32_t slot = ring0 + (j & 3) * kTileBytes;
    const int nvalid = ok ? min(kTileTok, t1 - tok) : 0;
    if (nvalid == kTileTok) {
      const uint64_t tile = reinterpret_cast<uint64_t>(
          pool + (static_cast<int64_t>(pg) * kPage + (tok & (kPage - 1))) * kRowBytes);
      if (stream)
        tile_issue_full<true>(tile, voff_lo, voff_hi, voff_rope, slot + kPitch * 8 * wv,
                              slot + kRopeOff + 1024 * wv);
      else
        tile_issue_full<false>(tile, voff_lo, voff_hi, voff_rope, slot + kPitch * 8 * wv,
                               slot + kRopeOff + 1024 * wv);
    } else if (stream) {
      tile_issue<true>(pool, pg, ok, tok, t1, slot, wv, lane);
    } else {
      tile_issue<false>(pool, pg, ok, tok, t1, slot, wv, lane);
    }
    return nvalid;
  };
  auto issue = [&](int j) { return issue_pg(j, page_load(j)); };


  float seen = -INFINITY;     // largest raw score of this lane in this pass
  float p[16];                // softmax weights of the tile being scored
  // weight i of scores x: exp2(x cs - m) (m: reference in log2 units)
  auto weight = [&](const f32x16_t& x, int i, float mr) {
    seen = fmaxf(seen, x[i]);
    p[i] = __builtin_amdgcn_exp2f(fmaf(x[i], cs, -mr));
  };
  // O += P . C over the tile in slot T (pp0/pp1: packed weights of that tile);
  // with `next`, the weights of the following tile (scores x) are computed
  // between the products
  auto pv_product = [&](uint32_t T, const bf16x8_t& pp0, const bf16x8_t& pp1, bool next,
                        const f32x16_t& x, float mr) {
    const uint32_t b0 = T + toff[0], b1 = T + toff[1];
    // product m: column block m >> 1, token half m & 1
    auto ldb = [&](int m, s16x4_t (&dst)[2]) {
      const int off = 64 * (m >> 1) + 16 * kPitch * (m & 1);
      dst[0] = lds_tr16(b0 + off);
      dst[1] = lds_tr16(b1 + off);
    };
    // operands of products m, m+1 are awaited together; kBRing - 2 products read ahead
    s16x4_t br[kBRing][2];
#pragma unroll
    for (int d = 0; d < kBRing - 2; ++d) ldb(d, br[d]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < 2 * kColBlocks; m += 2) {
#pragma unroll
      for (int e = 0; e < 2; ++e)
        if (m + kBRing - 2 + e < 2 * kColBlocks) ldb(m + kBRing - 2 + e, br[(m + kBRing - 2 + e) % kBRing]);
      wait_lgkm(2 * min(kBRing - 2, 2 * kColBlocks - m - 2));
#pragma unroll
      for (int e = 0; e < 2; ++e)
        o[(m + e) >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            e ? pp1 : pp0, __builtin_bit_cast(bf16x8_t, br[(m + e) % kBRing]), o[(m + e) >> 1], 0, 0, 0);
      if (next) weight(x, m >> 1, mr);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // the normaliser sums the weights as rounded to bf16 for the P.C product, so the
  // split's output is an exact convex combination of its rows (a dominant weight
  // carries no rounding bias into the output)
  auto weight_sum = [&](const bf16x8_t& a, const bf16x8_t& b) {
    const u32x4_t ua = __builtin_bit_cast(u32x4_t, a), ub = __builtin_bit_cast(u32x4_t, b);
    float v[16];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(ua[k] << 16);
      v[2 * k + 1] = __uint_as_float(ua[k] & 0xFFFF0000u);
      v[8 + 2 * k] = __uint_as_float(ub[k] << 16);
      v[9 + 2 * k] = __uint_as_float(ub[k] & 0xFFFF0000u);
    }
    l_part += ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7])) +
              (((v[8] + v[9]) + (v[10] + v[11])) + ((v[12] + v[13]) + (v[14] + v[15])));
  };

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int nb = 0; nb < kColBlocks; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[nb][i] = 0.f;
    l_part = 0.f;
    seen = -INFINITY;

    if (wbase != p_first) load_window(p_first);
    bf16x8_t pp0, pp1;        // packed weights of the previous tile
    f32x16_t sc;
    float mr;
    int nv0 = issue(0), nv1 = 0, nv2 = 0;   // valid rows of tiles t, t+1, t+2
    if (ntiles > 1) nv1 = issue(1);
    // ---- tile 0: scores and weights (tile 2's copy starts among the products)
    const int pgv2 = ntiles > 2 ? page_load(2) : 0;
    wait_tile(ntiles > 1 ? 1 : 0);
    lds_barrier();
    sc = scores(ring0, [&] { if (ntiles > 2) nv2 = issue_pg(2, pgv2); });
    mask(sc, nv0);
    if (pass == 0) {            // the first tile fixes the reference
      float tm = sc[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) tm = fmaxf(tm, sc[i]);
      m_ref = fmaxf(tm, __shfl_xor(tm, 32, 64)) * cs;
    }
    mr = fmaxf(m_ref, -1e30f);
#pragma unroll
    for (int i = 0; i < 16; ++i) weight(sc, i, mr);
    pp0 = pack8(p);   // k = 16kk + 8(j >> 2) + 4g2 + (j & 3)
    pp1 = pack8(p + 8);
    weight_sum(pp0, pp1);
    nv0 = nv1; nv1 = nv2;
    // ---- tile t: scores, then the products of tile t-1 with the weights of tile t between them
    for (int t = 1; t < ntiles; ++t) {
      const bool more = t + 2 < ntiles;
      const int pgv = more ? page_load(t + 2) : 0;
      wait_tile(t + 1 < ntiles ? 1 : 0);
      lds_barrier();   // tile t is in LDS for every wave; the slot of tile t-2 is free
      sc = scores(ring0 + (t & 3) * kTileBytes, [&] { if (more) nv2 = issue_pg(t + 2, pgv); });
      mask(sc, nv0);
      pv_product(ring0 + ((t - 1) & 3) * kTileBytes, pp0, pp1, true, sc, mr);
      pp0 = pack8(p);
      pp1 = pack8(p + 8);
      weight_sum(pp0, pp1);
      nv0 = nv1; nv1 = nv2;
    }
    pv_product(ring0 + ((ntiles - 1) & 3) * kTileBytes, pp0, pp1, false, sc, mr);
    // every copy has landed (the last tile was waited for with vmcnt 0)
    seen = fmaxf(seen, __shfl_xor(seen, 32, 64)) * cs;
    if (!__syncthreads_or(seen > m_ref + kHeadroom)) break;
    m_ref = seen;              // run the unit again with the largest score as reference
  }
  if (bad_page && tid == 0) set_err(a.err, ERR_PAGE);

  // ---- epilogue: o_part = O / l, lse = (m + log2 l) ln 2; lane holds heads 8(i>>2) + 4g2 + (i&3)
  const float l_sum = l_part + __shfl_xor(l_part, 32, 64);
  const float inv = l_sum > 0.f ? 1.f / l_sum : 0.f;
  if (g2 == 0) {
    xch[wv][r32] = inv;
    lse_out[r32] = l_sum > 0.f ? (m_ref + __log2f(l_sum)) * 0.6931471805599453f : -INFINITY;
  }
  __builtin_amdgcn_wave_barrier();
  float ilv[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 il = *reinterpret_cast<const float4*>(&xch[wv][8 * q + 4 * g2]);
    ilv[4 * q] = il.x; ilv[4 * q + 1] = il.y; ilv[4 * q + 2] = il.z; ilv[4 * q + 3] = il.w;
  }
#pragma unroll
  for (int nb = 0; nb < kColBlocks; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      o_out[(8 * (i >> 2) + 4 * g2 + (i & 3)) * kDc + 32 * nb + r32] = o[nb][i] * ilv[i];
}


// ---- FP8 pool on the FP8 matrix cores ---------------------------------------
// The staged codes feed v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e4m3, K = 64)
// as stored, with no conversion per element.  A lane of that product holds row
// (A) or column (B) lane & 31 and 32 bytes; byte j of A lane (r, g) meets byte j
// of B lane (n, g), and each operand row / column carries a power-of-two scale.
//   scores  S^T[t, h] = sum_k code[t, k] 2^e_t q[h, k] + k^R[t] . q_pe[h]: the
//           row scale 2^e_t is the hardware scale of A row t (E8M0 = the
//           exponent field of the staged fp32 scale).  q is carried as two e4m3
//           terms, q = 2^s_h (hi + lo), hi = RNE(q 2^-s_h), lo = RNE(q 2^-s_h - hi)
//           (relative error <= 2^-8, as for bf16), s_h putting the head's
//           largest |q| in [128, 256).  Step st (64 latent columns): lane (r, g)
//           holds columns 64st + 32g .. +31 of row r (two 16-byte chunks of the
//           staged row), the queries laid out to match; one product with hi,
//           one with lo.  Then the k^R part as four bf16 products.
//   P.C     O[h, d] += sum_t P'[h, t] code[t, d], P' = p 2^e_t split the same
//           way with a scale per head and tile.  The two terms share one
//           product: K = 64 holds the tile's 32 tokens twice, A lane (h, g) =
//           [hi | lo] of its 16 weights (tokens in the order of the score
//           accumulator, so the weights never move across lanes) and B lane
//           (n, g) = the same 16 codes of column n twice (two transposed 8-byte
//           reads, duplicated in registers).
// Per tile and wave that is 16 + 4 products for the scores and 16 for P.C, as
// many matrix cycles as the bf16 pool, with 644 instead of 1152 bytes per token
// and no conversion of the codes.
typedef int i32x8_t __attribute__((ext_vector_type(8)));

// scaled e4m3 product with the accumulator in VGPRs (asm for the same reason as
// mfma_v); the first of a chain gets 5 wait states after VALU writes of its
// operands, chains on one accumulator need none
__device__ __forceinline__ f32x16_t mfma8_first(const i32x8_t& a, const i32x8_t& b, uint32_t sa,
                                                uint32_t sb) {
  f32x16_t d;
  asm("s_nop 4\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel_hi:[0,0,0]"
      : "=&v"(d)
      : "v"(a), "v"(b), "v"(sa), "v"(sb));
  return d;
}
__device__ __forceinline__ void mfma8(f32x16_t& d, const i32x8_t& a, const i32x8_t& b, uint32_t sa,
                                      uint32_t sb) {
  asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
      : "+v"(d)
      : "v"(a), "v"(b), "v"(sa), "v"(sb));
}

// Two-term e4m3 split of 4 values already scaled into (-256, 256): hi = RNE(x),
// lo = RNE(x - hi), each packed as 4 bytes (value 0 in byte 0).
__device__ __forceinline__ void split4(float x0, float x1, float x2, float x3, uint32_t& hi,
                                       uint32_t& lo) {
  int h = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  h = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, h, true);
  const f32x2_t b0 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
  const f32x2_t b1 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
  int l = __builtin_amdgcn_cvt_pk_fp8_f32(x0 - b0[0], x1 - b0[1], 0, false);
  l = __builtin_amdgcn_cvt_pk_fp8_f32(x2 - b1[0], x3 - b1[1], l, true);
  hi = static_cast<uint32_t>(h);
  lo = static_cast<uint32_t>(l);
}

// E8M0 scale k + 127 and multiplier 2^-k that put a largest magnitude m >= 0 in
// [128, 256) (k clamped to [-126, 126]; m = 0 gives the smallest scale)
__device__ __forceinline__ void e4m3_scale(float m, uint32_t& e8, float& mul) {
  const int ex = static_cast<int>((__float_as_uint(m) >> 23) & 255u);   // m in [2^(ex-127), 2^(ex-126))
  const int k = min(max(ex - 134, -126), 126);
  e8 = static_cast<uint32_t>(k + 127);
  mul = __uint_as_float(static_cast<uint32_t>(127 - k) << 23);
}

constexpr int kF8mSlots = 6, kF8mAhead = 4;   // staging slots; tiles copied ahead

__global__ __launch_bounds__(kThreads, 1) void k_attn_f8mma_h128(
    AttnArgs a, const int32_t* __restrict__ block_table, const char* __restrict__ pool) {
  __shared__ __attribute__((aligned(1024))) char ring[kF8mSlots * kF8Stage];
  __shared__ __attribute__((aligned(16))) float xch[kWaves][kHeads];
  __shared__ int pwin[kPageWin];
  // the k^R part of the queries as bf16 B fragments, wave w fragment q of lane l
  // at 16 (64 (4w + q) + l) (registers are short: the latent part stays in VGPRs)
  __shared__ __attribute__((aligned(16))) char qrope[kWaves * 4 * 64 * 16];
  // the two e4m3 terms of the last latent step (st = 7) of the queries, wave w
  // lane l: hi at 64 (64 w + l), lo 32 bytes after it
  __shared__ __attribute__((aligned(16))) char qlast[kWaves * 64 * 64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g2 = lane >> 5;
  const int r32 = lane & 31;
  const int unit = unit_of(blockIdx.x, a.units);
  const int nh = 128;

  int b, sq, t0, t1;
  attn_unit(a, unit, tid == 0, &b, &sq, &t0, &t1);
  b = __builtin_amdgcn_readfirstlane(b);     // uniform by construction; say so for the
  sq = __builtin_amdgcn_readfirstlane(sq);   // scalar operands of the copies
  t0 = __builtin_amdgcn_readfirstlane(t0);
  t1 = __builtin_amdgcn_readfirstlane(t1);

  const int64_t ob = static_cast<int64_t>(unit) * nh + kHeads * wv;
  float* o_out = a.o_part + ob * kDc;
  float* lse_out = a.lse_part + ob;

  if (t0 >= t1) {  // empty split (uniform across the workgroup)
    for (int e = lane; e < kHeads * kDc; e += 64) o_out[e] = 0.f;
    if (lane < kHeads) lse_out[lane] = -INFINITY;
    return;
  }
  const int32_t* bt = block_table + static_cast<int64_t>(sq) * a.max_pages;
  const int p_first = t0 / kPage, p_end = (t1 - 1) / kPage + 1;
  int wbase = -1;
  auto load_window = [&](int base) {
    wait_vmcnt<0>();
    lds_barrier();
    for (int i = tid; i < kPageWin; i += kThreads) {
      const int pg = base + i;
      pwin[i] = pg < p_end ? bt[pg] : 0;
    }
    __syncthreads();
    wbase = base;
  };

  // ---- queries of head h = 32wv + r32: two e4m3 terms of the latent part
  // (lane (r32, g2), step st: columns 64st + 32g2 + j) with the head's scale,
  // and the k^R part as bf16 fragments (k = 16q + 8g2 + j)
  i32x8_t qh[7], ql[7];
  uint32_t q_e8;
  const uint32_t ql_lds = lds_addr(qlast) + 64 * (64 * wv + lane);
  const uint32_t qr_lds = lds_addr(qrope) + 16 * (256 * wv + lane);
  {
    // The wave's 32 query rows are read as whole cache lines (two 512-byte row
    // pieces per load) into a staging area in the still unused tile ring (wave w
    // at 32 kQS w, row r at kQS r: 128 fp32 columns + 16 bytes of pad, so the
    // fragment reads below are conflict-free), a quarter of the columns at a
    // time, twice: once for the head's largest |q|, once for the two-term split.
    constexpr int kQS = 128 * 4 + 16;
    const uint32_t qst = lds_addr(ring) + static_cast<uint32_t>(kHeads * kQS) * wv;
    const float* qlb = a.q_lat + (static_cast<int64_t>(b) * nh + kHeads * wv) * kDc;
    const int sr = lane >> 5, sc4 = 4 * (lane & 31);
    auto stage = [&](int qq) {   // columns 128qq.. of the 32 rows: row 2i + sr, columns sc4..+3
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float4 v = *reinterpret_cast<const float4*>(qlb + (2 * i + sr) * kDc + 128 * qq + sc4);
        lds_st128(qst + kQS * (2 * i + sr) + 4 * sc4, __builtin_bit_cast(u32x4_t, v));
        if ((i & 7) == 7) __builtin_amdgcn_sched_barrier(0);   // bounded loads in flight
      }
      wait_lgkm(0);
    };
    // columns 64 sp + 32 g2 + 4c .. +3 of row r32 within the staged quarter
    auto frag = [&](int sp, int c) {
      return __builtin_bit_cast(float4, lds_ld128(qst + kQS * r32 + 4 * (64 * sp + 32 * g2 + 4 * c)));
    };
    float mx = 0.f;
    for (int qq = 0; qq < 4; ++qq) {
      stage(qq);
#pragma unroll
      for (int sp = 0; sp < 2; ++sp)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float4 v = frag(sp, c);
          mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    float mul;
    e4m3_scale(mx, q_e8, mul);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      stage(qq);
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        const int st = 2 * qq + sp;
        i32x8_t th, tl;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float4 v = frag(sp, c);
          uint32_t hi, lo;
          split4(v.x * mul, v.y * mul, v.z * mul, v.w * mul, hi, lo);
          th[c] = static_cast<int>(hi);
          tl[c] = static_cast<int>(lo);
        }
        if (st < 7) {
          qh[st] = th;
          ql[st] = tl;
        } else {
          const u32x4_t* hv = reinterpret_cast<const u32x4_t*>(&th);
          const u32x4_t* lv = reinterpret_cast<const u32x4_t*>(&tl);
          lds_st128(ql_lds, hv[0]);
          lds_st128(ql_lds + 16, hv[1]);
          lds_st128(ql_lds + 32, lv[0]);
          lds_st128(ql_lds + 48, lv[1]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // k^R part: the 32 rows of 64 fp32 (8 KB, contiguous) staged the same way
    // (row 4i + (lane >> 4), columns 4 (lane & 15)..+3), then packed as bf16 fragments
    const float* qpb = a.q_pe + (static_cast<int64_t>(b) * nh + kHeads * wv) * kDr;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + (lane >> 4), c = 4 * (lane & 15);
      const float4 v = *reinterpret_cast<const float4*>(qpb + r * kDr + c);
      lds_st128(qst + kQS * r + 4 * c, __builtin_bit_cast(u32x4_t, v));
    }
    wait_lgkm(0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[8];
      const float4 lo = __builtin_bit_cast(float4, lds_ld128(qst + kQS * r32 + 4 * (16 * q + 8 * g2)));
      const float4 hi = __builtin_bit_cast(float4, lds_ld128(qst + kQS * r32 + 4 * (16 * q + 8 * g2 + 4)));
      v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
      v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
      lds_st128(qr_lds + 1024 * q, __builtin_bit_cast(u32x4_t, pack8(v)));
    }
    wait_lgkm(0);
    lds_barrier();   // every wave is done with the staging area before tiles are copied
  }

  // ---- per-lane constant offsets inside a staged tile
  // score A operand, step st, half hh: chunk 4st + 2g2 + hh of row r32, stored at
  // chunk (4st + 2g2 + hh) ^ f8key(r32)
  const int fk = f8key(r32);
  const uint32_t a_row = kDc * r32;
  const int a_kh = fk >> 2, a_kl = fk & 3;
  // k^R fragment q of row r32: chunk 2q + g2 of its 128 bytes
  const int vy = rkey(r32);
  uint32_t roff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) roff[q] = kF8RopeOff + 128 * r32 + 16 * ((2 * q + g2) ^ vy);
  // P.C B operand, column block nb, token half kk of a tile: one transposed read
  // (ds_read_b64_tr_b8) at f8_toff[kk] + 32 ((nb & 8) | ((nb & 7) ^ f8_m)).  Lane
  // s16 of 16-lane group (ch, g2) addresses token row 16kk + 8(m >> 2) + 4g2 + (m & 3),
  // m = s16 >> 1, columns 32nb + 16ch + 8(s16 & 1)..+7, and receives column
  // 32nb + 16ch + s16 of tokens 16kk + 8(j >> 2) + 4g2 + (j & 3), j = 0..7 (f8key of
  // that row is 2m + g2, so the 8 rows of a read fall on distinct banks)
  const int s16 = lane & 15, ch = (lane >> 4) & 1;
  const int f8_m = s16 >> 1;
  uint32_t f8_toff[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
    f8_toff[kk] = kDc * (16 * kk + 8 * (f8_m >> 2) + 4 * g2 + (f8_m & 3)) + 16 * (ch ^ g2) +
                  8 * (s16 & 1);
  const uint32_t ring0 = lds_addr(ring);

  // scores S^T[t, h] of the staged tile at T (lane: head r32, tokens
  // 8(i >> 2) + 4g2 + (i & 3)); `hook` runs after the first products
  auto scores = [&](uint32_t T, auto&& hook) {
    // per-lane offsets are recomputed per call (opaque): hoisted out of the tile
    // loop they would hold registers for the whole unit
    const uint32_t arow = opaque(T + a_row), akh = opaque(a_kh);
    const uint32_t c0 = 16 * ((2 * g2) ^ a_kl), c1 = c0 ^ 16;
    const uint32_t sa = (__float_as_uint(lds_f32(T + kF8ScaleLds + 4 * r32)) >> 23) & 255u;
    auto lda = [&](int st) {
      const uint32_t base = arow + 64 * ((st & 4) | ((st & 3) ^ akh));
      const u32x4_t x0 = lds_ld128(base + c0);
      const u32x4_t x1 = lds_ld128(base + c1);
      return (i32x8_t){static_cast<int>(x0[0]), static_cast<int>(x0[1]), static_cast<int>(x0[2]),
                       static_cast<int>(x0[3]), static_cast<int>(x1[0]), static_cast<int>(x1[1]),
                       static_cast<int>(x1[2]), static_cast<int>(x1[3])};
    };
    // queries of step 7 come from LDS, read along with the A operand of step 7
    auto ldq = [&](uint32_t off) {
      const u32x4_t x0 = lds_ld128(opaque(ql_lds) + off), x1 = lds_ld128(opaque(ql_lds) + off + 16);
      return (i32x8_t){static_cast<int>(x0[0]), static_cast<int>(x0[1]), static_cast<int>(x0[2]),
                       static_cast<int>(x0[3]), static_cast<int>(x1[0]), static_cast<int>(x1[1]),
                       static_cast<int>(x1[2]), static_cast<int>(x1[3])};
    };
    i32x8_t q7h, q7l;
    constexpr int kAh = 2;   // steps read ahead
    i32x8_t ar[kAh + 1];
#pragma unroll
    for (int d = 0; d < kAh; ++d) ar[d] = lda(d);
    f32x16_t acc;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (st + kAh < 8) ar[(st + kAh) % (kAh + 1)] = lda(st + kAh);
      if (st + kAh == 7) {   // with the last A operand: the step-7 queries (4 more reads)
        q7h = ldq(0);
        q7l = ldq(32);
      }
      wait_lgkm(st + kAh >= 7 ? 2 * (7 - st) + (st < 7 ? 4 : 0) : 2 * kAh);
      const i32x8_t& av = ar[st % (kAh + 1)];
      if (st < 7) {
        if (st == 0) acc = mfma8_first(av, qh[0], sa, q_e8);
        else mfma8(acc, av, qh[st], sa, q_e8);
        mfma8(acc, av, ql[st], sa, q_e8);
      } else {
        mfma8(acc, av, q7h, sa, q_e8);
        mfma8(acc, av, q7l, sa, q_e8);
      }
      if (st == 0) hook();
      __builtin_amdgcn_sched_barrier(0);
    }
    // k^R part: tile fragment and query fragment of step q, one step read ahead
    bf16x8_t rr[2], rq[2];
    const uint32_t qrb = opaque(qr_lds);
    rr[0] = lds_b128(opaque(T + roff[0]));
    rq[0] = lds_b128(qrb);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q < 3) {
        rr[(q + 1) & 1] = lds_b128(opaque(T + roff[q + 1]));
        rq[(q + 1) & 1] = lds_b128(qrb + 1024 * (q + 1));
      }
      wait_lgkm(q < 3 ? 2 : 0);
      if (q < 3) mfma_v(acc, rr[q & 1], rq[q & 1]);
      else mfma_v_last(acc, rr[q & 1], rq[q & 1]);
    }
    __builtin_amdgcn_sched_barrier(0);
    return acc;
  };
  // scores of rows nvalid.. of a partial tile to -inf (one compare against an
  // immediate per element)
  auto mask = [&](f32x16_t& x, int nvalid) {
    if (nvalid < kTileTok) {
      asm volatile("");
      const int lim = nvalid - 4 * g2;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + (i & 3) >= lim) x[i] = -INFINITY;
    }
  };
  // rows nvalid..31 of a partial staged tile (copied by this wave) get zero codes
  // and a zero scale, so that they add nothing to the products
  auto zero_tail = [&](uint32_t T, int nvalid) {
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    // row 8wv + 2i + (lane >> 5), chunk lane & 31: zb + 1024 i
    const int lim = nvalid - 8 * wv - (lane >> 5);
    const uint32_t zb = opaque(T + kDc * (8 * wv + (lane >> 5)) + 16 * (lane & 31));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (2 * i >= lim) lds_st128(zb + 1024 * i, zero);
    if (lane < 8 && 8 * wv + lane >= nvalid) lds_st32(T + kF8ScaleLds + 4 * (8 * wv + lane), 0u);
    wait_lgkm(0);
  };
  float m_ref = -INFINITY;
  float l_part = 0.f;
  f32x16_t o[kColBlocks];
  float seen = -INFINITY;     // largest raw score of this lane in this pass
  float p[16];                // softmax weights of the tile being scored
  const float cs = a.scale * kLog2e;
  auto weight = [&](const f32x16_t& x, int i, float mr) {
    seen = fmaxf(seen, x[i]);
    p[i] = __builtin_amdgcn_exp2f(fmaf(x[i], cs, -mr));
  };
  // O += P'.codes over the staged tile at T (pa: [hi | lo] of the lane's P', e8
  // their scale); with `next`, the weights of the following tile (scores x) are
  // computed between the products
  auto pv_product = [&](uint32_t T, const i32x8_t& pa, uint32_t e8, bool next, const f32x16_t& x,
                        float mr, auto&& copy) {
    // token half 1 of a tile sits 16 rows (kDc 16 bytes) after token half 0; the
    // operand's upper 16 bytes are the same two reads again (no register copies)
    const uint32_t fm = opaque(f8_m), b0 = opaque(T + f8_toff[0]);
    auto ldb = [&](int nb) {
      const uint32_t c = b0 + 32 * ((nb & 8) | ((nb & 7) ^ fm));
      const u32x2_t x0 = lds_tr8(c), x1 = lds_tr8(c + kDc * 16);
      const uint32_t cc = opaque(c);   // a second load of the same bytes, not a copy
      const u32x2_t x2 = lds_tr8(cc), x3 = lds_tr8(cc + kDc * 16);
      return (i32x8_t){static_cast<int>(x0[0]), static_cast<int>(x0[1]), static_cast<int>(x1[0]),
                       static_cast<int>(x1[1]), static_cast<int>(x2[0]), static_cast<int>(x2[1]),
                       static_cast<int>(x3[0]), static_cast<int>(x3[1])};
    };
    constexpr int kBh = 2;   // column blocks read ahead
    i32x8_t br[kBh + 1];
#pragma unroll
    for (int d = 0; d < kBh; ++d) br[d] = ldb(d);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int nb = 0; nb < kColBlocks; ++nb) {
      if (nb + kBh < kColBlocks) br[(nb + kBh) % (kBh + 1)] = ldb(nb + kBh);
      wait_lgkm(4 * min(kBh, kColBlocks - 1 - nb));
      const i32x8_t& bv = br[nb % (kBh + 1)];
      o[nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pa, bv, o[nb], 0, 0, 0,
                                                              static_cast<int>(e8), 0, 127);
      if (next) weight(x, nb, mr);
      if ((nb & 1) && nb < 2 * (kF8Copies - 1)) copy(nb >> 1);   // copy k after product 2k + 1
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // P' = p times the row scale of each of the lane's 16 tokens of the staged tile
  // at T, as [hi | lo] e4m3 with a scale per head
  auto pack_p = [&](uint32_t T, i32x8_t& pa, uint32_t& e8) {
    float (&pw)[16] = p;   // scaled in place (the sum of the weights is taken first)
    float mx = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4_t sv = lds_ld128(T + kF8ScaleLds + 4 * (8 * q + 4 * g2));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pw[4 * q + e] = p[4 * q + e] * __uint_as_float(sv[e]);
        mx = fmaxf(mx, pw[4 * q + e]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    float mul;
    e4m3_scale(mx, e8, mul);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t hi, lo;
      split4(pw[4 * d] * mul, pw[4 * d + 1] * mul, pw[4 * d + 2] * mul, pw[4 * d + 3] * mul, hi, lo);
      pa[d] = static_cast<int>(hi);
      pa[d + 4] = static_cast<int>(lo);
    }
  };
  auto weight_sum = [&]() {
    l_part += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])) +
              (((p[8] + p[9]) + (p[10] + p[11])) + ((p[12] + p[13]) + (p[14] + p[15])));
  };

  bool bad_page = false;
  const int ntiles = (t1 - t0 + kTileTok - 1) / kTileTok;

  auto page_load = [&](int j) {
    const int tok = t0 + j * kTileTok;
    if (tok / kPage - wbase >= kPageWin) load_window(tok / kPage);
    return pwin[tok / kPage - wbase];
  };
  auto stage_of = [&](int j) { return ring0 + static_cast<uint32_t>(j % kF8mSlots) * kF8Stage; };
  auto issue_pg = [&](int j, int pgv) {
    const int tok = t0 + j * kTileTok;
    const int pg = __builtin_amdgcn_readfirstlane(pgv);
    const bool ok = pg >= 0 && pg < a.num_pages;
    bad_page |= !ok;
    tile_issue_f8(pool, pg, ok, tok, t1, stage_of(j), wv, lane);
    return ok ? min(kTileTok, t1 - tok) : 0;
  };
  auto issue = [&](int j) { return issue_pg(j, page_load(j)); };
  // the copies of one tile issued one at a time (spread over the products of a
  // tile rather than as one burst): cp_begin fixes the tile and issues its scale
  // copy, cp_part(k) issues code copy k (k < 4, rows 8wv + 2k, +1) or the k^R
  // copy (k = 4); kF8Copies in all, as tile_issue_f8
  uint64_t cp_rows = 0, cp_scales = 0;
  int cp_nvalid = 0;
  uint32_t cp_stage = 0;
  auto cp_begin = [&](int j, int pgv) {
    const int tok = t0 + j * kTileTok;
    const int pg = __builtin_amdgcn_readfirstlane(pgv);
    const bool ok = pg >= 0 && pg < a.num_pages;
    bad_page |= !ok;
    cp_nvalid = ok ? min(kTileTok, t1 - tok) : 0;
    const int64_t pbase = ok ? static_cast<int64_t>(pg) * kF8PageBytes : 0;
    cp_rows = reinterpret_cast<uint64_t>(pool + pbase + (tok & (kPage - 1)) * kF8Row);
    cp_scales = reinterpret_cast<uint64_t>(pool + pbase + kF8ScaleOff + 4 * (tok & (kPage - 1)));
    cp_stage = stage_of(j);
    // the scale copy (two lanes) goes out here, the others among the products
    if (lane < 2) dma_block(cp_scales, 32 * wv + 16 * lane, cp_stage + kF8ScaleLds + 32 * wv);
    return cp_nvalid;
  };
  auto cp_part = [&](int k) {
    const int ln = static_cast<int>(opaque(static_cast<uint32_t>(lane)));
    if (k < 4) {
      const int r = 8 * wv + 2 * k + (ln >> 5);
      dma_block(cp_rows, (r < cp_nvalid ? r : 0) * kF8Row + 16 * ((ln & 31) ^ f8key(r)),
                cp_stage + kDc * (8 * wv + 2 * k));
    } else {
      const int rr = 8 * wv + (ln >> 3);
      dma_block(cp_rows, (rr < cp_nvalid ? rr : 0) * kF8Row + kDc + 16 * ((ln & 7) ^ rkey(rr)),
                cp_stage + kF8RopeOff + 1024 * wv);
    }
  };

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int nb = 0; nb < kColBlocks; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[nb][i] = 0.f;
    l_part = 0.f;
    seen = -INFINITY;
    if (wbase != p_first) load_window(p_first);

    // valid rows of tiles t .. t + kF8mAhead (tiles are copied kF8mAhead ahead)
    int nv0 = issue(0), nv1 = 0, nv2 = 0, nv3 = 0, nv4 = 0;
    if (ntiles > 1) nv1 = issue(1);
    if (ntiles > 2) nv2 = issue(2);
    if (ntiles > 3) nv3 = issue(3);
    i32x8_t pa;        // [hi | lo] of the previous tile's P'
    uint32_t pe8;      // their scale
    f32x16_t sc;
    float mr;
    // ---- tile 0: scores and weights (tile kF8mAhead's copy starts among the products)
    {
      const int pgv = ntiles > kF8mAhead ? page_load(kF8mAhead) : 0;
      wait_tile_f8(min(kF8mAhead - 1, ntiles - 1));
      if (nv0 < kTileTok) zero_tail(stage_of(0), nv0);
      lds_barrier();
      sc = scores(stage_of(0), [&] { if (ntiles > kF8mAhead) nv4 = issue_pg(kF8mAhead, pgv); });
      mask(sc, nv0);
      if (pass == 0) {          // the first tile fixes the reference
        float tm = sc[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) tm = fmaxf(tm, sc[i]);
        m_ref = fmaxf(tm, __shfl_xor(tm, 32, 64)) * cs;
      }
      mr = fmaxf(m_ref, -1e30f);
#pragma unroll
      for (int i = 0; i < 16; ++i) weight(sc, i, mr);
      weight_sum();
      pack_p(stage_of(0), pa, pe8);
      nv0 = nv1; nv1 = nv2; nv2 = nv3; nv3 = nv4;
    }
    // ---- tile t: scores, then the products of tile t-1 with the weights of tile t
    // between them and the copies of tile t + kF8mAhead among those products.
    // Tiles with a copy to start and the last kF8mAhead tiles run separate
    // copies of the body, so that no branch splits the product sequence.
    auto body = [&](int t, auto more_c) {
      constexpr bool more = decltype(more_c)::value;
      const int pgv = more ? page_load(t + kF8mAhead) : 0;
      wait_tile_f8(more ? kF8mAhead - 1 : min(kF8mAhead - 1, ntiles - 1 - t));
      if (nv0 < kTileTok) zero_tail(stage_of(t), nv0);
      lds_barrier();   // tile t is staged for every wave; the slot of tile t-2 is free
      if (more) nv4 = cp_begin(t + kF8mAhead, pgv);
      sc = scores(stage_of(t), [&] {});
      mask(sc, nv0);
      pv_product(stage_of(t - 1), pa, pe8, true, sc, mr, [&](int k) { if (more) cp_part(k); });
      weight_sum();
      pack_p(stage_of(t), pa, pe8);
      nv0 = nv1; nv1 = nv2; nv2 = nv3; nv3 = nv4;
    };
    int t = 1;
    for (; t + kF8mAhead < ntiles; ++t) body(t, std::true_type{});
    for (; t < ntiles; ++t) body(t, std::false_type{});
    pv_product(stage_of(ntiles - 1), pa, pe8, false, sc, mr, [&](int) {});
    // every copy has landed (the last tile was waited for with vmcnt 0)
    seen = fmaxf(seen, __shfl_xor(seen, 32, 64)) * cs;
    if (!__syncthreads_or(seen > m_ref + kHeadroom)) break;
    m_ref = seen;              // run the unit again with the largest score as reference
  }
  if (bad_page && tid == 0) set_err(a.err, ERR_PAGE);

  // ---- epilogue: o_part = O / l, lse = (m + log2 l) ln 2
  const float l_sum = l_part + __shfl_xor(l_part, 32, 64);
  const float inv = l_sum > 0.f ? 1.f / l_sum : 0.f;
  if (g2 == 0) {
    xch[wv][r32] = inv;
    lse_out[r32] = l_sum > 0.f ? (m_ref + __log2f(l_sum)) * 0.6931471805599453f : -INFINITY;
  }
  __builtin_amdgcn_wave_barrier();
  float ilv[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 il = *reinterpret_cast<const float4*>(&xch[wv][8 * q + 4 * g2]);
    ilv[4 * q] = il.x; ilv[4 * q + 1] = il.y; ilv[4 * q + 2] = il.z; ilv[4 * q + 3] = il.w;
  }
#pragma unroll
  for (int nb = 0; nb < kColBlocks; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      o_out[(8 * (i >> 2) + 4 * g2 + (i & 3)) * kDc + 32 * nb + r32] = o[nb][i] * ilv[i];
}


// ---- 16 heads (the Lite shape) ---------------------------------------------
// With n_h = 16 the heads fill one 16-wide MFMA dimension and the work per
// cached token is an eighth of the 128-head kernel's, so the kernel is a pure
// cache stream.  Work unit = (sequence, split) as above; its 4 waves stream
// disjoint 16-token tiles (wave w takes tiles w, w+4, ...) through two LDS slots
// each and never wait for one another inside the loop: a wave's copies land in
// its own slots and it waits only on its own copy counter.  Per tile and wave:
//   scores  S^T[t, h] = sum_k C[t, k] Q[h, k]: 18 mfma_f32_16x16x32_bf16
//           (M = the tile's 16 tokens, N = the 16 heads, K = 576), A = tile
//           rows from LDS, B = the queries (all 18 k-steps in VGPRs).  MFMA row
//           t reads LDS row pi(t) (rows 4g..4g+3 of row group g taken from LDS
//           row group (0, 2, 1, 3)[g]), which keeps both LDS reads below free
//           of bank conflicts.
//   softmax per head in the exp2 domain with a per-wave reference fixed at the
//           wave's first tile (the single-reference scheme of the 128-head
//           kernel: a unit's wave re-runs its tiles when a later score exceeds
//           it by more than 2^64).
//   P.C     O[h, d] += sum_t P[h, t] C[t, d]: 32 mfma_f32_16x16x16bf16_1k
//           (M = heads, N = 16 columns, K = the 16 tokens).  A lane's score
//           accumulator holds head lane & 15 and MFMA rows 4g..4g+3
//           (g = lane >> 4), which is exactly the A operand; the B operand (4
//           tokens of one column) is one ds_read_b64_tr_b16.
// At the end the 4 waves' (reference, sum, O) are combined through LDS.
// LDS slot (19,456 B): latent row r at 1088 r, 16-byte chunk c at
// c ^ h16key(r); the 16 RoPE rows after them, row r at 128 r, chunk c' at
// c' ^ rkey(r).
constexpr int kH16Tok = 16;                                   // tokens per tile
constexpr int kH16Slot = kH16Tok * kPitch + kH16Tok * 2 * kDr;  // 19456
constexpr int kH16Copies = kH16Tok + 2;                       // per tile: rows, then 2 RoPE blocks
constexpr int kH16Steps = (kDc + kDr) / 32;                   // 18 score k-steps
constexpr int kH16Blocks = kDc / 16;                          // 32 output column blocks

__device__ __forceinline__ int h16key(int r) { return 2 * ((r >> 2) & 1) ^ 3 * ((r >> 3) & 1); }
__device__ __forceinline__ int h16row(int t) {   // LDS row of MFMA row t
  return (((t >> 2) & 1) << 3) | (((t >> 3) & 1) << 2) | (t & 3);
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---- pieces of the two 16-head kernels (bf16 and FP8 pools) ----------------

// queries of head h as B fragments: k = 32 ks + 8 g .. + 7, rounded to bf16
__device__ __forceinline__ void h16_queries(const AttnArgs& a, int b, int h, int g,
                                            bf16x8_t (&qf)[kH16Steps]) {
  constexpr int nh = 16;
  const float* ql = a.q_lat + (static_cast<int64_t>(b) * nh + h) * kDc;
  const float* qp = a.q_pe + (static_cast<int64_t>(b) * nh + h) * kDr;
#pragma unroll
  for (int ks = 0; ks < kH16Steps; ++ks) {
    const float* src = ks < kDc / 32 ? ql + 32 * ks + 8 * g : qp + 32 * (ks - kDc / 32) + 8 * g;
    const float4 v0 = *reinterpret_cast<const float4*>(src);
    const float4 v1 = *reinterpret_cast<const float4*>(src + 4);
    const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    qf[ks] = pack8(v);
  }
}

// per-lane operand offsets inside a slot.  Score A operand of MFMA row t = lane & 15
// (LDS row h16row(t)), latent chunk 4 ks + g: aoff + 16 ((4 ks + g) ^ akey); RoPE
// chunk 4 (ks - 16) + g: roff[ks - 16].  P.C B operand (transposed read) of row group
// g, lane s16 = lane & 15: LDS row h16row(4 g + (s16 >> 2)), bytes 8 (s16 & 3) of
// column block nb's 32 bytes: boff + 16 ((2 nb + bsub) ^ bkey)
struct H16Lane {
  uint32_t aoff, roff[2], boff;
  int akey, bkey, bsub;
};

__device__ __forceinline__ H16Lane h16_lane(int lane) {
  const int g = lane >> 4, s16 = lane & 15;
  H16Lane L;
  const int ar = h16row(lane & 15);
  L.aoff = kPitch * ar;
  L.akey = h16key(ar);
#pragma unroll
  for (int q = 0; q < 2; ++q)
    L.roff[q] = kH16Tok * kPitch + 128 * ar + 16 * ((4 * q + g) ^ rkey(ar));
  const int br = h16row(4 * g + (s16 >> 2));
  L.bkey = h16key(br);
  L.boff = kPitch * br + 8 * (s16 & 1);
  L.bsub = (s16 & 3) >> 1;
  return L;
}

// One staged tile in slot T (nv valid rows): scores of the 16 heads (lane: head
// lane & 15, MFMA rows 4g + i), weights against the reference (`fix_ref`: the
// wave's first tile sets it), O += P.C.  `seen` tracks the largest raw score.
__device__ __forceinline__ void h16_tile(uint32_t T, int nv, const bf16x8_t (&qf)[kH16Steps],
                                         const H16Lane& L, int g, float cs, bool fix_ref,
                                         f32x4_t (&o)[kH16Blocks], float& m_ref, float& l_part,
                                         float& seen) {
  constexpr int kAAhead = 4, kARing = 6;    // score operands read ahead
  constexpr int kBAhead = 6, kBRing = 8;    // P.C operands read ahead
  // scores: operands read kAAhead steps ahead, waited for one by one
  auto lda = [&](int ks) {
    return ks < kDc / 32 ? lds_b128(T + L.aoff + 16 * ((4 * ks + g) ^ L.akey))
                         : lds_b128(T + L.roff[ks - kDc / 32]);
  };
  bf16x8_t ar[kARing];
#pragma unroll
  for (int d = 0; d < kAAhead; ++d) ar[d] = lda(d);
  f32x4_t x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < kH16Steps; ++ks) {
    if (ks + kAAhead < kH16Steps) ar[(ks + kAAhead) % kARing] = lda(ks + kAAhead);
    wait_lgkm(min(kAAhead, kH16Steps - 1 - ks));
    x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar[ks % kARing], qf[ks], x, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  // the P.C operands of the first blocks are read while the weights are formed
  auto ldb = [&](int nb) { return lds_tr16(T + L.boff + 16 * ((2 * nb + L.bsub) ^ L.bkey)); };
  s16x4_t bb[kBRing];
#pragma unroll
  for (int d = 0; d < kBAhead; ++d) bb[d] = ldb(d);
  if (nv < kH16Tok) {   // rows past the split's end (or of an unusable page)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (h16row(4 * g + i) >= nv) x[i] = -INFINITY;
  }
  if (fix_ref) {   // the wave's first tile fixes its reference
    float tm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    tm = fmaxf(tm, __shfl_xor(tm, 16, 64));
    tm = fmaxf(tm, __shfl_xor(tm, 32, 64));
    m_ref = tm * cs;
  }
  const float mr = fmaxf(m_ref, -1e30f);
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    seen = fmaxf(seen, x[i]);
    p[i] = __builtin_amdgcn_exp2f(fmaf(x[i], cs, -mr));
  }
  // P as bf16 (the A operand as it stands); the sum takes the rounded values
  const unsigned w01 = cvt2(p[0], p[1]), w23 = cvt2(p[2], p[3]);
  l_part += (__uint_as_float(w01 << 16) + __uint_as_float(w01 & 0xFFFF0000u)) +
            (__uint_as_float(w23 << 16) + __uint_as_float(w23 & 0xFFFF0000u));
  const u32x2_t pw = {w01, w23};
  const s16x4_t pa = __builtin_bit_cast(s16x4_t, pw);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int nb = 0; nb < kH16Blocks; ++nb) {
    if (nb + kBAhead < kH16Blocks) bb[(nb + kBAhead) % kBRing] = ldb(nb + kBAhead);
    wait_lgkm(min(kBAhead, kH16Blocks - 1 - nb));
    o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, bb[nb % kBRing], o[nb], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Combine the 4 waves: common reference M_h per head, each wave's share of O
// scaled by 2^(m_w - M_h), summed per column by the wave that owns the column
// block; the normaliser and the lse are formed once per head.  The ring is free
// once every wave's copies have landed and been read (the first barrier).
__device__ __forceinline__ void h16_combine(char* ring, float (*wstate)[2][16],
                                            const f32x4_t (&o)[kH16Blocks], float l_part,
                                            float m_ref, int mine, int wv, int lane, float* o_out,
                                            float* lse_out) {
  constexpr int nh = 16;
  const int h = lane & 15, g = lane >> 4, s16 = lane & 15;
  float lsum = l_part + __shfl_xor(l_part, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  const float mw = mine > 0 ? m_ref : -INFINITY;
  __syncthreads();
  if (g == 0) {
    wstate[wv][0][h] = mw;
    wstate[wv][1][h] = mine > 0 ? lsum : 0.f;
  }
  __syncthreads();
  float mh = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) mh = fmaxf(mh, wstate[w][0][h]);
  const float f = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - mh);
  if (wv == 0 && g == 0) {   // head h: 1 / sum_w l_w 2^(m_w - M) and the lse
    float z = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float m = wstate[w][0][h];
      if (m != -INFINITY) z += wstate[w][1][h] * __builtin_amdgcn_exp2f(m - mh);
    }
    wstate[0][1][h] = z > 0.f ? 1.f / z : 0.f;   // read back below (after the barrier)
    lse_out[h] = z > 0.f ? (mh + __log2f(z)) * 0.6931471805599453f : -INFINITY;
  }
  // this wave's scaled O: head row hr at kRowW hr floats (padded: conflict-free writes)
  constexpr int kRowW = kDc + 4;
  float* stage = reinterpret_cast<float*>(ring) + wv * nh * kRowW;
  float fh[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) fh[i] = __shfl(f, 4 * g + i, 64);   // scale of head 4g + i
#pragma unroll
  for (int nb = 0; nb < kH16Blocks; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) stage[(4 * g + i) * kRowW + 16 * nb + s16] = o[nb][i] * fh[i];
  __syncthreads();
  // wave wv: columns 128 wv .. 128 wv + 127 of every head; step i covers head i / 2
  const float* st_all = reinterpret_cast<const float*>(ring);
#pragma unroll 4
  for (int i = 0; i < 2 * nh; ++i) {
    const int hr = i >> 1, c = 128 * wv + 64 * (i & 1) + lane;
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) acc += st_all[(w * nh + hr) * kRowW + c];
    o_out[hr * kDc + c] = acc * wstate[0][1][hr];
  }
}

// The unit's range and outputs (an empty split writes its empty result and says so).
struct H16Unit {
  int b, sq, t0, t1;
  float* o_out;
  float* lse_out;
};

__device__ __forceinline__ bool h16_unit(const AttnArgs& a, int tid, H16Unit& U) {
  constexpr int nh = 16;
  const int unit = unit_of(blockIdx.x, a.units);
  int b, sq, t0, t1;
  attn_unit(a, unit, tid == 0, &b, &sq, &t0, &t1);
  U.b = __builtin_amdgcn_readfirstlane(b);
  U.sq = __builtin_amdgcn_readfirstlane(sq);
  U.t0 = __builtin_amdgcn_readfirstlane(t0);
  U.t1 = __builtin_amdgcn_readfirstlane(t1);
  const int64_t ob = static_cast<int64_t>(unit) * nh;
  U.o_out = a.o_part + ob * kDc;
  U.lse_out = a.lse_part + ob;
  if (U.t0 >= U.t1) {   // empty split (uniform across the workgroup)
    for (int e = tid; e < nh * kDc; e += kThreads) U.o_out[e] = 0.f;
    if (tid < nh) U.lse_out[tid] = -INFINITY;
    return false;
  }
  return true;
}

__global__ __launch_bounds__(kThreads, 1) void k_attn_mfma_h16(
    AttnArgs a, const int32_t* __restrict__ block_table, const char* __restrict__ pool) {
  __shared__ __attribute__((aligned(1024))) char ring[kWaves * 2 * kH16Slot];   // 155,648 B
  __shared__ float wstate[kWaves][2][16];   // per wave: reference and sum of each head

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane & 15, g = lane >> 4;   // head (B/D column) and row group of this lane
  H16Unit U;
  if (!h16_unit(a, tid, U)) return;
  const bool stream = a.q_seq == nullptr;   // decode: rows read once (non-temporal copies)
  const int t0 = U.t0, t1 = U.t1;
  const int32_t* bt = block_table + static_cast<int64_t>(U.sq) * a.max_pages;
  const int ntiles = (t1 - t0 + kH16Tok - 1) / kH16Tok;
  const int mine = ntiles > wv ? (ntiles - wv + kWaves - 1) / kWaves : 0;   // this wave's tiles

  bf16x8_t qf[kH16Steps];
  h16_queries(a, U.b, h, g, qf);
  const uint32_t slot0 = lds_addr(ring) + static_cast<uint32_t>(2 * kH16Slot) * wv;
  const H16Lane L = h16_lane(lane);

  const float cs = a.scale * kLog2e;
  bool bad_page = false;

  // page ids: t0 is page-aligned and a page holds 4 tiles, so this wave's tile u
  // is the quarter wv of page t0/64 + u.  Lane i of `pwin` holds the id of page
  // t0/64 + wbase + i (a window of 64 pages, reloaded when a tile is past it)
  const int p0 = t0 / kPage, p_end = (t1 - 1) / kPage + 1;
  int pwin = 0, wbase = -kPage;
  auto page_of = [&](int u) {
    if (u - wbase >= 64) {        // uniform; drains this wave's copies in flight
      wbase = u;
      const int pg = p0 + wbase + lane;
      pwin = pg < p_end ? bt[pg] : 0;
      wait_vmcnt<0>();
    }
    return __builtin_amdgcn_readlane(pwin, u - wbase);
  };
  // tile u of this wave (tokens t0 + 16 (wv + 4u) ..) into slot u & 1
  auto issue = [&](int u) {
    const int tok = t0 + kH16Tok * (wv + kWaves * u);
    const int pg = page_of(u);
    const bool ok = pg >= 0 && pg < a.num_pages;
    bad_page |= !ok;
    const int nvalid = ok ? min(kH16Tok, t1 - tok) : 0;
    const uint64_t tile = reinterpret_cast<uint64_t>(
        ok ? pool + (static_cast<int64_t>(pg) * kPage + (tok & (kPage - 1))) * kRowBytes : pool);
    const uint32_t slot = slot0 + (u & 1) * kH16Slot;
    auto copies = [&](auto policy) {
      constexpr bool kS = decltype(policy)::value;
#pragma unroll
      for (int r = 0; r < kH16Tok; ++r) {
        const int rv = r < nvalid ? r : 0;
        dma_block<kS>(tile, kRowBytes * rv + 16 * (lane ^ h16key(r)), slot + kPitch * r);
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int rr = 8 * q + (lane >> 3);
        const int rv = rr < nvalid ? rr : 0;
        dma_block<kS>(tile, kRowBytes * rv + 2 * kDc + 16 * ((lane & 7) ^ rkey(rr)),
                      slot + kH16Tok * kPitch + 1024 * q);
      }
    };
    if (stream) copies(std::true_type{});
    else copies(std::false_type{});
    return nvalid;
  };

  // O starts at zero also for a wave without tiles (its share is scaled by 0 below)
  f32x4_t o[kH16Blocks];
#pragma unroll
  for (int nb = 0; nb < kH16Blocks; ++nb) o[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_part = 0.f;
  for (int pass = 0; pass < 2 && mine > 0; ++pass) {
    if (pass > 0) {
#pragma unroll
      for (int nb = 0; nb < kH16Blocks; ++nb) o[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    l_part = 0.f;
    float seen = -INFINITY;
    int nv0 = issue(0), nv1 = mine > 1 ? issue(1) : 0;
    for (int u = 0; u < mine; ++u) {
      if (u + 1 < mine) wait_vmcnt<kH16Copies>();
      else wait_vmcnt<0>();
      h16_tile(slot0 + (u & 1) * kH16Slot, nv0, qf, L, g, cs, pass == 0 && u == 0, o, m_ref,
               l_part, seen);
      // every read of this slot has returned (the last wait was lgkmcnt(0)): refill it
      nv0 = nv1;
      if (u + 2 < mine) nv1 = issue(u + 2);
    }
    // largest score of each head over this wave's tiles (log2 units)
    seen = fmaxf(seen, __shfl_xor(seen, 16, 64));
    seen = fmaxf(seen, __shfl_xor(seen, 32, 64));
    seen *= cs;
    // wave-uniform: the pass loop holds copies and matrix products, which must run
    // with every lane active
    if (__ballot(seen > m_ref + kHeadroom) == 0) break;
    m_ref = seen;                // this wave runs its tiles again with its heads' maxima
  }
  if (bad_page) set_err(a.err, ERR_PAGE);
  h16_combine(ring, wstate, o, l_part, m_ref, mine, wv, lane, U.o_out, U.lse_out);
}

// ---- FP8 pool, 16 heads --------------------------------------------------------
// The 16-head kernel above over the FP8 pool: each wave's tile copy is split in
// two.  The k^R part (bf16 in the page) is copied asynchronously into the slot as
// before; the latent codes and the row scales go to registers one tile ahead and
// are dequantized into the slot's bf16 latent rows when the tile's turn comes.
// e4m3 times a power-of-two scale is exact in bf16, so from there on the tile is
// the bf16 tile of the dequantized rows and the products, softmax and combine are
// the bf16 kernel's.  Rows past the split's end or of an unusable page are written
// as zeros (NaN codes of a foreign page never reach a product).
// Per tile and lane: 8 loads of 16 codes (rows 2i + (lane >> 5), codes
// 16 (lane & 31) ..) and 8 of the rows' scales, then the 2 k^R copies.
constexpr int kH16F8Copies = 8 + 8 + 2;

struct F8H16Regs {
  u32x4_t code[8];
  float scale[8];
};

__global__ __launch_bounds__(kThreads, 1) void k_attn_f8_h16(
    AttnArgs a, const int32_t* __restrict__ block_table, const char* __restrict__ pool) {
  __shared__ __attribute__((aligned(1024))) char ring[kWaves * 2 * kH16Slot];   // 155,648 B
  __shared__ float wstate[kWaves][2][16];   // per wave: reference and sum of each head

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane & 15, g = lane >> 4;
  H16Unit U;
  if (!h16_unit(a, tid, U)) return;
  const int t0 = U.t0, t1 = U.t1;
  const int32_t* bt = block_table + static_cast<int64_t>(U.sq) * a.max_pages;
  const int ntiles = (t1 - t0 + kH16Tok - 1) / kH16Tok;
  const int mine = ntiles > wv ? (ntiles - wv + kWaves - 1) / kWaves : 0;

  bf16x8_t qf[kH16Steps];
  h16_queries(a, U.b, h, g, qf);
  const uint32_t slot0 = lds_addr(ring) + static_cast<uint32_t>(2 * kH16Slot) * wv;
  const H16Lane L = h16_lane(lane);
  // dequantization: this lane's rows 2i + (lane >> 5) and code chunk lane & 31
  // (latent columns 16 (lane & 31) .. + 15, bf16 chunks 2 (lane & 31) and + 1)
  const int crow = lane >> 5, cchunk = lane & 31;

  const float cs = a.scale * kLog2e;
  bool bad_page = false;

  const int p0 = t0 / kPage, p_end = (t1 - 1) / kPage + 1;
  int pwin = 0, wbase = -kPage;
  auto page_of = [&](int u) {
    if (u - wbase >= 64) {        // uniform; drains this wave's copies in flight
      wbase = u;
      const int pg = p0 + wbase + lane;
      pwin = pg < p_end ? bt[pg] : 0;
      wait_vmcnt<0>();
    }
    return __builtin_amdgcn_readlane(pwin, u - wbase);
  };
  // tile u of this wave (tokens t0 + 16 (wv + 4u) ..): codes and scales into `rg`,
  // the k^R rows into slot u & 1; returns the valid rows
  auto issue = [&](int u, F8H16Regs& rg) {
    const int tok = t0 + kH16Tok * (wv + kWaves * u);
    const int pg = page_of(u);
    const bool ok = pg >= 0 && pg < a.num_pages;
    bad_page |= !ok;
    const int nvalid = ok ? min(kH16Tok, t1 - tok) : 0;
    const char* page = pool + (ok ? static_cast<int64_t>(pg) * kF8PageBytes : 0);
    const int r0 = tok & (kPage - 1);   // the tile's first row in its page
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 2 * i + crow, rv = r < nvalid ? r : 0;
      rg.code[i] = *reinterpret_cast<const u32x4_t*>(page + (r0 + rv) * kF8Row + 16 * cchunk);
      rg.scale[i] = *reinterpret_cast<const float*>(page + kF8ScaleOff + 4 * (r0 + rv));
    }
    const uint64_t rows = reinterpret_cast<uint64_t>(page + r0 * kF8Row);
    const uint32_t slot = slot0 + (u & 1) * kH16Slot;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int rr = 8 * q + (lane >> 3);
      const int rv = rr < nvalid ? rr : 0;
      dma_block(rows, kF8Row * rv + kDc + 16 * ((lane & 7) ^ rkey(rr)),
                slot + kH16Tok * kPitch + 1024 * q);
    }
    return nvalid;
  };
  // the codes of `rg` as bf16 latent rows of slot T (zeros for rows nvalid..)
  auto dequantize = [&](const F8H16Regs& rg, uint32_t T, int nvalid) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 2 * i + crow;
      const float sc = r < nvalid ? rg.scale[i] : 0.f;
      u32x4_t lo, hi;   // bf16 columns 16 cchunk + 0..7 and + 8..15
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int c = static_cast<int>(rg.code[i][w]);
        const f32x2_t f0 = __builtin_amdgcn_cvt_pk_f32_fp8(c, false);
        const f32x2_t f1 = __builtin_amdgcn_cvt_pk_f32_fp8(c, true);
        // a zero scale must give zeros even for NaN codes
        const unsigned p0 = r < nvalid ? cvt2(f0[0] * sc, f0[1] * sc) : 0u;
        const unsigned p1 = r < nvalid ? cvt2(f1[0] * sc, f1[1] * sc) : 0u;
        if (w < 2) { lo[2 * w] = p0; lo[2 * w + 1] = p1; }
        else { hi[2 * (w - 2)] = p0; hi[2 * (w - 2) + 1] = p1; }
      }
      const int key = h16key(r);
      lds_st128(T + kPitch * r + 16 * ((2 * cchunk) ^ key), lo);
      lds_st128(T + kPitch * r + 16 * ((2 * cchunk + 1) ^ key), hi);
    }
  };

  f32x4_t o[kH16Blocks];
#pragma unroll
  for (int nb = 0; nb < kH16Blocks; ++nb) o[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_part = 0.f;
  F8H16Regs rga, rgb;   // codes of tiles u (even u: rga) and u + 1
  for (int pass = 0; pass < 2 && mine > 0; ++pass) {
    if (pass > 0) {
#pragma unroll
      for (int nb = 0; nb < kH16Blocks; ++nb) o[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    l_part = 0.f;
    float seen = -INFINITY;
    int nv0 = issue(0, rga), nv1 = mine > 1 ? issue(1, rgb) : 0;
    // tile u, its codes in `cur` (refilled with tile u + 2 at the end)
    auto tile = [&](int u, F8H16Regs& cur) {
      if (u + 1 < mine) wait_vmcnt<kH16F8Copies>();
      else wait_vmcnt<0>();
      const uint32_t T = slot0 + (u & 1) * kH16Slot;
      dequantize(cur, T, nv0);
      wait_lgkm(0);   // the wave's own rows are in LDS before it reads them
      h16_tile(T, nv0, qf, L, g, cs, pass == 0 && u == 0, o, m_ref, l_part, seen);
      // every read of this slot has returned (the last wait was lgkmcnt(0)): refill it
      nv0 = nv1;
      if (u + 2 < mine) nv1 = issue(u + 2, cur);
    };
    for (int u = 0; u < mine; u += 2) {
      tile(u, rga);
      if (u + 1 < mine) tile(u + 1, rgb);
    }
    seen = fmaxf(seen, __shfl_xor(seen, 16, 64));
    seen = fmaxf(seen, __shfl_xor(seen, 32, 64));
    seen *= cs;
    if (__ballot(seen > m_ref + kHeadroom) == 0) break;
    m_ref = seen;
  }
  if (bad_page) set_err(a.err, ERR_PAGE);
  h16_combine(ring, wstate, o, l_part, m_ref, mine, wv, lane, U.o_out, U.lse_out);
}

}  // namespace

// the matrix-core kernels read the fp32 queries 16 bytes at a time
static bool queries_aligned(const AttnArgs& a) {
  return ((reinterpret_cast<uintptr_t>(a.q_lat) | reinterpret_cast<uintptr_t>(a.q_pe)) & 15) == 0;
}

bool fast_attention_ok(const AttnArgs& a) {
  return a.n_heads == 128 && a.d_latent == kDc && a.d_rope == kDr && a.page_size == kPage &&
         queries_aligned(a);
}

bool fast_attention_h16_ok(const AttnArgs& a) {
  return a.n_heads == 16 && a.d_latent == kDc && a.d_rope == kDr && a.page_size == kPage &&
         queries_aligned(a);
}

hipError_t launch_attention_fast(const AttnArgs& a, hipStream_t stream) {
  if (a.units == 0) return hipSuccess;
  const int units = a.units;
  if (fast_attention_h16_ok(a))
    hipLaunchKernelGGL(k_attn_mfma_h16, dim3(units), dim3(kThreads), 0, stream, a, a.block_table,
                       static_cast<const char*>(a.pool));
  else
    hipLaunchKernelGGL(k_attn_mfma_h128, dim3(units), dim3(kThreads), 0, stream, a,
                       a.block_table, static_cast<const char*>(a.pool));
  return hipGetLastError();
}

hipError_t launch_attention_fp8(const AttnArgs& a, hipStream_t stream) {
  if (a.units == 0) return hipSuccess;
  const int units = a.units;
  if (fast_attention_h16_ok(a))
    hipLaunchKernelGGL(k_attn_f8_h16, dim3(units), dim3(kThreads), 0, stream, a, a.block_table,
                       static_cast<const char*>(a.pool));
  else
    hipLaunchKernelGGL(k_attn_f8mma_h128, dim3(units), dim3(kThreads), 0, stream, a,
                       a.block_table, static_cast<const char*>(a.pool));
  return hipGetLastError();
}

// Log-sum-exp merge of split partials: one wave per (sequence, head) row, one
// float4 of the row per lane and split, so every byte of o_part is read once
// with 16-byte coalesced loads.  The split weights exp(lse_s - max) are
// wave-uniform and recomputed by every lane.
__global__ __launch_bounds__(256) void k_merge_rows(MergeArgs a, int rows) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int nh = a.n_heads, dq = a.d_latent / 4;
  const int b = row / nh, i = row - b * nh;
  int first, S;
  merge_units(a, b, lane == 0 && i == 0, &first, &S);
  const float* lse = a.lse_part + static_cast<int64_t>(first) * nh + i;
  float m = -INFINITY;
  for (int s = lane; s < S; s += 64) m = fmaxf(m, lse[static_cast<int64_t>(s) * nh]);
  m = wave_max(m);
  const float4* src =
      reinterpret_cast<const float4*>(a.o_part) + (static_cast<int64_t>(first) * nh + i) * dq;
  const int64_t split_stride = static_cast<int64_t>(nh) * dq;   // float4s between splits
  float4* dst = reinterpret_cast<float4*>(a.o_lat) + static_cast<int64_t>(row) * dq;
  float z = 0.f;
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  constexpr int kB = 8;   // splits per load batch (all in flight at once)
  for (int v = lane; v < dq; v += 64) {   // lane 0 always runs: dq >= 1
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float zz = 0.f;
    if (m != -INFINITY) {
      for (int s0 = 0; s0 < S; s0 += kB) {
        f32x4_t x[kB];
        float w[kB];
#pragma unroll
        for (int j = 0; j < kB; ++j) {
          const int sc = s0 + j < S ? s0 + j : s0;   // past S: split s0 again, weight 0
          x[j] = reinterpret_cast<const f32x4_t*>(src)[sc * split_stride + v];
          const float l = lse[static_cast<int64_t>(sc) * nh];
          w[j] = (s0 + j >= S || l == -INFINITY) ? 0.f : __expf(l - m);
        }
        // the batch is issued before its first use (the skip of a zero weight is a
        // select, which the compiler would otherwise turn into a branch around a load)
#pragma unroll
        for (int j = 0; j < kB; ++j) asm volatile("" : "+v"(x[j]));
#pragma unroll
        for (int j = 0; j < kB; ++j) {
          zz += w[j];   // (+0 past S: exact)
          float n0 = acc.x, n1 = acc.y, n2 = acc.z, n3 = acc.w;
          n0 += w[j] * x[j][0]; n1 += w[j] * x[j][1]; n2 += w[j] * x[j][2]; n3 += w[j] * x[j][3];
          const bool on = w[j] != 0.f;
          acc.x = on ? n0 : acc.x;
          acc.y = on ? n1 : acc.y;
          acc.z = on ? n2 : acc.z;
          acc.w = on ? n3 : acc.w;
        }
      }
    }
    z = zz;
    const float inv = zz > 0.f ? 1.f / zz : 0.f;
    const float4 r = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    if (a.o_lat_bf16)
      reinterpret_cast<uint2*>(a.o_lat_bf16)[static_cast<int64_t>(row) * dq + v] =
          make_uint2(cvt2(r.x, r.y), cvt2(r.z, r.w));
    else
      dst[v] = r;
  }
  if (a.lse && lane == 0) a.lse[row] = z > 0.f ? m + __logf(z) : -INFINITY;
}

// Rows of many uniform splits (64 per row at 128K context): one workgroup per
// (b, i) row, wave w weighing splits w, w + 4, ... in batches of kMergeWideB (every
// load of a batch in flight at once), the four partial sums added in a fixed order
// through LDS.  Same weights as k_merge_rows; the sums go in another (fixed) order.
// d_c = 512: a lane holds float4 columns lane and lane + 64.
constexpr int kMergeWideS = 16;   // uniform splits above this take the wide form
constexpr int kMergeWideB = 8;    // splits per load batch of a wave

__global__ __launch_bounds__(256) void k_merge_rows_wide(MergeArgs a) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  __shared__ f32x4_t part[4][128];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nh = a.n_heads, S = a.num_splits;
  const int b = row / nh, i = row - b * nh;
  const float* lse = a.lse_part + static_cast<int64_t>(b) * S * nh + i;
  float m = -INFINITY;
  for (int s = lane; s < S; s += 64) m = fmaxf(m, lse[static_cast<int64_t>(s) * nh]);
  m = wave_max(m);
  float z = 0.f;
  for (int s = lane; s < S; s += 64) {
    const float l = lse[static_cast<int64_t>(s) * nh];
    z += (m == -INFINITY || l == -INFINITY) ? 0.f : __expf(l - m);
  }
  z = wave_sum(z);
  const f32x4_t* src =
      reinterpret_cast<const f32x4_t*>(a.o_part) + (static_cast<int64_t>(b) * S * nh + i) * 128;
  const int64_t split_stride = static_cast<int64_t>(nh) * 128;   // float4s between splits
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  if (m != -INFINITY) {
    for (int s0 = wv; s0 < S; s0 += 4 * kMergeWideB) {
      f32x4_t x0[kMergeWideB], x1[kMergeWideB];
      float w[kMergeWideB];
#pragma unroll
      for (int j = 0; j < kMergeWideB; ++j) {
        const int s = s0 + 4 * j;
        const int sc = s < S ? s : s0;   // past S: reload split s0, weight 0
        x0[j] = src[sc * split_stride + lane];
        x1[j] = src[sc * split_stride + lane + 64];
        const float l = lse[static_cast<int64_t>(sc) * nh];
        w[j] = (s >= S || l == -INFINITY) ? 0.f : __expf(l - m);
      }
      // the whole batch is issued before its first use (the skip of a zero weight
      // below is a select, which the compiler would otherwise turn into a branch
      // around a load of its own)
#pragma unroll
      for (int j = 0; j < kMergeWideB; ++j) {
        asm volatile("" : "+v"(x0[j]));
        asm volatile("" : "+v"(x1[j]));
      }
#pragma unroll
      for (int j = 0; j < kMergeWideB; ++j) {
        const f32x4_t n0 = acc0 + w[j] * x0[j], n1 = acc1 + w[j] * x1[j];
        acc0 = w[j] != 0.f ? n0 : acc0;
        acc1 = w[j] != 0.f ? n1 : acc1;
      }
    }
  }
  part[wv][lane] = acc0;
  part[wv][lane + 64] = acc1;
  __syncthreads();
  const float inv = z > 0.f ? 1.f / z : 0.f;
  if (tid < 128) {
    const f32x4_t o = ((part[0][tid] + part[1][tid]) + (part[2][tid] + part[3][tid])) * inv;
    reinterpret_cast<f32x4_t*>(a.o_lat)[static_cast<int64_t>(row) * 128 + tid] = o;
  }
  if (a.lse && tid == 0) a.lse[row] = z > 0.f ? m + __logf(z) : -INFINITY;
}

// The bf16 output form (k_merge_rows only: a plan, or at most kMergeWideS
// uniform splits; 8-byte aligned rows).
bool merge_bf16_ok(const MergeArgs& a) {
  return (a.unit_start != nullptr || a.num_splits <= kMergeWideS) && a.d_latent % 4 == 0 &&
         (reinterpret_cast<uintptr_t>(a.o_lat_bf16) & 7) == 0;
}

bool fast_merge_ok(const MergeArgs& a) {
  return a.d_latent % 4 == 0 && (reinterpret_cast<uintptr_t>(a.o_part) & 15) == 0 &&
         (reinterpret_cast<uintptr_t>(a.o_lat) & 15) == 0 &&
         static_cast<int64_t>(a.batch) * a.n_heads < (int64_t{1} << 31) - 4;
}

hipError_t launch_merge_fast(const MergeArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  const int rows = a.batch * a.n_heads;
  if (a.o_lat_bf16 && !merge_bf16_ok(a)) return hipErrorInvalidValue;
  if (!a.unit_start && a.num_splits > kMergeWideS && a.d_latent == 512) {
    hipLaunchKernelGGL(k_merge_rows_wide, dim3(rows), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_merge_rows, dim3((rows + 3) / 4), dim3(256), 0, stream, a, rows);
  return hipGetLastError();
}

}  // namespace mla
