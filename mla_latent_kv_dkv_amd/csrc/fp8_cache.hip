// FP8 latent pool: quantization of cache rows into FP8 pages.
//
// [Report] §4.2 of "《DeepSeek-V2》深度解读报告": inference quantizes the
// (already 576-wide) latent cache to about 6 bits per element; the scheme is not
// given.  The format used here: a page holds page_size rows of
// [c^KV as e4m3 bytes (d_c) | k^R as bf16 (d_R)], then page_size fp32 row scales.
// A row's scale is the power of two 2^e with e the smallest integer such that
// max|c| / 2^e <= 448 (the largest e4m3 value); code = round-to-nearest-even of
// c / 2^e into e4m3 (the division is exact).  k^R stays bf16 (round to nearest
// even), RoPE'd at the row's position when the rows come from the projection.
#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// One wave per row (4 rows per 256-thread block).  The row's first 512 latent
// values and first 64 k^R pairs (all of them at d_c <= 512, d_R <= 128) are loaded,
// and their RoPE angles evaluated, before the slot lookup resolves: the three
// do not depend on one another, so their latencies overlap.
__global__ __launch_bounds__(256) void k_quantize_rows(QuantArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= a.n_rows) return;
  const float* src = a.rows + static_cast<int64_t>(row) * a.ld_rows;
  const int seq = a.row_seq[row], pos = a.row_pos[row];
  const int c0 = 8 * lane, p0 = lane;
  f32x4_t lo0 = (f32x4_t){0.f, 0.f, 0.f, 0.f}, hi0 = lo0;
  if (c0 < a.d_latent) {
    lo0 = *reinterpret_cast<const f32x4_t*>(src + c0);
    hi0 = *reinterpret_cast<const f32x4_t*>(src + c0 + 4);
  }
  float k0 = 0.f, k1 = 0.f, cs0 = 1.f, sn0 = 0.f;
  if (p0 < a.d_rope / 2) {
    k0 = src[a.d_latent + 2 * p0];
    k1 = src[a.d_latent + 2 * p0 + 1];
    if (a.rope) rope_cs(pos, p0, a.d_rope, a.rs, &cs0, &sn0);
  }
  if (seq < 0 || seq >= a.n_seqs) { if (lane == 0) set_err(a.err, ERR_SEQ); return; }
  if (pos < 0 || pos >= a.max_pages * a.page_size) { if (lane == 0) set_err(a.err, ERR_POS); return; }
  const int page = a.block_table[static_cast<int64_t>(seq) * a.max_pages + pos / a.page_size];
  if (page < 0 || page >= a.num_pages) { if (lane == 0) set_err(a.err, ERR_PAGE); return; }
  const int slot = pos % a.page_size;
  uint8_t* pg = a.pool + static_cast<int64_t>(page) * a.page_bytes;
  uint8_t* dst = pg + static_cast<int64_t>(slot) * a.row_bytes;

  // row scale exponent from the largest |c| (exact: frexp and the comparison)
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fmaxf(fabsf(lo0[j]), fabsf(hi0[j])));
  for (int c = c0 + 512; c < a.d_latent; c += 512) {
    const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(src + c);
    const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(src + c + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fmaxf(fabsf(lo[j]), fabsf(hi[j])));
  }
  amax = wave_max(amax);
  int e = 0;
  if (amax > 0.f) {
    int x;
    const float m = frexpf(amax, &x);
    e = x - 9 + (m > 0.875f ? 1 : 0);
    e = e < -126 ? -126 : (e > 127 ? 127 : e);
  }
  // codes: 8 latent values per lane and step, round to nearest even into e4m3
  // (rows are 4-byte aligned in the page: d_c % 8 == 0, d_R even)
  auto put_codes = [&](int c, const f32x4_t& lo, const f32x4_t& hi) {
    int q0 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(lo[0], -e), ldexpf(lo[1], -e), 0, false);
    q0 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(lo[2], -e), ldexpf(lo[3], -e), q0, true);
    int q1 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(hi[0], -e), ldexpf(hi[1], -e), 0, false);
    q1 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(hi[2], -e), ldexpf(hi[3], -e), q1, true);
    reinterpret_cast<uint32_t*>(dst + c)[0] = static_cast<uint32_t>(q0);
    reinterpret_cast<uint32_t*>(dst + c)[1] = static_cast<uint32_t>(q1);
  };
  if (c0 < a.d_latent) put_codes(c0, lo0, hi0);
  for (int c = c0 + 512; c < a.d_latent; c += 512)
    put_codes(c, *reinterpret_cast<const f32x4_t*>(src + c),
              *reinterpret_cast<const f32x4_t*>(src + c + 4));
  // k^R in bf16, rotated at the row's position when asked
  auto put_pair = [&](int p, float v0, float v1, float cs, float sn) {
    if (a.rope) {
      const float r0 = v0 * cs - v1 * sn, r1 = v0 * sn + v1 * cs;
      v0 = r0;
      v1 = r1;
    }
    const uint32_t w = static_cast<uint32_t>(f32_to_bf16(v0)) |
                       (static_cast<uint32_t>(f32_to_bf16(v1)) << 16);
    *reinterpret_cast<uint32_t*>(dst + a.d_latent + 4 * p) = w;
  };
  if (p0 < a.d_rope / 2) put_pair(p0, k0, k1, cs0, sn0);
  for (int p = p0 + 64; p < a.d_rope / 2; p += 64) {
    float cs = 1.f, sn = 0.f;
    if (a.rope) rope_cs(pos, p, a.d_rope, a.rs, &cs, &sn);
    put_pair(p, src[a.d_latent + 2 * p], src[a.d_latent + 2 * p + 1], cs, sn);
  }
  if (lane == 0)
    *reinterpret_cast<float*>(pg + static_cast<int64_t>(a.page_size) * a.row_bytes + 4 * slot) =
        ldexpf(1.f, e);
}

}  // namespace

hipError_t launch_quantize_rows(const QuantArgs& a, hipStream_t stream) {
  if (a.n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_quantize_rows, dim3((a.n_rows + 3) / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
