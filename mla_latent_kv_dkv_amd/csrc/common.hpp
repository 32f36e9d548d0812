// Device-side helpers shared by the MLA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef uint16_t bf16_t;

// Sticky device error bits (mirrors mla_device_error in include/mla.h).
enum : int { ERR_PAGE = 1, ERR_POS = 2, ERR_SEQ = 4 };

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

__device__ __forceinline__ float ld(const float* p) { return *p; }
__device__ __forceinline__ float ld(const bf16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ void st(float* p, float v) { *p = v; }
__device__ __forceinline__ void st(bf16_t* p, float v) { *p = f32_to_bf16(v); }

__device__ __forceinline__ void set_err(int* err, int bits) {
  if (err) atomicOr(err, bits);
}

// RoPE frequencies: theta_k = rope_base^(-2k/d_R); with yarn_scale > 1 they are
// stretched by YaRN ("YaRN: Efficient Context Window Extension of Large Language
// Models", Peng et al. 2023; the long-context extension of "《DeepSeek-V2》深度解读报告"
// §3.3): pair k turns r = orig_len theta_k / (2 pi) times over the original window,
// gamma = clamp((r - alpha) / (beta - alpha), 0, 1), theta'_k = theta_k ((1 - gamma) /
// yarn_scale + gamma).
struct RopeSpec {
  double log_base;     // ln(rope_base)
  double yarn_scale;   // <= 1: plain RoPE
  double orig_len, alpha, beta;
};

// cos/sin of pos * theta_k (as RopeSpec defines it), evaluated in fp64 and rounded to fp32.
__device__ __forceinline__ void rope_cs(int pos, int k, int d_rope, const RopeSpec& rs, float* c,
                                        float* s) {
  double theta = exp(-2.0 * static_cast<double>(k) / static_cast<double>(d_rope) * rs.log_base);
  if (rs.yarn_scale > 1.0) {
    const double r = rs.orig_len * theta / 6.283185307179586;
    const double g = fmin(fmax((r - rs.alpha) / (rs.beta - rs.alpha), 0.0), 1.0);
    theta *= (1.0 - g) / rs.yarn_scale + g;
  }
  double sd, cd;
  sincos(static_cast<double>(pos) * theta, &sd, &cd);
  *c = static_cast<float>(cd);
  *s = static_cast<float>(sd);
}

// Block-table row and attended length of attention unit b.  Decode (q_seq null):
// sequence b, length seq_lens[b].  Prefill: query token b at position q_pos[b] of
// sequence q_seq[b], length q_pos[b] + 1 (causal, the token itself included).  A
// value out of range flags the error word (when `flag`) and gives length 0.
__device__ __forceinline__ void unit_seq_len(const int32_t* seq_lens, const int32_t* q_seq,
                                             const int32_t* q_pos, int n_seqs, int max_len, int b,
                                             bool flag, int* err, int* seq, int* len) {
  int s = b, L;
  if (q_seq) {
    s = q_seq[b];
    const int p = q_pos[b];
    L = p + 1;
    if (s < 0 || s >= n_seqs) {
      if (flag) set_err(err, ERR_SEQ);
      s = 0;
      L = 0;
    } else if (p < 0 || p >= max_len) {
      if (flag) set_err(err, ERR_POS);
      L = 0;
    }
  } else {
    L = seq_lens[b];
    if (L < 0 || L > max_len) {
      if (flag) set_err(err, ERR_POS);
      L = 0;
    }
  }
  *seq = s;
  *len = L;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Split s of a length-L sequence under S splits: page-aligned equal chunks.
__device__ __forceinline__ void split_range(int L, int S, int s, int page, int* t0, int* t1) {
  const int per = (L + S - 1) / S;
  const int chunk = ((per + page - 1) / page) * page;
  const long a = static_cast<long>(s) * chunk;
  *t0 = static_cast<int>(a < L ? a : L);
  const long b = a + chunk;
  *t1 = static_cast<int>(b < L ? b : L);
}

}  // namespace mla
