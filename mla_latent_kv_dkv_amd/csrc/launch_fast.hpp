// Host-side launchers of the MFMA (gfx950 matrix core) kernels and the shape
// predicates that decide when they apply.  Shapes they do not cover go to the
// plain vector kernels in kernels_generic.hip.
#pragma once

#include "launch.hpp"

namespace mla {

// Address of the sticky device error word on the current device (nullptr on failure).
int* error_word_address();

bool fast_gemm_ok(const GemmArgs& a);
// the product runs on the tiled kernels (M >= 256 and enough output tiles)
bool gemm_tiled_ok(const GemmArgs& a);
// the query projection with the fused latent append (EPI_QPROJ_APPEND) on k_gemm_xs
bool fused_qa_ok(const GemmArgs& a);
// fp32 scratch the fast GEMM needs for its K-split partials (0 if none)
size_t gemm_partial_bytes(const GemmArgs& a);
hipError_t launch_gemm_fast(const GemmArgs& a, void* partial, size_t partial_bytes,
                            hipStream_t stream);

bool fast_attention_ok(const AttnArgs& a);      // n_h = 128 (bf16 and FP8 pools)
bool fast_attention_h16_ok(const AttnArgs& a);  // n_h = 16 (bf16 and FP8 pools)
hipError_t launch_attention_fast(const AttnArgs& a, hipStream_t stream);
// FP8 pool (pages of 64 rows [512 e4m3 | 64 bf16] + 64 fp32 scales); the shapes of
// fast_attention_ok or fast_attention_h16_ok
hipError_t launch_attention_fp8(const AttnArgs& a, hipStream_t stream);

bool fast_merge_ok(const MergeArgs& a);
bool merge_bf16_ok(const MergeArgs& a);
hipError_t launch_merge_fast(const MergeArgs& a, hipStream_t stream);
// the per-head W_UV product (`a`, as mla_absorb_out sets it up, x unused) with
// the split merge `m` folded into its operand loads (m.o_lat unused)
bool uv_merge_ok(const GemmArgs& a, const MergeArgs& m);
// the shapes where the fused form beats the merge and the product run apart
bool uv_merge_pays(const GemmArgs& a, const MergeArgs& m);
hipError_t launch_uv_merge(const GemmArgs& a, const MergeArgs& m, hipStream_t stream);

}  // namespace mla
