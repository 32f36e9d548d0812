// The sticky device error word written by kernels that meet out-of-range
// block-table entries, positions or sequence indexes.
#include <hip/hip_runtime.h>

#include "launch_fast.hpp"

static __device__ int g_mla_err_word;

namespace mla {

int* error_word_address() {
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_mla_err_word)) != hipSuccess) return nullptr;
  return static_cast<int*>(p);
}

}  // namespace mla
