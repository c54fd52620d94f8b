// gla_bwd_bf16_lr.hip -- GLA backward chunk kernels for bfloat16 activations whose key gate is
// the rank-16 product formed inside the kernels (every head-dim class and chunk size).  Kernel
// source: gla_bwd_kernel.h.
#include "gla_bwd_kernel.h"

namespace dig {
template hipError_t launch_gla_bwd_t<bf16, true>(const GlaShape&, GlaBwdParams, hipStream_t, int*,
                                                 size_t*);
}  // namespace dig
