// gla_bwd_bf16.hip -- GLA backward chunk kernels for bfloat16 activations (every head-dim
// class and chunk size).  Kernel source: gla_bwd_kernel.h.
#include "gla_bwd_kernel.h"

namespace dig {
template hipError_t launch_gla_bwd_t<bf16, false>(const GlaShape&, GlaBwdParams, hipStream_t, int*,
                                           size_t*);
}  // namespace dig
