// gla_fwd_bf16_lr.hip -- GLA forward chunk kernels for bfloat16 activations whose key gate is
// the rank-16 product formed inside the kernels (every head-dim class and chunk size).  Kernel
// source: gla_fwd_kernel.h.
#include "gla_fwd_kernel.h"

namespace dig {
template hipError_t launch_gla_fwd_t<bf16, true>(const GlaShape&, GlaFwdParams, hipStream_t, int*);
}  // namespace dig
