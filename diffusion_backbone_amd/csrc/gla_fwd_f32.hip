// gla_fwd_f32.hip -- GLA forward chunk kernels for fp32 activations (every head-dim class and
// chunk size).  Kernel source: gla_fwd_kernel.h.
#include "gla_fwd_kernel.h"

namespace dig {
template hipError_t launch_gla_fwd_t<float, false>(const GlaShape&, GlaFwdParams, hipStream_t, int*);
}  // namespace dig
