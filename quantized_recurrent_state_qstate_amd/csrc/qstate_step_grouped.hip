// Step kernels for key-axis and per-head scale groups for one qbits x
// rounding pair: the build compiles this unit once per pair, with QS_QB (8 or
// 4) and QS_RND (0 nearest, 1 stochastic 16-bit, 2 stochastic 8-bit) defined.
#include "qstate_grouped_kernel.hpp"

namespace qs {
template hipError_t launch_grouped<QS_QB, QS_RND>(int delta, const Args& a, hipStream_t s);
}  // namespace qs
