// Mixed step kernels (the general path for mixed heads) for one qbits x rounding pair: the
// build compiles this unit once per pair, with QS_QB (8 or 4) and QS_RND (0
// nearest, 1 stochastic 16-bit, 2 stochastic 8-bit) defined, so the
// instantiations compile in parallel.
#include "qstate_mixed_kernel.hpp"

namespace qs {
template hipError_t launch_mixed<QS_QB, QS_RND>(int delta, const Args& a, hipStream_t s);
}  // namespace qs
