// Low-rank-bypass step kernels for one qbits x rounding pair and one kind:
// the build compiles this unit once per combination, with QS_QB (8 or 4),
// QS_RND (0 nearest, 1 stochastic 16-bit, 2 stochastic 8-bit) and QS_DELTA
// (0 additive, 1 delta rule) defined, so the instantiations compile in
// parallel.
#include "qstate_lrb_kernel.hpp"

namespace qs {
template hipError_t launch_lrb<QS_QB, QS_RND, QS_DELTA>(const Args& a, hipStream_t s);
}  // namespace qs
