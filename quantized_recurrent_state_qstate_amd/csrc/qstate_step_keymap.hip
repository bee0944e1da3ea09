// Key-map step kernels (per-channel precision map) for one qbits x rounding
// pair and one dk: the build compiles this unit once per triple, with QS_QB
// (8 or 4), QS_RND (0 nearest, 1 stochastic 16-bit, 2 stochastic 8-bit) and
// QS_DK (64, 128 or 256) defined, so the instantiations compile in parallel.
#include "qstate_keymap_kernel.hpp"

namespace qs {
template hipError_t launch_keymap<QS_QB, QS_RND, QS_DK>(int delta, const Args& a, hipStream_t s);
}  // namespace qs
