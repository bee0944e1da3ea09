// Step kernels for int8 codes with sr16 rounding (one translation unit
// per qbits x rounding mode so the instantiations compile in parallel).
#include "qstate_step_launch.hpp"

namespace qs {
template hipError_t launch_step_qr<8, 1>(int family, int delta, const Args& a, hipStream_t s);
}  // namespace qs
