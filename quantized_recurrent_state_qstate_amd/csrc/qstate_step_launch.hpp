// Launchers of the dense step kernel, templated on qbits and rounding mode;
// qstate_step_dense.hip is compiled once per (qbits, rounding) pair so the
// instantiations build in parallel.
#pragma once
#include "qstate_step_kernels.hpp"

namespace qs {

namespace {

template <int QB, int RND, int DELTA, int EPL, int LPR, int RPL, int BDR, int DKEY, int INBF>
void launch_dense_one(const Args& a, hipStream_t s) {
  const uint64_t grid = (uint64_t)a.B * (uint64_t)a.H * (uint64_t)a.row_chunks;
  hipLaunchKernelGGL((k_step_dense<QB, RND, DELTA, EPL, LPR, RPL, BDR, DKEY, INBF>), dim3((uint32_t)grid),
                     dim3((uint32_t)a.dense_threads), 0, s, a);
}

template <int QB, int RND, int DELTA, int EPL, int LPR, int RPL, int INBF>
hipError_t launch_dense_rpl(const Args& a, hipStream_t s) {
  if (a.bdr) {
    if (a.decay_key) launch_dense_one<QB, RND, DELTA, EPL, LPR, RPL, 1, 1, INBF>(a, s);
    else launch_dense_one<QB, RND, DELTA, EPL, LPR, RPL, 1, 0, INBF>(a, s);
  } else {
    if (a.decay_key) launch_dense_one<QB, RND, DELTA, EPL, LPR, RPL, 0, 1, INBF>(a, s);
    else launch_dense_one<QB, RND, DELTA, EPL, LPR, RPL, 0, 0, INBF>(a, s);
  }
  return hipGetLastError();
}

template <int QB, int RND, int DELTA, int EPL, int LPR>
hipError_t launch_dense_t(const Args& a, hipStream_t s) {
  if constexpr (LPR == 4) {
    // 32 keys per lane: one row per lane
    if (a.dense_rpl != 1) return hipErrorInvalidValue;
    return a.in_bf16 ? launch_dense_rpl<QB, RND, DELTA, EPL, LPR, 1, 1>(a, s)
                     : launch_dense_rpl<QB, RND, DELTA, EPL, LPR, 1, 0>(a, s);
  } else {
    if (a.in_bf16) {
      if (a.dense_rpl == 1) return launch_dense_rpl<QB, RND, DELTA, EPL, LPR, 1, 1>(a, s);
      if (a.dense_rpl == 2) return launch_dense_rpl<QB, RND, DELTA, EPL, LPR, 2, 1>(a, s);
    } else {
      if (a.dense_rpl == 1) return launch_dense_rpl<QB, RND, DELTA, EPL, LPR, 1, 0>(a, s);
      if (a.dense_rpl == 2) return launch_dense_rpl<QB, RND, DELTA, EPL, LPR, 2, 0>(a, s);
    }
    return hipErrorInvalidValue;
  }
}

template <int QB, int RND, int DELTA>
hipError_t launch_dense_dk(const Args& a, hipStream_t s) {
  switch (a.dk) {
    case 64: return launch_dense_t<QB, RND, DELTA, 8, 8>(a, s);
    case 128:
      return a.dense_lpr == 4 ? launch_dense_t<QB, RND, DELTA, 32, 4>(a, s)
                              : launch_dense_t<QB, RND, DELTA, 16, 8>(a, s);
    case 256: return launch_dense_t<QB, RND, DELTA, 32, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

template <int QB, int RND>
hipError_t launch_dense(int delta, const Args& a, hipStream_t s) {
  return delta ? launch_dense_dk<QB, RND, 1>(a, s) : launch_dense_dk<QB, RND, 0>(a, s);
}

}  // namespace qs
