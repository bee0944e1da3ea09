// Step-kernel launchers of libqstate, templated on qbits and rounding mode;
// each qstate_step_q*_r*.hip translation unit instantiates one pair so the
// kernels compile in parallel.
#pragma once
#include "qstate_keymap_kernel.hpp"
#include "qstate_lrb_kernel.hpp"

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

template <int QB, int RND, int DELTA, int EPL>
hipError_t launch_mixed_t(const Args& a, hipStream_t s) {
  const uint64_t grid = (uint64_t)a.B * (uint64_t)a.H;
  hipLaunchKernelGGL((k_step_mixed<QB, RND, DELTA, EPL>), dim3((uint32_t)grid), dim3(256), a.mixed_lds, s, a);
  return hipGetLastError();
}

template <int QB, int RND, int DELTA, int EPL, int RANK>
hipError_t launch_lrb_r(const Args& a, hipStream_t s) {
  const dim3 grid((uint32_t)((uint64_t)a.B * (uint64_t)a.H));
  if (a.bdr && a.bdr_bound == 0.0f) {   // the rule's zero-bound form
    if (a.decay_key) hipLaunchKernelGGL((k_step_lrb<QB, RND, DELTA, EPL, RANK, 2, 1>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_step_lrb<QB, RND, DELTA, EPL, RANK, 2, 0>), grid, dim3(256), 0, s, a);
  } else if (a.bdr) {
    if (a.decay_key) hipLaunchKernelGGL((k_step_lrb<QB, RND, DELTA, EPL, RANK, 1, 1>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_step_lrb<QB, RND, DELTA, EPL, RANK, 1, 0>), grid, dim3(256), 0, s, a);
  } else {
    if (a.decay_key) hipLaunchKernelGGL((k_step_lrb<QB, RND, DELTA, EPL, RANK, 0, 1>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_step_lrb<QB, RND, DELTA, EPL, RANK, 0, 0>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <int QB, int RND, int DELTA, int EPL>
hipError_t launch_lrb_t(const Args& a, hipStream_t s) {
  return a.lrb_rank <= 8 ? launch_lrb_r<QB, RND, DELTA, EPL, 8>(a, s)
                         : launch_lrb_r<QB, RND, DELTA, EPL, 16>(a, s);
}

template <int QB, int RND, int DELTA, int LPR, int EH, int RPL, int INBF>
hipError_t launch_keymap_eh(const Args& a, hipStream_t s) {
  constexpr int EPL = 128 / LPR;
  const dim3 grid((uint32_t)((uint64_t)a.B * (uint64_t)a.H * (uint64_t)a.row_chunks));
  if (a.bdr) {
    if (a.decay_key) hipLaunchKernelGGL((k_step_keymap<QB, RND, DELTA, EPL, LPR, EH, 1, 1, RPL, INBF>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_step_keymap<QB, RND, DELTA, EPL, LPR, EH, 1, 0, RPL, INBF>), grid, dim3(256), 0, s, a);
  } else {
    if (a.decay_key) hipLaunchKernelGGL((k_step_keymap<QB, RND, DELTA, EPL, LPR, EH, 0, 1, RPL, INBF>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_step_keymap<QB, RND, DELTA, EPL, LPR, EH, 0, 0, RPL, INBF>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <int QB, int RND, int DELTA, int EH>
hipError_t launch_keymap_rpl(const Args& a, hipStream_t s) {
  switch (a.keymap_rpl) {
    case 1: return a.in_bf16 ? launch_keymap_eh<QB, RND, DELTA, 8, EH, 1, 1>(a, s)
                             : launch_keymap_eh<QB, RND, DELTA, 8, EH, 1, 0>(a, s);
    case 2: return a.in_bf16 ? launch_keymap_eh<QB, RND, DELTA, 8, EH, 2, 1>(a, s)
                             : launch_keymap_eh<QB, RND, DELTA, 8, EH, 2, 0>(a, s);
  }
  return hipErrorInvalidValue;
}

// dk 128: 8 lanes per row (16 code slots each); keymap_eh protected slots
// per lane, keymap_rpl (1 or 2) rows per lane group
template <int QB, int RND, int DELTA>
hipError_t launch_keymap_t(const Args& a, hipStream_t s) {
  switch (a.keymap_eh) {
    case 2: return launch_keymap_rpl<QB, RND, DELTA, 2>(a, s);
    case 4: return launch_keymap_rpl<QB, RND, DELTA, 4>(a, s);
    case 8: return launch_keymap_rpl<QB, RND, DELTA, 8>(a, s);
    case 16: return launch_keymap_rpl<QB, RND, DELTA, 16>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int QB, int RND, int DELTA>
hipError_t launch_fam(int family, const Args& a, hipStream_t s) {
  if (family == kFamKeymap) return a.dk == 128 ? launch_keymap_t<QB, RND, DELTA>(a, s) : hipErrorInvalidValue;
  if (family == kFamDense) {
    switch (a.dk) {
      case 64: return launch_dense_t<QB, RND, DELTA, 8, 8>(a, s);
      case 128:
        return a.dense_lpr == 4 ? launch_dense_t<QB, RND, DELTA, 32, 4>(a, s)
                                : launch_dense_t<QB, RND, DELTA, 16, 8>(a, s);
      case 256: return launch_dense_t<QB, RND, DELTA, 32, 8>(a, s);
    }
  } else if (family == kFamMixed) {
    switch (a.dk) {
      case 64: return launch_mixed_t<QB, RND, DELTA, 8>(a, s);
      case 128: return launch_mixed_t<QB, RND, DELTA, 16>(a, s);
      case 256: return launch_mixed_t<QB, RND, DELTA, 32>(a, s);
    }
  } else if (family == kFamLrb) {
    switch (a.dk) {
      case 64: return launch_lrb_t<QB, RND, DELTA, 8>(a, s);
      case 128: return launch_lrb_t<QB, RND, DELTA, 16>(a, s);
      case 256: return launch_lrb_t<QB, RND, DELTA, 32>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

template <int QB, int RND>
hipError_t launch_step_qr(int family, int delta, const Args& a, hipStream_t s) {
  return delta ? launch_fam<QB, RND, 1>(family, a, s) : launch_fam<QB, RND, 0>(family, a, s);
}

}  // namespace qs
