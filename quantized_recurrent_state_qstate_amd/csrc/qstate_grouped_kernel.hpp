// Step kernel for scale groups other than the value axis (abstract of
// "Quantizing Recurrent Language Models Is Easier Than You Think": scales
// grouped along the value axis match output channel magnitude; the key axis
// and one scale per head are the groupings that choice is measured against).
//
// A key-axis group is a column of S[v][k] and a head group the whole head, so
// a group's maximum needs every row of the head before any element can be
// rounded.  One workgroup of 256 threads per head (8 lanes per row, rows grp,
// grp + 32, ...; map NONE, no buffer), two passes over the rows:
//   1. dequantize, decay and update, readout (stored), and the running group
//      maxima of |S_pre| (per lane per key, then LDS atomics);
//   2. the group scales from the maxima, then every row again: the same
//      S_pre recomputed from the unchanged codes (the write vector of each
//      row kept in LDS), rounded against its group's scale and stored.
// An ablation path: plain loads, the state read twice.
#pragma once
#include "qstate_step_kernels.hpp"

namespace qs {

template <int QB, int RND, int DELTA, int EPL, int BDR, int DKEY, int AXIS>
__global__ __launch_bounds__(256) void k_step_grouped(const Args a) {
  static_assert(AXIS == 1 || AXIS == 2, "key-axis or per-head groups");
  constexpr int DK = EPL * 8;
  constexpr int SRB = sr_bits_of<RND>();
  constexpr int RB = DK * QB / 8;          // code bytes per row
  constexpr int CW = EPL * QB / 32;        // code words per lane and row
  constexpr int G = AXIS == 1 ? DK : 1;    // groups per head
  const int tid = threadIdx.x;
  const int lane8 = tid & 7;
  const int grp = tid >> 3;
  const int k0 = lane8 * EPL;
  const uint32_t h = blockIdx.x % (uint32_t)a.H;
  bool ok;
  const HeadIx ix = head_ix(a, blockIdx.x / (uint32_t)a.H, h, ok);
  if (!ok) return;   // uniform: a batch element with no valid state slot
  const uint64_t bh = ix.in;                               // inputs and outputs
  const uint64_t bhs = ix.st;                              // state
  const uint32_t bs = (uint32_t)(bhs / (uint64_t)a.H);
  uint8_t* blk = const_cast<uint8_t*>(code_block(a, bs, h));
  const int dv = a.dv;

  __shared__ uint32_t gmax[G];             // group maxima of |S_pre| (bit patterns, all >= 0)
  __shared__ float ginv[G], ginvb[G];
  __shared__ float ul[256];                // each row's write vector u
  for (int t = tid; t < G; t += 256) gmax[t] = 0u;

  // the lane's keys: k, q, decay, and the old scales of their groups
  float kf[EPL], qf[EPL], df[EPL], so[AXIS == 1 ? EPL : 1];
  load_in<EPL>(a.k, a.in_bf16, bh * DK + (uint64_t)k0, kf);
  load_in<EPL>(a.q, a.in_bf16, bh * DK + (uint64_t)k0, qf);
  load_decay<EPL>(a, bh, k0, df);
  if constexpr (AXIS == 1) load_f32<EPL>(a.scales + bhs * DK + (uint64_t)k0, so);
  else so[0] = a.scales[bhs];
  const float beta = a.beta ? a.beta[bh] : 1.0f;
  auto s_of = [&](int i) -> float { return so[AXIS == 1 ? i : 0]; };
  __syncthreads();

  // S_pre of a row slice from its codes and the row's write vector; sh the
  // dequantized old values (for BDR)
  auto row_pre = [&](const uint32_t (&w)[CW], float u, float (&sp)[EPL], float (&sh)[EPL]) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      float c;
      if constexpr (QB == 8) c = (float)(int32_t)(int8_t)(w[i >> 2] >> (8 * (i & 3)));
      else c = (float)((int32_t)(w[i >> 3] << (28 - 4 * (i & 7))) >> 28);
      sh[i] = s_of(i) * c;
      sp[i] = fmaf(u, kf[i], (df[i] * s_of(i)) * c);
    }
  };

  // pass 1: update, readout, group maxima
  float cm[AXIS == 1 ? EPL : 1];
#pragma unroll
  for (int i = 0; i < (AXIS == 1 ? EPL : 1); ++i) cm[i] = 0.0f;
  for (int v = grp; v < dv; v += 32) {
    uint32_t w[CW];
    load_bytes<EPL * QB / 8>(blk + (uint64_t)v * RB + k0 * QB / 8, w);
    const float vin = load_in1(a.v, a.in_bf16, bh * (uint64_t)dv + (uint64_t)v);
    float u;
    if constexpr (DELTA) {
      // the decayed old state times k: head decay alpha (S_hat k), key decay
      // sum_k ((d_k s) c) k_k
      float wk = 0.0f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        float c;
        if constexpr (QB == 8) c = (float)(int32_t)(int8_t)(w[i >> 2] >> (8 * (i & 3)));
        else c = (float)((int32_t)(w[i >> 3] << (28 - 4 * (i & 7))) >> 28);
        wk = fmaf(DKEY ? (df[i] * s_of(i)) * c : s_of(i) * c, kf[i], wk);
      }
      wk = sum8(wk);
      u = DKEY ? beta * (vin - wk) : beta * (vin - df[0] * wk);
    } else {
      u = beta * vin;
    }
    float sp[EPL], sh[EPL];
    row_pre(w, u, sp, sh);
    float o = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      o = fmaf(sp[i], qf[i], o);
      if constexpr (AXIS == 1) cm[i] = fmaxf(cm[i], fabsf(sp[i]));
      else cm[0] = fmaxf(cm[0], fabsf(sp[i]));
    }
    o = sum8(o);
    if (lane8 == 0) {
      st_nt(a.out + bh * (uint64_t)dv + (uint64_t)v, o);
      ul[v] = u;
    }
  }
  if constexpr (AXIS == 1) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) atomicMax(&gmax[k0 + i], __float_as_uint(cm[i]));
  } else {
    atomicMax(&gmax[0], __float_as_uint(cm[0]));
  }
  __syncthreads();

  // group scales (IEEE quotient and toward-zero inverse, as for rows)
  for (int t = tid; t < G; t += 256) {
    float scale, inv, invb;
    row_scale<QB, SRB>(__uint_as_float(gmax[t]), scale, inv, invb);
    ginv[t] = inv;
    ginvb[t] = invb;
    st_nt(a.scales + bhs * G + (uint64_t)t, scale);
  }
  __syncthreads();

  // pass 2: the same S_pre again, rounded against the group scales
  for (int v = grp; v < dv; v += 32) {
    uint32_t w[CW];
    load_bytes<EPL * QB / 8>(blk + (uint64_t)v * RB + k0 * QB / 8, w);
    float sp[EPL], sh[EPL];
    row_pre(w, ul[v], sp, sh);
    const uint64_t row = bhs * (uint64_t)dv + (uint64_t)v;   // Philox element index of the row's first key
    uint32_t rb[EPL];
    if constexpr (RND != 0) rand_bits<RND, EPL>(row * DK + (uint64_t)k0, a.seed_lo, a.seed_hi, ix.step_lo, ix.step_hi, rb);
    int32_t code[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int g = AXIS == 1 ? k0 + i : 0;
      code[i] = round_elem<QB, RND, BDR>(sp[i], sh[i], ginv[g], ginvb[g], (RND != 0) ? rb[i] : 0u, a.bdr_bound);
    }
    uint32_t out[CW];
    pack_codes<QB, EPL>(code, out);
    store_bytes<EPL * QB / 8, true>(blk + (uint64_t)v * RB + k0 * QB / 8, out);
  }
}

// ---------------------------------------------------------------------------
// Launchers (qstate_step_grouped.hip instantiates launch_grouped once per
// qbits x rounding pair).
// ---------------------------------------------------------------------------
namespace {

template <int QB, int RND, int DELTA, int EPL, int AXIS>
hipError_t launch_grouped_a(const Args& a, hipStream_t s) {
  const dim3 grid((uint32_t)((uint64_t)a.B * (uint64_t)a.H));
  if (a.bdr) {
    if (a.decay_key) hipLaunchKernelGGL((k_step_grouped<QB, RND, DELTA, EPL, 1, 1, AXIS>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_step_grouped<QB, RND, DELTA, EPL, 1, 0, AXIS>), grid, dim3(256), 0, s, a);
  } else {
    if (a.decay_key) hipLaunchKernelGGL((k_step_grouped<QB, RND, DELTA, EPL, 0, 1, AXIS>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_step_grouped<QB, RND, DELTA, EPL, 0, 0, AXIS>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <int QB, int RND, int DELTA, int EPL>
hipError_t launch_grouped_t(const Args& a, hipStream_t s) {
  if (a.scale_axis == 1) return launch_grouped_a<QB, RND, DELTA, EPL, 1>(a, s);
  if (a.scale_axis == 2) return launch_grouped_a<QB, RND, DELTA, EPL, 2>(a, s);
  return hipErrorInvalidValue;
}

template <int QB, int RND, int DELTA>
hipError_t launch_grouped_dk(const Args& a, hipStream_t s) {
  switch (a.dk) {
    case 64: return launch_grouped_t<QB, RND, DELTA, 8>(a, s);
    case 128: return launch_grouped_t<QB, RND, DELTA, 16>(a, s);
    case 256: return launch_grouped_t<QB, RND, DELTA, 32>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

template <int QB, int RND>
hipError_t launch_grouped(int delta, const Args& a, hipStream_t s) {
  return delta ? launch_grouped_dk<QB, RND, 1>(a, s) : launch_grouped_dk<QB, RND, 0>(a, s);
}

}  // namespace qs
