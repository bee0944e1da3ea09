// Step kernel with the Low-Rank Bypass (abstract of "Preserving Updates in
// Low-Bit Recurrent State Quantization": small updates accumulate in a
// compact low-rank buffer whose sufficiently large elements are merged into
// the state periodically).  Both kinds the page names (additive: GLA,
// Mamba2, RetNet; delta rule: Gated DeltaNet), map NONE.
//
// Buffer of one head: L = W U^T, W [dv][r] with orthonormal columns
// 0..n-1, U [dk][r].  One workgroup of 256 threads per head (dv, dk <= 256):
// thread t holds row t of W (t < dv) and row t of U (t < dk) in registers,
// RANK >= r entries each.  Phase A follows the buffer steps (decay U, grow
// the basis while n < r, project u on the basis, route the in-span part of
// small key channels to U, merge on a merge step, buffer readout); the r
// dot products of a projection are one vector reduction.  For the delta
// rule a phase before A forms the write vector from the decayed effective
// state: each row's codes give w_v = (decayed S_hat k)_v, the decayed buffer
// adds W (U^T k), and u = beta (v - that).  Phase B is the
// row step of the dense kernel: 8 lanes per row, every row's codes loaded
// first, u_perp on small channels, merged buffer columns added before
// rounding.
#pragma once
#include "qstate_step_kernels.hpp"

namespace qs {

namespace {

// Block sums of the R-vector p and block max of mx; every thread gets them
// in out[] and the return value.  Through LDS: each thread writes its R
// partial values to P [R][256], 256/R threads sum one component (a fixed
// order), and a shuffle tree finishes it.  red: R + 4 floats.
template <int R>
__device__ __forceinline__ float block_sum_vec(const float (&p)[R], float mx, float (&out)[R], float* P,
                                               float* red) {
  static_assert(R == 8 || R == 16, "rank bound 8 or 16");
  constexpr int TPC = 256 / R;   // threads per component
  constexpr int EPT = 256 / TPC; // entries each of them sums
  const int t = threadIdx.x;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  __syncthreads();   // P and red may still be read by an earlier reduction
#pragma unroll
  for (int j = 0; j < R; ++j) P[j * 256 + t] = p[j];
  if ((t & 63) == 0) red[R + (t >> 6)] = mx;
  __syncthreads();
  const int j = t / TPC, part = t % TPC;
  float sum = 0.0f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) sum += P[j * 256 + part * EPT + e];
#pragma unroll
  for (int off = TPC / 2; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if (part == 0) red[j] = sum;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < R; ++i) out[i] = red[i];
  return fmaxf(fmaxf(red[R], red[R + 1]), fmaxf(red[R + 2], red[R + 3]));
}

// Element j (runtime) of a register array, by selects.
template <int R>
__device__ __forceinline__ float pick(const float (&p)[R], int j) {
  float x = p[0];
#pragma unroll
  for (int i = 1; i < R; ++i) x = (j == i) ? p[i] : x;
  return x;
}

}  // namespace

// Register budget: 5 waves per SIMD for int4 codes with nearest rounding at
// rank bound 8, where it needs no spills (except with the delta rule and a
// per-key decay together); otherwise the compiler's choice.
template <int QB, int RND, int RANK, int DELTA, int DKEY>
constexpr int lrb_min_waves() {
  return (QB == 4 && RND == 0 && RANK == 8 && !(DELTA && DKEY)) ? 5 : 1;
}

template <int QB, int RND, int DELTA, int EPL, int RANK, int BDR, int DKEY>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(lrb_min_waves<QB, RND, RANK, DELTA, DKEY>(), 8))) void k_step_lrb(const Args a) {
  constexpr int DK = EPL * 8;
  constexpr int SRB = sr_bits_of<RND>();
  constexpr int CW = EPL * QB / 32;
  const int tid = threadIdx.x;
  const int dv = a.dv;
  const int r = a.lrb_rank;
  const uint32_t h = blockIdx.x % (uint32_t)a.H;
  bool ok;
  const HeadIx ix = head_ix(a, blockIdx.x / (uint32_t)a.H, h, ok);
  if (!ok) return;   // uniform: a batch element with no valid state slot
  const uint64_t bh = ix.in;                               // inputs and outputs
  const uint64_t bhs = ix.st;                              // state: buffer, scales, codes
  const uint32_t bs = (uint32_t)(bhs / (uint64_t)a.H);
  const float theta = a.lrb_theta;

  __shared__ __align__(16) float Wt[RANK][256];   // W transposed, for merges and rows
  __shared__ __align__(16) float Ut[RANK][DK];    // U rows of merged channels (before clearing)
  __shared__ __align__(16) float ul[256], upl[256], sol[256], lrl[256];
  __shared__ __align__(16) float kl[DK], ql[DK], dl[DK];
  __shared__ __align__(16) float P[RANK * 256];   // reduction transpose
  // Arrays whose lives do not overlap share LDS (less LDS per workgroup, more
  // resident heads): the delta rule's per-row S_hat k is read before the
  // buffer readout lrl is written, and the per-row outputs and scales of the
  // row pass are written after the last reduction through P.
  float* const wl = lrl;
  float* const ol = P;
  float* const sl_ = P + 256;
  __shared__ float red[RANK + 4];
  __shared__ uint8_t smalll[DK], mflagl[DK];

  float* Wg = a.W + bhs * (uint64_t)dv * (uint64_t)r;
  float* Ug = a.U + bhs * (uint64_t)DK * (uint64_t)r;
  const float beta = a.beta ? a.beta[bh] : 1.0f;
  int n = a.n[bhs];

  // Every load at entry, in one burst with no lane-dependent branch (a load
  // inside such a branch makes the compiler wait for it where the branch
  // joins): this thread's W row (t < dv) and U row (t < dk), its v, s_old,
  // k, q, decay (inputs read as raw 16- or 32-bit words, widened later),
  // and the codes of its lane group's first NPF rows, which phase B (and
  // the delta rule's row pass) use after the buffer steps.
  const int lane8 = tid & 7;
  const int grp = tid >> 3;
  const int k0 = lane8 * EPL;
  constexpr int NPF = 4;                       // rows grp + 32 i, i < NPF
  const uint8_t* gc = code_block(a, bs, h);
  uint32_t pf[NPF][CW];
#pragma unroll
  for (int i = 0; i < NPF; ++i) {
    const int v = grp + 32 * i;
    load_bytes<EPL * QB / 8, true>(gc + (uint64_t)(v < dv ? v : 0) * (DK * QB / 8) + k0 * QB / 8, pf[i]);
  }
  const int tv = tid < dv ? tid : 0, tk = tid < DK ? tid : 0;
  float Wr[RANK], Ur[RANK];
#pragma unroll
  for (int j = 0; j < RANK; ++j) {
    Wr[j] = j < r ? Wg[tv * r + j] : 0.0f;   // j < r: uniform
    Ur[j] = j < r ? Ug[tk * r + j] : 0.0f;
  }
  const uint64_t trow = bh * (uint64_t)dv + (uint64_t)tv;
  const uint64_t tkey = bh * DK + (uint64_t)tk;
  const InRaw vraw = in_raw_load(a.v, a.in_bf16, trow);
  const float so_raw = ld_nt(a.scales + bhs * (uint64_t)dv + (uint64_t)tv);
  const InRaw kraw = in_raw_load(a.k, a.in_bf16, tkey);
  const InRaw qraw = in_raw_load(a.q, a.in_bf16, tkey);
  const float dd_raw = DKEY ? a.decay[tkey] : a.decay[bh];
  // widen and mask, after the burst
  const bool tv_ok = tid < dv, tk_ok = tid < DK;
#pragma unroll
  for (int j = 0; j < RANK; ++j) {
    Wr[j] = tv_ok ? Wr[j] : 0.0f;
    Ur[j] = tk_ok ? Ur[j] : 0.0f;
  }
  float uv = tv_ok ? in_raw_value(vraw, a.in_bf16) : 0.0f;
  if constexpr (!DELTA) uv = beta * uv;
  const float so = tv_ok ? so_raw : 0.0f;
  const float kk = tk_ok ? in_raw_value(kraw, a.in_bf16) : 0.0f;
  const float qq = tk_ok ? in_raw_value(qraw, a.in_bf16) : 0.0f;
  const float dd = tk_ok ? dd_raw : 0.0f;

  if constexpr (DELTA) {
    // rows: w_v = sum_k (decayed S_hat)[v][k] k_k, 8 lanes per row, four
    // rows' codes in flight at a time.  With one decay per head the sum is
    // over S_hat and alpha multiplies it below.
    if (tid < DK) {
      kl[tid] = kk;
      dl[tid] = dd;
    }
    if (tid < dv) sol[tid] = so;
    __syncthreads();
    float kf[EPL], df[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      kf[i] = kl[k0 + i];
      df[i] = dl[k0 + i];
    }
    for (int v0 = grp; v0 < dv; v0 += 32 * NPF) {
      uint32_t cw[NPF][CW];
#pragma unroll
      for (int rr = 0; rr < NPF; ++rr) {
        if (v0 == grp) {   // uniform: the prefetched rows
#pragma unroll
          for (int j = 0; j < CW; ++j) cw[rr][j] = pf[rr][j];
        } else {
          const int v = v0 + 32 * rr;
          load_bytes<EPL * QB / 8, false>(gc + (uint64_t)(v < dv ? v : 0) * (DK * QB / 8) + k0 * QB / 8, cw[rr]);
        }
      }
#pragma unroll
      for (int rr = 0; rr < NPF; ++rr) {
        const int v = v0 + 32 * rr;
        if (v < dv) {   // uniform over the 8 lanes of a row
          const float s = sol[v];
          float w = 0.0f;
#pragma unroll
          for (int i = 0; i < EPL; ++i) {
            float cf;
            if constexpr (QB == 8) cf = (float)(int32_t)(int8_t)(cw[rr][i >> 2] >> (8 * (i & 3)));
            else cf = (float)((int32_t)(cw[rr][i >> 3] << (28 - 4 * (i & 7))) >> 28);
            const float dec = DKEY ? (df[i] * s) * cf : s * cf;
            w = fmaf(dec, kf[i], w);
          }
          w = red_sum<8>(w);
          if (lane8 == 0) wl[v] = w;
        }
      }
    }
  }

  // 1. the buffer decays with the state (decay acts on the key side)
#pragma unroll
  for (int j = 0; j < RANK; ++j) Ur[j] = dd * Ur[j];

  if constexpr (DELTA) {
    // the decayed buffer's part: W (U^T k); U's columns from n on are zero,
    // so their coefficients are exact zeros.  Then u = beta (v - w_eff).
    float p[RANK], zk[RANK];
#pragma unroll
    for (int j = 0; j < RANK; ++j) p[j] = Ur[j] * kk;
    (void)block_sum_vec<RANK>(p, 0.0f, zk, P, red);   // its barriers also publish wl
    if (tid < dv) {
      float wb = 0.0f;
#pragma unroll
      for (int j = 0; j < RANK; ++j) wb = fmaf(Wr[j], zk[j], wb);
      const float w = wl[tid];
      uv = DKEY ? beta * (uv - (w + wb)) : beta * (uv - (a.decay[bh] * w + wb));
    }
  }

  // 2. grow the basis while n < r (two Gram-Schmidt passes)
  bool grown = false;
  float wnew = 0.0f;   // the new basis column's entry of this thread's row
  if (n < r) {
    float y = uv;
    for (int pass = 0; pass < 2; ++pass)
      for (int j = 0; j < n; ++j) {
        const float wv = pick<RANK>(Wr, j);
        const float p = block_sum(wv * y, red);
        y = fmaf(-p, wv, y);
      }
    const float ny = sqrtf(block_sum(y * y, red));
    const float nu = sqrtf(block_sum(uv * uv, red));
    if (ny > ldexpf(nu, -10)) {
      wnew = tid < dv ? y / ny : 0.0f;
#pragma unroll
      for (int j = 0; j < RANK; ++j) Wr[j] = (j == n) ? wnew : Wr[j];
      n += 1;
      grown = true;
    }
  }

  // Columns from n on are not part of the basis: zero them once here, so
  // every sum below runs over all RANK columns (their terms add exact zeros)
  // and no column test is needed.  U's columns from n on are zero already.
#pragma unroll
  for (int j = 0; j < RANK; ++j) Wr[j] = (j < n) ? Wr[j] : 0.0f;

  // 3. coefficients c = W^T u and g = max_v |u_v| / s_v
  float c[RANK];
  float g;
  {
    float p[RANK];
#pragma unroll
    for (int j = 0; j < RANK; ++j) p[j] = Wr[j] * uv;
    const float au = fabsf(uv);
    const float gv = (so > 0.0f) ? au / so : (au > 0.0f ? __builtin_inff() : 0.0f);
    g = block_sum_vec<RANK>(p, tid < dv ? gv : 0.0f, c, P, red);
  }
  // remainder u_perp = u - W c, in column order
  float up = uv;
#pragma unroll
  for (int j = 0; j < RANK; ++j) up = fmaf(-c[j], Wr[j], up);

  // 4. small key channels send c k_k into U
  bool sm = false;
  if (tid < DK) {
    sm = __builtin_isfinite(g) && (fabsf(kk) * g < theta);
    if (sm) {
#pragma unroll
      for (int j = 0; j < RANK; ++j) Ur[j] = fmaf(kk, c[j], Ur[j]);
    }
  }
  // W transposed into LDS for the merge test and the rows
#pragma unroll
  for (int j = 0; j < RANK; ++j) Wt[j][tid] = Wr[j];
  if (tid < dv) {
    ul[tid] = uv;
    upl[tid] = up;
    sol[tid] = so;
  }
  __syncthreads();

  // 5. merge: a channel whose buffered column reaches theta LSB in some row
  // is added to the state and cleared; a clear buffer resets the basis
  bool merged = false;
  int n_new = n;
  const uint64_t step = ((uint64_t)ix.step_hi << 32) | ix.step_lo;
  if (a.lrb_period > 0 && ((step + 1u) % (uint64_t)a.lrb_period) == 0u) {
    int left = 0;
    if (tid < DK) {
      for (int v = 0; v < dv && !merged; ++v) {
        float col = 0.0f;
#pragma unroll
        for (int j = 0; j < RANK; ++j) col = fmaf(Wt[j][v], Ur[j], col);
        if (col != 0.0f && fabsf(col) >= theta * sol[v]) merged = true;
      }
      if (merged) {
#pragma unroll
        for (int j = 0; j < RANK; ++j) {
          Ut[j][tid] = Ur[j];
          Ur[j] = 0.0f;
        }
      }
#pragma unroll
      for (int j = 0; j < RANK; ++j)
        if (j < r && Ur[j] != 0.0f) left = 1;
    }
    if (!block_or(left, red)) n_new = 0;
  }

  // 6. buffer readout z = U^T q (merged channels are clear), lr = W z
  float z[RANK];
  {
    float p[RANK];
#pragma unroll
    for (int j = 0; j < RANK; ++j) p[j] = Ur[j] * qq;   // all zero after a reset
    (void)block_sum_vec<RANK>(p, 0.0f, z, P, red);
  }
  if (tid < dv) {
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < RANK; ++j) acc = fmaf(Wr[j], z[j], acc);
    lrl[tid] = acc;
  }
  // write the buffer back
  if (tid < DK) {
#pragma unroll
    for (int j = 0; j < RANK; ++j)
      if (j < r) Ug[tid * r + j] = Ur[j];
    kl[tid] = kk;
    ql[tid] = qq;
    dl[tid] = dd;
    smalll[tid] = sm ? 1 : 0;
    mflagl[tid] = merged ? 1 : 0;
  }
  if (grown && tid < dv) Wg[tid * r + (n - 1)] = wnew;   // only the new column changed
  if (tid == 0) a.n[bhs] = n_new;
  __syncthreads();

  // Phase B: rows, 8 lanes per row, rows grp, grp + 32, ...
  // k, q and the decay of the lane's keys are read from LDS where used
  // (registers for more resident waves, which hide the buffer steps)
  const float* kf = kl + k0;
  const float* qf = ql + k0;
  const float* df = dl + k0;
  uint32_t smask = 0u, mmask = 0u;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    smask |= (smalll[k0 + i] ? 1u : 0u) << i;
    mmask |= (mflagl[k0 + i] ? 1u : 0u) << i;
  }
  uint8_t* gcode = const_cast<uint8_t*>(gc);
  auto row_step = [&](const int v, const uint32_t (&cw)[CW]) {
    const uint64_t row = bhs * (uint64_t)dv + (uint64_t)v;   // state row (Philox counter)
    const float s_old = sol[v];
    const float uu = ul[v], upv = upl[v];
    float sp[EPL], sh[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      float cf;
      if constexpr (QB == 8) cf = (float)(int32_t)(int8_t)(cw[i >> 2] >> (8 * (i & 3)));
      else cf = (float)((int32_t)(cw[i >> 3] << (28 - 4 * (i & 7))) >> 28);
      sh[i] = s_old * cf;
      sp[i] = fmaf(((smask >> i) & 1u) ? upv : uu, kf[i], (df[i] * s_old) * cf);
    }
    if (mmask) {
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if ((mmask >> i) & 1u) {
          float col = 0.0f;
#pragma unroll
          for (int j = 0; j < RANK; ++j) col = fmaf(Wt[j][v], Ut[j][k0 + i], col);
          sp[i] = sp[i] + col;
        }
    }
    float o = 0.0f, mx = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      o = fmaf(sp[i], qf[i], o);
      mx = fmaxf(mx, fabsf(sp[i]));
    }
    o = red_sum<8>(o);
    const float m = red_absmax<8>(mx);
    float scale, inv, invb;
    row_scale_fast<QB, SRB>(m, scale, inv, invb);
    uint32_t rb[EPL];
    if constexpr (RND != 0) rand_bits<RND, EPL>(row * DK + (uint64_t)k0, a.seed_lo, a.seed_hi, ix.step_lo, ix.step_hi, rb);
    int32_t code[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      code[i] = round_elem<QB, RND, BDR>(sp[i], sh[i], inv, invb, (RND != 0) ? rb[i] : 0u, a.bdr_bound);
    uint32_t out[CW];
    pack_codes<QB, EPL>(code, out);
    store_bytes<EPL * QB / 8, true>(gcode + (uint64_t)v * (DK * QB / 8) + k0 * QB / 8, out);
    if (lane8 == 0) {   // collected in LDS, stored below as whole cache lines
      ol[v] = o + lrl[v];
      sl_[v] = scale;
    }
  };
#pragma unroll
  for (int i = 0; i < NPF; ++i)
    if (grp + 32 * i < dv) row_step(grp + 32 * i, pf[i]);   // whole row groups
  for (int v = grp + 32 * NPF; v < dv; v += 32) {            // dv > 32 NPF only
    uint32_t cw[CW];
    load_bytes<EPL * QB / 8, true>(gcode + (uint64_t)v * (DK * QB / 8) + k0 * QB / 8, cw);
    row_step(v, cw);
  }
  __syncthreads();
  if (tid < dv) {
    st_nt(a.out + bh * (uint64_t)dv + (uint64_t)tid, ol[tid]);
    st_nt(a.scales + bhs * (uint64_t)dv + (uint64_t)tid, sl_[tid]);
  }
}

}  // namespace qs
