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

// ---------------------------------------------------------------------------
// Reductions across the workgroup (256 threads, 4 waves) with DPP steps: the
// row steps of the 8-lane sums (swap neighbours, swap pairs, mirror the half
// row), then the row mirror, which leaves every lane of a 16-lane row with
// the row's total, and the GFX9 row broadcasts, which add lane 15 of each
// row into the next row (row mask 1010b) and lane 31 into the upper half
// (row mask 1100b).  A masked-off row reads the 0 that update_dpp supplies,
// an exact no-op for sums (and for maxima of non-negative bit patterns).
// ---------------------------------------------------------------------------
template <int CTRL, int ROWS>
__device__ __forceinline__ float dppf_rows(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xF, false));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dppu_rows(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWS, 0xF, false);
}
constexpr int kDppRowMirror = 0x140;
constexpr int kDppBcast15 = 0x142;
constexpr int kDppBcast31 = 0x143;

// Sum over groups of L = 16, 32 or 64 consecutive lanes; the group's last
// lane holds the total (every lane of the group for L = 16).
template <int L>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(L == 16 || L == 32 || L == 64, "16, 32 or 64 lanes");
  x = x + dppf_rows<0xB1, 0xF>(x);
  x = x + dppf_rows<0x4E, 0xF>(x);
  x = x + dppf_rows<0x141, 0xF>(x);
  x = x + dppf_rows<kDppRowMirror, 0xF>(x);
  if constexpr (L >= 32) x = x + dppf_rows<kDppBcast15, 0xA>(x);
  if constexpr (L == 64) x = x + dppf_rows<kDppBcast31, 0xC>(x);
  return x;
}
// Maximum of non-negative floats over the wave (on their bit patterns, whose
// unsigned order is the numeric order); lane 63 holds it.
__device__ __forceinline__ float wave_absmax(float x) {
  uint32_t u = __float_as_uint(x);
  u = max(u, dppu_rows<0xB1, 0xF>(u));
  u = max(u, dppu_rows<0x4E, 0xF>(u));
  u = max(u, dppu_rows<0x141, 0xF>(u));
  u = max(u, dppu_rows<kDppRowMirror, 0xF>(u));
  u = max(u, dppu_rows<kDppBcast15, 0xA>(u));
  u = max(u, dppu_rows<kDppBcast31, 0xC>(u));
  return __uint_as_float(u);
}

// Block sum; every thread gets the same value.  red: 4 floats.
__device__ __forceinline__ float block_sum_dpp(float x, float* red) {
  x = group_sum<64>(x);
  __syncthreads();   // red may still be read by an earlier reduction
  if ((threadIdx.x & 63) == 63) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Block sums of the R-vector p and block max of mx (mx >= 0); every thread
// gets them in out[] and the return value.  Through LDS: each thread writes
// its R partial values to P [R][256], 256/R consecutive threads sum one
// component (a fixed order: EPT entries each, then the DPP steps).  red:
// R + 4 floats.
template <int R>
__device__ __forceinline__ float block_sum_vec(const float (&p)[R], float mx, float (&out)[R], float* P,
                                               float* red) {
  static_assert(R == 8 || R == 16, "rank bound 8 or 16");
  constexpr int TPC = 256 / R;   // threads per component: 32 or 16
  constexpr int EPT = 256 / TPC; // entries each of them sums
  const int t = threadIdx.x;
  mx = wave_absmax(mx);
  __syncthreads();   // P and red may still be read by an earlier reduction
#pragma unroll
  for (int j = 0; j < R; ++j) P[j * 256 + t] = p[j];
  if ((t & 63) == 63) red[R + (t >> 6)] = mx;
  __syncthreads();
  const int j = t / TPC, part = t % TPC;
  float sum = 0.0f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) sum += P[j * 256 + part * EPT + e];
  sum = group_sum<TPC>(sum);
  if (part == TPC - 1) red[j] = sum;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < R; ++i) out[i] = red[i];
  return fmaxf(fmaxf(red[R], red[R + 1]), fmaxf(red[R + 2], red[R + 3]));
}

// Nearest rounding of x = sp inv, with BDR, as the bit pattern of a float
// whose low bits hold the code: BDR's limits are whole numbers (or
// infinite), and at most one of them is finite, so clamping x before
// rounding gives the code the rule gives after it (rint is monotone and
// fixes whole numbers).  Adding 1.5 * 2^23 rounds |x| <= Q to the nearest
// whole number, ties to even (the sum's last place is 1), and leaves it in
// the low mantissa bits: bits = c + 0x4B400000, whose low byte is c mod 256.
template <int BDR>
__device__ __forceinline__ uint32_t round_nearest_bits(float sp, float sh, float inv, float bound) {
  float x = sp * inv;
  if constexpr (BDR) x = bdr_clamp<BDR>(x, sp, sh, inv, bound);
  return __float_as_uint(x + 12582912.0f);
}

// Pack N codes given as such bit patterns (c + 0x4B400000).  int8: the low
// byte of each.  int4: the digit sum of the offset codes as in pack_codes,
// with the constant sum of 0x4B400000 16^i (mod 2^32) taken out of the base.
constexpr uint32_t magic_digit_sum() {
  uint32_t k = 0u;
  for (int i = 0; i < 8; ++i) k += 0x4B400000u << (4 * i);
  return k;
}
template <int QB, int N>
__device__ __forceinline__ void pack_code_bits(const uint32_t (&b)[N], uint32_t (&w)[(N * QB + 31) / 32]) {
  constexpr int NW = (N * QB + 31) / 32;
  if constexpr (QB == 8) {
#pragma unroll
    for (int j = 0; j < NW; ++j) w[j] = 0u;
#pragma unroll
    for (int i = 0; i < N; ++i) w[i >> 2] |= (b[i] & 0xFFu) << (8 * (i & 3));
  } else {
    static_assert(N % 8 == 0, "whole words of int4 codes");
    constexpr uint32_t base = 0x88888888u - magic_digit_sum();
#pragma unroll
    for (int j = 0; j < NW; ++j) w[j] = base;
#pragma unroll
    for (int i = 0; i < N; ++i) w[i >> 3] += b[i] << (4 * (i & 7));
#pragma unroll
    for (int j = 0; j < NW; ++j) w[j] ^= 0x88888888u;
  }
}

// Element j (runtime) of a register array, by selects.
template <int R>
__device__ __forceinline__ float pick(const float (&p)[R], int j) {
  float x = p[0];
#pragma unroll
  for (int i = 1; i < R; ++i) x = (j == i) ? p[i] : x;
  return x;
}

// A buffer row of R entries from element index i (R * entry bytes a multiple
// of 16 and the row 16-byte aligned): fp32, or bf16 (BF) widened exactly.
template <int R, int BF>
__device__ __forceinline__ void load_buf_row(const float* base, uint64_t i, float (&x)[R]) {
  if constexpr (BF) {
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(base) + i);
#pragma unroll
    for (int c = 0; c < R / 8; ++c) {
      const u32x4_t t = p[c];
      const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * c + 2 * e] = __uint_as_float(w[e] << 16);
        x[8 * c + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(base + i);
#pragma unroll
    for (int c = 0; c < R / 4; ++c) {
      const float4 t = p[c];
      x[4 * c] = t.x; x[4 * c + 1] = t.y; x[4 * c + 2] = t.z; x[4 * c + 3] = t.w;
    }
  }
}
// The same row stored; bf16 entries are already bf16 values (the low half of
// each pattern is zero), so keeping the high half is exact.
template <int R, int BF>
__device__ __forceinline__ void store_buf_row(float* base, uint64_t i, const float (&x)[R]) {
  if constexpr (BF) {
    u32x4_t* p = reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(base) + i);
#pragma unroll
    for (int c = 0; c < R / 8; ++c) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = (__float_as_uint(x[8 * c + 2 * e]) >> 16) | (__float_as_uint(x[8 * c + 2 * e + 1]) & 0xFFFF0000u);
      p[c] = u32x4_t{w[0], w[1], w[2], w[3]};
    }
  } else {
    float4* p = reinterpret_cast<float4*>(base + i);
#pragma unroll
    for (int c = 0; c < R / 4; ++c) p[c] = make_float4(x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]);
  }
}

}  // namespace

// Register budget: 5 waves per SIMD for int4 codes with nearest rounding at
// rank bound 8, where it needs no spills (except with the delta rule and a
// per-key decay together); otherwise the compiler's choice.
//
// BF = 1: the bf16 layout (row scales and the buffer factors W, U stored as
// bf16; instantiated at rank bound 8).  A new basis column is rounded to
// bf16 when made and used rounded; U is updated in fp32 and rounded before
// the merge test; the row scale is the smallest bf16 s with Q s >= max.
template <int QB, int RND, int RANK, int DELTA, int DKEY>
constexpr int lrb_min_waves() {
  return (QB == 4 && RND == 0 && RANK == 8 && !(DELTA && DKEY)) ? 5 : 1;
}

template <int QB, int RND, int DELTA, int EPL, int RANK, int BDR, int DKEY, int BF>
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
  __shared__ uint64_t smallw[4], mflagw[4];   // per-key flags, bit k of the DK-bit words
  __shared__ uint64_t dbadw[4];               // keys whose decay lies outside [2^-20, 1]

  // the buffer factors and the row scales, fp32 or bf16 (BF)
  const uint64_t woff = bhs * (uint64_t)dv * (uint64_t)r, uoff = bhs * (uint64_t)DK * (uint64_t)r;
  auto ld_buf = [&](const float* base, uint64_t i) -> float {
    if constexpr (BF) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[i]);
    else return base[i];
  };
  auto st_buf = [&](float* base, uint64_t i, float x) {
    if constexpr (BF) reinterpret_cast<uint16_t*>(base)[i] = (uint16_t)(__float_as_uint(x) >> 16);   // exact
    else base[i] = x;
  };
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
  if (r == RANK) {   // uniform: whole 16-byte-aligned rows of RANK entries, vector loads
    load_buf_row<RANK, BF>(a.W, woff + (uint64_t)tv * RANK, Wr);
    load_buf_row<RANK, BF>(a.U, uoff + (uint64_t)tk * RANK, Ur);
  } else {
#pragma unroll
    for (int j = 0; j < RANK; ++j) {
      Wr[j] = j < r ? ld_buf(a.W, woff + (uint64_t)(tv * r + j)) : 0.0f;   // j < r: uniform
      Ur[j] = j < r ? ld_buf(a.U, uoff + (uint64_t)(tk * r + j)) : 0.0f;
    }
  }
  const uint64_t trow = bh * (uint64_t)dv + (uint64_t)tv;
  const uint64_t tkey = bh * DK + (uint64_t)tk;
  const InRaw vraw = in_raw_load(a.v, a.in_bf16, trow);
  float so_raw;
  if constexpr (BF) so_raw = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(a.scales)[bhs * (uint64_t)dv + tv]);
  else so_raw = ld_nt(a.scales + bhs * (uint64_t)dv + (uint64_t)tv);
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

  // Waves that hold neither a buffer row of W nor one of U (every thread
  // from max(dv, dk) on: two of the four waves at dv = dk = 128) skip the
  // per-thread buffer arithmetic below; their rows are zero, so they only
  // add zeros to the block reductions, in which they still take part.
  const bool act = (int)__builtin_amdgcn_readfirstlane((uint32_t)tid >> 6) * 64 < (dv > DK ? dv : DK);

  // 1. the buffer decays with the state (decay acts on the key side)
  if (act) {
#pragma unroll
    for (int j = 0; j < RANK; ++j) Ur[j] = dd * Ur[j];
  }

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
        const float p = block_sum_dpp(wv * y, red);
        y = fmaf(-p, wv, y);
      }
    const float ny = sqrtf(block_sum_dpp(y * y, red));
    const float nu = sqrtf(block_sum_dpp(uv * uv, red));
    if (ny > ldexpf(nu, -10)) {
      wnew = tid < dv ? y / ny : 0.0f;
      if constexpr (BF) wnew = round_bf16(wnew);   // stored and used in the buffer's format
#pragma unroll
      for (int j = 0; j < RANK; ++j) Wr[j] = (j == n) ? wnew : Wr[j];
      n += 1;
      grown = true;
    }
  }

  // Columns from n on are not part of the basis: zero them once here, so
  // every sum below runs over all RANK columns (their terms add exact zeros)
  // and no column test is needed.  U's columns from n on are zero already.
  if (act) {
#pragma unroll
    for (int j = 0; j < RANK; ++j) Wr[j] = (j < n) ? Wr[j] : 0.0f;
  }

  // 3. coefficients c = W^T u and g = max_v |u_v| / s_v
  float c[RANK];
  float g;
  {
    float p[RANK];
    float gv = 0.0f;
#pragma unroll
    for (int j = 0; j < RANK; ++j) p[j] = 0.0f;
    if (act) {
#pragma unroll
      for (int j = 0; j < RANK; ++j) p[j] = Wr[j] * uv;
      const float au = fabsf(uv);
      gv = (so > 0.0f) ? au / so : (au > 0.0f ? __builtin_inff() : 0.0f);
    }
    g = block_sum_vec<RANK>(p, tid < dv ? gv : 0.0f, c, P, red);
  }
  // remainder u_perp = u - W c, in column order
  float up = uv;
  if (act) {
#pragma unroll
    for (int j = 0; j < RANK; ++j) up = fmaf(-c[j], Wr[j], up);
  }

  // 4. small key channels send c k_k into U
  bool sm = false;
  if (tid < DK) {
    sm = __builtin_isfinite(g) && (fabsf(kk) * g < theta);
    if (sm) {
#pragma unroll
      for (int j = 0; j < RANK; ++j) Ur[j] = fmaf(kk, c[j], Ur[j]);
    }
  }
  if constexpr (BF) {   // the updated buffer in its storage format, before the merge test
    if (act) {
#pragma unroll
      for (int j = 0; j < RANK; ++j) Ur[j] = round_bf16(Ur[j]);
    }
  }
  // W transposed into LDS for the merge test and the rows (rows below dv only)
  if (act) {
#pragma unroll
    for (int j = 0; j < RANK; ++j) Wt[j][tid] = Wr[j];
  }
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
    for (int j = 0; j < RANK; ++j) p[j] = 0.0f;
    if (act) {
#pragma unroll
      for (int j = 0; j < RANK; ++j) p[j] = Ur[j] * qq;   // all zero after a reset
    }
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
    if (r == RANK) {
      store_buf_row<RANK, BF>(a.U, uoff + (uint64_t)tid * RANK, Ur);
    } else {
#pragma unroll
      for (int j = 0; j < RANK; ++j)
        if (j < r) st_buf(a.U, uoff + (uint64_t)(tid * r + j), Ur[j]);
    }
    kl[tid] = kk;
    ql[tid] = qq;
    dl[tid] = dd;
  }
  {
    const uint64_t bs_ = __ballot(sm), bm_ = __ballot(merged);   // wave w: keys 64w .. 64w + 63
    const uint64_t bd_ = __ballot(tid < DK && !(dd >= 0x1p-20f && dd <= 1.0f));
    if ((tid & 63) == 0 && tid < DK) {
      smallw[tid >> 6] = bs_;
      dbadw[tid >> 6] = bd_;
      mflagw[tid >> 6] = bm_;
    }
  }
  if (grown && tid < dv) st_buf(a.W, woff + (uint64_t)(tid * r + (n - 1)), wnew);   // only the new column changed
  if (tid == 0) a.n[bhs] = n_new;
  __syncthreads();

  // Phase B: rows, 8 lanes per row, rows grp, grp + 32, ...
  // k, q and the decay of the lane's keys are read from LDS where used
  // (registers for more resident waves, which hide the buffer steps)
  const float* kf = kl + k0;
  const float* qf = ql + k0;
  const float* df = dl + k0;
  // the lane's keys k0 .. k0 + EPL - 1 lie in one 64-bit word (EPL <= 32 divides 64)
  constexpr uint64_t kLaneBits = EPL == 32 ? 0xFFFFFFFFull : ((1ull << EPL) - 1ull);
  const uint32_t smask = (uint32_t)((smallw[k0 >> 6] >> (k0 & 63)) & kLaneBits);
  uint64_t dw = 0;   // some key's decay outside [2^-20, 1] (workgroup-uniform)
#pragma unroll
  for (int w = 0; w < (DK + 63) / 64; ++w) dw |= dbadw[w];
  const bool dbad = __builtin_amdgcn_readfirstlane((uint32_t)((dw | (dw >> 32)) != 0)) != 0;
  uint64_t mw = 0;   // some channel of the head merged on this step
#pragma unroll
  for (int w = 0; w < (DK + 63) / 64; ++w) mw |= mflagw[w];
  const bool any_merge = __builtin_amdgcn_readfirstlane((uint32_t)((mw | (mw >> 32)) != 0)) != 0;
  uint8_t* gcode = const_cast<uint8_t*>(gc);
  auto row_step = [&](const int v, const uint32_t (&cw)[CW]) {
    const uint64_t row = bhs * (uint64_t)dv + (uint64_t)v;   // state row (Philox counter)
    const float s_old = sol[v];
    const float uu = ul[v], upv = upl[v];
    float sp[EPL], sh[EPL];
    if constexpr (QB == 8 || DELTA) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        float cf;
        if constexpr (QB == 8) cf = (float)(int32_t)(int8_t)(cw[i >> 2] >> (8 * (i & 3)));
        else cf = (float)((int32_t)(cw[i >> 3] << (28 - 4 * (i & 7))) >> 28);
        sh[i] = s_old * cf;
        sp[i] = fmaf(((smask >> i) & 1u) ? upv : uu, kf[i], (df[i] * s_old) * cf);
      }
    } else {
      // int4 codes (additive kinds) as c/16 from v_cvt_off_f32_i4 (the low
      // nibble of a selected byte: 9 instructions per 8 codes instead of a
      // sign-extending extract and a conversion each), with the 16 moved into
      // the row scale.  (Under the delta rule the same change measured 3%
      // slower, so that instantiation keeps the extract.)
      // (16 s) (c/16) is s c exactly, and (d (16 s)) (c/16) is (d s) c exactly
      // while d s stays a normal float and 16 d s finite, which holds for
      // s in [2^-100, 2^100] (or s = 0) and every decay of the head in [2^-20, 1].
      // Other rows (a uniform branch, never taken by ordinary states) scale
      // their codes back to c and keep s.
      const bool fast = !dbad && ((s_old >= 0x1p-100f && s_old <= 0x1p100f) || s_old == 0.0f);
      const bool anyslow = __ballot(!fast) != 0;
      const float sf = fast ? 16.0f * s_old : s_old;
#pragma unroll
      for (int j = 0; j < EPL / 8; ++j) {
        float cv[8];
        const uint32_t wd = cw[j], wo = wd >> 4;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          cv[2 * b] = __builtin_amdgcn_cvt_off_f32_i4((int)((wd >> (8 * b)) & 0xFFu));
          cv[2 * b + 1] = __builtin_amdgcn_cvt_off_f32_i4((int)((wo >> (8 * b)) & 0xFFu));
        }
        if (anyslow) {
#pragma unroll
          for (int e = 0; e < 8; ++e) cv[e] = fast ? cv[e] : 16.0f * cv[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 8 * j + e;
          sh[i] = sf * cv[e];
          sp[i] = fmaf(((smask >> i) & 1u) ? upv : uu, kf[i], (df[i] * sf) * cv[e]);
        }
      }
    }
    if (any_merge) {   // workgroup-uniform
      // The lane's merge flags are read here, past a compiler barrier, so
      // that their per-key tests stay in this rare branch: as loop-invariant
      // values of the whole kernel they were hoisted out of the row loop and
      // cost two vector instructions per key on every step.
      asm volatile("" ::: "memory");
      const uint32_t mmask = (uint32_t)((mflagw[k0 >> 6] >> (k0 & 63)) & kLaneBits);
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
    if constexpr (BF) row_scale_bf16<QB, SRB>(m, div_by_q<QB>(m), scale, inv, invb);
    else row_scale_fast<QB, SRB>(m, scale, inv, invb);
    uint32_t rb[EPL];
    if constexpr (RND != 0) rand_bits<RND, EPL>(row * DK + (uint64_t)k0, a.seed_lo, a.seed_hi, ix.step_lo, ix.step_hi, rb);
    uint32_t out[CW];
    if constexpr (RND == 0) {
      uint32_t cb[EPL];
#pragma unroll
      for (int i = 0; i < EPL; ++i) cb[i] = round_nearest_bits<BDR>(sp[i], sh[i], inv, a.bdr_bound);
      pack_code_bits<QB, EPL>(cb, out);
    } else {
      int32_t code[EPL];
#pragma unroll
      for (int i = 0; i < EPL; ++i) code[i] = round_elem<QB, RND, BDR>(sp[i], sh[i], inv, invb, rb[i], a.bdr_bound);
      pack_codes<QB, EPL>(code, out);
    }
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
    if constexpr (BF)
      reinterpret_cast<uint16_t*>(a.scales)[bhs * (uint64_t)dv + tid] = (uint16_t)(__float_as_uint(sl_[tid]) >> 16);
    else
      st_nt(a.scales + bhs * (uint64_t)dv + (uint64_t)tid, sl_[tid]);
  }
}

// ---------------------------------------------------------------------------
// Launchers (qstate_step_lrb.hip instantiates launch_lrb once per qbits x
// rounding x kind).
// ---------------------------------------------------------------------------
namespace {

template <int QB, int RND, int DELTA, int EPL, int RANK, int BF>
hipError_t launch_lrb_r(const Args& a, hipStream_t s) {
  const dim3 grid((uint32_t)((uint64_t)a.B * (uint64_t)a.H));
  if (a.bdr && a.bdr_bound == 0.0f) {   // the rule's zero-bound form
    if (a.decay_key) hipLaunchKernelGGL((k_step_lrb<QB, RND, DELTA, EPL, RANK, 2, 1, BF>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_step_lrb<QB, RND, DELTA, EPL, RANK, 2, 0, BF>), grid, dim3(256), 0, s, a);
  } else if (a.bdr) {
    if (a.decay_key) hipLaunchKernelGGL((k_step_lrb<QB, RND, DELTA, EPL, RANK, 1, 1, BF>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_step_lrb<QB, RND, DELTA, EPL, RANK, 1, 0, BF>), grid, dim3(256), 0, s, a);
  } else {
    if (a.decay_key) hipLaunchKernelGGL((k_step_lrb<QB, RND, DELTA, EPL, RANK, 0, 1, BF>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_step_lrb<QB, RND, DELTA, EPL, RANK, 0, 0, BF>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

// rank bound 8 or 16; the bf16 layout at rank bound 8 only
template <int QB, int RND, int DELTA, int EPL>
hipError_t launch_lrb_t(const Args& a, hipStream_t s) {
  if (a.bf16_layout) return a.lrb_rank <= 8 ? launch_lrb_r<QB, RND, DELTA, EPL, 8, 1>(a, s) : hipErrorInvalidValue;
  return a.lrb_rank <= 8 ? launch_lrb_r<QB, RND, DELTA, EPL, 8, 0>(a, s)
                         : launch_lrb_r<QB, RND, DELTA, EPL, 16, 0>(a, s);
}

template <int QB, int RND, int DELTA>
hipError_t launch_lrb_dk(const Args& a, hipStream_t s) {
  switch (a.dk) {
    case 64: return launch_lrb_t<QB, RND, DELTA, 8>(a, s);
    case 128: return launch_lrb_t<QB, RND, DELTA, 16>(a, s);
    case 256: return launch_lrb_t<QB, RND, DELTA, 32>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

template <int QB, int RND, int DELTA>
hipError_t launch_lrb(const Args& a, hipStream_t s) {
  return launch_lrb_dk<QB, RND, DELTA>(a, s);
}

}  // namespace qs
