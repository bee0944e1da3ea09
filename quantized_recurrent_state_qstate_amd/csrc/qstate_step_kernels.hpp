// gfx950 step kernels of libqstate (templates; instantiated per qbits and
// rounding mode in qstate_step_q*_r*.hip): the fused quantized-state decode step.
//
// One decode step = dequantize -> decay + update -> readout -> requantize,
// in one pass over the stored state (abstract of "Preserving Updates in
// Low-Bit Recurrent State Quantization": the state is requantized after
// every update; abstract of "Quantizing Recurrent Language Models Is Easier
// Than You Think": value-axis scale grouping, decay-based mixed precision,
// stochastic rounding).  The step is HBM-bound (about 2-4 flop per state
// byte), so it runs on the vector ALUs: no MFMA.
//
// Work mapping (dense kernels): a row v of a head (one value-axis scale
// group) is owned by 8 consecutive lanes; lane j of the group holds key
// channels [j*EPL, (j+1)*EPL), EPL = dk/8, loaded with 128-bit accesses.
// Every reduction of the step (delta-rule S k, readout S q, row max) is
// over k inside one row, so it is three DPP steps inside the 8-lane group;
// rows never exchange data.  A 256-thread workgroup covers 32 rows of one
// head per row a lane holds (two rows per lane when a head has more than 32).
// Within a wave the row groups take consecutive rows (group g row g, g + 8,
// ...), so each state load of the wave covers one contiguous stretch of
// rows, and a 16-bit row is split into 128-byte pieces that 8 lanes cover
// whole (lane j: bytes 16j + 128i); every access moves whole cache lines.
#pragma once
#include <type_traits>

#include "qstate_device.hpp"
#include "qstate_internal.hpp"

namespace qs {

namespace {

__device__ __forceinline__ const uint8_t* code_block(const Args& a, uint32_t b, uint32_t h) {
  return a.codes + (uint64_t)b * a.code_bstride + a.t.code_off[h];
}
__device__ __forceinline__ const uint8_t* hp_block(const Args& a, uint32_t b, uint32_t h) {
  return a.hp + (uint64_t)b * a.hp_bstride + a.t.hp_off[h];
}
__device__ __forceinline__ int hp_elem_bytes(int dt) { return dt == 0 ? 4 : 2; }

// Head indices of batch element b, head h: state slot and step from the
// batch tables when given (read as scalar loads: b is uniform), else b and
// the launch's step.  ok = false for a slot outside the pool: that element
// is skipped (its state and outputs untouched).
__device__ __forceinline__ HeadIx head_ix(const Args& a, uint32_t b, uint32_t h, bool& ok) {
  typedef const int32_t __attribute__((address_space(4)))* cint_p;
  typedef const uint64_t __attribute__((address_space(4)))* cu64_p;
  HeadIx x;
  uint32_t bs = b;
  ok = true;
  if (a.slot) {
    const int32_t sl = ((cint_p)a.slot)[b];
    ok = sl >= 0 && sl < a.nslots;
    bs = ok ? (uint32_t)sl : 0u;
  }
  x.in = (uint64_t)b * (uint64_t)a.H + h;
  x.st = (uint64_t)bs * (uint64_t)a.H + h;
  x.step_lo = a.step_lo;
  x.step_hi = a.step_hi;
  if (a.seq_step) {
    const uint64_t st = ((cu64_p)a.seq_step)[b];
    x.step_lo = (uint32_t)st;
    x.step_hi = (uint32_t)(st >> 32);
  }
  return x;
}

// Per-lane decay factors of a head: one per key channel, or the head's
// scalar broadcast.
template <int EPL>
__device__ __forceinline__ void load_decay(const Args& a, uint64_t bh, int k0, float (&df)[EPL]) {
  if (a.decay_key) {
    load_f32<EPL>(a.decay + bh * (uint64_t)(EPL * 8) + k0, df);
  } else {
    const float d = a.decay[bh];
#pragma unroll
    for (int i = 0; i < EPL; ++i) df[i] = d;
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Dense step: every head either fully quantized or fully protected
// (precision map NONE or HEAD).  A workgroup has NG row groups of 8 lanes
// (NG = blockDim / 8) and covers NG * RPL rows of one head: lane group g
// holds the consecutive rows g*RPL .. g*RPL + RPL-1, so the per-lane inputs
// (q, k, decay) are loaded and widened once for RPL rows and a wave's rows
// are one contiguous stretch of the state, scales and outputs; every row's
// state load is issued before any row is computed.
// ---------------------------------------------------------------------------

// Pack four 32-bit words' byte B into one word (byte i from word i).
template <int B>
__device__ __forceinline__ uint32_t pack4(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3) {
  constexpr uint32_t sel = 0x0c0c0000u | ((4u + B) << 8) | (uint32_t)B;
  const uint32_t p01 = __builtin_amdgcn_perm(c1, c0, sel);
  const uint32_t p23 = __builtin_amdgcn_perm(c3, c2, sel);
  return __builtin_amdgcn_perm(p23, p01, 0x05040100u);
}

template <int INBF>
__device__ __forceinline__ float load_in_scalar(const void* base, uint64_t idx) {
  if constexpr (INBF) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
  else return reinterpret_cast<const float*>(base)[idx];
}

// max / Q, correctly rounded, as a multiply by fp32(1/Q) and one fused
// correction step: equal to the IEEE quotient for every non-negative fp32
// max, in 3 instructions (the test suite checks all 2^31 non-negative
// floats for Q = 127 and Q = 7, and inv_toward_zero over the same range).
template <int QB>
__device__ __forceinline__ float div_by_q(float m) {
  constexpr float Q = (QB == 8) ? 127.0f : 7.0f;
  constexpr float RQ = 1.0f / Q;
  const float q0 = m * RQ;
  const float r = fmaf(-q0, Q, m);
  return fmaf(r, RQ, q0);
}

// Row scale and inverse for one row: scale = max/Q correctly rounded, inv =
// Q/max rounded toward zero, invb = inv * 2^SRB; zero when the nearest Q/max
// times 2^SRB overflows (max 0 gives Q/0 = inf).
//
// The overflow test is one compare: the nearest Q/m times 2^SRB is finite
// exactly when m > Q 2^(SRB-128).  (It overflows when the nearest Q/m
// reaches 2^(128-SRB), i.e. when Q/m reaches the midpoint 2^(128-SRB)
// (1 - 2^-25) below it, and Q 2^(SRB-128) is the largest float m with Q/m at
// or above that midpoint: the next float up is larger by more than a factor
// 1 + 2^-25.)  Q 2^(SRB-128) is Q's bit pattern with the exponent lowered by
// 128 - SRB, a normal float for both Q and every SRB used.
//
// inv needs no correctly rounded quotient: inv_toward_zero takes any
// estimate within one unit in the last place of Q/m to the quotient rounded
// toward zero.  v_rcp_f32 (within 1 ulp of 1/m for normal m whose reciprocal
// is normal) and one Newton correction give such an estimate in 4
// instructions instead of the IEEE division's 10, for m in [lo, 2^126];
// rows outside that range (a max above 2^126, or, with SRB = 0, a Q/m within
// a factor 4 of the float range's top, where Q * rcp(m) may overflow) take
// the IEEE division, under a wave-uniform branch that never runs for
// ordinary states.  The test suite checks the estimate path exhaustively on
// the CPU for every float m in range, with the reciprocal taken as each of
// the three floats nearest 1/m.
template <int QB, int SRB>
__device__ __forceinline__ void row_scale_fast(float m, float& scale, float& inv, float& invb) {
  constexpr float Q = (QB == 8) ? 127.0f : 7.0f;
  constexpr uint32_t kQBits = (QB == 8) ? 0x42FE0000u : 0x40E00000u;   // bit pattern of Q
  const float lim = __uint_as_float(kQBits - ((128u - (uint32_t)SRB) << 23));   // Q 2^(SRB-128)
  const bool ok = m > lim;   // false for NaN
  const float r = __builtin_amdgcn_rcpf(m);
  const float q0 = Q * r;
  float qf = fmaf(fmaf(-q0, m, Q), r, q0);
  bool slow = m > 0x1p126f;
  if constexpr (SRB == 0) slow = slow || (ok && m < Q * 0x1p-126f);
  if (__ballot(slow)) qf = slow ? Q / m : qf;   // wave-uniform; not taken for ordinary rows
  const float iz = inv_toward_zero(Q, m, qf);
  scale = ok ? div_by_q<QB>(m) : 0.0f;
  inv = ok ? iz : 0.0f;
  invb = ok ? iz * (float)(1u << SRB) : 0.0f;
}

// A lane's k and q slices (EPL keys from k0, or the split slice of a row
// stored in pieces of GW lanes x 16 bytes of VPP values each: keys
// GW VPP (i / VPP) + VPP lane + i % VPP; VPP = 8 for 16-bit rows, 4 for fp32).
// REG: held in registers, for lanes that compute several rows; otherwise
// read from the LDS copy where they are used, which keeps 2*EPL registers free.
template <int EPL, bool REG, bool SPLIT = false, int VPP = 8, int GW = 8>
struct KQ {
  float kr[REG ? EPL : 1], qr[REG ? EPL : 1];
  const float* kl;   // the lane's first key in LDS
  const float* ql;
  static __device__ __forceinline__ int off(int i) { return SPLIT ? GW * VPP * (i / VPP) + (i % VPP) : i; }
  __device__ __forceinline__ float k(int i) const {
    if constexpr (REG) return kr[i];
    else return kl[off(i)];
  }
  __device__ __forceinline__ float q(int i) const {
    if constexpr (REG) return qr[i];
    else return ql[off(i)];
  }
};

// Key of element i of a lane's slice: contiguous (k0 + i), or, for rows
// split into pieces of GW x 16 bytes (SPLIT; GW lanes per row, VPP values
// per 16 bytes), GW VPP (i / VPP) + VPP lane + i % VPP.
template <int EPL, bool SPLIT, int VPP = 8, int GW = 8>
__device__ __forceinline__ int slice_key(int lane8, int i) {
  return SPLIT ? GW * VPP * (i / VPP) + VPP * lane8 + (i % VPP) : lane8 * EPL + i;
}

// Staging of the head's k and q into LDS as fp32 (one conversion per value
// per workgroup instead of one per value and row-lane), in two parts so the
// loads go out with the state loads: qk_load reads this thread's first
// values (unconditionally, from clamped indices: a load inside a branch makes
// the compiler wait for it where the branch joins); stage_qk stores them,
// loads any rest (workgroups smaller than 2*dk threads), synchronizes the
// workgroup, and points the lane at its slices or loads them.
template <int DK>
constexpr int qk_first() { return (2 * DK + 255) / 256; }

template <int DK, int INBF>
__device__ __forceinline__ void qk_load(const Args& a, uint64_t bh, float (&f)[qk_first<DK>()]) {
#pragma unroll
  for (int i = 0; i < qk_first<DK>(); ++i) {
    const int t = (int)threadIdx.x + i * (int)blockDim.x;
    const int tc = t < 2 * DK ? t : 0;
    const void* src = tc < DK ? a.k : a.q;
    f[i] = load_in_scalar<INBF>(src, bh * DK + (uint64_t)(tc < DK ? tc : tc - DK));
  }
}

template <int EPL, int LPR, int INBF, bool SPLIT, bool REG, int VPP = 8>
__device__ __forceinline__ void stage_qk(const Args& a, uint64_t bh, int lane8, float* lds,
                                         const float (&f)[qk_first<EPL * LPR>()],
                                         KQ<EPL, REG, SPLIT, VPP, LPR>& kq) {
  constexpr int DK = EPL * LPR;
  constexpr int NF = qk_first<DK>();
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    const int t = (int)threadIdx.x + i * (int)blockDim.x;
    if (t < 2 * DK) lds[t] = f[i];
  }
  for (int t = (int)threadIdx.x + NF * (int)blockDim.x; t < 2 * DK; t += (int)blockDim.x) {
    const void* src = t < DK ? a.k : a.q;
    lds[t] = load_in_scalar<INBF>(src, bh * DK + (uint64_t)(t < DK ? t : t - DK));
  }
  __syncthreads();
  const int k0 = slice_key<EPL, SPLIT, VPP, LPR>(lane8, 0);
  kq.kl = lds + k0;
  kq.ql = lds + DK + k0;
  if constexpr (REG) {
#pragma unroll
    for (int i = 0; i < EPL; i += 4) {
      const int kk = slice_key<EPL, SPLIT, VPP, LPR>(lane8, i);
      const float4 kv = *reinterpret_cast<const float4*>(lds + kk);
      const float4 qv = *reinterpret_cast<const float4*>(lds + DK + kk);
      kq.kr[i] = kv.x; kq.kr[i + 1] = kv.y; kq.kr[i + 2] = kv.z; kq.kr[i + 3] = kv.w;
      kq.qr[i] = qv.x; kq.qr[i + 1] = qv.y; kq.qr[i + 2] = qv.z; kq.qr[i + 3] = qv.w;
    }
  }
}

// Outputs (and scales) of a wave's GPW*RPL rows wrow0 .. (group gi holds
// rows wrow0 + gi + GPW r): lane r of a group takes its group's row r, then
// one lane permute hands lane L the value of row wrow0 + L, so each array
// gets one contiguous store per wave.  Called with every lane active.
template <int RPL, int LPR>
__device__ __forceinline__ void store_row_values(const Args& a, const HeadIx& ix, int wrow0, int lane8,
                                                 const float (&o_row)[RPL], const float* s_row) {
  constexpr int GPW = 64 / LPR;
  float ov = o_row[0], sv = s_row ? s_row[0] : 0.0f;
#pragma unroll
  for (int r = 1; r < RPL; ++r) {
    ov = lane8 == r ? o_row[r] : ov;
    if (s_row) sv = lane8 == r ? s_row[r] : sv;
  }
  const int lane = (int)(threadIdx.x & 63u);
  const int src = (LPR * (lane % GPW) + lane / GPW) * 4;   // byte address of the source lane
  ov = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(ov)));
  if (s_row) sv = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(sv)));
  if (lane < GPW * RPL && wrow0 + lane < a.dv) {
    const uint64_t v = (uint64_t)(wrow0 + lane);
    st_nt(a.out + ix.in * (uint64_t)a.dv + v, ov);
    if (s_row) st_nt(a.scales + ix.st * (uint64_t)a.dv + v, sv);
  }
}

template <int QB, int RND, int DELTA, int EPL, int LPR, int RPL, int BDR, int DKEY, int INBF>
__device__ __forceinline__ void dense_quant_rows(const Args& a, uint8_t* blk, const HeadIx& ix, int v0, int wrow0,
                                                 int lane8, float* lds) {
  const uint64_t bh = ix.in;   // inputs and outputs; the state (scales, Philox counter) at ix.st
  constexpr int DK = EPL * LPR;
  constexpr int GPW = 64 / LPR;             // row groups per wave: rows v0 + GPW r
  constexpr bool KQREG = (LPR == 8) && !(QB == 8 && RND != 0 && !BDR);   // see below
  constexpr int RB = DK * QB / 8;           // code bytes per row
  constexpr int NW = EPL * QB / 32;         // code words per lane and row
  constexpr int SRB = sr_bits_of<RND>();
  const int k0 = lane8 * EPL;
  // every load first: state rows (HBM), then per-row scalars, then the
  // head's inputs; rows past dv read row 0 and are not used (no branch
  // around a load: the compiler would wait for it where the branch joins)
  uint32_t w[RPL][NW];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const int v = v0 + GPW * r;
    load_bytes<EPL * QB / 8, true>(blk + (uint64_t)(v < a.dv ? v : 0) * RB + k0 * QB / 8, w[r]);
  }
  float s_old[RPL], vin[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const int v = v0 + GPW * r;
    const uint64_t vc = (uint64_t)(v < a.dv ? v : 0);
    s_old[r] = ld_nt(a.scales + ix.st * (uint64_t)a.dv + vc);
    vin[r] = load_in_scalar<INBF>(a.v, bh * (uint64_t)a.dv + vc);
  }
  float df[DKEY ? EPL : 1];
  float dh = 1.0f;
  if constexpr (DKEY) load_f32<EPL>(a.decay + (uint64_t)bh * DK + k0, df);
  else dh = a.decay[bh];
  const float beta = a.beta ? a.beta[bh] : 1.0f;
  float qkf[qk_first<DK>()];
  qk_load<DK, INBF>(a, bh, qkf);
  if (a.load_prio) __builtin_amdgcn_s_setprio(0);
  // Stochastic rounding's Philox blocks depend only on the element index and
  // the step, not on the state: computed while the state loads are in flight
  // (the empty asm keeps them ahead of the barrier that waits for the loads).
  constexpr int PER = (RND == 1) ? 8 : 16;                 // elements per Philox block
  constexpr int NB = (RND == 0) ? 1 : (EPL + PER - 1) / PER;
  constexpr bool PRE = (RND != 0) && QB == 8 && !BDR;
  uint32_t px[PRE ? RPL : 1][NB][4];
  if constexpr (PRE) {
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      const uint64_t row = ix.st * (uint64_t)a.dv + (uint64_t)(v0 + GPW * r);   // rows past dv: unused
#pragma unroll
      for (int gblk = 0; gblk < NB; ++gblk) {
        // element indices stay below 2^35 (checked at init): the counter's
        // high word is 0
        const uint64_t e0w = row * DK + (uint64_t)k0 + (uint64_t)(gblk * PER);
        px[r][gblk][0] = (RND == 1) ? (uint32_t)(e0w >> 3) : (uint32_t)(e0w >> 4);
        px[r][gblk][1] = 0u;
        px[r][gblk][2] = ix.step_lo;
        px[r][gblk][3] = ix.step_hi;
        philox10(px[r][gblk], a.seed_lo, a.seed_hi);
        asm volatile("" : "+v"(px[r][gblk][0]), "+v"(px[r][gblk][1]), "+v"(px[r][gblk][2]), "+v"(px[r][gblk][3]));
      }
    }
  }
  KQ<EPL, KQREG, false, 8, LPR> kq;
  stage_qk<EPL, LPR, INBF, false>(a, bh, lane8, lds, qkf, kq);
  float o_row[RPL], s_row[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const int v = v0 + GPW * r;
    o_row[r] = 0.0f;
    s_row[r] = 0.0f;
    if (v >= a.dv) continue;   // whole 8-lane groups skip together
    const uint64_t row = ix.st * (uint64_t)a.dv + (uint64_t)v;   // the element's state row
    // decay + update, readout, row maximum
    float u;
    if constexpr (DELTA) {
      // head decay: S_hat k = s * sum_k code_k k_k, u = beta (v - alpha S_hat k);
      // key decay: u = beta (v - sum_k ((d_k s) code_k) k_k)
      float wk = 0.0f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        float c;
        if constexpr (QB == 8) c = (float)(int32_t)(int8_t)(w[r][i >> 2] >> (8 * (i & 3)));
        else c = (float)((int32_t)(w[r][i >> 3] << (28 - 4 * (i & 7))) >> 28);
        wk = fmaf(DKEY ? (df[i] * s_old[r]) * c : c, kq.k(i), wk);
      }
      wk = red_sum<LPR>(wk);
      u = DKEY ? beta * (vin[r] - wk) : beta * (vin[r] - dh * (s_old[r] * wk));
    } else {
      u = beta * vin[r];
    }
    const float ds = dh * s_old[r];
    float sp[EPL];
    float o = 0.0f, mx = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      float c;
      if constexpr (QB == 8) c = (float)(int32_t)(int8_t)(w[r][i >> 2] >> (8 * (i & 3)));
      else c = (float)((int32_t)(w[r][i >> 3] << (28 - 4 * (i & 7))) >> 28);
      sp[i] = fmaf(u, kq.k(i), (DKEY ? df[i] * s_old[r] : ds) * c);
      o = fmaf(sp[i], kq.q(i), o);
    }
#pragma unroll
    for (int i = 0; i < EPL; i += 2) mx = fmaxf(fmaxf(mx, fabsf(sp[i])), fabsf(sp[i + 1]));
    o = red_sum<LPR>(o);
    const float m = red_absmax<LPR>(mx);
    o_row[r] = o;
    float scale, inv, invb;
    row_scale_fast<QB, SRB>(m, scale, inv, invb);
    s_row[r] = scale;
    // requantize
    uint32_t out[NW];
    if constexpr (QB == 8 && !BDR) {
      // byte B of y holds the code: nearest, y = rint(x); stochastic,
      // y = floor(x 2^SRB + 1/2) + rb and code = y >> SRB (|x| <= Q, so no
      // clamp)
      constexpr int BYTE = SRB / 8;
#pragma unroll
      for (int gblk = 0; gblk < NB; ++gblk) {
        uint32_t x[4] = {0u, 0u, 0u, 0u};
        uint32_t sel = 0u;   // RND 2, EPL 8: which half of the 16-element block
        if constexpr (RND != 0) {
#pragma unroll
          for (int j = 0; j < 4; ++j) x[j] = px[r][gblk][j];
          const uint32_t e0 = (uint32_t)(row * DK) + (uint32_t)k0 + (uint32_t)(gblk * PER);
          if constexpr (RND == 2 && EPL < 16) sel = (e0 >> 3) & 1u;
        }
        constexpr int CNT = (RND == 0) ? EPL : ((PER < EPL) ? PER : EPL);
        uint32_t y[CNT];
#pragma unroll
        for (int j = 0; j < CNT; ++j) {
          const int i = gblk * PER + j;
          if constexpr (RND == 0) {
            y[j] = (uint32_t)(int32_t)rintf(sp[i] * inv);   // in [-Q, Q]
          } else {
            uint32_t rbits;
            if constexpr (RND == 1) rbits = (j & 1) ? (x[j >> 1] >> 16) : (x[j >> 1] & 0xFFFFu);
            else {
              const int jj = (EPL < 16) ? (j + 8 * (int)sel) : j;
              const uint32_t word = (EPL < 16) ? (sel ? x[2 + (j >> 2)] : x[j >> 2]) : x[jj >> 2];
              rbits = (word >> (8 * (jj & 3))) & 0xFFu;
            }
            // |X| <= Q 2^SRB: the code byte (X + rbits) >> SRB stays in [-Q, Q]
            const int32_t X = cvt_rpi(sp[i] * invb);
            y[j] = (uint32_t)(X + (int32_t)rbits);
          }
        }
#pragma unroll
        for (int j = 0; j < CNT / 4; ++j)
          out[(gblk * PER) / 4 + j] = pack4<BYTE>(y[4 * j], y[4 * j + 1], y[4 * j + 2], y[4 * j + 3]);
      }
    } else if constexpr (QB == 4 && RND != 0 && !BDR) {
      // int4 with stochastic rounding: y = floor(x 2^SRB + 1/2) + rb holds
      // the code (two's complement) from bit SRB up, so byte SRB/8 of y is the
      // code's low byte and its low nibble the stored digit.  Byte permutes
      // gather that byte of the even and of the odd elements of each 8, and
      // one masked merge interleaves their nibbles: about one instruction per
      // element for what took a shift and a shift-add
      uint32_t rb[EPL];
      rand_bits<RND, EPL>(row * DK + (uint64_t)k0, a.seed_lo, a.seed_hi, ix.step_lo, ix.step_hi, rb);
      constexpr int BYTE = SRB / 8;
#pragma unroll
      for (int j = 0; j < EPL / 8; ++j) {
        uint32_t y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          y[e] = (uint32_t)(cvt_rpi(sp[8 * j + e] * invb) + (int32_t)rb[8 * j + e]);
        const uint32_t ev = pack4<BYTE>(y[0], y[2], y[4], y[6]);
        const uint32_t od = pack4<BYTE>(y[1], y[3], y[5], y[7]);
        out[j] = (ev & 0x0F0F0F0Fu) | ((od << 4) & 0xF0F0F0F0u);
      }
    } else {
      uint32_t rb[EPL];
      if constexpr (RND != 0)
        rand_bits<RND, EPL>(row * DK + (uint64_t)k0, a.seed_lo, a.seed_hi, ix.step_lo, ix.step_hi, rb);
      int32_t code[EPL];
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        float shi = 0.0f;
        if constexpr (BDR) {
          if constexpr (QB == 8) shi = s_old[r] * (float)(int32_t)(int8_t)(w[r][i >> 2] >> (8 * (i & 3)));
          else shi = s_old[r] * (float)((int32_t)(w[r][i >> 3] << (28 - 4 * (i & 7))) >> 28);
        }
        code[i] = round_elem<QB, RND, BDR>(sp[i], shi, inv, invb, (RND != 0) ? rb[i] : 0u, a.bdr_bound);
      }
      pack_codes<QB, EPL>(code, out);
    }
    store_bytes<EPL * QB / 8, true>(blk + (uint64_t)v * RB + k0 * QB / 8, out);
  }
  store_row_values<RPL, LPR>(a, ix, wrow0, lane8, o_row, s_row);
}

// Protected heads of a head map, stored as HP (0 fp32, 1 bf16, 2 fp16).  A
// row is split into pieces of 16 LPR bytes, lane j holding bytes 16j + 16 LPR i
// of each (VPP = 16 / value bytes consecutive keys per 16 bytes): with 8 lanes
// per row every load and store of the wave covers whole cache lines, with 4
// half lines.
template <int HP, int DELTA, int EPL, int LPR, int RPL, int DKEY, int INBF>
__device__ __forceinline__ void dense_prot_rows_t(const Args& a, uint8_t* blk, const HeadIx& ix, int v0,
                                                  int wrow0, int lane8, float* lds) {
  const uint64_t bh = ix.in;   // inputs and outputs
  constexpr int DK = EPL * LPR;
  constexpr int GPW = 64 / LPR;
  // Rows are split into pieces of LPR x 16 bytes: lane j of a row group holds
  // bytes 16 j + 16 LPR i, so each load covers whole 16 LPR-byte runs of a
  // row (whole cache lines with 8 lanes a row, half lines with 4) instead of
  // one 16-byte piece per line.
  constexpr bool SPLIT = true;
  constexpr int VB = HP == 0 ? 4 : 2;        // bytes per stored value
  constexpr int VPP = 16 / VB;               // values per 16-byte piece
  constexpr int NW = EPL * VB / 4;           // words per lane and row
  constexpr int NPC = NW / 4;                // 16-byte pieces per lane and row
  // byte offset of the lane's piece i within a row
  auto piece = [&](int i) -> uint32_t { return (uint32_t)(16 * LPR * i + 16 * lane8); };
  uint32_t hw[RPL][NW];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const int v = v0 + GPW * r;
    const uint8_t* rowp = blk + (uint64_t)(v < a.dv ? v : 0) * (DK * VB);   // rows past dv: unused
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
      const u32x4_t t = ld_nt(reinterpret_cast<const u32x4_t*>(rowp + piece(i)));
      hw[r][4 * i] = t.x; hw[r][4 * i + 1] = t.y; hw[r][4 * i + 2] = t.z; hw[r][4 * i + 3] = t.w;
    }
  }
  float vin[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const int v = v0 + GPW * r;
    vin[r] = load_in_scalar<INBF>(a.v, bh * (uint64_t)a.dv + (uint64_t)(v < a.dv ? v : 0));
  }
  float df[DKEY ? EPL : 1];
  float dh = 1.0f;
  if constexpr (DKEY) {
#pragma unroll
    for (int i = 0; i < EPL; i += 4) {
      const float4 t =
          *reinterpret_cast<const float4*>(a.decay + (uint64_t)bh * DK + slice_key<EPL, SPLIT, VPP, LPR>(lane8, i));
      df[i] = t.x; df[i + 1] = t.y; df[i + 2] = t.z; df[i + 3] = t.w;
    }
  } else {
    dh = a.decay[bh];
  }
  const float beta = a.beta ? a.beta[bh] : 1.0f;
  float qkf[qk_first<DK>()];
  qk_load<DK, INBF>(a, bh, qkf);
  if (a.load_prio) __builtin_amdgcn_s_setprio(0);
  KQ<EPL, false, SPLIT, VPP, LPR> kq;   // one pass over the rows' k and q: read from LDS where used
  stage_qk<EPL, LPR, INBF, SPLIT, false, VPP>(a, bh, lane8, lds, qkf, kq);
  auto value = [&](int r, int i) -> float {
    if constexpr (HP == 0) return __uint_as_float(hw[r][i]);
    const uint32_t bits = (hw[r][i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
    return HP == 1 ? bf16_bits_to_f32(bits) : f16_bits_to_f32(bits);
  };
  float o_row[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const int v = v0 + GPW * r;
    o_row[r] = 0.0f;
    if (v >= a.dv) continue;
    float u;
    if constexpr (DELTA) {
      float wk = 0.0f;   // key decay: sum_k (d_k value_k) k_k
#pragma unroll
      for (int i = 0; i < EPL; ++i) wk = fmaf(DKEY ? df[i] * value(r, i) : value(r, i), kq.k(i), wk);
      wk = red_sum<LPR>(wk);
      u = DKEY ? beta * (vin[r] - wk) : beta * (vin[r] - dh * wk);
    } else {
      u = beta * vin[r];
    }
    float sp[EPL];
    float o = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      sp[i] = fmaf(u, kq.k(i), (DKEY ? df[i] : dh) * value(r, i));
      o = fmaf(sp[i], kq.q(i), o);
    }
    o_row[r] = red_sum<LPR>(o);
    uint32_t ow[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      if constexpr (HP == 0) ow[i] = __float_as_uint(sp[i]);
      else if constexpr (HP == 1) ow[i] = pack_bf16x2(sp[2 * i], sp[2 * i + 1]);
      else ow[i] = pack_f16x2(sp[2 * i], sp[2 * i + 1]);
    }
    uint8_t* rowp = blk + (uint64_t)v * (DK * VB);
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
      const u32x4_t t = {ow[4 * i], ow[4 * i + 1], ow[4 * i + 2], ow[4 * i + 3]};
      st_nt(reinterpret_cast<u32x4_t*>(rowp + piece(i)), t);
    }
  }
  store_row_values<RPL, LPR>(a, ix, wrow0, lane8, o_row, nullptr);
}

// One body per storage format (a uniform branch).
template <int DELTA, int EPL, int LPR, int RPL, int DKEY, int INBF>
__device__ __forceinline__ void dense_prot_rows(const Args& a, uint8_t* blk, const HeadIx& ix, int v0, int wrow0,
                                                int lane8, float* lds) {
  if (a.hp_dtype == 1) dense_prot_rows_t<1, DELTA, EPL, LPR, RPL, DKEY, INBF>(a, blk, ix, v0, wrow0, lane8, lds);
  else if (a.hp_dtype == 2) dense_prot_rows_t<2, DELTA, EPL, LPR, RPL, DKEY, INBF>(a, blk, ix, v0, wrow0, lane8, lds);
  else dense_prot_rows_t<0, DELTA, EPL, LPR, RPL, DKEY, INBF>(a, blk, ix, v0, wrow0, lane8, lds);
}

// Register budget (minimum waves per SIMD the body is compiled for), chosen
// per shape as the highest occupancy at which it needs no spills: with 8
// lanes per row, dk 128 takes 7 waves with one row per lane (72 VGPRs) and 6
// with two (80 VGPRs); with 4 lanes per row (32 keys per lane) 4 waves;
// fewer with BDR, per-key decay, fp32 inputs or the delta rule; dk 64 fits
// 8; dk 256 is left to the compiler.
template <int EPL, int LPR, int RPL, int BDR, int DKEY, int INBF, int DELTA>
constexpr int dense_min_waves() {
  const int less = (BDR ? 2 : 0) + (DKEY ? 1 : 0) + (INBF ? 0 : 1) + (DELTA ? 1 : 0);
  const int w = LPR == 4 ? 4 - less
              : EPL >= 32 ? 1
              : EPL <= 8 ? (BDR ? 6 : 8)
              : (RPL == 1 ? 7 : 6) - less;
  return w < 1 ? 1 : w;
}

template <int QB, int RND, int DELTA, int EPL, int LPR, int RPL, int BDR, int DKEY, int INBF>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(dense_min_waves<EPL, LPR, RPL, BDR, DKEY, INBF, DELTA>(), 8)))
void k_step_dense(const Args a) {
  // A starting wave runs at raised priority until its loads are issued, so
  // its address arithmetic is not queued behind the rounding work of older
  // waves and the memory pipeline stays fed.
  if (a.load_prio) __builtin_amdgcn_s_setprio(3);
  const int lane8 = threadIdx.x & (LPR - 1);   // lane within the row group
  const int g = threadIdx.x / LPR;
  const int ng = blockDim.x / LPR;
  // Workgroups are dealt to the XCDs round-robin, so with the plain order an
  // XCD would only ever see the heads h = x (mod 8): under a head map some
  // XCDs would hold only quantized heads (VALU-heavy) and others most of the
  // 16-bit ones (traffic-heavy).  Rotating the (head, chunk) order by the
  // batch index gives every XCD every head in turn.
  const uint32_t per_b = (uint32_t)a.H * (uint32_t)a.row_chunks;
  const uint32_t b = blockIdx.x / per_b;
  uint32_t r = blockIdx.x - b * per_b + b % per_b;
  r = r >= per_b ? r - per_b : r;
  const uint32_t chunk = r % (uint32_t)a.row_chunks;
  const uint32_t h = r / (uint32_t)a.row_chunks;
  bool ok;
  const HeadIx ix = head_ix(a, b, h, ok);
  if (!ok) return;   // uniform: a batch element with no valid state slot
  const uint32_t bs = (uint32_t)(ix.st / (uint64_t)a.H);   // state slot
  // rows: a wave owns GPW * RPL consecutive rows from wrow0, its group gi the
  // rows wrow0 + gi + GPW r; groups past dv stay for the barrier
  constexpr int GPW = 64 / LPR;
  const int wrow0 = ((int)chunk * ng + (g / GPW) * GPW) * RPL;
  const int v0 = wrow0 + g % GPW;
  __shared__ __align__(16) float lds[2 * EPL * LPR];
  // head storage from the protected-head mask (bit h % 64 of word h / 64;
  // a head map here has at most 256 heads, and heads past 256 are
  // quantized): no table lookup stands between the launch and the state
  // loads, only scalar bit counts over the kernel arguments
  uint32_t np = 0;   // protected heads below h
  bool prot = false;
#pragma unroll
  for (uint32_t w = 0; w < 4u; ++w) {
    const uint64_t m = a.prot_mask[w];
    const uint32_t lo = 64u * w;
    if (h >= lo + 64u) {
      np += (uint32_t)__builtin_popcountll(m);
    } else if (h >= lo) {
      const uint32_t bit = h - lo;
      np += (uint32_t)__builtin_popcountll(m & ((1ull << bit) - 1ull));
      prot = ((m >> bit) & 1ull) != 0ull;
    }
  }
  if (!prot) {
    uint8_t* blk = a.codes + (uint64_t)bs * a.code_bstride + (uint64_t)(h - np) * a.code_hblk;
    dense_quant_rows<QB, RND, DELTA, EPL, LPR, RPL, BDR, DKEY, INBF>(a, blk, ix, v0, wrow0, lane8, lds);
  } else {
    uint8_t* blk = a.hp + (uint64_t)bs * a.hp_bstride + (uint64_t)np * a.hp_hblk;
    dense_prot_rows<DELTA, EPL, LPR, RPL, DKEY, INBF>(a, blk, ix, v0, wrow0, lane8, lds);
  }
}

// ---------------------------------------------------------------------------
// Block-wide reductions for the LRB kernel (256 threads = 4 waves).
// ---------------------------------------------------------------------------
namespace {
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}
// Sum over the block; every thread gets the same value.  `red` holds 4 floats.
__device__ __forceinline__ float block_sum(float x, float* red) {
  x = wave_sum(x);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}
__device__ __forceinline__ int block_or(int x, float* red) {
  x = __any(x) ? 1 : 0;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = (float)x;
  __syncthreads();
  return (red[0] + red[1] + red[2] + red[3]) > 0.0f;
}
}  // namespace

}  // namespace qs
