// Step kernel for key-channel precision maps (dk 64, 128 or 256), protected
// storage 16-bit or fp32 (decay-based mixed precision per channel, abstract of
// "Quantizing Recurrent Language Models Is Easier Than You Think").
//
// A row of a mixed head is stored as two packed rows: the codes of its nq
// quantized channels in ascending key order (slot j = the j-th quantized
// channel) and the 16-bit or fp32 values of its nhp protected channels, each
// row padded to 4 bytes.  The kernel works in that storage order instead of key
// order: LPR lanes own a row, lane l holding code slots [l*EPL, l*EPL+EPL) and
// protected slots [l*EH, l*EH+EH), so every lane reads and writes
// consecutive dwords of both rows and runs the dense kernel's arithmetic on
// them.  The per-key inputs (k, q, and the decay when it is per key) are
// permuted into slot order once per workgroup in LDS; every sum of the step
// (delta term, readout) and the row maximum are order-free, and an element's
// Philox counter is its slot index, so nothing needs key order.
#pragma once
#include "qstate_step_kernels.hpp"

namespace qs {

namespace {

// 16 bytes at a dword-aligned address (global memory takes 128-bit accesses
// at 4-byte alignment).
typedef uint32_t u32x4a4_t __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2a4_t __attribute__((ext_vector_type(2), aligned(4)));

// A lane's slice of a stored row: the NW dwords at byte `off` of the row that
// starts at byte `rowo` of its head block (rowbytes long, a multiple of 4),
// of which the first nb exist.  Read in pieces of up to 16 bytes with no
// branch (a load inside a lane-dependent branch makes the compiler wait for
// it where the branch joins): a whole piece from its own address; a partial
// one from the piece-sized window that ends at the row end, moved up to the
// block start when the row is shorter than a piece (a non-empty block is a
// whole number of 16-byte units, so the window stays inside it); a missing
// one from `so` bytes past the block (the start of whichever of the head's
// two blocks is non-empty).  slice_fix, applied once the loads have landed,
// moves the valid dwords down and zeroes the rest.
template <int NW>
constexpr int slice_pw() { return NW >= 4 ? 4 : NW; }   // dwords per piece

template <int NW>
__device__ __forceinline__ void slice_load(const uint8_t* blk, uint32_t rowo, uint32_t rowbytes, uint32_t off,
                                           int64_t so, uint32_t (&w)[NW], uint32_t (&sh)[NW / slice_pw<NW>()],
                                           uint32_t (&nbv)[NW / slice_pw<NW>()]) {
  constexpr int PW = slice_pw<NW>();
  constexpr uint32_t PB = 4u * PW;
#pragma unroll
  for (int c = 0; c < NW / PW; ++c) {
    const uint32_t po = off + PB * (uint32_t)c;
    const uint32_t nb = rowbytes > po ? (rowbytes - po < PB ? rowbytes - po : PB) : 0u;
    const uint32_t end = rowo + rowbytes;                       // row end within the block
    const uint32_t win = end >= PB ? end - PB : 0u;             // window ending there, clamped
    const uint32_t o = nb == PB ? rowo + po : win;
    const uint8_t* a = blk + (nb > 0u ? (int64_t)o : so);
    nbv[c] = nb;
    sh[c] = nb > 0u ? (rowo + po - o) / 4u : 0u;
    if constexpr (PW == 4) {
      // the builtin keeps the 4-byte alignment of the type (a template
      // parameter would not)
      const u32x4a4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4a4_t*>(a));
      w[4 * c] = v.x; w[4 * c + 1] = v.y; w[4 * c + 2] = v.z; w[4 * c + 3] = v.w;
    } else if constexpr (PW == 2) {
      const u32x2a4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2a4_t*>(a));
      w[2 * c] = v.x; w[2 * c + 1] = v.y;
    } else {
      w[c] = ld_nt(reinterpret_cast<const uint32_t*>(a));
    }
  }
}

template <int NW>
__device__ __forceinline__ void slice_fix(uint32_t (&w)[NW], const uint32_t (&sh)[NW / slice_pw<NW>()],
                                          const uint32_t (&nbv)[NW / slice_pw<NW>()]) {
  constexpr int PW = slice_pw<NW>();
#pragma unroll
  for (int c = 0; c < NW / PW; ++c) {
    uint32_t t[PW];
#pragma unroll
    for (int i = 0; i < PW; ++i) t[i] = w[PW * c + i];
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      uint32_t x = t[i];
#pragma unroll
      for (int d = 1; d < PW; ++d)
        if (i + d < PW) x = sh[c] == (uint32_t)d ? t[i + d] : x;
      w[PW * c + i] = 4u * (uint32_t)i < nbv[c] ? x : 0u;
    }
  }
}

// Stores without the nontemporal hint: rows of a mixed head are not whole
// cache lines (115 int8 and 13 fp16 key channels: rows of 116 and 28
// bytes), so a line is written by pieces of several lanes and rows.  With the streaming hint a line left the L2
// part-written and was written again: counter-measured writes were 1.27x the
// bytes stored and the step 2.7-3.2% slower; plain stores let the L2 merge
// the pieces (writes equal the bytes stored).
template <int NW>
__device__ __forceinline__ void store_dwords(uint8_t* p, uint32_t nbytes, const uint32_t (&w)[NW]) {
  if constexpr (NW % 4 == 0) {
    if (nbytes == 4u * NW) {
#pragma unroll
      for (int i = 0; i < NW / 4; ++i) {
        const u32x4a4_t t = {w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
        reinterpret_cast<u32x4a4_t*>(p)[i] = t;
      }
      return;
    }
  }
  uint32_t* q = reinterpret_cast<uint32_t*>(p);
#pragma unroll
  for (int i = 0; i < NW; ++i)
    if (4u * (uint32_t)i < nbytes) q[i] = w[i];
}

}  // namespace

// LPR lanes per row, EPL = dk/LPR code slots and EH protected slots per
// lane; a lane group holds RPL rows, 256/LPR*RPL rows per workgroup.  Within
// a wave the groups take consecutive rows (group gi rows wrow0 + gi + GPW r),
// so each state access of the wave covers one contiguous stretch; the
// workgroup's per-row outputs and scales are collected in LDS and stored as
// whole cache lines.
// HP4: protected values stored as fp32 (one dword per slot), else 16-bit
// (bf16 or fp16, two slots per dword).
template <int QB, int RND, int DELTA, int EPL, int LPR, int EH, int BDR, int DKEY, int RPL, int INBF, int HP4>
__global__ __launch_bounds__(256) void k_step_keymap(const Args a) {
  constexpr int DK = EPL * LPR;
  constexpr int GPW = 64 / LPR;            // row groups per wave
  constexpr int RW = 256 / LPR * RPL;      // rows per workgroup
  constexpr int SRB = sr_bits_of<RND>();
  constexpr int CW = EPL * QB / 32;        // code words per lane and row
  constexpr int HPB = HP4 ? 4 : 2;         // bytes per protected value
  constexpr int HW = EH * HPB / 4;         // protected-value words per lane and row
  static_assert(EH % 2 == 0 && EH >= 2, "protected slots come in dword pairs");
  static_assert(DK <= 256, "one key per thread in the slot permutation");
  if (a.load_prio) __builtin_amdgcn_s_setprio(3);   // raised until the loads are issued
  const int lane = threadIdx.x & (LPR - 1);
  const int g = threadIdx.x / LPR;         // row group

  // work item (b, h, chunk of RW rows), head order rotated by b across XCDs
  const uint32_t per_b = (uint32_t)a.H * (uint32_t)a.row_chunks;
  const uint32_t b = blockIdx.x / per_b;
  uint32_t r0 = blockIdx.x - b * per_b + b % per_b;
  r0 = r0 >= per_b ? r0 - per_b : r0;
  const uint32_t chunk = r0 % (uint32_t)a.row_chunks;
  const uint32_t h = r0 / (uint32_t)a.row_chunks;
  bool ok;
  const HeadIx ix = head_ix(a, b, h, ok);
  if (!ok) return;   // uniform: a batch element with no valid state slot
  const uint64_t bh = ix.in;                               // inputs and outputs
  const uint32_t bs = (uint32_t)(ix.st / (uint64_t)a.H);   // state slot
  const int crow0 = (int)chunk * RW;                          // first row of the workgroup
  const int v0 = crow0 + (g / GPW) * GPW * RPL + g % GPW;     // rows v0 + GPW r

  // per-head layout: read-only tables at a uniform index, read through the
  // constant address space (scalar loads, all three issued together)
  typedef const int32_t __attribute__((address_space(4)))* cint_p;
  typedef const uint64_t __attribute__((address_space(4)))* cu64_p;
  const int nq = ((cint_p)a.t.nq)[h];
  const uint64_t coff_h = ((cu64_p)a.t.code_off)[h];
  const uint64_t hoff_h = ((cu64_p)a.t.hp_off)[h];
  const int nhp = DK - nq;
  const uint32_t rq = code_row_bytes(nq, QB);
  const uint32_t rh = hp_row_bytes(nhp, HPB);
  const uint8_t* cblk = a.codes + (uint64_t)bs * a.code_bstride + coff_h;
  const uint8_t* hblk = a.hp + (uint64_t)bs * a.hp_bstride + hoff_h;

  // this lane's byte ranges in the two rows, and how many of them exist
  constexpr uint32_t CB = EPL * QB / 8, HB = EH * HPB;
  const uint32_t coff = (uint32_t)lane * CB, hoff = (uint32_t)lane * HB;
  const uint32_t cvalid = rq > coff ? (rq - coff < CB ? rq - coff : CB) : 0u;
  const uint32_t hvalid = rh > hoff ? (rh - hoff < HB ? rh - hoff : HB) : 0u;

  // state loads first, then the per-row and per-head inputs: all issued
  // before anything waits (rows past dv read row 0 and are not used; a head
  // has at least one of its two blocks, whose start is readable)
  const uint8_t* sblk = rq > 0u ? cblk : hblk;
  const int64_t cso = sblk - cblk, hso = sblk - hblk;   // the readable block start, from each block
  uint32_t cw[RPL][CW], hw[RPL][HW];
  uint32_t csh[RPL][CW / slice_pw<CW>()], cnb[RPL][CW / slice_pw<CW>()];
  uint32_t hsh[RPL][HW / slice_pw<HW>()], hnb[RPL][HW / slice_pw<HW>()];
  float s_old[RPL], vin[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const int v = v0 + GPW * r;
    const uint32_t vr = (uint32_t)(v < a.dv ? v : 0);
    slice_load<CW>(cblk, vr * rq, rq, coff, cso, cw[r], csh[r], cnb[r]);
    slice_load<HW>(hblk, vr * rh, rh, hoff, hso, hw[r], hsh[r], hnb[r]);
  }
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const int v = v0 + GPW * r;
    const uint64_t vc = (uint64_t)(v < a.dv ? v : 0);
    s_old[r] = ld_nt(a.scales + ix.st * (uint64_t)a.dv + vc);
    vin[r] = load_in_scalar<INBF>(a.v, bh * (uint64_t)a.dv + vc);
  }
  const float dh = DKEY ? 1.0f : a.decay[bh];
  const float beta = a.beta ? a.beta[bh] : 1.0f;
  // this thread's k, q (and per-key decay) value for the slot permutation
  const int tk = (int)threadIdx.x < DK ? (int)threadIdx.x : 0;
  const uint64_t kidx = bh * DK + (uint64_t)tk;
  const float kv0 = load_in_scalar<INBF>(a.k, kidx);
  const float qv0 = load_in_scalar<INBF>(a.q, kidx);
  const float dd0 = DKEY ? a.decay[kidx] : 0.0f;
  const uint16_t sl0 = a.t.slots[(uint64_t)h * DK + tk];
  if (a.load_prio) __builtin_amdgcn_s_setprio(0);

  // k, q (and per-key decay) permuted into slot order: code slots in
  // lc[0..DK), protected slots in lh[0..DK); slots past nq (nhp) hold 0
  __shared__ __align__(16) float lc[3][DK];
  __shared__ __align__(16) float lh[3][DK];
  if ((int)threadIdx.x < DK) {   // 256 threads, dk 128: one key each
    const int t = (int)threadIdx.x;
    const uint16_t sl = sl0;
    const float kv = kv0, qv = qv0, dd = dd0;
    float(*dst)[DK] = (sl & kSlotProt) ? lh : lc;
    const int s = sl & 0x7FFF;
    dst[0][s] = kv;
    dst[1][s] = qv;
    if constexpr (DKEY) dst[2][s] = dd;
    if (t >= nq) {
      lc[0][t] = 0.0f;
      lc[1][t] = 0.0f;
      if constexpr (DKEY) lc[2][t] = 0.0f;
    }
    if (t >= nhp) {
      lh[0][t] = 0.0f;
      lh[1][t] = 0.0f;
      if constexpr (DKEY) lh[2][t] = 0.0f;
    }
  }
  __syncthreads();
  // valid bits of each loaded word: a row's padding (to 4 bytes) is not a
  // slot, so whatever it holds must not reach the row maximum or the sums
  uint32_t cmask[CW], hmask[HW];
  {
    const int cbits = min(max(nq - lane * EPL, 0), EPL) * QB;
    const int hbits = min(max(nhp - lane * EH, 0), EH) * 8 * HPB;
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      const int b = cbits - 32 * i;
      cmask[i] = b >= 32 ? ~0u : (b <= 0 ? 0u : (1u << b) - 1u);
    }
#pragma unroll
    for (int i = 0; i < HW; ++i) {
      const int b = hbits - 32 * i;
      hmask[i] = b >= 32 ? ~0u : (b <= 0 ? 0u : (1u << b) - 1u);
    }
  }
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    slice_fix<CW>(cw[r], csh[r], cnb[r]);
    slice_fix<HW>(hw[r], hsh[r], hnb[r]);
#pragma unroll
    for (int i = 0; i < CW; ++i) cw[r][i] &= cmask[i];
#pragma unroll
    for (int i = 0; i < HW; ++i) hw[r][i] &= hmask[i];
  }

  const float* kc = lc[0] + lane * EPL;
  const float* qc = lc[1] + lane * EPL;
  const float* dc = lc[2] + lane * EPL;
  const float* kh = lh[0] + lane * EH;
  const float* qh = lh[1] + lane * EH;
  const float* dhk = lh[2] + lane * EH;
  const bool is_bf16 = a.hp_dtype == 1;
  // per-row outputs and scales of the workgroup, stored at the end
  __shared__ float ol[RW], sl_[RW];

#pragma unroll
  for (int r = 0; r < RPL; ++r) {
  const int v = v0 + GPW * r;
  if (v < a.dv) {   // whole row groups
  const uint64_t row = ix.st * (uint64_t)a.dv + (uint64_t)v;   // state row (Philox counter)
  // old values: codes (0 past nq: padding is masked, unloaded dwords are zero)
  auto code_at = [&](int i) -> float {
    if constexpr (QB == 8) return (float)(int32_t)(int8_t)(cw[r][i >> 2] >> (8 * (i & 3)));
    else return (float)((int32_t)(cw[r][i >> 3] << (28 - 4 * (i & 7))) >> 28);
  };
  auto hp_at = [&](int i) -> float {
    if constexpr (HP4) return __uint_as_float(hw[r][i]);
    const uint32_t bits = (hw[r][i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
    return is_bf16 ? bf16_bits_to_f32(bits) : f16_bits_to_f32(bits);
  };

  float u;
  if constexpr (DELTA) {
    // head decay: S_hat k = s * sum code k + sum value k, u = beta (v - alpha
    // S_hat k); key decay: u = beta (v - sum decayed k)
    float wc = 0.0f, wh = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) wc = fmaf(DKEY ? (dc[i] * s_old[r]) * code_at(i) : code_at(i), kc[i], wc);
#pragma unroll
    for (int i = 0; i < EH; ++i) wh = fmaf(DKEY ? dhk[i] * hp_at(i) : hp_at(i), kh[i], wh);
    if constexpr (DKEY) {
      u = beta * (vin[r] - red_sum<LPR>(wc + wh));
    } else {
      const float wk = red_sum<LPR>(fmaf(s_old[r], wc, wh));
      u = beta * (vin[r] - dh * wk);
    }
  } else {
    u = beta * vin[r];
  }

  // protected slots: update, readout share, store (16-bit: rounded to nearest even)
  float o = 0.0f;
  {
    float sp[EH];
#pragma unroll
    for (int i = 0; i < EH; ++i) {
      sp[i] = fmaf(u, kh[i], (DKEY ? dhk[i] : dh) * hp_at(i));
      o = fmaf(sp[i], qh[i], o);
    }
    uint32_t ow[HW > 0 ? HW : 1];
#pragma unroll
    for (int i = 0; i < HW; ++i) {
      if constexpr (HP4) ow[i] = __float_as_uint(sp[i]);
      else ow[i] = is_bf16 ? pack_bf16x2(sp[2 * i], sp[2 * i + 1]) : pack_f16x2(sp[2 * i], sp[2 * i + 1]);
    }
    store_dwords<HW>(const_cast<uint8_t*>(hblk) + (uint64_t)v * rh + hoff, hvalid, ow);
  }

  // quantized slots: update, readout, row maximum, requantize
  const float ds = dh * s_old[r];
  float sp[EPL];
  float mx = 0.0f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    sp[i] = fmaf(u, kc[i], (DKEY ? dc[i] * s_old[r] : ds) * code_at(i));
    o = fmaf(sp[i], qc[i], o);
  }
#pragma unroll
  for (int i = 0; i < EPL; i += 2) mx = fmaxf(fmaxf(mx, fabsf(sp[i])), fabsf(sp[i + 1]));
  o = red_sum<LPR>(o);
  const float m = red_absmax<LPR>(mx);
  float scale, inv, invb;
  row_scale_fast<QB, SRB>(m, scale, inv, invb);
  uint32_t out[CW];
  const uint64_t e0 = row * DK + (uint64_t)lane * EPL;   // slot-indexed element of the first slot
  if constexpr (QB == 8 && !BDR) {
    constexpr int BYTE = SRB / 8;
    constexpr int PER = (RND == 1) ? 8 : 16;
    constexpr int NB = (RND == 0) ? 1 : (EPL + PER - 1) / PER;
#pragma unroll
    for (int gblk = 0; gblk < NB; ++gblk) {
      uint32_t x[4] = {0u, 0u, 0u, 0u};
      uint32_t sel = 0u;
      if constexpr (RND != 0) {
        const uint64_t ew = e0 + (uint64_t)(gblk * PER);
        x[0] = (RND == 1) ? (uint32_t)(ew >> 3) : (uint32_t)(ew >> 4);
        x[1] = 0u;
        x[2] = ix.step_lo;
        x[3] = ix.step_hi;
        philox10(x, a.seed_lo, a.seed_hi);
        if constexpr (RND == 2 && EPL < 16) sel = (uint32_t)((ew >> 3) & 1u);
      }
      constexpr int CNT = (RND == 0) ? EPL : ((PER < EPL) ? PER : EPL);
      uint32_t y[CNT];
#pragma unroll
      for (int j = 0; j < CNT; ++j) {
        const int i = gblk * PER + j;
        if constexpr (RND == 0) {
          y[j] = (uint32_t)(int32_t)rintf(sp[i] * inv);
        } else {
          uint32_t rbits;
          if constexpr (RND == 1) rbits = (j & 1) ? (x[j >> 1] >> 16) : (x[j >> 1] & 0xFFFFu);
          else {
            const int jj = (EPL < 16) ? (j + 8 * (int)sel) : j;
            const uint32_t word = (EPL < 16) ? (sel ? x[2 + (j >> 2)] : x[j >> 2]) : x[jj >> 2];
            rbits = (word >> (8 * (jj & 3))) & 0xFFu;
          }
          y[j] = (uint32_t)(cvt_rpi(sp[i] * invb) + (int32_t)rbits);
        }
      }
#pragma unroll
      for (int j = 0; j < CNT / 4; ++j)
        out[(gblk * PER) / 4 + j] = pack4<BYTE>(y[4 * j], y[4 * j + 1], y[4 * j + 2], y[4 * j + 3]);
    }
  } else {
    uint32_t rb[EPL];
    if constexpr (RND != 0) rand_bits<RND, EPL>(e0, a.seed_lo, a.seed_hi, ix.step_lo, ix.step_hi, rb);
    int32_t code[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const float shi = BDR ? s_old[r] * code_at(i) : 0.0f;
      code[i] = round_elem<QB, RND, BDR>(sp[i], shi, inv, invb, (RND != 0) ? rb[i] : 0u, a.bdr_bound);
    }
    pack_codes<QB, EPL>(code, out);
  }
  store_dwords<CW>(const_cast<uint8_t*>(cblk) + (uint64_t)v * rq + coff, cvalid, out);
  if (lane == 0) {
    ol[v - crow0] = o;
    sl_[v - crow0] = scale;
  }
  }   // v < dv
  }   // rows
  __syncthreads();
  const int t = (int)threadIdx.x;
  if (t < RW && crow0 + t < a.dv) {
    const uint64_t vt = (uint64_t)(crow0 + t);
    st_nt(a.out + bh * (uint64_t)a.dv + vt, ol[t]);
    st_nt(a.scales + ix.st * (uint64_t)a.dv + vt, sl_[t]);
  }
}

// ---------------------------------------------------------------------------
// Launchers (qstate_step_keymap.hip instantiates launch_keymap once per
// qbits x rounding pair).
// ---------------------------------------------------------------------------
namespace {

template <int QB, int RND, int DELTA, int DK, int EH, int RPL, int INBF, int HP4>
hipError_t launch_keymap_hp(const Args& a, hipStream_t s) {
  constexpr int LPR = 8;
  constexpr int EPL = DK / LPR;
  const dim3 grid((uint32_t)((uint64_t)a.B * (uint64_t)a.H * (uint64_t)a.row_chunks));
  if (a.bdr) {
    if (a.decay_key) hipLaunchKernelGGL((k_step_keymap<QB, RND, DELTA, EPL, LPR, EH, 1, 1, RPL, INBF, HP4>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_step_keymap<QB, RND, DELTA, EPL, LPR, EH, 1, 0, RPL, INBF, HP4>), grid, dim3(256), 0, s, a);
  } else {
    if (a.decay_key) hipLaunchKernelGGL((k_step_keymap<QB, RND, DELTA, EPL, LPR, EH, 0, 1, RPL, INBF, HP4>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_step_keymap<QB, RND, DELTA, EPL, LPR, EH, 0, 0, RPL, INBF, HP4>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <int QB, int RND, int DELTA, int DK, int EH, int RPL, int INBF>
hipError_t launch_keymap_eh(const Args& a, hipStream_t s) {
  return a.hp_dtype == 0 ? launch_keymap_hp<QB, RND, DELTA, DK, EH, RPL, INBF, 1>(a, s)
                         : launch_keymap_hp<QB, RND, DELTA, DK, EH, RPL, INBF, 0>(a, s);
}

template <int QB, int RND, int DELTA, int DK, int EH>
hipError_t launch_keymap_rpl(const Args& a, hipStream_t s) {
  if constexpr (EH * 8 > DK) {   // more protected slots than keys: never planned
    return hipErrorInvalidValue;
  } else {
    switch (a.keymap_rpl) {
      case 1: return a.in_bf16 ? launch_keymap_eh<QB, RND, DELTA, DK, EH, 1, 1>(a, s)
                               : launch_keymap_eh<QB, RND, DELTA, DK, EH, 1, 0>(a, s);
      case 2: return a.in_bf16 ? launch_keymap_eh<QB, RND, DELTA, DK, EH, 2, 1>(a, s)
                               : launch_keymap_eh<QB, RND, DELTA, DK, EH, 2, 0>(a, s);
    }
    return hipErrorInvalidValue;
  }
}

// 8 lanes per row (dk/8 code slots each); keymap_eh protected slots per lane,
// keymap_rpl (1 or 2) rows per lane group
template <int QB, int RND, int DELTA, int DK>
hipError_t launch_keymap_t(const Args& a, hipStream_t s) {
  switch (a.keymap_eh) {
    case 2: return launch_keymap_rpl<QB, RND, DELTA, DK, 2>(a, s);
    case 4: return launch_keymap_rpl<QB, RND, DELTA, DK, 4>(a, s);
    case 8: return launch_keymap_rpl<QB, RND, DELTA, DK, 8>(a, s);
    case 16: return launch_keymap_rpl<QB, RND, DELTA, DK, 16>(a, s);
    case 32: return launch_keymap_rpl<QB, RND, DELTA, DK, 32>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// dk 64, 128 or 256: 8 lanes per row (dk/8 code slots each); keymap_eh
// protected slots per lane, keymap_rpl (1 or 2) rows per lane group
template <int QB, int RND, int DK>
hipError_t launch_keymap(int delta, const Args& a, hipStream_t s) {
  if (a.dk != DK) return hipErrorInvalidValue;
  return delta ? launch_keymap_t<QB, RND, 1, DK>(a, s) : launch_keymap_t<QB, RND, 0, DK>(a, s);
}

}  // namespace qs
