// The LDS-staged step kernel, the general path for precision maps the
// streaming kernels do not take (key maps at dk 64 and 256, head maps over
// more than 256 heads), and its launchers; qstate_step_mixed.hip is compiled
// once per (qbits, rounding) pair.
#pragma once
#include "qstate_step_kernels.hpp"

namespace qs {

// ---------------------------------------------------------------------------
// Mixed step, the general path for heads that mix quantized and protected
// key channels (key maps at dk 64 and 256, and head maps over more than 256
// heads): a row holds the two kinds in two packed areas.  The head's code and protected blocks are staged through LDS with
// 128-bit accesses; each lane gathers its logical channels by slot, computes
// as the dense kernel, scatters back, and the workgroup writes the blocks
// out.  One workgroup per head.
// ---------------------------------------------------------------------------
template <int QB, int RND, int DELTA, int EPL>
__global__ __launch_bounds__(256) void k_step_mixed(const Args a) {
  constexpr int DK = EPL * 8;
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane8 = tid & 7;
  const int rloc = tid >> 3;
  const uint32_t h = blockIdx.x % (uint32_t)a.H;
  const uint32_t b = blockIdx.x / (uint32_t)a.H;
  bool ok;
  const HeadIx ix = head_ix(a, b, h, ok);
  if (!ok) return;   // uniform: a batch element with no valid state slot
  const uint64_t bh = ix.in;                               // inputs and outputs
  const uint32_t bs = (uint32_t)(ix.st / (uint64_t)a.H);   // state slot
  const int nq = a.t.nq[h];
  const int nhp = DK - nq;
  const int hpb = hp_elem_bytes(a.hp_dtype);
  const uint32_t rq = code_row_bytes(nq, QB);
  const uint32_t rh = hp_row_bytes(nhp, hpb);
  const uint32_t code_bytes = ((uint32_t)a.dv * rq + 15u) & ~15u;
  const uint32_t hp_bytes = ((uint32_t)a.dv * rh + 15u) & ~15u;
  uint8_t* gcode = const_cast<uint8_t*>(code_block(a, bs, h));
  uint8_t* ghp = const_cast<uint8_t*>(hp_block(a, bs, h));
  uint8_t* lcode = lds;
  uint8_t* lhp = lds + code_bytes;

  for (uint32_t i = (uint32_t)tid * 16u; i < code_bytes; i += 256u * 16u)
    *reinterpret_cast<u32x4_t*>(lcode + i) = ld_nt(reinterpret_cast<const u32x4_t*>(gcode + i));
  for (uint32_t i = (uint32_t)tid * 16u; i < hp_bytes; i += 256u * 16u)
    *reinterpret_cast<u32x4_t*>(lhp + i) = ld_nt(reinterpret_cast<const u32x4_t*>(ghp + i));

  const int k0 = lane8 * EPL;
  uint16_t sl[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) sl[i] = a.t.slots[(uint64_t)h * DK + k0 + i];
  float kf[EPL], df[EPL], qf[EPL];
  load_in<EPL>(a.k, a.in_bf16, (uint64_t)bh * DK + k0, kf);
  load_in<EPL>(a.q, a.in_bf16, (uint64_t)bh * DK + k0, qf);
  load_decay<EPL>(a, bh, k0, df);
  const float beta = a.beta ? a.beta[bh] : 1.0f;
  // random bits by slot (stochastic rounding of a mixed head): this row
  // group's DK 16-bit values, after the staged blocks
  uint16_t* rbuf = reinterpret_cast<uint16_t*>(lds + code_bytes + hp_bytes) + rloc * DK;
  __syncthreads();

  for (int v = rloc; v < a.dv; v += 32) {
    const uint64_t row = ix.st * (uint64_t)a.dv + (uint64_t)v;      // state row
    const uint64_t orow = bh * (uint64_t)a.dv + (uint64_t)v;        // input / output row
    const float s_old = ld_nt(a.scales + row);
    const float vin = load_in1(a.v, a.in_bf16, orow);
    uint8_t* crow = lcode + (uint32_t)v * rq;
    uint8_t* hrow = lhp + (uint32_t)v * rh;
    float sh[EPL], dec[EPL];   // dequantized value; decayed value (d s) c or d h
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const uint32_t s = sl[i] & 0x7FFFu;
      if (sl[i] & kSlotProt) {
        if (a.hp_dtype == 0) sh[i] = *reinterpret_cast<const float*>(hrow + s * 4u);
        else {
          const uint32_t bits = *reinterpret_cast<const uint16_t*>(hrow + s * 2u);
          sh[i] = (a.hp_dtype == 1) ? bf16_bits_to_f32(bits) : f16_bits_to_f32(bits);
        }
        dec[i] = df[i] * sh[i];
      } else {
        int32_t c;
        if constexpr (QB == 8) c = (int32_t)(int8_t)crow[s];
        else c = (int32_t)((uint32_t)crow[s >> 1] << (28 - 4 * (s & 1))) >> 28;
        sh[i] = s_old * (float)c;
        dec[i] = (df[i] * s_old) * (float)c;
      }
    }
    float u;
    if constexpr (DELTA) {
      // head decay: u = beta (v - alpha S_hat k); key decay: u = beta (v -
      // sum_k decayed_k k_k)
      float w = 0.0f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) w = fmaf(a.decay_key ? dec[i] : sh[i], kf[i], w);
      w = sum8(w);
      u = a.decay_key ? beta * (vin - w) : beta * (vin - df[0] * w);
    } else {
      u = beta * vin;
    }
    float sp[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) sp[i] = fmaf(u, kf[i], dec[i]);
    float o = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) o = fmaf(sp[i], qf[i], o);
    o = sum8(o);
    if (lane8 == 0) st_nt(a.out + orow, o);

    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (!(sl[i] & kSlotProt)) m = fmaxf(m, fabsf(sp[i]));
    m = max8(m);
    float scale, inv, invb;
    row_scale<QB, sr_bits_of<RND>()>(m, scale, inv, invb);
    // random bits by stored slot: rand_bits over the lane's keys when the
    // whole head is quantized (slot = key), one Philox block per element
    // otherwise
    uint32_t rb[EPL];
    if constexpr (RND != 0) {
      if (nq == DK) {
        rand_bits<RND, EPL>(row * DK + (uint64_t)k0, a.seed_lo, a.seed_hi, ix.step_lo, ix.step_hi, rb);
      } else if (a.mixed_rbuf) {
        // the values of slots k0 .. k0 + EPL - 1 (element row * DK + slot, as
        // for a fully quantized head), then each of this lane's elements by
        // its own slot; the 8 lanes of the row are one wave's, so their LDS
        // writes land before these reads
        rand_bits<RND, EPL>(row * DK + (uint64_t)k0, a.seed_lo, a.seed_hi, ix.step_lo, ix.step_hi, rb);
#pragma unroll
        for (int i = 0; i < EPL; ++i) rbuf[k0 + i] = (uint16_t)rb[i];
#pragma unroll
        for (int i = 0; i < EPL; ++i) rb[i] = (sl[i] & kSlotProt) ? 0u : (uint32_t)rbuf[sl[i] & 0x7FFFu];
      } else {
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          rb[i] = (sl[i] & kSlotProt) ? 0u
                                      : rand_one<RND>(row * DK + (uint64_t)(sl[i] & 0x7FFFu), a.seed_lo, a.seed_hi,
                                                      ix.step_lo, ix.step_hi);
      }
    }
    int32_t code[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const uint32_t rbi = (RND != 0) ? rb[i] : 0u;
      code[i] = a.bdr ? round_elem<QB, RND, 1>(sp[i], sh[i], inv, invb, rbi, a.bdr_bound)
                      : round_elem<QB, RND, 0>(sp[i], sh[i], inv, invb, rbi, a.bdr_bound);
    }

    // scatter: protected values and int8 codes are whole bytes of their own
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const uint32_t s = sl[i] & 0x7FFFu;
      if (sl[i] & kSlotProt) {
        if (a.hp_dtype == 0) *reinterpret_cast<float*>(hrow + s * 4u) = sp[i];
        else *reinterpret_cast<uint16_t*>(hrow + s * 2u) =
            (uint16_t)((a.hp_dtype == 1) ? f32_to_bf16_bits(sp[i]) : f32_to_f16_bits(sp[i]));
      } else if constexpr (QB == 8) {
        crow[s] = (uint8_t)code[i];
      }
    }
    if constexpr (QB == 4) {
      // int4: first every byte whose even (low-nibble) slot this lane holds,
      // with the odd nibble too when the lane holds it; then the odd nibble
      // of a byte whose even slot the previous lane holds, by atomic OR.
      // Both passes are instructions of this wave, so they land in order.
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        if (sl[i] & kSlotProt) continue;
        const uint32_t s = sl[i];
        if ((s & 1u) == 0u) {
          uint32_t byte = (uint32_t)code[i] & 0xFu;
          // the odd partner is the next quantized channel of this lane, if any
          for (int j = i + 1; j < EPL; ++j)
            if (!(sl[j] & kSlotProt)) {
              if (sl[j] == s + 1u) byte |= ((uint32_t)code[j] & 0xFu) << 4;
              break;
            }
          crow[s >> 1] = (uint8_t)byte;
        }
      }
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        if (sl[i] & kSlotProt) continue;
        const uint32_t s = sl[i];
        if (s & 1u) {
          bool partner_here = false;
          for (int j = i - 1; j >= 0; --j)
            if (!(sl[j] & kSlotProt)) {
              partner_here = (sl[j] == s - 1u);
              break;
            }
          if (!partner_here) {
            const uint32_t addr = (uint32_t)(crow - lds) + (s >> 1);
            atomicOr(reinterpret_cast<uint32_t*>(lds + (addr & ~3u)),
                     (((uint32_t)code[i] & 0xFu) << 4) << (8 * (addr & 3u)));
          }
        }
      }
    }
    if (lane8 == 0) st_nt(a.scales + row, scale);
  }
  __syncthreads();
  for (uint32_t i = (uint32_t)tid * 16u; i < code_bytes; i += 256u * 16u)
    st_nt(reinterpret_cast<u32x4_t*>(gcode + i), *reinterpret_cast<const u32x4_t*>(lcode + i));
  for (uint32_t i = (uint32_t)tid * 16u; i < hp_bytes; i += 256u * 16u)
    st_nt(reinterpret_cast<u32x4_t*>(ghp + i), *reinterpret_cast<const u32x4_t*>(lhp + i));
}

namespace {

template <int QB, int RND, int DELTA, int EPL>
hipError_t launch_mixed_t(const Args& a, hipStream_t s) {
  const uint64_t grid = (uint64_t)a.B * (uint64_t)a.H;
  hipLaunchKernelGGL((k_step_mixed<QB, RND, DELTA, EPL>), dim3((uint32_t)grid), dim3(256), a.mixed_lds, s, a);
  return hipGetLastError();
}

template <int QB, int RND, int DELTA>
hipError_t launch_mixed_dk(const Args& a, hipStream_t s) {
  switch (a.dk) {
    case 64: return launch_mixed_t<QB, RND, DELTA, 8>(a, s);
    case 128: return launch_mixed_t<QB, RND, DELTA, 16>(a, s);
    case 256: return launch_mixed_t<QB, RND, DELTA, 32>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

template <int QB, int RND>
hipError_t launch_mixed(int delta, const Args& a, hipStream_t s) {
  return delta ? launch_mixed_dk<QB, RND, 1>(a, s) : launch_mixed_dk<QB, RND, 0>(a, s);
}

}  // namespace qs
