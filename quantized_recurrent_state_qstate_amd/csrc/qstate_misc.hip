// libqstate kernels off the decode path (quantize, dequantize, fill) and the
// dispatch of the step launch to its qbits x rounding translation unit.
#include <cstdio>

#include "qstate_step_kernels.hpp"

namespace qs {

namespace {
__device__ __forceinline__ const uint8_t* code_block_m(const Args& a, uint32_t b, uint32_t h) {
  return a.codes + (uint64_t)b * a.code_bstride + a.t.code_off[h];
}
__device__ __forceinline__ const uint8_t* hp_block_m(const Args& a, uint32_t b, uint32_t h) {
  return a.hp + (uint64_t)b * a.hp_bstride + a.t.hp_off[h];
}
}  // namespace

// ---------------------------------------------------------------------------
// Quantize / dequantize: one thread per row, channels in order (any layout).
// Not on the decode path.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quantize(const Args a) {
  const uint64_t row = (uint64_t)blockIdx.x * 256u + threadIdx.x;
  const uint64_t nrows = (uint64_t)a.B * (uint64_t)a.H * (uint64_t)a.dv;
  if (row >= nrows) return;
  const int dk = a.dk;
  const uint64_t bh = row / (uint64_t)a.dv;
  const uint32_t v = (uint32_t)(row % (uint64_t)a.dv);
  const uint32_t h = (uint32_t)(bh % (uint64_t)a.H);
  const uint32_t b = (uint32_t)(bh / (uint64_t)a.H);
  const int nq = a.t.nq[h];
  const int nhp = dk - nq;
  const int hpb = hp_elem_bytes(a.hp_dtype);
  const uint32_t rq = code_row_bytes(nq, a.qbits);
  uint8_t* crow = const_cast<uint8_t*>(a.codes ? code_block_m(a, b, h) : nullptr);
  if (crow) crow += (uint64_t)v * rq;
  uint8_t* hrow = const_cast<uint8_t*>(a.hp ? hp_block_m(a, b, h) : nullptr);
  if (hrow) hrow += (uint64_t)v * hp_row_bytes(nhp, hpb);
  const uint16_t* sl = a.t.slots + (uint64_t)h * dk;
  const float* srow = a.S + row * (uint64_t)dk;
  float m = 0.0f;
  for (int k = 0; k < dk; ++k)
    if (!(sl[k] & kSlotProt)) m = fmaxf(m, fabsf(srow[k]));
  float scale, inv, invb;
  const int srb = a.rounding ? a.sr_bits : 0;
  if (a.bf16_layout) {   // bf16 scale rounded up, codes against it
    const float mq = m / (a.qbits == 8 ? 127.0f : 7.0f);
    if (a.qbits == 8) {
      if (srb == 16) row_scale_bf16<8, 16>(m, mq, scale, inv, invb);
      else if (srb == 8) row_scale_bf16<8, 8>(m, mq, scale, inv, invb);
      else row_scale_bf16<8, 0>(m, mq, scale, inv, invb);
    } else {
      if (srb == 16) row_scale_bf16<4, 16>(m, mq, scale, inv, invb);
      else if (srb == 8) row_scale_bf16<4, 8>(m, mq, scale, inv, invb);
      else row_scale_bf16<4, 0>(m, mq, scale, inv, invb);
    }
  } else if (a.qbits == 8) {
    if (srb == 16) row_scale<8, 16>(m, scale, inv, invb);
    else if (srb == 8) row_scale<8, 8>(m, scale, inv, invb);
    else row_scale<8, 0>(m, scale, inv, invb);
  } else {
    if (srb == 16) row_scale<4, 16>(m, scale, inv, invb);
    else if (srb == 8) row_scale<4, 8>(m, scale, inv, invb);
    else row_scale<4, 0>(m, scale, inv, invb);
  }
  uint64_t cached = ~(uint64_t)0;
  uint32_t x[4] = {0, 0, 0, 0};
  uint32_t pend = 0;
  for (int k = 0; k < dk; ++k) {
    const uint32_t s = sl[k] & 0x7FFFu;
    const float val = srow[k];
    if (sl[k] & kSlotProt) {
      if (a.hp_dtype == 0) reinterpret_cast<float*>(hrow)[s] = val;
      else reinterpret_cast<uint16_t*>(hrow)[s] =
          (uint16_t)((a.hp_dtype == 1) ? f32_to_bf16_bits(val) : f32_to_f16_bits(val));
      continue;
    }
    uint32_t rbits = 0;
    if (a.rounding) {
      const uint64_t e = row * (uint64_t)dk + (uint64_t)s;   // slot-indexed element
      const uint64_t g = (a.sr_bits == 16) ? (e >> 3) : (e >> 4);
      if (g != cached) {
        x[0] = (uint32_t)g;
        x[1] = (uint32_t)(g >> 32);
        x[2] = a.step_lo;
        x[3] = a.step_hi;
        philox10(x, a.seed_lo, a.seed_hi);
        cached = g;
      }
      rbits = (a.sr_bits == 16) ? ((e & 1u) ? (x[(e >> 1) & 3u] >> 16) : (x[(e >> 1) & 3u] & 0xFFFFu))
                                : ((x[(e >> 2) & 3u] >> (8u * (uint32_t)(e & 3u))) & 0xFFu);
    }
    int32_t c;
    if (a.qbits == 8) {
      c = !a.rounding ? round_elem<8, 0, 0>(val, 0.0f, inv, invb, 0u, 0.0f)
                      : (a.sr_bits == 16 ? round_elem<8, 1, 0>(val, 0.0f, inv, invb, rbits, 0.0f)
                                         : round_elem<8, 2, 0>(val, 0.0f, inv, invb, rbits, 0.0f));
      crow[s] = (uint8_t)c;
    } else {
      c = !a.rounding ? round_elem<4, 0, 0>(val, 0.0f, inv, invb, 0u, 0.0f)
                      : (a.sr_bits == 16 ? round_elem<4, 1, 0>(val, 0.0f, inv, invb, rbits, 0.0f)
                                         : round_elem<4, 2, 0>(val, 0.0f, inv, invb, rbits, 0.0f));
      if ((s & 1u) == 0u) {
        pend = (uint32_t)c & 0xFu;
        if ((int)s == nq - 1) crow[s >> 1] = (uint8_t)pend;
      } else {
        crow[s >> 1] = (uint8_t)(pend | (((uint32_t)c & 0xFu) << 4));
      }
    }
  }
  // Padding is part of the format (rows to 4 bytes, blocks to 16): written
  // as zeros, so a state quantized into memory of any prior content is the
  // same state (the key-map step reads whole dwords of a row).
  if (crow) {
    for (uint32_t i = ((uint32_t)nq * (uint32_t)a.qbits + 7u) / 8u; i < rq; ++i) crow[i] = 0u;
    if (v == (uint32_t)a.dv - 1u) {
      const uint32_t used = (uint32_t)a.dv * rq;
      for (uint32_t i = used; i < ((used + 15u) & ~15u); ++i) crow[i - v * rq] = 0u;
    }
  }
  if (hrow) {
    const uint32_t rh = hp_row_bytes(nhp, hpb);
    for (uint32_t i = (uint32_t)(nhp * hpb); i < rh; ++i) hrow[i] = 0u;
    if (v == (uint32_t)a.dv - 1u) {
      const uint32_t used = (uint32_t)a.dv * rh;
      for (uint32_t i = used; i < ((used + 15u) & ~15u); ++i) hrow[i - v * rh] = 0u;
    }
  }
  if (a.bf16_layout) reinterpret_cast<uint16_t*>(a.scales)[row] = (uint16_t)(__float_as_uint(scale) >> 16);
  else a.scales[row] = scale;
}

// Quantize with key-axis or per-head groups (map NONE): one workgroup per
// head; the groups' maxima through LDS, then one thread per row.
__global__ __launch_bounds__(256) void k_quantize_grouped(const Args a) {
  const int dk = a.dk, dv = a.dv;
  const uint64_t bh = blockIdx.x;
  const uint32_t h = (uint32_t)(bh % (uint64_t)a.H), b = (uint32_t)(bh / (uint64_t)a.H);
  const int G = a.scale_axis == 1 ? dk : 1;
  __shared__ uint32_t gmax[256];
  __shared__ float ginv[256], ginvb[256];
  const float* S = a.S + bh * (uint64_t)dv * (uint64_t)dk;
  for (int t = threadIdx.x; t < G; t += 256) gmax[t] = 0u;
  __syncthreads();
  for (int e = threadIdx.x; e < dv * dk; e += 256)
    atomicMax(&gmax[a.scale_axis == 1 ? e % dk : 0], __float_as_uint(fabsf(S[e])));
  __syncthreads();
  const int srb = a.rounding ? a.sr_bits : 0;
  for (int t = threadIdx.x; t < G; t += 256) {
    const float m = __uint_as_float(gmax[t]);
    float scale, inv, invb;
    if (a.qbits == 8) {
      if (srb == 16) row_scale<8, 16>(m, scale, inv, invb);
      else if (srb == 8) row_scale<8, 8>(m, scale, inv, invb);
      else row_scale<8, 0>(m, scale, inv, invb);
    } else {
      if (srb == 16) row_scale<4, 16>(m, scale, inv, invb);
      else if (srb == 8) row_scale<4, 8>(m, scale, inv, invb);
      else row_scale<4, 0>(m, scale, inv, invb);
    }
    ginv[t] = inv;
    ginvb[t] = invb;
    a.scales[bh * (uint64_t)G + t] = scale;
  }
  __syncthreads();
  uint8_t* cblk = const_cast<uint8_t*>(code_block_m(a, b, h));
  const uint32_t rq = code_row_bytes(dk, a.qbits);
  for (int v = threadIdx.x; v < dv; v += 256) {
    uint8_t* crow = cblk + (uint64_t)v * rq;
    const uint64_t row = bh * (uint64_t)dv + (uint64_t)v;
    uint64_t cached = ~(uint64_t)0;
    uint32_t x[4] = {0, 0, 0, 0};
    uint32_t pend = 0;
    for (int k = 0; k < dk; ++k) {
      const int g = a.scale_axis == 1 ? k : 0;
      const float val = S[(uint64_t)v * dk + k];
      uint32_t rbits = 0;
      if (a.rounding) {
        const uint64_t e = row * (uint64_t)dk + (uint64_t)k;
        const uint64_t gi = (a.sr_bits == 16) ? (e >> 3) : (e >> 4);
        if (gi != cached) {
          x[0] = (uint32_t)gi;
          x[1] = (uint32_t)(gi >> 32);
          x[2] = a.step_lo;
          x[3] = a.step_hi;
          philox10(x, a.seed_lo, a.seed_hi);
          cached = gi;
        }
        rbits = (a.sr_bits == 16) ? ((e & 1u) ? (x[(e >> 1) & 3u] >> 16) : (x[(e >> 1) & 3u] & 0xFFFFu))
                                  : ((x[(e >> 2) & 3u] >> (8u * (uint32_t)(e & 3u))) & 0xFFu);
      }
      const float inv = ginv[g], invb = ginvb[g];
      int32_t c;
      if (a.qbits == 8) {
        c = !a.rounding ? round_elem<8, 0, 0>(val, 0.0f, inv, invb, 0u, 0.0f)
                        : (a.sr_bits == 16 ? round_elem<8, 1, 0>(val, 0.0f, inv, invb, rbits, 0.0f)
                                           : round_elem<8, 2, 0>(val, 0.0f, inv, invb, rbits, 0.0f));
        crow[k] = (uint8_t)c;
      } else {
        c = !a.rounding ? round_elem<4, 0, 0>(val, 0.0f, inv, invb, 0u, 0.0f)
                        : (a.sr_bits == 16 ? round_elem<4, 1, 0>(val, 0.0f, inv, invb, rbits, 0.0f)
                                           : round_elem<4, 2, 0>(val, 0.0f, inv, invb, rbits, 0.0f));
        if ((k & 1) == 0) pend = (uint32_t)c & 0xFu;
        else crow[k >> 1] = (uint8_t)(pend | (((uint32_t)c & 0xFu) << 4));
      }
    }
  }
}

__global__ __launch_bounds__(256) void k_dequantize(const Args a) {
  const uint64_t row = (uint64_t)blockIdx.x * 256u + threadIdx.x;
  const uint64_t nrows = (uint64_t)a.B * (uint64_t)a.H * (uint64_t)a.dv;
  if (row >= nrows) return;
  const int dk = a.dk;
  const uint64_t bh = row / (uint64_t)a.dv;
  const uint32_t v = (uint32_t)(row % (uint64_t)a.dv);
  const uint32_t h = (uint32_t)(bh % (uint64_t)a.H);
  const uint32_t b = (uint32_t)(bh / (uint64_t)a.H);
  const int nq = a.t.nq[h];
  const int nhp = dk - nq;
  const int hpb = hp_elem_bytes(a.hp_dtype);
  const uint32_t rq = code_row_bytes(nq, a.qbits);
  const uint8_t* crow = a.codes ? code_block_m(a, b, h) + (uint64_t)v * rq : nullptr;
  const uint8_t* hrow = a.hp ? hp_block_m(a, b, h) + (uint64_t)v * hp_row_bytes(nhp, hpb) : nullptr;
  const uint16_t* sl = a.t.slots + (uint64_t)h * dk;
  const int bf = a.bf16_layout;
  // a scale or buffer element, fp32 or bf16
  auto ld = [bf](const float* base, uint64_t i) -> float {
    return bf ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[i]) : base[i];
  };
  // scale groups: the row (value axis), the key channel, or the head
  const int G = a.scale_axis == 0 ? a.dv : (a.scale_axis == 1 ? dk : 1);
  const float row_scale_v = a.scales && a.scale_axis == 0 ? ld(a.scales, row) : 0.0f;
  const int r = a.lrb_rank;
  const int n = r > 0 ? a.n[bh] : 0;
  const uint64_t w0 = (bh * (uint64_t)a.dv + v) * (uint64_t)r, u0 = bh * (uint64_t)dk * (uint64_t)r;
  float* orow = a.S_out + row * (uint64_t)dk;
  for (int k = 0; k < dk; ++k) {
    const uint32_t s = sl[k] & 0x7FFFu;
    float val;
    if (sl[k] & kSlotProt) {
      if (a.hp_dtype == 0) val = reinterpret_cast<const float*>(hrow)[s];
      else {
        const uint32_t bits = reinterpret_cast<const uint16_t*>(hrow)[s];
        val = (a.hp_dtype == 1) ? bf16_bits_to_f32(bits) : f16_bits_to_f32(bits);
      }
    } else {
      int32_t c;
      if (a.qbits == 8) c = (int32_t)(int8_t)crow[s];
      else c = (int32_t)((uint32_t)crow[s >> 1] << (28 - 4 * (s & 1))) >> 28;
      const float scale = a.scale_axis == 0 ? row_scale_v
                          : (a.scales ? ld(a.scales, bh * (uint64_t)G + (a.scale_axis == 1 ? (uint64_t)k : 0u)) : 0.0f);
      val = scale * (float)c;
    }
    if (n > 0) {
      float col = 0.0f;
      for (int j = 0; j < n; ++j) col = fmaf(ld(a.W, w0 + j), ld(a.U, u0 + (uint64_t)k * r + j), col);
      val = val + col;
    }
    orow[k] = val;
  }
}

__global__ __launch_bounds__(256) void k_zero(uint32_t* p, uint64_t nwords) {
  for (uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x; i < nwords; i += (uint64_t)gridDim.x * 256u)
    p[i] = 0u;
}
__global__ __launch_bounds__(256) void k_zero16(uint16_t* p, uint64_t n) {
  for (uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x; i < n; i += (uint64_t)gridDim.x * 256u)
    p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
namespace {
template <int QB, int RND>
hipError_t launch_step_qr(int family, int delta, const Args& a, hipStream_t s) {
  switch (family) {
    case kFamDense: return launch_dense<QB, RND>(delta, a, s);
    case kFamMixed: return launch_mixed<QB, RND>(delta, a, s);
    case kFamKeymap:
      switch (a.dk) {
        case 64: return launch_keymap<QB, RND, 64>(delta, a, s);
        case 128: return launch_keymap<QB, RND, 128>(delta, a, s);
        case 256: return launch_keymap<QB, RND, 256>(delta, a, s);
      }
      return hipErrorInvalidValue;
    case kFamLrb: return delta ? launch_lrb<QB, RND, 1>(a, s) : launch_lrb<QB, RND, 0>(a, s);
    case kFamGrouped: return launch_grouped<QB, RND>(delta, a, s);
  }
  return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_step(int family, int qbits, int rnd, int delta, const Args& a, hipStream_t s) {
  if (qbits == 8) {
    switch (rnd) {
      case 0: return launch_step_qr<8, 0>(family, delta, a, s);
      case 1: return launch_step_qr<8, 1>(family, delta, a, s);
      case 2: return launch_step_qr<8, 2>(family, delta, a, s);
    }
  } else {
    switch (rnd) {
      case 0: return launch_step_qr<4, 0>(family, delta, a, s);
      case 1: return launch_step_qr<4, 1>(family, delta, a, s);
      case 2: return launch_step_qr<4, 2>(family, delta, a, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_quantize(const Args& a, hipStream_t s) {
  const uint64_t nrows = (uint64_t)a.B * (uint64_t)a.H * (uint64_t)a.dv;
  if (nrows == 0) return hipSuccess;
  if (a.scale_axis != 0) {   // key-axis or per-head groups: one workgroup per head
    hipLaunchKernelGGL(k_quantize_grouped, dim3((uint32_t)((uint64_t)a.B * (uint64_t)a.H)), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_quantize, dim3((uint32_t)((nrows + 255u) / 256u)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.lrb_rank == 0) return e;
  const uint64_t bh = (uint64_t)a.B * (uint64_t)a.H;
  const uint64_t nW = bh * (uint64_t)a.dv * (uint64_t)a.lrb_rank;
  const uint64_t nU = bh * (uint64_t)a.dk * (uint64_t)a.lrb_rank;
  if (a.bf16_layout) {
    hipLaunchKernelGGL(k_zero16, dim3(1024), dim3(256), 0, s, reinterpret_cast<uint16_t*>(a.W), nW);
    hipLaunchKernelGGL(k_zero16, dim3(1024), dim3(256), 0, s, reinterpret_cast<uint16_t*>(a.U), nU);
  } else {
    hipLaunchKernelGGL(k_zero, dim3(1024), dim3(256), 0, s, reinterpret_cast<uint32_t*>(a.W), nW);
    hipLaunchKernelGGL(k_zero, dim3(1024), dim3(256), 0, s, reinterpret_cast<uint32_t*>(a.U), nU);
  }
  hipLaunchKernelGGL(k_zero, dim3(64), dim3(256), 0, s, reinterpret_cast<uint32_t*>(a.n), bh);
  return hipGetLastError();
}

hipError_t launch_dequantize(const Args& a, hipStream_t s) {
  const uint64_t nrows = (uint64_t)a.B * (uint64_t)a.H * (uint64_t)a.dv;
  if (nrows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_dequantize, dim3((uint32_t)((nrows + 255u) / 256u)), dim3(256), 0, s, a);
  return hipGetLastError();
}

const char* step_kernel_name(int family, int qbits, int rnd, int delta, int dk) {
  static thread_local char buf[96];
  const char* fam = family == kFamDense ? "dense"
                    : family == kFamMixed ? "mixed"
                    : family == kFamKeymap ? "keymap"
                    : family == kFamGrouped ? "grouped" : "lrb";
  const char* rn = rnd == 0 ? "rtn" : (rnd == 1 ? "sr16" : "sr8");
  snprintf(buf, sizeof(buf), "k_step_%s<int%d,%s,%s,dk%d>", fam, qbits, rn, delta ? "delta" : "additive", dk);
  return buf;
}

}  // namespace qs
