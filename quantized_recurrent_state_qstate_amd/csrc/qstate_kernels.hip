// gfx950 kernels of libqstate: the fused quantized-state decode step.
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
// head.
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
// (precision map NONE or HEAD).
// ---------------------------------------------------------------------------
template <int QB, int RND, int DELTA, int EPL>
__global__ __launch_bounds__(256) void k_step_dense(const Args a) {
  constexpr int DK = EPL * 8;
  const int lane8 = threadIdx.x & 7;
  const int rloc = threadIdx.x >> 3;
  const uint32_t wg = blockIdx.x;
  const uint32_t chunk = wg % (uint32_t)a.row_chunks;
  const uint32_t bh = wg / (uint32_t)a.row_chunks;
  const uint32_t h = bh % (uint32_t)a.H;
  const uint32_t b = bh / (uint32_t)a.H;
  const int v = (int)chunk * 32 + rloc;
  if (v >= a.dv) return;   // whole 8-lane groups leave together
  const int k0 = lane8 * EPL;
  const uint64_t row = (uint64_t)bh * (uint64_t)a.dv + (uint64_t)v;
  const bool quant = a.t.head_type[h] == kHeadQuant;

  float kf[EPL], df[EPL];
  load_in<EPL>(a.k, a.in_bf16, (uint64_t)bh * DK + k0, kf);
  load_decay<EPL>(a, bh, k0, df);
  const float beta = a.beta ? a.beta[bh] : 1.0f;
  const float vin = load_in1(a.v, a.in_bf16, row);

  // dequantize
  float sh[EPL];
  uint8_t* cp = nullptr;
  uint8_t* hpp = nullptr;
  if (quant) {
    cp = const_cast<uint8_t*>(code_block(a, b, h)) + (uint64_t)v * (DK * QB / 8) + k0 * QB / 8;
    load_codes<QB, EPL>(cp, a.scales[row], sh);
  } else {
    hpp = const_cast<uint8_t*>(hp_block(a, b, h)) +
          ((uint64_t)v * DK + (uint64_t)k0) * (uint64_t)hp_elem_bytes(a.hp_dtype);
    load_hp<EPL>(hpp, a.hp_dtype, sh);
  }

  // write vector u: beta v (additive) or beta (v - alpha S k) (delta rule)
  float u;
  if constexpr (DELTA) {
    float w = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) w = fmaf(sh[i], kf[i], w);
    w = sum8(w);
    u = beta * (vin - df[0] * w);
  } else {
    u = beta * vin;
  }

  // decay + update
  float sp[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) sp[i] = fmaf(u, kf[i], df[i] * sh[i]);

  // readout from the pre-rounding state
  float qf[EPL];
  load_in<EPL>(a.q, a.in_bf16, (uint64_t)bh * DK + k0, qf);
  float o = 0.0f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) o = fmaf(sp[i], qf[i], o);
  o = sum8(o);
  if (lane8 == 0) a.out[row] = o;

  // requantize
  if (quant) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) m = fmaxf(m, fabsf(sp[i]));
    m = max8(m);
    float scale, inv;
    row_scale<QB>(m, scale, inv);
    uint32_t rb[EPL];
    if constexpr (RND != 0) rand_bits<RND, EPL>(row * DK + (uint64_t)k0, a.seed_lo, a.seed_hi, a.step_lo, a.step_hi, rb);
    int32_t code[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      code[i] = round_elem<QB, RND>(sp[i], sh[i], inv, (RND != 0) ? rb[i] : 0u, a.bdr, a.bdr_bound);
    store_codes<QB, EPL>(cp, code);
    if (lane8 == 0) a.scales[row] = scale;
  } else {
    store_hp<EPL>(hpp, a.hp_dtype, sp);
  }
}

// ---------------------------------------------------------------------------
// Mixed step (precision map KEY): a row holds quantized and protected key
// channels in two packed areas.  The head's code and protected blocks are
// staged through LDS with 128-bit accesses; each lane gathers its logical
// channels by slot, computes as the dense kernel, scatters back, and the
// workgroup writes the blocks out.  One workgroup per head.
// ---------------------------------------------------------------------------
template <int QB, int RND, int DELTA, int EPL>
__global__ __launch_bounds__(256) void k_step_mixed(const Args a) {
  constexpr int DK = EPL * 8;
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane8 = tid & 7;
  const int rloc = tid >> 3;
  const uint32_t bh = blockIdx.x;
  const uint32_t h = bh % (uint32_t)a.H;
  const uint32_t b = bh / (uint32_t)a.H;
  const int nq = a.t.nq[h];
  const int nhp = DK - nq;
  const int hpb = hp_elem_bytes(a.hp_dtype);
  const uint32_t rq = (uint32_t)(nq * QB + 7) / 8u;
  const uint32_t code_bytes = ((uint32_t)a.dv * rq + 15u) & ~15u;
  const uint32_t hp_bytes = ((uint32_t)a.dv * (uint32_t)nhp * (uint32_t)hpb + 15u) & ~15u;
  uint8_t* gcode = const_cast<uint8_t*>(code_block(a, b, h));
  uint8_t* ghp = const_cast<uint8_t*>(hp_block(a, b, h));
  uint8_t* lcode = lds;
  uint8_t* lhp = lds + code_bytes;

  for (uint32_t i = (uint32_t)tid * 16u; i < code_bytes; i += 256u * 16u)
    *reinterpret_cast<uint4*>(lcode + i) = *reinterpret_cast<const uint4*>(gcode + i);
  for (uint32_t i = (uint32_t)tid * 16u; i < hp_bytes; i += 256u * 16u)
    *reinterpret_cast<uint4*>(lhp + i) = *reinterpret_cast<const uint4*>(ghp + i);

  const int k0 = lane8 * EPL;
  uint16_t sl[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) sl[i] = a.t.slots[(uint64_t)h * DK + k0 + i];
  float kf[EPL], df[EPL], qf[EPL];
  load_in<EPL>(a.k, a.in_bf16, (uint64_t)bh * DK + k0, kf);
  load_in<EPL>(a.q, a.in_bf16, (uint64_t)bh * DK + k0, qf);
  load_decay<EPL>(a, bh, k0, df);
  const float beta = a.beta ? a.beta[bh] : 1.0f;
  __syncthreads();

  for (int v = rloc; v < a.dv; v += 32) {
    const uint64_t row = (uint64_t)bh * (uint64_t)a.dv + (uint64_t)v;
    const float s_old = a.scales[row];
    const float vin = load_in1(a.v, a.in_bf16, row);
    uint8_t* crow = lcode + (uint32_t)v * rq;
    uint8_t* hrow = lhp + (uint32_t)v * (uint32_t)nhp * (uint32_t)hpb;
    float sh[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const uint32_t s = sl[i] & 0x7FFFu;
      if (sl[i] & kSlotProt) {
        if (a.hp_dtype == 0) sh[i] = *reinterpret_cast<const float*>(hrow + s * 4u);
        else {
          const uint32_t bits = *reinterpret_cast<const uint16_t*>(hrow + s * 2u);
          sh[i] = (a.hp_dtype == 1) ? bf16_bits_to_f32(bits) : f16_bits_to_f32(bits);
        }
      } else {
        int32_t c;
        if constexpr (QB == 8) c = (int32_t)(int8_t)crow[s];
        else c = (int32_t)((uint32_t)crow[s >> 1] << (28 - 4 * (s & 1))) >> 28;
        sh[i] = s_old * (float)c;
      }
    }
    float u;
    if constexpr (DELTA) {
      float w = 0.0f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) w = fmaf(sh[i], kf[i], w);
      w = sum8(w);
      u = beta * (vin - df[0] * w);
    } else {
      u = beta * vin;
    }
    float sp[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) sp[i] = fmaf(u, kf[i], df[i] * sh[i]);
    float o = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) o = fmaf(sp[i], qf[i], o);
    o = sum8(o);
    if (lane8 == 0) a.out[row] = o;

    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (!(sl[i] & kSlotProt)) m = fmaxf(m, fabsf(sp[i]));
    m = max8(m);
    float scale, inv;
    row_scale<QB>(m, scale, inv);
    uint32_t rb[EPL];
    if constexpr (RND != 0) rand_bits<RND, EPL>(row * DK + (uint64_t)k0, a.seed_lo, a.seed_hi, a.step_lo, a.step_hi, rb);
    int32_t code[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      code[i] = round_elem<QB, RND>(sp[i], sh[i], inv, (RND != 0) ? rb[i] : 0u, a.bdr, a.bdr_bound);

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
    if (lane8 == 0) a.scales[row] = scale;
  }
  __syncthreads();
  for (uint32_t i = (uint32_t)tid * 16u; i < code_bytes; i += 256u * 16u)
    *reinterpret_cast<uint4*>(gcode + i) = *reinterpret_cast<const uint4*>(lcode + i);
  for (uint32_t i = (uint32_t)tid * 16u; i < hp_bytes; i += 256u * 16u)
    *reinterpret_cast<uint4*>(ghp + i) = *reinterpret_cast<const uint4*>(lhp + i);
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
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
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
__device__ __forceinline__ float block_max(float x, float* red) {
  x = wave_max(x);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
__device__ __forceinline__ int block_or(int x, float* red) {
  x = __any(x) ? 1 : 0;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = (float)x;
  __syncthreads();
  return (red[0] + red[1] + red[2] + red[3]) > 0.0f;
}
}  // namespace

// ---------------------------------------------------------------------------
// Step with Low-Rank Bypass (additive recurrences, map NONE).  One
// workgroup per head.  Phase A keeps the head's buffer (W [dv][r], U
// [dk][r]) in LDS: decay U with the state, grow the orthonormal value basis
// from the write vector while fewer than r columns exist, split u into its
// in-span coefficients c and remainder u_perp, send c k_k into U for key
// channels whose update is under theta LSB in every row, and on a merge step
// flag buffer channels that reach theta LSB somewhere.  Phase B is the dense
// row step with u_perp on small channels and the flagged buffer columns
// added before rounding; the readout adds W (U^T q).
// ---------------------------------------------------------------------------
template <int QB, int RND, int EPL>
__global__ __launch_bounds__(256) void k_step_lrb(const Args a) {
  constexpr int DK = EPL * 8;
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x;
  const int dv = a.dv;
  const int r = a.lrb_rank;
  const uint32_t bh = blockIdx.x;
  const uint32_t h = bh % (uint32_t)a.H;
  const uint32_t b = bh / (uint32_t)a.H;
  const float theta = a.lrb_theta;

  float* Wl = reinterpret_cast<float*>(lds);           // [dv][r]
  float* Ul = Wl + dv * r;                              // [DK][r]
  float* ul = Ul + DK * r;                              // [dv]
  float* upl = ul + dv;                                 // [dv]
  float* sol = upl + dv;                                // [dv] scales on entry
  float* lrl = sol + dv;                                // [dv] buffer readout
  float* kl = lrl + dv;                                 // [DK]
  float* ql = kl + DK;                                  // [DK]
  float* dl = ql + DK;                                  // [DK]
  float* cl = dl + DK;                                  // [16]
  float* zl = cl + 16;                                  // [16]
  float* red = zl + 16;                                 // [4]
  uint8_t* small = reinterpret_cast<uint8_t*>(red + 4); // [DK]
  uint8_t* mflag = small + DK;                          // [DK]

  float* Wg = a.W + (uint64_t)bh * (uint64_t)dv * (uint64_t)r;
  float* Ug = a.U + (uint64_t)bh * (uint64_t)DK * (uint64_t)r;
  const float beta = a.beta ? a.beta[bh] : 1.0f;
  int n = a.n[bh];

  if (tid < dv) {
    const uint64_t row = (uint64_t)bh * (uint64_t)dv + (uint64_t)tid;
    ul[tid] = beta * load_in1(a.v, a.in_bf16, row);
    sol[tid] = a.scales[row];
  }
  if (tid < DK) {
    kl[tid] = load_in1(a.k, a.in_bf16, (uint64_t)bh * DK + tid);
    ql[tid] = load_in1(a.q, a.in_bf16, (uint64_t)bh * DK + tid);
    dl[tid] = a.decay_key ? a.decay[(uint64_t)bh * DK + tid] : a.decay[bh];
  }
  for (int i = tid; i < dv * r; i += 256) Wl[i] = Wg[i];
  for (int i = tid; i < DK * r; i += 256) Ul[i] = Ug[i];
  __syncthreads();

  // 1. the buffer decays with the state (decay acts on the key side)
  for (int i = tid; i < DK * r; i += 256) Ul[i] = dl[i / r] * Ul[i];

  // 2. grow the basis (two Gram-Schmidt passes)
  bool grown = false;
  if (n < r) {
    float y = (tid < dv) ? ul[tid] : 0.0f;
    for (int pass = 0; pass < 2; ++pass)
      for (int j = 0; j < n; ++j) {
        const float wv = (tid < dv) ? Wl[tid * r + j] : 0.0f;
        const float p = block_sum(wv * y, red);
        if (tid < dv) y = fmaf(-p, wv, y);
      }
    const float ny = sqrtf(block_sum(y * y, red));
    const float uu = (tid < dv) ? ul[tid] : 0.0f;
    const float nu = sqrtf(block_sum(uu * uu, red));
    if (ny > ldexpf(nu, -10)) {
      if (tid < dv) Wl[tid * r + n] = y / ny;
      n += 1;
      grown = true;
    }
  }
  __syncthreads();

  // 3. project the write vector on the basis
  for (int j = 0; j < n; ++j) {
    const float c = block_sum((tid < dv) ? Wl[tid * r + j] * ul[tid] : 0.0f, red);
    if (tid == 0) cl[j] = c;
  }
  __syncthreads();
  float gv = 0.0f;
  if (tid < dv) {
    float t = ul[tid];
    for (int j = 0; j < n; ++j) t = fmaf(-cl[j], Wl[tid * r + j], t);
    upl[tid] = t;
    const float au = fabsf(ul[tid]);
    gv = (sol[tid] > 0.0f) ? au / sol[tid] : (au > 0.0f ? __builtin_inff() : 0.0f);
  }
  // 4. small key channels go to the buffer
  const float g = block_max(gv, red);
  if (tid < DK) {
    const bool sm = __builtin_isfinite(g) && (fabsf(kl[tid]) * g < theta);
    small[tid] = sm ? 1 : 0;
    if (sm)
      for (int j = 0; j < n; ++j) Ul[tid * r + j] = fmaf(kl[tid], cl[j], Ul[tid * r + j]);
    mflag[tid] = 0;
  }
  __syncthreads();

  // 5. merge
  int n_new = n;
  const uint64_t step = ((uint64_t)a.step_hi << 32) | a.step_lo;
  if (a.lrb_period > 0 && ((step + 1u) % (uint64_t)a.lrb_period) == 0u) {
    int left = 0;
    if (tid < DK) {
      int big = 0;
      for (int v = 0; v < dv; ++v) {
        float col = 0.0f;
        for (int j = 0; j < n; ++j) col = fmaf(Wl[v * r + j], Ul[tid * r + j], col);
        if (col != 0.0f && fabsf(col) >= theta * sol[v]) big = 1;
      }
      mflag[tid] = (uint8_t)big;
      if (!big)
        for (int j = 0; j < r; ++j)
          if (Ul[tid * r + j] != 0.0f) left = 1;
    }
    if (!block_or(left, red)) n_new = 0;
  }
  __syncthreads();

  // 6. buffer readout term z = U^T q over unmerged channels; lr = W z
  for (int j = 0; j < n; ++j) {
    const float zj = block_sum((tid < DK && !mflag[tid]) ? Ul[tid * r + j] * ql[tid] : 0.0f, red);
    if (tid == 0) zl[j] = zj;
  }
  __syncthreads();
  if (tid < dv) {
    float acc = 0.0f;
    for (int j = 0; j < n; ++j) acc = fmaf(Wl[tid * r + j], zl[j], acc);
    lrl[tid] = acc;
  }
  // write the buffer back
  for (int i = tid; i < DK * r; i += 256) Ug[i] = mflag[i / r] ? 0.0f : Ul[i];
  if (grown)
    for (int i = tid; i < dv * r; i += 256) Wg[i] = Wl[i];
  if (tid == 0) a.n[bh] = n_new;
  __syncthreads();

  // Phase B: rows
  const int lane8 = tid & 7;
  const int rloc = tid >> 3;
  const int k0 = lane8 * EPL;
  float kf[EPL], df[EPL], qf[EPL];
  bool smf[EPL], mgf[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    kf[i] = kl[k0 + i];
    df[i] = dl[k0 + i];
    qf[i] = ql[k0 + i];
    smf[i] = small[k0 + i] != 0;
    mgf[i] = mflag[k0 + i] != 0;
  }
  uint8_t* gcode = const_cast<uint8_t*>(code_block(a, b, h));
  for (int v = rloc; v < dv; v += 32) {
    const uint64_t row = (uint64_t)bh * (uint64_t)dv + (uint64_t)v;
    uint8_t* cp = gcode + (uint64_t)v * (DK * QB / 8) + k0 * QB / 8;
    float sh[EPL];
    load_codes<QB, EPL>(cp, sol[v], sh);
    const float uv = ul[v], upv = upl[v];
    float sp[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      float x = fmaf(smf[i] ? upv : uv, kf[i], df[i] * sh[i]);
      if (mgf[i]) {
        float col = 0.0f;
        for (int j = 0; j < n; ++j) col = fmaf(Wl[v * r + j], Ul[(k0 + i) * r + j], col);
        x = x + col;
      }
      sp[i] = x;
    }
    float o = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) o = fmaf(sp[i], qf[i], o);
    o = sum8(o);
    if (lane8 == 0) a.out[row] = o + lrl[v];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) m = fmaxf(m, fabsf(sp[i]));
    m = max8(m);
    float scale, inv;
    row_scale<QB>(m, scale, inv);
    uint32_t rb[EPL];
    if constexpr (RND != 0) rand_bits<RND, EPL>(row * DK + (uint64_t)k0, a.seed_lo, a.seed_hi, a.step_lo, a.step_hi, rb);
    int32_t code[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      code[i] = round_elem<QB, RND>(sp[i], sh[i], inv, (RND != 0) ? rb[i] : 0u, a.bdr, a.bdr_bound);
    store_codes<QB, EPL>(cp, code);
    if (lane8 == 0) a.scales[row] = scale;
  }
}

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
  const uint32_t rq = (uint32_t)(nq * a.qbits + 7) / 8u;
  uint8_t* crow = const_cast<uint8_t*>(a.codes ? code_block(a, b, h) : nullptr);
  if (crow) crow += (uint64_t)v * rq;
  uint8_t* hrow = const_cast<uint8_t*>(a.hp ? hp_block(a, b, h) : nullptr);
  if (hrow) hrow += (uint64_t)v * (uint64_t)nhp * (uint64_t)hpb;
  const uint16_t* sl = a.t.slots + (uint64_t)h * dk;
  const float* srow = a.S + row * (uint64_t)dk;
  float m = 0.0f;
  for (int k = 0; k < dk; ++k)
    if (!(sl[k] & kSlotProt)) m = fmaxf(m, fabsf(srow[k]));
  float scale, inv;
  if (a.qbits == 8) row_scale<8>(m, scale, inv);
  else row_scale<4>(m, scale, inv);
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
      const uint64_t e = row * (uint64_t)dk + (uint64_t)k;
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
      c = !a.rounding ? round_elem<8, 0>(val, 0.0f, inv, 0u, 0, 0.0f)
                      : (a.sr_bits == 16 ? round_elem<8, 1>(val, 0.0f, inv, rbits, 0, 0.0f)
                                         : round_elem<8, 2>(val, 0.0f, inv, rbits, 0, 0.0f));
      crow[s] = (uint8_t)c;
    } else {
      c = !a.rounding ? round_elem<4, 0>(val, 0.0f, inv, 0u, 0, 0.0f)
                      : (a.sr_bits == 16 ? round_elem<4, 1>(val, 0.0f, inv, rbits, 0, 0.0f)
                                         : round_elem<4, 2>(val, 0.0f, inv, rbits, 0, 0.0f));
      if ((s & 1u) == 0u) {
        pend = (uint32_t)c & 0xFu;
        if ((int)s == nq - 1) crow[s >> 1] = (uint8_t)pend;
      } else {
        crow[s >> 1] = (uint8_t)(pend | (((uint32_t)c & 0xFu) << 4));
      }
    }
  }
  a.scales[row] = scale;
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
  const uint32_t rq = (uint32_t)(nq * a.qbits + 7) / 8u;
  const uint8_t* crow = a.codes ? code_block(a, b, h) + (uint64_t)v * rq : nullptr;
  const uint8_t* hrow = a.hp ? hp_block(a, b, h) + (uint64_t)v * (uint64_t)nhp * (uint64_t)hpb : nullptr;
  const uint16_t* sl = a.t.slots + (uint64_t)h * dk;
  const float scale = a.scales ? a.scales[row] : 0.0f;
  const int r = a.lrb_rank;
  const int n = r > 0 ? a.n[bh] : 0;
  const float* W = r > 0 ? a.W + (bh * (uint64_t)a.dv + v) * (uint64_t)r : nullptr;
  const float* U = r > 0 ? a.U + bh * (uint64_t)dk * (uint64_t)r : nullptr;
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
      val = scale * (float)c;
    }
    if (n > 0) {
      float col = 0.0f;
      for (int j = 0; j < n; ++j) col = fmaf(W[j], U[(uint64_t)k * r + j], col);
      val = val + col;
    }
    orow[k] = val;
  }
}

__global__ __launch_bounds__(256) void k_zero(uint32_t* p, uint64_t nwords) {
  for (uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x; i < nwords; i += (uint64_t)gridDim.x * 256u)
    p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
namespace {

template <int QB, int RND, int DELTA, int EPL>
hipError_t launch_dense_t(const Args& a, hipStream_t s) {
  const uint64_t grid = (uint64_t)a.B * (uint64_t)a.H * (uint64_t)a.row_chunks;
  hipLaunchKernelGGL((k_step_dense<QB, RND, DELTA, EPL>), dim3((uint32_t)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int QB, int RND, int DELTA, int EPL>
hipError_t launch_mixed_t(const Args& a, hipStream_t s) {
  const uint64_t grid = (uint64_t)a.B * (uint64_t)a.H;
  hipLaunchKernelGGL((k_step_mixed<QB, RND, DELTA, EPL>), dim3((uint32_t)grid), dim3(256), a.mixed_lds, s, a);
  return hipGetLastError();
}

template <int QB, int RND, int EPL>
hipError_t launch_lrb_t(const Args& a, hipStream_t s) {
  const uint64_t grid = (uint64_t)a.B * (uint64_t)a.H;
  hipLaunchKernelGGL((k_step_lrb<QB, RND, EPL>), dim3((uint32_t)grid), dim3(256), a.mixed_lds, s, a);
  return hipGetLastError();
}

template <int QB, int RND, int DELTA>
hipError_t launch_fam(int family, const Args& a, hipStream_t s) {
  if (family == kFamDense) {
    switch (a.dk) {
      case 64: return launch_dense_t<QB, RND, DELTA, 8>(a, s);
      case 128: return launch_dense_t<QB, RND, DELTA, 16>(a, s);
      case 256: return launch_dense_t<QB, RND, DELTA, 32>(a, s);
    }
  } else if (family == kFamMixed) {
    switch (a.dk) {
      case 64: return launch_mixed_t<QB, RND, DELTA, 8>(a, s);
      case 128: return launch_mixed_t<QB, RND, DELTA, 16>(a, s);
      case 256: return launch_mixed_t<QB, RND, DELTA, 32>(a, s);
    }
  } else if (family == kFamLrb && !DELTA) {
    switch (a.dk) {
      case 64: return launch_lrb_t<QB, RND, 8>(a, s);
      case 128: return launch_lrb_t<QB, RND, 16>(a, s);
      case 256: return launch_lrb_t<QB, RND, 32>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

template <int QB, int RND>
hipError_t launch_kind(int family, int delta, const Args& a, hipStream_t s) {
  return delta ? launch_fam<QB, RND, 1>(family, a, s) : launch_fam<QB, RND, 0>(family, a, s);
}

template <int QB>
hipError_t launch_rnd(int family, int rnd, int delta, const Args& a, hipStream_t s) {
  switch (rnd) {
    case 0: return launch_kind<QB, 0>(family, delta, a, s);
    case 1: return launch_kind<QB, 1>(family, delta, a, s);
    case 2: return launch_kind<QB, 2>(family, delta, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_step(int family, int qbits, int rnd, int delta, const Args& a, hipStream_t s) {
  return qbits == 8 ? launch_rnd<8>(family, rnd, delta, a, s) : launch_rnd<4>(family, rnd, delta, a, s);
}

hipError_t launch_quantize(const Args& a, hipStream_t s) {
  const uint64_t nrows = (uint64_t)a.B * (uint64_t)a.H * (uint64_t)a.dv;
  if (nrows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_quantize, dim3((uint32_t)((nrows + 255u) / 256u)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.lrb_rank == 0) return e;
  const uint64_t bh = (uint64_t)a.B * (uint64_t)a.H;
  const uint64_t nW = bh * (uint64_t)a.dv * (uint64_t)a.lrb_rank;
  const uint64_t nU = bh * (uint64_t)a.dk * (uint64_t)a.lrb_rank;
  hipLaunchKernelGGL(k_zero, dim3(1024), dim3(256), 0, s, reinterpret_cast<uint32_t*>(a.W), nW);
  hipLaunchKernelGGL(k_zero, dim3(1024), dim3(256), 0, s, reinterpret_cast<uint32_t*>(a.U), nU);
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
  const char* fam = family == kFamDense ? "dense" : (family == kFamMixed ? "mixed" : "lrb");
  const char* rn = rnd == 0 ? "rtn" : (rnd == 1 ? "sr16" : "sr8");
  snprintf(buf, sizeof(buf), "k_step_%s<int%d,%s,%s,dk%d>", fam, qbits, rn, delta ? "delta" : "additive", dk);
  return buf;
}

}  // namespace qs
