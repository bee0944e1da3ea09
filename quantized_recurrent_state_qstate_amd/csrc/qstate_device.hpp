// Device helpers of libqstate's gfx950 kernels: Philox4x32-10, 8-lane DPP
// reductions, vector loads/stores, 16-bit conversions, element rounding.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qs {

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon et al., SC'11, Philox family): ten rounds, each
// multiplying counter words 0 and 2 by the two Philox multipliers; the high
// product halves are xored with the other counter words and the round key,
// the low halves move into words 1 and 3; the key advances by the two Weyl
// constants after every round.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void philox10(uint32_t (&x)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)x[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)x[2];
    // three-input xor in one v_bitop3_b32 (truth table 0x96 = a ^ b ^ c)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), x[1], k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), x[3], k1, 0x96);
    x[1] = (uint32_t)p1;
    x[3] = (uint32_t)p0;
    x[0] = n0;
    x[2] = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

// Random integers for EPL consecutive elements starting at element index e0
// (e0 a multiple of 8).  RND 1: 16 bits per element, block g = e>>3, low
// half of word (e>>1)&3 for even e.  RND 2: 8 bits, block g = e>>4, byte
// e&3 of word (e>>2)&3.  Counter = (g lo, g hi, step lo, step hi); element
// indices stay below 2^35 (checked at init), so g hi is 0.
template <int RND, int EPL>
__device__ __forceinline__ void rand_bits(uint64_t e0, uint32_t s0, uint32_t s1, uint32_t t0,
                                          uint32_t t1, uint32_t (&rb)[EPL]) {
  if constexpr (RND == 1) {
#pragma unroll
    for (int g = 0; g < EPL / 8; ++g) {
      const uint32_t n = (uint32_t)(e0 >> 3) + (uint32_t)g;
      uint32_t x[4] = {n, 0u, t0, t1};
      philox10(x, s0, s1);
#pragma unroll
      for (int j = 0; j < 8; ++j) rb[g * 8 + j] = (j & 1) ? (x[j >> 1] >> 16) : (x[j >> 1] & 0xFFFFu);
    }
  } else if constexpr (RND == 2) {
    if constexpr (EPL >= 16) {
#pragma unroll
      for (int g = 0; g < EPL / 16; ++g) {
        const uint32_t n = (uint32_t)(e0 >> 4) + (uint32_t)g;
        uint32_t x[4] = {n, 0u, t0, t1};
        philox10(x, s0, s1);
#pragma unroll
        for (int j = 0; j < 16; ++j) rb[g * 16 + j] = (x[j >> 2] >> (8 * (j & 3))) & 0xFFu;
      }
    } else {
      const uint32_t n = (uint32_t)(e0 >> 4);
      uint32_t x[4] = {n, 0u, t0, t1};
      philox10(x, s0, s1);
      const bool hi = (e0 & 8u) != 0;   // second half of the 16-element block
      const uint32_t w0 = hi ? x[2] : x[0];
      const uint32_t w1 = hi ? x[3] : x[1];
#pragma unroll
      for (int j = 0; j < EPL; ++j) rb[j] = (((j < 4) ? w0 : w1) >> (8 * (j & 3))) & 0xFFu;
    }
  }
}

// Random integer of one element e (same mapping as rand_bits), one Philox
// block per call.
template <int RND>
__device__ __forceinline__ uint32_t rand_one(uint64_t e, uint32_t s0, uint32_t s1, uint32_t t0, uint32_t t1) {
  if constexpr (RND == 1) {
    uint32_t x[4] = {(uint32_t)(e >> 3), 0u, t0, t1};
    philox10(x, s0, s1);
    const uint32_t w = x[(e >> 1) & 3u];
    return (e & 1u) ? (w >> 16) : (w & 0xFFFFu);
  } else {
    uint32_t x[4] = {(uint32_t)(e >> 4), 0u, t0, t1};
    philox10(x, s0, s1);
    return (x[(e >> 2) & 3u] >> (8u * (uint32_t)(e & 3u))) & 0xFFu;
  }
}

// ---------------------------------------------------------------------------
// Reductions over the 8 lanes of a row group (lanes 8i..8i+7) with DPP:
// swap neighbours, swap pairs, mirror the half-row.  Every lane ends with
// the same bits (each step combines two equal multisets commutatively).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dppf(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror

__device__ __forceinline__ float sum8(float x) {
  x = x + dppf<kDppXor1>(x);
  x = x + dppf<kDppXor2>(x);
  x = x + dppf<kDppHalfMirror>(x);
  return x;
}
__device__ __forceinline__ float max8(float x) {
  x = fmaxf(x, dppf<kDppXor1>(x));
  x = fmaxf(x, dppf<kDppXor2>(x));
  x = fmaxf(x, dppf<kDppHalfMirror>(x));
  return x;
}

// The same reductions over a group of L = 4 or 8 lanes (4: the two quad
// steps only).
template <int L>
__device__ __forceinline__ float red_sum(float x) {
  static_assert(L == 4 || L == 8, "row groups of 4 or 8 lanes");
  x = x + dppf<kDppXor1>(x);
  x = x + dppf<kDppXor2>(x);
  if constexpr (L == 8) x = x + dppf<kDppHalfMirror>(x);
  return x;
}

// Maximum of non-negative floats over the row group, on their bit patterns
// (for x >= 0 the unsigned order of the bits is the numeric order), so each
// step is one v_max_u32 with a DPP operand.
template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float absmax8(float x) {
  uint32_t u = __float_as_uint(x);
  u = max(u, dppu<kDppXor1>(u));
  u = max(u, dppu<kDppXor2>(u));
  u = max(u, dppu<kDppHalfMirror>(u));
  return __uint_as_float(u);
}
template <int L>
__device__ __forceinline__ float red_absmax(float x) {
  static_assert(L == 4 || L == 8, "row groups of 4 or 8 lanes");
  uint32_t u = __float_as_uint(x);
  u = max(u, dppu<kDppXor1>(u));
  u = max(u, dppu<kDppXor2>(u));
  if constexpr (L == 8) u = max(u, dppu<kDppHalfMirror>(u));
  return __uint_as_float(u);
}

// Stored row strides: the codes of nq quantized channels and the values of
// nhp protected ones (hpb bytes each), each row padded to 4 bytes.
__device__ __forceinline__ uint32_t code_row_bytes(int nq, int qbits) {
  return (((uint32_t)(nq * qbits + 7) / 8u) + 3u) & ~3u;
}
__device__ __forceinline__ uint32_t hp_row_bytes(int nhp, int hpb) { return ((uint32_t)(nhp * hpb) + 3u) & ~3u; }

// ---------------------------------------------------------------------------
// Vector memory access of N bytes (N = 4, 8 or a multiple of 16; p aligned).
// NT = nontemporal: the stored state is streamed once per step, so its loads
// and stores carry the streaming hint (no reuse expected in the caches).
// ---------------------------------------------------------------------------
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ T ld_nt(const T* p) { return __builtin_nontemporal_load(p); }
template <typename T>
__device__ __forceinline__ void st_nt(T* p, T v) { __builtin_nontemporal_store(v, p); }

template <int N, bool NT = false>
__device__ __forceinline__ void load_bytes(const uint8_t* p, uint32_t (&w)[N / 4]) {
  if constexpr (N == 4) {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
    w[0] = NT ? ld_nt(q) : *q;
  } else if constexpr (N == 8) {
    const u32x2_t* q = reinterpret_cast<const u32x2_t*>(p);
    const u32x2_t t = NT ? ld_nt(q) : *q;
    w[0] = t.x;
    w[1] = t.y;
  } else {
#pragma unroll
    for (int i = 0; i < N / 16; ++i) {
      const u32x4_t* q = reinterpret_cast<const u32x4_t*>(p) + i;
      const u32x4_t t = NT ? ld_nt(q) : *q;
      w[4 * i + 0] = t.x;
      w[4 * i + 1] = t.y;
      w[4 * i + 2] = t.z;
      w[4 * i + 3] = t.w;
    }
  }
}

template <int N, bool NT = false>
__device__ __forceinline__ void store_bytes(uint8_t* p, const uint32_t (&w)[N / 4]) {
  if constexpr (N == 4) {
    uint32_t* q = reinterpret_cast<uint32_t*>(p);
    if constexpr (NT) st_nt(q, w[0]); else *q = w[0];
  } else if constexpr (N == 8) {
    u32x2_t* q = reinterpret_cast<u32x2_t*>(p);
    const u32x2_t t = {w[0], w[1]};
    if constexpr (NT) st_nt(q, t); else *q = t;
  } else {
#pragma unroll
    for (int i = 0; i < N / 16; ++i) {
      u32x4_t* q = reinterpret_cast<u32x4_t*>(p) + i;
      const u32x4_t t = {w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
      if constexpr (NT) st_nt(q, t); else *q = t;
    }
  }
}

// ---------------------------------------------------------------------------
// 16-bit formats.  bf16: round to nearest even on the fp32 bit pattern (add
// 0x7FFF plus the lowest kept bit), NaN -> quiet NaN.  fp16: the hardware
// conversion (round to nearest even, subnormals kept).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) & 0x8000u) | 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values to a packed bf16 pair (round to nearest even), one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// fp32 -> fp16 bits with one v_cvt_f16_f32 (nearest even, subnormals kept).
// Written as asm so that the compiler cannot fuse the fma that produced f
// into a mixed-precision fma, which rounds once straight to fp16 instead of
// to fp32 and then to fp16.
__device__ __forceinline__ uint32_t cvt_f16_raw(float f) {
  uint32_t r;
  asm("v_cvt_f16_f32 %0, %1" : "=v"(r) : "v"(f));
  return r;
}
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) { return cvt_f16_raw(f) & 0xFFFFu; }
// Two values packed, lo in the low half.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_amdgcn_perm(cvt_f16_raw(hi), cvt_f16_raw(lo), 0x05040100u);
}

// Scalar input element (bf16 or fp32).
__device__ __forceinline__ float load_in1(const void* base, int bf16, uint64_t idx) {
  if (bf16) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
  return reinterpret_cast<const float*>(base)[idx];
}

// One input element (bf16 or fp32 by a runtime flag) read with no branch:
// the 16-bit word at element idx (inside the array either way) and the
// 32-bit word at element idx, or at element 0 for bf16 input (so it stays
// inside the array); in_raw_value picks and widens, once the loads landed.
struct InRaw {
  uint16_t h;
  uint32_t w;
};
__device__ __forceinline__ InRaw in_raw_load(const void* base, int bf16, uint64_t idx) {
  InRaw r;
  r.h = reinterpret_cast<const uint16_t*>(base)[idx];
  r.w = reinterpret_cast<const uint32_t*>(base)[bf16 ? 0 : idx];
  return r;
}
__device__ __forceinline__ float in_raw_value(const InRaw& r, int bf16) {
  return bf16 ? bf16_bits_to_f32(r.h) : __uint_as_float(r.w);
}

// EPL consecutive input elements (bf16 or fp32) starting at element idx.
template <int EPL>
__device__ __forceinline__ void load_in(const void* base, int bf16, uint64_t idx, float (&f)[EPL]) {
  if (bf16) {
    uint32_t w[EPL / 2];
    load_bytes<EPL * 2>(reinterpret_cast<const uint8_t*>(base) + idx * 2u, w);
#pragma unroll
    for (int i = 0; i < EPL; ++i) f[i] = bf16_bits_to_f32((w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
  } else {
    uint32_t w[EPL];
    load_bytes<EPL * 4>(reinterpret_cast<const uint8_t*>(base) + idx * 4u, w);
#pragma unroll
    for (int i = 0; i < EPL; ++i) f[i] = __uint_as_float(w[i]);
  }
}

template <int EPL>
__device__ __forceinline__ void load_f32(const float* p, float (&f)[EPL]) {
  uint32_t w[EPL];
  load_bytes<EPL * 4>(reinterpret_cast<const uint8_t*>(p), w);
#pragma unroll
  for (int i = 0; i < EPL; ++i) f[i] = __uint_as_float(w[i]);
}

// Dequantize EPL codes of one row slice held in words w: scale * code.
template <int QB, int EPL>
__device__ __forceinline__ void dequant_words(const uint32_t (&w)[EPL * QB / 32], float s, float (&sh)[EPL]) {
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    int32_t c;
    if constexpr (QB == 8) c = (int32_t)(int8_t)(w[i >> 2] >> (8 * (i & 3)));
    else c = (int32_t)(w[i >> 3] << (28 - 4 * (i & 7))) >> 28;
    sh[i] = s * (float)c;
  }
}

template <int QB, int EPL>
__device__ __forceinline__ void load_codes(const uint8_t* p, float s, float (&sh)[EPL]) {
  uint32_t w[EPL * QB / 32];
  load_bytes<EPL * QB / 8, true>(p, w);
  dequant_words<QB, EPL>(w, s, sh);
}



// Protected row slice: widen / store in hp_dtype (0 fp32, 1 bf16, 2 fp16).
template <int EPL>
__device__ __forceinline__ void load_hp(const uint8_t* p, int dt, float (&f)[EPL]) {
  if (dt == 0) {
    uint32_t w[EPL];
    load_bytes<EPL * 4, true>(p, w);
#pragma unroll
    for (int i = 0; i < EPL; ++i) f[i] = __uint_as_float(w[i]);
  } else {
    uint32_t w[EPL / 2];
    load_bytes<EPL * 2, true>(p, w);
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const uint32_t b = (w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      f[i] = (dt == 1) ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
    }
  }
}

template <int EPL>
__device__ __forceinline__ void store_hp(uint8_t* p, int dt, const float (&f)[EPL]) {
  if (dt == 0) {
    uint32_t w[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) w[i] = __float_as_uint(f[i]);
    store_bytes<EPL * 4, true>(p, w);
  } else {
    uint32_t w[EPL / 2];
    if (dt == 1) {
#pragma unroll
      for (int i = 0; i < EPL / 2; ++i) w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    } else {
#pragma unroll
      for (int i = 0; i < EPL / 2; ++i) w[i] = pack_f16x2(f[2 * i], f[2 * i + 1]);
    }
    store_bytes<EPL * 2, true>(p, w);
  }
}

// ---------------------------------------------------------------------------
// Row scale (value-axis grouping): scale = max / Q correctly rounded; the
// rounding inverse inv = Q / max rounded toward zero (the largest fp32 with
// inv * max <= Q, so every |x| = |value * inv| <= Q and no code needs a
// clamp); invb = inv * 2^SRB (exact scaling) for stochastic rounding with
// SRB random bits.  A zero row, or one whose nearest Q / max (times 2^SRB)
// overflows, is stored as zero.
// ---------------------------------------------------------------------------

// q / m rounded toward zero from an estimate rn within one unit in the last
// place of it (q, m > 0, rn finite and positive): one of the two floats
// around the quotient.  The residual q - rn * m is exact in one fma, and a
// negative one means rn lies above the quotient, so the next float down is
// taken.
__device__ __forceinline__ float inv_toward_zero(float q, float m, float rn) {
  const float e = fmaf(-rn, m, q);
  return e < 0.0f ? __uint_as_float(__float_as_uint(rn) - 1u) : rn;
}

template <int QB, int SRB>
__device__ __forceinline__ void row_scale(float m, float& scale, float& inv, float& invb) {
  constexpr float Q = (QB == 8) ? 127.0f : 7.0f;
  scale = 0.0f;
  inv = 0.0f;
  invb = 0.0f;
  if (m > 0.0f) {
    const float s = m / Q;
    const float i = Q / m;
    const float ib = i * (float)(1u << SRB);
    if (__builtin_isfinite(ib)) {
      scale = s;
      inv = inv_toward_zero(Q, m, i);
      invb = inv * (float)(1u << SRB);
    }
  }
}

// Row scale stored as bf16 (the bf16 layout of the low-rank bypass): the
// smallest bf16 value s with Q s >= m, and codes are taken against it: inv =
// the largest fp32 with inv s <= 1, so |value * inv| <= m / s <= Q.  q =
// m / Q (nearest) rounded up to bf16 on its bit pattern is that s unless q
// fell below m / Q while being a bf16 value itself; then the next bf16 up
// is (a bf16 value times Q is exact in fp32, so the test is exact).  A row
// with m = 0, or whose s overflows, or whose 2^SRB / s is not finite, is
// stored as zero.  `mq` is m / Q, correctly rounded.
template <int QB, int SRB>
__device__ __forceinline__ void row_scale_bf16(float m, float mq, float& scale, float& inv, float& invb) {
  constexpr float Q = (QB == 8) ? 127.0f : 7.0f;
  uint32_t b = (__float_as_uint(mq) + 0xFFFFu) & 0xFFFF0000u;
  if (__uint_as_float(b) * Q < m) b += 0x10000u;
  const float sb = __uint_as_float(b);
  const float i = 1.0f / sb;
  const bool ok = __builtin_isfinite(sb) && __builtin_isfinite(i * (float)(1u << SRB));
  const float iz = inv_toward_zero(1.0f, sb, i);
  scale = ok ? sb : 0.0f;
  inv = ok ? iz : 0.0f;
  invb = ok ? iz * (float)(1u << SRB) : 0.0f;
}

// x rounded to bf16 (nearest even) and widened back.
__device__ __forceinline__ float round_bf16(float x) { return bf16_bits_to_f32(f32_to_bf16_bits(x)); }

// floor(x + 1/2) as an integer, one v_cvt_rpi_i32_f32 (exact for |x| < 2^23,
// where x + 1/2 is representable).
__device__ __forceinline__ int32_t cvt_rpi(float x) {
  int32_t r;
  asm("v_cvt_rpi_i32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// Random bits per element for rounding mode RND (0 nearest, 1: 16, 2: 8).
template <int RND>
constexpr int sr_bits_of() { return RND == 1 ? 16 : (RND == 2 ? 8 : 0); }

// Round one element to a code.  Nearest: rint(sp * inv), ties to even.
// Stochastic (fixed point): X = floor(sp * invb + 1/2) is x rounded to SRB
// fractional bits; the element's SRB-bit integer rb is added below the LSB
// and the sum truncated, code = (X + rb) >> SRB.  BDR: with x = sp * inv and
// xo = sh * inv (old value on the new grid), a code below xo - bound while
// the element grew takes ceil(x); above xo + bound while it shrank takes
// floor(x).  |x| <= Q (inv rounded toward zero) keeps every code in
// [-Q, Q].  A zero row (inv = 0) gives 0.
// BDR as one clamp.  The rule: an element that grew (sp > sh, so x >= xo:
// rounding is monotone) whose code c fell below t = xo - bound takes ceil(x);
// one that shrank whose code rose above xo + bound takes floor(x).  Both
// codes here (nearest, or stochastic from x rounded to sr_bits fractional
// bits) lie in {floor(x), floor(x) + 1}; so c < t <= x forces c = floor(x)
// with t in (c, c + 1), where ceil(x) = c + 1 = ceil(t), and c >= t means
// c >= ceil(t).  Hence the rule is c' = max(c, ceil(t)) for a grown element,
// and likewise min(c, floor(xo + bound)) for a shrunk one: med3 of c and the
// two limits (infinite when they do not apply).
// BDR 2 is the same rule for a bound known to be zero (xo -/+ 0 is xo up to
// the sign of a zero, which no code depends on), two instructions fewer.
template <int BDR>
__device__ __forceinline__ float bdr_clamp(float cf, float sp, float sh, float inv, float bound) {
  const float xo = sh * inv;
  const float tl = (BDR == 2) ? xo : xo - bound;
  const float th = (BDR == 2) ? xo : xo + bound;
  const float lo = sp > sh ? ceilf(tl) : -__builtin_inff();
  const float hi = sp < sh ? floorf(th) : __builtin_inff();
  return __builtin_amdgcn_fmed3f(cf, lo, hi);
}

template <int QB, int RND, int BDR>
__device__ __forceinline__ int32_t round_elem(float sp, float sh, float inv, float invb, uint32_t rb,
                                              float bound) {
  if constexpr (RND == 0) {
    // decided in float (ceil, floor and rint of |x| <= Q are exact), one
    // conversion at the end
    float cf = rintf(sp * inv);
    if constexpr (BDR) cf = bdr_clamp<BDR>(cf, sp, sh, inv, bound);
    return (int32_t)cf;
  } else {
    constexpr int SRB = sr_bits_of<RND>();
    int32_t c = (cvt_rpi(sp * invb) + (int32_t)rb) >> SRB;
    if constexpr (BDR) c = (int32_t)bdr_clamp<BDR>((float)c, sp, sh, inv, bound);
    return c;
  }
}

// N codes packed into N * QB / 32 words, code i at bits QB*i.. of the
// stream (low bits first).  int8: byte i & 3 of word i >> 2.  int4, codes
// in [-8, 7]: each offset code c + 8 is a digit in [0, 15], so the word of
// offset codes is the plain sum of (c_i + 8) 16^i, with no carry between
// digits; in wrapping 32-bit arithmetic that is 0x88888888 + sum c_i 16^i,
// one shift-add per code, and xor 0x88888888 turns every digit c + 8 back
// into c mod 16 (c >= 0: c + 8 has bit 3 set; c < 0: it has not, and
// c + 8 + 8 = c + 16).  Unused digits of a partial word come out 0.
template <int QB, int N>
__device__ __forceinline__ void pack_codes(const int32_t (&c)[N], uint32_t (&w)[(N * QB + 31) / 32]) {
  constexpr int NW = (N * QB + 31) / 32;
  if constexpr (QB == 8) {
#pragma unroll
    for (int j = 0; j < NW; ++j) w[j] = 0u;
#pragma unroll
    for (int i = 0; i < N; ++i) w[i >> 2] |= ((uint32_t)c[i] & 0xFFu) << (8 * (i & 3));
  } else {
#pragma unroll
    for (int j = 0; j < NW; ++j) w[j] = 0x88888888u;
#pragma unroll
    for (int i = 0; i < N; ++i) w[i >> 3] += (uint32_t)c[i] << (4 * (i & 7));
#pragma unroll
    for (int j = 0; j < NW; ++j) w[j] ^= 0x88888888u;
  }
}

}  // namespace qs
