/*
 * qs_oracle.c -- CPU oracle for the quantized recurrent-state decode step.
 *
 * TEST INFRASTRUCTURE ONLY (see qs_oracle.h).  Plain scalar C; every
 * function follows one stated passage and is written for reading, not speed.
 *
 * Logical state per (b,h): S[v][k], v the value index (a "value column" of
 * the pages' S, i.e. one output channel), k the key index.  One row v is one
 * value-axis scale group.
 */
#include "qs_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon et al., SC'11, the Philox family section): a       */
/* counter-based generator.  One round multiplies counter words 0 and 2 by  */
/* the two Philox multipliers, keeps both halves of the 64-bit products and */
/* mixes the high halves with the other two counter words and the key; the  */
/* key is bumped by the two Weyl constants between rounds.                  */
/* ------------------------------------------------------------------------ */
#define PHILOX_MUL0 0xD2511F53u
#define PHILOX_MUL1 0xCD9E8D57u
#define PHILOX_WEYL0 0x9E3779B9u
#define PHILOX_WEYL1 0xBB67AE85u

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += PHILOX_WEYL0;
      k1 += PHILOX_WEYL1;
    }
    uint64_t p0 = (uint64_t)PHILOX_MUL0 * (uint64_t)x0;
    uint64_t p1 = (uint64_t)PHILOX_MUL1 * (uint64_t)x2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t y0 = hi1 ^ x1 ^ k0;
    uint32_t y1 = lo1;
    uint32_t y2 = hi0 ^ x3 ^ k1;
    uint32_t y3 = lo0;
    x0 = y0; x1 = y1; x2 = y2; x3 = y3;
  }
  out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* Random integer for element index e at decode step `step`.
 * Key = seed; counter = (element group as 64 bits, step as 64 bits).
 * 16-bit mode: 8 elements per Philox block, element e takes the low half of
 * word (e>>1)&3 when e is even, the high half when odd.
 * 8-bit mode: 16 elements per block, byte e&3 of word (e>>2)&3. */
uint32_t orc_random_bits(const orc_cfg* c, uint64_t e, uint64_t step) {
  uint32_t key[2] = {(uint32_t)c->seed, (uint32_t)(c->seed >> 32)};
  uint64_t grp = (c->sr_bits == 16) ? (e >> 3) : (e >> 4);
  uint32_t ctr[4] = {(uint32_t)grp, (uint32_t)(grp >> 32), (uint32_t)step,
                     (uint32_t)(step >> 32)};
  uint32_t out[4];
  orc_philox4x32_10(ctr, key, out);
  if (c->sr_bits == 16) {
    uint32_t w = out[(e >> 1) & 3];
    return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
  }
  uint32_t w = out[(e >> 2) & 3];
  return (w >> (8 * (e & 3))) & 0xFFu;
}

/* Stochastic rounding (LoReS abstract) in fixed point: x is first rounded
 * to sr_bits fractional bits, halves up, X = floor(x * 2^sr_bits + 1/2);
 * the element's sr_bits-bit uniform integer u is added below the LSB and the
 * sum truncated: code = floor((X + u) / 2^sr_bits).  Integer arithmetic, so
 * the decision is exact; E[code] = X / 2^sr_bits, within 2^-(sr_bits+1) of
 * x.  `xb` is x * 2^sr_bits. */
/* q / m rounded toward zero, for finite q, m > 0 whose quotient is finite:
 * the nearest float, stepped down once when it exceeds the exact quotient.
 * A product of two floats is exact in double, so the comparison is exact. */
float orc_inv_rtz(float q, float m) {
  float f = q / m;
  if ((double)f * (double)m > (double)q) f = nextafterf(f, 0.0f);
  return f;
}

float orc_sr_round(float xb, uint32_t u, int32_t sr_bits) {
  double X = floor((double)xb + 0.5);
  return (float)floor((X + (double)u) / ldexp(1.0, sr_bits));
}

/* ------------------------------------------------------------------------ */
/* Round-to-nearest-even into a binary format with `mbits` fraction bits and */
/* `ebits` exponent bits (IEEE-style bias, subnormals, infinities).  Written */
/* from the format's definition with exact fp64 scaling; used for bf16      */
/* (8,7) and fp16 (5,10) storage of protected units.                        */
/* ------------------------------------------------------------------------ */
static uint32_t rne_encode(float f, int ebits, int mbits) {
  const uint32_t sign = signbit(f) ? 1u : 0u;
  const int bias = (1 << (ebits - 1)) - 1;
  const int emin = 1 - bias, emax = bias;
  const uint32_t eall = (1u << ebits) - 1u;
  const uint32_t sbit = sign << (ebits + mbits);
  if (isnan(f)) return sbit | (eall << mbits) | (1u << (mbits - 1));
  if (isinf(f)) return sbit | (eall << mbits);
  double a = fabs((double)f);
  if (a == 0.0) return sbit;
  int e;
  (void)frexp(a, &e);
  e -= 1;                       /* a = m * 2^e with m in [1,2) */
  if (e < emin) e = emin;       /* subnormal range: fixed exponent */
  double q = rint(ldexp(a, mbits - e));   /* units in the last place */
  if (q >= ldexp(1.0, mbits + 1)) {       /* rounding carried into the exponent */
    q = ldexp(q, -1);
    e += 1;
  }
  if (e > emax) return sbit | (eall << mbits);
  if (q < ldexp(1.0, mbits)) return sbit | (uint32_t)q;  /* subnormal */
  return sbit | ((uint32_t)(e + bias) << mbits) | ((uint32_t)q - (1u << mbits));
}

static float decode_bits(uint32_t bits, int ebits, int mbits) {
  const int bias = (1 << (ebits - 1)) - 1;
  const uint32_t eall = (1u << ebits) - 1u;
  uint32_t sign = (bits >> (ebits + mbits)) & 1u;
  uint32_t ex = (bits >> mbits) & eall;
  uint32_t man = bits & ((1u << mbits) - 1u);
  double v;
  if (ex == eall) v = man ? NAN : INFINITY;
  else if (ex == 0) v = ldexp((double)man, 1 - bias - mbits);
  else v = ldexp((double)(man | (1u << mbits)), (int)ex - bias - mbits);
  return (float)(sign ? -v : v);
}

uint16_t orc_to_bf16(float f) { return (uint16_t)rne_encode(f, 8, 7); }
uint16_t orc_to_fp16(float f) { return (uint16_t)rne_encode(f, 5, 10); }
float orc_from_bf16(uint16_t h) { return decode_bits(h, 8, 7); }
float orc_from_fp16(uint16_t h) { return decode_bits(h, 5, 10); }

/* The smallest bf16 value s with q * s >= m (m > 0, q > 0 small integer):
 * start from the nearest bf16 of m / q and step by one bf16 unit either way
 * while the exact comparison (a bf16 times a small integer is exact in
 * double) asks for it.  Returns +inf when no finite bf16 qualifies. */
float orc_scale_bf16_up(float m, float q) {
  uint16_t b = orc_to_bf16(m / q);
  /* down while the next smaller positive bf16 still qualifies */
  while ((b & 0x7FFFu) > 0u && (double)orc_from_bf16((uint16_t)(b - 1u)) * (double)q >= (double)m) b -= 1u;
  /* up while b does not qualify */
  while ((double)orc_from_bf16(b) * (double)q < (double)m) {
    if ((b & 0x7F80u) == 0x7F80u) return INFINITY;
    b += 1u;
  }
  return orc_from_bf16(b);
}

/* ------------------------------------------------------------------------ */
/* Decay-based mixed precision (LoReS abstract: protect slowly decaying      */
/* heads or channels).  Within each group of `per_group` units, flag the     */
/* round-half-up(frac * per_group) units with the smallest decay-rate        */
/* statistic (slowest decay); ties go to the lower index.                    */
/* ------------------------------------------------------------------------ */
int orc_build_map(const double* stat, int32_t groups, int32_t per_group, double frac,
                  uint8_t* map) {
  if (groups < 0 || per_group <= 0 || !(frac >= 0.0 && frac <= 1.0)) return -1;
  int32_t count = (int32_t)floor(frac * per_group + 0.5);
  for (int32_t g = 0; g < groups; ++g) {
    const double* s = stat + (int64_t)g * per_group;
    uint8_t* m = map + (int64_t)g * per_group;
    for (int32_t i = 0; i < per_group; ++i) {
      /* rank of unit i = number of units that come before it in the order
       * (smaller statistic, or equal statistic and lower index) */
      int32_t rank = 0;
      for (int32_t j = 0; j < per_group; ++j)
        if (s[j] < s[i] || (s[j] == s[i] && j < i)) ++rank;
      m[i] = (rank < count) ? 1 : 0;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Storage layout (the library's documented format, written out here         */
/* independently).  Per head h: nq(h) quantized key channels, in ascending   */
/* k, each row taking ceil(nq*qbits/8) bytes (int4: two codes per byte, low  */
/* nibble first); the head's code block is dv rows, padded to 16 bytes.      */
/* Protected channels, in ascending k, form a second per-head block of dv    */
/* rows of 16-bit (or fp32) values, also padded to 16 bytes.  Blocks of one  */
/* batch element follow head order; batch elements follow each other.        */
/* ------------------------------------------------------------------------ */
static int is_quantized(const orc_cfg* c, int h, int k) {
  if (c->map_mode == 0) return 1;
  if (c->map_mode == 1) return c->map[h] == 0;
  return c->map[(int64_t)h * c->dk + k] == 0;
}

static int hp_bytes(const orc_cfg* c) { return c->hp_dtype == 0 ? 4 : 2; }

static uint64_t round16(uint64_t x) { return (x + 15u) & ~(uint64_t)15u; }
static uint64_t round4(uint64_t x) { return (x + 3u) & ~(uint64_t)3u; }

/* Bytes of one stored row: the quantized channels' codes, and the protected
 * channels' values, each padded to a multiple of 4 bytes (a fully quantized
 * or fully protected row already is one). */
static uint64_t code_row_bytes(const orc_cfg* c, int nq) {
  return round4(((uint64_t)nq * (uint64_t)c->qbits + 7u) / 8u);
}
static uint64_t hp_row_bytes(const orc_cfg* c, int nhp) {
  return round4((uint64_t)nhp * (uint64_t)hp_bytes(c));
}

/* Scale groups of a head: value axis (a row, scale_axis 0), key axis (a
 * column, 1), the whole head (2). */
static int n_groups(const orc_cfg* c) { return c->scale_axis == 0 ? c->dv : (c->scale_axis == 1 ? c->dk : 1); }
static int group_of(const orc_cfg* c, int v, int k) {
  return c->scale_axis == 0 ? v : (c->scale_axis == 1 ? k : 0);
}

static int check_cfg(const orc_cfg* c) {
  if (c->kind != 0 && c->kind != 1) return -1;
  if (c->decay_mode != 0 && c->decay_mode != 1) return -1;
  if (c->B < 0 || c->H <= 0 || c->dk <= 0 || c->dv <= 0) return -1;
  if (c->qbits != 8 && c->qbits != 4) return -1;
  if (c->hp_dtype < 0 || c->hp_dtype > 2) return -1;
  if (c->map_mode < 0 || c->map_mode > 2) return -1;
  if (c->map_mode != 0 && !c->map) return -1;
  if (c->rounding != 0 && c->rounding != 1) return -1;
  if (c->rounding == 1 && c->sr_bits != 16 && c->sr_bits != 8) return -1;
  if (c->lrb_rank < 0) return -1;
  if (c->lrb_rank > 0 && (c->map_mode != 0 || c->lrb_period <= 0)) return -1;
  if ((c->scale_dtype != 0 && c->scale_dtype != 1) || (c->lrb_dtype != 0 && c->lrb_dtype != 1)) return -1;
  /* key-axis and per-head groups: every channel quantized, no buffer */
  if (c->scale_axis < 0 || c->scale_axis > 2) return -1;
  if (c->scale_axis != 0 && (c->map_mode != 0 || c->lrb_rank != 0)) return -1;
  return 0;
}

/* A stored fp32 or bf16 element, widened; a value stored, bf16 rounded to
 * nearest even.  `bf` selects the format. */
static float get_f(const void* p, uint64_t i, int bf) {
  if (bf) return orc_from_bf16(((const uint16_t*)p)[i]);
  return ((const float*)p)[i];
}
static void put_f(void* p, uint64_t i, float x, int bf) {
  if (bf) ((uint16_t*)p)[i] = orc_to_bf16(x);
  else ((float*)p)[i] = x;
}
/* x rounded to the storage format of the low-rank buffer (and widened back). */
static float lrb_round(const orc_cfg* c, float x) {
  return c->lrb_dtype ? orc_from_bf16(orc_to_bf16(x)) : x;
}

int orc_layout(const orc_cfg* c, orc_sizes* s, uint64_t* code_off, uint64_t* hp_off,
               int32_t* nq_out) {
  if (check_cfg(c)) return -1;
  uint64_t coff = 0, hoff = 0;
  for (int h = 0; h < c->H; ++h) {
    int nq = 0;
    for (int k = 0; k < c->dk; ++k) nq += is_quantized(c, h, k);
    int nhp = c->dk - nq;
    if (code_off) code_off[h] = coff;
    if (hp_off) hp_off[h] = hoff;
    if (nq_out) nq_out[h] = nq;
    coff += round16((uint64_t)c->dv * code_row_bytes(c, nq));
    hoff += round16((uint64_t)c->dv * hp_row_bytes(c, nhp));
  }
  uint64_t BH = (uint64_t)c->B * (uint64_t)c->H;
  s->code_bstride = coff;
  s->hp_bstride = hoff;
  s->codes = (uint64_t)c->B * coff;
  s->hp = (uint64_t)c->B * hoff;
  s->scales = BH * (uint64_t)n_groups(c) * (c->scale_dtype ? 2u : 4u);
  s->W = BH * (uint64_t)c->dv * (uint64_t)c->lrb_rank * (c->lrb_dtype ? 2u : 4u);
  s->U = BH * (uint64_t)c->dk * (uint64_t)c->lrb_rank * (c->lrb_dtype ? 2u : 4u);
  s->n = c->lrb_rank > 0 ? BH * 4u : 0u;
  return 0;
}

/* Whole-config layout, computed once per call. */
typedef struct {
  orc_sizes s;
  uint64_t* code_off;
  uint64_t* hp_off;
  int32_t* nq;
} layout_t;

static int layout_make(const orc_cfg* c, layout_t* L) {
  L->code_off = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)c->H);
  L->hp_off = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)c->H);
  L->nq = (int32_t*)malloc(sizeof(int32_t) * (size_t)c->H);
  return orc_layout(c, &L->s, L->code_off, L->hp_off, L->nq);
}

static void layout_free(layout_t* L) {
  free(L->code_off);
  free(L->hp_off);
  free(L->nq);
}

/* Addressing of one head: its code block, its protected block, and for each
 * key channel its slot among the quantized (>= 0) or protected (~slot) ones. */
typedef struct {
  uint8_t* code;
  uint8_t* hpb;
  uint64_t row_bytes;      /* code row stride */
  uint64_t hp_row_bytes;   /* protected row stride */
  int nq, nhp;
  int* slot;
} head_addr;

static void head_address(const orc_cfg* c, const layout_t* L, const orc_state* st,
                         int64_t bh, head_addr* a, int* slot_buf) {
  int64_t b = bh / c->H;
  int h = (int)(bh % c->H);
  a->nq = L->nq[h];
  a->nhp = c->dk - a->nq;
  a->row_bytes = code_row_bytes(c, a->nq);
  a->hp_row_bytes = hp_row_bytes(c, a->nhp);
  a->code = st->codes ? st->codes + (uint64_t)b * L->s.code_bstride + L->code_off[h] : NULL;
  a->hpb = st->hp ? (uint8_t*)st->hp + (uint64_t)b * L->s.hp_bstride + L->hp_off[h] : NULL;
  int iq = 0, ih = 0;
  for (int k = 0; k < c->dk; ++k) slot_buf[k] = is_quantized(c, h, k) ? iq++ : ~(ih++);
  a->slot = slot_buf;
}

static int32_t get_code(const orc_cfg* c, const head_addr* a, int v, int slot) {
  const uint8_t* row = a->code + (uint64_t)v * a->row_bytes;
  if (c->qbits == 8) return (int32_t)(int8_t)row[slot];
  uint8_t byte = row[slot >> 1];
  int32_t nib = (slot & 1) ? (byte >> 4) : (byte & 0xF);
  return nib >= 8 ? nib - 16 : nib;   /* two's-complement nibble */
}

static void put_code(const orc_cfg* c, const head_addr* a, int v, int slot, int32_t code) {
  uint8_t* row = a->code + (uint64_t)v * a->row_bytes;
  if (c->qbits == 8) {
    row[slot] = (uint8_t)(int8_t)code;
    return;
  }
  uint8_t nib = (uint8_t)(code & 0xF);
  uint8_t* byte = &row[slot >> 1];
  if (slot & 1) *byte = (uint8_t)((*byte & 0x0F) | (nib << 4));
  else *byte = (uint8_t)((*byte & 0xF0) | nib);
}

static float get_hp(const orc_cfg* c, const head_addr* a, int v, int hslot) {
  const uint8_t* row = a->hpb + (uint64_t)v * a->hp_row_bytes;
  if (c->hp_dtype == 0) {
    float f;
    memcpy(&f, row + (uint64_t)hslot * 4u, 4);
    return f;
  }
  uint16_t bits;
  memcpy(&bits, row + (uint64_t)hslot * 2u, 2);
  return c->hp_dtype == 1 ? orc_from_bf16(bits) : orc_from_fp16(bits);
}

static void put_hp(const orc_cfg* c, const head_addr* a, int v, int hslot, float x) {
  uint8_t* row = a->hpb + (uint64_t)v * a->hp_row_bytes;
  if (c->hp_dtype == 0) {
    memcpy(row + (uint64_t)hslot * 4u, &x, 4);
    return;
  }
  uint16_t bits = c->hp_dtype == 1 ? orc_to_bf16(x) : orc_to_fp16(x);
  memcpy(row + (uint64_t)hslot * 2u, &bits, 2);
}

/* Dequantized value of element (v,k) of a head: scale times code for a
 * quantized channel, the widened stored value for a protected one. */
static float dequant_elem(const orc_cfg* c, const head_addr* a, float scale, int v, int k) {
  int slot = a->slot[k];
  if (slot < 0) return get_hp(c, a, v, ~slot);
  return scale * (float)get_code(c, a, v, slot);
}

/* ------------------------------------------------------------------------ */
/* Requantization (LoReS abstract: value-axis scale grouping; the groups of  */
/* the other axes are the ablations the abstract contrasts it with).  A      */
/* group's scale is its largest magnitude over quantized channels divided by */
/* Q (127 for 8 bits, 7 for 4 bits; symmetric grid, no zero point).  Each    */
/* element is x = value * (Q / max), rounded to nearest even or              */
/* stochastically (LoReS abstract); with BDR (abstract of the page on        */
/* preserving updates: reversed elements are rounded toward their update) an */
/* element whose new level lies on the wrong side of its previous value by   */
/* more than the bound takes the other neighbour of x instead.  Codes are    */
/* clamped to [-Q, Q].  Protected channels store the nearest 16-bit (or the  */
/* fp32) value.  `old` is the value before the step (BDR only; may be NULL). */
/* ------------------------------------------------------------------------ */
typedef struct {
  float scale, inv, invb;
} group_scale;

/* Scale and rounding inverse of a group whose largest magnitude is m. */
static group_scale scale_of(const orc_cfg* c, float m) {
  const float Q = (c->qbits == 8) ? 127.0f : 7.0f;
  /* A group whose nearest inverse Q / max (times 2^sr_bits under stochastic
   * rounding) overflows, i.e. max below about Q*2^16/FLT_MAX, is stored as
   * zero.  The inverse used for rounding is Q / max rounded toward zero: the
   * largest float inv with inv * max <= Q exactly, so |value * inv| <= Q for
   * every element of the group and no code ever reaches the clamp. */
  group_scale g = {0.0f, 0.0f, 0.0f};
  if (m > 0.0f && c->scale_dtype == 0) {
    g.scale = m / Q;
    g.inv = Q / m;
    g.invb = (c->rounding == 1) ? ldexpf(g.inv, c->sr_bits) : g.inv;
    if (!isfinite(g.inv) || !isfinite(g.invb)) {
      g.scale = g.inv = g.invb = 0.0f;
    } else {
      g.inv = orc_inv_rtz(Q, m);
      g.invb = (c->rounding == 1) ? ldexpf(g.inv, c->sr_bits) : g.inv;
    }
  } else if (m > 0.0f) {
    /* bf16 scales: the stored scale s is the smallest bf16 value with
     * Q s >= m (Q s is exact in double), and codes are taken against s:
     * inv is the largest float with inv s <= 1, so |value * inv| <= m / s
     * <= Q.  A group whose s overflows, or whose inv (times 2^sr_bits) is
     * not finite, is stored as zero. */
    g.scale = orc_scale_bf16_up(m, Q);
    if (isfinite(g.scale)) {
      g.inv = orc_inv_rtz(1.0f, g.scale);
      g.invb = (c->rounding == 1) ? ldexpf(g.inv, c->sr_bits) : g.inv;
    }
    if (!isfinite(g.scale) || !isfinite(g.inv) || !isfinite(g.invb)) g.scale = g.inv = g.invb = 0.0f;
  }
  return g;
}

/* The code of one quantized element (stored slot `slot` of row v). */
static int32_t round_code(const orc_cfg* c, int64_t bh, int v, int slot, float sp, const float* old,
                          group_scale g, uint64_t step) {
  const float Q = (c->qbits == 8) ? 127.0f : 7.0f;
  float x = sp * g.inv;
  float code;
  if (c->rounding == 0) {
    code = rintf(x);
  } else {
    /* the element's index in the stored code rows: its slot, which is the
     * key channel itself when the whole head is quantized */
    uint64_t e = ((uint64_t)bh * (uint64_t)c->dv + (uint64_t)v) * (uint64_t)c->dk + (uint64_t)slot;
    code = orc_sr_round(sp * g.invb, orc_random_bits(c, e, step), c->sr_bits);
  }
  if (c->bdr && old) {
    float xo = *old * g.inv;
    float d = sp - *old;
    if (d > 0.0f && code < xo - c->bdr_bound) code = ceilf(x);
    else if (d < 0.0f && code > xo + c->bdr_bound) code = floorf(x);
  }
  if (code > Q) code = Q;
  if (code < -Q) code = -Q;
  return (int32_t)code;
}

/* Value-axis groups: one row.  Returns the row's new scale. */
static float requantize_row(const orc_cfg* c, const head_addr* a, int64_t bh, int v,
                            const float* sp, const float* old, uint64_t step) {
  const int dk = c->dk;
  float m = 0.0f;
  for (int k = 0; k < dk; ++k)
    if (a->slot[k] >= 0) {
      float mag = fabsf(sp[k]);
      if (mag > m) m = mag;
    }
  group_scale g = scale_of(c, m);
  for (int k = 0; k < dk; ++k) {
    int slot = a->slot[k];
    if (slot < 0) {
      put_hp(c, a, v, ~slot, sp[k]);
      continue;
    }
    put_code(c, a, v, slot, round_code(c, bh, v, slot, sp[k], old ? &old[k] : NULL, g, step));
  }
  return g.scale;
}

/* Requantization of a whole head with key-axis or per-head groups (map NONE,
 * every channel quantized, slot = k): the groups' maxima over sp [dv][dk],
 * then every element against its group's scale.  scales[G] receives them. */
static void requantize_grouped(const orc_cfg* c, const head_addr* a, int64_t bh, const float* sp,
                               const float* old, uint64_t step, float* scales) {
  const int dk = c->dk, dv = c->dv, G = n_groups(c);
  float* m = (float*)calloc((size_t)G, sizeof(float));
  group_scale* g = (group_scale*)malloc(sizeof(group_scale) * (size_t)G);
  for (int v = 0; v < dv; ++v)
    for (int k = 0; k < dk; ++k) {
      float mag = fabsf(sp[v * dk + k]);
      int gi = group_of(c, v, k);
      if (mag > m[gi]) m[gi] = mag;
    }
  for (int i = 0; i < G; ++i) {
    g[i] = scale_of(c, m[i]);
    scales[i] = g[i].scale;
  }
  for (int v = 0; v < dv; ++v)
    for (int k = 0; k < dk; ++k)
      put_code(c, a, v, k, round_code(c, bh, v, k, sp[v * dk + k], old ? &old[v * dk + k] : NULL,
                                      g[group_of(c, v, k)], step));
  free(m);
  free(g);
}

/* fp32 logical state [B,H,dv,dk] -> stored state.  No previous value, so no
 * BDR; the low-rank bypass buffer starts empty. */
int orc_quantize(const orc_cfg* c, const float* S, orc_state* st, uint64_t step) {
  layout_t L;
  if (layout_make(c, &L)) {
    layout_free(&L);
    return -1;
  }
  const int dk = c->dk, dv = c->dv, r = c->lrb_rank;
  int* slot = (int*)malloc(sizeof(int) * (size_t)dk);
  int64_t BH = (int64_t)c->B * c->H;
  for (int64_t bh = 0; bh < BH; ++bh) {
    head_addr a;
    head_address(c, &L, st, bh, &a, slot);
    if (c->scale_axis == 0) {
      for (int v = 0; v < dv; ++v) {
        const float* row = S + ((uint64_t)bh * dv + (uint64_t)v) * (uint64_t)dk;
        put_f(st->scales, (uint64_t)bh * dv + v, requantize_row(c, &a, bh, v, row, NULL, step), c->scale_dtype);
      }
    } else {
      const int G = n_groups(c);
      float* sc = (float*)malloc(sizeof(float) * (size_t)G);
      requantize_grouped(c, &a, bh, S + (uint64_t)bh * dv * dk, NULL, step, sc);
      for (int i = 0; i < G; ++i) put_f(st->scales, (uint64_t)bh * G + i, sc[i], c->scale_dtype);
      free(sc);
    }
    if (r > 0) {
      for (uint64_t i = 0; i < (uint64_t)dv * r; ++i) put_f(st->W, (uint64_t)bh * dv * r + i, 0.0f, c->lrb_dtype);
      for (uint64_t i = 0; i < (uint64_t)dk * r; ++i) put_f(st->U, (uint64_t)bh * dk * r + i, 0.0f, c->lrb_dtype);
      st->n[bh] = 0;
    }
  }
  free(slot);
  layout_free(&L);
  return 0;
}

/* Low-rank buffer column k as seen by row v: sum over the first n basis
 * vectors of W[v][j] * U[k][j], as an fp32 fused multiply-add chain in
 * ascending j. */
static float lrb_entry(const float* W, const float* U, int r, int n, int v, int k) {
  float acc = 0.0f;
  for (int j = 0; j < n; ++j) acc = fmaf(W[v * r + j], U[k * r + j], acc);
  return acc;
}

/* stored state -> fp32 effective state [B,H,dv,dk]: dequantized state plus
 * the low-rank bypass buffer W U^T when it is on. */
int orc_dequantize(const orc_cfg* c, const orc_state* st, float* S) {
  layout_t L;
  if (layout_make(c, &L)) {
    layout_free(&L);
    return -1;
  }
  const int dk = c->dk, dv = c->dv, r = c->lrb_rank;
  int* slot = (int*)malloc(sizeof(int) * (size_t)dk);
  int64_t BH = (int64_t)c->B * c->H;
  for (int64_t bh = 0; bh < BH; ++bh) {
    head_addr a;
    head_address(c, &L, st, bh, &a, slot);
    float* W = (float*)malloc(sizeof(float) * (size_t)(dv * r + 1));
    float* U = (float*)malloc(sizeof(float) * (size_t)(dk * r + 1));
    for (int i = 0; i < dv * r; ++i) W[i] = get_f(st->W, (uint64_t)bh * dv * r + i, c->lrb_dtype);
    for (int i = 0; i < dk * r; ++i) U[i] = get_f(st->U, (uint64_t)bh * dk * r + i, c->lrb_dtype);
    const int G = n_groups(c);
    for (int v = 0; v < dv; ++v) {
      float* row = S + ((uint64_t)bh * dv + (uint64_t)v) * (uint64_t)dk;
      for (int k = 0; k < dk; ++k) {
        float scale = get_f(st->scales, (uint64_t)bh * G + group_of(c, v, k), c->scale_dtype);
        float x = dequant_elem(c, &a, scale, v, k);
        if (r > 0) x = x + lrb_entry(W, U, r, st->n[bh], v, k);
        row[k] = x;
      }
    }
    free(W);
    free(U);
  }
  free(slot);
  layout_free(&L);
  return 0;
}

static double dot_d(const float* a, const float* b, int n) {
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += (double)a[i] * (double)b[i];
  return s;
}

/* ------------------------------------------------------------------------ */
/* Low-Rank Bypass (abstract of the page on preserving updates: small        */
/* updates accumulate in a compact low-rank buffer whose sufficiently large  */
/* elements are merged into the state periodically).  The page names Gated  */
/* DeltaNet, GLA, Mamba2 and RetNet, so both kinds.  Buffer of one head:     */
/* L = W U^T, W [dv][r] with orthonormal columns 0..n-1, U [dk][r].  Reading */
/* taken (the page gives one sentence):                                      */
/*  1. the buffer decays with the state: U[k][:] *= d[k] (lrb_decay, done    */
/*     before the write vector, which for the delta rule reads the decayed   */
/*     buffer);                                                              */
/*  2. while n < r, the write vector u (Gram-Schmidt, two passes, against the */
/*     basis) adds a basis column when its new part is above 2^-10 |u|;      */
/*  3. coefficients c = W^T u, remainder u_perp = u - W c;                   */
/*  4. key channel k is small when |k_k| * max_v(|u_v| / s_v) < theta (the   */
/*     update is under theta LSB in every row, s = scales on entry); a small */
/*     channel sends c k_k into U[k] and only u_perp k_k into the state;     */
/*  5. on a merge step, a buffer column whose entry reaches theta * s_v in   */
/*     some row is added to the state before rounding and cleared; when the  */
/*     whole buffer is clear the basis is reset (n = 0).                     */
/* Outputs: per-channel flags, u_perp, merged columns [dv][dk] (0 if none). */
/* ------------------------------------------------------------------------ */
static void lrb_decay(const orc_cfg* c, float* U, const float* d) {
  const int dk = c->dk, r = c->lrb_rank;
  for (int k = 0; k < dk; ++k)
    for (int j = 0; j < r; ++j) U[k * r + j] = d[k] * U[k * r + j];
}

/* Steps 2-5 (the buffer has decayed already). */
static void lrb_phase(const orc_cfg* c, float* W, float* U, int32_t* np_, const float* u,
                      const float* kk, const float* s_old, uint64_t step,
                      int* small, float* u_perp, float* merged, int* merge_flag) {
  const int dk = c->dk, dv = c->dv, r = c->lrb_rank;
  const float theta = c->lrb_theta;
  int n = *np_;
  /* 2. grow the basis */
  if (n < r) {
    float* y = (float*)malloc(sizeof(float) * (size_t)dv);
    float* wj = (float*)malloc(sizeof(float) * (size_t)dv);
    for (int v = 0; v < dv; ++v) y[v] = u[v];
    for (int pass = 0; pass < 2; ++pass)
      for (int j = 0; j < n; ++j) {
        for (int v = 0; v < dv; ++v) wj[v] = W[v * r + j];
        float p = (float)dot_d(wj, y, dv);
        for (int v = 0; v < dv; ++v) y[v] = fmaf(-p, W[v * r + j], y[v]);
      }
    float ny = sqrtf((float)dot_d(y, y, dv));
    float nu = sqrtf((float)dot_d(u, u, dv));
    if (ny > ldexpf(nu, -10)) {
      /* stored (and used from this step on) in the buffer's format */
      for (int v = 0; v < dv; ++v) W[v * r + n] = lrb_round(c, y[v] / ny);
      n += 1;
    }
    free(y);
    free(wj);
  }
  /* 3. project */
  float* cj = (float*)calloc((size_t)r, sizeof(float));
  float* wj = (float*)malloc(sizeof(float) * (size_t)dv);
  for (int j = 0; j < n; ++j) {
    for (int v = 0; v < dv; ++v) wj[v] = W[v * r + j];
    cj[j] = (float)dot_d(wj, u, dv);
  }
  for (int v = 0; v < dv; ++v) {
    float t = u[v];
    for (int j = 0; j < n; ++j) t = fmaf(-cj[j], W[v * r + j], t);
    u_perp[v] = t;
  }
  /* 4. small key channels */
  float g = 0.0f;
  for (int v = 0; v < dv; ++v) {
    float au = fabsf(u[v]);
    float gv = (s_old[v] > 0.0f) ? au / s_old[v] : (au > 0.0f ? INFINITY : 0.0f);
    if (gv > g) g = gv;
  }
  for (int k = 0; k < dk; ++k) {
    small[k] = isfinite(g) && (fabsf(kk[k]) * g < theta);
    if (small[k])
      for (int j = 0; j < n; ++j) U[k * r + j] = fmaf(kk[k], cj[j], U[k * r + j]);
  }
  /* the updated buffer in its storage format, before the merge test (what is
   * stored is what the state holds) */
  for (int i = 0; i < dk * r; ++i) U[i] = lrb_round(c, U[i]);
  /* 5. merge */
  for (int k = 0; k < dk; ++k) merge_flag[k] = 0;
  memset(merged, 0, sizeof(float) * (size_t)dv * (size_t)dk);
  if (c->lrb_period > 0 && ((step + 1u) % (uint64_t)c->lrb_period) == 0u) {
    int any_left = 0;
    for (int k = 0; k < dk; ++k) {
      int big = 0;
      for (int v = 0; v < dv; ++v) {
        float col = lrb_entry(W, U, r, n, v, k);
        if (col != 0.0f && fabsf(col) >= theta * s_old[v]) big = 1;
      }
      if (big) {
        merge_flag[k] = 1;
        for (int v = 0; v < dv; ++v) merged[v * dk + k] = lrb_entry(W, U, r, n, v, k);
        for (int j = 0; j < r; ++j) U[k * r + j] = 0.0f;
      }
    }
    for (int k = 0; k < dk; ++k)
      for (int j = 0; j < r; ++j)
        if (U[k * r + j] != 0.0f) any_left = 1;
    if (!any_left) n = 0;
  }
  *np_ = n;
  free(cj);
  free(wj);
}

/* ------------------------------------------------------------------------ */
/* One decode step of one head, in the order the method states: dequantize  */
/* the state, apply decay and the update, compute the output from the        */
/* pre-rounding state, requantize.                                           */
/*   additive (GLA, Mamba2, RetNet): S <- diag-decay(S) + u k^T, u = beta v  */
/*   delta rule (Gated DeltaNet):   S <- alpha S + u k^T,                     */
/*                                   u = beta (v - alpha S k)                 */
/* i.e. alpha (S - beta S k k^T) + beta v k^T written in factored form.      */
/* bh indexes the head's state (and its Philox element indices), bi its     */
/* inputs and output: equal for a plain step, slot and batch position for a  */
/* batched one.                                                              */
/* Element update: Sp = fmaf(u_v, k_k, (d_k * s_v) * code) for a quantized   */
/* channel (the decay scales the row scale), fmaf(u_v, k_k, d_k * value) for */
/* a protected one; readout o_v = sum_k Sp[v][k] q_k (+ buffer term).        */
/* ------------------------------------------------------------------------ */
static void head_step(const orc_cfg* c, const layout_t* L, orc_state* st, int64_t bh, int64_t bi,
                      const float* q, const float* kin, const float* vin, const float* decay,
                      const float* beta, float* out, uint64_t step, float* sp_dbg,
                      const orc_lrb_trace* tr) {
  const int dk = c->dk, dv = c->dv, r = c->lrb_rank;
  int* slot = (int*)malloc(sizeof(int) * (size_t)dk);
  head_addr a;
  head_address(c, L, st, bh, &a, slot);
  const float* qh = q + (uint64_t)bi * dk;
  const float* kh = kin + (uint64_t)bi * dk;
  const float* vh = vin + (uint64_t)bi * dv;
  float* d = (float*)malloc(sizeof(float) * (size_t)dk);
  for (int k = 0; k < dk; ++k)
    d[k] = (c->decay_mode == 0) ? decay[bi] : decay[(uint64_t)bi * dk + k];
  const float bt = beta ? beta[bi] : 1.0f;

  float* sh = (float*)malloc(sizeof(float) * (size_t)dv * (size_t)dk);
  float* sp = (float*)malloc(sizeof(float) * (size_t)dv * (size_t)dk);
  float* u = (float*)malloc(sizeof(float) * (size_t)dv);
  const int G = n_groups(c);
  float* s_old = (float*)malloc(sizeof(float) * (size_t)G);   /* group scales on entry */

  /* dequantize */
  for (int i = 0; i < G; ++i) s_old[i] = get_f(st->scales, (uint64_t)bh * G + i, c->scale_dtype);
  for (int v = 0; v < dv; ++v)
    for (int k = 0; k < dk; ++k) sh[v * dk + k] = dequant_elem(c, &a, s_old[group_of(c, v, k)], v, k);
  /* the low-rank buffer decays first: the delta rule reads it decayed */
  float* W = NULL;
  float* U = NULL;
  float* wb = (float*)calloc((size_t)dv, sizeof(float));
  if (r > 0) {
    /* the buffer's factors, widened to fp32 for the step (stored back below) */
    W = (float*)malloc(sizeof(float) * (size_t)dv * (size_t)r);
    U = (float*)malloc(sizeof(float) * (size_t)dk * (size_t)r);
    for (int i = 0; i < dv * r; ++i) W[i] = get_f(st->W, (uint64_t)bh * dv * r + i, c->lrb_dtype);
    for (int i = 0; i < dk * r; ++i) U[i] = get_f(st->U, (uint64_t)bh * dk * r + i, c->lrb_dtype);
    lrb_decay(c, U, d);
    /* buffer part of the decayed effective state times k:
     * wb_v = sum_j W[v][j] zk_j, zk = U^T k (fp64 sums, rounded once) */
    if (c->kind == 1) {
      const int n = st->n[bh];
      for (int j = 0; j < n; ++j) {
        double zk = 0.0;
        for (int k = 0; k < dk; ++k) zk += (double)U[k * r + j] * (double)kh[k];
        for (int v = 0; v < dv; ++v) wb[v] = fmaf(W[v * r + j], (float)zk, wb[v]);
      }
    }
  }
  /* write vector.  Delta rule with one decay per head (Gated DeltaNet):
   * u = beta (v - alpha (S_hat k)).  With a decay per key channel (the
   * channel-gated delta rule of Kimi-Linear, named in the LoReS abstract):
   * u = beta (v - (S_hat diag(d)) k), the decayed values being exactly the
   * ones the update adds u k^T to: (d_k s_v) code, or d_k value.  With the
   * low-rank buffer the rule acts on the effective state: wb is added to the
   * decayed state's product with k. */
  for (int v = 0; v < dv; ++v) {
    if (c->kind == 0) {
      u[v] = bt * vh[v];
    } else if (c->decay_mode == 0) {
      float w = (float)dot_d(sh + (uint64_t)v * dk, kh, dk);
      u[v] = (r > 0) ? bt * (vh[v] - (d[0] * w + wb[v])) : bt * (vh[v] - d[0] * w);
    } else {
      double w = 0.0;
      for (int k = 0; k < dk; ++k) {
        float dec = (a.slot[k] >= 0) ? (d[k] * s_old[group_of(c, v, k)]) * (float)get_code(c, &a, v, a.slot[k])
                                     : d[k] * sh[v * dk + k];
        w += (double)dec * (double)kh[k];
      }
      u[v] = (r > 0) ? bt * (vh[v] - ((float)w + wb[v])) : bt * (vh[v] - (float)w);
    }
  }
  /* low-rank bypass, steps 2-5 */
  int* small = (int*)calloc((size_t)dk, sizeof(int));
  int* mflag = (int*)calloc((size_t)dk, sizeof(int));
  float* u_perp = (float*)malloc(sizeof(float) * (size_t)dv);
  float* merged = NULL;
  if (r > 0) {
    merged = (float*)malloc(sizeof(float) * (size_t)dv * (size_t)dk);
    const int32_t n_before = st->n[bh];
    lrb_phase(c, W, U, &st->n[bh], u, kh, s_old, step, small, u_perp, merged, mflag);
    if (tr) {
      for (int k = 0; k < dk; ++k) {
        tr->small[(uint64_t)bh * dk + k] = small[k];
        tr->merged[(uint64_t)bh * dk + k] = mflag[k];
      }
      tr->n_before[bh] = n_before;
      tr->n_after[bh] = st->n[bh];
    }
  }
  /* decay + update (+ merged buffer columns).  The decay multiplies the
   * row scale before the code: (d_k * s_v) * code for a quantized channel,
   * d_k * value for a protected one. */
  for (int v = 0; v < dv; ++v)
    for (int k = 0; k < dk; ++k) {
      float uu = small[k] ? u_perp[v] : u[v];
      float decayed;
      if (a.slot[k] >= 0) decayed = (d[k] * s_old[group_of(c, v, k)]) * (float)get_code(c, &a, v, a.slot[k]);
      else decayed = d[k] * sh[v * dk + k];
      float x = fmaf(uu, kh[k], decayed);
      if (mflag[k]) x = x + merged[v * dk + k];
      sp[v * dk + k] = x;
    }
  /* readout from the pre-rounding state (+ buffer W (U^T q)) */
  double* z = NULL;
  if (r > 0) {
    z = (double*)calloc((size_t)r, sizeof(double));
    int n = st->n[bh];
    for (int j = 0; j < n; ++j)
      for (int k = 0; k < dk; ++k) z[j] += (double)U[k * r + j] * (double)qh[k];
  }
  for (int v = 0; v < dv; ++v) {
    double acc = dot_d(sp + (uint64_t)v * dk, qh, dk);
    if (r > 0)
      for (int j = 0; j < st->n[bh]; ++j) acc += (double)W[v * r + j] * z[j];
    out[(uint64_t)bi * dv + v] = (float)acc;
  }
  if (sp_dbg) memcpy(sp_dbg + (uint64_t)bi * dv * dk, sp, sizeof(float) * (size_t)dv * (size_t)dk);
  /* requantize */
  if (c->scale_axis == 0) {
    for (int v = 0; v < dv; ++v)
      put_f(st->scales, (uint64_t)bh * dv + v,
            requantize_row(c, &a, bh, v, sp + (uint64_t)v * dk, sh + (uint64_t)v * dk, step), c->scale_dtype);
  } else {
    float* sc = (float*)malloc(sizeof(float) * (size_t)G);
    requantize_grouped(c, &a, bh, sp, sh, step, sc);
    for (int i = 0; i < G; ++i) put_f(st->scales, (uint64_t)bh * G + i, sc[i], c->scale_dtype);
    free(sc);
  }
  if (r > 0) {   /* values already in the buffer's format: stored exactly */
    for (int i = 0; i < dv * r; ++i) put_f(st->W, (uint64_t)bh * dv * r + i, W[i], c->lrb_dtype);
    for (int i = 0; i < dk * r; ++i) put_f(st->U, (uint64_t)bh * dk * r + i, U[i], c->lrb_dtype);
    free(W);
    free(U);
  }

  free(z);
  free(wb);
  free(merged);
  free(u_perp);
  free(small);
  free(mflag);
  free(s_old);
  free(u);
  free(sp);
  free(sh);
  free(d);
  free(slot);
}

int orc_step(const orc_cfg* c, orc_state* st, const float* q, const float* k, const float* v,
             const float* decay, const float* beta, float* out, uint64_t step, float* sp_dbg,
             const int64_t* heads, int64_t nheads) {
  layout_t L;
  if (layout_make(c, &L)) {
    layout_free(&L);
    return -1;
  }
  int64_t BH = (int64_t)c->B * c->H;
  if (heads) {
    for (int64_t i = 0; i < nheads; ++i) {
      if (heads[i] < 0 || heads[i] >= BH) {
        layout_free(&L);
        return -1;
      }
      head_step(c, &L, st, heads[i], heads[i], q, k, v, decay, beta, out, step, sp_dbg, NULL);
    }
  } else {
    for (int64_t bh = 0; bh < BH; ++bh)
      head_step(c, &L, st, bh, bh, q, k, v, decay, beta, out, step, sp_dbg, NULL);
  }
  layout_free(&L);
  return 0;
}

/* A step for a batch of n sequences held in slots of the state pool (the
 * config's B states): batch element b reads its inputs and writes its
 * output at b and its state at slot[b], with its own step.  An element
 * whose slot lies outside [0, B) is skipped. */
int orc_step_batch(const orc_cfg* c, orc_state* st, const float* q, const float* k, const float* v,
                   const float* decay, const float* beta, float* out, int32_t n, const int32_t* slot,
                   const uint64_t* step) {
  layout_t L;
  if (n < 0 || n > c->B || layout_make(c, &L)) {
    if (n >= 0 && n <= c->B) layout_free(&L);
    return -1;
  }
  for (int32_t b = 0; b < n; ++b) {
    if (slot[b] < 0 || slot[b] >= c->B) continue;
    for (int32_t h = 0; h < c->H; ++h)
      head_step(c, &L, st, (int64_t)slot[b] * c->H + h, (int64_t)b * c->H + h, q, k, v, decay, beta, out,
                step[b], NULL, NULL);
  }
  layout_free(&L);
  return 0;
}

/* orc_step over every head, also reporting the low-rank bypass decisions the
 * step took (for tests that check them against a separate simulation). */
int orc_step_lrb_trace(const orc_cfg* c, orc_state* st, const float* q, const float* k,
                       const float* v, const float* decay, const float* beta, float* out,
                       uint64_t step, float* sp_dbg, const orc_lrb_trace* tr) {
  layout_t L;
  if (c->lrb_rank <= 0 || layout_make(c, &L)) {
    if (c->lrb_rank > 0) layout_free(&L);
    return -1;
  }
  int64_t BH = (int64_t)c->B * c->H;
  for (int64_t bh = 0; bh < BH; ++bh)
    head_step(c, &L, st, bh, bh, q, k, v, decay, beta, out, step, sp_dbg, tr);
  layout_free(&L);
  return 0;
}
