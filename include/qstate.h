/*
 * qstate.h -- C ABI of libqstate: the decode step of a gated linear
 * recurrence whose fixed-size per-head state is stored in low-bit integers,
 * for AMD Instinct MI355X (gfx950).
 *
 * Method sources (cited by page title and passage):
 *  [LoReS]  "Quantizing Recurrent Language Models Is Easier Than You Think"
 *           (arXiv 2611.01864), abstract: the recurrent state is a
 *           fixed-size matrix updated at every decode step; the state
 *           quantization pipeline combines value-axis scale grouping,
 *           decay-based mixed precision for slowly decaying heads or
 *           channels, and stochastic rounding under repeated requantization.
 *  [PU]     "Preserving Updates in Low-Bit Recurrent State Quantization"
 *           (arXiv 2610.15709), abstract: the state is requantized after
 *           every update; Low-Rank Bypass (LRB) accumulates small updates in
 *           a low-rank buffer and periodically merges its large elements;
 *           Bounded Directional Rounding (BDR) rounds reversed elements
 *           toward their updates; INT4 states; families Gated DeltaNet, GLA,
 *           Mamba2 and RetNet.
 *  [Philox] Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
 *           as 1, 2, 3" (SC'11): the Philox4x32-10 counter-based generator.
 *
 * Logical state of one (batch b, head h): S[v][k], v in [0,dv) the value
 * index (one output channel: a "value column" of the pages' S), k in
 * [0,dk) the key index.  Recurrences (one decode step, inputs of that step):
 *   additive (GLA per key channel decay; Mamba2 / RetNet scalar decay):
 *       S <- S diag(d) + u k^T,   u = beta * v
 *   delta rule (Gated DeltaNet), alpha = the (scalar) decay d:
 *       S <- alpha (S - beta S k k^T) + beta v k^T
 *          = alpha S + u k^T,      u = beta * (v - alpha * (S k))
 *   delta rule with a decay per key channel (channel-gated, Kimi-Linear):
 *       D = S diag(d),  S <- D - beta (D k) k^T + beta v k^T
 *          = D + u k^T,            u = beta * (v - D k), D's entries being
 *       the decayed values of the element update below
 *   readout: o = S_pre q, from the updated state before it is rounded.
 * Every step dequantizes the state, applies decay and update, computes o,
 * and requantizes (one fused kernel, one pass over the state in HBM).
 *
 * Stored state layout (bytes; all device memory owned by the caller):
 *   A key channel of head h is "quantized" unless the precision map marks
 *   it (map_mode HEAD: the whole head; KEY: that channel of that head).
 *   nq(h) = quantized channels of head h, nhp(h) = dk - nq(h).
 *   codes: per (b,h) a block of dv rows; a row holds the codes of the
 *     quantized channels in ascending k (slot j = the j-th quantized
 *     channel), ceil(nq*qbits/8) bytes padded to a multiple of 4 (qbits 8:
 *     int8; qbits 4: two's-complement nibbles, even slot in the low nibble);
 *     the block is padded to a multiple of 16 bytes; blocks follow head order
 *     within a batch element, then batch order.  Padding bytes stay zero.
 *   scales: fp32 [B][H][dv], one per row (value-axis grouping [LoReS]):
 *     scale = max_k |S_pre[v][k]| / Q over quantized k, Q = 127 (int8) or
 *     7 (int4); a row with max 0 has scale 0 and codes 0.  With scale_axis
 *     QS_AXIS_KEY: [B][H][dk], one per key channel (max over v); with
 *     QS_AXIS_HEAD: [B][H], one per head (max over the head) -- the groupings
 *     [LoReS] contrasts value-axis grouping with.
 *   hp: per (b,h) a block of dv rows of nhp(h) protected values in
 *     ascending k (bf16, fp16 or fp32 per hp_dtype), each row padded to a
 *     multiple of 4 bytes, the block to 16 bytes.
 *   lrb_W fp32 [B][H][dv][r], lrb_U fp32 [B][H][dk][r], lrb_n int32 [B][H]
 *     (LRB only): effective state = dequantized state + W U^T using the
 *     first lrb_n columns.
 *   bf16 layout (scale_dtype = lrb_dtype = QS_BF16, LRB on): scales, W and
 *     U are bf16 [same shapes]; at a 128 x 128 head with int4 codes and
 *     rank 8 the state is 5.22x smaller than fp32 (the "up to 5.3x" of
 *     [PU] counts codes and factors: 5.33x).  A row's scale is the smallest
 *     bf16 s with Q s >= max, and codes are taken against it: inv = the
 *     largest fp32 with inv s <= 1 (a row whose s overflows, or whose inverse
 *     times 2^sr_bits is not finite, is stored as zero).  A new basis column
 *     is rounded to bf16 (nearest even) when made and used rounded; U is
 *     updated in fp32 from its stored values and rounded to bf16 before the
 *     merge test, so merge, readout and stored state see the same buffer.
 *   All-zero buffers are the state S = 0.
 *
 * Rounding of a quantized element x = S_pre * inv, inv = Q / max rounded
 * toward zero (the largest fp32 with inv * max <= Q, so |x| <= Q; a row
 * whose nearest Q / max, times 2^sr_bits under stochastic rounding,
 * overflows is stored as zero):
 *   nearest: ties to even.  stochastic (fixed point, b = sr_bits):
 *   X = floor(x * 2^b + 1/2), code = floor((X + u) / 2^b), with u the
 *   element's b-bit Philox integer, key = seed, counter = (g as 64 bits,
 *   step as 64 bits); e = ((b*H+h)*dv+v)*dk+j, j the element's slot in its
 *   stored code row (j = k when the whole head is quantized);
 *   16 bits: g = e>>3, half (e&1) of word (e>>1)&3 (low half for even e);
 *   8 bits: g = e>>4, byte e&3 of word (e>>2)&3.  E[code] = X / 2^b
 *   (X uses invb = inv * 2^b).
 *   BDR: with D = S_pre - S_old and xo = S_old * inv, an element with
 *   D > 0 and code < xo - bound takes ceil(x); with D < 0 and code > xo +
 *   bound takes floor(x).  Codes lie in [-Q, Q] by the choice of inv.  Protected values
 *   are stored as the nearest (ties to even) bf16/fp16.
 *   Element update: S_pre = fma(u_v, k_k, (d_k * s_v) * code) for a
 *   quantized channel, fma(u_v, k_k, d_k * value) for a protected one.
 *
 * Low-Rank Bypass [PU] (lrb_rank r > 0, map NONE, both kinds), per (b,h),
 * with s_v the row scales on entry and n the basis size:
 *   1. U[k][:] *= d_k (the buffer decays with the state);
 *   2. delta rule only: u = beta * (v - w), w the decayed effective state
 *      times k: (decayed S_hat) k + W (U^T k);
 *   3. while n < r: the part of u orthogonal to W's n columns (two
 *      Gram-Schmidt passes) becomes column n, normalised, when its norm
 *      exceeds 2^-10 |u|;
 *   4. c = W^T u; key channel k is small when |k_k| * max_v |u_v| / s_v <
 *      theta: it adds k_k c to U[k] and only (u - W c) k_k to S_pre;
 *   5. when (step+1) % period == 0, a channel whose buffered column
 *      reaches theta * s_v in some row is added to S_pre and cleared; an
 *      all-clear buffer resets n to 0;
 *   6. o gains W (U^T q); requantization sees S_pre with the merged columns.
 *
 * Conventions: every call is asynchronous on `stream` (a hipStream_t; NULL
 * = the null stream).  The return code reports errors found on the host
 * (arguments) and launch failures; a fault inside a kernel surfaces at the
 * caller's next synchronizing HIP call.  qstate_decode_step allocates
 * nothing and never synchronizes.  A handle is read-only after init and
 * may be shared by threads; calls that write the same state race.
 */
#ifndef QSTATE_H
#define QSTATE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QSTATE_ABI_VERSION 2u

typedef enum {
  QS_OK = 0,
  QS_EINVAL = -1,        /* malformed argument (null, misaligned, out of range) */
  QS_EUNSUPPORTED = -2,  /* well-formed but outside the supported set */
  QS_ENOMEM = -3,        /* host or device allocation failed (init only) */
  QS_EHIP = -4           /* a HIP runtime call or kernel launch failed */
} qs_status;

typedef enum { QS_KIND_ADDITIVE = 0, QS_KIND_DELTA = 1 } qs_kind;
typedef enum { QS_DECAY_HEAD = 0, QS_DECAY_KEY = 1 } qs_decay_mode;
typedef enum { QS_FP32 = 0, QS_BF16 = 1, QS_FP16 = 2 } qs_dtype;
typedef enum { QS_MAP_NONE = 0, QS_MAP_HEAD = 1, QS_MAP_KEY = 2 } qs_map_mode;
typedef enum { QS_ROUND_NEAREST = 0, QS_ROUND_STOCHASTIC = 1 } qs_rounding;
typedef enum { QS_AXIS_VALUE = 0, QS_AXIS_KEY = 1, QS_AXIS_HEAD = 2 } qs_scale_axis;

typedef struct {
  uint32_t abi_version;   /* QSTATE_ABI_VERSION */
  int32_t kind;           /* qs_kind */
  int32_t decay_mode;     /* qs_decay_mode (both kinds) */
  int32_t B, H;           /* batch (>= 0; 0 = every call is a no-op), heads (>= 1);
                             B*H*dv*dk must stay below 2^35 */
  int32_t dk;             /* key dim: 64, 128 or 256 */
  int32_t dv;             /* value dim: 1..256 */
  int32_t qbits;          /* 8 or 4 */
  int32_t hp_dtype;       /* storage of protected channels: QS_BF16, QS_FP16, QS_FP32 */
  int32_t map_mode;       /* qs_map_mode */
  const uint8_t* map;     /* host: [H] (HEAD) or [H*dk] (KEY), nonzero = protected;
                             copied by qstate_init */
  int32_t in_dtype;       /* q, k, v element type: QS_BF16 or QS_FP32 */
  int32_t rounding;       /* qs_rounding */
  int32_t sr_bits;        /* stochastic rounding: 16 or 8 random bits per element */
  int32_t bdr;            /* 1 = bounded directional rounding [PU] */
  float bdr_bound;        /* tolerated reversal in LSB (>= 0) */
  int32_t lrb_rank;       /* 0 = off; 1..16 = low-rank bypass rank [PU] (map NONE) */
  int32_t lrb_period;     /* merge when (step+1) % period == 0 */
  float lrb_theta;        /* merge / smallness threshold in LSB (> 0) */
  uint64_t seed;          /* Philox key for stochastic rounding */
  int32_t scale_dtype;    /* row scales: QS_FP32, or QS_BF16 (low-rank bypass on, with
                             lrb_dtype QS_BF16) */
  int32_t lrb_dtype;      /* low-rank buffer factors W, U: QS_FP32, or QS_BF16 (with
                             scale_dtype QS_BF16, lrb_rank <= 8) */
  int32_t scale_axis;     /* qs_scale_axis: scale groups are rows (QS_AXIS_VALUE, the
                             method's grouping), key channels or whole heads (ablations;
                             map NONE, no low-rank bypass, fp32 scales) */
} qstate_config;

/* Byte sizes of the caller-owned device buffers (0 = buffer unused). */
typedef struct {
  uint64_t codes, scales, hp, lrb_W, lrb_U, lrb_n;
} qstate_sizes;

/* Device pointers of one stored state (16-byte aligned; unused ones may be NULL).
 * scales, lrb_W and lrb_U hold fp32 or bf16 elements per scale_dtype / lrb_dtype. */
typedef struct {
  void* codes;
  void* scales;
  void* hp;
  void* lrb_W;
  void* lrb_U;
  int32_t* lrb_n;
} qstate_tensors;

/* Device pointers of one step's inputs (16-byte aligned).
 * q, k: [B][H][dk] and v: [B][H][dv] in in_dtype; decay: fp32 [B][H]
 * (HEAD) or [B][H][dk] (KEY), the multiplicative decay of this step (for
 * Mamba2: exp(dt*A)); beta: fp32 [B][H] or NULL (= 1; for Mamba2: dt). */
typedef struct {
  const void* q;
  const void* k;
  const void* v;
  const float* decay;
  const float* beta;
} qstate_inputs;

typedef struct qstate_handle qstate_handle;

/* Validate `cfg` and compute buffer sizes.  Host only (no HIP call); usable
 * without a GPU.  Errors: QS_EINVAL, QS_EUNSUPPORTED. */
qs_status qstate_plan(const qstate_config* cfg, qstate_sizes* sizes);

/* Validate, plan, and build a handle for the current HIP device: copies the
 * precision map and uploads the per-head layout tables (the handle owns
 * them).  `sizes` (optional) receives the buffer sizes.  Decay-based mixed
 * precision [LoReS] enters here through cfg->map.
 * Errors: QS_EINVAL, QS_EUNSUPPORTED, QS_ENOMEM, QS_EHIP. */
qs_status qstate_init(const qstate_config* cfg, qstate_handle** out, qstate_sizes* sizes);

/* fp32 logical state S [B][H][dv][dk] (device) -> stored state `dst`, with
 * the configured rounding (nearest or stochastic at Philox step `step`;
 * no BDR: there is no previous value) and an empty LRB buffer.  Used to
 * hand a state over (e.g. after a prefill) and as the exact parity hook of
 * the quantizer ([LoReS] value-axis scales and stochastic rounding). */
qs_status qstate_quantize(qstate_handle* h, const float* S, const qstate_tensors* dst,
                          uint64_t step, void* stream);

/* One decode step for every (b,h), in place on `state` [LoReS, PU]:
 * dequantize, decay + update (additive or delta rule), LRB bypass and
 * merge when on, readout o = S_pre q (+ W U^T q) into out fp32 [B][H][dv],
 * requantize with value-axis scales, stochastic or nearest rounding, BDR
 * when on; protected channels stored in hp_dtype.  `step` is the Philox
 * counter word and the LRB merge clock.  Never allocates or synchronizes. */
qs_status qstate_decode_step(qstate_handle* h, const qstate_tensors* state,
                             const qstate_inputs* in, float* out, uint64_t step,
                             void* stream);

/* One decode step for a batch of n sequences whose states live in a pool
 * of B state slots (the handle's B), as a server with continuous batching
 * keeps them; the operation on each (sequence, head) is that of
 * qstate_decode_step [LoReS, PU].
 *   pool: the stored state of all B slots, in place.
 *   in, out: the batch's inputs and outputs, laid out as for
 *     qstate_decode_step with B replaced by n (batch element b first).
 *   slot: device int32 [n]; batch element b reads and writes state slot
 *     slot[b].  An element whose slot lies outside [0, B) is skipped: no
 *     state is touched and its outputs are not written.  Two elements with
 *     the same slot race.
 *   step: device uint64 [n]; element b's step: its Philox counter word (with
 *     the element index taken in the pool, e = ((slot*H+h)*dv+v)*dk+j, so
 *     its random bits do not depend on its batch position) and the LRB merge
 *     clock.
 * n = 0 is a no-op; n > B is QS_EINVAL.  Never allocates or synchronizes. */
qs_status qstate_decode_step_batch(qstate_handle* h, const qstate_tensors* pool,
                                   const qstate_inputs* in, float* out, int32_t n,
                                   const int32_t* slot, const uint64_t* step, void* stream);

/* Stored state -> fp32 effective state S [B][H][dv][dk] (device), the
 * state the method's readout sees: scale * code for quantized channels (one
 * scale per row, the value-axis grouping of [LoReS]), the widened 16-bit or
 * fp32 value for protected ones (decay-based mixed precision, [LoReS]), plus
 * the low-rank buffer W U^T when LRB is on ([PU]: small updates held in the
 * buffer are part of the state until merged).  Not on the decode path: for
 * checks, checkpoints and hand-back.  Errors: QS_EINVAL (null handle or
 * pointers, misaligned pointer). */
qs_status qstate_dequantize(qstate_handle* h, const qstate_tensors* src, float* S,
                            void* stream);

/* Decay-based mixed precision map [LoReS]: within each of `groups` groups
 * of `per_group` units (heads, or key channels of one head), mark the
 * floor(frac*per_group + 0.5) units with the smallest decay-rate statistic
 * `stat` (e.g. |A_h| for Mamba2, -log(decay)); ties go to the lower index.
 * Host only.  map: [groups*per_group] output.  Errors: QS_EINVAL. */
qs_status qstate_build_map(const float* stat, int32_t groups, int32_t per_group,
                           float frac, uint8_t* map);

/* Release a handle (NULL is a no-op).  The caller synchronizes first. */
void qstate_destroy(qstate_handle* h);

/* Static text for a status code. */
const char* qstate_strerror(qs_status s);

/* Detail of the last error reported on the calling thread ("" if none). */
const char* qstate_last_error(void);

/* Name of the step kernel instantiation the handle launches (for logs and
 * profiles); NULL handle -> "". */
const char* qstate_kernel_name(const qstate_handle* h);

#ifdef __cplusplus
}
#endif
#endif /* QSTATE_H */
