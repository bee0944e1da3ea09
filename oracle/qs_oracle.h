/*
 * qs_oracle.h -- CPU oracle for the quantized recurrent-state decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  This oracle is a plain, slow, scalar C
 * implementation of what the decode step computes.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it.
 * It shares no code, header, table or constant with the HIP library.
 *
 * What it follows (pages as cited in the repository's design notes):
 *  - "Quantizing Recurrent Language Models Is Easier Than You Think"
 *    (LoReS, arXiv 2611.01864), abstract: value-axis scale grouping,
 *    decay-based mixed precision for slowly decaying heads or channels,
 *    stochastic rounding under repeated requantization.
 *  - "Preserving Updates in Low-Bit Recurrent State Quantization"
 *    (arXiv 2610.15709), abstract: requantization after every update,
 *    Low-Rank Bypass (LRB), Bounded Directional Rounding (BDR), INT4.
 *  - Philox4x32-10 from Salmon, Moraes, Dror, Shaw, "Parallel Random
 *    Numbers: As Easy as 1, 2, 3" (SC'11), section on the Philox family.
 *
 * Element arithmetic is fp32 (the stored state format is fp32 scales times
 * integer codes, so that is the precision every rounding decision is taken
 * in); every reduction (dot products, norms) accumulates in fp64 and is
 * rounded to fp32 once.  Build with -ffp-contract=off: each fused
 * multiply-add below is an explicit fmaf().
 */
#ifndef QS_ORACLE_H
#define QS_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t kind;        /* 0 additive (GLA, Mamba2, RetNet), 1 delta rule (Gated DeltaNet) */
  int32_t decay_mode;  /* 0 one decay per (b,h); 1 one decay per (b,h,k) */
  int32_t B, H, dk, dv;
  int32_t qbits;       /* 8 or 4 */
  int32_t hp_dtype;    /* storage of protected units: 0 fp32, 1 bf16, 2 fp16 */
  int32_t map_mode;    /* 0 none, 1 one flag per head, 2 one flag per (head, key channel) */
  const uint8_t* map;  /* [H] or [H*dk]; nonzero = kept in high precision */
  int32_t rounding;    /* 0 round to nearest even, 1 stochastic */
  int32_t sr_bits;     /* random bits per element for stochastic rounding: 16 or 8 */
  int32_t bdr;         /* bounded directional rounding on/off */
  float   bdr_bound;   /* tolerated reversal, in LSB of the new grid */
  int32_t lrb_rank;    /* 0 = low-rank bypass off */
  int32_t lrb_period;  /* merge when (step+1) % period == 0 */
  float   lrb_theta;   /* merge / smallness threshold, in LSB */
  uint64_t seed;       /* Philox key */
  int32_t scale_dtype; /* storage of row scales: 0 fp32, 1 bf16 (rounded up, see requantize_row) */
  int32_t lrb_dtype;   /* storage of the low-rank buffer factors W and U: 0 fp32, 1 bf16 */
  int32_t scale_axis;  /* scale groups: 0 value axis (one scale per row v), 1 key axis (one
                          per column k), 2 one per head; 1 and 2 need map 0 and no buffer.
                          scales are [B,H,G], G = dv, dk or 1 */
} orc_cfg;

typedef struct {
  uint8_t* codes;   /* packed codes, per-head blocks */
  void*    scales;  /* [B,H,G] (G per scale_axis), fp32 or bf16 bits per scale_dtype */
  void*    hp;      /* protected values, per-head blocks (uint16 bits or fp32) */
  void*    W;       /* [B,H,dv,r], fp32 or bf16 bits per lrb_dtype */
  void*    U;       /* [B,H,dk,r], fp32 or bf16 bits per lrb_dtype */
  int32_t* n;       /* [B,H] */
} orc_state;

typedef struct {
  uint64_t codes, scales, hp, W, U, n;   /* bytes */
  uint64_t code_bstride, hp_bstride;     /* bytes per batch element */
} orc_sizes;

int  orc_layout(const orc_cfg* c, orc_sizes* s, uint64_t* code_off, uint64_t* hp_off,
                int32_t* nq);
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
uint32_t orc_random_bits(const orc_cfg* c, uint64_t e, uint64_t step);
float orc_sr_round(float xb, uint32_t rbits, int32_t sr_bits);  /* xb = x * 2^sr_bits */
float orc_inv_rtz(float q, float m);   /* q / m rounded toward zero */
float orc_scale_bf16_up(float m, float q);   /* smallest bf16 s with q s >= m (+inf if none) */
uint16_t orc_to_bf16(float f);
uint16_t orc_to_fp16(float f);
float orc_from_bf16(uint16_t h);
float orc_from_fp16(uint16_t h);
int  orc_build_map(const double* stat, int32_t groups, int32_t per_group, double frac,
                   uint8_t* map);
int  orc_quantize(const orc_cfg* c, const float* S, orc_state* st, uint64_t step);
int  orc_dequantize(const orc_cfg* c, const orc_state* st, float* S);
int  orc_step(const orc_cfg* c, orc_state* st, const float* q, const float* k,
              const float* v, const float* decay, const float* beta, float* out,
              uint64_t step, float* sp_dbg, const int64_t* heads, int64_t nheads);
/* A step for n sequences held in slots of the pool (the config's B states):
 * element b's inputs and output at b, its state at slot[b] (skipped when
 * outside [0, B)), its step step[b].  Returns 0, or -1 for n outside [0, B]. */
int  orc_step_batch(const orc_cfg* c, orc_state* st, const float* q, const float* k,
                    const float* v, const float* decay, const float* beta, float* out,
                    int32_t n, const int32_t* slot, const uint64_t* step);

/* Decisions of the low-rank bypass in one step, per (b,h) and key channel:
 * small[bh*dk+k] = channel k was small (its in-span update went to the
 * buffer), merged[bh*dk+k] = channel k was merged into the state; the basis
 * size before and after the step. */
typedef struct {
  int32_t* small;
  int32_t* merged;
  int32_t* n_before;
  int32_t* n_after;
} orc_lrb_trace;
int  orc_step_lrb_trace(const orc_cfg* c, orc_state* st, const float* q, const float* k,
                        const float* v, const float* decay, const float* beta, float* out,
                        uint64_t step, float* sp_dbg, const orc_lrb_trace* tr);

#ifdef __cplusplus
}
#endif
#endif
