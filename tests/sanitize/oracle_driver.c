/* CPU driver of the oracle under AddressSanitizer and UndefinedBehaviorSanitizer
 * (built by tests/test_sanitizers.py with gcc): quantize, steps, traced steps,
 * batched steps and dequantize over small configurations of every feature
 * (both kinds and decay modes, int8/int4, nearest/stochastic/BDR, head and key
 * maps in every storage, the low-rank bypass with fp32 and bf16 layouts, key
 * and head scale groups), plus the map builder and Philox. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "qs_oracle.h"

static uint64_t rng = 88172645463325252ull;
static double urand(void) {
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (double)(rng >> 11) / 9007199254740992.0;
}
static float nrand(void) {
  double u = urand() + 1e-12, v = urand();
  return (float)(sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v));
}

static int run(orc_cfg* c, int steps) {
  orc_sizes z;
  const int dk = c->dk, dv = c->dv;
  const int64_t BH = (int64_t)c->B * c->H;
  if (orc_layout(c, &z, NULL, NULL, NULL)) return 0;
  orc_state st;
  st.codes = (uint8_t*)calloc(z.codes + 1, 1);
  st.scales = calloc(z.scales + 1, 1);
  st.hp = calloc(z.hp + 1, 1);
  st.W = calloc(z.W + 1, 1);
  st.U = calloc(z.U + 1, 1);
  st.n = (int32_t*)calloc(z.n / 4 + 1, 4);
  float* S = (float*)malloc(sizeof(float) * (size_t)(BH * dv * dk));
  float* q = (float*)malloc(sizeof(float) * (size_t)(BH * dk));
  float* k = (float*)malloc(sizeof(float) * (size_t)(BH * dk));
  float* v = (float*)malloc(sizeof(float) * (size_t)(BH * dv));
  float* d = (float*)malloc(sizeof(float) * (size_t)(BH * dk));
  float* beta = (float*)malloc(sizeof(float) * (size_t)BH);
  float* out = (float*)malloc(sizeof(float) * (size_t)(BH * dv));
  float* sp = (float*)malloc(sizeof(float) * (size_t)(BH * dv * dk));
  for (int64_t i = 0; i < BH * dv * dk; ++i) S[i] = nrand() * (float)exp(4.0 * urand() - 2.0);
  if (orc_quantize(c, S, &st, 1)) return -1;
  int32_t* small = (int32_t*)malloc(sizeof(int32_t) * (size_t)(BH * dk));
  int32_t* merged = (int32_t*)malloc(sizeof(int32_t) * (size_t)(BH * dk));
  int32_t* nb = (int32_t*)malloc(sizeof(int32_t) * (size_t)BH);
  int32_t* na = (int32_t*)malloc(sizeof(int32_t) * (size_t)BH);
  orc_lrb_trace tr = {small, merged, nb, na};
  for (int t = 0; t < steps; ++t) {
    for (int64_t i = 0; i < BH * dk; ++i) {
      q[i] = nrand();
      k[i] = nrand() * (i % 2 ? 0.05f : 1.0f);
      d[i] = (float)(1.0 / (1.0 + exp(-(nrand() + 3.0))));
    }
    for (int64_t i = 0; i < BH * dv; ++i) v[i] = nrand();
    for (int64_t i = 0; i < BH; ++i) beta[i] = (float)(1.0 / (1.0 + exp(-nrand())));
    int rc;
    if (c->lrb_rank > 0 && t % 2) rc = orc_step_lrb_trace(c, &st, q, k, v, d, beta, out, (uint64_t)t, sp, &tr);
    else rc = orc_step(c, &st, q, k, v, d, (t % 3) ? beta : NULL, out, (uint64_t)t, (t % 2) ? sp : NULL, NULL, 0);
    if (rc) return -1;
  }
  if (c->B >= 2) {
    int32_t slot[2] = {1, -1};
    uint64_t stp[2] = {5, 6};
    if (orc_step_batch(c, &st, q, k, v, d, beta, out, 2, slot, stp)) return -1;
  }
  if (orc_dequantize(c, &st, S)) return -1;
  for (int64_t i = 0; i < BH * dv * dk; ++i)
    if (isnan(S[i])) return -1;
  free(st.codes); free(st.scales); free(st.hp); free(st.W); free(st.U); free(st.n);
  free(S); free(q); free(k); free(v); free(d); free(beta); free(out); free(sp);
  free(small); free(merged); free(nb); free(na);
  return 1;
}

int main(void) {
  int ran = 0, bad = 0;
  const int dks[3] = {4, 16, 64};
  for (int it = 0; it < 600; ++it) {
    orc_cfg c;
    memset(&c, 0, sizeof c);
    c.kind = it % 2;
    c.decay_mode = (it / 2) % 2;
    c.B = 1 + it % 3;
    c.H = 1 + (it / 3) % 3;
    c.dk = dks[(it / 9) % 3];
    c.dv = 1 + (int)(urand() * 20);
    c.qbits = (it / 27) % 2 ? 4 : 8;
    c.hp_dtype = (int)(urand() * 3);
    c.rounding = (it / 54) % 2;
    c.sr_bits = urand() < 0.5 ? 16 : 8;
    c.bdr = urand() < 0.4;
    c.bdr_bound = urand() < 0.5 ? 0.0f : 0.4f;
    c.seed = (uint64_t)it * 7919u;
    const int feature = it % 5;   /* 0 plain, 1 head map, 2 key map, 3 buffer, 4 other scale groups */
    uint8_t map[3 * 64];
    for (int i = 0; i < 3 * 64; ++i) map[i] = urand() < 0.3;
    if (feature == 1 || feature == 2) {
      c.map_mode = feature;
      c.map = map;
    } else if (feature == 3) {
      c.lrb_rank = 1 + (int)(urand() * 8);
      c.lrb_period = 2 + (int)(urand() * 3);
      c.lrb_theta = 0.5f;
      if (urand() < 0.5) c.scale_dtype = c.lrb_dtype = 1;
    } else if (feature == 4) {
      c.scale_axis = 1 + (int)(urand() * 2);
    }
    int rc = run(&c, 7);
    if (rc < 0) ++bad;
    if (rc > 0) ++ran;
  }
  /* the map builder: ties, infinities */
  double stat[40];
  uint8_t m[40];
  for (int i = 0; i < 40; ++i) stat[i] = (i % 5) * 0.25;
  stat[3] = INFINITY;
  if (orc_build_map(stat, 4, 10, 0.3, m)) ++bad;
  uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, o4[4];
  orc_philox4x32_10(ctr, key, o4);
  printf("oracle driver: %d configurations run, %d failures\n", ran, bad);
  return (bad == 0 && ran > 500) ? 0 : 1;
}
