/*
 * cce_oracle.c -- plain fp64 CPU reference for the flash cut-cross-entropy head.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file: it is used by tests/, by __graft_entry__.smoke() and by the
 * cpu_baseline leg of bench.py.  It shares no code, header or table with the
 * HIP library (linear_cross_entropy_libcce_amd/csrc); the two meet only in the
 * seeded input arrays handed to both.
 *
 * What it computes is the plain definition, one token at a time, in double
 * precision, with no blocking, fusion or reordering:
 *
 *   1. dequantize every head element from its packed code
 *      (page "mlx-bun 0.0.4 -> 0.0.6", src/train/flash-cce.ts: the
 *      FlashCceHead interface -- packed uint32 [V, H*bits/32], per-group affine
 *      scale and bias of shape [V, H/group] -- and the scalar forward kernel,
 *      which reads element k of a word as (word >> bits*k) & (2^bits-1) and
 *      forms scale*q + bias);
 *   2. logit z_v = sum_d h_d * w[v][d]; optional softcap y = cap*tanh(z/cap),
 *      identity when cap == 0 (same file, scalar forward kernel epilogue);
 *   3. lse = log sum_v exp(y_v); logp = y_target - lse (same file, header
 *      comment and the host-side cross-block merge in flashCceForward);
 *   4. backward coefficient coeff_v = g * (1[v == target] - exp(y_v - lse))
 *      * c'(z_v) with c' = 1 - tanh^2(z/cap) under a softcap, else 1, and
 *      dh = sum_v coeff_v * w[v][:] (same file, scalar backward kernel's
 *      phase 1 and phase 2).
 *
 * Readings where the pages leave a step open:
 *   - a target outside [0, V) matches no row: its target term is 0, so
 *     logp = -lse and there is no one-hot term in the gradient;
 *   - a masked token (mask[t] == 0) has logp = lse = 0 and a zero dh row;
 *   - g is the cotangent of logp: dh_t = g_t * d logp_t / d h_t.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 bits -> double: a bf16 value is the top half of an fp32. */
static double bf16_bits_to_double(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* One dequantized head element w[v][d] (step 1 above). */
static double head_elem(const uint32_t *wq, const float *scales,
                        const float *biases, int64_t H, int bits, int group,
                        int64_t v, int64_t d) {
  const int64_t per_word = 32 / bits;
  const int64_t words_per_row = H * bits / 32;
  const int64_t groups_per_row = H / group;
  const uint32_t code_mask = (bits == 32) ? 0xffffffffu : ((1u << bits) - 1u);
  const uint32_t word = wq[v * words_per_row + d / per_word];
  const uint32_t q = (word >> (bits * (d % per_word))) & code_mask;
  const int64_t gi = v * groups_per_row + d / group;
  return (double)scales[gi] * (double)q + (double)biases[gi];
}

int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Evaluate the tokens listed in `tokens` (ntok entries; NULL means all M).
 * Outputs are indexed by position in that list: logp[i], lse[i] and, when dh
 * is not NULL, dh[i*H .. i*H+H).  g may be NULL (then g_t = 1); mask may be
 * NULL (all tokens active).  Returns 0, or -1 on bad arguments / no memory.
 */
int oracle_cce(const uint16_t *h, int64_t M, int64_t H, const uint32_t *wq,
               const float *scales, const float *biases, int64_t V, int bits,
               int group, double softcap, const int32_t *targets,
               const uint8_t *mask, const double *g, const int64_t *tokens,
               int64_t ntok, double *logp, double *lse, double *dh) {
  if (!h || !wq || !scales || !biases || !targets || !logp || !lse) return -1;
  if (M < 0 || H <= 0 || V <= 0 || group <= 0 || H % group != 0) return -1;
  if (bits != 4 && bits != 8) return -1;
  if (softcap < 0) return -1;
  if (!tokens) ntok = M;

  double *hd = malloc(sizeof(double) * H);
  double *z = malloc(sizeof(double) * V);
  double *y = malloc(sizeof(double) * V);
  double *coeff = malloc(sizeof(double) * V);
  if (!hd || !z || !y || !coeff) {
    free(hd); free(z); free(y); free(coeff);
    return -1;
  }

  for (int64_t i = 0; i < ntok; ++i) {
    const int64_t t = tokens ? tokens[i] : i;
    if (t < 0 || t >= M) { free(hd); free(z); free(y); free(coeff); return -1; }
    if (mask && mask[t] == 0) {
      logp[i] = 0.0;
      lse[i] = 0.0;
      if (dh) memset(dh + i * H, 0, sizeof(double) * H);
      continue;
    }
    for (int64_t d = 0; d < H; ++d) hd[d] = bf16_bits_to_double(h[t * H + d]);

    /* step 2: every logit of this token */
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < V; ++v) {
      double acc = 0.0;
      for (int64_t d = 0; d < H; ++d)
        acc += hd[d] * head_elem(wq, scales, biases, H, bits, group, v, d);
      z[v] = acc;
    }
    for (int64_t v = 0; v < V; ++v)
      y[v] = (softcap > 0.0) ? softcap * tanh(z[v] / softcap) : z[v];

    /* step 3: log-sum-exp (max-shifted) and the log-prob of the target */
    double mx = -INFINITY;
    for (int64_t v = 0; v < V; ++v) mx = y[v] > mx ? y[v] : mx;
    double se = 0.0;
    for (int64_t v = 0; v < V; ++v) se += exp(y[v] - mx);
    const double l = mx + log(se);
    const int32_t tg = targets[t];
    const int tgt_in = (tg >= 0 && (int64_t)tg < V);
    lse[i] = l;
    logp[i] = (tgt_in ? y[tg] : 0.0) - l;

    if (!dh) continue;
    /* step 4: coefficients, then dh = sum_v coeff_v * w[v][:] */
    const double gt = g ? g[t] : 1.0;
    for (int64_t v = 0; v < V; ++v) {
      double dc = 1.0;
      if (softcap > 0.0) {
        const double th = tanh(z[v] / softcap);
        dc = 1.0 - th * th;
      }
      const double onehot = (tgt_in && v == (int64_t)tg) ? 1.0 : 0.0;
      coeff[v] = gt * (onehot - exp(y[v] - l)) * dc;
    }
    /* Each dh[d] is summed over v in increasing order; the d axis is cut
     * into 64-wide slices only so that each thread walks W row by row. */
    double *out = dh + i * H;
    const int64_t nslice = (H + 63) / 64;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < nslice; ++c) {
      const int64_t d0 = c * 64, d1 = (d0 + 64 < H) ? d0 + 64 : H;
      for (int64_t d = d0; d < d1; ++d) out[d] = 0.0;
      for (int64_t v = 0; v < V; ++v)
        for (int64_t d = d0; d < d1; ++d)
          out[d] += coeff[v] * head_elem(wq, scales, biases, H, bits, group, v, d);
    }
  }
  free(hd); free(z); free(y); free(coeff);
  return 0;
}
