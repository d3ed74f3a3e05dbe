/*
 * ref_decode.c -- fp64 CPU oracle for decode attention: one new query per
 * (sequence, query head) against that sequence's cached keys and values.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct reference
 * that the HIP decode kernels are checked against.  Only tests/, the smoke check
 * and the CPU-baseline leg of the benchmark may load it.  It shares no code,
 * header, table or helper with the HIP library, and it never calls it.
 *
 * What it computes (plain definition, all arithmetic in double).  For batch
 * entry b with n = len[b] cached positions, query head h and its kv head
 * g = floor(h / group), group = H / Hkv:
 *     s_j = scale * sum_d q[b,h,d] * K[b,g,j,d]            for j < n
 *     m   = max_j s_j,   l = sum_j exp(s_j - m)
 *     o[b,h,:] = sum_j exp(s_j - m) * V[b,g,j,:] / l,   lse[b,h] = m + ln(l)
 * With n = 0 there is nothing to attend to: o = 0 and lse = -inf (the log of
 * an empty sum).  Positions j >= n are never read.
 *
 * Sources (the pages this follows):
 *   - "xtrain evolution overview", post-training stage, milestone M2a: decode
 *     attention is one query against the cached K/V, built from a plain
 *     strided product and an ordinary softmax, and must equal the last row of
 *     full causal attention; M2b: a group of rows decoded together shares the
 *     kernel (bh = G * nh) and GQA broadcasts each kv head to its group;
 *     M2c: the cache lives on the device as [bh, T, hd] per layer.
 *   - same page, infra table row T15: query head kvh*group + r reads kv head
 *     kvh, i.e. kv head floor(h / group).
 *
 * Layout (all contiguous, row-major): q, o: [B][H][hd]; k, v: [B][Hkv][T][hd]
 * (T = cache capacity, the first len[b] positions of sequence b are valid);
 * lse: [B][H]; len: [B] (NULL means every sequence holds T positions).
 */
#include <math.h>
#include <stddef.h>

enum { REFD_OK = 0, REFD_ERR_ARG = 1 };

int xattn_ref_decode(const double* q, const double* k, const double* v, const int* len,
                     double* o, double* lse, int B, int T, int H, int Hkv, int hd,
                     double scale) {
  if (!q || !k || !v || !o || !lse) return REFD_ERR_ARG;
  if (B <= 0 || T <= 0 || H <= 0 || Hkv <= 0 || hd <= 0 || H % Hkv != 0) return REFD_ERR_ARG;
  const int group = H / Hkv;
  for (int b = 0; b < B; ++b) {
    const int n = len ? len[b] : T;
    if (n < 0 || n > T) return REFD_ERR_ARG;
  }
  for (int b = 0; b < B; ++b) {
    const int n = len ? len[b] : T;
    for (int h = 0; h < H; ++h) {
      const int g = h / group;
      const double* qh = q + ((size_t)b * H + h) * hd;
      const double* kg = k + ((size_t)b * Hkv + g) * (size_t)T * hd;
      const double* vg = v + ((size_t)b * Hkv + g) * (size_t)T * hd;
      double* oh = o + ((size_t)b * H + h) * hd;
      if (n == 0) {
        for (int d = 0; d < hd; ++d) oh[d] = 0.0;
        lse[(size_t)b * H + h] = -INFINITY;
        continue;
      }
      /* scores and their maximum */
      double m = -INFINITY;
      for (int j = 0; j < n; ++j) {
        double s = 0.0;
        for (int d = 0; d < hd; ++d) s += qh[d] * kg[(size_t)j * hd + d];
        s *= scale;
        if (s > m) m = s;
      }
      /* softmax weights (recomputed from the scores) and the weighted values */
      double l = 0.0;
      for (int d = 0; d < hd; ++d) oh[d] = 0.0;
      for (int j = 0; j < n; ++j) {
        double s = 0.0;
        for (int d = 0; d < hd; ++d) s += qh[d] * kg[(size_t)j * hd + d];
        const double p = exp(scale * s - m);
        l += p;
        for (int d = 0; d < hd; ++d) oh[d] += p * vg[(size_t)j * hd + d];
      }
      for (int d = 0; d < hd; ++d) oh[d] /= l;
      lse[(size_t)b * H + h] = m + log(l);
    }
  }
  return REFD_OK;
}
