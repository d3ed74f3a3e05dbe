/*
 * ref_attn.c -- fp64 CPU oracle for batched causal scaled-dot-product attention,
 * forward and analytic backward, with grouped-query (GQA) key/value heads.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct reference
 * that the HIP path is checked against.  Only tests/, the smoke check and the
 * CPU-baseline leg of the benchmark may load it.  It shares no code, header,
 * table or helper with the HIP library, and it never calls it.
 *
 * What it computes (plain definition, all arithmetic in double):
 *   For every batch b and query head h, with group = H / Hkv and kv head
 *   g = floor(h / group):
 *     s_ij  = scale * sum_d Q[b,h,i,d] * K[b,g,j,d]          for j <= i only
 *     P_ij  = exp(s_ij - m_i) / l_i,  m_i = max_{j<=i} s_ij,  l_i = sum_{j<=i} exp(s_ij - m_i)
 *     O_i   = sum_{j<=i} P_ij V_j ;   LSE_i = m_i + ln(l_i)   (natural log, scale included)
 *   Backward for an upstream gradient dO:
 *     dP_ij = dO_i . V_j
 *     dS_ij = P_ij * (dP_ij - sum_{k<=i} P_ik dP_ik)          (softmax Jacobian product, written out)
 *     dQ_i  = scale * sum_{j<=i} dS_ij K_j
 *     dK_j  = scale * sum_{h in group} sum_{i>=j} dS_ij Q_i
 *     dV_j  =         sum_{h in group} sum_{i>=j} P_ij dO_i
 *
 * Sources (the pages this follows):
 *   - "xtrain -- Known Issues & Perf Backlog", KI-1 fix: attention is a batched
 *     scaled dot product, Q.K^T then a causal softmax then P.V, over a
 *     head-major [B, heads, S, hd] layout.
 *   - "xtrain evolution overview", section 一 (infra phases), row T14: the fused
 *     kernel's online softmax and its backward that recomputes the scores; the
 *     backward's per-row D = sum(dO * O) is an identity of the row sum written
 *     out above, which the tests check instead of assuming it here.
 *   - same table, row T15: GQA by repeating each kv head group = nh/num_kv times
 *     with destination head kvh*group + r, and a backward that sums the group's
 *     gradients deterministically without atomics.  This oracle does GQA in
 *     exactly that way: it materialises the repeated K/V, runs plain multi-head
 *     attention, and sums dK/dV over r in ascending order.
 *
 * Readings taken where the pages are silent: causal mask is top-left aligned with
 * Sq == Sk (key j visible to query i iff j <= i); masked keys are excluded from the
 * sums (weight exactly 0), not given a large negative score; LSE uses the natural
 * log and includes the scale.
 *
 * Layout (all contiguous, row-major): q, o, dO, dq: [B][H][S][hd];
 * k, v, dk, dv: [B][Hkv][S][hd]; lse: [B][H][S].
 *
 * Parallelism: optional OpenMP over independent (b, kv head) units only.  Each
 * unit is computed by one thread in a fixed order, so results do not depend on
 * the thread count.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { REF_OK = 0, REF_ERR_ARG = 1, REF_ERR_NOMEM = 2 };

static int g_threads = 0; /* 0 = OpenMP default */

void xattn_ref_set_threads(int n) { g_threads = n > 0 ? n : 0; }

int xattn_ref_max_threads(void) {
#ifdef _OPENMP
  return g_threads > 0 ? g_threads : omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---------------------------------------------------------------------------
 * One head of plain causal attention.  q, k, v, dO: [S][hd].
 * Any output pointer may be NULL.  When a backward output (dq, dk, dv, dP, dS,
 * rowdot) is wanted, dO must be given.  P is [S][S] with zeros above the
 * diagonal; dP and dS likewise.  dk and dv are OVERWRITTEN (not accumulated).
 * ------------------------------------------------------------------------- */
static int head_ref(const double* q, const double* k, const double* v, const double* dO,
                    int S, int hd, double scale,
                    double* P_out, double* dP_out, double* dS_out, double* rowdot_out,
                    double* o, double* lse, double* dq, double* dk, double* dv) {
  const size_t SS = (size_t)S * (size_t)S;
  double* P = (double*)calloc(SS, sizeof(double));
  if (!P) return REF_ERR_NOMEM;
  const int want_bwd = (dq || dk || dv || dP_out || dS_out || rowdot_out);
  double* dS = NULL;
  double* dPm = NULL;
  if (want_bwd) {
    dS = (double*)calloc(SS, sizeof(double));
    dPm = (double*)calloc(SS, sizeof(double));
    if (!dS || !dPm) { free(P); free(dS); free(dPm); return REF_ERR_NOMEM; }
  }

  /* scores and softmax, row by row over the visible keys j <= i */
  for (int i = 0; i < S; ++i) {
    double* Pi = P + (size_t)i * S;
    double m = -INFINITY;
    for (int j = 0; j <= i; ++j) {
      double s = 0.0;
      for (int d = 0; d < hd; ++d) s += q[(size_t)i * hd + d] * k[(size_t)j * hd + d];
      s *= scale;
      Pi[j] = s;
      if (s > m) m = s;
    }
    double l = 0.0;
    for (int j = 0; j <= i; ++j) {
      Pi[j] = exp(Pi[j] - m);
      l += Pi[j];
    }
    for (int j = 0; j <= i; ++j) Pi[j] /= l;
    if (lse) lse[i] = m + log(l);
    if (o) {
      for (int d = 0; d < hd; ++d) {
        double acc = 0.0;
        for (int j = 0; j <= i; ++j) acc += Pi[j] * v[(size_t)j * hd + d];
        o[(size_t)i * hd + d] = acc;
      }
    }
  }

  if (want_bwd) {
    /* dP_ij = dO_i . V_j ; dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik) */
    for (int i = 0; i < S; ++i) {
      const double* Pi = P + (size_t)i * S;
      double* dPi = dPm + (size_t)i * S;
      double* dSi = dS + (size_t)i * S;
      for (int j = 0; j <= i; ++j) {
        double acc = 0.0;
        for (int d = 0; d < hd; ++d) acc += dO[(size_t)i * hd + d] * v[(size_t)j * hd + d];
        dPi[j] = acc;
      }
      double rd = 0.0;
      for (int j = 0; j <= i; ++j) rd += Pi[j] * dPi[j];
      if (rowdot_out) rowdot_out[i] = rd;
      for (int j = 0; j <= i; ++j) dSi[j] = Pi[j] * (dPi[j] - rd);
    }
    if (dq) {
      for (int i = 0; i < S; ++i) {
        for (int d = 0; d < hd; ++d) {
          double acc = 0.0;
          for (int j = 0; j <= i; ++j) acc += dS[(size_t)i * S + j] * k[(size_t)j * hd + d];
          dq[(size_t)i * hd + d] = scale * acc;
        }
      }
    }
    if (dk) {
      for (int j = 0; j < S; ++j) {
        for (int d = 0; d < hd; ++d) {
          double acc = 0.0;
          for (int i = j; i < S; ++i) acc += dS[(size_t)i * S + j] * q[(size_t)i * hd + d];
          dk[(size_t)j * hd + d] = scale * acc;
        }
      }
    }
    if (dv) {
      for (int j = 0; j < S; ++j) {
        for (int d = 0; d < hd; ++d) {
          double acc = 0.0;
          for (int i = j; i < S; ++i) acc += P[(size_t)i * S + j] * dO[(size_t)i * hd + d];
          dv[(size_t)j * hd + d] = acc;
        }
      }
    }
  }

  if (P_out) memcpy(P_out, P, SS * sizeof(double));
  if (dP_out) memcpy(dP_out, dPm, SS * sizeof(double));
  if (dS_out) memcpy(dS_out, dS, SS * sizeof(double));
  free(P);
  free(dS);
  free(dPm);
  return REF_OK;
}

/* Single-head entry point for the tests (multi-head attention, no batching). */
int xattn_ref_head(const double* q, const double* k, const double* v, const double* dO,
                   int S, int hd, double scale,
                   double* P, double* dP, double* dS, double* rowdot,
                   double* o, double* lse, double* dq, double* dk, double* dv) {
  if (!q || !k || S <= 0 || hd <= 0) return REF_ERR_ARG;
  if ((v == NULL) && (o || dv || dP || dS || rowdot || dq || dk)) return REF_ERR_ARG;
  if (dO == NULL && (dq || dk || dv || dP || dS || rowdot)) return REF_ERR_ARG;
  return head_ref(q, k, v, dO, S, hd, scale, P, dP, dS, rowdot, o, lse, dq, dk, dv);
}

/* repeat_kv: src [Hkv][S][hd] of one batch entry -> dst [H][S][hd], with
 * dst head kvh*group + r taking a copy of src head kvh. */
static void repeat_kv(const double* src, double* dst, int Hkv, int group, int S, int hd) {
  const size_t head = (size_t)S * hd;
  for (int kvh = 0; kvh < Hkv; ++kvh)
    for (int r = 0; r < group; ++r)
      memcpy(dst + (size_t)(kvh * group + r) * head, src + (size_t)kvh * head, head * sizeof(double));
}

static int check_dims(int B, int S, int H, int Hkv, int hd) {
  if (B <= 0 || S <= 0 || H <= 0 || Hkv <= 0 || hd <= 0) return REF_ERR_ARG;
  if (H % Hkv != 0) return REF_ERR_ARG;
  return REF_OK;
}

/*
 * Batched forward + (optional) backward.  The work is split into independent
 * units (b, kvh); each unit repeats its kv head group times, runs the plain
 * per-head attention for query heads kvh*group .. kvh*group+group-1, and sums
 * the repeated heads' dK/dV in ascending r.
 *
 * Any of o, lse may be NULL.  If dO is NULL, dq, dk and dv must be NULL too.
 * units_lo/units_hi restrict the computation to units [lo, hi) of the
 * flattened b*Hkv + kvh index; the other outputs are left untouched.  This is
 * how a test computes sampled outputs of a large configuration.
 */
int xattn_ref_run(const double* q, const double* k, const double* v, const double* dO,
                  double* o, double* lse, double* dq, double* dk, double* dv,
                  int B, int S, int H, int Hkv, int hd, double scale,
                  int units_lo, int units_hi) {
  int rc = check_dims(B, S, H, Hkv, hd);
  if (rc) return rc;
  if (!q || !k || !v) return REF_ERR_ARG;
  if (!dO && (dq || dk || dv)) return REF_ERR_ARG;
  const int group = H / Hkv;
  const int n_units = B * Hkv;
  if (units_lo < 0) units_lo = 0;
  if (units_hi < 0 || units_hi > n_units) units_hi = n_units;
  if (units_lo >= units_hi) return REF_OK;

  const size_t head = (size_t)S * hd;
  int err = REF_OK;

#ifdef _OPENMP
  const int nthr = xattn_ref_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthr)
#endif
  for (int u = units_lo; u < units_hi; ++u) {
    const int b = u / Hkv;
    const int kvh = u % Hkv;
    /* repeated K/V for this batch entry (all kv heads, as repeat_kv does),
     * then the group of query heads that read kv head kvh */
    double* krep = (double*)malloc((size_t)H * head * sizeof(double));
    double* vrep = (double*)malloc((size_t)H * head * sizeof(double));
    double* dk_rep = dk ? (double*)malloc((size_t)group * head * sizeof(double)) : NULL;
    double* dv_rep = dv ? (double*)malloc((size_t)group * head * sizeof(double)) : NULL;
    if (!krep || !vrep || (dk && !dk_rep) || (dv && !dv_rep)) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      err = REF_ERR_NOMEM;
      free(krep); free(vrep); free(dk_rep); free(dv_rep);
      continue;
    }
    repeat_kv(k + (size_t)b * Hkv * head, krep, Hkv, group, S, hd);
    repeat_kv(v + (size_t)b * Hkv * head, vrep, Hkv, group, S, hd);

    for (int r = 0; r < group; ++r) {
      const int h = kvh * group + r;
      const size_t qoff = ((size_t)b * H + h) * head;
      int hrc = head_ref(q + qoff, krep + (size_t)h * head, vrep + (size_t)h * head,
                         dO ? dO + qoff : NULL, S, hd, scale,
                         NULL, NULL, NULL, NULL,
                         o ? o + qoff : NULL,
                         lse ? lse + ((size_t)b * H + h) * S : NULL,
                         dq ? dq + qoff : NULL,
                         dk_rep ? dk_rep + (size_t)r * head : NULL,
                         dv_rep ? dv_rep + (size_t)r * head : NULL);
      if (hrc) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
        err = hrc;
      }
    }
    /* deterministic group sum, ascending r */
    const size_t kvoff = ((size_t)b * Hkv + kvh) * head;
    if (dk) {
      for (size_t e = 0; e < head; ++e) {
        double acc = 0.0;
        for (int r = 0; r < group; ++r) acc += dk_rep[(size_t)r * head + e];
        dk[kvoff + e] = acc;
      }
    }
    if (dv) {
      for (size_t e = 0; e < head; ++e) {
        double acc = 0.0;
        for (int r = 0; r < group; ++r) acc += dv_rep[(size_t)r * head + e];
        dv[kvoff + e] = acc;
      }
    }
    free(krep); free(vrep); free(dk_rep); free(dv_rep);
  }
  return err;
}
