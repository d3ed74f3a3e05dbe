/*
 * ref_qknorm_rope.c -- fp64 CPU oracle for the per-head RMS QK-norm followed by
 * the rotary position embedding (the step that prepares q and k for attention),
 * forward and analytic backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the CPU-baseline
 * leg of the benchmark may load it.  It shares no code, header, table or helper
 * with the HIP library, and it never calls it.
 *
 * What it computes (plain definition, all arithmetic in double).  For every
 * token (b, s) and head h, with the head vector x = X[b,s,h,:] (hd values) and
 * the per-dimension weight w[0..hd-1] shared by all heads:
 *   r      = sqrt( (1/hd) sum_d x_d^2 + eps )          RMS over the head dim
 *   xh_d   = x_d / r ;   y_d = w_d * xh_d              QK-norm
 *   with half = hd/2 and, for i < half, theta_i = s * base^(-2i/hd):
 *     Out[b,h,s,i]      = y_i      cos(theta_i) - y_{i+half} sin(theta_i)
 *     Out[b,h,s,i+half] = y_{i+half} cos(theta_i) + y_i      sin(theta_i)
 *   (the position is the index s inside the sequence; the output is head-major)
 * Backward for an upstream gradient G = dOut[b,h,s,:], by the chain rule with
 * every Jacobian written out:
 *   gy_i      =  G_i cos(theta_i) + G_{i+half} sin(theta_i)    (rotation^T)
 *   gy_{i+half} = -G_i sin(theta_i) + G_{i+half} cos(theta_i)
 *   dw_d     +=  xh_d gy_d                                (summed over b, s, h)
 *   gxh_d     =  w_d gy_d
 *   dX[b,s,h,k] = sum_d gxh_d * d xh_d / d x_k,
 *                 d xh_d / d x_k = delta_dk / r - x_d x_k / (hd r^3)
 *
 * Sources (the pages this follows):
 *   - "xtrain evolution overview", section 一 (infra phases): row T5 (the tiny
 *     decoder uses RoPE and RMSNorm), row T9 (a per-head QK-norm, compatible
 *     with Qwen3), row T10 (batched forward with RoPE positions per sequence).
 *   - "xtrain -- Known Issues & Perf Backlog", KI-1 fix: activations are
 *     [B*S, dim] rows; RoPE positions restart per sequence (row % S); the
 *     attention input is the head-major [B, heads, S, hd] layout that
 *     transpose_4d12 produces.
 * Readings taken where the pages are silent (they print no formula): the norm
 * is RMSNorm over each head's hd values with a weight per head dimension shared
 * by all heads (Qwen3's q_norm / k_norm); the rotation pairs dimension i with
 * i + hd/2 (half split) with theta_i = pos * base^(-2i/hd), base 10000; the
 * norm comes before the rotation.
 *
 * Layout (all contiguous, row-major): X, dX: [B][S][H][hd] (token-major, as the
 * projection writes it); Out, dOut: [B][H][S][hd]; w, dw: [hd].
 *
 * Parallelism: optional OpenMP over tokens for Out and dX (each element is
 * written by one thread); dw is summed in one fixed order (b, s, h ascending), so
 * results do not depend on the thread count.
 */
#include <math.h>
#include <stddef.h>

enum { REFN_OK = 0, REFN_ERR_ARG = 1 };

static int bad_args(int B, int S, int H, int hd) {
  return B < 1 || S < 1 || H < 1 || hd < 2 || hd > 512 || (hd % 2) != 0;
}

/* angle of rotation pair i at position s */
static double angle(int s, int i, int hd, double base) {
  return (double)s * pow(base, -2.0 * (double)i / (double)hd);
}

int xattn_ref_qknorm_rope_fwd(const double* X, const double* w, double* Out, int B, int S,
                              int H, int hd, double eps, double base) {
  if (!X || !w || !Out || bad_args(B, S, H, hd) || !(eps >= 0.0) || !(base > 0.0))
    return REFN_ERR_ARG;
  const int half = hd / 2;
#pragma omp parallel for schedule(static)
  for (long t = 0; t < (long)B * S; ++t) {
    const int b = (int)(t / S), s = (int)(t % S);
    for (int h = 0; h < H; ++h) {
      const double* x = X + (((size_t)b * S + s) * H + h) * hd;
      double* o = Out + (((size_t)b * H + h) * S + s) * hd;
      double ss = 0.0;
      for (int d = 0; d < hd; ++d) ss += x[d] * x[d];
      const double r = sqrt(ss / hd + eps);
      for (int i = 0; i < half; ++i) {
        const double th = angle(s, i, hd, base);
        const double y1 = w[i] * (x[i] / r), y2 = w[i + half] * (x[i + half] / r);
        o[i] = y1 * cos(th) - y2 * sin(th);
        o[i + half] = y2 * cos(th) + y1 * sin(th);
      }
    }
  }
  return REFN_OK;
}

int xattn_ref_qknorm_rope_bwd(const double* X, const double* w, const double* dOut, double* dX,
                              double* dw, int B, int S, int H, int hd, double eps, double base) {
  if (!X || !w || !dOut || !dX || !dw || bad_args(B, S, H, hd) || !(eps >= 0.0) || !(base > 0.0))
    return REFN_ERR_ARG;
  const int half = hd / 2;
#pragma omp parallel for schedule(static)
  for (long t = 0; t < (long)B * S; ++t) {
    const int b = (int)(t / S), s = (int)(t % S);
    double gy[512], gxh[512];
    for (int h = 0; h < H; ++h) {
      const double* x = X + (((size_t)b * S + s) * H + h) * hd;
      const double* G = dOut + (((size_t)b * H + h) * S + s) * hd;
      double* dx = dX + (((size_t)b * S + s) * H + h) * hd;
      double ss = 0.0;
      for (int d = 0; d < hd; ++d) ss += x[d] * x[d];
      const double r = sqrt(ss / hd + eps);
      for (int i = 0; i < half; ++i) {
        const double th = angle(s, i, hd, base);
        gy[i] = G[i] * cos(th) + G[i + half] * sin(th);
        gy[i + half] = -G[i] * sin(th) + G[i + half] * cos(th);
      }
      for (int d = 0; d < hd; ++d) gxh[d] = w[d] * gy[d];
      for (int k = 0; k < hd; ++k) {
        double acc = 0.0;
        for (int d = 0; d < hd; ++d) {
          const double jac = (d == k ? 1.0 / r : 0.0) - x[d] * x[k] / (hd * r * r * r);
          acc += gxh[d] * jac;
        }
        dx[k] = acc;
      }
    }
  }
  /* weight gradient: one fixed order over every (b, s, h) */
  for (int d = 0; d < hd; ++d) dw[d] = 0.0;
  double gy[512];
  for (int b = 0; b < B; ++b)
    for (int s = 0; s < S; ++s)
      for (int h = 0; h < H; ++h) {
        const double* x = X + (((size_t)b * S + s) * H + h) * hd;
        const double* G = dOut + (((size_t)b * H + h) * S + s) * hd;
        double ss = 0.0;
        for (int d = 0; d < hd; ++d) ss += x[d] * x[d];
        const double r = sqrt(ss / hd + eps);
        for (int i = 0; i < half; ++i) {
          const double th = angle(s, i, hd, base);
          gy[i] = G[i] * cos(th) + G[i + half] * sin(th);
          gy[i + half] = -G[i] * sin(th) + G[i + half] * cos(th);
        }
        for (int d = 0; d < hd; ++d) dw[d] += (x[d] / r) * gy[d];
      }
  return REFN_OK;
}
