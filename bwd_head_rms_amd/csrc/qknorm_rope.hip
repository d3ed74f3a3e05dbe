// qknorm_rope.hip -- per-head RMS QK-norm + rotary position embedding, forward
// and backward, for gfx950.  The step that turns the q (or k) projection output
// into the attention input: RMSNorm over each head's hd values with a weight per
// head dimension (the per-head QK-norm of the "xtrain evolution overview",
// section 一, row T9), then the rotary embedding at the token's position in its
// sequence (rows T5 and T10; position = row % S as in the KI-1 fix of "xtrain --
// Known Issues & Perf Backlog"), written head-major [B][H][S][hd] -- the
// transpose the KI-1 fix does separately (transpose_4d12) is folded into the
// store.  The rotation pairs dimension i with i + hd/2 at angle
// s * base^(-2i/hd).
//
// Both kernels are HBM-bound elementwise passes: one thread owns four rotation
// pairs (8 of a head vector's hd values: two 8- or 16-byte loads), hd/8 adjacent
// threads own one head vector and reduce its sums with cross-lane exchanges.
// Angles are formed in fp64 (in turns) and reduced to [-1/2, 1/2] turn before the
// hardware sine and cosine, so positions up to 2^31 keep full fp32 accuracy.
//
// Backward, per head vector, with g = dOut (fp32, head-major):
//   gy = R(theta)^T g,  xh = x / r,  gxh = w * gy,
//   dx = (gxh - xh * mean(xh * gxh)) / r            (fp32, token-major)
//   dw = sum over every (b, s, h) of xh * gy         (fp32)
// dw is summed deterministically: each workgroup of a fixed grid walks a fixed
// set of vectors, reduces its threads' partial sums in a fixed order into one
// workspace row, and a second kernel adds the rows in a fixed order.
#include <type_traits>

#include "attn_device.hpp"
#include "launch.hpp"

namespace xattn {

template <int HD>
struct NormCfg {
  static constexpr int HALF = HD / 2;
  static constexpr int TPV = HALF / 4;  // threads per head vector
  static constexpr int NT = 256;
  static_assert(TPV >= 1 && NT % TPV == 0, "head dimension");
};

constexpr double kTwoPi = 6.283185307179586;
constexpr long kNormFwdBlocks = 2048;  // forward grid cap: each thread then walks several vectors

// cos and sin of s * inv_freq: the angle, in turns (inv_freq is given in turns
// per position), is reduced to [-1/2, 1/2] in fp64, then the hardware sine and
// cosine (which take turns) finish in fp32
__device__ __forceinline__ void rope_cs(int s, double turns_per_pos, float& c, float& sn) {
  const double a = (double)s * turns_per_pos;
  const float red = (float)(a - rint(a));
  sn = __builtin_amdgcn_sinf(red);
  c = __builtin_amdgcn_cosf(red);
}

// rotation frequency of pair i, in turns per position: base^(-2i/hd) / (2 pi)
__device__ __forceinline__ double turns_per_pos(int i, int hd, double log2_base) {
  return exp2(-2.0 * i / hd * log2_base) * (1.0 / kTwoPi);
}

// four consecutive values of a row (bf16 or float) as float
template <typename T>
__device__ __forceinline__ float4 load4(const T* p) {
  if constexpr (sizeof(T) == 2) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    const bf16x4 v = __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(p));
    return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
  } else {
    return *reinterpret_cast<const float4*>(p);
  }
}

template <int TPV>
__device__ __forceinline__ float vec_sum(float x) {
#pragma unroll
  for (int off = TPV / 2; off >= 1; off /= 2) x += __shfl_xor(x, off, TPV);
  return x;
}

template <typename T, int HD>
__global__ __launch_bounds__(256) void qknorm_rope_fwd_kernel(const T* __restrict__ x,
                                                              const float* __restrict__ w,
                                                              T* __restrict__ out, int S, int H,
                                                              long nvec, float eps,
                                                              double log2_base) {
  using C = NormCfg<HD>;
  const int j = threadIdx.x % C::TPV;  // fixed: the grid stride is a multiple of TPV
  const int i0 = 4 * j;
  double fr[4];
  float w1[4], w2[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    fr[e] = turns_per_pos(i0 + e, HD, log2_base);
    w1[e] = w[i0 + e];
    w2[e] = w[C::HALF + i0 + e];
  }
  const long stride = (long)gridDim.x * C::NT / C::TPV;  // vectors per grid pass
  // whole vectors only: a vector's TPV threads are adjacent lanes
  for (long v = ((long)blockIdx.x * C::NT + threadIdx.x) / C::TPV; v < nvec; v += stride) {
    const int h = (int)(v % H);
    const long bs = v / H;
    const int s = (int)(bs % S);
    const long b = bs / S;
    const T* xv = x + v * HD;
    const float4 a = load4(xv + i0), c4 = load4(xv + C::HALF + i0);
    const float x1[4] = {a.x, a.y, a.z, a.w}, x2[4] = {c4.x, c4.y, c4.z, c4.w};
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) ss += x1[e] * x1[e] + x2[e] * x2[e];
    ss = vec_sum<C::TPV>(ss);
    const float rinv = 1.f / sqrtf(ss * (1.f / HD) + eps);

    float o1[4], o2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float cs, sn;
      rope_cs(s, fr[e], cs, sn);
      const float y1 = w1[e] * (x1[e] * rinv), y2 = w2[e] * (x2[e] * rinv);
      o1[e] = y1 * cs - y2 * sn;
      o2[e] = y2 * cs + y1 * sn;
    }
    T* ov = out + ((b * H + h) * S + s) * HD;
    store4<T>(ov + i0, o1[0], o1[1], o1[2], o1[3]);
    store4<T>(ov + C::HALF + i0, o2[0], o2[1], o2[2], o2[3]);
  }
}

template <typename T, int HD>
__global__ __launch_bounds__(256) void qknorm_rope_bwd_kernel(
    const T* __restrict__ x, const float* __restrict__ w, const float* __restrict__ dout,
    float* __restrict__ dx, float* __restrict__ dw_part, int S, int H, long nvec, float eps,
    double log2_base) {
  using C = NormCfg<HD>;
  __shared__ float red[C::NT][8];
  const int j = threadIdx.x % C::TPV;  // fixed: the grid stride is a multiple of TPV
  const int i0 = 4 * j;
  double inv[4];
  float w1[4], w2[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    inv[e] = turns_per_pos(i0 + e, HD, log2_base);
    w1[e] = w[i0 + e];
    w2[e] = w[C::HALF + i0 + e];
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

  const long stride = (long)gridDim.x * C::NT / C::TPV;  // vectors per grid pass
  for (long v = ((long)blockIdx.x * C::NT + threadIdx.x) / C::TPV; v < nvec; v += stride) {
    const int h = (int)(v % H);
    const long bs = v / H;
    const int s = (int)(bs % S);
    const long b = bs / S;
    const T* xv = x + v * HD;
    const float* gv = dout + ((b * H + h) * S + s) * HD;
    const float4 a = load4(xv + i0), c4 = load4(xv + C::HALF + i0);
    const float4 ga = *reinterpret_cast<const float4*>(gv + i0);
    const float4 gb = *reinterpret_cast<const float4*>(gv + C::HALF + i0);
    const float x1[4] = {a.x, a.y, a.z, a.w}, x2[4] = {c4.x, c4.y, c4.z, c4.w};
    const float g1[4] = {ga.x, ga.y, ga.z, ga.w}, g2[4] = {gb.x, gb.y, gb.z, gb.w};
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) ss += x1[e] * x1[e] + x2[e] * x2[e];
    ss = vec_sum<C::TPV>(ss);
    const float rinv = 1.f / sqrtf(ss * (1.f / HD) + eps);

    float xh1[4], xh2[4], gx1[4], gx2[4], dot = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float cs, sn;
      rope_cs(s, inv[e], cs, sn);
      const float gy1 = g1[e] * cs + g2[e] * sn;    // rotation transposed
      const float gy2 = -g1[e] * sn + g2[e] * cs;
      xh1[e] = x1[e] * rinv;
      xh2[e] = x2[e] * rinv;
      acc[e] += xh1[e] * gy1;
      acc[4 + e] += xh2[e] * gy2;
      gx1[e] = w1[e] * gy1;
      gx2[e] = w2[e] * gy2;
      dot += xh1[e] * gx1[e] + xh2[e] * gx2[e];
    }
    const float mean = vec_sum<C::TPV>(dot) * (1.f / HD);
    float* dv = dx + v * HD;
    store4<float>(dv + i0, (gx1[0] - xh1[0] * mean) * rinv, (gx1[1] - xh1[1] * mean) * rinv,
                  (gx1[2] - xh1[2] * mean) * rinv, (gx1[3] - xh1[3] * mean) * rinv);
    store4<float>(dv + C::HALF + i0, (gx2[0] - xh2[0] * mean) * rinv,
                  (gx2[1] - xh2[1] * mean) * rinv, (gx2[2] - xh2[2] * mean) * rinv,
                  (gx2[3] - xh2[3] * mean) * rinv);
  }

  // this workgroup's dw: thread slot e of lane group j holds dimension
  // i0 + e (e < 4) or HALF + i0 + e - 4; summed over the threads of equal j in
  // ascending thread order
#pragma unroll
  for (int e = 0; e < 8; ++e) red[threadIdx.x][e] = acc[e];
  __syncthreads();
  if (threadIdx.x < HD) {
    const int d = threadIdx.x;
    const int dj = (d % C::HALF) / 4, de = d % 4 + (d >= C::HALF ? 4 : 0);
    float sum = 0.f;
    for (int tt = dj; tt < C::NT; tt += C::TPV) sum += red[tt][de];
    dw_part[(size_t)blockIdx.x * HD + d] = sum;
  }
}

// dw[d] = sum of the workgroups' partial rows in a fixed order: one workgroup
// per dimension d; thread t adds rows t, t + 256, t + 512, ... (independent
// loads), then a fixed pairwise tree over the 256 thread sums
constexpr int kReduceThreads = 256;

template <int HD>
__global__ __launch_bounds__(kReduceThreads) void qknorm_dw_reduce_kernel(
    const float* __restrict__ part, int nblk, float* __restrict__ dw) {
  __shared__ float t_sum[kReduceThreads];
  const int d = blockIdx.x, t = threadIdx.x;
  float sum = 0.f;
#pragma unroll 4
  for (int k = t; k < nblk; k += kReduceThreads) sum += part[(size_t)k * HD + d];
  t_sum[t] = sum;
  __syncthreads();
#pragma unroll
  for (int n = kReduceThreads / 2; n >= 1; n /= 2) {
    if (t < n) t_sum[t] += t_sum[t + n];
    __syncthreads();
  }
  if (t == 0) dw[d] = t_sum[0];
}

template <typename T, int HD>
static void norm_fwd_typed(const NormDims& d, const void* x, const float* w, void* out,
                           float eps, float base, hipStream_t stream) {
  using C = NormCfg<HD>;
  const long nvec = (long)d.B * d.S * d.H;
  const long need = (nvec * C::TPV + C::NT - 1) / C::NT;
  const long blocks = need < kNormFwdBlocks ? need : kNormFwdBlocks;
  hipLaunchKernelGGL((qknorm_rope_fwd_kernel<T, HD>), dim3((unsigned)blocks), dim3(C::NT), 0,
                     stream, (const T*)x, w, (T*)out, d.S, d.H, nvec, eps, log2((double)base));
}

template <typename T, int HD>
static void norm_bwd_typed(const NormDims& d, const void* x, const float* w, const float* dout,
                           float* dx, float* dw, float* ws, float eps, float base,
                           hipStream_t stream) {
  using C = NormCfg<HD>;
  const long nvec = (long)d.B * d.S * d.H;
  const int blocks = qknorm_bwd_blocks(nvec, HD);
  hipLaunchKernelGGL((qknorm_rope_bwd_kernel<T, HD>), dim3(blocks), dim3(C::NT), 0, stream,
                     (const T*)x, w, dout, dx, ws, d.S, d.H, nvec, eps, log2((double)base));
  hipLaunchKernelGGL((qknorm_dw_reduce_kernel<HD>), dim3(HD), dim3(kReduceThreads), 0, stream, ws,
                     blocks, dw);
}

void launch_qknorm_rope_fwd(int dtype, const NormDims& d, const void* x, const float* w,
                            void* out, float eps, float base, hipStream_t stream) {
  if (dtype == 0) {
    if (d.hd == 16) norm_fwd_typed<float, 16>(d, x, w, out, eps, base, stream);
    else if (d.hd == 32) norm_fwd_typed<float, 32>(d, x, w, out, eps, base, stream);
    else norm_fwd_typed<float, 64>(d, x, w, out, eps, base, stream);
  } else {
    if (d.hd == 16) norm_fwd_typed<bf16, 16>(d, x, w, out, eps, base, stream);
    else if (d.hd == 32) norm_fwd_typed<bf16, 32>(d, x, w, out, eps, base, stream);
    else norm_fwd_typed<bf16, 64>(d, x, w, out, eps, base, stream);
  }
}

void launch_qknorm_rope_bwd(int dtype, const NormDims& d, const void* x, const float* w,
                            const float* dout, float* dx, float* dw, float* ws, float eps,
                            float base, hipStream_t stream) {
  if (dtype == 0) {
    if (d.hd == 16) norm_bwd_typed<float, 16>(d, x, w, dout, dx, dw, ws, eps, base, stream);
    else if (d.hd == 32) norm_bwd_typed<float, 32>(d, x, w, dout, dx, dw, ws, eps, base, stream);
    else norm_bwd_typed<float, 64>(d, x, w, dout, dx, dw, ws, eps, base, stream);
  } else {
    if (d.hd == 16) norm_bwd_typed<bf16, 16>(d, x, w, dout, dx, dw, ws, eps, base, stream);
    else if (d.hd == 32) norm_bwd_typed<bf16, 32>(d, x, w, dout, dx, dw, ws, eps, base, stream);
    else norm_bwd_typed<bf16, 64>(d, x, w, dout, dx, dw, ws, eps, base, stream);
  }
}

}  // namespace xattn
