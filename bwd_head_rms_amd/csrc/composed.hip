// composed.hip -- the composed attention path for gfx950: scores, causal
// softmax and the value product as separate passes through an S x S fp32
// buffer per (batch, head), and the backward the same way.
//
// This is the pages' other implementation of the same operation (the batched
// path of the KI-1 fix on "xtrain -- Known Issues & Perf Backlog": a strided
// batched Q.K^T, a causal softmax, then P.V; the fused kernel of row T14 in the
// "xtrain evolution overview" infra table replaces it).  It keeps the
// probabilities as an activation, which is its memory cost: 4*B*H*S*S bytes
// (1.07 GB at B4 S2048 H16), against the fused path's 8*B*H*S.  It exists to
// compare the two paths on the same inputs (results and time).
//
//   forward:  S  = scale * Q.K^T          (lower-triangle 128x128 tiles)
//             P  = softmax_causal(S), LSE (row pass; zeros up to the tile end)
//             O  = P.V
//   backward: dP = dO.V^T                 (same tiles as S)
//             dS = P * (dP - rowsum(P * dP))
//             dQ = scale * dS.K,  dK = scale * sum_group dS^T.Q,  dV = sum_group P^T.dO
//
// The products run on MFMA with fp32 accumulation and the operand layouts of
// the fused kernels (attn_device.hpp): Q.K^T-shaped products compute the
// transposed tile (keys are rows, queries are lanes); X.Y-shaped products
// (P.V, dS.K) read each lane's row of X straight from HBM in the permuted
// contraction order of the accumulator layout; X^T.Y-shaped products
// (P^T.dO, dS^T.Q) stage an X tile in LDS and read it with transpose reads.
// In bf16 mode P and dS are rounded to bf16 (nearest-even) where they enter a
// product, as in the fused kernels.  Query head h reads kv head h / group; the
// group sum of dK and dV runs in registers in a fixed order.
#include <type_traits>

#include "attn_device.hpp"
#include "launch.hpp"

namespace xattn {


// --------------------------------------------------------------------------
// out[bh][i][j] = c * a[bh][i] . bm[kv][j] on the lower-triangle tiles
// (j tile <= i tile); one workgroup per tile.
template <typename T, int HD>
__global__ __launch_bounds__(256) void cmp_scores_kernel(const T* __restrict__ a,
                                                         const T* __restrict__ bm,
                                                         float* __restrict__ out, int S, int H,
                                                         int Hkv, int ntri, float c) {
  using M = Mma<T>;
  constexpr int NKS = HD / M::KSTEP;
  __shared__ __align__(16) T sB[Tile<T, HD, kCmpTile>::ELEMS];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int li = lane & 31, g = lane >> 5;
  const int bh = blockIdx.x / ntri;
  const int t = blockIdx.x % ntri;
  int it = (int)((sqrtf(8.f * (float)t + 1.f) - 1.f) * 0.5f);
  while ((it + 1) * (it + 2) / 2 <= t) ++it;
  while (it * (it + 1) / 2 > t) --it;
  const int jt = t - it * (it + 1) / 2;
  const int b = bh / H, h = bh % H, kvh = h / (H / Hkv);

  const int i = it * kCmpTile + wave * 32 + li;
  const bool i_ok = i < S;
  typename M::frag af[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    af[ks] = i_ok ? row_frag_global<T, HD>(a + ((size_t)bh * S + i) * HD, g, ks) : zero_frag<T>();
  Stager<T, HD, kCmpTile, 4> st;
  st.issue(bm + ((size_t)b * Hkv + kvh) * S * HD, jt * kCmpTile, S, sB, wave, lane, tid);
  wait_global_loads();
  st.commit(sB, tid);
  __syncthreads();

  float* orow = out + ((size_t)bh * S + (i_ok ? i : 0)) * S;
  const bool vec = (S & 3) == 0;
#pragma unroll
  for (int cb = 0; cb < kCmpTile / 32; ++cb) {
    const int kb0 = jt * kCmpTile + 32 * cb;
    if (kb0 >= S) break;
    f32x16 s = zero_acc();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      M::mma(s, row_frag_lds<T, HD, kCmpTile>(sB, 32 * cb + li, g, ks), af[ks]);
    if (!i_ok) continue;
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int j = kb0 + 8 * rg + 4 * g;  // keys j .. j+3 (accumulator rows 4rg .. 4rg+3)
      if (vec && j + 3 < S) {
        store4<float>(orow + j, c * s[4 * rg], c * s[4 * rg + 1], c * s[4 * rg + 2],
                      c * s[4 * rg + 3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j + e < S) orow[j + e] = c * s[4 * rg + e];
      }
    }
  }
}

// --------------------------------------------------------------------------
// Row passes: one wave per row i of a (batch, head) plane.  Entries past the
// diagonal, up to the end of the row's 128-key tile, are written as zero (the
// products below read whole tiles).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off /= 2) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off /= 2) x += __shfl_xor(x, off);
  return x;
}

// Rows up to kRowCache floats (S a multiple of 4) are held in registers, four
// consecutive floats per lane and chunk, so each buffer is read once; longer
// rows take a strided loop that reads them again per pass.
constexpr int kRowChunks = 8;  // float4 chunks per lane
constexpr int kRowCache = kRowChunks * 4 * kWave;

__device__ __forceinline__ float4 masked_load4(const float* row, int j, int n, float fill) {
  if (j + 3 < n) return *reinterpret_cast<const float4*>(row + j);
  return make_float4(j < n ? row[j] : fill, j + 1 < n ? row[j + 1] : fill,
                     j + 2 < n ? row[j + 2] : fill, fill);
}

// P = softmax over j <= i of the scores, in place; lse = natural-log LSE
__global__ __launch_bounds__(256) void cmp_softmax_kernel(float* __restrict__ p,
                                                          float* __restrict__ lse, int S,
                                                          long rows) {
  const long row = (long)blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (row >= rows) return;
  const int i = (int)(row % S);
  float* pr = p + row * S;
  const int n = i + 1;
  const int end = min(S, (i / kCmpTile + 1) * kCmpTile);
  if (S <= kRowCache && (S & 3) == 0) {
    float4 v[kRowChunks];
    float m = -INFINITY;
#pragma unroll
    for (int c = 0; c < kRowChunks; ++c) {
      const int j = 4 * (lane + kWave * c);
      v[c] = j < n ? masked_load4(pr, j, n, -INFINITY)
                   : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      m = fmaxf(m, fmaxf(fmaxf(v[c].x, v[c].y), fmaxf(v[c].z, v[c].w)));
    }
    m = wave_max(m);
    float l = 0.f;
#pragma unroll
    for (int c = 0; c < kRowChunks; ++c) {  // masked entries give exp2(-inf) = 0
      v[c].x = fast_exp2((v[c].x - m) * kLog2e);
      v[c].y = fast_exp2((v[c].y - m) * kLog2e);
      v[c].z = fast_exp2((v[c].z - m) * kLog2e);
      v[c].w = fast_exp2((v[c].w - m) * kLog2e);
      l += (v[c].x + v[c].y) + (v[c].z + v[c].w);
    }
    l = wave_sum(l);
    const float inv = 1.f / l;
#pragma unroll
    for (int c = 0; c < kRowChunks; ++c) {
      const int j = 4 * (lane + kWave * c);
      if (j < end)
        *reinterpret_cast<float4*>(pr + j) =
            make_float4(v[c].x * inv, v[c].y * inv, v[c].z * inv, v[c].w * inv);
    }
    if (lane == 0) lse[row] = m + logf(l);
    return;
  }
  float m = -INFINITY;
  for (int j = lane; j < n; j += kWave) m = fmaxf(m, pr[j]);
  m = wave_max(m);
  float l = 0.f;
  for (int j = lane; j < n; j += kWave) l += fast_exp2((pr[j] - m) * kLog2e);
  l = wave_sum(l);
  const float inv = 1.f / l;
  for (int j = lane; j < end; j += kWave) pr[j] = j < n ? fast_exp2((pr[j] - m) * kLog2e) * inv : 0.f;
  if (lane == 0) lse[row] = m + logf(l);
}

// dS = P * (dP - sum_{k<=i} P_ik dP_ik), in place of dP
__global__ __launch_bounds__(256) void cmp_softmax_bwd_kernel(const float* __restrict__ p,
                                                              float* __restrict__ dp, int S,
                                                              long rows) {
  const long row = (long)blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (row >= rows) return;
  const int i = (int)(row % S);
  const float* pr = p + row * S;
  float* dr = dp + row * S;
  const int n = i + 1;
  const int end = min(S, (i / kCmpTile + 1) * kCmpTile);
  if (S <= kRowCache && (S & 3) == 0) {
    float4 pv[kRowChunks], dv[kRowChunks];
    float rd = 0.f;
#pragma unroll
    for (int c = 0; c < kRowChunks; ++c) {
      const int j = 4 * (lane + kWave * c);
      const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
      pv[c] = j < n ? masked_load4(pr, j, n, 0.f) : z;
      dv[c] = j < n ? masked_load4(dr, j, n, 0.f) : z;
      rd += (pv[c].x * dv[c].x + pv[c].y * dv[c].y) + (pv[c].z * dv[c].z + pv[c].w * dv[c].w);
    }
    rd = wave_sum(rd);
#pragma unroll
    for (int c = 0; c < kRowChunks; ++c) {
      const int j = 4 * (lane + kWave * c);
      if (j < end)
        *reinterpret_cast<float4*>(dr + j) =
            make_float4(pv[c].x * (dv[c].x - rd), pv[c].y * (dv[c].y - rd),
                        pv[c].z * (dv[c].z - rd), pv[c].w * (dv[c].w - rd));
    }
    return;
  }
  float rd = 0.f;
  for (int j = lane; j < n; j += kWave) rd += pr[j] * dr[j];
  rd = wave_sum(rd);
  for (int j = lane; j < end; j += kWave) dr[j] = j < n ? pr[j] * (dr[j] - rd) : 0.f;
}

// --------------------------------------------------------------------------
// out[bh][i] = c * sum_{j <= i} x[bh][i][j] * y[kv][j]  (O = P.V, dQ = dS.K).
// One workgroup per (bh, 128-row tile), 4 waves x 32 rows; y tiles of 64 keys
// double-buffered in LDS; each lane reads its own row of x from HBM.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag x_frag(const float* xrow, int kb0, int ks, int g,
                                                         bool ok, int S, bool vec);
template <>
__device__ __forceinline__ bf16x8 x_frag<bf16>(const float* xrow, int kb0, int ks, int g, bool ok,
                                               int S, bool vec) {
  // elements t = 0..3: keys kb0 + 16ks + 4g + t;  t = 4..7: 8 further on
  float v[8];
  const int k0 = kb0 + 16 * ks + 4 * g;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int k = k0 + 8 * half;
    if (ok && vec && k + 3 < S) {
      const float4 f = *reinterpret_cast<const float4*>(xrow + k);
      v[4 * half] = f.x; v[4 * half + 1] = f.y; v[4 * half + 2] = f.z; v[4 * half + 3] = f.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * half + e] = (ok && k + e < S) ? xrow[k + e] : 0.f;
    }
  }
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)v[e];
  return r;
}
template <>
__device__ __forceinline__ float x_frag<float>(const float* xrow, int kb0, int ks, int g, bool ok,
                                               int S, bool vec) {
  (void)vec;
  const int k = kb0 + acc_row(ks, g);
  return (ok && k < S) ? xrow[k] : 0.f;
}

template <typename T, int HD, typename OutT>
__global__ __launch_bounds__(256) void cmp_nn_kernel(const float* __restrict__ x,
                                                     const T* __restrict__ y,
                                                     OutT* __restrict__ out, int S, int H, int Hkv,
                                                     int nqt, int BH, float c) {
  using M = Mma<T>;
  constexpr int BN = 64, ND = HD >= 32 ? HD / 32 : 1, NAS = 32 / M::KSTEP;
  __shared__ __align__(16) T sY[2][Tile<T, HD, BN>::ELEMS];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int li = lane & 31, g = lane >> 5;
  const int qt = nqt - 1 - blockIdx.x / BH;  // heaviest tiles first
  const int bh = blockIdx.x % BH;
  const int b = bh / H, h = bh % H, kvh = h / (H / Hkv);
  const T* yp = y + ((size_t)b * Hkv + kvh) * S * HD;
  const int q0 = qt * kCmpTile + wave * 32;
  const int my_q = q0 + li;
  const bool q_ok = my_q < S;
  const bool wave_live = q0 < S;
  const int wave_kv_end = min(S, q0 + 32);
  const float* xrow = x + ((size_t)bh * S + (q_ok ? my_q : 0)) * S;
  const bool vec = (S & 3) == 0;

  f32x16 acc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) acc[d] = zero_acc();
  const int kv_end = min(S, qt * kCmpTile + kCmpTile);
  const int ntiles = (kv_end + BN - 1) / BN;
  Stager<T, HD, BN, 4> st;
  st.issue(yp, 0, S, sY[0], wave, lane, tid);
  wait_global_loads();
  st.commit(sY[0], tid);
  __syncthreads();
  for (int jt = 0; jt < ntiles; ++jt) {
    const int cur = jt & 1;
    const int kv_t0 = jt * BN;
    const bool more = jt + 1 < ntiles;
    if (more) st.issue(yp, kv_t0 + BN, S, sY[cur ^ 1], wave, lane, tid);
    if (wave_live && kv_t0 < wave_kv_end) {
#pragma unroll
      for (int cb = 0; cb < BN / 32; ++cb) {
        const int kb0 = kv_t0 + 32 * cb;
        if (kb0 >= wave_kv_end) continue;
#pragma unroll
        for (int ks = 0; ks < NAS; ++ks) {
          const typename M::frag xf = x_frag<T>(xrow, kb0, ks, g, q_ok, S, vec);
#pragma unroll
          for (int db = 0; db < ND; ++db)
            M::mma(acc[db], accrow_frag<T, HD, BN>(sY[cur], 32 * cb, ks, 32 * db, lane), xf);
        }
      }
    }
    if (more) {
      wait_global_loads();
      st.commit(sY[cur ^ 1], tid);
    }
    __syncthreads();
  }
  if (!q_ok) return;
  OutT* orow = out + ((size_t)bh * S + my_q) * HD;
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = 32 * db + 8 * rg + 4 * g;
      if (d0 < HD)
        store4<OutT>(orow + d0, c * acc[db][4 * rg], c * acc[db][4 * rg + 1],
                     c * acc[db][4 * rg + 2], c * acc[db][4 * rg + 3]);
    }
}

// --------------------------------------------------------------------------
// out[kv][j] = c * sum_{r < group} sum_{i >= j} x[b, h_r][i][j] * y[b, h_r][i]
// (dV = sum P^T.dO, dK = scale * sum dS^T.Q).  One workgroup per (b, kv head,
// 128-key tile), 4 waves x 32 keys; per query head of the group (r ascending)
// and query tile at or below the diagonal (ascending): the 128 x 128 tile of x
// is staged in LDS (converted to T) next to the 128-row tile of y.
template <typename T>
__device__ __forceinline__ void put4(T* tile, int off, float4 f);
template <>
__device__ __forceinline__ void put4<bf16>(bf16* tile, int off, float4 f) {
  store4<bf16>(tile + off, f.x, f.y, f.z, f.w);
}
template <>
__device__ __forceinline__ void put4<float>(float* tile, int off, float4 f) {
  tile[off] = f.x; tile[off + 1] = f.y; tile[off + 2] = f.z; tile[off + 3] = f.w;
}

template <typename T, int HD>
__global__ __launch_bounds__(256) void cmp_tn_kernel(const float* __restrict__ x,
                                                     const T* __restrict__ y,
                                                     float* __restrict__ out, int S, int H,
                                                     int Hkv, int BG, float c) {
  using M = Mma<T>;
  constexpr int ND = HD >= 32 ? HD / 32 : 1, NAS = 32 / M::KSTEP;
  using TX = Tile<T, kCmpTile, kCmpTile>;  // rows: queries, columns: the tile's keys
  __shared__ __align__(16) T sX[TX::ELEMS];
  __shared__ __align__(16) T sY[Tile<T, HD, kCmpTile>::ELEMS];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int li = lane & 31;
  const int kt = blockIdx.x / BG;  // key tile 0 (the heaviest) first
  const int bg = blockIdx.x % BG;
  const int b = bg / Hkv, kvh = bg % Hkv;
  const int group = H / Hkv;
  const int kv0 = kt * kCmpTile + wave * 32;
  const int my_kv = kv0 + li;
  const int col0 = kt * kCmpTile;
  const bool vec = (S & 3) == 0;
  const int nq = (S + kCmpTile - 1) / kCmpTile;

  f32x16 acc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) acc[d] = zero_acc();
  Stager<T, HD, kCmpTile, 4> stY;
  for (int r = 0; r < group; ++r) {
    const size_t bh = (size_t)b * H + (size_t)kvh * group + r;
    const float* xp = x + bh * S * S;
    for (int qt = kt; qt < nq; ++qt) {
      const int row0 = qt * kCmpTile;
      __syncthreads();  // the previous tiles are no longer read
      stY.issue(y + bh * S * HD, row0, S, sY, wave, lane, tid);
      // x tile: 128 rows x 32 chunks of 4 floats, 16 chunks per thread
#pragma unroll 4
      for (int e = tid; e < kCmpTile * (kCmpTile / 4); e += 256) {
        const int rr = e / (kCmpTile / 4), cc = 4 * (e % (kCmpTile / 4));
        const int i = row0 + rr, j = col0 + cc;
        float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i < S) {
          const float* src = xp + (size_t)i * S + j;
          if (vec && j + 3 < S) {
            f = *reinterpret_cast<const float4*>(src);
          } else {
            f.x = j < S ? src[0] : 0.f;
            f.y = j + 1 < S ? src[1] : 0.f;
            f.z = j + 2 < S ? src[2] : 0.f;
            f.w = j + 3 < S ? src[3] : 0.f;
          }
        }
        put4<T>(sX, TX::off(rr, cc), f);
      }
      wait_global_loads();
      stY.commit(sY, tid);
      __syncthreads();
      if (kv0 < S) {
#pragma unroll
        for (int qb = 0; qb < kCmpTile / 32; ++qb) {
          if (row0 + 32 * qb + 31 < kv0 || row0 + 32 * qb >= S) continue;  // above the diagonal, or past S
#pragma unroll
          for (int ks = 0; ks < NAS; ++ks) {
            const typename M::frag xf = accrow_frag<T, kCmpTile, kCmpTile>(sX, 32 * qb, ks, 32 * wave, lane);
#pragma unroll
            for (int db = 0; db < ND; ++db)
              M::mma(acc[db], accrow_frag<T, HD, kCmpTile>(sY, 32 * qb, ks, 32 * db, lane), xf);
          }
        }
      }
    }
  }
  if (my_kv >= S) return;
  const int g = lane >> 5;
  float* krow = out + (((size_t)b * Hkv + kvh) * S + my_kv) * HD;
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = 32 * db + 8 * rg + 4 * g;
      if (d0 < HD)
        store4<float>(krow + d0, c * acc[db][4 * rg], c * acc[db][4 * rg + 1],
                      c * acc[db][4 * rg + 2], c * acc[db][4 * rg + 3]);
    }
}

// --------------------------------------------------------------------------
template <typename T, int HD>
static void cmp_fwd_typed(const Dims& d, const void* q, const void* k, const void* v, void* o,
                          float* lse, float* p, float scale, hipStream_t stream) {
  const int nt = (d.S + kCmpTile - 1) / kCmpTile;
  const int ntri = nt * (nt + 1) / 2;
  const int BH = d.B * d.H;
  hipLaunchKernelGGL((cmp_scores_kernel<T, HD>), dim3((unsigned)(BH * ntri)), dim3(256), 0, stream,
                     (const T*)q, (const T*)k, p, d.S, d.H, d.Hkv, ntri, scale);
  const long rows = (long)BH * d.S;
  hipLaunchKernelGGL(cmp_softmax_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, p,
                     lse, d.S, rows);
  hipLaunchKernelGGL((cmp_nn_kernel<T, HD, T>), dim3((unsigned)(nt * BH)), dim3(256), 0, stream,
                     (const float*)p, (const T*)v, (T*)o, d.S, d.H, d.Hkv, nt, BH, 1.f);
}

template <typename T, int HD>
static void cmp_bwd_typed(const Dims& d, const void* q, const void* k, const void* v,
                          const float* p, const void* dO, float* dq, float* dk, float* dv,
                          float* ds, float scale, hipStream_t stream) {
  const int nt = (d.S + kCmpTile - 1) / kCmpTile;
  const int ntri = nt * (nt + 1) / 2;
  const int BH = d.B * d.H, BG = d.B * d.Hkv;
  hipLaunchKernelGGL((cmp_scores_kernel<T, HD>), dim3((unsigned)(BH * ntri)), dim3(256), 0, stream,
                     (const T*)dO, (const T*)v, ds, d.S, d.H, d.Hkv, ntri, 1.f);
  const long rows = (long)BH * d.S;
  hipLaunchKernelGGL(cmp_softmax_bwd_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                     stream, p, ds, d.S, rows);
  hipLaunchKernelGGL((cmp_nn_kernel<T, HD, float>), dim3((unsigned)(nt * BH)), dim3(256), 0,
                     stream, (const float*)ds, (const T*)k, dq, d.S, d.H, d.Hkv, nt, BH, scale);
  hipLaunchKernelGGL((cmp_tn_kernel<T, HD>), dim3((unsigned)(nt * BG)), dim3(256), 0, stream,
                     (const float*)ds, (const T*)q, dk, d.S, d.H, d.Hkv, BG, scale);
  hipLaunchKernelGGL((cmp_tn_kernel<T, HD>), dim3((unsigned)(nt * BG)), dim3(256), 0, stream, p,
                     (const T*)dO, dv, d.S, d.H, d.Hkv, BG, 1.f);
}

void launch_composed_fwd(int dtype, const Dims& d, const void* q, const void* k, const void* v,
                         void* o, float* lse, float* p, float scale, hipStream_t stream) {
  if (dtype == 0) {
    if (d.hd == 16) cmp_fwd_typed<float, 16>(d, q, k, v, o, lse, p, scale, stream);
    else if (d.hd == 32) cmp_fwd_typed<float, 32>(d, q, k, v, o, lse, p, scale, stream);
    else cmp_fwd_typed<float, 64>(d, q, k, v, o, lse, p, scale, stream);
  } else {
    if (d.hd == 16) cmp_fwd_typed<bf16, 16>(d, q, k, v, o, lse, p, scale, stream);
    else if (d.hd == 32) cmp_fwd_typed<bf16, 32>(d, q, k, v, o, lse, p, scale, stream);
    else cmp_fwd_typed<bf16, 64>(d, q, k, v, o, lse, p, scale, stream);
  }
}

void launch_composed_bwd(int dtype, const Dims& d, const void* q, const void* k, const void* v,
                         const float* p, const void* dO, float* dq, float* dk, float* dv,
                         float* ds, float scale, hipStream_t stream) {
  if (dtype == 0) {
    if (d.hd == 16) cmp_bwd_typed<float, 16>(d, q, k, v, p, dO, dq, dk, dv, ds, scale, stream);
    else if (d.hd == 32) cmp_bwd_typed<float, 32>(d, q, k, v, p, dO, dq, dk, dv, ds, scale, stream);
    else cmp_bwd_typed<float, 64>(d, q, k, v, p, dO, dq, dk, dv, ds, scale, stream);
  } else {
    if (d.hd == 16) cmp_bwd_typed<bf16, 16>(d, q, k, v, p, dO, dq, dk, dv, ds, scale, stream);
    else if (d.hd == 32) cmp_bwd_typed<bf16, 32>(d, q, k, v, p, dO, dq, dk, dv, ds, scale, stream);
    else cmp_bwd_typed<bf16, 64>(d, q, k, v, p, dO, dq, dk, dv, ds, scale, stream);
  }
}

}  // namespace xattn
