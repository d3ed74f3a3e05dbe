// decode_attn.hip -- decode attention for gfx950: one new query per (sequence,
// query head) against that sequence's cached keys and values.
//
// The operation is the last row of causal attention ("xtrain evolution
// overview", post-training stage, milestone M2a: one query against the cached
// K/V with an ordinary softmax, equal to the last row of full causal attention;
// M2b: sequences decoded together each bring their own cache; M2c: the cache is
// device-resident, one [T, hd] plane per (sequence, kv head)).  Query head h
// reads kv head h / group as in row T15 of the same page's infra table.
//
// It is HBM-bound: every cached key and value is read once and the arithmetic
// per byte is small (4 * group flops per 2 bytes of bf16 cache), so the design
// goal is a streaming read of the cache with enough bytes in flight, not matrix
// cores.  Work split ("split-K" over the cache):
//   * a workgroup takes one kv head of one sequence, a chunk of C positions of
//     its cache, and GC of the query heads that read that kv head (all of the
//     group when it is at most 8), so each K/V byte is read once per GC heads;
//   * lanes split a key row into 16-byte pieces (TPK lanes per key), so a wave
//     reads KPW consecutive rows, one contiguous 1 KB (bf16 hd 64) block, per
//     load instruction;
//   * pass 1 computes the chunk's scores into LDS and their maximum, an exp
//     pass turns them into weights and their sum, pass 2 accumulates the
//     weighted values -- no rescaling of running sums is ever needed (bf16
//     rounds the weights to bf16 for pass 2, as the forward's P.V product
//     does, and adds two positions per v_dot2_f32_bf16);
//   * with more than one chunk per sequence each workgroup writes its partial
//     (unnormalised sum, max, weight sum) and a second kernel merges the chunks
//     in ascending order.  Fixed orders throughout: results are bitwise
//     reproducible run to run.
// Scores are kept in base-2 units (multiplied by scale * log2 e); bf16 scores
// use v_dot2_f32_bf16 on the packed query and key pieces.
#include "attn_device.hpp"
#include "launch.hpp"

namespace xattn {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / kWave;
// Most chunks per sequence the merge kernel takes (its LDS holds one weight per
// chunk); longer caches use longer chunks.
constexpr int kDecMaxChunkRecords = 4096;
static_assert((long)kDecMaxChunk * kDecMaxChunkRecords == kDecodeMaxT, "decode limits");

template <typename T, int HD>
struct DecCfg {
  static constexpr int EPL = 16 / (int)sizeof(T);  // elements per lane per load
  static constexpr int TPK = HD / EPL;             // lanes per key row
  static constexpr int KPW = kWave / TPK;          // keys per wave per round
  static constexpr int KPR = kDecWaves * KPW;      // keys per workgroup per round
  static_assert(TPK >= 1 && TPK <= kWave && kDecMaxChunk % KPR == 0, "decode tiling");
};

// 16 bytes of a row, kept raw while the load is in flight, widened to EPL
// floats where they are used
__device__ __forceinline__ uint4 load_raw(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
template <typename T>
__device__ __forceinline__ void widen(const uint4& r, float* out);
template <>
__device__ __forceinline__ void widen<float>(const uint4& r, float* out) {
  out[0] = __builtin_bit_cast(float, r.x); out[1] = __builtin_bit_cast(float, r.y);
  out[2] = __builtin_bit_cast(float, r.z); out[3] = __builtin_bit_cast(float, r.w);
}
template <>
__device__ __forceinline__ void widen<bf16>(const uint4& r, float* out) {
  const bf16x8 v = __builtin_bit_cast(bf16x8, r);
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = (float)v[e];
}
template <typename T>
__device__ __forceinline__ void load_piece(const T* p, float* out) {
  widen<T>(load_raw(p), out);
}

template <typename T>
__device__ __forceinline__ void store_one(T* p, float x);
template <>
__device__ __forceinline__ void store_one<float>(float* p, float x) { *p = x; }
template <>
__device__ __forceinline__ void store_one<bf16>(bf16* p, float x) { *p = (bf16)x; }

// Partial record of one (sequence, query head, chunk) in the workspace:
// HD unnormalised weighted-value sums, then the chunk's max score (base 2) and
// its weight sum.
template <int HD>
struct Part {
  static constexpr int STRIDE = HD + 2;
};

template <typename T, int HD, int GC>
__global__ __launch_bounds__(kDecThreads) void decode_attn_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int* __restrict__ lens, T* __restrict__ o, float* __restrict__ lse,
    float* __restrict__ part, int Tc, int H, int Hkv, int group, int nsplit, int chunk,
    float scale_log2) {
  using C = DecCfg<T, HD>;
  constexpr int EPL = C::EPL, TPK = C::TPK, KPW = C::KPW, KPR = C::KPR;
  // loads in flight per thread; a chunk's rounds (chunk / KPR, chunk a power of
  // two >= kDecMinChunk) are a multiple of U
  // (4 measured best: deeper pipelines cost registers, hence resident waves)
  constexpr int U = 4 < kDecMinChunk / KPR ? 4 : kDecMinChunk / KPR;
  // scores, then weights, position-major: the GC heads of a position are one
  // 4-16 byte LDS read in pass 2
  __shared__ __align__(16) float sc[kDecMaxChunk][GC];
  __shared__ float red[kDecWaves][GC][HD];
  __shared__ float wred[kDecWaves][GC];

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int slot = lane / TPK, piece = lane % TPK;
  const int split = blockIdx.x % nsplit;
  const int unit = blockIdx.x / nsplit;  // (b * Hkv + g) * nhc + hc
  const int nhc = group / GC;
  const int hc = unit % nhc;
  const int bg = unit / nhc;  // b * Hkv + g
  const int b = bg / Hkv, g = bg % Hkv;
  const int h0 = g * group + hc * GC;

  int n = lens ? lens[b] : Tc;
  n = n < 0 ? 0 : (n > Tc ? Tc : n);
  const int j0 = split * chunk;
  const int j1 = min(j0 + chunk, n);

  if (j0 >= j1) {  // nothing cached in this chunk
    if (nsplit == 1) {
      for (int i = tid; i < GC * HD; i += kDecThreads)
        store_one<T>(o + (size_t)(b * H + h0 + i / HD) * HD + i % HD, 0.f);
      if (tid < GC) lse[b * H + h0 + tid] = -__builtin_inff();
    } else {
      for (int i = tid; i < GC * (HD + 2); i += kDecThreads) {
        const int t = i / (HD + 2), d = i % (HD + 2);
        part[((size_t)(b * H + h0 + t) * nsplit + split) * Part<HD>::STRIDE + d] =
            d == HD ? -__builtin_inff() : 0.f;
      }
    }
    return;
  }

  // the query piece: bf16 stays packed (its products with bf16 keys are exact
  // in fp32 and go through v_dot2_f32_bf16, scaled after the sum); fp32 is
  // pre-scaled by scale * log2 e
  float qv[GC][sizeof(T) == 2 ? 1 : EPL];
  uint4 qraw[GC];
#pragma unroll
  for (int t = 0; t < GC; ++t) {
    qraw[t] = load_raw(q + (size_t)(b * H + h0 + t) * HD + piece * EPL);
    if constexpr (sizeof(T) == 4) {
      widen<T>(qraw[t], qv[t]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) qv[t][e] *= scale_log2;
    }
  }

  const size_t plane = ((size_t)b * Hkv + g) * (size_t)Tc * HD;
  const T* kp = k + plane + piece * EPL;
  const T* vp = v + plane + piece * EPL;
  const int rounds = chunk / KPR;

  // pass 1: scores of the chunk (base 2) into LDS, and this thread's maximum.
  // Rolling pipeline: slot u holds the key piece of round r0 + u and is refilled
  // with round r0 + u + U as soon as it is used, so U loads stay in flight.
  // A round past the cached length loads the last cached row instead (always
  // in bounds) and scores -inf.
  auto row_of = [&](int r) __attribute__((always_inline)) {
    const int j = j0 + r * KPR + wave * KPW + slot;
    return (size_t)(j < j1 ? j : j1 - 1) * HD;
  };
  float mloc[GC];
#pragma unroll
  for (int t = 0; t < GC; ++t) mloc[t] = -__builtin_inff();
  uint4 buf[U];
#pragma unroll
  for (int u = 0; u < U; ++u) buf[u] = load_raw(kp + row_of(u));
  for (int r0 = 0; r0 < rounds; r0 += U) {  // rounds is a multiple of U
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u;
      const int jj = r * KPR + wave * KPW + slot;  // position within the chunk
      const bool live = j0 + jj < j1;
      float sv[GC];
      if constexpr (sizeof(T) == 2) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x8 kb = __builtin_bit_cast(bf16x8, buf[u]);
#pragma unroll
        for (int t = 0; t < GC; ++t) {
          const bf16x8 qb = __builtin_bit_cast(bf16x8, qraw[t]);
          float a = 0.f;
#pragma unroll
          for (int e = 0; e < 8; e += 2)
            a = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{qb[e], qb[e + 1]}, bf16x2{kb[e], kb[e + 1]}, a,
                                                false);
          sv[t] = a * scale_log2;
        }
      } else {
        float kv[EPL];
        widen<T>(buf[u], kv);
#pragma unroll
        for (int t = 0; t < GC; ++t) {
          float acc1 = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc1 += qv[t][e] * kv[e];
          sv[t] = acc1;
        }
      }
      // refill (past the last round: the chunk's last row again, a cache hit)
      buf[u] = load_raw(kp + row_of(r + U < rounds ? r + U : rounds - 1));
#pragma unroll
      for (int off = 1; off < TPK; off *= 2) {
#pragma unroll
        for (int t = 0; t < GC; ++t) sv[t] += __shfl_xor(sv[t], off);
      }
#pragma unroll
      for (int t = 0; t < GC; ++t) {
        const float st = live ? sv[t] : -__builtin_inff();
        mloc[t] = fmaxf(mloc[t], st);
        if (t % TPK == piece) sc[jj][t] = st;
      }
    }
  }

  // maximum of each head's scores over the workgroup
#pragma unroll
  for (int t = 0; t < GC; ++t) {
#pragma unroll
    for (int off = TPK; off < kWave; off *= 2) mloc[t] = fmaxf(mloc[t], __shfl_xor(mloc[t], off));
  }
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < GC; ++t) wred[wave][t] = mloc[t];
  }
  __syncthreads();
  float M[GC];
#pragma unroll
  for (int t = 0; t < GC; ++t) {
    M[t] = wred[0][t];
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w) M[t] = fmaxf(M[t], wred[w][t]);
  }
  __syncthreads();  // wred is reused for the weight sums

  // first U rounds of values in flight while the weights are formed
#pragma unroll
  for (int u = 0; u < U; ++u) buf[u] = load_raw(vp + row_of(u));

  // weights exp2(s - M) in place, and each head's weight sum
  float lsum[GC];
#pragma unroll
  for (int t = 0; t < GC; ++t) lsum[t] = 0.f;
  for (int jj = tid; jj < chunk; jj += kDecThreads) {
#pragma unroll
    for (int t = 0; t < GC; ++t) {
      const float p = fast_exp2(sc[jj][t] - M[t]);
      sc[jj][t] = p;
      lsum[t] += p;
    }
  }
#pragma unroll
  for (int t = 0; t < GC; ++t) {
#pragma unroll
    for (int off = 1; off < kWave; off *= 2) lsum[t] += __shfl_xor(lsum[t], off);
  }
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < GC; ++t) wred[wave][t] = lsum[t];
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < GC; ++t) {
    lsum[t] = wred[0][t];
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w) lsum[t] += wred[w][t];
  }

  // pass 2: weighted values, the same rolling pipeline over V (a round past the
  // cached length has weight 0 and its piece is zeroed)
  float acc[GC][EPL];
#pragma unroll
  for (int t = 0; t < GC; ++t)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[t][e] = 0.f;
  if constexpr (sizeof(T) == 2) {
    // bf16 takes the rounds in pairs: the two weights of a head are rounded to
    // bf16 (as the forward rounds P before its P.V product) and each element
    // of the two value pieces forms a bf16 pair, so one v_dot2_f32_bf16 adds
    // both rounds' terms of an element (exact products, fp32 sum)
    static_assert(U % 2 == 0, "rounds are taken in pairs");
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const uint4 zero = {0u, 0u, 0u, 0u};
    for (int r0 = 0; r0 < rounds; r0 += U) {
#pragma unroll
      for (int u = 0; u < U; u += 2) {
        const int r = r0 + u;
        const int jj = r * KPR + wave * KPW + slot;  // round r; round r + 1 is jj + KPR
        const bf16x8 va = __builtin_bit_cast(bf16x8, j0 + jj < j1 ? buf[u] : zero);
        const bf16x8 vb = __builtin_bit_cast(bf16x8, j0 + jj + KPR < j1 ? buf[u + 1] : zero);
        buf[u] = load_raw(vp + row_of(r + U < rounds ? r + U : rounds - 1));
        buf[u + 1] = load_raw(vp + row_of(r + 1 + U < rounds ? r + 1 + U : rounds - 1));
#pragma unroll
        for (int t = 0; t < GC; ++t) {
          const bf16x2 pp = {(__bf16)sc[jj][t], (__bf16)sc[jj + KPR][t]};
#pragma unroll
          for (int e = 0; e < EPL; ++e)
            acc[t][e] = __builtin_amdgcn_fdot2_f32_bf16(pp, bf16x2{va[e], vb[e]}, acc[t][e], false);
        }
      }
    }
  } else {
    for (int r0 = 0; r0 < rounds; r0 += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = r0 + u;
        const int jj = r * KPR + wave * KPW + slot;
        const bool live = j0 + jj < j1;
        float vv[EPL];
        widen<T>(buf[u], vv);
#pragma unroll
        for (int e = 0; e < EPL; ++e) vv[e] = live ? vv[e] : 0.f;
        buf[u] = load_raw(vp + row_of(r + U < rounds ? r + U : rounds - 1));
#pragma unroll
        for (int t = 0; t < GC; ++t) {
          const float p = sc[jj][t];
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[t][e] += p * vv[e];
        }
      }
    }
  }

  // sum over the key slots of a wave (lanes of equal piece), then over waves
#pragma unroll
  for (int off = TPK; off < kWave; off *= 2) {
#pragma unroll
    for (int t = 0; t < GC; ++t)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[t][e] += __shfl_xor(acc[t][e], off);
  }
  if (slot == 0) {
#pragma unroll
    for (int t = 0; t < GC; ++t)
#pragma unroll
      for (int e = 0; e < EPL; ++e) red[wave][t][piece * EPL + e] = acc[t][e];
  }
  __syncthreads();
  for (int i = tid; i < GC * HD; i += kDecThreads) {
    const int t = i / HD, d = i % HD;
    float a = red[0][t][d];
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w) a += red[w][t][d];
    const int h = h0 + t;
    float mt = M[0], lt = lsum[0];
#pragma unroll
    for (int u = 1; u < GC; ++u)
      if (t == u) { mt = M[u]; lt = lsum[u]; }
    if (nsplit == 1) {
      store_one<T>(o + (size_t)(b * H + h) * HD + d, a / lt);
      if (d == 0) lse[b * H + h] = (mt + fast_log2(lt)) * kLn2;
    } else {
      float* pr = part + ((size_t)(b * H + h) * nsplit + split) * Part<HD>::STRIDE;
      pr[d] = a;
      if (d == 0) {
        pr[HD] = mt;
        pr[HD + 1] = lt;
      }
    }
  }
}

// Merge the chunks of each (sequence, query head): one workgroup per row.
// Every load is issued up front (the weighted sums do not depend on the row
// max): thread c brings chunk c's max and weight sum, thread t the element
// d = t % HD of chunks t / HD, t / HD + NG, ... (NG = 256 / HD groups).  The
// row max and the merged weight sum are reduced in a fixed order (within each
// wave, then across the 4 waves in ascending order), the NG group sums of each
// element in ascending group order.
template <typename T, int HD>
__global__ __launch_bounds__(kDecThreads) void decode_combine_kernel(
    const float* __restrict__ part, T* __restrict__ o, float* __restrict__ lse, int nsplit) {
  constexpr int NG = kDecThreads / HD;
  constexpr int CR = 8;  // chunk records per thread held in registers
  constexpr int STRIDE = Part<HD>::STRIDE;
  __shared__ float wmax[kDecWaves], wsum[kDecWaves];
  __shared__ float wsc[kDecMaxChunkRecords];
  __shared__ float acc_g[NG][HD];
  const int row = blockIdx.x, t = threadIdx.x, wave = t / kWave;
  const int d = t % HD, g0 = t / HD;
  const float* pr = part + (size_t)row * nsplit * STRIDE;

  float pre[CR];
#pragma unroll
  for (int i = 0; i < CR; ++i) {
    const int c = g0 + NG * i;
    pre[i] = c < nsplit ? pr[(size_t)c * STRIDE + d] : 0.f;
  }
  float m0 = -__builtin_inff(), l0 = 0.f;  // chunk t's record
  if (t < nsplit) {
    m0 = pr[(size_t)t * STRIDE + HD];
    l0 = pr[(size_t)t * STRIDE + HD + 1];
  }
  float m = m0;
  for (int c = t + kDecThreads; c < nsplit; c += kDecThreads)
    m = fmaxf(m, pr[(size_t)c * STRIDE + HD]);

#pragma unroll
  for (int off = 1; off < kWave; off *= 2) m = fmaxf(m, __shfl_xor(m, off));
  if (t % kWave == 0) wmax[wave] = m;
  __syncthreads();
  float M = wmax[0];
#pragma unroll
  for (int w = 1; w < kDecWaves; ++w) M = fmaxf(M, wmax[w]);
  if (M == -__builtin_inff()) {  // empty sequence
    if (t < HD) store_one<T>(o + (size_t)row * HD + t, 0.f);
    if (t == 0) lse[row] = -__builtin_inff();
    return;
  }
  // chunk weights (0 for an empty chunk, whose max is -inf) and the merged weight sum
  float l = 0.f;
  if (t < nsplit) {
    const float w = fast_exp2(m0 - M);
    wsc[t] = w;
    l = w * l0;
  }
  for (int c = t + kDecThreads; c < nsplit; c += kDecThreads) {
    const float w = fast_exp2(pr[(size_t)c * STRIDE + HD] - M);
    wsc[c] = w;
    l += w * pr[(size_t)c * STRIDE + HD + 1];
  }
#pragma unroll
  for (int off = 1; off < kWave; off *= 2) l += __shfl_xor(l, off);
  if (t % kWave == 0) wsum[wave] = l;
  __syncthreads();
  float L = wsum[0];
#pragma unroll
  for (int w = 1; w < kDecWaves; ++w) L += wsum[w];

  float a = 0.f;
#pragma unroll
  for (int i = 0; i < CR; ++i) {
    const int c = g0 + NG * i;
    if (c < nsplit) a += wsc[c] * pre[i];
  }
  for (int c = g0 + NG * CR; c < nsplit; c += NG) a += wsc[c] * pr[(size_t)c * STRIDE + d];
  acc_g[g0][d] = a;
  __syncthreads();
  if (t < HD) {
    float sum = acc_g[0][t];
#pragma unroll
    for (int g = 1; g < NG; ++g) sum += acc_g[g][t];
    store_one<T>(o + (size_t)row * HD + t, sum / L);
    if (t == 0) lse[row] = (M + fast_log2(L)) * kLn2;
  }
}

template <typename T, int HD, int GC>
static void decode_launch(const Dims& d, const DecodePlan& p, const void* q, const void* k,
                          const void* v, const int* lens, void* o, float* lse, float* part,
                          float scale, hipStream_t stream) {
  const int group = d.H / d.Hkv;
  const dim3 grid((unsigned)p.blocks);
  hipLaunchKernelGGL((decode_attn_kernel<T, HD, GC>), grid, dim3(kDecThreads), 0, stream,
                     (const T*)q, (const T*)k, (const T*)v, lens, (T*)o, lse, part, d.S, d.H,
                     d.Hkv, group, p.nsplit, p.chunk, scale * kLog2e);
  if (p.nsplit > 1) {
    hipLaunchKernelGGL((decode_combine_kernel<T, HD>), dim3((unsigned)p.combine_blocks),
                       dim3(kDecThreads), 0, stream, part, (T*)o, lse, p.nsplit);
  }
}

template <typename T, int HD>
static void decode_hd(const Dims& d, const DecodePlan& p, const void* q, const void* k,
                      const void* v, const int* lens, void* o, float* lse, float* part,
                      float scale, hipStream_t stream) {
  switch (p.heads_per_wg) {
    case 8: decode_launch<T, HD, 8>(d, p, q, k, v, lens, o, lse, part, scale, stream); break;
    case 4: decode_launch<T, HD, 4>(d, p, q, k, v, lens, o, lse, part, scale, stream); break;
    case 2: decode_launch<T, HD, 2>(d, p, q, k, v, lens, o, lse, part, scale, stream); break;
    default: decode_launch<T, HD, 1>(d, p, q, k, v, lens, o, lse, part, scale, stream); break;
  }
}

void launch_decode(int dtype, const Dims& d, const void* q, const void* k, const void* v,
                   const int* lens, void* o, float* lse, float* part, float scale,
                   hipStream_t stream) {
  const DecodePlan p = decode_plan(d.B, d.S, d.H, d.Hkv, d.hd);
  if (dtype == 0) {
    if (d.hd == 16) decode_hd<float, 16>(d, p, q, k, v, lens, o, lse, part, scale, stream);
    else if (d.hd == 32) decode_hd<float, 32>(d, p, q, k, v, lens, o, lse, part, scale, stream);
    else decode_hd<float, 64>(d, p, q, k, v, lens, o, lse, part, scale, stream);
  } else {
    if (d.hd == 16) decode_hd<bf16, 16>(d, p, q, k, v, lens, o, lse, part, scale, stream);
    else if (d.hd == 32) decode_hd<bf16, 32>(d, p, q, k, v, lens, o, lse, part, scale, stream);
    else decode_hd<bf16, 64>(d, p, q, k, v, lens, o, lse, part, scale, stream);
  }
}

}  // namespace xattn
