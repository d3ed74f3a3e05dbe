// attn_fwd.hip -- fused causal attention forward for gfx950.
//
// One workgroup (4 waves) per (batch, head, 128-row query tile); each wave owns
// 32 query rows.  Key/value tiles of 64 rows are copied into a double-buffered
// LDS ring (bf16: asynchronously, straight from HBM into swizzled tiles; the
// copy of tile j+1 overlaps the arithmetic on tile j; one barrier per tile) and
// shared by the four waves.  Per tile and wave:
//   S^T = K . Q^T            (MFMA; keys are rows, queries are lanes, so every
//                              softmax row lives in one lane pair)
//   online softmax in the log2 domain: reference max m and sum l per query,
//   P = exp2(S*scale*log2e - m) (the row sum l accumulates P as rounded for
//   the product below); the row max is only taken, and the accumulator
//   rescaled by exp2(m_old - m_new), when the weights of a row outgrow a wide
//   bound (the online softmax of the fused kernel in the "xtrain evolution
//   overview", infra table row T14)
//   O^T += V^T . P^T          (MFMA; P feeds the product from registers, V^T
//                              comes from the row-major tile by transpose reads)
// Tiles wholly above the diagonal are never visited; blocks of 32 keys wholly
// above a wave's rows are skipped; the mask is applied only on the diagonal
// block and at the end of the sequence.  The epilogue writes O and the
// natural-log LSE = (m + log2 l) * ln 2.  Query head h reads kv head
// h / (H / Hkv) by address (GQA without a copy, row T15 of the same table).
// Work order: heaviest query tiles first.
#include "attn_device.hpp"
#include "launch.hpp"

namespace xattn {

// Bound on a row's per-tile sum of weights exp2(S*c - m) before its reference
// max m is renewed: weights stay below 2^64 (bf16 and fp32 reach 2^127), and the
// row sum l below 2^64 * S, so no precision or range is lost.
constexpr float kRescaleBound = 18446744073709551616.f;  // 2^64

template <typename T, int HD>
struct FwdCfg {
  static constexpr int NW = 4, NT = NW * kWave, BM = 32 * NW, BN = 64, NB = BN / 32;
  static constexpr int ND = HD >= 32 ? HD / 32 : 1;
  static constexpr int NKS = HD / Mma<T>::KSTEP;  // head-dim contraction steps
  static constexpr int NAS = 32 / Mma<T>::KSTEP;  // key contraction steps per 32-key block
  static constexpr int TILE = Tile<T, HD, BN>::ELEMS;
};

template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_fwd_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    T* __restrict__ o, float* __restrict__ lse, int S, int H, int Hkv, int nqt, int BH, float c) {
  using C = FwdCfg<T, HD>;
  using M = Mma<T>;
  __shared__ __align__(16) T sK[2][C::TILE];
  __shared__ __align__(16) T sV[2][C::TILE];

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int li = lane & 31, g = lane >> 5;
  const int bid = blockIdx.x;
  const int qt = nqt - 1 - bid / BH;
  const int bh = bid % BH;
  const int b = bh / H, h = bh % H;
  const int kvh = h / (H / Hkv);
  const T* qp = q + (size_t)bh * S * HD;
  const T* kp = k + ((size_t)b * Hkv + kvh) * S * HD;
  const T* vp = v + ((size_t)b * Hkv + kvh) * S * HD;

  const int q0 = qt * C::BM + wave * 32;
  const int my_q = q0 + li;
  const bool q_ok = my_q < S;
  const bool wave_live = q0 < S;
  const int wave_kv_end = min(S, q0 + 32);  // keys visible to some row of this wave

  typename M::frag qf[C::NKS];
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks)
    qf[ks] = q_ok ? row_frag_global<T, HD>(qp + (size_t)my_q * HD, g, ks) : zero_frag<T>();

  f32x16 oacc[C::ND];
#pragma unroll
  for (int d = 0; d < C::ND; ++d) oacc[d] = zero_acc();
  float m = -INFINITY, l = 0.f;

  const int kv_end = min(S, qt * C::BM + C::BM);
  const int ntiles = (kv_end + C::BN - 1) / C::BN;

  wait_global_loads();  // the query operand above is in registers
  Stager<T, HD, C::BN, C::NW> stK, stV;
  stK.issue(kp, 0, S, sK[0], wave, lane, tid);
  stV.issue(vp, 0, S, sV[0], wave, lane, tid);
  wait_global_loads();
  stK.commit(sK[0], tid);
  stV.commit(sV[0], tid);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int cur = j & 1;
    const int kv_t0 = j * C::BN;
    const bool more = j + 1 < ntiles;
    if (more) {  // the other buffer was last read before the previous barrier
      stK.issue(kp, kv_t0 + C::BN, S, sK[cur ^ 1], wave, lane, tid);
      stV.issue(vp, kv_t0 + C::BN, S, sV[cur ^ 1], wave, lane, tid);
    }
    if (wave_live && kv_t0 < wave_kv_end) {
      const T* tK = sK[cur];
      const T* tV = sV[cur];
      // Scores of the (up to) two 32-key blocks of this tile.  Key blocks are
      // 32-aligned like the wave's rows: a visited block is wholly visible or
      // the diagonal block, and only the diagonal block and the sequence tail
      // carry a mask (masked scores become -inf, i.e. weight exactly 0).
      bool act[C::NB];
#pragma unroll
      for (int cb = 0; cb < C::NB; ++cb) act[cb] = kv_t0 + 32 * cb < wave_kv_end;
      f32x16 s[C::NB];
      auto scores = [&]() {
#pragma unroll
        for (int cb = 0; cb < C::NB; ++cb) {
          const int kb0 = kv_t0 + 32 * cb;
          s[cb] = zero_acc();
          if (act[cb]) {
#pragma unroll
            for (int ks = 0; ks < C::NKS; ++ks)
              M::mma(s[cb], row_frag_lds<T, HD, C::BN>(tK, 32 * cb + li, g, ks), qf[ks]);
            if (kb0 + 31 > q0 || kb0 + 32 > S) {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int kv = kb0 + acc_row(r, g);
                s[cb][r] = (kv <= my_q && kv < S) ? s[cb][r] : -INFINITY;
              }
            }
          }
        }
      };
      // P = exp2(S*c - m) as operand fragments, and the row's partial sum of P
      // (the same rounded weights that enter the product below).
      typename M::frag pf[C::NB][C::NAS];
      float tsum = 0.f;
      auto probs = [&]() {
        tsum = 0.f;
#pragma unroll
        for (int cb = 0; cb < C::NB; ++cb) {
          if (!act[cb]) continue;
#pragma unroll
          for (int r = 0; r < 16; ++r) s[cb][r] = fast_exp2(fmaf(s[cb][r], c, -m));
#pragma unroll
          for (int ks = 0; ks < C::NAS; ++ks) {
            pf[cb][ks] = acc_frag<T>(s[cb], ks * M::KPL);
            tsum = frag_sum(pf[cb][ks], tsum);
          }
        }
      };
      scores();
      probs();
      // Each row keeps a reference max m and uses it as long as its weights
      // stay below 2^kRescaleSlack (their sum bounds every weight).  Only when
      // that fails -- the row's first tile (m = -inf), or scores that really
      // outgrew m -- are the scores recomputed, the row max taken and the
      // accumulator rescaled.  The decision is per row (rows that pass keep m
      // and recompute the same weights), so every row's result depends only
      // on that row's scores.
      const bool fail = halves_max(tsum <= kRescaleBound ? 0.f : 1.f) != 0.f;
      if (__ballot(fail)) {
        scores();
        float mx = -INFINITY;
#pragma unroll
        for (int cb = 0; cb < C::NB; ++cb)
          if (act[cb]) {
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[cb][r]);
          }
        mx = halves_max(mx) * c;
        const float m_new = fail ? fmaxf(m, mx) : m;
        const float alpha = fail ? fast_exp2(m - m_new) : 1.f;
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int d = 0; d < C::ND; ++d) oacc[d] *= alpha;
        probs();
      }
      l += tsum;
#pragma unroll
      for (int cb = 0; cb < C::NB; ++cb) {
        if (!act[cb]) continue;
#pragma unroll
        for (int ks = 0; ks < C::NAS; ++ks)
#pragma unroll
          for (int db = 0; db < C::ND; ++db)
            M::mma(oacc[db], accrow_frag<T, HD, C::BN>(tV, 32 * cb, ks, 32 * db, lane), pf[cb][ks]);
      }
    }
    if (more) {
      wait_global_loads();
      stK.commit(sK[cur ^ 1], tid);
      stV.commit(sV[cur ^ 1], tid);
    }
    __syncthreads();
  }

  if (!wave_live) return;
  l = halves_sum(l);
  const float inv = 1.f / l;
  if (q_ok) {
    T* orow = o + ((size_t)bh * S + my_q) * HD;
#pragma unroll
    for (int db = 0; db < C::ND; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = 32 * db + 8 * rg + 4 * g;
        if (d0 < HD)
          store4<T>(orow + d0, oacc[db][4 * rg] * inv, oacc[db][4 * rg + 1] * inv,
                    oacc[db][4 * rg + 2] * inv, oacc[db][4 * rg + 3] * inv);
      }
    if (g == 0) lse[(size_t)bh * S + my_q] = (m + fast_log2(l)) * kLn2;
  }
}

template <typename T, int HD>
static void fwd_typed(const Dims& d, const void* q, const void* k, const void* v, void* o,
                      float* lse, float scale, hipStream_t stream) {
  using C = FwdCfg<T, HD>;
  const int nqt = (d.S + C::BM - 1) / C::BM;
  const int BH = d.B * d.H;
  dim3 grid((unsigned)(nqt * BH)), block(C::NT);
  hipLaunchKernelGGL((attn_fwd_kernel<T, HD>), grid, block, 0, stream,
                     (const T*)q, (const T*)k, (const T*)v, (T*)o, lse, d.S, d.H, d.Hkv, nqt, BH,
                     scale * kLog2e);
}

void launch_fwd(int dtype, const Dims& d, const void* q, const void* k, const void* v, void* o,
                float* lse, float scale, hipStream_t stream) {
  if (dtype == 0) {
    if (d.hd == 16) fwd_typed<float, 16>(d, q, k, v, o, lse, scale, stream);
    else if (d.hd == 32) fwd_typed<float, 32>(d, q, k, v, o, lse, scale, stream);
    else fwd_typed<float, 64>(d, q, k, v, o, lse, scale, stream);
  } else {
    if (d.hd == 16) fwd_typed<bf16, 16>(d, q, k, v, o, lse, scale, stream);
    else if (d.hd == 32) fwd_typed<bf16, 32>(d, q, k, v, o, lse, scale, stream);
    else fwd_typed<bf16, 64>(d, q, k, v, o, lse, scale, stream);
  }
}

}  // namespace xattn
