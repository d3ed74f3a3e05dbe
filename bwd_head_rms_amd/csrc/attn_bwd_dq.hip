// attn_bwd_dq.hip -- causal attention backward, query side, for gfx950.
//
// One workgroup per (batch, head, query tile): bf16 runs 4 waves of 32 query
// rows (128-row tiles), as in the forward; fp32 runs 64-row tiles, two waves
// of 32 rows at hd 64, and at hd <= 32 two waves per 32 rows, each taking half
// of every key tile, their partial dQ added at the end.  The prologue computes
//   D_i = sum_d dO_id * o_id
// (the simplification of the softmax Jacobian in the fused kernel of the
// "xtrain evolution overview", infra table row T14) and stores it for the
// dK/dV kernel.  Then, over the key tiles j <= i:
//   S^T  = K . Q^T,   P^T = exp2(S^T*scale*log2e - LSE_i*log2e)   (recompute)
//   dP^T = V . dO^T
//   dS^T = P^T * (dP^T - D_i)    (the product accumulates onto -D_i)
//   dQ^T += K^T . dS^T          (dS feeds the product from registers)
// and dq = scale * dQ is written in fp32.  The workspace receives -D and
// LSE*log2e per row ([2][B][H][S] floats) for the dK/dV kernel.  K and V tiles are copied into a
// double-buffered LDS ring (bf16: asynchronously, straight from HBM; one
// barrier per tile); K^T for the last product comes from the same K tile by
// transpose reads.  Query head h reads kv
// head h / (H / Hkv) by address.
#include <type_traits>

#include "attn_device.hpp"
#include "launch.hpp"

namespace xattn {

template <typename T, int HD>
struct DqCfg {
  // fp32 at hd 64 runs two waves (64 query rows) per workgroup: its kernel
  // then has a register budget of its own (277 + 21, one wave per SIMD)
  // instead of fitting four waves into 256, and runs a third faster
  // (measured: GQA fp32 workload 481 -> 314 us).  Everything else runs four,
  // one on each SIMD of the CU.
  // fp32 at hd <= 32: two row blocks of 32, each split over two waves by key
  // (KC = 2: wave (r, c) takes 32-key block c of every 64-key tile), the two
  // partial dQ added through LDS at the end
  static constexpr int KC = sizeof(T) == 4 && HD <= 32 ? 2 : 1;
  static constexpr int NR = sizeof(T) == 4 ? 2 : 4;  // row blocks
  static constexpr int NW = NR * KC, NT = NW * kWave, BM = 32 * NR, BN = 64, NB = BN / 32;
  static constexpr int ND = HD >= 32 ? HD / 32 : 1;
  static constexpr int NKS = HD / Mma<T>::KSTEP;
  static constexpr int NAS = 32 / Mma<T>::KSTEP;
  static constexpr int TILE = Tile<T, HD, BN>::ELEMS;
};

template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ o, const float* __restrict__ lse, const T* __restrict__ dO,
    float* __restrict__ dq, float* __restrict__ dws, const int* __restrict__ lens, int S, int H,
    int Hkv, int nqt, int BH, int ncu, float c, float scale) {
  using C = DqCfg<T, HD>;
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
  const size_t qplane = (size_t)bh * S * HD;
  const T* kp = k + ((size_t)b * Hkv + kvh) * S * HD;
  const T* vp = v + ((size_t)b * Hkv + kvh) * S * HD;
  const int n = seq_len(lens, b, S);  // rows and keys past n are padding
  if (qt * C::BM >= n) {              // a tile of padding only: dq = 0
    for (int r = tid; r < C::BM; r += C::NT)
      if (qt * C::BM + r < S) zero_row<HD>(dq + qplane + (size_t)(qt * C::BM + r) * HD);
    return;
  }

  // fp32 with four waves (hd <= 32: two row blocks x two key halves): the
  // role of a wave follows its SIMD, slot s for SIMD s in the first workgroup
  // a CU holds (blockIdx below the CU count), slot 3 - s in the second.  Slots
  // 0-1 hold the tile's first (lighter) row block, 2-3 the second, so each
  // SIMD pairs a heavy causal row block of one workgroup with a light one of
  // the other.  Any placement gives a permutation of the slots, so the results
  // do not depend on it.  (bf16, whose blocks are a quarter as long, measured
  // no gain.)
  int rw = wave, kc = 0;
  if constexpr (C::NW == 4 && sizeof(T) == 4) {
    __shared__ int simd_of[C::NW];
    const int rank = simd_rank<C::NW>(wave, lane, simd_of);
    const int slot = ncu > 0 && (blockIdx.x / ncu) % 2 == 1 ? C::NW - 1 - rank : rank;
    rw = slot / C::KC;
    kc = slot % C::KC;
  }
  const int q0 = qt * C::BM + rw * 32;
  const int my_q = q0 + li;
  const bool q_ok = my_q < n;
  const bool wave_live = q0 < n;
  const int wave_kv_end = min(n, q0 + 32);

  // bf16: the first key / value tile's copies into LDS go out before the
  // per-row loads, so the two fetches overlap (fp32 stages through registers
  // and copies after them)
  Stager<T, HD, C::BN, C::NW> stK, stV;
  if constexpr (sizeof(T) == 2) {
    stK.issue(kp, 0, n, sK[0], wave, lane, tid);
    stV.issue(vp, 0, n, sV[0], wave, lane, tid);
  }

  // Every per-row load goes out before any use, so they share one round trip:
  // a row past the sequence end reads row n-1 and its operands are zeroed.
  const int lrow = q_ok ? my_q : n - 1;
  typename M::frag qf[C::NKS], df[C::NKS], of[C::NKS];
  row_frags_global<T, HD>(q + qplane + (size_t)lrow * HD, g, qf);
  row_frags_global<T, HD>(dO + qplane + (size_t)lrow * HD, g, df);
  row_frags_global<T, HD>(o + qplane + (size_t)lrow * HD, g, of);
  const float lse_row = lse[(size_t)bh * S + lrow];
  float Dp = 0.f;
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int t = 0; t < 8; ++t) Dp += (float)of[ks][t] * (float)df[ks][t];
    } else {
      Dp += of[ks] * df[ks];
    }
  }
  if (!q_ok) {
    Dp = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      qf[ks] = zero_frag<T>();
      df[ks] = zero_frag<T>();
    }
  }
  const float Drow = halves_sum(Dp);
  const float lse2 = q_ok ? lse_row * kLog2e : 0.f;
  if (q_ok && g == 0 && kc == 0) {
    dws[(size_t)bh * S + my_q] = -Drow;  // negated: the dk/dv kernel starts dP from it
    dws[(size_t)BH * S + (size_t)bh * S + my_q] = lse2;  // for the dk/dv kernel
  }

  f32x16 acc[C::ND];
#pragma unroll
  for (int d = 0; d < C::ND; ++d) acc[d] = zero_acc();
  // dP^T accumulates onto -D, so the product yields dP - D directly
  f32x16 negD;
#pragma unroll
  for (int r = 0; r < 16; ++r) negD[r] = -Drow;

  const int kv_end = min(n, qt * C::BM + C::BM);
  const int ntiles = (kv_end + C::BN - 1) / C::BN;

  if constexpr (sizeof(T) == 4) {
    wait_global_loads();  // the per-row operands above are in registers
    stK.issue(kp, 0, n, sK[0], wave, lane, tid);
    stV.issue(vp, 0, n, sV[0], wave, lane, tid);
  }
  wait_global_loads();
  stK.commit(sK[0], tid);
  stV.commit(sV[0], tid);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int cur = j & 1;
    const int kv_t0 = j * C::BN;
    const bool more = j + 1 < ntiles;
    if (more) {  // the other buffer was last read before the previous barrier
      stK.issue(kp, kv_t0 + C::BN, n, sK[cur ^ 1], wave, lane, tid);
      stV.issue(vp, kv_t0 + C::BN, n, sV[cur ^ 1], wave, lane, tid);
    }
    if (wave_live && kv_t0 < wave_kv_end) {
      const T* tK = sK[cur];
      const T* tV = sV[cur];
      // One 32-key block.  Key blocks are 32-aligned like the wave's rows, so a
      // visited block is either wholly visible or the diagonal block; only the
      // diagonal block and the sequence tail carry a mask.
      auto block = [&](const int cb, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int kb0 = kv_t0 + 32 * cb;
        f32x16 s = zero_acc(), dp = negD;
        // A wave issuing matrix products runs at raised priority, so that its
        // products queue on the matrix core while the other waves of the SIMD
        // run their VALU work (measured: the kernel 5% faster).
        __builtin_amdgcn_s_setprio(2);
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
          M::mma(s, row_frag_lds<T, HD, C::BN>(tK, 32 * cb + li, g, ks), qf[ks]);
          M::mma(dp, row_frag_lds<T, HD, C::BN>(tV, 32 * cb + li, g, ks), df[ks]);
        }
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(fmaf(s[r], c, -lse2));
          if constexpr (MASK) {
            const int kv = kb0 + acc_row(r, g);
            p = (kv <= my_q && kv < n) ? p : 0.f;
          }
          s[r] = p * dp[r];  // dS^T = P (dP - D)
        }
        __builtin_amdgcn_s_setprio(2);
#pragma unroll
        for (int ks = 0; ks < C::NAS; ++ks) {
          const typename M::frag sf = acc_frag<T>(s, ks * M::KPL);
#pragma unroll
          for (int db = 0; db < C::ND; ++db) {
            M::mma(acc[db], accrow_frag<T, HD, C::BN>(tK, 32 * cb, ks, 32 * db, lane), sf);
          }
        }
        __builtin_amdgcn_s_setprio(0);
      };

#pragma unroll
      for (int cb = 0; cb < C::NB; ++cb) {
        const int kb0 = kv_t0 + 32 * cb;
        if (cb % C::KC != kc) continue;    // the other key half's block
        if (kb0 >= wave_kv_end) continue;  // wholly above this wave's rows, or past S
        if (kb0 + 31 > q0 || kb0 + 32 > n)
          block(cb, std::true_type{});
        else
          block(cb, std::false_type{});
      }
    }
    if (more) {
      wait_global_loads();
      stK.commit(sK[cur ^ 1], tid);
      stV.commit(sV[cur ^ 1], tid);
    }
    __syncthreads();
  }

  if constexpr (C::KC == 2) {
    // the second key half of each row block hands its partial dQ to the first
    // through the K buffers (every read of them ended at the last barrier)
    static_assert(C::NR * C::ND * 16 * kWave <= 2 * C::TILE, "partial dQ exceeds the K buffers");
    float* red = reinterpret_cast<float*>(&sK[0][0]);
    if (kc == 1) {
#pragma unroll
      for (int db = 0; db < C::ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[((rw * C::ND + db) * 16 + r) * kWave + lane] = acc[db][r];
    }
    __syncthreads();
    if (kc == 1) return;
#pragma unroll
    for (int db = 0; db < C::ND; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] += red[((rw * C::ND + db) * 16 + r) * kWave + lane];
  }

  if (!q_ok) {  // padding rows inside the sequence's last tile
    if (g == 0 && my_q < S) zero_row<HD>(dq + qplane + (size_t)my_q * HD);
    return;
  }
  float* qrow = dq + qplane + (size_t)my_q * HD;
#pragma unroll
  for (int db = 0; db < C::ND; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = 32 * db + 8 * rg + 4 * g;
      if (d0 < HD)
        store4<float>(qrow + d0, scale * acc[db][4 * rg], scale * acc[db][4 * rg + 1],
                      scale * acc[db][4 * rg + 2], scale * acc[db][4 * rg + 3]);
    }
}

template <typename T, int HD>
static void dq_typed(const Dims& d, const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dO, float* dq, float* dws, const int* lens,
                     float scale, hipStream_t stream) {
  using C = DqCfg<T, HD>;
  static_assert(C::BM == dq_tile_rows(sizeof(T) == 4 ? 0 : 1, HD) && C::NT <= kThreads,
                "tiling differs from the plan");
  const int nqt = (d.S + C::BM - 1) / C::BM;
  const int BH = d.B * d.H;
  dim3 grid((unsigned)attn_plan(d, sizeof(T) == 4 ? 0 : 1).dq_blocks), block(C::NT);
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, HD>), grid, block, 0, stream, (const T*)q,
                     (const T*)k, (const T*)v, (const T*)o, lse, (const T*)dO, dq, dws, lens, d.S,
                     d.H, d.Hkv, nqt, BH, device_cu_count(), scale * kLog2e, scale);
}

void launch_bwd_dq(int dtype, const Dims& d, const void* q, const void* k, const void* v,
                   const void* o, const float* lse, const void* dO, float* dq, float* dws,
                   const int* lens, float scale, hipStream_t stream) {
  if (dtype == 0) {
    if (d.hd == 16) dq_typed<float, 16>(d, q, k, v, o, lse, dO, dq, dws, lens, scale, stream);
    else if (d.hd == 32) dq_typed<float, 32>(d, q, k, v, o, lse, dO, dq, dws, lens, scale, stream);
    else dq_typed<float, 64>(d, q, k, v, o, lse, dO, dq, dws, lens, scale, stream);
  } else {
    if (d.hd == 16) dq_typed<bf16, 16>(d, q, k, v, o, lse, dO, dq, dws, lens, scale, stream);
    else if (d.hd == 32) dq_typed<bf16, 32>(d, q, k, v, o, lse, dO, dq, dws, lens, scale, stream);
    else dq_typed<bf16, 64>(d, q, k, v, o, lse, dO, dq, dws, lens, scale, stream);
  }
}

}  // namespace xattn
