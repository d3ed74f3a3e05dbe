// attn_bwd_dkdv.hip -- causal attention backward, key/value side, for gfx950.
//
// One workgroup (4 waves) per (batch, kv head, key tile): 128 keys, a wave per
// 32 (fp32 at hd <= 32: 64 keys, two waves per 32, each taking every other
// query block, their sums added at the end).  A wave's K and V operands stay in
// registers for the whole kernel.
// The workgroup walks every query head of its GQA group (r ascending) and, for
// each, the query tiles (128 rows for bf16, 64 for fp32) at or below the
// diagonal (ascending), copying Q and dO (bf16: asynchronously, straight from
// HBM into swizzled tiles), LSE and D into a double-buffered LDS ring (one
// barrier per tile).  Per 32-row query block and wave:
//   S  = Q . K^T,   P = exp2(S*scale*log2e - LSE_i*log2e)     (recompute)
//   dP = dO . V^T,  dS = P * (dP - D_i)
//   dV^T += dO^T . P          (P feeds the product from registers; dO^T and
//   dK^T += Q^T . dS           Q^T come from the row-major tiles by transpose
//                              reads)
// dk = scale * dK and dv are written in fp32 once.  The GQA group sum happens in
// registers in a fixed order (head r, then query tile), with no atomics, so the
// result is bitwise reproducible (the deterministic group sum of the
// "xtrain evolution overview", infra table row T15).  D comes from the dq
// kernel, which runs first on the same stream.  Work order: heaviest key tiles
// (those near the start of the sequence) first, dealt so that the two
// workgroups a CU holds at once carry about equal work.
#include <type_traits>

#include "attn_device.hpp"
#include "launch.hpp"

namespace xattn {

template <typename T, int HD>
struct DkvCfg {
  // fp32 at hd <= 32 gives each 32-key block two waves, each taking every
  // other query block (QS = 2), and adds their sums through LDS at the end:
  // the first key block's serial chain of 64-cycle fp32 products is halved
  // (at S = 256 its 8 query blocks become 4 per wave)
  static constexpr int QS = sizeof(T) == 4 && HD <= 32 ? 2 : 1;
  static constexpr int NW = 4, NT = NW * kWave, BN = 32 * NW / QS;
  static constexpr int BMQ = sizeof(T) == 2 ? 128 : 64;  // query rows per staged tile
  static constexpr int NQB = BMQ / 32;
  static constexpr int ND = HD >= 32 ? HD / 32 : 1;
  static constexpr int NKS = HD / Mma<T>::KSTEP;
  static constexpr int NAS = 32 / Mma<T>::KSTEP;
  static constexpr int TILE = Tile<T, HD, BMQ>::ELEMS;
};

// bf16 keeps the long-lived dK/dV sums in AGPRs at hd 64 (two waves per SIMD
// either way); at hd 32 they stay in VGPRs so that the kernel fits three waves
// per SIMD (168 registers) without the compiler's even VGPR/AGPR split.
template <int HD>
constexpr bool kDkvAgpr = HD == 64;

template <typename T, int HD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(HD == 32 ? 3 : 1))) void attn_bwd_dkdv_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ lse, const T* __restrict__ dO, const float* __restrict__ dws,
    float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ part,
    const int* __restrict__ lens, int B, int S, int H, int Hkv, int nkt, int BG, int R, int ncu,
    float c, float scale) {
  using C = DkvCfg<T, HD>;
  using M = Mma<T>;
  __shared__ __align__(16) T sQ[2][C::TILE];
  __shared__ __align__(16) T sO[2][C::TILE];  // dO
  __shared__ __align__(16) float sL[2][C::BMQ];  // LSE * log2e (rows read four at a time)
  __shared__ __align__(16) float sD[2][C::BMQ];

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int li = lane & 31, g = lane >> 5;
  // key tile 0 (the heaviest) first, balanced over the two workgroups a CU
  // holds at once (two waves per SIMD)
  const int bid = balanced_rank(blockIdx.x, gridDim.x, ncu, 2);
  const int kt = bid / (BG * R);
  const int bg = bid % BG;
  const int rs = (bid / BG) % R;  // which of the R slices of the group's query heads
  const int b = bg / Hkv, kvh = bg % Hkv;
  const int group = H / Hkv;
  const size_t kvplane = ((size_t)b * Hkv + kvh) * S * HD;
  // With R > 1 the group is split over R workgroups, each taking H/Hkv/R
  // consecutive query heads: slice rs writes its partial dK, dV into plane rs
  // of `part` ([2][R][B][Hkv][S][hd] in the workspace), summed afterwards in
  // ascending rs by dkdv_group_sum_kernel.
  const size_t kv_elems = (size_t)B * Hkv * S * HD;
  float* outk = R > 1 ? part + (size_t)rs * kv_elems : dk;
  float* outv = R > 1 ? part + (size_t)(R + rs) * kv_elems : dv;
  const int n = seq_len(lens, b, S);  // rows and keys past n are padding
  if (kt * C::BN >= n) {              // a tile of padding keys only: dk = dv = 0
    for (int r = tid; r < C::BN; r += C::NT)
      if (kt * C::BN + r < S) {
        zero_row<HD>(outk + kvplane + (size_t)(kt * C::BN + r) * HD);
        zero_row<HD>(outv + kvplane + (size_t)(kt * C::BN + r) * HD);
      }
    return;
  }

  // The key block a wave owns follows its SIMD: block s for SIMD s in the first
  // workgroup a CU holds (blockIdx below the CU count), block 3 - s in the
  // second.  Causal key blocks near the start of a tile carry the most query
  // blocks, so each SIMD pairs a heavy block of one workgroup with a light
  // block of the other (at S = 256: 8 + 1, 7 + 2, 6 + 3, 5 + 4 query blocks,
  // where wave-index order put 8 + 3 on one SIMD).  Any placement gives a
  // permutation of the blocks, so the results do not depend on it.
  __shared__ int simd_of[C::NW];
  const int rank = simd_rank<C::NW>(wave, lane, simd_of);
  const int slot = ncu > 0 && (blockIdx.x / ncu) % 2 == 1 ? C::NW - 1 - rank : rank;
  const int kb_w = slot / C::QS, qh = slot % C::QS;  // key block, query half
  const int kv0 = kt * C::BN + kb_w * 32;
  const int my_kv = kv0 + li;
  const bool kv_ok = my_kv < n;
  const bool wave_live = kv0 < n;

  const int qt_first = (kt * C::BN) / C::BMQ;
  const int nq = (n + C::BMQ - 1) / C::BMQ;  // query tiles holding rows of the sequence
  const int per_head = nq - qt_first;
  const int heads = group / R;  // query heads this workgroup sums over
  const int r_lo = rs * heads;
  const int iters = heads * per_head;

  Stager<T, HD, C::BMQ, C::NW> stQ, stO;
  const float* lse2 = dws + (size_t)B * H * S;  // LSE*log2e, written by the dq kernel
  // issue the copies of tile `it` (Q, dO, LSE*log2e, D) into buffer `buf`
  auto issue = [&](int it, int buf) {
    const int r = r_lo + it / per_head, qt = qt_first + it % per_head;
    const size_t bh = (size_t)b * H + (size_t)kvh * group + r;
    const int row0 = qt * C::BMQ;
    // rows past n (padding, or past S) read zero: their Q, dO, LSE and D are
    // zero, so they add exactly zero to dV (P * dO) and dK (dS * Q)
    stQ.issue(q + bh * S * HD, row0, n, sQ[buf], wave, lane, tid);
    stO.issue(dO + bh * S * HD, row0, n, sO[buf], wave, lane, tid);
    // per-row statistics: 64 rows per wave instruction
    constexpr int NST = C::BMQ / kWave;
    const v4i rl = make_rsrc(lse2 + bh * S, (uint32_t)n * 4u);
    const v4i rd = make_rsrc(dws + bh * S, (uint32_t)n * 4u);
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      if (wave == i) {
        const uint32_t voff = (uint32_t)(row0 + kWave * i + lane) * 4u;
        lds_copy4(rl, voff, &sL[buf][kWave * i]);
        lds_copy4(rd, voff, &sD[buf][kWave * i]);
      }
    }
  };
  auto commit = [&](int buf) {
    wait_global_loads();
    stQ.commit(sQ[buf], tid);
    stO.commit(sO[buf], tid);
  };
  // bf16: the first tile's copies into LDS go out before the key / value
  // loads, so the two fetches overlap (fp32 stages through registers and
  // copies after them)
  if constexpr (sizeof(T) == 2) issue(0, 0);
  typename M::frag kf[C::NKS], vf[C::NKS];
  if constexpr (sizeof(T) == 4 && HD <= 32) {
    // fp32: four operands per 16-byte load (a key past the sequence end reads
    // key n-1 and its operands are zeroed); at hd 64 the wide loads' registers
    // would cost a wave per SIMD
    const size_t krow = (size_t)(kv_ok ? my_kv : n - 1) * HD;
    row_frags_global<T, HD>(k + kvplane + krow, g, kf);
    row_frags_global<T, HD>(v + kvplane + krow, g, vf);
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      kf[ks] = kv_ok ? kf[ks] : zero_frag<T>();
      vf[ks] = kv_ok ? vf[ks] : zero_frag<T>();
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      kf[ks] = kv_ok ? row_frag_global<T, HD>(k + kvplane + (size_t)my_kv * HD, g, ks) : zero_frag<T>();
      vf[ks] = kv_ok ? row_frag_global<T, HD>(v + kvplane + (size_t)my_kv * HD, g, ks) : zero_frag<T>();
    }
  }

  // dK^T / dV^T accumulators live for the whole kernel: bf16 keeps them in AGPRs
  f32x16 dkacc[C::ND], dvacc[C::ND];
#pragma unroll
  for (int d = 0; d < C::ND; ++d) {
    dkacc[d] = zero_acc();
    dvacc[d] = zero_acc();
  }
  auto acc_mma = [](f32x16& acc, const typename M::frag& a, const typename M::frag& b) {
    if constexpr (sizeof(T) == 2 && kDkvAgpr<HD>)
      mma_agpr(acc, a, b);
    else
      M::mma(acc, a, b);
  };

  if constexpr (sizeof(T) == 4) issue(0, 0);
  commit(0);  // waits for every load above
  __syncthreads();

  for (int it = 0; it < iters; ++it) {
    const int cur = it & 1;
    const int qt = qt_first + it % per_head;
    const bool more = it + 1 < iters;
    if (more) issue(it + 1, cur ^ 1);  // the other buffer was last read before the previous barrier
    if (wave_live) {
      const T* tQ = sQ[cur];
      const T* tO = sO[cur];
      const float* tL = sL[cur];
      const float* tD = sD[cur];
      // One 32-row query block.  Blocks are 32-aligned like the wave's keys, so
      // a block is either wholly visible, the diagonal block, or wholly masked
      // (skipped); only the diagonal block and the sequence tail carry a mask.
      auto block = [&](const int qb, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int qb0 = qt * C::BMQ + 32 * qb;
        // dP accumulates onto -D of the block's rows (the workspace holds -D)
        // and comes out as dP - D
        f32x16 s = zero_acc(), dp;
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const float4 d4 = *reinterpret_cast<const float4*>(tD + 32 * qb + 8 * rg + 4 * g);
          dp[4 * rg] = d4.x;
          dp[4 * rg + 1] = d4.y;
          dp[4 * rg + 2] = d4.z;
          dp[4 * rg + 3] = d4.w;
        }
        __builtin_amdgcn_s_setprio(2);
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
          M::mma(s, row_frag_lds<T, HD, C::BMQ>(tQ, 32 * qb + li, g, ks), kf[ks]);
          M::mma(dp, row_frag_lds<T, HD, C::BMQ>(tO, 32 * qb + li, g, ks), vf[ks]);
        }
        __builtin_amdgcn_s_setprio(0);
        // bf16: transposed operands of both products read before the softmax
        // gradient, so their LDS latency overlaps it (fp32's would take 32-64
        // registers)
        typename M::frag to[C::NAS][C::ND], tq[C::NAS][C::ND];
        if constexpr (sizeof(T) == 2) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ks = 0; ks < C::NAS; ++ks)
#pragma unroll
            for (int db = 0; db < C::ND; ++db) {
              to[ks][db] = accrow_frag<T, HD, C::BMQ>(tO, 32 * qb, ks, 32 * db, lane);
              tq[ks][db] = accrow_frag<T, HD, C::BMQ>(tQ, 32 * qb, ks, 32 * db, lane);
            }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const float4 lv = *reinterpret_cast<const float4*>(tL + 32 * qb + 8 * rg + 4 * g);
          const float lr[4] = {lv.x, lv.y, lv.z, lv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * rg + e;
            float p = fast_exp2(fmaf(s[r], c, -lr[e]));
            if constexpr (MASK) {
              const int qi = qb0 + acc_row(r, g);
              p = (qi >= my_kv && qi < n) ? p : 0.f;
            }
            s[r] = p;
            dp[r] = p * dp[r];  // dS = P (dP - D)
          }
        }
        __builtin_amdgcn_s_setprio(2);
#pragma unroll
        for (int ks = 0; ks < C::NAS; ++ks) {
          const typename M::frag pf = acc_frag<T>(s, ks * M::KPL);
          const typename M::frag sf = acc_frag<T>(dp, ks * M::KPL);
#pragma unroll
          for (int db = 0; db < C::ND; ++db) {
            if constexpr (sizeof(T) == 2) {
              acc_mma(dvacc[db], to[ks][db], pf);
              acc_mma(dkacc[db], tq[ks][db], sf);
            } else {
              acc_mma(dvacc[db], accrow_frag<T, HD, C::BMQ>(tO, 32 * qb, ks, 32 * db, lane), pf);
              acc_mma(dkacc[db], accrow_frag<T, HD, C::BMQ>(tQ, 32 * qb, ks, 32 * db, lane), sf);
            }
          }
        }
        __builtin_amdgcn_s_setprio(0);
      };

      const int qt0 = qt * C::BMQ;
      if (qt0 >= kv0 + 32 && qt0 + C::BMQ <= n) {
        // Every block of the tile is below the diagonal and inside the
        // sequence.  Phases are pinned with scheduling barriers so that each
        // LDS operand is read a whole phase before the instruction that needs
        // it (the loads would otherwise sit right in front of their MFMAs):
        //   [S, dP MFMAs of block qb] [transpose operands and row statistics
        //   of qb] [softmax-gradient VALU of qb] [dV, dK MFMAs of qb; row
        //   operands of qb+1]
        if constexpr (sizeof(T) == 2) {
          typename M::frag aq[C::NKS], ao[C::NKS];
#pragma unroll
          for (int ks = 0; ks < C::NKS; ++ks) {
            aq[ks] = row_frag_lds<T, HD, C::BMQ>(tQ, li, g, ks);
            ao[ks] = row_frag_lds<T, HD, C::BMQ>(tO, li, g, ks);
          }
          // -D of the block's rows in accumulator order: dP accumulates onto
          // it and comes out as dP - D
          auto neg_d = [&](int qb) {
            f32x16 d;
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
              const float4 v4 = *reinterpret_cast<const float4*>(tD + 32 * qb + 8 * rg + 4 * g);
              d[4 * rg] = v4.x;
              d[4 * rg + 1] = v4.y;
              d[4 * rg + 2] = v4.z;
              d[4 * rg + 3] = v4.w;
            }
            return d;
          };
          f32x16 dnext = neg_d(0);
#pragma unroll
          for (int qb = 0; qb < C::NQB; ++qb) {
            f32x16 s = zero_acc(), dp = dnext;
            // raised priority while issuing matrix products, so that they queue
            // on the matrix core while the other wave of the SIMD runs VALU
            // work (measured: the kernel 3-4% faster)
            __builtin_amdgcn_s_setprio(2);
#pragma unroll
            for (int ks = 0; ks < C::NKS; ++ks) {
              M::mma(s, aq[ks], kf[ks]);
              M::mma(dp, ao[ks], vf[ks]);
            }
            __builtin_amdgcn_s_setprio(0);
            __builtin_amdgcn_sched_barrier(0);
            typename M::frag to[C::NAS][C::ND], tq[C::NAS][C::ND];
#pragma unroll
            for (int ks = 0; ks < C::NAS; ++ks)
#pragma unroll
              for (int db = 0; db < C::ND; ++db) {
                to[ks][db] = accrow_frag<T, HD, C::BMQ>(tO, 32 * qb, ks, 32 * db, lane);
                tq[ks][db] = accrow_frag<T, HD, C::BMQ>(tQ, 32 * qb, ks, 32 * db, lane);
              }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
              const float4 lv = *reinterpret_cast<const float4*>(tL + 32 * qb + 8 * rg + 4 * g);
              const float lr[4] = {lv.x, lv.y, lv.z, lv.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = 4 * rg + e;
                const float p = fast_exp2(fmaf(s[r], c, -lr[e]));
                s[r] = p;
                dp[r] = p * dp[r];  // dS = P (dP - D)
              }
            }
            typename M::frag pf[C::NAS], sf[C::NAS];
#pragma unroll
            for (int ks = 0; ks < C::NAS; ++ks) {
              pf[ks] = acc_frag<T>(s, ks * M::KPL);
              sf[ks] = acc_frag<T>(dp, ks * M::KPL);
            }
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(2);
#pragma unroll
            for (int ks = 0; ks < C::NAS; ++ks)
#pragma unroll
              for (int db = 0; db < C::ND; ++db) {
                acc_mma(dvacc[db], to[ks][db], pf[ks]);
                acc_mma(dkacc[db], tq[ks][db], sf[ks]);
              }
            __builtin_amdgcn_s_setprio(0);
            if (qb + 1 < C::NQB) {
#pragma unroll
              for (int ks = 0; ks < C::NKS; ++ks) {
                aq[ks] = row_frag_lds<T, HD, C::BMQ>(tQ, 32 * (qb + 1) + li, g, ks);
                ao[ks] = row_frag_lds<T, HD, C::BMQ>(tO, 32 * (qb + 1) + li, g, ks);
              }
              dnext = neg_d(qb + 1);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
#pragma unroll
          for (int qb = 0; qb < C::NQB; ++qb)
            if (qb % C::QS == qh) block(qb, std::false_type{});
        }
      } else {
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) {
          if (qb % C::QS != qh) continue;  // the other query half's block
          const int qb0 = qt0 + 32 * qb;
          if (qb0 + 31 < kv0 || qb0 >= n) continue;  // wholly above the diagonal, or past n
          if (qb0 < kv0 + 32 || qb0 + 32 > n)
            block(qb, std::true_type{});
          else
            block(qb, std::false_type{});
        }
      }
    }
    if (more) commit(cur ^ 1);
    __syncthreads();
  }

  if constexpr (sizeof(T) == 2 && kDkvAgpr<HD>) mma_agpr_drain();
  if constexpr (C::QS == 2) {
    // the second query half of each key block hands its sums to the first
    // through the Q and dO buffers (every read of them ended at the last
    // barrier); added in that fixed order
    static_assert(2 * C::ND * 16 * kWave <= 2 * C::TILE, "partial sums exceed the tile buffers");
    float* red_k = reinterpret_cast<float*>(&sQ[0][0]);
    float* red_v = reinterpret_cast<float*>(&sO[0][0]);
    if (qh == 1) {
#pragma unroll
      for (int db = 0; db < C::ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          red_k[((kb_w * C::ND + db) * 16 + r) * kWave + lane] = dkacc[db][r];
          red_v[((kb_w * C::ND + db) * 16 + r) * kWave + lane] = dvacc[db][r];
        }
    }
    __syncthreads();
    if (qh == 1) return;
#pragma unroll
    for (int db = 0; db < C::ND; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dkacc[db][r] += red_k[((kb_w * C::ND + db) * 16 + r) * kWave + lane];
        dvacc[db][r] += red_v[((kb_w * C::ND + db) * 16 + r) * kWave + lane];
      }
  }
  if (!kv_ok) {  // padding keys inside the sequence's last tile
    if (g == 0 && my_kv < S) {
      zero_row<HD>(outk + kvplane + (size_t)my_kv * HD);
      zero_row<HD>(outv + kvplane + (size_t)my_kv * HD);
    }
    return;
  }
  float* krow = outk + kvplane + (size_t)my_kv * HD;
  float* vrow = outv + kvplane + (size_t)my_kv * HD;
#pragma unroll
  for (int db = 0; db < C::ND; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = 32 * db + 8 * rg + 4 * g;
      if (d0 < HD) {
        store4<float>(krow + d0, scale * dkacc[db][4 * rg], scale * dkacc[db][4 * rg + 1],
                      scale * dkacc[db][4 * rg + 2], scale * dkacc[db][4 * rg + 3]);
        store4<float>(vrow + d0, dvacc[db][4 * rg], dvacc[db][4 * rg + 1], dvacc[db][4 * rg + 2],
                      dvacc[db][4 * rg + 3]);
      }
    }
}

// dk = sum over r of part_k[r], dv = sum over r of part_v[r], r ascending
// (the group sum of a split group), four floats per thread.
__global__ __launch_bounds__(kThreads) void dkdv_group_sum_kernel(const float* __restrict__ part,
                                                             float* __restrict__ dk,
                                                             float* __restrict__ dv, long n4,
                                                             int R) {
  const long i = (long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= 2 * n4) return;
  const bool is_v = i >= n4;
  const long e = is_v ? i - n4 : i;
  const float4* src = reinterpret_cast<const float4*>(part) + (is_v ? (long)R * n4 : 0) + e;
  float4 a = src[0];
  for (int r = 1; r < R; ++r) {
    const float4 b = src[(long)r * n4];
    a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
  }
  reinterpret_cast<float4*>(is_v ? dv : dk)[e] = a;
}

template <typename T, int HD>
static void dkdv_typed(const Dims& d, const void* q, const void* k, const void* v,
                       const float* lse, const void* dO, float* dws, float* dk, float* dv,
                       const int* lens, float scale, bool split_groups, hipStream_t stream) {
  using C = DkvCfg<T, HD>;
  static_assert(C::BN == dkdv_tile_keys(sizeof(T) == 4 ? 0 : 1, HD) && C::NT == kThreads,
                "tiling differs from the plan");
  const AttnPlan p = attn_plan(d, sizeof(T) == 4 ? 0 : 1, split_groups);
  const int nkt = (d.S + C::BN - 1) / C::BN;
  const int BG = d.B * d.Hkv;
  const int R = p.split;
  // the partials follow the per-row statistics in the workspace
  float* part = R > 1 ? dws + dkdv_part_offset(d) : nullptr;
  dim3 grid((unsigned)p.dkdv_blocks), block(C::NT);
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, HD>), grid, block, 0, stream, (const T*)q,
                     (const T*)k, (const T*)v, lse, (const T*)dO, dws, dk, dv, part, lens, d.B,
                     d.S, d.H, d.Hkv, nkt, BG, R, device_cu_count(), scale * kLog2e, scale);
  if (R > 1) {
    const long n4 = (long)d.B * d.Hkv * d.S * HD / 4;
    hipLaunchKernelGGL(dkdv_group_sum_kernel, dim3((unsigned)p.dkdv_sum_blocks), dim3(kThreads),
                       0, stream, (const float*)part, dk, dv, n4, R);
  }
}

void launch_bwd_dkdv(int dtype, const Dims& d, const void* q, const void* k, const void* v,
                     const float* lse, const void* dO, float* dws, float* dk, float* dv,
                     const int* lens, float scale, bool split_groups, hipStream_t stream) {
  if (dtype == 0) {
    if (d.hd == 16) dkdv_typed<float, 16>(d, q, k, v, lse, dO, dws, dk, dv, lens, scale, split_groups, stream);
    else if (d.hd == 32) dkdv_typed<float, 32>(d, q, k, v, lse, dO, dws, dk, dv, lens, scale, split_groups, stream);
    else dkdv_typed<float, 64>(d, q, k, v, lse, dO, dws, dk, dv, lens, scale, split_groups, stream);
  } else {
    if (d.hd == 16) dkdv_typed<bf16, 16>(d, q, k, v, lse, dO, dws, dk, dv, lens, scale, split_groups, stream);
    else if (d.hd == 32) dkdv_typed<bf16, 32>(d, q, k, v, lse, dO, dws, dk, dv, lens, scale, split_groups, stream);
    else dkdv_typed<bf16, 64>(d, q, k, v, lse, dO, dws, dk, dv, lens, scale, split_groups, stream);
  }
}

}  // namespace xattn
