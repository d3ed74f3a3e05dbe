// attn_bwd_short.hip -- causal attention backward in one kernel for short bf16
// sequences (S <= 256, hd <= 32, one query head per kv head), for gfx950.
//
// One workgroup (4 waves) per (batch, head) copies the head's whole Q, K, V and
// dO planes (at most 256 rows each) into LDS, then
//   phase 0: D_i = sum_d dO_id * o_id and LSE_i * log2e per row into LDS
//            (the simplification of the softmax Jacobian in the fused kernel of
//            the "xtrain evolution overview", infra table row T14);
//   phase 1: the key side, per 32-key block j and 32-row query block i >= j
//            (ascending):
//              S = Q_i . K_j^T,  P = exp2(S*scale*log2e - LSE_i*log2e)
//              dS = P * (dO_i . V_j^T - D_i)
//              dV_j^T += dO_i^T . P,   dK_j^T += Q_i^T . dS
//            (a lane owns one key), then dk = scale * dK and dv are written;
//   phase 2: the query side, per query block i and key block j <= i
//            (ascending):
//              S^T = K_j . Q_i^T, dS^T = P^T * (V_j . dO_i^T - D_i)
//              dQ_i^T += K_j^T . dS^T
//            (a lane owns one query row), then dq = scale * dQ is written.
// Each product, the operand rounding and the order of every sum are those of
// the dq and dk/dv kernels, so the results are bitwise those of the two-kernel
// backward.  What changes is the traffic and the launch count: q, k, v, dO and
// o are read from HBM once, nothing goes through the workspace, and one launch
// replaces two.  Rows and keys past the sequence length read as zero and their
// gradients are written as zeros.
//
// Work split: with nb = ceil(n/32) blocks, wave w takes key blocks w and
// nb-1-w in phase 1 (nb - j query blocks each) and query blocks w and nb-1-w in
// phase 2 (i + 1 key blocks each), so every wave carries nb + 1 block steps in
// each phase.
#include <type_traits>

#include "attn_device.hpp"
#include "launch.hpp"

namespace xattn {

template <int HD>
struct ShortCfg {
  static constexpr int NW = 4, NT = NW * kWave, ROWS = kShortMaxS, NBLK = ROWS / 32;
  static constexpr int ND = HD >= 32 ? HD / 32 : 1;
  static constexpr int NKS = HD / Mma<bf16>::KSTEP;
  static constexpr int NAS = 32 / Mma<bf16>::KSTEP;
  static constexpr int TILE = Tile<bf16, HD, ROWS>::ELEMS;
  static_assert(NBLK <= 2 * NW, "a wave takes at most two blocks per phase");
};

template <int HD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_bwd_short_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ o, const float* __restrict__ lse, const bf16* __restrict__ dO,
    float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv,
    const int* __restrict__ lens, int S, int H, int nfull, float c, float scale) {
  using C = ShortCfg<HD>;
  using M = Mma<bf16>;
  using TL = Tile<bf16, HD, C::ROWS>;
  using frag = M::frag;
  __shared__ __align__(16) bf16 sK[C::TILE];
  __shared__ __align__(16) bf16 sV[C::TILE];
  __shared__ __align__(16) bf16 sQ[C::TILE];
  __shared__ __align__(16) bf16 sO[C::TILE];     // dO
  __shared__ __align__(16) float sL[C::ROWS];    // LSE * log2e
  __shared__ __align__(16) float sD[C::ROWS];    // -D

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int li = lane & 31, g = lane >> 5;
  // workgroups below nfull take a whole head; the rest come in pairs that
  // split one head: the first takes its key side (phase 1), the second its
  // query side (phase 2), each computing the per-row values itself
  int bh = blockIdx.x, role = 0;  // 0: both sides, 1: key side, 2: query side
  if (bh >= nfull) {
    const int x = bh - nfull;
    bh = nfull + x / 2;
    role = 1 + x % 2;
  }
  const int b = bh / H;
  const size_t plane = (size_t)bh * S * HD;
  const int n = seq_len(lens, b, S);  // rows and keys past n are padding
  const int nb = (n + 31) / 32;

  // rows past the last block (whole blocks of padding) are written as zeros
  // here; padding rows inside the last block are handled by their lanes
  {
    constexpr int CPR = HD / 4;
    const int r0 = 32 * nb;
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int item = tid; item < (S - r0) * CPR; item += C::NT) {
      const size_t off = plane + (size_t)(r0 + item / CPR) * HD + 4 * (item % CPR);
      if (role != 1) *reinterpret_cast<float4*>(dq + off) = z;
      if (role != 2) {
        *reinterpret_cast<float4*>(dk + off) = z;
        *reinterpret_cast<float4*>(dv + off) = z;
      }
    }
  }
  if (nb == 0) return;

  // the wave's two blocks (either may be absent: -1; blkA < 0 implies blkB < 0)
  const int blkA = wave <= nb - 1 - wave ? wave : -1;
  const int blkB = nb - 1 - wave > wave ? nb - 1 - wave : -1;

  // rows past n read zero
  TL::template issue<C::NW>(k + plane, 0, n, sK, wave, lane);
  TL::template issue<C::NW>(v + plane, 0, n, sV, wave, lane);
  TL::template issue<C::NW>(q + plane, 0, n, sQ, wave, lane);
  TL::template issue<C::NW>(dO + plane, 0, n, sO, wave, lane);

  // phase 0: the per-row values of the wave's query blocks, computed as the dq
  // kernel computes them (a lane pair per row, halves over the head dimension;
  // a row past the sequence end reads row n-1 and counts zero)
  frag of[2][C::NKS];
  float lse_row[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int blk = a == 0 ? blkA : blkB;
    if (blk < 0) continue;
    const int my_q = 32 * blk + li;
    const int lrow = my_q < n ? my_q : n - 1;
    row_frags_global<bf16, HD>(o + plane + (size_t)lrow * HD, g, of[a]);
    lse_row[a] = lse[(size_t)bh * S + lrow];
  }
  wait_global_loads();
  __syncthreads();  // K, V, Q, dO in LDS
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int blk = a == 0 ? blkA : blkB;
    if (blk < 0) continue;
    const int my_q = 32 * blk + li;
    const bool q_ok = my_q < n;
    float Dp = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      const frag df = row_frag_lds<bf16, HD, C::ROWS>(sO, my_q, g, ks);
#pragma unroll
      for (int t = 0; t < 8; ++t) Dp += (float)of[a][ks][t] * (float)df[t];
    }
    if (!q_ok) Dp = 0.f;
    const float Drow = halves_sum(Dp);
    if (g == 0) {
      sD[my_q] = -Drow;
      sL[my_q] = q_ok ? lse_row[a] * kLog2e : 0.f;
    }
  }
  __syncthreads();  // D and LSE of every row

  // phase 1: key blocks blkA, blkB, each against the query blocks at or below it
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int blk = a == 0 ? blkA : blkB;
    if (blk < 0 || role == 2) continue;
    const int my_kv = 32 * blk + li;
    frag kf[C::NKS], vf[C::NKS];
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {  // keys past n read zero
      kf[ks] = row_frag_lds<bf16, HD, C::ROWS>(sK, my_kv, g, ks);
      vf[ks] = row_frag_lds<bf16, HD, C::ROWS>(sV, my_kv, g, ks);
    }
    f32x16 dkacc[C::ND], dvacc[C::ND];
#pragma unroll
    for (int d = 0; d < C::ND; ++d) {
      dkacc[d] = zero_acc();
      dvacc[d] = zero_acc();
    }
    // one 32-row query block i
    auto step = [&](const int i, auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      f32x16 s = zero_acc(), dp;  // dP accumulates onto -D
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const float4 d4 = *reinterpret_cast<const float4*>(sD + 32 * i + 8 * rg + 4 * g);
        dp[4 * rg] = d4.x;
        dp[4 * rg + 1] = d4.y;
        dp[4 * rg + 2] = d4.z;
        dp[4 * rg + 3] = d4.w;
      }
      __builtin_amdgcn_s_setprio(2);
#pragma unroll
      for (int ks = 0; ks < C::NKS; ++ks) {
        M::mma(s, row_frag_lds<bf16, HD, C::ROWS>(sQ, 32 * i + li, g, ks), kf[ks]);
        M::mma(dp, row_frag_lds<bf16, HD, C::ROWS>(sO, 32 * i + li, g, ks), vf[ks]);
      }
      __builtin_amdgcn_s_setprio(0);
      // transposed operands read before the softmax gradient, so their LDS
      // latency overlaps it
      frag to[C::NAS][C::ND], tq[C::NAS][C::ND];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < C::NAS; ++ks)
#pragma unroll
        for (int db = 0; db < C::ND; ++db) {
          to[ks][db] = accrow_frag<bf16, HD, C::ROWS>(sO, 32 * i, ks, 32 * db, lane);
          tq[ks][db] = accrow_frag<bf16, HD, C::ROWS>(sQ, 32 * i, ks, 32 * db, lane);
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const float4 lv = *reinterpret_cast<const float4*>(sL + 32 * i + 8 * rg + 4 * g);
        const float lr[4] = {lv.x, lv.y, lv.z, lv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rr = 4 * rg + e;
          float p = fast_exp2(fmaf(s[rr], c, -lr[e]));
          if constexpr (MASK) {
            const int qi = 32 * i + acc_row(rr, g);
            p = (qi >= my_kv && qi < n) ? p : 0.f;
          }
          s[rr] = p;
          dp[rr] = p * dp[rr];  // dS = P (dP - D)
        }
      }
      __builtin_amdgcn_s_setprio(2);
#pragma unroll
      for (int ks = 0; ks < C::NAS; ++ks) {
        const frag pf = acc_frag<bf16>(s, ks * M::KPL);
        const frag sf = acc_frag<bf16>(dp, ks * M::KPL);
#pragma unroll
        for (int db = 0; db < C::ND; ++db) {
          M::mma(dvacc[db], to[ks][db], pf);
          M::mma(dkacc[db], tq[ks][db], sf);
        }
      }
      __builtin_amdgcn_s_setprio(0);
    };
    step(blk, std::true_type{});  // the diagonal block
    for (int i = blk + 1; i < nb; ++i) {
      if (32 * i + 32 > n)
        step(i, std::true_type{});  // the sequence tail
      else
        step(i, std::false_type{});
    }
    // dk = scale * dK and dv of the block's keys
    if (my_kv >= n) {  // padding keys inside the sequence's last block
      if (g == 0 && my_kv < S) {
        zero_row<HD>(dk + plane + (size_t)my_kv * HD);
        zero_row<HD>(dv + plane + (size_t)my_kv * HD);
      }
    } else {
      float* krow = dk + plane + (size_t)my_kv * HD;
      float* vrow = dv + plane + (size_t)my_kv * HD;
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
  }

  // phase 2: query blocks blkA, blkB, each against the key blocks at or below it
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int blk = a == 0 ? blkA : blkB;
    if (blk < 0 || role == 1) continue;
    const int my_q = 32 * blk + li;
    const bool q_ok = my_q < n;
    frag qf[C::NKS], df[C::NKS];
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {  // rows past n read zero
      qf[ks] = row_frag_lds<bf16, HD, C::ROWS>(sQ, my_q, g, ks);
      df[ks] = row_frag_lds<bf16, HD, C::ROWS>(sO, my_q, g, ks);
    }
    const float lse2 = sL[my_q];
    const float nd = sD[my_q];
    f32x16 acc[C::ND];
#pragma unroll
    for (int d = 0; d < C::ND; ++d) acc[d] = zero_acc();
    // one 32-key block j
    auto step = [&](const int j, auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      const int kb0 = 32 * j;
      f32x16 s = zero_acc(), dp;  // dP^T accumulates onto -D
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) dp[rr] = nd;
      __builtin_amdgcn_s_setprio(2);
#pragma unroll
      for (int ks = 0; ks < C::NKS; ++ks) {
        M::mma(s, row_frag_lds<bf16, HD, C::ROWS>(sK, kb0 + li, g, ks), qf[ks]);
        M::mma(dp, row_frag_lds<bf16, HD, C::ROWS>(sV, kb0 + li, g, ks), df[ks]);
      }
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        float p = fast_exp2(fmaf(s[rr], c, -lse2));
        if constexpr (MASK) {
          const int kv = kb0 + acc_row(rr, g);
          p = (kv <= my_q && kv < n) ? p : 0.f;
        }
        s[rr] = p * dp[rr];  // dS^T = P (dP - D)
      }
      __builtin_amdgcn_s_setprio(2);
#pragma unroll
      for (int ks = 0; ks < C::NAS; ++ks) {
        const frag sf = acc_frag<bf16>(s, ks * M::KPL);
#pragma unroll
        for (int db = 0; db < C::ND; ++db)
          M::mma(acc[db], accrow_frag<bf16, HD, C::ROWS>(sK, kb0, ks, 32 * db, lane), sf);
      }
      __builtin_amdgcn_s_setprio(0);
    };
    // key blocks below the diagonal lie wholly inside the sequence
    for (int j = 0; j < blk; ++j) step(j, std::false_type{});
    step(blk, std::true_type{});  // the diagonal block
    if (!q_ok) {  // padding rows inside the sequence's last block
      if (g == 0 && my_q < S) zero_row<HD>(dq + plane + (size_t)my_q * HD);
      continue;
    }
    float* qrow = dq + plane + (size_t)my_q * HD;
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
}

template <int HD>
static void short_typed(const Dims& d, const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dO, float* dq, float* dk, float* dv,
                        const int* lens, float scale, hipStream_t stream) {
  using C = ShortCfg<HD>;
  static_assert(C::NT <= kThreads, "workgroup size differs from the plan");
  const ShortSplit sp = short_split(d, device_cu_count());
  dim3 grid((unsigned)sp.blocks), block(C::NT);
  hipLaunchKernelGGL((attn_bwd_short_kernel<HD>), grid, block, 0, stream, (const bf16*)q,
                     (const bf16*)k, (const bf16*)v, (const bf16*)o, lse, (const bf16*)dO, dq, dk,
                     dv, lens, d.S, d.H, (int)sp.full, scale * kLog2e, scale);
}

void launch_bwd_short(const Dims& d, const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dO, float* dq, float* dk, float* dv,
                      const int* lens, float scale, hipStream_t stream) {
  if (d.hd == 16) short_typed<16>(d, q, k, v, o, lse, dO, dq, dk, dv, lens, scale, stream);
  else short_typed<32>(d, q, k, v, o, lse, dO, dq, dk, dv, lens, scale, stream);
}

}  // namespace xattn
