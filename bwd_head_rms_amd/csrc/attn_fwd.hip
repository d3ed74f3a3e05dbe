// attn_fwd.hip -- fused causal attention forward for gfx950.
//
// One workgroup (4 waves) per (batch, head, query tile): fp32 at hd <= 32
// (attn_fwd_kernel) runs 64-row tiles, two waves per 32 rows, each taking one
// 32-key block of every key tile and merged at the end; otherwise 128 rows, a
// wave per 32 (bf16: attn_fwd_pipe_kernel, below).  Key/value tiles of 64 rows are copied into a double-buffered
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
#include <atomic>
#include <type_traits>

#include "attn_device.hpp"
#include "launch.hpp"

namespace xattn {

// Bound on a row's per-tile sum of weights exp2(S*c - m) before its reference
// max m is renewed: weights stay below 2^64 (bf16 and fp32 reach 2^127), and the
// row sum l below 2^64 * S, so no precision or range is lost.
constexpr float kRescaleBound = 18446744073709551616.f;  // 2^64

// A padding row of the output: o = 0, lse = -inf (nothing to attend to).
template <typename T, int HD>
__device__ __forceinline__ void store_padding_row(T* o, float* lse, int bh, int S, int row) {
  T* orow = o + ((size_t)bh * S + row) * HD;
#pragma unroll
  for (int d = 0; d < HD; d += 4) store4<T>(orow + d, 0.f, 0.f, 0.f, 0.f);
  lse[(size_t)bh * S + row] = -INFINITY;
}

// Rows [row0, row0 + rows) of (b, h) that lie inside the tensor, all padding.
template <typename T, int HD>
__device__ __forceinline__ void store_padding_rows(T* o, float* lse, int bh, int S, int row0,
                                                   int rows, int tid, int nt) {
  for (int r = tid; r < rows; r += nt)
    if (row0 + r < S) store_padding_row<T, HD>(o, lse, bh, S, row0 + r);
}

template <typename T, int HD>
struct FwdCfg {
  // hd <= 32: two row blocks of 32 queries, each split over two waves by key:
  // wave (r, c) takes 32-key block c of every 64-key tile for rows r, keeping
  // its own softmax state, and the two states of a row block are merged at
  // the end.  A causal row block's serial chain of blocks is halved (at
  // S = 256 the last rows' 8 blocks of 64-cycle fp32 products become 4 per
  // wave).  At hd 64 the merge's registers would cost a wave per SIMD, so
  // there each of four waves owns its 32 rows and every key.
  static constexpr int KC = HD <= 32 ? 2 : 1, NR = 4 / KC;
  static constexpr int NW = NR * KC, NT = NW * kWave, BM = 32 * NR, BN = 64, NB = BN / 32;
  static constexpr int ND = HD >= 32 ? HD / 32 : 1;
  static constexpr int NKS = HD / Mma<T>::KSTEP;  // head-dim contraction steps
  static constexpr int NAS = 32 / Mma<T>::KSTEP;  // key contraction steps per 32-key block
  static constexpr int TILE = Tile<T, HD, BN>::ELEMS;
};

template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_fwd_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    T* __restrict__ o, float* __restrict__ lse, const int* __restrict__ lens, int S, int H,
    int Hkv, int nqt, int BH, float c) {
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
  const int n = seq_len(lens, b, S);  // rows and keys past n are padding
  if (qt * C::BM >= n) {              // a tile of padding only
    store_padding_rows<T, HD>(o, lse, bh, S, qt * C::BM, C::BM, tid, C::NT);
    return;
  }

  // row block, and key block of each tile
  const int rw = C::KC == 1 ? wave : wave % C::NR, kc = C::KC == 1 ? 0 : wave / C::NR;
  const int q0 = qt * C::BM + rw * 32;
  const int my_q = q0 + li;
  const bool q_ok = my_q < n;
  const bool wave_live = q0 < n;
  const int wave_kv_end = min(n, q0 + 32);  // keys visible to some row of this wave
  // padding rows of this tile are written first, while nothing is live
  if (!q_ok && g == 0 && kc == 0 && my_q < S) store_padding_row<T, HD>(o, lse, bh, S, my_q);

  // the query operands by wide loads; a row past the sequence end reads row
  // n-1 and its operands are zeroed
  typename M::frag qf[C::NKS];
  row_frags_global<T, HD>(qp + (size_t)(q_ok ? my_q : n - 1) * HD, g, qf);
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) qf[ks] = q_ok ? qf[ks] : zero_frag<T>();

  f32x16 oacc[C::ND];
#pragma unroll
  for (int d = 0; d < C::ND; ++d) oacc[d] = zero_acc();
  float m = -INFINITY, l = 0.f;

  const int kv_end = min(n, qt * C::BM + C::BM);
  const int ntiles = (kv_end + C::BN - 1) / C::BN;

  wait_global_loads();  // the query operand above is in registers
  Stager<T, HD, C::BN, C::NW> stK, stV;
  stK.issue(kp, 0, n, sK[0], wave, lane, tid);
  stV.issue(vp, 0, n, sV[0], wave, lane, tid);
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
      // Scores of the (up to) two 32-key blocks of this tile.  Key blocks are
      // 32-aligned like the wave's rows: a visited block is wholly visible or
      // the diagonal block, and only the diagonal block and the sequence tail
      // carry a mask (masked scores become -inf, i.e. weight exactly 0).
      bool act[C::NB];
#pragma unroll
      for (int cb = 0; cb < C::NB; ++cb) act[cb] = cb % C::KC == kc && kv_t0 + 32 * cb < wave_kv_end;
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
            if (kb0 + 31 > q0 || kb0 + 32 > n) {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int kv = kb0 + acc_row(r, g);
                s[cb][r] = (kv <= my_q && kv < n) ? s[cb][r] : -INFINITY;
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
      // Each row keeps a reference max m and uses it as long as its weights
      // stay below 2^kRescaleSlack (their sum bounds every weight).  Only when
      // that fails -- the row's first tile (m = -inf), or scores that really
      // outgrew m -- are the scores recomputed, the row max taken and the
      // accumulator rescaled.  The decision is per row (rows that pass keep m
      // and recompute the same weights), so every row's result depends only
      // on that row's scores.  Every row fails on the first tile (m = -inf),
      // so there m is the tile's row max directly, with nothing to rescale; a
      // wave whose block of that tile lies wholly above its rows sees none of
      // the row's keys at all and keeps m = -inf, l = 0, O = 0.
      if (j == 0) {
        float mx = -INFINITY;
#pragma unroll
        for (int cb = 0; cb < C::NB; ++cb)
          if (act[cb]) {
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[cb][r]);
          }
        m = halves_max(mx) * c;
        probs();
      } else {
        probs();
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

  // merge the two key halves of each row block (every read of the K and V
  // buffers ended at the last barrier): wave (r, 1) hands m, l and O to wave
  // (r, 0), which rescales both to the larger m.  A half that saw no key of a
  // row has m = -inf and weight exp2(-inf) = 0.
  if constexpr (C::KC == 2) {
    static_assert(C::NR * C::ND * 16 * kWave <= 2 * C::TILE && C::NR * 2 * kWave <= 2 * C::TILE,
                  "partial softmax states exceed the K and V buffers");
    float* red_o = reinterpret_cast<float*>(&sK[0][0]);
    float* red_ml = reinterpret_cast<float*>(&sV[0][0]);
    if (kc == 1) {
#pragma unroll
      for (int db = 0; db < C::ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) red_o[((rw * C::ND + db) * 16 + r) * kWave + lane] = oacc[db][r];
      red_ml[(rw * 2) * kWave + lane] = m;
      red_ml[(rw * 2 + 1) * kWave + lane] = l;
    }
    __syncthreads();
    if (kc == 1) return;
    const float m1 = red_ml[(rw * 2) * kWave + lane], l1 = red_ml[(rw * 2 + 1) * kWave + lane];
    const float mm = fmaxf(m, m1);
    const float a0 = fast_exp2(m - mm), a1 = fast_exp2(m1 - mm);
    l = l * a0 + l1 * a1;
    m = mm;
#pragma unroll
    for (int db = 0; db < C::ND; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        oacc[db][r] = oacc[db][r] * a0 + red_o[((rw * C::ND + db) * 16 + r) * kWave + lane] * a1;
  }

  if (!wave_live) return;  // a wave of padding rows (stored at the start)
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

// ---------------------------------------------------------------------------
// bf16: software-pipelined forward.  Same work split (4 waves x 32 query rows
// per workgroup), but each wave walks its key range in 32-key blocks and, in
// sub-step i, overlaps three stages of consecutive blocks:
//   A(i+1): S^T_{i+1} = K_{i+1} . Q^T            (matrix cores)
//   B(i)  : P_i = exp2(S_i*c - m), row sums      (vector ALU)
//   C(i-1): O^T += V_{i-1}^T . P_{i-1}^T         (matrix cores)
// so the matrix cores work while the softmax of the previous block runs,
// instead of one wave stalling on the chain S -> softmax -> P.V of a single
// block.  K and V blocks are copied straight from HBM into rings of four
// 32-row LDS slots; one step (one barrier) covers two sub-steps, i.e. 64 keys,
// and copies the four blocks the next step reads.  The loop is unrolled over
// the ring so every slot address is a constant.
//
// Softmax reference: step 0 (the first block) uses the exact online update
// (m starts at -inf).  Later sub-steps keep m and only check that each row's
// weights exp2(S*c - m) stay below 2^63 per half block (no overflow or loss of
// precision in bf16/fp32).  A row that ever fails that check is recomputed at
// the end by an exact, unpipelined pass over HBM (scores that rise by more
// than ~44 natural-log units past the first block's max; never seen with
// normalised inputs).  Every row's result depends only on its own scores.
template <int HD>
struct FwdPipe {
  static constexpr int NW = 4, NT = NW * kWave, BM = 32 * NW;
  static constexpr int NKS = HD / 16;                // S contraction steps
  static constexpr int ND = HD >= 32 ? HD / 32 : 1;  // output column blocks
  static constexpr int NAS = 2;                      // key steps per block
  static constexpr int NC = NAS * ND;                // P.V products per block
  static constexpr int NSL = 4;                      // ring slots (K and V)
  using TL = Tile<bf16, HD, 32>;
  static constexpr int TE = TL::ELEMS;
  static constexpr int CPR = TL::CPR, RPI = TL::ROWS_PER_INST, NINST = TL::NINST;
  static_assert(NINST <= NW, "one copy per wave and block");
};

constexpr float kHalfBlockBound = 9223372036854775808.f;  // 2^63

// Issue priority from the sub-steps a workgroup still has (rem): the SIMD
// serves higher-priority waves first, so of the causal tiles that share a
// compute unit the ones with the most blocks ahead go first and the tiles end
// closer together (measured: the forward 1% faster on the causal 2048-row
// and GQA 1024-row workloads; 4 sub-steps per level was the best of 1-16).
__device__ __forceinline__ void prio_by_remaining(int rem) {
  if (rem > 12)
    __builtin_amdgcn_s_setprio(3);
  else if (rem > 8)
    __builtin_amdgcn_s_setprio(2);
  else if (rem > 4)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

// Four workgroups per CU (128 VGPRs): every workgroup of the long-context
// workload is resident from the start.
template <int HD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void attn_fwd_pipe_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    bf16* __restrict__ o, float* __restrict__ lse, const int* __restrict__ lens, int S, int H,
    int Hkv, int nqt, int BH, int ncu, float c) {
  using P = FwdPipe<HD>;
  using M = Mma<bf16>;
  using frag = M::frag;
  __shared__ __align__(16) bf16 sK[P::NSL][P::TE];
  __shared__ __align__(16) bf16 sV[P::NSL][P::TE];

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int li = lane & 31, g = lane >> 5;
  // heaviest tiles first, balanced over the four workgroups a CU holds at once
  const int bid = balanced_rank(blockIdx.x, gridDim.x, ncu, 4);
  const int qt = nqt - 1 - bid / BH;
  const int bh = bid % BH;
  const int b = bh / H, h = bh % H;
  const int kvh = h / (H / Hkv);
  const bf16* qp = q + (size_t)bh * S * HD;
  const size_t kvoff = ((size_t)b * Hkv + kvh) * S * HD;
  const int n = seq_len(lens, b, S);  // rows and keys past n are padding
  if (qt * P::BM >= n) {              // a tile of padding only
    store_padding_rows<bf16, HD>(o, lse, bh, S, qt * P::BM, P::BM, tid, P::NT);
    return;
  }

  const int q0 = qt * P::BM + wave * 32;
  const int my_q = q0 + li;
  const bool q_ok = my_q < n;
  // Blocks of the workgroup and of this wave; a wave's last block is its
  // diagonal block, which also holds the end of the sequence when n is not a
  // multiple of 32.  A wave wholly past the end (last tile of a sequence) runs
  // over all blocks like a live one and stores padding rows.
  const int nbw = (min(n, qt * P::BM + P::BM) + 31) / 32;
  const int nb = (min(n, q0 + 32) + 31) / 32;
  // padding rows of this tile are written first, while nothing is live
  if (!q_ok && g == 0 && my_q < S) store_padding_row<bf16, HD>(o, lse, bh, S, my_q);

  f32x16 oacc[P::ND];
#pragma unroll
  for (int d = 0; d < P::ND; ++d) oacc[d] = zero_acc();
  float m = -INFINITY, l = 0.f;
  bool bad = false;  // this lane's half of the row failed the weight bound

  // Copies: wave w < NINST copies rows w*RPI .. +RPI-1 of a block; a block past
  // the workgroup's last one is addressed past the end of the plane and reads
  // zero without a memory access.
  const uint32_t plane_bytes = (uint32_t)n * HD * 2u;  // keys past n read zero
  const v4i rK = make_rsrc(k + kvoff, plane_bytes);
  const v4i rV = make_rsrc(v + kvoff, plane_bytes);
  const int crow = wave * P::RPI + lane / P::CPR;
  const uint32_t cvoff = (uint32_t)(crow * HD + (((lane % P::CPR) ^ P::TL::swz(crow)) << 3)) * 2u;
  auto copy = [&](const v4i& rs, bf16* slot, int blk) __attribute__((always_inline)) {
    if (wave < P::NINST)
      lds_copy16(rs, cvoff + (blk < nbw ? (uint32_t)blk * 32u * HD * 2u : plane_bytes),
                 slot + wave * 512);
  };

  // first copies (K_0..K_3, V_0, V_1) and the query operand, in flight together
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) copy(rK, sK[blk], blk);
  copy(rV, sV[0], 0);
  copy(rV, sV[1], 1);
  frag qf[P::NKS];
#pragma unroll
  for (int ks = 0; ks < P::NKS; ++ks)
    qf[ks] = q_ok ? row_frag_global<bf16, HD>(qp + (size_t)my_q * HD, g, ks) : zero_frag<bf16>();
  wait_global_loads();
  __syncthreads();

  // S^T of the block in K slot `slot`
  auto scores = [&](int slot, f32x16& s) __attribute__((always_inline)) {
    const bf16* tK = sK[slot];
    s = zero_acc();
#pragma unroll
    for (int ks = 0; ks < P::NKS; ++ks) M::mma(s, row_frag_lds<bf16, HD, 32>(tK, li, g, ks), qf[ks]);
  };
  // weights exp2(s*c - m) as operand fragments; returns their sum over this
  // lane's half of the block (the same rounded weights that enter the product)
  auto weights = [&](f32x16& s, frag* p) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = fast_exp2(fmaf(s[r], c, -m));
    p[0] = acc_frag<bf16>(s, 0);
    p[1] = acc_frag<bf16>(s, 8);
    return frag_sum(p[0], 0.f) + frag_sum(p[1], 0.f);
  };
  // diagonal block / sequence end: scores of keys past a row or past S are -inf
  auto mask = [&](int i, f32x16& s) __attribute__((always_inline)) {
    const int kb0 = 32 * i;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kv = kb0 + acc_row(r, g);
      s[r] = (kv <= my_q && kv < n) ? s[r] : -INFINITY;
    }
  };

  // Step 0: A(0), A(1), B(0) with the exact update (m starts at -inf).
  // Afterwards sA = S_1 and pA = P_0, the roles sub-step 1 expects.
  f32x16 sA, sB;
  frag pA[2], pB[2];
  scores(0, sB);
  scores(1, sA);
  if (nb == 1) mask(0, sB);
  {
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sB[r]);
    m = halves_max(mx) * c;  // finite: every row sees key 0
    l = weights(sB, pA);
  }
  __syncthreads();  // K_0, K_1 read before step 1 refills their slots

  // Sub-step i >= 1, J = i mod 4 (fixes the slots): A(i+1), B(i), C(i-1), the
  // same code for every wave, software-pipelined.  From its diagonal block on
  // (i >= nb-1) a wave masks B(i): past its rows every score is -inf, every
  // weight 0, so its last sub-steps add nothing and its A products are unused.
  // Only the mask is a branch, before the pipelined region; the products always
  // run, so the accumulators never change registers.
  auto sub = [&](auto jtag, f32x16& s_cur, f32x16& s_nxt, frag* p_prev, frag* p_cur,
                 int i) __attribute__((always_inline)) {
    constexpr int J = decltype(jtag)::value;
    if (i + 1 >= nb) mask(i, s_cur);
    __builtin_amdgcn_sched_barrier(0);
    // operands of both products first, so their LDS latency overlaps the
    // softmax arithmetic
    const bf16* tK = sK[(J + 1) % P::NSL];
    const bf16* tV = sV[(J + P::NSL - 1) % P::NSL];
    frag kf[P::NKS], vf[P::NC];
#pragma unroll
    for (int ks = 0; ks < P::NKS; ++ks) kf[ks] = row_frag_lds<bf16, HD, 32>(tK, li, g, ks);
#pragma unroll
    for (int t = 0; t < P::NC; ++t)
      vf[t] = accrow_frag<bf16, HD, 32>(tV, 0, t / P::ND, 32 * (t % P::ND), lane);
    float tsum = weights(s_cur, p_cur);
    // keep B(i) in this sub-step (it would otherwise sink next to its use in C(i))
    asm volatile("" : "+v"(p_cur[0]), "+v"(p_cur[1]), "+v"(tsum));
    s_nxt = zero_acc();
#pragma unroll
    for (int t = 0; t < (P::NKS > P::NC ? P::NKS : P::NC); ++t) {
      if (t < P::NKS) M::mma(s_nxt, kf[t], qf[t]);
      if (t < P::NC) M::mma(oacc[t % P::ND], vf[t], p_prev[t / P::ND]);
    }
    bad = bad || !(tsum <= kHalfBlockBound);
    l += tsum;
    // issue order: LDS reads, then the products (queued on the matrix
    // cores), then the softmax arithmetic
    __builtin_amdgcn_sched_group_barrier(0x100, P::NKS + 2 * P::NC, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, P::NKS + P::NC, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // Step u >= 1 (sub-steps 2u-1 and 2u; J0 = (2u-1) mod 4): first copies the
  // blocks of step u+1 (K_{2u+2}, K_{2u+3}, V_{2u}, V_{2u+1}; their slots were
  // last read in step u-1), then both sub-steps, then waits for the copies
  // and the barrier that publishes them.
  auto step = [&](auto j0tag, int u) __attribute__((always_inline)) {
    constexpr int J0 = decltype(j0tag)::value;  // 1 or 3
    prio_by_remaining(nbw - 2 * u);
    __builtin_amdgcn_sched_barrier(0);
    copy(rK, sK[(J0 + 3) % P::NSL], 2 * u + 2);
    copy(rK, sK[(J0 + 4) % P::NSL], 2 * u + 3);
    copy(rV, sV[(J0 + 1) % P::NSL], 2 * u);
    copy(rV, sV[(J0 + 2) % P::NSL], 2 * u + 1);
    sub(std::integral_constant<int, J0>{}, sA, sB, pA, pB, 2 * u - 1);
    sub(std::integral_constant<int, (J0 + 1) % P::NSL>{}, sB, sA, pB, pA, 2 * u);
    wait_global_loads();
    __syncthreads();
  };

  // steps 1 .. ceil(nbw/2): sub-step nbw is the drain of the last wave
  for (int u = 1;; u += 2) {
    step(std::integral_constant<int, 1>{}, u);
    if (2 * u >= nbw) break;
    step(std::integral_constant<int, 3>{}, u + 1);
    if (2 * u + 2 >= nbw) break;
  }

  if (q0 >= n) return;  // a wave of padding rows (stored at the start)
  const bool row_bad = halves_max(bad ? 1.f : 0.f) != 0.f;
  if (__builtin_expect(__ballot(row_bad) != 0, 0)) {
    // exact recompute of this wave's rows from HBM: running max, rescale per
    // block; only the failed rows take its result
    const bf16* kp = k + kvoff;
    const bf16* vp = v + kvoff;
    f32x16 acc2[P::ND];
#pragma unroll
    for (int d = 0; d < P::ND; ++d) acc2[d] = zero_acc();
    float m2 = -INFINITY, l2 = 0.f;
    for (int j = 0; j < nb; ++j) {
      const int key = 32 * j + li;
      f32x16 s2 = zero_acc();
#pragma unroll
      for (int ks = 0; ks < P::NKS; ++ks)
        M::mma(s2, key < n ? row_frag_global<bf16, HD>(kp + (size_t)key * HD, g, ks) : zero_frag<bf16>(),
               qf[ks]);
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kv = 32 * j + acc_row(r, g);
        s2[r] = (kv <= my_q && kv < n) ? s2[r] : -INFINITY;
        mx = fmaxf(mx, s2[r]);
      }
      const float m_new = fmaxf(m2, halves_max(mx) * c);
      const float alpha = m_new == m2 ? 1.f : fast_exp2(m2 - m_new);
      m2 = m_new;
      l2 *= alpha;
#pragma unroll
      for (int d = 0; d < P::ND; ++d) acc2[d] *= alpha;
      frag p2[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) s2[r] = fast_exp2(fmaf(s2[r], c, -m2));
      p2[0] = acc_frag<bf16>(s2, 0);
      p2[1] = acc_frag<bf16>(s2, 8);
      l2 += frag_sum(p2[0], 0.f) + frag_sum(p2[1], 0.f);
#pragma unroll
      for (int ks = 0; ks < P::NAS; ++ks)
#pragma unroll
        for (int db = 0; db < P::ND; ++db) {
          // V^T operand: head-dim column 32*db + li (clamped for hd 16), keys
          // of the permuted contraction order, read one by one
          const int d = min(32 * db + li, HD - 1);
          frag vf;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int kv = 32 * j + acc_row(8 * ks + t, g);
            vf[t] = kv < n ? vp[(size_t)kv * HD + d] : (bf16)0.f;
          }
          M::mma(acc2[db], vf, p2[ks]);
        }
    }
    if (row_bad) {
      m = m2;
      l = l2;
#pragma unroll
      for (int d = 0; d < P::ND; ++d) oacc[d] = acc2[d];
    }
  }

  l = halves_sum(l);
  const float inv = 1.f / l;
  if (q_ok) {
    bf16* orow = o + ((size_t)bh * S + my_q) * HD;
#pragma unroll
    for (int db = 0; db < P::ND; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = 32 * db + 8 * rg + 4 * g;
        if (d0 < HD)
          store4<bf16>(orow + d0, oacc[db][4 * rg] * inv, oacc[db][4 * rg + 1] * inv,
                       oacc[db][4 * rg + 2] * inv, oacc[db][4 * rg + 3] * inv);
      }
    if (g == 0) lse[(size_t)bh * S + my_q] = (m + fast_log2(l)) * kLn2;
  }
}

template <typename T, int HD>
static void fwd_typed(const Dims& d, const void* q, const void* k, const void* v, void* o,
                      float* lse, const int* lens, float scale, hipStream_t stream) {
  using C = FwdCfg<T, HD>;
  static_assert(C::BM == fwd_tile_rows(0, HD) && C::NT == kThreads, "tiling differs from the plan");
  const int nqt = (d.S + C::BM - 1) / C::BM;
  const int BH = d.B * d.H;
  dim3 grid((unsigned)attn_plan(d, 0).fwd_blocks), block(C::NT);
  hipLaunchKernelGGL((attn_fwd_kernel<T, HD>), grid, block, 0, stream,
                     (const T*)q, (const T*)k, (const T*)v, (T*)o, lse, lens, d.S, d.H, d.Hkv,
                     nqt, BH, scale * kLog2e);
}

// Compute units of the current device, read once per device.
int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return 0;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int HD>
static void fwd_pipe(const Dims& d, const void* q, const void* k, const void* v, void* o,
                     float* lse, const int* lens, float scale, hipStream_t stream) {
  using P = FwdPipe<HD>;
  static_assert(P::BM == fwd_tile_rows(1, HD) && P::NT == kThreads, "tiling differs from the plan");
  const int nqt = (d.S + P::BM - 1) / P::BM;
  const int BH = d.B * d.H;
  dim3 grid((unsigned)attn_plan(d, 1).fwd_blocks), block(P::NT);
  hipLaunchKernelGGL((attn_fwd_pipe_kernel<HD>), grid, block, 0, stream,
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, lse, lens, d.S,
                     d.H, d.Hkv, nqt, BH, device_cu_count(), scale * kLog2e);
}

void launch_fwd(int dtype, const Dims& d, const void* q, const void* k, const void* v, void* o,
                float* lse, const int* lens, float scale, hipStream_t stream) {
  if (dtype == 0) {
    if (d.hd == 16) fwd_typed<float, 16>(d, q, k, v, o, lse, lens, scale, stream);
    else if (d.hd == 32) fwd_typed<float, 32>(d, q, k, v, o, lse, lens, scale, stream);
    else fwd_typed<float, 64>(d, q, k, v, o, lse, lens, scale, stream);
  } else {
    if (d.hd == 16) fwd_pipe<16>(d, q, k, v, o, lse, lens, scale, stream);
    else if (d.hd == 32) fwd_pipe<32>(d, q, k, v, o, lse, lens, scale, stream);
    else fwd_pipe<64>(d, q, k, v, o, lse, lens, scale, stream);
  }
}

}  // namespace xattn
