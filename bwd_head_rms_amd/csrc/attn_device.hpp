// attn_device.hpp -- device building blocks shared by the attention kernels
// (gfx950 / CDNA4, wave64).
//
// Matrix products use the 32x32 MFMA family with fp32 accumulation:
//   fp32 : v_mfma_f32_32x32x2_f32   (each lane feeds 1 element of A and B)
//   bf16 : v_mfma_f32_32x32x16_bf16 (each lane feeds 8 elements of A and B)
// Operand layout (M = N = 32, lane l, group g = l / 32):
//   A: lane l supplies row m = l % 32, contraction elements of group g
//   B: lane l supplies column n = l % 32, contraction elements of group g
//   C: lane l holds column n = l % 32, rows acc_row(r, g) for r = 0..15
// The contraction index may be permuted freely as long as A and B use the same
// permutation; the kernels use two permutations:
//   * over the head dimension d: group g takes the half [g*hd/2, (g+1)*hd/2),
//     instruction ks takes KPL consecutive elements of it, so every lane's
//     operand is a contiguous run of memory;
//   * over the rows of an accumulator (the key index in P.V and dS.K, the query
//     index in P^T.dO and dS^T.Q): element t of instruction ks in group g is
//     accumulator row acc_row(ks*KPL + t, g), so an accumulator tile feeds the
//     next product as its B operand straight from registers, with no LDS
//     round trip and no cross-lane shuffle.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xattn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Row of accumulator register r held by lane group g in a 32x32 MFMA result.
__device__ __forceinline__ constexpr int acc_row(int r, int g) {
  return 8 * (r >> 2) + 4 * g + (r & 3);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Position of workgroup `bid` in a heaviest-first list of tiles, rearranged so
// that the workgroups one CU holds at the same time carry about equal work.  A
// fresh grid is dealt breadth-first: CU c receives workgroups c, c + ncu,
// c + 2 ncu, ... (measured on MI355X).  While the first `resident` passes of ncu
// workgroups are all in flight together, odd passes take the list backwards, so
// a CU that got one of the heaviest tiles of the first pass gets one of the
// lightest of the second.  The reversal moves whole blocks of 8, which keeps
// bid mod 8 (the XCD a workgroup lands on, and with it the head's shared L2).
// Later passes, dispatched as CUs free up, and grids whose CU count is not a
// multiple of 8 keep the plain order (as does an unknown CU count, ncu <= 0).
__device__ __forceinline__ int balanced_rank(int bid, int nwg, int ncu, int resident) {
  if (ncu <= 0 || (ncu & 7) != 0) return bid;
  const int j = bid / ncu, c = bid % ncu;
  if ((j & 1) == 0 || j >= resident || (j + 1) * ncu > nwg) return bid;
  return j * ncu + (ncu - 8 - (c & ~7)) + (c & 7);
}

// SIMD (0-3) of the compute unit that runs this wave: bits 5:4 of HW_ID.
__device__ __forceinline__ int wave_simd() {
  return (__builtin_amdgcn_s_getreg((4) | (0 << 6) | (31 << 11)) >> 4) & 3;
}

// Rank of this wave among the workgroup's NW waves ordered by (SIMD, wave
// index): a permutation of 0 .. NW-1 whatever the placement.  With NW = 4 and
// one wave on each SIMD of the CU it is the SIMD itself.  `scratch` holds NW
// ints of LDS; the call contains a workgroup barrier.
template <int NW>
__device__ __forceinline__ int simd_rank(int wave, int lane, int* scratch) {
  const int s = wave_simd();
  if (lane == 0) scratch[wave] = s;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int s2 = scratch[w];
    r += (s2 < s || (s2 == s && w < wave)) ? 1 : 0;
  }
  return r;
}

// Combine lanes l and l^32 (v_permlane32_swap exchanges the two half-waves: the
// two results hold x of lanes 0..31 and 32..63 in every lane's position).
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x),
                                                  __builtin_bit_cast(int, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x),
                                                  __builtin_bit_cast(int, x), false, false);
  return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

template <typename T> struct Mma;

template <> struct Mma<float> {
  static constexpr int KPL = 1;    // contraction elements per lane per instruction
  static constexpr int KSTEP = 2;  // contraction length per instruction
  static constexpr int PADR = 1;   // row padding (elements) of row-major LDS tiles
  typedef float frag;
  static __device__ __forceinline__ void mma(f32x16& acc, const frag& a, const frag& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
  }
};

template <> struct Mma<bf16> {
  static constexpr int KPL = 8;
  static constexpr int KSTEP = 16;
  static constexpr int PADR = 8;
  typedef bf16x8 frag;
  static __device__ __forceinline__ void mma(f32x16& acc, const frag& a, const frag& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }
};

// Accumulation into an accumulator kept in AGPRs (bf16 operands).  Written as
// inline assembly so that long-lived accumulators stay in the AGPR file and the
// VGPR file is left to the tiles that VALU code post-processes.  The compiler
// cannot see hazards inside the assembly, so it carries its own wait states: two
// before the MFMA (a VALU write of an operand just before), and mma_agpr_drain()
// (24) must run between the last accumulation and any read of the result.
__device__ __forceinline__ void mma_agpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mma_agpr_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"); }

// ---------------------------------------------------------------------------
// fp32 -> operand conversion of accumulator registers [r0, r0 + KPL)
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag acc_frag(const f32x16& x, int r0);

template <>
__device__ __forceinline__ float acc_frag<float>(const f32x16& x, int r0) { return x[r0]; }

// Sum of the eight bf16 values of an operand fragment, added to `acc`
// (v_dot2_f32_bf16 against (1, 1): four instructions, fp32 accumulation).
__device__ __forceinline__ float frag_sum(const bf16x8& f, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(bf16)1.f, (bf16)1.f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 4, 5), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 6, 7), one, acc, false);
  return acc;
}
__device__ __forceinline__ float frag_sum(float f, float acc) { return acc + f; }

template <>
__device__ __forceinline__ bf16x8 acc_frag<bf16>(const f32x16& x, int r0) {
  bf16x8 f;
#pragma unroll
  for (int t = 0; t < 8; ++t) f[t] = (bf16)x[r0 + t];  // v_cvt_pk_bf16_f32: nearest-even
  return f;
}

// ---------------------------------------------------------------------------
// Head-dimension operand of one row, straight from global memory:
// elements d = g*HD/2 + ks*KPL + t of `row` (a pointer to HD elements).
template <typename T, int HD>
__device__ __forceinline__ typename Mma<T>::frag row_frag_global(const T* row, int g, int ks) {
  if constexpr (sizeof(T) == 2) {
    uint4 u = *reinterpret_cast<const uint4*>(row + g * (HD / 2) + ks * 8);
    return __builtin_bit_cast(bf16x8, u);
  } else {
    return row[g * (HD / 2) + ks];
  }
}

// All head-dimension operands of one row, f[ks] = row_frag_global(row, g, ks),
// with 16-byte loads: bf16 one per operand, fp32 one per four operands (a
// lane's elements g*HD/2 .. g*HD/2 + HD/2 - 1 are contiguous).  Every row of a
// 16-byte aligned plane is 16-byte aligned.
template <typename T, int HD>
__device__ __forceinline__ void row_frags_global(const T* row, int g,
                                                 typename Mma<T>::frag (&f)[HD / Mma<T>::KSTEP]) {
  constexpr int NKS = HD / Mma<T>::KSTEP;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) f[ks] = row_frag_global<T, HD>(row, g, ks);
  } else {
    static_assert(NKS % 4 == 0, "fp32 operands come in fours");
    const float4* p = reinterpret_cast<const float4*>(row + g * (HD / 2));
#pragma unroll
    for (int i = 0; i < NKS / 4; ++i) {
      const float4 u = p[i];
      f[4 * i] = u.x;
      f[4 * i + 1] = u.y;
      f[4 * i + 2] = u.z;
      f[4 * i + 3] = u.w;
    }
  }
}

// ---------------------------------------------------------------------------
// LDS tiles of ROWS x HD elements.
//
// bf16: rows of HD elements with no padding, filled by global_load_lds_dwordx4
//   (buffer_load_dwordx4 with lds: each lane's 16 bytes land at the
//   instruction's LDS base + 16 * lane, so a wave instruction writes 1 KB of
//   consecutive rows and no per-row padding is possible).  Instead the 16-byte chunks of each row are XOR-swizzled by row:
//   logical chunk c of row r lives at physical chunk c ^ swz(r).  swz is chosen
//   (for 64 banks of 4 bytes) so that both read patterns are conflict free: 16
//   lanes reading one chunk of 16 consecutive rows, and the transpose reads
//   (4 consecutive rows x 4 consecutive chunks per half wave).  Rows past the
//   sequence end read as zero.
// fp32: rows padded to HD+1 elements (odd stride), staged through registers.
// Raw buffer resource (gfx9 layout) for `bytes` bytes at `base`: loads at byte
// offsets past the end return zero.  All fields are wave-uniform.
typedef int v4i __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4i make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return v4i{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
             __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xFFFFu)),
             __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

// One wave instruction copying 16 (or 4) bytes per lane from a buffer into LDS:
// lane l's bytes, read at byte offset voff, land at lds_dst + 16*l (4*l)
// (buffer_load_dwordx4 / _dword with lds, LDS base in M0).  The whole offset
// is passed in the VGPR operand, the part of the address that the buffer range
// check covers (the SGPR offset is added after the check), so every byte at or
// past the end of the resource reads as zero.
//
// The LDS base is an input operand bound to M0 ("{m0}"): the compiler itself
// writes M0 before the statement and knows it is read there, so M0 is never
// changed behind its back.  The leading s_nop is the one wait state an M0
// write needs before an LDS DMA reads it (the compiler's hazard check does not
// look inside assembly).  The copy is assembly rather than the compiler's
// buffer-load-to-LDS builtin because with the builtin the compiler cannot tell
// a copy into one ring slot from reads of another and waits for every copy in
// flight before the first LDS read that follows it, which serialises the
// next tile's copy with the arithmetic on the current one.  Completion is
// awaited explicitly (wait_global_loads) before the barrier that publishes a
// tile.
__device__ __forceinline__ void lds_copy16(v4i rsrc, uint32_t voff, const void* lds_dst) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_dst);
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "{m0}"(base)
               : "memory");
}
__device__ __forceinline__ void lds_copy4(v4i rsrc, uint32_t voff, const void* lds_dst) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_dst);
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "{m0}"(base)
               : "memory");
}

template <typename T, int HD, int ROWS>
struct Tile;

template <int HD, int ROWS>
struct Tile<bf16, HD, ROWS> {
  static constexpr int CPR = HD / 8;          // 16-byte chunks per row
  static constexpr int ELEMS = ROWS * HD;
  static constexpr int ROWS_PER_INST = 64 / CPR;
  static constexpr int NINST = ROWS / ROWS_PER_INST;
  static_assert(ROWS % ROWS_PER_INST == 0, "tile rows must fill whole wave loads");

  __device__ static constexpr int swz(int r) {
    if constexpr (CPR == 8) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    else if constexpr (CPR == 4) return (r >> 2) & 3;
    else return (r >> 3) & 1;
  }
  // Element offset of (row r, column col); valid for accesses inside one chunk.
  __device__ static int off(int r, int col) {
    return r * HD + ((((col >> 3) ^ swz(r))) << 3) + (col & 7);
  }
  // Issue the asynchronous copy of rows [row0, row0 + ROWS) of a head plane of
  // S rows (row stride HD) into `tile`, shared by NW waves; rows past S read
  // zero.  Completion is tracked by vmcnt: wait for it before the barrier that
  // publishes the tile.
  template <int NW>
  __device__ static void issue(const bf16* plane, int row0, int S, bf16* tile, int wave, int lane) {
    const v4i rsrc = make_rsrc(plane, (uint32_t)S * HD * 2u);
#pragma unroll
    for (int i = wave; i < NINST; i += NW) {
      const int r = i * ROWS_PER_INST + lane / CPR;
      const int chunk = (lane % CPR) ^ swz(r);
      lds_copy16(rsrc, (uint32_t)((row0 + r) * HD + chunk * 8) * 2u, tile + i * 512);
    }
  }
};

template <int HD, int ROWS>
struct Tile<float, HD, ROWS> {
  static constexpr int RS = HD + 1;
  static constexpr int ELEMS = ROWS * RS;
  __device__ static int off(int r, int col) { return r * RS + col; }
};

// Register staging of an fp32 tile: load() issues the global loads (rows past
// the sequence end read as zero), store() writes them to LDS.
template <int HD, int ROWS, int NT>
struct F32Stage {
  static constexpr int CPR = HD / 4;
  static constexpr int ITEMS = ROWS * CPR;
  static constexpr int PER = (ITEMS + NT - 1) / NT;
  float4 buf[PER];

  __device__ __forceinline__ void load(const float* plane, int row0, int S, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int item = tid + i * NT;
      const int r = item / CPR, c = item % CPR;
      float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
      if ((ITEMS % NT == 0 || item < ITEMS) && row0 + r < S)
        val = *reinterpret_cast<const float4*>(plane + (size_t)(row0 + r) * HD + c * 4);
      buf[i] = val;
    }
  }
  __device__ __forceinline__ void store(float* tile, int tid) const {
    constexpr int RS = Tile<float, HD, ROWS>::RS;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int item = tid + i * NT;
      if (ITEMS % NT != 0 && item >= ITEMS) continue;
      const int r = item / CPR, c = item % CPR;
      tile[r * RS + c * 4 + 0] = buf[i].x;
      tile[r * RS + c * 4 + 1] = buf[i].y;
      tile[r * RS + c * 4 + 2] = buf[i].z;
      tile[r * RS + c * 4 + 3] = buf[i].w;
    }
  }
};

// Double-buffered staging of one tensor's tiles: issue(next) before the
// arithmetic on the current tile, commit(next) after it; a barrier follows.
// bf16 copies asynchronously straight into LDS; fp32 goes through registers.
template <typename T, int HD, int ROWS, int NW>
struct Stager {
  using TL = Tile<T, HD, ROWS>;
  F32Stage<HD, ROWS, NW * kWave> regs;  // unused for bf16
  __device__ __forceinline__ void issue(const T* plane, int row0, int S, T* tile, int wave,
                                        int lane, int tid) {
    if constexpr (sizeof(T) == 2)
      TL::template issue<NW>(plane, row0, S, tile, wave, lane);
    else
      regs.load(plane, row0, S, tid);
  }
  __device__ __forceinline__ void commit(T* tile, int tid) const {
    if constexpr (sizeof(T) == 4) regs.store(tile, tid);
  }
};

// Wait for all of this wave's outstanding global loads, including copies into
// LDS.  The wait is the compiler's own s_waitcnt (vmcnt(0); expcnt and lgkmcnt
// left at their maximum, gfx9 encoding), so the compiler also knows that no
// load is pending afterwards and adds no waits of its own later; the empty asm
// keeps memory accesses from moving across it.
__device__ __forceinline__ void wait_global_loads() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  asm volatile("" ::: "memory");
}

// Head-dimension operand of tile row r (elements d = g*HD/2 + ks*KPL + t).
template <typename T, int HD, int ROWS>
__device__ __forceinline__ typename Mma<T>::frag row_frag_lds(const T* tile, int r, int g, int ks) {
  using TL = Tile<T, HD, ROWS>;
  if constexpr (sizeof(T) == 2) {
    const uint4 u = *reinterpret_cast<const uint4*>(tile + TL::off(r, g * (HD / 2) + ks * 8));
    return __builtin_bit_cast(bf16x8, u);
  } else {
    return tile[TL::off(r, g * (HD / 2) + ks)];
  }
}

// ---------------------------------------------------------------------------
// Accumulator-row operand of instruction ks for a 32-row block starting at tile
// row `base`: element t for lane group g is tile row base + acc_row(ks*KPL+t, g),
// at head-dimension column col0 + l%32 (duplicated for hd 16).
//
// bf16: ds_read_b64_tr_b16.  Within each 16-lane group that instruction hands
//   lane i element (i mod 4) of the 8 bytes addressed by lane 4t + floor(i/4),
//   as its element t (t = 0..3).  So lane j of the group addresses row
//   base' + floor(j/4), columns 4*(j mod 4) .. +3, and lane i receives column i
//   of rows base' .. base'+3: four consecutive rows of one column, as the
//   contraction needs.  Two reads give the two runs of four rows
//   (16ks + 4g + 0..3 and 16ks + 8 + 4g + 0..3) of the permuted contraction
//   order.  No transposed copy of a tile is ever stored.
// fp32: one element per lane, read directly.
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

template <typename T, int HD, int ROWS>
__device__ __forceinline__ typename Mma<T>::frag accrow_frag(const T* tile, int base, int ks,
                                                              int col0, int lane) {
  using TL = Tile<T, HD, ROWS>;
  const int g = lane >> 5;
  if constexpr (sizeof(T) == 2) {
    const int j = lane & 15, G = lane >> 4;
    const int row = base + 16 * ks + 4 * g + (j >> 2);
    const int col = col0 + (HD >= 32 ? 16 * (G & 1) : 0) + 4 * (j & 3);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(tile + TL::off(row, col)));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(tile + TL::off(row + 8, col)));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const v8i16 u = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, u);
  } else {
    return tile[TL::off(base + acc_row(ks, g), min(col0 + (lane & 31), HD - 1))];
  }
}

template <typename T>
__device__ __forceinline__ typename Mma<T>::frag zero_frag() {
  if constexpr (sizeof(T) == 2) {
    return __builtin_bit_cast(bf16x8, make_uint4(0u, 0u, 0u, 0u));
  } else {
    return 0.f;
  }
}

__device__ __forceinline__ f32x16 zero_acc() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Valid length of sequence b of a right-padded batch: lens[b] clamped to
// [0, S], or S when there are no lengths.
__device__ __forceinline__ int seq_len(const int* lens, int b, int S) {
  if (!lens) return S;
  const int n = lens[b];
  return n < 0 ? 0 : (n > S ? S : n);
}

// hd zeros (fp32), 16-byte stores
template <int HD>
__device__ __forceinline__ void zero_row(float* row) {
#pragma unroll
  for (int d = 0; d < HD; d += 4) *reinterpret_cast<float4*>(row + d) = make_float4(0.f, 0.f, 0.f, 0.f);
}

// Store four consecutive fp32 values (d0 .. d0+3 of one row) as T.
template <typename T>
__device__ __forceinline__ void store4(T* dst, float a, float b, float c, float d);

template <>
__device__ __forceinline__ void store4<float>(float* dst, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
}

template <>
__device__ __forceinline__ void store4<bf16>(bf16* dst, float a, float b, float c, float d) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 v;
  v[0] = (bf16)a; v[1] = (bf16)b; v[2] = (bf16)c; v[3] = (bf16)d;
  *reinterpret_cast<uint2*>(dst) = __builtin_bit_cast(uint2, v);
}

}  // namespace xattn
