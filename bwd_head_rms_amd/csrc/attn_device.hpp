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

// ---------------------------------------------------------------------------
// fp32 -> operand conversion of accumulator registers [r0, r0 + KPL)
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag acc_frag(const f32x16& x, int r0);

template <>
__device__ __forceinline__ float acc_frag<float>(const f32x16& x, int r0) { return x[r0]; }

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

// Same, from a row-major LDS tile.
template <typename T, int HD>
__device__ __forceinline__ typename Mma<T>::frag row_frag_lds(const T* row, int g, int ks) {
  if constexpr (sizeof(T) == 2) {
    uint4 u = *reinterpret_cast<const uint4*>(row + g * (HD / 2) + ks * 8);
    return __builtin_bit_cast(bf16x8, u);
  } else {
    return row[g * (HD / 2) + ks];
  }
}

// ---------------------------------------------------------------------------
// Accumulator-row operand: element t of instruction ks for lane group g is tile
// row acc_row(ks*KPL + t, g) (rows relative to a 32-row block base), at
// head-dimension column col0 + l%32 (clamped to the head dimension for hd 16).
//
// bf16: read from the row-major LDS tile with ds_read_b64_tr_b16.  Within each
//   16-lane group that instruction hands lane i element (i mod 4) of the 8 bytes
//   addressed by lane 4t + floor(i/4), as its element t (t = 0..3).  So lane j of
//   the group addresses row base + floor(j/4), columns 4*(j mod 4) .. +3, and lane
//   i receives column i of rows base .. base+3: four consecutive rows of one
//   column, as the contraction needs.  Two reads give the two runs of four rows
//   (16ks + 4g + 0..3 and 16ks + 8 + 4g + 0..3) of the permuted contraction order.
//   No transposed copy of the tile is ever stored.
// fp32: one element per lane, read directly from the row-major tile.
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

template <int HD, int RS>
__device__ __forceinline__ bf16x8 accrow_frag_bf16(const bf16* tile, int row_base, int col0,
                                                   int lane) {
  const int j = lane & 15, G = lane >> 4, g = lane >> 5;
  const int row = row_base + 4 * g + (j >> 2);
  const int col = col0 + (HD >= 32 ? 16 * (G & 1) : 0) + 4 * (j & 3);
  const bf16* p = tile + row * RS + col;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 8 * RS));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 u = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, u);
}

template <int RS>
__device__ __forceinline__ float accrow_frag_f32(const float* rt, int col, int g, int ks) {
  return rt[acc_row(ks, g) * RS + col];
}

// ---------------------------------------------------------------------------
// Cooperative global -> LDS staging of a ROWS x HD tile, rows [row0, row0+ROWS)
// of a head plane, zero-filling rows >= nvalid.  Work items are 16-byte chunks;
// each thread keeps its items in registers between load() and store() so the
// global loads of a later tile overlap the current tile's arithmetic.  store()
// writes the tile row-major with row stride RS elements.
template <typename T, int HD, int ROWS, int NT>
struct TileStage {
  static constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  static constexpr int CPR = HD / EPC;             // chunks per row
  static constexpr int ITEMS = ROWS * CPR;
  static constexpr int PER = (ITEMS + NT - 1) / NT;
  uint4 buf[PER];

  __device__ __forceinline__ void load(const T* plane, int row0, int nvalid, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int item = tid + i * NT;
      const int r = item / CPR, c = item % CPR;
      uint4 val = make_uint4(0u, 0u, 0u, 0u);
      if ((ITEMS % NT == 0 || item < ITEMS) && r < nvalid)
        val = *reinterpret_cast<const uint4*>(plane + (size_t)(row0 + r) * HD + c * EPC);
      buf[i] = val;
    }
  }

  template <int RS>
  __device__ __forceinline__ void store(T* tile, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int item = tid + i * NT;
      if (ITEMS % NT != 0 && item >= ITEMS) continue;
      const int r = item / CPR, c = item % CPR;
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<uint4*>(tile + r * RS + c * EPC) = buf[i];
      } else {
        const float* f = reinterpret_cast<const float*>(&buf[i]);
#pragma unroll
        for (int e = 0; e < 4; ++e) tile[r * RS + c * EPC + e] = f[e];
      }
    }
  }
};

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
