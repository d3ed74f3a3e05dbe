// launch.hpp -- host-side launchers of the attention kernels (one per kernel
// family), called by the C ABI after it has validated every argument, and the
// launch sizing they share with that validation (plan.cpp).
#pragma once
#include <hip/hip_runtime_api.h>

#include <stddef.h>

namespace xattn {

struct Dims {
  int B, S, H, Hkv, hd;
};

// Threads per workgroup of every kernel in the library.
constexpr int kThreads = 256;
// HIP takes at most 2^32 - 1 work-items in one launch: with kThreads per
// workgroup, at most this many workgroups.
constexpr long long kMaxBlocks = 0xFFFFFFFFLL / kThreads;

// Tiling of the attention kernels (each kernel static_asserts its own).
// query rows per forward workgroup: four waves of 32 rows, except fp32 at
// hd <= 32 (two row blocks of 32, each split over two waves by key)
constexpr int fwd_tile_rows(int dtype, int hd) { return dtype == 0 && hd <= 32 ? 64 : 128; }
// query rows per dq workgroup: four waves, except fp32 at hd 64 (two)
constexpr int dq_tile_rows(int dtype, int hd) { return dtype == 0 ? 64 : 128; }
// keys per dk/dv workgroup: 128 (a wave per 32 keys), except fp32 at hd <= 32:
// 64, two waves per 32 keys, each taking half of the query blocks
constexpr int dkdv_tile_keys(int dtype, int hd) { return dtype == 0 && hd <= 32 ? 64 : 128; }
constexpr int kCmpTile = 128;      // rows and keys per composed-path tile

// Workgroups of each launch one attention call makes, and its workspace.
struct AttnPlan {
  long long fwd_blocks, dq_blocks, dkdv_blocks, dkdv_sum_blocks;
  int split;               // slices a GQA group is split into by the dk/dv kernel
  size_t workspace_bytes;  // backward workspace
};
// split_groups = false keeps each GQA group in one dk/dv workgroup (split = 1),
// so the workspace is the per-row part only.
AttnPlan attn_plan(const Dims& d, int dtype, bool split_groups = true);

// Largest grid of the composed path's launches.
long long composed_max_blocks(const Dims& d);

// `lens` ([B] int32 on the device, or NULL): sequence b holds lens[b] rows
// (clamped to [0, S]) of its right-padded S-row planes; rows and keys past it
// are padding, never read, and their outputs are written as zeros (lse -inf).

// Forward: o, lse from q, k, v.  dtype: 0 = fp32, 1 = bf16.
void launch_fwd(int dtype, const Dims& d, const void* q, const void* k, const void* v, void* o,
                float* lse, const int* lens, float scale, hipStream_t stream);

// Backward, first kernel: dq, and D = rowsum(dO * o) into `dws` ([B][H][S] float).
void launch_bwd_dq(int dtype, const Dims& d, const void* q, const void* k, const void* v,
                   const void* o, const float* lse, const void* dO, float* dq, float* dws,
                   const int* lens, float scale, hipStream_t stream);

// Backward, second kernel: dk, dv (group-summed), reading D from `dws`.  When
// split_groups and dkdv_split(d, dtype) > 1 the query heads of a group are
// spread over workgroups that write partial dk, dv into `dws` at
// dkdv_part_offset(d) floats ([2][group][B][Hkv][S][hd]), summed in ascending
// head order by a second kernel.
void launch_bwd_dkdv(int dtype, const Dims& d, const void* q, const void* k, const void* v,
                     const float* lse, const void* dO, float* dws, float* dk, float* dv,
                     const int* lens, float scale, bool split_groups, hipStream_t stream);

// Short bf16 sequences: one backward kernel per (batch, head) that holds the
// whole head in LDS and writes dq, dk and dv (bitwise the two kernels'
// results).  Taken for bf16, hd <= 32, S <= kShortMaxS and one query head per
// kv head.
constexpr int kShortMaxS = 256;
bool bwd_short_path(const Dims& d, int dtype);
// Its grid: `full` workgroups of one head each, then pairs of workgroups that
// split one head into its key side and its query side.  Two workgroups fit a
// CU at once; with ncu CUs and B*H heads between ncu and 2*ncu, 2*ncu - B*H
// heads are split, so that each CU holds one whole head and one half (fewer
// heads: every head split; ncu unknown or more heads: none).
struct ShortSplit {
  long long full, blocks;
};
ShortSplit short_split(const Dims& d, int ncu);
void launch_bwd_short(const Dims& d, const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dO, float* dq, float* dk, float* dv,
                      const int* lens, float scale, hipStream_t stream);

// Device address of the fixed scratch array of the allocation-free backward on
// the current device (looked up once per device), or NULL if it cannot be
// read.  Holds kNoAllocScratchBytes.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
float* noalloc_scratch();
int dkdv_split(const Dims& d, int dtype);

// Compute units of the current device (0 if it cannot be read), cached per device.
int device_cu_count();
size_t dkdv_part_offset(const Dims& d);

// Per-head RMS QK-norm + rotary embedding.  x [B][S][H][hd] (token-major),
// out and dout [B][H][S][hd], dx [B][S][H][hd], w and dw [hd].
struct NormDims {
  int B, S, H, hd;
};

// Largest grid of the backward kernel: its workspace holds one fp32 row of hd
// partial weight-gradient sums per workgroup.
constexpr int kNormMaxBlocks = 1024;

// Workgroups the backward launches for nvec = B*S*H head vectors.
int qknorm_bwd_blocks(long nvec, int hd);

void launch_qknorm_rope_fwd(int dtype, const NormDims& d, const void* x, const float* w,
                            void* out, float eps, float base, hipStream_t stream);

void launch_qknorm_rope_bwd(int dtype, const NormDims& d, const void* x, const float* w,
                            const float* dout, float* dx, float* dw, float* ws, float eps,
                            float base, hipStream_t stream);

// Composed path: scores, causal softmax and products through S x S fp32
// buffers p (probabilities, kept from forward to backward) and ds ([B][H][S][S]).
void launch_composed_fwd(int dtype, const Dims& d, const void* q, const void* k, const void* v,
                         void* o, float* lse, float* p, float scale, hipStream_t stream);
void launch_composed_bwd(int dtype, const Dims& d, const void* q, const void* k, const void* v,
                         const float* p, const void* dO, float* dq, float* dk, float* dv,
                         float* ds, float scale, hipStream_t stream);

// Decode attention: q, o [B][H][hd]; k, v [B][Hkv][T][hd] with T in Dims::S;
// lens [B] (nullable); part is the workspace (nullable when part_bytes == 0).
constexpr int kDecMinChunk = 256, kDecMaxChunk = 1024;  // cache positions per workgroup
struct DecodePlan {
  int chunk;            // cache positions per workgroup
  int nsplit;           // chunks per sequence
  int heads_per_wg;     // query heads of a GQA group one workgroup serves
  long blocks;          // workgroups of the main kernel
  long combine_blocks;  // workgroups of the merge kernel (0: no merge)
  size_t part_bytes;    // workspace: partial records when nsplit > 1
};
DecodePlan decode_plan(int B, int T, int H, int Hkv, int hd);

// Longest cache decode accepts: 4096 chunks of at most 1024 positions.
constexpr long kDecodeMaxT = 4096L * 1024;

void launch_decode(int dtype, const Dims& d, const void* q, const void* k, const void* v,
                   const int* lens, void* o, float* lse, float* part, float scale,
                   hipStream_t stream);

}  // namespace xattn
