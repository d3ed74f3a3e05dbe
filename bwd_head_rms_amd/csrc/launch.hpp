// launch.hpp -- host-side launchers of the attention kernels (one per kernel
// family), called by the C ABI after it has validated every argument.
#pragma once
#include <hip/hip_runtime.h>

namespace xattn {

struct Dims {
  int B, S, H, Hkv, hd;
};

// Forward: o, lse from q, k, v.  dtype: 0 = fp32, 1 = bf16.
void launch_fwd(int dtype, const Dims& d, const void* q, const void* k, const void* v, void* o,
                float* lse, float scale, hipStream_t stream);

// Backward, first kernel: dq, and D = rowsum(dO * o) into `dws` ([B][H][S] float).
void launch_bwd_dq(int dtype, const Dims& d, const void* q, const void* k, const void* v,
                   const void* o, const float* lse, const void* dO, float* dq, float* dws,
                   float scale, hipStream_t stream);

// Backward, second kernel: dk, dv (group-summed), reading D from `dws`.
void launch_bwd_dkdv(int dtype, const Dims& d, const void* q, const void* k, const void* v,
                     const float* lse, const void* dO, const float* dws, float* dk, float* dv,
                     float scale, hipStream_t stream);

}  // namespace xattn
