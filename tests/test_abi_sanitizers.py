"""The C ABI's host code (api.cpp, plan.cpp) built with AddressSanitizer and
UndefinedBehaviorSanitizer (g++, host only) against stub launchers that only
count what would be enqueued, and driven through every status code the header
defines: valid calls enqueue their kernels, every invalid call returns its
status and enqueues nothing (including shapes whose grids exceed what one HIP
launch takes), a failed launch reports XATTN_ERR_HIP.  CPU only: no HIP call
is ever made."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bwd_head_rms_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
ROCM_INCLUDE = "/opt/rocm/include"

DRIVER = r"""
#include <cmath>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <limits>

#include "launch.hpp"
#include "xattn.h"

static int g_launches = 0;
static bool g_fail = false;  // the next hipGetLastError reports a failure
static bool g_no_scratch = false;  // the scratch address lookup fails

hipError_t hipGetLastError() {
  const bool f = g_fail;
  g_fail = false;
  return f ? hipErrorInvalidConfiguration : hipSuccess;
}

namespace xattn {
void launch_fwd(int, const Dims&, const void*, const void*, const void*, void*, float*, const int*,
                float, hipStream_t) { ++g_launches; }
void launch_bwd_dq(int, const Dims&, const void*, const void*, const void*, const void*,
                   const float*, const void*, float*, float*, const int*, float, hipStream_t) {
  ++g_launches;
}
void launch_bwd_dkdv(int, const Dims&, const void*, const void*, const void*, const float*,
                     const void*, float*, float*, float*, const int*, float, bool, hipStream_t) {
  ++g_launches;
}
void launch_bwd_short(const Dims&, const void*, const void*, const void*, const void*,
                      const float*, const void*, float*, float*, float*, const int*, float,
                      hipStream_t) {
  ++g_launches;
}
alignas(256) static float g_scratch_stub[64];
float* noalloc_scratch() { return g_no_scratch ? nullptr : g_scratch_stub; }
int device_cu_count() { return 256; }
void launch_qknorm_rope_fwd(int, const NormDims&, const void*, const float*, void*, float, float,
                            hipStream_t) { ++g_launches; }
void launch_qknorm_rope_bwd(int, const NormDims&, const void*, const float*, const float*, float*,
                            float*, float*, float, float, hipStream_t) { ++g_launches; }
void launch_composed_fwd(int, const Dims&, const void*, const void*, const void*, void*, float*,
                         float*, float, hipStream_t) { ++g_launches; }
void launch_composed_bwd(int, const Dims&, const void*, const void*, const void*, const float*,
                         const void*, float*, float*, float*, float*, float, hipStream_t) {
  ++g_launches;
}
void launch_decode(int, const Dims&, const void*, const void*, const void*, const int*, void*,
                   float*, float*, float, hipStream_t) { ++g_launches; }
}  // namespace xattn

static int g_failures = 0, g_checks = 0;
#define EXPECT(call, status, launches)                                                      \
  do {                                                                                      \
    g_launches = 0;                                                                         \
    const int rc_ = (call);                                                                 \
    ++g_checks;                                                                             \
    if (rc_ != (status) || g_launches != (launches)) {                                      \
      std::printf("FAIL line %d: %s -> %d (want %d), %d launches (want %d)\n", __LINE__,   \
                  #call, rc_, (int)(status), g_launches, (int)(launches));                  \
      ++g_failures;                                                                         \
    }                                                                                       \
  } while (0)

alignas(64) static unsigned char g_mem[16][256];

int main() {
  void* p[16];
  for (int i = 0; i < 16; ++i) p[i] = g_mem[i];
  float* f[16];
  for (int i = 0; i < 16; ++i) f[i] = reinterpret_cast<float*>(g_mem[i]);
  const void* q = p[0]; const void* k = p[1]; const void* v = p[2]; void* o = p[3];
  float* lse = f[4]; const void* dO = p[5]; float* dq = f[6]; float* dk = f[7]; float* dv = f[8];
  void* ws = p[9];
  const int* lens = reinterpret_cast<const int*>(g_mem[10]);
  const void* mis = g_mem[11] + 4;  // 4-byte aligned, not 16
  const float nan = std::numeric_limits<float>::quiet_NaN();
  const float inf = std::numeric_limits<float>::infinity();
  const size_t WS = (size_t)1 << 40;  // "large enough" for every shape below

  // --- forward
  EXPECT(xattn_fwd(q, k, v, o, lse, 2, 100, 4, 2, 64, 0.125f, XATTN_BF16, nullptr), XATTN_OK, 1);
  EXPECT(xattn_fwd(q, k, v, o, lse, 2, 100, 4, 2, 32, 0.125f, XATTN_F32, nullptr), XATTN_OK, 1);
  EXPECT(xattn_fwd(nullptr, k, v, o, lse, 2, 100, 4, 2, 64, 0.125f, 1, nullptr), XATTN_ERR_NULL, 0);
  EXPECT(xattn_fwd(q, k, v, o, nullptr, 2, 100, 4, 2, 64, 0.125f, 1, nullptr), XATTN_ERR_NULL, 0);
  EXPECT(xattn_fwd(q, k, v, o, lse, 0, 100, 4, 2, 64, 0.125f, 1, nullptr), XATTN_ERR_SHAPE, 0);
  EXPECT(xattn_fwd(q, k, v, o, lse, 2, -1, 4, 2, 64, 0.125f, 1, nullptr), XATTN_ERR_SHAPE, 0);
  EXPECT(xattn_fwd(q, k, v, o, lse, 2, 100, 0, 2, 64, 0.125f, 1, nullptr), XATTN_ERR_SHAPE, 0);
  EXPECT(xattn_fwd(q, k, v, o, lse, 2, 100, 4, 3, 64, 0.125f, 1, nullptr), XATTN_ERR_GQA, 0);
  EXPECT(xattn_fwd(q, k, v, o, lse, 2, 100, 4, 2, 48, 0.125f, 1, nullptr), XATTN_ERR_HEAD_DIM, 0);
  EXPECT(xattn_fwd(q, k, v, o, lse, 2, 100, 4, 2, 128, 0.125f, 1, nullptr), XATTN_ERR_HEAD_DIM, 0);
  EXPECT(xattn_fwd(q, k, v, o, lse, 2, 100, 4, 2, 64, 0.125f, 2, nullptr), XATTN_ERR_DTYPE, 0);
  EXPECT(xattn_fwd(q, k, v, o, lse, 2, 100, 4, 2, 64, 0.125f, -1, nullptr), XATTN_ERR_DTYPE, 0);
  EXPECT(xattn_fwd(q, k, v, o, lse, 2, 100, 4, 2, 64, nan, 1, nullptr), XATTN_ERR_SCALE, 0);
  EXPECT(xattn_fwd(q, k, v, o, lse, 2, 100, 4, 2, 64, inf, 1, nullptr), XATTN_ERR_SCALE, 0);
  EXPECT(xattn_fwd(q, k, v, o, lse, 2, 100, 4, 2, 64, 0.f, 1, nullptr), XATTN_ERR_SCALE, 0);
  EXPECT(xattn_fwd(q, k, v, o, lse, 2, 100, 4, 2, 64, -0.5f, 1, nullptr), XATTN_ERR_SCALE, 0);
  EXPECT(xattn_fwd(mis, k, v, o, lse, 2, 100, 4, 2, 64, 0.125f, 1, nullptr), XATTN_ERR_ALIGN, 0);
  EXPECT(xattn_fwd(q, k, v, (void*)mis, lse, 2, 100, 4, 2, 64, 0.125f, 1, nullptr),
         XATTN_ERR_ALIGN, 0);
  // one (batch, head) plane of 2^31 elements or more
  EXPECT(xattn_fwd(q, k, v, o, lse, 1, 1 << 25, 1, 1, 64, 0.125f, 1, nullptr), XATTN_ERR_SHAPE, 0);
  // 65536 * 256 * 1 = 2^24 forward workgroups: one more than a launch takes
  EXPECT(xattn_fwd(q, k, v, o, lse, 65536, 128, 256, 256, 16, 0.25f, 1, nullptr),
         XATTN_ERR_SHAPE, 0);
  EXPECT(xattn_fwd(q, k, v, o, lse, 65535, 128, 256, 256, 16, 0.25f, 1, nullptr), XATTN_OK, 1);
  // a launch the runtime rejects
  g_fail = true;
  EXPECT(xattn_fwd(q, k, v, o, lse, 2, 100, 4, 2, 64, 0.125f, 1, nullptr), XATTN_ERR_HIP, 1);

  // --- ragged forward / backward: lens is required and 4-byte aligned
  EXPECT(xattn_fwd_ragged(q, k, v, lens, o, lse, 2, 100, 4, 2, 64, 0.125f, 1, nullptr), XATTN_OK, 1);
  EXPECT(xattn_fwd_ragged(q, k, v, nullptr, o, lse, 2, 100, 4, 2, 64, 0.125f, 1, nullptr),
         XATTN_ERR_NULL, 0);
  EXPECT(xattn_fwd_ragged(q, k, v, reinterpret_cast<const int*>(g_mem[10] + 2), o, lse, 2, 100, 4,
                          2, 64, 0.125f, 1, nullptr), XATTN_ERR_ALIGN, 0);
  EXPECT(xattn_bwd_ragged(q, k, v, o, lse, dO, lens, dq, dk, dv, 2, 100, 4, 2, 64, 0.125f, 1, ws,
                          WS, nullptr), XATTN_OK, 2);
  EXPECT(xattn_bwd_ragged(q, k, v, o, lse, dO, nullptr, dq, dk, dv, 2, 100, 4, 2, 64, 0.125f, 1,
                          ws, WS, nullptr), XATTN_ERR_NULL, 0);

  // --- workspace sizes
  {
    const size_t a = xattn_bwd_workspace_bytes(4, 2048, 16, 16, 64, XATTN_BF16);
    if (a != 8ull * 4 * 16 * 2048) { std::printf("FAIL ws size %zu\n", a); ++g_failures; }
    // few kv tiles: the group is split and the partials need room
    const size_t b = xattn_bwd_workspace_bytes(16, 1024, 8, 2, 64, XATTN_BF16);
    if (b <= 8ull * 16 * 8 * 1024) { std::printf("FAIL split ws size %zu\n", b); ++g_failures; }
    const size_t z[] = {xattn_bwd_workspace_bytes(0, 16, 2, 2, 16, 0),
                        xattn_bwd_workspace_bytes(1, 16, 3, 2, 16, 0),
                        xattn_bwd_workspace_bytes(1, 16, 2, 2, 24, 0),
                        xattn_bwd_workspace_bytes(1, 16, 2, 2, 16, 7),
                        xattn_bwd_workspace_bytes(65536, 128, 256, 256, 16, 1)};
    for (size_t x : z)
      if (x != 0) { std::printf("FAIL invalid ws size %zu\n", x); ++g_failures; }
    g_checks += 7;
  }

  // --- backward (two launches, or none)
  const size_t need = xattn_bwd_workspace_bytes(2, 100, 4, 2, 64, XATTN_BF16);
  EXPECT(xattn_bwd(q, k, v, o, lse, dO, dq, dk, dv, 2, 100, 4, 2, 64, 0.125f, 1, ws, need, nullptr),
         XATTN_OK, 2);
  EXPECT(xattn_bwd(q, k, v, o, lse, dO, dq, dk, dv, 2, 100, 4, 2, 64, 0.125f, 1, ws, need - 1,
                   nullptr), XATTN_ERR_WORKSPACE, 0);
  EXPECT(xattn_bwd(q, k, v, o, lse, dO, dq, dk, dv, 2, 100, 4, 2, 64, 0.125f, 1, nullptr, WS,
                   nullptr), XATTN_ERR_WORKSPACE, 0);
  EXPECT(xattn_bwd(q, k, v, o, lse, dO, dq, dk, dv, 2, 100, 4, 2, 64, 0.125f, 1, (void*)mis, WS,
                   nullptr), XATTN_ERR_ALIGN, 0);
  EXPECT(xattn_bwd(q, k, v, o, lse, dO, (float*)mis, dk, dv, 2, 100, 4, 2, 64, 0.125f, 1, ws, WS,
                   nullptr), XATTN_ERR_ALIGN, 0);
  EXPECT(xattn_bwd(q, k, v, o, lse, dO, dq, (float*)mis, dv, 2, 100, 4, 2, 64, 0.125f, 1, ws, WS,
                   nullptr), XATTN_ERR_ALIGN, 0);
  EXPECT(xattn_bwd(q, k, v, o, lse, dO, dq, dk, (float*)mis, 2, 100, 4, 2, 64, 0.125f, 1, ws, WS,
                   nullptr), XATTN_ERR_ALIGN, 0);
  EXPECT(xattn_bwd(q, k, v, nullptr, lse, dO, dq, dk, dv, 2, 100, 4, 2, 64, 0.125f, 1, ws, WS,
                   nullptr), XATTN_ERR_NULL, 0);
  EXPECT(xattn_bwd(q, k, v, o, lse, dO, dq, dk, nullptr, 2, 100, 4, 2, 64, 0.125f, 1, ws, WS,
                   nullptr), XATTN_ERR_NULL, 0);
  EXPECT(xattn_bwd(q, k, v, o, lse, dO, dq, dk, dv, 2, 100, 4, 2, 64, 0.125f, 9, ws, WS, nullptr),
         XATTN_ERR_DTYPE, 0);
  EXPECT(xattn_bwd(q, k, v, o, lse, dO, dq, dk, dv, 2, 100, 6, 4, 64, 0.125f, 1, ws, WS, nullptr),
         XATTN_ERR_GQA, 0);
  // fp32 dq tiles are 64 rows: 65536 * 256 * 2 dq workgroups for S = 128, too many,
  // while the bf16 backward of the same shape fits (a short sequence: one kernel)
  EXPECT(xattn_bwd(q, k, v, o, lse, dO, dq, dk, dv, 65536, 128, 256, 256, 16, 0.25f, XATTN_F32, ws,
                   WS, nullptr), XATTN_ERR_SHAPE, 0);
  EXPECT(xattn_bwd(q, k, v, o, lse, dO, dq, dk, dv, 32768, 128, 256, 256, 16, 0.25f, XATTN_BF16, ws,
                   WS, nullptr), XATTN_OK, 1);
  EXPECT(xattn_bwd(q, k, v, o, lse, dO, dq, dk, dv, 65536, 128, 256, 256, 16, 0.25f, XATTN_BF16, ws,
                   WS, nullptr), XATTN_ERR_SHAPE, 0);
  g_fail = true;
  EXPECT(xattn_bwd(q, k, v, o, lse, dO, dq, dk, dv, 2, 100, 4, 2, 64, 0.125f, 1, ws, WS, nullptr),
         XATTN_ERR_HIP, 1);
  EXPECT(xattn_bwd_dq(q, k, v, o, lse, dO, dq, 2, 100, 4, 2, 64, 0.125f, 1, ws, need, nullptr),
         XATTN_OK, 1);
  EXPECT(xattn_bwd_dkdv(q, k, v, lse, dO, dk, dv, 2, 100, 4, 2, 64, 0.125f, 1, ws, need, nullptr),
         XATTN_OK, 1);
  EXPECT(xattn_bwd_dkdv(q, k, v, lse, dO, dk, dv, 2, 100, 4, 2, 64, 0.125f, 1, ws, need - 4,
                        nullptr), XATTN_ERR_WORKSPACE, 0);
  EXPECT(xattn_bwd_dq(q, k, v, o, lse, nullptr, dq, 2, 100, 4, 2, 64, 0.125f, 1, ws, need, nullptr),
         XATTN_ERR_NULL, 0);

  // --- short bf16 MHA sequences: one launch, the same checks
  EXPECT(xattn_bwd(q, k, v, o, lse, dO, dq, dk, dv, 2, 100, 4, 4, 32, 0.125f, 1, ws, WS, nullptr),
         XATTN_OK, 1);
  EXPECT(xattn_bwd(q, k, v, o, lse, dO, dq, dk, dv, 2, 256, 4, 4, 16, 0.125f, 1, ws, WS, nullptr),
         XATTN_OK, 1);
  EXPECT(xattn_bwd(q, k, v, o, lse, dO, dq, dk, dv, 2, 257, 4, 4, 16, 0.125f, 1, ws, WS, nullptr),
         XATTN_OK, 2);
  EXPECT(xattn_bwd(q, k, v, o, lse, dO, dq, dk, dv, 2, 100, 4, 4, 32, 0.125f, 0, ws, WS, nullptr),
         XATTN_OK, 2);
  EXPECT(xattn_bwd(mis, k, v, o, lse, dO, dq, dk, dv, 2, 100, 4, 4, 32, 0.125f, 1, ws, WS, nullptr),
         XATTN_ERR_ALIGN, 0);
  EXPECT(xattn_bwd(q, k, v, o, lse, dO, (float*)mis, dk, dv, 2, 100, 4, 4, 32, 0.125f, 1, ws, WS,
                   nullptr), XATTN_ERR_ALIGN, 0);
  EXPECT(xattn_bwd(q, k, v, o, lse, dO, dq, dk, dv, 2, 100, 4, 4, 32, 0.125f, 1, ws, 8 * 2 * 4 * 100 - 1,
                   nullptr), XATTN_ERR_WORKSPACE, 0);
  EXPECT(xattn_bwd_ragged(q, k, v, o, lse, dO, lens, dq, dk, dv, 2, 100, 4, 4, 32, 0.125f, 1, ws,
                          WS, nullptr), XATTN_OK, 1);
  EXPECT(xattn_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, 2, 100, 4, 4, 32, 0.125f, 1, nullptr),
         XATTN_OK, 1);
  g_fail = true;
  EXPECT(xattn_bwd(q, k, v, o, lse, dO, dq, dk, dv, 2, 100, 4, 4, 32, 0.125f, 1, ws, WS, nullptr),
         XATTN_ERR_HIP, 1);
  {
    const int c[] = {xattn_bwd_kernel_count(2, 100, 4, 4, 32, 1), xattn_bwd_kernel_count(2, 100, 4, 2, 64, 1),
                     xattn_bwd_kernel_count(16, 1024, 8, 2, 64, 1), xattn_bwd_kernel_count(1, 16, 3, 2, 16, 1)};
    if (c[0] != 1 || c[1] != 3 || c[2] != 3 || c[3] != 0) {
      std::printf("FAIL kernel counts %d %d %d %d\n", c[0], c[1], c[2], c[3]);
      ++g_failures;
    }
    g_checks += 4;
  }

  // --- allocation-free backward: same checks, plus the fixed scratch's limit
  EXPECT(xattn_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, 2, 100, 4, 2, 64, 0.125f, 1, nullptr),
         XATTN_OK, 2);
  EXPECT(xattn_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, 16, 1024, 8, 2, 64, 0.125f, 0, nullptr),
         XATTN_OK, 2);
  // 8 * B * H * S = 16 MiB exactly, then one query row more per head
  EXPECT(xattn_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, 1, 131072, 16, 16, 64, 0.125f, 1,
                           nullptr), XATTN_OK, 2);
  EXPECT(xattn_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, 1, 131073, 16, 16, 64, 0.125f, 1,
                           nullptr), XATTN_ERR_SCRATCH, 0);
  EXPECT(xattn_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, nullptr, 2, 100, 4, 2, 64, 0.125f, 1,
                           nullptr), XATTN_ERR_NULL, 0);
  EXPECT(xattn_bwd_noalloc(q, k, v, o, lse, dO, dq, (float*)mis, dv, 2, 100, 4, 2, 64, 0.125f, 1,
                           nullptr), XATTN_ERR_ALIGN, 0);
  EXPECT(xattn_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, 2, 100, 4, 2, 64, 0.125f, 5, nullptr),
         XATTN_ERR_DTYPE, 0);
  EXPECT(xattn_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, 2, 100, 4, 2, 64, nan, 1, nullptr),
         XATTN_ERR_SCALE, 0);
  g_no_scratch = true;
  EXPECT(xattn_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, 2, 100, 4, 2, 64, 0.125f, 1, nullptr),
         XATTN_ERR_HIP, 0);
  g_no_scratch = false;
  g_fail = true;
  EXPECT(xattn_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, 2, 100, 4, 2, 64, 0.125f, 1, nullptr),
         XATTN_ERR_HIP, 1);

  // --- QK-norm + RoPE
  const float* w = f[12];
  const size_t nws = xattn_qknorm_rope_bwd_workspace_bytes(2, 64, 4, 64);
  EXPECT(xattn_qknorm_rope_fwd(q, w, o, 2, 64, 4, 64, 1e-6f, 10000.f, 1, nullptr), XATTN_OK, 1);
  EXPECT(xattn_qknorm_rope_fwd(q, w, o, 2, 64, 4, 64, -1e-6f, 10000.f, 1, nullptr), XATTN_ERR_PARAM,
         0);
  EXPECT(xattn_qknorm_rope_fwd(q, w, o, 2, 64, 4, 64, nan, 10000.f, 1, nullptr), XATTN_ERR_PARAM, 0);
  EXPECT(xattn_qknorm_rope_fwd(q, w, o, 2, 64, 4, 64, 1e-6f, 1.f, 1, nullptr), XATTN_ERR_PARAM, 0);
  EXPECT(xattn_qknorm_rope_fwd(q, w, o, 2, 64, 4, 64, 1e-6f, inf, 1, nullptr), XATTN_ERR_PARAM, 0);
  EXPECT(xattn_qknorm_rope_fwd(q, w, o, 2, 64, 4, 8, 1e-6f, 10000.f, 1, nullptr),
         XATTN_ERR_HEAD_DIM, 0);
  EXPECT(xattn_qknorm_rope_fwd(q, w, o, 2, 64, 4, 64, 1e-6f, 10000.f, 3, nullptr), XATTN_ERR_DTYPE,
         0);
  EXPECT(xattn_qknorm_rope_fwd(q, nullptr, o, 2, 64, 4, 64, 1e-6f, 10000.f, 1, nullptr),
         XATTN_ERR_NULL, 0);
  EXPECT(xattn_qknorm_rope_fwd(q, w, o, 2, 0, 4, 64, 1e-6f, 10000.f, 1, nullptr), XATTN_ERR_SHAPE, 0);
  EXPECT(xattn_qknorm_rope_fwd(mis, w, o, 2, 64, 4, 64, 1e-6f, 10000.f, 1, nullptr),
         XATTN_ERR_ALIGN, 0);
  EXPECT(xattn_qknorm_rope_bwd(q, w, f[13], dq, f[14], 2, 64, 4, 64, 1e-6f, 10000.f, 1, ws, nws,
                               nullptr), XATTN_OK, 1);
  EXPECT(xattn_qknorm_rope_bwd(q, w, f[13], dq, f[14], 2, 64, 4, 64, 1e-6f, 10000.f, 1, ws, nws - 1,
                               nullptr), XATTN_ERR_WORKSPACE, 0);
  EXPECT(xattn_qknorm_rope_bwd(q, w, f[13], dq, nullptr, 2, 64, 4, 64, 1e-6f, 10000.f, 1, ws, nws,
                               nullptr), XATTN_ERR_NULL, 0);
  if (xattn_qknorm_rope_bwd_workspace_bytes(2, 64, 4, 24) != 0) {
    std::printf("FAIL qknorm ws for invalid hd\n");
    ++g_failures;
  }

  // --- decode
  const size_t dws = xattn_decode_workspace_bytes(8, 32768, 16, 4, 64);
  if (dws == 0) { std::printf("FAIL decode ws size\n"); ++g_failures; }
  EXPECT(xattn_decode(q, k, v, lens, o, lse, 8, 32768, 16, 4, 64, 0.125f, 1, ws, dws, nullptr),
         XATTN_OK, 1);
  EXPECT(xattn_decode(q, k, v, nullptr, o, lse, 8, 32768, 16, 4, 64, 0.125f, 1, ws, dws, nullptr),
         XATTN_OK, 1);
  EXPECT(xattn_decode(q, k, v, lens, o, lse, 8, 32768, 16, 4, 64, 0.125f, 1, ws, dws - 1, nullptr),
         XATTN_ERR_WORKSPACE, 0);
  EXPECT(xattn_decode(q, k, v, lens, o, lse, 8, 32768, 16, 4, 64, 0.125f, 1, nullptr, dws, nullptr),
         XATTN_ERR_WORKSPACE, 0);
  EXPECT(xattn_decode(q, k, v, lens, o, lse, 1, (4 << 20) + 1, 1, 1, 64, 0.125f, 1, ws, WS, nullptr),
         XATTN_ERR_SHAPE, 0);
  EXPECT(xattn_decode(q, k, v, reinterpret_cast<const int*>(g_mem[10] + 1), o, lse, 8, 32768, 16, 4,
                      64, 0.125f, 1, ws, dws, nullptr), XATTN_ERR_ALIGN, 0);
  EXPECT(xattn_decode(q, k, v, lens, o, lse, 8, 32768, 16, 5, 64, 0.125f, 1, ws, dws, nullptr),
         XATTN_ERR_GQA, 0);
  EXPECT(xattn_decode(q, k, v, lens, o, lse, 8, 32768, 16, 4, 64, -1.f, 1, ws, dws, nullptr),
         XATTN_ERR_SCALE, 0);
  // a short cache needs no workspace
  if (xattn_decode_workspace_bytes(1, 100, 2, 2, 64) != 0) {
    std::printf("FAIL decode ws for one chunk\n");
    ++g_failures;
  }
  EXPECT(xattn_decode(q, k, v, nullptr, o, lse, 1, 100, 2, 2, 64, 0.125f, 0, nullptr, 0, nullptr),
         XATTN_OK, 1);

  // --- composed path
  const size_t pb = xattn_composed_buffer_bytes(2, 100, 4);
  if (pb != 4ull * 2 * 4 * 100 * 100) { std::printf("FAIL composed bytes %zu\n", pb); ++g_failures; }
  EXPECT(xattn_composed_fwd(q, k, v, o, lse, f[12], pb, 2, 100, 4, 2, 64, 0.125f, 1, nullptr),
         XATTN_OK, 1);
  EXPECT(xattn_composed_fwd(q, k, v, o, lse, f[12], pb - 1, 2, 100, 4, 2, 64, 0.125f, 1, nullptr),
         XATTN_ERR_WORKSPACE, 0);
  EXPECT(xattn_composed_bwd(q, k, v, f[12], pb, dO, dq, dk, dv, f[13], pb, 2, 100, 4, 2, 64, 0.125f,
                            1, nullptr), XATTN_OK, 1);
  EXPECT(xattn_composed_bwd(q, k, v, f[12], pb, dO, dq, dk, dv, f[13], pb - 1, 2, 100, 4, 2, 64,
                            0.125f, 1, nullptr), XATTN_ERR_WORKSPACE, 0);
  EXPECT(xattn_composed_bwd(q, k, v, f[12], pb, dO, dq, dk, dv, nullptr, pb, 2, 100, 4, 2, 64,
                            0.125f, 1, nullptr), XATTN_ERR_NULL, 0);

  // --- status text: never NULL, distinct for the defined codes
  const char* seen[12] = {};
  for (int s = -2; s <= 12; ++s) {
    const char* t = xattn_strerror(s);
    if (!t || !*t) { std::printf("FAIL strerror(%d)\n", s); ++g_failures; }
    if (s >= 0 && s <= 11) {
      for (int u = 0; u < s; ++u)
        if (std::strcmp(seen[u], t) == 0) { std::printf("FAIL strerror dup %d\n", s); ++g_failures; }
      seen[s] = t;
    }
  }
  std::printf("checks=%d failures=%d\n", g_checks, g_failures);
  return g_failures != 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the HIP headers")
def test_c_abi_validation_clean_under_asan_and_ubsan(tmp_path):
    drv = tmp_path / "driver.cpp"
    drv.write_text(DRIVER)
    exe = tmp_path / "driver"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I", ROCM_INCLUDE, "-I", INCLUDE, "-I", CSRC, str(drv),
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "failures=0" in r.stdout, r.stdout
