// api.cpp -- the C ABI of libxattn.so (declared in include/xattn.h).
//
// Every argument is checked here, on the host, before any HIP call, including
// the grid of every launch the call would make (sized by plan.cpp, as the
// launchers size them); only a fully valid call enqueues kernels.  The library
// holds no state: no handles, no allocations, no synchronisation.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <limits>

#include "launch.hpp"
#include "xattn.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// dtype must already be valid.
int check_shape(int B, int S, int H, int Hkv, int hd, int dtype) {
  if (B <= 0 || S <= 0 || H <= 0 || Hkv <= 0 || hd <= 0) return XATTN_ERR_SHAPE;
  if (H % Hkv != 0) return XATTN_ERR_GQA;
  if (hd != 16 && hd != 32 && hd != 64) return XATTN_ERR_HEAD_DIM;
  const int64_t plane = (int64_t)S * hd;  // elements of one (batch, head) plane
  if (plane > std::numeric_limits<int32_t>::max()) return XATTN_ERR_SHAPE;
  if ((int64_t)B * H * S > std::numeric_limits<int64_t>::max() / 8) return XATTN_ERR_SHAPE;
  // every launch of the forward and backward fits one HIP grid
  const xattn::AttnPlan p = xattn::attn_plan(xattn::Dims{B, S, H, Hkv, hd}, dtype);
  for (const long long n : {p.fwd_blocks, p.dq_blocks, p.dkdv_blocks, p.dkdv_sum_blocks})
    if (n > xattn::kMaxBlocks) return XATTN_ERR_SHAPE;
  return XATTN_OK;
}

int check_common(int B, int S, int H, int Hkv, int hd, float scale, int dtype) {
  if (dtype != XATTN_F32 && dtype != XATTN_BF16) return XATTN_ERR_DTYPE;
  const int rc = check_shape(B, S, H, Hkv, hd, dtype);
  if (rc != XATTN_OK) return rc;
  if (!std::isfinite(scale) || !(scale > 0.f)) return XATTN_ERR_SCALE;
  return XATTN_OK;
}

int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? XATTN_OK : XATTN_ERR_HIP;
}

}  // namespace

namespace {

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int fwd_impl(const void* q, const void* k, const void* v, const int* lens, void* o, float* lse,
             int B, int S, int H, int Hkv, int hd, float scale, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return XATTN_ERR_NULL;
  int rc = check_common(B, S, H, Hkv, hd, scale, dtype);
  if (rc != XATTN_OK) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned4(lens))
    return XATTN_ERR_ALIGN;
  xattn::launch_fwd(dtype, xattn::Dims{B, S, H, Hkv, hd}, q, k, v, o, lse, lens, scale,
                    static_cast<hipStream_t>(stream));
  return launch_status();
}

int check_bwd_common(int B, int S, int H, int Hkv, int hd, float scale, int dtype,
                     const void* workspace, size_t workspace_bytes);

int bwd_dq_impl(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dO, const int* lens, float* dq, int B, int S, int H, int Hkv, int hd,
                float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse || !dO || !dq) return XATTN_ERR_NULL;
  const int rc = check_bwd_common(B, S, H, Hkv, hd, scale, dtype, workspace, workspace_bytes);
  if (rc != XATTN_OK) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(dO) || !aligned16(dq) || !aligned16(workspace) || !aligned4(lens))
    return XATTN_ERR_ALIGN;
  xattn::launch_bwd_dq(dtype, xattn::Dims{B, S, H, Hkv, hd}, q, k, v, o, lse, dO, dq,
                       static_cast<float*>(workspace), lens, scale,
                       static_cast<hipStream_t>(stream));
  return launch_status();
}

int bwd_dkdv_impl(const void* q, const void* k, const void* v, const float* lse, const void* dO,
                  const int* lens, float* dk, float* dv, int B, int S, int H, int Hkv, int hd,
                  float scale, int dtype, void* workspace, size_t workspace_bytes,
                  void* stream) {
  if (!q || !k || !v || !lse || !dO || !dk || !dv) return XATTN_ERR_NULL;
  const int rc = check_bwd_common(B, S, H, Hkv, hd, scale, dtype, workspace, workspace_bytes);
  if (rc != XATTN_OK) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(lse) || !aligned16(dO) ||
      !aligned16(dk) || !aligned16(dv) || !aligned16(workspace) || !aligned4(lens))
    return XATTN_ERR_ALIGN;
  xattn::launch_bwd_dkdv(dtype, xattn::Dims{B, S, H, Hkv, hd}, q, k, v, lse, dO,
                         static_cast<float*>(workspace), dk, dv, lens, scale,
                         /*split_groups=*/true, static_cast<hipStream_t>(stream));
  return launch_status();
}

int bwd_impl(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dO, const int* lens, float* dq, float* dk, float* dv, int B, int S, int H,
             int Hkv, int hd, float scale, int dtype, void* workspace, size_t workspace_bytes,
             void* stream) {
  // Validate everything up front so that an invalid call enqueues nothing.
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return XATTN_ERR_NULL;
  int rc = check_bwd_common(B, S, H, Hkv, hd, scale, dtype, workspace, workspace_bytes);
  if (rc != XATTN_OK) return rc;
  if (!aligned16(dk) || !aligned16(dv)) return XATTN_ERR_ALIGN;
  const xattn::Dims d{B, S, H, Hkv, hd};
  if (xattn::bwd_short_path(d, dtype)) {
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
        !aligned16(dO) || !aligned16(dq) || !aligned16(workspace) || !aligned4(lens))
      return XATTN_ERR_ALIGN;
    xattn::launch_bwd_short(d, q, k, v, o, lse, dO, dq, dk, dv, lens, scale,
                            static_cast<hipStream_t>(stream));
    return launch_status();
  }
  rc = bwd_dq_impl(q, k, v, o, lse, dO, lens, dq, B, S, H, Hkv, hd, scale, dtype, workspace,
                   workspace_bytes, stream);
  if (rc != XATTN_OK) return rc;
  return bwd_dkdv_impl(q, k, v, lse, dO, lens, dk, dv, B, S, H, Hkv, hd, scale, dtype, workspace,
                       workspace_bytes, stream);
}

}  // namespace

extern "C" {

int xattn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int S,
              int H, int Hkv, int hd, float scale, int dtype, void* stream) {
  return fwd_impl(q, k, v, nullptr, o, lse, B, S, H, Hkv, hd, scale, dtype, stream);
}

size_t xattn_bwd_workspace_bytes(int B, int S, int H, int Hkv, int hd, int dtype) {
  if (dtype != XATTN_F32 && dtype != XATTN_BF16) return 0;
  if (check_shape(B, S, H, Hkv, hd, dtype) != XATTN_OK) return 0;
  // D and LSE*log2e per query row, plus the partial dk, dv of a group split
  // over workgroups
  return xattn::attn_plan(xattn::Dims{B, S, H, Hkv, hd}, dtype).workspace_bytes;
}

int xattn_bwd_kernel_count(int B, int S, int H, int Hkv, int hd, int dtype) {
  if (dtype != XATTN_F32 && dtype != XATTN_BF16) return 0;
  if (check_shape(B, S, H, Hkv, hd, dtype) != XATTN_OK) return 0;
  const xattn::Dims d{B, S, H, Hkv, hd};
  if (xattn::bwd_short_path(d, dtype)) return 1;
  return xattn::attn_plan(d, dtype).split > 1 ? 3 : 2;
}

int xattn_bwd_dq(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dO, float* dq, int B, int S, int H, int Hkv, int hd, float scale,
                 int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_dq_impl(q, k, v, o, lse, dO, nullptr, dq, B, S, H, Hkv, hd, scale, dtype, workspace,
                     workspace_bytes, stream);
}

int xattn_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                   const void* dO, float* dk, float* dv, int B, int S, int H, int Hkv, int hd,
                   float scale, int dtype, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return bwd_dkdv_impl(q, k, v, lse, dO, nullptr, dk, dv, B, S, H, Hkv, hd, scale, dtype,
                       workspace, workspace_bytes, stream);
}

int xattn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dO, float* dq, float* dk, float* dv, int B, int S, int H, int Hkv,
              int hd, float scale, int dtype, void* workspace, size_t workspace_bytes,
              void* stream) {
  return bwd_impl(q, k, v, o, lse, dO, nullptr, dq, dk, dv, B, S, H, Hkv, hd, scale, dtype,
                  workspace, workspace_bytes, stream);
}

int xattn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dO, float* dq, float* dk, float* dv, int B, int S, int H,
                      int Hkv, int hd, float scale, int dtype, void* stream) {
  // the checks of xattn_bwd, all before anything is enqueued
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return XATTN_ERR_NULL;
  const int rc = check_common(B, S, H, Hkv, hd, scale, dtype);
  if (rc != XATTN_OK) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(dO) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return XATTN_ERR_ALIGN;
  // GQA groups stay whole (no partial dk, dv planes): the per-row part only
  const xattn::Dims d{B, S, H, Hkv, hd};
  if (xattn::attn_plan(d, dtype, /*split_groups=*/false).workspace_bytes >
      xattn::kNoAllocScratchBytes)
    return XATTN_ERR_SCRATCH;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (xattn::bwd_short_path(d, dtype)) {  // needs no scratch
    xattn::launch_bwd_short(d, q, k, v, o, lse, dO, dq, dk, dv, nullptr, scale, st);
    return launch_status();
  }
  float* ws = xattn::noalloc_scratch();
  if (!ws) return XATTN_ERR_HIP;
  xattn::launch_bwd_dq(dtype, d, q, k, v, o, lse, dO, dq, ws, nullptr, scale, st);
  int s2 = launch_status();
  if (s2 != XATTN_OK) return s2;
  xattn::launch_bwd_dkdv(dtype, d, q, k, v, lse, dO, ws, dk, dv, nullptr, scale,
                         /*split_groups=*/false, st);
  return launch_status();
}

int xattn_fwd_ragged(const void* q, const void* k, const void* v, const int* lens, void* o,
                     float* lse, int B, int S, int H, int Hkv, int hd, float scale, int dtype,
                     void* stream) {
  if (!lens) return XATTN_ERR_NULL;
  return fwd_impl(q, k, v, lens, o, lse, B, S, H, Hkv, hd, scale, dtype, stream);
}

int xattn_bwd_ragged(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dO, const int* lens, float* dq, float* dk, float* dv, int B,
                     int S, int H, int Hkv, int hd, float scale, int dtype, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!lens) return XATTN_ERR_NULL;
  return bwd_impl(q, k, v, o, lse, dO, lens, dq, dk, dv, B, S, H, Hkv, hd, scale, dtype,
                  workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {
int check_bwd_common(int B, int S, int H, int Hkv, int hd, float scale, int dtype,
                     const void* workspace, size_t workspace_bytes) {
  const int rc = check_common(B, S, H, Hkv, hd, scale, dtype);
  if (rc != XATTN_OK) return rc;
  if (!workspace || workspace_bytes < xattn_bwd_workspace_bytes(B, S, H, Hkv, hd, dtype))
    return XATTN_ERR_WORKSPACE;
  return XATTN_OK;
}
}  // namespace

namespace {
int check_norm(int B, int S, int H, int hd, float eps, float base, int dtype) {
  if (dtype != XATTN_F32 && dtype != XATTN_BF16) return XATTN_ERR_DTYPE;
  if (B <= 0 || S <= 0 || H <= 0 || hd <= 0) return XATTN_ERR_SHAPE;
  if (hd != 16 && hd != 32 && hd != 64) return XATTN_ERR_HEAD_DIM;
  if ((int64_t)B * S * H * hd > std::numeric_limits<int32_t>::max()) return XATTN_ERR_SHAPE;
  if (!std::isfinite(eps) || eps < 0.f || !std::isfinite(base) || !(base > 1.f))
    return XATTN_ERR_PARAM;
  return XATTN_OK;
}
}  // namespace

extern "C" {

int xattn_qknorm_rope_fwd(const void* x, const float* w, void* out, int B, int S, int H, int hd,
                          float eps, float rope_base, int dtype, void* stream) {
  if (!x || !w || !out) return XATTN_ERR_NULL;
  const int rc = check_norm(B, S, H, hd, eps, rope_base, dtype);
  if (rc != XATTN_OK) return rc;
  if (!aligned16(x) || !aligned16(w) || !aligned16(out)) return XATTN_ERR_ALIGN;
  xattn::launch_qknorm_rope_fwd(dtype, xattn::NormDims{B, S, H, hd}, x, w, out, eps, rope_base,
                                static_cast<hipStream_t>(stream));
  return launch_status();
}

size_t xattn_qknorm_rope_bwd_workspace_bytes(int B, int S, int H, int hd) {
  if (check_norm(B, S, H, hd, 0.f, 10000.f, XATTN_F32) != XATTN_OK) return 0;
  return sizeof(float) * (size_t)hd *
         (size_t)xattn::qknorm_bwd_blocks((long)B * S * H, hd);
}

int xattn_qknorm_rope_bwd(const void* x, const float* w, const float* dout, float* dx, float* dw,
                          int B, int S, int H, int hd, float eps, float rope_base, int dtype,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !w || !dout || !dx || !dw) return XATTN_ERR_NULL;
  const int rc = check_norm(B, S, H, hd, eps, rope_base, dtype);
  if (rc != XATTN_OK) return rc;
  if (!workspace || workspace_bytes < xattn_qknorm_rope_bwd_workspace_bytes(B, S, H, hd))
    return XATTN_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(w) || !aligned16(dout) || !aligned16(dx) || !aligned16(dw) ||
      !aligned16(workspace))
    return XATTN_ERR_ALIGN;
  xattn::launch_qknorm_rope_bwd(dtype, xattn::NormDims{B, S, H, hd}, x, w, dout, dx, dw,
                                static_cast<float*>(workspace), eps, rope_base,
                                static_cast<hipStream_t>(stream));
  return launch_status();
}

namespace {
int check_decode(int B, int T, int H, int Hkv, int hd, float scale, int dtype) {
  if (dtype != XATTN_F32 && dtype != XATTN_BF16) return XATTN_ERR_DTYPE;
  if (B <= 0 || T <= 0 || H <= 0 || Hkv <= 0 || hd <= 0) return XATTN_ERR_SHAPE;
  if (H % Hkv != 0) return XATTN_ERR_GQA;
  if (hd != 16 && hd != 32 && hd != 64) return XATTN_ERR_HEAD_DIM;
  if ((int64_t)T * hd > std::numeric_limits<int32_t>::max()) return XATTN_ERR_SHAPE;
  if (T > xattn::kDecodeMaxT) return XATTN_ERR_SHAPE;
  if ((int64_t)B * H * hd > std::numeric_limits<int32_t>::max()) return XATTN_ERR_SHAPE;
  const xattn::DecodePlan p = xattn::decode_plan(B, T, H, Hkv, hd);
  if (p.blocks > xattn::kMaxBlocks || p.combine_blocks > xattn::kMaxBlocks) return XATTN_ERR_SHAPE;
  if (!std::isfinite(scale) || !(scale > 0.f)) return XATTN_ERR_SCALE;
  return XATTN_OK;
}
}  // namespace

size_t xattn_decode_workspace_bytes(int B, int T, int H, int Hkv, int hd) {
  if (check_decode(B, T, H, Hkv, hd, 1.f, XATTN_F32) != XATTN_OK) return 0;
  return xattn::decode_plan(B, T, H, Hkv, hd).part_bytes;
}

int xattn_decode(const void* q, const void* k, const void* v, const int* lens, void* o,
                 float* lse, int B, int T, int H, int Hkv, int hd, float scale, int dtype,
                 void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse) return XATTN_ERR_NULL;
  const int rc = check_decode(B, T, H, Hkv, hd, scale, dtype);
  if (rc != XATTN_OK) return rc;
  const size_t need = xattn::decode_plan(B, T, H, Hkv, hd).part_bytes;
  if (need > 0 && (!workspace || workspace_bytes < need)) return XATTN_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      (need > 0 && !aligned16(workspace)) || (reinterpret_cast<uintptr_t>(lens) & 3u) != 0)
    return XATTN_ERR_ALIGN;
  xattn::launch_decode(dtype, xattn::Dims{B, T, H, Hkv, hd}, q, k, v, lens, o, lse,
                       static_cast<float*>(workspace), scale, static_cast<hipStream_t>(stream));
  return launch_status();
}

size_t xattn_composed_buffer_bytes(int B, int S, int H) {
  if (B <= 0 || S <= 0 || H <= 0) return 0;
  return sizeof(float) * (size_t)B * (size_t)H * (size_t)S * (size_t)S;
}

int xattn_composed_fwd(const void* q, const void* k, const void* v, void* o, float* lse, float* p,
                       size_t p_bytes, int B, int S, int H, int Hkv, int hd, float scale,
                       int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse || !p) return XATTN_ERR_NULL;
  const int rc = check_common(B, S, H, Hkv, hd, scale, dtype);
  if (rc != XATTN_OK) return rc;
  if (xattn::composed_max_blocks(xattn::Dims{B, S, H, Hkv, hd}) > xattn::kMaxBlocks)
    return XATTN_ERR_SHAPE;
  if (p_bytes < xattn_composed_buffer_bytes(B, S, H)) return XATTN_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(p))
    return XATTN_ERR_ALIGN;
  xattn::launch_composed_fwd(dtype, xattn::Dims{B, S, H, Hkv, hd}, q, k, v, o, lse, p, scale,
                             static_cast<hipStream_t>(stream));
  return launch_status();
}

int xattn_composed_bwd(const void* q, const void* k, const void* v, const float* p,
                       size_t p_bytes, const void* dO, float* dq, float* dk, float* dv, float* ds,
                       size_t ds_bytes, int B, int S, int H, int Hkv, int hd, float scale,
                       int dtype, void* stream) {
  if (!q || !k || !v || !p || !dO || !dq || !dk || !dv || !ds) return XATTN_ERR_NULL;
  const int rc = check_common(B, S, H, Hkv, hd, scale, dtype);
  if (rc != XATTN_OK) return rc;
  if (xattn::composed_max_blocks(xattn::Dims{B, S, H, Hkv, hd}) > xattn::kMaxBlocks)
    return XATTN_ERR_SHAPE;
  const size_t need = xattn_composed_buffer_bytes(B, S, H);
  if (p_bytes < need || ds_bytes < need) return XATTN_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(p) || !aligned16(dO) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(ds))
    return XATTN_ERR_ALIGN;
  xattn::launch_composed_bwd(dtype, xattn::Dims{B, S, H, Hkv, hd}, q, k, v, p, dO, dq, dk, dv, ds,
                             scale, static_cast<hipStream_t>(stream));
  return launch_status();
}

const char* xattn_strerror(int status) {
  switch (status) {
    case XATTN_OK: return "success";
    case XATTN_ERR_NULL: return "a required pointer is NULL";
    case XATTN_ERR_SHAPE: return "invalid shape: B, S, H, Hkv and hd must be positive and within size limits";
    case XATTN_ERR_GQA: return "H must be a multiple of Hkv";
    case XATTN_ERR_HEAD_DIM: return "head dimension must be 16, 32 or 64";
    case XATTN_ERR_DTYPE: return "dtype must be XATTN_F32 or XATTN_BF16";
    case XATTN_ERR_WORKSPACE: return "workspace is NULL or smaller than the required size";
    case XATTN_ERR_SCALE: return "scale must be positive and finite";
    case XATTN_ERR_HIP: return "the HIP runtime rejected a kernel launch";
    case XATTN_ERR_ALIGN: return "a data pointer is not 16-byte aligned";
    case XATTN_ERR_PARAM: return "eps must be finite and >= 0, and the rope base finite and > 1";
    case XATTN_ERR_SCRATCH:
      return "shape too large for the fixed scratch of xattn_bwd_noalloc (8*B*H*S bytes above 16 MiB)";
    default: return "unknown xattn status";
  }
}

}  // extern "C"
