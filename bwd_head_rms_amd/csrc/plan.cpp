// plan.cpp -- launch sizing of every kernel family, host code only.
//
// The launchers size their grids from these functions and the C ABI checks
// the same numbers before it enqueues anything, so a shape that some launch
// could not take is rejected up front and no call enqueues part of its work.
// Nothing here touches the HIP runtime.
#include "launch.hpp"

namespace xattn {

namespace {

long long cdiv(long long a, long long b) { return (a + b - 1) / b; }

// Query heads of a GQA group that one decode workgroup serves.
int heads_per_wg(int group) {
  for (int gc = 8; gc > 1; gc /= 2)
    if (group % gc == 0) return gc;
  return 1;
}

// dk/dv: below this many key tiles a GQA group is split over workgroups.
constexpr long kDkvSplitBelow = 512;
// Workgroups a split aims for.  Each slice adds a partial dK, dV plane to
// write and re-read; the fp32 kernel spends longer per tile, so it gains from
// more slices than bf16 loses to the extra traffic.
constexpr long kDkvSplitTargetF32 = 1024, kDkvSplitTargetBf16 = 512;

}  // namespace

int dkdv_split(const Dims& d, int dtype) {
  const int group = d.H / d.Hkv;
  const long tiles = (long)d.B * d.Hkv * cdiv(d.S, dkdv_tile_keys(dtype, d.hd));
  if (group == 1 || tiles >= kDkvSplitBelow) return 1;
  // fewer workgroups than two per CU: split each group into the fewest slices
  // (a divisor of the group) that reach the target
  const long target = dtype == 0 ? kDkvSplitTargetF32 : kDkvSplitTargetBf16;
  int R = 1;
  while (R < group && tiles * R < target) {
    do { ++R; } while (group % R != 0);
  }
  return R;
}

bool bwd_short_path(const Dims& d, int dtype) {
  return dtype == 1 && d.hd <= 32 && d.S <= kShortMaxS && d.H == d.Hkv;
}

ShortSplit short_split(const Dims& d, int ncu) {
  const long long BH = (long long)d.B * d.H;
  long long split = ncu > 0 ? 2LL * ncu - BH : 0;
  split = split < 0 ? 0 : (split > BH ? BH : split);
  return ShortSplit{BH - split, BH + split};
}

size_t dkdv_part_offset(const Dims& d) {
  return (2 * (size_t)d.B * d.H * d.S + 3) / 4 * 4;  // floats, keeps 16-byte alignment
}

AttnPlan attn_plan(const Dims& d, int dtype, bool split_groups) {
  AttnPlan p;
  const long long BH = (long long)d.B * d.H, BG = (long long)d.B * d.Hkv;
  p.fwd_blocks = cdiv(d.S, fwd_tile_rows(dtype, d.hd)) * BH;
  p.dq_blocks = cdiv(d.S, dq_tile_rows(dtype, d.hd)) * BH;
  p.split = split_groups ? dkdv_split(d, dtype) : 1;
  p.dkdv_blocks = cdiv(d.S, dkdv_tile_keys(dtype, d.hd)) * BG * p.split;
  // the partial-sum kernel: 4 floats per thread over dk and dv
  p.dkdv_sum_blocks = p.split > 1 ? cdiv(2 * (BG * d.S * d.hd / 4), kThreads) : 0;
  p.workspace_bytes = p.split == 1
                          ? 2 * sizeof(float) * (size_t)BH * (size_t)d.S  // D and LSE*log2e
                          : sizeof(float) * (dkdv_part_offset(d) +
                                             2 * (size_t)p.split * (size_t)BG * (size_t)d.S *
                                                 (size_t)d.hd);
  return p;
}

DecodePlan decode_plan(int B, int T, int H, int Hkv, int hd) {
  const int group = H / Hkv;
  DecodePlan p;
  p.heads_per_wg = heads_per_wg(group);
  const long units = (long)B * Hkv * (group / p.heads_per_wg);
  int chunk = kDecMinChunk;
  // about four workgroups per CU (one resident wave of them), chunks as short as that allows
  while (chunk < kDecMaxChunk && units * ((T + chunk - 1) / chunk) > 1024) chunk *= 2;
  p.chunk = chunk;
  p.nsplit = (T + chunk - 1) / chunk;
  p.blocks = p.nsplit * units;
  p.combine_blocks = p.nsplit > 1 ? (long)B * H : 0;
  p.part_bytes = p.nsplit > 1 ? sizeof(float) * (size_t)B * H * p.nsplit * (hd + 2) : 0;
  return p;
}

int qknorm_bwd_blocks(long nvec, int hd) {
  const long threads = nvec * (hd / 8);
  const long blocks = (threads + 255) / 256;
  return (int)(blocks < kNormMaxBlocks ? blocks : kNormMaxBlocks);
}

long long composed_max_blocks(const Dims& d) {
  const long long nt = cdiv(d.S, kCmpTile);
  const long long BH = (long long)d.B * d.H;
  const long long scores = BH * (nt * (nt + 1) / 2);  // lower-triangle tiles
  const long long softmax = cdiv(BH * d.S, 4);        // one row per wave
  const long long products = nt * BH;
  long long m = scores > softmax ? scores : softmax;
  return m > products ? m : products;
}

}  // namespace xattn
