// BF16 paged decode attention: the full-precision cache the INT2 tiers are
// measured against ("OSCAR：面向2-bit KV缓存量化的谱协方差感知旋转方法" (zingnex.cn),
// 系统级收益 / 解码加速 compares decode speed with BF16).  Same structure as
// the INT2 kernel: XCD-aware work items of (sequence, KV head, page range),
// per-split partials, then the same log-sum-exp merge kernel.
#include "attn_common.h"
#include "launchers.h"

namespace oscar {

template <int G>
__global__ __launch_bounds__(256) void decode_bf16_kernel(DecodeBf16Args a) {
  __shared__ SplitSmem<G> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int item = (blockIdx.x & 7) * a.grid_per_xcd + (blockIdx.x >> 3);
  if (item >= a.n_groups_total * a.n_splits) return;
  const int grp = item / a.n_splits, split = item % a.n_splits;
  // group = (sequence b, KV head hk, column group cg); column x is virtual
  // head cg * G + x = (query token t, head h), as in the INT2 kernel
  const int cg = grp % a.n_colgroups;
  const int b = grp / (a.hkv * a.n_colgroups), hk = (grp / a.n_colgroups) % a.hkv;
  const int slot = a.seq_slot ? a.seq_slot[b] : b;
  const int n = a.seq_len[b];
  const int npages = (n + kPage - 1) / kPage;
  const int act = (npages + a.pages_per_split - 1) / a.pages_per_split;
  if (split >= act) return;
  const int t0 = split * a.pages_per_split * kPage;
  const int count = min(a.pages_per_split * kPage, n - t0);
  const int32_t* pt_row = a.page_table + (size_t)slot * a.max_pages;
  auto row = [&](int uu, int kv) -> const uint16_t* {
    const int tok = t0 + uu;
    const int page = pt_row[tok >> 4];
    return a.kv + ((((size_t)page * a.hkv + hk) * 2 + kv) * kPage + (tok & 15)) * kD;
  };
  const int hq_total = a.hkv * a.g_model;
  auto q_row = [&](int x) -> const uint16_t* {
    const int vh = cg * G + x, t = vh / a.g_model, h = vh - t * a.g_model;
    return a.q + (((size_t)b * a.q_tokens + t) * hq_total + hk * a.g_model + h) * kD;
  };
  // causal limit of column x: its query's position n - q_tokens + t
  bf16_span_wave<G>(q_row, count, [&](int uu) { return row(uu, 0); }, [&](int uu) { return row(uu, 1); },
                    [&](int uu) { return t0 + uu; },
                    [&](int x) { return n - a.q_tokens + (cg * G + x) / a.g_model; }, n - a.q_tokens, sm, wave,
                    lane);
  float* part_base = a.partials + (size_t)grp * a.n_splits * G * kPartStride;
  store_split<G>(sm, part_base + (size_t)split * G * kPartStride, tid);
}

DecodePlan plan_decode_bf16(int batch, int hkv, int group, int n_colgroups, int max_seq_len) {
  DecodePlan p{};
  p.ok = true;
  const int max_pages = (max_seq_len + kPage - 1) / kPage;
  const long n_groups = (long)batch * hkv * n_colgroups;
  const long total_pages = n_groups * max_pages;
  long pps = (total_pages + 479) / 480;
  pps = ((pps + 1) / 2) * 2;
  if (pps < 2) pps = 2;
  while ((max_pages + pps - 1) / pps > kMaxSplits) pps += 2;
  p.pages_per_split = (int)pps;
  p.n_hist_splits = (int)((max_pages + pps - 1) / pps);
  p.n_tile_splits = 0;
  p.n_splits_total = p.n_hist_splits;
  p.n_work = (int)(n_groups * p.n_splits_total);
  p.grid = ((p.n_work + 7) / 8) * 8;
  p.partial_floats = (size_t)n_groups * p.n_splits_total * group * kPartStride;
  p.workspace_bytes = p.partial_floats * sizeof(float);
  return p;
}

hipError_t launch_decode_bf16(const DecodeBf16Args& a, int group, int grid, hipStream_t st) {
  switch (group) {
    case 1: hipLaunchKernelGGL(decode_bf16_kernel<1>, dim3(grid), dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL(decode_bf16_kernel<2>, dim3(grid), dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL(decode_bf16_kernel<4>, dim3(grid), dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL(decode_bf16_kernel<8>, dim3(grid), dim3(256), 0, st, a); break;
    case 16: hipLaunchKernelGGL(decode_bf16_kernel<16>, dim3(grid), dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace oscar
