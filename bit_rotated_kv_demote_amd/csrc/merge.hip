// Log-sum-exp merge of the split partials that the decode kernels leave in
// the workspace (flash-decoding split-K).  The history tier is attended in the
// rotated space, so its merged output is turned back with the inverse
// rotation before it joins the sink/recent part ("OSCAR: Offline Spectral
// Covariance-Aware Rotation for 2-bit KV Cache Quantization" (gist.science),
// 2.2 B "Kernel-Integration": inverse rotation inside the attention kernel).
//
// A second kernel on the same stream, one workgroup per (sequence, query
// head): the kernel boundary publishes every record, so no ticket or
// device-scope fence is needed, and all of a head's loads - its (m, l) pairs,
// its record columns and its rows of R - are issued together, which makes the
// merge one memory round trip instead of a chain of them in a single
// workgroup per KV head.
#include "attn_common.h"
#include "launchers.h"

namespace oscar {

namespace {

constexpr int kParts = 8;          // record rows handled side by side (256 threads / 32 float4 columns)
constexpr int kMergeBatch = 8;     // record loads in flight per thread: 64 splits per round

// kRB workgroups per head, each writing kD / kRB output rows: every one
// merges the head's records (the whole rotated sum is needed for any output
// row) but loads only its kD / kRB rows of R.  kRB = 4 when the heads are
// few (the loads of R, 64 KiB per head, then dominate each workgroup).
template <int kRB>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int kRows = kD / kRB;          // output rows of this workgroup
  constexpr int kColParts = 256 / kRows;   // threads sharing one row of R
  constexpr int kCols = kD / kColParts;    // columns of R per thread
  __shared__ float w[4][kMaxSplits];       // per wave: the weight of every slot
  __shared__ float4 red[kParts][2][kD / 4];
  __shared__ float oh[2][kD];      // weighted sums: plain part, rotated part
  __shared__ float rr[kColParts][kRows];   // partial sums of (rotated part . R^T)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.group;
  // output row head = (b * q_tokens + t) * Hq + hq; its records: work-item
  // group (b, hk, cg) and column x, with virtual head t * g_model + h = cg * G + x
  const int head = blockIdx.x;
  const int hq_total = a.hkv * a.g_model;
  const int b = head / (a.q_tokens * hq_total);
  const int t = (head / hq_total) % a.q_tokens, hq = head % hq_total;
  const int vh = t * a.g_model + hq % a.g_model;
  const int grp = (b * a.hkv + hq / a.g_model) * a.n_colgroups + vh / G, h = vh % G;
  const int n_slots = a.n_splits_total;
  // record slot s of this head: slots [0, n_plain_slots) hold output-space
  // partials, the rest rotated-space ones (history)
  const float* base = a.partials + (size_t)grp * n_slots * G * kPartStride + (size_t)h * kPartStride;
  auto rec = [&](int s) { return base + (size_t)min(s, n_slots - 1) * G * kPartStride; };

  const int row0 = kRows * blockIdx.y;     // first output row of this workgroup
  // Every load first, before the sequence length is known: (m, l) of every
  // slot (each wave loads all of them, lane s taking slots s + 64 k), the
  // first round of record columns and this thread's slice of R (row
  // row0 + ri, columns [kCols jh, kCols jh + kCols)).  Slots the first kernel
  // left untouched for this length are masked below, never multiplied in.
  constexpr int kMlRounds = (kMaxSplits + 63) / 64;
  float2 ml[kMlRounds];
#pragma unroll
  for (int k = 0; k < kMlRounds; ++k) ml[k] = *reinterpret_cast<const float2*>(rec(lane + 64 * k) + kD);
  const int c4 = tid & 31, part = tid >> 5;
  float4 v[kMergeBatch];
#pragma unroll
  for (int u = 0; u < kMergeBatch; ++u) v[u] = *reinterpret_cast<const float4*>(rec(part + kParts * u) + 4 * c4);
  const int ri = tid % kRows, jh = tid / kRows;
  float4 rrow[kCols / 4];
  if (a.tiered) {
    const float* rot = a.rot + (size_t)(hq / a.g_model) * a.rot_kv_stride;
    const float4* rp = reinterpret_cast<const float4*>(rot + (size_t)(row0 + ri) * kD + kCols * jh);
#pragma unroll
    for (int e = 0; e < kCols / 4; ++e) rrow[e] = rp[e];
  }

  // the splits the first kernel filled for this sequence (clamped to the
  // slots, so that a length outside [1, max_seq_len] stays in bounds)
  const int n = a.seq_len[b] + a.len_offset;
  int n_plain, n_rot;
  if (a.tiered) {
    const int hist_len = max(0, n - kSink - kRecent);
    const int n_hist_pages = (hist_len + kPage - 1) / kPage;
    const int n_tile = min(n, kSink) + min(max(n - kSink, 0), kRecent);
    n_plain = min((n_tile + a.tile_tokens - 1) / a.tile_tokens, a.n_plain_slots);
    n_rot = min((n_hist_pages + a.pages_per_split - 1) / a.pages_per_split, n_slots - a.n_plain_slots);
  } else {
    const int npages = (max(n, 0) + kPage - 1) / kPage;
    n_plain = min((npages + a.pages_per_split - 1) / a.pages_per_split, a.n_plain_slots);
    n_rot = 0;
  }
  if (n_plain + n_rot <= 0) {       // no tokens: nothing to attend
    if (tid < kRows) a.out[(size_t)head * kD + row0 + tid] = 0.0f;
    return;
  }
  auto active = [&](int s) { return s < a.n_plain_slots ? s < n_plain : s - a.n_plain_slots < n_rot; };

  // maximum over the head's active splits, weights and total sum: every wave
  // computes them itself, so no workgroup barrier is needed before the sums
  float mm = kMInit;
#pragma unroll
  for (int k = 0; k < kMlRounds; ++k) {
    const int s = lane + 64 * k;
    if (s < n_slots && active(s)) mm = fmaxf(mm, ml[k].x);
  }
  const float m_all = wave_max(mm);
  float ll = 0.0f;
#pragma unroll
  for (int k = 0; k < kMlRounds; ++k) {
    const int s = lane + 64 * k;
    if (s < n_slots && active(s)) {
      const float wk = __builtin_amdgcn_exp2f(ml[k].x - m_all);
      w[wave][s] = wk;
      ll = fmaf(wk, ml[k].y, ll);
    }
  }
  const float l_all = wave_sum(ll);
  __builtin_amdgcn_wave_barrier();

  // weighted sums of the record columns, plain and rotated kept apart
  float4 ap = make_float4(0.f, 0.f, 0.f, 0.f), ar = ap;
  auto acc_into = [&](int s, const float4& x) {
    if (s >= n_slots || !active(s)) return;
    const float wk = w[wave][s];
    float4& acc = s < a.n_plain_slots ? ap : ar;
    acc.x = fmaf(wk, x.x, acc.x); acc.y = fmaf(wk, x.y, acc.y);
    acc.z = fmaf(wk, x.z, acc.z); acc.w = fmaf(wk, x.w, acc.w);
  };
#pragma unroll
  for (int u = 0; u < kMergeBatch; ++u) acc_into(part + kParts * u, v[u]);
  for (int s0 = part + kParts * kMergeBatch; s0 < n_slots; s0 += kParts * kMergeBatch) {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) v[u] = *reinterpret_cast<const float4*>(rec(s0 + kParts * u) + 4 * c4);
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) acc_into(s0 + kParts * u, v[u]);
  }
  red[part][0][c4] = ap;
  red[part][1][c4] = ar;
  __syncthreads();
  {
    const int which = tid >> 7, j = tid & (kD - 1);
    const float* rp = reinterpret_cast<const float*>(&red[0][which][0]) + j;
    float s = 0.0f;
#pragma unroll
    for (int p = 0; p < kParts; ++p) s += rp[p * 2 * kD];
    oh[which][j] = s;
  }
  __syncthreads();
  // inverse rotation of the history part: (y R^T)_i = sum_j y_j R[i][j]
  float acc = 0.0f;
  if (n_rot > 0) {
#pragma unroll
    for (int e = 0; e < kCols / 4; ++e) {
      const float4 y = *reinterpret_cast<const float4*>(&oh[1][kCols * jh + 4 * e]);
      acc = fmaf(y.x, rrow[e].x, acc);
      acc = fmaf(y.y, rrow[e].y, acc);
      acc = fmaf(y.z, rrow[e].z, acc);
      acc = fmaf(y.w, rrow[e].w, acc);
    }
  }
  rr[jh][ri] = acc;
  __syncthreads();
  // (l_all is 0 only if every token was masked for this query, a length
  // shorter than the query count)
  if (tid < kRows) {
    float r = 0.0f;
#pragma unroll
    for (int p = 0; p < kColParts; ++p) r += rr[p][tid];
    const int i = row0 + tid;
    a.out[(size_t)head * kD + i] = l_all > 0.0f ? (oh[0][i] + r) / l_all : 0.0f;
  }
}

// Large grids: `parts` workgroups per record group (sequence, KV head,
// column group) of G columns, each taking G / parts >= 4 consecutive
// columns.  Wave w merges the part's columns w, w + 4, ...; the workgroup
// then applies R^T to each of them with one load of its slice of R, so the
// R traffic (the bound when thousands of heads are merged) falls
// (G / parts)-fold.
__global__ __launch_bounds__(256) void merge_group_kernel(MergeArgs a, int parts) {
  __shared__ float w[4][kMaxSplits];
  __shared__ float oh[16][2][kD];
  __shared__ float rr[16][2][kD];
  __shared__ float lsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.group;
  const int grp = blockIdx.x / parts;
  const int h0 = (blockIdx.x % parts) * (G / parts), h1 = h0 + G / parts;
  const int b = grp / (a.hkv * a.n_colgroups), hk = (grp / a.n_colgroups) % a.hkv, cg = grp % a.n_colgroups;
  const int n_slots = a.n_splits_total;
  const float* gbase = a.partials + (size_t)grp * n_slots * G * kPartStride;
  const int hq_total = a.hkv * a.g_model;
  auto out_row = [&](int h) {
    const int vh = cg * G + h, t = vh / a.g_model;
    return a.out + (((size_t)b * a.q_tokens + t) * hq_total + hk * a.g_model + (vh - t * a.g_model)) * kD;
  };
  const int ri = tid & (kD - 1), jh = tid >> 7;
  float4 rrow[16];
  if (a.tiered) {
    const float* rot = a.rot + (size_t)hk * a.rot_kv_stride;
    const float4* rp = reinterpret_cast<const float4*>(rot + (size_t)ri * kD + 64 * jh);
#pragma unroll
    for (int e = 0; e < 16; ++e) rrow[e] = rp[e];
  }
  const int n = a.seq_len[b] + a.len_offset;
  int n_plain, n_rot;
  if (a.tiered) {
    const int hist_len = max(0, n - kSink - kRecent);
    const int n_hist_pages = (hist_len + kPage - 1) / kPage;
    const int n_tile = min(n, kSink) + min(max(n - kSink, 0), kRecent);
    n_plain = min((n_tile + a.tile_tokens - 1) / a.tile_tokens, a.n_plain_slots);
    n_rot = min((n_hist_pages + a.pages_per_split - 1) / a.pages_per_split, n_slots - a.n_plain_slots);
  } else {
    const int npages = (max(n, 0) + kPage - 1) / kPage;
    n_plain = min((npages + a.pages_per_split - 1) / a.pages_per_split, a.n_plain_slots);
    n_rot = 0;
  }
  if (n_plain + n_rot <= 0) {       // no tokens: nothing to attend
    for (int idx = tid; idx < (h1 - h0) * kD; idx += 256) out_row(h0 + idx / kD)[idx % kD] = 0.0f;
    return;
  }
  auto active = [&](int s) { return s < a.n_plain_slots ? s < n_plain : s - a.n_plain_slots < n_rot; };

  const int c4 = lane & 31, part = lane >> 5;
  for (int h = h0 + wave; h < h1; h += 4) {
    const float* hb = gbase + (size_t)h * kPartStride;
    auto rec = [&](int s) { return hb + (size_t)min(s, n_slots - 1) * G * kPartStride; };
    // max, weights and total over the column's active splits (lanes stride 64)
    float mm = kMInit;
    for (int s = lane; s < n_slots; s += 64)
      if (active(s)) mm = fmaxf(mm, rec(s)[kD]);
    mm = wave_max(mm);
    float ll = 0.0f;
    for (int s = lane; s < n_slots; s += 64) {
      const float2 ml = *reinterpret_cast<const float2*>(rec(s) + kD);
      const float wk = active(s) ? __builtin_amdgcn_exp2f(ml.x - mm) : 0.0f;
      w[wave][s] = wk;
      ll = active(s) ? fmaf(wk, ml.y, ll) : ll;
    }
    ll = wave_sum(ll);
    if (lane == 0) lsum[h] = ll;
    __builtin_amdgcn_wave_barrier();
    // weighted sums of the record columns: lanes l and l + 32 take alternate splits
    float4 ap = make_float4(0.f, 0.f, 0.f, 0.f), ar = ap;
    for (int s0 = part; s0 < n_slots; s0 += 8) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const float4*>(rec(s0 + 2 * u) + 4 * c4);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int sl = s0 + 2 * u;
        if (sl >= n_slots || !active(sl)) continue;
        const float wk = w[wave][sl];
        float4& acc = sl < a.n_plain_slots ? ap : ar;
        acc.x = fmaf(wk, v[u].x, acc.x); acc.y = fmaf(wk, v[u].y, acc.y);
        acc.z = fmaf(wk, v[u].z, acc.z); acc.w = fmaf(wk, v[u].w, acc.w);
      }
    }
    ap.x = half_swap_sum(ap.x); ap.y = half_swap_sum(ap.y); ap.z = half_swap_sum(ap.z); ap.w = half_swap_sum(ap.w);
    ar.x = half_swap_sum(ar.x); ar.y = half_swap_sum(ar.y); ar.z = half_swap_sum(ar.z); ar.w = half_swap_sum(ar.w);
    if (part == 0) {
      *reinterpret_cast<float4*>(&oh[h][0][4 * c4]) = ap;
      *reinterpret_cast<float4*>(&oh[h][1][4 * c4]) = ar;
    }
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  // inverse rotation of every column's history part: (y R^T)_i = sum_j y_j R[i][j]
  for (int h = h0; h < h1; ++h) {
    float acc = 0.0f;
    if (n_rot > 0) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float4 y = *reinterpret_cast<const float4*>(&oh[h][1][64 * jh + 4 * e]);
        acc = fmaf(y.x, rrow[e].x, acc);
        acc = fmaf(y.y, rrow[e].y, acc);
        acc = fmaf(y.z, rrow[e].z, acc);
        acc = fmaf(y.w, rrow[e].w, acc);
      }
    }
    rr[h][jh][ri] = acc;
  }
  __syncthreads();
  for (int idx = tid; idx < (h1 - h0) * kD; idx += 256) {
    const int h = h0 + idx / kD, i = idx % kD;
    const float l = lsum[h];
    out_row(h)[i] = l > 0.0f ? (oh[h][0][i] + (rr[h][0][i] + rr[h][1][i])) / l : 0.0f;
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int n_heads, hipStream_t st) {
  if (n_heads <= 0) return hipSuccess;
  // few heads: four workgroups per head (a quarter of R each); up to about
  // three workgroups per compute unit: one workgroup per head spreads the
  // latency; beyond that, record groups share R, split over up to four
  // workgroups (at least four columns each) while fewer than 512 run
  if (n_heads <= 64) {
    hipLaunchKernelGGL(merge_kernel<4>, dim3(n_heads, 4), dim3(256), 0, st, a);
  } else if (n_heads <= 768 || a.group < 2) {
    hipLaunchKernelGGL(merge_kernel<1>, dim3(n_heads), dim3(256), 0, st, a);
  } else {
    const int n_groups = n_heads / a.group;
    int parts = 1;
    while (4 * parts < a.group && n_groups * parts < 512) parts *= 2;
    hipLaunchKernelGGL(merge_group_kernel, dim3(n_groups * parts), dim3(256), 0, st, a, parts);
  }
  return hipGetLastError();
}

}  // namespace oscar
