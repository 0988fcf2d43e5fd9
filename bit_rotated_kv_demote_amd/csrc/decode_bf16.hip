// BF16 paged decode attention: the full-precision cache the INT2 tiers are
// measured against ("OSCAR：面向2-bit KV缓存量化的谱协方差感知旋转方法" (zingnex.cn),
// 系统级收益 / 解码加速 compares decode speed with BF16).  Same split-K
// structure as the INT2 kernel: XCD-aware work items of (sequence, KV head,
// column group, page range), per-split partials, then the same log-sum-exp
// merge kernel.
//
// A wave walks its share of a split in steps of one page (16 tokens, 8 KiB
// of K and V) with a four-stage register ring: while one step is processed
// the wave's next three are in flight.  Scores: each lane loads exactly its K
// operands of the 16x16x32 bf16 products (16 B per token row per k-slice), q
// in the columns.  Values on the vector unit: lane l loads 16 B of V rows
// (channels 8 (l & 15) .. + 8 of tokens 4 i + (l >> 4)), reads its tokens'
// weights from LDS once per step, and accumulates G x 8 outputs; the four
// lane groups that share channels are summed once at the end of the split.
#include "attn_common.h"
#include "launchers.h"

namespace oscar {

namespace {

constexpr int kBfStepPages = 1;
constexpr int kBfRing = 4;                                   // steps in registers per wave
constexpr int kBfMaxPagesPerSplit = 4 * 64 * kBfStepPages;   // 64 steps per wave (one page id per lane)

template <int G>
struct alignas(16) Bf16Smem {
  float pt[4][16 * kBfStepPages][G];   // per wave: one step's weights [token][column]
  float am[4][16];           // per wave: rescale factor of each column's sums when its max grew
  float wm[4][16];           // per-wave records (max, sum, output) for store
  float wl[4][16];
  float wo[4][G][kD];
};

// One step's operands in registers: K as 4 k-slices of 8 bf16 per page, V as
// 4 row groups of 16 B per page.
struct Bf16Step {
  bf16x8_t k[kBfStepPages][4];
  u32x4_t v[kBfStepPages][4];
};

__device__ __forceinline__ void issue_bf16_step(const DecodeBf16Args& a, int32_t ids, int hk, int k, int lane,
                                                Bf16Step& s) {
  const int x = lane & 15, qa = lane >> 4;
#pragma unroll
  for (int p = 0; p < kBfStepPages; ++p) {
    const int pid = __builtin_amdgcn_readlane(ids, kBfStepPages * k + p);
    const uint8_t* blk = reinterpret_cast<const uint8_t*>(a.kv) + (((size_t)pid * a.hkv + hk) * 2) * (kPage * kD * 2);
    const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blk), (short)0, 2 * kPage * kD * 2, 0x00020000);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      s.k[p][kk] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(r, x * 256 + 64 * kk + 16 * qa, 0, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s.v[p][i] = __builtin_amdgcn_raw_buffer_load_b128(r, kPage * kD * 2 + (4 * i + qa) * 256 + 16 * x, 0, 0);
  }
}

template <int G, class Lim>
__device__ void bf16_split_wave(const DecodeBf16Args& a, Bf16Smem<G>& sm, const bf16x8_t (&bq)[4], int32_t ids, int hk,
                                int count, int t0, Lim lim, int lim_min, int wave, int lane) {
  const int x = lane & 15, qa = lane >> 4;
  const int lim_x = lim(x < G ? x : 0);
  float m_run = kMInit, l_run = 0.0f;
  float o[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.0f;
  constexpr int kTok = 16 * kBfStepPages;          // tokens per step
  const int nsteps = (count + kTok - 1) / kTok;
  auto body = [&](const Bf16Step& cur, int st) __attribute__((always_inline)) {
    const int base = kTok * st;                     // first token of the step within the split
    const int cn = min(kTok, count - base);
    const bool partial = t0 + base + kTok - 1 > lim_min;  // some token may be past a query's position
    float sc[kBfStepPages][4];
#pragma unroll
    for (int p = 0; p < kBfStepPages; ++p) {
      float4_t d = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.k[p][kk], bq[kk], d, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * p + 4 * qa + r;
        sc[p][r] = (x < G && t < cn) ? d[r] * kC0 : -INFINITY;
      }
    }
    if (partial) {
#pragma unroll
      for (int p = 0; p < kBfStepPages; ++p)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (t0 + base + 16 * p + 4 * qa + r > lim_x) sc[p][r] = -INFINITY;
    }
    float mx = sc[0][0];
#pragma unroll
    for (int p = 0; p < kBfStepPages; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[p][r]);
    mx = rows_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const bool grew = __builtin_amdgcn_ballot_w64(m_new > m_run) != 0ull;
    if (grew) {
      // lanes own a column for the scores but channels for p . V: publish
      // the per-column rescale factor through LDS
      if (qa == 0) sm.am[wave][x] = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
    }
#pragma unroll
    for (int p = 0; p < kBfStepPages; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pv = __builtin_amdgcn_exp2f(sc[p][r] - m_run);
        l_run += pv;
        if (x < G) sm.pt[wave][16 * p + 4 * qa + r][x] = pv;
      }
    __builtin_amdgcn_wave_barrier();
    if (grew) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float alpha = sm.am[wave][h];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] *= alpha;
      }
    }
    // this lane's tokens: 16 p + 4 i + qa, channels 8 x .. 8 x + 7
#pragma unroll
    for (int p = 0; p < kBfStepPages; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * p + 4 * i + qa;
        float w[G];
        if constexpr (G >= 4) {
#pragma unroll
          for (int h4 = 0; h4 < G; h4 += 4) {
            const float4 w4 = *reinterpret_cast<const float4*>(&sm.pt[wave][t][h4]);
            w[h4] = w4.x; w[h4 + 1] = w4.y; w[h4 + 2] = w4.z; w[h4 + 3] = w4.w;
          }
        } else {
#pragma unroll
          for (int h = 0; h < G; ++h) w[h] = sm.pt[wave][t][h];
        }
        u32x4_t vv = cur.v[p][i];
        // rows past the split's tokens (a partly filled last page) may hold
        // anything: they enter with weight 0 and value 0
        if (cn < kTok && t >= cn) vv = (u32x4_t){0u, 0u, 0u, 0u};
        float vf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vf[2 * e] = bf16_bits_to_float(vv[e] & 0xFFFFu);
          vf[2 * e + 1] = __uint_as_float(vv[e] & 0xFFFF0000u);
        }
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < 8; ++e) o[h][e] = fmaf(w[h], vf[e], o[h][e]);
      }
    __builtin_amdgcn_wave_barrier();
  };
  // kBfRing-stage ring: while step st is processed, the wave's next
  // kBfRing - 1 steps are in flight.  Every slot is refilled on every round
  // (past the wave's last step it re-reads that step, an L2 hit), so each
  // body waits only for its own step's loads.
  Bf16Step ring[kBfRing];
  const int last_st = nsteps > wave ? wave + ((nsteps - 1 - wave) / 4) * 4 : wave;
  auto issue = [&](int st_, Bf16Step& s_) { issue_bf16_step(a, ids, hk, (min(st_, last_st) - wave) >> 2, lane, s_); };
#pragma unroll
  for (int r = 0; r < kBfRing - 1; ++r) issue(wave + 4 * r, ring[r]);
  for (int st = wave; st < nsteps; st += 4 * kBfRing) {
#pragma unroll
    for (int r = 0; r < kBfRing; ++r) {
      const int s_r = st + 4 * r;
      if (s_r >= nsteps) break;                        // wave-uniform
      issue(s_r + 4 * (kBfRing - 1), ring[(r + kBfRing - 1) % kBfRing]);
      body(ring[r], s_r);
    }
  }
  // the four lane groups (l >> 4) hold the same channels for different tokens
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = rows_sum(o[h][e]);
  l_run = rows_sum(l_run);
  if (qa == 0) {
    sm.wm[wave][x] = m_run;
    sm.wl[wave][x] = l_run;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      *reinterpret_cast<float4*>(&sm.wo[wave][h][8 * x]) = make_float4(o[h][0], o[h][1], o[h][2], o[h][3]);
      *reinterpret_cast<float4*>(&sm.wo[wave][h][8 * x + 4]) = make_float4(o[h][4], o[h][5], o[h][6], o[h][7]);
    }
  }
}

template <int G>
__device__ void store_bf16_split(Bf16Smem<G>& sm, float* rec, int tid) {
  __syncthreads();
  for (int c = tid; c < G * kD / 4; c += 256) {
    const int h = c / (kD / 4), j4 = c % (kD / 4);
    float mm = kMInit;
#pragma unroll
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, sm.wm[w][h]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float ll = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = __builtin_amdgcn_exp2f(sm.wm[w][h] - mm);
      const float4 o = *reinterpret_cast<const float4*>(&sm.wo[w][h][4 * j4]);
      acc.x = fmaf(f, o.x, acc.x); acc.y = fmaf(f, o.y, acc.y);
      acc.z = fmaf(f, o.z, acc.z); acc.w = fmaf(f, o.w, acc.w);
      ll = fmaf(f, sm.wl[w][h], ll);
    }
    *reinterpret_cast<float4*>(rec + h * kPartStride + 4 * j4) = acc;
    if (j4 == 0) *reinterpret_cast<float2*>(rec + h * kPartStride + kD) = make_float2(mm, ll);
  }
}

}  // namespace

template <int G>
__global__ __launch_bounds__(256, 2) void decode_bf16_kernel(DecodeBf16Args a) {
  __shared__ Bf16Smem<G> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int item = (blockIdx.x & 7) * a.grid_per_xcd + (blockIdx.x >> 3);
  if (item >= a.n_groups_total * a.n_splits) return;
  const int grp = item / a.n_splits, split = item % a.n_splits;
  // group = (sequence b, KV head hk, column group cg); column x is virtual
  // head cg * G + x = (query token t, head h), as in the INT2 kernel
  const int cg = grp % a.n_colgroups;
  const int b = grp / (a.hkv * a.n_colgroups), hk = (grp / a.n_colgroups) % a.hkv;
  const int hq_total = a.hkv * a.g_model;
  const int x = lane & 15, qa = lane >> 4;
  // q of column x (bf16, the B operand of the score products): requested
  // before the sequence's length is known
  bf16x8_t bq[4];
  {
    const int vh = cg * G + (x < G ? x : 0), t = vh / a.g_model, h = vh - t * a.g_model;
    const uint16_t* qrow = a.q + (((size_t)b * a.q_tokens + t) * hq_total + hk * a.g_model + h) * kD;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(qrow + 32 * kk + 8 * qa);
      if (x >= G) v = (bf16x8_t){};
      bq[kk] = v;
    }
  }
  const int slot = a.seq_slot ? a.seq_slot[b] : b;
  const int32_t* pt_row = a.page_table + (size_t)slot * a.max_pages;
  // this wave's page ids (lane 2 k + i: page i of the wave's k-th step),
  // requested before the length (clamped to the page-table row)
  const int pg0 = split * a.pages_per_split;
  const int idx_in_split = kBfStepPages * (wave + 4 * (lane / kBfStepPages)) + lane % kBfStepPages;
  const int32_t ids_spec = pt_row[pg0 + min(idx_in_split, a.max_pages - 1 - pg0)];
  const int32_t first_id = pt_row[pg0];
  const int n = a.seq_len[b];
  const int npages = (n + kPage - 1) / kPage;
  const int act = (npages + a.pages_per_split - 1) / a.pages_per_split;
  if (split >= act) return;
  const int t0 = pg0 * kPage;
  const int count = min(a.pages_per_split * kPage, n - t0);
  const int n_valid_pages = (count + kPage - 1) / kPage;
  // lanes past the split's last valid page take its first page (never a page past the sequence)
  const int32_t ids = idx_in_split < n_valid_pages ? ids_spec : first_id;
  // causal limit of column x: its query's position n - q_tokens + t
  bf16_split_wave<G>(a, sm, bq, ids, hk, count, t0,
                     [&](int xx) { return n - a.q_tokens + (cg * G + xx) / a.g_model; }, n - a.q_tokens, wave, lane);
  float* part_base = a.partials + (size_t)grp * a.n_splits * G * kPartStride;
  store_bf16_split<G>(sm, part_base + (size_t)split * G * kPartStride, tid);
}

DecodePlan plan_decode_bf16(int batch, int hkv, int group, int n_colgroups, int max_seq_len) {
  DecodePlan p{};
  const int max_pages = (max_seq_len + kPage - 1) / kPage;
  const long n_groups = (long)batch * hkv * n_colgroups;
  // the most splits per group that keep the grid within two workgroups per
  // compute unit; each split a multiple of 4 waves x one step (8 pages)
  const long per_group = kDecodeSplitTarget / n_groups;
  long pps = per_group >= 1 ? (max_pages + per_group - 1) / per_group : kBfMaxPagesPerSplit;
  pps = (pps + 4 * kBfStepPages - 1) / (4 * kBfStepPages) * (4 * kBfStepPages);
  if (pps < 4 * kBfStepPages) pps = 4 * kBfStepPages;
  if (pps > kBfMaxPagesPerSplit) pps = kBfMaxPagesPerSplit;
  p.ok = (max_pages + pps - 1) / pps <= kMaxSplits;
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
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace oscar
