// Single-token decode attention over the three-tier pool (BF16 sink, INT2
// history, BF16 recent) -- the fused INT2 attention of "OSCAR: Offline
// Spectral Covariance-Aware Rotation for 2-bit KV Cache Quantization"
// (gist.science), 2.2 B "Kernel-Integration" (unpack, dequantise, inverse
// rotation and attention in one kernel, paged cache), and of
// "OSCAR：面向2-bit KV缓存量化的谱协方差感知旋转方法" (zingnex.cn), section
// 自定义INT2注意力内核.  Tiers: "大模型KV Cache 2bit量化实战" (yunpan.plus), 三.1.
//
// One launch per call.  Workgroups are "work items" of one (sequence, KV
// head) group: BF16 tile splits (sink + recent tokens) and history splits
// (runs of INT2 pages).  Each writes a partial (running max m, sum l and
// unnormalised output, all G query heads of the group) to the workspace; the
// last workgroup of the group to finish (atomic ticket) merges the partials
// by log-sum-exp, rotates the history part back with R_V^T, and writes the
// fp32 output.
//
// History scoring works in the rotated space: with q' = q . R_K and the
// dequantised key k'_t = s_{t,g} c_{t,j} + z_{t,g},
//   q . k~_t = sum_g s_{t,g} sum_{j in g} q'_j c_{t,j} + sum_g z_{t,g} sum_{j in g} q'_j.
// The per-group code sums run on the matrix cores: 2-bit codes are placed in
// fp16 operands as exact subnormals (one AND per two codes, c * 4^f * 2^-24)
// and q' is split into fp16 hi + lo halves occupying two operand columns.
// The value side accumulates p_t s_{t,g} c_{t,j} on the matrix cores and
// p_t z_{t,g} with one more small product, all in the rotated space.
#include "attn_common.h"
#include "launchers.h"

namespace oscar {

// 2-bit field f (0..7) of both 16-bit halves of w as fp16 subnormals c * 4^s * 2^-24,
// s = f for f <= 4 and f - 3 otherwise (w6 = w >> 6).
template <int F>
__device__ __forceinline__ uint32_t field_pair(uint32_t w, uint32_t w6) {
  constexpr int s = F <= 4 ? F : F - 3;
  constexpr uint32_t mask = (3u << (2 * s)) | (3u << (16 + 2 * s));
  return (F <= 4 ? w : w6) & mask;
}
__host__ __device__ constexpr int field_shift(int f) { return f <= 4 ? f : f - 3; }

// Shared memory of one workgroup (256 threads = 4 waves).
template <int G>
struct alignas(16) DecodeSmem : SplitSmem<G> {
  float q[G][kD];            // q (fp32)
  float qr[G][kD];           // q' = q . R_K
  float sexp[G];             // S_h: q' operands are scaled by 2^S_h
  float qs[G][kGroups];      // per-group sums of q'
  uint8_t meta[4][2][512];   // per wave, two pages of scale/zero metadata
  float zs[4][kGroups][16];  // per-wave V zero-point accumulators
};

// ---------------------------------------------------------------------------
// Per-wave partial of a history split: pages [pg_begin, pg_end) of the
// sequence's history (hist_len valid tokens).
// ---------------------------------------------------------------------------
// Loads of one page pair for a wave: codes (16 B per lane per page) and
// scale/zero metadata (8 B per lane per page).  ids: this wave's page ids,
// lane 2k + i holding page 2 (wave + 4k) + i of the split (clamped to its
// last page), so the k-th pair of the wave needs no memory access for its
// page ids.
__device__ __forceinline__ void issue_pair(const DecodeArgs& a, int32_t ids, int hk, int k, int lane,
                                           u32x4_t* c, u32x2_t* md) {
  const int p0 = __builtin_amdgcn_readlane(ids, 2 * k);
  const int p1 = __builtin_amdgcn_readlane(ids, 2 * k + 1);
  const uint8_t* b0 = a.hist + ((size_t)p0 * a.hkv + hk) * kBlock;
  const uint8_t* b1 = a.hist + ((size_t)p1 * a.hkv + hk) * kBlock;
  c[0] = *reinterpret_cast<const u32x4_t*>(b0 + 16 * lane);
  c[1] = *reinterpret_cast<const u32x4_t*>(b1 + 16 * lane);
  md[0] = *reinterpret_cast<const u32x2_t*>(b0 + 1024 + 8 * lane);
  md[1] = *reinterpret_cast<const u32x2_t*>(b1 + 1024 + 8 * lane);
}

template <int G>
__device__ void hist_wave(const DecodeArgs& a, DecodeSmem<G>& sm, int32_t ids, int hk, int hist_len,
                          int pg_begin, int pg_end, int wave, int lane, const u32x4_t* c_first,
                          const u32x2_t* m_first, const u32x4_t* c_second, const u32x2_t* m_second) {
  const int x = lane & 15, qa = lane >> 4;
  const int col_head = x < G ? x : (x < 2 * G ? x - G : -1);
  // ---- score operands: q' in fp16 hi (columns 0..G-1) and lo (G..2G-1)
  half8_t bq[4];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int j = 32 * g + 8 * qa + 2 * i + hf;
        const int s = field_shift(4 * (g & 1) + i);
        _Float16 e = (_Float16)0.0f;
        if (col_head >= 0) {
          const float v = ldexpf(sm.qr[col_head][j] * kC0, (int)sm.sexp[col_head] - 2 * s);
          const _Float16 hi = (_Float16)v;
          e = (x < G) ? hi : (_Float16)(v - (float)hi);
        }
        bq[g][2 * i + hf] = e;
      }
  // zero-point term operand (fp32 product, 4 groups = K of 4)
  const float be = (x < G) ? ldexpf(sm.qs[x][qa] * kC0, (int)sm.sexp[x] - 24) : 0.0f;
  const float mult = (x < G) ? ldexpf(1.0f, 24 - (int)sm.sexp[x]) : 1.0f;

  float4_t acc_o[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc_o[m] = (float4_t){0.f, 0.f, 0.f, 0.f};
  float4_t acc_z = (float4_t){0.f, 0.f, 0.f, 0.f};
  float m_run = kMInit, l_run = 0.0f;

  const int npairs = (pg_end - pg_begin + 1) >> 1;
  uint8_t* mbuf = &sm.meta[wave][0][0];

  // three-stage prefetch ring: while pair pr is processed, pairs pr + 4 and
  // pr + 8 of this wave are in flight (the first two were issued before the
  // prologue)
  u32x4_t cA[2] = {c_first[0], c_first[1]}, cB[2] = {c_second[0], c_second[1]}, cC[2];
  u32x2_t mA[2] = {m_first[0], m_first[1]}, mB[2] = {m_second[0], m_second[1]}, mC[2];
  auto issue = [&](int pr_, u32x4_t* c, u32x2_t* md) { issue_pair(a, ids, hk, (pr_ - wave) >> 2, lane, c, md); };
  int pr = wave;
  auto body = [&](const u32x4_t* c_cur, const u32x2_t* m_cur) __attribute__((always_inline)) {
    const int pg0 = pg_begin + 2 * pr;
    const bool has1 = pg0 + 1 < pg_end;
    // stage this pair's metadata in LDS (wave-private)
    *reinterpret_cast<u32x2_t*>(mbuf + 8 * lane) = m_cur[0];
    *reinterpret_cast<u32x2_t*>(mbuf + 512 + 8 * lane) = m_cur[1];
    __builtin_amdgcn_wave_barrier();

    // valid tokens of the pair: token t of page p is history index 16 (pg0 + p) + t
    const int base_tok = 16 * pg0;
    const bool full = has1 && (base_tok + 32 <= hist_len);

    // ---------------- scores
    float sc[2][4];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const uint32_t w0 = c_cur[p][0], w1 = c_cur[p][1];
      const uint32_t w0s = w0 >> 6, w1s = w1 >> 6;
      half8_t ak[4];
      uint32_t* ak32 = reinterpret_cast<uint32_t*>(ak);
      ak32[0] = field_pair<0>(w0, w0s);  ak32[1] = field_pair<1>(w0, w0s);
      ak32[2] = field_pair<2>(w0, w0s);  ak32[3] = field_pair<3>(w0, w0s);
      ak32[4] = field_pair<4>(w0, w0s);  ak32[5] = field_pair<5>(w0, w0s);
      ak32[6] = field_pair<6>(w0, w0s);  ak32[7] = field_pair<7>(w0, w0s);
      ak32[8] = field_pair<0>(w1, w1s);  ak32[9] = field_pair<1>(w1, w1s);
      ak32[10] = field_pair<2>(w1, w1s); ak32[11] = field_pair<3>(w1, w1s);
      ak32[12] = field_pair<4>(w1, w1s); ak32[13] = field_pair<5>(w1, w1s);
      ak32[14] = field_pair<6>(w1, w1s); ak32[15] = field_pair<7>(w1, w1s);
      float4_t d[4];
#pragma unroll
      for (int g = 0; g < 4; ++g)
        d[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak[g], bq[g], (float4_t){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      // scales of tokens 4qa..4qa+3 (K scale area [token][group])
      const uint8_t* mp = mbuf + 512 * p;
      const u32x4_t s01 = *reinterpret_cast<const u32x4_t*>(mp + 32 * qa);
      const u32x4_t s23 = *reinterpret_cast<const u32x4_t*>(mp + 32 * qa + 16);
      const _Float16* sh0 = reinterpret_cast<const _Float16*>(&s01);
      const _Float16* sh1 = reinterpret_cast<const _Float16*>(&s23);
      float4_t cacc;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const _Float16* sr = (r < 2) ? sh0 + 4 * r : sh1 + 4 * (r - 2);
        float v = (float)sr[0] * d[0][r];
        v = fmaf((float)sr[1], d[1][r], v);
        v = fmaf((float)sr[2], d[2][r], v);
        v = fmaf((float)sr[3], d[3][r], v);
        cacc[r] = v;
      }
      // + sum_g zero[t][g] * (scaled group sums of q'), t = lane's row token
      const _Float16 zk = *reinterpret_cast<const _Float16*>(mp + 128 + 8 * x + 2 * qa);
      cacc = __builtin_amdgcn_mfma_f32_16x16x4f32((float)zk, be, cacc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float other = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
            0u, __float_as_uint(cacc[r]), 0x120 + (16 - G), 0xF, 0xF, false));
        float l = cacc[r] + other;
        const int tok = base_tok + 16 * p + 4 * qa + r;
        const bool ok = (x < G) && (p == 0 || has1) && (full || tok < hist_len);
        sc[p][r] = ok ? l : -INFINITY;
      }
    }
    // ---------------- online softmax over the 32 tokens of the pair
    float mx = sc[0][0];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[p][r]);
    mx = rows_max(mx);
    const float m_new = fmaxf(m_run, mx * mult);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0ull) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int m = 0; m < 8; ++m) acc_o[m] *= alpha;
      acc_z *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    float pv[2][4];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[p][r] = __builtin_amdgcn_exp2f(fmaf(sc[p][r], mult, -m_run));
        l_run += pv[p][r];
      }
    // ---------------- values
    uint32_t pp[4];                 // fp16 p pairs: (page i>>1, tokens 2(i&1), +1)
    pp[0] = pack_h2(pv[0][0], pv[0][1]);
    pp[1] = pack_h2(pv[0][2], pv[0][3]);
    pp[2] = pack_h2(pv[1][0], pv[1][1]);
    pp[3] = pack_h2(pv[1][2], pv[1][3]);
    // V scales [token/4][group][token%4]: lane reads its token quad of both pages
    u32x4_t vs[2][2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      vs[p][0] = *reinterpret_cast<const u32x4_t*>(mbuf + 512 * p + 256 + 32 * qa);
      vs[p][1] = *reinterpret_cast<const u32x4_t*>(mbuf + 512 * p + 256 + 32 * qa + 16);
    }
    u32x2_t vz[2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
      vz[p] = (x < 4) ? *reinterpret_cast<const u32x2_t*>(mbuf + 512 * p + 384 + 32 * qa + 8 * x)
                      : (u32x2_t){0u, 0u};
    if (!full) {
      // tokens past the end may hold stale bytes: zero their scales and zeros
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        uint32_t keep[2];
#pragma unroll
        for (int hw = 0; hw < 2; ++hw) {
          const int t0 = base_tok + 16 * p + 4 * qa + 2 * hw;
          const bool pg_ok = (p == 0) || has1;
          keep[hw] = (pg_ok && t0 < hist_len ? 0x0000FFFFu : 0u) | (pg_ok && t0 + 1 < hist_len ? 0xFFFF0000u : 0u);
        }
        vs[p][0][0] &= keep[0]; vs[p][0][1] &= keep[1]; vs[p][0][2] &= keep[0]; vs[p][0][3] &= keep[1];
        vs[p][1][0] &= keep[0]; vs[p][1][1] &= keep[1]; vs[p][1][2] &= keep[0]; vs[p][1][3] &= keep[1];
        vz[p][0] &= keep[0]; vz[p][1] &= keep[1];
      }
    }
    // B operands per group: p * scale (fp16)
    half8_t bv[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t* b32 = reinterpret_cast<uint32_t*>(&bv[g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = i >> 1, hw = i & 1;
        // group g's scale pair (tokens 2hw, 2hw+1 of the quad) is word 2g + hw of the 32 bytes
        const uint32_t sw = (g < 2) ? vs[p][0][2 * g + hw] : vs[p][1][2 * (g - 2) + hw];
        b32[i] = mul_h2(pp[i], sw);
      }
    }
    const uint32_t v00 = c_cur[0][2], v01 = c_cur[0][3], v10 = c_cur[1][2], v11 = c_cur[1][3];
    const uint32_t v00s = v00 >> 6, v01s = v01 >> 6, v10s = v10 >> 6, v11s = v11 >> 6;
#define OSCAR_VBLOCK(M)                                                                   \
    {                                                                                     \
      half8_t av;                                                                         \
      uint32_t* a32 = reinterpret_cast<uint32_t*>(&av);                                   \
      a32[0] = field_pair<M>(v00, v00s);                                                  \
      a32[1] = field_pair<M>(v01, v01s);                                                  \
      a32[2] = field_pair<M>(v10, v10s);                                                  \
      a32[3] = field_pair<M>(v11, v11s);                                                  \
      acc_o[M] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv[(M) >> 1], acc_o[M], 0, 0, 0); \
    }
    OSCAR_VBLOCK(0) OSCAR_VBLOCK(1) OSCAR_VBLOCK(2) OSCAR_VBLOCK(3)
    OSCAR_VBLOCK(4) OSCAR_VBLOCK(5) OSCAR_VBLOCK(6) OSCAR_VBLOCK(7)
#undef OSCAR_VBLOCK
    {
      half8_t az, bz;
      uint32_t* az32 = reinterpret_cast<uint32_t*>(&az);
      uint32_t* bz32 = reinterpret_cast<uint32_t*>(&bz);
      az32[0] = vz[0][0]; az32[1] = vz[0][1]; az32[2] = vz[1][0]; az32[3] = vz[1][1];
      bz32[0] = pp[0]; bz32[1] = pp[1]; bz32[2] = pp[2]; bz32[3] = pp[3];
      acc_z = __builtin_amdgcn_mfma_f32_16x16x32_f16(az, bz, acc_z, 0, 0, 0);
    }
  };
  // The prefetch is issued unconditionally (past the end it re-reads this
  // wave's last pair, an L2 hit) so that every body sees the same number of
  // loads in flight and waits only for its own pair's.
  const int last_pr = npairs > wave ? wave + ((npairs - 1 - wave) / 4) * 4 : wave;
  while (pr < npairs) {
    issue(min(pr + 8, last_pr), cC, mC);
    body(cA, mA);
    pr += 4;
    if (pr >= npairs) break;
    issue(min(pr + 8, last_pr), cA, mA);
    body(cB, mB);
    pr += 4;
    if (pr >= npairs) break;
    issue(min(pr + 8, last_pr), cB, mB);
    body(cC, mC);
    pr += 4;
  }
  // ---- wave epilogue: true-unit rotated outputs to LDS
  l_run = rows_sum(l_run);
  if (qa == 0) {
    sm.wm[wave][x] = m_run;
    sm.wl[wave][x] = l_run;
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.zs[wave][r][x] = acc_z[r];
  }
  __builtin_amdgcn_wave_barrier();
  if (x < G) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float sc = ldexpf(1.0f, 24 - 2 * field_shift(m));
      const float zg = sm.zs[wave][m >> 1][x];
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.wo[wave][x][16 * m + 4 * qa + r] = fmaf(acc_o[m][r], sc, zg);
    }
  }
}

template <int G>
__global__ __launch_bounds__(256) void decode_int2_kernel(DecodeArgs a) {
  __shared__ DecodeSmem<G> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // XCD-aware order: consecutive workgroup ids go to different XCDs, so work
  // item = xcd * grid_per_xcd + local keeps a group's splits on one XCD.
  const int item = (blockIdx.x & 7) * a.grid_per_xcd + (blockIdx.x >> 3);
  const int n_split_total = a.n_tile_splits + a.n_hist_splits;
  if (item >= a.n_groups_total * n_split_total) return;
  const int grp = item / n_split_total, split = item % n_split_total;
  const int b = grp / a.hkv, hk = grp % a.hkv;
  const int slot = a.seq_slot ? a.seq_slot[b] : b;
  const int n = a.seq_len[b];
  const int hist_len = max(0, n - kSink - kRecent);
  const int n_hist_pages = (hist_len + kPage - 1) / kPage;
  const int act_hist = (n_hist_pages + a.pages_per_split - 1) / a.pages_per_split;
  const int n_sink_used = min(n, kSink);
  const int n_recent_used = min(max(n - kSink, 0), kRecent);
  const int n_tile = n_sink_used + n_recent_used;
  const int act_tile = (n_tile + kTileTokens - 1) / kTileTokens;
  const bool is_tile = split < a.n_tile_splits;
  const int hs = split - a.n_tile_splits;
  if (is_tile ? (split >= act_tile) : (hs >= act_hist)) return;

  float* part_base = a.partials + (size_t)grp * n_split_total * G * kPartStride;
  if (is_tile) {
    const int u0 = split * kTileTokens;
    const int recent_first = max(kSink, n - kRecent);
    const size_t sink_base = ((size_t)slot * a.hkv + hk) * kSink;
    const size_t ring_base = ((size_t)slot * a.hkv + hk) * kRecent;
    auto row = [&](const uint16_t* sink, const uint16_t* ring, int uu) -> const uint16_t* {
      const int u = u0 + uu;
      if (u < n_sink_used) return sink + (sink_base + u) * kD;
      const int pos = recent_first + (u - n_sink_used);
      return ring + (ring_base + ((pos - kSink) & (kRecent - 1))) * kD;
    };
    bf16_span_wave<G>(a.q + ((size_t)b * a.hkv * G + hk * G) * kD, min(kTileTokens, n_tile - u0),
                      [&](int uu) { return row(a.sink_k, a.recent_k, uu); },
                      [&](int uu) { return row(a.sink_v, a.recent_v, uu); }, sm, wave, lane);
  } else {
    const int pg_begin = hs * a.pages_per_split;
    const int pg_end = min(pg_begin + a.pages_per_split, n_hist_pages);
    const int32_t* pt_row = a.page_table + (size_t)slot * a.max_pages;
    // page ids of this wave's pairs (pairs wave, wave + 4, ...): one load per lane
    const int32_t ids = pt_row[pg_begin + min(2 * (wave + 4 * (lane >> 1)) + (lane & 1), pg_end - pg_begin - 1)];
    // q . R_K operands first (thread (c4, rs) takes output columns
    // [4 c4, 4 c4 + 4) and rows [16 rs, 16 rs + 16) of R_K: 16 float4 loads),
    // then this wave's first two page pairs: the prologue waits only for the
    // older loads, so the loop is entered with exactly the page loads in
    // flight that every later iteration also has.
    const uint16_t* qg = a.q + ((size_t)b * a.hkv * G + hk * G) * kD;
    const int c4 = tid & 31, rs = tid >> 5;
    float4 rq[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) rq[e] = *reinterpret_cast<const float4*>(a.rot_k + (size_t)(16 * rs + e) * kD + 4 * c4);
    constexpr int kQPer = (G * kD + 255) / 256;
    uint16_t qv[kQPer];
#pragma unroll
    for (int e = 0; e < kQPer; ++e) qv[e] = qg[min(tid + 256 * e, G * kD - 1)];   // unconditional
    u32x4_t c_first[2] = {}, c_second[2] = {};
    u32x2_t m_first[2] = {}, m_second[2] = {};
    // unconditional (the ids are clamped to pages of this split): the same
    // loads are in flight on every path into the loop
    // (kept in the loop's per-pair issue order, so the wait counts the loop
    // computes for its first iteration are exact)
    issue_pair(a, ids, hk, 0, lane, c_first, m_first);
    __builtin_amdgcn_sched_barrier(0);
    issue_pair(a, ids, hk, 1, lane, c_second, m_second);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < kQPer; ++e) {
      const int idx = tid + 256 * e;
      if (idx < G * kD) sm.q[idx / kD][idx % kD] = bf16_bits_to_float(qv[e]);
    }
    __syncthreads();
    // lanes l and l + 32 of a wave hold row slices 2 wave and 2 wave + 1 of
    // the same columns: add them with one lane swap, then sum the four waves
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const float4 q4 = *reinterpret_cast<const float4*>(&sm.q[h][16 * rs + 4 * e4]);
        const float qe[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 r = rq[4 * e4 + i];
          acc.x = fmaf(qe[i], r.x, acc.x);
          acc.y = fmaf(qe[i], r.y, acc.y);
          acc.z = fmaf(qe[i], r.z, acc.z);
          acc.w = fmaf(qe[i], r.w, acc.w);
        }
      }
      acc.x = half_swap_sum(acc.x);
      acc.y = half_swap_sum(acc.y);
      acc.z = half_swap_sum(acc.z);
      acc.w = half_swap_sum(acc.w);
      if (lane < 32) *reinterpret_cast<float4*>(&sm.wo[wave][h][4 * c4]) = acc;
    }
    __syncthreads();
    for (int idx = tid; idx < G * kD; idx += 256) {
      const int h = idx / kD, jj = idx % kD;
      sm.qr[h][jj] = (sm.wo[0][h][jj] + sm.wo[1][h][jj]) + (sm.wo[2][h][jj] + sm.wo[3][h][jj]);
    }
    __syncthreads();
    for (int h = wave; h < G; h += 4) {
      const float v0 = sm.qr[h][lane], v1 = sm.qr[h][lane + 64];
      const float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1))) * kC0;
      int e2 = 0;
      frexpf(amax, &e2);
      const int s_exp = amax > 0.0f ? min(15 - e2, 100) : 0;
      // group sums: lanes 0..31 hold groups 0 (v0) and 2 (v1), lanes 32..63 groups 1 and 3
      float g0 = v0, g1 = v1;
      for (int m = 16; m >= 1; m >>= 1) { g0 += __shfl_xor(g0, m); g1 += __shfl_xor(g1, m); }
      if (lane == 0) { sm.sexp[h] = (float)s_exp; sm.qs[h][0] = g0; sm.qs[h][2] = g1; }
      if (lane == 32) { sm.qs[h][1] = g0; sm.qs[h][3] = g1; }
    }
    __syncthreads();
    hist_wave<G>(a, sm, ids, hk, hist_len, pg_begin, pg_end, wave, lane, c_first, m_first, c_second, m_second);
  }
  float* rec = part_base + (size_t)split * G * kPartStride;
  store_split<G>(sm, rec, tid);

  // ---- completion ticket: the last workgroup of the group merges
  if (!finish_ticket<G>(sm, &a.counters[grp], (uint32_t)(act_tile + act_hist), tid)) return;
  // active splits: tile 0..act_tile-1 (unrotated), history n_tile_splits + 0..act_hist-1 (rotated)
  merge_group<G>(sm, part_base, (uint32_t)(n_split_total * G * kPartStride * 4), act_tile + act_hist, act_tile,
                 [&](int k) { return k < act_tile ? k : a.n_tile_splits + (k - act_tile); }, a.rot_v,
                 a.out + ((size_t)b * a.hkv * G + hk * G) * kD, tid, wave, lane);
  if (tid == 0) a.counters[grp] = 0u;
}

DecodePlan plan_decode(int batch, int hkv, int group, int max_seq_len) {
  DecodePlan p{};
  const int max_hist = max(0, max_seq_len - kSink - kRecent);
  const int max_pages = (max_hist + kPage - 1) / kPage;
  const long total_pages = (long)batch * hkv * max_pages;
  // aim at roughly two workgroups per compute unit (256 CUs)
  long pps = (total_pages + 479) / 480;
  pps = ((pps + 7) / 8) * 8;
  if (pps < 8) pps = 8;
  if (pps > kMaxPagesPerSplit) pps = kMaxPagesPerSplit;
  while (max_pages > 0 && (max_pages + pps - 1) / pps > kMaxSplits - 4 && pps < kMaxPagesPerSplit) pps += 8;
  p.ok = max_pages == 0 || (max_pages + pps - 1) / pps <= kMaxSplits - 4;
  p.pages_per_split = (int)pps;
  p.n_hist_splits = max_pages > 0 ? (int)((max_pages + pps - 1) / pps) : 0;
  const int max_tile = min(max_seq_len, kSink + kRecent);
  p.n_tile_splits = (max_tile + kTileTokens - 1) / kTileTokens;
  p.n_splits_total = p.n_hist_splits + p.n_tile_splits;
  p.n_work = batch * hkv * p.n_splits_total;
  p.grid = ((p.n_work + 7) / 8) * 8;
  p.partial_floats = (size_t)batch * hkv * p.n_splits_total * group * kPartStride;
  p.workspace_bytes = p.partial_floats * sizeof(float) + (size_t)batch * hkv * sizeof(uint32_t);
  (void)group;
  return p;
}

hipError_t launch_decode(const DecodeArgs& a, int group, int grid, hipStream_t st) {
  switch (group) {
    case 1: hipLaunchKernelGGL(decode_int2_kernel<1>, dim3(grid), dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL(decode_int2_kernel<2>, dim3(grid), dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL(decode_int2_kernel<4>, dim3(grid), dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL(decode_int2_kernel<8>, dim3(grid), dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace oscar
