// Single-token decode attention over the three-tier pool (BF16 sink, INT2
// history, BF16 recent) -- the fused INT2 attention of "OSCAR: Offline
// Spectral Covariance-Aware Rotation for 2-bit KV Cache Quantization"
// (gist.science), 2.2 B "Kernel-Integration" (unpack, dequantise, inverse
// rotation and attention in one kernel, paged cache), and of
// "OSCAR：面向2-bit KV缓存量化的谱协方差感知旋转方法" (zingnex.cn), section
// 自定义INT2注意力内核.  Tiers: "大模型KV Cache 2bit量化实战" (yunpan.plus), 三.1.
//
// Two launches per call.  Workgroups of the first are "work items" of one
// (sequence, KV head) group: BF16 tile splits (sink + recent tokens) and
// history splits (runs of INT2 pages).  Each writes a partial (running max m,
// sum l and unnormalised output, all G query heads of the group) to the
// workspace; the merge kernel then combines them by log-sum-exp, rotates the
// history part back with R_V^T, and writes the fp32 output.
//
// History scoring works in the rotated space: with q' = q . R_K and the
// dequantised key k'_t = s_{t,g} c_{t,j} + z_{t,g},
//   q . k~_t = sum_g s_{t,g} sum_{j in g} q'_j c_{t,j} + sum_g z_{t,g} sum_{j in g} q'_j.
// The per-group code sums run on the matrix cores: 2-bit codes are placed in
// fp16 operands as exact subnormals (one AND per two codes, c * 4^f * 2^-24)
// and q' is split into fp16 hi + lo halves: two operand columns per head (up
// to 8 heads), or two products into one tile with a head per column (16).
// The value side accumulates p_t s_{t,g} c_{t,j} on the matrix cores and
// p_t z_{t,g} with one more small product, all in the rotated space.
#include "attn_common.h"
#include "launchers.h"
#include "quant_token.h"

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

// INT4: nibble field f (0..3) of both 16-bit halves of w as fp16 subnormals
// c * 16^(f & 1) * 2^-24 (w8 = w >> 8 brings nibbles 2 and 3 down).
template <int F>
__device__ __forceinline__ uint32_t nibble_pair(uint32_t w, uint32_t w8) {
  constexpr uint32_t mask = (F & 1) ? 0x00F000F0u : 0x000F000Fu;
  return (F < 2 ? w : w8) & mask;
}

// One page's codes as a lane loads them: INT2, K codes in words 0-1 and V
// codes in words 2-3 of one 16-byte chunk; INT4, a 16-byte K chunk and a
// 16-byte V chunk.
template <int kBits>
struct PageCodes {
  u32x4_t w;
};
template <>
struct PageCodes<4> {
  u32x4_t k, v;
};

// A wave walks its share of a split in steps of kStepPages pages (64
// tokens, 6 KiB of INT2 blocks): wave w takes steps w, w + 4, ...  While one
// step is processed the next one is in flight.  The two steps' registers
// take the kernel past three workgroups per compute unit; the decode plan
// fills two.
constexpr int kStepPages = 4;

// Shared memory of one workgroup (256 threads = 4 waves).
template <int G>
struct alignas(16) DecodeSmem : SplitSmem<G> {
  float q[G][kD];            // q (fp32)
  float qr[G][kD];           // q' = q . R_K
  float sexp[G];             // S_h: q' operands are scaled by 2^S_h
  float qs[G][kGroups];      // per-group sums of q'
  uint8_t meta[4][kStepPages][512];   // per wave, one step's scale/zero metadata
  float zs[4][kGroups][16];  // per-wave V zero-point accumulators
};

// ---------------------------------------------------------------------------
// Per-wave partial of a history split: pages [pg_begin, pg_end) of the
// sequence's history (hist_len valid tokens).
// ---------------------------------------------------------------------------
// Loads of one step for a wave: codes (16 B per lane per page) and
// scale/zero metadata (8 B per lane per page), as buffer loads whose base is
// the page block (scalar address arithmetic only).  ids: this wave's page
// ids, lane kStepPages k + i holding page kStepPages (wave + 4k) + i of the
// split (clamped to its last page), so the k-th step of the wave needs no
// memory access for its page ids.
template <int kBits>
__device__ __forceinline__ void issue_step(const DecodeArgs& a, int32_t ids, int hk, int k, int lane,
                                           PageCodes<kBits>* c, u32x2_t* md) {
  constexpr int kBytes = block_bytes(kBits);
#pragma unroll
  for (int i = 0; i < kStepPages; ++i) {
    const int pid = __builtin_amdgcn_readlane(ids, kStepPages * k + i);
    const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.hist) + ((size_t)pid * a.hkv + hk) * kBytes,
                                                     (short)0, kBytes, 0x00020000);
    if constexpr (kBits == 4) {
      c[i].k = __builtin_amdgcn_raw_buffer_load_b128(r, 16 * lane, 0, 0);
      c[i].v = __builtin_amdgcn_raw_buffer_load_b128(r, kVCodeOff4 + 16 * lane, 0, 0);
    } else {
      c[i].w = __builtin_amdgcn_raw_buffer_load_b128(r, 16 * lane, 0, 0);
    }
    md[i] = __builtin_amdgcn_raw_buffer_load_b64(r, 1024 + meta_shift(kBits) + 8 * lane, 0, 0);
  }
}

// masked score (finite, so that a zero weight times it stays 0)
constexpr float kMasked = -1.0e30f;

template <int G, int kBits>
__device__ void hist_wave(const DecodeArgs& a, DecodeSmem<G>& sm, int32_t ids, int hk, int hist_len,
                          int pg_begin, int pg_end, int wave, int lane, const PageCodes<kBits>* c_first,
                          const u32x2_t* m_first) {
  const int x = lane & 15, qa = lane >> 4;
  // ---- score operands: q' in fp16 hi and lo halves
  // Up to 8 heads: one operand set, hi halves in columns [0, G) and lo halves
  // in [G, 2G); one rotate by 8 lanes then pairs the halves of every head.
  // 16 heads: head = column, and two operand sets (hi, then lo) whose
  // products accumulate into one tile, so that the scale and the scores are
  // applied once per head.
  constexpr int kSets = G > 8 ? 2 : 1;
  half8_t bq[kSets][4];
  float be;
#pragma unroll
  for (int st = 0; st < kSets; ++st) {
    const bool hi_col = kSets == 2 ? st == 0 : x < G;
    const bool col_used = kSets == 2 ? true : x < 2 * G;
    const int col_head = kSets == 2 ? x : (!col_used ? 0 : (x < G ? x : x - G));
    const float col_scale = ldexpf(kC0, (int)sm.sexp[col_head]);
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int j = 32 * g + 8 * qa + 2 * i + hf;
          // the code of channel j enters the product as c * 4^sh * 2^-24
          // (INT2) or c * 16^(i & 1) * 2^-24 (INT4): q' carries the inverse
          const int lsh = kBits == 4 ? 4 * (i & 1) : 2 * field_shift(4 * (g & 1) + i);
          const float v = ldexpf(sm.qr[col_head][j] * col_scale, -lsh);
          const _Float16 hi = (_Float16)v;
          const _Float16 e = hi_col ? hi : (_Float16)(v - (float)hi);
          bq[st][g][2 * i + hf] = col_used ? e : (_Float16)0.0f;
        }
    // zero-point term operand (fp32 product, 4 groups = K of 4), hi columns only
    if (st == 0)
      be = (hi_col && col_used) ? ldexpf(sm.qs[col_head][qa] * kC0, (int)sm.sexp[col_head] - 24) : 0.0f;
  }
  // matrix-core units -> log2 units; 0 for the columns that hold no head, so
  // that their (unused) scores stay at 0 and never move the running maximum
  const float mult = (x < G) ? ldexpf(1.0f, 24 - (int)sm.sexp[x]) : 0.0f;
  // row 4 of the value zero-point operand is all ones: that product row
  // accumulates sum_t p_t, the softmax denominator
  const uint32_t ones_row = (x == 4) ? 0x3C003C00u : 0u;

  float4_t acc_o[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc_o[m] = (float4_t){0.f, 0.f, 0.f, 0.f};
  float4_t acc_z = (float4_t){0.f, 0.f, 0.f, 0.f};
  float m_run = kMInit;

  const int nsteps = (pg_end - pg_begin + kStepPages - 1) / kStepPages;
  uint8_t* mbuf = &sm.meta[wave][0][0];

  // two-stage prefetch ring: while step st is processed, step st + 4 of this
  // wave is in flight (the first step was issued before the prologue)
  PageCodes<kBits> cA[kStepPages], cB[kStepPages];
  u32x2_t mA[kStepPages], mB[kStepPages];
#pragma unroll
  for (int i = 0; i < kStepPages; ++i) { cA[i] = c_first[i]; mA[i] = m_first[i]; }
  auto issue = [&](int st_, PageCodes<kBits>* c, u32x2_t* md) {
    issue_step<kBits>(a, ids, hk, (st_ - wave) >> 2, lane, c, md);
  };
  int st = wave;
  // A partial step (only the last step of a sequence) has tokens past the end
  // of the history: their scores are masked, so their weights are exactly 0.
  // Their slots hold either zeros or bytes an earlier demotion wrote (finite
  // scales and zeros), so 0 times them stays 0.
  auto body = [&](const PageCodes<kBits>* c_cur, const u32x2_t* m_cur) __attribute__((always_inline)) {
    const int pg0 = pg_begin + kStepPages * st;
    const int n_valid = min(kStepPages, pg_end - pg0);
    // valid tokens of the step: token t of page p is history index 16 (pg0 + p) + t
    const int base_tok = 16 * pg0;
    const int lim = min(hist_len - base_tok, 16 * n_valid);
    const bool partial = lim < 16 * kStepPages;
    // stage this step's metadata in LDS (wave-private)
#pragma unroll
    for (int p = 0; p < kStepPages; ++p) *reinterpret_cast<u32x2_t*>(mbuf + 512 * p + 8 * lane) = m_cur[p];
    __builtin_amdgcn_wave_barrier();

    // ---------------- scores
    float sc[kStepPages][4];
    float4_t cacc_all[kStepPages];
#pragma unroll
    for (int p = 0; p < kStepPages; ++p) {
      const uint8_t* mp = mbuf + 512 * p;
      // sum_g zero[t][g] * (scaled group sums of q'), t = lane's row token
      const _Float16 zk = *reinterpret_cast<const _Float16*>(mp + 128 + 8 * x + 2 * qa);
      half8_t ak[4];
      uint32_t* ak32 = reinterpret_cast<uint32_t*>(ak);
      if constexpr (kBits == 4) {
        // word g holds group g's eight channels of this lane: one operand
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t w = c_cur[p].k[g], w8 = w >> 8;
          ak32[4 * g + 0] = nibble_pair<0>(w, w8);
          ak32[4 * g + 1] = nibble_pair<1>(w, w8);
          ak32[4 * g + 2] = nibble_pair<2>(w, w8);
          ak32[4 * g + 3] = nibble_pair<3>(w, w8);
        }
      } else {
        const uint32_t w0 = c_cur[p].w[0], w1 = c_cur[p].w[1];
        const uint32_t w0s = w0 >> 6, w1s = w1 >> 6;
        ak32[0] = field_pair<0>(w0, w0s);  ak32[1] = field_pair<1>(w0, w0s);
        ak32[2] = field_pair<2>(w0, w0s);  ak32[3] = field_pair<3>(w0, w0s);
        ak32[4] = field_pair<4>(w0, w0s);  ak32[5] = field_pair<5>(w0, w0s);
        ak32[6] = field_pair<6>(w0, w0s);  ak32[7] = field_pair<7>(w0, w0s);
        ak32[8] = field_pair<0>(w1, w1s);  ak32[9] = field_pair<1>(w1, w1s);
        ak32[10] = field_pair<2>(w1, w1s); ak32[11] = field_pair<3>(w1, w1s);
        ak32[12] = field_pair<4>(w1, w1s); ak32[13] = field_pair<5>(w1, w1s);
        ak32[14] = field_pair<6>(w1, w1s); ak32[15] = field_pair<7>(w1, w1s);
      }
      // scales of tokens 4qa..4qa+3 (K scale area [token][group])
      const u32x4_t s01 = *reinterpret_cast<const u32x4_t*>(mp + 32 * qa);
      const u32x4_t s23 = *reinterpret_cast<const u32x4_t*>(mp + 32 * qa + 16);
      const _Float16* sh0 = reinterpret_cast<const _Float16*>(&s01);
      const _Float16* sh1 = reinterpret_cast<const _Float16*>(&s23);
      float4_t& cacc = cacc_all[p];
      cacc = __builtin_amdgcn_mfma_f32_16x16x4f32((float)zk, be, (float4_t){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      float4_t d[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        d[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak[g], bq[0][g], (float4_t){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        if constexpr (kSets == 2) d[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak[g], bq[1][g], d[g], 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const _Float16* sr = (r < 2) ? sh0 + 4 * r : sh1 + 4 * (r - 2);
#pragma unroll
        for (int g = 0; g < 4; ++g) cacc[r] = fmaf((float)sr[g], d[g][r], cacc[r]);
      }
    }
    // hi + lo columns (up to 8 heads), once every page's products are in
    // (the lane moves then read registers written well before)
#pragma unroll
    for (int p = 0; p < kStepPages; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (kSets == 2) {
          sc[p][r] = cacc_all[p][r];
        } else {
          const float other = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
              0u, __float_as_uint(cacc_all[p][r]), 0x120 + (16 - G), 0xF, 0xF, false));
          sc[p][r] = cacc_all[p][r] + other;
        }
      }
    if (partial) {
#pragma unroll
      for (int p = 0; p < kStepPages; ++p)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * p + 4 * qa + r >= lim) sc[p][r] = kMasked;
    }
    // ---------------- online softmax over the step's tokens
    float mx = sc[0][0];
#pragma unroll
    for (int p = 0; p < kStepPages; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[p][r]);
    // A column's maximum needs its four lane quarters only when one of them
    // passes the running maximum (mult >= 0); otherwise the step leaves the
    // maximum where it was and nothing is rescaled.
    if (__builtin_amdgcn_ballot_w64(mx * mult > m_run) != 0ull) {
      const float m_new = fmaxf(m_run, rows_max(mx) * mult);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int m = 0; m < 8; ++m) acc_o[m] *= alpha;
      acc_z *= alpha;
      m_run = m_new;
    }
    // ---------------- values, one page pair (32 tokens = one k block) at a time
#pragma unroll
    for (int j = 0; j < kStepPages / 2; ++j) {
      float pv[2][4];
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int r = 0; r < 4; ++r) pv[p][r] = __builtin_amdgcn_exp2f(fmaf(sc[2 * j + p][r], mult, -m_run));
      uint32_t pp[4];                 // fp16 p pairs: (page i>>1, tokens 2(i&1), +1)
      pp[0] = pack_h2(pv[0][0], pv[0][1]);
      pp[1] = pack_h2(pv[0][2], pv[0][3]);
      pp[2] = pack_h2(pv[1][0], pv[1][1]);
      pp[3] = pack_h2(pv[1][2], pv[1][3]);
      const uint8_t* mq = mbuf + 512 * (2 * j);
      // V scales [token/4][group][token%4]: lane reads its token quad of both pages
      u32x4_t vs[2][2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        vs[p][0] = *reinterpret_cast<const u32x4_t*>(mq + 512 * p + 256 + 32 * qa);
        vs[p][1] = *reinterpret_cast<const u32x4_t*>(mq + 512 * p + 256 + 32 * qa + 16);
      }
      u32x2_t vz[2];
#pragma unroll
      for (int p = 0; p < 2; ++p)
        vz[p] = (x < 4) ? *reinterpret_cast<const u32x2_t*>(mq + 512 * p + 384 + 32 * qa + 8 * x)
                        : (u32x2_t){ones_row, ones_row};
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
      if constexpr (kBits == 4) {
        // block M (channels 16M + row): nibble M & 3 of words 2(M >> 2) and
        // 2(M >> 2) + 1 of each page's V chunk (tokens 4qa + 0, 1 and + 2, 3)
        uint32_t vw[2][4], vw8[2][4];
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            vw[p][e] = c_cur[2 * j + p].v[e];
            vw8[p][e] = vw[p][e] >> 8;
          }
#define OSCAR_VBLOCK4(M)                                                                  \
        {                                                                                 \
          half8_t av;                                                                     \
          uint32_t* a32 = reinterpret_cast<uint32_t*>(&av);                               \
          constexpr int e0 = 2 * ((M) >> 2);                                              \
          a32[0] = nibble_pair<(M) & 3>(vw[0][e0], vw8[0][e0]);                           \
          a32[1] = nibble_pair<(M) & 3>(vw[0][e0 + 1], vw8[0][e0 + 1]);                   \
          a32[2] = nibble_pair<(M) & 3>(vw[1][e0], vw8[1][e0]);                           \
          a32[3] = nibble_pair<(M) & 3>(vw[1][e0 + 1], vw8[1][e0 + 1]);                   \
          acc_o[M] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv[(M) >> 1], acc_o[M], 0, 0, 0); \
        }
        OSCAR_VBLOCK4(0) OSCAR_VBLOCK4(1) OSCAR_VBLOCK4(2) OSCAR_VBLOCK4(3)
        OSCAR_VBLOCK4(4) OSCAR_VBLOCK4(5) OSCAR_VBLOCK4(6) OSCAR_VBLOCK4(7)
#undef OSCAR_VBLOCK4
      } else {
        const uint32_t v00 = c_cur[2 * j].w[2], v01 = c_cur[2 * j].w[3], v10 = c_cur[2 * j + 1].w[2],
                       v11 = c_cur[2 * j + 1].w[3];
        const uint32_t v00s = v00 >> 6, v01s = v01 >> 6, v10s = v10 >> 6, v11s = v11 >> 6;
#define OSCAR_VBLOCK(M)                                                                   \
        {                                                                                 \
          half8_t av;                                                                     \
          uint32_t* a32 = reinterpret_cast<uint32_t*>(&av);                               \
          a32[0] = field_pair<M>(v00, v00s);                                              \
          a32[1] = field_pair<M>(v01, v01s);                                              \
          a32[2] = field_pair<M>(v10, v10s);                                              \
          a32[3] = field_pair<M>(v11, v11s);                                              \
          acc_o[M] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv[(M) >> 1], acc_o[M], 0, 0, 0); \
        }
        OSCAR_VBLOCK(0) OSCAR_VBLOCK(1) OSCAR_VBLOCK(2) OSCAR_VBLOCK(3)
        OSCAR_VBLOCK(4) OSCAR_VBLOCK(5) OSCAR_VBLOCK(6) OSCAR_VBLOCK(7)
#undef OSCAR_VBLOCK
      }
      {
        // rows 0..3: sum_t p_t zero[t][g]; row 4: sum_t p_t
        half8_t az, bz;
        uint32_t* az32 = reinterpret_cast<uint32_t*>(&az);
        uint32_t* bz32 = reinterpret_cast<uint32_t*>(&bz);
        az32[0] = vz[0][0]; az32[1] = vz[0][1]; az32[2] = vz[1][0]; az32[3] = vz[1][1];
        bz32[0] = pp[0]; bz32[1] = pp[1]; bz32[2] = pp[2]; bz32[3] = pp[3];
        acc_z = __builtin_amdgcn_mfma_f32_16x16x32_f16(az, bz, acc_z, 0, 0, 0);
      }
    }
  };
  // The prefetch is issued unconditionally (past the end it re-reads this
  // wave's last step, an L2 hit) so that every body sees the same number of
  // loads in flight and waits only for its own step's.
  const int last_st = nsteps > wave ? wave + ((nsteps - 1 - wave) / 4) * 4 : wave;
  while (st < nsteps) {
    issue(min(st + 4, last_st), cB, mB);
    body(cA, mA);
    st += 4;
    if (st >= nsteps) break;
    issue(min(st + 4, last_st), cA, mA);
    body(cB, mB);
    st += 4;
  }
  // ---- wave epilogue: true-unit rotated outputs to LDS
  if (qa == 0) {
    sm.wm[wave][x] = m_run;
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.zs[wave][r][x] = acc_z[r];
  }
  if (qa == 1) sm.wl[wave][x] = acc_z[0];
  __builtin_amdgcn_wave_barrier();
  if (x < G) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      // codes of block m entered as c * 4^field_shift(m) (INT2) or
      // c * 16^(m & 1) (INT4) times 2^-24
      const float scl = ldexpf(1.0f, 24 - (kBits == 4 ? 4 * (m & 1) : 2 * field_shift(m)));
      const float zg = sm.zs[wave][m >> 1][x];
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.wo[wave][x][16 * m + 4 * qa + r] = fmaf(acc_o[m][r], scl, zg);
    }
  }
}

// The fused step's demotion, by the history split that owns the newest
// history token (history index hidx = n - 321, position n - 257): the token
// leaves the ring slot that position n - 1 (the step's new token) takes.
// The workgroup reads the leaving K and V rows, writes the new token into
// the slot, rotates the leaving token by R_K and R_V, clips, quantises and
// stores it exactly as oscar_append does (same routine, same association),
// and records its attention from the dequantised values in the rotated
// space (record slot 4: score q' . k~' for every query head, weight 1,
// value v~').  ([yunpan] 三.1 append before attend, 三.2 demotion.)
// rq holds R_K's row slices on entry (loaded for q . R_K) and is reused for
// R_V.  Every thread of the workgroup calls it.
template <int G, int kBits>
__device__ void demote_in_split(const DecodeArgs& a, DecodeSmem<G>& sm, float4 (&rq)[16], int b, int slot, int hk,
                                int n, int hidx, int tid, int wave, int lane) {
  // scratch in the (not yet used) metadata staging area of the page walk
  float* dx = reinterpret_cast<float*>(&sm.meta[0][0][0]);          // [2][128] leaving K, V
  float* dpart = dx + 2 * kD;                                        // [4][128] rotation partials
  uint32_t* dsh = reinterpret_cast<uint32_t*>(dpart + 4 * kD);       // [32] packing words
  const int p = n - 1;
  const size_t ring_row = (((size_t)slot * a.hkv + hk) * kRecent + ((p - kSink) & (kRecent - 1))) * kD;
  const size_t new_row = ((size_t)b * a.hkv + hk) * kD;
  const int pid = a.page_table[(size_t)slot * a.max_pages + (hidx >> 4)];
  uint32_t fresh = 0u;
  if (tid < kD) {
    const int which = tid >> 6, w = tid & 63;
    const uint32_t old = reinterpret_cast<const uint32_t*>((which ? a.recent_v : a.recent_k) + ring_row)[w];
    fresh = reinterpret_cast<const uint32_t*>((which ? a.v_new : a.k_new) + new_row)[w];
    dx[which * kD + 2 * w] = bf16_bits_to_float(old & 0xFFFFu);
    dx[which * kD + 2 * w + 1] = bf16_bits_to_float(old >> 16);
  }
  __syncthreads();
  // the leaving token is in LDS (its loads completed): the slot takes the new token
  // (the pool's tiers are writable device memory; the decode reads them through const pointers)
  if (tid < kD) {
    uint16_t* row = const_cast<uint16_t*>((tid >> 6) ? a.recent_v : a.recent_k) + ring_row;
    reinterpret_cast<uint32_t*>(row)[tid & 63] = fresh;
  }
  uint8_t* blk = const_cast<uint8_t*>(a.hist) + ((size_t)pid * a.hkv + hk) * block_bytes(kBits);
  const float* tau_k = a.clip_k + (size_t)hk * a.clip_kv_stride;
  const float* tau_v = a.clip_v + (size_t)hk * a.clip_kv_stride;
  rotate_partial(dx, rq, dpart, tid);
  __syncthreads();
  float y = tid < kD ? clip_value(rotated_channel(dpart, tid), tau_k[tid]) : 0.0f;
  // (the quantiser's barriers order every read of dpart before the V rotation rewrites it)
  const float kdq = quantize_pack_channel_per_thread(y, false, blk, hidx & 15, dsh, kBits);
  load_rot_slices(a.rot_v + (size_t)hk * a.rot_kv_stride, rq, tid);
  rotate_partial(dx + kD, rq, dpart, tid);
  __syncthreads();
  y = tid < kD ? clip_value(rotated_channel(dpart, tid), tau_v[tid]) : 0.0f;
  const float vdq = quantize_pack_channel_per_thread(y, true, blk, hidx & 15, dsh, kBits);
  // the demoted token's record: dequantised key (rotated) for the scores,
  // dequantised value row for every column
  if (tid < kD) {
    dx[tid] = kdq;
#pragma unroll
    for (int h = 0; h < G; ++h) sm.wo[4][h][tid] = vdq;
  }
  __syncthreads();
  for (int h = wave; h < G; h += 4) {
    const float d = wave_sum(sm.qr[h][lane] * dx[lane] + sm.qr[h][lane + 64] * dx[lane + 64]);
    if (lane == 0) {
      sm.wm[4][h] = d * kC0;          // log2 units, as the page walk's scores
      sm.wl[4][h] = 1.0f;
    }
  }
  __syncthreads();                   // dx (metadata staging) is free again for the page walk
}

template <int G, int kBits>
__device__ __forceinline__ void decode_body(const DecodeArgs& a, DecodeSmem<G>& sm) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // XCD-aware order: consecutive workgroup ids go to different XCDs, so work
  // item = xcd * grid_per_xcd + local keeps a group's splits on one XCD.
  // When the grid takes more than one round of workgroup slots (tiles_last:
  // then the groups divide evenly over the XCDs), each XCD takes whole
  // groups and dispatches their history splits first and their tile splits
  // last, so that the short tile workgroups fill the slots the history
  // splits leave at the end.
  const int n_split_total = a.n_tile_splits + a.n_hist_splits;
  const int local = blockIdx.x >> 3;
  int grp, split;
  if (a.tiles_last) {
    const int gx = a.grid_per_xcd / n_split_total;     // groups per XCD
    const int n_hist_x = gx * a.n_hist_splits;
    const int g0 = (blockIdx.x & 7) * gx;
    if (local < n_hist_x) {
      grp = g0 + local / a.n_hist_splits;
      split = a.n_tile_splits + local % a.n_hist_splits;
    } else {
      grp = g0 + (local - n_hist_x) / a.n_tile_splits;
      split = (local - n_hist_x) % a.n_tile_splits;
    }
  } else {
    const int item = (blockIdx.x & 7) * a.grid_per_xcd + local;
    grp = item / n_split_total;
    split = item % n_split_total;
  }
  if (grp >= a.n_groups_total) return;
  // group = (sequence b, KV head hk, column group cg); column x of the group
  // is virtual head cg * G + x = (query token t, head h of the KV head)
  const int cg = grp % a.n_colgroups;
  const int b = grp / (a.hkv * a.n_colgroups), hk = (grp / a.n_colgroups) % a.hkv;
  const int hq_total = a.hkv * a.g_model;
  auto q_row = [&](int x) -> const uint16_t* {
    const int vh = cg * G + x, t = vh / a.g_model, h = vh - t * a.g_model;
    return a.q + (((size_t)b * a.q_tokens + t) * hq_total + hk * a.g_model + h) * kD;
  };
  const bool is_tile = split < a.n_tile_splits;
  // History splits need q . R_K, whose operands do not depend on the
  // sequence's length: their loads go out before the lengths are read.
  // (Thread (c4, rs) takes output columns [4 c4, 4 c4 + 4) and rows
  // [16 rs, 16 rs + 16) of R_K: 16 float4 loads.)
  const int c4 = tid & 31, rs = tid >> 5;
  constexpr int kQWords = G * kD / 2;               // q as 32-bit words (two bf16 each)
  constexpr int kQPer = (kQWords + 255) / 256;
  float4 rq[16];
  uint32_t qv[kQPer];
  if (!is_tile) {
    load_rot_slices(a.rot_k + (size_t)hk * a.rot_kv_stride, rq, tid);
#pragma unroll
    for (int e = 0; e < kQPer; ++e) {                 // unconditional
      const int w = min(tid + 256 * e, kQWords - 1);
      qv[e] = reinterpret_cast<const uint32_t*>(q_row(w >> 6))[w & 63];
    }
  }
  const int slot = a.seq_slot ? a.seq_slot[b] : b;
  // History splits: this wave's page ids are requested before the length is
  // known (clamped to the page-table row: the split's first page lies in it),
  // together with the split's first page id.  Lanes past the split's last
  // valid page are given that first page once the length has arrived, so
  // no page past the sequence's end is ever addressed.
  const int idx_in_split = kStepPages * (wave + 4 * (lane / kStepPages)) + lane % kStepPages;
  int32_t ids_spec = 0, first_id = 0;
  if (!is_tile) {
    const int pg0 = (split - a.n_tile_splits) * a.pages_per_split;
    const int32_t* row = a.page_table + (size_t)slot * a.max_pages;
    ids_spec = row[pg0 + min(idx_in_split, a.max_pages - 1 - pg0)];
    first_id = row[pg0];
  }
  const int n = a.seq_len[b] + a.len_offset;
  const int hist_len = max(0, n - kSink - kRecent);
  const int n_hist_pages = (hist_len + kPage - 1) / kPage;
  const int act_hist = (n_hist_pages + a.pages_per_split - 1) / a.pages_per_split;
  // The fused step (k_new given) from position 320 on: the newest history
  // token is the one leaving the ring this step.  The history split that
  // owns it demotes it inside this launch and attends to it from its own
  // registers; the page walk covers the older history tokens.
  const bool step_demote = a.k_new != nullptr && hist_len > 0;
  const int walk_len = hist_len - (step_demote ? 1 : 0);
  const int n_walk_pages = (walk_len + kPage - 1) / kPage;
  const int n_sink_used = min(n, kSink);
  const int n_recent_used = min(max(n - kSink, 0), kRecent);
  const int n_tile = n_sink_used + n_recent_used;
  const int act_tile = (n_tile + a.tile_tokens - 1) / a.tile_tokens;
  const int hs = split - a.n_tile_splits;
  if (is_tile ? (split >= act_tile) : (hs >= act_hist)) return;

  float* part_base = a.partials + (size_t)grp * n_split_total * G * kPartStride;
  if (is_tile) {
    const int u0 = split * a.tile_tokens;
    const int recent_first = max(kSink, n - kRecent);
    const size_t sink_base = ((size_t)slot * a.hkv + hk) * kSink;
    const size_t ring_base = ((size_t)slot * a.hkv + hk) * kRecent;
    // the fused step: the token at position n - 1 is still in k_new / v_new
    const size_t new_row = ((size_t)b * a.hkv + hk) * kD;
    const bool from_args = a.k_new != nullptr;
    if (from_args && !step_demote && split == 0 && cg == 0 && tid < kD) {
      // before any demotion, tile split 0 of the group moves it into its
      // sink or free ring slot (no other workgroup of this launch reads that
      // slot); from position 320 on the demoting history split does
      const int pn = n - 1, half_sel = tid >> 6, w = tid & 63;
      // (the pool's tiers are writable device memory; the decode reads them
      // through const pointers)
      uint16_t* dst = const_cast<uint16_t*>(
          pn < kSink ? (half_sel ? a.sink_v : a.sink_k) + (sink_base + pn) * kD
                     : (half_sel ? a.recent_v : a.recent_k) + (ring_base + ((pn - kSink) & (kRecent - 1))) * kD);
      reinterpret_cast<uint32_t*>(dst)[w] =
          reinterpret_cast<const uint32_t*>((half_sel ? a.v_new : a.k_new) + new_row)[w];
    }
    auto row = [&](const uint16_t* sink, const uint16_t* ring, const uint16_t* fresh, int uu) -> const uint16_t* {
      const int u = u0 + uu;
      const int pos = u < n_sink_used ? u : recent_first + (u - n_sink_used);
      if (from_args && pos == n - 1) return fresh + new_row;
      if (u < n_sink_used) return sink + (sink_base + u) * kD;
      return ring + (ring_base + ((pos - kSink) & (kRecent - 1))) * kD;
    };
    // causal limit of column x: its query's position n - q_tokens + t
    bf16_span_wave<G>(q_row, min(a.tile_tokens, n_tile - u0),
                      [&](int uu) { return row(a.sink_k, a.recent_k, a.k_new, uu); },
                      [&](int uu) { return row(a.sink_v, a.recent_v, a.v_new, uu); },
                      [&](int uu) { const int u = u0 + uu; return u < n_sink_used ? u : recent_first + (u - n_sink_used); },
                      [&](int x) { return n - a.q_tokens + (cg * G + x) / a.g_model; }, n - a.q_tokens, sm, wave,
                      lane);
    if (split == 0 && cg == 0 && act_hist > 0) {
      // The merge kernel that follows applies R_V^T to the history part and
      // waits on its rows first thing.  Tile splits end well before the
      // history splits, so tile split 0 of each (sequence, KV head) reads
      // that R_V once (64 KiB) and leaves it in the caches for the merge.
      const float4* rv = reinterpret_cast<const float4*>(a.rot_v + (size_t)hk * a.rot_kv_stride);
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float4 r = rv[tid + 256 * e];
        acc.x += r.x; acc.y += r.y; acc.z += r.z; acc.w += r.w;
      }
      asm volatile("" :: "v"(acc.x), "v"(acc.y), "v"(acc.z), "v"(acc.w));   // keeps the loads
    }
  } else {
    const int pg_begin = hs * a.pages_per_split;
    // (empty for a demoting split whose only page holds just the new token)
    const int pg_end = min(pg_begin + a.pages_per_split, n_walk_pages);
    // page ids of this wave's steps (steps wave, wave + 4, ...), lane
    // kStepPages k + i holding page i of the k-th; then this wave's first
    // step: the prologue below waits only for the older loads, so the loop
    // is entered with exactly the page loads in flight that every later
    // iteration also has.
    const int32_t ids = idx_in_split < pg_end - pg_begin ? ids_spec : first_id;
    PageCodes<kBits> c_first[kStepPages];
    u32x2_t m_first[kStepPages];
    // unconditional (the ids are clamped to pages of this split): the same
    // loads are in flight on every path into the loop
    // (kept in the loop's issue order, so the wait counts the loop computes
    // for its first iteration are exact)
    issue_step<kBits>(a, ids, hk, 0, lane, c_first, m_first);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < kQPer; ++e) {
      const int idx = tid + 256 * e;
      if (idx < kQWords) {
        sm.q[(2 * idx) / kD][(2 * idx) % kD] = bf16_bits_to_float(qv[e] & 0xFFFFu);
        sm.q[(2 * idx) / kD][(2 * idx) % kD + 1] = bf16_bits_to_float(qv[e] >> 16);
      }
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
    // wave w finishes heads w, w + 4, ...: the four waves' partials, then the
    // head's scale exponent and group sums
    for (int h = wave; h < G; h += 4) {
      auto wsum = [&](int jj) {
        return (sm.wo[0][h][jj] + sm.wo[1][h][jj]) + (sm.wo[2][h][jj] + sm.wo[3][h][jj]);
      };
      const float v0 = wsum(lane), v1 = wsum(lane + 64);
      sm.qr[h][lane] = v0;
      sm.qr[h][lane + 64] = v1;
      const float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1))) * kC0;
      int e2 = 0;
      frexpf(amax, &e2);
      const int s_exp = amax > 0.0f ? min(15 - e2, 100) : 0;
      // group sums: lanes 0..31 hold groups 0 (v0) and 2 (v1), lanes 32..63 groups 1 and 3
      const float g0 = half_wave_sum(v0), g1 = half_wave_sum(v1);
      if (lane == 0) { sm.sexp[h] = (float)s_exp; sm.qs[h][0] = g0; sm.qs[h][2] = g1; }
      if (lane == 32) { sm.qs[h][1] = g0; sm.qs[h][3] = g1; }
    }
    __syncthreads();
    const bool demote_here = step_demote && hs == act_hist - 1;
    if (demote_here) demote_in_split<G, kBits>(a, sm, rq, b, slot, hk, n, hist_len - 1, tid, wave, lane);
    hist_wave<G, kBits>(a, sm, ids, hk, walk_len, pg_begin, pg_end, wave, lane, c_first, m_first);
    store_split<G>(sm, part_base + (size_t)split * G * kPartStride, tid, demote_here);
    return;
  }
  store_split<G>(sm, part_base + (size_t)split * G * kPartStride, tid);
}

// Two workgroups per compute unit (up to 256 VGPRs per lane).
template <int G>
__global__ __launch_bounds__(256, 2) void decode_int2_kernel(DecodeArgs a) {
  __shared__ DecodeSmem<G> sm;
  decode_body<G, 2>(a, sm);
}

// INT4 pool: the same kernel over 2560-byte blocks (twice the code registers
// per step in flight)
template <int G>
__global__ __launch_bounds__(256, 2) void decode_int4_kernel(DecodeArgs a) {
  __shared__ DecodeSmem<G> sm;
  decode_body<G, 4>(a, sm);
}

DecodePlan plan_decode(int batch, int hkv, int group, int n_colgroups, int max_seq_len, int target) {
  DecodePlan p{};
  const int max_hist = max(0, max_seq_len - kSink - kRecent);
  const int max_pages = (max_hist + kPage - 1) / kPage;
  const long n_groups = (long)batch * hkv * n_colgroups;
  const int max_tile = min(max_seq_len, kSink + kRecent);
  p.tile_tokens = tile_tokens_for(group);
  const int n_tile = (max_tile + p.tile_tokens - 1) / p.tile_tokens;
  // The most history splits per group that keep the grid within `target`
  // workgroups; each split then gets the smallest multiple of kStepPages
  // pages (one wave step) that covers the history with that many.
  const long hist_max = target / n_groups - n_tile;
  long pps = hist_max >= 1 ? (max_pages + hist_max - 1) / hist_max : kMaxPagesPerSplit;
  pps = (pps + kStepPages - 1) / kStepPages * kStepPages;
  if (pps < 8) pps = 8;
  if (pps > kMaxPagesPerSplit) pps = kMaxPagesPerSplit;
  while (max_pages > 0 && (max_pages + pps - 1) / pps > kMaxSplits - 4 && pps < kMaxPagesPerSplit) pps += 8;
  p.ok = max_pages == 0 || (max_pages + pps - 1) / pps <= kMaxSplits - 4;
  p.pages_per_split = (int)pps;
  p.n_hist_splits = max_pages > 0 ? (int)((max_pages + pps - 1) / pps) : 0;
  p.n_tile_splits = n_tile;
  p.n_splits_total = p.n_hist_splits + p.n_tile_splits;
  p.n_work = (int)(n_groups * p.n_splits_total);
  // more than one round of workgroups with groups that divide over the 8
  // XCDs: whole groups per XCD, tile splits last; else contiguous items
  p.tiles_last = p.n_work > target && n_groups % 8 == 0 && p.n_hist_splits > 0;
  p.grid = ((p.n_work + 7) / 8) * 8;
  p.partial_floats = (size_t)n_groups * p.n_splits_total * group * kPartStride;
  p.workspace_bytes = p.partial_floats * sizeof(float);
  return p;
}

hipError_t launch_decode(const DecodeArgs& a, int group, int grid, hipStream_t st) {
  if (a.code_bits == 4) {
    switch (group) {
      case 1: hipLaunchKernelGGL((decode_int4_kernel<1>), dim3(grid), dim3(256), 0, st, a); break;
      case 2: hipLaunchKernelGGL((decode_int4_kernel<2>), dim3(grid), dim3(256), 0, st, a); break;
      case 4: hipLaunchKernelGGL((decode_int4_kernel<4>), dim3(grid), dim3(256), 0, st, a); break;
      case 8: hipLaunchKernelGGL((decode_int4_kernel<8>), dim3(grid), dim3(256), 0, st, a); break;
      case 16: hipLaunchKernelGGL((decode_int4_kernel<16>), dim3(grid), dim3(256), 0, st, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (group) {
    case 1: hipLaunchKernelGGL((decode_int2_kernel<1>), dim3(grid), dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((decode_int2_kernel<2>), dim3(grid), dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((decode_int2_kernel<4>), dim3(grid), dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL((decode_int2_kernel<8>), dim3(grid), dim3(256), 0, st, a); break;
    case 16: hipLaunchKernelGGL((decode_int2_kernel<16>), dim3(grid), dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace oscar
