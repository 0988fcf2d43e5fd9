// Pieces shared by the decode kernels: BF16 span attention on the matrix
// cores and the per-workgroup partial records that the log-sum-exp merge
// kernel combines (flash-decoding style split-K).
#pragma once

#include "device_common.h"

namespace oscar {

constexpr float kC0 = 0.12751743082459868f;     // log2(e) / sqrt(128)
constexpr float kMInit = -1.0e30f;
constexpr int kPartStride = 132;                // floats per (split, head) record: acc[128], m, l
// BF16 tokens per tile split: 128 for work items of up to 8 columns; one
// split of all 320 sink and recent tokens for 16-column work items (several
// query tokens), whose groups are many, so that tile splits take fewer
// workgroup slots from the history splits
constexpr int kTileTokens = 128;
constexpr int kTileTokensWide = 320;
__host__ __device__ constexpr int tile_tokens_for(int columns) { return columns == 16 ? kTileTokensWide : kTileTokens; }
constexpr int kMaxSplits = 320;                 // per (sequence, KV head)

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  const half2_t h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ uint32_t mul_h2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, a) * __builtin_bit_cast(half2_t, b));
}

// Per-wave partials of a workgroup; slot 4 holds one extra token's record
// (the history token the fused step demotes inside the decode launch).
template <int G>
struct alignas(16) SplitSmem {
  float pt[4][32][G];        // probabilities of a 32-token BF16 chunk, per wave
  float wm[5][16];           // per-wave running max per column (head)
  float wl[5][16];           // per-wave running sum per column
  float wo[5][G][kD];        // per-wave unnormalised outputs
};

// ---------------------------------------------------------------------------
// One wave's share of a BF16 span of `count` tokens: the wave takes 32-token
// chunks wave, wave + 4, ...  Scores q . k use bf16 MFMA (q is bf16, exact;
// fp32 accumulation); p . V runs on the vector unit with each lane owning two
// channels.  rowk(u), rowv(u) give the bf16 rows of token u.
// ---------------------------------------------------------------------------
// qrow(x): the bf16 query row of column x.  Causal limit (several query
// tokens per sequence): column x sees token uu only if pos(uu) <= lim(x).
// pos is increasing in uu and every lim(x) >= lim_min, so a 32-token chunk
// that ends at or before lim_min needs no per-token test.
template <int G, class QRow, class RowK, class RowV, class Pos, class Lim>
__device__ void bf16_span_wave(QRow qrow_of, int count, RowK rowk, RowV rowv, Pos pos, Lim lim, int lim_min,
                               SplitSmem<G>& sm, int wave, int lane) {
  const int x = lane & 15, qa = lane >> 4;
  bf16x8_t bq[4];
  const uint16_t* qrow = qrow_of(x < G ? x : 0);
  const int lim_x = lim(x < G ? x : 0);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(qrow + 32 * kk + 8 * qa);
    if (x >= G) v = (bf16x8_t){};
    bq[kk] = v;
  }
  float m_run = kMInit, l_run = 0.0f;
  float o[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) o[h][0] = o[h][1] = 0.0f;
  for (int c = wave; 32 * c < count; c += 4) {
    const int cbase = 32 * c;
    const int cn = min(32, count - cbase);
    const bool partial = pos(cbase + cn - 1) > lim_min;     // some token may be past a query
    // issue every load of the chunk first: 2 x 4 K fragments and 32 V words per lane
    bf16x8_t ka[2][4];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const uint16_t* kr = rowk(cbase + min(16 * blk + x, cn - 1));
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) ka[blk][kk] = *reinterpret_cast<const bf16x8_t*>(kr + 32 * kk + 8 * qa);
    }
    uint32_t vw[32];
#pragma unroll
    for (int t = 0; t < 32; ++t)
      vw[t] = *reinterpret_cast<const uint32_t*>(rowv(cbase + min(t, cn - 1)) + 2 * lane);
    float sc[2][4];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      float4_t d = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[blk][kk], bq[kk], d, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * blk + 4 * qa + r;
        sc[blk][r] = (x < G && t < cn) ? d[r] * kC0 : -INFINITY;
      }
    }
    if (partial) {                       // uniform: only chunks that reach past a query
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (pos(cbase + 16 * blk + 4 * qa + r) > lim_x) sc[blk][r] = -INFINITY;
    }
    float mx = sc[0][0];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[blk][r]);
    mx = rows_max(mx);
    const float m_new = fmaxf(m_run, mx);
    // lanes own a column (head) for the scores but two channels for p . V:
    // publish old and new maxima per head through LDS
    if (qa == 0) { sm.wm[wave][x] = m_run; sm.wl[wave][x] = m_new; }
    l_run *= __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pv = __builtin_amdgcn_exp2f(sc[blk][r] - m_new);
        l_run += pv;
        if (x < G) sm.pt[wave][16 * blk + 4 * qa + r][x] = pv;
      }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float alpha = __builtin_amdgcn_exp2f(sm.wm[wave][h] - sm.wl[wave][h]);
      o[h][0] *= alpha;
      o[h][1] *= alpha;
    }
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const float v0 = bf16_bits_to_float(vw[t] & 0xFFFFu), v1 = bf16_bits_to_float(vw[t] >> 16);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pw = sm.pt[wave][t][h];     // 0 for t >= cn
        o[h][0] = fmaf(pw, v0, o[h][0]);
        o[h][1] = fmaf(pw, v1, o[h][1]);
      }
    }
    __builtin_amdgcn_wave_barrier();
    m_run = m_new;
  }
  l_run = rows_sum(l_run);
  if (qa == 0) {
    sm.wm[wave][x] = m_run;
    sm.wl[wave][x] = l_run;
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    sm.wo[wave][h][2 * lane] = o[h][0];
    sm.wo[wave][h][2 * lane + 1] = o[h][1];
  }
}

// Combine the four waves' partials of a workgroup into its split record
// rec[h * kPartStride + (0..127 acc, 128 m, 129 l)] (16-byte stores; the
// merge kernel, next on the stream, reads them).
template <int G>
__device__ void store_split(SplitSmem<G>& sm, float* rec, int tid, bool extra = false) {
  __syncthreads();
  const int n_rec = extra ? 5 : 4;
  for (int c = tid; c < G * kD / 4; c += 256) {
    const int h = c / (kD / 4), j4 = c % (kD / 4);
    float mm = kMInit;
    for (int w = 0; w < n_rec; ++w) mm = fmaxf(mm, sm.wm[w][h]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float ll = 0.0f;
    for (int w = 0; w < n_rec; ++w) {
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

}  // namespace oscar
