// Pieces shared by the decode kernels: BF16 span attention on the matrix
// cores, per-workgroup partial records, the completion ticket and the
// log-sum-exp merge of split partials (flash-decoding style split-K).
#pragma once

#include "device_common.h"

namespace oscar {

constexpr float kC0 = 0.12751743082459868f;     // log2(e) / sqrt(128)
constexpr float kMInit = -1.0e30f;
constexpr int kPartStride = 132;                // floats per (split, head) record: acc[128], m, l
constexpr int kTileTokens = 128;                // BF16 tokens per tile split
constexpr int kMaxSplits = 320;                 // per (sequence, KV head)

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  const half2_t h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ uint32_t mul_h2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, a) * __builtin_bit_cast(half2_t, b));
}
// max / sum over the four 16-lane rows of a wave (lanes x, x+16, x+32, x+48)
__device__ __forceinline__ float rows_max(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
__device__ __forceinline__ float wave_max(float v) {
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

template <int G>
struct alignas(16) SplitSmem {
  float pt[4][32][G];        // probabilities of a 32-token BF16 chunk, per wave
  float wm[4][16];           // per-wave running max per column (head)
  float wl[4][16];           // per-wave running sum per column
  float wo[4][G][kD];        // per-wave unnormalised outputs
  float mw[G][kMaxSplits];   // merge: per-split weights
  float ohist[G][kD];        // merge: rotated part
  float lsum[G];
  int last;
};

// ---------------------------------------------------------------------------
// One wave's share of a BF16 span of `count` tokens: the wave takes 32-token
// chunks wave, wave + 4, ...  Scores q . k use bf16 MFMA (q is bf16, exact;
// fp32 accumulation); p . V runs on the vector unit with each lane owning two
// channels.  rowk(u), rowv(u) give the bf16 rows of token u.
// ---------------------------------------------------------------------------
template <int G, class RowK, class RowV>
__device__ void bf16_span_wave(const uint16_t* qg, int count, RowK rowk, RowV rowv, SplitSmem<G>& sm,
                               int wave, int lane) {
  const int x = lane & 15, qa = lane >> 4;
  bf16x8_t bq[4];
  const uint16_t* qrow = qg + (size_t)(x < G ? x : 0) * kD;
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
    float sc[2][4];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int ut = min(16 * blk + x, cn - 1);
      const uint16_t* kr = rowk(cbase + ut);
      float4_t d = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(kr + 32 * kk + 8 * qa);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, bq[kk], d, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * blk + 4 * qa + r;
        sc[blk][r] = (x < G && t < cn) ? d[r] * kC0 : -INFINITY;
      }
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
    for (int t = 0; t < cn; ++t) {
      const uint32_t vv = *reinterpret_cast<const uint32_t*>(rowv(cbase + t) + 2 * lane);
      const float v0 = bf16_bits_to_float(vv & 0xFFFFu), v1 = bf16_bits_to_float(vv >> 16);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pw = sm.pt[wave][t][h];
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
// rec[h * kPartStride + (0..127 acc, 128 m, 129 l)].
template <int G>
__device__ void store_split(SplitSmem<G>& sm, float* rec, int tid) {
  __syncthreads();
  for (int idx = tid; idx < G * kD; idx += 256) {
    const int h = idx / kD, j = idx % kD;
    float mm = kMInit;
#pragma unroll
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, sm.wm[w][h]);
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) acc = fmaf(__builtin_amdgcn_exp2f(sm.wm[w][h] - mm), sm.wo[w][h][j], acc);
    rec[h * kPartStride + j] = acc;
    if (j == 0) {
      float ll = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) ll = fmaf(__builtin_amdgcn_exp2f(sm.wm[w][h] - mm), sm.wl[w][h], ll);
      rec[h * kPartStride + kD] = mm;
      rec[h * kPartStride + kD + 1] = ll;
    }
  }
}

// Release this workgroup's record and take a ticket; true for the last
// workgroup of the group (which then owns the merge and resets the counter).
template <int G>
__device__ bool finish_ticket(SplitSmem<G>& sm, uint32_t* counter, uint32_t target, int tid) {
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = atomicAdd(counter, 1u);
    sm.last = (prev == target - 1u) ? 1 : 0;
  }
  __syncthreads();
  if (!sm.last) return false;
  __threadfence();
  return true;
}

// LSE merge of n_act split records of one group.  Records k < n_plain are in
// the output space; the others are in the rotated space and are summed, then
// rotated back with R^T ((y R^T)_i = sum_j y_j R[i][j]).  out: [G][128] fp32.
template <int G, class SplitId>
__device__ void merge_group(SplitSmem<G>& sm, const float* part_base, int n_act, int n_plain, SplitId split_id,
                            const float* rot, float* out, int tid, int wave, int lane) {
  for (int h = wave; h < G; h += 4) {
    float mm = kMInit;
    for (int k = lane; k < n_act; k += 64)
      mm = fmaxf(mm, __builtin_nontemporal_load(&part_base[((size_t)split_id(k) * G + h) * kPartStride + kD]));
    mm = wave_max(mm);
    float ll = 0.0f;
    for (int k = lane; k < n_act; k += 64) {
      const float* r = &part_base[((size_t)split_id(k) * G + h) * kPartStride];
      const float wk = __builtin_amdgcn_exp2f(__builtin_nontemporal_load(&r[kD]) - mm);
      sm.mw[h][k] = wk;
      ll = fmaf(wk, __builtin_nontemporal_load(&r[kD + 1]), ll);
    }
    ll = wave_sum(ll);
    if (lane == 0) sm.lsum[h] = ll;
  }
  __syncthreads();
  constexpr int kPer = (G * kD + 255) / 256;
  float oplain[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int idx = tid + 256 * e;
    oplain[e] = 0.0f;
    if (idx >= G * kD) continue;
    const int h = idx / kD, j = idx % kD;
    float ar = 0.0f, ap = 0.0f;
    for (int k = 0; k < n_act; ++k) {
      const float v = __builtin_nontemporal_load(&part_base[((size_t)split_id(k) * G + h) * kPartStride + j]);
      if (k < n_plain) ap = fmaf(sm.mw[h][k], v, ap);
      else ar = fmaf(sm.mw[h][k], v, ar);
    }
    sm.ohist[h][j] = ar;
    oplain[e] = ap;
  }
  __syncthreads();
  const bool any_rot = n_act > n_plain;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int idx = tid + 256 * e;
    if (idx >= G * kD) continue;
    const int h = idx / kD, i = idx % kD;
    float acc = oplain[e];
    if (any_rot) {
      const float4* rrow = reinterpret_cast<const float4*>(rot + (size_t)i * kD);
#pragma unroll 4
      for (int j4 = 0; j4 < kD / 4; ++j4) {
        const float4 r4 = rrow[j4];
        acc = fmaf(sm.ohist[h][4 * j4], r4.x, acc);
        acc = fmaf(sm.ohist[h][4 * j4 + 1], r4.y, acc);
        acc = fmaf(sm.ohist[h][4 * j4 + 2], r4.z, acc);
        acc = fmaf(sm.ohist[h][4 * j4 + 3], r4.w, acc);
      }
    }
    out[(size_t)h * kD + i] = acc / sm.lsum[h];
  }
}

}  // namespace oscar
