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
// v(lane) + v(lane ^ 32)
__device__ __forceinline__ float half_swap_sum(float v) {
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

// Split records cross workgroups (and XCDs, each with its own L2).  They are
// written and read through buffer instructions with the device-scope cache
// policy (sc1), which the hardware keeps coherent across L2s without
// whole-cache writeback or invalidation.  A workgroup's record is complete
// once every thread has waited for its stores (s_waitcnt), which precedes the
// ticket below.  Buffer accesses outside the resource's byte range read 0 and
// write nothing.
constexpr int kCachePolicyDevice = 16;          // sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void st_dev4(__amdgpu_buffer_rsrc_t r, uint32_t off, float4 v) {
  const u32x4_t w = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, (int)off, 0, kCachePolicyDevice);
}
__device__ __forceinline__ void st_dev2(__amdgpu_buffer_rsrc_t r, uint32_t off, float a, float b) {
  const u32x2_t w = {__float_as_uint(a), __float_as_uint(b)};
  __builtin_amdgcn_raw_buffer_store_b64(w, r, (int)off, 0, kCachePolicyDevice);
}
__device__ __forceinline__ float4 ld_dev4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCachePolicyDevice);
  return make_float4(__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]), __uint_as_float(w[3]));
}
__device__ __forceinline__ float2 ld_dev2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x2_t w = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kCachePolicyDevice);
  return make_float2(__uint_as_float(w[0]), __uint_as_float(w[1]));
}
constexpr uint32_t kOutOfRange = 0x7FFFFFF0u;   // a byte offset past every resource: reads 0

template <int G>
struct alignas(16) SplitSmem {
  float pt[4][32][G];        // probabilities of a 32-token BF16 chunk, per wave
  float wm[4][16];           // per-wave running max per column (head)
  float wl[4][16];           // per-wave running sum per column
  float wo[4][G][kD];        // per-wave unnormalised outputs
  float mw[G][kMaxSplits];   // merge: per-split weights
  float ohist[G][kD];        // merge: rotated part
  // merge: split sums l [G][kMaxSplits], then per-part sums [parts][2][G*128] (parts * G * 128 == 1024)
  float mred[G * kMaxSplits > 2048 ? G * kMaxSplits : 2048];
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
// rec[h * kPartStride + (0..127 acc, 128 m, 129 l)] (16-byte stores).
template <int G>
__device__ void store_split(SplitSmem<G>& sm, float* rec, int tid) {
  __syncthreads();
  const auto r = dev_rsrc(rec, G * kPartStride * 4);
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
    st_dev4(r, 4u * (h * kPartStride + 4 * j4), acc);
    if (j4 == 0) st_dev2(r, 4u * (h * kPartStride + kD), mm, ll);
  }
}

// Publish this workgroup's record and take a ticket; true for the last
// workgroup of the group (which then owns the merge and resets the counter).
template <int G>
__device__ bool finish_ticket(SplitSmem<G>& sm, uint32_t* counter, uint32_t target, int tid) {
  __builtin_amdgcn_s_waitcnt(0);     // this thread's record stores are complete
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.last = (prev == target - 1u) ? 1 : 0;
  }
  __syncthreads();
  return sm.last != 0;
}

// LSE merge of n_act split records of one group (part_bytes: the group's
// record area).  Records k < n_plain are in the output space; the others are
// in the rotated space and are summed, then rotated back with R^T
// ((y R^T)_i = sum_j y_j R[i][j]).  out: [G][128] fp32.
// The merge runs after the rest of the grid has drained, so its latency is
// the kernel's tail: every load is issued up front, in the order the phases
// consume them ((m, l) pairs, record columns, rows of R), and out-of-range
// slots read 0 instead of branching.
template <int G, class SplitId>
__device__ void merge_group(SplitSmem<G>& sm, const float* part_base, uint32_t part_bytes, int n_act, int n_plain,
                            SplitId split_id, const float* rot, float* out, int tid, int wave, int lane) {
  const bool any_rot = n_act > n_plain;
  const auto rsrc = dev_rsrc(part_base, part_bytes);
  // (m, l) of every (split, head): slot idx = k * G + h
  constexpr int kMl = (kMaxSplits * G + 255) / 256;
  float2 ml[kMl];
#pragma unroll
  for (int r = 0; r < kMl; ++r) {
    const int idx = tid + 256 * r, k = idx / G, h = idx % G;
    ml[r] = ld_dev2(rsrc, idx < n_act * G ? 4u * ((split_id(k) * G + h) * kPartStride + kD) : kOutOfRange);
  }
  // record columns: thread (col, part) takes the float4 column col of splits
  // k = part, part + kParts, ...
  constexpr int kCols = G * kD / 4;
  constexpr int kParts = 256 / kCols;
  constexpr int kBatch = 16;
  const int col = tid % kCols, part = tid / kCols;
  const int ch = col / (kD / 4), j4 = col % (kD / 4);
  auto rec_off = [&](int k) -> uint32_t {
    return k < n_act ? 4u * ((split_id(k) * G + ch) * kPartStride + 4 * j4) : kOutOfRange;
  };
  float4 v[kBatch];
#pragma unroll
  for (int u = 0; u < kBatch; ++u) v[u] = ld_dev4(rsrc, rec_off(part + u * kParts));
  // this thread's slice of R for the inverse rotation: row ri, columns [64 jh, 64 jh + 64)
  const int ri = tid & (kD - 1), jh = tid >> 7;
  float4 rrow[16];
  if (any_rot) {
    const float4* rp = reinterpret_cast<const float4*>(rot + (size_t)ri * kD + 64 * jh);
#pragma unroll
    for (int e = 0; e < 16; ++e) rrow[e] = rp[e];
  }
  // A: per-head global max, split weights and the total sum
  float* lbuf = sm.mred;     // l values [G][kMaxSplits], consumed before phase B reuses mred
#pragma unroll
  for (int r = 0; r < kMl; ++r) {
    const int idx = tid + 256 * r, k = idx / G, h = idx % G;
    if (idx < n_act * G) {
      sm.mw[h][k] = ml[r].x;
      lbuf[h * kMaxSplits + k] = ml[r].y;
    }
  }
  __syncthreads();
  for (int h = wave; h < G; h += 4) {
    float mm = kMInit;
    for (int k = lane; k < n_act; k += 64) mm = fmaxf(mm, sm.mw[h][k]);
    mm = wave_max(mm);
    float ll = 0.0f;
    for (int k = lane; k < n_act; k += 64) {
      const float wk = __builtin_amdgcn_exp2f(sm.mw[h][k] - mm);
      sm.mw[h][k] = wk;
      ll = fmaf(wk, lbuf[h * kMaxSplits + k], ll);
    }
    ll = wave_sum(ll);
    if (lane == 0) sm.lsum[h] = ll;
  }
  __syncthreads();
  // B: weighted sums
  {
    float4 ap = make_float4(0.f, 0.f, 0.f, 0.f), ar = ap;
    auto acc_into = [&](int kk, const float4& x) {
      const float w = sm.mw[ch][kk];
      float4& acc = kk < n_plain ? ap : ar;
      acc.x = fmaf(w, x.x, acc.x); acc.y = fmaf(w, x.y, acc.y);
      acc.z = fmaf(w, x.z, acc.z); acc.w = fmaf(w, x.w, acc.w);
    };
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int k = part + u * kParts;
      if (k < n_act) acc_into(k, v[u]);
    }
    for (int k0 = part + kBatch * kParts; k0 < n_act; k0 += kBatch * kParts) {
#pragma unroll
      for (int u = 0; u < kBatch; ++u) v[u] = ld_dev4(rsrc, rec_off(k0 + u * kParts));
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int k = k0 + u * kParts;
        if (k < n_act) acc_into(k, v[u]);
      }
    }
    __syncthreads();   // every l value has been read before mred is reused
    reinterpret_cast<float4*>(&sm.mred[(part * 2 + 0) * G * kD])[col] = ap;
    reinterpret_cast<float4*>(&sm.mred[(part * 2 + 1) * G * kD])[col] = ar;
  }
  __syncthreads();
  // C: reduce the residue classes; plain part -> wo[0], rotated part -> ohist
  float* plain = &sm.wo[0][0][0];
  for (int idx = tid; idx < G * kD; idx += 256) {
    float ap = 0.f, ar = 0.f;
#pragma unroll
    for (int pp = 0; pp < kParts; ++pp) {
      ap += sm.mred[(pp * 2 + 0) * G * kD + idx];
      ar += sm.mred[(pp * 2 + 1) * G * kD + idx];
    }
    plain[idx] = ap;
    sm.ohist[idx / kD][idx % kD] = ar;
  }
  __syncthreads();
  // D: half of (ohist . R^T) per thread, into wo[1 + jh]
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float acc = 0.0f;
    if (any_rot) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float4 oh = *reinterpret_cast<const float4*>(&sm.ohist[h][64 * jh + 4 * e]);
        acc = fmaf(oh.x, rrow[e].x, acc);
        acc = fmaf(oh.y, rrow[e].y, acc);
        acc = fmaf(oh.z, rrow[e].z, acc);
        acc = fmaf(oh.w, rrow[e].w, acc);
      }
    }
    sm.wo[1 + jh][h][ri] = acc;
  }
  __syncthreads();
  // E: normalise and store
  for (int idx = tid; idx < G * kD; idx += 256) {
    const int h = idx / kD, i = idx % kD;
    out[(size_t)h * kD + i] = (plain[idx] + sm.wo[1][h][i] + sm.wo[2][h][i]) / sm.lsum[h];
  }
}

}  // namespace oscar
