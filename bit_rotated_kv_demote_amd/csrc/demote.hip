// KV demotion kernels: rotate -> clip -> quantise to INT2 -> pack -> store.
//
// The online demotion pipeline of "大模型KV Cache 2bit量化实战：OSCAR让显存暴降90%且
// 智商不掉线" (yunpan.plus), section 三.2: when the recent BF16 window is full,
// its oldest token is rotated, clipped, quantised, packed four codes per byte
// and moved to the INT2 history; the tiers are those of section 三.1 and of
// "OSCAR: Offline Spectral Covariance-Aware Rotation for 2-bit KV Cache
// Quantization" (gist.science), 2.2 B.  The rotation R and the per-channel
// clip thresholds are fixed offline (same page, 2.2 A).
//
// Three kernels (the fused step, oscar_step, demotes its token inside the
// decode launch with the same per-token routine as append_kernel):
//   append_kernel      one decode step: demote the ring slot about to be
//                      reused (fp32 VALU rotation, latency-bound), then write
//                      the new token into sink or ring.
//   demote_bulk_kernel many tokens: 64-token units per wave; the rotation is
//                      a 128x128x64 product on the matrix cores with R split
//                      into bf16 hi + lo terms (fp32 accumulation), or the
//                      input is already-rotated fp32.
//   prefill_route_kernel  copies of the sink and recent tiers of a prefill.
#include <algorithm>

#include "device_common.h"
#include "launchers.h"
#include "quant_token.h"

namespace oscar {

// ---------------------------------------------------------------------------
// append (oscar_append): grid (batch, Hkv, 2 = {K, V}), 256 threads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  __shared__ float xs[kD];
  __shared__ float part[4][kD];
  __shared__ uint32_t sh[32];
  const int b = blockIdx.x, hk = blockIdx.y, is_v = blockIdx.z == 1;
  const int tid = threadIdx.x;
  // y_j = sum_i x_i R[i][j].  The rotation's operands do not depend on the
  // position, so they are requested first: thread (c4, rs) takes columns
  // [4 c4, 4 c4 + 4) and rows [16 rs, 16 rs + 16) of R (16 float4 loads).
  // (Unused when the token only enters the sink or a free ring slot.)
  const float* R = (is_v ? a.rot_v : a.rot_k) + (size_t)hk * a.rot_kv_stride;
  float4 rq[16];
  load_rot_slices(R, rq, tid);
  const float* tau = (is_v ? a.clip_v : a.clip_k) + (size_t)hk * a.clip_kv_stride;
  const float tau_j = tau[tid & (kD - 1)];
  const int slot = a.seq_slot ? a.seq_slot[b] : b;
  const int p = a.position[b];
  const uint16_t* src = (is_v ? a.v_new : a.k_new) + ((size_t)b * a.hkv + hk) * kD;
  const int r = (p - kSink) & (kRecent - 1);
  uint16_t* ring = (is_v ? a.recent_v : a.recent_k) + (((size_t)slot * a.hkv + hk) * kRecent + r) * kD;
  // from position 320 on, the token leaving the ring (p - 256) is demoted
  // into history index h
  const bool demote = p >= kSink + kRecent;
  const int h = p - kSink - kRecent;
  int page = 0;
  if (demote) {
    page = a.page_table[(size_t)slot * a.max_pages + (h >> 4)];
    if (tid < kD / 2) {
      const uint32_t w = reinterpret_cast<const uint32_t*>(ring)[tid];
      xs[2 * tid] = bf16_bits_to_float(w & 0xFFFFu);
      xs[2 * tid + 1] = bf16_bits_to_float(w >> 16);
    }
  }
  if (demote) {                        // block-uniform
    __syncthreads();
    rotate_partial(xs, rq, &part[0][0], tid);
    __syncthreads();  // also orders the ring read above before the overwrite below
    float yc = 0.0f;
    if (tid < kD) yc = clip_value(rotated_channel(&part[0][0], tid), tau_j);
    uint8_t* blk = a.hist + ((size_t)page * a.hkv + hk) * block_bytes(a.code_bits);
    (void)quantize_pack_channel_per_thread(yc, is_v != 0, blk, h & 15, sh, a.code_bits);
  }
  // then the new token enters the sink or the ring slot
  if (tid < kD / 2) {
    uint16_t* dst = p < kSink ? (is_v ? a.sink_v : a.sink_k) + (((size_t)slot * a.hkv + hk) * kSink + p) * kD : ring;
    reinterpret_cast<uint32_t*>(dst)[tid] = reinterpret_cast<const uint32_t*>(src)[tid];
  }
}

// ---------------------------------------------------------------------------
// Bulk demotion.  grid (nwg, 2): blockIdx.y picks K or V, 256 threads.  The
// workgroup stages R^T once (bf16 hi + lo) and its four waves then take work
// units of 64 tokens of one (sequence, KV head) in turn: unit u goes to wave
// u mod (4 nwg).  A unit is four 16-token tiles; every R^T fragment read
// from LDS feeds the four tiles' products.  In a tile, lane l = 16a + t owns
// token t and channels j = 16 m + 4 a + i (m = 0..7, i = 0..3): the layout
// of the 16x16 result blocks of the rotation product
// D[j][t] = sum_i R[i][j] x[t][i].
// ---------------------------------------------------------------------------
// LDS copy of R^T: row j holds R[:, j] as 16 chunks of 8 bf16; chunk c of row j
// is stored at chunk position c ^ (j & 15) so that the 16 rows read by one
// fragment load fall on different banks.
__device__ __forceinline__ int rt_index(int j, int i) { return j * kD + ((((i >> 3) ^ (j & 15))) << 3) + (i & 7); }

// Clip, quantise, pack and store one token's vector held as y[m][i] =
// channel 16 m + 4 qa + i (the lanes qa = 0..3 with the same token hold the
// rest).  tau: LDS [128].  Every lane of the wave must call it (lane swaps).
// kBits: 2 (INT2 block) or 4 (INT4 block).
template <int kBits>
__device__ __forceinline__ void quant_store_token(float (&y)[8][4], const float* tau, bool is_v, bool valid,
                                                  uint8_t* blk, int ps, int qa) {
  float gmn[4], gmx[4];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const float4 t4 = *reinterpret_cast<const float4*>(&tau[16 * m + 4 * qa]);
    y[m][0] = clip_med3(y[m][0], t4.x);
    y[m][1] = clip_med3(y[m][1], t4.y);
    y[m][2] = clip_med3(y[m][2], t4.z);
    y[m][3] = clip_med3(y[m][3], t4.w);
  }
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float mn = y[2 * g][0], mx = y[2 * g][0];
#pragma unroll
    for (int e = 1; e < 8; ++e) {
      const float v = y[2 * g + (e >> 2)][e & 3];
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
    }
    // across the four lanes a = 0..3 that share this token
    const auto pn = __builtin_amdgcn_permlane16_swap(__float_as_uint(mn), __float_as_uint(mn), false, false);
    const auto px = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mn = fminf(__uint_as_float(pn[0]), __uint_as_float(pn[1]));
    mx = fmaxf(__uint_as_float(px[0]), __uint_as_float(px[1]));
    const auto qn = __builtin_amdgcn_permlane32_swap(__float_as_uint(mn), __float_as_uint(mn), false, false);
    const auto qx = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    gmn[g] = fminf(__uint_as_float(qn[0]), __uint_as_float(qn[1]));
    gmx[g] = fmaxf(__uint_as_float(qx[0]), __uint_as_float(qx[1]));
  }
  __half sc[4], zr[4];
  float zf[4];
  CodeCut cut[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    group_scale_zero(gmn[g], gmx[g], &sc[g], &zr[g], kBits == 4 ? 15.0f : 3.0f);
    zf[g] = __half2float(zr[g]);
    cut[g] = code_cut(__half2float(sc[g]));
  }
  uint32_t code[8][4];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      code[m][i] = kBits == 4 ? quant_code(y[m][i], zf[m >> 1], __half2float(sc[m >> 1]), 15.0f)
                              : quant_code_cut(y[m][i] - zf[m >> 1], cut[m >> 1]);
  auto push = [&](uint32_t acc, int sh, int m, int i) { return (acc << sh) + code[m][i]; };

  if constexpr (kBits == 4) {
    if (!is_v) {
      // K: channel j = 16m + 4a + i is in chunk 2(m & 1) + (a >> 1), word
      // m >> 1, nibble at bit 16(i & 1) + 8(a & 1) + 4(i >> 1); lanes a and
      // a ^ 1 fill the two byte halves of each 16-bit half of the same word.
      uint32_t wd[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        uint32_t w = code[m][0] | (code[m][1] << 16) | (code[m][2] << 4) | (code[m][3] << 20);
        w <<= 8 * (qa & 1);
        const auto pr = __builtin_amdgcn_permlane16_swap(w, w, false, false);
        wd[m] = pr[0] | pr[1];
      }
      if (valid && (qa & 1) == 0) {
        *reinterpret_cast<u32x4_t*>(blk + 16 * (16 * (qa >> 1) + ps)) = (u32x4_t){wd[0], wd[2], wd[4], wd[6]};
        *reinterpret_cast<u32x4_t*>(blk + 16 * (16 * (2 + (qa >> 1)) + ps)) = (u32x4_t){wd[1], wd[3], wd[5], wd[7]};
      }
    } else {
      // V: channel 4a + i of this token: codes of channels 16m with m < 4 in
      // one half-word (nibble m), m >= 4 in another (nibble m - 4)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = code[0][i] | (code[1][i] << 4) | (code[2][i] << 8) | (code[3][i] << 12);
        const uint32_t hi = code[4][i] | (code[5][i] << 4) | (code[6][i] << 8) | (code[7][i] << 12);
        if (valid) {
          *reinterpret_cast<uint16_t*>(blk + v4_halfword_byte(ps, 4 * qa + i, 0)) = (uint16_t)lo;
          *reinterpret_cast<uint16_t*>(blk + v4_halfword_byte(ps, 4 * qa + i, 1)) = (uint16_t)hi;
        }
      }
    }
  } else if (!is_v) {
    // K: channel j = 16m + 4a + i lands in word (2(m&1) + (a>>1), m>>2) at
    // field 4((m>>1)&1) + 2(a&1) + (i>>1) + 8(i&1); lanes a and a^1 fill
    // complementary fields of the same four words.  A lane builds its eight
    // fields at 4hb + (i>>1) + 8(i&1) from the highest down, then moves them
    // up by 2(a&1) fields.
    uint32_t wd[2][2];
#pragma unroll
    for (int ai = 0; ai < 2; ++ai)
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int m0 = ai + 4 * w, m1 = ai + 2 + 4 * w;   // hb = 0, 1
        uint32_t acc = push(0u, 0, m1, 3);               // field 13
        acc = push(acc, 2, m1, 1);                       // 12
        acc = push(acc, 6, m0, 3);                       // 9
        acc = push(acc, 2, m0, 1);                       // 8
        acc = push(acc, 6, m1, 2);                       // 5
        acc = push(acc, 2, m1, 0);                       // 4
        acc = push(acc, 6, m0, 2);                       // 1
        acc = push(acc, 2, m0, 0);                       // 0
        acc <<= 4 * (qa & 1);
        const auto pr = __builtin_amdgcn_permlane16_swap(acc, acc, false, false);
        wd[ai][w] = pr[0] | pr[1];
      }
    if (valid && (qa & 1) == 0) {
#pragma unroll
      for (int ai = 0; ai < 2; ++ai) {
        const int aa = 2 * ai + (qa >> 1);
        *reinterpret_cast<u32x2_t*>(blk + 16 * (16 * aa + ps)) = (u32x2_t){wd[ai][0], wd[ai][1]};
      }
    }
  } else {
    // V: the 8 codes of (token, channel 4a + i) form one half-word, code of
    // channel 16m + 4a + i at bits 2m.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t hw = push(0u, 0, 7, i);
#pragma unroll
      for (int m = 6; m >= 0; --m) hw = push(hw, 2, m, i);
      if (valid) *reinterpret_cast<uint16_t*>(blk + v_halfword_byte(ps, 4 * qa + i)) = (uint16_t)hw;
    }
  }
  if (valid) {
    // lane a stores group a's scale and zero (selects, not a dynamic index)
    const int g = qa;
    const uint32_t s01 = half_bits(sc[0]) | ((uint32_t)half_bits(sc[1]) << 16);
    const uint32_t s23 = half_bits(sc[2]) | ((uint32_t)half_bits(sc[3]) << 16);
    const uint32_t z01 = half_bits(zr[0]) | ((uint32_t)half_bits(zr[1]) << 16);
    const uint32_t z23 = half_bits(zr[2]) | ((uint32_t)half_bits(zr[3]) << 16);
    const int sh = 16 * (g & 1);
    const int so = (is_v ? v_scale_byte(ps, g) : k_scale_byte(ps, g)) + meta_shift(kBits);
    const int zo = (is_v ? v_zero_byte(ps, g) : k_zero_byte(ps, g)) + meta_shift(kBits);
    *reinterpret_cast<uint16_t*>(blk + so) = (uint16_t)(((g < 2) ? s01 : s23) >> sh);
    *reinterpret_cast<uint16_t*>(blk + zo) = (uint16_t)(((g < 2) ? z01 : z23) >> sh);
  }
}

template <bool kRotatedInput, int kBits>
__global__ __launch_bounds__(256) void demote_bulk_kernel(DemoteArgs a) {
  __shared__ __bf16 rt_hi[kRotatedInput ? 1 : kD * kD];
  __shared__ __bf16 rt_lo[kRotatedInput ? 1 : kD * kD];
  __shared__ float tau_s[kD];
  const int is_v = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tcol = lane & 15, qa = lane >> 4;
  // One R and tau per KV head: workgroup z serves KV head z alone (its R is
  // the one staged in LDS); with a shared pair every workgroup serves all.
  const bool per_head = a.clip_kv_stride != 0;
  const int heads_here = per_head ? 1 : a.hkv;
  const int hk_base = per_head ? (int)blockIdx.z : 0;

  if constexpr (!kRotatedInput) {
    // R (row-major fp32) -> LDS R^T split into bf16 hi + lo.
    const float* R = (is_v ? a.rot_v : a.rot_k) + (size_t)hk_base * a.rot_kv_stride;
    for (int idx = tid; idx < kD * kD / 4; idx += 256) {
      const float4 v4 = reinterpret_cast<const float4*>(R)[idx];
      const int i = idx / (kD / 4), j0 = (idx % (kD / 4)) * 4;
      const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const __bf16 hi = (__bf16)vv[e];
        const __bf16 lo = (__bf16)(vv[e] - (float)hi);
        rt_hi[rt_index(j0 + e, i)] = hi;
        rt_lo[rt_index(j0 + e, i)] = lo;
      }
    }
  }
  if (tid < kD) tau_s[tid] = (is_v ? a.clip_v : a.clip_k)[(size_t)hk_base * a.clip_kv_stride + tid];
  __syncthreads();

  const int ups = a.unit_tiles;                       // units per (sequence, KV head)
  const int n_units = a.batch * heads_here * ups;
  for (int u = blockIdx.x * 4 + wave; u < n_units; u += gridDim.x * 4) {
    const int b = u / (heads_here * ups), rem = u % (heads_here * ups);
    const int hk = hk_base + rem / ups, tok0 = kUnitTokens * (rem % ups);
    const int count = a.length ? max(0, a.length[b] - kSink - kRecent) : a.n_tokens;
    if (tok0 >= count) continue;                       // wave-uniform
    const int slot = a.seq_slot ? a.seq_slot[b] : b;
    const int h0 = a.hist_start ? a.hist_start[b] : 0;
    // token of tile t for this lane (clamped to the last valid token)
    auto src_token = [&](int t) { return min(tok0 + 16 * t + tcol, count - 1); };
    auto page_of = [&](int t) { return a.page_table[(size_t)slot * a.max_pages + ((h0 + src_token(t)) >> 4)]; };
    auto store = [&](float (&y)[8][4], int t, int page) {
      const int tok = tok0 + 16 * t + tcol;
      uint8_t* blk = a.hist + ((size_t)page * a.hkv + hk) * block_bytes(kBits);
      quant_store_token<kBits>(y, tau_s, is_v != 0, tok < count, blk, (h0 + src_token(t)) & 15, qa);
    };
    if constexpr (kRotatedInput) {
      for (int t = 0; t < kUnitTokens / 16; ++t) {
        if (tok0 + 16 * t >= count) break;             // wave-uniform
        const float* src = (is_v ? a.src_v_f32 : a.src_k_f32) +
                           (((size_t)b * a.src_tokens + a.src_tok0 + src_token(t)) * a.hkv + hk) * kD;
        float y[8][4];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const float4 v4 = *reinterpret_cast<const float4*>(src + 16 * m + 4 * qa);
          y[m][0] = v4.x; y[m][1] = v4.y; y[m][2] = v4.z; y[m][3] = v4.w;
        }
        store(y, t, page_of(t));
      }
    } else {
      constexpr int kT = kUnitTokens / 16;
      bf16x8_t xb[kT][4];
#pragma unroll
      for (int t = 0; t < kT; ++t) {
        const uint16_t* src = (is_v ? a.src_v : a.src_k) +
                              (((size_t)b * a.src_tokens + a.src_tok0 + src_token(t)) * a.hkv + hk) * kD;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) xb[t][kk] = *reinterpret_cast<const bf16x8_t*>(src + 32 * kk + 8 * qa);
      }
      // page ids travel with the inputs, so the stores never wait for them
      int pg[kT];
#pragma unroll
      for (int t = 0; t < kT; ++t) pg[t] = page_of(t);
      float4_t acc[kT][8];
#pragma unroll
      for (int t = 0; t < kT; ++t)
#pragma unroll
        for (int m = 0; m < 8; ++m) acc[t][m] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const int row = rt_index(16 * m + tcol, 32 * kk + 8 * qa);
          const bf16x8_t ah = *reinterpret_cast<const bf16x8_t*>(&rt_hi[row]);
          const bf16x8_t al = *reinterpret_cast<const bf16x8_t*>(&rt_lo[row]);
#pragma unroll
          for (int t = 0; t < kT; ++t) acc[t][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, xb[t][kk], acc[t][m], 0, 0, 0);
#pragma unroll
          for (int t = 0; t < kT; ++t) acc[t][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, xb[t][kk], acc[t][m], 0, 0, 0);
        }
      }
#pragma unroll
      for (int t = 0; t < kT; ++t) {
        if (tok0 + 16 * t >= count) break;             // wave-uniform
        float y[8][4];
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) y[m][i] = acc[t][m][i];
        store(y, t, pg[t]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Prefill routing of the BF16 tiers.  grid (20, batch*Hkv, 2), 256 threads:
// 16 tokens x 16 threads of 16 bytes.  Compact index u in [0, 320): u < 64 is
// sink position u, u >= 64 is position max(64, n-256) + (u-64).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prefill_route_kernel(PrefillArgs a) {
  const int bh = blockIdx.y;
  const int b = bh / a.hkv, hk = bh % a.hkv, is_v = blockIdx.z;
  const int n = a.length[b];
  const int u = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int part = threadIdx.x & 15;
  const int p = u < kSink ? u : max(kSink, n - kRecent) + (u - kSink);
  if (p >= n) return;
  const int slot = a.seq_slot ? a.seq_slot[b] : b;
  const uint16_t* src = (is_v ? a.src_v : a.src_k) + (((size_t)b * a.max_len + p) * a.hkv + hk) * kD;
  uint16_t* dst;
  if (p < kSink)
    dst = (is_v ? a.sink_v : a.sink_k) + (((size_t)slot * a.hkv + hk) * kSink + p) * kD;
  else
    dst = (is_v ? a.recent_v : a.recent_k) +
          (((size_t)slot * a.hkv + hk) * kRecent + ((p - kSink) & (kRecent - 1))) * kD;
  reinterpret_cast<uint4*>(dst)[part] = reinterpret_cast<const uint4*>(src)[part];
}

hipError_t launch_append(const AppendArgs& a, int batch, hipStream_t st) {
  hipLaunchKernelGGL(append_kernel, dim3(batch, a.hkv, 2), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_demote(const DemoteArgs& a_in, int batch, int max_count, bool rotated, hipStream_t st) {
  if (max_count <= 0) return hipSuccess;
  DemoteArgs a = a_in;
  a.batch = batch;
  a.unit_tiles = (max_count + kUnitTokens - 1) / kUnitTokens;
  // two workgroups per compute unit per tensor at most (each stages R once);
  // with one R per KV head, a slice of them per KV head (grid z)
  const bool per_head = a.clip_kv_stride != 0;
  const int heads = per_head ? a.hkv : 1;
  const long units = (long)batch * (per_head ? 1 : a.hkv) * a.unit_tiles;
  const int nwg = (int)std::min<long>((units + 3) / 4, std::max(1, 256 / heads));
  const dim3 grid(nwg, 2, heads);
  if (a.code_bits == 4) {
    if (rotated)
      hipLaunchKernelGGL((demote_bulk_kernel<true, 4>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((demote_bulk_kernel<false, 4>), grid, dim3(256), 0, st, a);
  } else {
    if (rotated)
      hipLaunchKernelGGL((demote_bulk_kernel<true, 2>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((demote_bulk_kernel<false, 2>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_route(const PrefillArgs& a, int batch, hipStream_t st) {
  hipLaunchKernelGGL(prefill_route_kernel, dim3((kSink + kRecent) / 16, batch * a.hkv, 2), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace oscar
