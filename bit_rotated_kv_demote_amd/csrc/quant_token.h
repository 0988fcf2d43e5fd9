// One token's demotion by a 256-thread workgroup: rotation by R, clip,
// group quantisation, pack and store into its history block.  Shared by
// the append kernel (oscar_append) and the decode kernel of the fused step
// (oscar_step), so both write the same bytes for the same token: the sum
// over R's rows is associated identically, and the quantiser is one
// function.  Pipeline: "大模型KV Cache 2bit量化实战" (yunpan.plus), 三.2; the
// rotation and clip thresholds are fixed offline ("OSCAR: Offline Spectral
// Covariance-Aware Rotation for 2-bit KV Cache Quantization" (gist.science),
// 2.2 A).
#pragma once

#include "device_common.h"

namespace oscar {

// Thread (c4, rs) = (tid & 31, tid >> 5) holds rows [16 rs, 16 rs + 16) and
// columns [4 c4, 4 c4 + 4) of R (row-major fp32 [128][128]).
__device__ __forceinline__ void load_rot_slices(const float* R, float4 (&rq)[16], int tid) {
  const int c4 = tid & 31, rs = tid >> 5;
#pragma unroll
  for (int e = 0; e < 16; ++e) rq[e] = *reinterpret_cast<const float4*>(R + (size_t)(16 * rs + e) * kD + 4 * c4);
}

// y_j = sum_i x_i R[i][j] for x in LDS (128 fp32): per thread, fma chains
// over rows [8 r, 8 r + 8) for r = 2 rs and 2 rs + 1, added; then the pair
// sums of lanes l and l + 32 (row slices 2w and 2w + 1); the four waves'
// sums land in part[w][j] (LDS [4][128]).  Every thread of the block calls
// it; read the result with rotated_channel after a barrier.
__device__ __forceinline__ void rotate_partial(const float* x, const float4 (&rq)[16], float* part, int tid) {
  const int c4 = tid & 31, rs = tid >> 5;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f), acc2 = acc;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float xe = x[16 * rs + e], xf = x[16 * rs + 8 + e];
    acc.x = fmaf(xe, rq[e].x, acc.x);
    acc.y = fmaf(xe, rq[e].y, acc.y);
    acc.z = fmaf(xe, rq[e].z, acc.z);
    acc.w = fmaf(xe, rq[e].w, acc.w);
    acc2.x = fmaf(xf, rq[8 + e].x, acc2.x);
    acc2.y = fmaf(xf, rq[8 + e].y, acc2.y);
    acc2.z = fmaf(xf, rq[8 + e].z, acc2.z);
    acc2.w = fmaf(xf, rq[8 + e].w, acc2.w);
  }
  acc.x += acc2.x;
  acc.y += acc2.y;
  acc.z += acc2.z;
  acc.w += acc2.w;
  acc.x = half_swap_sum(acc.x);
  acc.y = half_swap_sum(acc.y);
  acc.z = half_swap_sum(acc.z);
  acc.w = half_swap_sum(acc.w);
  if ((tid & 32) == 0) *reinterpret_cast<float4*>(&part[(tid >> 6) * kD + 4 * c4]) = acc;
}

__device__ __forceinline__ float rotated_channel(const float* part, int j) {
  return (part[j] + part[kD + j]) + (part[2 * kD + j] + part[3 * kD + j]);
}

// Quantise + pack one vector held one channel per thread (threads 0..127 of
// the block; every thread of the block must call it).  `sh` is 32 words of
// LDS.  Writes token slot `ps` of the block `blk` (an INT2 block, or an INT4
// block when bits == 4).  Returns the thread's dequantised value
// code * scale + zero (rotated space; 0 for threads >= 128).
__device__ float quantize_pack_channel_per_thread(float yc, bool is_v, uint8_t* blk, int ps, uint32_t* sh,
                                                  int bits) {
  const int c = threadIdx.x;
  const bool act = c < kD;
  const float mn = half_wave_min(yc), mx = half_wave_max(yc);   // the thread's 32-channel group
  __half s, z;
  const bool int4 = bits == 4;
  group_scale_zero(mn, mx, &s, &z, int4 ? 15.0f : 3.0f);
  const float sf = __half2float(s), zf = __half2float(z);
  const uint32_t code = quant_code(yc, zf, sf, int4 ? 15.0f : 3.0f);
  if (c < 32) sh[c] = 0u;
  __syncthreads();
  if (act) {
    if (int4) {
      // K: word (chunk (c >> 3) & 3, group c >> 5); V: half-word (channel
      // c & 15, channels 16m with m >> 2 == c >> 6) of this token
      if (!is_v)
        atomicOr(&sh[4 * ((c >> 3) & 3) + (c >> 5)], code << (16 * (c & 1) + 4 * ((c >> 1) & 3)));
      else
        atomicOr(&sh[2 * (c & 15) + (c >> 6)], code << (4 * ((c >> 4) & 3)));
    } else if (!is_v) {
      atomicOr(&sh[2 * ((c >> 3) & 3) + (c >> 6)], code << (2 * k_field(c)));
    } else {
      atomicOr(&sh[8 + (c & 15)], code << (2 * v_field_in_half(c)));
    }
  }
  __syncthreads();
  if (int4) {
    if (!is_v) {
      if (c < 16) *reinterpret_cast<uint32_t*>(blk + 16 * (16 * (c >> 2) + ps) + 4 * (c & 3)) = sh[c];
    } else {
      if (c < 32) *reinterpret_cast<uint16_t*>(blk + v4_halfword_byte(ps, c >> 1, c & 1)) = (uint16_t)sh[c];
    }
  } else if (!is_v) {
    if (c < 8) *reinterpret_cast<uint32_t*>(blk + 16 * (16 * (c >> 1) + ps) + 4 * (c & 1)) = sh[c];
  } else {
    if (c < 16) *reinterpret_cast<uint16_t*>(blk + v_halfword_byte(ps, c)) = (uint16_t)sh[8 + c];
  }
  if (act && (c & 31) == 0) {
    const int g = c >> 5;
    const int so = (is_v ? v_scale_byte(ps, g) : k_scale_byte(ps, g)) + meta_shift(bits);
    const int zo = (is_v ? v_zero_byte(ps, g) : k_zero_byte(ps, g)) + meta_shift(bits);
    *reinterpret_cast<uint16_t*>(blk + so) = half_bits(s);
    *reinterpret_cast<uint16_t*>(blk + zo) = half_bits(z);
  }
  return act ? fmaf((float)code, sf, zf) : 0.0f;
}

}  // namespace oscar
