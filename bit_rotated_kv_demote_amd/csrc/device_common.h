// Device-side helpers shared by the HIP kernels of libamdoscar (gfx950).
//
// Page-block format (one 1536-byte block per (page, KV head)); see
// include/oscar.h for the full description.  The format is designed around
// the decode kernel's matrix-core operands: lane l = 16a + b of a wave loads
// the 16-byte chunk l of the code area, whose low 8 bytes are exactly the
// 2-bit K codes the lane feeds to the score MFMAs and whose high 8 bytes are
// the V codes it feeds to the value MFMAs.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace oscar {

constexpr int kD = 128;          // head_dim
constexpr int kPage = 16;        // tokens per page
constexpr int kSink = 64;        // BF16 sink tokens
constexpr int kRecent = 256;     // BF16 recent ring
constexpr int kGroup = 32;       // channels per quantisation group
constexpr int kGroups = 4;
constexpr int kBlock = 1536;     // bytes per (page, KV head)
constexpr int kKScaleOff = 1024;
constexpr int kKZeroOff = 1152;
constexpr int kVScaleOff = 1280;
constexpr int kVZeroOff = 1408;

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

// ---- position of K code (token t, channel j): byte of its 32-bit word and field
__device__ __forceinline__ int k_word_byte(int t, int j) { return 16 * (16 * ((j >> 3) & 3) + t) + 4 * (j >> 6); }
__device__ __forceinline__ int k_field(int j) { return 4 * ((j >> 5) & 1) + ((j >> 1) & 3) + 8 * (j & 1); }
// ---- V codes: the 16-bit half-word holding the 8 codes of (token t, channel j & 15)
__device__ __forceinline__ int v_halfword_byte(int t, int j) {
  return 16 * (16 * (t >> 2) + (j & 15)) + 8 + 4 * ((t & 3) >> 1) + 2 * (t & 1);
}
__device__ __forceinline__ int v_field_in_half(int j) { return j >> 4; }
__device__ __forceinline__ int k_scale_byte(int t, int g) { return kKScaleOff + 8 * t + 2 * g; }
__device__ __forceinline__ int k_zero_byte(int t, int g) { return kKZeroOff + 8 * t + 2 * g; }
__device__ __forceinline__ int v_scale_byte(int t, int g) { return kVScaleOff + 32 * (t >> 2) + 8 * g + 2 * (t & 3); }
__device__ __forceinline__ int v_zero_byte(int t, int g) { return kVZeroOff + 32 * (t >> 2) + 8 * g + 2 * (t & 3); }

// ---- INT4 blocks (2560 bytes per (page, KV head)).  Lane l = 16a + b of a
// decode wave loads the 16-byte K chunk l at 16 l (token b's channels j with
// (j >> 3) & 3 == a: word j >> 5 holds one group's eight, channel j's nibble at
// bit 16 (j & 1) + 4 ((j >> 1) & 3)) and the 16-byte V chunk l at 1024 + 16 l
// (tokens 4a..4a+3, channels j with j & 15 == b: word 2 ((j >> 4) >> 2) +
// ((t & 3) >> 1), nibble at bit 16 (t & 1) + 4 ((j >> 4) & 3)).  The
// scale/zero metadata follows at 2048, laid out as in the INT2 block.
constexpr int kBlock4 = 2560;
constexpr int kVCodeOff4 = 1024;
constexpr int kMetaShift4 = 1024;   // INT4 metadata offset minus the INT2 one
__host__ __device__ constexpr int block_bytes(int bits) { return bits == 4 ? kBlock4 : kBlock; }
__host__ __device__ constexpr int meta_shift(int bits) { return bits == 4 ? kMetaShift4 : 0; }
__device__ __forceinline__ int v4_halfword_byte(int t, int b, int hi_m) {
  return kVCodeOff4 + 16 * (16 * (t >> 2) + b) + 4 * (2 * hi_m + ((t & 3) >> 1)) + 2 * (t & 1);
}

// ---- cross-lane reductions (DPP within 16-lane rows, lane swaps across rows)
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
// v from another lane of the same 16-lane row (DPP control kCtrl)
template <int kCtrl>
__device__ __forceinline__ float dpp_from(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}
// max / sum over the whole wave, the result in every lane: lane pairs, quad
// pairs (quad_perm), the two quads of each half row (row_half_mirror), the
// two halves of each row (row_mirror), then the four rows
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_from<0xB1>(v));      // quad_perm [1, 0, 3, 2]
  v = fmaxf(v, dpp_from<0x4E>(v));      // quad_perm [2, 3, 0, 1]
  v = fmaxf(v, dpp_from<0x141>(v));     // row_half_mirror
  v = fmaxf(v, dpp_from<0x140>(v));     // row_mirror
  return rows_max(v);
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_from<0xB1>(v);
  v += dpp_from<0x4E>(v);
  v += dpp_from<0x141>(v);
  v += dpp_from<0x140>(v);
  return rows_sum(v);
}
// min / max / sum within each 32-lane half of a wave (lanes [0, 32) and
// [32, 64) separately), the result in every lane of the half
__device__ __forceinline__ float half_wave_min(float v) {
  v = fminf(v, dpp_from<0xB1>(v));
  v = fminf(v, dpp_from<0x4E>(v));
  v = fminf(v, dpp_from<0x141>(v));
  v = fminf(v, dpp_from<0x140>(v));
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fminf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float half_wave_max(float v) {
  v = fmaxf(v, dpp_from<0xB1>(v));
  v = fmaxf(v, dpp_from<0x4E>(v));
  v = fmaxf(v, dpp_from<0x141>(v));
  v = fmaxf(v, dpp_from<0x140>(v));
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float half_wave_sum(float v) {
  v += dpp_from<0xB1>(v);
  v += dpp_from<0x4E>(v);
  v += dpp_from<0x141>(v);
  v += dpp_from<0x140>(v);
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// ---- INT2 quantiser of one 32-channel group (asymmetric min-max, four levels).
// zero = fp16 rounded toward -inf of the group minimum, scale = fp16 rounded
// toward +inf of (max - zero) / 3, code = clamp(rint((y - zero) / scale), 0, 3)
// in IEEE fp32 with the correctly rounded quotient; code 0 when scale == 0.
// The INT4 quantiser is the same with 16 levels: (max - zero) / 15 and codes
// clamped to [0, 15].
__device__ __forceinline__ void group_scale_zero(float mn, float mx, __half* scale, __half* zero,
                                                 float n_steps = 3.0f) {
  const __half z = __float2half_rd(mn);
  const float span = mx - __half2float(z);
  *zero = z;
  *scale = __float2half_ru(span / n_steps);
}

// The quotient fl(x / s) without a division, for an fp16 value s > 0 and
// x >= 0 in the quantiser's range (Markstein's correction step): y = fl(1/s)
// from the hardware reciprocal (within one ulp) and one residual step, then
// q0 = fl(x y), r = x - s q0 (exact in fp32 by an fma) and q = fl(q0 + r y).
// With y the correctly rounded reciprocal and q0 within one ulp of x / s,
// q is the correctly rounded quotient.  Checked exhaustively in exact
// arithmetic for every fp16 significand of s (the steps scale with powers
// of two): y = fl(1/s) from any start within two ulps, and q = fl(x / s) for
// x within four ulps of every midpoint (k + 1/2) s, k = 0..15.
__device__ __forceinline__ float recip_of_half(float s) {
  const float y0 = __builtin_amdgcn_rcpf(s);
  return fmaf(fmaf(-s, y0, 1.0f), y0, y0);
}
__device__ __forceinline__ uint32_t quant_code(float yc, float zf, float sf, float max_code = 3.0f) {
  if (!(sf > 0.0f)) return 0u;
  const float x = yc - zf;
  const float y = recip_of_half(sf);
  const float q0 = __fmul_rn(x, y);
  const float q = fmaf(fmaf(-q0, sf, x), y, q0);     // fl(x / s)
  const float c = fminf(fmaxf(rintf(q), 0.0f), max_code);
  return (uint32_t)c;
}

// Cuts that give the INT2 code without forming the quotient, for
// x = fl(y - zero) >= 0 and an fp16 group scale s > 0.  With q = fl(x / s)
// correctly rounded: rint(q) >= 1 iff q > 0.5, >= 2 iff q >= 1.5 and 3 iff
// q > 2.5 (ties to even send 0.5 and 2.5 down and 1.5 up); over the exact quotient these are x/s > 0.5 + 2^-25,
// x/s >= 1.5 - 2^-24 and x/s > 2.5 + 2^-23 (half an fp32 spacing past each
// midpoint).  k s is exact in fp32 for k = 0.5, 1.5, 2.5 (s has 11
// significant bits), and the fp32 spacing next to k s exceeds s 2^-25,
// s 2^-24 and s 2^-23 respectively, so for fp32 x the three tests are exactly
// x > 0.5 s, x >= 1.5 s and x > 2.5 s.  For s == 0 (then x == 0) the middle
// cut is moved above 0 so that the code is 0.
struct CodeCut {
  float c0, c1, c2;
};
__device__ __forceinline__ CodeCut code_cut(float sf) {
  return {0.5f * sf, sf > 0.0f ? 1.5f * sf : 1.0f, 2.5f * sf};
}

__device__ __forceinline__ float clip_value(float y, float tau) { return fminf(fmaxf(y, -tau), tau); }
// The same clip in one instruction (median of three; a NaN y gives -tau, as
// the IEEE minNum / maxNum form does).
__device__ __forceinline__ float clip_med3(float y, float tau) { return __builtin_amdgcn_fmed3f(y, -tau, tau); }

__device__ __forceinline__ uint16_t half_bits(__half h) { return __half_as_ushort(h); }

}  // namespace oscar
