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
//   demote_bulk_kernel many tokens: units of two pages (INT2) or one
//                      (INT4) per wave, one tensor per wave; the rotation is
//                      a 128x128x32 (INT2) product on the matrix cores with
//                      R split into bf16
//                      hi + lo terms (fp32 accumulation), or the input is
//                      already-rotated fp32.
//   prefill_route_kernel  copies of the sink and recent tiers of a prefill.
#include <algorithm>
#include <type_traits>

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
// Bulk demotion.  grid (nwg, 1, heads), one workgroup per compute unit of
// 2 W waves (INT2: W = 6, three waves per SIMD; INT4: W = 8, four).  The
// workgroup stages R_K^T and R_V^T as bf16 hi + lo terms in LDS once.  Waves
// 0..W-1 demote K and waves W..2W-1 V; each takes work units of kPages
// history pages of one (sequence, KV head) in turn (unit u goes to the
// u mod (W nwg)-th wave of its tensor).  A wave builds its tensor's bytes of each page block in a
// wave-private LDS image (codes, then scales and zeros) and stores them with
// one store per lane for the codes and one for the metadata; the K and V
// halves of a block meet in L2.  A page only partly covered by the demoted
// tokens is read into the image first, so its other slots keep their bytes.
//
// Rotation: D[c][t] = sum_i R[i][c] x[t][i] on 16x16x32 bf16 matrix-core
// products, x . R_hi + x . R_lo with fp32 accumulation, one page of tokens
// in the columns.  The 16 rows of output block m are the rotated channels
// 32 (r >> 2) + 4 m + (r & 3), so lane l = 16 g + t ends up holding all 32
// channels of quantisation group g of token t (channel 32 g + 4 m + i in
// y[m][i]): clip, minimum and maximum, scale and zero and the codes are
// each computed once per group, in one lane, with no exchange.
// ---------------------------------------------------------------------------
template <int kBits>
struct DemCfg {
  static constexpr int kPages = kBits == 4 ? 1 : 2;        // pages per work unit
  // waves per tensor: the unit's accumulators (32 VGPRs per page) set the
  // waves a SIMD can hold, and more waves hide the LDS and memory waits
  static constexpr int kTensorWaves = kBits == 4 ? 8 : 6;
  static constexpr int kThreads = 2 * 64 * kTensorWaves;
  static constexpr int kCodeBytes = kBits == 4 ? 1024 : 512;   // one tensor's code bytes in a block
  static constexpr int kPart = kCodeBytes + 256;            // one tensor's bytes in a block (codes + meta)
  static constexpr int kMetaBase = kBits == 4 ? 2048 : 1024;   // block offset of the K metadata
};

// Each wave handles one tensor, so its LDS image of a page holds only that
// tensor's bytes of the block, packed: the code bytes first, then the 256
// bytes of scales and zeros.  part_off maps a block offset of the tensor's
// bytes to the image.  INT2: the code area's 16-byte rows carry K in bytes
// 0..7 and V in bytes 8..15; INT4: K codes in [0, 1024), V in [1024, 2048).
template <int kBits>
__device__ __forceinline__ int part_off(bool is_v, int off) {
  constexpr int kMeta = DemCfg<kBits>::kMetaBase;
  if (off >= kMeta) return DemCfg<kBits>::kCodeBytes + off - kMeta - (is_v ? 256 : 0);
  if constexpr (kBits == 4) return off - (is_v ? 1024 : 0);
  return 8 * (off >> 4) + (off & 7);
}

// LDS copy of R^T: row c holds R[:, c] as 16 chunks of 8 bf16; chunk k of row c
// sits at position k ^ swz(c).  One fragment load reads the rows
// 32 (r >> 2) + 4 m + (r & 3), r = 0..15, whose swz values are r itself, so
// the 16 rows fall on different banks.
__device__ __forceinline__ int rt_swz(int c) { return (c & 3) | (((c >> 5) & 3) << 2); }
__device__ __forceinline__ int rt_index(int c, int i) { return c * kD + ((((i >> 3) ^ rt_swz(c))) << 3) + (i & 7); }
__device__ __forceinline__ int out_channel(int m, int r) { return 32 * (r >> 2) + 4 * m + (r & 3); }

// Clip one lane's group in place (32 values, channel 32 g + 4 m + i in
// y[m][i]; tau_g: LDS, the group's 32 thresholds) and take its minimum and
// maximum.
__device__ __forceinline__ void clip_group(float (&y)[8][4], const float* tau_g, float& mn, float& mx) {
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const float4 t4 = *reinterpret_cast<const float4*>(&tau_g[4 * m]);
    y[m][0] = clip_med3(y[m][0], t4.x);
    y[m][1] = clip_med3(y[m][1], t4.y);
    y[m][2] = clip_med3(y[m][2], t4.z);
    y[m][3] = clip_med3(y[m][3], t4.w);
  }
  mn = y[0][0];
  mx = y[0][0];
#pragma unroll
  for (int e = 1; e < 31; e += 2) {
    const float v0 = y[e >> 2][e & 3], v1 = y[(e + 1) >> 2][(e + 1) & 3];
    mn = fminf(fminf(mn, v0), v1);
    mx = fmaxf(fmaxf(mx, v0), v1);
  }
  mn = fminf(mn, y[7][3]);
  mx = fmaxf(mx, y[7][3]);
}

// INT4: clip, group parameters and codes (correctly rounded division) of
// one lane's group.
__device__ __forceinline__ void quant_lane_group4(float (&y)[8][4], const float* tau_g, uint32_t (&code)[8][4],
                                                  __half& sc, __half& zr) {
  float mn, mx;
  clip_group(y, tau_g, mn, mx);
  group_scale_zero(mn, mx, &sc, &zr, 15.0f);
  const float zf = __half2float(zr), sf = __half2float(sc);
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) code[m][i] = quant_code(y[m][i], zf, sf, 15.0f);
}

// INT2 fast path of one lane's group: clip, group parameters, then each
// code as two bits shifted straight into the packed words, with no compare.
// x = y - zero is >= 0, so the order of x against a cut c >= 0 is the order
// of their bit patterns as integers, and the cut tests of code_cut are sign
// bits: x > c0 iff c0 - x < 0, x >= c1 iff (c1 - 1) - x < 0 (bit patterns),
// x > c2 iff c2 - x < 0.  The three tests are nested, so bit 1 of the code
// is the middle one and bit 0 the parity of all three;
// alignbit(w, z, 31) = (w << 1) | (z >> 31) shifts a sign bit into w.
__device__ __forceinline__ void quant_pack_int2(float (&y)[8][4], const float* tau_g, bool is_v, int t, int g,
                                                bool valid, uint8_t* img) {
  float mn, mx;
  clip_group(y, tau_g, mn, mx);
  __half sc, zr;
  group_scale_zero(mn, mx, &sc, &zr, 3.0f);
  const float zf = __half2float(zr);
  const CodeCut cut = code_cut(__half2float(sc));
  const uint32_t k0 = __float_as_uint(cut.c0), k1 = __float_as_uint(cut.c1) - 1u, k2 = __float_as_uint(cut.c2);
  // w <- 4 w + code of value y[m][i]
  auto push = [&](uint32_t w, int m, int i) {
    const uint32_t xb = __float_as_uint(y[m][i] - zf);
    const uint32_t d1 = k1 - xb;
    w = __builtin_amdgcn_alignbit(w, d1, 31);
    return __builtin_amdgcn_alignbit(w, __builtin_amdgcn_bitop3_b32(k0 - xb, d1, k2 - xb, 0x96), 31);   // xor of three
  };
  if (!is_v) {
    // chunk row a: channels 32 g + 8 a + e (value y[2a + (e >> 2)][e & 3]) go to
    // field ((e >> 1) & 3) + 8 (e & 1) + 4 (g & 1) of word g >> 1; the lane of
    // group g ^ 1 fills the other fields
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      uint32_t w = 0;
#pragma unroll
      for (int k = 3; k >= 0; --k) w = push(w, 2 * a + (k >> 1), 2 * (k & 1) + 1);    // e = 2k + 1
      w <<= 8;
#pragma unroll
      for (int k = 3; k >= 0; --k) w = push(w, 2 * a + (k >> 1), 2 * (k & 1));        // e = 2k
      w <<= 8 * (g & 1);
      const auto pr = __builtin_amdgcn_permlane16_swap(w, w, false, false);
      w = pr[0] | pr[1];
      if (valid && (g & 1) == 0) *reinterpret_cast<uint32_t*>(img + part_off<2>(false, 16 * (16 * a + t) + 4 * (g >> 1))) = w;
    }
  } else {
    // the half-word of (token t, channel residue b) holds channels b + 16 k,
    // k = 0..7, two bits each; this lane's group has k = 2 g (value
    // y[b >> 2][b & 3]) and 2 g + 1 (y[(b >> 2) + 4][b & 3]).  dword j carries
    // residues 2 j and 2 j + 1, this lane's nibble at bit 4 g of each half.
    uint32_t d[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int b0 = 2 * j, b1 = 2 * j + 1;
      uint32_t w = push(0u, (b1 >> 2) + 4, b1 & 3);
      w = push(w, b1 >> 2, b1 & 3);
      w <<= 12;
      w = push(w, (b0 >> 2) + 4, b0 & 3);
      w = push(w, b0 >> 2, b0 & 3);
      d[j] = w << (4 * g);
    }
    // reduce-scatter over the four groups: lanes g and g ^ 1, then g and g ^ 2
    uint32_t e[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const auto pr = __builtin_amdgcn_permlane16_swap(d[j], d[j + 4], false, false);
      e[j] = pr[0] | pr[1];          // g even: residues 2j, 2j+1; g odd: 2j+8, 2j+9
    }
    uint32_t f[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const auto pr = __builtin_amdgcn_permlane32_swap(e[j], e[j + 2], false, false);
      f[j] = pr[0] | pr[1];
    }
    // this lane now holds residues bb .. bb + 3
    const int bb = 8 * (g & 1) + 4 * (g >> 1);
    const int tq = t >> 2, tw = (t & 3) >> 1, th = t & 1;
    if (valid) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        *reinterpret_cast<uint16_t*>(img + part_off<2>(true, 16 * (16 * tq + bb + k) + 8 + 4 * tw + 2 * th)) =
            (uint16_t)(f[k >> 1] >> (16 * (k & 1)));
    }
  }
  if (valid) {
    *reinterpret_cast<uint16_t*>(img + part_off<2>(is_v, is_v ? v_scale_byte(t, g) : k_scale_byte(t, g))) = half_bits(sc);
    *reinterpret_cast<uint16_t*>(img + part_off<2>(is_v, is_v ? v_zero_byte(t, g) : k_zero_byte(t, g))) = half_bits(zr);
  }
}

// INT4: write one lane's group of codes, scale and zero (token slot t, group
// g) into the tensor's page image `img`.  Every lane of the wave calls it:
// the V half-words combine two groups by a lane swap.  Only lanes of valid
// tokens write.
__device__ __forceinline__ void pack_lane_group4(const uint32_t (&c)[8][4], __half sc, __half zr, bool is_v, int t,
                                                 int g, bool valid, uint8_t* img) {
  if (!is_v) {
    // K: chunk row a holds channels 32 g + 8 a + e, e = 0..7 (code c[2a + (e >> 2)][e & 3])
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      uint32_t w = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) w |= c[2 * a + (e >> 2)][e & 3] << (16 * (e & 1) + 4 * ((e >> 1) & 3));
      if (valid) *reinterpret_cast<uint32_t*>(img + part_off<4>(false, 16 * (16 * a + t) + 4 * g)) = w;
    }
  } else {
    // V: the half-word of (token t, channel residue b) holds channels b + 16 k
    // for the four k of one half (4 bits each); this lane's group g holds
    // k = 2 g and 2 g + 1: codes c[b >> 2][b & 3] and c[(b >> 2) + 4][b & 3].
    // dword j carries residues 2 j and 2 j + 1.
    const int sh = 8 * (g & 1);
    uint32_t d[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int b0 = 2 * j, b1 = 2 * j + 1;
      const uint32_t h0 = c[b0 >> 2][b0 & 3] | (c[(b0 >> 2) + 4][b0 & 3] << 4);
      const uint32_t h1 = c[b1 >> 2][b1 & 3] | (c[(b1 >> 2) + 4][b1 & 3] << 4);
      d[j] = (h0 | (h1 << 16)) << sh;
    }
    // lanes g and g ^ 1 complete the half-words
    uint32_t e[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const auto pr = __builtin_amdgcn_permlane16_swap(d[j], d[j + 4], false, false);
      e[j] = pr[0] | pr[1];          // g even: residues 2j, 2j+1; g odd: 2j+8, 2j+9
    }
    const int tq = t >> 2, tw = (t & 3) >> 1, th = t & 1;
    const int bb = 8 * (g & 1);
    if (valid) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int b = bb + 2 * j + hh;
          *reinterpret_cast<uint16_t*>(
              img + part_off<4>(true, kVCodeOff4 + 16 * (16 * tq + b) + 4 * (2 * (g >> 1) + tw) + 2 * th)) =
              (uint16_t)(e[j] >> (16 * hh));
        }
    }
  }
  if (valid) {
    const int so = (is_v ? v_scale_byte(t, g) : k_scale_byte(t, g)) + meta_shift(4);
    const int zo = (is_v ? v_zero_byte(t, g) : k_zero_byte(t, g)) + meta_shift(4);
    *reinterpret_cast<uint16_t*>(img + part_off<4>(is_v, so)) = half_bits(sc);
    *reinterpret_cast<uint16_t*>(img + part_off<4>(is_v, zo)) = half_bits(zr);
  }
}

template <bool kRotatedInput, int kBits>
__global__ __launch_bounds__(DemCfg<kBits>::kThreads, 1) void demote_bulk_kernel(DemoteArgs a) {
  constexpr int kPages = DemCfg<kBits>::kPages;
  constexpr int kTW = DemCfg<kBits>::kTensorWaves;
  constexpr int kPart = DemCfg<kBits>::kPart;
  constexpr int kCodeBytes = DemCfg<kBits>::kCodeBytes;
  constexpr int kBytes = block_bytes(kBits);
  constexpr int kRt = kRotatedInput ? 1 : kD * kD;
  __shared__ __bf16 rt_hi[2][kRt];            // [K|V] R^T hi terms
  __shared__ __bf16 rt_lo[2][kRt];
  __shared__ float tau_s[2][kD];
  __shared__ __attribute__((aligned(16))) uint8_t img_all[2 * kTW][kPages * kPart];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = lane & 15, g = lane >> 4;
  // One R and tau per KV head: workgroup z serves KV head z alone (its Rs are
  // the ones staged in LDS); with a shared pair every workgroup serves all.
  const bool per_head = a.clip_kv_stride != 0;
  const int heads_here = per_head ? 1 : a.hkv;
  const int hk_base = per_head ? (int)blockIdx.z : 0;

  if constexpr (!kRotatedInput) {
    // R (row-major fp32) -> LDS R^T split into bf16 hi + lo, for K and V, in
    // chunks of 8 input rows of one column: lanes take consecutive columns
    // (coalesced reads), each chunk leaves as one 16-byte store per term
    for (int c = tid; c < 2 * kD * (kD / 8); c += DemCfg<kBits>::kThreads) {
      const int which = c / (kD * (kD / 8)), rem = c % (kD * (kD / 8));
      const int j = rem % kD, i0 = 8 * (rem / kD);
      const float* R = (which ? a.rot_v : a.rot_k) + (size_t)hk_base * a.rot_kv_stride;
      bf16x8_t hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = R[(size_t)(i0 + e) * kD + j];
        hi[e] = (__bf16)v;
        lo[e] = (__bf16)(v - (float)hi[e]);
      }
      *reinterpret_cast<bf16x8_t*>(&rt_hi[which][rt_index(j, i0)]) = hi;
      *reinterpret_cast<bf16x8_t*>(&rt_lo[which][rt_index(j, i0)]) = lo;
    }
  }
  if (tid < 2 * kD)
    tau_s[tid >> 7][tid & 127] = ((tid >> 7) ? a.clip_v : a.clip_k)[(size_t)hk_base * a.clip_kv_stride + (tid & 127)];
  __syncthreads();

  // waves 0..kTW-1 demote K, the others V; the loop is compiled once per
  // tensor
  auto run = [&](auto tensor) {
  constexpr int is_v = decltype(tensor)::value;
  uint8_t* img = img_all[wave];
  const int ups = a.unit_tiles;                       // units per (sequence, KV head)
  const int n_units = a.batch * heads_here * ups;
  const int stride = gridDim.x * kTW;
  const int u_first = blockIdx.x * kTW + wave % kTW;  // this wave's units: u_first + stride * j
  // A work unit: kPages history pages of one (sequence, KV head), starting at
  // the page that holds the sequence's first demoted token; one K wave and
  // one V wave take it.  Its metadata (demoted count, first demoted
  // position, physical pages) is loaded for kMeta units at a time into
  // lanes: lane kPages * jj + p holds page p of unit jj of the batch, so the
  // loop body issues no dependent loads.
  constexpr int kMeta = 64 / kPages;
  int m_pg = 0, m_cnt = 0, m_h0 = 0;
  auto fill_meta = [&](int j0) {
    const int jj = lane / kPages, p = lane % kPages;
    const int uu = u_first + stride * (j0 + jj);
    m_pg = 0;
    m_cnt = 0;
    m_h0 = 0;
    if (jj < kMeta && uu < n_units) {
      const int b = uu / (heads_here * ups), ui = (uu % (heads_here * ups)) % ups;
      const int cnt = a.length ? max(0, a.length[b] - kSink - kRecent) : a.n_tokens;
      const int h0 = a.hist_start ? a.hist_start[b] : 0;
      const int page = (h0 >> 4) + kPages * ui + p;
      m_cnt = cnt;
      m_h0 = h0;
      if (cnt > 0 && 16 * page < h0 + cnt) {
        const int slot = a.seq_slot ? a.seq_slot[b] : b;
        m_pg = a.page_table[(size_t)slot * a.max_pages + page];
      }
    }
    // wait here (vmcnt 0), so that reading the lanes later never waits on
    // the stores and tile loads in flight
    __builtin_amdgcn_s_waitcnt(0x0F70);
  };
  struct Unit {
    int b, hk, count, h0, page0, n_pg;
    int pg[kPages];
    bool live;
  };
  // unit j of the wave, jj = j - (first unit of the loaded metadata)
  auto unit_at = [&](int j, int jj) {
    Unit w{};
    const int uu = u_first + stride * j;
    w.live = false;
    if (uu >= n_units) return w;
    w.b = uu / (heads_here * ups);
    const int rem = uu % (heads_here * ups);
    w.hk = hk_base + rem / ups;
    w.count = __builtin_amdgcn_readlane(m_cnt, kPages * jj);
    w.h0 = __builtin_amdgcn_readlane(m_h0, kPages * jj);
    w.page0 = (w.h0 >> 4) + kPages * (rem % ups);
    w.n_pg = 0;
#pragma unroll
    for (int p = 0; p < kPages; ++p) {
      w.pg[p] = __builtin_amdgcn_readlane(m_pg, kPages * jj + p);
      w.n_pg += (16 * (w.page0 + p) < w.h0 + w.count) ? 1 : 0;
    }
    w.live = w.count > 0 && w.n_pg > 0;
    return w;
  };
  // this lane's source token of page p of unit w (clamped to a demoted one;
  // a unit with no work reads its sequence's first source row, or that of
  // sequence 0 past the last unit, which a launch always has)
  auto src_row = [&](const Unit& w, int p) -> size_t {
    const int idx = w.live ? min(max(16 * (w.page0 + p) + t - w.h0, 0), w.count - 1) : 0;
    return (((size_t)w.b * a.src_tokens + a.src_tok0 + idx) * a.hkv + w.hk) * kD;
  };
  // this wave's tensor inputs of a unit, as the B operands of the rotation
  // (lane (t, g): token t of each page, input channels 32 kk + 8 g .. + 7)
  typedef bf16x8_t UnitX[kPages][4];
  const uint16_t* src_x = is_v ? a.src_v : a.src_k;
  auto load_x = [&](const Unit& w, UnitX& x) {
    if constexpr (!kRotatedInput) {
#pragma unroll
      for (int p = 0; p < kPages; ++p) {
        const uint16_t* src = src_x + src_row(w, p);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) x[p][kk] = *reinterpret_cast<const bf16x8_t*>(src + 32 * kk + 8 * g);
      }
    }
  };
  const __bf16* rth = rt_hi[is_v];
  const __bf16* rtl = rt_lo[is_v];
  // acc[p][m] = rotated channels 32 g + 4 m + i of token t of page p
  auto rotate = [&](const UnitX& x, float4_t (&acc)[kPages][8]) {
    // R^T fragments f = 8 kk + m stream from LDS kAhead steps ahead of the
    // products that use them (a ring of kAhead + 1)
    constexpr int kAhead = 3;
    bf16x8_t fh[kAhead + 1], fl[kAhead + 1];
    auto frag = [&](int f, bf16x8_t& h, bf16x8_t& l) {
      const int row = rt_index(out_channel(f & 7, t), 32 * (f >> 3) + 8 * g);
      h = *reinterpret_cast<const bf16x8_t*>(&rth[row]);
      l = *reinterpret_cast<const bf16x8_t*>(&rtl[row]);
    };
#pragma unroll
    for (int f = 0; f < kAhead; ++f) frag(f, fh[f], fl[f]);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 0);     // LDS reads
#pragma unroll
    for (int f = 0; f < 32; ++f) {
      const int kk = f >> 3, m = f & 7;
      if (f + kAhead < 32) {
        frag(f + kAhead, fh[(f + kAhead) % (kAhead + 1)], fl[(f + kAhead) % (kAhead + 1)]);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * kPages, 0);   // matrix products
      const bf16x8_t ah = fh[f % (kAhead + 1)], al = fl[f % (kAhead + 1)];
      // the first product of each accumulator takes a zero C operand
#pragma unroll
      for (int p = 0; p < kPages; ++p)
        acc[p][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, x[p][kk], kk == 0 ? (float4_t){0.f, 0.f, 0.f, 0.f} : acc[p][m],
                                                            0, 0, 0);
#pragma unroll
      for (int p = 0; p < kPages; ++p) acc[p][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, x[p][kk], acc[p][m], 0, 0, 0);
    }
  };
  // this wave's bytes of a block <-> its image of the page: the code bytes
  // (INT2: 8 bytes of each 16-byte row, INT4: 16 contiguous bytes per lane)
  // and 4 bytes per lane of the tensor's 256 metadata bytes
  constexpr int kCodeOff = kBits == 4 ? 1024 * is_v : 8 * is_v;   // first code byte of lane 0 in the block
  constexpr int kCodeStride = kBits == 4 ? 16 : 16;                // block bytes between lanes' code bytes
  constexpr int kMetaOff = DemCfg<kBits>::kMetaBase + 256 * is_v;
  auto part_read = [&](const uint8_t* blk, uint8_t* im) {
    if constexpr (kBits == 4)
      *reinterpret_cast<u32x4_t*>(im + 16 * lane) = *reinterpret_cast<const u32x4_t*>(blk + kCodeOff + kCodeStride * lane);
    else
      *reinterpret_cast<uint64_t*>(im + 8 * lane) = *reinterpret_cast<const uint64_t*>(blk + kCodeOff + kCodeStride * lane);
    *reinterpret_cast<uint32_t*>(im + kCodeBytes + 4 * lane) = *reinterpret_cast<const uint32_t*>(blk + kMetaOff + 4 * lane);
  };
  // stores through a buffer resource: a page with nothing to store gets an
  // empty range, which the hardware drops, so every path issues the same
  // stores (and the waits before the next products need not cover them)
  auto part_store = [&](uint8_t* blk, bool store, const uint8_t* im) {
    const auto r = __builtin_amdgcn_make_buffer_rsrc(blk, (short)0, store ? kBytes : 0, 0x00020000);
    if constexpr (kBits == 4)
      __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4_t*>(im + 16 * lane), r, kCodeOff + kCodeStride * lane, 0, 0);
    else
      __builtin_amdgcn_raw_buffer_store_b64(*reinterpret_cast<const u32x2_t*>(im + 8 * lane), r, kCodeOff + kCodeStride * lane, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(*reinterpret_cast<const uint32_t*>(im + kCodeBytes + 4 * lane), r, kMetaOff + 4 * lane, 0, 0);
  };

  int jb = 0;                                          // first unit of the loaded metadata
  fill_meta(0);
  Unit cur = unit_at(0, 0);
  UnitX x;
  load_x(cur, x);
  // the stores that follow the loads in every round, here with empty ranges,
  // so that the loop is entered with the memory counter it keeps
#pragma unroll
  for (int p = 0; p < kPages; ++p) part_store(a.hist, false, img + p * kPart);
  for (int j = 0; u_first + stride * j < n_units; ++j) {
    if (j + 1 - jb == kMeta) {                           // wave-uniform
      jb += kMeta;
      fill_meta(jb);
    }
    const Unit nxt = unit_at(j + 1, j + 1 - jb);
    // (the branches below are wave-uniform; the next unit's loads sit at the
    // same point whether or not this unit has work, into the same registers)
    uint8_t* blk[kPages];
#pragma unroll
    for (int p = 0; p < kPages; ++p) blk[p] = a.hist + ((size_t)cur.pg[p] * a.hkv + cur.hk) * kBytes;
    if (cur.live) {
      // pages only partly covered keep their other slots: read them into the image
#pragma unroll
      for (int p = 0; p < kPages; ++p) {
        const int first = 16 * (cur.page0 + p);
        if (p < cur.n_pg && (first < cur.h0 || first + 16 > cur.h0 + cur.count)) part_read(blk[p], img + p * kPart);
      }
    }
    auto valid_tok = [&](int p) {
      const int h = 16 * (cur.page0 + p) + t;
      return p < cur.n_pg && h >= cur.h0 && h < cur.h0 + cur.count;
    };
    float4_t acc[kPages][8];
    if constexpr (kRotatedInput) {
      if (cur.live) {
#pragma unroll
        for (int p = 0; p < kPages; ++p) {
          const float* src = (is_v ? a.src_v_f32 : a.src_k_f32) + src_row(cur, p) + 32 * g;
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const float4 v4 = *reinterpret_cast<const float4*>(src + 4 * m);
            acc[p][m] = (float4_t){v4.x, v4.y, v4.z, v4.w};
          }
        }
      }
    } else {
      // (on every path: a dead unit rotates the valid rows it loaded, so the
      // loads are always consumed here)
      rotate(x, acc);
    }
    auto quant_page = [&](int p) {
      float y[8][4];
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) y[m][i] = acc[p][m][i];
      if constexpr (kBits == 2) {
        quant_pack_int2(y, &tau_s[is_v][32 * g], is_v != 0, t, g, valid_tok(p), img + p * kPart);
      } else {
        uint32_t code[8][4];
        __half sc, zr;
        quant_lane_group4(y, &tau_s[is_v][32 * g], code, sc, zr);
        pack_lane_group4(code, sc, zr, is_v != 0, t, g, valid_tok(p), img + p * kPart);
      }
    };
    if (cur.live) quant_page(0);                       // a live unit has its first page
    // the next unit's inputs go out once the products have consumed the
    // current ones and the first page's accumulators are free; they are
    // issued on every path (a dead unit reads a valid row), so the waits
    // before the next products count exactly the loads and stores issued since
    load_x(nxt, x);
    if (cur.live) {
#pragma unroll
      for (int p = 1; p < kPages; ++p) {
        __builtin_amdgcn_sched_barrier(0);
        if (p < cur.n_pg) quant_page(p);
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int p = 0; p < kPages; ++p) part_store(blk[p], cur.live && p < cur.n_pg, img + p * kPart);
    __builtin_amdgcn_wave_barrier();
    cur = nxt;
  }
  };
  if (wave < kTW) run(std::integral_constant<int, 0>{});
  else run(std::integral_constant<int, 1>{});
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
  // units of kPages history pages from the page holding each sequence's
  // first demoted token (up to 15 slots before it)
  const int pages_per_unit = a.code_bits == 4 ? DemCfg<4>::kPages : DemCfg<2>::kPages;
  a.unit_tiles = (15 + max_count + 16 * pages_per_unit - 1) / (16 * pages_per_unit);
  // one workgroup per compute unit (each stages R_K and R_V once); with one
  // R per KV head, a slice of them per KV head (grid z)
  const bool per_head = a.clip_kv_stride != 0;
  const int heads = per_head ? a.hkv : 1;
  const long units = (long)batch * (per_head ? 1 : a.hkv) * a.unit_tiles;
  const int tw = a.code_bits == 4 ? DemCfg<4>::kTensorWaves : DemCfg<2>::kTensorWaves;   // units per round
  const int nwg = (int)std::min<long>((units + tw - 1) / tw, std::max(1, 256 / heads));
  const dim3 grid(nwg, 1, heads);
  if (a.code_bits == 4) {
    constexpr int kT = DemCfg<4>::kThreads;
    if (rotated)
      hipLaunchKernelGGL((demote_bulk_kernel<true, 4>), grid, dim3(kT), 0, st, a);
    else
      hipLaunchKernelGGL((demote_bulk_kernel<false, 4>), grid, dim3(kT), 0, st, a);
  } else {
    constexpr int kT = DemCfg<2>::kThreads;
    if (rotated)
      hipLaunchKernelGGL((demote_bulk_kernel<true, 2>), grid, dim3(kT), 0, st, a);
    else
      hipLaunchKernelGGL((demote_bulk_kernel<false, 2>), grid, dim3(kT), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_route(const PrefillArgs& a, int batch, hipStream_t st) {
  hipLaunchKernelGGL(prefill_route_kernel, dim3((kSink + kRecent) / 16, batch * a.hkv, 2), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace oscar
