/*
 * oscar.h -- C ABI of libamdoscar.so: OSCAR-style 2-bit KV-cache demotion and
 * tiered decode attention on AMD Instinct MI355X (gfx950), with an INT4
 * variant of the same history pool.
 *
 * Pages cited (title, site):
 *   [gist]    "OSCAR: Offline Spectral Covariance-Aware Rotation for 2-bit KV
 *             Cache Quantization" (gist.science), "Technische Zusammenfassung"
 *             sections 2.1, 2.2 A (Offline-Kalibrierungsphase), 2.2 B
 *             (Online-Betriebsphase).
 *   [zingnex] "OSCAR：面向2-bit KV缓存量化的谱协方差感知旋转方法" (zingnex.cn),
 *             sections 离线协方差估计, 自定义INT2注意力内核, 离线优化的优势.
 *   [yunpan]  "大模型KV Cache 2bit量化实战：OSCAR让显存暴降90%且智商不掉线"
 *             (yunpan.plus), sections 三.1 三段式 Token 池, 三.2 在线量化与反量化,
 *             三.3 兼容现有架构.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - head_dim = 128, page = 16 tokens, sink = 64 tokens, recent ring = 256
 *   tokens, quantisation group = 32 channels.  Other values return
 *   OSCAR_ERR_UNSUPPORTED.  num_q_heads / num_kv_heads (the GQA group G) must
 *   be 1, 2, 4 or 8.
 * - Rotations act on row vectors: y = x . R, R stored row-major fp32
 *   [128][128]; the inverse rotation is y . R^T.  A pool holds either one
 *   R_K, R_V and clip-threshold pair per layer, shared by its KV heads, or
 *   one per KV head (oscar_pool.rot_per_kv_head).
 * - "device" pointers are HIP device memory owned by the caller (for example
 *   torch tensors); "host" pointers are ordinary host memory.  The library
 *   never allocates, frees or retains any caller buffer.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   Device entry points only enqueue work on it and return; they do not
 *   synchronise.  Argument checks happen on the host before anything is
 *   enqueued: a negative status means nothing was enqueued.  A launch failure
 *   reported by the runtime returns OSCAR_ERR_HIP.  Values inside device
 *   buffers (page ids, lengths, positions) are not checked on the host: an
 *   out-of-range value there is undefined behaviour.
 * - Calls are stateless and reentrant apart from the decode workspace, which
 *   one call at a time may use.
 *
 * Pool layout (device)
 * --------------------
 *   sink_k/sink_v     bf16 [n_slots][Hkv][64][128]      positions 0..63
 *   recent_k/recent_v bf16 [n_slots][Hkv][256][128]     position p >= 64 in
 *                                                        ring slot (p-64) mod 256
 *   hist              u8   [num_pages][Hkv][1536]       INT2 history blocks
 *   page_table        i32  [n_slots][max_pages_per_seq] history index h (= p-64)
 *                                                        lives in page
 *                                                        page_table[s][h/16],
 *                                                        slot h%16
 * Three tiers as in [yunpan] 三.1 and [gist] 2.2 B: BF16 sink, INT2 history
 * of rotated and clipped vectors, BF16 recent tokens.
 *
 * History block of one (page, KV head), 1536 bytes (this library's format;
 * the pages fix only "four 2-bit codes per byte", [yunpan] 三.2):
 *   [0,1024)    64 chunks of 16 bytes.  Chunk c = 16a + b:
 *               bytes 0..7  = K codes of token b, channels with ((j>>3)&3)==a:
 *                             32-bit word w = j>>6, 2-bit field
 *                             4((j>>5)&1) + ((j>>1)&3) + 8(j&1);
 *               bytes 8..15 = V codes of tokens 4a..4a+3, channels with
 *                             (j&15)==b: word (t&3)>>1, field (j>>4) + 8(t&1).
 *   [1024,1152) K scale fp16 [token][group]
 *   [1152,1280) K zero  fp16 [token][group]
 *   [1280,1408) V scale fp16 [token/4][group][token%4]
 *   [1408,1536) V zero  fp16 [token/4][group][token%4]
 * A code c of group g dequantises to c * scale + zero in the rotated space.
 *
 * INT4 pools (oscar_pool.code_bits = 4; the INT4 baseline of [gist] 4): 16
 * levels (scale from (max - zero) / 15, codes 0..15), two codes per byte, one
 * 2560-byte block per (page, KV head), so hist is u8 [num_pages][Hkv][2560]:
 *   [0,1024)    K codes, 64 chunks of 16 bytes.  Chunk 16a + t holds token
 *               t's channels j with ((j>>3)&3)==a: 32-bit word j>>5, 4-bit
 *               field at bit 16(j&1) + 4((j>>1)&3).
 *   [1024,2048) V codes, 64 chunks of 16 bytes.  Chunk 16a + b holds tokens
 *               4a..4a+3, channels j with (j&15)==b: word 2((j>>4)>>2) +
 *               ((t&3)>>1), field at bit 16(t&1) + 4((j>>4)&3).
 *   [2048,2560) K scale, K zero, V scale, V zero: the INT2 block's
 *               [1024,1536) layout moved up by 1024 bytes.
 * The caller zero-fills hist when it allocates it; afterwards every byte of
 * a block is either zero or written by this library.  (Decode reads whole
 * pages and relies on the metadata of not-yet-written slots being finite.)
 */
#ifndef OSCAR_H
#define OSCAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OSCAR_ABI_VERSION 6

typedef enum {
  OSCAR_OK = 0,
  OSCAR_ERR_INVALID = -1,     /* null pointer, bad count, inconsistent sizes   */
  OSCAR_ERR_UNSUPPORTED = -2, /* shape outside the supported set (see above)   */
  OSCAR_ERR_CAPACITY = -3,    /* workspace or page table too small            */
  OSCAR_ERR_HIP = -4,         /* the HIP runtime reported a launch failure     */
  OSCAR_ERR_NUMERIC = -5      /* calibration produced a non-finite or too large
                                 value (clip threshold > 65504)               */
} oscar_status;

typedef struct {
  int32_t num_q_heads;  /* Hq                                 */
  int32_t num_kv_heads; /* Hkv; Hq % Hkv == 0, Hq/Hkv in {1,2,4,8} */
  int32_t head_dim;     /* must be 128                        */
  int32_t page_size;    /* must be 16                         */
  int32_t n_sink;       /* must be 64                         */
  int32_t n_recent;     /* must be 256                        */
  int32_t group_size;   /* must be 32                         */
} oscar_layer_desc;

typedef struct {
  void* sink_k;                /* device bf16, layout above                  */
  void* sink_v;
  void* recent_k;              /* device bf16, layout above                  */
  void* recent_v;
  uint8_t* hist;               /* device, [num_pages][Hkv][1536] (INT2) or
                                  [num_pages][Hkv][2560] (INT4)              */
  const int32_t* page_table;   /* device, [n_slots][max_pages_per_seq]       */
  int32_t n_slots;
  int32_t max_pages_per_seq;
  int32_t num_pages;
  const float* rot_k;          /* device fp32 [128][128]: R_K, y = x . R_K   */
  const float* rot_v;          /* device fp32 [128][128]: R_V                */
  const float* clip_k;         /* device fp32 [128]: per rotated channel     */
  const float* clip_v;         /*   clip thresholds, 0 < tau <= 65504        */
  int32_t code_bits;           /* 2: INT2 history (1536-byte blocks); 4: INT4
                                  (2560-byte blocks, see above)              */
  int32_t rot_per_kv_head;     /* 0: the four arrays above are the layer's,
                                  shared by every KV head.  1: one per KV
                                  head, rot_k/rot_v [Hkv][128][128] and
                                  clip_k/clip_v [Hkv][128]; KV head j's
                                  vectors (and its query heads' queries) are
                                  rotated by its own pair.                   */
} oscar_pool;

/* Rotation that oscar_calibrate builds (oscar_calib_opts.rotation). */
enum {
  OSCAR_ROT_SPECTRAL = 0,      /* the method: R_K = U_Q H P_br, R_V = U_S H P_br
                                  ([gist] 2.2 A)                               */
  OSCAR_ROT_KEY_ATTN = 1,      /* R_K from the eigenbasis of the attention-
                                  weighted key covariance
                                  C_SK = (1/(N Hq)) sum_h (S_h K)^T (S_h K),
                                  the value target with keys in place of
                                  values; R_V as in OSCAR_ROT_SPECTRAL        */
  OSCAR_ROT_HADAMARD = 2,      /* R_K = R_V = H P_br: the data-blind rotation
                                  the pages compare against ([gist] 3 and 4) */
  OSCAR_ROT_IDENTITY = 3       /* R_K = R_V = I: plain INT2 ([gist] 4)        */
};

typedef struct {
  int32_t hadamard_block;      /* 32 (one quantisation group) or 128         */
  float clip_percentile;       /* e.g. 99.0                                   */
  int32_t rotation;            /* OSCAR_ROT_*                                 */
  int32_t per_kv_head;         /* 0: one R_K, R_V, tau per layer; 1: one per
                                  KV head (outputs [Hkv][128][128] and
                                  [Hkv][128]), each calibrated from that KV
                                  head's G query heads, keys and values alone */
} oscar_calib_opts;

/* Source formats accepted by oscar_demote. */
enum {
  OSCAR_SRC_BF16 = 0,          /* unrotated bf16 K/V: rotate, clip, quantise */
  OSCAR_SRC_F32_ROTATED = 1    /* already-rotated fp32 K/V: clip, quantise   */
};

/* ABI version of the loaded library (OSCAR_ABI_VERSION). */
int32_t oscar_abi_version(void);

/* Human-readable name of a status code (static storage). */
const char* oscar_status_string(oscar_status s);

/*
 * oscar_calibrate -- offline calibration of one layer, on the host.
 * [gist] 2.1 and 2.2 A; [zingnex] 离线协方差估计 and 离线优化的优势 (fixed
 * rotation computed offline).
 *   C_Q = (1/(N Hq)) sum_{n,h} q_{n,h}^T q_{n,h}                 (key target)
 *   C_S = (1/(N Hq)) sum_h (S_h V_{h/G})^T (S_h V_{h/G}),  S_h the causal
 *         softmax of Q_h K_{h/G}^T / sqrt(128)                    (value target)
 *   U_Q, U_S = eigenvectors, descending eigenvalues, each column's largest
 *         entry made positive;  R = U . H_Had . P_br with H_Had block-diagonal
 *         normalised Sylvester Hadamard and P_br the 7-bit bit reversal;
 *   tau = per rotated channel percentile of |x . R| over all tokens and KV
 *         heads, separately for K and V.
 * In:  q host fp32 [n_tokens][Hq][128]; k, v host fp32 [n_tokens][Hkv][128]
 *      (token-major, one calibration sequence, causal).
 * opts->rotation picks the rotation (OSCAR_ROT_SPECTRAL is the method; the
 * others are the baselines and the alternative key target above); the clip
 * thresholds are always the percentiles of the chosen rotation's outputs.
 * Out: rot_k, rot_v host fp32 [128][128]; clip_k, clip_v host fp32 [128].
 * With opts->per_kv_head = 1 every KV head j is calibrated as a layer of its
 * own (its query heads jG..jG+G-1, its keys and values), and the outputs are
 * rot_k, rot_v [Hkv][128][128], clip_k, clip_v [Hkv][128].
 * Synchronous, CPU only, uses up to the machine's cores.  Errors:
 * OSCAR_ERR_INVALID (null pointer, n_tokens < 2, unknown rotation or
 * per_kv_head not 0/1), OSCAR_ERR_UNSUPPORTED, OSCAR_ERR_NUMERIC (non-finite
 * input or tau > 65504).
 */
oscar_status oscar_calibrate(const oscar_layer_desc* desc, const oscar_calib_opts* opts,
                             const float* q, const float* k, const float* v, int64_t n_tokens,
                             float* rot_k, float* rot_v, float* clip_k, float* clip_v);

/*
 * oscar_calibrate_layers -- one calibration shared by n_layers layers of the
 * same shape ([zingnex] 离线优化的优势: layers may share their rotation
 * parameters).  The key and value targets are the means of the layers' own
 * targets (each layer's attention causal within its own n_tokens tokens);
 * the clip thresholds are the percentiles over every layer's rotated keys
 * (values).  In: q host fp32 [n_layers][n_tokens][Hq][128]; k, v host fp32
 * [n_layers][n_tokens][Hkv][128].  Outputs, options and errors as for
 * oscar_calibrate (n_layers < 1: OSCAR_ERR_INVALID); n_layers = 1 is
 * oscar_calibrate.
 */
oscar_status oscar_calibrate_layers(const oscar_layer_desc* desc, const oscar_calib_opts* opts,
                                    int32_t n_layers, const float* q, const float* k, const float* v,
                                    int64_t n_tokens, float* rot_k, float* rot_v, float* clip_k,
                                    float* clip_v);

/*
 * oscar_append -- route one new token per sequence into the tiered pool
 * ([yunpan] 三.1 and 三.2; [gist] 2.2 B).  For batch entry b with slot
 * s = seq_slot[b] (seq_slot may be NULL: s = b) and new position
 * p = position[b] (the number of tokens already cached):
 *   p < 64:   write the token to sink[s][:, p];
 *   p >= 64:  ring slot r = (p-64) mod 256; if p >= 320 the token at ring
 *             slot r (position p-256) is first demoted -- rotated by R,
 *             clipped, quantised to INT2 and packed -- into history index
 *             p-320; then the new token overwrites ring slot r.
 * k_new, v_new: device bf16 [batch][Hkv][128].  position, seq_slot: device
 * int32 [batch].  The caller guarantees page_table[s][(p-320)/16] is a valid
 * page when p >= 320, and that no two batch entries name the same slot.
 * Positions are not advanced by the call.
 */
oscar_status oscar_append(const oscar_layer_desc* desc, const oscar_pool* pool,
                          const int32_t* seq_slot, const int32_t* position,
                          const void* k_new, const void* v_new, int32_t batch, void* stream);

/*
 * oscar_demote -- bulk demotion of n_tokens consecutive history tokens per
 * sequence (rotate -> clip -> quantise -> pack, [yunpan] 三.2), written to
 * history indices hist_start[b] .. hist_start[b]+n_tokens-1 of slot
 * seq_slot[b].  Source k, v: device [batch][n_tokens][Hkv][128], bf16
 * unrotated (OSCAR_SRC_BF16; the rotation uses the matrix cores) or fp32
 * already rotated (OSCAR_SRC_F32_ROTATED; only clip, quantise, pack -- the
 * bit-exact reference entry).  hist_start, seq_slot: device int32 [batch]
 * (seq_slot may be NULL).  Pages touched must be valid in page_table; tokens
 * outside the written range keep their bytes.
 */
oscar_status oscar_demote(const oscar_layer_desc* desc, const oscar_pool* pool,
                          const int32_t* seq_slot, const int32_t* hist_start,
                          const void* k, const void* v, int32_t src_kind,
                          int32_t batch, int32_t n_tokens, void* stream);

/*
 * oscar_prefill -- place whole fresh sequences into the tiers, with the
 * same result as appending their tokens one at a time: positions [0, 64)
 * to the sink, [64, n-256) demoted to history, the last min(n-64, 256)
 * positions to the recent ring.  k, v: device bf16
 * [batch][max_len][Hkv][128]; length: device int32 [batch], n = length[b]
 * <= max_len.  seq_slot as above.
 */
oscar_status oscar_prefill(const oscar_layer_desc* desc, const oscar_pool* pool,
                           const int32_t* seq_slot, const int32_t* length,
                           const void* k, const void* v, int32_t batch, int32_t max_len,
                           void* stream);

/*
 * oscar_decode -- single-token decode attention over the tiered pool
 * ([gist] 2.2 B "Kernel-Integration": unpack, dequantise, inverse rotation and
 * attention fused; [zingnex] 自定义INT2注意力内核).  For batch entry b with
 * slot s and n = seq_len[b] cached tokens (counting the token appended this
 * step) and each query head h (KV head h / G):
 *   out[b][h] = softmax(q[b][h] . K~^T / sqrt(128)) . V~
 * where K~, V~ hold the BF16 sink and recent tokens and, for history,
 * dequant(codes) . R^T.  History is scored in the rotated space (q . R_K),
 * accumulated there, and rotated back once (. R_V^T) after the split-K
 * partial results are merged by log-sum-exp.
 * q: device bf16 [batch][Hq][128].  out: device fp32 [batch][Hq][128].
 * seq_len, seq_slot: device int32 [batch]; every seq_len[b] must be in
 * [1, max_seq_len].  workspace: device, at least
 * oscar_decode_workspace_bytes(desc, batch, max_seq_len) bytes, needing no
 * initialisation: the call runs as two kernels on `stream` (the split
 * partials, then their merge) that pass the partials through it, so calls
 * sharing one workspace must be ordered (one stream).  Errors:
 * OSCAR_ERR_CAPACITY if ws_bytes is too small or max_seq_len needs more pages
 * than max_pages_per_seq.
 */
oscar_status oscar_decode(const oscar_layer_desc* desc, const oscar_pool* pool,
                          const int32_t* seq_slot, const int32_t* seq_len, const void* q,
                          float* out, void* workspace, size_t ws_bytes, int32_t batch,
                          int32_t max_seq_len, void* stream);

size_t oscar_decode_workspace_bytes(const oscar_layer_desc* desc, int32_t batch,
                                    int32_t max_seq_len);

/*
 * oscar_decode_partials, oscar_decode_merge -- the two phases of
 * oscar_decode as separate calls ([gist] 2.2 B; split-K over the paged
 * history with a log-sum-exp merge).  oscar_decode_partials runs the split
 * kernel only: every split of every (sequence, KV head) writes its running
 * maximum, softmax sum and unnormalised output (history splits in the
 * rotated space) to the workspace.  oscar_decode_merge then merges them,
 * rotates the history part back with R_V^T and writes out.  The two calls in
 * this order on one stream, with the same desc, pool, seq_len, batch,
 * max_seq_len and workspace, compute exactly what oscar_decode computes (it
 * is these two launches).  The records are private to the library: the
 * workspace holds them only from a partials call to the next call that uses
 * the workspace, and a merge is meaningful only after a partials call with
 * the same arguments.  For callers that schedule or time the phases apart.
 * Arguments as for oscar_decode; the partials call does not read `out`, the
 * merge does not read q or seq_slot (either may be NULL there).  Errors as
 * for oscar_decode.
 */
oscar_status oscar_decode_partials(const oscar_layer_desc* desc, const oscar_pool* pool,
                                   const int32_t* seq_slot, const int32_t* seq_len, const void* q,
                                   void* workspace, size_t ws_bytes, int32_t batch,
                                   int32_t max_seq_len, void* stream);
oscar_status oscar_decode_merge(const oscar_layer_desc* desc, const oscar_pool* pool,
                                const int32_t* seq_len, float* out, void* workspace, size_t ws_bytes,
                                int32_t batch, int32_t max_seq_len, void* stream);

/*
 * oscar_step -- one decode step of a layer in one call: oscar_append of the
 * new token (k_new, v_new at position[b], as there) followed by oscar_decode
 * of q over the position[b] + 1 cached tokens ([yunpan] 三.1: the new token is
 * appended before it attends; [gist] 2.2 B).  Two launches, the decode's:
 * the split launch also appends.  Before position 320 the new token goes
 * into its sink or free ring slot; from position 320 on, the history split
 * that owns the newest history token reads the token leaving the ring,
 * writes the new token into that ring slot, demotes the leaving token
 * (rotate, clip, quantise, pack, store; the same routine and rotation
 * arithmetic as oscar_append) and attends to it from its registers, while
 * the page walk covers the older history.  The BF16 tiles read the new
 * token from k_new / v_new.  Results equal oscar_append followed by
 * oscar_decode up to fp32 summation order, and the pool afterwards holds
 * the same bytes.
 * position, seq_slot: device int32 [batch] (positions before the append, not
 * advanced by the call); q: device bf16 [batch][Hq][128]; out: device fp32
 * [batch][Hq][128]; max_seq_len >= max(position) + 1.  workspace: device,
 * at least oscar_step_workspace_bytes(desc, batch, max_seq_len) bytes, no
 * initialisation needed, one call at a time.  Errors as oscar_append and
 * oscar_decode.
 */
oscar_status oscar_step(const oscar_layer_desc* desc, const oscar_pool* pool, const int32_t* seq_slot,
                        const int32_t* position, const void* k_new, const void* v_new, const void* q,
                        float* out, void* workspace, size_t ws_bytes, int32_t batch, int32_t max_seq_len,
                        void* stream);

/* Workspace of oscar_step: the decode's (oscar_decode_workspace_bytes);
 * 0 for an unsupported shape. */
size_t oscar_step_workspace_bytes(const oscar_layer_desc* desc, int32_t batch, int32_t max_seq_len);

/*
 * oscar_step_noalloc -- oscar_step for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels and results as oscar_step, with the
 * workspace in a static device array of OSCAR_NOALLOC_SCRATCH_BYTES bytes
 * that the library holds on each GPU it runs on until the process ends.
 * The call allocates and frees nothing.  Arguments as for oscar_step
 * without workspace and ws_bytes; the GPU is the device of `stream` (the
 * current device for the null stream).  Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (concurrent streams or
 * threads) race and must be serialised by the caller.  No byte of the array
 * has to start at any value (each call writes everything it reads first).
 * Errors: as oscar_step; OSCAR_ERR_CAPACITY when
 * oscar_step_workspace_bytes(desc, batch, max_seq_len) exceeds
 * OSCAR_NOALLOC_SCRATCH_BYTES (use oscar_step with a caller workspace);
 * OSCAR_ERR_HIP if the array's device address cannot be resolved.
 */
#define OSCAR_NOALLOC_SCRATCH_BYTES (8u << 20)
oscar_status oscar_step_noalloc(const oscar_layer_desc* desc, const oscar_pool* pool, const int32_t* seq_slot,
                                const int32_t* position, const void* k_new, const void* v_new, const void* q,
                                float* out, int32_t batch, int32_t max_seq_len, void* stream);

/*
 * oscar_decode_multi -- several query tokens per sequence over the tiered
 * pool (speculative verification of draft tokens, chunked prefill), the
 * same attention as oscar_decode ([gist] 2.2 B; [zingnex] 自定义INT2注意力内核)
 * with a causal limit.  The n_query queries of batch entry b are its last
 * n_query positions: with n = seq_len[b] cached tokens (the queries' own
 * tokens already appended), query t (0 <= t < n_query) sits at position
 * p = n - n_query + t and, for each query head h,
 *   out[b][t][h] = softmax(q[b][t][h] . K~[0..p]^T / sqrt(128)) . V~[0..p].
 * n_query <= 256 keeps every query inside the BF16 recent tier, so every
 * INT2 history token is visible to every query and the causal limit only
 * cuts the BF16 tiers.
 * q: device bf16 [batch][n_query][Hq][128]; out: device fp32
 * [batch][n_query][Hq][128]; seq_len[b] must be in [n_query, max_seq_len]
 * (a shorter length leaves queries that see no token, whose output is 0).
 * The work is split as for oscar_decode, with the (query token, head) pairs
 * of a KV head as the columns of the matrix-core products (up to 16 per work
 * item); n_query = 1 is exactly oscar_decode.  Workspace: oscar_decode_multi_workspace_bytes(desc,
 * batch, n_query, max_seq_len) bytes, rules as for oscar_decode.  Errors as
 * for oscar_decode, plus OSCAR_ERR_INVALID for n_query < 1 or
 * n_query > max_seq_len and OSCAR_ERR_UNSUPPORTED for n_query > 256.
 */
oscar_status oscar_decode_multi(const oscar_layer_desc* desc, const oscar_pool* pool,
                                const int32_t* seq_slot, const int32_t* seq_len, const void* q,
                                int32_t n_query, float* out, void* workspace, size_t ws_bytes,
                                int32_t batch, int32_t max_seq_len, void* stream);

size_t oscar_decode_multi_workspace_bytes(const oscar_layer_desc* desc, int32_t batch,
                                          int32_t n_query, int32_t max_seq_len);

/*
 * BF16 paged baseline (the full-precision cache INT2 is compared against;
 * [zingnex] 系统级收益 / 解码加速 report speed-ups over BF16).
 *   kv: device bf16 [num_pages][Hkv][2][16][128] (K page then V page);
 *   page_table: device int32 [n_slots][max_pages_per_seq]; token p of slot s
 *   lives in page page_table[s][p/16], row p%16.
 * oscar_decode_bf16 computes out[b][h] = softmax(q . K^T / sqrt(128)) . V over
 * all seq_len[b] tokens, with the same split-K / log-sum-exp structure as
 * oscar_decode.  Workspace rules as for oscar_decode.
 */
typedef struct {
  const void* kv;
  const int32_t* page_table;
  int32_t n_slots;
  int32_t max_pages_per_seq;
  int32_t num_pages;
} oscar_bf16_pool;

oscar_status oscar_decode_bf16(const oscar_layer_desc* desc, const oscar_bf16_pool* pool,
                               const int32_t* seq_slot, const int32_t* seq_len, const void* q,
                               float* out, void* workspace, size_t ws_bytes, int32_t batch,
                               int32_t max_seq_len, void* stream);

size_t oscar_decode_bf16_workspace_bytes(const oscar_layer_desc* desc, int32_t batch,
                                         int32_t max_seq_len);

/*
 * oscar_decode_bf16_multi -- the baseline for oscar_decode_multi: the last
 * n_query positions of each sequence attend causally over the BF16 paged
 * cache (query t at position n - n_query + t sees [0, n - n_query + t]).
 * q, out, seq_len and errors as for oscar_decode_multi; n_query = 1 is
 * exactly oscar_decode_bf16.  Workspace:
 * oscar_decode_bf16_multi_workspace_bytes(desc, batch, n_query, max_seq_len).
 */
oscar_status oscar_decode_bf16_multi(const oscar_layer_desc* desc, const oscar_bf16_pool* pool,
                                     const int32_t* seq_slot, const int32_t* seq_len, const void* q,
                                     int32_t n_query, float* out, void* workspace, size_t ws_bytes,
                                     int32_t batch, int32_t max_seq_len, void* stream);

size_t oscar_decode_bf16_multi_workspace_bytes(const oscar_layer_desc* desc, int32_t batch,
                                               int32_t n_query, int32_t max_seq_len);

#ifdef __cplusplus
}
#endif

#endif /* OSCAR_H */
