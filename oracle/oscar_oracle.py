"""Plain, slow, obviously-correct CPU oracle (NumPy; fp64 unless noted).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.
It shares no code with the HIP library: the page layout, the quantiser and
the attention are all written out here again from their definitions.

Pages cited (title, site), with the sections used:

* [gist]    "OSCAR: Offline Spectral Covariance-Aware Rotation for 2-bit KV
            Cache Quantization" (gist.science explainer of arXiv 2605.17757),
            "Technische Zusammenfassung" sections 2.1 (Theoretische
            Motivation), 2.2 A (Offline-Kalibrierungsphase), 2.2 B
            (Online-Betriebsphase), 4 (Experimentelle Ergebnisse).
* [zingnex] "OSCAR：面向2-bit KV缓存量化的谱协方差感知旋转方法" (zingnex.cn),
            sections 离线协方差估计, 注意力对齐的量化, 自定义INT2注意力内核,
            离线优化的优势.
* [yunpan]  "大模型KV Cache 2bit量化实战：OSCAR让显存暴降90%且智商不掉线"
            (yunpan.plus), sections 二 (2-bit has four states), 三.1
            三段式 Token 池, 三.2 在线量化与反量化, 三.3 兼容现有架构.

Readings taken where the pages are silent (each one is also listed in the
design notes of the repository):

R1  Row vectors: a rotated vector is y = x . R, and the inverse is y . R^T.
R2  C_Q pools all query heads of a layer; C_S pools all query heads, each
    attending causally to its GQA key/value head.  One R_K and one R_V per
    layer, shared by every KV head.
R3  Eigenvectors in descending eigenvalue order; each column's sign makes
    its largest-magnitude entry positive (ties: lowest index).
R4  H_Had is block-diagonal normalised Sylvester Hadamard, block 32 (one
    quantisation group); P_br is the 7-bit bit-reversal permutation,
    y_j = x_{bitrev(j)}.
R5  Clip thresholds: per rotated channel, the 99th percentile (linear
    interpolation) of |x . R| over all calibration tokens and KV heads,
    separately for K and V; clipping is to [-tau_j, tau_j] with IEEE
    minNum/maxNum.  0 < tau <= 65504 is a precondition.
R6  INT2 codes: groups of 32 rotated channels, asymmetric min-max with an
    fp16 zero z = fp16 rounded toward -inf of the group minimum, and an fp16
    scale s = fp16 rounded toward +inf of fp32((max - z) / 3); code
    c = clamp(rint_even(fp32(fp32(y - z) / s)), 0, 3), c = 0 when s = 0.
    All of this is IEEE fp32 with no fused multiply-add.  Dequantisation is
    c * s + z.
R7  Page = 16 tokens.  One 1536-byte block per (page, KV head); its byte
    layout is defined by the ``*_offset`` / ``*_bitpos`` functions below.
R8  Tiers: positions [0, 64) are the BF16 sink, the last 256 positions the
    BF16 recent ring (position p in slot (p - 64) mod 256), everything in
    between INT2 history (history index h = p - 64, page h // 16, slot
    h % 16).  A decode step appends before it attends.
R9  Softmax scale 1/sqrt(128); GQA head h reads KV head h // (Hq / Hkv);
    output in fp32 (oracle: fp64).
R10 Rotation variants for comparison: besides the method's R, the key
    eigenbasis may come from the attention-weighted key covariance
    (1/N) K^T S^T S K (pooled like C_S), and the baselines are R = H P_br
    (data-blind Hadamard) and R = I (plain INT2); the clip thresholds are
    always taken after the chosen rotation.
R11 Several query tokens per sequence: the T queries of a step are the last
    T positions n - T, ..., n - 1 of a cache that already holds all n tokens,
    and query t attends causally to positions [0, n - T + t].  With
    T <= 256 every INT2 history token precedes every query, so the causal
    limit only ever falls inside the BF16 tiers.
R12 Scope of a calibration ([zingnex] 离线优化的优势: layers may share their
    rotation).  Shared across layers: the key and value targets are the mean
    of the layers' own targets (each layer's attention stays causal within
    that layer's tokens), and tau pools every layer's rotated activations.
    Per KV head: each KV head is calibrated as a layer of its own, from its
    G query heads and its own keys and values, giving R and tau per KV head
    ([Hkv, 128, 128] and [Hkv, 128]); every vector of that KV head is
    rotated, clipped and inverse-rotated with its own pair.
R13 INT4 variant of the pool ([gist] 4 runs an INT4 baseline): the same
    quantiser with 16 levels, scale = fp16 rounded toward +inf of
    fp32((max - z) / 15), code = clamp(rint_even(...), 0, 15), two codes per
    byte; the history block of one (page, KV head) is 2560 bytes (1024 of K
    codes, 1024 of V codes, the same 512 bytes of scale/zero metadata).
"""
from __future__ import annotations

import math
import numpy as np

HEAD_DIM = 128
GROUP = 32
N_GROUPS = HEAD_DIM // GROUP
PAGE = 16
N_SINK = 64
N_RECENT = 256
BLOCK_BYTES = 1536                 # INT2 history block (reading R7)
BLOCK_BYTES_INT4 = 2560            # INT4 history block (reading R13)


def block_bytes(bits: int = 2) -> int:
    return {2: BLOCK_BYTES, 4: BLOCK_BYTES_INT4}[bits]


def levels(bits: int = 2) -> int:
    """Largest code: 3 for INT2 (four levels, [yunpan] 二), 15 for INT4."""
    return (1 << bits) - 1
MAX_TAU = 65504.0


# ---------------------------------------------------------------------------
# small numeric helpers
# ---------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> exact float64 values."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f16_round_down(x: np.ndarray) -> np.ndarray:
    """Largest float16 <= x (x float32).  Returns float16."""
    x = np.asarray(x, dtype=np.float32)
    h = x.astype(np.float16)                       # nearest, ties to even
    over = h.astype(np.float32) > x
    return np.where(over, np.nextafter(h, np.float16(-np.inf)), h).astype(np.float16)


def f16_round_up(x: np.ndarray) -> np.ndarray:
    """Smallest float16 >= x (x float32).  Returns float16."""
    x = np.asarray(x, dtype=np.float32)
    h = x.astype(np.float16)
    under = h.astype(np.float32) < x
    return np.where(under, np.nextafter(h, np.float16(np.inf)), h).astype(np.float16)


# ---------------------------------------------------------------------------
# Offline calibration  ([gist] 2.1 and 2.2 A; [zingnex] 离线协方差估计)
# ---------------------------------------------------------------------------

def query_covariance(q: np.ndarray) -> np.ndarray:
    """Query-aware key target C_Q = (1/N) sum_n q_n^T q_n ([gist] 2.2 A).

    q: [N, Hq, d]; every (token, head) row is one sample (reading R2).
    """
    x = np.asarray(q, dtype=np.float64).reshape(-1, q.shape[-1])
    return x.T @ x / x.shape[0]


def causal_attention_probs(qh: np.ndarray, kh: np.ndarray) -> np.ndarray:
    """Row-stochastic causal softmax matrix S for one head: S[n, m] for m <= n."""
    n, d = qh.shape
    logits = (qh @ kh.T) / math.sqrt(d)
    logits[np.triu_indices(n, 1)] = -np.inf
    logits -= logits.max(axis=1, keepdims=True)
    e = np.exp(logits)
    return e / e.sum(axis=1, keepdims=True)


def score_covariance(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Score-aware value target C_S = (1/N) V^T S^T S V ([gist] 2.1, 2.2 A).

    Written through the identity V^T S^T S V = (S V)^T (S V): the covariance
    of the attention outputs, pooled over query heads (reading R2).
    q: [N, Hq, d], k, v: [N, Hkv, d].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, hq, d = q.shape
    g = hq // k.shape[1]
    acc = np.zeros((d, d))
    for h in range(hq):
        s = causal_attention_probs(q[:, h, :], k[:, h // g, :])
        o = s @ v[:, h // g, :]
        acc += o.T @ o
    return acc / (n * hq)


def eigenbasis(c: np.ndarray) -> np.ndarray:
    """Eigenvectors of a symmetric matrix as columns, descending eigenvalues,
    sign fixed per reading R3 ([gist] 2.2 A "Rotationsermittlung")."""
    w, u = np.linalg.eigh(np.asarray(c, dtype=np.float64))
    order = np.argsort(-w, kind="stable")
    u = u[:, order].copy()
    for col in range(u.shape[1]):
        i = int(np.argmax(np.abs(u[:, col])))       # first index on ties
        if u[i, col] < 0:
            u[:, col] = -u[:, col]
    return u


def sylvester_hadamard(n: int) -> np.ndarray:
    """Unnormalised Sylvester Hadamard matrix of order n (a power of two)."""
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard_block(d: int = HEAD_DIM, block: int = GROUP) -> np.ndarray:
    """Block-diagonal orthonormal Hadamard H_Had (reading R4; [gist] 2.2 A)."""
    hb = sylvester_hadamard(block) / math.sqrt(block)
    out = np.zeros((d, d))
    for b0 in range(0, d, block):
        out[b0:b0 + block, b0:b0 + block] = hb
    return out


def bit_reverse(j: int, bits: int) -> int:
    r = 0
    for _ in range(bits):
        r = (r << 1) | (j & 1)
        j >>= 1
    return r


def bitrev_permutation(d: int = HEAD_DIM) -> np.ndarray:
    """P_br as a matrix acting on row vectors: (x P)_j = x_{bitrev(j)}."""
    bits = d.bit_length() - 1
    p = np.zeros((d, d))
    for j in range(d):
        p[bit_reverse(j, bits), j] = 1.0
    return p


def composite_rotation(u: np.ndarray, block: int = GROUP) -> np.ndarray:
    """R = U . H_Had . P_br ([gist] 2.2 A "Aufbau der zusammengesetzten Rotation")."""
    d = u.shape[0]
    return u @ hadamard_block(d, block) @ bitrev_permutation(d)


def clip_thresholds(x: np.ndarray, r: np.ndarray, percentile: float = 99.0) -> np.ndarray:
    """Per rotated channel percentile of |x . R| (reading R5; [gist] 2.2 A
    "Clipping-Schwellenwerte"). x: [..., d] values; returns float32 [d]."""
    y = np.asarray(x, dtype=np.float64).reshape(-1, r.shape[0]) @ np.asarray(r, np.float64)
    return np.percentile(np.abs(y), percentile, axis=0, method="linear").astype(np.float32)


def key_attention_covariance(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Attention-weighted key covariance C_SK = (1/N) K^T S^T S K: the value
    target of [gist] 2.2 A with the keys in the place of the values (the
    alternative key target, reading R10)."""
    return score_covariance(q, k, k)


# rotations calibrate() can build (reading R10): the method and the baselines
ROTATIONS = ("spectral", "key_attn", "hadamard", "identity")


def calibrate_layers(qs, ks, vs, hadamard_block_size: int = GROUP, percentile: float = 99.0,
                     rotation: str = "spectral", per_kv_head: bool = False):
    """Offline calibration shared by L layers (reading R12): returns
    (R_K, R_V, tau_K, tau_V), R as float32 [d, d] (y = x . R), tau as
    float32 [d]; with per_kv_head, float32 [Hkv, d, d] and [Hkv, d].

    qs: [L, N, Hq, d], ks / vs: [L, N, Hkv, d] (L = 1 is one layer).
    rotation "spectral" is the method ([gist] 2.2 A: R_K = U_Q H P_br,
    R_V = U_S H P_br); "key_attn" takes the key eigenbasis from C_SK instead
    of C_Q; "hadamard" (R = H P_br, data-blind) and "identity" (R = I, plain
    INT2) are the baselines of [gist] 3 and 4."""
    qs, ks, vs = (np.asarray(x) for x in (qs, ks, vs))
    if per_kv_head:
        g = qs.shape[2] // ks.shape[2]
        parts = [calibrate_layers(qs[:, :, j * g:(j + 1) * g], ks[:, :, j:j + 1], vs[:, :, j:j + 1],
                                  hadamard_block_size, percentile, rotation)
                 for j in range(ks.shape[2])]
        return tuple(np.stack([p[i] for p in parts]) for i in range(4))
    d = HEAD_DIM
    n_layers = qs.shape[0]
    if rotation in ("spectral", "key_attn"):
        if rotation == "spectral":
            c_k = sum(query_covariance(qs[l]) for l in range(n_layers)) / n_layers
        else:
            c_k = sum(key_attention_covariance(qs[l], ks[l]) for l in range(n_layers)) / n_layers
        c_s = sum(score_covariance(qs[l], ks[l], vs[l]) for l in range(n_layers)) / n_layers
        r_k = composite_rotation(eigenbasis(c_k), hadamard_block_size)
        r_v = composite_rotation(eigenbasis(c_s), hadamard_block_size)
    elif rotation == "hadamard":
        r_k = r_v = composite_rotation(np.eye(d), hadamard_block_size)
    elif rotation == "identity":
        r_k = r_v = np.eye(d)
    else:
        raise ValueError(rotation)
    r_k = np.asarray(r_k, np.float32)
    r_v = np.asarray(r_v, np.float32)
    tau_k = clip_thresholds(ks, r_k, percentile)
    tau_v = clip_thresholds(vs, r_v, percentile)
    return r_k, r_v, tau_k, tau_v


def calibrate(q, k, v, hadamard_block_size: int = GROUP, percentile: float = 99.0, rotation: str = "spectral",
              per_kv_head: bool = False):
    """Offline calibration of one layer (q [N, Hq, d], k, v [N, Hkv, d]):
    calibrate_layers with L = 1."""
    return calibrate_layers(np.asarray(q)[None], np.asarray(k)[None], np.asarray(v)[None], hadamard_block_size,
                            percentile, rotation, per_kv_head)


# ---------------------------------------------------------------------------
# Demotion: rotate -> clip -> quantise -> pack  ([yunpan] 三.2; [gist] 2.2 B)
# ---------------------------------------------------------------------------

def rotate_fp32(x: np.ndarray, r: np.ndarray) -> np.ndarray:
    """y = fp32(x . R) with the product taken in fp64 (reading R1).

    r: [d, d], or [H, d, d] with one R per KV head (R12) for x [..., H, d]."""
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    if r.ndim == 2:
        return (x @ r).astype(np.float32)
    return np.matmul(x[..., None, :], r)[..., 0, :].astype(np.float32)


def heads_of(a, kv_heads, per_head_ndim: int):
    """The KV heads' own entries of a per-KV-head R or tau (R12); a layer's
    single R or tau (fewer dimensions) is returned as it is."""
    a = np.asarray(a)
    return a[list(kv_heads)] if a.ndim == per_head_ndim else a


def clip(y: np.ndarray, tau: np.ndarray) -> np.ndarray:
    """Symmetric per-channel clip to [-tau, tau] (IEEE minNum/maxNum)."""
    y = np.asarray(y, np.float32)
    t = np.asarray(tau, np.float32)
    return np.fmin(np.fmax(y, -t), t)


def group_params(yc: np.ndarray, bits: int = 2):
    """Per 32-channel group: (scale, zero) as float16, reading R6 (R13 for
    bits = 4: the span is divided by 15 instead of 3).

    yc: float32 [..., 128] -> scale, zero: float16 [..., 4].
    """
    g = np.asarray(yc, np.float32).reshape(yc.shape[:-1] + (N_GROUPS, GROUP))
    mn = g.min(axis=-1)
    mx = g.max(axis=-1)
    zero = f16_round_down(mn)
    span = (mx - zero.astype(np.float32)).astype(np.float32)
    scale = f16_round_up((span / np.float32(levels(bits))).astype(np.float32))
    return scale, zero


def quant_codes(yc: np.ndarray, scale: np.ndarray, zero: np.ndarray, bits: int = 2) -> np.ndarray:
    """INT2 codes (4 levels; [yunpan] 二) for clipped rotated values, R6; INT4
    codes (16 levels) for bits = 4, R13."""
    g = np.asarray(yc, np.float32).reshape(yc.shape[:-1] + (N_GROUPS, GROUP))
    s = scale.astype(np.float32)[..., None]
    z = zero.astype(np.float32)[..., None]
    diff = (g - z).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = np.where(s > 0, diff / np.where(s > 0, s, np.float32(1)), np.float32(0))
    c = np.clip(np.rint(quot.astype(np.float32)), 0, levels(bits)).astype(np.uint8)
    return c.reshape(yc.shape)


def dequantize(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray) -> np.ndarray:
    """c * s + z in fp64, per group. codes [..., 128], scale/zero [..., 4]."""
    c = np.asarray(codes, np.float64).reshape(codes.shape[:-1] + (N_GROUPS, GROUP))
    out = c * scale.astype(np.float64)[..., None] + zero.astype(np.float64)[..., None]
    return out.reshape(codes.shape)


def quantize_rotated(y: np.ndarray, tau: np.ndarray, bits: int = 2):
    """Clip + quantise already-rotated fp32 vectors: returns codes, scale, zero."""
    yc = clip(y, tau)
    scale, zero = group_params(yc, bits)
    return quant_codes(yc, scale, zero, bits), scale, zero


# ---------------------------------------------------------------------------
# Page block layout (reading R7).  "Four 2-bit values per byte" is the only
# thing the pages fix ([yunpan] 三.2); the rest is this format's own choice.
#
# Block of one (page, KV head), 1536 bytes:
#   [   0, 1024)  codes: 64 chunks of 16 bytes; chunk c = 16*a + b holds
#                 K codes in bytes 0..7 and V codes in bytes 8..15.
#   [1024, 1152)  K scales  fp16, index [token][group]
#   [1152, 1280)  K zeros   fp16, index [token][group]
#   [1280, 1408)  V scales  fp16, index [token // 4][group][token % 4]
#   [1408, 1536)  V zeros   fp16, same index
# Codes are 2-bit fields of little-endian 32-bit words; field f occupies
# bits 2f, 2f+1 of its word.
#
# INT4 block (reading R13), 2560 bytes:
#   [   0, 1024)  K codes: 64 chunks of 16 bytes; chunk 16*a + t holds token
#                 t's channels j with (j >> 3) & 3 == a, word j >> 5 (one
#                 group per word), nibble at bit 16*(j & 1) + 4*((j >> 1) & 3)
#   [1024, 2048)  V codes: chunk 16*a + b holds tokens 4a..4a+3, channels j
#                 with j & 15 == b; word 2*((j >> 4) >> 2) + ((t & 3) >> 1),
#                 nibble at bit 16*(t & 1) + 4*((j >> 4) & 3)
#   [2048, 2560)  scales and zeros, laid out as the INT2 block's [1024, 1536)
# ---------------------------------------------------------------------------

def meta_base(bits: int = 2) -> int:
    return {2: 1024, 4: 2048}[bits]


def k_code_bitpos(t: int, j: int, bits: int = 2) -> int:
    """Absolute bit index (byte*8 + bit) of K code (token t, channel j)."""
    if bits == 4:
        byte = 16 * (16 * ((j >> 3) & 3) + t) + 4 * (j >> 5)
        return byte * 8 + 16 * (j & 1) + 4 * ((j >> 1) & 3)
    a = (j >> 3) & 3                 # which quarter of the group
    word = j >> 6                    # groups {0,1} -> word 0, {2,3} -> word 1
    field = 4 * ((j >> 5) & 1) + ((j >> 1) & 3) + 8 * (j & 1)
    byte = 16 * (16 * a + t) + 4 * word
    return byte * 8 + 2 * field


def v_code_bitpos(t: int, j: int, bits: int = 2) -> int:
    """Absolute bit index of V code (token t, channel j)."""
    if bits == 4:
        m = j >> 4
        byte = 1024 + 16 * (16 * (t >> 2) + (j & 15)) + 4 * (2 * (m >> 2) + ((t & 3) >> 1))
        return byte * 8 + 16 * (t & 1) + 4 * (m & 3)
    x = j & 15
    blk = j >> 4
    tq, u = t >> 2, t & 3
    word = u >> 1
    field = blk + 8 * (u & 1)
    byte = 16 * (16 * tq + x) + 8 + 4 * word
    return byte * 8 + 2 * field


def k_scale_offset(t: int, g: int, bits: int = 2) -> int:
    return meta_base(bits) + 8 * t + 2 * g


def k_zero_offset(t: int, g: int, bits: int = 2) -> int:
    return meta_base(bits) + 128 + 8 * t + 2 * g


def v_scale_offset(t: int, g: int, bits: int = 2) -> int:
    return meta_base(bits) + 256 + 32 * (t >> 2) + 8 * g + 2 * (t & 3)


def v_zero_offset(t: int, g: int, bits: int = 2) -> int:
    return meta_base(bits) + 384 + 32 * (t >> 2) + 8 * g + 2 * (t & 3)


def _put_code(block: np.ndarray, bitpos: int, c: int, bits: int = 2) -> None:
    byte, bit = divmod(bitpos, 8)
    mask = levels(bits)
    block[byte] = (int(block[byte]) & ~(mask << bit) | ((int(c) & mask) << bit)) & 0xFF


def _get_code(block: np.ndarray, bitpos: int, bits: int = 2) -> int:
    byte, bit = divmod(bitpos, 8)
    return (int(block[byte]) >> bit) & levels(bits)


def _put_f16(block: np.ndarray, off: int, val) -> None:
    b = np.asarray(val, dtype=np.float16).reshape(1).view(np.uint8)
    block[off] = b[0]
    block[off + 1] = b[1]


def _get_f16(block: np.ndarray, off: int) -> np.float16:
    return block[off:off + 2].copy().view(np.float16)[0]


def write_token(block: np.ndarray, slot: int, kc, ks, kz, vc, vs, vz, bits: int = 2) -> None:
    """Store one token's K and V codes [128] and scale/zero [4] into a block."""
    for j in range(HEAD_DIM):
        _put_code(block, k_code_bitpos(slot, j, bits), kc[j], bits)
        _put_code(block, v_code_bitpos(slot, j, bits), vc[j], bits)
    for g in range(N_GROUPS):
        _put_f16(block, k_scale_offset(slot, g, bits), ks[g])
        _put_f16(block, k_zero_offset(slot, g, bits), kz[g])
        _put_f16(block, v_scale_offset(slot, g, bits), vs[g])
        _put_f16(block, v_zero_offset(slot, g, bits), vz[g])


def read_token(block: np.ndarray, slot: int, bits: int = 2):
    """Inverse of write_token: (kc, ks, kz, vc, vs, vz)."""
    kc = np.array([_get_code(block, k_code_bitpos(slot, j, bits), bits) for j in range(HEAD_DIM)], np.uint8)
    vc = np.array([_get_code(block, v_code_bitpos(slot, j, bits), bits) for j in range(HEAD_DIM)], np.uint8)
    ks = np.array([_get_f16(block, k_scale_offset(slot, g, bits)) for g in range(N_GROUPS)], np.float16)
    kz = np.array([_get_f16(block, k_zero_offset(slot, g, bits)) for g in range(N_GROUPS)], np.float16)
    vs = np.array([_get_f16(block, v_scale_offset(slot, g, bits)) for g in range(N_GROUPS)], np.float16)
    vz = np.array([_get_f16(block, v_zero_offset(slot, g, bits)) for g in range(N_GROUPS)], np.float16)
    return kc, ks, kz, vc, vs, vz


# ---------------------------------------------------------------------------
# Three-tier pool ([yunpan] 三.1, 三.2; [gist] 2.2 B "Mixed-Precision-Layout")
# ---------------------------------------------------------------------------

def tier_of(p: int, n: int) -> str:
    """Tier of position p in a sequence of n tokens (reading R8)."""
    if p < N_SINK:
        return "sink"
    if p >= max(N_SINK, n - N_RECENT):
        return "recent"
    return "history"


def ring_slot(p: int) -> int:
    return (p - N_SINK) % N_RECENT


class Pool:
    """Tiered KV pool state, byte-for-byte in the library's formats.

    sink_k/v, recent_k/v: uint16 bf16 bits [S, Hkv, 64|256, 128]
    hist: uint8 [num_pages, Hkv, 1536] (INT2; 2560 for INT4, bits = 4);
    page_table: int32 [S, max_pages]
    """

    def __init__(self, n_slots, n_kv_heads, num_pages, page_table, bits: int = 2):
        self.hkv = n_kv_heads
        self.bits = bits
        self.sink_k = np.zeros((n_slots, n_kv_heads, N_SINK, HEAD_DIM), np.uint16)
        self.sink_v = np.zeros_like(self.sink_k)
        self.recent_k = np.zeros((n_slots, n_kv_heads, N_RECENT, HEAD_DIM), np.uint16)
        self.recent_v = np.zeros_like(self.recent_k)
        self.hist = np.zeros((num_pages, n_kv_heads, block_bytes(bits)), np.uint8)
        self.page_table = np.asarray(page_table, np.int32)
        self.length = np.zeros(n_slots, np.int64)

    def demote_rotated(self, slot: int, h_index: int, yk, yv, tau_k, tau_v) -> None:
        """Quantise already-rotated fp32 K/V [Hkv, 128] into history index h."""
        page = int(self.page_table[slot, h_index // PAGE])
        ps = h_index % PAGE
        kc, ks, kz = quantize_rotated(yk, tau_k, self.bits)
        vc, vs, vz = quantize_rotated(yv, tau_v, self.bits)
        for hd in range(self.hkv):
            write_token(self.hist[page, hd], ps, kc[hd], ks[hd], kz[hd], vc[hd], vs[hd], vz[hd], self.bits)

    def demote(self, slot, h_index, k_bits, v_bits, r_k, r_v, tau_k, tau_v) -> None:
        """Rotate bf16 K/V [Hkv, 128] by R and demote them ([yunpan] 三.2)."""
        yk = rotate_fp32(bf16_to_f64(k_bits), r_k)
        yv = rotate_fp32(bf16_to_f64(v_bits), r_v)
        self.demote_rotated(slot, h_index, yk, yv, tau_k, tau_v)

    def append(self, slot, k_bits, v_bits, r_k, r_v, tau_k, tau_v) -> None:
        """Route one new token (k, v: bf16 bits [Hkv, 128]) into the tiers.

        When the recent ring is full, its oldest token (position p - 256)
        is demoted first, then the new token takes its ring slot.
        """
        p = int(self.length[slot])
        if p < N_SINK:
            self.sink_k[slot, :, p] = k_bits
            self.sink_v[slot, :, p] = v_bits
        else:
            r = ring_slot(p)
            if p >= N_SINK + N_RECENT:
                self.demote(slot, p - N_SINK - N_RECENT, self.recent_k[slot, :, r],
                            self.recent_v[slot, :, r], r_k, r_v, tau_k, tau_v)
            self.recent_k[slot, :, r] = k_bits
            self.recent_v[slot, :, r] = v_bits
        self.length[slot] = p + 1

    def demote_rotated_many(self, slot, h_indices, yk, yv, tau_k, tau_v, kv_heads=None):
        """Vectorised demote_rotated for many history indices of one slot.
        yk, yv: float32 [N, H, 128] for the KV heads in `kv_heads` (default all)."""
        heads = list(range(self.hkv)) if kv_heads is None else list(kv_heads)
        h = np.asarray(h_indices, np.int64)
        pages = self.page_table[slot, h // PAGE]
        kc, ks, kz = quantize_rotated(yk, heads_of(tau_k, heads, 2), self.bits)
        vc, vs, vz = quantize_rotated(yv, heads_of(tau_v, heads, 2), self.bits)
        for i, hd in enumerate(heads):
            write_tokens(self.hist, hd, pages, h % PAGE, kc[:, i], ks[:, i], kz[:, i], vc[:, i], vs[:, i], vz[:, i],
                         self.bits)

    def demote_many(self, slot, h_indices, k_bits, v_bits, r_k, r_v, tau_k, tau_v, kv_heads=None):
        """Rotate (fp64 product rounded to fp32) and demote many bf16 tokens [N, H, 128]."""
        heads = list(range(self.hkv)) if kv_heads is None else list(kv_heads)
        yk = rotate_fp32(bf16_to_f64(k_bits), heads_of(r_k, heads, 3))
        yv = rotate_fp32(bf16_to_f64(v_bits), heads_of(r_v, heads, 3))
        self.demote_rotated_many(slot, h_indices, yk, yv, tau_k, tau_v, kv_heads)

    @classmethod
    def from_state(cls, state, n_kv_heads):
        """Oracle pool holding given bytes (e.g. copied back from a device)."""
        bits = {BLOCK_BYTES: 2, BLOCK_BYTES_INT4: 4}[state["hist"].shape[-1]]
        pool = cls(state["sink_k"].shape[0], n_kv_heads, state["hist"].shape[0], state["page_table"], bits)
        for name in ("sink_k", "sink_v", "recent_k", "recent_v", "hist"):
            setattr(pool, name, np.array(state[name], copy=True))
        return pool

    def reconstruct(self, slot, n, r_k, r_v, kv_heads=None):
        """K~, V~ [H, n, 128] fp64 in the unrotated space (plain definition):
        BF16 values for sink/recent, dequant(c, s, z) . R^T for history.
        kv_heads selects the KV heads returned (default: all)."""
        heads = np.arange(self.hkv) if kv_heads is None else np.asarray(kv_heads)
        kt = np.zeros((len(heads), n, HEAD_DIM))
        vt = np.zeros((len(heads), n, HEAD_DIM))
        pos = np.arange(n)
        sink = pos < N_SINK
        recent = (pos >= max(N_SINK, n - N_RECENT))
        hist = ~sink & ~recent
        kt[:, sink] = bf16_to_f64(self.sink_k[slot][heads][:, pos[sink]])
        vt[:, sink] = bf16_to_f64(self.sink_v[slot][heads][:, pos[sink]])
        ring = (pos[recent] - N_SINK) % N_RECENT
        kt[:, recent] = bf16_to_f64(self.recent_k[slot][heads][:, ring])
        vt[:, recent] = bf16_to_f64(self.recent_v[slot][heads][:, ring])
        if hist.any():
            h = pos[hist] - N_SINK
            pages = self.page_table[slot, h // PAGE]
            blocks = self.hist[pages][:, heads]                        # [n_hist, H, 1536]
            kc, ks, kz, vc, vs, vz = unpack_tokens(blocks, h % PAGE, self.bits)   # [n_hist, Hkv, ...]
            kt[:, hist] = np.moveaxis(rotate_back(dequantize(kc, ks, kz), heads_of(r_k, heads, 3)), 1, 0)
            vt[:, hist] = np.moveaxis(rotate_back(dequantize(vc, vs, vz), heads_of(r_v, heads, 3)), 1, 0)
        return kt, vt


def rotate_back(y: np.ndarray, r: np.ndarray) -> np.ndarray:
    """y . R^T in fp64 (the inverse rotation, R1); r [d, d] or, per KV head,
    [H, d, d] for y [..., H, d] (R12)."""
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    if r.ndim == 2:
        return y @ r.T
    return np.matmul(y[..., None, :], np.swapaxes(r, -1, -2))[..., 0, :]


_BIT_TABLES = {}


def _bit_tables(bits: int = 2):
    """(byte, bit) of every K and V code of a block, from the *_bitpos definitions."""
    if bits not in _BIT_TABLES:
        kb = np.array([[k_code_bitpos(t, j, bits) for j in range(HEAD_DIM)] for t in range(PAGE)])
        vb = np.array([[v_code_bitpos(t, j, bits) for j in range(HEAD_DIM)] for t in range(PAGE)])
        ks = np.array([[k_scale_offset(t, g, bits) for g in range(N_GROUPS)] for t in range(PAGE)])
        kz = np.array([[k_zero_offset(t, g, bits) for g in range(N_GROUPS)] for t in range(PAGE)])
        vs = np.array([[v_scale_offset(t, g, bits) for g in range(N_GROUPS)] for t in range(PAGE)])
        vz = np.array([[v_zero_offset(t, g, bits) for g in range(N_GROUPS)] for t in range(PAGE)])
        _BIT_TABLES[bits] = (kb // 8, kb % 8, vb // 8, vb % 8, ks, kz, vs, vz)
    return _BIT_TABLES[bits]


def write_tokens(hist, head, pages, slots, kc, ks, kz, vc, vs, vz, bits: int = 2):
    """Vectorised write_token into a pool hist array uint8 [num_pages, Hkv, block]:
    token i goes to block (pages[i], head), slot slots[i]."""
    kby, kbi, vby, vbi, kso, kzo, vso, vzo = _bit_tables(bits)
    flat = hist.reshape(-1)
    assert np.shares_memory(flat, hist), "hist must be contiguous"
    assert hist.shape[-1] == block_bytes(bits)
    mask = np.uint8(levels(bits))
    base = ((np.asarray(pages, np.int64) * hist.shape[1] + head) * block_bytes(bits))[:, None]
    t = np.asarray(slots, np.int64)
    for byt, bit, codes in ((kby, kbi, kc), (vby, vbi, vc)):
        idx = (base + byt[t]).ravel()
        sh = bit[t].ravel().astype(np.uint8)
        np.bitwise_and.at(flat, idx, (~(mask << sh)).astype(np.uint8))
        np.bitwise_or.at(flat, idx, ((np.asarray(codes, np.uint8).ravel() & mask) << sh).astype(np.uint8))
    for off, vals in ((kso, ks), (kzo, kz), (vso, vs), (vzo, vz)):
        b = np.asarray(vals, np.float16).view(np.uint16)
        idx = base + off[t]
        flat[idx] = (b & 0xFF).astype(np.uint8)
        flat[idx + 1] = (b >> 8).astype(np.uint8)

def unpack_tokens(blocks: np.ndarray, slots: np.ndarray, bits: int = 2):
    """Codes and scale/zero of token slot slots[i] of blocks[i, ...] (vectorised
    read_token).  blocks: uint8 [N, ..., block bytes]; slots: [N]."""
    kby, kbi, vby, vbi, kso, kzo, vso, vzo = _bit_tables(bits)
    mask = levels(bits)
    b = np.asarray(blocks)
    idx = np.asarray(slots)
    extra = (1,) * (b.ndim - 2)

    def gather(off):                      # off: [16, m] byte offsets -> [N, ..., m] bytes
        o = off[idx].reshape((len(idx),) + extra + (off.shape[1],))
        return np.take_along_axis(b, np.broadcast_to(o, b.shape[:-1] + (off.shape[1],)), axis=-1)

    def f16(off):
        lo = gather(off).astype(np.uint16)
        hi = gather(off + 1).astype(np.uint16)
        return (lo | (hi << 8)).view(np.float16)

    sh_k = kbi[idx].reshape((len(idx),) + extra + (HEAD_DIM,))
    sh_v = vbi[idx].reshape((len(idx),) + extra + (HEAD_DIM,))
    kc = ((gather(kby) >> sh_k) & mask).astype(np.uint8)
    vc = ((gather(vby) >> sh_v) & mask).astype(np.uint8)
    return kc, f16(kso), f16(kzo), vc, f16(vso), f16(vzo)


# ---------------------------------------------------------------------------
# Attention (the plain definition; [gist] 2.2 B, [zingnex] 自定义INT2注意力内核)
# ---------------------------------------------------------------------------

def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """softmax(q K^T / sqrt(d)) V for one query vector or rows of queries (fp64)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    logits = q @ k.T / math.sqrt(q.shape[-1])
    logits -= logits.max(axis=-1, keepdims=True)
    w = np.exp(logits)
    w /= w.sum(axis=-1, keepdims=True)
    return w @ v


def decode_tiered(q_bits, pool: Pool, seq_slot, seq_len, r_k, r_v, heads=None) -> np.ndarray:
    """Single-token decode over the tiered pool: out [B, Hq, 128] fp64.

    q_bits: bf16 bits [B, Hq, 128]; seq_len[b] counts the tokens in the cache
    after this step's append, so the new token attends to itself (R8).
    heads: optional list of (b, h) to evaluate (others are left at zero).
    """
    q = bf16_to_f64(q_bits)
    b_n, hq, _ = q.shape
    g = hq // pool.hkv
    out = np.zeros((b_n, hq, HEAD_DIM))
    want = None if heads is None else set((int(b), int(h)) for b, h in heads)
    for b in range(b_n):
        hs = [h for h in range(hq) if want is None or (b, h) in want]
        if not hs:
            continue
        kvh = sorted(set(h // g for h in hs))
        kt, vt = pool.reconstruct(int(seq_slot[b]), int(seq_len[b]), r_k, r_v, kvh)
        for h in hs:
            i = kvh.index(h // g)
            out[b, h] = attention(q[b, h], kt[i], vt[i])
    return out


def attend_tail_tiered(q_bits, pool: Pool, seq_slot, seq_len, r_k, r_v, heads=None) -> np.ndarray:
    """Attention of the last T positions of each sequence over the tiered pool
    (several query tokens per step: speculative verification, chunked
    prefill), reading R11: out [B, T, Hq, 128] fp64.

    q_bits: bf16 bits [B, T, Hq, 128]; query t of sequence b sits at position
    p = n_b - T + t and attends causally to positions [0, p] of the cache
    (which already holds all n_b tokens).  heads: optional list of (b, h).
    """
    q = bf16_to_f64(q_bits)
    b_n, t_n, hq, _ = q.shape
    g = hq // pool.hkv
    out = np.zeros((b_n, t_n, hq, HEAD_DIM))
    want = None if heads is None else set((int(b), int(h)) for b, h in heads)
    for b in range(b_n):
        hs = [h for h in range(hq) if want is None or (b, h) in want]
        if not hs:
            continue
        n = int(seq_len[b])
        kvh = sorted(set(h // g for h in hs))
        kt, vt = pool.reconstruct(int(seq_slot[b]), n, r_k, r_v, kvh)
        for t in range(t_n):
            p = n - t_n + t
            for h in hs:
                i = kvh.index(h // g)
                out[b, t, h] = attention(q[b, t, h], kt[i, :p + 1], vt[i, :p + 1])
    return out


# BF16 baseline pool: [num_pages, Hkv, 2, 16, 128] bf16 (K page, then V page).

def bf16_pool_gather(pool_bits, page_table_row, n):
    """All n tokens of one sequence from a BF16 paged pool: K, V [Hkv, n, 128]."""
    hkv = pool_bits.shape[1]
    k = np.zeros((hkv, n, HEAD_DIM))
    v = np.zeros((hkv, n, HEAD_DIM))
    for p in range(n):
        page = int(page_table_row[p // PAGE])
        k[:, p] = bf16_to_f64(pool_bits[page, :, 0, p % PAGE])
        v[:, p] = bf16_to_f64(pool_bits[page, :, 1, p % PAGE])
    return k, v


def decode_bf16(q_bits, pool_bits, page_table, seq_slot, seq_len) -> np.ndarray:
    """Full-precision decode over a BF16 paged pool (the comparison baseline)."""
    q = bf16_to_f64(q_bits)
    b_n, hq, _ = q.shape
    g = hq // pool_bits.shape[1]
    out = np.zeros((b_n, hq, HEAD_DIM))
    for b in range(b_n):
        k, v = bf16_pool_gather(pool_bits, page_table[int(seq_slot[b])], int(seq_len[b]))
        for h in range(hq):
            out[b, h] = attention(q[b, h], k[h // g], v[h // g])
    return out


def attend_tail_bf16(q_bits, pool_bits, page_table, seq_slot, seq_len) -> np.ndarray:
    """The BF16 baseline for several query tokens (reading R11): query t of
    sequence b (position n_b - T + t) attends causally over the BF16 paged
    pool.  q_bits [B, T, Hq, 128]; out [B, T, Hq, 128] fp64."""
    q = bf16_to_f64(q_bits)
    b_n, t_n, hq, _ = q.shape
    g = hq // pool_bits.shape[1]
    out = np.zeros((b_n, t_n, hq, HEAD_DIM))
    for b in range(b_n):
        n = int(seq_len[b])
        k, v = bf16_pool_gather(pool_bits, page_table[int(seq_slot[b])], n)
        for t in range(t_n):
            p = n - t_n + t
            for h in range(hq):
                out[b, t, h] = attention(q[b, t, h], k[h // g][:p + 1], v[h // g][:p + 1])
    return out
