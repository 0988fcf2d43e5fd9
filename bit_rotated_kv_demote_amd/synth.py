"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module draws random numbers and casts them; it holds none of the
method's arithmetic (no rotation, clipping, quantisation or attention).
Both the CPU oracle's tests and the HIP path's tests take their inputs
from here, so the two sides see identical bytes.

Workload recipe (stand-in for the Qwen3-family layers the OSCAR pages
evaluate on -- "OSCAR: Offline Spectral Covariance-Aware Rotation for 2-bit
KV Cache Quantization" (gist.science), section 4 "Experimentelle
Ergebnisse" -- whose weights and datasets are not available):

* K and V are drawn from N(0, 1), four seeded "outlier" channels are scaled
  by 16, every token is scaled by one lognormal(0, 0.5) factor per tensor
  (shared across heads), then the values are rounded to bfloat16.
* q is drawn from N(0, 1) and rounded to bfloat16.
* A random rotation is the Q factor of the QR decomposition of a seeded
  Gaussian matrix, with column signs fixed so that diag(R) > 0.
* Every stream comes from ``numpy.random.default_rng(1000 + config_index)``
  spawned into named children, so each tensor has its own stream.
"""
from __future__ import annotations

import dataclasses
import numpy as np

HEAD_DIM = 128
PAGE = 16
N_SINK = 64
N_RECENT = 256

STREAM_NAMES = ("k", "v", "q", "rot", "outliers", "lognormal", "calib",
                "lengths", "perm", "steps")


def streams(config_index: int) -> dict[str, np.random.Generator]:
    """Named independent generators for one workload configuration."""
    ss = np.random.SeedSequence(1000 + int(config_index))
    kids = ss.spawn(len(STREAM_NAMES))
    return {name: np.random.default_rng(k) for name, k in zip(STREAM_NAMES, kids)}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def outlier_channels(rng: np.random.Generator, d: int = HEAD_DIM, n: int = 4) -> np.ndarray:
    return np.sort(rng.choice(d, size=n, replace=False))


def kv_tokens(rng: np.random.Generator, rng_lognormal: np.random.Generator,
              n_tokens: int, n_kv_heads: int, outliers: np.ndarray,
              d: int = HEAD_DIM) -> np.ndarray:
    """One K or V tensor [n_tokens, n_kv_heads, d] as bfloat16 bits."""
    x = rng.standard_normal((n_tokens, n_kv_heads, d), dtype=np.float32)
    x[:, :, outliers] *= np.float32(16.0)
    scale = rng_lognormal.lognormal(0.0, 0.5, size=(n_tokens, 1, 1)).astype(np.float32)
    return to_bf16_bits(x * scale)


def queries(rng: np.random.Generator, shape) -> np.ndarray:
    """q ~ N(0, 1) as bfloat16 bits."""
    return to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def random_rotation(rng: np.random.Generator, d: int = HEAD_DIM) -> np.ndarray:
    """Seeded Haar-like orthogonal matrix (float32)."""
    a = rng.standard_normal((d, d))
    qm, rm = np.linalg.qr(a)
    qm = qm * np.sign(np.diag(rm))[None, :]
    return qm.astype(np.float32)


def page_permutation(rng: np.random.Generator, num_pages: int) -> np.ndarray:
    return rng.permutation(num_pages).astype(np.int32)


def ragged_lengths(rng: np.random.Generator, batch: int, lo: int, hi: int) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=batch).astype(np.int64)


@dataclasses.dataclass(frozen=True)
class LayerShape:
    name: str
    num_q_heads: int
    num_kv_heads: int
    batch: int
    context: int          # tokens already in the cache before the first step
    steps: int            # decode steps (one appended token each)
    head_dim: int = HEAD_DIM


# The five workload shapes: a tiny parity case, Qwen3-4B / 8B / 32B-shaped
# attention layers, and a fixed-memory batch sweep at 16K context.
CONFIGS = {
    0: LayerShape("tiny-gqa2-1k", 2, 1, 1, 1024, 32),
    1: LayerShape("qwen3-4b-32k", 32, 8, 1, 32768, 1),
    2: LayerShape("qwen3-8b-128k", 32, 8, 1, 131072, 64),
    3: LayerShape("qwen3-fixedmem-16k", 32, 8, 1, 16384, 1),
    4: LayerShape("qwen3-32b-ragged", 64, 8, 16, 65536, 1),
}


def planted_layer(rng: np.random.Generator, n: int, hq: int, hkv: int, n_query_dirs: int = 16,
                  key_side_scale: float = 8.0, n_key_side_dirs: int = 8, per_head_bases: bool = False):
    """A layer with planted covariance structure, for comparing rotations.

    One seeded orthonormal basis B: queries have energy 1 in its first
    ``n_query_dirs`` directions and 0.05 elsewhere; keys have standard
    deviation ``key_side_scale`` in the next ``n_key_side_dirs`` directions
    (energy the queries never look at) and 1 elsewhere; values have standard
    deviation 3 in the first 8 directions of a second basis and 1 elsewhere.
    With ``per_head_bases`` every KV head has its own pair of bases (its
    query heads use its B).  Four seeded raw channels of K are scaled by 6
    and two of V by 4.  The structure is drawn first, then the n tokens:
    calibration and context tokens of one layer come from one call, split.
    Returns q as float32 [n, hq, 128] (bf16-representable) and K, V as bf16
    bits [n, hkv, 128].  Random draws and casts only.
    """
    d = HEAD_DIM
    b_qk = random_rotation(rng, d).astype(np.float64)
    b_v = random_rotation(rng, d).astype(np.float64)
    g = hq // hkv
    bq = [b_qk] * hkv
    bv = [b_v] * hkv
    if per_head_bases:
        bq = [random_rotation(rng, d).astype(np.float64) for _ in range(hkv)]
        bv = [random_rotation(rng, d).astype(np.float64) for _ in range(hkv)]
    sq = np.full(d, 0.05)
    sq[:n_query_dirs] = 1.0
    sk = np.ones(d)
    sk[n_query_dirs:n_query_dirs + n_key_side_dirs] = key_side_scale
    sv = np.ones(d)
    sv[:8] = 3.0
    zq = rng.standard_normal((n, hq, d)) * sq
    zk = rng.standard_normal((n, hkv, d)) * sk
    zv = rng.standard_normal((n, hkv, d)) * sv
    q = np.stack([zq[:, h] @ bq[h // g].T for h in range(hq)], axis=1)
    k = np.stack([zk[:, j] @ bq[j].T for j in range(hkv)], axis=1)
    v = np.stack([zv[:, j] @ bv[j].T for j in range(hkv)], axis=1)
    oc = np.sort(rng.choice(d, 4, replace=False))
    k[..., oc] *= 6.0
    v[..., oc[:2]] *= 4.0
    return (bf16_bits_to_f32(to_bf16_bits(q)), to_bf16_bits(k), to_bf16_bits(v))
