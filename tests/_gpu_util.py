"""Helpers for the GPU parity tests (not collected by pytest).

Inputs come from the shared seeded generator; expected values come from the
oracle only.  Where a device kernel needs pool bytes, they are the oracle's
bytes uploaded to the device (never the other way round).
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle as orc
from bit_rotated_kv_demote_amd import synth
from bit_rotated_kv_demote_amd.pool import TieredKV, bf16_tensor, bf16_bits

DEV = "cuda"


def i32(a):
    return torch.as_tensor(np.asarray(a, np.int32), device=DEV).contiguous()


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


class Layer:
    """Seeded synthetic layer: B sequences of up to max_len tokens (bf16 bits)."""

    def __init__(self, seed, batch, hq, hkv, max_len, n_q=1, tau_tokens=4096, shuffle=True, extra_pages=0,
                 per_kv_head=False, code_bits=2):
        self.code_bits = code_bits
        st = synth.streams(seed)
        self.batch, self.hq, self.hkv, self.max_len = batch, hq, hkv, max_len
        out = synth.outlier_channels(st["outliers"])
        self.k = synth.kv_tokens(st["k"], st["lognormal"], batch * max_len, hkv, out).reshape(batch, max_len, hkv, 128)
        self.v = synth.kv_tokens(st["v"], st["lognormal"], batch * max_len, hkv, out).reshape(batch, max_len, hkv, 128)
        self.q = synth.queries(st["q"], (n_q, batch, hq, 128))
        self.rot = synth.random_rotation(st["rot"])
        sample = self.k[0, :min(tau_tokens, max_len)]
        samp_v = self.v[0, :min(tau_tokens, max_len)]
        self.tau_k = orc.clip_thresholds(synth.bf16_bits_to_f32(sample), self.rot)
        self.tau_v = orc.clip_thresholds(synth.bf16_bits_to_f32(samp_v), self.rot)
        # the pool's rotations: the layer's one R for K and V, or (per_kv_head)
        # a distinct R_K and R_V per KV head with each head's own tau
        self.r_k = self.r_v = self.rot
        if per_kv_head:
            self.r_k = np.stack([synth.random_rotation(st["rot"]) for _ in range(hkv)])
            self.r_v = np.stack([synth.random_rotation(st["rot"]) for _ in range(hkv)])
            self.tau_k = np.stack([orc.clip_thresholds(synth.bf16_bits_to_f32(sample[:, j]), self.r_k[j])
                                   for j in range(hkv)])
            self.tau_v = np.stack([orc.clip_thresholds(synth.bf16_bits_to_f32(samp_v[:, j]), self.r_v[j])
                                   for j in range(hkv)])
        self.max_pages = max(1, math.ceil(max(0, max_len - 320) / 16) + extra_pages)
        self.num_pages = batch * self.max_pages
        perm = synth.page_permutation(st["perm"], self.num_pages) if shuffle else np.arange(self.num_pages)
        self.page_table = perm.reshape(batch, self.max_pages).astype(np.int32)

    def device_pool(self, n_slots=None):
        return TieredKV(self.hq, self.hkv, n_slots or self.batch, self.max_pages, self.num_pages, self.r_k, self.r_v,
                        self.tau_k, self.tau_v, page_table=self.page_table, code_bits=self.code_bits)

    def oracle_pool(self, lengths, kv_heads=None):
        """Oracle pool after each sequence b has taken lengths[b] tokens."""
        pool = orc.Pool(self.batch, self.hkv, self.num_pages, self.page_table, bits=self.code_bits)
        heads = list(range(self.hkv)) if kv_heads is None else list(kv_heads)
        for b, n in enumerate(lengths):
            ns = min(n, 64)
            pool.sink_k[b][:, :ns] = self.k[b, :ns].transpose(1, 0, 2)
            pool.sink_v[b][:, :ns] = self.v[b, :ns].transpose(1, 0, 2)
            first = max(64, n - 256)
            pos = np.arange(first, n)
            pool.recent_k[b][:, (pos - 64) % 256] = self.k[b, pos].transpose(1, 0, 2)
            pool.recent_v[b][:, (pos - 64) % 256] = self.v[b, pos].transpose(1, 0, 2)
            if n > 320:
                h = np.arange(n - 320)
                pool.demote_many(b, h, self.k[b, 64 + h][:, heads], self.v[b, 64 + h][:, heads], self.r_k, self.r_v,
                                 self.tau_k, self.tau_v, kv_heads=heads)
            pool.length[b] = n
        return pool


def upload(dev: TieredKV, opool: orc.Pool, kv_heads=None):
    """Copy the oracle's pool bytes into the device pool (all or some KV heads)."""
    heads = list(range(opool.hkv)) if kv_heads is None else list(kv_heads)
    for hd in heads:
        dev.sink_k[:, hd] = bf16_tensor(opool.sink_k[:, hd])
        dev.sink_v[:, hd] = bf16_tensor(opool.sink_v[:, hd])
        dev.recent_k[:, hd] = bf16_tensor(opool.recent_k[:, hd])
        dev.recent_v[:, hd] = bf16_tensor(opool.recent_v[:, hd])
        dev.hist[:, hd] = torch.from_numpy(np.ascontiguousarray(opool.hist[:, hd])).to(DEV)
    torch.cuda.synchronize()


def code_diff_stats(hist_a, hist_b, pages, slots):
    """Compare codes of given (page, slot) tokens of two hist arrays [P, Hkv, block]
    (INT2 or INT4 blocks, told apart by their size)."""
    bits = 4 if hist_a.shape[-1] == orc.BLOCK_BYTES_INT4 else 2
    ua = orc.unpack_tokens(hist_a[pages], slots, bits)
    ub = orc.unpack_tokens(hist_b[pages], slots, bits)
    kd = ua[0].astype(int) - ub[0].astype(int)
    vd = ua[3].astype(int) - ub[3].astype(int)
    diffs = np.concatenate([kd.ravel(), vd.ravel()])
    meta = []
    for i in (1, 2, 4, 5):
        a = ua[i].astype(np.float16).view(np.int16).astype(int)
        b = ub[i].astype(np.float16).view(np.int16).astype(int)
        same_sign = np.sign(ua[i].astype(np.float32)) == np.sign(ub[i].astype(np.float32))
        ulp = np.where(same_sign, np.abs(a - b), np.abs(a) + np.abs(b))
        meta.append(ulp.max() if ulp.size else 0)
    return float(np.mean(diffs != 0)), int(np.abs(diffs).max()) if diffs.size else 0, max(meta)


# Bounds of the fused path (the accuracy contract): at most 0.1 % of the
# codes of demoted tokens differ from the oracle's, each by at most one level,
# and scale / zero lie within 2 fp16 ulp; decode outputs over identical pool
# bytes match within 2e-3 relative L2.
FLIP_RATE, FLIP_MAX, META_ULP = 1e-3, 1, 2
DECODE_TOL = 2e-3


def check_state_vs_oracle(state, opool: orc.Pool, demoted):
    """Device pool bytes after device appends / demotions against the oracle's
    pool after the same appends: the BF16 tiers byte for byte, the history
    codes of the demoted tokens within the flip budget.

    demoted: list of (slot, history indices) the compared path demoted."""
    for name in ("sink_k", "sink_v", "recent_k", "recent_v"):
        assert np.array_equal(state[name], getattr(opool, name)), name
    pages, slots = [], []
    for slot, h in demoted:
        h = np.asarray(h, np.int64)
        if h.size:
            pages.append(opool.page_table[slot, h // 16])
            slots.append(h % 16)
    if not pages:
        return 0.0
    pages, slots = np.concatenate(pages), np.concatenate(slots)
    # in chunks of tokens (a 128K history is 1.6 GB of gathered blocks at once)
    n_diff = n_codes = maxd = meta_ulp = 0
    for i in range(0, len(pages), 8192):
        rate, md, mu = code_diff_stats(state["hist"], opool.hist, pages[i:i + 8192], slots[i:i + 8192])
        n = len(pages[i:i + 8192]) * opool.hkv * 256
        n_diff += rate * n
        n_codes += n
        maxd, meta_ulp = max(maxd, md), max(meta_ulp, mu)
    rate = n_diff / n_codes
    assert rate <= FLIP_RATE and maxd <= FLIP_MAX and meta_ulp <= META_ULP, (rate, maxd, meta_ulp)
    return rate


def decode_over_device_bytes(state, hkv, q_bits, slots, lengths, r_k, r_v, heads=None):
    """The oracle's decode over the device's own pool bytes (copied back)."""
    return orc.decode_tiered(q_bits, orc.Pool.from_state(state, hkv), slots, lengths, r_k, r_v, heads=heads)
