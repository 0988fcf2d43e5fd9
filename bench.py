"""Benchmark of the OSCAR-style INT2 tiered decode step on one MI355X.

A step is one pass of the whole hot path over one batch: the append of the
new token (route it; demote the ring slot it reuses: rotate, clip, quantise,
pack) followed by tiered decode attention, as one oscar_step call: two
launches, the split kernel (which also writes the new token, demotes the
leaving one and computes q . R_K) and the merge.  The same steps as
separate oscar_append + oscar_decode calls are timed beside it.  The default workload is
the Qwen3-4B-shaped layer: 32 q / 8 KV heads, head_dim 128, batch 1, 32768
cached tokens (64 BF16 sink + INT2 history + 256 BF16 recent, 16-token pages),
seeded synthetic K/V/q, R and clip thresholds from oscar_calibrate on 4096
seeded calibration tokens.  Steps cycle through distinct per-layer pools
totalling more than 512 MB so that repeated steps are served from HBM, not
from the 256 MB last-level cache.

Prints one JSON line.  Also reported: the 128K-context decode (Qwen3-8B
shape), the BF16 paged baseline at both contexts, bulk demotion tok/s
(16 sequences x 4096-token chunks, 8 KV heads) and the CPU oracle timed on
a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "INT2 decode-attn µs/step + HBM GB/s (% roofline) at 32K–128K ctx; demote tok/s"


def hist_token_bytes(code_bits=2):
    """History bytes per token per KV head, K + V codes and metadata: INT2 96, INT4 160."""
    return 2 * (128 * code_bits // 8) + 2 * 16


def decode_bytes(lengths, hq, hkv, code_bits=2):
    """Algorithmic HBM bytes of one oscar_decode call (see the design notes)."""
    total = 0
    for n in lengths:
        hist = max(0, n - 320)
        total += hist * hkv * hist_token_bytes(code_bits) + min(n, 320) * hkv * 512 + 4 * math.ceil(hist / 16)
    total += len(lengths) * hq * 128 * (2 + 4) + 2 * 128 * 128 * 4
    return total


def split_kernel_bytes(lengths, hq, hkv, code_bits=2):
    """Algorithmic HBM bytes of the decode's split kernel alone (oscar_decode_partials):
    history, sink/recent tiles, page ids, q and R_K; not the merge's R_V and output."""
    total = 0
    for n in lengths:
        hist = max(0, n - 320)
        total += hist * hkv * hist_token_bytes(code_bits) + min(n, 320) * hkv * 512 + 4 * math.ceil(hist / 16)
    return total + len(lengths) * hq * 128 * 2 + 128 * 128 * 4


def bf16_decode_bytes(lengths, hq, hkv):
    total = 0
    for n in lengths:
        total += n * hkv * 512 + 4 * math.ceil(n / 16)
    return total + len(lengths) * hq * 128 * (2 + 4)


_HOLD_CYCLES_PER_MS = None


def gpu_hold(torch, ms):
    """Enqueue a bounded spin kernel of about `ms` milliseconds on the current
    stream, so that the host can queue the timed launches ahead of the GPU
    (the timed region then measures back-to-back GPU execution, not the
    Python launch loop)."""
    global _HOLD_CYCLES_PER_MS
    if _HOLD_CYCLES_PER_MS is None:
        n = 1_000_000
        torch.cuda._sleep(n)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(n)
        b.record()
        torch.cuda.synchronize()
        _HOLD_CYCLES_PER_MS = n / max(a.elapsed_time(b), 1e-3)
    torch.cuda._sleep(int(_HOLD_CYCLES_PER_MS * ms))


class Timer:
    """HIP events on the current stream around each launch of one kernel."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, s):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.append((s, e))

    def mean_us(self):
        return 1000.0 * sum(s.elapsed_time(e) for s, e in self.pairs) / max(1, len(self.pairs))


def build_layers(torch, hq, hkv, n0, n_layers, steps_per_layer, seed, calib_tokens=4096, calib=None, code_bits=2):
    """n_layers distinct pools holding the same seeded context of n0 tokens.
    calib: (rot_k, rot_v, tau_k, tau_v) to reuse; default: oscar_calibrate."""
    from bit_rotated_kv_demote_amd import binding, synth
    from bit_rotated_kv_demote_amd.pool import TieredKV, bf16_tensor

    st = synth.streams(seed)
    out = synth.outlier_channels(st["outliers"])
    n_tot = n0 + steps_per_layer
    k = synth.kv_tokens(st["k"], st["lognormal"], n_tot, hkv, out)
    v = synth.kv_tokens(st["v"], st["lognormal"], n_tot, hkv, out)
    calib_s = 0.0
    if calib is None:
        # offline calibration on seeded calibration tokens (host C++ in the library)
        cq = synth.bf16_bits_to_f32(synth.queries(st["calib"], (calib_tokens, hq, 128)))
        ck = synth.bf16_bits_to_f32(synth.kv_tokens(st["calib"], st["lognormal"], calib_tokens, hkv, out))
        cv = synth.bf16_bits_to_f32(synth.kv_tokens(st["calib"], st["lognormal"], calib_tokens, hkv, out))
        rot_k = torch.zeros((128, 128), dtype=torch.float32)
        rot_v = torch.zeros((128, 128), dtype=torch.float32)
        tau_k = torch.zeros(128, dtype=torch.float32)
        tau_v = torch.zeros(128, dtype=torch.float32)
        t0 = time.time()
        binding.oscar_calibrate(binding.layer_desc(hq, hkv), torch.from_numpy(cq), torch.from_numpy(ck),
                                torch.from_numpy(cv), rot_k, rot_v, tau_k, tau_v)
        calib_s = time.time() - t0
        calib = (rot_k.numpy(), rot_v.numpy(), tau_k.numpy(), tau_v.numpy())
    max_pages = math.ceil((n_tot - 320) / 16)
    layers = []
    kd = bf16_tensor(k[None, :n0])
    vd = bf16_tensor(v[None, :n0])
    for li in range(n_layers):
        pt = synth.page_permutation(np.random.default_rng(seed * 100 + li), max_pages)[None, :]
        pool = TieredKV(hq, hkv, 1, max_pages, max_pages, *calib, page_table=pt, code_bits=code_bits)
        pool.prefill(torch.tensor([n0], dtype=torch.int32, device="cuda"), kd, vd)
        layers.append(pool)
    new_k = bf16_tensor(np.ascontiguousarray(k[n0:]))    # [steps, Hkv, 128]
    new_v = bf16_tensor(np.ascontiguousarray(v[n0:]))
    q = bf16_tensor(synth.queries(st["q"], (steps_per_layer, 1, hq, 128)))
    torch.cuda.synchronize()
    del kd, vd
    return layers, new_k, new_v, q, calib_s, (k, v) + tuple(calib)


def run_tiered(torch, hq, hkv, n0, n_layers, steps, warmup, seed, calib=None, code_bits=2, fused=True):
    """Time exactly `steps` decode steps cycling through n_layers pools (fused:
    oscar_step, append and decode in one call; else oscar_append then
    oscar_decode), then as many again as separate calls with HIP events around
    every call (append and decode-call durations), then as many fused steps
    with events around every call."""
    rounds = math.ceil((warmup + 4 * steps) / n_layers)
    layers, new_k, new_v, q, calib_s, host = build_layers(torch, hq, hkv, n0, n_layers, rounds, seed, calib=calib,
                                                          code_bits=code_bits)
    positions = torch.arange(n0, n0 + rounds, dtype=torch.int32, device="cuda")
    lens = positions + 1
    max_len = n0 + rounds
    outs = [torch.empty((1, hq, 128), dtype=torch.float32, device="cuda") for _ in range(2)]
    for pool in layers:
        pool.workspace(1, max_len)

    def fused_step(i, t_step=None):
        li, r = i % n_layers, i // n_layers
        s = t_step.start() if t_step else None
        layers[li].step(positions[r:r + 1], new_k[r:r + 1], new_v[r:r + 1], q[r], max_len, out=outs[i & 1])
        if t_step:
            t_step.stop(s)

    def step(i, t_dec=None, t_app=None):
        li, r = i % n_layers, i // n_layers
        pool = layers[li]
        s = t_app.start() if t_app else None
        pool.append(positions[r:r + 1], new_k[r:r + 1], new_v[r:r + 1])
        if t_app:
            t_app.stop(s)
        s = t_dec.start() if t_dec else None
        pool.decode(q[r], lens[r:r + 1], max_len, out=outs[i & 1])
        if t_dec:
            t_dec.stop(s)

    run = fused_step if fused else step
    for i in range(warmup):
        run(i)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    gpu_hold(torch, 20 + 0.1 * steps)
    e0.record()
    for i in range(warmup, warmup + steps):
        run(i)
    e1.record()
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    # the same number of steps as separate oscar_append + oscar_decode calls
    torch.cuda.synchronize()
    gpu_hold(torch, 20 + 0.1 * steps)
    e0.record()
    for i in range(warmup + steps, warmup + 2 * steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    separate_ms = e0.elapsed_time(e1)
    t_dec, t_app, t_step = Timer(torch), Timer(torch), Timer(torch)
    gpu_hold(torch, 20 + 0.2 * steps)
    for i in range(warmup + 2 * steps, warmup + 3 * steps):
        step(i, t_dec, t_app)
    torch.cuda.synchronize()
    gpu_hold(torch, 20 + 0.2 * steps)
    for i in range(warmup + 3 * steps, warmup + 4 * steps):
        fused_step(i, t_step)
    torch.cuda.synchronize()
    # the decode's two kernels apart: `steps` back-to-back oscar_decode_partials
    # launches (the split kernel) between two events, then as many
    # oscar_decode_merge launches; each layer decodes at the length it has reached
    n_done = warmup + 4 * steps
    last_len = [n0 + (n_done - 1 - li) // n_layers + 1 for li in range(n_layers)]
    last_lens = torch.tensor(last_len, dtype=torch.int32, device="cuda")
    q_last = q[(n_done - 1) // n_layers]
    phase_ms = []
    for phase in ("partials", "merge"):
        torch.cuda.synchronize()
        gpu_hold(torch, 20 + 0.1 * steps)
        e0.record()
        for i in range(steps):
            li = i % n_layers
            if phase == "partials":
                layers[li].decode_partials(q_last, last_lens[li:li + 1], max_len)
            else:
                layers[li].decode_merge(last_lens[li:li + 1], 1, max_len, out=outs[i & 1])
        e1.record()
        torch.cuda.synchronize()
        phase_ms.append(e0.elapsed_time(e1))
    pool_bytes = sum(p.hist.numel() + 4 * p.sink_k.numel() + 4 * p.recent_k.numel() for p in layers)
    mid_len = n0 + (warmup + steps) // n_layers + 1
    return dict(total_ms=total_ms, us_per_step=1000.0 * total_ms / steps, decode_us=t_dec.mean_us(),
                us_per_step_separate=1000.0 * separate_ms / steps, step_call_us=t_step.mean_us(),
                append_us=t_app.mean_us(), decode_bytes=decode_bytes([mid_len], hq, hkv, code_bits), layers=n_layers,
                split_us=1000.0 * phase_ms[0] / steps, merge_us=1000.0 * phase_ms[1] / steps,
                split_bytes=sum(split_kernel_bytes([n], hq, hkv, code_bits) for n in last_len) / n_layers,
                pool_mb=pool_bytes / 1e6, calib_s=calib_s, host=host, n_mid=mid_len, max_len=max_len)


def run_bf16(torch, hq, hkv, n, n_layers, steps, seed, k_bits, v_bits):
    from bit_rotated_kv_demote_amd import synth
    from bit_rotated_kv_demote_amd.pool import PagedBF16, bf16_tensor

    pages = math.ceil(n / 16)
    kv = np.zeros((pages, hkv, 2, 16, 128), np.uint16)
    kp = np.zeros((pages * 16, hkv, 128), np.uint16)
    vp = np.zeros((pages * 16, hkv, 128), np.uint16)
    kp[:n] = k_bits[:n]
    vp[:n] = v_bits[:n]
    kv[:, :, 0] = kp.reshape(pages, 16, hkv, 128).transpose(0, 2, 1, 3)
    kv[:, :, 1] = vp.reshape(pages, 16, hkv, 128).transpose(0, 2, 1, 3)
    q = bf16_tensor(synth.queries(synth.streams(seed)["q"], (1, hq, 128)))
    pools = []
    for li in range(n_layers):
        perm = synth.page_permutation(np.random.default_rng(7000 + li), pages)
        phys = np.empty_like(kv)
        phys[perm] = kv
        pools.append(PagedBF16(hq, hkv, phys, perm[None, :]))
    lens = torch.tensor([n], dtype=torch.int32, device="cuda")
    out = torch.empty((1, hq, 128), dtype=torch.float32, device="cuda")
    for p in pools:
        p.decode(q, lens, n, out=out)
    torch.cuda.synchronize()
    t = Timer(torch)
    gpu_hold(torch, 20 + 0.2 * steps)
    for i in range(steps):
        s = t.start()
        pools[i % n_layers].decode(q, lens, n, out=out)
        t.stop(s)
    torch.cuda.synchronize()
    return dict(decode_us=t.mean_us(), decode_bytes=bf16_decode_bytes([n], hq, hkv), layers=n_layers,
                pool_mb=n_layers * kv.nbytes / 1e6)


def _seq_kv(hkv, n, seed):
    """One seeded sequence of n tokens (bf16 bits [n, Hkv, 128]) for K and V."""
    from bit_rotated_kv_demote_amd import synth
    st = synth.streams(seed)
    out = synth.outlier_channels(st["outliers"])
    return (synth.kv_tokens(st["k"], st["lognormal"], n, hkv, out),
            synth.kv_tokens(st["v"], st["lognormal"], n, hkv, out))


def _int2_pool(torch, hq, hkv, lengths, k1, v1, calib, seed, chunk=4, code_bits=2):
    """INT2 (or INT4) tiered pool holding len(lengths) sequences; sequence b holds
    the first lengths[b] tokens of the seeded sequence (k1, v1); shuffled page table."""
    from bit_rotated_kv_demote_amd import synth
    from bit_rotated_kv_demote_amd.pool import TieredKV, bf16_tensor
    B = len(lengths)
    max_pages = max(1, math.ceil((max(lengths) + 1 - 320) / 16))
    perm = synth.page_permutation(np.random.default_rng(seed), B * max_pages).reshape(B, max_pages)
    pool = TieredKV(hq, hkv, B, max_pages, B * max_pages, *calib, page_table=perm, code_bits=code_bits)
    kd, vd = bf16_tensor(k1), bf16_tensor(v1)
    for b0 in range(0, B, chunk):
        bs = list(range(b0, min(B, b0 + chunk)))
        n = max(lengths[b] for b in bs)
        kk = kd[None, :n].expand(len(bs), -1, -1, -1).contiguous()
        vv = vd[None, :n].expand(len(bs), -1, -1, -1).contiguous()
        pool.prefill(torch.tensor([lengths[b] for b in bs], dtype=torch.int32, device="cuda"), kk, vv,
                     seq_slot=torch.tensor(bs, dtype=torch.int32, device="cuda"))
        del kk, vv
    torch.cuda.synchronize()
    return pool


def _bf16_pool(torch, hq, hkv, B, n, k1, v1, seed):
    """BF16 paged pool of B copies of the first n tokens of (k1, v1), built on the device."""
    from bit_rotated_kv_demote_amd import synth
    from bit_rotated_kv_demote_amd.pool import PagedBF16, bf16_tensor
    P = math.ceil(n / 16)
    base = torch.zeros((P, hkv, 2, 16, 128), dtype=torch.bfloat16, device="cuda")
    for c, src in ((0, k1), (1, v1)):
        t = torch.zeros((P * 16, hkv, 128), dtype=torch.bfloat16, device="cuda")
        t[:n] = bf16_tensor(src[:n])
        base[:, :, c] = t.view(P, 16, hkv, 128).permute(0, 2, 1, 3)
    perm = synth.page_permutation(np.random.default_rng(seed), B * P)
    phys = torch.empty((B * P, hkv, 2, 16, 128), dtype=torch.bfloat16, device="cuda")
    phys[torch.as_tensor(perm, device="cuda").long()] = base.repeat(B, 1, 1, 1, 1)
    del base
    return PagedBF16(hq, hkv, phys, perm.reshape(B, P))


def _time_decode(torch, pool, q, lens, max_len, steps, seq_slot=None):
    out = torch.empty((q.shape[0], q.shape[1], 128), dtype=torch.float32, device="cuda")
    pool.decode(q, lens, max_len, out=out, seq_slot=seq_slot)
    torch.cuda.synchronize()
    t = Timer(torch)
    gpu_hold(torch, 5 + 0.5 * steps)
    for _ in range(steps):
        s0 = t.start()
        pool.decode(q, lens, max_len, out=out, seq_slot=seq_slot)
        t.stop(s0)
    torch.cuda.synchronize()
    return t.mean_us()


def run_ragged_gqa8(torch, steps, calib, seed=1005):
    """Qwen3-32B-shaped ragged batch: 64 q / 8 KV heads (G = 8), batch 16,
    contexts uniform in [8192, 65536], shuffled page tables; INT2 decode and the
    BF16 baseline on the same batch."""
    from bit_rotated_kv_demote_amd import synth
    from bit_rotated_kv_demote_amd.pool import bf16_tensor
    hq, hkv, B = 64, 8, 16
    st = synth.streams(seed)
    lengths = [int(x) for x in synth.ragged_lengths(st["lengths"], B, 8192, 65536)]
    n_max = max(lengths)
    k1, v1 = _seq_kv(hkv, n_max, seed)
    pool = _int2_pool(torch, hq, hkv, lengths, k1, v1, calib, seed)
    q = bf16_tensor(synth.queries(st["q"], (B, hq, 128)))
    lens = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    us = _time_decode(torch, pool, q, lens, n_max, steps)
    nbytes = decode_bytes(lengths, hq, hkv)
    del pool
    torch.cuda.empty_cache()
    # BF16 baseline: one shared page layout with the longest context, per-sequence lengths
    bpool = _bf16_pool(torch, hq, hkv, B, n_max, k1, v1, seed + 1)
    bus = _time_decode(torch, bpool, q, lens, n_max, steps)
    bbytes = bf16_decode_bytes(lengths, hq, hkv)
    del bpool
    torch.cuda.empty_cache()
    return {"workload": "64 q / 8 KV heads, batch 16, contexts U[8192, 65536] (seeded), shuffled pages",
            "total_tokens": int(sum(lengths)), "decode_us": round(us, 3), "decode_GBps": round(nbytes / (us * 1e3), 1),
            "decode_algorithmic_bytes": nbytes, "bf16_decode_us": round(bus, 3),
            "bf16_decode_GBps": round(bbytes / (bus * 1e3), 1), "int2_vs_bf16_decode_speedup": round(bus / us, 3)}


def run_fixed_memory(torch, steps, calib, seed=1004, layers=36, budget_gb=64.0, n=16384):
    """Fixed-memory batch sweep: 32 q / 8 KV heads at n tokens per sequence;
    the INT2 pool and the BF16 cache each get the same per-layer share of a
    64 GB budget (over an assumed 36 layers); decode tokens/s (batch / step
    time) per batch, and the largest batch each format fits."""
    from bit_rotated_kv_demote_amd import synth
    from bit_rotated_kv_demote_amd.pool import bf16_tensor
    hq, hkv = 32, 8
    per_layer = budget_gb * 1e9 / layers
    int2_seq = (n - 320) * hkv * hist_token_bytes(2) + 320 * hkv * 512
    int4_seq = (n - 320) * hkv * hist_token_bytes(4) + 320 * hkv * 512
    bf16_seq = n * hkv * 512
    max_int2, max_bf16 = int(per_layer // int2_seq), int(per_layer // bf16_seq)
    max_int4 = int(per_layer // int4_seq)
    st = synth.streams(seed)
    k1, v1 = _seq_kv(hkv, n, seed)
    q_all = bf16_tensor(synth.queries(st["q"], (max_int2, hq, 128)))
    batches = sorted({b for b in (1, 2, 4, 8, 16, 32, 64, 128) if b <= max_int2} | {max_int2, max_int4, max_bf16})
    res = {"workload": f"32 q / 8 KV heads, {n} tokens per sequence, {budget_gb:g} GB over {layers} layers "
                       f"= {per_layer / 1e9:.3f} GB per layer",
           "max_batch_int2": max_int2, "max_batch_int4": max_int4, "max_batch_bf16": max_bf16,
           "int2_tok_per_s": {}, "int4_tok_per_s": {}, "bf16_tok_per_s": {}}
    pool = _int2_pool(torch, hq, hkv, [n] * max_int2, k1, v1, calib, seed)
    for b in batches:
        lens = torch.full((b,), n, dtype=torch.int32, device="cuda")
        us = _time_decode(torch, pool, q_all[:b], lens, n, steps)
        res["int2_tok_per_s"][str(b)] = round(b / (us * 1e-6), 1)
    del pool
    torch.cuda.empty_cache()
    pool = _int2_pool(torch, hq, hkv, [n] * max_int4, k1, v1, calib, seed, code_bits=4)
    for b in batches:
        if b > max_int4:
            continue
        lens = torch.full((b,), n, dtype=torch.int32, device="cuda")
        us = _time_decode(torch, pool, q_all[:b], lens, n, steps)
        res["int4_tok_per_s"][str(b)] = round(b / (us * 1e-6), 1)
    del pool
    torch.cuda.empty_cache()
    bpool = _bf16_pool(torch, hq, hkv, max_bf16, n, k1, v1, seed + 1)
    for b in batches:
        if b > max_bf16:
            continue
        lens = torch.full((b,), n, dtype=torch.int32, device="cuda")
        us = _time_decode(torch, bpool, q_all[:b], lens, n, steps)
        res["bf16_tok_per_s"][str(b)] = round(b / (us * 1e-6), 1)
    del bpool
    torch.cuda.empty_cache()
    res["throughput_ratio_at_max_batch"] = round(res["int2_tok_per_s"][str(max_int2)] /
                                                 res["bf16_tok_per_s"][str(max_bf16)], 3)
    res["int2_vs_int4_at_max_batch"] = round(res["int2_tok_per_s"][str(max_int2)] /
                                             res["int4_tok_per_s"][str(max_int4)], 3)
    return res


def run_multi_query(torch, steps, calib, seed=1007, hq=32, hkv=8, n=32768, n_pools=12,
                    counts=(1, 2, 4, 8, 16, 64)):
    """Several query tokens per sequence (oscar_decode_multi) on the
    Qwen3-4B-shaped layer at a 32K context: the last T positions attend
    causally (speculative verification, chunked prefill).  Pools are cycled
    so the history comes from HBM; HIP events around every call."""
    from bit_rotated_kv_demote_amd import synth
    from bit_rotated_kv_demote_amd.pool import bf16_tensor
    k1, v1 = _seq_kv(hkv, n, seed)
    pools = [_int2_pool(torch, hq, hkv, [n], k1, v1, calib, seed + 10 + i) for i in range(n_pools)]
    lens = torch.tensor([n], dtype=torch.int32, device="cuda")
    res = {}
    t_one = None
    for t_n in counts:
        q = bf16_tensor(synth.queries(np.random.default_rng(seed + t_n), (1, t_n, hq, 128)))
        out = torch.empty((1, t_n, hq, 128), dtype=torch.float32, device="cuda")
        for i in range(n_pools):
            pools[i].decode_multi(q, lens, n, out=out)
        torch.cuda.synchronize()
        tm = Timer(torch)
        gpu_hold(torch, 5 + 0.5 * steps)
        for i in range(steps):
            s0 = tm.start()
            pools[i % n_pools].decode_multi(q, lens, n, out=out)
            tm.stop(s0)
        torch.cuda.synchronize()
        us = tm.mean_us()
        nbytes = decode_bytes([n], hq, hkv) + (t_n - 1) * hq * 128 * (2 + 4)
        t_one = us if t_n == 1 else t_one
        res[str(t_n)] = {"us_per_call": round(us, 3), "us_per_query_token": round(us / t_n, 3),
                         "GBps": round(nbytes / (us * 1e3), 1),
                         "speedup_vs_single_token_calls": round(t_n * t_one / us, 2)}
    del pools
    torch.cuda.empty_cache()
    # the BF16 baseline on the same tokens (4 cycled copies, 537 MB)
    bpools = [_bf16_pool(torch, hq, hkv, 1, n, k1, v1, seed + 30 + i) for i in range(4)]
    for t_n in counts:
        q = bf16_tensor(synth.queries(np.random.default_rng(seed + t_n), (1, t_n, hq, 128)))
        out = torch.empty((1, t_n, hq, 128), dtype=torch.float32, device="cuda")
        for bp in bpools:
            bp.decode_multi(q, lens, n, out=out)
        torch.cuda.synchronize()
        tm = Timer(torch)
        gpu_hold(torch, 5 + 0.5 * steps)
        for i in range(steps):
            s0 = tm.start()
            bpools[i % 4].decode_multi(q, lens, n, out=out)
            tm.stop(s0)
        torch.cuda.synchronize()
        bus = tm.mean_us()
        res[str(t_n)]["bf16_us_per_call"] = round(bus, 3)
        res[str(t_n)]["int2_vs_bf16_speedup"] = round(bus / res[str(t_n)]["us_per_call"], 2)
    del bpools
    torch.cuda.empty_cache()
    return {"workload": f"{hq} q / {hkv} KV heads, one sequence of {n} tokens, the last T positions as queries "
                        f"(causal among them), {n_pools} pools cycled", "by_query_tokens": res}


def _planted_split(seed, n_calib, n_ctx, hq, hkv, per_head_bases=False, q_scale=1.0):
    """Calibration tokens and a decode context drawn from one planted layer
    (same covariance structure, disjoint tokens); q_scale sharpens attention."""
    from bit_rotated_kv_demote_amd import synth
    q, k, v = synth.planted_layer(np.random.default_rng(seed), n_calib + n_ctx, hq, hkv,
                                  per_head_bases=per_head_bases)
    q = (q * np.float32(q_scale)).astype(np.float32)
    calib = (np.ascontiguousarray(q[:n_calib]), synth.bf16_bits_to_f32(k[:n_calib]),
             synth.bf16_bits_to_f32(v[:n_calib]))
    return calib, (q[n_calib:], np.ascontiguousarray(k[n_calib:]), np.ascontiguousarray(v[n_calib:]))


def _decode_error(torch, ctx, hq, hkv, rots, seed, n_query=16):
    """Device prefill of the context and a decode of its last n_query
    positions (each query attending causally, every query head); relative L2
    over all outputs against fp64 attention over the BF16 keys and values,
    computed in NumPy here: the tiers' quantisation error only."""
    from bit_rotated_kv_demote_amd import synth
    from bit_rotated_kv_demote_amd.pool import TieredKV, bf16_tensor
    qt, kt, vt = ctx
    n_ctx = kt.shape[0]
    q = np.ascontiguousarray(synth.to_bf16_bits(qt[-n_query:]))[None]          # [1, T, Hq, 128]
    qf = synth.bf16_bits_to_f32(q)[0].astype(np.float64)
    kf = synth.bf16_bits_to_f32(kt).astype(np.float64)
    vf = synth.bf16_bits_to_f32(vt).astype(np.float64)
    g = hq // hkv
    exact = np.empty((n_query, hq, 128))
    for t in range(n_query):
        p = n_ctx - n_query + t
        for h in range(hq):
            lg = kf[:p + 1, h // g] @ qf[t, h] / math.sqrt(128.0)
            w = np.exp(lg - lg.max())
            exact[t, h] = (w / w.sum()) @ vf[:p + 1, h // g]
    max_pages = math.ceil((n_ctx - 320) / 16)
    pt = synth.page_permutation(np.random.default_rng(seed), max_pages)[None, :].astype(np.int32)
    lens = torch.tensor([n_ctx], dtype=torch.int32, device="cuda")
    pool = TieredKV(hq, hkv, 1, max_pages, max_pages, *rots, page_table=pt)
    pool.prefill(lens, bf16_tensor(kt[None]), bf16_tensor(vt[None]))
    out = pool.decode_multi(bf16_tensor(q), lens, n_ctx).cpu().numpy()[0].astype(np.float64)
    del pool
    return round(float(np.linalg.norm(out - exact) / np.linalg.norm(exact)), 4)


def _host_calibration(torch, hq, hkv, calibs, rotation, per_kv_head=False):
    """oscar_calibrate (one layer) or oscar_calibrate_layers (several) on host tensors."""
    from bit_rotated_kv_demote_amd import binding
    lead = (hkv,) if per_kv_head else ()
    outs = [torch.zeros(lead + (128, 128), dtype=torch.float32), torch.zeros(lead + (128, 128), dtype=torch.float32),
            torch.zeros(lead + (128,), dtype=torch.float32), torch.zeros(lead + (128,), dtype=torch.float32)]
    desc = binding.layer_desc(hq, hkv)
    t0 = time.perf_counter()
    if len(calibs) == 1:
        q, k, v = (torch.from_numpy(x) for x in calibs[0])
        binding.oscar_calibrate(desc, q, k, v, *outs, rotation=rotation, per_kv_head=per_kv_head)
    else:
        q, k, v = (torch.from_numpy(np.ascontiguousarray(np.stack([c[i] for c in calibs]))) for i in range(3))
        binding.oscar_calibrate_layers(desc, q, k, v, *outs, rotation=rotation, per_kv_head=per_kv_head)
    return [o.numpy() for o in outs], round(time.perf_counter() - t0, 2)


def run_rotation_study(torch, seed=1006, hq=32, hkv=8, n_calib=1024, n_ctx=8192, q_scale=1.0):
    """Rotation variants on a layer with planted covariance structure (Qwen3-4B
    attention shape): host calibration with each rotation on n_calib tokens
    of the layer, device prefill of an n_ctx-token context of the same layer
    (bulk demotion) and one device decode; error = relative L2 of the output
    against fp64 attention over the BF16 keys and values.

    Second part, the calibration's scope: a layer whose KV heads each have
    their own planted bases, calibrated layer-wide, per KV head, and shared
    with a second such layer (different bases), each decoded on the first
    layer's context."""
    from bit_rotated_kv_demote_amd import binding
    calib, ctx = _planted_split(seed, n_calib, n_ctx, hq, hkv, q_scale=q_scale)
    errs, calib_s = {}, {}
    for name, code in (("spectral", binding.ROT_SPECTRAL), ("key_attn", binding.ROT_KEY_ATTN),
                       ("hadamard", binding.ROT_HADAMARD), ("identity", binding.ROT_IDENTITY)):
        rots, calib_s[name] = _host_calibration(torch, hq, hkv, [calib], code)
        errs[name] = _decode_error(torch, ctx, hq, hkv, rots, seed + 2)
    calib_a, ctx_a = _planted_split(seed + 10, n_calib, n_ctx, hq, hkv, per_head_bases=True, q_scale=q_scale)
    calib_b, _ = _planted_split(seed + 11, n_calib, 1, hq, hkv, per_head_bases=True, q_scale=q_scale)
    scope_errs, scope_s = {}, {}
    for name, calibs, per_head in (("layer", [calib_a], False), ("per_kv_head", [calib_a], True),
                                   ("shared_with_other_layer", [calib_a, calib_b], False),
                                   ("shared_with_other_layer_per_kv_head", [calib_a, calib_b], True)):
        rots, scope_s[name] = _host_calibration(torch, hq, hkv, calibs, binding.ROT_SPECTRAL, per_head)
        scope_errs[name] = _decode_error(torch, ctx_a, hq, hkv, rots, seed + 12)
    rots, _ = _host_calibration(torch, hq, hkv, [calib_a], binding.ROT_IDENTITY)
    scope_errs["identity"] = _decode_error(torch, ctx_a, hq, hkv, rots, seed + 12)
    torch.cuda.empty_cache()
    return {"workload": f"planted covariance layer, {hq} q / {hkv} KV heads, calibration {n_calib} tokens, "
                        f"context {n_ctx} further tokens of the same layer (64 sink / {n_ctx - 320} INT2 / 256 recent), "
                        "16 decode queries per head",
            "error": "relative L2 over the decode of the context's last 16 positions (causal), all query heads",
            "rel_l2_vs_bf16_attention": errs, "calibrate_host_s": calib_s,
            "scope": {"workload": "spectral rotation on a layer whose KV heads have distinct planted bases; "
                                  "'shared' calibrates over it and a second such layer",
                      "rel_l2_vs_bf16_attention": scope_errs, "calibrate_host_s": scope_s}}


def run_demote(torch, reps, seed, code_bits=2):
    """Bulk demotion of a 4096-token chunk for 16 sequences x 8 KV heads."""
    from bit_rotated_kv_demote_amd import synth
    from bit_rotated_kv_demote_amd.pool import TieredKV, bf16_tensor

    batch, chunk, hkv, hq = 16, 4096, 8, 64
    st = synth.streams(seed)
    out = synth.outlier_channels(st["outliers"])
    k = synth.kv_tokens(st["k"], st["lognormal"], batch * chunk, hkv, out).reshape(batch, chunk, hkv, 128)
    v = synth.kv_tokens(st["v"], st["lognormal"], batch * chunk, hkv, out).reshape(batch, chunk, hkv, 128)
    rot = synth.random_rotation(st["rot"])
    tau = np.full(128, 64.0, np.float32)
    max_pages = 4096 // 16 + 2
    pt = synth.page_permutation(st["perm"], batch * max_pages).reshape(batch, max_pages)
    pool = TieredKV(hq, hkv, batch, max_pages, batch * max_pages, rot, rot, tau, tau, page_table=pt,
                    code_bits=code_bits)
    starts = torch.tensor(synth.ragged_lengths(st["lengths"], batch, 0, 15), dtype=torch.int32, device="cuda")
    kd, vd = bf16_tensor(k), bf16_tensor(v)
    pool.demote(starts, kd, vd)
    torch.cuda.synchronize()
    # back-to-back launches between two events (events around every call
    # would add their own microseconds to each)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gpu_hold(torch, 20)
    e0.record()
    for _ in range(reps):
        pool.demote(starts, kd, vd)
    e1.record()
    torch.cuda.synchronize()
    us = 1000.0 * e0.elapsed_time(e1) / reps
    tokens = batch * chunk
    nbytes = tokens * hkv * (2 * 256 + hist_token_bytes(code_bits))
    return dict(us=us, tok_per_s=tokens / (us * 1e-6), gbps=nbytes / (us * 1e3), tokens=tokens, bytes=nbytes)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_int2_qwen3-4b_32k_traffic.md")


def kernel_source_digest():
    """Digest of the device code (comments and blank lines dropped) and build
    flags of the library; a counter summary taken on other code no longer
    describes the kernel."""
    import hashlib
    from bit_rotated_kv_demote_amd import build
    import re
    h = hashlib.sha256(" ".join(build.DEVICE_FLAGS).encode())
    csrc = os.path.join(ROOT, "bit_rotated_kv_demote_amd", "csrc")
    # the device translation units and the local headers they include (host
    # code such as the calibration does not change what the kernels do)
    todo, seen = list(build.HIP_SOURCES), set()
    while todo:
        name = todo.pop()
        if name in seen or not os.path.exists(os.path.join(csrc, name)):
            continue
        seen.add(name)
        with open(os.path.join(csrc, name), "rb") as f:
            text = f.read()
        todo += re.findall(r'#include "([^"/]+)"', text.decode())
    for name in sorted(seen):
        with open(os.path.join(csrc, name), "rb") as f:
            text = f.read().decode()
        # comments and layout do not change the kernels: hash the code alone
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        code = [ln.split("//", 1)[0].strip() for ln in text.splitlines()]
        h.update(name.encode() + "\n".join(ln for ln in code if ln).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode launch from the committed counter summary (FETCH_SIZE
    + WRITE_SIZE, scaled by the copy-kernel calibration), or None when the
    summary is missing or was taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    block = text.split("```json", 1)[-1].split("```", 1)[0] if "```json" in text else ""
    try:
        rec = json.loads(block)
    except ValueError:
        return None
    if rec.get("source_digest") != kernel_source_digest():
        return None
    return rec.get("bytes_per_launch")


DEMOTE_COUNTERS_FILE = os.path.join(ROOT, "profiles", "demote_bulk_int2_16x4096x8_counters.md")


def demote_counters():
    """Counter figures of the bulk demotion kernel (HBM traffic, matrix-core
    use) from the committed summary, or None when it is missing or was taken
    on other kernel sources."""
    try:
        with open(DEMOTE_COUNTERS_FILE) as f:
            text = f.read()
    except OSError:
        return None
    block = text.split("```json", 1)[-1].split("```", 1)[0] if "```json" in text else ""
    try:
        rec = json.loads(block)
    except ValueError:
        return None
    if rec.get("source_digest") != kernel_source_digest():
        return None
    return {k: rec[k] for k in ("traffic_MB_per_launch", "traffic_vs_algorithmic", "mfma_busy_frac",
                                "mfma_tflops_at_trace_time", "mfma_frac_of_bf16_dense", "valu_issue_frac",
                                "trace_us") if k in rec}


def _oracle_pool(hkv, n0, k, v, rot_k, rot_v, tau_k, tau_v):
    """The oracle's pool after n0 tokens of one sequence (its own demotion of the history)."""
    import oracle as orc
    max_pages = math.ceil((n0 + 1 - 320) / 16)
    pt = np.arange(max_pages, dtype=np.int32)[None, :]
    pool = orc.Pool(1, hkv, max_pages, pt)
    pool.sink_k[0][:, :64] = k[:64].transpose(1, 0, 2)
    pool.sink_v[0][:, :64] = v[:64].transpose(1, 0, 2)
    pos = np.arange(n0 - 256, n0)
    pool.recent_k[0][:, (pos - 64) % 256] = k[pos].transpose(1, 0, 2)
    pool.recent_v[0][:, (pos - 64) % 256] = v[pos].transpose(1, 0, 2)
    h = np.arange(n0 - 320)
    pool.demote_many(0, h, k[64 + h], v[64 + h], rot_k, rot_v, tau_k, tau_v)
    pool.length[0] = n0
    return pool


def cpu_baseline(hq, hkv, n0, host, seed, min_seconds=10.0, host128=None):
    """The oracle, as it stands, on bounded samples of the same work: successive
    32K steps for about min_seconds (all threads), one step on one thread, one
    128K step, and the oracle's demotion of all 16 bulk chunks."""
    import oracle as orc
    from bit_rotated_kv_demote_amd import synth
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threadpool_limits, blas = None, 1
    k, v, rot_k, rot_v, tau_k, tau_v = host
    pool = _oracle_pool(hkv, n0, k, v, rot_k, rot_v, tau_k, tau_v)
    q = synth.queries(synth.streams(seed)["q"], (1, hq, 128))

    def one_step(n):
        t = time.time()
        pool.append(0, k[n], v[n], rot_k, rot_v, tau_k, tau_v)
        orc.decode_tiered(q, pool, [0], [n + 1], rot_k, rot_v)
        return time.time() - t

    # successive steps (append token n, decode all query heads at length n + 1)
    # until about min_seconds of CPU work; one token is kept for the
    # single-thread step
    t0 = time.time()
    n_steps = 0
    while n_steps < len(k) - n0 - 1 and (n_steps == 0 or time.time() - t0 < min_seconds):
        one_step(n0 + n_steps)
        n_steps += 1
    secs = time.time() - t0
    base = {"value": round(secs * 1e6 / n_steps, 1), "unit": "us/step", "cores": int(blas), "kind": "oracle",
            "sample": f"{n_steps} successive steps of the timed workload, each one append (all {hkv} KV heads) "
                      f"+ decode of all {hq} query heads from {n0 + 1} tokens, {secs:.1f} s in total"}
    extra = {"threads_all": int(blas)}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            extra["decode_step_us_one_thread"] = round(one_step(n0 + n_steps) * 1e6, 1)
    # one step at 131072 cached tokens (Qwen3-8B-shaped), all threads
    if host128 is not None:
        k8, v8, rk8, rv8, tk8, tv8, n8 = host128
        t = time.time()
        pool8 = _oracle_pool(hkv, n8, k8, v8, rk8, rv8, tk8, tv8)
        build_s = time.time() - t
        t = time.time()
        pool8.append(0, k8[n8], v8[n8], rk8, rv8, tk8, tv8)
        orc.decode_tiered(q, pool8, [0], [n8 + 1], rk8, rv8)
        extra["ctx128k_step_us"] = round((time.time() - t) * 1e6, 1)
        extra["ctx128k_pool_build_s"] = round(build_s, 1)
        del pool8
    # the oracle's demotion of the bulk workload: 16 chunks of 4096 tokens x
    # all KV heads, K and V (the same token rows stand in for each chunk)

    def demote_chunk():
        cp = orc.Pool(1, hkv, 4096 // 16, np.arange(4096 // 16, dtype=np.int32)[None, :])
        t = time.time()
        cp.demote_many(0, np.arange(4096), k[64:64 + 4096], v[64:64 + 4096], rot_k, rot_v, tau_k, tau_v)
        return (time.time() - t) * 1e6

    chunks = [demote_chunk() for _ in range(16)]
    extra["demote_16_chunks_4096x8_us"] = round(sum(chunks), 1)
    extra["demote_tok_per_s"] = round(16 * 4096 / (sum(chunks) * 1e-6), 1)
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            extra["demote_chunk_4096x8_us_one_thread"] = round(demote_chunk(), 1)
    return base, extra


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=24)
    ap.add_argument("--layers", type=int, default=24, help="distinct pools cycled (>512 MB total)")
    ap.add_argument("--no-extra", action="store_true", help="only the tiered step")
    ap.add_argument("--ctx", type=int, default=32768,
                    help="cached tokens of the timed step (default 32768, the Qwen3-4B-shaped workload; "
                         "other values for profiling runs)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="append one plain device copy of this many MB (counter calibration runs)")
    ap.add_argument("--workload", choices=("step", "demote", "bf16"), default="step",
                    help="step: the timed decode step (the metric, default); demote: only the bulk demotion "
                         "(16 x 4096 tokens x 8 KV heads), --steps launches; bf16: only the BF16 baseline "
                         "decode at --ctx tokens, --steps calls (profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    from bit_rotated_kv_demote_amd import binding
    binding.load()

    hq, hkv, n0 = 32, 8, args.ctx

    def copy_probe():
        # a plain streaming kernel of known size (reads and writes n bytes once):
        # the counter calibration for the traffic figures
        if args.copy_probe_mb:
            src = torch.ones((args.copy_probe_mb << 20) // 4, dtype=torch.float32, device="cuda")
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            torch.neg(src, out=dst)
            torch.cuda.synchronize()

    if args.workload != "step":
        if args.workload == "demote":
            d = run_demote(torch, args.steps, 1004)
            rec = {"workload": "bulk demotion, 16 sequences x 4096 tokens x 8 KV heads, K+V",
                   "us_per_launch": round(d["us"], 3), "tok_per_s": round(d["tok_per_s"], 0),
                   "algorithmic_bytes": d["bytes"], "GBps": round(d["gbps"], 1)}
        else:
            k1, v1 = _seq_kv(hkv, n0, 1001)
            b = run_bf16(torch, hq, hkv, n0, args.layers, args.steps, 1001, k1, v1)
            rec = {"workload": f"BF16 paged decode, {hq} q / {hkv} KV heads, batch 1, {n0} tokens",
                   "us_per_call": round(b["decode_us"], 3), "algorithmic_bytes": b["decode_bytes"],
                   "GBps": round(b["decode_bytes"] / (b["decode_us"] * 1e3), 1)}
        copy_probe()
        print(json.dumps(rec))
        return
    host128 = None
    res = run_tiered(torch, hq, hkv, n0, args.layers, args.steps, args.warmup, seed=1001 if n0 == 32768 else 1002)
    dec_gbps = res["decode_bytes"] / (res["decode_us"] * 1e3)
    # the roofline kernel: the decode's split kernel (oscar_decode_partials)
    split_gbps = res["split_bytes"] / (res["split_us"] * 1e3)
    extra = {"step_mode": "oscar_step (append + decode in one call, two launches: the split kernel writes the new "
                          "token, demotes the leaving one and computes q . R_K; then the merge)",
             "us_per_step_separate_calls": round(res["us_per_step_separate"], 3),
             "step_call_us": round(res["step_call_us"], 3),
             "decode_call_us": round(res["decode_us"], 3), "append_kernel_us": round(res["append_us"], 3),
             "decode_algorithmic_bytes": res["decode_bytes"], "decode_GBps": round(dec_gbps, 1),
             "step_GBps": round(res["decode_bytes"] / (res["us_per_step"] * 1e3), 1),
             "step_frac_of_8TBps": round(res["decode_bytes"] / (res["us_per_step"] * 1e3) / HBM_PEAK_GBPS, 4),
             "roofline_kernel": "decode_int2_kernel<4, false>: the decode's split kernel alone "
                                 "(oscar_decode_partials, back-to-back launches between two events)",
             "split_kernel_us": round(res["split_us"], 3), "split_kernel_bytes": round(res["split_bytes"]),
             "merge_kernel_us": round(res["merge_us"], 3),
             "pools": res["layers"], "pool_MB_total": round(res["pool_mb"], 1),
             "calibrate_host_s": round(res["calib_s"], 2)}
    if not args.no_extra:
        b = run_bf16(torch, hq, hkv, res["n_mid"], 8, min(args.steps, 200), 1001, res["host"][0], res["host"][1])
        extra["bf16_decode_us"] = round(b["decode_us"], 3)
        extra["bf16_decode_GBps"] = round(b["decode_bytes"] / (b["decode_us"] * 1e3), 1)
        extra["int2_vs_bf16_decode_speedup"] = round(b["decode_us"] / res["decode_us"], 3)
        del b
        r128 = run_tiered(torch, hq, hkv, 131072, 8, min(args.steps, 160), 8, seed=1002, calib=res["host"][2:])
        g128 = r128["decode_bytes"] / (r128["decode_us"] * 1e3)
        extra["ctx128k"] = {"us_per_step": round(r128["us_per_step"], 3),
                            "us_per_step_separate_calls": round(r128["us_per_step_separate"], 3),
                            "decode_call_us": round(r128["decode_us"], 3),
                            "append_kernel_us": round(r128["append_us"], 3), "decode_GBps": round(g128, 1),
                            "decode_frac_of_8TBps": round(g128 / HBM_PEAK_GBPS, 4),
                            "split_kernel_us": round(r128["split_us"], 3),
                            "split_kernel_GBps": round(r128["split_bytes"] / (r128["split_us"] * 1e3), 1),
                            "split_kernel_frac_of_8TBps": round(r128["split_bytes"] / (r128["split_us"] * 1e3)
                                                                / HBM_PEAK_GBPS, 4),
                            "merge_kernel_us": round(r128["merge_us"], 3),
                            "decode_algorithmic_bytes": r128["decode_bytes"], "pools": r128["layers"],
                            "pool_MB_total": round(r128["pool_mb"], 1)}
        b128 = run_bf16(torch, hq, hkv, r128["n_mid"], 4, 60, 1002, r128["host"][0], r128["host"][1])
        extra["ctx128k"]["bf16_decode_us"] = round(b128["decode_us"], 3)
        extra["ctx128k"]["bf16_decode_GBps"] = round(b128["decode_bytes"] / (b128["decode_us"] * 1e3), 1)
        extra["ctx128k"]["int2_vs_bf16_decode_speedup"] = round(b128["decode_us"] / r128["decode_us"], 3)
        host128 = tuple(r128["host"]) + (131072,)
        del r128, b128
        extra["ragged_gqa8"] = run_ragged_gqa8(torch, min(args.steps, 50), res["host"][2:])
        extra["fixed_memory_16k"] = run_fixed_memory(torch, min(args.steps, 20), res["host"][2:])
        extra["fixed_memory_100k"] = run_fixed_memory(torch, min(args.steps, 20), res["host"][2:], n=100000)
        extra["multi_query_32k"] = run_multi_query(torch, min(args.steps, 100), res["host"][2:])
        extra["rotation_study"] = run_rotation_study(torch)
        d = run_demote(torch, 20, 1004)
        extra["demote_tok_per_s"] = round(d["tok_per_s"], 0)
        extra["demote_us_per_chunk"] = round(d["us"], 2)
        extra["demote_GBps"] = round(d["gbps"], 1)
        extra["demote_workload"] = "16 sequences x 4096-token chunk, 8 KV heads, K+V, bf16 in, MFMA rotation"
        extra["demote_counters"] = demote_counters()
        # INT4 variant of the pool: the same step, the 128K decode and bulk demotion
        r4 = run_tiered(torch, hq, hkv, n0, args.layers, min(args.steps, 200), args.warmup, seed=1001,
                        calib=res["host"][2:], code_bits=4)
        r4_128 = run_tiered(torch, hq, hkv, 131072, 8, min(args.steps, 160), 8, seed=1002, calib=res["host"][2:],
                            code_bits=4)
        d4 = run_demote(torch, 20, 1004, code_bits=4)
        extra["int4"] = {"us_per_step": round(r4["us_per_step"], 3),
                         "us_per_step_separate_calls": round(r4["us_per_step_separate"], 3),
                         "decode_call_us": round(r4["decode_us"], 3),
                         "append_kernel_us": round(r4["append_us"], 3),
                         "decode_algorithmic_bytes": r4["decode_bytes"],
                         "decode_GBps": round(r4["decode_bytes"] / (r4["decode_us"] * 1e3), 1),
                         "int2_vs_int4_decode_speedup": round(r4["decode_us"] / res["decode_us"], 3),
                         "ctx128k_decode_call_us": round(r4_128["decode_us"], 3),
                         "ctx128k_decode_GBps": round(r4_128["decode_bytes"] / (r4_128["decode_us"] * 1e3), 1),
                         "demote_tok_per_s": round(d4["tok_per_s"], 0), "demote_us_per_chunk": round(d4["us"], 2)}
        del r4, r4_128
    copy_probe()
    cpu = None
    if not args.no_cpu:
        cpu, extra["cpu_oracle"] = cpu_baseline(hq, hkv, n0, res["host"], 1001, host128=host128)
    line = {
        "metric": METRIC,
        "value": round(res["us_per_step"], 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["us_per_step"] / 1000.0, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int2-kv/fp32-acc",
        "data": "synthetic",
        "config": {"workload": {32768: "qwen3-4b-shaped ", 131072: "qwen3-8b-shaped "}.get(n0, "") +
                               "tiered decode step (oscar_step: append + decode): 32 q / 8 KV heads, "
                               f"head_dim 128, batch 1, {n0} cached tokens + 1 appended per step, "
                               "64 bf16 sink / int2 history / 256 bf16 recent, 16-token pages",
                   "global_batch": 1, "seq_len": n0, "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": round(split_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(split_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic() if n0 == 32768 else None},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    extra["source_digest"] = kernel_source_digest()
    print(json.dumps(line))


if __name__ == "__main__":
    main()
