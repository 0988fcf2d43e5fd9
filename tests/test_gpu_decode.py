"""GPU parity of tiered decode attention (and the BF16 baseline).

Decode parity runs on identical pool bytes: the oracle builds the pool from
the seeded inputs, the bytes are uploaded to the device, and the device
decode is compared with the oracle's decode of the same bytes.  Tolerance:
relative L2 over the compared heads <= 2e-3 (fp32 accumulation)."""
import math

import numpy as np
import pytest
import torch

import oracle as orc
from bit_rotated_kv_demote_amd import synth
from bit_rotated_kv_demote_amd.pool import PagedBF16, bf16_tensor

from _gpu_util import Layer, check_state_vs_oracle, decode_over_device_bytes, i32, rel_l2, upload

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _decode_vs_oracle(layer, lengths, kv_heads=None, max_seq_len=None, q_index=0, prefill_device=False):
    opool = layer.oracle_pool(lengths, kv_heads)
    dev = layer.device_pool()
    if prefill_device:
        dev.prefill(i32(lengths), bf16_tensor(layer.k), bf16_tensor(layer.v))
    upload(dev, opool, kv_heads)
    q = np.ascontiguousarray(layer.q[q_index])
    out = dev.decode(bf16_tensor(q), i32(lengths), max_seq_len or max(lengths)).cpu().numpy()
    g = layer.hq // layer.hkv
    heads = None
    if kv_heads is not None:
        heads = [(b, h) for b in range(layer.batch) for h in range(layer.hq) if h // g in kv_heads]
    ref = orc.decode_tiered(q, opool, list(range(layer.batch)), lengths, layer.rot, layer.rot, heads=heads)
    if heads is None:
        return out, ref
    idx = tuple(np.array(heads).T)
    return out[idx], ref[idx]


def test_decode_tiny_config_32_steps():
    # 1 layer, batch 1, 2 q heads / 1 KV head, context 1024 (64 sink + 704 INT2
    # + 256 recent), then 32 steps, each appending one token before decoding.
    n0, steps = 1024, 32
    layer = Layer(seed=1000, batch=1, hq=2, hkv=1, max_len=n0 + steps, n_q=steps)
    opool = layer.oracle_pool([n0])
    dev = layer.device_pool()
    for s in range(steps):
        p = n0 + s
        opool.append(0, layer.k[0, p], layer.v[0, p], layer.rot, layer.rot, layer.tau_k, layer.tau_v)
        upload(dev, opool)
        q = np.ascontiguousarray(layer.q[s])
        out = dev.decode(bf16_tensor(q), i32([p + 1]), n0 + steps).cpu().numpy()
        ref = orc.decode_tiered(q, opool, [0], [p + 1], layer.rot, layer.rot)
        err = rel_l2(out, ref)
        assert err <= TOL, (s, err)


def test_decode_end_to_end_with_device_appends():
    # Device append + device decode, checked in two parts against the oracle:
    # the device's bytes after its own appends against the oracle's pool after
    # the same appends (tiers byte for byte, demoted codes within the fused
    # budget), and each decode against the oracle's decode of the device's
    # own bytes (2e-3).
    n0, steps = 700, 24
    layer = Layer(seed=1001, batch=1, hq=4, hkv=1, max_len=n0 + steps, n_q=steps)
    opool = layer.oracle_pool([n0])
    dev = layer.device_pool()
    upload(dev, opool)
    for s in range(steps):
        p = n0 + s
        opool.append(0, layer.k[0, p], layer.v[0, p], layer.rot, layer.rot, layer.tau_k, layer.tau_v)
        dev.append(i32([p]), bf16_tensor(np.ascontiguousarray(layer.k[:, p])),
                   bf16_tensor(np.ascontiguousarray(layer.v[:, p])))
        q = np.ascontiguousarray(layer.q[s])
        out = dev.decode(bf16_tensor(q), i32([p + 1]), n0 + steps).cpu().numpy()
        ref = decode_over_device_bytes(dev.host_state(), 1, q, [0], [p + 1], layer.rot, layer.rot)
        assert rel_l2(out, ref) <= TOL, s
    check_state_vs_oracle(dev.host_state(), opool, [(0, np.arange(n0 - 320, n0 + steps - 320))])


@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_decode_edge_lengths_all_groups(group):
    lengths = [1, 17, 63, 64, 65, 200, 320, 321, 336, 337, 1000, 1531]
    layer = Layer(seed=1100 + group, batch=len(lengths), hq=2 * group, hkv=2, max_len=max(lengths))
    out, ref = _decode_vs_oracle(layer, lengths)
    for b in range(len(lengths)):
        assert rel_l2(out[b], ref[b]) <= TOL, (group, lengths[b])


def test_decode_invariant_to_split_count_and_page_order():
    lengths = [3000, 1200]
    layer = Layer(seed=1200, batch=2, hq=8, hkv=2, max_len=max(lengths), extra_pages=200)
    opool = layer.oracle_pool(lengths)
    dev = layer.device_pool()
    upload(dev, opool)
    q = bf16_tensor(np.ascontiguousarray(layer.q[0]))
    a = dev.decode(q, i32(lengths), 3000).cpu().numpy()
    b = dev.decode(q, i32(lengths), 3000 + 16 * 200).cpu().numpy()   # larger split size
    c = dev.decode(q, i32(lengths), 3000).cpu().numpy()              # workspace reuse
    assert rel_l2(b, a) <= 1e-5 and np.array_equal(a, c)
    # same tokens under a different page permutation
    perm_layer = Layer(seed=1200, batch=2, hq=8, hkv=2, max_len=max(lengths), extra_pages=200)
    perm_layer.page_table = np.ascontiguousarray(perm_layer.page_table[:, ::-1])
    opool2 = perm_layer.oracle_pool(lengths)
    dev2 = perm_layer.device_pool()
    upload(dev2, opool2)
    d = dev2.decode(q, i32(lengths), 3000).cpu().numpy()
    assert rel_l2(d, a) <= 1e-5
    ref = orc.decode_tiered(layer.q[0], opool, [0, 1], lengths, layer.rot, layer.rot)
    assert rel_l2(a, ref) <= TOL


def test_decode_ragged_batch_gqa8_shuffled_pages():
    # Qwen3-32B-shaped heads (64 q / 8 KV) on a ragged batch of 16 with
    # shuffled page tables; context lengths scaled down 10x for the oracle.
    rng = synth.streams(4)["lengths"]
    lengths = synth.ragged_lengths(rng, 16, 820, 6554).tolist()
    layer = Layer(seed=1004, batch=16, hq=64, hkv=8, max_len=max(lengths))
    out, ref = _decode_vs_oracle(layer, lengths, kv_heads=[2, 7], prefill_device=True)
    assert rel_l2(out, ref) <= TOL


def test_decode_ragged_gqa8_full_size_sampled_heads():
    # The ragged Qwen3-32B-shaped workload at full size, in the launch
    # configuration the bench times: 64 q / 8 KV heads, 16 sequences with
    # seeded lengths U[8192, 65536], each a prefix of one seeded token stream,
    # shuffled pages.  The device prefills and decodes the whole batch; the
    # oracle's bytes replace the device's for two KV heads, and their 16 query
    # heads are checked on four sequences (the longest, the shortest and two
    # others; the oracle's share stays at seconds).
    from bit_rotated_kv_demote_amd.pool import TieredKV
    hq, hkv, B, kv_heads = 64, 8, 16, [2, 7]
    st = synth.streams(1005)
    lengths = [int(x) for x in synth.ragged_lengths(st["lengths"], B, 8192, 65536)]
    n_max = max(lengths)
    out_ch = synth.outlier_channels(st["outliers"])
    k = synth.kv_tokens(st["k"], st["lognormal"], n_max, hkv, out_ch)
    v = synth.kv_tokens(st["v"], st["lognormal"], n_max, hkv, out_ch)
    rot = synth.random_rotation(st["rot"])
    tau_k = orc.clip_thresholds(synth.bf16_bits_to_f32(k[:4096]), rot)
    tau_v = orc.clip_thresholds(synth.bf16_bits_to_f32(v[:4096]), rot)
    max_pages = math.ceil((n_max - 320) / 16)
    pt = synth.page_permutation(st["perm"], B * max_pages).reshape(B, max_pages).astype(np.int32)
    dev = TieredKV(hq, hkv, B, max_pages, B * max_pages, rot, rot, tau_k, tau_v, page_table=pt)
    kd, vd = bf16_tensor(k), bf16_tensor(v)
    for b0 in range(0, B, 4):
        bs = list(range(b0, b0 + 4))
        n = max(lengths[b] for b in bs)
        dev.prefill(i32([lengths[b] for b in bs]), kd[None, :n].expand(4, -1, -1, -1).contiguous(),
                    vd[None, :n].expand(4, -1, -1, -1).contiguous(), seq_slot=i32(bs))
    del kd, vd
    checked = sorted({int(np.argmax(lengths)), int(np.argmin(lengths)), 0, 5})
    opool = orc.Pool(B, hkv, B * max_pages, pt)
    for b in checked:
        n = lengths[b]
        opool.sink_k[b] = k[:64].transpose(1, 0, 2)
        opool.sink_v[b] = v[:64].transpose(1, 0, 2)
        pos = np.arange(n - 256, n)
        opool.recent_k[b][:, (pos - 64) % 256] = k[pos].transpose(1, 0, 2)
        opool.recent_v[b][:, (pos - 64) % 256] = v[pos].transpose(1, 0, 2)
        h = np.arange(n - 320)
        opool.demote_many(b, h, k[64 + h][:, kv_heads], v[64 + h][:, kv_heads], rot, rot, tau_k, tau_v,
                          kv_heads=kv_heads)
        opool.length[b] = n
    # (the unchecked sequences' blocks of these heads become zeros: their
    # outputs are computed but not compared)
    upload(dev, opool, kv_heads)
    q = synth.queries(st["q"], (B, hq, 128))
    out = dev.decode(bf16_tensor(q), i32(lengths), n_max).cpu().numpy()
    heads = [(b, h) for b in checked for h in range(hq) if h // 8 in kv_heads]
    ref = orc.decode_tiered(q, opool, list(range(B)), lengths, rot, rot, heads=heads)
    idx = tuple(np.array(heads).T)
    assert rel_l2(out[idx], ref[idx]) <= TOL


def test_decode_fixed_memory_max_batch_sampled():
    # The fixed-memory workload's largest INT2 batch: 130 sequences of 16384
    # tokens (32 q / 8 KV heads), 4160 merged heads (the per-record-group
    # merge), all sequences prefixes of one seeded stream, shuffled pages.
    # The oracle's bytes replace the device's for two KV heads; three
    # sequences are checked.
    from bit_rotated_kv_demote_amd.pool import TieredKV
    hq, hkv, B, n, kv_heads = 32, 8, 130, 16384, [1, 6]
    st = synth.streams(1004)
    out_ch = synth.outlier_channels(st["outliers"])
    k = synth.kv_tokens(st["k"], st["lognormal"], n, hkv, out_ch)
    v = synth.kv_tokens(st["v"], st["lognormal"], n, hkv, out_ch)
    rot = synth.random_rotation(st["rot"])
    tau_k = orc.clip_thresholds(synth.bf16_bits_to_f32(k[:4096]), rot)
    tau_v = orc.clip_thresholds(synth.bf16_bits_to_f32(v[:4096]), rot)
    max_pages = math.ceil((n - 320) / 16)
    pt = synth.page_permutation(st["perm"], B * max_pages).reshape(B, max_pages).astype(np.int32)
    dev = TieredKV(hq, hkv, B, max_pages, B * max_pages, rot, rot, tau_k, tau_v, page_table=pt)
    kd = bf16_tensor(k)[None].expand(10, -1, -1, -1).contiguous()
    vd = bf16_tensor(v)[None].expand(10, -1, -1, -1).contiguous()
    for b0 in range(0, B, 10):
        dev.prefill(i32([n] * 10), kd, vd, seq_slot=i32(list(range(b0, b0 + 10))))
    del kd, vd
    checked = [0, 77, 129]
    opool = orc.Pool(B, hkv, B * max_pages, pt)
    h = np.arange(n - 320)
    pos = np.arange(n - 256, n)
    for b in checked:
        opool.sink_k[b] = k[:64].transpose(1, 0, 2)
        opool.sink_v[b] = v[:64].transpose(1, 0, 2)
        opool.recent_k[b][:, (pos - 64) % 256] = k[pos].transpose(1, 0, 2)
        opool.recent_v[b][:, (pos - 64) % 256] = v[pos].transpose(1, 0, 2)
        opool.demote_many(b, h, k[64 + h][:, kv_heads], v[64 + h][:, kv_heads], rot, rot, tau_k, tau_v,
                          kv_heads=kv_heads)
        opool.length[b] = n
    upload(dev, opool, kv_heads)
    q = synth.queries(st["q"], (B, hq, 128))
    out = dev.decode(bf16_tensor(q), i32([n] * B), n).cpu().numpy()
    heads = [(b, hh) for b in checked for hh in range(hq) if hh // 4 in kv_heads]
    ref = orc.decode_tiered(q, opool, list(range(B)), [n] * B, rot, rot, heads=heads)
    idx = tuple(np.array(heads).T)
    assert rel_l2(out[idx], ref[idx]) <= TOL


def test_decode_qwen3_4b_32k_sampled_heads():
    # Full size of the 32K workload, in the bench's launch configuration:
    # 32 q / 8 KV heads, 32768 cached tokens + the appended one.
    n = 32768 + 1
    layer = Layer(seed=1001, batch=1, hq=32, hkv=8, max_len=n)
    out, ref = _decode_vs_oracle(layer, [n], kv_heads=[0, 5], max_seq_len=n, prefill_device=True)
    assert rel_l2(out, ref) <= TOL


def test_decode_qwen3_8b_128k_sampled_head():
    n = 131072 + 1
    layer = Layer(seed=1002, batch=1, hq=32, hkv=8, max_len=n)
    out, ref = _decode_vs_oracle(layer, [n], kv_heads=[3], max_seq_len=n, prefill_device=True)
    assert rel_l2(out, ref) <= TOL


def test_bf16_baseline_matches_oracle():
    lengths = [1, 500, 2000]
    hq, hkv = 8, 2
    st = synth.streams(77)
    out_ch = synth.outlier_channels(st["outliers"])
    max_pages = math.ceil(max(lengths) / 16)
    num_pages = len(lengths) * max_pages
    pt = synth.page_permutation(st["perm"], num_pages).reshape(len(lengths), max_pages)
    kv = np.zeros((num_pages, hkv, 2, 16, 128), np.uint16)
    for b, n in enumerate(lengths):
        k = synth.kv_tokens(st["k"], st["lognormal"], n, hkv, out_ch)
        v = synth.kv_tokens(st["v"], st["lognormal"], n, hkv, out_ch)
        for p in range(n):
            kv[pt[b, p // 16], :, 0, p % 16] = k[p]
            kv[pt[b, p // 16], :, 1, p % 16] = v[p]
    q = synth.queries(st["q"], (len(lengths), hq, 128))
    pool = PagedBF16(hq, hkv, kv, pt)
    out = pool.decode(bf16_tensor(q), i32(lengths), max(lengths)).cpu().numpy()
    ref = orc.decode_bf16(q, kv, pt, [0, 1, 2], lengths)
    for b in range(len(lengths)):
        assert rel_l2(out[b], ref[b]) <= TOL, lengths[b]


@pytest.mark.parametrize("n,kv_heads", [(32768, [0, 3, 6]), (131072, [1, 6])])
def test_bf16_baseline_full_size_sampled_heads(n, kv_heads):
    # The BF16 baseline at the sizes the benchmark times it (32 q / 8 KV heads,
    # one sequence of 32768 or 131072 tokens, shuffled pages): the query heads
    # of some KV heads against the oracle's decode of the same pool bytes.
    hq, hkv = 32, 8
    st = synth.streams(1700 + n % 1000)
    out_ch = synth.outlier_channels(st["outliers"])
    k = synth.kv_tokens(st["k"], st["lognormal"], n, hkv, out_ch)
    v = synth.kv_tokens(st["v"], st["lognormal"], n, hkv, out_ch)
    pages = math.ceil(n / 16)
    pt = synth.page_permutation(st["perm"], pages)[None, :].astype(np.int32)
    kv = np.zeros((pages, hkv, 2, 16, 128), np.uint16)
    pos = np.arange(n)
    kv[pt[0, pos // 16], :, 0, pos % 16] = k
    kv[pt[0, pos // 16], :, 1, pos % 16] = v
    q = synth.queries(st["q"], (1, hq, 128))
    pool = PagedBF16(hq, hkv, kv, pt)
    out = pool.decode(bf16_tensor(q), i32([n]), n).cpu().numpy()
    # the oracle over the sampled KV heads only (a pool view of those heads)
    sub = np.ascontiguousarray(kv[:, kv_heads])
    q_sub = np.ascontiguousarray(np.concatenate([q[:, 4 * j:4 * j + 4] for j in kv_heads], axis=1))
    ref = orc.decode_bf16(q_sub, sub, pt, [0], [n])
    got = np.concatenate([out[:, 4 * j:4 * j + 4] for j in kv_heads], axis=1)
    assert rel_l2(got, ref) <= TOL


@pytest.mark.parametrize("hq,hkv,lengths", [(8, 2, [1500, 300, 2047]), (16, 2, [5000, 64])])
def test_decode_phases_equal_decode_and_oracle(hq, hkv, lengths):
    # oscar_decode_partials then oscar_decode_merge on one stream are the two
    # launches of oscar_decode: the outputs are identical, and match the oracle.
    layer = Layer(seed=1011, batch=len(lengths), hq=hq, hkv=hkv, max_len=max(lengths) + 16)
    opool = layer.oracle_pool(lengths)
    dev = layer.device_pool()
    upload(dev, opool)
    q = bf16_tensor(np.ascontiguousarray(layer.q[0]))
    lens = i32(lengths)
    max_len = max(lengths) + 16
    whole = dev.decode(q, lens, max_len).cpu().numpy()
    dev.workspace(len(lengths), max_len).fill_(0xA5)     # stale bytes: the partials call must overwrite them
    dev.decode_partials(q, lens, max_len)
    split = dev.decode_merge(lens, len(lengths), max_len).cpu().numpy()
    assert np.array_equal(whole, split)
    ref = orc.decode_tiered(np.ascontiguousarray(layer.q[0]), opool, list(range(len(lengths))), lengths, layer.rot,
                            layer.rot)
    assert rel_l2(split, ref) <= TOL
