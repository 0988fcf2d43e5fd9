"""GPU parity of the INT4 variant of the history pool (16 levels, two codes
per byte, 2560-byte blocks; the INT4 baseline of "OSCAR: Offline Spectral
Covariance-Aware Rotation for 2-bit KV Cache Quantization" (gist.science),
section 4).

Same bars as the INT2 pool: bulk demotion from rotated fp32 bit-exact
against the oracle; from bf16 (rotation on the matrix cores) and through
append / prefill at most 0.1 % of codes off by one with scales and zeros
within 2 fp16 ulp; decode (one and several queries, every column grouping,
the large-grid merge and the 32K workload on sampled KV heads) within a
relative L2 of 2e-3 of the oracle's attention over the oracle's own bytes."""
import numpy as np
import pytest
import torch

import oracle as orc
from bit_rotated_kv_demote_amd import binding, synth
from bit_rotated_kv_demote_amd.pool import bf16_tensor

from _gpu_util import Layer, code_diff_stats, i32, rel_l2, upload
from test_gpu_demote import _rotated_inputs

pytestmark = pytest.mark.gpu

FLIP_RATE = 1e-3
TOL = 2e-3


def test_int4_demote_from_rotated_fp32_is_bit_exact():
    batch, n_tokens = 3, 70
    layer = Layer(seed=1400, batch=batch, hq=8, hkv=4, max_len=64 + 48 + n_tokens + 256 + 16, code_bits=4)
    starts = [0, 5, 37]
    yk, yv = _rotated_inputs(layer, batch, n_tokens, starts)
    dev = layer.device_pool()
    dev.demote(i32(starts), torch.from_numpy(yk).cuda(), torch.from_numpy(yv).cuda(),
               src_kind=binding.OSCAR_SRC_F32_ROTATED)
    torch.cuda.synchronize()
    ref = orc.Pool(batch, layer.hkv, layer.num_pages, layer.page_table, bits=4)
    for b in range(batch):
        ref.demote_rotated_many(b, np.arange(starts[b], starts[b] + n_tokens), yk[b], yv[b], layer.tau_k, layer.tau_v)
    got = dev.hist.cpu().numpy()
    assert got.shape[-1] == 2560
    assert np.array_equal(got, ref.hist), f"{np.count_nonzero(got != ref.hist)} bytes differ"


def test_int4_demote_bf16_fused_rotation_within_flip_budget():
    batch, n_tokens = 2, 600
    layer = Layer(seed=1401, batch=batch, hq=16, hkv=8, max_len=64 + n_tokens + 256 + 32, code_bits=4)
    starts = [0, 9]
    k = np.ascontiguousarray(np.stack([layer.k[b, 64 + starts[b]:64 + starts[b] + n_tokens] for b in range(batch)]))
    v = np.ascontiguousarray(np.stack([layer.v[b, 64 + starts[b]:64 + starts[b] + n_tokens] for b in range(batch)]))
    dev = layer.device_pool()
    dev.demote(i32(starts), bf16_tensor(k), bf16_tensor(v))
    torch.cuda.synchronize()
    ref = orc.Pool(batch, layer.hkv, layer.num_pages, layer.page_table, bits=4)
    for b in range(batch):
        ref.demote_many(b, np.arange(starts[b], starts[b] + n_tokens), k[b], v[b], layer.rot, layer.rot,
                        layer.tau_k, layer.tau_v)
    got = dev.hist.cpu().numpy()
    pages = np.concatenate([layer.page_table[b, (starts[b] + np.arange(n_tokens)) // 16] for b in range(batch)])
    slots = np.concatenate([(starts[b] + np.arange(n_tokens)) % 16 for b in range(batch)])
    rate, maxd, meta_ulp = code_diff_stats(got, ref.hist, pages, slots)
    assert rate <= FLIP_RATE and maxd <= 1 and meta_ulp <= 2, (rate, maxd, meta_ulp)
    untouched = np.ones(got.shape[0], bool)
    untouched[np.unique(pages)] = False
    assert not got[untouched].any()


def test_int4_prefill_and_append_match_oracle_state_machine():
    lengths, n_app = [50, 333, 700], 30
    layer = Layer(seed=1402, batch=3, hq=8, hkv=2, max_len=max(lengths) + n_app, code_bits=4)
    dev = layer.device_pool()
    dev.prefill(i32(lengths), bf16_tensor(np.ascontiguousarray(layer.k[:, :max(lengths)])),
                bf16_tensor(np.ascontiguousarray(layer.v[:, :max(lengths)])))
    for s in range(n_app):
        pos = [n + s for n in lengths]
        dev.append(i32(pos), bf16_tensor(np.ascontiguousarray(layer.k[np.arange(3), pos])),
                   bf16_tensor(np.ascontiguousarray(layer.v[np.arange(3), pos])))
    torch.cuda.synchronize()
    final = [n + n_app for n in lengths]
    ref = layer.oracle_pool(final)
    st = dev.host_state()
    for name in ("sink_k", "sink_v", "recent_k", "recent_v"):
        assert np.array_equal(st[name], getattr(ref, name)), name
    pages, sl = [], []
    for b, n in enumerate(final):
        h = np.arange(max(0, n - 320))
        pages.append(layer.page_table[b, h // 16])
        sl.append(h % 16)
    rate, maxd, meta_ulp = code_diff_stats(st["hist"], ref.hist, np.concatenate(pages), np.concatenate(sl))
    assert rate <= FLIP_RATE and maxd <= 1 and meta_ulp <= 2, (rate, maxd, meta_ulp)


@pytest.mark.parametrize("hq,hkv,n_query", [(8, 2, 1), (2, 2, 1), (16, 2, 1), (8, 8, 1), (8, 2, 4), (8, 2, 8),
                                            (32, 8, 16)])
def test_int4_decode_matches_oracle(hq, hkv, n_query):
    # G = 4, 1, 8, 1 with one query; 4 and 8 queries (8- and 16-column
    # groups); GQA-4 with 16 queries (16-column groups, two score tiles)
    lengths = [1500, 333, 70]
    layer = Layer(seed=1410 + hq + 10 * n_query, batch=3, hq=hq, hkv=hkv, max_len=max(lengths), code_bits=4)
    opool = layer.oracle_pool(lengths)
    dev = layer.device_pool()
    upload(dev, opool)
    q = synth.queries(np.random.default_rng(30 + n_query), (3, n_query, hq, 128))
    out = dev.decode_multi(bf16_tensor(q), i32(lengths), max(lengths)).cpu().numpy()
    ref = orc.attend_tail_tiered(q, opool, [0, 1, 2], lengths, layer.rot, layer.rot)
    for b in range(3):
        assert rel_l2(out[b], ref[b]) <= TOL, (b, rel_l2(out[b], ref[b]))
    if n_query == 1:
        single = dev.decode(bf16_tensor(np.ascontiguousarray(q[:, 0])), i32(lengths), max(lengths)).cpu().numpy()
        assert np.array_equal(single, out[:, 0])


def test_int4_large_grid_merge_per_record_group():
    lengths = [330 + 14 * b for b in range(26)]
    layer = Layer(seed=1420, batch=26, hq=32, hkv=8, max_len=max(lengths), code_bits=4)
    opool = layer.oracle_pool(lengths)
    dev = layer.device_pool()
    upload(dev, opool)
    q = synth.queries(np.random.default_rng(31), (26, 1, 32, 128))
    out = dev.decode_multi(bf16_tensor(q), i32(lengths), max(lengths)).cpu().numpy()
    ref = orc.attend_tail_tiered(q, opool, list(range(26)), lengths, layer.rot, layer.rot)
    assert rel_l2(out, ref) <= TOL


@pytest.mark.parametrize("n,kv_heads,seed", [(32768, [1, 6], 1430), (131072, [4], 1431)])
def test_int4_full_size_sampled_heads(n, kv_heads, seed):
    # the 32K and 128K workloads' shape (32 q / 8 KV heads): device prefill
    # for every KV head, the oracle's bytes for the compared KV heads
    layer = Layer(seed=seed, batch=1, hq=32, hkv=8, max_len=n, code_bits=4)
    opool = layer.oracle_pool([n], kv_heads)
    dev = layer.device_pool()
    dev.prefill(i32([n]), bf16_tensor(layer.k), bf16_tensor(layer.v))
    upload(dev, opool, kv_heads)
    q = synth.queries(np.random.default_rng(32), (1, 32, 128))
    out = dev.decode(bf16_tensor(q), i32([n]), n).cpu().numpy()
    heads = [(0, h) for h in range(32) if h // 4 in kv_heads]
    ref = orc.decode_tiered(q, opool, [0], [n], layer.rot, layer.rot, heads=heads)
    idx = [h for _, h in heads]
    assert rel_l2(out[0][idx], ref[0][idx]) <= TOL
