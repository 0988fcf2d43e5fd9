"""GPU parity of several query tokens per sequence (oscar_decode_multi).

The device decodes the oracle's own pool bytes (uploaded), and is compared
with the oracle's attention of the last T positions (reading R11: query t at
position n - T + t attends causally to [0, n - T + t]).  Tolerance: relative
L2 <= 2e-3 over the output, as for single-token decode.  The cases cover
every column grouping the library picks (T * G virtual heads in work items
of 1, 2, 4 or 8 columns), causal limits inside the sink, inside the recent
ring and across the ring's wrap, ragged batches with slot indirection, and a
64-token chunk."""
import math

import numpy as np
import pytest
import torch

import oracle as orc
from bit_rotated_kv_demote_amd import synth
from bit_rotated_kv_demote_amd.pool import PagedBF16, bf16_tensor

from _gpu_util import Layer, i32, rel_l2, upload

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _multi_vs_oracle(layer, lengths, n_query, seed, seq_slot=None):
    # batch entry b reads slot seq_slot[b] (default b); slot s holds sequence
    # s's tokens, as many as the batch entry that reads it asks for
    slots = list(range(layer.batch)) if seq_slot is None else list(seq_slot)
    lens_by_slot = [0] * layer.batch
    for b, s in enumerate(slots):
        lens_by_slot[s] = lengths[b]
    opool = layer.oracle_pool(lens_by_slot)
    dev = layer.device_pool()
    upload(dev, opool)
    q = synth.queries(np.random.default_rng(seed), (layer.batch, n_query, layer.hq, 128))
    out = dev.decode_multi(bf16_tensor(q), i32(lengths), max(lengths),
                           seq_slot=None if seq_slot is None else i32(slots)).cpu().numpy()
    ref = orc.attend_tail_tiered(q, opool, slots, lengths, layer.rot, layer.rot)
    return out, ref


@pytest.mark.parametrize("n_query", [1, 2, 3, 4, 8])
def test_multi_query_gqa4_with_history(n_query):
    layer = Layer(seed=1100 + n_query, batch=1, hq=8, hkv=2, max_len=1000)
    out, ref = _multi_vs_oracle(layer, [1000], n_query, 7)
    assert rel_l2(out, ref) <= TOL


@pytest.mark.parametrize("hq,hkv,n_query", [(2, 2, 5), (16, 2, 2)])
def test_multi_query_mha_and_gqa8(hq, hkv, n_query):
    layer = Layer(seed=1110 + hq, batch=1, hq=hq, hkv=hkv, max_len=900)
    out, ref = _multi_vs_oracle(layer, [900], n_query, 8)
    assert rel_l2(out, ref) <= TOL


def test_multi_query_single_equals_decode():
    layer = Layer(seed=1120, batch=1, hq=8, hkv=2, max_len=700)
    opool = layer.oracle_pool([700])
    dev = layer.device_pool()
    upload(dev, opool)
    q = synth.queries(np.random.default_rng(9), (1, 1, 8, 128))
    multi = dev.decode_multi(bf16_tensor(q), i32([700]), 700).cpu().numpy()
    single = dev.decode(bf16_tensor(np.ascontiguousarray(q[:, 0])), i32([700]), 700).cpu().numpy()
    assert np.array_equal(multi[:, 0], single)


@pytest.mark.parametrize("n,n_query", [(40, 8), (70, 16), (330, 12), (2000, 64)])
def test_multi_query_causal_limits_in_every_tier(n, n_query):
    # n = 40: all queries in the sink; 70: queries straddle sink and ring;
    # 330: the ring has wrapped and history starts; 2000: a 64-token chunk.
    layer = Layer(seed=1130 + n, batch=1, hq=8, hkv=2, max_len=n)
    out, ref = _multi_vs_oracle(layer, [n], n_query, 10)
    assert rel_l2(out, ref) <= TOL


def test_multi_query_ragged_batch_with_slots():
    layer = Layer(seed=1140, batch=3, hq=8, hkv=2, max_len=1500)
    lengths = [1500, 333, 860]
    out, ref = _multi_vs_oracle(layer, lengths, 4, 11, seq_slot=[2, 0, 1])
    for b in range(3):
        assert rel_l2(out[b], ref[b]) <= TOL, b


@pytest.mark.parametrize("n_query", [1, 3, 4, 16])
def test_bf16_baseline_multi_query(n_query):
    # 8 q / 2 KV heads: T * 4 virtual heads in work items of up to 16 columns
    lengths = [1200, 70]
    hq, hkv = 8, 2
    st = synth.streams(1150 + n_query)
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
    q = synth.queries(st["q"], (len(lengths), n_query, hq, 128))
    pool = PagedBF16(hq, hkv, kv, pt)
    out = pool.decode_multi(bf16_tensor(q), i32(lengths), max(lengths)).cpu().numpy()
    ref = orc.attend_tail_bf16(q, kv, pt, [0, 1], lengths)
    for b in range(len(lengths)):
        assert rel_l2(out[b], ref[b]) <= TOL, lengths[b]


@pytest.mark.parametrize("n_query", [4, 8, 64])
def test_multi_query_qwen3_4b_32k_sampled_heads(n_query):
    # Full size of the bench's multi-query workload: 32 q / 8 KV heads, 32768
    # cached tokens, the last T as queries; device prefill for every KV head,
    # the oracle's bytes for the two compared KV heads.
    n = 32768
    layer = Layer(seed=1160 + n_query, batch=1, hq=32, hkv=8, max_len=n)
    kv_heads = [0, 5]
    opool = layer.oracle_pool([n], kv_heads)
    dev = layer.device_pool()
    dev.prefill(i32([n]), bf16_tensor(layer.k), bf16_tensor(layer.v))
    upload(dev, opool, kv_heads)
    q = synth.queries(np.random.default_rng(12), (1, n_query, 32, 128))
    out = dev.decode_multi(bf16_tensor(q), i32([n]), n).cpu().numpy()
    heads = [(0, h) for h in range(32) if h // 4 in kv_heads]
    ref = orc.attend_tail_tiered(q, opool, [0], [n], layer.rot, layer.rot, heads=heads)
    idx = [h for _, h in heads]
    assert rel_l2(out[0][:, idx], ref[0][:, idx]) <= TOL


def test_large_grid_merge_per_record_group():
    # 26 sequences x 32 query heads = 832 merged heads: past the size where
    # the merge switches to one workgroup per record group (shared R load).
    lengths = [330 + 14 * b for b in range(26)]
    layer = Layer(seed=1170, batch=26, hq=32, hkv=8, max_len=max(lengths))
    out, ref = _multi_vs_oracle(layer, lengths, 1, 13)
    assert rel_l2(out, ref) <= TOL


def test_large_grid_merge_multi_query_16_columns():
    # 4 sequences x 8 queries x 32 heads = 1024 merged heads in 64 groups of
    # 16 columns: four merge workgroups per group, four columns each
    lengths = [900, 410, 1300, 333]
    layer = Layer(seed=1171, batch=4, hq=32, hkv=8, max_len=max(lengths))
    out, ref = _multi_vs_oracle(layer, lengths, 8, 14)
    for b in range(4):
        assert rel_l2(out[b], ref[b]) <= TOL, b


def test_large_grid_merge_two_parts_per_record_group():
    # 20 sequences x 8 queries x 32 heads = 5120 merged heads in 320 groups of
    # 16 columns: two merge workgroups per group, eight columns each
    lengths = [330 + 17 * b for b in range(20)]
    layer = Layer(seed=1172, batch=20, hq=32, hkv=8, max_len=max(lengths))
    out, ref = _multi_vs_oracle(layer, lengths, 8, 15)
    for b in range(20):
        assert rel_l2(out[b], ref[b]) <= TOL, b