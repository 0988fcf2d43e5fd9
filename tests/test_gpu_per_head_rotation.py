"""GPU parity with one R_K, R_V and clip-threshold pair per KV head (the
per-KV-head calibration scope; the zingnex page's section on offline
optimisation speaks of the rotation's sharing scope).

Every kernel that reads a rotation or a threshold is covered: bulk demotion
from rotated fp32 (bit-exact) and from bf16 (fused-rotation budget: at most
0.1 % of codes off by one, metadata within 2 fp16 ulp), per-token demotion
in append, the decode's q . R_K and its merge's inverse R_V (relative L2 <=
2e-3 against the oracle over the oracle's own pool bytes), for one and
several query tokens and for the per-record-group merge of large grids.
Each KV head gets its own seeded R_K != R_V, so a head or tensor mix-up
changes the result."""
import numpy as np
import pytest
import torch

import oracle as orc
from bit_rotated_kv_demote_amd import binding, synth
from bit_rotated_kv_demote_amd.pool import bf16_tensor

from _gpu_util import Layer, code_diff_stats, i32, rel_l2, upload

pytestmark = pytest.mark.gpu

FLIP_RATE = 1e-3
TOL = 2e-3


def test_per_head_demote_from_rotated_fp32_is_bit_exact():
    batch, n_tokens, starts = 2, 90, [0, 11]
    layer = Layer(seed=1300, batch=batch, hq=8, hkv=4, max_len=64 + 11 + n_tokens + 256 + 16, per_kv_head=True)
    yk = np.zeros((batch, n_tokens, layer.hkv, 128), np.float32)
    yv = np.zeros_like(yk)
    for b in range(batch):
        src = slice(64 + starts[b], 64 + starts[b] + n_tokens)
        yk[b] = orc.rotate_fp32(synth.bf16_bits_to_f32(layer.k[b, src]), layer.r_k)
        yv[b] = orc.rotate_fp32(synth.bf16_bits_to_f32(layer.v[b, src]), layer.r_v)
    dev = layer.device_pool()
    dev.demote(i32(starts), torch.from_numpy(yk).cuda(), torch.from_numpy(yv).cuda(),
               src_kind=binding.OSCAR_SRC_F32_ROTATED)
    torch.cuda.synchronize()
    ref = orc.Pool(batch, layer.hkv, layer.num_pages, layer.page_table)
    for b in range(batch):
        ref.demote_rotated_many(b, np.arange(starts[b], starts[b] + n_tokens), yk[b], yv[b], layer.tau_k, layer.tau_v)
    got = dev.hist.cpu().numpy()
    assert np.array_equal(got, ref.hist), f"{np.count_nonzero(got != ref.hist)} bytes differ"


@pytest.mark.parametrize("code_bits", [2, 4])
def test_per_head_prefill_and_append_within_flip_budget(code_bits):
    # prefill (bulk demotion, one R per KV head staged per workgroup slice),
    # then appends that demote one token per step (per-token rotation)
    lengths, n_app = [700, 333, 1000], 40
    layer = Layer(seed=1301, batch=3, hq=16, hkv=8, max_len=max(lengths) + n_app, per_kv_head=True,
                  code_bits=code_bits)
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
        h = np.arange(n - 320)
        pages.append(layer.page_table[b, h // 16])
        sl.append(h % 16)
    rate, maxd, meta_ulp = code_diff_stats(st["hist"], ref.hist, np.concatenate(pages), np.concatenate(sl))
    assert rate <= FLIP_RATE and maxd <= 1 and meta_ulp <= 2, (rate, maxd, meta_ulp)


@pytest.mark.parametrize("n_query,code_bits", [(1, 2), (4, 2), (1, 4), (4, 4)])
def test_per_head_decode_matches_oracle(n_query, code_bits):
    lengths = [1500, 420]
    layer = Layer(seed=1310 + n_query, batch=2, hq=8, hkv=2, max_len=max(lengths), per_kv_head=True,
                  code_bits=code_bits)
    opool = layer.oracle_pool(lengths)
    dev = layer.device_pool()
    upload(dev, opool)
    q = synth.queries(np.random.default_rng(20 + n_query), (2, n_query, 8, 128))
    out = dev.decode_multi(bf16_tensor(q), i32(lengths), max(lengths)).cpu().numpy()
    ref = orc.attend_tail_tiered(q, opool, [0, 1], lengths, layer.r_k, layer.r_v)
    for b in range(2):
        assert rel_l2(out[b], ref[b]) <= TOL, b
    if n_query == 1:
        single = dev.decode(bf16_tensor(np.ascontiguousarray(q[:, 0])), i32(lengths), max(lengths)).cpu().numpy()
        assert np.array_equal(single, out[:, 0])


def test_per_head_large_grid_merge_per_record_group():
    # 26 sequences x 32 heads: the merge runs one workgroup per record group,
    # each loading its own KV head's R_V
    lengths = [330 + 14 * b for b in range(26)]
    layer = Layer(seed=1320, batch=26, hq=32, hkv=8, max_len=max(lengths), per_kv_head=True)
    opool = layer.oracle_pool(lengths)
    dev = layer.device_pool()
    upload(dev, opool)
    q = synth.queries(np.random.default_rng(21), (26, 1, 32, 128))
    out = dev.decode_multi(bf16_tensor(q), i32(lengths), max(lengths)).cpu().numpy()
    ref = orc.attend_tail_tiered(q, opool, list(range(26)), lengths, layer.r_k, layer.r_v)
    assert rel_l2(out, ref) <= TOL
