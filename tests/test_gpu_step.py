"""GPU parity of the fused decode step (oscar_step): append of the new token,
then decode of the step's query over the grown cache, with q . R_K computed
by the append launch and read by the decode instead of R_K.

Each case is checked in two independent parts, both against the oracle:

* the device's pool bytes after its own appends against the oracle's pool
  after the same appends: BF16 tiers byte for byte, the codes of every token
  the steps demoted within the fused-path budget (<= 0.1 % of codes differ,
  by +-1; scale / zero within 2 fp16 ulp);
* every step's output against the oracle's decode over the device's own
  post-step bytes (copied back), 2e-3 relative L2.

Beside that, the step equals the device's separate oscar_append +
oscar_decode on a twin pool: identical bytes (both appends associate the
rotation's sums the same way), outputs equal up to fp32 summation order.

Cases: GQA-4 and GQA-8 shapes, ragged batch with slot indirection (some
sequences still in the sink, some in the ring, some demoting), per-KV-head
rotations, an INT4 pool, and the full-size 32K (Qwen3-4B-shaped) and 128K
(Qwen3-8B-shaped) layers in the launch configuration the benchmark times."""
import math

import numpy as np
import pytest
import torch

import oracle as orc
from bit_rotated_kv_demote_amd import synth
from bit_rotated_kv_demote_amd.pool import TieredKV, bf16_tensor

from _gpu_util import (DECODE_TOL, Layer, check_state_vs_oracle, decode_over_device_bytes, i32, rel_l2,
                       upload)

pytestmark = pytest.mark.gpu


def _run_steps(layer, lengths, steps, seq_slot=None):
    slots = list(range(layer.batch)) if seq_slot is None else list(seq_slot)
    by_slot = [0] * layer.batch
    for b, s in enumerate(slots):
        by_slot[s] = lengths[b]
    opool = layer.oracle_pool(by_slot)
    dev, twin = layer.device_pool(), layer.device_pool()
    upload(dev, opool)
    upload(twin, opool)
    slot_t = None if seq_slot is None else i32(slots)
    max_len = max(lengths) + steps
    demoted = []
    for s in range(steps):
        pos = [n + s for n in lengths]
        kn = np.ascontiguousarray(np.stack([layer.k[slots[b], pos[b]] for b in range(layer.batch)]))
        vn = np.ascontiguousarray(np.stack([layer.v[slots[b], pos[b]] for b in range(layer.batch)]))
        q = np.ascontiguousarray(layer.q[s])
        for b in range(layer.batch):
            opool.append(slots[b], kn[b], vn[b], layer.r_k, layer.r_v, layer.tau_k, layer.tau_v)
            if pos[b] >= 320:
                demoted.append((slots[b], [pos[b] - 320]))
        out = dev.step(i32(pos), bf16_tensor(kn), bf16_tensor(vn), bf16_tensor(q), max_len,
                       seq_slot=slot_t).cpu().numpy()
        twin.append(i32(pos), bf16_tensor(kn), bf16_tensor(vn), seq_slot=slot_t)
        sep = twin.decode(bf16_tensor(q), i32([p + 1 for p in pos]), max_len, seq_slot=slot_t).cpu().numpy()
        ref = decode_over_device_bytes(dev.host_state(), layer.hkv, q, slots, [p + 1 for p in pos], layer.r_k,
                                       layer.r_v)
        for b in range(layer.batch):
            assert rel_l2(out[b], ref[b]) <= DECODE_TOL, (s, b, rel_l2(out[b], ref[b]))
        assert rel_l2(out, sep) <= 1e-5, (s, rel_l2(out, sep))
    st, st2 = dev.host_state(), twin.host_state()
    check_state_vs_oracle(st, opool, demoted)
    for name in ("sink_k", "sink_v", "recent_k", "recent_v", "hist"):
        assert np.array_equal(st[name], st2[name]), name


@pytest.mark.parametrize("hq,hkv", [(8, 2), (16, 2)])
def test_step_matches_oracle_and_separate_calls(hq, hkv):
    layer = Layer(seed=1500 + hq, batch=1, hq=hq, hkv=hkv, max_len=1200, n_q=12)
    _run_steps(layer, [1180], 12)


def test_step_ragged_batch_with_slots_across_tiers():
    # lengths before the steps: in the sink, in the ring, at the first
    # demotion, and well into history
    lengths = [30, 200, 318, 900]
    layer = Layer(seed=1510, batch=4, hq=8, hkv=2, max_len=max(lengths) + 8, n_q=8)
    _run_steps(layer, lengths, 8, seq_slot=[2, 0, 3, 1])


@pytest.mark.parametrize("per_kv_head,code_bits", [(True, 2), (False, 4), (True, 4)])
def test_step_per_head_rotations_and_int4(per_kv_head, code_bits):
    layer = Layer(seed=1520 + code_bits, batch=2, hq=8, hkv=2, max_len=1000, n_q=6, per_kv_head=per_kv_head,
                  code_bits=code_bits)
    _run_steps(layer, [990, 700], 6)


def _full_size_steps(hq, hkv, n0, steps, seed, check_steps, kv_checked):
    """The benchmark's step at full size: one sequence of n0 cached tokens
    (device prefill: BF16 tiers + bulk demotion), then `steps` oscar_step
    calls, each appending one seeded token and decoding the step's query.
    The first step's demotion opens a new history page (n0 - 320 is a
    multiple of 16 here), so the steps cross a page boundary."""
    st = synth.streams(seed)
    out_ch = synth.outlier_channels(st["outliers"])
    n_tot = n0 + steps
    k = synth.kv_tokens(st["k"], st["lognormal"], n_tot, hkv, out_ch)
    v = synth.kv_tokens(st["v"], st["lognormal"], n_tot, hkv, out_ch)
    rot = synth.random_rotation(st["rot"])
    tau_k = orc.clip_thresholds(synth.bf16_bits_to_f32(k[:4096]), rot)
    tau_v = orc.clip_thresholds(synth.bf16_bits_to_f32(v[:4096]), rot)
    # the benchmark's plan: max_seq_len covers its warm-up and timed rounds
    max_len = n0 + 64
    max_pages = math.ceil((max_len - 320) / 16)
    pt = synth.page_permutation(st["perm"], max_pages)[None, :].astype(np.int32)
    dev = TieredKV(hq, hkv, 1, max_pages, max_pages, rot, rot, tau_k, tau_v, page_table=pt)
    dev.prefill(i32([n0]), bf16_tensor(k[None, :n0]), bf16_tensor(v[None, :n0]))
    q = synth.queries(st["q"], (steps, 1, hq, 128))
    g = hq // hkv
    heads = [(0, h) for h in range(hq) if h // g in kv_checked]
    idx = tuple(np.array(heads).T)
    errs = []
    for s in range(steps):
        p = n0 + s
        out = dev.step(i32([p]), bf16_tensor(k[None, p]), bf16_tensor(v[None, p]), bf16_tensor(q[s]),
                       max_len).cpu().numpy()
        if s in check_steps:
            state = dev.host_state()
            ref = decode_over_device_bytes(state, hkv, q[s], [0], [p + 1], rot, rot, heads=heads)
            err = rel_l2(out[idx], ref[idx])
            errs.append(err)
            assert err <= DECODE_TOL, (s, err)
    state = dev.host_state()
    # the oracle's pool after the same tokens: its own demotion of every
    # history token (bulk prefill and the steps' appends)
    opool = orc.Pool(1, hkv, max_pages, pt)
    opool.sink_k[0] = k[:64].transpose(1, 0, 2)
    opool.sink_v[0] = v[:64].transpose(1, 0, 2)
    pos = np.arange(n_tot - 256, n_tot)
    opool.recent_k[0][:, (pos - 64) % 256] = k[pos].transpose(1, 0, 2)
    opool.recent_v[0][:, (pos - 64) % 256] = v[pos].transpose(1, 0, 2)
    h_all = np.arange(n_tot - 320)
    opool.demote_many(0, h_all, k[64 + h_all], v[64 + h_all], rot, rot, tau_k, tau_v)
    # the steps' own demotions alone, then the whole history
    check_state_vs_oracle(state, opool, [(0, np.arange(n0 - 320, n_tot - 320))])
    check_state_vs_oracle(state, opool, [(0, h_all)])
    return errs


@pytest.mark.parametrize("hq", [32, 64])
def test_step_full_size_32k_all_kv_heads(hq):
    # Qwen3-4B-shaped (32 q / 8 KV, GQA-4) and the GQA-8 shape (64 q / 8 KV)
    # at 32768 cached tokens: every query head of every KV head is checked
    # at the first, a middle and the last of 20 steps.
    _full_size_steps(hq, 8, 32768, 20, 1600 + hq, {0, 9, 19}, set(range(8)))


def test_step_full_size_128k_four_kv_heads():
    # Qwen3-8B-shaped, 131072 cached tokens, 16 steps; four of the eight KV
    # heads (their 16 query heads) checked at the first and last step.
    _full_size_steps(32, 8, 131072, 16, 1602, {0, 15}, {0, 2, 5, 7})
