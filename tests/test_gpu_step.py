"""GPU parity of the fused decode step (oscar_step): append of the new token,
then decode of the step's query over the grown cache, with q . R_K computed
by the append launch and read by the decode instead of R_K.

Two checks per case: against oracle append + oracle decode over the same
steps (end-to-end bound 5e-3 relative L2, as for separate device append and
decode: the fused rotation's rare code flips differ between the pools), and
against the device's own separate oscar_append + oscar_decode on a twin
pool (identical appended bytes; outputs equal up to fp32 summation order,
1e-5).  Cases: GQA-4 and GQA-8 shapes, ragged batch with slot indirection
(some sequences still in the sink, some in the ring, some demoting),
per-KV-head rotations, and an INT4 pool."""
import numpy as np
import pytest
import torch

import oracle as orc
from bit_rotated_kv_demote_amd import binding
from bit_rotated_kv_demote_amd.pool import bf16_tensor

from _gpu_util import Layer, i32, rel_l2, upload

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
    for s in range(steps):
        pos = [n + s for n in lengths]
        kn = np.ascontiguousarray(np.stack([layer.k[slots[b], pos[b]] for b in range(layer.batch)]))
        vn = np.ascontiguousarray(np.stack([layer.v[slots[b], pos[b]] for b in range(layer.batch)]))
        q = np.ascontiguousarray(layer.q[s])
        for b in range(layer.batch):
            opool.append(slots[b], kn[b], vn[b], layer.r_k, layer.r_v, layer.tau_k, layer.tau_v)
        out = dev.step(i32(pos), bf16_tensor(kn), bf16_tensor(vn), bf16_tensor(q), max_len,
                       seq_slot=slot_t).cpu().numpy()
        twin.append(i32(pos), bf16_tensor(kn), bf16_tensor(vn), seq_slot=slot_t)
        sep = twin.decode(bf16_tensor(q), i32([p + 1 for p in pos]), max_len, seq_slot=slot_t).cpu().numpy()
        ref = orc.decode_tiered(q, opool, slots, [p + 1 for p in pos], layer.r_k, layer.r_v)
        for b in range(layer.batch):
            assert rel_l2(out[b], ref[b]) <= 5e-3, (s, b, rel_l2(out[b], ref[b]))
        assert rel_l2(out, sep) <= 1e-5, (s, rel_l2(out, sep))
    st, st2 = dev.host_state(), twin.host_state()
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
