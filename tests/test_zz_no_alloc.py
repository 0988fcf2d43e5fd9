"""oscar_step_noalloc (workspace in the library's static device array)
against oscar_step with a caller workspace, through the C ABI, on twin pools:
two calls in a row, the second with a smaller batch and context than the
first (the array keeps the first call's bytes, which the second must not
depend on).  Same kernels, so outputs and pool bytes must be identical; the
outputs also match the oracle's decode of the device's bytes (2e-3)."""
import ctypes

import numpy as np
import pytest
import torch

from bit_rotated_kv_demote_amd import binding
from bit_rotated_kv_demote_amd.pool import bf16_tensor

from _gpu_util import DECODE_TOL, Layer, decode_over_device_bytes, i32, rel_l2, upload

pytestmark = pytest.mark.gpu


def _one_call(layer, lengths):
    opool = layer.oracle_pool(lengths)
    dev, twin = layer.device_pool(), layer.device_pool()
    upload(dev, opool)
    upload(twin, opool)
    pos = list(lengths)
    b_n = len(lengths)
    kn = np.ascontiguousarray(np.stack([layer.k[b, pos[b]] for b in range(b_n)]))
    vn = np.ascontiguousarray(np.stack([layer.v[b, pos[b]] for b in range(b_n)]))
    q = np.ascontiguousarray(layer.q[0][:b_n])
    max_len = max(pos) + 1
    want = twin.step(i32(pos), bf16_tensor(kn), bf16_tensor(vn), bf16_tensor(q), max_len).cpu().numpy()
    out = torch.full((b_n, layer.hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    binding.oscar_step_noalloc(dev.desc, dev.pool, None, i32(pos), bf16_tensor(kn), bf16_tensor(vn),
                               bf16_tensor(q), out, b_n, max_len)
    got = out.cpu().numpy()
    assert np.array_equal(got, want)
    st, st2 = dev.host_state(), twin.host_state()
    for name in ("sink_k", "sink_v", "recent_k", "recent_v", "hist"):
        assert np.array_equal(st[name], st2[name]), name
    ref = decode_over_device_bytes(st, layer.hkv, q, list(range(b_n)), [p + 1 for p in pos], layer.r_k, layer.r_v)
    assert rel_l2(got, ref) <= DECODE_TOL


def test_noalloc_step_equals_step_twice_second_smaller():
    big = Layer(seed=1900, batch=3, hq=16, hkv=4, max_len=6000, n_q=1)
    _one_call(big, [5990, 3000, 700])
    small = Layer(seed=1901, batch=1, hq=8, hkv=2, max_len=1300, n_q=1)
    _one_call(small, [1250])


def test_noalloc_rejects_workspace_beyond_its_array():
    lib = binding.load()
    desc = binding.layer_desc(32, 8)
    need = binding.oscar_step_workspace_bytes(desc, 512, 131072)
    assert need > binding.NOALLOC_SCRATCH_BYTES
    one = 256
    pool = binding.Pool(one, one, one, one, one, one, 512, 8192, 8192 * 512, one, one, one, one, 2, 0)
    st = lib.oscar_step_noalloc(ctypes.byref(desc), ctypes.byref(pool), None, one, one, one, one, one, 512, 131072,
                                None)
    assert st == -3
