"""CPU tests of the C ABI: the library loads, exports every declared symbol,
rejects bad arguments before touching a device, and its host-side
calibration satisfies the oracle's invariants.  No GPU compute calls."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as orc
from bit_rotated_kv_demote_amd import binding, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "oscar.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(oscar_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return binding.load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(binding.EXPORTED)
    assert lib.oscar_abi_version() == binding.ABI_VERSION


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.oscar_status_string(code)
    assert lib.oscar_status_string(0) == b"ok"


def _null_pool(n_slots=1, max_pages=4):
    # Non-null dummy pointers: validation must fail on something else first.
    one = 256
    return binding.Pool(one, one, one, one, one, one, n_slots, max_pages, 8, one, one, one, one)


def test_validation_rejects_bad_shapes_without_launching(lib):
    good = binding.layer_desc(32, 8)
    pool = _null_pool()
    bad_dim = binding.layer_desc(32, 8)
    bad_dim.head_dim = 64
    assert lib.oscar_decode(ctypes.byref(bad_dim), ctypes.byref(pool), None, 256, 256, 256, 256, 1 << 30, 1, 100,
                            None) == -2
    g16 = binding.layer_desc(32, 2)
    assert lib.oscar_decode(ctypes.byref(g16), ctypes.byref(pool), None, 256, 256, 256, 256, 1 << 30, 1, 100,
                            None) == -2
    not_div = binding.layer_desc(30, 8)
    assert lib.oscar_append(ctypes.byref(not_div), ctypes.byref(pool), None, 256, 256, 256, 1, None) == -1
    # null q / out / workspace
    assert lib.oscar_decode(ctypes.byref(good), ctypes.byref(pool), None, 256, None, 256, 256, 1 << 30, 1, 100,
                            None) == -1
    # workspace too small
    assert lib.oscar_decode(ctypes.byref(good), ctypes.byref(pool), None, 256, 256, 256, 256, 16, 1, 100,
                            None) == -3
    # page table too short for the requested context
    assert lib.oscar_decode(ctypes.byref(good), ctypes.byref(pool), None, 256, 256, 256, 256, 1 << 30, 1,
                            320 + 16 * 5, None) == -3
    # batch larger than the slot count without a slot map
    assert lib.oscar_append(ctypes.byref(good), ctypes.byref(pool), None, 256, 256, 256, 2, None) == -1
    # bad source kind for demotion
    assert lib.oscar_demote(ctypes.byref(good), ctypes.byref(pool), None, 256, 256, 256, 7, 1, 4, None) == -1
    # prefill longer than the page table allows
    assert lib.oscar_prefill(ctypes.byref(good), ctypes.byref(pool), None, 256, 256, 256, 1, 320 + 16 * 5,
                             None) == -3


def test_workspace_sizes_monotone(lib):
    d = binding.layer_desc(32, 8)
    a = binding.oscar_decode_workspace_bytes(d, 1, 32768)
    b = binding.oscar_decode_workspace_bytes(d, 1, 131072)
    c = binding.oscar_decode_workspace_bytes(d, 16, 65536)
    assert 0 < a <= b and c > 0
    assert binding.oscar_decode_bf16_workspace_bytes(d, 1, 32768) > 0
    bad = binding.layer_desc(32, 8)
    bad.page_size = 32
    assert binding.oscar_decode_workspace_bytes(bad, 1, 100) == 0


def _calib_inputs(n=192, hq=4, hkv=2, seed=0):
    st = synth.streams(seed)
    out = synth.outlier_channels(st["outliers"])
    k = synth.bf16_bits_to_f32(synth.kv_tokens(st["k"], st["lognormal"], n, hkv, out))
    v = synth.bf16_bits_to_f32(synth.kv_tokens(st["v"], st["lognormal"], n, hkv, out))
    q = synth.bf16_bits_to_f32(synth.queries(st["q"], (n, hq, 128)))
    return q, k, v


def _host_calibrate(q, k, v, hq, hkv, block=32, pct=99.0, rotation=0):
    import torch
    outs = [torch.zeros((128, 128), dtype=torch.float32), torch.zeros((128, 128), dtype=torch.float32),
            torch.zeros(128, dtype=torch.float32), torch.zeros(128, dtype=torch.float32)]
    binding.oscar_calibrate(binding.layer_desc(hq, hkv), torch.from_numpy(np.ascontiguousarray(q)),
                            torch.from_numpy(np.ascontiguousarray(k)), torch.from_numpy(np.ascontiguousarray(v)),
                            *outs, hadamard_block=block, clip_percentile=pct, rotation=rotation)
    return [o.numpy() for o in outs]


def _same_subspace_rotation(r_a, r_b, tol):
    # Rotations built from eigenbases agree up to the sign of each eigenvector
    # and rotations inside degenerate eigenspaces: compare R^T C R spectra instead.
    return np.allclose(np.sort(np.abs(r_a).ravel()), np.sort(np.abs(r_b).ravel()), atol=tol)


def test_host_calibrate_matches_oracle_invariants():
    q, k, v = _calib_inputs()
    r_k, r_v, t_k, t_v = _host_calibrate(q, k, v, 4, 2)
    o_rk, o_rv, o_tk, o_tv = orc.calibrate(q, k, v)
    for r in (r_k, r_v):
        r64 = r.astype(np.float64)
        assert np.linalg.norm(r64 @ r64.T - np.eye(128)) < 1e-5
    # Same target covariances: R^T C R is block-structured identically, so
    # U^T C U (recovered as R P^T H^T) is diagonal with the oracle's spectrum.
    c_q = orc.query_covariance(q)
    hp = orc.hadamard_block() @ orc.bitrev_permutation()
    u = r_k.astype(np.float64) @ hp.T                 # U = R P^T H^T (H, P orthogonal)
    d = u.T @ c_q @ u
    w = np.sort(np.linalg.eigvalsh(c_q))[::-1]
    assert np.allclose(np.diag(d), w, rtol=1e-6, atol=1e-9)
    assert np.abs(d - np.diag(np.diag(d))).max() < 1e-6 * w[0]
    c_s = orc.score_covariance(q, k, v)
    uv = r_v.astype(np.float64) @ hp.T
    dv = uv.T @ c_s @ uv
    wv = np.sort(np.linalg.eigvalsh(c_s))[::-1]
    assert np.allclose(np.diag(dv), wv, rtol=1e-5, atol=1e-9)
    # Each column's largest entry is positive (sign rule), as in the oracle.
    for col in range(128):
        assert u[np.argmax(np.abs(u[:, col])), col] > 0
    # Clip thresholds follow from R: the oracle's percentile on the host R.
    assert np.allclose(t_k, orc.clip_thresholds(k, r_k), rtol=1e-5)
    assert np.allclose(t_v, orc.clip_thresholds(v, r_v), rtol=1e-5)
    # With a well-separated spectrum the rotations match the oracle's outright.
    gaps = np.abs(np.diff(w)) / w[0]
    if gaps.min() > 1e-3:
        assert np.allclose(r_k, o_rk, atol=1e-4)


def test_host_calibrate_planted_spectrum_matches_oracle_rotation():
    # Queries with a planted, well-separated covariance: the eigenbasis is
    # unique up to sign, so R_K must agree with the oracle element-wise.
    rng = np.random.default_rng(12)
    basis = synth.random_rotation(rng).astype(np.float64)
    scales = np.linspace(4.0, 0.5, 128)
    z = rng.standard_normal((4096, 2, 128))
    q = ((z * scales) @ basis.T).astype(np.float32)
    q, k, v = q, _calib_inputs(4096, 2, 1, 3)[1], _calib_inputs(4096, 2, 1, 4)[2]
    # keep the causal score pass small: only C_Q matters here, use few tokens for k/v
    r_k, _, _, _ = _host_calibrate(q[:512], k[:512], v[:512], 2, 1)
    o_rk = orc.composite_rotation(orc.eigenbasis(orc.query_covariance(q[:512]))).astype(np.float32)
    assert np.allclose(r_k, o_rk, atol=2e-4)


def test_host_calibrate_rejects_non_finite():
    q, k, v = _calib_inputs(16)
    q[3, 0, 5] = np.nan
    with pytest.raises(binding.OscarError) as e:
        _host_calibrate(q, k, v, 4, 2)
    assert e.value.status == -5


@pytest.mark.parametrize("rotation", ["hadamard", "identity"])
def test_host_calibrate_baselines_equal_oracle(rotation):
    q, k, v = _calib_inputs(64)
    code = {"hadamard": binding.ROT_HADAMARD, "identity": binding.ROT_IDENTITY}[rotation]
    r_k, r_v, t_k, t_v = _host_calibrate(q, k, v, 4, 2, rotation=code)
    o_rk, o_rv, o_tk, o_tv = orc.calibrate(q, k, v, rotation=rotation)
    assert np.allclose(r_k, o_rk, atol=1e-7) and np.allclose(r_v, o_rv, atol=1e-7)
    assert np.allclose(t_k, o_tk, rtol=1e-5) and np.allclose(t_v, o_tv, rtol=1e-5)


def test_host_calibrate_key_attention_target_matches_oracle():
    q, k, v = _calib_inputs()
    r_k, r_v, t_k, _ = _host_calibrate(q, k, v, 4, 2, rotation=binding.ROT_KEY_ATTN)
    _, r_v_s, _, _ = _host_calibrate(q, k, v, 4, 2, rotation=binding.ROT_SPECTRAL)
    assert np.array_equal(r_v, r_v_s)                 # the value rotation is the method's
    c = orc.key_attention_covariance(q, k)
    hp = orc.hadamard_block() @ orc.bitrev_permutation()
    u = r_k.astype(np.float64) @ hp.T
    d = u.T @ c @ u
    w = np.sort(np.linalg.eigvalsh(c))[::-1]
    assert np.allclose(np.diag(d), w, rtol=1e-5, atol=1e-7 * w[0])
    assert np.abs(d - np.diag(np.diag(d))).max() < 1e-5 * w[0]
    assert np.allclose(t_k, orc.clip_thresholds(k, r_k), rtol=1e-5)


def test_host_calibrate_rejects_unknown_rotation():
    q, k, v = _calib_inputs(16)
    with pytest.raises(binding.OscarError) as e:
        _host_calibrate(q, k, v, 4, 2, rotation=7)
    assert e.value.status == -1


def test_multi_query_validation_and_workspace(lib):
    d = binding.layer_desc(32, 8)
    pool = _null_pool(max_pages=4096)
    args = (None, 256, 256)
    # n_query outside [1, 256] or above max_seq_len: rejected before any launch
    for nq, max_len, want in ((0, 100, -1), (257, 4096, -2), (8, 4, -1)):
        assert lib.oscar_decode_multi(ctypes.byref(d), ctypes.byref(pool), *args, nq, 256, 256, 1 << 30, 1, max_len,
                                      None) == want, (nq, max_len)
    # one query is exactly the single-token decode's workspace; more queries need more records
    one = binding.oscar_decode_multi_workspace_bytes(d, 2, 1, 32768)
    assert one == binding.oscar_decode_workspace_bytes(d, 2, 32768)
    assert binding.oscar_decode_multi_workspace_bytes(d, 2, 4, 32768) > one
    assert binding.oscar_decode_multi_workspace_bytes(d, 2, 0, 32768) == 0
