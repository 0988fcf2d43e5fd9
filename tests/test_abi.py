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
    return binding.Pool(one, one, one, one, one, one, n_slots, max_pages, 8, one, one, one, one, 2)


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


def _host_calibrate(q, k, v, hq, hkv, block=32, pct=99.0, rotation=0, per_kv_head=False, layers=False):
    import torch
    lead = (hkv,) if per_kv_head else ()
    outs = [torch.zeros(lead + (128, 128), dtype=torch.float32), torch.zeros(lead + (128, 128), dtype=torch.float32),
            torch.zeros(lead + (128,), dtype=torch.float32), torch.zeros(lead + (128,), dtype=torch.float32)]
    fn = binding.oscar_calibrate_layers if layers else binding.oscar_calibrate
    fn(binding.layer_desc(hq, hkv), torch.from_numpy(np.ascontiguousarray(q)),
       torch.from_numpy(np.ascontiguousarray(k)), torch.from_numpy(np.ascontiguousarray(v)),
       *outs, hadamard_block=block, clip_percentile=pct, rotation=rotation, per_kv_head=per_kv_head)
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


def _planted_q(n, hq, seed):
    # distinct well-separated spectra per query-head pair, so that every
    # eigenbasis is unique up to sign and the host and oracle R agree outright
    rng = np.random.default_rng(seed)
    q = np.zeros((n, hq, 128))
    for h in range(0, hq, 2):
        basis = np.linalg.qr(rng.standard_normal((128, 128)))[0]
        z = rng.standard_normal((n, 2, 128))
        q[:, h:h + 2] = (z * np.linspace(4.0, 0.5, 128)) @ basis.T
    return q.astype(np.float32)


def test_host_calibrate_per_kv_head_matches_oracle():
    _, k, v = _calib_inputs(256, 4, 2, 7)
    q = _planted_q(256, 4, 8)
    r_k, r_v, t_k, t_v = _host_calibrate(q, k, v, 4, 2, per_kv_head=True)
    o_rk, o_rv, o_tk, o_tv = orc.calibrate(q, k, v, per_kv_head=True)
    assert r_k.shape == (2, 128, 128) and t_v.shape == (2, 128)
    assert np.allclose(r_k, o_rk, atol=2e-4)
    hp = orc.hadamard_block() @ orc.bitrev_permutation()
    for j in range(2):
        # value side: same target spectrum per head (eigenvectors unique up to degeneracy)
        c_s = orc.score_covariance(q[:, 2 * j:2 * j + 2], k[:, j:j + 1], v[:, j:j + 1])
        uv = r_v[j].astype(np.float64) @ hp.T
        wv = np.sort(np.linalg.eigvalsh(c_s))[::-1]
        assert np.allclose(np.diag(uv.T @ c_s @ uv), wv, rtol=1e-5, atol=1e-9), j
        assert np.allclose(t_k[j], orc.clip_thresholds(k[:, j], r_k[j]), rtol=1e-5), j
        assert np.allclose(t_v[j], orc.clip_thresholds(v[:, j], r_v[j]), rtol=1e-5), j


def test_host_calibrate_layers_matches_oracle():
    ks, vs, qs = [], [], []
    for layer in range(3):
        _, k, v = _calib_inputs(160, 4, 2, 20 + layer)
        qs.append(_planted_q(160, 4, 30 + layer))
        ks.append(k)
        vs.append(v)
    qs, ks, vs = np.stack(qs), np.stack(ks), np.stack(vs)
    r_k, r_v, t_k, t_v = _host_calibrate(qs, ks, vs, 4, 2, layers=True)
    o_rk, o_rv, o_tk, o_tv = orc.calibrate_layers(qs, ks, vs)
    hp = orc.hadamard_block() @ orc.bitrev_permutation()
    for r, c in ((r_k, np.mean([orc.query_covariance(qs[l]) for l in range(3)], axis=0)),
                 (r_v, np.mean([orc.score_covariance(qs[l], ks[l], vs[l]) for l in range(3)], axis=0))):
        u = r.astype(np.float64) @ hp.T
        w = np.sort(np.linalg.eigvalsh(c))[::-1]
        assert np.allclose(np.diag(u.T @ c @ u), w, rtol=1e-5, atol=1e-9)
    assert np.allclose(t_k, o_tk, rtol=1e-5) and np.allclose(t_v, o_tv, rtol=1e-5)
    assert np.allclose(t_k, orc.clip_thresholds(ks, r_k), rtol=1e-5)
    # per KV head and shared across the layers at once
    p_rk, _, p_tk, _ = _host_calibrate(qs, ks, vs, 4, 2, layers=True, per_kv_head=True)
    op_rk, _, op_tk, _ = orc.calibrate_layers(qs, ks, vs, per_kv_head=True)
    assert np.allclose(p_tk, op_tk, rtol=1e-5)
    for j in range(2):
        c = np.mean([orc.query_covariance(qs[l][:, 2 * j:2 * j + 2]) for l in range(3)], axis=0)
        u = p_rk[j].astype(np.float64) @ hp.T
        assert np.allclose(np.diag(u.T @ c @ u), np.sort(np.linalg.eigvalsh(c))[::-1], rtol=1e-5, atol=1e-9), j
    # one layer through the layers entry point is oscar_calibrate
    one = _host_calibrate(qs[0], ks[0], vs[0], 4, 2)
    via = _host_calibrate(qs[:1], ks[:1], vs[:1], 4, 2, layers=True)
    for a, b in zip(one, via):
        assert np.array_equal(a, b)


def test_calibration_scope_and_pool_flag_validation(lib):
    import torch
    d = binding.layer_desc(4, 2)
    z = torch.zeros((2, 8, 4, 128), dtype=torch.float32)
    zk = torch.zeros((2, 8, 2, 128), dtype=torch.float32)
    out = [torch.zeros((2, 128, 128)), torch.zeros((2, 128, 128)), torch.zeros((2, 128)), torch.zeros((2, 128))]
    ptrs = [ctypes.c_void_p(t.data_ptr()) for t in out]
    bad = binding.CalibOpts(32, 99.0, 0, 2)
    assert lib.oscar_calibrate_layers(ctypes.byref(d), ctypes.byref(bad), 2, ctypes.c_void_p(z.data_ptr()),
                                      ctypes.c_void_p(zk.data_ptr()), ctypes.c_void_p(zk.data_ptr()), 8,
                                      *ptrs) == -1
    ok = binding.CalibOpts(32, 99.0, 0, 1)
    assert lib.oscar_calibrate_layers(ctypes.byref(d), ctypes.byref(ok), 0, ctypes.c_void_p(z.data_ptr()),
                                      ctypes.c_void_p(zk.data_ptr()), ctypes.c_void_p(zk.data_ptr()), 8,
                                      *ptrs) == -1
    pool = _null_pool()
    pool.rot_per_kv_head = 2
    good = binding.layer_desc(32, 8)
    assert lib.oscar_append(ctypes.byref(good), ctypes.byref(pool), None, 256, 256, 256, 1, None) == -1
    pool = _null_pool()
    pool.code_bits = 3                                   # only INT2 and INT4 pools
    assert lib.oscar_append(ctypes.byref(good), ctypes.byref(pool), None, 256, 256, 256, 1, None) == -2
    pool = _null_pool()
    pool.rot_per_kv_head = 2
    assert lib.oscar_append(ctypes.byref(good), ctypes.byref(pool), None, 256, 256, 256, 1, None) == -1
    assert lib.oscar_decode(ctypes.byref(good), ctypes.byref(pool), None, 256, 256, 256, 256, 1 << 30, 1, 100,
                            None) == -1


def test_step_validation_and_workspace(lib):
    d = binding.layer_desc(32, 8)
    pool = _null_pool(max_pages=4096)
    dec = binding.oscar_decode_workspace_bytes(d, 2, 32768)
    step = binding.oscar_step_workspace_bytes(d, 2, 32768)
    # the step is one decode launch plus the merge: the decode's workspace
    assert step == dec
    assert binding.oscar_step_workspace_bytes(d, 0, 32768) == 0
    # null q, too small a workspace, bad slot count: rejected before any launch
    assert lib.oscar_step(ctypes.byref(d), ctypes.byref(pool), None, 256, 256, 256, None, 256, 256, 1 << 30, 1,
                          1000, None) == -1
    assert lib.oscar_step(ctypes.byref(d), ctypes.byref(pool), None, 256, 256, 256, 256, 256, 256, 64, 1, 1000,
                          None) == -3
    assert lib.oscar_step(ctypes.byref(d), ctypes.byref(pool), None, 256, 256, 256, 256, 256, 256, 1 << 30, 2,
                          1000, None) == -1


def test_decode_phase_calls_validation(lib):
    d = binding.layer_desc(32, 8)
    pool = _null_pool(max_pages=4096)
    P = lambda fn, *a: getattr(lib, fn)(ctypes.byref(d), ctypes.byref(pool), *a)  # noqa: E731
    # partials: null q or seq_len, small workspace, short page table, batch beyond the slots
    assert P("oscar_decode_partials", None, 256, None, 256, 1 << 30, 1, 1000, None) == -1
    assert P("oscar_decode_partials", None, None, 256, 256, 1 << 30, 1, 1000, None) == -1
    assert P("oscar_decode_partials", None, 256, 256, 256, 16, 1, 1000, None) == -3
    assert P("oscar_decode_partials", None, 256, 256, 256, 1 << 30, 1, 320 + 16 * 4097, None) == -3
    assert P("oscar_decode_partials", None, 256, 256, 256, 1 << 30, 2, 1000, None) == -1
    # merge: null out or workspace, small workspace; it needs no slot map (batch 2 > 1 slot is fine to validate)
    assert P("oscar_decode_merge", 256, None, 256, 1 << 30, 1, 1000, None) == -1
    assert P("oscar_decode_merge", 256, 256, None, 1 << 30, 1, 1000, None) == -1
    assert P("oscar_decode_merge", 256, 256, 256, 16, 1, 1000, None) == -3
    bad = binding.layer_desc(32, 8)
    bad.page_size = 8
    assert lib.oscar_decode_merge(ctypes.byref(bad), ctypes.byref(pool), 256, 256, 256, 1 << 30, 1, 1000,
                                  None) == -2


def test_decode_plan_fills_two_workgroups_per_cu():
    # The split plan: at most 512 workgroups (two per compute unit), each
    # (sequence, KV head) group takes ceil(min(n, 320) / 128) tile splits and
    # as many history splits as fit, each a multiple of four pages (one wave
    # step); one record of G x 132 fp32 per split and column group.
    d = binding.layer_desc(32, 8)
    rec = 4 * 132 * 4                       # G = 4 heads, 132 floats each
    # 32K: 2029 pages -> 61 splits would need 34 pages, rounded to 36 -> 57 + 3 tile splits
    assert binding.oscar_decode_workspace_bytes(d, 1, 32769) == 8 * 60 * rec
    # 128K: 8173 pages -> 136 pages per split -> 61 + 3
    assert binding.oscar_decode_workspace_bytes(d, 1, 131073) == 8 * 64 * rec
    # batch 2 at 32K: 29 history splits of 72 pages + 3 per group
    assert binding.oscar_decode_workspace_bytes(d, 2, 32769) == 16 * 32 * rec
    # 1040 groups cannot split within 512: one history split of up to 256 pages per 1004 -> 4, + 3
    assert binding.oscar_decode_workspace_bytes(d, 130, 16384) == 1040 * 7 * rec
    # the fused step uses the same plan plus its rotated queries and lengths
    assert binding.oscar_step_workspace_bytes(d, 1, 32769) == 8 * 60 * rec
