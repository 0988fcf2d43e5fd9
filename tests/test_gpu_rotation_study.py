"""Rotation variants end to end on the GPU: host calibration with each
rotation, device prefill (bulk demotion) and device decode over a layer with
planted covariance structure.

Per variant: the device's demotion against the oracle's demotion of the same
tokens with the same R and tau, within the fused-rotation budget (at most
0.1 % of codes off by one, scale and zero within 2 fp16 ulp); the device
decode against the oracle's decode of the device's own pool bytes
(relative L2 <= 2e-3); and the attention error of the INT2 tiers against
fp64 attention over the BF16 keys and values.  (An end-to-end bound on this
layer would be ill-conditioned: attention is nearly uniform over zero-mean
values, so the output is a small residue of large terms.)  The plain INT2
baseline (R = I) must be the worst of the four: its outlier channels set
the range of their quantisation groups, which every rotation spreads out
("OSCAR: Offline Spectral Covariance-Aware Rotation for 2-bit KV Cache
Quantization" (gist.science), sections 1 and 4)."""
import math

import numpy as np
import pytest
import torch

import oracle as orc
from bit_rotated_kv_demote_amd import binding, synth
from bit_rotated_kv_demote_amd.pool import TieredKV, bf16_tensor

from _gpu_util import code_diff_stats, i32, rel_l2

pytestmark = pytest.mark.gpu

HQ, HKV, N_CALIB, N_CTX = 8, 2, 512, 2048
ROTATIONS = {"spectral": binding.ROT_SPECTRAL, "key_attn": binding.ROT_KEY_ATTN,
             "hadamard": binding.ROT_HADAMARD, "identity": binding.ROT_IDENTITY}


def _layer():
    # calibration tokens and the decode context come from one planted layer
    # (same structure, disjoint tokens)
    q, k, v = synth.planted_layer(np.random.default_rng(2024), N_CALIB + N_CTX, HQ, HKV)
    qc, kc, vc = np.ascontiguousarray(q[:N_CALIB]), k[:N_CALIB], v[:N_CALIB]
    qt, kt, vt = q[N_CALIB:], np.ascontiguousarray(k[N_CALIB:]), np.ascontiguousarray(v[N_CALIB:])
    return qc, synth.bf16_bits_to_f32(kc), synth.bf16_bits_to_f32(vc), qt, kt, vt


def _calibrate(qc, kc, vc, rotation):
    outs = [torch.zeros((128, 128), dtype=torch.float32), torch.zeros((128, 128), dtype=torch.float32),
            torch.zeros(128, dtype=torch.float32), torch.zeros(128, dtype=torch.float32)]
    binding.oscar_calibrate(binding.layer_desc(HQ, HKV), torch.from_numpy(qc), torch.from_numpy(kc),
                            torch.from_numpy(vc), *outs, rotation=rotation)
    return [o.numpy() for o in outs]


def test_rotation_variants_parity_and_error_ordering():
    qc, kc, vc, qt, kt, vt = _layer()
    q = np.ascontiguousarray(synth.to_bf16_bits(qt[-1:]))             # one decode query per head
    qf = synth.bf16_bits_to_f32(q)[0].astype(np.float64)
    kf = synth.bf16_bits_to_f32(kt).astype(np.float64)
    vf = synth.bf16_bits_to_f32(vt).astype(np.float64)
    g = HQ // HKV
    exact = np.stack([orc.attention(qf[h:h + 1], kf[:, h // g], vf[:, h // g])[0] for h in range(HQ)])
    max_pages = math.ceil((N_CTX - 320) / 16)
    pt = synth.page_permutation(np.random.default_rng(3), max_pages)[None, :].astype(np.int32)
    errors = {}
    for name, code in ROTATIONS.items():
        r_k, r_v, t_k, t_v = _calibrate(qc, kc, vc, code)
        dev = TieredKV(HQ, HKV, 1, max_pages, max_pages, r_k, r_v, t_k, t_v, page_table=pt)
        dev.prefill(i32([N_CTX]), bf16_tensor(kt[None]), bf16_tensor(vt[None]))
        out = dev.decode(bf16_tensor(q), i32([N_CTX]), N_CTX).cpu().numpy()[0]
        # the oracle's own demotion of the same tokens with the same R and tau
        # (the history bytes are compared; the tiers' BF16 bytes are copies)
        op = orc.Pool(1, HKV, max_pages, pt)
        op.sink_k[0][:, :64] = kt[:64].transpose(1, 0, 2)
        op.sink_v[0][:, :64] = vt[:64].transpose(1, 0, 2)
        pos = np.arange(N_CTX - 256, N_CTX)
        op.recent_k[0][:, (pos - 64) % 256] = kt[pos].transpose(1, 0, 2)
        op.recent_v[0][:, (pos - 64) % 256] = vt[pos].transpose(1, 0, 2)
        h = np.arange(N_CTX - 320)
        op.demote_many(0, h, kt[64 + h], vt[64 + h], r_k, r_v, t_k, t_v)
        op.length[0] = N_CTX
        got = dev.host_state()
        rate, maxd, meta_ulp = code_diff_stats(got["hist"], op.hist, pt[0, h // 16], h % 16)
        assert rate <= 1e-3 and maxd <= 1 and meta_ulp <= 2, (name, rate, maxd, meta_ulp)
        ref = orc.decode_tiered(q, orc.Pool.from_state(got, HKV), [0], [N_CTX], r_k, r_v)[0]
        assert rel_l2(out, ref) <= 2e-3, name
        errors[name] = rel_l2(out, exact)
    assert errors["identity"] > errors["hadamard"] and errors["identity"] > errors["spectral"], errors
