"""GPU parity of the demotion path (rotate -> clip -> quantise -> pack)."""
import numpy as np
import pytest
import torch

import oracle as orc
from bit_rotated_kv_demote_amd import binding, synth
from bit_rotated_kv_demote_amd.pool import bf16_bits, bf16_tensor

pytestmark = pytest.mark.gpu

from _gpu_util import Layer, code_diff_stats, i32  # noqa: E402

# fused-path budget: at most 0.1% of codes differ from the oracle, each by 1,
# scales / zeros within 2 fp16 ulp
FLIP_RATE = 1e-3


def _rotated_inputs(layer, batch, n_tokens, starts):
    yk = np.zeros((batch, n_tokens, layer.hkv, 128), np.float32)
    yv = np.zeros_like(yk)
    for b in range(batch):
        src = slice(64 + starts[b], 64 + starts[b] + n_tokens)
        yk[b] = orc.rotate_fp32(synth.bf16_bits_to_f32(layer.k[b, src]), layer.rot)
        yv[b] = orc.rotate_fp32(synth.bf16_bits_to_f32(layer.v[b, src]), layer.rot)
    # edge cases in the first tokens of sequence 0: a constant group, a group at
    # the clip bound, exact half-step ties, values far beyond the clip
    yk[0, 0, 0, :32] = np.float32(0.75)
    yk[0, 1, 0, 32:64] = layer.tau_k[32:64]
    z, s = np.float16(-1.0), np.float16(0.5)
    yk[0, 2, 0, :32] = (np.float32(z) + (np.arange(32) % 4 + 0.5).astype(np.float32) * np.float32(s)).clip(-1, 0.5)
    yk[0, 2, 0, 0], yk[0, 2, 0, 1] = np.float32(-1.0), np.float32(0.5)
    yv[0, 3, 0, 64:96] = np.float32(1e4)
    yv[0, 3, 0, 96:] = np.float32(-3e4)
    # one fp32 step either side of each half-step tie (zero -1, scale 0.5):
    # the code decision must follow the correctly rounded quotient exactly
    t = np.array([-0.75, -0.25, 0.25], np.float32)
    near = np.concatenate([np.nextafter(t, np.float32(-np.inf)), np.nextafter(t, np.float32(np.inf)), t])
    for arr, hd in ((yk, 1), (yv, 2)):
        row = np.zeros(32, np.float32)
        row[:9] = near
        row[9], row[10] = np.float32(-1.0), np.float32(0.5)
        arr[0, 4, hd, 32:64] = row
    # non-finite inputs clip to the bounds (NaN to -tau)
    yk[0, 5, 2, 7] = np.float32(np.nan)
    yk[0, 5, 2, 40] = np.float32(np.inf)
    yv[0, 5, 3, 100] = np.float32(-np.inf)
    yv[0, 6, 1, 3] = np.float32(np.nan)
    return yk, yv


def test_demote_from_rotated_fp32_is_bit_exact():
    batch, n_tokens = 3, 70
    layer = Layer(seed=11, batch=batch, hq=8, hkv=4, max_len=64 + 48 + n_tokens + 256 + 16)
    starts = [0, 5, 37]                                   # mid-page starts
    yk, yv = _rotated_inputs(layer, batch, n_tokens, starts)
    dev = layer.device_pool()
    dev.demote(i32(starts), torch.from_numpy(yk).cuda(), torch.from_numpy(yv).cuda(),
               src_kind=binding.OSCAR_SRC_F32_ROTATED)
    torch.cuda.synchronize()
    ref = orc.Pool(batch, layer.hkv, layer.num_pages, layer.page_table)
    for b in range(batch):
        ref.demote_rotated_many(b, np.arange(starts[b], starts[b] + n_tokens), yk[b], yv[b], layer.tau_k, layer.tau_v)
    got = dev.hist.cpu().numpy()
    assert np.array_equal(got, ref.hist), f"{np.count_nonzero(got != ref.hist)} bytes differ"


def test_demote_bf16_fused_rotation_within_flip_budget():
    batch, n_tokens = 2, 600
    layer = Layer(seed=12, batch=batch, hq=16, hkv=8, max_len=64 + n_tokens + 256 + 32)
    starts = [0, 9]
    k = np.ascontiguousarray(np.stack([layer.k[b, 64 + starts[b]:64 + starts[b] + n_tokens] for b in range(batch)]))
    v = np.ascontiguousarray(np.stack([layer.v[b, 64 + starts[b]:64 + starts[b] + n_tokens] for b in range(batch)]))
    dev = layer.device_pool()
    dev.demote(i32(starts), bf16_tensor(k), bf16_tensor(v))
    torch.cuda.synchronize()
    ref = orc.Pool(batch, layer.hkv, layer.num_pages, layer.page_table)
    for b in range(batch):
        ref.demote_many(b, np.arange(starts[b], starts[b] + n_tokens), k[b], v[b], layer.rot, layer.rot,
                        layer.tau_k, layer.tau_v)
    got = dev.hist.cpu().numpy()
    pages = np.concatenate([layer.page_table[b, (starts[b] + np.arange(n_tokens)) // 16] for b in range(batch)])
    slots = np.concatenate([(starts[b] + np.arange(n_tokens)) % 16 for b in range(batch)])
    rate, maxd, meta_ulp = code_diff_stats(got, ref.hist, pages, slots)
    assert rate <= FLIP_RATE and maxd <= 1 and meta_ulp <= 2, (rate, maxd, meta_ulp)
    # bytes outside the demoted tokens stay untouched (zero)
    untouched = np.ones(got.shape[0], bool)
    untouched[np.unique(pages)] = False
    assert not got[untouched].any()


def test_append_sequence_matches_oracle_state_machine():
    # Two sequences in swapped slots, appended token by token from empty
    # through several demotions; new tokens attend to nothing here.
    n_steps = 420
    layer = Layer(seed=13, batch=2, hq=4, hkv=2, max_len=n_steps)
    dev = layer.device_pool()
    slots = [1, 0]
    ref = orc.Pool(2, layer.hkv, layer.num_pages, layer.page_table)
    slot_t = i32(slots)
    for p in range(n_steps):
        kn = np.ascontiguousarray(layer.k[:, p])
        vn = np.ascontiguousarray(layer.v[:, p])
        dev.append(i32([p, p]), bf16_tensor(kn), bf16_tensor(vn), seq_slot=slot_t)
        for b in range(2):
            ref.append(slots[b], kn[b], vn[b], layer.rot, layer.rot, layer.tau_k, layer.tau_v)
    torch.cuda.synchronize()
    st = dev.host_state()
    for name in ("sink_k", "sink_v", "recent_k", "recent_v"):
        assert np.array_equal(st[name], getattr(ref, name)), name
    n_hist = n_steps - 320
    pages, sl = [], []
    for s in range(2):
        pages.append(layer.page_table[s, np.arange(n_hist) // 16])
        sl.append(np.arange(n_hist) % 16)
    rate, maxd, meta_ulp = code_diff_stats(st["hist"], ref.hist, np.concatenate(pages), np.concatenate(sl))
    assert rate <= FLIP_RATE and maxd <= 1 and meta_ulp <= 2, (rate, maxd, meta_ulp)


def test_prefill_ragged_matches_oracle():
    lengths = [50, 320, 333, 1000]
    layer = Layer(seed=14, batch=4, hq=8, hkv=2, max_len=max(lengths))
    dev = layer.device_pool()
    dev.prefill(i32(lengths), bf16_tensor(layer.k), bf16_tensor(layer.v))
    torch.cuda.synchronize()
    ref = layer.oracle_pool(lengths)
    st = dev.host_state()
    for name in ("sink_k", "sink_v", "recent_k", "recent_v"):
        assert np.array_equal(st[name], getattr(ref, name)), name
    pages, sl = [], []
    for b, n in enumerate(lengths):
        h = np.arange(max(0, n - 320))
        pages.append(layer.page_table[b, h // 16])
        sl.append(h % 16)
    rate, maxd, meta_ulp = code_diff_stats(st["hist"], ref.hist, np.concatenate(pages), np.concatenate(sl))
    assert rate <= FLIP_RATE and maxd <= 1 and meta_ulp <= 2, (rate, maxd, meta_ulp)


@pytest.mark.parametrize("code_bits", [2, 4])
def test_bulk_demotion_full_size_sampled(code_bits):
    # The bulk-demotion workload at full size, one launch: 16 sequences x
    # 4096 tokens x 8 KV heads, bf16 in, seeded mid-page starts, shuffled
    # fresh pages.  Three sequences are compared with the oracle (all heads,
    # K and V) within the fused-rotation budget; the rest of the pool is
    # untouched outside the demoted pages.
    import math
    from bit_rotated_kv_demote_amd.pool import TieredKV
    batch, chunk, hkv, hq = 16, 4096, 8, 64
    st = synth.streams(1004)
    out_ch = synth.outlier_channels(st["outliers"])
    k = synth.kv_tokens(st["k"], st["lognormal"], batch * chunk, hkv, out_ch).reshape(batch, chunk, hkv, 128)
    v = synth.kv_tokens(st["v"], st["lognormal"], batch * chunk, hkv, out_ch).reshape(batch, chunk, hkv, 128)
    rot = synth.random_rotation(st["rot"])
    tau_k = orc.clip_thresholds(synth.bf16_bits_to_f32(k[0, :2048]), rot)
    tau_v = orc.clip_thresholds(synth.bf16_bits_to_f32(v[0, :2048]), rot)
    max_pages = chunk // 16 + 2
    pt = synth.page_permutation(st["perm"], batch * max_pages).reshape(batch, max_pages).astype(np.int32)
    starts = [int(x) for x in synth.ragged_lengths(st["lengths"], batch, 0, 15)]
    dev = TieredKV(hq, hkv, batch, max_pages, batch * max_pages, rot, rot, tau_k, tau_v, page_table=pt,
                   code_bits=code_bits)
    dev.demote(i32(starts), bf16_tensor(k), bf16_tensor(v))
    torch.cuda.synchronize()
    got = dev.hist.cpu().numpy()
    checked = [0, 7, 15]
    ref = orc.Pool(batch, hkv, batch * max_pages, pt, bits=code_bits)
    pages, slots = [], []
    for b in checked:
        h = starts[b] + np.arange(chunk)
        ref.demote_many(b, h, k[b], v[b], rot, rot, tau_k, tau_v)
        pages.append(pt[b, h // 16])
        slots.append(h % 16)
    rate, maxd, meta_ulp = code_diff_stats(got, ref.hist, np.concatenate(pages), np.concatenate(slots))
    assert rate <= FLIP_RATE and maxd <= 1 and meta_ulp <= 2, (rate, maxd, meta_ulp)
    used = np.zeros(got.shape[0], bool)
    for b in range(batch):
        used[pt[b, (starts[b] + np.arange(chunk)) // 16]] = True
    assert not got[~used].any()


@pytest.mark.parametrize("code_bits,batch", [(2, 16), (4, 32)])
def test_bulk_demotion_reloads_unit_metadata(code_bits, batch):
    # Long enough that the first waves of the launch take more work units than
    # one batch of lane-resident unit metadata covers (64 lanes / pages per
    # unit: 32 units of two pages for INT2, 64 one-page units for INT4), so the
    # kernel reloads it mid-loop: 16 (INT2) or 32 (INT4) sequences x 16384
    # tokens x 8 KV heads, 256 workgroups of 6 (INT2) or 8 (INT4) waves per
    # tensor.  The units past the reload are the last ones of the index space;
    # the last sequence holds some of them and is compared with the oracle in
    # full (all heads, K and V), with sequence 0 beside it.  Every sequence
    # demotes the same tokens (with its own start slot and pages).
    import math
    from bit_rotated_kv_demote_amd.pool import TieredKV
    chunk, hkv, hq = 16384, 8, 64
    pages_per_unit, meta_units, tensor_waves = (2, 32, 6) if code_bits == 2 else (1, 64, 8)
    ups = math.ceil((15 + chunk) / (16 * pages_per_unit))
    units, waves = batch * hkv * ups, 256 * tensor_waves
    first_reloaded = meta_units * waves               # lowest unit index taken after a reload
    assert first_reloaded < units                     # some waves run past one metadata batch
    assert first_reloaded // (hkv * ups) <= batch - 1 < units // (hkv * ups)
    st = synth.streams(1005)
    out_ch = synth.outlier_channels(st["outliers"])
    k1 = synth.kv_tokens(st["k"], st["lognormal"], chunk, hkv, out_ch)
    v1 = synth.kv_tokens(st["v"], st["lognormal"], chunk, hkv, out_ch)
    rot = synth.random_rotation(st["rot"])
    tau_k = orc.clip_thresholds(synth.bf16_bits_to_f32(k1[:2048]), rot)
    tau_v = orc.clip_thresholds(synth.bf16_bits_to_f32(v1[:2048]), rot)
    max_pages = chunk // 16 + 2
    pt = synth.page_permutation(st["perm"], batch * max_pages).reshape(batch, max_pages).astype(np.int32)
    starts = [int(x) for x in synth.ragged_lengths(st["lengths"], batch, 0, 15)]
    dev = TieredKV(hq, hkv, batch, max_pages, batch * max_pages, rot, rot, tau_k, tau_v, page_table=pt,
                   code_bits=code_bits)
    kd = bf16_tensor(k1)[None].expand(batch, -1, -1, -1).contiguous()
    vd = bf16_tensor(v1)[None].expand(batch, -1, -1, -1).contiguous()
    dev.demote(i32(starts), kd, vd)
    torch.cuda.synchronize()
    del kd, vd
    got = dev.hist.cpu().numpy()
    ref = orc.Pool(batch, hkv, batch * max_pages, pt, bits=code_bits)
    pages, slots = [], []
    for b in (0, batch - 1):
        h = starts[b] + np.arange(chunk)
        ref.demote_many(b, h, k1, v1, rot, rot, tau_k, tau_v)
        pages.append(pt[b, h // 16])
        slots.append(h % 16)
    rate, maxd, meta_ulp = code_diff_stats(got, ref.hist, np.concatenate(pages), np.concatenate(slots))
    assert rate <= FLIP_RATE and maxd <= 1 and meta_ulp <= 2, (rate, maxd, meta_ulp)
    used = np.zeros(got.shape[0], bool)
    for b in range(batch):
        used[pt[b, (starts[b] + np.arange(chunk)) // 16]] = True
    assert not got[~used].any()
