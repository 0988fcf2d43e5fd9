"""Thin ctypes binding of libamdoscar.so (include/oscar.h).

Argument marshalling only: every computation happens inside the library.
Tensors are torch tensors (device memory for the device entry points, host
memory for ``oscar_calibrate``); pointers are taken with ``data_ptr()`` and the
current torch stream is passed as the HIP stream.  A non-OK status raises
``OscarError``; a missing library raises at load time -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libamdoscar.so")

OSCAR_SRC_BF16 = 0
OSCAR_SRC_F32_ROTATED = 1
ABI_VERSION = 6

EXPORTED = ("oscar_abi_version", "oscar_status_string", "oscar_calibrate", "oscar_calibrate_layers", "oscar_append", "oscar_demote",
            "oscar_prefill", "oscar_decode", "oscar_decode_workspace_bytes", "oscar_decode_partials", "oscar_decode_merge", "oscar_decode_multi",
            "oscar_decode_multi_workspace_bytes", "oscar_decode_bf16", "oscar_decode_bf16_workspace_bytes",
            "oscar_decode_bf16_multi", "oscar_decode_bf16_multi_workspace_bytes", "oscar_step",
            "oscar_step_workspace_bytes", "oscar_step_noalloc")


class OscarError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class LayerDesc(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("n_sink", ctypes.c_int32), ("n_recent", ctypes.c_int32),
                ("group_size", ctypes.c_int32)]


class Pool(ctypes.Structure):
    _fields_ = [("sink_k", ctypes.c_void_p), ("sink_v", ctypes.c_void_p), ("recent_k", ctypes.c_void_p),
                ("recent_v", ctypes.c_void_p), ("hist", ctypes.c_void_p), ("page_table", ctypes.c_void_p),
                ("n_slots", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("rot_k", ctypes.c_void_p), ("rot_v", ctypes.c_void_p), ("clip_k", ctypes.c_void_p),
                ("clip_v", ctypes.c_void_p), ("code_bits", ctypes.c_int32), ("rot_per_kv_head", ctypes.c_int32)]


class Bf16Pool(ctypes.Structure):
    _fields_ = [("kv", ctypes.c_void_p), ("page_table", ctypes.c_void_p), ("n_slots", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32)]


class CalibOpts(ctypes.Structure):
    _fields_ = [("hadamard_block", ctypes.c_int32), ("clip_percentile", ctypes.c_float), ("rotation", ctypes.c_int32),
                ("per_kv_head", ctypes.c_int32)]


# oscar_calib_opts.rotation
ROT_SPECTRAL, ROT_KEY_ATTN, ROT_HADAMARD, ROT_IDENTITY = 0, 1, 2, 3


_lib = None


def load():
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise OSError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.oscar_abi_version.restype = I32
    lib.oscar_status_string.restype = ctypes.c_char_p
    lib.oscar_status_string.argtypes = [ctypes.c_int]
    lib.oscar_calibrate.restype = ctypes.c_int
    lib.oscar_calibrate.argtypes = [P, P, P, P, P, I64, P, P, P, P]
    lib.oscar_calibrate_layers.restype = ctypes.c_int
    lib.oscar_calibrate_layers.argtypes = [P, P, I32, P, P, P, I64, P, P, P, P]
    lib.oscar_append.restype = ctypes.c_int
    lib.oscar_append.argtypes = [P, P, P, P, P, P, I32, P]
    lib.oscar_demote.restype = ctypes.c_int
    lib.oscar_demote.argtypes = [P, P, P, P, P, P, I32, I32, I32, P]
    lib.oscar_prefill.restype = ctypes.c_int
    lib.oscar_prefill.argtypes = [P, P, P, P, P, P, I32, I32, P]
    lib.oscar_decode.restype = ctypes.c_int
    lib.oscar_decode.argtypes = [P, P, P, P, P, P, P, SZ, I32, I32, P]
    lib.oscar_decode_workspace_bytes.restype = SZ
    lib.oscar_decode_workspace_bytes.argtypes = [P, I32, I32]
    lib.oscar_decode_partials.restype = ctypes.c_int
    lib.oscar_decode_partials.argtypes = [P, P, P, P, P, P, SZ, I32, I32, P]
    lib.oscar_decode_merge.restype = ctypes.c_int
    lib.oscar_decode_merge.argtypes = [P, P, P, P, P, SZ, I32, I32, P]
    lib.oscar_step.restype = ctypes.c_int
    lib.oscar_step.argtypes = [P, P, P, P, P, P, P, P, P, SZ, I32, I32, P]
    lib.oscar_step_noalloc.restype = ctypes.c_int
    lib.oscar_step_noalloc.argtypes = [P, P, P, P, P, P, P, P, I32, I32, P]
    lib.oscar_step_workspace_bytes.restype = SZ
    lib.oscar_step_workspace_bytes.argtypes = [P, I32, I32]
    lib.oscar_decode_multi.restype = ctypes.c_int
    lib.oscar_decode_multi.argtypes = [P, P, P, P, P, I32, P, P, SZ, I32, I32, P]
    lib.oscar_decode_multi_workspace_bytes.restype = SZ
    lib.oscar_decode_multi_workspace_bytes.argtypes = [P, I32, I32, I32]
    lib.oscar_decode_bf16.restype = ctypes.c_int
    lib.oscar_decode_bf16.argtypes = [P, P, P, P, P, P, P, SZ, I32, I32, P]
    lib.oscar_decode_bf16_workspace_bytes.restype = SZ
    lib.oscar_decode_bf16_workspace_bytes.argtypes = [P, I32, I32]
    lib.oscar_decode_bf16_multi.restype = ctypes.c_int
    lib.oscar_decode_bf16_multi.argtypes = [P, P, P, P, P, I32, P, P, SZ, I32, I32, P]
    lib.oscar_decode_bf16_multi_workspace_bytes.restype = SZ
    lib.oscar_decode_bf16_multi_workspace_bytes.argtypes = [P, I32, I32, I32]
    if lib.oscar_abi_version() != ABI_VERSION:
        raise OSError("libamdoscar ABI version mismatch")
    _lib = lib
    return lib


def _check(fn, status):
    if status != 0:
        msg = load().oscar_status_string(status).decode()
        raise OscarError(fn, status, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def layer_desc(num_q_heads: int, num_kv_heads: int) -> LayerDesc:
    return LayerDesc(num_q_heads, num_kv_heads, 128, 16, 64, 256, 32)


def make_pool(sink_k, sink_v, recent_k, recent_v, hist, page_table, rot_k, rot_v, clip_k, clip_v,
              rot_per_kv_head=False, code_bits=2) -> Pool:
    return Pool(sink_k.data_ptr(), sink_v.data_ptr(), recent_k.data_ptr(), recent_v.data_ptr(),
                hist.data_ptr() if hist is not None else None,
                page_table.data_ptr() if page_table is not None else None,
                sink_k.shape[0], page_table.shape[1] if page_table is not None else 0,
                hist.shape[0] if hist is not None else 0,
                rot_k.data_ptr(), rot_v.data_ptr(), clip_k.data_ptr(), clip_v.data_ptr(), int(code_bits),
                int(bool(rot_per_kv_head)))


def make_bf16_pool(kv, page_table) -> Bf16Pool:
    return Bf16Pool(kv.data_ptr(), page_table.data_ptr(), page_table.shape[0], page_table.shape[1], kv.shape[0])


def oscar_calibrate(desc, q, k, v, rot_k, rot_v, clip_k, clip_v, hadamard_block=32, clip_percentile=99.0,
                    rotation=ROT_SPECTRAL, per_kv_head=False):
    """Host tensors: q [N,Hq,128], k/v [N,Hkv,128] fp32; outputs fp32 [128,128] / [128]
    (per KV head: [Hkv,128,128] / [Hkv,128])."""
    opts = CalibOpts(hadamard_block, clip_percentile, rotation, int(bool(per_kv_head)))
    _check("oscar_calibrate", load().oscar_calibrate(ctypes.byref(desc), ctypes.byref(opts), _ptr(q), _ptr(k),
                                                      _ptr(v), q.shape[0], _ptr(rot_k), _ptr(rot_v),
                                                      _ptr(clip_k), _ptr(clip_v)))


def oscar_calibrate_layers(desc, q, k, v, rot_k, rot_v, clip_k, clip_v, hadamard_block=32, clip_percentile=99.0,
                           rotation=ROT_SPECTRAL, per_kv_head=False):
    """Host tensors: q [L,N,Hq,128], k/v [L,N,Hkv,128] fp32; one calibration shared by the L layers."""
    opts = CalibOpts(hadamard_block, clip_percentile, rotation, int(bool(per_kv_head)))
    _check("oscar_calibrate_layers",
           load().oscar_calibrate_layers(ctypes.byref(desc), ctypes.byref(opts), q.shape[0], _ptr(q), _ptr(k),
                                         _ptr(v), q.shape[1], _ptr(rot_k), _ptr(rot_v), _ptr(clip_k),
                                         _ptr(clip_v)))


def oscar_append(desc, pool, seq_slot, position, k_new, v_new, batch, stream=None):
    _check("oscar_append", load().oscar_append(ctypes.byref(desc), ctypes.byref(pool), _ptr(seq_slot),
                                                _ptr(position), _ptr(k_new), _ptr(v_new), batch, _stream(stream)))


def oscar_demote(desc, pool, seq_slot, hist_start, k, v, src_kind, batch, n_tokens, stream=None):
    _check("oscar_demote", load().oscar_demote(ctypes.byref(desc), ctypes.byref(pool), _ptr(seq_slot),
                                                _ptr(hist_start), _ptr(k), _ptr(v), src_kind, batch, n_tokens,
                                                _stream(stream)))


def oscar_prefill(desc, pool, seq_slot, length, k, v, batch, max_len, stream=None):
    _check("oscar_prefill", load().oscar_prefill(ctypes.byref(desc), ctypes.byref(pool), _ptr(seq_slot),
                                                  _ptr(length), _ptr(k), _ptr(v), batch, max_len, _stream(stream)))


def oscar_decode_workspace_bytes(desc, batch, max_seq_len) -> int:
    return int(load().oscar_decode_workspace_bytes(ctypes.byref(desc), batch, max_seq_len))


def oscar_decode(desc, pool, seq_slot, seq_len, q, out, workspace, batch, max_seq_len, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("oscar_decode", load().oscar_decode(ctypes.byref(desc), ctypes.byref(pool), _ptr(seq_slot),
                                                _ptr(seq_len), _ptr(q), _ptr(out), _ptr(workspace), ws_bytes,
                                                batch, max_seq_len, _stream(stream)))


def oscar_decode_partials(desc, pool, seq_slot, seq_len, q, workspace, batch, max_seq_len, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("oscar_decode_partials", load().oscar_decode_partials(ctypes.byref(desc), ctypes.byref(pool),
                                                                  _ptr(seq_slot), _ptr(seq_len), _ptr(q),
                                                                  _ptr(workspace), ws_bytes, batch, max_seq_len,
                                                                  _stream(stream)))


def oscar_decode_merge(desc, pool, seq_len, out, workspace, batch, max_seq_len, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("oscar_decode_merge", load().oscar_decode_merge(ctypes.byref(desc), ctypes.byref(pool), _ptr(seq_len),
                                                            _ptr(out), _ptr(workspace), ws_bytes, batch,
                                                            max_seq_len, _stream(stream)))


def oscar_step_workspace_bytes(desc, batch, max_seq_len) -> int:
    return int(load().oscar_step_workspace_bytes(ctypes.byref(desc), batch, max_seq_len))


def oscar_step(desc, pool, seq_slot, position, k_new, v_new, q, out, workspace, batch, max_seq_len, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("oscar_step", load().oscar_step(ctypes.byref(desc), ctypes.byref(pool), _ptr(seq_slot), _ptr(position),
                                            _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out), _ptr(workspace), ws_bytes,
                                            batch, max_seq_len, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 8 << 20


def oscar_step_noalloc(desc, pool, seq_slot, position, k_new, v_new, q, out, batch, max_seq_len, stream=None):
    _check("oscar_step_noalloc", load().oscar_step_noalloc(ctypes.byref(desc), ctypes.byref(pool), _ptr(seq_slot),
                                                            _ptr(position), _ptr(k_new), _ptr(v_new), _ptr(q),
                                                            _ptr(out), batch, max_seq_len, _stream(stream)))


def oscar_decode_multi_workspace_bytes(desc, batch, n_query, max_seq_len) -> int:
    return int(load().oscar_decode_multi_workspace_bytes(ctypes.byref(desc), batch, n_query, max_seq_len))


def oscar_decode_multi(desc, pool, seq_slot, seq_len, q, n_query, out, workspace, batch, max_seq_len, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("oscar_decode_multi", load().oscar_decode_multi(ctypes.byref(desc), ctypes.byref(pool), _ptr(seq_slot),
                                                            _ptr(seq_len), _ptr(q), n_query, _ptr(out),
                                                            _ptr(workspace), ws_bytes, batch, max_seq_len,
                                                            _stream(stream)))


def oscar_decode_bf16_workspace_bytes(desc, batch, max_seq_len) -> int:
    return int(load().oscar_decode_bf16_workspace_bytes(ctypes.byref(desc), batch, max_seq_len))


def oscar_decode_bf16(desc, pool, seq_slot, seq_len, q, out, workspace, batch, max_seq_len, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("oscar_decode_bf16", load().oscar_decode_bf16(ctypes.byref(desc), ctypes.byref(pool), _ptr(seq_slot),
                                                          _ptr(seq_len), _ptr(q), _ptr(out), _ptr(workspace),
                                                          ws_bytes, batch, max_seq_len, _stream(stream)))


def oscar_decode_bf16_multi_workspace_bytes(desc, batch, n_query, max_seq_len) -> int:
    return int(load().oscar_decode_bf16_multi_workspace_bytes(ctypes.byref(desc), batch, n_query, max_seq_len))


def oscar_decode_bf16_multi(desc, pool, seq_slot, seq_len, q, n_query, out, workspace, batch, max_seq_len,
                            stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("oscar_decode_bf16_multi",
           load().oscar_decode_bf16_multi(ctypes.byref(desc), ctypes.byref(pool), _ptr(seq_slot), _ptr(seq_len),
                                          _ptr(q), n_query, _ptr(out), _ptr(workspace), ws_bytes, batch,
                                          max_seq_len, _stream(stream)))
