"""Device-side tiered KV pool: torch allocations plus calls into the library.

Plumbing only -- this module owns no arithmetic of the method; every step
(append, demotion, decode) is a call into libamdoscar.so through ``binding``.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding

HEAD_DIM = 128


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bfloat16 bit patterns -> torch.bfloat16 tensor on `device`."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """torch.bfloat16 tensor -> uint16 bit patterns on the host."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


class TieredKV:
    """One layer's three-tier pool (BF16 sink, INT2 history, BF16 recent ring)."""

    def __init__(self, num_q_heads, num_kv_heads, n_slots, max_pages_per_seq, num_pages,
                 rot_k, rot_v, clip_k, clip_v, page_table=None, device="cuda", code_bits=2):
        self.hq, self.hkv, self.device = num_q_heads, num_kv_heads, device
        if code_bits not in (2, 4):
            raise ValueError("code_bits must be 2 (INT2 history) or 4 (INT4)")
        self.code_bits = code_bits
        f32 = dict(dtype=torch.float32, device=device)
        self.sink_k = torch.zeros((n_slots, num_kv_heads, 64, HEAD_DIM), dtype=torch.bfloat16, device=device)
        self.sink_v = torch.zeros_like(self.sink_k)
        self.recent_k = torch.zeros((n_slots, num_kv_heads, 256, HEAD_DIM), dtype=torch.bfloat16, device=device)
        self.recent_v = torch.zeros_like(self.recent_k)
        self.hist = torch.zeros((max(num_pages, 1), num_kv_heads, 1536 if code_bits == 2 else 2560),
                                dtype=torch.uint8, device=device)
        if page_table is None:
            page_table = np.arange(n_slots * max_pages_per_seq, dtype=np.int32).reshape(n_slots, max_pages_per_seq)
        self.page_table = torch.as_tensor(np.asarray(page_table, np.int32), device=device).contiguous()
        self.rot_k = torch.as_tensor(np.asarray(rot_k, np.float32), **f32).contiguous()
        self.rot_v = torch.as_tensor(np.asarray(rot_v, np.float32), **f32).contiguous()
        self.clip_k = torch.as_tensor(np.asarray(clip_k, np.float32), **f32).contiguous()
        self.clip_v = torch.as_tensor(np.asarray(clip_v, np.float32), **f32).contiguous()
        # one R and tau per layer ([128, 128] / [128]) or per KV head ([Hkv, 128, 128] / [Hkv, 128])
        self.per_kv_head = self.rot_k.dim() == 3
        want_r = (num_kv_heads, HEAD_DIM, HEAD_DIM) if self.per_kv_head else (HEAD_DIM, HEAD_DIM)
        want_t = want_r[:-1]
        for t, want in ((self.rot_k, want_r), (self.rot_v, want_r), (self.clip_k, want_t), (self.clip_v, want_t)):
            if tuple(t.shape) != want:
                raise ValueError(f"rotation / clip shape {tuple(t.shape)}, expected {want}")
        self.desc = binding.layer_desc(num_q_heads, num_kv_heads)
        self.pool = binding.make_pool(self.sink_k, self.sink_v, self.recent_k, self.recent_v, self.hist,
                                      self.page_table, self.rot_k, self.rot_v, self.clip_k, self.clip_v,
                                      self.per_kv_head, code_bits)
        self._ws = None
        self._step_ws = None

    # -- hot path --------------------------------------------------------
    def append(self, position, k_new, v_new, seq_slot=None):
        binding.oscar_append(self.desc, self.pool, seq_slot, position, k_new, v_new, k_new.shape[0])

    def demote(self, hist_start, k, v, src_kind=binding.OSCAR_SRC_BF16, seq_slot=None):
        binding.oscar_demote(self.desc, self.pool, seq_slot, hist_start, k, v, src_kind, k.shape[0], k.shape[1])

    def prefill(self, length, k, v, seq_slot=None):
        binding.oscar_prefill(self.desc, self.pool, seq_slot, length, k, v, k.shape[0], k.shape[1])

    def workspace(self, batch, max_seq_len):
        nbytes = binding.oscar_decode_workspace_bytes(self.desc, batch, max_seq_len)
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.zeros(((nbytes + 255) // 256) * 256, dtype=torch.uint8, device=self.device)
        return self._ws

    def decode(self, q, seq_len, max_seq_len, out=None, seq_slot=None):
        batch = q.shape[0]
        if out is None:
            out = torch.empty((batch, self.hq, HEAD_DIM), dtype=torch.float32, device=self.device)
        ws = self.workspace(batch, max_seq_len)
        binding.oscar_decode(self.desc, self.pool, seq_slot, seq_len, q, out, ws, batch, max_seq_len)
        return out

    def decode_partials(self, q, seq_len, max_seq_len, seq_slot=None):
        """The split phase of decode alone: partial records into this pool's workspace."""
        batch = q.shape[0]
        ws = self.workspace(batch, max_seq_len)
        binding.oscar_decode_partials(self.desc, self.pool, seq_slot, seq_len, q, ws, batch, max_seq_len)

    def decode_merge(self, seq_len, batch, max_seq_len, out=None):
        """The merge phase of decode alone, over the records decode_partials left."""
        if out is None:
            out = torch.empty((batch, self.hq, HEAD_DIM), dtype=torch.float32, device=self.device)
        ws = self.workspace(batch, max_seq_len)
        binding.oscar_decode_merge(self.desc, self.pool, seq_len, out, ws, batch, max_seq_len)
        return out

    def step(self, position, k_new, v_new, q, max_seq_len, out=None, seq_slot=None):
        """One fused decode step: append (k_new, v_new) at position, then decode q
        over position + 1 tokens.  k_new, v_new: bf16 [B, Hkv, 128]; q: bf16 [B, Hq, 128]."""
        batch = q.shape[0]
        if out is None:
            out = torch.empty((batch, self.hq, HEAD_DIM), dtype=torch.float32, device=self.device)
        nbytes = binding.oscar_step_workspace_bytes(self.desc, batch, max_seq_len)
        if self._step_ws is None or self._step_ws.numel() < nbytes:
            self._step_ws = torch.zeros(((nbytes + 255) // 256) * 256, dtype=torch.uint8, device=self.device)
        binding.oscar_step(self.desc, self.pool, seq_slot, position, k_new, v_new, q, out, self._step_ws, batch,
                           max_seq_len)
        return out

    def decode_multi(self, q, seq_len, max_seq_len, out=None, seq_slot=None):
        """q: bf16 [B, T, Hq, 128], the queries of each sequence's last T positions."""
        batch, n_query = q.shape[0], q.shape[1]
        if out is None:
            out = torch.empty((batch, n_query, self.hq, HEAD_DIM), dtype=torch.float32, device=self.device)
        nbytes = binding.oscar_decode_multi_workspace_bytes(self.desc, batch, n_query, max_seq_len)
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.zeros(((nbytes + 255) // 256) * 256, dtype=torch.uint8, device=self.device)
        binding.oscar_decode_multi(self.desc, self.pool, seq_slot, seq_len, q, n_query, out, self._ws, batch,
                                   max_seq_len)
        return out

    # -- host copies for checking ---------------------------------------
    def host_state(self):
        return dict(sink_k=bf16_bits(self.sink_k), sink_v=bf16_bits(self.sink_v),
                    recent_k=bf16_bits(self.recent_k), recent_v=bf16_bits(self.recent_v),
                    hist=self.hist.cpu().numpy(), page_table=self.page_table.cpu().numpy())


class PagedBF16:
    """BF16 paged cache [num_pages, Hkv, 2, 16, 128] for the baseline decode."""

    def __init__(self, num_q_heads, num_kv_heads, kv_bits, page_table, device="cuda"):
        """kv_bits: bf16 bit patterns (host uint16 array) or a device bf16 tensor, used as is."""
        self.hq, self.hkv, self.device = num_q_heads, num_kv_heads, device
        self.kv = kv_bits.contiguous() if isinstance(kv_bits, torch.Tensor) else bf16_tensor(kv_bits, device)
        self.page_table = torch.as_tensor(np.asarray(page_table, np.int32), device=device).contiguous()
        self.desc = binding.layer_desc(num_q_heads, num_kv_heads)
        self.pool = binding.make_bf16_pool(self.kv, self.page_table)
        self._ws = None

    def decode(self, q, seq_len, max_seq_len, out=None, seq_slot=None):
        batch = q.shape[0]
        if out is None:
            out = torch.empty((batch, self.hq, HEAD_DIM), dtype=torch.float32, device=self.device)
        nbytes = binding.oscar_decode_bf16_workspace_bytes(self.desc, batch, max_seq_len)
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.zeros(((nbytes + 255) // 256) * 256, dtype=torch.uint8, device=self.device)
        binding.oscar_decode_bf16(self.desc, self.pool, seq_slot, seq_len, q, out, self._ws, batch, max_seq_len)
        return out

    def decode_multi(self, q, seq_len, max_seq_len, out=None, seq_slot=None):
        """q: bf16 [B, T, Hq, 128], the queries of each sequence's last T positions."""
        batch, n_query = q.shape[0], q.shape[1]
        if out is None:
            out = torch.empty((batch, n_query, self.hq, HEAD_DIM), dtype=torch.float32, device=self.device)
        nbytes = binding.oscar_decode_bf16_multi_workspace_bytes(self.desc, batch, n_query, max_seq_len)
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.zeros(((nbytes + 255) // 256) * 256, dtype=torch.uint8, device=self.device)
        binding.oscar_decode_bf16_multi(self.desc, self.pool, seq_slot, seq_len, q, n_query, out, self._ws, batch,
                                        max_seq_len)
        return out
