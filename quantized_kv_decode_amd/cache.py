"""Tensor-level convenience over the C ABI: PyTorch allocates the arena and supplies the
stream; every call marshals tensors to device pointers and calls the library."""
from __future__ import annotations

import numpy as np
import torch

from . import loopkv as L


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


class LoopKVCache:
    """One plan over one arena. `plan` is uint8 [num_loops, num_layers]."""

    def __init__(self, shape: L.Shape, plan, device="cuda", stream=None, arena: torch.Tensor | None = None,
                 zero_arena: bool = False):
        self.shape = shape
        self.plan = np.asarray(plan, dtype=np.uint8).reshape(shape.num_loops, shape.num_layers)
        self.bytes = L.loopkv_cache_bytes(shape, self.plan)
        nbytes = int(self.bytes.arena_bytes)
        if arena is None:
            arena = (torch.zeros if zero_arena else torch.empty)(nbytes, dtype=torch.uint8, device=device)
        assert arena.numel() >= nbytes and arena.data_ptr() % 256 == 0
        self.arena = arena
        self.handle = L.loopkv_plan_load(shape, self.plan, arena.data_ptr(), arena.numel(), _stream(stream))

    def close(self):
        if self.handle:
            L.loopkv_plan_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---------------------------------------------------------------- calls
    def append(self, layer: int, loop: int, k_new: torch.Tensor, v_new: torch.Tensor,
               seq_lens: torch.Tensor, page_table: torch.Tensor, n_new: torch.Tensor | None = None,
               stream=None) -> None:
        """k_new, v_new: bf16 [B, n_new, H, D]; seq_lens: int32 [B] before the append;
        n_new: optional int32 [B] tokens per request (the first rows of each)."""
        assert k_new.dtype == torch.bfloat16 and v_new.dtype == torch.bfloat16
        assert k_new.is_contiguous() and v_new.is_contiguous() and k_new.shape == v_new.shape
        assert seq_lens.dtype == torch.int32 and page_table.dtype == torch.int32
        B = k_new.shape[0]
        if n_new is not None:
            assert n_new.dtype == torch.int32
        L.loopkv_quantize_append(self.handle, layer, loop, _ptr(k_new), _ptr(v_new), B, k_new.shape[1],
                                 _ptr(n_new), _ptr(seq_lens), _ptr(page_table), page_table.stride(0),
                                 _stream(stream))

    def decode(self, layer: int, loop: int, q: torch.Tensor, seq_lens: torch.Tensor,
               page_table: torch.Tensor, *, tau: float = 0.0, sm_scale: float = 0.0,
               split_tokens: int = 0, seed: torch.Tensor | None = None,
               fetch_mask: torch.Tensor | None = None, stats: torch.Tensor | None = None,
               out: torch.Tensor | None = None, sink_seed: bool = True, stream=None,
               static_workspace: bool = False) -> torch.Tensor:
        """q: bf16 [B, H, D]; seq_lens: int32 [B] including the new token. Returns fp32 [B, H, D].
        static_workspace: call loopkv_decode_attention_static (split workspace in the library's
        fixed per-GPU array) instead of loopkv_decode_attention."""
        assert q.dtype == torch.bfloat16 and q.is_contiguous()
        B = q.shape[0]
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        opts = L.DecodeOpts(float(tau), float(sm_scale), int(split_tokens),
                            int(fetch_mask.stride(1)) if fetch_mask is not None else 0,
                            _ptr(seed), _ptr(fetch_mask), _ptr(stats), 0 if sink_seed else 1)
        if fetch_mask is not None:
            assert fetch_mask.dtype == torch.uint8 and fetch_mask.stride(2) == 1
            assert fetch_mask.stride(0) == fetch_mask.stride(1) * q.shape[1]
        fn = L.loopkv_decode_attention_static if static_workspace else L.loopkv_decode_attention
        fn(self.handle, layer, loop, _ptr(q), B, _ptr(seq_lens), _ptr(page_table), page_table.stride(0),
           opts, _ptr(out), _stream(stream))
        return out

    def auto_split(self, batch: int, page_table: torch.Tensor) -> int:
        """The split_tokens that split_tokens=L.SPLIT_AUTO resolves to for this batch and table."""
        return L.loopkv_auto_split(self.handle, batch, page_table.stride(0))

    def cell_info(self, layer: int, loop: int) -> L.CellInfo:
        return L.loopkv_get_cell_info(self.handle, layer, loop)

    def device_errors(self, stream=None) -> int:
        return L.loopkv_device_errors(self.handle, _stream(stream))

    def own_pool(self, layer: int, loop: int) -> torch.Tensor:
        """A uint8 view [num_pages, page_bytes] of the pool cell (layer, loop) writes."""
        info = self.cell_info(layer, loop)
        assert info.own_pool_dev, "a REUSE cell has no pool of its own"
        off = info.own_pool_dev - self.arena.data_ptr()
        n = int(self.shape.num_pages) * int(info.page_bytes)
        return self.arena[off:off + n].view(int(self.shape.num_pages), int(info.page_bytes))

    def tail(self, layer: int, loop: int) -> tuple[torch.Tensor, torch.Tensor]:
        """bf16 views [max_batch, tail_tokens, H, D] of the cell's exact rings (K, V)."""
        info = self.cell_info(layer, loop)
        s = self.shape
        n = s.max_batch * s.tail_tokens * s.num_kv_heads * s.head_dim * 2
        views = []
        for p in (info.tail_k_dev, info.tail_v_dev):
            off = p - self.arena.data_ptr()
            views.append(self.arena[off:off + n].view(torch.bfloat16).view(
                s.max_batch, s.tail_tokens, s.num_kv_heads, s.head_dim))
        return views[0], views[1]

    def sink(self, layer: int, loop: int) -> tuple[torch.Tensor, torch.Tensor]:
        """bf16 views [max_batch, sink_tokens, H, D] of the cell's exact sink (K, V)."""
        info = self.cell_info(layer, loop)
        s = self.shape
        assert s.sink_tokens > 0 and info.sink_k_dev
        n = s.max_batch * s.sink_tokens * s.num_kv_heads * s.head_dim * 2
        views = []
        for p in (info.sink_k_dev, info.sink_v_dev):
            off = p - self.arena.data_ptr()
            views.append(self.arena[off:off + n].view(torch.bfloat16).view(
                s.max_batch, s.sink_tokens, s.num_kv_heads, s.head_dim))
        return views[0], views[1]

    def qgroups(self, layer: int, loop: int) -> torch.Tensor:
        info = self.cell_info(layer, loop)
        off = info.qgroups_dev - self.arena.data_ptr()
        return self.arena[off:off + 4 * self.shape.max_batch].view(torch.int32)
