"""Binding of the native block manager (include/block_manager.h).

Argument marshalling only: token ids and sequence ids become host arrays, the
native manager does every step, and the metadata comes back as int32 CPU
tensors in the layouts the attention entry points read (move them to the
device with `.to(device)`). A non-OK status raises; PA_ERR_NO_BLOCKS raises
`NoFreeBlocks`, the signal to preempt a sequence and retry.
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional, Sequence

import torch

from ._lib import PA_ERR_NO_BLOCKS, PA_OK, PagedAttnError, library


class NoFreeBlocks(PagedAttnError):
    """The free list cannot supply the blocks the call needs."""


def _check(status: int, where: str) -> None:
    if status == PA_ERR_NO_BLOCKS:
        raise NoFreeBlocks(status, where)
    if status != PA_OK:
        raise PagedAttnError(status, where)


def _i32(values: Sequence[int]) -> torch.Tensor:
    return torch.as_tensor(list(values) if not isinstance(values, torch.Tensor) else values,
                           dtype=torch.int32).contiguous()


def _i64(values: Sequence[int]) -> torch.Tensor:
    if isinstance(values, torch.Tensor):
        return values.to(torch.int64).contiguous()
    return torch.as_tensor(list(values), dtype=torch.int64).contiguous()


def xxh64(data: bytes, seed: int = 0) -> int:
    """The library's XXH64 of `data` (used for the prefix-cache block hashes)."""
    buf = ctypes.create_string_buffer(data, len(data))
    return int(library().pa_xxh64(buf if data else None, len(data), ctypes.c_uint64(seed)))


class BlockManager:
    """Free list, reference counts and prefix-cache table of a pool of
    `num_blocks` blocks of `block_size` tokens, plus the per-step metadata."""

    def __init__(self, num_blocks: int, block_size: int = 256):
        self._lib = library()
        h = ctypes.c_void_p()
        _check(self._lib.pa_bm_create(num_blocks, block_size, ctypes.byref(h)), "pa_bm_create")
        self._h = h
        self.num_blocks = num_blocks
        self.block_size = block_size

    def close(self) -> None:
        if self._h:
            self._lib.pa_bm_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- pool and sequence state -------------------------------------------
    def num_free_blocks(self) -> int:
        return int(self._lib.pa_bm_num_free_blocks(self._h))

    def ref_count(self, block_id: int) -> int:
        return int(self._lib.pa_bm_ref_count(self._h, block_id))

    def seq_info(self, seq_id: int):
        """(tokens held, tokens emitted so far, blocks held)."""
        a, b, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(self._lib.pa_bm_seq_info(self._h, seq_id, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)),
               "pa_bm_seq_info")
        return a.value, b.value, c.value

    def block_table(self, seq_id: int) -> list:
        nb = self.seq_info(seq_id)[2]
        out = torch.empty(max(nb, 1), dtype=torch.int32)
        _check(self._lib.pa_bm_block_table(self._h, seq_id, out.data_ptr(), out.numel()), "pa_bm_block_table")
        return out[:nb].tolist()

    # -- lifecycle ----------------------------------------------------------
    def can_allocate(self, token_ids: Sequence[int]) -> bool:
        t = _i32(token_ids)
        ok = ctypes.c_int32()
        _check(self._lib.pa_bm_can_allocate(self._h, t.data_ptr(), t.numel(), ctypes.byref(ok)),
               "pa_bm_can_allocate")
        return bool(ok.value)

    def allocate(self, seq_id: int, token_ids: Sequence[int]) -> int:
        """Admit a prompt; returns the number of leading tokens already cached."""
        t = _i32(token_ids)
        cached = ctypes.c_int32()
        _check(self._lib.pa_bm_allocate(self._h, seq_id, t.data_ptr(), t.numel(), ctypes.byref(cached)),
               "pa_bm_allocate")
        return cached.value

    def append_token(self, seq_id: int, token_id: int) -> None:
        _check(self._lib.pa_bm_append_token(self._h, seq_id, token_id), "pa_bm_append_token")

    def append_tokens(self, seq_ids, token_ids) -> None:
        """One token for each sequence (the step's sampled tokens), all or nothing."""
        ids, toks = _i64(seq_ids), _i32(token_ids)
        if ids.numel() != toks.numel():
            raise ValueError("append_tokens: one token per sequence")
        _check(self._lib.pa_bm_append_tokens(self._h, ids.data_ptr(), toks.data_ptr(), ids.numel()),
               "pa_bm_append_tokens")

    def free(self, seq_id: int) -> None:
        _check(self._lib.pa_bm_free(self._h, seq_id), "pa_bm_free")

    # -- metadata of a step -------------------------------------------------
    def prepare_prefill(self, seq_ids: Sequence[int], max_blocks_per_seq: int,
                        max_new_tokens: Optional[Sequence[int]] = None,
                        max_total_q: Optional[int] = None) -> Dict[str, torch.Tensor]:
        ids = _i64(seq_ids)
        b = ids.numel()
        if max_total_q is None:
            max_total_q = sum(self.seq_info(int(i))[0] - self.seq_info(int(i))[1] for i in seq_ids)
        cap = max(max_total_q, 1)
        mn = None if max_new_tokens is None else _i32(max_new_tokens)
        positions = torch.empty(cap, dtype=torch.int32)
        slots = torch.empty(cap, dtype=torch.int32)
        tables = torch.empty((max(b, 1), max_blocks_per_seq), dtype=torch.int32)
        ctx = torch.empty(max(b, 1), dtype=torch.int32)
        cu = torch.empty(b + 1, dtype=torch.int32)
        tq = ctypes.c_int32()
        _check(self._lib.pa_bm_prepare_prefill(self._h, ids.data_ptr(), b, None if mn is None else mn.data_ptr(),
                                               max_blocks_per_seq, max_total_q, positions.data_ptr(),
                                               slots.data_ptr(), tables.data_ptr(), ctx.data_ptr(), cu.data_ptr(),
                                               ctypes.byref(tq)), "pa_bm_prepare_prefill")
        n = tq.value
        return {"positions": positions[:n], "slot_mapping": slots[:n], "block_tables": tables[:b],
                "context_lens": ctx[:b], "cu_seqlens": cu, "total_q": n}

    def prepare_decode(self, seq_ids: Sequence[int], max_blocks_per_seq: int,
                       out: Optional[Dict[str, torch.Tensor]] = None) -> Dict[str, torch.Tensor]:
        """Decode metadata; `out` may hold preallocated contiguous int32 CPU
        tensors (e.g. pinned) "positions", "slot_mapping", "context_lens"
        ([>= B]) and "block_tables" ([>= B, max_blocks_per_seq]) to fill."""
        ids = _i64(seq_ids)
        b = ids.numel()
        if out is not None:
            positions, slots, tables, ctx = (out["positions"], out["slot_mapping"], out["block_tables"],
                                             out["context_lens"])
            for t in (positions, slots, tables, ctx):
                if t.dtype != torch.int32 or t.is_cuda or not t.is_contiguous() or t.shape[0] < b:
                    raise ValueError("prepare_decode: out tensors must be contiguous int32 CPU tensors of >= B rows")
            if tables.dim() != 2 or tables.shape[1] != max_blocks_per_seq:
                raise ValueError("prepare_decode: out block_tables must be [>= B, max_blocks_per_seq]")
        else:
            positions = torch.empty(max(b, 1), dtype=torch.int32)
            slots = torch.empty(max(b, 1), dtype=torch.int32)
            tables = torch.empty((max(b, 1), max_blocks_per_seq), dtype=torch.int32)
            ctx = torch.empty(max(b, 1), dtype=torch.int32)
        _check(self._lib.pa_bm_prepare_decode(self._h, ids.data_ptr(), b, max_blocks_per_seq, positions.data_ptr(),
                                              slots.data_ptr(), tables.data_ptr(), ctx.data_ptr()),
               "pa_bm_prepare_decode")
        return {"positions": positions[:b], "slot_mapping": slots[:b], "block_tables": tables[:b],
                "context_lens": ctx[:b]}
