"""Binding of the decode-step graphs (pa_decode_graphs_* in
include/paged_attn.h): one HIP graph per batch bucket of the step's KV store
followed by paged decode, replayed with one launch per step.

Argument marshalling only: the static tensors become device pointers and
torch's current stream becomes the launch stream; capture, bucket choice,
padding and replay all happen in the library.
"""
from __future__ import annotations

import ctypes
from typing import Dict

import torch

from ._lib import PA_OK, PagedAttnError, _dev_tensor, _dtype_code, _stream, library


class _Buffers(ctypes.Structure):
    _fields_ = [
        ("out", ctypes.c_void_p),
        ("q", ctypes.c_void_p),
        ("k_new", ctypes.c_void_p),
        ("v_new", ctypes.c_void_p),
        ("slot_mapping", ctypes.c_void_p),
        ("block_tables", ctypes.c_void_p),
        ("context_lens", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class DecodeGraphs:
    """Decode-step graphs over static buffers.

    `bufs` holds device tensors, rows for max_batch sequences: "out", "q"
    ([B, Hq, D]), "k_new", "v_new" ([B, Hkv, D]), "slot_mapping",
    "context_lens" ([B] int32), "block_tables" ([B, max_blocks] int32),
    "k_cache", "v_cache" (the pools) and "workspace" (uint8, zero-filled,
    at least decode_workspace_bytes(max_batch, Hq, D, max_blocks * 256)).
    Fill the first n rows, then call launch(n)."""

    def __init__(self, bufs: Dict[str, torch.Tensor], scale: float):
        self._lib = library()
        self._h = ctypes.c_void_p()
        kc = bufs["k_cache"]
        for name in ("out", "q", "k_new", "v_new", "k_cache", "v_cache"):
            _dev_tensor(bufs[name], name, kc.dtype)
        for name in ("slot_mapping", "context_lens", "block_tables"):
            _dev_tensor(bufs[name], name, torch.int32)
        if bufs.get("workspace") is not None:
            _dev_tensor(bufs["workspace"], "workspace")
        nb, bs, hkv, d = kc.shape
        max_batch, hq, _ = bufs["q"].shape
        if (bufs["out"].shape != bufs["q"].shape or bufs["q"].shape[2] != d or bufs["v_cache"].shape != kc.shape
                or bufs["k_new"].shape != (max_batch, hkv, d) or bufs["v_new"].shape != (max_batch, hkv, d)
                or bufs["slot_mapping"].shape != (max_batch,) or bufs["context_lens"].shape != (max_batch,)
                or bufs["block_tables"].dim() != 2 or bufs["block_tables"].shape[0] != max_batch):
            raise ValueError("DecodeGraphs: buffer shapes do not match q [B, Hq, D] and the pools")
        self.bufs = bufs  # keeps the tensors alive as long as the graphs
        ws = bufs.get("workspace")
        b = _Buffers(bufs["out"].data_ptr(), bufs["q"].data_ptr(), bufs["k_new"].data_ptr(),
                     bufs["v_new"].data_ptr(), bufs["slot_mapping"].data_ptr(), bufs["block_tables"].data_ptr(),
                     bufs["context_lens"].data_ptr(), kc.data_ptr(), bufs["v_cache"].data_ptr(),
                     None if ws is None else ws.data_ptr(), 0 if ws is None else ws.numel() * ws.element_size())
        h = ctypes.c_void_p()
        st = self._lib.pa_decode_graphs_create(ctypes.addressof(b), max_batch, hq, hkv, d, bs, nb,
                                               bufs["block_tables"].shape[1], float(scale), _dtype_code(kc),
                                               ctypes.addressof(h))
        if st != PA_OK:
            raise PagedAttnError(st, "pa_decode_graphs_create")
        self._h = h
        self.max_batch = max_batch

    def bucket(self, num_seqs: int) -> int:
        return int(self._lib.pa_decode_graphs_bucket(self._h, num_seqs))

    def launch(self, num_seqs: int) -> None:
        st = self._lib.pa_decode_graphs_launch(self._h, num_seqs, _stream(self.bufs["q"]))
        if st != PA_OK:
            raise PagedAttnError(st, "pa_decode_graphs_launch")

    def close(self) -> None:
        if self._h:
            self._lib.pa_decode_graphs_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
