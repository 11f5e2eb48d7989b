"""ctypes binding of libpagedattn.so (include/paged_attn.h).

Argument marshalling only: tensors become device pointers, torch's current
HIP stream becomes the stream argument, and a non-OK status becomes an
exception. Every step of the computation runs in the library's kernels; there
is no fallback of any kind. Loading fails loudly if the library is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpagedattn.so")

PA_OK = 0
PA_ERR_INVALID_ARG = -1
PA_ERR_UNSUPPORTED = -2
PA_ERR_WORKSPACE = -3
PA_ERR_HIP = -4
PA_ERR_NO_BLOCKS = -5

PA_F32 = 0
PA_BF16 = 1

_DTYPES = {torch.float32: PA_F32, torch.bfloat16: PA_BF16}

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_f32 = ctypes.c_float

# name -> (restype, argtypes), mirroring include/paged_attn.h
SIGNATURES = {
    "pa_version": (ctypes.c_char_p, []),
    "pa_status_string": (ctypes.c_char_p, [_i32]),
    "pa_kv_store": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pa_rope_kv_store": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                _i32, _vp]),
    "pa_qknorm_rope_kv_store": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _i32, _i32, _i32, _i32,
                                       _i32, _i32, _f32, _i32, _vp]),
    "pa_paged_attn_decode": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                    _f32, _i32, _vp, _sz, _vp]),
    "pa_paged_attn_decode_ex": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                       _i32, _f32, _i32, _i32, _vp, _sz, _vp]),
    "pa_paged_attn_decode_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                            _i32, _f32, _i32, _vp]),
    "pa_decode_noalloc_scratch_bytes": (_sz, []),
    "pa_paged_attn_decode_store": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                          _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp]),
    "pa_decode_num_workgroups": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "pa_paged_attn_prefill": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                     _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp]),
    "pa_paged_attn_prefill_ex": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                        _i32, _i32, _i32, _i32, _i32, _f32, _i32, _i32, _vp, _sz, _vp]),
    "pa_prefill_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "pa_workspace_status": (_i32, [_vp, _sz, _vp]),
    "pa_kv_store_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _f32, _vp]),
    "pa_decode_fp8_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "pa_paged_attn_decode_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                        _i32, _f32, _f32, _f32, _vp, _sz, _vp]),
    # decode-step graphs (the buffer struct and the handle are passed by address)
    "pa_decode_graphs_create": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp]),
    "pa_decode_graphs_launch": (_i32, [_vp, _i32, _vp]),
    "pa_decode_graphs_bucket": (_i32, [_vp, _i32]),
    "pa_decode_graphs_destroy": (None, [_vp]),
    # host-side block manager (include/block_manager.h)
    "pa_xxh64": (ctypes.c_uint64, [_vp, _sz, ctypes.c_uint64]),
    "pa_bm_create": (_i32, [_i32, _i32, _vp]),
    "pa_bm_destroy": (None, [_vp]),
    "pa_bm_num_free_blocks": (_i32, [_vp]),
    "pa_bm_ref_count": (_i32, [_vp, _i32]),
    "pa_bm_allocate": (_i32, [_vp, _i64, _vp, _i32, _vp]),
    "pa_bm_can_allocate": (_i32, [_vp, _vp, _i32, _vp]),
    "pa_bm_append_token": (_i32, [_vp, _i64, _i32]),
    "pa_bm_append_tokens": (_i32, [_vp, _vp, _vp, _i32]),
    "pa_bm_free": (_i32, [_vp, _i64]),
    "pa_bm_seq_info": (_i32, [_vp, _i64, _vp, _vp, _vp]),
    "pa_bm_block_table": (_i32, [_vp, _i64, _vp, _i32]),
    "pa_bm_prepare_prefill": (_i32, [_vp, _vp, _i32, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "pa_bm_prepare_decode": (_i32, [_vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp]),
}

_lib: Optional[ctypes.CDLL] = None


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = library().pa_status_string(status).decode()
        super().__init__(f"{where}: {msg} ({status})")


def library() -> ctypes.CDLL:
    """Load libpagedattn.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_209_amd.build` "
                               "(or __graft_entry__.build())")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def version() -> str:
    return library().pa_version().decode()


def _check(status: int, where: str) -> None:
    if status != PA_OK:
        raise PagedAttnError(status, where)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev_tensor(t: torch.Tensor, name: str, dtype=None) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {t.dtype}") from None


# ---------------------------------------------------------------------------
# workspace: zero-filled once per device, reused (the kernels tag their piece
# counters per call, so nothing is cleared between calls)
# ---------------------------------------------------------------------------

_workspaces = {}


def workspace(device: torch.device, nbytes: int, kind: str = "decode", stream: Optional[int] = None
              ) -> Optional[torch.Tensor]:
    """Zero-filled scratch for one entry point kind ("decode", "decode_fp8"
    or "prefill") on one device and stream. The kinds lay their counters out
    differently, so they never share a buffer; calls on different streams may
    run at the same time, so each stream gets its own (the library's rule: one
    workspace per stream of calls)."""
    if nbytes == 0:
        return None
    key = (device.type, device.index, kind, stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def check_workspace(ws: Optional[torch.Tensor]) -> None:
    """pa_workspace_status: wait for the work queued on the current stream and
    raise PagedAttnError(PA_ERR_WORKSPACE) if a call on `ws` met piece
    counters it could not reuse (a workspace that was not zero-filled before
    its first use; the affected output rows hold NaN). Clears the error word.
    A diagnostic: it synchronises the stream."""
    if ws is None:
        return
    _check(library().pa_workspace_status(_ptr(ws), ws.numel() * ws.element_size(), _stream(ws)),
           "pa_workspace_status")


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------


def kv_store(k_cache: torch.Tensor, v_cache: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
             slot_mapping: torch.Tensor) -> None:
    """pa_kv_store: write k/v rows into the pools at slot_mapping (in place)."""
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache), ("k", k), ("v", v)):
        _dev_tensor(t, name, k_cache.dtype)
    _dev_tensor(slot_mapping, "slot_mapping", torch.int32)
    nb, bs, hkv, d = k_cache.shape
    _check(library().pa_kv_store(_ptr(k_cache), _ptr(v_cache), _ptr(k), _ptr(v), _ptr(slot_mapping), k.shape[0],
                                 hkv, d, bs, nb, _dtype_code(k_cache), _stream(k_cache)), "pa_kv_store")


def rope_kv_store(q_out: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, q: torch.Tensor,
                  k: torch.Tensor, v: torch.Tensor, positions: torch.Tensor, slot_mapping: torch.Tensor,
                  rope_theta: float) -> None:
    """pa_rope_kv_store: q_out = q rotated by positions (q_out may be q), and the
    rotated k with the plain v written into the pools at slot_mapping."""
    for name, t in (("q_out", q_out), ("k_cache", k_cache), ("v_cache", v_cache), ("q", q), ("k", k), ("v", v)):
        _dev_tensor(t, name, k_cache.dtype)
    _dev_tensor(positions, "positions", torch.int32)
    _dev_tensor(slot_mapping, "slot_mapping", torch.int32)
    nb, bs, hkv, d = k_cache.shape
    if q.dim() != 3 or q.shape[2] != d or q_out.shape != q.shape or k.shape != (q.shape[0], hkv, d) or v.shape != k.shape:
        raise ValueError("rope_kv_store: q/q_out [T, Hq, D], k/v [T, Hkv, D] expected")
    if positions.shape != (q.shape[0],) or slot_mapping.shape != (q.shape[0],):
        raise ValueError("rope_kv_store: positions and slot_mapping must be [T]")
    _check(library().pa_rope_kv_store(_ptr(q_out), _ptr(k_cache), _ptr(v_cache), _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(positions), _ptr(slot_mapping), q.shape[0], q.shape[1], hkv, d, bs, nb,
                                      float(rope_theta), _dtype_code(k_cache), _stream(k_cache)), "pa_rope_kv_store")


def kv_store_fp8(k_cache: torch.Tensor, v_cache: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                 slot_mapping: torch.Tensor, k_scale: float, v_scale: float) -> None:
    """pa_kv_store_fp8: bf16 k/v rows quantised to E4M3 codes (uint8 pools,
    one fp32 scale per pool) at slot_mapping."""
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev_tensor(t, name, torch.uint8)
    for name, t in (("k", k), ("v", v)):
        _dev_tensor(t, name, torch.bfloat16)
    _dev_tensor(slot_mapping, "slot_mapping", torch.int32)
    nb, bs, hkv, d = k_cache.shape
    if v_cache.shape != k_cache.shape or k.shape != v.shape or k.dim() != 3 or k.shape[1:] != (hkv, d):
        raise ValueError("kv_store_fp8: pools [NB, 256, Hkv, D] and k/v [T, Hkv, D] expected")
    if slot_mapping.shape != (k.shape[0],):
        raise ValueError("kv_store_fp8: slot_mapping must be [T]")
    _check(library().pa_kv_store_fp8(_ptr(k_cache), _ptr(v_cache), _ptr(k), _ptr(v), _ptr(slot_mapping), k.shape[0],
                                     hkv, d, bs, nb, float(k_scale), float(v_scale), _stream(k_cache)),
           "pa_kv_store_fp8")


def decode_fp8_workspace_bytes(num_seqs: int, num_q_heads: int, head_dim: int, max_context_len: int) -> int:
    return int(library().pa_decode_fp8_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len))


def paged_attn_decode_fp8(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float, k_scale: float,
                          v_scale: float, max_context_len: int,
                          workspace_tensor: Optional[torch.Tensor] = None) -> torch.Tensor:
    """pa_paged_attn_decode_fp8: bf16 out[B, Hq, D] = attention of bf16 q over
    the dequantised fp8 pools."""
    for name, t in (("out", out), ("q", q)):
        _dev_tensor(t, name, torch.bfloat16)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev_tensor(t, name, torch.uint8)
    _dev_tensor(block_tables, "block_tables", torch.int32)
    _dev_tensor(context_lens, "context_lens", torch.int32)
    nb, bs, hkv, d = k_cache.shape
    b, hq, dq = q.shape
    if out.shape != q.shape or dq != d or v_cache.shape != k_cache.shape or block_tables.dim() != 2 \
            or block_tables.shape[0] != b or context_lens.shape != (b,):
        raise ValueError("paged_attn_decode_fp8: shapes do not match")
    need = decode_fp8_workspace_bytes(b, hq, d, max_context_len)
    ws = workspace_tensor if workspace_tensor is not None else workspace(q.device, need, "decode_fp8", _stream(q))
    ws_ptr = None if ws is None else ws.data_ptr()
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(library().pa_paged_attn_decode_fp8(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                              _ptr(context_lens), b, hq, hkv, d, bs, nb, block_tables.shape[1],
                                              int(max_context_len), float(scale), float(k_scale), float(v_scale),
                                              ws_ptr, ws_bytes, _stream(q)), "pa_paged_attn_decode_fp8")
    return out


def qknorm_rope_kv_store(q_out: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, q: torch.Tensor,
                         k: torch.Tensor, v: torch.Tensor, q_norm_weight: torch.Tensor, k_norm_weight: torch.Tensor,
                         eps: float, positions: torch.Tensor, slot_mapping: torch.Tensor, rope_theta: float) -> None:
    """pa_qknorm_rope_kv_store: RMSNorm (weights [D]) of q and k head rows,
    then rope_kv_store."""
    for name, t in (("q_out", q_out), ("k_cache", k_cache), ("v_cache", v_cache), ("q", q), ("k", k), ("v", v),
                    ("q_norm_weight", q_norm_weight), ("k_norm_weight", k_norm_weight)):
        _dev_tensor(t, name, k_cache.dtype)
    _dev_tensor(positions, "positions", torch.int32)
    _dev_tensor(slot_mapping, "slot_mapping", torch.int32)
    nb, bs, hkv, d = k_cache.shape
    if q.dim() != 3 or q.shape[2] != d or q_out.shape != q.shape or k.shape != (q.shape[0], hkv, d) or v.shape != k.shape:
        raise ValueError("qknorm_rope_kv_store: q/q_out [T, Hq, D], k/v [T, Hkv, D] expected")
    if q_norm_weight.shape != (d,) or k_norm_weight.shape != (d,):
        raise ValueError("qknorm_rope_kv_store: norm weights must be [D]")
    if positions.shape != (q.shape[0],) or slot_mapping.shape != (q.shape[0],):
        raise ValueError("qknorm_rope_kv_store: positions and slot_mapping must be [T]")
    _check(library().pa_qknorm_rope_kv_store(_ptr(q_out), _ptr(k_cache), _ptr(v_cache), _ptr(q), _ptr(k), _ptr(v),
                                             _ptr(q_norm_weight), _ptr(k_norm_weight), float(eps), _ptr(positions),
                                             _ptr(slot_mapping), q.shape[0], q.shape[1], hkv, d, bs, nb,
                                             float(rope_theta), _dtype_code(k_cache), _stream(k_cache)),
           "pa_qknorm_rope_kv_store")


def decode_num_workgroups(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int, max_context_len: int,
                          dtype: torch.dtype = torch.bfloat16) -> int:
    return int(library().pa_decode_num_workgroups(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                                                  _DTYPES[dtype]))


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, head_dim: int, max_context_len: int) -> int:
    return int(library().pa_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, 1, max_context_len))


def paged_attn_decode(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float, max_context_len: int,
                      num_workgroups: int = 0, workspace_tensor: Optional[torch.Tensor] = None) -> torch.Tensor:
    """pa_paged_attn_decode(_ex): out[B, Hq, D] = attention of q over each
    sequence's paged context. max_context_len is a host int >= every context
    length (no device sync is made to find it); num_workgroups = 0 lets the
    library choose how many workgroups share the work."""
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("paged_attn_decode: q [B, Hq, D] and pools [NB, 256, Hkv, D] expected")
    b, hq, d = q.shape
    nb, bs, hkv, dk = k_cache.shape
    if out.shape != q.shape or dk != d or v_cache.shape != k_cache.shape or block_tables.dim() != 2 \
            or block_tables.shape[0] != b or context_lens.shape != (b,):
        raise ValueError("paged_attn_decode: shapes do not match (out == q [B, Hq, D], pools [NB, 256, Hkv, D], "
                         "block_tables [B, *], context_lens [B])")
    for name, t in (("out", out), ("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _dev_tensor(t, name, q.dtype)
    _dev_tensor(block_tables, "block_tables", torch.int32)
    _dev_tensor(context_lens, "context_lens", torch.int32)
    need = decode_workspace_bytes(b, hq, d, max_context_len)
    ws = workspace_tensor if workspace_tensor is not None else workspace(q.device, need, "decode", _stream(q))
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    status = library().pa_paged_attn_decode_ex(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), b, hq, hkv, d, bs,
        nb, block_tables.shape[1], int(max_context_len), float(scale), _dtype_code(q), int(num_workgroups),
        _ptr(ws), ws_bytes, _stream(q))
    _check(status, "pa_paged_attn_decode")
    return out


def paged_attn_decode_noalloc(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                              block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                              max_context_len: int) -> torch.Tensor:
    """pa_paged_attn_decode_noalloc: paged_attn_decode with the library's own
    per-GPU scratch instead of a workspace (the call allocates nothing; calls
    on one GPU must not overlap in time)."""
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("paged_attn_decode_noalloc: q [B, Hq, D] and pools [NB, 256, Hkv, D] expected")
    b, hq, d = q.shape
    nb, bs, hkv, dk = k_cache.shape
    if out.shape != q.shape or dk != d or v_cache.shape != k_cache.shape or block_tables.dim() != 2 \
            or block_tables.shape[0] != b or context_lens.shape != (b,):
        raise ValueError("paged_attn_decode_noalloc: shapes do not match")
    for name, t in (("out", out), ("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _dev_tensor(t, name, q.dtype)
    _dev_tensor(block_tables, "block_tables", torch.int32)
    _dev_tensor(context_lens, "context_lens", torch.int32)
    _check(library().pa_paged_attn_decode_noalloc(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                                  _ptr(block_tables), _ptr(context_lens), b, hq, hkv, d, bs, nb,
                                                  block_tables.shape[1], int(max_context_len), float(scale),
                                                  _dtype_code(q), _stream(q)), "pa_paged_attn_decode_noalloc")
    return out


def paged_attn_decode_store(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                            block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float, max_context_len: int,
                            workspace_tensor: Optional[torch.Tensor] = None) -> torch.Tensor:
    """pa_paged_attn_decode_store: store k_new/v_new [B, Hkv, D] at
    slot_mapping and decode over the contexts in one launch (the new token of
    sequence t is read in flight as its last position)."""
    for name, t in (("out", out), ("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("k_new", k_new),
                    ("v_new", v_new)):
        _dev_tensor(t, name, q.dtype)
    _dev_tensor(slot_mapping, "slot_mapping", torch.int32)
    _dev_tensor(block_tables, "block_tables", torch.int32)
    _dev_tensor(context_lens, "context_lens", torch.int32)
    nb, bs, hkv, d = k_cache.shape
    b, hq, dq = q.shape
    if out.shape != q.shape or dq != d or v_cache.shape != k_cache.shape or k_new.shape != (b, hkv, d) \
            or v_new.shape != k_new.shape or slot_mapping.shape != (b,) or block_tables.dim() != 2 \
            or block_tables.shape[0] != b or context_lens.shape != (b,):
        raise ValueError("paged_attn_decode_store: shapes do not match")
    need = decode_workspace_bytes(b, hq, d, max_context_len)
    ws = workspace_tensor if workspace_tensor is not None else workspace(q.device, need, "decode", _stream(q))
    ws_ptr = None if ws is None else ws.data_ptr()
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(library().pa_paged_attn_decode_store(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_new),
                                                _ptr(v_new), _ptr(slot_mapping), _ptr(block_tables),
                                                _ptr(context_lens), b, hq, hkv, d, bs, nb, block_tables.shape[1],
                                                int(max_context_len), float(scale), _dtype_code(q), ws_ptr, ws_bytes,
                                                _stream(q)), "pa_paged_attn_decode_store")
    return out


def prefill_workspace_bytes(num_seqs: int, num_q_heads: int, head_dim: int, max_q_len: int,
                            max_context_len: int) -> int:
    return int(library().pa_prefill_workspace_bytes(num_seqs, num_q_heads, head_dim, max_q_len, max_context_len))


def paged_attn_prefill(out: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, k_cache: torch.Tensor,
                       v_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                       cu_seqlens: torch.Tensor, scale: float, max_q_len: int, max_context_len: int,
                       workspace_tensor: Optional[torch.Tensor] = None, num_workgroups: int = 0) -> torch.Tensor:
    """pa_paged_attn_prefill(_ex): causal attention of the new tokens (rows of
    q/k/v per cu_seqlens) over each sequence's cached blocks plus the new
    tokens; num_workgroups = 0 lets the library choose the grid."""
    if q.dim() != 3 or k_cache.dim() != 4 or context_lens.dim() != 1:
        raise ValueError("paged_attn_prefill: q [T, Hq, D], pools [NB, 256, Hkv, D], context_lens [B] expected")
    total_q, hq, d = q.shape
    nb, bs, hkv, dk = k_cache.shape
    b = context_lens.shape[0]
    if out.shape != q.shape or dk != d or v_cache.shape != k_cache.shape or k.shape != (total_q, hkv, d) \
            or v.shape != k.shape or block_tables.dim() != 2 or block_tables.shape[0] != b \
            or cu_seqlens.shape != (b + 1,):
        raise ValueError("paged_attn_prefill: shapes do not match (out == q [T, Hq, D], k/v [T, Hkv, D], pools "
                         "[NB, 256, Hkv, D], block_tables [B, *], context_lens [B], cu_seqlens [B + 1])")
    for name, t in (("out", out), ("q", q), ("k", k), ("v", v), ("k_cache", k_cache), ("v_cache", v_cache)):
        _dev_tensor(t, name, q.dtype)
    for name, t in (("block_tables", block_tables), ("context_lens", context_lens), ("cu_seqlens", cu_seqlens)):
        _dev_tensor(t, name, torch.int32)
    need = prefill_workspace_bytes(b, hq, d, max_q_len, max_context_len)
    ws = workspace_tensor if workspace_tensor is not None else workspace(q.device, need, "prefill", _stream(q))
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    status = library().pa_paged_attn_prefill_ex(
        _ptr(out), _ptr(q), _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        _ptr(cu_seqlens), b, total_q, int(max_q_len), hq, hkv, d, bs, nb, block_tables.shape[1],
        int(max_context_len), float(scale), _dtype_code(q), int(num_workgroups), _ptr(ws), ws_bytes, _stream(q))
    _check(status, "pa_paged_attn_prefill")
    return out
