"""Plain, slow fp64 CPU oracle for paged KV-cache attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module:
only the tests, the smoke check of the package entry file and the CPU-baseline
leg of the benchmark may import or call it. It shares no code with the HIP
library and imports nothing from it.

What it computes (the exact result of the definition, no blocking or fusion):

* Attention itself is softmax(q k^T) v, written on the Baidu article about
  Nano-vLLM, section "Computational Acceleration / TorchScript Optimization"
  (the plain `attention(q, k, v)` function: two matmuls around a softmax).
  That snippet has no scale and no mask; the caller's `scale` multiplies the
  scores and the causal mask is bottom-right aligned (query j of a chunk that
  starts after c cached tokens sees keys 0 .. c + j).
* The paged cache: "Nano-vLLM System Architecture Analysis", section 2 "Core
  Components", items "Paged KV Cache" (fixed 256-token blocks) and "Attention
  with Paged Cache": K/V entries are stored via slot_mapping; prefill with a
  prefix cache gathers the cached K/V from the paged cache and concatenates
  the newly computed ones; decode gathers all cached K/V from the paged blocks
  before the attention call. The oracle does exactly that gather, block by
  block in table order, and then runs the dense definition in float64.
* GQA ("Differences from Normal nanoGPT Inference", item 6): query head g
  reads KV head g // (Hq / Hkv).

Readings where the pages are silent: the pool layout is
[num_blocks, 256, Hkv, D] with flat slot = block_id * 256 + row; a negative
slot means "do not store"; decode context lengths include the token stored in
the same step; prefill context lengths count cached + new tokens and the new
tokens' K/V come from the call's k/v, not from the pool.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Tuple

import torch

TOKENS_PER_BLOCK = 256


def _bits(t: torch.Tensor) -> torch.Tensor:
    """Same-size integer view, so that copies move raw bits (NaN payloads kept)."""
    size = t.element_size()
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[size])


def kv_store(k_cache: torch.Tensor, v_cache: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
             slot_mapping: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Store new K/V rows into copies of the pools through slot_mapping.

    Follows "Nano-vLLM System Architecture Analysis", section 2, "Attention with
    Paged Cache": computed K/V entries are stored into the paged cache via
    slot_mapping. Token t goes to block slot // 256, row slot % 256 of both
    pools; a negative slot is skipped. The copy is a bit copy in the pools'
    own dtype. Duplicate or out-of-range slots are rejected (several results
    would be "correct" for a duplicate).
    """
    nb, bs, hkv, d = k_cache.shape
    assert bs == TOKENS_PER_BLOCK
    assert k.shape == v.shape and k.shape[1:] == (hkv, d)
    assert k.dtype == k_cache.dtype == v.dtype == v_cache.dtype
    slots = [int(s) for s in slot_mapping.tolist()]
    assert len(slots) == k.shape[0]
    stored = [s for s in slots if s >= 0]
    assert len(set(stored)) == len(stored), "duplicate slots"
    assert all(s < nb * bs for s in stored), "slot outside the pool"
    kc = k_cache.clone()
    vc = v_cache.clone()
    kcb, vcb, kb, vb = _bits(kc), _bits(vc), _bits(k), _bits(v)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        block, row = divmod(s, bs)
        kcb[block, row] = kb[t]
        vcb[block, row] = vb[t]
    return kc, vc


def gather_sequence(head_pool: torch.Tensor, block_row: torch.Tensor, length: int) -> torch.Tensor:
    """Logical rows 0 .. length-1 of one sequence for one KV head.

    `head_pool` is one head's slice of a pool, [num_blocks, 256, D]. The
    sequence's blocks are concatenated in block-table order and cut to
    `length` rows ("gathers cached K/V from the paged cache").
    """
    d = head_pool.shape[-1]
    if length == 0:
        return head_pool.new_zeros((0, d))
    nblk = -(-length // TOKENS_PER_BLOCK)
    ids = [int(b) for b in block_row[:nblk].tolist()]
    assert all(0 <= b < head_pool.shape[0] for b in ids), "block id outside the pool"
    rows = torch.cat([head_pool[b] for b in ids], dim=0)
    return rows[:length]


def attend(q_rows: torch.Tensor, keys: torch.Tensor, values: torch.Tensor, scale: float,
           visible: List[int]) -> torch.Tensor:
    """softmax(q k^T * scale) v in float64 for a few query rows.

    q_rows [n, D], keys/values [L, D]; query row j sees keys 0 .. visible[j]-1.
    Every row sees at least one key. The max is subtracted before exp only to
    keep exp finite; it cancels in the normalisation.
    """
    q64 = q_rows.to(torch.float64)
    k64 = keys.to(torch.float64)
    v64 = values.to(torch.float64)
    scores = (q64 @ k64.T) * scale
    for j, vis in enumerate(visible):
        assert 1 <= vis <= k64.shape[0]
        scores[j, vis:] = -math.inf
    scores = scores - scores.max(dim=1, keepdim=True).values
    weights = torch.exp(scores)
    return (weights @ v64) / weights.sum(dim=1, keepdim=True)


def _check_common(q_heads: int, k_cache: torch.Tensor, v_cache: torch.Tensor, d: int) -> Tuple[int, int]:
    nb, bs, hkv, dk = k_cache.shape
    assert bs == TOKENS_PER_BLOCK and dk == d and v_cache.shape == k_cache.shape
    assert q_heads % hkv == 0
    return hkv, q_heads // hkv


def paged_attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                      seqs: Optional[Iterable[int]] = None) -> torch.Tensor:
    """Decode attention: one query token per sequence over its whole context.

    Follows "Nano-vLLM System Architecture Analysis", section 2, "Attention with
    Paged Cache" (decode gathers all cached K/V from the paged blocks before the
    attention call) and section 3 (decode produces one token per sequence).
    q [B, Hq, D]; pools [NB, 256, Hkv, D]; context_lens[i] >= 1 counts every
    token the query sees, including the one stored in the same step.
    Returns float64 [B, Hq, D]; rows of sequences not in `seqs` stay zero.
    """
    b, hq, d = q.shape
    hkv, group = _check_common(hq, k_cache, v_cache, d)
    out = torch.zeros((b, hq, d), dtype=torch.float64)
    for i in (range(b) if seqs is None else seqs):
        length = int(context_lens[i])
        assert length >= 1
        for h in range(hkv):
            keys = gather_sequence(k_cache[:, :, h, :], block_tables[i], length)
            values = gather_sequence(v_cache[:, :, h, :], block_tables[i], length)
            for g in range(h * group, (h + 1) * group):
                out[i, g] = attend(q[i, g].unsqueeze(0), keys, values, scale, [length])[0]
    return out


def paged_attn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, k_cache: torch.Tensor,
                       v_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                       cu_seqlens: torch.Tensor, scale: float,
                       seqs: Optional[Iterable[int]] = None) -> torch.Tensor:
    """Causal attention of new tokens over cached blocks plus the new tokens.

    Follows "Nano-vLLM System Architecture Analysis", section 2, "Attention with
    Paged Cache" (prefill with a prefix cache gathers the cached K/V and
    concatenates the newly computed ones) and "Scheduler" (chunked prefill: a
    long prompt is split over steps, so a chunk starts after cached tokens).
    Speculative verify is the same computation with a few new tokens ("What Is
    an Inference Engine, Anyway?", Technical details: the target model checks
    the proposed tokens in one parallel mini-prefill).

    Sequence i owns rows cu_seqlens[i] .. cu_seqlens[i+1]-1 of q/k/v (n_i new
    tokens) and c_i = context_lens[i] - n_i cached tokens in the pool. New
    token j sits at position c_i + j and sees keys 0 .. c_i + j.
    Returns float64 [total_q, Hq, D]; rows of sequences not in `seqs` stay zero.
    """
    total_q, hq, d = q.shape
    hkv, group = _check_common(hq, k_cache, v_cache, d)
    assert k.shape == v.shape == (total_q, hkv, d)
    cu = [int(x) for x in cu_seqlens.tolist()]
    out = torch.zeros((total_q, hq, d), dtype=torch.float64)
    for i in (range(len(cu) - 1) if seqs is None else seqs):
        start, end = cu[i], cu[i + 1]
        n = end - start
        cached = int(context_lens[i]) - n
        assert cached >= 0 and n >= 0
        if n == 0:
            continue
        visible = [cached + j + 1 for j in range(n)]
        for h in range(hkv):
            old_k = gather_sequence(k_cache[:, :, h, :], block_tables[i], cached)
            old_v = gather_sequence(v_cache[:, :, h, :], block_tables[i], cached)
            keys = torch.cat([old_k.to(torch.float64), k[start:end, h, :].to(torch.float64)], dim=0)
            values = torch.cat([old_v.to(torch.float64), v[start:end, h, :].to(torch.float64)], dim=0)
            for g in range(h * group, (h + 1) * group):
                out[start:end, g] = attend(q[start:end, g], keys, values, scale, visible)
    return out
