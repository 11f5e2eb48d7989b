"""Seeded synthetic inputs for paged KV-cache attention.

This module only builds inputs: the paging metadata an engine's input
preparation step produces (block tables, slot mappings, context lengths,
cumulative query offsets) and N(0, 1) values for queries, new keys/values and
the KV pools. It holds none of the attention arithmetic. The fp64 CPU oracle
and the HIP library both consume what it builds, and neither is imported here.

Sources for the shapes:
  * 256-token KV blocks, a free pool of blocks, prefix blocks shared by id:
    "Nano-vLLM System Architecture Analysis", section 2 "Core Components",
    item "Paged KV Cache (block_manager.py)".
  * K/V stored through a per-token slot mapping, block tables built per step:
    same page, section 2 item "Attention with Paged Cache" and section 3
    "Lifecycle of a Request" (prepare_inputs).
  * GQA head layout of the Qwen3 family: same page, "Differences from Normal
    nanoGPT Inference", item 6 "Architecture Support".
  * Chunked prefill and speculative verify as a short causal prefill:
    same page, section 2 "Scheduler" and "Differences" item 3; "What Is an
    Inference Engine, Anyway?", "Technical details" (speculative decoding).

Layout convention used throughout (the pages leave it open): a pool is
[num_blocks, 256, num_kv_heads, head_dim]; the token at logical position p of
a sequence lives in block block_table[p // 256], row p % 256, i.e. at flat
slot block_id * 256 + row of the pool viewed as [num_blocks * 256, Hkv, D].

Integer structure is drawn with numpy.random.default_rng(seed); values with a
torch.Generator seeded with seed + 1000, drawn in float32 and rounded to the
case dtype by torch's round-to-nearest-even cast.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

BLOCK_SIZE = 256
VALUE_SEED_OFFSET = 1000

# Chunk of pool blocks drawn per randn call, so that multi-GB pools never need
# a multi-GB float32 temporary.
_POOL_CHUNK_BLOCKS = 64


def _value_generator(seed: int, device):
    if str(device) == "meta":  # metadata-only cases: shapes without values
        return None
    g = torch.Generator(device=device)
    g.manual_seed(seed + VALUE_SEED_OFFSET)
    return g


def _randn(shape, gen, dtype: torch.dtype, device) -> torch.Tensor:
    if gen is None:
        return torch.empty(tuple(shape), dtype=dtype, device="meta")
    return torch.randn(tuple(shape), generator=gen, dtype=torch.float32, device=device).to(dtype)


def _randn_pool(num_blocks: int, hkv: int, d: int, gen, dtype, device) -> torch.Tensor:
    pool = torch.empty((num_blocks, BLOCK_SIZE, hkv, d), dtype=dtype, device=device)
    if gen is None:
        return pool
    for s in range(0, num_blocks, _POOL_CHUNK_BLOCKS):
        e = min(num_blocks, s + _POOL_CHUNK_BLOCKS)
        pool[s:e] = _randn((e - s, BLOCK_SIZE, hkv, d), gen, dtype, device)
    return pool


def blocks_for(length: int) -> int:
    """Number of 256-token blocks that hold `length` tokens."""
    return -(-int(length) // BLOCK_SIZE)


def slot_of(block_row: Sequence[int], position: int) -> int:
    """Flat pool slot of logical position `position` of a sequence whose block
    table row is `block_row` (the layout convention in the module docstring)."""
    return int(block_row[position // BLOCK_SIZE]) * BLOCK_SIZE + position % BLOCK_SIZE


def _table(rows: List[List[int]]) -> torch.Tensor:
    width = max(1, max(len(r) for r in rows))
    bt = torch.full((len(rows), width), -1, dtype=torch.int32)
    for i, r in enumerate(rows):
        if r:
            bt[i, : len(r)] = torch.tensor(r, dtype=torch.int32)
    return bt


@dataclass
class DecodeCase:
    """One decode step: optionally store one new token per sequence at
    position context_lens[i] - 1, then attend over context_lens[i] tokens."""

    name: str
    q: torch.Tensor  # [B, Hq, D]
    k_cache: torch.Tensor  # [NB, 256, Hkv, D]
    v_cache: torch.Tensor
    block_tables: torch.Tensor  # int32 [B, max_blocks], -1 padded
    context_lens: torch.Tensor  # int32 [B], >= 1
    scale: float
    k_new: Optional[torch.Tensor] = None  # [B, Hkv, D]
    v_new: Optional[torch.Tensor] = None
    slot_mapping: Optional[torch.Tensor] = None  # int32 [B]
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_q_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k_cache.shape[2])

    @property
    def head_dim(self) -> int:
        return int(self.q.shape[2])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max())


@dataclass
class PrefillCase:
    """One prefill (or speculative-verify) step: sequence i has n_i new tokens
    (rows cu_seqlens[i]:cu_seqlens[i+1] of q/k/v) after c_i = context_lens[i] - n_i
    cached tokens held in the pool through block_tables[i]."""

    name: str
    q: torch.Tensor  # [total_q, Hq, D]
    k: torch.Tensor  # [total_q, Hkv, D]
    v: torch.Tensor
    k_cache: torch.Tensor  # [NB, 256, Hkv, D]
    v_cache: torch.Tensor
    block_tables: torch.Tensor  # int32 [B, max_blocks], -1 padded
    context_lens: torch.Tensor  # int32 [B] = cached + new
    cu_seqlens: torch.Tensor  # int32 [B + 1]
    scale: float
    slot_mapping: Optional[torch.Tensor] = None  # int32 [total_q], -1 = not stored
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_q_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k_cache.shape[2])

    @property
    def head_dim(self) -> int:
        return int(self.q.shape[2])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_q_len(self) -> int:
        cu = self.cu_seqlens
        return int((cu[1:] - cu[:-1]).max()) if cu.numel() > 1 else 0

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max())


# ---------------------------------------------------------------------------
# generic builders
# ---------------------------------------------------------------------------


def build_decode_case(
    name: str,
    context_lens: Sequence[int],
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    dtype: torch.dtype,
    seed: int,
    *,
    rng: Optional[np.random.Generator] = None,
    pool_blocks: Optional[int] = None,
    pool_factor: float = 1.25,
    shared_seqs: Sequence[int] = (),
    shared_blocks: int = 0,
    with_new_tokens: bool = True,
    scale: Optional[float] = None,
    device="cpu",
) -> DecodeCase:
    """Ragged decode batch with shuffled block ids.

    Every sequence needs ceil(ctx/256) blocks. Sequences listed in
    `shared_seqs` take their first `shared_blocks` blocks from one common
    chain of ids (a shared system-prompt prefix); every other block is
    private. Unique ids are drawn as rng.permutation(pool)[:needed] and
    handed out in order: the common chain first, then each sequence's private
    blocks in sequence order.
    """
    if rng is None:
        rng = np.random.default_rng(seed)
    ctx = [int(c) for c in context_lens]
    assert all(c >= 1 for c in ctx)
    shared = set(int(s) for s in shared_seqs)
    for s in shared:
        assert blocks_for(ctx[s]) >= shared_blocks
    private = [blocks_for(c) - (shared_blocks if i in shared else 0) for i, c in enumerate(ctx)]
    unique = sum(private) + (shared_blocks if shared else 0)
    nb = pool_blocks if pool_blocks is not None else int(math.ceil(pool_factor * unique))
    assert nb >= unique
    ids = [int(x) for x in rng.permutation(nb)[:unique]]
    pos = 0
    chain = []
    if shared:
        chain = ids[:shared_blocks]
        pos = shared_blocks
    rows = []
    for i in range(len(ctx)):
        r = list(chain) if i in shared else []
        r += ids[pos : pos + private[i]]
        pos += private[i]
        rows.append(r)
    bt = _table(rows)
    hkv, hq, d = num_kv_heads, num_q_heads, head_dim
    gen = _value_generator(seed, device)
    k_cache = _randn_pool(nb, hkv, d, gen, dtype, device)
    v_cache = _randn_pool(nb, hkv, d, gen, dtype, device)
    q = _randn((len(ctx), hq, d), gen, dtype, device)
    case = DecodeCase(
        name=name,
        q=q,
        k_cache=k_cache,
        v_cache=v_cache,
        block_tables=bt,
        context_lens=torch.tensor(ctx, dtype=torch.int32),
        scale=float(scale if scale is not None else 1.0 / math.sqrt(d)),
        meta={"seed": seed, "unique_blocks": unique, "shared_seqs": sorted(shared),
              "shared_blocks": shared_blocks if shared else 0},
    )
    if with_new_tokens:
        case.k_new = _randn((len(ctx), hkv, d), gen, dtype, device)
        case.v_new = _randn((len(ctx), hkv, d), gen, dtype, device)
        case.slot_mapping = torch.tensor(
            [slot_of(rows[i], ctx[i] - 1) for i in range(len(ctx))], dtype=torch.int32)
    return case


def build_prefill_case(
    name: str,
    cached_lens: Sequence[int],
    new_lens: Sequence[int],
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    dtype: torch.dtype,
    seed: int,
    *,
    rng: Optional[np.random.Generator] = None,
    shared_chain: bool = False,
    skip_prob: float = 0.0,
    pool_factor: float = 1.25,
    pool_blocks: Optional[int] = None,
    with_slots: bool = True,
    scale: Optional[float] = None,
    device="cpu",
) -> PrefillCase:
    """Ragged prefill batch: sequence i has cached_lens[i] tokens in the pool
    and new_lens[i] new tokens whose K/V arrive with the call.

    Each sequence owns blocks for positions [0, cached + new). With
    `shared_chain`, cached prefixes (multiples of 256) are all taken from one
    common chain of block ids, so that sequences with cached prefixes of
    256*m tokens share the chain's first m blocks (prefix-cache reuse).
    `skip_prob` marks a Bernoulli subset of new tokens with slot -1.
    """
    if rng is None:
        rng = np.random.default_rng(seed)
    c = [int(x) for x in cached_lens]
    n = [int(x) for x in new_lens]
    assert len(c) == len(n) and all(x >= 0 for x in c) and all(x >= 0 for x in n)
    chain_len = 0
    if shared_chain:
        assert all(x % BLOCK_SIZE == 0 for x in c)
        chain_len = max(c) // BLOCK_SIZE if c else 0
    private = []
    for ci, ni in zip(c, n):
        total = blocks_for(ci + ni)
        private.append(total - (ci // BLOCK_SIZE if shared_chain else 0))
    unique = chain_len + sum(private)
    nb = pool_blocks if pool_blocks is not None else max(1, int(math.ceil(pool_factor * unique)))
    assert nb >= unique
    ids = [int(x) for x in rng.permutation(nb)[:unique]]
    chain = ids[:chain_len]
    pos = chain_len
    rows = []
    for i in range(len(c)):
        r = list(chain[: c[i] // BLOCK_SIZE]) if shared_chain else []
        r += ids[pos : pos + private[i]]
        pos += private[i]
        rows.append(r)
    bt = _table(rows)
    cu = [0]
    for ni in n:
        cu.append(cu[-1] + ni)
    total_q = cu[-1]
    slots = None
    if with_slots:
        sl = []
        for i in range(len(c)):
            for j in range(n[i]):
                sl.append(slot_of(rows[i], c[i] + j))
        sl = np.array(sl, dtype=np.int64)
        if skip_prob > 0 and total_q > 0:
            skip = rng.random(total_q) < skip_prob
            sl[skip] = -1
        slots = torch.tensor(sl, dtype=torch.int32)
    hkv, hq, d = num_kv_heads, num_q_heads, head_dim
    gen = _value_generator(seed, device)
    k_cache = _randn_pool(nb, hkv, d, gen, dtype, device)
    v_cache = _randn_pool(nb, hkv, d, gen, dtype, device)
    q = _randn((total_q, hq, d), gen, dtype, device)
    k = _randn((total_q, hkv, d), gen, dtype, device)
    v = _randn((total_q, hkv, d), gen, dtype, device)
    return PrefillCase(
        name=name,
        q=q,
        k=k,
        v=v,
        k_cache=k_cache,
        v_cache=v_cache,
        block_tables=bt,
        context_lens=torch.tensor([ci + ni for ci, ni in zip(c, n)], dtype=torch.int32),
        cu_seqlens=torch.tensor(cu, dtype=torch.int32),
        scale=float(scale if scale is not None else 1.0 / math.sqrt(d)),
        slot_mapping=slots,
        meta={"seed": seed, "unique_blocks": unique, "cached_lens": c, "new_lens": n},
    )


def covered_rows(block_tables: torch.Tensor, context_lens: torch.Tensor, num_blocks: int) -> torch.Tensor:
    """Bool mask [num_blocks, 256]: pool rows some sequence's context reaches."""
    mask = torch.zeros((num_blocks, BLOCK_SIZE), dtype=torch.bool)
    bt = block_tables.cpu()
    for i, L in enumerate(context_lens.cpu().tolist()):
        for b in range(blocks_for(L)):
            rows = min(BLOCK_SIZE, L - b * BLOCK_SIZE)
            mask[int(bt[i, b]), :rows] = True
    return mask


def poison_uncovered(pool: torch.Tensor, covered: torch.Tensor) -> torch.Tensor:
    """Return a copy of `pool` with every row outside `covered` set to NaN."""
    out = pool.clone()
    out[~covered.to(out.device)] = float("nan")
    return out


def paginate(sequences: Sequence[torch.Tensor], block_rows: Sequence[Sequence[int]], num_blocks: int,
             fill: float = float("nan")) -> torch.Tensor:
    """Place logical per-sequence rows ([L_i, Hkv, D] each) into a pool of
    `num_blocks` blocks following each sequence's block list. Rows no sequence
    covers hold `fill`. Sequences may share leading blocks only if their rows
    there are equal."""
    ref = sequences[0]
    pool = torch.full((num_blocks, BLOCK_SIZE) + tuple(ref.shape[1:]), fill, dtype=ref.dtype)
    for seq, row in zip(sequences, block_rows):
        for p in range(seq.shape[0]):
            pool[int(row[p // BLOCK_SIZE]), p % BLOCK_SIZE] = seq[p]
    return pool


def table_from_rows(rows: Sequence[Sequence[int]]) -> torch.Tensor:
    """int32 block table, -1 padded, from per-sequence block-id lists."""
    return _table([list(map(int, r)) for r in rows])


# ---------------------------------------------------------------------------
# the five named workloads (Qwen3-shaped, synthetic)
# ---------------------------------------------------------------------------


def config1(seed: int = 0, device="cpu") -> DecodeCase:
    """Tiny fp32 decode + store: 4 sequences with contexts {1, 37, 256, 513},
    2 query heads over 1 KV head, head_dim 64, 16-block pool, scale 1/8."""
    rng = np.random.default_rng(seed)
    return build_decode_case("c1_tiny_fp32_decode", [1, 37, 256, 513], 2, 1, 64, torch.float32, seed,
                             rng=rng, pool_blocks=16, scale=1.0 / 8.0, device=device)


def config2(seed: int = 1, device="cpu") -> DecodeCase:
    """Qwen3-0.6B-shaped decode, bf16: batch 64, 16 Q / 8 KV heads, D 128,
    contexts uniform in [128, 4096], pool 1.25x the blocks needed."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(128, 4096, size=64, endpoint=True)
    return build_decode_case("c2_qwen3_0.6b_decode", ctx, 16, 8, 128, torch.bfloat16, seed, rng=rng,
                             device=device)


def config3(seed: int = 2, device="cpu") -> PrefillCase:
    """Chunked prefill with prefix cache, bf16: 8 sequences, 16 Q / 8 KV heads,
    D 128, cached prefixes 256*U{0..8} taken from one shared chain of block
    ids, 512 new tokens each, 1/8 of the new tokens' slots set to -1."""
    rng = np.random.default_rng(seed)
    cached = (BLOCK_SIZE * rng.integers(0, 8, size=8, endpoint=True)).tolist()
    return build_prefill_case("c3_chunked_prefill_prefix", cached, [512] * 8, 16, 8, 128, torch.bfloat16,
                              seed, rng=rng, shared_chain=True, skip_prob=1.0 / 8.0, device=device)


def config4(seed: int = 3, device="cpu") -> DecodeCase:
    """Qwen3-8B-shaped decode, bf16: batch 256, 32 Q / 8 KV heads, D 128,
    contexts uniform in [1024, 8192]; a random half of the sequences share
    one 1024-token prefix (4 common block ids). No store step: the last
    position of a sharer may sit in a shared block."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(1024, 8192, size=256, endpoint=True)
    sharers = rng.choice(256, 128, replace=False)
    return build_decode_case("c4_qwen3_8b_decode_shared_prefix", ctx, 32, 8, 128, torch.bfloat16, seed,
                             rng=rng, shared_seqs=sharers.tolist(), shared_blocks=4,
                             with_new_tokens=False, device=device)


def config5(seed: int = 4, device="cpu") -> PrefillCase:
    """Speculative-verify mini-prefill, bf16: batch 128, 5 query tokens per
    sequence (causal among them), 32 Q / 8 KV heads, D 128, total contexts
    (including the 5 drafts) uniform in [2048, 16384], shuffled pool. The
    drafts' slots are their positions in each sequence's own blocks."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(2048, 16384, size=128, endpoint=True)
    cached = (ctx - 5).tolist()
    return build_prefill_case("c5_spec_verify", cached, [5] * 128, 32, 8, 128, torch.bfloat16, seed,
                              rng=rng, device=device)


CONFIGS = {
    "c1": config1,
    "c2": config2,
    "c3": config3,
    "c4": config4,
    "c5": config5,
}
