"""The seeded generators build the documented structure (metadata only; the
"meta" device skips value generation for the multi-GB configs)."""
import math

import torch

import workloads as w
from workloads import BLOCK_SIZE


def _check_tables(bt, ctx, nb):
    for i, L in enumerate(ctx.tolist()):
        need = -(-L // BLOCK_SIZE)
        row = bt[i].tolist()
        assert all(0 <= b < nb for b in row[:need])
        assert all(b == -1 for b in row[need:])


def test_config1_structure():
    c = w.config1()
    assert c.context_lens.tolist() == [1, 37, 256, 513]
    assert c.k_cache.shape == (16, 256, 1, 64) and c.k_cache.dtype == torch.float32
    assert c.q.shape == (4, 2, 64) and c.scale == 1.0 / 8.0
    assert c.block_tables.shape == (4, 3)
    _check_tables(c.block_tables, c.context_lens, 16)
    used = [b for b in c.block_tables.flatten().tolist() if b >= 0]
    assert len(used) == 6 and len(set(used)) == 6
    for i, L in enumerate(c.context_lens.tolist()):
        p = L - 1
        assert int(c.slot_mapping[i]) == int(c.block_tables[i, p // 256]) * 256 + p % 256


def test_config2_structure():
    c = w.config2(device="meta")
    ctx = c.context_lens
    assert ctx.shape == (64,) and int(ctx.min()) >= 128 and int(ctx.max()) <= 4096
    need = sum(-(-L // 256) for L in ctx.tolist())
    assert c.num_blocks == math.ceil(1.25 * need)
    _check_tables(c.block_tables, ctx, c.num_blocks)
    used = [b for b in c.block_tables.flatten().tolist() if b >= 0]
    assert len(used) == len(set(used)) == need
    assert (c.num_q_heads, c.num_kv_heads, c.head_dim) == (16, 8, 128)


def test_config3_structure():
    c = w.config3(device="meta")
    n = (c.cu_seqlens[1:] - c.cu_seqlens[:-1]).tolist()
    assert n == [512] * 8 and c.total_q == 4096
    cached = (c.context_lens - 512).tolist()
    assert all(x % 256 == 0 and 0 <= x <= 2048 for x in cached)
    chain = None
    for i, x in enumerate(cached):
        row = c.block_tables[i].tolist()
        if x == max(cached):
            chain = row[: x // 256]
    for i, x in enumerate(cached):
        assert c.block_tables[i, : x // 256].tolist() == chain[: x // 256]
    sl = c.slot_mapping
    stored = sl[sl >= 0].tolist()
    assert len(set(stored)) == len(stored)
    assert 0.05 < (sl < 0).float().mean() < 0.2
    # every stored slot is the token's own position in its own blocks
    for i in range(8):
        for j in range(0, 512, 37):
            s = int(sl[512 * i + j])
            if s >= 0:
                p = cached[i] + j
                assert s == int(c.block_tables[i, p // 256]) * 256 + p % 256


def test_config4_structure():
    c = w.config4(device="meta")
    ctx = c.context_lens
    assert ctx.shape == (256,) and int(ctx.min()) >= 1024 and int(ctx.max()) <= 8192
    sharers = c.meta["shared_seqs"]
    assert len(sharers) == 128
    first = c.block_tables[sharers[0], :4].tolist()
    for s in sharers:
        assert c.block_tables[s, :4].tolist() == first
    others = [i for i in range(256) if i not in set(sharers)]
    private = set()
    for i in others:
        for b in c.block_tables[i, : -(-int(ctx[i]) // 256)].tolist():
            assert b not in first and b not in private
            private.add(b)
    assert c.slot_mapping is None
    _check_tables(c.block_tables, ctx, c.num_blocks)


def test_config5_structure():
    c = w.config5(device="meta")
    assert c.total_q == 640 and c.q.shape == (640, 32, 128)
    ctx = c.context_lens
    assert int(ctx.min()) >= 2048 and int(ctx.max()) <= 16384
    _check_tables(c.block_tables, ctx, c.num_blocks)
    used = [b for b in c.block_tables.flatten().tolist() if b >= 0]
    assert len(used) == len(set(used))
    sl = c.slot_mapping.tolist()
    assert min(sl) >= 0 and len(set(sl)) == len(sl)


def test_seeded_values_repeat():
    a, b = w.config1(), w.config1()
    assert torch.equal(a.k_cache, b.k_cache) and torch.equal(a.q, b.q)
    c = w.config1(seed=100)
    assert not torch.equal(a.q, c.q)


def test_poison_marks_uncovered_rows():
    c = w.config1()
    cov = w.covered_rows(c.block_tables, c.context_lens, c.num_blocks)
    assert int(cov.sum()) == int(c.context_lens.sum())
    p = w.poison_uncovered(c.k_cache, cov)
    assert torch.isnan(p[~cov]).all() and torch.equal(p[cov], c.k_cache[cov])
