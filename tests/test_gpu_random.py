"""Seeded random decode and prefill cases on the GPU against the fp64 oracle:
head counts, head dims, dtypes, batch sizes, context and chunk lengths and
grid sizes drawn per case (each case's parameters are printed before it
runs), so the work split, the split-item pieces and their merges meet shapes
the named workloads do not have."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_209_amd as pa
import workloads as w
from gpu_util import DEV, compare, say, to_dev

pytestmark = pytest.mark.gpu

N_DECODE = 24
N_PREFILL = 24


def _poison(c, kept_lens):
    cov = w.covered_rows(c.block_tables, kept_lens, c.num_blocks)
    c.k_cache = w.poison_uncovered(c.k_cache, cov)
    c.v_cache = w.poison_uncovered(c.v_cache, cov)
    return c


def _lengths(rng, n, lo, hi):
    kind = rng.integers(0, 3)
    if kind == 0:
        return rng.integers(lo, min(hi, lo + 80), size=n, endpoint=True)
    if kind == 1:
        return rng.integers(lo, hi, size=n, endpoint=True)
    return np.where(rng.random(n) < 0.5, rng.integers(lo, min(hi, lo + 80), size=n, endpoint=True),
                    rng.integers(max(lo, hi // 2), hi, size=n, endpoint=True))


def _grid(rng, hi):
    """0 (the library's grid) a third of the time, one workgroup a sixth of
    the time, else a size drawn from [2, hi) (the launcher caps it)."""
    u = rng.random()
    return 0 if u < 1 / 3 else (1 if u < 0.5 else int(rng.integers(2, hi)))


@pytest.mark.parametrize("i", range(N_DECODE))
def test_random_decode(i):
    rng = np.random.default_rng(9000 + i)
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 3, 4, 8]))
    d = int(rng.choice([64, 128]))
    dtype = torch.float32 if rng.random() < 0.3 else torch.bfloat16
    b = int(rng.integers(1, 24, endpoint=True))
    ctx = _lengths(rng, b, 1, 6000).tolist()
    grid = _grid(rng, 600)
    scale = float(rng.uniform(0.25, 2.0)) / d ** 0.5
    shared = [s for s in range(b) if ctx[s] > 512 and rng.random() < 0.5]  # a common 2-block prefix chain
    say(f"random decode {i}: hq {hkv * group} hkv {hkv} d {d} {dtype} b {b} grid {grid} scale {scale:.4f} "
        f"shared {shared} ctx {ctx}")
    c = w.build_decode_case(f"rd{i}", ctx, hkv * group, hkv, d, dtype, 9000 + i, rng=rng, with_new_tokens=False,
                            shared_seqs=shared, shared_blocks=2 if shared else 0, scale=scale)
    c = _poison(c, c.context_lens)
    ref = oracle.paged_attn_decode(c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, c.scale)
    q = to_dev(c.q)
    out = torch.empty_like(q)
    pa.paged_attn_decode(out, q, to_dev(c.k_cache), to_dev(c.v_cache), to_dev(c.block_tables),
                         to_dev(c.context_lens), c.scale, c.max_context_len, num_workgroups=grid)
    torch.cuda.synchronize()
    compare(out, ref, dtype)


@pytest.mark.parametrize("i", range(N_PREFILL))
def test_random_prefill(i):
    rng = np.random.default_rng(7000 + i)
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 4]))
    d = int(rng.choice([64, 128]))
    b = int(rng.integers(1, 6, endpoint=True))
    cached = _lengths(rng, b, 0, 2000).tolist()
    short = rng.random() < 0.4  # verify-like chunks (32-row tiles) or longer ones
    new = (rng.integers(1, 8, size=b, endpoint=True) if short else _lengths(rng, b, 1, 200)).tolist()
    if b > 1 and rng.random() < 0.3:
        new[int(rng.integers(0, b))] = 0  # a sequence with no new rows in the batch
    grid = _grid(rng, 1000)
    scale = float(rng.uniform(0.25, 2.0)) / d ** 0.5
    say(f"random prefill {i}: hq {hkv * group} hkv {hkv} d {d} b {b} grid {grid} scale {scale:.4f} "
        f"cached {cached} new {new}")
    c = w.build_prefill_case(f"rp{i}", cached, new, hkv * group, hkv, d, torch.bfloat16, 7000 + i, rng=rng,
                             with_slots=False, scale=scale)
    c = _poison(c, c.context_lens - (c.cu_seqlens[1:] - c.cu_seqlens[:-1]))
    ref = oracle.paged_attn_prefill(c.q, c.k, c.v, c.k_cache, c.v_cache, c.block_tables, c.context_lens,
                                    c.cu_seqlens, c.scale)
    q = to_dev(c.q)
    out = torch.empty_like(q)
    pa.paged_attn_prefill(out, q, to_dev(c.k), to_dev(c.v), to_dev(c.k_cache), to_dev(c.v_cache),
                          to_dev(c.block_tables), to_dev(c.context_lens), to_dev(c.cu_seqlens), c.scale,
                          c.max_q_len, c.max_context_len, num_workgroups=grid)
    torch.cuda.synchronize()
    compare(out, ref, torch.bfloat16)
