"""Seeded random cases of every entry point on the GPU against the oracle:
decode, prefill, the one-launch decode step, fp8 decode and the two stores,
with head counts, head dims, dtypes, batch sizes, context and chunk lengths,
scales, slots and grid sizes drawn per case (each case's parameters are
printed before it runs), so the work split, the split-item pieces and their
merges meet shapes the named workloads do not have. Stores are compared bit
for bit, attention at the dtype's bar."""
import numpy as np
import pytest
import torch

import oracle
import oracle.fp8_kv as f8
import paged_kv_cache_209_amd as pa
import workloads as w
from gpu_util import DEV, bits, compare, say, to_dev

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


N_STORE = 12


@pytest.mark.parametrize("i", range(N_STORE))
def test_random_kv_store(i):
    """Seeded random stores: pool dtype, head shape, token count, the pool's
    size and slots (distinct, about a quarter of them -1); the whole pools
    after the call equal the oracle's bit for bit."""
    rng = np.random.default_rng(11000 + i)
    g = torch.Generator().manual_seed(11000 + i)
    dtype = torch.float32 if rng.random() < 0.3 else torch.bfloat16
    hkv = int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    nb = int(rng.integers(1, 9))
    t = int(rng.integers(1, min(nb * 256, 3000), endpoint=True))
    slots = torch.from_numpy(rng.permutation(nb * 256)[:t].astype(np.int32))
    slots[torch.from_numpy(rng.random(t) < 0.25)] = -1
    say(f"random kv_store {i}: {dtype} hkv {hkv} d {d} blocks {nb} tokens {t} skipped {int((slots < 0).sum())}")
    kc = torch.randn(nb, 256, hkv, d, generator=g).to(dtype)
    vc = torch.randn(nb, 256, hkv, d, generator=g).to(dtype)
    k = torch.randn(t, hkv, d, generator=g).to(dtype)
    v = torch.randn(t, hkv, d, generator=g).to(dtype)
    ref_k, ref_v = oracle.kv_store(kc, vc, k, v, slots)
    dkc, dvc = to_dev(kc), to_dev(vc)
    pa.kv_store(dkc, dvc, to_dev(k), to_dev(v), to_dev(slots))
    torch.cuda.synchronize()
    assert torch.equal(bits(dkc.cpu()), bits(ref_k))
    assert torch.equal(bits(dvc.cpu()), bits(ref_v))


@pytest.mark.parametrize("i", range(N_STORE))
def test_random_kv_store_fp8(i):
    """Seeded random fp8 stores: scales over four decades, values from
    subnormal codes to saturation with a few NaN and infinite elements;
    both code pools equal the oracle's bit for bit."""
    rng = np.random.default_rng(12000 + i)
    g = torch.Generator().manual_seed(12000 + i)
    hkv = int(rng.choice([1, 2, 8]))
    nb = int(rng.integers(1, 5))
    t = int(rng.integers(1, min(nb * 256, 1500), endpoint=True))
    ks, vs = (float(10.0 ** rng.uniform(-3, 1)) for _ in range(2))
    slots = torch.from_numpy(rng.permutation(nb * 256)[:t].astype(np.int32))
    slots[torch.from_numpy(rng.random(t) < 0.2)] = -1
    k = torch.randn(t, hkv, 128, generator=g) * float(10.0 ** rng.uniform(-4, 3))
    v = torch.randn(t, hkv, 128, generator=g) * float(10.0 ** rng.uniform(-4, 3))
    for x in (k, v):
        idx = torch.from_numpy(rng.integers(0, x.numel(), size=4))
        x.view(-1)[idx] = torch.tensor([float("nan"), -float("inf"), float("inf"), -float("nan")])
    k, v = k.to(torch.bfloat16), v.to(torch.bfloat16)
    say(f"random kv_store_fp8 {i}: hkv {hkv} blocks {nb} tokens {t} scales {ks:.3g} {vs:.3g}")
    kc = torch.randint(0, 256, (nb, 256, hkv, 128), generator=g, dtype=torch.uint8)
    vc = torch.randint(0, 256, (nb, 256, hkv, 128), generator=g, dtype=torch.uint8)
    ref_k, ref_v = f8.kv_store_fp8(kc, vc, k, v, slots, ks, vs)
    dkc, dvc = to_dev(kc), to_dev(vc)
    pa.kv_store_fp8(dkc, dvc, to_dev(k), to_dev(v), to_dev(slots), ks, vs)
    torch.cuda.synchronize()
    assert torch.equal(dkc.cpu(), ref_k)
    assert torch.equal(dvc.cpu(), ref_v)


@pytest.mark.parametrize("i", range(N_STORE))
def test_random_decode_fp8(i):
    """Seeded random fp8 decode: GQA group, batch, context mix, pool scales;
    NaN codes in every pool row that no context covers."""
    rng = np.random.default_rng(13000 + i)
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 3, 4, 8]))
    b = int(rng.integers(1, 24, endpoint=True))
    ctx = _lengths(rng, b, 1, 6000).tolist()
    ks, vs = (float(10.0 ** rng.uniform(-2.5, -0.5)) for _ in range(2))
    say(f"random decode_fp8 {i}: hq {hkv * group} hkv {hkv} b {b} scales {ks:.3g} {vs:.3g} ctx {ctx}")
    c = w.build_decode_case(f"rf{i}", ctx, hkv * group, hkv, 128, torch.bfloat16, 13000 + i, rng=rng,
                            with_new_tokens=False)
    cov = w.covered_rows(c.block_tables, c.context_lens, c.num_blocks)
    kq = f8.quantize(c.k_cache, ks).clone()
    vq = f8.quantize(c.v_cache, vs).clone()
    kq[~cov] = 0x7F
    vq[~cov] = 0x7F
    ref = f8.paged_attn_decode_fp8(c.q, kq, vq, c.block_tables, c.context_lens, c.scale, ks, vs)
    q = to_dev(c.q)
    out = torch.empty_like(q)
    pa.paged_attn_decode_fp8(out, q, to_dev(kq), to_dev(vq), to_dev(c.block_tables), to_dev(c.context_lens), c.scale,
                             ks, vs, c.max_context_len)
    torch.cuda.synchronize()
    compare(out, ref, torch.bfloat16)


@pytest.mark.parametrize("i", range(N_STORE))
def test_random_decode_store(i):
    """Seeded random one-launch decode steps (store + decode): the output
    against the oracle's store-then-decode, and both pools afterwards bit for
    bit against the oracle's store."""
    rng = np.random.default_rng(14000 + i)
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 3, 4, 8]))
    d = int(rng.choice([64, 128]))
    dtype = torch.float32 if rng.random() < 0.3 else torch.bfloat16
    b = int(rng.integers(1, 40, endpoint=True))
    ctx = _lengths(rng, b, 1, 5000).tolist()
    say(f"random decode_store {i}: hq {hkv * group} hkv {hkv} d {d} {dtype} b {b} ctx {ctx}")
    c = w.build_decode_case(f"rs{i}", ctx, hkv * group, hkv, d, dtype, 14000 + i, rng=rng)
    kc_ref, vc_ref = oracle.kv_store(c.k_cache, c.v_cache, c.k_new, c.v_new, c.slot_mapping)
    ref = oracle.paged_attn_decode(c.q, kc_ref, vc_ref, c.block_tables, c.context_lens, c.scale)
    q = to_dev(c.q)
    out = torch.empty_like(q)
    kc, vc = to_dev(c.k_cache), to_dev(c.v_cache)
    pa.paged_attn_decode_store(out, q, kc, vc, to_dev(c.k_new), to_dev(c.v_new), to_dev(c.slot_mapping),
                               to_dev(c.block_tables), to_dev(c.context_lens), c.scale, c.max_context_len)
    torch.cuda.synchronize()
    compare(out, ref, dtype)
    assert torch.equal(bits(kc.cpu()), bits(kc_ref))
    assert torch.equal(bits(vc.cpu()), bits(vc_ref))
