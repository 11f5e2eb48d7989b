"""kv_store on the GPU against the oracle: bit-exact pools (the whole pools,
so untouched slots must keep their previous bytes, NaN payloads included)."""
import pytest
import torch

import oracle
import paged_kv_cache_209_amd as pa
import workloads as w
from gpu_util import DEV, bits, say, to_dev

pytestmark = pytest.mark.gpu


def _run_and_check(kc, vc, k, v, slots):
    ref_k, ref_v = oracle.kv_store(kc, vc, k, v, slots)
    dk, dv = to_dev(kc), to_dev(vc)
    pa.kv_store(dk, dv, to_dev(k), to_dev(v), to_dev(slots))
    torch.cuda.synchronize()
    assert torch.equal(bits(dk.cpu()), bits(ref_k))
    assert torch.equal(bits(dv.cpu()), bits(ref_v))


def test_kv_store_config1_fp32():
    say("kv_store c1")
    c = w.config1()
    _run_and_check(c.k_cache, c.v_cache, c.k_new, c.v_new, c.slot_mapping)


def test_kv_store_config3_bf16_with_skips():
    say("kv_store c3")
    c = w.config3()
    assert int((c.slot_mapping < 0).sum()) > 0
    _run_and_check(c.k_cache, c.v_cache, c.k, c.v, c.slot_mapping)


@pytest.mark.parametrize("dtype,hkv,d", [(torch.bfloat16, 1, 64), (torch.float32, 3, 128), (torch.bfloat16, 8, 128)])
def test_kv_store_sentinel_pool_and_nan_payloads(dtype, hkv, d):
    say("kv_store sentinel", dtype, hkv, d)
    g = torch.Generator().manual_seed(5)
    nb, T = 5, 300
    kc = torch.full((nb, 256, hkv, d), -3.0, dtype=dtype)
    vc = torch.full((nb, 256, hkv, d), 7.0, dtype=dtype)
    k = torch.randn((T, hkv, d), generator=g).to(dtype)
    v = torch.randn((T, hkv, d), generator=g).to(dtype)
    k[3] = float("nan")
    v[4] = float("-inf")
    perm = torch.randperm(nb * 256, generator=g)[:T].to(torch.int32)
    perm[::7] = -1
    _run_and_check(kc, vc, k, v, perm)


def test_kv_store_zero_tokens():
    kc = torch.zeros((2, 256, 1, 64), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    e = torch.empty((0, 1, 64), dtype=torch.bfloat16, device=DEV)
    pa.kv_store(kc, vc, e, e, torch.empty((0,), dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert int(kc.abs().sum()) == 0
