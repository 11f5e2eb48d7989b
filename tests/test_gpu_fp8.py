"""fp8 KV cache on the GPU against the oracle (oracle/fp8_kv.py): the
quantising store bit for bit (including saturating and subnormal values and
skipped slots), and decode attention over fp8 pools within the bf16 bar for
GQA groups 1, 2 and 4, ragged contexts, NaN codes in every row no context
covers, batches from a few sequences to 480 and 512 (sequence, head-group)
items with contexts up to 12000 tokens, the Qwen3-0.6B- and Qwen3-8B-shaped
decode workloads at full size, and repeated runs bit-identical."""
import numpy as np
import pytest
import torch

import oracle
import oracle.fp8_kv as f8
import paged_kv_cache_209_amd as pa
import workloads as w
from gpu_util import DEV, compare, say, to_dev

pytestmark = pytest.mark.gpu


def test_store_bit_exact():
    say("fp8 store")
    g = torch.Generator().manual_seed(8)
    rng = np.random.default_rng(8)
    t, hkv, d, nb = 300, 8, 128, 6
    k = torch.randn(t, hkv, d, generator=g)
    v = torch.randn(t, hkv, d, generator=g)
    k[::7] *= 1000.0   # saturates at +-448 codes
    v[1::9] *= 1e-4    # subnormal codes
    # non-finite elements: NaN of either sign keeps its sign in the NaN code
    # S.1111.111, infinities saturate to +-448
    k[3, 0, :4] = torch.tensor([float("nan"), -float("nan"), float("inf"), -float("inf")])
    v[5, 1, 8:12] = torch.tensor([-float("inf"), float("inf"), -float("nan"), float("nan")])
    k[10, 2, 100] = float("nan")
    v[11, 3, 127] = -float("nan")
    k, v = k.to(torch.bfloat16), v.to(torch.bfloat16)
    kc = torch.randint(0, 256, (nb, 256, hkv, d), generator=g, dtype=torch.uint8)
    vc = torch.randint(0, 256, (nb, 256, hkv, d), generator=g, dtype=torch.uint8)
    slots = torch.from_numpy(rng.permutation(nb * 256)[:t].astype(np.int32))
    slots[2::5] = -1
    ks, vs = 0.05, 0.02
    assert all(int(slots[r]) >= 0 for r in (3, 5, 10, 11))  # the non-finite rows are stored
    ref_k, ref_v = f8.kv_store_fp8(kc, vc, k, v, slots, ks, vs)
    assert int(ref_k[int(slots[3]) // 256, int(slots[3]) % 256, 0, 0]) in (0x7F, 0xFF)  # NaN code
    dkc, dvc = to_dev(kc), to_dev(vc)
    pa.kv_store_fp8(dkc, dvc, to_dev(k), to_dev(v), to_dev(slots), ks, vs)
    torch.cuda.synchronize()
    assert torch.equal(dkc.cpu(), ref_k)
    assert torch.equal(dvc.cpu(), ref_v)


def fp8_case(seed, ctx, hq, hkv, scales=(0.0125, 0.0125), poison=True):
    c = w.build_decode_case(f"fp8_{seed}", ctx, hq, hkv, 128, torch.bfloat16, seed)
    kq = f8.quantize(c.k_cache, scales[0])
    vq = f8.quantize(c.v_cache, scales[1])
    if poison:
        cov = w.covered_rows(c.block_tables, c.context_lens, c.num_blocks)
        kq = kq.clone()
        vq = vq.clone()
        kq[~cov] = 0x7F  # NaN codes wherever no context reads
        vq[~cov] = 0x7F
    return c, kq, vq


def run(c, kq, vq, scales):
    q = to_dev(c.q)
    out = torch.empty_like(q)
    pa.paged_attn_decode_fp8(out, q, to_dev(kq), to_dev(vq), to_dev(c.block_tables), to_dev(c.context_lens),
                             c.scale, scales[0], scales[1], c.max_context_len)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (32, 8)], ids=["g1", "g2", "g4"])
def test_decode_matches_oracle(hq, hkv):
    say(f"fp8 decode hq={hq} hkv={hkv}")
    scales = (0.0125, 0.02)
    c, kq, vq = fp8_case(3 + hq, [1, 37, 256, 257, 513, 1000, 2048], hq, hkv, scales)
    out = run(c, kq, vq, scales)
    ref = f8.paged_attn_decode_fp8(c.q, kq, vq, c.block_tables, c.context_lens, c.scale, *scales)
    compare(out, ref, torch.bfloat16)
    again = run(c, kq, vq, scales)
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))


def test_one_token_context_returns_dequantised_v():
    scales = (0.0125, 0.02)
    c, kq, vq = fp8_case(41, [1, 1, 300], 16, 8, scales)
    out = run(c, kq, vq, scales).cpu()
    for i in (0, 1):
        blk = int(c.block_tables[i, 0])
        want = f8.dequantize(vq[blk, 0], scales[1])  # [Hkv, D]
        for g in range(16):
            assert torch.equal(out[i, g], want[g // 2].to(torch.float32).to(torch.bfloat16))


def test_contexts_within_one_unit_need_no_workspace():
    """Contexts of at most 64 tokens are never split, so the call needs no
    workspace (the binding passes none)."""
    scales = (0.0125, 0.02)
    c, kq, vq = fp8_case(42, [1, 17, 64, 63], 16, 8, scales)
    assert pa.decode_fp8_workspace_bytes(4, 16, 128, 64) == 0
    out = run(c, kq, vq, scales)
    ref = f8.paged_attn_decode_fp8(c.q, kq, vq, c.block_tables, c.context_lens, c.scale, *scales)
    compare(out, ref, torch.bfloat16)


def test_qwen3_0_6b_decode_workload_full_size():
    """Batch 64, 16 Q / 8 KV heads, contexts U[128, 4096], the pools of the
    bf16 workload quantised with scale 1/80."""
    say("fp8 decode c2 full size")
    c = w.config2()
    s = 1.0 / 80.0
    kq, vq = f8.quantize(c.k_cache, s), f8.quantize(c.v_cache, s)
    out = run(c, kq, vq, (s, s))
    ref = f8.paged_attn_decode_fp8(c.q, kq, vq, c.block_tables, c.context_lens, c.scale, s, s)
    compare(out, ref, torch.bfloat16)


@pytest.mark.parametrize("max_ctx,blocks", [(9216, 4), (4352, 2)], ids=["9216", "4352"])
def test_decode_long_ragged_contexts(max_ctx, blocks):
    """60 sequences, 32 Q / 8 KV heads (480 items), contexts uniform in
    [1, max_ctx] with one of each extreme: many items split over several
    workgroups and merged in the kernel."""
    say(f"fp8 decode contexts up to {max_ctx}")
    rng = np.random.default_rng(77 + blocks)
    ctx = [int(x) for x in rng.integers(1, max_ctx, endpoint=True, size=60)]
    ctx[0], ctx[1] = max_ctx, 1
    scales = (0.0125, 0.0125)
    c, kq, vq = fp8_case(77 + blocks, ctx, 32, 8, scales)
    out = run(c, kq, vq, scales)
    ref = f8.paged_attn_decode_fp8(c.q, kq, vq, c.block_tables, c.context_lens, c.scale, *scales)
    compare(out, ref, torch.bfloat16)


def test_decode_short_contexts_and_long_outliers():
    """64 sequences x 8 query-head groups = 512 items, contexts up to 2000
    tokens plus three of 12000, 8193 and 8192: the cost-balanced split gives
    the outliers' items to several workgroups each."""
    say("fp8 decode short contexts and long outliers")
    rng = np.random.default_rng(78)
    ctx = [int(x) for x in rng.integers(1, 2000, endpoint=True, size=64)]
    ctx[0], ctx[1], ctx[2] = 12000, 8193, 8192
    scales = (0.0125, 0.02)
    c, kq, vq = fp8_case(78, ctx, 32, 8, scales)
    out = run(c, kq, vq, scales)
    ref = f8.paged_attn_decode_fp8(c.q, kq, vq, c.block_tables, c.context_lens, c.scale, *scales)
    compare(out, ref, torch.bfloat16)
    again = run(c, kq, vq, scales)
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))


def test_qwen3_8b_shared_prefix_full_size():
    """The Qwen3-8B-shaped workload with a shared prefix at full size (batch
    256, 32 Q / 8 KV heads, contexts U[1024, 8192], as the benchmark runs
    it): its bf16 pools quantised with scale 1/80 by torch on the device
    (input generation), every (sequence, head) row against the oracle."""
    say("fp8 decode c4 full size, all rows")
    c = w.config4(device=DEV)
    s = 1.0 / 80.0

    def codes(x):
        return (x.to(torch.float32) * 80.0).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)

    kq, vq = codes(c.k_cache), codes(c.v_cache)
    del c.k_cache, c.v_cache
    out = torch.empty_like(c.q)
    pa.paged_attn_decode_fp8(out, c.q, kq, vq, to_dev(c.block_tables), to_dev(c.context_lens), c.scale, s, s,
                             c.max_context_len)
    torch.cuda.synchronize()
    ref = f8.paged_attn_decode_fp8(c.q.cpu(), kq.cpu(), vq.cpu(), c.block_tables.cpu(), c.context_lens.cpu(), c.scale,
                                   s, s)
    compare(out, ref, torch.bfloat16)


def test_zero_length_contexts_are_skipped():
    """A context length of 0 leaves that output row unwritten and does not
    disturb the others."""
    say("fp8 decode zero-length contexts")
    scales = (0.0125, 0.02)
    c, kq, vq = fp8_case(44, [1, 700, 1, 300, 1], 16, 8, scales, poison=False)
    ctx = c.context_lens.clone()
    ctx[0] = 0
    ctx[2] = 0
    ctx[4] = 0
    q = to_dev(c.q)
    out = torch.full_like(q, 7.0)
    pa.paged_attn_decode_fp8(out, q, to_dev(kq), to_dev(vq), to_dev(c.block_tables), to_dev(ctx), c.scale,
                             scales[0], scales[1], c.max_context_len)
    torch.cuda.synchronize()
    got = out.cpu()
    for i in (0, 2, 4):
        assert torch.all(got[i] == 7.0)
    ref = f8.paged_attn_decode_fp8(c.q, kq, vq, c.block_tables, c.context_lens, c.scale, *scales, seqs=[1, 3])
    compare(got, ref, torch.bfloat16, rows=[1, 3])
