"""Paged prefill / speculative verify on the GPU against the fp64 oracle,
and the device-side invariants: chunked prefill equals one-shot prefill,
decode equals a one-token prefill, verify equals five decodes, block
relabelling and repeated runs are bit-identical."""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_209_amd as pa
import workloads as w
from gpu_util import DEV, bits, compare, say, to_dev

pytestmark = pytest.mark.gpu


def run_prefill(case, k_cache=None, v_cache=None, block_tables=None):
    q = to_dev(case.q)
    out = torch.empty_like(q)
    pa.paged_attn_prefill(out, q, to_dev(case.k), to_dev(case.v),
                          k_cache if k_cache is not None else to_dev(case.k_cache),
                          v_cache if v_cache is not None else to_dev(case.v_cache),
                          to_dev(block_tables if block_tables is not None else case.block_tables),
                          to_dev(case.context_lens), to_dev(case.cu_seqlens), case.scale, case.max_q_len,
                          case.max_context_len)
    torch.cuda.synchronize()
    return out


def oracle_prefill(c, seqs=None):
    return oracle.paged_attn_prefill(c.q, c.k, c.v, c.k_cache, c.v_cache, c.block_tables, c.context_lens,
                                     c.cu_seqlens, c.scale, seqs=seqs)


def poisoned(c):
    cov = w.covered_rows(c.block_tables, c.context_lens - (c.cu_seqlens[1:] - c.cu_seqlens[:-1]), c.num_blocks)
    c.k_cache = w.poison_uncovered(c.k_cache, cov)
    c.v_cache = w.poison_uncovered(c.v_cache, cov)
    return c


def test_config3_store_then_prefill():
    """Chunked prefill with a shared prefix cache: store the new tokens (1/8
    of them skipped), then attend; all rows against the oracle."""
    say("prefill c3")
    c = w.config3()
    kc, vc = oracle.kv_store(c.k_cache, c.v_cache, c.k, c.v, c.slot_mapping)
    ref = oracle.paged_attn_prefill(c.q, c.k, c.v, kc, vc, c.block_tables, c.context_lens, c.cu_seqlens, c.scale)
    dk, dv = to_dev(c.k_cache), to_dev(c.v_cache)
    pa.kv_store(dk, dv, to_dev(c.k), to_dev(c.v), to_dev(c.slot_mapping))
    out = run_prefill(c, k_cache=dk, v_cache=dv)
    mx, mean = compare(out, ref, torch.bfloat16)
    say(f"  c3 max {mx:.3g} mean {mean:.3g}")


def check_config5(seed):
    """Config 5 at full size (values drawn on the device, batch 128, 5 drafts
    each, 32 Q / 8 KV heads, contexts U[2048, 16384]): every row of all 640
    query tokens against the oracle, which reads host copies of the pools."""
    c = w.config5(seed, device=DEV)
    out = run_prefill(c, k_cache=c.k_cache, v_cache=c.v_cache)
    host = w.PrefillCase(c.name, c.q.cpu(), c.k.cpu(), c.v.cpu(), c.k_cache.cpu(), c.v_cache.cpu(), c.block_tables,
                         c.context_lens, c.cu_seqlens, c.scale)
    ref = oracle_prefill(host)
    mx, mean = compare(out, ref, torch.bfloat16)
    say(f"  c5 seed {seed}: max {mx:.3g} mean {mean:.3g}")


def test_config5_full():
    say("prefill c5 full size, all rows")
    check_config5(4)


@pytest.mark.parametrize("seed", [100, 101, 102, 103, 104])
def test_config5_seeds(seed):
    say("prefill c5 seed", seed)
    check_config5(seed)


@pytest.mark.parametrize("seed", [100, 101, 102, 103, 104])
def test_config3_seeds(seed):
    """Config 3 (store with skipped slots, then chunked prefill over the shared
    prefix chain; all rows, pools bit-exact) at the repeat seeds."""
    say("prefill c3 seed", seed)
    c = w.config3(seed)
    kc, vc = oracle.kv_store(c.k_cache, c.v_cache, c.k, c.v, c.slot_mapping)
    ref = oracle.paged_attn_prefill(c.q, c.k, c.v, kc, vc, c.block_tables, c.context_lens, c.cu_seqlens, c.scale)
    dk, dv = to_dev(c.k_cache), to_dev(c.v_cache)
    pa.kv_store(dk, dv, to_dev(c.k), to_dev(c.v), to_dev(c.slot_mapping))
    out = run_prefill(c, k_cache=dk, v_cache=dv)
    assert torch.equal(bits(dk.cpu()), bits(kc)) and torch.equal(bits(dv.cpu()), bits(vc))
    compare(out, ref, torch.bfloat16)


SHAPES = [
    # hq, hkv, d
    (16, 8, 128), (32, 8, 128), (8, 8, 128), (16, 2, 128), (12, 4, 64), (4, 2, 64), (6, 1, 128),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"hq{s[0]}_hkv{s[1]}_d{s[2]}" for s in SHAPES])
@pytest.mark.parametrize("mix", ["long", "short", "mixed"])
def test_ragged_poisoned(shape, mix):
    hq, hkv, d = shape
    if mix == "long":
        cached, new = [0, 1, 63, 256, 700, 1500], [1, 130, 64, 300, 77, 5]
    elif mix == "short":
        cached, new = [0, 5, 255, 256, 1000, 2047, 3000], [5, 5, 1, 5, 3, 5, 4]
    else:
        cached, new = [300, 0, 2000, 17], [2, 400, 9, 1]
    say("prefill ragged", shape, mix)
    c = poisoned(w.build_prefill_case(f"pf_{mix}", cached, new, hq, hkv, d, torch.bfloat16, 21, with_slots=False))
    compare(run_prefill(c), oracle_prefill(c), torch.bfloat16)


@pytest.mark.parametrize("cfg", ["c3", "c5"])
def test_full_size_repeats_bit_identical(cfg):
    """A split item is merged by whichever of its workgroups finishes last,
    either from the workspace alone or with its own piece still in registers;
    both fold the pieces in piece order with the same arithmetic, so repeated
    launches on the full-size chunked-prefill and verify workloads (where
    that choice varies from launch to launch) give the same bits."""
    say("prefill repeats", cfg)
    c = w.config3(device=DEV) if cfg == "c3" else w.config5(device=DEV)
    first = run_prefill(c)
    for _ in range(7):
        assert torch.equal(bits(first), bits(run_prefill(c)))


# Row-tile kinds the launcher picks from max_q_len * group: 256-row tiles
# (8 waves), 128-row tiles (4 waves) and 32-row tiles (1 wave).
GRID_CASES = {
    "rows256": ([2000, 300, 0, 1500, 777], [300, 129, 200, 64, 1], 16, 8),
    "rows128": ([1800, 0, 900, 3000], [64, 40, 1, 17], 16, 8),
    "rows32": ([2500, 130, 4000, 0, 700], [5, 8, 3, 7, 1], 32, 8),
}
_grid_refs = {}


def _grid_case(kind):
    cached, new, hq, hkv = GRID_CASES[kind]
    c = poisoned(w.build_prefill_case(f"grid_{kind}", cached, new, hq, hkv, 128, torch.bfloat16, 33,
                                      with_slots=False))
    if kind not in _grid_refs:
        _grid_refs[kind] = oracle_prefill(c)
    return c, _grid_refs[kind]


@pytest.mark.parametrize("kind", list(GRID_CASES))
@pytest.mark.parametrize("grid", [1, 2, 3, 7, 50, 131, 1000])
def test_split_items_at_grid_sizes(kind, grid):
    """The split-item protocol (a piece stored and counted when its range's
    first segment ends or when the workgroup ends, or merged at once from
    registers when the other pieces are in; merges of up to many pieces) at
    many grid sizes and all three row-tile kinds: every row against the
    oracle, and a second launch bit-identical to the first."""
    say("prefill grid", kind, grid)
    c, ref = _grid_case(kind)
    q = to_dev(c.q)
    args = (to_dev(c.k), to_dev(c.v), to_dev(c.k_cache), to_dev(c.v_cache), to_dev(c.block_tables),
            to_dev(c.context_lens), to_dev(c.cu_seqlens), c.scale, c.max_q_len, c.max_context_len)
    outs = []
    for _ in range(2):
        out = torch.empty_like(q)
        pa.paged_attn_prefill(out, q, *args, num_workgroups=grid)
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.equal(bits(outs[0]), bits(outs[1]))
    compare(outs[0], ref, torch.bfloat16)


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.5])
def test_zero_negative_and_large_scale(scale):
    """Prefill with the scale as the caller gives it: 0 (every visible key
    weighs 1: the causal mean of V), negative (the library negates q and
    keeps a positive factor) and large; split and unsplit grids against the
    oracle."""
    say("prefill scale", scale)
    c = poisoned(w.build_prefill_case("scale", [700, 0, 1300], [200, 64, 9], 16, 8, 128, torch.bfloat16, 44,
                                      with_slots=False))
    c.scale = scale
    ref = oracle_prefill(c)
    q = to_dev(c.q)
    for grid in (0, 1, 40):
        out = torch.empty_like(q)
        pa.paged_attn_prefill(out, q, to_dev(c.k), to_dev(c.v), to_dev(c.k_cache), to_dev(c.v_cache),
                              to_dev(c.block_tables), to_dev(c.context_lens), to_dev(c.cu_seqlens), scale,
                              c.max_q_len, c.max_context_len, num_workgroups=grid)
        torch.cuda.synchronize()
        compare(out, ref, torch.bfloat16)


def test_block_permutation_and_repeat_bit_identical():
    say("prefill permutation")
    c = w.build_prefill_case("perm", [600, 37, 1200], [100, 5, 260], 16, 8, 128, torch.bfloat16, 5,
                             with_slots=False)
    base = run_prefill(c)
    again = run_prefill(c)
    assert torch.equal(bits(base.cpu()), bits(again.cpu()))
    perm = torch.from_numpy(np.random.default_rng(8).permutation(c.num_blocks))
    kc = torch.empty_like(c.k_cache)
    vc = torch.empty_like(c.v_cache)
    kc[perm] = c.k_cache
    vc[perm] = c.v_cache
    bt = c.block_tables.clone()
    valid = bt >= 0
    bt[valid] = perm[bt[valid].long()].to(torch.int32)
    moved = run_prefill(c, k_cache=to_dev(kc), v_cache=to_dev(vc), block_tables=bt)
    assert torch.equal(bits(base.cpu()), bits(moved.cpu()))


def _full_sequence_case(seed, total, hq, hkv, d):
    """One sequence of `total` tokens: logical K/V rows, queries, and a block list."""
    g = torch.Generator().manual_seed(seed)
    ks = torch.randn((total, hkv, d), generator=g).to(torch.bfloat16)
    vs = torch.randn((total, hkv, d), generator=g).to(torch.bfloat16)
    qs = torch.randn((total, hq, d), generator=g).to(torch.bfloat16)
    nb = -(-total // 256) + 3
    rows = [list(np.random.default_rng(seed).permutation(nb)[: -(-total // 256)])]
    return ks, vs, qs, rows, nb


def _prefill_chunk(ks, vs, qs, rows, nb, c0, c1, scale):
    """Prefill of tokens [c0, c1) over c0 cached tokens."""
    kc = w.paginate([ks[:c0]], rows, nb, fill=0.0) if c0 else torch.zeros((nb, 256) + tuple(ks.shape[1:]),
                                                                          dtype=ks.dtype)
    vc = w.paginate([vs[:c0]], rows, nb, fill=0.0) if c0 else torch.zeros_like(kc)
    case = w.PrefillCase("chunk", qs[c0:c1].contiguous(), ks[c0:c1].contiguous(), vs[c0:c1].contiguous(), kc, vc,
                         w.table_from_rows(rows), torch.tensor([c1], dtype=torch.int32),
                         torch.tensor([0, c1 - c0], dtype=torch.int32), scale)
    return run_prefill(case)


def test_chunked_equals_one_shot():
    """Prefill of [c, c+n) after c cached tokens matches the last n rows of a
    one-shot prefill, and splitting a chunk in two matches too."""
    say("prefill chunked vs one shot")
    hq, hkv, d, total = 16, 8, 128, 900
    ks, vs, qs, rows, nb = _full_sequence_case(31, total, hq, hkv, d)
    scale = 1 / math.sqrt(d)
    one = _prefill_chunk(ks, vs, qs, rows, nb, 0, total, scale).cpu().double()
    for c0 in (1, 64, 255, 600):
        part = _prefill_chunk(ks, vs, qs, rows, nb, c0, total, scale).cpu().double()
        compare(part, one[c0:], torch.bfloat16)
    a = _prefill_chunk(ks, vs, qs, rows, nb, 300, 500, scale).cpu().double()
    b = _prefill_chunk(ks, vs, qs, rows, nb, 500, total, scale).cpu().double()
    compare(torch.cat([a, b]), one[300:], torch.bfloat16)


def test_decode_equals_one_token_prefill_and_verify_equals_decodes():
    say("prefill vs decode")
    hq, hkv, d = 32, 8, 128
    scale = 1 / math.sqrt(d)
    for total in (1, 256, 257, 2000):
        ks, vs, qs, rows, nb = _full_sequence_case(40 + total, total + 5, hq, hkv, d)
        full_k = w.paginate([ks], rows, nb, fill=0.0)
        full_v = w.paginate([vs], rows, nb, fill=0.0)
        bt = w.table_from_rows(rows)
        # verify of 5 drafts after `total` cached tokens
        ver = _prefill_chunk(ks, vs, qs, rows, nb, total, total + 5, scale).cpu().double()
        for j in range(5):
            dec_case = w.DecodeCase("dec", qs[total + j: total + j + 1].contiguous(), full_k, full_v, bt,
                                    torch.tensor([total + j + 1], dtype=torch.int32), scale)
            qd = to_dev(dec_case.q)
            out = torch.empty_like(qd)
            pa.paged_attn_decode(out, qd, to_dev(full_k), to_dev(full_v), to_dev(bt), to_dev(dec_case.context_lens),
                                 scale, total + j + 1)
            torch.cuda.synchronize()
            compare(out.cpu().double(), ver[j: j + 1], torch.bfloat16)


def test_empty_and_zero_length_sequences():
    say("prefill empty")
    c = w.build_prefill_case("zeros", [10, 300, 0], [3, 0, 4], 8, 2, 128, torch.bfloat16, 3, with_slots=False)
    out = run_prefill(c)
    ref = oracle_prefill(c)
    compare(out, ref, torch.bfloat16)
    q = torch.empty((0, 8, 128), dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros((1, 256, 2, 128), dtype=torch.bfloat16, device=DEV)
    pa.paged_attn_prefill(torch.empty_like(q), q, q[:, :2], q[:, :2], kc, kc,
                          torch.zeros((1, 1), dtype=torch.int32, device=DEV),
                          torch.zeros((1,), dtype=torch.int32, device=DEV),
                          torch.zeros((2,), dtype=torch.int32, device=DEV), 0.1, 0, 1)
    torch.cuda.synchronize()


def test_workspace_reused_across_sizes():
    """One prefill workspace, zero-filled once, serves calls of different sizes
    in any order (the counters sit after fixed-size partial regions)."""
    say("prefill workspace reuse")
    few = w.build_prefill_case("pf_few", [300, 1500], [5, 3], 8, 8, 128, torch.bfloat16, 31, with_slots=False)
    many = w.build_prefill_case("pf_many", [1000, 17, 2047, 256, 640, 3000], [40, 300, 5, 64, 2, 9], 12, 4, 64,
                                torch.bfloat16, 32, with_slots=False)
    need = max(pa.prefill_workspace_bytes(len(c.context_lens), c.q.shape[1], c.q.shape[2], c.max_q_len,
                                          c.max_context_len) for c in (few, many))
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for c in (few, many, few, many):
        q = to_dev(c.q)
        out = torch.empty_like(q)
        pa.paged_attn_prefill(out, q, to_dev(c.k), to_dev(c.v), to_dev(c.k_cache), to_dev(c.v_cache),
                              to_dev(c.block_tables), to_dev(c.context_lens), to_dev(c.cu_seqlens), c.scale,
                              c.max_q_len, c.max_context_len, workspace_tensor=ws)
        torch.cuda.synchronize()
        compare(out, oracle_prefill(c), torch.bfloat16)


@pytest.mark.parametrize("shape", [(16, 8, 128), (4, 2, 64)], ids=["hq16_hkv8_d128", "hq4_hkv2_d64"])
@pytest.mark.parametrize("new", [[5, 3, 1], [200, 40, 7]], ids=["verify_rows", "prefill_rows"])
def test_cached_prefix_beyond_64_blocks(shape, new):
    """Cached prefixes longer than 64 blocks (16384 tokens): a segment's block
    ids are read 64 at a time, so these cross a refill of that window."""
    hq, hkv, d = shape
    cached = [17000, 16400, 300]
    say("prefill long prefix", shape, new)
    c = poisoned(w.build_prefill_case("pf_long", cached, new, hq, hkv, d, torch.bfloat16, 23, with_slots=False))
    compare(run_prefill(c), oracle_prefill(c), torch.bfloat16)
