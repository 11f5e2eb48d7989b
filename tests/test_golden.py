"""The oracle against hand-worked cases in tests/golden/hand_worked.json."""
import json
import os

import torch

import oracle
from workloads import BLOCK_SIZE, paginate, table_from_rows

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")))
f64 = torch.float64


def _close(got, expected, tol):
    exp = torch.tensor(expected, dtype=f64)
    assert got.shape == exp.shape
    assert torch.allclose(got, exp, rtol=0, atol=tol), (got, exp)


def _decode(case, keys, values):
    rows = case["block_rows"]
    kc = paginate([keys], rows, case["num_blocks"])
    vc = paginate([values], rows, case["num_blocks"])
    q = torch.tensor(case["q"], dtype=f64)
    return oracle.paged_attn_decode(q, kc, vc, table_from_rows(rows),
                                    torch.tensor([keys.shape[0]], dtype=torch.int32), case["scale"])


def test_decode_two_keys():
    c = GOLDEN["decode_two_keys"]
    out = _decode(c, torch.tensor(c["context"][0], dtype=f64), torch.tensor(c["values"][0], dtype=f64))
    _close(out, c["expected"], c["tol"])


def test_decode_gqa_grouping():
    c = GOLDEN["decode_gqa_grouping"]
    out = _decode(c, torch.tensor(c["context"][0], dtype=f64), torch.tensor(c["values"][0], dtype=f64))
    _close(out, c["expected"], c["tol"])


def test_decode_across_block_boundary():
    c = GOLDEN["decode_across_block_boundary"]
    L = c["context_len"]
    keys = torch.zeros((L, 1, 1), dtype=f64)
    values = torch.arange(L, dtype=f64).view(L, 1, 1)
    out = _decode(c, keys, values)
    _close(out, c["expected"], c["tol"])


def test_prefill_cached_plus_new():
    c = GOLDEN["prefill_cached_plus_new"]
    rows = c["block_rows"]
    kc = paginate([torch.tensor(c["cached_k"], dtype=f64)], rows, c["num_blocks"])
    vc = paginate([torch.tensor(c["cached_v"], dtype=f64)], rows, c["num_blocks"])
    k = torch.tensor(c["k"], dtype=f64)
    v = torch.tensor(c["v"], dtype=f64)
    q = torch.tensor(c["q"], dtype=f64)
    out = oracle.paged_attn_prefill(q, k, v, kc, vc, table_from_rows(rows), torch.tensor([3], dtype=torch.int32),
                                    torch.tensor([0, 2], dtype=torch.int32), c["scale"])
    _close(out, c["expected"], c["tol"])


def test_kv_store_slots():
    c = GOLDEN["kv_store_slots"]
    nb = c["num_blocks"]
    kc = torch.zeros((nb, BLOCK_SIZE, 1, 1), dtype=torch.float32)
    vc = torch.zeros_like(kc)
    k = torch.tensor(c["k"], dtype=torch.float32)
    v = torch.tensor(c["v"], dtype=torch.float32)
    nk, nv = oracle.kv_store(kc, vc, k, v, torch.tensor(c["slot_mapping"], dtype=torch.int32))
    fk, fv = nk.view(-1, 1, 1), nv.view(-1, 1, 1)
    for s, row in c["expected_k_rows"].items():
        assert fk[int(s)].tolist() == row
    for s, row in c["expected_v_rows"].items():
        assert fv[int(s)].tolist() == row
    written = [int(s) for s in c["expected_k_rows"]]
    mask = torch.ones(nb * BLOCK_SIZE, dtype=torch.bool)
    mask[written] = False
    assert torch.all(fk[mask] == 0) and torch.all(fv[mask] == 0)
