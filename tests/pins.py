"""Pins for the fp64 oracle: facts fixed by the pages or by mathematics that the
oracle must reproduce. Each pin takes the oracle module as an argument so that
the mutation tests can run the same pins against deliberately broken copies.

Sources: attention = softmax(q k^T) v (Baidu article on Nano-vLLM, section
"TorchScript Optimization"); paged store/gather semantics and 256-token blocks
("Nano-vLLM System Architecture Analysis", section 2, "Paged KV Cache" and
"Attention with Paged Cache"); chunked prefill ("Scheduler", same section);
speculative verify as a mini-prefill ("What Is an Inference Engine, Anyway?",
Technical details); GQA (same analysis page, "Differences", item 6).
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F

from workloads import BLOCK_SIZE, paginate, table_from_rows

TOL = 1e-12


# ---------------------------------------------------------------------------
# tiny case builders (logical sequences first, then paged)
# ---------------------------------------------------------------------------


def _rand(shape, gen, dtype=torch.float64):
    return torch.randn(shape, generator=gen, dtype=torch.float64).to(dtype)


def _block_rows(lengths, num_blocks, rng, shared=None):
    """Shuffled block ids for each length; `shared` = (seq_a, seq_b, nblocks)
    makes seq_b reuse seq_a's first nblocks ids."""
    need = [-(-L // BLOCK_SIZE) for L in lengths]
    ids = list(rng.permutation(num_blocks)[: sum(need)])
    rows, pos = [], 0
    for n in need:
        rows.append([int(x) for x in ids[pos : pos + n]])
        pos += n
    if shared is not None:
        a, b, m = shared
        rows[b][:m] = rows[a][:m]
    return rows


def tiny_decode(seed=0, lengths=(1, 5, 300, 513), hq=4, hkv=2, d=4, scale=0.7, dtype=torch.float64):
    gen = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    nb = 12
    rows = _block_rows(lengths, nb, rng)
    ks = [_rand((L, hkv, d), gen, dtype) for L in lengths]
    vs = [_rand((L, hkv, d), gen, dtype) for L in lengths]
    q = _rand((len(lengths), hq, d), gen, dtype)
    return dict(q=q, ks=ks, vs=vs, rows=rows, nb=nb, scale=scale, lengths=list(lengths),
                k_cache=paginate(ks, rows, nb), v_cache=paginate(vs, rows, nb),
                block_tables=table_from_rows(rows),
                context_lens=torch.tensor(lengths, dtype=torch.int32))


def tiny_prefill(seed=1, cached=(0, 3, 260, 256), new=(4, 1, 6, 3), hq=4, hkv=2, d=4, scale=0.55,
                 dtype=torch.float64):
    gen = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    nb = 10
    totals = [c + n for c, n in zip(cached, new)]
    rows = _block_rows(totals, nb, rng)
    ks = [_rand((L, hkv, d), gen, dtype) for L in totals]
    vs = [_rand((L, hkv, d), gen, dtype) for L in totals]
    q = _rand((sum(new), hq, d), gen, dtype)
    cu = [0]
    for n in new:
        cu.append(cu[-1] + n)
    # the pool holds only the cached part; new K/V travel with the call
    kc = paginate([k[:c] for k, c in zip(ks, cached)], rows, nb)
    vc = paginate([v[:c] for v, c in zip(vs, cached)], rows, nb)
    k_new = torch.cat([k[c:] for k, c in zip(ks, cached)])
    v_new = torch.cat([v[c:] for v, c in zip(vs, cached)])
    return dict(q=q, k=k_new, v=v_new, ks=ks, vs=vs, rows=rows, nb=nb, scale=scale, cached=list(cached),
                new=list(new), k_cache=kc, v_cache=vc, block_tables=table_from_rows(rows),
                context_lens=torch.tensor(totals, dtype=torch.int32),
                cu_seqlens=torch.tensor(cu, dtype=torch.int32))


def run_decode(orc, c, **over):
    a = dict(c)
    a.update(over)
    return orc.paged_attn_decode(a["q"], a["k_cache"], a["v_cache"], a["block_tables"], a["context_lens"],
                                 a["scale"])


def run_prefill(orc, c, **over):
    a = dict(c)
    a.update(over)
    return orc.paged_attn_prefill(a["q"], a["k"], a["v"], a["k_cache"], a["v_cache"], a["block_tables"],
                                  a["context_lens"], a["cu_seqlens"], a["scale"])


# ---------------------------------------------------------------------------
# independent references
# ---------------------------------------------------------------------------


def brute_attend(qv, keys, values, scale):
    """Pure-Python softmax attention of one query vector over lists of rows."""
    s = [scale * math.fsum(a * b for a, b in zip(qv, k)) for k in keys]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    z = math.fsum(w)
    return [math.fsum(w[t] * values[t][e] for t in range(len(values))) / z for e in range(len(values[0]))]


def sdpa_reference(qh, kh, vh, scale, cached):
    """torch SDPA (CPU, fp64) with an explicit bottom-right causal mask.
    qh [H, n, D], kh/vh [H, cached + n, D]."""
    n, L = qh.shape[1], kh.shape[1]
    mask = torch.arange(L)[None, :] <= (cached + torch.arange(n))[:, None]
    return F.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask, scale=scale)


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------


def pin_decode_brute_force(orc):
    """P1: paged decode equals a pure-Python loop over the logical sequence."""
    c = tiny_decode()
    out = run_decode(orc, c)
    g = c["q"].shape[1] // c["ks"][0].shape[1]
    for i, L in enumerate(c["lengths"]):
        for h in range(c["q"].shape[1]):
            kv = h // g
            ref = brute_attend(c["q"][i, h].tolist(), c["ks"][i][:, kv].tolist(), c["vs"][i][:, kv].tolist(),
                               c["scale"])
            assert torch.allclose(out[i, h], torch.tensor(ref, dtype=torch.float64), rtol=0, atol=TOL), (i, h)


def pin_prefill_brute_force(orc):
    """P1: paged prefill equals a pure-Python causal loop over the logical sequence."""
    c = tiny_prefill()
    out = run_prefill(orc, c)
    g = c["q"].shape[1] // c["ks"][0].shape[1]
    cu = c["cu_seqlens"].tolist()
    for i, (cached, n) in enumerate(zip(c["cached"], c["new"])):
        for j in range(n):
            for h in range(c["q"].shape[1]):
                kv = h // g
                vis = cached + j + 1
                ref = brute_attend(c["q"][cu[i] + j, h].tolist(), c["ks"][i][:vis, kv].tolist(),
                                   c["vs"][i][:vis, kv].tolist(), c["scale"])
                got = out[cu[i] + j, h]
                assert torch.allclose(got, torch.tensor(ref, dtype=torch.float64), rtol=0, atol=TOL), (i, j, h)


def pin_prefill_matches_sdpa(orc):
    """P1: paged prefill equals torch's fp64 SDPA on the contiguous sequence with
    KV heads repeated per group (library routine)."""
    c = tiny_prefill(seed=7, cached=(5, 0, 257), new=(3, 7, 2), hq=6, hkv=3, d=5)
    out = run_prefill(orc, c)
    g = 2
    cu = c["cu_seqlens"].tolist()
    for i, (cached, n) in enumerate(zip(c["cached"], c["new"])):
        qh = c["q"][cu[i] : cu[i + 1]].permute(1, 0, 2)
        kh = c["ks"][i].repeat_interleave(g, dim=1).permute(1, 0, 2)
        vh = c["vs"][i].repeat_interleave(g, dim=1).permute(1, 0, 2)
        ref = sdpa_reference(qh, kh, vh, c["scale"], cached).permute(1, 0, 2)
        assert torch.allclose(out[cu[i] : cu[i + 1]], ref, rtol=0, atol=TOL), i


def pin_decode_matches_sdpa(orc):
    """P1: paged decode equals torch's fp64 SDPA over the gathered context."""
    c = tiny_decode(seed=3, lengths=(2, 256, 257, 700), hq=6, hkv=2, d=8)
    out = run_decode(orc, c)
    for i, L in enumerate(c["lengths"]):
        qh = c["q"][i].unsqueeze(1)  # [H, 1, D]
        kh = c["ks"][i].repeat_interleave(3, dim=1).permute(1, 0, 2)
        vh = c["vs"][i].repeat_interleave(3, dim=1).permute(1, 0, 2)
        ref = sdpa_reference(qh, kh, vh, c["scale"], L - 1)[:, 0]
        assert torch.allclose(out[i], ref, rtol=0, atol=TOL), i


def pin_block_permutation(orc):
    """P2: relabelling pool blocks (and the tables with them) leaves the output
    bit-identical."""
    c = tiny_decode(seed=5)
    base = run_decode(orc, c)
    perm = torch.from_numpy(np.random.default_rng(11).permutation(c["nb"]))
    kc = torch.empty_like(c["k_cache"])
    vc = torch.empty_like(c["v_cache"])
    kc[perm] = c["k_cache"]
    vc[perm] = c["v_cache"]
    bt = c["block_tables"].clone()
    valid = bt >= 0
    bt[valid] = perm[bt[valid].long()].to(torch.int32)
    moved = run_decode(orc, c, k_cache=kc, v_cache=vc, block_tables=bt)
    assert torch.equal(base, moved)
    p = tiny_prefill(seed=6)
    base = run_prefill(orc, p)
    kc = torch.empty_like(p["k_cache"])
    vc = torch.empty_like(p["v_cache"])
    perm = torch.from_numpy(np.random.default_rng(12).permutation(p["nb"]))
    kc[perm] = p["k_cache"]
    vc[perm] = p["v_cache"]
    bt = p["block_tables"].clone()
    valid = bt >= 0
    bt[valid] = perm[bt[valid].long()].to(torch.int32)
    assert torch.equal(base, run_prefill(orc, p, k_cache=kc, v_cache=vc, block_tables=bt))


def pin_shared_prefix(orc):
    """P3: sequences whose tables share prefix block ids give the same output
    as private copies of those blocks; equal tokens and queries give equal rows."""
    gen = torch.Generator().manual_seed(21)
    hkv, hq, d = 2, 4, 4
    prefix_k = _rand((512, hkv, d), gen)
    prefix_v = _rand((512, hkv, d), gen)
    tails_k = [_rand((t, hkv, d), gen) for t in (40, 300)]
    tails_v = [_rand((t, hkv, d), gen) for t in (40, 300)]
    ks = [torch.cat([prefix_k, t]) for t in tails_k]
    vs = [torch.cat([prefix_v, t]) for t in tails_v]
    q = _rand((2, hq, d), gen)
    lengths = [k.shape[0] for k in ks]
    shared_rows = [[7, 2, 5], [7, 2, 0, 9]]
    private_rows = [[7, 2, 5], [1, 3, 0, 9]]
    ctx = torch.tensor(lengths, dtype=torch.int32)
    out_shared = orc.paged_attn_decode(q, paginate(ks, shared_rows, 10), paginate(vs, shared_rows, 10),
                                       table_from_rows(shared_rows), ctx, 0.4)
    out_private = orc.paged_attn_decode(q, paginate(ks, private_rows, 10), paginate(vs, private_rows, 10),
                                        table_from_rows(private_rows), ctx, 0.4)
    assert torch.equal(out_shared, out_private)
    # two identical sequences sharing every block, same queries -> identical rows
    q2 = torch.stack([q[0], q[0]])
    rows = [[4, 6, 8], [4, 6, 8]]
    out = orc.paged_attn_decode(q2, paginate([ks[0], ks[0]], rows, 10), paginate([vs[0], vs[0]], rows, 10),
                                table_from_rows(rows), torch.tensor([lengths[0]] * 2, dtype=torch.int32), 0.4)
    assert torch.equal(out[0], out[1])
    # and the shared-prefix row of sequence 0 agrees with a fully private layout
    assert torch.equal(out[0], out_private[0])


def pin_one_token_context(orc):
    """P4: with one visible key the softmax weight is exactly 1, so the output
    is that token's V row, bit for bit."""
    c = tiny_decode(seed=8, lengths=(1, 1, 1), hq=4, hkv=2, d=6, dtype=torch.float32)
    out = run_decode(orc, c)
    for i in range(3):
        for h in range(4):
            assert torch.equal(out[i, h], c["vs"][i][0, h // 2].to(torch.float64))
    p = tiny_prefill(seed=9, cached=(0, 0), new=(1, 3), hq=2, hkv=1, d=3)
    out = run_prefill(orc, p)
    assert torch.equal(out[0, 0], p["v"][0, 0]) and torch.equal(out[1, 1], p["v"][1, 0])


def pin_zero_query_mean(orc):
    """P5: q = 0 (or scale = 0) makes every visible weight equal, so each output
    row is the mean of the visible V rows."""
    c = tiny_decode(seed=10)
    zq = torch.zeros_like(c["q"])
    out = run_decode(orc, c, q=zq)
    out2 = run_decode(orc, c, scale=0.0)
    g = 2
    for i, L in enumerate(c["lengths"]):
        for h in range(c["q"].shape[1]):
            mean = c["vs"][i][:, h // g].mean(dim=0)
            assert torch.allclose(out[i, h], mean, rtol=0, atol=TOL)
            assert torch.allclose(out2[i, h], mean, rtol=0, atol=TOL)
    p = tiny_prefill(seed=11)
    out = run_prefill(orc, p, q=torch.zeros_like(p["q"]))
    cu = p["cu_seqlens"].tolist()
    for i, (cached, n) in enumerate(zip(p["cached"], p["new"])):
        for j in range(n):
            for h in range(p["q"].shape[1]):
                mean = p["vs"][i][: cached + j + 1, h // 2].mean(dim=0)
                assert torch.allclose(out[cu[i] + j, h], mean, rtol=0, atol=TOL)


def pin_constant_values(orc):
    """P6: if every V row equals v0 the output is v0 whatever the weights."""
    c = tiny_decode(seed=12)
    v0 = torch.tensor([0.5, -1.25, 3.0, 2.0], dtype=torch.float64)
    vc = torch.empty_like(c["v_cache"])
    vc[:] = v0
    out = run_decode(orc, c, v_cache=vc)
    assert torch.allclose(out, v0.expand_as(out), rtol=0, atol=TOL)
    p = tiny_prefill(seed=13)
    vcp = torch.empty_like(p["v_cache"])
    vcp[:] = v0
    vnew = torch.empty_like(p["v"])
    vnew[:] = v0
    out = run_prefill(orc, p, v_cache=vcp, v=vnew)
    assert torch.allclose(out, v0.expand_as(out), rtol=0, atol=TOL)


def pin_gqa_equals_repeated_mha(orc):
    """P7: grouped-query attention equals multi-head attention over KV heads
    repeated group-wise (query head g reads KV head g // group)."""
    c = tiny_decode(seed=14, hq=6, hkv=2)
    out = run_decode(orc, c)
    rep = run_decode(orc, c, k_cache=c["k_cache"].repeat_interleave(3, dim=2),
                     v_cache=c["v_cache"].repeat_interleave(3, dim=2))
    assert torch.equal(out, rep)
    p = tiny_prefill(seed=15, hq=6, hkv=3)
    out = run_prefill(orc, p)
    rep = run_prefill(orc, p, k_cache=p["k_cache"].repeat_interleave(2, dim=2),
                      v_cache=p["v_cache"].repeat_interleave(2, dim=2),
                      k=p["k"].repeat_interleave(2, dim=1), v=p["v"].repeat_interleave(2, dim=1))
    assert torch.equal(out, rep)


def pin_decode_equals_prefill_of_one(orc):
    """P8: a decode step over L tokens equals a prefill of one new token after
    L - 1 cached tokens (the last token's K/V passed in flight)."""
    c = tiny_decode(seed=16, lengths=(3, 257, 512))
    dec = run_decode(orc, c)
    lengths = c["lengths"]
    kc = paginate([k[: L - 1] for k, L in zip(c["ks"], lengths)], c["rows"], c["nb"])
    vc = paginate([v[: L - 1] for v, L in zip(c["vs"], lengths)], c["rows"], c["nb"])
    k_new = torch.stack([k[L - 1] for k, L in zip(c["ks"], lengths)])
    v_new = torch.stack([v[L - 1] for v, L in zip(c["vs"], lengths)])
    cu = torch.arange(len(lengths) + 1, dtype=torch.int32)
    pre = orc.paged_attn_prefill(c["q"], k_new, v_new, kc, vc, c["block_tables"], c["context_lens"], cu,
                                 c["scale"])
    assert torch.allclose(dec, pre, rtol=0, atol=TOL)


def pin_chunked_equals_one_shot(orc):
    """P9: prefill of [c, c+n) over c cached tokens equals the last n rows of a
    one-shot causal prefill of c+n tokens; splitting the chunk in two gives the
    same rows."""
    gen = torch.Generator().manual_seed(17)
    hq, hkv, d, total = 4, 2, 4, 300
    ks, vs = _rand((total, hkv, d), gen), _rand((total, hkv, d), gen)
    q = _rand((total, hq, d), gen)
    rows = [[3, 1]]
    bt = table_from_rows(rows)
    one = orc.paged_attn_prefill(q, ks, vs, paginate([ks[:0]], rows, 4), paginate([vs[:0]], rows, 4), bt,
                                 torch.tensor([total], dtype=torch.int32),
                                 torch.tensor([0, total], dtype=torch.int32), 0.6)
    for c0 in (1, 255, 256, 290):
        part = orc.paged_attn_prefill(q[c0:], ks[c0:], vs[c0:], paginate([ks[:c0]], rows, 4),
                                      paginate([vs[:c0]], rows, 4), bt, torch.tensor([total], dtype=torch.int32),
                                      torch.tensor([0, total - c0], dtype=torch.int32), 0.6)
        assert torch.allclose(part, one[c0:], rtol=0, atol=TOL), c0
    # split [200, 300) into [200, 250) and [250, 300)
    a = orc.paged_attn_prefill(q[200:250], ks[200:250], vs[200:250], paginate([ks[:200]], rows, 4),
                               paginate([vs[:200]], rows, 4), bt, torch.tensor([250], dtype=torch.int32),
                               torch.tensor([0, 50], dtype=torch.int32), 0.6)
    b = orc.paged_attn_prefill(q[250:], ks[250:], vs[250:], paginate([ks[:250]], rows, 4),
                               paginate([vs[:250]], rows, 4), bt, torch.tensor([300], dtype=torch.int32),
                               torch.tensor([0, 50], dtype=torch.int32), 0.6)
    assert torch.allclose(torch.cat([a, b]), one[200:], rtol=0, atol=TOL)


def pin_verify_equals_decodes(orc):
    """P10: verifying 5 drafts causally equals 5 decode steps at contexts
    c+1 .. c+5 after the drafts' K/V are stored."""
    p = tiny_prefill(seed=18, cached=(251, 3), new=(5, 5))
    ver = run_prefill(orc, p)
    cu = p["cu_seqlens"].tolist()
    full_k = paginate(p["ks"], p["rows"], p["nb"])
    full_v = paginate(p["vs"], p["rows"], p["nb"])
    for j in range(5):
        q = torch.stack([p["q"][cu[i] + j] for i in range(2)])
        ctx = torch.tensor([c + j + 1 for c in p["cached"]], dtype=torch.int32)
        dec = orc.paged_attn_decode(q, full_k, full_v, p["block_tables"], ctx, p["scale"])
        for i in range(2):
            assert torch.allclose(ver[cu[i] + j], dec[i], rtol=0, atol=TOL), (i, j)


def pin_kv_store_round_trip(orc):
    """P11: stored rows read back bit-exactly through their slots; skipped (-1)
    tokens and every other slot keep the pool's previous bytes."""
    gen = torch.Generator().manual_seed(19)
    for dtype in (torch.float32, torch.bfloat16):
        nb, hkv, d = 3, 2, 8
        kc = torch.full((nb, BLOCK_SIZE, hkv, d), -7.0, dtype=dtype)
        vc = torch.full((nb, BLOCK_SIZE, hkv, d), 9.0, dtype=dtype)
        k = _rand((5, hkv, d), gen, dtype)
        v = _rand((5, hkv, d), gen, dtype)
        k[1, 0, 0] = float("nan")
        slots = torch.tensor([0, 257, -1, 766, 300], dtype=torch.int32)
        nk, nv = orc.kv_store(kc, vc, k, v, slots)
        bits = {2: torch.int16, 4: torch.int32}[k.element_size()]
        touched = torch.zeros(nb * BLOCK_SIZE, dtype=torch.bool)
        for t, s in enumerate(slots.tolist()):
            if s < 0:
                continue
            touched[s] = True
            assert torch.equal(nk.view(-1, hkv, d)[s].view(bits), k[t].view(bits))
            assert torch.equal(nv.view(-1, hkv, d)[s].view(bits), v[t].view(bits))
        assert torch.equal(nk.view(-1, hkv, d)[~touched].view(bits), kc.view(-1, hkv, d)[~touched].view(bits))
        assert torch.equal(nv.view(-1, hkv, d)[~touched].view(bits), vc.view(-1, hkv, d)[~touched].view(bits))
        assert int(touched.sum()) == 4
        # the inputs themselves are untouched
        assert torch.all(kc == -7.0) and torch.all(vc == 9.0)


PINS = [
    pin_decode_brute_force,
    pin_prefill_brute_force,
    pin_prefill_matches_sdpa,
    pin_decode_matches_sdpa,
    pin_block_permutation,
    pin_shared_prefix,
    pin_one_token_context,
    pin_zero_query_mean,
    pin_constant_values,
    pin_gqa_equals_repeated_mha,
    pin_decode_equals_prefill_of_one,
    pin_chunked_equals_one_shot,
    pin_verify_equals_decodes,
    pin_kv_store_round_trip,
]
