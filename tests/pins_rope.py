"""Pins for the fp64 RoPE oracle (oracle/rotary.py): facts fixed by the
mathematics of a rotation and by closed-form worked examples of the reading
the oracle takes (pairs (i, i + D/2), angle p * base^(-2i/D), (a, b) ->
(a cos t - b sin t, b cos t + a sin t)). The pages only name RoPE ("Nano-vLLM
System Architecture Analysis", section "Differences from Normal nanoGPT
Inference", item 6), so every fact below is either a property any rotary
embedding has or a hand-worked case of that reading. Each pin takes the module
so that the mutation tests can run the same pins against broken copies.
"""
from __future__ import annotations

import math

import torch

TOL = 1e-12


def _x(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64)


def pin_rope_position_zero_is_identity(r):
    x = _x((3, 2, 8), 1)
    out = r.rope(x, torch.zeros(3, dtype=torch.int32), 10000.0)
    assert torch.equal(out, x)


def pin_rope_keeps_pair_lengths(r):
    x = _x((5, 3, 16), 2)
    pos = torch.tensor([0, 1, 7, 300, 16383], dtype=torch.int32)
    out = r.rope(x, pos, 1.0e6)
    h = 8
    n_in = x[..., :h] ** 2 + x[..., h:] ** 2
    n_out = out[..., :h] ** 2 + out[..., h:] ** 2
    assert torch.allclose(n_in, n_out, rtol=0, atol=TOL * 100)


def pin_rope_relative_positions(r):
    """<R(q, m), R(k, n)> depends on m - n only (per head, summed over D)."""
    q, k = _x((1, 1, 32), 3), _x((1, 1, 32), 4)
    for m, n, s in [(5, 2, 11), (100, 0, 1000), (7, 7, 3)]:
        a = (r.rope(q, torch.tensor([m]), 500.0) * r.rope(k, torch.tensor([n]), 500.0)).sum()
        b = (r.rope(q, torch.tensor([m + s]), 500.0) * r.rope(k, torch.tensor([n + s]), 500.0)).sum()
        assert abs(float(a - b)) < 1e-10


def pin_rope_composes(r):
    """Rotating by m and then by n is rotating by m + n."""
    x = _x((2, 1, 8), 5)
    m = torch.tensor([3, 40], dtype=torch.int32)
    n = torch.tensor([9, 2], dtype=torch.int32)
    twice = r.rope(r.rope(x, m, 77.0), n, 77.0)
    once = r.rope(x, m + n, 77.0)
    assert torch.allclose(twice, once, rtol=0, atol=1e-12)


def pin_rope_worked_d4(r):
    """D = 4, base 10000, x = (1, 2, 3, 4), p = 1. theta = (1, 10000^-1/2 =
    0.01): pair (x0, x2) = (1, 3) turns by 1 rad, pair (x1, x3) = (2, 4) by
    0.01 rad."""
    x = torch.tensor([[[1.0, 2.0, 3.0, 4.0]]], dtype=torch.float64)
    out = r.rope(x, torch.tensor([1]), 10000.0).flatten().tolist()
    c1, s1, c2, s2 = math.cos(1.0), math.sin(1.0), math.cos(0.01), math.sin(0.01)
    want = [1 * c1 - 3 * s1, 2 * c2 - 4 * s2, 3 * c1 + 1 * s1, 4 * c2 + 2 * s2]
    assert max(abs(a - b) for a, b in zip(out, want)) < TOL


def pin_rope_worked_d8(r):
    """D = 8, base 16, p = 2, x = e0 + e5: theta_i = 16^(-i/4) = 2^-i. Pair 0
    (x0, x4) = (1, 0) turns by 2 rad -> (cos 2, sin 2); pair 1 (x1, x5) =
    (0, 1) by 1 rad -> (-sin 1, cos 1); pairs 2 and 3 stay zero."""
    x = torch.zeros(1, 1, 8, dtype=torch.float64)
    x[0, 0, 0] = 1.0
    x[0, 0, 5] = 1.0
    out = r.rope(x, torch.tensor([2]), 16.0).flatten().tolist()
    want = [math.cos(2.0), -math.sin(1.0), 0.0, 0.0, math.sin(2.0), math.cos(1.0), 0.0, 0.0]
    assert max(abs(a - b) for a, b in zip(out, want)) < TOL


def pin_rope_kv_store_placement(r):
    """The stored K row is the rotated k, the stored V row the plain v; a
    negative slot stores nothing but its query is still rotated; the rest of
    both pools is untouched."""
    t, hq, hkv, d, nb = 3, 4, 2, 8, 2
    q, k, v = _x((t, hq, d), 6), _x((t, hkv, d), 7), _x((t, hkv, d), 8)
    kc, vc = _x((nb, 256, hkv, d), 9), _x((nb, 256, hkv, d), 10)
    pos = torch.tensor([4, 0, 9], dtype=torch.int32)
    slots = torch.tensor([300, -1, 5], dtype=torch.int32)
    qo, kc2, vc2 = r.rope_kv_store(q, k, v, pos, kc, vc, slots, 1000.0)
    assert torch.equal(qo, r.rope(q, pos, 1000.0))
    kr = r.rope(k, pos, 1000.0)
    assert torch.equal(kc2[1, 44], kr[0]) and torch.equal(kc2[0, 5], kr[2])
    assert torch.equal(vc2[1, 44], v[0]) and torch.equal(vc2[0, 5], v[2])
    touched = torch.zeros(nb, 256, dtype=torch.bool)
    touched[1, 44] = touched[0, 5] = True
    assert torch.equal(kc2[~touched], kc[~touched]) and torch.equal(vc2[~touched], vc[~touched])


def pin_norm_unit_mean_square(r):
    """Weight 1 and eps 0: every normalised head row has mean square 1."""
    x = _x((4, 3, 16), 11) * 5.0
    out = r.rms_norm(x, torch.ones(16, dtype=torch.float64), 0.0)
    assert torch.allclose((out * out).mean(dim=-1), torch.ones(4, 3, dtype=torch.float64), rtol=0, atol=1e-13)


def pin_norm_scale_invariant(r):
    """eps 0: scaling a row by c > 0 does not change its normalised value."""
    x = _x((2, 2, 8), 12)
    w = _x((8,), 13)
    assert torch.allclose(r.rms_norm(3.7 * x, w, 0.0), r.rms_norm(x, w, 0.0), rtol=0, atol=1e-13)


def pin_norm_matches_library(r):
    """The library's RMSNorm (torch, float64) over the last dimension."""
    x = _x((3, 4, 32), 14)
    w = _x((32,), 15)
    ref = torch.nn.functional.rms_norm(x, (32,), w, 1e-6)
    assert torch.allclose(r.rms_norm(x, w, 1e-6), ref, rtol=0, atol=1e-13)


def pin_qknorm_rope_worked_d4(r):
    """D = 4, x = (1, 2, 3, 4), weight (1, 2, 1, 0.5), eps 0.5, base 10000,
    p = 1, worked by hand: mean square 7.5, + eps = 8, so x / sqrt 8 * w =
    (1, 4, 3, 2) / (2 sqrt 2); pairs (x0, x2) turn by 1 rad and (x1, x3) by
    10000^(-1/2) = 0.01 rad."""
    x = torch.tensor([[[1.0, 2.0, 3.0, 4.0]]], dtype=torch.float64)
    w = torch.tensor([1.0, 2.0, 1.0, 0.5], dtype=torch.float64)
    z = torch.zeros(1, 1, 4, dtype=torch.float64)
    kc = torch.zeros(1, 256, 1, 4, dtype=torch.float64)
    q_rot, kcache, _ = r.qknorm_rope_kv_store(x, x, z, torch.tensor([1], dtype=torch.int32), kc, kc.clone(),
                                              torch.tensor([5], dtype=torch.int32), 10000.0, w, w, 0.5)
    c = 2.0 * math.sqrt(2.0)
    a, b = 1.0, 0.01
    want = torch.tensor([(1 * math.cos(a) - 3 * math.sin(a)) / c, (4 * math.cos(b) - 2 * math.sin(b)) / c,
                         (3 * math.cos(a) + 1 * math.sin(a)) / c, (2 * math.cos(b) + 4 * math.sin(b)) / c],
                        dtype=torch.float64)
    assert torch.allclose(q_rot[0, 0], want, rtol=0, atol=1e-14)
    assert torch.allclose(kcache[0, 5, 0], want, rtol=0, atol=1e-14)


PINS = [
    pin_norm_unit_mean_square,
    pin_norm_scale_invariant,
    pin_norm_matches_library,
    pin_qknorm_rope_worked_d4,
    pin_rope_position_zero_is_identity,
    pin_rope_keeps_pair_lengths,
    pin_rope_relative_positions,
    pin_rope_composes,
    pin_rope_worked_d4,
    pin_rope_worked_d8,
    pin_rope_kv_store_placement,
]
