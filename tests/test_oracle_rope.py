"""The fp64 RoPE oracle against its pins (tests/pins_rope.py), and mutation
tests: each plants one plausible mistake in a copy of oracle/rotary.py (on the
CPU) and checks that some pin fails."""
import os
import types

import pytest

import oracle.rotary
from pins_rope import PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "rotary.py")

MUTATIONS = {
    "interleaved_pairs": ("a, b = x64[..., :half], x64[..., half:]", "a, b = x64[..., 0::2], x64[..., 1::2]"),
    "sine_sign_flipped": ("a * cos - b * sin, b * cos + a * sin", "a * cos + b * sin, b * cos - a * sin"),
    "not_a_rotation": ("a * cos - b * sin, b * cos + a * sin", "a * cos - b * sin, b * cos - a * sin"),
    "theta_exponent_halved": ("base ** (-2.0 * i / head_dim)", "base ** (-1.0 * i / head_dim)"),
    "theta_reversed": ("for i in range(half)]", "for i in reversed(range(half))]"),
    "position_shifted": ("positions.to(torch.float64).reshape(-1, 1)", "(positions.to(torch.float64) + 1).reshape(-1, 1)"),
    "v_rotated": ("kv_store(k_cache, v_cache, k_rot, v, slot_mapping)",
                  "kv_store(k_cache, v_cache, k_rot, rope(v, positions, base).to(v.dtype), slot_mapping)"),
    "k_stored_plain": ("kv_store(k_cache, v_cache, k_rot, v, slot_mapping)", "kv_store(k_cache, v_cache, k, v, slot_mapping)"),
    "norm_eps_dropped": ("torch.sqrt(ms + eps)", "torch.sqrt(ms)"),
    "norm_sum_not_mean": ("(x64 * x64).mean(dim=-1, keepdim=True)", "(x64 * x64).sum(dim=-1, keepdim=True)"),
    "norm_over_heads": ("(x64 * x64).mean(dim=-1, keepdim=True)", "(x64 * x64).mean(dim=(-2, -1), keepdim=True)"),
    "norm_weight_dropped": ("/ torch.sqrt(ms + eps) * weight.to(torch.float64)", "/ torch.sqrt(ms + eps)"),
    "norm_after_rope": ("q_rot = rope(rms_norm(q, q_weight, eps), positions, base).to(q.dtype)",
                        "q_rot = rms_norm(rope(q, positions, base).unsqueeze(0)[0], q_weight, eps).to(q.dtype)"),
}


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle.rotary)


def _mutant(name):
    old, new = MUTATIONS[name]
    text = open(SRC).read()
    assert old in text, f"mutation anchor for {name} not found"
    mod = types.ModuleType(f"oracle.rotary_mutant_{name}")
    mod.__package__ = "oracle"
    exec(compile(text.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_catches(name):
    mod = _mutant(name)
    failed = []
    for pin in PINS:
        try:
            pin(mod)
        except Exception:  # an assertion or a crash both count as caught
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutation {name}"
