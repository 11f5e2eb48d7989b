"""Mutation tests for the oracle's pins.

Each case plants one plausible mistake in a copy of the oracle's source (on the
CPU, never in the product path) and checks that at least one pin fails. This
shows the pins are strong enough that a dropped term, a wrong index or sign,
or a swapped operand in the oracle could not go unnoticed.
"""
import importlib.util
import os
import types

import pytest

from pins import PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "paged_attention.py")

MUTATIONS = {
    "gqa_modulo_mapping": ("for g in range(h * group, (h + 1) * group):", "for g in range(h, hq, hkv):"),
    "scale_dropped": ("scores = (q64 @ k64.T) * scale", "scores = (q64 @ k64.T)"),
    "causal_mask_dropped": ("visible = [cached + j + 1 for j in range(n)]", "visible = [cached + n for j in range(n)]"),
    "causal_off_by_one": ("visible = [cached + j + 1 for j in range(n)]",
                          "visible = [cached + j + (2 if j + 1 < n else 1) for j in range(n)]"),
    "block_order_reversed": ("ids = [int(b) for b in block_row[:nblk].tolist()]",
                             "ids = [int(b) for b in block_row[:nblk].tolist()][::-1]"),
    "cached_len_misread": ("cached = int(context_lens[i]) - n", "cached = max(0, int(context_lens[i]) - n - 1)"),
    "values_are_keys": ("return (weights @ v64) / weights.sum(dim=1, keepdim=True)",
                        "return (weights @ k64) / weights.sum(dim=1, keepdim=True)"),
    "normalisation_dropped": ("return (weights @ v64) / weights.sum(dim=1, keepdim=True)",
                              "return (weights @ v64)"),
    "slot_divmod_swapped": ("block, row = divmod(s, bs)", "row, block = divmod(s, bs)"),
    "skip_ignored": ("        if s < 0:\n            continue\n        block, row", "        block, row"),
    "v_pool_gets_k": ("vcb[block, row] = vb[t]", "vcb[block, row] = kb[t]"),
    "decode_drops_last_token": ("keys = gather_sequence(k_cache[:, :, h, :], block_tables[i], length)\n",
                                "keys = gather_sequence(k_cache[:, :, h, :], block_tables[i], length)\n"
                                "            keys = keys.clone(); keys[-1] = keys[0] if length > 1 else keys[-1]\n"),
    "new_keys_from_values": ("k[start:end, h, :].to(torch.float64)], dim=0)", "v[start:end, h, :].to(torch.float64)], dim=0)"),
    "new_keys_wrong_head": ("keys = torch.cat([old_k.to(torch.float64), k[start:end, h, :]",
                            "keys = torch.cat([old_k.to(torch.float64), k[start:end, 0, :]"),
    "block_rows_shifted": ("rows = torch.cat([head_pool[b] for b in ids], dim=0)",
                           "rows = torch.cat([head_pool[b].roll(1, dims=0) for b in ids], dim=0)"),
    "softmax_max_not_subtracted_per_row": ("scores = scores - scores.max(dim=1, keepdim=True).values",
                                           "scores = scores - scores.max(dim=0, keepdim=True).values"),
}


def _mutant(name):
    old, new = MUTATIONS[name]
    text = open(SRC).read()
    assert old in text, f"mutation anchor for {name} not found"
    text = text.replace(old, new)
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(text, f"<mutant {name}>", "exec"), mod.__dict__)
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
