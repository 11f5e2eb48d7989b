"""Pins of the fp8 KV-cache oracle (CPU only).

* The E4M3 value table against values worked by hand from the format's
  definition (bias 7, subnormals m * 2^-9, S.1111.111 = NaN, max 448).
* The quantiser (a library cast) against a brute-force nearest-code search
  over the 254 finite codes with ties to the even code, on random values,
  exact midpoints, subnormals, signed zeros and out-of-range values.
* Decode over fp8 pools equals the plain paged-attention oracle on pools that
  hold the same values exactly; the quantising store round-trips.
* Planted mistakes (no clamp, truncation, wrong bias) fail these pins.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8_kv as f8
import workloads as w

HAND = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2.0 ** -6,
        0x38: 1.0, 0x39: 1.125, 0x40: 2.0, 0x48: 4.0, 0x7E: 448.0, 0x77: 240.0, 0x80: -0.0, 0xB8: -1.0,
        0xFE: -448.0, 0x30: 0.5, 0x3C: 1.5}


def check_table(value_fn):
    for code, v in HAND.items():
        got = value_fn(code)
        assert got == v and math.copysign(1.0, got) == math.copysign(1.0, v), (hex(code), got, v)
    assert math.isnan(value_fn(0x7F)) and math.isnan(value_fn(0xFF))


def test_value_table_hand_worked():
    check_table(f8.e4m3_value)


def brute_force_code(y: float) -> int:
    """Nearest finite code to y (already clamped), ties to the even code."""
    table = f8.e4m3_table()
    best, best_err = None, None
    for c in range(256):
        v = table[c]
        if math.isnan(v):
            continue
        if v == 0.0 and math.copysign(1.0, v) != math.copysign(1.0, y if y != 0 else math.copysign(1.0, y)):
            continue  # the zero of y's sign
        err = abs(y - v)
        if best is None or err < best_err or (err == best_err and (c & 1) == 0 and (best & 1) == 1):
            best, best_err = c, err
    return best


def quantize_cases():
    rng = np.random.default_rng(3)
    vals = list(rng.normal(0, 4, 300)) + list(rng.uniform(-500, 500, 100)) + list(rng.normal(0, 0.01, 100))
    table = f8.e4m3_table()
    finite = sorted(v for v in table if not math.isnan(v))
    mids = [(a + b) / 2 for a, b in zip(finite, finite[1:]) if a != b]
    vals += mids[::3] + [0.0, -0.0, 1000.0, -1000.0, 448.0, 464.0, 2.0 ** -10, -(2.0 ** -10), 3 * 2.0 ** -11]
    return torch.tensor(vals, dtype=torch.float32)


def check_quantizer(qfn):
    x = quantize_cases()
    codes = qfn(x, 1.0)
    for xi, c in zip(x.tolist(), codes.tolist()):
        y = min(max(xi, -448.0), 448.0)
        assert c == brute_force_code(y), (xi, hex(c), hex(brute_force_code(y)))


def test_quantizer_is_nearest_even():
    check_quantizer(f8.quantize)


def test_quantizer_scale_uses_fp32_reciprocal():
    """A value where the reading (1/s formed in fp32, the product rounded to
    fp32, then the nearest code) and exact division disagree, worked by hand.
    s = 0.7 is held as the fp32 0.699999988079071044921875; its fp32
    reciprocal is 1.4285714626312255859375. For x = -17.5 the product
    -25.00000059604644775390625 rounds to the fp32 -25.0, which lies exactly
    halfway between the codes -24 (0xDC, 1.100b x 2^4) and -26 (0xDD,
    1.101b x 2^4): ties go to the even mantissa, 0xDC. Exact division gives
    -25.0000004257..., past the midpoint, hence -26 (0xDD)."""
    assert int(f8.quantize(torch.tensor([-17.5], dtype=torch.float32), 0.7)[0]) == 0xDC
    assert int(f8.quantize(torch.tensor([17.5], dtype=torch.bfloat16), 0.7)[0]) == 0x5C
    assert dividing_quantizer(torch.tensor([-17.5]), 0.7)[0] == 0xDD


def dividing_quantizer(x, s):
    """A plausible mistake: the code nearest to x / s computed exactly (fp64
    division, then the nearest code of the fp64 quotient)."""
    y = np.clip(x.double().numpy() / float(np.float32(s)), -448.0, 448.0)
    table = f8.e4m3_table()
    return [brute_force_code_f64(float(v), table) for v in y]


def brute_force_code_f64(y, table):
    best, best_err = None, None
    for c in range(256):
        v = table[c]
        if math.isnan(v) or (v == 0.0 and math.copysign(1.0, v) != math.copysign(1.0, y)):
            continue
        err = abs(y - v)
        if best is None or err < best_err or (err == best_err and (c & 1) == 0 and (best & 1) == 1):
            best, best_err = c, err
    return best


def test_quantizer_non_finite_hand_worked():
    """Reading of the non-finite inputs: a NaN keeps its sign in the NaN
    pattern S.1111.111 (0x7F, 0xFF); infinities are clamped to +-448 (0x7E,
    0xFE) like every other out-of-range value."""
    pos_nan = torch.tensor([0x7FC00000], dtype=torch.int32).view(torch.float32)
    neg_nan = torch.tensor([-0x400000], dtype=torch.int32).view(torch.float32)  # 0xFFC00000
    x = torch.cat([pos_nan, neg_nan, torch.tensor([float("inf"), -float("inf")])])
    assert f8.quantize(x, 0.05).tolist() == [0x7F, 0xFF, 0x7E, 0xFE]
    assert math.isnan(f8.e4m3_value(0x7F)) and math.isnan(f8.e4m3_value(0xFF))


def test_decode_equals_plain_oracle_on_exact_values():
    """Pools whose values are fp8 values times the scale: the fp8 decode is
    the plain decode of those (exactly representable) float pools."""
    c = w.build_decode_case("fp8pin", [1, 37, 300, 513], 4, 2, 64, torch.float32, 5)
    s_k, s_v = 0.05, 0.125
    kq = f8.quantize(c.k_cache, s_k)
    vq = f8.quantize(c.v_cache, s_v)
    kf = f8.dequantize(kq, s_k)
    vf = f8.dequantize(vq, s_v)
    got = f8.paged_attn_decode_fp8(c.q, kq, vq, c.block_tables, c.context_lens, c.scale, s_k, s_v)
    ref = oracle.paged_attn_decode(c.q.double(), kf, vf, c.block_tables, c.context_lens, c.scale)
    assert torch.allclose(got, ref, rtol=0, atol=1e-12)
    # a one-token context returns that token's dequantised V row
    i = 0
    b0 = int(c.block_tables[i, 0])
    for g in range(4):
        assert torch.equal(got[i, g], vf[b0, 0, g // 2])


def test_store_round_trip():
    g = torch.Generator().manual_seed(4)
    kc = torch.randint(0, 255, (3, 256, 2, 64), generator=g, dtype=torch.uint8)
    vc = torch.randint(0, 255, (3, 256, 2, 64), generator=g, dtype=torch.uint8)
    k = torch.randn(5, 2, 64, generator=g).to(torch.bfloat16)
    v = torch.randn(5, 2, 64, generator=g).to(torch.bfloat16)
    slots = torch.tensor([3, -1, 700, 256, 5], dtype=torch.int32)
    nk, nv = f8.kv_store_fp8(kc, vc, k, v, slots, 0.02, 0.03)
    fk, fv = nk.reshape(-1, 2, 64), nv.reshape(-1, 2, 64)
    for t, s in enumerate(slots.tolist()):
        if s >= 0:
            assert torch.equal(fk[s], f8.quantize(k[t], 0.02)) and torch.equal(fv[s], f8.quantize(v[t], 0.03))
            err = (f8.dequantize(fk[s], 0.02) - k[t].double()).abs()
            assert float(err.max()) <= 0.0625 * float(k[t].double().abs().max()) + 2.0 ** -10 * 0.02
    untouched = torch.ones(fk.shape[0], dtype=torch.bool)
    untouched[[3, 700, 256, 5]] = False
    assert torch.equal(fk[untouched], kc.reshape(-1, 2, 64)[untouched])


# planted mistakes ------------------------------------------------------------
def no_clamp(x, s):
    inv = torch.tensor(float(f8.inverse_scale(s)), dtype=torch.float32)
    return (x.to(torch.float32) * inv).to(torch.float8_e4m3fn).view(torch.uint8)


def truncating(x, s):
    codes = f8.quantize(x, s)
    y = (x.to(torch.float32) * float(f8.inverse_scale(s))).clamp(-448, 448)
    table = torch.from_numpy(f8.e4m3_table())
    over = table[codes.long()].abs() > y.double().abs()
    return torch.where(over & (codes & 0x7F > 0), codes - 1, codes).to(torch.uint8)


def bias8(code):
    v = f8.e4m3_value(code)
    return v / 2 if not math.isnan(v) else v


@pytest.mark.parametrize("mistake", ["no_clamp", "truncating", "bias8"])
def test_planted_mistakes_fail(mistake):
    with pytest.raises(AssertionError):
        if mistake == "bias8":
            check_table(bias8)
        else:
            check_quantizer({"no_clamp": no_clamp, "truncating": truncating}[mistake])
