"""Helpers for the GPU parity tests: move seeded cases to the device, run the
HIP path through the binding, and compare with the fp64 oracle."""
import sys

import torch

DEV = "cuda:0"

# Tolerances of the parity bar: fp32 inputs max-abs 1e-5; bf16 inputs (fp32
# accumulation) max-abs 2e-2 and mean-abs 2e-3 over all compared elements.
TOL = {torch.float32: (1e-5, None), torch.bfloat16: (2e-2, 2e-3)}


def say(*args):
    print(*args, file=sys.stderr, flush=True)


def to_dev(t):
    return None if t is None else t.to(DEV, non_blocking=False).contiguous()


def compare(got, ref, dtype, rows=None):
    """Compare a device output with an fp64 oracle result (CPU). `rows` selects
    the leading-dimension rows the oracle computed."""
    g = got.detach().to("cpu", torch.float64)
    r = ref
    if rows is not None:
        idx = torch.as_tensor(list(rows), dtype=torch.long)
        g, r = g[idx], r[idx]
    assert torch.isfinite(g).all(), "non-finite output"
    err = (g - r).abs()
    max_tol, mean_tol = TOL[dtype]
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= max_tol, f"max abs err {mx:.3g} > {max_tol}"
    if mean_tol is not None:
        assert mean <= mean_tol, f"mean abs err {mean:.3g} > {mean_tol}"
    return mx, mean


def bits(t):
    return t.view({2: torch.int16, 4: torch.int32}[t.element_size()])
