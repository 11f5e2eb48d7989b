"""Plain CPU oracle for an fp8 KV cache: quantising store and decode attention
over the dequantised pools.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module:
only the tests, the smoke check of the package entry file and the CPU-baseline
leg of the benchmark may import or call it. It shares no code with the HIP
library and imports nothing from it.

The pages mention quantised KV-cache transfers ("Why Understand Inference
Engine Architecture?", Tensor Parallelism Optimization, item 3) but fix no
format, so this is the reading taken:

* codes are FP8 E4M3 in the OCP form: 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits; exponent field 0 holds the subnormals m * 2^-9; the all-ones
  pattern S.1111.111 is NaN; there is no infinity; the largest finite value is
  448;
* each pool has one fp32 scale s (a caller argument): a stored element x
  (the K or V value, upcast to fp32) becomes the code nearest to
  x * (1/s), ties to even, after clamping to [-448, 448]; 1/s is formed in
  fp32 and the product rounded to fp32 before the code is chosen;
* the value of a code c in a pool with scale s is value(c) * s; decode
  attention is the ordinary definition over those values (the paged-attention
  oracle's, in fp64).
"""
from __future__ import annotations

from typing import Iterable, Optional, Tuple

import numpy as np
import torch

from .paged_attention import attend, kv_store

FP8_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of one E4M3 code from the format's definition (NaN for S.1111.111)."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_table() -> np.ndarray:
    """float64 values of all 256 codes."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def inverse_scale(scale: float) -> np.float32:
    """1/s formed in fp32 (IEEE division, correctly rounded)."""
    return np.float32(1.0) / np.float32(scale)


def quantize(x: torch.Tensor, scale: float) -> torch.Tensor:
    """uint8 codes of x (any float dtype): nearest E4M3 code of
    clamp(fp32(x) * fp32(1/s), -448, 448), ties to even."""
    inv = torch.tensor(float(inverse_scale(scale)), dtype=torch.float32)
    y = (x.to(torch.float32) * inv).clamp(-FP8_MAX, FP8_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8)


def dequantize(codes: torch.Tensor, scale: float) -> torch.Tensor:
    """float64 values value(code) * s."""
    table = torch.from_numpy(e4m3_table())
    return table[codes.to(torch.long)] * float(scale)


def kv_store_fp8(k_cache: torch.Tensor, v_cache: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                 slot_mapping: torch.Tensor, k_scale: float, v_scale: float) -> Tuple[torch.Tensor, torch.Tensor]:
    """Copies of the uint8 pools with the quantised k and v rows stored
    through slot_mapping (a negative slot stores nothing)."""
    assert k_cache.dtype == torch.uint8 and v_cache.dtype == torch.uint8
    return kv_store(k_cache, v_cache, quantize(k, k_scale), quantize(v, v_scale), slot_mapping)


def paged_attn_decode_fp8(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                          context_lens: torch.Tensor, scale: float, k_scale: float, v_scale: float,
                          seqs: Optional[Iterable[int]] = None) -> torch.Tensor:
    """Decode attention over the dequantised pools, fp64 [B, Hq, D]: for each
    sequence its blocks are gathered in table order, dequantised, and
    softmax(q k^T * scale) v is formed for each query head (GQA: query head g
    reads KV head g // (Hq / Hkv))."""
    num_seqs, hq, d = q.shape
    hkv = k_cache.shape[2]
    bs = k_cache.shape[1]
    group = hq // hkv
    out = torch.zeros((num_seqs, hq, d), dtype=torch.float64)
    for i in (range(num_seqs) if seqs is None else seqs):
        length = int(context_lens[i])
        nb = -(-length // bs)
        ids = [int(b) for b in block_tables[i, :nb]]
        kk = dequantize(k_cache[ids].reshape(nb * bs, hkv, d)[:length], k_scale)
        vv = dequantize(v_cache[ids].reshape(nb * bs, hkv, d)[:length], v_scale)
        for g in range(hq):
            h = g // group
            out[i, g] = attend(q[i, g].reshape(1, d), kk[:, h, :], vv[:, h, :], scale, [length])[0]
    return out
