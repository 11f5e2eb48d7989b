"""Plain fp64 CPU oracle for rotary position embedding (RoPE) followed by the
KV store.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module:
only the tests, the smoke check of the package entry file and the CPU-baseline
leg of the benchmark may import or call it. It shares no code with the HIP
library and imports nothing from it.

The pages name RoPE among the features of the model Nano-vLLM serves (Qwen3):
"Nano-vLLM System Architecture Analysis", section "Differences from Normal
nanoGPT Inference", item 6 "Architecture Support". They give no formula, so
this oracle takes the plainest reading, the rotary embedding as it is usually
applied to Qwen-family checkpoints:

* head dimension D is split in halves; element i of the first half and
  element i + D/2 form pair i (i < D/2);
* pair i of a token at position p is rotated by the angle p * theta_i, with
  theta_i = base^(-2i / D) and `base` the model's rope theta (a caller
  argument);
* every query head and every KV head of the token is rotated the same way;
  V is not rotated;
* the rotated K and the unrotated V are then stored through slot_mapping
  exactly as `kv_store` does (a negative slot stores nothing; the query is
  rotated regardless).

The arithmetic is float64 throughout; the result is rounded to the inputs'
dtype once at the end.
"""
from __future__ import annotations

from typing import Tuple

import torch

from .paged_attention import kv_store


def rope_angles(positions: torch.Tensor, head_dim: int, base: float) -> torch.Tensor:
    """Angles p * theta_i, float64 [T, D/2], theta_i = base^(-2i/D)."""
    assert head_dim % 2 == 0
    half = head_dim // 2
    theta = torch.tensor([base ** (-2.0 * i / head_dim) for i in range(half)], dtype=torch.float64)
    return positions.to(torch.float64).reshape(-1, 1) * theta.reshape(1, -1)


def rope(x: torch.Tensor, positions: torch.Tensor, base: float) -> torch.Tensor:
    """Rotate x [T, H, D] by its tokens' positions; float64 result.

    For pair i: (a, b) = (x[..., i], x[..., i + D/2]) becomes
    (a cos t - b sin t, b cos t + a sin t) with t = p * theta_i.
    """
    t_count, _, d = x.shape
    assert positions.shape == (t_count,)
    half = d // 2
    ang = rope_angles(positions, d, base).unsqueeze(1)  # [T, 1, D/2]
    cos, sin = torch.cos(ang), torch.sin(ang)
    x64 = x.to(torch.float64)
    a, b = x64[..., :half], x64[..., half:]
    return torch.cat([a * cos - b * sin, b * cos + a * sin], dim=-1)


def rms_norm(x: torch.Tensor, weight: torch.Tensor, eps: float) -> torch.Tensor:
    """RMSNorm of every head row of x [T, H, D] over its D elements, float64:
    x / sqrt(mean(x^2) + eps) * weight, weight [D] shared by all heads.

    The pages name QK-Norm among the features of the served model ("Nano-vLLM
    System Architecture Analysis", "Differences from Normal nanoGPT
    Inference", item 6) without a formula; the reading taken is the RMS
    normalisation of each query and key head row with a learned per-dimension
    weight, applied before the rotary embedding.
    """
    x64 = x.to(torch.float64)
    ms = (x64 * x64).mean(dim=-1, keepdim=True)
    return x64 / torch.sqrt(ms + eps) * weight.to(torch.float64)


def qknorm_rope_kv_store(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, positions: torch.Tensor,
                         k_cache: torch.Tensor, v_cache: torch.Tensor, slot_mapping: torch.Tensor, base: float,
                         q_weight: torch.Tensor, k_weight: torch.Tensor,
                         eps: float) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """rope_kv_store with RMSNorm (QK-Norm) of q and k first: q and k head
    rows are normalised (float64), rotated, and rounded once to the inputs'
    dtype; v is stored as given."""
    assert q.dtype == k.dtype == v.dtype
    q_rot = rope(rms_norm(q, q_weight, eps), positions, base).to(q.dtype)
    k_rot = rope(rms_norm(k, k_weight, eps), positions, base).to(k.dtype)
    kc, vc = kv_store(k_cache, v_cache, k_rot, v, slot_mapping)
    return q_rot, kc, vc


def rope_kv_store(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, positions: torch.Tensor,
                  k_cache: torch.Tensor, v_cache: torch.Tensor, slot_mapping: torch.Tensor,
                  base: float) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Rotated q (in q's dtype) and copies of the pools with the rotated k and
    the plain v stored through slot_mapping."""
    assert q.dtype == k.dtype == v.dtype
    q_rot = rope(q, positions, base).to(q.dtype)
    k_rot = rope(k, positions, base).to(k.dtype)
    kc, vc = kv_store(k_cache, v_cache, k_rot, v, slot_mapping)
    return q_rot, kc, vc
