"""fp64 rotary position embedding of packed rows, positions from `indexes`.

Test infrastructure only (see ``oracle/__init__``).

Sources:
  * InternEvo documentation, page "数据加载与流程" (data flow), section
    "获取Dataloader数据": `indexes` holds each token's position inside its
    segment, counting from 0 (a carried-over fragment and the padding tail
    restart at 0 too); section "Forward过程数据格式": the attention module of the
    model holds a RotaryEmbedding.
  * XTuner documentation, sequence-parallel page, section "实现方案": q and k are
    rotated by apply_rotary_pos_emb(q, k, cos, sin) right after the projection,
    before attention.
  * "Sample Packing：长序列 LLM 训练的 Attention 问题及优化", section 4.1: with
    packed documents the position ids must restart per document as well.

Reading (the pages print no formula): RoFormer's rotary
embedding in the rotate-half layout that an apply_rotary_pos_emb(q, k, cos,
sin) call works on.  For head dimension D, dimensions i and i + D/2
(0 <= i < D/2) form a pair that is rotated by the angle
    theta_i = pos * base ** (-2 i / D),   base = 10000 by default,
    (x_i, x_{i+D/2}) -> (x_i cos - x_{i+D/2} sin,  x_{i+D/2} cos + x_i sin),
with pos = indexes[token].  The backward pass (gradient with respect to the
unrotated vectors) is the rotation by -theta.

Pins: tests/test_oracle_rope.py (position 0 is the identity, D = 2 and D = 4
closed forms, the complex-multiplication form, norm preservation, inverse,
relative-position property, packed rows equal documents rotated alone).
"""
from __future__ import annotations

import numpy as np


def inv_freq(head_dim: int, base: float = 10000.0) -> np.ndarray:
    """base ** (-2 i / D) for i = 0 .. D/2 - 1, in fp64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / head_dim)


def rope(x, positions, base: float = 10000.0, inverse: bool = False) -> np.ndarray:
    """Rotate x [T, H, D] (any float type, upcast to fp64) by positions [T]."""
    x = np.asarray(x, dtype=np.float64)
    T, H, D = x.shape
    assert D % 2 == 0
    pos = np.asarray(positions, dtype=np.float64).reshape(T)
    theta = pos[:, None] * inv_freq(D, base)[None, :]          # [T, D/2]
    if inverse:
        theta = -theta
    c = np.cos(theta)[:, None, :]
    s = np.sin(theta)[:, None, :]
    x1 = x[..., : D // 2]
    x2 = x[..., D // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
