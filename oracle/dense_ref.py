"""Whole-row attention under a dense document-causal mask (tiny inputs only).

Test infrastructure only (see ``oracle/__init__``).

The mask is built the way the Megatron ``reset_attention_mask`` option is
described in "Sample Packing：长序列 LLM 训练的 Attention 问题及优化", section
4.2 (性能问题): start from the plain lower-triangular causal mask over the whole
row, then, for every document after the first, clear that document's rows over
all columns before its start (for documents of 3,4,5,4 tokens the cleared
blocks are 4x3, 5x7 and 4x12).  Attention is then ordinary masked softmax over
the whole row, forward and backward written out on the dense T x T matrices.

This shares nothing with ``attn_ref`` (which never forms a mask and works per
segment) and serves as its brute-force pin on small rows.
"""
from __future__ import annotations

import math

import numpy as np


def megatron_mask(cu_seqlens):
    cu = [int(c) for c in np.asarray(cu_seqlens).reshape(-1)]
    T = cu[-1]
    mask = np.tril(np.ones((T, T), dtype=np.int8))
    for d in range(1, len(cu) - 1):
        s, e = cu[d], cu[d + 1]
        mask[s:e, :s] = 0
    return mask


def dense_fwd_bwd(q, k, v, do, cu_seqlens, softmax_scale=None):
    """q [T,Hq,D], k/v [T,Hkv,D], do [T,Hq,D] (fp64 arrays).

    Returns o, lse [Hq,T], dq, dk, dv.  Query head h uses key/value head
    h // (Hq/Hkv).
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else softmax_scale
    keep = megatron_mask(cu_seqlens).astype(bool)
    o = np.zeros_like(q)
    lse = np.zeros((Hq, T))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(Hq):
        g = h // G
        S = scale * q[:, h] @ k[:, g].T
        S = np.where(keep, S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        Z = E.sum(axis=1, keepdims=True)
        P = E / Z
        o[:, h] = P @ v[:, g]
        lse[h] = (m + np.log(Z))[:, 0]
        # softmax Jacobian: dS = P * (dP - rowsum(P * dP))
        dP = do[:, h] @ v[:, g].T
        dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
        dq[:, h] = scale * dS @ k[:, g]
        dk[:, g] += scale * dS.T @ q[:, h]
        dv[:, g] += P.T @ do[:, h]
    return o, lse, dq, dk, dv
