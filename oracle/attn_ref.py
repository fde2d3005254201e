"""fp64 per-document causal softmax attention, forward and backward.

Test infrastructure only (see ``oracle/__init__``).

What is computed (the plain definition; no tiling, no online softmax):
  For every segment [s, e) of ``cu_seqlens`` (a padding tail is a segment like
  any other), every query head h and its key/value head g = h // G with
  G = Hq / Hkv:
    S_ij  = scale * <q_i, k_j>            for s <= j <= i < e
    lse_i = log sum_j exp(S_ij)           (natural log)
    P_ij  = exp(S_ij - lse_i)
    o_i   = sum_j P_ij v_j
  Backward, for an upstream gradient dO:
    dP_ij = <dO_i, v_j>,   D_i = sum_j P_ij dP_ij  (= <dO_i, o_i>)
    dS_ij = P_ij (dP_ij - D_i)
    dq_i  = scale * sum_j dS_ij k_j
    dk_j  = scale * sum_i dS_ij q_i   (summed over the G query heads of g)
    dv_j  = sum_i P_ij dO_i           (summed over the G query heads of g)

Sources:
  * "Sample Packing：长序列 LLM 训练的 Attention 问题及优化", section 三
    (Attention Mask): the block-diagonal mask is one lower-triangular causal
    block per document (diagonal included), and packed attention is the same as
    running each document on its own;
  * InternEvo "数据加载与流程", section "ISP并行模式下数据流程" (qkv split and
    attention): the grouped qkv layout, where the first G slots of each
    key/value head's group are its query heads, so query head h reads
    key/value head h // G;
  * softmax scale 1/sqrt(D) unless given (the pages do not fix it).

Inputs of any float dtype are converted exactly to fp64 first, so the oracle
sees the same quantised values as a bf16 kernel.  Query rows are processed in
blocks of at most ``block`` rows so one long document never needs its full
L x L score matrix.

Pins: tests/test_oracle_attn.py (dense Megatron-mask brute force, per-document
torch SDPA + autograd in fp64, closed forms, central finite differences, the
packed == documents-alone invariant).
"""
from __future__ import annotations

import math

import numpy as np


def _f64(x):
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def _segments(cu_seqlens):
    cu = [int(c) for c in np.asarray(cu_seqlens).reshape(-1)]
    return [(cu[i], cu[i + 1]) for i in range(len(cu) - 1) if cu[i + 1] > cu[i]]


def _scale(head_dim, softmax_scale):
    return 1.0 / math.sqrt(head_dim) if softmax_scale is None else float(softmax_scale)


def _causal_block_scores(Qb, Kpre, i0, scale):
    """Scores of query rows i0.. (segment-local) against keys 0..i1-1, with the
    entries j > i set to -inf."""
    b = Qb.shape[0]
    S = scale * (Qb @ Kpre.T)
    rows = i0 + np.arange(b)[:, None]
    cols = np.arange(Kpre.shape[0])[None, :]
    S[cols > rows] = -np.inf
    return S


def attn_fwd(q, k, v, cu_seqlens, softmax_scale=None, block=512):
    """Returns (o [T,Hq,D] fp64, lse [Hq,T] fp64)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    scale = _scale(D, softmax_scale)
    o = np.zeros_like(q)
    lse = np.zeros((Hq, T))
    for s, e in _segments(cu_seqlens):
        L = e - s
        for h in range(Hq):
            g = h // G
            Q, K, V = q[s:e, h], k[s:e, g], v[s:e, g]
            for i0 in range(0, L, block):
                i1 = min(i0 + block, L)
                S = _causal_block_scores(Q[i0:i1], K[:i1], i0, scale)
                m = S.max(axis=1, keepdims=True)
                l = np.log(np.exp(S - m).sum(axis=1, keepdims=True)) + m
                P = np.exp(S - l)
                o[s + i0:s + i1, h] = P @ V[:i1]
                lse[h, s + i0:s + i1] = l[:, 0]
    return o, lse


def attn_bwd(q, k, v, do, cu_seqlens, softmax_scale=None, block=512):
    """Gradients of sum(dO * o) w.r.t. q, k, v.  Returns (dq, dk, dv) fp64."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = _scale(D, softmax_scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for s, e in _segments(cu_seqlens):
        L = e - s
        for h in range(Hq):
            g = h // G
            Q, K, V, dO = q[s:e, h], k[s:e, g], v[s:e, g], do[s:e, h]
            for i0 in range(0, L, block):
                i1 = min(i0 + block, L)
                S = _causal_block_scores(Q[i0:i1], K[:i1], i0, scale)
                m = S.max(axis=1, keepdims=True)
                P = np.exp(S - m)
                P /= P.sum(axis=1, keepdims=True)
                dP = dO[i0:i1] @ V[:i1].T
                Drow = (P * dP).sum(axis=1, keepdims=True)
                dS = P * (dP - Drow)
                dq[s + i0:s + i1, h] = scale * (dS @ K[:i1])
                dk[s:s + i1, g] += scale * (dS.T @ Q[i0:i1])
                dv[s:s + i1, g] += P.T @ dO[i0:i1]
    return dq, dk, dv


def _slice64(x, *idx):
    """fp64 copy of x[idx] only (inputs at full size may be large bf16 arrays)."""
    return _f64(x[idx])


def attn_rows(q, k, v, cu_seqlens, rows, heads, softmax_scale=None):
    """Forward output and lse for selected (token, head) pairs only, each from
    its own segment prefix; cheap spot checks at full size.

    Returns o [n, D], lse [n].
    """
    D = q.shape[2]
    G = q.shape[1] // k.shape[1]
    scale = _scale(D, softmax_scale)
    cu = np.asarray(cu_seqlens).reshape(-1).astype(np.int64)
    outs, lses = [], []
    for t, h in zip(rows, heads):
        t, h = int(t), int(h)
        sidx = int(np.searchsorted(cu, t, side="right")) - 1
        s = int(cu[sidx])
        g = h // G
        srow = scale * (_slice64(k, slice(s, t + 1), g) @ _slice64(q, t, h))
        m = srow.max()
        l = m + math.log(np.exp(srow - m).sum())
        p = np.exp(srow - l)
        outs.append(p @ _slice64(v, slice(s, t + 1), g))
        lses.append(l)
    return np.array(outs), np.array(lses)


def attn_rows_dq(q, k, v, do, cu_seqlens, rows, heads, softmax_scale=None):
    """dq for selected (token, head) pairs; row t of dq depends only on row t's
    scores, so each is computed alone."""
    D = q.shape[2]
    G = q.shape[1] // k.shape[1]
    scale = _scale(D, softmax_scale)
    cu = np.asarray(cu_seqlens).reshape(-1).astype(np.int64)
    out = []
    for t, h in zip(rows, heads):
        t, h = int(t), int(h)
        sidx = int(np.searchsorted(cu, t, side="right")) - 1
        s = int(cu[sidx])
        g = h // G
        K, V = _slice64(k, slice(s, t + 1), g), _slice64(v, slice(s, t + 1), g)
        srow = scale * (K @ _slice64(q, t, h))
        p = np.exp(srow - srow.max())
        p /= p.sum()
        dp = V @ _slice64(do, t, h)
        ds = p * (dp - (p * dp).sum())
        out.append(scale * (ds @ K))
    return np.array(out)


def attn_bwd_keys(q, k, v, do, cu_seqlens, seg, key_lo, kv_heads, softmax_scale=None, block=512, key_hi=None):
    """dk, dv for the keys [key_lo, key_hi) of segment ``seg`` = [s, e) and the
    listed key/value heads only (key_hi defaults to e).

    dk_j and dv_j need every query row i >= j of the document, and each such
    row's lse_i and D_i come from its full causal prefix: for every row block,
    the scores against the whole prefix give lse_i and o_i = sum_j P_ij v_j,
    D_i = <dO_i, o_i>, and then only the key columns [key_lo, key_hi) form P,
    dP and dS and are accumulated.  fp64 throughout (torch CPU tensors, whose
    exp and matmul use every core; the arithmetic is the plain definition).
    Returns arrays [key_hi - key_lo, len(kv_heads), D].
    """
    import torch

    Hq, D = q.shape[1], q.shape[2]
    G = Hq // k.shape[1]
    scale = _scale(D, softmax_scale)
    cu = [int(c) for c in np.asarray(cu_seqlens).reshape(-1)]
    s, e = cu[seg], cu[seg + 1]
    key_hi = e if key_hi is None else min(int(key_hi), e)
    assert s <= key_lo < key_hi, (s, key_lo, key_hi)
    n = key_hi - key_lo
    c0, c1 = key_lo - s, key_hi - s
    t64 = lambda x: torch.from_numpy(np.ascontiguousarray(x))
    dk = torch.zeros((n, len(kv_heads), D), dtype=torch.float64)
    dv = torch.zeros((n, len(kv_heads), D), dtype=torch.float64)
    for gi, g in enumerate(kv_heads):
        K, V = t64(_slice64(k, slice(s, e), g)), t64(_slice64(v, slice(s, e), g))
        for h in range(g * G, (g + 1) * G):
            Q, dO = t64(_slice64(q, slice(s, e), h)), t64(_slice64(do, slice(s, e), h))
            for i0 in range(c0, e - s, block):
                i1 = min(i0 + block, e - s)
                S = scale * (Q[i0:i1] @ K[:i1].T)
                rows = torch.arange(i0, i1)[:, None]
                S.masked_fill_(torch.arange(i1)[None, :] > rows, -math.inf)
                m = S.max(dim=1, keepdim=True).values
                E = torch.exp(S - m)
                lsum = E.sum(dim=1, keepdim=True)
                o = (E @ V[:i1]) / lsum                       # o_i
                Drow = (dO[i0:i1] * o).sum(dim=1, keepdim=True)  # D_i = <dO_i, o_i>
                ce = min(c1, i1)  # rows i0.. see keys up to i1 - 1 only
                P = E[:, c0:ce] / lsum
                dP = dO[i0:i1] @ V[c0:ce].T
                dS = P * (dP - Drow)
                dk[: ce - c0, gi] += scale * (dS.T @ Q[i0:i1])
                dv[: ce - c0, gi] += P.T @ dO[i0:i1]
    return dk.numpy(), dv.numpy()
