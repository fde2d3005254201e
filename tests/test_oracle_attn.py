"""Pins of the fp64 attention oracle and the mask statistics.

Each pin is chosen so that a plausible slip in ``oracle/attn_ref.py`` (a
dropped scale, the mask diagonal off by one, a wrong query->kv head mapping, a
transposed operand, a missing sum over a head group, a leak across documents)
fails at least one of them:

* brute force over the whole row with the dense Megatron-style mask
  (``oracle/dense_ref``), forward and backward;
* torch's fp64 scaled_dot_product_attention(is_causal=True) run on each
  document alone, with autograd for the backward and GQA formed by repeating
  key/value heads;
* closed forms: a one-token document, and identical keys inside a document;
* central finite differences of sum(dO * o);
* packed result == every document run alone;
* block sparsity 74.80% for two 16K documents in a 32K row at 128 x 128 tiles
  (the page's figure), and the >= 75% element sparsity bound when no document
  is longer than half the row.
"""
import math

import numpy as np
import pytest
import torch

from conftest import golden
from oracle import attn_ref, dense_ref, mask_stats
import workloads

TINY_CU = [0, 3, 7, 12, 16]


def _rand(shape, rng):
    return rng.standard_normal(shape)


def _inputs(T, hq, hkv, D, seed):
    rng = np.random.default_rng(seed)
    return (_rand((T, hq, D), rng), _rand((T, hkv, D), rng),
            _rand((T, hkv, D), rng), _rand((T, hq, D), rng))


def test_megatron_mask_matches_page_construction():
    g = golden("p3_mask.json")
    cu = np.concatenate([[0], np.cumsum(g["doc_lengths"])])
    m = dense_ref.megatron_mask(cu)
    tril = np.tril(np.ones((16, 16), dtype=np.int8))
    cleared = tril - m
    # the cleared regions are exactly doc_k's rows x all earlier columns
    for (rows, cols), s, e in zip(g["cleared_blocks"], cu[1:-1], cu[2:]):
        assert (e - s, s) == (rows, cols)
        assert cleared[s:e, :s].all()
    assert cleared.sum() == sum(r * c for r, c in g["cleared_blocks"])
    # the result is block diagonal with one lower triangle per document
    for s, e in zip(cu[:-1], cu[1:]):
        assert (m[s:e, s:e] == np.tril(np.ones((e - s, e - s)))).all()
        assert m[s:e, e:].sum() == 0 and m[s:e, :s].sum() == 0


@pytest.mark.parametrize("hq,hkv,D,seed", [(2, 2, 32, 0), (4, 2, 16, 1), (6, 3, 8, 2), (4, 1, 8, 3)])
def test_against_dense_brute_force_tiny(hq, hkv, D, seed):
    T = 16
    q, k, v, do = _inputs(T, hq, hkv, D, seed)
    o, lse = attn_ref.attn_fwd(q, k, v, TINY_CU)
    dq, dk, dv = attn_ref.attn_bwd(q, k, v, do, TINY_CU)
    ro, rl, rdq, rdk, rdv = dense_ref.dense_fwd_bwd(q, k, v, do, TINY_CU)
    for a, b in [(o, ro), (lse, rl), (dq, rdq), (dk, rdk), (dv, rdv)]:
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(5))
def test_against_dense_brute_force_random_layouts(seed):
    rng = np.random.default_rng(1000 + seed)
    T = int(rng.integers(8, 65))
    cu = workloads.random_layout(rng, T, 1, 20)
    hkv = int(rng.integers(1, 3))
    hq = hkv * int(rng.integers(1, 4))
    q, k, v, do = _inputs(T, hq, hkv, 8, seed)
    scale = float(rng.uniform(0.1, 1.0))
    o, lse = attn_ref.attn_fwd(q, k, v, cu, softmax_scale=scale, block=5)
    dq, dk, dv = attn_ref.attn_bwd(q, k, v, do, cu, softmax_scale=scale, block=7)
    ro, rl, rdq, rdk, rdv = dense_ref.dense_fwd_bwd(q, k, v, do, cu, softmax_scale=scale)
    for a, b in [(o, ro), (lse, rl), (dq, rdq), (dk, rdk), (dv, rdv)]:
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11)


def _sdpa_per_doc(q, k, v, do, cu):
    """Library special case: each document alone through torch SDPA in fp64."""
    T, hq, D = q.shape
    G = hq // k.shape[1]
    outs, grads = [], []
    o = torch.zeros(T, hq, D, dtype=torch.float64)
    lse = torch.zeros(hq, T, dtype=torch.float64)
    dq = torch.zeros_like(o)
    dk = torch.zeros(T, k.shape[1], D, dtype=torch.float64)
    dv = torch.zeros_like(dk)
    for s, e in zip(cu[:-1], cu[1:]):
        Q = torch.tensor(q[s:e]).transpose(0, 1).contiguous().requires_grad_()
        K = torch.tensor(k[s:e]).transpose(0, 1).contiguous().requires_grad_()
        V = torch.tensor(v[s:e]).transpose(0, 1).contiguous().requires_grad_()
        Kr = K.repeat_interleave(G, dim=0)
        Vr = V.repeat_interleave(G, dim=0)
        out = torch.nn.functional.scaled_dot_product_attention(Q, Kr, Vr, is_causal=True)
        out.backward(torch.tensor(do[s:e]).transpose(0, 1))
        o[s:e] = out.detach().transpose(0, 1)
        dq[s:e], dk[s:e], dv[s:e] = (x.grad.transpose(0, 1) for x in (Q, K, V))
        # log-sum-exp of the causal scores, from torch's own logsumexp
        S = (Q @ Kr.transpose(1, 2)) / math.sqrt(D)
        S = S.masked_fill(torch.ones(e - s, e - s, dtype=torch.bool).triu(1), float("-inf"))
        lse[:, s:e] = torch.logsumexp(S, dim=-1).detach()
    return o.numpy(), lse.numpy(), dq.numpy(), dk.numpy(), dv.numpy()


@pytest.mark.parametrize("hq,hkv,D,T,seed", [(2, 2, 32, 16, 0), (8, 2, 32, 200, 1), (4, 4, 64, 150, 2)])
def test_against_torch_sdpa_per_document(hq, hkv, D, T, seed):
    rng = np.random.default_rng(seed)
    cu = TINY_CU if T == 16 else list(workloads.random_layout(rng, T, 1, 90))
    q, k, v, do = _inputs(T, hq, hkv, D, seed)
    o, lse = attn_ref.attn_fwd(q, k, v, cu, block=32)
    dq, dk, dv = attn_ref.attn_bwd(q, k, v, do, cu, block=32)
    ro, rl, rdq, rdk, rdv = _sdpa_per_doc(q, k, v, do, cu)
    for a, b in [(o, ro), (lse, rl), (dq, rdq), (dk, rdk), (dv, rdv)]:
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11)


def test_closed_form_one_token_documents():
    T, hq, hkv, D = 6, 4, 2, 8
    q, k, v, do = _inputs(T, hq, hkv, D, 7)
    cu = list(range(T + 1))
    scale = 0.3
    o, lse = attn_ref.attn_fwd(q, k, v, cu, softmax_scale=scale)
    dq, dk, dv = attn_ref.attn_bwd(q, k, v, do, cu, softmax_scale=scale)
    for h in range(hq):
        g = h // 2
        np.testing.assert_allclose(o[:, h], v[:, g], atol=1e-14)
        np.testing.assert_allclose(lse[h], scale * (q[:, h] * k[:, g]).sum(-1), atol=1e-14)
    np.testing.assert_allclose(dq, 0, atol=1e-14)
    np.testing.assert_allclose(dk, 0, atol=1e-14)
    np.testing.assert_allclose(dv[:, 0], do[:, 0] + do[:, 1], atol=1e-14)
    np.testing.assert_allclose(dv[:, 1], do[:, 2] + do[:, 3], atol=1e-14)


def test_closed_form_identical_keys():
    # equal scores inside a document: uniform weights over the causal prefix
    T, D = 12, 8
    cu = [0, 5, 12]
    rng = np.random.default_rng(3)
    q = rng.standard_normal((T, 1, D))
    k = np.repeat(rng.standard_normal((1, 1, D)), T, axis=0)
    v = rng.standard_normal((T, 1, D))
    o, lse = attn_ref.attn_fwd(q, k, v, cu)
    for s, e in zip(cu[:-1], cu[1:]):
        for i in range(s, e):
            np.testing.assert_allclose(o[i, 0], v[s:i + 1, 0].mean(0), atol=1e-14)
            sc = (q[i, 0] @ k[i, 0]) / math.sqrt(D)
            np.testing.assert_allclose(lse[0, i], sc + math.log(i - s + 1), atol=1e-13)


def test_finite_differences_tiny():
    hq, hkv, D, T = 2, 1, 4, 16
    q, k, v, do = _inputs(T, hq, hkv, D, 11)
    dq, dk, dv = attn_ref.attn_bwd(q, k, v, do, TINY_CU)

    def f(q_, k_, v_):
        o, _ = attn_ref.attn_fwd(q_, k_, v_, TINY_CU)
        return float((o * do).sum())

    eps = 1e-6
    rng = np.random.default_rng(0)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num = (f(*args_p) - f(*args_m)) / (2 * eps)
            assert abs(num - g[idx]) < 1e-7, (name, idx, num, g[idx])


def test_packed_equals_documents_alone():
    rng = np.random.default_rng(5)
    T = 120
    cu = workloads.random_layout(rng, T, 1, 40)
    q, k, v, do = _inputs(T, 4, 2, 16, 5)
    o, lse = attn_ref.attn_fwd(q, k, v, cu, block=16)
    dq, dk, dv = attn_ref.attn_bwd(q, k, v, do, cu, block=16)
    for s, e in zip(cu[:-1], cu[1:]):
        one = [0, e - s]
        o1, l1 = attn_ref.attn_fwd(q[s:e], k[s:e], v[s:e], one)
        g1 = attn_ref.attn_bwd(q[s:e], k[s:e], v[s:e], do[s:e], one)
        np.testing.assert_allclose(o[s:e], o1, atol=1e-13)
        np.testing.assert_allclose(lse[:, s:e], l1, atol=1e-13)
        for a, b in zip((dq, dk, dv), g1):
            np.testing.assert_allclose(a[s:e], b, atol=1e-13)


def test_row_spot_checks_match_full_oracle():
    rng = np.random.default_rng(9)
    T = 300
    cu = workloads.random_layout(rng, T, 1, 120)
    q, k, v, do = _inputs(T, 6, 2, 16, 9)
    o, lse = attn_ref.attn_fwd(q, k, v, cu)
    dq, _, _ = attn_ref.attn_bwd(q, k, v, do, cu)
    rows = rng.integers(0, T, 40)
    heads = rng.integers(0, 6, 40)
    ro, rl = attn_ref.attn_rows(q, k, v, cu, rows, heads)
    rdq = attn_ref.attn_rows_dq(q, k, v, do, cu, rows, heads)
    np.testing.assert_allclose(ro, o[rows, heads], atol=1e-13)
    np.testing.assert_allclose(rl, lse[heads, rows], atol=1e-13)
    np.testing.assert_allclose(rdq, dq[rows, heads], atol=1e-13)


def test_block_sparsity_page_figure():
    g = golden("p3_mask.json")["two_16k_docs_in_32k"]
    cu = np.concatenate([[0], np.cumsum(g["doc_lengths"])])
    sp = mask_stats.block_sparsity(cu, 128)
    assert round(100 * sp, 2) == g["sparsity_percent"]
    # element granularity would not give the printed figure
    el = 1.0 - sum(L * (L + 1) / 2 for L in g["doc_lengths"]) / 32768.0 ** 2
    assert round(100 * el, 2) != g["sparsity_percent"]


def test_element_sparsity_closed_form_and_half_row_bound():
    rng = np.random.default_rng(2)
    for _ in range(20):
        S = int(rng.integers(8, 200))
        cu = workloads.random_layout(rng, S, 1, S // 2)
        lens = np.diff(cu)
        sp = mask_stats.element_sparsity(cu)
        assert abs(sp - (1.0 - (lens * (lens + 1) / 2).sum() / S ** 2)) < 1e-12
        # no document longer than half the row: sum a_i^2 <= S^2 / 2, so with
        # causality at least ~75% of the mask is empty
        assert (lens ** 2).sum() <= S * S / 2
        assert sp >= 0.75 - 1.0 / (2 * S) - 1e-12
    # the page's 16-token example at 4 x 4 tiles (documents 3,4,5,4): counted
    # by hand, row blocks touch 1, 2, 2 and 1 non-empty tiles, so 10 of the 16
    # tiles are empty
    cu = [0, 3, 7, 12, 16]
    assert abs(mask_stats.block_sparsity(cu, 4) - 10 / 16) < 1e-12


def test_key_tail_gradients_match_full_oracle():
    rng = np.random.default_rng(21)
    T = 260
    cu = np.array([0, 37, 200, 260], dtype=np.int32)
    q, k, v, do = _inputs(T, 4, 2, 16, 21)
    _, dk, dv = attn_ref.attn_bwd(q, k, v, do, cu)
    for seg, key_lo in [(1, 150), (1, 37), (2, 259), (0, 10)]:
        e = int(cu[seg + 1])
        tk, tv = attn_ref.attn_bwd_keys(q, k, v, do, cu, seg, key_lo, [1, 0], block=23)
        np.testing.assert_allclose(tk[:, 0], dk[key_lo:e, 1], atol=1e-13)
        np.testing.assert_allclose(tk[:, 1], dk[key_lo:e, 0], atol=1e-13)
        np.testing.assert_allclose(tv[:, 0], dv[key_lo:e, 1], atol=1e-13)


def test_key_window_gradients_match_full_oracle():
    # a window [key_lo, key_hi) anywhere in a document, the head of a document
    # included: only those key columns accumulate, every later query row
    # contributes, and rows before key_lo do not
    T = 260
    cu = np.array([0, 37, 200, 260], dtype=np.int32)
    q, k, v, do = _inputs(T, 4, 2, 16, 22)
    _, dk, dv = attn_ref.attn_bwd(q, k, v, do, cu)
    for seg, key_lo, key_hi in [(1, 37, 37 + 16), (1, 37, 38), (1, 100, 131), (2, 200, 259), (0, 0, 37)]:
        for block in (7, 512):
            tk, tv = attn_ref.attn_bwd_keys(q, k, v, do, cu, seg, key_lo, [1, 0], block=block, key_hi=key_hi)
            assert tk.shape == (key_hi - key_lo, 2, 16)
            np.testing.assert_allclose(tk[:, 0], dk[key_lo:key_hi, 1], atol=1e-13)
            np.testing.assert_allclose(tk[:, 1], dk[key_lo:key_hi, 0], atol=1e-13)
            np.testing.assert_allclose(tv[:, 0], dv[key_lo:key_hi, 1], atol=1e-13)
            np.testing.assert_allclose(tv[:, 1], dv[key_lo:key_hi, 0], atol=1e-13)
    # a window past the document end is cut at the end
    tk, _ = attn_ref.attn_bwd_keys(q, k, v, do, cu, 0, 30, [0], key_hi=1000)
    np.testing.assert_allclose(tk[:, 0], dk[30:37, 0], atol=1e-13)
