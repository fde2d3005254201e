"""GPU document-causal attention vs the fp64 oracle.

Tolerances: fp32 inputs max-abs 1e-5; bf16 inputs max-abs 2e-2 and rel-L2
(||x - ref|| / ||ref|| over the compared elements) <= 5e-3, on O, lse, dQ, dK
and dV.  Small cases compare every element against the full oracle; the
full-size workloads, run exactly as the benchmark launches them, compare
sampled outputs that the oracle computes one by one (random and tail rows of
O / lse / dQ, the key tail of the longest document and whole short documents
for dK / dV).  Also: results repeat bit for bit, writes stay inside their
buffers (guard bands), and k / v may be strided views of one packed kv buffer.
"""
import numpy as np
import pytest
import torch

import packed_sequence_causal_amd as psc
from oracle import attn_ref, pack_ref
import workloads

pytestmark = pytest.mark.gpu

BF16_MAX_ABS, BF16_REL_L2 = 2e-2, 5e-3
F32_MAX_ABS = 1e-5


def close(name, got, ref, dtype, max_abs=BF16_MAX_ABS):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), name
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    if dtype == "f32":
        assert mx <= F32_MAX_ABS, f"{name}: max-abs {mx:.3e}"
        return
    # rel-L2 is undefined against an all-zero reference (e.g. dq and dk of
    # one-token documents are exactly 0); max-abs alone governs there
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / nref) if nref > 0 else 0.0
    assert mx <= max_abs and rel <= BF16_REL_L2, f"{name}: max-abs {mx:.3e} rel-L2 {rel:.3e}"


def run(q, k, v, do, cu, backward=True, scale=None):
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    cud = torch.as_tensor(np.asarray(cu, dtype=np.int32)).to(dev)
    maxlen = int(np.diff(np.asarray(cu)).max())
    out, lse = psc.varlen_attn_fwd(qd, kd, vd, cud, maxlen, softmax_scale=scale)
    res = {"o": out, "lse": lse}
    if backward:
        dq, dk, dv = psc.varlen_attn_bwd(qd, kd, vd, out, do.to(dev), lse, cud, maxlen, softmax_scale=scale)
        res.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {key: val.float().cpu() for key, val in res.items()}


def full_compare(q, k, v, do, cu, dtype, backward=True, scale=None):
    got = run(q, k, v, do, cu, backward, scale)
    o, lse = attn_ref.attn_fwd(q, k, v, cu, softmax_scale=scale)
    close("o", got["o"], o, dtype)
    close("lse", got["lse"], lse, dtype)
    if backward:
        dq, dk, dv = attn_ref.attn_bwd(q, k, v, do, cu, softmax_scale=scale)
        close("dq", got["dq"], dq, dtype)
        # dK and dV sum the contributions of the G = hq / hkv query heads of
        # their key/value head, each carrying the bf16 rounding of P and dS;
        # the 2e-2 bar is the one stated for the workloads (G <= 4) and scales
        # by G / 4 beyond that (rel-L2 keeps its bar)
        g = q.shape[1] // k.shape[1]
        kv_abs = BF16_MAX_ABS * max(1.0, g / 4)
        close("dk", got["dk"], dk, dtype, kv_abs)
        close("dv", got["dv"], dv, dtype, kv_abs)
    return got


# ------------------------------------------------------------- fp32 path

def test_tiny_fp32_workload():
    w = workloads.make("tiny")
    cu = w.attn_cu_seqlens
    q, k, v, do = workloads.qkv_do(16, 2, 2, 32, seed=0, dtype="f32")
    full_compare(q, k, v, do, cu, "f32")


@pytest.mark.parametrize("hq,hkv,D,seed", [(4, 2, 32, 1), (2, 1, 64, 2), (3, 3, 128, 3)])
def test_fp32_random_layouts(hq, hkv, D, seed):
    rng = np.random.default_rng(seed)
    T = 240
    cu = workloads.random_layout(rng, T, 1, 60)
    q, k, v, do = workloads.qkv_do(T, hq, hkv, D, seed=seed, dtype="f32")
    full_compare(q, k, v, do, cu, "f32")


# ------------------------------------------------------------- bf16 path

# segment lengths around the 64 / 128 tile edges, one-token documents, and a
# longer document with a ragged tail
EDGE_LAYOUT = [1, 63, 64, 65, 127, 128, 129, 1, 1, 200, 300, 431]


@pytest.mark.parametrize("hq,hkv,D", [(8, 2, 128), (4, 4, 64), (4, 1, 128), (6, 3, 64)])
def test_bf16_edge_layout(hq, hkv, D):
    cu = np.concatenate([[0], np.cumsum(EDGE_LAYOUT)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v, do = workloads.qkv_do(T, hq, hkv, D, seed=hq * 10 + D, dtype="bf16")
    full_compare(q, k, v, do, cu, "bf16")


# Query-head groups the forward and dQ pack differently: 8 heads per key/value
# head (two 4-head workgroups per group), 2 (64-row x 2-head tiles) and odd
# groups of 3 and 5 (128-row x 1-head tiles), on lengths around the 32-, 64-
# and 128-row tile edges.
@pytest.mark.parametrize("hq,hkv,D", [(16, 2, 128), (8, 1, 64), (4, 2, 128), (6, 2, 128), (5, 1, 64)])
def test_bf16_head_groups(hq, hkv, D):
    lens = [31, 32, 33, 1, 96, 97, 160, 255, 64, 300]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v, do = workloads.qkv_do(T, hq, hkv, D, seed=hq * 7 + hkv, dtype="bf16")
    full_compare(q, k, v, do, cu, "bf16")


@pytest.mark.parametrize("seed", range(3))
def test_bf16_random_layouts(seed):
    rng = np.random.default_rng(500 + seed)
    T = int(rng.integers(900, 2500))
    cu = workloads.random_layout(rng, T, 1, int(rng.integers(50, 1200)))
    D = [64, 128][seed % 2]
    hkv = int(rng.integers(1, 3))
    hq = hkv * int(rng.integers(1, 5))
    q, k, v, do = workloads.qkv_do(T, hq, hkv, D, seed=seed, dtype="bf16")
    full_compare(q, k, v, do, cu, "bf16")


# Randomised layouts mixing lengths across the tile edges: long and short
# documents in one row, so the document-major schedule, tiles whose last key
# block lands in either LDS stage (odd and even block counts), ragged tails
# and several GQA ratios are all exercised against the oracle.
@pytest.mark.parametrize("seed", range(6))
def test_bf16_mixed_layout_sweep(seed):
    rng = np.random.default_rng(9000 + seed)
    lens = list(rng.integers(1, 40, int(rng.integers(3, 12))))
    lens += list(rng.integers(100, 700, int(rng.integers(2, 5))))
    lens.append(int(rng.integers(900, 1800)))
    rng.shuffle(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    D = [64, 128][seed % 2]
    hkv = [1, 2, 4][seed % 3]
    hq = hkv * [1, 2, 4][(seed // 2) % 3]
    q, k, v, do = workloads.qkv_do(T, hq, hkv, D, seed=seed, dtype="bf16")
    full_compare(q, k, v, do, cu, "bf16")


@pytest.mark.parametrize("factor", [0.5, 1.25])
def test_bf16_explicit_softmax_scale(factor):
    # the scale argument is honoured (a factor around the default 1/sqrt(D));
    # much sharper softmax than this grows the bf16 rounding error of dS in dQ
    rng = np.random.default_rng(77)
    T, D = 1500, 128
    cu = workloads.random_layout(rng, T, 1, 700)
    q, k, v, do = workloads.qkv_do(T, 4, 2, D, seed=77, dtype="bf16")
    full_compare(q, k, v, do, cu, "bf16", scale=factor / np.sqrt(D))


def test_bf16_single_long_document_and_one_token_rows():
    for cu in ([0, 3000], list(range(0, 257))):
        cu = np.asarray(cu, dtype=np.int32)
        T = int(cu[-1])
        q, k, v, do = workloads.qkv_do(T, 4, 2, 128, seed=T, dtype="bf16")
        full_compare(q, k, v, do, cu, "bf16")


def test_bf16_many_tiny_documents_large_schedule_path():
    # more than 4095 segments: the tile schedule is built by its multi-kernel
    # path instead of the one-workgroup kernel used for common sizes
    rng = np.random.default_rng(91)
    lens = rng.integers(1, 9, 4600)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v, do = workloads.qkv_do(T, 2, 1, 64, seed=91, dtype="bf16")
    full_compare(q, k, v, do, cu, "bf16")


def test_bf16_packed_kv_views_match_contiguous():
    # kv stacked as [T, 2, Hkv, D]: k = kv[:, 0], v = kv[:, 1] (token stride 2*Hkv*D)
    cu = np.array([0, 100, 333, 700], dtype=np.int32)
    T, hq, hkv, D = 700, 8, 2, 128
    q, k, v, do = workloads.qkv_do(T, hq, hkv, D, seed=5, dtype="bf16")
    dev = torch.device("cuda:0")
    kv = torch.stack([k, v], dim=1).to(dev)
    cud = torch.as_tensor(cu).to(dev)
    qd, dod = q.to(dev), do.to(dev)
    o1, l1 = psc.varlen_attn_fwd(qd, kv[:, 0], kv[:, 1], cud, 367)
    g1 = psc.varlen_attn_bwd(qd, kv[:, 0], kv[:, 1], o1, dod, l1, cud, 367)
    o2, l2 = psc.varlen_attn_fwd(qd, k.to(dev), v.to(dev), cud, 367)
    g2 = psc.varlen_attn_bwd(qd, k.to(dev), v.to(dev), o2, dod, l2, cud, 367)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_bf16_repeat_is_bit_identical_and_guards_hold():
    cu = np.concatenate([[0], np.cumsum(EDGE_LAYOUT)]).astype(np.int32)
    T, hq, hkv, D = int(cu[-1]), 8, 2, 128
    q, k, v, do = workloads.qkv_do(T, hq, hkv, D, seed=9, dtype="bf16")
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    cud = torch.as_tensor(cu).to(dev)
    G = 4096  # guard elements on each side
    sent = -12288.0  # exactly representable in bf16 and fp32

    def guarded(n, dtype):
        buf = torch.full((n + 2 * G,), sent, dtype=dtype, device=dev)
        return buf, buf[G:G + n]

    runs = []
    for _ in range(2):
        ob, o = guarded(T * hq * D, torch.bfloat16)
        lb, l = guarded(hq * T, torch.float32)
        qb, dq = guarded(T * hq * D, torch.float32)
        kb, dk = guarded(T * hkv * D, torch.float32)
        vb, dv = guarded(T * hkv * D, torch.float32)
        o, l = o.view(T, hq, D), l.view(hq, T)
        psc.varlen_attn_fwd(qd, kd, vd, cud, 431, out=o, lse=l)
        psc.varlen_attn_bwd(qd, kd, vd, o, dod, l, cud, 431, dq=dq.view(T, hq, D), dk=dk.view(T, hkv, D),
                            dv=dv.view(T, hkv, D))
        torch.cuda.synchronize()
        for buf in (ob, lb, qb, kb, vb):
            assert (buf[:G].float() == sent).all() and (buf[-G:].float() == sent).all()
        runs.append([x.clone() for x in (o, l, dq, dk, dv)])
    for a, b in zip(*runs):
        assert torch.equal(a, b)


# ------------------------------------------------- full-size workloads

def _layout(w):
    if w.attn_cu_seqlens is not None:
        return np.asarray(w.attn_cu_seqlens, dtype=np.int32)
    p = w.pack
    rows = pack_ref.build_pack(p.docs, p.micro_bsz, p.seq_len)[: p.keep_rows]
    return np.asarray(pack_ref.flatten(rows, p.packed_length)["cu_seqlens"], dtype=np.int32)


def sampled_check(q, k, v, do, cu, a_hq, a_hkv, dtype, backward, got, seed=1):
    """Sampled comparison with the oracle at full size: random rows and the
    tail of the longest document (o, lse, dq), the last keys of the longest
    document (dk, dv for one kv head) and two whole short documents."""
    T = int(cu[-1])
    rng = np.random.default_rng(seed)
    lens = np.diff(cu)
    longest = int(np.argmax(lens))
    s_long, e_long = int(cu[longest]), int(cu[longest + 1])
    rows = np.concatenate([rng.integers(0, T, 96), np.arange(e_long - 32, e_long)])
    heads = rng.integers(0, a_hq, rows.size)
    o, lse = attn_ref.attn_rows(q, k, v, cu, rows, heads)
    close("o", got["o"][rows, heads].numpy(), o, dtype)
    close("lse", got["lse"][heads, rows].numpy(), lse, dtype)
    if not backward:
        return
    dq = attn_ref.attn_rows_dq(q, k, v, do, cu, rows[:64], heads[:64])
    close("dq", got["dq"][rows[:64], heads[:64]].numpy(), dq, dtype)
    g = int(rng.integers(0, a_hkv))
    key_lo = max(s_long, e_long - 160)
    dk, dv = attn_ref.attn_bwd_keys(q, k, v, do, cu, longest, key_lo, [g])
    close("dk tail", got["dk"][key_lo:e_long, [g]].numpy(), dk, dtype)
    close("dv tail", got["dv"][key_lo:e_long, [g]].numpy(), dv, dtype)
    short = [i for i in np.argsort(lens) if lens[i] > 8][:2]
    if len(lens) < 2:
        return
    heads_kv = list(range(a_hkv))
    for si in short:
        s, e = int(cu[si]), int(cu[si + 1])
        if e - s > 4096:
            continue  # whole-document key gradients only for short documents
        dk, dv = attn_ref.attn_bwd_keys(q, k, v, do, cu, int(si), s, heads_kv)
        close("dk doc", got["dk"][s:e].numpy(), dk, dtype)
        close("dv doc", got["dv"][s:e].numpy(), dv, dtype)


@pytest.mark.parametrize("name", ["uniform_8k", "lognormal_32k", "seqpar_share_128k", "skewed_32k"])
def test_full_size_sampled(name):
    w = workloads.make(name)
    cu = _layout(w)
    T = int(cu[-1])
    a = w.attn
    q, k, v, do = workloads.qkv_do(T, a.hq, a.hkv, a.head_dim, seed=0, dtype=a.dtype)
    print(f"[{name}] T={T} segments={len(cu) - 1} hq={a.hq} hkv={a.hkv} D={a.head_dim}", flush=True)
    got = run(q, k, v, do, cu, backward=a.backward)
    sampled_check(q, k, v, do, cu, a.hq, a.hkv, a.dtype, a.backward, got)


# The document-length sweep's rows (one 32768-token row, GQA 32/8, D 128):
# with the document mask and as one whole-row causal segment.
@pytest.mark.parametrize("name,whole_row", [("16K+16K", False), ("2K+30K", False), ("2K+30K", True),
                                            ("32x1K", False)])
def test_doc_sweep_layouts_sampled(name, whole_row):
    cu = workloads.doc_sweep_cu(name, whole_row)
    T = int(cu[-1])
    q, k, v, do = workloads.qkv_do(T, 32, 8, 128, seed=0, dtype="bf16")
    print(f"[sweep {name} whole_row={whole_row}] T={T} segments={len(cu) - 1}", flush=True)
    got = run(q, k, v, do, cu, backward=True)
    sampled_check(q, k, v, do, cu, 32, 8, "bf16", True, got)
