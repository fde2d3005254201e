"""Rotary embedding fused with document-causal attention
(psc_varlen_attn_fwd_rope / psc_varlen_attn_bwd_rope).

(a) Against this library's separate steps, bit for bit: psc_rope on q and k,
    psc_varlen_attn_fwd / _bwd on the rotated q~, k~, then psc_rope's inverse on
    the fp32 dq and dk.  The fused kernels use the same angles and arithmetic,
    so q~, k~, O, lse, dQ, dK and dV must be identical.
(b) Against the oracle: rope_ref rotates q and k (fp64), the rotated values are
    rounded to bf16 as the rotation step stores them, attn_ref runs on them, and
    the inverse rope_ref turns dq~, dk~ back; bf16 bar (max-abs 2e-2, rel-L2
    5e-3).  Small layouts in full; the 2 x 32K and 128K workloads sampled (rows
    of O, lse, dQ; the first 128 keys of the longest document for dK, dV), with
    the packer's indexes as positions.
"""
import numpy as np
import pytest
import torch

import packed_sequence_causal_amd as psc
from oracle import attn_ref, pack_ref, rope_ref
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
BAR_ABS, BAR_REL = 2e-2, 5e-3


def close(name, got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    err = float(np.abs(got - ref).max())
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / nref) if nref > 0 else 0.0
    assert err <= BAR_ABS and rel <= BAR_REL, f"{name}: max-abs {err:.3e} rel-L2 {rel:.3e}"


def positions_of(cu):
    """Offset of each token inside its segment (what the packer's indexes hold)."""
    cu = np.asarray(cu, dtype=np.int64)
    T = int(cu[-1])
    seg = np.searchsorted(cu, np.arange(T), side="right") - 1
    return (np.arange(T) - cu[seg]).astype(np.int32)


def rotated_bf16(x, pos, chunk=4096):
    """The oracle's rotation, rounded to bf16 as the rotation step stores it
    (token chunks only bound the fp64 temporaries; rows are independent)."""
    out = torch.empty(x.shape, dtype=torch.bfloat16)
    for t0 in range(0, x.shape[0], chunk):
        r = rope_ref.rope(x[t0:t0 + chunk].float().numpy(), pos[t0:t0 + chunk])
        out[t0:t0 + chunk] = torch.from_numpy(r).to(torch.bfloat16)
    return out


def fused(q, k, v, do, cu, pos, grad_dtype=None, base=10000.0):
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    cud = torch.as_tensor(np.asarray(cu, np.int32)).to(DEV)
    posd = torch.as_tensor(pos).to(DEV)
    ml = int(np.diff(np.asarray(cu)).max())
    o, lse = psc.varlen_attn_fwd_rope(qd, kd, vd, cud, ml, posd, base)
    g = psc.varlen_attn_bwd_rope(qd, kd, vd, o, dod, lse, cud, ml, posd, base, grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    return {"q_rot": qd.cpu(), "k_rot": kd.cpu(), "o": o.cpu(), "lse": lse.cpu(), "dq": g[0].cpu(),
            "dk": g[1].cpu(), "dv": g[2].cpu()}


def separate(q, k, v, do, cu, pos, base=10000.0):
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    cud = torch.as_tensor(np.asarray(cu, np.int32)).to(DEV)
    posd = torch.as_tensor(pos).to(DEV)
    ml = int(np.diff(np.asarray(cu)).max())
    psc.rope(qd, kd, posd, base)
    o, lse = psc.varlen_attn_fwd(qd, kd, vd, cud, ml)
    dq, dk, dv = psc.varlen_attn_bwd(qd, kd, vd, o, dod, lse, cud, ml)
    psc.rope(dq, dk, posd, base, inverse=True)
    torch.cuda.synchronize()
    return {"q_rot": qd.cpu(), "k_rot": kd.cpu(), "o": o.cpu(), "lse": lse.cpu(), "dq": dq.cpu(), "dk": dk.cpu(),
            "dv": dv.cpu()}


EDGE = [1, 63, 64, 65, 127, 128, 129, 1, 1, 200, 300, 431]


@pytest.mark.parametrize("hq,hkv,D,base", [(8, 2, 128, 10000.0), (4, 4, 64, 10000.0), (6, 3, 64, 500000.0),
                                           (4, 1, 128, 10000.0)])
def test_fused_equals_separate_steps_bit_for_bit(hq, hkv, D, base):
    cu = np.concatenate([[0], np.cumsum(EDGE)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v, do = workloads.qkv_do(T, hq, hkv, D, seed=hq + D, dtype="bf16")
    pos = positions_of(cu)
    a = fused(q, k, v, do, cu, pos, base=base)
    b = separate(q, k, v, do, cu, pos, base=base)
    for name in ("q_rot", "k_rot", "o", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[name], b[name]), name


@pytest.mark.parametrize("hq,hkv,D", [(8, 2, 128), (4, 4, 64)])
def test_fused_against_oracle(hq, hkv, D):
    cu = np.concatenate([[0], np.cumsum(EDGE)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v, do = workloads.qkv_do(T, hq, hkv, D, seed=7 * hq + D, dtype="bf16")
    pos = positions_of(cu)
    got = fused(q, k, v, do, cu, pos)
    qr, kr = rotated_bf16(q, pos), rotated_bf16(k, pos)
    o, lse = attn_ref.attn_fwd(qr, kr, v, cu)
    dqr, dkr, dv = attn_ref.attn_bwd(qr, kr, v, do, cu)
    close("o", got["o"].float(), o)
    close("lse", got["lse"], lse)
    close("dq", got["dq"], rope_ref.rope(dqr, pos, inverse=True))
    close("dk", got["dk"], rope_ref.rope(dkr, pos, inverse=True))
    close("dv", got["dv"], dv)


def test_fused_bf16_gradients_round_the_fp32_ones():
    cu = np.concatenate([[0], np.cumsum(EDGE)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v, do = workloads.qkv_do(T, 8, 2, 128, seed=3, dtype="bf16")
    pos = positions_of(cu)
    a = fused(q, k, v, do, cu, pos)
    b = fused(q, k, v, do, cu, pos, grad_dtype=psc.BF16)
    for name in ("dq", "dk", "dv"):
        assert b[name].dtype == torch.bfloat16
        assert torch.equal(b[name], a[name].to(torch.bfloat16)), name


def _packed(name):
    w = workloads.make(name)
    p = w.pack
    rows = pack_ref.build_pack(p.docs, p.micro_bsz, p.seq_len)[: p.keep_rows]
    flat = pack_ref.flatten(rows, p.packed_length)
    return w, np.asarray(flat["cu_seqlens"], dtype=np.int32), np.asarray(flat["indexes"], dtype=np.int32)


@pytest.mark.parametrize("name", ["lognormal_32k", "seqpar_share_128k"])
def test_fused_full_size_sampled(name):
    w, cu, pos = _packed(name)
    T = int(cu[-1])
    assert pos.size == T
    a = w.attn
    q, k, v, do = workloads.qkv_do(T, a.hq, a.hkv, a.head_dim, seed=0, dtype="bf16")
    print(f"[{name}] fused rotary attention, T={T}", flush=True)
    got = fused(q, k, v, do, cu, pos)
    qr, kr = rotated_bf16(q, pos), rotated_bf16(k, pos)
    # the rotated k as the rotation step stores it: within half a bf16 ulp of
    # the exact rotation plus 2e-5 (an fp32 result rounded once), elementwise
    kref = np.concatenate([rope_ref.rope(k[t0:t0 + 8192].float().numpy(), pos[t0:t0 + 8192])
                           for t0 in range(0, T, 8192)])
    kerr = np.abs(got["k_rot"].float().numpy() - kref)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(kref), 2.0 ** -126))) - 7)
    assert (kerr <= 0.5 * ulp + 2e-5).all(), f"k rotation off by up to {kerr.max():.3g}"
    rng = np.random.default_rng(3)
    lens = np.diff(cu)
    longest = int(np.argmax(lens))
    s_long, e_long = int(cu[longest]), int(cu[longest + 1])
    rows = np.concatenate([rng.integers(0, T, 128), np.arange(e_long - 64, e_long)])
    heads = rng.integers(0, a.hq, rows.size)
    o, lse = attn_ref.attn_rows(qr, kr, v, cu, rows, heads)
    close("o", got["o"][rows, heads].float().numpy(), o)
    close("lse", got["lse"][heads, rows].numpy(), lse)
    dqr = attn_ref.attn_rows_dq(qr, kr, v, do, cu, rows, heads)
    close("dq", got["dq"][rows, heads].numpy(), rope_ref.rope(dqr[:, None, :], pos[rows], inverse=True)[:, 0])
    key_hi = min(e_long, s_long + 128)
    g = int(rng.integers(0, a.hkv))
    print(f"  dk/dv head keys [{s_long}, {key_hi}) of the {e_long - s_long}-token document", flush=True)
    dkr, dv = attn_ref.attn_bwd_keys(qr, kr, v, do, cu, longest, s_long, [g], key_hi=key_hi)
    close("dk head", got["dk"][s_long:key_hi, [g]].numpy(), rope_ref.rope(dkr, pos[s_long:key_hi], inverse=True))
    close("dv head", got["dv"][s_long:key_hi, [g]].numpy(), dv)


def test_fused_full_size_equals_separate_steps():
    _, cu, pos = _packed("lognormal_32k")
    T = int(cu[-1])
    q, k, v, do = workloads.qkv_do(T, 32, 8, 128, seed=0, dtype="bf16")
    a = fused(q, k, v, do, cu, pos)
    b = separate(q, k, v, do, cu, pos)
    for name in ("q_rot", "k_rot", "o", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[name], b[name]), name
