"""Every call stays inside the workspace it is given.

Each workspace is exactly the size the sizing call returns
(psc_varlen_attn_workspace for passes 0-3, psc_pack_sizes for the packer),
placed between two 4 KiB guard bands of a sentinel byte in one allocation;
after the call (and a synchronisation) both bands must still hold the
sentinel.  Cases: the edge layout at every head width and both input dtypes,
the many-segment layout that takes the schedule's large path, the 2 x 32K
workload at full size, the rotary-fused passes, the debug library (whose
workspaces carry the cu_seqlens flags word) and the packer.
"""
import numpy as np
import pytest
import torch

import packed_sequence_causal_amd as psc
import workloads
from oracle import pack_ref

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
GUARD = 4096
SENT = 0xA5
EDGE = [1, 63, 64, 65, 127, 128, 129, 1, 1, 200, 300, 431]


def guarded(nbytes):
    buf = torch.full((nbytes + 2 * GUARD,), SENT, dtype=torch.uint8, device=DEV)
    return buf, buf[GUARD:GUARD + nbytes]


def assert_guards(buf, what):
    torch.cuda.synchronize()
    head, tail = buf[:GUARD], buf[-GUARD:]
    assert bool((head == SENT).all()) and bool((tail == SENT).all()), f"{what}: a guard band was overwritten"


def positions_of(cu):
    cu = np.asarray(cu, dtype=np.int64)
    T = int(cu[-1])
    seg = np.searchsorted(cu, np.arange(T), side="right") - 1
    return (np.arange(T) - cu[seg]).astype(np.int32)


def run_passes(cu, hq, hkv, D, dtype="bf16", rope=False, library=None):
    cu = np.asarray(cu, dtype=np.int32)
    T, nseg = int(cu[-1]), len(cu) - 1
    ml = int(np.diff(cu).max())
    q, k, v, do = workloads.qkv_do(T, hq, hkv, D, seed=5, dtype=dtype)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    cud = torch.as_tensor(cu).to(DEV)
    dt = psc.BF16 if dtype == "bf16" else psc.F32
    sizes = [psc.varlen_attn_workspace(p, dt, T, nseg, ml, hq, hkv, D, library=library)
             for p in range(4 if rope else 2)]
    print(f"  T={T} segments={nseg} heads {hq}/{hkv} D={D} {dtype} workspace bytes {sizes}", flush=True)
    kw = {} if library is None else {"library": library}
    b0, w0 = guarded(sizes[0])
    o, lse = psc.varlen_attn_fwd(qd, kd, vd, cud, ml, workspace=w0, **kw)
    assert_guards(b0, "forward")
    b1, w1 = guarded(sizes[1])
    psc.varlen_attn_bwd(qd, kd, vd, o, dod, lse, cud, ml, workspace=w1, **kw)
    assert_guards(b1, "backward")
    if rope:
        pos = torch.as_tensor(positions_of(cu)).to(DEV)
        b2, w2 = guarded(sizes[2])
        o2, lse2 = psc.varlen_attn_fwd_rope(qd, kd, vd, cud, ml, pos, workspace=w2)
        assert_guards(b2, "rotary forward")
        b3, w3 = guarded(sizes[3])
        psc.varlen_attn_bwd_rope(qd, kd, vd, o2, dod, lse2, cud, ml, pos, workspace=w3)
        assert_guards(b3, "rotary backward")


def edge_cu():
    return np.concatenate([[0], np.cumsum(EDGE)])


@pytest.mark.parametrize("hq,hkv,D,dtype,rope", [
    (8, 2, 128, "bf16", True),
    (4, 4, 64, "bf16", True),
    (4, 2, 32, "bf16", False),
    (2, 2, 32, "f32", False),
])
def test_edge_layout_stays_inside_its_workspaces(hq, hkv, D, dtype, rope):
    run_passes(edge_cu(), hq, hkv, D, dtype, rope)


def test_large_schedule_path_stays_inside_its_workspaces():
    rng = np.random.default_rng(11)
    lens = rng.integers(1, 40, 4600)
    run_passes(np.concatenate([[0], np.cumsum(lens)]), 4, 1, 64)


def test_debug_library_stays_inside_its_longer_workspaces():
    run_passes(edge_cu(), 8, 2, 128, library=psc.debug_lib())


def test_full_size_workload_stays_inside_its_workspaces():
    w = workloads.make("lognormal_32k")
    p = w.pack
    rows = pack_ref.build_pack(p.docs, p.micro_bsz, p.seq_len)[: p.keep_rows]
    cu = pack_ref.flatten(rows, p.packed_length)["cu_seqlens"]
    run_passes(cu, w.attn.hq, w.attn.hkv, w.attn.head_dim, rope=True)


@pytest.mark.parametrize("mode", [psc.PACK, psc.UNPACK])
def test_packer_stays_inside_its_workspace(mode):
    w = workloads.make("tiny")
    toks = torch.from_numpy(w.pack.tokens).to(DEV)
    offs = torch.from_numpy(w.pack.doc_offsets).to(DEV)
    _, _, ws = psc.pack_sizes(mode, len(w.pack.doc_offsets) - 1, len(w.pack.tokens), 2, 8)
    buf, wsp = guarded(ws)
    psc.pack_build(toks, offs, 2, 8, mode, workspace=wsp)
    assert_guards(buf, "packer")
