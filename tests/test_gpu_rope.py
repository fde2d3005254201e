"""GPU rotary embedding (psc_rope) vs the fp64 oracle (oracle/rope_ref.py).

bf16: every element within half a bf16 ulp of the exact value plus 2e-5 (the
kernel rounds an fp32 result once); fp32: within 1e-5 absolute.  Cases: the
packer's indexes of the page's example and of the lognormal 32k pack (the full
q and k of that workload, in place), positions up to 131071, head dims 32, 64,
128, grouped heads, k as a view into a packed kv buffer (v untouched), q
alone, and the inverse rotation.
"""
import numpy as np
import pytest
import torch

import packed_sequence_causal_amd as psc
from oracle import pack_ref, rope_ref
import workloads

pytestmark = pytest.mark.gpu


def _ulp_bf16(x):
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def check(name, got, ref, dtype):
    got = got.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    tol = 0.5 * _ulp_bf16(ref) + 2e-5 if dtype == torch.bfloat16 else np.full(ref.shape, 1e-5)
    bad = err > tol
    assert not bad.any(), f"{name}: {bad.sum()} elements off, worst {err.max():.3g}"


def _rope_gpu(q, k, pos, **kw):
    qd = q.cuda()
    kd = None if k is None else k.cuda()
    psc.rope(qd, kd, torch.from_numpy(np.asarray(pos, np.int32)).cuda(), **kw)
    torch.cuda.synchronize()
    return qd.cpu(), None if kd is None else kd.cpu()


def _qk(T, hq, hkv, D, seed, dtype):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(T, hq, D, generator=g).to(dtype)
    k = torch.randn(T, hkv, D, generator=g).to(dtype)
    return q, k


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D", [32, 64, 128])
def test_page_example_positions(dtype, D):
    # the page's example docs (lengths 4, 7, 8, 5; micro_bsz 2, SEQ_LEN 8),
    # positions = the packer's indexes
    docs = [[1] * 4, [2] * 7, [3] * 8, [4] * 5]
    rows = pack_ref.build_pack(docs, 2, 8)
    pos = np.concatenate([r["indexes"] for r in rows])
    q, k = _qk(len(pos), 4, 2, D, 0, dtype)
    gq, gk = _rope_gpu(q, k, pos)
    check("q", gq, rope_ref.rope(q.float().numpy(), pos), dtype)
    check("k", gk, rope_ref.rope(k.float().numpy(), pos), dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_long_positions_and_base(dtype):
    rng = np.random.default_rng(5)
    T = 777
    pos = rng.integers(0, 131072, T)
    pos[:3] = [0, 131071, 65536]
    q, k = _qk(T, 6, 3, 128, 1, dtype)
    for base in (10000.0, 1000000.0):
        gq, gk = _rope_gpu(q, k, pos, base=base)
        check(f"q base {base}", gq, rope_ref.rope(q.float().numpy(), pos, base=base), dtype)
        check(f"k base {base}", gk, rope_ref.rope(k.float().numpy(), pos, base=base), dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_inverse_and_q_alone(dtype):
    rng = np.random.default_rng(6)
    T = 300
    pos = rng.integers(0, 40000, T)
    q, k = _qk(T, 4, 4, 64, 2, dtype)
    gq, _ = _rope_gpu(q, None, pos, inverse=True)
    check("q inverse", gq, rope_ref.rope(q.float().numpy(), pos, inverse=True), dtype)


def test_packed_kv_view_rotates_k_only():
    T, hkv, D = 513, 2, 128
    rng = np.random.default_rng(7)
    pos = rng.integers(0, 5000, T)
    g = torch.Generator().manual_seed(3)
    q = torch.randn(T, 8, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(T, 2, hkv, D, generator=g).to(torch.bfloat16)
    kvd = kv.cuda()
    qd = q.cuda()
    psc.rope(qd, kvd[:, 0], torch.from_numpy(pos.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    check("q", qd.cpu(), rope_ref.rope(q.float().numpy(), pos), torch.bfloat16)
    check("k view", kvd[:, 0].cpu(), rope_ref.rope(kv[:, 0].float().numpy(), pos), torch.bfloat16)
    assert torch.equal(kvd[:, 1].cpu(), kv[:, 1]), "v must be untouched"


def test_lognormal_32k_full_size_with_gpu_packer_indexes():
    w = workloads.make("lognormal_32k")
    a = w.attn
    dev = torch.device("cuda:0")
    pk = psc.pack_build(torch.from_numpy(w.pack.tokens).to(dev), torch.from_numpy(w.pack.doc_offsets).to(dev),
                        w.pack.micro_bsz, w.pack.seq_len, psc.PACK)
    PL = w.pack.micro_bsz * w.pack.seq_len
    pos_d = pk["indexes"][: w.pack.keep_rows].reshape(-1).contiguous()
    T = pos_d.numel()
    q, k, _, _ = workloads.qkv_do(T, a.hq, a.hkv, a.head_dim, seed=0, dtype="bf16")
    qd, kd = q.to(dev), k.to(dev)
    psc.rope(qd, kd, pos_d)
    torch.cuda.synchronize()
    pos = pos_d.cpu().numpy()
    rng = np.random.default_rng(8)
    rows = np.concatenate([rng.integers(0, T, 256), [0, T - 1, PL - 1, PL]])
    check("q rows", qd[rows].cpu(), rope_ref.rope(q[rows].float().numpy(), pos[rows]), torch.bfloat16)
    check("k rows", kd[rows].cpu(), rope_ref.rope(k[rows].float().numpy(), pos[rows]), torch.bfloat16)
