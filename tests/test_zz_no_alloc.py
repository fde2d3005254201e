"""The allocation-free forward (psc_varlen_attn_fwd_noalloc) against the
forward with a caller workspace, through the C ABI: bit for bit, on two calls
in a row with the second smaller (the scratch keeps the first call's contents,
which must not leak into the second), on bf16 and fp32 inputs, plus its
rejection of sizes beyond the built-in scratch (host side, nothing launched)."""
import ctypes

import numpy as np
import pytest
import torch

import packed_sequence_causal_amd as psc
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _raw_noalloc(q, k, v, cu, max_seqlen, out, lse, stream=None):
    T, hq, D = q.shape
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    s = torch.cuda.current_stream() if stream is None else stream
    return psc.lib().psc_varlen_attn_fwd_noalloc(
        psc.BF16 if q.dtype == torch.bfloat16 else psc.F32, vp(q), vp(k), vp(v), q.stride(0), k.stride(0),
        v.stride(0), vp(cu), cu.numel() - 1, max_seqlen, T, hq, k.shape[1], D, 0.0, vp(out), out.stride(0), vp(lse),
        ctypes.c_void_p(s.cuda_stream))


def _case(lens, hq, hkv, D, seed, dtype="bf16"):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v, _ = workloads.qkv_do(T, hq, hkv, D, seed=seed, dtype=dtype)
    return q.to(DEV), k.to(DEV), v.to(DEV), torch.as_tensor(cu).to(DEV), int(np.diff(cu).max())


def _check_pair(q, k, v, cu, ml):
    T, hq, D = q.shape
    ref_o, ref_l = psc.varlen_attn_fwd(q, k, v, cu, ml)
    out = torch.full((T, hq, D), 5.0, dtype=q.dtype, device=DEV)
    lse = torch.full((hq, T), 5.0, dtype=torch.float32, device=DEV)
    assert _raw_noalloc(q, k, v, cu, ml, out, lse) == psc.OK
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o)
    assert torch.equal(lse, ref_l)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_forward_twice_second_smaller(dtype):
    big = [1, 63, 64, 65, 127, 128, 129, 1, 1, 200, 300, 431, 2000, 37]
    small = [5, 70, 3]
    for lens, seed in ((big, 1), (small, 2)):
        _check_pair(*_case(lens, 8, 2, 128 if dtype == "bf16" else 64, seed, dtype))


def test_noalloc_full_size_workload_then_smaller():
    w = workloads.make("lognormal_32k")
    from oracle import pack_ref

    p = w.pack
    rows = pack_ref.build_pack(p.docs, p.micro_bsz, p.seq_len)[: p.keep_rows]
    cu = np.asarray(pack_ref.flatten(rows, p.packed_length)["cu_seqlens"], dtype=np.int32)
    T = int(cu[-1])
    q, k, v, _ = workloads.qkv_do(T, 32, 8, 128, seed=0, dtype="bf16")
    _check_pair(q.to(DEV), k.to(DEV), v.to(DEV), torch.as_tensor(cu).to(DEV), int(np.diff(cu).max()))
    _check_pair(*_case([3, 900, 17, 64], 32, 8, 128, 5))


def test_noalloc_on_a_side_stream():
    q, k, v, cu, ml = _case([100, 33, 700], 4, 1, 64, 7)
    ref_o, ref_l = psc.varlen_attn_fwd(q, k, v, cu, ml)
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    out = torch.empty_like(ref_o)
    lse = torch.empty_like(ref_l)
    st.wait_stream(torch.cuda.current_stream())
    assert _raw_noalloc(q, k, v, cu, ml, out, lse, stream=st) == psc.OK
    st.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    # 2^28 tokens need a 128 MiB tile list; rejected before any HIP call, so
    # the fake pointers below are never used
    T = 1 << 28
    v = ctypes.c_void_p(256)
    st = psc.lib().psc_varlen_attn_fwd_noalloc(psc.BF16, v, v, v, 1024, 256, 256, v, 1, T, T, 8, 2, 128, 0.0, v,
                                               1024, v, None)
    assert st == psc.ERR_WORKSPACE
