"""C ABI checks that need no GPU: the library loads, exports every function
include/psc.h declares, sizes come out as documented, and invalid arguments
are rejected on the host (these paths make no HIP call)."""
import ctypes
import os
import re

import pytest

import packed_sequence_causal_amd as psc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "psc.h")

pytestmark = pytest.mark.skipif(not os.path.exists(psc.LIB_PATH), reason="libpsc.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(psc_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"psc_pack_build", "psc_varlen_attn_fwd", "psc_varlen_attn_bwd"} <= set(names)
    L = psc.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(psc._SIGNATURES), "binding and header disagree"


def test_strerror_and_version():
    assert psc.strerror(0) == "ok"
    assert "workspace" in psc.strerror(psc.ERR_WORKSPACE)
    assert psc.lib().psc_version() >= 100


@pytest.mark.parametrize("mode,n_docs,n_tok,mb,sl,rows,segs", [
    (psc.PACK, 4, 24, 2, 8, 2, 8),
    (psc.UNPACK, 6, 44, 2, 8, 3, 9),
    (psc.PACK, 0, 0, 2, 8, 0, 0),
    (psc.PACK, 47, 70000, 1, 32768, 3, 53),
    (psc.UNPACK, 980, 100000, 16, 2048, 62, 1042),
])
def test_pack_sizes(mode, n_docs, n_tok, mb, sl, rows, segs):
    r, s, ws = psc.pack_sizes(mode, n_docs, n_tok, mb, sl)
    assert (r, s) == (rows, segs)
    assert ws > 0


@pytest.mark.parametrize("args", [
    (2, 4, 24, 2, 8),          # unknown mode
    (0, -1, 24, 2, 8),         # negative docs
    (0, 4, 24, 0, 8),          # micro_bsz < 1
    (0, 4, 24, 2, 0),          # seq_len < 1
    (0, 4, 24, 1 << 16, 1 << 15),  # packed length beyond 2^30
])
def test_pack_sizes_rejects(args):
    with pytest.raises(psc.PscError) as e:
        psc.pack_sizes(*args)
    assert e.value.status == psc.ERR_INVALID


def _pack_build_raw(**kw):
    a = dict(mode=0, tokens=1, offs=1, n_docs=4, n_tok=24, mb=2, sl=8, rows=2, ids=1, lab=1, idx=1, cu=1, cap=8,
             rsp=1, rvl=None, stats=1, ws=1, wsb=1 << 20)
    a.update(kw)
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return psc.lib().psc_pack_build(a["mode"], v(a["tokens"]), v(a["offs"]), a["n_docs"], a["n_tok"], a["mb"],
                                    a["sl"], a["rows"], v(a["ids"]), v(a["lab"]), v(a["idx"]), v(a["cu"]),
                                    a["cap"], v(a["rsp"]), v(a["rvl"]), v(a["stats"]), v(a["ws"]), a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(rows=3), psc.ERR_INVALID),
    (dict(offs=None), psc.ERR_INVALID),
    (dict(tokens=None), psc.ERR_INVALID),
    (dict(ids=None), psc.ERR_INVALID),
    (dict(stats=None), psc.ERR_INVALID),
    (dict(cap=7), psc.ERR_CAPACITY),
    (dict(ws=None), psc.ERR_WORKSPACE),
    (dict(wsb=16), psc.ERR_WORKSPACE),
    (dict(n_docs=0, n_tok=24), psc.ERR_INVALID),
])
def test_pack_build_rejects_on_host(kw, code):
    assert _pack_build_raw(**kw) == code


def _fwd_raw(**kw):
    a = dict(dtype=psc.BF16, q=16, k=16, v=16, sq=256, sk=128, sv=128, cu=16, nseg=1, maxlen=16, T=16, hq=2, hkv=1,
             d=128, scale=0.0, out=16, so=256, lse=16, ws=16, wsb=1 << 24)
    a.update(kw)
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return psc.lib().psc_varlen_attn_fwd(a["dtype"], v(a["q"]), v(a["k"]), v(a["v"]), a["sq"], a["sk"], a["sv"],
                                         v(a["cu"]), a["nseg"], a["maxlen"], a["T"], a["hq"], a["hkv"], a["d"],
                                         a["scale"], v(a["out"]), a["so"], v(a["lse"]), v(a["ws"]), a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), psc.ERR_UNSUPPORTED),
    (dict(d=48, wsb=8), psc.ERR_UNSUPPORTED),   # checked before the workspace
    (dict(hq=3, hkv=2), psc.ERR_INVALID),        # hq % hkv != 0
    (dict(dtype=7), psc.ERR_INVALID),
    (dict(q=None), psc.ERR_INVALID),
    (dict(q=8), psc.ERR_INVALID),                # misaligned base for bf16
    (dict(sq=200), psc.ERR_INVALID),             # stride below heads*D
    (dict(sk=130), psc.ERR_INVALID),             # stride*2 not a multiple of 16 bytes
    (dict(sv=(1 << 25) + 8), psc.ERR_INVALID),   # a 64-row bf16 tile would need byte offsets >= 2^32
    (dict(cu=None), psc.ERR_INVALID),
    (dict(lse=None), psc.ERR_INVALID),
    (dict(nseg=0), psc.ERR_INVALID),
    (dict(maxlen=17), psc.ERR_INVALID),          # longer than T
    (dict(ws=None), psc.ERR_WORKSPACE),
    (dict(wsb=8), psc.ERR_WORKSPACE),
    (dict(scale=float("nan")), psc.ERR_INVALID),
])
def test_attn_fwd_rejects_on_host(kw, code):
    assert _fwd_raw(**kw) == code


# The cases below pass fake device pointers that are otherwise valid, so only
# the check under test stands between them and a launch: they run only where
# no GPU driver is present (a missing check then shows as PSC_ERR_HIP).
no_gpu_driver = pytest.mark.skipif(os.path.exists("/dev/kfd"),
                                   reason="launch-capable fake pointers: run on hosts without a GPU only")


@no_gpu_driver
def test_misaligned_workspace_is_rejected():
    assert _fwd_raw(ws=24) == psc.ERR_INVALID
    assert _pack_build_raw(ws=24) == psc.ERR_INVALID
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    bwd = [psc.BF16, psc.F32, v(16), v(16), v(16), v(16), v(16), v(16), 256, 128, 128, 256, 256, v(16), 1, 16, 16,
           2, 1, 128, 0.0, v(16), v(16), v(16), v(24), 1 << 24, None]
    assert psc.lib().psc_varlen_attn_bwd(*bwd) == psc.ERR_INVALID
    assert _rope_fwd_raw(ws=24, wsb=1 << 24) == psc.ERR_INVALID
    bwd_rope = [psc.BF16, psc.F32, v(16), v(16), v(16), v(16), v(16), v(16), 256, 128, 128, 256, 256, v(16), 1, 16,
                16, 2, 1, 128, v(16), 10000.0, 0.0, v(16), v(16), v(16), v(24), 1 << 24, None]
    assert psc.lib().psc_varlen_attn_bwd_rope(*bwd_rope) == psc.ERR_INVALID


def test_attn_empty_is_a_no_op():
    assert _fwd_raw(T=0, nseg=0, maxlen=0, q=None, k=None, v=None, out=None, lse=None, cu=None, ws=None) == 0


def test_attn_bwd_rejects_on_host():
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    L = psc.lib()
    # every case below also has too small a workspace, so nothing could be
    # launched on these fake pointers even if the check under test were missing
    base = [psc.BF16, psc.F32, v(16), v(16), v(16), v(16), v(16), v(16), 256, 128, 128, 256, 256, v(16), 1, 16, 16,
            2, 1, 128, 0.0, v(16), v(16), v(16), v(16), 8, None]
    assert L.psc_varlen_attn_bwd(*base) == psc.ERR_WORKSPACE
    bad_dq = list(base)
    bad_dq[21] = None
    assert L.psc_varlen_attn_bwd(*bad_dq) == psc.ERR_INVALID
    bad_hd = list(base)
    bad_hd[19] = 48
    assert L.psc_varlen_attn_bwd(*bad_hd) == psc.ERR_UNSUPPORTED
    mis = list(base)
    mis[22] = v(20)  # dk not 16-byte aligned
    assert L.psc_varlen_attn_bwd(*mis) == psc.ERR_INVALID
    for g, code in ((7, psc.ERR_INVALID), (-1, psc.ERR_INVALID)):
        bad_g = list(base)
        bad_g[1] = g
        assert L.psc_varlen_attn_bwd(*bad_g) == code
    f32_bf16 = list(base)
    f32_bf16[0], f32_bf16[1] = psc.F32, psc.BF16  # bf16 gradients need bf16 inputs
    assert L.psc_varlen_attn_bwd(*f32_bf16) == psc.ERR_UNSUPPORTED
    bf16_bf16 = list(base)
    bf16_bf16[1] = psc.BF16
    assert L.psc_varlen_attn_bwd(*bf16_bf16) == psc.ERR_WORKSPACE  # accepted up to the workspace check


def test_head_dim_32_is_supported_for_both_dtypes():
    for dt in (psc.F32, psc.BF16):
        assert psc.varlen_attn_workspace(0, dt, 4096, 8, 1024, 8, 2, 32) > 0
        assert psc.varlen_attn_workspace(1, dt, 4096, 8, 1024, 8, 2, 32) > 0
    with pytest.raises(psc.PscError) as e:
        psc.varlen_attn_workspace(0, psc.BF16, 4096, 8, 1024, 8, 2, 96)
    assert e.value.status == psc.ERR_UNSUPPORTED


def test_cu_seqlens_status_host_mapping():
    # the flags word psc_check_cu_seqlens writes, mapped on the host
    assert psc.cu_seqlens_status(0) == psc.OK
    for f in (psc.CU_BAD_START, psc.CU_BAD_END, psc.CU_NOT_INCREASING, 3, 5, 6, 7):
        assert psc.cu_seqlens_status(f) == psc.ERR_INVALID
    assert psc.lib().psc_debug_checks() == 0


def test_debug_library_reports_its_checks():
    if not os.path.exists(psc.DEBUG_LIB_PATH):
        pytest.skip("libpsc_debug.so not built")
    D = psc.debug_lib()
    assert D.psc_debug_checks() == 1
    assert D.psc_cu_seqlens_status(psc.CU_NOT_INCREASING) == psc.ERR_INVALID
    # the debug build keeps a flags word at the end of each attention workspace
    b_rel, b_dbg = ctypes.c_size_t(), ctypes.c_size_t()
    assert psc.lib().psc_varlen_attn_workspace(0, psc.BF16, 4096, 8, 1024, 8, 2, 128, ctypes.byref(b_rel)) == 0
    assert D.psc_varlen_attn_workspace(0, psc.BF16, 4096, 8, 1024, 8, 2, 128, ctypes.byref(b_dbg)) == 0
    assert b_dbg.value == b_rel.value + 256
    # and the binding's sizing call asks the library it is given
    assert psc.varlen_attn_workspace(1, psc.BF16, 4096, 8, 1024, 8, 2, 128, library=D) == \
        psc.varlen_attn_workspace(1, psc.BF16, 4096, 8, 1024, 8, 2, 128) + 256


@pytest.mark.parametrize("cu,n,T,flags", [(None, 3, 16, 16), (16, 3, 16, None), (16, -1, 16, 16),
                                          (16, 3, -1, 16), (16, 3, 1 << 31, 16)])
def test_check_cu_seqlens_rejects_on_host(cu, n, T, flags):
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    assert psc.lib().psc_check_cu_seqlens(v(cu), n, T, v(flags), None) == psc.ERR_INVALID


def test_binding_rejects_mismatched_buffers_before_the_call():
    import torch

    T, hq, hkv, D = 16, 2, 1, 64
    q = torch.zeros(T, hq, D, dtype=torch.bfloat16)
    k = torch.zeros(T, hkv, D, dtype=torch.bfloat16)
    cu = torch.tensor([0, T], dtype=torch.int32)
    lse = torch.zeros(hq, T)
    with pytest.raises(ValueError):  # k in another dtype than q
        psc.varlen_attn_fwd(q, k.float(), k, cu, T)
    with pytest.raises(ValueError):  # cu_seqlens not int32
        psc.varlen_attn_fwd(q, k, k, cu.long(), T)
    with pytest.raises(ValueError):  # lse of the wrong shape
        psc.varlen_attn_fwd(q, k, k, cu, T, out=q.clone(), lse=torch.zeros(T, hq))
    with pytest.raises(ValueError):  # out in another dtype
        psc.varlen_attn_fwd(q, k, k, cu, T, out=q.float(), lse=lse)
    g32 = dict(dtype=torch.float32)
    with pytest.raises(ValueError):  # dq in bf16 while fp32 gradients are asked for
        psc.varlen_attn_bwd(q, k, k, q, q, lse, cu, T, dq=torch.zeros(T, hq, D, dtype=torch.bfloat16),
                            dk=torch.zeros(T, hkv, D, **g32), dv=torch.zeros(T, hkv, D, **g32))
    with pytest.raises(ValueError):  # dk too small
        psc.varlen_attn_bwd(q, k, k, q, q, lse, cu, T, dq=torch.zeros(T, hq, D, **g32),
                            dk=torch.zeros(T - 1, hkv, D, **g32), dv=torch.zeros(T, hkv, D, **g32))
    with pytest.raises(ValueError):  # dv not contiguous
        psc.varlen_attn_bwd(q, k, k, q, q, lse, cu, T, dq=torch.zeros(T, hq, D, **g32),
                            dk=torch.zeros(T, hkv, D, **g32), dv=torch.zeros(T, hkv, 2 * D, **g32)[..., ::2])
    with pytest.raises(ValueError):  # bf16 gradients asked for, fp32 buffers given
        psc.varlen_attn_bwd(q, k, k, q, q, lse, cu, T, dq=torch.zeros(T, hq, D, **g32),
                            dk=torch.zeros(T, hkv, D, **g32), dv=torch.zeros(T, hkv, D, **g32),
                            grad_dtype=psc.BF16)
    # a caller's workspace is checked, never replaced
    ws = psc.varlen_attn_workspace(0, psc.BF16, T, 1, T, hq, hkv, D)
    wb = psc.varlen_attn_workspace(1, psc.BF16, T, 1, T, hq, hkv, D)
    with pytest.raises(ValueError, match="needs"):  # one byte short
        psc.varlen_attn_fwd(q, k, k, cu, T, out=q.clone(), lse=lse, workspace=torch.zeros(ws - 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="uint8"):  # not bytes
        psc.varlen_attn_fwd(q, k, k, cu, T, out=q.clone(), lse=lse, workspace=torch.zeros(ws, dtype=torch.int32))
    with pytest.raises(ValueError, match="contiguous"):  # strided
        psc.varlen_attn_fwd(q, k, k, cu, T, out=q.clone(), lse=lse,
                            workspace=torch.zeros(2 * ws, dtype=torch.uint8)[::2])
    with pytest.raises(ValueError, match="needs"):
        psc.varlen_attn_bwd(q, k, k, q, q, lse, cu, T, dq=torch.zeros(T, hq, D, **g32),
                            dk=torch.zeros(T, hkv, D, **g32), dv=torch.zeros(T, hkv, D, **g32),
                            workspace=torch.zeros(wb - 1, dtype=torch.uint8))


def test_attn_workspace_sizes():
    fwd = psc.varlen_attn_workspace(0, psc.BF16, 65536, 48, 4654, 32, 8, 128)
    bwd = psc.varlen_attn_workspace(1, psc.BF16, 65536, 48, 4654, 32, 8, 128)
    assert 0 < fwd < (1 << 20)
    assert bwd >= 4 * 32 * 65536  # D row sums in fp32
    # the fused-rotary passes add the (cos, sin) table: max_seqlen x D/2 float2
    fr = psc.varlen_attn_workspace(2, psc.BF16, 65536, 48, 4654, 32, 8, 128)
    br = psc.varlen_attn_workspace(3, psc.BF16, 65536, 48, 4654, 32, 8, 128)
    assert fr >= fwd + 4654 * 64 * 8 and br >= bwd + 4654 * 64 * 8
    for bad in (4, -1):
        with pytest.raises(psc.PscError):
            psc.varlen_attn_workspace(bad, psc.BF16, 16, 1, 16, 2, 1, 128)


def _rope_raw(**kw):
    a = dict(dtype=psc.BF16, q=16, sq=256, hq=2, k=16, sk=128, hkv=1, T=16, D=128, pos=16, base=10000.0, inv=0)
    a.update(kw)
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return psc.lib().psc_rope(a["dtype"], v(a["q"]), a["sq"], a["hq"], v(a["k"]), a["sk"], a["hkv"], a["T"],
                              a["D"], v(a["pos"]), a["base"], a["inv"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), psc.ERR_INVALID),
    (dict(q=None), psc.ERR_INVALID),
    (dict(pos=None), psc.ERR_INVALID),
    (dict(q=24), psc.ERR_INVALID),             # q not 16-byte aligned
    (dict(sq=200), psc.ERR_INVALID),           # stride below heads*D
    (dict(dtype=psc.F32, sq=258), psc.ERR_INVALID),  # stride*4 not a multiple of 16 bytes
    (dict(k=16, hkv=0), psc.ERR_INVALID),
    (dict(base=0.0), psc.ERR_INVALID),
    (dict(base=-2.0), psc.ERR_INVALID),
    (dict(base=float("inf")), psc.ERR_INVALID),
    (dict(base=float("nan")), psc.ERR_INVALID),
    (dict(D=96), psc.ERR_UNSUPPORTED),
    (dict(T=-1), psc.ERR_INVALID),
])
def test_rope_rejects_on_host(kw, code):
    assert _rope_raw(**kw) == code


def test_rope_empty_is_a_no_op():
    assert _rope_raw(T=0, q=None, k=None, pos=None) == 0
    assert _rope_raw(T=0) == 0



def _vp(x):
    return None if x is None else ctypes.c_void_p(x)


def _unpack_raw(**kw):
    a = dict(ids=16, labels=16, n_rows=2, PL=16, cu=16, n_cu=8, rsp=16, rvl=16, mb=2, sl=8, oi=16, ol=16)
    a.update(kw)
    return psc.lib().psc_unpack_data(_vp(a["ids"]), _vp(a["labels"]), a["n_rows"], a["PL"], _vp(a["cu"]), a["n_cu"],
                                     _vp(a["rsp"]), _vp(a["rvl"]), a["mb"], a["sl"], _vp(a["oi"]), _vp(a["ol"]),
                                     None)


@pytest.mark.parametrize("kw", [dict(n_rows=-1), dict(PL=0), dict(mb=0), dict(sl=0), dict(n_cu=0),
                                dict(ids=None), dict(rvl=None), dict(oi=None), dict(cu=None),
                                dict(n_rows=1 << 20, PL=1 << 12)])
def test_unpack_data_rejects_on_host(kw):
    assert _unpack_raw(**kw) == psc.ERR_INVALID


def test_unpack_data_no_rows_is_a_no_op():
    assert _unpack_raw(n_rows=0, ids=None, labels=None, cu=None, rsp=None, rvl=None, oi=None, ol=None) == 0


@pytest.mark.parametrize("args", [(16, -1, 16, 2, 0, 16), (16, 2, 16, 0, 0, 16), (16, 2, 16, 2, 2, 16),
                                  (16, 2, 16, 2, -1, 16), (16, 2, 15, 2, 0, 16), (None, 2, 16, 2, 0, 16),
                                  (16, 2, 16, 2, 0, None)])
def test_split_sequence_rejects_on_host(args):
    i, rows, length, tp, rank, o = args
    assert psc.lib().psc_split_sequence(_vp(i), rows, length, tp, rank, _vp(o), None) == psc.ERR_INVALID


def test_split_and_row_max_no_ops():
    L = psc.lib()
    assert L.psc_split_sequence(None, 0, 16, 4, 1, None, None) == 0
    assert L.psc_row_max_seqlen(None, 1, None, 0, None, None) == 0
    assert L.psc_row_max_seqlen(None, 0, None, 0, None, None) == psc.ERR_INVALID
    assert L.psc_row_max_seqlen(_vp(16), 4, _vp(16), 2, None, None) == psc.ERR_INVALID
    assert L.psc_row_max_seqlen(_vp(16), 4, _vp(16), -1, _vp(16), None) == psc.ERR_INVALID


def test_noalloc_forward_rejects_sizes_beyond_its_scratch():
    # 2^28 tokens need a 128 MiB tile list, beyond the 4 MiB built-in scratch:
    # rejected before any HIP call (the fake pointers are never used)
    T = 1 << 28
    v = ctypes.c_void_p(256)
    L = psc.lib()
    assert L.psc_varlen_attn_fwd_noalloc(psc.BF16, v, v, v, 1024, 256, 256, v, 1, T, T, 8, 2, 128, 0.0, v, 1024, v,
                                         None) == psc.ERR_WORKSPACE
    # argument checks come first, as in psc_varlen_attn_fwd
    assert L.psc_varlen_attn_fwd_noalloc(psc.BF16, None, v, v, 1024, 256, 256, v, 1, 16, 16, 8, 2, 128, 0.0, v,
                                         1024, v, None) == psc.ERR_INVALID
    assert L.psc_varlen_attn_fwd_noalloc(psc.BF16, v, v, v, 1024, 256, 256, v, 1, 16, 16, 8, 2, 96, 0.0, v, 1024,
                                         v, None) == psc.ERR_UNSUPPORTED


def _rope_fwd_raw(**kw):
    a = dict(dtype=psc.BF16, q=16, k=16, v=16, sq=256, sk=128, sv=128, cu=16, nseg=1, maxlen=16, T=16, hq=2, hkv=1,
             d=128, pos=16, base=10000.0, scale=0.0, out=16, so=256, lse=16, ws=16, wsb=8)
    a.update(kw)
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return psc.lib().psc_varlen_attn_fwd_rope(a["dtype"], v(a["q"]), v(a["k"]), v(a["v"]), a["sq"], a["sk"], a["sv"],
                                              v(a["cu"]), a["nseg"], a["maxlen"], a["T"], a["hq"], a["hkv"], a["d"],
                                              v(a["pos"]), a["base"], a["scale"], v(a["out"]), a["so"], v(a["lse"]),
                                              v(a["ws"]), a["wsb"], None)


# every case has too small a workspace (8 bytes): nothing can be launched on
# these fake pointers even if the check under test were missing
@pytest.mark.parametrize("kw,code", [
    (dict(), psc.ERR_WORKSPACE),                       # otherwise valid
    (dict(dtype=psc.F32, sq=256, sk=128, sv=128), psc.ERR_UNSUPPORTED),  # fp32 inputs
    (dict(d=32, sq=64, sk=32, sv=32, so=64), psc.ERR_UNSUPPORTED),      # head_dim 32
    (dict(pos=None), psc.ERR_INVALID),
    (dict(base=0.0), psc.ERR_INVALID),
    (dict(base=float("nan")), psc.ERR_INVALID),
    (dict(q=None), psc.ERR_INVALID),
])
def test_attn_fwd_rope_rejects_on_host(kw, code):
    assert _rope_fwd_raw(**kw) == code


def test_attn_bwd_rope_rejects_on_host():
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    L = psc.lib()
    base = [psc.BF16, psc.F32, v(16), v(16), v(16), v(16), v(16), v(16), 256, 128, 128, 256, 256, v(16), 1, 16, 16,
            2, 1, 128, v(16), 10000.0, 0.0, v(16), v(16), v(16), v(16), 8, None]
    assert L.psc_varlen_attn_bwd_rope(*base) == psc.ERR_WORKSPACE
    for idx, val, code in ((20, None, psc.ERR_INVALID), (21, -1.0, psc.ERR_INVALID), (19, 64, psc.ERR_WORKSPACE),
                           (1, 7, psc.ERR_INVALID)):
        bad = list(base)
        bad[idx] = val
        assert L.psc_varlen_attn_bwd_rope(*bad) == code, (idx, val)
    f32 = list(base)
    f32[0] = psc.F32
    assert L.psc_varlen_attn_bwd_rope(*f32) == psc.ERR_UNSUPPORTED
