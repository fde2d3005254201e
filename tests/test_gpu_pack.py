"""GPU packer vs the scalar oracle: bit-exact on every output.

Cases: the page's printed examples, every workload's document stream (the
skewed one through the literal truncate-and-pad rule, 62 rows), and edge cases
(a document ending exactly at a row end, a stream that fills its rows exactly,
one-token documents, empty documents, a last truncate row with fewer than
micro_bsz documents, no documents at all), random sweeps, and one row of the
largest length the ABI accepts (2^30 tokens).
"""
import numpy as np
import pytest
import torch

import packed_sequence_causal_amd as psc
from conftest import golden
from oracle import pack_ref
import workloads

pytestmark = pytest.mark.gpu


def _gpu_pack(docs, mb, sl, mode):
    lens = [len(d) for d in docs]
    toks = np.concatenate([np.asarray(d, dtype=np.int32) for d in docs]) if sum(lens) else np.zeros(0, np.int32)
    offs = np.zeros(len(docs) + 1, dtype=np.int64)
    offs[1:] = np.cumsum(lens)
    t = torch.from_numpy(toks).cuda()
    o = torch.from_numpy(offs).cuda()
    r = psc.pack_build(t, o, mb, sl, mode)
    torch.cuda.synchronize()
    stats = r["stats"].cpu().tolist()
    n_seg = stats[0]
    return {
        "ids": r["input_ids"].cpu().numpy(),
        "labels": r["labels"].cpu().numpy(),
        "indexes": r["indexes"].cpu().numpy(),
        "cu": r["cu_seqlens"][: n_seg + 1].cpu().numpy(),
        "row_seg_ptr": r["row_seg_ptr"].cpu().numpy(),
        "row_valid": r["row_valid_len"].cpu().numpy(),
        "stats": stats,
    }


def check(docs, mb, sl, mode):
    PL = mb * sl
    ref_rows = (pack_ref.build_pack if mode == psc.PACK else pack_ref.build_unpack)(docs, mb, sl)
    f = pack_ref.flatten(ref_rows, PL)
    g = _gpu_pack(docs, mb, sl, mode)
    n = len(ref_rows)
    n_seg, max_seqlen, filled, flag = g["stats"]
    assert flag == 0
    assert filled == n
    assert n_seg == f["n_seg"]
    assert max_seqlen == f["max_seqlen"]
    assert g["ids"][:n].reshape(-1).tolist() == f["input_ids"]
    assert g["labels"][:n].reshape(-1).tolist() == f["labels"]
    assert g["indexes"][:n].reshape(-1).tolist() == f["indexes"]
    assert g["cu"].tolist() == f["cu_seqlens"]
    assert g["row_seg_ptr"][: n + 1].tolist() == f["row_seg_ptr"]
    if n:
        assert g["row_valid"][:n].tolist() == f["row_valid_len"]
    # rows past the filled ones (truncate mode with empty documents) are padding
    rows = g["ids"].shape[0]
    if rows > n:
        assert (g["ids"][n:] == 0).all() and (g["labels"][n:] == -100).all()
        assert (g["row_seg_ptr"][n:] == n_seg).all()
    return f


def test_page_build_pack_example():
    gd = golden("p1_build_pack.json")
    f = check(gd["docs"], gd["micro_bsz"], gd["seq_len"], psc.PACK)
    assert f["cu_seqlens"] == [0, 4, 11, 16, 19, 24, 32]


def test_page_build_unpack_example():
    gd = golden("p1_build_unpack.json")
    check(gd["docs"], gd["micro_bsz"], gd["seq_len"], psc.UNPACK)


@pytest.mark.parametrize("mode", [psc.PACK, psc.UNPACK])
def test_tiny_workload_both_modes(mode):
    w = workloads.make("tiny")
    check(w.pack.docs, 2, 8, mode)


@pytest.mark.parametrize("name", ["uniform_8k", "lognormal_32k", "seqpar_share_128k"])
def test_carry_over_workloads(name):
    w = workloads.make(name)
    f = check(w.pack.docs, w.pack.micro_bsz, w.pack.seq_len, psc.PACK)
    assert len(f["row_valid_len"]) >= w.pack.keep_rows


def test_skewed_workload_literal_unpack():
    w = workloads.make("skewed_32k")
    f = check(w.pack.docs, 16, 2048, psc.UNPACK)
    assert len(f["row_valid_len"]) == 62


@pytest.mark.parametrize("docs,mb,sl", [
    ([[1, 2, 3, 4], [5, 6, 7, 8], [9]], 1, 4),            # documents end exactly at row ends
    ([[1] * 8, [2] * 8], 2, 4),                           # exact fill, no padding
    ([[7]] * 11, 2, 3),                                   # one-token documents
    ([[1, 2], [], [3, 4, 5], [], [], [6]], 2, 2),         # empty documents
    ([[1, 2, 3], [4, 5, 6, 7, 8, 9, 10, 11]], 3, 4),      # one long document across rows
    ([], 2, 8),                                           # nothing
])
@pytest.mark.parametrize("mode", [psc.PACK, psc.UNPACK])
def test_edge_cases(docs, mb, sl, mode):
    check(docs, mb, sl, mode)


def test_unpack_last_row_short_and_truncation():
    docs = [[i] * (i + 3) for i in range(1, 8)]  # 7 docs, some longer than SEQ_LEN
    check(docs, 3, 5, psc.UNPACK)


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("mode", [psc.PACK, psc.UNPACK])
def test_random_sweep(seed, mode):
    rng = np.random.default_rng(7000 + seed)
    mb, sl = int(rng.integers(1, 9)), int(rng.integers(1, 300))
    docs = workloads.random_docs(rng, int(rng.integers(1, 3000)), 1, 3 * sl, allow_empty=True)
    check(docs, mb, sl, mode)


def test_repeat_is_identical():
    w = workloads.make("lognormal_32k")
    a = _gpu_pack(w.pack.docs, 1, 32768, psc.PACK)
    b = _gpu_pack(w.pack.docs, 1, 32768, psc.PACK)
    for key in ("ids", "labels", "indexes", "cu", "row_seg_ptr"):
        assert np.array_equal(a[key], b[key])


@pytest.mark.parametrize("mode", [psc.PACK, psc.UNPACK])
def test_row_of_the_largest_length(mode):
    # one row of 2^30 tokens (the limit: rows x row length must fit cu_seqlens'
    # int32): two documents, then 2^30 - 12 padding tokens.  The document part
    # is compared with the oracle packing the same documents into a 28-token
    # row; padding at sampled positions with its closed form (id 0, label
    # -100, indexes counting from the end of the documents).
    docs = [[11, 12, 13, 14, 15], [21, 22, 23, 24, 25, 26, 27]]
    used = sum(len(d) for d in docs)
    mb, sl = (1, 1 << 30) if mode == psc.PACK else (2, 1 << 29)
    PL = mb * sl
    toks = torch.tensor([t for d in docs for t in d], dtype=torch.int32).cuda()
    offs = torch.tensor([0, 5, 12], dtype=torch.int64).cuda()
    print(f"  packed row length {PL}, mode {mode}", flush=True)
    r = psc.pack_build(toks, offs, mb, sl, mode)
    torch.cuda.synchronize()
    n_seg, max_seqlen, filled, flag = r["stats"].cpu().tolist()
    assert (n_seg, max_seqlen, filled, flag) == (3, PL - used, 1, 0)
    assert r["cu_seqlens"][:4].cpu().tolist() == [0, 5, used, PL]
    assert r["row_seg_ptr"][:2].cpu().tolist() == [0, 3]
    assert r["row_valid_len"][:1].cpu().tolist() == [used]
    small_mb, small_sl = (1, 28) if mode == psc.PACK else (2, 14)
    ref_rows = (pack_ref.build_pack if mode == psc.PACK else pack_ref.build_unpack)(docs, small_mb, small_sl)
    f = pack_ref.flatten(ref_rows, 28)
    head = 28
    assert r["input_ids"][0, :head].cpu().tolist() == f["input_ids"]
    assert r["labels"][0, :head].cpu().tolist() == f["labels"]
    assert r["indexes"][0, :head].cpu().tolist() == f["indexes"]
    rng = np.random.default_rng(5)
    pos = np.concatenate([rng.integers(used, PL, 4096), [used, PL - 2, PL - 1]])
    idx = torch.from_numpy(pos).cuda()
    assert (r["input_ids"][0, idx] == 0).all()
    assert (r["labels"][0, idx] == -100).all()
    assert r["indexes"][0, idx].cpu().numpy().tolist() == (pos - used).tolist()
