"""GPU data steps after the packer vs the scalar oracle, bit-exact:
packed_data_normalizer's per-row max_seqlen (psc_row_max_seqlen), unpack_data
(psc_unpack_data) and split_data_sequence_parallel (psc_split_sequence).

Cases: the page's printed examples (the normalised micro batch, both tp = 2
splits, the unpack_data result), every workload's document stream in both
packing modes, carry-over rows (documents longer than SEQ_LEN and more than
micro_bsz documents per row), empty documents, short last rows, tp from 1 to
the full length, and no rows at all.
"""
import numpy as np
import pytest
import torch

import packed_sequence_causal_amd as psc
from conftest import golden
from oracle import pack_ref
import workloads

pytestmark = pytest.mark.gpu


def _pack(docs, mb, sl, mode):
    lens = [len(d) for d in docs]
    toks = np.concatenate([np.asarray(d, dtype=np.int32) for d in docs]) if sum(lens) else np.zeros(0, np.int32)
    offs = np.zeros(len(docs) + 1, dtype=np.int64)
    offs[1:] = np.cumsum(lens)
    return psc.pack_build(torch.from_numpy(toks).cuda(), torch.from_numpy(offs).cuda(), mb, sl, mode)


def check_steps(docs, mb, sl, mode, tps=(1, 2, 4)):
    ref = (pack_ref.build_pack if mode == psc.PACK else pack_ref.build_unpack)(docs, mb, sl)
    pk = _pack(docs, mb, sl, mode)
    n = len(ref)
    # normaliser
    ms = psc.row_max_seqlen(pk).cpu().numpy()
    assert ms[:n].tolist() == [pack_ref.max_seqlen(r["cu_seqlens"]) for r in ref]
    # unpack_data
    ids, labels = psc.unpack_data(pk, mb, sl)
    ids, labels = ids.cpu().numpy(), labels.cpu().numpy()
    for r, row in enumerate(ref):
        un = pack_ref.unpack_data(row, mb, sl)
        assert ids[r * mb:(r + 1) * mb].tolist() == un["input_ids"], f"ids row {r}"
        assert labels[r * mb:(r + 1) * mb].tolist() == un["labels"], f"labels row {r}"
    # split of the packed rows and of the unpacked batch
    PL = mb * sl
    for tp in tps:
        if PL % tp or sl % tp:
            continue
        for rank in sorted({0, tp // 2, tp - 1}):
            for key in ("input_ids", "labels", "indexes"):
                got = psc.split_sequence(pk[key], tp, rank).cpu().numpy()[:n].tolist()
                assert got == pack_ref.split_sequence_parallel([r[key] for r in ref], tp, rank), (tp, rank, key)
            got = psc.split_sequence(torch.from_numpy(ids).cuda(), tp, rank).cpu().numpy()[: n * mb].tolist()
            assert got == pack_ref.split_sequence_parallel(ids[: n * mb].tolist(), tp, rank)


def test_page_examples():
    g = golden("p1_split_sp.json")
    gp = golden("p1_build_pack.json")
    pk = _pack(gp["docs"], gp["micro_bsz"], gp["seq_len"], psc.PACK)
    assert psc.row_max_seqlen(pk).cpu().tolist() == [g["packed"]["max_seqlen"], 8]
    for r, want in enumerate(g["packed"]["ranks"]):
        for key, gkey in (("input_ids", "input_ids"), ("indexes", "indexes"), ("labels", "label")):
            got = psc.split_sequence(pk[key], g["tp"], r).cpu().tolist()[0]
            assert got == want[gkey], (r, key)
    gu = golden("p1_unpack_data.json")
    pku = _pack(gu["docs"], gu["micro_bsz"], gu["seq_len"], psc.UNPACK)
    ids, labels = psc.unpack_data(pku, gu["micro_bsz"], gu["seq_len"])
    assert ids.cpu().tolist() == gu["input_ids"] and labels.cpu().tolist() == gu["labels"]
    for r, want in enumerate(g["unpacked"]["ranks"]):
        assert psc.split_sequence(ids, g["tp"], r).cpu().tolist() == want["input_ids"]
        assert psc.split_sequence(labels, g["tp"], r).cpu().tolist() == want["label"]


@pytest.mark.parametrize("name", ["tiny", "uniform_8k", "lognormal_32k", "seqpar_share_128k", "skewed_32k"])
@pytest.mark.parametrize("mode", [psc.PACK, psc.UNPACK])
def test_workload_streams(name, mode):
    w = workloads.make(name)
    docs = w.pack.docs
    mb, sl = w.pack.micro_bsz, w.pack.seq_len
    if mode == psc.UNPACK and w.pack.mode != workloads.BUILD_UNPACK and sl > 2048:
        mb, sl = 8, 2048  # truncate-and-pad rows of the same stream
    check_steps(docs, mb, sl, mode, tps=(2, 8))


@pytest.mark.parametrize("docs,mb,sl,mode", [
    ([[1] * 3, [2] * 9, [3] * 2, [4] * 2], 2, 8, psc.PACK),          # carry-over: a doc longer than SEQ_LEN
    ([[5] * 2, [6] * 2, [7] * 2, [8] * 2, [9] * 3], 2, 8, psc.PACK),  # more than micro_bsz docs per row
    ([[1] * 5, [], [2] * 3, [], [], [3] * 9], 2, 4, psc.UNPACK),      # empty documents, truncation
    ([[1] * 4, [2] * 4, [3] * 4], 2, 4, psc.UNPACK),                  # short last row
    ([[7] * 8, [8] * 8], 1, 8, psc.UNPACK),                           # rows exactly full, no padding
])
def test_edge_cases(docs, mb, sl, mode):
    check_steps(docs, mb, sl, mode, tps=(1, 2, mb * sl))


def test_split_full_width_and_no_rows():
    x = torch.arange(3 * 16, dtype=torch.int32, device="cuda").reshape(3, 16)
    for tp in (1, 16):
        for rank in (0, tp - 1):
            got = psc.split_sequence(x, tp, rank).cpu().tolist()
            assert got == pack_ref.split_sequence_parallel(x.cpu().tolist(), tp, rank)
    empty = torch.empty(0, 16, dtype=torch.int32, device="cuda")
    assert psc.split_sequence(empty, 4, 1).shape == (0, 4)
