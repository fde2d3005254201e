"""The seeded workloads follow their recipe (lengths, counts, segment layout).

Expected figures are those the recipe yields for seed 0; the segment layouts of
the carry-over workloads come from the oracle packer (first ``keep_rows`` rows).
"""
import numpy as np
import pytest

from oracle import pack_ref
import workloads


def _attn_layout(w):
    if w.attn_cu_seqlens is not None:
        return np.asarray(w.attn_cu_seqlens)
    p = w.pack
    rows = pack_ref.build_pack(p.docs, p.micro_bsz, p.seq_len)[: p.keep_rows]
    return np.asarray(pack_ref.flatten(rows, p.packed_length)["cu_seqlens"])


def _tri(cu, skip_last_per_row=0):
    L = np.diff(cu).astype(np.int64)
    return int((L * (L + 1) // 2).sum())


def test_tiny():
    w = workloads.make("tiny")
    assert [len(d) for d in w.pack.docs] == [4, 7, 8, 5]
    toks = w.pack.tokens
    assert toks.min() >= 1 and toks.max() < 50000
    assert list(w.attn_cu_seqlens) == [0, 3, 7, 12, 16]


@pytest.mark.parametrize("name,n_docs,first,n_seg,tri,max_len", [
    ("uniform_8k", 30, [1752, 1328, 1078, 599, 675, 145], 33, 21798476, None),
    ("lognormal_32k", 47, [1161, 897, 1943], 48, 77201323, 4654),
    ("seqpar_share_128k", 11, [9526, 6991, 17666], 11, 1459273673, 39172),
])
def test_carry_over_streams(name, n_docs, first, n_seg, tri, max_len):
    w = workloads.make(name)
    lens = [len(d) for d in w.pack.docs]
    assert len(lens) == n_docs
    assert lens[: len(first)] == first
    cu = _attn_layout(w)
    assert cu[-1] == w.pack.keep_rows * w.pack.packed_length
    assert len(cu) - 1 == n_seg
    assert _tri(cu) == tri
    if max_len:
        assert np.diff(cu).max() == max_len


def test_skewed():
    w = workloads.make("skewed_32k")
    cu = w.attn_cu_seqlens
    assert cu[-1] == 65536
    assert len(cu) - 1 == 982
    assert len(w.pack.docs) == 980
    L = np.diff(cu).astype(np.int64)
    pad_idx = np.nonzero(w.attn_is_pad)[0]
    assert L[pad_idx].tolist() == [24, 4]
    assert [int(cu[i + 1]) for i in pad_idx] == [32768, 65536]
    # real tokens and in-document pairs exclude each row's padding segment
    real = L.sum() - L[pad_idx].sum()
    assert real == 65508
    tri_real = int((L * (L + 1) // 2).sum() - (L[pad_idx] * (L[pad_idx] + 1) // 2).sum())
    assert tri_real == 269183538
    rows = pack_ref.build_unpack(w.pack.docs, 16, 2048)
    assert len(rows) == 62


def test_qkv_shapes_and_dtype():
    import torch

    q, k, v, do = workloads.qkv_do(16, 4, 2, 32, seed=0, dtype="bf16")
    assert q.shape == (16, 4, 32) and k.shape == (16, 2, 32) and do.dtype == torch.bfloat16
    q2, *_ = workloads.qkv_do(16, 4, 2, 32, seed=0, dtype="bf16")
    assert torch.equal(q, q2)
