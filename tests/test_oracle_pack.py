"""Pins of the scalar packer oracle.

* the page's printed build_pack / build_unpack / unpack_data examples, value
  for value (tests/golden/p1_*.json, each citing its section);
* invariants on random document sets that any correct packer satisfies, stated
  independently of the oracle's own construction (token conservation, the
  label rule per document, boundary / indexes consistency, row counts).
"""
import numpy as np
import pytest

from conftest import golden
from oracle import pack_ref
import workloads


def test_build_pack_page_example():
    g = golden("p1_build_pack.json")
    rows = pack_ref.build_pack(g["docs"], g["micro_bsz"], g["seq_len"])
    assert [r["input_ids"] for r in rows] == g["input_ids"]
    assert [r["labels"] for r in rows] == g["labels"]
    assert [r["cu_seqlens"] for r in rows] == g["cu_seqlens"]
    assert [r["indexes"] for r in rows] == g["indexes"]
    assert rows[0]["max_seqlen"] == g["max_seqlen_row0"]


def test_build_unpack_page_example():
    g = golden("p1_build_unpack.json")
    rows = pack_ref.build_unpack(g["docs"], g["micro_bsz"], g["seq_len"])
    assert [r["input_ids"] for r in rows] == g["input_ids"]
    assert [r["labels"] for r in rows] == g["labels"]


def test_unpack_data_page_example_pins_unpack_boundaries():
    # build_unpack's cu_seqlens are not printed; splitting its row at them must
    # give back the page's unpack_data result.
    g = golden("p1_unpack_data.json")
    rows = pack_ref.build_unpack(g["docs"], g["micro_bsz"], g["seq_len"])
    assert len(rows) == 1
    assert rows[0]["input_ids"] == g["packed_input_ids"]
    assert rows[0]["labels"] == g["packed_labels"]
    assert rows[0]["cu_seqlens"] == [0, 4, 11, 16]
    un = pack_ref.unpack_data(rows[0], g["micro_bsz"], g["seq_len"])
    assert un["input_ids"] == g["input_ids"]
    assert un["labels"] == g["labels"]


def test_normalizer_and_split_sp_page_examples():
    # the first micro batch of the page's build_pack example after
    # packed_data_normalizer, and both tp = 2 splits (packed and unpacked)
    g = golden("p1_split_sp.json")
    gp = golden("p1_build_pack.json")
    row = pack_ref.build_pack(gp["docs"], gp["micro_bsz"], gp["seq_len"])[0]
    pk = g["packed"]
    assert row["input_ids"] == pk["input_ids"]
    assert row["labels"] == pk["label"]
    assert row["indexes"] == pk["indexes"]
    assert row["cu_seqlens"] == pk["cu_seqlens"]
    assert pack_ref.max_seqlen(row["cu_seqlens"]) == pk["max_seqlen"] == row["max_seqlen"]
    for r, want in enumerate(pk["ranks"]):
        for key, src in (("input_ids", row["input_ids"]), ("indexes", row["indexes"]), ("label", row["labels"])):
            assert pack_ref.split_sequence_parallel([src], g["tp"], r) == [want[key]], (r, key)
    gu = golden("p1_unpack_data.json")
    urow = pack_ref.build_unpack(gu["docs"], gu["micro_bsz"], gu["seq_len"])[0]
    un = pack_ref.unpack_data(urow, gu["micro_bsz"], gu["seq_len"])
    up = g["unpacked"]
    assert un["input_ids"] == up["input_ids"] and un["labels"] == up["label"]
    for r, want in enumerate(up["ranks"]):
        assert pack_ref.split_sequence_parallel(un["input_ids"], g["tp"], r) == want["input_ids"]
        assert pack_ref.split_sequence_parallel(un["labels"], g["tp"], r) == want["label"]


@pytest.mark.parametrize("tp", [1, 2, 4, 8, 16])
def test_split_sp_ranks_concatenate_back(tp):
    rng = np.random.default_rng(tp)
    rows = [list(rng.integers(-100, 50000, 32)) for _ in range(3)]
    parts = [pack_ref.split_sequence_parallel(rows, tp, r) for r in range(tp)]
    for i, row in enumerate(rows):
        assert sum((p[i] for p in parts), []) == row


def test_unpack_data_of_carry_over_rows_keeps_first_docs_cut():
    # reading: at most micro_bsz documents, each cut to seq_len
    row = pack_ref.build_pack([[1] * 3, [2] * 9, [3] * 2, [4] * 2], 2, 8)[0]  # segments 3, 9, 2, 2
    un = pack_ref.unpack_data(row, 2, 8)
    assert un["input_ids"] == [[1, 1, 1, 0, 0, 0, 0, 0], [2] * 8]
    assert un["labels"][1] == [2] * 8  # the cut keeps the document's own next-token labels


def _check_row_structure(row, PL):
    cu = row["cu_seqlens"]
    assert cu[0] == 0 and cu[-1] == PL
    assert all(b > a for a, b in zip(cu, cu[1:]))
    starts = set(cu[:-1])
    idx = row["indexes"]
    for p in range(PL):
        if p in starts:
            assert idx[p] == 0
        else:
            assert idx[p] == idx[p - 1] + 1
    assert row["max_seqlen"] == max(b - a for a, b in zip(cu, cu[1:]))
    v = row["valid_len"]
    assert all(t == 0 for t in row["input_ids"][v:])
    assert all(t == -100 for t in row["labels"][v:])
    if v < PL:
        assert v in cu


def _doc_walk(rows, PL):
    """Positions of all valid tokens in row-major order."""
    out = []
    for r, row in enumerate(rows):
        for p in range(row["valid_len"]):
            out.append((r, p))
    return out


@pytest.mark.parametrize("seed", range(6))
def test_build_pack_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    micro_bsz, seq_len = int(rng.integers(1, 4)), int(rng.integers(2, 12))
    PL = micro_bsz * seq_len
    docs = workloads.random_docs(rng, int(rng.integers(1, 30)), 1, 3 * PL, allow_empty=True)
    rows = pack_ref.build_pack(docs, micro_bsz, seq_len)
    nonempty = [list(map(int, d)) for d in docs if len(d)]
    total = sum(len(d) for d in nonempty)
    assert len(rows) == -(-total // PL)
    for row in rows:
        _check_row_structure(row, PL)
    # token conservation and the per-document label rule across row cuts
    walk = _doc_walk(rows, PL)
    assert len(walk) == total
    k = 0
    for d in nonempty:
        for t in range(len(d)):
            r, p = walk[k]
            assert rows[r]["input_ids"][p] == d[t]
            assert rows[r]["labels"][p] == (d[t + 1] if t + 1 < len(d) else -100)
            # a document start inside a row is a boundary; a row start always is
            if t == 0 or p == 0:
                assert p in rows[r]["cu_seqlens"]
            else:
                assert p not in rows[r]["cu_seqlens"]
            k += 1
    # only the last row may hold padding
    assert all(r["valid_len"] == PL for r in rows[:-1])


@pytest.mark.parametrize("seed", range(6))
def test_build_unpack_invariants(seed):
    rng = np.random.default_rng(200 + seed)
    micro_bsz, seq_len = int(rng.integers(1, 5)), int(rng.integers(2, 10))
    PL = micro_bsz * seq_len
    docs = workloads.random_docs(rng, int(rng.integers(1, 25)), 1, 2 * seq_len, allow_empty=True)
    rows = pack_ref.build_unpack(docs, micro_bsz, seq_len)
    kept = [list(map(int, d))[:seq_len] for d in docs if len(d)]
    assert len(rows) == -(-len(kept) // micro_bsz)
    for r, row in enumerate(rows):
        _check_row_structure(row, PL)
        group = kept[r * micro_bsz:(r + 1) * micro_bsz]
        p = 0
        for d in group:
            assert p in row["cu_seqlens"]
            for t in range(len(d)):
                assert row["input_ids"][p] == d[t]
                assert row["labels"][p] == (d[t + 1] if t + 1 < len(d) else -100)
                if t:
                    assert p not in row["cu_seqlens"]
                p += 1
        assert row["valid_len"] == p
        un = pack_ref.unpack_data(row, micro_bsz, seq_len)
        for i, d in enumerate(group):
            assert un["input_ids"][i][: len(d)] == d


def test_flatten_global_view():
    g = golden("p1_build_pack.json")
    rows = pack_ref.build_pack(g["docs"], g["micro_bsz"], g["seq_len"])
    f = pack_ref.flatten(rows, 16)
    assert f["cu_seqlens"] == [0, 4, 11, 16, 19, 24, 32]
    assert f["row_seg_ptr"] == [0, 3, 6]
    assert f["n_seg"] == 6 and f["max_seqlen"] == 8
    assert f["row_valid_len"] == [16, 8]
    for r in range(2):
        a, b = f["row_seg_ptr"][r], f["row_seg_ptr"][r + 1]
        assert [c - 16 * r for c in f["cu_seqlens"][a:b + 1]] == rows[r]["cu_seqlens"]


def test_empty_inputs():
    assert pack_ref.build_pack([], 2, 8) == []
    assert pack_ref.build_unpack([[], []], 2, 8) == []
    f = pack_ref.flatten([], 16)
    assert f["cu_seqlens"] == [0] and f["n_seg"] == 0


def test_exact_fill_has_no_padding_segment():
    rows = pack_ref.build_pack([[1, 2, 3], [4, 5, 6, 7, 8]], 1, 8)
    assert len(rows) == 1 and rows[0]["cu_seqlens"] == [0, 3, 8]
    rows = pack_ref.build_pack([[1] * 8, [2] * 8], 2, 4)
    assert [r["cu_seqlens"] for r in rows] == [[0, 8], [0, 8]]
