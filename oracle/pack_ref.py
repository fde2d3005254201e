"""Scalar packer oracle: build_pack (carry-over) and build_unpack (truncate, pad).

Test infrastructure only (see ``oracle/__init__``).

Source: InternEvo documentation, page "数据加载与流程" (data flow):
  * section "Dataloader加载数据": the two packing rules with worked examples
    (micro_bsz 2, SEQ_LEN 8) for build_pack and build_unpack, and the label rule;
  * section "获取Dataloader数据": the batch contract (input_ids, cu_seqlens,
    indexes, label) with the same example's cu_seqlens and indexes;
  * section "处理数据": packed_data_normalizer's max_seqlen, unpack_data and
    split_data_sequence_parallel (tp = 2 examples for packed and unpacked data).

Readings taken where the page is silent:
  * labels are formed per whole document before a row split, so the last token
    of a row whose document continues gets the next document token as label;
  * a carried-over fragment at a row start is its own segment; a zero-padded
    tail is one final segment; indexes restart at 0 in every segment;
  * build_unpack truncates a document to SEQ_LEN before forming its labels;
  * documents with no tokens are dropped before packing (they add no tokens, no
    segment, and do not count towards micro_bsz);
  * build_unpack's rows take the documents in order, micro_bsz per row, and its
    cu_seqlens / indexes follow the same convention as build_pack's;
  * unpack_data keeps a row's first micro_bsz documents, each cut to seq_len
    (both always hold for build_unpack rows; they only matter for carry-over
    rows, which the page never unpacks);
  * split_data_sequence_parallel cuts the last (sequence) dimension of every
    row into tp equal contiguous slices, rank r taking slice r; the length
    must be a multiple of tp.

Pins: tests/test_oracle_pack.py (the page's printed examples, byte for byte,
plus invariants on random inputs).
"""
from __future__ import annotations

from typing import Dict, List, Sequence

PAD_ID = 0
IGNORE = -100


def _row_from_pieces(ids, labels, boundaries, packed_length):
    """Pad one row and derive cu_seqlens / indexes / max_seqlen.

    ``boundaries`` are the segment starts inside the row (document starts,
    row start).  The valid length ends one more segment when padding follows.
    """
    valid = len(ids)
    ids = list(ids) + [PAD_ID] * (packed_length - valid)
    labels = list(labels) + [IGNORE] * (packed_length - valid)
    cuts = set(boundaries)
    cuts.add(0)
    cuts.add(packed_length)
    if valid < packed_length:
        cuts.add(valid)
    cu = sorted(cuts)
    # indexes: position of each token counted from the start of its segment
    indexes = []
    seg = 0
    for p in range(packed_length):
        while seg + 1 < len(cu) and cu[seg + 1] <= p:
            seg += 1
        indexes.append(p - cu[seg])
    max_seqlen = max(cu[i + 1] - cu[i] for i in range(len(cu) - 1))
    return {
        "input_ids": ids,
        "labels": labels,
        "cu_seqlens": cu,
        "indexes": indexes,
        "max_seqlen": max_seqlen,
        "valid_len": valid,
    }


def build_pack(docs: Sequence[Sequence[int]], micro_bsz: int, seq_len: int) -> List[Dict]:
    """Carry-over packing.

    All documents are laid end to end in one stream that is cut every
    ``micro_bsz * seq_len`` tokens; a document that crosses a cut continues at
    the start of the next row; only the last row is padded (ids 0, labels -100).
    Labels are each document's tokens shifted left by one, -100 at its end.
    """
    packed_length = micro_bsz * seq_len
    stream, lab, starts = [], [], []
    for d in docs:
        d = [int(t) for t in d]
        if not d:
            continue
        starts.append(len(stream))
        stream.extend(d)
        lab.extend(d[1:] + [IGNORE])
    n_rows = -(-len(stream) // packed_length)
    rows = []
    for r in range(n_rows):
        lo, hi = r * packed_length, (r + 1) * packed_length
        inner = [s - lo for s in starts if lo < s < hi]
        rows.append(_row_from_pieces(stream[lo:hi], lab[lo:hi], inner, packed_length))
    return rows


def build_unpack(docs: Sequence[Sequence[int]], micro_bsz: int, seq_len: int) -> List[Dict]:
    """Truncate-and-pad packing.

    Each row holds at most ``micro_bsz`` documents, even when space is left;
    every document is cut to its first ``seq_len`` tokens (the rest is thrown
    away) before its labels are formed; the row is padded to
    ``micro_bsz * seq_len`` with ids 0 and labels -100.  (The third rule, cutting
    a row that exceeds micro_bsz * seq_len, can never fire after the first two.)
    """
    packed_length = micro_bsz * seq_len
    kept = [[int(t) for t in d][:seq_len] for d in docs if len(d) > 0]
    rows = []
    for g in range(0, len(kept), micro_bsz):
        group = kept[g:g + micro_bsz]
        ids, labels, starts = [], [], []
        for d in group:
            starts.append(len(ids))
            ids.extend(d)
            labels.extend(d[1:] + [IGNORE])
        assert len(ids) <= packed_length
        rows.append(_row_from_pieces(ids, labels, starts, packed_length))
    return rows


def flatten(rows: List[Dict], packed_length: int) -> Dict:
    """Global view of a list of rows: rows laid end to end.

    cu_seqlens of all rows become one strictly increasing array from 0 to
    n_rows * packed_length (a row end is always a segment end, so rows never
    share a segment); row_seg_ptr[r] is the index of row r's first boundary.
    """
    cu, row_seg_ptr = [0], [0]
    for r, row in enumerate(rows):
        base = r * packed_length
        cu.extend(base + b for b in row["cu_seqlens"][1:])
        row_seg_ptr.append(len(cu) - 1)
    return {
        "input_ids": [t for row in rows for t in row["input_ids"]],
        "labels": [t for row in rows for t in row["labels"]],
        "indexes": [t for row in rows for t in row["indexes"]],
        "cu_seqlens": cu,
        "row_seg_ptr": row_seg_ptr,
        "row_valid_len": [row["valid_len"] for row in rows],
        "n_seg": len(cu) - 1,
        "max_seqlen": max((row["max_seqlen"] for row in rows), default=0),
    }


def unpack_data(row: Dict, micro_bsz: int, seq_len: int) -> Dict:
    """Inverse view of one packed row (section "处理数据", unpack_data).

    Splits the row at its cu_seqlens into its documents and places document i
    in slot i of a [micro_bsz, seq_len] batch, padded with ids 0 and labels
    -100.  The padding tail segment, if any, is not a document.  Used here to
    check the build_unpack boundary reading against the page's printed
    unpack_data example.
    """
    cu = row["cu_seqlens"]
    ends = cu[1:]
    if row["valid_len"] < cu[-1]:
        ends = [e for e in ends if e <= row["valid_len"]]
    starts = cu[:len(ends)]
    ids = [[PAD_ID] * seq_len for _ in range(micro_bsz)]
    labels = [[IGNORE] * seq_len for _ in range(micro_bsz)]
    for i, (s, e) in enumerate(zip(starts, ends)):
        if i >= micro_bsz:
            break
        e = min(e, s + seq_len)
        ids[i][: e - s] = row["input_ids"][s:e]
        labels[i][: e - s] = row["labels"][s:e]
    return {"input_ids": ids, "labels": labels}


def split_sequence_parallel(rows: Sequence[Sequence[int]], tp: int, rank: int) -> List[List[int]]:
    """Slice `rank` of the sequence dimension cut into `tp` equal parts
    (section "处理数据", split_data_sequence_parallel)."""
    out = []
    for r in rows:
        n = len(r)
        assert n % tp == 0 and 0 <= rank < tp
        w = n // tp
        out.append(list(r[rank * w:(rank + 1) * w]))
    return out


def max_seqlen(cu_seqlens: Sequence[int]) -> int:
    """packed_data_normalizer's max_seqlen: the longest segment of a row."""
    return max(b - a for a, b in zip(cu_seqlens[:-1], cu_seqlens[1:]))
