"""Seeded synthetic inputs for the packing + document-causal attention path.

This module is the only code that the CPU oracle (``oracle/``) and the HIP path
share.  It draws random numbers and lays them out; it holds none of the
method's arithmetic (no packing, no boundaries, no attention).  The one
exception that is still pure input layout is the skewed-pack attention layout,
whose rows the workload itself defines segment by segment (see ``skewed_rows``).

Recipe (identical for every caller):
  * every length draw comes from ``numpy.random.default_rng(seed)``, one scalar
    draw at a time and in order; token ids are drawn after all lengths as
    ``rng.integers(1, 50000, size=n_tok, dtype=int32)``;
  * log-normal lengths: ``min(max(round(exp(ln(median) + sigma * z)), lo), hi)``
    with ``z = rng.standard_normal()`` and Python's ``round``;
  * a carry-over stream draws documents until their total reaches
    ``rows * packed_length``; the packer then yields one spill row more than
    needed, and callers keep the first ``rows`` rows;
  * Q, K, V, dO come from ``torch.Generator().manual_seed(seed)`` on the CPU,
    drawn N(0, 1) in fp32 in the order Q, K, V, dO with shapes [T, H, D], then
    cast to the workload dtype (bf16 rounds to nearest even).

The five workloads are named for what they are: ``tiny`` (4 docs of 4,7,8,5
tokens; a 16-token attention row of documents 3,4,5,4), ``uniform_8k``
(4 x 8192-token rows, lengths uniform [64, 2048], MHA 32 x 128, forward only),
``lognormal_32k`` (2 x 32768-token rows, log-normal median 1024 sigma 1.0,
GQA 32/8 x 128), ``seqpar_share_128k`` (one 131072-token row, log-normal
median 8192 sigma 1.2, GQA 4/1 x 128: one GPU's head share under
head-sharded sequence parallelism) and ``skewed_32k`` (2 x 32768-token rows,
one 16384-token document then documents uniform [1, 64], zero-padded tail,
MHA 64 x 64).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional

import numpy as np

TOKEN_LO, TOKEN_HI = 1, 50000

BUILD_PACK = "pack"
BUILD_UNPACK = "unpack"


@dataclass
class PackInput:
    """Documents for the packer, as the flat token array plus offsets."""

    docs: List[np.ndarray]
    micro_bsz: int
    seq_len: int
    mode: str
    keep_rows: Optional[int] = None  # rows of the pack that feed attention

    @property
    def packed_length(self) -> int:
        return self.micro_bsz * self.seq_len

    @property
    def tokens(self) -> np.ndarray:
        if not self.docs:
            return np.zeros(0, dtype=np.int32)
        return np.concatenate(self.docs).astype(np.int32, copy=False)

    @property
    def doc_offsets(self) -> np.ndarray:
        off = np.zeros(len(self.docs) + 1, dtype=np.int64)
        off[1:] = np.cumsum([len(d) for d in self.docs])
        return off


@dataclass
class AttnShape:
    hq: int
    hkv: int
    head_dim: int
    dtype: str  # "f32" or "bf16"
    backward: bool


@dataclass
class Workload:
    name: str
    pack: PackInput
    attn: AttnShape
    # Attention layout given directly by the workload (tiny, skewed); None means
    # "the first keep_rows rows of the packer's output".
    attn_cu_seqlens: Optional[np.ndarray] = None
    # Per segment of the directly given layout: True where the segment is a
    # row's zero-padded tail (computed like any segment, never counted as work).
    attn_is_pad: Optional[np.ndarray] = None


def _lognormal_len(rng, median, sigma, lo, hi):
    z = rng.standard_normal()
    return min(max(round(math.exp(math.log(median) + sigma * z)), lo), hi)


def _ids(rng, lengths):
    n = int(sum(lengths))
    toks = rng.integers(TOKEN_LO, TOKEN_HI, size=n, dtype=np.int32)
    out, p = [], 0
    for L in lengths:
        out.append(toks[p:p + L].copy())
        p += L
    return out


def _carry_stream(rng, draw, total):
    lengths, acc = [], 0
    while acc < total:
        L = int(draw(rng))
        lengths.append(L)
        acc += L
    return lengths


def tiny(seed: int = 0) -> Workload:
    rng = np.random.default_rng(seed)
    docs = _ids(rng, [4, 7, 8, 5])
    layout = np.array([0, 3, 7, 12, 16], dtype=np.int32)
    return Workload("tiny", PackInput(docs, 2, 8, BUILD_PACK),
                    AttnShape(2, 2, 32, "f32", True), attn_cu_seqlens=layout)


def uniform_8k(seed: int = 0) -> Workload:
    rng = np.random.default_rng(seed)
    lengths = _carry_stream(rng, lambda r: r.integers(64, 2049), 4 * 8192)
    return Workload("uniform_8k", PackInput(_ids(rng, lengths), 8, 1024, BUILD_PACK, keep_rows=4),
                    AttnShape(32, 32, 128, "bf16", False))


def lognormal_32k(seed: int = 0) -> Workload:
    rng = np.random.default_rng(seed)
    lengths = _carry_stream(rng, lambda r: _lognormal_len(r, 1024, 1.0, 16, 32768), 2 * 32768)
    # SEQ_LEN is not fixed by the workload; carry-over packing depends only on
    # micro_bsz * SEQ_LEN, so one 32768-token micro-batch slot is used.
    return Workload("lognormal_32k", PackInput(_ids(rng, lengths), 1, 32768, BUILD_PACK, keep_rows=2),
                    AttnShape(32, 8, 128, "bf16", True))


def seqpar_share_128k(seed: int = 0) -> Workload:
    rng = np.random.default_rng(seed)
    lengths = _carry_stream(rng, lambda r: _lognormal_len(r, 8192, 1.2, 128, 131072), 131072)
    return Workload("seqpar_share_128k", PackInput(_ids(rng, lengths), 1, 131072, BUILD_PACK, keep_rows=1),
                    AttnShape(4, 1, 128, "bf16", True))


def skewed_rows(rng, rows=2, row_len=32768, long_doc=16384, lo=1, hi=64):
    """Per row: one long document, then short documents drawn uniform [lo, hi]
    while they still fit; the first draw that does not fit is discarded and the
    rest of the row is a zero-padded tail.  Returns (per-row doc lengths,
    per-row pad lengths)."""
    per_row, pads = [], []
    for _ in range(rows):
        lens, used = [long_doc], long_doc
        while True:
            L = int(rng.integers(lo, hi + 1))
            if used + L > row_len:
                break
            lens.append(L)
            used += L
        per_row.append(lens)
        pads.append(row_len - used)
    return per_row, pads


def skewed_32k(seed: int = 0) -> Workload:
    rng = np.random.default_rng(seed)
    per_row, pads = skewed_rows(rng)
    lengths = [L for row in per_row for L in row]
    docs = _ids(rng, lengths)
    # Attention layout: each row's documents, then its padding tail as the last
    # segment of the row.  Offsets are the running total of these lengths.
    seg, is_pad = [], []
    for row, pad in zip(per_row, pads):
        seg.extend(row)
        is_pad.extend([False] * len(row))
        if pad:
            seg.append(pad)
            is_pad.append(True)
    layout = np.zeros(len(seg) + 1, dtype=np.int32)
    layout[1:] = np.cumsum(seg)
    # The packer itself runs the literal truncate-and-pad rule over the same
    # document stream (micro_bsz 16, SEQ_LEN 2048).
    return Workload("skewed_32k", PackInput(docs, 16, 2048, BUILD_UNPACK),
                    AttnShape(64, 64, 64, "bf16", True), attn_cu_seqlens=layout,
                    attn_is_pad=np.array(is_pad, dtype=bool))


WORKLOADS = {
    "tiny": tiny,
    "uniform_8k": uniform_8k,
    "lognormal_32k": lognormal_32k,
    "seqpar_share_128k": seqpar_share_128k,
    "skewed_32k": skewed_32k,
}


def make(name: str, seed: int = 0) -> Workload:
    return WORKLOADS[name](seed)


def qkv_do(T: int, hq: int, hkv: int, head_dim: int, seed: int = 0, dtype: str = "bf16"):
    """Q [T,hq,D], K [T,hkv,D], V [T,hkv,D], dO [T,hq,D] as CPU torch tensors of
    the workload dtype, drawn N(0,1) in fp32 in that order."""
    import torch

    g = torch.Generator().manual_seed(seed)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    q = torch.randn(T, hq, head_dim, generator=g, dtype=torch.float32).to(tdt)
    k = torch.randn(T, hkv, head_dim, generator=g, dtype=torch.float32).to(tdt)
    v = torch.randn(T, hkv, head_dim, generator=g, dtype=torch.float32).to(tdt)
    do = torch.randn(T, hq, head_dim, generator=g, dtype=torch.float32).to(tdt)
    return q, k, v, do


def random_docs(rng, n_docs, lo, hi, allow_empty=False):
    """Documents with lengths uniform [lo, hi] (0 allowed if allow_empty) and
    token ids uniform [1, 50000); used by property tests."""
    lengths = [int(rng.integers(0 if allow_empty else lo, hi + 1)) for _ in range(n_docs)]
    return _ids(rng, lengths)


def random_layout(rng, total, lo, hi):
    """Segment lengths uniform [lo, hi] (last one clipped) that exactly fill
    ``total`` tokens, as offsets; for attention property tests."""
    lens, acc = [], 0
    while acc < total:
        L = min(int(rng.integers(lo, hi + 1)), total - acc)
        lens.append(L)
        acc += L
    off = np.zeros(len(lens) + 1, dtype=np.int32)
    off[1:] = np.cumsum(lens)
    return off


# Document layouts of one 32768-token row for the document-length sweep: the
# three named on the Sample Packing page (section 5.3: one 32K document,
# 16K + 16K, 2K + 30K) and further splits, longest document from S to S/32.
DOC_SWEEP_ROW = 32768
DOC_SWEEP = {
    "32K": [32768],
    "30K+2K": [30720, 2048],
    "2K+30K": [2048, 30720],
    "24K+8K": [24576, 8192],
    "16K+16K": [16384, 16384],
    "4x8K": [8192] * 4,
    "8x4K": [4096] * 8,
    "16x2K": [2048] * 16,
    "32x1K": [1024] * 32,
}


def doc_sweep_cu(name: str, whole_row: bool = False) -> np.ndarray:
    """cu_seqlens of a sweep layout, or of the same row as one causal segment."""
    lens = [DOC_SWEEP_ROW] if whole_row else DOC_SWEEP[name]
    assert sum(lens) == DOC_SWEEP_ROW
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)

