"""Sparsity of the document-causal mask, by element and by square block.

Test infrastructure only (see ``oracle/__init__``).

Definitions (plain): the mask over a row of S tokens keeps (i, j) when i and j
lie in the same document and j <= i.  Element sparsity is the fraction of the
S*S entries that are cleared.  Block sparsity at block size B is the fraction
of the (S/B)^2 tiles of B x B entries in which every entry is cleared: the
tiles a tiled kernel can skip outright ("Sample Packing：长序列 LLM 训练的
Attention 问题及优化", section 5.1 on FlashAttention's three kinds of tiles,
and section 5.3 whose two-16K-documents-in-32K example reports the sparsity
that holds at 128 x 128 tiles).

The block count is formed from explicit rows of the mask, a chunk of B rows at
a time, so no S x S matrix is ever held.
"""
from __future__ import annotations

import numpy as np


def _doc_ids(cu_seqlens):
    cu = np.asarray(cu_seqlens, dtype=np.int64).reshape(-1)
    T = int(cu[-1])
    ids = np.zeros(T, dtype=np.int64)
    for d in range(len(cu) - 1):
        ids[cu[d]:cu[d + 1]] = d
    return ids


def element_sparsity(cu_seqlens):
    ids = _doc_ids(cu_seqlens)
    T = ids.shape[0]
    kept = 0
    for i in range(T):
        # entries j <= i in the same document as i
        kept += int(np.count_nonzero(ids[: i + 1] == ids[i]))
    return 1.0 - kept / float(T * T)


def block_sparsity(cu_seqlens, block):
    ids = _doc_ids(cu_seqlens)
    T = ids.shape[0]
    assert T % block == 0
    nb = T // block
    cols = np.arange(T)
    nonempty = 0
    for bi in range(nb):
        r = np.arange(bi * block, (bi + 1) * block)
        m = (ids[r][:, None] == ids[None, :]) & (cols[None, :] <= r[:, None])
        tiles = m.reshape(block, nb, block).any(axis=(0, 2))
        nonempty += int(np.count_nonzero(tiles))
    return 1.0 - nonempty / float(nb * nb)
