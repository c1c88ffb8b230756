"""Plain CPU gather of the rows that sparse_indices select (oracle of li_gather).

TEST INFRASTRUCTURE ONLY: tests/, the smoke check and the bench's CPU-baseline
leg use it to check the HIP library against; the product package never imports it.

Follows the aclnnSparseFlashAttentionGrad page, calculation formula: the
selected key (and value) is the gather of key (value) by topkIndices[i] for
i < selectBlockCount, each index selecting a block of selectedBlockSize tokens.
Readings: index i selects the tokens i*bs .. i*bs + bs - 1 of the query row's
own sequence (sequence-local positions, as the indexer writes them); an index
of -1 (the indexer's padding), or a token at or past the sequence's key count,
gives a row of zero bytes.  Rows are opaque byte strings of the key layout
(BSND [B, S2, R], TND [T2, R], or a paged pool [num_blocks, block_size, R]
through block_table).
"""
from __future__ import annotations

import numpy as np


def gather(inst: dict, kv: np.ndarray, idx: np.ndarray, select_block: int) -> np.ndarray:
    """kv: uint8 [..., R] in the key layout of `inst`; idx: int32 [rows, topk].
    Returns uint8 [rows, topk * select_block, R]."""
    R = kv.shape[-1]
    rows, topk = idx.shape
    out = np.zeros((rows, topk * select_block, R), dtype=np.uint8)
    B = inst["batch"]
    lq, lk = inst["seqlens_q"], inst["seqlens_k"]
    row0 = 0
    for b in range(B):
        k0 = sum(lk[:b])                       # TND token offset of batch b
        for i in range(lq[b]):
            r = row0 + i
            for j in range(topk):
                sel = int(idx[r, j])
                if sel < 0:
                    continue
                for u in range(select_block):
                    s = sel * select_block + u
                    if s >= lk[b]:
                        continue
                    if inst["layout_k"] == "PA_BSND":
                        bs = inst["block_size"]
                        blk = int(inst["block_table"][b, s // bs])
                        src = kv[blk, s % bs]
                    elif inst["layout_k"] == "TND":
                        src = kv[k0 + s]
                    else:
                        src = kv[b, s]
                    out[r, j * select_block + u] = src
        row0 += lq[b]
    return out
