"""Small helpers for hand-built problem instances in tests."""
from __future__ import annotations

import numpy as np
import torch


def bsnd_inst(q, k, w, topk, mask_mode=3, qk_dtype="bf16", w_dtype="bf16", q_descale=None,
              k_descale=None):
    """Instance dict (same keys as synth.make) for BSND q [B,S1,N1,D], k [B,S2,1,D]."""
    B, S1, N1, D = q.shape
    S2 = k.shape[1]
    return dict(batch=B, n1=N1, d=D, topk=topk, layout_q="BSND", layout_k="BSND",
                mask_mode=mask_mode, qk_dtype=qk_dtype, w_dtype=w_dtype, block_size=0,
                num_blocks=0, max_blocks_per_seq=0, total_q=0, total_k=0, cu_seqlens_q=None,
                cu_seqlens_k=None, seqused_k=None, block_table=None, q_descale=q_descale,
                k_descale=k_descale, max_seqlen_q=S1, max_seqlen_k=S2, seqlens_q=[S1] * B,
                seqlens_k=[S2] * B, q=q.contiguous(), k=k.contiguous(), w=w.contiguous(),
                name="custom", seed=-1)


def int_tensor(g, shape, lo, hi, dtype=torch.bfloat16):
    """Small integers (exact in bf16 / fp16 / e4m3 for |v| <= 16)."""
    return torch.randint(lo, hi + 1, shape, generator=g).to(torch.float32).to(dtype)


def valid_prefix_len(idx_row: np.ndarray) -> int:
    n = int((idx_row >= 0).sum())
    assert (idx_row[:n] >= 0).all() and (idx_row[n:] == -1).all(), "valid entries not a prefix"
    return n
