"""Seeded synthetic inputs for the Lightning Indexer forward pass.

This module is shared by the HIP path's tests/bench and by the CPU oracle's
tests.  It only draws random numbers and lays them out; it holds none of the
indexer's arithmetic (no scores, no masking, no selection).  Every tensor it
returns lives on the CPU; callers copy what they need to the device.

Shapes and names follow the lightning_indexer API page (CANN ops-transformer,
"Parameters" note): q [B,S1,N1,D] (BSND) or [T1,N1,D] (TND), k [B,S2,1,D],
[T2,1,D] or a paged pool [num_blocks, block_size, 1, D] (PA_BSND), w [B,S1,N1]
or [T1,N1].  cu_seqlens are B inclusive prefix sums (the Constraints section of
the same page: "cumulative number of valid tokens of the current batch and
preceding batches").

Draw order for a seed (torch.Generator on the CPU, fp32, then a round-to-
nearest-even cast): sequence lengths (TND / PA only), q, k, w, the block
permutation (PA only), then the per-batch compression residuals (cmp_ratio > 1
with mask 3) and output index offsets (idx_offset_max > 0).  Compressed keys
are drawn like any other keys: the generator does not compress anything, k
simply holds S2_b keys that each stand for cmp_ratio original positions.  fp8 data is quantized per token from fp32 N(0,1) draws:
descale = amax/448 over the token's values, code = e4m3fn(x/descale) after a
clamp to +-448.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

LAYOUTS = ("BSND", "TND", "PA_BSND")
QK_DTYPES = ("bf16", "fp8", "fp16")
W_DTYPES = ("bf16", "fp32")

E4M3_MAX = 448.0


@dataclasses.dataclass
class Spec:
    """One synthetic workload.  Lengths are drawn when lo/hi ranges are set."""

    name: str = "custom"
    batch: int = 1
    s1: int = 256                  # BSND query length (or per-seq when TND and fixed)
    s2: int = 256                  # BSND key length
    n1: int = 8
    d: int = 128
    topk: int = 32
    layout_q: str = "BSND"
    layout_k: str = "BSND"
    mask_mode: int = 3
    qk_dtype: str = "bf16"
    w_dtype: str = "bf16"
    w_scale: float = 1.0 / math.sqrt(8.0)   # w ~ N(0,1) * w_scale
    # TND: per-sequence lengths drawn uniformly in [len_lo, len_hi] (inclusive)
    # and shared by q and k unless kv_extra > 0 (keys = queries + kv_extra).
    len_lo: int = 0
    len_hi: int = 0
    kv_extra: int = 0
    kv_div: int = 1                # TND keys = queries // kv_div + kv_extra (compressed keys)
    # PA_BSND: one query row per sequence by default (decode); key lengths drawn
    # uniformly in [len_lo, len_hi]; pool holds batch*max_blocks_per_seq blocks.
    block_size: int = 128
    block_pad: int = 0             # extra rows per block in the pool (axis-0 stride)
    # chunked prefill / decode: key count S2 > S1 (right-down causal aligns the
    # last query with the last key).
    fixed_lengths: Optional[list] = None    # overrides the drawn lengths
    # compressed keys: each key stands for cmp_ratio original positions; with
    # mask 3 every batch draws a residual in [0, cmp_ratio) (trailing original
    # keys not yet compressed), unless fixed_residuals gives them
    cmp_ratio: int = 1
    fixed_residuals: Optional[list] = None
    # output index offsets: per batch, drawn in [1, idx_offset_max] when > 0
    idx_offset_max: int = 0


PRESETS = {
    # Tiny oracle case (runs in the oracle in milliseconds).
    "tiny": Spec(name="tiny", batch=1, s1=256, s2=256, n1=8, topk=32,
                 w_scale=1.0 / math.sqrt(8.0)),
    # Prefill: S1 = S2 = 4096, 64 heads, top-2048, right-down causal.
    "prefill": Spec(name="prefill", batch=1, s1=4096, s2=4096, n1=64, topk=2048,
                    w_scale=1.0 / 8.0),
    # Batched paged decode: 64 sequences, one query each, keys U[8192, 32768],
    # block_size 128, a seeded random permutation block table.
    "decode": Spec(name="decode", batch=64, s1=1, n1=64, topk=2048, layout_k="PA_BSND",
                   len_lo=8192, len_hi=32768, block_size=128, w_scale=1.0 / 8.0),
    # Varlen TND prefill: 8 sequences, lengths U[1024, 16384], cu_seqlens_q == cu_seqlens_k.
    "varlen": Spec(name="varlen", batch=8, n1=64, topk=2048, layout_q="TND", layout_k="TND",
                   len_lo=1024, len_hi=16384, w_scale=1.0 / 8.0),
    # Long-context chunked prefill in fp8: 8192 queries at the end of 131072 keys.
    "longfp8": Spec(name="longfp8", batch=1, s1=8192, s2=131072, n1=64, topk=2048,
                    qk_dtype="fp8", w_scale=1.0 / 8.0),
}


def _randn(g: torch.Generator, shape) -> torch.Tensor:
    return torch.randn(*shape, generator=g, dtype=torch.float32)


def quantize_e4m3_per_token(x: torch.Tensor, token_dims: int):
    """Per-token amax quantization of fp32 data to e4m3fn codes + fp32 descales.

    x has shape [tokens..., rest...]; the first `token_dims` dims index tokens.
    Returns (codes as torch.float8_e4m3fn, descale fp32 of the token shape).
    """
    tok_shape = x.shape[:token_dims]
    flat = x.reshape(*tok_shape, -1)
    amax = flat.abs().amax(dim=-1)
    descale = (amax / E4M3_MAX).to(torch.float32)
    descale = torch.where(descale > 0, descale, torch.ones_like(descale))
    scaled = flat / descale.unsqueeze(-1)
    scaled = scaled.clamp(-E4M3_MAX, E4M3_MAX)
    codes = scaled.to(torch.float8_e4m3fn).reshape(x.shape)
    return codes, descale.contiguous()


def _cast(x: torch.Tensor, dt: str) -> torch.Tensor:
    if dt == "bf16":
        return x.to(torch.bfloat16)
    if dt == "fp16":
        return x.to(torch.float16)
    if dt == "fp32":
        return x.to(torch.float32)
    raise ValueError(dt)


def make(spec: Spec | str, seed: int = 0) -> dict:
    """Build one seeded problem instance.  Returns a dict of CPU tensors + scalars.

    Keys: q, k, w, q_descale, k_descale (None unless fp8), cu_seqlens_q,
    cu_seqlens_k, seqused_k, block_table (None where the layout has none),
    plus the scalar fields of the problem (batch, max_seqlen_q, max_seqlen_k,
    total_q, total_k, n1, d, topk, layout_q, layout_k, mask_mode, qk_dtype,
    w_dtype, block_size, num_blocks, max_blocks_per_seq, seqlens_q, seqlens_k).
    """
    if isinstance(spec, str):
        spec = PRESETS[spec]
    g = torch.Generator().manual_seed(int(seed))
    B, N1, D = spec.batch, spec.n1, spec.d
    out = dict(batch=B, n1=N1, d=D, topk=spec.topk, layout_q=spec.layout_q,
               layout_k=spec.layout_k, mask_mode=spec.mask_mode, qk_dtype=spec.qk_dtype,
               w_dtype=spec.w_dtype, block_size=0, num_blocks=0, max_blocks_per_seq=0,
               total_q=0, total_k=0, cu_seqlens_q=None, cu_seqlens_k=None,
               seqused_k=None, block_table=None, q_descale=None, k_descale=None,
               cmp_ratio=spec.cmp_ratio, cmp_residual_k=None, output_idx_offset=None,
               name=spec.name, seed=int(seed))

    # ---- lengths ---------------------------------------------------------
    if spec.layout_q == "TND":
        if spec.fixed_lengths is not None:
            lq = [int(v) for v in spec.fixed_lengths]
        else:
            lq = torch.randint(spec.len_lo, spec.len_hi + 1, (B,), generator=g).tolist()
        lk = [v // spec.kv_div + spec.kv_extra for v in lq]
        out["seqlens_q"], out["seqlens_k"] = lq, lk
        out["total_q"], out["total_k"] = sum(lq), sum(lk)
        out["max_seqlen_q"], out["max_seqlen_k"] = max(lq) if lq else 0, max(lk) if lk else 0
        out["cu_seqlens_q"] = torch.tensor(_inclusive_cumsum(lq), dtype=torch.int32)
        out["cu_seqlens_k"] = torch.tensor(_inclusive_cumsum(lk), dtype=torch.int32)
    elif spec.layout_k == "PA_BSND":
        if spec.fixed_lengths is not None:
            lk = [int(v) for v in spec.fixed_lengths]
        else:
            lk = torch.randint(spec.len_lo, spec.len_hi + 1, (B,), generator=g).tolist()
        out["seqlens_q"], out["seqlens_k"] = [spec.s1] * B, lk
        out["max_seqlen_q"] = spec.s1
        out["max_seqlen_k"] = max(lk) if lk else 0
        out["seqused_k"] = torch.tensor(lk, dtype=torch.int32)
    else:
        out["seqlens_q"], out["seqlens_k"] = [spec.s1] * B, [spec.s2] * B
        out["max_seqlen_q"], out["max_seqlen_k"] = spec.s1, spec.s2

    # ---- q ---------------------------------------------------------------
    if spec.layout_q == "TND":
        qshape = (out["total_q"], N1, D)
        tok_dims = 1
    else:
        qshape = (B, spec.s1, N1, D)
        tok_dims = 2
    qf = _randn(g, qshape)

    # ---- k ---------------------------------------------------------------
    if spec.layout_k == "TND":
        kshape = (out["total_k"], 1, D)
        ktok = 1
    elif spec.layout_k == "PA_BSND":
        bs = spec.block_size
        mb = max(1, -(-out["max_seqlen_k"] // bs))
        nblk = B * mb
        out["block_size"], out["num_blocks"], out["max_blocks_per_seq"] = bs, nblk, mb
        kshape = (nblk, bs + spec.block_pad, 1, D)
        ktok = 2
    else:
        kshape = (B, spec.s2, 1, D)
        ktok = 2
    kf = _randn(g, kshape)

    # ---- w ---------------------------------------------------------------
    wshape = qshape[:-1]
    wf = _randn(g, wshape) * spec.w_scale
    out["w"] = _cast(wf, spec.w_dtype).contiguous()

    if spec.qk_dtype == "fp8":
        qc, qd = quantize_e4m3_per_token(qf, tok_dims)
        kc, kd = quantize_e4m3_per_token(kf, ktok)
        out["q"], out["q_descale"] = qc.contiguous(), qd
        out["k"], out["k_descale"] = kc, kd
    else:
        out["q"] = _cast(qf, spec.qk_dtype).contiguous()
        out["k"] = _cast(kf, spec.qk_dtype)

    if spec.layout_k == "PA_BSND":
        # the pool may carry padding rows per block: hand out the [:, :bs] view
        # (axis 0 then has a stride of (bs + pad) * D elements).
        bs = spec.block_size
        out["k"] = out["k"][:, :bs]
        if out["k_descale"] is not None:
            # descale of physical slot (block pb, row r) sits at [pb, r]
            out["k_descale"] = out["k_descale"][:, :bs].contiguous()
        perm = torch.randperm(out["num_blocks"], generator=g).to(torch.int32)
        bt = perm.reshape(B, out["max_blocks_per_seq"]).clone()
        for b in range(B):
            used = -(-lk[b] // bs)
            bt[b, used:] = -1
        out["block_table"] = bt.contiguous()

    if spec.cmp_ratio > 1 and spec.mask_mode == 3:
        if spec.fixed_residuals is not None:
            res = torch.tensor([int(v) for v in spec.fixed_residuals], dtype=torch.int32)
        else:
            res = torch.randint(0, spec.cmp_ratio, (B,), generator=g).to(torch.int32)
        out["cmp_residual_k"] = res.contiguous()
    if spec.idx_offset_max > 0:
        out["output_idx_offset"] = torch.randint(1, spec.idx_offset_max + 1, (B,),
                                                 generator=g).to(torch.int32).contiguous()
    return out


def _inclusive_cumsum(v):
    acc, res = 0, []
    for x in v:
        acc += int(x)
        res.append(acc)
    return res


def scaled_spec(name: str, **overrides) -> Spec:
    """A preset with some fields replaced (smaller parity-test variants)."""
    return dataclasses.replace(PRESETS[name], **overrides)


# ---------------------------------------------------------------------------
# Inputs of the indexer backward fused with the KL loss
# (npu_sparse_lightning_indexer_grad_kl_loss page, parameter list): the main
# attention's q / k (+ rope parts) and its saved softmax statistics, the
# indexer's q / k / weights, and the top-k selection sparse_indices.
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class GradSpec:
    name: str = "grad"
    batch: int = 1
    s1: int = 256                  # BSND query length (= key length)
    layout: str = "BSND"           # BSND or TND (query and key sides alike)
    len_lo: int = 0                # TND: sequence lengths drawn in [len_lo, len_hi]
    len_hi: int = 0
    fixed_lengths: Optional[list] = None
    n_main: int = 16               # main-attention query heads (one key head)
    d_main: int = 128
    d_rope: int = 64               # 0: no rope inputs
    n_idx: int = 64                # index query heads
    d_idx: int = 128
    topk: int = 64
    dtype: str = "bf16"            # q, k, q_rope, k_rope, qi, ki
    w_dtype: str = "bf16"
    w_scale: float = 1.0 / 8.0
    scale: Optional[float] = None  # scale_value; default 1/sqrt(d_main + d_rope)
    # saved softmax statistics per (row, head): max ~ N(max_mu, max_sd), sum ~ U[sum_lo, sum_hi]
    max_mu: float = 3.0
    max_sd: float = 0.5
    sum_lo: float = 50.0
    sum_hi: float = 500.0


GRAD_PRESETS = {
    "grad_tiny": GradSpec(name="grad_tiny", batch=1, s1=256, n_main=4, n_idx=8, topk=32,
                          w_scale=1.0 / math.sqrt(8.0)),
    # training-shaped: 64 index heads of 128, top-2048 over a 4096-token causal
    # sequence, 32 main heads of 128 + 64 rope
    "grad_train": GradSpec(name="grad_train", batch=1, s1=4096, n_main=32, n_idx=64,
                           topk=2048),
    # the same shape at a size the CPU oracle runs in full (every row, every key)
    "grad_mid": GradSpec(name="grad_mid", batch=2, s1=1024, n_main=16, n_idx=64, topk=256),
}


def make_grad(spec: GradSpec | str, seed: int = 0) -> dict:
    """One seeded backward instance (CPU tensors).  sparse_indices holds, per query
    row, min(topk, visible) distinct keys drawn uniformly from the row's right-down
    causal window (the shape of a top-k selection; no score is computed), in
    random order, then -1 padding."""
    if isinstance(spec, str):
        spec = GRAD_PRESETS[spec]
    g = torch.Generator().manual_seed(int(seed))
    B = spec.batch
    if spec.layout == "TND":
        if spec.fixed_lengths is not None:
            lens = [int(v) for v in spec.fixed_lengths]
        else:
            lens = torch.randint(spec.len_lo, spec.len_hi + 1, (B,), generator=g).tolist()
    else:
        lens = [spec.s1] * B
    rows = sum(lens)
    lead = (rows,) if spec.layout == "TND" else (B, spec.s1)
    cast = lambda x, dt: _cast(x, dt).contiguous()
    out = dict(name=spec.name, seed=int(seed), batch=B, layout=spec.layout, seqlens=lens,
               max_seqlen_q=max(lens) if lens else 0, max_seqlen_k=max(lens) if lens else 0,
               n_main=spec.n_main, d_main=spec.d_main, d_rope=spec.d_rope, n_idx=spec.n_idx,
               d_idx=spec.d_idx, topk=spec.topk,
               scale=spec.scale if spec.scale else 1.0 / math.sqrt(spec.d_main + spec.d_rope),
               cu_seqlens_q=None, cu_seqlens_k=None)
    if spec.layout == "TND":
        cu = torch.tensor(_inclusive_cumsum(lens), dtype=torch.int32)
        out["cu_seqlens_q"], out["cu_seqlens_k"] = cu, cu.clone()
    out["q"] = cast(_randn(g, lead + (spec.n_main, spec.d_main)), spec.dtype)
    out["k"] = cast(_randn(g, lead + (1, spec.d_main)), spec.dtype)
    if spec.d_rope > 0:
        out["q_rope"] = cast(_randn(g, lead + (spec.n_main, spec.d_rope)), spec.dtype)
        out["k_rope"] = cast(_randn(g, lead + (1, spec.d_rope)), spec.dtype)
    else:
        out["q_rope"] = out["k_rope"] = None
    out["qi"] = cast(_randn(g, lead + (spec.n_idx, spec.d_idx)), spec.dtype)
    out["ki"] = cast(_randn(g, lead + (1, spec.d_idx)), spec.dtype)
    out["w"] = cast(_randn(g, lead + (spec.n_idx,)) * spec.w_scale, spec.w_dtype)
    # the selection: a seeded random subset of each row's causal window
    sel = torch.full((rows, spec.topk), -1, dtype=torch.int32)
    r0 = 0
    for L in lens:
        for i0 in range(0, L, 1024):                 # row chunks bound the draw's memory
            i1 = min(L, i0 + 1024)
            u = torch.rand((i1 - i0, L), generator=g)
            lim = torch.arange(i0, i1).unsqueeze(1) + 1          # keys 0 .. i visible
            u = torch.where(torch.arange(L).unsqueeze(0) < lim, u, torch.full_like(u, 2.0))
            order = torch.argsort(u, dim=1)[:, :spec.topk].to(torch.int32)
            keep = torch.arange(order.shape[1]).unsqueeze(0) < lim
            sel[r0 + i0:r0 + i1, :order.shape[1]] = torch.where(keep, order,
                                                                 torch.full_like(order, -1))
        r0 += L
    out["sparse_indices"] = sel.contiguous()
    G = spec.n_main
    out["softmax_max"] = (spec.max_mu + spec.max_sd * _randn(g, (rows, G))).contiguous()
    out["softmax_sum"] = (spec.sum_lo + (spec.sum_hi - spec.sum_lo) *
                          torch.rand((rows, G), generator=g)).contiguous()
    return out
