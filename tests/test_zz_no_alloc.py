"""li_forward_noalloc (the entry point for callers that cannot allocate) against
li_forward through the C ABI: the same kernels on the same inputs, so the
outputs must be bitwise equal; two calls in a row, the second on a smaller
problem, so the scratch array's leftovers from the first call must not leak
into the second."""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import pytest
import torch

from score_top_token_amd import binding, synth

pytestmark = pytest.mark.gpu


def _dev(inst, dev):
    g = {n: (inst[n].to(dev) if isinstance(inst.get(n), torch.Tensor) else None)
         for n in ("q", "k", "w", "q_descale", "k_descale", "cu_seqlens_q", "cu_seqlens_k",
                   "seqused_k", "block_table", "cmp_residual_k", "output_idx_offset")}
    if inst["layout_k"] == "PA_BSND":
        kc = inst["k"]
        base = kc.as_strided((kc.shape[0], kc.stride(0)), (kc.stride(0), 1)).to(dev)
        g["k"] = base.as_strided(kc.shape, kc.stride())
    return g


def _both(inst, values=True):
    print(f"[gpu] noalloc {inst['name']} B={inst['batch']} S1={inst['max_seqlen_q']} "
          f"S2={inst['max_seqlen_k']} {inst['layout_k']}", flush=True)
    sys.stdout.flush()
    dev = torch.device("cuda")
    g = _dev(inst, dev)
    p = binding.problem_for(inst, g["k"])
    meta = binding.lightning_indexer_metadata(p, cu_seqlens_q=g["cu_seqlens_q"],
                                              cu_seqlens_k=g["cu_seqlens_k"],
                                              seqused_k=g["seqused_k"],
                                              cmp_residual_k=g["cmp_residual_k"], device=dev)
    ref_i, ref_v = binding.lightning_indexer(
        p, g["q"], g["k"], g["w"], metadata=meta, q_descale=g["q_descale"],
        k_descale=g["k_descale"], cu_seqlens_q=g["cu_seqlens_q"], cu_seqlens_k=g["cu_seqlens_k"],
        seqused_k=g["seqused_k"], cmp_residual_k=g["cmp_residual_k"],
        block_table=g["block_table"], output_idx_offset=g["output_idx_offset"])
    idx = torch.full_like(ref_i, 7)
    val = torch.full_like(ref_v, 7.0) if values else None
    ptr = lambda t: None if t is None else t.data_ptr()
    st = binding.li_forward_noalloc(p, ptr(g["q"]), ptr(g["k"]), ptr(g["w"]), ptr(g["q_descale"]),
                                    ptr(g["k_descale"]), ptr(g["cu_seqlens_q"]),
                                    ptr(g["cu_seqlens_k"]), ptr(g["seqused_k"]),
                                    ptr(g["cmp_residual_k"]), ptr(g["block_table"]),
                                    ptr(g["output_idx_offset"]), meta.data_ptr(), idx.data_ptr(),
                                    ptr(val), torch.cuda.current_stream().cuda_stream)
    assert st == 0, binding.li_status_str(st)
    torch.cuda.synchronize()
    assert torch.equal(idx, ref_i)
    if values:
        assert torch.equal(val.view(torch.int32), ref_v.view(torch.int32))
    return p


def test_noalloc_equals_forward_twice():
    # decode (the scratch holds every row's scores), then a smaller decode
    big = synth.make(dataclasses.replace(synth.PRESETS["decode"], name="noalloc_decode",
                                         batch=16), 0)
    p = _both(big)
    st, wsb = binding.li_workspace_size(p)
    assert st == 0 and wsb > (1 << 20)
    small = synth.make(dataclasses.replace(synth.PRESETS["decode"], name="noalloc_decode_small",
                                           batch=3, len_lo=700, len_hi=2500, topk=512), 1)
    _both(small)


def test_noalloc_rows_in_workspace_then_lds():
    # prefill rows in the workspace (6000 keys), then rows kept in LDS
    _both(synth.make(synth.Spec(name="noalloc_global", batch=1, s1=64, s2=6000, n1=64,
                                topk=512, w_scale=0.125), 2))
    _both(synth.make(synth.Spec(name="noalloc_lds", batch=2, s1=300, s2=300, n1=16, topk=64), 3))


def test_noalloc_candidate_lists():
    # rows past 32768 keys (candidate lists) without values: the running top-k's
    # values then live in the scratch array; then a smaller list problem with values
    _both(synth.make(synth.Spec(name="noalloc_lists", batch=1, s1=8, s2=40000, n1=16,
                                topk=512, w_scale=0.25), 4), values=False)
    _both(synth.make(synth.Spec(name="noalloc_lists_small", batch=1, s1=5, s2=34000, n1=8,
                                topk=256), 5))
