"""li_gather on the GPU vs the CPU gather oracle (oracle/gather.py), byte for byte.

Indices come either from a seeded draw (with -1 padding and positions past the
sequence, so every branch of the rule is hit) or from li_forward itself (the
indexer feeding the gather, as in sparse attention).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle.gather import gather as oracle_gather
from score_top_token_amd import binding, synth

pytestmark = pytest.mark.gpu


def _kv(inst, row_bytes, seed):
    """Random token rows in the key layout of `inst` (uint8, last dim = one row)."""
    g = torch.Generator().manual_seed(seed)
    if inst["layout_k"] == "PA_BSND":
        pool = inst["k"]                                  # [nb, bs, 1, D] view of a padded pool
        nb, bs = pool.shape[0], pool.shape[1]
        full = torch.randint(0, 256, (nb, bs + 3, row_bytes), generator=g, dtype=torch.int32)
        return full.to(torch.uint8)[:, :bs]               # blocks (bs + 3) rows apart
    if inst["layout_k"] == "TND":
        return torch.randint(0, 256, (inst["total_k"], row_bytes), generator=g,
                             dtype=torch.int32).to(torch.uint8)
    return torch.randint(0, 256, (inst["batch"], inst["max_seqlen_k"], row_bytes), generator=g,
                         dtype=torch.int32).to(torch.uint8)


def _to_dev(kv):
    if kv.is_contiguous():
        return kv.cuda()
    base = kv.as_strided((kv.shape[0], kv.stride(0)), (kv.stride(0), 1))
    return base.cuda().as_strided(kv.shape, kv.stride())


def _run(inst, kv, idx, sel):
    dev = torch.device("cuda")
    p = binding.problem_for(inst)
    args = {n: (inst[n].to(dev) if isinstance(inst.get(n), torch.Tensor) else None)
            for n in ("cu_seqlens_q", "cu_seqlens_k", "seqused_k")}
    meta = binding.lightning_indexer_metadata(p, device=dev, **args)
    bt = inst["block_table"].to(dev) if inst.get("block_table") is not None else None
    out = binding.gather_selected(p, _to_dev(kv), idx.to(dev).contiguous(), metadata=meta,
                                  select_block=sel, block_table=bt)
    torch.cuda.synchronize()
    return out.cpu().numpy()


CASES = {
    "bsnd": (dict(batch=2, s1=70, s2=300, n1=8, topk=24), 16, 1),
    "bsnd_sel4": (dict(batch=2, s1=33, s2=130, n1=8, topk=9), 48, 4),
    "tnd": (dict(batch=4, n1=8, topk=40, layout_q="TND", layout_k="TND", len_lo=20,
                 len_hi=300), 256, 1),
    "tnd_sel2": (dict(batch=3, n1=8, topk=17, layout_q="TND", layout_k="TND", len_lo=5,
                      len_hi=90, kv_extra=11), 32, 2),
    "paged": (dict(batch=5, s1=1, n1=8, topk=100, layout_k="PA_BSND", len_lo=50, len_hi=2000,
                   block_size=64), 1024, 1),
    "paged_rows3_sel3": (dict(batch=3, s1=3, n1=8, topk=30, layout_k="PA_BSND", len_lo=1,
                              len_hi=500, block_size=32), 80, 3),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_gather_random_indices(name):
    spec, row_bytes, sel = CASES[name]
    inst = synth.make(synth.Spec(name=name, **spec), 40)
    rows = sum(inst["seqlens_q"])
    g = np.random.default_rng(3)
    hi = max(inst["seqlens_k"]) // sel + 3                 # some positions past the sequence
    idx = g.integers(-1, hi, size=(rows, inst["topk"])).astype(np.int32)
    kv = _kv(inst, row_bytes, 41)
    want = oracle_gather(inst, kv.numpy(), idx, sel)
    got = _run(inst, kv, torch.from_numpy(idx), sel)
    assert got.shape == want.shape
    assert np.array_equal(got, want)


def test_gather_after_the_indexer():
    """The indexer's own output (decode rows, paged keys, -1 padding on short rows)
    drives the gather of 1 KiB rows."""
    spec = synth.Spec(name="idx_gather", batch=6, s1=1, n1=64, topk=1024, layout_k="PA_BSND",
                      len_lo=100, len_hi=3000, block_size=128, w_scale=0.125)
    inst = synth.make(spec, 42)
    idx, _ = binding.run_instance(inst, return_value=0)
    idx = idx.reshape(-1, inst["topk"]).cpu()
    assert (idx == -1).any() and (idx >= 0).any()
    kv = _kv(inst, 1024, 43)
    want = oracle_gather(inst, kv.numpy(), idx.numpy(), 1)
    got = _run(inst, kv, idx, 1)
    assert np.array_equal(got, want)


def test_gather_indices_far_out_of_range():
    """Block indices whose position index * select_block passes 2^31 (or wraps
    to a small value in 32 bits) select nothing: their rows come out as zeros."""
    spec, row_bytes, sel = CASES["bsnd_sel4"]
    inst = synth.make(synth.Spec(name="far", **spec), 42)
    rows = sum(inst["seqlens_q"])
    g = np.random.default_rng(5)
    idx = g.integers(-1, 20, size=(rows, inst["topk"])).astype(np.int32)
    idx[:, 0] = 1 << 30                          # 2^30 * 4 = 2^32: wraps to 0 in int32
    idx[:, 1] = (1 << 30) + 3                    # wraps to 12 (+ the row in the block)
    idx[:, 2] = np.iinfo(np.int32).max
    kv = _kv(inst, row_bytes, 43)
    want = oracle_gather(inst, kv.numpy(), idx, sel)
    got = _run(inst, kv, torch.from_numpy(idx), sel)
    assert np.array_equal(got, want)
    per = sel
    assert not got.reshape(rows, inst["topk"] * per, row_bytes)[:, :3 * per].any()
