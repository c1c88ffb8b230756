"""HIP path vs the CPU oracle on seeded inputs (needs an MI355X).

Every case runs li_metadata + li_forward through the C ABI, then compares the
outputs with the oracle row by row (tests/compare.py: exact structure and
padding, values within 1e-2 * max(1, |I|), index sets equal up to swaps at the
k-th score).  Small cases are compared on every row.  The five full-size
workloads run at seeds 0, 1 and 2: prefill, decode and the tiny case on every
row; varlen and longfp8 on stratified rows (first / last rows of every sequence,
rows around |V| = k, rows of the items every grid slot of the persistent
kernels (rows in workspace rows or in candidate lists) runs in its first and
later rounds, evenly spaced and seeded random rows), and structurally on every
row.
"""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

import oracle
from score_top_token_amd import binding, synth
from tests import compare
from tests.util import bsnd_inst, int_tensor

pytestmark = pytest.mark.gpu

try:
    ORACLE_THREADS = min(16, len(os.sched_getaffinity(0)))   # the host's CPU share
except AttributeError:
    ORACLE_THREADS = min(16, os.cpu_count() or 1)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _gpu(inst, return_value=1):
    _say(f"[gpu] {inst.get('name')} seed={inst.get('seed')} B={inst['batch']} "
         f"S1={inst['max_seqlen_q']} S2={inst['max_seqlen_k']} N1={inst['n1']} "
         f"topk={inst['topk']} {inst['layout_q']}/{inst['layout_k']} {inst['qk_dtype']}")
    idx, val = binding.run_instance(inst, return_value=return_value)
    torch.cuda.synchronize()
    topk = inst["topk"]
    gi = idx.cpu().numpy().reshape(-1, topk)
    gv = None if val is None else val.cpu().numpy().reshape(-1, topk)
    return gi, gv


def structural_check(gi, gv, inst, ob):
    """Vectorised checks on every row: valid prefix of exactly min(k, |V|), padding,
    indices inside the visible window, no duplicates."""
    topk = inst["topk"]
    nrows = gi.shape[0]
    vis = np.empty(nrows, dtype=np.int64)
    r = 0
    for b in range(inst["batch"]):
        s1, s2 = inst["seqlens_q"][b], inst["seqlens_k"][b]
        i = np.arange(s1)
        if (inst.get("cmp_ratio") or 1) > 1:         # compressed keys: the oracle's rule
            v = np.array([ob.visible_count(b, x) for x in range(s1)], dtype=np.int64)
        else:
            v = np.full(s1, s2) if inst["mask_mode"] == 0 else np.clip(i + s2 - s1 + 1, 0, s2)
        vis[r:r + s1] = v
        r += s1
    assert r == nrows
    n = np.minimum(vis, topk)
    valid = gi >= 0
    assert (valid.sum(1) == n).all(), "number of valid entries"
    col = np.arange(topk)[None, :]
    assert (valid == (col < n[:, None])).all(), "valid entries not a prefix"
    assert ((gi < vis[:, None]) | ~valid).all(), "index outside the visible window"
    s = np.sort(np.where(valid, gi, -1 - col), axis=1)
    assert (np.diff(s, axis=1) != 0).all(), "duplicate index"
    if gv is not None:
        assert np.isneginf(gv[~valid]).all(), "value padding"
        assert np.isfinite(gv[valid]).all(), "non-finite value"


def _without_offsets(idx, inst):
    """Valid indices minus their batch's output index offset (checked to be
    there); padding untouched."""
    off = inst.get("output_idx_offset")
    if off is None:
        return idx
    per_row = np.repeat(off.numpy().astype(np.int64), inst["seqlens_q"])
    valid = idx >= 0
    assert (idx[valid] >= np.broadcast_to(per_row[:, None], idx.shape)[valid]).all(), \
        "index below its batch offset"
    return np.where(valid, idx - per_row[:, None], idx).astype(np.int32)


def compare_all(inst, rows=None, return_value=1, seed_rows=0):
    gi, gv = _gpu(inst, return_value)
    ob = oracle.Bound(inst)
    gi = _without_offsets(gi, inst)
    structural_check(gi, gv, inst, ob)
    if rows is None:
        rows = np.arange(gi.shape[0])
    rows = np.asarray(rows, dtype=np.int64)
    _say(f"    oracle on {len(rows)} rows ({ORACLE_THREADS} threads)")
    oi, ov = ob.forward(rows=rows, nthreads=ORACLE_THREADS)
    _say("    comparing")
    if inst.get("output_idx_offset") is not None:
        per_row = np.repeat(inst["output_idx_offset"].numpy().astype(np.int64),
                            inst["seqlens_q"])[rows]
        oi = np.where(oi >= 0, oi - per_row[:, None], oi).astype(np.int32)
    rep = compare.check_rows(gi[rows], None if gv is None else gv[rows], oi, ov, rows, ob)
    _say(f"    rows={rep.rows} max_abs={rep.max_abs:.3g} max_rel={rep.max_rel:.3g} "
         f"swaps={rep.swaps}")
    return gi, gv, rep


# --------------------------------------------------------------------------
# small cases, every row compared
# --------------------------------------------------------------------------

SMALL = {
    "tiny_s0": ("tiny", 0, {}), "tiny_s1": ("tiny", 1, {}), "tiny_s2": ("tiny", 2, {}),
    "prefill_700_k64": (None, 3, dict(batch=2, s1=700, s2=700, n1=64, topk=64, w_scale=0.125)),
    "prefill_700_k256": (None, 4, dict(batch=1, s1=700, s2=700, n1=64, topk=256, w_scale=0.125)),
    "prefill_k1_mask0": (None, 5, dict(batch=1, s1=130, s2=333, n1=16, topk=1, mask_mode=0)),
    "heads1_k7": (None, 6, dict(batch=2, s1=77, s2=77, n1=1, topk=7)),
    "heads33_chunked": (None, 7, dict(batch=1, s1=90, s2=1500, n1=33, topk=100)),
    "s1_gt_s2": (None, 8, dict(batch=2, s1=200, s2=70, n1=8, topk=32)),
    "k2048_long": (None, 9, dict(batch=1, s1=24, s2=9000, n1=64, topk=2048, w_scale=0.125)),
    "w_fp32": (None, 10, dict(batch=1, s1=150, s2=150, n1=20, topk=40, w_dtype="fp32")),
    "fp16_qk": (None, 11, dict(batch=2, s1=64, s2=32, n1=16, topk=32, qk_dtype="fp16",
                               w_dtype="fp32")),
    "fp8_chunked": (None, 12, dict(batch=1, s1=300, s2=2000, n1=64, topk=256, qk_dtype="fp8",
                                   w_scale=0.125)),
    "fp8_heads8": (None, 13, dict(batch=2, s1=100, s2=100, n1=8, topk=16, qk_dtype="fp8")),
    "tnd_small": (None, 14, dict(batch=4, n1=64, topk=128, layout_q="TND", layout_k="TND",
                                 len_lo=50, len_hi=900, w_scale=0.125)),
    "tnd_kv_extra": (None, 15, dict(batch=3, n1=12, topk=40, layout_q="TND", layout_k="TND",
                                    len_lo=5, len_hi=120, kv_extra=37)),
    "decode_small": (None, 16, dict(batch=5, s1=1, n1=64, topk=128, layout_k="PA_BSND",
                                    len_lo=300, len_hi=3000, block_size=64, block_pad=5,
                                    w_scale=0.125)),
    "decode_rows3": (None, 17, dict(batch=3, s1=3, n1=24, topk=50, layout_k="PA_BSND",
                                    len_lo=2, len_hi=700, block_size=32)),
    "decode_fp8": (None, 18, dict(batch=4, s1=2, n1=64, topk=200, layout_k="PA_BSND",
                                  len_lo=100, len_hi=2500, block_size=128, qk_dtype="fp8",
                                  w_scale=0.125)),
    "decode_bsnd_mask0": (None, 19, dict(batch=6, s1=1, s2=5000, n1=64, topk=1000, mask_mode=0,
                                         w_scale=0.125)),
    "prefill_paged": (None, 20, dict(batch=2, s1=40, n1=32, topk=64, layout_k="PA_BSND",
                                     len_lo=300, len_hi=600, block_size=16, block_pad=2)),
    # decode rows of 32768 and 32769 visible keys: the select keeps the first in
    # registers and streams the second from the workspace
    "decode_rows_32k_edge": (None, 21, dict(batch=1, s1=2, s2=32769, n1=8, topk=300,
                                            w_scale=0.35)),
    "decode_long_rows": (None, 22, dict(batch=2, s1=1, s2=40000, n1=16, topk=512,
                                        w_scale=0.25)),
    # topk above 2048 (3072 .. 8192 in steps of 1024): rows past the LDS rows
    # (workspace rows, bf16 and fp8) and decode
    "k8192_dense": (None, 23, dict(batch=1, s1=40, s2=9000, n1=64, topk=8192, w_scale=0.125)),
    "k3072_stream": (None, 24, dict(batch=1, s1=30, s2=12000, n1=64, topk=3072, w_scale=0.125)),
    "k8192_stream": (None, 25, dict(batch=1, s1=20, s2=20000, n1=64, topk=8192, w_scale=0.125)),
    "k5120_fp8_stream": (None, 26, dict(batch=1, s1=24, s2=16000, n1=64, topk=5120,
                                        qk_dtype="fp8", w_scale=0.125)),
    "k8192_decode": (None, 27, dict(batch=4, s1=1, n1=64, topk=8192, layout_k="PA_BSND",
                                    len_lo=5000, len_hi=20000, block_size=128, w_scale=0.125)),
    # compressed keys (cmp_ratio): the pages' example (130 original keys -> 32 with
    # residual 2), a longer dense case, workspace rows, TND with per-sequence
    # residuals, decode rows with compression; output index offsets on every path
    "cmp_pages_example": (None, 28, dict(batch=2, s1=64, s2=32, n1=16, topk=32,
                                         qk_dtype="fp16", w_dtype="fp32", cmp_ratio=4,
                                         fixed_residuals=[2, 2])),
    "cmp_dense": (None, 29, dict(batch=1, s1=4003, s2=1000, n1=64, topk=256, cmp_ratio=4,
                                 w_scale=0.125)),
    "cmp_stream": (None, 30, dict(batch=1, s1=200, s2=12000, n1=64, topk=512, cmp_ratio=3,
                                  w_scale=0.125)),
    "cmp_tnd": (None, 31, dict(batch=3, n1=24, topk=64, layout_q="TND", layout_k="TND",
                               len_lo=200, len_hi=1500, kv_div=4, cmp_ratio=4)),
    "cmp_decode": (None, 32, dict(batch=5, s1=3, n1=64, topk=128, layout_k="PA_BSND",
                                  len_lo=300, len_hi=3000, block_size=64, cmp_ratio=2,
                                  w_scale=0.125)),
    "idx_offset_dense": (None, 33, dict(batch=3, s1=300, s2=300, n1=16, topk=64,
                                        idx_offset_max=1 << 20)),
    "idx_offset_stream": (None, 34, dict(batch=1, s1=40, s2=11000, n1=64, topk=512,
                                         idx_offset_max=1 << 20, w_scale=0.125)),
    # rows past 262144 keys through candidate lists (bf16, fp8, fp16 at topk
    # 8192: many merges per row, the top-k larger than the list)
    "stream_long_bf16": (None, 36, dict(batch=1, s1=6, s2=270000, n1=8, topk=300,
                                        idx_offset_max=1000)),
    "stream_long_fp8": (None, 37, dict(batch=1, s1=5, s2=263000, n1=16, topk=512,
                                       qk_dtype="fp8", w_scale=0.25)),
    "stream_long_k8192": (None, 38, dict(batch=1, s1=5, s2=265000, n1=8, topk=8192,
                                         qk_dtype="fp16", w_dtype="fp32")),
    # 64 heads with a paged block size that is not a multiple of 32 (per-key lookups)
    "decode_paged_bs16_h64": (None, 39, dict(batch=3, s1=1, n1=64, topk=100, layout_k="PA_BSND",
                                             len_lo=100, len_hi=2000, block_size=16,
                                             w_scale=0.125)),
    "idx_offset_decode": (None, 35, dict(batch=6, s1=1, n1=64, topk=200, layout_k="PA_BSND",
                                         len_lo=100, len_hi=4000, block_size=128,
                                         idx_offset_max=1 << 20, w_scale=0.125)),
    # fp8 keys with rows in the workspace: odd and even tile counts, and TND
    # items of 1-2 tiles next to long ones
    "fp8_global_rows_odd": (None, 44, dict(batch=1, s1=70, s2=7000, n1=64, topk=300,
                                           qk_dtype="fp8", w_scale=0.125)),
    "fp8_global_rows_even_mask0": (None, 45, dict(batch=1, s1=37, s2=6016, n1=32, topk=500,
                                                  qk_dtype="fp8", mask_mode=0)),
    "fp8_global_tnd": (None, 46, dict(batch=4, n1=16, topk=64, layout_q="TND", layout_k="TND",
                                      len_lo=20, len_hi=6500, qk_dtype="fp8")),
    # score magnitudes far from 1 (weights scaled by 1e-30 or 1e25): the selects'
    # linear bucket maps over [row minimum, row maximum] at both ends of the range
    "scores_tiny_lds": (None, 40, dict(batch=1, s1=600, s2=600, n1=16, topk=100, w_scale=1e-30)),
    "scores_huge_lds": (None, 41, dict(batch=1, s1=600, s2=600, n1=16, topk=100, w_scale=1e25)),
    "scores_huge_global": (None, 42, dict(batch=1, s1=20, s2=6000, n1=16, topk=300, w_scale=1e25)),
    "scores_huge_decode": (None, 43, dict(batch=3, s1=1, n1=16, topk=100, layout_k="PA_BSND",
                                          len_lo=500, len_hi=3000, block_size=64, w_scale=1e25)),
    # rows past 32768 keys: candidate lists.  bf16 at topk 2048 (the top-k larger
    # than the list), fp8 TND items of 8-24 rows, fp16 keys in 64-key pages at
    # topk 4096, per-key pages of 16 keys, compressed keys, index offsets
    "list_bf16_k2048": (None, 47, dict(batch=1, s1=12, s2=40000, n1=64, topk=2048,
                                       w_scale=0.125)),
    "list_fp8_tnd": (None, 48, dict(batch=3, n1=16, topk=512, layout_q="TND", layout_k="TND",
                                    len_lo=8, len_hi=24, kv_extra=36000, qk_dtype="fp8")),
    "list_fp16_paged_k4096": (None, 49, dict(batch=2, s1=8, n1=32, topk=4096, layout_k="PA_BSND",
                                             len_lo=33000, len_hi=40000, block_size=64,
                                             qk_dtype="fp16", w_dtype="fp32")),
    "list_paged_bs16": (None, 50, dict(batch=1, s1=8, n1=8, topk=256, layout_k="PA_BSND",
                                       len_lo=34000, len_hi=36000, block_size=16)),
    "list_cmp": (None, 51, dict(batch=1, s1=16, s2=36000, n1=16, topk=700, cmp_ratio=2,
                                w_scale=0.25)),
    "list_idx_offset": (None, 52, dict(batch=1, s1=8, s2=34000, n1=8, topk=1000,
                                       idx_offset_max=1 << 20)),
    # the boundary between workspace rows (up to 32768 keys) and candidate lists
    "rows_32768_workspace": (None, 53, dict(batch=1, s1=6, s2=32768, n1=16, topk=2048,
                                            w_scale=0.25)),
    "rows_32769_lists": (None, 54, dict(batch=1, s1=6, s2=32769, n1=16, topk=2048,
                                        w_scale=0.25)),
    # decode with packed (TND) queries: 0..4 query rows per sequence, so the
    # select kernel's grid holds (batch, row) slots a sequence does not have,
    # and key lengths from cu_seqlens_k; bf16 and fp8
    "decode_tnd_q": (None, 55, dict(batch=7, n1=32, topk=256, layout_q="TND", layout_k="TND",
                                    len_lo=0, len_hi=4, kv_extra=3000, w_scale=0.25)),
    # 256 sequences: the largest batch whose work list one wave plans
    "decode_b256": (None, 57, dict(batch=256, s1=2, n1=8, topk=32, layout_k="PA_BSND",
                                   len_lo=0, len_hi=1500, block_size=32)),
    "decode_tnd_q_fp8": (None, 56, dict(batch=5, n1=64, topk=128, layout_q="TND",
                                        layout_k="TND", len_lo=0, len_hi=3, kv_extra=900,
                                        qk_dtype="fp8", w_scale=0.125)),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_case(name):
    preset, seed, over = SMALL[name]
    spec = synth.scaled_spec(preset, **over) if preset else synth.Spec(name=name, **over)
    spec.name = name
    compare_all(synth.make(spec, seed))


@pytest.mark.parametrize("spec", [
    dict(batch=2, s1=40, s2=6000, n1=16, topk=300),         # workspace rows
    dict(batch=1, s1=12, s2=40000, n1=16, topk=512),        # candidate lists
])
def test_metadata_reused_across_calls(spec):
    """The persistent prefill kernels take items through a counter in the metadata
    header and leave it at zero: three calls on one metadata give the same bits."""
    inst = synth.make(synth.Spec(name="meta_reuse", **spec), 7)
    dev = torch.device("cuda")
    g = {n: (inst[n].to(dev) if isinstance(inst.get(n), torch.Tensor) else None)
         for n in ("q", "k", "w")}
    p = binding.problem_for(inst, g["k"])
    meta = binding.lightning_indexer_metadata(p, device=dev)
    outs = [binding.lightning_indexer(p, g["q"], g["k"], g["w"], metadata=meta)
            for _ in range(3)]
    torch.cuda.synchronize()
    for i, v in outs[1:]:
        assert torch.equal(i, outs[0][0])
        assert torch.equal(v.view(torch.int32), outs[0][1].view(torch.int32))
    hdr = meta[:256].view(torch.int32).cpu()
    assert hdr[7].item() == 0 and hdr[8].item() == 0        # work_next, work_done
    ref = binding.run_instance(inst)
    assert torch.equal(outs[0][0], ref[0])


@pytest.mark.parametrize("spec", [
    # decode: split kernel, select kernel (lengths from the arguments), metadata
    dict(batch=4, s1=1, n1=16, topk=100, layout_k="PA_BSND", len_lo=500, len_hi=3000,
         block_size=64),
    # prefill with rows in LDS, sized from max_seqlen_k
    dict(batch=2, s1=40, n1=16, topk=64, layout_k="PA_BSND", len_lo=300, len_hi=900,
         block_size=32),
])
def test_paged_lengths_past_max_are_cut(spec):
    """A seqused_k entry above max_seqlen_k (outside the contract) is held to
    max_seqlen_k by every kernel: the same bits as the call with that length cut
    to the maximum, which itself matches the oracle; nothing reads past the
    buffers sized from the maximum (the block table has room for it: the host
    checks max_seqlen_k <= max_blocks_per_seq * block_size)."""
    inst = synth.make(synth.Spec(name="len_cut", **spec), 9)
    lens = [int(x) for x in inst["seqlens_k"]]
    cap = max(lens) - 37
    assert sum(x > cap for x in lens) >= 1
    longer = dict(inst)
    longer["max_seqlen_k"] = cap                   # seqused_k keeps the longer lengths
    cut = dict(inst)
    cut["max_seqlen_k"] = cap
    cut["seqlens_k"] = [min(x, cap) for x in lens]
    cut["seqused_k"] = torch.tensor(cut["seqlens_k"], dtype=torch.int32)
    gi_l, gv_l = _gpu(longer)
    gi_c, gv_c, _ = compare_all(cut)
    assert np.array_equal(gi_l, gi_c)
    assert np.array_equal(gv_l.view(np.int32), gv_c.view(np.int32))


@pytest.mark.parametrize("spec", [
    None,                                                   # rows in LDS (tiny)
    dict(batch=1, s1=16, s2=6000, n1=16, topk=300),         # workspace rows
    dict(batch=1, s1=8, s2=40000, n1=16, topk=700),         # candidate lists: values in the workspace
])
def test_return_value_zero_gives_same_indices(spec):
    inst = synth.make("tiny", 3) if spec is None else synth.make(synth.Spec(name="rv0", **spec), 6)
    gi1, gv1 = _gpu(inst, 1)
    gi0, gv0 = _gpu(inst, 0)
    assert gv0 is None
    assert np.array_equal(gi0, gi1)


# (S1, S2): rows in LDS, workspace rows, and candidate lists (ties across merges)
@pytest.mark.parametrize("s1,s2", [(300, 300), (40, 6000), (8, 40000)])
def test_all_zero_scores_pick_smallest_indices(s1, s2):
    topk = 50
    q = torch.zeros(1, s1, 8, 128).bfloat16()
    g = torch.Generator().manual_seed(0)
    k = torch.randn(1, s2, 1, 128, generator=g).bfloat16()
    w = torch.rand(1, s1, 8, generator=g).bfloat16()
    inst = bsnd_inst(q, k, w, topk=topk, mask_mode=3)
    inst["name"] = "zero_scores"
    gi, gv = _gpu(inst)
    for i in range(s1):
        n = min(topk, i + s2 - s1 + 1)
        assert list(gi[i, :n]) == list(range(n))
        assert (gv[i, :n] == 0).all() and not np.signbit(gv[i, :n]).any()


@pytest.mark.parametrize("s1,s2,topk", [(500, 500, 37), (48, 6000, 300)])
def test_integer_scores_exact_with_ties(s1, s2, topk):
    # small integers: every score is an exact integer in fp32, so the GPU must
    # equal the oracle exactly, ties at the k-th place included (many equal
    # scores: the bucket of the k-th element holds more than a gather's worth)
    g = torch.Generator().manual_seed(1)
    B, N1 = 2, 16
    q = int_tensor(g, (B, s1, N1, 128), -1, 1)
    k = int_tensor(g, (B, s2, 1, 128), -1, 1)
    w = int_tensor(g, (B, s1, N1), -2, 3)
    inst = bsnd_inst(q, k, w, topk=topk, mask_mode=3)
    inst["name"] = "integer_ties"
    gi, gv = _gpu(inst)
    oi, ov = oracle.Bound(inst).forward(nthreads=ORACLE_THREADS)
    for r in range(B * s1):
        n = int((oi[r] >= 0).sum())
        order = np.argsort(gi[r, :n], kind="stable")
        assert sorted(gi[r, :n].tolist()) == sorted(oi[r, :n].tolist()), f"row {r}"
        o_map = dict(zip(oi[r, :n].tolist(), ov[r, :n].tolist()))
        assert all(o_map[s] == v for s, v in zip(gi[r, :n].tolist(), gv[r, :n].tolist()))
        del order


def test_determinism_bitwise():
    for s1, s2 in ((600, 600), (64, 9000)):
        spec = synth.Spec(name="det", batch=1, s1=s1, s2=s2, n1=64, topk=128, w_scale=0.125)
        inst = synth.make(spec, 21)
        a = _gpu(inst)
        b = _gpu(inst)
        assert np.array_equal(a[0], b[0])
        assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    dec = synth.Spec(name="det_dec", batch=3, s1=1, n1=64, topk=256, layout_k="PA_BSND",
                     len_lo=1000, len_hi=4000, block_size=128, w_scale=0.125)
    inst = synth.make(dec, 22)
    a = _gpu(inst)
    b = _gpu(inst)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def test_paged_equals_contiguous():
    spec = synth.Spec(name="pa_eq", batch=3, s1=1, n1=64, topk=300, layout_k="PA_BSND",
                      len_lo=2000, len_hi=2000, block_size=128, w_scale=0.125)
    inst = synth.make(spec, 23)
    bs = inst["block_size"]
    gi, gv = _gpu(inst)
    L = inst["seqlens_k"][0]
    kb = torch.stack([torch.stack([inst["k"][inst["block_table"][b, s // bs], s % bs]
                                   for s in range(L)]) for b in range(3)])      # [3, L, 1, D]
    ref = bsnd_inst(inst["q"], kb, inst["w"], topk=300, mask_mode=3)
    ref["name"] = "pa_eq_ref"
    ri, rv = _gpu(ref)
    assert np.array_equal(gi, ri) and np.array_equal(gv, rv)


# (S1, S2): decode (S1 <= 4 query rows), the dense kernel with rows in LDS, in
# workspace rows, and in candidate lists (rows past 32768 keys, one past 262144)
@pytest.mark.parametrize("s1,s2", [(3, 300), (8, 300), (8, 12000), (8, 40000), (8, 270000)])
def test_negative_infinite_scores(s1, s2):
    """Scores of -inf (from infinite inputs) still fill the top-k: ties broken by
    the smaller key, values reported as -inf, no padding while keys remain."""
    N1, topk = 8, 64
    q = torch.full((1, s1, N1, 128), float("inf")).bfloat16()
    k = torch.ones(1, s2, 1, 128).bfloat16()
    k[0, 100:110] = -1.0                          # q.k = -inf -> ReLU 0 -> score 0
    w = -torch.ones(1, s1, N1).bfloat16()          # every other key: -1 * ReLU(+inf) = -inf
    inst = bsnd_inst(q, k, w, topk=topk, mask_mode=0)
    inst["name"] = f"neg_inf_{s1}x{s2}"
    gi, gv = _gpu(inst)
    want = sorted(list(range(100, 110)) + list(range(topk - 10)))
    for r in range(s1):
        assert sorted(gi[r].tolist()) == want
        for j, e in enumerate(gi[r].tolist()):
            if 100 <= e < 110:
                assert gv[r, j] == 0.0
            else:
                assert np.isneginf(gv[r, j])


def _meta_items(inst):
    """Runs li_metadata for an instance; returns (header int32[6], items [n, 4])."""
    dev = torch.device("cuda")
    p = binding.problem_for(inst)
    args = {n: (inst[n].to(dev) if isinstance(inst.get(n), torch.Tensor) else None)
            for n in ("cu_seqlens_q", "cu_seqlens_k", "seqused_k")}
    meta = binding.lightning_indexer_metadata(p, device=dev, **args)
    torch.cuda.synchronize()
    m = meta.cpu().numpy()
    hdr = m[:24].view(np.int32)
    B = inst["batch"]
    off = 256
    off = -(-(off + 16 * B) // 16) * 16           # counts
    off = -(-(off + 4 * B) // 16) * 16            # starts
    off = -(-(off + 4 * B) // 16) * 16            # items
    items = m[off:off + 16 * int(hdr[0])].view(np.int32).reshape(-1, 4)
    return hdr, items


@pytest.mark.parametrize("spec", [
    dict(batch=64, s1=1, n1=64, topk=2048, layout_k="PA_BSND", len_lo=8192, len_hi=32768,
         block_size=128),
    dict(batch=7, s1=3, n1=8, topk=64, layout_k="PA_BSND", len_lo=1, len_hi=5000, block_size=32),
    dict(batch=300, s1=2, n1=8, topk=16, layout_k="PA_BSND", len_lo=0, len_hi=3000,
         block_size=64),
    # the largest batch the metadata kernel plans in one wave (4 batches per lane)
    dict(batch=256, s1=4, n1=8, topk=16, layout_k="PA_BSND", len_lo=0, len_hi=2500,
         block_size=64),
])
def test_decode_work_list(spec):
    """Decode segments tile every row's visible keys exactly, start on 32-key
    boundaries, share one length and stay within the segment budget."""
    inst = synth.make(synth.Spec(name="wl", **spec), 5)
    hdr, items = _meta_items(inst)
    assert hdr[1] == 2 and hdr[3] == 0x4C494D44            # decode mode, magic
    chunk = int(hdr[2])
    assert chunk % 32 == 0 and chunk >= 64
    nrows = spec["batch"] * spec["s1"]
    target = 1024
    while target < 2 * nrows:
        target += 1024
    real = items[items[:, 3] > items[:, 2]]
    assert len(real) <= target
    assert (items[items[:, 3] <= items[:, 2]] == 0).all()       # padding items are empty
    seen = {}
    for b, i, k0, k1 in real.tolist():
        assert k0 % 32 == 0 and 0 < k1 - k0 <= chunk
        seen.setdefault((b, i), []).append((k0, k1))
    if spec["batch"] <= 256:
        # whole rounds of 8 workgroups x 4 items; workgroup w runs on XCD w % 8:
        # every XCD gets the same number of full segments and of short ones, +-1
        assert len(items) % 32 == 0
        xcd = (np.arange(len(items)) // 4) % 8
        full = items[:, 3] - items[:, 2] == chunk
        short = (items[:, 3] > items[:, 2]) & ~full
        for m in (full, short):
            per = np.bincount(xcd[m], minlength=8)
            assert per.max() - per.min() <= 1, per
    for b in range(spec["batch"]):
        s2 = inst["seqlens_k"][b]
        for i in range(spec["s1"]):
            lim = max(0, min(s2, i + s2 - spec["s1"] + 1))
            segs = sorted(seen.get((b, i), []))
            covered = 0
            for k0, k1 in segs:
                assert k0 == covered
                covered = k1
            assert covered == lim, (b, i, segs[:3], lim)
    # the segment length is the shortest of eight candidates (multiples of 32
    # from max(64, total / budget) up to total / (budget - rows), which always
    # fits) whose segments fit the budget
    lims = [max(0, min(inst["seqlens_k"][b], i + inst["seqlens_k"][b] - spec["s1"] + 1))
            for b in range(spec["batch"]) for i in range(spec["s1"])]
    cdiv = lambda x, y: -(-x // y)
    tot = sum(lims)
    c_lo = max(64, cdiv(cdiv(tot, target), 32) * 32)
    c_hi = max(c_lo, cdiv(cdiv(tot, target - nrows), 32) * 32)
    step = max(32, cdiv(cdiv(c_hi - c_lo, 7), 32) * 32)
    cands = [c_lo + j * step for j in range(7)] + [c_hi]
    fits = [c for c in cands if c <= c_hi and sum(cdiv(x, c) for x in lims) <= target]
    assert chunk == min(fits), (chunk, cands, fits)


@pytest.mark.parametrize("spec", [
    dict(batch=8, n1=64, topk=2048, layout_q="TND", layout_k="TND", len_lo=1024, len_hi=16384),
    dict(batch=3, n1=8, topk=64, layout_q="TND", layout_k="TND", len_lo=10, len_hi=3000),
    dict(batch=1, s1=4096, s2=4096, n1=64, topk=2048),
])
def test_prefill_work_list(spec):
    """Prefill items cover every block of every sequence exactly once, each
    batch's blocks come last-row-first, and no XCD (index mod 8) is fed the
    blocks of a single batch only."""
    inst = synth.make(synth.Spec(name="wlp", **spec), 3)
    hdr, items = _meta_items(inst)
    assert hdr[1] in (0, 1, 3)                            # rows in LDS, workspace rows, lists
    rows = 4
    want = set()
    for b in range(spec["batch"]):
        s1 = inst["seqlens_q"][b]
        for q0 in range(0, s1, rows):
            want.add((b, q0, min(rows, s1 - q0)))
    got = [tuple(x[:3]) for x in items.tolist()]
    assert len(got) == len(want) and set(got) == want
    for b in range(spec["batch"]):
        q0s = [q0 for bb, q0, _ in got if bb == b]
        assert q0s == sorted(q0s, reverse=True)
    if spec["batch"] > 1:
        for b in range(spec["batch"]):
            xcds = {u % 8 for u, (bb, _, _) in enumerate(got) if bb == b}
            assert len(xcds) > 1


# --------------------------------------------------------------------------
# the five workloads at full size
# --------------------------------------------------------------------------

def _row_offsets(inst):
    return np.concatenate([[0], np.cumsum(inst["seqlens_q"])]).astype(np.int64)


def strata_rows(inst):
    """First and last row of every sequence and the rows around |V| = k."""
    off = _row_offsets(inst)
    topk = inst["topk"]
    rows = set()
    for b in range(inst["batch"]):
        s1, s2 = inst["seqlens_q"][b], inst["seqlens_k"][b]
        if s1 == 0:
            continue
        rows.update({int(off[b]), int(off[b] + s1 - 1)})
        if inst["mask_mode"] == 3:
            i_k = topk - 1 - (s2 - s1)          # row whose visible count is exactly k
            for d in (-2, -1, 0, 1, 2):
                if 0 <= i_k + d < s1:
                    rows.add(int(off[b] + i_k + d))
    return rows


def slot_rows(inst, items, grid, rounds, slots):
    """One row of the item that grid slot j runs in round r (item j + r * grid),
    for the listed slots and rounds: rows whose workspace rows other items of
    the same slot used before them."""
    off = _row_offsets(inst)
    rows = set()
    for r in rounds:
        for j in slots:
            u = j + r * grid
            if u >= len(items):
                continue
            b, q0, nr = (int(x) for x in items[u][:3])
            rows.add(int(off[b] + q0 + (u + r) % max(nr, 1)))
    return rows


def full_size_rows(name, inst, seed):
    """Rows compared value by value with the oracle; None = every row."""
    if name in ("tiny", "prefill", "decode"):
        return None
    total = int(sum(inst["seqlens_q"]))
    rng = np.random.default_rng(1000 + seed)
    rows = strata_rows(inst)
    _, items = _meta_items(inst)
    grid = min(len(items), 512)                   # resident slots of the list kernel
    if name == "varlen":
        # every slot in its first two rounds, every 4th slot in every later round,
        # and seeded random rows
        rows |= slot_rows(inst, items, grid, (0, 1), range(grid))
        later = range(2, -(-len(items) // grid))
        rows |= slot_rows(inst, items, grid, later, range(0, grid, 64))
        rows.update(rng.integers(0, total, 128).tolist())
        assert len(rows) >= 1024
    else:                                         # longfp8
        rows.update(np.linspace(0, total - 1, 256).round().astype(np.int64).tolist())
        rows |= slot_rows(inst, items, grid, range(-(-len(items) // grid)), range(0, grid, 32))
        assert len(rows) >= 256
    return sorted(rows)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("name", ["tiny", "prefill", "decode", "varlen", "longfp8"])
def test_full_size_config(name, seed):
    inst = synth.make(name, seed)
    rows = full_size_rows(name, inst, seed)
    _say(f"    comparing {'every' if rows is None else len(rows)} rows with the oracle")
    compare_all(inst, rows=rows)


def _by_index(idx, val):
    """Each row's entries sorted by index (the order inside the valid prefix is
    not part of the contract), values carried along as raw bits."""
    order = np.argsort(idx, axis=1, kind="stable")
    return np.take_along_axis(idx, order, 1), np.take_along_axis(val.view(np.uint32), order, 1)


def test_determinism_across_splits():
    """A row's output does not depend on how the work was cut: the same
    sequences run in one batch (one decode segment length, one work list) and
    each on its own (other segment lengths, other items, and for the TND case
    rows in LDS instead of the workspace) give the same index set per row with
    bitwise equal values."""
    dec = synth.Spec(name="split_dec", batch=6, s1=2, n1=64, topk=300, layout_k="PA_BSND",
                     len_lo=1000, len_hi=30000, block_size=128, w_scale=0.125)
    inst = synth.make(dec, 31)
    gi, gv = _gpu(inst)
    bs, nq = inst["block_size"], 2
    for b in range(inst["batch"]):
        L = inst["seqlens_k"][b]
        nb = -(-L // bs)
        one = dict(inst, batch=1, seqlens_q=[nq], seqlens_k=[L], max_seqlen_k=L,
                   max_blocks_per_seq=nb, seqused_k=inst["seqused_k"][b:b + 1].clone(),
                   block_table=inst["block_table"][b:b + 1, :nb].clone(),
                   q=inst["q"][b:b + 1].clone(), w=inst["w"][b:b + 1].clone(),
                   name=f"split_dec_b{b}")
        oi, ov = _gpu(one)
        a, b_ = _by_index(oi, ov), _by_index(gi[b * nq:(b + 1) * nq], gv[b * nq:(b + 1) * nq])
        assert np.array_equal(a[0], b_[0]) and np.array_equal(a[1], b_[1]), b
    # prefill: TND sequences alone and packed with others (rows in LDS and in the workspace)
    tnd = synth.Spec(name="split_tnd", batch=4, n1=64, topk=256, layout_q="TND",
                     layout_k="TND", fixed_lengths=[3000, 700, 5200, 64], w_scale=0.125)
    inst = synth.make(tnd, 32)
    gi, gv = _gpu(inst)
    off = _row_offsets(inst)
    for b in (0, 2, 3):
        L = inst["seqlens_q"][b]
        sl = slice(int(off[b]), int(off[b] + L))
        one = dict(inst, batch=1, seqlens_q=[L], seqlens_k=[L], max_seqlen_q=L,
                   max_seqlen_k=L, total_q=L, total_k=L,
                   cu_seqlens_q=torch.tensor([L], dtype=torch.int32),
                   cu_seqlens_k=torch.tensor([L], dtype=torch.int32),
                   q=inst["q"][sl].clone(), k=inst["k"][sl].clone(), w=inst["w"][sl].clone(),
                   name=f"split_tnd_b{b}")
        oi, ov = _gpu(one)
        a, b_ = _by_index(oi, ov), _by_index(gi[sl], gv[sl])
        assert np.array_equal(a[0], b_[0]) and np.array_equal(a[1], b_[1]), b


def _device_inputs(inst, dev):
    g = {n: (inst[n].to(dev) if isinstance(inst.get(n), torch.Tensor) else None)
         for n in ("q", "k", "w", "q_descale", "k_descale", "cu_seqlens_q", "cu_seqlens_k",
                   "seqused_k", "block_table", "cmp_residual_k", "output_idx_offset")}
    if inst["layout_k"] == "PA_BSND":
        kc = inst["k"]
        base = kc.as_strided((kc.shape[0], kc.stride(0)), (kc.stride(0), 1)).to(dev)
        g["k"] = base.as_strided(kc.shape, kc.stride())
    return g


def _forward(p, g, meta):
    st, wsb = binding.li_workspace_size(p)
    assert st == 0
    ws = torch.empty(wsb, dtype=torch.uint8, device=g["q"].device)
    idx, val = binding.lightning_indexer(
        p, g["q"], g["k"], g["w"], metadata=meta, q_descale=g["q_descale"],
        k_descale=g["k_descale"], cu_seqlens_q=g["cu_seqlens_q"], cu_seqlens_k=g["cu_seqlens_k"],
        seqused_k=g["seqused_k"], block_table=g["block_table"], workspace=ws)
    return idx, val, binding.forward_status(ws)


@pytest.mark.parametrize("spec", [
    dict(batch=2, s1=300, s2=300, n1=16, topk=64),                      # rows in LDS
    dict(batch=1, s1=20, s2=6000, n1=16, topk=64),                      # rows in the workspace
    dict(batch=3, s1=1, n1=16, topk=64, layout_k="PA_BSND", len_lo=500, len_hi=3000,
         block_size=64),                                                # decode
])
def test_metadata_of_another_problem(spec):
    """Metadata built for another problem is refused on the device: the same batch
    and lengths with another topk (so that every item read would stay in bounds even
    without the check) give -1 / -inf everywhere and the mismatch status word, and
    li_gather then writes zero rows; the matching call reports LI_OK."""
    dev = torch.device("cuda")
    inst = synth.make(synth.Spec(name="meta_mismatch", **spec), 40)
    _say(f"[gpu] metadata mismatch {spec}")
    g = _device_inputs(inst, dev)
    p = binding.problem_for(inst, g["k"])
    meta = binding.lightning_indexer_metadata(p, cu_seqlens_q=g["cu_seqlens_q"],
                                              cu_seqlens_k=g["cu_seqlens_k"],
                                              seqused_k=g["seqused_k"], device=dev)
    idx, val, st = _forward(p, g, meta)
    assert st == 0
    ok_idx = idx.reshape(-1, p.topk)
    assert (ok_idx[:, 0] >= 0).any()
    p2 = binding.problem_for(dict(inst, topk=2 * p.topk), g["k"])
    assert binding.li_metadata_size(p2)[1] == binding.li_metadata_size(p)[1]
    idx2, val2, st2 = _forward(p2, g, meta)
    assert st2 == 5 and binding.li_status_str(st2) == "LI_ERR_METADATA_MISMATCH"
    assert (idx2 == -1).all() and torch.isneginf(val2).all()
    # li_gather with the same foreign metadata: valid indices (from the matching
    # call, so reads would stay in bounds) still give zero rows
    sel = torch.cat([ok_idx, ok_idx], dim=1).clamp(min=0).contiguous()
    kv = (torch.arange(int(inst["k"].numel()) // 128 * 16, device=dev) % 251 + 1).to(torch.uint8)
    if inst["layout_k"] == "PA_BSND":
        kv = kv.reshape(inst["k"].shape[0], inst["block_size"], 16)
    else:
        kv = kv.reshape(*inst["k"].shape[:-2], 16)
    out = binding.gather_selected(p2, kv, sel, metadata=meta, block_table=g["block_table"])
    torch.cuda.synchronize()
    assert (out == 0).all()
    out_ok = binding.gather_selected(p, kv, ok_idx.contiguous(), metadata=meta,
                                     block_table=g["block_table"])
    torch.cuda.synchronize()
    assert (out_ok != 0).any()
