"""Pins of the CPU oracle to facts outside itself.

Each `pin_*` function raises AssertionError when the oracle disagrees with
something the pages or the mathematics fix:
  - the element decoders against torch's own bf16 / fp16 / e4m3fn converters;
  - closed forms (one-hot queries, a single negative weight, two one-hot heads);
  - exact integer arithmetic: with small integer q, k, w every score is an
    integer, so the oracle must equal an int64 matmul-based brute force exactly;
  - the visible-set size of right-down causal masking and of mask 0, and the
    -1 / -inf padding of the invalid tail (lightning_indexer page, Constraints);
  - the top-k rule by pairwise dominance (every kept key beats every dropped key,
    ties going to the smaller index) and the all-zero-score case;
  - layout equivalences: paged K with a random block table and padded pool,
    TND packing, fp8 codes with unit descales, fp16 codes, fp32 weights;
  - exact power-of-two scaling laws of w and of the fp8 descales;
  - compressed keys (cmp_ratio): visible counts against a walk over the original
    sequence for the pages' example shapes and a closed form, scores unchanged by
    compression; output index offsets.
tests/test_oracle_pins.py runs them on the real oracle; tests/test_oracle_mutants.py
runs them on copies of the oracle with planted mistakes and requires each mistake
to be caught.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from score_top_token_amd import synth
from tests.util import bsnd_inst, int_tensor, valid_prefix_len


# --------------------------------------------------------------------------
# element decoding
# --------------------------------------------------------------------------

def pin_decode_bf16():
    codes = torch.arange(0, 65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    ref = codes.to(torch.float64).numpy()
    got = oracle.decode("bf16", codes)
    ok = np.isnan(ref) == np.isnan(got)
    ok &= (ref == got) | np.isnan(ref)
    assert ok.all(), "bf16 decoding differs from torch"


def pin_decode_fp16():
    codes = torch.arange(0, 65536, dtype=torch.int32).to(torch.int16).view(torch.float16)
    ref = codes.to(torch.float64).numpy()
    got = oracle.decode("fp16", codes)
    ok = np.isnan(ref) == np.isnan(got)
    ok &= (ref == got) | np.isnan(ref)
    assert ok.all(), "fp16 decoding differs from torch"


def pin_decode_e4m3():
    codes = torch.arange(0, 256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = codes.to(torch.float64).numpy()
    got = oracle.decode("fp8", codes)
    ok = np.isnan(ref) == np.isnan(got)
    ok &= (ref == got) | np.isnan(ref)
    assert ok.all(), "e4m3fn decoding differs from torch"
    # published anchor points of OCP e4m3fn
    raw = lambda c: float(oracle.decode("fp8", torch.tensor([c], dtype=torch.uint8))[0])
    assert raw(0x38) == 1.0 and raw(0xB8) == -1.0
    assert raw(0x7E) == 448.0 and raw(0x01) == 2.0 ** -9 and raw(0x08) == 2.0 ** -6
    assert math.isnan(raw(0x7F))


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def _onehot_case(weight: float, seed: int, mask_mode=0):
    g = torch.Generator().manual_seed(seed)
    S, D, a, d0 = 48, 128, 3, 37
    q = torch.zeros(1, S, 1, D)
    q[..., d0] = 2.0 ** a
    k = torch.randn(1, S, 1, D, generator=g)
    w = torch.full((1, S, 1), weight)
    inst = bsnd_inst(q.bfloat16(), k.bfloat16(), w.bfloat16(), topk=16, mask_mode=mask_mode)
    kk = inst["k"].to(torch.float64)[0, :, 0, d0].numpy()
    expect = weight * (2.0 ** a) * np.maximum(kk, 0.0)   # exact: power-of-two scaling
    return inst, expect


def pin_onehot_single_head():
    inst, expect = _onehot_case(1.0, 1)
    ob = oracle.Bound(inst)
    idx, val = ob.forward()
    order = np.lexsort((np.arange(expect.size), -expect))[:16]
    for r in range(idx.shape[0]):
        assert list(idx[r]) == list(order), "ranking of one-hot scores"
        assert np.array_equal(val[r], expect[order].astype(np.float32))
    for s in (0, 5, 47):
        assert ob.score(0, 3, s) == expect[s]


def pin_negative_weight():
    inst, expect = _onehot_case(-1.0, 2)
    ob = oracle.Bound(inst)
    idx, val = ob.forward()
    assert (val <= 0).all()
    order = np.lexsort((np.arange(expect.size), -expect))[:16]
    assert list(idx[0]) == list(order)
    assert np.array_equal(val[0], expect[order].astype(np.float32))


def pin_negative_zero_is_canonical():
    # A negative weight times a positive dot product far below fp32's smallest
    # subnormal (2^-149) is a negative fp64 score that rounds to -0 in fp32; a
    # zero ReLU gives an exact zero.  Every written value must then be +0 (sign
    # bit clear), while the ranking still follows the exact fp64 scores: the
    # exact zeros first (ascending key), then the tiny negatives by magnitude.
    g = torch.Generator().manual_seed(12)
    S, D, d0 = 48, 128, 11
    wt, a = -(2.0 ** -120), -40
    q = torch.zeros(1, 1, 1, D)
    q[..., d0] = 2.0 ** a
    k = torch.randn(1, S, 1, D, generator=g)
    w = torch.full((1, 1, 1), wt)
    inst = bsnd_inst(q.bfloat16(), k.bfloat16(), w.bfloat16(), topk=S, mask_mode=0)
    kk = inst["k"].to(torch.float64)[0, :, 0, d0].numpy()
    expect = wt * (2.0 ** a) * np.maximum(kk, 0.0)      # exact in fp64, |x| < 2^-150
    assert (kk > 0).any() and (kk <= 0).any()
    idx, val = oracle.Bound(inst).forward()
    order = np.lexsort((np.arange(S), -expect))
    assert list(idx[0]) == list(order), "ranking by the exact fp64 scores"
    assert (val[0] == 0).all(), "tiny scores round to zero"
    assert not np.signbit(val[0]).any(), "-0 written where +0 is due"


def pin_two_onehot_heads():
    g = torch.Generator().manual_seed(3)
    S, D, d0, d1 = 40, 128, 5, 90
    w0, w1 = 0.75, -2.5
    q = torch.zeros(1, S, 2, D)
    q[:, :, 0, d0] = 1.0
    q[:, :, 1, d1] = 4.0
    k = torch.randn(1, S, 1, D, generator=g)
    w = torch.tensor([w0, w1]).expand(1, S, 2).contiguous()
    inst = bsnd_inst(q.bfloat16(), k.bfloat16(), w.bfloat16(), topk=40, mask_mode=0)
    kk = inst["k"].to(torch.float64)[0, :, 0].numpy()
    expect = w0 * np.maximum(kk[:, d0], 0) + w1 * 4.0 * np.maximum(kk[:, d1], 0)
    ob = oracle.Bound(inst)
    for s in range(S):
        assert ob.score(0, 7, s) == expect[s], "two one-hot heads"


def pin_duplicated_heads():
    # two identical heads with weights a, b equal one head with weight a + b
    g = torch.Generator().manual_seed(4)
    S, D = 32, 128
    q1 = torch.randn(1, S, 1, D, generator=g).bfloat16()
    k = torch.randn(1, S, 1, D, generator=g).bfloat16()
    a, b = 0.375, 1.25
    inst2 = bsnd_inst(q1.expand(1, S, 2, D).contiguous(), k,
                      torch.tensor([a, b]).expand(1, S, 2).contiguous().bfloat16(), topk=8)
    inst1 = bsnd_inst(q1, k, torch.full((1, S, 1), a + b).bfloat16(), topk=8)
    i2, v2 = oracle.Bound(inst2).forward()
    i1, v1 = oracle.Bound(inst1).forward()
    assert np.array_equal(i1, i2) and np.array_equal(v1, v2), "duplicated heads"


# --------------------------------------------------------------------------
# exact integer brute force
# --------------------------------------------------------------------------

def _int_case(seed, B=2, S1=24, S2=24, N1=5, topk=7, mask_mode=3):
    g = torch.Generator().manual_seed(seed)
    q = int_tensor(g, (B, S1, N1, 128), -3, 3)
    k = int_tensor(g, (B, S2, 1, 128), -3, 3)
    w = int_tensor(g, (B, S1, N1), -4, 4)
    return bsnd_inst(q, k, w, topk=topk, mask_mode=mask_mode)


def _brute_force(inst):
    """int64 brute force: every visible (row, key) score, then a full ranking."""
    q = inst["q"].to(torch.float64).numpy().astype(np.int64)
    k = inst["k"].to(torch.float64).numpy().astype(np.int64)
    w = inst["w"].to(torch.float64).numpy().astype(np.int64)
    B, S1, N1, _ = q.shape
    S2 = k.shape[1]
    topk = inst["topk"]
    out_i = np.full((B * S1, topk), -1, dtype=np.int64)
    out_v = np.full((B * S1, topk), -np.inf)
    for b in range(B):
        x = np.einsum("ihd,sd->ihs", q[b], k[b, :, 0])          # exact int64 contraction
        score = (w[b][:, :, None] * np.maximum(x, 0)).sum(axis=1)   # [S1, S2]
        for i in range(S1):
            keys = [s for s in range(S2)
                    if inst["mask_mode"] == 0 or s <= i + S2 - S1]
            ranked = sorted(keys, key=lambda s: (-score[i, s], s))[:topk]
            for j, s in enumerate(ranked):
                out_i[b * S1 + i, j] = s
                out_v[b * S1 + i, j] = score[i, s]
    return out_i, out_v


def pin_integer_bruteforce():
    for seed, kw in ((10, {}), (11, dict(mask_mode=0)), (12, dict(S1=9, S2=30, topk=12)),
                     (13, dict(S1=30, S2=9, topk=4)), (14, dict(N1=1, topk=1))):
        inst = _int_case(seed, **kw)
        bi, bv = _brute_force(inst)
        oi, ov = oracle.Bound(inst).forward()
        assert np.array_equal(oi, bi), f"indices vs integer brute force (seed {seed})"
        assert np.array_equal(ov.astype(np.float64), bv), f"values vs brute force (seed {seed})"


# --------------------------------------------------------------------------
# masking, padding, top-k rule
# --------------------------------------------------------------------------

def pin_visible_counts():
    for (S1, S2, mask) in ((20, 20, 3), (6, 30, 3), (30, 6, 3), (7, 13, 0), (1, 50, 3)):
        g = torch.Generator().manual_seed(S1 * 100 + S2)
        q = torch.randn(1, S1, 2, 128, generator=g).bfloat16()
        k = torch.randn(1, S2, 1, 128, generator=g).bfloat16()
        w = torch.randn(1, S1, 2, generator=g).bfloat16()
        topk = 8
        inst = bsnd_inst(q, k, w, topk=topk, mask_mode=mask)
        ob = oracle.Bound(inst)
        idx, val = ob.forward()
        for i in range(S1):
            vis = S2 if mask == 0 else min(max(i + S2 - S1 + 1, 0), S2)
            assert ob.visible_count(0, i) == vis
            n = valid_prefix_len(idx[i])
            assert n == min(topk, vis), "number of valid entries"
            assert (idx[i, :n] < vis).all(), "index outside the visible window"
            assert len(set(idx[i, :n].tolist())) == n, "duplicate index"
            pad = val[i, n:]
            assert np.all(np.isneginf(pad)) and np.all(np.signbit(pad)), "value padding"
            if vis <= topk:
                assert sorted(idx[i, :n].tolist()) == list(range(vis)), "short row keeps all keys"


def pin_dominance():
    g = torch.Generator().manual_seed(21)
    S1, S2, N1, topk = 12, 40, 6, 9
    q = torch.randn(1, S1, N1, 128, generator=g).bfloat16()
    k = torch.randn(1, S2, 1, 128, generator=g).bfloat16()
    w = (torch.randn(1, S1, N1, generator=g) / 3).bfloat16()
    inst = bsnd_inst(q, k, w, topk=topk, mask_mode=3)
    ob = oracle.Bound(inst)
    idx, val = ob.forward()
    for i in range(S1):
        vis = ob.visible_count(0, i)
        sc = {s: ob.score(0, i, s) for s in range(vis)}
        n = valid_prefix_len(idx[i])
        kept = set(idx[i, :n].tolist())
        for s in kept:
            assert np.float32(sc[s]) == val[i][list(idx[i]).index(s)], "value of a kept key"
            for t in set(range(vis)) - kept:
                assert sc[s] > sc[t] or (sc[s] == sc[t] and s < t), "dominance"
        # oracle order: score descending, index ascending
        for j in range(n - 1):
            a, b = idx[i, j], idx[i, j + 1]
            assert sc[a] > sc[b] or (sc[a] == sc[b] and a < b), "oracle output order"


def pin_all_zero_scores():
    S, topk = 30, 11
    q = torch.zeros(1, S, 3, 128).bfloat16()
    k = torch.ones(1, S, 1, 128).bfloat16()
    w = torch.ones(1, S, 3).bfloat16()
    inst = bsnd_inst(q, k, w, topk=topk, mask_mode=3)
    idx, val = oracle.Bound(inst).forward()
    for i in range(S):
        n = min(topk, i + 1)
        assert list(idx[i, :n]) == list(range(n)), "ties go to the smallest indices"
        assert np.all(val[i, :n] == 0.0) and not np.any(np.signbit(val[i, :n]))


def pin_exact_ties():
    # scores take few integer values, so ties straddle the k-th place often
    g = torch.Generator().manual_seed(31)
    B, S, N1, topk = 1, 60, 2, 13
    q = int_tensor(g, (B, S, N1, 128), 0, 1)
    q[..., 2:] = 0
    k = int_tensor(g, (B, S, 1, 128), 0, 1)
    w = torch.ones(B, S, N1).bfloat16()
    inst = bsnd_inst(q, k, w, topk=topk, mask_mode=0)
    bi, _ = _brute_force(inst)
    oi, _ = oracle.Bound(inst).forward()
    assert np.array_equal(oi, bi), "tie-break by index"


# --------------------------------------------------------------------------
# layouts and dtypes
# --------------------------------------------------------------------------

def pin_paged_equals_bsnd():
    spec = synth.Spec(name="pa", batch=3, s1=4, n1=4, topk=10, layout_k="PA_BSND",
                      len_lo=40, len_hi=90, block_size=16, block_pad=3, mask_mode=3)
    inst = synth.make(spec, seed=5)
    oi, ov = oracle.Bound(inst).forward()
    bs = inst["block_size"]
    for b in range(inst["batch"]):
        L = inst["seqlens_k"][b]
        rows = [inst["k"][inst["block_table"][b, s // bs], s % bs] for s in range(L)]
        kb = torch.stack(rows).unsqueeze(0)                       # [1, L, 1, D]
        ref = bsnd_inst(inst["q"][b:b + 1], kb, inst["w"][b:b + 1], topk=10, mask_mode=3)
        ri, rv = oracle.Bound(ref).forward()
        S1 = inst["max_seqlen_q"]
        assert np.array_equal(oi[b * S1:(b + 1) * S1], ri), "paged indices"
        assert np.array_equal(ov[b * S1:(b + 1) * S1], rv), "paged values"


def pin_tnd_equals_bsnd():
    spec = synth.Spec(name="tnd", batch=3, n1=3, topk=6, layout_q="TND", layout_k="TND",
                      fixed_lengths=[9, 17, 5], mask_mode=3)
    inst = synth.make(spec, seed=6)
    oi, ov = oracle.Bound(inst).forward()
    off = 0
    for b, L in enumerate(inst["seqlens_q"]):
        ref = bsnd_inst(inst["q"][off:off + L].unsqueeze(0), inst["k"][off:off + L].unsqueeze(0),
                        inst["w"][off:off + L].unsqueeze(0), topk=6, mask_mode=3)
        ri, rv = oracle.Bound(ref).forward()
        assert np.array_equal(oi[off:off + L], ri) and np.array_equal(ov[off:off + L], rv), "TND"
        off += L


def pin_tnd_chunked_keys():
    # TND with more keys than queries: right-down causal aligns the last query with the last key
    spec = synth.Spec(name="tndc", batch=2, n1=2, topk=5, layout_q="TND", layout_k="TND",
                      fixed_lengths=[4, 6], kv_extra=7, mask_mode=3)
    inst = synth.make(spec, seed=7)
    ob = oracle.Bound(inst)
    oi, _ = ob.forward()
    for b, (Lq, Lk) in enumerate(zip(inst["seqlens_q"], inst["seqlens_k"])):
        for i in range(Lq):
            assert ob.visible_count(b, i) == i + Lk - Lq + 1


def pin_fp8_unit_descale_equals_bf16():
    g = torch.Generator().manual_seed(8)
    S, N1 = 20, 4
    qv = int_tensor(g, (1, S, N1, 128), -8, 8, torch.float32)
    kv = int_tensor(g, (1, S, 1, 128), -8, 8, torch.float32)
    w = (torch.randn(1, S, N1, generator=g)).bfloat16()
    ones_q, ones_k = torch.ones(1, S), torch.ones(1, S)
    i8 = bsnd_inst(qv.to(torch.float8_e4m3fn), kv.to(torch.float8_e4m3fn), w, topk=6,
                   qk_dtype="fp8", q_descale=ones_q, k_descale=ones_k)
    ib = bsnd_inst(qv.bfloat16(), kv.bfloat16(), w, topk=6)
    a = oracle.Bound(i8).forward()
    b = oracle.Bound(ib).forward()
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), "fp8 with unit descales"
    # fp16 codes of the same small integers give the same result
    i16 = bsnd_inst(qv.half(), kv.half(), w, topk=6, qk_dtype="fp16")
    c = oracle.Bound(i16).forward()
    assert np.array_equal(c[0], b[0]) and np.array_equal(c[1], b[1]), "fp16 codes"
    # fp32 weights holding bf16 values give the same result
    i32 = bsnd_inst(qv.bfloat16(), kv.bfloat16(), w.float(), topk=6, w_dtype="fp32")
    d = oracle.Bound(i32).forward()
    assert np.array_equal(d[0], b[0]) and np.array_equal(d[1], b[1]), "fp32 weights"


def pin_power_of_two_scaling():
    spec = synth.Spec(name="f8", batch=1, s1=24, s2=40, n1=4, topk=7, qk_dtype="fp8", mask_mode=3)
    inst = synth.make(spec, seed=9)
    base_i, base_v = oracle.Bound(inst).forward()
    scaled = dict(inst)
    scaled["q_descale"] = inst["q_descale"] * 4.0
    scaled["k_descale"] = inst["k_descale"] * 0.125
    scaled["w"] = (inst["w"].float() * 8.0).bfloat16()
    si, sv = oracle.Bound(scaled).forward()
    assert np.array_equal(si, base_i), "scaling must not change the ranking"
    ok = base_v > -np.inf
    assert np.array_equal(sv[ok], base_v[ok] * 4.0), "values scale by 2^2 exactly"
    # a descale that is not a power of two changes the values by that factor (within fp32)
    s2 = dict(inst)
    s2["k_descale"] = inst["k_descale"] * 3.0
    ti, tv = oracle.Bound(s2).forward()
    assert np.array_equal(ti, base_i)
    assert np.allclose(tv[ok], base_v[ok] * 3.0, rtol=1e-6, atol=0)


def pin_pages_example_shape():
    """The lightning_indexer page's example call: B=2, S1=64, compressed S2=32, N1=16,
    topk=32, mask_mode=3 -> outputs [2, 64, 1, 32] (its printed output is the shape only)."""
    import json
    import os
    here = os.path.dirname(os.path.abspath(__file__))
    with open(os.path.join(here, "golden", "pages_example_shape.json")) as f:
        ex = json.load(f)
    g = torch.Generator().manual_seed(0)
    B, S1, S2, N1, D, topk = (ex[n] for n in ("B", "S1", "S2", "N1", "D", "topk"))
    q = torch.randn(B, S1, N1, D, generator=g).half()
    k = torch.randn(B, S2, 1, D, generator=g).half()
    w = torch.randn(B, S1, N1, generator=g)
    inst = bsnd_inst(q, k, w, topk=topk, mask_mode=ex["mask_mode"], qk_dtype="fp16",
                     w_dtype="fp32")
    idx, val = oracle.Bound(inst).forward()
    assert list(idx.reshape(B, S1, 1, topk).shape) == ex["output_shape"]
    for r in range(B * S1):
        i = r % S1
        vis = min(max(i + S2 - S1 + 1, 0), S2)
        assert valid_prefix_len(idx[r]) == min(topk, vis)


def _simulated_compressed_counts(S1, S2_orig, r):
    """Visible compressed keys per query row, by walking the original sequence:
    a compressed key exists once all r of its original positions have passed;
    the trailing S2_orig % r positions never complete a key.  The S1 query rows
    are the last S1 original positions (right-down alignment)."""
    done, counts = 0, []
    for t in range(S2_orig):
        if (t + 1) % r == 0:
            done += 1
        if t >= S2_orig - S1:
            counts.append(done)
    return counts


def pin_pages_example_compressed():
    """The same example with its compression: 130 original keys, cmp_ratio 4 ->
    32 keys with residual 2; row i sees the keys whose 4 original positions all
    lie at or before its own original position."""
    import json
    import os
    here = os.path.dirname(os.path.abspath(__file__))
    with open(os.path.join(here, "golden", "pages_example_compressed.json")) as f:
        ex = json.load(f)
    B, S1, S2o, r, N1, D, topk = (ex[n] for n in ("B", "S1", "S2_original", "cmp_ratio", "N1",
                                                  "D", "topk"))
    S2, res = S2o // r, S2o % r
    g = torch.Generator().manual_seed(1)
    q = torch.randn(B, S1, N1, D, generator=g).half()
    k = torch.randn(B, S2, 1, D, generator=g).half()
    w = torch.randn(B, S1, N1, generator=g)
    inst = bsnd_inst(q, k, w, topk=topk, mask_mode=ex["mask_mode"], qk_dtype="fp16",
                     w_dtype="fp32")
    inst["cmp_ratio"] = r
    inst["cmp_residual_k"] = torch.full((B,), res, dtype=torch.int32)
    ob = oracle.Bound(inst)
    idx, _ = ob.forward()
    assert list(idx.reshape(B, S1, 1, topk).shape) == ex["output_shape"]
    want = _simulated_compressed_counts(S1, S2o, r)
    assert want[-1] == S2 and want[0] == (S2o - S1 + 1) // r
    for b in range(B):
        for i in range(S1):
            assert ob.visible_count(b, i) == want[i], (b, i)
            n = valid_prefix_len(idx[b * S1 + i])
            assert n == min(topk, want[i])
            assert (idx[b * S1 + i, :n] < want[i]).all()


def pin_compressed_counts_closed_form():
    """Full compressed prefill (S1 = original length, residual 0..r-1): row i
    sees floor((i + 1) / r) keys; a residual shifts the rows by it."""
    g = torch.Generator().manual_seed(3)
    for r, res in ((2, 0), (3, 2), (5, 1)):
        S2 = 7
        S1 = S2 * r + res
        q = torch.randn(1, S1, 2, 128, generator=g).bfloat16()
        k = torch.randn(1, S2, 1, 128, generator=g).bfloat16()
        w = torch.randn(1, S1, 2, generator=g).bfloat16()
        inst = bsnd_inst(q, k, w, topk=4, mask_mode=3)
        inst["cmp_ratio"] = r
        inst["cmp_residual_k"] = torch.tensor([res], dtype=torch.int32)
        ob = oracle.Bound(inst)
        for i in range(S1):
            assert ob.visible_count(0, i) == min(S2, (i + 1) // r), (r, res, i)
        assert _simulated_compressed_counts(S1, S1, r) == [min(S2, (i + 1) // r)
                                                          for i in range(S1)]
        inst["mask_mode"] = 0
        inst["cmp_residual_k"] = None
        ob0 = oracle.Bound(inst)
        assert all(ob0.visible_count(0, i) == S2 for i in range(S1))


def pin_compression_keeps_scores():
    """Compression changes which keys are visible, never their scores: a row that
    sees every key ranks exactly as with mask 0."""
    g = torch.Generator().manual_seed(4)
    B, S1, S2, r = 1, 10, 24, 4
    q = torch.randn(B, S1, 3, 128, generator=g).bfloat16()
    k = torch.randn(B, S2, 1, 128, generator=g).bfloat16()
    w = torch.randn(B, S1, 3, generator=g).bfloat16()
    inst = bsnd_inst(q, k, w, topk=6, mask_mode=3)
    inst["cmp_ratio"] = r
    inst["cmp_residual_k"] = torch.tensor([3], dtype=torch.int32)
    ic, vc = oracle.Bound(inst).forward()
    i0, v0 = oracle.Bound(bsnd_inst(q, k, w, topk=6, mask_mode=0)).forward()
    last = S1 - 1            # original position S2*r + 3 - 1 >= every block end
    assert np.array_equal(ic[last], i0[last]) and np.array_equal(vc[last], v0[last])


def pin_output_idx_offset():
    """output_idx_offset adds the batch's offset to every kept index and leaves the
    -1 padding and the values alone."""
    inst = synth.make(synth.Spec(name="off", batch=3, s1=40, s2=40, n1=4, topk=50,
                                 idx_offset_max=1000), 6)
    off = inst["output_idx_offset"].numpy()
    i1, v1 = oracle.Bound(inst).forward()
    plain = dict(inst)
    plain["output_idx_offset"] = None
    i0, v0 = oracle.Bound(plain).forward()
    assert np.array_equal(v1, v0)
    for r in range(i0.shape[0]):
        b = r // 40
        n = valid_prefix_len(i0[r])
        assert np.array_equal(i1[r, :n], i0[r, :n] + off[b]) and (i1[r, n:] == -1).all()


def pin_gather_closed_form():
    """Gathering rows that hold their own token number returns the selected token
    numbers: index i with block size bs gives tokens i*bs .. i*bs + bs - 1, -1
    and tokens past the sequence give zero rows (aclnnSparseFlashAttentionGrad
    page, calculation formula)."""
    from oracle.gather import gather
    for layout, extra in (("BSND", {}), ("TND", dict(layout_q="TND", layout_k="TND", len_lo=9,
                                                     len_hi=30)),
                          ("PA_BSND", dict(layout_k="PA_BSND", len_lo=9, len_hi=30,
                                           block_size=4, block_pad=1))):
        inst = synth.make(synth.Spec(name="g", batch=3, s1=5, s2=21, n1=2, topk=6, **extra), 2)
        B = inst["batch"]
        # every key slot's row = 16 bytes of 1 + its position + 40 * its sequence
        if layout == "PA_BSND":
            nb, bsz = inst["num_blocks"], inst["block_size"]
            kv = np.zeros((nb, bsz, 16), dtype=np.uint8)
            bt = inst["block_table"].numpy()
            for b in range(B):
                for s in range(inst["seqlens_k"][b]):
                    kv[bt[b, s // bsz], s % bsz, :] = s + 1 + 40 * b
        elif layout == "TND":
            kv = np.zeros((sum(inst["seqlens_k"]), 16), dtype=np.uint8)
            o = 0
            for b in range(B):
                for s in range(inst["seqlens_k"][b]):
                    kv[o + s, :] = s + 1 + 40 * b
                o += inst["seqlens_k"][b]
        else:
            kv = np.zeros((B, inst["max_seqlen_k"], 16), dtype=np.uint8)
            for b in range(B):
                for s in range(inst["max_seqlen_k"]):
                    kv[b, s, :] = s + 1 + 40 * b
        rows = sum(inst["seqlens_q"])
        g = np.random.default_rng(7)
        for sb in (1, 3):
            idx = g.integers(-1, 10, size=(rows, 6)).astype(np.int32)
            out = gather(inst, kv, idx, sb)
            r = 0
            for b in range(B):
                for _ in range(inst["seqlens_q"][b]):
                    for j in range(6):
                        for u in range(sb):
                            s = idx[r, j] * sb + u
                            want = (0 if idx[r, j] < 0 or s >= inst["seqlens_k"][b]
                                    else s + 1 + 40 * b)
                            assert (out[r, j * sb + u] == want).all(), (layout, sb, r, j, u)
                    r += 1


def pin_thread_count_invariance():
    inst = synth.make("tiny", seed=1)
    ob = oracle.Bound(inst)
    a = ob.forward(nthreads=1)
    b = ob.forward(nthreads=7)
    rows = [255, 3, 100]
    c = ob.forward(rows=rows, nthreads=2)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.array_equal(c[0], a[0][rows]) and np.array_equal(c[1], a[1][rows])


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
