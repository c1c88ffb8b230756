"""Pins of the backward + KL-loss oracle (oracle/li_grad_oracle.c) to facts
outside itself (npu_sparse_lightning_indexer_grad_kl_loss page, 计算公式 items 1-4).

Each `pin_*` raises AssertionError when the oracle disagrees with:
  - central finite differences of its own loss: the gradients of item 4 against
    the loss of items 1-3 (fp64 inputs, so every perturbation is exact);
  - PyTorch's library routines: with softmax statistics that are the max and
    sum of exp over the selected keys, the target is the head mean of
    torch.softmax, the loss torch.nn.functional.kl_div of torch.log_softmax, and
    the gradients torch.autograd's;
  - closed forms: two selected keys with equal scores and a target of (1, 0)
    give a loss of log 2 (the direction of the KL divergence); uniform target and
    scores, and rows with a single selected key, give zero loss and gradients;
  - the per-head use of the statistics (a head whose softmax_sum is huge drops
    out) and their invariances (every sum scaled, every max shifted alike);
  - -1 padding entries are skipped; TND packing equals BSND; the thread count
    does not change a bit.
tests/test_grad_oracle_pins.py runs them on the oracle; tests/test_grad_oracle_mutants.py
runs them on copies with planted mistakes.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import grad
from score_top_token_amd import synth


def _small(seed, **over):
    """A small fp64 instance (exact perturbations for the finite differences)."""
    kw = dict(name="pin", batch=2, s1=20, n_main=3, d_main=16, d_rope=8, n_idx=5, d_idx=16,
              topk=6, dtype="fp32", w_dtype="fp32", w_scale=0.5, max_mu=1.0, max_sd=0.5,
              sum_lo=2.0, sum_hi=9.0)
    kw.update(over)
    inst = synth.make_grad(synth.GradSpec(**kw), seed)
    for n in ("q", "k", "q_rope", "k_rope", "qi", "ki", "w"):
        if inst.get(n) is not None:
            inst[n] = inst[n].to(torch.float64).contiguous()
    return inst


def _total_loss(inst):
    return float(grad.Bound(inst).backward(nthreads=1)[0].sum())


def pin_finite_differences():
    inst = _small(1)
    loss, dqi, dki, dw = grad.Bound(inst).backward(nthreads=2)
    # every selected score stays far from the ReLU's kink under the perturbations
    B, S, Ni = inst["batch"], inst["max_seqlen_q"], inst["n_idx"]
    qi, ki, sel = inst["qi"].reshape(B * S, Ni, -1), inst["ki"].reshape(B * S, -1), \
        inst["sparse_indices"]
    for t in range(B * S):
        kidx = (t // S) * S + sel[t][sel[t] >= 0].long()
        assert (qi[t] @ ki[kidx].T).abs().min() > 1e-4
    h = 1e-6
    rng = np.random.default_rng(0)
    for name, ana in (("qi", dqi), ("ki", dki), ("w", dw)):
        t = inst[name]
        flat = t.view(-1)
        picks = rng.choice(flat.numel(), size=min(60, flat.numel()), replace=False)
        for e in picks:
            x0 = float(flat[e])
            flat[e] = x0 + h
            up = _total_loss(inst)
            flat[e] = x0 - h
            dn = _total_loss(inst)
            flat[e] = x0
            fd = (up - dn) / (2 * h)
            a = float(ana.reshape(-1)[e])
            assert abs(fd - a) <= 1e-6 * max(1.0, abs(a)), f"d{name}[{e}]: {a} vs fd {fd}"


def _torch_reference(inst):
    """Loss and gradients from torch's softmax / log_softmax / kl_div and autograd,
    for statistics consistent with the selected keys."""
    qi = inst["qi"].clone().requires_grad_(True)
    ki = inst["ki"].clone().requires_grad_(True)
    w = inst["w"].clone().requires_grad_(True)
    B, S = inst["batch"], inst["max_seqlen_q"]
    G, Ni = inst["n_main"], inst["n_idx"]
    sel = inst["sparse_indices"]
    total = 0.0
    losses = []
    for t in range(B * S):
        b = t // S
        s = sel[t][sel[t] >= 0].long()
        kidx = (b * S + s)
        Si = qi.reshape(B * S, Ni, -1)[t] @ ki.reshape(B * S, -1)[kidx].T          # [Ni, n]
        I = w.reshape(B * S, Ni)[t] @ torch.relu(Si)
        x = inst["q"].reshape(B * S, G, -1)[t] @ inst["k"].reshape(B * S, -1)[kidx].T
        x = x + inst["q_rope"].reshape(B * S, G, -1)[t] @ inst["k_rope"].reshape(B * S, -1)[kidx].T
        p = torch.softmax(inst["scale"] * x, dim=1).mean(0)
        lt = torch.nn.functional.kl_div(torch.log_softmax(I, 0), p, reduction="sum")
        losses.append(float(lt.detach()))
        total = total + lt
    total.backward()
    return np.array(losses), qi.grad.numpy(), ki.grad.numpy(), w.grad.numpy()


def _consistent_stats(inst):
    """softmax_max / softmax_sum of each (row, head) over the selected keys."""
    B, S, G = inst["batch"], inst["max_seqlen_q"], inst["n_main"]
    sel = inst["sparse_indices"]
    mx = torch.zeros(B * S, G, dtype=torch.float64)
    sm = torch.zeros(B * S, G, dtype=torch.float64)
    for t in range(B * S):
        b = t // S
        kidx = b * S + sel[t][sel[t] >= 0].long()
        x = inst["q"].reshape(B * S, G, -1)[t] @ inst["k"].reshape(B * S, -1)[kidx].T
        x = inst["scale"] * (x + inst["q_rope"].reshape(B * S, G, -1)[t] @
                             inst["k_rope"].reshape(B * S, -1)[kidx].T)
        mx[t] = x.max(1).values
        sm[t] = torch.exp(x - mx[t].unsqueeze(1)).sum(1)
    # the statistics are fp32 inputs: keep the values they round to consistent by
    # rounding the max first and recomputing the sum from it
    mx32 = mx.to(torch.float32)
    for t in range(B * S):
        b = t // S
        kidx = b * S + sel[t][sel[t] >= 0].long()
        x = inst["q"].reshape(B * S, G, -1)[t] @ inst["k"].reshape(B * S, -1)[kidx].T
        x = inst["scale"] * (x + inst["q_rope"].reshape(B * S, G, -1)[t] @
                             inst["k_rope"].reshape(B * S, -1)[kidx].T)
        sm[t] = torch.exp(x - mx32[t].to(torch.float64).unsqueeze(1)).sum(1)
    return mx32.contiguous(), sm.to(torch.float32).contiguous()


def pin_matches_torch_library():
    inst = _small(2)
    inst["softmax_max"], inst["softmax_sum"] = _consistent_stats(inst)
    loss, dqi, dki, dw = grad.Bound(inst).backward(nthreads=3)
    rl, rqi, rki, rw = _torch_reference(inst)
    # the fp32 softmax_sum rounds the normalisation (relative 2^-24 per head)
    assert np.allclose(loss, rl, rtol=1e-6, atol=1e-7), "loss"
    for name, a, r in (("d_qi", dqi, rqi), ("d_ki", dki, rki), ("d_w", dw, rw)):
        r = r.reshape(a.shape)
        assert np.allclose(a, r, rtol=1e-5, atol=1e-6 * max(1.0, np.abs(r).max())), name


def pin_kl_direction_is_log2():
    # two selected keys with equal index scores (qi = 0) and a target of (1, 0):
    # KL(p || pi) = log 2 (the reverse direction would be about 25)
    inst = _small(3, batch=1, s1=2, n_main=1, d_rope=0, topk=2)
    inst["q_rope"] = inst["k_rope"] = None
    inst["qi"].zero_()
    inst["q"].zero_()
    inst["q"][0, 1, 0, 0] = 1.0
    inst["k"][0, :, 0, :] = 0.0
    inst["k"][0, 0, 0, 0] = 50.0 / inst["scale"]          # key 0: logit 50, key 1: logit 0
    inst["sparse_indices"] = torch.tensor([[0, -1], [0, 1]], dtype=torch.int32)
    loss, dqi, dki, dw = grad.Bound(inst).backward(nthreads=1)
    assert loss[0] == 0.0                                  # one key: p = pi = 1
    assert abs(loss[1] - math.log(2.0)) <= 1e-12, loss[1]
    assert not dqi.any() and not dki.any() and not dw.any()   # qi = 0: every S is 0


def pin_uniform_gives_zero():
    # w = 0 makes every index score 0 (uniform pi); q = 0 makes every main logit 0
    # (uniform p): no loss, no gradient
    inst = _small(4)
    inst["w"].zero_()
    inst["q"].zero_()
    inst["q_rope"].zero_()
    loss, dqi, dki, dw = grad.Bound(inst).backward(nthreads=2)
    assert np.abs(loss).max() <= 1e-14
    assert np.abs(dqi).max() == 0 and np.abs(dki).max() == 0
    assert np.abs(dw).max() <= 1e-13


def pin_single_key_rows():
    # row 0 of every sequence selects only key 0: p = pi = 1
    inst = _small(5)
    loss, dqi, dki, dw = grad.Bound(inst).backward(nthreads=2)
    S = inst["max_seqlen_q"]
    for b in range(inst["batch"]):
        t = b * S
        assert (inst["sparse_indices"][t] >= 0).sum() == 1
        assert loss[t] == 0.0 and not dw[t].any() and not dqi[t].any()


def pin_per_head_statistics():
    inst = _small(6)
    base = grad.Bound(inst).backward(nthreads=2)[0]
    # the same factor on every head's sum and the same shift of every max cancel
    # in the L1 normalisation
    # (x 8 is exact in fp32; the shift rounds each fp32 max by up to 2^-22 * 2.5,
    # which moves the heads' weights by about 1e-6)
    inst2 = dict(inst, softmax_sum=(inst["softmax_sum"] * 8.0).contiguous(),
                 softmax_max=(inst["softmax_max"] + 1.5).contiguous())
    assert np.allclose(grad.Bound(inst2).backward(nthreads=2)[0], base, rtol=1e-5, atol=1e-9)
    # a head whose sum is huge drops out of the target: it equals the target of
    # the other heads alone
    G = inst["n_main"]
    ssum = inst["softmax_sum"].clone()
    ssum[:, G - 1] = 1e30
    big = grad.Bound(dict(inst, softmax_sum=ssum.contiguous())).backward(nthreads=2)[0]
    fewer = dict(inst, n_main=G - 1,
                 q=inst["q"][:, :, :G - 1].contiguous(),
                 q_rope=inst["q_rope"][:, :, :G - 1].contiguous(),
                 softmax_max=inst["softmax_max"][:, :G - 1].contiguous(),
                 softmax_sum=inst["softmax_sum"][:, :G - 1].contiguous())
    ref = grad.Bound(fewer).backward(nthreads=2)[0]
    assert np.allclose(big, ref, rtol=1e-9, atol=1e-12)
    assert not np.allclose(big, base, rtol=1e-6)


def pin_padding_entries_skipped():
    inst = _small(7)
    sel = inst["sparse_indices"]
    n = (sel >= 0).sum(1)
    # interleave the valid entries with -1 entries (topk doubled)
    wide = torch.full((sel.shape[0], 2 * sel.shape[1]), -1, dtype=torch.int32)
    wide[:, 1::2] = sel
    a = grad.Bound(inst).backward(nthreads=2)
    b = grad.Bound(dict(inst, topk=2 * inst["topk"], sparse_indices=wide.contiguous())).backward(
        nthreads=2)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert n.min() >= 1


def pin_tnd_equals_bsnd():
    inst = _small(8)
    B, S = inst["batch"], inst["max_seqlen_q"]
    tnd = dict(inst, layout="TND",
               cu_seqlens_q=torch.tensor([S * (b + 1) for b in range(B)], dtype=torch.int32),
               cu_seqlens_k=torch.tensor([S * (b + 1) for b in range(B)], dtype=torch.int32))
    for n in ("q", "k", "q_rope", "k_rope", "qi", "ki", "w"):
        tnd[n] = inst[n].reshape(B * S, *inst[n].shape[2:]).contiguous()
    a = grad.Bound(inst).backward(nthreads=2)
    b = grad.Bound(tnd).backward(nthreads=2)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def pin_thread_count_invariance():
    inst = _small(9)
    a = grad.Bound(inst).backward(nthreads=1)
    b = grad.Bound(inst).backward(nthreads=7)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def pin_homogeneity():
    # I is positively homogeneous of degree 1 in qi, in ki and in w separately
    # (ReLU(c x) = c ReLU(x) for c >= 0), so Euler's identity gives
    # <d_qi, qi> = <d_ki, ki> = <d_w, w> = sum over rows and entries of dI * I
    inst = _small(10)
    loss, dqi, dki, dw = grad.Bound(inst).backward(nthreads=2)
    a = float((dqi * inst["qi"].numpy().reshape(dqi.shape)).sum())
    b = float((dki * inst["ki"].numpy().reshape(dki.shape)).sum())
    c = float((dw * inst["w"].numpy().reshape(dw.shape)).sum())
    assert abs(a) > 1e-3
    assert abs(a - b) <= 1e-9 * abs(a) and abs(a - c) <= 1e-9 * abs(a), (a, b, c)


def pin_rows_subset_matches():
    inst = _small(11)
    ob = grad.Bound(inst)
    loss, dqi, dki, dw = ob.backward(nthreads=2)
    rows = [0, 5, 21, 39]
    l2, q2, w2 = ob.backward_rows(rows)
    assert np.array_equal(l2, loss[rows]) and np.array_equal(q2, dqi[rows])
    assert np.array_equal(w2, dw[rows])


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
