"""HIP backward of the indexer fused with its KL loss (li_grad_kl) against the
CPU oracle (oracle/li_grad_oracle.c), through the C ABI (needs an MI355X).

Tolerance (fp32 arithmetic on 16-bit inputs; the oracle is fp64): scores and
logits come from MFMA with exact 16-bit products and fp32 sums, exp / log are
the hardware's fp32 ones (a few ulp), and dS enters the gradient contractions as
a 16-bit high part plus a 16-bit low part (about 2^-16 of relative error), so
each output element is within 2e-3 * |ref| + 2e-4 * rms(ref tensor) of the
oracle; the scalar loss within 1e-4 relative.  The one decision floating point
takes, the ReLU's gate [S > 0], is taken on an fp32 sum by the GPU and on an
fp64 sum by the oracle: for (row, head, key) triples whose |S| is within the
fp32 sum's rounding band of zero either side is right, and the bound of the
gradient elements they touch grows by the most such a flip can move them
(kink_allowance).  d_k_index is summed with fp32 atomics: only its rounding
order varies between runs.
"""
from __future__ import annotations

import dataclasses
import os
import sys

import numpy as np
import pytest
import torch

from oracle import grad as grad_oracle
from score_top_token_amd import binding, synth

pytestmark = pytest.mark.gpu

try:
    THREADS = min(16, len(os.sched_getaffinity(0)))
except AttributeError:
    THREADS = min(16, os.cpu_count() or 1)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _to_dev(inst, dev):
    return {n: (inst[n].to(dev) if isinstance(inst.get(n), torch.Tensor) else None)
            for n in binding.GRAD_INPUTS}


def _run(inst):
    _say(f"[gpu] grad {inst['name']} seed={inst['seed']} B={inst['batch']} {inst['layout']} "
         f"rows={sum(inst['seqlens'])} G={inst['n_main']} rope={inst['d_rope']} "
         f"Ni={inst['n_idx']} topk={inst['topk']} {inst['qi'].dtype} w={inst['w'].dtype}")
    dev = torch.device("cuda")
    p = binding.grad_problem_for(inst)
    st, wsb = binding.li_grad_workspace_size(p)
    assert st == 0
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    loss, dq, dk, dw = binding.lightning_indexer_grad_kl(p, _to_dev(inst, dev), workspace=ws)
    torch.cuda.synchronize()
    rows = sum(inst["seqlens"])
    loss_rows = ws[:4 * rows].view(torch.float32).cpu().numpy().astype(np.float64)
    dq = dq.reshape(rows, inst["n_idx"], inst["d_idx"])
    return (float(loss.item()), loss_rows, dq.cpu().numpy().astype(np.float64),
            dk.cpu().numpy().astype(np.float64), dw.cpu().numpy().astype(np.float64))


def _close(name, got, ref, rel=2e-3, floor=2e-4, extra=None):
    shape = np.asarray(ref).shape
    got, ref = np.asarray(got).reshape(-1), np.asarray(ref).reshape(-1)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = np.abs(got - ref)
    bound = rel * np.abs(ref) + floor * max(rms, 1e-30)
    if extra is not None:
        bound = bound + np.asarray(extra).reshape(-1)
    ratio = err / np.maximum(bound, 1e-300)
    worst = float(ratio.max()) if ref.size else 0.0
    where = np.unravel_index(int(ratio.argmax()), shape) if ref.size else ()
    _say(f"    {name}: max |d| {err.max() if ref.size else 0:.3g}, rms(ref) {rms:.3g}, "
         f"worst err/bound {worst:.3g} at {tuple(int(x) for x in where)}")
    assert (err <= bound).all(), f"{name}: {int((err > bound).sum())} elements off"


def kink_allowance(inst, rows=None, band=2e-6):
    """Where the GPU (fp32 MFMA sums) and the oracle (fp64) may take the ReLU's
    gate [S > 0] differently: a (row, head, key) whose |S| lies within
    band * sum_d |qi_d ki_d| of zero (four times the bound of the fp32 sum's rounding,
    8 roundings of 2^-24 over the 8 k-steps of the MFMA chain).  Such
    a flip moves d_q_index[t, h] by up to |dI w_h| |ki| and d_k_index[key] by up
    to |dI w_h| |qi[t, h]|, with |dI| <= 1.  Returns the allowances (d_q for the
    listed rows, d_k for every key; d_w needs none: ReLU is continuous there) and
    the number of ambiguous triples."""
    B, Ni = inst["batch"], inst["n_idx"]
    qi = inst["qi"].to(torch.float64).reshape(-1, Ni, 128)
    ki = inst["ki"].to(torch.float64).reshape(-1, 128)
    w = inst["w"].to(torch.float64).reshape(-1, Ni)
    sel = inst["sparse_indices"].long()
    lens = inst["seqlens"]
    starts = np.concatenate([[0], np.cumsum(lens)])
    row_b = np.repeat(np.arange(B), lens)
    rows = np.arange(qi.shape[0]) if rows is None else np.asarray(rows)
    aq = torch.zeros(len(rows), Ni, 128, dtype=torch.float64)
    ak = torch.zeros(ki.shape[0], 128, dtype=torch.float64)
    n_amb = 0
    for c0 in range(0, len(rows), 128):
        rr = torch.as_tensor(rows[c0:c0 + 128])
        sl = sel[rr]
        ok = sl >= 0
        tok = torch.as_tensor(starts[row_b[rr.numpy()]]).unsqueeze(1) + sl.clamp(min=0)
        kg = ki[tok]                                            # [r, K, 128]
        S = torch.einsum("rhd,rkd->rhk", qi[rr], kg)
        mag = torch.einsum("rhd,rkd->rhk", qi[rr].abs(), kg.abs())
        amb = (S.abs() <= band * mag) & ok.unsqueeze(1)         # [r, h, K]
        if not amb.any():
            continue
        n_amb += int(amb.sum())
        wa = w[rr].abs().unsqueeze(2) * amb                     # |w_h| on the ambiguous entries
        aq[c0:c0 + len(rr)] = torch.einsum("rhk,rkd->rhd", wa, kg.abs())
        contrib = torch.einsum("rhk,rhd->rkd", wa, qi[rr].abs())
        ak.index_add_(0, tok.reshape(-1), contrib.reshape(-1, 128))
    return aq.numpy(), ak.numpy(), n_amb


def compare_full(inst):
    loss, loss_rows, dq, dk, dw = _run(inst)
    _say(f"    oracle ({THREADS} threads)")
    rl, rq, rk, rw = grad_oracle.Bound(inst).backward(nthreads=THREADS)
    aq, ak, n_amb = kink_allowance(inst)
    _say(f"    {n_amb} (row, head, key) scores within the fp32 band of the ReLU kink")
    _close("loss per row", loss_rows, rl)
    assert abs(loss - rl.sum()) <= 1e-4 * max(1.0, abs(rl.sum())), (loss, rl.sum())
    _close("d_q_index", dq, rq, extra=aq)
    _close("d_k_index", dk, rk, extra=ak)
    _close("d_w", dw, rw)


CASES = {
    "tiny_s0": ("grad_tiny", 0, {}),
    "tiny_s1": ("grad_tiny", 1, {}),
    "tnd_no_rope": (None, 2, dict(layout="TND", batch=3, fixed_lengths=[100, 37, 300], n_main=8,
                                  d_rope=0, n_idx=16, topk=64)),
    "fp16_w32_odd_heads": (None, 3, dict(batch=2, s1=150, n_main=20, n_idx=40, topk=100,
                                         dtype="fp16", w_dtype="fp32")),
    "one_head_each": (None, 4, dict(batch=1, s1=70, n_main=1, n_idx=1, topk=7, w_scale=1.0)),
    "mid": ("grad_mid", 5, {}),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_grad_case(name):
    preset, seed, over = CASES[name]
    base = synth.GRAD_PRESETS[preset] if preset else synth.GradSpec()
    spec = dataclasses.replace(base, name=name, **over)
    compare_full(synth.make_grad(spec, seed))


def test_grad_train_shape():
    """The training-shaped workload (64 index heads, top-2048 over a 4096-token
    causal sequence, 32 main heads with rope): sampled rows against the oracle,
    and for every row and key Euler's identity of the degree-1 homogeneous score
    (<d_q_index, q_index> = <d_k_index, k_index> = <d_w, w>)."""
    inst = synth.make_grad("grad_train", 0)
    loss, loss_rows, dq, dk, dw = _run(inst)
    rows = np.unique(np.concatenate([[0, 1, 2047, 2048, 4095],
                                     np.random.default_rng(0).integers(0, 4096, 27)]))
    _say(f"    oracle on {len(rows)} rows")
    rl, rq, rw = grad_oracle.Bound(inst).backward_rows(rows)
    aq, _, n_amb = kink_allowance(inst, rows)
    _say(f"    {n_amb} (row, head, key) scores within the fp32 band of the ReLU kink")
    _close("loss per row", loss_rows[rows], rl)
    _close("d_q_index", dq[rows], rq, extra=aq)
    _close("d_w", dw[rows], rw)
    qi = inst["qi"].to(torch.float64).numpy()
    ki = inst["ki"].to(torch.float64).numpy()
    w = inst["w"].to(torch.float64).numpy()
    a = float((dq.reshape(qi.shape) * qi).sum())
    b = float((dk.reshape(ki.shape[0] * ki.shape[1], -1) * ki.reshape(-1, ki.shape[-1])).sum())
    c = float((dw.reshape(w.shape) * w).sum())
    _say(f"    <dq,q> {a:.6g}  <dk,k> {b:.6g}  <dw,w> {c:.6g}")
    assert abs(a - c) <= 1e-3 * abs(c) and abs(b - c) <= 1e-3 * abs(c)
    assert np.isfinite(loss) and loss > 0
