"""GPU-vs-oracle comparison of Lightning Indexer outputs, row by row.

Rules (per query row, with n = min(topk, |visible|)):
  * structure: exactly n valid entries forming the prefix [0, n); the tail holds
    index -1 and value -inf exactly; no duplicate index; every index visible
    (visible keys are 0 .. |V|-1 under both mask modes);
  * values: every valid (s, v) satisfies |v - I(s)| <= TOL * max(1, |I(s)|), with
    I(s) the oracle's fp64 score of key s and TOL = 1e-2 (bf16 / fp8 inputs,
    fp32 accumulation);
  * index set: equal to the oracle's, except for swaps between keys whose oracle
    scores lie within TOL * max(1, |v_k|) of v_k, the oracle's k-th score.
The order inside the valid prefix is not compared (the oracle sorts by score,
the GPU writes ascending key order).
"""
from __future__ import annotations

import dataclasses

import numpy as np

TOL = 1e-2


@dataclasses.dataclass
class Report:
    rows: int = 0
    max_abs: float = 0.0
    max_rel: float = 0.0
    swaps: int = 0

    def merge(self, o: "Report"):
        self.rows += o.rows
        self.max_abs = max(self.max_abs, o.max_abs)
        self.max_rel = max(self.max_rel, o.max_rel)
        self.swaps += o.swaps


def check_row(g_idx: np.ndarray, g_val, o_idx: np.ndarray, o_val: np.ndarray, n_visible: int,
              score_of, where: str = "", tol: float = TOL) -> Report:
    """score_of(s) -> oracle fp64 score of key s (only called for swapped keys)."""
    topk = o_idx.shape[0]
    n = min(topk, n_visible)
    rep = Report(rows=1)
    gv = int((g_idx >= 0).sum())
    assert gv == n, f"{where}: {gv} valid GPU entries, expected {n}"
    assert (g_idx[:n] >= 0).all() and (g_idx[n:] == -1).all(), f"{where}: valid part not a prefix"
    assert (g_idx[:n] < n_visible).all(), f"{where}: index outside the visible window"
    assert len(set(g_idx[:n].tolist())) == n, f"{where}: duplicate index"
    if g_val is not None:
        tail = g_val[n:]
        assert np.all(np.isneginf(tail)), f"{where}: value padding is not -inf"
    o_set = dict(zip(o_idx[:n].tolist(), o_val[:n].astype(np.float64).tolist()))
    g_keys = g_idx[:n].tolist()
    g_set = set(g_keys)
    extra = [s for s in g_keys if s not in o_set]
    missing = [s for s in o_set if s not in g_set]
    ref = dict(o_set)
    for s in extra:
        ref[s] = float(score_of(s))
    if g_val is not None:
        gvv = g_val[:n].astype(np.float64)
        rv = np.array([ref[s] for s in g_keys])
        err = np.abs(gvv - rv)
        bound = tol * np.maximum(1.0, np.abs(rv))
        bad = err > bound
        assert not bad.any(), (f"{where}: value error {err[bad].max():.3g} at key "
                               f"{np.array(g_keys)[bad][0]} (score {rv[bad][0]:.6g})")
        if n:
            rep.max_abs = float(err.max())
            rep.max_rel = float((err / np.maximum(1.0, np.abs(rv))).max())
    if extra or missing:
        assert n == topk, f"{where}: set differs although every visible key fits"
        vk = min(o_set.values())
        band = tol * max(1.0, abs(vk))
        for s in extra + missing:
            assert abs(ref[s] - vk) <= band, (f"{where}: key {s} (score {ref[s]:.6g}) swapped, "
                                              f"k-th score {vk:.6g}")
        rep.swaps = len(extra)
    return rep


def check_rows(g_idx, g_val, o_idx, o_val, rows, oracle_bound, tol: float = TOL) -> Report:
    """g_* / o_* are [len(rows), topk] arrays for the listed global rows."""
    rep = Report()
    for j, row in enumerate(rows):
        b, i = oracle_bound.row_coords(int(row))
        nv = oracle_bound.visible_count(b, i)
        r = check_row(g_idx[j], None if g_val is None else g_val[j], o_idx[j], o_val[j], nv,
                      lambda s, b=b, i=i: oracle_bound.score(b, i, s), where=f"row {row}", tol=tol)
        rep.merge(r)
    return rep
