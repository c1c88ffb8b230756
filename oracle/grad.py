"""Python access to the plain CPU oracle of the indexer backward + KL loss
(oracle/li_grad_oracle.c).

TEST INFRASTRUCTURE ONLY: tests/, the smoke check and the bench's CPU-baseline
leg use it to check the HIP library against.  The product package never imports it.

Instances come from score_top_token_amd.synth.make_grad (CPU tensors); the
outputs are fp64 numpy arrays: per-row loss [rows], d_qi [rows, Ni, Di],
d_ki [keys, Di], d_w [rows, Ni].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "li_grad_oracle.c")
_LIB = os.path.join(_HERE, "libgradoracle.so")

_DTYPE = {torch.bfloat16: 0, torch.float32: 2, torch.float16: 3, torch.float64: 4}


class _Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("s1", ctypes.c_int32), ("s2", ctypes.c_int32),
        ("layout", ctypes.c_int32), ("n_main", ctypes.c_int32), ("d_main", ctypes.c_int32),
        ("d_rope", ctypes.c_int32), ("n_idx", ctypes.c_int32), ("d_idx", ctypes.c_int32),
        ("topk", ctypes.c_int32), ("dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32),
        ("scale", ctypes.c_double),
    ]


class _Inputs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "q", "k", "q_rope", "k_rope", "qi", "ki", "w", "sparse_indices", "softmax_max",
        "softmax_sum", "cu_seqlens_q", "cu_seqlens_k")]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C11, -O2, POSIX threads)."""
    hdr = os.path.join(_HERE, "li_grad_oracle.h")
    newest = max(os.path.getmtime(_SRC), os.path.getmtime(hdr))
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < newest:
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-shared", "-fPIC", "-o", tmp,
                               _SRC, "-lpthread", "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load(path):
    L = ctypes.CDLL(path)
    P, I = ctypes.POINTER(_Problem), ctypes.POINTER(_Inputs)
    vp = ctypes.c_void_p
    L.liog_backward.argtypes = [P, I, vp, vp, vp, vp, ctypes.c_int]
    L.liog_backward.restype = ctypes.c_int
    L.liog_backward_rows.argtypes = [P, I, vp, ctypes.c_int64, vp, vp, vp]
    L.liog_backward_rows.restype = ctypes.c_int
    L.liog_num_rows.argtypes = [P, I]
    L.liog_num_rows.restype = ctypes.c_int64
    L.liog_num_keys.argtypes = [P, I]
    L.liog_num_keys.restype = ctypes.c_int64
    return L


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = _load(_LIB)
    return _lib


class use_library:
    """Routes the calls through another build of li_grad_oracle.c (the mutation tests)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _lib
        _lib = _load(self.path)
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved


def _ptr(t):
    if t is None:
        return None
    assert t.device.type == "cpu" and t.is_contiguous()
    return t.data_ptr()


class Bound:
    """A backward instance marshalled for the C oracle (keeps the tensors alive)."""

    def __init__(self, inst: dict):
        self.inst = inst
        names = ("q", "k", "q_rope", "k_rope", "qi", "ki", "w", "sparse_indices",
                 "softmax_max", "softmax_sum", "cu_seqlens_q", "cu_seqlens_k")
        self._keep = [inst.get(n) for n in names]
        dt = _DTYPE[inst["qi"].dtype]
        for n in ("q", "k", "ki"):
            assert _DTYPE[inst[n].dtype] == dt, n
        self.p = _Problem(
            batch=inst["batch"], s1=inst["max_seqlen_q"] if inst["layout"] == "BSND" else 0,
            s2=inst["max_seqlen_k"] if inst["layout"] == "BSND" else 0,
            layout=0 if inst["layout"] == "BSND" else 1, n_main=inst["n_main"],
            d_main=inst["d_main"], d_rope=inst["d_rope"], n_idx=inst["n_idx"],
            d_idx=inst["d_idx"], topk=inst["topk"], dtype=dt, w_dtype=_DTYPE[inst["w"].dtype],
            scale=float(inst["scale"]))
        self.i = _Inputs(**{n: _ptr(inst.get(n)) for n in names})

    @property
    def num_rows(self) -> int:
        return int(lib().liog_num_rows(ctypes.byref(self.p), ctypes.byref(self.i)))

    @property
    def num_keys(self) -> int:
        return int(lib().liog_num_keys(ctypes.byref(self.p), ctypes.byref(self.i)))

    def backward(self, nthreads=None):
        """Returns (loss_rows [rows], d_qi [rows, Ni, Di], d_ki [keys, Di], d_w [rows, Ni])."""
        rows, keys = self.num_rows, self.num_keys
        Ni, Di = self.inst["n_idx"], self.inst["d_idx"]
        loss = np.empty(rows)
        dqi = np.empty((rows, Ni, Di))
        dki = np.empty((keys, Di))
        dw = np.empty((rows, Ni))
        if nthreads is None:
            nthreads = os.cpu_count() or 1
        rc = lib().liog_backward(ctypes.byref(self.p), ctypes.byref(self.i), loss.ctypes.data,
                                 dqi.ctypes.data, dki.ctypes.data, dw.ctypes.data, int(nthreads))
        if rc != 0:
            raise ValueError("gradient oracle rejected the problem")
        return loss, dqi, dki, dw

    def backward_rows(self, rows):
        """(loss [n], d_qi [n, Ni, Di], d_w [n, Ni]) of the listed rows (no d_ki)."""
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        Ni, Di = self.inst["n_idx"], self.inst["d_idx"]
        loss = np.empty(len(rows))
        dqi = np.empty((len(rows), Ni, Di))
        dw = np.empty((len(rows), Ni))
        rc = lib().liog_backward_rows(ctypes.byref(self.p), ctypes.byref(self.i), rows.ctypes.data,
                                      len(rows), loss.ctypes.data, dqi.ctypes.data, dw.ctypes.data)
        if rc != 0:
            raise ValueError("gradient oracle rejected the rows")
        return loss, dqi, dw
