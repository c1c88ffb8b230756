"""Python access to the plain CPU oracle (oracle/li_oracle.c).

TEST INFRASTRUCTURE ONLY: tests/, the smoke check and the bench's CPU-baseline
leg use it to check the HIP library against.  The product package never imports it.

`build()` compiles li_oracle.c with gcc into oracle/liboracle.so; the other
functions take a problem instance as produced by score_top_token_amd.synth.make
(CPU tensors) and call the C code through ctypes.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "li_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_LAYOUT = {"BSND": 0, "TND": 1, "PA_BSND": 2}
_DTYPE = {"bf16": 0, "fp8": 1, "fp32": 2, "fp16": 3}


class _Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("s1", ctypes.c_int32), ("s2", ctypes.c_int32),
        ("n1", ctypes.c_int32), ("d", ctypes.c_int32), ("topk", ctypes.c_int32),
        ("layout_q", ctypes.c_int32), ("layout_k", ctypes.c_int32),
        ("mask_mode", ctypes.c_int32), ("qk_dtype", ctypes.c_int32),
        ("w_dtype", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32), ("k_block_stride", ctypes.c_int64),
        ("cmp_ratio", ctypes.c_int32),
    ]


class _Inputs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("w", ctypes.c_void_p),
        ("q_descale", ctypes.c_void_p), ("k_descale", ctypes.c_void_p),
        ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
        ("seqused_k", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
        ("cmp_residual_k", ctypes.c_void_p), ("output_idx_offset", ctypes.c_void_p),
    ]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C11, -O2, POSIX threads)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-shared", "-fPIC", "-o", tmp,
                               _SRC, "-lpthread", "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _load(_LIB)
    return _lib


@contextlib.contextmanager
def use_library(path: str):
    """Temporarily route every oracle call through another build of li_oracle.c
    (the mutation tests load copies with planted mistakes this way)."""
    global _lib
    saved = _lib
    _lib = _load(path)
    try:
        yield _lib
    finally:
        _lib = saved


def _load(path: str):
    if True:
        L = ctypes.CDLL(path)
        L.lio_forward.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(_Inputs),
                                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_int]
        L.lio_forward.restype = ctypes.c_int
        L.lio_score.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(_Inputs), ctypes.c_int,
                                ctypes.c_int, ctypes.c_int]
        L.lio_score.restype = ctypes.c_double
        L.lio_visible_count.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(_Inputs),
                                        ctypes.c_int, ctypes.c_int]
        L.lio_visible_count.restype = ctypes.c_int
        L.lio_num_rows.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(_Inputs)]
        L.lio_num_rows.restype = ctypes.c_int64
        L.lio_row_coords.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(_Inputs),
                                     ctypes.c_int64, ctypes.POINTER(ctypes.c_int),
                                     ctypes.POINTER(ctypes.c_int)]
        L.lio_row_coords.restype = ctypes.c_int
        L.lio_decode.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64]
        L.lio_decode.restype = ctypes.c_double
        return L


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    assert t.device.type == "cpu"
    return t.data_ptr()


class Bound:
    """A problem instance marshalled for the C oracle (keeps the tensors alive)."""

    def __init__(self, inst: dict):
        self.inst = inst
        q, k, w = inst["q"], inst["k"], inst["w"]
        assert q.is_contiguous() and w.is_contiguous()
        kstride = 0
        if inst["layout_k"] == "PA_BSND":
            kstride = k.stride(0)
            assert k.stride(1) == k.shape[-1] and k.stride(3) == 1
        else:
            assert k.is_contiguous()
        s1 = inst["max_seqlen_q"] if inst["layout_q"] != "TND" else 0
        s2 = inst["max_seqlen_k"] if inst["layout_k"] == "BSND" else 0
        self.p = _Problem(
            batch=inst["batch"], s1=s1, s2=s2, n1=inst["n1"], d=inst["d"], topk=inst["topk"],
            layout_q=_LAYOUT[inst["layout_q"]], layout_k=_LAYOUT[inst["layout_k"]],
            mask_mode=inst["mask_mode"], qk_dtype=_DTYPE[inst["qk_dtype"]],
            w_dtype=_DTYPE[inst["w_dtype"]], block_size=inst.get("block_size", 0) or 0,
            max_blocks_per_seq=inst.get("max_blocks_per_seq", 0) or 0, k_block_stride=kstride,
            cmp_ratio=inst.get("cmp_ratio", 1) or 1)
        self._keep = [inst.get(n) for n in ("q", "k", "w", "q_descale", "k_descale",
                                            "cu_seqlens_q", "cu_seqlens_k", "seqused_k",
                                            "block_table", "cmp_residual_k",
                                            "output_idx_offset")]
        for t in self._keep:
            if t is not None:
                assert t.device.type == "cpu"
        self.i = _Inputs(
            q=_ptr(q), k=_ptr(k), w=_ptr(w), q_descale=_ptr(inst.get("q_descale")),
            k_descale=_ptr(inst.get("k_descale")), cu_seqlens_q=_ptr(inst.get("cu_seqlens_q")),
            cu_seqlens_k=_ptr(inst.get("cu_seqlens_k")), seqused_k=_ptr(inst.get("seqused_k")),
            block_table=_ptr(inst.get("block_table")),
            cmp_residual_k=_ptr(inst.get("cmp_residual_k")),
            output_idx_offset=_ptr(inst.get("output_idx_offset")))

    @property
    def num_rows(self) -> int:
        return int(lib().lio_num_rows(ctypes.byref(self.p), ctypes.byref(self.i)))

    def forward(self, rows: Optional[Sequence[int]] = None, nthreads: Optional[int] = None):
        """Returns (indices int32 [nrows, topk], values float32 [nrows, topk])."""
        topk = self.inst["topk"]
        if rows is None:
            nrows = self.num_rows
            rows_arr = None
        else:
            rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
            nrows = rows_arr.shape[0]
        idx = np.empty((nrows, topk), dtype=np.int32)
        val = np.empty((nrows, topk), dtype=np.float32)
        if nthreads is None:
            nthreads = os.cpu_count() or 1
        rc = lib().lio_forward(ctypes.byref(self.p), ctypes.byref(self.i),
                               None if rows_arr is None else rows_arr.ctypes.data, nrows,
                               idx.ctypes.data, val.ctypes.data, int(nthreads))
        if rc != 0:
            raise ValueError("oracle rejected the problem")
        return idx, val

    def score(self, b: int, i: int, s: int) -> float:
        return float(lib().lio_score(ctypes.byref(self.p), ctypes.byref(self.i), b, i, s))

    def visible_count(self, b: int, i: int) -> int:
        return int(lib().lio_visible_count(ctypes.byref(self.p), ctypes.byref(self.i), b, i))

    def row_coords(self, row: int):
        b, i = ctypes.c_int(), ctypes.c_int()
        rc = lib().lio_row_coords(ctypes.byref(self.p), ctypes.byref(self.i), int(row),
                                  ctypes.byref(b), ctypes.byref(i))
        if rc != 0:
            raise IndexError(row)
        return b.value, i.value


def decode(dtype: str, codes: torch.Tensor) -> np.ndarray:
    """Exact fp64 values of a flat tensor of element codes, via the oracle's decoder."""
    c = codes.contiguous().reshape(-1)
    L = lib()
    return np.array([L.lio_decode(_DTYPE[dtype], c.data_ptr(), j) for j in range(c.numel())],
                    dtype=np.float64)
