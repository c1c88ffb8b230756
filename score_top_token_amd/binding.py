"""ctypes binding of the C ABI in include/li.h.

Argument marshalling only: every step of the computation runs in the HIP
library.  The library must have been built (score_top_token_amd.build or
__graft_entry__.build()); loading fails loudly otherwise -- there is no fallback.

Low level: li_metadata_size, li_workspace_size, li_metadata, li_forward and
li_status_str take the same arguments as the C functions (device pointers as
ints, a Problem structure, a raw stream handle).

High level (torch tensors on the GPU, mirroring the lightning_indexer page's
Prototype section): problem_from(...), lightning_indexer_metadata(...) and
lightning_indexer(...).  torch only supplies device memory and the stream.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblightning_indexer.so")

LAYOUT = {"BSND": 0, "TND": 1, "PA_BSND": 2, "PA_BBND": 2}
DTYPE = {torch.bfloat16: 0, torch.float8_e4m3fn: 1, torch.float32: 2, torch.float16: 3}
STATUS = {0: "LI_OK", 1: "LI_ERR_INVALID_ARGUMENT", 2: "LI_ERR_UNSUPPORTED",
          3: "LI_ERR_WORKSPACE_TOO_SMALL", 4: "LI_ERR_HIP", 5: "LI_ERR_METADATA_MISMATCH"}

EXPORTED = ("li_metadata_size", "li_workspace_size", "li_metadata", "li_forward",
            "li_forward_noalloc", "li_gather", "li_grad_workspace_size", "li_grad_kl",
            "li_status_str")


class Problem(ctypes.Structure):
    """Mirror of li_problem."""

    _fields_ = [
        ("batch", ctypes.c_int32), ("max_seqlen_q", ctypes.c_int32),
        ("max_seqlen_k", ctypes.c_int32), ("total_q", ctypes.c_int32),
        ("total_k", ctypes.c_int32), ("num_heads_q", ctypes.c_int32),
        ("num_heads_k", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("topk", ctypes.c_int32), ("layout_q", ctypes.c_int32), ("layout_k", ctypes.c_int32),
        ("mask_mode", ctypes.c_int32), ("qk_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32), ("cmp_ratio", ctypes.c_int32),
        ("k_block_stride", ctypes.c_int64),
    ]


class GradProblem(ctypes.Structure):
    """Mirror of li_grad_problem."""

    _fields_ = [
        ("batch", ctypes.c_int32), ("max_seqlen_q", ctypes.c_int32),
        ("max_seqlen_k", ctypes.c_int32), ("total_q", ctypes.c_int32),
        ("total_k", ctypes.c_int32), ("layout", ctypes.c_int32), ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("rope_dim", ctypes.c_int32),
        ("num_heads_index", ctypes.c_int32), ("head_dim_index", ctypes.c_int32),
        ("topk", ctypes.c_int32), ("dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


class LIError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}")
        self.status = status


_lib = None


def load():
    """Loads the built HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library missing: {LIB_PATH} (build it first)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(Problem)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        L.li_metadata_size.argtypes = [P, ctypes.POINTER(sz)]
        L.li_workspace_size.argtypes = [P, ctypes.POINTER(sz)]
        L.li_metadata.argtypes = [P, vp, vp, vp, vp, vp, sz, vp]
        L.li_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                 vp, vp]
        L.li_forward_noalloc.argtypes = [P] + [vp] * 15
        L.li_gather.argtypes = [P, vp, ctypes.c_int32, ctypes.c_int64, vp, ctypes.c_int32, vp, vp,
                                vp, vp]
        GP = ctypes.POINTER(GradProblem)
        L.li_grad_workspace_size.argtypes = [GP, ctypes.POINTER(sz)]
        L.li_grad_kl.argtypes = [GP] + [vp] * 12 + [vp, sz, vp, vp, vp, vp, vp]
        L.li_status_str.argtypes = [ctypes.c_int]
        L.li_status_str.restype = ctypes.c_char_p
        for n in ("li_metadata_size", "li_workspace_size", "li_metadata", "li_forward",
                  "li_forward_noalloc", "li_gather", "li_grad_workspace_size", "li_grad_kl"):
            getattr(L, n).restype = ctypes.c_int
        _lib = L
    return _lib


# ---------------------------------------------------------------------------
# same-name wrappers of the C entry points
# ---------------------------------------------------------------------------

def li_metadata_size(p: Problem) -> tuple[int, int]:
    n = ctypes.c_size_t(0)
    st = load().li_metadata_size(ctypes.byref(p), ctypes.byref(n))
    return st, n.value


def li_workspace_size(p: Problem) -> tuple[int, int]:
    n = ctypes.c_size_t(0)
    st = load().li_workspace_size(ctypes.byref(p), ctypes.byref(n))
    return st, n.value


def li_metadata(p: Problem, cu_seqlens_q, cu_seqlens_k, seqused_k, cmp_residual_k, metadata,
                metadata_bytes, stream) -> int:
    return load().li_metadata(ctypes.byref(p), cu_seqlens_q, cu_seqlens_k, seqused_k,
                              cmp_residual_k, metadata, metadata_bytes, stream)


def li_forward(p: Problem, q, k, w, q_descale, k_descale, cu_seqlens_q, cu_seqlens_k, seqused_k,
               cmp_residual_k, block_table, output_idx_offset, metadata, workspace,
               workspace_bytes, sparse_indices, sparse_values, stream) -> int:
    return load().li_forward(ctypes.byref(p), q, k, w, q_descale, k_descale, cu_seqlens_q,
                             cu_seqlens_k, seqused_k, cmp_residual_k, block_table,
                             output_idx_offset, metadata, workspace, workspace_bytes,
                             sparse_indices, sparse_values, stream)


def li_forward_noalloc(p: Problem, q, k, w, q_descale, k_descale, cu_seqlens_q, cu_seqlens_k,
                       seqused_k, cmp_residual_k, block_table, output_idx_offset, metadata,
                       sparse_indices, sparse_values, stream) -> int:
    return load().li_forward_noalloc(ctypes.byref(p), q, k, w, q_descale, k_descale, cu_seqlens_q,
                                     cu_seqlens_k, seqused_k, cmp_residual_k, block_table,
                                     output_idx_offset, metadata, sparse_indices, sparse_values,
                                     stream)


def li_gather(p: Problem, kv, row_bytes, kv_block_stride, sparse_indices, select_block,
              block_table, metadata, out, stream) -> int:
    return load().li_gather(ctypes.byref(p), kv, row_bytes, kv_block_stride, sparse_indices,
                            select_block, block_table, metadata, out, stream)


def li_grad_workspace_size(p: GradProblem) -> tuple[int, int]:
    n = ctypes.c_size_t(0)
    st = load().li_grad_workspace_size(ctypes.byref(p), ctypes.byref(n))
    return st, n.value


def li_grad_kl(p: GradProblem, q, k, q_rope, k_rope, q_index, k_index, w, sparse_indices,
               softmax_max, softmax_sum, cu_seqlens_q, cu_seqlens_k, workspace, workspace_bytes,
               d_q_index, d_k_index, d_w, loss, stream) -> int:
    return load().li_grad_kl(ctypes.byref(p), q, k, q_rope, k_rope, q_index, k_index, w,
                             sparse_indices, softmax_max, softmax_sum, cu_seqlens_q, cu_seqlens_k,
                             workspace, workspace_bytes, d_q_index, d_k_index, d_w, loss, stream)


def li_status_str(status: int) -> str:
    return load().li_status_str(status).decode()


# ---------------------------------------------------------------------------
# torch-facing helpers
# ---------------------------------------------------------------------------

def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _check(st: int, where: str):
    if st != 0:
        raise LIError(st, where)


def problem_from(q: torch.Tensor, k: torch.Tensor, w: torch.Tensor, topk: int, *,
                 layout_q: str = "BSND", layout_k: str = "BSND", mask_mode: int = 0,
                 batch_size: Optional[int] = None, max_seqlen_q: Optional[int] = None,
                 max_seqlen_k: Optional[int] = None, block_table: Optional[torch.Tensor] = None,
                 cmp_ratio: int = 1) -> Problem:
    """Fills a Problem from tensor shapes (no device data is read)."""
    p = Problem()
    p.num_heads_q = q.shape[-2]
    p.head_dim = q.shape[-1]
    p.num_heads_k = k.shape[-2]
    p.topk = int(topk)
    p.layout_q, p.layout_k = LAYOUT[layout_q], LAYOUT[layout_k]
    p.mask_mode = int(mask_mode)
    p.qk_dtype = DTYPE.get(q.dtype, -1)
    p.w_dtype = DTYPE.get(w.dtype, -1)
    p.cmp_ratio = int(cmp_ratio)
    if layout_q == "TND":
        p.total_q = q.shape[0]
        if batch_size is None or max_seqlen_q is None:
            raise ValueError("TND queries need batch_size and max_seqlen_q")
        p.batch, p.max_seqlen_q = int(batch_size), int(max_seqlen_q)
    else:
        p.batch, p.max_seqlen_q = q.shape[0], q.shape[1]
    if layout_k == "TND":
        p.total_k = k.shape[0]
        if max_seqlen_k is None:
            raise ValueError("TND keys need max_seqlen_k")
        p.max_seqlen_k = int(max_seqlen_k)
    elif layout_k in ("PA_BSND", "PA_BBND"):
        if block_table is None or max_seqlen_k is None:
            raise ValueError("paged keys need block_table and max_seqlen_k")
        p.block_size = k.shape[1]
        p.num_blocks = k.shape[0]
        p.max_blocks_per_seq = block_table.shape[1]
        p.k_block_stride = k.stride(0)
        p.max_seqlen_k = int(max_seqlen_k)
    else:
        p.max_seqlen_k = k.shape[1]
    return p


def lightning_indexer_metadata(p: Problem, *, cu_seqlens_q=None, cu_seqlens_k=None,
                               seqused_k=None, cmp_residual_k=None, device=None) -> torch.Tensor:
    """Allocates and fills the metadata (work list) on the current stream."""
    st, nbytes = li_metadata_size(p)
    _check(st, "li_metadata_size")
    dev = device or (cu_seqlens_q.device if cu_seqlens_q is not None else torch.device("cuda"))
    meta = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    _check(li_metadata(p, _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(seqused_k),
                       _ptr(cmp_residual_k), meta.data_ptr(), meta.numel(), stream),
           "li_metadata")
    return meta


def lightning_indexer(p: Problem, q, k, w, *, metadata: torch.Tensor, q_descale=None,
                      k_descale=None, cu_seqlens_q=None, cu_seqlens_k=None, seqused_k=None,
                      cmp_residual_k=None, block_table=None, output_idx_offset=None,
                      return_value: int = 1, workspace=None, out=None):
    """Runs li_forward; returns (sparse_indices, sparse_values or None).  Pass a
    `workspace` (uint8, li_workspace_size bytes) to read its status word with
    forward_status afterwards."""
    st, ws_bytes = li_workspace_size(p)
    _check(st, "li_workspace_size")
    dev = q.device
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    if p.layout_q == LAYOUT["TND"]:
        oshape = (p.total_q, 1, p.topk)
    else:
        oshape = (p.batch, p.max_seqlen_q, 1, p.topk)
    if out is None:
        idx = torch.empty(oshape, dtype=torch.int32, device=dev)
        val = torch.empty(oshape, dtype=torch.float32, device=dev) if return_value else None
    else:
        idx, val = out
    stream = torch.cuda.current_stream(dev).cuda_stream
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(li_forward(p, _ptr(q), _ptr(k), _ptr(w), _ptr(q_descale), _ptr(k_descale),
                      _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(seqused_k),
                      _ptr(cmp_residual_k), _ptr(block_table), _ptr(output_idx_offset),
                      metadata.data_ptr(), _ptr(workspace), wsb, idx.data_ptr(), _ptr(val),
                      stream), "li_forward")
    return idx, val


def forward_status(workspace: torch.Tensor) -> int:
    """The status word li_forward left at the start of its workspace (0 = LI_OK,
    5 = LI_ERR_METADATA_MISMATCH); waits for the work queued on the device."""
    return int(workspace[:4].view(torch.int32).item())


def gather_selected(p: Problem, kv: torch.Tensor, sparse_indices: torch.Tensor, *,
                    metadata: torch.Tensor, select_block: int = 1, block_table=None,
                    out=None) -> torch.Tensor:
    """Runs li_gather: the rows of `kv` (its last dimension holds one token's row,
    the leading ones the key layout of `p`) that sparse_indices select.  Returns
    uint8 [rows, topk * select_block, row_bytes] on the device."""
    row_bytes = kv.shape[-1] * kv.element_size()
    rows = sparse_indices.numel() // p.topk
    stride = kv.stride(0) * kv.element_size() if p.layout_k == LAYOUT["PA_BSND"] else 0
    if out is None:
        out = torch.empty((rows, p.topk * select_block, row_bytes), dtype=torch.uint8,
                          device=kv.device)
    stream = torch.cuda.current_stream(kv.device).cuda_stream
    _check(li_gather(p, kv.data_ptr(), row_bytes, stride, sparse_indices.data_ptr(), select_block,
                     _ptr(block_table), metadata.data_ptr(), out.data_ptr(), stream), "li_gather")
    return out


def run_instance(inst: dict, device="cuda", return_value: int = 1):
    """Convenience: runs metadata + forward on a synth-style instance dict (CPU
    tensors are copied to `device`).  Returns (indices, values) on the device."""
    dev = torch.device(device)
    g = {n: (inst[n].to(dev) if isinstance(inst.get(n), torch.Tensor) else None)
         for n in ("q", "k", "w", "q_descale", "k_descale", "cu_seqlens_q", "cu_seqlens_k",
                   "seqused_k", "block_table", "cmp_residual_k", "output_idx_offset")}
    if inst["layout_k"] == "PA_BSND":
        # keep the pool's block stride: copy the whole padded pool, then view it
        kc = inst["k"]
        base = kc.as_strided((kc.shape[0], kc.stride(0)), (kc.stride(0), 1))
        pool = base.to(dev)
        g["k"] = pool.as_strided(kc.shape, kc.stride())
    p = problem_for(inst, g["k"])
    meta = lightning_indexer_metadata(p, cu_seqlens_q=g["cu_seqlens_q"],
                                      cu_seqlens_k=g["cu_seqlens_k"], seqused_k=g["seqused_k"],
                                      cmp_residual_k=g["cmp_residual_k"], device=dev)
    return lightning_indexer(p, g["q"], g["k"], g["w"], metadata=meta, q_descale=g["q_descale"],
                             k_descale=g["k_descale"], cu_seqlens_q=g["cu_seqlens_q"],
                             cu_seqlens_k=g["cu_seqlens_k"], seqused_k=g["seqused_k"],
                             cmp_residual_k=g["cmp_residual_k"], block_table=g["block_table"],
                             output_idx_offset=g["output_idx_offset"], return_value=return_value)


def problem_for(inst: dict, k_dev: Optional[torch.Tensor] = None) -> Problem:
    """Problem scalars of a synth-style instance dict."""
    k = inst["k"] if k_dev is None else k_dev
    return problem_from(inst["q"], k, inst["w"], inst["topk"], layout_q=inst["layout_q"],
                        layout_k=inst["layout_k"], mask_mode=inst["mask_mode"],
                        batch_size=inst["batch"], max_seqlen_q=inst["max_seqlen_q"],
                        max_seqlen_k=inst["max_seqlen_k"], block_table=inst.get("block_table"),
                        cmp_ratio=inst.get("cmp_ratio", 1) or 1)


# ---------------------------------------------------------------------------
# backward of the indexer fused with its KL loss
# ---------------------------------------------------------------------------

def grad_problem_for(inst: dict) -> GradProblem:
    """GradProblem scalars of a synth.make_grad instance."""
    p = GradProblem()
    p.batch = inst["batch"]
    p.max_seqlen_q = inst["max_seqlen_q"]
    p.max_seqlen_k = inst["max_seqlen_k"]
    p.layout = LAYOUT[inst["layout"]]
    if inst["layout"] == "TND":
        p.total_q = p.total_k = int(sum(inst["seqlens"]))
    p.num_heads, p.head_dim, p.rope_dim = inst["n_main"], inst["d_main"], inst["d_rope"]
    p.num_heads_index, p.head_dim_index = inst["n_idx"], inst["d_idx"]
    p.topk = inst["topk"]
    p.dtype = DTYPE.get(inst["qi"].dtype, -1)
    p.w_dtype = DTYPE.get(inst["w"].dtype, -1)
    p.scale = float(inst["scale"])
    return p


GRAD_INPUTS = ("q", "k", "q_rope", "k_rope", "qi", "ki", "w", "sparse_indices", "softmax_max",
               "softmax_sum", "cu_seqlens_q", "cu_seqlens_k")


def lightning_indexer_grad_kl(p: GradProblem, t: dict, workspace=None):
    """Runs li_grad_kl on device tensors (a dict with the GRAD_INPUTS names);
    returns (loss [1], d_q_index, d_k_index, d_w), fp32 on the device."""
    dev = t["qi"].device
    rows = t["qi"].shape[0] * (t["qi"].shape[1] if t["qi"].dim() == 4 else 1)
    keys = t["ki"].numel() // t["ki"].shape[-1]
    st, wsb = li_grad_workspace_size(p)
    _check(st, "li_grad_workspace_size")
    if workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    dq = torch.empty(t["qi"].shape, dtype=torch.float32, device=dev)
    dk = torch.empty((keys, p.head_dim_index), dtype=torch.float32, device=dev)
    dw = torch.empty((rows, p.num_heads_index), dtype=torch.float32, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    _check(li_grad_kl(p, *[_ptr(t.get(n)) for n in GRAD_INPUTS], workspace.data_ptr(),
                      workspace.numel(), dq.data_ptr(), dk.data_ptr(), dw.data_ptr(),
                      loss.data_ptr(), stream), "li_grad_kl")
    return loss, dq, dk, dw
