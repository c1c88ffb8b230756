"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
its host-side validation maps each invalid argument to its status code before
any HIP call.  No test here launches a kernel."""
import ctypes
import os
import re

import pytest
import torch

from score_top_token_amd import binding, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, TOO_SMALL = 0, 1, 2, 3


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "li.h")).read()
    return sorted(set(re.findall(r"^\s*(?:li_status|const char\*)\s+(li_\w+)\s*\(", src, re.M)))


def test_library_exports_every_declared_symbol():
    lib = binding.load()
    syms = declared_symbols()
    assert set(syms) == set(binding.EXPORTED)
    for s in syms:
        assert hasattr(lib, s), s


def test_status_strings():
    assert binding.li_status_str(0) == "LI_OK"
    assert binding.li_status_str(5) == "LI_ERR_METADATA_MISMATCH"
    assert binding.li_status_str(2) == "LI_ERR_UNSUPPORTED"
    assert binding.li_status_str(99) == "LI_UNKNOWN_STATUS"


def base_problem(**kw):
    p = binding.Problem(batch=1, max_seqlen_q=256, max_seqlen_k=256, num_heads_q=8,
                        num_heads_k=1, head_dim=128, topk=32, layout_q=0, layout_k=0,
                        mask_mode=3, qk_dtype=0, w_dtype=0, cmp_ratio=1)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def pa_problem(**kw):
    base = dict(batch=2, max_seqlen_q=1, max_seqlen_k=1000, layout_k=2, block_size=128,
                num_blocks=16, max_blocks_per_seq=8)
    base.update(kw)
    return base_problem(**base)


@pytest.mark.parametrize("kw,status", [
    ({}, OK),
    (dict(num_heads_q=0), INVALID), (dict(num_heads_q=65), INVALID), (dict(num_heads_q=64), OK),
    (dict(num_heads_q=1), OK),
    (dict(num_heads_k=2), INVALID), (dict(head_dim=64), INVALID),
    (dict(topk=0), INVALID), (dict(topk=2048), OK), (dict(topk=2049), INVALID),
    (dict(topk=3072), OK), (dict(topk=8192), OK), (dict(topk=9216), INVALID),
    (dict(topk=3000), INVALID), (dict(topk=5120), OK),
    (dict(mask_mode=1), INVALID), (dict(mask_mode=0), OK),
    (dict(layout_q=2), INVALID), (dict(layout_k=7), INVALID),
    (dict(qk_dtype=2), INVALID), (dict(qk_dtype=1), OK), (dict(qk_dtype=3), OK),
    (dict(w_dtype=1), INVALID), (dict(w_dtype=2), OK),
    (dict(cmp_ratio=4), OK), (dict(cmp_ratio=0), INVALID),
    (dict(batch=-1), INVALID), (dict(max_seqlen_q=-1), INVALID),
    (dict(batch=0), OK),
])
def test_scalar_validation(kw, status):
    st, _ = binding.li_metadata_size(base_problem(**kw))
    assert st == status
    st2, _ = binding.li_workspace_size(base_problem(**kw))
    assert st2 == status


@pytest.mark.parametrize("kw,status", [
    ({}, OK), (dict(block_size=0), INVALID), (dict(block_size=1025), INVALID),
    (dict(block_size=1, max_seqlen_k=8), OK), (dict(num_blocks=0), INVALID), (dict(max_blocks_per_seq=0), INVALID),
    (dict(k_block_stride=100), INVALID), (dict(k_block_stride=128 * 130), OK),
    (dict(max_seqlen_k=1025), INVALID),
])
def test_paged_validation(kw, status):
    st, _ = binding.li_metadata_size(pa_problem(**kw))
    assert st == status


def test_sizes_prefill_and_decode():
    p = binding.problem_for(synth.make("tiny", 0))
    st, mb = binding.li_metadata_size(p)
    st2, wb = binding.li_workspace_size(p)
    assert st == OK and st2 == OK and mb > 256 and wb == 256      # the status block only
    dec = synth.scaled_spec("decode", batch=4, len_lo=300, len_hi=900, block_size=64)
    inst = synth.make(dec, 0)
    pd = binding.problem_for(inst)
    st, mb = binding.li_metadata_size(pd)
    st2, wb = binding.li_workspace_size(pd)
    assert st == OK and st2 == OK and wb >= 4 * inst["max_seqlen_k"] * 4
    assert binding.li_metadata_size(pd)[1] == mb          # sizes are pure functions


FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation first


def test_metadata_pointer_rules():
    p = base_problem()
    _, mb = binding.li_metadata_size(p)
    assert binding.li_metadata(p, None, None, None, None, None, mb, None) == INVALID
    assert binding.li_metadata(p, FAKE, None, None, None, FAKE, mb, None) == INVALID   # cu_q with BSND
    assert binding.li_metadata(p, None, FAKE, None, None, FAKE, mb, None) == INVALID   # cu_k with BSND
    assert binding.li_metadata(p, None, None, FAKE, None, FAKE, mb, None) == INVALID   # seqused_k w/o PA
    assert binding.li_metadata(p, None, None, None, None, FAKE, mb - 1, None) == TOO_SMALL
    assert binding.li_metadata(p, None, None, None, None, FAKE + 1, mb, None) == INVALID  # misaligned
    tnd = base_problem(layout_q=1, layout_k=1, total_q=10, total_k=10)
    _, mt = binding.li_metadata_size(tnd)
    assert binding.li_metadata(tnd, None, FAKE, None, None, FAKE, mt, None) == INVALID  # TND needs cu_q
    assert binding.li_metadata(tnd, FAKE, None, None, None, FAKE, mt, None) == INVALID  # TND needs cu_k
    pa = pa_problem()
    _, mp = binding.li_metadata_size(pa)
    assert binding.li_metadata(pa, None, None, None, None, FAKE, mp, None) == INVALID   # PA needs seqused_k


def test_forward_pointer_rules():
    p = base_problem()
    _, mb = binding.li_metadata_size(p)
    F = FAKE
    _, wb0 = binding.li_workspace_size(p)
    args = dict(q=F, k=F, w=F, qd=None, kd=None, cq=None, ck=None, su=None, cr=None, bt=None,
                off=None, meta=F, ws=F, wsb=wb0, idx=F, val=F)

    def call(prob=p, **over):
        a = dict(args)
        a.update(over)
        return binding.li_forward(prob, a["q"], a["k"], a["w"], a["qd"], a["kd"], a["cq"], a["ck"],
                                  a["su"], a["cr"], a["bt"], a["off"], a["meta"], a["ws"],
                                  a["wsb"], a["idx"], a["val"], None)

    assert call(q=None) == INVALID
    assert call(k=None) == INVALID
    assert call(w=None) == INVALID
    assert call(meta=None) == INVALID
    assert call(idx=None) == INVALID
    assert call(ws=None) == INVALID                       # the status block is always needed
    assert call(wsb=wb0 - 1) == TOO_SMALL
    assert call(q=F + 2) == INVALID                       # q not 16-byte aligned
    assert call(qd=F) == INVALID                          # descales only with fp8
    assert call(bt=F) == INVALID                          # block_table only with PA
    f8 = base_problem(qk_dtype=1)
    assert call(prob=f8) == INVALID                       # fp8 needs both descales
    assert call(prob=f8, qd=F) == INVALID
    pa = pa_problem()
    _, wb = binding.li_workspace_size(pa)
    assert wb > 0
    assert call(prob=pa, su=F) == INVALID                 # PA needs block_table
    assert call(prob=pa, su=F, bt=F, ws=F, wsb=wb - 1) == TOO_SMALL
    assert call(prob=pa, su=F, bt=F, ws=None, wsb=wb) == INVALID
    cmp = base_problem(cmp_ratio=4)                       # compressed keys, mask 3
    assert call(prob=cmp) == INVALID                      # needs cmp_residual_k
    assert call(cr=F) == INVALID                          # residuals only with compression
    assert call(prob=base_problem(cmp_ratio=4, mask_mode=0), cr=F) == INVALID   # not with mask 0


def test_empty_problem_launches_nothing():
    # zero query rows: LI_OK without touching the (fake) buffers or the device
    p = base_problem(batch=0)
    _, mb = binding.li_metadata_size(p)
    assert binding.li_metadata(p, None, None, None, None, FAKE, mb, None) == OK
    _, wb = binding.li_workspace_size(p)
    assert binding.li_forward(p, FAKE, FAKE, FAKE, None, None, None, None, None, None, None,
                              None, FAKE, FAKE, wb, FAKE, None, None) == OK
    tnd = base_problem(layout_q=1, layout_k=1, total_q=0, total_k=0, batch=3)
    _, mt = binding.li_metadata_size(tnd)
    assert binding.li_metadata(tnd, FAKE, FAKE, None, None, FAKE, mt, None) == OK


def test_problem_struct_matches_header():
    # field order and size of the ctypes mirror follow include/li.h
    src = open(os.path.join(ROOT, "include", "li.h")).read()
    body = re.search(r"typedef struct \{(.*?)\} li_problem;", src, re.S).group(1)
    names = re.findall(r"int(?:32|64)_t\s+(\w+)\s*;", body)
    names += []
    decl = []
    for line in body.splitlines():
        m = re.match(r"\s*int(32|64)_t\s+([\w, ]+);", line)
        if m:
            decl += [n.strip() for n in m.group(2).split(",")]
    assert [f[0] for f in binding.Problem._fields_] == decl
    assert ctypes.sizeof(binding.Problem) == 18 * 4 + 8


def test_gather_pointer_rules():
    p = base_problem()
    _, mb = binding.li_metadata_size(p)
    F = FAKE

    def call(prob=p, kv=F, rb=64, stride=0, idx=F, sel=1, bt=None, meta=F, out=F):
        return binding.li_gather(prob, kv, rb, stride, idx, sel, bt, meta, out, None)

    assert call(rb=0) == INVALID                           # row bytes > 0
    assert call(rb=40) == INVALID                          # multiple of 16
    assert call(sel=0) == INVALID                          # select block >= 1
    assert call(kv=None) == INVALID
    assert call(idx=None) == INVALID
    assert call(meta=None) == INVALID
    assert call(out=None) == INVALID
    assert call(kv=F + 8) == INVALID                       # 16-byte alignment
    assert call(bt=F) == INVALID                           # block_table only with PA
    pa = pa_problem()
    assert call(prob=pa) == INVALID                        # PA needs block_table
    assert call(prob=pa, bt=F, stride=16) == INVALID       # stride below a block
    assert call(prob=base_problem(batch=0)) == OK          # nothing to gather


def test_noalloc_rejects_workspace_past_its_scratch():
    # 64 sequences of 4 query rows and 200000 keys: decode score rows of 205 MB,
    # past the 128 MiB scratch array of li_forward_noalloc -> rejected before any
    # HIP call
    p = base_problem(batch=64, max_seqlen_q=4, max_seqlen_k=200000, num_heads_q=64, topk=2048)
    st, wsb = binding.li_workspace_size(p)
    assert st == OK and wsb > (128 << 20)
    F = FAKE
    assert binding.li_forward_noalloc(p, F, F, F, None, None, None, None, None, None, None, None,
                                      F, F, F, None) == TOO_SMALL
    # argument checks come first, as in li_forward
    assert binding.li_forward_noalloc(p, None, F, F, None, None, None, None, None, None, None,
                                      None, F, F, F, None) == INVALID
    # an empty problem is LI_OK without touching the device
    e = base_problem(batch=0)
    assert binding.li_forward_noalloc(e, F, F, F, None, None, None, None, None, None, None, None,
                                      F, F, F, None) == OK
