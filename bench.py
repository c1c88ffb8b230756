#!/usr/bin/env python3
"""Benchmark of the Lightning Indexer forward pass on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
li_metadata (work list) + li_forward (scores, ReLU / weight / head sum, fused
top-k, outputs).  Default workload: prefill, B=1, S1=S2=4096, BSND, 64
query-index heads, D=128, bf16 q/k/w, top-2048, right-down causal mask.

Prints one JSON line with the throughput (query tokens per second), the
roofline of the dominant kernel (its average duration measured with HIP events
on the launch stream, algorithmic FLOP = 2 * N1 * D per visible query-key pair)
and the CPU oracle timed on a bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--workload prefill|decode|varlen|longfp8|tiny]
                  [--no-cpu-baseline] [--gpus 1]

Without --workload the line's headline (value, roofline, cpu_baseline) is the
prefill workload, and "workloads" holds the same record for decode (% of HBM
bandwidth), varlen and longfp8 (% of MFMA peak), each with its own roofline and
CPU-baseline sample, all timed in the same run, and for grad_train: the
indexer backward fused with its KL loss (li_grad_kl) on a training-shaped
problem (4096 causal tokens, 64 index heads, top-2048, 32 main heads with rope).

--workload gather times li_gather instead: the rows that the decode workload's
top-2048 selects, gathered from a paged pool of 1 KiB token rows (HBM-bound).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from score_top_token_amd import binding, synth  # noqa: E402

PEAK_TFLOPS = {"bf16": 2516.6, "fp16": 2516.6, "fp8": 5033.2}   # dense MFMA, MI355X
PEAK_HBM_GBS = 8000.0
HBM_BOUND = {"decode"}
WARMUP_MIN_S = 0.5

# HBM traffic of the dominant kernel per launch, from rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE runs scaled by the same counters on a plain copy of known size.  Kept in
# profiles/traffic.json together with a hash of the kernel sources it was measured on;
# reported only while the sources still match (null otherwise).
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["li_device.h", "li_common_kernels.h", "li_pipe.h", "li_select.h",
                  "li_prefill_kernels.h", "li_prefill.hip", "li_prefill_bf16.hip",
                  "li_prefill_fp16.hip", "li_prefill_fp8.hip", "li_decode.hip", "li_metadata.hip",
                  "li_host.cpp", "li_internal.h", "li_gather.hip", "li_bucket.h", "li_grad.hip"]


def kernel_source_hash(root: str = ROOT) -> str:
    """Hash of the kernel sources with comments and blank space removed, so that a
    comment edit does not count as a kernel change."""
    import hashlib
    import re
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(root, "score_top_token_amd", "csrc", name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def copy_calibration(nbytes: int, reps: int) -> None:
    """A plain device-to-device copy of nbytes, reps times (the counter calibration)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def visible_pairs(inst) -> int:
    tot = 0
    for s1, s2 in zip(inst["seqlens_q"], inst["seqlens_k"]):
        if inst["mask_mode"] == 0:
            tot += s1 * s2
        else:
            i = np.arange(s1, dtype=np.int64)
            tot += int(np.clip(i + s2 - s1 + 1, 0, s2).sum())
    return tot


def algorithmic_bytes(inst) -> int:
    """Bytes the path must move at least: q, w, the visible K rows, descales,
    block-table entries used, and the outputs (indices + values)."""
    esz = 1 if inst["qk_dtype"] == "fp8" else 2
    rows = sum(inst["seqlens_q"])
    q = rows * inst["n1"] * 128 * esz
    w = rows * inst["n1"] * (4 if inst["w_dtype"] == "fp32" else 2)
    keys = sum(inst["seqlens_k"])            # every key is visible to some row
    k = keys * 128 * esz
    extra = 0
    if inst["qk_dtype"] == "fp8":
        extra += rows * 4 + keys * 4
    if inst["layout_k"] == "PA_BSND":
        bs = inst["block_size"]
        extra += sum(-(-s2 // bs) for s2 in inst["seqlens_k"]) * 4
    out = rows * inst["topk"] * 8
    return q + w + k + extra + out


def to_device(inst, dev):
    g = {n: (inst[n].to(dev) if isinstance(inst.get(n), torch.Tensor) else None)
         for n in ("q", "k", "w", "q_descale", "k_descale", "cu_seqlens_q", "cu_seqlens_k",
                   "seqused_k", "block_table")}
    if inst["layout_k"] == "PA_BSND":
        kc = inst["k"]
        base = kc.as_strided((kc.shape[0], kc.stride(0)), (kc.stride(0), 1)).to(dev)
        g["k"] = base.as_strided(kc.shape, kc.stride())
    return g


def host_cpu():
    """(model name, logical CPUs this process may run on) of the host."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return model, n


# The host's CPU share next to one GPU: the oracle's thread pool is capped here.
CPU_SHARE = 16


def cpu_baseline(inst, max_rows: int):
    """The oracle as it is, on a bounded, evenly spaced sample of the workload's rows."""
    import oracle
    model, ncpu = host_cpu()
    cores = min(ncpu, CPU_SHARE)
    ob = oracle.Bound(inst)
    total = ob.num_rows
    nrows = min(total, max_rows)
    rows = np.unique(np.linspace(0, total - 1, nrows).round().astype(np.int64))
    t0 = time.perf_counter()
    ob.forward(rows=rows, nthreads=cores)
    dt = time.perf_counter() - t0
    return {"value": len(rows) / dt, "unit": "query-tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": model, "host_cpus": ncpu,
            "sample": f"{len(rows)} of {total} query rows, evenly spaced, plain fp64 C oracle "
                      f"with {cores} POSIX threads (the host's CPU share next to one GPU); "
                      f"{dt:.1f} s wall"}


# rows of the CPU-baseline sample per workload (a few seconds to about 10 s of oracle
# time each on 16 cores of the GPU host)
CPU_ROWS = {"prefill": 4096, "decode": 64, "varlen": 4096, "longfp8": 320, "tiny": 256}
# the workloads timed in the default run: the headline first, then the rest of the metric
DEFAULT_WORKLOADS = ("prefill", "decode", "varlen", "longfp8", "grad_train")


def run_workload(name, args, dev, steps):
    """Times `steps` steps of li_metadata + li_forward on one workload; returns its record."""
    inst = synth.make(name, args.seed)
    g = to_device(inst, dev)
    p = binding.problem_for(inst, g["k"])
    st, meta_bytes = binding.li_metadata_size(p)
    assert st == 0, binding.li_status_str(st)
    st, ws_bytes = binding.li_workspace_size(p)
    assert st == 0, binding.li_status_str(st)
    meta = torch.empty(max(meta_bytes, 16), dtype=torch.uint8, device=dev)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    rows = sum(inst["seqlens_q"])
    topk = inst["topk"]
    idx = torch.empty(rows * topk, dtype=torch.int32, device=dev)
    val = torch.empty(rows * topk, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    ptr = lambda t: None if t is None else t.data_ptr()

    def metadata():
        st = binding.li_metadata(p, ptr(g["cu_seqlens_q"]), ptr(g["cu_seqlens_k"]),
                                 ptr(g["seqused_k"]), None, meta.data_ptr(), meta.numel(), sh)
        assert st == 0, binding.li_status_str(st)

    def forward():
        st = binding.li_forward(p, ptr(g["q"]), ptr(g["k"]), ptr(g["w"]), ptr(g["q_descale"]),
                                ptr(g["k_descale"]), ptr(g["cu_seqlens_q"]),
                                ptr(g["cu_seqlens_k"]), ptr(g["seqused_k"]), None,
                                ptr(g["block_table"]), None, meta.data_ptr(), ws.data_ptr(),
                                ws.numel(), idx.data_ptr(), val.data_ptr(), sh)
        assert st == 0, binding.li_status_str(st)

    # decode streams K from HBM: evict it from the caches (256 MB infinity cache)
    # between steps by reading 1 GiB of other data.  A read leaves the caches
    # holding clean lines; a fill would leave dirty ones whose write-back would
    # be charged to the next kernel.
    flush = None
    if name in HBM_BOUND:
        # float32: the sum reads it in place (an integer sum would first widen
        # it to int64 in a temporary, writing 2 GiB)
        flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)

    # untimed warm-up: at least W steps, and at least WARMUP_MIN_S seconds of
    # them, so that the timed steps run at the GPU's steady clocks (a cold GPU
    # runs the first ~0.2 s of work up to 10% slower)
    t_w = time.perf_counter()
    done = 0
    while done < args.warmup or time.perf_counter() - t_w < args.min_warmup_s:
        if flush is not None:
            flush.sum()
        metadata()
        forward()
        done += 1
        if done % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        if flush is not None:
            flush.sum()
        metadata()
        starts[s].record(stream)
        forward()
        ends[s].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    fwd_avg = float(np.mean(fwd_ms))

    # the metadata kernel alone (reported separately)
    m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    m0.record(stream)
    for _ in range(10):
        metadata()
    m1.record(stream)
    torch.cuda.synchronize()
    meta_ms = m0.elapsed_time(m1) / 10

    dtype = inst["qk_dtype"]
    pairs = visible_pairs(inst)
    flop = 2.0 * inst["n1"] * 128 * pairs
    hbm = algorithmic_bytes(inst)
    # with the cache eviction inside the loop the wall clock would count it: the
    # step is then the events' forward plus the metadata kernel
    ms_step = wall * 1000.0 / steps if flush is None else fwd_avg + meta_ms
    if name in HBM_BOUND:
        achieved = hbm / (fwd_avg / 1000.0) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": measured_traffic(name)}
    else:
        achieved = flop / (fwd_avg / 1000.0) / 1e12
        peak = PEAK_TFLOPS[dtype]
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": measured_traffic(name)}
    cfg = {"workload": name, "batch": inst["batch"], "seq_len_q": inst["max_seqlen_q"],
           "seq_len_k": inst["max_seqlen_k"], "query_rows": rows, "heads_q": inst["n1"],
           "head_dim": 128, "topk": topk, "layout_q": inst["layout_q"],
           "layout_k": inst["layout_k"], "mask_mode": inst["mask_mode"], "seed": args.seed}
    rec = {
        "value": rows / (ms_step / 1000.0), "unit": "query-tokens/s", "steps": steps,
        "warmup_steps_run": done, "ms_per_step": ms_step, "dtype": dtype, "config": cfg,
        "forward_ms": fwd_avg, "forward_ms_p10": float(np.percentile(fwd_ms, 10)),
        "forward_ms_p90": float(np.percentile(fwd_ms, 90)), "metadata_ms": meta_ms,
        "tflops": flop / (fwd_avg / 1000.0) / 1e12, "algorithmic_flop": flop,
        "algorithmic_bytes": hbm, "visible_pairs": pairs, "roofline": roof,
    }
    if dtype == "fp8":
        rec["frac_of_bf16_peak"] = rec["tflops"] / PEAK_TFLOPS["bf16"]
    del g, meta, ws, idx, val, flush
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(inst, CPU_ROWS.get(name, args.cpu_rows))
    return rec


def run_grad(name, args, dev, steps):
    """Times li_grad_kl (the backward fused with its KL loss) on a make_grad workload."""
    inst = synth.make_grad(name, args.seed)
    t = {n: (inst[n].to(dev) if isinstance(inst.get(n), torch.Tensor) else None)
         for n in binding.GRAD_INPUTS}
    p = binding.grad_problem_for(inst)
    st, wsb = binding.li_grad_workspace_size(p)
    assert st == 0, binding.li_status_str(st)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    run = lambda: binding.lightning_indexer_grad_kl(p, t, workspace=ws)
    t_w = time.perf_counter()
    done = 0
    while done < args.warmup or time.perf_counter() - t_w < args.min_warmup_s:
        run()
        done += 1
        if done % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for k in range(steps):
        starts[k].record(stream)
        run()
        ends[k].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    avg = float(np.mean(ms))
    rows = int(sum(inst["seqlens"]))
    pairs = int((inst["sparse_indices"] >= 0).sum())
    # per selected (row, key) pair: index scores, d_q_index and d_k_index (2 * Ni * 128
    # each) and the main-attention logits (2 * G * (128 + rope))
    flop_pair = 6 * inst["n_idx"] * inst["d_idx"] + 2 * inst["n_main"] * (inst["d_main"] +
                                                                          inst["d_rope"])
    flop = float(flop_pair) * pairs
    achieved = flop / (avg / 1000.0) / 1e12
    peak = PEAK_TFLOPS["bf16" if inst["qi"].dtype == torch.bfloat16 else "fp16"]
    rec = {
        "value": rows / (wall / steps), "unit": "query-tokens/s", "steps": steps,
        "warmup_steps_run": done, "ms_per_step": wall * 1000.0 / steps,
        "dtype": "bf16" if inst["qi"].dtype == torch.bfloat16 else "fp16",
        "config": {"workload": name, "batch": inst["batch"], "seq_len": inst["max_seqlen_q"],
                   "query_rows": rows, "heads_main": inst["n_main"], "rope_dim": inst["d_rope"],
                   "heads_index": inst["n_idx"], "topk": inst["topk"], "layout": inst["layout"],
                   "seed": args.seed},
        "forward_ms": avg, "forward_ms_p10": float(np.percentile(ms, 10)),
        "forward_ms_p90": float(np.percentile(ms, 90)), "selected_pairs": pairs,
        "algorithmic_flop": flop, "tflops": achieved,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": measured_traffic(name)},
    }
    del t, ws
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        from oracle import grad as grad_oracle
        model, ncpu = host_cpu()
        sample = np.linspace(0, rows - 1, 48).round().astype(np.int64)
        t0 = time.perf_counter()
        grad_oracle.Bound(inst).backward_rows(sample)
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {
            "value": len(sample) / dt, "unit": "query-tokens/s", "cores": 1, "kind": "oracle",
            "cpu_model": model, "host_cpus": ncpu,
            "sample": f"{len(sample)} of {rows} query rows, evenly spaced: loss, d_q_index and "
                      f"d_w of each row by the plain fp64 C oracle on one thread (d_k_index "
                      f"needs every row); {dt:.1f} s wall"}
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    choices=sorted(synth.PRESETS) + sorted(synth.GRAD_PRESETS) + ["gather"],
                    help="time this workload only (default: prefill as the headline, then "
                         "decode, varlen and longfp8 as sub-records)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--min-warmup-s", type=float, default=WARMUP_MIN_S,
                    help="warm-up lasts at least this long (0 under a profiler)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=1024)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES (counter calibration) and exit")
    ap.add_argument("--print-kernel-hash", action="store_true")
    args = ap.parse_args()
    if args.print_kernel_hash:
        print(kernel_source_hash())
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 4)
        return

    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (got --gpus {args.gpus}); "
              "sharding across GPUs is designed, not implemented", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    binding.load()
    if args.workload == "gather":
        bench_gather(args, dev)
        return
    names = (args.workload,) if args.workload else DEFAULT_WORKLOADS
    head = names[0]
    recs = {}
    for n in names:
        print(f"[bench] {n}: {args.steps} steps", file=sys.stderr, flush=True)
        if n in synth.GRAD_PRESETS:
            recs[n] = run_grad(n, args, dev, args.steps)
        else:
            recs[n] = run_workload(n, args, dev, args.steps)
    h = recs[head]
    out = {
        "metric": "query-tokens/s (prefill score + top-k), TFLOPS and % of MFMA peak",
        "value": h["value"], "unit": "query-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": h["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": h["dtype"], "data": "synthetic",
    }
    if head in HBM_BOUND:
        out["metric"] = "query-tokens/s (paged decode score + top-k) and % of HBM bandwidth"
    if head in synth.GRAD_PRESETS:
        out["metric"] = "query-tokens/s (indexer backward fused with its KL loss), % of MFMA peak"
    out.update({k: v for k, v in h.items() if k not in ("value", "unit", "steps", "ms_per_step",
                                                         "dtype")})
    if len(names) > 1:
        out["workloads"] = {n: recs[n] for n in names[1:]}
    print(json.dumps(out), flush=True)


GATHER_ROW_BYTES = 1024      # one token's row in the pool (e.g. 512 bf16 values)


def bench_gather(args, dev):
    """li_gather of the decode workload's selection: 64 query rows x 2048 indices
    into a paged pool of GATHER_ROW_BYTES-byte token rows (same block table)."""
    inst = synth.make("decode", args.seed)
    g = to_device(inst, dev)
    p = binding.problem_for(inst, g["k"])
    meta = binding.lightning_indexer_metadata(p, seqused_k=g["seqused_k"], device=dev)
    idx, _ = binding.lightning_indexer(p, g["q"], g["k"], g["w"], metadata=meta,
                                       seqused_k=g["seqused_k"], block_table=g["block_table"],
                                       return_value=0)
    idx = idx.reshape(-1, p.topk).contiguous()
    rows, topk = idx.shape
    R = GATHER_ROW_BYTES
    gen = torch.Generator(device=dev).manual_seed(args.seed)
    pool = torch.randint(0, 256, (inst["num_blocks"], inst["block_size"], R), dtype=torch.uint8,
                         device=dev, generator=gen)
    out = torch.empty((rows, topk, R), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    bt = g["block_table"]

    def gather():
        st = binding.li_gather(p, pool.data_ptr(), R, pool.stride(0), idx.data_ptr(), 1,
                               bt.data_ptr(), meta.data_ptr(), out.data_ptr(), sh)
        assert st == 0, binding.li_status_str(st)

    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # read-evicts the caches
    t_w = time.perf_counter()
    done = 0
    while done < args.warmup or time.perf_counter() - t_w < args.min_warmup_s:
        flush.sum()
        gather()
        done += 1
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for s in range(args.steps):
        flush.sum()
        starts[s].record(stream)
        gather()
        ends[s].record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    t = float(np.mean(ms))
    valid = int((idx >= 0).sum().item())
    nbytes = valid * R + rows * topk * R + rows * topk * 4      # rows read, rows written, indices
    achieved = nbytes / (t / 1000.0) / 1e9
    out_json = {
        "metric": "query-tokens/s (gather of the selected rows) and % of HBM bandwidth",
        "value": rows / (t / 1000.0), "unit": "query-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "warmup_steps_run": done, "ms_per_step": t,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": "gather", "query_rows": rows, "topk": topk, "row_bytes": R,
                   "select_block": 1, "layout_k": "PA_BSND", "block_size": inst["block_size"],
                   "seed": args.seed},
        "forward_ms": t, "forward_ms_p10": float(np.percentile(ms, 10)),
        "forward_ms_p90": float(np.percentile(ms, 90)), "algorithmic_bytes": nbytes,
        "selected_rows": valid,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": measured_traffic("gather")},
    }
    if not args.no_cpu_baseline:
        from oracle.gather import gather as oracle_gather
        sub = rows                                # every query row, timed on the host
        kv = pool.cpu().numpy()
        sub_inst = dict(inst, batch=sub, seqlens_q=inst["seqlens_q"][:sub],
                        seqlens_k=inst["seqlens_k"][:sub])
        t0 = time.perf_counter()
        oracle_gather(sub_inst, kv, idx[:sub].cpu().numpy(), 1)
        dt = time.perf_counter() - t0
        out_json["cpu_baseline"] = {"value": sub / dt, "unit": "query-tokens/s", "cores": 1,
                                    "kind": "oracle",
                                    "sample": f"all {sub} query rows, plain Python/numpy "
                                              f"gather; {dt:.2f} s wall"}
    print(json.dumps(out_json), flush=True)


if __name__ == "__main__":
    main()
