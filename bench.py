"""Benchmark: split-KV attention forward on one MI355X.

Workload: the long-context packed-varlen prefill (one sequence, H = 12,
Sq = 4096, Sk = 42700, D_qk = 192, D_v = 128, split_kv = 3, non-causal, bf16
inputs N(0, 1) from a seeded generator, scale 1/sqrt(192)).  A step is the
whole path: sk_valid_split_counts -> sk_attn_partial -> sk_attn_combine, with
inputs already resident in HBM.  Prints ONE JSON line.  After the timed
forward steps, the backward (sk_attn_backward: dQ, dK, dV of the same
problem for a seeded dO) is timed on its own and reported under "backward".

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--backward-steps N] [--copy-check]
    python bench.py --write-traffic FETCH_DIR WRITE_DIR   (traffic file from
                    two rocprofv3 counter runs; see write_traffic)
    python bench.py --sweep    (every parity workload, one JSON line each)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s (% bf16 MFMA peak) at Sq4096 Sk42700 H12; combine GB/s"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "partial_bf16_hbm_traffic.json")
# the partial entry point's kernels and the host code that plans their launch
PARTIAL_SOURCES = ["split_kv_attention_amd/csrc/partial_bf16.hip", "split_kv_attention_amd/csrc/pieces.hpp",
                   "split_kv_attention_amd/csrc/mfma_common.hpp",
                   "split_kv_attention_amd/csrc/sk_common.hpp", "split_kv_attention_amd/csrc/splitkv_api.cpp"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in PARTIAL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the partial entry point from the committed
    rocprofv3 counter summary, or None when absent or taken on different
    kernel code."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def write_traffic(fetch_dir: str, write_dir: str, path: str = TRAFFIC_FILE) -> dict:
    """Write the traffic file (TRAFFIC_FILE unless `path` is given) from two
    rocprofv3 counter runs of this script with --copy-check: `--pmc
    FETCH_SIZE` into fetch_dir and `--pmc WRITE_SIZE` into write_dir (csv
    output, file prefix "run").  Each counter is averaged over the split
    launches of the partial kernel (those followed by their piece merge; the
    unsplit comparison's launches have no pieces) and the piece merge's
    dispatches, and scaled by what it reads for the plain 1 GiB device copy
    (the largest dispatch that is not one of this library's kernels)."""
    import csv
    from collections import defaultdict

    def per_dispatch(d: str, counter: str):
        vals = defaultdict(float)
        names = {}
        with open(os.path.join(d, "run_counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                vals[r["Dispatch_Id"]] += float(r["Counter_Value"])
                names[r["Dispatch_Id"]] = r["Kernel_Name"]
        return vals, names

    def summarize(d: str, counter: str):
        vals, names = per_dispatch(d, counter)
        mine = {"partial_bf16_kernel": [], "merge_pieces_kernel": []}
        other = []
        for i, v in vals.items():
            key = next((k for k in mine if k in names[i]), None)
            if key == "partial_bf16_kernel":
                # the split-3 launches only: each is followed by its piece
                # merge (the unsplit comparison's launches have no pieces)
                nxt = str(int(i) + 1)
                if nxt in names and "merge_pieces_kernel" in names[nxt]:
                    mine[key].append(v)
            elif key:
                mine[key].append(v)
            elif "sk::" not in names[i] and "_ZN2sk" not in names[i]:
                other.append(v)
        if not all(mine.values()) or not other:
            raise SystemExit(f"{d}: partial kernel, piece merge or copy dispatch missing")
        return {k: sum(v) / len(v) for k, v in mine.items()}, max(other)

    fetch, copy_fetch = summarize(fetch_dir, "FETCH_SIZE")
    write, copy_write = summarize(write_dir, "WRITE_SIZE")
    gib = 1 << 30
    fetch_scale = gib / (copy_fetch * 1024.0)
    write_scale = gib / (copy_write * 1024.0)
    total = sum(fetch.values()) * 1024.0 * fetch_scale + sum(write.values()) * 1024.0 * write_scale
    from split_kv_attention_amd import workloads

    w = workloads.LONG_PREFILL
    H, Sq, Sk, S = w.heads, w.sq[0], w.sk[0], w.split_kv
    algorithmic = Sq * H * w.d_qk * 2 + Sk * H * (w.d_qk + w.d_v) * 2 + S * H * Sq * (w.d_v + 1) * 4
    out = {
        "kernel": "sk_attn_partial: partial_bf16_kernel<192,128> (256-row workgroups) + merge_pieces_kernel<256,128>",
        "workload": w.name,
        "kernel_source_sha256": kernel_source_hash(),
        "kernel_sources": PARTIAL_SOURCES,
        "fetch_size_kib_per_dispatch": fetch,
        "write_size_kib_per_dispatch": write,
        "copy_reference": {"bytes_read": gib, "bytes_written": gib, "fetch_size_kib": copy_fetch,
                           "write_size_kib": copy_write},
        "fetch_scale": fetch_scale,
        "write_scale": write_scale,
        "hbm_bytes_per_launch": round(total),
        "algorithmic_bytes_per_launch": algorithmic,
        "commands": [
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o run -- python3 bench.py "
            "--no-cpu-baseline --steps 3 --warmup 1 --cold-iters 1 --backward-steps 1 --copy-check",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o run -- python3 bench.py "
            "--no-cpu-baseline --steps 3 --warmup 1 --cold-iters 1 --backward-steps 1 --copy-check",
            f"python3 bench.py --write-traffic {fetch_dir} {write_dir}",
        ],
    }
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    return out


def visible_pairs(w) -> int:
    """(query, key) pairs the mask leaves visible, per head: row q of
    sequence b sees keys 0 .. min(q + offset_b, lastValid_b) (no mask: 0 ..
    lastValid_b), lastValid_b = Sk_b - 1 unless given."""
    import numpy as np

    total = 0
    for b, (sq, sk) in enumerate(zip(w.sq, w.sk)):
        lv = w.last_valid_per_seq[b] if w.last_valid_per_seq else w.last_valid_kv_index
        lv = sk - 1 if lv < 0 else min(lv, sk - 1)
        q = np.arange(sq, dtype=np.int64)
        if w.mask == "none":
            last = np.full(sq, lv, dtype=np.int64)
        else:
            off = 0 if w.mask == "causal" else (w.prefix_offset_per_seq[b] if w.prefix_offset_per_seq
                                                  else w.prefix_offset)
            last = np.minimum(q + off, lv)
        total += int(np.clip(last + 1, 0, sk).sum())
    return total


def time_step_eager_and_graph(prob, q, k, v, counts, o_part, lse_part, out, lse_out, stream, n: int):
    """Per-step time of counts -> partial -> combine run n times back to back
    on `stream`: eager launches, then the same three launches captured once
    as a HIP graph and replayed n times (small workloads are bound by the
    launches, not the kernels), and eagerly with two launches, the combine
    computing each row's count itself (no counts array).  The replays and
    the two-launch steps must reproduce the eager output bit for bit."""
    import torch

    from split_kv_attention_amd import _lib

    def run_on(s):
        _lib.sk_valid_split_counts(prob.c, counts, s)
        _lib.sk_attn_partial(prob.c, q, k, v, o_part, lse_part, s)
        _lib.sk_attn_combine(prob.c, o_part, lse_part, counts, out, lse_out, s)

    def timed(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    t_eager = timed(lambda: run_on(stream.cuda_stream))
    expect = (out.clone(), lse_out.clone())
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            run_on(side.cuda_stream)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    out.fill_(float("nan"))
    graph.replay()
    torch.cuda.synchronize()
    if not (torch.equal(out, expect[0]) and torch.equal(lse_out, expect[1])):
        raise RuntimeError("the replayed step differs from the eager one")
    t_graph = timed(graph.replay)
    del graph

    def two_launches():
        _lib.sk_attn_partial(prob.c, q, k, v, o_part, lse_part, stream.cuda_stream)
        _lib.sk_attn_combine(prob.c, o_part, lse_part, None, out, lse_out, stream.cuda_stream)

    out.fill_(float("nan"))
    t_inline = timed(two_launches)
    if not (torch.equal(out, expect[0]) and torch.equal(lse_out, expect[1])):
        raise RuntimeError("the step with inline counts differs from the eager one")
    return t_eager, t_graph, t_inline


def sweep(only: str | None = None, oracle_budget_s: float = 0.0) -> None:
    """Every workload of the parity suite (or those whose name starts with
    `only`) through counts -> partial -> combine, medians of HIP-event
    timings on one stream; one JSON line per workload with the partial's
    rate against its roofline (bf16 MFMA or HBM, whichever bounds it; the f32
    kernel against the fp32 vector peak) and the combine's against HBM.
    With oracle_budget_s > 0 the line also holds the oracle timed on the
    host's cores over the same workload (cpu_baseline, that budget each)."""
    import numpy as np
    import torch

    from split_kv_attention_amd import _lib, attention, workloads

    torch.cuda.set_device(0)
    for w in workloads.CONFIGS:
        if only and not w.name.startswith(only):
            continue
        inputs = workloads.make_inputs(w, "cuda:0", seed=3)
        prob = attention.build_problem(inputs["q"], inputs["k"], inputs["v"], **workloads.problem_kwargs(w, inputs))
        counts, o_part, lse_part, out, lse_out = attention.alloc_outputs(prob, inputs["q"], inputs["v"])
        stream = torch.cuda.current_stream()
        sh = stream.cuda_stream
        q, k, v = inputs["q"], inputs["k"], inputs["v"]

        def step(ev=None):
            if ev:
                ev[0].record(stream)
            _lib.sk_valid_split_counts(prob.c, counts, sh)
            if ev:
                ev[1].record(stream)
            _lib.sk_attn_partial(prob.c, q, k, v, o_part, lse_part, sh)
            if ev:
                ev[2].record(stream)
            _lib.sk_attn_combine(prob.c, o_part, lse_part, counts, out, lse_out, sh)
            if ev:
                ev[3].record(stream)

        n = 20 if sum(w.sk) * w.heads * w.batch > 1e8 else 50
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
        for i in range(n):
            step(evs[i])
        torch.cuda.synchronize()
        t_part = sorted(e[1].elapsed_time(e[2]) for e in evs)[n // 2]
        t_comb = sorted(e[2].elapsed_time(e[3]) for e in evs)[n // 2]
        t_eager, t_graph, t_inline = time_step_eager_and_graph(prob, q, k, v, counts, o_part, lse_part, out, lse_out,
                                                               stream, n)

        H, es = w.heads, q.element_size()
        rows = sum(w.sq)
        keys = sum(w.sk) if w.packed else w.batch * w.sk[0]
        splits = w.split_kv_per_seq or (w.split_kv,) * w.batch
        flop = 2.0 * (w.d_qk + w.d_v) * H * visible_pairs(w)
        part_bytes = (rows * w.d_qk + keys * (w.d_qk + w.d_v)) * H * es + \
            sum(s * r for s, r in zip(splits, w.sq)) * H * (w.d_v + 1) * 4
        c = counts.cpu().numpy().astype(np.int64)
        comb_bytes = int(c.sum()) * H * (w.d_v * 4 + 4) + rows * 4 + rows * H * (w.d_v * out.element_size() + 4)
        if w.dtype == "f32":
            bound, peak, unit, achieved = "alu", 157.3, "TFLOP/s", flop / (t_part * 1e-3) / 1e12
        elif flop / part_bytes > PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9):
            bound, peak, unit, achieved = "mfma", PEAK_BF16_TFLOPS, "TFLOP/s", flop / (t_part * 1e-3) / 1e12
        else:
            bound, peak, unit, achieved = "hbm", PEAK_HBM_GBPS, "GB/s", part_bytes / (t_part * 1e-3) / 1e9
        comb_gbps = comb_bytes / (t_comb * 1e-3) / 1e9
        line = {
            "workload": w.name, "calls": n,
            "partial": {"ms": t_part, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                        "frac": achieved / peak, "flop": flop, "algorithmic_bytes": part_bytes},
            "combine": {"ms": t_comb, "gbps": comb_gbps, "frac": comb_gbps / PEAK_HBM_GBPS,
                        "algorithmic_bytes": comb_bytes},
            "step": {"ms_eager": t_eager, "ms_graph": t_graph, "ms_inline_counts": t_inline,
                     "tflops_eager": flop / (t_eager * 1e-3) / 1e12, "tflops_graph": flop / (t_graph * 1e-3) / 1e12},
        }
        if oracle_budget_s > 0:
            base = cpu_baseline(w, inputs, prob.m_per_block, budget_s=oracle_budget_s)
            base["gpu_speedup"] = (flop / ((t_part + t_comb) * 1e-3) / 1e12) / base["value"]
            line["cpu_baseline"] = base
        print(json.dumps(line), flush=True)
        del inputs, prob, counts, o_part, lse_part, out, lse_out, q, k, v
        torch.cuda.empty_cache()


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def _blas_info() -> str:
    try:
        from threadpoolctl import threadpool_info

        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        return ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in libs) or "unknown"
    except Exception:  # pragma: no cover
        return "unknown"


def _visible_pairs_rows(w, b: int, rows) -> int:
    """Visible (query, key) pairs of `rows` of sequence b, per head (the rule
    of visible_pairs)."""
    import numpy as np

    sk = w.sk[b]
    lv = w.last_valid_per_seq[b] if w.last_valid_per_seq else w.last_valid_kv_index
    lv = sk - 1 if lv < 0 else min(lv, sk - 1)
    q = np.asarray(rows, dtype=np.int64)
    if w.mask == "none":
        last = np.full(len(q), lv, dtype=np.int64)
    else:
        off = 0 if w.mask == "causal" else (w.prefix_offset_per_seq[b] if w.prefix_offset_per_seq else w.prefix_offset)
        last = np.minimum(q + off, lv)
    return int(np.clip(last + 1, 0, sk).sum())


def cpu_baseline(w, inputs, m_per_block: int, budget_s: float = 45.0, max_workers: int = 16,
                 max_host_bytes: float = 4e9):
    """The oracle (as it stands) timed on the host's cores over the whole
    workload: units of (sequence, head, 32 query rows), each the full split
    method (counts, partials at the kernel's query block, merge) against all
    of the sequence's keys, run on a thread pool with one BLAS thread per
    worker and as many workers as the process may use (its CPU affinity,
    capped at the GPU's 16-core share).  Units run in a seeded random order;
    if the wall-clock budget runs out first, the finished units are the
    sample and the rate is scaled from them.  The inputs are copied to the
    host before the clock starts; a workload whose K and V exceed
    max_host_bytes is sampled by whole sequences (seeded) to fit."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor, wait, FIRST_COMPLETED
    from threadpoolctl import threadpool_limits

    from oracle import adapter

    affinity = len(os.sched_getaffinity(0))
    workers = max(1, min(affinity, max_workers))
    nseq = len(w.sq)
    per_seq = [w.heads * w.sk[b] * (w.d_qk + w.d_v) * inputs["k"].element_size() for b in range(nseq)]
    seqs = list(range(nseq))
    if sum(per_seq) > max_host_bytes:
        keep, tot = [], 0.0
        for b in np.random.default_rng(1).permutation(nseq):
            if tot + per_seq[b] <= max_host_bytes or not keep:
                keep.append(int(b))
                tot += per_seq[b]
        seqs = sorted(keep)
    if len(seqs) == nseq:
        host = {k: (v.cpu() if hasattr(v, "cpu") else v) for k, v in inputs.items()}
    else:
        # dense batch [B, H, S, D]: only the kept sequences, indexed [b, h, ...]
        host = {}
        for k, v in inputs.items():
            if hasattr(v, "cpu") and v.dim() == 4:
                host[k] = _HostSequences({b: v[b].cpu() for b in seqs})
            else:
                host[k] = v.cpu() if hasattr(v, "cpu") else v
    chunk = 32
    units = [(b, h, r0) for b in seqs for h in range(w.heads) for r0 in range(0, w.sq[b], chunk)]
    units_total = sum(w.heads * ((w.sq[b] + chunk - 1) // chunk) for b in range(nseq))
    order = np.random.default_rng(0).permutation(len(units))

    def run_unit(i):
        b, h, r0 = units[i]
        rows = np.arange(r0, min(r0 + chunk, w.sq[b]))
        adapter.expected(w, host, m_per_block, rows_per_seq={bb: (rows if bb == b else rows[:0])
                                                              for bb in range(nseq)}, heads=[h])
        return float(_visible_pairs_rows(w, b, rows))

    pairs = 0.0
    done = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1), ThreadPoolExecutor(workers) as ex:
        it = iter(order)
        pending = set()
        for _ in range(2 * workers):
            i = next(it, None)
            if i is not None:
                pending.add(ex.submit(run_unit, int(i)))
        while pending:
            fin, pending = wait(pending, return_when=FIRST_COMPLETED)
            for f in fin:
                pairs += f.result()
                done += 1
            if time.perf_counter() - t0 < budget_s:
                for _ in fin:
                    i = next(it, None)
                    if i is not None:
                        pending.add(ex.submit(run_unit, int(i)))
    dt = time.perf_counter() - t0
    flops = 2.0 * (w.d_qk + w.d_v) * pairs
    full = done == units_total
    what = "the whole workload" if full else \
        f"{done} of {units_total} units (seeded random order; budget {budget_s:.0f} s" + \
        (f"; {len(seqs)} of {nseq} sequences on the host)" if len(seqs) < nseq else ")")
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{what}: units of (sequence, head, {chunk} query rows) x all the sequence's keys, full split "
                  f"method in f64, {dt:.1f} s wall on a {workers}-thread pool, one BLAS thread each",
        "seconds": dt,
        "units_done": done,
        "units_total": units_total,
        "cpu_model": _cpu_model(),
        "affinity_cpus": affinity,
        "numpy": np.__version__,
        "blas": _blas_info(),
    }


class _HostSequences:
    """Some sequences of a dense [B, H, S, D] batch on the host, indexed like
    the batch by [b, h, ...] (only the kept b)."""

    def __init__(self, per_seq):
        self.per_seq = per_seq

    def __getitem__(self, key):
        return self.per_seq[key[0]][key[1:]]


def time_unsplit(w, inputs, stream, steps: int, warmup: int):
    """The same inputs through the same kernels with split_kv = 1 (one
    partial per row, the combine a plain cast), timed with HIP events like
    the split path: the comparison the aiter page's "Test Result" makes
    between its unsplit and split-3 kernels (MI325X: 3.065 ms and 2.269 ms,
    26% faster; another machine, quoted as context only)."""
    import dataclasses

    import torch

    from split_kv_attention_amd import _lib, attention, workloads

    w1 = dataclasses.replace(w, split_kv=1)
    prob = attention.build_problem(inputs["q"], inputs["k"], inputs["v"], **workloads.problem_kwargs(w1, inputs))
    counts, o_part, lse_part, out, lse_out = attention.alloc_outputs(prob, inputs["q"], inputs["v"])
    q, k, v = inputs["q"], inputs["k"], inputs["v"]
    sh = stream.cuda_stream

    def step(ev=None):
        _lib.sk_valid_split_counts(prob.c, counts, sh)
        if ev:
            ev[0].record(stream)
        _lib.sk_attn_partial(prob.c, q, k, v, o_part, lse_part, sh)
        if ev:
            ev[1].record(stream)
        _lib.sk_attn_combine(prob.c, o_part, lse_part, counts, out, lse_out, sh)
        if ev:
            ev[2].record(stream)

    for _ in range(max(3, min(warmup, 10))):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    t_part = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    t_comb = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    H, Sq, Sk = w.heads, w.sq[0], w.sk[0]
    flops = 2.0 * (w.d_qk + w.d_v) * H * Sq * Sk
    return {
        "split_kv": 1,
        "ms_partial": t_part,
        "ms_combine": t_comb,
        "ms_partial_plus_combine": t_part + t_comb,
        "tflops_partial_plus_combine": flops / ((t_part + t_comb) * 1e-3) / 1e12,
        "pages_context_mi325x": {"unsplit_ms": 3.065, "split3_ms": 2.269, "split_time_saved_frac": 0.26},
    }


def compare_split(unsplit: dict, t_partial_split: float, t_combine_split: float) -> dict:
    """The unsplit timing beside the split step's partial + combine."""
    split_total = t_partial_split + t_combine_split
    both = unsplit["ms_partial_plus_combine"]
    return dict(unsplit, split_ms_partial_plus_combine=split_total, split_speedup=both / split_total,
                split_time_saved_frac=1.0 - split_total / both)


def time_backward(w, prob, inputs, out, lse, stream, steps: int):
    """sk_attn_backward on the forward's out / LSE and a seeded dO, timed
    with HIP events on `stream` over `steps` calls after 10 warmup calls
    (about 50 ms: the clock settles under them).

    FLOPs: the five products of attention's gradient over the Sq x Sk pairs
    (recomputed scores Q K^T and dO V^T, dV = P^T dO, dQ = dS K,
    dK = dS^T Q), 2 Sq Sk H (3 D_qk + 2 D_v).  The kernels compute the scores
    and dO V^T twice (once in the dQ pass, once in the dK/dV pass):
    2 Sq Sk H (4 D_qk + 3 D_v) executed."""
    import torch

    from split_kv_attention_amd import _lib, workloads

    q, k, v = inputs["q"], inputs["k"], inputs["v"]
    dout = workloads.make_dout(w, q.device, 3)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nbytes = _lib.sk_backward_workspace_bytes(prob.c)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    sh = stream.cuda_stream

    def call():
        _lib.sk_attn_backward(prob.c, q, k, v, out, dout, lse, dq, dk, dv, ws, nbytes, sh)

    for _ in range(10):
        call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    H, Sq, Sk = w.heads, w.sq[0], w.sk[0]
    flop = 2.0 * Sq * Sk * H * (3 * w.d_qk + 2 * w.d_v)
    executed = 2.0 * Sq * Sk * H * (4 * w.d_qk + 3 * w.d_v)
    achieved = flop / (ms * 1e-3) / 1e12
    return {
        "bound": "mfma",
        "kernels": "bwd_rowdot, bwd_dq (per split), bwd_dkdv, bwd_dq_reduce",
        "ms": ms,
        "calls": steps,
        "algorithmic_flop": flop,
        "executed_flop": executed,
        "achieved": achieved,
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": achieved / PEAK_BF16_TFLOPS,
        "workspace_bytes": nbytes,
    }


COLD_COPIES = 8


def time_combine_cold_back_to_back(prob, o_part, lse_part, counts, out, lse_out, flush, stream, iters):
    """Median per-launch time of COLD_COPIES combines launched back to back
    after a cache flush, each on its own copy of the partials, counts and
    outputs: every launch reads data no earlier launch touched (the copies
    together exceed the 256 MB infinity cache), while the dispatch of each
    overlaps the previous one's execution as in a pipeline."""
    import torch

    from split_kv_attention_amd import _lib

    sh = stream.cuda_stream
    copies = [(o_part.clone(), lse_part.clone(), counts.clone(), torch.empty_like(out), torch.empty_like(lse_out))
              for _ in range(COLD_COPIES)]
    per_launch = []
    for _ in range(max(iters, 1)):
        flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for o, l, c, y, ly in copies:
            _lib.sk_attn_combine(prob.c, o, l, c, y, ly, sh)
        b.record(stream)
        per_launch.append((a, b))
    torch.cuda.synchronize()
    for _, _, _, y, ly in copies:  # every copy merged the same partials
        if not (torch.equal(y, out) and torch.equal(ly, lse_out)):
            raise RuntimeError("a back-to-back combine differs from the pipeline's")
    del copies
    return sorted(a.elapsed_time(b) for a, b in per_launch)[len(per_launch) // 2] / COLD_COPIES


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The shader clock takes tens of milliseconds to settle under this load;
    # the other measurements run before the warm-up steps (main), and 50
    # untimed steps (~60 ms) precede the 100 timed ones.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-iters", type=int, default=10, help="combine timings after a cache flush")
    ap.add_argument("--backward-steps", type=int, default=10, help="timed backward calls (0: skip)")
    ap.add_argument("--copy-check", action="store_true",
                    help="also run one plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    ap.add_argument("--only", default=None, help="with --sweep: only workloads whose name starts with this")
    ap.add_argument("--oracle-seconds", type=float, default=0.0,
                    help="with --sweep: also time the oracle on the host for up to this many seconds per workload")
    ap.add_argument("--sweep", action="store_true",
                    help="time every workload of the parity suite (one JSON line each), then exit")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the partial kernel's HBM traffic file from two rocprofv3 counter runs, then exit")
    args = ap.parse_args()
    if args.write_traffic:
        print(json.dumps(write_traffic(*args.write_traffic), indent=1))
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the path has no multi-GPU mode",
              file=sys.stderr)
        return 2
    if args.sweep:
        sweep(args.only, args.oracle_seconds)
        return 0

    import torch

    from split_kv_attention_amd import _lib, attention, workloads

    w = workloads.LONG_PREFILL
    dev = "cuda:0"
    torch.cuda.set_device(0)
    inputs = workloads.make_inputs(w, dev, seed=3)
    prob = attention.build_problem(inputs["q"], inputs["k"], inputs["v"], **workloads.problem_kwargs(w, inputs))
    counts, o_part, lse_part, out, lse_out = attention.alloc_outputs(prob, inputs["q"], inputs["v"])
    q, k, v = inputs["q"], inputs["k"], inputs["v"]
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        _lib.sk_valid_split_counts(prob.c, counts, sh)
        if ev:
            ev[1].record(stream)
        _lib.sk_attn_partial(prob.c, q, k, v, o_part, lse_part, sh)
        if ev:
            ev[2].record(stream)
        _lib.sk_attn_combine(prob.c, o_part, lse_part, counts, out, lse_out, sh)
        if ev:
            ev[3].record(stream)

    # The measurements beside the headline run first, on the outputs of one
    # untimed step: the combine after a cache flush, the backward and the
    # unsplit comparison (about 0.1-0.2 s of GPU work).  The shader clock
    # takes tens of milliseconds of load to settle, so the warm-up and timed
    # steps below then start at the clock the GPU holds under sustained load
    # whatever the warm-up count.
    step()
    torch.cuda.synchronize()

    # combine after evicting L2 and the 256 MB infinity cache: reading a
    # 512 MB buffer leaves no dirty lines whose write-back would be charged
    # to the combine
    flush = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    cold = []
    for _ in range(args.cold_iters):
        flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        _lib.sk_attn_combine(prob.c, o_part, lse_part, counts, out, lse_out, sh)
        b.record(stream)
        cold.append((a, b))
    # The same bracket around a kernel that does almost nothing (a 64-float
    # fill) after the same flush: the fixed cost every cold event-timed
    # launch pays (dispatch, start-up, completion), reported beside the
    # combine's time.
    tiny = torch.empty(64, dtype=torch.float32, device=dev)
    floor = []
    for _ in range(args.cold_iters):
        flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        tiny.fill_(1.0)
        b.record(stream)
        floor.append((a, b))
    torch.cuda.synchronize()
    t_combine_cold = sorted(x.elapsed_time(y) for x, y in cold)[len(cold) // 2]
    t_launch_floor = sorted(x.elapsed_time(y) for x, y in floor)[len(floor) // 2]
    t_combine_cold_b2b = time_combine_cold_back_to_back(prob, o_part, lse_part, counts, out, lse_out, flush, stream,
                                                        args.cold_iters)
    del flush, tiny

    backward = None
    if args.backward_steps > 0:
        backward = time_backward(w, prob, inputs, out, lse_out, stream, args.backward_steps)

    unsplit = time_unsplit(w, inputs, stream, args.steps, args.warmup)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    t_counts = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    t_partial = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    t_combine = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps
    unsplit = compare_split(unsplit, t_partial, t_combine)

    if args.copy_check:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        src.zero_()
        torch.cuda.synchronize()
        dst.copy_(src)  # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst

    H, Sq, Sk, S = w.heads, w.sq[0], w.sk[0], w.split_kv
    flops = 2.0 * (w.d_qk + w.d_v) * H * Sq * Sk  # non-causal: every (query, key) pair is visible
    rows = Sq
    combine_bytes = (S * H * rows * w.d_v * 4 + S * H * rows * 4 + rows * 4 + rows * H * w.d_v * 2 + H * rows * 4)
    partial_bytes = (rows * H * w.d_qk * 2 + Sk * H * (w.d_qk + w.d_v) * 2 + S * H * rows * (w.d_v + 1) * 4)
    achieved = flops / (t_partial * 1e-3) / 1e12
    traffic = measured_traffic()
    res = {
        "metric": METRIC,
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic N(0,1) bf16 inputs from a seeded generator",
        "measurement_order": "one untimed step; the cold-cache combine, backward and unsplit timings; then the "
                             "warm-up steps and the timed steps",
        "config": {
            "workload": w.name,
            "batch": 1, "heads": H, "seqlen_q": Sq, "seqlen_k": Sk, "d_qk": w.d_qk, "d_v": w.d_v,
            "split_kv": S, "n_per_block": w.n_per_block, "mask": w.mask, "layout": "packed varlen",
            "m_per_block": prob.m_per_block,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "kernel": f"sk_attn_partial (partial_bf16_kernel<192,128> in {prob.m_per_block}-row workgroups, then "
                      f"merge_pieces_kernel<{prob.m_per_block},128> for the last round's key pieces)",
            "kernel_ms": t_partial,
            "algorithmic_flop": flops,
            "algorithmic_bytes": partial_bytes,
        },
        "combine": {
            "bound": "hbm",
            "ms_in_pipeline": t_combine,
            "ms_cold_cache": t_combine_cold,
            "algorithmic_bytes": combine_bytes,
            "gbps_in_pipeline": combine_bytes / (t_combine * 1e-3) / 1e9,
            "gbps_cold_cache": combine_bytes / (t_combine_cold * 1e-3) / 1e9,
            "frac_cold_cache": combine_bytes / (t_combine_cold * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "frac_in_pipeline": combine_bytes / (t_combine * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "peak": PEAK_HBM_GBPS,
            "ms_cold_launch_floor": t_launch_floor,
            "ms_cold_back_to_back": t_combine_cold_b2b,
            "frac_cold_back_to_back": combine_bytes / (t_combine_cold_b2b * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "cold_back_to_back_launches": COLD_COPIES,
        },
        "counts_ms": t_counts,
        "unsplit": unsplit,
        "attention_tflops_partial_plus_combine": flops / ((t_partial + t_combine) * 1e-3) / 1e12,
        "backward": backward,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, inputs, prob.m_per_block)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
