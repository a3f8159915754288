#!/usr/bin/env python3
"""Benchmark of the fused QSA decode step on one MI355X.

One step = one qsa_decode call = block scoring, top-k block selection, the
position buffer and gather attention for the whole batch of one QSA layer.
Inputs are resident in HBM before timing starts.  To measure HBM rather than
the 256 MB last-level cache, R identical copies of every input are rotated so
that the calls of a rotation touch at least 1 GiB of distinct bytes, and when
the K timed calls touch less than 1 GiB in all, every timed replay starts after
1 GiB of other memory has been written.  The K timed calls are captured in one
HIP graph and bracketed by HIP events.  The workload the metric is quoted on
(50,000-token MTP verify at batch 1) is the headline; the batch-32 FP8
workload, the 1M-token context and the 8K, 262K (BF16 and FP8, tied scores) and
ragged 64-request batches are reported beside it, each with the roofline of its
dominant kernel.  The CPU oracle on the headline workload is timed first, on
one thread and on all host cores.

Prints one JSON line (see the keys below); human-readable detail goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "qsa_decode steps/sec at 50K ctx (B=1,32) + achieved HBM GB/s vs peak"
HBM_PEAK_GBPS = 8000.0
K_TOP = 512
WIDTH = 4 * K_TOP + 3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ byte counts
def query_geometry(w):
    """(request, L, nf, n_pos) for every query."""
    out = []
    for r in range(w.num_req):
        nq = int(w.q_start[r + 1] - w.q_start[r])
        for j in range(nq):
            L = int(w.seq_len[r]) - nq + 1 + j
            nf = L // 4
            out.append((r, L, nf, 4 * min(nf, K_TOP) + L % 4))
    return out


def algorithmic_bytes(w) -> dict:
    """Compulsory HBM bytes per call: every compressed key once per request, the
    gathered K and V rows, index query, attention query and FP32 output.  The
    FP32 score buffer and position buffer round trips are listed per kernel."""
    e = 2 if w.kv_dtype == "bf16" else 1
    hq, hkv = w.num_q_heads, w.num_kv_heads
    geo = query_geometry(w)
    keys = 256 * int(sum(int(s) // 4 for s in w.seq_len))
    kv = sum(n * hkv * 128 * 2 * e for (_, _, _, n) in geo)
    step = keys + kv + w.num_q * (256 + hq * 256 + hq * 512)
    nblk_q = sum(int(w.seq_len[r]) // 4 for (r, _, _, _) in geo)
    score = keys + 256 * w.num_q + 4 * nblk_q
    select = sum(4 * nf for (_, _, nf, _) in geo if nf > K_TOP) + w.num_q * 4 * (K_TOP + WIDTH)
    attn = kv + w.num_q * (hq * 256 + hq * 512) + sum(4 * n for (_, _, _, n) in geo)
    return {"step": step, "score": score, "select": select, "attn": attn}


# ------------------------------------------------------------------ GPU timing
class Rig:
    """R rotating device copies of one workload plus the library handles."""

    def __init__(self, w, copies: int):
        import torch
        import block_sparse_attention_qsa_amd as qsa
        from workloads.device import upload
        self.torch, self.qsa, self.w = torch, qsa, w
        base = upload(w)
        self.copies = [base]
        for _ in range(copies - 1):
            self.copies.append({k: (v.clone() if v is not None else None) for k, v in base.items()})
        self.batch = qsa.Batch(w.q_start, w.seq_len, w.kv_start, w.blk_start)
        hq = w.num_q_heads
        self.outs = [torch.empty((w.num_q, hq, 128), dtype=torch.float32, device="cuda") for _ in self.copies]
        self.ws = qsa.alloc_workspace(self.batch, hq, w.num_kv_heads)
        self.sm = 1.0 / math.sqrt(128)
        # stage inputs for the per-kernel timings
        self.scores = torch.zeros((w.num_q, max(self.batch.max_blocks, 1)), dtype=torch.float32, device="cuda")
        self.sel = torch.empty((w.num_q, K_TOP), dtype=torch.int32, device="cuda")
        self.n_sel = torch.empty((w.num_q,), dtype=torch.int32, device="cuda")
        self.pos = torch.empty((w.num_q, WIDTH), dtype=torch.int32, device="cuda")
        self.n_pos = torch.empty((w.num_q,), dtype=torch.int32, device="cuda")
        self.attn_ws = qsa.alloc_workspace(self.batch, hq, w.num_kv_heads)
        self.sel_ws = qsa.alloc_workspace(self.batch, 1, 1)

    def decode(self, i):
        c = self.copies[i % len(self.copies)]
        self.qsa.qsa_decode(self.batch, c["idx_q"], c["ckeys"], c["q"], c["k_cache"], c["v_cache"],
                            self.outs[i % len(self.copies)], self.ws, k_scale=c["k_scale"],
                            v_scale=c["v_scale"], sm_scale=self.sm)

    def prepare_stage_inputs(self):
        c = self.copies[0]
        self.qsa.qsa_score(self.batch, c["idx_q"], c["ckeys"], self.scores)
        self.qsa.qsa_select_topk(self.batch, self.scores, self.sel, self.n_sel, workspace=self.sel_ws)
        self.qsa.qsa_build_index(self.batch, self.sel, self.n_sel, self.pos, self.n_pos)
        self.torch.cuda.synchronize()

    def stage(self, name, i):
        c = self.copies[i % len(self.copies)]
        if name == "score":
            self.qsa.qsa_score(self.batch, c["idx_q"], c["ckeys"], self.scores)
        elif name == "select":
            # selection and positions in one launch, the kernel qsa_decode runs
            self.qsa.qsa_select_positions(self.batch, self.scores, self.sel, self.n_sel, self.pos, self.n_pos,
                                          workspace=self.sel_ws)
        elif name == "attn":
            self.qsa.qsa_sparse_attn(self.batch, c["q"], c["k_cache"], c["v_cache"], self.pos, self.n_pos,
                                     self.outs[i % len(self.copies)], k_scale=c["k_scale"], v_scale=c["v_scale"],
                                     sm_scale=self.sm, workspace=self.attn_ws)
        else:
            raise KeyError(name)

    def timed_graph(self, fn, steps: int, warmup: int, reps: int = 5, flush: bool = False):
        """Capture `steps` calls of fn(i) in a HIP graph; return (median ms per
        call over reps replays, wall-clock ms per call of the last replay).
        With flush, every timed replay is preceded (outside the timed region)
        by writes to 1 GiB of other memory, so that calls which together touch
        less than the last-level cache still start from HBM."""
        torch = self.torch
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                fn(i)
        torch.cuda.synchronize()
        g.replay()                      # untimed first replay
        torch.cuda.synchronize()
        sink = torch.empty(1 << 28, dtype=torch.float32, device="cuda") if flush else None
        times = []
        wall = None
        for _ in range(reps):
            if flush:
                sink.zero_()
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            start.record()
            g.replay()
            end.record()
            torch.cuda.synchronize()
            wall = (time.perf_counter() - t0) * 1e3 / steps
            times.append(start.elapsed_time(end) / steps)
        del g, sink
        return float(np.median(times)), wall


def rotation_copies(w, touched: int, limit_bytes: float = 80e9) -> int:
    per_copy = (w.k_cache.nbytes + w.v_cache.nbytes + w.ckeys.nbytes + w.q.nbytes + w.idx_q.nbytes)
    want = max(1, math.ceil((1 << 30) / max(touched, 1)))
    return int(max(1, min(want, limit_bytes // max(per_copy, 1))))


def measure(name: str, steps: int, warmup: int, kernels: bool = True) -> dict:
    from workloads import make_workload
    t0 = time.perf_counter()
    w = make_workload(name)
    log(f"[{name}] generated in {time.perf_counter() - t0:.1f}s: {w.num_req} requests, {w.num_q} queries")
    nbytes = algorithmic_bytes(w)
    R = rotation_copies(w, nbytes["step"])
    rig = Rig(w, R)
    # the timed calls rotate over the copies; when they touch less than 1 GiB
    # in all, each timed replay starts after a cache flush
    flush = steps * nbytes["step"] < (1 << 30)
    log(f"[{name}] {R} rotating copies, {nbytes['step'] / 1e6:.2f} MB algorithmic per step"
        f"{', cache flushed before each timed replay' if flush else ''}")
    ms, wall_ms = rig.timed_graph(rig.decode, steps, warmup, flush=flush)
    gbps = nbytes["step"] / (ms * 1e-3) / 1e9
    log(f"[{name}] qsa_decode: {ms * 1e3:.2f} us/step (graph, events), wall {wall_ms * 1e3:.2f} us/step, "
        f"{gbps:.0f} GB/s = {gbps / HBM_PEAK_GBPS:.1%} of HBM peak")
    res = {"workload": name, "w": w, "copies": R, "max_blocks": rig.batch.max_blocks, "flushed": flush,
           "ms_per_step": ms, "wall_ms_per_step": wall_ms,
           "steps_per_s": 1e3 / ms, "step_bytes": nbytes["step"], "step_gbps": gbps, "kernels": {}}
    if kernels:
        rig.prepare_stage_inputs()
        for st in ("score", "select", "attn"):
            kflush = steps * nbytes[st] < (1 << 30)
            kms, _ = rig.timed_graph(lambda i, st=st: rig.stage(st, i), steps, warmup, flush=kflush)
            kg = nbytes[st] / (kms * 1e-3) / 1e9
            res["kernels"][st] = {"us": kms * 1e3, "bytes": nbytes[st], "gbps": kg}
            log(f"[{name}]   {st:6s}: {kms * 1e3:8.2f} us/launch, {nbytes[st] / 1e6:8.3f} MB, {kg:7.0f} GB/s")
    del rig
    import torch
    torch.cuda.empty_cache()
    return res


KERNEL_NAMES = {"score": "qsa::score_kernel", "select": "qsa::select_reg_kernel", "attn": "qsa::attn_kernel"}
# rows over 32,768 blocks take the two-launch top-k (slices, then their candidates)
LONG_SELECT_NAME = "qsa::select_slice_kernel + qsa::select_cand_kernel (2 launches)"
LONG_ROW_BLOCKS = 32768


def _long_select(kernel: str) -> bool:
    """One of the two launches of the top-k for rows over 32,768 blocks."""
    return "select_slice_kernel" in kernel or "select_cand_kernel" in kernel
CSRC = os.path.join(ROOT, "block_sparse_attention_qsa_amd", "csrc")


def _code_text(src: bytes) -> bytes:
    """Source text without /* */ and // comments, trailing blanks and empty
    lines: edits to comments leave the hash (and the counters tied to it)
    valid."""
    import re
    src = re.sub(rb"/\*.*?\*/", b"", src, flags=re.S)
    lines = (re.sub(rb"//.*$", b"", l).rstrip() for l in src.splitlines())
    return b"\n".join(l for l in lines if l)


def kernel_source_hash(read=None) -> str:
    """sha256 over the code of every HIP source and header of the library
    (sorted by name) and the public header, comments stripped."""
    import hashlib
    if read is None:
        def read(rel):
            with open(os.path.join(ROOT, rel), "rb") as f:
                return f.read()
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp", ".h")):
            h.update(name.encode() + b"\0" + _code_text(read(f"block_sparse_attention_qsa_amd/csrc/{name}")))
    h.update(_code_text(read("include/qsa.h")))
    return h.hexdigest()


def roofline_of(res: dict, traffic: dict | None) -> dict:
    """Roofline of the dominant kernel.  `traffic` is HBM bytes per launch from
    rocprofv3 FETCH_SIZE + WRITE_SIZE counters (each scaled by what the counter
    reads for a 1 GiB device copy), taken only while the library's sources are
    unchanged since the counters were collected."""
    ks = res["kernels"]
    dom = max(ks, key=lambda s: ks[s]["us"])
    k = ks[dom]
    tr = None
    name = KERNEL_NAMES[dom]
    if dom == "select" and res.get("max_blocks", 0) > LONG_ROW_BLOCKS:
        name = LONG_SELECT_NAME
    key = f"{name}@{res['workload']}"
    if traffic and key in traffic.get("entries", {}) and traffic.get("source_sha256") == kernel_source_hash():
        tr = traffic["entries"][key]["bytes_per_launch"]
    return {"kernel": name, "bound": "hbm", "achieved": round(k["gbps"], 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(k["gbps"] / HBM_PEAK_GBPS, 4), "traffic": tr,
            "algorithmic_bytes_per_launch": k["bytes"], "avg_launch_us": round(k["us"], 3)}


def calibrate_copy(gib: int = 1, reps: int = 3) -> None:
    """A plain device-to-device copy of known size, for scaling memory counters."""
    import torch
    src = torch.empty(gib << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[calibrate] copied {gib} GiB x {reps}")
    del src, dst
    torch.cuda.empty_cache()


def stream_ceiling(gib: int = 1, reps: int = 7) -> dict:
    """Measured context for the roofline on `gib` GiB of zero-filled device
    memory: a streaming read (the probe library's whole-line non-temporal
    read kernel, 4,096 workgroups) and torch's device-to-device copy (bytes
    read + written per second), each the median of `reps` event-timed runs."""
    import ctypes

    import torch
    from block_sparse_attention_qsa_amd.build import PROBE_LIB
    probe = ctypes.CDLL(PROBE_LIB)
    probe.qsa_probe_stream_read.restype = ctypes.c_int
    probe.qsa_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                            ctypes.c_void_p]
    src = torch.zeros(gib << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def read():
        rc = probe.qsa_probe_stream_read(src.data_ptr(), src.numel() * 4, sink.data_ptr(), 4096,
                                         torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"stream-read probe failed: hipError {rc}")

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            times.append(a.elapsed_time(b) * 1e-3)
        return sorted(times)[reps // 2]

    nbytes = gib << 30
    read_gbps = nbytes / timed(read) / 1e9
    copy_gbps = 2 * nbytes / timed(lambda: dst.copy_(src)) / 1e9
    del src, dst, sink
    torch.cuda.empty_cache()
    return {"read_gbps": round(read_gbps, 1), "read_frac_of_peak": round(read_gbps / HBM_PEAK_GBPS, 4),
            "copy_gbps": round(copy_gbps, 1),
            "kind": f"streaming read of {gib} GiB (probe kernel); torch copy ({gib} GiB read + {gib} GiB written)"}


# ------------------------------------------------------------------ profile summaries
PROFILE_WORKLOADS = ("mtp50k", "mtp50k_b32_fp8", "mtp1m", "single8k", "mtp262k_ties", "mtp262k_ties_fp8", "ragged64")
# run from /tmp with TMPDIR=/tmp; REPO is the repository root
PROF_STATS_CMD = ("rocprofv3 --kernel-trace --stats -d {d}/stats_{W} -o qsa --output-format csv -- "
                  "python -u $REPO/bench.py --config {W} --b32 none --long none --legs none --steps 200 --warmup 20 "
                  "--cpu-seconds 0")
PROF_PMC_CMD = ("rocprofv3 --pmc {C} --kernel-trace -d {d}/pmc_{C}_{W} -o qsa --output-format csv -- "
                "python -u $REPO/bench.py --config {W} --b32 none --long none --legs none --steps 10 --warmup 2 "
                "--cpu-seconds 0 --no-kernels --calibrate-copy")


def _stage_of(kernel: str):
    if "attn_kernel" in kernel:
        return "attn"
    if "score_kernel" in kernel:
        return "score"
    if "select_reg_kernel" in kernel or _long_select(kernel):
        return "select"
    return None


def summarize_profiles(prof_dir: str, out_dir: str) -> None:
    """Turn the rocprofv3 CSV output of PROF_STATS_CMD and PROF_PMC_CMD (one
    directory per workload and counter under prof_dir) into one markdown
    summary per workload and traffic.json under out_dir.  The memory counters
    are scaled by what they read for the 1 GiB device copy of --calibrate-copy;
    the two launches of the long-row top-k are summed into one entry."""
    import collections
    import csv
    from workloads import make_workload

    def rows(path):
        with open(path) as f:
            return list(csv.DictReader(f))

    traffic = {"source_sha256": kernel_source_hash(), "entries": {}}
    for W in PROFILE_WORKLOADS:
        stats_csv = os.path.join(prof_dir, f"stats_{W}", "qsa_kernel_stats.csv")
        if not os.path.exists(stats_csv):
            log(f"[summarize] no profile for {W}")
            continue
        pmc = {}
        for C in ("FETCH_SIZE", "WRITE_SIZE"):
            agg = collections.defaultdict(list)
            for r in rows(os.path.join(prof_dir, f"pmc_{C}_{W}", "qsa_counter_collection.csv")):
                agg[r["Kernel_Name"].split("(")[0]].append(float(r["Counter_Value"]))
            pmc[C] = agg
        copy = "__amd_rocclr_copyBuffer"
        cf, cw = 1048576.0 / max(pmc["FETCH_SIZE"][copy]), 1048576.0 / max(pmc["WRITE_SIZE"][copy])
        alg = algorithmic_bytes(make_workload(W))
        line = {}
        log_path = os.path.join(prof_dir, f"stats_{W}.log")
        if os.path.exists(log_path):
            with open(log_path) as f:
                js = [l for l in f if l.startswith("{")]
            line = json.loads(js[-1]) if js else {}
        fmt = dict(d=prof_dir, W=W)
        out = [f"# rocprofv3 summary: QSA kernels on `{W}`", "",
               f"MI355X (gfx950), one GPU.  Library code sha256 (comments stripped) `{traffic['source_sha256'][:16]}`.", "",
               "## Kernel trace statistics", "", "```", PROF_STATS_CMD.format(**fmt), "```", "",
               "| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
        for r in rows(stats_csv):
            n = r["Name"].split("(")[0]
            if "qsa::" in n or "copyBuffer" in n:
                out.append(f"| `{n}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                           f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} | "
                           f"{float(r['Percentage']):.2f} |")
        if line:
            out += ["", f"bench.py in the same run (HIP events around graph replays): step "
                        f"{line['ms_per_step'] * 1e3:.2f} us, per kernel {line.get('kernels_us')} us."]
        out += ["", "## HBM traffic (memory counters, fused qsa_decode only)", "", "```",
                PROF_PMC_CMD.format(C="FETCH_SIZE", **fmt), PROF_PMC_CMD.format(C="WRITE_SIZE", **fmt),
                f"python bench.py --summarize-profiles {prof_dir}", "```", "",
                f"Calibration: a 1 GiB device copy reads FETCH_SIZE {max(pmc['FETCH_SIZE'][copy]):.1f} KiB and "
                f"WRITE_SIZE {max(pmc['WRITE_SIZE'][copy]):.1f} KiB per dispatch: scale factors {cf:.4f} (FETCH) "
                f"and {cw:.4f} (WRITE).", "",
                "| kernel | dispatches | FETCH KiB | WRITE KiB | scaled HBM MB / launch | algorithmic MB / launch "
                "| ratio |", "|---|---|---|---|---|---|---|"]
        summed = collections.defaultdict(lambda: [0.0, 0.0, 0.0])
        for n in sorted(pmc["FETCH_SIZE"]):
            st = _stage_of(n)
            if st is None:
                continue
            fv, wv = pmc["FETCH_SIZE"][n], pmc["WRITE_SIZE"].get(n, [0.0])
            fk, wk = sum(fv) / len(fv), sum(wv) / len(wv)
            tot = (fk * cf + wk * cw) * 1024
            out.append(f"| `{n}` | {len(fv)} | {fk:.1f} | {wk:.1f} | {tot / 1e6:.3f} | "
                       f"{alg[st] / 1e6 if not _long_select(n) else float('nan'):.3f} | "
                       f"{tot / alg[st] if not _long_select(n) else float('nan'):.3f} |")
            key = LONG_SELECT_NAME if _long_select(n) else KERNEL_NAMES[st]
            acc = summed[key]
            acc[0] += fk
            acc[1] += wk
            acc[2] += tot
        for key, (fk, wk, tot) in summed.items():
            st = [s for s in KERNEL_NAMES if KERNEL_NAMES[s] == key or (key == LONG_SELECT_NAME and s == "select")][0]
            if key == LONG_SELECT_NAME:
                out.append(f"| {key}, summed | | {fk:.1f} | {wk:.1f} | {tot / 1e6:.3f} | {alg[st] / 1e6:.3f} | "
                           f"{tot / alg[st]:.3f} |")
            traffic["entries"][f"{key}@{W}"] = {"bytes_per_launch": int(round(tot)), "fetch_kib": fk,
                                                "write_kib": wk, "fetch_scale": cf, "write_scale": cw,
                                                "algorithmic_bytes": alg[st]}
        with open(os.path.join(out_dir, f"qsa_kernels__{W}.md"), "w") as f:
            f.write("\n".join(out) + "\n")
        log(f"[summarize] {W}: wrote qsa_kernels__{W}.md")
    with open(os.path.join(out_dir, "traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)


# ------------------------------------------------------------------ CPU baseline
_CPU_W = None


def _oracle_args(w):
    return (w.q_start, w.seq_len, w.kv_start, w.blk_start, w.idx_q, w.ckeys, w.q, w.k_cache, w.v_cache,
            w.kv_dtype, w.k_scale, w.v_scale)


def _cpu_worker_init(name):
    """Each worker process of the all-cores leg: one BLAS thread, its own
    copy of the workload."""
    global _CPU_W
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)
    from workloads import make_workload
    _CPU_W = make_workload(name)


def _cpu_worker_run(seconds):
    """Full oracle steps for about `seconds`; returns (steps, elapsed)."""
    import oracle
    args = _oracle_args(_CPU_W)
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.decode(*args, sm_scale=1.0 / math.sqrt(128), want_scores=False)
        n += 1
        if time.perf_counter() - t0 >= seconds:
            return n, time.perf_counter() - t0


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(name: str, seconds: float) -> dict:
    """The CPU oracle on full steps of the workload, median of 3 runs each:
    on one thread, and on every host core available (one process per core,
    one BLAS thread each, all running steps at once; steps/s is their sum).
    Runs before the GPU is touched (the worker processes are forked)."""
    import multiprocessing as mp
    import oracle
    from threadpoolctl import threadpool_limits
    from workloads import make_workload
    w = make_workload(name)
    args = _oracle_args(w)
    per = max(seconds / 6.0, 0.5)
    single = []
    with threadpool_limits(limits=1):
        for _ in range(3):
            n, t0 = 0, time.perf_counter()
            while True:
                oracle.decode(*args, sm_scale=1.0 / math.sqrt(128), want_scores=False)
                n += 1
                if time.perf_counter() - t0 >= per:
                    break
            single.append(n / (time.perf_counter() - t0))
    cores = len(os.sched_getaffinity(0))
    multi = []
    ctx = mp.get_context("fork")
    with ctx.Pool(cores, initializer=_cpu_worker_init, initargs=(name,)) as pool:
        for _ in range(3):
            res = pool.map(_cpu_worker_run, [per] * cores)
            multi.append(sum(n / dt for n, dt in res))
    v1, vn = float(np.median(single)), float(np.median(multi))
    model = cpu_model()
    log(f"[cpu] oracle on {name}: {v1:.2f} steps/s on 1 thread, {vn:.2f} steps/s on {cores} cores ({model})")
    return {"value": round(vn, 4), "unit": "steps/s", "cores": cores, "kind": "oracle",
            "sample": f"full {name} steps ({w.num_q} queries each), median of 3 runs of about {per:.1f} s: "
                      f"{cores} processes with one BLAS thread each, steps/s summed; "
                      f"{os.cpu_count()} CPUs in the host, {cores} available to the run",
            "cpu_model": model,
            "single_core": {"value": round(v1, 4), "unit": "steps/s", "cores": 1}}


LEG_STEPS = {"mtp50k_b32_fp8": 200, "mtp1m": 100, "single8k": 1000, "mtp262k_ties": 300, "mtp262k_ties_fp8": 300,
             "ragged64": 300}
LEG_KEYS = {"mtp50k_b32_fp8": "b32", "mtp1m": "long"}


def leg_line(r: dict, w, traffic) -> dict:
    d = {"workload": r["workload"], "steps_per_s": round(r["steps_per_s"], 2),
         "ms_per_step": round(r["ms_per_step"], 6), "step_gbps": round(r["step_gbps"], 1),
         "step_frac_of_peak": round(r["step_gbps"] / HBM_PEAK_GBPS, 4),
         "kernels_us": {k: round(v["us"], 3) for k, v in r["kernels"].items()},
         "requests": w.num_req, "queries": w.num_q, "seq_len": int(w.seq_len.max()), "kv_dtype": w.kv_dtype,
         "rotation_copies": r["copies"], "cache_flushed": r["flushed"]}
    if r["kernels"]:
        d["roofline"] = roofline_of(r, traffic)
    return d


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="mtp50k")
    ap.add_argument("--b32", default="mtp50k_b32_fp8", help="the batch-32 workload reported beside (or 'none')")
    ap.add_argument("--b32-steps", type=int, default=LEG_STEPS["mtp50k_b32_fp8"])
    ap.add_argument("--long", default="mtp1m", help="long-context workload reported beside (or 'none')")
    ap.add_argument("--long-steps", type=int, default=LEG_STEPS["mtp1m"])
    ap.add_argument("--legs", default="single8k,mtp262k_ties,mtp262k_ties_fp8,ragged64",
                    help="further workloads reported under 'legs' (comma list, or 'none')")
    ap.add_argument("--cpu-seconds", type=float, default=18.0)
    ap.add_argument("--no-kernels", action="store_true", help="skip the per-kernel timings")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM traffic per launch measured by rocprofv3 counters")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a 1 GiB device copy (reference for memory-counter scaling)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="no GPU: summarize rocprofv3 output under DIR into profiles/ and exit")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, os.path.join(ROOT, "profiles"))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    # the CPU baseline first: its worker processes fork before the GPU is touched
    cpu = cpu_baseline(args.config, args.cpu_seconds) if args.cpu_seconds > 0 else None

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import block_sparse_attention_qsa_amd as qsa
    qsa.lib()
    if args.calibrate_copy:
        calibrate_copy()

    res = measure(args.config, args.steps, args.warmup, kernels=not args.no_kernels)
    w = res.pop("w")
    traffic = None
    if os.path.exists(args.traffic):
        with open(args.traffic) as f:
            traffic = json.load(f)
    line = {
        "metric": METRIC, "value": round(res["steps_per_s"], 2), "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.kv_dtype == "bf16" else "bf16+fp8kv", "data": "synthetic",
        "config": {"workload": args.config, "requests": w.num_req, "queries": w.num_q,
                   "seq_len": int(w.seq_len.max()), "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                   "kv_dtype": w.kv_dtype, "topk": K_TOP, "rotation_copies": res["copies"],
                   "cache_flushed": res["flushed"]},
        "step_gbps": round(res["step_gbps"], 1), "step_frac_of_peak": round(res["step_gbps"] / HBM_PEAK_GBPS, 4),
        "wall_ms_per_step": round(res["wall_ms_per_step"], 6),
        "kernels_us": {k: round(v["us"], 3) for k, v in res["kernels"].items()},
    }
    if res["kernels"]:
        line["roofline"] = roofline_of(res, traffic)
    del w
    legs = []
    if args.b32 != "none":
        legs.append((args.b32, args.b32_steps, "b32"))
    if args.long != "none":
        legs.append((args.long, args.long_steps, "long"))
    if args.legs != "none":
        for nm in [x for x in args.legs.split(",") if x]:
            legs.append((nm, LEG_STEPS.get(nm, 200), None))
    for nm, st, key in legs:
        r = measure(nm, st, min(args.warmup, 20), kernels=not args.no_kernels)
        wl = r.pop("w")
        d = leg_line(r, wl, traffic)
        if key:
            line[key] = d
        else:
            line.setdefault("legs", {})[nm] = d
        del wl
    if not args.no_kernels:
        line["stream_ceiling"] = stream_ceiling()
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
