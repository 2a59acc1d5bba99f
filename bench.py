#!/usr/bin/env python3
"""Benchmark: one pass of the UniPrefill pruning path on MI355X.

A step is the whole hot path over one packed batch already resident in HBM:
up_score (tail-query scores + block means) -> up_select_topp (Top-p mask) ->
up_compact_record (gather of kept rows, and the ledger append in the same
copy launch: up_compact + up_drop_history in one call).

Default workload: Llama-3.1-8B-shaped full-attention layer, one request of
L = 131072 tokens, 32 q / 8 KV heads, head_dim 128, hidden 4096 bf16, n=128,
G=64, p=0.99, 128 sink / 128 tail tokens, 5% planted blocks (seeded).

Prints ONE JSON line (rank 0).  Besides the required fields it reports the
roofline of the dominant kernel (HIP events on the stream the kernels run
on), a per-call time breakdown, the scoring kernels' MFMA fraction, and the
plain C++ CPU oracle timed on one pinned host core on a bounded sample of the
same input bytes, and a full-size parity check of the GPU result against the
numpy oracle.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s of score+select+compact at L=128K; % MFMA peak, % HBM peak"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "token_block_sparsification_amd", "csrc")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama8b_L131072")
    ap.add_argument("--tail", type=int, default=None,
                    help="override the always-kept tail tokens (-1: the workload's n_query)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle leg (for profiler runs)")
    ap.add_argument("--cpu-threads", type=int, default=1,
                    help="BLAS threads of the numpy oracle in the full-size parity check")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 1 GiB device copy (the reference for counter scaling)")
    ap.add_argument("--stack", action="store_true",
                    help="instead of the path step, time a synthetic hybrid stack (random weights) "
                         "with and without pruning and print its own JSON line")
    ap.add_argument("--stack-top-p", default="0.99,0.9,0.7",
                    help="comma-separated top_p values for --stack")
    ap.add_argument("--stack-len", type=int, default=32768, help="tokens of the --stack request")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of a "
                         "--copy-probe run into profiles/traffic.json and exit")
    return ap.parse_args()


def source_sha(names) -> str:
    """Hash of the source file(s) a kernel is built from."""
    h = hashlib.sha256()
    for name in ([names] if isinstance(names, str) else names):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, src: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs of this
    workload, or None when they were taken on another workload or the
    kernel's source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != source_sha(src) or rec.get("workload") != workload:
        return None
    return rec.get("bytes_per_launch")


COPY_BYTES = 1 << 30
EVENT_EVERY = 10  # timed steps per bracketed dominant call
# name in traffic.json -> (source file, pattern of the dispatch names it covers)
TRAFFIC_KERNELS = {
    "up_compact_copy_kernel": ("up_compact.hip", r"\bup_compact_copy_kernel<\d+, false>"),
    "up_revive_copy_kernel": ("up_compact.hip", r"\bup_compact_copy_kernel<\d+, true>"),
    "up_compact_scan_kernel": ("up_compact.hip", r"\bup_compact_scan_kernel\b"),
    "up_rowstats_kernel": ("up_score.hip", r"\bup_rowstats_kernel\b"),
    "up_colsum_kernel": ("up_score.hip", r"\bup_colsum_kernel\b"),
    "up_select_kernel": (("up_select.hip", "up_select_impl.h", "up_wave.h"), r"\bup_select_kernel\b"),
    "up_rowop_kernel_norm": ("up_compact.hip", r"\bup_rowop_kernel<0, "),
    "up_rowop_kernel_add": ("up_compact.hip", r"\bup_rowop_kernel<1, "),
}


def write_traffic(fetch_csv: str, write_csv: str, workload: str) -> None:
    """HBM bytes per dispatch of the path's kernels from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by the factor that makes the plain copy of
    COPY_BYTES read and write exactly COPY_BYTES."""
    import csv
    import re
    from collections import defaultdict

    def load(path, counter):
        per = defaultdict(list)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            per[name].append(float(r["Counter_Value"]) * 1024.0)
        return per

    out = {}
    for counter, path, key in (("FETCH_SIZE", fetch_csv, "fetch"), ("WRITE_SIZE", write_csv, "write")):
        per = load(path, counter)
        # the probe is the runtime's device-to-device copy of COPY_BYTES (the
        # largest such copy in the run); torch's dtype-conversion kernels also
        # carry "copy" in their names and are not it
        copies = [max(v) for n, v in per.items() if "copyBuffer" in n]
        if not copies:
            raise SystemExit(f"no copy kernel in {path}")
        scale = COPY_BYTES / max(copies)
        for short, (src, pat) in TRAFFIC_KERNELS.items():
            vals = [x for n, v in per.items() if re.search(pat, n) for x in v]
            if not vals:
                continue
            rec = out.setdefault(short, {"source_sha": source_sha(src), "workload": workload,
                                         "source": src if isinstance(src, str) else "+".join(src)})
            rec[key + "_bytes_per_launch"] = sum(vals) / len(vals) * scale
            rec[key + "_scale"] = scale
            rec[key + "_raw_kib_per_launch"] = sum(vals) / len(vals) / 1024.0
    for rec in out.values():
        rec["bytes_per_launch"] = rec.get("fetch_bytes_per_launch", 0.0) + rec.get("write_bytes_per_launch", 0.0)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print(json.dumps(out, indent=1))


def main():
    args = parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic, args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py: the path runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the head-parallel design is described, not built)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import token_block_sparsification_amd as U
    import workloads as W

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU (no HIP device visible)")
    U.lib()  # fail loudly if the HIP library is not built
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.stack:
        stack_bench(args, dev)
        return

    w = W.get_workload(args.workload)
    if args.tail is not None:
        w = w.with_(tail=args.tail if args.tail >= 0 else w.n_query)
    t_gen = time.perf_counter()
    inp = W.make_inputs(w, device=dev)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen

    batch = U.Batch.make(inp["cu_seqlens"], w.block, dev)
    q, k, hidden, pos = inp["q"], inp["k"], inp["hidden"], inp["positions"]
    ws = U.Workspace.make(batch, w.hq, w.hkv, w.head_dim, w.n_query, hidden, dev)
    cap = 64
    ledger = torch.empty(U.up_history_bytes(batch.num_seqs, cap) // 4, dtype=torch.int32,
                         device=dev)
    U.up_history_init(ledger, batch.num_seqs, cap)
    T, N, B = batch.num_tokens, batch.num_blocks, batch.num_seqs

    calls = ["up_score", "up_select_topp", "up_compact_record"]

    def step(layer=0, marks=None):
        """One pass of the path.  marks: {call: (start, end) HIP events} for
        the calls to bracket (events are recorded on the current stream, the
        one the library launches on)."""
        def run(name, fn):
            if marks and name in marks:
                marks[name][0].record()
            fn()
            if marks and name in marks:
                marks[name][1].record()
        run("up_score", lambda: U.up_score(
            batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, q, k, w.n_query, w.block,
            0.0, ws.token_scores, ws.block_scores, ws.score_ws))
        run("up_select_topp", lambda: U.up_select_topp(
            batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, ws.block_scores, w.block,
            w.top_p, w.sink, w.tail, ws.block_mask, ws.kept_tokens))
        copy_ev = marks.get("copy_kernel") if marks else None
        if copy_ev:   # the library records these right around its copy kernel
            U.up_set_copy_events(*copy_ev)
        run("up_compact_record", lambda: U.up_compact_record(
            batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, w.block, ws.block_mask,
            hidden, pos, ws.hidden_out, ws.positions_out, ws.cu_seqlens_out, ws.compact_ws,
            ledger, cap, layer % cap))
        if copy_ev:
            U.up_set_copy_events(None, None)

    def new_marks(names):
        m = {n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for n in names}
        if "copy_kernel" in m:   # handed to the library: create the HIP events now
            for e in m["copy_kernel"]:
                e.record()
        return m

    def mean_us(marks_list, name):
        return float(np.mean([m[name][0].elapsed_time(m[name][1]) for m in marks_list])) * 1e3

    def med_us(marks_list, name):
        """Median: the side measurements below are robust to one host stall
        (the GPU idles inside an event bracket while the host is held up)."""
        return float(np.median([m[name][0].elapsed_time(m[name][1]) for m in marks_list])) * 1e3

    # No garbage-collector pauses while anything is timed.
    gc.collect()
    gc.disable()

    # Warm-up (untimed).
    for i in range(args.warmup):
        step(layer=i)
        U.up_history_init(ledger, B, cap)
    if args.copy_probe:
        src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        del src, dst
    torch.cuda.synchronize()
    kept = int(ws.cu_seqlens_out[-1].item())

    # Timed region: K steps; on every EVENT_EVERY-th step the two large
    # pieces are bracketed by events: the up_score call, and the compaction
    # copy kernel alone (events the library records right around its launch,
    # up_set_copy_events); the larger of them over the timed region is the
    # dominant one.  Each event record leaves the GPU idle for ~5 us, so
    # bracketing every step would add ~11 us per piece bracketed; one step in
    # ten adds ~2 us per step on average and still averages 10 launches of
    # each piece over a 100-step run.
    K = args.steps
    big = ("up_score", "copy_kernel")
    sampled = [i for i in range(K) if i % EVENT_EVERY == 0]
    timed_marks = {i: new_marks(list(big)) for i in sampled}
    U.up_history_init(ledger, B, cap)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(layer=i, marks=timed_marks.get(i))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    timed_marks = [timed_marks[i] for i in sampled]
    dominant = max(big, key=lambda n: mean_us(timed_marks, n))
    dominant_us = mean_us(timed_marks, dominant)
    dom_all = [m[dominant][0].elapsed_time(m[dominant][1]) * 1e3 for m in timed_marks]

    # Per-call breakdown from extra steps outside the timed region.
    nb = min(K, 20)
    brk = [new_marks(calls) for _ in range(nb)]
    for i in range(nb):
        step(layer=K + i, marks=brk[i])
    torch.cuda.synchronize()

    # Cold-cache chains: before each, 512 MiB of scratch writes evict K and
    # the hidden rows from L2 and the Infinity Cache; then one bracketed step.
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for i in range(nb):
        flush.fill_(i & 0xFF)
        m = new_marks(["chain"])
        m["chain"][0].record()
        step(layer=K + nb + i)
        m["chain"][1].record()
        cold.append(m)
    torch.cuda.synchronize()
    cold_us = sorted(m["chain"][0].elapsed_time(m["chain"][1]) * 1e3 for m in cold)
    del flush

    # Neighbours of the path, timed outside the timed region: revival (the
    # packed rows written back over the full buffer; here they are unchanged,
    # so `hidden` keeps its bytes) and the ledger read-back.
    kv_len = torch.empty(max(B, 1), dtype=torch.int32, device=dev)
    # Each side loop below runs one extra, discarded first iteration: a
    # first call can stall the host (lazy kernel loading) inside its events.
    rv_marks = []
    for i in range(nb + 1):
        m = new_marks(["up_revive", "up_kv_len"])
        m["up_revive"][0].record()
        U.up_revive(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, w.block,
                    ws.block_mask, ws.hidden_out, hidden, ws.compact_ws)
        m["up_revive"][1].record()
        m["up_kv_len"][0].record()
        U.up_kv_len(ledger, B, cap, 1 << 20, batch.cu_seqlens_d, kv_len)
        m["up_kv_len"][1].record()
        if i:
            rv_marks.append(m)
    torch.cuda.synchronize()

    # Fused pipeline, outside the timed region: selection in the column-sum
    # kernel, and the next layer's normalised operand / residual sum read
    # straight from the frozen rows, against the unfused calls (compaction,
    # then torch's RMSNorm of the compacted rows).
    D = hidden.shape[1]
    normed = torch.empty((T, D), dtype=hidden.dtype, device=dev)
    delta = torch.randn((max(kept, 1), D), device=dev).to(hidden.dtype)
    fz = []
    for i in range(nb + 1):
        m = new_marks(["up_score_select", "up_compact_rmsnorm", "up_gather_add", "torch_rmsnorm",
                       "chain_fused"])
        m["chain_fused"][0].record()
        m["up_score_select"][0].record()
        U.up_score_select(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, q, k,
                          w.n_query, w.block, 0.0, ws.token_scores, ws.block_scores, w.top_p,
                          w.sink, w.tail, ws.block_mask, ws.kept_tokens, ws.score_ws)
        m["up_score_select"][1].record()
        m["up_compact_rmsnorm"][0].record()
        U.up_compact_rmsnorm(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, w.block,
                             ws.block_mask, hidden, None, 1e-6, pos, normed, None, ws.positions_out,
                             ws.cu_seqlens_out, ws.compact_ws)
        m["up_compact_rmsnorm"][1].record()
        U.up_drop_history(ledger, B, cap, (K + i) % cap, ws.cu_seqlens_out)
        m["chain_fused"][1].record()
        m["up_gather_add"][0].record()
        U.up_gather_add(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, w.block,
                        ws.block_mask, hidden, delta, normed[:max(kept, 1)], ws.compact_ws)
        m["up_gather_add"][1].record()
        m["torch_rmsnorm"][0].record()
        torch.nn.functional.rms_norm(ws.hidden_out[:kept], (D,), eps=1e-6)
        m["torch_rmsnorm"][1].record()
        if i:
            fz.append(m)
    torch.cuda.synchronize()
    U.up_history_init(ledger, B, cap)
    del normed, delta

    # The same step captured once as a HIP graph and replayed: the kernels
    # without the host's per-call work (validation, launches).
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(layer=0)   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(layer=1)
    U.up_history_init(ledger, B, cap)
    gm = new_marks(["graph"])
    torch.cuda.synchronize()
    gm["graph"][0].record()
    for _ in range(nb):
        graph.replay()
    gm["graph"][1].record()
    torch.cuda.synchronize()
    graph_step_us = gm["graph"][0].elapsed_time(gm["graph"][1]) * 1e3 / nb
    del graph
    U.up_history_init(ledger, B, cap)

    measured = measured_peaks(dev)
    gc.enable()

    ms_per_step = (t1 - t0) * 1e3 / K
    per_call_us = {n: med_us(brk, n) for n in calls}
    if dominant == "up_score":
        per_call_us["up_score"] = dominant_us
    tokens_per_s = T / (ms_per_step / 1e3)

    # --- algorithmic work -------------------------------------------------
    lens = [int(x) for x in inp["lengths"]]
    pairs = 0
    for L in lens:
        ne = min(w.n_query, L)
        pairs += ne * L - ne * (ne - 1) // 2          # causal-visible (row, key) pairs per head
    flops_alg = 2.0 * w.head_dim * w.hq * pairs        # one Q K^T over visible pairs
    flops_exec = 2.0 * flops_alg                       # exact column sums recompute S once
    row_bytes = hidden[0].numel() * hidden.element_size()
    compact_bytes = 2 * kept * row_bytes + 2 * 4 * kept + N
    compact_bytes_rv = 2 * kept * row_bytes + N                   # revival moves no positions
    score_bytes = T * w.hkv * w.head_dim * 2 + sum(min(w.n_query, L) for L in lens) * w.hq * w.head_dim * 2

    t_score = per_call_us["up_score"] * 1e-6
    t_compact = per_call_us["up_compact_record"] * 1e-6
    t_select = per_call_us["up_select_topp"] * 1e-6
    copy_us = mean_us(timed_marks, "copy_kernel")
    copy_gbs = compact_bytes / (copy_us * 1e-6) / 1e9
    score_tflops_exec = flops_exec / t_score / 1e12
    score_tflops_alg = flops_alg / t_score / 1e12

    if dominant == "copy_kernel":
        # The copy kernel moves every byte the compaction moves; its events
        # are recorded by the library right around its launch.
        roofline = {"kernel": "up_compact_copy_kernel", "bound": "hbm", "achieved": round(copy_gbs, 1),
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(copy_gbs / PEAK_HBM_GBS, 4),
                    "traffic": load_traffic("up_compact_copy_kernel", "up_compact.hip", w.name),
                    "algorithmic_bytes_per_launch": int(compact_bytes),
                    "duration": ("HIP events recorded by the library right around the copy kernel's "
                                 f"launch (up_set_copy_events) on every {EVENT_EVERY}th step of the "
                                 f"timed region ({len(dom_all)} launches), mean {copy_us:.2f} us")}
    else:
        roofline = {"kernel": "up_score (rowstats+colsum+blockmean)", "bound": "mfma",
                    "achieved": round(score_tflops_exec, 1), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(score_tflops_exec / PEAK_BF16_TFLOPS, 4),
                    "traffic": None, "algorithmic_flops_per_launch": flops_exec}

    # fused pipeline figures
    fz_us = {n: med_us(fz, n) for n in fz[0]}
    norm_bytes = 2 * kept * row_bytes + 2 * 4 * kept + N     # kept rows read, operand written
    add_bytes = 3 * kept * row_bytes + N                      # frozen + delta read, sum written
    unfused_chain_us = sum(per_call_us[n] for n in calls) + fz_us["torch_rmsnorm"]

    def gbs(b, us):
        return round(b / (us * 1e-6) / 1e9, 1)

    fused_rec = {
        "up_score_select_us": round(fz_us["up_score_select"], 2),
        "up_score_plus_select_us": round(per_call_us["up_score"] + per_call_us["up_select_topp"], 2),
        "up_compact_rmsnorm_us": round(fz_us["up_compact_rmsnorm"], 2),
        "up_compact_rmsnorm_gbs": gbs(norm_bytes, fz_us["up_compact_rmsnorm"]),
        "up_compact_rmsnorm_frac_of_hbm_peak": round(gbs(norm_bytes, fz_us["up_compact_rmsnorm"]) / PEAK_HBM_GBS, 4),
        "up_compact_rmsnorm_algorithmic_bytes": int(norm_bytes),
        "up_compact_rmsnorm_traffic": (lambda a, b: a + b if a is not None and b is not None else None)(
            load_traffic("up_rowop_kernel_norm", "up_compact.hip", w.name),
            load_traffic("up_compact_scan_kernel", "up_compact.hip", w.name)),
        "up_gather_add_us": round(fz_us["up_gather_add"], 2),
        "up_gather_add_gbs": gbs(add_bytes, fz_us["up_gather_add"]),
        "up_gather_add_frac_of_hbm_peak": round(gbs(add_bytes, fz_us["up_gather_add"]) / PEAK_HBM_GBS, 4),
        "up_gather_add_algorithmic_bytes": int(add_bytes),
        "unfused_compact_then_torch_rmsnorm_us": round(per_call_us["up_compact_record"] + fz_us["torch_rmsnorm"], 2),
        "chain_fused_us": round(fz_us["chain_fused"], 2),
        "chain_unfused_with_torch_rmsnorm_us": round(unfused_chain_us, 2),
        "note": ("chain_fused = up_score_select + up_compact_rmsnorm + up_drop_history (the "
                 "next layer's normalised operand produced from the frozen rows); the unfused "
                 "chain adds torch's RMSNorm of the compacted rows to the step's calls"),
    }

    rec = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": B, "tokens": T, "seq_len": max(lens),
                   "hq": w.hq, "hkv": w.hkv, "head_dim": w.head_dim, "n_query": w.n_query,
                   "block": w.block, "top_p": w.top_p, "sink": w.sink, "tail": w.tail,
                   "hidden_dim": w.hidden_dim, "hidden_dtype": w.hidden_dtype,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "breakdown_us": {k2: round(v, 2) for k2, v in per_call_us.items()},
        "dominant_call_us": {"call": {"copy_kernel": "up_compact_copy_kernel (in up_compact_record)"}.get(dominant, dominant),
                             "p10": round(float(np.percentile(dom_all, 10)), 2),
                             "median": round(float(np.median(dom_all)), 2),
                             "p90": round(float(np.percentile(dom_all, 90)), 2)},
        "chain_us_cold_cache": {"p10": round(float(np.percentile(cold_us, 10)), 2),
                                "median": round(float(np.median(cold_us)), 2),
                                "p90": round(float(np.percentile(cold_us, 90)), 2),
                                "chains": len(cold_us)},
        "score_mfma": {"executed_tflops": round(score_tflops_exec, 1),
                       "algorithmic_tflops": round(score_tflops_alg, 1),
                       "frac_of_peak_executed": round(score_tflops_exec / PEAK_BF16_TFLOPS, 4),
                       "frac_of_peak_algorithmic": round(score_tflops_alg / PEAK_BF16_TFLOPS, 4),
                       "frac_of_measured_gemm_executed": round(score_tflops_exec / measured["gemm_bf16_tflops"], 4),
                       "executed_flops_per_call": flops_exec, "k_bytes_per_call": int(score_bytes)},
        "select_compact_hbm": {"bytes": int(compact_bytes + 5 * N),
                               "gbs": round((compact_bytes + 5 * N) / (t_select + t_compact) / 1e9, 1),
                               "frac_of_peak": round((compact_bytes + 5 * N) / (t_select + t_compact) / 1e9 / PEAK_HBM_GBS, 4),
                               "frac_of_measured_copy": round((compact_bytes + 5 * N) / (t_select + t_compact) / 1e9
                                                              / measured["copy_gbs"], 4)},
        "measured_peaks": measured,
        "revive": {"us": round(med_us(rv_marks, "up_revive"), 2),
                   "gbs": round(compact_bytes_rv / (med_us(rv_marks, "up_revive") * 1e-6) / 1e9, 1),
                   "frac_of_hbm_peak": round(compact_bytes_rv / (med_us(rv_marks, "up_revive") * 1e-6)
                                             / 1e9 / PEAK_HBM_GBS, 4),
                   "algorithmic_bytes": int(compact_bytes_rv),
                   "traffic": (lambda a, b: a + b if a is not None and b is not None else None)(
                       load_traffic("up_revive_copy_kernel", "up_compact.hip", w.name),
                       load_traffic("up_compact_scan_kernel", "up_compact.hip", w.name))},
        "kv_len_us": round(med_us(rv_marks, "up_kv_len"), 2),
        "graph_step_us": round(graph_step_us, 2),
        "fused_pipeline": fused_rec,
        "keep_ratio": round(kept / T, 5),
        "input_generation_s": round(t_gen, 2),
    }

    if not args.no_cpu_baseline:
        rec["cpu_baseline"], rec["parity"] = cpu_leg(w, inp, ws, kept, args.cpu_threads, T)
    print(json.dumps(rec), flush=True)


def measured_peaks(dev) -> dict:
    """What library code reaches on this GPU, as a second yardstick beside the
    datasheet peaks: a device-to-device copy of 1 GiB (bytes read + written)
    and a bf16 GEMM of 8192^3 through torch.matmul (hipBLASLt)."""
    import torch

    def timed(fn, reps):
        fn()
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src), 10)
    del src, dst
    n = 8192
    a = torch.randn(n, n, dtype=torch.bfloat16, device=dev)
    b = torch.randn(n, n, dtype=torch.bfloat16, device=dev)
    c = torch.empty(n, n, dtype=torch.bfloat16, device=dev)
    t_gemm = timed(lambda: torch.matmul(a, b, out=c), 10)
    del a, b, c
    torch.cuda.synchronize()
    return {"copy_gbs": round(2 * COPY_BYTES / t_copy / 1e9, 1),
            "gemm_bf16_tflops": round(2.0 * n ** 3 / t_gemm / 1e12, 1),
            "note": "torch device-to-device copy of 1 GiB (read + write bytes) and torch.matmul "
                    "bf16 8192x8192x8192 (hipBLASLt), timed with HIP events after the steps"}


def stack_bench(args, dev):
    """Synthetic hybrid stack (random weights; token-local MLP layers between
    full-attention layers): forward time with the pruning path at each
    full-attention layer vs the same stack carrying every token."""
    import torch

    from token_block_sparsification_amd.stack import HybridStack, StackConfig

    L = args.stack_len
    base = StackConfig()
    g = torch.Generator().manual_seed(123)
    h = torch.randn(L, base.d_model, generator=g).to(torch.bfloat16).to(dev)
    cu = torch.tensor([0, L], dtype=torch.int32)
    pos = torch.arange(L, dtype=torch.int32, device=dev)

    def timed(stack, prune, reps=5, fused=False):
        for _ in range(2):
            stack.forward(h, cu, pos, prune=prune, fused=fused)
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            t0 = time.perf_counter()
            r = stack.forward(h, cu, pos, prune=prune, fused=fused)
            torch.cuda.synchronize()
            times.append(time.perf_counter() - t0)
        return float(np.median(times)), r

    import numpy as np
    runs = []
    t_full = None
    for p in [float(x) for x in args.stack_top_p.split(",")]:
        cfg = StackConfig(top_p=p)
        stack = HybridStack(cfg, dev)
        if t_full is None:
            t_full, _ = timed(stack, False)
        t, r = timed(stack, True)
        tf, rf = timed(stack, True, fused=True)
        runs.append({"top_p": p, "ms": round(t * 1e3, 3), "speedup_vs_unpruned": round(t_full / t, 4),
                     "fused_ms": round(tf * 1e3, 3), "fused_speedup_vs_unpruned": round(t_full / tf, 4),
                     "fused_tokens_per_layer": rf.tokens_per_layer,
                     "tokens_per_layer": r.tokens_per_layer,
                     "layer_tokens_fraction": round(sum(r.tokens_per_layer) /
                                                    (L * len(cfg.pattern)), 4)})
        del stack
    first = runs[0]
    rec = {
        "metric": "synthetic hybrid stack forward tokens/s with pruning at full-attention layers",
        "value": round(L / (first["ms"] * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": 5, "warmup": 2, "ms_per_step": first["ms"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (random weights and embeddings)",
        "config": {"workload": f"hybrid_stack_L{L}", "pattern": base.pattern, "d_model": base.d_model,
                   "d_ff": base.d_ff, "hq": base.hq, "hkv": base.hkv, "head_dim": base.head_dim,
                   "n_query": base.n_query, "block": base.block, "parallelism": "single GPU"},
        "unpruned_ms": round(t_full * 1e3, 3),
        "runs": runs,
    }
    print(json.dumps(rec), flush=True)


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or "unknown"."""
    try:
        for line in open("/proc/cpuinfo", encoding="utf-8", errors="replace"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_leg(w, inp, ws, kept, threads, T):
    """The CPU baseline (the C++ oracle, one thread pinned to one core, on a
    bounded sample of the bench batch) and a full-size parity check of the GPU
    result against the numpy oracle (fp64, BLAS with `threads` threads, not
    timed)."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import oracle as O
    import oracle.cxx as CX

    cu = inp["cu_seqlens"].numpy()
    lens = inp["lengths"]
    q_bits = inp["q"].view(torch.int16).cpu().numpy()
    k_bits = inp["k"].view(torch.int16).cpu().numpy()
    hid = inp["hidden"].view(torch.int16).cpu().numpy()
    pos = inp["positions"].cpu().numpy()

    # --- CPU baseline: the plain single-threaded C++ oracle ---------------
    # Sample: steps 1-2 for the query heads of KV heads 0, 1, ... (hq/hkv
    # query heads each), one KV group at a time until at least ten seconds of
    # CPU work are timed; scores are a sum over heads, so the full step costs
    # hkv / (groups timed) times as much and is scaled so.  Steps 3-5 then run
    # on those partial scores over every token.
    cx = CX.module()
    group = w.hq // w.hkv
    allowed = sorted(os.sched_getaffinity(0))
    core = allowed[0]
    os.sched_setaffinity(0, {core})      # this thread only (no re-exec)
    try:
        t0 = time.perf_counter()
        c = np.zeros(T, dtype=np.float64)
        groups = 0
        while groups < w.hkv and (groups == 0 or time.perf_counter() - t0 < 10.0):
            heads = list(range(groups * group, (groups + 1) * group))
            c += cx.token_scores(q_bits, k_bits, cu, w.n_query, None, heads=heads)
            groups += 1
        bsc = cx.block_scores(c, cu, w.block)
        t1 = time.perf_counter()
        mask_s, _ = cx.select_topp(bsc, cu, w.block, w.top_p, w.sink, w.tail)
        t2 = time.perf_counter()
        _, _, cu_s = cx.compact(mask_s, hid, pos, cu, w.block)
        t3 = time.perf_counter()
        led = cx.history_new(len(lens))
        cx.history_append(led, 0, cu_s)
        t4 = time.perf_counter()
    finally:
        os.sched_setaffinity(0, set(allowed))
    score_full = (t1 - t0) * w.hkv / groups
    total = score_full + (t4 - t1)
    cpu = {"value": round(T / total, 1), "unit": "tokens/s", "cores": 1,
           "kind": "oracle (plain C++17, fp64, single thread)",
           "seconds": round(total, 2),
           "seconds_timed": round(t4 - t0, 2),
           "seconds_per_step": {"score_s": round(score_full, 2),
                                "score_sample_s": round(t1 - t0, 2),
                                "select_s": round(t2 - t1, 3), "compact_s": round(t3 - t2, 3),
                                "history_s": round(t4 - t3, 5)},
           "sample": (f"the bench batch ({len(lens)} request(s), {T} tokens): steps 1-2 (scores, "
                      f"block means) over the {groups * group} query heads of KV heads "
                      f"0..{groups - 1}, timed and scaled by hkv/{groups} = {w.hkv / groups:g} to "
                      f"all {w.hq} heads; steps 3-5 (Top-p, compaction of {w.hidden_dim}-wide "
                      f"rows, ledger) on the whole batch; one thread pinned to core {core} of "
                      f"{cpu_model()}; the process may use {len(allowed)} of the host's "
                      f"{os.cpu_count()} logical CPUs")}

    # --- full-size parity of this run: numpy oracle (fp64) vs the GPU -------
    q64 = np.zeros(tuple(inp["q"].shape), dtype=np.float64)   # untouched pages stay virtual
    for r, L in enumerate(lens):
        ne = min(w.n_query, L)
        s1 = int(cu[r + 1])
        q64[s1 - ne:s1] = O.widen_bf16(q_bits[s1 - ne:s1])
    k64 = O.widen_bf16(k_bits)
    with threadpool_limits(threads):
        c = O.token_scores(q64, k64, cu, w.n_query, None)
        bsc = O.block_scores(c, cu, w.block)
        mask, kept_ref = O.select_topp(bsc, cu, w.block, w.top_p, w.sink, w.tail)
        h_out, p_out, cu_out = O.compact(mask, hid, pos, cu, w.block)
    del q64, k64
    out = {"token_scores": c, "block_scores": bsc, "mask": mask, "hidden_out": h_out,
           "positions_out": p_out, "cu_out": cu_out}
    gpu_ts = ws.token_scores[:T].double().cpu().numpy()
    ref = out["token_scores"]
    rel_err = np.abs(gpu_ts - ref) / np.abs(ref)
    gpu_mask = ws.block_mask[:len(out["mask"])].cpu().numpy()
    mism = int((gpu_mask.astype(bool) != out["mask"].astype(bool)).sum())
    band = 0
    if mism:
        cub = O.block_offsets(cu, w.block)
        for r, L in enumerate(lens):
            bsl = slice(int(cub[r]), int(cub[r + 1]))
            bd = O.band_blocks(out["block_scores"][bsl], L, w.block, w.top_p, w.sink, w.tail)
            diff = np.flatnonzero(gpu_mask[bsl].astype(bool) != out["mask"][bsl].astype(bool))
            band += int(bd[diff].sum())
    same_mask = mism == 0
    bit_exact = None
    if same_mask:
        n = int(out["cu_out"][-1])
        got = ws.hidden_out[:n].view(torch.int16).cpu().numpy()
        bit_exact = bool(np.array_equal(got, out["hidden_out"]) and
                         np.array_equal(ws.positions_out[:n].cpu().numpy(), out["positions_out"]) and
                         n == kept)
    parity = {"max_rel_token_score_err": float(rel_err.max()),
              "score_within_2e-3": bool((np.abs(gpu_ts - ref) <= 2e-3 * np.abs(ref) + 1e-12 * ref.sum()).all()),
              "mask_mismatches": mism, "mask_mismatches_in_band": band,
              "compaction_bit_exact": bit_exact}
    return cpu, parity


if __name__ == "__main__":
    main()
