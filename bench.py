"""Benchmark of the paged-attention decode hot path on one MI355X.

A step is one pass of the hot path over one batch: reshape_and_cache of the
batch's new K/V tokens, then paged_attention_decode over every sequence (and,
for the long mixed workload, paged_attention_chunked).  Inputs are seeded and
synthetic and resident in HBM before timing starts.

Default workload: GQA decode, 32 query / 8 kv heads, head_dim 128, bf16,
block 16, 256 sequences with lognormal context lengths (median 1024, sigma 1,
clipped to [16, 8192]).  The metric is the algorithmic KV+Q bytes read per
second (every logical token's K and V for every kv head once, plus the
queries), with sequences per second alongside.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gqa|opt13b|tiny|long|cow|beam|shapes]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged-attn decode achieved HBM GB/s (% of MI355X peak) + sequences/sec"
PEAK_HBM_GBS = 8000.0
PEAK_MFMA_TFLOPS = 2500.0  # dense bf16 / f16 matrix-core peak of MI355X
PROFILES = os.path.join(ROOT, "profiles")
# sources of the decode kernels: counter summaries are valid only for these exact files
KERNEL_SOURCES = [os.path.join(ROOT, "paged_kv_cache_265_amd", "csrc", f)
                  for f in ("decode.hip", "decode_kernels.h", "decode_inner.h", "device.h", "internal.h")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str):
    """HBM bytes per decode launch from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"decode_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not sha or not val or sha.group(1) != source_sha():
        return None
    return float(val.group(1))


def build_workload(name: str):
    import workloads
    if name == "gqa":
        c = workloads.config_decode(3)
        return {"decode": c, "new": (c.new_key, c.new_value, c.slot_mapping), "partition_size": 0,
                "config": {"workload": "GQA decode 32 q heads / 8 kv heads, head_dim 128, bf16, block 16, "
                                       "256 seqs, context lognormal(median 1024, sigma 1) clipped to [16, 8192], "
                                       "plus reshape_and_cache of 256 new tokens",
                           "num_seqs": c.num_seqs, "num_q_heads": 32, "num_kv_heads": 8, "head_dim": 128,
                           "block_size": 16, "total_context_tokens": int(c.context_lens.sum()),
                           "max_context": int(c.context_lens.max()), "parallelism": "none (one GPU)"}}
    if name == "tiny":
        c = workloads.config_decode(1)
        return {"decode": c, "new": None, "partition_size": 0,
                "config": {"workload": "tiny paged decode: 4 seqs, contexts {1, 7, 16, 33}, 4 heads MHA, head_dim 64, "
                                       "fp32, block 16, 32-block pool (launch latency; a parity case)",
                           "num_seqs": 4, "total_context_tokens": int(c.context_lens.sum())}}
    if name == "opt13b":
        c = workloads.config_decode(2)
        return {"decode": c, "new": None, "partition_size": 0,
                "config": {"workload": "OPT-13B-shaped layer decode, 40 heads MHA, head_dim 128, fp16, block 16, "
                                       "64 seqs, context uniform [128, 2048]",
                           "num_seqs": 64, "total_context_tokens": int(c.context_lens.sum())}}
    raise ValueError(name)


def build_long():
    import workloads
    p, qd, qc, cu = workloads.config_long_mixed()
    return p, qd, qc, cu


def cpu_baseline(case, budget_s: float = 10.0):
    """The fp64 oracle on the same batch (its pending new tokens written first on the
    host), repeated whole until about budget_s of wall time, on this host's cores."""
    import oracle
    import workloads
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    pool = case.pool.clone()
    if case.new_key is not None:
        oracle.reshape_and_cache(case.new_key, case.new_value, pool.key_cache, pool.value_cache, case.slot_mapping,
                                 case.dtype)
    runs, spent = 0, 0.0
    while spent < budget_s or runs == 0:
        t0 = time.perf_counter()
        oracle.decode(case.query, pool.key_cache, pool.value_cache, case.block_tables, case.context_lens,
                      case.num_kv_heads, case.block_size, case.scale, case.dtype)
        spent += time.perf_counter() - t0
        runs += 1
    nbytes = workloads.algorithmic_decode_bytes(case.context_lens, case.num_q_heads, case.num_kv_heads,
                                                case.head_dim, workloads.DTYPES[case.dtype][2])
    res = {"value": round(nbytes * runs / spent / 1e9, 2), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"the whole batch ({case.num_seqs} sequences, {int(case.context_lens.sum())} context "
                     f"tokens) decoded {runs} times by the fp64 C oracle in {spent:.1f} s wall",
           "seqs_per_s": round(case.num_seqs * runs / spent, 1)}
    # the same on one thread: one pass over the whole batch
    oracle.set_threads(1)
    try:
        t0 = time.perf_counter()
        oracle.decode(case.query, pool.key_cache, pool.value_cache, case.block_tables, case.context_lens,
                      case.num_kv_heads, case.block_size, case.scale, case.dtype)
        one = time.perf_counter() - t0
    finally:
        oracle.set_threads(threads)
    res["single_thread"] = {"value": round(nbytes / one / 1e9, 3), "unit": "GB/s", "cores": 1,
                            "sample": f"the whole batch decoded once in {one:.1f} s wall",
                            "seqs_per_s": round(case.num_seqs / one, 1)}
    cpu = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    res["cpu_model"] = cpu
    res["os_cpu_count"] = os.cpu_count()
    return res


def cold_calls(torch, pkv, dev, call, n: int = 20):
    """Times of `call` with the 256 MB last-level cache evicted before each one (a
    512 MiB write outside the timed events)."""
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        scratch.fill_(i & 255)
        evs[i][0].record()
        call()
        evs[i][1].record()
    torch.cuda.synchronize()
    del scratch
    torch.cuda.empty_cache()
    return np.array([a.elapsed_time(b) for a, b in evs])


def graph_timing(torch, args, step, call, out, nbytes):
    """The step, and the decode call alone, captured once in a HIP graph and
    replayed, as a serving loop would launch them: the same kernels with shorter
    gaps between launches.  The replayed output must match the eager one bit for bit."""
    eager = out.clone()
    res = {}
    for name, fn in (("step", step), ("call", call)):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(g):
            fn()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        res[f"{name}_ms"] = round(ms, 4)
        res[f"{name}_GBs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
        res[f"{name}_bitwise_equal_to_eager"] = bool(torch.equal(out.view(torch.uint8), eager.view(torch.uint8)))
        del g
    return res


def read_ceiling(torch, pkv, dev, nbytes: int = 4 << 30) -> float:
    """GB/s of pkv_read_probe over a 4 GiB buffer: the decode kernels' load shape
    with nothing else to do, a practical read ceiling of this device."""
    buf = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(2):
        pkv.read_probe(buf, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        pkv.read_probe(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    gbs = 5 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf
    torch.cuda.empty_cache()
    return gbs


def copy_probe(torch, dev, nbytes: int = 4 << 30) -> float:
    """Read+write GB/s of a plain device-to-device copy (torch), a practical ceiling."""
    a = torch.empty(nbytes // 2, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    gbs = 5 * 2 * a.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return gbs


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gqa", choices=["gqa", "opt13b", "tiny", "long", "cow", "beam", "shapes",
                                                             "prefill"])
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--paging-study", action="store_true",
                    help="time the decode call on the same batch with shuffled and with contiguous block "
                         "placement, and with blocks of 8 and 32 tokens, in one process, and print all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--shape-filter", default=None,
                    help="--workload shapes: time only the shapes whose label contains this text")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain 1 GiB device copy (reference kernel for the HBM counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU: the decode hot path has no multi-GPU "
                                   "leg here (sequences would shard across GPUs with no exchange); run with "
                                   "--gpus 1"}))
        sys.exit(2)

    import torch
    import paged_kv_cache_265_amd as pkv
    import workloads

    assert torch.cuda.is_available(), "needs a GPU"
    pkv.load_library()
    dev = torch.device("cuda:0")

    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))
        return

    t_gen = time.perf_counter()
    if args.workload == "long":
        p, qd, qc, cu = build_long()
        run = run_long(args, p, qd, qc, cu, torch, pkv, workloads, dev)
        return run
    if args.workload == "cow":
        return run_cow(args, torch, pkv, workloads, dev)
    if args.workload == "beam":
        return run_beam(args, torch, pkv, workloads, dev)
    if args.workload == "shapes":
        return run_shapes(args, torch, pkv, workloads, dev)
    if args.workload == "prefill":
        return run_prefill(args, torch, pkv, workloads, dev)
    W = build_workload(args.workload)
    case = W["decode"]
    part = W["partition_size"] if args.partition_size is None else args.partition_size
    log(f"generated {args.workload} in {time.perf_counter() - t_gen:.1f} s; moving to the GPU")

    kc = case.pool.key_cache.to(dev)
    vc = case.pool.value_cache.to(dev)
    q = case.query.to(dev)
    bt = torch.from_numpy(case.block_tables).to(dev)
    cl = torch.from_numpy(case.context_lens).to(dev)
    out = torch.empty_like(q)
    ws_bytes = pkv.decode_workspace_size(case.num_seqs, case.num_q_heads, case.num_kv_heads, case.head_dim,
                                         case.block_size, case.max_blocks_per_seq, part)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    new = None
    if W["new"] is not None:
        nk, nv, sm = W["new"]
        new = (nk.to(dev), nv.to(dev), torch.from_numpy(sm).to(dev))
    torch.cuda.synchronize()
    if args.paging_study:
        return paging_study(args, torch, pkv, workloads, dev, case, kc, vc, q, bt, cl, new, part, ws)

    def call():
        pkv.paged_attention_decode(out, q, kc, vc, bt, cl, case.scale, partition_size=part, workspace=ws)

    def step():
        if new is not None:
            pkv.reshape_and_cache(new[0], new[1], kc, vc, new[2])
        call()

    def timed(fn, n):
        # n back-to-back launches between one pair of events on the launch stream:
        # (GPU ms per launch, wall ms per launch)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, (time.perf_counter() - t0) * 1e3 / n

    for _ in range(args.warmup):
        step()
    # the timed region: K whole steps back to back
    ms_step, wall_ms_step = timed(step, args.steps)
    # the decode call alone, K calls back to back (the roofline's launch average)
    dec_ms, _ = timed(call, args.steps)
    # per-call spread: each call between its own pair of events
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        if new is not None:
            pkv.reshape_and_cache(new[0], new[1], kc, vc, new[2])
        evs[i][0].record()
        call()
        evs[i][1].record()
    torch.cuda.synchronize()

    eb = workloads.DTYPES[case.dtype][2]
    nbytes = workloads.algorithmic_decode_bytes(case.context_lens, case.num_q_heads, case.num_kv_heads,
                                                case.head_dim, eb)
    value = nbytes / (ms_step * 1e-3) / 1e9
    achieved = nbytes / (dec_ms * 1e-3) / 1e9
    traffic = traffic_from_profiles(args.workload)
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "wall_ms_per_step": round(wall_ms_step, 4),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": case.dtype, "data": "synthetic (seeded N(0,1) K/V/q, shuffled block placement)",
        "config": W["config"],
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "seqs_per_s": round(case.num_seqs / (ms_step * 1e-3), 1),
        "algorithmic_bytes_per_step": nbytes,
        "partition_size": pkv.decode_partition_size(case.num_seqs, case.num_q_heads, case.num_kv_heads,
                                                    case.head_dim, case.block_size, case.max_blocks_per_seq, part),
        "roofline": {"bound": "hbm", "kernel": "paged_attention_decode (decode kernel + partition merge)",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "avg_call_ms": round(dec_ms, 4),
                     "traffic": traffic},
    }
    call_ms = np.array([a.elapsed_time(b) for a, b in evs])
    res["call_ms_p10_p50_p90"] = [round(float(np.percentile(call_ms, q)), 4) for q in (10, 50, 90)]
    res["graph"] = graph_timing(torch, args, step, call, out, nbytes)
    res["warm_median_GBs"] = round(nbytes / (float(np.median(call_ms)) * 1e-3) / 1e9, 1)
    cold = cold_calls(torch, pkv, dev, call)
    res["cold_call_ms_p10_p50_p90"] = [round(float(np.percentile(cold, q)), 4) for q in (10, 50, 90)]
    res["cold_median_GBs"] = round(nbytes / (float(np.median(cold)) * 1e-3) / 1e9, 1)
    ceiling = read_ceiling(torch, pkv, dev)
    res["read_probe_GBs"] = round(ceiling, 1)
    res["roofline"]["frac_of_read_probe"] = round(achieved / ceiling, 4)
    res["device_copy_GBs"] = round(copy_probe(torch, dev), 1)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        res["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(res), flush=True)


def run_long(args, p, qd, qc, cu, torch, pkv, workloads, dev):
    S = qd.shape[0]
    kc = p.pool.key_cache.to(dev)
    vc = p.pool.value_cache.to(dev)
    q = qd.to(dev)
    qcd = qc.to(dev)
    cud = torch.from_numpy(cu).to(dev)
    bt = torch.from_numpy(p.block_tables).to(dev)
    cl = torch.from_numpy(p.context_lens).to(dev)
    pend = np.nonzero(p.pending)[0]
    nk = p.logical_k[torch.from_numpy(pend)].to(dev)
    nv = p.logical_v[torch.from_numpy(pend)].to(dev)
    sm = torch.from_numpy(p.token_slots[pend]).to(dev)
    out = torch.empty_like(q)
    outc = torch.empty_like(qcd)
    ws = torch.empty(pkv.decode_workspace_size(S, 32, 1, 128, 16, p.block_tables.shape[1], 0), dtype=torch.uint8,
                     device=dev)
    scale = 1.0 / np.sqrt(128)
    torch.cuda.synchronize()

    def dec():
        pkv.paged_attention_decode(out, q, kc, vc, bt[:S], cl[:S], scale, partition_size=0, workspace=ws)

    def chk():
        pkv.paged_attention_chunked(outc, qcd, cud, 512, kc, vc, bt[S:], cl[S:], scale)

    def step():
        pkv.reshape_and_cache(nk, nv, kc, vc, sm)
        dec()
        chk()

    def timed(fn, n):
        # n back-to-back launches between one pair of events: (GPU ms, wall ms) per launch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, (time.perf_counter() - t0) * 1e3 / n

    for _ in range(args.warmup):
        step()
    ms_step, wall_ms_step = timed(step, args.steps)
    dec_ms, _ = timed(dec, args.steps)
    chk_ms, _ = timed(chk, args.steps)
    # the same decode with fixed 512-token partitions instead of the balanced split
    wsf = torch.empty(pkv.decode_workspace_size(S, 32, 1, 128, 16, p.block_tables.shape[1], 512),
                      dtype=torch.uint8, device=dev)
    outf = torch.empty_like(q)
    for _ in range(args.warmup):
        pkv.paged_attention_decode(outf, q, kc, vc, bt[:S], cl[:S], scale, partition_size=512, workspace=wsf)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        pkv.paged_attention_decode(outf, q, kc, vc, bt[:S], cl[:S], scale, partition_size=512, workspace=wsf)
    e1.record()
    torch.cuda.synchronize()
    fix_ms = e0.elapsed_time(e1) / args.steps
    # the whole flattened batch in one attention launch: decode tokens as one-row
    # segments beside the prefill chunks, against the two calls back to back
    cum = np.concatenate([np.arange(S + 1), S + cu[1:]]).astype(np.int32)
    cumd = torch.from_numpy(cum).to(dev)
    qm = torch.cat([q, qcd]).contiguous()
    outm = torch.empty_like(qm)
    wsm = torch.empty(pkv.mixed_workspace_size(len(cum) - 1, 32, 1, 128, 16), dtype=torch.uint8, device=dev)

    def mixed():
        pkv.paged_attention_mixed(outm, qm, cumd, 512, kc, vc, bt, cl, scale, workspace=wsm)

    def separate():
        pkv.paged_attention_decode(out, q, kc, vc, bt[:S], cl[:S], scale, partition_size=0, workspace=ws)
        pkv.paged_attention_chunked(outc, qcd, cud, 512, kc, vc, bt[S:], cl[S:], scale)

    times = {"mixed": [], "separate": []}
    for rep in range(4):
        for name, fn in (("mixed", mixed), ("separate", separate)):
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            times[name].append(e0.elapsed_time(e1) / args.steps)
    mix_ms, sep_ms = float(np.median(times["mixed"])), float(np.median(times["separate"]))
    mixed_vs_separate = {
        "decode_rows_max_abs_diff": float((outm[:S].float() - out.float()).abs().max()),
        "prefill_rows_max_abs_diff": float((outm[S:].float() - outc.float()).abs().max())}
    nbytes = workloads.algorithmic_decode_bytes(p.context_lens[:S], 32, 1, 128, 2)
    flops = workloads.algorithmic_chunked_flops(p.context_lens[S:], np.diff(cu), 32, 128)
    res = {"metric": METRIC, "value": round(nbytes / (dec_ms * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
           "wall_ms_per_step": round(wall_ms_step, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "long-context mixed batch: MQA 32/1 decode of 32 seqs (context uniform "
                                  "[16384, 131072]) + 8 chunked-prefill segments of 512 rows over 4096 cached "
                                  "tokens"},
           "decode_ms": round(dec_ms, 4), "chunked_ms": round(chk_ms, 4),
           "decode_partition512_ms": round(fix_ms, 4),
           "decode_partition512_GBs": round(nbytes / (fix_ms * 1e-3) / 1e9, 1),
           "chunked_tflops": round(flops / (chk_ms * 1e-3) / 1e12, 2),
           "mixed_single_launch_ms": round(mix_ms, 4), "separate_calls_ms": round(sep_ms, 4),
           "mixed_speedup": round(sep_ms / mix_ms, 4), "mixed_vs_separate": mixed_vs_separate,
           "roofline": {"bound": "hbm", "kernel": "paged_attention_decode", "achieved":
                        round(nbytes / (dec_ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(nbytes / (dec_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "traffic": None}}
    print(json.dumps(res), flush=True)


def paging_study(args, torch, pkv, workloads, dev, case, kc, vc, q, bt, cl, new, part, ws):
    """The pages report the paged kernel 20-26 % slower than a contiguous one on
    their GPU, and weigh the block size: small blocks waste fewer slots in each
    sequence's last block but need longer tables ([P1] paging section).  Here: the
    same batch and kernel with the generator's shuffled placement, with every
    sequence's blocks laid out contiguously in logical order (identity placement),
    and with the same tokens re-laid in shuffled pools of 8- and 32-token blocks;
    all timed alternately.  The re-layout is plain tensor indexing on the GPU."""
    if new is not None:
        pkv.reshape_and_cache(new[0], new[1], kc, vc, new[2])
    S = case.num_seqs
    ctx = case.context_lens.astype(np.int64)
    nb = (ctx + 15) // 16
    order = np.concatenate([case.block_tables[s, :nb[s]] for s in range(S)]).astype(np.int64)
    new_id = np.arange(len(order), dtype=np.int32)
    bt_id = np.full_like(case.block_tables, 0x7FFFFFFF)
    pos = 0
    for s in range(S):
        bt_id[s, :nb[s]] = new_id[pos:pos + nb[s]]
        pos += nb[s]
    idx = torch.from_numpy(order).to(dev)
    kc_id, vc_id = kc[idx].contiguous(), vc[idx].contiguous()
    bt_id_d = torch.from_numpy(bt_id).to(dev)
    layouts = {"shuffled": (kc, vc, bt), "contiguous": (kc_id, vc_id, bt_id_d)}

    # every token of the batch, gathered from the 16-token pool: [T, Hkv, D]
    seq_of = np.repeat(np.arange(S), ctx)
    tok = np.arange(int(ctx.sum()), dtype=np.int64) - np.repeat(np.concatenate([[0], np.cumsum(ctx)[:-1]]), ctx)
    p16 = torch.from_numpy(case.block_tables[seq_of, tok // 16].astype(np.int64)).to(dev)
    o16 = torch.from_numpy(tok % 16).to(dev)
    k_log, v_log = kc[p16, :, o16, :], vc[p16, :, :, o16]
    rng = np.random.default_rng(265)
    geometry = {16: (int(nb.sum()), int((nb * 16).sum()))}
    for bs in (8, 32):
        nbb = (ctx + bs - 1) // bs
        need = int(nbb.sum())
        perm = rng.permutation(need).astype(np.int32)
        btb = np.full((S, int(nbb.max())), 0x7FFFFFFF, dtype=np.int32)
        first = np.concatenate([[0], np.cumsum(nbb)[:-1]])
        for s in range(S):
            btb[s, :nbb[s]] = perm[first[s]:first[s] + nbb[s]]
        pb = torch.from_numpy(btb[seq_of, tok // bs].astype(np.int64)).to(dev)
        ob = torch.from_numpy(tok % bs).to(dev)
        kb = torch.full((need, case.num_kv_heads, bs, case.head_dim), float("nan"), dtype=kc.dtype, device=dev)
        vb = torch.full((need, case.num_kv_heads, case.head_dim, bs), float("nan"), dtype=vc.dtype, device=dev)
        kb[pb, :, ob, :] = k_log
        vb[pb, :, :, ob] = v_log
        layouts[f"block_size_{bs}"] = (kb, vb, torch.from_numpy(btb).to(dev))
        geometry[bs] = (need, int((nbb * bs).sum()))
    del k_log, v_log, p16, o16

    outs, times = {}, {k: [] for k in layouts}
    for rep in range(6):
        for name, (k_, v_, b_) in layouts.items():
            out = torch.empty_like(q)
            for _ in range(3):
                pkv.paged_attention_decode(out, q, k_, v_, b_, cl, case.scale, partition_size=part, workspace=ws)
            torch.cuda.synchronize()
            outs[name] = out
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                pkv.paged_attention_decode(out, q, k_, v_, b_, cl, case.scale, partition_size=part, workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            times[name].append(e0.elapsed_time(e1) / args.steps)
    nbytes = workloads.algorithmic_decode_bytes(case.context_lens, case.num_q_heads, case.num_kv_heads,
                                                case.head_dim, workloads.DTYPES[case.dtype][2])
    med = {k: float(np.median(v)) for k, v in times.items()}
    used = int(ctx.sum())
    print(json.dumps({
        "paging_study": args.workload,
        "call_ms_median": {k: round(v, 4) for k, v in med.items()},
        "GBs": {k: round(nbytes / (v * 1e-3) / 1e9, 1) for k, v in med.items()},
        "paged_over_contiguous": round(med["shuffled"] / med["contiguous"], 4),
        "block_size": {str(bs): {"table_entries": g[0], "slots_allocated": g[1],
                                 "unused_slot_fraction": round(1 - used / g[1], 5),
                                 "call_ms": round(med["shuffled" if bs == 16 else f"block_size_{bs}"], 4)}
                       for bs, g in sorted(geometry.items())},
        "same_bits_as_block_size_16": {k: bool(torch.equal(outs[k].view(torch.int16), outs["shuffled"].view(
            torch.int16))) for k in outs if k.startswith("block_size")},
    }), flush=True)


def run_cow(args, torch, pkv, workloads, dev):
    """Prefix sharing: 16 prompts x 8 samples share their prompt blocks; a step runs
    the copy-on-write copies, writes every sample's private tokens, then decodes.
    Logical bytes count each sample's whole context; unique bytes count every
    distinct (block, kv head) tile once (shared prompt blocks are read by all eight
    samples, so the logical rate can exceed the HBM peak)."""
    c = workloads.config_cow()
    kc = c.pool.key_cache.to(dev)
    vc = c.pool.value_cache.to(dev)
    q = c.query.to(dev)
    bt = torch.from_numpy(c.block_tables).to(dev)
    cl = torch.from_numpy(c.context_lens).to(dev)
    bm = torch.from_numpy(c.block_mapping).to(dev)
    nk, nv = c.new_key.to(dev), c.new_value.to(dev)
    sm = torch.from_numpy(c.slot_mapping).to(dev)
    out = torch.empty_like(q)
    ws = torch.empty(pkv.decode_workspace_size(c.num_seqs, c.num_q_heads, c.num_kv_heads, c.head_dim,
                                               c.block_size, c.max_blocks_per_seq, 0), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def dec():
        pkv.paged_attention_decode(out, q, kc, vc, bt, cl, c.scale, workspace=ws)

    def step():
        pkv.copy_blocks([kc], [vc], bm)
        pkv.reshape_and_cache(nk, nv, kc, vc, sm)
        dec()

    def timed(fn, n):
        # n back-to-back launches between one pair of events: (GPU ms, wall ms) per launch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, (time.perf_counter() - t0) * 1e3 / n

    for _ in range(args.warmup):
        step()
    ms_step, wall_ms_step = timed(step, args.steps)
    dec_ms, _ = timed(dec, args.steps)
    eb = workloads.DTYPES[c.dtype][2]
    logical = workloads.algorithmic_decode_bytes(c.context_lens, c.num_q_heads, c.num_kv_heads, c.head_dim, eb)
    nb = (c.context_lens.astype(np.int64) + c.block_size - 1) // c.block_size
    used = np.unique(np.concatenate([c.block_tables[s, :nb[s]] for s in range(c.num_seqs)]))
    unique = int(len(used)) * c.num_kv_heads * c.block_size * c.head_dim * 2 * eb
    res = {"metric": METRIC, "value": round(logical / (ms_step * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
           "wall_ms_per_step": round(wall_ms_step, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": c.dtype, "data": "synthetic",
           "config": {"workload": "prefix sharing: 16 prompts (1024 - U{1..15} tokens) x 8 samples with U{0..256} "
                                  "private tokens, GQA 32/8, head_dim 128, bf16; step = copy_blocks of the "
                                  "copy-on-write pairs + reshape_and_cache of the private tokens + decode",
                      "num_seqs": c.num_seqs, "cow_pairs": int(c.block_mapping.shape[0])},
           "decode_ms": round(dec_ms, 4),
           "logical_bytes": logical, "unique_bytes": unique,
           "decode_logical_GBs": round(logical / (dec_ms * 1e-3) / 1e9, 1),
           "decode_unique_GBs": round(unique / (dec_ms * 1e-3) / 1e9, 1),
           # logical bytes, as for the other workloads: a shared prompt tile counts once per sample that
           # reads it (the repeats mostly come from the 256 MB last-level cache, so this rate can pass
           # the HBM peak); decode_unique_GBs counts every distinct tile once
           "roofline": {"bound": "hbm", "kernel": "paged_attention_decode (logical bytes)",
                        "achieved": round(logical / (dec_ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(logical / (dec_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "avg_call_ms": round(dec_ms, 4),
                        "traffic": None}}
    print(json.dumps(res), flush=True)


# (label, dtype, context lengths, query heads, kv heads): batches from one long sequence
# to many short ones, whose split streams are merged in different ways; ("uniform", n,
# lo, hi) draws n lengths from U{lo..hi} (seeded)
SHAPES = [
    ("GQA 32/8 bf16, 1 x 131072", "bf16", [131072], 32, 8),
    ("GQA 32/8 bf16, 2 x 65536", "bf16", [65536] * 2, 32, 8),
    ("GQA 32/8 bf16, 8 x 16384", "bf16", [16384] * 8, 32, 8),
    ("GQA 32/8 bf16, 64 x 2048", "bf16", [2048] * 64, 32, 8),
    ("MQA 32/1 bf16, 1 x 131072", "bf16", [131072], 32, 1),
    ("MQA 32/1 bf16, 4 x 131072", "bf16", [131072] * 4, 32, 1),
    ("MQA 32/1 bf16, 256 x 4096", "bf16", [4096] * 256, 32, 1),
    ("MHA 40 f16, 1 x 65536", "f16", [65536], 40, 40),
    ("GQA 32/8 bf16, 256 x U{64..512}", "bf16", ("uniform", 256, 64, 512), 32, 8),
    ("GQA 32/8 bf16, 1024 x U{64..512}", "bf16", ("uniform", 1024, 64, 512), 32, 8),
    ("GQA 32/8 bf16, 4096 x U{64..512}", "bf16", ("uniform", 4096, 64, 512), 32, 8),
    ("GQA 32/8 bf16, 16384 x U{64..512}", "bf16", ("uniform", 16384, 64, 512), 32, 8),
]


def run_shapes(args, torch, pkv, workloads, dev):
    """The decode call on batches of equal-length sequences, from one long context to
    many short ones (seeded N(0,1) K/V/q, shuffled placement): the best of three
    rounds of `steps` calls back to back per shape."""
    from workloads.gen import make_decode_case
    rows = []
    import numpy as np
    only = args.shape_filter
    for i, (label, dt, ctx, hq, hkv) in enumerate(SHAPES):
        if only and only not in label:
            continue
        if isinstance(ctx, tuple):
            _, n, lo, hi = ctx
            ctx = np.random.default_rng([265, 91, i]).integers(lo, hi, size=n, endpoint=True)
        c = make_decode_case([265, 90, i], dt, ctx, hq, hkv, 128)
        kc, vc, q = c.pool.key_cache.to(dev), c.pool.value_cache.to(dev), c.query.to(dev)
        bt, cl = torch.from_numpy(c.block_tables).to(dev), torch.from_numpy(c.context_lens).to(dev)
        out = torch.empty_like(q)
        ws = torch.empty(pkv.decode_workspace_size(c.num_seqs, hq, hkv, 128, 16, c.max_blocks_per_seq, 0),
                         dtype=torch.uint8, device=dev)
        nbytes = workloads.algorithmic_decode_bytes(c.context_lens, hq, hkv, 128, workloads.DTYPES[dt][2])
        best = None
        for _ in range(3):
            for _ in range(args.warmup):
                pkv.paged_attention_decode(out, q, kc, vc, bt, cl, c.scale, workspace=ws)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                pkv.paged_attention_decode(out, q, kc, vc, bt, cl, c.scale, workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            best = ms if best is None else min(best, ms)
        rows.append({"shape": label, "call_us": round(best * 1e3, 1), "bytes": nbytes,
                     "GBs": round(nbytes / (best * 1e-3) / 1e9, 1)})
        log(f"{label}: {best * 1e3:.1f} us")
        del kc, vc, q, out, ws, c
        torch.cuda.empty_cache()
    print(json.dumps({"metric": METRIC, "workload": "decode call over batch shapes", "unit": "GB/s",
                      "steps": args.steps, "warmup": args.warmup, "shapes": rows}), flush=True)


# (label, dtype, query heads, kv heads): the chunked-prefill shapes timed by
# --workload prefill, each 8 segments of 512 query rows over 4096 cached tokens
PREFILL = [
    ("MQA 32/1 bf16", "bf16", 32, 1),
    ("GQA 32/8 bf16", "bf16", 32, 8),
    ("MHA 32 f16", "f16", 32, 32),
]


def run_prefill(args, torch, pkv, workloads, dev):
    """The chunked-prefill call alone on the long mixed workload's prefill shape (8
    segments of 512 query rows over 4096 cached tokens plus the chunk, head_dim 128;
    seeded N(0,1), shuffled placement; the chunks written by reshape_and_cache first)
    for three head layouts: the best of three rounds of `steps` calls back to back.
    Lighter than --workload long (no long decode pool), for profiling the kernel."""
    from workloads.gen import make_chunked_case
    rows = []
    for i, (label, dt, hq, hkv) in enumerate(PREFILL):
        c = make_chunked_case([265, 95, i], dt, [4096] * 8, [512] * 8, hq, hkv, 128)
        p = c.paged
        kc, vc = p.pool.key_cache.to(dev), p.pool.value_cache.to(dev)
        pkv.reshape_and_cache(c.new_key.to(dev), c.new_value.to(dev), kc, vc, torch.from_numpy(c.slot_mapping).to(dev))
        q, cu = c.query.to(dev), torch.from_numpy(c.cu_q_lens).to(dev)
        bt, cl = torch.from_numpy(p.block_tables).to(dev), torch.from_numpy(p.context_lens).to(dev)
        out = torch.empty_like(q)
        flops = workloads.algorithmic_chunked_flops(p.context_lens, np.diff(c.cu_q_lens), hq, 128)
        best = None
        for _ in range(3):
            for _ in range(args.warmup):
                pkv.paged_attention_chunked(out, q, cu, 512, kc, vc, bt, cl, c.scale)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                pkv.paged_attention_chunked(out, q, cu, 512, kc, vc, bt, cl, c.scale)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            best = ms if best is None else min(best, ms)
        tf = flops / (best * 1e-3) / 1e12
        rows.append({"shape": label, "call_us": round(best * 1e3, 1), "flops": flops, "TFLOPs": round(tf, 1),
                     "frac_of_bf16_f16_mfma_peak": round(tf / PEAK_MFMA_TFLOPS, 4)})
        log(f"{label}: {best * 1e3:.1f} us, {tf:.0f} TFLOP/s")
        del kc, vc, q, out, c, p
        torch.cuda.empty_cache()
    print(json.dumps({"metric": METRIC, "workload": "chunked-prefill call, 8 x 512 rows over 4608 keys",
                      "unit": "TFLOP/s", "steps": args.steps, "warmup": args.warmup, "shapes": rows}), flush=True)


def run_beam(args, torch, pkv, workloads, dev):
    """Beam search over 4 layers: 16 prompts sharing a 256-token system prefix,
    width 4, one token per beam per step.  The native block manager plans each
    step (slots, copy-on-write, prefix-cache hits); the GPU runs one copy_blocks
    for the step's copies, then reshape_and_cache and decode per layer.  Timed:
    the whole replay of --steps steps (after --warmup steps); the decode calls'
    logical bytes over their event time give `value`."""
    from paged_kv_cache_265_amd.block_manager import BlockManager
    from workloads.beam import make_beam_script
    total = args.warmup + args.steps
    sc = make_beam_script(seed=(265, 8), num_prompts=16, system_len=256, tail_len=(128, 512), steps=total,
                          width=4, num_layers=4, num_q_heads=32, num_kv_heads=8, head_dim=128, decode_every=1)
    L, Hkv, D, BS = sc.num_layers, sc.num_kv_heads, sc.head_dim, 16
    NB = 16 * 4 * ((256 + 512 + total) // BS + 2)
    kcs = [torch.zeros((NB, Hkv, BS, D), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    vcs = [torch.zeros((NB, Hkv, D, BS), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    kt, vt = sc.k_table.to(dev), sc.v_table.to(dev)
    bm = BlockManager(NB, BS)
    hist = {}
    pend_slots, pend_pos, pend_ids, pend_copies = [], [], [], []
    host_s, dec_events, dec_bytes, copies_total, cached_total = 0.0, [], 0, 0, 0
    ws = None

    def plan(seq, toks):
        nonlocal host_s
        t0 = time.perf_counter()
        slots, copies = bm.append(seq, len(toks))
        host_s += time.perf_counter() - t0
        n0 = len(hist[seq])
        pend_slots.extend(slots)
        pend_pos.extend(range(n0, n0 + len(toks)))
        pend_ids.extend(toks)
        pend_copies.extend(copies)
        hist[seq].extend(toks)

    step, t_start = 0, None
    for op in sc.ops:
        kind = op[0]
        t0 = time.perf_counter()
        if kind == "add":
            prompt = sc.prompts[op[2]]
            cached = bm.add_sequence(op[1], prompt)
            host_s += time.perf_counter() - t0
            cached_total += cached
            hist[op[1]] = list(prompt[:cached])
            plan(op[1], list(prompt[cached:]))
        elif kind == "append":
            plan(op[1], op[2])
        elif kind == "fork":
            bm.fork(op[1], op[2])
            host_s += time.perf_counter() - t0
            hist[op[2]] = list(hist[op[1]])
        elif kind == "free":
            bm.free_sequence(op[1])
            host_s += time.perf_counter() - t0
            del hist[op[1]]
        elif kind == "commit":
            bm.commit_prompt(op[1], hist[op[1]])
            host_s += time.perf_counter() - t0
        elif kind == "decode":
            if step == args.warmup:  # the timed region starts after the warm-up steps
                torch.cuda.synchronize()
                t_start, host_s, dec_events, dec_bytes, copies_total = time.perf_counter(), 0.0, [], 0, 0
            if pend_copies:
                pkv.copy_blocks(kcs, vcs, torch.tensor(pend_copies, dtype=torch.int64, device=dev))
                copies_total += len(pend_copies)
            if pend_slots:
                sm = torch.tensor(pend_slots, dtype=torch.int64, device=dev)
                pos = torch.tensor(pend_pos, dtype=torch.int64, device=dev)
                ids = torch.tensor(pend_ids, dtype=torch.int64, device=dev)
                for l in range(L):
                    pkv.reshape_and_cache(kt[l, pos, ids].contiguous(), vt[l, pos, ids].contiguous(), kcs[l], vcs[l],
                                          sm)
            pend_slots.clear(), pend_pos.clear(), pend_ids.clear(), pend_copies.clear()
            seqs = sorted(hist)
            lens = np.array([len(hist[s]) for s in seqs])
            mb = int(-(-lens.max() // BS))
            t0 = time.perf_counter()
            bt_host = np.full((len(seqs), mb), 0x7FFFFFFF, dtype=np.int32)
            for i, s in enumerate(seqs):
                row = bm.block_table(s, mb)
                bt_host[i, :len(row)] = row
            host_s += time.perf_counter() - t0
            bt = torch.from_numpy(bt_host).to(dev)
            cl = torch.from_numpy(lens.astype(np.int32)).to(dev)
            q = sc.queries[op[1]][:len(seqs)].to(dev).contiguous()
            need = pkv.decode_workspace_size(len(seqs), 32, 8, 128, BS, mb, 0)
            if ws is None or ws.numel() < need:
                ws = torch.empty(need, dtype=torch.uint8, device=dev)
            out = torch.empty_like(q)
            for l in range(L):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                pkv.paged_attention_decode(out, q, kcs[l], vcs[l], bt, cl, sc.scale, workspace=ws)
                e1.record()
                dec_events.append((e0, e1))
                dec_bytes += workloads.algorithmic_decode_bytes(lens, 32, 8, 128, 2)
            step += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    dec_ms = sum(a.elapsed_time(b) for a, b in dec_events)
    nsteps = step - args.warmup
    res = {"metric": METRIC, "value": round(dec_bytes / (dec_ms * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
           "steps": nsteps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / nsteps, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "beam search, 4 layers: 16 prompts (256-token shared system prefix + U{128..512}), "
                                  "width 4, GQA 32/8, head_dim 128, bf16; per step the native block manager plans, "
                                  "then copy_blocks + reshape_and_cache + decode per layer"},
           "decode_ms_per_step": round(dec_ms / nsteps, 4),
           "manager_host_us_per_step": round(host_s * 1e6 / nsteps, 1),
           "cow_copies_timed": copies_total, "prefix_cached_tokens": cached_total,
           "roofline": {"bound": "hbm", "kernel": "paged_attention_decode", "achieved":
                        round(dec_bytes / (dec_ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(dec_bytes / (dec_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "traffic": None}}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
