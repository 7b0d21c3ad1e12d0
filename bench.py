"""Benchmark of one speculative-decode verification step on one MI355X.

A step is one pass of the whole hot path over one batch: the N_spec new
tokens of every sequence (all KV heads) are stored and the N_spec queries of
every sequence attend to the full quantised cache, in one tqkv_store_verify
call (the separate tqkv_store + tqkv_verify pair is timed beside it).  Inputs are
seeded synthetic tensors (tests/synth.py) already resident in HBM.

Cold-cache protocol: the MI355X's 256 MB Infinity Cache would hold the
PoC-size caches, so the benchmark keeps R byte-identical replicas of the
cache (R * bytes >= 512 MB) and step i uses replica i % R.  The K timed
steps are captured in one HIP graph (launch-bound loop) and replayed once,
bracketed by device synchronisation; the eager (non-graph) rate is reported
beside it.

Output: one JSON line: the step rate (value, effective KV GB/s), per-call
times of every entry point timed, the roofline of the verify launch and the
CPU oracle baseline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X published dense fp16 matrix peak
PAGES_FUSED_TRITON_MS = {"poc_k8v4": 3.229, "poc_k3v4_nc": 4.83}  # Arc Pro B70, context


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="poc_k8v4")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--cold-mb", type=float, default=512.0)
    ap.add_argument("--kernel-calls", type=int, default=200,
                    help="back-to-back verify calls for the per-launch kernel timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--replay-check", action="store_true",
                    help="replay the timed graph a second time and print its duration (stderr)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-reference", type=float, default=0.0, metavar="MB",
                    help="instead of the benchmark, run 20 plain device-to-device copies of MB "
                         "megabytes (the calibration kernel for the HBM byte counters)")
    return ap.parse_args()


TRAFFIC_DIR = os.path.join(ROOT, "profiles")


def kernel_source_digest():
    """sha256 over the code (comments and blank space removed) of the sources
    the verify kernel is built from: counter readings taken on another
    version of the kernel are not reported, edits to comments keep them."""
    import hashlib
    import re
    h = hashlib.sha256()
    for name in ("verify.hip", "quant.h", "common.h", "codebook.h", "api.hip"):
        with open(os.path.join(ROOT, "quantized_kv_attention_amd", "csrc", name)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)    # block comments
        src = re.sub(r"//[^\n]*", " ", src)                   # line comments
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()


def recorded_traffic(workload):
    """HBM bytes per verify call from the committed counter summary of this
    workload (profiles/traffic_<workload>.md), or None when there is none or
    it was taken on a different version of the kernel source."""
    path = os.path.join(TRAFFIC_DIR, "traffic_%s.md" % workload)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_code_sha256") != kernel_source_digest():
        return None
    try:
        return int(fields["hbm_bytes_per_verify_call"])
    except (KeyError, ValueError):
        return None


def copy_reference(mb):
    """Plain device-to-device copies of a known size: what FETCH_SIZE and
    WRITE_SIZE read for them calibrates the counters."""
    import torch
    n = int(mb * 1e6)
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(20):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_reference_bytes": n, "copies": 20}))


def main():
    args = parse()
    if args.copy_reference > 0:
        copy_reference(args.copy_reference)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only (the verify path needs no "
              "communication: every (sequence, KV head) is independent). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import quantized_kv_attention_amd as tq
    from tests import synth
    from tests.gputil import gpu_paged_store_all, gpu_store_all, page_table, to_dev

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.config(args.workload)
    N, B, Hq, Hk, S = cfg["N"], cfg["B"], cfg["Hq"], cfg["Hk"], cfg["S"]
    preset = cfg["preset"]
    slot = tq.tqkv_slot_bytes(preset)
    print("bench: workload %s, generating inputs" % args.workload, file=sys.stderr, flush=True)
    inp = synth.make_inputs(cfg)

    # ---- device-resident inputs
    base = gpu_store_all(cfg, inp, device=dev)
    nbytes = base.nbytes
    R = max(1, int(math.ceil(args.cold_mb * 2 ** 20 / nbytes)))
    caches = [base]
    for _ in range(R - 1):
        caches.append(tq.Cache(preset, B, Hk, S, device=dev, buffer=base.buffer.clone()))
    # the same tokens in a paged pool (random page order), R replicas
    table = page_table(B, S)
    pbase = gpu_paged_store_all(cfg, inp, table, device=dev)
    pools = [pbase]
    for _ in range(R - 1):
        pools.append(tq.PagedCache(preset, Hk, pbase.num_pages, device=dev, buffer=pbase.buffer.clone(),
                                   block_table=pbase.block_table))
    si, po = synth.token_lists(B, S, S - N, S)
    Kn = to_dev(synth.rows(inp["K"], S - N, S), dev)
    Vn = to_dev(synth.rows(inp["V"], S - N, S), dev)
    # the same new tokens as [N, B, Hk, 128] for the fused store + verify call
    Kf = to_dev(np.ascontiguousarray(inp["K"][:, S - N:S].transpose(1, 0, 2, 3)), dev)
    Vf = to_dev(np.ascontiguousarray(inp["V"][:, S - N:S].transpose(1, 0, 2, 3)), dev)
    si_d, po_d = to_dev(si, dev), to_dev(po, dev)
    Q = to_dev(inp["Q"], dev)
    sl = to_dev(inp["seq_lens"], dev)
    out = torch.empty((N, B, Hq, 128), dtype=torch.float32, device=dev)
    ws_bytes = max(tq.tqkv_verify_workspace_bytes(base, N, Hq, args.num_splits),
                   tq.tqkv_paged_verify_workspace_bytes(pbase, N, Hq, args.num_splits))
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    splits = tq.tqkv_verify_num_splits(base, N, Hq, args.num_splits)
    torch.cuda.synchronize()
    del inp["K"], inp["V"]

    def store(i):
        tq.tqkv_store(caches[i % R], Kn, Vn, si_d, po_d)

    def verify(i):
        tq.tqkv_verify(caches[i % R], Q, sl, N, Hq, cfg["causal"], num_splits=args.num_splits,
                       out=out, workspace=ws)

    def step(i):
        tq.tqkv_store_verify(caches[i % R], Kf, Vf, Q, sl, N, Hq, cfg["causal"], num_splits=args.num_splits,
                             out=out, workspace=ws)

    def verify_paged(i):
        tq.tqkv_paged_verify(pools[i % R], Q, sl, N, Hq, cfg["causal"], num_splits=args.num_splits,
                             out=out, workspace=ws)

    def step_paged(i):
        tq.tqkv_paged_store_verify(pools[i % R], Kf, Vf, Q, sl, N, Hq, cfg["causal"],
                                   num_splits=args.num_splits, out=out, workspace=ws)

    def step_unfused(i):
        store(i)
        verify(i)

    def capture(fn, n, offset=0):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(offset + i)
        return g

    def time_graph(g):
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        g.replay()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)  # ms

    # ---- eager warmup (also loads the code objects), then graphs
    for i in range(max(1, args.warmup)):
        step(i)
    torch.cuda.synchronize()
    print("bench: capturing graphs (R=%d replicas of %.1f MB, splits=%d)" % (R, nbytes / 1e6, splits),
          file=sys.stderr, flush=True)
    g_warm = capture(step, max(1, args.warmup))
    g_steps = capture(step, args.steps)
    g_verify = capture(verify, args.kernel_calls)
    g_store = capture(store, args.kernel_calls)
    g_unfused = capture(step_unfused, args.kernel_calls)
    g_vpaged = capture(verify_paged, args.kernel_calls)
    g_spaged = capture(step_paged, args.kernel_calls)
    # the first launch of a graph also copies it to the device; that one-time
    # set-up (like the capture) stays out of the timed region, and the
    # warmup steps run right before it (no idle gap for the clocks to drop)
    upload_graph(g_steps)
    g_warm.replay()

    # ---- timed region: exactly K steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g_steps.replay()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms_per_step = wall_ms / args.steps
    print("bench: %d steps in %.3f ms" % (args.steps, wall_ms), file=sys.stderr, flush=True)
    if args.replay_check:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g_steps.replay()
        torch.cuda.synchronize()
        print("bench: second replay %.3f ms" % ((time.perf_counter() - t0) * 1e3), file=sys.stderr, flush=True)

    # the same step graph timed with HIP events (best of 3 replays)
    def median5(g, n):
        return statistics.median(time_graph(g) for _ in range(5)) / n

    step_events_ms = median5(g_steps, args.steps)
    # per-launch durations with HIP events on the launch stream, median of 5
    # replays of a graph of back-to-back calls
    verify_ms = median5(g_verify, args.kernel_calls)
    store_ms = median5(g_store, args.kernel_calls)
    unfused_ms = median5(g_unfused, args.kernel_calls)
    vpaged_ms = median5(g_vpaged, args.kernel_calls)
    spaged_ms = median5(g_spaged, args.kernel_calls)
    # warm (MALL-resident) verify: one replica only
    g_warmv = capture(lambda i: verify(0), args.kernel_calls)
    verify_warm_ms = median5(g_warmv, args.kernel_calls)
    # what a plain read+write stream reaches on this machine: device copies of
    # 256 MB (bytes moved = 2 x 256 MB per copy), median of 5 graphs of 10
    csrc = torch.empty(256 * 10**6, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(csrc)
    g_copy = capture(lambda i: cdst.copy_(csrc), 10)
    copy_gbs = 2 * csrc.numel() / (median5(g_copy, 10) * 1e-3) / 1e9
    del g_copy, csrc, cdst
    # eager steps, for reference
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    kv_bytes = B * S * Hk * slot
    qo_bytes = 2 * N * B * Hq * 128 * 4
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = (kv_bytes + qo_bytes) / (verify_ms * 1e-3) / 1e9
    # the two fp16 contractions Q K^T and P V: 2 FLOPs per (row, token, d) each
    flops = 4 * N * B * Hq * S * 128
    tflops = flops / (verify_ms * 1e-3) / 1e12

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, args.cpu_seconds)

    pages_ms = PAGES_FUSED_TRITON_MS.get(args.workload)
    rec = {
        "metric": "verify-attention µs/call + effective KV GB/s (frac of HBM peak), PoC shape",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(pages_ms / verify_ms, 2) if pages_ms else None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "%s: preset=%s N_spec=%d B=%d Hq=%d Hk=%d D=128 seqlen=%d causal=%s"
                        % (args.workload, {1: "k8v4", 2: "k3v4_nc", 3: "k4v4_nc"}[preset], N, B, Hq, Hk, S,
                           cfg["causal"]),
            "num_splits": splits,
            "cold_replicas": R,
            "step": "tqkv_store_verify: store(N_spec new tokens x B x Hk) + verify(all tokens), one launch",
            "timing": "HIP graph of K steps, one replay",
        },
        "us_per_step": round(ms_per_step * 1e3, 3),
        "us_per_step_events_median_of_5": round(step_events_ms * 1e3, 3),
        "us_per_verify_call": round(verify_ms * 1e3, 3),
        "us_per_store_call": round(store_ms * 1e3, 3),
        "us_per_step_store_then_verify": round(unfused_ms * 1e3, 3),
        "us_per_verify_call_mall_warm": round(verify_warm_ms * 1e3, 3),
        "us_per_verify_call_paged": round(vpaged_ms * 1e3, 3),
        "us_per_step_paged": round(spaged_ms * 1e3, 3),
        "us_per_step_eager": round(eager_ms * 1e3, 3),
        "kv_bytes_per_call": kv_bytes,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(args.workload),
            "kernel": "tqkv_verify: verify_kernel (+ combine_kernel when splits > 1)",
            "bytes_per_launch": kv_bytes + qo_bytes,
            "measured_copy_GBps": round(copy_gbs, 1),
            "frac_of_measured_copy": round(achieved / copy_gbs, 4),
            "mfma": {"flops_per_launch": flops, "achieved": round(tflops, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4)},
        },
        "cpu_baseline": cpu,
    }
    if pages_ms:
        rec["context_pages_b70_fused_triton_us"] = pages_ms * 1e3
    print(json.dumps(rec))


def upload_graph(g):
    """hipGraphUpload of a captured torch graph on the current stream (the
    HIP runtime torch loaded: libtqkv.so and torch share it by soname)."""
    import ctypes

    import torch
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipGraphUpload.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    hip.hipGraphUpload.restype = ctypes.c_int
    rc = hip.hipGraphUpload(ctypes.c_void_p(g.raw_cuda_graph_exec()),
                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != 0:
        raise RuntimeError("hipGraphUpload failed: %d" % rc)
    torch.cuda.synchronize()


def cpu_baseline(cfg, seconds):
    """The oracle (as it stands) timed on this host's cores on a sample of
    the same workload: the full step for as many (b, hk) units as fit in
    about `seconds` of CPU time."""
    import oracle
    from tests import synth

    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    threads = int(os.environ["OMP_NUM_THREADS"])
    N, B, Hq, Hk, S = cfg["N"], cfg["B"], cfg["Hq"], cfg["Hk"], cfg["S"]
    preset = cfg["preset"]
    inp = synth.make_inputs(cfg)
    slot = oracle.slot_bytes(preset)
    # sample: the first nb sequences (all of their KV heads), as many as give
    # every thread a (b, hk) unit -- the oracle's verify, the bulk of the
    # step, runs one thread per unit; the sequences are stored once outside
    # the timing, and the timed part is one step (store of their N new
    # tokens + verify), repeated until `seconds` have passed
    nb = min(B, max(1, threads // Hk))
    cache = np.zeros(oracle.cache_bytes(preset, nb, Hk, S), np.uint8)
    si, po = synth.token_lists(nb, S)
    oracle.store(preset, cache, nb, Hk, S, synth.rows(inp["K"][:nb]), synth.rows(inp["V"][:nb]), si, po)
    si_n, po_n = synth.token_lists(nb, S, S - N, S)
    Kn = synth.rows(inp["K"][:nb], S - N, S)
    Vn = synth.rows(inp["V"][:nb], S - N, S)
    Q = np.ascontiguousarray(inp["Q"][:, :nb])
    sl = inp["seq_lens"][:nb]
    reps, t_total = 0, 0.0
    while t_total < seconds or reps == 0:
        t0 = time.perf_counter()
        oracle.store(preset, cache, nb, Hk, S, Kn, Vn, si_n, po_n)
        oracle.verify(preset, cache, nb, Hk, S, Q, sl, Hq, cfg["causal"])
        t_total += time.perf_counter() - t0
        reps += 1
    per_step = t_total / reps
    kv = nb * S * Hk * slot
    used = min(threads, nb * Hk)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {
        "value": round(kv / per_step / 1e9, 4),
        "unit": "GB/s",
        "cores": used,
        "threads_available": threads,
        "cpu_model": model,
        "kind": "oracle",
        "sample": "%d of %d sequences (all %d KV heads, %d tokens, %d queries each): store of the "
                  "%d new tokens + binary64 verify, %d reps, %.3f s per step" % (
                      nb, B, Hk, S, N * Hq, N, reps, per_step),
    }


if __name__ == "__main__":
    main()
