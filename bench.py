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
    ap.add_argument("--no-nested", action="store_true",
                    help="time only --workload (not the other workloads' nested entries)")
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


ALL_WORKLOADS = ("poc_k8v4", "poc_k3v4_nc", "poc_k4v4_nc", "long_k3v4_nc", "decode_k3v4_nc")
PRESET_NAME = {1: "k8v4", 2: "k3v4_nc", 3: "k4v4_nc"}


def workload_label(name, cfg):
    return "%s: preset=%s N_spec=%d B=%d Hq=%d Hk=%d D=128 seqlen=%d causal=%s" % (
        name, PRESET_NAME[cfg["preset"]], cfg["N"], cfg["B"], cfg["Hq"], cfg["Hk"], cfg["S"], cfg["causal"])


def capture(fn, n, offset=0):
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(offset + i)
    return g


def time_graph(g):
    """Duration (ms) of one replay, HIP events on the launch stream."""
    import torch
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    g.replay()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def median5(g, n):
    """Per-call ms of a graph of n calls: median of 5 replays."""
    return statistics.median(time_graph(g) for _ in range(5)) / n


class Workload:
    """Device-resident inputs of one workload: R byte-identical cache
    replicas (R * bytes >= cold_mb), a paged pool with its replicas (primary
    only), the queries, the N_spec new tokens of the step and the outputs.

    host=True: the inputs of tests/synth.py (the host generator the parity
    tests use); host=False: the same distributions drawn on the device with
    torch's seeded generator (the decode inputs take about a minute on the
    host), the cache filled by one bulk tqkv_store call of every token."""

    def __init__(self, name, args, dev, host, paged):
        import torch

        import quantized_kv_attention_amd as tq
        from tests import synth
        from tests.gputil import gpu_paged_store_all, gpu_store_all, page_table, to_dev

        self.name, self.dev = name, dev
        cfg = self.cfg = synth.config(name)
        N, B, Hq, Hk, S = cfg["N"], cfg["B"], cfg["Hq"], cfg["Hk"], cfg["S"]
        self.preset = cfg["preset"]
        print("bench: workload %s, generating inputs" % name, file=sys.stderr, flush=True)
        if host:
            inp = synth.make_inputs(cfg)
            base = gpu_store_all(cfg, inp, device=dev)
            self.Q = to_dev(inp["Q"], dev)
            # the step's N new tokens of every sequence as [N, B, Hk, 128]
            self.Kf = to_dev(np.ascontiguousarray(inp["K"][:, S - N:S].transpose(1, 0, 2, 3)), dev)
            self.Vf = to_dev(np.ascontiguousarray(inp["V"][:, S - N:S].transpose(1, 0, 2, 3)), dev)
            self.host_inputs = inp
        else:
            g = torch.Generator(device=dev)
            g.manual_seed(cfg["seed"])
            self.Q = torch.randn((N, B, Hq, 128), generator=g, device=dev, dtype=torch.float32)
            K = torch.randn((B, S, Hk, 128), generator=g, device=dev, dtype=torch.float16)
            V = torch.randn((B, S, Hk, 128), generator=g, device=dev, dtype=torch.float16)
            base = tq.Cache(self.preset, B, Hk, S, device=dev)
            si = torch.arange(B, dtype=torch.int32, device=dev).repeat_interleave(S)
            po = torch.arange(S, dtype=torch.int32, device=dev).repeat(B)
            tq.tqkv_store(base, K.view(B * S, Hk, 128), V.view(B * S, Hk, 128), si, po)
            self.Kf = K[:, S - N:S].transpose(0, 1).contiguous()
            self.Vf = V[:, S - N:S].transpose(0, 1).contiguous()
            self.host_inputs = None
            self.bulk = (K.view(B * S, Hk, 128), V.view(B * S, Hk, 128), si, po)
        self.sl = torch.full((B,), S, dtype=torch.int32, device=dev)
        self.nbytes = base.nbytes
        self.R = max(1, int(math.ceil(args.cold_mb * 2 ** 20 / self.nbytes)))
        self.caches = [base] + [tq.Cache(self.preset, B, Hk, S, device=dev, buffer=base.buffer.clone())
                                for _ in range(self.R - 1)]
        self.pools = None
        if paged:
            table = page_table(B, S)
            pbase = gpu_paged_store_all(cfg, self.host_inputs, table, device=dev)
            self.pools = [pbase] + [tq.PagedCache(self.preset, Hk, pbase.num_pages, device=dev,
                                                  buffer=pbase.buffer.clone(), block_table=pbase.block_table)
                                    for _ in range(self.R - 1)]
        self.out = torch.empty((N, B, Hq, 128), dtype=torch.float32, device=dev)
        ws = 16
        for ns in (args.num_splits, 8):
            ws = max(ws, tq.tqkv_verify_workspace_bytes(base, N, Hq, ns))
            if paged:
                ws = max(ws, tq.tqkv_paged_verify_workspace_bytes(self.pools[0], N, Hq, ns))
        self.ws = torch.empty(ws, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    def verify(self, i, ns):
        import quantized_kv_attention_amd as tq
        c = self.cfg
        tq.tqkv_verify(self.caches[i % self.R], self.Q, self.sl, c["N"], c["Hq"], c["causal"], num_splits=ns,
                       out=self.out, workspace=self.ws)

    def step(self, i, ns):
        import quantized_kv_attention_amd as tq
        c = self.cfg
        tq.tqkv_store_verify(self.caches[i % self.R], self.Kf, self.Vf, self.Q, self.sl, c["N"], c["Hq"],
                             c["causal"], num_splits=ns, out=self.out, workspace=self.ws)

    def verify_paged(self, i, ns):
        import quantized_kv_attention_amd as tq
        c = self.cfg
        tq.tqkv_paged_verify(self.pools[i % self.R], self.Q, self.sl, c["N"], c["Hq"], c["causal"],
                             num_splits=ns, out=self.out, workspace=self.ws)

    def step_paged(self, i, ns):
        import quantized_kv_attention_amd as tq
        c = self.cfg
        tq.tqkv_paged_store_verify(self.pools[i % self.R], self.Kf, self.Vf, self.Q, self.sl, c["N"], c["Hq"],
                                   c["causal"], num_splits=ns, out=self.out, workspace=self.ws)

    def store_bulk_us(self, calls):
        """Per-call us of a bulk tqkv_store of every token of the workload
        (all B * S tokens, all KV heads) into a scratch cache."""
        import torch

        import quantized_kv_attention_amd as tq
        from tests import synth
        from tests.gputil import to_dev
        c = self.cfg
        B, S, Hk = c["B"], c["S"], c["Hk"]
        if self.host_inputs is not None:
            si, po = synth.token_lists(B, S)
            K = to_dev(synth.rows(self.host_inputs["K"]), self.dev)
            V = to_dev(synth.rows(self.host_inputs["V"]), self.dev)
            si, po = to_dev(si, self.dev), to_dev(po, self.dev)
        else:
            K, V, si, po = self.bulk
        dst = tq.Cache(self.preset, B, Hk, S, device=self.dev)
        tq.tqkv_store(dst, K, V, si, po)
        g = capture(lambda i: tq.tqkv_store(dst, K, V, si, po), calls)
        us = median5(g, calls) * 1e3
        del g, dst
        torch.cuda.empty_cache()
        return us

    def release(self):
        import torch
        self.caches = self.pools = self.bulk = self.host_inputs = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def verify_kernels(cfg, splits):
    """The launches of one plain tqkv_verify call at this configuration, as
    the library chooses them: one 64-row work-group per compute unit for more
    than 32 query rows per KV head (verify_wide_kernel, four wavefronts for
    k8v4 / k4v4_nc key ranges of at most 32 tiles of 32 tokens, eight
    otherwise), 32-row work-groups (verify_kernel) for fewer rows; then the
    key-range merge when there is more than one range."""
    rows = cfg["Hq"] // cfg["Hk"] * cfg["N"]
    tiles = (cfg["S"] + 31) // 32
    per_range = (tiles + splits - 1) // splits
    if rows > 32:
        waves = 4 if cfg["preset"] != 2 and per_range <= 32 else 8
        names = "verify_wide_kernel (%d wavefronts)" % waves
    else:
        names = "verify_kernel"
    return names + (" + combine_kernel" if splits > 1 else "")


def verify_entry(w, args):
    """us per call of the verify launch (auto splits and 8 splits), of the
    fused step, of a bulk store of every token, and the verify roofline."""
    import quantized_kv_attention_amd as tq
    c = w.cfg
    N, B, Hq, Hk, S = c["N"], c["B"], c["Hq"], c["Hk"], c["S"]
    slot = tq.tqkv_slot_bytes(w.preset)
    calls = args.kernel_calls
    ns = args.num_splits
    # warm the code objects outside the graphs
    w.verify(0, ns)
    w.step(0, ns)
    verify_ms = median5(capture(lambda i: w.verify(i, ns), calls), calls)
    verify8_ms = median5(capture(lambda i: w.verify(i, 8), calls), calls)
    step_ms = median5(capture(lambda i: w.step(i, ns), calls), calls)
    bulk_us = w.store_bulk_us(max(2, calls // 20))
    kv_bytes = B * S * Hk * slot
    qo_bytes = 2 * N * B * Hq * 128 * 4
    achieved = (kv_bytes + qo_bytes) / (verify_ms * 1e-3) / 1e9
    flops = 4 * N * B * Hq * S * 128
    tflops = flops / (verify_ms * 1e-3) / 1e12
    th = B * S * Hk
    bulk_bytes = th * (2 * 128 * 2 + slot)  # fp16 K and V read, the packed token-head written
    return {
        "workload": workload_label(w.name, c),
        "num_splits": tq.tqkv_verify_num_splits(w.caches[0], N, Hq, ns),
        "cold_replicas": w.R,
        "us_per_verify_call": round(verify_ms * 1e3, 3),
        "us_per_verify_call_splits8": round(verify8_ms * 1e3, 3),
        "us_per_step": round(step_ms * 1e3, 3),
        "kv_bytes_per_call": kv_bytes,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(w.name),
            "bytes_per_launch": kv_bytes + qo_bytes,
            "kernel": "tqkv_verify: " + verify_kernels(c, tq.tqkv_verify_num_splits(w.caches[0], N, Hq, ns)),
            "mfma": {"flops_per_launch": flops, "achieved": round(tflops, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4)},
        },
        "store_bulk": {
            "token_heads": th,
            "bytes_per_token_head": 2 * 128 * 2 + slot,
            "us_per_call": round(bulk_us, 3),
            "achieved": round(bulk_bytes / (bulk_us * 1e-6) / 1e9, 1),
            "unit": "GB/s",
            "frac": round(bulk_bytes / (bulk_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        },
    }


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

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = Workload(args.workload, args, dev, host=True, paged=True)
    cfg = w.cfg
    N, B, Hq, Hk, S = cfg["N"], cfg["B"], cfg["Hq"], cfg["Hk"], cfg["S"]
    slot = tq.tqkv_slot_bytes(w.preset)
    ns = args.num_splits
    splits = tq.tqkv_verify_num_splits(w.caches[0], N, Hq, ns)
    # the step's store alone (N new tokens per sequence), for the unfused pair
    from tests import synth
    from tests.gputil import to_dev
    si, po = synth.token_lists(B, S, S - N, S)
    Kn = to_dev(synth.rows(w.host_inputs["K"], S - N, S), dev)
    Vn = to_dev(synth.rows(w.host_inputs["V"], S - N, S), dev)
    si_d, po_d = to_dev(si, dev), to_dev(po, dev)

    def store(i):
        tq.tqkv_store(w.caches[i % w.R], Kn, Vn, si_d, po_d)

    def step_unfused(i):
        store(i)
        w.verify(i, ns)

    # ---- eager warmup (also loads the code objects), then graphs
    for i in range(max(1, args.warmup)):
        w.step(i, ns)
    torch.cuda.synchronize()
    print("bench: capturing graphs (R=%d replicas of %.1f MB, splits=%d)" % (w.R, w.nbytes / 1e6, splits),
          file=sys.stderr, flush=True)
    g_warm = capture(lambda i: w.step(i, ns), max(1, args.warmup))
    # the timed steps continue the replica sequence where the warmup stops,
    # so no timed step starts on a replica the warmup has just touched
    g_steps = capture(lambda i: w.step(i, ns), args.steps, offset=max(1, args.warmup))
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

    calls = args.kernel_calls
    step_events_ms = median5(g_steps, args.steps)
    del g_steps, g_warm
    # per-launch durations with HIP events on the launch stream, median of 5
    # replays of a graph of back-to-back calls
    entry = verify_entry(w, args)
    verify_ms = entry["us_per_verify_call"] * 1e-3
    store_ms = median5(capture(store, calls), calls)
    unfused_ms = median5(capture(step_unfused, calls), calls)
    vpaged_ms = median5(capture(lambda i: w.verify_paged(i, ns), calls), calls)
    spaged_ms = median5(capture(lambda i: w.step_paged(i, ns), calls), calls)
    # warm (MALL-resident) verify: one replica only
    verify_warm_ms = median5(capture(lambda i: w.verify(0, ns), calls), calls)
    # what a plain read+write stream reaches on this machine: device copies of
    # 256 MB (bytes moved = 2 x 256 MB per copy), median of 5 graphs of 10
    csrc = torch.empty(256 * 10**6, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(csrc)
    copy_gbs = 2 * csrc.numel() / (median5(capture(lambda i: cdst.copy_(csrc), 10), 10) * 1e-3) / 1e9
    del csrc, cdst
    # eager steps, for reference
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        w.step(i, ns)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    host_inputs = w.host_inputs
    w.release()

    # ---- the other workloads: verify, step and bulk store, nested
    nested = {}
    if not args.no_nested:
        for name in ALL_WORKLOADS:
            if name == args.workload:
                continue
            wn = Workload(name, args, dev, host=False, paged=False)
            nested[name] = verify_entry(wn, args)
            wn.release()
            del wn

    kv_bytes = B * S * Hk * slot
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, host_inputs, args.cpu_seconds)

    pages_ms = PAGES_FUSED_TRITON_MS.get(args.workload)
    roof = dict(entry["roofline"])
    roof["measured_copy_GBps"] = round(copy_gbs, 1)
    roof["frac_of_measured_copy"] = round(roof["achieved"] / copy_gbs, 4)
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
            "workload": workload_label(args.workload, cfg),
            "num_splits": splits,
            "cold_replicas": w.R,
            "step": "tqkv_store_verify: store(N_spec new tokens x B x Hk) + verify(all tokens), one launch",
            "timing": "HIP graph of K steps, one replay",
        },
        "us_per_step": round(ms_per_step * 1e3, 3),
        "us_per_step_events_median_of_5": round(step_events_ms * 1e3, 3),
        "us_per_verify_call": entry["us_per_verify_call"],
        "us_per_verify_call_splits8": entry["us_per_verify_call_splits8"],
        "us_per_store_call": round(store_ms * 1e3, 3),
        "us_per_step_store_then_verify": round(unfused_ms * 1e3, 3),
        "us_per_verify_call_mall_warm": round(verify_warm_ms * 1e3, 3),
        "us_per_verify_call_paged": round(vpaged_ms * 1e3, 3),
        "us_per_step_paged": round(spaged_ms * 1e3, 3),
        "us_per_step_eager": round(eager_ms * 1e3, 3),
        "kv_bytes_per_call": kv_bytes,
        "store_bulk": entry["store_bulk"],
        "roofline": roof,
        "cpu_baseline": cpu,
        "workloads": nested,
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


def _omp_set_threads(n):
    """Thread count of the oracle's OpenMP loops (the runtime libtqoracle.so
    links is process-wide)."""
    import ctypes
    ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))


def cpu_baseline(cfg, inp, seconds):
    """The oracle (as it stands) timed on this host's cores on a sample of
    the same workload, with every available thread and with one: one step
    (store of the N new tokens + verify) for a few (b, hk) units, repeated
    until about `seconds` have passed in each leg."""
    import oracle
    from tests import synth

    cores = len(os.sched_getaffinity(0))
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    N, B, Hq, Hk, S = cfg["N"], cfg["B"], cfg["Hq"], cfg["Hk"], cfg["S"]
    preset = cfg["preset"]
    slot = oracle.slot_bytes(preset)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass

    def leg(nthreads):
        _omp_set_threads(nthreads)
        # sample: the first nb sequences (all of their KV heads), as many as
        # give every thread a (b, hk) unit -- the oracle's verify, the bulk of
        # the step, runs one thread per unit; the sequences are stored once
        # outside the timing
        nb = min(B, max(1, nthreads // Hk))
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
        return {
            "value": round(kv / per_step / 1e9, 4),
            "unit": "GB/s",
            "cores": min(nthreads, nb * Hk),
            "kind": "oracle",
            "sample": "%d of %d sequences (all %d KV heads, %d tokens, %d queries each): store of the "
                      "%d new tokens + binary64 verify, %d reps, %.3f s per step" % (
                          nb, B, Hk, S, N * Hq, N, reps, per_step),
        }

    rec = leg(threads)
    rec["threads_available"] = threads
    rec["cpu_model"] = model
    rec["single_thread"] = leg(1)
    _omp_set_threads(threads)
    return rec


if __name__ == "__main__":
    main()
