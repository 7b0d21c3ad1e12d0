"""Phase timeline of verify_wide_kernel (the 64-row work-groups).

Builds a separate copy of the library with -DTQKV_PHASE_TRACE
(libtqkv_phase_trace.so next to this file: the kernel keeps s_memrealtime
stamps in registers and stores them after its key loop and at its end), runs
a graph of back-to-back calls of one workload on synthetic inputs (cold
cache replicas, like bench.py), and prints the median time of every phase
from the work-group's start, for the work-groups that store new tokens (a
fused store + verify step) and for the others, plus the shader clock the
loop ran at.

    python -m quantized_kv_attention_amd.phase_trace --workload poc_k8v4 [--fused]

Run from the repository root (the synthetic inputs come from tests/synth.py).
Timing only: the trace copy is not the library the package loads.
"""
from __future__ import annotations

import argparse
import ctypes
import math
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
TRACE_LIB = os.path.join(HERE, "libtqkv_phase_trace.so")
WGS, SLOTS = 4096, 24  # kTraceWGs, kTraceSlots of verify.hip
LABELS = {0: "start", 16: "store start", 17: "stores issued", 1: "query landed", 2: "key loop start",
          3: "tile 1 landed", 4: "tile 1 max", 5: "tile 1 issued", 6: "tile 2 landed", 7: "tile 2 max",
          8: "tile 2 issued", 9: "tile 3 landed", 12: "tile 4 landed", 15: "key loop end", 18: "merge done",
          19: "outputs start"}
ORDER = (0, 16, 17, 1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 15, 18, 19)


def build_trace_library() -> str:
    sys.path.insert(0, HERE)
    import build as B
    return B.build(["-DTQKV_PHASE_TRACE"], out=TRACE_LIB)


def run(workload: str, fused: bool, calls: int = 40):
    import torch

    import quantized_kv_attention_amd as tq
    from tests import synth
    from tests.gputil import gpu_store_all, to_dev

    tq._lib = None
    tq.library_path = TRACE_LIB
    lib = tq._load()
    lib.tqkv_debug_phase_trace.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    cfg = synth.config(workload)
    inp = synth.make_inputs(cfg)
    N, B, Hq, Hk, S = cfg["N"], cfg["B"], cfg["Hq"], cfg["Hk"], cfg["S"]
    base = gpu_store_all(cfg, inp)
    R = max(1, int(math.ceil(512 * 2**20 / base.nbytes)))
    caches = [base] + [tq.Cache(cfg["preset"], B, Hk, S, buffer=base.buffer.clone()) for _ in range(R - 1)]
    Kf = to_dev(np.ascontiguousarray(inp["K"][:, S - N:S].transpose(1, 0, 2, 3)))
    Vf = to_dev(np.ascontiguousarray(inp["V"][:, S - N:S].transpose(1, 0, 2, 3)))
    Q, sl = to_dev(inp["Q"]), to_dev(inp["seq_lens"])
    out = torch.empty((N, B, Hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(16, tq.tqkv_verify_workspace_bytes(base, N, Hq, 0)), dtype=torch.uint8, device="cuda")

    def call(i):
        if fused:
            tq.tqkv_store_verify(caches[i % R], Kf, Vf, Q, sl, N, Hq, cfg["causal"], out=out, workspace=ws)
        else:
            tq.tqkv_verify(caches[i % R], Q, sl, N, Hq, cfg["causal"], out=out, workspace=ws)

    for i in range(3):
        call(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            call(i)
    for _ in range(2):
        g.replay()
        torch.cuda.synchronize()
    buf = np.zeros(WGS * 8 * SLOTS, np.uint32)
    if lib.tqkv_debug_phase_trace(buf.ctypes.data, buf.nbytes) != 0:
        raise RuntimeError("tqkv_debug_phase_trace failed")
    return buf.reshape(WGS, 8, SLOTS).astype(np.int64)


def summarise(t: np.ndarray, title: str) -> str:
    n = int((t[:, :, 2] != 0).any(axis=1).sum())  # work-groups that reached the key loop
    if n == 0:
        return "%s: no work-group of verify_wide_kernel ran (the call took the 32-row work-groups)" % title
    t = t[:n]
    start = np.where(t[:, :, 0] != 0, t[:, :, 0], np.iinfo(np.int64).max)
    ws0 = start.min(axis=1)  # the work-group's first wavefront start (four-wavefront groups fill slots 0-3)
    rel = lambda v, s0: ((v - s0) % 2**32) / 100.0  # noqa: E731  100 MHz ticks -> us
    lines = ["%s: %d work-groups; us from each work-group's start, median over work-groups" % (title, n)]
    storing = t[:, 0, 20] == 1
    for name, m in (("storing new tokens", storing), ("other", ~storing)):
        if not m.any():
            continue
        lines.append("%s (%d):" % (name, int(m.sum())))
        for w in range(8):
            if not (t[m][:, w, 0] != 0).any():
                continue  # a work-group of four wavefronts
            row = []
            for k in ORDER:
                v = t[m][:, w, k]
                ok = v != 0
                if ok.sum() == 0 or (k != 0 and ok.sum() < m.sum() // 2):
                    continue
                row.append("%s %.2f" % (LABELS[k], np.median(rel(v[ok], ws0[m][ok]))))
            loop_ticks = (t[m][:, w, 15] - t[m][:, w, 2]) % 2**32
            cyc = (t[m][:, w, 23] - t[m][:, w, 22]) % 2**32
            okc = loop_ticks > 0
            clk = np.median(cyc[okc] / (loop_ticks[okc] / 100.0)) / 1e3 if okc.any() else float("nan")
            lines.append("  wavefront %d (%.2f GHz in the loop): %s" % (w, clk, ", ".join(row)))
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="poc_k8v4")
    ap.add_argument("--fused", action="store_true", help="trace tqkv_store_verify instead of tqkv_verify")
    ap.add_argument("--no-build", action="store_true", help="use an existing libtqkv_phase_trace.so")
    args = ap.parse_args()
    if not args.no_build or not os.path.exists(TRACE_LIB):
        build_trace_library()
    t = run(args.workload, args.fused)
    print(summarise(t, "%s %s" % (args.workload, "store + verify" if args.fused else "verify")))


if __name__ == "__main__":
    main()
