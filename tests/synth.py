"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests,
the smoke check and the benchmark.

This module holds no arithmetic of the method: it only draws standard normal
numbers and names the workloads.  Recipe: numpy ``Generator(PCG64(seed))``,
``standard_normal(dtype=float32)`` in C order, draw order Q, then K, then V,
each cast to its stated dtype with round-to-nearest-even.  K and V are drawn
as ``[B, S, Hk, 128]`` (every token of every sequence); Q as
``[N, B, Hq, 128]``.  Every sequence holds ``S`` tokens (the N speculative
tokens included), so ``seq_lens[b] = S`` and ``cached_len = S - N``.

Workloads (names describe the shapes: the pages' PoC shape, a plain decode
and a long-context step):
  tiny_k8v4        N=8 B=1  Hq=8  Hk=1 S=512    causal, Q/K/V fp16, seed 0
  poc_k8v4         N=8 B=4  Hq=32 Hk=4 S=8192   causal, Q fp32,     seed 1
  poc_k3v4_nc      same shape and inputs as poc_k8v4,                 seed 1
  poc_k4v4_nc      same shape and inputs as poc_k8v4,                 seed 1
  decode_k3v4_nc   N=1 B=32 Hq=32 Hk=8 S=32768  non-causal, Q fp32,   seed 3
  long_k3v4_nc     N=8 B=1  Hq=32 Hk=4 S=262144 causal, Q fp32,       seed 4
Held-out parity seeds: 101, 202, 303, 404, 505.
"""
from __future__ import annotations

import numpy as np

K8V4 = 1
K3V4_NC = 2
K4V4_NC = 3
D = 128

HELD_OUT_SEEDS = (101, 202, 303, 404, 505)

CONFIGS = {
    "tiny_k8v4": dict(preset=K8V4, N=8, B=1, Hq=8, Hk=1, S=512, causal=True,
                      q_dtype=np.float16, seed=0),
    "poc_k8v4": dict(preset=K8V4, N=8, B=4, Hq=32, Hk=4, S=8192, causal=True,
                     q_dtype=np.float32, seed=1),
    "poc_k3v4_nc": dict(preset=K3V4_NC, N=8, B=4, Hq=32, Hk=4, S=8192, causal=True,
                        q_dtype=np.float32, seed=1),
    "poc_k4v4_nc": dict(preset=K4V4_NC, N=8, B=4, Hq=32, Hk=4, S=8192, causal=True,
                        q_dtype=np.float32, seed=1),
    "decode_k3v4_nc": dict(preset=K3V4_NC, N=1, B=32, Hq=32, Hk=8, S=32768, causal=False,
                           q_dtype=np.float32, seed=3),
    "long_k3v4_nc": dict(preset=K3V4_NC, N=8, B=1, Hq=32, Hk=4, S=262144, causal=True,
                         q_dtype=np.float32, seed=4),
}


def config(name: str, **override) -> dict:
    cfg = dict(CONFIGS[name])
    cfg["name"] = name
    cfg.update(override)
    return cfg


def _normal(rng: np.random.Generator, shape, dtype, chunk: int = 1 << 24) -> np.ndarray:
    """standard_normal(float32) in C order, cast to dtype; drawn in chunks so
    that large arrays never hold a full float32 copy (the stream is the same
    as one call of the full size)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=dtype)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32).astype(dtype)
    return out.reshape(shape)


def make_inputs(cfg: dict, seed: int | None = None) -> dict:
    """Q [N,B,Hq,D], K/V [B,S,Hk,D] float16, seq_lens [B] int32."""
    seed = cfg["seed"] if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    N, B, Hq, Hk, S = cfg["N"], cfg["B"], cfg["Hq"], cfg["Hk"], cfg["S"]
    Q = _normal(rng, (N, B, Hq, D), cfg["q_dtype"])
    K = _normal(rng, (B, S, Hk, D), np.float16)
    V = _normal(rng, (B, S, Hk, D), np.float16)
    seq_lens = np.full(B, S, dtype=np.int32)
    return dict(Q=Q, K=K, V=V, seq_lens=seq_lens)


def token_lists(B: int, S: int, start: int = 0, stop: int | None = None):
    """seq_idx / pos arrays (int32) for storing positions [start, stop) of
    every sequence, sequence-major (the row order of K[:, start:stop])."""
    stop = S if stop is None else stop
    L = stop - start
    seq_idx = np.repeat(np.arange(B, dtype=np.int32), L)
    pos = np.tile(np.arange(start, stop, dtype=np.int32), B)
    return seq_idx, pos


def rows(K: np.ndarray, start: int = 0, stop: int | None = None) -> np.ndarray:
    """K[:, start:stop] flattened to the [T, Hk, D] token order of token_lists."""
    B, S, Hk, Dd = K.shape
    stop = S if stop is None else stop
    return np.ascontiguousarray(K[:, start:stop].reshape(B * (stop - start), Hk, Dd))
