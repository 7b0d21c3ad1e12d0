"""Helpers shared by the GPU parity tests, the smoke check and the benchmark:
moving seeded host inputs to the device and calling the HIP library, and
computing oracle reference rows for one (b, hk) unit.  No method arithmetic
lives here: the oracle and the HIP library do all of it."""
from __future__ import annotations

import numpy as np
import torch

import quantized_kv_attention_amd as tq
from tests import synth


def to_dev(x: np.ndarray, device="cuda") -> torch.Tensor:
    if x.dtype == np.float16:
        return torch.from_numpy(np.ascontiguousarray(x)).to(device)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def gpu_store_all(cfg: dict, inp: dict, device="cuda", max_seq: int | None = None,
                  chunk_tokens: int = 1 << 22) -> tq.Cache:
    """Store every token of every sequence with tqkv_store (in chunks)."""
    B, S, Hk = cfg["B"], cfg["S"], cfg["Hk"]
    cache = tq.Cache(cfg["preset"], B, Hk, max_seq or S, device=device)
    per = max(1, chunk_tokens // (B * Hk * 128))
    for s0 in range(0, S, per):
        s1 = min(S, s0 + per)
        si, po = synth.token_lists(B, S, s0, s1)
        K = to_dev(synth.rows(inp["K"], s0, s1), device)
        V = to_dev(synth.rows(inp["V"], s0, s1), device)
        tq.tqkv_store(cache, K, V, to_dev(si, device), to_dev(po, device))
    return cache


def page_table(B: int, S: int, seed: int = 1234) -> np.ndarray:
    """A block table [B, ceil(S/16)] holding a random permutation of the
    pool's B * ceil(S/16) pages (neighbouring blocks in unrelated pages)."""
    nblk = (S + 15) // 16
    perm = np.random.default_rng(seed).permutation(B * nblk).astype(np.int32)
    return perm.reshape(B, nblk)


def gpu_paged_store_all(cfg: dict, inp: dict, table: np.ndarray, device="cuda",
                        chunk_tokens: int = 1 << 22) -> tq.PagedCache:
    """Store every token of every sequence into a pool of table.size pages
    with tqkv_paged_store (slot = table[b, t // 16] * 16 + t % 16)."""
    B, S, Hk = cfg["B"], cfg["S"], cfg["Hk"]
    pc = tq.PagedCache(cfg["preset"], Hk, int(table.size), device=device, block_table=to_dev(table, device))
    per = max(1, chunk_tokens // (B * Hk * 128))
    for s0 in range(0, S, per):
        s1 = min(S, s0 + per)
        si, po = synth.token_lists(B, S, s0, s1)
        slots = (table[si, po // 16] * 16 + po % 16).astype(np.int32)
        K = to_dev(synth.rows(inp["K"], s0, s1), device)
        V = to_dev(synth.rows(inp["V"], s0, s1), device)
        tq.tqkv_paged_store(pc, K, V, to_dev(slots, device))
    return pc


def oracle_unit(oracle, cfg: dict, inp: dict, b: int, hk: int, heads=None, causal=None):
    """Oracle output rows [N, nh, 128] (float64) of KV head hk of sequence b,
    for query heads `heads` (default: the whole group), from the raw inputs."""
    N, Hq, Hk, S = cfg["N"], cfg["Hq"], cfg["Hk"], cfg["S"]
    G = Hq // Hk
    heads = list(range(hk * G, (hk + 1) * G)) if heads is None else list(heads)
    causal = cfg["causal"] if causal is None else causal
    L = int(inp["seq_lens"][b])
    preset = cfg["preset"]
    cache = np.zeros(oracle.cache_bytes(preset, 1, 1, S), np.uint8)
    K = np.ascontiguousarray(inp["K"][b, :L, hk][:, None, :])
    V = np.ascontiguousarray(inp["V"][b, :L, hk][:, None, :])
    si = np.zeros(L, np.int32)
    po = np.arange(L, dtype=np.int32)
    oracle.store(preset, cache, 1, 1, S, K, V, si, po)
    # each query head is its own one-head problem against the single KV head
    out = np.zeros((N, len(heads), 128))
    for j, hq in enumerate(heads):
        Q = np.ascontiguousarray(inp["Q"][:, b:b + 1, hq:hq + 1])
        out[:, j] = oracle.verify(preset, cache, 1, 1, S, Q, np.array([L], np.int32), 1, causal)[:, 0, 0]
    return out


def assert_close(got: np.ndarray, ref: np.ndarray, atol=5e-3, rtol=1e-2, what=""):
    """|got - ref| <= atol + rtol * |ref| elementwise, NaN where and only where ref is NaN."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    nan_ref, nan_got = np.isnan(ref), np.isnan(got)
    assert np.array_equal(nan_ref, nan_got), "%s: NaN pattern differs (%d vs %d)" % (
        what, nan_ref.sum(), nan_got.sum())
    ok = ~nan_ref
    err = np.abs(got[ok] - ref[ok])
    bound = atol + rtol * np.abs(ref[ok])
    bad = err > bound
    assert not bad.any(), "%s: %d/%d elements out of tolerance, max err %.3g (bound %.3g)" % (
        what, bad.sum(), bad.size, err.max(), bound[np.argmax(err - bound)])
