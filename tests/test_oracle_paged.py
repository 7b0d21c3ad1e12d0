"""Pins of the oracle's paged-pool store and ragged-query verify (CPU only).

The paged store is pinned to the contiguous store: gathered through its
block table, the pool must hold the contiguous cache byte for byte (the
pages count the cache as 16-token blocks of every KV head: "Speculative
decoding on Intel Arc", Part 2, Roofline).  The ragged verify is pinned to
the dense verify (equal counts) and to torch's scaled_dot_product_attention
in float64 with each sequence's own causal window (Part 4: query n of a
window of q queries attends to cached_len + n + 1 tokens, cached_len =
seq_len - q; Part 6: continuation chunks of up to 128 queries)."""
import numpy as np
import pytest
import torch

import oracle
from tests import synth
from tests.test_oracle_verify import _hadamard


def _layout(lens, max_pages, num_pages, seed):
    """A random block table (distinct pages for the live blocks, -1 past
    them) and the slot of every (b, position < lens[b])."""
    rng = np.random.default_rng(seed)
    need = [(L + 15) // 16 for L in lens]
    pages = rng.permutation(num_pages)[:sum(need)]
    table = np.full((len(lens), max_pages), -1, np.int32)
    k = 0
    for b, n in enumerate(need):
        table[b, :n] = pages[k:k + n]
        k += n
    si = np.concatenate([np.full(L, b, np.int32) for b, L in enumerate(lens)])
    po = np.concatenate([np.arange(L, dtype=np.int32) for L in lens])
    slots = table[si, po // 16] * 16 + po % 16
    return table, si, po, slots.astype(np.int32)


@pytest.mark.parametrize("preset", [oracle.K8V4, oracle.K3V4_NC, oracle.K4V4_NC])
def test_paged_store_gathers_to_contiguous_store(preset):
    rng = np.random.default_rng(3)
    lens, Hk, max_pages, num_pages = [37, 16, 50], 2, 4, 19
    table, si, po, slots = _layout(lens, max_pages, num_pages, seed=4)
    T = len(si)
    K = rng.standard_normal((T, Hk, 128)).astype(np.float16)
    V = rng.standard_normal((T, Hk, 128)).astype(np.float16)
    # padding rows (slot -1) carry other data and must not land anywhere
    Kp = np.concatenate([K, rng.standard_normal((3, Hk, 128)).astype(np.float16)])
    Vp = np.concatenate([V, rng.standard_normal((3, Hk, 128)).astype(np.float16)])
    sp = np.concatenate([slots, np.full(3, -1, np.int32)])
    pool = np.zeros(oracle.paged_cache_bytes(preset, Hk, num_pages), np.uint8)
    oracle.store_paged(preset, pool, Hk, num_pages, Kp, Vp, sp)
    contig = np.zeros(oracle.cache_bytes(preset, len(lens), Hk, 16 * max_pages), np.uint8)
    oracle.store(preset, contig, len(lens), Hk, 16 * max_pages, K, V, si, po)
    gathered = oracle.gather_pages(preset, pool, Hk, num_pages, table)
    assert np.array_equal(gathered, contig)
    # pages no table entry names were never written
    used = set(table[table >= 0].tolist())
    blocks = pool.reshape(num_pages, -1)
    for p in range(num_pages):
        if p not in used:
            assert not blocks[p].any()


def test_paged_store_rejects_page_outside_pool():
    pool = np.zeros(oracle.paged_cache_bytes(oracle.K8V4, 1, 2), np.uint8)
    K = np.ones((1, 1, 128), np.float16)
    with pytest.raises(ValueError):
        oracle.store_paged(oracle.K8V4, pool, 1, 2, K, K, np.array([2 * 16], np.int32))


def _contig(preset, B, Hk, S, K, V, lens):
    cache = np.zeros(oracle.cache_bytes(preset, B, Hk, S), np.uint8)
    si = np.concatenate([np.full(L, b, np.int32) for b, L in enumerate(lens)])
    po = np.concatenate([np.arange(L, dtype=np.int32) for L in lens])
    oracle.store(preset, cache, B, Hk, S, K[si, po], V[si, po], si, po)
    return cache


@pytest.mark.parametrize("preset", [oracle.K8V4, oracle.K3V4_NC, oracle.K4V4_NC])
@pytest.mark.parametrize("causal", [True, False])
def test_varlen_with_equal_counts_is_dense_verify(preset, causal):
    rng = np.random.default_rng(8)
    N, B, Hq, Hk, S = 3, 3, 4, 2, 40
    lens = [40, 23, 9]
    K = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
    V = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
    Q = rng.standard_normal((N, B, Hq, 128)).astype(np.float32)
    cache = _contig(preset, B, Hk, S, K, V, lens)
    sl = np.array(lens, np.int32)
    dense = oracle.verify(preset, cache, B, Hk, S, Q, sl, Hq, causal)
    packed = np.ascontiguousarray(Q.transpose(1, 0, 2, 3).reshape(B * N, Hq, 128))
    cu = np.arange(B + 1, dtype=np.int32) * N
    got = oracle.verify_varlen(preset, cache, B, Hk, S, packed, cu, sl, Hq, causal)
    assert np.array_equal(got, dense.transpose(1, 0, 2, 3).reshape(B * N, Hq, 128))


@pytest.mark.parametrize("preset", [oracle.K8V4, oracle.K3V4_NC, oracle.K4V4_NC])
def test_varlen_ragged_matches_sdpa(preset):
    """Counts 1, 0, 12, 5: each sequence's rows against SDPA over its own
    dequantised tokens with the per-row window cached_len + n + 1."""
    rng = np.random.default_rng(9)
    B, Hq, Hk, S = 4, 4, 2, 48
    lens, counts = [30, 11, 48, 5], [1, 0, 12, 5]
    K = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
    V = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
    cache = _contig(preset, B, Hk, S, K, V, lens)
    cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    Q = rng.standard_normal((int(cu[-1]), Hq, 128)).astype(np.float32)
    got = oracle.verify_varlen(preset, cache, B, Hk, S, Q, cu, np.array(lens, np.int32), Hq, True)
    H = _hadamard()
    G = Hq // Hk
    for b in range(B):
        q, L = counts[b], lens[b]
        if q == 0:
            continue
        for hk in range(Hk):
            kv = [oracle.dequant(preset, cache, Hk, S, b, hk, t) for t in range(L)]
            Kh = torch.tensor(np.stack([k for k, _ in kv]))
            Vh = torch.tensor(np.stack([v for _, v in kv]))
            mask = torch.zeros(q, L, dtype=torch.bool)
            for n in range(q):
                mask[n, :max(0, L - q + n + 1)] = True
            for g in range(G):
                hq = hk * G + g
                qv = Q[cu[b]:cu[b + 1], hq].astype(np.float64)
                if preset != oracle.K8V4:
                    qv = qv @ H.T
                ref = torch.nn.functional.scaled_dot_product_attention(
                    torch.tensor(qv)[None, None], Kh[None, None], Vh[None, None],
                    attn_mask=mask[None, None], scale=1 / np.sqrt(128.0))[0, 0].numpy()
                assert np.allclose(got[cu[b]:cu[b + 1], hq], ref, rtol=1e-12, atol=1e-12)
