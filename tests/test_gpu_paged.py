"""GPU parity of the paged-cache and ragged-query entry points (run with -m gpu).

Paged store: the whole pool written by tqkv_paged_store equals, byte for
byte, the pool the oracle's paged store writes.  Paged verify: the output
matches the oracle's attention over the contiguous cache the pool holds
(gathered through the block table), within atol 5e-3, rtol 1e-2, NaN where
the oracle has NaN.  Ragged verify: every sequence's rows match the oracle's
verify of that sequence with its own query count.  The block tables are
random permutations, so the two blocks of a 32-token tile sit in unrelated
pages (also in reverse order).
"""
import numpy as np
import pytest
import torch

import oracle
from tests import synth
from tests.gputil import assert_close, to_dev
from tests.test_oracle_paged import _layout

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("quantized_kv_attention_amd")

PRESETS = [synth.K8V4, synth.K3V4_NC, synth.K4V4_NC]
PNAME = {synth.K8V4: "k8v4", synth.K3V4_NC: "k3v4_nc", synth.K4V4_NC: "k4v4_nc"}


def _kv(rng, B, S, Hk):
    K = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
    V = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
    return K, V


def _pools(preset, K, V, lens, Hk, max_pages, num_pages, seed):
    """(oracle pool, GPU PagedCache with its block table, table) with every
    token below lens[b] stored."""
    table, si, po, slots = _layout(lens, max_pages, num_pages, seed)
    Kr, Vr = np.ascontiguousarray(K[si, po]), np.ascontiguousarray(V[si, po])
    ref = np.zeros(oracle.paged_cache_bytes(preset, Hk, num_pages), np.uint8)
    oracle.store_paged(preset, ref, Hk, num_pages, Kr, Vr, slots)
    pc = tq.PagedCache(preset, Hk, num_pages, block_table=to_dev(table))
    tq.tqkv_paged_store(pc, to_dev(Kr), to_dev(Vr), to_dev(slots))
    return ref, pc, table


def _oracle_dense(preset, ref_pool, Hk, num_pages, table, Q, lens, Hq, causal):
    contig = oracle.gather_pages(preset, ref_pool, Hk, num_pages, table)
    B, max_pages = table.shape
    return oracle.verify(preset, contig, B, Hk, 16 * max_pages, Q, np.array(lens, np.int32), Hq, causal)


# ------------------------------------------------------------------ store ---

@pytest.mark.parametrize("preset", PRESETS, ids=PNAME.get)
def test_paged_store_bit_exact(preset):
    rng = np.random.default_rng(11)
    lens, Hk, max_pages, num_pages = [203, 77, 16], 2, 16, 300
    K, V = _kv(rng, 3, 203, Hk)
    print("paged store", PNAME[preset], flush=True)
    ref, pc, _ = _pools(preset, K, V, lens, Hk, max_pages, num_pages, seed=12)
    torch.cuda.synchronize()
    got = pc.buffer.cpu().numpy()
    assert np.array_equal(got, ref), "%d bytes differ" % int((got != ref).sum())


def test_paged_store_skips_padding_and_pages_outside_the_pool():
    pc = tq.PagedCache(synth.K8V4, 1, 4)
    K = torch.ones((3, 1, 128), dtype=torch.float16, device="cuda")
    sm = torch.tensor([-1, 4 * 16, -100], dtype=torch.int32, device="cuda")
    tq.tqkv_paged_store(pc, K, K, sm)
    torch.cuda.synchronize()
    assert int(pc.buffer.count_nonzero()) == 0


# ----------------------------------------------------------------- verify ---

CASES = [
    dict(N=8, B=2, Hq=16, Hk=2, lens=(203, 150), max_pages=16, num_pages=80, splits=(0, 1, 3)),
    dict(N=1, B=3, Hq=32, Hk=8, lens=(100, 17, 64), max_pages=8, num_pages=40, splits=(0, 2)),
    dict(N=3, B=1, Hq=11, Hk=1, lens=(64,), max_pages=4, num_pages=9, splits=(0,)),
    dict(N=8, B=1, Hq=8, Hk=1, lens=(8,), max_pages=1, num_pages=3, splits=(0,)),
    # one key range over 8192 tokens: 64 tiles per wavefront (both page-id registers)
    dict(N=8, B=1, Hq=8, Hk=1, lens=(8192,), max_pages=512, num_pages=700, splits=(1, 0)),
]


@pytest.mark.parametrize("preset", PRESETS, ids=PNAME.get)
@pytest.mark.parametrize("case", CASES, ids=lambda c: "N%d_Hq%d_Hk%d_L%s" % (
    c["N"], c["Hq"], c["Hk"], "-".join(map(str, c["lens"]))))
def test_paged_verify(preset, case):
    rng = np.random.default_rng(21)
    N, B, Hq, Hk, lens = case["N"], case["B"], case["Hq"], case["Hk"], case["lens"]
    K, V = _kv(rng, B, max(lens), Hk)
    Q = rng.standard_normal((N, B, Hq, 128)).astype(np.float32)
    print("paged verify", PNAME[preset], case, flush=True)
    ref_pool, pc, table = _pools(preset, K, V, lens, Hk, case["max_pages"], case["num_pages"], seed=22)
    ref = _oracle_dense(preset, ref_pool, Hk, case["num_pages"], table, Q, lens, Hq, True)
    for ns in case["splits"]:
        out = tq.tqkv_paged_verify(pc, to_dev(Q), to_dev(np.array(lens, np.int32)), N, Hq, True, num_splits=ns)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), ref, what="num_splits=%d" % ns)


@pytest.mark.parametrize("preset", PRESETS, ids=PNAME.get)
def test_paged_verify_table_entries_outside_the_pool(preset):
    """Entries past a sequence's blocks are never read; an entry outside the
    pool for a live block reads page 0 (the documented behaviour)."""
    rng = np.random.default_rng(31)
    N, B, Hq, Hk, lens, max_pages, num_pages = 4, 2, 8, 2, (90, 40), 8, 20
    K, V = _kv(rng, B, 90, Hk)
    Q = rng.standard_normal((N, B, Hq, 128)).astype(np.float32)
    ref_pool, pc, table = _pools(preset, K, V, lens, Hk, max_pages, num_pages, seed=32)
    bad = table.copy()
    bad[0, 6:] = 1 << 30         # past sequence 0's 6 blocks
    bad[1, 3:] = -7              # past sequence 1's 3 blocks
    bad[1, 1] = num_pages + 5    # a live block outside the pool
    pc.set_block_table(to_dev(bad))
    expect = bad.copy()
    expect[1, 1] = 0
    expect[expect >= num_pages] = -1
    print("paged verify bad table", PNAME[preset], flush=True)
    ref = _oracle_dense(preset, ref_pool, Hk, num_pages, expect, Q, lens, Hq, True)
    out = tq.tqkv_paged_verify(pc, to_dev(Q), to_dev(np.array(lens, np.int32)), N, Hq, True)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, what="bad table")


# ------------------------------------------------------- store + verify ---

@pytest.mark.parametrize("preset", PRESETS, ids=PNAME.get)
@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
# (8, 16): one 64-row work-group per KV head; (16, 16): 16 x 4 row tiles, the
# store runs as its own launch; (8, 32): 128 rows, two 64-row work-groups per
# KV head that both quantise the new tokens inside the verify launch
@pytest.mark.parametrize("N,Hq", [(8, 16), (16, 16), (8, 32)], ids=lambda x: str(x))
@pytest.mark.parametrize("num_splits", [0, 3])
def test_store_verify(preset, paged, N, Hq, num_splits):
    rng = np.random.default_rng(41)
    B, Hk, lens, max_pages, num_pages = 2, 2, (203, 166), 14, 40
    K, V = _kv(rng, B, 203, Hk)
    Q = rng.standard_normal((N, B, Hq, 128)).astype(np.float32)
    sl = np.array(lens, np.int32)
    Kn = np.stack([K[np.arange(B), sl - N + n] for n in range(N)])  # [N, B, Hk, 128]
    Vn = np.stack([V[np.arange(B), sl - N + n] for n in range(N)])
    print("store_verify", PNAME[preset], "paged" if paged else "contiguous", N, Hq, num_splits, flush=True)
    if paged:
        table, si, po, slots = _layout(lens, max_pages, num_pages, seed=42)
        ref_pool = np.zeros(oracle.paged_cache_bytes(preset, Hk, num_pages), np.uint8)
        oracle.store_paged(preset, ref_pool, Hk, num_pages, K[si, po], V[si, po], slots)
        ref = _oracle_dense(preset, ref_pool, Hk, num_pages, table, Q, lens, Hq, True)
        cache = tq.PagedCache(preset, Hk, num_pages, block_table=to_dev(table))
        old = po < sl[si] - N
        tq.tqkv_paged_store(cache, to_dev(np.ascontiguousarray(K[si[old], po[old]])),
                            to_dev(np.ascontiguousarray(V[si[old], po[old]])), to_dev(slots[old]))
    else:
        S = 203
        si = np.concatenate([np.full(L, b, np.int32) for b, L in enumerate(lens)])
        po = np.concatenate([np.arange(L, dtype=np.int32) for L in lens])
        ref_pool = np.zeros(oracle.cache_bytes(preset, B, Hk, S), np.uint8)
        oracle.store(preset, ref_pool, B, Hk, S, K[si, po], V[si, po], si, po)
        ref = oracle.verify(preset, ref_pool, B, Hk, S, Q, sl, Hq, True)
        cache = tq.Cache(preset, B, Hk, S)
        old = po < sl[si] - N
        tq.tqkv_store(cache, to_dev(np.ascontiguousarray(K[si[old], po[old]])),
                      to_dev(np.ascontiguousarray(V[si[old], po[old]])), to_dev(si[old]), to_dev(po[old]))
    out = tq.tqkv_store_verify(cache, to_dev(Kn), to_dev(Vn), to_dev(Q), to_dev(sl), N, Hq, True, num_splits)
    torch.cuda.synchronize()
    got = cache.buffer.cpu().numpy()
    assert np.array_equal(got, ref_pool), "%d bytes differ" % int((got != ref_pool).sum())
    assert_close(out.cpu().numpy(), ref, what="store_verify")


# ----------------------------------------------------- ragged / many rows ---

RAGGED = [
    dict(Hq=8, Hk=2, lens=(100, 40, 203, 8), counts=(1, 0, 17, 8)),   # 68 rows max: 3 row tiles
    dict(Hq=8, Hk=1, lens=(300, 129), counts=(128, 3)),                # 1024 rows: 32 row tiles
    dict(Hq=32, Hk=8, lens=(64, 65, 66), counts=(5, 6, 7)),            # per-sequence draft lengths
    dict(Hq=4, Hk=2, lens=(90, 33, 7, 200), counts=(1, 4, 0, 3)),      # at most 8 rows per KV head
]


@pytest.mark.parametrize("preset", PRESETS, ids=PNAME.get)
@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
@pytest.mark.parametrize("case", RAGGED, ids=lambda c: "q" + "-".join(map(str, c["counts"])))
def test_verify_varlen(preset, paged, case):
    rng = np.random.default_rng(51)
    Hq, Hk, lens, counts = case["Hq"], case["Hk"], case["lens"], case["counts"]
    B, S = len(lens), max(lens)
    K, V = _kv(rng, B, S, Hk)
    cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    Q = rng.standard_normal((int(cu[-1]), Hq, 128)).astype(np.float32)
    sl = np.array(lens, np.int32)
    max_q = max(counts)
    print("varlen", PNAME[preset], "paged" if paged else "contiguous", case, flush=True)
    si = np.concatenate([np.full(L, b, np.int32) for b, L in enumerate(lens)])
    po = np.concatenate([np.arange(L, dtype=np.int32) for L in lens])
    contig = np.zeros(oracle.cache_bytes(preset, B, Hk, S), np.uint8)
    oracle.store(preset, contig, B, Hk, S, K[si, po], V[si, po], si, po)
    ref = oracle.verify_varlen(preset, contig, B, Hk, S, Q, cu, sl, Hq, True)
    if paged:
        max_pages = (S + 15) // 16 + 1
        num_pages = B * max_pages + 3
        _, cache, _ = _pools(preset, K, V, lens, Hk, max_pages, num_pages, seed=52)
    else:
        cache = tq.Cache(preset, B, Hk, S)
        tq.tqkv_store(cache, to_dev(np.ascontiguousarray(K[si, po])), to_dev(np.ascontiguousarray(V[si, po])),
                      to_dev(si), to_dev(po))
    for ns in (0, 2):
        out = tq.tqkv_verify_varlen(cache, to_dev(Q), to_dev(cu), max_q, to_dev(sl), Hq, True, num_splits=ns)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), ref, what="num_splits=%d" % ns)


@pytest.mark.parametrize("preset", PRESETS, ids=PNAME.get)
def test_verify_max_rows(preset):
    """The largest step the library takes: 128 queries x 64 query heads per
    KV head = 8192 rows (the row -> (query, head) split at its limit),
    causal, against the oracle; one more query head is refused."""
    rng = np.random.default_rng(62)
    B, Hq, Hk, N, S = 1, 64, 1, 128, 150
    K, V = _kv(rng, B, S, Hk)
    Q = rng.standard_normal((N, B, Hq, 128)).astype(np.float16)
    sl = np.array([S], np.int32)
    si, po = synth.token_lists(B, S)
    print("max rows", PNAME[preset], flush=True)
    contig = np.zeros(oracle.cache_bytes(preset, B, Hk, S), np.uint8)
    oracle.store(preset, contig, B, Hk, S, K[si, po], V[si, po], si, po)
    ref = oracle.verify(preset, contig, B, Hk, S, Q, sl, Hq, True)
    cache = tq.Cache(preset, B, Hk, S)
    tq.tqkv_store(cache, to_dev(np.ascontiguousarray(K[si, po])), to_dev(np.ascontiguousarray(V[si, po])),
                  to_dev(si), to_dev(po))
    out = tq.tqkv_verify(cache, to_dev(Q), to_dev(sl), N, Hq, True)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, what="8192 rows")
    with pytest.raises(tq.TqkvError):
        tq.tqkv_verify(cache, to_dev(np.zeros((N, B, 72, 128), np.float16)), to_dev(sl), N, 72, True)


@pytest.mark.parametrize("preset", PRESETS, ids=PNAME.get)
@pytest.mark.parametrize("N", [16, 40, 128])
def test_verify_many_queries(preset, N):
    """Dense steps beyond 8 queries (continuation chunks): up to 1024 rows
    per KV head, causal."""
    rng = np.random.default_rng(61)
    B, Hq, Hk, lens = 2, 8, 1, (333, 140)
    S = max(lens)
    K, V = _kv(rng, B, S, Hk)
    Q = rng.standard_normal((N, B, Hq, 128)).astype(np.float16)
    sl = np.array(lens, np.int32)
    si = np.concatenate([np.full(L, b, np.int32) for b, L in enumerate(lens)])
    po = np.concatenate([np.arange(L, dtype=np.int32) for L in lens])
    print("many queries", PNAME[preset], N, flush=True)
    contig = np.zeros(oracle.cache_bytes(preset, B, Hk, S), np.uint8)
    oracle.store(preset, contig, B, Hk, S, K[si, po], V[si, po], si, po)
    ref = oracle.verify(preset, contig, B, Hk, S, Q, sl, Hq, True)
    cache = tq.Cache(preset, B, Hk, S)
    tq.tqkv_store(cache, to_dev(np.ascontiguousarray(K[si, po])), to_dev(np.ascontiguousarray(V[si, po])),
                  to_dev(si), to_dev(po))
    for ns in (0, 3):
        out = tq.tqkv_verify(cache, to_dev(Q), to_dev(sl), N, Hq, True, num_splits=ns)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), ref, what="N=%d splits=%d" % (N, ns))
