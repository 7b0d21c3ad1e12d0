"""GPU parity of the HIP library against the CPU oracle (run with -m gpu).

Codes: the whole physical cache written by tqkv_store must equal, byte for
byte, the cache the oracle writes from the same fp16 inputs.  Outputs:
tqkv_verify must match the oracle's binary64 attention within atol 5e-3,
rtol 1e-2 (the tolerance of the pages' integration test, Part 6 of
"Speculative decoding on Intel Arc: TurboQuant KV + a fused N_spec kernel"),
with NaN exactly where the oracle has NaN.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
from tests import synth
from tests.gputil import assert_close, gpu_store_all, oracle_unit, to_dev

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("quantized_kv_attention_amd")

PRESETS = [synth.K8V4, synth.K3V4_NC, synth.K4V4_NC]
PNAME = {synth.K8V4: "k8v4", synth.K3V4_NC: "k3v4_nc", synth.K4V4_NC: "k4v4_nc"}


def _small(preset, **kw):
    cfg = dict(preset=preset, N=8, B=2, Hq=16, Hk=2, S=203, causal=True, q_dtype=np.float32, seed=7)
    cfg.update(kw)
    return cfg


@functools.lru_cache(maxsize=2)
def _config_inputs(name):
    """Inputs of a named configuration, kept for the large ones (decode: 4.3 GB,
    about a minute to draw) so the store and verify tests draw them once."""
    return synth.make_inputs(synth.config(name))


def _oracle_cache(cfg, inp, max_seq=None):
    B, S, Hk = cfg["B"], cfg["S"], cfg["Hk"]
    max_seq = max_seq or S
    cache = np.zeros(oracle.cache_bytes(cfg["preset"], B, Hk, max_seq), np.uint8)
    si, po = synth.token_lists(B, S)
    oracle.store(cfg["preset"], cache, B, Hk, max_seq, synth.rows(inp["K"]), synth.rows(inp["V"]), si, po)
    return cache


def _gpu_verify(cache, cfg, inp, **kw):
    Q = to_dev(inp["Q"])
    sl = to_dev(inp["seq_lens"])
    out = tq.tqkv_verify(cache, Q, sl, cfg["N"], cfg["Hq"], cfg["causal"], **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy()


# ------------------------------------------------------------------ store ---

@pytest.mark.parametrize("preset", PRESETS, ids=PNAME.get)
@pytest.mark.parametrize("seed", [0] + list(synth.HELD_OUT_SEEDS))
def test_store_bit_exact_small(preset, seed):
    cfg = _small(preset, seed=seed)
    inp = synth.make_inputs(cfg)
    print("store small", PNAME[preset], "seed", seed, flush=True)
    ref = _oracle_cache(cfg, inp)
    got = gpu_store_all(cfg, inp).buffer.cpu().numpy()
    assert np.array_equal(got, ref), "%d bytes differ" % int((got != ref).sum())


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["tiny_k8v4", "poc_k8v4", "poc_k3v4_nc", "poc_k4v4_nc", "decode_k3v4_nc",
                                  "long_k3v4_nc"])
def test_store_bit_exact_config(name):
    """The whole cache of every configuration, byte for byte (decode: 8.4M
    token-heads, 1 GB; long context: 1M token-heads)."""
    cfg = synth.config(name)
    print("store", name, "generating inputs", flush=True)
    inp = _config_inputs(name) if name in ("decode_k3v4_nc", "long_k3v4_nc") else synth.make_inputs(cfg)
    print("store", name, "oracle", flush=True)
    ref = _oracle_cache(cfg, inp)
    print("store", name, "gpu", flush=True)
    got = gpu_store_all(cfg, inp).buffer.cpu().numpy()
    torch.cuda.empty_cache()
    assert np.array_equal(got, ref), "%d bytes differ" % int((got != ref).sum())


@pytest.mark.parametrize("preset", PRESETS, ids=PNAME.get)
def test_store_edge_vectors(preset):
    """Zero, constant, tiny, huge, mixed-sign-zero and tie-prone vectors."""
    rng = np.random.default_rng(99)
    vecs = [
        np.zeros(128), np.full(128, 1.5), np.full(128, -3.0), rng.standard_normal(128) * 1e-4,
        rng.standard_normal(128) * 3e4, np.where(rng.random(128) < 0.5, 0.0, -0.0),
        np.round(rng.standard_normal(128) * 4) / 4, np.arange(128) - 64.0, (np.arange(128) % 16) * 0.5,
        rng.standard_normal(128) * 1e-6, np.concatenate([[-0.0], np.linspace(0.1, 3.0, 127)]),
    ]
    T = len(vecs)
    K = np.stack(vecs).astype(np.float16)[:, None, :]
    V = np.stack(vecs[::-1]).astype(np.float16)[:, None, :]
    si = np.zeros(T, np.int32)
    po = (np.arange(T, dtype=np.int32) * 5) % 37  # scattered, distinct positions
    ref = np.zeros(oracle.cache_bytes(preset, 1, 1, 40), np.uint8)
    oracle.store(preset, ref, 1, 1, 40, K, V, si, po)
    cache = tq.Cache(preset, 1, 1, 40)
    tq.tqkv_store(cache, to_dev(K), to_dev(V), to_dev(si), to_dev(po))
    got = cache.buffer.cpu().numpy()
    assert np.array_equal(got, ref), "%d bytes differ" % int((got != ref).sum())


def _binary16_up_to(a):
    """Every finite binary16 x with |x| <= a, both signs (+0 and -0 included)."""
    mags = np.arange(0x7C00, dtype=np.uint16).view(np.float16)
    mags = mags[mags <= np.float16(a)]
    return np.concatenate([mags, -mags])


def _every_binary16_rows():
    """Token-head rows [T, 128] (T = 3168) holding every finite binary16 below
    each of a range of maxima (subnormal, tiny, near 1, 448, the binary16
    maximum): each row is its maximum and 127 values at most as large."""
    maxima = [2.0**-24, 2.0**-17, 2.0**-14, 1e-3, 0.1, 1.0, 1.5, np.pi, 100.0, 448.0, 1000.0, 3e4, 65504.0]
    rng = np.random.default_rng(5)
    rows = []
    for a in maxima:
        xs = rng.permutation(_binary16_up_to(a))
        for i in range(0, len(xs), 127):
            chunk = xs[i:i + 127]
            if len(chunk) < 127:
                chunk = np.concatenate([chunk, rng.choice(xs, 127 - len(chunk))])
            rows.append(np.concatenate([[np.float16(a)], chunk]))
    return np.stack(rows).astype(np.float16)


@pytest.mark.parametrize("preset", PRESETS, ids=PNAME.get)
def test_store_every_binary16_value(preset):
    """With these rows as keys and (reversed) as values, the FP8 key codes meet
    every quotient x / s that their scale s allows, and the value codes every
    (v - zero) / s of a wide range (rounding boundaries and ties included)."""
    K = _every_binary16_rows()[:, None, :]
    V = np.ascontiguousarray(K[:, :, ::-1])
    T = K.shape[0]
    si = np.zeros(T, np.int32)
    po = np.arange(T, dtype=np.int32)
    print("store every binary16", PNAME[preset], T, "token-heads", flush=True)
    ref = np.zeros(oracle.cache_bytes(preset, 1, 1, T), np.uint8)
    oracle.store(preset, ref, 1, 1, T, K, V, si, po)
    cache = tq.Cache(preset, 1, 1, T)
    tq.tqkv_store(cache, to_dev(K), to_dev(V), to_dev(si), to_dev(po))
    got = cache.buffer.cpu().numpy()
    assert np.array_equal(got, ref), "%d bytes differ" % int((got != ref).sum())


def test_store_skips_out_of_range_and_empty():
    cache = tq.Cache(synth.K8V4, 2, 1, 20)
    K = torch.ones((3, 1, 128), dtype=torch.float16, device="cuda")
    si = torch.tensor([0, 2, -1], dtype=torch.int32, device="cuda")
    po = torch.tensor([20, 0, 3], dtype=torch.int32, device="cuda")
    tq.tqkv_store(cache, K, K, si, po)
    tq.tqkv_store(cache, K[:0], K[:0], si[:0], po[:0])
    torch.cuda.synchronize()
    assert int(cache.buffer.count_nonzero()) == 0


# ----------------------------------------------------------------- verify ---

@pytest.mark.parametrize("preset", PRESETS, ids=PNAME.get)
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("q_dtype", [np.float32, np.float16])
def test_verify_small(preset, causal, q_dtype):
    cfg = _small(preset, causal=causal, q_dtype=q_dtype)
    inp = synth.make_inputs(cfg)
    inp["seq_lens"] = np.array([203, 150], np.int32)  # ragged: a tail tile, two lengths
    print("verify small", PNAME[preset], causal, q_dtype.__name__, flush=True)
    ocache = _oracle_cache(cfg, inp)
    ref = oracle.verify(preset, ocache, cfg["B"], cfg["Hk"], cfg["S"], inp["Q"], inp["seq_lens"],
                        cfg["Hq"], causal)
    cache = gpu_store_all(cfg, inp)
    for ns in (0, 1, 2, 3):
        got = _gpu_verify(cache, cfg, inp, num_splits=ns)
        assert_close(got, ref, what="num_splits=%d" % ns)


# Inputs at the edges of the binary16 operand precision: sharper softmax
# (queries times 2 and 4), outlier key channels (two coordinates 20 times
# larger, which also set every FP8 token scale), and values far from zero
# (mean 50: the value zero point, not the spread, dominates each output).
def _envelope(inp, case):
    if case == "q_x2":
        inp["Q"] = (inp["Q"] * 2).astype(inp["Q"].dtype)
    elif case == "q_x4":
        inp["Q"] = (inp["Q"] * 4).astype(inp["Q"].dtype)
    elif case == "key_outliers":
        K = inp["K"].astype(np.float32)
        K[..., [3, 77]] *= 20
        inp["K"] = K.astype(np.float16)
    elif case == "v_mean_50":
        inp["V"] = (inp["V"].astype(np.float32) + 50).astype(np.float16)
    return inp


@pytest.mark.parametrize("preset", PRESETS, ids=PNAME.get)
@pytest.mark.parametrize("case", ["q_x2", "q_x4", "key_outliers", "v_mean_50"])
@pytest.mark.parametrize("rows", [64, 32, 8], ids=lambda r: "rows%d" % r)
def test_verify_precision_envelope(preset, case, rows):
    """The envelope cases in each row path (64 rows: eight-wavefront
    work-groups, except k8v4 with eight key ranges of at most 16 tiles, which
    takes two 32-row work-groups; 32: one row tile; 8: the transposed few-row
    path), with one key range and with eight, against the oracle's
    tolerance."""
    N = {64: 8, 32: 4, 8: 1}[rows]
    cfg = _small(preset, N=N, S=1000, seed=31)
    inp = _envelope(synth.make_inputs(cfg), case)
    inp["seq_lens"] = np.array([1000, 777], np.int32)
    print("verify envelope", PNAME[preset], case, rows, flush=True)
    ocache = _oracle_cache(cfg, inp)
    ref = oracle.verify(preset, ocache, cfg["B"], cfg["Hk"], cfg["S"], inp["Q"], inp["seq_lens"],
                        cfg["Hq"], cfg["causal"])
    cache = gpu_store_all(cfg, inp)
    for ns in (1, 8):
        assert tq.tqkv_verify_num_splits(cache, N, cfg["Hq"], ns) == ns
        assert_close(_gpu_verify(cache, cfg, inp, num_splits=ns), ref, what="%s splits=%d" % (case, ns))


@pytest.mark.parametrize("preset", PRESETS, ids=PNAME.get)
@pytest.mark.parametrize("scale", [0.02, 0.15, 0.3])
def test_verify_explicit_scale(preset, scale):
    """A caller's softmax scale (instead of 1/sqrt(D) = 0.088), in both the
    64-row and the transposed few-row paths.  The binary16 operands' score
    error grows with the scale; 0.3 (3.4 x 1/sqrt(D)) is the sharpest
    softmax tested."""
    for shape in (dict(N=8, Hq=16, Hk=2), dict(N=2, Hq=4, Hk=1)):
        cfg = _small(preset, **shape)
        inp = synth.make_inputs(cfg)
        print("verify scale", PNAME[preset], scale, shape, flush=True)
        ocache = _oracle_cache(cfg, inp)
        ref = oracle.verify(preset, ocache, cfg["B"], cfg["Hk"], cfg["S"], inp["Q"], inp["seq_lens"],
                            cfg["Hq"], cfg["causal"], sm_scale=scale)
        cache = gpu_store_all(cfg, inp)
        assert_close(_gpu_verify(cache, cfg, inp, sm_scale=scale), ref, what="sm_scale=%g" % scale)


@pytest.mark.parametrize("preset", PRESETS, ids=PNAME.get)
@pytest.mark.parametrize("ns", [1, 2, 3, 9])
def test_verify_long_key_ranges(preset, ns):
    """64 rows per KV head over 2100 tokens (66 tiles): key ranges of 66, 33,
    22 and 8 tiles, which run the 64-row work-groups with eight wavefronts
    (long ranges, and every k3v4_nc range) or four (ranges of at most 32
    tiles), and for plain k8v4 at 8 tiles the 32-row work-groups."""
    cfg = _small(preset, N=8, B=1, Hq=16, Hk=2, S=2100)
    inp = synth.make_inputs(cfg)
    inp["seq_lens"] = np.array([2093], np.int32)  # a partial last tile
    print("verify long ranges", PNAME[preset], ns, flush=True)
    ocache = _oracle_cache(cfg, inp)
    ref = oracle.verify(preset, ocache, cfg["B"], cfg["Hk"], cfg["S"], inp["Q"], inp["seq_lens"], cfg["Hq"], True)
    cache = gpu_store_all(cfg, inp)
    assert tq.tqkv_verify_num_splits(cache, cfg["N"], cfg["Hq"], ns) == ns
    assert_close(_gpu_verify(cache, cfg, inp, num_splits=ns), ref, what="num_splits=%d" % ns)


@pytest.mark.parametrize("preset", PRESETS, ids=PNAME.get)
@pytest.mark.parametrize("shape", [
    dict(N=1, Hq=1, Hk=1, B=1, S=17),          # one row, partial block
    dict(N=1, Hq=32, Hk=8, B=3, S=100),        # plain decode, 4 rows per KV head
    dict(N=3, Hq=11, Hk=1, B=1, S=64),         # 33 rows: two row tiles, padding
    dict(N=16, Hq=4, Hk=1, B=1, S=300),        # 64 rows from a long window
    dict(N=2, Hq=6, Hk=6, B=2, S=48),          # MHA
    dict(N=8, Hq=8, Hk=1, B=1, S=8),           # the whole sequence is speculative
], ids=lambda s: "N%d_Hq%d_Hk%d_B%d_S%d" % (s["N"], s["Hq"], s["Hk"], s["B"], s["S"]))
def test_verify_shapes(preset, shape):
    cfg = _small(preset, **shape)
    inp = synth.make_inputs(cfg)
    print("verify shape", PNAME[preset], shape, flush=True)
    ocache = _oracle_cache(cfg, inp)
    ref = oracle.verify(preset, ocache, cfg["B"], cfg["Hk"], cfg["S"], inp["Q"], inp["seq_lens"],
                        cfg["Hq"], True)
    cache = gpu_store_all(cfg, inp)
    assert_close(_gpu_verify(cache, cfg, inp), ref, what=str(shape))


@pytest.mark.parametrize("name", ["tiny_k8v4", "poc_k8v4", "poc_k3v4_nc", "poc_k4v4_nc"])
@pytest.mark.parametrize("seed", [None] + list(synth.HELD_OUT_SEEDS))
def test_verify_config_full(name, seed):
    """Every output of the small configurations against the oracle, in the
    launch configuration the benchmark times (auto splits), at the
    configuration's seed and at the held-out seeds."""
    cfg = synth.config(name)
    if seed is not None:
        cfg["seed"] = seed
    inp = synth.make_inputs(cfg)
    print("verify", name, "seed", cfg["seed"], flush=True)
    ocache = _oracle_cache(cfg, inp)
    ref = oracle.verify(cfg["preset"], ocache, cfg["B"], cfg["Hk"], cfg["S"], inp["Q"],
                        inp["seq_lens"], cfg["Hq"], cfg["causal"])
    cache = gpu_store_all(cfg, inp)
    got = _gpu_verify(cache, cfg, inp)
    assert_close(got, ref, what=name)
    # the pages' configured split count (8) gives the same answer
    assert_close(_gpu_verify(cache, cfg, inp, num_splits=8), ref, what=name + " splits=8")


@pytest.mark.timeout(400)
@pytest.mark.parametrize("name", ["decode_k3v4_nc", "long_k3v4_nc"])
def test_verify_config_sampled(name):
    """Large configurations: full GPU run, oracle on sampled (b, hk) units."""
    cfg = synth.config(name)
    print("verify sampled", name, "generating inputs", flush=True)
    inp = _config_inputs(name)
    cache = gpu_store_all(cfg, inp)
    got = _gpu_verify(cache, cfg, inp)
    del cache
    torch.cuda.empty_cache()
    G = cfg["Hq"] // cfg["Hk"]
    # every (b, hk) unit when there are at most 16 (long context: 4), else
    # the first, the last and 14 other distinct units; all query heads of each
    n_units = cfg["B"] * cfg["Hk"]
    if n_units <= 16:
        picks = list(range(n_units))
    else:
        rng = np.random.default_rng(5)
        picks = [0, n_units - 1] + [int(u) for u in rng.choice(np.arange(1, n_units - 1), 14, replace=False)]
    assert len(set(picks)) == min(16, n_units)
    for u in picks:
        b, hk = divmod(u, cfg["Hk"])
        print("  oracle unit", b, hk, flush=True)
        ref = oracle_unit(oracle, cfg, inp, b, hk)
        assert_close(got[:, b, hk * G:(hk + 1) * G], ref, what="%s b=%d hk=%d" % (name, b, hk))


@pytest.mark.parametrize("preset", PRESETS, ids=PNAME.get)
def test_verify_nan_parity(preset):
    """A NaN key element poisons exactly the rows that can see its token."""
    cfg = _small(preset, B=1, Hk=1, Hq=2, N=8, S=64)
    inp = synth.make_inputs(cfg)
    inp["K"][0, 60, 0, 5] = np.float16(np.nan)  # position 60: row n sees 57 + n tokens
    ocache = _oracle_cache(cfg, inp)
    ref = oracle.verify(preset, ocache, 1, 1, 64, inp["Q"], inp["seq_lens"], 2, True)
    assert np.isnan(ref[4:]).all() and not np.isnan(ref[:4]).any()
    cache = gpu_store_all(cfg, inp)
    for ns in (1, 3):
        assert_close(_gpu_verify(cache, cfg, inp, num_splits=ns), ref, what="nan splits=%d" % ns)


@pytest.mark.parametrize("preset", PRESETS, ids=PNAME.get)
@pytest.mark.parametrize("Hq", [2, 8], ids=["rows16", "rows64"])
@pytest.mark.parametrize("val", [np.inf, -np.inf], ids=["inf", "neg_inf"])
def test_verify_infinite_value_parity(preset, Hq, val):
    """An infinite value element makes its token's value scale infinite (and,
    for -inf, its zero): exactly the rows that can see the token turn NaN,
    in the 32-row work-groups (16 rows) and the 64-row ones alike."""
    cfg = _small(preset, B=1, Hk=1, Hq=Hq, N=8, S=64)
    inp = synth.make_inputs(cfg)
    inp["V"][0, 60, 0, 5] = np.float16(val)  # position 60: row n sees 57 + n tokens
    ocache = _oracle_cache(cfg, inp)
    ref = oracle.verify(preset, ocache, 1, 1, 64, inp["Q"], inp["seq_lens"], Hq, True)
    assert np.isnan(ref[4:]).all() and np.isfinite(ref[:4]).all()
    cache = gpu_store_all(cfg, inp)
    for ns in (1, 3):
        assert_close(_gpu_verify(cache, cfg, inp, num_splits=ns), ref, what="infinite value splits=%d" % ns)


@pytest.mark.parametrize("preset", PRESETS, ids=PNAME.get)
def test_verify_causality_and_determinism(preset):
    cfg = _small(preset)
    inp = synth.make_inputs(cfg)
    cache = gpu_store_all(cfg, inp)
    a = _gpu_verify(cache, cfg, inp)
    b = _gpu_verify(cache, cfg, inp)
    assert np.array_equal(a, b)  # bitwise reproducible for a fixed launch
    # rewrite the last two tokens: rows n < N-2 must not change
    S, N = cfg["S"], cfg["N"]
    inp2 = dict(inp)
    inp2["K"] = inp["K"].copy()
    inp2["V"] = inp["V"].copy()
    inp2["K"][:, S - 2:] *= -3
    inp2["V"][:, S - 2:] += 5
    si, po = synth.token_lists(cfg["B"], S, S - 2, S)
    tq.tqkv_store(cache, to_dev(synth.rows(inp2["K"], S - 2, S)), to_dev(synth.rows(inp2["V"], S - 2, S)),
                  to_dev(si), to_dev(po))
    c = _gpu_verify(cache, cfg, inp)
    assert np.array_equal(a[:N - 2], c[:N - 2], equal_nan=True)
    assert not np.allclose(a[N - 2:], c[N - 2:])


def test_verify_rejects_bad_workspace():
    cfg = _small(synth.K8V4)
    inp = synth.make_inputs(cfg)
    cache = gpu_store_all(cfg, inp)
    need = tq.tqkv_verify_workspace_bytes(cache, cfg["N"], cfg["Hq"], 3)
    assert need > 0
    small = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(tq.TqkvError) as e:
        tq.tqkv_verify(cache, to_dev(inp["Q"]), to_dev(inp["seq_lens"]), cfg["N"], cfg["Hq"], True,
                       num_splits=3, workspace=small)
    assert e.value.status == -4


# ------------------------------------------------------- fused store+verify ---

def _token_lists_ragged(lens, start_from_end=None):
    """(seq_idx, pos) of positions [0, lens[b]) of every sequence, or only
    the last `start_from_end` positions of each when given."""
    si, po = [], []
    for b, L in enumerate(lens):
        lo = 0 if start_from_end is None else L - start_from_end
        si += [b] * (L - lo)
        po += list(range(lo, L))
    return np.array(si, np.int32), np.array(po, np.int32)


def _rows_at(X, si, po):
    """X[b, p] for the listed (b, p): [T, Hk, 128]."""
    return np.ascontiguousarray(X[si, po])


@pytest.mark.parametrize("preset", PRESETS, ids=PNAME.get)
@pytest.mark.parametrize("shape", [
    dict(N=8, B=2, Hq=16, Hk=2, S=203, lens=(196, 166), ns=0),   # 64 rows: two row tiles
    dict(N=8, B=2, Hq=16, Hk=2, S=203, lens=(196, 166), ns=3),   # new tokens straddle key ranges / wavefronts
    dict(N=4, B=3, Hq=8, Hk=1, S=100, lens=(100, 37, 64), ns=1),  # 32 rows, one key range
    dict(N=8, B=1, Hq=8, Hk=1, S=8, lens=(8,), ns=0),             # the whole sequence is new
    dict(N=1, B=2, Hq=4, Hk=1, S=50, lens=(50, 17), ns=2),        # plain decode
    dict(N=8, B=2, Hq=16, Hk=2, S=2100, lens=(2100, 1500), ns=1), # 66-tile key ranges (eight wavefronts)
    dict(N=8, B=2, Hq=16, Hk=2, S=2100, lens=(2100, 1500), ns=3), # 22-tile key ranges (four, except k3v4_nc)
], ids=lambda s: "N%d_Hq%d_Hk%d_S%d_ns%d" % (s["N"], s["Hq"], s["Hk"], s["S"], s["ns"]))
def test_store_verify_fused(preset, shape):
    """tqkv_store_verify writes the same cache bytes as tqkv_store and returns
    the oracle's attention over the updated cache."""
    lens, ns = shape["lens"], shape["ns"]
    cfg = _small(preset, **{k: v for k, v in shape.items() if k not in ("lens", "ns")})
    inp = synth.make_inputs(cfg)
    inp["seq_lens"] = np.array(lens, np.int32)
    N, B, Hk, S = cfg["N"], cfg["B"], cfg["Hk"], cfg["S"]
    print("store_verify", PNAME[preset], shape, flush=True)
    # oracle: every token below seq_lens stored, then verify
    si, po = _token_lists_ragged(lens)
    ref_cache = np.zeros(oracle.cache_bytes(preset, B, Hk, S), np.uint8)
    oracle.store(preset, ref_cache, B, Hk, S, _rows_at(inp["K"], si, po), _rows_at(inp["V"], si, po), si, po)
    ref = oracle.verify(preset, ref_cache, B, Hk, S, inp["Q"], inp["seq_lens"], cfg["Hq"], True)
    # GPU: the cached part with tqkv_store, the N new tokens with the fused call
    cache = tq.Cache(preset, B, Hk, S)
    si0, po0 = _token_lists_ragged([L - N for L in lens])
    if len(si0):
        tq.tqkv_store(cache, to_dev(_rows_at(inp["K"], si0, po0)), to_dev(_rows_at(inp["V"], si0, po0)),
                      to_dev(si0), to_dev(po0))
    Kn = np.stack([inp["K"][np.arange(B), np.array(lens) - N + n] for n in range(N)])  # [N, B, Hk, 128]
    Vn = np.stack([inp["V"][np.arange(B), np.array(lens) - N + n] for n in range(N)])
    out = tq.tqkv_store_verify(cache, to_dev(Kn), to_dev(Vn), to_dev(inp["Q"]), to_dev(inp["seq_lens"]),
                               N, cfg["Hq"], True, num_splits=ns)
    torch.cuda.synchronize()
    got_cache = cache.buffer.cpu().numpy()
    assert np.array_equal(got_cache, ref_cache), "%d bytes differ" % int((got_cache != ref_cache).sum())
    assert_close(out.cpu().numpy(), ref, what="fused " + str(shape))


@pytest.mark.parametrize("preset", PRESETS, ids=PNAME.get)
def test_store_verify_fused_every_binary16_value(preset):
    """The fused store (one wavefront per token-head) on the every-binary16
    rows as the new tokens of 396 sequences (64 query rows each): the same
    cache bytes as the oracle's store."""
    rows = _every_binary16_rows()
    N, Hk, Hq, S = 8, 1, 8, 16
    B = rows.shape[0] // N
    cfg = _small(preset, N=N, B=B, Hq=Hq, Hk=Hk, S=S)
    inp = synth.make_inputs(cfg)
    Kn = np.ascontiguousarray(rows[:B * N].reshape(B, N, 1, 128).transpose(1, 0, 2, 3))  # [N, B, Hk, 128]
    Vn = np.ascontiguousarray(Kn[..., ::-1])
    lens = np.full(B, S, np.int32)
    print("store_verify every binary16", PNAME[preset], B, "sequences", flush=True)
    si0, po0 = _token_lists_ragged([S - N] * B)
    si1, po1 = _token_lists_ragged([S] * B, start_from_end=N)
    ref = np.zeros(oracle.cache_bytes(preset, B, Hk, S), np.uint8)
    oracle.store(preset, ref, B, Hk, S, _rows_at(inp["K"], si0, po0), _rows_at(inp["V"], si0, po0), si0, po0)
    oracle.store(preset, ref, B, Hk, S, np.ascontiguousarray(Kn[po1 - (S - N), si1]),
                 np.ascontiguousarray(Vn[po1 - (S - N), si1]), si1, po1)
    cache = tq.Cache(preset, B, Hk, S)
    tq.tqkv_store(cache, to_dev(_rows_at(inp["K"], si0, po0)), to_dev(_rows_at(inp["V"], si0, po0)),
                  to_dev(si0), to_dev(po0))
    out = tq.tqkv_store_verify(cache, to_dev(Kn), to_dev(Vn), to_dev(inp["Q"]), to_dev(lens), N, Hq, True)
    torch.cuda.synchronize()
    assert out.shape == (N, B, Hq, 128)
    got = cache.buffer.cpu().numpy()
    assert np.array_equal(got, ref), "%d bytes differ" % int((got != ref).sum())


# ------------------------------------------------ units of at most 8 rows ---
# (plain decode and small groups run the transposed-score path)

@pytest.mark.parametrize("preset", PRESETS, ids=PNAME.get)
@pytest.mark.parametrize("shape", [
    dict(N=1, Hq=1, Hk=1, B=2, S=77, causal=True),      # 1 row
    dict(N=3, Hq=1, Hk=1, B=1, S=300, causal=True),     # 3 rows, causal window over several tiles
    dict(N=8, Hq=2, Hk=2, B=2, S=129, causal=True),     # 8 rows (MHA speculative step)
    dict(N=1, Hq=16, Hk=2, B=3, S=1000, causal=False),  # 8 rows, plain decode
    dict(N=2, Hq=12, Hk=4, B=1, S=40, causal=False),    # 6 rows, partial tail tile
], ids=lambda s: "N%d_Hq%d_Hk%d_S%d_%s" % (s["N"], s["Hq"], s["Hk"], s["S"], "c" if s["causal"] else "nc"))
@pytest.mark.parametrize("q_dtype", [np.float32, np.float16])
def test_verify_few_rows(preset, shape, q_dtype):
    cfg = _small(preset, q_dtype=q_dtype, **shape)
    inp = synth.make_inputs(cfg)
    if cfg["B"] > 1:
        inp["seq_lens"][1] = max(cfg["N"], cfg["S"] - 23)  # a second, shorter length
    print("verify few rows", PNAME[preset], shape, q_dtype.__name__, flush=True)
    ocache = _oracle_cache(cfg, inp)
    ref = oracle.verify(preset, ocache, cfg["B"], cfg["Hk"], cfg["S"], inp["Q"], inp["seq_lens"],
                        cfg["Hq"], cfg["causal"])
    cache = gpu_store_all(cfg, inp)
    for ns in (0, 1, 3):
        assert_close(_gpu_verify(cache, cfg, inp, num_splits=ns), ref, what="%s splits=%d" % (shape, ns))


@pytest.mark.parametrize("preset", PRESETS, ids=PNAME.get)
def test_verify_few_rows_nan_and_causality(preset):
    """8 rows (N=8, one query head per KV head): a NaN key poisons exactly the
    rows that see it; rewriting the last two tokens leaves rows n < N-2
    bitwise unchanged."""
    cfg = _small(preset, B=1, Hk=1, Hq=1, N=8, S=64)
    inp = synth.make_inputs(cfg)
    inp["K"][0, 60, 0, 5] = np.float16(np.nan)  # position 60: row n sees 57 + n tokens
    ocache = _oracle_cache(cfg, inp)
    ref = oracle.verify(preset, ocache, 1, 1, 64, inp["Q"], inp["seq_lens"], 1, True)
    assert np.isnan(ref[4:]).all() and not np.isnan(ref[:4]).any()
    cache = gpu_store_all(cfg, inp)
    for ns in (1, 2):
        assert_close(_gpu_verify(cache, cfg, inp, num_splits=ns), ref, what="nan splits=%d" % ns)
    a = _gpu_verify(cache, cfg, inp)
    S, N = cfg["S"], cfg["N"]
    K2 = inp["K"].copy()
    V2 = inp["V"].copy()
    K2[:, S - 2:] = 1.0
    V2[:, S - 2:] += 5
    si, po = synth.token_lists(1, S, S - 2, S)
    tq.tqkv_store(cache, to_dev(synth.rows(K2, S - 2, S)), to_dev(synth.rows(V2, S - 2, S)), to_dev(si), to_dev(po))
    c = _gpu_verify(cache, cfg, inp)
    assert np.array_equal(a[:N - 2], c[:N - 2], equal_nan=True)


@pytest.mark.timeout(400)
@pytest.mark.parametrize("name", ["poc_k8v4", "poc_k3v4_nc", "poc_k4v4_nc"])
def test_step_config_full(name):
    """The steps the benchmark times, at the PoC shape, against the oracle:
    tqkv_store_verify (the N new tokens stored in the launch) and the paged
    verify over a pool holding the same tokens in random page order."""
    from tests.gputil import gpu_paged_store_all, page_table
    cfg = synth.config(name)
    inp = synth.make_inputs(cfg)
    N, B, Hq, Hk, S = cfg["N"], cfg["B"], cfg["Hq"], cfg["Hk"], cfg["S"]
    print("step", name, flush=True)
    ocache = _oracle_cache(cfg, inp)
    ref = oracle.verify(cfg["preset"], ocache, B, Hk, S, inp["Q"], inp["seq_lens"], Hq, cfg["causal"])
    # fused step: the cached part stored first, the new tokens by the call
    cache = tq.Cache(cfg["preset"], B, Hk, S)
    si, po = synth.token_lists(B, S, 0, S - N)
    tq.tqkv_store(cache, to_dev(synth.rows(inp["K"], 0, S - N)), to_dev(synth.rows(inp["V"], 0, S - N)),
                  to_dev(si), to_dev(po))
    Kf = to_dev(np.ascontiguousarray(inp["K"][:, S - N:S].transpose(1, 0, 2, 3)))
    Vf = to_dev(np.ascontiguousarray(inp["V"][:, S - N:S].transpose(1, 0, 2, 3)))
    out = tq.tqkv_store_verify(cache, Kf, Vf, to_dev(inp["Q"]), to_dev(inp["seq_lens"]), N, Hq, cfg["causal"])
    torch.cuda.synchronize()
    got = cache.buffer.cpu().numpy()
    assert np.array_equal(got, ocache), "%d bytes differ" % int((got != ocache).sum())
    assert_close(out.cpu().numpy(), ref, what=name + " fused step")
    del cache
    # paged pool, random page order
    pc = gpu_paged_store_all(cfg, inp, page_table(B, S))
    out = tq.tqkv_paged_verify(pc, to_dev(inp["Q"]), to_dev(inp["seq_lens"]), N, Hq, cfg["causal"])
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, what=name + " paged")
