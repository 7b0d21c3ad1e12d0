"""Pins of the oracle's per-vector quantisers and record layout (CPU only)."""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
H128 = None


def _hadamard():
    global H128
    if H128 is None:
        i = np.arange(128)
        pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
        H128 = np.where(pc % 2 == 1, -1.0, 1.0) / np.sqrt(128.0)
    return H128


def h2f(bits):
    return float(np.array([bits], np.uint16).view(np.float16)[0])


# ------------------------------------------- Lloyd-Max keys (k3 and k4) ---

# (quantiser, codebook levels, Gaussian-model distortion of Max's table)
LM_KEYS = {"k3v4_nc": (oracle.quant_key_k3, 8, 0.03454), "k4v4_nc": (oracle.quant_key_k4, 16, 0.009497)}


@pytest.mark.parametrize("preset", list(LM_KEYS))
def test_lm_codes_are_nearest_centroid(preset):
    """Lloyd-Max coding of the rotated unit vector = nearest centroid, except
    within rounding distance of a threshold."""
    quant, levels, _ = LM_KEYS[preset]
    c, th = oracle.codebook(levels)
    rng = np.random.default_rng(21)
    H = _hadamard()
    for _ in range(200):
        k = rng.standard_normal(128).astype(np.float16)
        codes, nh, gh = quant(k)
        x = k.astype(np.float64)
        y = H @ x / np.linalg.norm(x)
        nearest = np.argmin(np.abs(y[:, None] - c.astype(np.float64)[None, :]), axis=1)
        close = np.min(np.abs(y[:, None] - th.astype(np.float64)[None, :]), axis=1) < 1e-6
        assert np.all((codes == nearest) | close)
        assert abs(h2f(nh) - np.linalg.norm(x)) <= 2.0 ** -11 * np.linalg.norm(x)


@pytest.mark.parametrize("preset", list(LM_KEYS))
def test_lm_norm_correction_restores_norm(preset):
    quant, levels, _ = LM_KEYS[preset]
    c, _ = oracle.codebook(levels)
    rng = np.random.default_rng(22)
    for _ in range(200):
        k = (rng.standard_normal(128) * rng.uniform(0.1, 10)).astype(np.float16)
        codes, nh, gh = quant(k)
        khat = c[codes].astype(np.float64) * h2f(nh) * h2f(gh)
        n = np.linalg.norm(k.astype(np.float64))
        # n and gamma are each rounded to binary16 (2^-11 relative each)
        assert abs(np.linalg.norm(khat) - n) <= 2.5 * 2.0 ** -11 * n


@pytest.mark.parametrize("preset", list(LM_KEYS))
def test_lm_distortion_near_gaussian_model(preset):
    """Mean squared error of the unit-vector reconstruction (before norm
    correction) is close to the Gaussian-model Lloyd-Max MSE of Max's table
    (0.03454 at 8 levels, 0.009497 at 16): within 6 %, the coordinates of a
    rotated unit vector being only nearly Gaussian."""
    quant, levels, mse = LM_KEYS[preset]
    c, _ = oracle.codebook(levels)
    rng = np.random.default_rng(23)
    H = _hadamard()
    errs = []
    for _ in range(3000):
        k = rng.standard_normal(128).astype(np.float16)
        codes, _, _ = quant(k)
        x = k.astype(np.float64)
        y = H @ x / np.linalg.norm(x)
        errs.append(np.sum((y - c[codes]) ** 2))
    assert abs(np.mean(errs) - mse) < 0.06 * mse


@pytest.mark.parametrize("preset", list(LM_KEYS))
def test_lm_zero_vector(preset):
    quant, levels, _ = LM_KEYS[preset]
    codes, nh, gh = quant(np.zeros(128, np.float16))
    assert np.all(codes == 0) and nh == 0
    c, _ = oracle.codebook(levels)
    assert h2f(gh) == pytest.approx(1 / np.sqrt(128 * c[0].astype(np.float64) ** 2), rel=1e-3)


def test_k4_refines_k3():
    """Sixteen levels reconstruct every key at least about as well as eight
    and about 3.6x better on average (Max's 0.03454 / 0.009497)."""
    c3, _ = oracle.codebook(8)
    c4, _ = oracle.codebook(16)
    rng = np.random.default_rng(24)
    H = _hadamard()
    e3, e4 = [], []
    for _ in range(500):
        k = rng.standard_normal(128).astype(np.float16)
        x = k.astype(np.float64)
        y = H @ x / np.linalg.norm(x)
        e3.append(np.sum((y - c3[oracle.quant_key_k3(k)[0]]) ** 2))
        e4.append(np.sum((y - c4[oracle.quant_key_k4(k)[0]]) ** 2))
    assert np.all(np.array(e4) < np.array(e3))
    assert 3.2 < np.mean(e3) / np.mean(e4) < 4.0


# --------------------------------------------------------------- k8 keys ---

def test_k8_relative_error_and_scale():
    rng = np.random.default_rng(24)
    for _ in range(200):
        k = (rng.standard_normal(128) * rng.uniform(0.01, 50)).astype(np.float16)
        codes, sh = oracle.quant_key_k8(k)
        s = h2f(sh)
        amax = np.max(np.abs(k.astype(np.float64)))
        assert abs(s - amax / 448) <= 2.0 ** -11 * amax / 448
        dec = np.array([oracle.e4m3_decode(int(cc)) for cc in codes], np.float64)
        assert not np.any(np.isnan(dec))
        kh = dec * s
        x = k.astype(np.float64)
        normal = np.abs(x / s) >= 2.0 ** -6
        # relative half-ulp of a 3-bit mantissa, plus the binary32 division
        assert np.all(np.abs(kh - x)[normal] <= (2.0 ** -4 + 1e-6) * np.abs(x)[normal])
        assert np.all(np.abs(kh - x)[~normal] <= 2.0 ** -10 * s * 1.0001)
        assert np.max(np.abs(dec)) <= 448


def test_k8_codes_are_torch_e4m3fn_of_x_over_rounded_scale():
    """Each k8 key code is the OCP E4M3 ("e4m3fn") encoding, round to nearest
    even, of x / s_h evaluated in binary32, where s_h is the binary16 scale
    (Part 6 of the speculative-decoding page keeps FP8 keys with one scale
    per token).  torch's float8_e4m3fn conversion is the independent
    reference; every |x / s_h| stays below 464, where it needs no
    saturation.  The rounding of the scale to binary16 matters: with the
    unrounded binary32 scale some codes come out different."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(81)
    flips = 0
    for _ in range(300):
        k = (rng.standard_normal(128) * rng.uniform(0.01, 50)).astype(np.float16)
        codes, sh = oracle.quant_key_k8(k)
        s = np.float32(h2f(sh))
        x = k.astype(np.float32) / s
        assert np.all(np.abs(x) < 464)
        ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(codes, ref), np.flatnonzero(codes != ref)[:5]
        s32 = np.float32(np.max(np.abs(k.astype(np.float32)))) / np.float32(448)
        alt = torch.from_numpy(k.astype(np.float32) / s32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        flips += int(not np.array_equal(alt, codes))
    assert flips > 0


def test_k8_zero_vector():
    codes, sh = oracle.quant_key_k8(np.zeros(128, np.float16))
    assert sh == 0 and np.all(codes == 0)


# ---------------------------------------------------------------- values ---

def test_values_error_bound_and_endpoints():
    rng = np.random.default_rng(25)
    for _ in range(300):
        v = (rng.standard_normal(128) * rng.uniform(0.01, 30) + rng.uniform(-5, 5)).astype(np.float16)
        codes, sh, zh = oracle.quant_val(v)
        s, z = h2f(sh), h2f(zh)
        x = v.astype(np.float64)
        assert z == x.min()
        vhat = codes * s + z
        assert np.all(np.abs(vhat - x) <= s / 2 * (1 + 1e-6) + 1e-7 * np.abs(x).max())
        assert codes[np.argmin(x)] == 0 and codes[np.argmax(x)] == 15
        assert codes.max() <= 15


@pytest.mark.parametrize("levels", [8, 16])
def test_lloyd_code_ties_go_up(levels):
    """[R5]: a coordinate exactly on a threshold is coded into the upper cell,
    one ulp below it into the lower one; NaN gives cell 0; the cells of the
    levels themselves are their own indices."""
    c, t = oracle.codebook(levels)
    for j, tj in enumerate(t):
        assert oracle.lloyd_code(levels, tj) == j + 1
        assert oracle.lloyd_code(levels, np.nextafter(tj, np.float32(-np.inf))) == j
    assert oracle.lloyd_code(levels, float("nan")) == 0
    assert [oracle.lloyd_code(levels, x) for x in c] == list(range(levels))


@pytest.mark.parametrize("preset", list(LM_KEYS))
def test_lm_norm_is_the_rounded_norm(preset):
    """n_h is the binary16 rounding of the key's norm: the binary32 tree sum
    only moves it across a rounding boundary when the norm lies within about
    2^-23 (relative) of one, so (almost) every key matches the float64 norm
    rounded to binary16."""
    quant, _, _ = LM_KEYS[preset]
    rng = np.random.default_rng(25)
    same = 0
    for _ in range(400):
        k = (rng.standard_normal(128) * rng.uniform(0.1, 10)).astype(np.float16)
        _, nh, _ = quant(k)
        same += nh == int(np.float16(np.linalg.norm(k.astype(np.float64))).view(np.uint16))
    assert same >= 398


def test_values_zero_point_is_positive_zero():
    """[R9]: a minimum of -0 is stored as the zero point +0."""
    v = np.linspace(0, 3, 128).astype(np.float16)
    v[0] = np.float16(-0.0)  # the first (and only) minimum
    _, _, zh = oracle.quant_val(v)
    assert zh == 0x0000


def test_values_constant_vector_exact():
    v = np.full(128, 1.5, np.float16)
    codes, sh, zh = oracle.quant_val(v)
    assert sh == 0 and np.all(codes == 0) and h2f(zh) == 1.5


# ---------------------------------------------------------------- layout ---

def _read_k3_examples():
    out = []
    with open(os.path.join(GOLDEN, "k3_pack_worked_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, nz, exp = line.split()
            codes = np.zeros(128, np.uint8)
            for item in nz.split(","):
                d, cc = item.split(":")
                codes[int(d)] = int(cc)
            expected = np.zeros(48, np.uint8)
            for item in exp.split(","):
                i, hx = item.split(":")
                expected[int(i)] = int(hx, 16)
            out.append((name, codes, expected))
    return out


def _read_k4_examples():
    out = []
    with open(os.path.join(GOLDEN, "k4_pack_worked_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, cs, exp = line.split()
            codes = np.zeros(128, np.uint8)
            for item in cs.split(","):
                d, cc = item.split(":")
                if d == "*":
                    codes[:] = int(cc)
                else:
                    codes[int(d)] = int(cc)
            expected = np.zeros(64, np.uint8)
            items = exp.split(",")
            for item in items:
                i, hx = item.split(":")
                if i == "*":
                    expected[:] = int(hx, 16)
            for item in items:
                i, hx = item.split(":")
                if i != "*":
                    expected[int(i)] = int(hx, 16)
            out.append((name, codes, expected))
    return out


@pytest.mark.parametrize("example", _read_k4_examples(), ids=lambda e: e[0])
def test_k4_pack_worked_examples(example):
    _, codes, expected = example
    block = np.zeros(oracle.block_bytes(oracle.K4V4_NC), np.uint8)
    oracle.write_record(oracle.K4V4_NC, block, 0, codes, np.zeros(128, np.uint8), 0, 0, 0, 0)
    assert np.array_equal(block[:64], expected)
    assert not np.any(block[64:])


@pytest.mark.parametrize("example", _read_k3_examples(), ids=lambda e: e[0])
def test_k3_pack_worked_examples(example):
    _, codes, expected = example
    block = np.zeros(oracle.block_bytes(oracle.K3V4_NC), np.uint8)
    oracle.write_record(oracle.K3V4_NC, block, 0, codes, np.zeros(128, np.uint8), 0, 0, 0, 0)
    assert np.array_equal(block[:48], expected)


def test_value_nibble_worked_examples():
    rows = []
    with open(os.path.join(GOLDEN, "value_nibble_worked_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(x, 16) if i == 5 else int(x) for i, x in enumerate(line.split())])
    for preset, voff in ((oracle.K3V4_NC, 768), (oracle.K4V4_NC, 1024), (oracle.K8V4, 2048)):
        for tb, p, lo, hi, off, byte in rows:
            block = np.zeros(oracle.block_bytes(preset), np.uint8)
            vc = np.zeros(128, np.uint8)
            vc[2 * p], vc[2 * p + 1] = lo, hi
            # key codes whose packed bytes are all zero (k4: code 8 is the nibble 0)
            kc = np.full(128, 8 if preset == oracle.K4V4_NC else 0, np.uint8)
            oracle.write_record(preset, block, tb, kc, vc, 0, 0, 0, 0)
            nz = np.nonzero(block)[0]
            assert list(nz) == ([voff + off] if byte else [])
            assert block[voff + off] == byte


KEY_CODES = {oracle.K8V4: 256, oracle.K3V4_NC: 8, oracle.K4V4_NC: 16}


@pytest.mark.parametrize("preset", [oracle.K8V4, oracle.K3V4_NC, oracle.K4V4_NC])
def test_record_round_trip_and_slot_size(preset):
    # 128 codes of 8, 3 or 4 bits + 64 B of value nibbles + 3 or 4 binary16 fields
    assert oracle.slot_bytes(preset) == {oracle.K8V4: 198, oracle.K3V4_NC: 120, oracle.K4V4_NC: 136}[preset]
    assert oracle.block_bytes(preset) == 16 * oracle.slot_bytes(preset)
    rng = np.random.default_rng(26)
    block = np.zeros(oracle.block_bytes(preset), np.uint8)
    recs = []
    for tb in rng.permutation(16):
        kc = rng.integers(0, KEY_CODES[preset], 128).astype(np.uint8)
        vc = rng.integers(0, 16, 128).astype(np.uint8)
        m = [int(x) for x in rng.integers(0, 65536, 4)]
        if preset == oracle.K8V4:
            m[1] = 0
        oracle.write_record(preset, block, int(tb), kc, vc, *m)
        recs.append((int(tb), kc, vc, m))
    for tb, kc, vc, m in recs:
        kc2, vc2, *m2 = oracle.read_record(preset, block, tb)
        assert np.array_equal(kc2, kc) and np.array_equal(vc2, vc) and m2 == m
    # every byte of the block belongs to exactly one token's record
    seen = np.zeros(block.size, np.int32)
    for tb in range(16):
        b2 = np.zeros_like(block)
        # (k4: code 0 is the nibble 15, every key bit set)
        full = {oracle.K8V4: 255, oracle.K3V4_NC: 7, oracle.K4V4_NC: 0}[preset]
        oracle.write_record(preset, b2, tb, np.full(128, full, np.uint8),
                            np.full(128, 15, np.uint8), 0xFFFF, 0 if preset == oracle.K8V4 else 0xFFFF,
                            0xFFFF, 0xFFFF)
        seen += (b2 != 0)
    assert np.all(seen == 1)


@pytest.mark.parametrize("preset", [oracle.K8V4, oracle.K3V4_NC, oracle.K4V4_NC])
def test_dequant_reconstructs_the_token(preset):
    """What the oracle's verify attends to, read back from a stored cache:
    Lloyd-Max keys come back in the rotated space with the key's norm (the
    norm correction) and close to H k; FP8 keys within the E4M3 relative
    error; values within half a quantisation step."""
    from tests import synth
    rng = np.random.default_rng(28)
    B, Hk, S = 1, 2, 24
    K = (rng.standard_normal((B, S, Hk, 128)) * rng.uniform(0.2, 5, (B, S, Hk, 1))).astype(np.float16)
    V = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
    cache = np.zeros(oracle.cache_bytes(preset, B, Hk, S), np.uint8)
    si, po = synth.token_lists(B, S)
    oracle.store(preset, cache, B, Hk, S, synth.rows(K), synth.rows(V), si, po)
    H = _hadamard()
    for t in range(S):
        for hk in range(Hk):
            k = K[0, t, hk].astype(np.float64)
            v = V[0, t, hk].astype(np.float64)
            khat, vhat = oracle.dequant(preset, cache, Hk, S, 0, hk, t)
            if preset == oracle.K8V4:
                assert np.all(np.abs(khat - k) <= 2.0 ** -4 * np.abs(k) + 2.0 ** -9 * np.abs(k).max() / 448)
            else:
                n = np.linalg.norm(k)
                assert abs(np.linalg.norm(khat) - n) <= 3 * 2.0 ** -11 * n
                cos = khat @ (H @ k) / (np.linalg.norm(khat) * n)
                # the Gaussian-model distortion (0.0345 / 0.0095) puts the mean
                # cosine near 0.983 / 0.995; a wrong or missing rotation gives ~0
                assert cos > (0.95 if preset == oracle.K3V4_NC else 0.98), cos
            _, vs, vz = oracle.quant_val(V[0, t, hk])
            assert np.all(np.abs(vhat - v) <= h2f(vs) / 2 + 2.0 ** -10 * np.abs(v).max())


def test_store_writes_the_quantised_record():
    from tests import synth
    rng = np.random.default_rng(27)
    for preset in (oracle.K8V4, oracle.K3V4_NC, oracle.K4V4_NC):
        B, Hk, S = 2, 2, 40
        cache = np.zeros(oracle.cache_bytes(preset, B, Hk, S), np.uint8)
        K = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
        V = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
        si, po = synth.token_lists(B, S)
        oracle.store(preset, cache, B, Hk, S, synth.rows(K), synth.rows(V), si, po)
        nblk = (S + 15) // 16
        bb = oracle.block_bytes(preset)
        for (b, s, hk) in [(0, 0, 0), (1, 39, 1), (0, 17, 1), (1, 16, 0)]:
            blk = cache[((b * Hk + hk) * nblk + s // 16) * bb:][:bb]
            kc, vc, m0, m1, vs, vz = oracle.read_record(preset, blk, s % 16)
            if preset != oracle.K8V4:
                quant = oracle.quant_key_k3 if preset == oracle.K3V4_NC else oracle.quant_key_k4
                c2, n2, g2 = quant(K[b, s, hk])
                assert (m0, m1) == (n2, g2)
            else:
                c2, s2 = oracle.quant_key_k8(K[b, s, hk])
                assert m0 == s2
            v2, vs2, vz2 = oracle.quant_val(V[b, s, hk])
            assert np.array_equal(kc, c2) and np.array_equal(vc, v2) and (vs, vz) == (vs2, vz2)
        # untouched tail of the last block stays zero
        with pytest.raises(ValueError):
            oracle.store(preset, cache, B, Hk, S, synth.rows(K)[:1], synth.rows(V)[:1],
                         np.array([2], np.int32), np.array([0], np.int32))
