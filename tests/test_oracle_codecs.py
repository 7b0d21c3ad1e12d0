"""Pins of the oracle's scalar codecs, Lloyd-Max codebook, WHT and reduction
against library routines, textbook values and closed forms (CPU only)."""
import os

import numpy as np
import pytest
import torch
from scipy import stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- binary16 ---

def test_half_to_float_exhaustive_matches_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.half_to_float(int(b)) for b in bits], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_float_to_half_matches_numpy_rne():
    rng = np.random.default_rng(7)
    xs = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(5000) * 1e-5).astype(np.float32),   # binary16 subnormals
        (rng.standard_normal(5000) * 7e4).astype(np.float32),    # overflow region
        # exact ties: midpoints between adjacent binary16 values
        ((np.arange(1, 2000, dtype=np.float32) + np.float32(0.5)) * np.float32(2.0 ** -10)),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, np.inf, -np.inf], np.float32),
    ])
    with np.errstate(over="ignore"):
        ref = xs.astype(np.float16).view(np.uint16)
    got = np.array([oracle.float_to_half(float(x)) for x in xs], np.uint16)
    assert np.array_equal(got, ref)
    assert oracle.float_to_half(float("nan")) == 0x7E00


# ------------------------------------------------------------- FP8 E4M3 ---

def test_e4m3_decode_exhaustive_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = np.array([oracle.e4m3_decode(c) for c in range(256)], np.float32)
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6 and got[0x7E] == 448.0


def test_e4m3_encode_matches_torch_rne_below_overflow():
    rng = np.random.default_rng(11)
    xs = np.concatenate([
        (rng.standard_normal(20000) * 100).astype(np.float32),
        (rng.standard_normal(5000) * 0.01).astype(np.float32),
        rng.uniform(-463.9, 463.9, 5000).astype(np.float32),
    ])
    # every midpoint between adjacent finite codes is a tie: RNE picks the even code
    finite = np.array([oracle.e4m3_decode(c) for c in range(0x7F)], np.float64)
    mids = ((finite[:-1] + finite[1:]) / 2).astype(np.float32)
    xs = np.concatenate([xs, mids, -mids])
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(x)) for x in xs], np.uint8)
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates_and_nan():
    assert oracle.e4m3_encode(448.0) == 0x7E
    assert oracle.e4m3_encode(463.9) == 0x7E
    assert oracle.e4m3_encode(464.0) == 0x7E   # saturating (torch would give NaN)
    assert oracle.e4m3_encode(1e9) == 0x7E
    assert oracle.e4m3_encode(-float("inf")) == 0xFE
    assert oracle.e4m3_encode(float("nan")) == 0x7F
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00  # tie between 0 and 2^-9 -> even (0)
    assert oracle.e4m3_encode(3 * 2.0 ** -10) == 0x02  # tie between 1 and 2 -> even (2)
    # round trip of every finite code
    for c in list(range(0x7F)) + list(range(0x80, 0xFF)):
        assert oracle.e4m3_encode(oracle.e4m3_decode(c)) == (c if c != 0x80 else 0x80)


# ----------------------------------------------------------- Lloyd-Max ---

def _golden_max(levels=8):
    vals = {}
    with open(os.path.join(GOLDEN, "lloyd_max_gaussian_%dlevel.txt" % levels)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, *v = line.split()
            vals[k] = [float(x) for x in v]
    return vals


@pytest.mark.parametrize("levels", [8, 16])
def test_lloyd_max_matches_max_1960_table(levels):
    g = _golden_max(levels)
    u, t = oracle.lloyd_max_unit(levels=levels)
    hl = levels // 2
    assert np.allclose(u[hl:], g["levels"], atol=6e-4)
    assert np.allclose(-u[:hl][::-1], g["levels"], atol=6e-4)
    assert np.allclose(t[hl - 1:], g["thresholds"], atol=6e-4)
    # distortion E[(Z - Q(Z))^2], closed form per cell
    edges = np.concatenate([[-np.inf], t, [np.inf]])
    mse = 0.0
    for j in range(levels):
        a, b = edges[j], edges[j + 1]
        P = stats.norm.cdf(b) - stats.norm.cdf(a)
        pa = 0.0 if np.isinf(a) else stats.norm.pdf(a)
        pb = 0.0 if np.isinf(b) else stats.norm.pdf(b)
        aa = 0.0 if np.isinf(a) else a * pa
        bb = 0.0 if np.isinf(b) else b * pb
        ez2 = P + aa - bb
        ez = pa - pb
        mse += ez2 - 2 * u[j] * ez + u[j] ** 2 * P
    assert abs(mse - g["mse"][0]) < 2e-5


@pytest.mark.parametrize("levels", [8, 16])
def test_lloyd_max_optimality_conditions(levels):
    u, t = oracle.lloyd_max_unit(levels=levels)
    edges = np.concatenate([[-np.inf], t, [np.inf]])
    for j in range(levels):
        m = stats.truncnorm.mean(edges[j], edges[j + 1])
        assert abs(m - u[j]) < 1e-12
    assert np.allclose(t, (u[:-1] + u[1:]) / 2, atol=0, rtol=0)
    assert np.allclose(u, -u[::-1], atol=1e-14)


@pytest.mark.parametrize("levels", [8, 16])
def test_codebook_float32_tables(levels):
    c, th = oracle.codebook(levels)
    u, t = oracle.lloyd_max_unit(levels=levels)
    assert c.dtype == np.float32 and th.dtype == np.float32
    assert np.all(np.diff(c) > 0) and np.all(np.diff(th) > 0)
    # each table entry is the binary32 value nearest to the scaled level
    s = np.sqrt(128.0)
    for x32, x64 in list(zip(c, u / s)) + list(zip(th, t / s)):
        nb = np.nextafter(x32, np.float32(np.inf)), np.nextafter(x32, np.float32(-np.inf))
        assert abs(float(x32) - x64) <= min(abs(float(v) - x64) for v in nb)
    # centroids interleave the thresholds
    assert np.all(c[:-1] < th) and np.all(th < c[1:])


# ------------------------------------------------------------------- WHT ---

def _hadamard(n=128):
    i = np.arange(n)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 1, -1.0, 1.0)


def test_wht_equals_closed_form():
    H = _hadamard()
    rng = np.random.default_rng(3)
    for _ in range(20):
        x = rng.standard_normal(128).astype(np.float32)
        ref = H @ x.astype(np.float64)
        got = oracle.wht128(x)
        assert np.allclose(got, ref, rtol=0, atol=2e-5 * np.abs(x).sum())


def test_wht_exact_on_pm1_and_self_inverse():
    rng = np.random.default_rng(4)
    x = rng.choice([-1.0, 1.0], 128).astype(np.float32)
    y = oracle.wht128(x)
    assert np.array_equal(y, (_hadamard() @ x).astype(np.float32))  # integers: exact
    assert np.array_equal(oracle.wht128(y) / 128, x)                 # H H = 128 I
    z = rng.standard_normal(128).astype(np.float32)
    back = oracle.wht128(oracle.wht128(z)) / np.float32(128)
    assert np.allclose(back, z, atol=1e-6)
    # orthogonality of the normalised transform: norm preserved
    assert abs(np.linalg.norm(oracle.wht128(z) / np.sqrt(128)) - np.linalg.norm(z)) < 1e-5


def test_tree_sumsq_within_error_bound():
    rng = np.random.default_rng(5)
    for _ in range(50):
        x = (rng.standard_normal(128) * rng.uniform(0.01, 100)).astype(np.float32)
        exact = float(np.sum(x.astype(np.float64) ** 2))
        got = oracle.tree_sumsq(x)
        # pairwise summation of 128 terms: |err| <= (log2(128) + 1) * u * sum
        assert abs(got - exact) <= 8 * 2.0 ** -24 * exact
