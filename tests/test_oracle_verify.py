"""Pins of the oracle's verify (attention) half against torch's
scaled_dot_product_attention in float64 and against special cases whose
answer is known in closed form (CPU only)."""
import numpy as np
import pytest
import torch

import oracle
from tests import synth


def _hadamard():
    i = np.arange(128)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 1, -1.0, 1.0) / np.sqrt(128.0)


def _build(preset, B, Hk, S, K, V, max_seq=None):
    max_seq = max_seq or S
    cache = np.zeros(oracle.cache_bytes(preset, B, Hk, max_seq), np.uint8)
    si, po = synth.token_lists(B, S)
    oracle.store(preset, cache, B, Hk, max_seq, synth.rows(K), synth.rows(V), si, po)
    return cache


def _sdpa_reference(preset, cache, B, Hk, max_seq, Q, seq_lens, Hq, causal, scale=None):
    """Materialise khat/vhat with the oracle's dequant, then attend with
    torch.nn.functional.scaled_dot_product_attention in float64."""
    N = Q.shape[0]
    G = Hq // Hk
    H = _hadamard()
    out = np.zeros((N, B, Hq, 128))
    for b in range(B):
        L = int(seq_lens[b])
        for hk in range(Hk):
            kv = [oracle.dequant(preset, cache, Hk, max_seq, b, hk, t) for t in range(L)]
            Kh = torch.tensor(np.stack([k for k, _ in kv]))
            Vh = torch.tensor(np.stack([v for _, v in kv]))
            for g in range(G):
                hq = hk * G + g
                q = Q[:, b, hq].astype(np.float64)
                if preset != oracle.K8V4:
                    q = q @ H.T
                mask = torch.ones(N, L, dtype=torch.bool)
                if causal:
                    for n in range(N):
                        mask[n, L - N + n + 1:] = False
                o = torch.nn.functional.scaled_dot_product_attention(
                    torch.tensor(q)[None, None], Kh[None, None], Vh[None, None],
                    attn_mask=mask[None, None], scale=scale or 1 / np.sqrt(128.0))
                out[:, b, hq] = o[0, 0].numpy()
    return out


@pytest.mark.parametrize("preset", [oracle.K8V4, oracle.K3V4_NC, oracle.K4V4_NC])
@pytest.mark.parametrize("causal", [True, False])
def test_verify_matches_torch_sdpa_float64(preset, causal):
    rng = np.random.default_rng(31)
    N, B, Hq, Hk, S = 4, 2, 4, 2, 40
    K = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
    V = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
    Q = rng.standard_normal((N, B, Hq, 128)).astype(np.float32)
    seq_lens = np.array([40, 29], np.int32)
    cache = _build(preset, B, Hk, S, K, V)
    got = oracle.verify(preset, cache, B, Hk, S, Q, seq_lens, Hq, causal)
    ref = _sdpa_reference(preset, cache, B, Hk, S, Q, seq_lens, Hq, causal)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_fp16_query_path():
    rng = np.random.default_rng(32)
    N, B, Hq, Hk, S = 2, 1, 2, 1, 20
    K = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
    V = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
    Q = rng.standard_normal((N, B, Hq, 128)).astype(np.float16)
    cache = _build(oracle.K8V4, B, Hk, S, K, V)
    a = oracle.verify(oracle.K8V4, cache, B, Hk, S, Q, np.array([S], np.int32), Hq, True)
    b = oracle.verify(oracle.K8V4, cache, B, Hk, S, Q.astype(np.float32), np.array([S], np.int32), Hq, True)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("preset", [oracle.K8V4, oracle.K3V4_NC, oracle.K4V4_NC])
def test_zero_query_gives_mean_of_values(preset):
    """All scores equal -> uniform softmax -> mean of the dequantised values."""
    rng = np.random.default_rng(33)
    N, B, Hq, Hk, S = 3, 1, 2, 1, 24
    K = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
    V = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
    cache = _build(preset, B, Hk, S, K, V)
    Q = np.zeros((N, B, Hq, 128), np.float32)
    out = oracle.verify(preset, cache, B, Hk, S, Q, np.array([S], np.int32), Hq, True)
    vh = np.stack([oracle.dequant(preset, cache, Hk, S, 0, 0, t)[1] for t in range(S)])
    for n in range(N):
        E = S - N + n + 1
        assert np.allclose(out[n, 0, 0], vh[:E].mean(0), atol=1e-12)


def test_dominant_score_selects_one_value():
    rng = np.random.default_rng(34)
    N, B, Hq, Hk, S = 1, 1, 1, 1, 16
    K = (rng.standard_normal((B, S, Hk, 128)) * 0.01).astype(np.float16)
    K[0, 5, 0] = 1.0
    V = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
    cache = _build(oracle.K8V4, B, Hk, S, K, V)
    Q = np.full((N, B, Hq, 128), 30.0, np.float32)  # score of token 5 ~ 340, others ~ 0
    out = oracle.verify(oracle.K8V4, cache, B, Hk, S, Q, np.array([S], np.int32), Hq, False)
    v5 = oracle.dequant(oracle.K8V4, cache, Hk, S, 0, 0, 5)[1]
    assert np.allclose(out[0, 0, 0], v5, atol=1e-12)


@pytest.mark.parametrize("preset", [oracle.K8V4, oracle.K3V4_NC, oracle.K4V4_NC])
def test_causal_special_cases_and_looped_equivalence(preset):
    rng = np.random.default_rng(35)
    N, B, Hq, Hk, S = 5, 2, 4, 1, 30
    K = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
    V = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
    Q = rng.standard_normal((N, B, Hq, 128)).astype(np.float32)
    sl = np.array([30, 22], np.int32)
    cache = _build(preset, B, Hk, S, K, V)
    causal = oracle.verify(preset, cache, B, Hk, S, Q, sl, Hq, True)
    full = oracle.verify(preset, cache, B, Hk, S, Q, sl, Hq, False)
    # the last speculative row sees every token
    assert np.array_equal(causal[N - 1], full[N - 1])
    # fused causal == one single-query call per row with seq_len = cached + n + 1
    for n in range(N):
        one = oracle.verify(preset, cache, B, Hk, S, Q[n:n + 1], sl - N + n + 1, Hq, False)
        assert np.array_equal(causal[n], one[0])
    # N = 1: causal and non-causal coincide (plain decode)
    d1 = oracle.verify(preset, cache, B, Hk, S, Q[:1], sl, Hq, True)
    d2 = oracle.verify(preset, cache, B, Hk, S, Q[:1], sl, Hq, False)
    assert np.array_equal(d1, d2)


@pytest.mark.parametrize("preset", [oracle.K8V4, oracle.K3V4_NC, oracle.K4V4_NC])
def test_causality_invariance(preset):
    """Changing K/V at positions a row may not see leaves that row bit-identical."""
    rng = np.random.default_rng(36)
    N, B, Hq, Hk, S = 4, 1, 2, 1, 26
    K = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
    V = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
    Q = rng.standard_normal((N, B, Hq, 128)).astype(np.float32)
    sl = np.array([S], np.int32)
    a = oracle.verify(preset, _build(preset, B, Hk, S, K, V), B, Hk, S, Q, sl, Hq, True)
    K2, V2 = K.copy(), V.copy()
    K2[0, S - 2:] = rng.standard_normal((2, Hk, 128)) * 5
    V2[0, S - 2:] = rng.standard_normal((2, Hk, 128)) * 5
    b = oracle.verify(preset, _build(preset, B, Hk, S, K2, V2), B, Hk, S, Q, sl, Hq, True)
    # rows n with E(n) = S - N + n + 1 <= S - 2 are n = 0, 1
    assert np.array_equal(a[:2], b[:2])
    assert not np.allclose(a[2:], b[2:])


@pytest.mark.parametrize("preset", [oracle.K8V4, oracle.K3V4_NC, oracle.K4V4_NC])
def test_rows_without_visible_tokens_are_nan(preset):
    """[R17]: with fewer tokens than queries (seq_len 3, n_spec 8, causal),
    query n sees cached + n + 1 = n - 4 tokens: rows 0..4 see none and are
    NaN, rows 5..7 match float64 SDPA over the tokens they see."""
    rng = np.random.default_rng(39)
    N, B, Hq, Hk, S, L = 8, 1, 2, 1, 16, 3
    K = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
    V = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
    Q = rng.standard_normal((N, B, Hq, 128)).astype(np.float32)
    cache = _build(preset, B, Hk, S, K, V)
    sl = np.array([L], np.int32)
    got = oracle.verify(preset, cache, B, Hk, S, Q, sl, Hq, True)
    assert np.all(np.isnan(got[:5])) and np.all(np.isfinite(got[5:]))
    ref = _sdpa_reference(preset, cache, B, Hk, S, Q[5:], sl, Hq, True)
    assert np.allclose(got[5:], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("scale", [0.02, 0.3])
def test_explicit_softmax_scale(scale):
    """A caller's softmax scale replaces 1/sqrt(D) exactly as SDPA's scale does."""
    rng = np.random.default_rng(40)
    N, B, Hq, Hk, S = 4, 1, 4, 2, 40
    K = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
    V = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
    Q = rng.standard_normal((N, B, Hq, 128)).astype(np.float32)
    sl = np.array([S], np.int32)
    for preset in (oracle.K8V4, oracle.K4V4_NC):
        cache = _build(preset, B, Hk, S, K, V)
        got = oracle.verify(preset, cache, B, Hk, S, Q, sl, Hq, True, sm_scale=scale)
        ref = _sdpa_reference(preset, cache, B, Hk, S, Q, sl, Hq, True, scale=scale)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
        assert not np.allclose(got, oracle.verify(preset, cache, B, Hk, S, Q, sl, Hq, True), atol=1e-3)


def test_mha_case_hq_equals_hk():
    rng = np.random.default_rng(37)
    N, B, H, S = 2, 1, 3, 18
    K = rng.standard_normal((B, S, H, 128)).astype(np.float16)
    V = rng.standard_normal((B, S, H, 128)).astype(np.float16)
    Q = rng.standard_normal((N, B, H, 128)).astype(np.float32)
    cache = _build(oracle.K3V4_NC, B, H, S, K, V)
    got = oracle.verify(oracle.K3V4_NC, cache, B, H, S, Q, np.array([S], np.int32), H, True)
    ref = _sdpa_reference(oracle.K3V4_NC, cache, B, H, S, Q, np.array([S], np.int32), H, True)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_quantised_attention_close_to_exact_attention():
    """Attention over the quantised keys stays near fp64 attention over the raw
    fp16 keys when both use the same (dequantised) values.  The method is
    lossy; this bounds gross mistakes such as a wrong rotation, a dropped norm
    or a transposed operand, which decorrelate the scores entirely."""
    rng = np.random.default_rng(38)
    N, B, Hq, Hk, S = 4, 1, 2, 1, 64
    K = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
    V = rng.standard_normal((B, S, Hk, 128)).astype(np.float16)
    Q = rng.standard_normal((N, B, Hq, 128)).astype(np.float32)
    sl = np.array([S], np.int32)
    Kt = torch.tensor(K[0, :, 0].astype(np.float64))
    errs = {}
    for preset, tol in ((oracle.K8V4, 0.05), (oracle.K3V4_NC, 0.25), (oracle.K4V4_NC, 0.14)):
        cache = _build(preset, B, Hk, S, K, V)
        Vh = torch.tensor(np.stack([oracle.dequant(preset, cache, Hk, S, 0, 0, t)[1] for t in range(S)]))
        got = oracle.verify(preset, cache, B, Hk, S, Q, sl, Hq, False)
        for hq in range(Hq):
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.tensor(Q[:, 0, hq].astype(np.float64))[None, None], Kt[None, None],
                Vh[None, None], scale=1 / np.sqrt(128.0))[0, 0].numpy()
            err = np.linalg.norm(got[:, 0, hq] - ref) / np.linalg.norm(ref)
            errs[(preset, hq)] = err
            assert err < tol, (preset, err)
    print(errs)
