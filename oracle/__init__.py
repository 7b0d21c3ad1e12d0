"""CPU oracle for TurboQuant speculative-decode verification attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  It shares no code with the HIP library (``quantized_kv_attention_amd``)
and must never be called on the product path.

The arithmetic lives in ``tq_oracle.c`` (plain C, binary32 store / binary64
verify, see that file's header for the method and its sources).  This module
only builds it with gcc and marshals numpy arrays through ctypes.

Parity status of each function is stated in ``PINS`` below: every function is
checked by the ``-m "not gpu"`` tests against closed forms, textbook values,
library routines or brute force, except the storage-layout choices, which no
page fixes ("parity unpinned": only self-consistency can be tested).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tq_oracle.c")
_LIB = os.path.join(_HERE, "libtqoracle.so")

K8V4 = 1
K3V4_NC = 2
K4V4_NC = 3
D = 128
BLOCK = 16

PINS = {
    "half_to_float/float_to_half": "numpy float16 casts (library routine), exhaustive / random",
    "e4m3_decode/e4m3_encode": "torch.float8_e4m3fn casts (library routine), exhaustive / random + tie cases",
    "codebook": "Max (1960) 8- and 16-level Gaussian tables; Lloyd optimality conditions and MSE via "
                "scipy.stats.norm / scipy.integrate",
    "wht128": "closed form H_ij=(-1)^popcount(i&j); orthogonality; self-inverse",
    "tree_sumsq": "binary64 sum of squares within the binary32 error bound",
    "quant_key_k3 / quant_key_k4": "norm correction |khat| = n; distortion vs Gaussian-model MSE; nearest "
                                   "level; n_h = binary16 of the float64 norm; zero vector",
    "lloyd_code": "ties on a threshold go to the upper cell, one ulp below to the lower; NaN -> 0",
    "dequant": "Lloyd-Max keys: norm n and cosine to H k from the distortion model; FP8 keys within "
               "2^-4; values within half a step",
    "quant_key_k8": "e4m3 relative error bound 2^-4; saturation never triggered",
    "quant_val": "|v - vhat| <= scale/2; endpoints hit codes 0 and 15; constant vector exact",
    "record layout": "parity unpinned (a layout choice): round trip pack/unpack and worked bytes only",
    "verify": "torch SDPA in float64 on materialised K/V; brute-force special cases; causality; rows "
              "that see no token are NaN",
    "store_paged / gather_pages": "a paged store gathered through its block table equals the contiguous "
                                  "store byte for byte (layout: parity unpinned, as above)",
    "verify_varlen": "equal query counts reduce to verify; each sequence equals a one-sequence verify "
                     "with its own count; SDPA on materialised K/V with the per-row causal window",
}


def build(force: bool = True) -> str:
    """Compile tq_oracle.c into libtqoracle.so with gcc (OpenMP, no fast-math)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-fopenmp", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32 = ctypes.c_int
        L.tqo_half_to_float.argtypes = [ctypes.c_uint16]
        L.tqo_half_to_float.restype = ctypes.c_float
        L.tqo_float_to_half.argtypes = [ctypes.c_float]
        L.tqo_float_to_half.restype = ctypes.c_uint16
        L.tqo_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.tqo_e4m3_decode.restype = ctypes.c_float
        L.tqo_e4m3_encode.argtypes = [ctypes.c_float]
        L.tqo_e4m3_encode.restype = ctypes.c_uint8
        L.tqo_lloyd_max_unit.argtypes = [P, P, i32]
        L.tqo_lloyd_max_unit_n.argtypes = [i32, P, P, i32]
        L.tqo_codebook.argtypes = [P, P]
        L.tqo_codebook_n.argtypes = [i32, P, P]
        L.tqo_wht128_f32.argtypes = [P]
        L.tqo_tree_sumsq_f32.argtypes = [P]
        L.tqo_tree_sumsq_f32.restype = ctypes.c_float
        L.tqo_quant_key_k3.argtypes = [P, P, P, P, P, P]
        L.tqo_quant_key_lm.argtypes = [i32, P, P, P, P, P, P]
        L.tqo_lloyd_code.argtypes = [i32, P, ctypes.c_float]
        L.tqo_lloyd_code.restype = i32
        L.tqo_quant_key_k8.argtypes = [P, P, P]
        L.tqo_quant_val.argtypes = [P, P, P, P]
        L.tqo_block_bytes.argtypes = [i32]
        L.tqo_block_bytes.restype = ctypes.c_size_t
        L.tqo_slot_bytes.argtypes = [i32]
        L.tqo_slot_bytes.restype = ctypes.c_size_t
        L.tqo_write_record.argtypes = [i32, P, i32, P, P, ctypes.c_uint16, ctypes.c_uint16,
                                       ctypes.c_uint16, ctypes.c_uint16]
        L.tqo_read_record.argtypes = [i32, P, i32, P, P, P, P, P, P]
        L.tqo_store.argtypes = [i32, i32, i32, i32, P, P, P, P, P, i32]
        L.tqo_store.restype = i32
        L.tqo_store_paged.argtypes = [i32, i32, i32, P, P, P, P, i32]
        L.tqo_store_paged.restype = i32
        L.tqo_dequant.argtypes = [i32, i32, i32, P, i32, i32, i32, P, P, P]
        L.tqo_verify.argtypes = [i32, i32, i32, i32, P, P, i32, P, i32, i32, i32,
                                 ctypes.c_double, P]
        L.tqo_verify.restype = i32
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# ----------------------------------------------------------------------------
# scalar codecs
# ----------------------------------------------------------------------------

def half_to_float(bits: int) -> float:
    return lib().tqo_half_to_float(int(bits))


def float_to_half(x: float) -> int:
    return int(lib().tqo_float_to_half(float(x)))


def e4m3_decode(code: int) -> float:
    return lib().tqo_e4m3_decode(int(code))


def e4m3_encode(x: float) -> int:
    return int(lib().tqo_e4m3_encode(float(x)))


# ----------------------------------------------------------------------------
# codebook, rotation, reduction
# ----------------------------------------------------------------------------

def lloyd_max_unit(iters: int = 2000, levels: int = 8):
    """Unit-Gaussian Lloyd-Max levels[levels] and thresholds[levels - 1] (float64)."""
    u = np.zeros(levels, np.float64)
    t = np.zeros(levels - 1, np.float64)
    lib().tqo_lloyd_max_unit_n(levels, _p(u), _p(t), iters)
    return u, t


def codebook(levels: int = 8):
    """(centroids[levels], thresholds[levels - 1]) as float32 for N(0, 1/128);
    levels 8 (k3v4_nc keys) or 16 (k4v4_nc keys)."""
    assert levels in (8, 16)
    c = np.zeros(levels, np.float32)
    t = np.zeros(levels - 1, np.float32)
    lib().tqo_codebook_n(levels, _p(c), _p(t))
    return c, t


def lloyd_code(levels: int, y: float) -> int:
    """The cell of a rotated coordinate y against the levels-level thresholds."""
    _, t = codebook(levels)
    return int(lib().tqo_lloyd_code(levels, _p(t), float(y)))


def key_levels(preset: int) -> int:
    """Codebook levels of a Lloyd-Max key preset (0 for FP8 keys)."""
    return {K3V4_NC: 8, K4V4_NC: 16}.get(preset, 0)


def wht128(x: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(x, dtype=np.float32).copy()
    assert a.shape == (D,)
    lib().tqo_wht128_f32(_p(a))
    return a


def tree_sumsq(x: np.ndarray) -> float:
    a = np.ascontiguousarray(x, dtype=np.float32)
    return float(lib().tqo_tree_sumsq_f32(_p(a)))


# ----------------------------------------------------------------------------
# per-vector quantisers (inputs: float16 arrays of 128)
# ----------------------------------------------------------------------------

def quant_key_k3(k: np.ndarray):
    kh = np.ascontiguousarray(k, dtype=np.float16).view(np.uint16)
    c, t = codebook()
    codes = np.zeros(D, np.uint8)
    n = np.zeros(1, np.uint16)
    g = np.zeros(1, np.uint16)
    lib().tqo_quant_key_k3(_p(kh), _p(c), _p(t), _p(codes), _p(n), _p(g))
    return codes, int(n[0]), int(g[0])


def quant_key_k4(k: np.ndarray):
    """k4v4_nc keys: codes 0..15 against the 16-level codebook, n_h, gamma_h."""
    kh = np.ascontiguousarray(k, dtype=np.float16).view(np.uint16)
    c, t = codebook(16)
    codes = np.zeros(D, np.uint8)
    n = np.zeros(1, np.uint16)
    g = np.zeros(1, np.uint16)
    lib().tqo_quant_key_lm(16, _p(kh), _p(c), _p(t), _p(codes), _p(n), _p(g))
    return codes, int(n[0]), int(g[0])


def quant_key_k8(k: np.ndarray):
    kh = np.ascontiguousarray(k, dtype=np.float16).view(np.uint16)
    codes = np.zeros(D, np.uint8)
    s = np.zeros(1, np.uint16)
    lib().tqo_quant_key_k8(_p(kh), _p(codes), _p(s))
    return codes, int(s[0])


def quant_val(v: np.ndarray):
    vh = np.ascontiguousarray(v, dtype=np.float16).view(np.uint16)
    codes = np.zeros(D, np.uint8)
    s = np.zeros(1, np.uint16)
    z = np.zeros(1, np.uint16)
    lib().tqo_quant_val(_p(vh), _p(codes), _p(s), _p(z))
    return codes, int(s[0]), int(z[0])


# ----------------------------------------------------------------------------
# layout
# ----------------------------------------------------------------------------

def block_bytes(preset: int) -> int:
    return int(lib().tqo_block_bytes(preset))


def slot_bytes(preset: int) -> int:
    return int(lib().tqo_slot_bytes(preset))


def cache_bytes(preset: int, B: int, Hk: int, max_seq: int) -> int:
    nblk = (max_seq + BLOCK - 1) // BLOCK
    return B * Hk * nblk * block_bytes(preset)


def write_record(preset, block: np.ndarray, tb, kcode, vcode, kmeta0, kmeta1, vscale, vzero):
    kc = np.ascontiguousarray(kcode, np.uint8)
    vc = np.ascontiguousarray(vcode, np.uint8)
    lib().tqo_write_record(preset, _p(block), tb, _p(kc), _p(vc), kmeta0, kmeta1, vscale, vzero)


def read_record(preset, block: np.ndarray, tb):
    kc = np.zeros(D, np.uint8)
    vc = np.zeros(D, np.uint8)
    m = np.zeros(4, np.uint16)
    mv = m.ctypes.data
    lib().tqo_read_record(preset, _p(block), tb, _p(kc), _p(vc), mv, mv + 2, mv + 4, mv + 6)
    return kc, vc, int(m[0]), int(m[1]), int(m[2]), int(m[3])


# ----------------------------------------------------------------------------
# store / dequant / verify
# ----------------------------------------------------------------------------

def store(preset: int, cache: np.ndarray, B: int, Hk: int, max_seq: int,
          K: np.ndarray, V: np.ndarray, seq_idx: np.ndarray, pos: np.ndarray) -> None:
    """Quantise K, V (float16 [T, Hk, 128]) into ``cache`` (uint8, in place)."""
    assert cache.dtype == np.uint8 and cache.size == cache_bytes(preset, B, Hk, max_seq)
    Kh = np.ascontiguousarray(K, np.float16).view(np.uint16)
    Vh = np.ascontiguousarray(V, np.float16).view(np.uint16)
    T = Kh.shape[0]
    assert Kh.shape == (T, Hk, D) and Vh.shape == (T, Hk, D)
    si = np.ascontiguousarray(seq_idx, np.int32)
    po = np.ascontiguousarray(pos, np.int32)
    rc = lib().tqo_store(preset, B, Hk, max_seq, _p(cache), _p(Kh), _p(Vh), _p(si), _p(po), T)
    if rc != 0:
        raise ValueError("oracle store: index out of range")


def dequant(preset: int, cache: np.ndarray, Hk: int, max_seq: int, b: int, hk: int, t: int):
    """(khat[128], vhat[128]) float64; Lloyd-Max keys are in the rotated space."""
    c, _ = codebook(key_levels(preset) or 8)
    kh = np.zeros(D, np.float64)
    vh = np.zeros(D, np.float64)
    lib().tqo_dequant(preset, Hk, max_seq, _p(cache), b, hk, t, _p(c), _p(kh), _p(vh))
    return kh, vh


def verify(preset: int, cache: np.ndarray, B: int, Hk: int, max_seq: int, Q: np.ndarray,
           seq_lens: np.ndarray, Hq: int, causal: bool, sm_scale: float = 0.0) -> np.ndarray:
    """float64 [N, B, Hq, 128] attention output; Q is float32 or float16."""
    if Q.dtype == np.float32:
        qd, Qc = 0, np.ascontiguousarray(Q)
    elif Q.dtype == np.float16:
        qd, Qc = 1, np.ascontiguousarray(Q).view(np.uint16)
    else:
        raise TypeError("Q must be float32 or float16")
    N = Q.shape[0]
    assert Q.shape == (N, B, Hq, D)
    sl = np.ascontiguousarray(seq_lens, np.int32)
    out = np.zeros((N, B, Hq, D), np.float64)
    rc = lib().tqo_verify(preset, B, Hk, max_seq, _p(cache), _p(Qc), qd, _p(sl), N, Hq,
                          int(bool(causal)), float(sm_scale), _p(out))
    if rc != 0:
        raise ValueError("oracle verify: bad arguments")
    return out


# ----------------------------------------------------------------------------
# paged pool and ragged queries
# ----------------------------------------------------------------------------

def paged_cache_bytes(preset: int, Hk: int, num_pages: int) -> int:
    """A pool of num_pages pages, each the 16-token blocks of all Hk heads."""
    return num_pages * Hk * block_bytes(preset)


def store_paged(preset: int, pool: np.ndarray, Hk: int, num_pages: int, K: np.ndarray, V: np.ndarray,
                slots: np.ndarray) -> None:
    """Quantise K, V (float16 [T, Hk, 128]) into the paged ``pool`` (uint8, in
    place) at slots[t] = page * 16 + position; negative slots are skipped."""
    assert pool.dtype == np.uint8 and pool.size == paged_cache_bytes(preset, Hk, num_pages)
    Kh = np.ascontiguousarray(K, np.float16).view(np.uint16)
    Vh = np.ascontiguousarray(V, np.float16).view(np.uint16)
    T = Kh.shape[0]
    assert Kh.shape == (T, Hk, D) and Vh.shape == (T, Hk, D)
    sl = np.ascontiguousarray(slots, np.int32)
    assert sl.shape == (T,)
    rc = lib().tqo_store_paged(preset, Hk, num_pages, _p(pool), _p(Kh), _p(Vh), _p(sl), T)
    if rc != 0:
        raise ValueError("oracle paged store: page out of range")


def gather_pages(preset: int, pool: np.ndarray, Hk: int, num_pages: int, block_table: np.ndarray) -> np.ndarray:
    """The contiguous cache (B sequences, max_seq = 16 * max_pages) whose block
    j of (b, hk) is head hk's block of page block_table[b, j]; entries outside
    the pool give zero blocks.  Pure byte movement: no arithmetic."""
    bb = block_bytes(preset)
    B, P = block_table.shape
    blocks = pool.reshape(num_pages, Hk, bb)
    out = np.zeros((B, Hk, P, bb), np.uint8)
    for b in range(B):
        for j in range(P):
            pg = int(block_table[b, j])
            if 0 <= pg < num_pages:
                out[b, :, j, :] = blocks[pg]
    return out.reshape(-1)


def verify_varlen(preset: int, cache: np.ndarray, B: int, Hk: int, max_seq: int, Q: np.ndarray,
                  cu_q: np.ndarray, seq_lens: np.ndarray, Hq: int, causal: bool,
                  sm_scale: float = 0.0) -> np.ndarray:
    """float64 [rows, Hq, 128]: sequence b's q_b = cu_q[b+1] - cu_q[b] queries
    (rows cu_q[b].. of Q [rows, Hq, 128]) are its last q_b tokens, attended
    exactly as ``verify`` attends a step of q_b queries of that sequence alone
    ("Speculative decoding on Intel Arc", Part 6: each continuation chunk of
    up to 128 queries is a decode over its own cached length)."""
    rows = Q.shape[0]
    assert Q.shape == (rows, Hq, D) and cu_q.shape == (B + 1,)
    out = np.full((rows, Hq, D), np.nan, np.float64)
    per_seq = cache_bytes(preset, 1, Hk, max_seq)
    for b in range(B):
        c0, c1 = int(cu_q[b]), int(cu_q[b + 1])
        if c1 <= c0:
            continue
        cb = cache[b * per_seq:(b + 1) * per_seq]
        out[c0:c1] = verify(preset, cb, 1, Hk, max_seq, Q[c0:c1][:, None], np.asarray(seq_lens[b:b + 1]),
                            Hq, causal, sm_scale)[:, 0]
    return out
