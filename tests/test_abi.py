"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/tqkv.h declares, sizes follow the documented
layout, and invalid arguments are rejected before any device work."""
import ctypes
import os
import re

import pytest

import quantized_kv_attention_amd as tq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "tqkv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tqkv_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 8
    L = ctypes.CDLL(tq.library_path)
    for n in names:
        assert hasattr(L, n), n


def test_binding_names_match_header():
    for n in _declared():
        assert hasattr(tq, n), n


def test_enum_values_match_header():
    """The binding's preset, query-type and status constants are the values
    include/tqkv.h gives them."""
    src = open(os.path.join(ROOT, "include", "tqkv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    vals = {k: int(v) for k, v in re.findall(r"\b(TQKV_[A-Z0-9_]+)\s*=\s*(-?\d+)", src)}
    assert vals["TQKV_K8V4"] == tq.K8V4 and vals["TQKV_K3V4_NC"] == tq.K3V4_NC and vals["TQKV_K4V4_NC"] == tq.K4V4_NC
    assert vals["TQKV_Q_F32"] == tq.Q_F32 and vals["TQKV_Q_F16"] == tq.Q_F16
    assert vals["TQKV_OK"] == 0 and all(v < 0 for k, v in vals.items() if k.startswith("TQKV_ERR_"))
    defines = dict(re.findall(r"#define\s+(TQKV_\w+)\s+(\d+)", src))
    assert int(defines["TQKV_HEAD_DIM"]) == tq.HEAD_DIM and int(defines["TQKV_BLOCK_TOKENS"]) == tq.BLOCK_TOKENS
    assert int(defines["TQKV_MAX_QLEN"]) == tq.MAX_QLEN


def test_sizes():
    assert tq.tqkv_slot_bytes(tq.K3V4_NC) == 120
    assert tq.tqkv_slot_bytes(tq.K4V4_NC) == 136
    assert tq.tqkv_slot_bytes(tq.K8V4) == 198
    assert tq.tqkv_slot_bytes(7) == 0
    assert tq.tqkv_slot_bytes(0) == 0
    assert tq.tqkv_block_bytes(tq.K3V4_NC) == 1920
    assert tq.tqkv_block_bytes(tq.K4V4_NC) == 2176
    assert tq.tqkv_block_bytes(tq.K8V4) == 3168
    # PoC shape: B=4, Hk=4, 8192 tokens
    assert tq.tqkv_cache_bytes(tq.K3V4_NC, 4, 4, 128, 8192) == 4 * 4 * 8192 * 120
    assert tq.tqkv_cache_bytes(tq.K8V4, 4, 4, 128, 8192) == 4 * 4 * 8192 * 198
    assert tq.tqkv_cache_bytes(tq.K8V4, 1, 1, 128, 17) == 2 * 3168  # partial block rounds up
    assert tq.tqkv_cache_bytes(tq.K8V4, 1, 1, 64, 16) == 0
    assert tq.tqkv_cache_bytes(tq.K8V4, 0, 1, 128, 16) == 0
    assert tq.tqkv_version() >= 100


def test_codebook_tables_match_oracle():
    """The library's constant codebook tables (written by its own generator)
    are, bit for bit, the oracle's binary32 levels and thresholds."""
    import numpy as np

    import oracle
    src = open(os.path.join(ROOT, "quantized_kv_attention_amd", "csrc", "codebook.h")).read()

    def table(name):
        body = re.search(r"\b%s\[\d+\] = \{([^}]*)\}" % name, src).group(1)
        return np.array([float.fromhex(x.strip().rstrip("f")) for x in body.split(",")], np.float32)

    for levels, cn, tn in ((8, "kCentroid", "kThreshold"), (16, "kCentroid16", "kThreshold16")):
        c, t = oracle.codebook(levels)
        assert table(cn).view(np.uint32).tolist() == c.view(np.uint32).tolist(), levels
        assert table(tn).view(np.uint32).tolist() == t.view(np.uint32).tolist(), levels


def _desc(**kw):
    d = dict(preset=tq.K8V4, B=1, Hk=1, D=128, max_seq=16, base=4096)
    d.update(kw)
    return tq._CacheDesc(d["preset"], d["B"], d["Hk"], d["D"], d["max_seq"], d["base"])


def test_status_strings():
    for s in range(-6, 1):
        assert tq.tqkv_status_string(s) != "unknown status"
    assert tq.tqkv_status_string(-99) == "unknown status"


@pytest.mark.parametrize("kw,status", [
    (dict(preset=4), -1), (dict(preset=0), -1), (dict(B=0), -1), (dict(base=0), -1), (dict(D=64), -2),
    (dict(base=4100), -3),
])
def test_store_rejects_bad_cache(kw, status):
    L = tq.lib()
    d = _desc(**kw)
    assert L.tqkv_store(ctypes.byref(d), 4096, 4096, 4096, 4096, 1, None) == status


def test_store_rejects_bad_arguments():
    L = tq.lib()
    d = _desc()
    assert L.tqkv_store(None, 4096, 4096, 4096, 4096, 1, None) == -1
    assert L.tqkv_store(ctypes.byref(d), 4096, 4096, 4096, 4096, -1, None) == -1
    assert L.tqkv_store(ctypes.byref(d), None, 4096, 4096, 4096, 1, None) == -1
    assert L.tqkv_store(ctypes.byref(d), 4097, 4096, 4096, 4096, 1, None) == -3
    assert L.tqkv_store(ctypes.byref(d), 4096, 4096, 4098, 4096, 1, None) == -3
    assert L.tqkv_store(ctypes.byref(d), None, None, None, None, 0, None) == 0  # T == 0: no-op


def test_verify_rejects_bad_arguments():
    L = tq.lib()
    d = _desc(Hk=2)
    ok = dict(Q=4096, qd=0, sl=4096, n=8, Hq=16, causal=1, ns=0, sc=0.0, out=4096)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.tqkv_verify(ctypes.byref(d), a["Q"], a["qd"], a["sl"], a["n"], a["Hq"], a["causal"],
                             a["ns"], a["sc"], a["out"], None, 0, None)

    assert call(Q=None) == -1
    assert call(sl=None) == -1
    assert call(out=None) == -1
    assert call(qd=2) == -1
    assert call(causal=2) == -1
    assert call(n=0) == -1
    assert call(ns=-1) == -1
    assert call(sc=-1.0) == -1
    assert call(sc=float("inf")) == -1
    assert call(sc=float("nan")) == -1
    assert call(Hq=15) == -2            # Hq % Hk != 0
    assert call(n=129) == -2            # more than 128 queries per sequence
    assert call(Q=4104) == -3           # Q must be 16-byte aligned
    assert call(out=4100) == -3
    n = ctypes.c_size_t(7)
    assert L.tqkv_verify_workspace_bytes(ctypes.byref(d), 8, 15, 0, ctypes.byref(n)) == -2
    assert n.value == 0
    assert L.tqkv_verify_workspace_bytes(ctypes.byref(d), 8, 16, 0, None) == -1
    assert L.tqkv_verify_num_splits(ctypes.byref(d), 0, 16, 0) == 0


def test_store_verify_rejects_bad_arguments():
    L = tq.lib()
    d = _desc(Hk=2)

    def call(K=4096, V=4096, Q=4096, n=8):
        return L.tqkv_store_verify(ctypes.byref(d), K, V, Q, 0, 4096, n, 16, 1, 0, 0.0, 4096, None, 0, None)

    assert call(K=None) == -1
    assert call(V=None) == -1
    assert call(K=4097) == -3           # K must be 2-byte aligned
    assert call(Q=None) == -1
    assert call(n=129) == -2


def test_row_limit():
    L = tq.lib()
    d = _desc(Hk=1)
    # 128 query heads per KV head x 65 queries = 8320 rows > 8192
    assert L.tqkv_verify(ctypes.byref(d), 4096, 0, 4096, 65, 128, 1, 0, 0.0, 4096, None, 0, None) == -2
    n = ctypes.c_size_t(0)
    assert L.tqkv_verify_workspace_bytes(ctypes.byref(d), 65, 128, 0, ctypes.byref(n)) == -2


def _pdesc(**kw):
    d = dict(preset=tq.K8V4, Hk=2, D=128, num_pages=64, base=4096, bt=8192, B=2, max_pages=8)
    d.update(kw)
    return tq._PagedDesc(d["preset"], d["Hk"], d["D"], d["num_pages"], d["base"], d["bt"], d["B"],
                         d["max_pages"])


def test_paged_sizes():
    assert tq.tqkv_paged_cache_bytes(tq.K3V4_NC, 4, 128, 2048) == 2048 * 4 * 1920
    assert tq.tqkv_paged_cache_bytes(tq.K8V4, 4, 128, 2048) == 2048 * 4 * 3168
    assert tq.tqkv_paged_cache_bytes(tq.K8V4, 4, 64, 2048) == 0
    assert tq.tqkv_paged_cache_bytes(tq.K8V4, 0, 128, 2048) == 0
    assert tq.tqkv_paged_cache_bytes(tq.K8V4, 1, 128, 0) == 0
    assert tq.tqkv_paged_cache_bytes(9, 1, 128, 1) == 0


def test_paged_store_rejects_bad_arguments():
    L = tq.lib()

    def call(d, K=4096, V=4096, sm=4096, T=1):
        return L.tqkv_paged_store(ctypes.byref(d) if d is not None else None, K, V, sm, T, None)

    assert call(None) == -1
    assert call(_pdesc(preset=5)) == -1
    assert call(_pdesc(num_pages=0)) == -1
    assert call(_pdesc(base=0)) == -1
    assert call(_pdesc(D=96)) == -2
    assert call(_pdesc(base=4104)) == -3
    assert call(_pdesc(), sm=None) == -1
    assert call(_pdesc(), T=-1) == -1
    assert call(_pdesc(), sm=4098) == -3
    assert call(_pdesc(), K=4097) == -3
    # the store needs no block table
    assert call(_pdesc(bt=None, B=0, max_pages=0), K=None, V=None, sm=None, T=0) == 0


def test_paged_verify_rejects_bad_arguments():
    L = tq.lib()

    def verify(d, n=8, Hq=16):
        return L.tqkv_paged_verify(ctypes.byref(d), 4096, 0, 4096, n, Hq, 1, 0, 0.0, 4096, None, 0, None)

    assert verify(_pdesc(bt=None)) == -1
    assert verify(_pdesc(B=0)) == -1
    assert verify(_pdesc(max_pages=0)) == -1
    assert verify(_pdesc(max_pages=524289)) == -2
    assert verify(_pdesc(bt=8194)) == -3
    assert verify(_pdesc(), Hq=15) == -2
    assert verify(_pdesc(), n=129) == -2
    n = ctypes.c_size_t(3)
    assert L.tqkv_paged_verify_workspace_bytes(ctypes.byref(_pdesc(bt=None)), 8, 16, 0, ctypes.byref(n)) == -1
    assert n.value == 0
    assert L.tqkv_paged_verify_num_splits(ctypes.byref(_pdesc(bt=None)), 8, 16, 0) == 0
    d = _pdesc()
    assert L.tqkv_paged_store_verify(ctypes.byref(d), None, 4096, 4096, 0, 4096, 8, 16, 1, 0, 0.0, 4096,
                                     None, 0, None) == -1
    assert L.tqkv_paged_verify_varlen(ctypes.byref(d), 4096, 0, None, 8, 4096, 16, 1, 0, 0.0, 4096,
                                      None, 0, None) == -1


def test_varlen_rejects_bad_arguments():
    L = tq.lib()
    d = _desc(Hk=2)

    def call(cu=4096, mq=8, Q=4096):
        return L.tqkv_verify_varlen(ctypes.byref(d), Q, 0, cu, mq, 4096, 16, 1, 0, 0.0, 4096, None, 0, None)

    assert call(cu=None) == -1
    assert call(mq=0) == -1
    assert call(mq=129) == -2
    assert call(cu=4098) == -3
    assert call(Q=4100) == -3


def test_noalloc_scratch_size_matches_header():
    src = open(os.path.join(ROOT, "include", "tqkv.h")).read()
    m = re.search(r"#define\s+TQKV_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == tq.NOALLOC_SCRATCH_BYTES


def test_binding_rejects_buffers_off_the_cache_device():
    """Every tensor a verify call hands to the kernels must live on the
    cache's device; the binding refuses others before calling the library
    (a CPU cache and meta tensors stand in for two devices here)."""
    import torch
    cache = tq.Cache(tq.K8V4, 1, 1, 64, device="cpu")
    N, Hq = 8, 8
    Q = torch.zeros(N, 1, Hq, 128)
    sl = torch.full((1,), 64, dtype=torch.int32)
    out = torch.zeros(N, 1, Hq, 128)
    meta = dict(device="meta")
    cases = [
        dict(Q=torch.zeros(N, 1, Hq, 128, **meta)),
        dict(seq_lens=torch.zeros(1, dtype=torch.int32, **meta)),
        dict(out=torch.zeros(N, 1, Hq, 128, **meta)),
        dict(workspace=torch.zeros(64, dtype=torch.uint8, **meta)),
    ]
    for c in cases:
        args = dict(Q=Q, seq_lens=sl, out=out, workspace=None)
        args.update(c)
        name = next(iter(c))
        with pytest.raises(ValueError, match="%s must be on the cache's device" % name):
            tq.tqkv_verify(cache, args["Q"], args["seq_lens"], N, Hq, True, out=args["out"],
                           workspace=args["workspace"])
    cu = torch.tensor([0, N], dtype=torch.int32, device="meta")
    with pytest.raises(ValueError, match="must be on"):
        tq.tqkv_verify_varlen(cache, Q.reshape(N, Hq, 128), cu, N, sl, Hq, True)
    for ws in (torch.zeros(16, dtype=torch.float32), torch.zeros(64, dtype=torch.uint8)[::2]):
        with pytest.raises(ValueError, match="workspace must be a contiguous uint8"):
            tq.tqkv_verify(cache, Q, sl, N, Hq, True, out=out, workspace=ws)
    with pytest.raises(ValueError, match="needs a caller-provided out"):
        tq.tqkv_verify_noalloc(cache, Q, sl, N, Hq, True)
    with pytest.raises(ValueError, match="out must be on"):
        tq.tqkv_verify_noalloc(cache, Q, sl, N, Hq, True, out=torch.zeros(N, 1, Hq, 128, **meta))
