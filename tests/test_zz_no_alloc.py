"""tqkv_verify_noalloc, the verify call for callers that cannot allocate
(its workspace is the library's per-device scratch array), against
tqkv_verify with a caller workspace on the same inputs (run with -m gpu).

Two calls in a row, the second on a smaller problem, each must give exactly
tqkv_verify's output (the same kernels and key-range split run on both; only
where the partial states live differs), and the first is also held to the
oracle's tolerance (atol 5e-3, rtol 1e-2).  A shape whose partial states
need more than the array holds is refused before anything is launched.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import synth
from tests.gputil import assert_close, gpu_store_all, oracle_unit, to_dev

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("quantized_kv_attention_amd")


def _run_pair(cfg, num_splits):
    """(noalloc output, tqkv_verify output, inputs) for one configuration."""
    inp = synth.make_inputs(cfg)
    cache = gpu_store_all(cfg, inp)
    Q = to_dev(inp["Q"])
    sl = to_dev(inp["seq_lens"])
    N, Hq = cfg["N"], cfg["Hq"]
    splits = tq.tqkv_verify_num_splits(cache, N, Hq, num_splits)
    need = tq.tqkv_verify_workspace_bytes(cache, N, Hq, num_splits)
    assert splits > 1 and 0 < need <= tq.NOALLOC_SCRATCH_BYTES, (splits, need)
    out_na = torch.full(Q.shape, 7.0, dtype=torch.float32, device=Q.device)
    tq.tqkv_verify_noalloc(cache, Q, sl, N, Hq, cfg["causal"], num_splits, out=out_na)
    ref = tq.tqkv_verify(cache, Q, sl, N, Hq, cfg["causal"], num_splits)
    torch.cuda.synchronize()
    return out_na.cpu().numpy(), ref.cpu().numpy(), inp


def test_noalloc_matches_verify_two_calls():
    # call 1: 64 rows per KV head (the eight-wavefront work-groups), FP8 keys
    cfg1 = dict(preset=synth.K8V4, N=8, B=2, Hq=16, Hk=2, S=1000, causal=True, q_dtype=np.float32, seed=21)
    print("noalloc call 1", cfg1, flush=True)
    got1, ref1, inp1 = _run_pair(cfg1, 0)
    assert np.array_equal(got1.view(np.uint32), ref1.view(np.uint32)), "call 1 differs from tqkv_verify"
    for b, hk in ((0, 0), (1, 1)):
        G = cfg1["Hq"] // cfg1["Hk"]
        want = oracle_unit(oracle, cfg1, inp1, b, hk)
        assert_close(got1[:, b, hk * G:(hk + 1) * G], want, what="noalloc call 1 unit (%d, %d)" % (b, hk))
    # call 2: a smaller problem (fewer rows, keys, splits) in the same array
    cfg2 = dict(preset=synth.K3V4_NC, N=4, B=1, Hq=8, Hk=1, S=300, causal=True, q_dtype=np.float16, seed=22)
    print("noalloc call 2", cfg2, flush=True)
    got2, ref2, inp2 = _run_pair(cfg2, 3)
    assert np.array_equal(got2.view(np.uint32), ref2.view(np.uint32)), "call 2 differs from tqkv_verify"
    want = oracle_unit(oracle, cfg2, inp2, 0, 0)
    assert_close(got2[:, 0], want, what="noalloc call 2")


def test_noalloc_refuses_oversized_shape():
    # 32 * 4 (b, hk) units x 16 key ranges x 64 rows: 34.6 MB of partial states
    cache = tq.Cache(synth.K3V4_NC, 32, 4, 2048, device="cuda")
    N, Hq = 8, 32
    need = tq.tqkv_verify_workspace_bytes(cache, N, Hq, 16)
    assert need > tq.NOALLOC_SCRATCH_BYTES
    Q = torch.zeros(N, 32, Hq, 128, dtype=torch.float32, device="cuda")
    sl = torch.full((32,), 2048, dtype=torch.int32, device="cuda")
    out = torch.full(Q.shape, 3.0, dtype=torch.float32, device="cuda")
    print("noalloc oversized", need, flush=True)
    with pytest.raises(tq.TqkvError) as e:
        tq.tqkv_verify_noalloc(cache, Q, sl, N, Hq, True, 16, out=out)
    assert e.value.status == -4  # TQKV_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()), "nothing may have been written"
