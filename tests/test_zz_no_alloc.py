"""The allocation-free entry point (domino_rollout_run_static) against the
ordinary run on the same handle: identical tokens and logits bit for bit,
on consecutive calls that share the library's static scratch array (the
second with a smaller batch), after a poisoned batch, at the 8B shapes, for
the fp32 model, and a batch too large for the array rejected without a
launch."""
import numpy as np
import pytest

from gru_corrected_draft_amd import rollout as R
from gru_corrected_draft_amd import synth
from tests import _gpu as G
from tests._parity import TOL, compare

pytestmark = pytest.mark.gpu

SMALL = synth.custom_shape(5003, 256, 128, 128, 128, "bf16", 77, name="small-bf16-ragged")
STRONG = (("embed", 16.0), ("fc1_w", 3.0), ("gru_w_hh", 3.0), ("gru_w_ih", 3.0))
WIDE5 = synth.custom_shape(1031, 256, 1280, 1280, 256, "bf16", 81, name="small-bf16-gru1280")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _both(h, shape, B, seed, K, verified=None):
    import torch
    hid, s, ver = R.device_inputs(synth.make_inputs(shape, B, seed, 0))
    if verified is not None:
        ver = verified
    ts, ls = h.run(hid, s, ver, K, static=True)
    torch.cuda.synchronize()
    ts, ls = ts.cpu().numpy(), ls.cpu().numpy()
    tr, lr = h.run(hid, s, ver, K)
    torch.cuda.synchronize()
    tr, lr = tr.cpu().numpy(), lr.cpu().numpy()
    assert np.array_equal(ts, tr), (B, K)
    assert np.array_equal(ls.view(np.uint32), lr.view(np.uint32)), (B, K)
    return ts, ls


def test_static_runs_equal_ordinary_runs():
    h = G.handle(SMALL, 64, 2048, STRONG)
    for B, K in ((8, 100), (3, 0), (64, 2048), (1, 300), (17, 0)):
        seed = 1700 + B
        G.log(f"[gpu-test] static scratch B={B} K={K}")
        ts, ls = _both(h, SMALL, B, seed, K)
        ref = G.oracle_run(SMALL, B, seed, 0, K, scales_key=STRONG)
        compare(ts, ls, ref, TOL["bf16"])


def test_static_run_after_a_poisoned_static_run():
    import torch
    h = G.handle(SMALL, 64, 2048, STRONG)
    B, seed = 6, 1801
    hid, s, ver = R.device_inputs(synth.make_inputs(SMALL, B, seed, 0))
    bad = ver.clone()
    bad[2] = -1
    G.log("[gpu-test] static scratch, poisoned then clean")
    t, _ = h.run(hid, s, bad, 100, static=True)
    torch.cuda.synchronize()
    assert torch.all(t[2] == -1)
    _both(h, SMALL, B, seed, 100)


def test_static_run_fp32_model():
    h = G.handle("tiny", 4, 256)
    G.log("[gpu-test] static scratch, fp32 model")
    for K in (0, 256):
        _both(h, synth.MODELS["tiny"], 1, 4096, K)


def test_static_run_full_size_8b():
    h = G.handle("qwen3-8b", 64, 2048)
    shape = synth.MODELS["qwen3-8b"]
    for B, K in ((8, 2048), (1, 0)):
        G.log(f"[gpu-test] static scratch, 8B B={B} K={K}")
        _both(h, shape, B, synth.WORKLOADS[f"8b_b{B}"].input_seed, K)


def test_static_run_rejects_a_batch_beyond_the_array():
    import torch
    h = G.handle(WIDE5, 64, 2048, STRONG)
    B = 64   # about 5.4 MB of scratch at g = 1280
    hid, s, ver = R.device_inputs(synth.make_inputs(WIDE5, B, 1802, 0))
    out = torch.full((B, 15), 7, dtype=torch.int32, device="cuda")
    G.log("[gpu-test] static scratch, batch beyond the array")
    with pytest.raises(R.DominoError) as ei:
        h.run(hid, s, ver, 0, out_tokens=out, static=True)
    assert ei.value.status == R.DOMINO_ERR_INVALID_ARG
    assert "static array" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.all(out == 7)
    _both(h, WIDE5, 40, 1803, 0)   # 40 requests fit
