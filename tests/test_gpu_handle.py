"""Life of one handle on the GPU: state a run leaves for the next, the graph
cache, and argument checks at the binding.

Each run's write-out clears the argmax words, bad-request flags and radix
histograms it used, so the next run on the handle starts from zeros without
a clearing launch; these tests run different batches, pool sizes and a
poisoned batch back to back on one handle and require every result to equal
a fresh handle's.
"""
import numpy as np
import pytest

from gru_corrected_draft_amd import rollout as R
from gru_corrected_draft_amd import synth
from tests import _gpu as G
from tests._parity import TOL, compare

pytestmark = pytest.mark.gpu

SMALL = synth.custom_shape(5003, 256, 128, 128, 128, "bf16", 77, name="small-bf16-ragged")
STRONG = (("embed", 16.0), ("fc1_w", 3.0), ("gru_w_hh", 3.0), ("gru_w_ih", 3.0))


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _fresh(B, seed, K):
    """Result of a brand-new handle's first run."""
    import torch
    _, dev, _ = G.model(SMALL, STRONG)
    h = R.DominoRollout(dev, max_batch=64, max_k=2048)
    try:
        hid, s, ver = R.device_inputs(synth.make_inputs(SMALL, B, seed, 0))
        t, l = h.run(hid, s, ver, K)
        torch.cuda.synchronize()
        return t.cpu().numpy(), l.cpu().numpy()
    finally:
        h.close()


def _same(a, b):
    return np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def test_runs_after_a_poisoned_batch_start_clean():
    import torch
    _, dev, _ = G.model(SMALL, STRONG)
    h = R.DominoRollout(dev, max_batch=64, max_k=2048)
    try:
        B, seed = 6, 1301
        hid, s, ver = R.device_inputs(synth.make_inputs(SMALL, B, seed, 0))
        bad = ver.clone()
        bad[1] = -7
        bad[5] = SMALL.vocab
        for K in (100, 0):
            G.log(f"[gpu-test] poisoned batch then clean, K={K}")
            t, l = h.run(hid, s, bad, K)
            torch.cuda.synchronize()
            assert torch.all(t[1] == -1) and torch.all(t[5] == -1)
            t, l = h.run(hid, s, ver, K)
            torch.cuda.synchronize()
            assert _same((t.cpu().numpy(), l.cpu().numpy()), _fresh(B, seed, K))
    finally:
        h.close()


def test_shapes_back_to_back_on_one_handle():
    """Pool B = 64, full vocabulary B = 1, pool B = 8 (another K), full
    vocabulary B = 64, pool B = 1: each equals a fresh handle's run bit for
    bit and meets the oracle."""
    import torch
    _, dev, _ = G.model(SMALL, STRONG)
    h = R.DominoRollout(dev, max_batch=64, max_k=2048)
    try:
        for B, K in ((64, 100), (1, 0), (8, 300), (64, 0), (1, 2048)):
            seed = 1400 + B
            G.log(f"[gpu-test] one handle, B={B} K={K}")
            hid, s, ver = R.device_inputs(synth.make_inputs(SMALL, B, seed, 0))
            t, l = h.run(hid, s, ver, K)
            torch.cuda.synchronize()
            got = (t.cpu().numpy(), l.cpu().numpy())
            assert _same(got, _fresh(B, seed, K)), (B, K)
            ref = G.oracle_run(SMALL, B, seed, 0, K, scales_key=STRONG)
            compare(got[0], got[1], ref, TOL["bf16"])
    finally:
        h.close()


def test_graph_cache_is_bounded():
    """100 distinct output buffers through run_graph: the cache never holds
    more than GRAPH_CACHE_MAX graphs, every replay equals the eager run, and
    a buffer set evicted earlier is captured again correctly."""
    import torch
    h = G.handle(SMALL, 64, 2048, STRONG)
    B, K = 3, 0
    hid, s, ver = R.device_inputs(synth.make_inputs(SMALL, B, 1501, 0))
    t_e, l_e = h.run(hid, s, ver, K)
    torch.cuda.synchronize()
    t_e, l_e = t_e.clone(), l_e.clone()
    outs = [(torch.full((B, 15), -9, dtype=torch.int32, device="cuda"),
             torch.zeros((B, 15), dtype=torch.float32, device="cuda")) for _ in range(100)]
    G.log("[gpu-test] graph cache: 100 output buffer sets")
    base = h.cached_graphs()
    for i, (ot, ol) in enumerate(outs + outs[:3]):
        h.run(hid, s, ver, K, out_tokens=ot, out_top1=ol, graph=True)
        assert h.cached_graphs() <= R.GRAPH_CACHE_MAX
        if i % 10 == 9:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    assert h.cached_graphs() == R.GRAPH_CACHE_MAX or base + 100 < R.GRAPH_CACHE_MAX
    for ot, ol in outs:
        assert torch.equal(ot, t_e) and torch.equal(ol.view(torch.int32), l_e.view(torch.int32))


def test_read_workspace_follows_a_replay():
    """After a graph replay the workspace holds the replayed run, even when
    an eager run of another shape came between its capture and the replay."""
    import torch
    h = G.handle(SMALL, 64, 2048, STRONG)
    hid8, s8, ver8 = R.device_inputs(synth.make_inputs(SMALL, 8, 1502, 0))
    hid1, s1, ver1 = R.device_inputs(synth.make_inputs(SMALL, 1, 1503, 0))
    ot = torch.empty((8, 15), dtype=torch.int32, device="cuda")
    ol = torch.empty((8, 15), dtype=torch.float32, device="cuda")
    G.log("[gpu-test] read_workspace after capture, eager run of another shape, replay")
    h.run(hid8, s8, ver8, 100, out_tokens=ot, out_top1=ol, graph=True)
    torch.cuda.synchronize()
    pool8 = h.read_workspace(1).clone()
    h.run(hid1, s1, ver1, 0)
    torch.cuda.synchronize()
    with pytest.raises(R.DominoError):
        h.read_workspace(1)                       # the last run had no pool
    h.run(hid8, s8, ver8, 100, out_tokens=ot, out_top1=ol, graph=True)
    torch.cuda.synchronize()
    assert h.read_workspace(0).numel() == 15 * 8 * SMALL.vocab
    assert torch.equal(h.read_workspace(1), pool8)


def test_host_output_buffer_rejected():
    import torch
    h = G.handle(SMALL, 64, 2048, STRONG)
    hid, s, ver = R.device_inputs(synth.make_inputs(SMALL, 2, 1504, 0))
    with pytest.raises(ValueError):
        h.run(hid, s, ver, 0, out_tokens=torch.zeros((2, 15), dtype=torch.int32))
    with pytest.raises(ValueError):
        h.run(hid, s, ver, 0, out_tokens=torch.zeros((2, 15), dtype=torch.int64, device="cuda"))
    with pytest.raises(ValueError):
        h.run(hid, s, ver, 0, forced=torch.zeros((15, 2), dtype=torch.int32, device="cuda").t())
