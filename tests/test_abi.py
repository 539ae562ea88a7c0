"""The C ABI library loads, exports what the header declares, and rejects bad
arguments on the host before touching a device (CPU only)."""
import ctypes
import os
import re

import pytest

from gru_corrected_draft_amd import rollout as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    inc = os.path.join(ROOT, "include")
    for f in sorted(os.listdir(inc)):
        if f.endswith(".h"):
            text = open(os.path.join(inc, f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"\b(domino_\w+)\s*\(", text)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return R.load_library()


def test_header_declares_the_binding_surface():
    assert set(_declared_functions()) == set(R.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def _cfg(**kw):
    base = dict(vocab=4096, hidden=256, emb_dim=128, gru_hidden=128, proj_dim=128, max_batch=4,
                max_k=256, dtype=R.DTYPE_FP32)
    base.update(kw)
    return R.make_config(**base)


def _create(lib, cfg, weights=None):
    if weights is None:
        weights = R.WeightPtrs(*([0x1000] * 7))
    h = ctypes.c_void_p(123)
    st = lib.domino_rollout_create(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("kw,status", [
    (dict(vocab=0), R.DOMINO_ERR_INVALID_CONFIG),
    (dict(hidden=-1), R.DOMINO_ERR_INVALID_CONFIG),
    (dict(block_size=8), R.DOMINO_ERR_INVALID_CONFIG),
    (dict(pure_draft_prefix_len=2), R.DOMINO_ERR_INVALID_CONFIG),
    (dict(max_batch=0), R.DOMINO_ERR_INVALID_CONFIG),
    (dict(max_batch=65), R.DOMINO_ERR_INVALID_CONFIG),
    (dict(max_k=-1), R.DOMINO_ERR_INVALID_CONFIG),
    (dict(dtype=7), R.DOMINO_ERR_INVALID_CONFIG),
    (dict(hidden=96), R.DOMINO_ERR_UNSUPPORTED),
    (dict(proj_dim=100), R.DOMINO_ERR_UNSUPPORTED),
])
def test_create_rejects_bad_configs(lib, kw, status):
    kwargs = dict(kw)
    cfg = _cfg(**{k: v for k, v in kwargs.items() if k not in ("block_size", "pure_draft_prefix_len")})
    if "block_size" in kwargs:
        cfg.block_size = kwargs["block_size"]
    if "pure_draft_prefix_len" in kwargs:
        cfg.pure_draft_prefix_len = kwargs["pure_draft_prefix_len"]
    st, h = _create(lib, cfg)
    assert st == status
    assert not h.value
    assert lib.domino_rollout_last_error(None).decode().startswith("create:")


def test_create_rejects_null_and_misaligned_weights(lib):
    w = R.WeightPtrs(*([0x1000] * 7))
    w.fc2_w = None
    st, h = _create(lib, _cfg(), w)
    assert st == R.DOMINO_ERR_INVALID_ARG and not h.value
    w = R.WeightPtrs(*([0x1000] * 7))
    w.lm_head = 0x1008
    st, h = _create(lib, _cfg(), w)
    assert st == R.DOMINO_ERR_INVALID_ARG
    assert "aligned" in lib.domino_rollout_last_error(None).decode()


def test_null_handle_is_rejected(lib):
    p = ctypes.c_void_p(0x1000)
    assert lib.domino_rollout_run(None, p, p, p, 1, 0, p, None, None) == R.DOMINO_ERR_INVALID_ARG
    assert lib.domino_rollout_run_graph(None, p, p, p, 1, 0, p, None, None) == R.DOMINO_ERR_INVALID_ARG
    n = ctypes.c_size_t()
    assert lib.domino_rollout_read_workspace(None, 0, None, 0, ctypes.byref(n), None) == \
        R.DOMINO_ERR_INVALID_ARG
    assert lib.domino_rollout_set_pool_strategy(None, 0) == R.DOMINO_ERR_INVALID_ARG
    assert lib.domino_rollout_set_timing(None, 1) == R.DOMINO_ERR_INVALID_ARG
    lib.domino_rollout_destroy(None)   # no-op


def test_output_tensors_checked_before_any_launch():
    """The binding refuses output buffers the library would write with the
    wrong layout or through a host address (no handle, no launch)."""
    import torch
    cpu, gpu = torch.device("cpu"), torch.device("cuda", 0)
    tok = torch.zeros((3, 15), dtype=torch.int32)
    top = torch.zeros((3, 15), dtype=torch.float32)
    R.check_outputs(tok, top, 3, 15, cpu)
    with pytest.raises(ValueError, match="on cuda"):
        R.check_outputs(tok, top, 3, 15, gpu)              # host tensors for a device run
    with pytest.raises(ValueError, match="int32"):
        R.check_outputs(tok.long(), top, 3, 15, cpu)
    with pytest.raises(ValueError, match="float32"):
        R.check_outputs(tok, top.double(), 3, 15, cpu)
    with pytest.raises(ValueError, match="contiguous"):
        R.check_outputs(torch.zeros((15, 3), dtype=torch.int32).t(), top, 3, 15, cpu)
    with pytest.raises(ValueError, match=r"\[B, P\]"):
        R.check_outputs(tok[:, :8], top, 3, 15, cpu)
    forced = torch.zeros((3, 15), dtype=torch.int32)
    R.check_forced(forced, 3, cpu)
    with pytest.raises(ValueError, match="contiguous"):
        R.check_forced(torch.zeros((15, 3), dtype=torch.int32).t(), 3, cpu)
    with pytest.raises(ValueError, match="contiguous"):
        R.check_forced(forced, 3, gpu)
    with pytest.raises(ValueError, match="int32"):
        R.check_forced(forced.long(), 3, cpu)


def test_graph_cache_query_rejects_null(lib):
    n = ctypes.c_int32(-1)
    assert lib.domino_rollout_cached_graphs(None, ctypes.byref(n)) == R.DOMINO_ERR_INVALID_ARG
