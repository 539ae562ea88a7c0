"""Shared GPU-test helpers: cached synthetic models, handles and oracle runs."""
import functools
import os
import sys

import numpy as np

from gru_corrected_draft_amd import rollout as R
from gru_corrected_draft_amd import synth
import oracle


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=4)
def model(name_or_shape, scales_key=()):
    """(synth.Weights, device weights, oracle float32 weights) for a model shape."""
    shape = synth.MODELS[name_or_shape] if isinstance(name_or_shape, str) else name_or_shape
    scales = dict(scales_key)
    log(f"[gpu-test] generating weights for {shape.name} {dict(scales)}")
    w = synth.make_weights(shape, scales)
    dev = R.device_weights(w)
    f32 = {n: w.f32(n) for n in R.WEIGHT_NAMES + R.OFFSET_WEIGHT_NAMES}
    return w, dev, f32


_handles = {}


def handle(name_or_shape, max_batch, max_k, scales_key=()):
    key = (name_or_shape, max_batch, max_k, scales_key)
    if key not in _handles:
        _, dev, _ = model(name_or_shape, scales_key)
        _handles[key] = R.DominoRollout(dev, max_batch=max_batch, max_k=max_k)
    return _handles[key]


def drop_handles():
    for h in _handles.values():
        h.close()
    _handles.clear()


@functools.lru_cache(maxsize=64)
def oracle_run(name_or_shape, batch, input_seed, trial, K, scales_key=(), forced_key=None,
               proposals=None):
    shape = synth.MODELS[name_or_shape] if isinstance(name_or_shape, str) else name_or_shape
    _, _, f32 = model(name_or_shape, scales_key)
    inp = synth.make_inputs(shape, batch, input_seed, trial)
    forced = None if forced_key is None else np.asarray(forced_key, np.int32).reshape(batch, 15)
    return oracle.rollout(f32, inp.hidden_f32(), inp.step_s, inp.verified, K, forced=forced,
                          proposals=proposals)


def gpu_run(name_or_shape, batch, input_seed, trial, K, max_batch=None, max_k=None,
            scales_key=(), graph=False, forced=None, proposals=None):
    import torch
    shape = synth.MODELS[name_or_shape] if isinstance(name_or_shape, str) else name_or_shape
    h = handle(name_or_shape, max_batch or batch, max_k if max_k is not None else max(K, 1),
               scales_key)
    inp = synth.make_inputs(shape, batch, input_seed, trial)
    hid, s, ver = R.device_inputs(inp)
    f = None if forced is None else torch.from_numpy(np.asarray(forced, np.int32)).cuda()
    tok, top = h.run(hid, s, ver, K, graph=graph, forced=f, proposals=proposals)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), top.cpu().numpy(), h


def env_trials(default):
    return int(os.environ.get("DOMINO_PARITY_TRIALS", default))
