"""Seeded synthetic weights and inputs for the Domino draft-block rollout.

This module only draws random numbers and rounds them to the storage
precision.  It performs none of the rollout's arithmetic, so both the HIP
path and the CPU oracle can consume what it produces without sharing any
method code.

Recipe (every array is reproducible from its seeds alone):

* Each weight tensor has its own stream id.  A tensor of n elements is cut
  into blocks of ``BLOCK`` elements; block j is filled with
  ``numpy.random.Generator(PCG64(SeedSequence([weight_seed, stream, j])))
  .standard_normal(float32)`` and multiplied by ``scale / sqrt(fan_in)``
  (fan_in = the tensor's second dimension, the PyTorch convention; the 1-D
  biases fc2_b and fc1_b use the projector width).  fc1_x_w [r, H] and fc1_b
  are the backbone-hidden half of the projector's first layer and its bias,
  used when the per-step offsets s are computed from the hiddens.  The block
  split makes the stream independent of how many threads fill it.
* bf16 tensors are the float32 draw rounded to bfloat16 with
  round-to-nearest-even, stored as uint16 bit patterns.
* Per-trial inputs use ``SeedSequence([input_seed, 1 + trial, stream])``:
  draft hiddens X ~ N(0,1) (rounded to bf16 for bf16 models), the per-step
  projector offsets s ~ N(0,1) in float32, and verified tokens uniform over
  [0, V).

The shapes follow the Qwen3-8B-class draft (vocab 151936, hidden 4096,
GRU / embedding / projector width 1024) the rollout was benchmarked with,
a 27B-class variant (hidden 5120, widths 1280) and a tiny fp32 model whose
oracle runs in milliseconds.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK = 1 << 22
BLOCK_SIZE = 16          # draft block: 1 verified position + 15 proposals
N_PROPOSALS = BLOCK_SIZE - 1
N_STEPS = BLOCK_SIZE - 2  # correction steps after the first proposal

# stream ids of the weight tensors
_STREAMS = {"lm_head": 1, "embed": 2, "gru_w_ih": 3, "gru_w_hh": 4,
            "fc1_w": 5, "fc2_w": 6, "fc2_b": 7, "fc1_x_w": 8, "fc1_b": 9}
_INPUT_STREAMS = {"hidden": 1, "step_s": 2, "verified": 3}


@dataclass(frozen=True)
class ModelShape:
    name: str
    vocab: int
    hidden: int
    emb_dim: int
    gru_hidden: int
    proj_dim: int
    dtype: str          # "bf16" or "fp32": storage type of weights and hiddens
    weight_seed: int

    def tensor_shapes(self):
        V, H, e, g, r = self.vocab, self.hidden, self.emb_dim, self.gru_hidden, self.proj_dim
        return {"lm_head": (V, H), "embed": (V, e), "gru_w_ih": (3 * g, e),
                "gru_w_hh": (3 * g, g), "fc1_w": (r, g), "fc2_w": (V, r), "fc2_b": (V,),
                "fc1_x_w": (r, H), "fc1_b": (r,)}

    def fan_in(self, name):
        shp = self.tensor_shapes()[name]
        return self.proj_dim if len(shp) == 1 else shp[1]


MODELS = {
    "tiny": ModelShape("tiny", 4096, 256, 128, 128, 128, "fp32", 4096),
    "qwen3-8b": ModelShape("qwen3-8b", 151936, 4096, 1024, 1024, 1024, "bf16", 8),
    "27b-class": ModelShape("27b-class", 151936, 5120, 1280, 1280, 1280, "bf16", 27),
}


@dataclass(frozen=True)
class Workload:
    """One configuration of the rollout: a model shape, a batch and K modes."""
    name: str
    model: str
    batch: int
    ks: tuple
    input_seed: int


WORKLOADS = {
    "tiny_b1": Workload("tiny_b1", "tiny", 1, (0, 256), 4096),
    "8b_b1": Workload("8b_b1", "qwen3-8b", 1, (0,), 8001),
    "8b_b8": Workload("8b_b8", "qwen3-8b", 8, (2048,), 8008),
    "8b_b64": Workload("8b_b64", "qwen3-8b", 64, (0, 2048), 8064),
    "27b_b64": Workload("27b_b64", "27b-class", 64, (2048,), 27064),
}


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round-to-nearest-even (no NaNs here)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal_blocks(seed_words, n, std, to_bf16):
    """n draws of N(0, std^2), block-seeded, optionally rounded to bf16 bits."""
    out = np.empty(n, np.uint16 if to_bf16 else np.float32)
    nblk = (n + BLOCK - 1) // BLOCK

    def fill(j):
        lo, hi = j * BLOCK, min(n, (j + 1) * BLOCK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed_words) + [j])))
        buf = g.standard_normal(hi - lo, dtype=np.float32)
        buf *= np.float32(std)
        out[lo:hi] = round_to_bf16_bits(buf) if to_bf16 else buf

    if nblk == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out


@dataclass
class Weights:
    """Synthetic weight set.  For bf16 models ``raw`` holds uint16 bit patterns,
    for fp32 models float32 arrays; ``f32(name)`` gives the exact float32 view."""
    shape: ModelShape
    raw: dict
    scales: dict = field(default_factory=dict)
    _f32: dict = field(default_factory=dict)

    def f32(self, name):
        if name not in self._f32:
            a = self.raw[name]
            self._f32[name] = bf16_bits_to_f32(a) if a.dtype == np.uint16 else a
        return self._f32[name]

    def drop_f32(self):
        self._f32.clear()


def make_weights(shape: ModelShape, scales: dict | None = None, seed: int | None = None) -> Weights:
    """Draw the weight set of ``shape``.  ``scales`` multiplies the N(0,1/fan_in)
    standard deviation per tensor (used by tests that need a strong GRU path)."""
    scales = dict(scales or {})
    seed = shape.weight_seed if seed is None else seed
    bf16 = shape.dtype == "bf16"
    raw = {}
    for name, shp in shape.tensor_shapes().items():
        std = scales.get(name, 1.0) / np.sqrt(shape.fan_in(name))
        flat = _normal_blocks((seed, _STREAMS[name]), int(np.prod(shp)), std, bf16)
        raw[name] = flat.reshape(shp)
    return Weights(shape, raw, scales)


@dataclass
class Inputs:
    hidden: np.ndarray      # [B,15,H] uint16 bf16 bits or float32
    step_s: np.ndarray      # [B,14,r] float32
    verified: np.ndarray    # [B] int32

    def hidden_f32(self):
        h = self.hidden
        return bf16_bits_to_f32(h) if h.dtype == np.uint16 else h


def make_inputs(shape: ModelShape, batch: int, input_seed: int, trial: int,
                s_scale: float = 1.0, hidden_scale: float = 1.0) -> Inputs:
    bf16 = shape.dtype == "bf16"
    base = (input_seed, 1 + trial)
    hid = _normal_blocks(base + (_INPUT_STREAMS["hidden"],),
                         batch * N_PROPOSALS * shape.hidden, hidden_scale, bf16)
    s = _normal_blocks(base + (_INPUT_STREAMS["step_s"],),
                       batch * N_STEPS * shape.proj_dim, s_scale, False)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(base) + [_INPUT_STREAMS["verified"]])))
    ver = g.integers(0, shape.vocab, size=batch, dtype=np.int64).astype(np.int32)
    return Inputs(hid.reshape(batch, N_PROPOSALS, shape.hidden),
                  s.reshape(batch, N_STEPS, shape.proj_dim), ver)


def custom_shape(vocab, hidden, emb_dim, gru_hidden, proj_dim, dtype, seed, name="custom"):
    return ModelShape(name, vocab, hidden, emb_dim, gru_hidden, proj_dim, dtype, seed)
