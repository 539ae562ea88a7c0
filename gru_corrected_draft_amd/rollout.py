"""Thin ctypes binding of ``libdomino_rollout.so``.

Argument marshalling only: every step of the rollout runs in the library's
HIP kernels.  PyTorch supplies device memory (``tensor.data_ptr()``) and the
stream (``torch.cuda.current_stream().cuda_stream``).  The library must be
built (``python -m gru_corrected_draft_amd.build``); importing this module
without it raises, there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.environ.get("DOMINO_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libdomino_rollout.so")

DOMINO_OK = 0
DOMINO_ERR_INVALID_ARG = -1
DOMINO_ERR_INVALID_CONFIG = -2
DOMINO_ERR_UNSUPPORTED = -3
DOMINO_ERR_OUT_OF_MEMORY = -4
DOMINO_ERR_HIP = -5
DTYPE_BF16, DTYPE_FP32 = 0, 1

BLOCK_SIZE = 16
N_PROPOSALS = 15
N_STEPS = 14

EXPORTED = ("domino_rollout_create", "domino_rollout_run", "domino_rollout_run_graph",
            "domino_rollout_run_prefix", "domino_rollout_run_forced",
            "domino_rollout_read_workspace", "domino_rollout_destroy",
            "domino_rollout_last_error", "domino_rollout_set_timing",
            "domino_rollout_kernel_times", "domino_rollout_set_pool_strategy",
            "domino_rollout_set_step_path", "domino_rollout_cached_graphs",
            "domino_rollout_run_static")
STATIC_SCRATCH_BYTES = 4 << 20  # DOMINO_STATIC_SCRATCH_BYTES
GRAPH_CACHE_MAX = 16  # DOMINO_GRAPH_CACHE_MAX
# gru: the GRU gates (prefix launch, separate gate kernel); step: projector
# layer 1 and W_hh of the new state (with the gates where fused)
PHASES = {"lmhead": 0, "correct": 1, "gru": 2, "step": 3, "pool": 4, "argmax0": 5, "offsets": 6}


class Config(ctypes.Structure):
    _fields_ = [("vocab", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("emb_dim", ctypes.c_int32), ("gru_hidden", ctypes.c_int32),
                ("proj_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("pure_draft_prefix_len", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("max_k", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class WeightPtrs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("lm_head", "embed", "gru_w_ih", "gru_w_hh", "fc1_w", "fc2_w", "fc2_b",
                 "fc1_x_w", "fc1_b")]


# required weights, and the optional pair that lets the library form step_s
WEIGHT_NAMES = ["lm_head", "embed", "gru_w_ih", "gru_w_hh", "fc1_w", "fc2_w", "fc2_b"]
OFFSET_WEIGHT_NAMES = ["fc1_x_w", "fc1_b"]

_lib = None


def load_library():
    """Load the in-tree library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    # torch first: its bundled HIP runtime carries the same soname, so the
    # library binds to that one copy instead of loading a second runtime
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m gru_corrected_draft_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i32p, f32p = ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p
    lib.domino_rollout_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(WeightPtrs),
                                          ctypes.POINTER(vp)]
    lib.domino_rollout_create.restype = ctypes.c_int
    run_args = [vp, vp, f32p, i32p, i32, i32, i32p, f32p, vp]
    lib.domino_rollout_run.argtypes = run_args
    lib.domino_rollout_run.restype = ctypes.c_int
    lib.domino_rollout_run_graph.argtypes = run_args
    lib.domino_rollout_run_graph.restype = ctypes.c_int
    lib.domino_rollout_run_static.argtypes = run_args
    lib.domino_rollout_run_static.restype = ctypes.c_int
    lib.domino_rollout_run_prefix.argtypes = [vp, vp, f32p, i32p, i32, i32, i32, i32p, f32p, i32,
                                              vp]
    lib.domino_rollout_run_prefix.restype = ctypes.c_int
    lib.domino_rollout_run_forced.argtypes = [vp, vp, f32p, i32p, i32p, i32, i32, i32p, f32p, vp]
    lib.domino_rollout_run_forced.restype = ctypes.c_int
    lib.domino_rollout_read_workspace.argtypes = [vp, i32, vp, ctypes.c_size_t,
                                                  ctypes.POINTER(ctypes.c_size_t), vp]
    lib.domino_rollout_read_workspace.restype = ctypes.c_int
    lib.domino_rollout_destroy.argtypes = [vp]
    lib.domino_rollout_destroy.restype = None
    lib.domino_rollout_last_error.argtypes = [vp]
    lib.domino_rollout_last_error.restype = ctypes.c_char_p
    lib.domino_rollout_set_timing.argtypes = [vp, i32]
    lib.domino_rollout_set_timing.restype = ctypes.c_int
    lib.domino_rollout_set_pool_strategy.argtypes = [vp, i32]
    lib.domino_rollout_set_pool_strategy.restype = ctypes.c_int
    lib.domino_rollout_set_step_path.argtypes = [vp, i32]
    lib.domino_rollout_set_step_path.restype = ctypes.c_int
    lib.domino_rollout_kernel_times.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_double),
                                                ctypes.POINTER(ctypes.c_int64)]
    lib.domino_rollout_kernel_times.restype = ctypes.c_int
    lib.domino_rollout_cached_graphs.argtypes = [vp, ctypes.POINTER(ctypes.c_int32)]
    lib.domino_rollout_cached_graphs.restype = ctypes.c_int
    _lib = lib
    return lib


class DominoError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"status {status}: {msg}")
        self.status = status


def make_config(vocab, hidden, emb_dim, gru_hidden, proj_dim, max_batch, max_k, dtype,
                block_size=BLOCK_SIZE, pure_draft_prefix_len=1):
    return Config(vocab, hidden, emb_dim, gru_hidden, proj_dim, block_size,
                  pure_draft_prefix_len, max_batch, max_k, dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def check_outputs(out_tokens, out_top1, B, P, device):
    """The library writes [B, P] int32 tokens and [B, P] float32 logits at
    the given addresses with row stride P: both must be contiguous tensors of
    exactly that shape and dtype on the inputs' device (a host tensor would
    be written through a host address by the device)."""
    import torch
    for name, t, dt in (("out_tokens", out_tokens, torch.int32),
                        ("out_top1", out_top1, torch.float32)):
        if tuple(t.shape) != (B, P):
            raise ValueError(f"{name} must be [B, P] = [{B}, {P}], got {list(t.shape)}")
        if t.dtype != dt:
            raise ValueError(f"{name} must be {dt}, got {t.dtype}")
        if t.device != device:
            raise ValueError(f"{name} must be on {device}, got {t.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def check_forced(forced, B, device):
    """Teacher-forced tokens are read as forced[b * 15 + j]: [B, 15] int32,
    contiguous, on the inputs' device."""
    import torch
    if tuple(forced.shape) != (B, N_PROPOSALS) or forced.dtype != torch.int32:
        raise ValueError("forced must be [B, 15] int32")
    if forced.device != device or not forced.is_contiguous():
        raise ValueError(f"forced must be a contiguous tensor on {device}")


class DominoRollout:
    """Handle over ``domino_rollout_t``.  ``weights`` maps the names of
    ``WEIGHT_NAMES`` to contiguous device tensors (bfloat16 or float32); the
    tensors are kept alive by this object because the library borrows them."""

    def __init__(self, weights: dict, max_batch: int, max_k: int):
        import torch
        self.lib = load_library()
        lm = weights["lm_head"]
        dt = lm.dtype
        if dt not in (torch.bfloat16, torch.float32):
            raise TypeError("weights must be bfloat16 or float32")
        self.has_offsets = all(n in weights for n in OFFSET_WEIGHT_NAMES)
        for n in WEIGHT_NAMES + (OFFSET_WEIGHT_NAMES if self.has_offsets else []):
            t = weights[n]
            if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
                raise TypeError(f"weight {n} must be a contiguous {dt} device tensor")
        V, H = lm.shape
        e = weights["embed"].shape[1]
        g = weights["gru_w_hh"].shape[1]
        r = weights["fc1_w"].shape[0]
        self.dtype = dt
        self.shape = (V, H, e, g, r)
        self.cfg = make_config(V, H, e, g, r, max_batch, max_k,
                               DTYPE_BF16 if dt == torch.bfloat16 else DTYPE_FP32)
        self._weights = dict(weights)
        names = WeightPtrs._fields_
        wp = WeightPtrs(*[weights[n].data_ptr() if n in weights and
                          (n not in OFFSET_WEIGHT_NAMES or self.has_offsets) else None
                          for n, _ in names])
        h = ctypes.c_void_p()
        st = self.lib.domino_rollout_create(ctypes.byref(self.cfg), ctypes.byref(wp), ctypes.byref(h))
        if st != DOMINO_OK:
            raise DominoError(st, self.lib.domino_rollout_last_error(None).decode())
        self.handle = h

    def _check(self, st):
        if st != DOMINO_OK:
            raise DominoError(st, self.lib.domino_rollout_last_error(self.handle).decode())

    def run(self, hidden, step_s, verified, K, out_tokens=None, out_top1=None, graph=False,
            forced=None, stream=None, proposals=None, static=False):
        """Enqueue one rollout; returns (out_tokens [B,P] int32, out_top1 [B,P] fp32),
        P = 15, or `proposals` for a truncated rollout (domino_rollout_run_prefix).
        static=True runs domino_rollout_run_static (per-run scratch in the
        library's static device array)."""
        import torch
        B = hidden.shape[0]
        V, H, e, g, r = self.shape
        if hidden.shape != (B, N_PROPOSALS, H) or hidden.dtype != self.dtype:
            raise ValueError("hidden must be [B, 15, H] in the weights' dtype")
        if step_s is None:
            if not self.has_offsets:
                raise ValueError("step_s is required: the handle holds no fc1_x_w / fc1_b")
        elif step_s.shape != (B, N_STEPS, r) or step_s.dtype != torch.float32:
            raise ValueError("step_s must be [B, 14, r] float32")
        if verified.shape != (B,) or verified.dtype != torch.int32:
            raise ValueError("verified must be [B] int32")
        dev = hidden.device
        for t in (hidden, verified) + (() if step_s is None else (step_s,)):
            if not t.is_cuda or not t.is_contiguous() or t.device != dev:
                raise ValueError("inputs must be contiguous tensors on one device")
        P = N_PROPOSALS if proposals is None else int(proposals)
        if out_tokens is None:
            out_tokens = torch.empty((B, P), dtype=torch.int32, device=dev)
        if out_top1 is None:
            out_top1 = torch.empty((B, P), dtype=torch.float32, device=dev)
        check_outputs(out_tokens, out_top1, B, P, dev)
        if forced is not None:
            check_forced(forced, B, dev)
        st_ptr = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream if stream is None
                                 else stream)
        if static:
            if proposals is not None or forced is not None or graph:
                raise ValueError("the static-scratch run is a plain full-block run")
            st = self.lib.domino_rollout_run_static(self.handle, _ptr(hidden), _ptr(step_s),
                                                    _ptr(verified), B, K, _ptr(out_tokens),
                                                    _ptr(out_top1), st_ptr)
        elif proposals is not None:
            if forced is not None:
                raise ValueError("teacher forcing runs the whole block")
            st = self.lib.domino_rollout_run_prefix(self.handle, _ptr(hidden), _ptr(step_s),
                                                    _ptr(verified), B, K, P, _ptr(out_tokens),
                                                    _ptr(out_top1), int(bool(graph)), st_ptr)
        elif forced is not None:
            st = self.lib.domino_rollout_run_forced(self.handle, _ptr(hidden), _ptr(step_s),
                                                    _ptr(verified), _ptr(forced), B, K,
                                                    _ptr(out_tokens), _ptr(out_top1), st_ptr)
        else:
            fn = self.lib.domino_rollout_run_graph if graph else self.lib.domino_rollout_run
            st = fn(self.handle, _ptr(hidden), _ptr(step_s), _ptr(verified), B, K,
                    _ptr(out_tokens), _ptr(out_top1), st_ptr)
        self._check(st)
        return out_tokens, out_top1

    def read_workspace(self, which):
        """Copy of a workspace buffer of the last run: 0 = base logits
        [15, B, V] fp32 (step-major), 1 = pool ids [B, K] int32, 2 = the step
        offsets [B, 14, r] fp32 the library formed (runs with step_s=None),
        3 = the pool union size of each group of 32 requests (24 or 16 when
        the projector is too wide for a 32-request panel), int32."""
        import torch
        n = ctypes.c_size_t()
        self._check(self.lib.domino_rollout_read_workspace(self.handle, which, None, 0,
                                                           ctypes.byref(n), None))
        dt = torch.int32 if which in (1, 3) else torch.float32
        out = torch.empty(n.value // 4, dtype=dt, device="cuda")
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        self._check(self.lib.domino_rollout_read_workspace(self.handle, which, _ptr(out), n.value,
                                                           ctypes.byref(n), st))
        return out

    def set_pool_strategy(self, strategy):
        """0 automatic, 1 per-request gather, 2 group unions where supported."""
        self._check(self.lib.domino_rollout_set_pool_strategy(self.handle, int(strategy)))

    def set_step_path(self, path):
        """0 automatic, 1 fused gates + rows, 2 gate kernel + rows, 3 gate kernel + matrix cores."""
        self._check(self.lib.domino_rollout_set_step_path(self.handle, int(path)))

    def cached_graphs(self):
        """Number of HIP graphs the handle holds (at most GRAPH_CACHE_MAX)."""
        n = ctypes.c_int32()
        self._check(self.lib.domino_rollout_cached_graphs(self.handle, ctypes.byref(n)))
        return n.value

    def set_timing(self, enable):
        self._check(self.lib.domino_rollout_set_timing(self.handle, 1 if enable else 0))

    def kernel_times(self):
        """{phase: (total ms, launches)} of the timed runs so far (waits on their events)."""
        out = {}
        for name, i in PHASES.items():
            ms, n = ctypes.c_double(), ctypes.c_int64()
            self._check(self.lib.domino_rollout_kernel_times(self.handle, i, ctypes.byref(ms),
                                                             ctypes.byref(n)))
            out[name] = (ms.value, n.value)
        return out

    def reset_kernel_times(self):
        self._check(self.lib.domino_rollout_kernel_times(self.handle, -1, None, None))

    def close(self):
        if getattr(self, "handle", None):
            self.lib.domino_rollout_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def device_weights(w, device="cuda"):
    """Upload a ``synth.Weights`` set: bf16 bit patterns -> torch.bfloat16."""
    import numpy as np
    import torch
    out = {}
    for n in WEIGHT_NAMES + [n for n in OFFSET_WEIGHT_NAMES if n in w.raw]:
        a = w.raw[n]
        if a.dtype == np.uint16:
            t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
        out[n] = t.to(device).contiguous()
    return out


def device_inputs(inp, device="cuda"):
    import numpy as np
    import torch
    h = inp.hidden
    if h.dtype == np.uint16:
        hid = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16)
    else:
        hid = torch.from_numpy(h)
    return (hid.to(device).contiguous(), torch.from_numpy(inp.step_s).to(device).contiguous(),
            torch.from_numpy(inp.verified).to(device).contiguous())
