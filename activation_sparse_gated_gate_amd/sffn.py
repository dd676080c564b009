"""Python binding of the C ABI in include/sffn.h (argument marshalling only).

Every function has the C name and takes the C arguments: device pointers as
Python ints (``tensor.data_ptr()``), sizes as ints, the stream as an int
handle. A non-OK status raises :class:`SffnError`. Nothing here computes any
part of the forward: all of it runs in the HIP kernels of ``libsffn.so``.
The library is loaded on first use; if it is missing it is built in-tree with
hipcc, and if that fails the import error propagates (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
# SFFN_LIBRARY points the loader at another build of the library (the host
# sanitizer test uses it); by default the in-tree build.
LIB_PATH = os.environ.get("SFFN_LIBRARY") or os.path.join(_PKG, "libsffn.so")

SFFN_OK = 0
SFFN_ERR_INVALID_ARG = -1
SFFN_ERR_UNSUPPORTED = -2
SFFN_ERR_HIP = -3
SFFN_ERR_WORKSPACE = -4

SFFN_F32 = 0
SFFN_BF16 = 1

SFFN_THRESHOLD = 0
SFFN_TOPK = 1
SFFN_LOPA = 2
SFFN_DENSE = 3
SFFN_DENSE_SILU = 4
SFFN_TOPK_2_8 = 5
SFFN_TOPP = 6

MODES = {"threshold": SFFN_THRESHOLD, "topk": SFFN_TOPK, "lopa": SFFN_LOPA,
         "dense": SFFN_DENSE, "dense_relu": SFFN_DENSE, "dense_silu": SFFN_DENSE_SILU,
         "topk_2_8": SFFN_TOPK_2_8, "topp": SFFN_TOPP}
DTYPES = {"f32": SFFN_F32, "bf16": SFFN_BF16}

# Names exported by the library, as declared in include/sffn.h.
EXPORTS = ("sffn_workspace_bytes", "sffn_create", "sffn_forward", "sffn_set_profile_events",
           "sffn_set_spin_limit", "sffn_destroy", "sffn_status_string", "sffn_train_workspace_bytes",
           "sffn_forward_train", "sffn_backward", "sffn_forward_noalloc", "sffn_set_token_groups")

# Bytes of the library's static device workspace (sffn_forward_noalloc).
SFFN_STATIC_SCRATCH_BYTES = 16 << 20

# Sticky error word of the workspace (include/sffn.h).
SFFN_WS_ERROR_OFFSET = 4
SFFN_ERR_BIT_DOWN_WAIT = 1


class sffn_shape(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int), ("d_ff", ctypes.c_int), ("rank", ctypes.c_int),
                ("max_tokens", ctypes.c_int), ("dtype", ctypes.c_int)]


class sffn_weights(ctypes.Structure):
    _fields_ = [("w_gate", ctypes.c_void_p), ("lopa_a", ctypes.c_void_p), ("lopa_b", ctypes.c_void_p),
                ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p)]


class sffn_saved(ctypes.Structure):
    _fields_ = [("cap", ctypes.c_int), ("cnt", ctypes.c_void_p), ("idx", ctypes.c_void_p),
                ("z", ctypes.c_void_p), ("u", ctypes.c_void_p)]


class SffnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {sffn_status_string(status)} ({status})")


_lib = None
_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """Load libsffn.so (building it first only if it does not exist)."""
    global _lib
    with _lock:
        if _lib is None:
            # torch ships its own HIP runtime under the same soname: when it
            # is importable it goes first, so the library binds to that
            # runtime (a second runtime loaded beside it finds no device)
            try:
                import torch  # noqa: F401
            except ImportError:
                pass
            if not os.path.exists(LIB_PATH):
                from . import _build
                _build.build()
            L = ctypes.CDLL(LIB_PATH)
            P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
            L.sffn_workspace_bytes.argtypes = [ctypes.POINTER(sffn_shape)]
            L.sffn_workspace_bytes.restype = Z
            L.sffn_create.argtypes = [ctypes.POINTER(sffn_shape), P, Z, ctypes.POINTER(P)]
            L.sffn_create.restype = I
            L.sffn_forward.argtypes = [P, P, I, ctypes.POINTER(sffn_weights), I, F, I, P, P, P, P, P, P]
            L.sffn_forward.restype = I
            L.sffn_forward_noalloc.argtypes = [ctypes.POINTER(sffn_shape), P, I, ctypes.POINTER(sffn_weights), I, F,
                                               I, P, P, P, P, P, P]
            L.sffn_forward_noalloc.restype = I
            L.sffn_set_profile_events.argtypes = [P, P, P]
            L.sffn_set_profile_events.restype = I
            L.sffn_set_token_groups.argtypes = [P, I]
            L.sffn_set_token_groups.restype = I
            L.sffn_set_spin_limit.argtypes = [P, I]
            L.sffn_set_spin_limit.restype = I
            L.sffn_destroy.argtypes = [P]
            L.sffn_destroy.restype = I
            L.sffn_train_workspace_bytes.argtypes = [ctypes.POINTER(sffn_shape)]
            L.sffn_train_workspace_bytes.restype = Z
            SV = ctypes.POINTER(sffn_saved)
            L.sffn_forward_train.argtypes = [P, P, I, ctypes.POINTER(sffn_weights), I, F, I, P, SV, P, Z, P]
            L.sffn_forward_train.restype = I
            L.sffn_backward.argtypes = [P, P, P, I, ctypes.POINTER(sffn_weights), I, F, I, SV, P, P, P, P, P, Z, P]
            L.sffn_backward.restype = I
            L.sffn_status_string.argtypes = [I]
            L.sffn_status_string.restype = ctypes.c_char_p
            _lib = L
    return _lib


def _check(status: int, where: str) -> None:
    if status != SFFN_OK:
        raise SffnError(status, where)


def sffn_status_string(status: int) -> str:
    return lib().sffn_status_string(int(status)).decode()


def make_shape(d_model: int, d_ff: int, rank: int, max_tokens: int, dtype) -> sffn_shape:
    dt = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    return sffn_shape(int(d_model), int(d_ff), int(rank), int(max_tokens), dt)


def sffn_workspace_bytes(shape: sffn_shape) -> int:
    return int(lib().sffn_workspace_bytes(ctypes.byref(shape)))


def sffn_create(shape: sffn_shape, workspace: int, workspace_bytes: int) -> int:
    h = ctypes.c_void_p()
    _check(lib().sffn_create(ctypes.byref(shape), ctypes.c_void_p(workspace), workspace_bytes,
                             ctypes.byref(h)), "sffn_create")
    return int(h.value)


def sffn_forward(handle: int, x: int, n_tokens: int, weights: sffn_weights, mode: int, tau: float,
                 k: int, y: int, active_idx: int = 0, active_cnt: int = 0, union_cnt: int = 0,
                 debug_z: int = 0, stream: int = 0) -> None:
    P = ctypes.c_void_p
    _check(lib().sffn_forward(P(handle), P(x), int(n_tokens), ctypes.byref(weights), int(mode),
                              float(tau), int(k), P(y), P(active_idx or None), P(active_cnt or None),
                              P(union_cnt or None), P(debug_z or None), P(stream or None)),
           "sffn_forward")


def sffn_forward_noalloc(shape: sffn_shape, x: int, n_tokens: int, weights: sffn_weights, mode: int, tau: float,
                         k: int, y: int, active_idx: int = 0, active_cnt: int = 0, union_cnt: int = 0,
                         debug_z: int = 0, stream: int = 0) -> None:
    P = ctypes.c_void_p
    _check(lib().sffn_forward_noalloc(ctypes.byref(shape), P(x), int(n_tokens), ctypes.byref(weights), int(mode),
                                      float(tau), int(k), P(y), P(active_idx or None), P(active_cnt or None),
                                      P(union_cnt or None), P(debug_z or None), P(stream or None)),
           "sffn_forward_noalloc")


def sffn_train_workspace_bytes(shape: sffn_shape) -> int:
    return int(lib().sffn_train_workspace_bytes(ctypes.byref(shape)))


def sffn_forward_train(handle: int, x: int, n_tokens: int, weights: sffn_weights, mode: int, tau: float,
                       k: int, y: int, saved: sffn_saved, train_ws: int, train_ws_bytes: int,
                       stream: int = 0) -> None:
    P = ctypes.c_void_p
    _check(lib().sffn_forward_train(P(handle), P(x), int(n_tokens), ctypes.byref(weights), int(mode),
                                    float(tau), int(k), P(y), ctypes.byref(saved), P(train_ws),
                                    int(train_ws_bytes), P(stream or None)), "sffn_forward_train")


def sffn_backward(handle: int, x: int, dy: int, n_tokens: int, weights: sffn_weights, mode: int, tau: float,
                  k: int, saved: sffn_saved, dx: int, dw_gate: int, dw_up: int, dw_down: int, train_ws: int,
                  train_ws_bytes: int, stream: int = 0) -> None:
    P = ctypes.c_void_p
    _check(lib().sffn_backward(P(handle), P(x), P(dy), int(n_tokens), ctypes.byref(weights), int(mode),
                               float(tau), int(k), ctypes.byref(saved), P(dx), P(dw_gate), P(dw_up), P(dw_down),
                               P(train_ws), int(train_ws_bytes), P(stream or None)), "sffn_backward")


def sffn_set_profile_events(handle: int, ev_start: int, ev_stop: int) -> None:
    _check(lib().sffn_set_profile_events(ctypes.c_void_p(handle), ctypes.c_void_p(ev_start or None),
                                         ctypes.c_void_p(ev_stop or None)), "sffn_set_profile_events")


def sffn_set_token_groups(handle: int, groups: int) -> None:
    _check(lib().sffn_set_token_groups(ctypes.c_void_p(handle), int(groups)), "sffn_set_token_groups")


def sffn_set_spin_limit(handle: int, polls: int) -> None:
    _check(lib().sffn_set_spin_limit(ctypes.c_void_p(handle), int(polls)), "sffn_set_spin_limit")


def sffn_destroy(handle: int) -> None:
    _check(lib().sffn_destroy(ctypes.c_void_p(handle)), "sffn_destroy")


# ---------------------------------------------------------------------------
# Convenience wrapper over torch tensors (still marshalling only): owns the
# workspace tensor and passes data pointers and torch's current stream.
# ---------------------------------------------------------------------------
class SparseFFN:
    """One handle plus its workspace for a layer shape on the current device."""

    def __init__(self, d_model: int, d_ff: int, max_tokens: int, dtype: str = "bf16", rank: int = 0,
                 device=None):
        import torch

        self.shape = make_shape(d_model, d_ff, rank, max_tokens, dtype)
        nbytes = sffn_workspace_bytes(self.shape)
        if nbytes == 0:
            raise SffnError(SFFN_ERR_INVALID_ARG, "sffn_workspace_bytes")
        self.workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device=device or "cuda")
        base = self.workspace.data_ptr()
        aligned = (base + 255) & ~255
        self.handle = sffn_create(self.shape, aligned, nbytes)
        self.dtype = dtype

    @staticmethod
    def weights(w_gate=None, w_up=None, w_down=None, lopa_a=None, lopa_b=None) -> sffn_weights:
        """Pointer struct for the C call. It keeps the tensors alive, so the
        memory cannot be recycled while the struct is in use."""
        ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
        w = sffn_weights(ptr(w_gate), ptr(lopa_a), ptr(lopa_b), ptr(w_up), ptr(w_down))
        w._keep = (w_gate, w_up, w_down, lopa_a, lopa_b)
        return w

    def forward(self, x, weights: sffn_weights, mode, y, tau: float = 0.0, k: int = 0,
                active_idx=None, active_cnt=None, union_cnt=None, debug_z=None,
                stream: Optional[int] = None) -> None:
        import torch

        m = MODES[mode] if isinstance(mode, str) else int(mode)
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        ptr = lambda t: 0 if t is None else t.data_ptr()  # noqa: E731
        sffn_forward(self.handle, x.data_ptr(), x.shape[0], weights, m, tau, k, y.data_ptr(),
                     ptr(active_idx), ptr(active_cnt), ptr(union_cnt), ptr(debug_z), stream)

    # ---- training ----
    def _train_ws(self):
        import torch

        if getattr(self, "train_workspace", None) is None:
            nbytes = sffn_train_workspace_bytes(self.shape)
            self.train_workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.workspace.device)
            self._train_bytes = nbytes
        return (self.train_workspace.data_ptr() + 255) & ~255, self._train_bytes

    @staticmethod
    def saved(cap: int, cnt, idx, z, u) -> sffn_saved:
        """Pointer struct of the stored activations (cnt int32 [n], idx int32
        [n][cap], z and u fp32 [n][cap]); keeps the tensors alive."""
        v = sffn_saved(int(cap), cnt.data_ptr(), idx.data_ptr(), z.data_ptr(), u.data_ptr())
        v._keep = (cnt, idx, z, u)
        return v

    def forward_train(self, x, weights: sffn_weights, mode, y, saved: sffn_saved, tau: float = 0.0, k: int = 0,
                      stream: Optional[int] = None) -> None:
        import torch

        m = MODES[mode] if isinstance(mode, str) else int(mode)
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        ws, nb = self._train_ws()
        sffn_forward_train(self.handle, x.data_ptr(), x.shape[0], weights, m, tau, k, y.data_ptr(), saved, ws, nb,
                           stream)

    def backward(self, x, dy, weights: sffn_weights, mode, saved: sffn_saved, dx, dw_gate, dw_up, dw_down,
                 tau: float = 0.0, k: int = 0, stream: Optional[int] = None) -> None:
        import torch

        m = MODES[mode] if isinstance(mode, str) else int(mode)
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        ws, nb = self._train_ws()
        sffn_backward(self.handle, x.data_ptr(), dy.data_ptr(), x.shape[0], weights, m, tau, k, saved,
                      dx.data_ptr(), dw_gate.data_ptr(), dw_up.data_ptr(), dw_down.data_ptr(), ws, nb, stream)

    def set_token_groups(self, groups: int) -> None:
        sffn_set_token_groups(self.handle, groups)

    def set_spin_limit(self, polls: int) -> None:
        sffn_set_spin_limit(self.handle, polls)

    def set_profile_events(self, start_event, stop_event) -> None:
        sffn_set_profile_events(self.handle, start_event.cuda_event if start_event is not None else 0,
                                stop_event.cuda_event if stop_event is not None else 0)

    def close(self) -> None:
        if getattr(self, "handle", None):
            sffn_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
