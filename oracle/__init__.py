"""CPU oracle for the activation-sparse gated FFN forward -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg import this package. The product path (the HIP library and its Python
binding) never imports it. Arithmetic lives in ``sffn_oracle.c`` (plain C,
fp64); this module only marshals numpy arrays and composes the steps in the
order the pages give them: gate first, then the selection, then the up and
down products over the selected channels.

Sources: "Model Casting and Low-Parameter Gating: Towards More Sparsely
Activated FFNs", Abstract (gate-first skipping, LoPA); "Mixture-of-Channels:
Exploiting Sparse FFNs for Efficient LLMs Pre-Training and Inference" (blog
summary), sections "Dentro il 'mixture'" and "'Dentro MoC'" (per-token Top-K of
the SwiGLU gate, binary mask, loading only active rows; the 2:8 structured
option).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sffn_oracle.c")
_SO = os.path.join(_HERE, "libsffn_oracle.so")
_SO_OMP = os.path.join(_HERE, "libsffn_oracle_omp.so")  # the same source with OpenMP (multi-core timing)

DT = {"f32": 0, "bf16": 1, "f64": 2}

# Band half-width around the decision boundary, from the stated parity rule:
# channels whose oracle pre-activation lies within 1e-5 of tau (threshold), or
# whose key lies within 1e-5 of the boundary between the last kept and the
# first dropped key (Top-K; 2:8 within each group), may be decided either way.
BAND = 1e-5


def build(force: bool = False, omp: bool = False) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, no FMA contraction);
    omp: the OpenMP build of the same source (for the multi-core timing)."""
    so = _SO_OMP if omp else _SO
    if force or not os.path.exists(so) or os.path.getmtime(so) < os.path.getmtime(_SRC):
        tmp = so + ".tmp"
        flags = ["-fopenmp"] if omp else ["-Wno-unknown-pragmas"]
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", *flags,
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, so)
    return so


_lib = None


def use_openmp() -> None:
    """Load the OpenMP build (before the first call; for the multi-core timing)."""
    global _lib
    assert _lib is None, "the oracle library is already loaded"
    os.environ["SFFN_ORACLE_SO"] = build(omp=True)


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        # SFFN_ORACLE_SO points the loader at another build of this source; the
        # mutation tests use it to check that the pins catch planted mistakes.
        _lib = ctypes.CDLL(os.environ.get("SFFN_ORACLE_SO") or build())
        P = ctypes.c_void_p
        I = ctypes.c_int
        L = ctypes.c_long
        D = ctypes.c_double
        _lib.oracle_widen.argtypes = [P, I, L, P]
        _lib.oracle_gate_full.argtypes = [I, I, I, P, I, P, I, P]
        _lib.oracle_gate_lopa.argtypes = [I, I, I, I, P, I, P, P, I, P, P]
        _lib.oracle_select_threshold.argtypes = [I, I, P, D, P, P]
        _lib.oracle_select_topk.argtypes = [I, I, I, P, P, P, P, P]
        _lib.oracle_select_topk.restype = I
        _lib.oracle_select_topp.argtypes = [I, I, D, P, P, P, P, P, P]
        _lib.oracle_select_topp.restype = I
        _lib.oracle_select_nm.argtypes = [I, I, I, I, P, P, P, P]
        _lib.oracle_select_nm.restype = I
        _lib.oracle_select_dense.argtypes = [I, I, I, P, D, P, P]
        _lib.oracle_up.argtypes = [I, I, I, P, I, P, I, P, P, I, P]
        _lib.oracle_down.argtypes = [I, I, I, P, P, I, P, I, P]
        _lib.oracle_union.argtypes = [I, I, P, P]
        _lib.oracle_backward.argtypes = [I, I, I, I, D, P, I, P, I, P, P, P, I, P, P, P, P, P]
        _lib.oracle_union.restype = I
    return _lib


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float64:
        return DT["f64"]
    if a.dtype == np.float32:
        return DT["f32"]
    if a.dtype == np.uint16:
        return DT["bf16"]
    raise TypeError(f"oracle input dtype {a.dtype} (expected float64, float32 or uint16 bf16 bits)")


def _c(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a)


def _p(a: np.ndarray) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data)


def widen(a: np.ndarray) -> np.ndarray:
    a = _c(a)
    out = np.empty(a.shape, dtype=np.float64)
    lib().oracle_widen(_p(a), _dt(a), a.size, _p(out))
    return out


def gate_full(x: np.ndarray, w_gate: np.ndarray) -> np.ndarray:
    x, w_gate = _c(x), _c(w_gate)
    n, d = x.shape
    f = w_gate.shape[0]
    assert w_gate.shape == (f, d)
    z = np.empty((n, f), dtype=np.float64)
    lib().oracle_gate_full(n, d, f, _p(x), _dt(x), _p(w_gate), _dt(w_gate), _p(z))
    return z


def gate_lopa(x: np.ndarray, a_t: np.ndarray, b_t: np.ndarray):
    """LoPA gate. a_t is A stored transposed [r][d]; b_t is B stored transposed [F][r]."""
    x, a_t, b_t = _c(x), _c(a_t), _c(b_t)
    n, d = x.shape
    r = a_t.shape[0]
    f = b_t.shape[0]
    assert a_t.shape == (r, d) and b_t.shape == (f, r)
    assert _dt(a_t) == _dt(b_t)
    t = np.empty((n, r), dtype=np.float64)
    z = np.empty((n, f), dtype=np.float64)
    lib().oracle_gate_lopa(n, d, r, f, _p(x), _dt(x), _p(a_t), _p(b_t), _dt(a_t), _p(t), _p(z))
    return t, z


def select_threshold(z: np.ndarray, tau: float):
    z = _c(np.asarray(z, dtype=np.float64))
    n, f = z.shape
    mask = np.empty((n, f), dtype=np.uint8)
    g = np.empty((n, f), dtype=np.float64)
    lib().oracle_select_threshold(n, f, _p(z), float(tau), _p(mask), _p(g))
    return mask, g


def select_topk(z: np.ndarray, k: int):
    z = _c(np.asarray(z, dtype=np.float64))
    n, f = z.shape
    mask = np.empty((n, f), dtype=np.uint8)
    g = np.empty((n, f), dtype=np.float64)
    kth = np.empty((n,), dtype=np.float64)
    nxt = np.empty((n,), dtype=np.float64)
    rc = lib().oracle_select_topk(n, f, int(k), _p(z), _p(mask), _p(g), _p(kth), _p(nxt))
    if rc != 0:
        raise ValueError(f"top-k with k={k} over {f} channels")
    return mask, g, kth, nxt


def select_topp(z: np.ndarray, p: float):
    """Top-p of the SiLU gate by cumulative softmax mass. Returns the mask, the
    gate values, the prefix masses [n][2] (without / with the last kept
    channel), and the last kept / first dropped keys."""
    z = _c(np.asarray(z, dtype=np.float64))
    n, f = z.shape
    mask = np.empty((n, f), dtype=np.uint8)
    g = np.empty((n, f), dtype=np.float64)
    cum = np.empty((n, 2), dtype=np.float64)
    kth = np.empty((n,), dtype=np.float64)
    nxt = np.empty((n,), dtype=np.float64)
    rc = lib().oracle_select_topp(n, f, float(p), _p(z), _p(mask), _p(g), _p(cum), _p(kth), _p(nxt))
    if rc != 0:
        raise ValueError(f"top-p with p={p}")
    return mask, g, cum, kth, nxt


def select_nm(z: np.ndarray, n_keep: int = 2, group: int = 8):
    """Structured n_keep:group selection of the SiLU gate (2:8 by default).
    Returns the mask, the gate values and each channel's group boundary
    (midway between the group's n_keep-th and next largest keys; -inf where
    the group keeps all)."""
    z = _c(np.asarray(z, dtype=np.float64))
    n, f = z.shape
    mask = np.empty((n, f), dtype=np.uint8)
    g = np.empty((n, f), dtype=np.float64)
    bound = np.empty((n, f), dtype=np.float64)
    rc = lib().oracle_select_nm(n, f, int(n_keep), int(group), _p(z), _p(mask), _p(g), _p(bound))
    if rc != 0:
        raise ValueError(f"{n_keep}:{group} selection")
    return mask, g, bound


def select_dense(z: np.ndarray, act: str, tau: float = 0.0):
    z = _c(np.asarray(z, dtype=np.float64))
    n, f = z.shape
    mask = np.empty((n, f), dtype=np.uint8)
    g = np.empty((n, f), dtype=np.float64)
    lib().oracle_select_dense(n, f, {"relu": 0, "silu": 1}[act], _p(z), float(tau), _p(mask), _p(g))
    return mask, g


def up(x: np.ndarray, w_up: np.ndarray, mask: np.ndarray, g: np.ndarray, skip: bool) -> np.ndarray:
    x, w_up = _c(x), _c(w_up)
    mask = _c(np.asarray(mask, dtype=np.uint8))
    g = _c(np.asarray(g, dtype=np.float64))
    n, d = x.shape
    f = w_up.shape[0]
    assert w_up.shape == (f, d) and mask.shape == (n, f) and g.shape == (n, f)
    h = np.empty((n, f), dtype=np.float64)
    lib().oracle_up(n, d, f, _p(x), _dt(x), _p(w_up), _dt(w_up), _p(mask), _p(g), int(skip), _p(h))
    return h


def down(h: np.ndarray, w_down: np.ndarray, mask: np.ndarray, skip: bool) -> np.ndarray:
    h = _c(np.asarray(h, dtype=np.float64))
    w_down = _c(w_down)
    mask = _c(np.asarray(mask, dtype=np.uint8))
    n, f = h.shape
    d = w_down.shape[1]
    assert w_down.shape == (f, d) and mask.shape == (n, f)
    y = np.empty((n, d), dtype=np.float64)
    lib().oracle_down(n, d, f, _p(h), _p(w_down), _dt(w_down), _p(mask), int(skip), _p(y))
    return y


def union(mask: np.ndarray):
    mask = _c(np.asarray(mask, dtype=np.uint8))
    n, f = mask.shape
    un = np.empty((f,), dtype=np.uint8)
    cnt = lib().oracle_union(n, f, _p(mask), _p(un))
    return un, cnt


@dataclasses.dataclass
class Result:
    z: np.ndarray          # gate pre-activation [n][F], fp64
    mask: np.ndarray       # active channels [n][F], uint8
    g: np.ndarray          # gate activation [n][F], fp64 (every channel)
    h: np.ndarray          # gated up values [n][F], fp64 (0 off the mask)
    y: np.ndarray          # output [n][d], fp64
    band: np.ndarray       # channels the parity rule leaves undecided [n][F], bool
    kth: Optional[np.ndarray] = None  # Top-K: the K-th largest key per token
    t: Optional[np.ndarray] = None    # LoPA: low-rank intermediate [n][r]


def forward(mode: str, x: np.ndarray, w_up: np.ndarray, w_down: np.ndarray, *,
            w_gate: Optional[np.ndarray] = None, lopa_a: Optional[np.ndarray] = None,
            lopa_b: Optional[np.ndarray] = None, tau: float = 0.0, k: int = 0,
            skip: bool = True, tau_f32: bool = True) -> Result:
    """The whole forward: gate, selection, up, down.

    mode: "threshold" (full gate, shifted ReLU), "lopa" (low-rank gate, shifted
    ReLU), "topk" (full gate, per-token Top-K of SiLU), "topk_2_8" (full gate,
    per-token top 2 of every aligned group of 8 SiLU keys), "topp" (full
    gate, per-token shortest prefix of the Top-K order whose softmax mass of
    the keys reaches p, passed as tau), "dense_relu" / "dense_silu" (every
    channel kept). tau is rounded to fp32 first when
    tau_f32 is set, so both sides compare against the same number.
    """
    if tau_f32:
        tau = float(np.float32(tau))  # also p of the top-p mode, an fp32 on the device
    t = kth = None
    if mode == "lopa":
        t, z = gate_lopa(x, lopa_a, lopa_b)
    else:
        z = gate_full(x, w_gate)
    if mode in ("threshold", "lopa"):
        mask, g = select_threshold(z, tau)
        band = np.abs(z - tau) <= BAND
    elif mode == "topk":
        mask, g, kth, nxt = select_topk(z, k)
        # the decision boundary lies between the K-th and (K+1)-th keys
        bnd = np.where(np.isfinite(nxt), 0.5 * (kth + nxt), -np.inf)
        band = np.abs(g - bnd[:, None]) <= BAND
    elif mode == "topp":
        # tau carries p; the band: a key within 1e-5 of the boundary, or a
        # boundary channel whose inclusion turns on a prefix mass within 1e-5
        # of p (the last kept one if the mass without it is that close, the
        # first dropped one if the mass with the last kept one is)
        mask, g, cum, kth, nxt = select_topp(z, tau)
        bnd = np.where(np.isfinite(nxt), 0.5 * (kth + nxt), -np.inf)
        band = np.abs(g - bnd[:, None]) <= BAND
        for tok in range(z.shape[0]):
            if tau - cum[tok, 0] <= BAND:
                band[tok] |= mask[tok].astype(bool) & (g[tok] == kth[tok])
            if cum[tok, 1] - tau <= BAND and np.isfinite(nxt[tok]):
                band[tok] |= ~mask[tok].astype(bool) & (g[tok] == nxt[tok])
    elif mode == "topk_2_8":
        mask, g, bound = select_nm(z, 2, 8)
        band = np.abs(g - bound) <= BAND
    elif mode == "dense_relu":
        mask, g = select_dense(z, "relu", tau)
        band = np.zeros(z.shape, dtype=bool)
    elif mode == "dense_silu":
        mask, g = select_dense(z, "silu")
        band = np.zeros(z.shape, dtype=bool)
    else:
        raise ValueError(f"unknown mode {mode!r}")
    h = up(x, w_up, mask, g, skip)
    y = down(h, w_down, mask, skip)
    return Result(z=z, mask=mask, g=g, h=h, y=y, band=band, kth=kth, t=t)


# Backward activation kind of each mode: 0 = shifted ReLU on its active branch
# (g = z - tau, g' = 1), 1 = SiLU.
BWD_KIND = {"threshold": 0, "dense_relu": 0, "topk": 1, "topk_2_8": 1, "topp": 1, "dense_silu": 1}


def saved_set(mode: str, res: "Result", tau: float) -> np.ndarray:
    """The channels whose activations a training forward keeps for the
    backward: the active set, except that the dense shifted ReLU keeps only
    the channels it leaves nonzero (z > tau): the others pass no gradient."""
    if mode == "dense_relu":
        return (res.z > tau).astype(np.uint8)
    return res.mask.astype(np.uint8)


def backward(mode: str, x: np.ndarray, dy: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray,
             w_down: np.ndarray, mask: np.ndarray, tau: float = 0.0) -> dict:
    """Gradients of sum(dy * y) over a fixed active set `mask` [n][F]: dx
    [n][d], dw_gate, dw_up, dw_down [F][d], all fp64 (oracle_backward)."""
    x, dy = _c(x), _c(dy)
    w_gate, w_up, w_down = _c(w_gate), _c(w_up), _c(w_down)
    assert w_gate.dtype == w_up.dtype == w_down.dtype
    mask = _c(np.asarray(mask, dtype=np.uint8))
    n, d = x.shape
    f = w_up.shape[0]
    assert dy.shape == (n, d) and mask.shape == (n, f)
    assert w_gate.shape == w_up.shape == w_down.shape == (f, d)
    out = {k: np.empty(s, dtype=np.float64) for k, s in
           (("dx", (n, d)), ("dw_gate", (f, d)), ("dw_up", (f, d)), ("dw_down", (f, d)))}
    lib().oracle_backward(n, d, f, BWD_KIND[mode], float(tau), _p(x), _dt(x), _p(dy), _dt(dy), _p(w_gate),
                          _p(w_up), _p(w_down), _dt(w_up), _p(mask), _p(out["dx"]), _p(out["dw_gate"]),
                          _p(out["dw_up"]), _p(out["dw_down"]))
    return out


def forward_with_mask(x: np.ndarray, w_up: np.ndarray, w_down: np.ndarray, g: np.ndarray,
                      mask: np.ndarray) -> np.ndarray:
    """y for a given active set and the oracle's own gate values (used when the
    GPU decided a channel inside the band the other way)."""
    h = up(x, w_up, mask, g, True)
    return down(h, w_down, mask, True)
