"""The C-ABI library on the CPU: it loads, exports every declared symbol, sizes
workspaces, and rejects bad arguments with the documented status before any
HIP call (so nothing here needs a GPU)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

from activation_sparse_gated_gate_amd import sffn as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sffn.h")
FAKE_WS = 0x7F0000000000  # never dereferenced: validation fails first


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sffn_[a-z_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert _declared() == sorted(S.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = S.lib()
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", S.LIB_PATH], stdout=subprocess.PIPE, text=True).stdout
    exported = set(re.findall(r" T (sffn_\w+)", out))
    assert set(_declared()) <= exported


def test_status_strings():
    assert S.sffn_status_string(0) == "SFFN_OK"
    assert S.sffn_status_string(-1) == "SFFN_ERR_INVALID_ARG"
    assert S.sffn_status_string(-2) == "SFFN_ERR_UNSUPPORTED"
    assert S.sffn_status_string(-3) == "SFFN_ERR_HIP"
    assert S.sffn_status_string(-4) == "SFFN_ERR_WORKSPACE"
    assert S.sffn_status_string(7) == "SFFN_ERR_UNKNOWN"


@pytest.mark.parametrize("bad", [
    dict(d_model=0), dict(d_model=12), dict(d_ff=0), dict(d_ff=262145), dict(rank=4), dict(rank=-8),
    dict(max_tokens=0), dict(dtype=2),
])
def test_workspace_bytes_zero_for_invalid_shape(bad):
    kw = dict(d_model=64, d_ff=100, rank=0, max_tokens=4, dtype=1)
    kw.update(bad)
    assert S.sffn_workspace_bytes(S.sffn_shape(**kw)) == 0


def test_workspace_bytes_grow_with_shape():
    a = S.sffn_workspace_bytes(S.make_shape(4096, 11008, 0, 1, "bf16"))
    b = S.sffn_workspace_bytes(S.make_shape(4096, 11008, 256, 1, "bf16"))
    c = S.sffn_workspace_bytes(S.make_shape(8192, 28672, 0, 2048, "bf16"))
    assert 0 < a < b < c
    assert a % 256 == 0


def _raw_create(shape, ws, nbytes):
    h = ctypes.c_void_p()
    st = S.lib().sffn_create(ctypes.byref(shape) if shape is not None else None, ctypes.c_void_p(ws), nbytes,
                             ctypes.byref(h))
    return st, h.value


def test_create_errors():
    sh = S.make_shape(64, 100, 0, 4, "bf16")
    need = S.sffn_workspace_bytes(sh)
    assert S.lib().sffn_create(ctypes.byref(sh), ctypes.c_void_p(FAKE_WS), need, None) == S.SFFN_ERR_INVALID_ARG
    assert _raw_create(None, FAKE_WS, need)[0] == S.SFFN_ERR_INVALID_ARG
    assert _raw_create(S.make_shape(63, 100, 0, 4, "bf16"), FAKE_WS, need)[0] == S.SFFN_ERR_INVALID_ARG
    assert _raw_create(sh, 0, need)[0] == S.SFFN_ERR_WORKSPACE
    assert _raw_create(sh, FAKE_WS + 16, need)[0] == S.SFFN_ERR_WORKSPACE
    assert _raw_create(sh, FAKE_WS, need - 1)[0] == S.SFFN_ERR_WORKSPACE
    st, h = _raw_create(sh, FAKE_WS, need)
    assert st == S.SFFN_OK and h
    assert S.lib().sffn_destroy(ctypes.c_void_p(h)) == S.SFFN_OK
    assert S.lib().sffn_destroy(None) == S.SFFN_ERR_INVALID_ARG


class _Fake:
    """A handle over a never-touched fake workspace, and fake aligned pointers."""

    def __init__(self, rank=0, max_tokens=8, dtype="bf16", d=64, f=100):
        self.sh = S.make_shape(d, f, rank, max_tokens, dtype)
        self.h = S.sffn_create(self.sh, FAKE_WS, S.sffn_workspace_bytes(self.sh))
        self.w = S.sffn_weights(0x10000, 0x20000, 0x30000, 0x40000, 0x50000)

    def fwd(self, x=0x60000, n=1, w=None, mode=S.SFFN_THRESHOLD, tau=0.5, k=1, y=0x70000, idx=None,
            cnt=None, ucnt=None, dz=None):
        P = ctypes.c_void_p
        return S.lib().sffn_forward(P(self.h), P(x), n, ctypes.byref(w or self.w) if w is not False else None,
                                    mode, tau, k, P(y), P(idx), P(cnt), P(ucnt), P(dz), None)


@pytest.fixture
def fake():
    f = _Fake()
    yield f
    S.sffn_destroy(f.h)


def test_forward_rejects_bad_arguments(fake):
    E = S.SFFN_ERR_INVALID_ARG
    P = ctypes.c_void_p
    assert S.lib().sffn_forward(None, P(0x60000), 1, ctypes.byref(fake.w), 0, 0.5, 1, P(0x70000),
                                None, None, None, None, None) == E
    assert fake.fwd(w=False) == E
    assert fake.fwd(x=0) == E
    assert fake.fwd(y=0) == E
    assert fake.fwd(x=0x60008) == E                     # x not 16-byte aligned
    assert fake.fwd(y=0x70004) == E                     # y not 16-byte aligned
    assert fake.fwd(n=-1) == E
    assert fake.fwd(n=9) == E                           # above max_tokens
    assert fake.fwd(mode=7) == E
    assert fake.fwd(mode=S.SFFN_TOPP, tau=0.0) == E      # p outside (0, 1]
    assert fake.fwd(mode=S.SFFN_TOPP, tau=1.5) == E
    assert fake.fwd(mode=S.SFFN_TOPP, tau=math.nan) == E
    assert fake.fwd(mode=-1) == E
    assert fake.fwd(mode=S.SFFN_TOPK_2_8, w=S.sffn_weights(None, 0x20000, 0x30000, 0x40000, 0x50000)) == E
    assert fake.fwd(tau=math.nan) == E
    assert fake.fwd(mode=S.SFFN_TOPK, k=0) == E
    assert fake.fwd(mode=S.SFFN_TOPK, k=101) == E
    assert fake.fwd(mode=S.SFFN_LOPA) == E              # handle has rank 0
    assert fake.fwd(w=S.sffn_weights(None, 0x20000, 0x30000, 0x40000, 0x50000)) == E
    assert fake.fwd(w=S.sffn_weights(0x10000, None, None, None, 0x50000)) == E
    assert fake.fwd(w=S.sffn_weights(0x10000, None, None, 0x40000, None)) == E
    assert fake.fwd(w=S.sffn_weights(0x10002, None, None, 0x40000, 0x50000)) == E
    assert fake.fwd(idx=0x80001) == E
    assert fake.fwd(cnt=0x80002) == E
    assert fake.fwd(ucnt=0x80003) == E
    assert fake.fwd(dz=0x80001) == E


def test_forward_lopa_needs_both_factors():
    f = _Fake(rank=16)
    try:
        E = S.SFFN_ERR_INVALID_ARG
        assert f.fwd(mode=S.SFFN_LOPA, w=S.sffn_weights(None, None, 0x30000, 0x40000, 0x50000)) == E
        assert f.fwd(mode=S.SFFN_LOPA, w=S.sffn_weights(None, 0x20000, None, 0x40000, 0x50000)) == E
        assert f.fwd(mode=S.SFFN_LOPA, w=S.sffn_weights(None, 0x20008, 0x30000, 0x40000, 0x50000)) == E
    finally:
        S.sffn_destroy(f.h)


def test_zero_tokens_is_a_no_op(fake):
    assert fake.fwd(n=0) == S.SFFN_OK


def test_batched_unsupported_forms_are_rejected_before_any_hip_call():
    f = _Fake(max_tokens=64, dtype="f32")
    try:
        assert f.fwd(n=16) == S.SFFN_ERR_UNSUPPORTED   # the union path is bf16 only
    finally:
        S.sffn_destroy(f.h)
    g = _Fake(max_tokens=64, rank=16)
    try:
        assert g.fwd(n=16, mode=S.SFFN_LOPA) == S.SFFN_ERR_UNSUPPORTED
    finally:
        S.sffn_destroy(g.h)


def test_profile_events_arguments(fake):
    P = ctypes.c_void_p
    assert S.lib().sffn_set_profile_events(P(fake.h), P(0x1000), None) == S.SFFN_ERR_INVALID_ARG
    assert S.lib().sffn_set_profile_events(None, None, None) == S.SFFN_ERR_INVALID_ARG
    assert S.lib().sffn_set_profile_events(P(fake.h), None, None) == S.SFFN_OK


def test_valid_call_without_a_gpu_reports_hip_error(fake):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present; this checks the no-device path")
    assert fake.fwd() == S.SFFN_ERR_HIP


# ---------------------------------------------------------------------------
# Training entry points
# ---------------------------------------------------------------------------
TRAIN_WS = 0x7E0000000000  # never dereferenced


def test_train_workspace_bytes():
    assert S.sffn_train_workspace_bytes(S.sffn_shape(0, 100, 0, 4, 1)) == 0
    a = S.sffn_train_workspace_bytes(S.make_shape(64, 100, 0, 4, "bf16"))
    b = S.sffn_train_workspace_bytes(S.make_shape(2048, 5632, 0, 64, "bf16"))
    assert 0 < a < b and a % 256 == 0


def _train_calls(fake, mode=S.SFFN_TOPK, k=5, tau=0.5, n=2, cap=8, sv=None, ws=TRAIN_WS, wsb=None, x=0x60000,
                 y=0x70000, dy=0x90000, dx=0xA0000, dws=(0xB0000, 0xC0000, 0xD0000), w=None):
    P = ctypes.c_void_p
    if wsb is None:
        wsb = S.sffn_train_workspace_bytes(fake.sh)
    if sv is None:
        sv = S.sffn_saved(cap, 0xE0000, 0xE1000, 0xE2000, 0xE3000)
    w = w or fake.w
    f = S.lib().sffn_forward_train(P(fake.h), P(x), n, ctypes.byref(w), mode, tau, k, P(y), ctypes.byref(sv),
                                   P(ws), wsb, None)
    b = S.lib().sffn_backward(P(fake.h), P(x), P(dy), n, ctypes.byref(w), mode, tau, k, ctypes.byref(sv), P(dx),
                              P(dws[0]), P(dws[1]), P(dws[2]), P(ws), wsb, None)
    return f, b


def test_train_entry_points_reject_bad_arguments(fake):
    E, W, U = S.SFFN_ERR_INVALID_ARG, S.SFFN_ERR_WORKSPACE, S.SFFN_ERR_UNSUPPORTED
    assert _train_calls(fake, cap=4) == (E, E)              # Top-K needs cap >= k
    assert _train_calls(fake, cap=0) == (E, E)
    assert _train_calls(fake, cap=101) == (E, E)            # above d_ff
    assert _train_calls(fake, mode=S.SFFN_TOPK_2_8, cap=25) == (E, E)   # 2:8 keeps 12 x 2 + 2 = 26 of 100
    assert _train_calls(fake, mode=S.SFFN_TOPK_2_8, cap=26, n=0) == (S.SFFN_OK, S.SFFN_OK)
    assert _train_calls(fake, mode=S.SFFN_DENSE_SILU, cap=99) == (E, E)
    assert _train_calls(fake, mode=S.SFFN_THRESHOLD, tau=math.nan) == (E, E)
    assert _train_calls(fake, mode=S.SFFN_TOPP, tau=1.5) == (E, E)
    assert _train_calls(fake, mode=7) == (E, E)
    assert _train_calls(fake, mode=S.SFFN_LOPA) == (U, U)
    assert _train_calls(fake, n=9) == (E, E)
    assert _train_calls(fake, sv=S.sffn_saved(8, 0xE0000, 0, 0xE2000, 0xE3000)) == (E, E)
    assert _train_calls(fake, sv=S.sffn_saved(8, 0xE0001, 0xE1000, 0xE2000, 0xE3000)) == (E, E)
    assert _train_calls(fake, w=S.sffn_weights(None, 0x20000, 0x30000, 0x40000, 0x50000)) == (E, E)
    assert _train_calls(fake, ws=0) == (W, W)
    assert _train_calls(fake, ws=TRAIN_WS + 16) == (W, W)
    assert _train_calls(fake, wsb=S.sffn_train_workspace_bytes(fake.sh) - 1) == (W, W)
    assert _train_calls(fake, x=0x60008) == (E, E)
    assert _train_calls(fake, y=0)[0] == E
    assert _train_calls(fake, dy=0)[1] == E
    assert _train_calls(fake, dx=0xA0004)[1] == E
    assert _train_calls(fake, dws=(0xB0000, 0, 0xD0000))[1] == E
    assert _train_calls(fake, n=0) == (S.SFFN_OK, S.SFFN_OK)


def test_train_entry_points_need_bf16():
    f = _Fake(dtype="f32")
    try:
        assert _train_calls(f) == (S.SFFN_ERR_UNSUPPORTED, S.SFFN_ERR_UNSUPPORTED)
    finally:
        S.sffn_destroy(f.h)


def test_token_groups_setter_checks_its_range():
    shape = S.make_shape(64, 100, 0, 300, "bf16")
    h = S.sffn_create(shape, FAKE_WS, S.sffn_workspace_bytes(shape))
    try:
        for bad in (0, -1, 9):
            assert S.lib().sffn_set_token_groups(ctypes.c_void_p(h), bad) == S.SFFN_ERR_INVALID_ARG
        for ok in (1, 2, 8):
            assert S.lib().sffn_set_token_groups(ctypes.c_void_p(h), ok) == S.SFFN_OK
        assert S.lib().sffn_set_token_groups(None, 2) == S.SFFN_ERR_INVALID_ARG
    finally:
        S.sffn_destroy(h)
