"""sffn_forward_noalloc, the forward for callers that cannot allocate: it
works in the library's static device array instead of a caller workspace.

GPU: its results equal the handle-based sffn_forward's, bit for bit (the same
kernels run), on consecutive calls where the second is smaller, and across a
change of layer shape (which clears the array's control block first).
CPU: it rejects what does not fit the array, and bad arguments, before any
HIP call."""
import ctypes

import numpy as np
import pytest
import torch

from activation_sparse_gated_gate_amd import inputs
from activation_sparse_gated_gate_amd import sffn as S

FAKE = 0x7F0000000000  # never dereferenced: validation fails first


def _status(shape, n, mode=S.SFFN_THRESHOLD, k=0, x=FAKE, y=FAKE, w=None):
    w = w or S.sffn_weights(FAKE, 0, 0, FAKE, FAKE)
    return S.lib().sffn_forward_noalloc(ctypes.byref(shape), ctypes.c_void_p(x), n, ctypes.byref(w), mode,
                                        ctypes.c_float(1.0), k, ctypes.c_void_p(y), None, None, None, None, None)


def test_rejects_what_does_not_fit_before_any_hip_call():
    big = S.make_shape(16384, 65536, 0, 8, "bf16")
    assert S.sffn_workspace_bytes(big) > S.SFFN_STATIC_SCRATCH_BYTES
    assert _status(big, 1) == S.SFFN_ERR_WORKSPACE
    assert _status(S.make_shape(4096, 11008, 0, 9, "bf16"), 1) == S.SFFN_ERR_UNSUPPORTED
    fits = S.make_shape(8192, 28672, 0, 8, "bf16")  # the 70B-shaped layer's decode fits
    assert S.sffn_workspace_bytes(fits) <= S.SFFN_STATIC_SCRATCH_BYTES
    assert _status(fits, 9) == S.SFFN_ERR_INVALID_ARG  # more tokens than the shape's maximum
    assert _status(fits, 1, x=0) == S.SFFN_ERR_INVALID_ARG
    assert _status(fits, 1, mode=S.SFFN_TOPK, k=0) == S.SFFN_ERR_INVALID_ARG
    assert _status(S.make_shape(12, 100, 0, 1, "bf16"), 1) == S.SFFN_ERR_INVALID_ARG
    assert S.lib().sffn_forward_noalloc(None, None, 1, None, 0, ctypes.c_float(0), 0, None, None, None, None,
                                        None, None) == S.SFFN_ERR_INVALID_ARG
    assert _status(fits, 0) == S.SFFN_OK  # zero tokens: nothing enqueued


def _run_both(torch, d, f, n, mode, tau=0.0, k=0, seed=0):
    """The same forward through sffn_forward (handle, caller workspace) and
    sffn_forward_noalloc; returns both results."""
    lay = inputs.make_layer(seed, d, f, "bf16")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()  # noqa: E731
    wt = [dev(lay.w_gate), dev(lay.w_up), dev(lay.w_down)]
    w = S.SparseFFN.weights(w_gate=wt[0], w_up=wt[1], w_down=wt[2])
    x = dev(inputs.make_x(seed, n, d, "bf16"))
    m = S.MODES[mode]
    out = []
    for path in ("handle", "noalloc"):
        y = torch.full((n, d), float("nan"), dtype=torch.float32, device="cuda")
        idx = torch.full((n, f), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((n,), -7, dtype=torch.int32, device="cuda")
        ucnt = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        if path == "handle":
            ffn = S.SparseFFN(d, f, 8, "bf16")
            ffn.forward(x, w, mode, y, tau=tau, k=k, active_idx=idx, active_cnt=cnt, union_cnt=ucnt)
        else:
            S.sffn_forward_noalloc(S.make_shape(d, f, 0, 8, "bf16"), x.data_ptr(), n, w, m, tau, k, y.data_ptr(),
                                   idx.data_ptr(), cnt.data_ptr(), ucnt.data_ptr(), 0, stream)
        torch.cuda.synchronize()
        out.append((y.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy(), int(ucnt.item())))
    return out


def _same(a, b):
    ya, ia, ca, ua = a
    yb, ib, cb, ub = b
    assert np.isfinite(ya).all()
    assert np.array_equal(ya.view(np.uint32), yb.view(np.uint32)), "y differs from sffn_forward's"
    assert np.array_equal(ca, cb) and ua == ub
    for t in range(ca.shape[0]):
        assert np.array_equal(ia[t, :ca[t]], ib[t, :cb[t]])


@pytest.mark.gpu
def test_noalloc_matches_the_handle_forward_on_consecutive_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("case noalloc: Llama-7B-shaped threshold, 8 tokens then 1", flush=True)
    _same(*_run_both(torch, 4096, 11008, 8, "threshold", tau=1.2816))
    _same(*_run_both(torch, 4096, 11008, 1, "threshold", tau=1.2816, seed=1))
    print("case noalloc: shape change, MoC Top-K 3 tokens, then a smaller threshold layer, 1 token", flush=True)
    _same(*_run_both(torch, 2048, 5632, 3, "topk", k=704, seed=2))
    _same(*_run_both(torch, 512, 1000, 1, "threshold", tau=0.5, seed=3))
