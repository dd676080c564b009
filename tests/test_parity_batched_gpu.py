"""GPU parity of the batched (MFMA union) path against the CPU oracle.

Small batches are checked token by token in full. The 70B-shaped prefill
layer is checked on sampled tokens (a token's output depends on that token
only), and the union on the whole batch through properties that hold at any
size: the union size equals the size of the union of the per-token lists, and
every sampled token's oracle set (outside the band) is in it.
"""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_gated_gate_amd import inputs
from activation_sparse_gated_gate_amd import sffn as S
from gpu_harness import TOL, compare, dev, oracle_forward, run_gpu, say

pytestmark = pytest.mark.gpu
W = inputs.WORKLOADS


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


# ---------------------------------------------------------------------------
# Mixture-of-Channels Top-K, batched decode (16 and 64 tokens)
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def moc_layer():
    wl = W["moc_topk_bf16_d2048_f5632"]
    return inputs.make_layer(0, wl.d_model, wl.d_ff, wl.dtype)


@pytest.mark.parametrize("k", W["moc_topk_bf16_d2048_f5632"].ks)
@pytest.mark.parametrize("n", [16, 64])
def test_moc_topk_batched(moc_layer, n, k):
    wl = W["moc_topk_bf16_d2048_f5632"]
    say(f"case moc topk batched bf16 d=2048 F=5632 n={n} K={k}")
    x = inputs.make_x(0, n, wl.d_model, wl.dtype)
    ref = oracle_forward(moc_layer, x, "topk", k=k)
    got = run_gpu(moc_layer, x, "topk", k=k)
    rep = compare(moc_layer, x, "topk", ref, got)
    assert (got.cnt[:n] == k).all()
    say(f"    union fraction {rep.union / wl.d_ff:.3f}")


@pytest.mark.parametrize("n", [16, 64])
def test_moc_2_8_batched(moc_layer, n):
    wl = W["moc_topk_bf16_d2048_f5632"]
    say(f"case moc 2:8 batched bf16 d=2048 F=5632 n={n}")
    x = inputs.make_x(0, n, wl.d_model, wl.dtype)
    ref = oracle_forward(moc_layer, x, "topk_2_8")
    got = run_gpu(moc_layer, x, "topk_2_8")
    rep = compare(moc_layer, x, "topk_2_8", ref, got)
    assert (got.sets.reshape(n, -1, 8).sum(axis=2) == 2).all()
    say(f"    union fraction {rep.union / wl.d_ff:.3f}")


@pytest.mark.parametrize("n", [16, 64])
def test_moc_topp_batched(moc_layer, n):
    wl = W["moc_topk_bf16_d2048_f5632"]
    say(f"case moc top-p batched bf16 d=2048 F=5632 n={n} p=0.5")
    x = inputs.make_x(0, n, wl.d_model, wl.dtype)
    ref = oracle_forward(moc_layer, x, "topp", tau=0.5)
    got = run_gpu(moc_layer, x, "topp", tau=0.5)
    rep = compare(moc_layer, x, "topp", ref, got)
    say(f"    union fraction {rep.union / wl.d_ff:.3f}")


# ---------------------------------------------------------------------------
# Ragged batches through every tile configuration and mode
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n", [9, 33, 100, 300, 600])
@pytest.mark.parametrize("mode", ["threshold", "topk", "topk_2_8", "topp", "dense_relu", "dense_silu"])
def test_batched_ragged(n, mode):
    d, f = 264, 1000
    say(f"case batched ragged bf16 d={d} F={f} n={n} {mode}")
    lay = inputs.make_layer(21, d, f, "bf16")
    x = inputs.make_x(21, n, d, "bf16", correlated=True)
    ref = oracle_forward(lay, x, mode, tau=1.0, k=150)
    got = run_gpu(lay, x, mode, tau=1.0, k=150, max_tokens=n)
    compare(lay, x, mode, ref, got)


@pytest.mark.parametrize("n,d,f", [(48, 1024, 2049), (520, 512, 777), (17, 4096, 600)])
def test_batched_threshold_shapes(n, d, f):
    say(f"case batched threshold bf16 d={d} F={f} n={n}")
    lay = inputs.make_layer(22, d, f, "bf16")
    x = inputs.make_x(22, n, d, "bf16", correlated=True)
    ref = oracle_forward(lay, x, "threshold", tau=1.2816)
    got = run_gpu(lay, x, "threshold", tau=1.2816, max_tokens=n)
    compare(lay, x, "threshold", ref, got)


def test_batched_no_active_channel_gives_zero():
    say("case batched tau above every z")
    lay = inputs.make_layer(23, 256, 300, "bf16")
    x = inputs.make_x(23, 40, 256, "bf16")
    got = run_gpu(lay, x, "threshold", tau=1e6)
    assert got.union == 0 and (got.cnt[:40] == 0).all()
    assert np.all(got.y == 0.0)


def test_batched_tau_below_every_z_equals_dense():
    say("case batched tau below every z == dense")
    lay = inputs.make_layer(24, 256, 300, "bf16")
    x = inputs.make_x(24, 40, 256, "bf16")
    sp = run_gpu(lay, x, "threshold", tau=-1e6)
    ref = oracle_forward(lay, x, "dense_relu", tau=-1e6)
    assert sp.sets.all() and sp.union == 300
    compare(lay, x, "threshold", ref, sp)


def test_batched_repeat_is_deterministic():
    say("case batched determinism")
    lay = inputs.make_layer(25, 512, 1500, "bf16")
    x = inputs.make_x(25, 100, 512, "bf16", correlated=True)
    ffn = S.SparseFFN(512, 1500, 100, "bf16")
    a = run_gpu(lay, x, "threshold", tau=1.0, ffn=ffn)
    b = run_gpu(lay, x, "threshold", tau=1.0, ffn=ffn, repeat=3)
    assert np.array_equal(a.y.view(np.uint32), b.y.view(np.uint32))
    assert np.array_equal(a.sets, b.sets)


def test_batched_handle_mixes_decode_and_batched_forwards():
    say("case handle serving decode and batched forwards")
    d, f = 512, 1200
    lay = inputs.make_layer(26, d, f, "bf16")
    ffn = S.SparseFFN(d, f, 64, "bf16")
    for n, mode in ((64, "threshold"), (1, "threshold"), (20, "topk"), (5, "topk"), (64, "dense_silu"), (30, "threshold")):
        x = inputs.make_x(26 + n, n, d, "bf16", correlated=True)
        ref = oracle_forward(lay, x, mode, tau=1.0, k=100)
        got = run_gpu(lay, x, mode, tau=1.0, k=100, ffn=ffn)
        compare(lay, x, mode, ref, got)


def test_batched_handle_larger_than_batch_splits_within_its_buffer():
    # A handle sized for 600 tokens serves smaller batches, whose GEMMs split
    # K (up to 16 ways at 64 tokens and below, 8 below 512, and the two-way
    # split gate from 256): every split must fit the handle's partial buffer.
    say("case handle of 600 tokens serving 12..511-token batches")
    d, f = 1024, 1500
    lay = inputs.make_layer(27, d, f, "bf16")
    ffn = S.SparseFFN(d, f, 600, "bf16")
    for n, mode in ((12, "topk"), (64, "threshold"), (100, "dense_silu"), (300, "threshold"), (511, "topk")):
        x = inputs.make_x(27 + n, n, d, "bf16", correlated=True)
        ref = oracle_forward(lay, x, mode, tau=1.0, k=200)
        got = run_gpu(lay, x, mode, tau=1.0, k=200, ffn=ffn)
        compare(lay, x, mode, ref, got)


# ---------------------------------------------------------------------------
# 70B-shaped prefill layer at full size, sampled tokens
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def prefill_layer():
    wl = W["prefill70b_ffn_bf16_d8192_f28672"]
    say("    generating the 70B-shaped layer (3 x 235M weights)")
    return inputs.make_layer(0, wl.d_model, wl.d_ff, wl.dtype)


@pytest.mark.parametrize("n", W["prefill70b_ffn_bf16_d8192_f28672"].tokens)
def test_prefill70b_sampled(prefill_layer, n):
    wl = W["prefill70b_ffn_bf16_d8192_f28672"]
    tau = wl.taus[0]
    d, f = wl.d_model, wl.d_ff
    say(f"case prefill70b bf16 d={d} F={f} T={n} tau={tau} (sampled tokens)")
    x = inputs.make_x(0, n, d, wl.dtype, correlated=True)
    lay = prefill_layer
    ffn = S.SparseFFN(d, f, n, "bf16")
    w = S.SparseFFN.weights(w_gate=dev(lay.w_gate), w_up=dev(lay.w_up), w_down=dev(lay.w_down))
    xt = dev(x)
    y = torch.full((n, d), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((n, f), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(n, dtype=torch.int32, device="cuda")
    ucnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    ffn.forward(xt, w, "threshold", y, tau=tau, active_idx=idx, active_cnt=cnt, union_cnt=ucnt)
    torch.cuda.synchronize()
    # union over the whole batch from the per-token lists, on the device
    mask = torch.zeros(n, f + 1, dtype=torch.bool, device="cuda")
    pos = torch.arange(f, device="cuda")[None, :] < cnt[:, None]
    mask.scatter_(1, torch.where(pos, idx, torch.full_like(idx, f)).long(), True)
    un = mask[:, :f].any(dim=0)
    assert int(ucnt.item()) == int(un.sum().item())
    frac = un.float().mean().item()
    say(f"    union fraction {frac:.3f}, mean active/token {cnt.float().mean().item():.1f}")
    assert 0.2 < frac < 0.7
    # sampled tokens against the oracle
    samples = sorted({0, 1, n // 3, n // 2, n - 2, n - 1})
    y_h, idx_h, cnt_h = y.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
    un_h = un.cpu().numpy()
    for t in samples:
        xs = x[t:t + 1]
        ref = oracle.forward("threshold", xs, lay.w_up, lay.w_down, w_gate=lay.w_gate, tau=tau)
        gset = np.zeros(f, dtype=bool)
        row = idx_h[t, :cnt_h[t]]
        assert np.all(np.diff(row) > 0)
        gset[row] = True
        oset = ref.mask[0].astype(bool)
        assert not ((gset ^ oset) & ~ref.band[0]).any()
        assert not (oset & ~ref.band[0] & ~un_h).any()
        if (gset ^ oset).any():
            y_ref = oracle.forward_with_mask(xs, lay.w_up, lay.w_down, ref.g, gset[None].astype(np.uint8))[0]
        else:
            y_ref = ref.y[0]
        rel = float(np.abs(y_h[t] - y_ref).max() / np.abs(y_ref).max())
        say(f"    token {t}: active {cnt_h[t]} band {int(ref.band.sum())} y_rel_err {rel:.2e}")
        assert rel <= TOL["bf16"]
