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
from gpu_harness import BATCHED_GUARD, compare, dev, oracle_forward, run_gpu, say

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


def _one_token_channel(ref, n):
    """A channel that exactly one token selects, outside every token's band."""
    m = ref.mask.astype(bool)
    counts = m.sum(axis=0)
    clean = ~ref.band.any(axis=0)
    cands = np.nonzero((counts == 1) & clean)[0]
    assert cands.size, "no channel selected by exactly one token"
    return int(cands[len(cands) // 2])


def _scale_down_row(lay, ch, factor=64.0):
    """A copy of the layer with W_down[ch] scaled by a power of two (exact in
    bf16; the selection does not depend on W_down)."""
    w = inputs.bf16_bits_to_f32(lay.w_down).copy()
    w[ch] *= factor
    return inputs.Layer(**{**lay.__dict__, "w_down": inputs.bf16_bits(w)})


@pytest.mark.parametrize("case", ["moc16_topk", "ragged33_threshold", "ragged100_topk", "ragged12_topk_2_8"])
def test_batched_single_token_channel_is_neither_dropped_nor_doubled(moc_layer, case):
    """The channel of the union that only one token selected has its W_down row
    scaled by 64, so it dominates that token's y: leaving its row out of the
    union gather, or counting it twice, misses the guard by a wide margin."""
    if case == "moc16_topk":
        wl = W["moc_topk_bf16_d2048_f5632"]
        lay, n, mode, kw = moc_layer, 16, "topk", dict(k=704)
        x = inputs.make_x(3, n, wl.d_model, wl.dtype)
    elif case == "ragged33_threshold":
        lay, n, mode, kw = inputs.make_layer(28, 264, 1000, "bf16"), 33, "threshold", dict(tau=1.5)
        x = inputs.make_x(28, n, 264, "bf16", correlated=True)
    elif case == "ragged100_topk":
        lay, n, mode, kw = inputs.make_layer(29, 264, 1000, "bf16"), 100, "topk", dict(k=20)
        x = inputs.make_x(29, n, 264, "bf16")
    else:
        lay, n, mode, kw = inputs.make_layer(30, 264, 1000, "bf16"), 12, "topk_2_8", {}
        x = inputs.make_x(30, n, 264, "bf16")
    say(f"case batched one-token channel x64: {case}")
    ref = oracle_forward(lay, x, mode, **kw)
    ch = _one_token_channel(ref, n)
    tok = int(np.nonzero(ref.mask[:, ch])[0][0])
    lay64 = _scale_down_row(lay, ch)
    ref64 = oracle_forward(lay64, x, mode, **kw)
    assert np.array_equal(ref64.mask, ref.mask)
    # the scaled channel carries most of that token's output
    share = float(np.abs(ref64.h[tok, ch] * inputs.bf16_bits_to_f32(lay64.w_down)[ch]).max()
                  / np.abs(ref64.y[tok]).max())
    say(f"    channel {ch} (token {tok}) share of max|y| {share:.2f}")
    assert share > 10 * BATCHED_GUARD
    got = run_gpu(lay64, x, mode, max_tokens=n, **kw)
    compare(lay64, x, mode, ref64, got)


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


@pytest.mark.parametrize("n", [9, 31, 64])
@pytest.mark.parametrize("f", [1000, 4100])
@pytest.mark.parametrize("mode,kw", [("threshold", dict(tau=2.0)), ("topk", dict(k=8)), ("topp", dict(tau=0.05)),
                                     ("threshold", dict(tau=0.0))])
def test_small_batch_union_compacted_from_every_channel(n, f, mode, kw):
    """Up to 64 tokens of a layer this small the up GEMM runs over every
    channel in the gate's launch. For the threshold and a small K the sum of
    its partials keeps the union's channels in the union's order for the down
    GEMM; top-p runs the down GEMM over every channel, its select writing the
    product rows. Unions from a few channels (high threshold, small K, small
    p) to most of them, d_ff neither a multiple of 256 nor of 32."""
    d = 512
    say(f"case small batch, union compacted from every channel bf16 d={d} F={f} n={n} {mode} {kw}")
    lay = inputs.make_layer(61, d, f, "bf16")
    x = inputs.make_x(61 + n, n, d, "bf16", correlated=True)
    ref = oracle_forward(lay, x, mode, **kw)
    got = run_gpu(lay, x, mode, max_tokens=n, **kw)
    say(f"    union {got.union} of {f}")
    compare(lay, x, mode, ref, got)


@pytest.mark.parametrize("n", [9, 40, 64])
@pytest.mark.parametrize("f", [1000, 4097, 4100])
@pytest.mark.parametrize("mode", ["topk", "topk_2_8"])
def test_small_batch_every_channel_select_writes_the_products(n, f, mode):
    """Where the union is nearly every channel (Top-K with a large K, 2:8) the
    select kernel of a small batch applies each token's gate values to the up
    GEMM's partials itself: d_ff ragged (pad columns of the product rows, rows
    not a multiple of 4) and the union size still reported."""
    d = 512
    kw = dict(k=3 * f // 8) if mode == "topk" else {}
    say(f"case small batch, every channel, products from the select bf16 d={d} F={f} n={n} {mode} {kw}")
    lay = inputs.make_layer(63, d, f, "bf16")
    x = inputs.make_x(63 + n, n, d, "bf16", correlated=True)
    ref = oracle_forward(lay, x, mode, **kw)
    got = run_gpu(lay, x, mode, max_tokens=n, **kw)
    say(f"    union {got.union} of {f}")
    compare(lay, x, mode, ref, got)


@pytest.mark.parametrize("n,d,f", [(17, 4096, 600), (40, 4096, 1000)])
@pytest.mark.parametrize("mode", ["threshold", "topk", "topk_2_8", "topp", "dense_silu"])
def test_small_batch_every_channel_many_splits(n, d, f, mode):
    """A wide d_model and a narrow d_ff split the joined gate and up GEMM K up
    to 16 ways: past 4 splits the Top-K and top-p selects leave the up half
    to its own sum kernel, while 2:8, the threshold and the dense forwards
    still take it in their own pass."""
    kw = dict(tau=1.0, k=3 * f // 8, tau_p=0.3)
    say(f"case small batch, every channel, many K splits bf16 d={d} F={f} n={n} {mode}")
    lay = inputs.make_layer(64, d, f, "bf16")
    x = inputs.make_x(64 + n, n, d, "bf16", correlated=True)
    tau = kw["tau_p"] if mode == "topp" else kw["tau"]
    ref = oracle_forward(lay, x, mode, tau=tau, k=kw["k"])
    got = run_gpu(lay, x, mode, tau=tau, k=kw["k"], max_tokens=n)
    say(f"    union {got.union} of {f}")
    compare(lay, x, mode, ref, got)


def test_small_batch_union_shrinks_on_one_handle():
    """Consecutive forwards on one handle whose unions shrink (and then grow):
    the compacted up values of a larger union left past the smaller one's
    end are never read."""
    say("case small batch, shrinking unions on one handle")
    d, f = 512, 2100
    lay = inputs.make_layer(62, d, f, "bf16")
    ffn = S.SparseFFN(d, f, 64, "bf16")
    for n, tau in ((64, 0.0), (40, 1.5), (12, 2.6), (64, 3.5), (33, 0.5)):
        x = inputs.make_x(62 + n, n, d, "bf16", correlated=True)
        ref = oracle_forward(lay, x, "threshold", tau=tau)
        got = run_gpu(lay, x, "threshold", tau=tau, ffn=ffn)
        say(f"    n={n} tau={tau} union {got.union}")
        compare(lay, x, "threshold", ref, got)


@pytest.mark.parametrize("n,f,mode,kw", [
    (2048, 8448, "dense_silu", {}),           # 33 N tiles: a whole round (32) and a rest of 1
    (2000, 8195, "dense_relu", {}),           # ragged tokens and union (pad columns in the rest)
    (2048, 8192, "dense_silu", {}),           # the union ends with the round: no rest
    (2048, 16000, "threshold", dict(tau=1.0)),
    (2048, 16000, "topk", dict(k=1500)),
    (2048, 8448, "threshold", dict(tau=1.0)),  # the gate's rest split four ways: union bits from its sum
    (2048, 8448, "topk", dict(k=1000)),        # ... and the SiLU keys
])
def test_up_gemm_whole_rounds_and_split_rest(n, f, mode, kw):
    """From 512 tokens the up GEMM's 256 x 256 tiles run in two launches: the
    N tiles of the whole rounds (on 256 CUs, 32 N tiles of 8 M tiles at 2048
    tokens), then the rest with K split so it still fills the CUs, summed in
    split order by its own pass; the gate GEMM (N = d_ff) does the same.
    Union sizes here put the end of the union in the round, one N tile past
    it, and several past it."""
    d = 128
    say(f"case up GEMM rounds + split rest bf16 d={d} F={f} n={n} {mode} {kw}")
    lay = inputs.make_layer(50, d, f, "bf16")
    x = inputs.make_x(50, n, d, "bf16", correlated=True)
    ref = oracle_forward(lay, x, mode, **kw)
    got = run_gpu(lay, x, mode, max_tokens=n, **kw)
    say(f"    union {got.union}")
    compare(lay, x, mode, ref, got)


# ---------------------------------------------------------------------------
# Token groups: each group's up and down products over its own union
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("groups", [2, 4, 8])
@pytest.mark.parametrize("mode", ["threshold", "topk", "topk_2_8", "topp"])
def test_token_groups_match_the_oracle(mode, groups):
    """Grouped forwards give the oracle's sets and y (a token's output uses
    only its own channels), and the batch's union count of the single-union
    forward; a repeated grouped forward is bit-identical."""
    d, f, n = 264, 1000, 64 * groups + 37
    say(f"case token groups bf16 d={d} F={f} n={n} {mode} groups={groups}")
    lay = inputs.make_layer(40, d, f, "bf16")
    x = inputs.make_x(40, n, d, "bf16", correlated=True)
    ref = oracle_forward(lay, x, mode, tau=1.0, k=150)
    one = run_gpu(lay, x, mode, tau=1.0, k=150, max_tokens=n)
    ffn = S.SparseFFN(d, f, n, "bf16")
    ffn.set_token_groups(groups)
    got = run_gpu(lay, x, mode, tau=1.0, k=150, ffn=ffn)
    compare(lay, x, mode, ref, got)
    assert got.union == one.union
    again = run_gpu(lay, x, mode, tau=1.0, k=150, ffn=ffn)
    assert np.array_equal(got.y.view(np.uint32), again.y.view(np.uint32))


def test_token_groups_too_few_tokens_use_one_union():
    """Below 64 tokens per group the forward keeps the single union (and
    matches the oracle either way)."""
    d, f, n = 264, 1000, 100
    lay = inputs.make_layer(41, d, f, "bf16")
    x = inputs.make_x(41, n, d, "bf16", correlated=True)
    ffn = S.SparseFFN(d, f, n, "bf16")
    ffn.set_token_groups(4)
    got = run_gpu(lay, x, "threshold", tau=1.0, ffn=ffn)
    compare(lay, x, "threshold", oracle_forward(lay, x, "threshold", tau=1.0), got)


# ---------------------------------------------------------------------------
# 70B-shaped prefill layer at full size, sampled tokens
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def prefill_layer():
    wl = W["prefill70b_ffn_bf16_d8192_f28672"]
    say("    generating the 70B-shaped layer (3 x 235M weights)")
    return inputs.make_layer(0, wl.d_model, wl.d_ff, wl.dtype)


@pytest.mark.parametrize("n,groups", [(t, 1) for t in W["prefill70b_ffn_bf16_d8192_f28672"].tokens] + [(2048, 4)])
def test_prefill70b_sampled(prefill_layer, n, groups):
    wl = W["prefill70b_ffn_bf16_d8192_f28672"]
    tau = wl.taus[0]
    d, f = wl.d_model, wl.d_ff
    say(f"case prefill70b bf16 d={d} F={f} T={n} tau={tau} groups={groups} (sampled tokens)")
    x = inputs.make_x(0, n, d, wl.dtype, correlated=True)
    lay = prefill_layer
    ffn = S.SparseFFN(d, f, n, "bf16")
    ffn.set_token_groups(groups)
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
        assert rel <= BATCHED_GUARD
