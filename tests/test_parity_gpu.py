"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case names itself before it touches the GPU. Workloads follow the
seeded recipe in activation_sparse_gated_gate_amd/inputs.py.
"""
import math

import numpy as np
import pytest
import torch

from activation_sparse_gated_gate_amd import inputs
from activation_sparse_gated_gate_amd import sffn as S
from gpu_harness import compare, oracle_forward, run_gpu, say

pytestmark = pytest.mark.gpu

W = inputs.WORKLOADS
# The decode kernels accumulate exact bf16 products in fp32, so their error is
# ~1e-6 of |y|; this guard sits far inside the 2e-2 contract to catch a dropped
# or doubled channel (each contributes ~1/sqrt(active) of |y|).
DECODE_GUARD = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


def _layer(wl, seed=0, rank=0):
    return inputs.make_layer(seed, wl.d_model, wl.d_ff, wl.dtype, rank=rank, with_gate=(rank == 0))


# ---------------------------------------------------------------------------
# Workload points
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n", [1, 8])
def test_tiny_fp32_threshold(n):
    wl = W["tiny_swiglu_fp32_d256_f1024"]
    say(f"case tiny fp32 d=256 F=1024 n={n} tau=1.2816 threshold")
    lay = _layer(wl)
    x = inputs.make_x(0, n, wl.d_model, wl.dtype)
    ref = oracle_forward(lay, x, "threshold", tau=1.2816)
    got = run_gpu(lay, x, "threshold", tau=1.2816)
    compare(lay, x, "threshold", ref, got)


@pytest.fixture(scope="module")
def llama_layer():
    wl = W["llama7b_ffn_bf16_d4096_f11008"]
    return _layer(wl), inputs.make_x(0, 1, wl.d_model, wl.dtype)


@pytest.mark.parametrize("tau", W["llama7b_ffn_bf16_d4096_f11008"].taus)
def test_llama7b_threshold_sweep(llama_layer, tau):
    lay, x = llama_layer
    say(f"case llama7b bf16 d=4096 F=11008 n=1 tau={tau} threshold")
    ref = oracle_forward(lay, x, "threshold", tau=tau)
    got = run_gpu(lay, x, "threshold", tau=tau)
    rep = compare(lay, x, "threshold", ref, got)
    assert rep.rel_err <= DECODE_GUARD


@pytest.mark.parametrize("rank", W["lopa_gate_bf16_d4096_f11008"].ranks)
@pytest.mark.parametrize("n", W["lopa_gate_bf16_d4096_f11008"].tokens)
def test_lopa(rank, n):
    wl = W["lopa_gate_bf16_d4096_f11008"]
    say(f"case lopa bf16 d=4096 F=11008 r={rank} n={n} tau=1.2816")
    lay = _layer(wl, rank=rank)
    x = inputs.make_x(0, n, wl.d_model, wl.dtype)
    ref = oracle_forward(lay, x, "lopa", tau=1.2816)
    got = run_gpu(lay, x, "lopa", tau=1.2816)
    rep = compare(lay, x, "lopa", ref, got)
    assert rep.rel_err <= DECODE_GUARD


@pytest.mark.parametrize("k", W["moc_topk_bf16_d2048_f5632"].ks)
def test_moc_topk_decode(k):
    wl = W["moc_topk_bf16_d2048_f5632"]
    say(f"case moc topk bf16 d=2048 F=5632 n=1 K={k}")
    lay = _layer(wl)
    x = inputs.make_x(0, 1, wl.d_model, wl.dtype)
    ref = oracle_forward(lay, x, "topk", k=k)
    got = run_gpu(lay, x, "topk", k=k)
    rep = compare(lay, x, "topk", ref, got)
    assert (got.cnt[:1] == k).all()
    assert rep.rel_err <= DECODE_GUARD


@pytest.mark.parametrize("case", ["lopa_r256", "lopa_r512", "threshold", "topk", "topp", "dense_silu"])
def test_short_gate_rows_two_tokens(case):
    """Two tokens on layers whose gate rows are at most 4 KB (LoPA's rows of
    B at ranks 256 and 512, the 2048-wide MoC layer): the gate kernel takes
    2 or 4 rows per lane group (more than two tokens ask for) and reads each
    selected up row with the whole wavefront, lane group by lane group."""
    n = 2
    if case.startswith("lopa"):
        wl = W["lopa_gate_bf16_d4096_f11008"]
        rank = int(case[len("lopa_r"):])
        lay = _layer(wl, rank=rank)
        mode, kw = "lopa", dict(tau=1.2816)
    else:
        wl = W["moc_topk_bf16_d2048_f5632"]
        lay = _layer(wl)
        mode = case
        kw = dict(tau=1.2816) if case == "threshold" else dict(k=704) if case == "topk" else \
            dict(tau=0.3) if case == "topp" else dict(tau=0.0)
    say(f"case short gate rows n={n} {case} d={wl.d_model} F={wl.d_ff}")
    x = inputs.make_x(3, n, wl.d_model, wl.dtype)
    ref = oracle_forward(lay, x, mode, **kw)
    got = run_gpu(lay, x, mode, **kw)
    rep = compare(lay, x, mode, ref, got)
    assert rep.rel_err <= DECODE_GUARD


@pytest.mark.parametrize("n", [1, 4, 8])
def test_moc_2_8_decode(n):
    """The 2:8 structured option at the MoC shape: exactly 2 of every 8
    channels per token (d_ff = 5632 is a multiple of 8)."""
    wl = W["moc_topk_bf16_d2048_f5632"]
    say(f"case moc 2:8 bf16 d=2048 F=5632 n={n}")
    lay = _layer(wl)
    x = inputs.make_x(0, n, wl.d_model, wl.dtype)
    ref = oracle_forward(lay, x, "topk_2_8")
    got = run_gpu(lay, x, "topk_2_8", max_tokens=8)
    rep = compare(lay, x, "topk_2_8", ref, got)
    assert (got.sets.reshape(n, -1, 8).sum(axis=2) == 2).all()
    assert rep.rel_err <= DECODE_GUARD


@pytest.mark.parametrize("p", [0.3, 0.5])
def test_moc_topp_decode(p):
    """Top-p at the MoC shape: p = 0.3 / 0.5 keep ~8.5 % / ~22.5 % of the
    channels of these keys."""
    wl = W["moc_topk_bf16_d2048_f5632"]
    say(f"case moc top-p bf16 d=2048 F=5632 n=1 p={p}")
    lay = _layer(wl)
    x = inputs.make_x(0, 1, wl.d_model, wl.dtype)
    ref = oracle_forward(lay, x, "topp", tau=p)
    got = run_gpu(lay, x, "topp", tau=p)
    rep = compare(lay, x, "topp", ref, got)
    assert rep.rel_err <= DECODE_GUARD


@pytest.mark.parametrize("f", [4096, 4097, 8193, 16385, 32769])
@pytest.mark.parametrize("n", [1, 3, 12])
@pytest.mark.parametrize("tied", [False, True])
def test_topp_select_sizes_and_ties(f, n, tied):
    """Every register-cache size of the top-p select (and the uncached one
    above 16384 channels), decode and batched. tied: the gate rows repeat 5
    distinct rows, so each token's keys take 5 values, each shared by about
    F/5 channels; the boundary then falls inside a large group of exact ties
    (the radix path), of which the lowest channel indices are kept."""
    d = 64
    say(f"case top-p select F={f} n={n} tied={tied}")
    lay = inputs.make_layer(33, d, f, "bf16")
    if tied:
        lay.w_gate[:] = lay.w_gate[np.arange(f) % 5]
    x = inputs.make_x(33, n, d, "bf16")
    for p in (0.2, 0.6):
        ref = oracle_forward(lay, x, "topp", tau=p)
        got = run_gpu(lay, x, "topp", tau=p, max_tokens=n)
        compare(lay, x, "topp", ref, got)
        if tied:
            for t in range(n):
                for r in range(5):
                    kept = got.sets[t, r::5]
                    assert not np.any(~kept[:-1] & kept[1:]), f"token {t}: tie kept out of index order"


@pytest.mark.parametrize("n", [1, 3, 12])
@pytest.mark.parametrize("f", [700, 20000])
def test_topp_all_keys_equal(n, f):
    """A zero token makes every key SiLU(0) = 0: equal masses, so the kept
    set is the first ceil(p d_ff) channels (ties in channel order). Token 1,
    when present, is an ordinary one."""
    d = 64
    say(f"case top-p all keys equal F={f} n={n}")
    lay = inputs.make_layer(35, d, f, "bf16")
    x = inputs.make_x(35, n, d, "bf16")
    x[0] = 0
    for p in (0.25, 0.5):
        ref = oracle_forward(lay, x, "topp", tau=p)
        got = run_gpu(lay, x, "topp", tau=p, max_tokens=n)
        compare(lay, x, "topp", ref, got)
        want = np.zeros(f, dtype=bool)
        want[:math.ceil(p * f)] = True
        assert np.array_equal(got.sets[0], want)


def test_topp_one_keeps_every_channel():
    say("case top-p p=1 == dense SiLU")
    lay = inputs.make_layer(34, 256, 700, "bf16")
    x = inputs.make_x(34, 2, 256, "bf16")
    got = run_gpu(lay, x, "topp", tau=1.0)
    assert got.sets.all()
    ref = oracle_forward(lay, x, "dense_silu")
    compare(lay, x, "dense_silu", ref, got)


@pytest.mark.parametrize("n", [1, 3, 12])
def test_2_8_ties_go_to_lower_index(n):
    """Gate rows duplicated inside a group of 8 give exactly tied keys: the
    lower channel index is kept. Ragged d_ff (a last group of 3)."""
    d, f = 64, 35
    say(f"case 2:8 exact ties n={n}")
    lay = inputs.make_layer(31, d, f, "bf16")
    for q0 in range(0, 32, 8):
        lay.w_gate[q0 + 5] = lay.w_gate[q0 + 2]
        lay.w_gate[q0 + 7] = lay.w_gate[q0 + 2]
    x = inputs.make_x(31, n, d, "bf16")
    ref = oracle_forward(lay, x, "topk_2_8")
    got = run_gpu(lay, x, "topk_2_8", max_tokens=n)
    compare(lay, x, "topk_2_8", ref, got)
    for t in range(n):
        for q0 in range(0, 32, 8):
            tied = got.sets[t, [q0 + 2, q0 + 5, q0 + 7]]
            assert not np.any(~tied[:-1] & tied[1:]), f"token {t} group {q0 // 8}: tie kept out of index order"
        assert got.sets[t, 32:].sum() == 2


# ---------------------------------------------------------------------------
# Shapes that span several tiles and ragged tails, every mode and dtype
# ---------------------------------------------------------------------------
RAGGED = [(264, 1000), (64, 37), (136, 333), (1024, 2049)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d,f", RAGGED)
@pytest.mark.parametrize("n", [1, 3, 8])
@pytest.mark.parametrize("mode", ["threshold", "topk", "topk_2_8", "topp", "dense_relu", "dense_silu"])
def test_ragged_shapes(dtype, d, f, n, mode):
    say(f"case ragged {dtype} d={d} F={f} n={n} {mode}")
    lay = inputs.make_layer(3, d, f, dtype)
    x = inputs.make_x(3, n, d, dtype)
    k = max(1, f // 5)
    ref = oracle_forward(lay, x, mode, tau=0.9, k=k)
    got = run_gpu(lay, x, mode, tau=0.9, k=k, max_tokens=8)
    rep = compare(lay, x, mode, ref, got)
    assert rep.rel_err <= (1e-5 if dtype == "f32" else DECODE_GUARD)


@pytest.mark.parametrize("f", [8193, 16385, 24600])
@pytest.mark.parametrize("n", [1, 5, 8])
@pytest.mark.parametrize("mode", ["threshold", "dense_relu"])
def test_down_channel_passes(f, n, mode):
    """The down projection lists the selected channels in passes of 12288
    channels: one, two and several passes, with ragged output pieces
    (d = 136) and every token count class."""
    d = 136
    say(f"case down passes bf16 d={d} F={f} n={n} {mode}")
    lay = inputs.make_layer(12, d, f, "bf16")
    x = inputs.make_x(12, n, d, "bf16")
    ref = oracle_forward(lay, x, mode, tau=1.0)
    got = run_gpu(lay, x, mode, tau=1.0, max_tokens=8)
    rep = compare(lay, x, mode, ref, got)
    assert rep.rel_err <= DECODE_GUARD


@pytest.mark.parametrize("f", [12289, 30000])
@pytest.mark.parametrize("n", [1, 8])
def test_down_list_overflow(f, n):
    """Every channel selected (tau below every pre-activation) on layers wider
    than one list pass: the down projection processes a full list before it
    lists the next pass."""
    d = 264
    say(f"case down list overflow bf16 d={d} F={f} n={n}")
    lay = inputs.make_layer(13, d, f, "bf16")
    x = inputs.make_x(13, n, d, "bf16")
    ref = oracle_forward(lay, x, "threshold", tau=-8.0)
    assert ref.mask.all()
    got = run_gpu(lay, x, "threshold", tau=-8.0, max_tokens=8)
    rep = compare(lay, x, "threshold", ref, got)
    assert rep.rel_err <= DECODE_GUARD


@pytest.mark.parametrize("rank", [8, 64, 264])
@pytest.mark.parametrize("n", [1, 5])
def test_lopa_ragged(rank, n):
    d, f = 520, 1001
    say(f"case lopa ragged bf16 d={d} F={f} r={rank} n={n}")
    lay = inputs.make_layer(4, d, f, "bf16", rank=rank, with_gate=False)
    x = inputs.make_x(4, n, d, "bf16")
    ref = oracle_forward(lay, x, "lopa", tau=0.5)
    got = run_gpu(lay, x, "lopa", tau=0.5, max_tokens=8)
    compare(lay, x, "lopa", ref, got)


@pytest.mark.parametrize("rank", [8, 264])
@pytest.mark.parametrize("n", [1, 3])
def test_lopa_ragged_f32(rank, n):
    d, f = 136, 333
    say(f"case lopa ragged f32 d={d} F={f} r={rank} n={n}")
    lay = inputs.make_layer(14, d, f, "f32", rank=rank, with_gate=False)
    x = inputs.make_x(14, n, d, "f32")
    ref = oracle_forward(lay, x, "lopa", tau=0.5)
    got = run_gpu(lay, x, "lopa", tau=0.5, max_tokens=8)
    compare(lay, x, "lopa", ref, got)


def test_lopa_consecutive_forwards_on_one_handle():
    """Forwards with new tokens on the same handle (token counts that shrink
    and grow) each match the oracle: nothing of t = x.A or of the selection
    carries over between forwards."""
    d, f, r = 520, 1001, 264
    lay = inputs.make_layer(15, d, f, "bf16", rank=r, with_gate=False)
    ffn = S.SparseFFN(d, f, 8, "bf16", r)
    for seed, n in ((1, 4), (2, 4), (3, 1), (4, 7)):
        say(f"case lopa consecutive seed={seed} n={n}")
        x = inputs.make_x(seed, n, d, "bf16")
        ref = oracle_forward(lay, x, "lopa", tau=0.5)
        got = run_gpu(lay, x, "lopa", tau=0.5, ffn=ffn)
        compare(lay, x, "lopa", ref, got)


# ---------------------------------------------------------------------------
# Degenerate cases of the method
# ---------------------------------------------------------------------------
def test_tau_above_every_preactivation_gives_zero():
    say("case tau above max z -> y = 0")
    lay = inputs.make_layer(5, 256, 700, "bf16")
    x = inputs.make_x(5, 2, 256, "bf16")
    got = run_gpu(lay, x, "threshold", tau=1e6)
    assert (got.cnt[:2] == 0).all() and got.union == 0
    assert np.all(got.y == 0.0)


def test_tau_below_every_preactivation_equals_dense():
    say("case tau below min z == dense")
    lay = inputs.make_layer(6, 256, 700, "bf16")
    x = inputs.make_x(6, 2, 256, "bf16")
    sp = run_gpu(lay, x, "threshold", tau=-1e6)
    de = run_gpu(lay, x, "dense_relu", tau=-1e6)
    assert sp.sets.all() and sp.union == 700
    ref = oracle_forward(lay, x, "dense_relu", tau=-1e6)
    compare(lay, x, "threshold", ref, sp)
    np.testing.assert_allclose(sp.y, de.y, rtol=1e-5, atol=1e-5 * np.abs(de.y).max())


def test_topk_all_channels_equals_swiglu():
    say("case topk K=F == dense SiLU")
    lay = inputs.make_layer(7, 512, 640, "bf16")
    x = inputs.make_x(7, 3, 512, "bf16")
    tk = run_gpu(lay, x, "topk", k=640)
    assert tk.sets.all()
    ref = oracle_forward(lay, x, "dense_silu")
    compare(lay, x, "topk", ref, tk)


def test_topk_k1_and_ties():
    say("case topk K=1 and exact ties")
    d, f = 64, 96
    lay = inputs.make_layer(8, d, f, "f32")
    # duplicate gate rows make exact ties between channels 5, 40 and 77
    lay.w_gate[40] = lay.w_gate[5]
    lay.w_gate[77] = lay.w_gate[5]
    x = inputs.make_x(8, 2, d, "f32")
    for k in (1, 2, 3):
        ref = oracle_forward(lay, x, "topk", k=k)
        got = run_gpu(lay, x, "topk", k=k)
        compare(lay, x, "topk", ref, got, tol=1e-5)


@pytest.mark.parametrize("f", [4096, 4097, 8193, 16385, 32769])
@pytest.mark.parametrize("n", [1, 3, 12])
def test_topk_select_sizes_and_tie_cut(f, n):
    """Every register-cache size of the per-token select (and the uncached one
    above 16384 channels), one token (fused select + up kernel), decode (n=3)
    and batched (n=12), with K chosen so
    that token 0's cut falls inside a group of four exactly tied channels
    spread over the channel range."""
    d = 64
    say(f"case topk select F={f} n={n} ties cut inside the tied group")
    lay = inputs.make_layer(30, d, f, "bf16")
    tied = [7, f // 3, f // 2, f - 1]
    for i in tied[1:]:
        lay.w_gate[i] = lay.w_gate[tied[0]]
    x = inputs.make_x(30, n, d, "bf16")
    z0 = oracle_forward(lay, x[:1], "dense_silu").z[0]
    key0 = z0 / (1.0 + np.exp(-z0))
    k = int((key0 > key0[tied[0]]).sum()) + 2
    ref = oracle_forward(lay, x, "topk", k=k)
    got = run_gpu(lay, x, "topk", k=k, max_tokens=n)
    compare(lay, x, "topk", ref, got)
    assert (got.cnt[:n] == k).all()
    for t in range(n):
        sel = got.sets[t, tied]
        assert not np.any(~sel[:-1] & sel[1:]), f"token {t}: tied channels kept out of index order"
    others = np.ones(f, dtype=bool)
    others[tied] = False
    if np.min(np.abs(key0[others] - key0[tied[0]])) > 1e-6:
        assert list(got.sets[0, tied]) == [True, True, False, False]


@pytest.mark.parametrize("n", [1, 2, 12])
def test_topk_select_crowded_bin(n):
    """More than 64 keys in the bin of the K-th value: 100 exactly tied
    channels at the cut, and a layer whose one huge gate row stretches the
    key range so that nearly every key shares the lowest value bin."""
    d, f = 64, 3000
    lay = inputs.make_layer(31, d, f, "bf16")
    tied = list(range(11, 3000, 29))[:100]
    for i in tied[1:]:
        lay.w_gate[i] = lay.w_gate[tied[0]]
    x = inputs.make_x(31, n, d, "bf16")
    z0 = oracle_forward(lay, x[:1], "dense_silu").z[0]
    key0 = z0 / (1.0 + np.exp(-z0))
    k = int((key0 > key0[tied[0]]).sum()) + 37
    say(f"case topk crowded bin: 100 ties, n={n} K={k}")
    ref = oracle_forward(lay, x, "topk", k=k)
    got = run_gpu(lay, x, "topk", k=k, max_tokens=n)
    compare(lay, x, "topk", ref, got)
    assert (got.cnt[:n] == k).all()
    for t in range(n):
        sel = got.sets[t, tied]
        assert not np.any(~sel[:-1] & sel[1:]), f"token {t}: tied channels kept out of index order"
    others = np.ones(f, dtype=bool)
    others[tied] = False
    if np.min(np.abs(key0[others] - key0[tied[0]])) > 1e-6:
        assert int(got.sets[0, tied].sum()) == 37

    lay = inputs.make_layer(32, d, f, "bf16")
    lay.w_gate[5] = inputs.bf16_bits(inputs.bf16_bits_to_f32(lay.w_gate[5]) * 4096.0)
    x = inputs.make_x(32, n, d, "bf16")
    say(f"case topk crowded bin: one huge gate row, n={n}")
    ref = oracle_forward(lay, x, "topk", k=400)
    got = run_gpu(lay, x, "topk", k=400, max_tokens=n)
    compare(lay, x, "topk", ref, got)
    assert (got.cnt[:n] == 400).all()

    # more than 512 equal keys at the cut, and a gate scaled so that about
    # half of the keys lie above the value-bin range (both: the radix path)
    lay = inputs.make_layer(36, d, f, "bf16")
    tied = list(range(3, f, 5))[:560]
    for i in tied[1:]:
        lay.w_gate[i] = lay.w_gate[tied[0]]
    x = inputs.make_x(36, n, d, "bf16")
    z0 = oracle_forward(lay, x[:1], "dense_silu").z[0]
    key0 = z0 / (1.0 + np.exp(-z0))
    k = int((key0 > key0[tied[0]]).sum()) + 301
    say(f"case topk crowded bin: 560 ties, n={n} K={k}")
    ref = oracle_forward(lay, x, "topk", k=k)
    got = run_gpu(lay, x, "topk", k=k, max_tokens=n)
    compare(lay, x, "topk", ref, got)
    assert (got.cnt[:n] == k).all()
    for t in range(n):
        sel = got.sets[t, tied]
        assert not np.any(~sel[:-1] & sel[1:]), f"token {t}: tied channels kept out of index order"

    lay = inputs.make_layer(37, d, f, "bf16")
    lay.w_gate[:] = inputs.bf16_bits(inputs.bf16_bits_to_f32(lay.w_gate) * 64.0)
    x = inputs.make_x(37, n, d, "bf16")
    z0 = oracle_forward(lay, x[:1], "dense_silu").z[0]
    assert (z0 / (1.0 + np.exp(-z0)) > 8.0).sum() > 1000
    say(f"case topk crowded bin: gate x64, n={n}")
    for k in (400, 1200):
        ref = oracle_forward(lay, x, "topk", k=k)
        got = run_gpu(lay, x, "topk", k=k, max_tokens=n)
        compare(lay, x, "topk", ref, got)
        assert (got.cnt[:n] == k).all()


@pytest.mark.parametrize("n", [1, 3])
@pytest.mark.parametrize("mode", ["topk", "topp"])
def test_topk_consecutive_forwards_take_their_own_boundary(n, mode):
    """Forwards in a row on one handle with a different K (or p) and input
    each time: every forward's select must use its own per-token boundary,
    never one left in the workspace by the forward before."""
    d, f = 256, 3000
    lay = inputs.make_layer(38, d, f, "bf16")
    ffn = S.SparseFFN(d, f, 8, "bf16")
    params = (37, 1500, 37, 2999, 1) if mode == "topk" else (0.05, 0.6, 0.05, 1.0, 0.3)
    for q, v in enumerate(params):
        say(f"case {mode} consecutive forwards n={n} param={v}")
        x = inputs.make_x(38 + q, n, d, "bf16")
        kw = dict(k=v) if mode == "topk" else dict(tau=v)
        ref = oracle_forward(lay, x, mode, **kw)
        got = run_gpu(lay, x, mode, ffn=ffn, **kw)
        compare(lay, x, mode, ref, got)
        if mode == "topk":
            assert (got.cnt[:n] == v).all()


@pytest.mark.parametrize("mode", ["topk", "topp"])
def test_topk_select_wait_give_up_selects_locally(mode):
    """With the poll limit at -1 no workgroup of the Top-K / top-p up kernel
    waits for the select workgroups: each runs the select itself, and the sets
    are those of a forward that waited (the down projection gives up too, so y
    is not compared). With the default limit back, the forward matches the
    oracle."""
    d, f, n = 512, 4096, 3
    kw = dict(k=500) if mode == "topk" else dict(tau=0.4)
    say(f"case {mode} select give-up d={d} F={f} n={n}")
    lay = inputs.make_layer(39, d, f, "bf16")
    x = inputs.make_x(39, n, d, "bf16")
    ffn = S.SparseFFN(d, f, n, "bf16")
    ref = oracle_forward(lay, x, mode, **kw)
    waited = run_gpu(lay, x, mode, ffn=ffn, **kw)
    compare(lay, x, mode, ref, waited)
    ffn.set_spin_limit(-1)
    local = run_gpu(lay, x, mode, ffn=ffn, **kw)
    assert np.array_equal(local.sets, waited.sets)
    ffn.set_spin_limit(1 << 18)
    got = run_gpu(lay, x, mode, ffn=ffn, **kw)
    compare(lay, x, mode, ref, got)


@pytest.mark.parametrize("n", [1, 2, 12])
def test_topk_all_keys_equal_takes_first_k(n):
    """A zero gate makes every key SiLU(0) = 0: the set is channels 0..K-1."""
    d, f, k = 64, 700, 123
    say(f"case topk all keys equal n={n}")
    lay = inputs.make_layer(33, d, f, "bf16")
    lay.w_gate[:] = 0
    x = inputs.make_x(33, n, d, "bf16")
    ref = oracle_forward(lay, x, "topk", k=k)
    got = run_gpu(lay, x, "topk", k=k, max_tokens=n)
    expect = np.zeros(f, dtype=bool)
    expect[:k] = True
    assert np.array_equal(ref.mask.astype(bool), np.tile(expect, (n, 1)))
    assert np.array_equal(got.sets, np.tile(expect, (n, 1)))
    compare(lay, x, "topk", ref, got)


def test_exact_dyadic_case_is_bit_exact():
    """Inputs on a coarse dyadic grid make every fp32 partial sum exact, so the
    GPU must equal the oracle bit for bit in any summation order."""
    say("case dyadic exact")
    rng = np.random.default_rng(9)
    d, f, n = 32, 80, 3
    grid = lambda shape: (rng.integers(-2, 3, size=shape) / 4.0).astype(np.float32)  # noqa: E731
    lay = inputs.Layer(d, f, "f32", 0, grid((f, d)), grid((f, d)), grid((f, d)))
    x = grid((n, d))
    for mode, tau in (("threshold", 0.25), ("threshold", 0.0), ("dense_relu", -1.0)):
        ref = oracle_forward(lay, x, mode, tau=tau)
        got = run_gpu(lay, x, mode, tau=tau)
        assert np.array_equal(got.sets, ref.mask.astype(bool))
        assert np.array_equal(got.y.astype(np.float64), ref.y)


def test_zero_tokens_writes_nothing():
    say("case n=0")
    ffn = S.SparseFFN(64, 100, 4, "bf16")
    wt = torch.zeros(100, 64, dtype=torch.int16, device="cuda")
    w = S.SparseFFN.weights(w_gate=wt, w_up=wt, w_down=wt)
    xy = torch.full((1, 64), 3.0, device="cuda")
    S.sffn_forward(ffn.handle, xy.data_ptr(), 0, w, S.SFFN_THRESHOLD, 0.0, 0, xy.data_ptr())
    torch.cuda.synchronize()
    assert torch.all(xy == 3.0)


def test_repeated_forwards_are_bitwise_deterministic():
    say("case determinism x20 on llama7b 90%")
    wl = W["llama7b_ffn_bf16_d4096_f11008"]
    lay = _layer(wl)
    x = inputs.make_x(0, 1, wl.d_model, wl.dtype)
    ffn = S.SparseFFN(wl.d_model, wl.d_ff, 1, "bf16")
    first = run_gpu(lay, x, "threshold", tau=1.2816, ffn=ffn)
    for _ in range(3):
        again = run_gpu(lay, x, "threshold", tau=1.2816, ffn=ffn, repeat=5)
        assert np.array_equal(first.y.view(np.uint32), again.y.view(np.uint32))
        assert np.array_equal(first.sets, again.sets)


def test_down_wait_give_up_is_reported_and_heals():
    """With the poll limit at -1 the down projection's summing workgroups give
    up at once (every kernel still exits normally): y holds NaN where they did,
    and the sticky error word in the workspace has the down-wait bit. The next
    forward with the default limit reproduces a forward from before the
    give-up bit for bit, and the word stays set until the caller clears it."""
    d, f, n = 1024, 4096, 2
    say(f"case down give-up bf16 d={d} F={f} n={n}")
    lay = inputs.make_layer(31, d, f, "bf16")
    x = torch.from_numpy(inputs.make_x(31, n, d, "bf16").view(np.int16)).cuda()
    tens = [torch.from_numpy(a.view(np.int16)).cuda() for a in (lay.w_gate, lay.w_up, lay.w_down)]
    w = S.SparseFFN.weights(w_gate=tens[0], w_up=tens[1], w_down=tens[2])
    ffn = S.SparseFFN(d, f, n, "bf16")
    off = ((ffn.workspace.data_ptr() + 255) & ~255) - ffn.workspace.data_ptr() + S.SFFN_WS_ERROR_OFFSET
    err_word = lambda: int(ffn.workspace[off:off + 4].view(torch.int32).item())  # noqa: E731
    ucnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    y0 = torch.empty(n, d, dtype=torch.float32, device="cuda")
    ffn.forward(x, w, "threshold", y0, tau=0.0, union_cnt=ucnt)
    torch.cuda.synchronize()
    assert int(ucnt.item()) > 1000  # several channel groups, so there are waits
    assert err_word() == 0 and torch.isfinite(y0).all()
    ffn.set_spin_limit(-1)
    y1 = torch.empty_like(y0)
    ffn.forward(x, w, "threshold", y1, tau=0.0)
    torch.cuda.synchronize()
    assert err_word() & S.SFFN_ERR_BIT_DOWN_WAIT
    assert torch.isnan(y1).any()
    ffn.set_spin_limit(1 << 18)
    y2 = torch.empty_like(y0)
    for _ in range(3):
        ffn.forward(x, w, "threshold", y2, tau=0.0)
        torch.cuda.synchronize()
        assert torch.equal(y2, y0)
    assert err_word() & S.SFFN_ERR_BIT_DOWN_WAIT  # sticky


def test_channel_permutation_permutes_the_set():
    say("case channel permutation")
    d, f = 256, 512
    lay = inputs.make_layer(10, d, f, "bf16")
    x = inputs.make_x(10, 2, d, "bf16")
    perm = np.random.default_rng(10).permutation(f)
    plain = run_gpu(lay, x, "threshold", tau=0.8)
    lay_p = inputs.Layer(d, f, "bf16", 0, lay.w_gate[perm], lay.w_up[perm], lay.w_down[perm])
    permd = run_gpu(lay_p, x, "threshold", tau=0.8)
    assert np.array_equal(plain.sets[:, perm], permd.sets)
    np.testing.assert_allclose(plain.y, permd.y, rtol=0, atol=1e-5 * np.abs(plain.y).max())


def test_handle_reuse_across_modes_and_batch_sizes():
    """One handle and workspace serve forwards of different modes and token
    counts back to back (the counters in the workspace reset themselves)."""
    say("case handle reuse")
    d, f = 512, 1500
    lay = inputs.make_layer(11, d, f, "bf16")
    ffn = S.SparseFFN(d, f, 8, "bf16")
    for n, mode in ((1, "threshold"), (8, "topk"), (3, "dense_relu"), (5, "threshold"), (2, "topk")):
        x = inputs.make_x(11 + n, n, d, "bf16")
        ref = oracle_forward(lay, x, mode, tau=1.0, k=100)
        got = run_gpu(lay, x, mode, tau=1.0, k=100, ffn=ffn)
        compare(lay, x, mode, ref, got)


# ---------------------------------------------------------------------------
# HIP graph capture: the forward enqueues only kernels (no allocation, no
# memset, no synchronisation), so it can be captured and replayed
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode,n", [("threshold", 1), ("topk", 3), ("topk_2_8", 1), ("topp", 2), ("lopa", 4),
                                    ("threshold", 40), ("topp", 20)])
def test_graph_replay_matches_eager(mode, n):
    """Replays of a captured forward equal the eager forward bit for bit, with
    eager forwards on other inputs between the replays."""
    d, f = 512, 1536
    say(f"case graph replay {mode} n={n}")
    rank = 64 if mode == "lopa" else 0
    lay = inputs.make_layer(40, d, f, "bf16", rank=rank, with_gate=(rank == 0))
    from gpu_harness import dev
    w = S.SparseFFN.weights(w_gate=dev(lay.w_gate), w_up=dev(lay.w_up), w_down=dev(lay.w_down),
                            lopa_a=dev(lay.lopa_a), lopa_b=dev(lay.lopa_b))
    x = dev(inputs.make_x(40, n, d, "bf16"))
    x_other = dev(inputs.make_x(41, n, d, "bf16"))
    ffn = S.SparseFFN(d, f, n, "bf16", rank)
    kw = dict(tau=0.7, k=200)
    y_eager = torch.empty(n, d, dtype=torch.float32, device="cuda")
    y_other = torch.empty_like(y_eager)
    y = torch.empty_like(y_eager)
    ffn.forward(x, w, mode, y_eager, **kw)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ffn.forward(x, w, mode, y, **kw)
    for _ in range(3):
        y.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager)
        ffn.forward(x_other, w, mode, y_other, **kw)
        torch.cuda.synchronize()
    ref = oracle_forward(lay, inputs.make_x(40, n, d, "bf16"), mode, tau=0.7, k=200)
    scale = float(np.abs(ref.y).max())
    assert float(np.abs(y.cpu().numpy() - ref.y).max()) / scale <= 2e-2
