"""Seeded generators: determinism, rounding and workload shapes (no GPU)."""
import numpy as np
import torch

from activation_sparse_gated_gate_amd import inputs


def test_same_seed_same_bytes():
    a = inputs.make_layer(0, 64, 96, inputs.BF16, rank=8)
    b = inputs.make_layer(0, 64, 96, inputs.BF16, rank=8)
    for name in ("w_gate", "w_up", "w_down", "lopa_a", "lopa_b"):
        assert getattr(a, name).tobytes() == getattr(b, name).tobytes()
    c = inputs.make_layer(1, 64, 96, inputs.BF16)
    assert a.w_up.tobytes() != c.w_up.tobytes()


def test_tensors_draw_independent_streams():
    lay = inputs.make_layer(0, 64, 64, inputs.F32)
    assert not np.array_equal(lay.w_gate, lay.w_up)


def test_first_token_does_not_depend_on_batch():
    x1 = inputs.make_x(0, 1, 128, inputs.BF16)
    x8 = inputs.make_x(0, 8, 128, inputs.BF16)
    assert np.array_equal(x1[0], x8[0])


def test_bf16_rounding_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0], np.float32)])
    ours = inputs.bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = inputs.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_weight_scales():
    lay = inputs.make_layer(0, 1024, 2048, inputs.F32)
    assert abs(lay.w_gate.std() * np.sqrt(1024) - 1) < 0.01
    assert abs(lay.w_down.std() * np.sqrt(2048) - 1) < 0.01


def test_correlated_tokens_keep_unit_variance_and_share_a_component():
    x = inputs.make_x(0, 64, 4096, inputs.F32, correlated=True)
    assert abs(x.std() - 1.0) < 0.02
    c = np.corrcoef(x[0], x[1])[0, 1]
    assert abs(c - 0.49 / 0.58) < 0.05


def test_workload_table():
    w = inputs.WORKLOADS
    assert w["llama7b_ffn_bf16_d4096_f11008"].taus == (0.0, 0.674, 1.2816, 1.645, 2.326)
    assert w["moc_topk_bf16_d2048_f5632"].ks == (5632 // 8, 5632 // 4)
    assert w["prefill70b_ffn_bf16_d8192_f28672"].correlated
