"""Input generator checks (CPU): bf16 rounding against torch's cast, shapes, determinism."""
import numpy as np
import torch

from head_latent_attention_proj_amd import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(1 << 20).astype(np.float32),
        (rng.standard_normal(1 << 16) * 1e-30).astype(np.float32),
        # exact ties between two bf16 values, both parities
        ((np.arange(1 << 12, dtype=np.uint32) << 16) | 0x8000).view(np.float32) * np.float32(1.0),
    ])
    x = x[np.isfinite(x)]
    mine = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    back = synth.bf16_bits_to_f32(mine)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy())


def test_weight_generation_is_seeded_and_shaped():
    d = synth.Dims(hidden=256, q_lora=128, kv_lora=128, heads=2, nope=64, rope=64, v=64)
    a = synth.make_weights_bf16(d, seed=0)
    b = synth.make_weights_bf16(d, seed=0)
    for name, shape in synth.weight_shapes(d):
        assert a[name].shape == shape and a[name].dtype == np.uint16
        assert np.array_equal(a[name], b[name])
    g = synth.bf16_bits_to_f64(a["q_a_norm"])
    assert abs(g.mean() - 1.0) < 0.05
    f = synth.make_weights_fp8(d, seed=0)
    assert f["kv_a"].dtype == np.uint8 and f["kv_a_s"].shape == (2, 2)
    assert not np.any((f["q_b"] & 0x7F) == 0x7F)


def test_packed_offsets():
    offs, caps, total = synth.packed_offsets(np.array([1, 16, 17]), 16)
    assert list(caps) == [16, 16, 32] and list(offs) == [0, 16, 32] and total == 64
