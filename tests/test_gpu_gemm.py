"""GPU parity of the projection kernel (mla_test_gemm) against float64 matmul of the same bf16 bits.

Covers the skinny (decode-sized M) and tile (prefill-sized M) kernels, split-K with its
fixed-order reduction kernel, batched per-head products with strides, and ragged M/N tails.
"""
import numpy as np
import pytest

from head_latent_attention_proj_amd import binding, synth
from oracle import mla as omla

from gpu_common import log

pytestmark = pytest.mark.gpu


def bf16_rand(shape, seed, std=1.0):
    rng = np.random.default_rng(seed)
    return synth.f32_to_bf16_bits(rng.normal(0, std, size=shape).astype(np.float32))


@pytest.mark.parametrize("M,N,K", [
    (1, 2112, 7168), (1, 7168, 8192), (2, 7168, 8192), (1, 12288, 1536), (2, 2112, 7168),
    (1, 1100, 1536), (2, 1100, 640), (1, 20, 128), (3, 12288, 1536), (16, 7168, 8192), (17, 2112, 7168),
    (33, 16384, 512), (64, 7168, 8192), (65, 2112, 7168), (100, 12288, 1536), (128, 7168, 8192),
    (300, 16384, 512), (1000, 2112, 7168), (1024, 1100, 1536), (2048, 7168, 8192),
    # LDS-ring kernel (16 < M <= 64, K >= 1024): 64- and 128-column tiles, K splits, ragged N
    (48, 12288, 1536), (32, 2112, 7168), (64, 16384, 1024), (20, 1100, 1024), (40, 7100, 8192),
])
def test_gemm_matches_float64(M, N, K):
    import torch

    log(f"gemm M={M} N={N} K={K}")
    a = bf16_rand((M, K), 1 + M)
    b = bf16_rand((N, K), 2 + N, std=0.02)
    A, B = binding.bf16_tensor(a), binding.bf16_tensor(b)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    binding.Gemm()(A, B, C, M, N, K)
    torch.cuda.synchronize()
    ref = omla.linear(synth.bf16_bits_to_f64(a), synth.bf16_bits_to_f64(b))
    got = C.cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    scale = np.sqrt(K) * 0.02  # typical |ref|
    log(f"  max err {err.max():.3e} (scale {scale:.3f})")
    assert np.all(np.isfinite(got))
    assert err.max() <= 2e-5 * scale * 8


@pytest.mark.parametrize("M,N,K", [
    # bf16 outputs of the tile kernels: 128 x 128 and 256 x 256 tiles with ragged M (the LDS-staged
    # row-chunk epilogue), N not a multiple of 8 (the per-value epilogue), and a split-K product
    # (the reduction's epilogue)
    (2100, 4096, 512), (4100, 8192, 128), (2100, 4100, 256), (200, 1536, 512),
])
def test_gemm_bf16_output_matches_float64(M, N, K):
    import torch

    log(f"gemm bf16 out M={M} N={N} K={K}")
    a = bf16_rand((M, K), 3 + M)
    b = bf16_rand((N, K), 4 + N, std=0.02)
    A, B = binding.bf16_tensor(a), binding.bf16_tensor(b)
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    binding.Gemm()(A, B, C, M, N, K)
    torch.cuda.synchronize()
    ref = omla.linear(synth.bf16_bits_to_f64(a), synth.bf16_bits_to_f64(b))
    got = C.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))  # every element written
    # bf16 rounding of the float32 sum: half a unit in the last place, plus the float32 sum's error
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6 * np.sqrt(K))


@pytest.mark.parametrize("Bt", [1, 2, 5, 33, 64, 100, 256])
def test_gemm_bf16_output_and_batched_strides(Bt):
    """Per-head batched product with row/batch strides (the decode absorption layout); above 64
    rows the per-head kernel runs in 64-row chunks (100: a ragged last chunk)."""
    import torch

    log(f"batched gemm Bt={Bt}")
    H = 64
    q = bf16_rand((Bt, H * 192), 11)
    w = bf16_rand((H, 512, 128), 12, std=0.05)
    Q, W = binding.bf16_tensor(q), binding.bf16_tensor(w)
    out = torch.empty((Bt, H, 512), dtype=torch.bfloat16, device="cuda")
    binding.Gemm()(Q, W, out, Bt, 512, 128, batch=H, lda=H * 192, sA=192, ldb=128, sB=512 * 128,
                   ldc=H * 512, sC=512, stage="absorb")
    torch.cuda.synchronize()
    got = synth.bf16_bits_to_f64(binding.tensor_to_bf16_bits(out))
    q64 = synth.bf16_bits_to_f64(q).reshape(Bt, H, 192)[:, :, :128]
    ref = np.einsum("bhd,hcd->bhc", q64, synth.bf16_bits_to_f64(w))
    err = np.abs(got - ref)
    assert err.max() <= 2 ** -8 * np.abs(ref).max() + 1e-6


@pytest.mark.parametrize("Bt", [1, 2, 20, 64, 200, 256])
def test_gemm_value_mix_layout(Bt):
    """Per-head W_UV product: o[b][h*128 + d] = sum_c o_lat[b][h][c] W_UV,h[d][c] (K = 512)."""
    import torch

    log(f"value-mix gemm Bt={Bt}")
    H = 64
    ol = bf16_rand((Bt, H * 512), 21)
    w = bf16_rand((H, 256, 512), 22, std=0.05)  # per head [128 key rows | 128 value rows]
    OL, W = binding.bf16_tensor(ol), binding.bf16_tensor(w)
    out = torch.empty((Bt, H * 128), dtype=torch.float32, device="cuda")
    binding.Gemm()(OL, W[:, 128:, :], out, Bt, 128, 512, batch=H, lda=H * 512, sA=512, ldb=512, sB=256 * 512,
                   ldc=H * 128, sC=128, stage="uv")
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = np.einsum("bhc,hdc->bhd", synth.bf16_bits_to_f64(ol).reshape(Bt, H, 512),
                    synth.bf16_bits_to_f64(w)[:, 128:, :]).reshape(Bt, H * 128)
    err = np.abs(got - ref)
    log(f"  max err {err.max():.3e}")
    assert err.max() <= 2e-5 * np.abs(ref).max()


def test_gemm_rejects_bad_shapes():
    import torch

    A = torch.zeros((4, 130), dtype=torch.bfloat16, device="cuda")
    C = torch.zeros((4, 4), dtype=torch.float32, device="cuda")
    with pytest.raises(binding.MlaError):
        binding.Gemm()(A, A, C, 4, 4, 130)
