"""GPU accuracy of the two FP8 projection forms (mla_test_gemm_fp8) against float64.

The FP8 layer's projections multiply E4M3FN codes with one float32 scale per 128 x 128 weight
block and per token and 128 activation features ("Key-value latent" page, linear excerpt). The
library forms each 128-wide K group's sum in one of two ways: "precise" widens the codes exactly to
bf16 and sums them with bf16 MFMAs into float32 (q_a|kv_a, kv_b), "native" uses one FP8 MFMA per
group (q_b, o_proj). The error is measured relative to sum_k |a_k b_k| of each output element (the
natural scale of a summation error), on the layer's own weights and activations quantised by the
oracle's quantiser, with ragged M: decode-sized, and prefill-sized for the 128 x 256 tiles fed
through a ring of LDS stages (the native form from 1024 rows, the precise one from a full round of
such tiles). Bars: precise within float32 summation (1e-5), native within
1e-3; both levels are logged, since they decide which projections may take the native form.
"""
import numpy as np
import pytest

from head_latent_attention_proj_amd import binding, synth
from oracle import fp8 as ofp8

from gpu_common import log

pytestmark = pytest.mark.gpu

PRECISE_BAR = 1e-5
NATIVE_BAR = 1e-3


def deq_rows(codes, scales):
    """[R, K] codes with [R, K/128] scales -> float64 values"""
    return ofp8.dequant_1x128(codes, scales)


def weight(wq, name):
    """codes and block scales of one projection; "qkva" is q_a and kv_a stacked as the layer fuses
    them (N = 2112: the last 128-row scale block and, at 256-column tiles, the last tile partial)"""
    if name == "qkva":
        return np.vstack([wq["q_a"], wq["kv_a"]]), np.vstack([wq["q_a_s"], wq["kv_a_s"]])
    return wq[name], wq[name + "_s"]


@pytest.mark.parametrize("name,M", [("q_a", 200), ("q_b", 129), ("kv_b", 300), ("o", 96), ("q_b", 1100), ("o", 1030),
                                    ("kv_b", 1100), ("q_a", 5600), ("qkva", 200), ("qkva", 4100)])
def test_fp8_gemm_forms_against_float64(name, M):
    import torch

    wq = synth.make_weights_fp8(seed=0)
    b_codes, b_scales = weight(wq, name)
    N, K = b_codes.shape
    rng = np.random.default_rng(7100 + M)
    a_codes, a_scales = ofp8.quantize_1x128(rng.standard_normal((M, K)))
    A = deq_rows(a_codes, a_scales)
    B = ofp8.dequant_weight(b_codes, b_scales)
    ref = A @ B.T
    mag = np.abs(A) @ np.abs(B).T
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    g = binding.Gemm()
    res = {}
    for precise in (True, False):
        C = torch.empty((M, N), dtype=torch.float32, device="cuda")
        g.fp8(dev(a_codes), dev(a_scales.astype(np.float32)), dev(b_codes), dev(b_scales.astype(np.float32)), C,
              M, N, K, precise)
        torch.cuda.synchronize()
        err = np.abs(C.cpu().numpy().astype(np.float64) - ref) / mag
        res[precise] = (float(err.max()), float(np.median(err)))
    log(f"  {name} {M}x{N}x{K}: error / sum|ab|  precise max {res[True][0]:.2e} median {res[True][1]:.2e}; "
        f"native max {res[False][0]:.2e} median {res[False][1]:.2e}")
    assert res[True][0] <= PRECISE_BAR, f"precise form: {res[True][0]:.2e} of sum|ab|"
    assert res[False][0] <= NATIVE_BAR, f"native form: {res[False][0]:.2e} of sum|ab|"


def test_fp8_gemm_rejects_bad_shapes():
    import torch

    z = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    f = torch.zeros(64, dtype=torch.float32, device="cuda")
    L = binding.lib()
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    args = lambda M, N, K: (M, N, K, binding._ptr(z), binding._ptr(f), binding._ptr(z), binding._ptr(f),
                            binding._ptr(f), 1, binding._ptr(ws), ws.numel(), None)
    assert L.mla_test_gemm_fp8(*args(4, 16, 100)) == 4  # K not a multiple of 128
    assert L.mla_test_gemm_fp8(*args(4, 12, 128)) == 4  # N not a multiple of 8
    assert L.mla_test_gemm_fp8(*args(0, 16, 128)) == 1
    assert L.mla_test_gemm_fp8_workspace_bytes(4, 16, 100) == 0
