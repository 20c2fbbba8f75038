// FP8 (OCP E4M3FN, 128x128 block-scaled weights, 1x128 dynamic activations) GEMM.
// Placeholder entry until the FP8 kernels land: reports "not supported".
#include "common.h"
#include "kernels.h"

namespace mla_k {
hipError_t gemm_fp8(const GemmArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace mla_k
