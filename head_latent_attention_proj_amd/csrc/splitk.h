// Fixed-order sum of split-K float32 partials, four output columns per thread, for the projection
// kernels of both weight formats (included by gemm.hip and gemm_fp8.hip).
#pragma once

#include "common.h"
#include "kernels.h"

namespace mla_k {
namespace {

// part[b][split][M][N] summed in split order, then (CSCALE: times the output scale of the row's
// 128-column block, c_scale[b * cs_stride + n / 128]) stored as float32 or as bf16 after adding the
// residual. 16-byte loads of every part, one vector store; rows and pointers as reduce_vec_ok requires.
template <int TAG, bool CSCALE>
__global__ __launch_bounds__(256) void splitk_reduce_vec_kernel(GemmArgs p, int splits) {
  const int64_t mn = (int64_t)p.M * p.N;
  const int64_t idx = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  const int b = blockIdx.y;
  if (idx >= mn) return;
  const float* base = p.part + (int64_t)b * splits * mn + idx;
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < splits; ++sp) s += *reinterpret_cast<const f32x4_t*>(base + sp * mn);
  const int m = (int)(idx / p.N), n = (int)(idx % p.N);
  if constexpr (CSCALE) {
    if (p.c_scale) s *= p.c_scale[b * p.cs_stride + (n >> 7)];
  }
  const int64_t ci = b * p.sC + (int64_t)m * p.ldc + n;
  if (p.epi == EPI_F32) {
    *reinterpret_cast<f32x4_t*>((float*)p.C + ci) = s;
  } else {
    if (p.resid) {
      const u32x2_t r = *reinterpret_cast<const u32x2_t*>(p.resid + (int64_t)m * p.ldr + n);
      s[0] += __uint_as_float(r[0] << 16);
      s[1] += __uint_as_float(r[0] & 0xffff0000u);
      s[2] += __uint_as_float(r[1] << 16);
      s[3] += __uint_as_float(r[1] & 0xffff0000u);
    }
    *reinterpret_cast<u32x2_t*>((uint16_t*)p.C + ci) = u32x2_t{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
  }
}

// float32 (16-byte aligned C) or bf16 (8-byte aligned C and residual) output, N, ldc, sC (and ldr)
// multiples of 4
bool reduce_vec_ok(const GemmArgs& a) {
  auto al = [](const void* q, uintptr_t n) { return (reinterpret_cast<uintptr_t>(q) & (n - 1)) == 0; };
  if ((a.N & 3) || (a.ldc & 3) || (a.sC & 3)) return false;
  if (a.epi == EPI_F32) return al(a.C, 16);
  if (a.epi == EPI_BF16) return al(a.C, 8) && (!a.resid || (al(a.resid, 8) && (a.ldr & 3) == 0));
  return false;
}

}  // namespace
}  // namespace mla_k
