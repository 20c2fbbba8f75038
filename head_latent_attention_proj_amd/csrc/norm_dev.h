// Device pieces of the two latent RMSNorms for a 256-thread workgroup, bf16 weights, decode.
// Used where the norms run inside the q_b projection instead of a kernel of their own; the
// arithmetic is that of norm_rope_append_kernel's bf16 path ("Key-value latent" page, rmsnorm
// excerpt: float32, y = g * x / sqrt(mean(x^2) + eps), rounded once to bf16; RoPE pairs
// (2i, 2i+1) turned by position * theta^(-2i/64)).
#pragma once

#include "common.h"
#include "kernels.h"

namespace mla_k {

// Block-wide sum over 256 threads (4 waves); `red` is 4 floats of LDS.
MLA_DEV float block_sum256(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  const float s = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return s;
}

// q_hat of decode token `tok` (the 1536 query-latent features of the fused q_a | kv_a sums,
// a.n_part parts added in part order, at most 4: bf16 weights at one or two tokens) as bf16 into
// dst[0 .. 1536).
MLA_DEV void q_norm_bf16(const NormArgs& a, int tok, uint16_t* dst, float* red) {
  using namespace mla_dims;
  const int tid = threadIdx.x;
  const float* row = a.cqkv + (int64_t)tok * QKVA_N;
  constexpr int MAX_PARTS = 4;
  float pv[MAX_PARTS][6];
#pragma unroll
  for (int p = 0; p < MAX_PARTS; ++p) {  // every load issued before any is used
    const float* r = row + (p < a.n_part ? p : 0) * a.part_stride;
#pragma unroll
    for (int i = 0; i < 6; ++i) pv[p][i] = r[tid + i * 256];
  }
  float x[6], ss = 0.f;
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    x[i] = pv[0][i];
#pragma unroll
    for (int p = 1; p < MAX_PARTS; ++p)
      if (p < a.n_part) x[i] += pv[p][i];
    ss += x[i] * x[i];
  }
  const float rq = 1.0f / sqrtf(block_sum256(ss, red) / (float)Q_LORA + a.eps);
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    const int c = tid + i * 256;
    dst[c] = f2bf(bf2f(a.g_q[c]) * (x[i] * rq));
  }
}

// Cache entry of decode token `tok` (sequence seq_ids[tok] at position len[seq]): c_hat (the
// normalised 512 latent features) and the rotated shared key, bf16; then len[seq] += 1.
// `red` is 4 floats and `kraw` 64 floats of LDS.
MLA_DEV void kv_norm_rope_append_bf16(const NormArgs& a, int tok, float* red, float* kraw) {
  using namespace mla_dims;
  const int tid = threadIdx.x;
  const int seq = a.seq_ids[tok];
  const int pos = a.len[seq];
  const int64_t slot = slot_of(a.map, seq, pos);
  const float* row = a.cqkv + (int64_t)tok * QKVA_N;
  constexpr int MAX_PARTS = 4;
  float pv[MAX_PARTS][3];
#pragma unroll
  for (int p = 0; p < MAX_PARTS; ++p) {
    const float* r = row + (p < a.n_part ? p : 0) * a.part_stride;
#pragma unroll
    for (int i = 0; i < 2; ++i) pv[p][i] = r[Q_LORA + tid + i * 256];
    pv[p][2] = tid < ROPE ? r[Q_LORA + KV_LORA + tid] : 0.f;
  }
  float v[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    v[i] = pv[0][i];
#pragma unroll
    for (int p = 1; p < MAX_PARTS; ++p)
      if (p < a.n_part) v[i] += pv[p][i];
  }
  const float rc = 1.0f / sqrtf(block_sum256(v[0] * v[0] + v[1] * v[1], red) / (float)KV_LORA + a.eps);
  uint16_t* e16 = (uint16_t*)(a.cache + slot * a.entry_bytes);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + i * 256;
    e16[c] = f2bf(bf2f(a.g_kv[c]) * (v[i] * rc));
  }
  if (tid < ROPE) kraw[tid] = v[2];
  __syncthreads();
  if (tid < ROPE / 2) {
    const float k0 = kraw[2 * tid], k1 = kraw[2 * tid + 1];
    const float c = a.rope_cs[(int64_t)pos * 32 + tid];
    const float s = a.rope_cs[(int64_t)a.max_pos * 32 + (int64_t)pos * 32 + tid];
    *(uint32_t*)(e16 + KV_LORA + 2 * tid) = pack_bf16x2(k0 * c - k1 * s, k0 * s + k1 * c);
  }
  __syncthreads();
  if (tid == 0) a.len[seq] = pos + 1;
}

}  // namespace mla_k
