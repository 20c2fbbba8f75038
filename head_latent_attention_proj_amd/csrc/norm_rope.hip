// RMSNorm + RoPE + latent cache append, per-call sequence planning, length commits, FP8
// activation quantisation.
//
// RMSNorm follows the rmsnorm excerpt on the "Key-value latent" page: float32,
// y = g * x / sqrt(mean(x^2) + eps). The normalised value is rounded once (to bf16, or to an
// E4M3FN code with its group scale in FP8 mode); the excerpt's intermediate cast to the input
// dtype before the gain is not reproduced.
// RoPE: pairs (2i, 2i+1) of the 64 rotary features turn by position * theta^(-2i/64)
// (cos/sin from a float32 table built on the host in double precision).
// The cache entry of a position is [c_hat (512) | rotated k_pe (64)] ("Key-value latent" page,
// mla-kv excerpt: the 512 + 64 split of kv_a_proj_with_mqa; the latent RMSNorm output is the
// input of kv_b, so it is what the keys and values are rebuilt from).
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "norm_dev.h"

namespace mla_k {

namespace {

__global__ void plan_kernel(const int32_t* seq_ids, const int32_t* q_start, SlotMap map, const int32_t* len, int B,
                            SeqMeta* meta) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int kbase = 0;
  for (int b = 0; b < B; ++b) {
    const int s = seq_ids[b];
    SeqMeta m;
    m.slot0 = map.table ? 0 : map.offset[s];
    m.krow0 = map.table ? kbase : m.slot0;  // block table: k_pe is read from the gathered copy
    m.l0 = len[s];
    m.q0 = q_start[b];
    m.t = q_start[b + 1] - q_start[b];
    m.kbase = kbase;
    m.seq = s;
    m.pad = 0;
    meta[b] = m;
    kbase += (m.l0 + m.t + 63) & ~63;  // rows of one sequence padded to the 64-key block
  }
}

__global__ void commit_kernel(const int32_t* seq_ids, const int32_t* q_start, int32_t* len, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) len[seq_ids[b]] += q_start[b + 1] - q_start[b];
}

// One workgroup (256 threads) per token.
template <int MAX_PARTS>
__global__ __launch_bounds__(256) void norm_rope_append_kernel(NormArgs a) {
  using namespace mla_dims;
  __shared__ float red[4];
  __shared__ float vals[KV_LORA];
  const int tok = blockIdx.x;
  const int tid = threadIdx.x;

  int64_t slot;
  int pos;
  int seq = -1;
  if (a.meta) {
    int lo = 0, hi = a.B - 1;  // last sequence whose first row is <= tok
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.meta[mid].q0 <= tok) lo = mid; else hi = mid - 1;
    }
    const SeqMeta m = a.meta[lo];
    pos = m.l0 + (tok - m.q0);
    slot = slot_of(a.map, m.seq, pos);
  } else {
    seq = a.seq_ids[tok];
    pos = a.len[seq];
    slot = slot_of(a.map, seq, pos);
  }

  const float* row = a.cqkv + (int64_t)tok * QKVA_N;
  // Every load of the token's row (all K-split parts, up to MAX_PARTS) is issued before any is
  // used: at decode this kernel is one workgroup per token and runs at load latency. The parts
  // are then added in part order.
  float pv[MAX_PARTS][9];
#pragma unroll
  for (int p = 0; p < MAX_PARTS; ++p) {
    const float* r = row + (p < a.n_part ? p : 0) * a.part_stride;
#pragma unroll
    for (int i = 0; i < 6; ++i) pv[p][i] = r[tid + i * 256];
#pragma unroll
    for (int i = 0; i < 2; ++i) pv[p][6 + i] = r[Q_LORA + tid + i * 256];
    pv[p][8] = tid < ROPE ? r[Q_LORA + KV_LORA + tid] : 0.f;
  }
  float v9[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    v9[i] = pv[0][i];
#pragma unroll
    for (int p = 1; p < MAX_PARTS; ++p)
      if (p < a.n_part) v9[i] += pv[p][i];
  }
  // ---- query latent RMSNorm (1536 = 6 per thread)
  float xq[6];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    xq[i] = v9[i];
    ss += xq[i] * xq[i];
  }
  const float rq = 1.0f / sqrtf(block_sum256(ss, red) / (float)Q_LORA + a.eps);
  // ---- kv latent RMSNorm (512 = 2 per thread)
  float xc[2];
  ss = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    xc[i] = v9[6 + i];
    ss += xc[i] * xc[i];
  }
  const float rc = 1.0f / sqrtf(block_sum256(ss, red) / (float)KV_LORA + a.eps);

  uint8_t* entry = a.cache + slot * a.entry_bytes;
  if (!a.fp8) {
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const int c = tid + i * 256;
      a.q_hat[(int64_t)tok * Q_LORA + c] = f2bf(bf2f(a.g_q[c]) * (xq[i] * rq));
    }
    uint16_t* e16 = (uint16_t*)entry;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * 256;
      e16[c] = f2bf(bf2f(a.g_kv[c]) * (xc[i] * rc));
    }
  } else {
    // q_hat: 12 groups of 128; c_hat: 4 groups. Values go through LDS so one wave owns a group.
    __shared__ float qv[Q_LORA];
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const int c = tid + i * 256;
      qv[c] = bf2f(a.g_q[c]) * (xq[i] * rq);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * 256;
      vals[c] = bf2f(a.g_kv[c]) * (xc[i] * rc);
    }
    __syncthreads();
    const int lane = tid & 63, wave = tid >> 6;
    for (int grp = wave; grp < 16; grp += 4) {
      const float* src = grp < 12 ? qv + grp * 128 : vals + (grp - 12) * 128;
      const float v0 = src[lane], v1 = src[lane + 64];
      const float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
      const float sc = amax == 0.f ? 1.0f : amax / 448.0f;
      const uint32_t c0 = e4m3_rne_sat(v0 / sc), c1 = e4m3_rne_sat(v1 / sc);
      if (grp < 12) {
        uint8_t* dst = a.q_hat_codes + (int64_t)tok * Q_LORA + grp * 128;
        dst[lane] = (uint8_t)c0;
        dst[lane + 64] = (uint8_t)c1;
        if (lane == 0) a.q_hat_scales[(int64_t)tok * (Q_LORA / 128) + grp] = sc;
      } else {
        uint8_t* dst = entry + (grp - 12) * 128;
        dst[lane] = (uint8_t)c0;
        dst[lane + 64] = (uint8_t)c1;
        if (lane == 0) ((float*)(entry + KV_LORA))[grp - 12] = sc;
      }
    }
  }
  // ---- shared rotary key: 32 pairs, rotated by this token's position (thread t < 64 holds
  // rotary feature t; pairs are exchanged through LDS)
  __shared__ float kraw[ROPE];
  if (tid < ROPE) kraw[tid] = v9[8];
  __syncthreads();
  if (tid < ROPE / 2) {
    const float k0 = kraw[2 * tid];
    const float k1 = kraw[2 * tid + 1];
    const float c = a.rope_cs[(int64_t)pos * 32 + tid];
    const float s = a.rope_cs[(int64_t)a.max_pos * 32 + (int64_t)pos * 32 + tid];
    if (a.fp8) {  // float32 rotary key: the scores it feeds stay exact to float32
      float* kpe = (float*)(entry + KV_LORA + 16);
      *(f32x2_t*)(kpe + 2 * tid) = f32x2_t{k0 * c - k1 * s, k0 * s + k1 * c};
    } else {
      uint16_t* kpe = (uint16_t*)(entry + KV_LORA * 2);
      *(uint32_t*)(kpe + 2 * tid) = pack_bf16x2(k0 * c - k1 * s, k0 * s + k1 * c);
    }
  }
  if (!a.meta) {
    __syncthreads();
    if (tid == 0) a.len[seq] = pos + 1;
  }
}

// 16 bytes per thread; entry e of the n goes to the slot of position pos0 + e.
__global__ void copy_append_kernel(uint8_t* cache, SlotMap map, const uint8_t* src, int eb, int64_t nvec, int32_t* len,
                                   int seq, int pos0, int n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nvec) {
    const int vpe = eb >> 4;  // 16-byte pieces per entry
    const int e = (int)(i / vpe), v = (int)(i - (int64_t)e * vpe);
    st16(cache + slot_of(map, seq, pos0 + e) * eb + v * 16, ld16(src + i * 16));
  }
  if (i == 0) len[seq] += n;
}

// Block-table prefill: sequence b's positions 0 .. l0 + t - 1 into rows kbase .. of dst.
// blockIdx.y = sequence of the batch; 16 bytes per thread.
__global__ void gather_kernel(const uint8_t* cache, SlotMap map, const SeqMeta* meta, int eb, uint8_t* dst) {
  const SeqMeta m = meta[blockIdx.y];
  const int vpe = eb >> 4;
  const int64_t nvec = (int64_t)(m.l0 + m.t) * vpe;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * blockDim.x) {
    const int p = (int)(i / vpe), v = (int)(i - (int64_t)p * vpe);
    st16(dst + ((int64_t)m.kbase + p) * eb + v * 16, ld16(cache + slot_of(map, m.seq, p) * eb + v * 16));
  }
}

// One wave per 128-feature group of one row.
// Dynamic FP8 activation quantiser: per row and aligned group of 128 features, s = amax / 448
// (1 when the group is all zero) and code = RNE-saturating e4m3 of v / s, both in IEEE float32.
// 16 lanes per group, 8 consecutive features per lane (one 16- or 32-byte load per operand, one
// 8-byte store of codes), 4 groups per wave; the group maximum is exact whatever the reduction
// order, so the codes do not depend on the layout.
template <typename T>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const T* x, const T* x2, int64_t ldx, int rows, int K,
                                                            uint8_t* codes, float* scales) {
  const int l16 = threadIdx.x & 15;
  const int64_t gid = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int groups = K / 128;
  if (gid >= (int64_t)rows * groups) return;  // whole 16-lane groups leave together
  const int r = (int)(gid / groups), gi = (int)(gid % groups);
  const int64_t off = (int64_t)r * ldx + gi * 128 + l16 * 8;
  float v[8];
  if constexpr (sizeof(T) == 2) {
    const u32x4_t raw = ld16(x + off);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf_lo(raw[j]);
      v[2 * j + 1] = bf_hi(raw[j]);
    }
  } else {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(x + off);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(x + off + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = a[j];
      v[4 + j] = b[j];
    }
    if (x2) {
      const f32x4_t c = *reinterpret_cast<const f32x4_t*>(x2 + off);
      const f32x4_t d = *reinterpret_cast<const f32x4_t*>(x2 + off + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] += c[j];
        v[4 + j] += d[j];
      }
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  const float sc = amax == 0.f ? 1.0f : amax / 448.0f;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    lo |= e4m3_rne_sat(v[j] / sc) << (8 * j);
    hi |= e4m3_rne_sat(v[4 + j] / sc) << (8 * j);
  }
  *reinterpret_cast<u32x2_t*>(codes + (int64_t)r * K + gi * 128 + l16 * 8) = u32x2_t{lo, hi};
  if (l16 == 0) scales[(int64_t)r * groups + gi] = sc;
}

// one thread per q_nope feature (n * 64 * 128 of them)
__global__ void split_q_nope_kernel(const float* q, int n, uint16_t* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)n * mla_dims::HEADS * mla_dims::NOPE;
  if (i >= total) return;
  const int64_t row = i >> 13;  // token (64 * 128 = 8192 features)
  const int hd = (int)(i & 8191);
  const float v = q[row * mla_dims::QB_N + (hd >> 7) * mla_dims::QK + (hd & 127)];
  const uint16_t hi = f2bf(v);
  out[i] = hi;
  out[total + i] = f2bf(v - bf2f(hi));
}

// Decoder-block input RMSNorm ("Attention input" page: the block excerpt normalises the block
// input before the attention; the rmsnorm excerpt computes in float32 and casts the normalised
// value back to the input dtype before the gain, and bf16 gain times bf16 activation is again
// bf16). One 128-thread workgroup per token, 7 16-byte chunks of the 7168 features per thread:
// y = bf16(g * bf16(x * r)), r = 1 / sqrt(mean(x^2) + eps).
__global__ __launch_bounds__(128) void input_rmsnorm_kernel(const uint16_t* x, const uint16_t* g, float eps,
                                                            uint16_t* y) {
  constexpr int K = mla_dims::HIDDEN;
  constexpr int CH = K / (128 * 8);
  static_assert(CH * 128 * 8 == K, "hidden size is a multiple of 1024");
  __shared__ float part[2];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * K;
  u32x4_t v[CH];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    v[c] = ld16(xr + (c * 128 + tid) * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = bf_lo(v[c][j]), b = bf_hi(v[c][j]);
      ss += a * a + b * b;
    }
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  const float r = 1.0f / sqrtf((part[0] + part[1]) / (float)K + eps);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int f = (c * 128 + tid) * 8;
    const u32x4_t gv = ld16(g + f);
    u32x4_t o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float t0 = bf2f(f2bf(bf_lo(v[c][j]) * r)), t1 = bf2f(f2bf(bf_hi(v[c][j]) * r));
      o[j] = pack_bf16x2(bf_lo(gv[j]) * t0, bf_hi(gv[j]) * t1);
    }
    st16(y + row * K + f, o);
  }
}

__global__ void fill_zero_kernel(int* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

hipError_t prefill_plan(const int32_t* seq_ids_d, const int32_t* q_start_d, const SlotMap& map,
                        const int32_t* len_d, int B, SeqMeta* meta, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(64), 0, s, seq_ids_d, q_start_d, map, len_d, B, meta);
  return hipGetLastError();
}

hipError_t gather_entries(const uint8_t* cache, const SlotMap& map, const SeqMeta* meta, int B, int max_rows,
                          int entry_bytes, uint8_t* dst, hipStream_t s) {
  const int64_t nvec = (int64_t)max_rows * (entry_bytes / 16);
  const unsigned gx = (unsigned)std::min<int64_t>((nvec + 255) / 256, 1024);
  hipLaunchKernelGGL(gather_kernel, dim3(gx, B), dim3(256), 0, s, cache, map, meta, entry_bytes, dst);
  return hipGetLastError();
}

hipError_t commit_lengths(const int32_t* seq_ids_d, const int32_t* q_start_d, int32_t* len_d, int B,
                          hipStream_t s) {
  hipLaunchKernelGGL(commit_kernel, dim3(cdiv(B, 256)), dim3(256), 0, s, seq_ids_d, q_start_d, len_d, B);
  return hipGetLastError();
}

hipError_t norm_rope_append(const NormArgs& a, hipStream_t s) {
  if (a.n_tokens <= 0) return hipSuccess;
  if (a.n_part < 1 || a.n_part > 8) return hipErrorInvalidValue;
  // one load per part and element, so the part capacity follows the call's part count
  if (a.n_part == 1)
    hipLaunchKernelGGL(norm_rope_append_kernel<1>, dim3(a.n_tokens), dim3(256), 0, s, a);
  else if (a.n_part <= 4)
    hipLaunchKernelGGL(norm_rope_append_kernel<4>, dim3(a.n_tokens), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(norm_rope_append_kernel<8>, dim3(a.n_tokens), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t cache_copy_append(uint8_t* cache, const SlotMap& map, const uint8_t* src, int entry_bytes, int n, int seq,
                             int pos0, int32_t* len_d, hipStream_t s) {
  const int64_t nvec = (int64_t)n * entry_bytes / 16;
  hipLaunchKernelGGL(copy_append_kernel, dim3((unsigned)((nvec + 255) / 256)), dim3(256), 0, s, cache, map, src,
                     entry_bytes, nvec, len_d, seq, pos0, n);
  return hipGetLastError();
}

hipError_t quantize_rows_f32(const float* x, const float* x2, int64_t ldx, int rows, int K, uint8_t* codes,
                             float* scales, hipStream_t s) {
  const int64_t waves = (int64_t)rows * (K / 128);
  if (waves == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_rows_kernel<float>, dim3((unsigned)((waves + 15) / 16)), dim3(256), 0, s, x, x2, ldx,
                     rows, K, codes, scales);
  return hipGetLastError();
}

hipError_t quantize_rows_bf16(const uint16_t* x, int64_t ldx, int rows, int K, uint8_t* codes, float* scales,
                              hipStream_t s) {
  const int64_t waves = (int64_t)rows * (K / 128);
  if (waves == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_rows_kernel<uint16_t>, dim3((unsigned)((waves + 15) / 16)), dim3(256), 0, s, x,
                     (const uint16_t*)nullptr, ldx, rows, K, codes, scales);
  return hipGetLastError();
}

hipError_t split_q_nope(const float* q, int n, uint16_t* out, hipStream_t s) {
  const int64_t total = (int64_t)n * mla_dims::HEADS * mla_dims::NOPE;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(split_q_nope_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, q, n, out);
  return hipGetLastError();
}

hipError_t input_rmsnorm(const uint16_t* x, const uint16_t* g, float eps, int n, uint16_t* y, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(input_rmsnorm_kernel, dim3(n), dim3(128), 0, s, x, g, eps, y);
  return hipGetLastError();
}

hipError_t fill_zero_i32(int* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace mla_k
