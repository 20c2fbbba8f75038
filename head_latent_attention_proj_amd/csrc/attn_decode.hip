// Decode attention in the 512-feature latent space, split over positions, then merged.
//
// For one new token of a sequence holding L positions (this step's entry included), head h:
//   s_j = scale * ( q_lat_h . c_hat_j + RoPE(q_pe_h) . k_pe_j ),  j = 0 .. L-1
//   o_lat_h = sum_j softmax(s)_j c_hat_j                            (512 features)
// with q_lat_h = W_UK,h^T q_nope_h. This equals the pages' scores q.k over 192 features and the
// value mix sum_j a_j v_j once W_UV,h is applied to o_lat_h afterwards (W_UK / W_UV are output
// features 0..127 / 128..255 of each head's 256 in kv_b: "Key content up-projection" page,
// Explanation). The cache therefore streams 1,152 bytes per position for all 64 heads at once
// instead of 64 x (192 + 128) rebuilt features ("KV cache" page: 20,480 vs 576 values).
//
// Work layout: one workgroup = (sequence, split of `chunk` positions), 8 waves = 4 head groups
// of 16 x 2 latent halves of 256. Heads are the MFMA column dimension, so one 64-position block
// staged in LDS feeds every head: S^T = C Q^T (A = cache rows, B = queries), then
// O^T = C^T P^T with the latent part also written transposed into LDS during staging. Each
// split writes (max, sum, unnormalised o) per head; the merge kernel combines the splits.
#include "common.h"
#include "kernels.h"

namespace mla_k {

namespace {

constexpr int DKB = 64;   // positions per block
constexpr int LDC = 584;  // sC row: 576 features + pad (1168 B)
constexpr int LDT = 68;   // sT row: 64 positions + pad (136 B)
constexpr float LOG2E = 1.4426950408889634f;

MLA_DEV u32x2_t ld8(const void* p) { return *reinterpret_cast<const u32x2_t*>(p); }

__global__ __launch_bounds__(512, 1) void decode_attn_kernel(DecodeAttnArgs a) {
  using namespace mla_dims;
  const int split = blockIdx.x, b = blockIdx.y;
  const int seq = a.seq_ids[b];
  const int L = a.len[seq];
  const int c0 = split * a.chunk;
  if (c0 >= L) return;
  const int c1 = min(L, c0 + a.chunk);
  const int64_t slot0 = a.offset[seq];
  const int nblk = cdiv(c1 - c0, DKB);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int hg = wave & 3, lh = wave >> 2;  // head group (16 heads), latent half (256 features)
  const int head = hg * 16 + l16;

  __shared__ __attribute__((aligned(16))) uint16_t sC[DKB * LDC];
  __shared__ __attribute__((aligned(16))) uint16_t sT[KV_LORA * LDT];

  // ---- query fragments (B operand): column = head, features ks*32 + g*8 .. +7
  bf16x8_t qf[18];
  {
    const uint16_t* ql = a.q_lat + ((int64_t)b * 64 + head) * KV_LORA;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qf[ks] = as_bf16x8(ld16(ql + ks * 32 + g * 8));
    const uint16_t* qp = a.q + ((int64_t)b * 64 + head) * QK + NOPE;
    const int pos = L - 1;
#pragma unroll
    for (int ks = 16; ks < 18; ++ks) {
      const u32x4_t raw = ld16(qp + (ks - 16) * 32 + g * 8);
      const int pair0 = ((ks - 16) * 32 + g * 8) >> 1;
      u32x4_t rot;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x0 = bf_lo(raw[j]), x1 = bf_hi(raw[j]);
        const float c = a.rope_cs[(int64_t)pos * 32 + pair0 + j];
        const float s = a.rope_cs[(int64_t)a.max_pos * 32 + (int64_t)pos * 32 + pair0 + j];
        rot[j] = pack_bf16x2(x0 * c - x1 * s, x0 * s + x1 * c);
      }
      qf[ks] = as_bf16x8(rot);
    }
  }

  // ---- staging: latent part as key pairs (row-major copy + transposed copy), k_pe row-major
  // item i: key pair kp = (lane & 15) + 16*(i & 1), 16-byte chunk ch = (lane >> 4) + 4*(wave + 8*(i >> 1))
  u32x4_t rl[4][2], rp;
  auto gload = [&](int blk) {
    const int kb = c0 + blk * DKB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kp = (lane & 15) + 16 * (i & 1);
      const int ch = (lane >> 4) + 4 * (wave + 8 * (i >> 1));
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int key = min(kb + 2 * kp + u, c1 - 1);
        rl[i][u] = ld16(a.cache + (slot0 + key) * a.entry_bytes + ch * 16);
      }
    }
    const int key = min(kb + (tid >> 3), c1 - 1);
    rp = ld16(a.cache + (slot0 + key) * a.entry_bytes + KV_LORA * 2 + (tid & 7) * 16);
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kp = (lane & 15) + 16 * (i & 1);
      const int ch = (lane >> 4) + 4 * (wave + 8 * (i >> 1));
      st16(sC + (2 * kp) * LDC + ch * 8, rl[i][0]);
      st16(sC + (2 * kp + 1) * LDC + ch * 8, rl[i][1]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t x = rl[i][0][j], y = rl[i][1][j];
        // features ch*8 + 2j (low halves) and ch*8 + 2j + 1 (high halves), keys 2kp, 2kp+1
        *reinterpret_cast<uint32_t*>(sT + (ch * 8 + 2 * j) * LDT + 2 * kp) = (x & 0xffffu) | (y << 16);
        *reinterpret_cast<uint32_t*>(sT + (ch * 8 + 2 * j + 1) * LDT + 2 * kp) = (x >> 16) | (y & 0xffff0000u);
      }
    }
    st16(sC + (tid >> 3) * LDC + KV_LORA + (tid & 7) * 8, rp);
  };

  const float sl2 = a.scale * LOG2E;
  float mrun = -INFINITY, lrun = 0.f;
  f32x4_t oacc[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) oacc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  gload(0);
  for (int blk = 0; blk < nblk; ++blk) {
    __syncthreads();
    sstore();
    __syncthreads();
    if (blk + 1 < nblk) gload(blk + 1);
    const int kb = c0 + blk * DKB;

    f32x4_t sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) sacc[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const bf16x8_t kf = as_bf16x8(ld16(sC + (kt * 16 + l16) * LDC + ks * 32 + g * 8));
        sacc[kt] = mfma_bf16_16x16x32(kf, qf[ks], sacc[kt]);
      }
    }
    float bmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float s = sacc[kt][e] * sl2;
        if (kb + kt * 16 + g * 4 + e >= c1) s = -INFINITY;
        sacc[kt][e] = s;
        bmax = fmaxf(bmax, s);
      }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    const float mnew = fmaxf(mrun, bmax);
    const float alpha = exp2f(mrun - mnew);
    mrun = mnew;
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = exp2f(sacc[kt][e] - mnew);
        sacc[kt][e] = p;
        psum += p;
      }
    lrun = lrun * alpha + psum;
#pragma unroll
    for (int c = 0; c < 16; ++c) oacc[c] *= alpha;
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      u32x4_t w;
      w[0] = pack_bf16x2(sacc[2 * ps][0], sacc[2 * ps][1]);
      w[1] = pack_bf16x2(sacc[2 * ps][2], sacc[2 * ps][3]);
      w[2] = pack_bf16x2(sacc[2 * ps + 1][0], sacc[2 * ps + 1][1]);
      w[3] = pack_bf16x2(sacc[2 * ps + 1][2], sacc[2 * ps + 1][3]);
      const bf16x8_t pf = as_bf16x8(w);
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const uint16_t* tp = sT + (lh * 256 + c * 16 + l16) * LDT + ps * 32 + g * 4;
        const u32x2_t lo = ld8(tp), hi = ld8(tp + 16);
        oacc[c] = mfma_bf16_16x16x32(as_bf16x8(u32x4_t{lo[0], lo[1], hi[0], hi[1]}), pf, oacc[c]);
      }
    }
  }

  // ---- split outputs: unnormalised o (relative to mrun), running max and sum per head
  lrun += __shfl_xor(lrun, 16);
  lrun += __shfl_xor(lrun, 32);
  const int64_t pidx = ((int64_t)b * a.max_splits + split) * 64 + head;
  float* po = a.part_o + pidx * KV_LORA + lh * 256;
#pragma unroll
  for (int c = 0; c < 16; ++c) *reinterpret_cast<f32x4_t*>(po + c * 16 + g * 4) = oacc[c];
  if (lh == 0 && g == 0) {
    a.part_ml[pidx * 2] = mrun;
    a.part_ml[pidx * 2 + 1] = lrun;
  }
}

// One workgroup (256 threads) per (sequence, head): combine the splits, write bf16 o_lat.
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeAttnArgs a) {
  using namespace mla_dims;
  const int head = blockIdx.x, b = blockIdx.y;
  const int L = a.len[a.seq_ids[b]];
  const int ns = cdiv(L, a.chunk);
  const int64_t base = (int64_t)b * a.max_splits * 64 + head;
  float mx = -INFINITY;
  for (int s = 0; s < ns; ++s) mx = fmaxf(mx, a.part_ml[(base + (int64_t)s * 64) * 2]);
  float l = 0.f, o0 = 0.f, o1 = 0.f;
  const int c = threadIdx.x * 2;
  for (int s = 0; s < ns; ++s) {
    const int64_t p = base + (int64_t)s * 64;
    const float w = exp2f(a.part_ml[p * 2] - mx);
    l += w * a.part_ml[p * 2 + 1];
    const f32x2_t v = *reinterpret_cast<const f32x2_t*>(a.part_o + p * KV_LORA + c);
    o0 += w * v[0];
    o1 += w * v[1];
  }
  const float inv = 1.0f / l;
  *reinterpret_cast<uint32_t*>(a.o_lat + ((int64_t)b * 64 + head) * KV_LORA + c) = pack_bf16x2(o0 * inv, o1 * inv);
}

}  // namespace

hipError_t decode_attention(const DecodeAttnArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  if (a.fp8) return hipErrorNotSupported;
  hipLaunchKernelGGL(decode_attn_kernel, dim3(a.max_splits, a.B), dim3(512), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(64, a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla_k
