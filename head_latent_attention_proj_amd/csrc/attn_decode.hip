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
// Work layout: one workgroup = (sequence, split of `chunk` positions), 8 waves = 4 head groups of
// 16 x 2 feature halves. Heads are the MFMA column dimension, so one 32-position block staged in
// LDS feeds every head: S^T = C Q^T (A = cache rows, B = queries held in registers), then
// O^T = C^T P^T from a transposed copy of the block's latent part written while staging. The next
// block's loads are in flight (in registers) while a block is used. Each split writes (max, sum,
// unnormalised o) per head; the merge kernel combines the splits.
#include "common.h"
#include "kernels.h"

namespace mla_k {

namespace {

constexpr int DKB = 32;    // positions per block
constexpr int LDC = 584;   // sC row: 576 features + pad (1168 B: 16 rows -> distinct bank groups)
constexpr int LDT = 36;    // sT row: 32 positions + pad (72 B: 16 rows -> distinct 8-byte slots)
constexpr int HALF = 288;  // score features per wave: [0, 288) or [288, 576)
constexpr float LOG2E = 1.4426950408889634f;

MLA_DEV u32x2_t ld8(const void* p) { return *reinterpret_cast<const u32x2_t*>(p); }

// 8 waves: wave = hg + 4*lh, head group hg (heads hg*16 .. +15), half lh. A wave forms the
// partial scores of its 16 heads over features [lh*288, lh*288+288) and, after the two halves
// are added through LDS, mixes latent features [lh*256, lh*256+256). Two waves per SIMD hide
// each other's LDS and memory latency; per-wave registers stay well under 256.
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
  const int hg = wave & 3, lh = wave >> 2;
  const int l16 = lane & 15, g = lane >> 4;
  const int head = hg * 16 + l16;

  __shared__ __attribute__((aligned(16))) uint16_t sC[DKB * LDC];
  __shared__ __attribute__((aligned(16))) uint16_t sT[KV_LORA * LDT];
  __shared__ __attribute__((aligned(16))) float xS[8][8][64];  // partial scores per wave

  // ---- staging through registers, one block ahead. Latent part as position pairs: item i (0..1)
  // of a thread is pair kp = lane & 15 and 16-byte chunk ch = (lane >> 4) + 4*(wave + 8*i);
  // k_pe: threads 0..255 one chunk each.
  u32x4_t rl[2][2], rp;
  auto gload = [&](int blk) {
    const int kb = c0 + blk * DKB;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int kp = lane & 15;
      const int ch = (lane >> 4) + 4 * (wave + 8 * i);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int key = min(kb + 2 * kp + u, c1 - 1);  // past the split's end: re-read (masked)
        rl[i][u] = ld16(a.cache + (slot0 + key) * a.entry_bytes + ch * 16);
      }
    }
    if (tid < 256) {
      const int key = min(kb + (tid >> 3), c1 - 1);
      rp = ld16(a.cache + (slot0 + key) * a.entry_bytes + KV_LORA * 2 + (tid & 7) * 16);
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int kp = lane & 15;
      const int ch = (lane >> 4) + 4 * (wave + 8 * i);
      st16(sC + (2 * kp) * LDC + ch * 8, rl[i][0]);
      st16(sC + (2 * kp + 1) * LDC + ch * 8, rl[i][1]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t x = rl[i][0][j], y = rl[i][1][j];
        // features ch*8 + 2j (low halves) and ch*8 + 2j + 1 (high halves), positions 2kp, 2kp+1
        *reinterpret_cast<uint32_t*>(sT + (ch * 8 + 2 * j) * LDT + 2 * kp) = (x & 0xffffu) | (y << 16);
        *reinterpret_cast<uint32_t*>(sT + (ch * 8 + 2 * j + 1) * LDT + 2 * kp) = (x >> 16) | (y & 0xffff0000u);
      }
    }
    if (tid < 256) st16(sC + (tid >> 3) * LDC + KV_LORA + (tid & 7) * 8, rp);
  };
  gload(0);  // in flight during the query set-up

  // ---- query fragments (B operand): column = head, features lh*288 + ks*32 + g*8 .. +7;
  // features >= 512 are the rotary part, rotated here at the query's position
  bf16x8_t qf[9];
  {
    const uint16_t* ql = a.q_lat + ((int64_t)b * 64 + head) * KV_LORA;
    const uint16_t* qp = a.q + ((int64_t)b * 64 + head) * QK + NOPE;
    const int pos = L - 1;
#pragma unroll
    for (int ks = 0; ks < 9; ++ks) {
      const int f = lh * HALF + ks * 32 + g * 8;
      if (f < KV_LORA) {
        qf[ks] = as_bf16x8(ld16(ql + f));
      } else {
        const u32x4_t raw = ld16(qp + (f - KV_LORA));
        const int pair0 = (f - KV_LORA) >> 1;
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
  }

  const float sl2 = a.scale * LOG2E;
  float mrun = -INFINITY, lrun = 0.f;
  f32x4_t oacc[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) oacc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int blk = 0; blk < nblk; ++blk) {
    __syncthreads();  // the previous block's LDS reads are done
    sstore();
    __syncthreads();
    if (blk + 1 < nblk) gload(blk + 1);
    const int kb = c0 + blk * DKB;

    // partial S^T[key][head] over this wave's 288 features, two key tiles
    f32x4_t sacc[2];
    sacc[0] = sacc[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    {
      const uint16_t* r0 = sC + l16 * LDC + lh * HALF + g * 8;
      const uint16_t* r1 = r0 + 16 * LDC;
      bf16x8_t k0[9], k1[9];
#pragma unroll
      for (int ks = 0; ks < 9; ++ks) {
        k0[ks] = as_bf16x8(ld16(r0 + ks * 32));
        k1[ks] = as_bf16x8(ld16(r1 + ks * 32));
      }
#pragma unroll
      for (int ks = 0; ks < 9; ++ks) {
        sacc[0] = mfma_bf16_16x16x32(k0[ks], qf[ks], sacc[0]);
        sacc[1] = mfma_bf16_16x16x32(k1[ks], qf[ks], sacc[1]);
      }
    }
    // add the other half's partial scores (same order in both waves of a pair)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) xS[wave][kt * 4 + e][lane] = sacc[kt][e];
    __syncthreads();
    const int other = wave ^ 4;
    float sv[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float mine = sacc[kt][e], theirs = xS[other][kt * 4 + e][lane];
        sv[kt][e] = lh == 0 ? mine + theirs : theirs + mine;
      }
    float bmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float s = sv[kt][e] * sl2;
        if (kb + kt * 16 + g * 4 + e >= c1) s = -INFINITY;
        sv[kt][e] = s;
        bmax = fmaxf(bmax, s);
      }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    const float mnew = fmaxf(mrun, bmax);
    const float alpha = exp2f(mrun - mnew);
    mrun = mnew;
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = exp2f(sv[kt][e] - mnew);
        sv[kt][e] = p;
        psum += p;
      }
    lrun = lrun * alpha + psum;
    u32x4_t w;
    w[0] = pack_bf16x2(sv[0][0], sv[0][1]);
    w[1] = pack_bf16x2(sv[0][2], sv[0][3]);
    w[2] = pack_bf16x2(sv[1][0], sv[1][1]);
    w[3] = pack_bf16x2(sv[1][2], sv[1][3]);
    const bf16x8_t pf = as_bf16x8(w);
    // O^T[dim][head] += C^T[dim][keys] P^T[keys][head] over this wave's 256 latent features;
    // lane group g holds keys g*4..+3 and 16+g*4..+3
    {
      const uint16_t* tp = sT + (lh * 256 + l16) * LDT + g * 4;
#pragma unroll
      for (int c0_ = 0; c0_ < 16; c0_ += 8) {
        u32x2_t lo[8], hi[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          lo[c] = ld8(tp + (c0_ + c) * 16 * LDT);
          hi[c] = ld8(tp + (c0_ + c) * 16 * LDT + 16);
        }
#pragma unroll
        for (int c = 0; c < 8; ++c)
          oacc[c0_ + c] = mfma_bf16_16x16x32(as_bf16x8(u32x4_t{lo[c][0], lo[c][1], hi[c][0], hi[c][1]}), pf,
                                             oacc[c0_ + c] * alpha);
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
// Split statistics are read first (independent loads), then the partial outputs, eight splits
// at a time so their loads overlap.
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeAttnArgs a) {
  using namespace mla_dims;
  const int head = blockIdx.x, b = blockIdx.y;
  const int L = a.len[a.seq_ids[b]];
  const int ns = cdiv(L, a.chunk);
  const int64_t base = (int64_t)b * a.max_splits * 64 + head;
  __shared__ float wsh[2048];
  __shared__ float red[4];
  float mx = -INFINITY;
  for (int s = threadIdx.x; s < ns; s += 256) mx = fmaxf(mx, a.part_ml[(base + (int64_t)s * 64) * 2]);
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float lpart = 0.f;
  for (int s = threadIdx.x; s < ns; s += 256) {
    const int64_t p = base + (int64_t)s * 64;
    const float w = exp2f(a.part_ml[p * 2] - mx);
    wsh[s] = w;
    lpart += w * a.part_ml[p * 2 + 1];
  }
  __syncthreads();
  lpart = wave_sum(lpart);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = lpart;
  __syncthreads();
  const float l = red[0] + red[1] + red[2] + red[3];
  const int c = threadIdx.x * 2;
  float o0 = 0.f, o1 = 0.f;
  int s = 0;
  for (; s + 8 <= ns; s += 8) {
    f32x2_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = *reinterpret_cast<const f32x2_t*>(a.part_o + (base + (int64_t)(s + u) * 64) * KV_LORA + c);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      o0 += wsh[s + u] * v[u][0];
      o1 += wsh[s + u] * v[u][1];
    }
  }
  for (; s < ns; ++s) {
    const f32x2_t v = *reinterpret_cast<const f32x2_t*>(a.part_o + (base + (int64_t)s * 64) * KV_LORA + c);
    o0 += wsh[s] * v[0];
    o1 += wsh[s] * v[1];
  }
  const float inv = 1.0f / l;
  *reinterpret_cast<uint32_t*>(a.o_lat + ((int64_t)b * 64 + head) * KV_LORA + c) = pack_bf16x2(o0 * inv, o1 * inv);
}

}  // namespace

hipError_t decode_attention(const DecodeAttnArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  if (a.fp8) return hipErrorNotSupported;
  if (a.max_splits > 2048) return hipErrorInvalidValue;  // the merge keeps split weights in LDS
  hipLaunchKernelGGL(decode_attn_kernel, dim3(a.max_splits, a.B), dim3(512), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(64, a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla_k
