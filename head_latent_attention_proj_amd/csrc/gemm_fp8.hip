// FP8 (OCP E4M3FN) projections: weights with one float32 scale per 128 x 128 block, activations
// quantised per token and per aligned group of 128 features ("Key-value latent" page, linear
// excerpt: quantization_config fmt e4m3, weight_block_size [128, 128], activation_scheme dynamic).
//
// C[m][n] = sum over 128-wide K groups kg of  sa[m][kg] * sb[n/128][kg] * sum_{k in kg} a[m][k] b[n][k]
// with a, b the code values. Each K group's partial sum is formed on the matrix cores and then
// scaled and accumulated in float32 registers. Two ways to form it:
//   * native: one 16x16x128 FP8 MFMA (unit hardware scales) per group;
//   * precise: the codes are widened to bf16 (exact: every E4M3 value is a bf16 value) and the
//     group is summed by four 16x16x32 bf16 MFMAs, which accumulate in float32.
// Measured on gfx950 against float64 on the layer's weights and quantised activations (the FP8
// GEMM GPU test), as a fraction of sum |a b| per output: native 1.2e-6 .. 6.9e-6 at most (medians
// 1.6e-7 .. 5.9e-7), precise 1e-8 .. 3.2e-8. Which projection may take the native form was decided
// by the layer's parity against the W8A8 float64 oracle with each one switched: q_a|kv_a fails
// (2.3e-2 max-abs at a 50-token prefill: its outputs are quantised again, into q_b's input codes
// and the cached latent codes, where a small error flips codes); q_b passes with unchanged margins
// (its output becomes fp16 attention operands) and is faster; kv_b passes too but gains nothing
// measurable, and its values are the attention operands kept to about 22 bits. So q_a|kv_a and
// kv_b take the precise form; q_b and o_proj the native one.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "splitk.h"

namespace mla_k {

namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// D = A(16x128 e4m3) * B(128x16 e4m3), hardware block scales fixed at 1 (E8M0 127).
MLA_DEV f32x4_t mfma_fp8_16x16x128(const i32x8_t& a, const i32x8_t& b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0x7f7f7f7f, 0,
                                                          0x7f7f7f7f);
}

// eight E4M3 codes (two words) -> eight bf16 values, exact (unit conversion scale)
MLA_DEV bf16x8_t widen8(uint32_t w0, uint32_t w1) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// One K group (128) of a 16x16 tile in float32 precision: the lane's 32 codes of A and B
// (k = g*32 .. g*32+31 of the group) in four bf16 MFMA steps of eight codes each.
MLA_DEV f32x4_t group_precise(const i32x8_t& a, const bf16x8_t (&bw)[4]) {
  f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) d = mfma_bf16_16x16x32(widen8(a[2 * s], a[2 * s + 1]), bw[s], d);
  return d;
}

MLA_DEV i32x8_t cat8(const u32x4_t& lo, const u32x4_t& hi) {
  return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

MLA_DEV void epi_store8(const GemmArgs& p, int b, int m, int n, float v) {
  if (p.epi == EPI_F32) {
    ((float*)p.C)[b * p.sC + (int64_t)m * p.ldc + n] = v;
  } else if (p.epi == EPI_F16) {
    ((uint16_t*)p.C)[b * p.sC + (int64_t)m * p.ldc + n] = (uint16_t)pack_f16x2(v, 0.f);
  } else if (p.epi == EPI_BF16) {
    if (p.resid) v += bf2f(p.resid[(int64_t)m * p.ldr + n]);
    ((uint16_t*)p.C)[b * p.sC + (int64_t)m * p.ldc + n] = f2bf(v);
  } else {  // EPI_KVB in fp16; with vt_lo set, the values' fp16 residuals go to a second plane
    const int h = n >> 8, r = n & 255;
    const int64_t key = p.key_base + m;
    const uint32_t hv = pack_f16x2(v, 0.f);
    if (r < 128) {
      p.knope[key * 8192 + h * 128 + r] = (uint16_t)hv;
    } else {
      const int64_t i = (int64_t)(h * 128 + r - 128) * p.vt_ld + key;
      p.vt[i] = (uint16_t)hv;
      if (p.vt_lo) p.vt_lo[i] = (uint16_t)pack_f16x2(v - f16_lo(hv), 0.f);
    }
  }
}

// ------------------------------------------------------------------------------------------
// Decode-sized M: one workgroup per 16-column tile, K groups split across its KW waves,
// partial tiles summed through LDS in a fixed order.
// ------------------------------------------------------------------------------------------
template <int MT, int KW, int TAG, bool PREC>
__global__ __launch_bounds__(KW * 64) void gemm_fp8_wsplit_kernel(GemmArgs p) {
  constexpr int U = MT >= 4 ? 1 : (MT == 2 ? 2 : 4);  // K groups per pipeline stage
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int batch = blockIdx.z;
  const uint8_t* A = (const uint8_t*)p.A + batch * p.sA;
  const uint8_t* B = (const uint8_t*)p.B + batch * p.sB;
  const int ngroups = p.K >> 7;
  const int ygroups = cdiv(ngroups, (int)gridDim.y);
  const int y0 = blockIdx.y * ygroups, y1 = min(ngroups, y0 + ygroups);
  const int gpw = cdiv(y1 - y0, KW);
  const int k0 = y0 + wave * gpw, k1 = min(y1, k0 + gpw);

  int rows[MT];
  const uint8_t* pa[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    rows[i] = min(i * 16 + l16, p.M - 1);
    pa[i] = A + (int64_t)rows[i] * p.lda + g * 32;
  }
  const uint8_t* pb = B + (int64_t)min(n0 + l16, p.N - 1) * p.ldb + g * 32;
  const float* sbp = p.b_scale + (int64_t)(min(n0, p.N - 1) >> 7) * p.bs_ld;
  // a-scale rows of this lane's result values: m = i*16 + g*4 + e
  const float* sap[MT][4];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) sap[i][e] = p.a_scale + (int64_t)min(i * 16 + g * 4 + e, p.M - 1) * p.as_ld;

  f32x4_t acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (k0 < k1) {
    for (int kg = k0; kg < k1; kg += U) {
      i32x8_t af[U][MT], bf[U];
      float sb[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = min(kg + u, k1 - 1);
        bf[u] = cat8(ld16(pb + kk * 128), ld16(pb + kk * 128 + 16));
        sb[u] = sbp[kk];
#pragma unroll
        for (int i = 0; i < MT; ++i) af[u][i] = cat8(ld16(pa[i] + kk * 128), ld16(pa[i] + kk * 128 + 16));
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (kg + u >= k1) break;  // wave-uniform
        bf16x8_t bw[4];
        if constexpr (PREC) {
#pragma unroll
          for (int st = 0; st < 4; ++st) bw[st] = widen8(bf[u][2 * st], bf[u][2 * st + 1]);
        }
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const f32x4_t d = PREC ? group_precise(af[u][i], bw) : mfma_fp8_16x16x128(af[u][i], bf[u]);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][e] += d[e] * (sap[i][e][kg + u] * sb[u]);
        }
      }
    }
  }

  if constexpr (KW > 1) {
    __shared__ float red[(KW - 1) * MT * 4 * 64];
    if (wave > 0) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[(((wave - 1) * MT + i) * 4 + e) * 64 + lane] = acc[i][e];
    }
    __syncthreads();
    if (wave != 0) return;
    for (int w = 0; w < KW - 1; ++w)
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][e] += red[((w * MT + i) * 4 + e) * 64 + lane];
  }
  if (gridDim.y > 1) {  // partial sum of this K split (EPI_F32 only; the consumer adds the parts)
    float* C = (float*)p.C + blockIdx.y * p.c_split_stride + batch * p.sC;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = i * 16 + g * 4 + e, n = n0 + l16;
        if (m < p.M && n < p.N) C[(int64_t)m * p.ldc + n] = acc[i][e];
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = i * 16 + g * 4 + e, n = n0 + l16;
      if (m < p.M && n < p.N) epi_store8(p, batch, m, n, acc[i][e]);
    }
}

// ------------------------------------------------------------------------------------------
// Prefill-sized M: BM x BN tile (128 x 256 or 128 x 128), one 128-wide K group per stage staged
// through LDS (144-byte
// rows: 8 consecutive rows hit 8 distinct 16-byte bank groups), double buffered.
// ------------------------------------------------------------------------------------------
// Stage rows of 128 bytes (one K group of codes) keep 16-byte chunk c of row r at position
// c ^ chunk_swz(r). A lane's operand halves are chunks 2g and 2g + 1 of row l16; gfx950 serves a
// 16-byte LDS read 16 lanes per cycle from 64 four-byte banks, those 16 lanes being the four quads
// (lane / 4) of one half-wave whose index has one parity of its low three bits, i.e. 8 rows of each
// of two values of g. With r's bits b1 and b3, chunk_swz = (b3, b3, b1) puts such 16 lanes on
// distinct banks (the plain (r / 2) % 8 left every read 2-way conflicted, as the bank-conflict counter
// showed); the stores of a row (8 consecutive lanes, 8 distinct chunks) stay conflict-free with any
// per-row swizzle.
MLA_DEV int chunk_swz(int r) { return (((r >> 3) & 1) * 6) | ((r >> 1) & 1); }

template <int BM, int BN, int WM, int WN, int TAG, bool PREC>
__global__ __launch_bounds__(WM* WN * 64) void gemm_fp8_tile_kernel(GemmArgs p, int splits, int ksplit) {
  constexpr int NT = WM * WN * 64;
  constexpr int BK = 128;  // bytes (= codes) per row per stage: one K group
  // unpadded 128-byte stage rows, 16-byte chunk c of row r at position c ^ chunk_swz(r)
  constexpr int LDK = BK;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 16, TN = WTN / 16;
  constexpr int CPR = BK / 16;
  constexpr int RPP = NT / CPR;
  constexpr int AP = BM / RPP, BP = BN / RPP;
  static_assert(BM % RPP == 0 && BN % RPP == 0, "tile rows must be a multiple of rows per pass");
  constexpr int SMEM = std::max(2 * (BM + BN) * LDK, WM * WN * (BM / WM) * (BN / WN + 8) * 4);  // tiles / epilogue
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  __shared__ __attribute__((aligned(16))) float sSa[2][BM];  // A scales of the stage's K group, per row
  static_assert((BM & (BM - 1)) == 0 && NT >= BM, "one A scale per thread");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int l16 = lane & 15, g = lane >> 4;

  const int tiles_m = cdiv(p.M, BM), tiles_n = cdiv(p.N, BN);
  const int ntile = tiles_m * tiles_n;
  int bid = blockIdx.x;
  if ((ntile & 7) == 0) bid = (bid & 7) * (ntile >> 3) + (bid >> 3);
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int fm = (bid / per_group) * GM;
  const int gs = min(tiles_m - fm, GM);
  const int tm = fm + (bid % per_group) % gs;
  const int tn = (bid % per_group) / gs;
  const int m0 = tm * BM, n0 = tn * BN;
  const int batch = blockIdx.z, split = blockIdx.y;

  const uint8_t* A = (const uint8_t*)p.A + batch * p.sA;
  const uint8_t* B = (const uint8_t*)p.B + batch * p.sB;

  const int lr = tid / CPR, lc = (tid % CPR) * 16;
  static_assert(CPR == 8 && RPP % 16 == 0, "swizzle: 8 chunks per row, passes of whole 16-row groups");
  const int lcs = ((tid % CPR) ^ chunk_swz(lr)) << 4;  // this thread's chunk, swizzled
  const uint8_t* ga[AP];
  const uint8_t* gb[BP];
#pragma unroll
  for (int i = 0; i < AP; ++i) ga[i] = A + (int64_t)min(m0 + i * RPP + lr, p.M - 1) * p.lda + lc;
#pragma unroll
  for (int i = 0; i < BP; ++i) gb[i] = B + (int64_t)min(n0 + i * RPP + lr, p.N - 1) * p.ldb + lc;

  // A scales staged with the tiles (row tid % BM of the tile, every thread loads one: the same loads
  // in every wave); a wave's columns lie in one 128-column weight block (WTN divides 128), whose
  // scale is read once per K group
  static_assert(128 % WTN == 0, "a wave's columns span one weight scale block");
  const float* gsa = p.a_scale + (int64_t)min(m0 + (tid & (BM - 1)), p.M - 1) * p.as_ld;
  const float* gsb = p.b_scale + (int64_t)(min(n0 + wn * WTN, p.N - 1) >> 7) * p.bs_ld;
  float rsa;

  u32x4_t ra[AP], rb[BP];
  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int kb = split * ksplit;
  const int ke = min(p.K, kb + ksplit);
  const int nk = (ke - kb) / BK;

  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < AP; ++i) ra[i] = ld16(ga[i] + k0);
#pragma unroll
    for (int i = 0; i < BP; ++i) rb[i] = ld16(gb[i] + k0);
    rsa = gsa[k0 >> 7];
  };
  auto sstore = [&](int buf) {
    uint8_t* sa = smem + buf * (BM + BN) * LDK;
    uint8_t* sb = sa + BM * LDK;
#pragma unroll
    for (int i = 0; i < AP; ++i) st16(sa + (i * RPP + lr) * LDK + lcs, ra[i]);
#pragma unroll
    for (int i = 0; i < BP; ++i) st16(sb + (i * RPP + lr) * LDK + lcs, rb[i]);
    if (tid < BM) sSa[buf][tid] = rsa;
  };

  if (nk > 0) {
    gload(kb);
    sstore(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const int kg = (kb >> 7) + kt;
    if (kt + 1 < nk) gload(kb + (kt + 1) * BK);
    // combined scale of this lane's result rows m = m0 + wm*WTM + i*16 + g*4 + e for this K group
    f32x4_t sab[TM];
    {
      const float sbk = gsb[kg];
#pragma unroll
      for (int i = 0; i < TM; ++i) sab[i] = *reinterpret_cast<const f32x4_t*>(&sSa[cur][wm * WTM + i * 16 + g * 4]) * sbk;
    }
    // this lane's rows (row l16 of each 16-row tile keeps its swizzle) and the positions of its
    // chunks 2g and 2g + 1
    const uint8_t* sA = smem + cur * (BM + BN) * LDK + (wm * WTM + l16) * LDK;
    const uint8_t* sB = smem + cur * (BM + BN) * LDK + BM * LDK + (wn * WTN + l16) * LDK;
    const int swz = chunk_swz(l16);
    const int c0 = ((2 * g) ^ swz) << 4, c1 = ((2 * g + 1) ^ swz) << 4;
    if constexpr (PREC) {
      // four steps of eight codes (k = g*32 + st*8 ..) widened to bf16 as they are read
      f32x4_t d[TM][TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) d[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        bf16x8_t bw[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const u32x2_t r = *reinterpret_cast<const u32x2_t*>(sB + j * 16 * LDK + (st < 2 ? c0 : c1) + (st & 1) * 8);
          bw[j] = widen8(r[0], r[1]);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const u32x2_t r = *reinterpret_cast<const u32x2_t*>(sA + i * 16 * LDK + (st < 2 ? c0 : c1) + (st & 1) * 8);
          const bf16x8_t aw = widen8(r[0], r[1]);
#pragma unroll
          for (int j = 0; j < TN; ++j) d[i][j] = mfma_bf16_16x16x32(aw, bw[j], d[i][j]);
        }
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][e] += d[i][j][e] * sab[i][e];
    } else {
      i32x8_t bfr[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = cat8(ld16(sB + j * 16 * LDK + c0), ld16(sB + j * 16 * LDK + c1));
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const i32x8_t af = cat8(ld16(sA + i * 16 * LDK + c0), ld16(sA + i * 16 * LDK + c1));
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const f32x4_t d = mfma_fp8_16x16x128(af, bfr[j]);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][e] += d[e] * sab[i][e];
        }
      }
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  if (splits == 1) {
    if (p.epi == EPI_BF16 && !p.resid && (p.N & 7) == 0 && (p.ldc & 7) == 0 && (p.sC & 7) == 0 &&
        (reinterpret_cast<uintptr_t>(p.C) & 15) == 0) {
      // bf16 output through LDS: each wave writes its WTM x WTN results to a private region of the
      // (then free) tile buffers and stores whole 16-byte pieces of output rows, eight lanes per
      // 128-byte row segment, instead of one 2-byte store per value
      constexpr int LDW = WTN + 8;
      static_assert(WM * WN * WTM * LDW * 2 <= SMEM, "epilogue staging fits the tile buffers");
      uint16_t* sw = reinterpret_cast<uint16_t*>(smem) + wave * (WTM * LDW);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) sw[(i * 16 + g * 4 + e) * LDW + j * 16 + l16] = f2bf(acc[i][j][e]);
      __syncthreads();
      const int lr8 = lane >> 3, lc8 = (lane & 7) * 8;
      const int n = n0 + wn * WTN + lc8;
      if (n < p.N) {  // N is a multiple of 8: a piece is whole or wholly outside
        uint16_t* cb = (uint16_t*)p.C + batch * p.sC + n;
#pragma unroll
        for (int k = 0; k < WTM / 8; ++k) {
          const int r = k * 8 + lr8;
          const int m = m0 + wm * WTM + r;
          if (m < p.M) st16(cb + (int64_t)m * p.ldc, ld16(sw + r * LDW + lc8));
        }
      }
      return;
    }
    if constexpr (WTN == 64 && WM * WN * WTM * (WTN + 8) * 4 <= SMEM) {
      if (p.epi == EPI_KVB && (p.key_base & 3) == 0 && (p.N & 7) == 0) {
        // kv_b (fp16): a wave's 64 columns lie in one half of a head's 256 (wave-uniform). Content
        // keys go through LDS and leave as 16-byte pieces of K_nope rows; values and their fp16
        // residuals go straight to V^T as 8-byte pieces (four consecutive keys of one feature per
        // lane). Every wave reaches the barrier.
        constexpr int LDW = WTN + 8;
        uint16_t* shi = reinterpret_cast<uint16_t*>(smem) + wave * (WTM * LDW);
        const int nw0 = n0 + wn * WTN;
        const bool khalf = (nw0 & 255) < 128;
        if (khalf) {
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                shi[(i * 16 + g * 4 + e) * LDW + j * 16 + l16] = (uint16_t)pack_f16x2(acc[i][j][e], 0.f);
        } else {
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
              const int mb = m0 + wm * WTM + i * 16 + g * 4;
              const int n = nw0 + j * 16 + l16;
              if (n >= p.N) continue;
              if (mb + 3 < p.M) {
                const f32x4_t v = acc[i][j];
                const uint32_t h01 = pack_f16x2(v[0], v[1]), h23 = pack_f16x2(v[2], v[3]);
                const int64_t at = (int64_t)((n >> 8) * 128 + (n & 255) - 128) * p.vt_ld + p.key_base + mb;
                *reinterpret_cast<u32x2_t*>(p.vt + at) = u32x2_t{h01, h23};
                if (p.vt_lo)
                  *reinterpret_cast<u32x2_t*>(p.vt_lo + at) =
                      u32x2_t{pack_f16x2(v[0] - f16_lo(h01), v[1] - f16_hi(h01)), pack_f16x2(v[2] - f16_lo(h23), v[3] - f16_hi(h23))};
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  if (mb + e < p.M) epi_store8(p, batch, mb + e, n, acc[i][j][e]);
              }
            }
        }
        __syncthreads();
        if (khalf) {
          const int lr8 = lane >> 3, lc8 = (lane & 7) * 8;
          const int n = nw0 + lc8;
          if (n < p.N) {
            const int64_t col = (n >> 8) * 128 + (n & 255);
#pragma unroll
            for (int k = 0; k < WTM / 8; ++k) {
              const int r = k * 8 + lr8;
              const int m = m0 + wm * WTM + r;
              if (m < p.M) {
                const int64_t at = (p.key_base + m) * 8192 + col;
                st16(p.knope + at, ld16(shi + r * LDW + lc8));
              }
            }
          }
        }
        return;
      }
    }
    if (p.epi == EPI_KVB && (p.key_base & 3) == 0) {
      // kv_b: a lane's four accumulators are four consecutive keys of one feature, i.e. four
      // adjacent elements of a value row of V^T (and of its residual plane): one 8-byte write
      // each instead of four 2-byte writes to four places
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int mb = m0 + wm * WTM + i * 16 + g * 4;
          const int n = n0 + wn * WTN + j * 16 + l16;
          if (n >= p.N) continue;
          if ((n & 255) >= 128 && mb + 3 < p.M) {
            const f32x4_t v = acc[i][j];
            const uint32_t h01 = pack_f16x2(v[0], v[1]), h23 = pack_f16x2(v[2], v[3]);
            const int64_t at = (int64_t)((n >> 8) * 128 + (n & 255) - 128) * p.vt_ld + p.key_base + mb;
            *reinterpret_cast<u32x2_t*>(p.vt + at) = u32x2_t{h01, h23};
            if (p.vt_lo)
              *reinterpret_cast<u32x2_t*>(p.vt_lo + at) =
                  u32x2_t{pack_f16x2(v[0] - f16_lo(h01), v[1] - f16_hi(h01)), pack_f16x2(v[2] - f16_lo(h23), v[3] - f16_hi(h23))};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (mb + e < p.M) epi_store8(p, batch, mb + e, n, acc[i][j][e]);
          }
        }
      return;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + wm * WTM + i * 16 + g * 4 + e;
          const int n = n0 + wn * WTN + j * 16 + l16;
          if (m < p.M && n < p.N) epi_store8(p, batch, m, n, acc[i][j][e]);
        }
    return;
  }
  float* part = p.part + ((int64_t)batch * splits + split) * p.M * p.N;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm * WTM + i * 16 + g * 4 + e;
        const int n = n0 + wn * WTN + j * 16 + l16;
        if (m < p.M && n < p.N) part[(int64_t)m * p.N + n] = acc[i][j][e];
      }
}

// ------------------------------------------------------------------------------------------
// K groups streamed through a ring of LDS stages (both forms; prefill and decode sizes)
// ------------------------------------------------------------------------------------------
// 128 x BN output tile (BN = 256, 128 or 64), waves of 64 x 64 (2 x BN/64). A stage is one K
// group: the A tile as 8 and the B tile as BN/16 blocks of 16 rows x 128 codes, and the tile's
// 128 A scales. Every piece is fetched by direct-to-LDS loads, which hold no registers: two stages
// are in flight while the third is multiplied (the register-staged tile kernel has one stage of
// compute to cover each load). One wave instruction fetches 8 whole rows of a block (lane l: row
// l / 8, one 16-byte chunk), so it touches 8 cache lines; a block lands row-major, chunk c of row r
// at position c ^ chunk_swz(r), where a lane's operand halves (row l16, chunks 2g and 2g + 1) are
// read on distinct banks. The row scales are fetched by one wave per 64
// rows. Three stages of 48.5 KB at BN = 256 (one workgroup per CU), 24.5 KB at BN = 64 (two).
namespace ring8 {
constexpr int BM = 128, S = 3;
constexpr int A_BYTES = BM * 128;
constexpr int SC_BYTES = BM * 4;
constexpr int LDW = 64 + 4;  // float32 epilogue staging row (a wave's 64 columns)
// stage bytes for a BN-column tile: 49,664 at 256 columns, 25,088 at 64
constexpr int stage_bytes(int bn) { return A_BYTES + bn * 128 + SC_BYTES; }
}  // namespace ring8

// One stage's operands of a wave (byte addresses of this lane's 16 bytes): A blocks at a0 / a1
// (chunk halves 0 / 1) + 2048 i, B blocks at b0 / b1 + 2048 j, the row scales (4 floats) at
// c + 64 i, and the stage's weight-block scale (a scalar load from sb). One asm block that waits
// for its own reads: the compiler cannot tell that they never touch the slots the direct-to-LDS
// loads are still filling and would wait for every load in flight (it also turns a plain load of
// the weight scale into a vector load, counted with the ring's). Early-clobber outputs, so no
// read's destination is an address of a later read.
MLA_DEV void ring8_operands(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, uint32_t c, const float* sb,
                            u32x4_t (&ra)[8], u32x4_t (&rb)[8], f32x4_t (&sc)[4], float& sbk) {
  asm volatile(
      "s_load_dword %20, %26, 0x0\n\t"
      "ds_read_b128 %0, %21\n\tds_read_b128 %1, %22\n\t"
      "ds_read_b128 %2, %21 offset:2048\n\tds_read_b128 %3, %22 offset:2048\n\t"
      "ds_read_b128 %4, %21 offset:4096\n\tds_read_b128 %5, %22 offset:4096\n\t"
      "ds_read_b128 %6, %21 offset:6144\n\tds_read_b128 %7, %22 offset:6144\n\t"
      "ds_read_b128 %8, %23\n\tds_read_b128 %9, %24\n\t"
      "ds_read_b128 %10, %23 offset:2048\n\tds_read_b128 %11, %24 offset:2048\n\t"
      "ds_read_b128 %12, %23 offset:4096\n\tds_read_b128 %13, %24 offset:4096\n\t"
      "ds_read_b128 %14, %23 offset:6144\n\tds_read_b128 %15, %24 offset:6144\n\t"
      "ds_read_b128 %16, %25\n\tds_read_b128 %17, %25 offset:64\n\t"
      "ds_read_b128 %18, %25 offset:128\n\tds_read_b128 %19, %25 offset:192\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(ra[0]), "=&v"(ra[1]), "=&v"(ra[2]), "=&v"(ra[3]), "=&v"(ra[4]), "=&v"(ra[5]), "=&v"(ra[6]), "=&v"(ra[7]),
        "=&v"(rb[0]), "=&v"(rb[1]), "=&v"(rb[2]), "=&v"(rb[3]), "=&v"(rb[4]), "=&v"(rb[5]), "=&v"(rb[6]), "=&v"(rb[7]),
        "=&v"(sc[0]), "=&v"(sc[1]), "=&v"(sc[2]), "=&v"(sc[3]), "=&s"(sbk)
      : "v"(a0), "v"(a1), "v"(b0), "v"(b1), "v"(c), "s"(sb)
      : "memory");
}

// Requirements (checked by ring8_ok): K a multiple of 128, 16-byte aligned operand rows, and
// EPI_F32, EPI_BF16 or EPI_F16 with 16-byte aligned C, ldc and N multiples of 8 (bf16, fp16) or 4 (f32), for a
// residual 16-byte alignment and ldr a multiple of 8; or EPI_KVB (batch 1) with key_base and vt_ld
// multiples of 4, N of 8, K_nope 16-byte and V^T planes 8-byte aligned.
// BN = 256 (prefill sizes: 8 waves, one workgroup per CU), 128 (4 waves, one per CU) or 64 (2 waves,
// two per CU); at decode sizes K is split over blockIdx.y into float32 partials (`splits` > 1).
template <int TAG, bool PREC, int BN>
__global__ __launch_bounds__(BN / 32 * 64) void gemm_fp8_ring_kernel(GemmArgs p, int splits, int ksplit) {
  using namespace ring8;
  constexpr int WN = BN / 64, NW = 2 * WN;  // waves: 2 x WN of 64 x 64
  constexpr int APW = 8 / NW;               // A blocks (16 rows) fetched per wave; B blocks: 2
  constexpr int B_BYTES = BN * 128;
  constexpr int STAGE = stage_bytes(BN);
  __shared__ __attribute__((aligned(1024))) uint8_t ring[S * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int l16 = lane & 15, g = lane >> 4;

  // tile order of the tile kernel: XCD-aware, then groups of 8 row tiles
  const int tiles_m = cdiv(p.M, BM), tiles_n = cdiv(p.N, BN);
  const int ntile = tiles_m * tiles_n;
  int bid = blockIdx.x;
  if ((ntile & 7) == 0) bid = (bid & 7) * (ntile >> 3) + (bid >> 3);
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int fm = (bid / per_group) * GM;
  const int gs = min(tiles_m - fm, GM);
  const int m0 = (fm + (bid % per_group) % gs) * BM;
  const int n0 = ((bid % per_group) / gs) * BN;
  const int batch = blockIdx.z, split = blockIdx.y;
  const uint8_t* A = (const uint8_t*)p.A + batch * p.sA;
  const uint8_t* B = (const uint8_t*)p.B + batch * p.sB;
  const int kg0 = split * (ksplit >> 7);                   // this split's first K group
  const int nk = min(p.K, (split + 1) * ksplit) / 128 - kg0;  // >= 1 (plan)

  // this wave's loads: A blocks APW wave .. +APW-1, B blocks 2 wave and 2 wave + 1, two
  // instructions of 8 rows each per block (rows past M and N re-read the last one); lane l reads
  // row 8 q + l / 8 of instruction q, the chunk that belongs at position l % 8 of that row
  const int lr = lane >> 3;
  auto src = [&](const uint8_t* base, int64_t ld, int r0, int lim, int q) {
    const int r = q * 8 + lr;
    return base + (int64_t)min(r0 + r, lim - 1) * ld + (((lane & 7) ^ chunk_swz(r)) << 4) + (int64_t)kg0 * 128;
  };
  const uint8_t* ga[APW][2];
#pragma unroll
  for (int a = 0; a < APW; ++a) {
    ga[a][0] = src(A, p.lda, m0 + (wave * APW + a) * 16, p.M, 0);
    ga[a][1] = src(A, p.lda, m0 + (wave * APW + a) * 16, p.M, 1);
  }
  const uint8_t* gb[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) gb[t] = src(B, p.ldb, n0 + wave * 32 + (t >> 1) * 16, p.N, t & 1);
  // the row scales: the waves of column 0 fetch rows wm * 64 + lane
  const bool scw = wn == 0;
  const float* gsa = p.a_scale + (int64_t)min(m0 + wm * 64 + lane, p.M - 1) * p.as_ld + kg0;
  auto issue = [&](int kt, int slot) {
    uint8_t* st = ring + slot * STAGE;
    const int64_t k0 = (int64_t)kt * 128;
#pragma unroll
    for (int a = 0; a < APW; ++a) {
      gl2lds16(ga[a][0] + k0, st + (wave * APW + a) * 2048);
      gl2lds16(ga[a][1] + k0, st + (wave * APW + a) * 2048 + 1024);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) gl2lds16(gb[t] + k0, st + A_BYTES + wave * 4096 + t * 1024);
    if (scw) gl2lds4(gsa + kt, st + A_BYTES + B_BYTES + wm * 256);
  };
  constexpr int LPS = 2 * APW + 4;  // loads per wave per stage, plus one on the scale waves

  // the wave's weight scales: its 64 columns lie in one 128-column block
  const float* gsb = p.b_scale + (int64_t)(min(n0 + wn * 64, p.N - 1) >> 7) * p.bs_ld + kg0;
  // operand addresses within a stage: row l16 of a block, chunk halves 2g and 2g + 1
  const int swz = chunk_swz(l16);
  const uint32_t oa0 = wm * 8192 + l16 * 128 + (((2 * g) ^ swz) << 4);
  const uint32_t oa1 = wm * 8192 + l16 * 128 + (((2 * g + 1) ^ swz) << 4);
  const uint32_t ob0 = A_BYTES + wn * 8192 + l16 * 128 + (((2 * g) ^ swz) << 4);
  const uint32_t ob1 = A_BYTES + wn * 8192 + l16 * 128 + (((2 * g + 1) ^ swz) << 4);
  const uint32_t osc = A_BYTES + B_BYTES + wm * 256 + g * 16;

  // acc: the scaled sum of the groups before the previous one; d, sp: the previous group's sums
  // and combined scales, added while this group's products run (a wave's scaling work then
  // overlaps its own MFMAs instead of following them; the order of the additions is unchanged)
  f32x4_t acc[4][4], d[4][4], sp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sp[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = d[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

#pragma unroll
  for (int t = 0; t < S - 1; ++t) issue(min(t, nk - 1), t);
  for (int t = 0; t < nk; ++t) {
    // this wave's part of stage t has landed (one stage of LPS or LPS + 1 loads may stay in flight) ...
    if (scw)
      wait_vmcnt<(S - 2) * (LPS + 1)>();
    else
      wait_vmcnt<(S - 2) * LPS>();
    // ... and every wave's; all are done with stage t - 1, whose slot is refilled next. A plain
    // barrier: __syncthreads' release fence would wait for every load in flight.
    asm volatile("s_barrier" ::: "memory");
    // past the last stage the same loads re-fetch it into a consumed slot, so every trip issues
    // the same loads and the wait counts stay exact
    issue(min(t + S - 1, nk - 1), (t + S - 1) % S);
    const uint32_t st = lds_addr(ring + (t % S) * STAGE);
    u32x4_t ra[8], rb[8];
    f32x4_t sc[4];
    float sbk;
    ring8_operands(st + oa0, st + oa1, st + ob0, st + ob1, st + osc, gsb + t, ra, rb, sc, sbk);
    i32x8_t bfr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bfr[j] = cat8(rb[2 * j], rb[2 * j + 1]);
    if constexpr (PREC) {
      // the same 32 codes per lane, widened to bf16 and summed in four steps of eight (the
      // group's sum is complete before it is scaled, as in the tile kernel)
      bf16x8_t bw[4][4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int s = 0; s < 4; ++s) bw[j][s] = widen8(bfr[j][2 * s], bfr[j][2 * s + 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const i32x8_t af = cat8(ra[2 * i], ra[2 * i + 1]);
        bf16x8_t aw[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) aw[s] = widen8(af[2 * s], af[2 * s + 1]);
        const f32x4_t sab = sc[i] * sbk;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4_t dd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 4; ++s) dd = mfma_bf16_16x16x32(aw[s], bw[j][s], dd);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][e] += dd[e] * sab[e];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const i32x8_t af = cat8(ra[2 * i], ra[2 * i + 1]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][e] += d[i][j][e] * sp[i][e];
          d[i][j] = mfma_fp8_16x16x128(af, bfr[j]);
        }
        sp[i] = sc[i] * sbk;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] += d[i][j][e] * sp[i][e];
  wait_vmcnt<0>();  // the tail's re-fetches have landed
  __syncthreads();  // every wave is done with the ring: it becomes the output staging
  static_assert(NW * 64 * LDW * 4 <= S * STAGE, "epilogue staging fits the ring");

  const int mw = m0 + wm * 64, nw = n0 + wn * 64;
  float* sw = reinterpret_cast<float*>(ring) + wave * (64 * LDW);
  if (splits > 1) {
    // K split: float32 partials of this split, whole 16-byte pieces of rows (N a multiple of 4)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) sw[(i * 16 + g * 4 + e) * LDW + j * 16 + l16] = acc[i][j][e];
    __syncthreads();
    float* part = p.part + ((int64_t)batch * splits + split) * p.M * p.N;
    const int lr4 = lane >> 4, lc4 = (lane & 15) * 4;
    const int n = nw + lc4;
    if (n < p.N) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int r = k * 4 + lr4, m = mw + r;
        if (m < p.M) *reinterpret_cast<f32x4_t*>(part + (int64_t)m * p.N + n) = *reinterpret_cast<const f32x4_t*>(sw + r * LDW + lc4);
      }
    }
    return;
  }
  if (p.epi == EPI_KVB) {
    // kv_b (fp16): a wave's 64 columns lie in one half of a head's 256. Content keys go through
    // LDS and leave as 16-byte pieces of K_nope rows; values and their fp16 residuals go straight
    // to V^T as 8-byte pieces (a lane's four accumulators are four consecutive keys of one feature)
    constexpr int LDH = 64 + 8;
    uint16_t* shi = reinterpret_cast<uint16_t*>(ring) + wave * (64 * LDH);
    const bool khalf = (nw & 255) < 128;
    if (khalf) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) shi[(i * 16 + g * 4 + e) * LDH + j * 16 + l16] = (uint16_t)pack_f16x2(acc[i][j][e], 0.f);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int mb = mw + i * 16 + g * 4;
          const int n = nw + j * 16 + l16;
          if (n >= p.N) continue;
          if (mb + 3 < p.M) {
            const f32x4_t v = acc[i][j];
            const uint32_t h01 = pack_f16x2(v[0], v[1]), h23 = pack_f16x2(v[2], v[3]);
            const int64_t at = (int64_t)((n >> 8) * 128 + (n & 255) - 128) * p.vt_ld + p.key_base + mb;
            *reinterpret_cast<u32x2_t*>(p.vt + at) = u32x2_t{h01, h23};
            if (p.vt_lo)
              *reinterpret_cast<u32x2_t*>(p.vt_lo + at) =
                  u32x2_t{pack_f16x2(v[0] - f16_lo(h01), v[1] - f16_hi(h01)), pack_f16x2(v[2] - f16_lo(h23), v[3] - f16_hi(h23))};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (mb + e < p.M) epi_store8(p, batch, mb + e, n, acc[i][j][e]);
          }
        }
    }
    __syncthreads();
    if (khalf) {
      const int lr8 = lane >> 3, lc8 = (lane & 7) * 8;
      const int n = nw + lc8;
      if (n < p.N) {
        const int64_t col = (n >> 8) * 128 + (n & 255);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int r = k * 8 + lr8, m = mw + r;
          if (m < p.M) st16(p.knope + (p.key_base + m) * 8192 + col, ld16(shi + r * LDH + lc8));
        }
      }
    }
    return;
  }

  // float32 results through LDS (a private region per wave), then whole 16-byte pieces of output
  // rows: bf16 rounds acc (+ residual) once, as the per-element epilogue does
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) sw[(i * 16 + g * 4 + e) * LDW + j * 16 + l16] = acc[i][j][e];
  __syncthreads();
  if (p.epi == EPI_F16) {
    const int lr = lane >> 3, lc = (lane & 7) * 8;
    const int n = nw + lc;
    if (n < p.N) {
      uint16_t* cb = (uint16_t*)p.C + batch * p.sC + n;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = k * 8 + lr, m = mw + r;
        if (m >= p.M) continue;
        const f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(sw + r * LDW + lc);
        const f32x4_t v1 = *reinterpret_cast<const f32x4_t*>(sw + r * LDW + lc + 4);
        st16(cb + (int64_t)m * p.ldc, u32x4_t{pack_f16x2(v0[0], v0[1]), pack_f16x2(v0[2], v0[3]),
                                              pack_f16x2(v1[0], v1[1]), pack_f16x2(v1[2], v1[3])});
      }
    }
  } else if (p.epi == EPI_BF16) {
    const int lr = lane >> 3, lc = (lane & 7) * 8;
    const int n = nw + lc;
    if (n < p.N) {
      uint16_t* cb = (uint16_t*)p.C + batch * p.sC + n;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = k * 8 + lr, m = mw + r;
        if (m >= p.M) continue;
        const f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(sw + r * LDW + lc);
        const f32x4_t v1 = *reinterpret_cast<const f32x4_t*>(sw + r * LDW + lc + 4);
        float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        if (p.resid) {
          const u32x4_t rr = ld16(p.resid + (int64_t)m * p.ldr + n);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v[2 * q] += bf_lo(rr[q]);
            v[2 * q + 1] += bf_hi(rr[q]);
          }
        }
        st16(cb + (int64_t)m * p.ldc, u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                              pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])});
      }
    }
  } else {
    const int lr = lane >> 4, lc = (lane & 15) * 4;
    const int n = nw + lc;
    if (n < p.N) {
      float* cf = (float*)p.C + batch * p.sC + n;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int r = k * 4 + lr, m = mw + r;
        if (m < p.M) *reinterpret_cast<f32x4_t*>(cf + (int64_t)m * p.ldc) = *reinterpret_cast<const f32x4_t*>(sw + r * LDW + lc);
      }
    }
  }
}

template <int TAG>
__global__ __launch_bounds__(256) void splitk_reduce8_kernel(GemmArgs p, int splits) {
  const int64_t mn = (int64_t)p.M * p.N;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.y;
  if (idx >= mn) return;
  const float* base = p.part + (int64_t)b * splits * mn + idx;
  float s = 0.f;
  for (int sp = 0; sp < splits; ++sp) s += base[sp * mn];
  epi_store8(p, b, (int)(idx / p.N), (int)(idx % p.N), s);
}

struct Plan8 {
  int kind;  // 0 wsplit, 1 tile 128 x 128, 2 tile 128 x 256, 3 tile 128 x 64
  int mt, kw, ysplit;
  int splits, ksplit;
  int tiles;
};

bool tag_precise(int tag) { return tag == TAG_QKVA || tag == TAG_KVB; }

// prec: the precise form keeps 128 x 128 tiles (two accumulator sets per lane do not fit the
// 128 x 256 tile's registers)
Plan8 plan_fp8(int M, int N, int K, int batch, int ysplit_max, bool prec, int parts_max) {
  Plan8 pl{};
  pl.splits = 1;
  pl.ksplit = K;
  pl.ysplit = 1;
  const int ngroups = K / 128;
  // streaming kernel up to 16 rows (64 when K is short), as for bf16; a K step is one 128 group
  if (M <= 16 || (M <= 64 && K <= 512)) {
    pl.kind = 0;
    pl.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    pl.tiles = cdiv(N, 16);
    while (pl.ysplit * 2 <= ysplit_max && pl.tiles * batch * pl.ysplit < 512 && ngroups / (pl.ysplit * 2) >= 8)
      pl.ysplit *= 2;
    int kw = 1;
    while (kw * 2 <= (pl.mt == 1 ? 16 : 8) && ngroups / (pl.ysplit * kw * 2) >= 6 &&
           pl.tiles * batch * pl.ysplit * kw * 2 <= 2048)
      kw *= 2;
    pl.kw = kw;
    return pl;
  }
  // Decode-sized M (up to 256 rows: one or two row tiles) takes 64-column tiles, twice the
  // workgroups of 128-column ones before any split of K.
  const bool big = !prec && M >= 1024 && N >= 1024;
  const bool narrow = M <= 256;
  pl.kind = big ? 2 : (narrow ? 3 : 1);
  pl.tiles = cdiv(M, 128) * cdiv(N, big ? 256 : (narrow ? 64 : 128));
  // K splits: as many as still fit one round of workgroups (two 128 x 64 or 128 x 128 tile
  // workgroups per CU: 512), and float32 partials (written and read back) adding at most the
  // operand bytes (codes) in traffic. Measured at 128 rows (decode of 128 sequences), forced split
  // counts 1 .. 16: o_proj best at 4 (38 us; 5 splits = 560 workgroups, a second round: 54 us),
  // q_b unsplit (19 us; 3 splits 27), q_a|kv_a 6-7 (19-20 us).
  int splits = 1;
  const int wgs = pl.tiles * batch;
  if (wgs < 256) splits = std::max(1, 512 / wgs);
  const int64_t operand_bytes = (int64_t)batch * ((int64_t)M * K + (int64_t)N * K);
  const int64_t part_bytes_per_split = 8 * (int64_t)batch * M * N;
  splits = (int)std::min<int64_t>(splits, std::max<int64_t>(1, operand_bytes / part_bytes_per_split));
  splits = std::max(1, std::min(splits, ngroups));
  const int per = cdiv(ngroups, splits);
  pl.ksplit = per * 128;
  pl.splits = cdiv(ngroups, per);
  // a consumer that adds up to parts_max parts takes the split partials straight from C: no
  // reduction launch (the sums are the reduction's: parts added in split order)
  if (pl.splits > 1 && pl.splits <= parts_max) pl.ysplit = pl.splits;
  return pl;
}

// The parts a call's consumer adds, for the K-split tile kernels: float32 output of one batch with
// its parts packed (C rows N floats apart, parts M N floats apart); otherwise none.
int parts_max_of(const GemmArgs& a) {
  return a.epi == EPI_F32 && a.batch == 1 && a.ldc == a.N && a.c_split_stride == (int64_t)a.M * a.N ? a.ysplit_max : 1;
}

template <int MT, int TAG, bool PREC>
void launch_fp8_wsplit(const GemmArgs& a, const Plan8& pl, hipStream_t s) {
  dim3 grid(pl.tiles, pl.ysplit, a.batch);
  switch (pl.kw) {
    case 1: hipLaunchKernelGGL((gemm_fp8_wsplit_kernel<MT, 1, TAG, PREC>), grid, dim3(64), 0, s, a); break;
    case 2: hipLaunchKernelGGL((gemm_fp8_wsplit_kernel<MT, 2, TAG, PREC>), grid, dim3(128), 0, s, a); break;
    case 4: hipLaunchKernelGGL((gemm_fp8_wsplit_kernel<MT, 4, TAG, PREC>), grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL((gemm_fp8_wsplit_kernel<MT, 8, TAG, PREC>), grid, dim3(512), 0, s, a); break;
    default:
      if constexpr (MT == 1)
        hipLaunchKernelGGL((gemm_fp8_wsplit_kernel<MT, 16, TAG, PREC>), grid, dim3(1024), 0, s, a);
      break;
  }
}

// The ring kernel's layout and epilogue requirements
bool ring8_ok(const GemmArgs& a) {
  auto al16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  if (a.K < 128 || (a.lda & 15) || (a.ldb & 15) || (a.sA & 15) || (a.sB & 15) || !al16(a.A) ||
      !al16(a.B) || !al16(a.C))
    return false;
  if (a.epi == EPI_BF16)
    return (a.N & 7) == 0 && (a.ldc & 7) == 0 && (a.sC & 7) == 0 && (!a.resid || (al16(a.resid) && (a.ldr & 7) == 0));
  if (a.epi == EPI_F16) return (a.N & 7) == 0 && (a.ldc & 7) == 0 && (a.sC & 7) == 0;
  if (a.epi == EPI_KVB) {
    auto al8 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 7) == 0; };
    return a.batch == 1 && (a.key_base & 3) == 0 && (a.vt_ld & 3) == 0 && (a.N & 7) == 0 && al16(a.knope) &&
           al8(a.vt) && (!a.vt_lo || al8(a.vt_lo));
  }
  return a.epi == EPI_F32 && (a.N & 3) == 0 && (a.ldc & 3) == 0 && (a.sC & 3) == 0;
}

template <int TAG, bool PREC>
void launch_fp8_tagged(const GemmArgs& a, const Plan8& pl, hipStream_t s) {
  if (pl.kind == 0) {
    if (pl.mt == 1) launch_fp8_wsplit<1, TAG, PREC>(a, pl, s);
    else if (pl.mt == 2) launch_fp8_wsplit<2, TAG, PREC>(a, pl, s);
    else launch_fp8_wsplit<4, TAG, PREC>(a, pl, s);
    return;
  }
  dim3 grid(pl.tiles, pl.splits, a.batch);
  // The ring kernel: at prefill sizes one 128 x 256 tile per CU (the precise form when it has at
  // least one round of workgroups), at decode sizes (up to 256 rows) 128 x 64 tiles with the
  // plan's K split, native form only (measured at 128 rows: q_b 22.7 -> 16.3 us, o_proj 31.1 ->
  // 28.7 us; the precise q_a|kv_a 14.0 -> 17.1 us, its one wave per SIMD left waiting on the
  // chained bf16 products); otherwise the register-staged tile kernel.
  bool ring = false;
  if (ring8_ok(a)) {
    const int rt = cdiv(a.M, ring8::BM) * cdiv(a.N, 256);
    if (pl.splits == 1 && (PREC ? (pl.kind == 1 && a.M >= 1024 && a.N >= 1024 && rt * a.batch >= 256) : pl.kind == 2)) {
      hipLaunchKernelGGL((gemm_fp8_ring_kernel<TAG, PREC, 256>), dim3(rt, 1, a.batch), dim3(512), 0, s, a, 1, a.K);
      return;
    }
    if constexpr (!PREC) {
      // 128 columns (one workgroup of 4 waves per CU, half the A re-reads per output) while that
      // still gives 192 workgroups: o_proj at 128 rows 28.7 -> 23.9 us with the plan's 4 splits
      const int t128 = cdiv(a.M, ring8::BM) * cdiv(a.N, 128);
      if (pl.kind == 3 && t128 * pl.splits * a.batch >= 192) {
        hipLaunchKernelGGL((gemm_fp8_ring_kernel<TAG, PREC, 128>), dim3(t128, pl.splits, a.batch), dim3(256), 0, s, a,
                           pl.splits, pl.ksplit);
        ring = true;
      } else if (pl.kind == 3) {
        hipLaunchKernelGGL((gemm_fp8_ring_kernel<TAG, PREC, 64>), grid, dim3(128), 0, s, a, pl.splits, pl.ksplit);
        ring = true;
      }
    }
  }
  if (ring) {
  } else if (pl.kind == 1)
    hipLaunchKernelGGL((gemm_fp8_tile_kernel<128, 128, 2, 2, TAG, PREC>), grid, dim3(256), 0, s, a, pl.splits,
                       pl.ksplit);
  else if (pl.kind == 3)
    hipLaunchKernelGGL((gemm_fp8_tile_kernel<128, 64, 2, 2, TAG, PREC>), grid, dim3(256), 0, s, a, pl.splits,
                       pl.ksplit);
  else if constexpr (!PREC)
    hipLaunchKernelGGL((gemm_fp8_tile_kernel<128, 256, 2, 4, TAG, PREC>), grid, dim3(512), 0, s, a, pl.splits,
                       pl.ksplit);
  if (pl.splits > 1 && pl.ysplit == 1) {
    if (reduce_vec_ok(a)) {
      dim3 rgrid((unsigned)(((int64_t)a.M * a.N / 4 + 255) / 256), a.batch);
      hipLaunchKernelGGL((splitk_reduce_vec_kernel<TAG, false>), rgrid, dim3(256), 0, s, a, pl.splits);
    } else {
      dim3 rgrid((unsigned)(((int64_t)a.M * a.N + 255) / 256), a.batch);
      hipLaunchKernelGGL((splitk_reduce8_kernel<TAG>), rgrid, dim3(256), 0, s, a, pl.splits);
    }
  }
}

}  // namespace

int64_t gemm_fp8_part_floats(int M, int N, int K, int batch) {
  int64_t mx = 0;
  for (bool prec : {false, true}) {
    const Plan8 pl = plan_fp8(M, N, K, batch, 1, prec, 1);
    if (pl.splits > 1) mx = std::max(mx, (int64_t)pl.splits * batch * M * N);
  }
  return mx;
}

int gemm_fp8_ysplit(const GemmArgs& a) {
  return plan_fp8(a.M, a.N, a.K, a.batch, a.epi == EPI_F32 ? a.ysplit_max : 1, tag_precise(a.tag), parts_max_of(a)).ysplit;
}

hipError_t gemm_fp8(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.K % 128 != 0 || !a.a_scale || !a.b_scale) return hipErrorInvalidValue;
  const Plan8 pl =
      plan_fp8(a.M, a.N, a.K, a.batch, a.epi == EPI_F32 ? a.ysplit_max : 1, tag_precise(a.tag), parts_max_of(a));
  const bool parts_in_c = pl.kind != 0 && pl.ysplit > 1;
  if (pl.splits > 1 && !parts_in_c && (int64_t)pl.splits * a.batch * a.M * a.N > a.part_cap) return hipErrorInvalidValue;
  GemmArgs b = a;
  if (parts_in_c) b.part = (float*)a.C;  // split s writes part s of C
  // q_a|kv_a and kv_b: precise; q_b, o_proj (and untagged test calls): native
  switch (a.tag) {
    case TAG_QKVA: launch_fp8_tagged<TAG_QKVA, true>(b, pl, s); break;
    case TAG_QB: launch_fp8_tagged<TAG_QB, false>(b, pl, s); break;
    case TAG_KVB: launch_fp8_tagged<TAG_KVB, true>(b, pl, s); break;
    case TAG_OPROJ: launch_fp8_tagged<TAG_OPROJ, false>(b, pl, s); break;
    default: launch_fp8_tagged<TAG_NONE, false>(b, pl, s); break;
  }
  return hipGetLastError();
}

}  // namespace mla_k
