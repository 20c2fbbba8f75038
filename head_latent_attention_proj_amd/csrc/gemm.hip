// bf16 GEMMs (MFMA tiles; VALU for one or two rows) for the five MLA projections and the per-head
// absorption products.
//
// C[b] = A[b] * B[b]^T with A [M, K] and B [N, K] both K-contiguous: nn.Linear keeps its weight
// [out, in] ("Key content up-projection" page, Parameters), so every projection y = x W^T is
// this "NT" form and both MFMA operands load 16 contiguous bytes per lane.
//
// Kernels:
//   * gemm_tile   -- prefill-sized M: BM x BN workgroup tile staged through LDS (double
//                    buffered, XOR-swizzled 128-byte rows so stores and 16-byte fragment reads
//                    are bank-conflict free), 16x16x32 bf16 MFMA, XCD-aware grouped tile order.
//                    Optional split-K.
//   * gemm_skinny -- 16 < M <= 64 with K >= 512: a ring of LDS stages filled by whole-row
//                    direct-to-LDS loads into swizzled rows, several stages in flight per workgroup.
//   * gemm_wsplit -- other decode-sized M (<= 64): operands go straight from global memory into
//                    MFMA fragments; the K range of a 16*NT-column tile is split across the waves
//                    of one workgroup (each wave streams its own contiguous slice of the weight
//                    rows), and the waves' partial tiles are summed through LDS in a fixed order.
//                    No cross-workgroup synchronisation, no float atomics: deterministic.
//   * gemm_head   -- per-head batched products up to 256 rows with K of 128 or 512 (optionally
//                    paired high / residual rows summed in the epilogue, with o_proj's FP8
//                    input quantiser applied there).
//   * gemm_rows   -- one or two rows of A: each load of a wave reads 1 KB (or 256 B) runs of
//                    single weight rows, dot products on the VALU with x staged in LDS.
//   Split-K of the tile kernel (few tiles, small M) writes fp32 partials and a separate
//   reduction kernel sums them in a fixed order.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "norm_dev.h"
#include "splitk.h"

namespace mla_k {

namespace {

MLA_DEV void epi_store(const GemmArgs& p, int b, int m, int n, float v) {
  if (p.c_scale) v *= p.c_scale[b * p.cs_stride + (n >> 7)];
  if (p.epi == EPI_F32) {
    ((float*)p.C)[b * p.sC + (int64_t)m * p.ldc + n] = v;
  } else if (p.epi == EPI_BF16) {
    if (p.resid) v += bf2f(p.resid[(int64_t)m * p.ldr + n]);
    ((uint16_t*)p.C)[b * p.sC + (int64_t)m * p.ldc + n] = f2bf(v);
  } else {  // EPI_KVB: per head [128 content-key | 128 value] features
    const int h = n >> 8, r = n & 255;
    const int64_t key = p.key_base + m;
    if (r < 128)
      p.knope[key * 8192 + h * 128 + r] = f2bf(v);
    else
      p.vt[(int64_t)(h * 128 + r - 128) * p.vt_ld + key] = f2bf(v);
  }
}

// ------------------------------------------------------------------------------------------
// Tile kernel
// ------------------------------------------------------------------------------------------
// TAG only names the projection (distinct kernel symbols per stage in traces); the code is shared.
template <int BM, int BN, int WM, int WN, int TAG>
__global__ __launch_bounds__(WM* WN * 64) void gemm_tile_kernel(GemmArgs p, int splits, int ksplit) {
  constexpr int NT = WM * WN * 64;
  constexpr int BK = 64;
  // Stage rows of 64 features (128 bytes) without padding; 16-byte chunk c of row r is kept at
  // position c ^ ((r / 2) % 8). The stores (8 lanes per row) and the operand reads (row l16, chunk
  // 4s + g) then meet distinct banks for every 16 lanes of an instruction; padded 144-byte rows left
  // the stores of two consecutive rows on four shared banks.
  constexpr int LDK = BK;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 16, TN = WTN / 16;
  constexpr int CPR = BK / 8;
  constexpr int RPP = NT / CPR;
  constexpr int AP = BM / RPP, BP = BN / RPP;
  static_assert(BM % RPP == 0 && BN % RPP == 0, "tile rows must be a multiple of rows per pass");
  constexpr int SMEM = std::max(2 * (BM + BN) * LDK, WM * WN * WTM * (WTN + 8));  // tiles / epilogue staging
  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int l16 = lane & 15, g = lane >> 4;

  const int tiles_m = cdiv(p.M, BM), tiles_n = cdiv(p.N, BN);
  const int ntile = tiles_m * tiles_n;
  int bid = blockIdx.x;
  // Workgroups are dealt round-robin to the 8 XCDs; renumber so that consecutive tile ids
  // (which share A rows / B columns through the grouped order below) sit on one XCD's L2.
  if ((ntile & 7) == 0) bid = (bid & 7) * (ntile >> 3) + (bid >> 3);
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int fm = (bid / per_group) * GM;
  const int gs = min(tiles_m - fm, GM);
  const int tm = fm + (bid % per_group) % gs;
  const int tn = (bid % per_group) / gs;
  const int m0 = tm * BM, n0 = tn * BN;
  const int batch = blockIdx.z, split = blockIdx.y;

  const uint16_t* A = (const uint16_t*)p.A + batch * p.sA;
  const uint16_t* B = (const uint16_t*)p.B + batch * p.sB;

  const int lr = tid / CPR, lc = (tid % CPR) * 8;
  static_assert(CPR == 8 && RPP % 16 == 0, "swizzle: 8 chunks per row, passes of whole 16-row groups");
  const int lcs = (((tid % CPR) ^ ((lr >> 1) & 7)) << 3);  // this thread's chunk, swizzled
  const uint16_t* ga[AP];
  const uint16_t* gb[BP];
#pragma unroll
  for (int i = 0; i < AP; ++i) ga[i] = A + (int64_t)min(m0 + i * RPP + lr, p.M - 1) * p.lda + lc;
#pragma unroll
  for (int i = 0; i < BP; ++i) gb[i] = B + (int64_t)min(n0 + i * RPP + lr, p.N - 1) * p.ldb + lc;

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
  };
  auto sstore = [&](int buf) {
    uint16_t* sa = smem + buf * (BM + BN) * LDK;
    uint16_t* sb = sa + BM * LDK;
#pragma unroll
    for (int i = 0; i < AP; ++i) st16(sa + (i * RPP + lr) * LDK + lcs, ra[i]);
#pragma unroll
    for (int i = 0; i < BP; ++i) st16(sb + (i * RPP + lr) * LDK + lcs, rb[i]);
  };

  if (nk > 0) {
    gload(kb);
    sstore(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kb + (kt + 1) * BK);
    const uint16_t* sa = smem + cur * (BM + BN) * LDK + (wm * WTM + l16) * LDK;
    const uint16_t* sb = smem + cur * (BM + BN) * LDK + BM * LDK + (wn * WTN + l16) * LDK;
    const int swz = (l16 >> 1) & 7;  // the operand rows' swizzle (16-row tiles keep it)
#pragma unroll
    for (int s = 0; s < BK / 32; ++s) {
      const int cs = ((4 * s + g) ^ swz) << 3;
      bf16x8_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = as_bf16x8(ld16(sa + i * 16 * LDK + cs));
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = as_bf16x8(ld16(sb + j * 16 * LDK + cs));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_bf16_16x16x32(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  if (splits == 1) {
    if (p.epi == EPI_BF16 && !p.resid && !p.c_scale && (p.N & 7) == 0 && (p.ldc & 7) == 0 && (p.sC & 7) == 0 &&
        (reinterpret_cast<uintptr_t>(p.C) & 15) == 0) {
      // bf16 output through LDS: each wave writes its WTM x WTN results to a private region (the
      // tile buffers are free after the loop's last barrier), then stores whole 16-byte pieces of
      // output rows, eight lanes per 128-byte row segment, instead of one 2-byte store per value
      constexpr int LDW = WTN + 8;
      static_assert(WM * WN * WTM * LDW <= SMEM, "epilogue staging fits the tile buffers");
      uint16_t* sw = smem + wave * (WTM * LDW);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) sw[(i * 16 + g * 4 + e) * LDW + j * 16 + l16] = f2bf(acc[i][j][e]);
      __syncthreads();
      const int lr8 = lane >> 3, lc8 = (lane & 7) * 8;
      const int n = n0 + wn * WTN + lc8;
      if (n < p.N) {  // N is a multiple of 8: a chunk is whole or wholly outside
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
    if (p.epi == EPI_KVB && (p.key_base & 3) == 0 && !p.c_scale && (p.N & 7) == 0) {
      // kv_b: a wave's 64 columns lie in one half of a head's 256 (wave-uniform). Content keys
      // go through LDS as for bf16 outputs and leave as 16-byte pieces of K_nope rows; values go
      // straight to V^T, a lane's four accumulators (four consecutive keys of one feature) as one
      // 8-byte store. Every wave reaches the barrier.
      static_assert(WTN == 64 && WM * WN * WTM * (WTN + 8) <= SMEM, "kv_b epilogue layout");
      constexpr int LDW = WTN + 8;
      uint16_t* sw = smem + wave * (WTM * LDW);
      const int nw0 = n0 + wn * WTN;
      const bool khalf = (nw0 & 255) < 128;
      if (khalf) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) sw[(i * 16 + g * 4 + e) * LDW + j * 16 + l16] = f2bf(acc[i][j][e]);
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
              *reinterpret_cast<u32x2_t*>(p.vt + (int64_t)((n >> 8) * 128 + (n & 255) - 128) * p.vt_ld + p.key_base + mb) =
                  u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (mb + e < p.M) epi_store(p, batch, mb + e, n, acc[i][j][e]);
            }
          }
      }
      __syncthreads();
      if (khalf) {
        const int lr8 = lane >> 3, lc8 = (lane & 7) * 8;
        const int n = nw0 + lc8;
        if (n < p.N) {
          uint16_t* kb0 = p.knope + (n >> 8) * 128 + (n & 255);
#pragma unroll
          for (int k = 0; k < WTM / 8; ++k) {
            const int r = k * 8 + lr8;
            const int m = m0 + wm * WTM + r;
            if (m < p.M) st16(kb0 + (p.key_base + m) * 8192, ld16(sw + r * LDW + lc8));
          }
        }
      }
      return;
    }
    if (p.epi == EPI_KVB && (p.key_base & 3) == 0) {
      // kv_b with an output scale: V^T as 8-byte pieces as above, content keys value by value
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int mb = m0 + wm * WTM + i * 16 + g * 4;
          const int n = n0 + wn * WTN + j * 16 + l16;
          if (n >= p.N) continue;
          if ((n & 255) >= 128 && mb + 3 < p.M) {
            f32x4_t v = acc[i][j];
            if (p.c_scale) v *= p.c_scale[batch * p.cs_stride + (n >> 7)];
            *reinterpret_cast<u32x2_t*>(p.vt + (int64_t)((n >> 8) * 128 + (n & 255) - 128) * p.vt_ld + p.key_base + mb) =
                u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (mb + e < p.M) epi_store(p, batch, mb + e, n, acc[i][j][e]);
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
          if (m < p.M && n < p.N) epi_store(p, batch, m, n, acc[i][j][e]);
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

// Sum of the split-K partials in split order, then the epilogue. One thread per output.
template <int TAG>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs p, int splits) {
  const int64_t mn = (int64_t)p.M * p.N;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.y;
  if (idx >= mn) return;
  const float* base = p.part + (int64_t)b * splits * mn + idx;
  float s = 0.f;
  for (int sp = 0; sp < splits; ++sp) s += base[sp * mn];
  epi_store(p, b, (int)(idx / p.N), (int)(idx % p.N), s);
}

template <int TAG>
void launch_reduce(const GemmArgs& a, int splits, hipStream_t s) {
  if (reduce_vec_ok(a)) {
    dim3 rgrid((unsigned)(((int64_t)a.M * a.N / 4 + 255) / 256), a.batch);
    hipLaunchKernelGGL((splitk_reduce_vec_kernel<TAG, true>), rgrid, dim3(256), 0, s, a, splits);
  } else {
    dim3 rgrid((unsigned)(((int64_t)a.M * a.N + 255) / 256), a.batch);
    hipLaunchKernelGGL((splitk_reduce_kernel<TAG>), rgrid, dim3(256), 0, s, a, splits);
  }
}

// ------------------------------------------------------------------------------------------
// Decode-sized M: one workgroup per 16*NT-column tile, K split across its KW waves
// ------------------------------------------------------------------------------------------
// Each wave streams its own contiguous slice of K for all MT*16 rows of A and NT*16 weight rows
// straight from global memory into MFMA fragments, U 32-wide K steps per pipeline stage, two
// stages in flight. A wave reads MT A fragments and NT weight fragments per step, so for M > 16
// a tile of NT > 1 columns keeps the (cached) activation reads near the weight stream instead
// of MT times it. The waves' partial tiles are then summed through LDS by halving (wave w adds
// wave w + KW/2, then w + KW/4, ...): a fixed order, so the result is deterministic.
template <int MT, int NT, int U, int KW, int TAG>
__global__ __launch_bounds__(KW * 64) void gemm_wsplit_kernel(GemmArgs p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int l16 = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16 * NT;
  const int batch = blockIdx.z;
  const uint16_t* A = (const uint16_t*)p.A + batch * p.sA;
  const uint16_t* B = (const uint16_t*)p.B + batch * p.sB;
  // K steps of this workgroup (blockIdx.y of gridDim.y splits), then of this wave
  const int ysteps = cdiv(p.K >> 5, (int)gridDim.y);
  const int y0 = blockIdx.y * ysteps;
  const int y1 = min(p.K >> 5, y0 + ysteps);
  const int spw = cdiv(y1 - y0, KW);
  const int s0 = y0 + wave * spw;
  const int s1 = min(y1, s0 + spw);

  // lane (l16, g): row l16 of each 16-row tile, features g*8 .. g*8+7 of each 32-wide step
  const uint16_t* pa[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) pa[i] = A + (int64_t)min(i * 16 + l16, p.M - 1) * p.lda + g * 8;
  const uint16_t* pb[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) pb[j] = B + (int64_t)min(n0 + j * 16 + l16, p.N - 1) * p.ldb + g * 8;

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (s0 < s1) {
    // Loads are unconditional (steps past the wave's range re-read its last step) so the
    // next stage's loads stay in flight while the current stage multiplies; a step past the
    // range multiplies zero weight fragments instead of being branched around.
    u32x4_t ca[U][MT], cb[U][NT];
    auto load = [&](int s, u32x4_t (&ra)[U][MT], u32x4_t (&rb)[U][NT]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int st = min(s + u, s1 - 1) * 32;
#pragma unroll
        for (int j = 0; j < NT; ++j) rb[u][j] = ld16(pb[j] + st);
#pragma unroll
        for (int i = 0; i < MT; ++i) ra[u][i] = ld16(pa[i] + st);
      }
    };
    load(s0, ca, cb);
    for (int s = s0; s < s1; s += U) {
      u32x4_t na[U][MT], nb[U][NT];
      load(min(s + U, s1 - 1), na, nb);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const u32x4_t zero = {0u, 0u, 0u, 0u};
        const bool live = s + u < s1;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const u32x4_t bw = live ? cb[u][j] : zero;
#pragma unroll
          for (int i = 0; i < MT; ++i) acc[i][j] = mfma_bf16_16x16x32(as_bf16x8(ca[u][i]), as_bf16x8(bw), acc[i][j]);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int j = 0; j < NT; ++j) cb[u][j] = nb[u][j];
#pragma unroll
        for (int i = 0; i < MT; ++i) ca[u][i] = na[u][i];
      }
    }
  }

  // fixed-order sum of the waves' partial tiles through LDS, halving the live waves each round
  if constexpr (KW > 1) {
    __shared__ float red[(KW / 2) * MT * NT * 4 * 64];
#pragma unroll
    for (int half = KW / 2; half >= 1; half >>= 1) {
      if (wave >= half && wave < 2 * half) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[((((wave - half) * MT + i) * NT + j) * 4 + e) * 64 + lane] = acc[i][j][e];
      }
      __syncthreads();
      if (wave < half) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] += red[(((wave * MT + i) * NT + j) * 4 + e) * 64 + lane];
      }
      __syncthreads();
    }
    if (wave != 0) return;
  }
  if (gridDim.y > 1) {  // partial sum of this K split (EPI_F32 only; the consumer adds the parts)
    float* C = (float*)p.C + blockIdx.y * p.c_split_stride + batch * p.sC;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = i * 16 + g * 4 + e, n = n0 + j * 16 + l16;
          if (m < p.M && n < p.N) C[(int64_t)m * p.ldc + n] = acc[i][j][e];
        }
    return;
  }
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = i * 16 + g * 4 + e, n = n0 + j * 16 + l16;
        if (m < p.M && n < p.N) epi_store(p, batch, m, n, acc[i][j][e]);
      }
}

// ------------------------------------------------------------------------------------------
// M <= 2: whole weight-row segments per load, dot products on the VALU
// ------------------------------------------------------------------------------------------
// With one or two activation rows the product is a pure weight stream, and the MFMA fragment
// layout (16 rows x 64 bytes per load) is not the best way to read it. Here one load of a wave
// covers RPI weight rows with 64/RPI lanes each, so a row segment is 1 KB (RPI = 1, K a multiple
// of 512) or 256 B (RPI = 4); x (this workgroup's K range) sits in LDS. Each wave owns `rw`
// groups of RPI rows, streams their segments in two sets of U loads, and sums a row over its lanes
// once its K range is done. The K range may be split over gridDim.y workgroups (EPI_F32 only:
// split y writes its partial sums to C + y * c_split_stride). Sums run in a fixed order.
MLA_DEV float dot8_bf16(const u32x4_t& w, const u32x4_t& x, float acc) {
  // whole-vector shuffles: element-wise bit casts of u32x4 lanes were miscompiled (every
  // element read as the first)
  const bf16x8_t a = as_bf16x8(w), b = as_bf16x8(x);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 0, 1), __builtin_shufflevector(b, b, 0, 1), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 2, 3), __builtin_shufflevector(b, b, 2, 3), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 4, 5), __builtin_shufflevector(b, b, 4, 5), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 6, 7), __builtin_shufflevector(b, b, 6, 7), acc, false);
  return acc;
}

constexpr int ROWS_LDS_MAX = 32768;  // bytes of x a rows workgroup stages

// Raw (stride 0) buffer descriptor over `bytes` bytes: a load at an offset past the end returns
// zero without touching memory, which lets a wave issue a fixed number of loads whatever its
// share of the rows. Third descriptor word: 32-bit data format, as the gfx9 family requires.
MLA_DEV __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
MLA_DEV u32x4_t buffer_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// QNORM (the q_b projection at decode, bf16): x is not read from A but built here as the query
// latent RMSNorm of the fused q_a | kv_a sums (na.cqkv), the same in every workgroup; workgroup
// (0, 0) also writes the tokens' cache entries (latent RMSNorm, rotated shared key) and
// advances their lengths. This replaces the norm kernel between q_a | kv_a and q_b.
template <int RPI, int MT, int U, int TAG, bool QNORM>
__global__ __launch_bounds__(256) void gemm_rows_kernel(GemmArgs p, int rw, NormArgs na) {
  constexpr int LPR = 64 / RPI;     // lanes per row
  constexpr int SEG = LPR * 8;      // K elements of a row segment
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane / LPR, j = lane % LPR;
  const int batch = blockIdx.z;
  const int ks = p.K / (int)gridDim.y, k0 = blockIdx.y * ks;
  // operand windows of this batch (the plan keeps both under 2 GiB)
  const uint32_t a_bytes = (uint32_t)(((int64_t)(p.M - 1) * p.lda + p.K) * 2);
  const uint32_t b_bytes = (uint32_t)(((int64_t)(p.N - 1) * p.ldb + p.K) * 2);
  const __amdgpu_buffer_rsrc_t ra_src = buffer_rsrc((const uint16_t*)p.A + batch * p.sA, a_bytes);
  const __amdgpu_buffer_rsrc_t rb_src = buffer_rsrc((const uint16_t*)p.B + batch * p.sB, b_bytes);
  const int nseg = ks / SEG;
  const int row0 = (blockIdx.x * 4 + wave) * rw * RPI;
  const int total = rw * nseg;  // loads of this wave
  // next load (lg = row group, ls = segment). The pipeline below issues whole register sets;
  // loads past the wave's last one point past the buffer end (zeros, no memory access) and
  // their products are never stored. Selects, not branches, between the loads.
  int lg = 0, ls = 0, issued = 0;
  auto next = [&]() -> u32x4_t {
    const bool live = issued < total;
    const int row = min(row0 + lg * RPI + r, p.N - 1);
    const uint32_t off = live ? (uint32_t)(row * p.ldb + k0 + ls * SEG + j * 8) * 2u : b_bytes;
    ++issued;
    const bool wrap = ls + 1 == nseg;
    lg = live && wrap ? lg + 1 : lg;
    ls = live ? (wrap ? 0 : ls + 1) : ls;
    return buffer_ld16(rb_src, off);
  };
  // two register sets of U loads: one is multiplied while the other is in flight
  u32x4_t ra[U], rb[U];
#pragma unroll
  for (int u = 0; u < U; ++u) ra[u] = next();
  // x into LDS behind the first weight loads: every thread issues all of its (at most
  // ROWS_LDS_MAX / 16 / 256) 16-byte loads before the first store
  __shared__ float red[4];
  if constexpr (QNORM) {
#pragma unroll
    for (int m = 0; m < MT; ++m) q_norm_bf16(na, min(m, p.M - 1), xs + m * ks, red);
  } else {
    constexpr int XC = ROWS_LDS_MAX / 16 / 256;
    const int cpr = ks / 8, nc = MT * cpr;
    u32x4_t xv[XC];
#pragma unroll
    for (int i = 0; i < XC; ++i) {
      const int c = (int)threadIdx.x + 256 * i;
      const int m = c / cpr, cc = c - m * cpr;
      xv[i] = buffer_ld16(ra_src, c < nc ? (uint32_t)(m * p.lda + k0 + cc * 8) * 2u : a_bytes);
    }
#pragma unroll
    for (int i = 0; i < XC; ++i) {
      const int c = (int)threadIdx.x + 256 * i;
      if (c < nc) st16(xs + c * 8, xv[i]);
    }
  }
  __syncthreads();
  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0.f;
  int cg = 0, cs = 0;  // row group and segment being multiplied
  auto consume = [&](const u32x4_t (&rr)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] = dot8_bf16(rr[u], ld16(xs + m * ks + cs * SEG + j * 8), acc[m]);
      if (++cs == nseg) {  // row group done: sum each row over its lanes
        const int n = row0 + cg * RPI + r;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          float v = acc[m];
#pragma unroll
          for (int o = LPR / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
          acc[m] = 0.f;
          if (j == 0 && cg < rw && n < p.N && m < p.M) {
            if (gridDim.y > 1)
              ((float*)p.C)[blockIdx.y * p.c_split_stride + batch * p.sC + (int64_t)m * p.ldc + n] = v;
            else
              epi_store(p, batch, m, n, v);
          }
        }
        cs = 0;
        ++cg;
      }
    }
  };
  for (int it = 0; it < total; it += 2 * U) {
#pragma unroll
    for (int u = 0; u < U; ++u) rb[u] = next();
    consume(ra);
#pragma unroll
    for (int u = 0; u < U; ++u) ra[u] = next();
    consume(rb);
  }
  if constexpr (QNORM) {
    if (blockIdx.x == 0 && blockIdx.y == 0) {
      __shared__ float kraw[mla_dims::ROPE];
      for (int t = 0; t < na.n_tokens; ++t) kv_norm_rope_append_bf16(na, t, red, kraw);
    }
  }
}

// ------------------------------------------------------------------------------------------
// Per-head products at M <= 256 with short K (decode W_UK absorb and W_UV)
// ------------------------------------------------------------------------------------------
// Workgroup = (head, 16 NWV output columns, 64-row chunk of x); the chunk x_h[m0 .. m0+63] (K =
// 32 KS) is staged in LDS once and every wave streams 16 weight rows over the whole K with all of
// its loads issued up front; 16x16x32 MFMA, A fragments from LDS (rows >= M are copies of row
// M - 1 and never stored). With pair_rows, a workgroup takes 32 rows and their 32 residual rows
// (tile rows 0..31 and 32..63) and stores the sums.
template <int KS, int NWV, int TAG>
__global__ __launch_bounds__(64 * NWV) void gemm_head_kernel(GemmArgs p) {
  // padded LDS row (32 bytes): the A fragment reads (row l16, 16 bytes at 16 g) meet distinct banks
  // under gfx950's grouping of a 16-byte read (16 lanes per cycle: the quads of a half-wave with one
  // parity of their low three index bits); a 16-byte pad left them 2-way conflicted
  constexpr int LDX = KS * 32 + 16;
  __shared__ __attribute__((aligned(16))) uint16_t xs[64 * LDX];
  const int batch = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.y * (16 * NWV) + wave * 16;
  const bool pair = p.pair_rows > 0;
  const int m0 = blockIdx.z * (pair ? 32 : 64);
  const uint16_t* A = (const uint16_t*)p.A + batch * p.sA + (int64_t)m0 * p.lda;
  const int mrows = pair ? min(32, p.pair_rows - m0) : min(64, p.M - m0);
  // A row (relative to m0) of tile row r
  auto arow = [&](int r) -> int64_t {
    if (!pair) return min(r, mrows - 1);
    return min(r & 31, mrows - 1) + (r >= 32 ? p.pair_rows : 0);
  };
  const uint16_t* B = (const uint16_t*)p.B + batch * p.sB;
  u32x4_t wb[KS];
  const uint16_t* wr = B + (int64_t)min(n0 + l16, p.N - 1) * p.ldb + 8 * g;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) wb[ks] = ld16(wr + 32 * ks);
  {
    constexpr int CH = KS * 4;              // 16-byte chunks per row
    constexpr int NT = 64 * NWV;
    constexpr int PER = 64 * CH / NT;       // chunks per thread
    u32x4_t xv[PER];
    // both rows of a pair as bf16 high = bf16(v) and residual = bf16(v - high) of a float32 v
    auto split8 = [&](const float (&v)[8], u32x4_t& hi, u32x4_t& lo) {
      uint32_t wh[4], wl[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint16_t h0 = f2bf(v[2 * j]), h1 = f2bf(v[2 * j + 1]);
        wh[j] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        wl[j] = (uint32_t)f2bf(v[2 * j] - bf2f(h0)) | ((uint32_t)f2bf(v[2 * j + 1] - bf2f(h1)) << 16);
      }
      hi = u32x4_t{wh[0], wh[1], wh[2], wh[3]};
      lo = u32x4_t{wl[0], wl[1], wl[2], wl[3]};
    };
    bool staged = false;
    if constexpr (KS == 16 && NWV == 8) {
      if (pair && p.a_f32_split && p.mg_ml) {
        // merge the attention splits of row b for this head (batch) while staging: this thread's
        // chunks i = 0 .. 3 are rows tid / 64 + 8 i (< 32), chunks i + 4 their residual rows
        static_assert(PER == 8 && CH == 64, "merge staging layout");
        const float* Po = (const float*)p.A;
        // the first two splits of every row are loaded at once (split 1 clamped to the array; its
        // values are used only where the row has it), further splits afterwards (rare): the common
        // case costs the sequence-length lookup and one round of loads instead of a chain per split
        const int sp1 = min(1, p.mg_max_splits - 1);
        int ns[PER / 2];
        int64_t q0[PER / 2];
        f32x2_t ml[PER / 2][2];
        f32x4_t ov[PER / 2][2][2];
#pragma unroll
        for (int i = 0; i < PER / 2; ++i) {
          const int c = tid + NT * i, row = c / CH, ch = c % CH;
          const int b = m0 + min(row, mrows - 1);
          ns[i] = cdiv(p.mg_len[p.mg_seq[b]], p.mg_chunk);
          q0[i] = (int64_t)b * p.mg_max_splits * 64 + batch;  // (b, split 0, head)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int64_t q = q0[i] + (int64_t)(u ? sp1 : 0) * 64;
            ml[i][u] = *reinterpret_cast<const f32x2_t*>(p.mg_ml + q * 2);
            const float* src = Po + q * 512 + ch * 8;
            ov[i][u][0] = *reinterpret_cast<const f32x4_t*>(src);
            ov[i][u][1] = *reinterpret_cast<const f32x4_t*>(src + 4);
          }
        }
#pragma unroll
        for (int i = 0; i < PER / 2; ++i) {
          const int ch = (tid + NT * i) % CH;
          float mx = ml[i][0][0];
          if (ns[i] > 1) mx = fmaxf(mx, ml[i][1][0]);
          for (int sp = 2; sp < ns[i]; ++sp) mx = fmaxf(mx, p.mg_ml[(q0[i] + (int64_t)sp * 64) * 2]);
          // splits added in order: 0, 1, then the rest
          const float w0 = exp2f(ml[i][0][0] - mx);
          float l = w0 * ml[i][0][1];
          f32x4_t a0 = ov[i][0][0] * w0, a1 = ov[i][0][1] * w0;
          if (ns[i] > 1) {
            const float w1 = exp2f(ml[i][1][0] - mx);
            l += w1 * ml[i][1][1];
            a0 += ov[i][1][0] * w1;
            a1 += ov[i][1][1] * w1;
          }
          for (int sp = 2; sp < ns[i]; ++sp) {
            const int64_t q = q0[i] + (int64_t)sp * 64;
            const float w = exp2f(p.mg_ml[q * 2] - mx);
            l += w * p.mg_ml[q * 2 + 1];
            const float* src = Po + q * 512 + ch * 8;
            a0 += *reinterpret_cast<const f32x4_t*>(src) * w;
            a1 += *reinterpret_cast<const f32x4_t*>(src + 4) * w;
          }
          const float inv = 1.0f / l, sc = p.mg_scale[(2 * batch + 1) * 4 + (ch >> 4)];
          float v[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = a0[e] * inv * sc;
            v[4 + e] = a1[e] * inv * sc;
          }
          split8(v, xv[i], xv[i + PER / 2]);
        }
        staged = true;
      }
    }
    if (staged) {
    } else if (pair && p.a_f32_split) {
      // both rows of a pair from the token's float32 values: high = bf16(v), residual = bf16(v - high)
      const float* Af = (const float*)p.A + batch * p.sA + (int64_t)m0 * p.lda;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int c = tid + NT * i, row = c / CH, ch = c % CH;
        const float* src = Af + (int64_t)min(row & 31, mrows - 1) * p.lda + ch * 8;
        const f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(src), v1 = *reinterpret_cast<const f32x4_t*>(src + 4);
        const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        u32x4_t hi, lo;
        split8(v, hi, lo);
        xv[i] = row >= 32 ? lo : hi;
      }
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int c = tid + NT * i, row = c / CH, ch = c % CH;
        xv[i] = ld16(A + arow(row) * p.lda + ch * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + NT * i, row = c / CH, ch = c % CH;
      st16(xs + row * LDX + ch * 8, xv[i]);
    }
  }
  __syncthreads();
  f32x4_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc[i] = mfma_bf16_16x16x32(as_bf16x8(ld16(xs + (16 * i + l16) * LDX + 32 * ks + 8 * g)), as_bf16x8(wb[ks]), acc[i]);
  if constexpr (NWV == 8) {
  if (pair && p.q8_codes) {
    // the row's 128 features (8 waves x 16 columns) are one quantisation group: v = high +
    // residual (one float32 addition), s = amax / 448 (1 for an all-zero group), code =
    // RNE-saturating E4M3 of v / s, as the row quantiser computes them
    __shared__ float red[NWV][32];
    float v[2][4], mx[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[i][e] = __fadd_rn(acc[i][e], acc[i + 2][e]);
        float a = fabsf(v[i][e]);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) a = fmaxf(a, __shfl_xor(a, o));
        mx[i][e] = a;
      }
    if (l16 == 0) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[wave][16 * i + 4 * g + e] = mx[i][e];
    }
    __syncthreads();
    const int col = wave * 16 + l16;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * i + 4 * g + e;
        float amax = red[0][m];
#pragma unroll
        for (int w = 1; w < NWV; ++w) amax = fmaxf(amax, red[w][m]);
        const float sc = amax == 0.f ? 1.0f : amax / 448.0f;
        if (m < mrows) {
          p.q8_codes[(int64_t)(m0 + m) * p.q8_ld + batch * 128 + col] = (uint8_t)e4m3_rne_sat(v[i][e] / sc);
          if (wave == 0 && l16 == 0) p.q8_scales[(int64_t)(m0 + m) * p.q8_sld + batch] = sc;
        }
      }
    return;
  }
  }
  if (pair) {
    // high part (tile rows 0..31) plus residual part (rows 32..63), each scaled, as two float32
    // roundings and one float32 addition (no fused multiply-add)
    const int n = n0 + l16;
    const float cs = p.c_scale ? p.c_scale[batch * p.cs_stride + (n >> 7)] : 1.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * i + 4 * g + e;
        const float hi = p.c_scale ? __fmul_rn(acc[i][e], cs) : acc[i][e];
        const float lo = p.c_scale ? __fmul_rn(acc[i + 2][e], cs) : acc[i + 2][e];
        const int64_t ci = batch * p.sC + (int64_t)(m0 + m) * p.ldc + n;
        if (m < mrows && n < p.N) {
          if (p.c_f16) ((_Float16*)p.C)[ci] = (_Float16)__fadd_rn(hi, lo);
          else ((float*)p.C)[ci] = __fadd_rn(hi, lo);
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 16 * i + 4 * g + e, n = n0 + l16;
      if (m < mrows && n < p.N) epi_store(p, batch, m0 + m, n, acc[i][e]);
    }
}

// ------------------------------------------------------------------------------------------
// 16 < M <= 64 with K >= 512: a ring of LDS stages filled by direct-to-LDS loads
// ------------------------------------------------------------------------------------------
// Workgroup = NW waves = 16*NW output columns over one K split. A stage covers 64 features
// (128 bytes per row): the A tile (16*MT rows, MT groups of 16) and each wave's own 16 weight
// rows. One wave instruction fetches 8 whole rows straight into LDS (lane l reads row l / 8, one
// 16-byte chunk, landing at byte 16*l), so it touches 8 cache lines; a 16-row group lands
// row-major with chunk c of row r at position c ^ ((r / 2) % 8), and a lane's operand (row l16,
// chunk 4h + g for the stage's feature half h) is read with the 16 lanes of one g on distinct
// banks. The loads hold no registers, so S-1 stages are in flight while one is multiplied, and
// one barrier per stage suffices.

// One stage's operands of a wave (byte addresses of this lane's 16 bytes): A row group i, feature
// half h at a_h + 2048 i; the wave's weight rows at w_h. Written as one asm block that waits for
// its own reads: the compiler does not know that these LDS reads never touch the ring slots the
// direct-to-LDS loads are still filling, and would otherwise wait for every load in flight. The
// outputs are early-clobber: a read's destination must not be an address register of a later read.
template <int MT>
MLA_DEV void lds_stage_operands(uint32_t a0, uint32_t a1, uint32_t w0, uint32_t w1, u32x4_t (&ra)[2 * MT],
                                u32x4_t (&rb)[2]) {
  if constexpr (MT == 4) {
    asm volatile(
        "ds_read_b128 %0, %10\n\tds_read_b128 %1, %11\n\t"
        "ds_read_b128 %2, %10 offset:2048\n\tds_read_b128 %3, %11 offset:2048\n\t"
        "ds_read_b128 %4, %10 offset:4096\n\tds_read_b128 %5, %11 offset:4096\n\t"
        "ds_read_b128 %6, %10 offset:6144\n\tds_read_b128 %7, %11 offset:6144\n\t"
        "ds_read_b128 %8, %12\n\tds_read_b128 %9, %13\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(ra[0]), "=&v"(ra[1]), "=&v"(ra[2]), "=&v"(ra[3]), "=&v"(ra[4]), "=&v"(ra[5]), "=&v"(ra[6]), "=&v"(ra[7]),
          "=&v"(rb[0]), "=&v"(rb[1])
        : "v"(a0), "v"(a1), "v"(w0), "v"(w1)
        : "memory");
  } else {
    static_assert(MT == 2, "MT 2 or 4");
    asm volatile(
        "ds_read_b128 %0, %6\n\tds_read_b128 %1, %7\n\t"
        "ds_read_b128 %2, %6 offset:2048\n\tds_read_b128 %3, %7 offset:2048\n\t"
        "ds_read_b128 %4, %8\n\tds_read_b128 %5, %9\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(ra[0]), "=&v"(ra[1]), "=&v"(ra[2]), "=&v"(ra[3]), "=&v"(rb[0]), "=&v"(rb[1])
        : "v"(a0), "v"(a1), "v"(w0), "v"(w1)
        : "memory");
  }
}

// mode 0: epilogue; 1: split y's partial sum to C + y * c_split_stride (the consumer adds the
// parts); 2: partials to p.part for splitk_reduce_kernel.
template <int MT, int NW, int S, int TAG>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_kernel(GemmArgs p, int ksplit, int mode) {
  constexpr int ABLK = 2 * MT;   // A instructions per stage (8 rows each)
  constexpr int APW = ABLK / NW;  // of which each wave issues APW
  static_assert(ABLK % NW == 0 && S >= 2, "A loads divide over the waves");
  constexpr int LPS = APW + 2;                  // loads per stage per wave
  constexpr int STAGE = (ABLK + 2 * NW) * 512;  // bf16 elements per stage
  __shared__ __attribute__((aligned(1024))) uint16_t ring[S * STAGE];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16 * NW + wave * 16;
  const int batch = blockIdx.z;
  const int kb = blockIdx.y * ksplit;
  const int nst = (min(p.K, kb + ksplit) - kb) >> 6;  // >= 1 (plan)
  const uint16_t* A = (const uint16_t*)p.A + batch * p.sA;
  const uint16_t* B = (const uint16_t*)p.B + batch * p.sB;

  // lane l of load instruction q (rows 8q .. 8q+7 of a 16-row group) reads row 8q + l/8, the chunk
  // that belongs at position l % 8 of that row
  const int lr = lane >> 3;
  auto chunk = [&](int q) { return (((lane & 7) ^ (((q * 8 + lr) >> 1) & 7)) << 3); };
  const uint16_t* ga[APW];
#pragma unroll
  for (int j = 0; j < APW; ++j) {
    const int ins = wave * APW + j;  // row group ins / 2, rows 8 (ins % 2) ..
    ga[j] = A + (int64_t)min((ins >> 1) * 16 + (ins & 1) * 8 + lr, p.M - 1) * p.lda + kb + chunk(ins & 1);
  }
  const uint16_t* gb[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) gb[q] = B + (int64_t)min(n0 + q * 8 + lr, p.N - 1) * p.ldb + kb + chunk(q);

  // Fetch stage st into ring slot buf. Callers clamp st to the last stage: in the tail the
  // re-fetch goes to the slot of a stage already consumed, so every iteration issues the same
  // number of loads and the wait count below stays exact.
  auto issue = [&](int st, int buf) {
    uint16_t* base = ring + buf * STAGE;
#pragma unroll
    for (int j = 0; j < APW; ++j) gl2lds16(ga[j] + st * 64, base + (wave * APW + j) * 512);
#pragma unroll
    for (int q = 0; q < 2; ++q) gl2lds16(gb[q] + st * 64, base + (ABLK + wave * 2 + q) * 512);
  };
  // this lane's operand positions: row l16 of a 16-row group, chunk 4h + g for feature half h
  const int swz = (l16 >> 1) & 7;
  const uint32_t o0 = l16 * 128 + ((g ^ swz) << 4), o1 = l16 * 128 + (((4 + g) ^ swz) << 4);

  f32x4_t acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < S - 1; ++t) issue(min(t, nst - 1), t);
  for (int t = 0; t < nst; ++t) {
    wait_vmcnt<(S - 2) * LPS>();  // this wave's part of stage t has landed
    // ... and every other wave's; all are done with stage t - 1. A plain barrier: __syncthreads'
    // release fence would wait for every load in flight, collapsing the ring to one stage.
    asm volatile("s_barrier" ::: "memory");
    issue(min(t + S - 1, nst - 1), (t + S - 1) % S);
    const uint32_t base = lds_addr(ring + (t % S) * STAGE);
    const uint32_t wb = base + (ABLK + wave * 2) * 1024;
    u32x4_t ra[2 * MT], rb[2];
    lds_stage_operands<MT>(base + o0, base + o1, wb + o0, wb + o1, ra, rb);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < MT; ++i) acc[i] = mfma_bf16_16x16x32(as_bf16x8(ra[2 * i + h]), as_bf16x8(rb[h]), acc[i]);
  }
  wait_vmcnt<0>();  // the tail's re-fetches land before the workgroup's LDS is released

  const int n = n0 + l16;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = i * 16 + g * 4 + e;
      if (m >= p.M || n >= p.N) continue;
      if (mode == 0)
        epi_store(p, batch, m, n, acc[i][e]);
      else if (mode == 1)
        ((float*)p.C)[blockIdx.y * p.c_split_stride + batch * p.sC + (int64_t)m * p.ldc + n] = acc[i][e];
      else
        p.part[((int64_t)batch * gridDim.y + blockIdx.y) * p.M * p.N + (int64_t)m * p.N + n] = acc[i][e];
    }
}

constexpr int TARGET_WGS = 512;  // two workgroups per CU on 256 CUs

struct Plan {
  int kind;  // 0 wsplit, 1 tile128, 2 tile256, 3 rows, 4 head, 5 skinny (LDS ring)
  int mt, nt, kw, ysplit;
  int nw;    // skinny kernel: waves (16 columns each) per workgroup
  int mode;  // skinny kernel: 0 epilogue, 1 K-split parts to C (consumer adds), 2 parts + reduce
  int rpi, rw, u;  // rows kernel: rows per load, row groups per wave, loads per register set
  int splits, ksplit;
  int tiles;  // workgroups per (split, batch)
};

Plan plan_gemm(int M, int N, int K, int batch, int ysplit_max = 1, bool rows_ok = true) {
  Plan pl{};
  pl.splits = 1;
  pl.ksplit = K;
  pl.ysplit = 1;
  // One or two rows of a single product: weight-row streaming on the VALU. Measured on MI355X:
  // ~1-2 thousand workgroups, at least four loads per wave (six when K is split over
  // workgroups), two register sets of 4 loads when a wave has 16 or more, else of 2 (more in
  // flight per wave was slower). The per-head batched products stay on the MFMA kernel.
  if (M <= 2 && batch == 1 && rows_ok) {
    pl.kind = 3;
    pl.mt = M;
    pl.rpi = K % 512 == 0 ? 1 : 4;
    const int nseg = K / (pl.rpi == 1 ? 512 : 128);
    auto wgs = [&]() { return (int64_t)cdiv(N, 4 * pl.rw * pl.rpi) * batch * pl.ysplit; };
    pl.rw = 1;
    while ((pl.rw * nseg < 4 || wgs() > 2048) && 4 * pl.rw * pl.rpi < N) pl.rw *= 2;
    while (pl.ysplit * 2 <= ysplit_max && wgs() < 1024 && nseg % (pl.ysplit * 2) == 0 &&
           pl.rw * nseg / (pl.ysplit * 2) >= 6)
      pl.ysplit *= 2;
    while ((int64_t)M * (K / pl.ysplit) * 2 > ROWS_LDS_MAX && pl.ysplit * 2 <= ysplit_max && nseg % (pl.ysplit * 2) == 0)
      pl.ysplit *= 2;
    pl.tiles = cdiv(N, 4 * pl.rw * pl.rpi);
    pl.u = pl.rw * nseg / pl.ysplit >= 16 ? 4 : 2;
    if ((int64_t)M * (K / pl.ysplit) * 2 <= ROWS_LDS_MAX) return pl;
    pl = Plan{};
    pl.splits = 1;
    pl.ksplit = K;
    pl.ysplit = 1;
  }
  // Per-head products, M <= 256, K of 128 or 512: x staged once per (head, 128 columns, 64 rows).
  // Measured on MI355X at M = 64: W_UK absorb and W_UV run in a fraction of the streaming
  // kernel's time, whose 16-column tiles re-read x for every tile; at M = 1 (decode of one
  // sequence) the absorb's 256 workgroups of 8 waves beat 2048 single-wave ones by ~1 us.
  if (M <= 256 && batch > 1 && (K == 128 || K == 512) && N % 128 == 0) {
    pl.kind = 4;
    pl.nw = K == 512 ? 4 : 8;  // W_UV (one 128-column tile per head): two workgroups per head, ~1 us faster at M = 64
    pl.tiles = N / (16 * pl.nw);
    return pl;
  }
  // 16 < M <= 64 with long K (single products: the projections at decode batch 17..64 and at
  // short prefills): the LDS-ring kernel. Measured on MI355X at M = 64: o_proj (7168 x 8192)
  // runs best with 128-column tiles and K split to about two workgroups per CU (40 us; the
  // 128 x 128 tile kernel 44 us), q_b (K = 1536) and kv_b-sized products with 64-column tiles
  // and no split (21.5 us against 25), q_a | kv_a with 64-column tiles and 4 splits.
  if (M > 16 && M <= 64 && batch == 1 && K >= 512) {
    pl.kind = 5;
    pl.mt = M <= 32 ? 2 : 4;
    pl.nw = (pl.mt == 4 && (int64_t)N * K >= ((int64_t)32 << 20)) ? 8 : 4;
    pl.tiles = cdiv(N, 16 * pl.nw);
    const int nst = K / 64;
    int sp = pl.nw == 8 ? (TARGET_WGS + pl.tiles / 2) / pl.tiles : (K <= 2048 ? 1 : 4);
    sp = std::max(1, std::min(sp, nst / 8));
    pl.ksplit = cdiv(nst, sp) * 64;
    sp = cdiv(K, pl.ksplit);
    if (sp == 1) pl.mode = 0;
    else if (sp <= ysplit_max) { pl.mode = 1; pl.ysplit = sp; }
    else { pl.mode = 2; pl.splits = sp; }
    return pl;
  }
  // Streaming kernel for decode-sized M: 16-column tiles up to 16 rows, 32-column tiles (two
  // weight fragments per step, so activation reads stay within twice the weight stream) up to
  // 64 rows.
  if (M <= 64) {
    pl.kind = 0;
    pl.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    pl.nt = M <= 16 ? 1 : 2;
    pl.tiles = cdiv(N, 16 * pl.nt);
    const int steps = K / 32;
    // Measured on MI355X: a stream runs best with at least ~24 K steps per wave and ~1-2
    // thousand waves in the grid. K is first split over workgroups where the consumer adds
    // the parts (ysplit), then over the waves of a workgroup.
    while (pl.ysplit * 2 <= ysplit_max && pl.tiles * batch * pl.ysplit < 512 && steps / (pl.ysplit * 2) >= 32)
      pl.ysplit *= 2;
    int kw = 1;
    while (kw * 2 <= (pl.mt == 1 ? 16 : 8) && steps / (pl.ysplit * kw * 2) >= 24 &&
           pl.tiles * batch * pl.ysplit * kw * 2 <= 2048)
      kw *= 2;
    pl.kw = kw;
    return pl;
  }
  // 256 x 256 tiles (one workgroup per CU) need at least two rounds of workgroups; below that the
  // last round leaves most CUs idle, and 128 x 128 tiles (two per CU) measured faster (q_a | kv_a at
  // 8192 tokens: 288 large tiles 482 us, 1088 small ones 355 us).
  const bool big = M >= 1024 && N >= 1024 && (int64_t)cdiv(M, 256) * cdiv(N, 256) * batch >= 512;
  pl.kind = big ? 2 : 1;
  const int bm = big ? 256 : 128;
  pl.tiles = cdiv(M, bm) * cdiv(N, bm);
  const int nsteps = K / 64;
  int splits = 1;
  const int wgs = pl.tiles * batch;
  if (wgs < TARGET_WGS / 2) splits = cdiv(TARGET_WGS, wgs);
  // split-K partials are written and read back in float32: at decode-sized M (a few hundred
  // rows) they can outweigh the operands themselves, so a split may add at most the operand
  // bytes in partial traffic
  const int64_t operand_bytes = 2 * (int64_t)batch * ((int64_t)M * K + (int64_t)N * K);
  const int64_t part_bytes_per_split = 8 * (int64_t)batch * M * N;
  splits = std::min<int64_t>(splits, std::max<int64_t>(1, operand_bytes / part_bytes_per_split));
  splits = std::max(1, std::min(splits, nsteps));
  const int steps_per = cdiv(nsteps, splits);
  pl.ksplit = steps_per * 64;
  pl.splits = cdiv(nsteps, steps_per);
  return pl;
}

template <int MT, int NT, int U, int TAG>
void launch_wsplit(const GemmArgs& a, const Plan& pl, hipStream_t s) {
  dim3 grid(pl.tiles, pl.ysplit, a.batch);
  switch (pl.kw) {
    case 1: hipLaunchKernelGGL((gemm_wsplit_kernel<MT, NT, U, 1, TAG>), grid, dim3(64), 0, s, a); break;
    case 2: hipLaunchKernelGGL((gemm_wsplit_kernel<MT, NT, U, 2, TAG>), grid, dim3(128), 0, s, a); break;
    case 4: hipLaunchKernelGGL((gemm_wsplit_kernel<MT, NT, U, 4, TAG>), grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL((gemm_wsplit_kernel<MT, NT, U, 8, TAG>), grid, dim3(512), 0, s, a); break;
    default:
      if constexpr (MT == 1) hipLaunchKernelGGL((gemm_wsplit_kernel<MT, NT, U, 16, TAG>), grid, dim3(1024), 0, s, a);
      break;
  }
}

template <int MT, int TAG>
void launch_skinny(const GemmArgs& a, const Plan& pl, hipStream_t s) {
  dim3 grid(pl.tiles, std::max(pl.splits, pl.ysplit), a.batch);
  if constexpr (MT == 4) {
    if (pl.nw == 8) {
      hipLaunchKernelGGL((gemm_skinny_kernel<MT, 8, 3, TAG>), grid, dim3(512), 0, s, a, pl.ksplit, pl.mode);
    } else {
      hipLaunchKernelGGL((gemm_skinny_kernel<MT, 4, 4, TAG>), grid, dim3(256), 0, s, a, pl.ksplit, pl.mode);
    }
  } else {
    hipLaunchKernelGGL((gemm_skinny_kernel<MT, 4, 4, TAG>), grid, dim3(256), 0, s, a, pl.ksplit, pl.mode);
  }
  if (pl.mode == 2) launch_reduce<TAG>(a, pl.splits, s);
}

template <int RPI, int U, int TAG>
void launch_rows(const GemmArgs& a, const Plan& pl, dim3 grid, size_t lds, hipStream_t s) {
  const NormArgs none{};
  if (pl.mt == 1) hipLaunchKernelGGL((gemm_rows_kernel<RPI, 1, U, TAG, false>), grid, dim3(256), lds, s, a, pl.rw, none);
  else hipLaunchKernelGGL((gemm_rows_kernel<RPI, 2, U, TAG, false>), grid, dim3(256), lds, s, a, pl.rw, none);
}

template <int TAG>
void launch_tagged(const GemmArgs& a, const Plan& pl, hipStream_t s) {
  if (pl.kind == 4) {
    dim3 grid(a.batch, pl.tiles, a.pair_rows > 0 ? cdiv(a.pair_rows, 32) : cdiv(a.M, 64));
    if (a.pair_rows > 0 && a.q8_codes) {  // the quantiser epilogue: all 128 columns in one workgroup
      grid.y = 1;
      if (a.K == 128) hipLaunchKernelGGL((gemm_head_kernel<4, 8, TAG>), grid, dim3(512), 0, s, a);
      else hipLaunchKernelGGL((gemm_head_kernel<16, 8, TAG>), grid, dim3(512), 0, s, a);
    } else if (pl.nw == 8) {
      if (a.K == 128) hipLaunchKernelGGL((gemm_head_kernel<4, 8, TAG>), grid, dim3(512), 0, s, a);
      else hipLaunchKernelGGL((gemm_head_kernel<16, 8, TAG>), grid, dim3(512), 0, s, a);
    } else {
      if (a.K == 128) hipLaunchKernelGGL((gemm_head_kernel<4, 4, TAG>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((gemm_head_kernel<16, 4, TAG>), grid, dim3(256), 0, s, a);
    }
    return;
  }
  if (pl.kind == 3) {
    dim3 grid(pl.tiles, pl.ysplit, a.batch);
    const size_t lds = (size_t)pl.mt * (a.K / pl.ysplit) * 2;
    if (pl.rpi == 1) {
      if (pl.u == 4) launch_rows<1, 4, TAG>(a, pl, grid, lds, s);
      else launch_rows<1, 2, TAG>(a, pl, grid, lds, s);
    } else {
      if (pl.u == 4) launch_rows<4, 4, TAG>(a, pl, grid, lds, s);
      else launch_rows<4, 2, TAG>(a, pl, grid, lds, s);
    }
    return;
  }
  if (pl.kind == 5) {
    if (pl.mt == 2) launch_skinny<2, TAG>(a, pl, s);
    else launch_skinny<4, TAG>(a, pl, s);
    return;
  }
  if (pl.kind == 0) {
    if (pl.mt == 1) launch_wsplit<1, 1, 8, TAG>(a, pl, s);
    else if (pl.mt == 2) launch_wsplit<2, 2, 4, TAG>(a, pl, s);
    else launch_wsplit<4, 2, 2, TAG>(a, pl, s);
    return;
  }
  dim3 grid(pl.tiles, pl.splits, a.batch);
  if (pl.kind == 1)
    hipLaunchKernelGGL((gemm_tile_kernel<128, 128, 2, 2, TAG>), grid, dim3(256), 0, s, a, pl.splits, pl.ksplit);
  else
    hipLaunchKernelGGL((gemm_tile_kernel<256, 256, 2, 4, TAG>), grid, dim3(512), 0, s, a, pl.splits, pl.ksplit);
  if (pl.splits > 1) launch_reduce<TAG>(a, pl.splits, s);
}

}  // namespace

int64_t gemm_part_floats(int M, int N, int K, int batch) {
  const Plan pl = plan_gemm(M, N, K, batch);
  return pl.splits > 1 ? (int64_t)pl.splits * batch * M * N : 0;
}


// The rows kernel addresses each operand through a buffer descriptor: windows under 2 GiB.
bool rows_ok(const GemmArgs& a) {
  constexpr int64_t LIM = (int64_t)1 << 31;
  return ((int64_t)(a.M - 1) * a.lda + a.K) * 2 < LIM && ((int64_t)(a.N - 1) * a.ldb + a.K) * 2 < LIM;
}

int gemm_ysplit(const GemmArgs& a) {
  return plan_gemm(a.M, a.N, a.K, a.batch, a.epi == EPI_F32 ? a.ysplit_max : 1, rows_ok(a)).ysplit;
}

bool gemm_bf16_fuses_qnorm(const GemmArgs& a) {
  const Plan pl = plan_gemm(a.M, a.N, a.K, a.batch, 1, rows_ok(a));
  return pl.kind == 3 && pl.ysplit == 1 && pl.rpi == 1 && a.K == mla_dims::Q_LORA && a.batch == 1;
}

hipError_t gemm_bf16_qnorm(const GemmArgs& a, const NormArgs& na, hipStream_t s) {
  if (!gemm_bf16_fuses_qnorm(a) || na.n_tokens != a.M || na.meta || na.fp8) return hipErrorInvalidValue;
  const Plan pl = plan_gemm(a.M, a.N, a.K, a.batch, 1, rows_ok(a));
  dim3 grid(pl.tiles, 1, 1);
  const size_t lds = (size_t)pl.mt * a.K * 2;
  if (pl.u == 4) {
    if (pl.mt == 1) hipLaunchKernelGGL((gemm_rows_kernel<1, 1, 4, TAG_QB, true>), grid, dim3(256), lds, s, a, pl.rw, na);
    else hipLaunchKernelGGL((gemm_rows_kernel<1, 2, 4, TAG_QB, true>), grid, dim3(256), lds, s, a, pl.rw, na);
  } else {
    if (pl.mt == 1) hipLaunchKernelGGL((gemm_rows_kernel<1, 1, 2, TAG_QB, true>), grid, dim3(256), lds, s, a, pl.rw, na);
    else hipLaunchKernelGGL((gemm_rows_kernel<1, 2, 2, TAG_QB, true>), grid, dim3(256), lds, s, a, pl.rw, na);
  }
  return hipGetLastError();
}

bool gemm_bf16_pairs(const GemmArgs& a) {
  return a.M == 2 * a.pair_rows && a.epi == EPI_F32 && (!a.q8_codes || (a.N == 128 && !a.c_scale)) &&
         (!a.mg_ml || (a.a_f32_split && a.q8_codes && a.K == 512 && a.mg_chunk > 0 && a.mg_max_splits > 0)) &&
         plan_gemm(a.M, a.N, a.K, a.batch, a.ysplit_max, rows_ok(a)).kind == 4;
}

hipError_t gemm_bf16(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.K % 128 != 0) return hipErrorInvalidValue;
  if (a.pair_rows > 0 && !gemm_bf16_pairs(a)) return hipErrorInvalidValue;  // only the per-head kernel pairs rows
  const Plan pl = plan_gemm(a.M, a.N, a.K, a.batch, a.epi == EPI_F32 ? a.ysplit_max : 1, rows_ok(a));
  if (pl.splits > 1 && (int64_t)pl.splits * a.batch * a.M * a.N > a.part_cap) return hipErrorInvalidValue;
  switch (a.tag) {
    case TAG_QKVA: launch_tagged<TAG_QKVA>(a, pl, s); break;
    case TAG_QB: launch_tagged<TAG_QB>(a, pl, s); break;
    case TAG_KVB: launch_tagged<TAG_KVB>(a, pl, s); break;
    case TAG_OPROJ: launch_tagged<TAG_OPROJ>(a, pl, s); break;
    case TAG_ABSORB: launch_tagged<TAG_ABSORB>(a, pl, s); break;
    case TAG_UV: launch_tagged<TAG_UV>(a, pl, s); break;
    default: launch_tagged<TAG_NONE>(a, pl, s); break;
  }
  return hipGetLastError();
}

}  // namespace mla_k
