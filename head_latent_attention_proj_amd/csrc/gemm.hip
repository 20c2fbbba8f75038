// bf16 MFMA GEMMs for the five MLA projections and the per-head absorption products.
//
// C[b] = A[b] * B[b]^T with A [M, K] and B [N, K] both K-contiguous: nn.Linear keeps its weight
// [out, in] ("Key content up-projection" page, Parameters), so every projection y = x W^T is
// this "NT" form and both MFMA operands load 16 contiguous bytes per lane.
//
// Two kernels:
//   * gemm_tile   -- prefill-sized M: BM x BN workgroup tile staged through LDS (double
//                    buffered, padded rows so 16-byte fragment reads are bank-conflict free),
//                    16x16x32 bf16 MFMA, XCD-aware grouped tile order. Optional split-K.
//   * gemm_wsplit -- decode-sized M (<= 64): operands go straight from global memory into MFMA
//                    fragments; the K range of a 16-column tile is split across the waves of one
//                    workgroup (each wave streams its own contiguous slice of the weight rows,
//                    four 32-wide K steps in flight), and the waves' partial tiles are summed
//                    through LDS in a fixed order. No cross-workgroup synchronisation, no float
//                    atomics: the result is deterministic.
//   Split-K of the tile kernel (few tiles, small M) writes fp32 partials and a separate
//   reduction kernel sums them in a fixed order.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace mla_k {

namespace {

MLA_DEV void epi_store(const GemmArgs& p, int b, int m, int n, float v) {
  if (p.c_scale) v *= p.c_scale[b * p.cs_stride + (n >> 7)];
  if (p.epi == EPI_F32) {
    ((float*)p.C)[b * p.sC + (int64_t)m * p.ldc + n] = v;
  } else if (p.epi == EPI_BF16) {
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
  constexpr int LDK = BK + 8;  // 144-byte rows: 8 consecutive rows hit 8 distinct 16-byte bank groups
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 16, TN = WTN / 16;
  constexpr int CPR = BK / 8;
  constexpr int RPP = NT / CPR;
  constexpr int AP = BM / RPP, BP = BN / RPP;
  static_assert(BM % RPP == 0 && BN % RPP == 0, "tile rows must be a multiple of rows per pass");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (BM + BN) * LDK];

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
    for (int i = 0; i < AP; ++i) st16(sa + (i * RPP + lr) * LDK + lc, ra[i]);
#pragma unroll
    for (int i = 0; i < BP; ++i) st16(sb + (i * RPP + lr) * LDK + lc, rb[i]);
  };

  if (nk > 0) {
    gload(kb);
    sstore(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kb + (kt + 1) * BK);
    const uint16_t* sa = smem + cur * (BM + BN) * LDK + (wm * WTM + l16) * LDK + g * 8;
    const uint16_t* sb = smem + cur * (BM + BN) * LDK + BM * LDK + (wn * WTN + l16) * LDK + g * 8;
#pragma unroll
    for (int s = 0; s < BK / 32; ++s) {
      bf16x8_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = as_bf16x8(ld16(sa + i * 16 * LDK + s * 32));
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = as_bf16x8(ld16(sb + j * 16 * LDK + s * 32));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_bf16_16x16x32(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  if (splits == 1) {
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

// ------------------------------------------------------------------------------------------
// Decode-sized M: one workgroup per 16-column tile, K split across its KW waves
// ------------------------------------------------------------------------------------------
template <int MT, int KW, int TAG>
__global__ __launch_bounds__(KW * 64) void gemm_wsplit_kernel(GemmArgs p) {
  constexpr int U = MT >= 4 ? 2 : (MT == 2 ? 4 : 8);  // 32-wide K steps per pipeline stage
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int l16 = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16;
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

  // lane (l16, g): row l16 of the tile, features g*8 .. g*8+7 of each 32-wide step
  const uint16_t* pa[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) pa[i] = A + (int64_t)min(i * 16 + l16, p.M - 1) * p.lda + g * 8;
  const uint16_t* pb = B + (int64_t)min(n0 + l16, p.N - 1) * p.ldb + g * 8;

  f32x4_t acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (s0 < s1) {
    // Loads are unconditional (steps past the wave's range re-read its last step) so the
    // next stage's loads stay in flight while the current stage multiplies; a step past the
    // range multiplies a zero weight fragment instead of being branched around.
    u32x4_t ca[U][MT], cb[U];
    auto load = [&](int s, u32x4_t (&ra)[U][MT], u32x4_t (&rb)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int st = min(s + u, s1 - 1) * 32;
        rb[u] = ld16(pb + st);
#pragma unroll
        for (int i = 0; i < MT; ++i) ra[u][i] = ld16(pa[i] + st);
      }
    };
    load(s0, ca, cb);
    for (int s = s0; s < s1; s += U) {
      u32x4_t na[U][MT], nb[U];
      load(min(s + U, s1 - 1), na, nb);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const u32x4_t zero = {0u, 0u, 0u, 0u};
        const u32x4_t bw = (s + u < s1) ? cb[u] : zero;
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[i] = mfma_bf16_16x16x32(as_bf16x8(ca[u][i]), as_bf16x8(bw), acc[i]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        cb[u] = nb[u];
#pragma unroll
        for (int i = 0; i < MT; ++i) ca[u][i] = na[u][i];
      }
    }
  }

  // fixed-order sum of the waves' partial tiles through LDS
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
      if (m < p.M && n < p.N) epi_store(p, batch, m, n, acc[i][e]);
    }
}

constexpr int TARGET_WGS = 512;  // two workgroups per CU on 256 CUs

struct Plan {
  int kind;  // 0 wsplit, 1 tile128, 2 tile256
  int mt, kw, ysplit;
  int splits, ksplit;
  int tiles;  // workgroups per (split, batch)
};

Plan plan_gemm(int M, int N, int K, int batch, int ysplit_max = 1) {
  Plan pl{};
  pl.splits = 1;
  pl.ksplit = K;
  pl.ysplit = 1;
  // Streaming kernel for decode-sized M: always up to 16 rows; up to 64 rows when K is short
  // (kv_b, W_UK / W_UV), where a staged tile would spend most of its time filling LDS.
  if (M <= 16 || (M <= 64 && K <= 512)) {
    pl.kind = 0;
    pl.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    pl.tiles = cdiv(N, 16);
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
  const bool big = (M >= 1024 && N >= 1024);
  pl.kind = big ? 2 : 1;
  const int bm = big ? 256 : 128;
  pl.tiles = cdiv(M, bm) * cdiv(N, bm);
  const int nsteps = K / 64;
  int splits = 1;
  const int wgs = pl.tiles * batch;
  if (wgs < TARGET_WGS / 2) splits = cdiv(TARGET_WGS, wgs);
  splits = std::max(1, std::min(splits, nsteps));
  const int steps_per = cdiv(nsteps, splits);
  pl.ksplit = steps_per * 64;
  pl.splits = cdiv(nsteps, steps_per);
  return pl;
}

template <int MT, int TAG>
void launch_wsplit(const GemmArgs& a, const Plan& pl, hipStream_t s) {
  dim3 grid(pl.tiles, pl.ysplit, a.batch);
  switch (pl.kw) {
    case 1: hipLaunchKernelGGL((gemm_wsplit_kernel<MT, 1, TAG>), grid, dim3(64), 0, s, a); break;
    case 2: hipLaunchKernelGGL((gemm_wsplit_kernel<MT, 2, TAG>), grid, dim3(128), 0, s, a); break;
    case 4: hipLaunchKernelGGL((gemm_wsplit_kernel<MT, 4, TAG>), grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL((gemm_wsplit_kernel<MT, 8, TAG>), grid, dim3(512), 0, s, a); break;
    default:
      if constexpr (MT == 1) hipLaunchKernelGGL((gemm_wsplit_kernel<MT, 16, TAG>), grid, dim3(1024), 0, s, a);
      break;
  }
}

template <int TAG>
void launch_tagged(const GemmArgs& a, const Plan& pl, hipStream_t s) {
  if (pl.kind == 0) {
    if (pl.mt == 1) launch_wsplit<1, TAG>(a, pl, s);
    else if (pl.mt == 2) launch_wsplit<2, TAG>(a, pl, s);
    else launch_wsplit<4, TAG>(a, pl, s);
    return;
  }
  dim3 grid(pl.tiles, pl.splits, a.batch);
  if (pl.kind == 1)
    hipLaunchKernelGGL((gemm_tile_kernel<128, 128, 2, 2, TAG>), grid, dim3(256), 0, s, a, pl.splits, pl.ksplit);
  else
    hipLaunchKernelGGL((gemm_tile_kernel<256, 256, 2, 4, TAG>), grid, dim3(512), 0, s, a, pl.splits, pl.ksplit);
  if (pl.splits > 1) {
    dim3 rgrid((unsigned)(((int64_t)a.M * a.N + 255) / 256), a.batch);
    hipLaunchKernelGGL((splitk_reduce_kernel<TAG>), rgrid, dim3(256), 0, s, a, pl.splits);
  }
}

}  // namespace

int64_t gemm_part_floats(int M, int N, int K, int batch) {
  const Plan pl = plan_gemm(M, N, K, batch);
  return pl.splits > 1 ? (int64_t)pl.splits * batch * M * N : 0;
}

int gemm_counters(int, int, int, int) { return 0; }

int gemm_ysplit(const GemmArgs& a) {
  return plan_gemm(a.M, a.N, a.K, a.batch, a.epi == EPI_F32 ? a.ysplit_max : 1).ysplit;
}

hipError_t gemm_bf16(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.K % 128 != 0) return hipErrorInvalidValue;
  const Plan pl = plan_gemm(a.M, a.N, a.K, a.batch, a.epi == EPI_F32 ? a.ysplit_max : 1);
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
