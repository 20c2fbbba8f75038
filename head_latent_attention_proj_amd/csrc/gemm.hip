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
//   * gemm_skinny -- decode-sized M (<= 64): activations and weights go straight from global
//                    memory into MFMA fragments (each lane streams 64 contiguous weight bytes
//                    per 128-wide K step), K split across workgroups so that every CU streams
//                    weights; the last workgroup of a tile reduces the fp32 partials in a fixed
//                    order (deterministic, no float atomics).
#include "common.h"
#include "kernels.h"

namespace mla_k {

namespace {

MLA_DEV void epi_store(const GemmArgs& p, int b, int m, int n, float v) {
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

MLA_DEV void part_store(float* ptr, float v) {
  __hip_atomic_store(ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
MLA_DEV float part_load(const float* ptr) {
  return __hip_atomic_load(ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Arrival count for split-K: returns true in the workgroup that arrives last for this tile
// (it then owns the reduction); that workgroup also resets the counter to zero.
MLA_DEV bool splitk_arrive(int* ctr, int splits) {
  __shared__ int last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = atomicAdd(ctr, 1);
    last = (old == splits - 1);
    if (last) atomicExch(ctr, 0);
  }
  __syncthreads();
  __threadfence();
  return last != 0;
}

// Last arrival: sum the partials of region [m0, m0+bm) x [n0, n0+bn) over splits 0..splits-1.
MLA_DEV void splitk_reduce(const GemmArgs& p, int b, int splits, int m0, int bm, int n0, int bn) {
  const float* base = p.part + (int64_t)b * splits * p.M * p.N;
  const int cnt = bm * bn;
  for (int idx = threadIdx.x; idx < cnt; idx += blockDim.x) {
    const int m = m0 + idx / bn, n = n0 + idx % bn;
    if (m >= p.M || n >= p.N) continue;
    float s = 0.f;
    for (int sp = 0; sp < splits; ++sp) s += part_load(base + ((int64_t)sp * p.M + m) * p.N + n);
    epi_store(p, b, m, n, s);
  }
}

// ------------------------------------------------------------------------------------------
// Tile kernel
// ------------------------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN>
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

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
        if (m < p.M && n < p.N) part_store(part + (int64_t)m * p.N + n, acc[i][j][e]);
      }
  if (splitk_arrive(p.counters + batch * ntile + tm * tiles_n + tn, splits))
    splitk_reduce(p, batch, splits, m0, BM, n0, BN);
}

// ------------------------------------------------------------------------------------------
// Skinny kernel: M <= 16*MT rows, 4 waves x TN column tiles of 16, K split over blockIdx.y
// ------------------------------------------------------------------------------------------
template <int MT, int TN>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs p, int splits, int ksplit) {
  constexpr int WCOLS = TN * 16, BCOLS = 4 * WCOLS;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int nb = blockIdx.x, split = blockIdx.y, batch = blockIdx.z;
  const int nw = nb * BCOLS + wave * WCOLS;
  const int kb = split * ksplit;
  const int ke = min(p.K, kb + ksplit);

  const uint16_t* A = (const uint16_t*)p.A + batch * p.sA;
  const uint16_t* B = (const uint16_t*)p.B + batch * p.sB;
  // lane (l16, g) owns bytes [g*64, g*64+64) of every 128-wide K step of its row
  const uint16_t* pa[MT];
  const uint16_t* pb[TN];
#pragma unroll
  for (int i = 0; i < MT; ++i) pa[i] = A + (int64_t)min(i * 16 + l16, p.M - 1) * p.lda + g * 32;
#pragma unroll
  for (int j = 0; j < TN; ++j) pb[j] = B + (int64_t)min(nw + j * 16 + l16, p.N - 1) * p.ldb + g * 32;

  f32x4_t acc[MT][TN];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll 2
  for (int k = kb; k < ke; k += 128) {
    u32x4_t va[MT][4], vb[TN][4];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int s = 0; s < 4; ++s) vb[j][s] = ld16(pb[j] + k + s * 8);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int s = 0; s < 4; ++s) va[i][s] = ld16(pa[i] + k + s * 8);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = mfma_bf16_16x16x32(as_bf16x8(va[i][s]), as_bf16x8(vb[j][s]), acc[i][j]);
  }

  if (splits == 1) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = i * 16 + g * 4 + e, n = nw + j * 16 + l16;
          if (m < p.M && n < p.N) epi_store(p, batch, m, n, acc[i][j][e]);
        }
    return;
  }
  float* part = p.part + ((int64_t)batch * splits + split) * p.M * p.N;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = i * 16 + g * 4 + e, n = nw + j * 16 + l16;
        if (m < p.M && n < p.N) part_store(part + (int64_t)m * p.N + n, acc[i][j][e]);
      }
  if (splitk_arrive(p.counters + batch * gridDim.x + nb, splits))
    splitk_reduce(p, batch, splits, 0, 16 * MT, nb * BCOLS, BCOLS);
}

constexpr int SKINNY_TN = 4;
constexpr int SKINNY_COLS = 4 * SKINNY_TN * 16;  // 256 columns per workgroup
constexpr int TARGET_WGS = 512;                  // two workgroups per CU on 256 CUs

struct Plan {
  int kind;  // 0 skinny, 1 tile128, 2 tile256
  int mt;
  int splits, ksplit;
  int tiles;  // workgroups per (split, batch)
};

Plan plan_gemm(int M, int N, int K, int batch) {
  Plan pl{};
  int kstep;
  if (M <= 64) {
    pl.kind = 0;
    pl.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    pl.tiles = cdiv(N, SKINNY_COLS);
    kstep = 128;
  } else {
    const bool big = (M >= 1024 && N >= 1024);
    pl.kind = big ? 2 : 1;
    const int bm = big ? 256 : 128;
    pl.tiles = cdiv(M, bm) * cdiv(N, bm);
    kstep = 64;
  }
  const int nsteps = K / kstep;
  int splits = 1;
  const int wgs = pl.tiles * batch;
  if (wgs < TARGET_WGS / 2) splits = cdiv(TARGET_WGS, wgs);
  if (splits > nsteps) splits = nsteps;
  if (splits < 1) splits = 1;
  const int steps_per = cdiv(nsteps, splits);
  pl.ksplit = steps_per * kstep;
  pl.splits = cdiv(nsteps, steps_per);
  return pl;
}

}  // namespace

int64_t gemm_part_floats(int M, int N, int K, int batch) {
  const Plan pl = plan_gemm(M, N, K, batch);
  return pl.splits > 1 ? (int64_t)pl.splits * batch * M * N : 0;
}

int gemm_counters(int M, int N, int K, int batch) {
  const Plan pl = plan_gemm(M, N, K, batch);
  return pl.splits > 1 ? pl.tiles * batch : 0;
}

hipError_t gemm_bf16(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.K % 128 != 0) return hipErrorInvalidValue;
  const Plan pl = plan_gemm(a.M, a.N, a.K, a.batch);
  if (pl.splits > 1) {
    if ((int64_t)pl.splits * a.batch * a.M * a.N > a.part_cap || pl.tiles * a.batch > a.counter_cap)
      return hipErrorInvalidValue;
  }
  dim3 grid(pl.tiles, pl.splits, a.batch);
  switch (pl.kind) {
    case 0:
      if (pl.mt == 1)
        hipLaunchKernelGGL((gemm_skinny_kernel<1, SKINNY_TN>), grid, dim3(256), 0, s, a, pl.splits, pl.ksplit);
      else if (pl.mt == 2)
        hipLaunchKernelGGL((gemm_skinny_kernel<2, SKINNY_TN>), grid, dim3(256), 0, s, a, pl.splits, pl.ksplit);
      else
        hipLaunchKernelGGL((gemm_skinny_kernel<4, SKINNY_TN>), grid, dim3(256), 0, s, a, pl.splits, pl.ksplit);
      break;
    case 1:
      hipLaunchKernelGGL((gemm_tile_kernel<128, 128, 2, 2>), grid, dim3(256), 0, s, a, pl.splits, pl.ksplit);
      break;
    default:
      hipLaunchKernelGGL((gemm_tile_kernel<256, 256, 2, 4>), grid, dim3(512), 0, s, a, pl.splits, pl.ksplit);
      break;
  }
  return hipGetLastError();
}

}  // namespace mla_k
