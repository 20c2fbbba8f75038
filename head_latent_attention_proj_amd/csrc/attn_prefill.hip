// Causal prefill attention over rebuilt keys and values (LDS-tiled, online softmax, MFMA).
//
// Per sequence, head h and query t at position p = l0 + t ("Key content up-projection" page,
// code excerpt): q = [q_nope | RoPE(q_pe)], k_j = [k_nope_j | k_pe_j] with the shared rotary
// key, s_j = scale * q.k_j for key positions j <= p (the causal mask), float32 softmax, and
// o = sum_j a_j v_j over 128 value features; o is stored at column h*128 + d (head merge of
// the mla-output excerpt on the dense-block attention page).
//
// Layout of the work: one workgroup = 128 queries of one (sequence, head); 4 waves x 32 queries.
// Scores are formed transposed, S^T = K Q^T, so that the MFMA result already holds, per lane,
// one query (column) and 16 keys: the row softmax needs only two cross-lane steps, and the
// probabilities are re-used in registers as the B operand of O^T = V^T P^T (values arrive
// key-contiguous from the kv_b epilogue). 64-key blocks are staged through LDS with a one-block
// register prefetch. Workgroups are numbered head-fastest so every query tile of one head
// lands on the same XCD (its L2 keeps that head's keys and values); query tiles run
// longest-first.
#include "common.h"
#include "kernels.h"

namespace mla_k {

namespace {

constexpr int PQ = 128;   // queries per workgroup
constexpr int PKB = 64;   // keys per block
constexpr int LDK = 200;  // sK row: 192 features + pad (400 B: 8 rows -> 8 distinct bank groups)
constexpr int LDV = 68;   // sV row: 64 keys + pad (136 B: 16 rows -> 16 distinct 8-byte slots)
constexpr float LOG2E = 1.4426950408889634f;

MLA_DEV u32x2_t ld8(const void* p) { return *reinterpret_cast<const u32x2_t*>(p); }
MLA_DEV void st8(void* p, const u32x2_t& v) { *reinterpret_cast<u32x2_t*>(p) = v; }

// SPLIT (FP8 weights): q arrives in float32 and K_nope, V^T, k_pe and the probabilities carry a
// bf16 residual next to their bf16 value; each product takes hi*hi + hi*lo + lo*hi, which is
// accurate to about 16 significant bits (the FP8 path's o_proj quantiser amplifies any rounding
// of its input, so bf16 alone is not enough there).
template <bool SPLIT>
__global__ __launch_bounds__(256, SPLIT ? 1 : 2) void prefill_attn_kernel(PrefillAttnArgs a) {
  const int h = blockIdx.x;
  const int b = blockIdx.z;
  const SeqMeta m = a.meta[b];
  const int nqt = cdiv(m.t, PQ);
  if ((int)blockIdx.y >= nqt) return;
  const int q0 = (nqt - 1 - (int)blockIdx.y) * PQ;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps per-wave skips scalar
  const int l16 = lane & 15, g = lane >> 4;
  const int n_keys = m.l0 + m.t;
  const int q_hi = min(q0 + PQ, m.t);
  const int kend = m.l0 + q_hi;
  const int nblk = cdiv(kend, PKB);

  __shared__ __attribute__((aligned(16))) uint16_t sK[PKB * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sV[128 * LDV];
  __shared__ __attribute__((aligned(16))) uint16_t sKl[SPLIT ? PKB * LDK : 8];  // residual planes
  __shared__ __attribute__((aligned(16))) uint16_t sVl[SPLIT ? 128 * LDV : 8];

  // ---- Q fragments: B operand of S^T, column = query, 8 features of group g per k-step
  bf16x8_t qf[2][6], ql[SPLIT ? 2 : 1][6];
  int qpos[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int qrel = q0 + wave * 32 + qt * 16 + l16;
    qpos[qt] = m.l0 + qrel;
    const int qi = min(qrel, m.t - 1);
    const int64_t qoff = ((int64_t)(m.q0 + qi) * 64 + h) * 192;
    const int pos = m.l0 + qi;
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) {
      float x[8];
      if constexpr (SPLIT) {
        const float* qf32 = (const float*)a.q + qoff + ks * 32 + g * 8;
        const f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(qf32), v1 = *reinterpret_cast<const f32x4_t*>(qf32 + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[j] = v0[j];
          x[4 + j] = v1[j];
        }
      } else {
        const u32x4_t raw = ld16((const uint16_t*)a.q + qoff + ks * 32 + g * 8);
        if (ks < 4) {
          qf[qt][ks] = as_bf16x8(raw);
          continue;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[2 * j] = bf_lo(raw[j]);
          x[2 * j + 1] = bf_hi(raw[j]);
        }
      }
      if (ks >= 4) {  // rotary part, rotated at the query's position
        const int pair0 = ((ks - 4) * 32 + g * 8) >> 1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float c = a.rope_cs[(int64_t)pos * 32 + pair0 + j];
          const float sn = a.rope_cs[(int64_t)a.max_pos * 32 + (int64_t)pos * 32 + pair0 + j];
          const float x0 = x[2 * j], x1 = x[2 * j + 1];
          x[2 * j] = x0 * c - x1 * sn;
          x[2 * j + 1] = x0 * sn + x1 * c;
        }
      }
      u32x4_t hi, lo;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        hi[j] = pack_bf16x2(x[2 * j], x[2 * j + 1]);
        lo[j] = pack_bf16x2(x[2 * j] - bf_lo(hi[j]), x[2 * j + 1] - bf_hi(hi[j]));
      }
      qf[qt][ks] = as_bf16x8(hi);
      if constexpr (SPLIT) ql[qt][ks] = as_bf16x8(lo);
    }
  }

  // ---- block staging (global -> registers -> LDS)
  u32x4_t pk[4], pp[2], pv[4];
  const int kr = tid >> 4, kc = (tid & 15) * 8;   // K_nope: 16 threads per key row (256 B)
  const int pr = tid >> 3, pc = (tid & 7) * 8;    // k_pe / V^T: 8 threads per 128-byte row
  // Bases common to the workgroup (scalar registers) plus 32-bit per-lane byte offsets: a load
  // costs one address register and a 32-bit add instead of a 64-bit multiply-add per block.
  const uint8_t* kn_base = (const uint8_t*)(a.knope + ((int64_t)m.kbase * 64 + h) * 128);
  const uint8_t* pe_base = a.cache + m.krow0 * a.entry_bytes + a.kpe_off;
  const uint8_t* vt_base = (const uint8_t*)(a.vt + (int64_t)(h * 128) * a.vt_ld + m.kbase);
  auto gload = [&](int blk) {
    if constexpr (SPLIT) return;  // split staging loads and stores in one step (stage_split)
    const int kb = blk * PKB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t key = (uint32_t)min(kb + i * 16 + kr, n_keys - 1);
      pk[i] = ld16(kn_base + (key * (64u * 128u * 2u) + (uint32_t)kc * 2u));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t key = (uint32_t)min(kb + i * 32 + pr, n_keys - 1);
      pp[i] = ld16(pe_base + (key * (uint32_t)a.entry_bytes + (uint32_t)pc * 2u));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t row = (uint32_t)(i * 32 + pr);
      pv[i] = ld16(vt_base + (row * (uint32_t)a.vt_ld + (uint32_t)(kb + pc)) * 2u);
    }
    if (kb + PKB > n_keys) {  // value rows past the last key are not written: zero them
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = kb + pc + 2 * j;
          uint32_t w = pv[i][j];
          if (key >= n_keys) w &= 0xffff0000u;
          if (key + 1 >= n_keys) w &= 0x0000ffffu;
          pv[i][j] = w;
        }
    }
  };
  // Split staging: hi and lo planes of K_nope and V^T, float32 k_pe split on the way to LDS.
  // Loads are not held across the block's math (the registers hold the split queries instead).
  auto stage_split = [&](int blk) {
    const int kb = blk * PKB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = min(kb + i * 16 + kr, n_keys - 1);
      const int64_t off = ((int64_t)(m.kbase + key) * 64 + h) * 128 + kc;
      const u32x4_t x = ld16(a.knope + off), y = ld16(a.knope_lo + off);
      st16(sK + (i * 16 + kr) * LDK + kc, x);
      st16(sKl + (i * 16 + kr) * LDK + kc, y);
    }
    {
      const int key = min(kb + (tid >> 2), n_keys - 1);
      const float* kp = (const float*)(a.cache + (m.krow0 + key) * a.entry_bytes + a.kpe_off) + (tid & 3) * 16;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(kp + 4 * c);
        const uint32_t h0 = pack_bf16x2(v[0], v[1]), h1 = pack_bf16x2(v[2], v[3]);
        const uint32_t r0 = pack_bf16x2(v[0] - bf_lo(h0), v[1] - bf_hi(h0));
        const uint32_t r1 = pack_bf16x2(v[2] - bf_lo(h1), v[3] - bf_hi(h1));
        const int col = 128 + (tid & 3) * 16 + 4 * c;
        st8(sK + (tid >> 2) * LDK + col, u32x2_t{h0, h1});
        st8(sKl + (tid >> 2) * LDK + col, u32x2_t{r0, r1});
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = i * 32 + pr;
      const int64_t off = (int64_t)(h * 128 + row) * a.vt_ld + m.kbase + kb + pc;
      u32x4_t x = ld16(a.vt + off), y = ld16(a.vt_lo + off);
      if (kb + PKB > n_keys) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = kb + pc + 2 * j;
          uint32_t mask = 0xffffffffu;
          if (key >= n_keys) mask &= 0xffff0000u;
          if (key + 1 >= n_keys) mask &= 0x0000ffffu;
          x[j] &= mask;
          y[j] &= mask;
        }
      }
      uint16_t* d = sV + row * LDV + pc;
      st8(d, u32x2_t{x[0], x[1]});
      st8(d + 4, u32x2_t{x[2], x[3]});
      uint16_t* dl = sVl + row * LDV + pc;
      st8(dl, u32x2_t{y[0], y[1]});
      st8(dl + 4, u32x2_t{y[2], y[3]});
    }
  };
  auto sstore = [&](int blk) {
    if constexpr (SPLIT) {
      stage_split(blk);
      return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) st16(sK + (i * 16 + kr) * LDK + kc, pk[i]);
#pragma unroll
    for (int i = 0; i < 2; ++i) st16(sK + (i * 32 + pr) * LDK + 128 + pc, pp[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t* d = sV + (i * 32 + pr) * LDV + pc;
      st8(d, u32x2_t{pv[i][0], pv[i][1]});
      st8(d + 4, u32x2_t{pv[i][2], pv[i][3]});
    }
  };

  const float sl2 = a.scale * LOG2E;
  float mrun[2] = {-INFINITY, -INFINITY};
  float lrun[2] = {0.f, 0.f};
  f32x4_t oacc[8][2];
#pragma unroll
  for (int d = 0; d < 8; ++d) oacc[d][0] = oacc[d][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int wq_lo = m.l0 + q0 + wave * 32;  // smallest / largest query position of this wave
  const int wq_hi = wq_lo + 31;

  gload(0);
  for (int blk = 0; blk < nblk; ++blk) {
    __syncthreads();
    sstore(blk);
    __syncthreads();
    if (blk + 1 < nblk) gload(blk + 1);
    const int kb = blk * PKB;
    if (kb > wq_hi) continue;  // every key of this block is in the future of this wave's queries

    f32x4_t sacc[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) sacc[kt][0] = sacc[kt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) {
      bf16x8_t kf[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) kf[kt] = as_bf16x8(ld16(sK + (kt * 16 + l16) * LDK + ks * 32 + g * 8));
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        sacc[kt][0] = mfma_bf16_16x16x32(kf[kt], qf[0][ks], sacc[kt][0]);
        sacc[kt][1] = mfma_bf16_16x16x32(kf[kt], qf[1][ks], sacc[kt][1]);
        if constexpr (SPLIT) {
          sacc[kt][0] = mfma_bf16_16x16x32(kf[kt], ql[0][ks], sacc[kt][0]);
          sacc[kt][1] = mfma_bf16_16x16x32(kf[kt], ql[1][ks], sacc[kt][1]);
        }
      }
      if constexpr (SPLIT) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const bf16x8_t kl = as_bf16x8(ld16(sKl + (kt * 16 + l16) * LDK + ks * 32 + g * 8));
          sacc[kt][0] = mfma_bf16_16x16x32(kl, qf[0][ks], sacc[kt][0]);
          sacc[kt][1] = mfma_bf16_16x16x32(kl, qf[1][ks], sacc[kt][1]);
        }
      }
    }

    const bool need_mask = kb + PKB - 1 > wq_lo;
    bf16x8_t pf[2][2], pl[SPLIT ? 2 : 1][2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      // scores stay unscaled here: the scale (softmax scale times log2 e, positive) commutes with
      // the maximum and is applied inside each exponent's fused multiply-add
      float bmax = -INFINITY;
      if (need_mask) {  // wave-uniform: only blocks that reach past the wave's first query
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (kb + kt * 16 + g * 4 + e > qpos[qt]) sacc[kt][qt][e] = -INFINITY;
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) bmax = fmaxf(bmax, sacc[kt][qt][e]);
      bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
      bmax *= sl2;
      // The running maximum is raised only when some query's block maximum exceeds it by more
      // than 8 (log2 units; wave-uniform decision): probabilities stay <= 256 and the output
      // accumulators are rescaled rarely. The first block holds key 0, visible to every query,
      // so mrun is finite after it.
      if (__any(bmax > mrun[qt] + 8.0f)) {
        const float mnew = fmaxf(mrun[qt], bmax);
        const float alpha = exp2_flush(mrun[qt] - mnew);
        mrun[qt] = mnew;
        lrun[qt] *= alpha;
#pragma unroll
        for (int d = 0; d < 8; ++d) oacc[d][qt] *= alpha;
      }
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = exp2_flush(fmaf(sacc[kt][qt][e], sl2, -mrun[qt]));
          sacc[kt][qt][e] = p;
          psum += p;
        }
      lrun[qt] += psum;
#pragma unroll
      for (int ps = 0; ps < 2; ++ps) {
        u32x4_t w;
        w[0] = pack_bf16x2(sacc[2 * ps][qt][0], sacc[2 * ps][qt][1]);
        w[1] = pack_bf16x2(sacc[2 * ps][qt][2], sacc[2 * ps][qt][3]);
        w[2] = pack_bf16x2(sacc[2 * ps + 1][qt][0], sacc[2 * ps + 1][qt][1]);
        w[3] = pack_bf16x2(sacc[2 * ps + 1][qt][2], sacc[2 * ps + 1][qt][3]);
        pf[ps][qt] = as_bf16x8(w);
        if constexpr (SPLIT) {
          u32x4_t r;
          r[0] = pack_bf16x2(sacc[2 * ps][qt][0] - bf_lo(w[0]), sacc[2 * ps][qt][1] - bf_hi(w[0]));
          r[1] = pack_bf16x2(sacc[2 * ps][qt][2] - bf_lo(w[1]), sacc[2 * ps][qt][3] - bf_hi(w[1]));
          r[2] = pack_bf16x2(sacc[2 * ps + 1][qt][0] - bf_lo(w[2]), sacc[2 * ps + 1][qt][1] - bf_hi(w[2]));
          r[3] = pack_bf16x2(sacc[2 * ps + 1][qt][2] - bf_lo(w[3]), sacc[2 * ps + 1][qt][3] - bf_hi(w[3]));
          pl[ps][qt] = as_bf16x8(r);
        }
      }
    }
    // O^T[d][q] += V^T[d][keys] P^T[keys][q]; lane group g holds keys {g*4..+3, 16+g*4..+3}
#pragma unroll
    for (int ps = 0; ps < 2; ++ps)
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const uint16_t* vp = sV + (d * 16 + l16) * LDV + ps * 32 + g * 4;
        const u32x2_t lo = ld8(vp), hi = ld8(vp + 16);
        const bf16x8_t vf = as_bf16x8(u32x4_t{lo[0], lo[1], hi[0], hi[1]});
        oacc[d][0] = mfma_bf16_16x16x32(vf, pf[ps][0], oacc[d][0]);
        oacc[d][1] = mfma_bf16_16x16x32(vf, pf[ps][1], oacc[d][1]);
        if constexpr (SPLIT) {
          const uint16_t* vl = sVl + (d * 16 + l16) * LDV + ps * 32 + g * 4;
          const u32x2_t lo2 = ld8(vl), hi2 = ld8(vl + 16);
          const bf16x8_t vfl = as_bf16x8(u32x4_t{lo2[0], lo2[1], hi2[0], hi2[1]});
          oacc[d][0] = mfma_bf16_16x16x32(vf, pl[ps][0], oacc[d][0]);
          oacc[d][1] = mfma_bf16_16x16x32(vf, pl[ps][1], oacc[d][1]);
          oacc[d][0] = mfma_bf16_16x16x32(vfl, pf[ps][0], oacc[d][0]);
          oacc[d][1] = mfma_bf16_16x16x32(vfl, pf[ps][1], oacc[d][1]);
        }
      }
  }

#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float l = lrun[qt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const float inv = 1.0f / l;
    const int qrel = q0 + wave * 32 + qt * 16 + l16;
    if (qrel >= m.t) continue;
    const int64_t row = m.q0 + qrel;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const int col = h * 128 + d * 16 + g * 4;
      if (a.o_f32) {
        float* dst = a.o_f32 + row * 8192 + col;
        *reinterpret_cast<f32x4_t*>(dst) = oacc[d][qt] * inv;
      } else {
        st8(a.o + row * 8192 + col,
            u32x2_t{pack_bf16x2(oacc[d][qt][0] * inv, oacc[d][qt][1] * inv),
                    pack_bf16x2(oacc[d][qt][2] * inv, oacc[d][qt][3] * inv)});
      }
    }
  }
}

}  // namespace

hipError_t prefill_attention(const PrefillAttnArgs& a, hipStream_t s) {
  if (a.B <= 0 || a.max_t <= 0) return hipSuccess;
  dim3 grid(64, cdiv(a.max_t, PQ), a.B);
  if (a.split)
    hipLaunchKernelGGL(prefill_attn_kernel<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(prefill_attn_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla_k
