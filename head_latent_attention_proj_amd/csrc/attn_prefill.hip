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
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mla_k {

namespace {

constexpr int PQ = 128;   // queries per workgroup
constexpr int PKB = 64;   // keys per block
// Padded LDS rows, sized for gfx950's LDS: a 16-byte read serves 16 lanes per cycle from 64 four-byte
// banks, namely the quads (lane / 4) of one half-wave whose index has one parity of its low three bits
// (8 rows l16 of each of two lane groups g); an 8-byte read serves a half-wave (16 rows x 2 g) per
// cycle. The key reads (row l16, 16 bytes at 16 g) meet distinct banks with 416-byte rows (400 left
// them 2-way conflicted), the value reads (row l16, 8 bytes at 8 g) with 144-byte rows (136: 2-way).
constexpr int LDK = 208;  // sK row: 192 features + pad (416 B)
constexpr int LDV = 72;   // sV row: 64 keys + pad (144 B)
constexpr float LOG2E = 1.4426950408889634f;

MLA_DEV u32x2_t ld8(const void* p) { return *reinterpret_cast<const u32x2_t*>(p); }
MLA_DEV void st8(void* p, const u32x2_t& v) { *reinterpret_cast<u32x2_t*>(p) = v; }

// SPLIT (FP8 weights): q arrives in fp16 (q_b's output; the rotary part is rotated here from the fp16
// values and rounded again), k_pe in float32, K_nope and V^T in fp16 with an fp16 residual plane of
// V^T. Keys are rounded to fp16 (11 significant bits) and the probabilities too; each score is one fp16 product, each value product two (value and its residual), so the
// values enter at about 22 bits. Chosen from a CPU emulation of these roundings against the W8A8
// float64 layer (the FP8 path's o_proj quantiser amplifies any rounding of its input): bf16
// hi + lo parts on every operand (three products each way) gave 8.0e-3 max-abs on the layer
// output, this form 9.8e-3, a single fp16 product for the values too 1.6e-2.
template <bool SPLIT>
__global__ __launch_bounds__(256, 2) void prefill_attn_kernel(PrefillAttnArgs a) {
  using frag_t = std::conditional_t<SPLIT, f16x8_t, bf16x8_t>;
  auto as_frag = [](const u32x4_t& v) {
    if constexpr (SPLIT) return as_f16x8(v);
    else return as_bf16x8(v);
  };
  auto mm = [](const frag_t& x, const frag_t& y, const f32x4_t& c) {
    if constexpr (SPLIT) return mfma_f16_16x16x32(x, y, c);
    else return mfma_bf16_16x16x32(x, y, c);
  };
  auto pack2 = [](float lo, float hi) {
    if constexpr (SPLIT) return pack_f16x2(lo, hi);
    else return pack_bf16x2(lo, hi);
  };
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
  __shared__ __attribute__((aligned(16))) uint16_t sVl[SPLIT ? 128 * LDV : 8];  // value residuals

  // ---- Q fragments: B operand of S^T, column = query, 8 features of group g per k-step
  frag_t qf[2][6];
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
      const u32x4_t raw = ld16((const uint16_t*)a.q + qoff + ks * 32 + g * 8);
      if (ks < 4) {
        qf[qt][ks] = as_frag(raw);
        continue;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = SPLIT ? f16_lo(raw[j]) : bf_lo(raw[j]);
        x[2 * j + 1] = SPLIT ? f16_hi(raw[j]) : bf_hi(raw[j]);
      }
      {  // rotary part, rotated at the query's position
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
      qf[qt][ks] = as_frag(u32x4_t{pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7])});
    }
  }

  // ---- block staging (global -> registers -> LDS), one block ahead; the value residuals (FP8) are
  // loaded at staging time instead (held across the block's math they would spill registers)
  constexpr int NPP = SPLIT ? 4 : 2;  // k_pe pieces per thread (float32 in FP8 entries)
  u32x4_t pk[4], pp[NPP], pv[4];
  const int kr = tid >> 4, kc = (tid & 15) * 8;   // K_nope: 16 threads per key row (256 B)
  const int pr = tid >> 3, pc = (tid & 7) * 8;    // V^T: 8 threads per 128-byte row; bf16 k_pe likewise
  const int fr = tid >> 2, fc = (tid & 3) * 16;   // float32 k_pe: 4 threads per 256-byte row
  // Bases common to the workgroup (scalar registers) plus 32-bit per-lane byte offsets: a load
  // costs one address register and a 32-bit add instead of a 64-bit multiply-add per block.
  const uint8_t* kn_base = (const uint8_t*)(a.knope + ((int64_t)m.kbase * 64 + h) * 128);
  const uint8_t* pe_base = a.cache + m.krow0 * a.entry_bytes + a.kpe_off;
  const uint8_t* vt_base = (const uint8_t*)(a.vt + (int64_t)(h * 128) * a.vt_ld + m.kbase);
  const uint8_t* vl_base = SPLIT ? (const uint8_t*)(a.vt_lo + (int64_t)(h * 128) * a.vt_ld + m.kbase) : nullptr;
  // value row piece (i, this thread) of block kb: byte offset from vt_base / vl_base
  auto voff = [&](int i, int kb) { return ((uint32_t)(i * 32 + pr) * (uint32_t)a.vt_ld + (uint32_t)(kb + pc)) * 2u; };
  // keys past the last one are not written by kv_b: their value pieces are zeroed
  auto vmask = [&](int kb, int j) {
    const int key = kb + pc + 2 * j;
    uint32_t mask = 0xffffffffu;
    if (key >= n_keys) mask &= 0xffff0000u;
    if (key + 1 >= n_keys) mask &= 0x0000ffffu;
    return mask;
  };
  auto gload = [&](int blk) {
    const int kb = blk * PKB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t key = (uint32_t)min(kb + i * 16 + kr, n_keys - 1);
      pk[i] = ld16(kn_base + (key * (64u * 128u * 2u) + (uint32_t)kc * 2u));
    }
    if constexpr (SPLIT) {
      const uint32_t key = (uint32_t)min(kb + fr, n_keys - 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) pp[i] = ld16(pe_base + (key * (uint32_t)a.entry_bytes + (uint32_t)(fc + 4 * i) * 4u));
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t key = (uint32_t)min(kb + i * 32 + pr, n_keys - 1);
        pp[i] = ld16(pe_base + (key * (uint32_t)a.entry_bytes + (uint32_t)pc * 2u));
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = ld16(vt_base + voff(i, kb));
    if (kb + PKB > n_keys) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) pv[i][j] &= vmask(kb, j);
    }
  };
  auto sstore = [&](int blk) {
    const int kb = blk * PKB;
    u32x4_t pvl[SPLIT ? 4 : 1];
    if constexpr (SPLIT) {
#pragma unroll
      for (int i = 0; i < 4; ++i) pvl[i] = ld16(vl_base + voff(i, kb));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) st16(sK + (i * 16 + kr) * LDK + kc, pk[i]);
    if constexpr (SPLIT) {  // float32 rotary key -> fp16
#pragma unroll
      for (int i = 0; i < 4; ++i)
        st8(sK + fr * LDK + 128 + fc + 4 * i,
            u32x2_t{pack_f16x2(__uint_as_float(pp[i][0]), __uint_as_float(pp[i][1])),
                    pack_f16x2(__uint_as_float(pp[i][2]), __uint_as_float(pp[i][3]))});
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) st16(sK + (i * 32 + pr) * LDK + 128 + pc, pp[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t* d = sV + (i * 32 + pr) * LDV + pc;
      st8(d, u32x2_t{pv[i][0], pv[i][1]});
      st8(d + 4, u32x2_t{pv[i][2], pv[i][3]});
      if constexpr (SPLIT) {
        if (kb + PKB > n_keys) {
#pragma unroll
          for (int j = 0; j < 4; ++j) pvl[i][j] &= vmask(kb, j);
        }
        uint16_t* dl = sVl + (i * 32 + pr) * LDV + pc;
        st8(dl, u32x2_t{pvl[i][0], pvl[i][1]});
        st8(dl + 4, u32x2_t{pvl[i][2], pvl[i][3]});
      }
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
    // the next block's loads, issued unconditionally (the last trip re-loads its own block, unused)
    // so that they sit in the same straight-line code as the score products
    gload(min(blk + 1, nblk - 1));
    const int kb = blk * PKB;
    if (kb > wq_hi) continue;  // every key of this block is in the future of this wave's queries

    f32x4_t sacc[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) sacc[kt][0] = sacc[kt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) {
      frag_t kf[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) kf[kt] = as_frag(ld16(sK + (kt * 16 + l16) * LDK + ks * 32 + g * 8));
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        sacc[kt][0] = mm(kf[kt], qf[0][ks], sacc[kt][0]);
        sacc[kt][1] = mm(kf[kt], qf[1][ks], sacc[kt][1]);
      }
    }

    if (kb + PKB - 1 > wq_lo) {  // wave-uniform: only blocks that reach past the wave's first query
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (kb + kt * 16 + g * 4 + e > qpos[qt]) sacc[kt][qt][e] = -INFINITY;
    }
    // scores stay unscaled here: the scale (softmax scale times log2 e, positive) commutes with
    // the maximum and is applied inside each exponent's fused multiply-add
    float bmax[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sacc[kt][qt][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      bmax[qt] = mx * sl2;
    }
    // The running maximum is raised only when some query's block maximum exceeds it by more than
    // 8 (log2 units; one wave-uniform decision for both query tiles): probabilities stay <= 256
    // and the output accumulators are rescaled rarely. The first block holds key 0, visible to
    // every query, so mrun is finite after it.
    if (__any(bmax[0] > mrun[0] + 8.0f || bmax[1] > mrun[1] + 8.0f)) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const float mnew = fmaxf(mrun[qt], bmax[qt]);
        const float alpha = exp2_flush(mrun[qt] - mnew);
        mrun[qt] = mnew;
        lrun[qt] *= alpha;
#pragma unroll
        for (int d = 0; d < 8; ++d) oacc[d][qt] *= alpha;
      }
    }
    // probabilities, their sums and the value products of both query tiles in one stretch of
    // straight-line code: one tile's exponentials can issue while the other's products run
    frag_t pf[2][2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
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
      for (int ps = 0; ps < 2; ++ps)
        pf[ps][qt] = as_frag(u32x4_t{pack2(sacc[2 * ps][qt][0], sacc[2 * ps][qt][1]),
                                     pack2(sacc[2 * ps][qt][2], sacc[2 * ps][qt][3]),
                                     pack2(sacc[2 * ps + 1][qt][0], sacc[2 * ps + 1][qt][1]),
                                     pack2(sacc[2 * ps + 1][qt][2], sacc[2 * ps + 1][qt][3])});
    }
    // O^T[d][q] += V^T[d][keys] P^T[keys][q]; lane group g holds keys {g*4..+3, 16+g*4..+3}
#pragma unroll
    for (int ps = 0; ps < 2; ++ps)
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const uint16_t* vp = sV + (d * 16 + l16) * LDV + ps * 32 + g * 4;
        const u32x2_t lo = ld8(vp), hi = ld8(vp + 16);
        const frag_t vf = as_frag(u32x4_t{lo[0], lo[1], hi[0], hi[1]});
        oacc[d][0] = mm(vf, pf[ps][0], oacc[d][0]);
        oacc[d][1] = mm(vf, pf[ps][1], oacc[d][1]);
        if constexpr (SPLIT) {
          const uint16_t* vl = sVl + (d * 16 + l16) * LDV + ps * 32 + g * 4;
          const u32x2_t lo2 = ld8(vl), hi2 = ld8(vl + 16);
          const frag_t vfl = as_frag(u32x4_t{lo2[0], lo2[1], hi2[0], hi2[1]});
          oacc[d][0] = mm(vfl, pf[ps][0], oacc[d][0]);
          oacc[d][1] = mm(vfl, pf[ps][1], oacc[d][1]);
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
    if (SPLIT && a.o_codes) {
      // the o_proj input quantiser ("Key-value latent" page, linear excerpt: dynamic activations,
      // one scale per token and 128 features = this head's 128 values of the token): s = amax/448
      // (1 for an all-zero group), code = RNE-saturating E4M3 of v/s, in float32. The token's 128
      // values sit in the four lanes l16 + 16g; all lanes take part in the exchange.
      float v[8][4], amax = 0.f;
#pragma unroll
      for (int d = 0; d < 8; ++d)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[d][e] = oacc[d][qt][e] * inv;
          amax = fmaxf(amax, fabsf(v[d][e]));
        }
      amax = fmaxf(amax, __shfl_xor(amax, 16));
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      if (qrel >= m.t) continue;
      const int64_t row = m.q0 + qrel;
      const float sc = amax == 0.f ? 1.0f : amax / 448.0f;
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) w |= e4m3_rne_sat(v[d][e] / sc) << (8 * e);
        *reinterpret_cast<uint32_t*>(a.o_codes + row * 8192 + h * 128 + d * 16 + g * 4) = w;
      }
      if (g == 0) a.o_scales[row * 64 + h] = sc;
      continue;
    }
    if (qrel >= m.t) continue;
    const int64_t row = m.q0 + qrel;
#pragma unroll
    for (int d = 0; d < 8; ++d)
      st8(a.o + row * 8192 + h * 128 + d * 16 + g * 4,
          u32x2_t{pack_bf16x2(oacc[d][qt][0] * inv, oacc[d][qt][1] * inv),
                  pack_bf16x2(oacc[d][qt][2] * inv, oacc[d][qt][3] * inv)});
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
