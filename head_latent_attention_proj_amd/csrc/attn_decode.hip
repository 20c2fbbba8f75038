// Decode attention in the 512-feature latent space, split over positions, then merged and
// mapped to the value heads.
//
// For one new token of a sequence holding L positions (this step's entry included), head h:
//   s_j = scale * ( q_lat_h . c_hat_j + RoPE(q_pe_h) . k_pe_j ),  j = 0 .. L-1
//   o_lat_h = sum_j softmax(s)_j c_hat_j                            (512 features)
//   o_h = W_UV,h o_lat_h                                            (128 value features)
// with q_lat_h = W_UK,h^T q_nope_h. This equals the pages' scores q.k over 192 features and the
// value mix sum_j a_j v_j (W_UK / W_UV are output features 0..127 / 128..255 of each head's 256
// in kv_b: "Key content up-projection" page, Explanation). The cache therefore streams one
// 576-feature entry per position for all 64 heads at once instead of 64 x (192 + 128) rebuilt
// features ("KV cache" page: 20,480 vs 576 values per position).
//
// FP8 cache entries hold the latent as E4M3FN codes with one float32 scale per 128 features
// (the quantised RMSNorm output, which is exactly what kv_b consumes). Codes are widened exactly
// to fp16 while staging (every E4M3 value is an fp16 value); the group scales are applied per
// position to the partial scores of each group and to the probabilities of the value mix.
// Operand precision (chosen from a CPU emulation of this kernel's roundings against the W8A8
// float64 layer, whose o_proj input quantiser turns any error of o into flipped codes): the
// queries and the rotary key are fp16 (11 significant bits; one MFMA per score product), the
// probabilities times the group scales are carried as fp16 high + residual parts (about 22 bits),
// because a single rounding of them moves the output of a one- or two-key decode by up to
// 1.9e-2 max-abs.
//
// Work layout: one workgroup = (sequence, split of `chunk` positions), 8 waves = 4 head groups of
// 16 x 2 feature halves. Heads are the MFMA column dimension, so one 32-position block staged in
// LDS feeds every head: S^T = C Q^T (A = cache rows, B = queries held in registers), then
// O^T = C^T P^T with the block's columns read by LDS transpose reads. The next
// block's loads are in flight (in registers) while a block is used. Each split writes (max, sum,
// unnormalised o) per head; the merge kernel combines the splits and normalises; W_UV is applied
// afterwards as a batched bf16 MFMA product (one 128 x 512 matrix per head).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mla_k {

namespace {

constexpr int DKB = 32;    // positions per block
constexpr int LDC = 576;   // sC row: 576 fp16 features in 16-byte chunks, swizzled per row (swz)
constexpr int HALF = 288;  // score features per wave: [0, 288) or [288, 576)
constexpr float LOG2E = 1.4426950408889634f;

MLA_DEV u32x2_t ld8(const void* p) { return *reinterpret_cast<const u32x2_t*>(p); }

// Chunk swizzle of a staged FP8 block: 16-byte chunk c of row r sits at chunk c ^ swz(r) (only the low
// three bits of c change, so a chunk stays in its aligned 128-byte group). gfx950's LDS, as its
// bank-conflict counter shows: a 16-byte read serves 16 lanes per cycle from 64 four-byte banks, those
// of one half-wave whose quad index (lane / 4) has one parity of its low three bits; an 8-byte read
// (the transposed one too) serves a half-wave per cycle; a 16-byte write serves 8 consecutive lanes per
// cycle from 32 banks. With r's bits b1..b3, swz = (b2 ^ b3, b1, b3) puts every one of this kernel's
// accesses on distinct banks: the score reads (rows 0..15 at one chunk per 16-lane group: 4 cycles
// instead of the 8 of a layout tuned for 16 consecutive lanes), the transposed value reads and the
// staging writes (8 rows of one parity at one chunk). swz(r + 16) = swz(r).
MLA_DEV int swz(int r) { return ((((r >> 2) ^ (r >> 3)) & 1) << 2) | (((r >> 1) & 1) << 1) | ((r >> 3) & 1); }

// element index of feature f of row r in the swizzled block
MLA_DEV int sidx(int r, int f) { return r * LDC + (((f >> 3) ^ swz(r)) << 3) + (f & 7); }

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// LDS transpose read (ds_read_b64_tr_b16): within each group of 16 lanes, lane i receives element
// (i % 4) of the 8-byte chunks addressed by lanes 4j + i/4, j = 0..3. With lane r of a group
// pointing at row (r/4), columns 4*(r%4) .. +3 of a row-major tile, lane i receives column i of
// rows 0..3: a K-major fragment read out of a K x N row-major tile. The value is bit-cast whole
// (per-element access of the 16-bit vector is avoided).
MLA_DEV u32x2_t ds_read_tr16(const uint16_t* p) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)p);
  return __builtin_bit_cast(u32x2_t, v);
}

// four E4M3FN codes (one 32-bit word) -> two packed fp16 pairs (exact; gfx950 converts a code
// pair to an fp16 pair in one instruction, unit scale)
MLA_DEV u32x2_t e4m3x4_to_f16(uint32_t w) {
  const f16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  const f16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  return u32x2_t{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// Probabilities enter the value mix times the position's group scale and this power of two, so that
// their fp16 high and residual parts stay in fp16's normal range (p <= 2^8 after the lazy rescale,
// group scales of RMSNorm outputs far below 1); the partial outputs are scaled back on the way out.
constexpr float P_PRESCALE = 64.0f;

// FP8 cache blocks whose loads are in flight while a block is used (at most 3)
constexpr int FP8_AHEAD = 2;

// FP8 cache entries. 8 waves: wave = hg + 4*lh, head group hg (heads hg*16 .. +15), half lh. A
// wave forms the partial scores of its 16 heads over features [lh*288, lh*288+288) and, after the
// two halves are added through LDS, mixes latent features [lh*256, lh*256+256). Two waves per SIMD
// hide each other's LDS and memory latency.
__global__ __launch_bounds__(512, 1) void decode_attn_fp8_kernel(DecodeAttnArgs a) {
  using namespace mla_dims;
  const int split = blockIdx.x, b = blockIdx.y;
  const int seq = a.seq_ids[b];
  const int L = a.len[seq];
  const int c0 = split * a.chunk;
  if (c0 >= L) return;
  const int c1 = min(L, c0 + a.chunk);
  const int nblk = cdiv(c1 - c0, DKB);
  const int eb = a.entry_bytes;
  constexpr int kpe_off = KV_LORA + 16;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave & 3, lh = wave >> 2;
  const int l16 = lane & 15, g = lane >> 4;
  const int head = hg * 16 + l16;

  __shared__ __attribute__((aligned(16))) uint16_t sC[DKB * LDC];      // fp16 [position][576], swizzled
  __shared__ __attribute__((aligned(16))) float xS[8][64][12];         // partial scores [wave][lane][8 + pad]
  __shared__ __attribute__((aligned(16))) float sScale[4][DKB];        // group scales x P_PRESCALE [group][position]

  // ---- staging through registers, FP8_AHEAD blocks ahead (one register set per block in flight):
  // codes as position pairs (pair kp = tid & 15, 16-code chunk cc = tid >> 4), the rotary key (every
  // thread one chunk of 4 float32 features), group scales (threads 256..287 one position each)
  u32x4_t rl[FP8_AHEAD][2], rp[FP8_AHEAD], rs[FP8_AHEAD];
  // A 32-position block lies in one run of consecutive slots (a page holds whole blocks): its first
  // slot is looked up once per block, rows are offsets from it.
  auto gload = [&](int blk, auto setc) {
    constexpr int S = decltype(setc)::value;
    const int kb = c0 + blk * DKB;
    const uint8_t* bb = a.cache + slot_of(a.map, seq, kb) * eb;
    const int kp = tid & 15, cc = tid >> 4;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int key = min(kb + 2 * kp + u, c1 - 1);  // past the split's end: re-read (masked)
      rl[S][u] = ld16(bb + (key - kb) * eb + cc * 16);
    }
    {  // every thread loads (threads 256..287 keep theirs): the same number of loads in every wave;
       // the other waves read one wave-uniform address (one cache line per instruction)
      const int key = min(kb + (wave == 4 ? (tid & (DKB - 1)) : 0), c1 - 1);
      rs[S] = ld16(bb + (key - kb) * eb + KV_LORA);
    }
    const int key = min(kb + (tid >> 4), c1 - 1);
    rp[S] = ld16(bb + (key - kb) * eb + kpe_off + (tid & 15) * 16);
  };
  auto sstore = [&](auto setc) {
    constexpr int S = decltype(setc)::value;
    const int kp = tid & 15, cc = tid >> 4;
#pragma unroll
    for (int hlf = 0; hlf < 2; ++hlf) {  // codes 8*hlf .. 8*hlf+7 of the chunk, positions 2kp and 2kp+1
      const u32x2_t x01 = e4m3x4_to_f16(rl[S][0][2 * hlf]), x23 = e4m3x4_to_f16(rl[S][0][2 * hlf + 1]);
      const u32x2_t y01 = e4m3x4_to_f16(rl[S][1][2 * hlf]), y23 = e4m3x4_to_f16(rl[S][1][2 * hlf + 1]);
      st16(sC + sidx(2 * kp, cc * 16 + hlf * 8), u32x4_t{x01[0], x01[1], x23[0], x23[1]});
      st16(sC + sidx(2 * kp + 1, cc * 16 + hlf * 8), u32x4_t{y01[0], y01[1], y23[0], y23[1]});
    }
    if (tid >= 256 && tid < 256 + DKB) {
#pragma unroll
      for (int q = 0; q < 4; ++q) sScale[q][tid - 256] = __uint_as_float(rs[S][q]) * P_PRESCALE;
    }
    // rotary key: 4 float32 features -> fp16
    const int pos = tid >> 4, f4 = (tid & 15) * 4;
    *reinterpret_cast<u32x2_t*>(sC + sidx(pos, KV_LORA + f4)) =
        u32x2_t{pack_f16x2(__uint_as_float(rp[S][0]), __uint_as_float(rp[S][1])),
                pack_f16x2(__uint_as_float(rp[S][2]), __uint_as_float(rp[S][3]))};
  };
  // the first blocks are in flight during the query set-up. Block indices past the split's last
  // block re-read the last block (never staged): every loop trip then issues the same loads, so the
  // compiler's wait before a set is used covers that set only, not the sets issued after it.
  gload(0, std::integral_constant<int, 0>{});
  if constexpr (FP8_AHEAD > 1) gload(min(1, nblk - 1), std::integral_constant<int, 1 % FP8_AHEAD>{});
  if constexpr (FP8_AHEAD > 2) gload(min(2, nblk - 1), std::integral_constant<int, 2 % FP8_AHEAD>{});

  // ---- query fragments (B operand), fp16: column = head, features lh*288 + ks*32 + g*8 .. +7;
  // the latent part is the absorbed product (or the sum of two float32 parts), features >= 512 are the rotary
  // part, rotated here at the query's position
  f16x8_t qf[9];
  {
    const int pos = L - 1;
#pragma unroll
    for (int ks = 0; ks < 9; ++ks) {
      const int f = lh * HALF + ks * 32 + g * 8;
      float v[8];
      if (f < KV_LORA && a.q_lat_f16) {
        qf[ks] = as_f16x8(ld16((const uint16_t*)a.q_lat + ((int64_t)b * 64 + head) * KV_LORA + f));
        continue;
      }
      if (f < KV_LORA) {
        const float* qlf = (const float*)a.q_lat + ((int64_t)b * 64 + head) * KV_LORA + f;
        const f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(qlf), v1 = *reinterpret_cast<const f32x4_t*>(qlf + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[j] = v0[j];
          v[4 + j] = v1[j];
        }
        if (a.q_lat_lo != 0) {
          const float* qlr = qlf + a.q_lat_lo;
          const f32x4_t r0 = *reinterpret_cast<const f32x4_t*>(qlr), r1 = *reinterpret_cast<const f32x4_t*>(qlr + 4);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[j] += r0[j];
            v[4 + j] += r1[j];
          }
        }
      } else {
        const int pair0 = (f - KV_LORA) >> 1;
        const float* qpf = (const float*)a.q + ((int64_t)b * 64 + head) * QK + NOPE + (f - KV_LORA);
        const f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(qpf), v1 = *reinterpret_cast<const f32x4_t*>(qpf + 4);
        const float x[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float c = a.rope_cs[(int64_t)pos * 32 + pair0 + j];
          const float sn = a.rope_cs[(int64_t)a.max_pos * 32 + (int64_t)pos * 32 + pair0 + j];
          v[2 * j] = x[2 * j] * c - x[2 * j + 1] * sn;
          v[2 * j + 1] = x[2 * j] * sn + x[2 * j + 1] * c;
        }
      }
      qf[ks] = as_f16x8(u32x4_t{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]), pack_f16x2(v[4], v[5]),
                                pack_f16x2(v[6], v[7])});
    }
  }

  // scores are formed with the group scales times P_PRESCALE (the rotary part times it too): the
  // power of two comes out exactly in the exponent's scale
  const float sl2 = a.scale * LOG2E * (1.0f / P_PRESCALE);
  float mrun = -INFINITY, lrun = 0.f;
  f32x4_t oacc[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) oacc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto step = [&](const int blk, auto setc) {
    __syncthreads();  // the previous block's LDS reads are done
    sstore(setc);
    __syncthreads();
    gload(min(blk + FP8_AHEAD, nblk - 1), setc);
    const int kb = c0 + blk * DKB;

    // partial S^T[key][head] over this wave's 288 features, two key tiles; each 128-wide feature
    // group is summed on its own and multiplied by its per-position scale
    f32x4_t sacc[2];
    sacc[0] = sacc[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    {
      // feature f = lh*288 + 32ks + 8g is chunk lh*36 + 4ks + g; its low three bits are 4*((lh+ks)&1) + g,
      // so two per-lane bases (even / odd lh+ks) plus a compile-time offset address every step
      const int sw = swz(l16);
      const uint16_t* rb[2] = {sC + l16 * LDC + ((g ^ sw) << 3), sC + l16 * LDC + (((4 + g) ^ sw) << 3)};
      // The half (lh) is wave-uniform; each half gets its own fully unrolled loop so that the
      // 128-feature group boundaries are compile-time; the group scales of the positions are read
      // once per block as 16-byte vectors, and the next step's fragments before this step's products.
      auto qk_half = [&](auto lhc) {
        constexpr int LH = decltype(lhc)::value;
        constexpr int G0 = (LH * HALF) >> 7;
        f32x4_t sc0[3], sc1[3];  // this half's groups (at most three below the rotary part)
#pragma unroll
        for (int gi = 0; gi < 3; ++gi) {
          const int grp = min(G0 + gi, 3);
          sc0[gi] = *reinterpret_cast<const f32x4_t*>(&sScale[grp][g * 4]);
          sc1[gi] = *reinterpret_cast<const f32x4_t*>(&sScale[grp][16 + g * 4]);
        }
        f32x4_t t0 = {0.f, 0.f, 0.f, 0.f}, t1 = t0;
        // chunk group (8 chunks) of step ks, as an element offset, and the base of its parity
        auto kaddr = [&](int ks) { return rb[(LH + ks) & 1] + (((LH * 36 + 4 * ks) >> 3) << 6); };
        f16x8_t k0 = as_f16x8(ld16(kaddr(0))), k1 = as_f16x8(ld16(kaddr(0) + 16 * LDC));
#pragma unroll
        for (int ks = 0; ks < 9; ++ks) {
          const int f = LH * HALF + ks * 32;
          const int grp = f < KV_LORA ? (f >> 7) : 4;
          f16x8_t n0 = k0, n1 = k1;
          if (ks + 1 < 9) {
            n0 = as_f16x8(ld16(kaddr(ks + 1)));
            n1 = as_f16x8(ld16(kaddr(ks + 1) + 16 * LDC));
          }
          t0 = mfma_f16_16x16x32(k0, qf[ks], t0);
          t1 = mfma_f16_16x16x32(k1, qf[ks], t1);
          const int fn = f + 32;
          const int gnext = ks + 1 < 9 ? (fn < KV_LORA ? (fn >> 7) : 4) : -1;
          if (gnext != grp) {  // group done: scale (rotary part: scale 1) and add
            if (grp < 4) {
              sacc[0] += t0 * sc0[grp - G0];
              sacc[1] += t1 * sc1[grp - G0];
            } else {
              sacc[0] += t0 * P_PRESCALE;
              sacc[1] += t1 * P_PRESCALE;
            }
            t0 = t1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
          k0 = n0;
          k1 = n1;
        }
      };
      if (lh == 0) qk_half(std::integral_constant<int, 0>{});
      else qk_half(std::integral_constant<int, 1>{});
    }
    // add the other half's partial scores (same order in both waves of a pair)
    // 16-byte LDS accesses on 48-byte lane rows: distinct banks for the writes (8 consecutive lanes
    // per cycle) and the reads (16 lanes per cycle)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) *reinterpret_cast<f32x4_t*>(&xS[wave][lane][4 * kt]) = sacc[kt];
    __syncthreads();
    const int other = wave ^ 4;
    float sv[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const f32x4_t theirs = *reinterpret_cast<const f32x4_t*>(&xS[other][lane][4 * kt]);
#pragma unroll
      for (int e = 0; e < 4; ++e) sv[kt][e] = lh == 0 ? sacc[kt][e] + theirs[e] : theirs[e] + sacc[kt][e];
    }
    // positions past the split's end occur in its last block only (wave-uniform test)
    if (kb + DKB > c1) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (kb + kt * 16 + g * 4 + e >= c1) sv[kt][e] = -INFINITY;
    }
    float bmax = -INFINITY;  // unscaled scores: the scale is applied in the exponent's fma
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) bmax = fmaxf(bmax, sv[kt][e]);
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    bmax *= sl2;  // the scale (positive) commutes with the maximum
    // the running maximum is raised only when a block's maximum exceeds it by more than 8 (log2
    // units): probabilities stay <= 256 and the accumulators are rescaled rarely (wave-uniform
    // decision; every split's first block has a valid position, so mrun is finite after it)
    if (__any(bmax > mrun + 8.0f)) {
      const float mnew = fmaxf(mrun, bmax);
      const float alpha = exp2_flush(mrun - mnew);
      lrun *= alpha;
#pragma unroll
      for (int c = 0; c < 16; ++c) oacc[c] *= alpha;
      mrun = mnew;
    }
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pv = exp2_flush(fmaf(sv[kt][e], sl2, -mrun));
        sv[kt][e] = pv;
        psum += pv;
      }
    lrun += psum;
    // probabilities as the B operand of the value mix: one copy per 128-feature group of this
    // wave's half, each position's probability times that position's group scale (and the
    // prescale), as fp16 high parts (pf) and residuals (pl)
    f16x8_t pf[2], pl[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float s_[2][4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const f32x4_t sc = *reinterpret_cast<const f32x4_t*>(&sScale[2 * lh + q][kt * 16 + g * 4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) s_[kt][e] = sv[kt][e] * sc[e];
      }
      u32x4_t w, r;
      w[0] = pack_f16x2(s_[0][0], s_[0][1]);
      w[1] = pack_f16x2(s_[0][2], s_[0][3]);
      w[2] = pack_f16x2(s_[1][0], s_[1][1]);
      w[3] = pack_f16x2(s_[1][2], s_[1][3]);
      r[0] = pack_f16x2(s_[0][0] - f16_lo(w[0]), s_[0][1] - f16_hi(w[0]));
      r[1] = pack_f16x2(s_[0][2] - f16_lo(w[1]), s_[0][3] - f16_hi(w[1]));
      r[2] = pack_f16x2(s_[1][0] - f16_lo(w[2]), s_[1][1] - f16_hi(w[2]));
      r[3] = pack_f16x2(s_[1][2] - f16_lo(w[3]), s_[1][3] - f16_hi(w[3]));
      pf[q] = as_f16x8(w);
      pl[q] = as_f16x8(r);
    }
    // O^T[dim][head] += C^T[dim][keys] P^T[keys][head] over this wave's 256 latent features;
    // lane group g holds keys g*4..+3 and 16+g*4..+3
    {
      // lane (l16, g): feature lh*256 + 16c + l16 at keys 4g..4g+3 (lo) and 16+4g.. (hi), read
      // as columns of the row-major block: lane r of the 16-lane group g points at key 4g + r/4,
      // features 4(r%4) .. +3 of the 16-feature tile
      // (swizzled: feature lh*256 + 16cc + 4(l16&3) is chunk lh*32 + 2cc + ((l16>>1)&1), whose low three
      // bits are 2(cc&3) + ((l16>>1)&1): four per-lane bases, one per cc mod 4, plus compile-time offsets)
      const int row = 4 * g + (l16 >> 2), swr = swz(row);
      const uint16_t* tp[4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        tp[m] = sC + row * LDC + lh * 256 + (((2 * m + ((l16 >> 1) & 1)) ^ swr) << 3) + 4 * (l16 & 1);
#pragma unroll
      for (int c0_ = 0; c0_ < 16; c0_ += 8) {
        u32x2_t lo[8], hi[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int cc = c0_ + c;
          lo[c] = ds_read_tr16(tp[cc & 3] + (cc >> 2) * 64);
          hi[c] = ds_read_tr16(tp[cc & 3] + 16 * LDC + (cc >> 2) * 64);
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const f16x8_t vt = as_f16x8(u32x4_t{lo[c][0], lo[c][1], hi[c][0], hi[c][1]});
          oacc[c0_ + c] = mfma_f16_16x16x32(vt, pf[c0_ >> 3], oacc[c0_ + c]);
          oacc[c0_ + c] = mfma_f16_16x16x32(vt, pl[c0_ >> 3], oacc[c0_ + c]);
        }
      }
    }
  };
  // one step per register set in every loop trip (each set named by a compile-time index), then the
  // last nblk % FP8_AHEAD blocks
  int blk = 0;
  for (; blk + FP8_AHEAD <= nblk; blk += FP8_AHEAD) {
    step(blk, std::integral_constant<int, 0>{});
    if constexpr (FP8_AHEAD > 1) step(blk + 1, std::integral_constant<int, 1 % FP8_AHEAD>{});
    if constexpr (FP8_AHEAD > 2) step(blk + 2, std::integral_constant<int, 2 % FP8_AHEAD>{});
  }
  if (FP8_AHEAD > 1 && blk < nblk) step(blk, std::integral_constant<int, 0>{});
  if (FP8_AHEAD > 2 && blk + 1 < nblk) step(blk + 1, std::integral_constant<int, 1 % FP8_AHEAD>{});

  // ---- split outputs: unnormalised o (relative to mrun, prescale taken out), running max and sum
  lrun += __shfl_xor(lrun, 16);
  lrun += __shfl_xor(lrun, 32);
  const int64_t pidx = ((int64_t)b * a.max_splits + split) * 64 + head;
  float* po = a.part_o + pidx * KV_LORA + lh * 256;
#pragma unroll
  for (int c = 0; c < 16; ++c)
    *reinterpret_cast<f32x4_t*>(po + c * 16 + g * 4) = oacc[c] * (1.0f / P_PRESCALE);
  if (lh == 0 && g == 0) {
    a.part_ml[pidx * 2] = mrun;
    a.part_ml[pidx * 2 + 1] = lrun;
  }
}

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// D(32x32) += A(32x16) B(16x32), bf16 in, float32 accumulate. Lane l supplies row (A) / column
// (B) l%32 and the eight k of group l/32; the result holds column l%32, rows
// 8*(e/4) + 4*(l/32) + e%4 for e = 0..15 (checked on gfx950).
MLA_DEV f32x16_t mfma_bf16_32x32x16(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}


// Latent decode attention, bf16 cache entries, 32x32 MFMA tiles. Workgroup = (sequence, split),
// 8 waves = 2 head groups of 32 x 4 feature quarters; each 16-byte cache fragment read from LDS
// feeds 32 heads. 32-position blocks are staged row-major through registers, two blocks ahead
// (two register sets alternate), so about 72 KB per CU are in flight while a block is used:
//   S^T = C Q^T      A = cache rows (ds_read_b128), B = queries in registers (9 k-steps of 16
//                    per wave); the four quarters' partial scores are added through LDS in a
//                    fixed order, identical in all four waves of a head group;
//   O^T += C^T P^T   A = cache columns via transpose reads (no transposed copy is written),
//                    B = probabilities straight from the score accumulators (same lane layout
//                    up to a fixed permutation of positions, used on both operands).
// The running maximum is raised only when a block's maximum exceeds it by more than 8 (log2
// units), so probabilities stay <= 256 and the output accumulators are rescaled rarely; the
// decision is taken for the whole wave.
// Staged bf16 block: unpadded 1152-byte rows, 16-byte chunk c of row r at c ^ swz2(r) (low three bits).
// With r's bits b1..b3, swz2 = (b1 ^ b3, b2, b1) puts the score reads (rows l32 at one chunk per lane
// half), the transposed value reads (rows 4 kg + l16 / 4 + 8 h, two chunks) and the staging writes (8
// consecutive chunks of a row) on distinct banks under gfx950's LDS grouping (see swz); 1168-byte
// padded rows left the value reads 2-way conflicted.
constexpr int LDC2 = 576;
MLA_DEV int swz2(int r) { return ((((r >> 1) ^ (r >> 3)) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 1) & 1); }

__global__ __launch_bounds__(512, 1) void decode_attn_bf16_kernel(DecodeAttnArgs a) {
  using namespace mla_dims;
  const int split = blockIdx.x, b = blockIdx.y;
  const int seq = a.seq_ids[b];
  const int L = a.len[seq];
  const int c0 = split * a.chunk;
  if (c0 >= L) return;
  const int c1 = min(L, c0 + a.chunk);
  const int nblk = cdiv(c1 - c0, DKB);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave & 1, fq = wave >> 1;
  const int l32 = lane & 31, kg = lane >> 5;
  const int head = hg * 32 + l32;

  // LDS: two cache blocks (+ a scratch row each; consecutive blocks alternate, so a block is
  // stored while no wave can still read the buffer: its previous block was last read before the
  // score exchange of the block in between) and the partial-score exchange; after the block loop
  // the same bytes stage the output rows
  constexpr int SC_ELEMS = (DKB + 1) * LDC2;
  constexpr int SC_BYTES = 2 * SC_ELEMS * 2;
  constexpr int XSL = 20;  // floats per lane in the score exchange: 16 + 4 (80-byte rows: distinct
                           // banks for the 16-byte writes and reads)
  constexpr int XS_BYTES = 8 * 64 * XSL * 4;
  constexpr int ST_LD = 256 + 4;  // staged half row: 256 floats + 16 bytes
  static_assert(SC_BYTES % 16 == 0 && 64 * ST_LD * 4 <= SC_BYTES + XS_BYTES, "LDS carve-up");
  __shared__ __attribute__((aligned(16))) uint8_t smem[SC_BYTES + XS_BYTES];
  uint16_t* sC = reinterpret_cast<uint16_t*>(smem);
  float* xS = reinterpret_cast<float*>(smem + SC_BYTES);  // [wave][lane][XSL]

  // staging: 32 rows x 72 chunks of 16 bytes; thread takes chunks c = tid + 512 i (i < 5, c < 2304).
  // Every load is issued unconditionally (an index past the block re-reads its last chunk and is
  // not stored): with no branch among them, the compiler's wait counts stay exact and the two
  // register sets really are in flight together.
  // Row and byte column of each of the thread's chunks are fixed; a load adds its row to a 32-bit
  // offset from the block's first slot (a uniform base in scalar registers: a 32-position block lies
  // in one run of consecutive slots, as a page holds whole blocks).
  int crow[5], ccol[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int c = min(tid + 512 * i, DKB * 72 - 1);
    crow[i] = c / 72;
    ccol[i] = (c % 72) * 16;
  }
  auto gload = [&](int blk, u32x4_t (&rs)[5]) {
    const int kb = c0 + blk * DKB;
    const uint8_t* bb = a.cache + slot_of(a.map, seq, kb) * BF16_ENTRY_BYTES;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int key = min(kb + crow[i], c1 - 1);  // rows past the split's end: re-read, masked later
      rs[i] = ld16(bb + (uint32_t)((key - kb) * BF16_ENTRY_BYTES + ccol[i]));
    }
  };
  auto sstore = [&](uint16_t* sCb, const u32x4_t (&rs)[5]) {
#pragma unroll
    for (int i = 0; i < 5; ++i) {  // chunks past the block go to a scratch row (no branch)
      const int c = tid + 512 * i;
      const int row = c / 72;
      st16(c < DKB * 72 ? sCb + row * LDC2 + (((c % 72) ^ swz2(row)) << 3) : sCb + DKB * LDC2 + (tid & 63) * 8, rs[i]);
    }
  };
  u32x4_t rA[5], rB[5];
  gload(0, rA);
  gload(min(1, nblk - 1), rB);

  // query fragments: column = head, features 144*fq + 16*ks + 8*kg .. +7 (>= 512: rotary part,
  // rotated at the query's position)
  bf16x8_t qf[9];
  {
    const int pos = L - 1;
    const uint16_t* ql = (const uint16_t*)a.q_lat + ((int64_t)b * 64 + head) * KV_LORA;
    const uint16_t* qp = (const uint16_t*)a.q + ((int64_t)b * 64 + head) * QK + NOPE;
#pragma unroll
    for (int ks = 0; ks < 9; ++ks) {
      const int f = 144 * fq + 16 * ks + 8 * kg;
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
          const float sn = a.rope_cs[(int64_t)a.max_pos * 32 + (int64_t)pos * 32 + pair0 + j];
          rot[j] = pack_bf16x2(x0 * c - x1 * sn, x0 * sn + x1 * c);
        }
        qf[ks] = as_bf16x8(rot);
      }
    }
  }
  // All prologue loads complete here, so that inside the block loop the compiler tracks only the
  // staging loads (otherwise it waits for every load before the first use of a query fragment
  // in each iteration, which drains the staging pipeline).
  __builtin_amdgcn_s_waitcnt(0);

  const float sl2 = a.scale * LOG2E;
  float m_used = -INFINITY, l_run = 0.f;
  f32x16_t o[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) o[t] = f32x16_t{};

  // One barrier between a block's store and its use; the exchange barrier of each block also
  // orders every read of the other buffer (two blocks back) before it is stored again, and every
  // read of the exchange area (one block back) before it is written again.
  auto step = [&](int blk, u32x4_t (&rs)[5]) {
    uint16_t* sCb = sC + (blk & 1) * SC_ELEMS;
    sstore(sCb, rs);
    __syncthreads();
    // unconditional (past the end: the last block again, from cache) so that no branch sits
    // among the loads and the compiler's wait counts stay exact
    gload(min(blk + 2, nblk - 1), rs);
    const int kb = c0 + blk * DKB;  // >= c1 for the masked extra block

    // partial S^T[pos][head] over this wave's 144 features (two chains, added at the end)
    f32x16_t s0 = f32x16_t{}, s1 = f32x16_t{};
    {
      // step ks reads chunk 18 fq + kg + 2 ks of row l32: one per-lane base for each ks mod 4 (the
      // swizzle changes the low three bits only) plus 8 chunks per 4 steps
      const int sw = swz2(l32);
      const uint16_t* ap[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) ap[m] = sCb + l32 * LDC2 + (((18 * fq + kg + 2 * m) ^ sw) << 3);
#pragma unroll
      for (int ks = 0; ks < 9; ks += 2) {
        s0 = mfma_bf16_32x32x16(as_bf16x8(ld16(ap[ks & 3] + 64 * (ks >> 2))), qf[ks], s0);
        if (ks + 1 < 9) s1 = mfma_bf16_32x32x16(as_bf16x8(ld16(ap[(ks + 1) & 3] + 64 * ((ks + 1) >> 2))), qf[ks + 1], s1);
      }
    }
    const f32x16_t sacc = s0 + s1;
    {
      float* xw = xS + (wave * 64 + lane) * XSL;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4_t*>(xw + 4 * q) = f32x4_t{sacc[4 * q], sacc[4 * q + 1], sacc[4 * q + 2], sacc[4 * q + 3]};
    }
    __syncthreads();
    // the four partial score sets of this head group, added in quarter order
    f32x4_t xs4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) xs4[q] = *reinterpret_cast<const f32x4_t*>(xS + (hg * 64 + lane) * XSL + 4 * q);
#pragma unroll
    for (int f = 1; f < 4; ++f)
#pragma unroll
      for (int q = 0; q < 4; ++q) xs4[q] += *reinterpret_cast<const f32x4_t*>(xS + ((hg + 2 * f) * 64 + lane) * XSL + 4 * q);
    float sv[16];
    float bmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) sv[e] = xs4[e >> 2][e & 3];  // unscaled: see the exponent below
    if (kb + DKB > c1) {  // the split's last block is partial (or a masked extra block): mask
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (kb + 8 * (e >> 2) + 4 * kg + (e & 3) >= c1) sv[e] = -INFINITY;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) bmax = fmaxf(bmax, sv[e]);
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    bmax *= sl2;  // the scale (positive) commutes with the maximum; exponents take it in a fma
    if (__any(bmax > m_used + 8.0f)) {  // wave-uniform
      const float mn = fmaxf(m_used, bmax);
      const float al = exp2_flush(m_used - mn);
      l_run *= al;
#pragma unroll
      for (int t = 0; t < 4; ++t) o[t] *= al;
      m_used = mn;
    }
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      sv[e] = exp2_flush(fmaf(sv[e], sl2, -m_used));
      psum += sv[e];
    }
    l_run += psum;
    bf16x8_t pf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      pf[ks] = as_bf16x8(u32x4_t{pack_bf16x2(sv[8 * ks], sv[8 * ks + 1]), pack_bf16x2(sv[8 * ks + 2], sv[8 * ks + 3]),
                                 pack_bf16x2(sv[8 * ks + 4], sv[8 * ks + 5]), pack_bf16x2(sv[8 * ks + 6], sv[8 * ks + 7])});

    // O^T[feature][head] over this wave's 128 latent features: 4 tiles x 2 position steps
    // lane (r, cc, kg) reads row 4 kg + r / 4 (+ 8, + 16 ks), feature 128 fq + cc + 4 (r % 4) + 32 t: chunk
    // 16 fq + cc / 8 + (r % 4) / 2 + 4 t at element 4 (r % 2) of it. Bases per (t mod 2, +8 rows): the
    // swizzle of row + 16 ks is that of row, t / 2 moves by 8 chunks.
    const int r = lane & 15, cc = 16 * ((lane >> 4) & 1);
    const uint16_t* tp[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 4 * kg + (r >> 2) + 8 * h;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        tp[tt][h] = sCb + row * LDC2 + 128 * fq + ((((cc >> 3) + ((r & 3) >> 1) + 4 * tt) ^ swz2(row)) << 3) + 4 * (r & 1);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x2_t w0 = ds_read_tr16(tp[t & 1][0] + 16 * ks * LDC2 + 64 * (t >> 1));
        const u32x2_t w1 = ds_read_tr16(tp[t & 1][1] + 16 * ks * LDC2 + 64 * (t >> 1));
        o[t] = mfma_bf16_32x32x16(as_bf16x8(u32x4_t{w0[0], w0[1], w1[0], w1[1]}), pf[ks], o[t]);
      }
  };
  // Both steps run unconditionally (with an odd block count the last step is a fully masked
  // block, which changes nothing): a branch around a step would again blur the wait counts.
  for (int blk = 0; blk < nblk; blk += 2) {
    step(blk, rA);
    step(blk + 1, rB);
  }

  // ---- split outputs: unnormalised o (relative to m_used), m_used and the sum per head
  l_run += __shfl_xor(l_run, 32);
  const int64_t prow = ((int64_t)b * a.max_splits + split) * 64;  // head 0 of this split
  if (fq == 0 && kg == 0) {
    a.part_ml[(prow + head) * 2] = m_used;
    a.part_ml[(prow + head) * 2 + 1] = l_run;
  }
  // The accumulators hold 32-byte runs of 32 different head rows; written straight out, every
  // store would touch 32 rows. Instead each half of the 512 features goes through LDS (the four
  // waves that own it write [head][256] rows), and every wave then stores whole 1 KB half rows.
  float* st = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    __syncthreads();  // LDS free: block loop done / previous half stored
    if ((fq >> 1) == half) {
      float* dst = st + head * ST_LD + 128 * (fq & 1) + 4 * kg;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<f32x4_t*>(dst + 32 * t + 8 * q) =
              f32x4_t{o[t][4 * q], o[t][4 * q + 1], o[t][4 * q + 2], o[t][4 * q + 3]};
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // wave w: heads 8w .. 8w+7, lane = 4 features of the half row
      const int hh = wave * 8 + i;
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(st + hh * ST_LD + 4 * lane);
      *reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(a.part_o) + (prow + hh) * KV_LORA + 256 * half + 4 * lane) =
          u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
  }
}

// Eight consecutive bf16 split-partial features (bf16 path: the attention kernel stores its
// unnormalised partial outputs in bf16) as two float32 quads.
MLA_DEV void load_part_bf16(const float* part, int64_t idx, f32x4_t& v0, f32x4_t& v1) {
  const u32x4_t raw = ld16(reinterpret_cast<const uint16_t*>(part) + idx);
  v0 = f32x4_t{bf_lo(raw[0]), bf_hi(raw[0]), bf_lo(raw[1]), bf_hi(raw[1])};
  v1 = f32x4_t{bf_lo(raw[2]), bf_hi(raw[2]), bf_lo(raw[3]), bf_hi(raw[3])};
}

// Merge of the splits, float32. One workgroup per (head h, sequence b): 4 groups of 64 threads
// take every 4th split each (8 latent features per thread, a running (max, sum, o) rescaled as
// splits arrive, four splits' loads in flight), then the 4 groups are combined through LDS in a
// fixed order:  o_lat = sum_s exp(m_s - m) o_s / sum_s exp(m_s - m) l_s.
// Output for the value up-projection (a bf16 MFMA product against W_UV):
//   bf16 weights: o_lat rounded to bf16, [B][64][512];
//   FP8 weights:  o_lat times the W_UV block scale of its 128-feature group (so the product runs
//                 on the exact code values), as bf16 high parts [B][64][512] followed by the bf16
//                 residuals [B][64][512]; the two products are added by the o_proj quantiser.
template <bool FP8>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeAttnArgs a) {
  using namespace mla_dims;
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, sg = tid >> 6, f = (tid & 63) * 8;
  __shared__ __attribute__((aligned(16))) float so[4][KV_LORA];
  __shared__ float sm[4], sl[4];
  const int ns = cdiv(a.len[a.seq_ids[b]], a.chunk);
  const int64_t base = (int64_t)b * a.max_splits * 64 + h;

  float m = -INFINITY, l = 0.f;
  f32x4_t o0 = {0.f, 0.f, 0.f, 0.f}, o1 = o0;
  for (int s0 = sg; s0 < ns; s0 += 16) {
    f32x2_t ml[4];
    f32x4_t v0[4], v1[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sp = min(s0 + 4 * u, ns - 1);  // past the end: re-read (not used)
      const int64_t p = base + (int64_t)sp * 64;
      ml[u] = *reinterpret_cast<const f32x2_t*>(a.part_ml + p * 2);
      if constexpr (FP8) {
        v0[u] = *reinterpret_cast<const f32x4_t*>(a.part_o + p * KV_LORA + f);
        v1[u] = *reinterpret_cast<const f32x4_t*>(a.part_o + p * KV_LORA + f + 4);
      } else {
        load_part_bf16(a.part_o, p * KV_LORA + f, v0[u], v1[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (s0 + 4 * u >= ns) break;
      const float mn = fmaxf(m, ml[u][0]);
      const float al = exp2f(m - mn), be = exp2f(ml[u][0] - mn);
      l = l * al + ml[u][1] * be;
      o0 = o0 * al + v0[u] * be;
      o1 = o1 * al + v1[u] * be;
      m = mn;
    }
  }
  *reinterpret_cast<f32x4_t*>(&so[sg][f]) = o0;
  *reinterpret_cast<f32x4_t*>(&so[sg][f + 4]) = o1;
  if ((tid & 63) == 0) {
    sm[sg] = m;
    sl[sg] = l;
  }
  __syncthreads();
  const float M = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
  float w[4], L = 0.f;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    w[g] = sl[g] > 0.f ? exp2f(sm[g] - M) : 0.f;  // a group with no split has l = 0, m = -inf
    L += w[g] * sl[g];
  }
  const float inv = 1.0f / L;
  const int c = 2 * tid;  // features c, c+1
  float v[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    float acc = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) acc += w[g] * so[g][c + e];
    v[e] = acc * inv;
  }
  const int64_t oi = ((int64_t)b * 64 + h) * KV_LORA + c;
  if constexpr (FP8) {
    const float sc = a.w_uv_s[(2 * h + 1) * 4 + (c >> 7)];
    v[0] *= sc;
    v[1] *= sc;
    const uint32_t hi = pack_bf16x2(v[0], v[1]);
    *reinterpret_cast<uint32_t*>(a.o_lat + oi) = hi;
    *reinterpret_cast<uint32_t*>(a.o_lat + (int64_t)a.B * 64 * KV_LORA + oi) =
        pack_bf16x2(v[0] - bf_lo(hi), v[1] - bf_hi(hi));
  } else {
    *reinterpret_cast<uint32_t*>(a.o_lat + oi) = pack_bf16x2(v[0], v[1]);
  }
}

// Merge of the splits followed by the value up-projection, bf16 weights, small batches (one
// launch instead of two; the W_UV rows are in flight while the partial outputs are merged).
// Workgroup = (head h, half of its 128 value rows, sequence b); both halves merge the head:
//   o_lat = sum_s exp(m_s - m) o_s / sum_s exp(m_s - m) l_s      (float32, in LDS)
//   o[b][h*128 + d] = sum_c W_UV,h[d][c] o_lat[c]                 (float32 sums, bf16 out)
// Wave w owns 8 rows of W_UV,h, one whole 1 KB row per load (lane = 8 features); the merge is
// split over the 8 waves by split index (8 features per thread) and combined through LDS in a
// fixed order. A wave's 8 row sums are reduced over its lanes by recursive halving (each step
// hands half of the rows to the partner lane), 10 lane exchanges instead of 48.
__global__ __launch_bounds__(512) void decode_merge_uv_kernel(DecodeAttnArgs a) {
  using namespace mla_dims;
  const int h = blockIdx.x >> 1, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int f = lane * 8;
  const int row0 = 64 * (blockIdx.x & 1) + 8 * wave;  // first value row of this wave
  __shared__ __attribute__((aligned(16))) float so[8][KV_LORA];
  __shared__ float sm[8], sl[8];

  u32x4_t wv[8];
  const uint16_t* wr = a.w_uv + h * a.uv_head_stride + (int64_t)row0 * KV_LORA + f;
#pragma unroll
  for (int i = 0; i < 8; ++i) wv[i] = ld16(wr + i * KV_LORA);

  const int ns = cdiv(a.len[a.seq_ids[b]], a.chunk);
  const int64_t base = (int64_t)b * a.max_splits * 64 + h;
  float m = -INFINITY, l = 0.f;
  f32x4_t o0 = {0.f, 0.f, 0.f, 0.f}, o1 = o0;
  for (int s0 = wave; s0 < ns; s0 += 16) {
    f32x2_t ml[2];
    f32x4_t v0[2], v1[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int sp = min(s0 + 8 * u, ns - 1);  // past the end: re-read (not used)
      const int64_t p = base + (int64_t)sp * 64;
      ml[u] = *reinterpret_cast<const f32x2_t*>(a.part_ml + p * 2);
      load_part_bf16(a.part_o, p * KV_LORA + f, v0[u], v1[u]);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (s0 + 8 * u >= ns) break;
      const float mn = fmaxf(m, ml[u][0]);
      const float al = exp2f(m - mn), be = exp2f(ml[u][0] - mn);
      l = l * al + ml[u][1] * be;
      o0 = o0 * al + v0[u] * be;
      o1 = o1 * al + v1[u] * be;
      m = mn;
    }
  }
  *reinterpret_cast<f32x4_t*>(&so[wave][f]) = o0;
  *reinterpret_cast<f32x4_t*>(&so[wave][f + 4]) = o1;
  if (lane == 0) {
    sm[wave] = m;
    sl[wave] = l;
  }
  __syncthreads();
  float M = sm[0];
#pragma unroll
  for (int g = 1; g < 8; ++g) M = fmaxf(M, sm[g]);
  float wg[8], L = 0.f;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    wg[g] = sl[g] > 0.f ? exp2f(sm[g] - M) : 0.f;  // a group with no split has l = 0, m = -inf
    L += wg[g] * sl[g];
  }
  const float inv = 1.0f / L;
  f32x4_t q0 = {0.f, 0.f, 0.f, 0.f}, q1 = q0;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    q0 += wg[g] * *reinterpret_cast<const f32x4_t*>(&so[g][f]);
    q1 += wg[g] * *reinterpret_cast<const f32x4_t*>(&so[g][f + 4]);
  }
  const float ol[8] = {q0[0] * inv, q0[1] * inv, q0[2] * inv, q0[3] * inv,
                       q1[0] * inv, q1[1] * inv, q1[2] * inv, q1[3] * inv};
  float r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc += bf_lo(wv[i][j]) * ol[2 * j];
      acc += bf_hi(wv[i][j]) * ol[2 * j + 1];
    }
    r[i] = acc;
  }
  // recursive halving: after the steps over lane bits 5, 4, 3 lane keeps row (lane >> 3) & 7
  // summed over 8 lanes; bits 2, 1, 0 finish the sum
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int n = 4 >> k;  // rows kept after this step
    const bool up = (lane >> (5 - k)) & 1;
#pragma unroll
    for (int j = 0; j < n; ++j) {
      const float give = up ? r[j] : r[j + n];
      const float keep = up ? r[j + n] : r[j];
      r[j] = keep + __shfl_xor(give, 32 >> k);
    }
  }
  float v = r[0];
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 1);
  if ((lane & 7) == 0) a.o[(int64_t)b * (HEADS * VD) + h * VD + row0 + (lane >> 3)] = f2bf(v);
}

}  // namespace

hipError_t decode_attention_splits(const DecodeAttnArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  dim3 g1(a.max_splits, a.B);
  if (a.fp8)
    hipLaunchKernelGGL(decode_attn_fp8_kernel, g1, dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL(decode_attn_bf16_kernel, g1, dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t decode_attention_merge(const DecodeAttnArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  dim3 g2(64, a.B);
  if (a.fp8) {
    hipLaunchKernelGGL(decode_merge_kernel<true>, g2, dim3(256), 0, s, a);
  } else {
    if (a.w_uv) {
      if (a.B > MERGE_UV_MAX_B) return hipErrorInvalidValue;
      hipLaunchKernelGGL(decode_merge_uv_kernel, dim3(128, a.B), dim3(512), 0, s, a);
    } else {
      hipLaunchKernelGGL(decode_merge_kernel<false>, g2, dim3(256), 0, s, a);
    }
  }
  return hipGetLastError();
}

}  // namespace mla_k
