// Shared device helpers for the gfx950 MLA kernels: bf16 handling, MFMA wrappers, launch structs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define MLA_DEV __device__ __forceinline__

// Kimi-K2 dimensions the kernels are specialised for.
namespace mla_dims {
constexpr int HIDDEN = 7168;
constexpr int Q_LORA = 1536;
constexpr int KV_LORA = 512;
constexpr int HEADS = 64;
constexpr int NOPE = 128;
constexpr int ROPE = 64;
constexpr int VD = 128;
constexpr int QK = NOPE + ROPE;          // 192
constexpr int ENTRY = KV_LORA + ROPE;    // 576 features per cached position
constexpr int QKVA_N = Q_LORA + ENTRY;   // 2112: fused q_a | kv_a output width
constexpr int KVB_N = HEADS * (NOPE + VD);  // 16384
constexpr int QB_N = HEADS * QK;         // 12288
constexpr int O_IN = HEADS * VD;         // 8192
constexpr int BF16_ENTRY_BYTES = ENTRY * 2;                 // 1152
constexpr int FP8_ENTRY_BYTES = KV_LORA + 16 + ROPE * 4;    // 784: codes | 4 scales | k_pe (fp32)
}  // namespace mla_dims

MLA_DEV float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

MLA_DEV uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

MLA_DEV uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// bf16 pair (packed in a uint32) -> two floats
MLA_DEV float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
MLA_DEV float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// D = A(16x32) * B(32x16) + C on one wave. Lane l holds row (A) / column (B) l%16 and eight
// consecutive k of group l/16; the result holds column l%16, rows 4*(l/16) .. +3. Any
// permutation of k applied identically to A and B leaves the product unchanged.
MLA_DEV f32x4_t mfma_bf16_16x16x32(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

MLA_DEV bf16x8_t as_bf16x8(const u32x4_t& v) { return __builtin_bit_cast(bf16x8_t, v); }

// fp16 (IEEE binary16, 11 significant bits) pair packed in a uint32, round to nearest even
MLA_DEV uint32_t pack_f16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
MLA_DEV float f16_lo(uint32_t u) { return (float)__builtin_bit_cast(f16x2_t, u)[0]; }
MLA_DEV float f16_hi(uint32_t u) { return (float)__builtin_bit_cast(f16x2_t, u)[1]; }
MLA_DEV f16x8_t as_f16x8(const u32x4_t& v) { return __builtin_bit_cast(f16x8_t, v); }

// D = A(16x32) * B(32x16) + C with fp16 operands, float32 accumulation; the lane layout is that of
// mfma_bf16_16x16x32.
MLA_DEV f32x4_t mfma_f16_16x16x32(const f16x8_t& a, const f16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// OCP E4M3FN encode of a float32, round to nearest even, saturating at +-448.
MLA_DEV uint32_t e4m3_rne_sat(float q) {
  const uint32_t sign = (__float_as_uint(q) >> 24) & 0x80u;
  const float a = fabsf(q);
  if (!(a < 448.f)) return sign | 0x7Eu;
  if (a < 0.015625f) {  // below 2^-6: subnormal grid m * 2^-9 (m = 8 is the smallest normal)
    const uint32_t m = (uint32_t)__builtin_rintf(a * 512.f);
    return sign | m;
  }
  const uint32_t ua = __float_as_uint(a);
  const uint32_t r = (ua + 0x7FFFFu + ((ua >> 20) & 1u)) >> 20;  // keep 3 mantissa bits, RNE
  const uint32_t e = (r >> 3) - 127u + 7u;
  return sign | (e << 3) | (r & 7u);
}

// Direct-to-LDS loads: every lane of the wave reads `size` bytes at its own global address and
// they land at l + size * lane (l wave-uniform).
MLA_DEV void gl2lds16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)l, 16, 0, 0);
}
MLA_DEV void gl2lds4(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)l, 4, 0, 0);
}

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt and lgkmcnt at their maxima).
template <int N>
MLA_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// LDS byte address of a __shared__ pointer.
MLA_DEV uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}


MLA_DEV u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
MLA_DEV void st16(void* p, const u32x4_t& v) { *reinterpret_cast<u32x4_t*>(p) = v; }

template <typename T>
MLA_DEV T wave_max(T v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
template <typename T>
MLA_DEV T wave_sum(T v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

// Where position `pos` of sequence `seq` lives in the cache: slot offset[seq] + pos (contiguous
// layout), or, with a block table, slot table[seq][pos >> page_shift] * page_size + the position's
// offset in its page (pages of 2^page_shift slots, page_shift >= 6).
struct SlotMap {
  const int64_t* offset = nullptr;
  const int32_t* table = nullptr;  // device [n_seqs][max_pages] page ids, or null
  int32_t page_shift = 0;
  int32_t max_pages = 0;
};
MLA_DEV int64_t slot_of(const SlotMap& m, int seq, int pos) {
  if (m.table) {
    const int pg = pos >> m.page_shift;
    return ((int64_t)m.table[(int64_t)seq * m.max_pages + pg] << m.page_shift) + (pos - (pg << m.page_shift));
  }
  return m.offset[seq] + pos;
}

// 2^x with the hardware's v_exp_f32 alone: exp2f adds a range fix-up (compare, select, scale)
// so that results below 2^-126 come out as denormals; softmax weights that small add nothing
// to a float32 sum, so the attention kernels take the flushed value. exp2(-inf) = 0.
MLA_DEV float exp2_flush(float x) { return __builtin_amdgcn_exp2f(x); }
