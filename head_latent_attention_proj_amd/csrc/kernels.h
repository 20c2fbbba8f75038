// Host-side launch interfaces of the gfx950 MLA kernels (implemented in the *.hip files).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla_k {

// ---------------------------------------------------------------------------------------------
// GEMM  C[b] = A[b] (M x K) * B[b]^T (B is N x K): both operands K-contiguous ("NT"), which is
// how nn.Linear stores its [out, in] weight. bf16 operands, fp32 accumulation.
// ---------------------------------------------------------------------------------------------
enum Epilogue : int {
  EPI_F32 = 0,   // C float32
  EPI_BF16 = 1,  // C bf16
  EPI_KVB = 2,   // kv_b output split per head: content keys -> knope[key][h*128+d] (bf16),
                 // values -> vt[(h*128+d) * vt_ld + key] (bf16, key-contiguous for P.V);
                 // FP8 kernels write fp16 there instead (see vt_lo)
  EPI_F16 = 3,   // C fp16 (FP8 kernels only: q_b's output at prefill, the attention's fp16 operand)
};

// Stage tags: one kernel symbol per projection so traces attribute time per stage.
enum GemmTag : int { TAG_NONE = 0, TAG_QKVA = 1, TAG_QB = 2, TAG_KVB = 3, TAG_OPROJ = 4, TAG_ABSORB = 5, TAG_UV = 6 };

struct GemmArgs {
  int tag = TAG_NONE;
  const void* A = nullptr;  int64_t lda = 0, sA = 0;  // elements; sA = batch stride
  const void* B = nullptr;  int64_t ldb = 0, sB = 0;
  void* C = nullptr;        int64_t ldc = 0, sC = 0;
  int M = 0, N = 0, K = 0, batch = 1;
  int epi = EPI_F32;
  // optional output scale per (batch, 128-column block): C *= c_scale[b * cs_stride + n / 128]
  const float* c_scale = nullptr;
  int64_t cs_stride = 0;
  // EPI_KVB destinations
  uint16_t* knope = nullptr;
  uint16_t* vt = nullptr;
  uint16_t* vt_lo = nullptr;     // FP8 kernels only: optional plane of the fp16 value residuals
                                 // (value - fp16(value)), same layout as vt
  int64_t vt_ld = 0;
  int64_t key_base = 0;
  // FP8 (E4M3FN codes) operands: A scales per (row, 128-group) with row stride as_ld floats;
  // B scales per (128-row block, 128-group) with row stride bs_ld floats.
  const float* a_scale = nullptr; int64_t as_ld = 0;
  const float* b_scale = nullptr; int64_t bs_ld = 0;
  // Decode-sized M with EPI_F32 only: the K range may be split over `ysplit_max` workgroups,
  // split y writing its partial sum to C + y * c_split_stride (the consumer adds the parts).
  int ysplit_max = 1;
  int64_t c_split_stride = 0;
  // EPI_BF16 only: residual added before the bf16 rounding, C[m][n] = bf16(acc + resid[m * ldr + n])
  // (batch 1; the decoder block's residual connection fused into o_proj)
  const uint16_t* resid = nullptr;
  int64_t ldr = 0;
  // Per-head kernel, EPI_F32 only: rows pair_rows .. 2 pair_rows - 1 of A are the residual parts of
  // rows 0 .. pair_rows - 1, and output row m (< pair_rows) is the sum of the two rows' products,
  // each multiplied by its c_scale first (high part + residual part, rounded as separate float32
  // operations). 0: off.
  int pair_rows = 0;
  // With pair_rows, without q8_codes: the sums stored as fp16 (round to nearest even; C in
  // 16-bit elements) instead of float32
  bool c_f16 = false;
  // With pair_rows and N = 128 (W_UV: one head's 128 features = one quantisation group per row):
  // instead of the float32 sums, the FP8 activation quantiser's codes (row stride q8_ld bytes, at
  // column batch * 128) and scales (row stride q8_sld floats, at index batch) of each row.
  // With pair_rows: A is float32 (lda, sA in floats) and the kernel forms each pair itself, the
  // bf16 high part bf16(v) and the residual bf16(v - high) of row m (< pair_rows).
  bool a_f32_split = false;
  // With a_f32_split and mg_ml (W_UV after the split decode attention; K = 512, N = 128): A is the
  // attention's partial outputs [b][mg_max_splits][64 heads][512] (unnormalised float32 sums, head
  // = batch), merged while staging with their (max, sum) pairs mg_ml (same index, log2 units; the
  // split count of row b is cdiv(mg_len[mg_seq[b]], mg_chunk)) and multiplied by mg_scale[(2 h + 1)
  // * 4 + k / 128]: row b's value is that scale times sum_s w_s o_s / sum_s w_s l_s, w_s =
  // 2^(m_s - max_s m_s).
  const float* mg_ml = nullptr;
  const int32_t* mg_seq = nullptr;
  const int32_t* mg_len = nullptr;
  int mg_chunk = 0, mg_max_splits = 0;
  const float* mg_scale = nullptr;
  uint8_t* q8_codes = nullptr;
  float* q8_scales = nullptr;
  int64_t q8_ld = 0, q8_sld = 0;
  // split-K scratch (workspace): fp32 partials, summed by a fixed-order reduction kernel
  float* part = nullptr;
  int64_t part_cap = 0;     // floats available in `part`
};

// Chooses a tile kernel (large M) or the in-workgroup split-K kernel (small M). Returns a
// hipError_t. gemm_ysplit() is the number of partial outputs a call writes (1 unless the
// caller allowed a split of K over workgroups).
hipError_t gemm_bf16(const GemmArgs& a, hipStream_t s);
int gemm_ysplit(const GemmArgs& a);
hipError_t gemm_fp8(const GemmArgs& a, hipStream_t s);
int64_t gemm_fp8_part_floats(int M, int N, int K, int batch);
int gemm_fp8_ysplit(const GemmArgs& a);
// Floats of split-K partials a (M, N, K, batch) GEMM may need.
int64_t gemm_part_floats(int M, int N, int K, int batch);

// ---------------------------------------------------------------------------------------------
// Per-call sequence metadata (device, filled by plan_kernel at the start of a prefill)
// ---------------------------------------------------------------------------------------------
struct SeqMeta {
  int64_t slot0;   // first cache slot of the sequence (contiguous layout)
  int64_t krow0;   // first row of the sequence's entries in the buffer the attention reads k_pe
                   // from: the cache's slot0, or (block table) the gathered copy's kbase
  int32_t l0;      // positions held before this call
  int32_t t;       // new tokens in this call
  int32_t q0;      // first row of this call's tokens in x / y
  int32_t kbase;   // first row of this sequence's rebuilt keys in the prefill workspace
  int32_t seq;     // sequence id
  int32_t pad;
};

hipError_t prefill_plan(const int32_t* seq_ids_d, const int32_t* q_start_d, const SlotMap& map,
                        const int32_t* len_d, int B, SeqMeta* meta, hipStream_t s);
// Block-table layout: the entries of each prefill sequence (positions 0 .. l0 + t - 1) copied into
// rows kbase .. of `dst` (row stride entry_bytes), so that kv_b and the attention read them
// contiguously. max_rows >= the largest l0 + t of the batch.
hipError_t gather_entries(const uint8_t* cache, const SlotMap& map, const SeqMeta* meta, int B, int max_rows,
                          int entry_bytes, uint8_t* dst, hipStream_t s);
hipError_t commit_lengths(const int32_t* seq_ids_d, const int32_t* q_start_d, int32_t* len_d, int B,
                          hipStream_t s);

// RMSNorm of the fused q_a | kv_a output (fp32 [n, 2112]): q_hat (bf16 [n, 1536]) and the cache
// entry [c_hat | rotated k_pe] of each token written to its slot. Prefill: token -> sequence
// through `meta`; decode (meta == nullptr): token b is sequence seq_ids[b] at position len[seq],
// and len[seq] is advanced by one after the entry is written.
struct NormArgs {
  const float* cqkv;     // [n_part][n][2112] partial sums (added here)
  int n_part;            // 1 .. 8
  int64_t part_stride;   // floats between parts
  const uint16_t* g_q;
  const uint16_t* g_kv;
  float eps;
  uint16_t* q_hat;
  const float* rope_cs;  // [max_pos][32] cos, then [max_pos][32] sin (float32)
  int max_pos;
  uint8_t* cache;
  int entry_bytes;
  int fp8;               // cache / q_hat in FP8 form
  uint8_t* q_hat_codes;  // FP8: q_hat codes [n, 1536] and scales [n, 12]
  float* q_hat_scales;
  int n_tokens;
  // prefill
  const SeqMeta* meta;
  int B;
  // decode
  const int32_t* seq_ids;
  int32_t* len;
  SlotMap map;           // where each position's entry lives
};
hipError_t norm_rope_append(const NormArgs& a, hipStream_t s);

// Decode q_b with the norms folded in (bf16 weights, the row-streaming plan): a.A is ignored,
// x = q_hat is built from na.cqkv in every workgroup, and the cache entries are written as
// norm_rope_append would. gemm_bf16_fuses_qnorm() tells whether the shape takes this path.
bool gemm_bf16_fuses_qnorm(const GemmArgs& a);
// Whether gemm_bf16 can take these arguments with a.pair_rows set (M = 2 pair_rows, EPI_F32, the
// per-head kernel's shapes); with pair_rows set on any other shape gemm_bf16 refuses the call.
bool gemm_bf16_pairs(const GemmArgs& a);
hipError_t gemm_bf16_qnorm(const GemmArgs& a, const NormArgs& na, hipStream_t s);

// Byte copy of n ready-made entries to positions pos0 .. pos0 + n - 1 of sequence seq (slots from
// `map`); len[seq] += n.
hipError_t cache_copy_append(uint8_t* cache, const SlotMap& map, const uint8_t* src, int entry_bytes, int n, int seq,
                             int pos0, int32_t* len_d, hipStream_t s);

// ---------------------------------------------------------------------------------------------
// Prefill attention (rebuilt keys/values, causal): o[row][h*128+d] bf16
// ---------------------------------------------------------------------------------------------
struct PrefillAttnArgs {
  const void* q;           // [n_tok][64][192] bf16 (split: fp16), rotary part not yet rotated
  const uint16_t* knope;   // [keys][64][128] bf16 (split: fp16)
  const uint16_t* vt;      // [64*128][vt_ld] bf16 (split: fp16)
  int64_t vt_ld;
  // split precision (FP8 weights): q is fp16, k_pe float32 in the entry; queries and keys enter as
  // fp16 and the values carry an fp16 residual plane vt_lo next to vt
  int split;
  const uint16_t* vt_lo;
  const uint8_t* cache;    // for the rotated shared key k_pe of each position
  int entry_bytes;
  int kpe_off;             // byte offset of k_pe inside an entry
  const float* rope_cs;
  int max_pos;
  const SeqMeta* meta;
  int B;
  int max_t;               // largest T_b (grid sizing)
  float scale;             // softmax scale
  uint16_t* o;             // [n_tok][8192] bf16 (when o_codes is null)
  // optional FP8 output, the o_proj input quantised in the epilogue (one 1 x 128 group = one
  // head of one token): E4M3FN codes [n_tok][8192] and float32 scales [n_tok][64]
  uint8_t* o_codes;
  float* o_scales;
};
hipError_t prefill_attention(const PrefillAttnArgs& a, hipStream_t s);

// ---------------------------------------------------------------------------------------------
// Decode attention in the latent space, split over positions, then merged
// ---------------------------------------------------------------------------------------------
struct DecodeAttnArgs {
  const void* q_lat;       // [B][64][512] q_nope absorbed through W_UK (bf16; FP8 mode: float32, or fp16)
  int64_t q_lat_lo;        // FP8 mode, when not 0: q_lat is the sum of two float32 arrays, this many floats apart
  bool q_lat_f16;          // FP8 mode: q_lat holds fp16 values (the attention's query precision)
  const void* q;           // [B][64][192] q (bf16; FP8 mode: float32): rotary part rotated on load
  const uint8_t* cache;
  int entry_bytes;
  int fp8;
  const float* rope_cs;
  int max_pos;
  const int32_t* seq_ids;
  SlotMap map;             // where each position's entry lives (pages hold whole 32-position blocks)
  const int32_t* len;      // positions held INCLUDING this step's entry
  int B;
  int chunk;               // positions per split
  int max_splits;          // splits per sequence in the grid
  float scale;
  float* part_o;           // [B][max_splits][64][512] unnormalised split outputs: fp32 (FP8), bf16 (bf16 weights)
  float* part_ml;          // [B][max_splits][64][2] (running max, sum)
  const float* w_uv_s;     // FP8: kv_b block scales [128][4] (W_UV,h blocks are rows 2h+1)
  uint16_t* o_lat;         // merged latent output, bf16 [B][64][512] (FP8: high parts, then residuals)
  // bf16 weights, B <= MERGE_UV_MAX_B: when w_uv is set the merge also applies W_UV and writes
  // o = [B][64 * 128] bf16 (o_lat is then not written)
  const uint16_t* w_uv;    // W_UV,h = rows [128][512] at w_uv + h * uv_head_stride
  int64_t uv_head_stride;
  uint16_t* o;
};
constexpr int MERGE_UV_MAX_B = 4;
// Split attention (partials) and the merge of the splits, as two launches. Output of the merge:
// o_lat (see DecodeAttnArgs), W_UV applied by the caller; or, with w_uv set, o.
hipError_t decode_attention_splits(const DecodeAttnArgs& a, hipStream_t s);
hipError_t decode_attention_merge(const DecodeAttnArgs& a, hipStream_t s);

// FP8 activation quantiser for a bf16/fp32 matrix [rows, K] (K multiple of 128).
// x2 (optional): a second matrix added to x element-wise before quantising (same layout).
hipError_t quantize_rows_f32(const float* x, const float* x2, int64_t ldx, int rows, int K, uint8_t* codes,
                             float* scales, hipStream_t s);
hipError_t quantize_rows_bf16(const uint16_t* x, int64_t ldx, int rows, int K, uint8_t* codes, float* scales,
                              hipStream_t s);

// q_nope parts of float32 q [n][64][192] -> bf16 high parts [n][64][128] followed by the bf16
// residuals [n][64][128] (the FP8 decode absorbs both and adds the two products).
hipError_t split_q_nope(const float* q, int n, uint16_t* out, hipStream_t s);

// Decoder-block input RMSNorm over the hidden features (K = 7168) of n bf16 rows:
// y = bf16(g * bf16(x * r)), r = 1 / sqrt(mean(x^2) + eps) in float32.
hipError_t input_rmsnorm(const uint16_t* x, const uint16_t* g, float eps, int n, uint16_t* y, hipStream_t s);

// Fill kernel for small control blocks (used instead of memset so callers may capture graphs).
hipError_t fill_zero_i32(int* p, int64_t n, hipStream_t s);

}  // namespace mla_k
