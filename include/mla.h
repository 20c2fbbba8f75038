/*
 * mla.h -- C ABI of an MI355X (gfx950) Multi-head Latent Attention layer at Kimi-K2 dimensions.
 *
 * What the layer computes (one call = one layer, prefill or KV-cached decode):
 *   - query path: q = q_b(RMSNorm_q(q_a(x))), per head [128 content | 64 rotary]
 *     (modules: "Key-value latent" page, mla-init excerpt; the query forward itself is not
 *     excerpted, this is the reading the module list supports);
 *   - kv path: kv_a_proj_with_mqa(x) split into the 512-feature latent and the 64-feature
 *     shared rotary key; latent RMSNorm in float32; kv_b into 64 heads x (128 key | 128 value)
 *     ("Key-value latent" page, mla-kv and rmsnorm excerpts);
 *   - RoPE (theta from the config) on the 64 rotary features of every query head and of the
 *     shared key; pairs are features (2i, 2i+1), angle = position * theta^(-2i/64);
 *   - causal softmax(q.k * softmax_scale) . v over every cached position so far, with the
 *     scores formed after this call's entries are appended ("Key content up-projection"
 *     page, code excerpt; "KV cache" page, state card);
 *   - heads flattened (index h*128 + d) and o_proj (dense-block attention page, mla-output).
 *
 * Conventions shared by every entry point:
 *   - Weights are [out, in] row-major (the module holds its weight output by input:
 *     "Key content up-projection" page, Parameters). bf16 tensors are IEEE bfloat16 bits.
 *   - "device" pointers are HIP device memory; "host" pointers are ordinary host memory.
 *     The caller owns every buffer; the library never allocates or frees device memory.
 *   - Every call validates all arguments on the host BEFORE it enqueues any work. On a
 *     validation error nothing is enqueued and no buffer (cache, lengths, outputs) is modified
 *     (for a HIP failure after the first enqueue see MLA_E_HIP). Calls do not
 *     throw; they return a status and leave a human-readable detail in mla_last_error()
 *     (thread-local).
 *   - Work is enqueued on the given stream (a hipStream_t, NULL = the default stream) and is
 *     asynchronous; outputs are valid once the stream has reached the call's end.
 *   - Calls on one context are safe from several threads if their caches and workspaces are
 *     distinct. A cache or workspace must not be used by two calls that may overlap.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mla_ctx mla_ctx;
typedef void* mla_stream; /* a hipStream_t; NULL selects the default stream */

typedef enum {
  MLA_OK = 0,
  MLA_E_ARG = 1,         /* null pointer, non-positive count, unknown sequence id, bad flag */
  MLA_E_SHAPE = 2,       /* token ranges inconsistent with the batch (cf. the size checks that
                            raise ValueError in the "Key content up-projection" code excerpt) */
  MLA_E_CAPACITY = 3,    /* len + new > cap of the sequence, or > max_positions. The pages'
                            code does not enforce max_position_embeddings ("KV cache" page);
                            this library does, so a slot is never written out of range. */
  MLA_E_UNSUPPORTED = 4, /* dimensions or a weight format the kernels are not built for, or more
                            than 4096 sequences in one prefill or decode call */
  MLA_E_WORKSPACE = 5,   /* workspace / packed buffer smaller than the call needs */
  MLA_E_HIP = 6,         /* a HIP runtime call failed (detail in mla_last_error). Validation has
                            passed by then, so work enqueued before the failure stays enqueued
                            and the call is partly applied; the host and device lengths stay
                            equal either way: both advance with the launch that appends the
                            entries (decode) or the final commit launch (prefill), and neither
                            advances if the failure comes before it */
  MLA_E_ALIGN = 7        /* a device pointer is not 16-byte aligned */
} mla_status;

/* Weight storage formats. */
enum {
  MLA_WDTYPE_BF16 = 0,          /* all five projections bf16 */
  MLA_WDTYPE_FP8_E4M3_B128 = 1  /* projections as OCP E4M3FN codes with one float32 scale per
                                   128 x 128 block ("Key-value latent" page, linear excerpt:
                                   quantization_config fmt e4m3, weight_block_size [128,128],
                                   activation_scheme dynamic). Activations entering each
                                   projection are quantised per token and per aligned group
                                   of 128 features: s = fl32(amax/448), code = RNE-e4m3 of
                                   fl32(a/s), saturating (s = 1 when amax = 0). */
};

/* Layer hyper-parameters ("KV cache" page, config.json excerpt). The kernels are built for
 * hidden 7168, q_lora 1536, kv_lora 512, 64 heads, qk_nope 128, qk_rope 64, v_head 128; other
 * dimensions give MLA_E_UNSUPPORTED. */
typedef struct {
  int32_t hidden, q_lora, kv_lora, heads, qk_nope, qk_rope, v_head;
  float rms_eps;        /* 1e-6 */
  float rope_theta;     /* 50000 */
  float softmax_scale;  /* 0 selects 1/sqrt(qk_nope + qk_rope); the pages use the scale
                           without defining it */
  int32_t max_positions;/* positions a sequence may hold, 1..131072 (max_position_embeddings) */
  int32_t wdtype;       /* MLA_WDTYPE_* */
  /* YaRN RoPE (rope_scaling in the config excerpt on the "KV cache" page: factor 32, original
   * 4096 positions, beta_fast = beta_slow = 1, mscale = mscale_all_dim = 1). The pages give the
   * parameters only; the rule is the published YaRN method (Peng et al. 2023): pair i of base
   * frequency theta_i makes r_i = rope_orig_max * theta_i / (2 pi) turns over the original
   * context; pairs with r_i >= beta_fast keep theta_i, pairs with r_i < beta_slow use
   * theta_i / rope_factor, pairs in between blend the two linearly in r_i (a step at beta_fast
   * when the two thresholds are equal). With f(m) = 0.1 m ln(rope_factor) + 1, cos/sin carry
   * f(rope_mscale) / f(rope_mscale_all_dim) and a softmax_scale of 0 selects
   * f(rope_mscale_all_dim)^2 / sqrt(qk_nope + qk_rope). rope_factor <= 1 (or 0, as a
   * zero-filled struct has) selects plain RoPE and ignores the other five fields. */
  float rope_factor;
  int32_t rope_orig_max;   /* > 0 when rope_factor > 1 */
  float rope_beta_fast;    /* >= rope_beta_slow > 0 when rope_factor > 1 */
  float rope_beta_slow;
  float rope_mscale;       /* >= 0 */
  float rope_mscale_all_dim;
} mla_config;

/* Device weights, [out, in] row-major. bf16 format: every pointer is bf16, *_s are NULL.
 * FP8 format: projections are uint8 E4M3FN codes, *_s are device float32 scale grids of shape
 * [ceil(out/128), ceil(in/128)] row-major; the two RMSNorm gains stay bf16.
 *   q_a [1536,7168]  q_a_norm [1536]  q_b [64*192,1536] (per head: 128 content, 64 rotary)
 *   kv_a [576,7168] (rows 0..511 latent, 512..575 shared rotary key)  kv_a_norm [512]
 *   kv_b [64*256,512] (per head: rows 0..127 content-key up-projection W_UK, 128..255 value
 *   up-projection W_UV: "Key content up-projection" page, Explanation)  o [7168,64*128]
 * q_b, kv_b, o (and their scales) are referenced, not copied: they must stay valid and
 * unchanged until mla_destroy. q_a, kv_a and the gains are copied into the packed buffer. */
typedef struct {
  const void *q_a, *q_a_norm, *q_b, *kv_a, *kv_a_norm, *kv_b, *o;
  const float *q_a_s, *q_b_s, *kv_a_s, *kv_b_s, *o_s;
} mla_weights;

/* Latent KV cache: one slot per position, mla_cache_entry_bytes() bytes per slot.
 *   bf16 format: 576 bf16 = [c_hat (512, the latent RMSNorm output that kv_b consumes) |
 *                k_pe (64, rotated)]                                   -> 1,152 bytes
 *   FP8 format:  [512 E4M3FN codes of c_hat | 4 float32 group scales | k_pe 64 float32]
 *                (the quantised latent is exactly what kv_b consumes; the rotary key is kept
 *                in float32 because the FP8 output quantiser amplifies any rounding of the
 *                scores)                                               ->   784 bytes
 * The rebuilt per-head keys and values of the pages' cache ("KV cache" page: 20,480 values
 * per position against 576) are derived from these entries inside the kernels; the cache
 * keeps the 576-feature form ("In numbers" on the dense-block attention page: 70,272 vs
 * 2,498,560 bytes per token over 61 layers).
 * Two slot layouts:
 *   contiguous (page_size = 0): sequence s owns slots [offset[s], offset[s] + cap[s]); position p
 *     of s is slot offset[s] + p;
 *   paged (page_size > 0, a power of two >= 64): the slots form pages of page_size consecutive
 *     slots, page k = slots [k * page_size, (k + 1) * page_size); position p of s lives in page
 *     block_table[s * max_pages + p / page_size] at offset p % page_size. The table rows name the
 *     pages of each sequence in position order; pages may be anywhere and in any order (a cache
 *     manager hands them out and takes them back, e.g. with mla_page_pool_*). offset_h/_d are
 *     ignored. A call touching positions 0 .. n-1 of s needs valid page ids (in [0, total_slots /
 *     page_size)) for pages 0 .. (n-1) / page_size of s's row, checked on the host before any
 *     enqueue (MLA_E_ARG); pages must not be shared by sequences that a call writes.
 * len[s] = positions held, cap[s] = positions the sequence may hold. The library advances len_h at
 * enqueue time and len_d on the stream; the caller must keep them equal between calls (initialise
 * both, e.g. to 0), and keep block_table_d equal to block_table_h. */
typedef struct {
  void* data;              /* device, total_slots * entry_bytes, 16-byte aligned */
  const int64_t* offset_h; /* host  [n_seqs] first slot of each sequence (contiguous layout) */
  const int64_t* offset_d; /* device[n_seqs] same values */
  int32_t* len_h;          /* host  [n_seqs] positions held */
  int32_t* len_d;          /* device[n_seqs] same values */
  const int32_t* cap_h;    /* host  [n_seqs] positions reserved per sequence */
  int32_t n_seqs;
  int64_t total_slots;
  /* paged layout (all zero / NULL: contiguous) */
  const int32_t* block_table_h; /* host  [n_seqs][max_pages] page ids */
  const int32_t* block_table_d; /* device, same values */
  int32_t page_size;            /* slots per page: 0, or a power of two >= 64 */
  int32_t max_pages;            /* row length of the block table (>= ceil(cap / page_size)) */
} mla_cache;

/* Bytes of the packed-weight buffer mla_init_weights fills (fused q_a|kv_a weight, transposed
 * per-head W_UK, scale grids, RoPE cos/sin table of max_positions x 32 float32).
 * Returns 0 for an invalid config. */
size_t mla_packed_weight_bytes(const mla_config* cfg);

/* Bytes per cache slot for cfg's weight format (1152 or 784); 0 for an invalid config. */
size_t mla_cache_entry_bytes(const mla_config* cfg);

/* Workspace bytes sufficient for any prefill call with at most max_tokens new tokens in total,
 * at most max_batch sequences, and at most max_keys positions summed over the call's sequences
 * after the call (sum of cached + new). Returns 0 on invalid arguments. */
size_t mla_prefill_workspace_bytes(const mla_ctx* ctx, int32_t max_tokens, int32_t max_batch, int64_t max_keys);

/* Workspace bytes sufficient for any decode call with at most max_batch sequences holding at
 * most max_keys positions in total after the step (sum over b of len_b + 1). */
size_t mla_decode_workspace_bytes(const mla_ctx* ctx, int32_t max_batch, int64_t max_keys);

/* Validate cfg and weights, build the packed buffer (device, packed_bytes >=
 * mla_packed_weight_bytes(cfg)) on `stream`, and return a host context in *out.
 * The RoPE table is computed on the host in double precision and stored as float32.
 * The stream is synchronised before returning (the host staging copy is freed). */
mla_status mla_init_weights(const mla_config* cfg, const mla_weights* w, void* packed, size_t packed_bytes,
                            mla_stream stream, mla_ctx** out);

/* Prefill: B sequences, sequence b's T_b = q_start[b+1] - q_start[b] new tokens are rows
 * q_start[b] .. q_start[b+1]-1 of x. Token t of sequence seq_ids[b] gets position
 * len[seq] + t (the cached prefix may be non-empty: chunked prefill). All new entries are
 * appended, then every new token attends causally to positions 0 .. its own.
 *   seq_ids_h/_d  host/device [B], distinct ids in [0, n_seqs)
 *   q_start_h/_d  host/device [B+1], q_start[0] = 0, non-decreasing, T_b >= 1
 *   x             device [q_start[B], 7168] bf16, y device [q_start[B], 7168] bf16
 *   ws            device workspace of ws_bytes >= mla_prefill_workspace_bytes(ctx, q_start[B], B,
 *                 sum over b of len + T_b). The workspace holds only scratch values of the call: it needs
 *                 no initialisation and its contents between calls do not matter. */
mla_status mla_prefill(mla_ctx* ctx, mla_cache* cache, const int32_t* seq_ids_h, const int32_t* seq_ids_d,
                       const int32_t* q_start_h, const int32_t* q_start_d, int32_t B, const void* x, void* y,
                       void* ws, size_t ws_bytes, mla_stream stream);

/* Decode: one new token for each of B sequences (x row b belongs to seq_ids[b]) at position
 * len[seq]; its entry is appended, then it attends to positions 0 .. len[seq] (so the scores
 * cover len + 1 positions, 1,001 at p = 1000 as on the "KV cache" page).
 * Attention runs in the latent space: q_nope is absorbed into the 512-feature latent through
 * W_UK, scores use [q_lat | q_pe] . [c_hat | k_pe], the value mix stays latent and W_UV is
 * applied after the softmax merge (algebraically the pages' scores and mix).
 *   x, y device [B, 7168] bf16; ws of ws_bytes >= mla_decode_workspace_bytes(ctx, B,
 *   sum over b of len + 1) (scratch only, as for prefill). */
mla_status mla_decode(mla_ctx* ctx, mla_cache* cache, const int32_t* seq_ids_h, const int32_t* seq_ids_d,
                      int32_t B, const void* x, void* y, void* ws, size_t ws_bytes, mla_stream stream);

/* ---- Decode without any allocation, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Same arguments,
 * semantics, validation and errors as mla_decode, minus the workspace: the call uses a
 * workspace inside the library, a static device array of MLA_STATIC_SCRATCH_BYTES (128 MiB) that
 * every GPU the library runs on holds once, from the first call on that device (or
 * mla_init_weights there) until the process ends. It calls no hipMalloc/hipFree and no
 * allocating routine.
 * Limit: the step's own workspace, from its B and the lengths its sequences reach (at most what
 * mla_decode_workspace_bytes reports, which bounds every split plan), must fit
 * MLA_STATIC_SCRATCH_BYTES, else the call returns MLA_E_WORKSPACE before anything is enqueued.
 * Measured needs: FP8, 128 sequences of 16384 positions: 124.7 MiB (fits); bf16, 64 sequences of
 * 1024..8192: 116.8 MiB (fits); bf16, 1000 sequences of one position: more (rejected).
 * All calls on one GPU share that GPU's array and it keeps the last call's values: two calls that
 * may overlap on one GPU (different streams or threads without ordering) race and must not be
 * issued; calls in stream order are safe. Nothing in the array needs clearing between calls. */
#define MLA_STATIC_SCRATCH_BYTES ((size_t)128 << 20)
mla_status mla_decode_static(mla_ctx* ctx, mla_cache* cache, const int32_t* seq_ids_h, const int32_t* seq_ids_d,
                             int32_t B, const void* x, void* y, mla_stream stream);

/* ---- Attention half of a decoder block ("Attention input" page, block excerpt): the block
 * keeps its input as the residual, feeds the attention its input RMSNorm and adds the attention
 * output back:  h = x + MLA(xn),  xn = RMSNorm(x) over the 7168 hidden features with gain
 * norm_weight and eps = cfg.rms_eps. xn follows the rmsnorm excerpt's dtypes: the normalised
 * value (float32) is rounded to bf16 before the gain and the product with the bf16 gain is
 * bf16, xn = bf16(g * bf16(x / sqrt(mean(x^2) + eps))). The residual is added to o_proj's
 * float32 sum before its single bf16 rounding.
 *   norm_weight  device [7168] bf16 (the block's input_layernorm weight), 16-byte aligned
 *   x, h         device [rows, 7168] bf16; h may be x itself (in place) or a buffer that does
 *                not overlap it (a partial overlap gives MLA_E_ARG)
 *   ws           workspace of ws_bytes >= mla_block_prefill_workspace_bytes(...) (or
 *                _decode_); its first
 *                rows * 7168 * 2 bytes (rounded up to 256) hold xn, the rest is the layer's.
 * Everything else (cache, positions, validation before any enqueue, errors) is exactly as for
 * mla_prefill / mla_decode. */
size_t mla_block_prefill_workspace_bytes(const mla_ctx* ctx, int32_t max_tokens, int32_t max_batch, int64_t max_keys);
size_t mla_block_decode_workspace_bytes(const mla_ctx* ctx, int32_t max_batch, int64_t max_keys);
mla_status mla_block_prefill(mla_ctx* ctx, mla_cache* cache, const int32_t* seq_ids_h, const int32_t* seq_ids_d,
                             const int32_t* q_start_h, const int32_t* q_start_d, int32_t B, const void* norm_weight,
                             const void* x, void* h, void* ws, size_t ws_bytes, mla_stream stream);
mla_status mla_block_decode(mla_ctx* ctx, mla_cache* cache, const int32_t* seq_ids_h, const int32_t* seq_ids_d,
                            int32_t B, const void* norm_weight, const void* x, void* h, void* ws, size_t ws_bytes,
                            mla_stream stream);

/* ---- One cache buffer for a stack of layers. The dense-block attention page ("In numbers") prices
 * the model's cache per position over its 61 layers: 2,498,560 B for rebuilt keys and values
 * against 70,272 B (61 x 1,152) for the latent form used here. A pool is one caller-owned device
 * buffer holding n_layers layer caches with one shared slot layout: sequence s owns slots
 * offset[s] .. offset[s] + cap[s] - 1 in every layer (each sequence's run rounded up to `align`
 * slots), and layer l's slots start at byte l * layer_bytes of the pool, so a position costs
 * n_layers * mla_cache_entry_bytes(cfg) bytes.
 *
 * mla_cache_pool_plan: host-only. cap_h [n_seqs] positions per sequence (0 .. max_positions),
 * align 1 .. 4096; writes offset_h [n_seqs] (caller-allocated), *total_slots (slots per layer),
 * *layer_bytes (= total_slots * entry bytes, a multiple of 16) and *pool_bytes
 * (= n_layers * layer_bytes). Errors: MLA_E_ARG (NULL, sizes), MLA_E_CAPACITY (a cap above
 * max_positions), the config's own status. */
mla_status mla_cache_pool_plan(const mla_config* cfg, int32_t n_layers, int32_t n_seqs, const int32_t* cap_h,
                               int32_t align, int64_t* offset_h, int64_t* total_slots, size_t* layer_bytes,
                               size_t* pool_bytes);

/* Point cache->data at layer `layer` of a pool of pool_bytes planned with layer_bytes per layer
 * (pool + layer * layer_bytes), after checking that the layer lies inside the pool and is 16-byte
 * aligned. The caller fills the rest of the descriptor: offsets, capacities, n_seqs and
 * total_slots from the plan (shared by all layers) and the layer's own len_h / len_d. Host-only;
 * on an error *cache is unchanged. */
mla_status mla_cache_pool_layer(void* pool, size_t pool_bytes, size_t layer_bytes, int32_t layer, mla_cache* cache);

/* ---- Page allocator for paged caches (host only; the cache manager of a serving loop): a pool
 * of n_pages page ids 0 .. n_pages-1. alloc hands out n free ids in ascending order of release
 * (freed pages are reused first-in, first-out) or fails with MLA_E_CAPACITY, leaving the pool
 * unchanged, when fewer are free; free takes ids back (MLA_E_ARG for an id out of range or not
 * allocated, nothing freed then). A pool is not thread-safe: one thread at a time. With
 * mla_cache_pool_plan-style stacks of layers, one page id addresses the same pages in every
 * layer's region, so one pool and one block table serve the whole stack. */
typedef struct mla_page_pool mla_page_pool;
mla_status mla_page_pool_create(int32_t n_pages, mla_page_pool** out);
mla_status mla_page_pool_alloc(mla_page_pool* pool, int32_t n, int32_t* ids);
mla_status mla_page_pool_free(mla_page_pool* pool, const int32_t* ids, int32_t n);
int32_t mla_page_pool_available(const mla_page_pool* pool); /* free pages; -1 for NULL */
void mla_page_pool_destroy(mla_page_pool* pool);

/* Append n ready-made entries (device, n * mla_cache_entry_bytes bytes, the slot format above)
 * to sequence seq_id at positions len .. len+n-1: a byte copy into the slots, then len += n.
 * Used to load a cache produced elsewhere (for example from a saved state). */
mla_status mla_cache_append(mla_ctx* ctx, mla_cache* cache, int32_t seq_id, const void* entries, int32_t n,
                            mla_stream stream);

/* Release the host context (device buffers stay owned by the caller). NULL is ignored. */
void mla_destroy(mla_ctx* ctx);

/* Static description of a status code. */
const char* mla_status_str(mla_status s);

/* Detail of the last error on this thread ("" if none). */
const char* mla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
