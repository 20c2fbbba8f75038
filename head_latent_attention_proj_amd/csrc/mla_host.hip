// Host side of the C ABI in include/mla.h: validation, weight packing, workspace planning and the
// launch sequences of prefill and decode. Nothing here allocates device memory; every device
// buffer is the caller's. All validation happens before the first enqueue of a call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/mla.h"
#include "../../include/mla_test.h"
#include "common.h"
#include "kernels.h"

using namespace mla_dims;

// ---- the allocation-free decode (mla_decode_static): its workspace is this file-scope device
// array, one copy per GPU the library runs on, held until the process ends. In host code the
// name `scratch` is only a host-side stand-in; kernels receive the device address obtained from
// hipGetSymbolAddress for the current device.
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)128 << 20;
static_assert(STATIC_SCRATCH_BYTES == MLA_STATIC_SCRATCH_BYTES, "header and library agree on the size");
static __device__ __align__(256) uint8_t scratch[STATIC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

mla_status fail(mla_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

#define HIP_TRY(expr)                                                                      \
  do {                                                                                     \
    hipError_t e_ = (expr);                                                                \
    if (e_ != hipSuccess) return fail(MLA_E_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---- stage probe (mla_test_probe_stage): one-shot, per thread. The next call on this thread
// that launches the armed stage records ev0 on its stream right before that stage's launches
// and ev1 right after them, then disarms.
thread_local int g_probe_stage = 0;
thread_local hipEvent_t g_probe_ev0 = nullptr, g_probe_ev1 = nullptr;

#define PROBED(stage, expr)                                     \
  do {                                                          \
    const bool on_ = g_probe_stage == (stage);                  \
    if (on_) HIP_TRY(hipEventRecord(g_probe_ev0, s));           \
    HIP_TRY(expr);                                              \
    if (on_) {                                                  \
      HIP_TRY(hipEventRecord(g_probe_ev1, s));                  \
      g_probe_stage = 0;                                        \
    }                                                           \
  } while (0)

int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// ---- per-head W_UK^T: ukT[h][c][d] = W_UK,h[d][c] = kv_b[h*256 + d][c]  (d < 128, c < 512), as bf16.
// bf16 weights are copied; FP8 codes are widened to their exact bf16 value (the block scale of
// (h, c/128) is applied to the product's output).
template <bool FP8>
__global__ void transpose_uk_kernel(const void* kvb, uint16_t* ukT) {
  const int h = blockIdx.y;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;  // over 512*128
  if (idx >= KV_LORA * NOPE) return;
  const int c = idx / NOPE, d = idx % NOPE;
  const int64_t src = ((int64_t)h * 256 + d) * KV_LORA + c;
  uint16_t v;
  if constexpr (FP8) {
    v = f2bf(__builtin_amdgcn_cvt_f32_fp8((int)((const uint8_t*)kvb)[src], 0));
  } else {
    v = ((const uint16_t*)kvb)[src];
  }
  ukT[((int64_t)h * KV_LORA + c) * NOPE + d] = v;
}

// FP8: W_UV,h codes widened to their exact bf16 values, uvw[h][d][c] = code(kv_b[h*256+128+d][c])
// (the block scales are applied to the other operand).
__global__ void widen_uv_kernel(const uint8_t* kvb, uint16_t* uvw) {
  const int h = blockIdx.y;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;  // over 128*512
  if (idx >= VD * KV_LORA) return;
  const int d = idx / KV_LORA, c = idx % KV_LORA;
  uvw[(int64_t)h * VD * KV_LORA + idx] =
      f2bf(__builtin_amdgcn_cvt_f32_fp8((int)kvb[((int64_t)h * 256 + 128 + d) * KV_LORA + c], 0));
}

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// Device address of this GPU's scratch array, resolved once per device with that device current.
mla_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MLA_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES) return fail(MLA_E_UNSUPPORTED, "device %d beyond the %d the library tracks", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(MLA_E_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

}  // namespace

struct mla_ctx {
  mla_config cfg;
  bool fp8;
  float scale;
  const uint16_t* g_q;
  const uint16_t* g_kv;
  const void* w_qkva;  // packed [2112, 7168]
  const float* s_qkva; // FP8: packed [17, 56]
  const void* w_qb;
  const float* s_qb;   // [96, 12]
  const void* w_kvb;
  const float* s_kvb;  // [128, 4]
  const uint16_t* w_ukT;  // packed [64][512][128] bf16
  const uint16_t* w_uv;   // W_UV,h rows as bf16: kv_b itself (row stride 512, head stride 256 rows)
  int64_t uv_head_stride; //   or, FP8, the packed widened codes [64][128][512]
  const void* w_o;
  const float* s_o;    // [56, 64]
  const float* rope_cs;
};

namespace {

mla_status check_config(const mla_config* c) {
  if (!c) return fail(MLA_E_ARG, "config is NULL");
  if (c->hidden != HIDDEN || c->q_lora != Q_LORA || c->kv_lora != KV_LORA || c->heads != HEADS ||
      c->qk_nope != NOPE || c->qk_rope != ROPE || c->v_head != VD)
    return fail(MLA_E_UNSUPPORTED,
                "kernels are built for hidden 7168, q_lora 1536, kv_lora 512, 64 heads, 128/64/128 head widths");
  if (!(c->rms_eps > 0.f) || !(c->rope_theta > 1.f) || c->softmax_scale < 0.f || !std::isfinite(c->softmax_scale))
    return fail(MLA_E_ARG, "rms_eps, rope_theta or softmax_scale out of range");
  if (c->max_positions < 1 || c->max_positions > 131072)
    return fail(MLA_E_ARG, "max_positions must be in [1, 131072]");
  if (!std::isfinite(c->rope_factor))
    return fail(MLA_E_ARG, "rope_factor must be finite");
  if (c->rope_factor > 1.f &&
      (c->rope_orig_max < 1 || !(c->rope_beta_slow > 0.f) || !(c->rope_beta_fast >= c->rope_beta_slow) ||
       !std::isfinite(c->rope_beta_fast) || !(c->rope_mscale >= 0.f) || !(c->rope_mscale_all_dim >= 0.f) ||
       !std::isfinite(c->rope_mscale) || !std::isfinite(c->rope_mscale_all_dim)))
    return fail(MLA_E_ARG, "YaRN RoPE: need rope_orig_max > 0, rope_beta_fast >= rope_beta_slow > 0, mscales >= 0");
  if (c->wdtype != MLA_WDTYPE_BF16 && c->wdtype != MLA_WDTYPE_FP8_E4M3_B128)
    return fail(MLA_E_ARG, "unknown weight format %d", c->wdtype);
  return MLA_OK;
}

struct PackedLayout {
  size_t qkva, s_qkva, ukT, uvw, g_q, g_kv, rope, total;
};

PackedLayout packed_layout(const mla_config* c) {
  PackedLayout L{};
  const bool fp8 = c->wdtype == MLA_WDTYPE_FP8_E4M3_B128;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = round_up(off + bytes, 256);
    return o;
  };
  L.qkva = take((size_t)QKVA_N * HIDDEN * (fp8 ? 1 : 2));
  L.s_qkva = take(fp8 ? (size_t)17 * 56 * sizeof(float) : 0);
  L.ukT = take((size_t)HEADS * KV_LORA * NOPE * 2);
  L.uvw = take(fp8 ? (size_t)HEADS * VD * KV_LORA * 2 : 0);
  L.g_q = take(Q_LORA * 2);
  L.g_kv = take(KV_LORA * 2);
  L.rope = take((size_t)c->max_positions * 32 * 2 * sizeof(float));
  L.total = off;
  return L;
}

// ---- workspace planning ----------------------------------------------------------------------
// K-split parts of the fused q_a|kv_a projection that the norm kernel adds: up to 4 at decode sizes;
// with FP8 weights up to 128 rows, 8 (the precise FP8 tile kernel splits K 7 ways at 65 .. 128 rows
// and then needs no reduction launch); none above (no projection kernel splits K there), so a
// prefill's workspace holds one copy of the sums
int qkva_parts_max(int ntok, bool fp8) { return ntok <= 64 ? 4 : (fp8 && ntok <= 128 ? 8 : 1); }
constexpr int DECODE_MAX_WG = 2048;
constexpr int MAX_BATCH = 4096;  // sequences per prefill or decode call (MLA_E_UNSUPPORTED above)

struct DecodePlan {
  int chunk = 32, max_splits = 1;
};

// Split size for decode attention: about total / D positions (at least 64), D = 384 for the bf16
// kernel and 256 for the FP8 kernel. Chosen by measurement on MI355X: bf16, 64 sequences of
// 1024..8192 positions: D = 256 took 194 us, 384 took 137 us, 512 took 160 us, a cost-model
// choice (640) 150 us; FP8, 128 sequences of about 16400 positions: D = 256 (two splits per
// sequence, one workgroup per CU) took 629 us, 512 (four) 644 us, 384 (three: one and a half
// workgroups per CU) 824 us; one sequence of 1000 positions: 64-position splits beat 32 (fewer
// float32 partials) and 128 or more (longer serial chains per workgroup).
DecodePlan plan_decode(int B, const int* lens_after, int n, bool fp8) {
  int64_t total = 0;
  int max_len = 1;
  for (int i = 0; i < n; ++i) {
    total += lens_after[i];
    max_len = std::max(max_len, lens_after[i]);
  }
  const int64_t D = fp8 ? 256 : 384;
  DecodePlan p;
  p.chunk = (int)std::max<int64_t>(64, round_up((total + D - 1) / D, 32));
  p.max_splits = (max_len + p.chunk - 1) / p.chunk;
  while ((int64_t)B * p.max_splits > DECODE_MAX_WG && p.max_splits > 1) {
    p.chunk *= 2;
    p.max_splits = (max_len + p.chunk - 1) / p.chunk;
  }
  return p;
}

struct WsLayout {
  size_t cqkv, q_hat, q, o, meta, knope, vt, q_lat, part_o, part_ml, gpart;
  size_t vt_lo, qs;  // FP8 only: fp16 residual plane of the values, split q_nope
  size_t o_lat;                // decode: merged latent attention output (bf16; FP8: 2 planes)
  size_t x8, x8s, qh8s, o32, o8, o8s, gath, total;
  int64_t gpart_floats;
  int64_t vt_ld;
};

// Largest split-K scratch any projection of a call may need (floats).
int64_t max_gemm_part(int ntok, int nkeys_seq, bool decode, bool fp8) {
  int64_t mx = 0;
  auto upd = [&](int M, int N, int K, int batch) {
    if (M > 0)
      mx = std::max(mx, fp8 ? mla_k::gemm_fp8_part_floats(M, N, K, batch) : mla_k::gemm_part_floats(M, N, K, batch));
  };
  upd(ntok, QKVA_N, HIDDEN, 1);
  upd(ntok, QB_N, Q_LORA, 1);
  upd(ntok, HIDDEN, O_IN, 1);
  if (decode) {  // absorb and W_UV (FP8: high and residual parts stacked as 2 * ntok rows)
    if (ntok > 0) {
      mx = std::max(mx, mla_k::gemm_part_floats(fp8 ? 2 * ntok : ntok, KV_LORA, NOPE, HEADS));
      mx = std::max(mx, mla_k::gemm_part_floats(fp8 ? 2 * ntok : ntok, VD, KV_LORA, HEADS));
    }
  } else {
    upd(nkeys_seq, KVB_N, KV_LORA, 1);
  }
  return mx;
}

WsLayout ws_layout(int ntok, int nbatch, int64_t nkeys, int decode_splits, int64_t gpart_floats, bool fp8) {
  WsLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = round_up(off + bytes, 256);
    return o;
  };
  L.cqkv = take((size_t)ntok * QKVA_N * 4 * qkva_parts_max(ntok, fp8));
  L.q_hat = take((size_t)ntok * Q_LORA * 2);  // bf16, or FP8 codes
  L.q = take((size_t)ntok * QB_N * (fp8 && decode_splits > 0 ? 4 : 2));  // FP8 decode: float32 q; prefill fp16
  L.o = take((size_t)ntok * O_IN * 2);
  L.meta = take((size_t)nbatch * sizeof(mla_k::SeqMeta));
  L.vt_ld = round_up(nkeys, 64);
  L.knope = take((size_t)L.vt_ld * HEADS * NOPE * 2);
  L.vt = take((size_t)L.vt_ld * HEADS * VD * 2);
  L.vt_lo = take(fp8 ? (size_t)L.vt_ld * HEADS * VD * 2 : 0);
  // q_lat: bf16 [B][64][512], or FP8: two float32 products (high and residual part of q_nope)
  L.q_lat = take(decode_splits > 0 ? (size_t)nbatch * HEADS * KV_LORA * (fp8 ? 8 : 2) : 0);
  L.qs = take(fp8 && decode_splits > 0 ? (size_t)2 * nbatch * HEADS * NOPE * 2 : 0);
  L.part_o = take((size_t)decode_splits * HEADS * KV_LORA * 4);
  L.part_ml = take((size_t)decode_splits * HEADS * 2 * 4);
  L.x8 = take(fp8 ? (size_t)ntok * HIDDEN : 0);
  L.x8s = take(fp8 ? (size_t)ntok * (HIDDEN / 128) * 4 : 0);
  L.qh8s = take(fp8 ? (size_t)ntok * (Q_LORA / 128) * 4 : 0);
  L.o32 = take(fp8 && decode_splits > 0 ? (size_t)ntok * O_IN * 4 * 2 : 0);  // decode: W_UV's two planes
  L.o_lat = take(decode_splits > 0 ? (size_t)nbatch * HEADS * KV_LORA * 2 * (fp8 ? 2 : 1) : 0);
  L.o8 = take(fp8 ? (size_t)ntok * O_IN : 0);
  L.o8s = take(fp8 ? (size_t)ntok * (O_IN / 128) * 4 : 0);
  L.gpart_floats = gpart_floats;
  L.gpart = take((size_t)gpart_floats * 4);
  // paged prefill: each sequence's entries gathered into rows kbase .. (same padding as the keys)
  L.gath = take(decode_splits > 0 ? 0 : (size_t)L.vt_ld * (fp8 ? FP8_ENTRY_BYTES : BF16_ENTRY_BYTES));
  L.total = off;
  return L;
}

mla_k::GemmArgs gemm_common(uint8_t* ws, const WsLayout& L) {
  mla_k::GemmArgs g;
  g.part = (float*)(ws + L.gpart);
  g.part_cap = L.gpart_floats;
  return g;
}

hipError_t run_proj(const mla_ctx* ctx, mla_k::GemmArgs& g, hipStream_t s) {
  return ctx->fp8 ? mla_k::gemm_fp8(g, s) : mla_k::gemm_bf16(g, s);
}

int proj_ysplit(const mla_ctx* ctx, const mla_k::GemmArgs& g) {
  return ctx->fp8 ? mla_k::gemm_fp8_ysplit(g) : mla_k::gemm_ysplit(g);
}

bool paged(const mla_cache* c) { return c->page_size != 0; }

int page_shift(int32_t page_size) {
  int sh = 0;
  while ((1 << sh) < page_size) ++sh;
  return sh;
}

mla_status check_cache(const mla_ctx* ctx, const mla_cache* c) {
  if (!c) return fail(MLA_E_ARG, "cache is NULL");
  if (!c->data || !c->len_h || !c->len_d || !c->cap_h) return fail(MLA_E_ARG, "cache has a NULL pointer");
  if (c->n_seqs <= 0 || c->total_slots <= 0) return fail(MLA_E_ARG, "cache has no sequences or slots");
  if (!aligned16(c->data)) return fail(MLA_E_ALIGN, "cache data is not 16-byte aligned");
  if (paged(c)) {
    if (c->page_size < 64 || (c->page_size & (c->page_size - 1)) || c->total_slots % c->page_size)
      return fail(MLA_E_ARG, "page_size %d must be a power of two >= 64 dividing total_slots", c->page_size);
    if (!c->block_table_h || !c->block_table_d || c->max_pages <= 0)
      return fail(MLA_E_ARG, "a paged cache needs both block tables and max_pages > 0");
  } else if (!c->offset_h || !c->offset_d) {
    return fail(MLA_E_ARG, "cache has a NULL offset array");
  }
  (void)ctx;
  return MLA_OK;
}

SlotMap slot_map(const mla_cache* c) {
  SlotMap m;
  if (paged(c)) {
    m.table = c->block_table_d;
    m.page_shift = page_shift(c->page_size);
    m.max_pages = c->max_pages;
  } else {
    m.offset = c->offset_d;
  }
  return m;
}

mla_status check_seq(const mla_ctx* ctx, const mla_cache* c, int s, int64_t add) {
  if (s < 0 || s >= c->n_seqs) return fail(MLA_E_ARG, "sequence id %d outside [0, %d)", s, c->n_seqs);
  const int64_t len = c->len_h[s];
  if (len < 0 || c->cap_h[s] < 0)
    return fail(MLA_E_ARG, "sequence %d has an inconsistent cap/len", s);
  if (paged(c)) {
    if ((int64_t)c->cap_h[s] > (int64_t)c->max_pages * c->page_size)
      return fail(MLA_E_ARG, "sequence %d: capacity %d exceeds its %d table pages", s, c->cap_h[s], c->max_pages);
  } else if (c->offset_h[s] < 0 || c->offset_h[s] + c->cap_h[s] > c->total_slots) {
    return fail(MLA_E_ARG, "sequence %d has an inconsistent offset/cap/len", s);
  }
  if (len + add > c->cap_h[s])
    return fail(MLA_E_CAPACITY, "sequence %d: %lld positions + %lld new exceed its %d slots", s, (long long)len,
                (long long)add, c->cap_h[s]);
  if (len + add > ctx->cfg.max_positions)
    return fail(MLA_E_CAPACITY, "sequence %d: %lld positions exceed max_positions %d", s, (long long)(len + add),
                ctx->cfg.max_positions);
  if (paged(c) && len + add > 0) {  // every page the call reads or writes names a page of the cache
    const int64_t n_pages = c->total_slots / c->page_size;
    const int32_t* row = c->block_table_h + (int64_t)s * c->max_pages;
    for (int64_t pg = 0; pg <= (len + add - 1) / c->page_size; ++pg)
      if (row[pg] < 0 || row[pg] >= n_pages)
        return fail(MLA_E_ARG, "sequence %d: page %lld of its table is %d, outside [0, %lld)", s, (long long)pg,
                    row[pg], (long long)n_pages);
  }
  return MLA_OK;
}

// Projection input of the o_proj / q_a|kv_a products: bf16 directly, or FP8 codes + scales.
void set_a(const mla_ctx* ctx, mla_k::GemmArgs& g, const void* bf16, int64_t ld_bf16, const uint8_t* codes,
           const float* scales, int64_t groups) {
  if (ctx->fp8) {
    g.A = codes;
    g.lda = ld_bf16;
    g.a_scale = scales;
    g.as_ld = groups;
  } else {
    g.A = bf16;
    g.lda = ld_bf16;
  }
}

}  // namespace

extern "C" {

const char* mla_status_str(mla_status s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_E_ARG: return "invalid argument";
    case MLA_E_SHAPE: return "inconsistent shapes";
    case MLA_E_CAPACITY: return "cache capacity exceeded";
    case MLA_E_UNSUPPORTED: return "unsupported configuration";
    case MLA_E_WORKSPACE: return "workspace too small";
    case MLA_E_HIP: return "HIP runtime error";
    case MLA_E_ALIGN: return "misaligned device pointer";
  }
  return "unknown status";
}

const char* mla_last_error(void) { return g_last_error.c_str(); }

size_t mla_packed_weight_bytes(const mla_config* cfg) {
  if (check_config(cfg) != MLA_OK) return 0;
  return packed_layout(cfg).total;
}

size_t mla_cache_entry_bytes(const mla_config* cfg) {
  if (check_config(cfg) != MLA_OK) return 0;
  return cfg->wdtype == MLA_WDTYPE_BF16 ? BF16_ENTRY_BYTES : FP8_ENTRY_BYTES;
}

size_t mla_prefill_workspace_bytes(const mla_ctx* ctx, int32_t max_tokens, int32_t max_batch, int64_t max_keys) {
  if (!ctx || max_tokens <= 0 || max_batch <= 0 || max_keys < max_tokens) return 0;
  // rebuilt keys: each sequence's rows are padded to a multiple of 64
  const int64_t keys = max_keys + 63LL * max_batch;
  int64_t gp = 0;
  for (int m = 1; m <= std::min(max_tokens, 4096); ++m) gp = std::max(gp, max_gemm_part(m, 0, false, ctx->fp8));
  const int64_t kmax = std::min<int64_t>(max_keys, 4096);
  for (int64_t k = 1; k <= kmax; ++k) gp = std::max(gp, max_gemm_part(0, (int)k, false, ctx->fp8));
  return ws_layout(max_tokens, max_batch, keys, 0, gp, ctx->fp8).total;
}

size_t mla_decode_workspace_bytes(const mla_ctx* ctx, int32_t max_batch, int64_t max_keys) {
  if (!ctx || max_batch <= 0 || max_keys < max_batch) return 0;
  int64_t gp = 0;
  for (int m = 1; m <= max_batch; ++m) gp = std::max(gp, max_gemm_part(m, 0, true, ctx->fp8));
  const int64_t splits = std::min<int64_t>((int64_t)max_batch * ((max_keys + 31) / 32), DECODE_MAX_WG);
  return ws_layout(max_batch, max_batch, 0, (int)std::max<int64_t>(splits, max_batch), gp, ctx->fp8).total;
}

mla_status mla_init_weights(const mla_config* cfg, const mla_weights* w, void* packed, size_t packed_bytes,
                            mla_stream stream, mla_ctx** out) {
  if (!out) return fail(MLA_E_ARG, "out is NULL");
  *out = nullptr;
  mla_status st = check_config(cfg);
  if (st != MLA_OK) return st;
  if (!w || !packed) return fail(MLA_E_ARG, "weights or packed buffer is NULL");
  const bool fp8 = cfg->wdtype == MLA_WDTYPE_FP8_E4M3_B128;
  const void* ptrs[] = {w->q_a, w->q_a_norm, w->q_b, w->kv_a, w->kv_a_norm, w->kv_b, w->o};
  for (const void* p : ptrs) {
    if (!p) return fail(MLA_E_ARG, "a weight pointer is NULL");
    if (!aligned16(p)) return fail(MLA_E_ALIGN, "a weight pointer is not 16-byte aligned");
  }
  if (fp8) {
    const float* sp[] = {w->q_a_s, w->q_b_s, w->kv_a_s, w->kv_b_s, w->o_s};
    for (const float* p : sp)
      if (!p) return fail(MLA_E_ARG, "FP8 weights need all five scale grids");
  }
  const PackedLayout L = packed_layout(cfg);
  if (packed_bytes < L.total) return fail(MLA_E_WORKSPACE, "packed buffer has %zu bytes, needs %zu", packed_bytes, L.total);
  if (!aligned16(packed)) return fail(MLA_E_ALIGN, "packed buffer is not 16-byte aligned");

  hipStream_t s = (hipStream_t)stream;
  uint8_t* pk = (uint8_t*)packed;
  const size_t eb = fp8 ? 1 : 2;
  HIP_TRY(hipMemcpyAsync(pk + L.qkva, w->q_a, (size_t)Q_LORA * HIDDEN * eb, hipMemcpyDeviceToDevice, s));
  HIP_TRY(hipMemcpyAsync(pk + L.qkva + (size_t)Q_LORA * HIDDEN * eb, w->kv_a, (size_t)ENTRY * HIDDEN * eb,
                         hipMemcpyDeviceToDevice, s));
  if (fp8) {  // scale grids of q_a [12, 56] and kv_a [5, 56] stacked: block rows of the fused weight
    HIP_TRY(hipMemcpyAsync(pk + L.s_qkva, w->q_a_s, 12 * 56 * sizeof(float), hipMemcpyDeviceToDevice, s));
    HIP_TRY(hipMemcpyAsync(pk + L.s_qkva + 12 * 56 * sizeof(float), w->kv_a_s, 5 * 56 * sizeof(float),
                           hipMemcpyDeviceToDevice, s));
  }
  HIP_TRY(hipMemcpyAsync(pk + L.g_q, w->q_a_norm, Q_LORA * 2, hipMemcpyDeviceToDevice, s));
  HIP_TRY(hipMemcpyAsync(pk + L.g_kv, w->kv_a_norm, KV_LORA * 2, hipMemcpyDeviceToDevice, s));
  if (fp8)
    hipLaunchKernelGGL(transpose_uk_kernel<true>, dim3(KV_LORA * NOPE / 256, HEADS), dim3(256), 0, s, w->kv_b,
                       (uint16_t*)(pk + L.ukT));
  else
    hipLaunchKernelGGL(transpose_uk_kernel<false>, dim3(KV_LORA * NOPE / 256, HEADS), dim3(256), 0, s, w->kv_b,
                       (uint16_t*)(pk + L.ukT));
  HIP_TRY(hipGetLastError());
  if (fp8) {
    hipLaunchKernelGGL(widen_uv_kernel, dim3(VD * KV_LORA / 256, HEADS), dim3(256), 0, s, (const uint8_t*)w->kv_b,
                       (uint16_t*)(pk + L.uvw));
    HIP_TRY(hipGetLastError());
  }
  // RoPE table: angle = position * frequency of pair i, computed in double, stored float32.
  // Plain RoPE: frequency theta^(-2i/64). YaRN (rope_factor > 1; the rule of the YaRN paper,
  // Peng et al. 2023, with the config's rope_scaling values): a pair making r turns over the
  // original context keeps its frequency when r >= beta_fast, is slowed by the factor when
  // r < beta_slow, and in between blends the two linearly in r; cos/sin carry the ratio of the
  // attention factors f(mscale) / f(mscale_all_dim), f(m) = 0.1 m ln(factor) + 1.
  const bool yarn = cfg->rope_factor > 1.f;
  const double yf = cfg->rope_factor;
  auto attn_factor = [&](double m) { return 0.1 * m * std::log(yf) + 1.0; };
  const double gain = yarn ? attn_factor(cfg->rope_mscale) / attn_factor(cfg->rope_mscale_all_dim) : 1.0;
  const int P = cfg->max_positions;
  std::vector<float> cs((size_t)P * 64);
  for (int i = 0; i < 32; ++i) {
    double freq = std::pow((double)cfg->rope_theta, -2.0 * i / 64.0);
    if (yarn) {
      const double turns = (double)cfg->rope_orig_max * freq / (2.0 * M_PI);
      const double lo = cfg->rope_beta_slow, hi = cfg->rope_beta_fast;
      const double keep = hi > lo ? std::min(1.0, std::max(0.0, (turns - lo) / (hi - lo))) : (turns >= hi ? 1.0 : 0.0);
      freq = keep * freq + (1.0 - keep) * freq / yf;
    }
    for (int p = 0; p < P; ++p) {
      const double ang = (double)p * freq;
      cs[(size_t)p * 32 + i] = (float)(gain * std::cos(ang));
      cs[(size_t)P * 32 + (size_t)p * 32 + i] = (float)(gain * std::sin(ang));
    }
  }
  HIP_TRY(hipMemcpyAsync(pk + L.rope, cs.data(), cs.size() * sizeof(float), hipMemcpyHostToDevice, s));
  HIP_TRY(hipStreamSynchronize(s));
  {  // resolve this device's static scratch address now, so the allocation-free decode need not
    void* unused = nullptr;
    const mla_status ss = scratch_for_current_device(&unused);
    if (ss != MLA_OK) return ss;
  }

  mla_ctx* c = new mla_ctx;
  c->cfg = *cfg;
  c->fp8 = fp8;
  {
    const double f = yarn ? attn_factor(cfg->rope_mscale_all_dim) : 1.0;
    c->scale = cfg->softmax_scale > 0.f ? cfg->softmax_scale : (float)(f * f / std::sqrt((double)QK));
  }
  c->g_q = (const uint16_t*)(pk + L.g_q);
  c->g_kv = (const uint16_t*)(pk + L.g_kv);
  c->w_qkva = pk + L.qkva;
  c->s_qkva = fp8 ? (const float*)(pk + L.s_qkva) : nullptr;
  c->w_qb = w->q_b;
  c->s_qb = w->q_b_s;
  c->w_kvb = w->kv_b;
  c->s_kvb = w->kv_b_s;
  c->w_ukT = (const uint16_t*)(pk + L.ukT);
  if (fp8) {
    c->w_uv = (const uint16_t*)(pk + L.uvw);
    c->uv_head_stride = (int64_t)VD * KV_LORA;
  } else {
    c->w_uv = (const uint16_t*)w->kv_b + (int64_t)NOPE * KV_LORA;
    c->uv_head_stride = (int64_t)256 * KV_LORA;
  }
  c->w_o = w->o;
  c->s_o = w->o_s;
  c->rope_cs = (const float*)(pk + L.rope);
  *out = c;
  g_last_error.clear();
  return MLA_OK;
}

void mla_destroy(mla_ctx* ctx) { delete ctx; }

mla_status mla_cache_append(mla_ctx* ctx, mla_cache* cache, int32_t seq_id, const void* entries, int32_t n,
                            mla_stream stream) {
  if (!ctx) return fail(MLA_E_ARG, "ctx is NULL");
  mla_status st = check_cache(ctx, cache);
  if (st != MLA_OK) return st;
  if (!entries) return fail(MLA_E_ARG, "entries is NULL");
  if (n <= 0) return fail(MLA_E_ARG, "n must be positive");
  if (!aligned16(entries)) return fail(MLA_E_ALIGN, "entries are not 16-byte aligned");
  st = check_seq(ctx, cache, seq_id, n);
  if (st != MLA_OK) return st;
  const int eb = (int)mla_cache_entry_bytes(&ctx->cfg);
  HIP_TRY(mla_k::cache_copy_append((uint8_t*)cache->data, slot_map(cache), (const uint8_t*)entries, eb, n, seq_id,
                                   cache->len_h[seq_id], cache->len_d, (hipStream_t)stream));
  cache->len_h[seq_id] += n;
  return MLA_OK;
}

}  // extern "C"

namespace {

// Bytes at the front of a block call's workspace that hold the normalised input [ntok][7168] bf16.
size_t block_xn_bytes(int64_t ntok) { return round_up((size_t)std::max<int64_t>(ntok, 0) * HIDDEN * 2, 256); }

// The block's h may be its x (in place: o_proj reads each residual element right before writing
// the same element) or a disjoint buffer; a partial overlap is rejected.
bool partial_overlap(const void* a, const void* b, size_t bytes) {
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  return pa != pb && pa < pb + bytes && pb < pa + bytes;
}

// One prefill call. norm_w == nullptr: the layer, y = MLA(x). Otherwise the attention half of a
// decoder block: the workspace starts with xn = input RMSNorm of x (gain norm_w), the layer runs
// on xn and o_proj adds the residual x: y = x + MLA(xn).
mla_status prefill_impl(mla_ctx* ctx, mla_cache* cache, const int32_t* seq_ids_h, const int32_t* seq_ids_d,
                        const int32_t* q_start_h, const int32_t* q_start_d, int32_t B, const void* x, void* y,
                        void* ws, size_t ws_bytes, mla_stream stream, const void* norm_w) {
  if (B <= 0) return fail(MLA_E_ARG, "B must be positive");
  if (B > MAX_BATCH) return fail(MLA_E_UNSUPPORTED, "B = %d exceeds the %d sequences a call may hold", B, MAX_BATCH);
  if (!ctx) return fail(MLA_E_ARG, "ctx is NULL");
  mla_status st = check_cache(ctx, cache);
  if (st != MLA_OK) return st;
  if (!seq_ids_h || !seq_ids_d || !q_start_h || !q_start_d || !x || !y || !ws)
    return fail(MLA_E_ARG, "a pointer argument is NULL");
  if (!aligned16(x) || !aligned16(y) || !aligned16(ws)) return fail(MLA_E_ALIGN, "x, y or ws is not 16-byte aligned");
  if (q_start_h[0] != 0) return fail(MLA_E_SHAPE, "q_start[0] must be 0");
  std::vector<int64_t> kbase(B);
  int64_t nkeys = 0;
  int max_t = 0;
  for (int b = 0; b < B; ++b) {
    const int t = q_start_h[b + 1] - q_start_h[b];
    if (t <= 0) return fail(MLA_E_SHAPE, "sequence %d of the batch has %d new tokens", b, t);
    for (int c = 0; c < b; ++c)
      if (seq_ids_h[c] == seq_ids_h[b]) return fail(MLA_E_ARG, "sequence id %d appears twice", seq_ids_h[b]);
    st = check_seq(ctx, cache, seq_ids_h[b], t);
    if (st != MLA_OK) return st;
    kbase[b] = nkeys;
    nkeys += round_up(cache->len_h[seq_ids_h[b]] + t, 64);
    max_t = std::max(max_t, t);
  }
  const int ntok = q_start_h[B];
  int64_t gp = max_gemm_part(ntok, 0, false, ctx->fp8);
  for (int b = 0; b < B; ++b)
    gp = std::max(gp, max_gemm_part(0, cache->len_h[seq_ids_h[b]] + q_start_h[b + 1] - q_start_h[b], false, ctx->fp8));
  const WsLayout L = ws_layout(ntok, B, nkeys, 0, gp, ctx->fp8);
  const size_t xn_bytes = norm_w ? block_xn_bytes(ntok) : 0;
  if (ws_bytes < xn_bytes + L.total)
    return fail(MLA_E_WORKSPACE, "workspace has %zu bytes, this call needs %zu", ws_bytes, xn_bytes + L.total);
  if (norm_w && partial_overlap(x, y, (size_t)ntok * HIDDEN * 2))
    return fail(MLA_E_ARG, "h must be x itself or not overlap it");

  hipStream_t s = (hipStream_t)stream;
  const void* resid = nullptr;
  if (norm_w) {
    HIP_TRY(mla_k::input_rmsnorm((const uint16_t*)x, (const uint16_t*)norm_w, ctx->cfg.rms_eps, ntok,
                                 (uint16_t*)ws, s));
    resid = x;
    x = ws;
  }
  uint8_t* w = (uint8_t*)ws + xn_bytes;
  const bool fp8 = ctx->fp8;
  const int eb = (int)mla_cache_entry_bytes(&ctx->cfg);
  auto* meta = (mla_k::SeqMeta*)(w + L.meta);
  const SlotMap map = slot_map(cache);
  HIP_TRY(mla_k::prefill_plan(seq_ids_d, q_start_d, map, cache->len_d, B, meta, s));

  // 1. fused q_a | kv_a projection (fp32 out); FP8: x quantised per token and 128-group first
  if (fp8)
    HIP_TRY(mla_k::quantize_rows_bf16((const uint16_t*)x, HIDDEN, ntok, HIDDEN, w + L.x8, (float*)(w + L.x8s), s));
  mla_k::GemmArgs g = gemm_common(w, L);
  set_a(ctx, g, x, HIDDEN, w + L.x8, (const float*)(w + L.x8s), HIDDEN / 128);
  g.B = ctx->w_qkva; g.ldb = HIDDEN; g.b_scale = ctx->s_qkva; g.bs_ld = HIDDEN / 128;
  g.C = w + L.cqkv; g.ldc = QKVA_N; g.M = ntok; g.N = QKVA_N; g.K = HIDDEN; g.epi = mla_k::EPI_F32;
  g.tag = mla_k::TAG_QKVA; g.ysplit_max = qkva_parts_max(ntok, ctx->fp8); g.c_split_stride = (int64_t)ntok * QKVA_N;
  const int qkva_parts = proj_ysplit(ctx, g);  // > 1 only at short prefills: the norm kernel adds them
  HIP_TRY(run_proj(ctx, g, s));
  // 2. RMSNorms, RoPE of the shared key, latent entries into the cache (FP8: quantised q_hat, c_hat)
  mla_k::NormArgs na{};
  na.cqkv = (const float*)(w + L.cqkv); na.n_part = qkva_parts; na.part_stride = (int64_t)ntok * QKVA_N;
  na.g_q = ctx->g_q; na.g_kv = ctx->g_kv;
  na.eps = ctx->cfg.rms_eps;
  na.q_hat = (uint16_t*)(w + L.q_hat); na.rope_cs = ctx->rope_cs; na.max_pos = ctx->cfg.max_positions;
  na.cache = (uint8_t*)cache->data; na.entry_bytes = eb; na.fp8 = fp8; na.n_tokens = ntok; na.meta = meta; na.B = B;
  na.map = map;
  na.q_hat_codes = w + L.q_hat; na.q_hat_scales = (float*)(w + L.qh8s);
  HIP_TRY(mla_k::norm_rope_append(na, s));
  // 3. q_b
  g = gemm_common(w, L);
  set_a(ctx, g, w + L.q_hat, Q_LORA, w + L.q_hat, (const float*)(w + L.qh8s), Q_LORA / 128);
  g.B = ctx->w_qb; g.ldb = Q_LORA; g.b_scale = ctx->s_qb; g.bs_ld = Q_LORA / 128;
  g.C = w + L.q; g.ldc = QB_N; g.M = ntok; g.N = QB_N; g.K = Q_LORA; g.tag = mla_k::TAG_QB;
  g.epi = fp8 ? mla_k::EPI_F16 : mla_k::EPI_BF16;  // FP8: fp16, the attention's operand precision
  HIP_TRY(run_proj(ctx, g, s));
  // 4. kv_b on every latent entry of each sequence (cached prefix + new): content keys, values.
  //    Paged cache: the sequences' entries are gathered into contiguous rows first (kv_b's rows and
  //    the attention's rotary keys are then read from the copy).
  const uint8_t* kv_rows = (const uint8_t*)cache->data;
  if (paged(cache)) {
    int max_rows = 0;
    for (int b = 0; b < B; ++b)
      max_rows = std::max(max_rows, cache->len_h[seq_ids_h[b]] + q_start_h[b + 1] - q_start_h[b]);
    HIP_TRY(mla_k::gather_entries((const uint8_t*)cache->data, map, meta, B, max_rows, eb, w + L.gath, s));
    kv_rows = w + L.gath;
  }
  for (int b = 0; b < B; ++b) {
    const int sid = seq_ids_h[b];
    const int n = cache->len_h[sid] + q_start_h[b + 1] - q_start_h[b];
    const uint8_t* rows = kv_rows + (paged(cache) ? kbase[b] : cache->offset_h[sid]) * (int64_t)eb;
    g = gemm_common(w, L);
    if (fp8) {  // entry = [512 codes | 4 group scales | k_pe]
      g.A = rows; g.lda = eb; g.a_scale = (const float*)(rows + KV_LORA); g.as_ld = eb / 4;
    } else {
      g.A = rows; g.lda = eb / 2;
    }
    g.B = ctx->w_kvb; g.ldb = KV_LORA; g.b_scale = ctx->s_kvb; g.bs_ld = KV_LORA / 128;
    g.M = n; g.N = KVB_N; g.K = KV_LORA; g.epi = mla_k::EPI_KVB; g.tag = mla_k::TAG_KVB;
    g.knope = (uint16_t*)(w + L.knope); g.vt = (uint16_t*)(w + L.vt); g.vt_ld = L.vt_ld; g.key_base = kbase[b];
    if (fp8) {
      g.vt_lo = (uint16_t*)(w + L.vt_lo);
    }
    HIP_TRY(run_proj(ctx, g, s));
  }
  // 5. causal attention (FP8: fp16 operands with value residuals; the epilogue applies the o_proj
  //    input quantiser and writes codes and scales)
  mla_k::PrefillAttnArgs pa{};
  pa.q = w + L.q; pa.knope = (const uint16_t*)(w + L.knope); pa.vt = (const uint16_t*)(w + L.vt);
  pa.split = fp8; pa.vt_lo = (const uint16_t*)(w + L.vt_lo);
  pa.vt_ld = L.vt_ld; pa.cache = kv_rows; pa.entry_bytes = eb;
  pa.kpe_off = fp8 ? KV_LORA + 16 : KV_LORA * 2;
  pa.rope_cs = ctx->rope_cs; pa.max_pos = ctx->cfg.max_positions; pa.meta = meta; pa.B = B; pa.max_t = max_t;
  pa.scale = ctx->scale; pa.o = (uint16_t*)(w + L.o);
  if (fp8) {  // the attention epilogue writes o_proj's quantised input
    pa.o_codes = w + L.o8;
    pa.o_scales = (float*)(w + L.o8s);
  }
  PROBED(MLA_STAGE_PREFILL_ATTN, mla_k::prefill_attention(pa, s));
  // 6. o_proj
  g = gemm_common(w, L);
  set_a(ctx, g, w + L.o, O_IN, w + L.o8, (const float*)(w + L.o8s), O_IN / 128);
  g.B = ctx->w_o; g.ldb = O_IN; g.b_scale = ctx->s_o; g.bs_ld = O_IN / 128;
  g.C = y; g.ldc = HIDDEN; g.M = ntok; g.N = HIDDEN; g.K = O_IN; g.epi = mla_k::EPI_BF16; g.tag = mla_k::TAG_OPROJ;
  g.resid = (const uint16_t*)resid; g.ldr = HIDDEN;
  PROBED(MLA_STAGE_OPROJ, run_proj(ctx, g, s));
  // 7. lengths
  HIP_TRY(mla_k::commit_lengths(seq_ids_d, q_start_d, cache->len_d, B, s));
  for (int b = 0; b < B; ++b) cache->len_h[seq_ids_h[b]] += q_start_h[b + 1] - q_start_h[b];
  return MLA_OK;
}

// One decode step; norm_w as in prefill_impl.
mla_status decode_impl(mla_ctx* ctx, mla_cache* cache, const int32_t* seq_ids_h, const int32_t* seq_ids_d, int32_t B,
                       const void* x, void* y, void* ws, size_t ws_bytes, mla_stream stream, const void* norm_w) {
  if (B <= 0) return fail(MLA_E_ARG, "B must be positive");
  if (B > MAX_BATCH) return fail(MLA_E_UNSUPPORTED, "B = %d exceeds the %d sequences a call may hold", B, MAX_BATCH);
  if (!ctx) return fail(MLA_E_ARG, "ctx is NULL");
  mla_status st = check_cache(ctx, cache);
  if (st != MLA_OK) return st;
  if (!seq_ids_h || !seq_ids_d || !x || !y || !ws) return fail(MLA_E_ARG, "a pointer argument is NULL");
  if (!aligned16(x) || !aligned16(y) || !aligned16(ws)) return fail(MLA_E_ALIGN, "x, y or ws is not 16-byte aligned");
  int lens[MAX_BATCH];  // no host allocation on the decode path (see mla_decode_static)
  for (int b = 0; b < B; ++b) {
    for (int c = 0; c < b; ++c)
      if (seq_ids_h[c] == seq_ids_h[b]) return fail(MLA_E_ARG, "sequence id %d appears twice", seq_ids_h[b]);
    st = check_seq(ctx, cache, seq_ids_h[b], 1);
    if (st != MLA_OK) return st;
    lens[b] = cache->len_h[seq_ids_h[b]] + 1;
  }
  const DecodePlan dp = plan_decode(B, lens, B, ctx->fp8);
  const int64_t gp = max_gemm_part(B, 0, true, ctx->fp8);
  const WsLayout L = ws_layout(B, B, 0, B * dp.max_splits, gp, ctx->fp8);
  const size_t xn_bytes = norm_w ? block_xn_bytes(B) : 0;
  if (ws_bytes < xn_bytes + L.total)
    return fail(MLA_E_WORKSPACE, "workspace has %zu bytes, this call needs %zu", ws_bytes, xn_bytes + L.total);
  if (norm_w && partial_overlap(x, y, (size_t)B * HIDDEN * 2))
    return fail(MLA_E_ARG, "h must be x itself or not overlap it");

  hipStream_t s = (hipStream_t)stream;
  const void* resid = nullptr;
  if (norm_w) {
    HIP_TRY(mla_k::input_rmsnorm((const uint16_t*)x, (const uint16_t*)norm_w, ctx->cfg.rms_eps, B, (uint16_t*)ws, s));
    resid = x;
    x = ws;
  }
  uint8_t* w = (uint8_t*)ws + xn_bytes;
  const bool fp8 = ctx->fp8;
  const int eb = (int)mla_cache_entry_bytes(&ctx->cfg);
  // 1. fused q_a | kv_a (K split over workgroups at small batch; the norm kernel adds the parts)
  if (fp8)
    HIP_TRY(mla_k::quantize_rows_bf16((const uint16_t*)x, HIDDEN, B, HIDDEN, w + L.x8, (float*)(w + L.x8s), s));
  mla_k::GemmArgs g = gemm_common(w, L);
  set_a(ctx, g, x, HIDDEN, w + L.x8, (const float*)(w + L.x8s), HIDDEN / 128);
  g.B = ctx->w_qkva; g.ldb = HIDDEN; g.b_scale = ctx->s_qkva; g.bs_ld = HIDDEN / 128;
  g.C = w + L.cqkv; g.ldc = QKVA_N; g.M = B; g.N = QKVA_N; g.K = HIDDEN; g.epi = mla_k::EPI_F32;
  g.tag = mla_k::TAG_QKVA; g.ysplit_max = qkva_parts_max(B, ctx->fp8); g.c_split_stride = (int64_t)B * QKVA_N;
  const int qkva_parts = proj_ysplit(ctx, g);
  HIP_TRY(run_proj(ctx, g, s));
  // 2. norms + shared-key RoPE + append at position len; len_d advances by one here
  mla_k::NormArgs na{};
  na.cqkv = (const float*)(w + L.cqkv); na.n_part = qkva_parts; na.part_stride = (int64_t)B * QKVA_N;
  na.g_q = ctx->g_q; na.g_kv = ctx->g_kv; na.eps = ctx->cfg.rms_eps;
  na.q_hat = (uint16_t*)(w + L.q_hat); na.rope_cs = ctx->rope_cs; na.max_pos = ctx->cfg.max_positions;
  na.cache = (uint8_t*)cache->data; na.entry_bytes = eb; na.fp8 = fp8; na.n_tokens = B; na.meta = nullptr;
  na.seq_ids = seq_ids_d; na.map = slot_map(cache); na.len = cache->len_d;
  na.q_hat_codes = w + L.q_hat; na.q_hat_scales = (float*)(w + L.qh8s);
  // 3. q_b. bf16 weights at one or two tokens: the norms of step 2 run inside the q_b kernel
  //    (one launch less on a latency-bound path); otherwise a norm kernel first.
  g = gemm_common(w, L);
  set_a(ctx, g, w + L.q_hat, Q_LORA, w + L.q_hat, (const float*)(w + L.qh8s), Q_LORA / 128);
  g.B = ctx->w_qb; g.ldb = Q_LORA; g.b_scale = ctx->s_qb; g.bs_ld = Q_LORA / 128;
  g.C = w + L.q; g.ldc = QB_N; g.M = B; g.N = QB_N; g.K = Q_LORA; g.tag = mla_k::TAG_QB;
  g.epi = fp8 ? mla_k::EPI_F32 : mla_k::EPI_BF16;
  if (!fp8 && mla_k::gemm_bf16_fuses_qnorm(g)) {
    HIP_TRY(mla_k::gemm_bf16_qnorm(g, na, s));
  } else {
    HIP_TRY(mla_k::norm_rope_append(na, s));
  }
  // the entries are appended and len_d advanced by the kernel just enqueued: the host mirror
  // follows at once, so the two stay equal even if a later launch fails
  for (int b = 0; b < B; ++b) cache->len_h[seq_ids_h[b]] += 1;
  if (fp8 || !mla_k::gemm_bf16_fuses_qnorm(g)) HIP_TRY(run_proj(ctx, g, s));
  // 4. absorb: q_lat[b,h,:] = q_nope[b,h,:] W_UK,h  (per-head batched). FP8: W_UK as its exact code
  //    values with the block scale of (head, latent block) on the output; q_nope is float32 and
  //    goes in as bf16 high parts (rows 0..B-1) and residuals (rows B..2B-1), float32 out. The
  //    per-head kernel (up to 128 sequences) forms the two parts while staging q_nope and adds the
  //    two products in its epilogue; otherwise the attention kernel adds them when it loads the query.
  g = gemm_common(w, L);
  if (fp8) {
    g.M = 2 * B; g.epi = mla_k::EPI_F32;
    g.c_scale = ctx->s_kvb;  // kv_b block (2h, c/128) scales W_UK,h
    g.cs_stride = 2 * (KV_LORA / 128);
  } else {
    g.A = w + L.q; g.lda = QB_N; g.sA = QK; g.M = B; g.epi = mla_k::EPI_BF16;
  }
  g.B = ctx->w_ukT; g.ldb = NOPE; g.sB = (int64_t)KV_LORA * NOPE;
  g.C = w + L.q_lat; g.ldc = HEADS * KV_LORA; g.sC = KV_LORA; g.N = KV_LORA; g.K = NOPE; g.batch = HEADS;
  g.tag = mla_k::TAG_ABSORB;
  bool absorb_paired = false;
  if (fp8) {
    // paired: the kernel splits q_nope (float32, in q) into high and residual rows while staging
    g.pair_rows = B; g.a_f32_split = true; g.c_f16 = true;  // q_lat in the attention's fp16
    g.A = w + L.q; g.lda = QB_N; g.sA = QK;
    absorb_paired = mla_k::gemm_bf16_pairs(g);
    if (!absorb_paired) {
      g.pair_rows = 0; g.a_f32_split = false; g.c_f16 = false;
      HIP_TRY(mla_k::split_q_nope((const float*)(w + L.q), B, (uint16_t*)(w + L.qs), s));
      g.A = w + L.qs; g.lda = HEADS * NOPE; g.sA = NOPE;
    }
  }
  HIP_TRY(mla_k::gemm_bf16(g, s));
  // 5. split attention over the latent cache and its merge -> o_lat
  mla_k::DecodeAttnArgs da{};
  da.q_lat = w + L.q_lat; da.q_lat_lo = (fp8 && !absorb_paired) ? (int64_t)B * HEADS * KV_LORA : 0; da.q = w + L.q;
  da.q_lat_f16 = fp8 && absorb_paired;
  da.cache = (const uint8_t*)cache->data;
  da.entry_bytes = eb; da.fp8 = fp8; da.rope_cs = ctx->rope_cs; da.max_pos = ctx->cfg.max_positions;
  da.seq_ids = seq_ids_d; da.map = slot_map(cache); da.len = cache->len_d; da.B = B; da.chunk = dp.chunk;
  da.max_splits = dp.max_splits; da.scale = ctx->scale; da.part_o = (float*)(w + L.part_o);
  da.part_ml = (float*)(w + L.part_ml); da.w_uv_s = ctx->s_kvb; da.o_lat = (uint16_t*)(w + L.o_lat);
  const bool fuse_uv = !fp8 && B <= mla_k::MERGE_UV_MAX_B;  // merge and W_UV in one kernel
  if (fuse_uv) {
    da.w_uv = (const uint16_t*)ctx->w_uv; da.uv_head_stride = ctx->uv_head_stride; da.o = (uint16_t*)(w + L.o);
  }
  PROBED(MLA_STAGE_DECODE_ATTN, mla_k::decode_attention_splits(da, s));
  // 6. W_UV per head: o[b][h*128 + d] = sum_c W_UV,h[d][c] o_lat[b][h][c]. FP8: o_lat (scaled by
  //    the blocks' scales) as high rows 0..B-1 and residual rows B..2B-1 against the exact code
  //    values, two float32 products that are added before o_proj's input quantiser. Up to 128
  //    sequences the per-head kernel merges the attention's splits itself while staging o_lat,
  //    forms the two rows, adds the two products and applies o_proj's input quantiser (a head's
  //    128 features are one quantisation group); otherwise the merge kernel writes o_lat first.
  bool uv_quantised = false;
  if (!fuse_uv) {
    g = gemm_common(w, L);
    g.A = w + L.o_lat; g.lda = HEADS * KV_LORA; g.sA = KV_LORA;
    g.B = ctx->w_uv; g.ldb = KV_LORA; g.sB = ctx->uv_head_stride;
    g.N = VD; g.K = KV_LORA; g.batch = HEADS; g.ldc = O_IN; g.sC = VD; g.tag = mla_k::TAG_UV;
    if (fp8) {
      g.M = 2 * B; g.C = w + L.o32; g.epi = mla_k::EPI_F32;
      mla_k::GemmArgs gm = g;
      gm.pair_rows = B; gm.q8_codes = w + L.o8; gm.q8_scales = (float*)(w + L.o8s); gm.q8_ld = O_IN;
      gm.q8_sld = O_IN / 128;
      gm.A = da.part_o; gm.lda = KV_LORA; gm.sA = KV_LORA; gm.a_f32_split = true;
      gm.mg_ml = da.part_ml; gm.mg_seq = seq_ids_d; gm.mg_len = cache->len_d; gm.mg_chunk = da.chunk;
      gm.mg_max_splits = da.max_splits; gm.mg_scale = ctx->s_kvb;
      uv_quantised = mla_k::gemm_bf16_pairs(gm);
      if (uv_quantised) g = gm;
    } else {
      g.M = B; g.C = w + L.o; g.epi = mla_k::EPI_BF16;
    }
    if (!uv_quantised) HIP_TRY(mla_k::decode_attention_merge(da, s));
    HIP_TRY(mla_k::gemm_bf16(g, s));
  } else {
    HIP_TRY(mla_k::decode_attention_merge(da, s));
  }
  // 7. o_proj
  if (fp8 && !uv_quantised)
    HIP_TRY(mla_k::quantize_rows_f32((const float*)(w + L.o32), (const float*)(w + L.o32) + (int64_t)B * O_IN, O_IN,
                                     B, O_IN, w + L.o8, (float*)(w + L.o8s), s));
  g = gemm_common(w, L);
  set_a(ctx, g, w + L.o, O_IN, w + L.o8, (const float*)(w + L.o8s), O_IN / 128);
  g.B = ctx->w_o; g.ldb = O_IN; g.b_scale = ctx->s_o; g.bs_ld = O_IN / 128;
  g.C = y; g.ldc = HIDDEN; g.M = B; g.N = HIDDEN; g.K = O_IN; g.epi = mla_k::EPI_BF16; g.tag = mla_k::TAG_OPROJ;
  g.resid = (const uint16_t*)resid; g.ldr = HIDDEN;
  PROBED(MLA_STAGE_OPROJ, run_proj(ctx, g, s));
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status mla_prefill(mla_ctx* ctx, mla_cache* cache, const int32_t* seq_ids_h, const int32_t* seq_ids_d,
                       const int32_t* q_start_h, const int32_t* q_start_d, int32_t B, const void* x, void* y,
                       void* ws, size_t ws_bytes, mla_stream stream) {
  return prefill_impl(ctx, cache, seq_ids_h, seq_ids_d, q_start_h, q_start_d, B, x, y, ws, ws_bytes, stream, nullptr);
}

mla_status mla_decode(mla_ctx* ctx, mla_cache* cache, const int32_t* seq_ids_h, const int32_t* seq_ids_d, int32_t B,
                      const void* x, void* y, void* ws, size_t ws_bytes, mla_stream stream) {
  return decode_impl(ctx, cache, seq_ids_h, seq_ids_d, B, x, y, ws, ws_bytes, stream, nullptr);
}

mla_status mla_decode_static(mla_ctx* ctx, mla_cache* cache, const int32_t* seq_ids_h, const int32_t* seq_ids_d,
                             int32_t B, const void* x, void* y, mla_stream stream) {
  if (B <= 0) return fail(MLA_E_ARG, "B must be positive");
  if (B > MAX_BATCH) return fail(MLA_E_UNSUPPORTED, "B = %d exceeds the %d sequences a call may hold", B, MAX_BATCH);
  if (!ctx) return fail(MLA_E_ARG, "ctx is NULL");
  void* ws = nullptr;
  const mla_status st = scratch_for_current_device(&ws);
  if (st != MLA_OK) return st;
  return decode_impl(ctx, cache, seq_ids_h, seq_ids_d, B, x, y, ws, STATIC_SCRATCH_BYTES, stream, nullptr);
}

mla_status mla_cache_pool_plan(const mla_config* cfg, int32_t n_layers, int32_t n_seqs, const int32_t* cap_h,
                               int32_t align, int64_t* offset_h, int64_t* total_slots, size_t* layer_bytes,
                               size_t* pool_bytes) {
  if (!cfg) return fail(MLA_E_ARG, "cfg is NULL");
  const mla_status st = check_config(cfg);
  if (st != MLA_OK) return st;
  if (!cap_h || !offset_h || !total_slots || !layer_bytes || !pool_bytes) return fail(MLA_E_ARG, "a pointer argument is NULL");
  if (n_layers <= 0 || n_seqs <= 0) return fail(MLA_E_ARG, "n_layers and n_seqs must be positive");
  if (align < 1 || align > 4096) return fail(MLA_E_ARG, "align %d outside [1, 4096]", align);
  int64_t slots = 0;
  for (int s = 0; s < n_seqs; ++s) {
    if (cap_h[s] < 0) return fail(MLA_E_ARG, "capacity of sequence %d is negative", s);
    if (cap_h[s] > cfg->max_positions)
      return fail(MLA_E_CAPACITY, "capacity %d of sequence %d exceeds max_positions %d", cap_h[s], s, cfg->max_positions);
    slots += ((int64_t)cap_h[s] + align - 1) / align * align;
  }
  if (slots == 0) return fail(MLA_E_ARG, "the pool would hold no slots");
  const uint64_t lb = (uint64_t)slots * mla_cache_entry_bytes(cfg);
  if (lb > UINT64_MAX / (uint64_t)n_layers) return fail(MLA_E_ARG, "pool size overflows");
  int64_t off = 0;
  for (int s = 0; s < n_seqs; ++s) {
    offset_h[s] = off;
    off += ((int64_t)cap_h[s] + align - 1) / align * align;
  }
  *total_slots = slots;
  *layer_bytes = (size_t)lb;
  *pool_bytes = (size_t)(lb * (uint64_t)n_layers);
  return MLA_OK;
}

mla_status mla_cache_pool_layer(void* pool, size_t pool_bytes, size_t layer_bytes, int32_t layer, mla_cache* cache) {
  if (!pool || !cache) return fail(MLA_E_ARG, "pool or cache is NULL");
  if (layer < 0 || layer_bytes == 0) return fail(MLA_E_ARG, "layer %d or layer_bytes %zu invalid", layer, layer_bytes);
  if (layer_bytes % 16) return fail(MLA_E_ALIGN, "layer_bytes %zu is not a multiple of 16", layer_bytes);
  if ((uint64_t)layer_bytes * (uint64_t)(layer + 1) > (uint64_t)pool_bytes)
    return fail(MLA_E_ARG, "layer %d ends past the pool's %zu bytes", layer, pool_bytes);
  if (!aligned16(pool)) return fail(MLA_E_ALIGN, "pool is not 16-byte aligned");
  cache->data = (uint8_t*)pool + (size_t)layer * layer_bytes;
  return MLA_OK;
}

}  // extern "C"

// Host page allocator: free ids in a FIFO ring (released pages are reused oldest first), plus an
// allocation bit per page so that a double free or a foreign id is refused.
struct mla_page_pool {
  std::vector<int32_t> ring;  // free ids, head .. head + count - 1 (mod n)
  std::vector<uint8_t> used;
  int32_t head = 0, count = 0;
};

extern "C" {

mla_status mla_page_pool_create(int32_t n_pages, mla_page_pool** out) {
  if (!out) return fail(MLA_E_ARG, "out is NULL");
  *out = nullptr;
  if (n_pages <= 0) return fail(MLA_E_ARG, "n_pages must be positive");
  mla_page_pool* p = new mla_page_pool;
  p->ring.resize(n_pages);
  p->used.assign(n_pages, 0);
  for (int32_t i = 0; i < n_pages; ++i) p->ring[i] = i;
  p->count = n_pages;
  *out = p;
  return MLA_OK;
}

mla_status mla_page_pool_alloc(mla_page_pool* pool, int32_t n, int32_t* ids) {
  if (!pool || (n > 0 && !ids)) return fail(MLA_E_ARG, "pool or ids is NULL");
  if (n < 0) return fail(MLA_E_ARG, "n must not be negative");
  if (n > pool->count) return fail(MLA_E_CAPACITY, "%d pages asked for, %d free", n, pool->count);
  const int32_t size = (int32_t)pool->ring.size();
  for (int32_t i = 0; i < n; ++i) {
    ids[i] = pool->ring[pool->head];
    pool->used[ids[i]] = 1;
    pool->head = (pool->head + 1) % size;
  }
  pool->count -= n;
  return MLA_OK;
}

mla_status mla_page_pool_free(mla_page_pool* pool, const int32_t* ids, int32_t n) {
  if (!pool || (n > 0 && !ids)) return fail(MLA_E_ARG, "pool or ids is NULL");
  if (n < 0) return fail(MLA_E_ARG, "n must not be negative");
  const int32_t size = (int32_t)pool->ring.size();
  for (int32_t i = 0; i < n; ++i) {  // validate everything before changing anything
    if (ids[i] < 0 || ids[i] >= size || !pool->used[ids[i]])
      return fail(MLA_E_ARG, "page %d is not an allocated page of this pool", ids[i]);
    for (int32_t j = 0; j < i; ++j)
      if (ids[j] == ids[i]) return fail(MLA_E_ARG, "page %d is freed twice", ids[i]);
  }
  for (int32_t i = 0; i < n; ++i) {
    pool->used[ids[i]] = 0;
    pool->ring[(pool->head + pool->count) % size] = ids[i];
    ++pool->count;
  }
  return MLA_OK;
}

int32_t mla_page_pool_available(const mla_page_pool* pool) { return pool ? pool->count : -1; }

void mla_page_pool_destroy(mla_page_pool* pool) { delete pool; }

size_t mla_block_prefill_workspace_bytes(const mla_ctx* ctx, int32_t max_tokens, int32_t max_batch, int64_t max_keys) {
  const size_t n = mla_prefill_workspace_bytes(ctx, max_tokens, max_batch, max_keys);
  return n ? n + block_xn_bytes(max_tokens) : 0;
}

size_t mla_block_decode_workspace_bytes(const mla_ctx* ctx, int32_t max_batch, int64_t max_keys) {
  const size_t n = mla_decode_workspace_bytes(ctx, max_batch, max_keys);
  return n ? n + block_xn_bytes(max_batch) : 0;
}

mla_status mla_block_prefill(mla_ctx* ctx, mla_cache* cache, const int32_t* seq_ids_h, const int32_t* seq_ids_d,
                             const int32_t* q_start_h, const int32_t* q_start_d, int32_t B, const void* norm_weight,
                             const void* x, void* h, void* ws, size_t ws_bytes, mla_stream stream) {
  if (!norm_weight) return fail(MLA_E_ARG, "norm_weight is NULL");
  if (!aligned16(norm_weight)) return fail(MLA_E_ALIGN, "norm_weight is not 16-byte aligned");
  return prefill_impl(ctx, cache, seq_ids_h, seq_ids_d, q_start_h, q_start_d, B, x, h, ws, ws_bytes, stream,
                      norm_weight);
}

mla_status mla_block_decode(mla_ctx* ctx, mla_cache* cache, const int32_t* seq_ids_h, const int32_t* seq_ids_d,
                            int32_t B, const void* norm_weight, const void* x, void* h, void* ws, size_t ws_bytes,
                            mla_stream stream) {
  if (!norm_weight) return fail(MLA_E_ARG, "norm_weight is NULL");
  if (!aligned16(norm_weight)) return fail(MLA_E_ALIGN, "norm_weight is not 16-byte aligned");
  return decode_impl(ctx, cache, seq_ids_h, seq_ids_d, B, x, h, ws, ws_bytes, stream, norm_weight);
}

size_t mla_test_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t batch) {
  if (M <= 0 || N <= 0 || K <= 0 || batch <= 0 || K % 128) return 0;
  return std::max<size_t>(256, (size_t)mla_k::gemm_part_floats(M, N, K, batch) * 4);
}

mla_status mla_test_probe_stage(int32_t stage, void* ev_before, void* ev_after) {
  if (stage == MLA_STAGE_NONE) {
    g_probe_stage = 0;
    return MLA_OK;
  }
  if (stage != MLA_STAGE_OPROJ && stage != MLA_STAGE_DECODE_ATTN && stage != MLA_STAGE_PREFILL_ATTN)
    return fail(MLA_E_ARG, "stage %d cannot be probed", stage);
  if (!ev_before || !ev_after) return fail(MLA_E_ARG, "an event is NULL");
  g_probe_ev0 = (hipEvent_t)ev_before;
  g_probe_ev1 = (hipEvent_t)ev_after;
  g_probe_stage = stage;
  return MLA_OK;
}

mla_status mla_test_gemm(int32_t M, int32_t N, int32_t K, int32_t batch, const void* A, int64_t lda, int64_t sA,
                         const void* B, int64_t ldb, int64_t sB, void* C, int64_t ldc, int64_t sC, int32_t out_bf16,
                         int32_t stage, void* ws, size_t ws_bytes, mla_stream stream) {
  if (M <= 0 || N <= 0 || K <= 0 || batch <= 0) return fail(MLA_E_ARG, "non-positive GEMM size");
  if (K % 128) return fail(MLA_E_UNSUPPORTED, "K must be a multiple of 128");
  if (!A || !B || !C || !ws) return fail(MLA_E_ARG, "a pointer argument is NULL");
  if (!aligned16(A) || !aligned16(B) || !aligned16(ws) || lda % 8 || ldb % 8 || (batch > 1 && (sA % 8 || sB % 8)))
    return fail(MLA_E_ALIGN, "operand rows must start on 16-byte boundaries");
  if (lda < K || ldb < K || ldc < N) return fail(MLA_E_SHAPE, "leading dimension smaller than the row");
  if (stage < 0 || stage > MLA_STAGE_UV) return fail(MLA_E_ARG, "unknown stage %d", stage);
  const size_t need = mla_test_gemm_workspace_bytes(M, N, K, batch);
  if (ws_bytes < need) return fail(MLA_E_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  mla_k::GemmArgs g;
  g.tag = stage;
  g.A = A; g.lda = lda; g.sA = sA; g.B = B; g.ldb = ldb; g.sB = sB; g.C = C; g.ldc = ldc; g.sC = sC;
  g.M = M; g.N = N; g.K = K; g.batch = batch; g.epi = out_bf16 ? mla_k::EPI_BF16 : mla_k::EPI_F32;
  g.part = (float*)ws;
  g.part_cap = mla_k::gemm_part_floats(M, N, K, batch);
  HIP_TRY(mla_k::gemm_bf16(g, (hipStream_t)stream));
  return MLA_OK;
}

size_t mla_test_gemm_fp8_workspace_bytes(int32_t M, int32_t N, int32_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 128) return 0;
  return std::max<size_t>(256, (size_t)mla_k::gemm_fp8_part_floats(M, N, K, 1) * 4);
}

mla_status mla_test_gemm_fp8(int32_t M, int32_t N, int32_t K, const void* A, const float* a_scale, const void* B,
                             const float* b_scale, float* C, int32_t precise, void* ws, size_t ws_bytes,
                             mla_stream stream) {
  if (M <= 0 || N <= 0 || K <= 0) return fail(MLA_E_ARG, "non-positive GEMM size");
  if (K % 128 || N % 8) return fail(MLA_E_UNSUPPORTED, "K must be a multiple of 128 and N of 8");
  if (!A || !a_scale || !B || !b_scale || !C || !ws) return fail(MLA_E_ARG, "a pointer argument is NULL");
  if (!aligned16(A) || !aligned16(B) || !aligned16(C) || !aligned16(ws))
    return fail(MLA_E_ALIGN, "operands must start on 16-byte boundaries");
  const size_t need = mla_test_gemm_fp8_workspace_bytes(M, N, K);
  if (ws_bytes < need) return fail(MLA_E_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  mla_k::GemmArgs g;
  g.tag = precise ? mla_k::TAG_QKVA : mla_k::TAG_OPROJ;  // the tag selects the form
  g.A = A; g.lda = K; g.B = B; g.ldb = K; g.C = C; g.ldc = N;
  g.a_scale = a_scale; g.as_ld = K / 128; g.b_scale = b_scale; g.bs_ld = K / 128;
  g.M = M; g.N = N; g.K = K; g.batch = 1; g.epi = mla_k::EPI_F32;
  g.part = (float*)ws;
  g.part_cap = mla_k::gemm_fp8_part_floats(M, N, K, 1);
  HIP_TRY(mla_k::gemm_fp8(g, (hipStream_t)stream));
  return MLA_OK;
}

}  // extern "C"
