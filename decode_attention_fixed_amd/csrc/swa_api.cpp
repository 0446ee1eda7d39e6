// C-ABI layer of libswa: argument validation (before any HIP call), the
// opaque ring-cache descriptor, workspace sizing, launches on the caller's
// stream and the thread-local error text.  See include/swa.h for the
// contract of every entry point.
#include "swa.h"

#include <hip/hip_runtime.h>  // __device__ storage (scratch) and HIP_SYMBOL

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <new>
#include <string>

#include "swa_internal.h"

struct swa_cache {
  swa_cache_config cfg;
  void* k;
  void* v;
  int32_t* slot_pos;
  size_t rows() const {
    return static_cast<size_t>(cfg.batch) * cfg.num_kv_heads *
           (static_cast<size_t>(cfg.num_sinks) + cfg.window);
  }
};

namespace {

thread_local std::string g_last_error;

swa_status fail(swa_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

swa_status ok() {
  g_last_error.clear();
  return SWA_OK;
}

swa_status from_hip(hipError_t err, const char* what) {
  if (err == hipSuccess) return ok();
  return fail(SWA_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_bytes(swa_dtype t) { return t == SWA_F32 ? 4 : 2; }  // rows given / queries

bool dtype_valid(swa_dtype t) { return t == SWA_F32 || t == SWA_BF16 || t == SWA_I8; }

bool out_dtype_valid(swa_dtype t) { return t == SWA_F32 || t == SWA_BF16; }

// Bytes of one K (or V) buffer of `rows` rows of d elements of `t`.
size_t rows_bytes(swa_dtype t, size_t rows, int32_t d) {
  if (t == SWA_I8) return swa::i8_codes_bytes(rows, d) + rows * sizeof(float);
  return rows * static_cast<size_t>(d) * (t == SWA_BF16 ? 2 : 4);
}

// Scales of an int8 buffer of `rows` rows: after the padded codes.
float* i8_scales(void* buf, size_t rows, int32_t d) {
  return reinterpret_cast<float*>(static_cast<char*>(buf) + swa::i8_codes_bytes(rows, d));
}

bool head_dim_supported(int32_t d) { return d == 64 || d == 128; }

swa_status check_config(const swa_cache_config* cfg) {
  if (cfg == nullptr) return fail(SWA_ERR_INVALID_ARG, "config is NULL");
  if (cfg->batch < 1) return fail(SWA_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", cfg->batch);
  if (cfg->num_kv_heads < 1)
    return fail(SWA_ERR_INVALID_ARG, "num_kv_heads must be >= 1 (got %d)", cfg->num_kv_heads);
  if (cfg->window < 1) return fail(SWA_ERR_INVALID_ARG, "window must be >= 1 (got %d)", cfg->window);
  if (cfg->num_sinks < 0)
    return fail(SWA_ERR_INVALID_ARG, "num_sinks must be >= 0 (got %d)", cfg->num_sinks);
  if (static_cast<int64_t>(cfg->window) + cfg->num_sinks > (int64_t{1} << 30))
    return fail(SWA_ERR_INVALID_ARG, "num_sinks + window too large");
  if (!dtype_valid(cfg->dtype)) return fail(SWA_ERR_INVALID_ARG, "unknown dtype %d", cfg->dtype);
  if (!head_dim_supported(cfg->head_dim))
    return fail(SWA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", cfg->head_dim);
  if (!(cfg->rope_base > 0.f) || !std::isfinite(cfg->rope_base))
    return fail(SWA_ERR_INVALID_ARG, "rope_base must be positive and finite");
  if (cfg->rope_style != SWA_ROPE_INTERLEAVED && cfg->rope_style != SWA_ROPE_HALF)
    return fail(SWA_ERR_INVALID_ARG, "unknown rope_style %d", cfg->rope_style);
  return SWA_OK;
}

swa_status check_group(int32_t num_q_heads, int32_t num_kv_heads) {
  if (num_q_heads < 1) return fail(SWA_ERR_INVALID_ARG, "num_q_heads must be >= 1");
  if (num_q_heads % num_kv_heads != 0)
    return fail(SWA_ERR_INVALID_ARG, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)",
                num_q_heads, num_kv_heads);
  if (!swa::group_supported(num_q_heads / num_kv_heads))
    return fail(SWA_ERR_UNSUPPORTED, "query heads per kv head = %d not supported",
                num_q_heads / num_kv_heads);
  return SWA_OK;
}

swa_status check_decode_common(const void* q, void* out, swa_dtype out_dtype, float* lse,
                               void* workspace, size_t workspace_bytes, size_t need) {
  if (q == nullptr) return fail(SWA_ERR_INVALID_ARG, "q is NULL");
  if (out == nullptr) return fail(SWA_ERR_INVALID_ARG, "out is NULL");
  if (!out_dtype_valid(out_dtype))
    return fail(SWA_ERR_INVALID_ARG, "out_dtype %d is not SWA_F32 or SWA_BF16", out_dtype);
  if (!aligned(q, 16) || !aligned(out, 16))
    return fail(SWA_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
  if (lse != nullptr && !aligned(lse, 4)) return fail(SWA_ERR_INVALID_ARG, "lse misaligned");
  if (workspace == nullptr) return fail(SWA_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(SWA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return fail(SWA_ERR_WORKSPACE, "workspace too small: %zu bytes given, %zu needed",
                workspace_bytes, need);
  return SWA_OK;
}

float resolve_scale(float scale, int32_t head_dim) {
  const float s = scale > 0.f ? scale : 1.f / std::sqrt(static_cast<float>(head_dim));
  return s * 1.44269504088896340736f;  // fold log2(e): softmax runs on exp2
}

void fill_workspace_ptrs(swa::DecodeParams& p, void* workspace,
                         const swa::WorkspaceLayout& lay) {
  char* base = static_cast<char*>(workspace);
  p.ws_o = reinterpret_cast<float*>(base + lay.o_offset);
  p.ws_lse = reinterpret_cast<float*>(base + lay.lse_offset);
  p.plan = reinterpret_cast<int32_t*>(base + lay.plan_offset);
  p.shared_base = lay.shared_base;
  p.prefix_chunks = swa::prefix_chunks(p.batch, p.num_q_heads, p.num_kv_heads);
}

// Split grid of a decode call.  The paged bf16 / head_dim 128 path runs a
// fixed balanced grid instead; num_splits then carries its size.
swa::SplitPlan plan_for(int bf16, int32_t head_dim, int32_t batch, int32_t num_kv_heads,
                        int32_t max_tokens, bool paged) {
  if (!swa::use_mfma_path(bf16, head_dim)) return swa::plan_splits(batch, num_kv_heads, max_tokens);
  if (!paged) return swa::plan_splits_mfma(batch, num_kv_heads, max_tokens);
  // rows of the pool at most (every sequence at its capacity)
  const int64_t rows = static_cast<int64_t>(batch) * num_kv_heads * max_tokens;
  swa::SplitPlan plan;
  plan.split_tokens = 0;
  plan.num_splits = rows / swa::kPoolGrid < swa::kPoolSmallRows ? swa::kPoolGrid / 2
                                                                : swa::kPoolGrid;
  return plan;
}

int log2_exact(int32_t x) {
  int s = 0;
  while ((int64_t{1} << s) < x) ++s;
  return (int64_t{1} << s) == x ? s : -1;
}

}  // namespace

// Error text shared with the other C-ABI sources (pager_api.cpp).
namespace swa {
int record_error(int code, const char* text) {
  g_last_error = text;
  return code;
}
void clear_error() { g_last_error.clear(); }
}  // namespace swa

extern "C" {

swa_status swa_cache_required_bytes(const swa_cache_config* cfg, size_t* kv_bytes_each,
                                    size_t* slot_pos_bytes) {
  swa_status st = check_config(cfg);
  if (st != SWA_OK) return st;
  if (kv_bytes_each == nullptr || slot_pos_bytes == nullptr)
    return fail(SWA_ERR_INVALID_ARG, "output pointer is NULL");
  const size_t slots = static_cast<size_t>(cfg->num_sinks) + cfg->window;
  *kv_bytes_each = rows_bytes(cfg->dtype, static_cast<size_t>(cfg->batch) * cfg->num_kv_heads * slots,
                              cfg->head_dim);
  *slot_pos_bytes = static_cast<size_t>(cfg->batch) * slots * sizeof(int32_t);
  return ok();
}

swa_status swa_cache_create(const swa_cache_config* cfg, void* k_cache, void* v_cache,
                            int32_t* slot_pos, swa_cache** out) {
  swa_status st = check_config(cfg);
  if (st != SWA_OK) return st;
  if (out == nullptr) return fail(SWA_ERR_INVALID_ARG, "out is NULL");
  if (k_cache == nullptr || v_cache == nullptr || slot_pos == nullptr)
    return fail(SWA_ERR_INVALID_ARG, "cache buffer is NULL");
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(slot_pos, 4))
    return fail(SWA_ERR_INVALID_ARG, "cache buffers must be 16-byte aligned");
  swa_cache* c = new (std::nothrow) swa_cache;
  if (c == nullptr) return fail(SWA_ERR_INVALID_ARG, "out of host memory");
  c->cfg = *cfg;
  c->k = k_cache;
  c->v = v_cache;
  c->slot_pos = slot_pos;
  *out = c;
  return ok();
}

swa_status swa_cache_reset(swa_cache* cache, void* stream) {
  if (cache == nullptr) return fail(SWA_ERR_INVALID_ARG, "cache is NULL");
  const size_t n =
      static_cast<size_t>(cache->cfg.batch) * (cache->cfg.num_sinks + cache->cfg.window);
  return from_hip(swa::launch_fill_i32(cache->slot_pos, n, -1, static_cast<hipStream_t>(stream)),
                  "swa_cache_reset");
}

void swa_cache_destroy(swa_cache* cache) { delete cache; }

swa_status kv_append_rope(swa_cache* cache, const void* k_new, const void* v_new,
                          const int32_t* pos, int32_t n_tokens, void* q_inout,
                          int32_t num_q_heads, void* stream) {
  if (cache == nullptr) return fail(SWA_ERR_INVALID_ARG, "cache is NULL");
  if (k_new == nullptr || v_new == nullptr || pos == nullptr)
    return fail(SWA_ERR_INVALID_ARG, "k_new, v_new and pos must not be NULL");
  if (n_tokens < 1) return fail(SWA_ERR_INVALID_ARG, "n_tokens must be >= 1 (got %d)", n_tokens);
  if (static_cast<int64_t>(n_tokens) * cache->cfg.batch > INT32_MAX)
    return fail(SWA_ERR_INVALID_ARG, "batch * n_tokens too large");
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(pos, 4))
    return fail(SWA_ERR_INVALID_ARG, "k_new / v_new must be 16-byte aligned");
  if (q_inout != nullptr) {
    swa_status st = check_group(num_q_heads, cache->cfg.num_kv_heads);
    if (st != SWA_OK) return st;
    if (!aligned(q_inout, 16)) return fail(SWA_ERR_INVALID_ARG, "q_inout must be 16-byte aligned");
  }
  swa::AppendParams p{};
  p.k_new = k_new;
  p.v_new = v_new;
  p.pos = pos;
  p.q_inout = q_inout;
  p.k_cache = cache->k;
  p.v_cache = cache->v;
  p.slot_pos = cache->slot_pos;
  p.batch = cache->cfg.batch;
  p.n_tokens = n_tokens;
  p.num_kv_heads = cache->cfg.num_kv_heads;
  p.num_q_heads = q_inout != nullptr ? num_q_heads : 0;
  p.head_dim = cache->cfg.head_dim;
  p.window = cache->cfg.window;
  p.sinks = cache->cfg.num_sinks;
  p.freq = swa::make_rope_freq(cache->cfg.rope_base, cache->cfg.head_dim);
  p.rope_half = cache->cfg.rope_style == SWA_ROPE_HALF;
  p.bf16 = cache->cfg.dtype != SWA_F32;
  if (cache->cfg.dtype == SWA_I8) {
    p.i8 = 1;
    p.k_scale = i8_scales(cache->k, cache->rows(), cache->cfg.head_dim);
    p.v_scale = i8_scales(cache->v, cache->rows(), cache->cfg.head_dim);
    return from_hip(swa::launch_append_i8(p, static_cast<hipStream_t>(stream)), "kv_append_rope");
  }
  return from_hip(swa::launch_append_rope(p, static_cast<hipStream_t>(stream)), "kv_append_rope");
}

swa_status decode_attn_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t max_kv_tokens, size_t* bytes) {
  if (bytes == nullptr) return fail(SWA_ERR_INVALID_ARG, "bytes is NULL");
  if (batch < 1 || num_kv_heads < 1 || max_kv_tokens < 0)
    return fail(SWA_ERR_INVALID_ARG, "batch, num_kv_heads must be >= 1, max_kv_tokens >= 0");
  swa_status st = check_group(num_q_heads, num_kv_heads);
  if (st != SWA_OK) return st;
  if (!head_dim_supported(head_dim))
    return fail(SWA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  *bytes = swa::workspace_layout(batch, num_q_heads, num_kv_heads, head_dim, max_kv_tokens).total;
  return ok();
}

// Checks a ring decode call and fills its parameters (shared by the plain
// and the fused step).
static swa_status ring_decode_params(const swa_cache* cache, const void* q, int32_t num_q_heads,
                                     float scale, void* out, swa_dtype out_dtype, float* lse,
                                     void* workspace, size_t workspace_bytes,
                                     swa::DecodeParams& p, swa::WorkspaceLayout& lay) {
  if (cache == nullptr) return fail(SWA_ERR_INVALID_ARG, "cache is NULL");
  const swa_cache_config& cfg = cache->cfg;
  swa_status st = check_group(num_q_heads, cfg.num_kv_heads);
  if (st != SWA_OK) return st;
  const int32_t slots = cfg.num_sinks + cfg.window;
  if (swa::use_mfma_path(cfg.dtype != SWA_F32, cfg.head_dim) && slots > swa::kMaxMfmaTokens)
    return fail(SWA_ERR_UNSUPPORTED, "num_sinks + window above %lld rows per sequence",
                static_cast<long long>(swa::kMaxMfmaTokens));
  const swa::SplitPlan plan =
      plan_for(cfg.dtype != SWA_F32, cfg.head_dim, cfg.batch, cfg.num_kv_heads, slots, false);
  lay = swa::workspace_layout(cfg.batch, num_q_heads, cfg.num_kv_heads, cfg.head_dim, slots);
  st = check_decode_common(q, out, out_dtype, lse, workspace, workspace_bytes, lay.total);
  if (st != SWA_OK) return st;

  p = swa::DecodeParams{};
  p.q = q;
  p.k = cache->k;
  p.v = cache->v;
  p.slot_pos = cache->slot_pos;
  p.batch = cfg.batch;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = cfg.num_kv_heads;
  p.head_dim = cfg.head_dim;
  p.slots = slots;
  p.split_tokens = plan.split_tokens;
  p.num_splits = plan.num_splits;
  p.score_scale_log2 = resolve_scale(scale, cfg.head_dim);
  p.out = out;
  p.lse = lse;
  p.out_bf16 = out_dtype == SWA_BF16;
  p.bf16 = cfg.dtype == SWA_BF16;
  if (cfg.dtype == SWA_I8) {
    p.i8 = 1;
    p.k_scale = i8_scales(cache->k, cache->rows(), cfg.head_dim);
    p.v_scale = i8_scales(cache->v, cache->rows(), cfg.head_dim);
  }
  p.sinks = cfg.num_sinks;
  p.window = cfg.window;
  p.rope_half = cfg.rope_style == SWA_ROPE_HALF;
  p.freq = swa::make_rope_freq(cfg.rope_base, cfg.head_dim);
  fill_workspace_ptrs(p, workspace, lay);
  return SWA_OK;
}

swa_status decode_attn_ring(const swa_cache* cache, const void* q, int32_t num_q_heads,
                            float scale, void* out, swa_dtype out_dtype, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream) {
  swa::DecodeParams p;
  swa::WorkspaceLayout lay;
  const swa_status st = ring_decode_params(cache, q, num_q_heads, scale, out, out_dtype, lse,
                                           workspace, workspace_bytes, p, lay);
  if (st != SWA_OK) return st;
  return from_hip(swa::launch_decode_ring(p, static_cast<hipStream_t>(stream)),
                  "decode_attn_ring");
}

static swa_status step_ring(swa_cache* cache, const void* k_new, const void* v_new,
                            const int32_t* pos, const void* q, int32_t num_q_heads, float scale,
                            void* out, swa_dtype out_dtype, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream, bool shift_sinks) {
  swa::DecodeParams p;
  swa::WorkspaceLayout lay;
  swa_status st = ring_decode_params(cache, q, num_q_heads, scale, out, out_dtype, lse, workspace,
                                     workspace_bytes, p, lay);
  if (st != SWA_OK) return st;
  if (shift_sinks && !swa::use_mfma_path(p.bf16, p.head_dim))
    return fail(SWA_ERR_UNSUPPORTED, "cache position shifting needs a bf16 cache with head_dim 128");
  p.shift_sinks = shift_sinks ? 1 : 0;
  if (k_new == nullptr || v_new == nullptr || pos == nullptr)
    return fail(SWA_ERR_INVALID_ARG, "k_new, v_new and pos must not be NULL");
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(pos, 4))
    return fail(SWA_ERR_INVALID_ARG, "k_new / v_new must be 16-byte aligned");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (swa::use_mfma_path(p.bf16 || p.i8, p.head_dim)) {  // one launch (plus the split merge)
    p.k_new = k_new;
    p.v_new = v_new;
    p.new_pos = pos;
    return from_hip(swa::launch_decode_ring(p, s), "decode_step_ring");
  }
  // Other shapes: the append (writing the rotated query into the workspace,
  // q itself is only read), then the decode over that rotated copy.
  void* q_copy = static_cast<char*>(workspace) + lay.q_offset;
  hipError_t err = hipSuccess;
  swa::AppendParams a{};
  a.k_new = k_new;
  a.v_new = v_new;
  a.pos = pos;
  a.q_inout = const_cast<void*>(q);  // read only: q_out is set
  a.q_out = q_copy;
  a.k_cache = cache->k;
  a.v_cache = cache->v;
  a.slot_pos = cache->slot_pos;
  a.batch = p.batch;
  a.n_tokens = 1;
  a.num_kv_heads = p.num_kv_heads;
  a.num_q_heads = num_q_heads;
  a.head_dim = p.head_dim;
  a.window = p.window;
  a.sinks = p.sinks;
  a.freq = p.freq;
  a.rope_half = p.rope_half;
  a.bf16 = p.bf16 || p.i8;
  if (p.i8) {
    a.i8 = 1;
    a.k_scale = const_cast<float*>(p.k_scale);
    a.v_scale = const_cast<float*>(p.v_scale);
    err = swa::launch_append_i8(a, s);
  } else {
    err = swa::launch_append_rope(a, s);
  }
  if (err != hipSuccess) return from_hip(err, "decode_step_ring");
  p.q = q_copy;
  return from_hip(swa::launch_decode_ring(p, s), "decode_step_ring");
}

swa_status decode_step_ring(swa_cache* cache, const void* k_new, const void* v_new,
                            const int32_t* pos, const void* q, int32_t num_q_heads, float scale,
                            void* out, swa_dtype out_dtype, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return step_ring(cache, k_new, v_new, pos, q, num_q_heads, scale, out, out_dtype, lse, workspace,
                   workspace_bytes, stream, false);
}

swa_status decode_step_ring_shifted(swa_cache* cache, const void* k_new, const void* v_new,
                                    const int32_t* pos, const void* q, int32_t num_q_heads,
                                    float scale, void* out, swa_dtype out_dtype, float* lse,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  return step_ring(cache, k_new, v_new, pos, q, num_q_heads, scale, out, out_dtype, lse, workspace,
                   workspace_bytes, stream, true);
}

swa_status swa_pos_advance(int32_t* pos, int32_t n, int32_t delta, void* stream) {
  if (n < 0) return fail(SWA_ERR_INVALID_ARG, "n must be >= 0 (got %d)", n);
  if (n == 0) return ok();
  if (pos == nullptr) return fail(SWA_ERR_INVALID_ARG, "pos is NULL");
  if (!aligned(pos, 4)) return fail(SWA_ERR_INVALID_ARG, "pos must be 4-byte aligned");
  return from_hip(swa::launch_add_i32(pos, static_cast<size_t>(n), delta,
                                      static_cast<hipStream_t>(stream)),
                  "swa_pos_advance");
}

swa_status swa_stream_read(const void* src, size_t bytes, void* sink, size_t sink_bytes,
                           void* stream) {
  static_assert(SWA_STREAM_READ_SINK_BYTES == swa::kStreamReadSinkBytes, "sink size");
  if (bytes % 16 != 0) return fail(SWA_ERR_INVALID_ARG, "bytes must be a multiple of 16");
  if (bytes == 0) return ok();
  if (src == nullptr || sink == nullptr) return fail(SWA_ERR_INVALID_ARG, "src or sink is NULL");
  if (!aligned(src, 16) || !aligned(sink, 4))
    return fail(SWA_ERR_INVALID_ARG, "src must be 16-byte and sink 4-byte aligned");
  if (sink_bytes < SWA_STREAM_READ_SINK_BYTES)
    return fail(SWA_ERR_INVALID_ARG, "sink needs %zu bytes", SWA_STREAM_READ_SINK_BYTES);
  return from_hip(swa::launch_stream_read(src, bytes, static_cast<uint32_t*>(sink),
                                          static_cast<hipStream_t>(stream)),
                  "swa_stream_read");
}

swa_status prefill_attn_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t n_tokens, size_t* bytes) {
  if (bytes == nullptr) return fail(SWA_ERR_INVALID_ARG, "bytes is NULL");
  if (batch < 1 || num_kv_heads < 1 || n_tokens < 1)
    return fail(SWA_ERR_INVALID_ARG, "batch, num_kv_heads, n_tokens must be >= 1");
  swa_status st = check_group(num_q_heads, num_kv_heads);
  if (st != SWA_OK) return st;
  if (head_dim != 128) return fail(SWA_ERR_UNSUPPORTED, "prefill needs head_dim 128");
  *bytes = swa::prefill_layout(batch, num_q_heads, num_kv_heads, head_dim, n_tokens).total;
  return ok();
}

swa_status prefill_attn_ring(swa_cache* cache, const void* k_new, const void* v_new,
                             const int32_t* pos, int32_t n_tokens, const void* q,
                             int32_t num_q_heads, float scale, void* out, swa_dtype out_dtype,
                             float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (cache == nullptr) return fail(SWA_ERR_INVALID_ARG, "cache is NULL");
  const swa_cache_config& cfg = cache->cfg;
  if (cfg.dtype != SWA_BF16 || cfg.head_dim != 128)
    return fail(SWA_ERR_UNSUPPORTED, "prefill needs a bf16 cache with head_dim 128");
  swa_status st = check_group(num_q_heads, cfg.num_kv_heads);
  if (st != SWA_OK) return st;
  if (k_new == nullptr || v_new == nullptr || pos == nullptr || q == nullptr || out == nullptr)
    return fail(SWA_ERR_INVALID_ARG, "k_new, v_new, pos, q and out must not be NULL");
  if (n_tokens < 1) return fail(SWA_ERR_INVALID_ARG, "n_tokens must be >= 1 (got %d)", n_tokens);
  if (static_cast<int64_t>(n_tokens) * cfg.batch * num_q_heads > INT32_MAX)
    return fail(SWA_ERR_INVALID_ARG, "batch * n_tokens * num_q_heads too large");
  // The attention kernel addresses one sequence's ring rows and one chunk's
  // rows of a kv head with 32-bit byte offsets.
  if ((static_cast<int64_t>(cfg.num_sinks) + cfg.window) * cfg.head_dim * 2 > INT32_MAX ||
      static_cast<int64_t>(n_tokens) * cfg.num_kv_heads * cfg.head_dim * 2 > INT32_MAX)
    return fail(SWA_ERR_UNSUPPORTED, "prefill needs (S + W) * d * 2 and n_tokens * Hkv * d * 2 "
                                     "below 2^31 bytes");
  // out holds float32 or bf16 rows only: an int8 code is not an output type
  if (!out_dtype_valid(out_dtype))
    return fail(SWA_ERR_INVALID_ARG, "out_dtype %d is not SWA_F32 or SWA_BF16", out_dtype);
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(q, 16) || !aligned(out, 16) ||
      !aligned(pos, 4) || (lse != nullptr && !aligned(lse, 4)))
    return fail(SWA_ERR_INVALID_ARG, "k_new / v_new / q / out must be 16-byte aligned");
  const swa::PrefillLayout lay =
      swa::prefill_layout(cfg.batch, num_q_heads, cfg.num_kv_heads, cfg.head_dim, n_tokens);
  if (workspace == nullptr) return fail(SWA_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(SWA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (workspace_bytes < lay.total)
    return fail(SWA_ERR_WORKSPACE, "workspace too small: %zu bytes, need %zu", workspace_bytes,
                lay.total);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const swa::RopeFreq freq = swa::make_rope_freq(cfg.rope_base, cfg.head_dim);

  swa::RotateChunkParams r{};
  r.q = q;
  r.k = k_new;
  r.pos = pos;
  r.q_rot = ws + lay.q_offset;
  r.k_rot = ws + lay.k_offset;
  r.batch = cfg.batch;
  r.n_tokens = n_tokens;
  r.num_q_heads = num_q_heads;
  r.num_kv_heads = cfg.num_kv_heads;
  r.rope_half = cfg.rope_style == SWA_ROPE_HALF;
  r.freq = freq;
  hipError_t err = swa::launch_rotate_chunk(r, s);
  if (err != hipSuccess) return from_hip(err, "prefill_attn_ring");

  swa::PrefillParams p{};
  p.q_rot = r.q_rot;
  p.k_rot = r.k_rot;
  p.v_new = v_new;
  p.k_cache = cache->k;
  p.v_cache = cache->v;
  p.slot_pos = cache->slot_pos;
  p.pos = pos;
  p.batch = cfg.batch;
  p.n_tokens = n_tokens;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = cfg.num_kv_heads;
  p.slots = cfg.num_sinks + cfg.window;
  p.sinks = cfg.num_sinks;
  p.window = cfg.window;
  const int32_t tokens_per_wg = swa::prefill_tokens_per_block(num_q_heads / cfg.num_kv_heads);
  p.token_blocks = (n_tokens + tokens_per_wg - 1) / tokens_per_wg;
  p.score_scale_log2 = resolve_scale(scale, cfg.head_dim);
  p.out = out;
  p.lse = lse;
  p.out_bf16 = out_dtype == SWA_BF16;
  err = swa::launch_prefill(p, s);
  if (err != hipSuccess) return from_hip(err, "prefill_attn_ring");

  swa::AppendParams a{};
  a.k_new = k_new;
  a.v_new = v_new;
  a.pos = pos;
  a.q_inout = nullptr;
  a.k_rotated = r.k_rot;  // rotated by the first launch exactly as the append would
  a.k_cache = cache->k;
  a.v_cache = cache->v;
  a.slot_pos = cache->slot_pos;
  a.batch = cfg.batch;
  a.n_tokens = n_tokens;
  a.num_kv_heads = cfg.num_kv_heads;
  a.num_q_heads = 0;
  a.head_dim = cfg.head_dim;
  a.window = cfg.window;
  a.sinks = cfg.num_sinks;
  a.freq = freq;
  a.rope_half = cfg.rope_style == SWA_ROPE_HALF;
  a.bf16 = 1;
  return from_hip(swa::launch_append_rope(a, s), "prefill_attn_ring");
}

static swa_status check_paged_desc(const swa_paged_desc* d) {
  if (d == nullptr) return fail(SWA_ERR_INVALID_ARG, "desc is NULL");
  if (d->batch < 1 || d->num_kv_heads < 1 || d->max_blocks_per_seq < 1 || d->num_phys_blocks < 1)
    return fail(SWA_ERR_INVALID_ARG,
                "batch, num_kv_heads, max_blocks_per_seq, num_phys_blocks must be >= 1");
  if (!dtype_valid(d->dtype)) return fail(SWA_ERR_INVALID_ARG, "unknown dtype %d", d->dtype);
  if (!head_dim_supported(d->head_dim))
    return fail(SWA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", d->head_dim);
  const int shift = log2_exact(d->block_size);
  if (shift < 4 || shift > 10)
    return fail(SWA_ERR_UNSUPPORTED, "block_size %d must be a power of two in [16, 1024]",
                d->block_size);
  if (static_cast<int64_t>(d->max_blocks_per_seq) * d->block_size > INT32_MAX ||
      static_cast<int64_t>(d->num_phys_blocks) * d->block_size > INT32_MAX)
    return fail(SWA_ERR_INVALID_ARG, "pool too large for 32-bit token indices");
  return SWA_OK;
}

swa_status swa_pool_required_bytes(const swa_paged_desc* desc, size_t* kv_bytes_each) {
  swa_status st = check_paged_desc(desc);
  if (st != SWA_OK) return st;
  if (kv_bytes_each == nullptr) return fail(SWA_ERR_INVALID_ARG, "kv_bytes_each is NULL");
  *kv_bytes_each = rows_bytes(desc->dtype,
                              static_cast<size_t>(desc->num_phys_blocks) * desc->num_kv_heads *
                                  desc->block_size,
                              desc->head_dim);
  return ok();
}

// Checks a paged decode call (workspace included) and launches it; shared by
// decode_attn_paged and decode_attn_paged_noalloc.
static swa_status paged_decode(const swa_paged_desc* desc, const void* q, const void* k_pool,
                               const void* v_pool, const int32_t* block_table,
                               const int32_t* seq_lens, const uint8_t* block_valid, float scale,
                               void* out, swa_dtype out_dtype, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream, const char* name,
                               const swa::PagerFuse* fuse = nullptr,
                               bool private_blocks = false) {
  swa_status st = check_paged_desc(desc);
  if (st != SWA_OK) return st;
  st = check_group(desc->num_q_heads, desc->num_kv_heads);
  if (st != SWA_OK) return st;
  if (k_pool == nullptr || v_pool == nullptr || block_table == nullptr || seq_lens == nullptr)
    return fail(SWA_ERR_INVALID_ARG, "k_pool, v_pool, block_table and seq_lens must not be NULL");
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(block_table, 4) ||
      !aligned(seq_lens, 4))
    return fail(SWA_ERR_INVALID_ARG, "pool buffers misaligned");
  const int32_t max_tokens = desc->max_blocks_per_seq * desc->block_size;
  if (swa::use_mfma_path(desc->dtype != SWA_F32, desc->head_dim) &&
      max_tokens > swa::kMaxMfmaTokens)
    return fail(SWA_ERR_UNSUPPORTED, "max_blocks_per_seq * block_size above %lld rows per sequence",
                static_cast<long long>(swa::kMaxMfmaTokens));
  const swa::SplitPlan plan = plan_for(desc->dtype != SWA_F32, desc->head_dim, desc->batch,
                                       desc->num_kv_heads, max_tokens, true);
  const swa::WorkspaceLayout lay = swa::workspace_layout(
      desc->batch, desc->num_q_heads, desc->num_kv_heads, desc->head_dim, max_tokens);
  st = check_decode_common(q, out, out_dtype, lse, workspace, workspace_bytes, lay.total);
  if (st != SWA_OK) return st;

  swa::DecodeParams p{};
  p.q = q;
  p.k = k_pool;
  p.v = v_pool;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.block_valid = block_valid;
  p.batch = desc->batch;
  p.num_q_heads = desc->num_q_heads;
  p.num_kv_heads = desc->num_kv_heads;
  p.head_dim = desc->head_dim;
  p.block_shift = log2_exact(desc->block_size);
  p.max_blocks = desc->max_blocks_per_seq;
  p.num_phys_blocks = desc->num_phys_blocks;
  p.split_tokens = plan.split_tokens;
  p.num_splits = plan.num_splits;
  p.score_scale_log2 = resolve_scale(scale, desc->head_dim);
  p.out = out;
  p.lse = lse;
  p.out_bf16 = out_dtype == SWA_BF16;
  p.bf16 = desc->dtype == SWA_BF16;
  if (desc->dtype == SWA_I8) {
    const size_t rows = static_cast<size_t>(desc->num_phys_blocks) * desc->num_kv_heads *
                        desc->block_size;
    p.i8 = 1;
    p.k_scale = i8_scales(const_cast<void*>(k_pool), rows, desc->head_dim);
    p.v_scale = i8_scales(const_cast<void*>(v_pool), rows, desc->head_dim);
  }
  fill_workspace_ptrs(p, workspace, lay);
  // no two sequences name the same block: the shared-prefix pass would find
  // nothing, so it is not launched
  if (private_blocks) p.plan = nullptr;
  return from_hip(swa::launch_decode_paged(p, static_cast<hipStream_t>(stream), fuse), name);
}

}  // extern "C"

namespace swa {
// The pager's decode (swa_pager_decode): decode_attn_paged, with the paging
// step `fuse` run after the attention in the same stream order.  The pager's
// slots are distinct pool blocks, so no two sequences share one.
swa_status paged_decode_with_copies(const swa_paged_desc* desc, const void* q, const void* k_pool,
                                    const void* v_pool, const int32_t* block_table,
                                    const int32_t* seq_lens, const uint8_t* block_valid,
                                    float scale, void* out, swa_dtype out_dtype, float* lse,
                                    void* workspace, size_t workspace_bytes, void* stream,
                                    const PagerFuse* fuse) {
  return paged_decode(desc, q, k_pool, v_pool, block_table, seq_lens, block_valid, scale, out,
                      out_dtype, lse, workspace, workspace_bytes, stream, "swa_pager_decode", fuse,
                      true);
}
}  // namespace swa

extern "C" {

swa_status decode_attn_paged(const swa_paged_desc* desc, const void* q, const void* k_pool,
                             const void* v_pool, const int32_t* block_table,
                             const int32_t* seq_lens, const uint8_t* block_valid, float scale,
                             void* out, swa_dtype out_dtype, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return paged_decode(desc, q, k_pool, v_pool, block_table, seq_lens, block_valid, scale, out,
                      out_dtype, lse, workspace, workspace_bytes, stream, "decode_attn_paged");
}

}  // extern "C"

// ---------------------------------------------------------------------------
// decode_attn_paged_noalloc: the paged decode with its partial results in a
// fixed device array of this library instead of a caller's workspace, for
// callers that cannot allocate.
// ---------------------------------------------------------------------------

namespace {

constexpr size_t kScratchBytes = size_t{32} << 20;
static_assert(SWA_NOALLOC_SCRATCH_BYTES == kScratchBytes, "swa.h states the scratch maximum");

// One copy per device, held from the module's load until the process ends.
// In host code this name is only a handle for hipGetSymbolAddress: kernels
// get the device address looked up below.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's `scratch`, looked up on the first
// call on that device (with the device current) and kept.
swa_status scratch_for_current_device(void** ptr) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return from_hip(err, "decode_attn_paged_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SWA_ERR_UNSUPPORTED, "decode_attn_paged_noalloc: device %d beyond %d", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess)
      return from_hip(err, "decode_attn_paged_noalloc: hipGetSymbolAddress(scratch)");
    if (p == nullptr || !aligned(p, 256))
      return fail(SWA_ERR_HIP, "decode_attn_paged_noalloc: scratch address unusable");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return SWA_OK;
}

}  // namespace

extern "C" {

swa_status decode_attn_paged_noalloc(const swa_paged_desc* desc, const void* q,
                                     const void* k_pool, const void* v_pool,
                                     const int32_t* block_table, const int32_t* seq_lens,
                                     const uint8_t* block_valid, float scale, void* out,
                                     swa_dtype out_dtype, float* lse, void* stream) {
  // The size check comes first, on the host: a call beyond the fixed
  // maximum is refused before any HIP call.
  swa_status st = check_paged_desc(desc);
  if (st != SWA_OK) return st;
  st = check_group(desc->num_q_heads, desc->num_kv_heads);
  if (st != SWA_OK) return st;
  const size_t need =
      swa::workspace_layout(desc->batch, desc->num_q_heads, desc->num_kv_heads, desc->head_dim,
                            desc->max_blocks_per_seq * desc->block_size)
          .total;
  if (need > kScratchBytes)
    return fail(SWA_ERR_WORKSPACE,
                "decode_attn_paged_noalloc: these sizes need %zu bytes of partial results, "
                "above the fixed %zu-byte maximum (use decode_attn_paged with a workspace)",
                need, kScratchBytes);
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != SWA_OK) return st;
  return paged_decode(desc, q, k_pool, v_pool, block_table, seq_lens, block_valid, scale, out,
                      out_dtype, lse, ws, kScratchBytes, stream, "decode_attn_paged_noalloc");
}

swa_status kv_write_paged(const swa_paged_desc* desc, void* k_pool, void* v_pool,
                          const void* k_src, const void* v_src, const int32_t* dst_rows,
                          const int32_t* pos, int32_t n_tokens, float rope_base,
                          swa_rope_style rope_style, void* stream) {
  swa_status st = check_paged_desc(desc);
  if (st != SWA_OK) return st;
  if (k_pool == nullptr || v_pool == nullptr || k_src == nullptr || v_src == nullptr ||
      dst_rows == nullptr)
    return fail(SWA_ERR_INVALID_ARG, "pool, source and dst_rows pointers must not be NULL");
  if (n_tokens < 1) return fail(SWA_ERR_INVALID_ARG, "n_tokens must be >= 1 (got %d)", n_tokens);
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(k_src, 16) || !aligned(v_src, 16))
    return fail(SWA_ERR_INVALID_ARG, "pool and source rows must be 16-byte aligned");
  if (pos != nullptr) {
    if (!(rope_base > 0.f) || !std::isfinite(rope_base))
      return fail(SWA_ERR_INVALID_ARG, "rope_base must be positive and finite");
    if (rope_style != SWA_ROPE_INTERLEAVED && rope_style != SWA_ROPE_HALF)
      return fail(SWA_ERR_INVALID_ARG, "unknown rope_style %d", rope_style);
  }
  swa::PagedWriteParams p{};
  p.k_src = k_src;
  p.v_src = v_src;
  p.dst_rows = dst_rows;
  p.pos = pos;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.n_tokens = n_tokens;
  p.num_kv_heads = desc->num_kv_heads;
  p.head_dim = desc->head_dim;
  p.block_size = desc->block_size;
  p.num_phys_blocks = desc->num_phys_blocks;
  p.freq = swa::make_rope_freq(rope_base, desc->head_dim);
  p.rope_half = rope_style == SWA_ROPE_HALF;
  p.bf16 = desc->dtype != SWA_F32;
  if (desc->dtype == SWA_I8) {
    const size_t rows = static_cast<size_t>(desc->num_phys_blocks) * desc->num_kv_heads *
                        desc->block_size;
    p.i8 = 1;
    p.k_scale = i8_scales(k_pool, rows, desc->head_dim);
    p.v_scale = i8_scales(v_pool, rows, desc->head_dim);
    return from_hip(swa::launch_write_paged_i8(p, static_cast<hipStream_t>(stream)),
                    "kv_write_paged");
  }
  return from_hip(swa::launch_write_paged(p, static_cast<hipStream_t>(stream)), "kv_write_paged");
}

const char* swa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
