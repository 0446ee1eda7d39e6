/* A plain C host program over the C-ABI of libswa (include/swa.h) and the
 * HIP runtime's C API only: no Python, no PyTorch.  It builds a ring cache
 * from a history, runs fused decode steps, and writes what it computed; or,
 * with --pool, fills a paged pool and runs paged decode steps.
 *
 *   capi_check <input file> <output file>
 *   capi_check --pool <input file> <output file>
 *
 * Ring input (little-endian): int32 B, Hq, Hkv, d, W, S, n_hist, n_steps,
 * rope_half; float32 rope_base; then bf16 arrays
 *   hist_k, hist_v  [B, n_hist, Hkv, d]   (positions pos0[b] + j)
 *   step_k, step_v  [n_steps, B, Hkv, d]
 *   step_q          [n_steps, B, Hq, d]   (not rotated)
 * then int32 pos0 [B] and step_pos [n_steps, B].
 * Output: float32 out [n_steps, B, Hq, d], float32 lse [n_steps, B, Hq],
 * int32 slot_pos [B, S + W] after the last step.
 *
 * Pool input: int32 B, Hq, Hkv, d, block_size, max_blocks, num_phys, n_rows,
 * n_steps, rope_half, i8 (1: an SWA_I8 pool, quantised by the write; the
 * rows and queries stay bf16); float32 rope_base; then bf16 k_src, v_src
 * [n_rows, Hkv, d] (K not rotated); int32 dst_rows [n_rows], pos [n_rows];
 * int32 block_table [B, max_blocks], seq_lens [B]; uint8 block_valid
 * [B, max_blocks]; bf16 q [n_steps, B, Hq, d] (already rotated).  Pool rows
 * that no dst_rows entry names hold NaN.
 * Output: float32 out [n_steps, B, Hq, d], float32 lse [n_steps, B, Hq].
 *
 * Exit status 0 on success; a failing call prints swa_last_error(). */

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "swa.h"

static int fail_hip(const char* what, hipError_t e) {
  fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return 1;
}

static int fail_swa(const char* what, swa_status s) {
  fprintf(stderr, "%s failed (%d): %s\n", what, (int)s, swa_last_error());
  return 1;
}

#define HIP(call)                               \
  do {                                          \
    hipError_t e_ = (call);                     \
    if (e_ != hipSuccess) return fail_hip(#call, e_); \
  } while (0)
#define SWA(call)                               \
  do {                                          \
    swa_status s_ = (call);                     \
    if (s_ != SWA_OK) return fail_swa(#call, s_); \
  } while (0)

static void* read_all(FILE* f, size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (p != NULL && bytes && fread(p, 1, bytes, f) != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

static void* to_device(const void* host, size_t bytes, int* err) {
  void* d = NULL;
  if (hipMalloc(&d, bytes ? bytes : 16) != hipSuccess ||
      hipMemcpy(d, host, bytes, hipMemcpyHostToDevice) != hipSuccess) {
    *err = 1;
    return NULL;
  }
  return d;
}

static int run_ring(const char* in_path, const char* out_path) {
  FILE* in = fopen(in_path, "rb");
  if (in == NULL) return 2;
  int32_t hdr[9];
  float rope_base;
  if (fread(hdr, sizeof(int32_t), 9, in) != 9 || fread(&rope_base, 4, 1, in) != 1) return 2;
  const int32_t B = hdr[0], Hq = hdr[1], Hkv = hdr[2], d = hdr[3], W = hdr[4], S = hdr[5];
  const int32_t n_hist = hdr[6], n_steps = hdr[7], rope_half = hdr[8];
  const size_t kv_hist = (size_t)B * n_hist * Hkv * d * 2;
  const size_t kv_step = (size_t)B * Hkv * d * 2;
  const size_t q_step = (size_t)B * Hq * d * 2;
  void* hk = read_all(in, kv_hist);
  void* hv = read_all(in, kv_hist);
  void* sk = read_all(in, kv_step * n_steps);
  void* sv = read_all(in, kv_step * n_steps);
  void* sq = read_all(in, q_step * n_steps);
  int32_t* pos0 = (int32_t*)read_all(in, (size_t)B * 4);
  int32_t* spos = (int32_t*)read_all(in, (size_t)B * n_steps * 4);
  fclose(in);
  if (!hk || !hv || !sk || !sv || !sq || !pos0 || !spos) return 2;

  swa_cache_config cfg = {B, Hkv, d, W, S, SWA_BF16, rope_base,
                          rope_half ? SWA_ROPE_HALF : SWA_ROPE_INTERLEAVED};
  size_t kv_bytes = 0, sp_bytes = 0, ws_bytes = 0;
  SWA(swa_cache_required_bytes(&cfg, &kv_bytes, &sp_bytes));
  SWA(decode_attn_workspace_bytes(B, Hq, Hkv, d, S + W, &ws_bytes));
  void *k_cache = NULL, *v_cache = NULL, *slot_pos = NULL, *ws = NULL, *out = NULL, *lse = NULL;
  HIP(hipMalloc(&k_cache, kv_bytes));
  HIP(hipMalloc(&v_cache, kv_bytes));
  HIP(hipMalloc(&slot_pos, sp_bytes));
  HIP(hipMalloc(&ws, ws_bytes));
  HIP(hipMalloc(&out, (size_t)B * Hq * d * 4));
  HIP(hipMalloc(&lse, (size_t)B * Hq * 4));
  int err = 0;
  void* d_hk = to_device(hk, kv_hist, &err);
  void* d_hv = to_device(hv, kv_hist, &err);
  void* d_pos0 = to_device(pos0, (size_t)B * 4, &err);
  void* d_sk = to_device(sk, kv_step * n_steps, &err);
  void* d_sv = to_device(sv, kv_step * n_steps, &err);
  void* d_sq = to_device(sq, q_step * n_steps, &err);
  void* d_spos = to_device(spos, (size_t)B * n_steps * 4, &err);
  if (err) return fail_hip("upload", hipErrorOutOfMemory);

  hipStream_t stream;
  HIP(hipStreamCreate(&stream));
  swa_cache* cache = NULL;
  SWA(swa_cache_create(&cfg, k_cache, v_cache, (int32_t*)slot_pos, &cache));
  SWA(swa_cache_reset(cache, stream));
  if (n_hist > 0)
    SWA(kv_append_rope(cache, d_hk, d_hv, (const int32_t*)d_pos0, n_hist, NULL, Hq, stream));

  FILE* o = fopen(out_path, "wb");
  if (o == NULL) return 2;
  float* h_out = (float*)malloc((size_t)B * Hq * d * 4 * n_steps);
  float* h_lse = (float*)malloc((size_t)B * Hq * 4 * n_steps);
  for (int32_t s = 0; s < n_steps; ++s) {
    SWA(decode_step_ring(cache, (char*)d_sk + kv_step * s, (char*)d_sv + kv_step * s,
                         (const int32_t*)d_spos + (size_t)B * s, (char*)d_sq + q_step * s, Hq,
                         0.0f, out, SWA_F32, (float*)lse, ws, ws_bytes, stream));
    HIP(hipMemcpyAsync(h_out + (size_t)B * Hq * d * s, out, (size_t)B * Hq * d * 4,
                       hipMemcpyDeviceToHost, stream));
    HIP(hipMemcpyAsync(h_lse + (size_t)B * Hq * s, lse, (size_t)B * Hq * 4,
                       hipMemcpyDeviceToHost, stream));
  }
  int32_t* h_sp = (int32_t*)malloc(sp_bytes);
  HIP(hipMemcpyAsync(h_sp, slot_pos, sp_bytes, hipMemcpyDeviceToHost, stream));
  HIP(hipStreamSynchronize(stream));
  fwrite(h_out, 4, (size_t)B * Hq * d * n_steps, o);
  fwrite(h_lse, 4, (size_t)B * Hq * n_steps, o);
  fwrite(h_sp, 1, sp_bytes, o);
  fclose(o);

  swa_cache_destroy(cache);
  HIP(hipStreamDestroy(stream));
  hipFree(k_cache);
  hipFree(v_cache);
  hipFree(slot_pos);
  hipFree(ws);
  hipFree(out);
  hipFree(lse);
  hipFree(d_hk);
  hipFree(d_hv);
  hipFree(d_pos0);
  hipFree(d_sk);
  hipFree(d_sv);
  hipFree(d_sq);
  hipFree(d_spos);
  printf("capi_check: %d steps\n", n_steps);
  return 0;
}

static int run_pool(const char* in_path, const char* out_path) {
  FILE* in = fopen(in_path, "rb");
  if (in == NULL) return 2;
  int32_t hdr[11];
  float rope_base;
  if (fread(hdr, sizeof(int32_t), 11, in) != 11 || fread(&rope_base, 4, 1, in) != 1) return 2;
  const int32_t B = hdr[0], Hq = hdr[1], Hkv = hdr[2], d = hdr[3], bs = hdr[4];
  const int32_t max_blocks = hdr[5], num_phys = hdr[6], n_rows = hdr[7], n_steps = hdr[8];
  const int32_t rope_half = hdr[9], i8 = hdr[10];
  const size_t src_bytes = (size_t)n_rows * Hkv * d * 2;
  const size_t q_step = (size_t)B * Hq * d * 2;
  const size_t table_n = (size_t)B * max_blocks;
  void* ks = read_all(in, src_bytes);
  void* vs = read_all(in, src_bytes);
  void* rows = read_all(in, (size_t)n_rows * 4);
  void* pos = read_all(in, (size_t)n_rows * 4);
  void* table = read_all(in, table_n * 4);
  void* lens = read_all(in, (size_t)B * 4);
  void* valid = read_all(in, table_n);
  void* q = read_all(in, q_step * n_steps);
  fclose(in);
  if (!ks || !vs || !rows || !pos || !table || !lens || !valid || !q) return 2;

  swa_paged_desc desc = {B, Hq, Hkv, d, bs, max_blocks, num_phys, i8 ? SWA_I8 : SWA_BF16};
  size_t pool_bytes = 0, ws_bytes = 0;
  SWA(swa_pool_required_bytes(&desc, &pool_bytes));
  SWA(decode_attn_workspace_bytes(B, Hq, Hkv, d, max_blocks * bs, &ws_bytes));
  void *k_pool = NULL, *v_pool = NULL, *ws = NULL, *out = NULL, *lse = NULL;
  HIP(hipMalloc(&k_pool, pool_bytes));
  HIP(hipMalloc(&v_pool, pool_bytes));
  HIP(hipMalloc(&ws, ws_bytes));
  HIP(hipMalloc(&out, (size_t)B * Hq * d * 4));
  HIP(hipMalloc(&lse, (size_t)B * Hq * 4));
  HIP(hipMemset(k_pool, 0xFF, pool_bytes));  /* bf16 NaN (int8: NaN scales) when unwritten */
  HIP(hipMemset(v_pool, 0xFF, pool_bytes));
  int err = 0;
  void* d_ks = to_device(ks, src_bytes, &err);
  void* d_vs = to_device(vs, src_bytes, &err);
  void* d_rows = to_device(rows, (size_t)n_rows * 4, &err);
  void* d_pos = to_device(pos, (size_t)n_rows * 4, &err);
  void* d_table = to_device(table, table_n * 4, &err);
  void* d_lens = to_device(lens, (size_t)B * 4, &err);
  void* d_valid = to_device(valid, table_n, &err);
  void* d_q = to_device(q, q_step * n_steps, &err);
  if (err) return fail_hip("upload", hipErrorOutOfMemory);

  hipStream_t stream;
  HIP(hipStreamCreate(&stream));
  SWA(kv_write_paged(&desc, k_pool, v_pool, d_ks, d_vs, (const int32_t*)d_rows,
                     (const int32_t*)d_pos, n_rows, rope_base,
                     rope_half ? SWA_ROPE_HALF : SWA_ROPE_INTERLEAVED, stream));
  float* h_out = (float*)malloc((size_t)B * Hq * d * 4 * n_steps);
  float* h_lse = (float*)malloc((size_t)B * Hq * 4 * n_steps);
  for (int32_t s = 0; s < n_steps; ++s) {
    SWA(decode_attn_paged(&desc, (char*)d_q + q_step * s, k_pool, v_pool,
                          (const int32_t*)d_table, (const int32_t*)d_lens,
                          (const uint8_t*)d_valid, 0.0f, out, SWA_F32, (float*)lse, ws,
                          ws_bytes, stream));
    HIP(hipMemcpyAsync(h_out + (size_t)B * Hq * d * s, out, (size_t)B * Hq * d * 4,
                       hipMemcpyDeviceToHost, stream));
    HIP(hipMemcpyAsync(h_lse + (size_t)B * Hq * s, lse, (size_t)B * Hq * 4,
                       hipMemcpyDeviceToHost, stream));
  }
  HIP(hipStreamSynchronize(stream));
  FILE* o = fopen(out_path, "wb");
  if (o == NULL) return 2;
  fwrite(h_out, 4, (size_t)B * Hq * d * n_steps, o);
  fwrite(h_lse, 4, (size_t)B * Hq * n_steps, o);
  fclose(o);

  HIP(hipStreamDestroy(stream));
  void* bufs[] = {k_pool, v_pool, ws, out, lse, d_ks, d_vs, d_rows, d_pos, d_table, d_lens,
                  d_valid, d_q};
  for (size_t i = 0; i < sizeof(bufs) / sizeof(bufs[0]); ++i) hipFree(bufs[i]);
  printf("capi_check --pool: %d steps\n", n_steps);
  return 0;
}

int main(int argc, char** argv) {
  if (argc == 4 && strcmp(argv[1], "--pool") == 0) return run_pool(argv[2], argv[3]);
  if (argc == 3) return run_ring(argv[1], argv[2]);
  fprintf(stderr, "usage: %s [--pool] <input> <output>\n", argv[0]);
  return 2;
}
