// Internal interface between the C-ABI layer (swa_api.cpp) and the HIP
// kernels (append_rope.hip, decode.hip).  Launchers return hipError_t from
// the launch; arguments reaching them have been validated by the caller.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include <cmath>

namespace swa {

constexpr int kMaxGroup = 8;
// Shapes of the bf16 / head_dim 128 decode kernel.  Ring caches: 8-wave
// workgroups (one per CU, whole sequences).  Paged pools: a fixed balanced
// grid of kPoolGrid 4-wave workgroups (two per CU), or kPoolGrid / 2 8-wave
// workgroups when the pool holds fewer than kPoolSmallRows rows per
// 4-wave workgroup (the per-workgroup start and the merge of many small
// shares would dominate).
#ifndef SWA_RING_WAVES
#define SWA_RING_WAVES 8
#endif
constexpr int kRingWaves = SWA_RING_WAVES;
constexpr int kPoolGrid = 512;  // a power of two, and so is kPoolGrid / 2
static_assert((kPoolGrid & (kPoolGrid - 1)) == 0, "balanced grid must be a power of two");
constexpr int64_t kPoolSmallRows = 2048;
constexpr int kMaxMfmaSplits = 512;             // ring splits per sequence on that path
constexpr int64_t kMaxMfmaTokens = 512 * 8192;  // rows per sequence on that path

// Shared-prefix pass of the paged decode (bf16 pools, head_dim 128, batch
// 2 .. kPrefixMaxBatch): the leading blocks that sequences' tables share with
// the longest sequence's table are attended once per kv head for all of them
// (their query heads stacked as matrix-core columns), in kPrefixChunks key
// chunks; the pool kernel then attends each sequence's remaining rows and
// the merge adds the chunks' partials.  The plan the pass finds lives in the
// workspace: plan[0] shared rows (0: nothing shared), plan[1] the reference
// sequence, plan[2] sharers, plan[kPlanHead + b] rows of sequence b served by
// the pass (0: not a sharer).
constexpr int kPrefixChunks = 16;      // key chunks per kv head, at most
constexpr int kPrefixCols = 128;       // query columns per workgroup of the pass
constexpr int kPrefixMaxBatch = 1024;
constexpr int kPrefixMaxRows = 16384;  // shared rows scanned for (more stay private)
constexpr int kPlanHead = 4;
// Key chunks per kv head: enough workgroups (kv heads x chunks x column
// blocks) to cover the chip, at most kPrefixChunks.  The workspace sizing,
// the pass and the merge all take it from here.
inline int prefix_chunks(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads) {
  const int64_t col_blocks =
      (static_cast<int64_t>(batch) * (num_q_heads / num_kv_heads) + kPrefixCols - 1) / kPrefixCols;
  const int64_t wgs = static_cast<int64_t>(num_kv_heads) * col_blocks;
  const int64_t c = (256 + wgs - 1) / wgs;
  return static_cast<int>(c < 1 ? 1 : (c > kPrefixChunks ? kPrefixChunks : c));
}

// RoPE frequencies theta_i = base^(-2i/d), i < d/2 (d <= 128), computed on
// the host in float64 and passed by value to every kernel that rotates.
constexpr int kMaxRopePairs = 64;
struct RopeFreq {
  double theta[kMaxRopePairs];
};
inline RopeFreq make_rope_freq(double base, int head_dim) {
  RopeFreq f{};
  for (int i = 0; i < head_dim / 2 && i < kMaxRopePairs; ++i)
    f.theta[i] = std::pow(base, -2.0 * static_cast<double>(i) / static_cast<double>(head_dim));
  return f;
}

struct AppendParams {
  const void* k_new;      // [B, T, Hkv, d]
  const void* v_new;      // [B, T, Hkv, d]
  const int32_t* pos;     // [B]
  void* q_inout;          // [B, T, Hq, d] or null
  void* q_out;            // [B, T, Hq, d] or null: rotated queries go here, q_inout is only read
  const void* k_rotated;  // [B, T, Hkv, d] or null: K rows already rotated (and rounded) exactly
                          // as this kernel would, copied instead of k_new
  void* k_cache;          // [B, Hkv, S+W, d]
  void* v_cache;
  int32_t* slot_pos;      // [B, S+W]
  int32_t batch, n_tokens, num_kv_heads, num_q_heads, head_dim, window, sinks;
  RopeFreq freq;
  int rope_half;          // 0: pairs (2i, 2i+1); 1: pairs (i, i + d/2)
  int bf16;               // storage dtype (inputs and queries: bf16 also when i8)
  int i8;                 // int8 rows: codes in k_cache / v_cache, scales below
  float* k_scale;         // [B, Hkv, S+W] (i8)
  float* v_scale;
};

struct PagedWriteParams {
  const void* k_src;      // [N, Hkv, d]
  const void* v_src;
  const int32_t* dst_rows;  // [N]
  const int32_t* pos;       // [N] or null
  void* k_pool;           // [Nphys, Hkv, bs, d]
  void* v_pool;
  int32_t n_tokens, num_kv_heads, head_dim, block_size, num_phys_blocks;
  RopeFreq freq;
  int rope_half;
  int bf16;
  int i8;                 // int8 rows (sources bf16): codes in the pools, scales below
  float* k_scale;         // [Nphys, Hkv, bs] (i8)
  float* v_scale;
};

// int8 row storage: codes of all rows first, padded to 256 bytes, then one
// float32 scale per row.
inline size_t i8_codes_bytes(size_t rows, int head_dim) {
  return (rows * static_cast<size_t>(head_dim) + 255) / 256 * 256;
}
inline size_t i8_buffer_bytes(size_t rows, int head_dim) {
  return i8_codes_bytes(rows, head_dim) + rows * sizeof(float);
}

// One decode step, both addressing modes.  The split kernel writes one
// partial (normalised output, base-2 log-sum-exp) per (sequence, query head,
// split); the merge kernel combines the partials of each (sequence, head).
struct DecodeParams {
  const void* q;              // [B, Hq, d]
  const void* k;              // ring [B, Hkv, slots, d] | pool [Nphys, Hkv, bs, d]
  const void* v;
  const int32_t* slot_pos;    // ring: [B, slots]
  const int32_t* block_table; // pool: [B, max_blocks]
  const int32_t* seq_lens;    // pool: [B]
  const uint8_t* block_valid; // pool: [B, max_blocks] or null
  int32_t batch, num_q_heads, num_kv_heads, head_dim;
  int32_t slots;              // ring: S + W
  int32_t block_shift;        // pool: log2(block_size)
  int32_t max_blocks, num_phys_blocks;
  int32_t split_tokens, num_splits;
  float score_scale_log2;     // softmax scale * log2(e)
  float* ws_o;                // [B, Hq, num_splits, d]
  float* ws_lse;              // [B, Hq, num_splits]
  void* out;                  // [B, Hq, d]
  float* lse;                 // [B, Hq] or null
  int out_bf16;
  int bf16;
  int i8;                     // int8 rows with per-row scales (queries bf16)
  const float* k_scale;       // scale of each row, in the row order of k / v
  const float* v_scale;
  // Fused decode step (ring): the new token of each sequence is appended by
  // the decode launch itself.  new_pos null: plain decode.
  const void* k_new;          // [B, Hkv, d], not rotated
  const void* v_new;          // [B, Hkv, d]
  const int32_t* new_pos;     // [B]
  int32_t sinks, window;
  int32_t rope_half;
  int32_t shift_sinks;        // fused step: positions inside the cache (sinks scored
                              // against the query rotated at its cache position)
  RopeFreq freq;
  // Paged pools: the shared-prefix plan in the workspace, or null when the
  // pass does not run; partial slot of chunk c of unit u: shared_base + c *
  // B * Hkv + u.
  int32_t* plan;
  int64_t shared_base;
  int32_t prefix_chunks;      // prefix_chunks(batch, Hq, Hkv)
};

struct SplitPlan {
  int32_t split_tokens;
  int32_t num_splits;
};

// How a sequence's token range is cut into splits (shared by the workspace
// query and the launch so both agree).  The bf16 / head_dim-128 path runs
// multi-wave workgroups and merges across workgroups inside the kernel; the
// generic path runs one wave per split and a separate merge kernel.
bool use_mfma_path(int bf16, int32_t head_dim);
SplitPlan plan_splits(int32_t batch, int32_t num_kv_heads, int32_t max_kv_tokens);
SplitPlan plan_splits_mfma(int32_t batch, int32_t num_kv_heads, int32_t max_kv_tokens);

// Workspace layout: [partial outputs | partial lse], each region 256-byte
// aligned, in partial slots of g = Hq/Hkv heads: enough slots for whichever
// path needs most (B*Hkv*splits for split grids, B*Hkv + kPoolGrid for the
// balanced pool grid).
struct WorkspaceLayout {
  size_t o_offset;
  size_t lse_offset;
  size_t q_offset;     // [B, Hq, d] query copy of a fused step that runs as two launches
  size_t plan_offset;  // [kPlanHead + B] int32: the shared-prefix plan
  int64_t shared_base; // first partial slot of the shared-prefix pass
  size_t total;
};
WorkspaceLayout workspace_layout(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_kv_tokens);

hipError_t launch_fill_i32(int32_t* dst, size_t n, int32_t value, hipStream_t stream);
hipError_t launch_add_i32(int32_t* dst, size_t n, int32_t delta, hipStream_t stream);
// Reads bytes (a multiple of 16, 16-byte aligned) of src once; one XOR word
// per wave of the kStreamReadGrid workgroups to sink.
constexpr int kStreamReadGrid = 2048;
constexpr size_t kStreamReadSinkBytes = 32768;
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);
hipError_t launch_append_rope(const AppendParams& p, hipStream_t stream);
hipError_t launch_append_i8(const AppendParams& p, hipStream_t stream);
hipError_t launch_write_paged_i8(const PagedWriteParams& p, hipStream_t stream);
hipError_t launch_write_paged(const PagedWriteParams& p, hipStream_t stream);
hipError_t launch_decode_ring(const DecodeParams& p, hipStream_t stream);
struct PagerFuse;
// fuse: a paging step to run after the attention (null: none).
hipError_t launch_decode_paged(const DecodeParams& p, hipStream_t stream,
                               const PagerFuse* fuse = nullptr);
hipError_t launch_decode_mfma_ring(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_mfma_pool(const DecodeParams& p, hipStream_t stream,
                                   const PagerFuse* fuse = nullptr);
// The shared-prefix pass (one launch; finds and writes the plan too).
bool prefix_pass_applies(const DecodeParams& p);
hipError_t launch_shared_prefix(const DecodeParams& p, hipStream_t stream);

bool group_supported(int g);

// Chunked prefill over a ring cache (bf16, head_dim 128): T new tokens per
// sequence attend the ring as it was before the chunk plus the chunk itself,
// causally, each with its own window; then the chunk is appended.
struct RotateChunkParams {
  const void* q;          // [B, T, Hq, d], not rotated
  const void* k;          // [B, T, Hkv, d], not rotated
  const int32_t* pos;     // [B]: position of token 0
  void* q_rot;            // [B, T, Hq, d]
  void* k_rot;            // [B, T, Hkv, d]
  int32_t batch, n_tokens, num_q_heads, num_kv_heads;
  int rope_half;
  RopeFreq freq;
};

struct PrefillParams {
  const void* q_rot;          // [B, T, Hq, d] bf16, rotated
  const void* k_rot;          // [B, T, Hkv, d] bf16, rotated
  const void* v_new;          // [B, T, Hkv, d] bf16
  const void* k_cache;        // [B, Hkv, slots, d]: the ring before the chunk
  const void* v_cache;
  const int32_t* slot_pos;    // [B, slots]
  const int32_t* pos;         // [B]: position of token 0
  int32_t batch, n_tokens, num_q_heads, num_kv_heads, slots, sinks, window;
  int32_t token_blocks;       // workgroups per (sequence, kv head)
  float score_scale_log2;
  void* out;                  // [B, T, Hq, d] f32 or bf16
  float* lse;                 // [B, T, Hq] or null
  int out_bf16;
};

// Workspace of a prefill call: rotated queries, then rotated K rows.
struct PrefillLayout {
  size_t q_offset, k_offset, total;
};
PrefillLayout prefill_layout(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t n_tokens);
// Tokens of one attention workgroup for a group of g = Hq / Hkv query heads.
int prefill_tokens_per_block(int group);
hipError_t launch_rotate_chunk(const RotateChunkParams& p, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);

// Block manager (refcounted blocks, prefix sharing, copy-on-write): updates
// of the device block table and lengths and copy-on-write block copies, by
// value; then the new tokens' rows, found through the updated table.
constexpr int kBlocksMaxTable = 160;  // block-table entries per update launch
constexpr int kBlocksMaxLens = 32;    // length entries per update launch
constexpr int kBlocksMaxCow = 16;     // copy-on-write copies per update launch
struct BlocksUpdateParams {
  int32_t* block_table;   // [max_seqs, max_blocks]
  int32_t* seq_lens;      // [max_seqs]
  void* k_pool;           // [Nphys, Hkv, bs, d]
  void* v_pool;
  int32_t num_kv_heads, block_size, head_dim, elem_bytes;
  int32_t n_table, n_lens, n_cow;
  int32_t table_idx[kBlocksMaxTable];
  int32_t table_val[kBlocksMaxTable];
  int32_t lens_idx[kBlocksMaxLens];
  int32_t lens_val[kBlocksMaxLens];
  int32_t cow_src[kBlocksMaxCow];   // physical block copied from
  int32_t cow_dst[kBlocksMaxCow];   // physical block copied to
  int32_t cow_rows[kBlocksMaxCow];  // rows 0 .. rows-1 of every head
};
constexpr int kAppendMaxSeqs = 128;  // sequences per paged-append launch
struct AppendPagedParams {
  const void* k_src;          // [n_all, n_tokens, Hkv, d]: rows of every listed sequence
  const void* v_src;
  void* k_pool;
  void* v_pool;
  const int32_t* block_table; // [max_seqs, max_blocks], device
  int32_t src_first;          // index of this launch's first sequence in k_src / v_src
  int32_t n_seqs, n_tokens;
  int32_t num_kv_heads, head_dim, block_shift, max_blocks, num_phys_blocks;
  int32_t rotate, rope_half, bf16;
  int32_t seqs[kAppendMaxSeqs];       // sequence of each listed row group
  int32_t first_pos[kAppendMaxSeqs];  // its length before the call
  RopeFreq freq;
};
hipError_t launch_blocks_update(const BlocksUpdateParams& p, hipStream_t stream);
hipError_t launch_append_paged(const AppendPagedParams& p, hipStream_t stream);

// Host-pool pager: block copies from pinned host memory, validity updates.
// The lists travel by value in the kernel arguments, so nothing is staged in
// memory that a later call could overwrite before the kernel runs.
constexpr int kPagerMaxCopies = 224;  // blocks per copy launch
constexpr int kPagerMaxValid = 448;   // validity updates per launch
constexpr int32_t kPagerCopyPieceU4 = 512;  // 16-byte units per copy workgroup (8 KiB)
struct PagerCopyParams {
  const void* host_k;   // device view of the pinned host store [B * L blocks]
  const void* host_v;
  void* k_pool;         // [num_phys_blocks blocks]
  void* v_pool;
  int32_t block_u4;     // 16-byte units per block of K (or V)
  int32_t piece_u4;     // 16-byte units per workgroup
  int32_t pieces;       // workgroups per block and tensor
  int32_t n;            // blocks in this launch
  int32_t src_block[kPagerMaxCopies];  // b * L + logical block
  int32_t dst_block[kPagerMaxCopies];  // physical pool block
};
struct PagerValidParams {
  uint8_t* valid;       // [B * C]
  int32_t n;
  int32_t entries[kPagerMaxValid];  // e >= 0: valid[e] = 1; e < 0: valid[-1 - e] = 0
};
// A paging step folded into the paged decode ([pool] section on copies
// overlapped with the attention), in two parts.  Fetch: workgroups added to
// the attention launch copy block src_block[i] (b * L + logical block) of the
// host store into staging block i while the attention reads the pool (the
// staging area is not part of the pool, so nothing the attention reads
// changes).  Place: workgroups added to the merge launch, which starts after
// the attention kernel has read the pool, move staging block i into pool
// block dst_block[i] and set the validity byte slot[i] (b * C + slot); so a
// slot may be overwritten even if this step's attention read its old block.
constexpr int kPagerFuseMax = 64;  // blocks per fused step (more: separate launches after)
static_assert(kPagerFuseMax <= kPagerMaxCopies && kPagerFuseMax <= kPagerMaxValid,
              "a fused step fits one copy and one validity launch");
struct PagerFuse {
  const void* host_k;   // device views of the pinned host store
  const void* host_v;
  void* stage_k;        // [n blocks] of K, then of V: device memory the attention does not read
  void* stage_v;
  void* k_pool;
  void* v_pool;
  uint8_t* valid;       // [B * C]
  int32_t block_u4;     // 16-byte units per block of K (or V)
  int32_t n;            // blocks (0: nothing to copy)
  int32_t src_block[kPagerFuseMax];
  int32_t dst_block[kPagerFuseMax];
  int32_t slot[kPagerFuseMax];
};
hipError_t launch_pager_copy(const PagerCopyParams& p, hipStream_t stream);
hipError_t launch_pager_valid(const PagerValidParams& p, hipStream_t stream);
hipError_t launch_fill_u8(uint8_t* dst, size_t n, uint8_t value, hipStream_t stream);

// The calling thread's error text (swa_last_error), set by every C-ABI source.
int record_error(int code, const char* text);
void clear_error();

}  // namespace swa
