// Host-pool pager ([pool] "paging"): every block of a sequence's history
// lives in pinned host memory; a fixed pool of device slots holds the blocks
// the attention needs, each slot with a validity byte that decode_attn_paged
// reads.  The residency policy is LRU ([pool] "residency policy": evict the
// block used longest ago).  The copies overlap the attention ([pool]: copies
// run beside the attention kernel): swa_pager_stage + swa_pager_decode fold
// them into the decode's own launches (fetched from the host store into a
// staging area of the workspace by workgroups of their own during the
// attention, placed into the pool by the merge launch after it); with
// swa_pager_advance they run as a launch of their own, on the attention
// stream or a stream of their own.
//
// State per sequence b (host only):
//   slot_block[b][j]  logical block in slot j, or -1
//   where[b][k]       slot of logical block k, or -1
//   last_use[b][k]    index of the last request that named block k
// A block is protected (never a victim) when the current request names it or
// the previous one did (last_use == clock - 1): the attention step that the
// previous request prepared is enqueued after this call and must still find
// every block it named.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <new>
#include <utility>
#include <vector>

#include "swa.h"
#include "swa_internal.h"

namespace swa {
// decode_attn_paged with a paging step run after the attention (swa_api.cpp).
swa_status paged_decode_with_copies(const swa_paged_desc* desc, const void* q, const void* k_pool,
                                    const void* v_pool, const int32_t* block_table,
                                    const int32_t* seq_lens, const uint8_t* block_valid,
                                    float scale, void* out, swa_dtype out_dtype, float* lse,
                                    void* workspace, size_t workspace_bytes, void* stream,
                                    const PagerFuse* fuse);
}  // namespace swa

// A block to bring in: host store block b * L + k, pool block, slot b * C + j.
struct PagerLoad {
  int32_t src;
  int32_t dst;
  int32_t slot;
};

struct swa_pager {
  swa_pager_config cfg;
  const void* host_k;  // device views of the pinned host store
  const void* host_v;
  void* k_pool;
  void* v_pool;
  int32_t* block_table;
  uint8_t* block_valid;
  std::vector<int32_t> slot_phys;   // [B * C]
  std::vector<int32_t> slot_block;  // [B * C]
  std::vector<int32_t> where;       // [B * L]
  std::vector<int64_t> last_use;    // [B * L]
  std::vector<int64_t> mark;        // [B * L] request stamp (dedup, membership)
  std::vector<int32_t> pending;     // global slots copied by the last advance, not yet valid
  std::vector<PagerLoad> staged;    // loads of the last swa_pager_stage, not yet launched
  int64_t clock = 1;                // index of the next request
  int64_t stamp = 0;
  size_t block_bytes = 0;           // bytes of one block of K (or V)
  hipEvent_t released = nullptr;    // on the attention stream: earlier reads done, victims cleared
  hipEvent_t copied = nullptr;      // on the copy stream: the last advance's copies done
  hipStream_t pending_stream = nullptr;  // the stream the pending copies run on
};

namespace {

swa_status fail(swa_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  return static_cast<swa_status>(swa::record_error(code, buf));
}

swa_status ok() {
  swa::clear_error();
  return SWA_OK;
}

swa_status from_hip(hipError_t err, const char* what) {
  if (err == hipSuccess) return ok();
  return fail(SWA_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool power_of_two_in(int32_t x, int32_t lo, int32_t hi) {
  return x >= lo && x <= hi && (x & (x - 1)) == 0;
}

swa_status check_config(const swa_pager_config* c) {
  if (c == nullptr) return fail(SWA_ERR_INVALID_ARG, "config is NULL");
  if (c->batch < 1 || c->num_kv_heads < 1 || c->logical_blocks < 1 || c->slots_per_seq < 1 ||
      c->num_phys_blocks < 1)
    return fail(SWA_ERR_INVALID_ARG, "batch, num_kv_heads, logical_blocks, slots_per_seq and "
                                     "num_phys_blocks must be >= 1");
  if (c->dtype == SWA_I8) return fail(SWA_ERR_UNSUPPORTED, "the pager moves f32 or bf16 blocks");
  if (c->dtype != SWA_F32 && c->dtype != SWA_BF16)
    return fail(SWA_ERR_INVALID_ARG, "unknown dtype %d", c->dtype);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(SWA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", c->head_dim);
  if (!power_of_two_in(c->block_size, 16, 1024))
    return fail(SWA_ERR_UNSUPPORTED, "block_size %d must be a power of two in [16, 1024]",
                c->block_size);
  if (static_cast<int64_t>(c->batch) * c->logical_blocks > INT32_MAX ||
      static_cast<int64_t>(c->batch) * c->slots_per_seq > INT32_MAX ||
      static_cast<int64_t>(c->slots_per_seq) * c->block_size > INT32_MAX ||
      static_cast<int64_t>(c->num_phys_blocks) * c->block_size > INT32_MAX)
    return fail(SWA_ERR_INVALID_ARG, "pager too large for 32-bit block and token indices");
  const int64_t block_u4 =
      static_cast<int64_t>(c->num_kv_heads) * c->block_size * c->head_dim *
      (c->dtype == SWA_BF16 ? 2 : 4) / 16;
  if (block_u4 > INT32_MAX / 2)
    return fail(SWA_ERR_INVALID_ARG, "block too large");
  return SWA_OK;
}

// One or more validity launches for a list of entries.
hipError_t launch_valid(uint8_t* valid, const std::vector<int32_t>& entries, hipStream_t s) {
  swa::PagerValidParams p{};
  p.valid = valid;
  for (size_t i = 0; i < entries.size(); i += swa::kPagerMaxValid) {
    const size_t n = std::min(entries.size() - i, static_cast<size_t>(swa::kPagerMaxValid));
    p.n = static_cast<int32_t>(n);
    std::copy(entries.begin() + i, entries.begin() + i + n, p.entries);
    const hipError_t err = swa::launch_pager_valid(p, s);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

// 16-byte units each copy workgroup moves: 8 KiB.
int32_t copy_piece_u4(const swa_pager* pg) {
  return std::min<int32_t>(static_cast<int32_t>(pg->block_bytes / 16), swa::kPagerCopyPieceU4);
}

hipError_t launch_copies(const swa_pager* pg, const std::vector<PagerLoad>& loads, hipStream_t s) {
  swa::PagerCopyParams p{};
  p.host_k = pg->host_k;
  p.host_v = pg->host_v;
  p.k_pool = pg->k_pool;
  p.v_pool = pg->v_pool;
  p.block_u4 = static_cast<int32_t>(pg->block_bytes / 16);
  p.piece_u4 = copy_piece_u4(pg);
  p.pieces = (p.block_u4 + p.piece_u4 - 1) / p.piece_u4;
  for (size_t i = 0; i < loads.size(); i += swa::kPagerMaxCopies) {
    const size_t n = std::min(loads.size() - i, static_cast<size_t>(swa::kPagerMaxCopies));
    p.n = static_cast<int32_t>(n);
    for (size_t j = 0; j < n; ++j) {
      p.src_block[j] = loads[i + j].src;
      p.dst_block[j] = loads[i + j].dst;
    }
    const hipError_t err = swa::launch_pager_copy(p, s);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

// Staging area of a fused step, at the end of the decode's workspace: K
// blocks, then as many V blocks; at most kStageBudget bytes, so a step with
// more (or larger) blocks runs its copies as separate launches instead.
constexpr size_t kStageBudget = size_t{16} << 20;
constexpr size_t kStageAlign = 256;

int32_t stage_blocks(const swa_pager* pg) {
  return static_cast<int32_t>(
      std::min<size_t>(swa::kPagerFuseMax, kStageBudget / (2 * pg->block_bytes)));
}

// Bytes swa_pager_decode needs: the decode's workspace for the pool, then the
// staging area.  Returns the offset of the staging area in *stage_at.
swa_status pager_workspace(const swa_pager* pg, int32_t num_q_heads, size_t* bytes,
                           size_t* stage_at) {
  const swa_pager_config& c = pg->cfg;
  size_t dec = 0;
  const swa_status st = decode_attn_workspace_bytes(c.batch, num_q_heads, c.num_kv_heads,
                                                    c.head_dim, c.slots_per_seq * c.block_size,
                                                    &dec);
  if (st != SWA_OK) return st;
  *stage_at = (dec + kStageAlign - 1) / kStageAlign * kStageAlign;
  *bytes = *stage_at + 2 * static_cast<size_t>(stage_blocks(pg)) * pg->block_bytes;
  return SWA_OK;
}

// The copies of a staged step and their validity bytes, as separate launches.
hipError_t launch_staged(const swa_pager* pg, hipStream_t s) {
  std::vector<int32_t> entries;
  for (const PagerLoad& l : pg->staged) entries.push_back(l.slot);
  hipError_t err = launch_copies(pg, pg->staged, s);
  return err != hipSuccess ? err : launch_valid(pg->block_valid, entries, s);
}

}  // namespace

extern "C" {

swa_status swa_pager_create(const swa_pager_config* cfg, const void* host_k, const void* host_v,
                            void* k_pool, void* v_pool, const int32_t* slot_phys,
                            int32_t* block_table, uint8_t* block_valid, swa_pager** out) {
  swa_status st = check_config(cfg);
  if (st != SWA_OK) return st;
  if (out == nullptr) return fail(SWA_ERR_INVALID_ARG, "out is NULL");
  if (host_k == nullptr || host_v == nullptr || k_pool == nullptr || v_pool == nullptr ||
      slot_phys == nullptr || block_table == nullptr || block_valid == nullptr)
    return fail(SWA_ERR_INVALID_ARG, "host store, pool, slot_phys, block_table and block_valid "
                                     "must not be NULL");
  if (!aligned(host_k, 16) || !aligned(host_v, 16) || !aligned(k_pool, 16) ||
      !aligned(v_pool, 16) || !aligned(block_table, 4))
    return fail(SWA_ERR_INVALID_ARG, "host store and pool must be 16-byte aligned");
  const size_t slots = static_cast<size_t>(cfg->batch) * cfg->slots_per_seq;
  std::vector<uint8_t> used(static_cast<size_t>(cfg->num_phys_blocks), 0);
  for (size_t i = 0; i < slots; ++i) {
    const int32_t ph = slot_phys[i];
    if (ph < 0 || ph >= cfg->num_phys_blocks)
      return fail(SWA_ERR_INVALID_ARG, "slot_phys[%zu] = %d outside [0, %d)", i, ph,
                  cfg->num_phys_blocks);
    if (used[ph]) return fail(SWA_ERR_INVALID_ARG, "pool block %d named by two slots", ph);
    used[ph] = 1;
  }
  void* dk = nullptr;
  void* dv = nullptr;
  if (hipHostGetDevicePointer(&dk, const_cast<void*>(host_k), 0) != hipSuccess ||
      hipHostGetDevicePointer(&dv, const_cast<void*>(host_v), 0) != hipSuccess || dk == nullptr ||
      dv == nullptr) {
    (void)hipGetLastError();
    return fail(SWA_ERR_INVALID_ARG, "host_k / host_v must be pinned host memory the device "
                                     "can read (hipHostMalloc or pin_memory)");
  }
  swa_pager* pg = new (std::nothrow) swa_pager;
  if (pg == nullptr) return fail(SWA_ERR_INVALID_ARG, "out of host memory");
  try {
    pg->slot_phys.assign(slot_phys, slot_phys + slots);
    pg->slot_block.assign(slots, -1);
    const size_t blocks = static_cast<size_t>(cfg->batch) * cfg->logical_blocks;
    pg->where.assign(blocks, -1);
    pg->last_use.assign(blocks, -1);
    pg->mark.assign(blocks, -1);
  } catch (const std::bad_alloc&) {
    delete pg;
    return fail(SWA_ERR_INVALID_ARG, "out of host memory");
  }
  pg->cfg = *cfg;
  pg->host_k = dk;
  pg->host_v = dv;
  pg->k_pool = k_pool;
  pg->v_pool = v_pool;
  pg->block_table = block_table;
  pg->block_valid = block_valid;
  pg->block_bytes = static_cast<size_t>(cfg->num_kv_heads) * cfg->block_size * cfg->head_dim *
                    (cfg->dtype == SWA_BF16 ? 2 : 4);
  hipError_t err = hipEventCreateWithFlags(&pg->released, hipEventDisableTiming);
  if (err == hipSuccess) err = hipEventCreateWithFlags(&pg->copied, hipEventDisableTiming);
  if (err != hipSuccess) {
    swa_pager_destroy(pg);
    return from_hip(err, "swa_pager_create");
  }
  *out = pg;
  return ok();
}

swa_status swa_pager_reset(swa_pager* pg, void* stream) {
  if (pg == nullptr) return fail(SWA_ERR_INVALID_ARG, "pager is NULL");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err = hipSuccess;
  if (!pg->pending.empty() && pg->pending_stream != s) err = hipStreamWaitEvent(s, pg->copied, 0);
  const size_t slots = pg->slot_phys.size();
  if (err == hipSuccess)
    err = hipMemcpyAsync(pg->block_table, pg->slot_phys.data(), slots * sizeof(int32_t),
                         hipMemcpyHostToDevice, s);
  if (err == hipSuccess) err = swa::launch_fill_u8(pg->block_valid, slots, 0, s);
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  if (err != hipSuccess) return from_hip(err, "swa_pager_reset");
  std::fill(pg->slot_block.begin(), pg->slot_block.end(), -1);
  std::fill(pg->where.begin(), pg->where.end(), -1);
  std::fill(pg->last_use.begin(), pg->last_use.end(), -1);
  std::fill(pg->mark.begin(), pg->mark.end(), -1);
  pg->pending.clear();
  pg->staged.clear();
  pg->clock = 1;
  pg->stamp = 0;
  return ok();
}

}  // extern "C"

namespace {

// Serves one request on the host state (LRU, the rules of
// swa_pager_advance): checks it, then lists the blocks to bring in and the
// slots whose block is evicted, in order.  A refused request changes nothing.
swa_status serve_request(swa_pager* pg, const int32_t* req_offsets, const int32_t* req_blocks,
                         std::vector<PagerLoad>& loads, std::vector<int32_t>& evicted,
                         const char* name) {
  if (pg == nullptr) return fail(SWA_ERR_INVALID_ARG, "%s: pager is NULL", name);
  if (req_offsets == nullptr) return fail(SWA_ERR_INVALID_ARG, "%s: req_offsets is NULL", name);
  const swa_pager_config& c = pg->cfg;
  const int32_t B = c.batch, C = c.slots_per_seq, L = c.logical_blocks;
  if (req_offsets[0] != 0) return fail(SWA_ERR_INVALID_ARG, "req_offsets[0] must be 0");
  for (int32_t b = 0; b < B; ++b)
    if (req_offsets[b + 1] < req_offsets[b])
      return fail(SWA_ERR_INVALID_ARG, "req_offsets must be non-decreasing");
  if (req_offsets[B] > 0 && req_blocks == nullptr)
    return fail(SWA_ERR_INVALID_ARG, "req_blocks is NULL");
  for (int32_t i = 0; i < req_offsets[B]; ++i)
    if (req_blocks[i] < 0 || req_blocks[i] >= L)
      return fail(SWA_ERR_INVALID_ARG, "req_blocks[%d] = %d outside [0, %d)", i, req_blocks[i], L);

  // Feasibility first, without touching the state: per sequence, the missing
  // blocks must fit in the empty slots plus the unprotected resident ones.
  const int64_t stamp = ++pg->stamp;
  for (int32_t b = 0; b < B; ++b) {
    int64_t* mark = pg->mark.data() + static_cast<size_t>(b) * L;
    const int64_t* last = pg->last_use.data() + static_cast<size_t>(b) * L;
    const int32_t* where = pg->where.data() + static_cast<size_t>(b) * L;
    const int32_t* held = pg->slot_block.data() + static_cast<size_t>(b) * C;
    int64_t missing = 0;
    for (int32_t i = req_offsets[b]; i < req_offsets[b + 1]; ++i) {
      const int32_t k = req_blocks[i];
      if (mark[k] == stamp) continue;
      mark[k] = stamp;
      if (where[k] < 0) ++missing;
    }
    int64_t room = 0;
    for (int32_t j = 0; j < C; ++j) {
      const int32_t k = held[j];
      if (k < 0 || (mark[k] != stamp && last[k] < pg->clock - 1)) ++room;
    }
    if (missing > room)
      return fail(SWA_ERR_INVALID_ARG,
                  "sequence %d: %lld blocks missing but only %lld slots are empty or hold a "
                  "block named by neither this request nor the previous one",
                  b, static_cast<long long>(missing), static_cast<long long>(room));
  }

  // Apply: choose slots, update the host state, list the device work.
  std::vector<std::pair<int64_t, int32_t>> cand;  // (last use, slot) of evictable blocks
  for (int32_t b = 0; b < B; ++b) {
    const size_t bl = static_cast<size_t>(b) * L;
    const size_t bc = static_cast<size_t>(b) * C;
    int64_t* mark = pg->mark.data() + bl;
    int64_t* last = pg->last_use.data() + bl;
    int32_t* where = pg->where.data() + bl;
    int32_t* held = pg->slot_block.data() + bc;
    // mark[] == stamp flags this request's blocks (set by the feasibility
    // pass); membership is read before their last_use moves to the clock.
    cand.clear();
    std::vector<int32_t> free_slots;
    for (int32_t j = 0; j < C; ++j) {
      const int32_t k = held[j];
      if (k < 0)
        free_slots.push_back(j);
      else if (mark[k] != stamp && last[k] < pg->clock - 1)
        cand.emplace_back(last[k], j);
    }
    int32_t missing = 0;
    for (int32_t i = req_offsets[b]; i < req_offsets[b + 1]; ++i)
      if (where[req_blocks[i]] == -1) {
        where[req_blocks[i]] = -2;  // missing: counted once (repeats see -2), assigned below
        ++missing;
      }
    const int32_t evict = std::max<int32_t>(0, missing - static_cast<int32_t>(free_slots.size()));
    if (evict > 0) {
      std::partial_sort(cand.begin(), cand.begin() + evict, cand.end());
    }
    size_t next_free = 0, next_victim = 0;
    for (int32_t i = req_offsets[b]; i < req_offsets[b + 1]; ++i) {
      const int32_t k = req_blocks[i];
      if (where[k] != -2) continue;
      int32_t j;
      if (next_free < free_slots.size()) {
        j = free_slots[next_free++];
      } else {
        j = cand[next_victim++].second;
        const int32_t old = held[j];
        where[old] = -1;
        evicted.push_back(static_cast<int32_t>(bc + j));
      }
      held[j] = k;
      where[k] = j;
      loads.push_back({static_cast<int32_t>(bl + k), pg->slot_phys[bc + j],
                       static_cast<int32_t>(bc + j)});
    }
    for (int32_t i = req_offsets[b]; i < req_offsets[b + 1]; ++i) last[req_blocks[i]] = pg->clock;
  }
  pg->clock += 1;
  return SWA_OK;
}

}  // namespace

extern "C" {

swa_status swa_pager_advance(swa_pager* pg, const int32_t* req_offsets, const int32_t* req_blocks,
                             void* stream, void* copy_stream, int32_t* n_loaded) {
  if (pg != nullptr && !pg->staged.empty())
    return fail(SWA_ERR_INVALID_ARG, "swa_pager_advance: the blocks of the last swa_pager_stage "
                                     "are not copied yet (call swa_pager_decode or "
                                     "swa_pager_commit first)");
  std::vector<PagerLoad> loads;
  std::vector<int32_t> evicted;
  swa_status st = serve_request(pg, req_offsets, req_blocks, loads, evicted, "swa_pager_advance");
  if (st != SWA_OK) return st;

  // Device work: the previous copies become valid and this call's victims
  // invalid (cleared before the copies land) on the attention stream; the
  // new copies start on the copy stream after everything enqueued on the
  // attention stream so far.
  std::vector<int32_t> entries(pg->pending);
  for (int32_t slot : evicted) entries.push_back(-1 - slot);
  std::vector<int32_t> new_pending;
  for (const PagerLoad& l : loads) new_pending.push_back(l.slot);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipStream_t cs = static_cast<hipStream_t>(copy_stream);
  // With one stream for both, stream order alone does it: no event is waited
  // on (a wait across streams costs the host ~16 us here).  The copies'
  // event is still recorded, for a later call on another stream.
  hipError_t err = hipSuccess;
  if (!pg->pending.empty() && pg->pending_stream != s) err = hipStreamWaitEvent(s, pg->copied, 0);
  if (err == hipSuccess && !entries.empty()) err = launch_valid(pg->block_valid, entries, s);
  if (err == hipSuccess && !loads.empty()) {
    if (cs != s) {
      err = hipEventRecord(pg->released, s);
      if (err == hipSuccess) err = hipStreamWaitEvent(cs, pg->released, 0);
    }
    if (err == hipSuccess) err = launch_copies(pg, loads, cs);
    if (err == hipSuccess) err = hipEventRecord(pg->copied, cs);
  }
  pg->pending_stream = cs;
  pg->pending.swap(new_pending);
  if (n_loaded != nullptr) *n_loaded = static_cast<int32_t>(loads.size());
  return from_hip(err, "swa_pager_advance");
}

swa_status swa_pager_stage(swa_pager* pg, const int32_t* req_offsets, const int32_t* req_blocks,
                           int32_t* n_loaded) {
  if (pg != nullptr && !pg->staged.empty())
    return fail(SWA_ERR_INVALID_ARG, "swa_pager_stage: the blocks of the last swa_pager_stage "
                                     "are not copied yet (call swa_pager_decode or "
                                     "swa_pager_commit first)");
  if (pg != nullptr && !pg->pending.empty())
    return fail(SWA_ERR_INVALID_ARG, "swa_pager_stage: the copies of the last swa_pager_advance "
                                     "are not visible yet (call swa_pager_commit first)");
  std::vector<PagerLoad> loads;
  std::vector<int32_t> evicted;  // overwritten in place after the attention: nothing to clear
  swa_status st = serve_request(pg, req_offsets, req_blocks, loads, evicted, "swa_pager_stage");
  if (st != SWA_OK) return st;
  pg->staged.swap(loads);
  if (n_loaded != nullptr) *n_loaded = static_cast<int32_t>(pg->staged.size());
  return ok();
}

swa_status swa_pager_decode(swa_pager* pg, const void* q, int32_t num_q_heads,
                            const int32_t* seq_lens, float scale, void* out, swa_dtype out_dtype,
                            float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (pg == nullptr) return fail(SWA_ERR_INVALID_ARG, "swa_pager_decode: pager is NULL");
  if (!pg->pending.empty())
    return fail(SWA_ERR_INVALID_ARG, "swa_pager_decode: the copies of the last "
                                     "swa_pager_advance are not visible yet (call "
                                     "swa_pager_commit first)");
  const swa_pager_config& c = pg->cfg;
  size_t need = 0, stage_at = 0;
  swa_status st = pager_workspace(pg, num_q_heads, &need, &stage_at);
  if (st != SWA_OK) return st;
  if (workspace_bytes < need)
    return fail(SWA_ERR_WORKSPACE, "swa_pager_decode: workspace too small: %zu bytes given, "
                                   "%zu needed (swa_pager_workspace_bytes)", workspace_bytes, need);
  swa_paged_desc d{};
  d.batch = c.batch;
  d.num_q_heads = num_q_heads;
  d.num_kv_heads = c.num_kv_heads;
  d.head_dim = c.head_dim;
  d.block_size = c.block_size;
  d.max_blocks_per_seq = c.slots_per_seq;
  d.num_phys_blocks = c.num_phys_blocks;
  d.dtype = c.dtype;
  // The staged copies run in the decode's launches when they fit the staging
  // area; otherwise as separate launches after the decode (the same order).
  const bool fused = !pg->staged.empty() &&
                     pg->staged.size() <= static_cast<size_t>(stage_blocks(pg));
  swa::PagerFuse f{};
  if (fused) {
    char* stage = static_cast<char*>(workspace) + stage_at;
    f.host_k = pg->host_k;
    f.host_v = pg->host_v;
    f.stage_k = stage;
    f.stage_v = stage + static_cast<size_t>(stage_blocks(pg)) * pg->block_bytes;
    f.k_pool = pg->k_pool;
    f.v_pool = pg->v_pool;
    f.valid = pg->block_valid;
    f.block_u4 = static_cast<int32_t>(pg->block_bytes / 16);
    f.n = static_cast<int32_t>(pg->staged.size());
    for (int32_t i = 0; i < f.n; ++i) {
      f.src_block[i] = pg->staged[i].src;
      f.dst_block[i] = pg->staged[i].dst;
      f.slot[i] = pg->staged[i].slot;
    }
  }
  st = swa::paged_decode_with_copies(
      &d, q, pg->k_pool, pg->v_pool, pg->block_table, seq_lens, pg->block_valid, scale, out,
      out_dtype, lse, workspace, workspace_bytes, stream, fused ? &f : nullptr);
  if (st != SWA_OK) return st;  // an argument error launched nothing: the stage still stands
  hipError_t err = hipSuccess;
  if (!fused && !pg->staged.empty()) err = launch_staged(pg, static_cast<hipStream_t>(stream));
  pg->staged.clear();
  return from_hip(err, "swa_pager_decode");
}

swa_status swa_pager_workspace_bytes(const swa_pager* pg, int32_t num_q_heads, size_t* bytes) {
  if (pg == nullptr || bytes == nullptr)
    return fail(SWA_ERR_INVALID_ARG, "swa_pager_workspace_bytes: pager or bytes is NULL");
  size_t stage_at = 0;
  const swa_status st = pager_workspace(pg, num_q_heads, bytes, &stage_at);
  return st != SWA_OK ? st : ok();
}

swa_status swa_pager_commit(swa_pager* pg, void* stream) {
  if (pg == nullptr) return fail(SWA_ERR_INVALID_ARG, "pager is NULL");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (!pg->staged.empty()) {  // a stage not yet decoded: its copies now, no attention
    const hipError_t err = launch_staged(pg, s);
    pg->staged.clear();
    if (err != hipSuccess) return from_hip(err, "swa_pager_commit");
  }
  if (pg->pending.empty()) return ok();
  hipError_t err = pg->pending_stream != s ? hipStreamWaitEvent(s, pg->copied, 0) : hipSuccess;
  if (err == hipSuccess) err = launch_valid(pg->block_valid, pg->pending, s);
  pg->pending.clear();
  return from_hip(err, "swa_pager_commit");
}

swa_status swa_pager_slot_blocks(const swa_pager* pg, int32_t seq, int32_t* out) {
  if (pg == nullptr || out == nullptr) return fail(SWA_ERR_INVALID_ARG, "pager or out is NULL");
  if (seq < 0 || seq >= pg->cfg.batch)
    return fail(SWA_ERR_INVALID_ARG, "seq %d outside [0, %d)", seq, pg->cfg.batch);
  const int32_t C = pg->cfg.slots_per_seq;
  std::copy_n(pg->slot_block.begin() + static_cast<size_t>(seq) * C, C, out);
  return ok();
}

void swa_pager_destroy(swa_pager* pg) {
  if (pg == nullptr) return;
  if (pg->released != nullptr) (void)hipEventDestroy(pg->released);
  if (pg->copied != nullptr) (void)hipEventDestroy(pg->copied);
  delete pg;
}

}  // extern "C"
