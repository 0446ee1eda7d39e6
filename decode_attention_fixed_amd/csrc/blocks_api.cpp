// Block manager for a paged KV pool ([share] §3.1-§3.2, §5.1, §6.1): fixed
// blocks, a block table per sequence, reference counts so that sequences
// with a common prefix share physical blocks, copy-on-write before a write
// into a shared block, and release only when no sequence references a
// block.  The host keeps the authoritative state; every change is mirrored
// into the caller's device block table and length array by small launches on
// the caller's stream, so decode_attn_paged on that stream sees it.
//
// Allocation takes the lowest-numbered free block (a min-heap), so the
// mapping is unique for a given order of operations.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <functional>
#include <new>
#include <queue>
#include <vector>

#include "swa.h"
#include "swa_internal.h"

struct swa_blocks {
  int32_t num_blocks = 0, block_size = 0, max_seqs = 0, max_blocks = 0;
  std::vector<int32_t> ref;    // [num_blocks] sequences referencing each block
  std::vector<int32_t> table;  // [max_seqs * max_blocks] physical block, -1 = none
  std::vector<int32_t> lens;   // [max_seqs] tokens
  std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>> free_q;
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

int32_t blocks_for(int64_t tokens, int32_t bs) { return static_cast<int32_t>((tokens + bs - 1) / bs); }

void reset_state(swa_blocks* m) {
  m->ref.assign(static_cast<size_t>(m->num_blocks), 0);
  m->table.assign(static_cast<size_t>(m->max_seqs) * m->max_blocks, -1);
  m->lens.assign(static_cast<size_t>(m->max_seqs), 0);
  m->free_q = {};
  for (int32_t b = 0; b < m->num_blocks; ++b) m->free_q.push(b);
}

int32_t take_block(swa_blocks* m) {
  const int32_t b = m->free_q.top();
  m->free_q.pop();
  m->ref[b] = 1;
  return b;
}

// Device-side updates collected while the host state changes; flushed in
// launches of bounded size (the lists travel in the kernel arguments).
struct Updates {
  std::vector<int32_t> table_idx, table_val, lens_idx, lens_val, cow_src, cow_dst, cow_rows;
};

hipError_t flush(const Updates& u, int32_t* block_table, int32_t* seq_lens, void* k_pool,
                 void* v_pool, int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                 int32_t elem_bytes, hipStream_t s) {
  size_t it = 0, il = 0, ic = 0;
  while (it < u.table_idx.size() || il < u.lens_idx.size() || ic < u.cow_src.size()) {
    swa::BlocksUpdateParams p{};
    p.block_table = block_table;
    p.seq_lens = seq_lens;
    p.k_pool = k_pool;
    p.v_pool = v_pool;
    p.num_kv_heads = num_kv_heads;
    p.block_size = block_size;
    p.head_dim = head_dim;
    p.elem_bytes = elem_bytes;
    for (; it < u.table_idx.size() && p.n_table < swa::kBlocksMaxTable; ++it, ++p.n_table) {
      p.table_idx[p.n_table] = u.table_idx[it];
      p.table_val[p.n_table] = u.table_val[it];
    }
    for (; il < u.lens_idx.size() && p.n_lens < swa::kBlocksMaxLens; ++il, ++p.n_lens) {
      p.lens_idx[p.n_lens] = u.lens_idx[il];
      p.lens_val[p.n_lens] = u.lens_val[il];
    }
    for (; ic < u.cow_src.size() && p.n_cow < swa::kBlocksMaxCow; ++ic, ++p.n_cow) {
      p.cow_src[p.n_cow] = u.cow_src[ic];
      p.cow_dst[p.n_cow] = u.cow_dst[ic];
      p.cow_rows[p.n_cow] = u.cow_rows[ic];
    }
    const hipError_t err = swa::launch_blocks_update(p, s);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

swa_status check_seq(const swa_blocks* m, int32_t seq, const char* what) {
  if (seq < 0 || seq >= m->max_seqs)
    return fail(SWA_ERR_INVALID_ARG, "%s: sequence %d outside [0, %d)", what, seq, m->max_seqs);
  return SWA_OK;
}

}  // namespace

extern "C" {

swa_status swa_blocks_create(int32_t num_blocks, int32_t block_size, int32_t max_seqs,
                             int32_t max_blocks_per_seq, swa_blocks** out) {
  if (out == nullptr) return fail(SWA_ERR_INVALID_ARG, "out is NULL");
  if (num_blocks < 1 || max_seqs < 1 || max_blocks_per_seq < 1)
    return fail(SWA_ERR_INVALID_ARG, "num_blocks, max_seqs, max_blocks_per_seq must be >= 1");
  if (block_size < 16 || block_size > 1024 || (block_size & (block_size - 1)) != 0)
    return fail(SWA_ERR_UNSUPPORTED, "block_size %d must be a power of two in [16, 1024]",
                block_size);
  if (static_cast<int64_t>(max_seqs) * max_blocks_per_seq > INT32_MAX ||
      static_cast<int64_t>(max_blocks_per_seq) * block_size > INT32_MAX ||
      static_cast<int64_t>(num_blocks) * block_size > INT32_MAX)
    return fail(SWA_ERR_INVALID_ARG, "too large for 32-bit block and token indices");
  swa_blocks* m = new (std::nothrow) swa_blocks;
  if (m == nullptr) return fail(SWA_ERR_INVALID_ARG, "out of host memory");
  m->num_blocks = num_blocks;
  m->block_size = block_size;
  m->max_seqs = max_seqs;
  m->max_blocks = max_blocks_per_seq;
  try {
    reset_state(m);
  } catch (const std::bad_alloc&) {
    delete m;
    return fail(SWA_ERR_INVALID_ARG, "out of host memory");
  }
  *out = m;
  return ok();
}

void swa_blocks_destroy(swa_blocks* m) { delete m; }

swa_status swa_blocks_sync(swa_blocks* m, int32_t* block_table, int32_t* seq_lens, void* stream) {
  if (m == nullptr || block_table == nullptr || seq_lens == nullptr)
    return fail(SWA_ERR_INVALID_ARG, "manager, block_table and seq_lens must not be NULL");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err = hipMemcpyAsync(block_table, m->table.data(), m->table.size() * sizeof(int32_t),
                                  hipMemcpyHostToDevice, s);
  if (err == hipSuccess)
    err = hipMemcpyAsync(seq_lens, m->lens.data(), m->lens.size() * sizeof(int32_t),
                         hipMemcpyHostToDevice, s);
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  return from_hip(err, "swa_blocks_sync");
}

swa_status swa_blocks_reset(swa_blocks* m) {
  if (m == nullptr) return fail(SWA_ERR_INVALID_ARG, "manager is NULL");
  reset_state(m);
  return ok();
}

swa_status swa_blocks_share_prefix(swa_blocks* m, int32_t src, int32_t dst, int32_t prefix_len,
                                   int32_t* block_table, int32_t* seq_lens, void* stream) {
  if (m == nullptr || block_table == nullptr || seq_lens == nullptr)
    return fail(SWA_ERR_INVALID_ARG, "manager, block_table and seq_lens must not be NULL");
  swa_status st = check_seq(m, src, "share_prefix");
  if (st == SWA_OK) st = check_seq(m, dst, "share_prefix");
  if (st != SWA_OK) return st;
  if (src == dst) return fail(SWA_ERR_INVALID_ARG, "share_prefix: src and dst are the same");
  if (m->lens[dst] != 0)
    return fail(SWA_ERR_INVALID_ARG, "share_prefix: sequence %d is not empty", dst);
  if (prefix_len < 0 || prefix_len > m->lens[src])
    return fail(SWA_ERR_INVALID_ARG, "share_prefix: prefix %d outside [0, %d]", prefix_len,
                m->lens[src]);
  const int32_t n = blocks_for(prefix_len, m->block_size);
  Updates u;
  for (int32_t j = 0; j < n; ++j) {
    const int32_t b = m->table[static_cast<size_t>(src) * m->max_blocks + j];
    m->ref[b] += 1;
    m->table[static_cast<size_t>(dst) * m->max_blocks + j] = b;
    u.table_idx.push_back(dst * m->max_blocks + j);
    u.table_val.push_back(b);
  }
  m->lens[dst] = prefix_len;
  u.lens_idx.push_back(dst);
  u.lens_val.push_back(prefix_len);
  return from_hip(flush(u, block_table, seq_lens, nullptr, nullptr, 0, m->block_size, 0, 0,
                        static_cast<hipStream_t>(stream)),
                  "swa_blocks_share_prefix");
}

swa_status swa_blocks_free(swa_blocks* m, int32_t seq, int32_t* seq_lens, void* stream) {
  if (m == nullptr || seq_lens == nullptr)
    return fail(SWA_ERR_INVALID_ARG, "manager and seq_lens must not be NULL");
  swa_status st = check_seq(m, seq, "free");
  if (st != SWA_OK) return st;
  const int32_t n = blocks_for(m->lens[seq], m->block_size);
  for (int32_t j = 0; j < n; ++j) {
    int32_t& e = m->table[static_cast<size_t>(seq) * m->max_blocks + j];
    if (--m->ref[e] == 0) m->free_q.push(e);
    e = -1;
  }
  m->lens[seq] = 0;
  Updates u;
  u.lens_idx.push_back(seq);
  u.lens_val.push_back(0);
  return from_hip(flush(u, nullptr, seq_lens, nullptr, nullptr, 0, m->block_size, 0, 0,
                        static_cast<hipStream_t>(stream)),
                  "swa_blocks_free");
}

swa_status swa_blocks_state(const swa_blocks* m, int32_t* table, int32_t* lens, int32_t* refs,
                            int32_t* free_blocks) {
  if (m == nullptr) return fail(SWA_ERR_INVALID_ARG, "manager is NULL");
  if (table != nullptr) std::copy(m->table.begin(), m->table.end(), table);
  if (lens != nullptr) std::copy(m->lens.begin(), m->lens.end(), lens);
  if (refs != nullptr) std::copy(m->ref.begin(), m->ref.end(), refs);
  if (free_blocks != nullptr) *free_blocks = static_cast<int32_t>(m->free_q.size());
  return ok();
}

swa_status kv_append_paged(swa_blocks* m, const swa_paged_desc* desc, void* k_pool, void* v_pool,
                           int32_t* block_table, int32_t* seq_lens, const int32_t* seqs,
                           int32_t n_seqs, int32_t n_tokens, const void* k_new, const void* v_new,
                           int32_t rotate, float rope_base, swa_rope_style rope_style,
                           void* stream) {
  if (m == nullptr || desc == nullptr) return fail(SWA_ERR_INVALID_ARG, "manager or desc is NULL");
  if (desc->batch != m->max_seqs || desc->max_blocks_per_seq != m->max_blocks ||
      desc->num_phys_blocks != m->num_blocks || desc->block_size != m->block_size)
    return fail(SWA_ERR_INVALID_ARG, "desc (batch, max_blocks_per_seq, num_phys_blocks, "
                                     "block_size) must match the manager");
  if (desc->dtype == SWA_I8)
    return fail(SWA_ERR_UNSUPPORTED, "kv_append_paged: int8 pools are not supported");
  if (desc->num_kv_heads < 1 || (desc->head_dim != 64 && desc->head_dim != 128) ||
      (desc->dtype != SWA_F32 && desc->dtype != SWA_BF16))
    return fail(SWA_ERR_INVALID_ARG, "desc: num_kv_heads >= 1, head_dim 64 or 128, f32 or bf16");
  if (k_pool == nullptr || v_pool == nullptr || block_table == nullptr || seq_lens == nullptr ||
      k_new == nullptr || v_new == nullptr || (n_seqs > 0 && seqs == nullptr))
    return fail(SWA_ERR_INVALID_ARG, "pool, table, lengths, sequences and rows must not be NULL");
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(k_new, 16) || !aligned(v_new, 16))
    return fail(SWA_ERR_INVALID_ARG, "pool and new rows must be 16-byte aligned");
  if (n_seqs < 0 || n_tokens < 1)
    return fail(SWA_ERR_INVALID_ARG, "n_seqs >= 0 and n_tokens >= 1 required");
  if (static_cast<int64_t>(n_seqs) * n_tokens > INT32_MAX)
    return fail(SWA_ERR_INVALID_ARG, "n_seqs * n_tokens too large");
  if (rotate) {
    if (!(rope_base > 0.f) || !std::isfinite(rope_base))
      return fail(SWA_ERR_INVALID_ARG, "rope_base must be positive and finite");
    if (rope_style != SWA_ROPE_INTERLEAVED && rope_style != SWA_ROPE_HALF)
      return fail(SWA_ERR_INVALID_ARG, "unknown rope_style %d", rope_style);
  }
  const int32_t bs = m->block_size;
  // Check everything before changing anything: distinct sequences, room in
  // each table, and enough free blocks for new blocks plus copies.
  std::vector<uint8_t> seen(static_cast<size_t>(m->max_seqs), 0);
  std::vector<int32_t> released;  // blocks an earlier copy-on-write of this call lets go of
  int64_t need = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    const int32_t b = seqs[i];
    swa_status st = check_seq(m, b, "kv_append_paged");
    if (st != SWA_OK) return st;
    if (seen[b]) return fail(SWA_ERR_INVALID_ARG, "kv_append_paged: sequence %d listed twice", b);
    seen[b] = 1;
    const int64_t len = m->lens[b];
    if (len + n_tokens > static_cast<int64_t>(m->max_blocks) * bs)
      return fail(SWA_ERR_INVALID_ARG, "kv_append_paged: sequence %d would exceed %d blocks", b,
                  m->max_blocks);
    need += blocks_for(len + n_tokens, bs) - blocks_for(len, bs);
    if (len % bs != 0) {  // copy-on-write of a shared, partly filled last block
      const int32_t last = m->table[static_cast<size_t>(b) * m->max_blocks + len / bs];
      const int64_t refs = m->ref[last] - std::count(released.begin(), released.end(), last);
      if (refs > 1) {
        need += 1;
        released.push_back(last);
      }
    }
  }
  if (need > static_cast<int64_t>(m->free_q.size()))
    return fail(SWA_ERR_INVALID_ARG, "kv_append_paged: %lld blocks needed, %zu free",
                static_cast<long long>(need), m->free_q.size());

  // Apply, sequence by sequence in the listed order, token by token.
  Updates u;
  std::vector<int32_t> first_pos(static_cast<size_t>(n_seqs));
  for (int32_t i = 0; i < n_seqs; ++i) {
    const int32_t b = seqs[i];
    int32_t* row = m->table.data() + static_cast<size_t>(b) * m->max_blocks;
    const int32_t len = m->lens[b];
    first_pos[i] = len;
    for (int32_t t = 0; t < n_tokens; ++t) {
      const int32_t p = len + t;
      const int32_t j = p / bs;
      if (p % bs == 0) {
        row[j] = take_block(m);
      } else if (t == 0 && m->ref[row[j]] > 1) {
        const int32_t old = row[j];
        const int32_t fresh = take_block(m);
        m->ref[old] -= 1;
        row[j] = fresh;
        u.cow_src.push_back(old);
        u.cow_dst.push_back(fresh);
        u.cow_rows.push_back(p % bs);
      } else {
        continue;  // the block is private and already in the table
      }
      u.table_idx.push_back(b * m->max_blocks + j);
      u.table_val.push_back(row[j]);
    }
    m->lens[b] = len + n_tokens;
    u.lens_idx.push_back(b);
    u.lens_val.push_back(len + n_tokens);
  }

  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t elem = desc->dtype == SWA_BF16 ? 2 : 4;
  hipError_t err = flush(u, block_table, seq_lens, k_pool, v_pool, desc->num_kv_heads, bs,
                         desc->head_dim, elem, s);
  swa::AppendPagedParams a{};
  a.k_src = k_new;
  a.v_src = v_new;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.n_tokens = n_tokens;
  a.num_kv_heads = desc->num_kv_heads;
  a.head_dim = desc->head_dim;
  int shift = 0;
  while ((1 << shift) < bs) ++shift;
  a.block_shift = shift;
  a.max_blocks = m->max_blocks;
  a.num_phys_blocks = m->num_blocks;
  a.rotate = rotate != 0;
  a.rope_half = rope_style == SWA_ROPE_HALF;
  a.bf16 = desc->dtype == SWA_BF16;
  if (rotate) a.freq = swa::make_rope_freq(rope_base, desc->head_dim);
  for (int32_t i0 = 0; err == hipSuccess && i0 < n_seqs; i0 += swa::kAppendMaxSeqs) {
    a.src_first = i0;
    a.n_seqs = std::min(n_seqs - i0, swa::kAppendMaxSeqs);
    for (int32_t i = 0; i < a.n_seqs; ++i) {
      a.seqs[i] = seqs[i0 + i];
      a.first_pos[i] = first_pos[i0 + i];
    }
    err = swa::launch_append_paged(a, s);
  }
  return from_hip(err, "kv_append_paged");
}

}  // extern "C"
