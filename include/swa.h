/*
 * swa.h - decode attention over a bounded KV cache on MI355X (gfx950).
 *
 * Two halves of one decode step:
 *   write: the new token's K (rotated by RoPE at its absolute position, the
 *          rotation baked into the stored row) and V go into a cache slot;
 *   read:  one query per head attends, with online softmax, to exactly the
 *          resident rows, found through a slot-position array (ring cache) or
 *          a block table plus a per-slot validity mask (paged pool).
 *
 * Pages cited (address, section):
 *   [ring]  http://www.2kiu.com/news/4318096/          sliding window + ring KV buffer
 *   [share] http://www.pwwt.cn/news/6215824/           KV sharing, block tables, GQA
 *   [sink]  https://openeuler.csdn.net/6ad3842349ed150a32d85530.html  attention sinks
 *   [kvc]   http://www.pwwt.cn/news/5010196/           KV cache fundamentals
 *   [pool]  https://www.cloudlnk.cn/blog/kv-cache-paging  fixed KV pool, slot mask
 *
 * Conventions for every entry point:
 *   - Plain C linkage; no exception crosses this boundary.
 *   - Every buffer is owned by the caller.  Device buffers are device
 *     pointers (hipMalloc'ed or equivalent); the library never allocates or
 *     frees device memory.  The only allocations are the opaque host objects
 *     (swa_cache, swa_blocks, and swa_pager with its two HIP events).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Compute calls
 *     are asynchronous on it; work on one stream runs in call order, so an
 *     append followed by a decode on the same stream reads the new token.
 *   - Arguments are validated on the host before any HIP call; a bad
 *     argument returns SWA_ERR_INVALID_ARG / SWA_ERR_UNSUPPORTED /
 *     SWA_ERR_WORKSPACE and launches nothing.  A failed launch returns
 *     SWA_ERR_HIP.  swa_last_error() gives the text of the last failure on
 *     the calling thread.
 *   - Values that live in device memory (positions, block ids, lengths) are
 *     not visible to the host: kernels skip out-of-range entries instead of
 *     reading or writing out of bounds (documented per entry point).
 *   - Device pointers to K/V/Q/output rows must be 16-byte aligned.
 *   - Entry points that compute cite the page passage that defines what they
 *     compute.  Calls marked "library helper" (sizing, reset, destroy, state
 *     copies, error text) are bookkeeping of this library that no page
 *     defines.
 */
#ifndef SWA_H_
#define SWA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum swa_status {
  SWA_OK = 0,
  SWA_ERR_INVALID_ARG = -1, /* null pointer, bad size, misalignment        */
  SWA_ERR_UNSUPPORTED = -2, /* valid but not built: head_dim, group, dtype */
  SWA_ERR_WORKSPACE = -3,   /* workspace missing or too small              */
  SWA_ERR_HIP = -4          /* the HIP runtime reported an error           */
} swa_status;

/* Element types of cached K / V rows.  SWA_I8 ([kvc] §5.1: quantise the
 * cache to INT8, half the bytes of 16-bit rows): every stored row (one head
 * of one token, d values) is int8 codes c with one float32 scale s,
 * s = float32(max|x| / 127), c = clamp(rint(x / s), -127, 127), value c * s.
 * A K / V buffer of SWA_I8 holds all rows' codes first (their total padded
 * to a multiple of 256 bytes), then all rows' scales in the same row order.
 * With SWA_I8 caches the queries and the new rows handed to appends and
 * writes are bf16; the rows are quantised when they are stored. */
typedef enum swa_dtype { SWA_F32 = 0, SWA_BF16 = 1, SWA_I8 = 2 } swa_dtype;

/* RoPE pairing: coordinates (2i, 2i+1) or (i, i + d/2) rotate together by
 * angle pos * base^(-2i/d).  The pages name RoPE without fixing a pairing. */
typedef enum swa_rope_style { SWA_ROPE_INTERLEAVED = 0, SWA_ROPE_HALF = 1 } swa_rope_style;

/* ------------------------------------------------------------------------- */
/* Ring cache: S pinned sink slots followed by a W-slot ring.                 */
/* ------------------------------------------------------------------------- */

typedef struct swa_cache_config {
  int32_t batch;          /* B sequences, each with its own cache ([ring] §5.3) */
  int32_t num_kv_heads;   /* Hkv */
  int32_t head_dim;       /* d: 64 or 128 */
  int32_t window;         /* W >= 1: last W positions kept ([ring] §2.2) */
  int32_t num_sinks;      /* S >= 0: first S positions kept forever ([sink], S = 4) */
  swa_dtype dtype;        /* storage dtype of K, V (and of queries, bf16 for SWA_I8) */
  float rope_base;        /* > 0, e.g. 10000 */
  swa_rope_style rope_style;
} swa_cache_config;

/* Opaque host descriptor: the config plus the caller's device pointers. */
typedef struct swa_cache swa_cache;

/* Bytes the caller must allocate for the cache of `cfg`:
 *   K and V, each  [B, Hkv, S+W, d]  elements of cfg->dtype (head-major, so
 *                   one head's slots are contiguous rows of d elements; for
 *                   SWA_I8 the codes, then [B, Hkv, S+W] float32 scales);
 *   slot_pos       [B, S+W] int32, the absolute position held by each slot,
 *                   -1 when empty ([ring] §3.2: a cache slot must remember its
 *                   true position, the slot index is not the position). */
swa_status swa_cache_required_bytes(const swa_cache_config* cfg, size_t* kv_bytes_each,
                                    size_t* slot_pos_bytes);

/* Wraps caller-owned device buffers of the sizes above in a descriptor.
 * Nothing is launched: call swa_cache_reset before the first append.
 * The buffers must outlive the descriptor.  *out is set only on SWA_OK. */
swa_status swa_cache_create(const swa_cache_config* cfg, void* k_cache, void* v_cache,
                            int32_t* slot_pos, swa_cache** out);

/* Library helper (no page defines it): marks every slot empty
 * (slot_pos := -1) with a fill kernel on `stream`. */
swa_status swa_cache_reset(swa_cache* cache, void* stream);

/* Library helper (no page defines it): frees the host descriptor (not the
 * device buffers).  NULL is a no-op. */
void swa_cache_destroy(swa_cache* cache);

/* Appends n_tokens consecutive tokens per sequence ([ring] §3.3 and §5.1:
 * overwrite the oldest entry in O(1), never move or allocate).
 *
 *   k_new, v_new  [B, n_tokens, Hkv, d] in the cache dtype, device.
 *   pos           [B] int32, device: absolute position of token 0 of
 *                 sequence b; token j has position pos[b] + j.
 *   q_inout       [B, n_tokens, Hq, d] in the cache dtype, or NULL.  When
 *                 given, query row (b, j) is rotated in place at pos[b] + j.
 *
 * Token at position p goes to slot p if p < S, else to slot S + (p mod W).
 * Its K row is rotated by RoPE at p and rounded (nearest-even) to the cache
 * dtype before it is stored ([pool] "bake RoPE into K"; [kvc] §4.5); V is
 * stored as given; slot_pos[b][slot] = p.  The result equals n_tokens
 * single-token appends in order: a token whose slot is taken again by a later
 * token of the same call is not written.  Tokens with a negative position are
 * ignored (nothing written, query left as is). */
swa_status kv_append_rope(swa_cache* cache, const void* k_new, const void* v_new,
                          const int32_t* pos, int32_t n_tokens, void* q_inout,
                          int32_t num_q_heads, void* stream);

/* Library helper (no page defines it; the pages' decode keeps no scratch).
 * Workspace (device bytes) that decode_attn_ring / decode_step_ring /
 * decode_attn_paged need for
 * these sizes; max_kv_tokens = S + W for a ring cache, max_blocks_per_seq *
 * block_size for a paged pool.  0 bytes is never returned.
 *
 * The workspace holds the per-split partial results of one call; it needs no
 * initialisation.  Calls that share a workspace must not overlap (use one
 * stream, or one workspace per stream). */
swa_status decode_attn_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t max_kv_tokens, size_t* bytes);

/* One decode step over a ring cache: every query head attends to the slots
 * with slot_pos >= 0 of its sequence (sinks united with the last W positions
 * after appends of 0..t: [sink] cache formula; [ring] §2.2, the current
 * token included).  Softmax weights exp(s) / sum exp(s) with
 * s = scale * <q, k> ([sink] weight formula; [kvc] §2.2); the order of the
 * slots does not matter, so the ring is read in place.
 *
 *   q         [B, Hq, d] in the cache dtype, already rotated at its position.
 *   Hq        multiple of Hkv; query head h reads kv head h / (Hq/Hkv)
 *             ([share] §2.2, §4.1 GQA); Hq/Hkv in {1, 2, 3, 4, 6, 8}.
 *   scale     <= 0 means 1/sqrt(d).
 *   out       [B, Hq, d] of out_dtype (SWA_F32 or SWA_BF16).
 *   lse       [B, Hq] float32 natural-log log-sum-exp of the scaled scores,
 *             or NULL.  A head with no resident row gets out = 0, lse = -inf.
 *   workspace decode_attn_workspace_bytes(B, Hq, Hkv, d, S + W) bytes,
 *             device, 256-byte aligned; contents need no initialisation.
 *   A bf16 cache with d = 128 takes up to 4,194,304 rows per sequence. */
swa_status decode_attn_ring(const swa_cache* cache, const void* q, int32_t num_q_heads,
                            float scale, void* out, swa_dtype out_dtype, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream);

/* A whole decode step on a ring cache in one call: appends one new token per
 * sequence and attends with its query ([ring] §4.3: append, then attend; the
 * write half as kv_append_rope, the read half as decode_attn_ring).
 *
 *   k_new, v_new  [B, Hkv, d] in the cache dtype, device: the new token.
 *   pos           [B] int32, device: its absolute position.
 *   q             [B, Hq, d] in the cache dtype, device, NOT rotated: it is
 *                 rotated at pos[b] (as kv_append_rope's q_inout would be)
 *                 for the attention, and left unchanged in memory.
 *   num_q_heads, scale, out, out_dtype, lse, workspace: as decode_attn_ring.
 *
 * Equivalent to kv_append_rope(cache, k_new, v_new, pos, 1, q', Hq) followed
 * by decode_attn_ring(cache, q', ...) on a copy q' of q: the cache ends in
 * the same state bit for bit, and out / lse agree up to float32 rounding (the
 * new token's score is summed in another order).  A sequence with
 * pos[b] < 0 appends nothing and attends with q as given, as that pair of
 * calls does.  bf16 and int8 caches with d = 128 do both in the decode
 * launch itself (the workgroup whose rows hold the new token's slot writes
 * the token, quantised as the int8 append quantises it, and takes it into
 * its softmax from on-chip memory); other configurations run the two steps
 * as separate launches on `stream`.  The cache is updated by
 * the same launch that reads it: do not read it concurrently. */
swa_status decode_step_ring(swa_cache* cache, const void* k_new, const void* v_new,
                            const int32_t* pos, const void* q, int32_t num_q_heads, float scale,
                            void* out, swa_dtype out_dtype, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream);

/* decode_step_ring with positions taken inside the cache ([sink] "cache
 * position shifting": the window's positions are moved left inside the
 * attention so that their distance to the sinks stays within the window).
 * The cache (sinks, then the window in order) gives every key its index
 * there as its position, and the query the last index,
 * c = min(pos[b], S + W - 1).  RoPE scores depend on distances only; a window
 * key keeps its distance pos[b] - p to the query, so only the sinks change:
 * they are scored against the query rotated at c (rounded to bf16 as an
 * append rounds it), the window against the query rotated at pos[b].  The
 * cache itself is the same as decode_step_ring's (K baked at absolute
 * positions) and ends in the same state.  Arguments as decode_step_ring;
 * bf16 caches with head_dim 128 only (SWA_ERR_UNSUPPORTED otherwise). */
swa_status decode_step_ring_shifted(swa_cache* cache, const void* k_new, const void* v_new,
                                    const int32_t* pos, const void* q, int32_t num_q_heads,
                                    float scale, void* out, swa_dtype out_dtype, float* lse,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Library helper (no page defines it): pos[i] += delta for i < n, on `stream` (one small kernel; results clamped
 * to the int32 range).  Positions live in device memory, so a HIP graph that
 * captures decode steps followed by this call replays with each step at the
 * next position; every decode and append entry point above only launches
 * kernels on `stream` (no allocation, synchronisation or memset), so it can
 * be captured.  pos: [n] int32, device, 4-byte aligned; n >= 0 (0 launches
 * nothing). */
swa_status swa_pos_advance(int32_t* pos, int32_t n, int32_t delta, void* stream);

/* Library helper (no page defines it): reads `bytes` of device memory at
 * `src` once, with nontemporal 16-byte loads spread over 2048 workgroups, on
 * `stream`; it measures the HBM read rate the chip achieves, the practical
 * ceiling for the decode kernels.  bytes: a multiple of 16 (0 launches
 * nothing); src: 16-byte aligned device memory the caller owns; sink:
 * device memory of at least SWA_STREAM_READ_SINK_BYTES, 4-byte aligned,
 * which receives a checksum per wave (its contents mean nothing else).
 * SWA_ERR_INVALID_ARG for NULL pointers, misalignment, a size that is not a
 * multiple of 16 or a sink that is too small. */
#define SWA_STREAM_READ_SINK_BYTES ((size_t)32768)
swa_status swa_stream_read(const void* src, size_t bytes, void* sink, size_t sink_bytes,
                           void* stream);

/* Library helper (no page defines it): workspace (device bytes) of a
 * prefill_attn_ring call with n_tokens tokens per sequence.  Needs no
 * initialisation. */
swa_status prefill_attn_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t n_tokens, size_t* bytes);

/* Chunked prefill on a ring cache ([pool] "paging": prefill in chunks of
 * 128-256 tokens; [ring] §1.3, [share] §2.3: prefill vs decode): n_tokens new
 * tokens per sequence, at positions pos[b] .. pos[b] + n_tokens - 1, are
 * attended and then appended.
 *
 *   k_new, v_new  [B, n_tokens, Hkv, d] in the cache dtype, device.
 *   pos           [B] int32, device: position of token 0 of sequence b.
 *   q             [B, n_tokens, Hq, d] in the cache dtype, device, NOT rotated
 *                 (rotated at its position for the attention, left unchanged
 *                 in memory).
 *   out           [B, n_tokens, Hq, d] of out_dtype; lse [B, n_tokens, Hq]
 *                 float32 natural-log, or NULL.
 *   workspace     prefill_attn_workspace_bytes(B, Hq, Hkv, d, n_tokens) bytes,
 *                 device, 256-byte aligned.
 *
 * Query row (b, j, h) equals what a decode step at position t = pos[b] + j
 * would give after the tokens before it were appended: attention over the
 * keys at positions p <= t with p < S or p > t - W ([sink] cache formula;
 * [ring] §2.2), from the ring as it was before the call (positions below
 * pos[b]) and from the chunk itself (causal).  Afterwards the cache is in the
 * state kv_append_rope(cache, k_new, v_new, pos, n_tokens, NULL) leaves, bit
 * for bit.  A token at a negative position, or at one beyond 2^31 - 1, is
 * neither attended nor appended; its query row gets out = 0, lse = -inf.
 *
 * Supported: bf16 caches with d = 128, Hq / Hkv in {1, 2, 3, 4, 6, 8},
 * (S + W) * 256 and n_tokens * Hkv * 256 below 2^31 (SWA_ERR_UNSUPPORTED
 * otherwise).  The product P V runs in fp16 with fp32
 * accumulation: V must stay below 65504 in magnitude.  Three launches on
 * `stream` (rotation, attention, append); the call reads and then writes the
 * cache: do not read it concurrently. */
swa_status prefill_attn_ring(swa_cache* cache, const void* k_new, const void* v_new,
                             const int32_t* pos, int32_t n_tokens, const void* q,
                             int32_t num_q_heads, float scale, void* out, swa_dtype out_dtype,
                             float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------- */
/* Paged pool: fixed-size blocks addressed through a block table.             */
/* ------------------------------------------------------------------------- */

typedef struct swa_paged_desc {
  int32_t batch;              /* B */
  int32_t num_q_heads;        /* Hq, a multiple of Hkv */
  int32_t num_kv_heads;       /* Hkv */
  int32_t head_dim;           /* d: 64 or 128 */
  int32_t block_size;         /* tokens per block: a power of two, 16..1024 */
  int32_t max_blocks_per_seq; /* columns of block_table / block_valid */
  int32_t num_phys_blocks;    /* blocks in the pool */
  swa_dtype dtype;            /* pool and query dtype */
} swa_paged_desc;

/* Bytes of each of the K and V pools of `desc`: [num_phys_blocks, Hkv,
 * block_size, d] elements of desc->dtype; for SWA_I8 the codes, padded to a
 * multiple of 256 bytes, then [num_phys_blocks, Hkv, block_size] float32
 * scales. */
swa_status swa_pool_required_bytes(const swa_paged_desc* desc, size_t* kv_bytes_each);

/* One decode step over a paged pool ([share] §3.1 block table; [pool]
 * "paging" and "the kernel forgets absent blocks").
 *
 *   k_pool, v_pool  [num_phys_blocks, Hkv, block_size, d], device.
 *   block_table     [B, max_blocks_per_seq] int32, device: entry j of
 *                   sequence b is the physical block holding its tokens
 *                   j*block_size .. (j+1)*block_size - 1.  Several sequences
 *                   may name the same block (a shared prefix, [share] §3.2).
 *   seq_lens        [B] int32, device: tokens of sequence b (clamped to
 *                   [0, max_blocks_per_seq * block_size]).
 *   block_valid     [B, max_blocks_per_seq] uint8, device, or NULL (all
 *                   valid): 0 marks a slot whose block is absent.
 *   (for SWA_I8 pools the query is bf16 and each pool holds codes then
 *   scales, swa_pool_required_bytes.)
 *
 * Resident rows of sequence b: tokens i < seq_lens[b] whose entry
 * j = i / block_size is valid and names a block in [0, num_phys_blocks);
 * every other row is never read into the arithmetic ("as if it did not
 * exist").  K rows are used as stored (RoPE, if any, already baked in), so
 * the call needs no positions.  q, scale, out, lse, workspace as for
 * decode_attn_ring with max_kv_tokens = max_blocks_per_seq * block_size. */
swa_status decode_attn_paged(const swa_paged_desc* desc, const void* q, const void* k_pool,
                             const void* v_pool, const int32_t* block_table,
                             const int32_t* seq_lens, const uint8_t* block_valid, float scale,
                             void* out, swa_dtype out_dtype, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream);

/* decode_attn_paged for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same computation and arguments as decode_attn_paged, with
 * no workspace: the partial results live in a fixed array of this library
 * in device memory, SWA_NOALLOC_SCRATCH_BYTES bytes per device, which each
 * device holds from the library's first use on it until the process ends.
 * Its device address is looked up on the first call on a device (that device
 * current); no call allocates or frees anything.
 *
 *   Limit: sizes whose decode_attn_workspace_bytes(batch, Hq, Hkv, d,
 *   max_blocks_per_seq * block_size) exceeds SWA_NOALLOC_SCRATCH_BYTES are
 *   refused with SWA_ERR_WORKSPACE before any HIP call.
 *   Sharing: every call on one device uses that device's one array; it needs
 *   no initialisation (each call writes every entry it reads) and keeps the
 *   last call's contents.  Calls that overlap on one device (two streams, two
 *   threads, two captured graphs replayed concurrently) race on it: issue
 *   them in one stream's order. */
#define SWA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
swa_status decode_attn_paged_noalloc(const swa_paged_desc* desc, const void* q,
                                     const void* k_pool, const void* v_pool,
                                     const int32_t* block_table, const int32_t* seq_lens,
                                     const uint8_t* block_valid, float scale, void* out,
                                     swa_dtype out_dtype, float* lse, void* stream);

/* Writes n_tokens rows into a paged pool, rotating K at a given position
 * first ([pool] "bake RoPE into K": each block becomes self-contained).
 *
 *   k_src, v_src  [n_tokens, Hkv, d] in the pool dtype, device.
 *   dst_rows      [n_tokens] int32, device: physical token row
 *                 block * block_size + r of each token.
 *   pos           [n_tokens] int32, device: RoPE position of each token, or
 *                 NULL to store K as given.
 * Tokens whose dst_rows entry is outside [0, num_phys_blocks * block_size) or
 * whose position is negative are skipped.  Two tokens naming the same row
 * race (one of them wins). */
swa_status kv_write_paged(const swa_paged_desc* desc, void* k_pool, void* v_pool,
                          const void* k_src, const void* v_src, const int32_t* dst_rows,
                          const int32_t* pos, int32_t n_tokens, float rope_base,
                          swa_rope_style rope_style, void* stream);

/* ------------------------------------------------------------------------- */
/* Block manager: refcounted pool blocks, prefix sharing, copy-on-write      */
/* ([share] §3.2 prefix sharing, §5.1 allocate / share_prefix / append_token, */
/* §6.1 release by reference count on every path).                           */
/* ------------------------------------------------------------------------- */

/* Opaque host object: per-block reference counts, per-sequence block lists
 * and lengths, and the free list.  Not thread-safe: one thread drives it. */
typedef struct swa_blocks swa_blocks;

/* A manager of num_blocks pool blocks of block_size tokens (a power of two,
 * 16..1024) for sequences 0 .. max_seqs-1 of up to max_blocks_per_seq blocks
 * each.  All blocks start free and every sequence empty.  Host only. */
swa_status swa_blocks_create(int32_t num_blocks, int32_t block_size, int32_t max_seqs,
                             int32_t max_blocks_per_seq, swa_blocks** out);

/* Library helper (no page defines it): frees the host object.  NULL is a
 * no-op. */
void swa_blocks_destroy(swa_blocks* mgr);

/* Library helper (no page defines it): every block free, every sequence
 * empty (host state only; follow with
 * swa_blocks_sync before the device mirrors are read). */
swa_status swa_blocks_reset(swa_blocks* mgr);

/* Library helper (no page defines it): writes the whole host state into
 * the device mirrors the paged decode reads:
 *   block_table  [max_seqs, max_blocks_per_seq] int32 (-1 = no block),
 *   seq_lens     [max_seqs] int32.
 * Returns when `stream` has done it (a set-up call). */
swa_status swa_blocks_sync(swa_blocks* mgr, int32_t* block_table, int32_t* seq_lens,
                           void* stream);

/* The first prefix_len tokens of the empty sequence dst point at src's blocks
 * (ceil(prefix_len / block_size) of them, each gaining a reference); dst's
 * length becomes prefix_len.  The device mirrors are updated on `stream`. */
swa_status swa_blocks_share_prefix(swa_blocks* mgr, int32_t src, int32_t dst, int32_t prefix_len,
                                   int32_t* block_table, int32_t* seq_lens, void* stream);

/* Ends sequence seq: each of its blocks loses a reference and returns to the
 * free list when no sequence references it any more; its length becomes 0
 * (device mirror updated on `stream`). */
swa_status swa_blocks_free(swa_blocks* mgr, int32_t seq, int32_t* seq_lens, void* stream);

/* Library helper (no page defines it): host copies of the state; each
 * output may be NULL:
 *   table [max_seqs * max_blocks_per_seq], lens [max_seqs],
 *   refs [num_blocks] reference counts, *free_blocks = free blocks. */
swa_status swa_blocks_state(const swa_blocks* mgr, int32_t* table, int32_t* lens, int32_t* refs,
                            int32_t* free_blocks);

/* Appends n_tokens tokens to each listed sequence ([share] §5.1
 * append_token, blocks allocated on demand).
 *
 *   desc          the pool: batch = max_seqs, max_blocks_per_seq, block_size
 *                 and num_phys_blocks as the manager's; num_kv_heads,
 *                 head_dim (64 or 128), dtype of the rows.
 *   k_pool, v_pool, block_table, seq_lens  device, as decode_attn_paged reads
 *                 them; the table and lengths are updated by this call.
 *   seqs          [n_seqs] int32, host: distinct sequences.
 *   k_new, v_new  [n_seqs, n_tokens, Hkv, d], device: row (i, t) is token
 *                 seq_lens[seqs[i]] + t of sequence seqs[i].
 *   rotate        nonzero: K is rotated by RoPE at the token's position in
 *                 its sequence before it is stored (rope_base, rope_style);
 *                 0: K is stored as given.
 *
 * Equivalent to appending the tokens one at a time, sequence by sequence in
 * the listed order: a token that starts a block takes the lowest-numbered
 * free block; a token written into a block that another sequence also
 * references first gets a private copy of that block's used rows
 * (copy-on-write: a shared block is never written in place).  If the blocks
 * would not suffice, or a table would overflow, SWA_ERR_INVALID_ARG is
 * returned and nothing changes.  Two launches or more on `stream`.  SWA_I8
 * pools are not supported here (SWA_ERR_UNSUPPORTED). */
swa_status kv_append_paged(swa_blocks* mgr, const swa_paged_desc* desc, void* k_pool, void* v_pool,
                           int32_t* block_table, int32_t* seq_lens, const int32_t* seqs,
                           int32_t n_seqs, int32_t n_tokens, const void* k_new, const void* v_new,
                           int32_t rotate, float rope_base, swa_rope_style rope_style,
                           void* stream);

/* ------------------------------------------------------------------------- */
/* Host-pool pager: a sequence's history in host memory, a fixed pool of     */
/* device slots filled on demand ([pool] "paging").                          */
/* ------------------------------------------------------------------------- */

typedef struct swa_pager_config {
  int32_t batch;           /* B sequences, each with its own slots */
  int32_t num_kv_heads;    /* Hkv */
  int32_t head_dim;        /* d: 64 or 128 */
  int32_t block_size;      /* tokens per block: a power of two, 16..1024 (64 on [pool]) */
  int32_t logical_blocks;  /* L: blocks of each sequence's history in the host store */
  int32_t slots_per_seq;   /* C: device slots of each sequence (columns of block_table) */
  int32_t num_phys_blocks; /* blocks in the device pool */
  swa_dtype dtype;         /* K / V element type: SWA_F32 or SWA_BF16 */
} swa_pager_config;

/* Opaque host object: the LRU state of every slot, the caller's pointers and
 * two HIP events that order the copies against the attention. */
typedef struct swa_pager swa_pager;

/* A pager over caller-owned memory.
 *
 *   host_k, host_v  [B, L, Hkv, block_size, d] in cfg->dtype: every block of
 *                   every sequence's history, K already rotated by RoPE at
 *                   its absolute position ([pool] "bake RoPE into K": a block
 *                   is self-contained, so it can sit in any slot).  Pinned
 *                   host memory that the device can read (hipHostMalloc, or
 *                   torch's pin_memory); otherwise SWA_ERR_INVALID_ARG.
 *   k_pool, v_pool  [num_phys_blocks, Hkv, block_size, d], device: the
 *                   layout decode_attn_paged reads.
 *   slot_phys       [B, C] int32, host, copied: the pool block behind slot j
 *                   of sequence b; all distinct, in [0, num_phys_blocks).
 *   block_table     [B, C] int32, device: written by swa_pager_reset
 *                   (slot_phys), then left alone.
 *   block_valid     [B, C] uint8, device: 1 where a slot's block may be read.
 *
 * decode_attn_paged with (block_table, block_valid, seq_lens = C * block_size,
 * max_blocks_per_seq = C) then attends exactly the blocks the pager has made
 * visible.  The pager never allocates device memory; it creates two HIP
 * events (so this call needs a device).  Call swa_pager_reset before the
 * first request.  Not thread-safe: one thread drives a pager. */
swa_status swa_pager_create(const swa_pager_config* cfg, const void* host_k, const void* host_v,
                            void* k_pool, void* v_pool, const int32_t* slot_phys,
                            int32_t* block_table, uint8_t* block_valid, swa_pager** out);

/* Library helper (no page defines it): every slot empty: block_table := slot_phys, block_valid := 0, no block
 * resident, LRU history cleared.  Waits for copies in flight and returns when
 * the stream has done it (a set-up call). */
swa_status swa_pager_reset(swa_pager* pager, void* stream);

/* Serves one request per sequence ([pool] "residency policy": LRU).
 *
 *   req_offsets  [B + 1] int32, host: sequence b names req_blocks[
 *                req_offsets[b] .. req_offsets[b+1]) (offsets[0] = 0,
 *                non-decreasing; a sequence may name nothing).
 *   req_blocks   int32, host: logical blocks in [0, L); repeats count once.
 *   stream       the stream the attention runs on.
 *   copy_stream  the stream the copies run on.  It may equal `stream`: then
 *                stream order alone orders everything and the copies do not
 *                overlap the attention, but no event is waited on across
 *                streams (on this platform such a wait costs the host more
 *                than a short attention step).
 *   n_loaded     host, or NULL: blocks this call starts copying.
 *
 * Every named block that is not resident gets a slot: the lowest empty one,
 * else the slot of the least recently named block (ties: lower slot), never
 * one named by this request or by the previous call (the attention step that
 * call prepared is enqueued after this one and still needs them).  Blocks of a sliding window stay
 * resident by being named in every request ([pool]: SWA layers keep their
 * window blocks, only the others are paged).  If a sequence misses more
 * blocks than it has empty plus evictable slots the call fails with
 * SWA_ERR_INVALID_ARG and changes nothing.
 *
 * Order on the streams: work enqueued on `stream` after this call sees the
 * blocks copied by the previous call (they become valid first) and no longer
 * sees the slots this call overwrites (cleared); the new copies start on
 * copy_stream once the work enqueued on `stream` before this call is done,
 * and become visible at the next swa_pager_advance or swa_pager_commit.  So
 *   advance(N_{t+1}); decode(t); advance(N_{t+2}); decode(t+1); ...
 * overlaps the copies for step t+1 with the attention of step t.  After
 * SWA_ERR_HIP the pager must be reset. */
swa_status swa_pager_advance(swa_pager* pager, const int32_t* req_offsets,
                             const int32_t* req_blocks, void* stream, void* copy_stream,
                             int32_t* n_loaded);
/* (SWA_ERR_INVALID_ARG while a swa_pager_stage is pending.) */

/* The paging step folded into the attention's launches ([pool] "paging", the
 * copies overlapping the attention kernel so that it only consumes resident
 * blocks).  swa_pager_stage serves the next step's request on the host
 * state exactly as swa_pager_advance does (same LRU decisions, same refusal)
 * but launches nothing; the next swa_pager_decode on the pager runs the
 * attention over the pool and, in the same launches, the staged copies:
 * extra workgroups of the attention launch read the staged blocks from the
 * host store into a staging area of the workspace while the attention reads
 * the pool, and extra workgroups of the merge launch (which starts after the
 * attention has read the pool) move them into their slots and set their
 * validity bytes.  Everything is ordered by `stream` alone: no event, no
 * second stream.  A step's attention therefore sees the blocks resident when
 * it starts, including blocks that the staged request evicts (their slots
 * are overwritten only after the attention has read them), and the staged
 * blocks are visible to every launch after the decode:
 *   stage(N_0); commit; stage(N_1); decode(step 0); stage(N_2); decode(step 1); ...
 *
 *   req_offsets, req_blocks, n_loaded  as for swa_pager_advance.
 *
 * SWA_ERR_INVALID_ARG when a stage is pending (not yet decoded or committed)
 * or when copies of swa_pager_advance are not yet visible (commit first).
 * Not thread-safe, as the rest of the pager. */
swa_status swa_pager_stage(swa_pager* pager, const int32_t* req_offsets, const int32_t* req_blocks,
                           int32_t* n_loaded);

/* decode_attn_paged over the pager's pool (block_table and block_valid of
 * the pager, max_blocks_per_seq = slots_per_seq, the config's batch, heads,
 * head_dim, block_size, pool size and dtype; no shared-prefix pass, since no
 * two of the pager's sequences share a block), followed in the same launches
 * by the copies of the last swa_pager_stage (see above; more staged blocks
 * than the staging area holds, min(64, 16 MiB / (2 x block bytes)), or a
 * pool the matrix-core decode does not take, run as separate launches after
 * the decode, with the same effect).  The arguments are decode_attn_paged's:
 * q [B, num_q_heads, d] rotated, seq_lens [B] device (C * block_size to
 * attend every visible slot), scale, out, out_dtype, lse, and a device
 * workspace of at least swa_pager_workspace_bytes(pager, num_q_heads) bytes,
 * 256-byte aligned (SWA_ERR_WORKSPACE if smaller).  An argument error
 * launches nothing and leaves the stage pending; SWA_ERR_INVALID_ARG when
 * copies of swa_pager_advance are not yet visible (commit first). */
swa_status swa_pager_decode(swa_pager* pager, const void* q, int32_t num_q_heads,
                            const int32_t* seq_lens, float scale, void* out, swa_dtype out_dtype,
                            float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Library helper (no page defines it): workspace bytes swa_pager_decode needs
 * with num_q_heads query heads: decode_attn_workspace_bytes(B, num_q_heads,
 * Hkv, d, slots_per_seq * block_size) rounded up to 256, plus the staging
 * area of the folded copies.  Also enough for decode_attn_paged over the
 * pager's pool.  *bytes, host. */
swa_status swa_pager_workspace_bytes(const swa_pager* pager, int32_t num_q_heads, size_t* bytes);

/* Library helper (no page defines it): makes the copies of the last advance visible to work enqueued on `stream`
 * after this call (it waits for them on the device, not on the host); a stage
 * not yet decoded has its copies launched on `stream` (no attention). */
swa_status swa_pager_commit(swa_pager* pager, void* stream);

/* Library helper (no page defines it): logical block held by each slot of sequence seq (-1 = empty), as the host
 * state stands (copies in flight included): out [C] int32, host. */
swa_status swa_pager_slot_blocks(const swa_pager* pager, int32_t seq, int32_t* out);

/* Library helper (no page defines it): frees the host object and its events (not the caller's memory).  Does not
 * wait for copies in flight.  NULL is a no-op. */
void swa_pager_destroy(swa_pager* pager);

/* Library helper (no page defines it): text of the last failure on the
 * calling thread ("" if none).  The pointer stays valid until the thread's
 * next call into the library. */
const char* swa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SWA_H_ */
