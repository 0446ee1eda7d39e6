// Write half of the decode step: fused RoPE + scatter of the new tokens into
// the cache.
//
// Ring cache ([ring] §3.3 and §5.1: overwrite the oldest entry in place, no
// allocation; [sink]: S pinned sink slots): token at absolute position p goes
// to slot p (p < S) or S + (p mod W); its K row is rotated at p and rounded to
// the storage dtype before the store ([pool] "bake RoPE into K"), V is copied
// bit for bit, and the slot's true position is recorded ([ring] §3.2, §7).
//
// The rotation angles pos * theta_i are formed and reduced in float64 (the
// theta_i come from the host), so positions up to 2^31 lose no accuracy; the
// rotation itself is done in f64 and rounded once to the storage dtype.
#include "device_common.h"
#include "swa_internal.h"

namespace swa {
namespace {

constexpr int kAppendThreads = 256;
constexpr int kMaxHalfDim = 64;  // head_dim <= 128

template <bool BF16>
struct Elem;
template <>
struct Elem<true> {
  using T = uint16_t;
  __device__ static double load(const T* p, int i) { return static_cast<double>(bf16_to_f32(p[i])); }
  __device__ static void store(T* p, int i, double x) { p[i] = f64_to_bf16_rne(x); }
};
template <>
struct Elem<false> {
  using T = float;
  __device__ static double load(const T* p, int i) { return static_cast<double>(p[i]); }
  __device__ static void store(T* p, int i, double x) { p[i] = static_cast<float>(x); }
};

// Angles of the token: cos/sin(pos * theta_i), i < d/2.
__device__ void rope_angles(double pos, const RopeFreq& freq, int head_dim, double* s_cos,
                            double* s_sin) {
  const int half = head_dim / 2;
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    double s, c;
    rope_sincos(pos, freq.theta[i], &s, &c);
    s_cos[i] = c;
    s_sin[i] = s;
  }
}

// Rotates `rows` rows of head_dim elements from src into dst (may alias);
// consecutive rows are src_stride / dst_stride elements apart.
template <bool BF16>
__device__ void rotate_rows(const typename Elem<BF16>::T* src, size_t src_stride,
                            typename Elem<BF16>::T* dst, size_t dst_stride, int rows,
                            int head_dim, int rope_half, const double* s_cos,
                            const double* s_sin) {
  using E = Elem<BF16>;
  const int half = head_dim / 2;
  for (int w = threadIdx.x; w < rows * half; w += blockDim.x) {
    const int r = w / half;
    const int i = w - r * half;
    const int i0 = rope_half ? i : 2 * i;
    const int i1 = rope_half ? i + half : 2 * i + 1;
    const typename E::T* s = src + static_cast<size_t>(r) * src_stride;
    typename E::T* d = dst + static_cast<size_t>(r) * dst_stride;
    double o0, o1;
    rope_rotate_pair(E::load(s, i0), E::load(s, i1), s_cos[i], s_sin[i], &o0, &o1);
    E::store(d, i0, o0);
    E::store(d, i1, o1);
  }
}

// Copies `rows` rows of row_bytes (a multiple of 16) with byte strides.
__device__ void copy_rows16(const void* src, size_t src_stride, void* dst, size_t dst_stride,
                            int rows, size_t row_bytes) {
  const size_t per_row = row_bytes / 16;
  for (size_t w = threadIdx.x; w < rows * per_row; w += blockDim.x) {
    const size_t r = w / per_row;
    const size_t c = w - r * per_row;
    const uint4* s = reinterpret_cast<const uint4*>(static_cast<const char*>(src) + r * src_stride);
    uint4* d = reinterpret_cast<uint4*>(static_cast<char*>(dst) + r * dst_stride);
    d[c] = s[c];
  }
}

// One thread per unit of work of one token: a rotated K pair, a rotated query
// pair, or a 16-byte chunk of the V row.  Each thread computes the angle of its
// own pair, so a single-token decode append spreads over many workgroups
// instead of looping inside a few.
template <bool BF16>
__global__ __launch_bounds__(kAppendThreads) void append_rope_kernel(AppendParams p,
                                                                     int items_per_token,
                                                                     int wgs_per_token) {
  using E = Elem<BF16>;
  using T = typename E::T;
  const int token = blockIdx.x / wgs_per_token;  // b * n_tokens + j
  const int item = (blockIdx.x - token * wgs_per_token) * kAppendThreads + threadIdx.x;
  if (item >= items_per_token) return;
  const int b = token / p.n_tokens;
  const int j = token - b * p.n_tokens;
  const int64_t pos = static_cast<int64_t>(p.pos[b]) + j;
  if (pos < 0 || pos > INT32_MAX) return;

  const int d = p.head_dim;
  const int half = d / 2;
  const int slots = p.sinks + p.window;
  const bool k_copy = p.k_rotated != nullptr;
  const int k_items = k_copy ? 0 : p.num_kv_heads * half;
  const int q_items = p.q_inout != nullptr ? p.num_q_heads * half : 0;
  // A later token of this call lands in the same ring slot: leave it the slot.
  const bool overwritten = pos >= p.sinks && j + p.window <= p.n_tokens - 1;
  const int slot = pos < p.sinks ? static_cast<int>(pos) : p.sinks + static_cast<int>(pos % p.window);

  if (item < k_items + q_items) {
    const bool is_k = item < k_items;
    if (is_k && overwritten) return;
    const int w = is_k ? item : item - k_items;
    const int h = w / half;
    const int i = w - h * half;
    double sn, cs;
    rope_sincos(static_cast<double>(pos), p.freq.theta[i], &sn, &cs);
    const int i0 = p.rope_half ? i : 2 * i;
    const int i1 = p.rope_half ? i + half : 2 * i + 1;
    const T* src;
    T* dst;
    if (is_k) {
      src = static_cast<const T*>(p.k_new) +
            ((static_cast<size_t>(b) * p.n_tokens + j) * p.num_kv_heads + h) * d;
      dst = static_cast<T*>(p.k_cache) +
            ((static_cast<size_t>(b) * p.num_kv_heads + h) * slots + slot) * d;
    } else {
      const size_t qrow = ((static_cast<size_t>(b) * p.n_tokens + j) * p.num_q_heads + h) * d;
      src = static_cast<const T*>(p.q_inout) + qrow;
      dst = static_cast<T*>(p.q_out != nullptr ? p.q_out : p.q_inout) + qrow;
    }
    double o0, o1;
    rope_rotate_pair(E::load(src, i0), E::load(src, i1), cs, sn, &o0, &o1);
    E::store(dst, i0, o0);
    E::store(dst, i1, o1);
    if (is_k && item == 0) p.slot_pos[static_cast<size_t>(b) * slots + slot] = static_cast<int32_t>(pos);
    return;
  }
  if (overwritten) return;
  // V (then the pre-rotated K rows): 16-byte chunks of the token's Hkv rows
  const int per_row = d * static_cast<int>(sizeof(T)) / 16;
  int w = item - k_items - q_items;
  const bool is_v = w < p.num_kv_heads * per_row;
  if (!is_v) w -= p.num_kv_heads * per_row;
  const int h = w / per_row;
  const int c = w - h * per_row;
  const uint4* src = reinterpret_cast<const uint4*>(
      static_cast<const T*>(is_v ? p.v_new : p.k_rotated) +
      ((static_cast<size_t>(b) * p.n_tokens + j) * p.num_kv_heads + h) * d);
  uint4* dst = reinterpret_cast<uint4*>(
      static_cast<T*>(is_v ? p.v_cache : p.k_cache) +
      ((static_cast<size_t>(b) * p.num_kv_heads + h) * slots + slot) * d);
  dst[c] = src[c];
  if (k_copy && !is_v && w == 0)
    p.slot_pos[static_cast<size_t>(b) * slots + slot] = static_cast<int32_t>(pos);
}

// One token's Hkv rows of K (rotated at pos when `rotate`) and V into pool
// row r of block blk ([Nphys, Hkv, bs, d]).  Run by a whole workgroup; the
// caller has checked blk and r.
template <bool BF16>
__device__ void write_token_rows(const void* k_src_all, const void* v_src_all, size_t src_token,
                                 void* k_pool, void* v_pool, int64_t blk, int r, int num_kv_heads,
                                 int block_size, int d, bool rotate, int32_t pos,
                                 const RopeFreq& freq, int rope_half, double* s_cos,
                                 double* s_sin) {
  using T = typename Elem<BF16>::T;
  if (rotate) {
    rope_angles(static_cast<double>(pos), freq, d, s_cos, s_sin);
    __syncthreads();
  }
  const size_t src_row = src_token * num_kv_heads * d;
  const T* k_src = static_cast<const T*>(k_src_all) + src_row;
  const T* v_src = static_cast<const T*>(v_src_all) + src_row;
  // head h of the token goes to row (blk, h, r) of the pool
  const size_t dst = (static_cast<size_t>(blk) * num_kv_heads * block_size + r) * d;
  const size_t head_stride = static_cast<size_t>(block_size) * d;
  T* k_dst = static_cast<T*>(k_pool) + dst;
  if (rotate)
    rotate_rows<BF16>(k_src, d, k_dst, head_stride, num_kv_heads, d, rope_half, s_cos, s_sin);
  else
    copy_rows16(k_src, d * sizeof(T), k_dst, head_stride * sizeof(T), num_kv_heads,
                d * sizeof(T));
  copy_rows16(v_src, d * sizeof(T), static_cast<T*>(v_pool) + dst, head_stride * sizeof(T),
              num_kv_heads, d * sizeof(T));
}

template <bool BF16>
__global__ __launch_bounds__(kAppendThreads) void write_paged_kernel(PagedWriteParams p) {
  __shared__ double s_cos[kMaxHalfDim];
  __shared__ double s_sin[kMaxHalfDim];

  const int n = blockIdx.x;
  const int64_t row = p.dst_rows[n];
  const int64_t rows_total = static_cast<int64_t>(p.num_phys_blocks) * p.block_size;
  if (row < 0 || row >= rows_total) return;
  const bool rotate = p.pos != nullptr;
  const int32_t pos = rotate ? p.pos[n] : 0;
  if (pos < 0) return;
  const int64_t blk = row / p.block_size;
  const int r = static_cast<int>(row - blk * p.block_size);
  write_token_rows<BF16>(p.k_src, p.v_src, static_cast<size_t>(n), p.k_pool, p.v_pool, blk, r,
                         p.num_kv_heads, p.block_size, p.head_dim, rotate, pos, p.freq,
                         p.rope_half, s_cos, s_sin);
}

// Paged append: token j of listed sequence i (workgroup i * n_tokens + j) is
// at position first_pos[i] + j of sequence seqs[i]; its row is found through
// the device block table, which the update launch before this one has
// already extended.
template <bool BF16>
__global__ __launch_bounds__(kAppendThreads) void append_paged_kernel(AppendPagedParams p) {
  __shared__ double s_cos[kMaxHalfDim];
  __shared__ double s_sin[kMaxHalfDim];
  const int i = static_cast<int>(blockIdx.x) / p.n_tokens;
  const int j = static_cast<int>(blockIdx.x) - i * p.n_tokens;
  if (i >= p.n_seqs) return;
  const int64_t pos = static_cast<int64_t>(p.first_pos[i]) + j;
  const int64_t q = pos >> p.block_shift;
  if (pos < 0 || q >= p.max_blocks) return;
  const int32_t blk = p.block_table[static_cast<size_t>(p.seqs[i]) * p.max_blocks + q];
  if (blk < 0 || blk >= p.num_phys_blocks) return;
  const int r = static_cast<int>(pos & ((int64_t{1} << p.block_shift) - 1));
  write_token_rows<BF16>(p.k_src, p.v_src, static_cast<size_t>(p.src_first + i) * p.n_tokens + j,
                         p.k_pool, p.v_pool, blk, r, p.num_kv_heads, 1 << p.block_shift,
                         p.head_dim, p.rotate != 0, static_cast<int32_t>(pos), p.freq,
                         p.rope_half, s_cos, s_sin);
}

// Block-manager updates by value: block-table entries, sequence lengths, and
// copy-on-write copies of the first `rows` rows of a block (all heads, K and
// V).  Workgroup 0 writes the entries; workgroup 1 + 2c + t copies tensor t of
// copy c.
__global__ __launch_bounds__(kAppendThreads) void blocks_update_kernel(BlocksUpdateParams p) {
  if (blockIdx.x == 0) {
    for (int e = threadIdx.x; e < p.n_table; e += blockDim.x) p.block_table[p.table_idx[e]] = p.table_val[e];
    for (int e = threadIdx.x; e < p.n_lens; e += blockDim.x) p.seq_lens[p.lens_idx[e]] = p.lens_val[e];
    return;
  }
  const int c = (static_cast<int>(blockIdx.x) - 1) / 2;
  const int t = (static_cast<int>(blockIdx.x) - 1) % 2;
  if (c >= p.n_cow) return;
  const size_t row_bytes = static_cast<size_t>(p.head_dim) * p.elem_bytes;
  const size_t head_bytes = row_bytes * p.block_size;
  const size_t block_bytes = head_bytes * p.num_kv_heads;
  char* base = static_cast<char*>(t == 0 ? p.k_pool : p.v_pool);
  const char* src = base + static_cast<size_t>(p.cow_src[c]) * block_bytes;
  char* dst = base + static_cast<size_t>(p.cow_dst[c]) * block_bytes;
  // rows 0 .. rows-1 of every head: Hkv runs of rows * row_bytes contiguous bytes
  copy_rows16(src, head_bytes, dst, head_bytes, p.num_kv_heads, row_bytes * p.cow_rows[c]);
}

// Quantises the row held by the wave (quantize_pair_row) and stores its
// codes, and its scale next to the codes' row.
__device__ void quantize_row_store(double x0, double x1, bool active, int e0, int e1,
                                   int8_t* codes, float* scale) {
  double c0, c1;
  const float s = quantize_pair_row(x0, x1, active, &c0, &c1);
  if (active) {
    codes[e0] = static_cast<int8_t>(c0);
    codes[e1] = static_cast<int8_t>(c1);
  }
  if ((threadIdx.x & 63) == 0) *scale = s;
}

// Elements of RoPE pair i of a row: (2i, 2i+1) or (i, i + d/2).
__device__ __forceinline__ void pair_elems(int i, int half, int rope_half, int* e0, int* e1) {
  *e0 = rope_half ? i : 2 * i;
  *e1 = rope_half ? i + half : 2 * i + 1;
}

// Ring append into an int8 cache: one wave per row of a token (its Hkv K
// rows, Hkv V rows, and Hq query rows when q_inout is given), four rows per
// workgroup, so a decode step's few tokens still spread over many CUs.  K
// is rotated at the token's position in float64 and quantised from there; V
// is quantised from its bf16 values; the query stays bf16, rotated and
// rounded exactly as the bf16 append does it.  Slot rule, skipping of a
// token whose slot a later token of the call takes, and slot_pos as in
// append_rope_kernel.
__global__ __launch_bounds__(kAppendThreads) void append_i8_kernel(AppendParams p,
                                                                   int wgs_per_token) {
  const int token = blockIdx.x / wgs_per_token;
  const int b = token / p.n_tokens;
  const int j = token - b * p.n_tokens;
  const int64_t pos = static_cast<int64_t>(p.pos[b]) + j;
  if (pos < 0 || pos > INT32_MAX) return;
  const int d = p.head_dim;
  const int half = d / 2;
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x - token * wgs_per_token) * (kAppendThreads / 64) + (threadIdx.x >> 6);
  const int slots = p.sinks + p.window;
  const bool overwritten = pos >= p.sinks && j + p.window <= p.n_tokens - 1;
  const int slot = pos < p.sinks ? static_cast<int>(pos) : p.sinks + static_cast<int>(pos % p.window);
  const bool active = lane < half;
  double sn = 0.0, cs = 1.0;
  if (active) rope_sincos(static_cast<double>(pos), p.freq.theta[lane], &sn, &cs);
  int e0 = 0, e1 = 0;
  pair_elems(active ? lane : 0, half, p.rope_half, &e0, &e1);
  const int q_rows = p.q_inout != nullptr ? p.num_q_heads : 0;
  const int rows = 2 * p.num_kv_heads + q_rows;
  for (int r = wave; r < rows; r += wgs_per_token * (kAppendThreads / 64)) {
    if (r < 2 * p.num_kv_heads) {
      if (overwritten) continue;
      const bool is_v = r >= p.num_kv_heads;
      const int h = is_v ? r - p.num_kv_heads : r;
      const uint16_t* src = static_cast<const uint16_t*>(is_v ? p.v_new : p.k_new) +
                            ((static_cast<size_t>(b) * p.n_tokens + j) * p.num_kv_heads + h) * d;
      double x0 = 0.0, x1 = 0.0;
      if (active) {
        x0 = static_cast<double>(bf16_to_f32(src[e0]));
        x1 = static_cast<double>(bf16_to_f32(src[e1]));
        if (!is_v) rope_rotate_pair(x0, x1, cs, sn, &x0, &x1);
      }
      const size_t row = (static_cast<size_t>(b) * p.num_kv_heads + h) * slots + slot;
      quantize_row_store(x0, x1, active, e0, e1,
                         static_cast<int8_t*>(is_v ? p.v_cache : p.k_cache) + row * d,
                         (is_v ? p.v_scale : p.k_scale) + row);
      if (!is_v && h == 0 && lane == 0)
        p.slot_pos[static_cast<size_t>(b) * slots + slot] = static_cast<int32_t>(pos);
    } else if (active) {
      const int h = r - 2 * p.num_kv_heads;
      const size_t qrow = ((static_cast<size_t>(b) * p.n_tokens + j) * p.num_q_heads + h) * d;
      const uint16_t* q = static_cast<const uint16_t*>(p.q_inout) + qrow;
      uint16_t* qo = static_cast<uint16_t*>(p.q_out != nullptr ? p.q_out : p.q_inout) + qrow;
      double o0, o1;
      rope_rotate_pair(static_cast<double>(bf16_to_f32(q[e0])),
                       static_cast<double>(bf16_to_f32(q[e1])), cs, sn, &o0, &o1);
      qo[e0] = f64_to_bf16_rne(o0);
      qo[e1] = f64_to_bf16_rne(o1);
    }
  }
}

// Pool write into int8 pools: one workgroup per token, one wave per K or V
// row; K rotated at pos[n] first when positions are given.
__global__ __launch_bounds__(kAppendThreads) void write_paged_i8_kernel(PagedWriteParams p) {
  const int n = blockIdx.x;
  const int64_t row = p.dst_rows[n];
  const int64_t rows_total = static_cast<int64_t>(p.num_phys_blocks) * p.block_size;
  if (row < 0 || row >= rows_total) return;
  const bool rotate = p.pos != nullptr;
  const int32_t pos = rotate ? p.pos[n] : 0;
  if (pos < 0) return;
  const int d = p.head_dim;
  const int half = d / 2;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const bool active = lane < half;
  double sn = 0.0, cs = 1.0;
  if (rotate && active) rope_sincos(static_cast<double>(pos), p.freq.theta[lane], &sn, &cs);
  int e0 = 0, e1 = 0;
  pair_elems(active ? lane : 0, half, p.rope_half, &e0, &e1);
  const int64_t blk = row / p.block_size;
  const int rr = static_cast<int>(row - blk * p.block_size);
  for (int r = wave; r < 2 * p.num_kv_heads; r += kAppendThreads / 64) {
    const bool is_v = r >= p.num_kv_heads;
    const int h = is_v ? r - p.num_kv_heads : r;
    const uint16_t* src = static_cast<const uint16_t*>(is_v ? p.v_src : p.k_src) +
                          (static_cast<size_t>(n) * p.num_kv_heads + h) * d;
    double x0 = 0.0, x1 = 0.0;
    if (active) {
      x0 = static_cast<double>(bf16_to_f32(src[e0]));
      x1 = static_cast<double>(bf16_to_f32(src[e1]));
      if (!is_v && rotate) rope_rotate_pair(x0, x1, cs, sn, &x0, &x1);
    }
    const size_t out_row = (static_cast<size_t>(blk) * p.num_kv_heads + h) * p.block_size + rr;
    quantize_row_store(x0, x1, active, e0, e1,
                       static_cast<int8_t*>(is_v ? p.v_pool : p.k_pool) + out_row * d,
                       (is_v ? p.v_scale : p.k_scale) + out_row);
  }
}

__global__ void fill_i32_kernel(int32_t* dst, size_t n, int32_t value) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    dst[i] = value;
}

}  // namespace

hipError_t launch_fill_i32(int32_t* dst, size_t n, int32_t value, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  const unsigned grid = static_cast<unsigned>(blocks < 4096 ? blocks : 4096);
  fill_i32_kernel<<<grid, 256, 0, stream>>>(dst, n, value);
  return hipGetLastError();
}

hipError_t launch_append_rope(const AppendParams& p, hipStream_t stream) {
  const int half = p.head_dim / 2;
  const int elem = p.bf16 ? 2 : 4;
  const int copies = p.k_rotated != nullptr ? 2 : 1;  // V, and K when it is copied
  const int items = (p.k_rotated != nullptr ? 0 : p.num_kv_heads * half) +
                    (p.q_inout != nullptr ? p.num_q_heads * half : 0) +
                    copies * p.num_kv_heads * (p.head_dim * elem / 16);
  const int wgs = (items + kAppendThreads - 1) / kAppendThreads;
  const size_t grid = static_cast<size_t>(p.batch) * p.n_tokens * wgs;
  if (grid > 0x7fffffffu) return hipErrorInvalidValue;
  if (p.bf16)
    append_rope_kernel<true><<<static_cast<unsigned>(grid), kAppendThreads, 0, stream>>>(p, items, wgs);
  else
    append_rope_kernel<false><<<static_cast<unsigned>(grid), kAppendThreads, 0, stream>>>(p, items, wgs);
  return hipGetLastError();
}

hipError_t launch_append_i8(const AppendParams& p, hipStream_t stream) {
  const int rows = 2 * p.num_kv_heads + (p.q_inout != nullptr ? p.num_q_heads : 0);
  const int wgs = (rows + kAppendThreads / 64 - 1) / (kAppendThreads / 64);
  const size_t grid = static_cast<size_t>(p.batch) * p.n_tokens * wgs;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffffu) return hipErrorInvalidValue;
  append_i8_kernel<<<static_cast<unsigned>(grid), kAppendThreads, 0, stream>>>(p, wgs);
  return hipGetLastError();
}

hipError_t launch_write_paged_i8(const PagedWriteParams& p, hipStream_t stream) {
  if (p.n_tokens <= 0) return hipSuccess;
  write_paged_i8_kernel<<<static_cast<unsigned>(p.n_tokens), kAppendThreads, 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_append_paged(const AppendPagedParams& p, hipStream_t stream) {
  if (p.n_seqs <= 0 || p.n_tokens <= 0) return hipSuccess;
  const size_t grid = static_cast<size_t>(p.n_seqs) * p.n_tokens;
  if (grid > 0x7fffffffu) return hipErrorInvalidValue;
  if (p.bf16)
    append_paged_kernel<true><<<static_cast<unsigned>(grid), kAppendThreads, 0, stream>>>(p);
  else
    append_paged_kernel<false><<<static_cast<unsigned>(grid), kAppendThreads, 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_blocks_update(const BlocksUpdateParams& p, hipStream_t stream) {
  if (p.n_table <= 0 && p.n_lens <= 0 && p.n_cow <= 0) return hipSuccess;
  blocks_update_kernel<<<1 + 2 * p.n_cow, kAppendThreads, 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_write_paged(const PagedWriteParams& p, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(p.n_tokens);
  if (p.bf16)
    write_paged_kernel<true><<<grid, kAppendThreads, 0, stream>>>(p);
  else
    write_paged_kernel<false><<<grid, kAppendThreads, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace swa
