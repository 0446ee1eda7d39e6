// Chunked prefill over a ring cache (bf16, head_dim 128).
//
// T new tokens of each sequence, at positions p0 .. p0 + T - 1, attend what a
// decode step at their own position would see: token j (position t = p0 + j)
// attends the keys at positions p with p <= t and (p < S or p > t - W) --
// the sinks united with its window ([sink] cache formula; [ring] §2.2, the
// current token included) -- taken from the ring as it was before the chunk
// (positions < p0) and from the chunk itself (positions p0 .. t, causal
// within the chunk; [pool] "paging": prefill in chunks of 128-256 tokens).
// Then the chunk is appended as kv_append_rope appends it.  Unlike a decode
// step this is compute-bound: every key tile is used by a block of query rows.
//
// Three launches: (1) rotate the chunk's queries and K rows into the
// workspace (angles and rounding of the append kernel), (2) the attention,
// (3) the append of the chunk into the ring (after the attention has read
// the ring, since the chunk may overwrite slots that earlier queries of the
// chunk still see).
//
// Attention kernel.  A workgroup of 4 waves takes one (sequence, kv head) and
// a block of 128 / g tokens, i.e. up to 128 query rows (row rho = g * token +
// head; wave w owns the two 16-row blocks 32w .. 32w + 31), and streams the
// keys of the ring and then of the chunk in tiles of 64, double-buffered in
// LDS (the next tile's loads are in flight while the current one is used).
// Per tile and wave, with v_mfma_f32_16x16x32 (A: lane l holds
// A[l % 16][8(l / 16) .. +7], B: lane l holds B[8(l / 16) .. +7][l % 16],
// D: lane l register r holds D[4(l / 16) + r][l % 16]):
//   S^T = K Q^T in bf16 (exact products, fp32 accumulation): A = 16 keys of
//         the tile from LDS, B = 16 query rows (registers); every K operand
//         read from LDS serves both row blocks.  Lane l holds the scores of
//         query row l % 16 for keys 16 kb + 4(l / 16) + r.
//   mask (only in tiles that some row sees partly), online softmax per query
//         row: its 16 scores per lane, then the four lanes of the column.  The
//         running maximum m is raised only when a tile's maximum exceeds it by
//         more than 8 (log2 units), so the accumulators are rescaled rarely;
//         P = 2^(s c - m) <= 2^8 stays well inside fp16.
//   O^T += V^T P^T in fp16 with fp32 accumulation: B = P^T, the lane's own
//         probabilities, if the 32 keys of each product are taken in the order
//         kappa = 8 ((key % 16) / 4) + 4 (key / 16) + key % 4 -- the order the
//         lane holds them in; A = V^T in that key order, written to LDS
//         transposed (and converted to fp16) by the tile loader.  A ninth
//         product with A = ones gives the row sums of the same fp16 P.  P and
//         V in fp16 (11-bit significands) keep the rounding of P well inside
//         the tolerance; fp16's range limits |V| to below 65504.
// LDS layouts (16-byte units u of a row, stored at u ^ swizzle(row), so that
// the lanes of every read and write reach distinct banks and each lane's
// read addresses differ only by constants): K [64 keys][16 units], swizzle
// key % 16; V^T [128 dims][8 units], swizzle (d ^ (d / 4)) % 8.
// Each tile carries two flags, set by the loader from the key positions and
// the workgroup's first and last query positions: some key is not visible
// to every row (mask needed), some key is visible to some row (else the tile
// is skipped).
// The workgroups of one (sequence, kv head) are placed on one XCD (XCD of a
// workgroup = its index mod 8), so the tiles they all stream come through one
// L2.
#include <algorithm>

#include "device_common.h"
#include "swa_internal.h"

namespace swa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kKSteps = kD / 32;     // k-steps of one S^T product
constexpr int kKeys = 64;            // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRowBlocks = 2;        // 16-row blocks per wave
constexpr int kRows = 16 * kRowBlocks * kWaves;  // query rows per workgroup
constexpr int kXcds = 8;
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kRescaleSlack = 8.f;  // log2 units

struct Tile {
  u32x4_t k[kKeys * 16];  // K (bf16): unit c of key r at r * 16 + (c ^ (r % 16))
  u32x4_t vt[kD * 8];     // V^T (fp16): unit u of dim d at d * 8 + (u ^ vt_swizzle(d))
  int32_t pos[kKeys];    // positions: ring slots as recorded, chunk rows p0 + i; -1: no key
};

__device__ __forceinline__ int vt_swizzle(int d) { return (d ^ (d >> 2)) & 7; }

// Raw buffer resource over `bytes` bytes at `base` (loads beyond return 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

// Loads that write LDS: lane l of the wave stores its 16 bytes at lds + 16 l
// (lds is the same for the whole wave).
__device__ __forceinline__ void buffer_load_to_lds16(__amdgpu_buffer_rsrc_t rsrc, void* lds,
                                                     int voffset, int soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, lds, 16, voffset, soffset, 0, 0);
}
__device__ __forceinline__ void global_load_to_lds16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}
// Waits until every vector memory load of the wave, those that write LDS
// included, has completed.
__device__ __forceinline__ void wait_vector_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Maximum over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lanes of one
// column of an MFMA result).  permlane16_swap(x, x) leaves in every lane the
// pair {x of its own row, x of the neighbouring row} (rows of 16 lanes, 0-1
// and 2-3 paired); permlane32_swap(x, x) the pair {x, x of the other half}.
__device__ __forceinline__ float column_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(x);
  const auto c = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// The bf16 in the low (hi = false) or high half of w, as a float.
__device__ __forceinline__ float bf16_half_to_f32(uint32_t w, bool hi) {
  return __uint_as_float(hi ? (w & 0xffff0000u) : (w << 16));
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats to fp16 (round to nearest even), lo in the low half.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, f16x2_t));
}

// Rotation of the chunk: one workgroup per token.  The token's d/2 angles are
// formed once (one wave, into LDS); then each thread rotates four pairs of a
// head at a time, query heads first, then key heads.  Rounding as the append
// kernel: f64 rotation, one rounding to bf16.
__global__ __launch_bounds__(256) void rotate_chunk_kernel(RotateChunkParams p) {
  constexpr int kHalf = kD / 2;
  constexpr int kQuads = kHalf / 4;  // four pairs per thread and head
  __shared__ double s_cos[kHalf], s_sin[kHalf];
  const int64_t token = blockIdx.x;  // b * T + j
  const int b = static_cast<int>(token / p.n_tokens);
  const int j = static_cast<int>(token - static_cast<int64_t>(b) * p.n_tokens);
  const int64_t pos = static_cast<int64_t>(p.pos[b]) + j;
  const bool rot = pos >= 0 && pos <= INT32_MAX;  // a token at such a position is never attended
  if (threadIdx.x < kHalf) {
    double sn = 0.0, cs = 1.0;
    if (rot) rope_sincos(static_cast<double>(pos), p.freq.theta[threadIdx.x], &sn, &cs);
    s_cos[threadIdx.x] = cs;
    s_sin[threadIdx.x] = sn;
  }
  __syncthreads();
  auto rotate = [&](uint16_t& a, uint16_t& c, int i) {
    if (!rot) return;
    double x0, x1;
    rope_rotate_pair(static_cast<double>(bf16_to_f32(a)), static_cast<double>(bf16_to_f32(c)),
                     s_cos[i], s_sin[i], &x0, &x1);
    a = f64_to_bf16_rne(x0);
    c = f64_to_bf16_rne(x1);
  };
  const int heads = p.num_q_heads + p.num_kv_heads;
  for (int w = threadIdx.x; w < heads * kQuads; w += blockDim.x) {
    const int h = w / kQuads;
    const int i0 = 4 * (w - h * kQuads);  // pairs i0 .. i0 + 3
    const bool is_q = h < p.num_q_heads;
    const int hh = is_q ? h : h - p.num_q_heads;
    const int nh = is_q ? p.num_q_heads : p.num_kv_heads;
    const size_t row = (static_cast<size_t>(token) * nh + hh) * kD;
    const uint16_t* sr = static_cast<const uint16_t*>(is_q ? p.q : p.k) + row;
    uint16_t* dr = static_cast<uint16_t*>(is_q ? p.q_rot : p.k_rot) + row;
    if (p.rope_half) {  // pairs (i, i + d/2): four elements from each half
      uint2 lo = *reinterpret_cast<const uint2*>(sr + i0);
      uint2 hi = *reinterpret_cast<const uint2*>(sr + i0 + kHalf);
      uint16_t* l = reinterpret_cast<uint16_t*>(&lo);
      uint16_t* u = reinterpret_cast<uint16_t*>(&hi);
#pragma unroll
      for (int e = 0; e < 4; ++e) rotate(l[e], u[e], i0 + e);
      *reinterpret_cast<uint2*>(dr + i0) = lo;
      *reinterpret_cast<uint2*>(dr + i0 + kHalf) = hi;
    } else {            // pairs (2i, 2i + 1): eight neighbouring elements
      uint4 v = *reinterpret_cast<const uint4*>(sr + 2 * i0);
      uint16_t* e16 = reinterpret_cast<uint16_t*>(&v);
#pragma unroll
      for (int e = 0; e < 4; ++e) rotate(e16[2 * e], e16[2 * e + 1], i0 + e);
      *reinterpret_cast<uint4*>(dr + 2 * i0) = v;
    }
  }
}

template <int G>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillParams p) {
  constexpr int TB = kRows / G;  // tokens per workgroup
  __shared__ Tile tiles[2];

  // XCD-aware placement: the k-th workgroup on XCD x takes token block
  // k % token_blocks of unit (k / token_blocks) * 8 + x.
  const int xcd = blockIdx.x % kXcds;
  const int kx = blockIdx.x / kXcds;
  const int unit = (kx / p.token_blocks) * kXcds + xcd;
  const int tblk = kx % p.token_blocks;
  if (unit >= p.batch * p.num_kv_heads) return;
  const int b = unit / p.num_kv_heads;
  const int kvh = unit - b * p.num_kv_heads;
  const int T = p.n_tokens;
  const int j0 = tblk * TB;
  if (j0 >= T) return;
  const int j_last = min(j0 + TB, T) - 1;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lq = lane >> 4;
  const int lc = lane & 15;
  const int32_t p0 = p.pos[b];
  const int64_t t_first = static_cast<int64_t>(p0) + j0;  // query positions of the block
  const int64_t t_last = static_cast<int64_t>(p0) + j_last;

  // This lane's query row in each row block.  t_row = -1: the row sees no
  // key (no such row, or its position is negative or beyond 2^31 - 1).
  bool row_ok[kRowBlocks];
  int32_t t_row[kRowBlocks], t_win[kRowBlocks];
  size_t qrow[kRowBlocks];
  bf16x8_t qop[kRowBlocks][kKSteps];  // B operand of S^T
#pragma unroll
  for (int rb = 0; rb < kRowBlocks; ++rb) {
    const int rho = 32 * wave + 16 * rb + lc;
    const int jr = j0 + rho / G;
    row_ok[rb] = rho < TB * G && jr < T;
    const int64_t t = static_cast<int64_t>(p0) + jr;
    t_row[rb] = row_ok[rb] && t >= 0 && t <= INT32_MAX ? static_cast<int32_t>(t) : -1;
    t_win[rb] = t_row[rb] - p.window;  // no overflow: window <= 2^31 - 1
    qrow[rb] = (static_cast<size_t>(b) * T + jr) * p.num_q_heads +
               static_cast<size_t>(kvh) * G + rho % G;
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) {
      Vec16 v{};
      if (row_ok[rb])
        v = load16(static_cast<const uint16_t*>(p.q_rot) + qrow[rb] * kD + 32 * s + 8 * lq);
      qop[rb][s] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // Keys: ring slots 0 .. slots-1, then chunk rows 0 .. j_last.
  const int n_keys = p.slots + j_last + 1;
  const int n_tiles = (n_keys + kKeys - 1) / kKeys;
  const size_t ring_row0 = static_cast<size_t>(unit) * p.slots;  // row (b, kvh, slot 0)
  const int32_t* sp = p.slot_pos + static_cast<size_t>(b) * p.slots;
  const size_t chunk_row0 = static_cast<size_t>(b) * T * p.num_kv_heads + kvh;
  const size_t chunk_stride = static_cast<size_t>(p.num_kv_heads) * kD;  // elements per chunk row
  const uint32_t chunk_row_bytes = static_cast<uint32_t>(chunk_stride * 2);
  const uint32_t ring_bytes = static_cast<uint32_t>(p.slots) * kD * 2;
  const uint32_t chunk_bytes = static_cast<uint32_t>(T - 1) * chunk_row_bytes + kD * 2;
  const __amdgpu_buffer_rsrc_t k_ring =
      buffer_rsrc(static_cast<const uint16_t*>(p.k_cache) + ring_row0 * kD, ring_bytes);
  const __amdgpu_buffer_rsrc_t v_ring =
      buffer_rsrc(static_cast<const uint16_t*>(p.v_cache) + ring_row0 * kD, ring_bytes);
  const __amdgpu_buffer_rsrc_t sp_ring = buffer_rsrc(sp, static_cast<uint32_t>(p.slots) * 4);
  const __amdgpu_buffer_rsrc_t k_chunk =
      buffer_rsrc(static_cast<const uint16_t*>(p.k_rot) + chunk_row0 * kD, chunk_bytes);
  const __amdgpu_buffer_rsrc_t v_chunk =
      buffer_rsrc(static_cast<const uint16_t*>(p.v_new) + chunk_row0 * kD, chunk_bytes);

  // Tile loader.  K goes straight from memory to LDS (loads that write LDS:
  // lane l of a wave's instruction fills the 16 bytes at the wave's LDS base
  // + 16 l): instruction e of wave w fills K rows 16 e + 4 w .. + 3, so lane
  // (kq = tid / 16, kpart = tid % 16) fills physical unit kpart of key row
  // kq + 16 e, i.e. fetches that row's logical unit kpart ^ kq.  V: thread
  // moves dims 4 vd .. 4 vd + 3
  // (vd = tid % 32) of the eight keys whose kappa positions in PV chunk vc
  // are 8 vj .. 8 vj + 7 (tid / 32 = 4 vc + vj): keys 32 vc + 4 vj + i and
  // 32 vc + 16 + 4 vj + i (i < 4), and their positions.  Tiles wholly in the
  // ring or wholly in the chunk's rows take the per-tile offset in a scalar
  // register (buffer loads); the others form each row's address.
  const int kpart = tid & 15;
  const int kq = tid >> 4;
  const int vd = tid & 31;
  const int vc = tid >> 7;
  const int vj = (tid >> 5) & 3;
  const int vkey0 = 32 * vc + 4 * vj;
  const int k_unit = kpart ^ kq;  // logical unit of K that this lane fetches
  u32x2_t vreg[8];
  int32_t vpos[8];
  auto v_key = [&](int i) { return vkey0 + 16 * (i >> 2) + (i & 3); };
  auto load = [&](int tile) {
    const int base = tile * kKeys;
    u32x4_t* k_lds = &tiles[tile & 1].k[(4 * wave) * 16];  // this wave's rows 4w .. 4w + 3
    if (base + kKeys <= p.slots) {  // the whole tile from the ring (uniform branch)
      const int sb = base * kD * 2;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        buffer_load_to_lds16(k_ring, k_lds + 256 * e, kq * 256 + k_unit * 16, sb + 4096 * e);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        vreg[i] = __builtin_amdgcn_raw_buffer_load_b64(v_ring, vkey0 * 256 + vd * 8 + (i & 3) * 256,
                                                       sb + 4096 * (i >> 2), 0);
      const i32x4_t r0 = __builtin_bit_cast(
          i32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sp_ring, vkey0 * 4, base * 4, 0));
      const i32x4_t r1 = __builtin_bit_cast(
          i32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sp_ring, vkey0 * 4 + 64, base * 4, 0));
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // raw slot positions (-1: empty)
        vpos[i] = r0[i];
        vpos[4 + i] = r1[i];
      }
      return;
    }
    const int i0 = base - p.slots;  // chunk row of the tile's first key
    if (i0 >= 0 && i0 + kKeys - 1 <= j_last) {  // the whole tile from the chunk (uniform)
      const int sb = i0 * static_cast<int>(chunk_row_bytes);
      const int rs = static_cast<int>(chunk_row_bytes);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        buffer_load_to_lds16(k_chunk, k_lds + 256 * e, kq * rs + k_unit * 16, sb + 16 * rs * e);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        vreg[i] = __builtin_amdgcn_raw_buffer_load_b64(v_chunk, vkey0 * rs + vd * 8,
                                                       sb + rs * (16 * (i >> 2) + (i & 3)), 0);
        const int64_t cp = static_cast<int64_t>(p0) + i0 + v_key(i);
        vpos[i] = ((cp >= 0) & (cp <= INT32_MAX)) ? static_cast<int32_t>(cp) : -1;
      }
      return;
    }
    // Ring rows, chunk rows, and past the end the last chunk row (absent key).
    auto row = [&](int kk, const void* ring, const void* chunk) {
      const int i = min(max(kk - p.slots, 0), j_last);
      const uint16_t* r = static_cast<const uint16_t*>(ring) + (ring_row0 + kk) * kD;
      const uint16_t* c = static_cast<const uint16_t*>(chunk) + chunk_row0 * kD + i * chunk_stride;
      return kk < p.slots ? r : c;
    };
#pragma unroll
    for (int e = 0; e < 4; ++e)
      global_load_to_lds16(row(base + kq + 16 * e, p.k_cache, p.k_rot) + 8 * k_unit,
                           k_lds + 256 * e);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int kk = base + v_key(i);
      vreg[i] = *reinterpret_cast<const u32x2_t*>(row(kk, p.v_cache, p.v_new) + 4 * vd);
      const int32_t rp = sp[min(kk, p.slots - 1)];
      const int64_t cp = static_cast<int64_t>(p0) + (kk - p.slots);
      const bool chunk_ok = (kk < n_keys) & (cp >= 0) & (cp <= INT32_MAX);
      vpos[i] = kk < p.slots ? rp : (chunk_ok ? static_cast<int32_t>(cp) : -1);
    }
  };
  auto store = [&](int buf) {
    Tile& t = tiles[buf];
    // An absent key's V bytes are whatever the memory held; its weight is 0,
    // but 0 * NaN is not, so such rows enter P V as zeros.
    bool live = true;
#pragma unroll
    for (int i = 0; i < 8; ++i) live &= vpos[i] >= 0;
    if (!__all(live)) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (vpos[i] < 0) vreg[i] = u32x2_t{0u, 0u};
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d = 4 * vd + r;
      uint32_t w[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t a = r < 2 ? vreg[2 * m].x : vreg[2 * m].y;
        const uint32_t c = r < 2 ? vreg[2 * m + 1].x : vreg[2 * m + 1].y;
        w[m] = pack_f16x2(bf16_half_to_f32(a, r & 1), bf16_half_to_f32(c, r & 1));
      }
      t.vt[d * 8 + ((4 * vc + vj) ^ vt_swizzle(d))] = u32x4_t{w[0], w[1], w[2], w[3]};
    }
    if (vd == 0) {
      *reinterpret_cast<i32x4_t*>(&t.pos[32 * vc + 4 * vj]) =
          i32x4_t{vpos[0], vpos[1], vpos[2], vpos[3]};
      *reinterpret_cast<i32x4_t*>(&t.pos[32 * vc + 16 + 4 * vj]) =
          i32x4_t{vpos[4], vpos[5], vpos[6], vpos[7]};
    }
  };

  // Per-lane LDS read offsets (in uint4 units) of the MFMA A operands.
  int k_off[kKSteps];
#pragma unroll
  for (int s = 0; s < kKSteps; ++s) k_off[s] = lc * 16 + ((4 * s + lq) ^ lc);
  const int vt_g = (lc ^ (lc >> 2)) & 7;
  const int vt_off[2] = {lc * 8 + ((0 + lq) ^ vt_g), lc * 8 + ((4 + lq) ^ vt_g)};

  const float c = p.score_scale_log2;
  float m[kRowBlocks];   // running maximum of the row's scaled scores (log2 units)
  f32x4_t acc[kRowBlocks][kD / 16 + 1];  // O^T blocks, then the row sums
#pragma unroll
  for (int rb = 0; rb < kRowBlocks; ++rb) {
    m[rb] = kNegInf;
#pragma unroll
    for (int blk = 0; blk <= kD / 16; ++blk) acc[rb][blk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  f16x8_t ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = static_cast<_Float16>(1.f);

  // A key at position kp (-1: none) is visible to every query row of the
  // workgroup iff it lies in [0, all_a] or [all_b, t_first], and to some row
  // iff it lies in [0, any_a] or [any_b, t_last] (sinks, then the window;
  // empty intervals have a < 0 or b > end).
  const int64_t sink_end = static_cast<int64_t>(p.sinks) - 1;
  const int32_t t_lo = static_cast<int32_t>(min<int64_t>(max<int64_t>(t_first, -1), INT32_MAX));
  const int32_t t_hi = static_cast<int32_t>(min<int64_t>(max<int64_t>(t_last, -1), INT32_MAX));
  const int32_t all_a = static_cast<int32_t>(min<int64_t>(t_lo, sink_end));
  const int32_t any_a = static_cast<int32_t>(min<int64_t>(t_hi, sink_end));
  const int32_t all_b = static_cast<int32_t>(
      min<int64_t>(max<int64_t>(t_last - p.window + 1, 0), static_cast<int64_t>(INT32_MAX)));
  const int32_t any_b = static_cast<int32_t>(
      min<int64_t>(max<int64_t>(t_first - p.window + 1, 0), static_cast<int64_t>(INT32_MAX)));
  auto in = [](int32_t x, int32_t a, int32_t b) {  // a <= x <= b (x >= -1, a >= 0)
    const uint32_t ua = static_cast<uint32_t>(a);
    return b >= a && static_cast<uint32_t>(x) - ua <= static_cast<uint32_t>(b) - ua;
  };

  load(0);
  store(0);
  wait_vector_loads();  // the K rows written to LDS by the loads
  __syncthreads();
  for (int it = 0; it < n_tiles; ++it) {
    const int cur = it & 1;
    const bool more = it + 1 < n_tiles;
    if (more) load(it + 1);
    const Tile& t = tiles[cur];
    const int tile_base = it * kKeys;
    // A ring slot holding a position at or after the chunk's start is
    // superseded by the chunk: no key.
    auto key_pos = [&](int32_t raw, int key) {
      return ((tile_base + key < p.slots) & (raw >= p0)) ? -1 : raw;
    };
    // Tile flags from the 64 key positions, one per lane: bit 0 some key is
    // not visible to every row (mask needed), bit 1 some key is visible.
    const int32_t kp_l = key_pos(t.pos[lane], lane);
    const bool all_l = in(kp_l, 0, all_a) || in(kp_l, all_b, t_lo);
    const bool any_l = in(kp_l, 0, any_a) || in(kp_l, any_b, t_hi);
    const int flags = (__ballot(!all_l) != 0 ? 1 : 0) | (__ballot(any_l) != 0 ? 2 : 0);
    if (flags & 2) {
      // S^T for the four 16-key blocks of the tile, both row blocks
      f32x4_t sc[kRowBlocks][4];
#pragma unroll
      for (int rb = 0; rb < kRowBlocks; ++rb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) sc[rb][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < kKSteps; ++s)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, t.k[k_off[s] + 256 * kb]);
#pragma unroll
          for (int rb = 0; rb < kRowBlocks; ++rb)
            sc[rb][kb] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[rb][s], sc[rb][kb], 0, 0, 0);
        }
      if (flags & 1) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const i32x4_t raw = *reinterpret_cast<const i32x4_t*>(&t.pos[16 * kb + 4 * lq]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int32_t kp = key_pos(raw[r], 16 * kb + 4 * lq + r);
#pragma unroll
            for (int rb = 0; rb < kRowBlocks; ++rb) {
              const bool vis = (kp >= 0) & (kp <= t_row[rb]) &
                               ((kp < p.sinks) | (kp > t_win[rb]));
              sc[rb][kb][r] = vis ? sc[rb][kb][r] : kNegInf;
            }
          }
        }
      }
      // online softmax: tile maximum per row, rare rescale, P = 2^(s c - m)
      float mt[kRowBlocks];
      bool need[kRowBlocks];
#pragma unroll
      for (int rb = 0; rb < kRowBlocks; ++rb) {
        float x = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) x = fmaxf(x, sc[rb][kb][r]);
        mt[rb] = column_max(x) * c;
        need[rb] = mt[rb] > m[rb] + kRescaleSlack;
      }
      if (__any(need[0] | need[1])) {
#pragma unroll
        for (int rb = 0; rb < kRowBlocks; ++rb) {
          const float mn = need[rb] ? mt[rb] : m[rb];
          const float alpha = need[rb] ? __builtin_amdgcn_exp2f(m[rb] - mn) : 1.f;
#pragma unroll
          for (int blk = 0; blk <= kD / 16; ++blk) acc[rb][blk] *= alpha;
          m[rb] = mn;
        }
      }
      float mu[kRowBlocks];
#pragma unroll
      for (int rb = 0; rb < kRowBlocks; ++rb) mu[rb] = m[rb] == kNegInf ? 0.f : m[rb];
      // P for the keys of PV chunk pc (key blocks 2 pc, 2 pc + 1)
      f16x8_t pb[kRowBlocks][2];
      auto probs = [&](int pc) __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < kRowBlocks; ++rb)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              pb[rb][pc][4 * h + r] = static_cast<_Float16>(
                  __builtin_amdgcn_exp2f(fmaf(sc[rb][2 * pc + h][r], c, -mu[rb])));
      };
      // O^T += V^T P^T over PV chunk pc, and the row sums
      auto pv = [&](int pc) __attribute__((always_inline)) {
#pragma unroll
        for (int blk = 0; blk < kD / 16; ++blk) {
          const f16x8_t a =
              __builtin_bit_cast(f16x8_t, t.vt[vt_off[pc ^ (blk & 1)] + 128 * blk]);
#pragma unroll
          for (int rb = 0; rb < kRowBlocks; ++rb)
            acc[rb][blk] =
                __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pb[rb][pc], acc[rb][blk], 0, 0, 0);
        }
#pragma unroll
        for (int rb = 0; rb < kRowBlocks; ++rb)
          acc[rb][kD / 16] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb[rb][pc],
                                                                    acc[rb][kD / 16], 0, 0, 0);
      };
      probs(0);
      pv(0);
      probs(1);
      pv(1);
    }
    if (more) store(cur ^ 1);  // that buffer was last read in tile it - 1
    wait_vector_loads();
    __syncthreads();
  }

  // out = O / l
#pragma unroll
  for (int rb = 0; rb < kRowBlocks; ++rb) {
    if (!row_ok[rb]) continue;
    const float l = acc[rb][kD / 16][0];
    const bool seen = t_row[rb] >= 0 && l > 0.f;
    const float inv = seen ? 1.f / l : 0.f;
#pragma unroll
    for (int blk = 0; blk < kD / 16; ++blk) {
      const size_t at = qrow[rb] * kD + 16 * blk + 4 * lq;
      const f32x4_t o = acc[rb][blk] * inv;
      if (p.out_bf16) {
        uint16_t* dst = static_cast<uint16_t*>(p.out) + at;
        *reinterpret_cast<uint2*>(dst) =
            make_uint2(static_cast<uint32_t>(f32_to_bf16_rne(o[0])) |
                           (static_cast<uint32_t>(f32_to_bf16_rne(o[1])) << 16),
                       static_cast<uint32_t>(f32_to_bf16_rne(o[2])) |
                           (static_cast<uint32_t>(f32_to_bf16_rne(o[3])) << 16));
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(p.out) + at) =
            make_float4(o[0], o[1], o[2], o[3]);
      }
    }
    if (p.lse != nullptr && lq == 0)
      p.lse[qrow[rb]] = seen ? (m[rb] + __log2f(l)) * kLn2 : kNegInf;
  }
}

}  // namespace

PrefillLayout prefill_layout(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t n_tokens) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t rows = static_cast<size_t>(batch) * n_tokens;
  PrefillLayout l;
  l.q_offset = 0;
  l.k_offset = up(rows * num_q_heads * head_dim * sizeof(uint16_t));
  l.total = l.k_offset + up(rows * num_kv_heads * head_dim * sizeof(uint16_t));
  return l;
}

hipError_t launch_rotate_chunk(const RotateChunkParams& p, hipStream_t stream) {
  const int64_t tokens = static_cast<int64_t>(p.batch) * p.n_tokens;
  if (tokens == 0) return hipSuccess;
  if (tokens > 0x7fffffff) return hipErrorInvalidValue;
  rotate_chunk_kernel<<<static_cast<unsigned>(tokens), 256, 0, stream>>>(p);
  return hipGetLastError();
}

int prefill_tokens_per_block(int group) { return kRows / group; }

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  const int units = p.batch * p.num_kv_heads;
  const int64_t grid =
      static_cast<int64_t>((units + kXcds - 1) / kXcds) * kXcds * p.token_blocks;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const unsigned g = static_cast<unsigned>(grid);
  switch (p.num_q_heads / p.num_kv_heads) {
    case 1: prefill_kernel<1><<<g, kThreads, 0, stream>>>(p); break;
    case 2: prefill_kernel<2><<<g, kThreads, 0, stream>>>(p); break;
    case 3: prefill_kernel<3><<<g, kThreads, 0, stream>>>(p); break;
    case 4: prefill_kernel<4><<<g, kThreads, 0, stream>>>(p); break;
    case 6: prefill_kernel<6><<<g, kThreads, 0, stream>>>(p); break;
    case 8: prefill_kernel<8><<<g, kThreads, 0, stream>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace swa
