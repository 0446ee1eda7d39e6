// Chunked prefill over a ring cache (bf16, head_dim 128).
//
// T new tokens of each sequence, at positions p0 .. p0 + T - 1, attend what a
// decode step at their own position would see: token j (position t = p0 + j)
// attends the keys at positions p with p <= t and (p < S or p > t - W) --
// the sinks united with its window ([sink] cache formula; [ring] §2.2, the
// current token included) -- taken from the ring as it was before the chunk
// (positions < p0) and from the chunk itself (positions p0 .. t, causal
// within the chunk; [pool] chunked prefill).  Then the chunk is appended as
// kv_append_rope appends it.  Unlike a decode step this is compute-bound:
// every key tile is used by a block of query rows.
//
// Three launches: (1) rotate the chunk's queries and K rows into the
// workspace (angles and rounding of the append kernel), (2) the attention,
// (3) the append of the chunk into the ring (after the attention has read
// the ring, since the chunk may overwrite slots that earlier queries of the
// chunk still see).
//
// Attention kernel.  A workgroup of 4 waves takes one (sequence, kv head) and
// a block of 64 / g tokens, i.e. up to 64 query rows (row rho = g * token +
// head, wave w owning rows 16w .. 16w + 15), and streams the keys of the ring
// and then of the chunk in tiles of 32, double-buffered in LDS (the next
// tile's loads are in flight while the current one is used).  Per tile and
// wave, with v_mfma_f32_16x16x32 (A: lane l holds A[l % 16][8(l / 16) .. +7],
// B: lane l holds B[8(l / 16) .. +7][l % 16], D: lane l register r holds
// D[4(l / 16) + r][l % 16]):
//   S^T = K Q^T in bf16 (exact products, fp32 accumulation): A = 16 keys of
//         the tile from LDS (chunk c of key r stored at c ^ (r & 15), so the
//         16 lanes of a row read 16 different bank groups), B = the wave's 16
//         query rows (registers).  Lane l holds the scores of query row
//         l % 16 for keys 4(l / 16) + r of each 16-key half.
//   mask, online softmax per query row (its 8 scores per lane, then the four
//         lanes of the column), P = 2^(x - m).
//   O^T += V^T P^T in fp16 with fp32 accumulation: B = P^T, the lane's own 8
//         probabilities, if the keys of the PV product are taken in the order
//         kappa = 8 (r / 4) + 4 (key / 16) + r % 4 (r = key % 16) -- the
//         order the lane holds them in; A = V^T in that key order, which the
//         tile loader writes to LDS transposed (and converted to fp16) so a
//         lane reads its operand with one 16-byte access.  P and V in fp16
//         (11-bit significands) keep the rounding of P well inside the
//         tolerance; fp16's range limits |V| to below 65504.
// The workgroups of one (sequence, kv head) are placed on one XCD (XCD of a
// workgroup = its index mod 8), so the tiles they all stream come through one
// L2.
#include "device_common.h"
#include "swa_internal.h"

namespace swa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kKSteps = kD / 32;
constexpr int kKeys = 32;            // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRows = 16 * kWaves;   // query rows per workgroup
constexpr int kVtStride = 40;        // fp16 per transposed V row (32 keys + 8 of padding)
constexpr int kXcds = 8;
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309417f;

struct Tile {
  uint4 k[kKeys * 16];                                // K: chunk c of key r at r * 16 + (c ^ (r & 15))
  __attribute__((aligned(16))) uint16_t vt[kD * kVtStride];  // V^T in fp16: [dim][kappa]
  int32_t pos[kKeys];                                 // key positions, -1: no key
};

__device__ __forceinline__ int kappa(int key) {
  return 8 * ((key & 15) >> 2) + 4 * (key >> 4) + (key & 3);
}

__device__ __forceinline__ uint16_t f16_bits_from_bf16(uint16_t x) {
  const _Float16 h = static_cast<_Float16>(bf16_to_f32(x));
  return __builtin_bit_cast(uint16_t, h);
}

__global__ __launch_bounds__(256) void rotate_chunk_kernel(RotateChunkParams p) {
  constexpr int kHalf = kD / 2;
  const int heads = p.num_q_heads + p.num_kv_heads;
  const int64_t items = static_cast<int64_t>(p.batch) * p.n_tokens * heads * kHalf;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (w >= items) return;
  const int i = static_cast<int>(w % kHalf);
  const int64_t row = w / kHalf;  // (b, j, head)
  const int h = static_cast<int>(row % heads);
  const int64_t bj = row / heads;
  const int b = static_cast<int>(bj / p.n_tokens);
  const int j = static_cast<int>(bj - static_cast<int64_t>(b) * p.n_tokens);
  const int64_t pos = static_cast<int64_t>(p.pos[b]) + j;
  const uint16_t* src;
  uint16_t* dst;
  if (h < p.num_q_heads) {
    const size_t off = (static_cast<size_t>(bj) * p.num_q_heads + h) * kD;
    src = static_cast<const uint16_t*>(p.q) + off;
    dst = static_cast<uint16_t*>(p.q_rot) + off;
  } else {
    const size_t off = (static_cast<size_t>(bj) * p.num_kv_heads + (h - p.num_q_heads)) * kD;
    src = static_cast<const uint16_t*>(p.k) + off;
    dst = static_cast<uint16_t*>(p.k_rot) + off;
  }
  const int i0 = p.rope_half ? i : 2 * i;
  const int i1 = p.rope_half ? i + kHalf : 2 * i + 1;
  uint16_t o0 = src[i0], o1 = src[i1];
  if (pos >= 0 && pos <= INT32_MAX) {  // a token at a negative position is never attended
    double sn, cs, x0, x1;
    rope_sincos(static_cast<double>(pos), p.freq.theta[i], &sn, &cs);
    rope_rotate_pair(static_cast<double>(bf16_to_f32(o0)), static_cast<double>(bf16_to_f32(o1)),
                     cs, sn, &x0, &x1);
    o0 = f64_to_bf16_rne(x0);
    o1 = f64_to_bf16_rne(x1);
  }
  dst[i0] = o0;
  dst[i1] = o1;
}

template <int G>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillParams p) {
  constexpr int TB = kRows / G;  // tokens per workgroup
  __shared__ Tile tiles[2];

  // XCD-aware placement: the k-th workgroup on XCD x takes token block
  // k % token_blocks of unit (k / token_blocks) * 8 + x.
  const int xcd = blockIdx.x % kXcds;
  const int kx = blockIdx.x / kXcds;
  const int unit = (kx / p.token_blocks) * kXcds + xcd;
  const int tb = kx % p.token_blocks;
  if (unit >= p.batch * p.num_kv_heads) return;
  const int b = unit / p.num_kv_heads;
  const int kvh = unit - b * p.num_kv_heads;
  const int T = p.n_tokens;
  const int j0 = tb * TB;
  if (j0 >= T) return;
  const int j_last = min(j0 + TB, T) - 1;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lq = lane >> 4;
  const int lc = lane & 15;
  const int rho = 16 * wave + lc;  // this lane's query row
  const int jr = j0 + rho / G;
  const int hr = rho % G;
  const bool row_ok = rho < TB * G && jr < T;
  const int32_t p0 = p.pos[b];
  const int64_t t_row = static_cast<int64_t>(p0) + jr;  // the row's query position
  const size_t qrow = (static_cast<size_t>(b) * T + jr) * p.num_q_heads +
                      static_cast<size_t>(kvh) * G + hr;

  // B operand of S^T: the wave's 16 query rows.
  bf16x8_t qop[kKSteps];
#pragma unroll
  for (int s = 0; s < kKSteps; ++s) {
    Vec16 v{};
    if (row_ok) v = load16(static_cast<const uint16_t*>(p.q_rot) + qrow * kD + 32 * s + 8 * lq);
    qop[s] = __builtin_bit_cast(bf16x8_t, v);
  }

  // Keys: ring slots 0 .. slots-1, then chunk rows 0 .. j_last.
  const int n_keys = p.slots + j_last + 1;
  const int n_tiles = (n_keys + kKeys - 1) / kKeys;
  const size_t ring_row0 = static_cast<size_t>(unit) * p.slots;  // row (b, kvh, slot 0)
  const int32_t* sp = p.slot_pos + static_cast<size_t>(b) * p.slots;

  // Tile loader: thread tid moves 16-byte chunk tid % 16 of keys tid / 16 and
  // tid / 16 + 16, of K and of V; the thread with chunk 0 also moves the two
  // keys' positions.
  const int part = tid & 15;
  Vec16 kreg[2], vreg[2];
  int32_t kp[2];
  auto load = [&](int tile) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int key = (tid >> 4) + 16 * e;
      const int kk = tile * kKeys + key;
      kreg[e] = Vec16{};
      vreg[e] = Vec16{};
      kp[e] = -1;
      if (kk < p.slots) {
        const size_t off = (ring_row0 + kk) * kD + 8 * part;
        kreg[e] = load16(static_cast<const uint16_t*>(p.k_cache) + off);
        vreg[e] = load16(static_cast<const uint16_t*>(p.v_cache) + off);
        const int32_t pp = sp[kk];
        kp[e] = pp < p0 ? pp : -1;  // a position the chunk brings again is taken from the chunk
      } else if (kk < n_keys) {
        const int i = kk - p.slots;
        const size_t off =
            ((static_cast<size_t>(b) * T + i) * p.num_kv_heads + kvh) * kD + 8 * part;
        kreg[e] = load16(static_cast<const uint16_t*>(p.k_rot) + off);
        vreg[e] = load16(static_cast<const uint16_t*>(p.v_new) + off);
        const int64_t pp = static_cast<int64_t>(p0) + i;
        kp[e] = pp >= 0 && pp <= INT32_MAX ? static_cast<int32_t>(pp) : -1;
      }
    }
  };
  auto store = [&](int buf) {
    Tile& t = tiles[buf];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int key = (tid >> 4) + 16 * e;
      t.k[key * 16 + (part ^ (key & 15))] =
          make_uint4(kreg[e].w[0], kreg[e].w[1], kreg[e].w[2], kreg[e].w[3]);
      const int kap = kappa(key);
      // An empty slot's V bytes are whatever the allocation held; its weight is
      // 0, but 0 * NaN is not, so such rows enter P V as zeros.
      const bool live = kp[e] >= 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t wv = live ? vreg[e].w[q] : 0u;
        t.vt[(8 * part + 2 * q) * kVtStride + kap] = f16_bits_from_bf16(static_cast<uint16_t>(wv));
        t.vt[(8 * part + 2 * q + 1) * kVtStride + kap] =
            f16_bits_from_bf16(static_cast<uint16_t>(wv >> 16));
      }
      if (part == 0) t.pos[key] = kp[e];
    }
  };

  const float c = p.score_scale_log2;
  float m = kNegInf;  // running max of this lane's row (log2 units)
  float lsum = 0.f;   // this lane's share of the row's running sum
  f32x4_t acc[kD / 16];
#pragma unroll
  for (int blk = 0; blk < kD / 16; ++blk) acc[blk] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  load(0);
  store(0);
  __syncthreads();
  for (int it = 0; it < n_tiles; ++it) {
    const int cur = it & 1;
    if (it + 1 < n_tiles) load(it + 1);
    const Tile& t = tiles[cur];

    // S^T for the two 16-key halves
    f32x4_t d[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      d[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < kKSteps; ++s) {
        const uint4 a = t.k[(16 * kb + lc) * 16 + ((4 * s + lq) ^ lc)];
        d[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), qop[s],
                                                        d[kb], 0, 0, 0);
      }
    }
    // mask and running max of the lane's row
    float x[2][4];
    float tmax = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int32_t kpos = t.pos[16 * kb + 4 * lq + r];
        const bool vis = row_ok && kpos >= 0 && kpos <= t_row &&
                         (kpos < p.sinks || kpos > t_row - p.window);
        x[kb][r] = vis ? d[kb][r] * c : kNegInf;
        tmax = fmaxf(tmax, x[kb][r]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float mn = fmaxf(m, tmax);
    const float alpha = mn == kNegInf ? 1.f : exp2f(m - mn);
    m = mn;
    f16x8_t pb;
    float tsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pr = x[kb][r] == kNegInf ? 0.f : exp2f(x[kb][r] - mn);
        tsum += pr;
        pb[4 * kb + r] = static_cast<_Float16>(pr);
      }
    lsum = lsum * alpha + tsum;
    // O^T = O^T * alpha + V^T P^T
#pragma unroll
    for (int blk = 0; blk < kD / 16; ++blk) {
      const uint4 a = *reinterpret_cast<const uint4*>(&t.vt[(16 * blk + lc) * kVtStride + 8 * lq]);
      f32x4_t o = acc[blk] * alpha;
      acc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), pb, o,
                                                        0, 0, 0);
    }
    if (it + 1 < n_tiles) store(cur ^ 1);  // that buffer was last read before the barrier below
    __syncthreads();
  }

  // Row totals over the four lanes of the column, then out = O / l.
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (!row_ok) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
  for (int blk = 0; blk < kD / 16; ++blk) {
    const size_t at = qrow * kD + 16 * blk + 4 * lq;
    if (p.out_bf16) {
      uint16_t* o = static_cast<uint16_t*>(p.out) + at;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = f32_to_bf16_rne(acc[blk][r] * inv);
    } else {
      float* o = static_cast<float*>(p.out) + at;
      *reinterpret_cast<float4*>(o) =
          make_float4(acc[blk][0] * inv, acc[blk][1] * inv, acc[blk][2] * inv, acc[blk][3] * inv);
    }
  }
  if (p.lse != nullptr && lq == 0) p.lse[qrow] = lsum > 0.f ? (m + __log2f(lsum)) * kLn2 : kNegInf;
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
  const int64_t items = static_cast<int64_t>(p.batch) * p.n_tokens *
                        (p.num_q_heads + p.num_kv_heads) * (kD / 2);
  const int64_t grid = (items + 255) / 256;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  rotate_chunk_kernel<<<static_cast<unsigned>(grid), 256, 0, stream>>>(p);
  return hipGetLastError();
}

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
