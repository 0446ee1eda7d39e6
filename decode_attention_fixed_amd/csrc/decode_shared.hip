// Shared-prefix pass of the paged decode (bf16 pools, head_dim 128).
//
// Requests with a common prefix point at the same physical blocks ([share]
// §3.2, prefix sharing through identical block ids).  Attending each
// sequence's rows separately reads such a block once per sequence; this pass
// reads it once per kv head and scores it against the queries of every
// sequence that shares it.
//
// Plan (found per call, on the device, by every workgroup alike; workgroup 0
// writes it to the workspace for the launches that follow):
//   reference  the longest sequence (lowest index on ties);
//   P_b        for b != reference, the number of leading block-table entries
//              j that name the same physical block as the reference's entry j,
//              both in range and valid, j below both sequences' block counts
//              (at most kPrefixMaxRows rows are scanned);
//   shared     S = max P_b blocks; rows [0, min(S bs, len_ref)) of the
//              reference's table are the shared region (nothing when S = 0);
//   sharers    every b with P_b > 0 sees rows [0, min(P_b bs, len_b)) of the
//              region, the reference rows [0, min(S bs, len_ref)).  Those rows
//              are exactly the rows of b that the block table places there,
//              so attention over them here plus attention over b's other rows
//              in the pool kernel, combined by log-sum-exp, is attention over
//              all of b's rows.
//
// Attention (one workgroup per kv head, key chunk and block of 128 query
// columns): a column is one query head of one sharer; the shared region of a
// kv head is cut into prefix_chunks(B, Hq, Hkv) chunks of whole 64-key tiles.  Per tile,
// staged in LDS (double-buffered) and with v_mfma_f32_16x16x32_bf16 (A: lane
// l holds A[l % 16][8(l / 16) .. +7], B: lane l holds B[8(l / 16) .. +7][l %
// 16], D: lane l register r holds D[4(l / 16) + r][l % 16]):
//   S^T = K Q^T  A = 16 keys of the tile (LDS), B = 16 query columns (wave w
//                of the eight holds columns 16w .. 16w + 15; two waves share
//                a SIMD, so one's VALU work overlaps the other's products);
//   mask         key index beyond the column's shared rows: -inf (only in
//                tiles that some column sees partly);
//   softmax      online per column, the running maximum raised only when a
//                tile's maximum exceeds it by more than 8 (log2 units);
//   O^T += V^T P^T  A = V^T in bf16 as stored (LDS, the keys of each 32-key
//                product in the order the lanes hold their probabilities),
//                B = P^T split into three bf16 terms (the high 16 bits of p,
//                of the remainder, of the last remainder: 24 significant bits,
//                no range limit on V); row sums on the VALU in float32.
// Output per column and chunk: the normalised partial and its base-2
// log-sum-exp in the partial slots the merge reads (an empty chunk: lse =
// -inf).
#include "device_common.h"
#include "swa_internal.h"

namespace swa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kD = 128;
constexpr int kKSteps = kD / 32;
constexpr int kKeys = 64;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowBlocks = 1;
constexpr int kCols = 16 * kRowBlocks * kWaves;  // query columns per workgroup
static_assert(kCols == kPrefixCols, "the pass's column blocks");
constexpr float kNegInf = -__builtin_inff();
constexpr float kRescaleSlack = 8.f;  // log2 units
constexpr int kScanRound = 64;        // block-table entries per sequence per scan round
constexpr int kMaxScanBlocks = kPrefixMaxRows / 16;  // entries scanned per sequence, at most
constexpr int kSpec = 8;  // table entries per lane loaded before the reference is known
static_assert(kSpec * kWaves >= 64, "the entries loaded ahead cover 64 sequences");
constexpr int kKRowsPerPass = kThreads / 16;  // K rows one load instruction covers
constexpr int kKLoads = kKeys / kKRowsPerPass;
static_assert(kThreads == 512, "the V loader gives each thread 4 keys of 4 dims");

struct Tile {
  u32x4_t k[kKeys * 16];  // K: unit c of key r at r * 16 + (c ^ (r % 16))
  u32x4_t vt[kD * 8];     // V^T (bf16): unit u of dim d at d * 8 + (u ^ vt_swizzle(d))
};

struct Plan {
  int32_t len[kPrefixMaxBatch];    // lengths, clamped to the table
  int32_t miss[kPrefixMaxBatch];   // first entry that differs from the reference's
  int32_t lim[kPrefixMaxBatch];    // rows served by this pass (0: not a sharer)
  int32_t seq[kPrefixMaxBatch];    // the k-th sharer
  int32_t ref_row[kMaxScanBlocks]; // the reference's scanned entries (-1: unusable)
  int32_t xch[5][4 * kWaves];      // per-wave values of the workgroup reductions
  int32_t ref, rows, sharers;
};

struct Smem {
  Tile tiles[2];
  Plan plan;
};

__device__ __forceinline__ int vt_swizzle(int d) { return (d ^ (d >> 2)) & 7; }

// Maximum over the four lanes of one column of an MFMA result (lanes l,
// l ^ 16, l ^ 32, l ^ 48).
__device__ __forceinline__ float column_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(x);
  const auto c = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// Max / min of one int over the wave, the result in every lane: DPP within
// rows of 16 lanes (quad swaps, then rotations by 4 and 8), then the swaps of
// rows across the wave.
struct MaxOp {
  __device__ int32_t operator()(int32_t a, int32_t b) const { return max(a, b); }
};
struct MinOp {
  __device__ int32_t operator()(int32_t a, int32_t b) const { return min(a, b); }
};
template <class Op>
__device__ __forceinline__ int32_t wave_reduce(int32_t x, Op op) {
  x = op(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xf, 0xf, false));   // quad_perm 1,0,3,2
  x = op(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xf, 0xf, false));   // quad_perm 2,3,0,1
  x = op(x, __builtin_amdgcn_update_dpp(x, x, 0x124, 0xf, 0xf, false));  // row_ror 4
  x = op(x, __builtin_amdgcn_update_dpp(x, x, 0x128, 0xf, 0xf, false));  // row_ror 8
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = op(static_cast<int32_t>(a[0]), static_cast<int32_t>(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return op(static_cast<int32_t>(c[0]), static_cast<int32_t>(c[1]));
}

// Workgroup reduction of one int per thread through exchange slots xch (each
// call site its own slots), the same result to all.
template <class Op>
__device__ int32_t block_reduce(int32_t x, int32_t* xch, Op op) {
  x = wave_reduce(x, op);
  if ((threadIdx.x & 63) == 0) xch[threadIdx.x >> 6] = x;
  __syncthreads();
  int32_t t = xch[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) t = op(t, xch[w]);
  return t;
}

// Finds the plan (every thread of the workgroup calls it).  Lane l of wave w
// compares table entry j0 + l of the sequences b = w + kWaves u with the
// reference's entry j0 + l; a ballot gives each sequence's first difference
// in a round of 64 entries (one wave owns a sequence).  For batches of up to
// 64 the first R rounds' entries (R = 2 up to 32 sequences, 1 up to 64) are
// loaded together with the lengths, before the reference is known, and the
// reference's entries reach every lane through LDS; further rounds, if some
// sequence still matches, load as they go.  Every load of a round is issued
// unconditionally (indexes clamped into the table, the result discarded
// where out of range), so a round costs one memory latency.
template <int R>
__device__ void find_plan(const DecodeParams& p, Plan& s) {
  constexpr int U = R > 0 ? kSpec / R : 0;  // sequences per wave loaded ahead
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int bs = 1 << p.block_shift;
  const int cap = p.max_blocks << p.block_shift;
  const int b_last = p.batch - 1, j_last = p.max_blocks - 1;
  auto at = [&](int b, int j) {
    return static_cast<size_t>(min(b, b_last)) * p.max_blocks + min(j, j_last);
  };
  // entry e = u R + r: sequence wave + kWaves u, table entry 64 r + lane
  int32_t sb[R > 0 ? kSpec : 1];
  uint32_t sv[R > 0 ? kSpec : 1];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int r = 0; r < R; ++r) sb[u * R + r] = p.block_table[at(wave + kWaves * u, 64 * r + lane)];
  if (p.block_valid != nullptr) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r) sv[u * R + r] = p.block_valid[at(wave + kWaves * u, 64 * r + lane)];
  } else {
#pragma unroll
    for (int e = 0; e < U * R; ++e) sv[e] = 1;
  }
  constexpr int kLenPerThread = kPrefixMaxBatch / kThreads;
  int32_t len_v[kLenPerThread];
#pragma unroll
  for (int k = 0; k < kLenPerThread; ++k) len_v[k] = p.seq_lens[min(tid + kThreads * k, b_last)];

  // the reference: the longest sequence, the lowest index among equals
  int32_t best = 0;
#pragma unroll
  for (int k = 0; k < kLenPerThread; ++k) {
    const int b = tid + kThreads * k;
    const int32_t n = len_v[k];
    len_v[k] = b < p.batch ? (n < 0 ? 0 : (n > cap ? cap : n)) : -1;
    if (b < p.batch) {
      s.len[b] = len_v[k];
      s.miss[b] = 0x7fffffff;
    }
    best = max(best, len_v[k]);
  }
  const int32_t wave_best = wave_reduce(best, MaxOp{});
  int32_t first = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < kLenPerThread; ++k)
    if (len_v[k] == wave_best) first = min(first, tid + kThreads * k);
  first = wave_reduce(first, MinOp{});
  if (lane == 0) {
    s.xch[0][wave] = wave_best;
    s.xch[0][kWaves + wave] = first;
  }
  __syncthreads();
  int32_t longest = s.xch[0][0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) longest = max(longest, s.xch[0][w]);
  int ref = 0x7fffffff;
#pragma unroll
  for (int w = 0; w < kWaves; ++w)
    if (s.xch[0][w] == longest) ref = min(ref, s.xch[0][kWaves + w]);
  const int ref_blocks = (longest + bs - 1) >> p.block_shift;
  const int scan = longest > 0 ? min(ref_blocks, kMaxScanBlocks >> (p.block_shift - 4)) : 0;
  auto usable = [&](int32_t blk, uint32_t valid) {
    return valid != 0 && blk >= 0 && blk < p.num_phys_blocks;
  };

  // the rounds loaded ahead: every sequence's first difference in them
  int32_t top = 0;     // most leading entries shared with the reference so far
  bool more = R == 0;  // some sequence matches through every round loaded
  if constexpr (R > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (wave + kWaves * u == ref) {
#pragma unroll
        for (int r = 0; r < R; ++r)
          if (64 * r + lane < scan)
            s.ref_row[64 * r + lane] = usable(sb[u * R + r], sv[u * R + r]) ? sb[u * R + r] : -1;
      }
    __syncthreads();
    int32_t rr[R], nbv[U];
#pragma unroll
    for (int r = 0; r < R; ++r) rr[r] = 64 * r + lane < scan ? s.ref_row[64 * r + lane] : -1;
#pragma unroll
    for (int u = 0; u < U; ++u) nbv[u] = (s.len[min(wave + kWaves * u, b_last)] + bs - 1) >> p.block_shift;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int b = wave + kWaves * u;
      if (b < p.batch && b != ref) {  // uniform over the wave
        int32_t m = 0x7fffffff;
#pragma unroll
        for (int r = R - 1; r >= 0; --r) {
          const int e = u * R + r;
          const bool same = 64 * r + lane < nbv[u] && rr[r] >= 0 && sb[e] == rr[r] && usable(sb[e], sv[e]);
          const uint64_t diff = __ballot(!same);
          if (diff != 0) m = 64 * r + static_cast<int>(__builtin_ctzll(diff));
        }
        if (lane == 0) s.miss[b] = m;
        top = max(top, min(m, scan));
        more |= m >= 64 * R;
      }
    }
    if (lane == 0) {
      s.xch[1][wave] = top;
      s.xch[1][kWaves + wave] = more ? 1 : 0;
    }
    __syncthreads();
    top = 0;
    more = false;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      top = max(top, s.xch[1][w]);
      more |= s.xch[1][kWaves + w] != 0;
    }
  }
  more = more && scan > 64 * R;
  if (more) {  // uniform over the workgroup
    constexpr int kSeqsPerPass = 8;
    for (int j0 = 64 * R; j0 < scan; j0 += kScanRound) {
      const int j = j0 + lane;
      int32_t br = p.block_table[at(ref, j)];
      const uint32_t vr = p.block_valid != nullptr ? p.block_valid[at(ref, j)] : 1u;
      for (int b0 = wave; b0 < p.batch; b0 += kWaves * kSeqsPerPass) {
        int32_t bb[kSeqsPerPass];
        uint32_t ok[kSeqsPerPass];
#pragma unroll
        for (int u = 0; u < kSeqsPerPass; ++u) bb[u] = p.block_table[at(b0 + kWaves * u, j)];
        if (p.block_valid != nullptr) {
#pragma unroll
          for (int u = 0; u < kSeqsPerPass; ++u) ok[u] = p.block_valid[at(b0 + kWaves * u, j)];
        } else {
#pragma unroll
          for (int u = 0; u < kSeqsPerPass; ++u) ok[u] = 1;
        }
        if (b0 == wave) {  // the reference's entries of this round
          br = j < scan && usable(br, vr) ? br : -1;
          if (wave == 0 && j < scan) s.ref_row[j] = br;
        }
#pragma unroll
        for (int u = 0; u < kSeqsPerPass; ++u) {
          const int b = b0 + kWaves * u;
          const bool live = b < p.batch && b != ref && s.miss[b] >= j0;  // not yet different
          const int nb = live ? (s.len[b] + bs - 1) >> p.block_shift : 0;
          const bool same = j < nb && br >= 0 && bb[u] == br && usable(bb[u], ok[u]);
          const uint64_t diff = __ballot(live && !same);
          if (lane == 0 && diff != 0) s.miss[b] = j0 + static_cast<int>(__builtin_ctzll(diff));
        }
      }
      __syncthreads();
      bool again = false;
      for (int b = tid; b < p.batch; b += kThreads)
        again |= b != ref && s.miss[b] >= j0 + kScanRound;
      if (!__syncthreads_or(again)) break;
    }
    int32_t t = 0;
    for (int b = tid; b < p.batch; b += kThreads)
      if (b != ref) t = max(t, min(s.miss[b], scan));
    top = block_reduce(t, s.xch[2], MaxOp{});
  }
  const int shared = top;
  const int32_t rows = shared > 0 ? min(shared * bs, longest) : 0;
  // rows served by the pass, and the sharers in increasing order (ballots
  // counted per wave and per group of kThreads sequences)
  int32_t lim_v[kLenPerThread];
  uint64_t bal[kLenPerThread];
#pragma unroll
  for (int k = 0; k < kLenPerThread; ++k) {
    const int b = tid + kThreads * k;
    int32_t lim = 0;
    if (b < p.batch && rows > 0)
      lim = b == ref ? rows : min(min(s.miss[b], scan) * bs, len_v[k]);
    lim_v[k] = lim;
    bal[k] = __ballot(lim > 0);
    if (lane == 0) s.xch[3][k * kWaves + wave] = __builtin_popcountll(bal[k]);
  }
  __syncthreads();
  int32_t total = 0;
#pragma unroll
  for (int k = 0; k < kLenPerThread; ++k) {
    const int b = tid + kThreads * k;
    int32_t before = total;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int32_t c = s.xch[3][k * kWaves + w];
      before += w < wave ? c : 0;
      total += c;
    }
    const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal[k] >> 32),
                                                __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal[k]), 0));
    if (b < p.batch) {
      s.lim[b] = lim_v[k];
      if (lim_v[k] > 0) s.seq[before + below] = b;
    }
  }
  if (tid == 0) {
    s.ref = ref;
    s.rows = rows;
    s.sharers = rows > 0 ? total : 0;
  }
  __syncthreads();
}

// Workgroup min of a and max of b through exchange slots xch, the same
// result to all.
__device__ void block_min_max(int32_t& a, int32_t& b, int32_t* xch) {
  a = wave_reduce(a, MinOp{});
  b = wave_reduce(b, MaxOp{});
  if ((threadIdx.x & 63) == 0) {
    xch[threadIdx.x >> 6] = a;
    xch[kWaves + (threadIdx.x >> 6)] = b;
  }
  __syncthreads();
  a = xch[0];
  b = xch[kWaves];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    a = min(a, xch[w]);
    b = max(b, xch[kWaves + w]);
  }
}

__global__ __launch_bounds__(kThreads, 1) void shared_prefix_kernel(DecodeParams p) {
  __shared__ Smem sm;
  Plan& pl = sm.plan;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lq = lane >> 4;
  const int lc = lane & 15;
  const int g = p.num_q_heads / p.num_kv_heads;
  const int chunks = p.prefix_chunks;
  const int h = blockIdx.x % p.num_kv_heads;
  const int chunk = (blockIdx.x / p.num_kv_heads) % chunks;
  const int cblk = blockIdx.x / (p.num_kv_heads * chunks);

  // Queries, loaded while the plan is found on the guess that sequence k is
  // the k-th sharer (column = k g + head in the group); a column whose sharer
  // differs loads again below.
  bf16x8_t qop[kRowBlocks][kKSteps];
  auto load_q = [&](int rb, int b, int j) {
    const size_t qrow = static_cast<size_t>(b) * p.num_q_heads + static_cast<size_t>(h) * g + j;
#pragma unroll
    for (int s = 0; s < kKSteps; ++s)
      qop[rb][s] = __builtin_bit_cast(
          bf16x8_t, load16(static_cast<const uint16_t*>(p.q) + qrow * kD + 32 * s + 8 * lq));
  };
#pragma unroll
  for (int rb = 0; rb < kRowBlocks; ++rb) {
    const int col = cblk * kCols + 16 * (kRowBlocks * wave + rb) + lc;
    const int k = col / g;
    if (k < p.batch) {
      load_q(rb, k, col - k * g);
    } else {
#pragma unroll
      for (int s = 0; s < kKSteps; ++s) qop[rb][s] = __builtin_bit_cast(bf16x8_t, Vec16{});
    }
  }

  if (p.batch <= 32)
    find_plan<2>(p, pl);
  else if (p.batch <= 64)
    find_plan<1>(p, pl);
  else
    find_plan<0>(p, pl);
  if (blockIdx.x == 0) {  // the plan for the launches that follow
    for (int b = tid; b < p.batch; b += kThreads) p.plan[kPlanHead + b] = pl.lim[b];
    if (tid == 0) {
      p.plan[0] = pl.rows;
      p.plan[1] = pl.ref;
      p.plan[2] = pl.sharers;
      p.plan[3] = 0;
    }
  }
  const int rows = pl.rows;
  const int ncols = pl.sharers * g;
  if (rows == 0 || cblk * kCols >= ncols) return;

  const int bs_shift = p.block_shift;
  const int per = ((rows + chunks * kKeys - 1) / (chunks * kKeys)) * kKeys;
  const int k0 = chunk * per;
  const int k1 = min(k0 + per, rows);
  const size_t units = static_cast<size_t>(p.batch) * p.num_kv_heads;

  const uint16_t* kpool = static_cast<const uint16_t*>(p.k);
  const uint16_t* vpool = static_cast<const uint16_t*>(p.v);
  const int bmask = (1 << bs_shift) - 1;
  // Element offset of key row kk (0 <= kk < rows) of kv head h: the
  // reference's table entries of the shared region are in the plan.
  auto row_at = [&](int kk) {
    const int32_t blk = pl.ref_row[kk >> bs_shift];
    return ((static_cast<size_t>(blk) * p.num_kv_heads + h) << bs_shift |
            static_cast<size_t>(kk & bmask)) * kD;
  };

  // Tile loader: K and V through registers, written to LDS after the current
  // tile's products (a read of LDS waits for every load to LDS issued before
  // it, so loads straight into LDS would stall the products on the next
  // tile).  Thread (kq, kpart) moves physical unit kpart (logical unit
  // kpart ^ (kq % 16)) of key rows kq + kKRowsPerPass e; thread (vd, vu, vh)
  // dims 4 vd .. + 3 of the keys of half vh of V^T unit vu, i.e. keys
  // 32 (vu / 4) + 16 vh + 4 (vu % 4) + i (i < 4).  Keys past the chunk read
  // its last row and enter with V = 0 (they are masked for every column).
  const int kpart = tid & 15;
  const int kq = tid >> 4;
  const int k_unit = kpart ^ (kq & 15);
  const int vd = tid & 31;
  const int vu = (tid >> 6) & 7;
  const int vh = (tid >> 5) & 1;
  const int vkey0 = 32 * (vu >> 2) + 16 * vh + 4 * (vu & 3);
  u32x4_t kreg[kKLoads];
  u32x2_t vreg[4];
  bool vlive[4];
  auto load = [&](int tile) {
    const int base = k0 + tile * kKeys;
#pragma unroll
    for (int e = 0; e < kKLoads; ++e) {
      const size_t at = row_at(min(base + kq + kKRowsPerPass * e, k1 - 1));
      kreg[e] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kpool + at + 8 * k_unit));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kk = base + vkey0 + i;
      vlive[i] = kk < k1;
      vreg[i] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x2_t*>(vpool + row_at(min(kk, k1 - 1)) + 4 * vd));
    }
  };
  auto store = [&](int buf) {
    Tile& t = sm.tiles[buf];
#pragma unroll
    for (int e = 0; e < kKLoads; ++e) t.k[(kq + kKRowsPerPass * e) * 16 + kpart] = kreg[e];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (!vlive[i]) vreg[i] = u32x2_t{0u, 0u};
    u32x2_t* vt2 = reinterpret_cast<u32x2_t*>(t.vt);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d = 4 * vd + r;
      const uint32_t sel = (r & 1) ? 0x07060302u : 0x05040100u;  // the dim's half of each word
      uint32_t w[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const uint32_t a = r < 2 ? vreg[2 * m].x : vreg[2 * m].y;
        const uint32_t c = r < 2 ? vreg[2 * m + 1].x : vreg[2 * m + 1].y;
        w[m] = __builtin_amdgcn_perm(c, a, sel);
      }
      vt2[(d * 8 + (vu ^ vt_swizzle(d))) * 2 + vh] = u32x2_t{w[0], w[1]};
    }
  };
  const int n_tiles = k1 > k0 ? (k1 - k0 + kKeys - 1) / kKeys : 0;
  if (n_tiles > 0) load(0);

  // This lane's column in each row block: sharer, query head, shared rows.
  bool col_ok[kRowBlocks];
  int32_t col_lim[kRowBlocks];
  size_t col_slot[kRowBlocks];  // partial slot * g + head in the group
  int32_t lo = 0x7fffffff, hi = 0;
#pragma unroll
  for (int rb = 0; rb < kRowBlocks; ++rb) {
    const int col = cblk * kCols + 16 * (kRowBlocks * wave + rb) + lc;
    col_ok[rb] = col < ncols;
    const int k = col_ok[rb] ? col / g : 0;
    const int j = col - k * g;
    const int b = pl.seq[k];
    col_lim[rb] = col_ok[rb] ? min(pl.lim[b], k1) : 0;
    col_slot[rb] = (static_cast<size_t>(p.shared_base) + static_cast<size_t>(chunk) * units +
                    static_cast<size_t>(b) * p.num_kv_heads + h) * g + j;
    if (col_ok[rb] && b != k) load_q(rb, b, j);
    if (col_ok[rb]) {
      lo = min(lo, col_lim[rb]);
      hi = max(hi, col_lim[rb]);
    }
  }
  block_min_max(lo, hi, pl.xch[4]);

  int k_off[kKSteps];
#pragma unroll
  for (int s = 0; s < kKSteps; ++s) k_off[s] = lc * 16 + ((4 * s + lq) ^ lc);
  const int vt_g = (lc ^ (lc >> 2)) & 7;
  const int vt_off[2] = {lc * 8 + ((0 + lq) ^ vt_g), lc * 8 + ((4 + lq) ^ vt_g)};

  const float c = p.score_scale_log2;
  float m[kRowBlocks], lsum[kRowBlocks];
  f32x4_t acc[kRowBlocks][kD / 16];
#pragma unroll
  for (int rb = 0; rb < kRowBlocks; ++rb) {
    m[rb] = kNegInf;
    lsum[rb] = 0.f;
#pragma unroll
    for (int blk = 0; blk < kD / 16; ++blk) acc[rb][blk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  if (n_tiles > 0) {
    store(0);
    __syncthreads();
  }
  for (int it = 0; it < n_tiles; ++it) {
    const int cur = it & 1;
    const bool more = it + 1 < n_tiles;
    if (more) load(it + 1);
    const Tile& t = sm.tiles[cur];
    const int base = k0 + it * kKeys;
    // every key of the tile seen by every column / some key by some column
    const bool whole = base + kKeys <= lo;
    if (base < hi) {
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
            sc[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[rb][s], sc[rb][kb], 0, 0, 0);
        }
      if (!whole) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int kk = base + 16 * kb + 4 * lq + r;
#pragma unroll
            for (int rb = 0; rb < kRowBlocks; ++rb)
              sc[rb][kb][r] = kk < col_lim[rb] ? sc[rb][kb][r] : kNegInf;
          }
      }
      float mt[kRowBlocks];
      bool need[kRowBlocks];
      bool any_need = false;
#pragma unroll
      for (int rb = 0; rb < kRowBlocks; ++rb) {
        float x = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) x = fmaxf(x, sc[rb][kb][r]);
        mt[rb] = column_max(x) * c;
        need[rb] = mt[rb] > m[rb] + kRescaleSlack;
        any_need |= need[rb];
      }
      if (__any(any_need)) {
#pragma unroll
        for (int rb = 0; rb < kRowBlocks; ++rb) {
          const float mn = need[rb] ? mt[rb] : m[rb];
          const float alpha = need[rb] ? __builtin_amdgcn_exp2f(m[rb] - mn) : 1.f;
#pragma unroll
          for (int blk = 0; blk < kD / 16; ++blk) acc[rb][blk] *= alpha;
          lsum[rb] *= alpha;
          m[rb] = mn;
        }
      }
#pragma unroll
      for (int pc = 0; pc < 2; ++pc) {
        // P^T of keys 32 pc .. + 31 for both row blocks, as three bf16 terms
        typedef short s16x8_t __attribute__((ext_vector_type(8)));
        uint32_t ph[kRowBlocks][4], pm[kRowBlocks][4], pl_[kRowBlocks][4];
#pragma unroll
        for (int rb = 0; rb < kRowBlocks; ++rb) {
          const float mu = m[rb] == kNegInf ? 0.f : m[rb];
          float pv[8];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              pv[4 * hh + r] = __builtin_amdgcn_exp2f(fmaf(sc[rb][2 * pc + hh][r], c, -mu));
              lsum[rb] += pv[4 * hh + r];
            }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            uint32_t hw[2], mw[2], lw[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
              const float x = pv[2 * e + k];
              hw[k] = __float_as_uint(x) & 0xffff0000u;
              const float r1 = x - __uint_as_float(hw[k]);  // exact
              mw[k] = __float_as_uint(r1) & 0xffff0000u;
              lw[k] = __float_as_uint(r1 - __uint_as_float(mw[k]));  // exact
            }
            ph[rb][e] = __builtin_amdgcn_perm(hw[1], hw[0], 0x07060302u);
            pm[rb][e] = __builtin_amdgcn_perm(mw[1], mw[0], 0x07060302u);
            pl_[rb][e] = __builtin_amdgcn_perm(lw[1], lw[0], 0x07060302u);
          }
        }
#pragma unroll
        for (int blk = 0; blk < kD / 16; ++blk) {
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, t.vt[vt_off[pc ^ (blk & 1)] + 128 * blk]);
#pragma unroll
          for (int rb = 0; rb < kRowBlocks; ++rb) {
            acc[rb][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                a, __builtin_bit_cast(bf16x8_t, pl_[rb]), acc[rb][blk], 0, 0, 0);
            acc[rb][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                a, __builtin_bit_cast(bf16x8_t, pm[rb]), acc[rb][blk], 0, 0, 0);
            acc[rb][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                a, __builtin_bit_cast(bf16x8_t, ph[rb]), acc[rb][blk], 0, 0, 0);
          }
        }
      }
    }
    if (more) store(cur ^ 1);  // that buffer was last read in tile it - 1
    __syncthreads();
  }

  // The column's row sum over its four lanes, then the normalised partial
  // and its base-2 log-sum-exp.
#pragma unroll
  for (int rb = 0; rb < kRowBlocks; ++rb) {
    float l = lsum[rb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (!col_ok[rb]) continue;
    const bool seen = l > 0.f;
    const float inv = seen ? 1.f / l : 0.f;
#pragma unroll
    for (int blk = 0; blk < kD / 16; ++blk) {
      const f32x4_t o = acc[rb][blk] * inv;
      *reinterpret_cast<float4*>(p.ws_o + col_slot[rb] * kD + 16 * blk + 4 * lq) =
          make_float4(o[0], o[1], o[2], o[3]);
    }
    if (lq == 0) p.ws_lse[col_slot[rb]] = seen ? m[rb] + __log2f(l) : kNegInf;
  }
}

}  // namespace

bool prefix_pass_applies(const DecodeParams& p) {
  return p.plan != nullptr && !p.i8 && p.head_dim == kD && p.batch >= 2 &&
         p.batch <= kPrefixMaxBatch && p.num_q_heads / p.num_kv_heads <= 8;
}

hipError_t launch_shared_prefix(const DecodeParams& p, hipStream_t stream) {
  const int g = p.num_q_heads / p.num_kv_heads;
  const int64_t col_blocks = (static_cast<int64_t>(p.batch) * g + kCols - 1) / kCols;
  const int64_t grid = static_cast<int64_t>(p.num_kv_heads) * p.prefix_chunks * col_blocks;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  shared_prefix_kernel<<<static_cast<unsigned>(grid), kThreads, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace swa
