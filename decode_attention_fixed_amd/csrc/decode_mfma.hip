// Read half of the decode step for bf16 caches with head_dim 128: split-K
// over the resident rows, q-group x K-tile scores on the matrix cores, online
// softmax and P*V in fp32 registers, in-workgroup merge of the waves.  A
// (sequence, kv head) processed by one workgroup gets its output written
// directly (one launch per decode call); one spread over several workgroups
// is combined by a small merge launch.
//
// Math as in decode.hip ([sink] weight formula; [kvc] §2.2).  Only the
// resident rows take part: empty ring slots, absent or out-of-range blocks and
// rows past the sequence length are removed with selects, never multiplied by
// zero ([pool] "absent blocks are as if they did not exist").
//
// Work units.  A piece is a contiguous range of rows of one (sequence b, kv
// head); a workgroup of NW waves attends a piece with all g query heads of the
// kv head, its tiles dealt to the waves round-robin so that the workgroup
// streams contiguous memory.
//   ring cache  all sequences have S + W slots: a grid of (b, kv head, split)
//               with equal splits, one piece per workgroup.
//   paged pool  lengths differ: a fixed grid of workgroups, each taking a
//               share of all resident rows (every sequence's rows padded to a
//               64-row multiple, kv heads laid end to end); its share may span
//               several pieces.  Shares balanced over the whole pool keep the
//               last round of workgroups from running half empty when long
//               and short sequences mix.
//
// Per tile of NS 16-row subtiles and wave (lane l, row group lq = l / 16,
// column lc = l % 16):
//   K  4NS x 16-byte loads, each covering four whole 256-byte rows (a load
//      in the operand layout would read 64-byte pieces of 16 rows per
//      instruction, which streams ~15% slower); the wave passes its K tile
//      through a swizzled LDS area so that lane l then holds
//      K[16u + lc][32s + 8lq .. +7] for row subtile u < NS and k-step s < 4,
//      the A operand of v_mfma_f32_16x16x32_bf16 (16 rows x 32 dims).  The B
//      operand holds the
//      g query heads of the kv head (padded to 16 with zeros): lane l holds
//      q[head lc][32s + 8lq .. +7].  The result D[row 4lq + r][head lc] lands
//      in lane l, register r: scores of rows 16u + 4lq + r for head lc.
//   V  4NS x 16-byte loads: lane l holds V[16u + 4lq + r][8lc .. +7], i.e.
//      exactly the rows whose scores live in its own 16-lane row of D.  Each
//      instruction covers four whole 256-byte rows.
//   softmax  per head (lanes with lc = h): running max over the tile (one
//      value per lane per row, reduced across the four row groups), p = 2^(x -
//      m), running sum; the rescale factor and p of head h reach every lane of
//      a 16-lane row through DPP row_newbcast:h.
//   P*V  acc[h][8 dims] += p[h][row] * V[row][8lc .. +7] in fp32.
// The MFMA products of bf16 values are exact and accumulate in fp32; the
// bf16 inputs are the stored values, so no precision is lost before the fp32
// accumulation.
//
// int8 caches (codes + one float32 scale per row): a 128-byte row is half a
// bf16 row, so one 16-byte load instruction covers eight whole rows (lane l:
// chunk l % 8 of row 8i + l / 8); the 16 codes of a chunk become 16 bf16
// values (exact: |code| <= 127) written as the two bf16 chunks of the same
// LDS layout, so the operand reads and the MFMA are the bf16 path's.  The
// score of a row is its MFMA dot product times the row's K scale; V is read
// as 8-byte pieces (8 codes of row 4lq + r, dims 8lc .. +7), and the row's V
// scale joins its softmax weight before the weight is broadcast.  Lane l
// loads the two scales of row 4lq + l % 4 of a subtile; a lane's rows 4lq + r
// take theirs from lane 16lq + r by a DPP row broadcast.
#include <type_traits>

#include "device_common.h"
#include "pager_copy.h"
#include "swa_internal.h"

namespace swa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309417f;
constexpr int kD = 128;
constexpr int kKSteps = kD / 32;

__device__ __forceinline__ bf16x8_t as_bf16x8(const Vec16& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ f16x8_t as_f16x8(const Vec16& v) {
  return __builtin_bit_cast(f16x8_t, v);
}

// Eight int8 codes (two 32-bit words) as the fp16 values 1152 + c, exactly:
// a code c, its sign bit flipped, is the byte c + 128; placed under the fp16
// exponent of 1024 (0x64, unit spacing) it reads 1152 + c (exact: |c| <= 127,
// and 1025 .. 1279 have unit spacing).  One XOR per four codes, one byte
// permute per two.  The matrix products take these biased values and the
// bias is taken off their results (1152 times a sum over the other operand,
// formed by products of its own), which saves the packed subtraction per two
// codes that would make each value c.
constexpr uint32_t kF16x2Bias = 0x64806480u;  // (1152, 1152) in fp16
__device__ __forceinline__ Vec16 codes8_to_f16_biased(uint32_t w0, uint32_t w1) {
  const uint32_t x0 = w0 ^ 0x80808080u, x1 = w1 ^ 0x80808080u;
  // v_perm_b32 byte selectors: 0..3 pick bytes of the second operand (the
  // codes), 4 picks the first operand's 0x64
  Vec16 r;
  r.w[0] = __builtin_amdgcn_perm(0x64646464u, x0, 0x04010400u);
  r.w[1] = __builtin_amdgcn_perm(0x64646464u, x0, 0x04030402u);
  r.w[2] = __builtin_amdgcn_perm(0x64646464u, x1, 0x04010400u);
  r.w[3] = __builtin_amdgcn_perm(0x64646464u, x1, 0x04030402u);
  return r;
}

// Four int8 codes (one 32-bit word) as exact floats.
__device__ __forceinline__ void i8x4_to_f32(uint32_t w, float* x) {
#pragma unroll
  for (int k = 0; k < 4; ++k) x[k] = static_cast<float>(static_cast<int8_t>((w >> (8 * k)) & 0xffu));
}

// K/V rows are read once per step and never again before the whole cache has
// streamed past: non-temporal loads keep them from displacing reused lines.
__device__ __forceinline__ Vec16 load16_stream(const void* p) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  Vec16 r;
  r.w[0] = v[0];
  r.w[1] = v[1];
  r.w[2] = v[2];
  r.w[3] = v[3];
  return r;
}

__device__ __forceinline__ uint2 load8_stream(const void* p) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v[0], v[1]);
}

// Value of lane (16 * (l / 16) + SRC) for every lane l: broadcast inside each
// 16-lane row.
template <int SRC>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + SRC, 0xf, 0xf,
                                         false));
}

// Broadcast of lane h of each 16-lane row; h is a compile-time constant after
// unrolling, so the switch folds to one DPP move.
__device__ __forceinline__ float row_bcast_dyn(float x, int h) {
  switch (h) {
    case 0: return row_bcast<0>(x);
    case 1: return row_bcast<1>(x);
    case 2: return row_bcast<2>(x);
    case 3: return row_bcast<3>(x);
    case 4: return row_bcast<4>(x);
    case 5: return row_bcast<5>(x);
    case 6: return row_bcast<6>(x);
    case 7: return row_bcast<7>(x);
    case 8: return row_bcast<8>(x);
    case 9: return row_bcast<9>(x);
    case 10: return row_bcast<10>(x);
    case 11: return row_bcast<11>(x);
    case 12: return row_bcast<12>(x);
    case 13: return row_bcast<13>(x);
    case 14: return row_bcast<14>(x);
    default: return row_bcast<15>(x);
  }
}

__device__ __forceinline__ float xor_max(float x, int mask) {
  return fmaxf(x, __shfl_xor(x, mask));
}

// Largest block-table span one split can touch: splits are at most 8192 rows
// and blocks at least 16 rows, plus one for a split that starts mid-block.
constexpr int kChunk = 8192;  // rows whose block ids are staged in LDS at a time
constexpr int kMaxSplitBlocks = kChunk / 16 + 1;
constexpr int kMaxSplits = 512;  // ring splits per sequence (the plan never exceeds it)


// Ring: rows of head (b, h) are contiguous, slot t at row t; a row is
// resident iff its slot holds a position.
struct RingRows {
  // a subtile may run past the last slot: rows beyond the range are clamped
  static constexpr bool kWholeSubtiles = false;
  const int32_t* slot_pos;
  size_t head_base;  // element offset of slot 0 of head (b, h)
  int skip = -1;     // slot taken out of the stream (the fused step's new token)
  __device__ RingRows(const DecodeParams& p, int b, int h)
      : slot_pos(p.slot_pos + static_cast<size_t>(b) * p.slots),
        head_base((static_cast<size_t>(b) * p.num_kv_heads + h) * p.slots * kD) {}
  __device__ static int tokens(const DecodeParams& p, int) { return p.slots; }
  __device__ void stage(const DecodeParams&, int, int, int32_t*) const {}
  // Element offset of the first row of the 16-row subtile starting at t
  // (t < t1); false when the whole subtile is known to be absent.
  __device__ bool subtile(const DecodeParams&, const int32_t*, int, int t, size_t& base) const {
    base = head_base + static_cast<size_t>(t) * kD;
    return true;
  }
  __device__ bool row_ok(int t) const { return slot_pos[t] >= 0 && t != skip; }
};

// Pool: token t lives in block block_table[b][t >> shift], row t & (bs - 1);
// a 16-row subtile never straddles a block (bs is a multiple of 16).  The
// split's block ids are staged in LDS once, with -1 for absent blocks (flagged
// invalid, negative or past the pool), so the row loop never waits on a
// dependent table load.
struct PoolRows {
  // a subtile lies inside one block, which is allocated whole: rows past the
  // range are read (and masked) without clamping
  static constexpr bool kWholeSubtiles = true;
  const int32_t* table;
  const uint8_t* valid;
  int h;
  __device__ PoolRows(const DecodeParams& p, int b, int h_)
      : table(p.block_table + static_cast<size_t>(b) * p.max_blocks),
        valid(p.block_valid ? p.block_valid + static_cast<size_t>(b) * p.max_blocks : nullptr),
        h(h_) {}
  __device__ static int tokens(const DecodeParams& p, int b) {
    const int n = p.seq_lens[b];
    const int cap = p.max_blocks << p.block_shift;
    return n < 0 ? 0 : (n > cap ? cap : n);
  }
  __device__ void stage(const DecodeParams& p, int t0, int t1, int32_t* s_blk) const {
    const int j0 = t0 >> p.block_shift;
    const int n = ((t1 - 1) >> p.block_shift) - j0 + 1;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const int j = j0 + i;
      const int blk = table[j];
      const bool ok = blk >= 0 && blk < p.num_phys_blocks && (valid == nullptr || valid[j] != 0);
      s_blk[i] = ok ? blk : -1;
    }
  }
  __device__ bool subtile(const DecodeParams& p, const int32_t* s_blk, int t0, int t,
                          size_t& base) const {
    // the same entry for every lane: keep the block id (and the row
    // address built from it) in scalar registers
    const int blk =
        __builtin_amdgcn_readfirstlane(s_blk[(t >> p.block_shift) - (t0 >> p.block_shift)]);
    const int r = t & ((1 << p.block_shift) - 1);
    base = ((static_cast<size_t>(blk < 0 ? 0 : blk) * p.num_kv_heads + h) << p.block_shift) * kD +
           static_cast<size_t>(r) * kD;
    return blk >= 0;
  }
  __device__ bool row_ok(int) const { return true; }
  int skip = -1;  // unused: pools have no fused step
};

// Row subtiles (16 rows each) per wave tile, as measured: 4 when few query
// heads share the kv head (2 for bf16 pools with g = 2, which keeps them
// clear of register spills); for g >= 3, one on bf16 pools (two were 1-2%
// slower) and two on bf16 rings.  int8 rows carry half the bytes and half
// the registers of bf16 ones: twice the subtiles on rings with g >= 3 and
// four times on pools (two on pools: 2-5% slower); g <= 2 keeps four (eight,
// or two tiles in flight, were slower).
template <int G, bool POOL, bool I8 = false>
constexpr int subtiles() {
  return G <= 2 ? (G == 2 && POOL && !I8 ? 2 : 4)
                : ((G < 8 && !POOL ? 2 : 1) * (I8 ? (POOL ? 4 : 2) : 1));
}

// RC: 16-byte chunks per staged K row (16 for bf16 rows, 8 for int8 codes).
template <int G, int NW, int NS_, int RC = 16>
struct Smem {
  static constexpr int NS = NS_;
  static constexpr int TILE = 16 * NS;
  static constexpr int KBUF = TILE * RC;  // 16-byte chunks per wave: TILE staged rows
  static constexpr size_t KBYTES = static_cast<size_t>(NW) * KBUF * 16;
  static constexpr size_t ABYTES = static_cast<size_t>(NW) * G * kD * sizeof(float);
  // each wave's K tile while streaming; the same bytes then hold the waves'
  // P*V accumulators for the workgroup merge
  __attribute__((aligned(16))) unsigned char raw[KBYTES > ABYTES ? KBYTES : ABYTES];
  float m[NW][G];
  float l[NW][G];
  int32_t blk[kMaxSplitBlocks];
};

// Fused decode step (ring caches): the token appended in the same launch.
// Every workgroup of the sequence rotates the query itself; the workgroup
// whose rows hold the token's slot also rotates and stores the token's K row,
// V row and position, takes that slot out of its stream (it may hold the
// evicted row, and the new row is being written meanwhile) and folds the new
// token in from LDS at the workgroup merge, so no workgroup reads a row
// written by this launch.
struct NewToken {
  bool app = false;   // the position is valid (>= 0): the token is appended
  bool mine = false;  // this workgroup attends the token's slot
  int slot = -1;
  int32_t pos = 0;
  double theta = 0.0;  // theta_(tid % 64), read first of all loads (they complete in order)
  // Cache position shifting ([sink]): positions inside the attention are
  // indices in the cache (sinks, then the window in order).  A window key
  // keeps its distance to the query, so only the sinks change: they are
  // scored against the query rotated at its cache position cpos.  `shift`:
  // this workgroup holds sink rows and cpos differs from pos.
  bool shift = false;
  int32_t cpos = 0;
};

template <int G>
struct NewRow {
  double cs[kD / 2], sn[kD / 2];  // the token's rotation angles
  double cs2[kD / 2], sn2[kD / 2];  // the angles at its cache position (shifting)
  uint16_t q[G][kD];              // rotated query heads (bf16, as an append stores them)
  uint16_t qs[G][kD];             // the query heads rotated at the cache position (shifting)
  float k[kD], v[kD];             // its rotated K row and its V row
  float x[G];                     // its score per head (log2 units)
};

// The fused step's work before the row loop, by every thread: read the raw
// query pairs and the new token's K pair / V chunk (unconditionally, every
// address is valid, so nothing waits on them early), compute the angles
// (threads < 64) meanwhile, then rotate the query heads into nr.q (one pair
// per thread) and, in the workgroup that attends the token's slot, store the
// rotated K row, the V row and the position, and compute the token's score
// per head into nr.x.  Angles, rotation and rounding are the append
// kernel's, so the cache is bit-identical to an append.  int8 caches: the
// K row is quantised from its float64 rotation and the V row from its bf16
// values by the wave that holds the K pairs (quantize_pair_row, as the int8
// append), and nr.k / nr.v hold the dequantised rows c * s.
template <int G, int NW, bool I8 = false>
__device__ void fused_step_prologue(const DecodeParams& p, NewRow<G>& nr, const NewToken& nt,
                                    int b, int kvh, RingRows& rows) {
  constexpr int kHalf = kD / 2;
  constexpr int kItems = (G + 1) * kHalf;  // the query pairs, then the K pairs
  constexpr int kPer = (kItems + NW * 64 - 1) / (NW * 64);
  const int tid = threadIdx.x;
  if (nt.mine) rows.skip = nt.slot;
  const size_t head0 = static_cast<size_t>(b) * p.num_q_heads + static_cast<size_t>(kvh) * G;
  const size_t nrow = (static_cast<size_t>(b) * p.num_kv_heads + kvh) * kD;
  const uint16_t* qb = static_cast<const uint16_t*>(p.q) + head0 * kD;
  const uint16_t* kn = static_cast<const uint16_t*>(p.k_new) + nrow;
  const uint16_t* vn = static_cast<const uint16_t*>(p.v_new) + nrow;
  uint16_t r0[kPer], r1[kPer];
  uint16_t w0[I8 ? kPer : 1], w1[I8 ? kPer : 1];  // int8: the V pair beside the K pair
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int w = min(tid + j * NW * 64, kItems - 1);
    const int h = w / kHalf, i = w - h * kHalf;
    const int i0 = p.rope_half ? i : 2 * i;
    const int i1 = p.rope_half ? i + kHalf : 2 * i + 1;
    const uint16_t* src = h < G ? qb + h * kD : kn;
    r0[j] = src[i0];
    r1[j] = src[i1];
    if constexpr (I8) {
      w0[j] = vn[i0];
      w1[j] = vn[i1];
    }
  }
  Vec16 vraw{};
  if constexpr (!I8) vraw = load16(vn + 8 * (tid & 15));
  if (nt.app && tid < kHalf) {
    double sn, cs;
    rope_sincos(static_cast<double>(nt.pos), nt.theta, &sn, &cs);
    nr.cs[tid] = cs;
    nr.sn[tid] = sn;
    if (nt.shift) {
      rope_sincos(static_cast<double>(nt.cpos), nt.theta, &sn, &cs);
      nr.cs2[tid] = cs;
      nr.sn2[tid] = sn;
    }
  }
  __syncthreads();
  const size_t row = (static_cast<size_t>(b) * p.num_kv_heads + kvh) * p.slots + nt.slot;
  const size_t crow = row * kD;  // elements (bytes of int8 codes) before the row
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int w = tid + j * NW * 64;
    if (w >= kItems) break;
    const int h = w / kHalf, i = w - h * kHalf;
    if (h == G && !nt.mine) break;
    const int i0 = p.rope_half ? i : 2 * i;
    const int i1 = p.rope_half ? i + kHalf : 2 * i + 1;
    uint16_t o0 = r0[j], o1 = r1[j];
    double x0 = 0.0, x1 = 0.0;  // the rotated pair in float64
    if (nt.app) {
      rope_rotate_pair(static_cast<double>(bf16_to_f32(r0[j])),
                       static_cast<double>(bf16_to_f32(r1[j])), nr.cs[i], nr.sn[i], &x0, &x1);
      o0 = f64_to_bf16_rne(x0);
      o1 = f64_to_bf16_rne(x1);
    }
    if (h < G) {
      nr.q[h][i0] = o0;
      nr.q[h][i1] = o1;
      if (nt.shift) {  // the same rotation and rounding at the cache position
        double x0, x1;
        rope_rotate_pair(static_cast<double>(bf16_to_f32(r0[j])),
                         static_cast<double>(bf16_to_f32(r1[j])), nr.cs2[i], nr.sn2[i], &x0, &x1);
        nr.qs[h][i0] = f64_to_bf16_rne(x0);
        nr.qs[h][i1] = f64_to_bf16_rne(x1);
      }
    } else if constexpr (I8) {  // the K and V rows, quantised, into the cache and LDS
      double c0, c1, d0, d1;
      const float ks = quantize_pair_row(x0, x1, true, &c0, &c1);
      const float vs = quantize_pair_row(static_cast<double>(bf16_to_f32(w0[j])),
                                         static_cast<double>(bf16_to_f32(w1[j])), true, &d0, &d1);
      int8_t* kc = const_cast<int8_t*>(static_cast<const int8_t*>(p.k)) + crow;
      int8_t* vc = const_cast<int8_t*>(static_cast<const int8_t*>(p.v)) + crow;
      kc[i0] = static_cast<int8_t>(c0);
      kc[i1] = static_cast<int8_t>(c1);
      vc[i0] = static_cast<int8_t>(d0);
      vc[i1] = static_cast<int8_t>(d1);
      if (i == 0) {
        const_cast<float*>(p.k_scale)[row] = ks;
        const_cast<float*>(p.v_scale)[row] = vs;
      }
      nr.k[i0] = static_cast<float>(c0 * static_cast<double>(ks));
      nr.k[i1] = static_cast<float>(c1 * static_cast<double>(ks));
      nr.v[i0] = static_cast<float>(d0 * static_cast<double>(vs));
      nr.v[i1] = static_cast<float>(d1 * static_cast<double>(vs));
    } else {  // the K row, rotated, into the cache and LDS
      uint16_t* kc = const_cast<uint16_t*>(static_cast<const uint16_t*>(p.k)) + crow;
      kc[i0] = o0;
      kc[i1] = o1;
      nr.k[i0] = bf16_to_f32(o0);
      nr.k[i1] = bf16_to_f32(o1);
    }
  }
  if (!I8 && nt.mine && tid < kD / 8) {  // the V row
    store16(const_cast<uint16_t*>(static_cast<const uint16_t*>(p.v)) + crow + 8 * tid, vraw);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      nr.v[8 * tid + 2 * e] = bf16_lo(vraw.w[e]);
      nr.v[8 * tid + 2 * e + 1] = bf16_hi(vraw.w[e]);
    }
  }
  if (nt.mine && kvh == 0 && tid == 0)
    const_cast<int32_t*>(p.slot_pos)[static_cast<size_t>(b) * p.slots + nt.slot] = nt.pos;
  __syncthreads();
  if (nt.mine) {  // the token's score: wave h sums head h
    const int wave = tid >> 6;
    const int lane = tid & 63;
    for (int h = wave; h < G; h += NW) {
      float d = bf16_to_f32(nr.q[h][2 * lane]) * nr.k[2 * lane] +
                bf16_to_f32(nr.q[h][2 * lane + 1]) * nr.k[2 * lane + 1];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) d += __shfl_xor(d, off);
      if (lane == 0) nr.x[h] = d * p.score_scale_log2;
    }
    // nr.x is read after the barriers of the row loop
  }
}

// Attention of the G query heads of (b, kvh) over rows [t0, t1) by the whole
// workgroup.  Writes the output and lse (direct) or, for a piece of a longer
// sequence, the normalised partial output and base-2 lse at partial slot
// `slot` (layout [slot][head][d]).  Every thread of the workgroup must call it
// with the same arguments; it returns with LDS free for reuse.
template <int G, class Rows, int NW, bool FUSED = false, bool I8 = false, int NS_>
__device__ void attend_piece(const DecodeParams& p, Smem<G, NW, NS_, I8 ? 8 : 16>& sm, int b, int kvh, int t0,
                             int t1, bool direct, size_t slot, NewRow<G>* nr = nullptr,
                             NewToken nt = NewToken{}) {
  using Sm = Smem<G, NW, NS_, I8 ? 8 : 16>;
  constexpr int NS = Sm::NS;
  constexpr int TILE = Sm::TILE;
  constexpr int KBUF = Sm::KBUF;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lq = lane >> 4;
  const int lc = lane & 15;
  const size_t head0 = static_cast<size_t>(b) * p.num_q_heads + static_cast<size_t>(kvh) * G;
  Rows rows(p, b, kvh);
  // element offsets index bf16 rows, or bytes of int8 rows
  using KT = std::conditional_t<I8, int8_t, uint16_t>;
  const KT* kb = static_cast<const KT*>(p.k);
  const KT* vb = static_cast<const KT*>(p.v);
  constexpr int KL = I8 ? 2 : 4;  // K load instructions per 16-row subtile
  // g >= 3 multiplies P*V on the matrix core: the VALU form costs g FMAs per
  // (row, dim), the MFMA form a fixed repacking of V
  constexpr bool kMfmaPV = G >= 3;

  // B operand: the g query heads of this kv head, zero-padded to 16 (the
  // fused step rotates them into LDS first).  Lane (lc, lq) holds 8 dims of
  // head lc per MFMA step s: dims 32s + 8lq .. for bf16 tiles; for int8
  // tiles the dims in the order the lane reads its row's codes back from
  // LDS, 64(s/2) + 16lq + 8(s%2) .. (the same permutation of the dims on
  // both operands).
  // int8 tiles multiply in fp16: the query is scaled per head by the power
  // of two 2^k that brings its largest |element| into [2^14, 2^15), which is
  // exact (a bf16 value has 8 significant bits), and the scores by 2^-k.
  if constexpr (FUSED) fused_step_prologue<G, NW, I8>(p, *nr, nt, b, kvh, rows);
  Vec16 qop[kKSteps];
  float qinv = 1.f;
  {
    const uint16_t* qb = static_cast<const uint16_t*>(p.q);
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) {
      const int off = I8 ? 64 * (s >> 1) + 16 * lq + 8 * (s & 1) : 32 * s + 8 * lq;
      Vec16 v{};
      if (lc < G) {
        if constexpr (FUSED)
          v = load16(&nr->q[lc][off]);
        else
          v = load16(qb + (head0 + lc) * kD + off);
      }
      qop[s] = v;
    }
    if constexpr (I8) {
      float amax = 0.f;
#pragma unroll
      for (int s = 0; s < kKSteps; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(qop[s].w[i])), fabsf(bf16_hi(qop[s].w[i]))));
      amax = xor_max(amax, 16);
      amax = xor_max(amax, 32);
      int k = 0;  // zero or non-finite heads keep their values
      if (amax > 0.f && amax <= 3.4e38f) {
        k = 15 - __builtin_amdgcn_frexp_expf(amax);  // amax = f 2^e, f in [1/2, 1)
        k = k < -126 ? -126 : (k > 126 ? 126 : k);
      }
      qinv = ldexpf(1.f, -k);
#pragma unroll
      for (int s = 0; s < kKSteps; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f16x2_t h = {static_cast<_Float16>(ldexpf(bf16_lo(qop[s].w[i]), k)),
                             static_cast<_Float16>(ldexpf(bf16_hi(qop[s].w[i]), k))};
          qop[s].w[i] = __builtin_bit_cast(uint32_t, h);
        }
    }
  }
  // int8 rows: the score products take the codes as 1152 + c; every score of
  // head lc then carries 1152 times the sum of the head's query, which the
  // same products with every code at 1152 form once per piece, and the score
  // accumulators start at its negation.
  f32x4_t score_init = {0.f, 0.f, 0.f, 0.f};
  if constexpr (I8) {
    Vec16 bias;
#pragma unroll
    for (int i = 0; i < 4; ++i) bias.w[i] = kF16x2Bias;
#pragma unroll
    for (int s = 0; s < kKSteps; ++s)
      score_init =
          __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(bias), as_f16x8(qop[s]), score_init, 0, 0, 0);
    score_init = -score_init;
  }

  const float c = p.score_scale_log2 * qinv;
  float m = kNegInf;  // running max of head lc (log2 units)
  float lsum = 0.f;   // this lane's share of the running sum of head lc
  // P*V accumulators.  VALU form: acc[h][e] = head h, dim 8lc + e, over this
  // lane's rows.  MFMA form (g >= 3): accm[nb][j] = head 4lq + j, dim
  // 8lc + nb, over all rows of the wave.
  float acc[kMfmaPV ? 1 : G][8];
  f32x4_t accm[kMfmaPV ? 8 : 1];
#pragma unroll
  for (int h = 0; h < (kMfmaPV ? 1 : G); ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
#pragma unroll
  for (int nb = 0; nb < (kMfmaPV ? 8 : 1); ++nb) accm[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // This wave's K staging area: row rho of subtile u, 16-byte chunk c lives at
  // chunk (u * 16 + rho) * 16 + (c ^ rho), so both the row-wise writes and the
  // operand-wise reads below touch 16 distinct bank groups per 16 lanes.
  uint4* s_k = reinterpret_cast<uint4*>(sm.raw) + wave * KBUF;

  // One wave tile: NS subtiles of 16 rows.
  struct Tile {
    Vec16 kr[NS][KL];  // row-wise K chunks: row 4i + lq of subtile u, chunk lc
                       // (int8: row 8i + l / 8, 16-byte chunk l % 8)
    std::conditional_t<I8, uint2, Vec16> vr[NS][4];  // V: row 4lq + r of subtile u, dims 8lc..
    float ksl[NS], vsl[NS];  // int8: K and V scales of row 4lq + (lc & 3) of subtile u
    uint32_t vm[NS];         // bit i: row ts + 16u + i is resident
    size_t base[NS];
    bool live[NS];
  };
  // Issues the tile's loads (rows ts .. of the staged chunk [c0, c1)).
  // `whole`: the tile lies inside [c0, c1), so no row needs clamping.
  auto load_tile = [&](Tile& T, int ts, int c0, int c1, auto whole) {
    constexpr bool kIn = decltype(whole)::value;
    constexpr bool kNoClamp = kIn || Rows::kWholeSubtiles;
    // Every load instruction reads four whole 256-byte rows; K first, so
    // the score phase waits on K while the V loads are still in flight.
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int tu = ts + 16 * u;
      T.vm[u] = 0;
      T.base[u] = 0;
      T.live[u] = (kIn || tu < c1) && rows.subtile(p, sm.blk, c0, tu, T.base[u]);
      if (T.live[u]) {
        const int tk = tu + lc;
        const bool okk = (kIn || tk < c1) && rows.row_ok(tk);
        T.vm[u] = static_cast<uint32_t>(__ballot(okk)) & 0xffffu;
        const KT* ks = kb + T.base[u];  // uniform: scalar base register
        if constexpr (I8) {
#pragma unroll
          for (int i = 0; i < KL; ++i) {
            const int rho = 8 * i + (lane >> 3);
            const int row = kNoClamp || tu + rho < c1 ? rho : 0;
            T.kr[u][i] = load16_stream(ks + static_cast<uint32_t>(row * kD + 16 * (lane & 7)));
          }
          // lane l loads the scales of row 4lq + (l % 4); row 4lq + r is then
          // lane 16lq + r's, one DPP broadcast away
          const int sr = 4 * lq + (lc & 3);
          const int rr = kNoClamp || tu + sr < c1 ? sr : 0;
          const size_t srow = (T.base[u] >> 7) + rr;  // kD = 128 codes per row
          T.ksl[u] = p.k_scale[srow];
          T.vsl[u] = p.v_scale[srow];
        } else {
#pragma unroll
          for (int i = 0; i < KL; ++i) {
            const int rho = 4 * i + lq;
            const int row = kNoClamp || tu + rho < c1 ? rho : 0;
            T.kr[u][i] = load16_stream(ks + static_cast<uint32_t>(row * kD + 8 * lc));
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < KL; ++i) T.kr[u][i] = Vec16{};
        T.ksl[u] = 0.f;
        T.vsl[u] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int tu = ts + 16 * u;
      if (T.live[u]) {
        const KT* vs = vb + T.base[u];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * lq + r;
          const int row = kNoClamp || tu + i < c1 ? i : 0;
          if constexpr (I8)
            T.vr[u][r] = load8_stream(vs + static_cast<uint32_t>(row * kD + 8 * lc));
          else
            T.vr[u][r] = load16_stream(vs + static_cast<uint32_t>(row * kD + 8 * lc));
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) T.vr[u][r] = {};
      }
    }

};
  // Scores, online softmax and P*V of a loaded tile.
  auto compute_tile = [&](Tile& T, int ts, int c1) {
    // K chunks into the MFMA A-operand layout through LDS (DS instructions
    // of one wave execute in order; the wave barriers only stop the compiler
    // from moving LDS accesses across each other).  int8 rows are staged as
    // codes, 8 chunks a row at chunk c ^ swz8(row), and read back as chunks
    // lq and 4 + lq of row lc (16 codes = two MFMA steps each); the XOR puts
    // every 8 and every 16 lanes of a read on distinct banks.
    Vec16 ka[NS][I8 ? 2 : kKSteps];  // lane l: row lc, dims 32s + 8lq .. +7
                                     // (int8: codes of chunks lq, 4 + lq)
    if constexpr (I8) {
      auto swz8 = [](int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; };
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int u = 0; u < NS; ++u)
#pragma unroll
        for (int i = 0; i < KL; ++i) {
          const int rho = 8 * i + (lane >> 3);
          s_k[(u * 16 + rho) * 8 + ((lane & 7) ^ swz8(rho))] =
              make_uint4(T.kr[u][i].w[0], T.kr[u][i].w[1], T.kr[u][i].w[2], T.kr[u][i].w[3]);
        }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int u = 0; u < NS; ++u)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint4 t = s_k[(u * 16 + lc) * 8 + ((4 * j + lq) ^ swz8(lc))];
          ka[u][j].w[0] = t.x;
          ka[u][j].w[1] = t.y;
          ka[u][j].w[2] = t.z;
          ka[u][j].w[3] = t.w;
        }
      __builtin_amdgcn_wave_barrier();
    } else {
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int u = 0; u < NS; ++u)
#pragma unroll
        for (int i = 0; i < KL; ++i) {
          const int rho = 4 * i + lq;
          s_k[(u * 16 + rho) * 16 + (lc ^ rho)] =
              make_uint4(T.kr[u][i].w[0], T.kr[u][i].w[1], T.kr[u][i].w[2], T.kr[u][i].w[3]);
        }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int u = 0; u < NS; ++u)
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) {
          const uint4 t = s_k[(u * 16 + lc) * 16 + ((4 * s + lq) ^ lc)];
          ka[u][s].w[0] = t.x;
          ka[u][s].w[1] = t.y;
          ka[u][s].w[2] = t.z;
          ka[u][s].w[3] = t.w;
        }
      __builtin_amdgcn_wave_barrier();
    }
    uint32_t all = 0xffffu;
#pragma unroll
    for (int u = 0; u < NS; ++u) all &= T.vm[u];
    const bool all_ok = all == 0xffffu;

    // scores (log2 units) of rows 16u + 4lq + r for head lc
    float x[NS][4];
    float tmax = kNegInf;
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      f32x4_t d = score_init;
#pragma unroll
      for (int s = 0; s < kKSteps; ++s) {
        if constexpr (I8) {  // 8 codes of row lc -> fp16 operand 1152 + c
          const Vec16& w = ka[u][s >> 1];
          const Vec16 a = codes8_to_f16_biased(w.w[2 * (s & 1)], w.w[2 * (s & 1) + 1]);
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(a), as_f16x8(qop[s]), d, 0, 0, 0);
        } else {
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka[u][s]), as_bf16x8(qop[s]), d, 0,
                                                      0, 0);
        }
      }
      if constexpr (FUSED && !I8) {  // (shifting: bf16 caches only)
        const int tu = ts + 16 * u;
        if (nt.shift && tu < p.sinks) {  // sink rows: the query at its cache position
          f32x4_t ds = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < kKSteps; ++s) {
            Vec16 v{};
            if (lc < G) v = load16(&nr->qs[lc][32 * s + 8 * lq]);
            ds = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka[u][s]), as_bf16x8(v), ds, 0,
                                                         0, 0);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (tu + 4 * lq + r < p.sinks) d[r] = ds[r];
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = (T.vm[u] >> (4 * lq + r)) & 1u;
        float dr = d[r];
        if constexpr (I8) dr *= row_bcast_dyn(T.ksl[u], r);  // the row's K scale
        x[u][r] = ok ? dr * c : kNegInf;
        tmax = fmaxf(tmax, x[u][r]);
      }
    }
    tmax = xor_max(tmax, 16);
    tmax = xor_max(tmax, 32);
    const float mn = fmaxf(m, tmax);
    // mn == -inf: nothing resident so far for this head; keep everything at 0
    // (the hardware 2^x: exact 0 at -inf; arguments are <= 0 and results
    // below 2^-126, far under anything a sum keeps, may flush to 0)
    const float alpha = mn == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    const float mb = mn == kNegInf ? 0.f : mn;  // absent rows (x = -inf) give 0
    float pr[NS][4];
    float tsum = 0.f;
#pragma unroll
    for (int u = 0; u < NS; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[u][r] = __builtin_amdgcn_exp2f(x[u][r] - mb);
        tsum += pr[u][r];
      }
    lsum = lsum * alpha + tsum;
    if constexpr (I8) {  // the row's V scale joins its weight (selected: an
                         // absent row's scale may hold anything)
#pragma unroll
      for (int u = 0; u < NS; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = (T.vm[u] >> (4 * lq + r)) & 1u;
          const float vsc = row_bcast_dyn(T.vsl[u], r);
          pr[u][r] = ok ? pr[u][r] * vsc : 0.f;
        }
    }

    // P * V
    if constexpr (kMfmaPV) {
      float aj[4];  // alpha of head 4lq + j (lanes 0..15 hold heads 0..15)
#pragma unroll
      for (int j = 0; j < 4; ++j) aj[j] = __shfl(alpha, 4 * lq + j);
      f32x4_t t[8];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) t[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if constexpr (I8) {
        // O[head][dim] += P[head][row] V[row][dim], v_mfma_f32_16x16x16_f16 per
        // 16 rows and 16 dims: A = P (lane (lc, lq): head lc, rows 4lq + i,
        // exactly pr[u][i]); B = V (lane (lc, lq): rows 4lq + i, dim 8lc + nb
        // in block nb, byte nb of the lane's own codes of those rows, made
        // fp16 as 1152 + c, as for K).  P carries the V scale; the tile's
        // weights are scaled by 2^k, k from the largest V scale of its present
        // rows, into fp16's range, and the tile's product by 2^-k on the way
        // into accm.  The bias, 1152 times each head's weight sum, is the
        // product of the same P with B = 1152 everywhere (tc), taken off once
        // per tile.
        float vmax = 0.f;
#pragma unroll
        for (int u = 0; u < NS; ++u) {
          // vsl[u]: the scale of row 4lq + (lc & 3); absent rows' may hold anything
          const bool okr = (T.vm[u] >> (4 * lq + (lc & 3))) & 1u;
          vmax = fmaxf(vmax, okr ? T.vsl[u] : 0.f);
        }
        vmax = xor_max(vmax, 1);
        vmax = xor_max(vmax, 2);
        vmax = xor_max(vmax, 16);
        vmax = xor_max(vmax, 32);
        int k = 0;
        if (vmax > 0.f && vmax <= 3.4e38f) {
          k = 15 - __builtin_amdgcn_frexp_expf(vmax);
          k = k < -126 ? -126 : (k > 126 ? 126 : k);
        }
        const float up = ldexpf(1.f, k), down = ldexpf(1.f, -k);
        const f16x4_t bias = __builtin_bit_cast(f16x4_t, make_uint2(kF16x2Bias, kF16x2Bias));
        f32x4_t tc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < NS; ++u) {
          const f16x2_t a01 = __builtin_convertvector(f32x2_t{pr[u][0] * up, pr[u][1] * up}, f16x2_t);
          const f16x2_t a23 = __builtin_convertvector(f32x2_t{pr[u][2] * up, pr[u][3] * up}, f16x2_t);
          const f16x4_t a = {a01[0], a01[1], a23[0], a23[1]};
          tc = __builtin_amdgcn_mfma_f32_16x16x16f16(a, bias, tc, 0, 0, 0);
          uint32_t x[4][2];  // codes of rows 4lq + i, sign bits flipped
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[i][0] = T.vr[u][i].x ^ 0x80808080u;
            x[i][1] = T.vr[u][i].y ^ 0x80808080u;
          }
#pragma unroll
          for (int nb = 0; nb < 8; ++nb) {
            const int w = nb >> 2, bsel = nb & 3;
            // bytes [row i, 0, row i + 1, 0], then 0x64 above each: 1152 + c
            const uint32_t sel = 0x0c000c00u | static_cast<uint32_t>((4 + bsel) << 16) |
                                 static_cast<uint32_t>(bsel);
            const uint32_t b01 = __builtin_amdgcn_perm(x[1][w], x[0][w], sel) | 0x64006400u;
            const uint32_t b23 = __builtin_amdgcn_perm(x[3][w], x[2][w], sel) | 0x64006400u;
            const f16x4_t bv = __builtin_bit_cast(f16x4_t, make_uint2(b01, b23));
            t[nb] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, bv, t[nb], 0, 0, 0);
          }
        }
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            accm[nb][j] = fmaf(t[nb][j] - tc[j], down, accm[nb][j] * aj[j]);
      } else {
        // O[head][dim] += P[head][row] V[row][dim] as above, with
        // v_mfma_f32_16x16x16_bf16: B = the bf16 V rows as stored (absent
        // rows zeroed: their bytes may be anything), A = P split into three
        // bf16 terms (p with its low 16 bits cleared, then the same of the
        // remainder, then the last remainder truncated), three products per
        // block: P keeps 21 or more significant bits.
        typedef short s16x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int u = 0; u < NS; ++u) {
          uint32_t hw[4], mw[4], lw[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            hw[i] = __float_as_uint(pr[u][i]) & 0xffff0000u;
            const float r1 = pr[u][i] - __uint_as_float(hw[i]);  // exact
            mw[i] = __float_as_uint(r1) & 0xffff0000u;
            lw[i] = __float_as_uint(r1 - __uint_as_float(mw[i]));  // exact
          }
          // the upper halves of two floats: one bf16 pair of the A operand
          auto pack = [](const uint32_t* x) {
            const uint32_t w[2] = {__builtin_amdgcn_perm(x[1], x[0], 0x07060302u),
                                   __builtin_amdgcn_perm(x[3], x[2], 0x07060302u)};
            return __builtin_bit_cast(s16x4_t, w);
          };
          const s16x4_t ah = pack(hw), am = pack(mw), al = pack(lw);
          uint32_t vw[4][4];  // rows 4lq + i: bf16 pairs (dims 8lc + 2w, + 1)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool ok = all_ok || ((T.vm[u] >> (4 * lq + i)) & 1u);
#pragma unroll
            for (int w = 0; w < 4; ++w) vw[i][w] = ok ? T.vr[u][i].w[w] : 0u;
          }
#pragma unroll
          for (int nb = 0; nb < 8; ++nb) {
            const int w = nb >> 1;
            const uint32_t sel = (nb & 1) ? 0x07060302u : 0x05040100u;  // the dim's half of each
            const uint32_t bw[2] = {__builtin_amdgcn_perm(vw[1][w], vw[0][w], sel),
                                    __builtin_amdgcn_perm(vw[3][w], vw[2][w], sel)};
            const s16x4_t bv = __builtin_bit_cast(s16x4_t, bw);
            t[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bv, t[nb], 0, 0, 0);
            t[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(am, bv, t[nb], 0, 0, 0);
            t[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bv, t[nb], 0, 0, 0);
          }
        }
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
#pragma unroll
          for (int j = 0; j < 4; ++j) accm[nb][j] = fmaf(accm[nb][j], aj[j], t[nb][j]);
      }
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float a = row_bcast_dyn(alpha, h);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= a;
      }
#pragma unroll
      for (int u = 0; u < NS; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v[8];
          if constexpr (I8) {
            i8x4_to_f32(T.vr[u][r].x, v);
            i8x4_to_f32(T.vr[u][r].y, v + 4);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              v[2 * i] = bf16_lo(T.vr[u][r].w[i]);
              v[2 * i + 1] = bf16_hi(T.vr[u][r].w[i]);
            }
          }
          if (!I8 && !all_ok) {
            const bool ok = (T.vm[u] >> (4 * lq + r)) & 1u;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = ok ? v[e] : 0.f;
          }
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float ph = row_bcast_dyn(pr[u][r], h);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(ph, v[e], acc[h][e]);
          }
        }
    }
  };

  for (int c0 = t0; c0 < t1; c0 += kChunk) {
    const int c1 = min(c0 + kChunk, t1);
    rows.stage(p, c0, c1, sm.blk);
    __syncthreads();
    for (int ts = c0 + wave * TILE; ts < c1; ts += NW * TILE) {
      Tile A;
      // (two copies of the loads cost bf16 g = 2 its last free registers)
      if (!(G == 2 && !I8) && ts + TILE <= c1)
        load_tile(A, ts, c0, c1, std::true_type{});
      else
        load_tile(A, ts, c0, c1, std::false_type{});
      compute_tile(A, ts, c1);
    }
    __syncthreads();  // the next chunk restages the block ids
  }

  // Wave totals: sum the four row groups (the MFMA form has summed them).
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if constexpr (!kMfmaPV) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        acc[h][e] += __shfl_xor(acc[h][e], 16);
        acc[h][e] += __shfl_xor(acc[h][e], 32);
      }
  }
  float(*s_acc)[G][kD] = reinterpret_cast<float(*)[G][kD]>(sm.raw);
  __syncthreads();  // every wave is done with its K staging area (aliases s_acc)
  if (lane < G) {
    sm.m[wave][lane] = m;
    sm.l[wave][lane] = lsum;
  }
  if constexpr (kMfmaPV) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (4 * lq + j < G) {
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) s_acc[wave][4 * lq + j][8 * lc + nb] = accm[nb][j];
      }
  } else if (lq == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[wave][h][8 * lc + e] = acc[h][e];
  }
  __syncthreads();

  // Workgroup merge: thread -> (head, dim) pairs.
  for (int i = threadIdx.x; i < G * kD; i += NW * 64) {
    const int h = i / kD;
    const int d = i - h * kD;
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, sm.m[w][h]);
    bool add_new = false;
    if constexpr (FUSED) {
      add_new = nt.mine;
      if (add_new) mx = fmaxf(mx, nr->x[h]);
    }
    float lt = 0.f, o = 0.f;
    if (mx != kNegInf) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float sc = sm.m[w][h] == kNegInf ? 0.f : exp2f(sm.m[w][h] - mx);
        lt = fmaf(sm.l[w][h], sc, lt);
        o = fmaf(s_acc[w][h][d], sc, o);
      }
      if constexpr (FUSED) {
        if (add_new) {  // the new token, as one more wave holding a single row
          const float sc = exp2f(nr->x[h] - mx);
          lt += sc;
          o = fmaf(nr->v[d], sc, o);
        }
      }
    }
    const float val = lt > 0.f ? o / lt : 0.f;
    const float lse2 = lt > 0.f ? mx + __log2f(lt) : kNegInf;
    if (direct) {
      const size_t idx = (head0 + h) * kD + d;
      if (p.out_bf16)
        static_cast<uint16_t*>(p.out)[idx] = f32_to_bf16_rne(val);
      else
        static_cast<float*>(p.out)[idx] = val;
      if (p.lse != nullptr && d == 0) p.lse[head0 + h] = lse2 * kLn2;
    } else {
      p.ws_o[(slot * G + h) * kD + d] = val;
      if (d == 0) p.ws_lse[slot * G + h] = lse2;
    }
  }
  __syncthreads();  // LDS free for the caller
}

// Ring caches: grid of (b, kv head, split), one piece per workgroup; partial
// slot (b * Hkv + kv head) * num_splits + split.
template <int G, int NW, bool FUSED, bool I8>
__global__ __launch_bounds__(NW * 64) void decode_ring_kernel(DecodeParams p) {
  __shared__ Smem<G, NW, subtiles<G, false, I8>(), I8 ? 8 : 16> sm;
  const int ns = p.num_splits;
  const int split = blockIdx.x % ns;
  const int unit = blockIdx.x / ns;
  const int b = unit / p.num_kv_heads;
  const int kvh = unit - b * p.num_kv_heads;
  const int ntok = p.slots;
  const int t0 = split * p.split_tokens;
  const int t1 = min(t0 + p.split_tokens, ntok);
  const size_t slot = static_cast<size_t>(unit) * ns + split;
  if constexpr (FUSED) {
    __shared__ NewRow<G> nr;
    NewToken nt;
    nt.theta = p.freq.theta[threadIdx.x & 63];
    nt.pos = p.new_pos[b];
    nt.app = nt.pos >= 0;
    if (nt.app) {
      nt.slot = nt.pos < p.sinks ? nt.pos : p.sinks + nt.pos % p.window;
      nt.mine = nt.slot >= t0 && nt.slot < t1;
      nt.cpos = min(nt.pos, p.sinks + p.window - 1);
      nt.shift = p.shift_sinks && nt.cpos != nt.pos && t0 < p.sinks;
    }
    attend_piece<G, RingRows, NW, true, I8>(p, sm, b, kvh, t0, t1, ns == 1, slot, &nr, nt);
  } else {
    attend_piece<G, RingRows, NW, false, I8>(p, sm, b, kvh, t0, t1, ns == 1, slot);
  }
}

// A paging step folded into a pool decode (PagerFuse), split by launch: the
// attention launch fetches the staged blocks from the host store into the
// staging area, the merge launch places them in the pool.
constexpr unsigned kFetchCus = 8;  // one per XCD
struct PoolFetch {
  const void* host_k;
  const void* host_v;
  void* stage_k;
  void* stage_v;
  int32_t block_u4, n;
  int32_t src_block[kPagerFuseMax];
};
struct PoolPlace {
  const void* stage_k;
  const void* stage_v;
  void* k_pool;
  void* v_pool;
  uint8_t* valid;
  int32_t block_u4, n;
  int32_t dst_block[kPagerFuseMax];
  int32_t slot[kPagerFuseMax];
};

// Balanced schedule of a paged pool, in granules of 64 rows.  Sequence b
// contributes Hkv ranges of n_b = ceil(len_b / 64) granules (one per kv head,
// heads laid end to end), sequences in order; the total is
// T = Hkv * sum_b n_b.  Workgroup w of W (see share_start) owns granules
// [s(w), s(w+1)).  On bf16 pools with the grid of 4-wave workgroups
// s(w) = floor((16 w + w mod 2) T / (16 W)): workgroups of even index take
// 17/16 of an equal share, those of odd index 15/16.  Workgroup w runs on XCD
// w mod 8, and the even XCDs stream faster: measured against equal shares in
// the same run, these weights brought paged and long-pool-b16 calls 1.5-3.4%
// lower (1/8 instead of 1/16 overshot).  Elsewhere the shares stay equal,
// s(w) = floor(w T / W): the int8 kernels are bound by their VALU work, not
// by the stream (the weights made them 1.5-3.5% slower), and on the small
// pools' grid of 8-wave workgroups the weights measured no better or slower
// (long-pool-b1 within noise, its folded paging step 3% slower).
// The piece of unit
// u = b * Hkv + h inside workgroup w uses partial slot u + w (pieces in
// granule order move u or w forward by one each, so the slots are distinct
// and fewer than units + W).
// Rows of sequence b that the shared-prefix pass attends (0 without a plan);
// the pool kernel attends rows [shared_rows, len) of each sequence.
__device__ __forceinline__ int shared_rows(const DecodeParams& p, int b) {
  return p.plan != nullptr ? p.plan[kPlanHead + b] : 0;
}

__device__ __forceinline__ int granules(const DecodeParams& p, int b) {
  return (PoolRows::tokens(p, b) - shared_rows(p, b) + 63) >> 6;
}

// W is kPoolGrid or kPoolGrid / 2, a power of two (no 64-bit division), or
// that less the workgroups of kFetchCus CUs in a call with a folded paging
// step.
__device__ __forceinline__ int64_t share_start(int64_t w, int64_t total, int64_t nwg,
                                               bool i8) {
  const bool weighted = !i8 && nwg > kPoolGrid / 2;
  const int64_t c = 16 * w + (weighted ? (w & 1) : 0);  // cumulative weight, in sixteenths
  if ((nwg & (nwg - 1)) != 0)
    return static_cast<int64_t>(static_cast<uint64_t>(c * total) / static_cast<uint64_t>(16 * nwg));
  const int shift = __builtin_ctzll(static_cast<unsigned long long>(nwg)) + 4;
  return (c * total) >> shift;
}

__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint64_t u = static_cast<uint64_t>(x);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Sums over the workgroup (NT threads) of one or two values, the same
// result returned to every thread.  s_red holds 2 * NT / 64 entries.
template <int NT>
__device__ int64_t block_sum(int64_t x, int64_t* s_red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = x;
  __syncthreads();
  int64_t t = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) t += s_red[w];
  __syncthreads();  // s_red free again
  return uniform64(t);
}

template <int NT>
__device__ void block_sum2(int64_t& x, int64_t& y, int64_t* s_red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    x += __shfl_xor(x, off);
    y += __shfl_xor(y, off);
  }
  if ((threadIdx.x & 63) == 0) {
    s_red[threadIdx.x >> 6] = x;
    s_red[NT / 64 + (threadIdx.x >> 6)] = y;
  }
  __syncthreads();
  int64_t tx = 0, ty = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    tx += s_red[w];
    ty += s_red[NT / 64 + w];
  }
  __syncthreads();  // s_red free again
  x = uniform64(tx);
  y = uniform64(ty);
}

// Lengths (rows, clamped to the table) of NT consecutive sequences
// [first, first + NT), the exclusive prefix sums of their granule counts, and
// the state of a workgroup's walk over the units of its share (kept here, not
// in registers, while a piece is attended).
template <int NT>
struct SeqChunk {
  int32_t len[NT];    // rows attended here (after the shared ones)
  int32_t start[NT];  // rows attended by the shared-prefix pass
  int32_t excl[NT];
  int64_t red[2 * NT / 64];
  int32_t wsum[NT / 64];
  int64_t g0, g1;  // the workgroup's share of granules
  int64_t base;    // granules per kv head of the sequences before the chunk
  int32_t first, csum, i, h;  // chunk start and total; next sequence and kv head
};

// Loads the chunk of sequences starting at `first` into LDS; returns its total
// granule count (per kv head).  Called by every thread.
template <int NT>
__device__ int32_t load_chunk(const DecodeParams& p, SeqChunk<NT>& sc, int first) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = first + static_cast<int>(threadIdx.x);
  const int start = b < p.batch ? shared_rows(p, b) : 0;
  const int len = b < p.batch ? PoolRows::tokens(p, b) - start : 0;
  const int x = (len + 63) >> 6;
  int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) sc.wsum[wave] = incl;
  __syncthreads();  // also: the previous chunk's entries are no longer read
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int v = sc.wsum[w];
    before += w < wave ? v : 0;
    total += v;
  }
  sc.len[threadIdx.x] = len;
  sc.start[threadIdx.x] = start;
  sc.excl[threadIdx.x] = before + incl - x;
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(total);
}

// A piece: rows [t0, t1) of unit (b, h), whether the unit lies wholly inside
// the share (its output is then final), and its partial slot.
struct Piece {
  int b, h, t0, t1;
  bool direct;
  size_t slot;
};

// Moves the walk on to the next piece of the workgroup's share; false when
// the share holds no further piece.  Called by every thread.  Everything it
// needs between pieces lives in LDS, so no register is held across a piece.
template <int NT>
__device__ bool next_piece(const DecodeParams& p, SeqChunk<NT>& sc, Piece& pc) {
  const int64_t hkv = p.num_kv_heads;
  const int64_t g0 = uniform64(sc.g0);
  const int64_t g1 = uniform64(sc.g1);
  int64_t base = uniform64(sc.base);
  int first = __builtin_amdgcn_readfirstlane(sc.first);
  int csum = __builtin_amdgcn_readfirstlane(sc.csum);
  int i = __builtin_amdgcn_readfirstlane(sc.i);
  int h = __builtin_amdgcn_readfirstlane(sc.h);
  bool found = false;
  for (;;) {
    if (i == NT) {  // on into the next chunk
      if (first + NT >= p.batch) break;
      base += csum;
      first += NT;
      csum = load_chunk<NT>(p, sc, first);
      i = 0;
      h = 0;
    }
    const int b = first + i;
    if (b >= p.batch) break;
    const int len = __builtin_amdgcn_readfirstlane(sc.len[i]);
    const int64_t n = (len + 63) >> 6;
    const int64_t start = (base + __builtin_amdgcn_readfirstlane(sc.excl[i])) * hkv;
    if (start >= g1) break;
    if (n == 0 || h >= hkv) {
      ++i;
      h = 0;
      continue;
    }
    const int64_t u0 = start + h * n;
    const int64_t u1 = u0 + n;
    if (u0 >= g1) break;
    if (u1 > g0) {
      const int64_t e = ((g1 < u1 ? g1 : u1) - u0) * 64;
      const int start = __builtin_amdgcn_readfirstlane(sc.start[i]);
      pc.b = b;
      pc.h = h;
      pc.t0 = start + static_cast<int>(((g0 > u0 ? g0 : u0) - u0) * 64);
      pc.t1 = start + static_cast<int>(e < len ? e : static_cast<int64_t>(len));
      if (pc.t1 < pc.t0) pc.t1 = pc.t0;
      // a sharer's output also has the shared pass's partials: never direct
      pc.direct = g0 <= u0 && u1 <= g1 && start == 0;
      pc.slot = static_cast<size_t>(static_cast<int64_t>(b) * hkv + h + blockIdx.x);
      found = true;
    }
    ++h;
    if (found) break;
  }
  __syncthreads();  // every thread has read the walk state
  if (threadIdx.x == 0) {
    sc.base = base;
    sc.first = first;
    sc.csum = csum;
    sc.i = i;
    sc.h = h;
  }
  __syncthreads();
  return found;
}

// 8 / NW workgroups per CU (two 4-wave or one 8-wave): two waves per SIMD, at
// most 256 registers per lane.  The balanced grid is the first p.num_splits
// workgroups; those past it fetch the staged blocks of a folded paging step
// (f.n > 0) from the host store into the staging area, over the bus, while
// the attention workgroups read the pool.  They take CUs of their own: a CU
// holding an attention workgroup has no room for another.
template <int G, int NW, bool I8>
__device__ __forceinline__ void pool_attend(const DecodeParams& p) {
  constexpr int NT = NW * 64;
  __shared__ Smem<G, NW, subtiles<G, true, I8>(), I8 ? 8 : 16> sm;
  __shared__ SeqChunk<NT> sc;
  const int64_t hkv = p.num_kv_heads;
  const int64_t nwg = p.num_splits;
  const int64_t w = blockIdx.x;

  // Total granules: the first chunk's sum, plus a strided sum over the
  // sequences past it when the batch is larger than the workgroup.
  int32_t csum = load_chunk<NT>(p, sc, 0);
  int64_t rest = 0;
  for (int b = NT + threadIdx.x; b < p.batch; b += NT) rest += granules(p, b);
  if (p.batch > NT) rest = block_sum<NT>(rest, sc.red);
  const int64_t total = (csum + rest) * hkv;
  const int64_t g0 = share_start(w, total, nwg, p.i8);
  const int64_t g1 = w + 1 == nwg ? total : share_start(w + 1, total, nwg, p.i8);
  if (g0 >= g1) return;

  // Chunk holding the first sequence that ends past g0, and that sequence.
  int first = 0;
  int64_t base = 0;
  while ((base + csum) * hkv <= g0) {
    base += csum;
    first += NT;
    csum = load_chunk<NT>(p, sc, first);
  }
  // sequences of the chunk that end at or before g0 (the ends are sorted)
  const int i = __builtin_amdgcn_readfirstlane(
      __syncthreads_count((base + sc.excl[threadIdx.x] + ((sc.len[threadIdx.x] + 63) >> 6)) *
                              hkv <= g0));
  if (threadIdx.x == 0) {
    sc.g0 = g0;
    sc.g1 = g1;
    sc.base = base;
    sc.first = first;
    sc.csum = csum;
    sc.i = i;
    sc.h = 0;
  }
  __syncthreads();
  Piece pc;
  while (next_piece<NT>(p, sc, pc))
    attend_piece<G, PoolRows, NW, false, I8>(p, sm, pc.b, pc.h, pc.t0, pc.t1, pc.direct, pc.slot);
}

template <int G, int NW, bool I8>
__global__ __launch_bounds__(NW * 64, 8 / NW) void decode_pool_kernel(DecodeParams p) {
  pool_attend<G, NW, I8>(p);
}

// The same with a folded paging step: the workgroups past the balanced grid
// fetch.  A kernel of its own, so that the calls without paging pass no fetch
// descriptor (its block list doubles the kernel arguments).
template <int G, int NW, bool I8>
__global__ __launch_bounds__(NW * 64, 8 / NW) void decode_pool_fetch_kernel(DecodeParams p,
                                                                              PoolFetch f) {
  constexpr int NT = NW * 64;
  const int64_t nwg = p.num_splits;
  const int64_t w = blockIdx.x;
  if (w >= nwg) {  // fetch workgroup w - nwg of gridDim.x - nwg takes every such piece
    const int pieces = f.n * 2 * copy_pieces(f.block_u4, NT);
    for (int j = static_cast<int>(w - nwg); j < pieces; j += static_cast<int>(gridDim.x - nwg)) {
      const CopyPiece c = copy_piece(j, f.block_u4, NT);
      const uint4* src = static_cast<const uint4*>(c.tensor == 0 ? f.host_k : f.host_v) +
                         static_cast<size_t>(f.src_block[c.item]) * f.block_u4;
      uint4* dst = static_cast<uint4*>(c.tensor == 0 ? f.stage_k : f.stage_v) +
                   static_cast<size_t>(c.item) * f.block_u4;
      copy_block_piece(src, dst, c.begin, c.end, NT);
    }
    return;
  }
  pool_attend<G, NW, I8>(p);
}

// Combines the partials of one (sequence, query head) spread over several
// workgroups (a separate launch, so the partials written by the attention
// kernels are visible without any cross-workgroup fence):
//   M = max_s lse_s,  w_s = 2^(lse_s - M),  out = sum_s w_s o_s / sum_s w_s,
//   lse = (M + log2 sum_s w_s) ln 2.
// The partials of a (sequence, kv head) sit in consecutive slots: ring
// splits at (b * Hkv + kv head) * num_splits + split; pool pieces at
// u + w for the workgroups w whose share of granules meets the unit
// (workgroups with an empty share own no piece and are skipped), then, for a
// sequence the shared-prefix pass served, its prefix_chunks chunk partials
// at shared_base + c * B * Hkv + u.  A unit done by one workgroup wrote its
// output directly and is skipped; a pool sequence with nothing resident gets
// out = 0, lse = -inf here.  256 threads = 8 slot groups x 32 float4 columns;
// the partial rows are read by independent loads in flight together, and
// slots with lse = -inf are dropped with selects.
// The place part of a paging step folded into the call (f.n > 0) runs in
// the same launch (merge_place_kernel): f.n * 2 * copy_pieces(block_u4, 256)
// workgroups after the B * Hq merge workgroups move its blocks from the
// staging area into the pool and set their validity bytes.
// The attention kernel that read the pool has finished when this launch
// starts, and nothing in this launch reads the pool or the validity bytes,
// so the moves overlap the merge and are visible to the launches after it.
template <int PER, bool SHARED>  // partial rows per thread held in registers;
                                 // SHARED: the call may have shared-prefix chunks
__device__ __forceinline__ void merge_head(const DecodeParams& p, int pool) {
  constexpr int COLS = kD / 4;
  constexpr int GROUPS = 256 / COLS;
  // pool pieces (at most the grid), plus the shared chunks
  constexpr int kSlots = SHARED ? 1024 : 512;
  static_assert(kMaxSplits + (SHARED ? kPrefixChunks : 0) <= kSlots &&
                    kPoolGrid + (SHARED ? kPrefixChunks : 0) <= kSlots,
                "kSlots / 256 slots per thread");
  __shared__ float s_lse[kSlots];
  __shared__ float s_red_f[8];
  __shared__ float4 s_part[GROUPS][COLS];
  const size_t bh = blockIdx.x;
  const int b = static_cast<int>(bh / p.num_q_heads);
  const int hq = static_cast<int>(bh - static_cast<size_t>(b) * p.num_q_heads);
  const int g = p.num_q_heads / p.num_kv_heads;
  const int kvh = hq / g;
  const int h = hq - kvh * g;
  const int64_t unit = static_cast<int64_t>(b) * p.num_kv_heads + kvh;
  const int col = threadIdx.x % COLS;
  const int grp = threadIdx.x / COLS;

  int64_t first;  // slot of the first piece partial
  int count;      // piece partials (consecutive slots)
  int shared = 0; // chunk partials of the shared-prefix pass
  int64_t w0 = 0, nwg = 1, total = 0;
  if (!pool) {
    first = unit * p.num_splits;
    count = p.num_splits;
  } else {
    // granules of all sequences and of those before b, summed by the
    // whole workgroup
    __shared__ int64_t s_red[8];
    const int64_t hkv = p.num_kv_heads;
    nwg = p.num_splits;
    const int64_t n = granules(p, b);
    if constexpr (SHARED) shared = shared_rows(p, b) > 0 ? p.prefix_chunks : 0;
    int64_t all = 0, pb = 0;
    for (int bb = threadIdx.x; bb < p.batch; bb += 256) {
      const int x = granules(p, bb);
      all += x;
      pb += bb < b ? x : 0;
    }
    block_sum2<256>(all, pb, s_red);
    total = all * hkv;
    if (n == 0) {
      count = 0;
      first = 0;
    } else {
      const int64_t u0 = pb * hkv + kvh * n, u1 = u0 + n;
      auto owner = [&](int64_t x) {  // workgroup whose share holds granule x
        int64_t wq = static_cast<int64_t>(static_cast<double>(x) * static_cast<double>(nwg) /
                                          static_cast<double>(total));
        wq = wq < 0 ? 0 : (wq >= nwg ? nwg - 1 : wq);
        while (wq > 0 && share_start(wq, total, nwg, p.i8) > x) --wq;
        while (wq + 1 < nwg && share_start(wq + 1, total, nwg, p.i8) <= x) ++wq;
        return wq;
      };
      w0 = owner(u0);
      const int64_t w1 = owner(u1 - 1);
      count = static_cast<int>(w1 - w0 + 1);
      first = unit + w0;
    }
  }
  if (count == 1 && shared == 0) return;  // written directly by the attention kernel
  const int slots = count + shared;
  // with T >= 2 W every share holds at least one granule (each is at least
  // 15/16 of T / W): all of them present
  const bool dense = !pool || total >= 2 * nwg;
  auto present = [&](int k) {  // pool: the k-th workgroup of the run owns rows
    if (dense || k >= count) return true;
    const int64_t wk = w0 + k;
    const int64_t a = share_start(wk, total, nwg, p.i8);
    const int64_t e = wk + 1 == nwg ? total : share_start(wk + 1, total, nwg, p.i8);
    return a < e;
  };
  auto slot_of = [&](int k) -> size_t {  // partial slot of the k-th partial
    if (!SHARED || k < count) return static_cast<size_t>(first + k);
    return static_cast<size_t>(p.shared_base) +
           static_cast<size_t>(k - count) * p.batch * p.num_kv_heads + static_cast<size_t>(unit);
  };
  const float* lse = p.ws_lse;
  const float4* po = reinterpret_cast<const float4*>(p.ws_o);
  auto at = [&](int k) { return (slot_of(k) * g + h) * COLS + col; };
  float4 v[PER];
  float lv[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int s = grp + GROUPS * k;
    lv[k] = kNegInf;
    if (s < slots && present(s)) {
      v[k] = po[at(s)];
      lv[k] = lse[slot_of(s) * g + h];
    }
  }
  // Every slot's lse (thread t holds slots t + 256 i), then the maximum and
  // the weight sum by block reductions.
  float la[kSlots / 256];
  float mx = kNegInf;
#pragma unroll
  for (int i = 0; i < kSlots / 256; ++i) {
    const int sa = threadIdx.x + 256 * i;
    la[i] = kNegInf;
    if (sa < slots && present(sa)) la[i] = lse[slot_of(sa) * g + h];
    if (sa < slots) s_lse[sa] = la[i];
    mx = fmaxf(mx, la[i]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((threadIdx.x & 63) == 0) s_red_f[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(s_red_f[0], s_red_f[1]), fmaxf(s_red_f[2], s_red_f[3]));
  float wsum = 0.f;
  if (mx != kNegInf) {
#pragma unroll
    for (int i = 0; i < kSlots / 256; ++i) wsum += la[i] == kNegInf ? 0.f : exp2f(la[i] - mx);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) wsum += __shfl_xor(wsum, off);
  if ((threadIdx.x & 63) == 0) s_red_f[4 + (threadIdx.x >> 6)] = wsum;
  __syncthreads();
  wsum = (s_red_f[4] + s_red_f[5]) + (s_red_f[6] + s_red_f[7]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const bool use = lv[k] != kNegInf && mx != kNegInf;
    const float w = use ? exp2f(lv[k] - mx) : 0.f;
    acc.x += use ? w * v[k].x : 0.f;
    acc.y += use ? w * v[k].y : 0.f;
    acc.z += use ? w * v[k].z : 0.f;
    acc.w += use ? w * v[k].w : 0.f;
  }
  for (int s = grp + GROUPS * PER; s < slots; s += GROUPS) {  // beyond the registers
    const float l = s_lse[s];
    if (l == kNegInf || mx == kNegInf) continue;
    const float w = exp2f(l - mx);
    const float4 t = po[at(s)];
    acc.x = fmaf(w, t.x, acc.x);
    acc.y = fmaf(w, t.y, acc.y);
    acc.z = fmaf(w, t.z, acc.z);
    acc.w = fmaf(w, t.w, acc.w);
  }
  s_part[grp][col] = acc;
  __syncthreads();
  if (threadIdx.x < COLS) {
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int gg = 0; gg < GROUPS; ++gg) {
      t.x += s_part[gg][col].x;
      t.y += s_part[gg][col].y;
      t.z += s_part[gg][col].z;
      t.w += s_part[gg][col].w;
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    const float vals[4] = {t.x * inv, t.y * inv, t.z * inv, t.w * inv};
    const size_t idx = bh * kD + 4 * col;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (p.out_bf16)
        static_cast<uint16_t*>(p.out)[idx + e] = f32_to_bf16_rne(vals[e]);
      else
        static_cast<float*>(p.out)[idx + e] = vals[e];
    }
    if (p.lse != nullptr && col == 0) p.lse[bh] = wsum > 0.f ? (mx + __log2f(wsum)) * kLn2 : kNegInf;
  }
}
// Workgroup (sequence, query head) of the merge launch.
template <int PER, bool SHARED>
__global__ __launch_bounds__(256) void merge_kernel(DecodeParams p, int pool) {
  merge_head<PER, SHARED>(p, pool);
}

// The merge launch of a call with a folded paging step: the B * Hq merge
// workgroups, then the place workgroups.  A kernel of its own, so that the
// calls without paging pass no place descriptor (its block lists make the
// kernel arguments three times larger).
__global__ __launch_bounds__(256) void merge_place_kernel(DecodeParams p, PoolPlace f) {
  const size_t heads = static_cast<size_t>(p.batch) * p.num_q_heads;
  if (blockIdx.x >= heads) {
    const CopyPiece c = copy_piece(static_cast<int>(blockIdx.x - heads), f.block_u4, 256);
    const uint4* src = static_cast<const uint4*>(c.tensor == 0 ? f.stage_k : f.stage_v) +
                       static_cast<size_t>(c.item) * f.block_u4;
    uint4* dst = static_cast<uint4*>(c.tensor == 0 ? f.k_pool : f.v_pool) +
                 static_cast<size_t>(f.dst_block[c.item]) * f.block_u4;
    copy_block_piece(src, dst, c.begin, c.end, 256);
    if (c.tensor == 0 && c.begin == 0 && threadIdx.x == 0) f.valid[f.slot[c.item]] = 1;
    return;
  }
  merge_head<8, true>(p, 1);
}

template <int NW, bool I8>
hipError_t decode_pool_kernel_launch(const DecodeParams& p, const PoolFetch& f,
                                     hipStream_t stream) {
  // the balanced grid, then the fetch workgroups of a folded paging step:
  // those of one CU per XCD
  const unsigned grid = static_cast<unsigned>(p.num_splits) + (f.n > 0 ? kFetchCus * (8 / NW) : 0u);
  auto go = [&](auto plain, auto fetch) {
    if (f.n > 0)
      fetch<<<grid, NW * 64, 0, stream>>>(p, f);
    else
      plain<<<grid, NW * 64, 0, stream>>>(p);
  };
  switch (p.num_q_heads / p.num_kv_heads) {
    case 1: go(decode_pool_kernel<1, NW, I8>, decode_pool_fetch_kernel<1, NW, I8>); break;
    case 2: go(decode_pool_kernel<2, NW, I8>, decode_pool_fetch_kernel<2, NW, I8>); break;
    case 3: go(decode_pool_kernel<3, NW, I8>, decode_pool_fetch_kernel<3, NW, I8>); break;
    case 4: go(decode_pool_kernel<4, NW, I8>, decode_pool_fetch_kernel<4, NW, I8>); break;
    case 6: go(decode_pool_kernel<6, NW, I8>, decode_pool_fetch_kernel<6, NW, I8>); break;
    case 8: go(decode_pool_kernel<8, NW, I8>, decode_pool_fetch_kernel<8, NW, I8>); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int NW, bool FUSED, bool I8>
hipError_t decode_ring_kernel_launch(const DecodeParams& p, unsigned grid, hipStream_t stream) {
  switch (p.num_q_heads / p.num_kv_heads) {
    case 1: decode_ring_kernel<1, NW, FUSED, I8><<<grid, NW * 64, 0, stream>>>(p); break;
    case 2: decode_ring_kernel<2, NW, FUSED, I8><<<grid, NW * 64, 0, stream>>>(p); break;
    case 3: decode_ring_kernel<3, NW, FUSED, I8><<<grid, NW * 64, 0, stream>>>(p); break;
    case 4: decode_ring_kernel<4, NW, FUSED, I8><<<grid, NW * 64, 0, stream>>>(p); break;
    case 6: decode_ring_kernel<6, NW, FUSED, I8><<<grid, NW * 64, 0, stream>>>(p); break;
    case 8: decode_ring_kernel<8, NW, FUSED, I8><<<grid, NW * 64, 0, stream>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mfma_ring(const DecodeParams& p, hipStream_t stream) {
  const unsigned grid =
      static_cast<unsigned>(p.batch) * static_cast<unsigned>(p.num_kv_heads) * p.num_splits;
  // p.new_pos set: the fused step (append of one token per sequence + decode)
  const bool fused = p.new_pos != nullptr;
  hipError_t err;
  if (p.i8)
    err = fused ? decode_ring_kernel_launch<kRingWaves, true, true>(p, grid, stream)
                : decode_ring_kernel_launch<kRingWaves, false, true>(p, grid, stream);
  else
    err = fused ? decode_ring_kernel_launch<kRingWaves, true, false>(p, grid, stream)
                : decode_ring_kernel_launch<kRingWaves, false, false>(p, grid, stream);
  if (err != hipSuccess || p.num_splits == 1) return err;
  const unsigned heads = static_cast<unsigned>(p.batch) * static_cast<unsigned>(p.num_q_heads);
  merge_kernel<8, false><<<heads, 256, 0, stream>>>(p, 0);
  return hipGetLastError();
}

hipError_t launch_decode_mfma_pool(const DecodeParams& p_in, hipStream_t stream,
                                   const PagerFuse* fuse) {
  // p.num_splits carries the size of the balanced grid: kPoolGrid 4-wave
  // workgroups, or half as many 8-wave ones for small pools
  DecodeParams p = p_in;
  hipError_t err;
  if (prefix_pass_applies(p)) {  // finds and attends the shared prefix, writes the plan
    err = launch_shared_prefix(p, stream);
    if (err != hipSuccess) return err;
  } else {
    p.plan = nullptr;
  }
  PoolFetch fetch{};
  PoolPlace place{};
  if (fuse != nullptr && fuse->n > 0) {
    fetch.host_k = fuse->host_k;
    fetch.host_v = fuse->host_v;
    fetch.stage_k = fuse->stage_k;
    fetch.stage_v = fuse->stage_v;
    place.stage_k = fuse->stage_k;
    place.stage_v = fuse->stage_v;
    place.k_pool = fuse->k_pool;
    place.v_pool = fuse->v_pool;
    place.valid = fuse->valid;
    fetch.block_u4 = place.block_u4 = fuse->block_u4;
    fetch.n = place.n = fuse->n;
    for (int i = 0; i < fuse->n; ++i) {
      fetch.src_block[i] = fuse->src_block[i];
      place.dst_block[i] = fuse->dst_block[i];
      place.slot[i] = fuse->slot[i];
    }
  }
  const bool wide = p.num_splits == kPoolGrid;  // 4-wave workgroups
  // a folded paging step leaves kFetchCus CUs to the fetch: the balanced
  // grid (and the merge) covers the rest
  if (fetch.n > 0) p.num_splits -= static_cast<int>(kFetchCus) * (wide ? 2 : 1);
  if (p.i8)
    err = wide ? decode_pool_kernel_launch<4, true>(p, fetch, stream)
               : decode_pool_kernel_launch<8, true>(p, fetch, stream);
  else
    err = wide ? decode_pool_kernel_launch<4, false>(p, fetch, stream)
               : decode_pool_kernel_launch<8, false>(p, fetch, stream);
  if (err != hipSuccess) return err;
  const unsigned heads = static_cast<unsigned>(p.batch) * static_cast<unsigned>(p.num_q_heads);
  if (place.n > 0) {
    const unsigned copy_wgs =
        static_cast<unsigned>(place.n * 2 * copy_pieces(place.block_u4, 256));
    merge_place_kernel<<<copy_wgs + heads, 256, 0, stream>>>(p, place);
  } else if (p.plan != nullptr) {  // the shared-prefix pass ran: chunk partials
    merge_kernel<8, true><<<heads, 256, 0, stream>>>(p, 1);
  } else {
    merge_kernel<8, false><<<heads, 256, 0, stream>>>(p, 1);
  }
  return hipGetLastError();
}

}  // namespace swa
