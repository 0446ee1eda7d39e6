// Read half of the decode step for bf16 caches with head_dim 128: split-K
// over the resident rows, q-group x K-tile scores on the matrix cores, online
// softmax and P*V in fp32 registers, in-workgroup merge of the waves.  A
// sequence that fits one split gets its output written directly (one launch
// per decode call); longer ones are combined by a small merge launch.
//
// Math as in decode.hip ([sink] weight formula; [kvc] §2.2).  Only the
// resident rows take part: empty ring slots, absent or out-of-range blocks and
// rows past the sequence length are removed with selects, never multiplied by
// zero ([pool] "absent blocks are as if they did not exist").
//
// Workgroup = NW waves = one (sequence b, kv head, split).  A split is a
// contiguous range of split_tokens rows; its tiles are dealt to the waves
// round-robin, so the workgroup streams contiguous memory.
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
#include <type_traits>

#include "device_common.h"
#include "swa_internal.h"

namespace swa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309417f;
constexpr int kD = 128;
constexpr int kKSteps = kD / 32;

__device__ __forceinline__ bf16x8_t as_bf16x8(const Vec16& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// K/V rows are read once per step and never again before the whole cache has
// streamed past: non-temporal loads keep them from displacing reused lines.
__device__ __forceinline__ Vec16 load16_stream(const uint16_t* p) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  Vec16 r;
  r.w[0] = v[0];
  r.w[1] = v[1];
  r.w[2] = v[2];
  r.w[3] = v[3];
  return r;
}

// Value of lane (16 * (l / 16) + SRC) for every lane l: broadcast inside each
// 16-lane row.
template <int SRC>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + SRC, 0xf, 0xf,
                                         false));
}

__device__ __forceinline__ float xor_max(float x, int mask) {
  return fmaxf(x, __shfl_xor(x, mask));
}

// Largest block-table span one split can touch: splits are at most 8192 rows
// and blocks at least 16 rows, plus one for a split that starts mid-block.
constexpr int kMaxSplitBlocks = 8192 / 16 + 1;
constexpr int kMaxSplits = 512;  // splits per sequence (the plan never exceeds it)

// Ring: rows of head (b, h) are contiguous, slot t at row t; a row is
// resident iff its slot holds a position.
struct RingRows {
  const int32_t* slot_pos;
  size_t head_base;  // element offset of slot 0 of head (b, h)
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
  __device__ bool row_ok(int t) const { return slot_pos[t] >= 0; }
};

// Pool: token t lives in block block_table[b][t >> shift], row t & (bs - 1);
// a 16-row subtile never straddles a block (bs is a multiple of 16).  The
// split's block ids are staged in LDS once, with -1 for absent blocks (flagged
// invalid, negative or past the pool), so the row loop never waits on a
// dependent table load.
struct PoolRows {
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
    const int blk = s_blk[(t >> p.block_shift) - (t0 >> p.block_shift)];
    const int r = t & ((1 << p.block_shift) - 1);
    base = ((static_cast<size_t>(blk < 0 ? 0 : blk) * p.num_kv_heads + h) << p.block_shift) * kD +
           static_cast<size_t>(r) * kD;
    return blk >= 0;
  }
  __device__ bool row_ok(int) const { return true; }
};

// Row subtiles (16 rows each) per wave tile: 4 when few query heads share the
// kv head, fewer when the P*V accumulators take more registers (8-wave
// workgroups cap a wave at 256 VGPRs).
template <int G>
constexpr int subtiles() { return G <= 2 ? 4 : (G < 8 ? 2 : 1); }

template <int G, class Rows, int NW>
__global__ __launch_bounds__(NW * 64) void decode_mfma_kernel(DecodeParams p) {
  static_assert(G >= 1 && G <= 16, "q heads per kv head");
  constexpr int NS = subtiles<G>();
  constexpr int TILE = 16 * NS;
  // LDS: each wave's K tile while streaming; the same bytes hold the waves'
  // P*V accumulators for the final merge.
  constexpr int KBUF = TILE * 16;  // 16-byte chunks per wave: TILE rows x 256 B
  constexpr size_t KBYTES = static_cast<size_t>(NW) * KBUF * 16;
  constexpr size_t ABYTES = static_cast<size_t>(NW) * G * kD * sizeof(float);
  __shared__ __attribute__((aligned(16))) unsigned char s_raw[KBYTES > ABYTES ? KBYTES : ABYTES];
  __shared__ float s_m[NW][G];
  __shared__ float s_l[NW][G];
  __shared__ int32_t s_blk[kMaxSplitBlocks];
  float(*s_acc)[G][kD] = reinterpret_cast<float(*)[G][kD]>(s_raw);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lq = lane >> 4;
  const int lc = lane & 15;
  const int ns = p.num_splits;
  const int split = blockIdx.x % ns;
  const int unit = blockIdx.x / ns;
  const int b = unit / p.num_kv_heads;
  const int kvh = unit - b * p.num_kv_heads;
  const int ntok = Rows::tokens(p, b);
  const int nsb = ntok > 0 ? (ntok + p.split_tokens - 1) / p.split_tokens : 1;
  if (split >= nsb) return;  // past the sequence: this workgroup takes no part
  const int t0 = split * p.split_tokens;
  const int t1 = min(t0 + p.split_tokens, ntok);
  const size_t head0 = static_cast<size_t>(b) * p.num_q_heads + static_cast<size_t>(kvh) * G;
  const Rows rows(p, b, kvh);
  if (t1 > t0) rows.stage(p, t0, t1, s_blk);
  __syncthreads();
  const uint16_t* kb = static_cast<const uint16_t*>(p.k);
  const uint16_t* vb = static_cast<const uint16_t*>(p.v);

  // B operand: the g query heads of this kv head, zero-padded to 16.
  bf16x8_t qop[kKSteps];
  {
    const uint16_t* qb = static_cast<const uint16_t*>(p.q);
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) {
      Vec16 v{};
      if (lc < G) v = load16(qb + (head0 + lc) * kD + 32 * s + 8 * lq);
      qop[s] = as_bf16x8(v);
    }
  }

  const float c = p.score_scale_log2;
  float m = kNegInf;  // running max of head lc (log2 units)
  float lsum = 0.f;   // this lane's share of the running sum of head lc
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

  // This wave's K staging area: row rho of subtile u, 16-byte chunk c lives at
  // chunk (u * 16 + rho) * 16 + (c ^ rho), so both the row-wise writes and the
  // operand-wise reads below touch 16 distinct bank groups per 16 lanes.
  uint4* s_k = reinterpret_cast<uint4*>(s_raw) + wave * KBUF;

  for (int ts = t0 + wave * TILE; ts < t1; ts += NW * TILE) {
    Vec16 kr[NS][4];  // row-wise K chunks: row 4i + lq of subtile u, chunk lc
    Vec16 vr[NS][4];  // V: row 4lq + r of subtile u, chunk lc
    uint32_t vm[NS];  // bit i: row ts + 16u + i is resident
    size_t base[NS];
    bool live[NS];
    // Every load instruction reads four whole 256-byte rows; K first, so the
    // score phase waits on K while the V loads are still in flight.
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int tu = ts + 16 * u;
      vm[u] = 0;
      base[u] = 0;
      live[u] = tu < t1 && rows.subtile(p, s_blk, t0, tu, base[u]);
      if (live[u]) {
        const int tk = tu + lc;
        const bool okk = tk < t1 && rows.row_ok(tk);
        vm[u] = static_cast<uint32_t>(__ballot(okk)) & 0xffffu;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rho = 4 * i + lq;
          const size_t koff = base[u] + static_cast<size_t>(tu + rho < t1 ? rho : 0) * kD;
          kr[u][i] = load16_stream(kb + koff + 8 * lc);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) kr[u][i] = Vec16{};
      }
    }
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int tu = ts + 16 * u;
      if (live[u]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * lq + r;
          const size_t voff = base[u] + static_cast<size_t>(tu + i < t1 ? i : 0) * kD;
          vr[u][r] = load16_stream(vb + voff + 8 * lc);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) vr[u][r] = Vec16{};
      }
    }

    // K chunks into the MFMA A-operand layout through LDS (DS instructions of
    // one wave execute in order; the wave barriers only stop the compiler from
    // moving LDS accesses across each other).
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < NS; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rho = 4 * i + lq;
        s_k[(u * 16 + rho) * 16 + (lc ^ rho)] =
            make_uint4(kr[u][i].w[0], kr[u][i].w[1], kr[u][i].w[2], kr[u][i].w[3]);
      }
    __builtin_amdgcn_wave_barrier();
    Vec16 ka[NS][kKSteps];  // lane l: row lc, dims 32s + 8lq .. +7
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
    uint32_t all = 0xffffu;
#pragma unroll
    for (int u = 0; u < NS; ++u) all &= vm[u];
    const bool all_ok = all == 0xffffu;

    // scores (log2 units) of rows 16u + 4lq + r for head lc
    float x[NS][4];
    float tmax = kNegInf;
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < kKSteps; ++s)
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka[u][s]), qop[s], d, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = (vm[u] >> (4 * lq + r)) & 1u;
        x[u][r] = ok ? d[r] * c : kNegInf;
        tmax = fmaxf(tmax, x[u][r]);
      }
    }
    tmax = xor_max(tmax, 16);
    tmax = xor_max(tmax, 32);
    const float mn = fmaxf(m, tmax);
    // mn == -inf: nothing resident so far for this head; keep everything at 0
    const float alpha = mn == kNegInf ? 1.f : exp2f(m - mn);
    m = mn;
    float pr[NS][4];
    float tsum = 0.f;
#pragma unroll
    for (int u = 0; u < NS; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[u][r] = x[u][r] == kNegInf ? 0.f : exp2f(x[u][r] - mn);
        tsum += pr[u][r];
      }
    lsum = lsum * alpha + tsum;

    // P * V
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float a = 1.f;
      switch (h) {  // compile-time dispatch of the DPP source lane
#define SWA_B(H) case H: a = row_bcast<H>(alpha); break;
        SWA_B(0) SWA_B(1) SWA_B(2) SWA_B(3) SWA_B(4) SWA_B(5) SWA_B(6) SWA_B(7)
        SWA_B(8) SWA_B(9) SWA_B(10) SWA_B(11) SWA_B(12) SWA_B(13) SWA_B(14) SWA_B(15)
#undef SWA_B
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= a;
    }
#pragma unroll
    for (int u = 0; u < NS; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = bf16_lo(vr[u][r].w[i]);
          v[2 * i + 1] = bf16_hi(vr[u][r].w[i]);
        }
        if (!all_ok) {
          const bool ok = (vm[u] >> (4 * lq + r)) & 1u;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = ok ? v[e] : 0.f;
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float ph = 0.f;
          switch (h) {
#define SWA_B(H) case H: ph = row_bcast<H>(pr[u][r]); break;
            SWA_B(0) SWA_B(1) SWA_B(2) SWA_B(3) SWA_B(4) SWA_B(5) SWA_B(6) SWA_B(7)
            SWA_B(8) SWA_B(9) SWA_B(10) SWA_B(11) SWA_B(12) SWA_B(13) SWA_B(14) SWA_B(15)
#undef SWA_B
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(ph, v[e], acc[h][e]);
        }
      }
  }

  // Wave totals: sum the four row groups.
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[h][e] += __shfl_xor(acc[h][e], 16);
      acc[h][e] += __shfl_xor(acc[h][e], 32);
    }
  __syncthreads();  // every wave is done with its K staging area (aliases s_acc)
  if (lane < G) {
    s_m[wave][lane] = m;
    s_l[wave][lane] = lsum;
  }
  if (lq == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[wave][h][8 * lc + e] = acc[h][e];
  }
  __syncthreads();

  // Workgroup merge: thread -> (head, dim) pairs.
  const bool direct = nsb == 1;  // the whole sequence in this workgroup: write the output
  float* ws_o = p.ws_o + (head0 * ns + static_cast<size_t>(split)) * kD;  // head h: + h * ns * kD
  float* ws_lse = p.ws_lse + head0 * ns + split;                          // head h: + h * ns
  for (int i = threadIdx.x; i < G * kD; i += NW * 64) {
    const int h = i / kD;
    const int d = i - h * kD;
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, s_m[w][h]);
    float lt = 0.f, o = 0.f;
    if (mx != kNegInf) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float sc = s_m[w][h] == kNegInf ? 0.f : exp2f(s_m[w][h] - mx);
        lt = fmaf(s_l[w][h], sc, lt);
        o = fmaf(s_acc[w][h][d], sc, o);
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
      ws_o[static_cast<size_t>(h) * ns * kD + d] = val;
      if (d == 0) ws_lse[static_cast<size_t>(h) * ns] = lse2;
    }
  }
}

// Combines the splits of one (sequence, query head) when its sequence was cut
// into several workgroups (a separate launch, so the partials written by the
// split kernel are visible without any cross-workgroup fence):
//   M = max_s lse_s,  w_s = 2^(lse_s - M),  out = sum_s w_s o_s / sum_s w_s,
//   lse = (M + log2 sum_s w_s) ln 2.
// Sequences that fitted one split wrote their output directly and are
// skipped.  256 threads = 8 split groups x 32 float4 columns, so every
// partial row is read by independent loads in flight together.  Splits with
// lse = -inf hold no row: weight 0, their partial is never read.
__global__ __launch_bounds__(256) void merge_splits_kernel(DecodeParams p, int ragged) {
  constexpr int COLS = kD / 4;
  constexpr int GROUPS = 256 / COLS;
  __shared__ float s_lse[kMaxSplits];
  __shared__ float4 s_part[GROUPS][COLS];
  const size_t bh = blockIdx.x;
  const int b = static_cast<int>(bh / p.num_q_heads);
  const int ns = p.num_splits;
  int nsb = ns;
  if (ragged) {
    const int ntok = PoolRows::tokens(p, b);
    nsb = ntok > 0 ? (ntok + p.split_tokens - 1) / p.split_tokens : 1;
  }
  if (nsb <= 1) return;
  const float* lse = p.ws_lse + bh * ns;
  for (int s = threadIdx.x; s < nsb; s += 256) s_lse[s] = lse[s];
  __syncthreads();
  float mx = kNegInf;
  for (int s = 0; s < nsb; ++s) mx = fmaxf(mx, s_lse[s]);
  float wsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const int col = threadIdx.x % COLS;
  const int grp = threadIdx.x / COLS;
  if (mx != kNegInf) {
    for (int s = 0; s < nsb; ++s) wsum += s_lse[s] == kNegInf ? 0.f : exp2f(s_lse[s] - mx);
    const float4* po = reinterpret_cast<const float4*>(p.ws_o + bh * ns * kD);
#pragma unroll 4
    for (int s = grp; s < nsb; s += GROUPS) {
      const float l = s_lse[s];
      if (l == kNegInf) continue;
      const float w = exp2f(l - mx);
      const float4 v = po[static_cast<size_t>(s) * COLS + col];
      acc.x = fmaf(w, v.x, acc.x);
      acc.y = fmaf(w, v.y, acc.y);
      acc.z = fmaf(w, v.z, acc.z);
      acc.w = fmaf(w, v.w, acc.w);
    }
  }
  s_part[grp][col] = acc;
  __syncthreads();
  if (threadIdx.x < COLS) {
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int g = 0; g < GROUPS; ++g) {
      t.x += s_part[g][col].x;
      t.y += s_part[g][col].y;
      t.z += s_part[g][col].z;
      t.w += s_part[g][col].w;
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

template <class Rows, int NW>
hipError_t launch_rows(const DecodeParams& p, int ragged, hipStream_t stream) {
  const unsigned grid =
      static_cast<unsigned>(p.batch) * static_cast<unsigned>(p.num_kv_heads) * p.num_splits;
  switch (p.num_q_heads / p.num_kv_heads) {
#define SWA_CASE(G)                                                             \
  case G:                                                                       \
    decode_mfma_kernel<G, Rows, NW><<<grid, NW * 64, 0, stream>>>(p);           \
    break;
    SWA_CASE(1)
    SWA_CASE(2)
    SWA_CASE(3)
    SWA_CASE(4)
    SWA_CASE(6)
    SWA_CASE(8)
#undef SWA_CASE
    default:
      return hipErrorInvalidValue;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.num_splits == 1) return err;
  const unsigned heads = static_cast<unsigned>(p.batch) * static_cast<unsigned>(p.num_q_heads);
  merge_splits_kernel<<<heads, 256, 0, stream>>>(p, ragged);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mfma_ring(const DecodeParams& p, hipStream_t stream) {
  return launch_rows<RingRows, kRingWaves>(p, 0, stream);
}

hipError_t launch_decode_mfma_pool(const DecodeParams& p, hipStream_t stream) {
  // Many workgroups (ragged or long pools): 4-wave workgroups, two per CU, so
  // one workgroup's start and end overlap the other's streaming.  Few
  // workgroups: 8 waves each, to keep enough waves per CU.
  const int64_t wgs = static_cast<int64_t>(p.batch) * p.num_kv_heads * p.num_splits;
  if (wgs >= kPoolManyWorkgroups) return launch_rows<PoolRows, 4>(p, 1, stream);
  return launch_rows<PoolRows, 8>(p, 1, stream);
}

}  // namespace swa
