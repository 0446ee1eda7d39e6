// Read half of the decode step: one query per head attends to the resident
// rows of its sequence, split-K over the rows, then a log-sum-exp merge.
//
// Math ([sink] weight formula; [kvc] §2.2): s = scale * <q, k>,
// out = sum_j exp(s_j) v_j / sum_j exp(s_j), over exactly the resident rows.
// Softmax does not care about row order, so the ring is read in place
// without restoring chronological order (the [ring] page, §5.2, warns that a
// FlashAttention-style call would need it reordered first).
//
// Work decomposition.  A workgroup is one wave64 and owns one (sequence,
// kv head, split) where a split is a contiguous range of split_tokens rows of
// that head.  All g = Hq/Hkv query heads of the kv head are handled by the
// same wave, so every K/V byte is read from HBM once per step (GQA: [share]
// §2.2, §4.1).  Rows are streamed with 16-byte loads, LPR lanes per row, so
// each wave load instruction covers RPI whole rows of contiguous memory
// (head-major layout: one head's rows are adjacent).  Per tile of
// TILE = RPI * NSTEP rows: partial dot products are reduced across the LPR
// lanes of a row, the running max / sum of the online softmax are updated
// (base-2 exponentials with the scale folded in), and P * V is accumulated
// in float32 registers.  At the end the RPI row groups are reduced and the
// wave writes its partial output (normalised) and base-2 log-sum-exp.
//
// Rows that are not resident (empty ring slot, absent or out-of-range
// block, past seq_len, past the split) are never read into arithmetic: their
// score is replaced by -inf and their V by 0 with selects, so NaN garbage in
// an empty slot cannot leak ([pool] "absent blocks are as if they did not
// exist").
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "swa_internal.h"

namespace swa {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309417f;
constexpr int kNumSteps = 8;  // load instructions per tensor per tile

// Stored element kinds: float32, bf16, int8 codes with one float32 scale per
// row (queries are bf16 for int8 caches).
enum Kind { kF32 = 0, kBF16 = 1, kI8 = 2 };

template <int KIND, int D>
struct Geo {
  static constexpr int kElemBytes = KIND == kF32 ? 4 : (KIND == kBF16 ? 2 : 1);
  // elements per lane per row: one 16-byte load (8-byte loads for int8, which
  // keeps the per-lane query and accumulator slices at 8 elements)
  static constexpr int kEPL = KIND == kI8 ? 8 : 16 / kElemBytes;
  static constexpr int kLPR = D / kEPL;         // lanes per row
  static constexpr int kRPI = 64 / kLPR;        // rows per wave load instruction
  static_assert(kLPR >= 1 && kLPR <= 64 && 64 % kLPR == 0, "row must split evenly over a wave");
};

template <int KIND>
struct Unpack;
template <>
struct Unpack<kBF16> {
  __device__ static void run(const Vec16& v, float* x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_lo(v.w[i]);
      x[2 * i + 1] = bf16_hi(v.w[i]);
    }
  }
};
template <>
struct Unpack<kF32> {
  __device__ static void run(const Vec16& v, float* x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(v.w[i]);
  }
};
template <>
struct Unpack<kI8> {  // 8 signed bytes in w[0], w[1]; exact in float
  __device__ static void run(const Vec16& v, float* x) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        x[4 * i + k] = static_cast<float>(static_cast<int8_t>((v.w[i] >> (8 * k)) & 0xffu));
  }
};

// One lane's slice of a row: 16 bytes, or 8 for int8.
template <int KIND>
__device__ __forceinline__ Vec16 load_slice(const void* p) {
  if constexpr (KIND == kI8) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    Vec16 r;
    r.w[0] = v.x;
    r.w[1] = v.y;
    r.w[2] = 0u;
    r.w[3] = 0u;
    return r;
  } else {
    return load16(p);
  }
}

// The EPL query elements of one lane: bf16 for bf16 and int8 caches.
template <int KIND, int EPL>
__device__ void load_q(const void* q, size_t elem, float* x) {
  if constexpr (KIND == kF32) {
    Unpack<kF32>::run(load16(static_cast<const float*>(q) + elem), x);
  } else {
#pragma unroll
    for (int c = 0; c < EPL; c += 8)
      Unpack<kBF16>::run(load16(static_cast<const uint16_t*>(q) + elem + c), x + c);
  }
}

// Ring cache: token index = slot; resident iff the slot holds a position.
struct RingAddr {
  __device__ static int tokens(const DecodeParams& p, int) { return p.slots; }
  template <int D>
  __device__ static bool row(const DecodeParams& p, int b, int h, int t, size_t& off) {
    off = ((static_cast<size_t>(b) * p.num_kv_heads + h) * p.slots + t) * D;
    return p.slot_pos[static_cast<size_t>(b) * p.slots + t] >= 0;
  }
};

// Paged pool: token t of sequence b lives in block block_table[b][t / bs],
// row t % bs; resident iff the entry is valid and names a pool block.
struct PoolAddr {
  __device__ static int tokens(const DecodeParams& p, int b) {
    const int n = p.seq_lens[b];
    const int cap = p.max_blocks << p.block_shift;
    return n < 0 ? 0 : (n > cap ? cap : n);
  }
  template <int D>
  __device__ static bool row(const DecodeParams& p, int b, int h, int t, size_t& off) {
    const int j = t >> p.block_shift;
    const int r = t & ((1 << p.block_shift) - 1);
    const size_t e = static_cast<size_t>(b) * p.max_blocks + j;
    const int blk = p.block_table[e];
    const bool ok = blk >= 0 && blk < p.num_phys_blocks &&
                    (p.block_valid == nullptr || p.block_valid[e] != 0);
    off = ok ? (((static_cast<size_t>(blk) * p.num_kv_heads + h) << p.block_shift) + r) * D : 0;
    return ok;
  }
};

template <int KIND, int D, int G, class Addr>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeParams p) {
  using Gm = Geo<KIND, D>;
  using T = std::conditional_t<KIND == kF32, float, std::conditional_t<KIND == kBF16, uint16_t, int8_t>>;
  constexpr bool I8 = KIND == kI8;
  constexpr int kShiftD = D == 64 ? 6 : 7;  // row index = element offset >> kShiftD
  constexpr int EPL = Gm::kEPL, LPR = Gm::kLPR, RPI = Gm::kRPI;
  constexpr int TILE = RPI * kNumSteps;

  const int lane = threadIdx.x;
  const int split = blockIdx.x % p.num_splits;
  const int unit = blockIdx.x / p.num_splits;
  const int b = unit / p.num_kv_heads;
  const int kvh = unit - b * p.num_kv_heads;
  const int ntok = Addr::tokens(p, b);
  const int t0 = split * p.split_tokens;
  const int t1 = min(t0 + p.split_tokens, ntok);
  const size_t head0 = static_cast<size_t>(b) * p.num_q_heads + static_cast<size_t>(kvh) * G;
  float* lse_out = p.ws_lse + head0 * p.num_splits + split;  // + g * num_splits

  const int rl = lane / LPR;  // row within a load instruction
  const int cl = lane % LPR;  // 16-byte column chunk within the row
  // One split per sequence: this wave's result is final and goes straight
  // to out / lse (what the merge of a single split would write), and the
  // merge is not launched.
  const bool direct = p.num_splits == 1;
  auto write_out = [&](int g, int e0, const float* v) {  // v[0..3]: dims cl * EPL + e0 ..
    const size_t at = (head0 + g) * D + cl * EPL + e0;
    if (p.out_bf16) {
      uint16_t* o = static_cast<uint16_t*>(p.out) + at;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = f32_to_bf16_rne(v[i]);
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(p.out) + at) =
          make_float4(v[0], v[1], v[2], v[3]);
    }
  };

  if (t0 >= t1) {  // nothing of this sequence falls in the split
    if (direct) {
      const float z[4] = {0.f, 0.f, 0.f, 0.f};
      if (lane < LPR)
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < EPL; e += 4) write_out(g, e, z);
      if (lane < G && p.lse != nullptr) p.lse[head0 + lane] = kNegInf;
    } else if (lane < G) {
      lse_out[static_cast<size_t>(lane) * p.num_splits] = kNegInf;
    }
    return;
  }

  const float c = p.score_scale_log2;

  float q[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) load_q<KIND, EPL>(p.q, (head0 + g) * D + cl * EPL, q[g]);

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }

  const T* kbase = static_cast<const T*>(p.k) + cl * EPL;
  const T* vbase = static_cast<const T*>(p.v) + cl * EPL;

  for (int ts = t0; ts < t1; ts += TILE) {
    Vec16 kr[kNumSteps], vr[kNumSteps];
    bool ok[kNumSteps];
    float ksc[kNumSteps], vsc[kNumSteps];  // int8: the rows' scales
#pragma unroll
    for (int i = 0; i < kNumSteps; ++i) {
      const int t = ts + i * RPI + rl;
      const bool in = t < t1;
      size_t off;
      ok[i] = Addr::template row<D>(p, b, kvh, in ? t : t0, off) && in;
      kr[i] = load_slice<KIND>(kbase + off);
      vr[i] = load_slice<KIND>(vbase + off);
      if constexpr (I8) {
        ksc[i] = p.k_scale[off >> kShiftD];
        vsc[i] = p.v_scale[off >> kShiftD];
      }
    }

    float s[G][kNumSteps];
#pragma unroll
    for (int i = 0; i < kNumSteps; ++i) {
      float kx[EPL];
      Unpack<KIND>::run(kr[i], kx);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) a = fmaf(q[g][e], kx[e], a);
#pragma unroll
        for (int o = 1; o < LPR; o <<= 1) a += __shfl_xor(a, o);
        if constexpr (I8) a *= ksc[i];  // <q, c * s> = s <q, c>
        s[g][i] = ok[i] ? a : kNegInf;
      }
    }

    float pr[G][kNumSteps];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mt = s[g][0];
#pragma unroll
      for (int i = 1; i < kNumSteps; ++i) mt = fmaxf(mt, s[g][i]);
#pragma unroll
      for (int o = LPR; o < 64; o <<= 1) mt = fmaxf(mt, __shfl_xor(mt, o));
      const float mn = fmaxf(m[g], mt);
      if (mn == kNegInf) {  // no resident row yet (uniform over the wave)
#pragma unroll
        for (int i = 0; i < kNumSteps; ++i) pr[g][i] = 0.f;
        continue;
      }
      const float alpha = exp2f((m[g] - mn) * c);
      m[g] = mn;
      l[g] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
#pragma unroll
      for (int i = 0; i < kNumSteps; ++i) {
        pr[g][i] = ok[i] ? exp2f((s[g][i] - mn) * c) : 0.f;
        l[g] += pr[g][i];
      }
    }

#pragma unroll
    for (int i = 0; i < kNumSteps; ++i) {
      float vx[EPL];
      Unpack<KIND>::run(vr[i], vx);
#pragma unroll
      for (int e = 0; e < EPL; ++e) vx[e] = ok[i] ? vx[e] : 0.f;
      // int8: the row's V scale joins the weight (selected, so that the
      // scale of an absent row, whatever it holds, never reaches arithmetic)
      const float vs = I8 ? (ok[i] ? vsc[i] : 0.f) : 1.f;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float w = I8 ? pr[g][i] * vs : pr[g][i];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(w, vx[e], acc[g][e]);
      }
    }
  }

  // Sum the RPI row groups (m is already wave-uniform).
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) {
      l[g] += __shfl_xor(l[g], o);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] += __shfl_xor(acc[g][e], o);
    }
  }

  if (rl == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float inv = l[g] > 0.f ? 1.f / l[g] : 0.f;
      float* dst = p.ws_o + ((head0 + g) * p.num_splits + split) * D + cl * EPL;
#pragma unroll
      for (int e = 0; e < EPL; e += 4) {
        const float v[4] = {acc[g][e] * inv, acc[g][e + 1] * inv, acc[g][e + 2] * inv,
                            acc[g][e + 3] * inv};
        if (direct)
          write_out(g, e, v);
        else
          *reinterpret_cast<float4*>(dst + e) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
    if (lane == g) {
      const float lse2 = l[g] > 0.f ? m[g] * c + __log2f(l[g]) : kNegInf;
      if (!direct)
        lse_out[static_cast<size_t>(g) * p.num_splits] = lse2;
      else if (p.lse != nullptr)
        p.lse[head0 + g] = lse2 * kLn2;
    }
}

// Combines the splits of one (sequence, query head):
//   M = max_s lse_s,  w_s = 2^(lse_s - M),  out = sum w_s o_s / sum w_s,
//   lse = (M + log2 sum w_s) * ln 2.
// Splits with lse = -inf hold no row and are skipped (their o is never read).
template <int D>
__global__ __launch_bounds__(64) void merge_kernel(DecodeParams p) {
  constexpr int PER = D / 64;
  const size_t bh = blockIdx.x;
  const int lane = threadIdx.x;
  const int ns = p.num_splits;
  const float* lse2 = p.ws_lse + bh * ns;

  float mx = kNegInf;
  for (int s = lane; s < ns; s += 64) mx = fmaxf(mx, lse2[s]);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));

  float o[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) o[k] = 0.f;
  float wsum = 0.f;
  if (mx != kNegInf) {
    for (int s = 0; s < ns; ++s) {
      const float ls = lse2[s];
      if (ls == kNegInf) continue;
      const float w = exp2f(ls - mx);
      wsum += w;
      const float* po = p.ws_o + (bh * ns + s) * D;
#pragma unroll
      for (int k = 0; k < PER; ++k) o[k] = fmaf(w, po[lane + 64 * k], o[k]);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const float val = o[k] * inv;
    const size_t idx = bh * D + lane + 64 * k;
    if (p.out_bf16)
      static_cast<uint16_t*>(p.out)[idx] = f32_to_bf16_rne(val);
    else
      static_cast<float*>(p.out)[idx] = val;
  }
  if (p.lse != nullptr && lane == 0) p.lse[bh] = wsum > 0.f ? (mx + __log2f(wsum)) * kLn2 : kNegInf;
}

template <int KIND, int D, class Addr>
hipError_t launch_split(const DecodeParams& p, int g, hipStream_t stream) {
  const unsigned grid =
      static_cast<unsigned>(p.batch) * static_cast<unsigned>(p.num_kv_heads) * p.num_splits;
  switch (g) {
#define SWA_CASE(G)                                                             \
  case G:                                                                       \
    decode_split_kernel<KIND, D, G, Addr><<<grid, 64, 0, stream>>>(p);          \
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
  return hipGetLastError();
}

template <class Addr>
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  const int g = p.num_q_heads / p.num_kv_heads;
  hipError_t err;
  if (p.i8)
    err = p.head_dim == 64 ? launch_split<kI8, 64, Addr>(p, g, stream)
                           : launch_split<kI8, 128, Addr>(p, g, stream);
  else if (p.bf16)
    err = p.head_dim == 64 ? launch_split<kBF16, 64, Addr>(p, g, stream)
                           : launch_split<kBF16, 128, Addr>(p, g, stream);
  else
    err = p.head_dim == 64 ? launch_split<kF32, 64, Addr>(p, g, stream)
                           : launch_split<kF32, 128, Addr>(p, g, stream);
  if (err != hipSuccess || p.num_splits == 1) return err;  // one split: written directly
  const unsigned grid = static_cast<unsigned>(p.batch) * static_cast<unsigned>(p.num_q_heads);
  if (p.head_dim == 64)
    merge_kernel<64><<<grid, 64, 0, stream>>>(p);
  else
    merge_kernel<128><<<grid, 64, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

bool group_supported(int g) {
  return g == 1 || g == 2 || g == 3 || g == 4 || g == 6 || g == 8;
}

// bf16 or int8 rows with head_dim 128 take the matrix-core kernel.
bool use_mfma_path(int bf16_or_i8, int32_t head_dim) { return bf16_or_i8 && head_dim == 128; }

SplitPlan plan_splits(int32_t batch, int32_t num_kv_heads, int32_t max_kv_tokens) {
  // One wave per split: aim for about eight waves per CU over the 256 CUs,
  // with splits a multiple of 64 rows and at least 128 rows long.
  const int64_t units = static_cast<int64_t>(batch) * num_kv_heads;
  const int64_t target_waves = 2048;
  const int64_t tokens = max_kv_tokens > 0 ? max_kv_tokens : 1;
  int64_t per = (tokens * units + target_waves - 1) / target_waves;
  per = (per + 63) / 64 * 64;
  if (per < 128) per = 128;
  const int64_t cap = (tokens + 63) / 64 * 64;
  if (per > cap) per = cap;
  SplitPlan plan;
  plan.split_tokens = static_cast<int32_t>(per);
  plan.num_splits = static_cast<int32_t>((tokens + per - 1) / per);
  return plan;
}

SplitPlan plan_splits_mfma(int32_t batch, int32_t num_kv_heads, int32_t max_kv_tokens) {
  // Ring caches on the bf16 / head_dim 128 path: one multi-wave workgroup per
  // split, enough splits per (sequence, kv head) that the grid covers the 256
  // CUs, splits of whole 64-row tiles and at most 8192 rows.
  const int64_t units = static_cast<int64_t>(batch) * num_kv_heads;
  const int64_t tokens = max_kv_tokens > 0 ? max_kv_tokens : 1;
  const int64_t fill = (256 + units - 1) / units;
  const int64_t by_len = (tokens + 8191) / 8192;
  int64_t per_unit = fill > by_len ? fill : by_len;
  if (per_unit > kMaxMfmaSplits) per_unit = kMaxMfmaSplits;
  int64_t per = (tokens + per_unit - 1) / per_unit;
  per = (per + 63) / 64 * 64;
  SplitPlan plan;
  plan.split_tokens = static_cast<int32_t>(per);
  plan.num_splits = static_cast<int32_t>((tokens + per - 1) / per);
  return plan;
}

WorkspaceLayout workspace_layout(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_kv_tokens) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t units = static_cast<size_t>(batch) * num_kv_heads;
  const size_t g = static_cast<size_t>(num_q_heads / num_kv_heads);
  size_t slots = units + kPoolGrid;
  for (const SplitPlan& pl : {plan_splits(batch, num_kv_heads, max_kv_tokens),
                              plan_splits_mfma(batch, num_kv_heads, max_kv_tokens)}) {
    const size_t n = units * static_cast<size_t>(pl.num_splits);
    slots = n > slots ? n : slots;
  }
  WorkspaceLayout w;
  w.shared_base = static_cast<int64_t>(slots);
  // partials of the shared-prefix pass
  slots += static_cast<size_t>(prefix_chunks(batch, num_q_heads, num_kv_heads)) * units;
  w.o_offset = 0;
  w.lse_offset = up(slots * g * head_dim * sizeof(float));
  w.q_offset = w.lse_offset + up(slots * g * sizeof(float));
  w.plan_offset = w.q_offset + up(static_cast<size_t>(batch) * num_q_heads * head_dim * sizeof(float));
  w.total = w.plan_offset + up((static_cast<size_t>(kPlanHead) + batch) * sizeof(int32_t));
  return w;
}

hipError_t launch_decode_ring(const DecodeParams& p, hipStream_t stream) {
  if (use_mfma_path(p.bf16 || p.i8, p.head_dim)) return launch_decode_mfma_ring(p, stream);
  return launch_decode<RingAddr>(p, stream);
}

hipError_t launch_decode_paged(const DecodeParams& p, hipStream_t stream, const PagerFuse* fuse) {
  if (use_mfma_path(p.bf16 || p.i8, p.head_dim)) return launch_decode_mfma_pool(p, stream, fuse);
  hipError_t err = launch_decode<PoolAddr>(p, stream);
  if (err != hipSuccess || fuse == nullptr || fuse->n == 0) return err;
  // this path's merge takes no copies: the paging step's launches follow it
  PagerCopyParams c{};
  c.host_k = fuse->host_k;
  c.host_v = fuse->host_v;
  c.k_pool = fuse->k_pool;
  c.v_pool = fuse->v_pool;
  c.block_u4 = fuse->block_u4;
  c.piece_u4 = std::min(fuse->block_u4, kPagerCopyPieceU4);
  c.pieces = (c.block_u4 + c.piece_u4 - 1) / c.piece_u4;
  c.n = fuse->n;
  PagerValidParams v{};
  v.valid = fuse->valid;
  v.n = fuse->n;
  for (int i = 0; i < fuse->n; ++i) {
    c.src_block[i] = fuse->src_block[i];
    c.dst_block[i] = fuse->dst_block[i];
    v.entries[i] = fuse->slot[i];
  }
  err = launch_pager_copy(c, stream);
  return err != hipSuccess ? err : launch_pager_valid(v, stream);
}

}  // namespace swa
