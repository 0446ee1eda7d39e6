// Host-only build of the block manager (blocks_api.cpp) and the host-pool
// pager (pager_api.cpp) for AddressSanitizer / UndefinedBehaviorSanitizer
// runs: the HIP runtime calls and kernel launches those two files make are
// defined here on the host, with "device" buffers in host memory and each
// launch doing its kernel's effect (table / length updates, copy-on-write
// row copies, the new rows, validity flips, block copies) at once.  A small
// command interpreter on stdin drives the C ABI and prints the state, which
// tests/test_host_sanitized.py compares with oracle/blocks.py and
// oracle/paging.py.  Test infrastructure: not part of the library.
//
// Commands (one per line):
//   blocks NB BS SEQS MAXB HKV D   new manager; "device" mirrors and f32 pools
//   share SRC DST N                swa_blocks_share_prefix
//   append T N S1 .. SN            kv_append_paged of T tokens to N sequences;
//                                  row (s, p) of head h holds s*100000 + p in
//                                  element 0 and h in element 1
//   free S                         swa_blocks_free
//   bstate                         host state; device table/lengths; every
//                                  sequence read back through the device table
//   pager B HKV D BS L C NPHYS     new pager, slot_phys a fixed permutation,
//                                  host store element 0 of block (b, k), head h,
//                                  row r = b*1000000 + k*1000 + h*100 + r
//   advance SPLIT n0 k.. n1 k..    swa_pager_advance; SPLIT 1: copies on a
//                                  second stream
//   commit                         swa_pager_commit
//   pstate                         slot blocks, device validity, and the count
//                                  of valid slots whose pool block differs
//                                  from the host store's block
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <iostream>
#include <memory>
#include <sstream>
#include <string>
#include <vector>

#include "swa.h"
#include "swa_internal.h"

// ---------------------------------------------------------------------------
// the HIP runtime on the host
// ---------------------------------------------------------------------------

namespace {
int g_live_events = 0;
}

extern "C" {

const char* hipGetErrorString(hipError_t) { return "host stub"; }
hipError_t hipGetLastError(void) { return hipSuccess; }

hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
  std::memcpy(dst, src, n);
  return hipSuccess;
}

hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

hipError_t hipHostGetDevicePointer(void** dev, void* host, unsigned int) {
  *dev = host;  // one address space here
  return hipSuccess;
}

hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) {
  *e = reinterpret_cast<hipEvent_t>(new int(0));
  ++g_live_events;
  return hipSuccess;
}

hipError_t hipEventDestroy(hipEvent_t e) {
  delete reinterpret_cast<int*>(e);
  --g_live_events;
  return hipSuccess;
}

hipError_t hipEventRecord(hipEvent_t e, hipStream_t) {
  *reinterpret_cast<int*>(e) += 1;  // touches the event: a freed one would show
  return hipSuccess;
}

hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t e, unsigned) {
  (void)*reinterpret_cast<volatile int*>(e);
  return hipSuccess;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// the launches, done on the host
// ---------------------------------------------------------------------------

// The decode's workspace size: any value serves the pager's arithmetic here
// (not a multiple of 256, so the staging area's alignment step is taken).
extern "C" swa_status decode_attn_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                                  int32_t num_kv_heads, int32_t head_dim,
                                                  int32_t max_kv_tokens, size_t* bytes) {
  if (batch < 1 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1 || max_kv_tokens < 0)
    return SWA_ERR_INVALID_ARG;
  *bytes = 1000 + static_cast<size_t>(batch) * num_q_heads * (head_dim + 1) * 4;
  return SWA_OK;
}

namespace swa {

namespace {
thread_local std::string g_error;
}
int record_error(int code, const char* text) {
  g_error = text;
  return code;
}
void clear_error() { g_error.clear(); }

hipError_t launch_blocks_update(const BlocksUpdateParams& p, hipStream_t) {
  for (int i = 0; i < p.n_table; ++i) p.block_table[p.table_idx[i]] = p.table_val[i];
  for (int i = 0; i < p.n_lens; ++i) p.seq_lens[p.lens_idx[i]] = p.lens_val[i];
  const size_t row = static_cast<size_t>(p.head_dim) * p.elem_bytes;
  const size_t head = row * p.block_size;
  for (int i = 0; i < p.n_cow; ++i)
    for (void* pool : {p.k_pool, p.v_pool})
      for (int h = 0; h < p.num_kv_heads; ++h) {
        char* base = static_cast<char*>(pool);
        char* dst = base + (static_cast<size_t>(p.cow_dst[i]) * p.num_kv_heads + h) * head;
        const char* src = base + (static_cast<size_t>(p.cow_src[i]) * p.num_kv_heads + h) * head;
        std::memcpy(dst, src, row * p.cow_rows[i]);
      }
  return hipSuccess;
}

hipError_t launch_append_paged(const AppendPagedParams& p, hipStream_t) {
  if (p.bf16 || p.rotate) return hipErrorInvalidValue;  // the harness writes f32, unrotated
  const int bs = 1 << p.block_shift;
  const size_t d = static_cast<size_t>(p.head_dim);
  for (int i = 0; i < p.n_seqs; ++i)
    for (int t = 0; t < p.n_tokens; ++t) {
      const int pos = p.first_pos[i] + t;
      const int blk = p.block_table[static_cast<size_t>(p.seqs[i]) * p.max_blocks + (pos >> p.block_shift)];
      if (blk < 0 || blk >= p.num_phys_blocks) return hipErrorInvalidValue;
      for (int h = 0; h < p.num_kv_heads; ++h) {
        const size_t src = ((static_cast<size_t>(p.src_first + i) * p.n_tokens + t) * p.num_kv_heads + h) * d;
        const size_t dst = ((static_cast<size_t>(blk) * p.num_kv_heads + h) * bs + (pos & (bs - 1))) * d;
        std::memcpy(static_cast<float*>(p.k_pool) + dst, static_cast<const float*>(p.k_src) + src, d * 4);
        std::memcpy(static_cast<float*>(p.v_pool) + dst, static_cast<const float*>(p.v_src) + src, d * 4);
      }
    }
  return hipSuccess;
}

hipError_t launch_pager_valid(const PagerValidParams& p, hipStream_t) {
  for (int i = 0; i < p.n; ++i) {
    const int e = p.entries[i];
    if (e >= 0) p.valid[e] = 1;
    else p.valid[-1 - e] = 0;
  }
  return hipSuccess;
}

hipError_t launch_pager_copy(const PagerCopyParams& p, hipStream_t) {
  const size_t bytes = static_cast<size_t>(p.block_u4) * 16;
  for (int i = 0; i < p.n; ++i) {
    std::memcpy(static_cast<char*>(p.k_pool) + p.dst_block[i] * bytes,
                static_cast<const char*>(p.host_k) + p.src_block[i] * bytes, bytes);
    std::memcpy(static_cast<char*>(p.v_pool) + p.dst_block[i] * bytes,
                static_cast<const char*>(p.host_v) + p.src_block[i] * bytes, bytes);
  }
  return hipSuccess;
}

hipError_t launch_fill_u8(uint8_t* dst, size_t n, uint8_t value, hipStream_t) {
  std::memset(dst, value, n);
  return hipSuccess;
}

// The pager's decode: the attention is not modelled here; the copies of a
// fused paging step and their validity bytes are (swa_api.cpp is not built).
swa_status paged_decode_with_copies(const swa_paged_desc* desc, const void* q, const void*,
                                    const void*, const int32_t* block_table,
                                    const int32_t* seq_lens, const uint8_t*, float, void* out,
                                    swa_dtype, float*, void* workspace, size_t, void*,
                                    const PagerFuse* fuse) {
  if (desc == nullptr || q == nullptr || block_table == nullptr || seq_lens == nullptr ||
      out == nullptr || workspace == nullptr)
    return SWA_ERR_INVALID_ARG;
  if (fuse == nullptr) return SWA_OK;
  // the two parts as the kernels run them: host store to staging area (during
  // the attention), then staging area to pool (in the merge launch)
  const size_t bytes = static_cast<size_t>(fuse->block_u4) * 16;
  for (int i = 0; i < fuse->n; ++i) {
    std::memcpy(static_cast<char*>(fuse->stage_k) + i * bytes,
                static_cast<const char*>(fuse->host_k) + fuse->src_block[i] * bytes, bytes);
    std::memcpy(static_cast<char*>(fuse->stage_v) + i * bytes,
                static_cast<const char*>(fuse->host_v) + fuse->src_block[i] * bytes, bytes);
  }
  for (int i = 0; i < fuse->n; ++i) {
    std::memcpy(static_cast<char*>(fuse->k_pool) + fuse->dst_block[i] * bytes,
                static_cast<const char*>(fuse->stage_k) + i * bytes, bytes);
    std::memcpy(static_cast<char*>(fuse->v_pool) + fuse->dst_block[i] * bytes,
                static_cast<const char*>(fuse->stage_v) + i * bytes, bytes);
    fuse->valid[fuse->slot[i]] = 1;
  }
  return SWA_OK;
}

}  // namespace swa

// ---------------------------------------------------------------------------
// the command-line front end of this test program
// ---------------------------------------------------------------------------

namespace {

hipStream_t fake_stream(int i) { return reinterpret_cast<hipStream_t>(static_cast<uintptr_t>(0x1000 + 16 * i)); }

struct Blocks {
  swa_blocks* m = nullptr;
  swa_paged_desc desc{};
  std::vector<int32_t> table, lens;
  std::vector<float> k, v;
  ~Blocks() { swa_blocks_destroy(m); }
};

struct Pager {
  swa_pager* pg = nullptr;
  swa_pager_config cfg{};
  std::vector<float> hk, hv, kp, vp;
  std::vector<int32_t> slot_phys, table;
  std::vector<uint8_t> valid;
  ~Pager() { swa_pager_destroy(pg); }
};

void print_vec(const char* name, const int32_t* x, size_t n) {
  std::printf("%s", name);
  for (size_t i = 0; i < n; ++i) std::printf(" %d", x[i]);
  std::printf("\n");
}

int run() {
  std::unique_ptr<Blocks> bl;
  std::unique_ptr<Pager> pa;
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string cmd;
    if (!(in >> cmd)) continue;
    if (cmd == "blocks") {
      int nb, bs, seqs, maxb, hkv, d;
      in >> nb >> bs >> seqs >> maxb >> hkv >> d;
      bl.reset(new Blocks);
      int rc = swa_blocks_create(nb, bs, seqs, maxb, &bl->m);
      bl->desc = swa_paged_desc{seqs, hkv, hkv, d, bs, maxb, nb, SWA_F32};
      bl->table.assign(static_cast<size_t>(seqs) * maxb, -7);
      bl->lens.assign(seqs, -7);
      bl->k.assign(static_cast<size_t>(nb) * hkv * bs * d, -1.f);
      bl->v.assign(bl->k.size(), -1.f);
      if (rc == SWA_OK) rc = swa_blocks_sync(bl->m, bl->table.data(), bl->lens.data(), nullptr);
      std::printf("rc %d\n", rc);
    } else if (cmd == "share") {
      int src, dst, n;
      in >> src >> dst >> n;
      std::printf("rc %d\n", swa_blocks_share_prefix(bl->m, src, dst, n, bl->table.data(),
                                                     bl->lens.data(), fake_stream(0)));
    } else if (cmd == "append") {
      int t, n;
      in >> t >> n;
      std::vector<int32_t> seqs(n);
      for (int& s : seqs) in >> s;
      const int hkv = bl->desc.num_kv_heads, d = bl->desc.head_dim;
      std::vector<int32_t> lens(bl->desc.batch);
      swa_blocks_state(bl->m, nullptr, lens.data(), nullptr, nullptr);
      std::vector<float> rows(static_cast<size_t>(n) * t * hkv * d, 0.f);
      for (int i = 0; i < n; ++i)
        for (int j = 0; j < t; ++j)
          for (int h = 0; h < hkv; ++h) {
            // out-of-range sequences are refused by the call; no row to tag
            const int s = seqs[i];
            const int pos = (s >= 0 && s < bl->desc.batch ? lens[s] : 0) + j;
            float* r = rows.data() + ((static_cast<size_t>(i) * t + j) * hkv + h) * d;
            r[0] = static_cast<float>(s * 100000 + pos);
            r[1] = static_cast<float>(h);
          }
      std::printf("rc %d\n", kv_append_paged(bl->m, &bl->desc, bl->k.data(), bl->v.data(),
                                              bl->table.data(), bl->lens.data(), seqs.data(), n, t,
                                              rows.data(), rows.data(), 0, 10000.f,
                                              SWA_ROPE_INTERLEAVED, fake_stream(0)));
    } else if (cmd == "free") {
      int s;
      in >> s;
      std::printf("rc %d\n", swa_blocks_free(bl->m, s, bl->lens.data(), fake_stream(0)));
    } else if (cmd == "reset") {
      std::printf("rc %d\n", swa_blocks_reset(bl->m));
    } else if (cmd == "bsync") {
      std::printf("rc %d\n", swa_blocks_sync(bl->m, bl->table.data(), bl->lens.data(), nullptr));
    } else if (cmd == "bstate") {
      const swa_paged_desc& d = bl->desc;
      std::vector<int32_t> table(bl->table.size()), lens(d.batch), refs(d.num_phys_blocks);
      int32_t free_blocks = -1;
      swa_blocks_state(bl->m, table.data(), lens.data(), refs.data(), &free_blocks);
      print_vec("table", table.data(), table.size());
      print_vec("lens", lens.data(), lens.size());
      print_vec("refs", refs.data(), refs.size());
      std::printf("free %d\n", free_blocks);
      print_vec("dlens", bl->lens.data(), bl->lens.size());
      // every sequence read back through the device table: tag, and a flag
      // for a head / K-V mismatch
      const int bs = d.block_size;
      for (int s = 0; s < d.batch; ++s) {
        std::printf("read %d", s);
        for (int i = 0; i < bl->lens[s]; ++i) {
          const int blk = bl->table[static_cast<size_t>(s) * d.max_blocks_per_seq + i / bs];
          if (blk < 0 || blk >= d.num_phys_blocks) {
            std::printf(" x");
            continue;
          }
          float tag = 0.f;
          bool ok = true;
          for (int h = 0; h < d.num_kv_heads; ++h) {
            const size_t at = ((static_cast<size_t>(blk) * d.num_kv_heads + h) * bs + i % bs) * d.head_dim;
            ok = ok && bl->k[at] == bl->v[at] && bl->k[at + 1] == static_cast<float>(h);
            if (h == 0) tag = bl->k[at];
            ok = ok && bl->k[at] == tag;
          }
          if (ok) std::printf(" %.0f", tag);
          else std::printf(" x");
        }
        std::printf("\n");
      }
    } else if (cmd == "pager") {
      swa_pager_config c{};
      in >> c.batch >> c.num_kv_heads >> c.head_dim >> c.block_size >> c.logical_blocks >>
          c.slots_per_seq >> c.num_phys_blocks;
      c.dtype = SWA_F32;
      pa.reset(new Pager);
      pa->cfg = c;
      const size_t blk = static_cast<size_t>(c.num_kv_heads) * c.block_size * c.head_dim;
      pa->hk.assign(blk * c.batch * c.logical_blocks, 0.f);
      for (int b = 0; b < c.batch; ++b)
        for (int k = 0; k < c.logical_blocks; ++k)
          for (int h = 0; h < c.num_kv_heads; ++h)
            for (int r = 0; r < c.block_size; ++r)
              pa->hk[((static_cast<size_t>(b) * c.logical_blocks + k) * c.num_kv_heads * c.block_size +
                      static_cast<size_t>(h) * c.block_size + r) * c.head_dim] =
                  static_cast<float>(b * 1000000 + k * 1000 + h * 100 + r);
      pa->hv = pa->hk;
      for (float& x : pa->hv) x = -x;
      pa->kp.assign(blk * c.num_phys_blocks, 0.5f);
      pa->vp.assign(blk * c.num_phys_blocks, 0.5f);
      const int slots = c.batch * c.slots_per_seq;
      pa->slot_phys.resize(slots);
      for (int i = 0; i < slots; ++i) pa->slot_phys[i] = (i * 7 + 3) % slots;  // a permutation for slots % 7 != 0
      pa->table.assign(slots, -7);
      pa->valid.assign(slots, 9);
      int rc = swa_pager_create(&c, pa->hk.data(), pa->hv.data(), pa->kp.data(), pa->vp.data(),
                                pa->slot_phys.data(), pa->table.data(), pa->valid.data(), &pa->pg);
      if (rc == SWA_OK) rc = swa_pager_reset(pa->pg, fake_stream(0));
      std::printf("rc %d\n", rc);
    } else if (cmd == "advance") {
      int split;
      in >> split;
      std::vector<int32_t> off{0}, blocks;
      for (int b = 0; b < pa->cfg.batch; ++b) {
        int n;
        in >> n;
        for (int i = 0; i < n; ++i) {
          int k;
          in >> k;
          blocks.push_back(k);
        }
        off.push_back(static_cast<int32_t>(blocks.size()));
      }
      int32_t loaded = -1;
      const int rc = swa_pager_advance(pa->pg, off.data(), blocks.empty() ? nullptr : blocks.data(),
                                       fake_stream(0), fake_stream(split ? 1 : 0), &loaded);
      std::printf("rc %d loaded %d\n", rc, loaded);
    } else if (cmd == "commit") {
      std::printf("rc %d\n", swa_pager_commit(pa->pg, fake_stream(0)));
    } else if (cmd == "stage") {
      std::vector<int32_t> off{0}, blocks;
      for (int b = 0; b < pa->cfg.batch; ++b) {
        int n;
        in >> n;
        for (int i = 0; i < n; ++i) {
          int k;
          in >> k;
          blocks.push_back(k);
        }
        off.push_back(static_cast<int32_t>(blocks.size()));
      }
      int32_t loaded = -1;
      const int rc = swa_pager_stage(pa->pg, off.data(), blocks.empty() ? nullptr : blocks.data(),
                                     &loaded);
      std::printf("rc %d loaded %d\n", rc, loaded);
    } else if (cmd == "pdecode") {
      float q = 0.f, o = 0.f;
      std::vector<int32_t> lens(pa->cfg.batch, pa->cfg.slots_per_seq * pa->cfg.block_size);
      size_t n = 0;
      if (swa_pager_workspace_bytes(pa->pg, pa->cfg.num_kv_heads, &n) != SWA_OK) {
        std::printf("rc -1\n");
        continue;
      }
      std::vector<char> ws(n);  // exactly the size asked for: an overrun is reported
      std::printf("rc %d\n", swa_pager_decode(pa->pg, &q, pa->cfg.num_kv_heads, lens.data(), 0.f,
                                               &o, SWA_F32, nullptr, ws.data(), ws.size(),
                                               fake_stream(0)));
    } else if (cmd == "pstate") {
      const swa_pager_config& c = pa->cfg;
      std::vector<int32_t> sb(c.slots_per_seq);
      const size_t blk = static_cast<size_t>(c.num_kv_heads) * c.block_size * c.head_dim;
      int bad = 0;
      for (int b = 0; b < c.batch; ++b) {
        swa_pager_slot_blocks(pa->pg, b, sb.data());
        print_vec("slots", sb.data(), sb.size());
        std::vector<int32_t> v(c.slots_per_seq);
        for (int j = 0; j < c.slots_per_seq; ++j) {
          const int g = b * c.slots_per_seq + j;
          v[j] = pa->valid[g];
          if (pa->table[g] != pa->slot_phys[g]) ++bad;
          if (v[j] == 1) {
            const size_t src = (static_cast<size_t>(b) * c.logical_blocks + sb[j]) * blk;
            const size_t dst = static_cast<size_t>(pa->slot_phys[g]) * blk;
            if (sb[j] < 0 || std::memcmp(&pa->kp[dst], &pa->hk[src], blk * 4) != 0 ||
                std::memcmp(&pa->vp[dst], &pa->hv[src], blk * 4) != 0)
              ++bad;
          }
        }
        print_vec("valid", v.data(), v.size());
      }
      std::printf("bad %d\n", bad);
    } else {
      std::fprintf(stderr, "unknown command %s\n", cmd.c_str());
      return 2;
    }
    std::fflush(stdout);
  }
  bl.reset();
  pa.reset();
  std::printf("events %d\n", g_live_events);  // every event created was destroyed
  return 0;
}

}  // namespace

int main() { return run(); }
