// Kernels of the host-pool pager ([pool] "paging": 64-token blocks move
// between host memory and a fixed pool of device slots; each slot carries a
// validity bit that the attention kernel reads).
//
//   pager_copy_kernel   whole blocks of K and V from pinned host memory into
//                       pool blocks.  A kernel, not the copy engine: on this
//                       GPU one engine copy of a 64 KiB block costs ~10 us
//                       (about 6 GB/s), while one launch of a few dozen
//                       workgroups reading host memory over the bus moves
//                       a list of blocks at ~55 GB/s.
//   pager_valid_kernel  sets or clears a list of validity bytes.
//   fill_u8_kernel      fills a byte array (reset).
#include "device_common.h"
#include "pager_copy.h"
#include "swa_internal.h"

namespace swa {

namespace {

constexpr int kCopyThreads = 256;

// Workgroup w copies piece (w % pieces) of tensor ((w / pieces) % 2) of item
// w / (2 * pieces).  Every index is checked against the item count and the
// block size, so a grid larger than the list is harmless.
__global__ __launch_bounds__(kCopyThreads) void pager_copy_kernel(PagerCopyParams p) {
  const int per_item = 2 * p.pieces;
  const int item = static_cast<int>(blockIdx.x) / per_item;
  if (item >= p.n) return;
  const int r = static_cast<int>(blockIdx.x) % per_item;
  const int tensor = r / p.pieces;
  const int piece = r % p.pieces;
  const uint4* src = static_cast<const uint4*>(tensor == 0 ? p.host_k : p.host_v) +
                     static_cast<size_t>(p.src_block[item]) * p.block_u4;
  uint4* dst = static_cast<uint4*>(tensor == 0 ? p.k_pool : p.v_pool) +
               static_cast<size_t>(p.dst_block[item]) * p.block_u4;
  const int begin = piece * p.piece_u4;
  copy_block_piece(src, dst, begin, min(begin + p.piece_u4, p.block_u4), kCopyThreads);
}

__global__ void pager_valid_kernel(PagerValidParams p) {
  const int i = static_cast<int>(blockIdx.x * blockDim.x + threadIdx.x);
  if (i >= p.n) return;
  const int32_t e = p.entries[i];
  if (e >= 0)
    p.valid[e] = 1;
  else
    p.valid[-1 - e] = 0;
}

__global__ void fill_u8_kernel(uint8_t* dst, size_t n, uint8_t value) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    dst[i] = value;
}

}  // namespace

hipError_t launch_pager_copy(const PagerCopyParams& p, hipStream_t stream) {
  if (p.n <= 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>(p.n) * 2u * static_cast<unsigned>(p.pieces);
  pager_copy_kernel<<<grid, kCopyThreads, 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_pager_valid(const PagerValidParams& p, hipStream_t stream) {
  if (p.n <= 0) return hipSuccess;
  pager_valid_kernel<<<(p.n + 255) / 256, 256, 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_fill_u8(uint8_t* dst, size_t n, uint8_t value, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  const unsigned grid = static_cast<unsigned>(blocks < 4096 ? blocks : 4096);
  fill_u8_kernel<<<grid, 256, 0, stream>>>(dst, n, value);
  return hipGetLastError();
}

}  // namespace swa
