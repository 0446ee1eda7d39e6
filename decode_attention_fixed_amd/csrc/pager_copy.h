// Copies of whole K and V blocks by workgroups, for the pager's copy kernel
// and for the paging step folded into the paged decode's launches.
#pragma once

#include "device_common.h"

namespace swa {

constexpr int kCopyUnroll = 4;  // independent 16-byte loads in flight per thread

// Units [begin, end) of a block (16-byte units) from src to dst, by the whole
// workgroup of `threads` threads.
__device__ __forceinline__ void copy_block_piece(const uint4* src, uint4* dst, int begin, int end,
                                                 int threads) {
  for (int i = begin + static_cast<int>(threadIdx.x); i < end; i += threads * kCopyUnroll) {
    uint4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int j = i + u * threads;
      if (j < end) v[u] = src[j];
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int j = i + u * threads;
      if (j < end) dst[j] = v[u];
    }
  }
}

// Workgroups of `threads` threads that copy one block of K (or V) of
// block_u4 units, one pass of kCopyUnroll loads per thread each.
__host__ __device__ __forceinline__ int copy_pieces(int block_u4, int threads) {
  const int piece = kCopyUnroll * threads;
  return (block_u4 + piece - 1) / piece;
}

// What workgroup w of a copy of n items (a K block and a V block each) moves:
// item w / (2 pieces), tensor (w / pieces) % 2 (0 = K), units [begin, end).
struct CopyPiece {
  int item, tensor, begin, end;
};
__device__ __forceinline__ CopyPiece copy_piece(int w, int block_u4, int threads) {
  const int pieces = copy_pieces(block_u4, threads);
  const int r = w % (2 * pieces);
  CopyPiece c;
  c.item = w / (2 * pieces);
  c.tensor = r / pieces;
  c.begin = (r % pieces) * kCopyUnroll * threads;
  c.end = min(c.begin + kCopyUnroll * threads, block_u4);
  return c;
}

}  // namespace swa
