// Copies of whole K and V blocks by workgroups, for the pager's copy kernel
// and for the paging step folded into the paged decode's launches.
#pragma once

#include "device_common.h"

namespace swa {

constexpr int kCopyUnroll = 4;  // independent 16-byte loads in flight per thread

// Units [begin, end) of a block (16-byte units) from src to dst, by the whole
// workgroup of `threads` threads.  Four named registers, not an array (an
// array indexed in a loop is placed in memory before the loop is unrolled),
// and the four loads are issued unconditionally, the addresses past the end
// clamped to the last unit, so none waits on its own; only the stores are
// conditional.
__device__ __forceinline__ void copy_block_piece(const uint4* src, uint4* dst, int begin, int end,
                                                 int threads) {
  static_assert(kCopyUnroll == 4, "four loads per thread and pass");
  for (int i = begin + static_cast<int>(threadIdx.x); i < end; i += threads * kCopyUnroll) {
    const int j1 = i + threads, j2 = i + 2 * threads, j3 = i + 3 * threads;
    const uint4 a0 = src[i];
    const uint4 a1 = src[min(j1, end - 1)];
    const uint4 a2 = src[min(j2, end - 1)];
    const uint4 a3 = src[min(j3, end - 1)];
    dst[i] = a0;
    if (j1 < end) dst[j1] = a1;
    if (j2 < end) dst[j2] = a2;
    if (j3 < end) dst[j3] = a3;
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
