// Walking the segment table of the sorted layout from a row block's first segment (internal to
// libmoelora). Segments are sorted by their first row; the segments that overlap a range of
// rows inside one row block start at or after the block's first segment.
#pragma once

#include "common.h"

namespace moelora {

// Most adapter runs a 64-row sub-block may hold for the 64-row shrink to take it; sub-blocks
// with more (many short runs, e.g. one token per adapter) go to the 16-row shrink.
constexpr int kShrink64MaxRuns = 4;

// Adapter runs (segments with an adapter) overlapping rows [row0, row0 + 64) of row block blk,
// counted up to limit + 1. Wavefront-uniform; every lane of the wavefront must call it.
__device__ __forceinline__ int count_runs64(const int* block_seg, const int* seg_table,
                                            int nseg, int nA, int blk, int row0, int limit) {
  const int first = block_seg[blk];
  if (first < 0) return 0;
  const int lane = threadIdx.x & 63;
  int n = 0;
  for (int c0 = first;; c0 += 64) {
    const int sj = c0 + lane;
    bool before_end = false, run = false;
    if (sj < nseg) {
      const u32x4 sg = *reinterpret_cast<const u32x4*>(seg_table + 4 * (size_t)sj);
      const int st = (int)sg[2], cnt = (int)sg[3];
      before_end = st < row0 + 64;
      run = before_end && st + cnt > row0 && sanitize_adapter((int)sg[1], nA) >= 0;
    }
    n += (int)__popcll(__ballot(run));
    if (n > limit || !(__ballot(before_end) >> 63)) break;
  }
  return n;
}

}  // namespace moelora
