// Work placement shared by the shrink and expand launches (device code): the
// matrix-core items of a launch split over the XCDs, and the module of a workgroup
// in a grouped launch.
#pragma once

#include "device_util.h"

namespace rax {

// Matrix-core work items of one launch, split over the XCDs: workgroup b runs on XCD
// b % 8, and XCD x takes the x-th contiguous eighth of the items (tiles in slot
// order within).  Consecutive tiles of a segment share their slot's weights, and the
// items of one tile share its tokens' data, so each XCD's L2 serves its own stretch
// of the batch and weights and partial sums are fetched from HBM about once.
// Worker i of an XCD takes items start + i, start + i + upx, ... (upx workers per
// XCD; the launch provides at least one worker per item).
struct MfmaItems {
  int j, end, step;
  __device__ __forceinline__ MfmaItems(int b, int n_blocks, int n_items) {
    const int x = b % kXcds, upx = n_blocks / kXcds;
    const int per = (n_items + kXcds - 1) / kXcds;
    j = min(n_items, x * per) + b / kXcds;
    end = min(n_items, (x + 1) * per);
    step = upx;
  }
};

// Workgroups of a launch: first the matrix-core workers (a multiple of 8, so the XCD
// of a worker is its index mod 8), then the decode units.
__host__ __device__ inline int mfma_blocks(int items_max) { return (items_max + kXcds - 1) / kXcds * kXcds; }

// The module of workgroup b of a grouped launch (modules in launch order, blk0 ascending)
__device__ __forceinline__ int group_module(const GroupView& G, int b) {
  int m = 0;
  while (m + 1 < G.n && b >= G.e[m + 1].blk0) ++m;
  return m;
}

}  // namespace rax
