// Shared host/device definitions of the LoRA library (not part of the public ABI).
//
// Device data layout of one pool (one target module with N output slices):
//   A   [S][N][Rmax][k]     shrink weights as given (rows j >= rank are zero)
//   Bt  [S][Rmax][D]        expand weights, B transposed to rank-major rows; slice n
//                           occupies columns [o_n, o_n + d_n) of every rank row
//   Bk  [S][D][Rmax]        expand weights with the rank contiguous (B as given,
//                           padded): the matrix-core operand layout
//   table [S]               rank, scale, present-slice mask per slot
// Slots are addressed by fixed strides, so no pointer table is needed: the
// address of slot s is base + s * stride, formed in 64-bit arithmetic.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "raxlora.h"

namespace rax {

constexpr int kMaxSlices = LORA_MAX_SLICES;
constexpr int kMaxSplit = 32;      // k-splits of the shrink (partials in the workspace)
constexpr int kDefaultSplit = 8;   // splits used when k allows
constexpr int kMaxChunksPerSplit = 4;  // 16-byte lane chunks per split (x held in registers)
constexpr int kColsPerLane = 8;    // expand: output columns owned by one lane
constexpr int kTileCols = 64 * kColsPerLane;  // expand: columns of one wave tile
constexpr int kRoutingThreads = 512;
constexpr int kRoutingWaves = kRoutingThreads / 64;
constexpr int kMfmaTileM = 64;     // tokens per matrix-core tile of a long segment
constexpr int kDefaultMfmaMinSeg = 32;  // segments at least this long use matrix cores
constexpr bool kHaveMfmaPath = false;   // matrix-core kernels compiled in

struct SlotEntry {
  int32_t rank;         // 0 = empty slot
  float scale;          // applied after the branch (1 when folded into B)
  uint32_t slice_mask;  // bit n set: slice n present
  int32_t pad;
};

// routing meta words
enum MetaIndex { kMetaT = 0, kMetaActive = 1, kMetaInvalid = 2, kMetaLora = 3, kMetaTiles = 4,
                 kMetaWords = 8 };

struct PoolView {
  const void* A;
  const void* Bt;
  const void* Bk;
  const SlotEntry* table;
  int S, Rmax, k, N, D, n_ctiles;
  int d[kMaxSlices];
  int o[kMaxSlices];
  int tile0[kMaxSlices + 1];  // first expand column tile of each slice; tile0[N] = n_ctiles
};

struct RouteView {
  const int* counts;   // [S+1]
  const int* offs;     // [S+2]
  const int* sorted;   // [T]
  const int* active;   // [S]
  const int* tiles;    // [max_tiles][3]: slot, first sorted position, length
  const int* meta;     // [kMetaWords]
  int S, T, mfma_min, tile_m, max_tiles;
};

// Rank-space intermediate u: element (split q, slice n, row, j) at
// p + q*q_stride + n*n_stride + row*row_stride + j, where row is the token index
// (by_token) or the token's position in sorted order.
struct UView {
  float* p;
  long long q_stride, n_stride, row_stride;
  int nsplit;
  int by_token;
};

// Optional per-launch timing: when start is non-null the kernel is launched with
// hipExtLaunchKernel, which stamps the two events at the kernel's own start and end.
struct KTimer {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// kernels the timing facility reports, in this order
enum KernelId { kKRouting = 0, kKShrink, kKExpand, kKReduce, kKShrinkMfma, kKExpandMfma, kKernelCount };

// launchers (device code in the .hip files); all return the launch status
hipError_t launch_routing(const int32_t* ids, int T, int S, int mfma_min, int tile_m, int max_tiles,
                          int* counts, int* offs, int* sorted, int* active, int* tiles, int* meta,
                          hipStream_t stream, const KTimer& tm);
hipError_t launch_pack_slice(int wdtype, const void* A_src, const void* B_src, void* A_dst,
                             void* Bt_dst, void* Bk_dst, int rank, int Rmax, int k, int d, int D,
                             float scale, int premultiply, hipStream_t stream);
hipError_t launch_set_slot(SlotEntry* table, int slot, SlotEntry entry, hipStream_t stream);
hipError_t launch_shrink(int wdtype, const PoolView& P, const RouteView& R, const void* x, int ldx,
                         const UView& U, int kc, int use_mfma, hipStream_t stream, const KTimer& tm);
hipError_t launch_expand(int wdtype, int ydtype, const PoolView& P, const RouteView& R,
                         const UView& U, void* y, int ldy, int use_mfma, hipStream_t stream,
                         const KTimer& tm);
hipError_t launch_reduce_splits(const PoolView& P, const RouteView& R, const UView& W, const UView& U,
                                hipStream_t stream, const KTimer& tm);
hipError_t launch_shrink_mfma(const PoolView& P, const RouteView& R, const void* x, int ldx,
                              const UView& U, int kc, hipStream_t stream, const KTimer& tm);
hipError_t launch_expand_mfma(int ydtype, const PoolView& P, const RouteView& R, const UView& U,
                              void* y, int ldy, hipStream_t stream, const KTimer& tm);

}  // namespace rax
