// Shared host/device definitions of the LoRA library (not part of the public ABI).
//
// Device data layout of one pool (one target module with N output slices):
//   A   [S][N][Rmax][k]     shrink weights as given (rows j >= rank are zero)
//   Bt  [S][Rmax][D]        expand weights, B transposed to rank-major rows; slice n
//                           occupies columns [o_n, o_n + d_n) of every rank row
//   Bk  [S][D * Rk]         expand weights with the rank contiguous (B as given),
//                           the matrix-core operand layout: slot s's region of
//                           D * Rk elements (Rk = Rmax rounded up to 32) holds
//                           column c at offset c * bk_stride(rank), the slot's rank
//                           rounded up to 8 (entries past the rank zero)
//   table [S]               rank, scale, present-slice mask per slot
// Slots are addressed by fixed strides, so no pointer table is needed: the
// address of slot s is base + s * stride, formed in 64-bit arithmetic.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "raxlora.h"

namespace rax {

constexpr int kMaxSlices = LORA_MAX_SLICES;
constexpr int kMaxOrderedSlots = 256;   // pools up to this size dispatch decode expand units by rank
constexpr int kMaxSplit = 16;         // k splits of a decode shrink (partial sums per split)
constexpr int kColsPerLane = 8;    // expand: output columns owned by one lane
constexpr int kTileCols = 64 * kColsPerLane;  // expand: columns of one wave tile
constexpr int kRoutingMaxThreads = 1024;   // routing workgroup: 16 waves (8 for large slot counts)
constexpr int kRoutingStageBatch = 16;   // ids each routing thread loads in one batch
constexpr int kMfmaTileM = 16;     // tokens per matrix-core tile of a long segment
constexpr int kMfmaK = 32;         // k of one bf16 matrix-core step (16x16x32)
constexpr int kMfmaCols = 128;     // output columns of one matrix-core expand block
// elements per column of a slot's Bk region: its rank rounded up to 8
__host__ __device__ constexpr int bk_stride(int rank) { return (rank + 7) / 8 * 8; }
constexpr int kMfmaColBlocksPerUnit = 4;   // most 128-column blocks of one matrix-core expand unit
constexpr int kDefaultMfmaMinSeg = 4;   // segments at least this long use matrix cores (bf16 pools)
constexpr int kRecInts = 32;       // ints of one slot record: tokens, first position, 2 spare, token ids
constexpr int kRecTokens = kRecInts - 4;   // token ids a slot record holds
constexpr bool kHaveMfmaPath = true;    // matrix-core kernels compiled in
constexpr int kSelfRouteTokens = 256;   // most tokens of a batch whose shrink launch builds its routing
constexpr int kSelfRouteKeys = 256;     // most keys (slots + 1) of such a batch
constexpr size_t kNoAllocScratchBytes = LORA_NOALLOC_SCRATCH_BYTES;   // the allocation-free call's scratch

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
  int S, Rmax, Rk, k, N, D, n_ctiles, n_mblocks;
  int d[kMaxSlices];
  int o[kMaxSlices];
  int tile0[kMaxSlices + 1];  // first expand column tile of each slice; tile0[N] = n_ctiles
  int mblk0[kMaxSlices + 1];  // first matrix-core column block of each slice; mblk0[N] = n_mblocks
};

// Dispatch order of a pool's slots for the decode expand units (a single-module
// launch): slots by descending rank when `ordered`, else by index.
struct SlotOrder {
  int ordered;                // 1: s below is valid (S <= kMaxOrderedSlots)
  uint8_t s[kMaxOrderedSlots];
};

struct RouteView {
  const int* counts;   // [S+1]
  const int* offs;     // [S+2]
  const int* sorted;   // [T]
  const int* active;   // [S]
  const int4* desc;    // [S]: per active slot (slot, tokens, first sorted position, 0)
  const int4* tiles;   // [max_tiles]: per matrix-core tile (slot, first sorted position, length, 0)
  const int* rec;      // [S][kRecInts]: per slot (tokens, first sorted position, 0, 0, first token ids)
  const int* meta;     // [kMetaWords]
  int S, T, mfma_min, tile_m, max_tiles;
};

// Rank-space values u (fp32): partial sum of k split s for (slice n, row, rank j)
// at p[s * split_stride + n * n_stride + row * row_stride + j], s < nsplit; the value
// is the sum of its nsplit partials in split order.  Rows are token indices when
// by_token is set (the caller's finished [N][T][Rmax] buffer, nsplit = 1), sorted
// positions otherwise (the pool's workspace [nsplit][N][max_tokens][Rk]); every
// token of a call has all nsplit partials, whether a vector or a matrix-core unit
// wrote them (the matrix-core units split k into the same nsplit parts).
struct UView {
  float* p;
  long long split_stride, n_stride, row_stride;
  int nsplit, by_token;
  // slot mode: the first kMfmaTileM tokens of slot s's segment have their rows at
  // head0 + kMfmaTileM * s + t instead of at their sorted positions, so the expand finds
  // them before it has read the slot's routing record (-1: all rows by sorted position)
  int head0 = -1;
};

// Launch shape of one shrink or expand call; every workgroup is one wave.
//   shrink: the first n_dec_blocks are decode units (one active slot, k split s of
//           nsplit, one block of 16 rank rows, token tiles tg, tg + ntg, ...; split s
//           takes the wave-wide 16-byte chunk steps c = s + nsplit * m, m < ns), then
//           tile_slots x nrg matrix-core units (tile slot, group of 64 rank rows).
//   expand: the first n_dec_blocks are decode items (column tile, active slot, token
//           tiles), then tile_slots x n_mblocks matrix-core units (tile slot, 128
//           columns).  Tile slot ts takes tiles ts, ts + tile_slots, ...
struct Plan {
  int nsplit, ns;          // decode shrink: k splits, chunk steps per split
  int nrg;                 // matrix-core shrink: groups of 64 rank rows (N * Rmax / 64)
  int nrb, ntg;            // decode: 16-row blocks, token-tile groups
  int n_dec_blocks;        // workgroups of the decode part
  int tile_slots;          // matrix-core part: tiles handled in parallel
  int cb;                  // matrix-core expand: 128-column blocks per unit (1 or kMfmaColBlocksPerUnit)
  int n_mgroups;           // matrix-core expand: column groups of cb blocks (per slice, summed)
  int use_mfma;            // long segments go to the matrix-core part
  int xcd_group;           // consecutive units dealt to one XCD (1 = plain round-robin)
  int slot_mode;           // 1: slot-major units in both kernels (every segment on the matrix
                           //    cores): shrink workgroups (slot, k part, 16-row block nrb) of
                           //    slot_waves waves, expand units (slot, column group); no decode units
  int slot_waves;          // slot mode: waves sharing one k part's steps (at most 8 steps each)
  int tile_interleave;     // matrix-core expand: n > 0 deals the tile list to the XCDs in runs of n
                           // tiles (run i on XCD i % 8); 0: XCD x takes the x-th eighth of the list
};

// One module of a grouped launch (several target modules of one batch, sharing its
// routing, in one shrink and one expand launch): its pool, input, output, rank-space
// buffer and launch shape, and where its workgroups start in the launch.  A module's
// workgroups are laid out exactly as in a launch of its own (matrix-core workers,
// then decode units), so its units compute what they would compute there.
constexpr int kMaxGroup = LORA_MAX_GROUP;
struct GroupEntry {
  PoolView P;
  const void* x;
  void* y;
  int ldx, ldy;
  UView U;
  Plan plan;
  int blk0;   // first workgroup of the module (a multiple of 8, so XCD numbering is kept)
  int nm;     // its matrix-core workers
};
struct GroupView {
  int n;
  GroupEntry e[kMaxGroup];
  SlotOrder order;   // dispatch order of the decode expand units: slots by descending rank
                     // (the largest over the modules), when ordered
};

// Optional per-launch timing: when start is non-null the kernel is launched with
// hipExtLaunchKernel, which stamps the two events at the kernel's own start and end.
struct KTimer {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// kernels the timing facility reports, in this order
enum KernelId { kKRouting = 0, kKShrink, kKExpand, kKFinish, kKGather, kKernelCount };

// launchers (device code in the .hip files); all return the launch status
// ids: one per token (tps = 1) or one per sequence of tps consecutive tokens
hipError_t launch_routing(const int32_t* ids, int T, int tps, int S, int mfma_min, int tile_m, int max_tiles,
                          int* counts, int* offs, int* sorted, int* active, int4* desc, int4* tiles,
                          int* rec, int* meta, hipStream_t stream, const KTimer& tm);
// a_by_row: store A transposed, [k][Rmax] (embedding pools: k = vocabulary size)
hipError_t launch_pack_slice(int wdtype, const void* A_src, const void* B_src, void* A_dst,
                             void* Bt_dst, void* Bk_dst, int rank, int Rmax, int Rk, int k, int d,
                             int D, float scale, int premultiply, int a_by_row, hipStream_t stream);
hipError_t launch_set_slot(SlotEntry* table, int slot, SlotEntry entry, hipStream_t stream);
// Output buffers of a routing (device memory; sizes as in RouteView).
struct RouteOut {
  int* counts;
  int* offs;
  int* sorted;
  int* active;
  int4* desc;
  int4* tiles;
  int* rec;
  int* meta;
};

// A shrink launch that also builds the routing of its batch (T <= 256 tokens, S < 256
// slots): the batch's slot ids (device) and the routing's output buffers.
struct SelfRoute {
  const int32_t* ids;
  RouteOut out;
};
// a grouped launch's arguments (module descriptors, routing, self-route) and the
// runtime's hidden arguments fit the 4 KB kernel-argument segment
static_assert(sizeof(GroupView) + sizeof(RouteView) + sizeof(SelfRoute) + 256 <= 4096, "grouped launch arguments");

hipError_t launch_shrink(int wdtype, const PoolView& P, const RouteView& R, const void* x, int ldx,
                         const UView& U, const Plan& plan, const SelfRoute* sr, hipStream_t stream,
                         const KTimer& tm);

hipError_t launch_expand(int wdtype, int ydtype, const PoolView& P, const SlotOrder& order, const RouteView& R,
                         const UView& U, void* y, int ldy, const Plan& plan, hipStream_t stream,
                         const KTimer& tm);
// Workgroups of one module in a launch of its own (matrix-core workers, then decode
// units rounded up for the XCD renumbering); a grouped launch concatenates them.
int shrink_blocks(int wdtype, const PoolView& P, const Plan& plan, int& n_mfma_blocks);
int expand_blocks(int wdtype, const PoolView& P, const Plan& plan, int& n_mfma_blocks);
size_t expand_smem_bytes(int wdtype, int Rmax, int use_mfma);
// Layout of a grouped launch: every module checked (shrink shapes) and its workgroups
// placed after the previous module's (G.e[m].blk0 / nm set); false if any is invalid
bool group_layout(int wdtype, GroupView& G, const RouteView& R, const SelfRoute* sr, bool expand, int& blocks);
// Grouped launches: G.e[m].blk0 / nm set from the functions above; with sr the shrink
// launch also builds the routing (T <= 256 tokens, S < 256 slots)
hipError_t launch_shrink_group(int wdtype, const GroupView& G, const RouteView& R, const SelfRoute* sr,
                               hipStream_t stream, const KTimer& tm);
hipError_t launch_expand_group(int wdtype, int ydtype, const GroupView& G, const RouteView& R, hipStream_t stream,
                               const KTimer& tm);
// embedding pools: u (workspace split 0, rows by sorted position) = the rows of the
// transposed A [V][Rmax] of each token's slot at its vocabulary id
hipError_t launch_embed_gather(int wdtype, const PoolView& P, const RouteView& R, const int32_t* vocab_ids, int V,
                               const UView& W, hipStream_t stream, const KTimer& tm);
// the same by token index, from the tokens' slot ids (W by_token); with sr, the
// launch also builds the routing (T <= 256, S < 256)
hipError_t launch_embed_gather_tok(int wdtype, const PoolView& P, const RouteView& R, const int32_t* slot_ids,
                                   const int32_t* vocab_ids, int V, const UView& W, const SelfRoute* sr,
                                   hipStream_t stream, const KTimer& tm);
// Device address of the allocation-free call's scratch array on `device`, which
// must be the current device (taken with hipGetSymbolAddress on the first call per
// device, then kept); kNoAllocScratchBytes long.
hipError_t noalloc_scratch(int device, void** ptr);
// diagnostics: a streaming read of read_bytes (ratio <= 0; one word per thread into dst),
// or a read with one 16-byte chunk written per `ratio` chunks read
hipError_t launch_bandwidth_probe(const void* src, size_t read_bytes, void* dst, size_t dst_bytes, int ratio,
                                  hipStream_t stream);
// finished u of a standalone shrink: workspace partials -> caller's [N][T][Rmax]
hipError_t launch_finish_u(const PoolView& P, const RouteView& R, const UView& W, const UView& U,
                           const Plan& plan, hipStream_t stream, const KTimer& tm);

}  // namespace rax
