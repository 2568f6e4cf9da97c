// Expand kernels (device code): the decode expand items, the per-module body
// shared by a single-module launch and a grouped one, and the kernels themselves.
// Included by one translation unit per (weight, output) type pair, each of which
// instantiates that pair's kernels (so the library's kernels compile in parallel).
//
// Decode expand unit (one wave: slot, column tile of one slice, token tiles).  Lanes
// own 8 consecutive output columns, so each rank-major row of B^T streams as one
// contiguous 1 KB request; the tile's rank-space values (split partials added) are
// staged in the wave's LDS and read as broadcasts; the contraction over the rank
// stays in registers.  The epilogue updates the token's row of y at its original
// index, adding s * acc in fp32, one rounding.  Long segments go to the matrix-core
// units of mfma_tiles.h.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_util.h"
#include "decode_units.h"
#include "launch_util.h"
#include "mfma_tiles.h"

namespace rax {

// ------------------------------------------------------------ decode expand

// Split partials of a decode expand tile's rank-space values, QV per lane: value
// idx = lane + 64 q is rank idx / 4 of token idx % 4 (token-fastest, as the tile reads
// them from LDS).  load() issues the first kUSplitBatch splits of every value
// unconditionally (clamped addresses; splits past nsplit re-read the last), so it
// can go out in the same batch as the tile's B^T and y rows; stage() adds them in
// split order (-0.0f, the exact identity, for splits past nsplit; any further batch
// loaded there) and writes usm, zero past the rank or the tile's tokens.
template <int QV>
struct DecodeUPartials {
  float pv[QV][kUSplitBatch];
  const float* base[QV];
  bool ok[QV];
  __device__ __forceinline__ void load(const UView& U, int n, int row0, int nt, int r) {
    const int lane = lane_id();
#pragma unroll
    for (int qv = 0; qv < QV; ++qv) {
      const int idx = lane + 64 * qv, j = idx >> 2, i = idx & 3;
      ok[qv] = i < nt && j < r;
      int row = row0 + (ok[qv] ? i : 0);
      RAX_CHECK_VAR(row, U.n_stride / U.row_stride);
      base[qv] = U.p + n * U.n_stride + (long long)row * U.row_stride + (ok[qv] ? j : 0);
#pragma unroll
      for (int q = 0; q < kUSplitBatch; ++q) pv[qv][q] = base[qv][(long long)min(q, U.nsplit - 1) * U.split_stride];
    }
  }
  __device__ __forceinline__ void stage(const UView& U, int rp, float* __restrict__ usm) {
    const int lane = lane_id();
#pragma unroll
    for (int qv = 0; qv < QV; ++qv) {
      float v = pv[qv][0];
#pragma unroll
      for (int q = 1; q < kUSplitBatch; ++q) v += q < U.nsplit ? pv[qv][q] : -0.f;
      for (int q0 = kUSplitBatch; q0 < U.nsplit; q0 += 4) {
        float w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = base[qv][(long long)min(q0 + q, U.nsplit - 1) * U.split_stride];
#pragma unroll
        for (int q = 0; q < 4; ++q) v += q0 + q < U.nsplit ? w[q] : -0.f;
      }
      const int idx = lane + 64 * qv;
      if (idx < kExpandTok * rp) usm[idx] = ok[qv] ? v : 0.f;
    }
  }
};

// One decode expand item: column tile [c0, c0 + 512) of slice n, token tiles
// tt0, tt0 + 4 * ntg, ... of slot s.  Per tile: the tile's rank-space values (split
// partials added in split order, from L2) are staged in the wave's LDS token-fastest,
// and the B^T rows and y rows are loaded, then the contraction.  For the first tile,
// when the padded rank gives at most QV values per lane (QV > 0), the partials go
// out in the same batch as the B^T and y rows, so the tile waits for one round trip
// after its record; other tiles stage first, then load B^T and y.
template <typename TW, typename TY, int QV>
__device__ __forceinline__ void expand_decode_tiles(const PoolView& P, const RouteView& R, const UView& U,
                                                    TY* __restrict__ y, int ldy, int s, const SlotEntry& e,
                                                    int n, int c0, int L, int p0, int tt0, int4 tq0, int ntg,
                                                    float* __restrict__ usm) {
  using Tile = ExpandTile<TW, TY>;
  const int lane = lane_id();
  const int r = e.rank;
  const int rp = (r + Tile::RB - 1) / Tile::RB * Tile::RB;   // rank padded to the row batch
  const TW* __restrict__ bt_slot = static_cast<const TW*>(P.Bt) + (size_t)s * P.Rmax * P.D + P.o[n];
  int tt = tt0;
  if constexpr (QV > 0) {
    if (!U.by_token && kExpandTok * rp <= 64 * QV) {
      const int nt = min(kExpandTok, L - tt);
      DecodeUPartials<QV> up;
      up.load(U, n, p0 + tt, nt, r);
      Tile tile;
      tile.issue(P, bt_slot, y, ldy, n, c0, r, tq0);
      sched_fence();
      up.stage(U, rp, usm);
      wave_lds_sync();
      tile.finish(P, r, nt, e.scale, reinterpret_cast<const float4*>(usm));
      wave_lds_sync();
      tt += ntg * kExpandTok;
    }
  }
  for (; tt < L; tt += ntg * kExpandTok) {
    const int nt = min(kExpandTok, L - tt);
    int4 tq = tt == tt0 ? tq0 : segment_tokens(R, s, tt, p0, L);
    RAX_CHECK_TOKENS(tq, R.T);
    for (int idx = lane; idx < kExpandTok * rp; idx += 64) {
      const int j = idx >> 2, i = idx & 3;
      const bool ok = i < nt && j < r;
      const int ic = ok ? i : 0, jc = ok ? j : 0;
      long long row = U.by_token ? (long long)R.sorted[p0 + tt + ic] : (long long)(p0 + tt + ic);
      RAX_CHECK_VAR(row, U.by_token ? R.T : U.n_stride / U.row_stride);
      const float v = sum_splits(U.p + n * U.n_stride + row * U.row_stride + jc, U.split_stride, U.nsplit);
      usm[idx] = ok ? v : 0.f;
    }
    Tile tile;
    tile.issue(P, bt_slot, y, ldy, n, c0, r, tq);
    wave_lds_sync();
    tile.finish(P, r, nt, e.scale, reinterpret_cast<const float4*>(usm));
    wave_lds_sync();
  }
}

// order(si): the slot of dispatch position si (high-rank slots first in a launch of
// one module; by index in a grouped launch)
template <typename TW, typename TY, int QV, typename Order>
__device__ __forceinline__ void expand_decode_item(const PoolView& P, const RouteView& R, const UView& U,
                                                   TY* __restrict__ y, int ldy, const Plan& plan,
                                                   int item, float* __restrict__ usm, const Order& order) {
  // token-tile siblings (same slot and columns, same rows of B^T) are neighbours
  const int tg = item % plan.ntg;
  const int rest = item / plan.ntg;
  const int ct = rest % P.n_ctiles, si = rest / P.n_ctiles;
  const int s = order(si);
  // first round trip: record header, token ids of the first tile, slot-table entry
  const int tt0 = tg * kExpandTok;
  const int4 hdr = *reinterpret_cast<const int4*>(R.rec + (size_t)s * kRecInts);
  int4 tq0 = tt0 + 4 <= kRecTokens ? *reinterpret_cast<const int4*>(R.rec + (size_t)s * kRecInts + 4 + tt0)
                                   : make_int4(0, 0, 0, 0);
  const SlotEntry e = P.table[s];
  const int L = hdr.x;
  int p0 = hdr.y;
  RAX_CHECK_VAR(p0, R.T - L + 1);
  if (tt0 >= L) return;
  if (plan.use_mfma && L >= R.mfma_min) return;
  if (e.rank == 0 || e.scale == 0.f) return;
  if (tt0 + 4 > kRecTokens) tq0 = segment_tokens(R, s, tt0, p0, L);
  RAX_CHECK_TOKENS(tq0, R.T);
  int n = 0;
  while (n + 1 < P.N && ct >= P.tile0[n + 1]) ++n;
  if (!((e.slice_mask >> n) & 1u)) return;
  const int c0 = (ct - P.tile0[n]) * kTileCols;
  expand_decode_tiles<TW, TY, QV>(P, R, U, y, ldy, s, e, n, c0, L, p0, tt0, tq0, plan.ntg, usm);
}

// One wave per workgroup: matrix-core (tile, column group) items, then decode items.
// Waves per SIMD asked of the compiler: 2 where the body fits 256 registers without
// spilling (up to two rank steps of 32, except FP8 weights with fp32 outputs); the
// higher-rank bodies keep their natural allocation (one wave per SIMD).
template <typename TW, typename TY, int KSM>
struct ExpandWaves {
  static constexpr int value = (KSM <= 2 && !(sizeof(TW) == 1 && sizeof(TY) == 4)) ? 2 : 1;
};

// One module's expand workgroup b (counted from the module's first workgroup).
template <typename TW, typename TY, int KSM, typename Order>
__device__ __forceinline__ void expand_body(const PoolView& P, const RouteView& R, const UView& U, TY* __restrict__ y,
                                            int ldy, const Plan& plan, int n_mfma_blocks, int b,
                                            float* __restrict__ smem, const Order& order) {
  if (b >= n_mfma_blocks) {
    const int d = xcd_logical_block(b - n_mfma_blocks, plan.xcd_group);
    // values per lane of the first tile's early partial loads: the padded rank over 16
    if (d < plan.n_dec_blocks)
      expand_decode_item<TW, TY, (KSM <= 2 ? 2 * KSM : 0)>(P, R, U, y, ldy, plan, d, smem, order);
    return;
  }
  if constexpr (sizeof(TW) <= 2) {   // bf16 and FP8 weights
    LaneTable lt;
    lt.load(P);   // in flight with the tile count
    // item l of this worker's XCD is (its tile l / n_mgroups, column group l % n_mgroups):
    // XCD x takes the x-th eighth of the tile list, or (tile_interleave = n > 0) the runs
    // of n tiles x, x + 8, x + 16, ...; one call site, so the unit is inlined once
    const int ntiles = R.meta[kMetaTiles];
    MfmaItems it(b, n_mfma_blocks, ntiles * plan.n_mgroups);
    const int run = plan.tile_interleave, x = b % kXcds;
    if (run > 0) {
      const int cyc = ntiles / (kXcds * run), rem = ntiles - cyc * kXcds * run;
      it.j = b / kXcds;
      it.end = (cyc * run + min(run, max(0, rem - x * run))) * plan.n_mgroups;
    }
    for (; it.j < it.end; it.j += it.step) {
      const int q = it.j / plan.n_mgroups, g = it.j - q * plan.n_mgroups;
      const int tile = run > 0 ? ((q / run) * kXcds + x) * run + q % run : q;
      expand_mfma_unit<TW, TY, KSM>(P, R, U, y, ldy, tile, g, plan.cb, lt, smem);
    }
  }
}

// Slot mode: workgroup b of a module takes slot s = 8 (b / 8 / n_mgroups) + b % 8 (so
// it shares an XCD with the slot's shrink items) and column group (b / 8) % n_mgroups.
// Kernels of their own, so the register allocation of the tile-list kernels is not
// affected by this body.
template <typename TW, typename TY, int KSM>
__device__ __forceinline__ void expand_slot_body(const PoolView& P, const RouteView& R, const UView& U,
                                                 TY* __restrict__ y, int ldy, const Plan& plan, int b,
                                                 float* __restrict__ smem) {
  if constexpr (sizeof(TW) <= 2) {
    const int per = plan.n_mgroups, q = b / kXcds;
    const int s = (q / per) * kXcds + b % kXcds, g = q - (q / per) * per;
    if (s < P.S) expand_slot_unit<TW, TY, KSM>(P, R, U, y, ldy, s, g, plan.cb, smem);
  }
}

template <typename TW, typename TY, int KSM>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(ExpandWaves<TW, TY, KSM>::value))) void expand_slot_kernel(
    PoolView P, RouteView R, UView U, TY* __restrict__ y, int ldy, Plan plan) {
  extern __shared__ float smem[];
  expand_slot_body<TW, TY, KSM>(P, R, U, y, ldy, plan, blockIdx.x, smem);
}

template <typename TW, typename TY, int KSM>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(ExpandWaves<TW, TY, KSM>::value))) void expand_slot_group_kernel(
    GroupView G, RouteView R) {
  extern __shared__ float smem[];
  const int b = blockIdx.x;
  const GroupEntry& e = G.e[group_module(G, b)];
  expand_slot_body<TW, TY, KSM>(e.P, R, e.U, static_cast<TY*>(e.y), e.ldy, e.plan, b - e.blk0, smem);
}

template <typename TW, typename TY, int KSM>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(ExpandWaves<TW, TY, KSM>::value))) void expand_kernel(PoolView P, SlotOrder O, RouteView R, UView U,
                                                    TY* __restrict__ y, int ldy, Plan plan, int n_mfma_blocks) {
  extern __shared__ float smem[];
  expand_body<TW, TY, KSM>(P, R, U, y, ldy, plan, n_mfma_blocks, blockIdx.x, smem,
                           [&](int si) { return O.ordered ? (int)O.s[si] : si; });
}

// Several modules of one batch in one launch (workgroup b runs as workgroup b - blk0
// of its module's own launch would, with the slots dispatched in the group's order)
template <typename TW, typename TY, int KSM>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(ExpandWaves<TW, TY, KSM>::value))) void expand_group_kernel(GroupView G, RouteView R) {
  extern __shared__ float smem[];
  const int b = blockIdx.x;
  const GroupEntry& e = G.e[group_module(G, b)];
  expand_body<TW, TY, KSM>(e.P, R, e.U, static_cast<TY*>(e.y), e.ldy, e.plan, e.nm, b - e.blk0, smem,
                           [&](int si) { return G.order.ordered ? (int)G.order.s[si] : si; });
}

template <typename TW, typename TY>
static void launch_expand_w(int ksm, dim3 grid, uint32_t lds, hipStream_t stream, const PoolView& P,
                            const SlotOrder& O, const RouteView& R, const UView& U, TY* y, int ldy, const Plan& plan,
                            int nm, const KTimer& tm) {
  if constexpr (sizeof(TW) <= 2) {
    if (plan.slot_mode) {
      switch (ksm) {
        case 1: RAX_LAUNCH(tm, (expand_slot_kernel<TW, TY, 1>), grid, dim3(64), lds, stream, P, R, U, y, ldy, plan); break;
        case 2: RAX_LAUNCH(tm, (expand_slot_kernel<TW, TY, 2>), grid, dim3(64), lds, stream, P, R, U, y, ldy, plan); break;
        case 4: RAX_LAUNCH(tm, (expand_slot_kernel<TW, TY, 4>), grid, dim3(64), lds, stream, P, R, U, y, ldy, plan); break;
        default: RAX_LAUNCH(tm, (expand_slot_kernel<TW, TY, 8>), grid, dim3(64), lds, stream, P, R, U, y, ldy, plan); break;
      }
      return;
    }
  }
  switch (ksm) {
    case 1: RAX_LAUNCH(tm, (expand_kernel<TW, TY, 1>), grid, dim3(64), lds, stream, P, O, R, U, y, ldy, plan, nm); break;
    case 2: RAX_LAUNCH(tm, (expand_kernel<TW, TY, 2>), grid, dim3(64), lds, stream, P, O, R, U, y, ldy, plan, nm); break;
    case 4: RAX_LAUNCH(tm, (expand_kernel<TW, TY, 4>), grid, dim3(64), lds, stream, P, O, R, U, y, ldy, plan, nm); break;
    default: RAX_LAUNCH(tm, (expand_kernel<TW, TY, 8>), grid, dim3(64), lds, stream, P, O, R, U, y, ldy, plan, nm); break;
  }
}

template <typename TW, typename TY>
static void launch_expand_group_w(int ksm, dim3 grid, uint32_t lds, hipStream_t stream, const GroupView& G,
                                  const RouteView& R, const KTimer& tm) {
  if constexpr (sizeof(TW) <= 2) {
    if (G.e[0].plan.slot_mode) {   // every module's plan takes the same mode
      switch (ksm) {
        case 1: RAX_LAUNCH(tm, (expand_slot_group_kernel<TW, TY, 1>), grid, dim3(64), lds, stream, G, R); break;
        case 2: RAX_LAUNCH(tm, (expand_slot_group_kernel<TW, TY, 2>), grid, dim3(64), lds, stream, G, R); break;
        case 4: RAX_LAUNCH(tm, (expand_slot_group_kernel<TW, TY, 4>), grid, dim3(64), lds, stream, G, R); break;
        default: RAX_LAUNCH(tm, (expand_slot_group_kernel<TW, TY, 8>), grid, dim3(64), lds, stream, G, R); break;
      }
      return;
    }
  }
  switch (ksm) {
    case 1: RAX_LAUNCH(tm, (expand_group_kernel<TW, TY, 1>), grid, dim3(64), lds, stream, G, R); break;
    case 2: RAX_LAUNCH(tm, (expand_group_kernel<TW, TY, 2>), grid, dim3(64), lds, stream, G, R); break;
    case 4: RAX_LAUNCH(tm, (expand_group_kernel<TW, TY, 4>), grid, dim3(64), lds, stream, G, R); break;
    default: RAX_LAUNCH(tm, (expand_group_kernel<TW, TY, 8>), grid, dim3(64), lds, stream, G, R); break;
  }
}

// The launches of one (weight, output) type pair, defined by the translation unit
// that instantiates the pair.
#define RAX_EXPAND_PAIR(NAME, TW, TY)                                                                   \
  void expand_launch_##NAME(int ksm, dim3 grid, uint32_t lds, hipStream_t stream, const PoolView& P,       \
                            const SlotOrder& O, const RouteView& R, const UView& U, void* y, int ldy,      \
                            const Plan& plan, int nm, const KTimer& tm) {                               \
    launch_expand_w<TW, TY>(ksm, grid, lds, stream, P, O, R, U, static_cast<TY*>(y), ldy, plan, nm, tm);   \
  }                                                                                                     \
  void expand_group_launch_##NAME(int ksm, dim3 grid, uint32_t lds, hipStream_t stream, const GroupView& G, \
                                  const RouteView& R, const KTimer& tm) {                               \
    launch_expand_group_w<TW, TY>(ksm, grid, lds, stream, G, R, tm);                                     \
  }                                                                                                     \
  RAX_INDEX_FAULTS_ACCESSOR(NAME)

}  // namespace rax
