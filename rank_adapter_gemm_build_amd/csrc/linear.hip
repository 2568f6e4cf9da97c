// Shrink kernels (and the launches shared with the expand: the grouped layout, the
// embedding gather, the finishing pass of a standalone shrink): one launch each per
// call, covering both the short
// (decode) segments on the vector ALUs and the long segments on the matrix cores.
//
// Page "第16章 LoRA 适配器热切换", §16.4.2: with tokens grouped by slot, all LoRA branches
// of a batch run as two kernels, a shrink on lora_a into a [tokens, r] buffer and an
// expand on lora_b back to [tokens, d]; each block takes a segment of same-slot tokens.
// §16.4.3: a decode segment is as long as the number of requests on that adapter, so
// it is short; a prefill segment is long.  Page "llama.cpp 源码完全拆解(十六)", sections
// "为什么低秩增量可以「后加」" and "性能与工程取舍": decode is bound by memory bandwidth,
// the adapter's A and B are small, and the extra cost is mostly kernel launches.
//
// Short segments (fewer than mfma_min tokens) go to decode units, long ones to the
// matrix cores (mfma_tiles.h); both share one launch per kernel, so a call costs two
// launches whatever its mix.  Every unit is one wave in a workgroup of its own, so
// a launch spreads over all compute units.
//
// Decode units are numbered by slot (inactive slots end at their first load).  A
// unit's first loads are independent of each other: the slot's 128-byte routing
// record (segment length, first sorted position and the first token ids) and the
// pool's slot-table entry (rank, scale, present slices); its operand loads follow, so
// a unit waits for two memory round trips before its arithmetic.
//
// Decode shrink unit (one wave: slot, k split s, 16 rank rows, token tiles of 4).
// Lane l owns the 16-byte chunks at k offsets (s + nsplit * m) * 64 * E + l * E
// (E = 8 bf16 or 4 fp32), so every row of A streams from HBM as contiguous 1 KB
// requests and is read once per token tile, not once per token; each lane loads
// exactly the k-slice of the tile's x rows it multiplies.  The 16 rows x 4 tokens =
// 64 lane partial sums are finished by one reduce-scatter across the wave, after
// which lane l holds output l, the partial sum of split s.  Splitting k over waves
// gives a short decode batch enough waves to keep HBM busy; the partials of a value
// are added in split order where they are read (the expand), so the result does not
// depend on timing and no atomics or cross-workgroup fences are needed.
//
// The expand kernels (decode units and matrix-core units) are in expand_kernels.h,
// compiled once per weight / output type pair.
//
// Operand loads are unconditional (addresses clamped into the operand, unused values
// replaced by zero) and issued as one batch before the math.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_util.h"
#include "decode_units.h"
#include "launch_util.h"
#include "mfma_tiles.h"
#include "route_wave.h"

namespace rax {

// ------------------------------------------------------------ decode shrink
// Token tiles tt0, tt0 + 4 ntg, ... of slot s's segment (L tokens from sorted
// position p0) against 16 rank rows (block rb) over k split sp; toks(tt) gives the
// token ids at positions tt .. tt + 3 of the segment (valid rows past its end).
template <typename T, typename TW, typename Toks>
__device__ __forceinline__ void shrink_decode_tiles(const PoolView& P, const T* __restrict__ x, int ldx,
                                                    const UView& U, const Plan& plan, int s, int sp, int rb,
                                                    int tt0, int L, int p0, const SlotEntry& e, const Toks& toks) {
  const int r = e.rank, F = P.N * r, fb = rb * kShrinkRows;
  if (r == 0 || fb >= F) return;                   // uniform per wave
  const int lane = lane_id();
  const ShrinkRows<TW> A(P, s, r, fb);
  // this lane's output after the reduce-scatter: row fb + lane / 4, token lane % 4
  const int orr = lane / kShrinkTok, oi = lane - orr * kShrinkTok, of = fb + orr;
  const int on = of < F ? of / r : 0, oj = of < F ? of - on * r : 0;
  float* __restrict__ uo = U.p + sp * U.split_stride + on * U.n_stride + oj;

  for (int tt = tt0; tt < L; tt += plan.ntg * kShrinkTok) {
    const int nt = min(kShrinkTok, L - tt);
    const int4 tq = toks(tt);
    const T* xrow[kShrinkTok];
#pragma unroll
    for (int i = 0; i < kShrinkTok; ++i) xrow[i] = x + (size_t)tok_at(tq, i) * ldx;
    const float v = shrink_block_partial<T, TW>(P, A, xrow, nt, sp, plan.nsplit, plan.ns);
    if (of < F && oi < nt) {   // rows by sorted position
      int row = p0 + tt + oi;
      RAX_CHECK_VAR(row, U.n_stride / U.row_stride);
      uo[(long long)row * U.row_stride] = v;
    }
  }
}

// Unit numbering, token group fastest, then k split, slot, and the 16-row block
// slowest: the blocks past a slot's rank (units that exit after their first round
// trip) then gather at the end of the grid instead of recurring in every slot's run
// of units.  Consecutive units go to one XCD in groups (xcd_logical_block); with the
// block inside the slot, every slot's block 0 fell on the same two XCDs, so a pool
// of mixed ranks loaded those XCDs with up to four times the work of others.
struct DecodeShrinkIndex {
  int tg, sp, rb, s;
  __device__ __forceinline__ DecodeShrinkIndex(const Plan& plan, int S, int unit) {
    tg = unit % plan.ntg;
    int rest = unit / plan.ntg;
    sp = rest % plan.nsplit;
    rest /= plan.nsplit;
    s = rest % S;
    rb = rest / S;
  }
};

template <typename T, typename TW>
__device__ __forceinline__ void shrink_decode_unit(const PoolView& P, const RouteView& R,
                                                   const T* __restrict__ x, int ldx, const UView& U,
                                                   const Plan& plan, int unit) {
  const DecodeShrinkIndex u(plan, P.S, unit);
  const int s = u.s, tt0 = u.tg * kShrinkTok;
  // first round trip: record header, first token ids, slot-table entry
  const int4 hdr = *reinterpret_cast<const int4*>(R.rec + (size_t)s * kRecInts);
  const int4 tq0 = tt0 + 4 <= kRecTokens ? *reinterpret_cast<const int4*>(R.rec + (size_t)s * kRecInts + 4 + tt0)
                                         : make_int4(0, 0, 0, 0);
  const SlotEntry e = P.table[s];
  const int L = hdr.x;
  int p0 = hdr.y;
  RAX_CHECK_VAR(p0, R.T - L + 1);
  if (tt0 >= L) return;
  if (plan.use_mfma && L >= R.mfma_min) return;   // long segment: matrix-core units
  shrink_decode_tiles<T, TW>(P, x, ldx, U, plan, s, u.sp, u.rb, tt0, L, p0, e, [&](int tt) {
    int4 q = tt == tt0 && tt0 + 4 <= kRecTokens ? tq0 : segment_tokens(R, s, tt, p0, L);
    RAX_CHECK_TOKENS(q, R.T);
    return q;
  });
}

// The same unit in a launch that builds the routing itself: the segment comes from
// the batch's slot ids (BatchKeys), its token ids through the wave's LDS.
template <typename T, typename TW>
__device__ __forceinline__ void shrink_decode_unit_self(const PoolView& P, const RouteView& R,
                                                        const int32_t* __restrict__ ids, const T* __restrict__ x,
                                                        int ldx, const UView& U, const Plan& plan, int unit,
                                                        int* __restrict__ tok) {
  const DecodeShrinkIndex u(plan, P.S, unit);
  const int s = u.s, tt0 = u.tg * kShrinkTok;
  // first round trip: the batch's ids, slot-table entry
  BatchKeys K;
  K.load(ids, R.T, R.S);
  const SlotEntry e = P.table[s];
  int L, p0;
  K.segment(s, L, p0, tok);
  if (tt0 >= L) return;
  if (plan.use_mfma && L >= R.mfma_min) return;
  wave_lds_sync();
  shrink_decode_tiles<T, TW>(P, x, ldx, U, plan, s, u.sp, u.rb, tt0, L, p0, e, [&](int tt) {
    const int last = L - 1;
    return make_int4(tok[min(tt, last)], tok[min(tt + 1, last)], tok[min(tt + 2, last)], tok[min(tt + 3, last)]);
  });
}

// LDS ints of a self-routing shrink workgroup
constexpr int kShrinkSelfLds = route_wave_lds_ints(kSelfRouteQ, kSelfRouteK / 64);
static_assert(kShrinkSelfLds >= kSelfRouteK + 2 * kSelfRouteT, "unit LDS");

// ------------------------------------------------------------ slot-major shrink
// Slot mode (small batches with most slots active): one workgroup per (slot s, k part,
// 16-row block rb of the pool's N x Rmax rows), every segment length on the matrix
// cores.  The part's k steps of 32 are split over the plan's slot_waves waves, at most
// 8 steps each (so a wave's loads go out as one batch of 8 A and 8 x fragments); the
// waves' products are added in wave order through LDS and written as the part's
// partial sum, by sorted position, as the tile items write theirs (a part with no k
// steps writes zeros).  Row f = 16 rb + lane % 16 is rank row f % Rmax of slice
// f / Rmax (rows past a slot's rank are zero in A and masked), so a wave's A fragments
// depend on nothing but the workgroup's index and go out first, in the same round trip
// as the batch's ids (SELF: the first wave derives the slot's segment from them) or
// the slot's routing record, and the slot-table entry.
constexpr int kSlotSteps = 8;        // k steps of 32 per wave
constexpr int kSlotMaxWaves = 8;     // waves per workgroup
struct SlotShared {
  float red[kSlotMaxWaves][kMfmaTileM][kMfmaTileM + 1];
  int tok[kSelfRouteT];
  int seg[2];
};

template <typename TW, bool SELF>
__device__ __forceinline__ void shrink_slot_wg(const PoolView& P, const RouteView& R, const int32_t* __restrict__ ids,
                                               const uint16_t* __restrict__ x, int ldx, const UView& U,
                                               const Plan& plan, int b, SlotShared& sm) {
  using W = WChunk<TW>;
  const int per = plan.nsplit * plan.nrb, q = b / kXcds;
  const int s = (q / per) * kXcds + b % kXcds, rest = q - (q / per) * per;
  if (s >= P.S) return;   // whole workgroup
  const int part = rest / plan.nrb, rb = rest - part * plan.nrb;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 15, lk = lane >> 4;
  const int nw = plan.slot_waves;   // waves past it (a grouped launch's wider workgroups) only join the barriers
  const int F = P.N * P.Rmax, f = 16 * rb + lr;
  const bool fv = f < F;
  const int n = fv ? f / P.Rmax : 0, j = fv ? f - n * P.Rmax : 0;
  int s0, s1;
  mfma_part_range(P.k, part, U.nsplit, s0, s1);
  const int spw = (s1 - s0 + nw - 1) / nw;               // <= kSlotSteps (the host's split)
  const int w0 = w < nw ? min(s0 + w * spw, s1) : s1, w1 = min(w0 + spw, s1);
  const int wlast = max(w1 - 1, w0);
  const TW* __restrict__ arow = static_cast<const TW*>(P.A) + (((size_t)s * P.N + n) * P.Rmax + j) * P.k;
  typename W::type af[kSlotSteps];
#pragma unroll
  for (int st = 0; st < kSlotSteps; ++st)
    af[st] = W::load(arow + min(min(w0 + st, wlast) * kMfmaK + 8 * lk, P.k - 8));
  const SlotEntry e = P.table[s];
  int L, p0, tok0 = 0;
  if constexpr (SELF) {
    if (w == 0) {
      BatchKeys K;
      K.load(ids, R.T, R.S);
      K.segment(s, L, p0, sm.tok);
      if (lane == 0) { sm.seg[0] = L; sm.seg[1] = p0; }
    }
    __syncthreads();
    L = __builtin_amdgcn_readfirstlane(sm.seg[0]);
    p0 = __builtin_amdgcn_readfirstlane(sm.seg[1]);
  } else {
    // the record's header and its first token ids (entries past the segment repeat a
    // valid token), so the first tile needs no further round trip
    const int* __restrict__ rec = R.rec + (size_t)s * kRecInts;
    const int2 hdr = *reinterpret_cast<const int2*>(rec);
    tok0 = rec[4 + lr];
    L = __builtin_amdgcn_readfirstlane(hdr.x);
    p0 = __builtin_amdgcn_readfirstlane(hdr.y);
    RAX_CHECK_VAR(p0, R.T - L + 1);
  }
  const int r = e.rank;
  const bool row_ok = fv && j < r;
  if (L == 0 || r == 0 || __ballot(row_ok) == 0ull) return;   // whole workgroup (same slot and rows)
  for (int t0 = 0; t0 < L; t0 += kMfmaTileM) {
    const int len = min(kMfmaTileM, L - t0), ti = t0 + min(lr, len - 1);
    int tk;
    if constexpr (SELF) tk = sm.tok[ti];
    else tk = t0 == 0 ? tok0 : (ti < kRecTokens ? R.rec[(size_t)s * kRecInts + 4 + ti] : R.sorted[p0 + ti]);
    RAX_CHECK_VAR(tk, R.T);
    const uint16_t* __restrict__ xrow = x + (size_t)tk * ldx;
    uint4 xa[kSlotSteps];
#pragma unroll
    for (int st = 0; st < kSlotSteps; ++st) xa[st] = ld16(xrow + min(min(w0 + st, wlast) * kMfmaK + 8 * lk, P.k - 8));
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const bool tval = lr < len;
#pragma unroll
    for (int st = 0; st < kSlotSteps; ++st) {
      // steps past the wave's share, and this lane's chunk past k in the last step
      // (k % 8 == 0: chunks are wholly in or out), contribute zero
      const bool inb = w0 + st < w1 && (w0 + st) * kMfmaK + 8 * lk < P.k;
      if constexpr (sizeof(TW) == 1) {
        const uint2 xq = W::keep(bf16x8_to_fp8x8(xa[st]), tval && inb);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(as_i64(xq), as_i64(W::keep(af[st], row_ok)), acc, 0, 0, 0);
      } else {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(keep_if(xa[st], tval && inb)),
                                                      as_bf16x8(W::keep(af[st], row_ok)), acc, 0, 0, 0);
      }
    }
    // lane holds D[token 4 lk + i][row f]; the waves' sums added in wave order
    if (w < nw) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.red[w][4 * lk + i][lr] = acc[i];
    }
    __syncthreads();
    for (int idx = tid; idx < kMfmaTileM * kMfmaTileM; idx += blockDim.x) {   // (token, row) of the tile
      const int t = idx >> 4, rr = idx & 15, fr = 16 * rb + rr;
      const int nn = fr / P.Rmax, jj = fr - nn * P.Rmax;
      if (t < len && fr < F && jj < r) {
        float v = sm.red[0][t][rr];
        for (int ww = 1; ww < nw; ++ww) v += sm.red[ww][t][rr];
        long long row = t0 == 0 && U.head0 >= 0 ? (long long)U.head0 + kMfmaTileM * s + t : p0 + t0 + t;
        RAX_CHECK_VAR(row, U.n_stride / U.row_stride);
        U.p[part * U.split_stride + nn * U.n_stride + row * U.row_stride + jj] = v;
      }
    }
    __syncthreads();
  }
}

template <typename TW, bool SELF>
__global__ __launch_bounds__(64 * kSlotMaxWaves) void shrink_slot_kernel(PoolView P, RouteView R,
                                                                         const uint16_t* __restrict__ x, int ldx,
                                                                         UView U, Plan plan, SelfRoute sr) {
  __shared__ __align__(16) char smem[sizeof(SlotShared) > kShrinkSelfLds * sizeof(int) ? sizeof(SlotShared)
                                                                                       : kShrinkSelfLds * sizeof(int)];
  int b = blockIdx.x;
  if constexpr (SELF) {
    if (b < kXcds) {
      if (b == 0 && threadIdx.x < 64)
        route_wave<kSelfRouteQ, kSelfRouteK / 64>(sr.ids, R.T, 1, R.S, R.mfma_min, R.tile_m, R.max_tiles, sr.out,
                                                  reinterpret_cast<int*>(smem));
      return;
    }
    b -= kXcds;
  }
  shrink_slot_wg<TW, SELF>(P, R, sr.ids, x, ldx, U, plan, b, *reinterpret_cast<SlotShared*>(smem));
}

template <typename TW, bool SELF>
__global__ __launch_bounds__(64 * kSlotMaxWaves) void shrink_slot_group_kernel(GroupView G, RouteView R, SelfRoute sr) {
  __shared__ __align__(16) char smem[sizeof(SlotShared) > kShrinkSelfLds * sizeof(int) ? sizeof(SlotShared)
                                                                                       : kShrinkSelfLds * sizeof(int)];
  int b = blockIdx.x;
  if constexpr (SELF) {
    if (b < kXcds) {
      if (b == 0 && threadIdx.x < 64)
        route_wave<kSelfRouteQ, kSelfRouteK / 64>(sr.ids, R.T, 1, R.S, R.mfma_min, R.tile_m, R.max_tiles, sr.out,
                                                  reinterpret_cast<int*>(smem));
      return;
    }
    b -= kXcds;
  }
  const GroupEntry& e = G.e[group_module(G, b)];
  shrink_slot_wg<TW, SELF>(e.P, R, sr.ids, static_cast<const uint16_t*>(e.x), e.ldx, e.U, e.plan, b - e.blk0,
                           *reinterpret_cast<SlotShared*>(smem));
}

// One module's shrink workgroup b (b counted from the module's first workgroup):
// matrix-core (k part, tile, row group) items, then decode units.  SELF: the launch
// also builds the routing (route_wave in its first workgroup), and the units take
// their segments and tiles from the batch's ids (BatchKeys, BatchTiles) instead of
// the routing outputs being written meanwhile; sh is the wave's LDS for that.  T is
// the type of x, TW of the weights (T, or FP8 with bf16 x).
template <typename T, typename TW, bool SELF>
__device__ __forceinline__ void shrink_body(const PoolView& P, const RouteView& R, const T* __restrict__ x, int ldx,
                                            const UView& U, const Plan& plan, int n_mfma_blocks,
                                            const int32_t* __restrict__ ids, int b, int* __restrict__ sh) {
  if constexpr (SELF) {
    int* tok = sh + kSelfRouteK;
    if (b >= n_mfma_blocks) {
      const int d = xcd_logical_block(b - n_mfma_blocks, plan.xcd_group);
      if (d < plan.n_dec_blocks) shrink_decode_unit_self<T, TW>(P, R, ids, x, ldx, U, plan, d, tok);
      return;
    }
    if constexpr (sizeof(T) == 2 && sizeof(TW) <= 2) {
      // LDS: slot counts [kSelfRouteK], then the tile's tokens, then the batch's keys
      int* keys = sh + kSelfRouteK + kSelfRouteT;
      int ntiles;
      // pools of up to 64 slots: lane l holds slot l's table entry, loaded with the ids,
      // so a tile's entry needs no round trip of its own
      const bool table_in_lanes = P.S <= 64;
      const int4 te = *reinterpret_cast<const int4*>(P.table + min(lane_id(), P.S - 1));
      {
        BatchKeys K;
        K.load(ids, R.T, R.S);
        K.store(keys);
        ntiles = BatchTiles::build(K, R.S, R.mfma_min, R.tile_m, R.max_tiles, sh);
      }
      const int per_part = ntiles * plan.nrg;
      for (MfmaItems it(b, n_mfma_blocks, per_part * plan.nsplit); it.j < it.end; it.j += it.step) {
        const int part = it.j / per_part, rem = it.j - part * per_part;
        const int tile = rem / plan.nrg, rg = rem - tile * plan.nrg;
        int slot, ti, L, p0;
        BatchTiles::find(sh, R.S, R.mfma_min, R.tile_m, tile, slot, ti);
        BatchKeys K;
        K.reload(keys);
        wave_lds_sync();
        K.segment(slot, L, p0, tok);
        wave_lds_sync();
        const int first = ti * R.tile_m, len = min(R.tile_m, L - first);
        SlotEntry e;
        if (table_in_lanes) {
          e.rank = __builtin_amdgcn_readfirstlane(__shfl(te.x, slot));   // wave-uniform
          e.scale = __int_as_float(__builtin_amdgcn_readfirstlane(__shfl(te.y, slot)));
          e.slice_mask = (uint32_t)__builtin_amdgcn_readfirstlane(__shfl(te.z, slot));
          e.pad = 0;
        } else {
          e = P.table[slot];
        }
        const uint16_t* __restrict__ xrow = x + (size_t)tok[first + min(lane_id() & 15, len - 1)] * ldx;
        shrink_mfma_tile<TW>(P, e, xrow, U, slot, p0 + first, len, rg, part, plan.nsplit);
      }
    }
    return;
  }
  if (b >= n_mfma_blocks) {
    const int d = xcd_logical_block(b - n_mfma_blocks, plan.xcd_group);
    if (d < plan.n_dec_blocks) shrink_decode_unit<T, TW>(P, R, x, ldx, U, plan, d);
    return;
  }
  if constexpr (sizeof(T) == 2 && sizeof(TW) <= 2) {
    // items part-major: an XCD's stretch covers whole k parts (with 8 parts, one
    // each), so the rows of A and the k-slices of x it reads are its own
    const int ntiles = R.meta[kMetaTiles], per_part = ntiles * plan.nrg;
    for (MfmaItems it(b, n_mfma_blocks, per_part * plan.nsplit); it.j < it.end; it.j += it.step) {
      const int part = it.j / per_part, rem = it.j - part * per_part;
      const int tile = rem / plan.nrg, rg = rem - tile * plan.nrg;
      shrink_mfma_unit<TW>(P, R, x, ldx, U, tile, rg, part, plan.nsplit);
    }
  }
}


// One wave per workgroup.  SELF: workgroup 0 runs route_wave and workgroups 1-7 are
// idle, so the others keep their XCD numbering.
// Two waves per SIMD: asked of the compiler (which then keeps the matrix-core
// accumulators in ordinary vector registers, 223 registers for the routing variant
// instead of 240 + 24 accumulation registers, which allowed only one wave per SIMD)
template <typename T, typename TW, bool SELF>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void shrink_kernel(PoolView P, RouteView R, const T* __restrict__ x,
                                                    int ldx, UView U, Plan plan, int n_mfma_blocks, SelfRoute sr) {
  int b = blockIdx.x;
  if constexpr (SELF) {
    __shared__ __align__(16) int sh[kShrinkSelfLds];
    if (b < kXcds) {
      if (b == 0)
        route_wave<kSelfRouteQ, kSelfRouteK / 64>(sr.ids, R.T, 1, R.S, R.mfma_min, R.tile_m, R.max_tiles, sr.out, sh);
      return;
    }
    shrink_body<T, TW, true>(P, R, x, ldx, U, plan, n_mfma_blocks, sr.ids, b - kXcds, sh);
  } else {
    shrink_body<T, TW, false>(P, R, x, ldx, U, plan, n_mfma_blocks, nullptr, b, nullptr);
  }
}

// Several modules of one batch in one launch: workgroup b runs as workgroup
// b - blk0 of its module's own launch would.
template <typename T, typename TW, bool SELF>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void shrink_group_kernel(GroupView G, RouteView R, SelfRoute sr) {
  int b = blockIdx.x;
  if constexpr (SELF) {
    __shared__ __align__(16) int sh[kShrinkSelfLds];
    if (b < kXcds) {
      if (b == 0)
        route_wave<kSelfRouteQ, kSelfRouteK / 64>(sr.ids, R.T, 1, R.S, R.mfma_min, R.tile_m, R.max_tiles, sr.out, sh);
      return;
    }
    b -= kXcds;
    const GroupEntry& e = G.e[group_module(G, b)];
    shrink_body<T, TW, true>(e.P, R, static_cast<const T*>(e.x), e.ldx, e.U, e.plan, e.nm, sr.ids, b - e.blk0, sh);
  } else {
    const GroupEntry& e = G.e[group_module(G, b)];
    shrink_body<T, TW, false>(e.P, R, static_cast<const T*>(e.x), e.ldx, e.U, e.plan, e.nm, nullptr, b - e.blk0,
                              nullptr);
  }
}

int shrink_blocks(int wdtype, const PoolView& P, const Plan& plan, int& n_mfma_blocks) {
  (void)wdtype;
  if (plan.slot_mode) {   // slot-major items only (XCD-aligned slot groups)
    n_mfma_blocks = (P.S + kXcds - 1) / kXcds * kXcds * plan.nsplit * plan.nrb;
    return n_mfma_blocks;
  }
  n_mfma_blocks = plan.use_mfma ? mfma_blocks(plan.tile_slots * plan.nrg * plan.nsplit) : 0;
  const int q = kXcds * plan.xcd_group;
  return n_mfma_blocks + (plan.n_dec_blocks + q - 1) / q * q;
}

template <typename T, typename TW>
static void launch_shrink_t(const PoolView& P, const RouteView& R, const T* x, int ldx, const UView& U,
                            const Plan& plan, const SelfRoute* sr, hipStream_t stream, const KTimer& tm) {
  int nm;
  const int blocks = shrink_blocks(0, P, plan, nm);
  if constexpr (sizeof(T) == 2 && sizeof(TW) <= 2) {
    if (plan.slot_mode) {
      const dim3 block(64 * plan.slot_waves);
      if (sr)
        RAX_LAUNCH(tm, (shrink_slot_kernel<TW, true>), dim3(kXcds + blocks), block, 0u, stream, P, R, x, ldx, U, plan,
                   *sr);
      else
        RAX_LAUNCH(tm, (shrink_slot_kernel<TW, false>), dim3(blocks), block, 0u, stream, P, R, x, ldx, U, plan,
                   SelfRoute{});
      return;
    }
  }
  if (sr)
    RAX_LAUNCH(tm, (shrink_kernel<T, TW, true>), dim3(kXcds + blocks), dim3(64), 0u, stream, P, R, x, ldx, U, plan, nm,
               *sr);
  else
    RAX_LAUNCH(tm, (shrink_kernel<T, TW, false>), dim3(blocks), dim3(64), 0u, stream, P, R, x, ldx, U, plan, nm,
               SelfRoute{});
}

// The checks of a shrink launch's shape, shared by single and grouped launches
static bool shrink_shape_ok(int wdtype, const PoolView& P, const RouteView& R, const UView& U, const Plan& plan,
                            const SelfRoute* sr) {
  const int cw = 64 * (wdtype == LORA_F32 ? 4 : 8);   // x is bf16 for FP8 pools
  const int chunks = (P.k + cw - 1) / cw;
  if (plan.slot_mode) {
    // every wave's share of its part fits its register-held A fragments
    const int steps = (P.k + kMfmaK - 1) / kMfmaK;
    const int per_part = (steps + plan.nsplit - 1) / std::max(plan.nsplit, 1);
    return !(U.by_token || wdtype == LORA_F32 || !plan.use_mfma || U.nsplit != plan.nsplit || plan.nsplit < 1 ||
             plan.nsplit > kMaxSplit || plan.slot_waves < 1 || plan.slot_waves > kSlotMaxWaves ||
             (per_part + plan.slot_waves - 1) / plan.slot_waves > kSlotSteps || plan.n_dec_blocks != 0 ||
             plan.nrb * kShrinkRows < P.N * P.Rmax || R.T > kSelfRouteT ||
             (sr && (!sr->ids || R.T < 1 || R.S + 1 > kSelfRouteK)));
  }
  return !(plan.xcd_group < 1 || U.by_token || U.nsplit != plan.nsplit || plan.nsplit < 1 || plan.nsplit > kMaxSplit ||
           plan.ns < 1 || plan.nsplit * plan.ns < chunks || plan.ntg < 1 || plan.nrb * kShrinkRows < P.N * P.Rmax ||
           plan.n_dec_blocks != P.S * plan.nrb * plan.nsplit * plan.ntg ||
           (plan.use_mfma && (wdtype == LORA_F32 || plan.tile_slots < 1 || plan.nrg * 64 < P.N * P.Rmax)) ||
           (sr && (!sr->ids || R.T < 1 || R.T > kSelfRouteT || R.S + 1 > kSelfRouteK)));
}

hipError_t launch_shrink(int wdtype, const PoolView& P, const RouteView& R, const void* x, int ldx,
                         const UView& U, const Plan& plan, const SelfRoute* sr, hipStream_t stream,
                         const KTimer& tm) {
  if (!shrink_shape_ok(wdtype, P, R, U, plan, sr)) return hipErrorInvalidValue;
  if (wdtype == LORA_BF16)
    launch_shrink_t<uint16_t, uint16_t>(P, R, static_cast<const uint16_t*>(x), ldx, U, plan, sr, stream, tm);
  else if (wdtype == LORA_FP8E4M3)
    launch_shrink_t<uint16_t, uint8_t>(P, R, static_cast<const uint16_t*>(x), ldx, U, plan, sr, stream, tm);
  else
    launch_shrink_t<float, float>(P, R, static_cast<const float*>(x), ldx, U, plan, sr, stream, tm);
  return hipGetLastError();
}

// Every module's shape checked, and its workgroups laid out as in a launch of its
// own, one module after the other (blk0 and nm set here).
bool group_layout(int wdtype, GroupView& G, const RouteView& R, const SelfRoute* sr, bool expand,
                         int& blocks) {
  if (G.n < 1 || G.n > kMaxGroup) return false;
  blocks = 0;
  for (int m = 0; m < G.n; ++m) {
    GroupEntry& e = G.e[m];
    if (!e.x && !expand) return false;
    if (!e.y && expand) return false;
    int nm;
    const int nb = expand ? expand_blocks(wdtype, e.P, e.plan, nm) : shrink_blocks(wdtype, e.P, e.plan, nm);
    if (!expand && !shrink_shape_ok(wdtype, e.P, R, e.U, e.plan, sr)) return false;
    e.blk0 = blocks;
    e.nm = nm;
    blocks += nb;
  }
  return blocks > 0;
}

template <typename T, typename TW>
static void launch_shrink_group_t(const GroupView& G, int blocks, const RouteView& R, const SelfRoute* sr,
                                  hipStream_t stream, const KTimer& tm) {
  if constexpr (sizeof(T) == 2 && sizeof(TW) <= 2) {
    if (G.e[0].plan.slot_mode) {   // every module's plan takes the same mode
      int nw = 1;
      for (int m = 0; m < G.n; ++m) nw = std::max(nw, G.e[m].plan.slot_waves);
      if (sr)
        RAX_LAUNCH(tm, (shrink_slot_group_kernel<TW, true>), dim3(kXcds + blocks), dim3(64 * nw), 0u, stream, G, R,
                   *sr);
      else
        RAX_LAUNCH(tm, (shrink_slot_group_kernel<TW, false>), dim3(blocks), dim3(64 * nw), 0u, stream, G, R,
                   SelfRoute{});
      return;
    }
  }
  if (sr)
    RAX_LAUNCH(tm, (shrink_group_kernel<T, TW, true>), dim3(kXcds + blocks), dim3(64), 0u, stream, G, R, *sr);
  else
    RAX_LAUNCH(tm, (shrink_group_kernel<T, TW, false>), dim3(blocks), dim3(64), 0u, stream, G, R, SelfRoute{});
}

hipError_t launch_shrink_group(int wdtype, const GroupView& G0, const RouteView& R, const SelfRoute* sr,
                               hipStream_t stream, const KTimer& tm) {
  GroupView G = G0;
  int blocks;
  if (!group_layout(wdtype, G, R, sr, false, blocks)) return hipErrorInvalidValue;
  if (wdtype == LORA_BF16)
    launch_shrink_group_t<uint16_t, uint16_t>(G, blocks, R, sr, stream, tm);
  else if (wdtype == LORA_FP8E4M3)
    launch_shrink_group_t<uint16_t, uint8_t>(G, blocks, R, sr, stream, tm);
  else
    launch_shrink_group_t<float, float>(G, blocks, R, sr, stream, tm);
  return hipGetLastError();
}

// Finished u of a standalone shrink: for every LoRA token of an active slot, the
// partials of the workspace W summed in split order into the caller's buffer U, by
// token.  One block per active slot.
__global__ __launch_bounds__(256) void finish_u_kernel(PoolView P, RouteView R, UView W, UView U) {
  const int a = blockIdx.x;
  if (a >= R.meta[kMetaActive]) return;
  const int4 d = R.desc[a];
  const int slot = d.x, L = d.y, p0 = d.z;
  const SlotEntry e = P.table[slot];
  const int r = e.rank;
  if (r == 0) return;
  const int per_tok = P.N * r;
  for (int idx = threadIdx.x; idx < L * per_tok; idx += blockDim.x) {
    const int t = idx / per_tok, f = idx - t * per_tok, n = f / r, j = f - n * r;
    const float v = sum_splits(W.p + n * W.n_stride + (long long)(p0 + t) * W.row_stride + j, W.split_stride, W.nsplit);
    U.p[n * U.n_stride + (long long)R.sorted[p0 + t] * U.row_stride + j] = v;
  }
}

hipError_t launch_finish_u(const PoolView& P, const RouteView& R, const UView& W, const UView& U,
                           const Plan& plan, hipStream_t stream, const KTimer& tm) {
  (void)plan;
  if (W.nsplit < 1 || W.nsplit > kMaxSplit || W.by_token || !U.by_token) return hipErrorInvalidValue;
  RAX_LAUNCH(tm, finish_u_kernel, dim3(R.S), dim3(256), 0u, stream, P, R, W, U);
  return hipGetLastError();
}

// Embedding LoRA (page "llama.cpp 源码完全拆解(十六)", section "嵌入层:查表后再加增量":
// get_rows takes each token's r-vector out of A by its vocabulary id, then B lifts it
// to the output width): the workspace row of sorted position p < offs[S] (split 0,
// slice 0) gets A^T[slot][v][j] for j < rank and a vocabulary id v in [0, V), else
// 0, for j < Rk; the expand then runs on it as on a finished shrink.  The slot of a
// position comes from the segment offsets, staged in LDS (binary search).  One thread
// per (position, rank) value, so a token's rank values are one contiguous read.
template <typename T>
__global__ __launch_bounds__(256) void embed_gather_kernel(PoolView P, RouteView R, const int32_t* __restrict__ vocab_ids,
                                                           int V, UView W) {
  extern __shared__ int offs[];   // [S + 2]
  for (int i = threadIdx.x; i < R.S + 2; i += blockDim.x) offs[i] = R.offs[i];
  __syncthreads();
  const long long n = (long long)offs[R.S] * P.Rk;   // LoRA tokens come first
  const T* __restrict__ At = static_cast<const T*>(P.A);
  for (long long idx = blockIdx.x * (long long)blockDim.x + threadIdx.x; idx < n;
       idx += (long long)gridDim.x * blockDim.x) {
    const int p = (int)(idx / P.Rk), j = (int)(idx - (long long)p * P.Rk);
    int lo = 0, hi = R.S - 1;   // the last slot whose segment starts at or before p
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (offs[mid] <= p) lo = mid; else hi = mid - 1;
    }
    const SlotEntry e = P.table[lo];
    const int v = vocab_ids[R.sorted[p]];
    float val = 0.f;
    if (j < e.rank && v >= 0 && v < V) {
      const T a = At[((size_t)lo * P.k + v) * P.Rmax + j];
      if constexpr (sizeof(T) == 2) val = __uint_as_float((uint32_t)a << 16); else val = a;
    }
    W.p[(long long)p * W.row_stride + j] = val;
  }
}

hipError_t launch_embed_gather(int wdtype, const PoolView& P, const RouteView& R, const int32_t* vocab_ids, int V,
                               const UView& W, hipStream_t stream, const KTimer& tm) {
  if (W.by_token || W.nsplit != 1 || W.row_stride < P.Rk || P.N != 1 || P.k != V || R.T < 1 || !vocab_ids)
    return hipErrorInvalidValue;
  const long long n = (long long)R.T * P.Rk;   // at least the LoRA tokens' values
  const int blocks = (int)std::min<long long>((n + 255) / 256, 4096);
  const uint32_t lds = (uint32_t)((R.S + 2) * sizeof(int));
  if (wdtype == LORA_BF16)
    RAX_LAUNCH(tm, embed_gather_kernel<uint16_t>, dim3(blocks), dim3(256), lds, stream, P, R, vocab_ids, V, W);
  else
    RAX_LAUNCH(tm, embed_gather_kernel<float>, dim3(blocks), dim3(256), lds, stream, P, R, vocab_ids, V, W);
  return hipGetLastError();
}

// The same gather by token index, for a call that also has the tokens' slot ids: row
// t of W gets A^T[slot_ids[t]][vocab_ids[t]][j] (zero for no-LoRA tokens, ranks past
// the slot's and out-of-vocabulary ids), read by the expand as a caller's finished u.
// ROUTE: the launch also builds the routing of the batch (route_wave on the first
// wave of workgroup 0, T <= 256 and S < 256), which only the expand reads.
template <typename T, bool ROUTE>
__global__ __launch_bounds__(256) void embed_gather_tok_kernel(PoolView P, RouteView R, const int32_t* __restrict__ slot_ids,
                                                               const int32_t* __restrict__ vocab_ids, int V, UView W,
                                                               SelfRoute sr) {
  int b = blockIdx.x;
  if constexpr (ROUTE) {
    __shared__ __align__(16) int sh[route_wave_lds_ints(kSelfRouteQ, kSelfRouteK / 64)];
    if (b == 0) {
      if (threadIdx.x < 64)
        route_wave<kSelfRouteQ, kSelfRouteK / 64>(sr.ids, R.T, 1, R.S, R.mfma_min, R.tile_m, R.max_tiles, sr.out, sh);
      return;
    }
    b -= 1;
  }
  const long long n = (long long)R.T * P.Rk;
  const long long step = (long long)(gridDim.x - (ROUTE ? 1 : 0)) * blockDim.x;
  const T* __restrict__ At = static_cast<const T*>(P.A);
  for (long long idx = b * (long long)blockDim.x + threadIdx.x; idx < n; idx += step) {
    const int t = (int)(idx / P.Rk), j = (int)(idx - (long long)t * P.Rk);
    const int s = slot_ids[t], v = vocab_ids[t];
    float val = 0.f;
    if (s >= 0 && s < P.S && v >= 0 && v < V && j < P.table[s].rank) {
      const T a = At[((size_t)s * P.k + v) * P.Rmax + j];
      if constexpr (sizeof(T) == 2) val = __uint_as_float((uint32_t)a << 16); else val = a;
    }
    W.p[(long long)t * W.row_stride + j] = val;
  }
}

hipError_t launch_embed_gather_tok(int wdtype, const PoolView& P, const RouteView& R, const int32_t* slot_ids,
                                   const int32_t* vocab_ids, int V, const UView& W, const SelfRoute* sr,
                                   hipStream_t stream, const KTimer& tm) {
  if (!W.by_token || W.nsplit != 1 || W.row_stride < P.Rk || P.N != 1 || P.k != V || R.T < 1 || !vocab_ids ||
      !slot_ids || (sr && (sr->ids != slot_ids || R.T > kSelfRouteT || R.S + 1 > kSelfRouteK)))
    return hipErrorInvalidValue;
  const long long n = (long long)R.T * P.Rk;
  const int blocks = (int)std::min<long long>((n + 255) / 256, 4096);
  const SelfRoute none{};
  if (wdtype == LORA_BF16) {
    if (sr)
      RAX_LAUNCH(tm, (embed_gather_tok_kernel<uint16_t, true>), dim3(blocks + 1), dim3(256), 0u, stream, P, R, slot_ids,
                 vocab_ids, V, W, *sr);
    else
      RAX_LAUNCH(tm, (embed_gather_tok_kernel<uint16_t, false>), dim3(blocks), dim3(256), 0u, stream, P, R, slot_ids,
                 vocab_ids, V, W, none);
  } else {
    if (sr)
      RAX_LAUNCH(tm, (embed_gather_tok_kernel<float, true>), dim3(blocks + 1), dim3(256), 0u, stream, P, R, slot_ids,
                 vocab_ids, V, W, *sr);
    else
      RAX_LAUNCH(tm, (embed_gather_tok_kernel<float, false>), dim3(blocks), dim3(256), 0u, stream, P, R, slot_ids,
                 vocab_ids, V, W, none);
  }
  return hipGetLastError();
}

RAX_INDEX_FAULTS_ACCESSOR(linear)

}  // namespace rax
