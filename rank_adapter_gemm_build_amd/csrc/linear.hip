// Shrink and expand kernels: one launch each per call, covering both the short
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
// Decode expand unit (one wave: slot, column tile of one slice, token tiles).  Lanes
// own 8 consecutive output columns, so each rank-major row of B^T streams as one
// contiguous 1 KB request; the tile's rank-space values (split partials added) are
// staged in the wave's LDS and read as broadcasts; the contraction over the rank
// stays in registers.  The epilogue updates the token's row of y at its original
// index (no permutation pass; page "TensorRT-LLM 源码完全拆解(二十一)", section "前向替换",
// restores the order with index_copy_ instead), adding s * acc in fp32, one rounding.
//
// Operand loads are unconditional (addresses clamped into the operand, unused values
// replaced by zero) and issued as one batch before the math.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_util.h"
#include "decode_units.h"
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
    if (of < F && oi < nt) uo[(long long)(p0 + tt + oi) * U.row_stride] = v;   // rows by sorted position
  }
}

struct DecodeShrinkIndex {
  int tg, sp, rb, s;
  __device__ __forceinline__ DecodeShrinkIndex(const Plan& plan, int unit) {
    tg = unit % plan.ntg;
    int rest = unit / plan.ntg;
    sp = rest % plan.nsplit;
    rest /= plan.nsplit;
    rb = rest % plan.nrb;
    s = rest / plan.nrb;
  }
};

template <typename T, typename TW>
__device__ __forceinline__ void shrink_decode_unit(const PoolView& P, const RouteView& R,
                                                   const T* __restrict__ x, int ldx, const UView& U,
                                                   const Plan& plan, int unit) {
  const DecodeShrinkIndex u(plan, unit);
  const int s = u.s, tt0 = u.tg * kShrinkTok;
  // first round trip: record header, first token ids, slot-table entry
  const int4 hdr = *reinterpret_cast<const int4*>(R.rec + (size_t)s * kRecInts);
  const int4 tq0 = tt0 + 4 <= kRecTokens ? *reinterpret_cast<const int4*>(R.rec + (size_t)s * kRecInts + 4 + tt0)
                                         : make_int4(0, 0, 0, 0);
  const SlotEntry e = P.table[s];
  const int L = hdr.x, p0 = hdr.y;
  if (tt0 >= L) return;
  if (plan.use_mfma && L >= R.mfma_min) return;   // long segment: matrix-core units
  shrink_decode_tiles<T, TW>(P, x, ldx, U, plan, s, u.sp, u.rb, tt0, L, p0, e, [&](int tt) {
    return tt == tt0 && tt0 + 4 <= kRecTokens ? tq0 : segment_tokens(R, s, tt, p0, L);
  });
}

// The same unit in a launch that builds the routing itself: the segment comes from
// the batch's slot ids (BatchKeys), its token ids through the wave's LDS.
template <typename T, typename TW>
__device__ __forceinline__ void shrink_decode_unit_self(const PoolView& P, const RouteView& R,
                                                        const int32_t* __restrict__ ids, const T* __restrict__ x,
                                                        int ldx, const UView& U, const Plan& plan, int unit,
                                                        int* __restrict__ tok) {
  const DecodeShrinkIndex u(plan, unit);
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

// One wave per workgroup: matrix-core (k part, tile, row group) items, then decode
// units.  SELF: the launch also builds the routing (route_wave in workgroup 0;
// workgroups 1-7 are idle, so the others keep their XCD numbering), and the units
// take their segments and tiles from the batch's ids (BatchKeys, BatchTiles) instead
// of the routing outputs being written meanwhile.  T is the type of x, TW of the
// weights (T, or FP8 with bf16 x).
// Two waves per SIMD: asked of the compiler (which then keeps the matrix-core
// accumulators in ordinary vector registers, 223 registers for the routing variant
// instead of 240 + 24 accumulation registers, which allowed only one wave per SIMD)
template <typename T, typename TW, bool SELF>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void shrink_kernel(PoolView P, RouteView R, const T* __restrict__ x,
                                                    int ldx, UView U, Plan plan, int n_mfma_blocks, SelfRoute sr) {
  int b = blockIdx.x;
  if constexpr (SELF) {
    __shared__ __align__(16) int sh[route_wave_lds_ints(kSelfRouteQ, kSelfRouteK / 64)];
    static_assert(route_wave_lds_ints(kSelfRouteQ, kSelfRouteK / 64) >= kSelfRouteK + 2 * kSelfRouteT, "unit LDS");
    if (b < kXcds) {
      if (b == 0)
        route_wave<kSelfRouteQ, kSelfRouteK / 64>(sr.ids, R.T, 1, R.S, R.mfma_min, R.tile_m, R.max_tiles, sr.out, sh);
      return;
    }
    b -= kXcds;
    int* tok = sh + kSelfRouteK;
    if (b >= n_mfma_blocks) {
      const int d = xcd_logical_block(b - n_mfma_blocks, plan.xcd_group);
      if (d < plan.n_dec_blocks) shrink_decode_unit_self<T, TW>(P, R, sr.ids, x, ldx, U, plan, d, tok);
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
        K.load(sr.ids, R.T, R.S);
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

template <typename T, typename TW>
static void launch_shrink_t(const PoolView& P, const RouteView& R, const T* x, int ldx, const UView& U,
                            const Plan& plan, const SelfRoute* sr, hipStream_t stream, const KTimer& tm) {
  const int nm = plan.use_mfma ? mfma_blocks(plan.tile_slots * plan.nrg * plan.nsplit) : 0;
  const int q = kXcds * plan.xcd_group;
  const int blocks = nm + (plan.n_dec_blocks + q - 1) / q * q;
  if (sr)
    RAX_LAUNCH(tm, (shrink_kernel<T, TW, true>), dim3(kXcds + blocks), dim3(64), 0u, stream, P, R, x, ldx, U, plan, nm,
               *sr);
  else
    RAX_LAUNCH(tm, (shrink_kernel<T, TW, false>), dim3(blocks), dim3(64), 0u, stream, P, R, x, ldx, U, plan, nm,
               SelfRoute{});
}

hipError_t launch_shrink(int wdtype, const PoolView& P, const RouteView& R, const void* x, int ldx,
                         const UView& U, const Plan& plan, const SelfRoute* sr, hipStream_t stream,
                         const KTimer& tm) {
  const int cw = 64 * (wdtype == LORA_F32 ? 4 : 8);   // x is bf16 for FP8 pools
  const int chunks = (P.k + cw - 1) / cw;
  if (plan.xcd_group < 1 || U.by_token || U.nsplit != plan.nsplit || plan.nsplit < 1 || plan.nsplit > kMaxSplit || plan.ns < 1 ||
      plan.nsplit * plan.ns < chunks || plan.ntg < 1 || plan.nrb * kShrinkRows < P.N * P.Rmax ||
      plan.n_dec_blocks != P.S * plan.nrb * plan.nsplit * plan.ntg ||
      (plan.use_mfma && (wdtype == LORA_F32 || plan.tile_slots < 1 || plan.nrg * 64 < P.N * P.Rmax)) ||
      (sr && (!sr->ids || R.T < 1 || R.T > kSelfRouteT || R.S + 1 > kSelfRouteK)))
    return hipErrorInvalidValue;
  if (wdtype == LORA_BF16)
    launch_shrink_t<uint16_t, uint16_t>(P, R, static_cast<const uint16_t*>(x), ldx, U, plan, sr, stream, tm);
  else if (wdtype == LORA_FP8E4M3)
    launch_shrink_t<uint16_t, uint8_t>(P, R, static_cast<const uint16_t*>(x), ldx, U, plan, sr, stream, tm);
  else
    launch_shrink_t<float, float>(P, R, static_cast<const float*>(x), ldx, U, plan, sr, stream, tm);
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

// ------------------------------------------------------------ decode expand
// LDS floats per wave for the decode expand: the rank padded to 16, times 4 tokens
__host__ __device__ constexpr int expand_usm_floats(int Rmax) { return kExpandTok * ((Rmax + 15) / 16 * 16); }

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
      base[qv] = U.p + n * U.n_stride + (long long)(row0 + (ok[qv] ? i : 0)) * U.row_stride + (ok[qv] ? j : 0);
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
    const int4 tq = tt == tt0 ? tq0 : segment_tokens(R, s, tt, p0, L);
    for (int idx = lane; idx < kExpandTok * rp; idx += 64) {
      const int j = idx >> 2, i = idx & 3;
      const bool ok = i < nt && j < r;
      const int ic = ok ? i : 0, jc = ok ? j : 0;
      const long long row = U.by_token ? (long long)R.sorted[p0 + tt + ic] : (long long)(p0 + tt + ic);
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

template <typename TW, typename TY, int QV>
__device__ __forceinline__ void expand_decode_item(const PoolView& P, const RouteView& R, const UView& U,
                                                   TY* __restrict__ y, int ldy, const Plan& plan,
                                                   int item, float* __restrict__ usm) {
  // token-tile siblings (same slot and columns, same rows of B^T) are neighbours
  const int tg = item % plan.ntg;
  const int rest = item / plan.ntg;
  const int ct = rest % P.n_ctiles, si = rest / P.n_ctiles;
  const int s = P.ordered ? (int)P.slot_order[si] : si;   // high-rank slots first
  // first round trip: record header, token ids of the first tile, slot-table entry
  const int tt0 = tg * kExpandTok;
  const int4 hdr = *reinterpret_cast<const int4*>(R.rec + (size_t)s * kRecInts);
  int4 tq0 = tt0 + 4 <= kRecTokens ? *reinterpret_cast<const int4*>(R.rec + (size_t)s * kRecInts + 4 + tt0)
                                   : make_int4(0, 0, 0, 0);
  const SlotEntry e = P.table[s];
  const int L = hdr.x, p0 = hdr.y;
  if (tt0 >= L) return;
  if (plan.use_mfma && L >= R.mfma_min) return;
  if (e.rank == 0 || e.scale == 0.f) return;
  if (tt0 + 4 > kRecTokens) tq0 = segment_tokens(R, s, tt0, p0, L);
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

template <typename TW, typename TY, int KSM>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(ExpandWaves<TW, TY, KSM>::value))) void expand_kernel(PoolView P, RouteView R, UView U,
                                                    TY* __restrict__ y, int ldy, Plan plan, int n_mfma_blocks) {
  extern __shared__ float smem[];
  const int b = blockIdx.x;
  if (b >= n_mfma_blocks) {
    const int d = xcd_logical_block(b - n_mfma_blocks, plan.xcd_group);
    // values per lane of the first tile's early partial loads: the padded rank over 16
    if (d < plan.n_dec_blocks) expand_decode_item<TW, TY, (KSM <= 2 ? 2 * KSM : 0)>(P, R, U, y, ldy, plan, d, smem);
    return;
  }
  if constexpr (sizeof(TW) <= 2) {   // bf16 and FP8 weights
    LaneTable lt;
    lt.load(P);   // in flight with the tile count
    for (MfmaItems it(b, n_mfma_blocks, R.meta[kMetaTiles] * plan.n_mgroups); it.j < it.end; it.j += it.step) {
      const int tile = it.j / plan.n_mgroups, g = it.j - tile * plan.n_mgroups;
      expand_mfma_unit<TW, TY, KSM>(P, R, U, y, ldy, tile, g, plan.cb, lt, smem);
    }
  }
}

template <typename TW, typename TY>
static void launch_expand_w(int ksm, dim3 grid, uint32_t lds, hipStream_t stream, const PoolView& P,
                            const RouteView& R, const UView& U, TY* y, int ldy, const Plan& plan, int nm,
                            const KTimer& tm) {
  switch (ksm) {
    case 1: RAX_LAUNCH(tm, (expand_kernel<TW, TY, 1>), grid, dim3(64), lds, stream, P, R, U, y, ldy, plan, nm); break;
    case 2: RAX_LAUNCH(tm, (expand_kernel<TW, TY, 2>), grid, dim3(64), lds, stream, P, R, U, y, ldy, plan, nm); break;
    case 4: RAX_LAUNCH(tm, (expand_kernel<TW, TY, 4>), grid, dim3(64), lds, stream, P, R, U, y, ldy, plan, nm); break;
    default: RAX_LAUNCH(tm, (expand_kernel<TW, TY, 8>), grid, dim3(64), lds, stream, P, R, U, y, ldy, plan, nm); break;
  }
}

size_t expand_smem_bytes(int wdtype, int Rmax, int use_mfma) {
  size_t f = (size_t)expand_usm_floats(Rmax);
  if (use_mfma && wdtype != LORA_F32 && (size_t)kExpandMfmaWaveFloats > f) f = kExpandMfmaWaveFloats;
  return f * sizeof(float);
}

hipError_t launch_expand(int wdtype, int ydtype, const PoolView& P, const RouteView& R,
                         const UView& U, void* y, int ldy, const Plan& plan, hipStream_t stream,
                         const KTimer& tm) {
  if (plan.xcd_group < 1 || plan.ntg < 1 || U.nsplit < 1 || U.nsplit > kMaxSplit || (U.by_token && U.nsplit != 1) ||
      (!U.by_token && (U.row_stride % 4 != 0 || U.row_stride < P.Rk)) ||
      plan.n_dec_blocks != P.n_ctiles * P.S * plan.ntg ||
      (plan.use_mfma && (wdtype == LORA_F32 || plan.tile_slots < 1 || plan.n_mgroups < 1 ||
                         (plan.cb != 1 && plan.cb != kMfmaColBlocksPerUnit))))
    return hipErrorInvalidValue;
  const int nm = plan.use_mfma ? mfma_blocks(plan.n_mgroups * plan.tile_slots) : 0;
  const int q = kXcds * plan.xcd_group;
  const dim3 grid(nm + (plan.n_dec_blocks + q - 1) / q * q);
  const uint32_t lds = (uint32_t)expand_smem_bytes(wdtype, P.Rmax, plan.use_mfma);
  // rank steps of 32 the matrix-core part keeps in registers: Rk / 32 rounded up to a power of 2
  const int ksm = P.Rk <= 32 ? 1 : P.Rk <= 64 ? 2 : P.Rk <= 128 ? 4 : 8;
  if (wdtype == LORA_BF16) {
    if (ydtype == LORA_BF16)
      launch_expand_w<uint16_t, uint16_t>(ksm, grid, lds, stream, P, R, U, static_cast<uint16_t*>(y), ldy, plan, nm, tm);
    else
      launch_expand_w<uint16_t, float>(ksm, grid, lds, stream, P, R, U, static_cast<float*>(y), ldy, plan, nm, tm);
  } else if (wdtype == LORA_FP8E4M3) {
    if (ydtype == LORA_BF16)
      launch_expand_w<uint8_t, uint16_t>(ksm, grid, lds, stream, P, R, U, static_cast<uint16_t*>(y), ldy, plan, nm, tm);
    else
      launch_expand_w<uint8_t, float>(ksm, grid, lds, stream, P, R, U, static_cast<float*>(y), ldy, plan, nm, tm);
  } else {
    RAX_LAUNCH(tm, (expand_kernel<float, float, 1>), grid, dim3(64), lds, stream, P, R, U,
               static_cast<float*>(y), ldy, plan, nm);
  }
  return hipGetLastError();
}

}  // namespace rax
