// Building blocks of the short-segment (decode) path of the shrink and expand
// kernels (device code).
//
// Shrink block: 16 flattened (slice, rank) rows of A against the 4 token rows of a
// tile over one k split.  Lane l owns the 16-byte chunks at k offsets
// (s + nsplit * m) * 64 * E + l * E (E = 8 bf16 or 4 fp32), so every row of A
// streams as contiguous 1 KB requests and each lane loads exactly the k-slice of
// the x rows it multiplies.  The 16 x 4 = 64 lane partial sums are finished by one
// reduce-scatter across the wave, after which lane l holds output (row l / 4,
// token l % 4) for split s.  Splits are added in split order by their single
// reader, so results do not depend on timing.
//
// Expand tile: a 512-column tile of one slice (lanes own 8 consecutive columns, so
// each rank-major row of B^T streams as one contiguous 1 KB request) for 4 tokens.
// The tile's rank-space values come from LDS, token-fastest (one 16-byte read gives
// rank j for all 4 tokens), and the contraction over the rank stays in registers,
// rows of B^T consumed four at a time behind scheduling fences to bound live
// ranges.  y gets one rounding from y + s * acc in fp32, at the token's own row.
#pragma once

#include "device_util.h"

namespace rax {

constexpr int kShrinkRows = 16;   // rank rows per decode shrink block
constexpr int kShrinkTok = 4;     // tokens per decode tile
constexpr int kExpandTok = 4;
// LDS floats per wave for the decode expand: the rank padded to 16, times 4 tokens
__host__ __device__ constexpr int expand_usm_floats(int Rmax) { return kExpandTok * ((Rmax + 15) / 16 * 16); }

// Token ids at positions tt .. tt + 3 of slot s's segment: from the slot's routing
// record when they are among its first kRecTokens (the record repeats the segment's
// first token past its end), else from sorted_ids (position clamped into the
// segment).  Entries at or past the segment's end name a valid row of the batch but
// are not a token of the tile: callers read them and do not store them.
__device__ __forceinline__ int4 segment_tokens(const RouteView& R, int s, int tt, int p0, int L) {
  if (tt + 4 <= kRecTokens) return *reinterpret_cast<const int4*>(R.rec + (size_t)s * kRecInts + 4 + tt);
  const int last = p0 + L - 1;
  return make_int4(R.sorted[min(p0 + tt, last)], R.sorted[min(p0 + tt + 1, last)], R.sorted[min(p0 + tt + 2, last)],
                   R.sorted[min(p0 + tt + 3, last)]);
}

// a token quad's ids checked against the batch's T (statement; nothing outside debug builds)
#ifdef RAXLORA_DEBUG
#define RAX_CHECK_TOKENS(q, T) \
  ((q) = make_int4(RAX_IDX((q).x, (T)), RAX_IDX((q).y, (T)), RAX_IDX((q).z, (T)), RAX_IDX((q).w, (T))))
#else
#define RAX_CHECK_TOKENS(q, T) ((void)0)
#endif

// element i (a compile-time constant after unrolling) of a token quad
__device__ __forceinline__ int tok_at(const int4& v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }

// ---------------------------------------------------------------- shrink block
// Row pointers of the 16-row block starting at flattened row fb of slot s (rank r).
template <typename T>
struct ShrinkRows {
  const T* arow[kShrinkRows];
  bool rval[kShrinkRows];
  __device__ __forceinline__ ShrinkRows(const PoolView& P, int s, int r, int fb) {
    const T* __restrict__ Aslot = static_cast<const T*>(P.A) + (size_t)s * P.N * P.Rmax * P.k;
    const int F = P.N * r;
    int n = fb / r, j = fb - (fb / r) * r;
#pragma unroll
    for (int rr = 0; rr < kShrinkRows; ++rr) {
      rval[rr] = fb + rr < F;
      arow[rr] = Aslot + ((size_t)(rval[rr] ? n : 0) * P.Rmax + (rval[rr] ? j : 0)) * P.k;
      if (++j == r) { j = 0; ++n; }
    }
  }
};

// Partial sums of split sp (chunk steps sp + nsplit * m, m < ns) for the block's 16
// rows and the tile's 4 token rows; tokens at or past nt contribute zero.  Returns
// this lane's value after the reduce-scatter: row fb + lane / 4, token lane % 4.
// TX is the x type, TW the weight type (TW = TX, or FP8 weights with bf16 x, whose
// chunks are first put on the e4m3 grid).
template <typename TX, typename TW>
__device__ __forceinline__ float shrink_block_partial(const PoolView& P, const ShrinkRows<TW>& A,
                                                      const TX* const (&xrow)[kShrinkTok], int nt, int sp,
                                                      int nsplit, int ns) {
  constexpr int E = Elem<TX>::kPerChunk;
  constexpr int CW = 64 * E;         // k elements of one wave-wide chunk step
  static_assert(Elem<TW>::kPerChunk == E, "weight and x chunks cover the same k range");
  using AC = WChunk<TW>;
  const int lane = lane_id();
  float acc[64];
#pragma unroll
  for (int m = 0; m < 64; ++m) acc[m] = 0.f;
  for (int c = 0; c < ns; ++c) {
    const int col = (sp + nsplit * c) * CW + lane * E;
    const bool inb = col < P.k;
    const int colc = min(col, P.k - E);
    // the x chunks and all 16 A rows of this chunk step in flight before the first product
    uint4 xv[kShrinkTok];
    typename AC::type av[kShrinkRows];
#pragma unroll
    for (int i = 0; i < kShrinkTok; ++i) xv[i] = ld16(xrow[i] + colc);
#pragma unroll
    for (int rr = 0; rr < kShrinkRows; ++rr) av[rr] = AC::load(A.arow[rr] + colc);
    sched_fence();
#pragma unroll
    for (int i = 0; i < kShrinkTok; ++i) {
      if constexpr (sizeof(TW) == 1) xv[i] = bf16x8_to_fp8_grid(xv[i]);
      xv[i] = keep_if(xv[i], i < nt && inb);
    }
#pragma unroll
    for (int rr = 0; rr < kShrinkRows; ++rr) {
      const uint4 a = AC::widen(AC::keep(av[rr], A.rval[rr]));
#pragma unroll
      for (int i = 0; i < kShrinkTok; ++i)
        acc[rr * kShrinkTok + i] = chunk_dot(a, xv[i], acc[rr * kShrinkTok + i], TX());
    }
  }
  reduce_scatter64(acc);
  return acc[0];
}

// ---------------------------------------------------------------- expand tile
// 8 consecutive elements of a row, kept packed: one 16-byte chunk for bf16, two for fp32
template <typename T> struct Row8;
template <> struct Row8<uint16_t> {
  uint4 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = ld16(p); }
  __device__ __forceinline__ void keep(bool ok) { w = keep_if(w, ok); }
  __device__ __forceinline__ void get(float (&v)[8]) const { unpack8(w, v); }
};
template <> struct Row8<float> {
  uint4 a, b;
  __device__ __forceinline__ void load(const float* p) { a = ld16(p); b = ld16(p + 4); }
  __device__ __forceinline__ void keep(bool ok) { a = keep_if(a, ok); b = keep_if(b, ok); }
  __device__ __forceinline__ void get(float (&v)[8]) const {
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  }
};

template <> struct Row8<uint8_t> {   // FP8 pools: 8 bytes, widened at use
  uint2 w;
  __device__ __forceinline__ void load(const uint8_t* p) { w = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void keep(bool ok) {
    const uint32_t m = ok ? 0xffffffffu : 0u;
    w = make_uint2(w.x & m, w.y & m);
  }
  __device__ __forceinline__ void get(float (&v)[8]) const { fp8x8_to_f32(w, v); }
};

// rank rows of B^T per load batch: 16 for bf16 and FP8 pools (64 or 32 registers), 8 for fp32
template <typename TW> struct ExpandRows { static constexpr int kBatch = sizeof(TW) <= 2 ? 16 : 8; };

// One expand tile in two halves, so a caller can put other work between issuing the
// loads and using them: issue() loads the first RB rows of B^T and the 4 token rows
// of y; finish() contracts with the rank-space values u4[j] (rank j, 4 tokens;
// zero past the rank and for tokens past nt) and stores rows i < nt.
template <typename TW, typename TY>
struct ExpandTile {
  static constexpr int RB = ExpandRows<TW>::kBatch;
  static constexpr int LT = kExpandTok;
  Row8<TW> b[RB];
  Row8<TY> yv[LT];
  TY* yrow[LT];
  const TW* bt;
  bool inb;

  // bt_slot: B^T of the slot at column o_n (row stride D); columns [c0, c0 + 512) of slice n
  __device__ __forceinline__ void issue(const PoolView& P, const TW* __restrict__ bt_slot, TY* __restrict__ y, int ldy,
                                        int n, int c0, int r, const int4& tq) {
    const int lane = lane_id(), dn = P.d[n];
    const int col = c0 + lane * kColsPerLane;
    inb = col < dn;
    const int colc = min(col, dn - kColsPerLane);
    bt = bt_slot + colc;
#pragma unroll
    for (int jj = 0; jj < RB; ++jj) b[jj].load(bt + (size_t)(jj < r ? jj : 0) * P.D);
#pragma unroll
    for (int i = 0; i < LT; ++i) {
      yrow[i] = y + (size_t)tok_at(tq, i) * ldy + P.o[n] + colc;
      yv[i].load(yrow[i]);
    }
  }

  __device__ __forceinline__ void finish(const PoolView& P, int r, int nt, float scale,
                                         const float4* __restrict__ u4) {
    const int rp = (r + RB - 1) / RB * RB;
    float acc[LT][kColsPerLane];
#pragma unroll
    for (int i = 0; i < LT; ++i)
#pragma unroll
      for (int c = 0; c < kColsPerLane; ++c) acc[i][c] = 0.f;
    // rows [jb, jb + RB) of B^T against the rank-space values
    auto contract = [&](int jb) {
#pragma unroll
      for (int j4 = 0; j4 < RB; j4 += 4) {
#pragma unroll
        for (int jj = j4; jj < j4 + 4; ++jj) {
          b[jj].keep(jb + jj < r);
          float bf[kColsPerLane];
          b[jj].get(bf);
          const float4 uq = u4[jb + jj];
          const float uv[LT] = {uq.x, uq.y, uq.z, uq.w};
#pragma unroll
          for (int i = 0; i < LT; ++i)
#pragma unroll
            for (int c = 0; c < kColsPerLane; ++c) acc[i][c] = fmaf(bf[c], uv[i], acc[i][c]);
        }
        sched_fence();
      }
    };
    sched_fence();
    contract(0);
    // ranks above RB: further batches of rows, each loaded after the previous is used
    for (int jb = RB; jb < rp; jb += RB) {
#pragma unroll
      for (int jj = 0; jj < RB; ++jj) b[jj].load(bt + (size_t)(jb + jj < r ? jb + jj : 0) * P.D);
      sched_fence();
      contract(jb);
    }
    if (inb) {
#pragma unroll
      for (int i = 0; i < LT; ++i) {
        if (i < nt) {
          float v[kColsPerLane];
          yv[i].get(v);
#pragma unroll
          for (int c = 0; c < kColsPerLane; ++c) v[c] = v[c] + scale * acc[i][c];
          store8f(yrow[i], v);
        }
      }
    }
  }
};

}  // namespace rax
