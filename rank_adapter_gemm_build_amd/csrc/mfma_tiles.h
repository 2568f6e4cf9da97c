// Matrix-core (MFMA) units for long same-slot segments (device code, included by linear.hip).
//
// Page "第16章 LoRA 适配器热切换", §16.4.3: in prefill a segment holds all tokens of the
// requests on one adapter, so it is long, and the per-segment shrink [L, k] x [k, r]
// and expand [L, r] x [r, d] are real matrix products.  Page "TensorRT-LLM 源码完全拆解
// (二十一)", section "前向替换": prefill batches take a grouped-GEMM path of their own.
// Here the routing cuts those segments into tiles of up to 16 tokens, and both
// products run on the gfx950 bf16 matrix cores (v_mfma_f32_16x16x32_bf16, fp32
// accumulation).  Fragment layouts of the 16x16x32 instruction: lane l supplies row
// l % 16 and the 8 consecutive k values 8 * (l / 16) .. +7 of each operand, and
// receives rows 4 * (l / 16) .. +3 of column l % 16 of the result.
//
// Every unit is one wave (a workgroup of 64 threads), so a launch spreads over all
// compute units: one workgroup streams only a few tens of GB/s, so bandwidth comes
// from having units on every CU, not from wide workgroups.
//
// Shrink unit (tile, row group, k part): D[token][f] = sum_c x[token][c] * A[f][c]
// for the tile's 16 tokens, up to 64 flattened (slice, rank) rows f and the k part's
// contiguous range of k; the wave writes the part's partial sums, which the expand
// adds in part order (as for the short segments), so a tile's k is spread over
// nsplit waves.  Operand rows are k-contiguous in both x and the pool's A, so each
// lane loads its 8 bf16 of a fragment with one 16-byte load; x rows are gathered
// through sorted_ids.  The k steps run in groups of kMfmaGroup whose fragments load
// together, double-buffered: the loads of group g + 1 are in flight while the
// products of group g run.
//
// Expand unit (tile, group of up to kMfmaColBlocksPerUnit 128-column blocks of one
// slice): D[token][col] = sum_j u[token][j] * B[col][j], from the pool's
// rank-contiguous copy of B (stride: the slot's rank rounded up to 8, so a low-rank
// slot of a mixed-rank pool reads no padding).  The wave finishes its tokens'
// rank-space values (partials added in split order) and keeps them as bf16 hi + lo
// parts (hi = bf16(u), lo = bf16(u - hi)), two products per step, so u keeps about 16
// mantissa bits instead of being rounded to bf16.  Per column block the B fragments
// and the tile's y chunks load in one batch, issued one block ahead of the products,
// and the 16 x 128 result goes through the wave's own LDS slice so that the
// read-modify-write of y (the dominant traffic) moves 16 bytes per lane along rows.
#pragma once

#include "device_util.h"

namespace rax {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ long as_i64(uint2 v) { return __builtin_bit_cast(long, v); }

constexpr int kMfmaGroup = 4;                    // shrink k-steps whose fragments load together
constexpr int kDsPitch = kMfmaCols + 4;          // LDS row pitch (floats) of the expand result tile
constexpr int kExpandMfmaWaveFloats = kMfmaTileM * kDsPitch;   // LDS floats per expand wave

// ------------------------------------------------------------------ shrink
// TW: weight type (bf16, or FP8 widened to bf16 at use; x is bf16 for both)
template <typename TW, int NB>
struct ShrinkFrags {
  uint4 xa[kMfmaGroup];
  typename WChunk<TW>::type wb[kMfmaGroup][NB];
};

// Loads of one group: raw values only, so that nothing consumes them before the
// products (a consumer in the load phase would make the wave wait for the group
// right after issuing it, defeating the double buffering).  Steps past the part's
// end reload its last step (a cache hit); the products zero them.
template <typename TW, int NB>
__device__ __forceinline__ void shrink_load_group(ShrinkFrags<TW, NB>& f, const uint16_t* __restrict__ xrow,
                                                  const TW* const (&arow)[NB], int sg, int last, int k, int lk) {
#pragma unroll
  for (int g = 0; g < kMfmaGroup; ++g) {
    const int st = min(sg + g, last);
    const int colc = min(st * kMfmaK + 8 * lk, k - 8);
    f.xa[g] = ld16(xrow + colc);
#pragma unroll
    for (int b = 0; b < NB; ++b) f.wb[g][b] = WChunk<TW>::load(arow[b] + colc);
  }
}

// Products of one group; fragments of steps outside [sg, s1), of rows past the last
// valid one and of tokens past the tile's length are zeroed here.  FP8 pools run on the
// FP8 matrix cores (v_mfma_f32_16x16x32_fp8_fp8: the same 16x16x32 shape and lane
// layout, 8 e4m3 bytes per lane and operand): the weights go in as stored and the
// activations are converted once, to e4m3 bytes (clamped, rounded to nearest even);
// the products of two e4m3 values are exact and accumulate in fp32.
template <typename TW, int NB>
__device__ __forceinline__ void shrink_mma_group(const ShrinkFrags<TW, NB>& f, bool tval, const bool (&rval)[NB],
                                                 int sg, int s1, int k, int lk, f32x4_t (&acc)[NB]) {
  using W = WChunk<TW>;
#pragma unroll
  for (int g = 0; g < kMfmaGroup; ++g) {
    const bool inb = sg + g < s1 && (sg + g) * kMfmaK + 8 * lk < k;  // k % 8 == 0: chunks wholly in or out
    if constexpr (sizeof(TW) == 1) {
      const uint2 xq = W::keep(bf16x8_to_fp8x8(f.xa[g]), tval && inb);
#pragma unroll
      for (int b = 0; b < NB; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(as_i64(xq), as_i64(W::keep(f.wb[g][b], rval[b])), acc[b],
                                                            0, 0, 0);
    } else {
      const uint4 xa = keep_if(f.xa[g], tval && inb);
#pragma unroll
      for (int b = 0; b < NB; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa), as_bf16x8(W::widen(W::keep(f.wb[g][b], rval[b]))),
                                                         acc[b], 0, 0, 0);
    }
  }
}

// Products of rows fr0 .. fr0 + 16 * NB of one tile over k steps [s0, s1): lane
// holds D[token 4 * lk + i][row fr0 + 16 b + lr] in acc[b][i].
template <typename TW, int NB>
__device__ __forceinline__ void shrink_mfma_acc(const PoolView& P, const uint16_t* __restrict__ xrow, int slot, int r,
                                                int len, int fr0, int s0, int s1, f32x4_t (&acc)[NB]) {
  const int lane = lane_id(), lr = lane & 15, lk = lane >> 4;
  const int F = P.N * r;
  const bool tval = lr < len;
  const TW* Aslot = static_cast<const TW*>(P.A) + (size_t)slot * P.N * P.Rmax * P.k;
  const TW* arow[NB];
  bool rval[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int f = fr0 + 16 * b + lr;
    rval[b] = f < F;
    const int fc = rval[b] ? f : 0;
    const int n = fc / r, j = fc - n * r;
    arow[b] = Aslot + ((size_t)n * P.Rmax + j) * P.k;
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int last = max(s1 - 1, 0);
  ShrinkFrags<TW, NB> f0, f1;
  shrink_load_group<TW, NB>(f0, xrow, arow, s0, last, P.k, lk);
  for (int sg = s0; sg < s1; sg += 2 * kMfmaGroup) {
    shrink_load_group<TW, NB>(f1, xrow, arow, sg + kMfmaGroup, last, P.k, lk);
    sched_fence();
    shrink_mma_group<TW, NB>(f0, tval, rval, sg, s1, P.k, lk, acc);
    sched_fence();
    shrink_load_group<TW, NB>(f0, xrow, arow, sg + 2 * kMfmaGroup, last, P.k, lk);
    sched_fence();
    shrink_mma_group<TW, NB>(f1, tval, rval, sg + kMfmaGroup, s1, P.k, lk, acc);
    sched_fence();
  }
}

// k range [s0, s1) of the steps of 32 that part `part` of nsplit takes (contiguous parts)
__device__ __forceinline__ void mfma_part_range(int k, int part, int nsplit, int& s0, int& s1) {
  const int steps = (k + kMfmaK - 1) / kMfmaK;
  const int per = (steps + nsplit - 1) / nsplit;
  s0 = min(steps, part * per);
  s1 = min(steps, s0 + per);
}

// Rows fr0 .. fr0 + 16 * NB of one tile over k steps [s0, s1); writes partial `part`.
template <typename TW, int NB>
__device__ __forceinline__ void shrink_mfma_rows(const PoolView& P, const uint16_t* __restrict__ xrow, const UView& U,
                                                 int slot, int r, int p0, int len, int fr0, int part, int s0, int s1) {
  const int lane = lane_id(), lr = lane & 15, lk = lane >> 4;
  const int F = P.N * r;
  f32x4_t acc[NB];
  shrink_mfma_acc<TW, NB>(P, xrow, slot, r, len, fr0, s0, s1, acc);
  // lane holds D[token 4 * lk + i][row fr0 + 16 b + lr]; rows by sorted position
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int fr = fr0 + 16 * b + lr;
    if (fr < F) {
      const int n = fr / r, j = fr - n * r;
      float* up = U.p + part * U.split_stride + n * U.n_stride + (long long)p0 * U.row_stride + j;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * lk + i;
        if (t < len) {
#ifdef RAXLORA_DEBUG
          if (RAX_IDX(p0 + t, U.n_stride / U.row_stride) != p0 + t) continue;
#endif
          up[t * U.row_stride] = acc[b][i];
        }
      }
    }
  }
}

// One shrink unit of the tile of `len` tokens of slot `slot` at sorted position p0
// (xrow: this lane's x row, token lane % 16, clamped into the tile), row group rg
// (rows 64 rg .. 64 rg + 63), k part `part` of nsplit.  Wave-uniform.  Parts with no
// k steps write zeros.
template <typename TW>
__device__ __forceinline__ void shrink_mfma_tile(const PoolView& P, const SlotEntry& e,
                                                 const uint16_t* __restrict__ xrow, const UView& U, int slot, int p0,
                                                 int len, int rg, int part, int nsplit) {
  const int r = e.rank, F = P.N * r, fr0 = 64 * rg;
  if (r == 0 || fr0 >= F) return;
  int s0, s1;
  mfma_part_range(P.k, part, nsplit, s0, s1);
  const int nb = min(4, (F - fr0 + 15) / 16);
  if (nb == 4)
    shrink_mfma_rows<TW, 4>(P, xrow, U, slot, r, p0, len, fr0, part, s0, s1);
  else if (nb == 3)
    shrink_mfma_rows<TW, 3>(P, xrow, U, slot, r, p0, len, fr0, part, s0, s1);
  else if (nb == 2)
    shrink_mfma_rows<TW, 2>(P, xrow, U, slot, r, p0, len, fr0, part, s0, s1);
  else
    shrink_mfma_rows<TW, 1>(P, xrow, U, slot, r, p0, len, fr0, part, s0, s1);
}

// One shrink unit: tile `tile` of the routing's list.
template <typename TW>
__device__ __forceinline__ void shrink_mfma_unit(const PoolView& P, const RouteView& R, const uint16_t* __restrict__ x,
                                                 int ldx, const UView& U, int tile, int rg, int part, int nsplit) {
  const int4 td = R.tiles[tile];
  int slot = td.x, p0 = td.y;
  const int len = td.z;
  RAX_CHECK_VAR(slot, P.S);
  RAX_CHECK_VAR(p0, R.T - len + 1);
  // the slot-table entry and this lane's token id (token lane % 16) in one round trip
  const SlotEntry e = P.table[slot];
  int tok = R.sorted[p0 + min(lane_id() & 15, len - 1)];
  RAX_CHECK_VAR(tok, R.T);
  const uint16_t* __restrict__ xrow = x + (size_t)tok * ldx;
  shrink_mfma_tile<TW>(P, e, xrow, U, slot, p0, len, rg, part, nsplit);
}

// ------------------------------------------------------------------ expand
// 8 fp32 values as the bf16 pair hi = bf16(v), lo = bf16(v - hi), packed as MFMA operands
__device__ __forceinline__ void u_hilo(const float (&v)[8], uint4& uh, uint4& ul) {
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t h0 = f32_to_bf16(v[2 * q]), h1 = f32_to_bf16(v[2 * q + 1]);
    hi[q] = h0 | (h1 << 16);
    lo[q] = f32_to_bf16(v[2 * q] - __uint_as_float(h0 << 16)) | (f32_to_bf16(v[2 * q + 1] - __uint_as_float(h1 << 16)) << 16);
  }
  uh = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  ul = make_uint4(lo[0], lo[1], lo[2], lo[3]);
}

constexpr int kUSplitBatch = 8;   // split partials of one u fragment loaded in one batch

// This lane's u fragment of rank step ks (token lr, ranks 32 ks + 8 lk .. +7), from
// the split partials of the workspace, NSB batches of kUSplitBatch splits (NSB *
// kUSplitBatch >= nsplit): load() issues the first batch, finish() issues any
// further one and adds all of them in split order.  Branch-free: a lane whose ranks
// lie past the rank, or whose token lies past the tile, reads a clamped address of
// the same row (a duplicate the memory pipeline merges); splits past nsplit re-read
// the last one and are added as -0.0f, the exact identity of IEEE addition; values
// of ranks past the rank and of tokens past the tile are zeroed at the end.
template <int NSB>
struct UPartials {
  float4 pa[kUSplitBatch], pb[kUSplitBatch];
  const float* base;
  __device__ __forceinline__ void load_batch(const UView& U, int q0) {
#pragma unroll
    for (int q = 0; q < kUSplitBatch; ++q) {
      const long long off = (long long)min(q0 + q, U.nsplit - 1) * U.split_stride;
      pa[q] = *reinterpret_cast<const float4*>(base + off);
      pb[q] = *reinterpret_cast<const float4*>(base + off + 4);
    }
  }
  __device__ __forceinline__ void load(const UView& U, int n, int p0, int len, int r, int ks) {
    const int lane = lane_id(), lr = lane & 15, lk = lane >> 4;
    const int j0 = ks * kMfmaK + 8 * lk;
    // j0 < r: j0 + 8 <= r rounded up to 8 <= row_stride, so the 8 floats stay in the row
    int row = p0 + min(lr, len - 1);
    RAX_CHECK_VAR(row, U.n_stride / U.row_stride);
    base = U.p + n * U.n_stride + (long long)row * U.row_stride + (j0 < r ? j0 : 0);
    load_batch(U, 0);
  }
  // rank step 0 of row `row` (slot mode's first-tile rows, known before the segment
  // is: the token and rank are masked in finish())
  __device__ __forceinline__ void load_head(const UView& U, int n, long long row) {
    const int j0 = 8 * (lane_id() >> 4);
    RAX_CHECK_VAR(row, U.n_stride / U.row_stride);
    base = U.p + n * U.n_stride + row * U.row_stride + (j0 + 8 <= U.row_stride ? j0 : 0);
    load_batch(U, 0);
  }
  __device__ __forceinline__ void add_batch(const UView& U, int q0, float (&v)[8]) const {
#pragma unroll
    for (int q = 0; q < kUSplitBatch; ++q) {
      if (q0 + q == 0) {
        v[0] = pa[0].x; v[1] = pa[0].y; v[2] = pa[0].z; v[3] = pa[0].w;
        v[4] = pb[0].x; v[5] = pb[0].y; v[6] = pb[0].z; v[7] = pb[0].w;
      } else {
        const bool in = q0 + q < U.nsplit;
        v[0] += in ? pa[q].x : -0.f; v[1] += in ? pa[q].y : -0.f; v[2] += in ? pa[q].z : -0.f;
        v[3] += in ? pa[q].w : -0.f; v[4] += in ? pb[q].x : -0.f; v[5] += in ? pb[q].y : -0.f;
        v[6] += in ? pb[q].z : -0.f; v[7] += in ? pb[q].w : -0.f;
      }
    }
  }
  __device__ __forceinline__ void finish(const UView& U, int len, int r, int ks, uint4& uh, uint4& ul) {
    const int lane = lane_id(), lr = lane & 15, lk = lane >> 4;
    float v[8];
    add_batch(U, 0, v);
#pragma unroll
    for (int b = 1; b < NSB; ++b) {
      sched_fence();   // one batch of partials in registers at a time
      load_batch(U, b * kUSplitBatch);
      add_batch(U, b * kUSplitBatch, v);
    }
    const int j0 = ks * kMfmaK + 8 * lk;
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = (lr < len && j0 + q < r) ? v[q] : 0.f;
    u_hilo(v, uh, ul);
  }
};

// The object a body with NSB batches loads its first rank step into: the caller's
// one-batch object when NSB == 1, else its own.
template <int NSB> struct UPartialsPick {
  __device__ __forceinline__ static UPartials<NSB>& get(UPartials<NSB>& own, UPartials<1>&) { return own; }
};
template <> struct UPartialsPick<1> {
  __device__ __forceinline__ static UPartials<1>& get(UPartials<1>&, UPartials<1>& ext) { return ext; }
};

// The same fragment from the caller's finished u (rows by token, row stride Rmax),
// branch-free like UPartials (rank clamped into the row, zeroed after).
__device__ __forceinline__ void u_frag_by_token(const RouteView& R, const UView& U, int n, int p0, int len, int r,
                                                int ks, uint4& uh, uint4& ul) {
  const int lane = lane_id(), lr = lane & 15, lk = lane >> 4;
  const int j0 = ks * kMfmaK + 8 * lk;
  int tok = R.sorted[p0 + min(lr, len - 1)];
  RAX_CHECK_VAR(tok, R.T);
  const float* base = U.p + n * U.n_stride + (long long)tok * U.row_stride;
  float v[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) v[q] = base[min(j0 + q, r - 1)];
#pragma unroll
  for (int q = 0; q < 8; ++q) v[q] = (lr < len && j0 + q < r) ? v[q] : 0.f;
  u_hilo(v, uh, ul);
}

// Column groups of the matrix-core expand: each slice's 128-column blocks in groups
// of cb; a group never spans two slices.  Returns the slice (or -1 past the last
// group) and the group's first block within the slice.
__device__ __forceinline__ int mfma_group_slice(const PoolView& P, int grp, int cb, int& blk0) {
  int g0 = 0;
  for (int n = 0; n < P.N; ++n) {
    const int nbn = P.mblk0[n + 1] - P.mblk0[n];
    const int gn = (nbn + cb - 1) / cb;
    if (grp < g0 + gn) {
      blk0 = (grp - g0) * cb;
      return n;
    }
    g0 += gn;
  }
  return -1;
}

// Per-lane y rows of a matrix-core expand tile for blocks of BC columns: chunk q of a
// lane belongs to token (64 q + lane) / RC of the tile (clamped to the tile), whose
// row of y starts at row[q] (slice offset included).  Set once per unit.
template <typename TY, int BC>
struct ExpandRows16 {
  static constexpr int YC = 16 / (int)sizeof(TY);                // y elements per 16-byte chunk
  static constexpr int RC = BC / YC;                             // chunks per token row of a block
  static constexpr int YCH = kMfmaTileM * RC / 64;               // y chunks per lane
  TY* row[YCH];
  // tok: this lane's token id of the tile (token lane % 16, clamped to the tile)
  __device__ __forceinline__ void load(int tok, TY* __restrict__ y, int ldy, int on) {
    const int lane = lane_id();
#pragma unroll
    for (int q = 0; q < YCH; ++q) {
      const int t = (q * 64 + lane) / RC;
      row[q] = y + (size_t)__shfl(tok, t) * ldy + on;
    }
  }
};

// Loads of one block of BC columns (BC / 16 column strips of 16) of one tile, all
// unconditional: the tile's y chunks (a lane past the tile re-reads its clamped
// token's chunk, never stored; columns past the slice re-read its last chunk, never
// stored) and the B fragments of the NKS rank steps (a lane whose ranks lie past the
// slot's Bk stride reads the rank-0 fragment of its column and zeroes it; columns
// past the slice read column 0, never stored).
template <typename TW, typename TY, int NKS, int BC>
struct ExpandMfmaBlock {
  using Rows = ExpandRows16<TY, BC>;
  using W = WChunk<TW>;
  static constexpr int YC = Rows::YC, RC = Rows::RC, YCH = Rows::YCH;
  static constexpr int NCB = BC / 16;                            // 16-column strips
  // 16-byte chunks per lane (FP8 B fragments are 8 bytes)
  static constexpr int kRegs = YCH + NCB * NKS * (int)sizeof(typename W::type) / 16;
  uint4 yv[YCH];
  typename W::type bv[NKS][NCB];
  int c0;

  __device__ __forceinline__ void issue(const Rows& Y, const TW* __restrict__ bk, int rs, int dn, int c0_,
                                        int nks) {
    issue_y(Y, dn, c0_);
    issue_b(bk, rs, dn, c0_, nks);
  }
  // the two halves, for a first block whose B can go out before the tile's token ids
  // (and so its y rows) are known
  __device__ __forceinline__ void issue_y(const Rows& Y, int dn, int c0_) {
    const int lane = lane_id();
    c0 = c0_;
#pragma unroll
    for (int q = 0; q < YCH; ++q) {
      const int cc = ((q * 64 + lane) % RC) * YC;
      yv[q] = ld16(Y.row[q] + min(c0 + cc, dn - YC));
    }
  }
  __device__ __forceinline__ void issue_b(const TW* __restrict__ bk, int rs, int dn, int c0_, int nks) {
    const int lane = lane_id(), lr = lane & 15, lk = lane >> 4;
    c0 = c0_;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (ks < nks) {   // compile-time true unless NKS covers a range of rank-step counts
        const int j0 = ks * kMfmaK + 8 * lk, jc = j0 < rs ? j0 : 0;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const int col = c0 + 16 * cb + lr;
          bv[ks][cb] = W::load(bk + (size_t)(col < dn ? col : 0) * rs + jc);
        }
      }
    }
  }

  // D[token][col] = sum_j u[token][j] B[col][j] for the block, then y += scale * D
  // for the tile's tokens, through the wave's LDS slice ds (16 rows of kDsPitch).
  __device__ __forceinline__ void finish(const Rows& Y, int rs, int dn, int len, int nks, float scale,
                                         const uint4 (&uh)[NKS], const uint4 (&ul)[NKS], float* __restrict__ ds) const {
    const int lane = lane_id(), lr = lane & 15, lk = lane >> 4;
    f32x4_t acc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (ks < nks) {
        const bool kin = ks * kMfmaK + 8 * lk < rs;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const uint4 b = W::widen(W::keep(bv[ks][cb], kin));
          acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(uh[ks]), as_bf16x8(b), acc[cb], 0, 0, 0);
          acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ul[ks]), as_bf16x8(b), acc[cb], 0, 0, 0);
        }
      }
    }
    // lane holds D[token 4 lk + i][column 16 cb + lr]
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) ds[(4 * lk + i) * kDsPitch + 16 * cb + lr] = acc[cb][i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int q = 0; q < YCH; ++q) {
      const int idx = q * 64 + lane;
      const int t = idx / RC, cc = (idx % RC) * YC;
      if (t < len && c0 + cc < dn) {
        TY* const yp = Y.row[q] + c0 + cc;
        const float* dp = ds + t * kDsPitch + cc;
        if constexpr (sizeof(TY) == 2) {
          float v[8];
          unpack8(yv[q], v);
#pragma unroll
          for (int c = 0; c < 8; ++c) v[c] = v[c] + scale * dp[c];
          store8f(yp, v);
        } else {
          uint4 o;
          o.x = __float_as_uint(__uint_as_float(yv[q].x) + scale * dp[0]);
          o.y = __float_as_uint(__uint_as_float(yv[q].y) + scale * dp[1]);
          o.z = __float_as_uint(__uint_as_float(yv[q].z) + scale * dp[2]);
          o.w = __float_as_uint(__uint_as_float(yv[q].w) + scale * dp[3]);
          st16(yp, o);
        }
      }
    }
    // the LDS slice is rewritten by the next block
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
};

// Block width of the expand body: 128 columns when two blocks' loads fit in 12
// chunks per lane, else 64 when they do, else 128 without overlap.
template <typename TW, typename TY, int NKS>
struct ExpandBlockWidth {
  static constexpr int value = ExpandMfmaBlock<TW, TY, NKS, 128>::kRegs <= 12  ? 128
                               : ExpandMfmaBlock<TW, TY, NKS, 64>::kRegs <= 12 ? 64
                                                                               : 128;
};

// Body of one expand unit with NKS rank steps of 32 (nks <= NKS of them real), NSB
// split batches of the workspace partials (0: the caller's finished u by token), CB
// 128-column blocks.  Order of the memory traffic: the u loads, then the first
// block's y chunks and B fragments, all in flight together; then, while a block's
// products run, the next block's loads are in flight (blocks narrowed to 64 columns
// when that is what lets two blocks' loads fit in 12 chunks per lane; one block at a
// time when even that does not fit).  A block past the slice's end loads clamped
// addresses and stores nothing.  There are no branches between a load and its use,
// so the compiler keeps the batches as written.
template <typename TW, typename TY, int NKS, int NSB, int CB>
__device__ __forceinline__ void expand_mfma_body(const RouteView& R, const UView& U, TY* __restrict__ y, int ldy,
                                                 const TW* __restrict__ bk, int rs, int n, int on, int dn,
                                                 int c00, int p0, int len, const int* __restrict__ tokp, int tokv, int r,
                                                 int nks, float scale, float* __restrict__ ds, UPartials<1>& ext,
                                                 bool ext_loaded) {
  constexpr int BC = ExpandBlockWidth<TW, TY, NKS>::value;
  constexpr int NB = CB * (kMfmaCols / BC);                     // blocks of the unit
  using Blk = ExpandMfmaBlock<TW, TY, NKS, BC>;
  constexpr bool kPipe = Blk::kRegs <= 12;
  typename Blk::Rows Y;
  uint4 uh[NKS], ul[NKS];
  Blk b0, b1;
  if constexpr (NSB > 0) {
    // this lane's token id first, then the partials and the first block's B: loads
    // complete in order, so the y rows can be addressed (and their loads issued) as
    // soon as the token id is in, while the rest is still in flight
    int tok = tokp ? *tokp : tokv;
    RAX_CHECK_VAR(tok, R.T);
    sched_fence();
    // one batch of partials: the caller's object, possibly already in flight (slot
    // mode's first tile)
    UPartials<NSB> own;
    UPartials<NSB>& up = UPartialsPick<NSB>::get(own, ext);
    if (!(NSB == 1 && ext_loaded)) up.load(U, n, p0, len, r, 0);
    b0.issue_b(bk, rs, dn, c00, nks);
    sched_fence();
    Y.load(tok, y, ldy, on);
    b0.issue_y(Y, dn, c00);
    sched_fence();
    up.finish(U, len, r, 0, uh[0], ul[0]);
#pragma unroll
    for (int ks = 1; ks < NKS; ++ks) {
      UPartials<NSB> uq;
      uq.load(U, n, p0, len, r, ks);
      uq.finish(U, len, r, ks, uh[ks], ul[ks]);
    }
  } else {
    int tok = tokp ? *tokp : tokv;
    RAX_CHECK_VAR(tok, R.T);
    Y.load(tok, y, ldy, on);
    b0.issue(Y, bk, rs, dn, c00, nks);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) u_frag_by_token(R, U, n, p0, len, r, ks, uh[ks], ul[ks]);
  }
  if constexpr (kPipe) {
#pragma unroll
    for (int i = 0; i < NB; i += 2) {
      if (i + 1 < NB) b1.issue(Y, bk, rs, dn, c00 + (i + 1) * BC, nks);
      sched_fence();
      b0.finish(Y, rs, dn, len, nks, scale, uh, ul, ds);
      if (i + 2 < NB) b0.issue(Y, bk, rs, dn, c00 + (i + 2) * BC, nks);
      sched_fence();
      if (i + 1 < NB) b1.finish(Y, rs, dn, len, nks, scale, uh, ul, ds);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (i > 0) b0.issue(Y, bk, rs, dn, c00 + i * BC, nks);
      sched_fence();
      b0.finish(Y, rs, dn, len, nks, scale, uh, ul, ds);
    }
  }
}

// One expand unit: tile `tile`, column group grp (cb blocks of one slice, cb = 1 or
// kMfmaColBlocksPerUnit).  KSM is the number of rank steps of 32 the pool's padded rank has at
// most (1, 2, 4 or 8); the body is specialised for the tile's own step count (1 or
// 2; for KSM >= 4 one body with run-time bounds) and split batches.  Wave-uniform; ds is the wave's
// kExpandMfmaWaveFloats floats of LDS.
// Slot-table entries held lane-wise (pools of up to 128 slots): lane l holds slots l
// and l + 64, loaded once per wave; a unit picks its slot's entry with lane
// shuffles instead of a round trip of its own.
struct LaneTable {
  int4 t0, t1;
  bool on;
  __device__ __forceinline__ void load(const PoolView& P) {
    on = P.S <= 128;
    const int lane = lane_id();
    t0 = *reinterpret_cast<const int4*>(P.table + min(lane, P.S - 1));
    t1 = *reinterpret_cast<const int4*>(P.table + min(lane + 64, P.S - 1));
  }
  // slot < P.S, wave-uniform
  __device__ __forceinline__ SlotEntry get(const PoolView& P, int slot) const {
    SlotEntry e;
    if (!on) return P.table[slot];
    const int l = slot & 63;
    const int4 a = slot < 64 ? t0 : t1;
    e.rank = __builtin_amdgcn_readfirstlane(__shfl(a.x, l));
    e.scale = __int_as_float(__builtin_amdgcn_readfirstlane(__shfl(a.y, l)));
    e.slice_mask = (uint32_t)__builtin_amdgcn_readfirstlane(__shfl(a.z, l));
    e.pad = 0;
    return e;
  }
};

// The body of one expand tile: `len` tokens at sorted position p0 of slot `slot` (table
// entry e, rank > 0, slice n present), columns c00 .. of slice n; this lane's token id
// (token lane % 16, clamped into the tile) at tokp, or tokv when tokp is null.
template <typename TW, typename TY, int KSM>
__device__ __forceinline__ void expand_mfma_tile(const PoolView& P, const RouteView& R, const UView& U,
                                                 TY* __restrict__ y, int ldy, int slot, const SlotEntry& e, int n,
                                                 int c00, int p0, int len, const int* __restrict__ tokp, int tokv,
                                                 int cb, float* __restrict__ ds, UPartials<1>& ext,
                                                 bool ext_loaded) {
  const int on = P.o[n], dn = P.d[n];
  const int r = e.rank, nks = (r + kMfmaK - 1) / kMfmaK, rs = bk_stride(r);
  const TW* __restrict__ bk = static_cast<const TW*>(P.Bk) + (size_t)slot * P.D * P.Rk + (size_t)on * rs;
  const int nsb = U.by_token ? 0 : U.nsplit <= kUSplitBatch ? 1 : 2;
#define RAX_EXPAND_BODY(NK, NB, CB) \
  expand_mfma_body<TW, TY, NK, NB, CB>(R, U, y, ldy, bk, rs, n, on, dn, c00, p0, len, tokp, tokv, r, nks, e.scale, ds, \
                                       ext, ext_loaded)
#define RAX_EXPAND_BODIES(NK)                                                          \
  do {                                                                                 \
    if (cb == 1) {                                                                     \
      if (nsb == 1) RAX_EXPAND_BODY(NK, 1, 1);                                         \
      else if (nsb == 2) RAX_EXPAND_BODY(NK, 2, 1);                                    \
      else RAX_EXPAND_BODY(NK, 0, 1);                                                  \
    } else {                                                                           \
      if (nsb == 1) RAX_EXPAND_BODY(NK, 1, kMfmaColBlocksPerUnit);                     \
      else if (nsb == 2) RAX_EXPAND_BODY(NK, 2, kMfmaColBlocksPerUnit);                \
      else RAX_EXPAND_BODY(NK, 0, kMfmaColBlocksPerUnit);                              \
    }                                                                                  \
  } while (0)
  if constexpr (KSM <= 2) {
    if (nks == 1) RAX_EXPAND_BODIES(1);
    else if constexpr (KSM == 2) RAX_EXPAND_BODIES(2);
  } else {
    RAX_EXPAND_BODIES(KSM);
  }
#undef RAX_EXPAND_BODIES
#undef RAX_EXPAND_BODY
}

template <typename TW, typename TY, int KSM>
__device__ __forceinline__ void expand_mfma_unit(const PoolView& P, const RouteView& R, const UView& U,
                                                 TY* __restrict__ y, int ldy, int tile, int grp, int cb,
                                                 const LaneTable& lt, float* __restrict__ ds) {
  int blk0;
  const int n = mfma_group_slice(P, grp, cb, blk0);
  if (n < 0) return;
  const int4 td = R.tiles[tile];
  int slot = td.x, p0 = td.y;
  const int len = td.z;
  RAX_CHECK_VAR(slot, P.S);
  RAX_CHECK_VAR(p0, R.T - len + 1);
  const SlotEntry e = lt.get(P, slot);
  // this lane's token id (token lane % 16): loaded by the body ahead of the partials
  const int* __restrict__ tokp = R.sorted + p0 + min(lane_id() & 15, len - 1);
  if (e.rank == 0 || e.scale == 0.f || !((e.slice_mask >> n) & 1u)) return;
  UPartials<1> ext;
  expand_mfma_tile<TW, TY, KSM>(P, R, U, y, ldy, slot, e, n, blk0 * kMfmaCols, p0, len, tokp, 0, cb, ds, ext, false);
}

// Slot-mode expand unit: every tile of slot s's segment (any length) for column group
// grp.  The first tile's partials are at first-tile rows when U.head0 >= 0 (rows that
// depend only on s), else at its sorted positions like the other tiles'.  For pools of
// one rank step with first-tile rows and one batch of partials, this lane's token id
// of the first tile goes out first, then that tile's partials, then the slot's routing
// record header and slot-table entry (scalar loads, counted apart from the vector
// loads): the y rows and B fragments are addressed as soon as the token id and the
// entry are in, while the partials, the longest round trip, are still on their way; a
// segment of one tile then needs nothing else (a longer one reads them again in its
// tile loop).  Otherwise the record, the token ids and the entry come first, the
// partials after them.  Tokens past the record's come from the sorted list.
template <typename TW, typename TY, int KSM>
__device__ __forceinline__ void expand_slot_unit(const PoolView& P, const RouteView& R, const UView& U,
                                                 TY* __restrict__ y, int ldy, int s, int grp, int cb,
                                                 float* __restrict__ ds) {
  int blk0;
  const int n = mfma_group_slice(P, grp, cb, blk0);
  if (n < 0) return;
  const int lr = lane_id() & 15;
  const int* __restrict__ rec = R.rec + (size_t)s * kRecInts;
  const bool head = U.head0 >= 0;   // the shrink put the first tile's partials at first-tile rows
  // issued ahead for pools of one rank step (their units have the registers for it)
  const bool ahead = KSM == 1 && head && U.nsplit <= kUSplitBatch;
  int tok0 = 0;
  UPartials<1> pre;
  if (ahead) {
    tok0 = rec[4 + lr];
    sched_fence();
    pre.load_head(U, n, (long long)U.head0 + kMfmaTileM * s + lr);
    sched_fence();
  }
  const int2 hdr = *reinterpret_cast<const int2*>(rec);
  if (!ahead) tok0 = rec[4 + lr];
  const SlotEntry e = P.table[s];
  const int L = __builtin_amdgcn_readfirstlane(hdr.x);
  int p0 = __builtin_amdgcn_readfirstlane(hdr.y);
  RAX_CHECK_VAR(p0, R.T - L + 1);
  if (L == 0 || e.rank == 0 || e.scale == 0.f || !((e.slice_mask >> n) & 1u)) return;
  if (ahead && L <= kMfmaTileM) {
    // a segment of one tile (the common decode case): its partials are already in flight
    expand_mfma_tile<TW, TY, KSM>(P, R, U, y, ldy, s, e, n, blk0 * kMfmaCols, U.head0 + kMfmaTileM * s, L, nullptr,
                                  tok0, cb, ds, pre, true);
    return;
  }
  UPartials<1> ext;
  for (int t0 = 0; t0 < L; t0 += kMfmaTileM) {
    const int len = min(kMfmaTileM, L - t0), ti = t0 + min(lr, len - 1);
    const int tk = t0 == 0 ? tok0 : (ti < kRecTokens ? rec[4 + ti] : R.sorted[p0 + ti]);
    // partial rows: the first tile's at its first-tile rows (read again), the others by
    // sorted position
    const int urow = head && t0 == 0 ? U.head0 + kMfmaTileM * s : p0 + t0;
    // values the tile body derives are recomputed per tile rather than held across
    // the loop (an opaque copy of the slot's entry and indices)
    SlotEntry ev = e;
    int sv = s, nv = n, cv = blk0 * kMfmaCols;
    asm volatile("" : "+s"(sv), "+s"(nv), "+s"(cv), "+s"(ev.rank), "+s"(ev.scale), "+s"(ev.slice_mask));
    expand_mfma_tile<TW, TY, KSM>(P, R, U, y, ldy, sv, ev, nv, cv, urow, len, nullptr, tk, cb, ds, ext, false);
  }
}

}  // namespace rax
