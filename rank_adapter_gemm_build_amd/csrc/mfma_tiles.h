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
// Expand unit (tile, group of kMfmaColBlocksPerUnit 128-column blocks):
// D[token][col] = sum_j u[token][j] * B[col][j], from the pool's rank-contiguous copy
// of B.  The wave first finishes its tokens' rank-space values (partials added in
// split order) and keeps them as bf16 hi + lo parts (hi = bf16(u), lo = bf16(u - hi)),
// two products per step, so u keeps about 16 mantissa bits instead of being rounded
// to bf16; then, per column block, the B fragments and the tile's y chunks load in
// one batch, and the 16 x 128 result goes through the wave's own LDS slice so that
// the read-modify-write of y (the dominant traffic) moves 16 bytes per lane along
// rows.
#pragma once

#include "device_util.h"

namespace rax {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

constexpr int kMfmaGroup = 4;                    // shrink k-steps whose fragments load together
constexpr int kDsPitch = kMfmaCols + 4;          // LDS row pitch (floats) of the expand result tile
constexpr int kExpandMfmaWaveFloats = kMfmaTileM * kDsPitch;   // LDS floats per expand wave

// ------------------------------------------------------------------ shrink
template <int NB>
struct ShrinkFrags {
  uint4 xa[kMfmaGroup];
  uint4 wb[kMfmaGroup][NB];
};

// Loads of one group: raw values only, so that nothing consumes them before the
// products (a consumer in the load phase would make the wave wait for the group
// right after issuing it, defeating the double buffering).  Steps past the part's
// end reload its last step (a cache hit); the products zero them.
template <int NB>
__device__ __forceinline__ void shrink_load_group(ShrinkFrags<NB>& f, const uint16_t* __restrict__ xrow,
                                                  const uint16_t* const (&arow)[NB], int sg, int last, int k,
                                                  int lk) {
#pragma unroll
  for (int g = 0; g < kMfmaGroup; ++g) {
    const int st = min(sg + g, last);
    const int colc = min(st * kMfmaK + 8 * lk, k - 8);
    f.xa[g] = ld16(xrow + colc);
#pragma unroll
    for (int b = 0; b < NB; ++b) f.wb[g][b] = ld16(arow[b] + colc);
  }
}

// Products of one group; fragments of steps outside [sg, s1), of rows past the last
// valid one and of tokens past the tile's length are zeroed here.
template <int NB>
__device__ __forceinline__ void shrink_mma_group(const ShrinkFrags<NB>& f, bool tval, const bool (&rval)[NB], int sg,
                                                 int s1, int k, int lk, f32x4_t (&acc)[NB]) {
#pragma unroll
  for (int g = 0; g < kMfmaGroup; ++g) {
    const bool inb = sg + g < s1 && (sg + g) * kMfmaK + 8 * lk < k;  // k % 8 == 0: chunks wholly in or out
    const uint4 xa = keep_if(f.xa[g], tval && inb);
#pragma unroll
    for (int b = 0; b < NB; ++b)
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa), as_bf16x8(keep_if(f.wb[g][b], rval[b])), acc[b],
                                                       0, 0, 0);
  }
}

// Products of rows fr0 .. fr0 + 16 * NB of one tile over k steps [s0, s1): lane
// holds D[token 4 * lk + i][row fr0 + 16 b + lr] in acc[b][i].
template <int NB>
__device__ __forceinline__ void shrink_mfma_acc(const PoolView& P, const RouteView& R, const uint16_t* __restrict__ x,
                                                int ldx, int slot, int r, int p0, int len, int fr0, int s0, int s1,
                                                f32x4_t (&acc)[NB]) {
  const int lane = lane_id(), lr = lane & 15, lk = lane >> 4;
  const int F = P.N * r;
  const bool tval = lr < len;
  const uint16_t* xrow = x + (size_t)R.sorted[p0 + min(lr, len - 1)] * ldx;
  const uint16_t* Aslot = static_cast<const uint16_t*>(P.A) + (size_t)slot * P.N * P.Rmax * P.k;
  const uint16_t* arow[NB];
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
  ShrinkFrags<NB> f0, f1;
  shrink_load_group<NB>(f0, xrow, arow, s0, last, P.k, lk);
  for (int sg = s0; sg < s1; sg += 2 * kMfmaGroup) {
    shrink_load_group<NB>(f1, xrow, arow, sg + kMfmaGroup, last, P.k, lk);
    sched_fence();
    shrink_mma_group<NB>(f0, tval, rval, sg, s1, P.k, lk, acc);
    sched_fence();
    shrink_load_group<NB>(f0, xrow, arow, sg + 2 * kMfmaGroup, last, P.k, lk);
    sched_fence();
    shrink_mma_group<NB>(f1, tval, rval, sg + kMfmaGroup, s1, P.k, lk, acc);
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
template <int NB>
__device__ __forceinline__ void shrink_mfma_rows(const PoolView& P, const RouteView& R, const uint16_t* __restrict__ x,
                                                 int ldx, const UView& U, int slot, int r, int p0, int len, int fr0,
                                                 int part, int s0, int s1) {
  const int lane = lane_id(), lr = lane & 15, lk = lane >> 4;
  const int F = P.N * r;
  f32x4_t acc[NB];
  shrink_mfma_acc<NB>(P, R, x, ldx, slot, r, p0, len, fr0, s0, s1, acc);
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
        if (t < len) up[t * U.row_stride] = acc[b][i];
      }
    }
  }
}

// One shrink unit: tile `tile`, row group rg (rows 64 rg .. 64 rg + 63), k part
// `part` of nsplit.  Wave-uniform.  Parts with no k steps write zeros.
__device__ __forceinline__ void shrink_mfma_unit(const PoolView& P, const RouteView& R, const uint16_t* __restrict__ x,
                                                 int ldx, const UView& U, int tile, int rg, int part, int nsplit) {
  const int4 td = R.tiles[tile];
  const int slot = td.x, p0 = td.y, len = td.z;
  const SlotEntry e = P.table[slot];
  const int r = e.rank, F = P.N * r, fr0 = 64 * rg;
  if (r == 0 || fr0 >= F) return;
  int s0, s1;
  mfma_part_range(P.k, part, nsplit, s0, s1);
  const int nb = min(4, (F - fr0 + 15) / 16);
  if (nb == 4)
    shrink_mfma_rows<4>(P, R, x, ldx, U, slot, r, p0, len, fr0, part, s0, s1);
  else if (nb == 3)
    shrink_mfma_rows<3>(P, R, x, ldx, U, slot, r, p0, len, fr0, part, s0, s1);
  else if (nb == 2)
    shrink_mfma_rows<2>(P, R, x, ldx, U, slot, r, p0, len, fr0, part, s0, s1);
  else
    shrink_mfma_rows<1>(P, R, x, ldx, U, slot, r, p0, len, fr0, part, s0, s1);
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

// This lane's rank-space values of slice n for the u fragment rows of the tile
// (token lr, ranks 32 ks + 8 lk .. +7), finished from their split partials in split
// order, as bf16 hi + lo parts.  Zero past the rank and past the tile's length.
template <int KSM>
__device__ __forceinline__ void expand_u_frags(const RouteView& R, const UView& U, int n, int p0, int len, int r,
                                               int nks, uint4 (&uh)[KSM], uint4 (&ul)[KSM]) {
  const int lane = lane_id(), lr = lane & 15, lk = lane >> 4;
  const int t = min(lr, len - 1);
#pragma unroll
  for (int ks = 0; ks < KSM; ++ks) {
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = 0.f;
    if (ks < nks) {
      const int j0 = ks * kMfmaK + 8 * lk;
      if (!U.by_token) {
        // workspace rows are padded to a multiple of 32 floats: two 16-byte loads per split
        const float* base = U.p + n * U.n_stride + (long long)(p0 + t) * U.row_stride + j0;
        for (int s0 = 0; s0 < U.nsplit; s0 += 4) {
          float4 pa[4], pb[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int sq = min(s0 + q, U.nsplit - 1);
            pa[q] = *reinterpret_cast<const float4*>(base + sq * U.split_stride);
            pb[q] = *reinterpret_cast<const float4*>(base + sq * U.split_stride + 4);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (s0 + q < U.nsplit) {
              if (s0 + q == 0) {
                v[0] = pa[q].x; v[1] = pa[q].y; v[2] = pa[q].z; v[3] = pa[q].w;
                v[4] = pb[q].x; v[5] = pb[q].y; v[6] = pb[q].z; v[7] = pb[q].w;
              } else {
                v[0] += pa[q].x; v[1] += pa[q].y; v[2] += pa[q].z; v[3] += pa[q].w;
                v[4] += pb[q].x; v[5] += pb[q].y; v[6] += pb[q].z; v[7] += pb[q].w;
              }
            }
          }
        }
      } else {
        // the caller's finished u, rows by token, row stride Rmax
        const float* base = U.p + n * U.n_stride + (long long)R.sorted[p0 + t] * U.row_stride;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int j = j0 + q;
          v[q] = base[j < r ? j : 0];
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = (lr < len && j0 + q < r) ? v[q] : 0.f;
    }
    u_hilo(v, uh[ks], ul[ks]);
  }
}

// One 128-column block (columns c0 .. c0 + 127 of slice n) of one tile.
template <typename TY, int KSM>
__device__ __forceinline__ void expand_mfma_block(const PoolView& P, const RouteView& R, TY* __restrict__ y, int ldy,
                                                  int slot, float scale, int n, int c0, int p0, int len, int nks,
                                                  const uint4 (&uh)[KSM], const uint4 (&ul)[KSM],
                                                  float* __restrict__ ds) {
  constexpr int YC = 16 / sizeof(TY);             // y elements per 16-byte chunk
  constexpr int YCHUNKS = kMfmaTileM * kMfmaCols / YC / 64;  // y chunks per lane
  constexpr int KP = 1;                           // rank steps per batch of B fragments
  const int lane = lane_id(), lr = lane & 15, lk = lane >> 4;
  const int dn = P.d[n];
  const uint16_t* __restrict__ bk = static_cast<const uint16_t*>(P.Bk) + ((size_t)slot * P.D + P.o[n]) * P.Rk;
  uint4 yv[YCHUNKS];
  TY* yp[YCHUNKS];
  bool yok[YCHUNKS];
#pragma unroll
  for (int q = 0; q < YCHUNKS; ++q) {
    const int idx = q * 64 + lane;
    const int t = idx / (kMfmaCols / YC), cc = (idx % (kMfmaCols / YC)) * YC;
    yok[q] = t < len && c0 + cc < dn;
    yp[q] = y + (size_t)R.sorted[p0 + min(t, len - 1)] * ldy + P.o[n] + min(c0 + cc, dn - YC);
    yv[q] = ld16(yp[q]);
  }
  f32x4_t acc[8];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks0 = 0; ks0 < KSM; ks0 += KP) {
    if (ks0 < nks) {
      uint4 bv[KP][8];
#pragma unroll
      for (int kk = 0; kk < KP; ++kk) {
        const int ks = ks0 + kk;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
          const int col = c0 + 16 * cb + lr;
          // (ks < nks) 32 ks + 8 lk + 8 <= 32 nks <= Rk: the load stays in the row
          bv[kk][cb] = ld16(bk + (size_t)(col < dn ? col : 0) * P.Rk + (ks < nks ? ks : 0) * kMfmaK + 8 * lk);
        }
      }
      sched_fence();
#pragma unroll
      for (int kk = 0; kk < KP; ++kk) {
        const int ks = ks0 + kk;
        if (ks < nks) {
#pragma unroll
          for (int cb = 0; cb < 8; ++cb) {
            const uint4 b = keep_if(bv[kk][cb], c0 + 16 * cb + lr < dn);
            acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(uh[ks]), as_bf16x8(b), acc[cb], 0, 0, 0);
            acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ul[ks]), as_bf16x8(b), acc[cb], 0, 0, 0);
          }
        }
      }
    }
  }
  // result through LDS: lane holds D[token 4 lk + i][column 16 cb + lr]
#pragma unroll
  for (int cb = 0; cb < 8; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) ds[(4 * lk + i) * kDsPitch + 16 * cb + lr] = acc[cb][i];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int q = 0; q < YCHUNKS; ++q) {
    if (yok[q]) {
      const int idx = q * 64 + lane;
      const int t = idx / (kMfmaCols / YC), cc = (idx % (kMfmaCols / YC)) * YC;
      const float* dp = ds + t * kDsPitch + cc;
      if constexpr (sizeof(TY) == 2) {
        float v[8];
        unpack8(yv[q], v);
#pragma unroll
        for (int c = 0; c < 8; ++c) v[c] = v[c] + scale * dp[c];
        store8f(yp[q], v);
      } else {
        uint4 o;
        o.x = __float_as_uint(__uint_as_float(yv[q].x) + scale * dp[0]);
        o.y = __float_as_uint(__uint_as_float(yv[q].y) + scale * dp[1]);
        o.z = __float_as_uint(__uint_as_float(yv[q].z) + scale * dp[2]);
        o.w = __float_as_uint(__uint_as_float(yv[q].w) + scale * dp[3]);
        st16(yp[q], o);
      }
    }
  }
  // the LDS slice is rewritten by the next block
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One expand unit: tile `tile`, global 128-column blocks mb0 .. mb0 + G - 1.  KSM is
// the number of rank steps of 32 the pool's padded rank has at most (1, 2, 4 or 8).
// Wave-uniform; ds is the wave's kExpandMfmaWaveFloats floats of LDS.
template <typename TY, int KSM>
__device__ __forceinline__ void expand_mfma_unit(const PoolView& P, const RouteView& R, const UView& U,
                                                 TY* __restrict__ y, int ldy, int tile, int mb0,
                                                 float* __restrict__ ds) {
  const int4 td = R.tiles[tile];
  const int slot = td.x, p0 = td.y, len = td.z;
  const SlotEntry e = P.table[slot];
  if (e.rank == 0 || e.scale == 0.f) return;
  const int r = e.rank, nks = (r + kMfmaK - 1) / kMfmaK;
  const int mb1 = min(P.n_mblocks, mb0 + kMfmaColBlocksPerUnit);
  int cur_n = -1;
  uint4 uh[KSM], ul[KSM];
  for (int mb = mb0; mb < mb1; ++mb) {
    int n = 0;
    while (n + 1 < P.N && mb >= P.mblk0[n + 1]) ++n;
    if (!((e.slice_mask >> n) & 1u)) continue;
    if (n != cur_n) {
      expand_u_frags<KSM>(R, U, n, p0, len, r, nks, uh, ul);
      cur_n = n;
    }
    expand_mfma_block<TY, KSM>(P, R, y, ldy, slot, e.scale, n, (mb - P.mblk0[n]) * kMfmaCols, p0, len, nks, uh, ul,
                               ds);
  }
}

}  // namespace rax
