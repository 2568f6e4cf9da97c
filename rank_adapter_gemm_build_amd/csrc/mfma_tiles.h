// Matrix-core (MFMA) tiles for long same-slot segments (device code, included by linear.hip).
//
// Page "第16章 LoRA 适配器热切换", §16.4.3: in prefill a segment holds all tokens of the
// requests on one adapter, so it is long, and the per-segment shrink [L, k] x [k, r]
// and expand [L, r] x [r, d] are real matrix products.  Page "TensorRT-LLM 源码完全拆解
// (二十一)", section "前向替换": prefill batches take a grouped-GEMM path of their own.
// Here those segments are cut by the routing into tiles of up to 64 tokens, and both
// products run on the gfx950 bf16 matrix cores (v_mfma_f32_16x16x32_bf16, fp32
// accumulation).  Fragment layouts of the 16x16x32 instruction: lane l supplies row
// l % 16 and the 8 consecutive k values 8 * (l / 16) .. +7 of each operand, and
// receives rows 4 * (l / 16) .. +3 of column l % 16 of the result.
//
// Shrink: D[token][f] = sum_c x[token][c] * A[f][c], f = the flattened (slice, rank)
// row.  A block of 4 * kq waves owns one 64-token tile: wave w takes the 16 tokens
// 16 * (w % 4) .. +15 over the k range w / 4 of kq contiguous parts.  Operand rows are
// k-contiguous in both x and the pool's A, so each lane loads its 8 bf16 of a fragment
// with one 16-byte load straight from HBM; x rows are gathered through sorted_ids and
// every x element is read once.  The fragments of kMfmaGroup k-steps are loaded
// together before their products.  The kq partial results meet in LDS in k order
// (group 0 first), so the finished values do not depend on timing.
//
// Expand: D[token][col] = sum_j u[token][j] * B[col][j], read from the pool's
// rank-contiguous copy of B.  Each lane loads its fp32 rank-space values once per tile
// and keeps them in registers as bf16 hi + lo parts (hi = bf16(u), lo = bf16(u - hi)),
// two products per step, so u keeps about 16 mantissa bits instead of being rounded to
// bf16; the same fragments serve a sweep over up to kMfmaColBlocksPerGroup column
// blocks.  Each 64 x 128 result block goes through LDS so that the read-modify-write of
// y (the dominant traffic) moves 16 bytes per lane along rows.
#pragma once

#include "device_util.h"

namespace rax {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

constexpr int kMfmaGroup = 4;                    // shrink k-steps whose fragments load together
constexpr int kDsPitch = kMfmaCols + 4;          // LDS row pitch of the expand result tile
constexpr int kExpandMfmaSmemFloats = kMfmaTileM * kDsPitch;
constexpr int kShrinkMfmaSmemFloats = 4 * 16 * 64;   // one k group's results: 4 token groups x 16 values x 64 lanes

// Products of one pass over k steps [s0, s1) for NB blocks of 16 rows, starting at
// flattened row fp: the B operand of block b is row fp + 16 b + (lane % 16) of A.
template <int NB>
__device__ __forceinline__ void shrink_mfma_pass(const uint16_t* __restrict__ xrow, bool tval,
                                                 const uint16_t* __restrict__ Aslot, int fp, int F, int r,
                                                 int Rmax, int s0, int s1, int k, int lr, int lk,
                                                 f32x4_t (&acc)[4]) {
  const uint16_t* arow[NB];
  bool rval[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int f = fp + 16 * b + lr;
    rval[b] = f < F;
    const int fc = rval[b] ? f : 0;
    const int n = fc / r, j = fc - n * r;
    arow[b] = Aslot + ((size_t)n * Rmax + j) * k;
  }
  for (int sg = s0; sg < s1; sg += kMfmaGroup) {
    uint4 xa[kMfmaGroup], wb[kMfmaGroup][NB];
#pragma unroll
    for (int g = 0; g < kMfmaGroup; ++g) {
      const int col = (sg + g) * kMfmaK + 8 * lk;
      const bool inb = sg + g < s1 && col < k;     // k % 8 == 0: a chunk is wholly in or out
      const int colc = min(col, k - 8);
      xa[g] = keep_if(ld16(xrow + colc), tval && inb);
#pragma unroll
      for (int b = 0; b < NB; ++b) wb[g][b] = keep_if(ld16(arow[b] + colc), rval[b] && inb);
    }
    sched_fence();
#pragma unroll
    for (int g = 0; g < kMfmaGroup; ++g)
#pragma unroll
      for (int b = 0; b < NB; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[g]), as_bf16x8(wb[g][b]), acc[b], 0, 0, 0);
  }
}

// One tile of the shrink: finished rank-space values of its tokens.  Block-uniform
// control flow; the block has 4 * kq waves and kShrinkMfmaSmemFloats floats of LDS.
__device__ __forceinline__ void shrink_mfma_tile(const PoolView& P, const RouteView& R,
                                                 const uint16_t* __restrict__ x, int ldx,
                                                 const UView& U, int kq, int tile, float* __restrict__ buf) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 15, lk = lane >> 4;
  const int tg = w & 3, kg = w >> 2;
  const int4 td = R.tiles[tile];
  const int slot = td.x, p0 = td.y, len = td.z;
  const SlotEntry e = P.table[slot];
  if (e.rank == 0) return;
  const int r = e.rank, F = P.N * r;
  const int t = 16 * tg + lr;                      // token of this lane's x fragment row
  const bool tval = t < len;
  const uint16_t* xrow = x + (size_t)R.sorted[p0 + min(t, len - 1)] * ldx;
  const uint16_t* Aslot = static_cast<const uint16_t*>(P.A) + (size_t)slot * P.N * P.Rmax * P.k;
  const int steps = (P.k + kMfmaK - 1) / kMfmaK;
  const int per = (steps + kq - 1) / kq;
  const int s0 = min(steps, kg * per), s1 = min(steps, s0 + per);
  for (int fp = 0; fp < F; fp += 64) {            // up to 4 blocks of 16 rows per pass
    f32x4_t acc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int nb = min(4, (F - fp + 15) / 16);
    if (nb == 4)
      shrink_mfma_pass<4>(xrow, tval, Aslot, fp, F, r, P.Rmax, s0, s1, P.k, lr, lk, acc);
    else if (nb == 3)
      shrink_mfma_pass<3>(xrow, tval, Aslot, fp, F, r, P.Rmax, s0, s1, P.k, lr, lk, acc);
    else if (nb == 2)
      shrink_mfma_pass<2>(xrow, tval, Aslot, fp, F, r, P.Rmax, s0, s1, P.k, lr, lk, acc);
    else
      shrink_mfma_pass<1>(xrow, tval, Aslot, fp, F, r, P.Rmax, s0, s1, P.k, lr, lk, acc);
    // k groups meet in LDS in order 0, 1, ..., kq - 1; the last one writes u
    float* mine = buf + (tg * 16) * 64 + lane;     // value v of this lane at mine[v * 64]
    for (int v = 0; v < kq; ++v) {
      if (kg == v) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float s = acc[b][i];
            if (v > 0) s = mine[(4 * b + i) * 64] + s;
            if (v + 1 < kq) {
              mine[(4 * b + i) * 64] = s;
            } else {
              const int f = fp + 16 * b + lr, tt = 16 * tg + 4 * lk + i;
              if (f < F && tt < len) {
                const int n = f / r, j = f - n * r;
                const long long row = U.by_token ? (long long)R.sorted[p0 + tt] : (long long)(p0 + tt);
                U.p[n * U.n_stride + row * U.row_stride + j] = s;
              }
            }
          }
      }
      __syncthreads();
    }
  }
}

// Column blocks [cb0, cb0 + kMfmaColBlocksPerGroup) of one tile of the expand, for
// pools whose padded rank Rk is at most 32 * KS (KS rank steps held in registers).
// Block-uniform control flow; 4 waves, kExpandMfmaSmemFloats floats of LDS.
template <typename TY, int KS>
__device__ __forceinline__ void expand_mfma_tile(const PoolView& P, const RouteView& R, const UView& U,
                                                 TY* __restrict__ y, int ldy, int cb0, int tile,
                                                 float* __restrict__ ds) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 15, lk = lane >> 4;
  const int4 td = R.tiles[tile];
  const int slot = td.x, p0 = td.y, len = td.z;
  const SlotEntry e = P.table[slot];
  if (e.rank == 0 || e.scale == 0.f) return;       // uniform per block
  const int r = e.rank;
  const int nks = (r + kMfmaK - 1) / kMfmaK;       // rank steps of 32 (<= KS)
  const int cb1 = min(P.n_mblocks, cb0 + kMfmaColBlocksPerGroup);
  const int t = 16 * w + lr;                       // token of this lane's u fragment row
  const bool tval = t < len;
  const long long urow = U.by_token ? (long long)R.sorted[p0 + min(t, len - 1)] : (long long)(p0 + min(t, len - 1));
  int cur_n = -1;
  uint4 uh[KS], ul[KS];
  for (int cb = cb0; cb < cb1; ++cb) {
    int n = 0;
    while (n + 1 < P.N && cb >= P.mblk0[n + 1]) ++n;
    if (!((e.slice_mask >> n) & 1u)) continue;
    if (n != cur_n) {                              // this lane's u fragments of slice n, as hi + lo
      const float* __restrict__ up = U.p + n * U.n_stride + urow * U.row_stride;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks < nks) {
          float uv[8];
#pragma unroll
          for (int e2 = 0; e2 < 8; ++e2) {
            const int j = ks * kMfmaK + 8 * lk + e2;
            const bool ok = tval && j < r;
            const float v = up[ok ? j : 0];
            uv[e2] = ok ? v : 0.f;
          }
          uint32_t hi[4], lo[4];
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const uint32_t h0 = f32_to_bf16(uv[2 * e2]), h1 = f32_to_bf16(uv[2 * e2 + 1]);
            hi[e2] = h0 | (h1 << 16);
            lo[e2] = f32_to_bf16(uv[2 * e2] - __uint_as_float(h0 << 16)) |
                     (f32_to_bf16(uv[2 * e2 + 1] - __uint_as_float(h1 << 16)) << 16);
          }
          uh[ks] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
          ul[ks] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        }
      }
      cur_n = n;
    }
    const int c0 = (cb - P.mblk0[n]) * kMfmaCols;
    const int dn = P.d[n];
    const uint16_t* __restrict__ bk = static_cast<const uint16_t*>(P.Bk) + ((size_t)slot * P.D + P.o[n]) * P.Rk;
    f32x4_t acc[8];
#pragma unroll
    for (int cbk = 0; cbk < 8; ++cbk) acc[cbk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks < nks) {
        const int jr = ks * kMfmaK + 8 * lk;       // jr + 8 <= 32 * nks <= Rk: the load stays in the row
        uint4 bv[8];
#pragma unroll
        for (int cbk = 0; cbk < 8; ++cbk) {
          const int col = c0 + 16 * cbk + lr;
          const bool cval = col < dn;
          bv[cbk] = keep_if(ld16(bk + (size_t)(cval ? col : 0) * P.Rk + jr), cval);
        }
        sched_fence();
#pragma unroll
        for (int cbk = 0; cbk < 8; ++cbk) {
          acc[cbk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(uh[ks]), as_bf16x8(bv[cbk]), acc[cbk], 0, 0, 0);
          acc[cbk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ul[ks]), as_bf16x8(bv[cbk]), acc[cbk], 0, 0, 0);
        }
      }
    }
    // result block to LDS: lane holds D[token 4*lk + i][column lr] of block cbk
#pragma unroll
    for (int cbk = 0; cbk < 8; ++cbk)
#pragma unroll
      for (int i = 0; i < 4; ++i) ds[(16 * w + 4 * lk + i) * kDsPitch + 16 * cbk + lr] = acc[cbk][i];
    __syncthreads();
    // y[row][o_n + c0 + cc .. +8] += s * D, 16 bytes of y per lane
    for (int idx = tid; idx < kMfmaTileM * (kMfmaCols / 8); idx += 256) {
      const int tt = idx / (kMfmaCols / 8), cc = (idx % (kMfmaCols / 8)) * 8;
      if (tt < len && c0 + cc < dn) {
        TY* yp = y + (size_t)R.sorted[p0 + tt] * ldy + P.o[n] + c0 + cc;
        float v[8];
        load8f(yp, true, v);
        const float* dp = ds + tt * kDsPitch + cc;
#pragma unroll
        for (int c = 0; c < 8; ++c) v[c] = v[c] + e.scale * dp[c];
        store8f(yp, v);
      }
    }
    __syncthreads();
  }
}

}  // namespace rax
