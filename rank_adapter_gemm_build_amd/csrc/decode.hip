// Decode-path shrink and expand: short same-slot segments on the vector ALUs.
//
// Page "第16章 LoRA 适配器热切换", §16.4.2: with tokens grouped by slot, all LoRA branches
// of a batch run as two kernels, a shrink on lora_a into a [tokens, r] buffer and an
// expand on lora_b back to [tokens, d]; each block takes a segment of same-slot tokens.
// §16.4.3: in decode a segment is as long as the number of requests on that adapter,
// so it is short.  Page "llama.cpp 源码完全拆解(十六)", section "为什么低秩增量可以「后加」":
// decode is bound by memory bandwidth, and the adapter's A and B are small.
//
// Shrink (one wave per (active slot, k-split)).  Lanes split the k axis: lane l owns
// the 16-byte chunks at k offsets kb + c*64*E + l*E (E = 8 bf16 or 4 fp32), so every
// row of A streams from HBM as one contiguous 1 KB request per wave and each row of A
// is read once per slot, not once per token.  The wave gathers the x rows of its
// segment (token order given by sorted_ids) into registers: each lane holds exactly the
// k-slice it multiplies, so no LDS round trip is needed.  For a block of rows x tokens
// (64 accumulators) it accumulates lane-partial dot products and finishes all 64 of
// them with one reduce-scatter across the wave, after which lane l holds output l.
// Split-K partials go to a workspace and are added in a fixed order by the expand.
//
// Expand (one wave per (active slot, 512-column tile of one slice)).  The rank-space
// values of the segment (split partials added in order q = 0, 1, ...) are staged in
// LDS and read as broadcasts.  Lanes own 8 consecutive output columns, so each
// rank-major row of B^T streams as one contiguous 1 KB request; the contraction over
// the rank stays in registers.  The epilogue reads the token's row of y at its original
// index (no permutation pass; page "TensorRT-LLM 源码完全拆解(二十一)", section
// "前向替换", restores order with index_copy_ - here rows are written in place), adds
// s * acc in fp32 and rounds once.
#include <hip/hip_runtime.h>

#include "device_util.h"

namespace rax {

// ------------------------------------------------------------------- shrink
// LT tokens x RB rows = 64 accumulators per lane; NS 16-byte chunk steps per split.
// All loads of one block are unconditional (addresses clamped into the operand,
// unused values replaced by zero), so the compiler can issue them together.
template <typename T, int LT, int NS>
__device__ __forceinline__ void shrink_segment(const PoolView& P, const RouteView& R,
                                               const T* __restrict__ x, int ldx, const UView& U,
                                               int slot, const SlotEntry& e, int L, int p0,
                                               int kb, int ke, int q) {
  constexpr int E = Elem<T>::kPerChunk;
  constexpr int CW = 64 * E;         // k elements covered by one wave-wide chunk step
  constexpr int RB = 64 / LT;        // rows per block
  const int lane = lane_id();
  const int r = e.rank, F = P.N * r;
  const T* __restrict__ Aslot = static_cast<const T*>(P.A) + (size_t)slot * P.N * P.Rmax * P.k;
  for (int tt = 0; tt < L; tt += LT) {
    const int nt = min(LT, L - tt);
    uint4 xv[LT][NS];
#pragma unroll
    for (int i = 0; i < LT; ++i) {
      const int tok = R.sorted[p0 + tt + min(i, nt - 1)];
      const T* xrow = x + (size_t)tok * ldx;
#pragma unroll
      for (int c = 0; c < NS; ++c) {
        const int col = kb + c * CW + lane * E;
        xv[i][c] = keep_if(ld16(xrow + min(col, P.k - E)), i < nt && col < ke);
      }
    }
    for (int fb = 0; fb < F; fb += RB) {
      float acc[64];
#pragma unroll
      for (int m = 0; m < 64; ++m) acc[m] = 0.f;
      const int n0 = fb / r, j0 = fb - n0 * r;
#pragma unroll
      for (int c = 0; c < NS; ++c) {
        const int col = kb + c * CW + lane * E;
        const bool inb = col < ke;
        const int colc = min(col, P.k - E);
        int n = n0, j = j0;
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) {
          const bool rv = fb + rr < F;
          const T* arow = Aslot + ((size_t)(rv ? n : 0) * P.Rmax + (rv ? j : 0)) * P.k;
          const uint4 av = keep_if(ld16(arow + colc), rv && inb);
#pragma unroll
          for (int i = 0; i < LT; ++i) acc[rr * LT + i] = chunk_dot(av, xv[i][c], acc[rr * LT + i], T());
          if (++j == r) { j = 0; ++n; }
        }
      }
      reduce_scatter64(acc);
      const int rr = lane / LT, i = lane - rr * LT, f = fb + rr;
      if (f < F && i < nt) {
        const int n = f / r, j = f - n * r;
        const long long row = U.by_token ? (long long)R.sorted[p0 + tt + i] : (long long)(p0 + tt + i);
        U.p[q * U.q_stride + n * U.n_stride + row * U.row_stride + j] = acc[0];
      }
    }
  }
}

template <typename T, int NS>
__global__ __launch_bounds__(64) void shrink_decode_kernel(PoolView P, RouteView R,
                                                           const T* __restrict__ x, int ldx,
                                                           UView U, int kc, int use_mfma) {
  const int a = blockIdx.y, q = blockIdx.x;
  if (a >= R.meta[kMetaActive]) return;
  const int slot = R.active[a];
  const SlotEntry e = P.table[slot];
  if (e.rank == 0) return;
  const int L = R.counts[slot];
  if (use_mfma && L >= R.mfma_min) return;   // long segment: matrix-core kernel
  const int kb = q * kc;
  if (kb >= P.k) return;
  const int ke = min(P.k, kb + kc);
  const int p0 = R.offs[slot];
  // 8-token tiles only where x for 8 tokens fits in registers next to the A rows
  if (L <= 4 || NS > 2)
    shrink_segment<T, 4, NS>(P, R, x, ldx, U, slot, e, L, p0, kb, ke, q);
  else
    shrink_segment<T, 8, NS>(P, R, x, ldx, U, slot, e, L, p0, kb, ke, q);
}

template <typename T>
static void launch_shrink_t(const PoolView& P, const RouteView& R, const T* x, int ldx, const UView& U,
                            int kc, int use_mfma, hipStream_t stream, const KTimer& tm) {
  const int ns = kc / (64 * Elem<T>::kPerChunk);
  const dim3 grid((P.k + kc - 1) / kc, P.S);
  switch (ns) {
    case 1: RAX_LAUNCH(tm, (shrink_decode_kernel<T, 1>), grid, dim3(64), 0u, stream, P, R, x, ldx, U, kc, use_mfma); break;
    case 2: RAX_LAUNCH(tm, (shrink_decode_kernel<T, 2>), grid, dim3(64), 0u, stream, P, R, x, ldx, U, kc, use_mfma); break;
    case 3: RAX_LAUNCH(tm, (shrink_decode_kernel<T, 3>), grid, dim3(64), 0u, stream, P, R, x, ldx, U, kc, use_mfma); break;
    default: RAX_LAUNCH(tm, (shrink_decode_kernel<T, 4>), grid, dim3(64), 0u, stream, P, R, x, ldx, U, kc, use_mfma); break;
  }
}

hipError_t launch_shrink(int wdtype, const PoolView& P, const RouteView& R, const void* x, int ldx,
                         const UView& U, int kc, int use_mfma, hipStream_t stream, const KTimer& tm) {
  const int cw = 64 * (wdtype == LORA_BF16 ? 8 : 4);
  if (kc % cw != 0 || kc / cw < 1 || kc / cw > kMaxChunksPerSplit) return hipErrorInvalidValue;
  if (wdtype == LORA_BF16)
    launch_shrink_t(P, R, static_cast<const uint16_t*>(x), ldx, U, kc, use_mfma, stream, tm);
  else
    launch_shrink_t(P, R, static_cast<const float*>(x), ldx, U, kc, use_mfma, stream, tm);
  return hipGetLastError();
}

// ------------------------------------------------------------------- expand
// Sum of the split partials of one rank-space value, in split order.
__device__ __forceinline__ float sum_splits(const float* __restrict__ up, long long q_stride, int nsplit) {
  float part[8];
  float s = 0.f;
  for (int q0 = 0; q0 < nsplit; q0 += 8) {
#pragma unroll
    for (int t = 0; t < 8; ++t) part[t] = (q0 + t < nsplit) ? up[(q0 + t) * q_stride] : 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      if (q0 + t < nsplit) s += part[t];
  }
  return s;
}

constexpr int kExpandRowBatch = 16;   // rank rows of B^T in flight per lane

// 8 consecutive elements of a row, kept packed: one 16-byte chunk for bf16, two for fp32
template <typename T> struct Row8;
template <> struct Row8<uint16_t> {
  uint4 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = ld16(p); }
  __device__ __forceinline__ void zero() { w = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void get(float (&v)[8]) const { unpack8(w, v); }
};
template <> struct Row8<float> {
  uint4 a, b;
  __device__ __forceinline__ void load(const float* p) { a = ld16(p); b = ld16(p + 4); }
  __device__ __forceinline__ void zero() { a = b = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void get(float (&v)[8]) const {
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  }
};

template <typename TW, typename TY, int LTE>
__device__ __forceinline__ void expand_segment(const PoolView& P, const RouteView& R, const UView& U,
                                               TY* __restrict__ y, int ldy, int slot,
                                               const SlotEntry& e, int n, int c0, int L, int p0,
                                               float* usm) {
  const int lane = lane_id();
  const int r = e.rank, dn = P.d[n];
  const int rp = (r + kExpandRowBatch - 1) / kExpandRowBatch * kExpandRowBatch;  // padded rank
  const int col = c0 + lane * kColsPerLane;
  const bool inb = col < dn;
  const int colc = min(col, dn - kColsPerLane);
  const TW* __restrict__ bt = static_cast<const TW*>(P.Bt) + (size_t)slot * P.Rmax * P.D + P.o[n];
  for (int tt = 0; tt < L; tt += LTE) {
    const int nt = min(LTE, L - tt);
    // rank-space values of this token tile: usm[i * rp + j], zero for j >= r
    for (int idx = lane; idx < LTE * rp; idx += 64) {
      const int i = idx / rp, j = idx - i * rp;
      float v = 0.f;
      if (i < nt && j < r) {
        const long long row = U.by_token ? (long long)R.sorted[p0 + tt + i] : (long long)(p0 + tt + i);
        v = sum_splits(U.p + n * U.n_stride + row * U.row_stride + j, U.q_stride, U.nsplit);
      }
      usm[idx] = v;
    }
    // the token rows of y this tile updates (clamped index; only i < nt is stored)
    Row8<TY> yv[LTE];
    TY* yrow[LTE];
#pragma unroll
    for (int i = 0; i < LTE; ++i) {
      yrow[i] = y + (size_t)R.sorted[p0 + tt + min(i, nt - 1)] * ldy + P.o[n] + colc;
      yv[i].load(yrow[i]);
    }
    __syncthreads();
    float acc[LTE][kColsPerLane];
#pragma unroll
    for (int i = 0; i < LTE; ++i)
#pragma unroll
      for (int c = 0; c < kColsPerLane; ++c) acc[i][c] = 0.f;
    for (int jb = 0; jb < rp; jb += kExpandRowBatch) {
      Row8<TW> b[kExpandRowBatch];
#pragma unroll
      for (int jj = 0; jj < kExpandRowBatch; ++jj) {
        const int j = jb + jj;
        b[jj].load(bt + (size_t)(j < r ? j : 0) * P.D + colc);
        if (j >= r) b[jj].zero();
      }
#pragma unroll
      for (int jj = 0; jj < kExpandRowBatch; ++jj) {
        float bf[kColsPerLane];
        b[jj].get(bf);
#pragma unroll
        for (int i = 0; i < LTE; ++i) {
          const float uij = usm[i * rp + jb + jj];
#pragma unroll
          for (int c = 0; c < kColsPerLane; ++c) acc[i][c] = fmaf(bf[c], uij, acc[i][c]);
        }
      }
    }
    if (inb) {
#pragma unroll
      for (int i = 0; i < LTE; ++i) {
        if (i < nt) {
          float v[kColsPerLane];
          yv[i].get(v);
#pragma unroll
          for (int c = 0; c < kColsPerLane; ++c) v[c] = v[c] + e.scale * acc[i][c];
          store8f(yrow[i], v);
        }
      }
    }
    __syncthreads();
  }
}

template <typename TW, typename TY>
__global__ __launch_bounds__(64) void expand_decode_kernel(PoolView P, RouteView R, UView U,
                                                           TY* __restrict__ y, int ldy, int use_mfma) {
  extern __shared__ float usm[];   // [8][Rmax padded to 16]
  const int a = blockIdx.y, ct = blockIdx.x;
  if (a >= R.meta[kMetaActive]) return;
  const int slot = R.active[a];
  const SlotEntry e = P.table[slot];
  if (e.rank == 0 || e.scale == 0.f) return;
  const int L = R.counts[slot];
  if (use_mfma && L >= R.mfma_min) return;
  int n = 0;
  while (n + 1 < P.N && ct >= P.tile0[n + 1]) ++n;
  if (!((e.slice_mask >> n) & 1u)) return;
  const int c0 = (ct - P.tile0[n]) * kTileCols;
  const int p0 = R.offs[slot];
  if (L == 1)
    expand_segment<TW, TY, 1>(P, R, U, y, ldy, slot, e, n, c0, L, p0, usm);
  else if (L == 2)
    expand_segment<TW, TY, 2>(P, R, U, y, ldy, slot, e, n, c0, L, p0, usm);
  else if (L <= 4)
    expand_segment<TW, TY, 4>(P, R, U, y, ldy, slot, e, n, c0, L, p0, usm);
  else
    expand_segment<TW, TY, 8>(P, R, U, y, ldy, slot, e, n, c0, L, p0, usm);
}

hipError_t launch_expand(int wdtype, int ydtype, const PoolView& P, const RouteView& R,
                         const UView& U, void* y, int ldy, int use_mfma, hipStream_t stream,
                         const KTimer& tm) {
  const dim3 grid(P.n_ctiles, P.S);
  const int rp = (P.Rmax + kExpandRowBatch - 1) / kExpandRowBatch * kExpandRowBatch;
  const uint32_t lds = (uint32_t)(8 * rp * sizeof(float));
  if (wdtype == LORA_BF16 && ydtype == LORA_BF16)
    RAX_LAUNCH(tm, (expand_decode_kernel<uint16_t, uint16_t>), grid, dim3(64), lds, stream, P, R, U,
               static_cast<uint16_t*>(y), ldy, use_mfma);
  else if (wdtype == LORA_BF16)
    RAX_LAUNCH(tm, (expand_decode_kernel<uint16_t, float>), grid, dim3(64), lds, stream, P, R, U,
               static_cast<float*>(y), ldy, use_mfma);
  else
    RAX_LAUNCH(tm, (expand_decode_kernel<float, float>), grid, dim3(64), lds, stream, P, R, U,
               static_cast<float*>(y), ldy, use_mfma);
  return hipGetLastError();
}

// ------------------------------------------------- split partials -> caller's u
// u[n][token][j] = sum over q = 0, 1, ... of W[q][n][sorted position][j], for the
// LoRA tokens of non-empty slots and j < rank.
__global__ __launch_bounds__(256) void reduce_splits_kernel(PoolView P, RouteView R, UView W, UView U) {
  const int a = blockIdx.x;
  if (a >= R.meta[kMetaActive]) return;
  const int slot = R.active[a];
  const int r = P.table[slot].rank;
  if (r == 0) return;
  const int L = R.counts[slot], p0 = R.offs[slot];
  const int per_slice = L * r;
  for (int idx = threadIdx.x; idx < P.N * per_slice; idx += blockDim.x) {
    const int n = idx / per_slice, rem = idx - n * per_slice;
    const int i = rem / r, j = rem - i * r;
    const int p = p0 + i;
    const float s = sum_splits(W.p + n * W.n_stride + (long long)p * W.row_stride + j, W.q_stride, W.nsplit);
    U.p[n * U.n_stride + (long long)R.sorted[p] * U.row_stride + j] = s;
  }
}

hipError_t launch_reduce_splits(const PoolView& P, const RouteView& R, const UView& W, const UView& U,
                                hipStream_t stream, const KTimer& tm) {
  RAX_LAUNCH(tm, reduce_splits_kernel, dim3(P.S), dim3(256), 0u, stream, P, R, W, U);
  return hipGetLastError();
}

}  // namespace rax
