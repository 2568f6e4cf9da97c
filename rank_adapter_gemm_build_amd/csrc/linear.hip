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
// launches whatever its mix.
//
// Decode shrink unit (one wave: active slot a, k split s, 16 rank rows, token tiles).
// Lane l owns the 16-byte chunks at k offsets (s + nsplit * m) * 64 * E + l * E
// (E = 8 bf16 or 4 fp32), so every row of A streams from HBM as contiguous 1 KB
// requests and is read once per token tile, not once per token; the x rows of the
// tile are gathered through sorted_ids, each lane loading exactly the k-slice it
// multiplies.  The 16 rows x 4 tokens = 64 lane partial sums are finished by one
// reduce-scatter across the wave, after which lane l holds output l, the partial sum
// of split s.  Splitting k over waves gives a short decode batch enough waves to
// keep HBM busy; the partials of a value are added in split order where they are
// read (the expand), so the result does not depend on timing and no atomics or
// cross-workgroup fences are needed.
//
// Decode expand item (one wave: column tile of one slice, active slot a, token tiles).
// Lanes own 8 consecutive output columns, so each rank-major row of B^T streams as one
// contiguous 1 KB request; the tile's rank-space values (split partials added) are
// staged in the wave's own LDS slice and read as broadcasts; the contraction over the rank stays in registers.
// The epilogue updates the token's row of y at its original index (no permutation
// pass; page "TensorRT-LLM 源码完全拆解(二十一)", section "前向替换", restores the order
// with index_copy_ instead), adding s * acc in fp32, one rounding.
//
// Every unit starts from the routing's 16-byte slot descriptor (slot, tokens, first
// sorted position), so its dependent loads are: descriptor, then slot table and token
// ids, then the operands.  Operand loads are unconditional (addresses clamped into the
// operand, unused values replaced by zero) and issued as one batch before the math.
#include <hip/hip_runtime.h>

#include "device_util.h"
#include "mfma_tiles.h"

namespace rax {

constexpr int kShrinkRows = 16;   // rank rows per decode shrink unit
constexpr int kShrinkTok = 4;     // tokens per decode shrink pass
constexpr int kExpandTok = 4;     // tokens per decode expand pass (at most)
constexpr int kExpandRowBatch = 8;    // rank rows of B^T in flight per lane

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ------------------------------------------------------------ decode shrink
template <typename T>
__device__ __forceinline__ void shrink_decode_unit(const PoolView& P, const RouteView& R,
                                                   const T* __restrict__ x, int ldx, const UView& U,
                                                   const Plan& plan, int unit) {
  constexpr int E = Elem<T>::kPerChunk;
  constexpr int CW = 64 * E;         // k elements of one wave-wide chunk step
  const int tg = unit % plan.ntg;
  int rest = unit / plan.ntg;
  const int sp = rest % plan.nsplit;
  rest /= plan.nsplit;
  const int rb = rest % plan.nrb, a = rest / plan.nrb;
  if (a >= R.S) return;
  const int4 d = R.desc[a];
  if (a >= R.meta[kMetaActive]) return;
  const int slot = d.x, L = d.y, p0 = d.z;
  if (plan.use_mfma && L >= R.mfma_min) return;   // long segment: matrix-core blocks
  const int tt0 = tg * kShrinkTok;
  if (tt0 >= L) return;
  const SlotEntry e = P.table[slot];
  const int r = e.rank, F = P.N * r, fb = rb * kShrinkRows;
  if (r == 0 || fb >= F) return;                   // all of the above is uniform per wave
  const int lane = lane_id();
  const T* __restrict__ Aslot = static_cast<const T*>(P.A) + (size_t)slot * P.N * P.Rmax * P.k;
  const T* arow[kShrinkRows];
  bool rval[kShrinkRows];
  {
    int n = fb / r, j = fb - (fb / r) * r;
#pragma unroll
    for (int rr = 0; rr < kShrinkRows; ++rr) {
      rval[rr] = fb + rr < F;
      arow[rr] = Aslot + ((size_t)(rval[rr] ? n : 0) * P.Rmax + (rval[rr] ? j : 0)) * P.k;
      if (++j == r) { j = 0; ++n; }
    }
  }
  // this lane's output after the reduce-scatter: row fb + lane / 4, token lane % 4
  const int orr = lane / kShrinkTok, oi = lane - orr * kShrinkTok, of = fb + orr;
  const int on = of < F ? of / r : 0, oj = of < F ? of - on * r : 0;
  float* __restrict__ uo = U.p + sp * U.split_stride + on * U.n_stride + oj;

  for (int tt = tt0; tt < L; tt += plan.ntg * kShrinkTok) {
    const int nt = min(kShrinkTok, L - tt);
    const T* xrow[kShrinkTok];
#pragma unroll
    for (int i = 0; i < kShrinkTok; ++i) xrow[i] = x + (size_t)R.sorted[p0 + tt + min(i, nt - 1)] * ldx;
    float acc[64];
#pragma unroll
    for (int m = 0; m < 64; ++m) acc[m] = 0.f;
    for (int c = 0; c < plan.ns; ++c) {
      const int col = (sp + plan.nsplit * c) * CW + lane * E;
      const bool inb = col < P.k;
      const int colc = min(col, P.k - E);
      // the x chunks and all 16 A rows of this chunk step in flight before the first product
      uint4 xv[kShrinkTok], av[kShrinkRows];
#pragma unroll
      for (int i = 0; i < kShrinkTok; ++i) xv[i] = keep_if(ld16(xrow[i] + colc), i < nt && inb);
#pragma unroll
      for (int rr = 0; rr < kShrinkRows; ++rr) av[rr] = keep_if(ld16(arow[rr] + colc), rval[rr] && inb);
      sched_fence();
#pragma unroll
      for (int rr = 0; rr < kShrinkRows; ++rr)
#pragma unroll
        for (int i = 0; i < kShrinkTok; ++i)
          acc[rr * kShrinkTok + i] = chunk_dot(av[rr], xv[i], acc[rr * kShrinkTok + i], T());
    }
    reduce_scatter64(acc);
    if (of < F && oi < nt) {
      const long long row = U.by_token ? (long long)R.sorted[p0 + tt + oi] : (long long)(p0 + tt + oi);
      uo[row * U.row_stride] = acc[0];
    }
  }
}

template <typename T>
__global__ __launch_bounds__(512) void shrink_kernel(PoolView P, RouteView R, const T* __restrict__ x,
                                                     int ldx, UView U, Plan plan) {
  __shared__ float smem[kShrinkMfmaSmemFloats];
  const int bw = 4 * plan.kq;                      // waves per block
  if ((int)blockIdx.x < plan.n_dec_blocks) {
    shrink_decode_unit<T>(P, R, x, ldx, U, plan, blockIdx.x * bw + (threadIdx.x >> 6));
    return;
  }
  if constexpr (sizeof(T) == 2) {
    const int ntiles = R.meta[kMetaTiles];
    for (int tile = blockIdx.x - plan.n_dec_blocks; tile < ntiles; tile += plan.tile_slots)
      shrink_mfma_tile(P, R, x, ldx, U, plan.kq, tile, smem);
  }
}

template <typename T>
static void launch_shrink_t(const PoolView& P, const RouteView& R, const T* x, int ldx, const UView& U,
                            const Plan& plan, hipStream_t stream, const KTimer& tm) {
  const int blocks = plan.n_dec_blocks + (plan.use_mfma ? plan.tile_slots : 0);
  RAX_LAUNCH(tm, shrink_kernel<T>, dim3(blocks), dim3(256 * plan.kq), 0u, stream, P, R, x, ldx, U, plan);
}

hipError_t launch_shrink(int wdtype, const PoolView& P, const RouteView& R, const void* x, int ldx,
                         const UView& U, const Plan& plan, hipStream_t stream, const KTimer& tm) {
  const int cw = 64 * (wdtype == LORA_BF16 ? 8 : 4);
  const int chunks = (P.k + cw - 1) / cw;
  if (plan.kq < 1 || plan.kq > 2 || plan.nsplit < 1 || plan.nsplit > kMaxSplit || plan.nsplit > U.nsplit ||
      plan.ns < 1 || plan.nsplit * plan.ns < chunks || plan.ntg < 1 || plan.nrb < 1 ||
      (plan.use_mfma && (wdtype != LORA_BF16 || plan.tile_slots < 1)))
    return hipErrorInvalidValue;
  if (wdtype == LORA_BF16)
    launch_shrink_t(P, R, static_cast<const uint16_t*>(x), ldx, U, plan, stream, tm);
  else
    launch_shrink_t(P, R, static_cast<const float*>(x), ldx, U, plan, stream, tm);
  return hipGetLastError();
}

// Finished u of a standalone shrink: for every LoRA token of an active slot, the
// partials of the workspace W summed in split order (matrix-core segments: split 0)
// into the caller's buffer U, by token.  One block per active slot.
__global__ __launch_bounds__(256) void finish_u_kernel(PoolView P, RouteView R, UView W, UView U, Plan plan) {
  const int a = blockIdx.x;
  if (a >= R.meta[kMetaActive]) return;
  const int4 d = R.desc[a];
  const int slot = d.x, L = d.y, p0 = d.z;
  const SlotEntry e = P.table[slot];
  const int r = e.rank;
  if (r == 0) return;
  const int ns = (plan.use_mfma && L >= R.mfma_min) ? 1 : W.nsplit;
  const int per_tok = P.N * r;
  for (int idx = threadIdx.x; idx < L * per_tok; idx += blockDim.x) {
    const int t = idx / per_tok, f = idx - t * per_tok, n = f / r, j = f - n * r;
    const float v = sum_splits(W.p + n * W.n_stride + (long long)(p0 + t) * W.row_stride + j, W.split_stride, ns);
    U.p[n * U.n_stride + (long long)R.sorted[p0 + t] * U.row_stride + j] = v;
  }
}

hipError_t launch_finish_u(const PoolView& P, const RouteView& R, const UView& W, const UView& U,
                           const Plan& plan, hipStream_t stream, const KTimer& tm) {
  if (W.nsplit < 1 || W.nsplit > kMaxSplit || W.by_token || !U.by_token) return hipErrorInvalidValue;
  RAX_LAUNCH(tm, finish_u_kernel, dim3(R.S), dim3(256), 0u, stream, P, R, W, U, plan);
  return hipGetLastError();
}

// ------------------------------------------------------------ decode expand
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

// LDS floats per wave for the decode expand: kExpandTok tokens x the padded rank
__host__ __device__ constexpr int expand_usm_floats(int Rmax) {
  return kExpandTok * ((Rmax + kExpandRowBatch - 1) / kExpandRowBatch * kExpandRowBatch);
}

template <typename TW, typename TY, int LTE>
__device__ __forceinline__ void expand_decode_tiles(const PoolView& P, const RouteView& R, const UView& U,
                                                    TY* __restrict__ y, int ldy, int slot,
                                                    const SlotEntry& e, int n, int c0, int L, int p0,
                                                    int tg, int ntg, float* __restrict__ usm) {
  const int lane = lane_id();
  const int r = e.rank, dn = P.d[n];
  const int rp = (r + kExpandRowBatch - 1) / kExpandRowBatch * kExpandRowBatch;  // padded rank
  const int col = c0 + lane * kColsPerLane;
  const bool inb = col < dn;
  const int colc = min(col, dn - kColsPerLane);
  const TW* __restrict__ bt = static_cast<const TW*>(P.Bt) + (size_t)slot * P.Rmax * P.D + P.o[n] + colc;
  for (int tt = tg * LTE; tt < L; tt += ntg * LTE) {
    const int nt = min(LTE, L - tt);
    // first batch of B^T rows in flight together with y and the rank-space values
    Row8<TW> b[kExpandRowBatch];
#pragma unroll
    for (int jj = 0; jj < kExpandRowBatch; ++jj) {
      b[jj].load(bt + (size_t)(jj < r ? jj : 0) * P.D);
      if (jj >= r) b[jj].zero();
    }
    // the token rows of y this tile updates (clamped index; only i < nt is stored)
    Row8<TY> yv[LTE];
    TY* yrow[LTE];
#pragma unroll
    for (int i = 0; i < LTE; ++i) {
      yrow[i] = y + (size_t)R.sorted[p0 + tt + min(i, nt - 1)] * ldy + P.o[n] + colc;
      yv[i].load(yrow[i]);
    }
    // rank-space values of this token tile: usm[i * rp + j], zero past the rank
    for (int idx = lane; idx < LTE * rp; idx += 64) {
      const int i = idx / rp, j = idx - i * rp;
      const bool ok = i < nt && j < r;
      const int ic = ok ? i : 0, jc = ok ? j : 0;
      const long long row = U.by_token ? (long long)R.sorted[p0 + tt + ic] : (long long)(p0 + tt + ic);
      const float v = sum_splits(U.p + n * U.n_stride + row * U.row_stride + jc, U.split_stride, U.nsplit);
      usm[idx] = ok ? v : 0.f;
    }
    wave_lds_sync();
    float acc[LTE][kColsPerLane];
#pragma unroll
    for (int i = 0; i < LTE; ++i)
#pragma unroll
      for (int c = 0; c < kColsPerLane; ++c) acc[i][c] = 0.f;
    for (int jb = 0; jb < rp; jb += kExpandRowBatch) {
      if (jb > 0) {
#pragma unroll
        for (int jj = 0; jj < kExpandRowBatch; ++jj) {
          const int j = jb + jj;
          b[jj].load(bt + (size_t)(j < r ? j : 0) * P.D);
          if (j >= r) b[jj].zero();
        }
        sched_fence();
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
    wave_lds_sync();
  }
}

template <typename TW, typename TY>
__device__ __forceinline__ void expand_decode_item(const PoolView& P, const RouteView& R, const UView& U,
                                                   TY* __restrict__ y, int ldy, const Plan& plan,
                                                   int item, float* __restrict__ usm) {
  const int ct = item % P.n_ctiles;
  const int rest = item / P.n_ctiles;
  const int tg = rest % plan.ntg, a = rest / plan.ntg;
  if (a >= R.S) return;
  const int4 d = R.desc[a];
  if (a >= R.meta[kMetaActive]) return;
  const int slot = d.x, L = d.y, p0 = d.z;
  if (plan.use_mfma && L >= R.mfma_min) return;
  const int LTE = L == 1 ? 1 : L == 2 ? 2 : kExpandTok;
  if (tg * LTE >= L) return;
  const SlotEntry e = P.table[slot];
  if (e.rank == 0 || e.scale == 0.f) return;
  int n = 0;
  while (n + 1 < P.N && ct >= P.tile0[n + 1]) ++n;
  if (!((e.slice_mask >> n) & 1u)) return;
  const int c0 = (ct - P.tile0[n]) * kTileCols;
  if (L == 1)
    expand_decode_tiles<TW, TY, 1>(P, R, U, y, ldy, slot, e, n, c0, L, p0, tg, plan.ntg, usm);
  else if (L == 2)
    expand_decode_tiles<TW, TY, 2>(P, R, U, y, ldy, slot, e, n, c0, L, p0, tg, plan.ntg, usm);
  else
    expand_decode_tiles<TW, TY, kExpandTok>(P, R, U, y, ldy, slot, e, n, c0, L, p0, tg, plan.ntg, usm);
}

template <typename TW, typename TY, int KS>
__global__ __launch_bounds__(256) void expand_kernel(PoolView P, RouteView R, UView U,
                                                     TY* __restrict__ y, int ldy, Plan plan) {
  extern __shared__ float smem[];
  if ((int)blockIdx.x < plan.n_dec_blocks) {
    const int w = threadIdx.x >> 6;
    expand_decode_item<TW, TY>(P, R, U, y, ldy, plan, blockIdx.x * 4 + w,
                               smem + w * expand_usm_floats(P.Rmax));
    return;
  }
  if constexpr (sizeof(TW) == 2) {
    const int mb = blockIdx.x - plan.n_dec_blocks;
    const int ng = (P.n_mblocks + kMfmaColBlocksPerGroup - 1) / kMfmaColBlocksPerGroup;
    const int cg = mb % ng, slot0 = mb / ng;
    const int ntiles = R.meta[kMetaTiles];
    for (int tile = slot0; tile < ntiles; tile += plan.tile_slots)
      expand_mfma_tile<TY, KS>(P, R, U, y, ldy, cg * kMfmaColBlocksPerGroup, tile, smem);
  }
}

template <typename TY>
static void launch_expand_bf16(int ks, dim3 grid, uint32_t lds, hipStream_t stream, const PoolView& P,
                               const RouteView& R, const UView& U, TY* y, int ldy, const Plan& plan,
                               const KTimer& tm) {
  switch (ks) {
    case 1: RAX_LAUNCH(tm, (expand_kernel<uint16_t, TY, 1>), grid, dim3(256), lds, stream, P, R, U, y, ldy, plan); break;
    case 2: RAX_LAUNCH(tm, (expand_kernel<uint16_t, TY, 2>), grid, dim3(256), lds, stream, P, R, U, y, ldy, plan); break;
    case 4: RAX_LAUNCH(tm, (expand_kernel<uint16_t, TY, 4>), grid, dim3(256), lds, stream, P, R, U, y, ldy, plan); break;
    default: RAX_LAUNCH(tm, (expand_kernel<uint16_t, TY, 8>), grid, dim3(256), lds, stream, P, R, U, y, ldy, plan); break;
  }
}

size_t expand_smem_bytes(int wdtype, int Rmax, int use_mfma) {
  size_t f = (size_t)4 * expand_usm_floats(Rmax);
  if (use_mfma && wdtype == LORA_BF16 && (size_t)kExpandMfmaSmemFloats > f) f = kExpandMfmaSmemFloats;
  return f * sizeof(float);
}

hipError_t launch_expand(int wdtype, int ydtype, const PoolView& P, const RouteView& R,
                         const UView& U, void* y, int ldy, const Plan& plan, hipStream_t stream,
                         const KTimer& tm) {
  if (plan.ntg < 1 || (plan.use_mfma && (wdtype != LORA_BF16 || plan.tile_slots < 1)))
    return hipErrorInvalidValue;
  const int ng = (P.n_mblocks + kMfmaColBlocksPerGroup - 1) / kMfmaColBlocksPerGroup;
  const int blocks = plan.n_dec_blocks + (plan.use_mfma ? ng * plan.tile_slots : 0);
  const dim3 grid(blocks);
  const uint32_t lds = (uint32_t)expand_smem_bytes(wdtype, P.Rmax, plan.use_mfma);
  if (wdtype == LORA_BF16) {
    // rank steps of 32 the matrix-core part keeps in registers: Rk / 32 rounded up to a power of 2
    const int ks = P.Rk <= 32 ? 1 : P.Rk <= 64 ? 2 : P.Rk <= 128 ? 4 : 8;
    if (ydtype == LORA_BF16)
      launch_expand_bf16<uint16_t>(ks, grid, lds, stream, P, R, U, static_cast<uint16_t*>(y), ldy, plan, tm);
    else
      launch_expand_bf16<float>(ks, grid, lds, stream, P, R, U, static_cast<float*>(y), ldy, plan, tm);
  } else {
    RAX_LAUNCH(tm, (expand_kernel<float, float, 1>), grid, dim3(256), lds, stream, P, R, U,
               static_cast<float*>(y), ldy, plan);
  }
  return hipGetLastError();
}

}  // namespace rax
