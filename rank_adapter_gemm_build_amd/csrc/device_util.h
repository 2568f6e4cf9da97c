// Device helpers for the LoRA kernels: number formats, 16-byte lane loads, the
// wave reduce-scatter and XCD-aware block numbering.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

// Launch through hipExtLaunchKernelGGL when the timer carries events (the events are
// then stamped at the kernel's own start and end), else a plain launch.
#define RAX_LAUNCH(tm, kernel, grid, block, shmem, stream, ...)                                  \
  do {                                                                                         \
    if ((tm).start)                                                                            \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, (tm).start, (tm).stop, 0u,      \
                            __VA_ARGS__);                                                      \
    else                                                                                       \
      hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                     \
  } while (0)

namespace rax {

// Index checks of the debug build (compiled with -DRAXLORA_DEBUG): an index taken from
// memory (a token id, a slot, a sorted position, a workspace row) that falls outside
// its range counts in this translation unit's counter and is replaced by 0, so the
// access stays in bounds and the fault shows as a count read back by
// lora_index_checks.  Other builds take the index as it is, with no code.
#ifdef RAXLORA_DEBUG
static __device__ unsigned int g_index_faults;
__device__ __forceinline__ int checked_index(int i, long long n) {
  if (i >= 0 && i < n) return i;
  atomicAdd(&g_index_faults, 1u);
  return 0;
}
// host accessor of a translation unit's counter (added to the others by lora_index_checks)
#define RAX_INDEX_FAULTS_ACCESSOR(name)                                                       \
  hipError_t index_faults_##name(unsigned int* out, bool reset) {                             \
    hipError_t e = hipMemcpyFromSymbol(out, HIP_SYMBOL(g_index_faults), sizeof(unsigned int)); \
    if (e == hipSuccess && reset) {                                                           \
      const unsigned int zero = 0;                                                            \
      e = hipMemcpyToSymbol(HIP_SYMBOL(g_index_faults), &zero, sizeof(unsigned int));         \
    }                                                                                         \
    return e;                                                                                 \
  }
#else
__device__ __forceinline__ int checked_index(int i, long long) { return i; }
#define RAX_INDEX_FAULTS_ACCESSOR(name)
#endif
#define RAX_IDX(i, n) ::rax::checked_index((i), (n))
// the same check on a variable, as a statement: nothing at all in other builds, so an
// expression's types and the code around it stay exactly as written there
#ifdef RAXLORA_DEBUG
#define RAX_CHECK_VAR(v, n) ((v) = ::rax::checked_index((int)(v), (n)))
#else
#define RAX_CHECK_VAR(v, n) ((void)0)
#endif

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bfloat16
// bfloat16 is the upper half of a float32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float32 -> bfloat16, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// ------------------------------------------------------------ float8 (e4m3)
// OCP e4m3 ("fn"): every value is exactly a bfloat16 value.  The matrix-core shrink
// multiplies e4m3 operands on the FP8 matrix cores; the vector units and the expand
// (whose other operand, u, is not an FP8 value) widen them to bf16 in registers and
// reuse the bf16 arithmetic.  The hardware conversions round to nearest even (checked
// against the format definition on every e4m3 byte and every bf16 value in
// [-448, 448]).
typedef short i16x2_t __attribute__((ext_vector_type(2)));
// 8 e4m3 bytes -> 8 bf16 (one 16-byte chunk): gfx950's byte-pair to bf16-pair
// conversion at scale 1, exact (checked on all 256 bytes against the fp32 conversion)
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint2 w) {
  return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.x, 1.0f, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.x, 1.0f, true)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.y, 1.0f, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.y, 1.0f, true)));
}
// 8 e4m3 bytes -> 8 floats
__device__ __forceinline__ void fp8x8_to_f32(uint2 w, float (&v)[8]) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false);
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
  const auto c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false);
  const auto d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
  v[0] = a[0]; v[1] = a[1]; v[2] = b[0]; v[3] = b[1]; v[4] = c[0]; v[5] = c[1]; v[6] = d[0]; v[7] = d[1];
}
constexpr float kFp8Max = 448.f;
// clamp to [-448, 448] keeping NaN (a comparison with NaN is false), as torch's clamp does
__device__ __forceinline__ float fp8_clamp(float v) { return v > kFp8Max ? kFp8Max : (v < -kFp8Max ? -kFp8Max : v); }
// Clamp of two packed bf16 values to [-448, 448] on their bit patterns, NaN kept: the
// magnitude m (15 bits) is offset by 0x807f modulo 2^16, which puts the non-NaN
// magnitudes 0 .. 0x7f80 at 0x807f .. 0xffff and the NaNs (0x7f81 ..) at 0 .. 0x7e;
// one unsigned minimum against 448's offset magnitude (0x43e0 + 0x807f) then caps
// exactly the finite and infinite magnitudes above 448, and the offset is taken back.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_clamp_fp8max(uint32_t w) {
  const u16x2_t off = {0x807f, 0x807f}, cap = {0xc45f, 0xc45f};
  const u16x2_t m = __builtin_elementwise_min(__builtin_bit_cast(u16x2_t, w & 0x7fff7fffu) + off, cap) - off;
  return (__builtin_bit_cast(uint32_t, m) & 0x7fff7fffu) | (w & 0x80008000u);
}
// FP8 pools' input conversion of 8 bf16 activations (page "TensorRT-LLM 源码完全拆解
// (二十一)", section "前向替换"): clamp to [-448, 448], round to e4m3; 8 bytes, in order.
// The clamp runs on the packed bf16 pairs, and gfx950's bf16-pair conversion (scale 1,
// round to nearest even) writes two bytes per instruction; it alone would turn values
// past 448 into NaN.  Checked on all 65536 bf16 bit patterns: the same bytes as the
// clamp in fp32 followed by the fp32 conversion.
__device__ __forceinline__ uint32_t bf16x4_to_fp8x4(uint32_t lo, uint32_t hi) {
  i16x2_t p = {0, 0};
  p = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(p, __builtin_bit_cast(bf16x2_t, bf16x2_clamp_fp8max(lo)), 1.0f, false);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(p, __builtin_bit_cast(bf16x2_t, bf16x2_clamp_fp8max(hi)), 1.0f, true);
  return __builtin_bit_cast(uint32_t, p);
}
__device__ __forceinline__ uint2 bf16x8_to_fp8x8(uint4 w) {
  return make_uint2(bf16x4_to_fp8x4(w.x, w.y), bf16x4_to_fp8x4(w.z, w.w));
}
// the same conversion, back to bf16 (for the vector units, which multiply in bf16)
__device__ __forceinline__ uint4 bf16x8_to_fp8_grid(uint4 w) { return fp8x8_to_bf16x8(bf16x8_to_fp8x8(w)); }

// One lane's 8 consecutive weight values as a bf16 operand (dot products, MFMA
// fragments): one 16-byte chunk for bf16 (and fp32: 4 values) pools; 8 bytes for
// FP8 pools, widened to 8 bf16 at use.  keep() zeroes a chunk that is not used.
template <typename TW> struct WChunk {
  using type = uint4;
  __device__ __forceinline__ static type load(const TW* p) { return *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ static uint4 widen(const type& c) { return c; }
  __device__ __forceinline__ static type keep(const type& c, bool ok) {
    const uint32_t m = ok ? 0xffffffffu : 0u;
    return make_uint4(c.x & m, c.y & m, c.z & m, c.w & m);
  }
};
template <> struct WChunk<uint8_t> {
  using type = uint2;
  __device__ __forceinline__ static type load(const uint8_t* p) { return *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ static uint4 widen(const type& c) { return fp8x8_to_bf16x8(c); }
  __device__ __forceinline__ static type keep(const type& c, bool ok) {
    const uint32_t m = ok ? 0xffffffffu : 0u;
    return make_uint2(c.x & m, c.y & m);
  }
};

// -------------------------------------------------------------- lane chunks
// Every lane moves 16 bytes per load: 8 bf16 or 4 fp32 elements.
template <typename T> struct Elem;
template <> struct Elem<uint16_t> { static constexpr int kPerChunk = 8; };
template <> struct Elem<float> { static constexpr int kPerChunk = 4; };
template <> struct Elem<uint8_t> { static constexpr int kPerChunk = 8; };   // 8-byte chunks, widened to bf16

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
// v if ok else zero, component-wise (a ternary on the whole vector makes the compiler
// pick between two stack copies through scratch memory)
__device__ __forceinline__ uint4 keep_if(uint4 v, bool ok) {
  const uint32_t m = ok ? 0xffffffffu : 0u;
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}
// 16-byte chunk -> 8 floats (bf16 pairs), or 4 floats into two chunks for fp32
__device__ __forceinline__ void unpack8(uint4 w, float (&v)[8]) {
  v[0] = __uint_as_float(w.x << 16); v[1] = __uint_as_float(w.x & 0xffff0000u);
  v[2] = __uint_as_float(w.y << 16); v[3] = __uint_as_float(w.y & 0xffff0000u);
  v[4] = __uint_as_float(w.z << 16); v[5] = __uint_as_float(w.z & 0xffff0000u);
  v[6] = __uint_as_float(w.w << 16); v[7] = __uint_as_float(w.w & 0xffff0000u);
}
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// acc + <a, b> over one 16-byte chunk
__device__ __forceinline__ float chunk_dot(uint4 a, uint4 b, float acc, uint16_t) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x), __builtin_bit_cast(bf16x2_t, b.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y), __builtin_bit_cast(bf16x2_t, b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z), __builtin_bit_cast(bf16x2_t, b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w), __builtin_bit_cast(bf16x2_t, b.w), acc, false);
  return acc;
}
__device__ __forceinline__ float chunk_dot(uint4 a, uint4 b, float acc, float) {
  acc = fmaf(__uint_as_float(a.x), __uint_as_float(b.x), acc);
  acc = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
  acc = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
  acc = fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
  return acc;
}

// 8 consecutive elements starting at p (16-byte aligned) as floats; zeros if !ok
__device__ __forceinline__ void load8f(const uint16_t* p, bool ok, float (&v)[8]) {
  uint4 w = ok ? ld16(p) : make_uint4(0, 0, 0, 0);
  v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}
__device__ __forceinline__ void load8f(const float* p, bool ok, float (&v)[8]) {
  uint4 a = ok ? ld16(p) : make_uint4(0, 0, 0, 0);
  uint4 b = ok ? ld16(p + 4) : make_uint4(0, 0, 0, 0);
  v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
  v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
}
__device__ __forceinline__ void store8f(uint16_t* p, const float (&v)[8]) {
  st16(p, make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                     pack_bf16x2(v[6], v[7])));
}
__device__ __forceinline__ void store8f(float* p, const float (&v)[8]) {
  st16(p, make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])));
  st16(p + 4, make_uint4(__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])));
}

// ------------------------------------------------------------ wave reductions
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Reduce-scatter across the 64 lanes of a wave: on entry every lane holds 64
// partial values v[0..64); on exit v[0] of lane l holds the sum over all lanes of
// entry value l.  Six exchange stages with partners 32, 16, 8, 4, 2, 1 lanes away:
// at the stage of width H a lane keeps the half of its values whose index bit H
// equals its own lane bit H and adds the partner's copy of that half, so the work
// halves at every stage (63 exchanges in all instead of 64 six-step reductions).
// The two cross-row stages use the gfx950 lane-swap instructions (v_permlane32_swap
// swaps the upper 32 lanes of its first operand with the lower 32 lanes of its
// second; v_permlane16_swap does the same for odd and even 16-lane rows), so one
// swap hands each lane both addends; the in-row stages use DPP lane moves (row
// mirror, half-row mirror, and two quad permutations: any pairing across the two
// halves of the group works, all four are involutions).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int H>
__device__ __forceinline__ void reduce_scatter_stage(float (&v)[64], int lane) {
#if defined(RAX_REDUCE_WITH_SHUFFLES)
  const bool upper = (lane & H) != 0;
#pragma unroll
  for (int i = 0; i < H; ++i) {
    const float send = upper ? v[i] : v[i + H];
    const float keep = upper ? v[i + H] : v[i];
    v[i] = keep + __shfl_xor(send, H);
  }
#else
  if constexpr (H == 32 || H == 16) {
#pragma unroll
    for (int i = 0; i < H; ++i) {
      const auto r = (H == 32)
          ? __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + H]), false, false)
          : __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + H]), false, false);
      v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
  } else {
    constexpr int CTRL = H == 8 ? 0x140 : H == 4 ? 0x141 : H == 2 ? 0x4E : 0xB1;
    const bool upper = (lane & H) != 0;
#pragma unroll
    for (int i = 0; i < H; ++i) {
      const float send = upper ? v[i] : v[i + H];
      const float keep = upper ? v[i + H] : v[i];
      v[i] = keep + dpp_move<CTRL>(send);
    }
  }
#endif
}

__device__ __forceinline__ void reduce_scatter64(float (&v)[64]) {
  const int lane = lane_id();
  reduce_scatter_stage<32>(v, lane);
  reduce_scatter_stage<16>(v, lane);
  reduce_scatter_stage<8>(v, lane);
  reduce_scatter_stage<4>(v, lane);
  reduce_scatter_stage<2>(v, lane);
  reduce_scatter_stage<1>(v, lane);
}

// Keep the compiler from moving instructions across this point: used between a
// phase that issues a batch of independent loads and the phase that consumes them,
// so all of the batch is in flight before the first wait.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Inclusive prefix sum over the 64 lanes, with all lanes active, by data-parallel
// primitives (DPP) that read neighbouring lanes' registers without a trip through
// the LDS crossbar: shifts right by 1, 2, 4, 8 within each row of 16 lanes (lanes
// with no source add 0), then row 0's total into row 1 and row 2's into row 3
// (row_bcast:15), then lanes 0..31's total into rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15, rows 1 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31, rows 2 and 3
  return x;
}

// LDS writes of this wave visible to all of its lanes (wave-scope fences around a
// wave barrier; no workgroup barrier needed for one-wave workgroups)
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d);
  return x;
}

// A rank-space value finished from its k-split partial sums p[0], p[stride], ...:
// added in split order, starting from split 0, wherever it is computed (the expand
// and the standalone shrink's finishing pass), so the two agree bitwise.  All loads
// are issued before the first addition.
__device__ __forceinline__ float sum_splits(const float* __restrict__ p, long long stride, int nsplit) {
  float pv[kMaxSplit];
#pragma unroll
  for (int q = 0; q < kMaxSplit; ++q)
    if (q < nsplit) pv[q] = p[q * stride];
  float v = pv[0];
#pragma unroll
  for (int q = 1; q < kMaxSplit; ++q)
    if (q < nsplit) v += pv[q];
  return v;
}

// Workgroups are handed to the 8 XCDs round-robin (workgroup b runs on XCD b % 8),
// and each XCD has its own L2.  The renumbering below deals logical units to the
// XCDs in groups of g consecutive units (group q to XCD q % 8), so units that read
// the same weights or rows (neighbours in the numbering) share one L2, while work
// spread unevenly along the numbering still lands on every XCD.  It is a bijection
// on [0, grid) when grid is a multiple of 8 * g; g = 1 is the identity.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_logical_block(int b, int g) {
  const int x = b % kXcds, i = b / kXcds;
  return ((i / g) * kXcds + x) * g + i % g;
}

}  // namespace rax
