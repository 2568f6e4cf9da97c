// Registration: write one adapter slice into its pool slot.
//
// Page "vLLM LoRA 实现深度解析" §5.3: activating an adapter copies its lora_a / lora_b
// into the slot's rows of the stacked buffers (set_lora(index, A, B)), zeroing rows it
// does not fill; §1 "推理优化:预合并 scaling": optionally B is multiplied by the scale
// once at this point.  Page "TensorRT-LLM 源码完全拆解(二十一)", section "一次 decode 批次
// 的路由": an empty slot must read as rank 0, so the slot-table entry (rank, scale,
// present slices) is written last, in stream order after the data.
#include <hip/hip_runtime.h>

#include "device_util.h"

namespace rax {

__device__ __forceinline__ float to_f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ void from_f(float f, uint16_t& v) { v = (uint16_t)f32_to_bf16(f); }
__device__ __forceinline__ void from_f(float f, float& v) { v = f; }
// FP8 pools: the scale fold of page "TensorRT-LLM 源码完全拆解(二十一)" (FP8 weights stay
// FP8; the scale is applied in bf16 and the result clamped back into the FP8 range):
// the fp32 product is rounded to bf16, clamped to [-448, 448] and rounded to e4m3
__device__ __forceinline__ float to_f(uint8_t v) { return __builtin_amdgcn_cvt_pk_f32_fp8((int)v, false)[0]; }
__device__ __forceinline__ void from_f(float f, uint8_t& v) {
  const float b = __uint_as_float(f32_to_bf16(f) << 16);
  const float c = fp8_clamp(b);
  v = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(c, 0.f, 0, false) & 0xff);
}

// A block [Rmax][k]: rows < rank copied from src [rank][k] (NULL -> zeros), the rest zero.
template <typename T>
__global__ void pack_a_kernel(const T* __restrict__ src, T* __restrict__ dst, long long n_src,
                              long long n_all) {
  for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < n_all;
       e += (long long)gridDim.x * blockDim.x)
    dst[e] = (src != nullptr && e < n_src) ? src[e] : T(0);
}

// B slice [d][rank] -> Bt rows [Rmax][D] (columns [0, d) of the slice) and Bk
// [d][rs] (rs = rank rounded up to 8); entries j >= rank are zero.  Optional fold of
// the scale: one fp32 product rounded once to T.
template <typename T>
__global__ void pack_b_kernel(const T* __restrict__ src, T* __restrict__ bt, T* __restrict__ bk,
                              int rank, int Rmax, int rs, int d, int D, float scale, int premultiply) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= d) return;
  const int jn = Rmax > rs ? Rmax : rs;
  for (int j = 0; j < jn; ++j) {
    T v = T(0);
    if (src != nullptr && j < rank) {
      v = src[(long long)i * rank + j];
      if (premultiply) from_f(scale * to_f(v), v);
    }
    if (j < Rmax) bt[(long long)j * D + i] = v;
    if (j < rs) bk[(long long)i * rs + j] = v;
  }
}

// Embedding pools: A [rank][V] (columns by vocabulary id) -> [V][Rmax], so a token's
// r values are one contiguous row (the get_rows layout); entries j >= rank zero.
template <typename T>
__global__ void pack_a_t_kernel(const T* __restrict__ src, T* __restrict__ dst, int rank, int Rmax, long long V) {
  const long long n_all = V * Rmax;
  for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < n_all;
       e += (long long)gridDim.x * blockDim.x) {
    const long long v = e / Rmax;
    const int j = (int)(e - v * Rmax);
    dst[e] = (src != nullptr && j < rank) ? src[(long long)j * V + v] : T(0);
  }
}

__global__ void set_slot_kernel(SlotEntry* table, int slot, SlotEntry entry) { table[slot] = entry; }

template <typename T>
static hipError_t pack(const void* A_src, const void* B_src, void* A_dst, void* Bt_dst, void* Bk_dst,
                       int rank, int Rmax, int Rk, int k, int d, int D, float scale, int premultiply,
                       int a_by_row, hipStream_t stream) {
  const long long n_all = (long long)Rmax * k, n_src = (long long)rank * k;
  const int blocks_a = (int)((n_all + 255) / 256 < 4096 ? (n_all + 255) / 256 : 4096);
  if (a_by_row)
    hipLaunchKernelGGL(pack_a_t_kernel<T>, dim3(blocks_a), dim3(256), 0, stream,
                       static_cast<const T*>(A_src), static_cast<T*>(A_dst), rank, Rmax, (long long)k);
  else
    hipLaunchKernelGGL(pack_a_kernel<T>, dim3(blocks_a), dim3(256), 0, stream,
                       static_cast<const T*>(A_src), static_cast<T*>(A_dst), n_src, n_all);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(pack_b_kernel<T>, dim3((d + 255) / 256), dim3(256), 0, stream,
                     static_cast<const T*>(B_src), static_cast<T*>(Bt_dst), static_cast<T*>(Bk_dst),
                     rank, Rmax, bk_stride(rank), d, D, scale, premultiply);
  return hipGetLastError();
}

hipError_t launch_pack_slice(int wdtype, const void* A_src, const void* B_src, void* A_dst,
                             void* Bt_dst, void* Bk_dst, int rank, int Rmax, int Rk, int k, int d,
                             int D, float scale, int premultiply, int a_by_row, hipStream_t stream) {
  if (wdtype == LORA_BF16)
    return pack<uint16_t>(A_src, B_src, A_dst, Bt_dst, Bk_dst, rank, Rmax, Rk, k, d, D, scale,
                          premultiply, a_by_row, stream);
  if (wdtype == LORA_FP8E4M3)
    return pack<uint8_t>(A_src, B_src, A_dst, Bt_dst, Bk_dst, rank, Rmax, Rk, k, d, D, scale,
                         premultiply, a_by_row, stream);
  return pack<float>(A_src, B_src, A_dst, Bt_dst, Bk_dst, rank, Rmax, Rk, k, d, D, scale,
                     premultiply, a_by_row, stream);
}

hipError_t launch_set_slot(SlotEntry* table, int slot, SlotEntry entry, hipStream_t stream) {
  hipLaunchKernelGGL(set_slot_kernel, dim3(1), dim3(1), 0, stream, table, slot, entry);
  return hipGetLastError();
}

}  // namespace rax
