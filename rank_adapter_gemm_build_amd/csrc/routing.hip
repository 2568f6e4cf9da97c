// Routing metadata for one batch: a stable counting sort of tokens by adapter slot.
//
// Definition followed (page "第16章 LoRA 适配器热切换", §16.4.2-§16.4.3): sort the tokens
// by slot, count the tokens per slot, take each segment's start offset, so a kernel
// can give every same-slot segment to its own blocks.  Page "TensorRT-LLM 源码完全拆解
// (二十一):LoRA 服务", section "一次 decode 批次的路由": the counts are a bincount and the
// offsets their cumulative sum (a counting sort), the offsets array is one longer than
// the counts, and requests without an adapter go to a sentinel slot after the real ones
// (section "adapter 池:AdapterSlotManager").
//
// One workgroup of 8 waves.  The token range is cut into 8 contiguous chunks, one per
// wave.  Pass 1 builds a per-wave histogram in LDS.  Pass 2 turns it, key by key, into
// the start of each wave's run inside the key's segment, and one wave scans the key
// totals into the segment offsets.  Pass 3 lets every wave walk its chunk in token
// order, 64 tokens at a time; lanes holding the same key are grouped with ballots and
// ranked by lane order, so each key's tokens land in increasing token order: the
// result is the unique stable order, identical on every run.  Every slot also gets a
// 128-byte record (tokens, first sorted position, then its first kRecTokens token ids
// in sorted order), so that a kernel unit of a short segment finds its token rows with
// the same load that tells it the segment; the active-slot list, a 16-byte descriptor
// per active slot (slot, tokens, first sorted position) and the matrix-core tile list
// are compacted in slot order by one wave.
#include <hip/hip_runtime.h>

#include "device_util.h"

namespace rax {

__global__ __launch_bounds__(kRoutingThreads) void routing_kernel(
    const int32_t* __restrict__ ids, int T, int S, int mfma_min, int tile_m, int max_tiles,
    int* __restrict__ counts, int* __restrict__ offs, int* __restrict__ sorted,
    int* __restrict__ active, int4* __restrict__ desc, int4* __restrict__ tiles,
    int* __restrict__ rec, int* __restrict__ meta) {
  extern __shared__ int lds[];
  const int K = S + 1;                         // keys 0..S-1 are slots, S is "no LoRA"
  int* hist = lds;                             // [kRoutingWaves][K]
  int* start = lds + kRoutingWaves * K;        // [K]: counts, then segment starts
  int* misc = start + K;                       // [4]
  int* first = misc + 4;                       // [K]: first token of each segment
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  for (int i = tid; i < kRoutingWaves * K; i += kRoutingThreads) hist[i] = 0;
  if (tid < 4) misc[tid] = 0;
  __syncthreads();

  const int chunk = (T + kRoutingWaves - 1) / kRoutingWaves;
  const int t0 = min(T, w * chunk), t1 = min(T, t0 + chunk);

  // pass 1: per-wave histograms, invalid ids counted
  int invalid = 0;
  for (int t = t0 + lane; t < t1; t += 64) {
    const int id = ids[t];
    const bool ok = id >= 0 && id < S;
    invalid += (!ok && id != -1) ? 1 : 0;
    atomicAdd(&hist[w * K + (ok ? id : S)], 1);
  }
  invalid = wave_sum(invalid);
  if (lane == 0 && invalid) atomicAdd(&misc[0], invalid);
  __syncthreads();

  // pass 2a: per key, exclusive prefix over the waves; key totals
  for (int key = tid; key < K; key += kRoutingThreads) {
    int run = 0;
    for (int ww = 0; ww < kRoutingWaves; ++ww) {
      const int h = hist[ww * K + key];
      hist[ww * K + key] = run;
      run += h;
    }
    start[key] = run;
    counts[key] = run;
  }
  __syncthreads();

  // pass 2b: one wave scans the key totals into segment starts
  if (w == 0) {
    const int per = (K + 63) / 64;
    const int k0 = min(K, lane * per), k1 = min(K, k0 + per);
    int sum = 0;
    for (int key = k0; key < k1; ++key) sum += start[key];
    const int incl = wave_inclusive_scan(sum);
    int run = incl - sum;
    for (int key = k0; key < k1; ++key) {
      const int c = start[key];
      start[key] = run;
      offs[key] = run;
      if (key < S) *reinterpret_cast<int4*>(rec + (size_t)key * kRecInts) = make_int4(c, run, 0, 0);
      run += c;
    }
    if (lane == 63) offs[K] = incl;            // == T
  }
  __syncthreads();

  // pass 3: stable scatter, each wave over its own chunk in token order
  for (int g = t0; g < t1; g += 64) {
    const int t = g + lane;
    const bool valid = t < t1;
    int key = -1;
    if (valid) {
      const int id = ids[t];
      key = (id >= 0 && id < S) ? id : S;
    }
    unsigned long long rem = __ballot(valid);
    while (rem) {
      const int leader = __ffsll(rem) - 1;
      const int k0 = __shfl(key, leader);
      const unsigned long long m = __ballot(valid && key == k0);
      int base = 0;
      if (lane == leader) base = atomicAdd(&hist[w * K + k0], __popcll(m));
      base = __shfl(base, leader);
      if (valid && key == k0) {
        const int rank = __popcll(m & ((1ull << lane) - 1ull));
        sorted[start[k0] + base + rank] = t;
        if (k0 < S && base + rank < kRecTokens) rec[(size_t)k0 * kRecInts + 4 + base + rank] = t;
        if (base + rank == 0) first[k0] = t;
      }
      rem &= ~m;
    }
  }
  __syncthreads();

  // record entries past a segment's tokens repeat its first token (token 0 for an
  // empty segment), so that every entry names a valid row of the batch
  for (int i = tid; i < S * kRecTokens; i += kRoutingThreads) {
    const int key = i / kRecTokens, e = i - key * kRecTokens;
    const int c = start[key + 1] - start[key];
    if (e >= c) rec[(size_t)key * kRecInts + 4 + e] = c > 0 ? first[key] : 0;
  }

  // lists, in slot order: active slots, and tiles of the segments long enough for
  // the matrix-core path (slot, first sorted position, length)
  if (w == 0) {
    int nact = 0, ntiles = 0;
    for (int b = 0; b < S; b += 64) {
      const int key = b + lane;
      const int c = key < S ? start[key + 1] - start[key] : 0;
      const unsigned long long ma = __ballot(c > 0);
      if (c > 0) {
        const int e = nact + __popcll(ma & ((1ull << lane) - 1ull));
        active[e] = key;
        desc[e] = make_int4(key, c, start[key], 0);
      }
      nact += __popcll(ma);
      const int nt = (c > 0 && c >= mfma_min) ? (c + tile_m - 1) / tile_m : 0;
      const int incl = wave_inclusive_scan(nt);
      for (int i = 0; i < nt; ++i) {
        const int e = ntiles + incl - nt + i;
        if (e < max_tiles) tiles[e] = make_int4(key, start[key] + i * tile_m, min(tile_m, c - i * tile_m), 0);
      }
      ntiles += __shfl(incl, 63);
    }
    if (lane == 0) {
      meta[kMetaT] = T;
      meta[kMetaActive] = nact;
      meta[kMetaInvalid] = misc[0];
      meta[kMetaLora] = start[S];
      meta[kMetaTiles] = min(ntiles, max_tiles);
    }
  }
}

hipError_t launch_routing(const int32_t* ids, int T, int S, int mfma_min, int tile_m, int max_tiles,
                          int* counts, int* offs, int* sorted, int* active, int4* desc, int4* tiles,
                          int* rec, int* meta, hipStream_t stream, const KTimer& tm) {
  const size_t lds = (size_t)(kRoutingWaves * (S + 1) + 2 * (S + 1) + 4) * sizeof(int);
  RAX_LAUNCH(tm, routing_kernel, dim3(1), dim3(kRoutingThreads), (uint32_t)lds, stream, ids, T, S,
             mfma_min, tile_m, max_tiles, counts, offs, sorted, active, desc, tiles, rec, meta);
  return hipGetLastError();
}

}  // namespace rax
