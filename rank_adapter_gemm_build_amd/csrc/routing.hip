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
// Sequences of several tokens (tokens_per_seq = p > 1, the linear-tree verification
// batch of speculative decoding): the ids are per sequence and token t takes the id of
// sequence t / p; a stable sort of the tokens is then the page's expansion of the
// sorted sequences, sequence q's tokens q p .. q p + p - 1 in order (section
// "一次 decode 批次的路由": token_sorted_ids and counts times tokens_per_seq).
//
// One workgroup of 8 waves (16 for large batches).  All ids are read once, in
// one batch of independent loads, and kept in LDS as 16-bit keys (when the batch
// fits; else each pass reads them again).  The token range is cut into contiguous
// chunks, one per wave.  Pass 1 builds a per-wave histogram in LDS.  Pass 2 turns
// it, key by key, into the start of each wave's run inside the key's segment, and
// one wave scans the key totals into the segment offsets.  Pass 3 lets every wave
// walk its chunk in token order, 64 tokens at a time; each lane finds the lanes
// holding its key with one ballot per key bit (the intersection of the matching bit
// masks) and ranks itself by lane order, so each key's tokens land in increasing
// token order: the result is the unique stable
// order, identical on every run.  Every slot also gets a
// 128-byte record (tokens, first sorted position, then its first kRecTokens token ids
// in sorted order), so that a kernel unit of a short segment finds its token rows with
// the same load that tells it the segment; the active-slot list, a 16-byte descriptor
// per active slot (slot, tokens, first sorted position) and the matrix-core tile list
// are compacted in slot order by one wave.
#include <hip/hip_runtime.h>

#include "device_util.h"
#include "route_wave.h"

namespace rax {

__global__ __launch_bounds__(kRoutingMaxThreads) void routing_kernel(
    const int32_t* __restrict__ ids, int T, int tps, int S, int mfma_min, int tile_m, int max_tiles, int stage,
    int* __restrict__ counts, int* __restrict__ offs, int* __restrict__ sorted,
    int* __restrict__ active, int4* __restrict__ desc, int4* __restrict__ tiles,
    int* __restrict__ rec, int* __restrict__ meta) {
  extern __shared__ int lds[];
  const int NW = blockDim.x / 64, NT = blockDim.x;   // waves and threads of the workgroup
  const int K = S + 1;                         // keys 0..S-1 are slots, S is "no LoRA"
  int* hist = lds;                             // [NW][K]
  int* start = lds + NW * K;                   // [K]: counts, then segment starts
  int* misc = start + K;                       // [4]
  int* first = misc + 4;                       // [K]: first token of each segment
  uint16_t* key16 = reinterpret_cast<uint16_t*>(first + K);   // [T] when staged
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int nbits = 0;
  while ((1 << nbits) <= S) ++nbits;           // keys 0..S fit in nbits bits

  for (int i = tid; i < NW * K; i += NT) hist[i] = 0;
  if (tid < 4) misc[tid] = 0;
  // all ids in batches of kRoutingStageBatch independent loads per thread; invalid ids counted
  int invalid = 0;
  if (stage) {
    for (int b0 = 0; b0 < T; b0 += NT * kRoutingStageBatch) {
      int v[kRoutingStageBatch];
#pragma unroll
      for (int q = 0; q < kRoutingStageBatch; ++q) {
        const int t = b0 + q * NT + tid;
        v[q] = t < T ? ids[t / tps] : -1;
      }
#pragma unroll
      for (int q = 0; q < kRoutingStageBatch; ++q) {
        const int t = b0 + q * NT + tid;
        if (t < T) {
          const bool ok = v[q] >= 0 && v[q] < S;
          invalid += (!ok && v[q] != -1) ? 1 : 0;
          key16[t] = (uint16_t)(ok ? v[q] : S);
        }
      }
    }
  }
  __syncthreads();

  const int chunk = (T + NW - 1) / NW;
  const int t0 = min(T, w * chunk), t1 = min(T, t0 + chunk);
  auto key_of = [&](int t) -> int {
    if (stage) return key16[t];
    const int id = ids[t / tps];
    return (id >= 0 && id < S) ? id : S;
  };

  // pass 1: per-wave histograms (one LDS add per distinct key of a group)
  for (int g = t0; g < t1; g += 64) {
    const int t = g + lane;
    int key = -1;
    if (t < t1) {
      key = key_of(t);
      if (!stage) {
        const int id = ids[t / tps];
        invalid += (id < -1 || id >= S) ? 1 : 0;
      }
    }
    const unsigned long long m = match_key(key, nbits);
    if (key >= 0 && (m >> lane) == 1ull) atomicAdd(&hist[w * K + key], __popcll(m));   // last lane of its key
  }
  invalid = wave_sum(invalid);
  if (lane == 0 && invalid) atomicAdd(&misc[0], invalid);
  __syncthreads();

  // pass 2a: per key, exclusive prefix over the waves; key totals
  for (int key = tid; key < K; key += NT) {
    int run = 0;
    for (int ww = 0; ww < NW; ++ww) {
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
    const int key = t < t1 ? key_of(t) : -1;
    const unsigned long long m = match_key(key, nbits);
    if (key >= 0) {
      const int base = hist[w * K + key];
      const int rank = base + __popcll(m & ((1ull << lane) - 1ull));
      sorted[start[key] + rank] = t;
      if (key < S && rank < kRecTokens) rec[(size_t)key * kRecInts + 4 + rank] = t;
      if (rank == 0) first[key] = t;
      // the key's last lane advances the wave's running offset (all lanes read it above)
      if ((m >> lane) == 1ull) hist[w * K + key] = base + __popcll(m);
    }
  }
  __syncthreads();

  // record entries past a segment's tokens repeat its first token (token 0 for an
  // empty segment), so that every entry names a valid row of the batch
  for (int i = tid; i < S * kRecTokens; i += NT) {
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

// Small batches (T <= kSmallRoutingT tokens, S + 1 <= kSmallRoutingK keys): the
// same outputs from one wave (route_wave).
constexpr int kSmallRoutingT = 128;    // most tokens of the one-wave kernel
constexpr int kSmallRoutingK = 128;    // most keys (S + 1) it can take

__global__ __launch_bounds__(64) void routing_small_kernel(const int32_t* __restrict__ ids, int T, int tps, int S,
                                                           int mfma_min, int tile_m, int max_tiles, RouteOut o) {
  __shared__ __align__(16) int lds[route_wave_lds_ints(kSmallRoutingT / 64, kSmallRoutingK / 64)];
  route_wave<kSmallRoutingT / 64, kSmallRoutingK / 64>(ids, T, tps, S, mfma_min, tile_m, max_tiles, o, lds);
}

hipError_t launch_routing(const int32_t* ids, int T, int tps, int S, int mfma_min, int tile_m, int max_tiles,
                          int* counts, int* offs, int* sorted, int* active, int4* desc, int4* tiles,
                          int* rec, int* meta, hipStream_t stream, const KTimer& tm) {
  // one wave up to 128 tokens (measured: 64 tokens 5.7 -> 4.8 us; at 256 tokens and
  // 64 slots the workgroup kernel is faster, 6.0 against 7.2 us)
  if (T <= kSmallRoutingT && S + 1 <= kSmallRoutingK) {
    const RouteOut o{counts, offs, sorted, active, desc, tiles, rec, meta};
    RAX_LAUNCH(tm, routing_small_kernel, dim3(1), dim3(64), 0u, stream, ids, T, tps, S, mfma_min, tile_m, max_tiles, o);
    return hipGetLastError();
  }
  // 16 waves for large batches when their histograms leave room (the per-token passes
  // are bound by the one CU's vector throughput), else 8 (fewer waves to start and
  // synchronise); keys kept in LDS when they fit next to the histograms (64 KB in all)
  const size_t fixed = (size_t)(2 * (S + 1) + 4) * sizeof(int);
  const int nw = T >= 2048 && fixed + (size_t)16 * (S + 1) * sizeof(int) <= 32768 ? 16 : 8;
  const size_t base = fixed + (size_t)nw * (S + 1) * sizeof(int);
  const size_t keys = ((size_t)T * sizeof(uint16_t) + 15) / 16 * 16;
  const int stage = base + keys <= 65536 ? 1 : 0;
  const size_t lds = base + (stage ? keys : 0);
  RAX_LAUNCH(tm, routing_kernel, dim3(1), dim3(64 * nw), (uint32_t)lds, stream, ids, T, tps, S,
             mfma_min, tile_m, max_tiles, stage, counts, offs, sorted, active, desc, tiles, rec, meta);
  return hipGetLastError();
}

}  // namespace rax
