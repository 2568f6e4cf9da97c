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
// One workgroup of 8 waves (16 for large batches).  The token range is cut into
// contiguous chunks, one per wave.  Each wave loads the ids
// of its chunk (up to kRoutingStageBatch groups per batch of independent loads; a
// chunk of at most that many groups stays in registers for the scatter) and counts
// them into its own LDS histogram row.  Then, key by key, the rows turn into the start
// of each wave's run inside the key's segment, and one wave scans the key totals into
// the segment offsets.  The scatter walks each chunk in token order, 64 tokens at a
// time: a group whose tokens all carry one key (the common case in prefill batches)
// ranks them by lane; otherwise each lane finds the lanes holding its key with one
// ballot per key bit (the intersection of the matching bit masks) and ranks itself by
// lane order, so each key's tokens land in increasing token order: the result is the
// unique stable order, identical on every run.  Every slot also gets a 128-byte record
// (tokens, first sorted position, then its first kRecTokens token ids in sorted
// order), so that a kernel unit of a short segment finds its token rows with the same
// load that tells it the segment.  One wave compacts the active-slot list and a
// 16-byte descriptor per active slot (slot, tokens, first sorted position) in slot
// order and scans the keys' tile counts into each long segment's first tile; then
// every thread writes matrix-core tiles, finding a tile's segment by binary search
// over the first tiles.
#include <hip/hip_runtime.h>

#include "device_util.h"
#include "route_wave.h"

namespace rax {

// Keys of one batch of up to kRoutingStageBatch 64-token groups of a wave's chunk
// (token g0 + 64 q + lane; -1 past the chunk's end), invalid ids counted.
__device__ __forceinline__ void routing_load_keys(const int32_t* __restrict__ ids, int g0, int t1, int tps, int S,
                                                  int (&kv)[kRoutingStageBatch], int& invalid) {
  const int lane = lane_id();
  int v[kRoutingStageBatch];
#pragma unroll
  for (int q = 0; q < kRoutingStageBatch; ++q) {
    const int t = g0 + 64 * q + lane;
    v[q] = t < t1 ? ids[tps == 1 ? t : t / tps] : -1;
  }
#pragma unroll
  for (int q = 0; q < kRoutingStageBatch; ++q) {
    const int t = g0 + 64 * q + lane;
    const bool ok = v[q] >= 0 && v[q] < S;
    invalid += (t < t1 && !ok && v[q] != -1) ? 1 : 0;
    kv[q] = t < t1 ? (ok ? v[q] : S) : -1;
  }
}

__global__ __launch_bounds__(kRoutingMaxThreads) void routing_kernel(
    const int32_t* __restrict__ ids, int T, int tps, int S, int mfma_min, int tile_m, int max_tiles,
    int* __restrict__ counts, int* __restrict__ offs, int* __restrict__ sorted,
    int* __restrict__ active, int4* __restrict__ desc, int4* __restrict__ tiles,
    int* __restrict__ rec, int* __restrict__ meta) {
  constexpr int G = kRoutingStageBatch;
  extern __shared__ int lds[];
  const int NW = blockDim.x / 64, NT = blockDim.x;   // waves and threads of the workgroup
  const int K = S + 1;                         // keys 0..S-1 are slots, S is "no LoRA"
  int* hist = lds;                             // [NW][K]; after the scatter: first tile per key [K]
  int* start = lds + NW * K;                   // [K]: counts, then segment starts
  int* misc = start + K;                       // [4]
  int* first = misc + 4;                       // [K]: first token of each segment
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int nbits = 0;
  while ((1 << nbits) <= S) ++nbits;           // keys 0..S fit in nbits bits

  // contiguous chunks, one per wave
  const int chunk = (T + NW - 1) / NW;
  const int t0 = min(T, w * chunk), t1 = min(T, t0 + chunk);
  const bool held = t1 - t0 <= 64 * G;         // the whole chunk in one batch of registers
  int kv[G];
  int invalid = 0;
  routing_load_keys(ids, t0, t1, tps, S, kv, invalid);   // in flight while the histograms clear
  for (int i = tid; i < NW * K; i += NT) hist[i] = 0;
  if (tid < 4) misc[tid] = 0;
  __syncthreads();

  // per-wave histograms: one LDS add per group for a single-key group, else one per token
  for (int g0 = t0; g0 < t1; g0 += 64 * G) {
    if (g0 != t0) routing_load_keys(ids, g0, t1, tps, S, kv, invalid);
#pragma unroll
    for (int q = 0; q < G; ++q) {
      if (g0 + 64 * q < t1) {
        const int key = kv[q];
        const int k0 = __builtin_amdgcn_readfirstlane(key);
        if (__ballot(key != k0) == 0ull) {
          if (lane == 0) atomicAdd(&hist[w * K + k0], 64);
        } else if (key >= 0) {
          atomicAdd(&hist[w * K + key], 1);
        }
      }
    }
  }
  invalid = wave_sum(invalid);
  if (lane == 0 && invalid) atomicAdd(&misc[0], invalid);
  __syncthreads();

  // per key, exclusive prefix over the waves; key totals
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

  // one wave scans the key totals into segment starts
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

  // stable scatter, each wave over its own chunk in token order; a run of single-key
  // groups of one key keeps that key's running offset and segment start in registers
  int ck = -1, cbase = 0, cstart = 0;          // wave-uniform cache (ck = -1: none)
  for (int g0 = t0; g0 < t1; g0 += 64 * G) {
    if (!held) routing_load_keys(ids, g0, t1, tps, S, kv, invalid);
#pragma unroll
    for (int q = 0; q < G; ++q) {
      if (g0 + 64 * q < t1) {
        const int t = g0 + 64 * q + lane, key = kv[q];
        const int k0 = __builtin_amdgcn_readfirstlane(key);
        int rank, pos;
        unsigned long long m;
        if (__ballot(key != k0) == 0ull) {     // one key for the whole group (never -1: g0 + 64 q < t1)
          if (k0 != ck) {
            cbase = hist[w * K + k0];
            cstart = start[k0];
            ck = k0;
          }
          rank = cbase + lane;
          pos = cstart + rank;
          cbase += 64;
          m = ~0ull;
        } else {
          m = match_key(key, nbits);
          rank = (key >= 0 ? hist[w * K + key] : 0) + __popcll(m & ((1ull << lane) - 1ull));
          pos = (key >= 0 ? start[key] : 0) + rank;
          ck = -1;                               // this group may advance any key's offset
        }
        if (key >= 0) {
          RAX_CHECK_VAR(pos, T);
          sorted[pos] = t;
          if (key < S && rank < kRecTokens) rec[(size_t)key * kRecInts + 4 + rank] = t;
          if (rank == 0) first[key] = t;
          // the key's last lane advances the wave's running offset (all lanes read it above)
          if ((m >> lane) == 1ull) hist[w * K + key] = rank + 1;
        }
      }
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

  // lists, in slot order: active slots, and tiles of the segments long enough for the
  // matrix-core path (slot, first sorted position, length); hist now holds each key's
  // first tile
  int* tfirst = hist;
  if (w == 0) {
    int nact = 0, ntiles = 0;
    for (int kb = 0; kb < S; kb += 64) {
      const int key = kb + lane;
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
      if (key < S) tfirst[key] = ntiles + incl - nt;
      ntiles += __builtin_amdgcn_readlane(incl, 63);
    }
    if (lane == 0) {
      tfirst[S] = ntiles;
      misc[1] = ntiles;
      meta[kMetaT] = T;
      meta[kMetaActive] = nact;
      meta[kMetaInvalid] = misc[0];
      meta[kMetaLora] = start[S];
      meta[kMetaTiles] = min(ntiles, max_tiles);
    }
  }
  __syncthreads();
  const int nt_out = min(misc[1], max_tiles);
  for (int e = tid; e < nt_out; e += NT) {
    // the last key whose first tile is <= e: keys without tiles share the next key's first tile
    int lo = 0, hi = S;                        // tfirst[lo] <= e < tfirst[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tfirst[mid] <= e) lo = mid; else hi = mid;
    }
    const int i = e - tfirst[lo], c = start[lo + 1] - start[lo];
    tiles[e] = make_int4(lo, start[lo] + i * tile_m, min(tile_m, c - i * tile_m), 0);
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

// batches from this many tokens get 16 routing waves (when their histograms fit)
constexpr int kRoutingWideT = 512;

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
  // synchronise)
  const size_t fixed = (size_t)(2 * (S + 1) + 4) * sizeof(int);
  const int nw = T >= kRoutingWideT && fixed + (size_t)16 * (S + 1) * sizeof(int) <= 32768 ? 16 : 8;
  const size_t lds = fixed + (size_t)nw * (S + 1) * sizeof(int);
  RAX_LAUNCH(tm, routing_kernel, dim3(1), dim3(64 * nw), (uint32_t)lds, stream, ids, T, tps, S,
             mfma_min, tile_m, max_tiles, counts, offs, sorted, active, desc, tiles, rec, meta);
  return hipGetLastError();
}

RAX_INDEX_FAULTS_ACCESSOR(routing)

}  // namespace rax
