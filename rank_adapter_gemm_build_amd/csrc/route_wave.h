// Routing of small batches by one wave (device code).
//
// route_wave builds the whole routing of a batch (the outputs of the routing kernel:
// counts, offsets, sorted ids, slot records, active list, descriptors, matrix-core
// tiles, meta) in one wave with no workgroup barriers.  The standalone routing launch
// runs it for batches of up to 128 tokens; the shrink launch of a fused route-and-apply
// call runs it in its first workgroup for batches of up to 256 tokens.
//
// BatchKeys / BatchTiles are what the other units of that fused shrink launch use
// instead of the routing outputs, which are being written by the same launch: each
// unit reads the batch's slot ids (at most 4 per lane, one round trip, like the
// routing record it replaces) and derives, for the segment or tile it works on, the
// same segment length, first sorted position and token ids in the same stable order
// (page "第16章 LoRA 适配器热切换", §16.4.2-§16.4.3: tokens grouped by slot, a segment per
// slot; page "TensorRT-LLM 源码完全拆解(二十一):LoRA 服务", "一次 decode 批次的路由": counts
// as a bincount, offsets as their cumulative sum, no-LoRA tokens in a sentinel slot
// after the real ones).
#pragma once

#include "device_util.h"

namespace rax {

// Lanes of this wave whose key equals this lane's (keys below 2^nbits; lanes with
// key < 0 match nothing), as a 64-bit mask.
__device__ __forceinline__ unsigned long long match_key(int key, int nbits) {
  unsigned long long m = __ballot(key >= 0);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1;
    const unsigned long long bal = __ballot(bit);
    m &= bit ? bal : ~bal;
  }
  return key >= 0 ? m : 0ull;
}

// LDS ints route_wave<Q, KQ> uses
__host__ __device__ constexpr int route_wave_lds_ints(int Q, int KQ) { return 3 * 64 * KQ + 64 * Q; }

// The routing of T <= 64 Q tokens over S + 1 <= 64 KQ keys, by one wave.  Each lane
// holds Q tokens (t = lane + 64 q), loaded in one batch.  Per 64-token group,
// bit-sliced key matching gives every token its rank among the group's equal keys
// and the group's count per key; a per-key running count in LDS makes the ranks
// stable across groups.  One wave scan over the counts (KQ consecutive keys per
// lane) gives the segment starts, then the tokens are scattered (to sorted_ids and
// an LDS copy from which the 128-byte slot records are written whole, 16 bytes per
// lane), and the active-slot and tile lists are compacted with ballots in slot order.
template <int Q, int KQ>
__device__ __forceinline__ void route_wave(const int32_t* __restrict__ ids, int T, int tps, int S, int mfma_min,
                                           int tile_m, int max_tiles, const RouteOut& o, int* __restrict__ lds) {
  constexpr int KMAX = 64 * KQ;
  int* cnt = lds;                 // [KMAX] running count per key, then the count
  int* off = lds + KMAX;          // [KMAX] segment starts
  int* first = lds + 2 * KMAX;    // [KMAX] first token of each segment
  int* tok = lds + 3 * KMAX;      // [64 Q] sorted token ids
  const int lane = lane_id(), K = S + 1;
  const unsigned long long lt = (1ull << lane) - 1ull;
  int nbits = 0;
  while ((1 << nbits) <= S) ++nbits;

  int v[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int t = 64 * q + lane;
    v[q] = t < T ? ids[t / tps] : -1;   // tps tokens per id (sequence)
  }
#pragma unroll
  for (int i = 0; i < KQ; ++i) cnt[lane + 64 * i] = 0;
  int key[Q], rank[Q], invalid = 0;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int t = 64 * q + lane;
    const bool ok = v[q] >= 0 && v[q] < S;
    invalid += (t < T && !ok && v[q] != -1) ? 1 : 0;
    key[q] = t < T ? (ok ? v[q] : S) : -1;
  }
  wave_lds_sync();
  // ranks, stable in token order; the last lane of each key advances its count
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    if (64 * q < T) {
      const unsigned long long m = match_key(key[q], nbits);
      const int base = key[q] >= 0 ? cnt[key[q]] : 0;
      rank[q] = base + __popcll(m & lt);
      wave_lds_sync();
      if (key[q] >= 0 && (m >> lane) == 1ull) cnt[key[q]] = base + __popcll(m);
      wave_lds_sync();
    } else {
      rank[q] = 0;
    }
  }
  // segment starts: lane holds keys KQ lane .. KQ lane + KQ - 1
  {
    int c[KQ], sum = 0;
#pragma unroll
    for (int i = 0; i < KQ; ++i) {
      const int k = KQ * lane + i;
      c[i] = k < K ? cnt[k] : 0;
      sum += c[i];
    }
    const int incl = wave_inclusive_scan(sum);
    int run = incl - sum;
#pragma unroll
    for (int i = 0; i < KQ; ++i) {
      const int k = KQ * lane + i;
      if (k < K) {
        off[k] = run;
        o.counts[k] = c[i];
        o.offs[k] = run;
      }
      run += c[i];
    }
    if (lane == 63) o.offs[K] = incl;   // == T
  }
  wave_lds_sync();
  // scatter
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    if (key[q] >= 0) {
      const int t = 64 * q + lane, pos = off[key[q]] + rank[q];
      o.sorted[pos] = t;
      tok[pos] = t;
      if (rank[q] == 0) first[key[q]] = t;
    }
  }
  wave_lds_sync();
  // slot records, whole: (tokens, first position, 0, 0) then the first kRecTokens token
  // ids, entries past the segment repeating its first token (token 0 if empty)
  for (int idx = lane; idx < S * (kRecInts / 4); idx += 64) {
    const int k = idx / (kRecInts / 4), part = idx - k * (kRecInts / 4);
    const int c = cnt[k], st = off[k];
    int4 w;
    if (part == 0) {
      w = make_int4(c, st, 0, 0);
    } else {
      const int pad = c > 0 ? first[k] : 0, e = 4 * (part - 1);
      w = make_int4(e < c ? tok[st + e] : pad, e + 1 < c ? tok[st + e + 1] : pad, e + 2 < c ? tok[st + e + 2] : pad,
                    e + 3 < c ? tok[st + e + 3] : pad);
    }
    *reinterpret_cast<int4*>(o.rec + (size_t)k * kRecInts + 4 * part) = w;
  }
  // active slots, descriptors and matrix-core tiles, in slot order
  int nact = 0, ntiles = 0;
#pragma unroll
  for (int h = 0; h < KQ; ++h) {
    const int k = lane + 64 * h;
    const int c = k < S ? cnt[k] : 0;
    const unsigned long long ma = __ballot(c > 0);
    if (c > 0) {
      const int e = nact + __popcll(ma & lt);
      o.active[e] = k;
      o.desc[e] = make_int4(k, c, off[k], 0);
    }
    nact += __popcll(ma);
    const int nt = (c > 0 && c >= mfma_min) ? (c + tile_m - 1) / tile_m : 0;
    const int incl = wave_inclusive_scan(nt);
    for (int i = 0; i < nt; ++i) {
      const int e = ntiles + incl - nt + i;
      if (e < max_tiles) o.tiles[e] = make_int4(k, off[k] + i * tile_m, min(tile_m, c - i * tile_m), 0);
    }
    ntiles += __shfl(incl, 63);
  }
  invalid = wave_sum(invalid);
  if (lane == 0) {
    o.meta[kMetaT] = T;
    o.meta[kMetaActive] = nact;
    o.meta[kMetaInvalid] = invalid;
    o.meta[kMetaLora] = off[S];
    o.meta[kMetaTiles] = min(ntiles, max_tiles);
  }
}

// ------------------------------------------------------------ self-routing units
constexpr int kSelfRouteQ = kSelfRouteTokens / 64;   // tokens per lane
constexpr int kSelfRouteT = kSelfRouteTokens;
constexpr int kSelfRouteK = kSelfRouteKeys;          // 4 keys per lane
static_assert(kSelfRouteQ == 4 && kSelfRouteK == 256, "BatchKeys / BatchTiles hold 4 tokens and 4 keys per lane");

// Slot ids of a batch of T <= kSelfRouteT tokens (1 <= T), the ids the routing would
// read: key = slot, S for no LoRA or an invalid id, -1 past the batch.  Lane l holds
// tokens l + 64 q.
struct BatchKeys {
  int key[kSelfRouteQ];
  __device__ __forceinline__ void load(const int32_t* __restrict__ ids, int T, int S) {
    const int lane = lane_id();
    int v[kSelfRouteQ];
#pragma unroll
    for (int q = 0; q < kSelfRouteQ; ++q) v[q] = ids[min(64 * q + lane, T - 1)];
#pragma unroll
    for (int q = 0; q < kSelfRouteQ; ++q) {
      const int t = 64 * q + lane;
      key[q] = t < T ? ((v[q] >= 0 && v[q] < S) ? v[q] : S) : -1;
    }
  }
  // keep the keys in LDS (keys[kSelfRouteT]) / take them back
  __device__ __forceinline__ void store(int* __restrict__ keys) const {
#pragma unroll
    for (int q = 0; q < kSelfRouteQ; ++q) keys[64 * q + lane_id()] = key[q];
  }
  __device__ __forceinline__ void reload(const int* __restrict__ keys) {
#pragma unroll
    for (int q = 0; q < kSelfRouteQ; ++q) key[q] = keys[64 * q + lane_id()];
  }
  // Slot s's segment: its length L and first sorted position p0 (tokens of lower
  // slots), and its token ids in token order written to tok[0 .. L) (LDS).  Wave-uniform.
  __device__ __forceinline__ void segment(int s, int& L, int& p0, int* __restrict__ tok) const {
    const int lane = lane_id();
    const unsigned long long lt = (1ull << lane) - 1ull;
    int c = 0, before = 0;
#pragma unroll
    for (int q = 0; q < kSelfRouteQ; ++q) {
      const unsigned long long m = __ballot(key[q] == s);
      const unsigned long long b = __ballot(key[q] >= 0 && key[q] < s);
      if (key[q] == s) tok[c + __popcll(m & lt)] = 64 * q + lane;
      c += __popcll(m);
      before += __popcll(b);
    }
    L = __builtin_amdgcn_readfirstlane(c);   // wave-uniform: keep it in scalar registers
    p0 = __builtin_amdgcn_readfirstlane(before);
  }
};

// The batch's matrix-core tiles as the routing lists them: segments of at least
// mfma_min tokens, in slot order, cut into tiles of tile_m tokens.  build() leaves
// the per-slot token counts in LDS (cnt[kSelfRouteK]) and returns the number of
// tiles; find() maps a tile to its slot from those counts (lane l looks at slots
// 4 l .. 4 l + 3), so nothing but LDS is kept between the two.
struct BatchTiles {
  __device__ __forceinline__ static int tiles_of_lane(const int* __restrict__ cnt, int S, int mfma_min, int tile_m,
                                                      int (&nt)[4]) {
    const int lane = lane_id();
    const int4 c4 = *reinterpret_cast<const int4*>(cnt + 4 * lane);
    const int c[4] = {c4.x, c4.y, c4.z, c4.w};
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      nt[i] = (4 * lane + i < S && c[i] > 0 && c[i] >= mfma_min) ? (c[i] + tile_m - 1) / tile_m : 0;
      sum += nt[i];
    }
    return sum;
  }
  __device__ __forceinline__ static int build(const BatchKeys& K, int S, int mfma_min, int tile_m, int max_tiles,
                                              int* __restrict__ cnt) {
    const int lane = lane_id();
    *reinterpret_cast<int4*>(cnt + 4 * lane) = make_int4(0, 0, 0, 0);
    wave_lds_sync();
#pragma unroll
    for (int q = 0; q < kSelfRouteQ; ++q)
      if (K.key[q] >= 0 && K.key[q] < S) atomicAdd(&cnt[K.key[q]], 1);
    wave_lds_sync();
    int nt[4];
    const int incl = wave_inclusive_scan(tiles_of_lane(cnt, S, mfma_min, tile_m, nt));
    return __builtin_amdgcn_readfirstlane(min(__shfl(incl, 63), max_tiles));
  }
  // slot of tile `tile` (below the count build() returned) and the tile's index
  // within the slot's segment
  __device__ __forceinline__ static void find(const int* __restrict__ cnt, int S, int mfma_min, int tile_m, int tile,
                                              int& slot, int& idx) {
    const int lane = lane_id();
    int nt[4];
    const int sum = tiles_of_lane(cnt, S, mfma_min, tile_m, nt);
    int t0 = wave_inclusive_scan(sum) - sum, s = 0, i0 = 0;
    bool mine = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (tile >= t0 && tile < t0 + nt[i]) {
        mine = true;
        s = 4 * lane + i;
        i0 = tile - t0;
      }
      t0 += nt[i];
    }
    const int owner = __builtin_ctzll(__ballot(mine) | (1ull << 63));   // one lane owns a tile < total
    slot = __builtin_amdgcn_readfirstlane(__shfl(s, owner));
    idx = __builtin_amdgcn_readfirstlane(__shfl(i0, owner));
  }
};

}  // namespace rax
