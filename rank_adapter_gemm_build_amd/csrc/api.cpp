// Host side of the C ABI declared in include/raxlora.h: argument checks, object
// lifetimes, and kernel dispatch.  Every argument check runs before the first HIP
// call, so a rejected call changes nothing and needs no device.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"

using rax::SlotEntry;

#ifdef RAXLORA_DEBUG
namespace rax {   // each kernel translation unit's count of failed index checks
hipError_t index_faults_linear(unsigned int*, bool);
hipError_t index_faults_routing(unsigned int*, bool);
hipError_t index_faults_w16_y16(unsigned int*, bool);
hipError_t index_faults_w16_y32(unsigned int*, bool);
hipError_t index_faults_w32_y32(unsigned int*, bool);
hipError_t index_faults_w8_y16(unsigned int*, bool);
hipError_t index_faults_w8_y32(unsigned int*, bool);
}  // namespace rax
#endif

struct lora_pool {
  int device = 0;
  int S = 0, Rmax = 0, Rk = 0, k = 0, N = 0, D = 0, max_tokens = 0;
  int d[LORA_MAX_SLICES] = {0};
  int o[LORA_MAX_SLICES] = {0};
  int tile0[LORA_MAX_SLICES + 1] = {0};
  int mblk0[LORA_MAX_SLICES + 1] = {0};
  lora_dtype wdtype = LORA_BF16;
  size_t esize = 2;
  bool embedding = false;     // A stored [S][V][Rmax] (rows by vocabulary id); k = V
  void* A = nullptr;
  void* Bt = nullptr;
  void* Bk = nullptr;
  SlotEntry* table = nullptr;
  float* ws = nullptr;        // k-split partials [nsplit][N][ws_rows][Rk]: rows by sorted position, then
                              // slot mode's first-tile rows (kMfmaTileM per slot) when `heads`
  int ws_rows = 0;
  bool heads = false;
  int nsplit = 1, ns = 1;     // decode shrink: k splits, chunk steps per split (fixed by k)
  std::vector<SlotEntry> mirror;
  std::vector<uint8_t> order;  // slots by descending rank, stable (S <= kMaxOrderedSlots)
};

namespace {
// Decode expand units of a high-rank slot run longest (one B^T batch per 16 ranks),
// so they are dispatched first: slots sorted by descending rank, ties by index.
void update_order(lora_pool* p) {
  if (p->S > rax::kMaxOrderedSlots) return;
  std::vector<int> idx(p->S);
  for (int s = 0; s < p->S; ++s) idx[s] = s;
  std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) { return p->mirror[a].rank > p->mirror[b].rank; });
  p->order.assign(idx.begin(), idx.end());
}
}  // namespace

struct lora_routing {
  int device = 0;
  int max_tokens = 0, S = 0, mfma_min = rax::kDefaultMfmaMinSeg, tile_m = rax::kMfmaTileM;
  int max_tiles = 0;
  int* buf = nullptr;
  int *counts = nullptr, *offs = nullptr, *sorted = nullptr, *active = nullptr, *meta = nullptr;
  int4 *desc = nullptr, *tiles = nullptr;
  int* rec = nullptr;
  int T = -1;  // tokens of the last build; -1 = never built
};

namespace {

thread_local std::string g_last_error;

lora_status fail(lora_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

lora_status ok() {
  g_last_error.clear();
  return LORA_OK;
}

lora_status hip_fail(hipError_t e, const char* what) {
  return fail(e == hipErrorOutOfMemory ? LORA_ERR_OOM : LORA_ERR_HIP, "%s: %s", what,
              hipGetErrorString(e));
}

// Make `device` current for the scope, restoring the previous device after.
struct DeviceGuard {
  int prev = -1;
  hipError_t err = hipSuccess;
  explicit DeviceGuard(int device) {
    err = hipGetDevice(&prev);
    if (err == hipSuccess && prev != device) err = hipSetDevice(device);
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

lora_status check_device(int device) {
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess || n <= 0) return fail(LORA_ERR_NO_DEVICE, "no GPU available (%s)", hipGetErrorString(e));
  if (device < 0 || device >= n) return fail(LORA_ERR_NO_DEVICE, "device %d out of range [0, %d)", device, n);
  return LORA_OK;
}

// ------------------------------------------------------------- kernel timing
// When enabled, each hot-path launch takes a pair of events that hipExtLaunchKernel
// stamps at the kernel's own start and end; lora_timing_report adds them up.
struct TimingRecord {
  int kernel;
  hipEvent_t start, stop;
};
std::mutex g_timing_mu;
bool g_timing_on = false;
std::vector<TimingRecord> g_timing_records;
std::vector<hipEvent_t> g_free_events;

hipEvent_t take_event() {
  if (!g_free_events.empty()) {
    hipEvent_t e = g_free_events.back();
    g_free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

rax::KTimer timer_for(int kernel) {
  rax::KTimer t;
  std::lock_guard<std::mutex> lk(g_timing_mu);
  if (!g_timing_on) return t;
  t.start = take_event();
  t.stop = take_event();
  if (!t.start || !t.stop) return rax::KTimer{};
  g_timing_records.push_back(TimingRecord{kernel, t.start, t.stop});
  return t;
}

const char* const kKernelNames[rax::kKernelCount] = {"routing", "shrink", "expand", "finish_u", "gather"};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  if (!v || !*v) return dflt;
  return atoi(v);
}

// RAXLORA_LOG=1: one line on stderr per launch of the LoRA kernels, with the launch
// shape the plan chose (read once per process; for diagnosing which path a call takes)
bool log_on() {
  static const bool on = env_int("RAXLORA_LOG", 0) != 0;
  return on;
}
void log_plan(const char* what, const lora_pool* p, const lora_routing* r, const rax::Plan& pl, int modules) {
  if (!log_on()) return;
  std::fprintf(stderr,
               "raxlora: %s T=%d S=%d k=%d N=%d D=%d Rmax=%d modules=%d mode=%s nsplit=%d waves=%d use_mfma=%d "
               "tile_slots=%d cb=%d n_dec=%d\n",
               what, r->T, r->S, p->k, p->N, p->D, p->Rmax, modules, pl.slot_mode ? "slot" : "tiles", pl.nsplit,
               pl.slot_mode ? pl.slot_waves : 1, pl.use_mfma, pl.tile_slots, pl.cb, pl.n_dec_blocks);
}

rax::PoolView pool_view(const lora_pool* p) {
  rax::PoolView v{};
  v.A = p->A;
  v.Bt = p->Bt;
  v.Bk = p->Bk;
  v.table = p->table;
  v.S = p->S;
  v.Rmax = p->Rmax;
  v.Rk = p->Rk;
  v.k = p->k;
  v.N = p->N;
  v.D = p->D;
  v.n_ctiles = p->tile0[p->N];
  v.n_mblocks = p->mblk0[p->N];
  for (int n = 0; n < rax::kMaxSlices; ++n) {
    v.d[n] = n < p->N ? p->d[n] : 0;
    v.o[n] = n < p->N ? p->o[n] : 0;
  }
  for (int n = 0; n <= rax::kMaxSlices; ++n) {
    v.tile0[n] = n <= p->N ? p->tile0[n] : p->tile0[p->N];
    v.mblk0[n] = n <= p->N ? p->mblk0[n] : p->mblk0[p->N];
  }
  return v;
}

rax::SlotOrder slot_order(const lora_pool* p) {
  rax::SlotOrder o{};
  o.ordered = (int)p->order.size() == p->S ? 1 : 0;
  for (size_t i = 0; i < p->order.size(); ++i) o.s[i] = p->order[i];
  return o;
}

rax::RouteOut route_out(const lora_routing* r) {
  return rax::RouteOut{r->counts, r->offs, r->sorted, r->active, r->desc, r->tiles, r->rec, r->meta};
}

rax::RouteView route_view(const lora_routing* r) {
  rax::RouteView v{};
  v.counts = r->counts;
  v.offs = r->offs;
  v.sorted = r->sorted;
  v.active = r->active;
  v.desc = r->desc;
  v.tiles = r->tiles;
  v.rec = r->rec;
  v.meta = r->meta;
  v.S = r->S;
  v.T = r->T;
  v.mfma_min = r->mfma_min;
  v.tile_m = r->tile_m;
  v.max_tiles = r->max_tiles;
  return v;
}

// k elements of one wave-wide chunk step of the decode shrink (x is bf16 for FP8 pools)
int chunk_width(lora_dtype t) { return 64 * (t == LORA_F32 ? 4 : 8); }

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// k split of the decode shrink, fixed by the pool's shape: one wave-wide 16-byte chunk
// step per split while k has at most kMaxSplit of them (so a short batch still has
// k / chunk width waves per 16 rank rows), else the fewest equal splits of at most
// kMaxSplit.
void choose_split(lora_pool* p) {
  const int chunks = ceil_div(p->k, chunk_width(p->wdtype));
  p->ns = ceil_div(chunks, rax::kMaxSplit);
  p->nsplit = ceil_div(chunks, p->ns);
}

// k split of the slot-major shrink (slot mode): workgroups of 1, 2, 4 or 8 waves, each
// wave taking at most 8 matrix-core steps of 32 of its part; the fewest waves that
// leave at most 8 parts (so the expand reads every value's partial sums in one batch;
// k <= 16384), else 8 waves and at most kMaxSplit parts (k <= 32768).  slot_nsplit is
// 0 when k is longer (no slot mode).
constexpr int kSlotStepsPerWave = 8;
int slot_waves(int k) {
  const int steps = ceil_div(k, rax::kMfmaK);
  for (int nw = 1; nw < 8; nw *= 2)
    if (steps <= kSlotStepsPerWave * nw * 8) return nw;
  return 8;
}
int slot_nsplit(int k) {
  const int steps = ceil_div(k, rax::kMfmaK), per = kSlotStepsPerWave * slot_waves(k);
  return steps <= per * rax::kMaxSplit ? ceil_div(steps, per) : 0;
}


// Common checks of shrink / expand / linear.
lora_status check_pair(const lora_pool* pool, const lora_routing* routing) {
  if (!pool || !routing) return fail(LORA_ERR_INVALID_ARG, "pool and routing must not be NULL");
  if (routing->T < 0) return fail(LORA_ERR_STATE, "routing was never built");
  if (routing->S != pool->S)
    return fail(LORA_ERR_SHAPE, "routing has %d slots, pool has %d", routing->S, pool->S);
  if (routing->device != pool->device)
    return fail(LORA_ERR_INVALID_ARG, "routing on device %d, pool on device %d", routing->device, pool->device);
  if (routing->T > pool->max_tokens)
    return fail(LORA_ERR_CAPACITY, "T = %d exceeds the pool's max_tokens = %d", routing->T, pool->max_tokens);
  return LORA_OK;
}

lora_status check_x(const lora_pool* pool, int T, const void* x, int ldx) {
  if (pool->embedding) return fail(LORA_ERR_INVALID_ARG, "embedding pool: use lora_embedding");
  if (T > 0 && !x) return fail(LORA_ERR_INVALID_ARG, "x is NULL");
  if (ldx < pool->k) return fail(LORA_ERR_SHAPE, "ldx = %d < in_features = %d", ldx, pool->k);
  if (ldx % 8 != 0 || !aligned16(x)) return fail(LORA_ERR_ALIGN, "x must be 16-byte aligned with ldx a multiple of 8");
  return LORA_OK;
}

lora_status check_y(const lora_pool* pool, int T, const void* y, int ldy, lora_dtype ydtype) {
  if (T > 0 && !y) return fail(LORA_ERR_INVALID_ARG, "y is NULL");
  if (ydtype != LORA_F32 && ydtype != LORA_BF16) return fail(LORA_ERR_DTYPE, "unknown ydtype %d", (int)ydtype);
  const lora_dtype act = pool->wdtype == LORA_FP8E4M3 ? LORA_BF16 : pool->wdtype;   // activation dtype
  if (ydtype != act && ydtype != LORA_F32)
    return fail(LORA_ERR_DTYPE, "y must be the pool's activation dtype or float32");
  if (ldy < pool->D) return fail(LORA_ERR_SHAPE, "ldy = %d < output width %d", ldy, pool->D);
  if (ldy % 8 != 0 || !aligned16(y)) return fail(LORA_ERR_ALIGN, "y must be 16-byte aligned with ldy a multiple of 8");
  return LORA_OK;
}

// k split of one call: the pool's (at most kMaxSplit parts), halved when segments
// are long on average (T / S >= 64 tokens, a prefill batch): there the matrix-core
// tiles alone fill the GPU, and fewer partial sums make the expand's first step
// cheaper.  Measured: the prefill workload 71 -> 68 us per step; decode batches keep
// the full split, which their short segments need for parallelism.
struct CallSplit {
  int nsplit, ns;
};
bool use_mfma(const lora_pool* pool);

// Slot mode (both kernels slot-major, every segment on the matrix cores; see the
// slot-major shrink and expand units): for small decode batches in which most of the
// pool's slots are active (4 S <= T <= 128), where a step is a chain of memory round
// trips rather than a stream and the usual units' chain of routing lookups (tile
// list, then token ids, then operands) dominates.  The units then issue their weight
// fragments before any routing data has arrived; an inactive slot costs its units
// those loads.  Measured on MI355X: the decode workload (T = 64, 8 slots) 12.2 -> 11.2
// us per step; at T = 256 over 64 slots (three packed modules, grouped) slot mode is
// slower (61 -> 73 us), so it stays off there.  RAXLORA_SLOT_MODE=0 turns it off, 1
// uses it wherever the shape allows (T <= 256, k <= 32768, bf16 or FP8 weights).  A
// grouped call uses it when every module would.
bool slot_mode(const lora_pool* p, const lora_routing* r) {
  const int env = env_int("RAXLORA_SLOT_MODE", -1);
  if (env == 0 || p->embedding || !use_mfma(p) || r->T < 1 || r->T > rax::kSelfRouteTokens || slot_nsplit(p->k) == 0)
    return false;
  return env == 1 || (r->T >= 4 * r->S && r->T <= 128);
}

CallSplit call_split(const lora_pool* p, const lora_routing* r, bool slot) {
  CallSplit c{p->nsplit, p->ns};
  if (slot) {
    c.nsplit = slot_nsplit(p->k);
    c.ns = ceil_div(ceil_div(p->k, chunk_width(p->wdtype)), c.nsplit);
    return c;
  }
  if (r->T >= 64 * std::max(1, r->S) && p->nsplit >= 2) {
    const int chunks = ceil_div(p->k, chunk_width(p->wdtype));
    c.ns = ceil_div(chunks, ceil_div(p->nsplit, 2));
    c.nsplit = ceil_div(chunks, c.ns);
  }
  return c;
}

// The pool's workspace: [nsplit][N][ws_rows][Rk], rows by sorted position (rows
// padded to Rk, a multiple of 32 floats, so they can be read 16 bytes at a time), then,
// for pools that can take slot mode by default (at most kHeadSlots slots), kMfmaTileM
// rows per slot for the first tile of its segment (`heads`: a slot-mode call's
// partials of a segment's first tile go there, where the expand finds them without the
// segment's first sorted position); a call uses its first nsplit parts.
constexpr int kHeadSlots = 32;   // slot mode is the default only for 4 S <= T <= 128
rax::UView workspace_view(const lora_pool* p, int nsplit, bool heads = false) {
  rax::UView v{p->ws, (long long)p->N * p->ws_rows * p->Rk, (long long)p->ws_rows * p->Rk, p->Rk, nsplit, 0};
  v.head0 = heads && p->heads ? p->max_tokens : -1;
  return v;
}

// The caller's u: finished values [N][T][Rmax], rows by token index.
rax::UView caller_u_view(const lora_pool* p, const lora_routing* r, float* u) {
  return rax::UView{u, 0, (long long)r->T * p->Rmax, p->Rmax, 1, 1};
}

bool use_mfma(const lora_pool* pool) {
  return rax::kHaveMfmaPath && pool->wdtype != LORA_F32 && env_int("RAXLORA_DISABLE_MFMA", 0) == 0;
}

// Launch shape of a call, from host-known sizes only (T, S, the pool's shape): the
// expected segment length T / S sets how many waves share one segment's token tiles
// (segments of at least mfma_min tokens go to the matrix cores when those are on),
// and the matrix-core tile slots cover every tile a batch of T tokens can produce
// (the kernels would loop over any excess).
rax::Plan make_plan(const lora_pool* pool, const lora_routing* r, bool expand, bool slot) {
  rax::Plan pl{};
  const CallSplit cs = call_split(pool, r, slot);
  pl.nsplit = cs.nsplit;
  pl.ns = cs.ns;
  pl.nrg = ceil_div(pool->N * pool->Rmax, 64);
  pl.xcd_group = std::max(1, std::min(64, env_int("RAXLORA_XCD_GROUP", 4)));
  if (slot) {
    // slot-major units: shrink (slot, k part, 16-row block), expand (slot, column
    // group); one 128-column block per expand unit while that leaves at most
    // RAXLORA_CB1_MAX units of four blocks
    pl.slot_mode = 1;
    pl.slot_waves = slot_waves(pool->k);
    pl.use_mfma = 1;
    pl.nrb = ceil_div(pool->N * pool->Rmax, 16);
    pl.ntg = 1;
    pl.tile_slots = 1;
    int g4 = 0, g1 = 0;
    for (int n = 0; n < pool->N; ++n) {
      g4 += ceil_div(pool->mblk0[n + 1] - pool->mblk0[n], rax::kMfmaColBlocksPerUnit);
      g1 += pool->mblk0[n + 1] - pool->mblk0[n];
    }
    pl.cb = (long long)g4 * pool->S <= env_int("RAXLORA_CB1_MAX", 512) ? 1 : rax::kMfmaColBlocksPerUnit;
    pl.n_mgroups = pl.cb == 1 ? g1 : g4;
    return pl;
  }
  pl.use_mfma = use_mfma(pool) && r->T >= r->mfma_min ? 1 : 0;
  int mean = std::max(1, ceil_div(r->T, r->S));
  if (pl.use_mfma) mean = std::min(mean, r->mfma_min - 1);
  const int tok = 4;                                   // tokens per decode pass, both kernels
  pl.ntg = std::max(1, std::min(expand ? 4 : 8, ceil_div(mean, tok)));
  pl.nrb = ceil_div(pool->N * pool->Rmax, 16);
  // one workgroup per decode unit
  pl.n_dec_blocks = expand ? pool->tile0[pool->N] * pool->S * pl.ntg : pool->S * pl.nrb * pl.nsplit * pl.ntg;
  // tiles <= T / tile_m + (segments of at least mfma_min tokens), rounded up
  pl.tile_slots = std::max(1, std::min(r->max_tiles, ceil_div(r->T, r->tile_m) + std::min(r->S, ceil_div(r->T, r->mfma_min))));
  // matrix-core expand units: kMfmaColBlocksPerUnit column blocks each (the u values
  // are finished once per unit), or one block each when that still leaves few units
  // (a short chain per unit matters more then)
  auto groups = [&](int cb) {
    int g = 0;
    for (int n = 0; n < pool->N; ++n) g += ceil_div(pool->mblk0[n + 1] - pool->mblk0[n], cb);
    return g;
  };
  const int g4 = groups(rax::kMfmaColBlocksPerUnit);
  pl.cb = (long long)g4 * pl.tile_slots <= env_int("RAXLORA_CB1_MAX", 512) ? 1 : rax::kMfmaColBlocksPerUnit;
  // Matrix-core expand tiles dealt to the XCDs one by one when segments are short on
  // average (T < 64 S): tiles cost what their slot's rank makes them, and the
  // contiguous eighths of the tile list gave some XCDs more high-rank tiles than
  // others.  Zipf workload expand: eighths 116.7 us, runs of 1 / 2 / 4 tiles 113.7 /
  // 112.9 / 115.9; packed three-module workload: eighths 31.0-31.2, runs of 1 30.7,
  // runs of 2 33.6.  Long segments keep one contiguous eighth per XCD: there an XCD's
  // tiles come from two or three slots, whose B fit its L2 (prefill workload: 30.9
  // us; runs of 1, 2 or 4 36.6-37.7).  RAXLORA_TILE_INTERLEAVE=0 keeps the eighths,
  // n > 0 deals runs of n tiles.
  const int il = env_int("RAXLORA_TILE_INTERLEAVE", -1);
  pl.tile_interleave = il >= 0 ? std::min(il, 1 << 20) : (r->T < 64 * std::max(1, r->S) ? 1 : 0);
  pl.n_mgroups = pl.cb == 1 ? groups(1) : g4;
  return pl;
}

// self_ids: build the routing inside the launch from these ids (small batches)
lora_status run_shrink(const lora_pool* pool, const lora_routing* routing, const void* x, int ldx,
                       const rax::UView& U, hipStream_t stream, bool slot, const int32_t* self_ids = nullptr) {
  const rax::Plan pl = make_plan(pool, routing, false, slot);
  log_plan(self_ids ? "shrink (routing inside)" : "shrink", pool, routing, pl, 1);
  rax::SelfRoute sr{self_ids, route_out(routing)};
  hipError_t e = rax::launch_shrink(pool->wdtype, pool_view(pool), route_view(routing), x, ldx, U, pl,
                                    self_ids ? &sr : nullptr, stream, timer_for(rax::kKShrink));
  if (e != hipSuccess) return hip_fail(e, "shrink launch");
  return LORA_OK;
}

lora_status run_expand(const lora_pool* pool, const lora_routing* routing, const rax::UView& U,
                       void* y, int ldy, lora_dtype ydtype, hipStream_t stream, bool slot) {
  const rax::Plan pl = make_plan(pool, routing, true, slot);
  log_plan(U.by_token ? "expand (u by token)" : "expand", pool, routing, pl, 1);
  hipError_t e = rax::launch_expand(pool->wdtype, ydtype, pool_view(pool), slot_order(pool), route_view(routing), U,
                                    y, ldy, pl, stream, timer_for(rax::kKExpand));
  if (e != hipSuccess) return hip_fail(e, "expand launch");
  return LORA_OK;
}

// Shrink, then (after the stream waits for y_ready, when given) the expand: the
// shrink reads only x, so it can run while another stream still writes the base
// output into y.
lora_status shrink_join_expand(const lora_pool* pool, const lora_routing* routing, const void* x, int ldx,
                               void* y, int ldy, lora_dtype ydtype, hipStream_t stream, hipEvent_t y_ready,
                               const int32_t* self_ids) {
  const bool slot = slot_mode(pool, routing);
  const rax::UView W = workspace_view(pool, call_split(pool, routing, slot).nsplit, slot);
  lora_status st = run_shrink(pool, routing, x, ldx, W, stream, slot, self_ids);
  if (st != LORA_OK) return st;
  if (y_ready) {
    hipError_t e = hipStreamWaitEvent(stream, y_ready, 0);
    if (e != hipSuccess) return hip_fail(e, "waiting for y_ready");
  }
  return run_expand(pool, routing, W, y, ldy, ydtype, stream, slot);
}

lora_status linear_impl(const lora_pool* pool, const lora_routing* routing, const void* x, int ldx, void* y,
                        int ldy, lora_dtype ydtype, hipStream_t stream, hipEvent_t y_ready) {
  lora_status st = check_pair(pool, routing);
  if (st != LORA_OK) return st;
  if ((st = check_x(pool, routing->T, x, ldx)) != LORA_OK) return st;
  if ((st = check_y(pool, routing->T, y, ldy, ydtype)) != LORA_OK) return st;
  DeviceGuard g(pool->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
  if (routing->T == 0) {
    // nothing to compute; the join is still honoured, so later work on the stream
    // stays ordered after y_ready as it would with a non-empty batch
    if (y_ready) {
      hipError_t e = hipStreamWaitEvent(stream, y_ready, 0);
      if (e != hipSuccess) return hip_fail(e, "waiting for y_ready");
    }
    return ok();
  }
  st = shrink_join_expand(pool, routing, x, ldx, y, ldy, ydtype, stream, y_ready, nullptr);
  return st == LORA_OK ? ok() : st;
}

lora_status route_linear_impl(const lora_pool* pool, lora_routing* routing, const int32_t* ids, int T,
                              const void* x, int ldx, void* y, int ldy, lora_dtype ydtype, hipStream_t stream,
                              hipEvent_t y_ready) {
  if (!pool || !routing) return fail(LORA_ERR_INVALID_ARG, "pool and routing must not be NULL");
  if (T < 0) return fail(LORA_ERR_SHAPE, "T = %d < 0", T);
  if (T > routing->max_tokens) return fail(LORA_ERR_CAPACITY, "T = %d exceeds max_tokens = %d", T, routing->max_tokens);
  if (T > 0 && !ids) return fail(LORA_ERR_INVALID_ARG, "token_slot_ids is NULL");
  if (routing->S != pool->S) return fail(LORA_ERR_SHAPE, "routing has %d slots, pool has %d", routing->S, pool->S);
  if (routing->device != pool->device)
    return fail(LORA_ERR_INVALID_ARG, "routing on device %d, pool on device %d", routing->device, pool->device);
  if (T > pool->max_tokens) return fail(LORA_ERR_CAPACITY, "T = %d exceeds the pool's max_tokens = %d", T, pool->max_tokens);
  lora_status st = check_x(pool, T, x, ldx);
  if (st != LORA_OK) return st;
  if ((st = check_y(pool, T, y, ldy, ydtype)) != LORA_OK) return st;
  // batches the shrink launch can route itself; others: the routing launch first
  if (T < 1 || T > rax::kSelfRouteTokens || pool->S + 1 > rax::kSelfRouteKeys) {
    if ((st = lora_build_routing(routing, ids, T, stream)) != LORA_OK) return st;
    return linear_impl(pool, routing, x, ldx, y, ldy, ydtype, stream, y_ready);
  }
  DeviceGuard g(pool->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
  routing->T = T;
  st = shrink_join_expand(pool, routing, x, ldx, y, ldy, ydtype, stream, y_ready, ids);
  if (st != LORA_OK) routing->T = -1;   // the routing may not have been built: unusable until rebuilt
  return st == LORA_OK ? ok() : st;
}

// Checks of a grouped call: 1..LORA_MAX_GROUP distinct linear pools on the routing's
// device with its slot count, one weight dtype and one padded rank, each with its
// own input and output.
lora_status check_group(const lora_pool* const* pools, int n, const lora_routing* routing, int T,
                        const void* const* x, const int* ldx, void* const* y, const int* ldy, lora_dtype ydtype) {
  if (!pools || !x || !ldx || !y || !ldy) return fail(LORA_ERR_INVALID_ARG, "pools, x, ldx, y and ldy must not be NULL");
  if (n < 1 || n > LORA_MAX_GROUP) return fail(LORA_ERR_SHAPE, "num_pools = %d outside [1, %d]", n, LORA_MAX_GROUP);
  for (int m = 0; m < n; ++m) {
    const lora_pool* p = pools[m];
    if (!p) return fail(LORA_ERR_INVALID_ARG, "pools[%d] is NULL", m);
    for (int q = 0; q < m; ++q)
      if (pools[q] == p) return fail(LORA_ERR_INVALID_ARG, "pools[%d] repeats pools[%d] (one workspace per pool)", m, q);
    if (p->embedding) return fail(LORA_ERR_INVALID_ARG, "pools[%d] is an embedding pool", m);
    if (p->S != routing->S) return fail(LORA_ERR_SHAPE, "pools[%d] has %d slots, the routing %d", m, p->S, routing->S);
    if (p->device != routing->device) return fail(LORA_ERR_INVALID_ARG, "pools[%d] is on another device", m);
    if (p->wdtype != pools[0]->wdtype) return fail(LORA_ERR_DTYPE, "pools[%d] has another weight dtype", m);
    if (p->Rk != pools[0]->Rk)
      return fail(LORA_ERR_SHAPE, "pools[%d]: max_lora_rank %d pads to another rank step than pools[0]'s %d", m,
                  p->Rmax, pools[0]->Rmax);
    if (T > p->max_tokens) return fail(LORA_ERR_CAPACITY, "T = %d exceeds pools[%d]'s max_tokens = %d", T, m, p->max_tokens);
    lora_status st = check_x(p, T, x[m], ldx[m]);
    if (st != LORA_OK) return st;
    if ((st = check_y(p, T, y[m], ldy[m], ydtype)) != LORA_OK) return st;
  }
  return LORA_OK;
}

lora_status group_impl(const lora_pool* const* pools, int n, const lora_routing* routing, const void* const* x,
                       const int* ldx, void* const* y, const int* ldy, lora_dtype ydtype, hipStream_t stream,
                       const int32_t* self_ids) {
  rax::GroupView G{};
  G.n = n;
  // slot mode for the whole launch when every module would take it on its own
  bool slot = true;
  for (int m = 0; m < n; ++m) slot = slot && slot_mode(pools[m], routing);
  // the shrink launch takes the modules with the longest items (most k steps per
  // part) first, so they are not the last workgroups dispatched; each module's
  // workgroups compute what they would in any order
  int ord[LORA_MAX_GROUP];
  for (int m = 0; m < n; ++m) ord[m] = m;
  auto part_steps = [&](int m) {
    return ceil_div(ceil_div(pools[m]->k, rax::kMfmaK), call_split(pools[m], routing, slot).nsplit);
  };
  if (env_int("RAXLORA_GROUP_ORDER", 1))
    std::stable_sort(ord, ord + n, [&](int a, int b) { return part_steps(a) > part_steps(b); });
  for (int i = 0; i < n; ++i) {
    const int m = ord[i];
    rax::GroupEntry& e = G.e[i];
    e.P = pool_view(pools[m]);
    e.x = x[m];
    e.ldx = ldx[m];
    e.y = y[m];
    e.ldy = ldy[m];
    e.U = workspace_view(pools[m], call_split(pools[m], routing, slot).nsplit, slot);
    e.plan = make_plan(pools[m], routing, false, slot);
  }
  const rax::RouteView R = route_view(routing);
  rax::SelfRoute sr{self_ids, route_out(routing)};
  log_plan(self_ids ? "grouped shrink (routing inside), first module" : "grouped shrink, first module", pools[0],
           routing, G.e[0].plan, n);
  hipError_t e = rax::launch_shrink_group(pools[0]->wdtype, G, R, self_ids ? &sr : nullptr, stream,
                                          timer_for(rax::kKShrink));
  if (e != hipSuccess) return hip_fail(e, "grouped shrink launch");
  for (int i = 0; i < n; ++i) G.e[i].plan = make_plan(pools[ord[i]], routing, true, slot);
  // decode expand units by descending slot rank (the longest first), the rank of a slot
  // taken as its largest over the modules; the order changes when units run, not what
  // they compute
  if (routing->S <= rax::kMaxOrderedSlots && env_int("RAXLORA_GROUP_ORDER", 1)) {
    std::vector<int> idx(routing->S), rk(routing->S, 0);
    for (int s = 0; s < routing->S; ++s) {
      idx[s] = s;
      for (int m = 0; m < n; ++m) rk[s] = std::max(rk[s], pools[m]->mirror[s].rank);
    }
    std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) { return rk[a] > rk[b]; });
    G.order.ordered = 1;
    for (int s = 0; s < routing->S; ++s) G.order.s[s] = (uint8_t)idx[s];
  }
  log_plan("grouped expand, first module", pools[0], routing, G.e[0].plan, n);
  e = rax::launch_expand_group(pools[0]->wdtype, ydtype, G, R, stream, timer_for(rax::kKExpand));
  if (e != hipSuccess) return hip_fail(e, "grouped expand launch");
  return LORA_OK;
}

}  // namespace

extern "C" {

const char* lora_last_error(void) { return g_last_error.c_str(); }

const char* lora_status_string(lora_status s) {
  switch (s) {
    case LORA_OK: return "LORA_OK";
    case LORA_ERR_INVALID_ARG: return "LORA_ERR_INVALID_ARG";
    case LORA_ERR_SHAPE: return "LORA_ERR_SHAPE";
    case LORA_ERR_DTYPE: return "LORA_ERR_DTYPE";
    case LORA_ERR_RANK: return "LORA_ERR_RANK";
    case LORA_ERR_SLOT: return "LORA_ERR_SLOT";
    case LORA_ERR_CAPACITY: return "LORA_ERR_CAPACITY";
    case LORA_ERR_HIP: return "LORA_ERR_HIP";
    case LORA_ERR_OOM: return "LORA_ERR_OOM";
    case LORA_ERR_NO_DEVICE: return "LORA_ERR_NO_DEVICE";
    case LORA_ERR_ALIGN: return "LORA_ERR_ALIGN";
    case LORA_ERR_STATE: return "LORA_ERR_STATE";
    default: return "LORA_ERR_UNKNOWN";
  }
}

lora_status lora_compute_scale(float alpha, int rank, int rslora, float adapter_scale, float* out_scale) {
  if (!out_scale) return fail(LORA_ERR_INVALID_ARG, "out_scale is NULL");
  if (rank < 1) return fail(LORA_ERR_RANK, "rank %d < 1", rank);
  if (!std::isfinite(alpha) || !std::isfinite(adapter_scale))
    return fail(LORA_ERR_INVALID_ARG, "alpha and adapter_scale must be finite");
  const double a = alpha, c = adapter_scale;
  double sigma;
  if (a == 0.0)
    sigma = c;                                   // alpha absent: the caller's scale alone
  else if (rslora)
    sigma = c * a / std::sqrt((double)rank);     // rank-stabilised
  else
    sigma = c * a / (double)rank;
  const float s = (float)sigma;
  if (!std::isfinite(s)) return fail(LORA_ERR_INVALID_ARG, "scale overflows float");
  *out_scale = s;
  return ok();
}

static lora_status create_pool(lora_pool** out, int device, int max_slots, int max_lora_rank, int in_features,
                               const int* slice_out, int num_slices, lora_dtype wdtype, int max_tokens,
                               bool embedding) {
  if (!out || !slice_out) return fail(LORA_ERR_INVALID_ARG, "out and slice_out must not be NULL");
  *out = nullptr;
  if (max_slots < 1 || max_slots > LORA_MAX_SLOTS)
    return fail(LORA_ERR_SHAPE, "max_slots %d outside [1, %d]", max_slots, LORA_MAX_SLOTS);
  if (max_lora_rank < 1 || max_lora_rank > LORA_MAX_RANK)
    return fail(LORA_ERR_SHAPE, "max_lora_rank %d outside [1, %d]", max_lora_rank, LORA_MAX_RANK);
  if (in_features < 1) return fail(LORA_ERR_SHAPE, "in_features %d < 1", in_features);
  if (num_slices < 1 || num_slices > LORA_MAX_SLICES)
    return fail(LORA_ERR_SHAPE, "num_slices %d outside [1, %d]", num_slices, LORA_MAX_SLICES);
  if (max_tokens < 1) return fail(LORA_ERR_SHAPE, "max_tokens %d < 1", max_tokens);
  if (wdtype != LORA_F32 && wdtype != LORA_BF16 && wdtype != LORA_FP8E4M3)
    return fail(LORA_ERR_DTYPE, "unknown wdtype %d", (int)wdtype);
  if (embedding && wdtype == LORA_FP8E4M3) return fail(LORA_ERR_DTYPE, "embedding pools take bf16 or fp32 weights");
  long long D = 0;
  for (int n = 0; n < num_slices; ++n) {
    if (slice_out[n] < 1) return fail(LORA_ERR_SHAPE, "slice %d width %d < 1", n, slice_out[n]);
    if (slice_out[n] % 8) return fail(LORA_ERR_ALIGN, "slice %d width %d not a multiple of 8", n, slice_out[n]);
    D += slice_out[n];
  }
  if (D > (1LL << 30)) return fail(LORA_ERR_SHAPE, "total output width too large");
  // the shrink's 16-byte chunks need k % 8 == 0 and bound k; an embedding pool has no shrink
  if (!embedding && in_features % 8) return fail(LORA_ERR_ALIGN, "in_features %d not a multiple of 8", in_features);
  if (!embedding && in_features > LORA_MAX_IN_FEATURES)
    return fail(LORA_ERR_SHAPE, "in_features %d above LORA_MAX_IN_FEATURES = %d", in_features, LORA_MAX_IN_FEATURES);

  lora_status st = check_device(device);
  if (st != LORA_OK) return st;
  DeviceGuard g(device);
  if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");

  lora_pool* p = new lora_pool();
  p->device = device;
  p->S = max_slots;
  p->Rmax = max_lora_rank;
  p->Rk = (max_lora_rank + rax::kMfmaK - 1) / rax::kMfmaK * rax::kMfmaK;
  p->k = in_features;
  p->N = num_slices;
  p->max_tokens = max_tokens;
  p->wdtype = wdtype;
  p->esize = wdtype == LORA_BF16 ? 2 : wdtype == LORA_FP8E4M3 ? 1 : 4;
  p->embedding = embedding;
  int o = 0, tiles = 0, mblocks = 0;
  for (int n = 0; n < num_slices; ++n) {
    p->d[n] = slice_out[n];
    p->o[n] = o;
    p->tile0[n] = tiles;
    p->mblk0[n] = mblocks;
    o += slice_out[n];
    tiles += (slice_out[n] + rax::kTileCols - 1) / rax::kTileCols;
    mblocks += (slice_out[n] + rax::kMfmaCols - 1) / rax::kMfmaCols;
  }
  p->D = o;
  p->tile0[num_slices] = tiles;
  p->mblk0[num_slices] = mblocks;
  p->mirror.assign(max_slots, SlotEntry{0, 0.f, 0u, 0});
  update_order(p);

  const size_t a_bytes = (size_t)max_slots * num_slices * max_lora_rank * in_features * p->esize;
  const size_t b_bytes = (size_t)max_slots * max_lora_rank * p->D * p->esize;
  const size_t bk_bytes = (size_t)max_slots * p->Rk * p->D * p->esize;
  choose_split(p);
  if (embedding) p->nsplit = p->ns = 1;   // the gathered u is final: one part
  // workspace parts: the most any call can use (the slot-major shrink may split finer)
  const int ws_parts = embedding || wdtype == LORA_F32 ? p->nsplit : std::max(p->nsplit, slot_nsplit(in_features));
  p->heads = !embedding && wdtype != LORA_F32 && max_slots <= kHeadSlots;
  p->ws_rows = max_tokens + (p->heads ? rax::kMfmaTileM * max_slots : 0);
  const size_t ws_bytes = (size_t)ws_parts * num_slices * p->ws_rows * p->Rk * sizeof(float);
  hipError_t e;
  if ((e = hipMalloc(&p->A, a_bytes)) != hipSuccess || (e = hipMalloc(&p->Bt, b_bytes)) != hipSuccess ||
      (e = hipMalloc(&p->Bk, bk_bytes)) != hipSuccess ||
      (e = hipMalloc((void**)&p->table, (size_t)max_slots * sizeof(SlotEntry))) != hipSuccess ||
      (e = hipMalloc((void**)&p->ws, ws_bytes)) != hipSuccess) {
    lora_pool_destroy(p);
    return hip_fail(e, "pool allocation");
  }
  // empty slots read as rank 0; weights start at zero so padding rows are inert
  if ((e = hipMemset(p->A, 0, a_bytes)) != hipSuccess || (e = hipMemset(p->Bt, 0, b_bytes)) != hipSuccess ||
      (e = hipMemset(p->Bk, 0, bk_bytes)) != hipSuccess ||
      (e = hipMemset(p->table, 0, (size_t)max_slots * sizeof(SlotEntry))) != hipSuccess ||
      (e = hipDeviceSynchronize()) != hipSuccess) {
    lora_pool_destroy(p);
    return hip_fail(e, "pool initialisation");
  }
  *out = p;
  return ok();
}

lora_status lora_pool_create(lora_pool** out, int device, int max_slots, int max_lora_rank,
                             int in_features, const int* slice_out, int num_slices,
                             lora_dtype wdtype, int max_tokens) {
  return create_pool(out, device, max_slots, max_lora_rank, in_features, slice_out, num_slices, wdtype, max_tokens,
                     false);
}

lora_status lora_embedding_pool_create(lora_pool** out, int device, int max_slots, int max_lora_rank, int vocab,
                                       int d, lora_dtype wdtype, int max_tokens) {
  const int slice_out[1] = {d};
  return create_pool(out, device, max_slots, max_lora_rank, vocab, slice_out, 1, wdtype, max_tokens, true);
}

lora_status lora_pool_destroy(lora_pool* p) {
  if (!p) return ok();
  DeviceGuard g(p->device);
  if (p->A) (void)hipFree(p->A);
  if (p->Bt) (void)hipFree(p->Bt);
  if (p->Bk) (void)hipFree(p->Bk);
  if (p->table) (void)hipFree(p->table);
  if (p->ws) (void)hipFree(p->ws);

  delete p;
  return ok();
}

lora_status lora_register_adapter(lora_pool* pool, int slot, const void* const* A_slices,
                                  const void* const* B_slices, float alpha, int rank, int rslora,
                                  float adapter_scale, unsigned flags, hipStream_t stream) {
  if (!pool) return fail(LORA_ERR_INVALID_ARG, "pool is NULL");
  if (slot < 0 || slot >= pool->S) return fail(LORA_ERR_SLOT, "slot %d outside [0, %d)", slot, pool->S);
  if (rank < 1 || rank > pool->Rmax)
    return fail(LORA_ERR_RANK, "rank %d outside [1, max_lora_rank = %d]", rank, pool->Rmax);
  if (flags & ~(LORA_SRC_DEVICE | LORA_PREMULTIPLY)) return fail(LORA_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  if (!A_slices || !B_slices) return fail(LORA_ERR_INVALID_ARG, "A_slices and B_slices must not be NULL");
  uint32_t mask = 0;
  for (int n = 0; n < pool->N; ++n) {
    const bool a = A_slices[n] != nullptr, b = B_slices[n] != nullptr;
    if (a != b) return fail(LORA_ERR_INVALID_ARG, "slice %d: lora_a and lora_b must both be given or both be NULL", n);
    if (a) mask |= 1u << n;
  }
  float s = 0.f;
  lora_status st = lora_compute_scale(alpha, rank, rslora, adapter_scale, &s);
  if (st != LORA_OK) return st;
  const bool premul = (flags & LORA_PREMULTIPLY) != 0;
  const bool on_device = (flags & LORA_SRC_DEVICE) != 0;

  DeviceGuard g(pool->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
  const size_t es = pool->esize;
  std::vector<void*> staging;
  auto cleanup = [&]() {
    for (void* q : staging) (void)hipFree(q);
  };
  hipError_t e = hipSuccess;
  for (int n = 0; n < pool->N; ++n) {
    const void* a_src = A_slices[n];
    const void* b_src = B_slices[n];
    if (a_src && !on_device) {
      const size_t abytes = (size_t)rank * pool->k * es, bbytes = (size_t)pool->d[n] * rank * es;
      void *da = nullptr, *db = nullptr;
      if ((e = hipMalloc(&da, abytes)) != hipSuccess) { cleanup(); return hip_fail(e, "staging"); }
      staging.push_back(da);
      if ((e = hipMalloc(&db, bbytes)) != hipSuccess) { cleanup(); return hip_fail(e, "staging"); }
      staging.push_back(db);
      if ((e = hipMemcpy(da, a_src, abytes, hipMemcpyHostToDevice)) != hipSuccess ||
          (e = hipMemcpy(db, b_src, bbytes, hipMemcpyHostToDevice)) != hipSuccess) {
        cleanup();
        return hip_fail(e, "copy of adapter weights");
      }
      a_src = da;
      b_src = db;
    }
    char* A_dst = static_cast<char*>(pool->A) + (((size_t)slot * pool->N + n) * pool->Rmax) * pool->k * es;
    char* Bt_dst = static_cast<char*>(pool->Bt) + ((size_t)slot * pool->Rmax * pool->D + pool->o[n]) * es;
    char* Bk_dst = static_cast<char*>(pool->Bk) +
                   ((size_t)slot * pool->D * pool->Rk + (size_t)pool->o[n] * rax::bk_stride(rank)) * es;
    e = rax::launch_pack_slice(pool->wdtype, a_src, b_src, A_dst, Bt_dst, Bk_dst, rank, pool->Rmax,
                               pool->Rk, pool->k, pool->d[n], pool->D, s, premul ? 1 : 0, pool->embedding ? 1 : 0,
                               stream);
    if (e != hipSuccess) { cleanup(); return hip_fail(e, "pack launch"); }
  }
  const SlotEntry entry{rank, premul ? 1.0f : s, mask, 0};
  e = rax::launch_set_slot(pool->table, slot, entry, stream);
  if (e != hipSuccess) { cleanup(); return hip_fail(e, "slot table update"); }
  if (!staging.empty()) {
    if ((e = hipStreamSynchronize(stream)) != hipSuccess) { cleanup(); return hip_fail(e, "registration sync"); }
    cleanup();
  }
  pool->mirror[slot] = entry;
  update_order(pool);
  return ok();
}

lora_status lora_unregister_adapter(lora_pool* pool, int slot, hipStream_t stream) {
  if (!pool) return fail(LORA_ERR_INVALID_ARG, "pool is NULL");
  if (slot < 0 || slot >= pool->S) return fail(LORA_ERR_SLOT, "slot %d outside [0, %d)", slot, pool->S);
  DeviceGuard g(pool->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
  const SlotEntry entry{0, 0.f, 0u, 0};
  hipError_t e = rax::launch_set_slot(pool->table, slot, entry, stream);
  if (e != hipSuccess) return hip_fail(e, "slot table update");
  pool->mirror[slot] = entry;
  update_order(pool);
  return ok();
}

lora_status lora_pool_slot_info(const lora_pool* pool, int slot, int* rank, float* scale,
                                uint32_t* slice_mask, uint64_t* a_offset, uint64_t* bt_offset) {
  if (!pool) return fail(LORA_ERR_INVALID_ARG, "pool is NULL");
  if (slot < 0 || slot >= pool->S) return fail(LORA_ERR_SLOT, "slot %d outside [0, %d)", slot, pool->S);
  const SlotEntry& e = pool->mirror[slot];
  if (rank) *rank = e.rank;
  if (scale) *scale = e.scale;
  if (slice_mask) *slice_mask = e.slice_mask;
  if (a_offset) *a_offset = (uint64_t)slot * pool->N * pool->Rmax * pool->k * pool->esize;
  if (bt_offset) *bt_offset = (uint64_t)slot * pool->Rmax * pool->D * pool->esize;
  return ok();
}

lora_status lora_pool_read_slot(const lora_pool* pool, int slot, int slice, void* A_host, void* Bt_host) {
  if (!pool) return fail(LORA_ERR_INVALID_ARG, "pool is NULL");
  if (slot < 0 || slot >= pool->S) return fail(LORA_ERR_SLOT, "slot %d outside [0, %d)", slot, pool->S);
  if (slice < 0 || slice >= pool->N) return fail(LORA_ERR_SHAPE, "slice %d outside [0, %d)", slice, pool->N);
  DeviceGuard g(pool->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
  const size_t es = pool->esize;
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "synchronize");
  if (A_host) {
    const char* src = static_cast<const char*>(pool->A) + (((size_t)slot * pool->N + slice) * pool->Rmax) * pool->k * es;
    if ((e = hipMemcpy(A_host, src, (size_t)pool->Rmax * pool->k * es, hipMemcpyDeviceToHost)) != hipSuccess)
      return hip_fail(e, "copy A");
  }
  if (Bt_host) {
    const char* src = static_cast<const char*>(pool->Bt) + ((size_t)slot * pool->Rmax * pool->D + pool->o[slice]) * es;
    if ((e = hipMemcpy2D(Bt_host, (size_t)pool->d[slice] * es, src, (size_t)pool->D * es,
                         (size_t)pool->d[slice] * es, pool->Rmax, hipMemcpyDeviceToHost)) != hipSuccess)
      return hip_fail(e, "copy Bt");
  }
  return ok();
}

lora_status lora_routing_create(lora_routing** out, int device, int max_tokens, int max_slots) {
  if (!out) return fail(LORA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (max_tokens < 1) return fail(LORA_ERR_SHAPE, "max_tokens %d < 1", max_tokens);
  if (max_slots < 1 || max_slots > LORA_MAX_SLOTS)
    return fail(LORA_ERR_SHAPE, "max_slots %d outside [1, %d]", max_slots, LORA_MAX_SLOTS);
  lora_status st = check_device(device);
  if (st != LORA_OK) return st;
  DeviceGuard g(device);
  if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
  lora_routing* r = new lora_routing();
  r->device = device;
  r->max_tokens = max_tokens;
  r->S = max_slots;
  r->mfma_min = env_int("RAXLORA_MFMA_MIN_SEG", rax::kDefaultMfmaMinSeg);
  if (r->mfma_min < 1) r->mfma_min = 1;
  r->tile_m = rax::kMfmaTileM;
  // sum over long segments of ceil(len / tile_m) <= T / tile_m + (number of long segments)
  r->max_tiles = max_tokens / r->tile_m + 1 + max_slots;
  // layout: meta, rec[S] (128-byte records), desc[S], tiles[max_tiles] (16-byte
  // entries first, so they stay 16-byte aligned), then counts[S+1], offs[S+2],
  // sorted[max_tokens], active[S]
  const size_t words = rax::kMetaWords + (size_t)rax::kRecInts * max_slots + 4 * (size_t)max_slots +
                       4 * (size_t)r->max_tiles + (size_t)(max_slots + 1) + (max_slots + 2) + max_tokens +
                       max_slots;
  hipError_t e = hipMalloc((void**)&r->buf, words * sizeof(int));
  if (e != hipSuccess) {
    delete r;
    return hip_fail(e, "routing allocation");
  }
  if ((e = hipMemset(r->buf, 0, words * sizeof(int))) != hipSuccess || (e = hipDeviceSynchronize()) != hipSuccess) {
    (void)hipFree(r->buf);
    delete r;
    return hip_fail(e, "routing initialisation");
  }
  int* w = r->buf;
  r->meta = w; w += rax::kMetaWords;
  r->rec = w; w += (size_t)rax::kRecInts * max_slots;
  r->desc = reinterpret_cast<int4*>(w); w += 4 * max_slots;
  r->tiles = reinterpret_cast<int4*>(w); w += 4 * r->max_tiles;
  r->counts = w; w += max_slots + 1;
  r->offs = w; w += max_slots + 2;
  r->sorted = w; w += max_tokens;
  r->active = w;
  *out = r;
  return ok();
}

lora_status lora_routing_destroy(lora_routing* r) {
  if (!r) return ok();
  DeviceGuard g(r->device);
  if (r->buf) (void)hipFree(r->buf);
  delete r;
  return ok();
}

lora_status lora_build_routing(lora_routing* r, const int32_t* ids, int T, hipStream_t stream) {
  return lora_build_routing_seq(r, ids, T, 1, stream);
}

lora_status lora_build_routing_seq(lora_routing* r, const int32_t* seq_slot_ids, int num_seqs, int tokens_per_seq,
                                   hipStream_t stream) {
  if (!r) return fail(LORA_ERR_INVALID_ARG, "routing is NULL");
  if (num_seqs < 0) return fail(LORA_ERR_SHAPE, "num_seqs = %d < 0", num_seqs);
  if (tokens_per_seq < 1) return fail(LORA_ERR_SHAPE, "tokens_per_seq = %d < 1", tokens_per_seq);
  const long long T = (long long)num_seqs * tokens_per_seq;
  if (T > r->max_tokens) return fail(LORA_ERR_CAPACITY, "T = %lld exceeds max_tokens = %d", T, r->max_tokens);
  if (T > 0 && !seq_slot_ids) return fail(LORA_ERR_INVALID_ARG, "slot ids are NULL");
  DeviceGuard g(r->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
  hipError_t e = rax::launch_routing(seq_slot_ids, (int)T, tokens_per_seq, r->S, r->mfma_min, r->tile_m, r->max_tiles,
                                     r->counts, r->offs, r->sorted, r->active, r->desc, r->tiles, r->rec, r->meta,
                                     stream, timer_for(rax::kKRouting));
  if (e != hipSuccess) return hip_fail(e, "routing launch");
  r->T = (int)T;
  return ok();
}

lora_status lora_routing_query(const lora_routing* r, int32_t* counts, int32_t* seg_offsets,
                               int32_t* sorted_ids, int32_t* active_slots, int* num_active,
                               int* n_invalid) {
  if (!r) return fail(LORA_ERR_INVALID_ARG, "routing is NULL");
  if (r->T < 0) return fail(LORA_ERR_STATE, "routing was never built");
  DeviceGuard g(r->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "synchronize");
  int meta[rax::kMetaWords];
  if ((e = hipMemcpy(meta, r->meta, sizeof meta, hipMemcpyDeviceToHost)) != hipSuccess) return hip_fail(e, "copy meta");
  if (counts && (e = hipMemcpy(counts, r->counts, (r->S + 1) * sizeof(int), hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "copy counts");
  if (seg_offsets && (e = hipMemcpy(seg_offsets, r->offs, (r->S + 2) * sizeof(int), hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "copy offsets");
  if (sorted_ids && r->T > 0 &&
      (e = hipMemcpy(sorted_ids, r->sorted, (size_t)r->T * sizeof(int), hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "copy sorted ids");
  if (active_slots && (e = hipMemcpy(active_slots, r->active, r->S * sizeof(int), hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "copy active slots");
  if (num_active) *num_active = meta[rax::kMetaActive];
  if (n_invalid) *n_invalid = meta[rax::kMetaInvalid];
  return ok();
}

lora_status lora_shrink(const lora_pool* pool, const lora_routing* routing, const void* x, int ldx,
                        float* u, hipStream_t stream) {
  lora_status st = check_pair(pool, routing);
  if (st != LORA_OK) return st;
  if ((st = check_x(pool, routing->T, x, ldx)) != LORA_OK) return st;
  if (routing->T > 0 && !u) return fail(LORA_ERR_INVALID_ARG, "u is NULL");
  if (!aligned16(u)) return fail(LORA_ERR_ALIGN, "u must be 16-byte aligned");
  if (routing->T == 0) return ok();
  DeviceGuard g(pool->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
  // split partials into the workspace, then finished in split order into the caller's u
  const bool slot = slot_mode(pool, routing);
  const rax::UView W = workspace_view(pool, call_split(pool, routing, slot).nsplit);
  if ((st = run_shrink(pool, routing, x, ldx, W, stream, slot)) != LORA_OK) return st;
  const rax::Plan pl = make_plan(pool, routing, false, slot);
  hipError_t e = rax::launch_finish_u(pool_view(pool), route_view(routing), W, caller_u_view(pool, routing, u),
                                      pl, stream, timer_for(rax::kKFinish));
  if (e != hipSuccess) return hip_fail(e, "finish launch");
  return ok();
}

lora_status lora_expand(const lora_pool* pool, const lora_routing* routing, const float* u, void* y,
                        int ldy, lora_dtype ydtype, hipStream_t stream) {
  lora_status st = check_pair(pool, routing);
  if (st != LORA_OK) return st;
  if ((st = check_y(pool, routing->T, y, ldy, ydtype)) != LORA_OK) return st;
  if (routing->T > 0 && !u) return fail(LORA_ERR_INVALID_ARG, "u is NULL");
  if (!aligned16(u)) return fail(LORA_ERR_ALIGN, "u must be 16-byte aligned");
  if (routing->T == 0) return ok();
  DeviceGuard g(pool->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
  const rax::UView U = caller_u_view(pool, routing, const_cast<float*>(u));
  if ((st = run_expand(pool, routing, U, y, ldy, ydtype, stream, false)) != LORA_OK) return st;
  return ok();
}

lora_status lora_linear(const lora_pool* pool, const lora_routing* routing, const void* x, int ldx,
                        void* y, int ldy, lora_dtype ydtype, hipStream_t stream) {
  return linear_impl(pool, routing, x, ldx, y, ldy, ydtype, stream, nullptr);
}

lora_status lora_linear_noalloc(const lora_pool* pool, const lora_routing* routing, const void* x, int ldx, void* y,
                                int ldy, lora_dtype ydtype, hipStream_t stream) {
  lora_status st = check_pair(pool, routing);
  if (st != LORA_OK) return st;
  if ((st = check_x(pool, routing->T, x, ldx)) != LORA_OK) return st;
  if ((st = check_y(pool, routing->T, y, ldy, ydtype)) != LORA_OK) return st;
  if (routing->T == 0) return ok();
  // the partials of this call: [nsplit][N][rows][Rk] fp32, rows by sorted position, then
  // in slot mode the first-tile rows of the pool's slots when they fit as well
  const bool slot = slot_mode(pool, routing);
  const CallSplit cs = call_split(pool, routing, slot);
  auto bytes = [&](long long rows) { return (size_t)cs.nsplit * pool->N * rows * pool->Rk * sizeof(float); };
  const bool heads = slot && pool->heads &&
                     bytes(routing->T + (long long)rax::kMfmaTileM * pool->S) <= rax::kNoAllocScratchBytes;
  const long long rows = routing->T + (heads ? (long long)rax::kMfmaTileM * pool->S : 0);
  const size_t need = bytes(rows);
  if (need > rax::kNoAllocScratchBytes)
    return fail(LORA_ERR_CAPACITY, "this call needs %zu bytes of scratch (%d k splits x %d slices x %d tokens x %d "
                "ranks x 4), above the %zu-byte array", need, cs.nsplit, pool->N, routing->T, pool->Rk,
                rax::kNoAllocScratchBytes);
  DeviceGuard g(pool->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
  void* scratch = nullptr;
  hipError_t e = rax::noalloc_scratch(pool->device, &scratch);
  if (e != hipSuccess) return hip_fail(e, "scratch address");
  rax::UView W{static_cast<float*>(scratch), (long long)pool->N * rows * pool->Rk, rows * pool->Rk, pool->Rk,
               cs.nsplit, 0};
  W.head0 = heads ? routing->T : -1;
  if ((st = run_shrink(pool, routing, x, ldx, W, stream, slot)) != LORA_OK) return st;
  if ((st = run_expand(pool, routing, W, y, ldy, ydtype, stream, slot)) != LORA_OK) return st;
  return ok();
}

lora_status lora_linear_join(const lora_pool* pool, const lora_routing* routing, const void* x, int ldx,
                             void* y, int ldy, lora_dtype ydtype, hipStream_t stream, hipEvent_t y_ready) {
  return linear_impl(pool, routing, x, ldx, y, ldy, ydtype, stream, y_ready);
}

lora_status lora_route_linear(const lora_pool* pool, lora_routing* routing, const int32_t* ids, int T,
                              const void* x, int ldx, void* y, int ldy, lora_dtype ydtype, hipStream_t stream) {
  return route_linear_impl(pool, routing, ids, T, x, ldx, y, ldy, ydtype, stream, nullptr);
}

lora_status lora_route_linear_join(const lora_pool* pool, lora_routing* routing, const int32_t* ids, int T,
                                   const void* x, int ldx, void* y, int ldy, lora_dtype ydtype, hipStream_t stream,
                                   hipEvent_t y_ready) {
  return route_linear_impl(pool, routing, ids, T, x, ldx, y, ldy, ydtype, stream, y_ready);
}

lora_status lora_linear_group(const lora_pool* const* pools, int num_pools, const lora_routing* routing,
                              const void* const* x, const int* ldx, void* const* y, const int* ldy, lora_dtype ydtype,
                              hipStream_t stream) {
  if (!routing) return fail(LORA_ERR_INVALID_ARG, "routing is NULL");
  if (routing->T < 0) return fail(LORA_ERR_STATE, "routing was never built");
  lora_status st = check_group(pools, num_pools, routing, routing->T, x, ldx, y, ldy, ydtype);
  if (st != LORA_OK) return st;
  if (routing->T == 0) return ok();
  DeviceGuard g(routing->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
  st = group_impl(pools, num_pools, routing, x, ldx, y, ldy, ydtype, stream, nullptr);
  return st == LORA_OK ? ok() : st;
}

lora_status lora_route_linear_group(const lora_pool* const* pools, int num_pools, lora_routing* routing,
                                    const int32_t* ids, int T, const void* const* x, const int* ldx, void* const* y,
                                    const int* ldy, lora_dtype ydtype, hipStream_t stream) {
  if (!routing) return fail(LORA_ERR_INVALID_ARG, "routing is NULL");
  if (T < 0) return fail(LORA_ERR_SHAPE, "T = %d < 0", T);
  if (T > routing->max_tokens) return fail(LORA_ERR_CAPACITY, "T = %d exceeds max_tokens = %d", T, routing->max_tokens);
  if (T > 0 && !ids) return fail(LORA_ERR_INVALID_ARG, "token_slot_ids is NULL");
  lora_status st = check_group(pools, num_pools, routing, T, x, ldx, y, ldy, ydtype);
  if (st != LORA_OK) return st;
  // batches the shrink launch can route itself; others: the routing launch first
  if (T < 1 || T > rax::kSelfRouteTokens || routing->S + 1 > rax::kSelfRouteKeys) {
    if ((st = lora_build_routing(routing, ids, T, stream)) != LORA_OK) return st;
    return lora_linear_group(pools, num_pools, routing, x, ldx, y, ldy, ydtype, stream);
  }
  DeviceGuard g(routing->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
  routing->T = T;
  st = group_impl(pools, num_pools, routing, x, ldx, y, ldy, ydtype, stream, ids);
  if (st != LORA_OK) routing->T = -1;   // the routing may not have been built: unusable until rebuilt
  return st == LORA_OK ? ok() : st;
}

lora_status lora_embedding(const lora_pool* pool, const lora_routing* routing, const int32_t* vocab_ids, void* y,
                           int ldy, lora_dtype ydtype, hipStream_t stream) {
  if (!pool || !routing) return fail(LORA_ERR_INVALID_ARG, "pool and routing must not be NULL");
  if (!pool->embedding) return fail(LORA_ERR_INVALID_ARG, "not an embedding pool (lora_embedding_pool_create)");
  lora_status st = check_pair(pool, routing);
  if (st != LORA_OK) return st;
  if ((st = check_y(pool, routing->T, y, ldy, ydtype)) != LORA_OK) return st;
  if (routing->T > 0 && !vocab_ids) return fail(LORA_ERR_INVALID_ARG, "vocab_ids is NULL");
  if (routing->T == 0) return ok();
  DeviceGuard g(pool->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
  const rax::UView W = workspace_view(pool, 1);
  hipError_t e = rax::launch_embed_gather(pool->wdtype, pool_view(pool), route_view(routing), vocab_ids, pool->k, W,
                                          stream, timer_for(rax::kKGather));
  if (e != hipSuccess) return hip_fail(e, "gather launch");
  if ((st = run_expand(pool, routing, W, y, ldy, ydtype, stream, false)) != LORA_OK) return st;
  return ok();
}

lora_status lora_route_embedding(const lora_pool* pool, lora_routing* routing, const int32_t* slot_ids, int T,
                                 const int32_t* vocab_ids, void* y, int ldy, lora_dtype ydtype, hipStream_t stream) {
  if (!pool || !routing) return fail(LORA_ERR_INVALID_ARG, "pool and routing must not be NULL");
  if (!pool->embedding) return fail(LORA_ERR_INVALID_ARG, "not an embedding pool (lora_embedding_pool_create)");
  if (T < 0) return fail(LORA_ERR_SHAPE, "T = %d < 0", T);
  if (T > routing->max_tokens) return fail(LORA_ERR_CAPACITY, "T = %d exceeds max_tokens = %d", T, routing->max_tokens);
  if (T > 0 && (!slot_ids || !vocab_ids)) return fail(LORA_ERR_INVALID_ARG, "slot ids or vocab_ids NULL");
  if (routing->S != pool->S) return fail(LORA_ERR_SHAPE, "routing has %d slots, pool has %d", routing->S, pool->S);
  if (routing->device != pool->device)
    return fail(LORA_ERR_INVALID_ARG, "routing on device %d, pool on device %d", routing->device, pool->device);
  if (T > pool->max_tokens) return fail(LORA_ERR_CAPACITY, "T = %d exceeds the pool's max_tokens = %d", T, pool->max_tokens);
  lora_status st = check_y(pool, T, y, ldy, ydtype);
  if (st != LORA_OK) return st;
  if (T == 0) return lora_build_routing(routing, slot_ids, 0, stream);
  DeviceGuard g(pool->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
  // u by token index in the workspace, read by the expand as a caller's finished u
  const rax::UView U{pool->ws, 0, (long long)pool->max_tokens * pool->Rk, pool->Rk, 1, 1};
  const bool fused = T <= rax::kSelfRouteTokens && pool->S + 1 <= rax::kSelfRouteKeys;
  if (!fused && (st = lora_build_routing(routing, slot_ids, T, stream)) != LORA_OK) return st;
  routing->T = T;
  rax::SelfRoute sr{slot_ids, route_out(routing)};
  hipError_t e = rax::launch_embed_gather_tok(pool->wdtype, pool_view(pool), route_view(routing), slot_ids, vocab_ids,
                                              pool->k, U, fused ? &sr : nullptr, stream, timer_for(rax::kKGather));
  if (e != hipSuccess) {
    if (fused) routing->T = -1;   // the routing was not built: unusable until rebuilt
    return hip_fail(e, "gather launch");
  }
  if ((st = run_expand(pool, routing, U, y, ldy, ydtype, stream, false)) != LORA_OK) return st;
  return ok();
}

lora_status lora_bandwidth_probe(const void* src, uint64_t read_bytes, void* dst, uint64_t dst_bytes, int ratio,
                                 hipStream_t stream) {
  if (!src || !dst) return fail(LORA_ERR_INVALID_ARG, "src and dst must not be NULL");
  if (!aligned16(src) || !aligned16(dst)) return fail(LORA_ERR_ALIGN, "src and dst must be 16-byte aligned");
  if (read_bytes < 16) return fail(LORA_ERR_SHAPE, "read_bytes %llu < 16", (unsigned long long)read_bytes);
  if (ratio <= 0 && dst_bytes < (uint64_t)256 * 16 * 256 * sizeof(uint32_t))
    return fail(LORA_ERR_SHAPE, "the read form needs dst_bytes >= 4 MiB");
  if (ratio > 0 && (read_bytes / 16 / (uint64_t)ratio == 0 || read_bytes / 16 / (uint64_t)ratio * 16 > dst_bytes))
    return fail(LORA_ERR_SHAPE, "dst_bytes below read_bytes / ratio");
  hipError_t e = rax::launch_bandwidth_probe(src, read_bytes, dst, dst_bytes, ratio, stream);
  if (e != hipSuccess) return hip_fail(e, "probe launch");
  return ok();
}

lora_status lora_index_checks(int* enabled, unsigned long long* faults, int reset) {
  if (!enabled || !faults) return fail(LORA_ERR_INVALID_ARG, "enabled and faults must not be NULL");
  *faults = 0;
#ifdef RAXLORA_DEBUG
  *enabled = 1;
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "synchronising before reading the index checks");
  using Reader = hipError_t (*)(unsigned int*, bool);
  const Reader readers[] = {rax::index_faults_linear,    rax::index_faults_routing,   rax::index_faults_w16_y16,
                            rax::index_faults_w16_y32,   rax::index_faults_w32_y32,   rax::index_faults_w8_y16,
                            rax::index_faults_w8_y32};
  for (Reader rd : readers) {
    unsigned int v = 0;
    if ((e = rd(&v, reset != 0)) != hipSuccess) return hip_fail(e, "reading the index checks");
    *faults += v;
  }
#else
  (void)reset;
  *enabled = 0;
#endif
  return ok();
}

lora_status lora_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  g_timing_on = on != 0;
  return ok();
}

const char* lora_timing_kernel_name(int kernel) {
  return (kernel >= 0 && kernel < rax::kKernelCount) ? kKernelNames[kernel] : "";
}

lora_status lora_timing_report(double* total_ms, int* launches, int max_kernels) {
  if (max_kernels < 0 || (max_kernels > 0 && (!total_ms || !launches)))
    return fail(LORA_ERR_INVALID_ARG, "total_ms and launches must hold max_kernels entries");
  std::vector<TimingRecord> recs;
  {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    recs.swap(g_timing_records);
  }
  for (int i = 0; i < max_kernels; ++i) {
    total_ms[i] = 0.0;
    launches[i] = 0;
  }
  lora_status st = LORA_OK;
  for (const TimingRecord& r : recs) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess && st == LORA_OK) st = hip_fail(e, "timing event");
    if (e == hipSuccess && r.kernel < max_kernels) {
      total_ms[r.kernel] += ms;
      launches[r.kernel] += 1;
    }
  }
  {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    for (const TimingRecord& r : recs) {
      g_free_events.push_back(r.start);
      g_free_events.push_back(r.stop);
    }
  }
  return st == LORA_OK ? ok() : st;
}

}  // extern "C"
