// Drives every entry point of the C ABI through its host code (argument checks, object
// lifetimes, registration bookkeeping, launch planning) under AddressSanitizer and
// UndefinedBehaviorSanitizer, with the HIP runtime and the kernel launchers replaced by
// host stand-ins (hip_stubs.cpp).  Exits non-zero on a wrong status code; the
// sanitizers abort on a memory or undefined-behaviour error.  Test infrastructure only.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "raxlora.h"

extern int g_launches;
static int g_fail = 0;

#define EXPECT(call, want)                                                                              \
  do {                                                                                                  \
    const lora_status st_ = (call);                                                                     \
    if (st_ != (want)) {                                                                                \
      std::fprintf(stderr, "%s:%d: %s -> %s (want %s): %s\n", __FILE__, __LINE__, #call,                  \
                   lora_status_string(st_), lora_status_string(want), lora_last_error());               \
      ++g_fail;                                                                                         \
    }                                                                                                   \
  } while (0)

int main() {
  std::mt19937 rng(5);
  // scale: every rank, signs, alpha missing, rsLoRA, overflow
  for (int i = 0; i < 20000; ++i) {
    float s = 0.f;
    const float alpha = (float)((int)(rng() % 257) - 128) * 0.5f;
    const int rank = 1 + (int)(rng() % 256);
    EXPECT(lora_compute_scale(alpha, rank, (int)(rng() & 1), 1.0f, &s), LORA_OK);
  }
  float s = 0.f;
  EXPECT(lora_compute_scale(3e38f, 1, 0, 3e38f, &s), LORA_ERR_INVALID_ARG);
  EXPECT(lora_compute_scale(NAN, 4, 0, 1.f, &s), LORA_ERR_INVALID_ARG);
  EXPECT(lora_compute_scale(1.f, 0, 0, 1.f, &s), LORA_ERR_RANK);

  // pools of several shapes and dtypes; registration from host memory
  const int slices_qkv[3] = {4096, 1024, 1024}, slices_gu[2] = {14336, 14336}, slices_down[1] = {4096};
  lora_pool *qkv = nullptr, *gu = nullptr, *down = nullptr, *f32 = nullptr, *fp8 = nullptr, *emb = nullptr;
  EXPECT(lora_pool_create(&qkv, 0, 64, 16, 4096, slices_qkv, 3, LORA_BF16, 256), LORA_OK);
  EXPECT(lora_pool_create(&gu, 0, 64, 16, 4096, slices_gu, 2, LORA_BF16, 256), LORA_OK);
  EXPECT(lora_pool_create(&down, 0, 64, 16, 14336, slices_down, 1, LORA_BF16, 256), LORA_OK);
  EXPECT(lora_pool_create(&f32, 0, 8, 9, 264, slices_down, 1, LORA_F32, 64), LORA_OK);
  EXPECT(lora_pool_create(&fp8, 0, 64, 16, 4096, slices_qkv, 3, LORA_FP8E4M3, 256), LORA_OK);
  const int bad_w[2] = {4096, 1020};
  lora_pool* bad = nullptr;
  EXPECT(lora_pool_create(&bad, 0, 64, 16, 4096, bad_w, 2, LORA_BF16, 256), LORA_ERR_ALIGN);
  EXPECT(lora_pool_create(&bad, 0, 0, 16, 4096, slices_down, 1, LORA_BF16, 256), LORA_ERR_SHAPE);
  EXPECT(lora_pool_create(&bad, 0, 64, 300, 4096, slices_down, 1, LORA_BF16, 256), LORA_ERR_SHAPE);
  EXPECT(lora_pool_create(&bad, 3, 64, 16, 4096, slices_down, 1, LORA_BF16, 256), LORA_ERR_NO_DEVICE);
  EXPECT(lora_embedding_pool_create(&emb, 0, 8, 16, 32000, 4096, LORA_BF16, 64), LORA_OK);

  std::vector<uint16_t> A(16 * 14336), B(14336 * 16);
  for (auto& v : A) v = (uint16_t)(rng() & 0x3fff);
  for (auto& v : B) v = (uint16_t)(rng() & 0x3fff);
  const void* a3[3] = {A.data(), A.data(), nullptr};
  const void* b3[3] = {B.data(), B.data(), nullptr};
  for (int slot = 0; slot < 64; ++slot) {
    const int rank = 1 + slot % 16;
    EXPECT(lora_register_adapter(qkv, slot, a3, b3, 16.f, rank, 1, 1.f, (slot & 1) ? LORA_PREMULTIPLY : 0u, nullptr),
           LORA_OK);
    EXPECT(lora_register_adapter(gu, slot, a3, b3, 32.f, rank, 0, 0.5f, 0u, nullptr), LORA_OK);
    EXPECT(lora_register_adapter(down, slot, a3, b3, 0.f, rank, 0, 2.f, 0u, nullptr), LORA_OK);
    EXPECT(lora_register_adapter(fp8, slot, a3, b3, 16.f, rank, 0, 1.f, LORA_PREMULTIPLY, nullptr), LORA_OK);
  }
  const void* half_a[3] = {A.data(), nullptr, nullptr};
  const void* half_b[3] = {nullptr, nullptr, nullptr};
  EXPECT(lora_register_adapter(qkv, 0, half_a, half_b, 16.f, 4, 0, 1.f, 0u, nullptr), LORA_ERR_INVALID_ARG);
  EXPECT(lora_register_adapter(qkv, 64, a3, b3, 16.f, 4, 0, 1.f, 0u, nullptr), LORA_ERR_SLOT);
  EXPECT(lora_register_adapter(qkv, 0, a3, b3, 16.f, 17, 0, 1.f, 0u, nullptr), LORA_ERR_RANK);
  EXPECT(lora_register_adapter(qkv, 0, a3, b3, 16.f, 4, 0, 1.f, 8u, nullptr), LORA_ERR_INVALID_ARG);
  EXPECT(lora_unregister_adapter(qkv, 5, nullptr), LORA_OK);
  EXPECT(lora_unregister_adapter(qkv, -1, nullptr), LORA_ERR_SLOT);
  int rank = 0;
  float scale = 0.f;
  uint32_t mask = 0;
  uint64_t ao = 0, bo = 0;
  EXPECT(lora_pool_slot_info(qkv, 3, &rank, &scale, &mask, &ao, &bo), LORA_OK);
  if (rank != 4 || mask != 3u) { std::fprintf(stderr, "slot info rank %d mask %u\n", rank, mask); ++g_fail; }
  std::vector<uint16_t> Ah(16 * 4096), Bh(16 * 4096);
  EXPECT(lora_pool_read_slot(qkv, 3, 0, Ah.data(), Bh.data()), LORA_OK);
  EXPECT(lora_pool_read_slot(qkv, 3, 3, Ah.data(), Bh.data()), LORA_ERR_SHAPE);

  // routing objects; the host code's view of a batch before and after a build
  lora_routing *r256 = nullptr, *r1024 = nullptr;
  EXPECT(lora_routing_create(&r256, 0, 256, 64), LORA_OK);
  EXPECT(lora_routing_create(&r1024, 0, 1024, 64), LORA_OK);
  std::vector<int32_t> ids(1024);
  for (auto& v : ids) v = (int32_t)(rng() % 66) - 1;
  std::vector<uint16_t> x(1024 * 14336), y(1024 * 28672);
  std::vector<float> u(3 * 256 * 16);
  EXPECT(lora_linear(qkv, r256, x.data(), 4096, y.data(), 6144, LORA_BF16, nullptr), LORA_ERR_STATE);
  EXPECT(lora_build_routing(r256, ids.data(), 257, nullptr), LORA_ERR_CAPACITY);
  EXPECT(lora_build_routing(r256, ids.data(), 256, nullptr), LORA_OK);
  EXPECT(lora_build_routing_seq(r256, ids.data(), 64, 4, nullptr), LORA_OK);
  EXPECT(lora_build_routing_seq(r256, ids.data(), 65, 4, nullptr), LORA_ERR_CAPACITY);
  int na = 0, ni = 0;
  std::vector<int32_t> counts(65), offs(66), sorted(256), active(64);
  EXPECT(lora_routing_query(r256, counts.data(), offs.data(), sorted.data(), active.data(), &na, &ni), LORA_OK);

  // every fused call, with the plans the host computes for these shapes
  EXPECT(lora_linear(qkv, r256, x.data(), 4096, y.data(), 6144, LORA_BF16, nullptr), LORA_OK);
  EXPECT(lora_linear(qkv, r256, x.data(), 4096, y.data(), 6144, LORA_F32, nullptr), LORA_OK);
  EXPECT(lora_linear(qkv, r256, x.data(), 4000, y.data(), 6144, LORA_BF16, nullptr), LORA_ERR_SHAPE);
  EXPECT(lora_linear(qkv, r256, x.data(), 4096, y.data() + 1, 6144, LORA_BF16, nullptr), LORA_ERR_ALIGN);
  EXPECT(lora_linear(qkv, r256, x.data(), 4096, y.data(), 6144, (lora_dtype)7, nullptr), LORA_ERR_DTYPE);
  EXPECT(lora_linear(f32, r256, x.data(), 264, y.data(), 4096, LORA_F32, nullptr), LORA_ERR_SHAPE);
  EXPECT(lora_shrink(qkv, r256, x.data(), 4096, u.data(), nullptr), LORA_OK);
  EXPECT(lora_expand(qkv, r256, u.data(), y.data(), 6144, LORA_BF16, nullptr), LORA_OK);
  EXPECT(lora_linear_noalloc(qkv, r256, x.data(), 4096, y.data(), 6144, LORA_BF16, nullptr), LORA_OK);
  EXPECT(lora_linear_join(qkv, r256, x.data(), 4096, y.data(), 6144, LORA_BF16, nullptr, nullptr), LORA_OK);
  EXPECT(lora_route_linear(qkv, r256, ids.data(), 256, x.data(), 4096, y.data(), 6144, LORA_BF16, nullptr), LORA_OK);
  EXPECT(lora_route_linear(fp8, r256, ids.data(), 200, x.data(), 4096, y.data(), 6144, LORA_BF16, nullptr), LORA_OK);
  EXPECT(lora_route_linear(qkv, r1024, ids.data(), 1024, x.data(), 4096, y.data(), 6144, LORA_BF16, nullptr),
         LORA_ERR_CAPACITY);   // the pool holds 256 tokens
  const lora_pool* group[3] = {qkv, gu, down};
  const void* xs[3] = {x.data(), x.data(), x.data()};
  void* ys[3] = {y.data(), y.data(), y.data()};
  const int ldx[3] = {4096, 4096, 14336}, ldy[3] = {6144, 28672, 4096};
  EXPECT(lora_route_linear_group(group, 3, r256, ids.data(), 256, xs, ldx, ys, ldy, LORA_BF16, nullptr), LORA_OK);
  EXPECT(lora_linear_group(group, 3, r256, xs, ldx, ys, ldy, LORA_BF16, nullptr), LORA_OK);
  const lora_pool* twice[2] = {qkv, qkv};
  EXPECT(lora_linear_group(twice, 2, r256, xs, ldx, ys, ldy, LORA_BF16, nullptr), LORA_ERR_INVALID_ARG);
  const lora_pool* mixed[2] = {qkv, fp8};
  EXPECT(lora_linear_group(mixed, 2, r256, xs, ldx, ys, ldy, LORA_BF16, nullptr), LORA_ERR_DTYPE);
  EXPECT(lora_linear_group(group, 9, r256, xs, ldx, ys, ldy, LORA_BF16, nullptr), LORA_ERR_SHAPE);
  EXPECT(lora_build_routing(r256, ids.data(), 0, nullptr), LORA_OK);
  EXPECT(lora_linear(qkv, r256, nullptr, 4096, nullptr, 6144, LORA_BF16, nullptr), LORA_OK);   // empty batch
  std::vector<int32_t> vocab(64, 7);
  EXPECT(lora_route_embedding(emb, r256, ids.data(), 64, vocab.data(), y.data(), 4096, LORA_BF16, nullptr),
         LORA_ERR_SHAPE);   // 8-slot pool, 64-slot routing
  lora_routing* r8 = nullptr;
  EXPECT(lora_routing_create(&r8, 0, 64, 8), LORA_OK);
  std::vector<int32_t> ids8(64, 3);
  EXPECT(lora_route_embedding(emb, r8, ids8.data(), 64, vocab.data(), y.data(), 4096, LORA_BF16, nullptr), LORA_OK);
  // a decode batch over few slots: the slot-major kernels (64 tokens, 8 slots)
  lora_pool* small = nullptr;
  EXPECT(lora_pool_create(&small, 0, 8, 16, 4096, slices_down, 1, LORA_BF16, 64), LORA_OK);
  for (int slot = 0; slot < 8; ++slot)
    EXPECT(lora_register_adapter(small, slot, a3, b3, 32.f, 16, 0, 1.f, 0u, nullptr), LORA_OK);
  EXPECT(lora_linear(small, r8, x.data(), 4096, y.data(), 4096, LORA_BF16, nullptr), LORA_OK);
  EXPECT(lora_route_linear(small, r8, ids8.data(), 64, x.data(), 4096, y.data(), 4096, LORA_BF16, nullptr), LORA_OK);
  EXPECT(lora_linear_noalloc(small, r8, x.data(), 4096, y.data(), 4096, LORA_BF16, nullptr), LORA_OK);
  EXPECT(lora_pool_destroy(small), LORA_OK);
  EXPECT(lora_embedding(emb, r8, vocab.data(), y.data(), 4096, LORA_BF16, nullptr), LORA_OK);
  EXPECT(lora_linear(emb, r8, x.data(), 32000, y.data(), 4096, LORA_BF16, nullptr), LORA_ERR_INVALID_ARG);

  // diagnostics
  EXPECT(lora_timing_enable(1), LORA_OK);
  EXPECT(lora_build_routing(r256, ids.data(), 128, nullptr), LORA_OK);
  EXPECT(lora_linear(qkv, r256, x.data(), 4096, y.data(), 6144, LORA_BF16, nullptr), LORA_OK);
  double ms[8];
  int launches[8];
  EXPECT(lora_timing_report(ms, launches, 8), LORA_OK);
  EXPECT(lora_timing_enable(0), LORA_OK);
  EXPECT(lora_bandwidth_probe(x.data(), 1 << 20, y.data(), 8 << 20, 0, nullptr), LORA_OK);
  EXPECT(lora_bandwidth_probe(x.data(), 1 << 20, y.data(), 1 << 10, 4, nullptr), LORA_ERR_SHAPE);

  for (lora_pool* p : {qkv, gu, down, f32, fp8, emb}) EXPECT(lora_pool_destroy(p), LORA_OK);
  for (lora_routing* r : {r256, r1024, r8}) EXPECT(lora_routing_destroy(r), LORA_OK);
  std::printf("host sanitizer run: %d launches asked for, %d failures\n", g_launches, g_fail);
  return g_fail ? 1 : 0;
}
