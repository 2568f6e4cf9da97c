// Expand launches: shape checks, the workgroup layout and the dispatch to the
// translation unit of the weight and output types.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_util.h"
#include "decode_units.h"
#include "launch_util.h"
#include "mfma_tiles.h"

namespace rax {

// launches of one (weight, output) type pair of the expand kernels, one translation
// unit each: w16 = bf16 weights, w8 = FP8, w32 = fp32; y16 = bf16 output, y32 = fp32
#define RAX_EXPAND_PAIR_DECL(NAME)                                                                       \
  void expand_launch_##NAME(int ksm, dim3 grid, uint32_t lds, hipStream_t stream, const PoolView& P,       \
                            const SlotOrder& O, const RouteView& R, const UView& U, void* y, int ldy,      \
                            const Plan& plan, int nm, const KTimer& tm);                                \
  void expand_group_launch_##NAME(int ksm, dim3 grid, uint32_t lds, hipStream_t stream, const GroupView& G, \
                                  const RouteView& R, const KTimer& tm);
RAX_EXPAND_PAIR_DECL(w16_y16)
RAX_EXPAND_PAIR_DECL(w16_y32)
RAX_EXPAND_PAIR_DECL(w8_y16)
RAX_EXPAND_PAIR_DECL(w8_y32)
RAX_EXPAND_PAIR_DECL(w32_y32)

size_t expand_smem_bytes(int wdtype, int Rmax, int use_mfma) {
  size_t f = (size_t)expand_usm_floats(Rmax);
  if (use_mfma && wdtype != LORA_F32 && (size_t)kExpandMfmaWaveFloats > f) f = kExpandMfmaWaveFloats;
  return f * sizeof(float);
}

// rank steps of 32 the matrix-core part keeps in registers: Rk / 32 rounded up to a power of 2
static int expand_ksm(const PoolView& P) { return P.Rk <= 32 ? 1 : P.Rk <= 64 ? 2 : P.Rk <= 128 ? 4 : 8; }

static bool expand_shape_ok(int wdtype, const PoolView& P, const UView& U, const Plan& plan) {
  if (plan.slot_mode)
    return !(wdtype == LORA_F32 || !plan.use_mfma || plan.n_dec_blocks != 0 || plan.n_mgroups < 1 || U.nsplit < 1 ||
             U.nsplit > kMaxSplit || (U.by_token && U.nsplit != 1) ||
             (!U.by_token && (U.row_stride % 4 != 0 || U.row_stride < P.Rk)) ||
             (plan.cb != 1 && plan.cb != kMfmaColBlocksPerUnit));
  return !(plan.xcd_group < 1 || plan.ntg < 1 || U.nsplit < 1 || U.nsplit > kMaxSplit ||
           (U.by_token && U.nsplit != 1) || (!U.by_token && (U.row_stride % 4 != 0 || U.row_stride < P.Rk)) ||
           plan.n_dec_blocks != P.n_ctiles * P.S * plan.ntg ||
           (plan.use_mfma && (wdtype == LORA_F32 || plan.tile_slots < 1 || plan.n_mgroups < 1 ||
                              (plan.cb != 1 && plan.cb != kMfmaColBlocksPerUnit))));
}

int expand_blocks(int wdtype, const PoolView& P, const Plan& plan, int& n_mfma_blocks) {
  (void)wdtype;
  if (plan.slot_mode) {   // slot-major units only (XCD-aligned slot groups)
    n_mfma_blocks = (P.S + kXcds - 1) / kXcds * kXcds * plan.n_mgroups;
    return n_mfma_blocks;
  }
  n_mfma_blocks = plan.use_mfma ? mfma_blocks(plan.n_mgroups * plan.tile_slots) : 0;
  const int q = kXcds * plan.xcd_group;
  return n_mfma_blocks + (plan.n_dec_blocks + q - 1) / q * q;
}

hipError_t launch_expand(int wdtype, int ydtype, const PoolView& P, const SlotOrder& O, const RouteView& R,
                         const UView& U, void* y, int ldy, const Plan& plan, hipStream_t stream,
                         const KTimer& tm) {
  if (!expand_shape_ok(wdtype, P, U, plan)) return hipErrorInvalidValue;
  int nm;
  const dim3 grid(expand_blocks(wdtype, P, plan, nm));
  const uint32_t lds = (uint32_t)expand_smem_bytes(wdtype, P.Rmax, plan.use_mfma);
  const int ksm = expand_ksm(P);
  const bool y16 = ydtype == LORA_BF16;
  if (wdtype == LORA_BF16)
    (y16 ? expand_launch_w16_y16 : expand_launch_w16_y32)(ksm, grid, lds, stream, P, O, R, U, y, ldy, plan, nm, tm);
  else if (wdtype == LORA_FP8E4M3)
    (y16 ? expand_launch_w8_y16 : expand_launch_w8_y32)(ksm, grid, lds, stream, P, O, R, U, y, ldy, plan, nm, tm);
  else   // fp32 pools: decode units only, one body
    expand_launch_w32_y32(1, grid, lds, stream, P, O, R, U, y, ldy, plan, nm, tm);
  return hipGetLastError();
}

hipError_t launch_expand_group(int wdtype, int ydtype, const GroupView& G0, const RouteView& R, hipStream_t stream,
                               const KTimer& tm) {
  GroupView G = G0;
  int blocks;
  if (!group_layout(wdtype, G, R, nullptr, true, blocks)) return hipErrorInvalidValue;
  size_t lds = 0;
  for (int m = 0; m < G.n; ++m) {
    if (!expand_shape_ok(wdtype, G.e[m].P, G.e[m].U, G.e[m].plan) || expand_ksm(G.e[m].P) != expand_ksm(G.e[0].P) ||
        G.e[m].plan.slot_mode != G.e[0].plan.slot_mode)
      return hipErrorInvalidValue;
    lds = std::max(lds, expand_smem_bytes(wdtype, G.e[m].P.Rmax, G.e[m].plan.use_mfma));
  }
  const int ksm = expand_ksm(G.e[0].P);
  const dim3 grid(blocks);
  const bool y16 = ydtype == LORA_BF16;
  if (wdtype == LORA_BF16)
    (y16 ? expand_group_launch_w16_y16 : expand_group_launch_w16_y32)(ksm, grid, (uint32_t)lds, stream, G, R, tm);
  else if (wdtype == LORA_FP8E4M3)
    (y16 ? expand_group_launch_w8_y16 : expand_group_launch_w8_y32)(ksm, grid, (uint32_t)lds, stream, G, R, tm);
  else
    expand_group_launch_w32_y32(1, grid, (uint32_t)lds, stream, G, R, tm);
  return hipGetLastError();
}

}  // namespace rax
