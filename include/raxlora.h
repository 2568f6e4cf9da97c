/*
 * raxlora.h - C ABI of the MI355X (gfx950) batched multi-adapter LoRA library.
 *
 * The library applies, for every token t with its own adapter slot i(t) in a
 * resident pool,
 *
 *     y[t] += s_i * B_i (A_i x[t])            (the base output W0 x[t] is the caller's)
 *
 * as a shrink (x -> rank space through lora_a = A) and an expand (rank space ->
 * output through lora_b = B), driven by per-batch routing metadata.
 *
 * Passages this interface follows (page title, then section):
 *   [llama.cpp] "llama.cpp 源码完全拆解(十六):LoRA 适配器——低秩补丁如何挂进 ggml 计算图"
 *   [TRT-LLM]   "TensorRT-LLM 源码完全拆解(二十一):LoRA 服务——adapter 池、批内多适配器与
 *               前向替换的完整链路"
 *   [vLLM-deep] "vLLM LoRA 实现深度解析"
 *   [vLLM-book] "第16章 LoRA 适配器热切换：一个引擎承载多个微调"
 *
 * Conventions for every call:
 *   - Matrices are row-major.  x is [T, k] with row stride ldx elements, y is
 *     [T, D] with D = sum of the slice widths and row stride ldy.  A adapter's
 *     A (shrink) is [rank, k] and its B (expand) is [d_n, rank] per output slice,
 *     as PEFT stores lora_a / lora_b ([vLLM-deep] §3.3).
 *   - "device pointer" means memory on the pool's GPU; "host pointer" ordinary
 *     process memory.  The library never takes ownership of caller memory.
 *   - Calls that take a hipStream_t only enqueue work on that stream (no host
 *     synchronisation) unless documented as synchronous.  The caller keeps its
 *     buffers alive until that work has completed.
 *   - Every call returns LORA_OK (0) or a negative lora_status; nothing throws
 *     across the ABI.  lora_last_error() gives a message for the calling thread.
 *     Argument checks run before any HIP call, so a rejected call has no effect.
 *   - Alignment: k and every slice width must be multiples of 8, ldx and ldy
 *     multiples of 8 elements, and x, y, u 16-byte aligned (the kernels move 16
 *     bytes per lane; [TRT-LLM] "前向替换" notes the grouped kernels assume K, N of
 *     at least 8).  Otherwise LORA_ERR_ALIGN.
 *   - Thread safety: distinct objects may be used from distinct threads.  One
 *     pool or routing object must not be mutated (register/unregister/build) while
 *     work that reads it may still run on another stream.  lora_linear and
 *     lora_shrink use a workspace owned by the pool, so two of them on one pool
 *     must not overlap in time (same stream is always safe).
 *   - Environment (read by the library; none is needed, all select among
 *     equivalent paths or launch shapes, and results stay within the tolerances
 *     the tests check):
 *       RAXLORA_MFMA_MIN_SEG  segments of at least this many tokens go to the
 *                             matrix cores (bf16 and FP8 pools; default 4; read when a
 *                             routing object is created)
 *       RAXLORA_DISABLE_MFMA  1: every segment on the vector units
 *       RAXLORA_CB1_MAX       matrix-core expand units take one 128-column block
 *                             instead of four when (column groups of four x tile
 *                             slots) is at most this (default 512)
 *       RAXLORA_XCD_GROUP     consecutive decode units kept on one XCD (default 4)
 *       RAXLORA_TILE_INTERLEAVE  matrix-core expand: 0 gives XCD x the x-th eighth
 *                             of the tile list, n > 0 deals runs of n tiles round
 *                             the XCDs (default: 1 when T < 64 S, else 0; the
 *                             results are the same either way)
 *       RAXLORA_GROUP_ORDER   0: grouped calls lay out their modules and decode units
 *                             in the order given (default 1: modules with the longest
 *                             shrink items first, decode expand units by descending
 *                             slot rank; results are the same either way)
 *       RAXLORA_LOG           1: one line on stderr per shrink or expand launch with
 *                             the launch shape chosen (path, k split, waves, units)
 *       RAXLORA_SLOT_MODE     0: never use the slot-major kernels (one unit per slot,
 *                             weight loads issued before the routing data arrives);
 *                             1: use them wherever the shape allows (T <= 256,
 *                             in_features <= 32768, bf16 or FP8 weights); default:
 *                             for 4 S <= T <= 128
 */
#ifndef RAXLORA_H
#define RAXLORA_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lora_pool lora_pool;
typedef struct lora_routing lora_routing;

/* LORA_FP8E4M3: adapter weights as OCP float8 e4m3 ("fn": 4 exponent bits, bias 7, 3
 * mantissa bits, largest finite 448), the native-FP8 adapter cache of [TRT-LLM]
 * (the FP8 special case of the weight preparation, and "前向替换").  A pool of this
 * weight type takes bf16 activations x, which the kernels clamp to [-448, 448]
 * and round to e4m3 before use, as the page converts the input; products are exact
 * and accumulate in fp32; y is bf16 or fp32.  The matrix-core shrink runs on the FP8
 * matrix cores (e4m3 x e4m3); the vector units and the expand widen the weights to
 * bf16 in registers (exact). */
typedef enum { LORA_F32 = 0, LORA_BF16 = 1, LORA_FP8E4M3 = 2 } lora_dtype;

typedef int lora_status;
#define LORA_OK                0
#define LORA_ERR_INVALID_ARG  (-1)   /* null handle or pointer, non-finite value, bad flag   */
#define LORA_ERR_SHAPE        (-2)   /* sizes or strides inconsistent                         */
#define LORA_ERR_DTYPE        (-3)   /* input dtype differs from the pool's                   */
#define LORA_ERR_RANK         (-4)   /* rank outside [1, max_lora_rank]                       */
#define LORA_ERR_SLOT         (-5)   /* slot outside [0, max_slots)                           */
#define LORA_ERR_CAPACITY     (-6)   /* more tokens than the object was created for           */
#define LORA_ERR_HIP          (-7)   /* a HIP runtime call failed                             */
#define LORA_ERR_OOM          (-8)   /* device allocation failed                              */
#define LORA_ERR_NO_DEVICE    (-9)   /* no usable GPU / device index out of range             */
#define LORA_ERR_ALIGN        (-10)  /* alignment rule above violated                         */
#define LORA_ERR_STATE        (-11)  /* object used out of order (e.g. routing never built)   */

/* register_adapter flags */
#define LORA_SRC_DEVICE   1u   /* A_slices / B_slices are device pointers (else host)          */
#define LORA_PREMULTIPLY  2u   /* fold the scale into B at registration                        */

/* Limits fixed at build time. */
#define LORA_MAX_SLICES    8
#define LORA_MAX_SLOTS     1024
#define LORA_MAX_RANK      256
#define LORA_MAX_IN_FEATURES 65536
#define LORA_MAX_GROUP     8      /* target modules of one grouped call */
#define LORA_NOALLOC_SCRATCH_BYTES (16u << 20)   /* scratch of lora_linear_noalloc, per GPU */

/* Message for the last failing call on this thread ("" if none). Never NULL. */
const char* lora_last_error(void);
/* Static name of a status code. */
const char* lora_status_string(lora_status status);

/*
 * Scale of the low-rank branch ([llama.cpp] "缩放系数到底乘在哪": adapter_scale *
 * alpha / rank, or adapter_scale alone when alpha is 0, i.e. absent; [TRT-LLM]
 * "LoraManager 的加载流水线" step 4 and [vLLM-deep] §1 "rsLoRA 变体": alpha/sqrt(rank)
 * when rslora is set).  Computed in double as adapter_scale*alpha, divided by rank
 * or sqrt(rank), and rounded once to float.  Pure host function, no device needed.
 * Errors: out_scale NULL -> INVALID_ARG; rank < 1 -> RANK; alpha or adapter_scale
 * not finite, or a non-finite result -> INVALID_ARG.
 */
lora_status lora_compute_scale(float alpha, int rank, int rslora, float adapter_scale,
                               float* out_scale);

/*
 * Create a pool of max_slots adapter slots for one target module (one linear
 * layer, or a packed group such as q/k/v or gate/up with num_slices output
 * slices of widths slice_out[0..num_slices)), like one layer's stacked LoRA
 * buffers ([vLLM-deep] §9: lora_a_stacked [max_loras, max_lora_rank, in],
 * lora_b_stacked [max_loras, out, max_lora_rank]).  max_lora_rank fixes the
 * padding of every slot ([TRT-LLM] "LoraConfig": a workspace bound, not
 * enlargeable later).  max_tokens bounds T for lora_linear / lora_shrink (it
 * sizes the pool-owned rank-space workspace: k-split partial sums, up to 16 x
 * num_slices x max_tokens x max_lora_rank fp32, and for pools of at most 32 slots
 * 16 more rows per slot, where a small decode batch's partial sums of each segment's
 * first 16 tokens go).  All slots start empty (rank 0).
 * slice_out is a host array, read during the call.  The pool owns its device
 * memory (allocated on `device` here) until lora_pool_destroy.
 * Errors: out/slice_out NULL -> INVALID_ARG; max_slots outside [1, LORA_MAX_SLOTS],
 * max_lora_rank outside [1, LORA_MAX_RANK], in_features < 1, num_slices outside
 * [1, LORA_MAX_SLICES], a slice width < 1, max_tokens < 1, in_features above
 * LORA_MAX_IN_FEATURES -> SHAPE; bad wdtype ->
 * DTYPE; in_features or a width not a multiple of 8 -> ALIGN; device missing ->
 * NO_DEVICE; allocation -> OOM.
 */
lora_status lora_pool_create(lora_pool** out, int device, int max_slots, int max_lora_rank,
                             int in_features, const int* slice_out, int num_slices,
                             lora_dtype wdtype, int max_tokens);

/*
 * A pool for the token embedding ([llama.cpp] "嵌入层:查表后再加增量": the lookup gets
 * a low-rank delta, get_rows of A by token id lifted by B; "token_embd" shape
 * contract: A is [r, V], B is [d, r]).  One slice of width d; vocab = V.  Adapters
 * are registered with lora_register_adapter as for other pools (A_slices[0] is
 * [rank, vocab], B_slices[0] is [d, rank]); the pool stores A transposed, one
 * contiguous row of max_lora_rank values per vocabulary id, so
 * lora_pool_read_slot returns A_host as [vocab, max_lora_rank].  Used only with
 * lora_embedding (and lora_expand); lora_shrink, lora_linear and lora_route_linear
 * reject it (INVALID_ARG).  Errors as lora_pool_create, except that vocab needs no
 * alignment and no upper bound (it is not a contraction length).
 */
lora_status lora_embedding_pool_create(lora_pool** out, int device, int max_slots, int max_lora_rank, int vocab,
                                       int d, lora_dtype wdtype, int max_tokens);

/* Free the pool.  All work that uses it must have completed.  NULL is a no-op. */
lora_status lora_pool_destroy(lora_pool* pool);

/*
 * Load an adapter into `slot` ([vLLM-deep] §5.3 set_lora(index, A, B): the
 * activation step writes the slot's buffers; [TRT-LLM] "AdapterSlotManager":
 * slots are fixed, their contents swapped).
 *   A_slices[n]: [rank, in_features] row-major, B_slices[n]: [slice_out[n], rank]
 *   row-major, both in the pool dtype.  A NULL pair marks a missing slice, which
 *   contributes nothing ([TRT-LLM] "LoraConfig": missing q/k/v padded with
 *   zeros); exactly one of the pair NULL is INVALID_ARG.
 *   Scale: see lora_compute_scale.  With LORA_PREMULTIPLY the pool stores
 *   round(s * B) (float32 product, one round to the pool dtype) and applies 1
 *   afterwards ([vLLM-deep] §1 "推理优化:预合并 scaling"); otherwise it stores B and
 *   multiplies the finished branch by s ([llama.cpp] "真正的核心").
 * With LORA_SRC_DEVICE the sources are device pointers and the copy is enqueued
 * on `stream`; otherwise they are host pointers and the call returns after the
 * copy has completed.  Re-registering a slot overwrites it in stream order.
 * Errors: pool NULL -> INVALID_ARG; slot -> SLOT; rank outside [1, max_lora_rank]
 * -> RANK; non-finite alpha / adapter_scale -> INVALID_ARG; unknown flag bit ->
 * INVALID_ARG; HIP failure -> HIP.
 */
lora_status lora_register_adapter(lora_pool* pool, int slot, const void* const* A_slices,
                                  const void* const* B_slices, float alpha, int rank, int rslora,
                                  float adapter_scale, unsigned flags, hipStream_t stream);

/* Empty `slot`: rank 0, so tokens still routed to it contribute nothing ([TRT-LLM]
 * "一次 decode 批次的路由": an empty slot has rank 0 and null pointers).  Enqueued on
 * `stream`.  Errors: pool NULL -> INVALID_ARG; slot -> SLOT. */
lora_status lora_unregister_adapter(lora_pool* pool, int slot, hipStream_t stream);

/* Host mirror of a slot's table entry (synchronous, no device access): rank,
 * scale still applied after the branch (1 when pre-multiplied), mask of present
 * slices, and the byte offsets of the slot's A and rank-major B blocks from the
 * pool base.  Any out pointer may be NULL. */
lora_status lora_pool_slot_info(const lora_pool* pool, int slot, int* rank, float* scale,
                                uint32_t* slice_mask, uint64_t* a_offset, uint64_t* bt_offset);

/* Copy a slot's stored slice back to host memory (synchronous; for tests):
 * A_host [max_lora_rank, in_features] (embedding pools: [vocab, max_lora_rank])
 * and Bt_host [max_lora_rank, slice_out[slice]]
 * (B transposed, rank-major), both in the pool dtype, rows >= rank zero.
 * Either pointer may be NULL. */
lora_status lora_pool_read_slot(const lora_pool* pool, int slot, int slice, void* A_host,
                                void* Bt_host);

/*
 * Routing metadata for one batch ([vLLM-book] §16.4.3 LoRAKernelMeta;
 * [TRT-LLM] "一次 decode 批次的路由": sorted_ids, per-slot counts and offsets in
 * fixed-address buffers).  The object owns fixed-address device buffers sized for
 * max_tokens tokens and max_slots slots, so the same addresses serve every batch.
 * Errors: out NULL -> INVALID_ARG; max_tokens < 1 or max_slots outside
 * [1, LORA_MAX_SLOTS] -> SHAPE; NO_DEVICE / OOM as for pools.
 */
lora_status lora_routing_create(lora_routing** out, int device, int max_tokens, int max_slots);
lora_status lora_routing_destroy(lora_routing* routing);

/*
 * Build the routing for T tokens from token_slot_ids[T] (device, int32): a slot
 * in [0, max_slots), or -1 for no LoRA.  Any other id is routed as -1 and
 * counted as invalid.  Key(t) = id, or S = max_slots for no LoRA (the sentinel
 * slot of [TRT-LLM] "AdapterSlotManager").  Produces, on the device:
 *   counts[S+1], seg_offsets[S+2] (exclusive prefix, [0] = 0, [S] = LoRA tokens,
 *   [S+1] = T), sorted_ids[T] (token indices grouped by key, ascending within a
 *   key), active slots (keys < S with tokens, ascending) and their number.
 * Enqueued on `stream`; T = 0 is allowed (ids may then be NULL).
 * Errors: routing NULL, or ids NULL with T > 0 -> INVALID_ARG; T < 0 -> SHAPE;
 * T > max_tokens -> CAPACITY.
 */
lora_status lora_build_routing(lora_routing* routing, const int32_t* token_slot_ids, int T,
                               hipStream_t stream);

/*
 * The same routing for num_seqs sequences of tokens_per_seq consecutive tokens each
 * ([TRT-LLM] "一次 decode 批次的路由": the linear-tree verification batch of speculative
 * decoding, where each sequence contributes its draft tokens plus one): seq_slot_ids
 * [num_seqs] (device, int32) holds one slot (or -1) per sequence; token t belongs to
 * sequence t / tokens_per_seq, so T = num_seqs * tokens_per_seq.  The outputs are
 * those of lora_build_routing on the per-token ids (each sequence's id repeated
 * tokens_per_seq times): the page's sequence-level sort expanded to tokens, sequence
 * q's tokens q p .. q p + p - 1 in order, counts p times the sequence counts; an
 * invalid sequence id counts its p tokens as invalid.  tokens_per_seq = 1 is
 * lora_build_routing.  Errors: NULL routing, or ids NULL with T > 0 -> INVALID_ARG;
 * num_seqs < 0 or tokens_per_seq < 1 -> SHAPE; T > max_tokens -> CAPACITY.
 */
lora_status lora_build_routing_seq(lora_routing* routing, const int32_t* seq_slot_ids, int num_seqs,
                                   int tokens_per_seq, hipStream_t stream);

/* Copy the last routing back to host memory (synchronous; for tests and
 * diagnostics).  counts[S+1], seg_offsets[S+2], sorted_ids[T], active_slots[S]
 * (entries past num_active unspecified); any pointer may be NULL.
 * Errors: STATE if the routing was never built. */
lora_status lora_routing_query(const lora_routing* routing, int32_t* counts, int32_t* seg_offsets,
                               int32_t* sorted_ids, int32_t* active_slots, int* num_active,
                               int* n_invalid);

/*
 * Shrink ([vLLM-book] §16.4.2 lora_shrink on lora_a; [vLLM-deep] §6):
 *   u[n][t][j] = sum_c A_slot(t)[n][j][c] * x[t][c]      (fp32 accumulate)
 * x: device [T, in_features] in the pool dtype (else DTYPE, [TRT-LLM] "三种输入
 * dtype": input and cache dtype must match).  u: device fp32 [num_slices, T,
 * max_lora_rank], caller-owned; written for LoRA tokens of non-empty slots and
 * j < rank (zero for a missing slice); other entries are left as they were.
 * Errors: INVALID_ARG (NULL), STATE (routing not built), SHAPE (ldx < in_features,
 * routing S != pool S), CAPACITY (T > pool max_tokens), ALIGN.
 */
lora_status lora_shrink(const lora_pool* pool, const lora_routing* routing, const void* x,
                        int ldx, float* u, hipStream_t stream);

/*
 * Expand and add ([vLLM-book] §16.4.2 lora_expand on lora_b; [TRT-LLM] "前向替换":
 * the correction is added in place onto the base output):
 *   y[t][o_n + i] = round_y( y[t][o_n + i] + s * sum_j B_slot(t)[n][i][j] * u[n][t][j] )
 * with fp32 arithmetic and one rounding to ydtype.  u as written by lora_shrink.
 * y: device [T, D], in/out, ydtype = the pool dtype or LORA_F32.  Rows of no-LoRA
 * tokens, of empty or zero-scale slots, and columns of missing slices are not
 * written.  Errors as lora_shrink, plus DTYPE for an unsupported ydtype.
 */
lora_status lora_expand(const lora_pool* pool, const lora_routing* routing, const float* u,
                        void* y, int ldy, lora_dtype ydtype, hipStream_t stream);

/*
 * Fused shrink + expand onto the caller's base output ([TRT-LLM] "前向替换":
 * forward_with_base adds the LoRA result onto the base projection; [vLLM-book]
 * §16.4.4 add_lora_linear).  Same result as lora_shrink then lora_expand, with the
 * intermediate kept in the pool's workspace as k-split partial sums, added in
 * split order by the expand, so repeated calls are bitwise identical (and equal
 * to lora_shrink then lora_expand).  Long same-slot segments of bf16 and FP8 pools go to
 * the matrix cores (MFMA).  Two kernel launches per call.
 * Errors as lora_expand.
 */
lora_status lora_linear(const lora_pool* pool, const lora_routing* routing, const void* x, int ldx,
                        void* y, int ldy, lora_dtype ydtype, hipStream_t stream);

/*
 * Routing and fused shrink + expand of one batch: lora_build_routing(routing,
 * token_slot_ids, T) followed by lora_linear(pool, routing, x, y), with the same
 * results (routing outputs and y bitwise identical).  For 1 <= T <= 256 tokens and
 * pools of at most 255 slots the routing is built inside the shrink launch, whose
 * units find their segments from token_slot_ids directly ([vLLM-book] §16.4.2: the
 * per-batch metadata that groups tokens by slot; [TRT-LLM] "一次 decode 批次的路由"), so
 * the call costs two launches instead of three; larger batches take the two calls.
 * The routing object then holds this batch's routing for further lora_linear calls
 * (other target modules of the same tokens).  token_slot_ids must stay unchanged
 * until the call's work has run.  Arguments and errors as lora_build_routing and
 * lora_linear (routing and pool must have the same slot count).
 */
lora_status lora_route_linear(const lora_pool* pool, lora_routing* routing, const int32_t* token_slot_ids,
                              int T, const void* x, int ldx, void* y, int ldy, lora_dtype ydtype,
                              hipStream_t stream);

/*
 * lora_linear / lora_route_linear joined to a base projection that another stream
 * is still computing ([llama.cpp] "为什么低秩增量可以「后加」" and [TRT-LLM] "前向替换": the
 * LoRA branch and the base output are independent until the final add).  The
 * routing and the shrink (which read only ids and x) are enqueued on `stream`
 * at once; then `stream` waits for y_ready (hipStreamWaitEvent), recorded by the
 * caller after the work that writes the base output into y; then the expand adds
 * onto y.  y_ready NULL: exactly lora_linear / lora_route_linear.  Results are
 * bitwise those of the base work followed by the plain call.  Arguments and errors
 * as lora_linear / lora_route_linear, plus HIP if the wait cannot be enqueued.
 */
lora_status lora_linear_join(const lora_pool* pool, const lora_routing* routing, const void* x, int ldx,
                             void* y, int ldy, lora_dtype ydtype, hipStream_t stream, hipEvent_t y_ready);
lora_status lora_route_linear_join(const lora_pool* pool, lora_routing* routing, const int32_t* token_slot_ids,
                                   int T, const void* x, int ldx, void* y, int ldy, lora_dtype ydtype,
                                   hipStream_t stream, hipEvent_t y_ready);

/*
 * lora_linear for callers that cannot allocate device memory at call time (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same shrink and expand launches with the same results bitwise, but the k-split
 * partial sums live in a fixed scratch array of LORA_NOALLOC_SCRATCH_BYTES inside the
 * library's device image instead of the pool's workspace.  The call allocates and
 * frees nothing (the array's device address is looked up once per GPU, on the first
 * call there).  The caller still passes x and y as for lora_linear.
 * Every call on one GPU shares that GPU's array and leaves its last contents there;
 * nothing in it needs to start at zero.  Calls that overlap in time on one GPU (other
 * streams, other threads) race on it: serialise them, e.g. on one stream.
 * Needs nsplit * num_slices * T * Rk * 4 bytes, where Rk is max_lora_rank rounded up
 * to 32 and nsplit at most 16 (in_features / 512 rounded up, halved for batches of at
 * least 64 tokens per slot); above the maximum the call fails with CAPACITY before any
 * work is enqueued (when 16 rows per slot more fit as well, a small decode batch uses
 * them as the pool's workspace would).  Arguments and other errors as lora_linear.
 */
lora_status lora_linear_noalloc(const lora_pool* pool, const lora_routing* routing, const void* x, int ldx, void* y,
                                int ldy, lora_dtype ydtype, hipStream_t stream);

/*
 * Several target modules of one batch in one shrink and one expand launch: for each
 * m < num_pools, lora_linear(pools[m], routing, x[m], ldx[m], y[m], ldy[m], ydtype),
 * with the same results bitwise (every module's units compute what its own call
 * computes).  This is the grouped form of the pages' layer step: [TRT-LLM] "前向替换:
 * LoraLayer 的三条路径" sizes one intermediate buffer [num_layer_modules, batch_size,
 * max_rank] and runs one grouped product over every (module, slot) problem of the
 * layer; [vLLM-book] §16.4.4 add_shrink / add_expand take several slices in one call.
 * A layer's q/k/v/o/gate/up/down modules then cost two launches instead of two each
 * ([llama.cpp] "性能与工程取舍": in decode the extra cost of LoRA is mostly launches).
 *   pools[m]: distinct linear pools with the routing's slot count, all of one weight
 *   dtype and of max_lora_rank padding to one multiple of 32; each keeps its own
 *   workspace, so no pool may appear twice.  x[m] is [T, in_features of pools[m]]
 *   with row stride ldx[m]; y[m] is [T, D of pools[m]] with row stride ldy[m]; the y
 *   of different modules must not share elements (they may be column ranges of one
 *   buffer).  Host arrays pools, x, ldx, y, ldy are read during the call.
 * Errors: INVALID_ARG (NULL array or entry, a repeated pool, an embedding pool),
 * SHAPE (num_pools outside [1, LORA_MAX_GROUP], slot count or rank padding differing),
 * DTYPE (weight dtypes differing, or as lora_linear), plus those of lora_linear for
 * each module.
 */
lora_status lora_linear_group(const lora_pool* const* pools, int num_pools, const lora_routing* routing,
                              const void* const* x, const int* ldx, void* const* y, const int* ldy, lora_dtype ydtype,
                              hipStream_t stream);

/*
 * lora_build_routing(routing, token_slot_ids, T) followed by lora_linear_group: for
 * 1 <= T <= 256 tokens and at most 255 slots the routing is built inside the grouped
 * shrink launch (two launches for the whole layer step); larger batches take the
 * routing launch first.  Routing outputs and y bitwise those of the separate calls.
 * Arguments and errors as lora_build_routing and lora_linear_group.
 */
lora_status lora_route_linear_group(const lora_pool* const* pools, int num_pools, lora_routing* routing,
                                    const int32_t* token_slot_ids, int T, const void* const* x, const int* ldx,
                                    void* const* y, const int* ldy, lora_dtype ydtype, hipStream_t stream);

/*
 * Embedding LoRA onto the caller's lookup result ([llama.cpp] "嵌入层:查表后再加增量"):
 *   y[t][i] = round_y( y[t][i] + s * sum_j B_slot(t)[i][j] * A_slot(t)[j][vocab_ids[t]] )
 * for LoRA tokens of the routing (built from the tokens' slot ids as usual).
 * vocab_ids: device int32 [T], the tokens' vocabulary ids; an id outside
 * [0, vocab) contributes zero (its row is rewritten as y + 0).  Two launches: a
 * gather of each token's row of A into the pool's workspace, then the expand of
 * lora_linear.  y as for lora_expand; the pool must come from
 * lora_embedding_pool_create (else INVALID_ARG).  Errors as lora_expand, plus
 * INVALID_ARG for vocab_ids NULL with T > 0.
 */
lora_status lora_embedding(const lora_pool* pool, const lora_routing* routing, const int32_t* vocab_ids, void* y,
                           int ldy, lora_dtype ydtype, hipStream_t stream);

/*
 * lora_build_routing(routing, slot_ids, T) followed by lora_embedding(pool,
 * routing, vocab_ids, y), with the same results (routing outputs and y bitwise
 * identical): the gather reads the tokens' slot ids directly and writes each
 * token's rank row by token index, and for T <= 256 tokens and pools of at most
 * 255 slots the routing is built inside the gather launch (two launches instead of
 * three).  slot_ids, vocab_ids: device int32 [T].  Errors as lora_build_routing and
 * lora_embedding.
 */
lora_status lora_route_embedding(const lora_pool* pool, lora_routing* routing, const int32_t* slot_ids, int T,
                                 const int32_t* vocab_ids, void* y, int ldy, lora_dtype ydtype, hipStream_t stream);

/*
 * Index checks (diagnostics): a library built with -DRAXLORA_DEBUG (build.py
 * --debug: libraxlora_debug.so) checks, in its kernels, every index it takes from
 * memory (token ids, slots, sorted positions, workspace rows) against its range; a
 * failed check is counted and the access goes to index 0 instead, so a wrong index
 * shows as a count rather than a fault.  *enabled = 1 in such a build, 0 otherwise
 * (where *faults is always 0); *faults = the checks failed on the current device since
 * the last reset (all kernels of the library, after the work enqueued so far has
 * finished: the call synchronises the device); reset != 0 clears the count.
 * Errors: NULL -> INVALID_ARG; a HIP error reading the counts -> HIP.
 */
lora_status lora_index_checks(int* enabled, unsigned long long* faults, int reset);

/*
 * Bandwidth probe (diagnostics): the rate this GPU's memory gives a plain streaming
 * kernel, the ceiling against which the LoRA kernels' traffic is read.  ratio <= 0:
 * read read_bytes from src (device, 16-byte aligned), 16 bytes per lane, and write
 * one 4-byte word per thread into dst (needs dst_bytes >= 4 MiB).  ratio > 0: read
 * read_bytes and write read_bytes / ratio bytes to dst (each 16-byte chunk of dst is
 * the xor of `ratio` chunks of src).  One launch, enqueued on `stream`.
 * Errors: NULL -> INVALID_ARG; alignment -> ALIGN; sizes -> SHAPE.
 */
lora_status lora_bandwidth_probe(const void* src, uint64_t read_bytes, void* dst, uint64_t dst_bytes, int ratio,
                                 hipStream_t stream);

/*
 * Kernel timing (diagnostics).  While enabled (process-wide), every kernel that
 * the routing, shrink, expand, linear and embedding calls launch is started
 * with hipExtLaunchKernel and a pair of events stamped at that kernel's own start
 * and end, on the stream it runs on.  lora_timing_report waits for the recorded
 * events, writes per kernel id (0 routing, 1 shrink, 2 expand, 3 finish_u: the
 * pass of lora_shrink that adds the k-split partial sums into the caller's u,
 * 4 gather: the embedding rows of lora_embedding; the shrink and expand launches
 * cover both short and long segments) the summed milliseconds and the
 * number of launches into total_ms[0..max_kernels) and launches[0..max_kernels), and
 * clears the record.  lora_timing_kernel_name gives the name of an id ("" if none).
 * Errors: INVALID_ARG for NULL arrays with max_kernels > 0; HIP if an event fails.
 */
lora_status lora_timing_enable(int on);
lora_status lora_timing_report(double* total_ms, int* launches, int max_kernels);
const char* lora_timing_kernel_name(int kernel);

#ifdef __cplusplus
}
#endif

#endif /* RAXLORA_H */
