"""CPU oracle for batched multi-adapter LoRA application.

TEST INFRASTRUCTURE ONLY.  This package is imported, called or executed only by
``tests/``, by ``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of
``bench.py``.  The product path (``rank_adapter_gemm_build_amd``) never touches it,
and it shares no code, table or helper with the HIP library.

It is deliberately plain and slow: numpy float64, one Python loop over tokens
where the pages define the operation per token, a library matmul only where the
pages' own description is a matmul.  Every function names the passage it follows.

Pages cited (title, then the section used):
  [llama.cpp]  "llama.cpp 源码完全拆解(十六):LoRA 适配器——低秩补丁如何挂进 ggml 计算图"
  [TRT-LLM]    "TensorRT-LLM 源码完全拆解(二十一):LoRA 服务——adapter 池、批内多适配器与
                前向替换的完整链路"
  [vLLM-deep]  "vLLM LoRA 实现深度解析"
  [vLLM-book]  "第16章 LoRA 适配器热切换：一个引擎承载多个微调"

Operator (all pages agree up to notation): for a token x in R^k routed to an
adapter with A in R^{r x k} (shrink, ``lora_a``) and B in R^{d x r} (expand,
``lora_b``), the output is  h = W0 x + s * B (A x).  Row-major batch form with
x stored [T, k] and W0 stored [d, k]:  Y = X W0^T + s (X A^T) B^T.

Readings taken where the pages are silent (each is also listed in the design
notes of the repository):
  * u = A x is kept in float64 here; the GPU keeps it in fp32 and never rounds it
    to bf16.
  * "alpha missing" is alpha == 0.
  * rsLoRA combines multiplicatively with the runtime adapter_scale.
  * the no-LoRA group (slot id -1, or any id outside [0, S)) sorts LAST, under
    the sentinel key S.
  * a slot with rank 0 or scale 0 contributes nothing and leaves its rows
    bit-untouched, as does a slice registered as missing.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
against something other than itself (hand-derived fixtures in ``tests/golden``,
closed forms, invariants, brute force on tiny inputs, a library implementation of
a number format), and planted mistakes are checked to fail those pins:
  lora_scale            scale_cases.json (the printed values), rank/alpha mutants
  f32_to_bf16_bits      hand values with ties, torch's bfloat16 conversion
  bf16_bits_to_f64      exact decode of every pattern class
  round_to_dtype        through the integer and linearity pins (f32 / bf16 paths)
  fp8_e4m3_decode       torch's float8_e4m3fn on all 256 bytes
  fp8_e4m3_encode       torch's conversion on every value, every tie, random values
  fp8_quantize          clamp cases, and fp8_case.json (conversion mutants fail it)
  fp8_fold_scale        the page's fold expression evaluated by torch
  effective_b           integer_case.json with and without premultiply, scale mutants
  route_by_sort,        routing_cases.json, invariants, brute force over every ids
  route_by_counting     vector of up to 6 tokens for S <= 3, unstable-sort mutant
  route_tokens_per_seq  routing_seq_cases.json, brute force against a token-level sort
  shrink_per_token,     integer_case.json (u and y), identity and single-entry
  expand_per_token,     closed forms, zero branches, packed = separate slices,
  lora_apply            rank padding, transposed-operand mutants
  lora_apply_fp8        fp8_case.json: activations past +-448, ties, subnormals,
                        integer e4m3 weights, an off-grid base (mutants: no
                        conversion, clamp only, no clamp, truncation, converted
                        base, dropped scale)
  lora_apply_grouped    equal to lora_apply within 1e-12, and integer_case.json
  merged_apply          equal to lora_apply within 1e-10 (linearity)
  embedding_apply       embedding_case.json, equality with lora_apply on one-hot rows
  extra_macs_per_token, the page's printed ratios and sizes (page_numbers.json)
  adapter_params
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

__all__ = [
    "lora_scale",
    "f32_to_bf16_bits",
    "bf16_bits_to_f64",
    "round_to_dtype",
    "effective_b",
    "Adapter",
    "Routing",
    "route_by_sort",
    "route_by_counting",
    "shrink_per_token",
    "expand_per_token",
    "lora_apply",
    "lora_apply_grouped",
    "merged_apply",
    "extra_macs_per_token",
    "adapter_params",
]


# --------------------------------------------------------------------------- scale
def lora_scale(alpha: float, rank: int, rslora: bool, adapter_scale: float = 1.0) -> np.float32:
    """Scale s applied to the low-rank branch.

    [llama.cpp] section "缩放系数到底乘在哪": the scale is adapter_scale*alpha/rank when
    alpha is present, and plain adapter_scale when the file carries no alpha (the
    loader then reads 0).  The rank is the adapter's own rank.
    [TRT-LLM] "从检查点到 GPU:LoraManager 的加载流水线", step 4, and [vLLM-deep] §1
    "rsLoRA 变体": with use_rslora the denominator is sqrt(r) instead of r.

    Evaluated in float64 left to right (adapter_scale * alpha, then divided by r or
    by sqrt(r)) and rounded once to float32.
    """
    if int(rank) != rank or rank < 1:
        raise ValueError("rank must be a positive integer")
    a = float(np.float32(alpha))
    c = float(np.float32(adapter_scale))
    if a == 0.0:
        sigma = c
    elif rslora:
        sigma = c * a / math.sqrt(float(rank))
    else:
        sigma = c * a / float(rank)
    return np.float32(sigma)


# ---------------------------------------------------------------- number formats
def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    bfloat16 keeps the upper 16 bits of a float32.  Written from the definition:
    add 0x7FFF plus the lowest kept bit, then truncate.  NaNs stay NaN (quiet bit
    forced).  Returns uint16 bit patterns.
    """
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    is_nan = np.isnan(f)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    r = np.where(is_nan, ((u >> 16) | 0x40) & 0xFFFF, r)
    return r.astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact float64 value of bfloat16 bit patterns (the bits are the top half of a float32)."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_to_dtype(a, dtype: str) -> np.ndarray:
    """Round float64 values to the storage format, returned as float64.

    'f32': one IEEE round-to-nearest-even to float32.  'bf16': to float32 first,
    then to bfloat16 with ties to even (the GPU produces fp32 results and rounds
    those once to bf16).
    """
    a = np.asarray(a, dtype=np.float64)
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(f32_to_bf16_bits(a.astype(np.float32)))
    raise ValueError(dtype)


# ------------------------------------------------------------------ FP8 (e4m3)
# [TRT-LLM] "LoraConfig"/FP8 special case (the fifth step of the weight preparation)
# and "前向替换" (the input conversion and the output restore): with a native-FP8
# adapter cache the adapter stays FP8; the scale is applied in BF16 and the result
# clamped back into the FP8 range; the BF16 activations are clamped to the FP8 range
# and converted; the correction is added to the BF16 base output.  The format is
# OCP float8 e4m3 ("fn": 1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
# exponent field 0 subnormal, S.1111.111 NaN, no infinities, largest finite 448).
FP8_MAX = 448.0


def fp8_e4m3_decode(bits) -> np.ndarray:
    """Exact float64 value of e4m3 bit patterns (NaN for S.1111.111)."""
    b = np.asarray(bits, dtype=np.int64) & 0xFF
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = s * mag
    return np.where((e == 15) & (m == 7), np.nan, out)


def fp8_e4m3_encode(x) -> np.ndarray:
    """Round values with |x| <= 448 to e4m3 bit patterns, to nearest, ties to even."""
    x = np.asarray(x, dtype=np.float64)
    assert np.all(np.abs(x) <= FP8_MAX), "clamp to the FP8 range first"
    out = np.zeros(x.shape, dtype=np.int64)
    for idx, v in np.ndenumerate(x):
        sign = 0x80 if np.signbit(v) else 0
        a = abs(float(v))
        if a < 2.0 ** -6:                          # subnormal range: steps of 2^-9
            q = int(np.rint(a * 512.0))            # rint: ties to even
            e, m = (1, 0) if q == 8 else (0, q)
        else:
            f, E = np.frexp(a)                     # a = f 2^E, f in [0.5, 1)
            eu = E - 1
            q = int(np.rint((a / 2.0 ** eu - 1.0) * 8.0))
            if q == 8:
                eu, q = eu + 1, 0
            e, m = eu + 7, q
        out[idx] = sign | (e << 3) | m
    return out


def fp8_quantize(x) -> np.ndarray:
    """The forward input conversion: clamp to [-448, 448], then round to e4m3
    ([TRT-LLM] "前向替换": x.clamp(-fp8_max, fp8_max).to(float8_e4m3fn)).  float64 out."""
    return fp8_e4m3_decode(fp8_e4m3_encode(np.clip(np.asarray(x, dtype=np.float64), -FP8_MAX, FP8_MAX)))


def fp8_fold_scale(b_fp8_values, scale) -> np.ndarray:
    """The FP8 scale fold at weight preparation: the FP8 weights go to BF16, are
    multiplied by the scale (a float32 product rounded once to BF16), clamped to the
    FP8 range and rounded back to e4m3.  Returns the new e4m3 values as float64."""
    prod32 = np.asarray(b_fp8_values, dtype=np.float32) * np.float32(scale)
    p = bf16_bits_to_f64(f32_to_bf16_bits(prod32))
    return fp8_e4m3_decode(fp8_e4m3_encode(np.clip(p, -FP8_MAX, FP8_MAX)))


# ------------------------------------------------------------------ adapter pool
@dataclass
class Adapter:
    """One adapter resident in one slot of one target module.

    A[n] is [rank, k] and B[n] is [d_n, rank] per output slice n, as stored by PEFT
    ([vLLM-deep] §3.3 LoRALayerWeights: lora_a (r, k), lora_b (d, r)); None marks a
    missing slice, which contributes nothing ([TRT-LLM] "LoraConfig:哪些矩阵可以被
    替换": missing q/k/v modules are padded with zeros).  Values are the exact stored
    numbers as float64.  One rank for every slice of the slot ([TRT-LLM] "一次 decode
    批次的路由": all modules of a slot share one rank).
    """

    rank: int
    A: List[Optional[np.ndarray]]
    B: List[Optional[np.ndarray]]
    alpha: float
    rslora: bool = False
    adapter_scale: float = 1.0
    premultiply: bool = False

    def scale(self) -> np.float32:
        return lora_scale(self.alpha, self.rank, self.rslora, self.adapter_scale)


def effective_b(adapter: Adapter, n: int, wdtype: str):
    """The B the expand multiplies, and the scale still applied after the branch.

    Without pre-multiplication: (B, s) - the scale multiplies the finished branch
    output ([llama.cpp] "真正的核心:建图时如何把低秩分支拼进去": ggml_scale on B(Ax)).
    With it: ([vLLM-deep] §1 "推理优化:预合并 scaling", LoRALayerWeights.optimize():
    lora_b *= scaling, then scaling = 1) the product s*B is formed once in float32 and
    stored back in the pool format, and the remaining scale is 1.
    """
    B = adapter.B[n]
    s = adapter.scale()
    if B is None:
        return None, float(s)
    if not adapter.premultiply:
        return np.asarray(B, dtype=np.float64), float(s)
    if wdtype == "fp8":   # folded in BF16 and clamped back into FP8 (fp8_fold_scale)
        return fp8_fold_scale(np.asarray(B, dtype=np.float64), s), 1.0
    prod32 = np.float32(s) * np.asarray(B, dtype=np.float32)  # one fp32 rounding
    return round_to_dtype(prod32.astype(np.float64), wdtype), 1.0


# ---------------------------------------------------------------------- routing
@dataclass
class Routing:
    keys: np.ndarray          # [T]   slot id, or S for "no LoRA"
    counts: np.ndarray        # [S+1] tokens per key
    seg_offsets: np.ndarray   # [S+2] exclusive prefix of counts; [0]=0, [S]=#LoRA tokens, [S+1]=T
    sorted_ids: np.ndarray    # [T]   token indices, grouped by key, ascending within a key
    active_slots: np.ndarray  # [num_active] keys < S with count > 0, ascending
    num_active: int
    n_invalid: int            # ids outside {-1} U [0, S)
    extra: Dict[str, object] = field(default_factory=dict)


def _keys(ids: Sequence[int], S: int):
    """Key of each token.

    [vLLM-book] §16.4.2: token_lora_mapping holds the slot index, -1 meaning no
    LoRA.  [TRT-LLM] "adapter 池:AdapterSlotManager 与两级缓存": requests without an
    adapter are mapped to the sentinel max_num_adapters, whose rank is 0.  Ids that
    are neither -1 nor a valid slot are treated as no-LoRA and counted.
    """
    ids = np.asarray(ids, dtype=np.int64)
    valid = (ids >= 0) & (ids < S)
    keys = np.where(valid, ids, S).astype(np.int64)
    n_invalid = int(np.count_nonzero(~valid & (ids != -1)))
    return keys, n_invalid


def _finish(keys, sorted_ids, counts, S, n_invalid) -> Routing:
    T = len(keys)
    offs = np.zeros(S + 2, dtype=np.int64)
    for k in range(S + 1):  # [vLLM-book] §16.4.3: lora_token_start_loc, length max_loras+2, first 0
        offs[k + 1] = offs[k] + counts[k]
    assert offs[S + 1] == T
    active = np.array([k for k in range(S) if counts[k] > 0], dtype=np.int64)
    return Routing(keys=keys, counts=np.asarray(counts, dtype=np.int64), seg_offsets=offs,
                   sorted_ids=np.asarray(sorted_ids, dtype=np.int64), active_slots=active,
                   num_active=len(active), n_invalid=n_invalid)


def route_by_sort(ids: Sequence[int], S: int) -> Routing:
    """Routing metadata, formulation (i): a stable sort of token indices by key.

    [vLLM-book] §16.4.2-§16.4.3: sort the tokens by slot, count the tokens of each
    slot, take the start offset of each segment; the five index tensors of
    LoRAKernelMeta.  Ties keep token order (a stable sort).
    """
    keys, n_invalid = _keys(ids, S)
    T = len(keys)
    order = sorted(range(T), key=lambda t: (int(keys[t]), t))
    counts = [int(np.count_nonzero(keys == k)) for k in range(S + 1)]
    return _finish(keys, order, counts, S, n_invalid)


def route_by_counting(ids: Sequence[int], S: int) -> Routing:
    """Routing metadata, formulation (ii): an explicit counting sort.

    [TRT-LLM] "一次 decode 批次的路由:从请求到 slot_ids", step 4: per-slot counts by
    bincount with a minimum length, then a cumulative sum gives each slot's first
    row; the offsets array is one longer than the counts.  Tokens are then placed
    in increasing token order at their key's running cursor.
    """
    keys, n_invalid = _keys(ids, S)
    T = len(keys)
    counts = [0] * (S + 1)
    for t in range(T):
        counts[int(keys[t])] += 1
    cursor = [0] * (S + 1)
    run = 0
    for k in range(S + 1):
        cursor[k] = run
        run += counts[k]
    sorted_ids = [0] * T
    for t in range(T):
        k = int(keys[t])
        sorted_ids[cursor[k]] = t
        cursor[k] += 1
    return _finish(keys, sorted_ids, counts, S, n_invalid)


def route_tokens_per_seq(seq_ids: Sequence[int], S: int, tokens_per_seq: int) -> Routing:
    """Routing of a batch whose sequences contribute tokens_per_seq tokens each.

    [TRT-LLM] "一次 decode 批次的路由:从请求到 slot_ids" (the speculative-decoding branch of
    the sorted-indices step, and the counts step): sequence q owns tokens
    q*p .. q*p + p - 1 (p = tokens_per_seq); the sequences are sorted by slot (the
    same stable counting sort as at token level), then each sorted sequence index
    is expanded to its p token indices in order; the per-slot counts are the
    sequence counts times p and the offsets their cumulative sum.  Reading: an
    invalid sequence id makes its p tokens no-LoRA and counts them all as invalid
    (the count is per token, as for per-token ids).
    """
    p = int(tokens_per_seq)
    assert p >= 1
    seq_keys, seq_invalid = _keys(seq_ids, S)
    Q = len(seq_keys)
    # sequence level: counting sort
    seq_counts = [0] * (S + 1)
    for q in range(Q):
        seq_counts[int(seq_keys[q])] += 1
    cursor, run = [0] * (S + 1), 0
    for k in range(S + 1):
        cursor[k] = run
        run += seq_counts[k]
    sorted_seqs = [0] * Q
    for q in range(Q):
        k = int(seq_keys[q])
        sorted_seqs[cursor[k]] = q
        cursor[k] += 1
    # expansion to tokens
    token_sorted = [q * p + j for q in sorted_seqs for j in range(p)]
    counts = [c * p for c in seq_counts]
    keys = np.repeat(np.asarray(seq_keys, dtype=np.int64), p)
    return _finish(keys, token_sorted, counts, S, seq_invalid * p)


# ------------------------------------------------------------- shrink / expand
def _slice_offsets(slices: Sequence[int]) -> List[int]:
    """Column offset of each output slice in the packed output ([TRT-LLM] "前向替换":
    output_hidden_sizes and output_sizes_offset of the packed output buffer)."""
    offs, o = [], 0
    for d in slices:
        offs.append(o)
        o += int(d)
    return offs


def _contributes(ad: Optional[Adapter]) -> bool:
    return ad is not None and ad.rank > 0 and float(ad.scale()) != 0.0


def shrink_per_token(x: np.ndarray, adapters: Dict[int, Adapter], slices: Sequence[int],
                     ids: Sequence[int], S: int, max_rank: int):
    """u[n, t, j] = sum_c A_slot[n][j, c] * x[t, c]  (the shrink, lora_a).

    [vLLM-book] §16.4.2: lora_shrink projects each token onto its adapter's rank
    space, buffer [num_tokens, r]; [vLLM-deep] §6: lora_shrink computes A*x.
    Defined for tokens routed to a registered slot and j < rank; a missing slice
    gives zeros.  Returns (u [N, T, max_rank] float64, mask of defined entries).
    """
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    N = len(slices)
    keys, _ = _keys(ids, S)
    u = np.zeros((N, T, max_rank), dtype=np.float64)
    mask = np.zeros((N, T, max_rank), dtype=bool)
    for t in range(T):
        ad = adapters.get(int(keys[t])) if keys[t] < S else None
        if ad is None or ad.rank == 0:
            continue
        for n in range(N):
            if ad.A[n] is not None:
                u[n, t, :ad.rank] = np.asarray(ad.A[n], dtype=np.float64) @ x[t]
            mask[n, t, :ad.rank] = True
    return u, mask


def expand_per_token(u: np.ndarray, adapters: Dict[int, Adapter], slices: Sequence[int],
                     ids: Sequence[int], S: int, wdtype: str):
    """delta[t, o_n + i] = s_eff * sum_j B_eff[n][i, j] * u[n, t, j]  (the expand, lora_b).

    [vLLM-book] §16.4.2: lora_expand maps the rank-space buffer back to the output,
    [num_tokens, d], one output slice at a time (§16.4.4 add_expand "按 output slice
    写回").  The scale multiplies the completed sum ([llama.cpp] "真正的核心").
    Returns (delta [T, sum d] float64, touched [T, N] bool: which (token, slice) the
    branch writes).
    """
    T = u.shape[1]
    N = len(slices)
    offs = _slice_offsets(slices)
    keys, _ = _keys(ids, S)
    delta = np.zeros((T, int(sum(slices))), dtype=np.float64)
    touched = np.zeros((T, N), dtype=bool)
    for t in range(T):
        ad = adapters.get(int(keys[t])) if keys[t] < S else None
        if not _contributes(ad):
            continue
        for n in range(N):
            Bn, s_eff = effective_b(ad, n, wdtype)
            if Bn is None:
                continue
            delta[t, offs[n]:offs[n] + slices[n]] = s_eff * (Bn @ u[n, t, :ad.rank])
            touched[t, n] = True
    return delta, touched


def lora_apply(x, y_base, adapters: Dict[int, Adapter], slices: Sequence[int], ids: Sequence[int],
               S: int, wdtype: str, max_rank: Optional[int] = None) -> np.ndarray:
    """y = y_base + s * B (A x) per token, in float64 (the definition).

    [llama.cpp] "为什么低秩增量可以「后加」": h = W0 x + (alpha/r) B A x, the base and the
    branch act on the same input and are summed; [TRT-LLM] "前向替换:LoraLayer 的三条
    路径": the correction is added in place onto the base output (output.add_).
    Rows of no-LoRA tokens, of empty or zero-scale slots and columns of missing
    slices are returned as y_base unchanged.
    """
    x = np.asarray(x, dtype=np.float64)
    y = np.array(y_base, dtype=np.float64, copy=True)
    if max_rank is None:
        max_rank = max([a.rank for a in adapters.values()] + [1])
    u, _ = shrink_per_token(x, adapters, slices, ids, S, max_rank)
    delta, touched = expand_per_token(u, adapters, slices, ids, S, wdtype)
    offs = _slice_offsets(slices)
    for t in range(x.shape[0]):
        for n in range(len(slices)):
            if touched[t, n]:
                sl = slice(offs[n], offs[n] + slices[n])
                y[t, sl] = y[t, sl] + delta[t, sl]
    return y


def lora_apply_fp8(x, y_base, adapters: Dict[int, Adapter], slices: Sequence[int], ids: Sequence[int],
                   S: int, max_rank: Optional[int] = None) -> np.ndarray:
    """The FP8 adapter path: x (the BF16 activations, exact values) is first
    converted to FP8 (fp8_quantize), the adapters' A and B hold e4m3 values (and a
    pre-multiplied B the folded values); then the definition as lora_apply."""
    return lora_apply(fp8_quantize(x), y_base, adapters, slices, ids, S, "fp8", max_rank=max_rank)


def embedding_apply(vocab_ids: Sequence[int], y_base, adapters: Dict[int, Adapter], vocab: int,
                    ids: Sequence[int], S: int, wdtype: str) -> np.ndarray:
    """Embedding LoRA: y_t = y_base_t + s * B A[:, v_t] per token, in float64.

    [llama.cpp] "嵌入层:查表后再加增量": the token embedding is a table lookup, so the
    branch takes each token's r-vector out of A by its vocabulary id (get_rows), lifts
    it to the output width with B and adds the scaled result onto the lookup;
    "适配器文件:形状约定" (token_embd exception): A is [r, V], its columns indexed by
    vocabulary id, B is [d, r].  Each adapter has one slice: A[0] [r, V], B[0] [d, r].
    Reading: a vocabulary id outside [0, V) contributes zero (the row still gets
    y + 0); no-LoRA tokens and empty or zero-scale slots leave their rows unchanged.
    """
    y = np.array(y_base, dtype=np.float64, copy=True)
    keys, _ = _keys(ids, S)
    for t in range(len(keys)):
        ad = adapters.get(int(keys[t])) if keys[t] < S else None
        if not _contributes(ad) or ad.A[0] is None:
            continue
        A = np.asarray(ad.A[0], dtype=np.float64)
        assert A.shape == (ad.rank, vocab)
        v = int(vocab_ids[t])
        u = A[:, v] if 0 <= v < vocab else np.zeros(ad.rank)
        Bn, s_eff = effective_b(ad, 0, wdtype)
        y[t] = y[t] + s_eff * (Bn @ u)
    return y


def lora_apply_grouped(x, y_base, adapters: Dict[int, Adapter], slices: Sequence[int],
                       ids: Sequence[int], S: int, wdtype: str) -> np.ndarray:
    """Second formulation: the naive loop over the adapters present in the batch.

    [vLLM-book] §16.4.1 "朴素方案的代价": for each adapter in the batch, gather its
    tokens, output[idx] += scaling * (x[idx] @ A) @ B (row-vector notation; here A
    is stored [r, k] and B [d, r], so the products are x A^T and then (.) B^T).
    """
    x = np.asarray(x, dtype=np.float64)
    y = np.array(y_base, dtype=np.float64, copy=True)
    keys, _ = _keys(ids, S)
    offs = _slice_offsets(slices)
    for slot in sorted(set(int(k) for k in keys if k < S)):
        ad = adapters.get(slot)
        if not _contributes(ad):
            continue
        idx = np.nonzero(keys == slot)[0]
        for n in range(len(slices)):
            Bn, s_eff = effective_b(ad, n, wdtype)
            if ad.A[n] is None or Bn is None:
                continue
            sl = slice(offs[n], offs[n] + slices[n])
            y[np.ix_(idx, np.arange(sl.start, sl.stop))] += s_eff * ((x[idx] @ np.asarray(ad.A[n]).T) @ Bn.T)
    return y


def merged_apply(x, W0, adapters: Dict[int, Adapter], slices: Sequence[int], ids: Sequence[int],
                 S: int, wdtype: str) -> np.ndarray:
    """Linearity check: y_t = (W0 + s B A) x_t with the delta merged into the weight.

    [llama.cpp] "为什么低秩增量可以「后加」" (W = W0 + BA acts linearly, so merging and
    adding afterwards agree) and "从 PEFT 到 GGUF" (export-lora merges W0 + scale*BA
    offline).  W0 is [sum d, k]; a slice whose A or B is missing merges nothing.
    """
    x = np.asarray(x, dtype=np.float64)
    W0 = np.asarray(W0, dtype=np.float64)
    keys, _ = _keys(ids, S)
    offs = _slice_offsets(slices)
    y = np.zeros((x.shape[0], W0.shape[0]), dtype=np.float64)
    for t in range(x.shape[0]):
        W = W0.copy()
        ad = adapters.get(int(keys[t])) if keys[t] < S else None
        if _contributes(ad):
            for n in range(len(slices)):
                Bn, s_eff = effective_b(ad, n, wdtype)
                if ad.A[n] is None or Bn is None:
                    continue
                W[offs[n]:offs[n] + slices[n], :] += s_eff * (Bn @ np.asarray(ad.A[n], dtype=np.float64))
        y[t] = W @ x[t]
    return y


# ------------------------------------------------------------------ arithmetic
def extra_macs_per_token(k: int, slices: Sequence[int], r: int) -> int:
    """Multiply-adds the unmerged branch adds per token: r*k for A x, then d*r for B(.).

    [llama.cpp] "为什么低秩增量可以「后加」": 2dr extra multiply-adds per token when
    d = k, against dk for the base matmul.
    """
    return int(r) * int(k) + int(sum(slices)) * int(r)


def adapter_params(k: int, slices: Sequence[int], r: int) -> int:
    """Elements of one adapter on one linear layer: r*(d + k) ([llama.cpp] "性能与工程取舍";
    [vLLM-deep] §9 "显存估算": in_features*rank + out_features*rank)."""
    return int(r) * (int(k) + int(sum(slices)))
