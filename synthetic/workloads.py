"""Seeded synthetic inputs for batched multi-adapter LoRA.

This module is shared by the oracle-side tests and the GPU-side tests and bench.
It holds none of the method's arithmetic: it draws random numbers, stores them in
the input format (float32, or bfloat16 bit patterns), and records the shapes.  No
scale, routing, shrink or expand is computed here.

The five workloads follow the shapes the pages discuss for LoRA serving: hidden
size 4096 with ranks 8-64 ("vLLM LoRA 实现深度解析" §9 memory estimate, r = 64;
the vLLM book ch.16 §16.1.2, d = 4096, r = 8/16/32/64), a 7B-class layer with
q/k/v/o/gate/up/down projections ("llama.cpp ... LoRA 适配器" page, section
"性能与工程取舍"), decode batches that mix adapters per token and prefill segments
(the vLLM book §16.4.3).  None of the pages measures on a public dataset; these
seeded inputs stand in for real traffic.

Recipe (seed = 1000 + workload number, numpy default_rng):
  draw order: routing (ids / sequence lengths / sequence slots), then ranks, then
  for each module, each slot (ascending), each slice: A then B; then for each
  module x, then W0 (workloads 1-2) or y_base (3-5).
  A ~ N(0, 1/k), B ~ N(0, 1/r), x ~ N(0, 1), W0 ~ N(0, 1/k), y_base ~ N(0, 1);
  workload 1 keeps float32, the others are stored as bfloat16 (float32 draw,
  rounded to nearest-even).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

RANK_CHOICES = (8, 16, 32, 64)


def _to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Store float32 draws as bfloat16 bit patterns (nearest, ties to even).

    Inputs are finite random draws, so no NaN or overflow handling is needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


@dataclass
class ModuleInput:
    """One target projection: its adapters (per slot, per slice) and its activations."""
    name: str
    k: int
    slices: List[int]
    A: Dict[int, List[Optional[np.ndarray]]]   # slot -> per slice [r, k] (stored format)
    B: Dict[int, List[Optional[np.ndarray]]]   # slot -> per slice [d_n, r]
    x: np.ndarray                               # [T, k]
    W0: Optional[np.ndarray] = None             # [sum d, k]  (workloads 1-2)
    y_base: Optional[np.ndarray] = None         # [T, sum d]  (workloads 3-5)

    @property
    def d_total(self) -> int:
        return int(sum(self.slices))


@dataclass
class Workload:
    name: str
    number: int
    dtype: str                  # "f32" or "bf16": storage format of A, B, x, W0/y_base
    S: int                      # resident slots
    Rmax: int                   # max_lora_rank (pool padding)
    T: int
    ids: np.ndarray             # [T] int32 slot per token, -1 = no LoRA
    ranks: Dict[int, int]       # slot -> rank (every registered slot)
    alpha: Dict[int, float]
    rslora: bool
    adapter_scale: float
    modules: List[ModuleInput]
    notes: Dict[str, object] = field(default_factory=dict)


def _store(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    a = (rng.standard_normal(shape, dtype=np.float64) * std).astype(np.float32)
    return a if dtype == "f32" else _to_bf16_bits(a)


def _draw_adapters(rng, mod_specs, ranks, dtype):
    out = []
    for name, k, slices in mod_specs:
        A, B = {}, {}
        for slot in sorted(ranks):
            r = ranks[slot]
            A[slot], B[slot] = [], []
            for d in slices:
                A[slot].append(_store(rng, (r, k), np.sqrt(1.0 / k), dtype))
                B[slot].append(_store(rng, (d, r), np.sqrt(1.0 / r), dtype))
        out.append((name, k, list(slices), A, B))
    return out


def _finish_modules(rng, drawn, T, dtype, with_w0: bool) -> List[ModuleInput]:
    mods = []
    for name, k, slices, A, B in drawn:
        x = _store(rng, (T, k), 1.0, dtype)
        mods.append(ModuleInput(name=name, k=k, slices=slices, A=A, B=B, x=x))
    for m in mods:
        if with_w0:
            m.W0 = _store(rng, (m.d_total, m.k), np.sqrt(1.0 / m.k), dtype)
        else:
            m.y_base = _store(rng, (T, m.d_total), 1.0, dtype)
    return mods


def zipf_pmf(n: int, s: float) -> np.ndarray:
    """Truncated Zipf popularity over n slots: p_i proportional to i^-s, i = 1..n."""
    w = np.arange(1, n + 1, dtype=np.float64) ** (-s)
    return w / w.sum()


def workload(number: int, seed: Optional[int] = None) -> Workload:
    """Build one of the five workloads (1..5) from its seed."""
    seed = 1000 + number if seed is None else seed
    rng = np.random.default_rng(seed)
    if number == 1:
        # single adapter, fp32, T=16, k=d=512, r=8, alpha=16 (scale 2), all tokens slot 0
        T, S, k, r = 16, 1, 512, 8
        ids = np.zeros(T, dtype=np.int32)
        ranks = {0: r}
        drawn = _draw_adapters(rng, [("proj", k, [512])], ranks, "f32")
        mods = _finish_modules(rng, drawn, T, "f32", with_w0=True)
        return Workload("single-adapter-fp32-T16-k512-r8", 1, "f32", S, r, T, ids, ranks,
                        {0: 16.0}, False, 1.0, mods)
    if number == 2:
        # decode, 8 slots, T=64 one token per sequence, k=d=4096, r=16, alpha=32
        T, S, k, r = 64, 8, 4096, 16
        ids = rng.integers(-1, S, size=T).astype(np.int32)   # uniform over {-1, 0..7}
        ranks = {s: r for s in range(S)}
        drawn = _draw_adapters(rng, [("proj", k, [4096])], ranks, "bf16")
        mods = _finish_modules(rng, drawn, T, "bf16", with_w0=True)
        return Workload("decode-8slots-T64-k4096-r16", 2, "bf16", S, r, T, ids, ranks,
                        {s: 32.0 for s in range(S)}, False, 1.0, mods)
    if number == 3:
        # prefill: 16 sequences of length U[32,512], slot per sequence from 32, mixed ranks
        S, k, nseq = 32, 4096, 16
        lengths = rng.integers(32, 513, size=nseq)
        seq_slots = rng.integers(0, S, size=nseq)
        ids = np.concatenate([np.full(L, s, dtype=np.int32) for L, s in zip(lengths, seq_slots)])
        T = int(ids.shape[0])
        ranks = {s: int(rng.choice(RANK_CHOICES)) for s in range(S)}
        drawn = _draw_adapters(rng, [("proj", k, [4096])], ranks, "bf16")
        mods = _finish_modules(rng, drawn, T, "bf16", with_w0=False)
        return Workload(f"prefill-16seq-T{T}-k4096-mixed-rank", 3, "bf16", S, 64, T, ids, ranks,
                        {s: 2.0 * ranks[s] for s in range(S)}, False, 1.0, mods,
                        notes={"lengths": lengths.tolist(), "seq_slots": seq_slots.tolist()})
    if number == 4:
        # packed QKV + gate_up + down decode, T=256, 64 slots, r=16, rsLoRA alpha=16 (scale 4)
        T, S, r = 256, 64, 16
        ids = rng.integers(0, S, size=T).astype(np.int32)
        ranks = {s: r for s in range(S)}
        specs = [("qkv", 4096, [4096, 1024, 1024]), ("gate_up", 4096, [14336, 14336]),
                 ("down", 14336, [4096])]
        drawn = _draw_adapters(rng, specs, ranks, "bf16")
        mods = _finish_modules(rng, drawn, T, "bf16", with_w0=False)
        return Workload("packed-qkv-gateup-down-T256-64slots-r16", 4, "bf16", S, r, T, ids, ranks,
                        {s: 16.0 for s in range(S)}, True, 1.0, mods)
    if number == 5:
        # 128 slots, Zipf(1.1) popularity, 768 decode tokens + 2 prefill segments of 128
        S = 128
        p = zipf_pmf(S, 1.1)
        dec = rng.choice(S, size=768, p=p)
        pre = rng.choice(S, size=2, p=p)
        ids = np.concatenate([dec, np.full(128, pre[0]), np.full(128, pre[1])]).astype(np.int32)
        T = int(ids.shape[0])
        ranks = {s: int(rng.choice(RANK_CHOICES)) for s in range(S)}
        specs = [("q", 4096, [4096]), ("k", 4096, [1024]), ("v", 4096, [1024]), ("o", 4096, [4096]),
                 ("gate", 4096, [14336]), ("up", 4096, [14336]), ("down", 14336, [4096])]
        drawn = _draw_adapters(rng, specs, ranks, "bf16")
        mods = _finish_modules(rng, drawn, T, "bf16", with_w0=False)
        return Workload("zipf-128slots-T1024-7proj-mixed-rank", 5, "bf16", S, 64, T, ids, ranks,
                        {s: 2.0 * ranks[s] for s in range(S)}, False, 1.0, mods,
                        notes={"prefill_slots": pre.tolist()})
    raise ValueError(f"unknown workload {number}")


def small_case(seed: int, T: int, S: int, k: int, slices, Rmax: int, dtype: str = "bf16",
               ranks: Optional[Dict[int, int]] = None, p_nolora: float = 0.125,
               invalid: int = 0, alpha_scale: float = 2.0, rslora: bool = False,
               segments: Optional[List[int]] = None) -> Workload:
    """A small seeded case for parity tests: ragged k, d, T and mixed ranks.

    ``segments`` (optional) lays tokens out as contiguous runs of one slot each
    (prefill-like); otherwise every token draws its slot independently, with
    probability ``p_nolora`` of -1 and ``invalid`` tokens given ids outside
    {-1} U [0, S).
    """
    rng = np.random.default_rng(seed)
    if segments is not None:
        slots = rng.integers(0, S, size=len(segments))
        ids = np.concatenate([np.full(L, s, dtype=np.int64) for L, s in zip(segments, slots)])
        T = int(ids.shape[0])
    else:
        ids = rng.integers(0, S, size=T)
        ids = np.where(rng.random(T) < p_nolora, -1, ids)
        if invalid:
            pos = rng.choice(T, size=min(invalid, T), replace=False)
            bad = rng.choice([S, S + 7, -2, -1000], size=len(pos))
            ids[pos] = bad
    ids = ids.astype(np.int32)
    if ranks is None:
        ranks = {s: int(rng.integers(1, Rmax + 1)) for s in range(S)}
    drawn = _draw_adapters(rng, [("proj", k, list(slices))], ranks, dtype)
    mods = _finish_modules(rng, drawn, T, dtype, with_w0=False)
    return Workload(f"small-{seed}", 0, dtype, S, Rmax, T, ids, ranks,
                    {s: alpha_scale * r for s, r in ranks.items()}, rslora, 1.0, mods)
