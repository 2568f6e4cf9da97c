#!/usr/bin/env python3
"""Benchmark of the batched multi-adapter LoRA hot path on one MI355X.

One step = one pass of the whole hot path over one batch: build the routing
metadata from the batch's token -> slot ids, then one fused shrink+expand per
target module, adding onto a base output already in HBM.  The first module's call
is lora_route_linear (routing + shrink + expand; for batches of up to 256 tokens the
routing is built inside the shrink launch), the others lora_linear on that routing.
--separate-routing times lora_build_routing + lora_linear instead.
Adapters are registered before timing (registration is once per adapter, off the
per-step path).  Inputs are seeded synthetic tensors shaped like the workload.

To keep the 256 MB Infinity Cache (and the L2) from serving repeated steps, the
timed loop rotates over M independent instances (pools, routing, x, y, ids) whose
algorithmic traffic adds up to at least --rotate-mib.

Prints ONE JSON line on stdout (progress goes to stderr).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LoRA tokens/sec and shrink+expand HBM GB/s (% peak), d=k=4096 r=16 multi-adapter"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, AMD published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------------ accounting
def step_accounting(W, mfma_min: int, use_mfma: bool):
    """Algorithmic HBM bytes per step, per kernel family, from the routing counts.

    Per module, for every slot with tokens and rank r > 0: the shrink must read the
    slot's A at its true rank (r * k elements per present slice) and each of its
    tokens' x rows once (k elements); the expand must read B at its true rank
    (r * d_n per present slice) and read and write each token's output row once
    (2 * sum d_n).  No-LoRA tokens, padding rows and the rank-space intermediate are
    not counted.  Segments of at least mfma_min tokens count toward the matrix-core
    kernels when those are in use.
    """
    import numpy as np
    wb = 2 if W.dtype == "bf16" else 4
    keys = np.where((W.ids >= 0) & (W.ids < W.S), W.ids, W.S)
    counts = np.bincount(keys, minlength=W.S + 1)
    acc = {"shrink": 0, "expand": 0}
    split = {"shrink_decode": 0, "expand_decode": 0, "shrink_mfma": 0, "expand_mfma": 0}
    flops = 0
    mfma_flops = 0
    for mod in W.modules:
        D = sum(mod.slices)
        for s, r in W.ranks.items():
            L = int(counts[s])
            if L == 0 or r == 0:
                continue
            fam = "mfma" if (use_mfma and L >= mfma_min) else "decode"
            sb = r * mod.k * len(mod.slices) * wb + L * mod.k * wb
            eb = r * D * wb + 2 * L * D * wb
            acc["shrink"] += sb
            acc["expand"] += eb
            split[f"shrink_{fam}"] += sb
            split[f"expand_{fam}"] += eb
            flops += 2 * L * r * (mod.k * len(mod.slices) + D)
            if fam == "mfma":
                mfma_flops += 2 * L * r * (mod.k * len(mod.slices) + D)
    split["mfma_flops"] = mfma_flops
    return acc, flops, split


# -------------------------------------------------------------------- workload
class Instance:
    """One independent copy of the step's device state."""

    def __init__(self, rx, torch, W, dev_src, ydt):
        self.mods = []
        self.routing = rx.Routing(0, W.T, W.S)
        self.ids = torch.from_numpy(W.ids.astype("int32")).cuda()
        for m, src in zip(W.modules, dev_src):
            pool = rx.Pool(0, W.S, W.Rmax, m.k, m.slices, rx.LORA_BF16 if W.dtype == "bf16" else rx.LORA_F32, W.T)
            for s, r in W.ranks.items():
                pool.register(s, src["A"][s], src["B"][s], W.alpha[s], r, W.rslora, W.adapter_scale,
                              device_src=True)
            x = src["x"].clone()
            y = src["y"].clone()
            self.mods.append((pool, x, y))
        self.calls = [(p.handle, x.data_ptr(), x.stride(0), y.data_ptr(), y.stride(0)) for p, x, y in self.mods]
        # the arguments of one grouped call over every module
        import ctypes as C
        n = len(self.calls)
        self.group = (n, (C.c_void_p * n)(*[c[0] for c in self.calls]), (C.c_void_p * n)(*[c[1] for c in self.calls]),
                      (C.c_int * n)(*[c[2] for c in self.calls]), (C.c_void_p * n)(*[c[3] for c in self.calls]),
                      (C.c_int * n)(*[c[4] for c in self.calls]))

    def close(self):
        for p, _, _ in self.mods:
            p.close()
        self.routing.close()


def upload_sources(torch, W):
    import numpy as np

    def dev(a):
        if a is None:
            return None
        if W.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()

    out = []
    for m in W.modules:
        src = {"A": {s: [dev(a) for a in m.A[s]] for s in W.ranks},
               "B": {s: [dev(b) for b in m.B[s]] for s in W.ranks},
               "x": dev(m.x)}
        if m.y_base is not None:
            src["y"] = dev(m.y_base)
        else:  # base output of the caller's own base GEMM (not part of the library)
            W0 = dev(m.W0)
            src["y"] = (src["x"].float() @ W0.float().T).to(src["x"].dtype)
            src["W0T"] = W0.t().contiguous()   # [k, d], for the base-GEMM overlap measurement
        out.append(src)
    return out


def source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rank_adapter_gemm_build_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload_name: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when the
    counters are missing or were taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload_name, {}).get(kernel)
    if not e or e.get("source_digest") != source_digest():
        return None
    return e.get("bytes_per_launch")


# ----------------------------------------------------------------- cpu baseline
def cpu_baseline(W, seconds: float):
    """The oracle as it stands, timed on this host: its grouped float64 formulation
    (per slot: gather the slot's rows, two matmuls, scatter) over the whole batch,
    with the BLAS threads set to the cores this process may run on; and, beside it,
    its per-token definition on a bounded share of the same time."""
    import numpy as np
    import oracle.lora_oracle as O
    import contextlib
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=cores, user_api="blas")
    except Exception:
        limit = contextlib.nullcontext()
    mods = []
    for m in W.modules:
        conv = (lambda a: None if a is None else O.bf16_bits_to_f64(a)) if W.dtype == "bf16" else \
               (lambda a: None if a is None else np.asarray(a, dtype=np.float64))
        ads = {s: O.Adapter(rank=r, A=[conv(a) for a in m.A[s]], B=[conv(b) for b in m.B[s]], alpha=W.alpha[s],
                            rslora=W.rslora, adapter_scale=W.adapter_scale) for s, r in W.ranks.items()}
        yb = conv(m.y_base) if m.y_base is not None else np.zeros((W.T, sum(m.slices)))
        mods.append((conv(m.x), yb, ads, m.slices))

    def timed(fn, budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            for x, yb, ads, slices in mods:
                fn(x, yb, ads, slices)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return reps, el

    with limit:
        reps, el = timed(lambda x, yb, ads, sl: O.lora_apply_grouped(x, yb, ads, sl, W.ids, W.S, W.dtype),
                         0.75 * seconds)
        preps, pel = timed(lambda x, yb, ads, sl: O.lora_apply(x, yb, ads, sl, W.ids, W.S, W.dtype,
                                                               max_rank=W.Rmax), 0.25 * seconds)
    return {"value": reps * W.T / el, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"the whole {W.name} batch ({W.T} tokens, {len(W.modules)} module(s)) through "
                      f"oracle.lora_apply_grouped (float64, per slot: gather, two matmuls, scatter; BLAS threads = "
                      f"{cores} cores of the affinity mask), repeated {reps} times in {el:.1f} s",
            "per_token_definition": {"value": preps * W.T / pel, "unit": "tokens/s",
                                     "sample": f"oracle.lora_apply (float64 per-token loop), the same batch "
                                               f"{preps} times in {pel:.1f} s"}}


# ------------------------------------------------------- graph replay, overlap
def measure_graph_and_overlap(torch, rx, lib, insts, src, W, ydt, args):
    """Two deployment forms of the same step, timed like the main loop (rotating
    instances, events around the whole run):
    - graph: the step of G consecutive instances captured once in a HIP graph
      (torch.cuda.CUDAGraph) and replayed; the launches then cost no host work;
    - overlap (workloads with a base weight W0): the caller's base GEMM y = x W0^T
      (torch.mm into y, one shared W0) followed by the LoRA step, serially on one
      stream, against the GEMM on stream A and the LoRA step on stream B joined to it
      (lora_route_linear_join: routing and shrink run beside the GEMM, the expand
      waits for its event)."""
    T = W.T
    M = len(insts)
    G = min(32, M)

    def step_on(inst, stream):
        calls = inst.calls
        pool, xp, ldx, yp, ldy = calls[0]
        st = lib.lora_route_linear(pool, inst.routing.handle, inst.ids.data_ptr(), T, xp, ldx, yp, ldy, ydt, stream)
        if st:
            raise rx.LoraError(st, "lora_route_linear")
        for pool, xp, ldx, yp, ldy in calls[1:]:
            st = lib.lora_linear(pool, inst.routing.handle, xp, ldx, yp, ldy, ydt, stream)
            if st:
                raise rx.LoraError(st, "lora_linear")

    res = {}
    if args.only_overlap:
        return measure_overlap(torch, rx, lib, insts, src, W, ydt, args, step_on, res)
    # graphs of G steps each, covering every instance
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(G):
            step_on(insts[i], side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for g0 in range(0, M - G + 1, G):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream().cuda_stream
            for i in range(g0, g0 + G):
                step_on(insts[i], cs)
        graphs.append(g)
    torch.cuda.synchronize()
    reps = max(1, args.steps // G)
    for g in graphs[:2]:
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for r in range(reps):
        graphs[r % len(graphs)].replay()
    e1.record()
    torch.cuda.synchronize()
    res["graph_us_per_step"] = round(e0.elapsed_time(e1) * 1e3 / (reps * G), 3)
    res["graph_steps_per_replay"] = G
    del graphs
    log(f"graph replay: {res['graph_us_per_step']:.2f} us/step ({G} steps per graph)")

    # speculative-decoding batch of the same size: T / 4 sequences of 4 tokens, the
    # routing built from one slot id per sequence (lora_build_routing_seq)
    if T % 4 == 0:
        p = 4
        seq = torch.from_numpy(W.ids[: T // p].astype("int32")).cuda()

        def seq_step(i):
            inst = insts[i % M]
            st = lib.lora_build_routing_seq(inst.routing.handle, seq.data_ptr(), T // p, p, torch.cuda.current_stream().cuda_stream)
            if st:
                raise rx.LoraError(st, "lora_build_routing_seq")
            for pool, xp, ldx, yp, ldy in inst.calls:
                st = lib.lora_linear(pool, inst.routing.handle, xp, ldx, yp, ldy, ydt, torch.cuda.current_stream().cuda_stream)
                if st:
                    raise rx.LoraError(st, "lora_linear")

        for i in range(10):
            seq_step(i)
        torch.cuda.synchronize()
        e0.record()
        for i in range(args.steps):
            seq_step(i)
        e1.record()
        torch.cuda.synchronize()
        res["seq_routing_step_us"] = round(e0.elapsed_time(e1) * 1e3 / args.steps, 3)
        res["seq_routing_step"] = f"lora_build_routing_seq ({T // p} sequences x {p} tokens) + lora_linear per module"
        log(f"sequence-routed step: {res['seq_routing_step_us']:.2f} us/step")

    return measure_overlap(torch, rx, lib, insts, src, W, ydt, args, step_on, res)


def measure_overlap(torch, rx, lib, insts, src, W, ydt, args, step_on, res):
    """The caller's base GEMM beside the LoRA step (see measure_graph_and_overlap)."""
    T, M = W.T, len(insts)
    if len(W.modules) == 1 and "W0T" in src[0]:
        W0T = src[0]["W0T"]
        sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
        n = args.steps
        evs = [torch.cuda.Event() for _ in range(M)]
        done = [torch.cuda.Event() for _ in range(M)]
        for d in done:
            d.record(sb)

        def gemm(inst):
            _, x, y = inst.mods[0]
            torch.mm(x, W0T, out=y)

        def timed(body):
            for i in range(min(n, 10)):
                body(i)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            sa.wait_stream(torch.cuda.current_stream())
            sb.wait_stream(torch.cuda.current_stream())
            for i in range(n):
                body(i)
            torch.cuda.current_stream().wait_stream(sa)
            torch.cuda.current_stream().wait_stream(sb)
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) * 1e3 / n

        def only_gemm(i):
            with torch.cuda.stream(sa):
                gemm(insts[i % M])

        def serial(i):
            inst = insts[i % M]
            with torch.cuda.stream(sa):
                gemm(inst)
                step_on(inst, sa.cuda_stream)

        def overlap(i):
            # step i's GEMM waits for step i-1's LoRA result (a next layer's input
            # depends on it); step i's routing and shrink then run beside the GEMM
            inst = insts[i % M]
            ev = evs[i % M]
            with torch.cuda.stream(sa):
                sa.wait_event(done[(i - 1) % M])
                gemm(inst)
                ev.record(sa)
            pool, xp, ldx, yp, ldy = inst.calls[0]
            st = lib.lora_route_linear_join(pool, inst.routing.handle, inst.ids.data_ptr(), T, xp, ldx, yp, ldy, ydt,
                                            sb.cuda_stream, ev.cuda_event)
            if st:
                raise rx.LoraError(st, "lora_route_linear_join")
            done[i % M].record(sb)

        def overlap_free(i):
            # throughput form: no dependency between consecutive steps
            inst = insts[i % M]
            ev = evs[i % M]
            with torch.cuda.stream(sa):
                gemm(inst)
                ev.record(sa)
            pool, xp, ldx, yp, ldy = inst.calls[0]
            st = lib.lora_route_linear_join(pool, inst.routing.handle, inst.ids.data_ptr(), T, xp, ldx, yp, ldy, ydt,
                                            sb.cuda_stream, ev.cuda_event)
            if st:
                raise rx.LoraError(st, "lora_route_linear_join")

        # the forms run one after the other, 2 ms apart (so a kernel trace separates them)
        res["base_gemm_us"] = round(timed(only_gemm), 3)
        time.sleep(0.002)
        res["gemm_then_lora_us_per_step"] = round(timed(serial), 3)
        time.sleep(0.002)
        res["gemm_beside_lora_us_per_step"] = round(timed(overlap), 3)
        time.sleep(0.002)
        res["gemm_beside_lora_independent_steps_us_per_step"] = round(timed(overlap_free), 3)
        time.sleep(0.002)

        # the two forms captured in HIP graphs of G2 chained steps each: serial (GEMM then
        # LoRA on one stream) and forked (each GEMM on a side stream that first waits for
        # the previous step, the LoRA branch on the capturing stream joined to the GEMM's
        # event); the graph holds the cross-stream edges instead of runtime event waits
        G2 = min(16, M)
        fa = torch.cuda.Stream()

        def capture(forked, lora=True):
            gr = torch.cuda.CUDAGraph()
            warm = torch.cuda.Stream()
            warm.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(warm):
                for i in range(G2):
                    gemm(insts[i])
                    step_on(insts[i], warm.cuda_stream)
            torch.cuda.current_stream().wait_stream(warm)
            torch.cuda.synchronize()
            with torch.cuda.graph(gr):
                cs = torch.cuda.current_stream()
                for i in range(G2):
                    inst = insts[i]
                    if not lora:
                        gemm(inst)
                    elif forked:
                        fa.wait_stream(cs)
                        with torch.cuda.stream(fa):
                            gemm(inst)
                            evs[i].record(fa)
                        pool, xp, ldx, yp, ldy = inst.calls[0]
                        st = lib.lora_route_linear_join(pool, inst.routing.handle, inst.ids.data_ptr(), T, xp, ldx,
                                                        yp, ldy, ydt, cs.cuda_stream, evs[i].cuda_event)
                        if st:
                            raise rx.LoraError(st, "lora_route_linear_join")
                    else:
                        gemm(inst)
                        step_on(inst, cs.cuda_stream)
                if forked:
                    cs.wait_stream(fa)
            torch.cuda.synchronize()
            return gr

        for key, forked, lora in (("graph_base_gemm_us", False, False), ("graph_gemm_then_lora_us_per_step", False, True),
                                  ("graph_gemm_beside_lora_us_per_step", True, True)):
            time.sleep(0.002)
            gr = capture(forked, lora)
            time.sleep(0.002)   # gaps around the first replay keep a kernel trace's phases apart
            gr.replay()
            torch.cuda.synchronize()
            time.sleep(0.002)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = max(2, n // G2)
            a.record()
            for _ in range(reps):
                gr.replay()
            b.record()
            torch.cuda.synchronize()
            res[key] = round(a.elapsed_time(b) * 1e3 / (reps * G2), 3)
            del gr
        log(f"graphs of {G2} steps: base GEMM alone {res['graph_base_gemm_us']:.2f} us, "
            f"GEMM then LoRA {res['graph_gemm_then_lora_us_per_step']:.2f} us/step, "
            f"GEMM beside LoRA {res['graph_gemm_beside_lora_us_per_step']:.2f} us/step")
        res["base_gemm"] = f"torch.mm [{T},{W0T.shape[0]}] x [{W0T.shape[0]},{W0T.shape[1]}] bf16, one W0 for all instances"
        log(f"base GEMM {res['base_gemm_us']:.2f} us; GEMM then LoRA {res['gemm_then_lora_us_per_step']:.2f} us/step; "
            f"GEMM beside LoRA (joined) {res['gemm_beside_lora_us_per_step']:.2f} us/step; independent steps "
            f"{res['gemm_beside_lora_independent_steps_us_per_step']:.2f} us/step")
    return res


# ------------------------------------------------------------- embedding LoRA
def measure_embedding(torch, rx, lib, W, args, vocab=32000):
    """Embedding LoRA on the workload's batch (one module): the same slots, ranks,
    ids and output width, A drawn as [r, vocab] per slot (seeded), vocabulary ids
    uniform; one step = lora_build_routing + lora_embedding (gather + expand) onto a
    resident bf16 lookup result.  Rotates over enough instances to exceed the
    256 MB Infinity Cache.  Algorithmic bytes per step: per LoRA token its rank row
    (r x 2 B) and the output row read and written (2 x d x 2 B), per active slot its
    B (r x d x 2 B)."""
    import numpy as np
    m = W.modules[0]
    d, T = m.slices[0], W.T
    if len(m.slices) != 1 or W.dtype != "bf16":
        return None
    rng = np.random.default_rng(4242)
    keys = np.where((W.ids >= 0) & (W.ids < W.S), W.ids, W.S)
    counts = np.bincount(keys, minlength=W.S + 1)
    step_bytes = sum(int(counts[s]) * (r * 2 + 4 * d) + r * d * 2 for s, r in W.ranks.items() if counts[s] > 0)
    per_inst = W.S * W.Rmax * vocab * 2 + W.S * W.Rmax * d * 4 + T * d * 2
    M = max(2, min(64, int(np.ceil(1.5 * 2 ** 30 / per_inst))))
    ids = torch.from_numpy(W.ids.astype(np.int32)).cuda()
    insts = []
    for i in range(M):
        pool = rx.Pool(0, W.S, W.Rmax, vocab, [d], rx.LORA_BF16, T, embedding=True)
        for s, r in W.ranks.items():
            A = torch.randn((r, vocab), device="cuda").to(torch.bfloat16)
            B = (torch.randn((d, r), device="cuda") / float(np.sqrt(r))).to(torch.bfloat16)
            pool.register(s, [A], [B], W.alpha[s], r, W.rslora, W.adapter_scale, device_src=True)
        R = rx.Routing(0, T, W.S)
        v = torch.from_numpy(rng.integers(0, vocab, size=T).astype(np.int32)).cuda()
        y = torch.randn((T, d), device="cuda").to(torch.bfloat16)
        insts.append((pool, R, v, y))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream

    ids_p = ids.data_ptr()
    calls = [(pool.handle, R.handle, v.data_ptr(), y.data_ptr(), y.stride(0)) for pool, R, v, y in insts]

    def step(i):
        ph, rh, vp, yp, ldy = calls[i % M]
        st = lib.lora_route_embedding(ph, rh, ids_p, T, vp, yp, ldy, rx.LORA_BF16, stream)
        if st:
            raise rx.LoraError(st, "lora_route_embedding")

    for i in range(min(args.warmup, 10) + M):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    kern = {k: round(v["avg_us"], 3) for k, v in kernel_times(rx, torch, step, args.steps).items()}
    for pool, R, _, _ in insts:
        pool.close()
        R.close()
    res = {"us_per_step": round(us, 3), "tokens_per_s": round(T / (us * 1e-6), 1),
           "step_algorithmic_bytes": step_bytes, "step_hbm_gbps": round(step_bytes / (us * 1e-6) / 1e9, 2),
           "kernels_avg_us": kern, "vocab": vocab, "rotation_instances": M,
           "step": "lora_route_embedding (routing + gather + expand), bf16, same slots/ids as the workload"}
    log(f"embedding LoRA: {us:.2f} us/step, kernels {kern}")
    return res


# ------------------------------------------------------------ FP8 adapter pools
def measure_fp8(torch, rx, lib, W, src, args, step_bytes_bf16, acc_bf16):
    """The same workload with FP8 (e4m3) adapter pools: every A and B converted to
    e4m3 by torch (float8_e4m3fn), activations and outputs bf16 as before; one step
    = lora_route_linear + lora_linear per further module, rotating over as many
    instances as the bf16 loop (their traffic still several times the 256 MB
    Infinity Cache; more instances, as many as the smaller FP8 step would take for
    the same traffic, were measured to slow both the bf16 and the FP8 decode step by
    about 1.2 us, so the two forms are compared at one rotation).  Algorithmic bytes:
    the bf16 step's with the weight bytes halved (x and y unchanged)."""
    import numpy as np
    if W.dtype != "bf16" or not hasattr(torch, "float8_e4m3fn"):
        return None
    T = W.T
    # weight bytes of the bf16 step (shrink: A, expand: B), halved for e4m3
    keys = np.where((W.ids >= 0) & (W.ids < W.S), W.ids, W.S)
    counts = np.bincount(keys, minlength=W.S + 1)
    wbytes = sum(r * (m.k * len(m.slices) + sum(m.slices)) * 2 for m in W.modules
                 for s, r in W.ranks.items() if counts[s] > 0)
    step_bytes = step_bytes_bf16 - wbytes // 2
    per_inst = sum(W.S * W.Rmax * (m.k * len(m.slices) + 2 * sum(m.slices)) for m in W.modules)
    M = max(2, min(args.max_instances, int(np.ceil(args.rotate_mib * 2 ** 20 / max(step_bytes_bf16, 1)))))
    M = min(M, max(2, int(40 * 2 ** 30 // max(per_inst, 1))))

    def fp8(t):
        return None if t is None else t.float().clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).contiguous()

    conv = [{"A": {s: [fp8(a) for a in src_m["A"][s]] for s in W.ranks},
             "B": {s: [fp8(b) for b in src_m["B"][s]] for s in W.ranks}} for src_m in src]
    ids = torch.from_numpy(W.ids.astype(np.int32)).cuda()
    insts = []
    for i in range(M):
        mods = []
        R = rx.Routing(0, T, W.S)
        for m, src_m, c in zip(W.modules, src, conv):
            pool = rx.Pool(0, W.S, W.Rmax, m.k, m.slices, rx.LORA_FP8E4M3, T)
            for s, r in W.ranks.items():
                pool.register(s, c["A"][s], c["B"][s], W.alpha[s], r, W.rslora, W.adapter_scale, device_src=True)
            mods.append((pool, src_m["x"].clone(), src_m["y"].clone()))
        insts.append((R, mods))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream

    import ctypes as C
    groups = []
    for R, mods in insts:
        n = len(mods)
        groups.append((n, (C.c_void_p * n)(*[p.handle for p, _, _ in mods]),
                       (C.c_void_p * n)(*[x.data_ptr() for _, x, _ in mods]), (C.c_int * n)(*[x.stride(0) for _, x, _ in mods]),
                       (C.c_void_p * n)(*[y.data_ptr() for _, _, y in mods]), (C.c_int * n)(*[y.stride(0) for _, _, y in mods])))
    grouped = len(W.modules) > 1 and not args.per_module

    # every pointer and stride taken once, so the timed loop makes no torch calls
    ids_p = ids.data_ptr()
    calls = [(R.handle, [(p.handle, x.data_ptr(), x.stride(0), y.data_ptr(), y.stride(0)) for p, x, y in mods])
             for R, mods in insts]

    def step(i):
        if grouped:
            n, P, X, LX, Y, LY = groups[i % M]
            st = lib.lora_route_linear_group(P, n, calls[i % M][0], ids_p, T, X, LX, Y, LY, rx.LORA_BF16, stream)
            if st:
                raise rx.LoraError(st, "lora_route_linear_group")
            return
        rh, mc = calls[i % M]
        pool, xp, ldx, yp, ldy = mc[0]
        st = lib.lora_route_linear(pool, rh, ids_p, T, xp, ldx, yp, ldy, rx.LORA_BF16, stream)
        if st:
            raise rx.LoraError(st, "lora_route_linear")
        for pool, xp, ldx, yp, ldy in mc[1:]:
            st = lib.lora_linear(pool, rh, xp, ldx, yp, ldy, rx.LORA_BF16, stream)
            if st:
                raise rx.LoraError(st, "lora_linear")

    for i in range(min(args.warmup, 10) + M):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    kern = {k: round(v["avg_us"], 3) for k, v in kernel_times(rx, torch, step, args.steps).items()}
    for R, mods in insts:
        R.close()
        for pool, _, _ in mods:
            pool.close()
    res = {"us_per_step": round(us, 3), "tokens_per_s": round(T / (us * 1e-6), 1), "step_algorithmic_bytes": step_bytes,
           "step_hbm_gbps": round(step_bytes / (us * 1e-6) / 1e9, 2), "kernels_avg_us": kern, "rotation_instances": M,
           "calls": "lora_route_linear_group" if grouped else "lora_route_linear + lora_linear per further module",
           "weights": "e4m3 (OCP), activations and outputs bf16; the matrix-core shrink on the FP8 matrix cores"}
    log(f"FP8 pools: {us:.2f} us/step ({step_bytes / 1e6:.1f} MB algorithmic), kernels {kern}")
    return res


# ------------------------------------------------------------------ timing core
def make_step(rx, lib, insts, T, ydt, stream, separate_routing: bool, grouped: bool = False):
    """One step on instance i % M: the routing and every module's fused call; grouped:
    the routing and one grouped call over all modules (lora_route_linear_group)."""
    M = len(insts)

    def group_step(i):
        inst = insts[i % M]
        n, P, X, LX, Y, LY = inst.group
        st = lib.lora_route_linear_group(P, n, inst.routing.handle, inst.ids.data_ptr(), T, X, LX, Y, LY, ydt, stream)
        if st:
            raise rx.LoraError(st, "lora_route_linear_group")

    def step(i):
        inst = insts[i % M]
        calls = inst.calls
        if separate_routing:
            st = lib.lora_build_routing(inst.routing.handle, inst.ids.data_ptr(), T, stream)
            if st:
                raise rx.LoraError(st, "lora_build_routing")
        else:
            pool, xp, ldx, yp, ldy = calls[0]
            st = lib.lora_route_linear(pool, inst.routing.handle, inst.ids.data_ptr(), T, xp, ldx, yp, ldy, ydt,
                                       stream)
            if st:
                raise rx.LoraError(st, "lora_route_linear")
            calls = calls[1:]
        for pool, xp, ldx, yp, ldy in calls:
            st = lib.lora_linear(pool, inst.routing.handle, xp, ldx, yp, ldy, ydt, stream)
            if st:
                raise rx.LoraError(st, "lora_linear")
    return group_step if grouped and len(insts[0].calls) > 1 else step


def time_steps(torch, step, steps: int):
    """Events around `steps` back-to-back steps: (ms per step, host wall us per step)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    return e0.elapsed_time(e1) / steps, wall * 1e6 / steps


def kernel_times(rx, torch, step, steps: int, chunk: int = 16):
    """Per-kernel average durations: the same steps again, each launch stamped by a
    pair of events at the kernel's own start and end (on the launch's stream).

    A start stamp is taken when the stream reaches it; if the host is still
    submitting the kernel then, the gap counts as kernel time.  So every chunk of
    steps is queued behind a spin kernel (torch.cuda._sleep) that outlasts the host's
    submission of the chunk, and the chunk's launches then run back to back as in the
    timed loop.  A first pass, not counted, measures the host's submission time and
    leaves the library holding enough events, so none is created in the second."""
    # spin cycles per microsecond of the gate, measured
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    torch.cuda._sleep(1_000_000)
    e1.record()
    torch.cuda.synchronize()
    cycles_per_us = 1_000_000 / max(e0.elapsed_time(e1) * 1e3, 1e-3)
    rx.lora_timing_enable(True)
    host_us = None
    for rep_pass in range(2):
        w0 = time.perf_counter()
        for c0 in range(0, steps, chunk):
            if host_us is not None:
                torch.cuda._sleep(int(cycles_per_us * (2 * host_us * chunk + 50)))
            for i in range(c0, min(steps, c0 + chunk)):
                step(i)
        host_us = (time.perf_counter() - w0) * 1e6 / steps
        torch.cuda.synchronize()
        rep = rx.lora_timing_report()
    rx.lora_timing_enable(False)
    return {k: {"avg_us": 1e3 * ms / n, "launches_per_step": n / steps} for k, (ms, n) in rep.items() if n}


def family_roofline(acc, kern):
    """Per kernel family: algorithmic bytes per launch over its average launch time."""
    out = {}
    for k, v in kern.items():
        if k not in acc or v["launches_per_step"] <= 0:
            continue
        per_launch = acc[k] / v["launches_per_step"]
        gbps = per_launch / (v["avg_us"] * 1e-6) / 1e9
        out[k] = {"bytes_per_launch": int(per_launch), "avg_launch_us": round(v["avg_us"], 3),
                  "launches_per_step": round(v["launches_per_step"], 3), "achieved_gbps": round(gbps, 1),
                  "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    return out


def build_instances(rx, torch, W, args, step_bytes):
    M = max(2, min(args.max_instances, math.ceil(args.rotate_mib * 2 ** 20 / max(step_bytes, 1))))
    src = upload_sources(torch, W)
    insts = [Instance(rx, torch, W, src, None) for _ in range(M)]
    torch.cuda.synchronize()
    return src, insts


def measure_workload(torch, rx, num: int, args):
    """A further workload timed like the headline one (rotating instances, events
    around the steps, per-kernel event stamps): µs per step, tokens/s, the step's
    algorithmic bytes and rate, and each kernel family's rate per launch."""
    from synthetic import workload
    t0 = time.perf_counter()
    W = workload(num)
    use_mfma = W.dtype == "bf16" and os.environ.get("RAXLORA_DISABLE_MFMA", "0") == "0"
    mfma_min = int(os.environ.get("RAXLORA_MFMA_MIN_SEG", "4"))
    acc, flops, by_path = step_accounting(W, mfma_min, use_mfma)
    step_bytes = sum(acc.values())
    src, insts = build_instances(rx, torch, W, args, step_bytes)
    ydt = rx.LORA_BF16 if W.dtype == "bf16" else rx.LORA_F32
    stream = torch.cuda.current_stream().cuda_stream
    grouped = len(W.modules) > 1 and not args.per_module
    step = make_step(rx, rx.lib, insts, W.T, ydt, stream, False, grouped=grouped)
    steps = max(args.steps, 20)
    for i in range(max(args.warmup, len(insts))):
        step(i)
    ms, wall = time_steps(torch, step, steps)
    kern = kernel_times(rx, torch, step, steps)
    per_module_us = None
    if grouped:
        # the same step as one fused call per module, for comparison
        pm = make_step(rx, rx.lib, insts, W.T, ydt, stream, False, grouped=False)
        for i in range(len(insts)):
            pm(i)
        per_module_us = round(time_steps(torch, pm, steps)[0] * 1e3, 3)
    for inst in insts:
        inst.close()
    insts = []
    torch.cuda.synchronize()
    fp8 = None
    if not args.no_extras and len(W.modules) > 1:
        fp8 = measure_fp8(torch, rx, rx.lib, W, src, args, step_bytes, acc)
    del src
    torch.cuda.synchronize()
    us = ms * 1e3
    res = {"us_per_step": round(us, 3), "tokens_per_s": round(W.T / (us * 1e-6), 1), "tokens": W.T,
           "modules": [m.name for m in W.modules], "launches_per_step": round(sum(v["launches_per_step"]
                                                                                   for v in kern.values()), 2),
           "step_algorithmic_bytes": step_bytes, "step_hbm_gbps": round(step_bytes / (us * 1e-6) / 1e9, 1),
           "step_frac_of_peak": round(step_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
           "kernels": family_roofline(acc, kern),
           "routing_avg_us": round(kern["routing"]["avg_us"], 3) if "routing" in kern else None,
           "steps_timed": steps, "setup_s": round(time.perf_counter() - t0, 1),
           "calls": "lora_route_linear_group (all modules in one shrink and one expand launch)" if grouped else
                    "lora_route_linear + lora_linear per further module",
           "per_module_calls_us_per_step": per_module_us, "fp8_pools": fp8}
    log(f"workload {W.name}: {us:.1f} us/step ({'grouped' if grouped else 'per module'}; per-module calls "
        f"{per_module_us} us/step), {res['step_hbm_gbps']} GB/s over the step "
        f"({100 * res['step_frac_of_peak']:.1f} % of 8 TB/s), kernels "
        + ", ".join(f"{k} {v['avg_launch_us']} us x{v['launches_per_step']} ({100 * v['frac_of_peak']:.1f} %)"
                    for k, v in res["kernels"].items()))
    return W.name, res


def device_ceilings(torch, rx):
    """The device's own floors and ceilings, measured in the same run: the shortest
    kernel (a one-element fill, back to back), a 512 MiB device copy (ROCclr), and
    the library's streaming probe (a 1 GiB read; a 1 GiB read with 256 MiB written)."""
    tiny = torch.zeros(1, device="cuda")
    src_c = torch.empty(1024 * 2 ** 20, dtype=torch.uint8, device="cuda")
    dst_c = torch.empty(512 * 2 ** 20, dtype=torch.uint8, device="cuda")
    half = src_c[: 512 * 2 ** 20]
    stream = torch.cuda.current_stream().cuda_stream

    def probe(ratio):
        st = rx.lib.lora_bandwidth_probe(src_c.data_ptr(), src_c.numel(), dst_c.data_ptr(), dst_c.numel(), ratio,
                                         stream)
        if st:
            raise rx.LoraError(st, "lora_bandwidth_probe")

    for _ in range(5):
        tiny.fill_(1.0)
        dst_c.copy_(half)
        probe(0)
        probe(4)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def rate(fn, n):
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n   # ms per call

    floor_us = rate(lambda: tiny.fill_(1.0), 100) * 1e3
    copy_gbps = 2 * half.numel() / (rate(lambda: dst_c.copy_(half), 10) * 1e-3) / 1e9
    read_gbps = src_c.numel() / (rate(lambda: probe(0), 10) * 1e-3) / 1e9
    rw_gbps = (src_c.numel() * 5 // 4) / (rate(lambda: probe(4), 10) * 1e-3) / 1e9
    del src_c, dst_c, half
    torch.cuda.synchronize()
    log(f"shortest-kernel floor {floor_us:.2f} us; copy {copy_gbps:.0f} GB/s; streaming read {read_gbps:.0f} GB/s; "
        f"read 4 : write 1 {rw_gbps:.0f} GB/s")
    return {"shortest_kernel_floor_us": round(floor_us, 3), "copy_gbps": round(copy_gbps, 1),
            "read_gbps": round(read_gbps, 1), "read4_write1_gbps": round(rw_gbps, 1)}


# ------------------------------------------------------------------------ main
def run(args):
    import torch

    import rank_adapter_gemm_build_amd as rx
    from synthetic import workload

    torch.cuda.set_device(0)
    W = workload(args.workload)
    use_mfma = W.dtype == "bf16" and os.environ.get("RAXLORA_DISABLE_MFMA", "0") == "0"
    mfma_min = int(os.environ.get("RAXLORA_MFMA_MIN_SEG", "4"))   # the library default
    acc, flops, by_path = step_accounting(W, mfma_min, use_mfma)
    step_bytes = sum(acc.values())
    log(f"workload {W.name}: T={W.T} S={W.S} modules={[m.name for m in W.modules]} "
        f"algorithmic bytes/step={step_bytes / 1e6:.2f} MB")
    src, insts = build_instances(rx, torch, W, args, step_bytes)
    M = len(insts)
    log(f"{M} rotation instances registered")
    stream = torch.cuda.current_stream().cuda_stream
    ydt = rx.LORA_BF16 if W.dtype == "bf16" else rx.LORA_F32
    lib, T = rx.lib, W.T
    grouped = len(W.modules) > 1 and not (args.per_module or args.separate_routing)
    step = make_step(rx, lib, insts, T, ydt, stream, args.separate_routing, grouped=grouped)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")
    if args.only_overlap:
        res = measure_graph_and_overlap(torch, rx, lib, insts, src, W, ydt, args)
        for inst in insts:
            inst.close()
        return {"only_overlap": res, "workload": W.name}
    ms_per_step, wall_us = time_steps(torch, step, args.steps)
    log(f"timed {args.steps} steps: {ms_per_step * 1e3:.2f} us/step (wall {wall_us:.2f} us/step)")

    kern = kernel_times(rx, torch, step, args.steps)
    log("kernels: " + ", ".join(f"{k} {v['avg_us']:.2f} us" for k, v in kern.items()))
    families = family_roofline(acc, kern)

    # dominant kernel: most time per step among the shrink/expand kernels
    cand = {k: v for k, v in kern.items() if k in acc}
    dom = max(cand, key=lambda k: cand[k]["avg_us"] * cand[k]["launches_per_step"])
    per_launch = acc[dom] / cand[dom]["launches_per_step"]
    achieved = per_launch / (cand[dom]["avg_us"] * 1e-6) / 1e9
    traffic = load_traffic(dom, W.name)
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic, "kernel": dom,
                "bytes_per_launch": int(per_launch), "avg_launch_us": round(cand[dom]["avg_us"], 3)}

    # per-step distribution (events around each step)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record()
        step(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    per_step = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    pct = {f"p{q}": round(per_step[min(len(per_step) - 1, int(q / 100 * len(per_step)))], 3) for q in (10, 50, 90)}
    log(f"per-step p10/p50/p90 {pct['p10']}/{pct['p50']}/{pct['p90']} us")

    ceil = device_ceilings(torch, rx)
    roofline["copy_ceiling_gbps"] = ceil["copy_gbps"]
    roofline["read_ceiling_gbps"] = ceil["read_gbps"]
    roofline["frac_of_copy"] = round(achieved / ceil["copy_gbps"], 4)
    roofline["frac_of_read_ceiling"] = round(achieved / ceil["read_gbps"], 4)

    # the eager legs first, each with only its own instances allocated (after the graph
    # and two-stream legs, eager launches on the current stream were measured slower:
    # the FP8 step 12.9 -> 19.3 us), then the graph and overlap legs on a new set
    for inst in insts:
        inst.close()
    insts = []
    torch.cuda.synchronize()
    embedding = None if args.no_extras else measure_embedding(torch, rx, lib, W, args)
    fp8 = None if args.no_extras else measure_fp8(torch, rx, lib, W, src, args, step_bytes, acc)
    graph_overlap = None
    if not args.no_extras:
        insts = [Instance(rx, torch, W, src, None) for _ in range(M)]
        torch.cuda.synchronize()
        graph_overlap = measure_graph_and_overlap(torch, rx, lib, insts, src, W, ydt, args)
        for inst in insts:
            inst.close()
        insts = []
    del src
    torch.cuda.synchronize()

    # matrix-core path: its algorithmic FLOPs over the shrink + expand kernel time of a
    # step (a lower bound of the MFMA utilisation: those launches also run the vector
    # units' work; the executed MFMA FLOPs from counters are in profiles/mfma_*.md)
    mfma_flops = by_path.pop("mfma_flops", 0)
    kt = sum(v["avg_us"] * v["launches_per_step"] for k, v in kern.items() if k in ("shrink", "expand"))
    mfma_path = None
    if mfma_flops and kt > 0:
        tf = mfma_flops / (kt * 1e-6) / 1e12
        mfma_path = {"algorithmic_flop_per_step": int(mfma_flops), "tflops_over_shrink_expand_time": round(tf, 2),
                     "peak_tflops_bf16_dense": 2500.0, "frac": round(tf / 2500.0, 5)}

    others = {}
    for num in ([] if args.no_workloads else [int(v) for v in args.workloads.split(",") if v.strip()]):
        if num == args.workload:
            continue
        name, res = measure_workload(torch, rx, num, args)
        others[name] = res

    tokens_per_s = T / (ms_per_step * 1e-3)
    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": W.dtype, "data": "synthetic",
        "config": {"workload": W.name, "tokens": T, "slots": W.S, "k": [m.k for m in W.modules],
                   "slices": [m.slices for m in W.modules], "ranks": sorted(set(W.ranks.values())),
                   "max_lora_rank": W.Rmax, "parallelism": "none (1 GPU)",
                   "calls": "lora_build_routing + lora_linear" if args.separate_routing else
                            "lora_route_linear_group" if grouped else "lora_route_linear + lora_linear"},
        "roofline": roofline,
        "extra": {"step_algorithmic_bytes": step_bytes, "step_hbm_gbps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 2),
                  "step_flops": flops, "bytes_by_path": by_path, "kernels": kern, "kernel_families": families,
                  "rotation_instances": M, "wall_us_per_step": round(wall_us, 3), "step_us_percentiles": pct,
                  "device": ceil, "source_digest": source_digest(),
                  "graph_and_overlap": graph_overlap, "embedding_lora": embedding, "fp8_pools": fp8,
                  "mfma_path": mfma_path, "workloads": others},
    }
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle for ~{args.cpu_seconds:.0f} s")
        out["cpu_baseline"] = cpu_baseline(W, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, help="1..5 (default 2: decode, 8 slots, T=64, k=d=4096, r=16)")
    ap.add_argument("--rotate-mib", type=float, default=1024.0)
    ap.add_argument("--max-instances", type=int, default=512)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the graph-replay, base-GEMM overlap, embedding and FP8 timings")
    ap.add_argument("--workloads", default="3,4,5",
                    help="further workloads timed after the headline one, reported under extra.workloads")
    ap.add_argument("--no-workloads", action="store_true", help="time the headline workload only")
    ap.add_argument("--only-overlap", action="store_true",
                    help="time only the base-GEMM overlap forms (for a kernel trace of them) and print their JSON")
    ap.add_argument("--per-module", action="store_true",
                    help="multi-module workloads: one fused call per module instead of one grouped call")
    ap.add_argument("--separate-routing", action="store_true",
                    help="lora_build_routing + lora_linear per step instead of lora_route_linear for the first module")
    ap.add_argument("--json-out", default=None, help="also write the JSON line to this file")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the path has no cross-GPU sharding or collectives)", file=sys.stderr)
        sys.exit(2)
    out = run(args)
    line = json.dumps(out)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")
    print(line, flush=True)


if __name__ == "__main__":
    main()
