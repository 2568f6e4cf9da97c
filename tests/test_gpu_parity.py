"""Parity of the HIP path against the CPU oracle, through the C ABI.

Bars: routing and index metadata bit-exact; fp32 max-abs error <= 1e-4; bf16
normwise relative error <= 2e-2 with fp32 accumulation, checked on the branch
output delta (base 0) and on y; exact-integer inputs bit-exact.
"""
import numpy as np
import pytest

import oracle.lora_oracle as O
from synthetic import small_case, workload

from lora_cases import (bits, check_close, from_device, make_pool, make_routing, oracle_adapters,
                         to_device, to_f64, y_base_of)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rx():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import rank_adapter_gemm_build_amd as m
    return m


def _log(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ routing
def _routing_case(rx, ids, S, max_tokens=None):
    import torch
    T = len(ids)
    R = rx.Routing(0, max_tokens or max(T, 1), S)
    t = torch.tensor(np.asarray(ids, dtype=np.int32), device="cuda")
    R.build(t)
    got = R.query()
    ref = O.route_by_counting(list(ids), S)
    assert np.array_equal(got["counts"], ref.counts)
    assert np.array_equal(got["seg_offsets"], ref.seg_offsets)
    assert np.array_equal(got["sorted_ids"], ref.sorted_ids)
    assert np.array_equal(got["active_slots"], ref.active_slots)
    assert got["num_active"] == ref.num_active and got["n_invalid"] == ref.n_invalid
    R.close()


def test_routing_golden(rx):
    import json, os
    with open(os.path.join(os.path.dirname(__file__), "golden", "routing_cases.json")) as f:
        for c in json.load(f)["cases"]:
            _routing_case(rx, c["ids"], c["S"])


@pytest.mark.parametrize("T,S,seed", [(1, 1, 0), (7, 3, 1), (64, 8, 2), (1000, 64, 3), (4096, 128, 4),
                                      (3333, 1024, 5), (20000, 17, 6), (513, 2, 7),
                                      # around the one-wave kernel's limits (launched for T <= 128, S < 128)
                                      (128, 127, 8), (127, 64, 9), (129, 100, 10), (257, 8, 11), (100, 128, 12)])
def test_routing_random(rx, T, S, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-1, S, size=T)
    bad = rng.random(T) < 0.05
    ids[bad] = rng.choice([S, S + 3, -2, -77], size=int(bad.sum()))
    _log(f"routing T={T} S={S}")
    _routing_case(rx, ids, S)


def test_routing_edges(rx):
    _routing_case(rx, [], 4)                       # empty batch
    _routing_case(rx, [-1] * 100, 4)               # no LoRA token
    _routing_case(rx, [3] * 777, 4)                # one segment
    _routing_case(rx, list(range(16)) * 4, 16, max_tokens=64)   # T == max_tokens
    _routing_case(rx, sorted(np.random.default_rng(9).integers(0, 32, 4352).tolist()), 32)  # prefill-like


def _runs_ids(rng, T, S, max_run=300):
    """Ids in runs: stretches of one slot (slots repeat across stretches) between
    stretches of mixed ids, including no-LoRA and invalid ones."""
    out = []
    while len(out) < T:
        n = int(rng.integers(1, max_run + 1))
        if rng.random() < 0.6:
            out += [int(rng.integers(-1, S))] * n
        else:
            mixed = rng.integers(-1, S, size=n)
            mixed[rng.random(n) < 0.05] = S + 7
            out += mixed.tolist()
    return out[:T]


# the workgroup kernel's scatter: 64-token groups of one key ranked by lane with the
# key's running offset kept in registers over a run, mixed groups by key matching
# (which may advance the cached key's offset); chunks held in registers and, above
# 16384 tokens, re-read per batch
@pytest.mark.parametrize("T,S,seed,max_run", [(6000, 24, 20, 300), (3000, 5, 21, 100), (5000, 1, 22, 200),
                                              (30000, 40, 23, 700), (1500, 300, 24, 90), (700, 3, 25, 64)])
def test_routing_runs(rx, T, S, seed, max_run):
    ids = _runs_ids(np.random.default_rng(seed), T, S, max_run)
    _log(f"routing runs T={T} S={S} max_run={max_run}")
    _routing_case(rx, ids, S)


def test_routing_single_key_batches(rx):
    _routing_case(rx, [-1] * 5000, 6)              # every group the no-LoRA key
    _routing_case(rx, [9] * 3000, 6)               # every id invalid
    _routing_case(rx, [2] * 2048 + [-1] * 2048, 3)  # two keys, both in whole groups
    _routing_case(rx, [0] * 64 * 16 * 16, 1)       # 16 waves of 16 whole groups each (the register limit)
    _routing_case(rx, [0] * (64 * 16 * 16 + 1), 1)  # one token past it


@pytest.mark.parametrize("num", [1, 2, 3, 4, 5])
def test_routing_workloads(rx, num):
    W = workload(num)
    _routing_case(rx, W.ids.tolist(), W.S)


# -------------------------------------------------------------- registration
@pytest.mark.parametrize("dtype,premultiply", [("bf16", False), ("bf16", True), ("f32", False), ("f32", True)])
def test_registration_bit_exact(rx, dtype, premultiply):
    W = small_case(11, T=8, S=4, k=136, slices=[40, 24], Rmax=12, dtype=dtype, alpha_scale=3.0,
                   rslora=True)
    mod = W.modules[0]
    pool = make_pool(rx, W, mod, premultiply=premultiply)
    ads = oracle_adapters(W, mod, premultiply=premultiply)
    for s, r in W.ranks.items():
        info = pool.slot_info(s)
        assert info["rank"] == r
        want_s = 1.0 if premultiply else float(O.lora_scale(W.alpha[s], r, W.rslora, W.adapter_scale))
        assert np.float32(info["scale"]).view(np.uint32) == np.float32(want_s).view(np.uint32)
        for n, d in enumerate(mod.slices):
            A, Bt = pool.read_slot(s, n)
            Bn, _ = O.effective_b(ads[s], n, dtype)
            assert np.array_equal(to_f64(A[:r], dtype), to_f64(mod.A[s][n], dtype))
            assert not to_f64(A[r:], dtype).any()
            assert np.array_equal(to_f64(Bt[:r], dtype), Bn.T), (s, n)
            assert not to_f64(Bt[r:], dtype).any()
    pool.unregister(1)
    assert pool.slot_info(1)["rank"] == 0
    pool.close()


def test_registration_device_sources_match_host(rx):
    import torch
    W = small_case(12, T=8, S=3, k=64, slices=[32], Rmax=8)
    mod = W.modules[0]
    p1 = make_pool(rx, W, mod, device_src=False)
    p2 = make_pool(rx, W, mod, device_src=True)
    torch.cuda.synchronize()
    for s in W.ranks:
        a1, b1 = p1.read_slot(s, 0)
        a2, b2 = p2.read_slot(s, 0)
        assert np.array_equal(a1, a2) and np.array_equal(b1, b2)
    p1.close(); p2.close()


# ------------------------------------------------------------------ linear
SMALL = [
    # seed, T, S, k, slices, Rmax, dtype, invalid
    (21, 37, 5, 520, [136, 24], 16, "bf16", 3),
    (22, 64, 8, 4096, [4096], 16, "bf16", 0),
    (23, 19, 3, 1032, [520], 64, "bf16", 2),
    (24, 45, 6, 264, [40, 8, 16], 9, "f32", 2),
    (25, 5, 2, 8, [8], 4, "f32", 0),
    (26, 130, 4, 2056, [1544], 32, "bf16", 0),
    (27, 300, 9, 1024, [1024, 512], 24, "bf16", 5),
    (28, 33, 4, 14336, [4096], 16, "bf16", 0),
]


def _run_linear(rx, W, mod, y0_bits, ydtype, premultiply=False):
    import torch
    pool = make_pool(rx, W, mod, premultiply=premultiply)
    R, ids = make_routing(rx, W)
    x = to_device(mod.x, W.dtype)
    y = to_device(y0_bits, ydtype)
    rx.linear(pool, R, x, y)
    torch.cuda.synchronize()
    out = y
    pool.close(); R.close()
    return out


@pytest.mark.parametrize("case", SMALL, ids=[f"seed{c[0]}" for c in SMALL])
@pytest.mark.parametrize("premultiply", [False, True])
def test_linear_small(rx, case, premultiply):
    seed, T, S, k, slices, Rmax, dtype, invalid = case
    _log(f"linear seed={seed} T={T} S={S} k={k} slices={slices} Rmax={Rmax} {dtype} pre={premultiply}")
    W = small_case(seed, T=T, S=S, k=k, slices=slices, Rmax=Rmax, dtype=dtype, invalid=invalid)
    mod = W.modules[0]
    ads = oracle_adapters(W, mod, premultiply=premultiply)
    x64 = to_f64(mod.x, dtype)
    D = sum(slices)
    # branch alone (base 0), output in fp32 for bf16 pools to isolate the branch error
    zero = np.zeros((T, D), dtype=np.float32)
    y = _run_linear(rx, W, mod, zero, "f32", premultiply)
    ref = O.lora_apply(x64, np.zeros((T, D)), ads, slices, W.ids, S, dtype, max_rank=Rmax)
    check_close(from_device(y), ref, dtype, "delta")
    # onto a base output in the pool dtype
    yb = mod.y_base
    y = _run_linear(rx, W, mod, yb, dtype, premultiply)
    ref = O.lora_apply(x64, to_f64(yb, dtype), ads, slices, W.ids, S, dtype, max_rank=Rmax)
    check_close(from_device(y), ref, dtype, "y")
    # rows with no LoRA are bit-untouched
    keys = np.where((W.ids >= 0) & (W.ids < S), W.ids, S)
    rows = keys == S
    assert np.array_equal(bits(y)[rows], (yb.view(np.uint32) if dtype == "f32" else yb)[rows])


def _integer_workload(seed, T, S, k, slices, Rmax, dtype):
    """Small integers: every partial sum and output is exact in fp32 and in bf16."""
    rng = np.random.default_rng(seed)
    W = small_case(seed, T=T, S=S, k=k, slices=slices, Rmax=Rmax, dtype=dtype,
                   ranks={s: int(rng.integers(1, min(Rmax, 4) + 1)) for s in range(S)})
    enc = (lambda a: O.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))) if dtype == "bf16" else \
          (lambda a: np.asarray(a, dtype=np.float32))
    mod = W.modules[0]
    for s, r in W.ranks.items():
        for n, d in enumerate(slices):
            A = np.zeros((r, k))
            for j in range(r):
                cols = rng.choice(k, size=min(8, k), replace=False)
                A[j, cols] = rng.integers(-1, 2, size=len(cols))
            mod.A[s][n] = enc(A)
            mod.B[s][n] = enc(rng.integers(-1, 2, size=(d, r)))
        W.alpha[s] = 2.0 * r        # scale 2 (a power of two)
    mod.x = enc(rng.integers(-2, 3, size=(T, k)))
    mod.y_base = enc(rng.integers(-64, 65, size=(T, sum(slices))))
    return W


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("premultiply", [False, True])
def test_exact_integer_inputs_bit_exact(rx, dtype, premultiply):
    W = _integer_workload(31, T=77, S=6, k=1040, slices=[520, 64], Rmax=8, dtype=dtype)
    mod = W.modules[0]
    ads = oracle_adapters(W, mod, premultiply=premultiply)
    y = _run_linear(rx, W, mod, mod.y_base, dtype, premultiply)
    ref = O.lora_apply(to_f64(mod.x, dtype), to_f64(mod.y_base, dtype), ads, mod.slices, W.ids, W.S, dtype,
                       max_rank=W.Rmax)
    assert np.abs(ref).max() < 256
    assert np.array_equal(from_device(y), ref)


def test_identity_adapter_closed_form(rx):
    """A = [I | 0], B = [I ; 0], s = 1: the branch copies x[:, :r] into y[:, :r]."""
    import torch
    T, k, d, r = 20, 64, 48, 8
    W = small_case(41, T=T, S=2, k=k, slices=[d], Rmax=r, dtype="bf16", ranks={0: r, 1: r}, p_nolora=0.0)
    mod = W.modules[0]
    A = np.zeros((r, k), dtype=np.float32); A[:, :r] = np.eye(r)
    B = np.zeros((d, r), dtype=np.float32); B[:r] = np.eye(r)
    for s in (0, 1):
        mod.A[s] = [O.f32_to_bf16_bits(A)]
        mod.B[s] = [O.f32_to_bf16_bits(B)]
        W.alpha[s] = float(r)
    y = _run_linear(rx, W, mod, np.zeros((T, d), dtype=np.float32), "f32")
    want = np.zeros((T, d)); want[:, :r] = to_f64(mod.x, "bf16")[:, :r]
    assert np.array_equal(from_device(y), want)


def test_shrink_and_expand_standalone(rx):
    import torch
    W = small_case(51, T=90, S=7, k=2048, slices=[264, 512], Rmax=16, invalid=2)
    mod = W.modules[0]
    N, D = len(mod.slices), sum(mod.slices)
    pool = make_pool(rx, W, mod)
    R, ids = make_routing(rx, W)
    x = to_device(mod.x, "bf16")
    u = torch.full((N, W.T, W.Rmax), float("nan"), device="cuda")
    rx.shrink(pool, R, x, u)
    torch.cuda.synchronize()
    ads = oracle_adapters(W, mod)
    u_ref, mask = O.shrink_per_token(to_f64(mod.x, "bf16"), ads, mod.slices, W.ids, W.S, W.Rmax)
    ug = u.double().cpu().numpy()
    assert not np.isnan(ug[mask]).any()
    err = np.abs(ug[mask] - u_ref[mask]).max() / np.abs(u_ref[mask]).max()
    assert err < 1e-4, err     # fp32 accumulation of exact bf16 products
    # expand from the oracle's u (rounded to fp32) onto a base
    u_in = torch.from_numpy(np.where(mask, u_ref, 0.0).astype(np.float32)).cuda()
    y = to_device(mod.y_base, "bf16")
    rx.expand(pool, R, u_in, y)
    torch.cuda.synchronize()
    delta, touched = O.expand_per_token(np.where(mask, u_ref, 0.0), ads, mod.slices, W.ids, W.S, "bf16")
    ref = to_f64(mod.y_base, "bf16") + delta
    check_close(from_device(y), ref, "bf16", "expand")
    # shrink then expand equals the fused call, bit for bit
    y1 = to_device(mod.y_base, "bf16")
    rx.expand(pool, R, u, y1)
    y2 = to_device(mod.y_base, "bf16")
    rx.linear(pool, R, x, y2)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    pool.close(); R.close()


def test_untouched_rows_and_columns(rx):
    """No-LoRA rows, empty slots, zero-scale slots and missing slices stay bit-identical
    (the tile-list kernels; slot mode has the same test of its own)."""
    import os
    import torch
    W = small_case(61, T=120, S=6, k=512, slices=[64, 128, 32], Rmax=8, invalid=4)
    mod = W.modules[0]
    mod.A[2][1] = None; mod.B[2][1] = None           # slot 2: slice 1 missing
    pool = make_pool(rx, W, mod)
    pool.unregister(3)                                 # slot 3 empty
    a, b = mod.A[4], mod.B[4]
    pool.register(4, a, b, W.alpha[4], W.ranks[4], adapter_scale=0.0)   # slot 4 unloaded by scale 0
    R, ids = make_routing(rx, W)
    y = to_device(mod.y_base, "bf16")
    os.environ["RAXLORA_SLOT_MODE"] = "0"
    try:
        rx.linear(pool, R, to_device(mod.x, "bf16"), y)
    finally:
        os.environ.pop("RAXLORA_SLOT_MODE", None)
    torch.cuda.synchronize()
    got, base = bits(y), mod.y_base
    keys = np.where((W.ids >= 0) & (W.ids < W.S), W.ids, W.S)
    for key in (W.S, 3, 4):
        rows = keys == key
        assert np.array_equal(got[rows], base[rows]), key
    rows = keys == 2
    assert np.array_equal(got[rows][:, 64:192], base[rows][:, 64:192])
    assert not np.array_equal(got[rows][:, :64], base[rows][:, :64])
    pool.close(); R.close()


def test_determinism_and_rerun(rx):
    import torch
    W = small_case(71, T=256, S=64, k=4096, slices=[4096, 1024, 1024], Rmax=16)
    mod = W.modules[0]
    pool = make_pool(rx, W, mod)
    R, ids = make_routing(rx, W)
    x = to_device(mod.x, "bf16")
    outs = []
    for _ in range(3):
        y = to_device(mod.y_base, "bf16")
        rx.linear(pool, R, x, y)
        outs.append(y)
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    assert torch.equal(outs[0].view(torch.int16), outs[2].view(torch.int16))
    pool.close(); R.close()


def test_reregister_smaller_rank(rx):
    import torch
    W = small_case(81, T=40, S=3, k=256, slices=[64], Rmax=16, ranks={0: 16, 1: 8, 2: 3}, p_nolora=0.0)
    mod = W.modules[0]
    pool = make_pool(rx, W, mod)
    # slot 0 re-registered with rank 5
    rng = np.random.default_rng(5)
    A = O.f32_to_bf16_bits(rng.standard_normal((5, 256)).astype(np.float32) / 16)
    B = O.f32_to_bf16_bits(rng.standard_normal((64, 5)).astype(np.float32) / 2)
    pool.register(0, [A], [B], 10.0, 5)
    W.ranks[0] = 5; mod.A[0] = [A]; mod.B[0] = [B]; W.alpha[0] = 10.0
    R, ids = make_routing(rx, W)
    y = to_device(mod.y_base, "bf16")
    rx.linear(pool, R, to_device(mod.x, "bf16"), y)
    torch.cuda.synchronize()
    ads = oracle_adapters(W, mod)
    ref = O.lora_apply(to_f64(mod.x, "bf16"), to_f64(mod.y_base, "bf16"), ads, [64], W.ids, 3, "bf16", 16)
    check_close(from_device(y), ref, "bf16", "y")
    pool.close(); R.close()


# ------------------------------------------------------------- errors on GPU
def test_error_paths_on_device(rx):
    import torch
    W = small_case(91, T=16, S=4, k=64, slices=[32], Rmax=8)
    mod = W.modules[0]
    pool = make_pool(rx, W, mod, max_tokens=16)
    R = rx.Routing(0, 64, 4)
    ids = torch.zeros(32, dtype=torch.int32, device="cuda")
    R.build(ids)
    x = torch.zeros(32, 64, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(32, 32, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(rx.LoraError) as e:
        rx.linear(pool, R, x, y)                       # T = 32 > pool max_tokens = 16
    assert e.value.status == rx.LORA_ERR_CAPACITY
    R16 = rx.Routing(0, 16, 4)
    with pytest.raises(rx.LoraError) as e:
        R16.build(ids)                                 # T = 32 > routing max_tokens
    assert e.value.status == rx.LORA_ERR_CAPACITY
    R16.build(ids[:16])
    R5 = rx.Routing(0, 16, 5)
    R5.build(ids[:16])
    with pytest.raises(rx.LoraError) as e:
        rx.linear(pool, R5, x[:16], y[:16])            # slot count mismatch
    assert e.value.status == rx.LORA_ERR_SHAPE
    xb = torch.zeros(16 * 64 + 8, dtype=torch.bfloat16, device="cuda")[1:1 + 16 * 64].view(16, 64)
    with pytest.raises(rx.LoraError) as e:
        rx.linear(pool, R16, xb, y[:16])               # misaligned x
    assert e.value.status == rx.LORA_ERR_ALIGN
    with pytest.raises(rx.LoraError) as e:
        rx.lora_linear(pool.handle, R16.handle, x.data_ptr(), 64, y.data_ptr(), 32, 7)
    assert e.value.status == rx.LORA_ERR_DTYPE
    a = np.zeros((9, 64), dtype=np.uint16); b = np.zeros((32, 9), dtype=np.uint16)
    with pytest.raises(rx.LoraError) as e:
        pool.register(0, [a], [b], 1.0, 9)             # rank above max_lora_rank
    assert e.value.status == rx.LORA_ERR_RANK
    with pytest.raises(rx.LoraError) as e:
        pool.register(4, [a[:4]], [b[:, :4].copy()], 1.0, 4)   # slot out of range
    assert e.value.status == rx.LORA_ERR_SLOT
    with pytest.raises(rx.LoraError) as e:
        rx.lora_register_adapter(pool.handle, 0, [a.ctypes.data], [0], 1.0, 4, False, 1.0, 0)
    assert e.value.status == rx.LORA_ERR_INVALID_ARG   # half-missing slice
    for o in (pool, R, R16, R5):
        o.close()


# ------------------------------------------------------ workloads at full size
def _sample_rows(W, rng, n=48):
    keys = np.where((W.ids >= 0) & (W.ids < W.S), W.ids, W.S)
    pick = set(rng.choice(W.T, size=min(n, W.T), replace=False).tolist())
    for s in np.unique(keys)[:2]:                    # every token of two segments too
        pick |= set(np.nonzero(keys == s)[0][:200].tolist())
    return np.array(sorted(pick))


@pytest.mark.parametrize("num", [1, 2, 3, 4, 5])
def test_workload_parity(rx, num):
    """Each workload at its full size, in the launch configuration the benchmark
    times (bf16 or fp32 output as the workload's).  The branch alone (base 0, fp32
    output) is checked on every row of every module against the oracle's grouped
    formulation (equal to the per-token definition within 1e-12); y on its base
    against the per-token definition, on all rows where that is quick (workloads 1
    and 2) and on sampled rows otherwise."""
    import torch
    W = workload(num)
    rng = np.random.default_rng(100 + num)
    R, ids = make_routing(rx, W)
    for mod in W.modules:
        _log(f"workload {num} module {mod.name} k={mod.k} slices={mod.slices} T={W.T}")
        pool = make_pool(rx, W, mod)
        ads = oracle_adapters(W, mod)
        x = to_device(mod.x, W.dtype)
        x64 = to_f64(mod.x, W.dtype)
        # the branch alone on every row
        d0 = torch.zeros((W.T, sum(mod.slices)), dtype=torch.float32, device="cuda")
        rx.linear(pool, R, x, d0)
        yb = y_base_of(W, mod)
        y = to_device(yb, W.dtype)
        rx.linear(pool, R, x, y)
        torch.cuda.synchronize()
        ref0 = O.lora_apply_grouped(x64, np.zeros(tuple(d0.shape)), ads, mod.slices, W.ids, W.S, W.dtype)
        check_close(d0.double().cpu().numpy(), ref0, W.dtype, f"workload {num} {mod.name} delta, all {W.T} rows")
        rows = np.arange(W.T) if num <= 2 else _sample_rows(W, rng)
        ref = O.lora_apply(x64[rows], to_f64(yb, W.dtype)[rows], ads, mod.slices, W.ids[rows], W.S, W.dtype,
                           max_rank=W.Rmax)
        got = from_device(y)[rows]
        check_close(got, ref, W.dtype, f"workload {num} {mod.name} y, {len(rows)} rows")
        untouched = (W.ids < 0) | (W.ids >= W.S)
        assert np.array_equal(bits(y)[untouched], (yb if W.dtype == "bf16" else yb.view(np.uint32))[untouched])
        if num == 2:
            W0 = to_f64(mod.W0, W.dtype)
            merged = O.merged_apply(x64, W0, ads, mod.slices, W.ids, W.S, W.dtype)
            check_close(got, merged, W.dtype, "merged-weight form")
        pool.close()
    R.close()


# ------------------------------------------------------ matrix-core segments
@pytest.mark.parametrize("segments,Rmax,slices", [
    ([16, 17, 31, 32, 33, 63, 64, 65, 300], 64, [4096]),  # around the tile size, mixed ranks
    ([128, 33, 200], 16, [4096, 1024, 1024]),          # packed slices
    ([40, 7, 90, 3, 129], 40, [520]),                  # rank not a multiple of 32, ragged d
    ([513], 8, [8200]),                                # one long segment, rank 8
])
def test_long_segments_matrix_cores(rx, segments, Rmax, slices):
    import os
    import torch
    W = small_case(300 + len(segments), T=0, S=12, k=2056, slices=slices, Rmax=Rmax, segments=segments)
    mod = W.modules[0]
    _log(f"segments {segments} Rmax={Rmax} slices={slices} T={W.T}")
    ads = oracle_adapters(W, mod)
    ref = O.lora_apply(to_f64(mod.x, "bf16"), np.zeros((W.T, sum(slices))), ads, slices, W.ids, W.S, "bf16",
                       max_rank=Rmax)
    outs = {}
    for mode in ("mfma", "vector"):
        if mode == "vector":
            os.environ["RAXLORA_DISABLE_MFMA"] = "1"
        try:
            y = _run_linear(rx, W, mod, np.zeros((W.T, sum(slices)), dtype=np.float32), "f32")
        finally:
            os.environ.pop("RAXLORA_DISABLE_MFMA", None)
        outs[mode] = from_device(y)
        err = check_close(outs[mode], ref, "bf16", f"delta ({mode})")
        _log(f"  {mode}: normwise rel err {err:.2e}")


@pytest.mark.parametrize("cb1", ["0", "1000000000"], ids=["four-block-units", "one-block-units"])
def test_expand_tiles_dealt_both_ways(rx, cb1):
    """The matrix-core expand's ways of dealing the tile list to the XCDs (one
    contiguous eighth per XCD, or runs of 1, 2 or 3 tiles dealt round the XCDs), with
    expand units of four column blocks and of one: bitwise equal to each other, and the
    branch alone against the oracle.  Segments of mixed lengths and ranks, 28 tiles
    (more than the XCDs, and partial runs at the end)."""
    import os
    segments = [40, 3, 70, 17, 100, 5, 33, 16, 64, 9, 48]
    slices = [1024, 384]
    W = small_case(640, T=0, S=10, k=1024, slices=slices, Rmax=64, segments=segments)
    mod = W.modules[0]
    ref = O.lora_apply(to_f64(mod.x, "bf16"), np.zeros((W.T, sum(slices))), oracle_adapters(W, mod), slices, W.ids,
                       W.S, "bf16", max_rank=W.Rmax)
    outs = {}
    for il in ("0", "1", "2", "3"):
        env = {"RAXLORA_TILE_INTERLEAVE": il, "RAXLORA_CB1_MAX": cb1, "RAXLORA_SLOT_MODE": "0"}
        saved = {k: os.environ.get(k) for k in env}
        os.environ.update(env)
        try:
            y = _run_linear(rx, W, mod, np.zeros((W.T, sum(slices)), dtype=np.float32), "f32")
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
        outs[il] = from_device(y)
        err = check_close(outs[il], ref, "bf16", f"delta (tile runs of {il}; 0: eighths)")
        _log(f"  interleave {il}, CB1_MAX {cb1}: normwise rel err {err:.2e}")
    for il in ("1", "2", "3"):
        assert np.array_equal(outs["0"], outs[il]), f"tiles dealt in runs of {il} differ from the eighths"


@pytest.mark.parametrize("mode", ["default", "tiles", "slot", "all-mfma", "all-mfma-wide", "mfma16", "vector"])
def test_short_segments_every_path(rx, mode):
    """Segments of 1..17 tokens through each split between the vector and matrix-core
    units: the default threshold, every segment on the matrix cores (1-token tiles;
    matrix-core expand units of one column block, then of four), a threshold of 16,
    and the vector units only."""
    import os
    segments = [1, 2, 3, 4, 5, 7, 8, 9, 12, 15, 16, 17]
    slices = [1024, 256, 256]
    W = small_case(520, T=0, S=14, k=1536, slices=slices, Rmax=48, segments=segments)
    mod = W.modules[0]
    _log(f"mode {mode} segments {segments} T={W.T}")
    ads = oracle_adapters(W, mod)
    ref = O.lora_apply(to_f64(mod.x, "bf16"), np.zeros((W.T, sum(slices))), ads, slices, W.ids, W.S, "bf16",
                       max_rank=W.Rmax)
    env = {"tiles": {"RAXLORA_SLOT_MODE": "0"}, "slot": {"RAXLORA_SLOT_MODE": "1"},
           "all-mfma": {"RAXLORA_MFMA_MIN_SEG": "1", "RAXLORA_CB1_MAX": "1000000000", "RAXLORA_SLOT_MODE": "0"},
           "all-mfma-wide": {"RAXLORA_MFMA_MIN_SEG": "1", "RAXLORA_CB1_MAX": "0", "RAXLORA_SLOT_MODE": "0"},
           "mfma16": {"RAXLORA_MFMA_MIN_SEG": "16", "RAXLORA_SLOT_MODE": "0"},
           "vector": {"RAXLORA_DISABLE_MFMA": "1"}}.get(mode, {})
    os.environ.update(env)
    try:
        y = _run_linear(rx, W, mod, np.zeros((W.T, sum(slices)), dtype=np.float32), "f32")
    finally:
        for key in env:
            os.environ.pop(key, None)
    err = check_close(from_device(y), ref, "bf16", f"delta ({mode})")
    _log(f"  normwise rel err {err:.2e}")


@pytest.mark.parametrize("Rmax", [96, 128, 256])
@pytest.mark.parametrize("mode", ["mfma", "slot", "vector"])
def test_high_rank_pools(rx, Rmax, mode):
    """Pools whose padded rank needs 3-8 matrix-core rank steps (the expand's general
    body) and several B^T row batches on the vector units; ranks mixed up to Rmax,
    short and long segments."""
    import os
    segments = [1, 3, 5, 17, 40, 2]
    slices = [520, 264]
    W = small_case(600 + Rmax, T=0, S=7, k=1032, slices=slices, Rmax=Rmax, segments=segments)
    mod = W.modules[0]
    _log(f"Rmax={Rmax} mode={mode} ranks={sorted(W.ranks.values())} T={W.T}")
    ads = oracle_adapters(W, mod)
    ref = O.lora_apply(to_f64(mod.x, "bf16"), np.zeros((W.T, sum(slices))), ads, slices, W.ids, W.S, "bf16",
                       max_rank=Rmax)
    env = {"vector": {"RAXLORA_DISABLE_MFMA": "1"}, "mfma": {"RAXLORA_SLOT_MODE": "0"},
           "slot": {"RAXLORA_SLOT_MODE": "1"}}[mode]
    os.environ.update(env)
    try:
        y = _run_linear(rx, W, mod, np.zeros((W.T, sum(slices)), dtype=np.float32), "f32")
    finally:
        for key in env:
            os.environ.pop(key, None)
    err = check_close(from_device(y), ref, "bf16", f"delta (Rmax={Rmax}, {mode})")
    _log(f"  normwise rel err {err:.2e}")


@pytest.mark.parametrize("S", [4, 3])
def test_shrink_matrix_cores_match_oracle(rx, S):
    """u from the matrix-core shrink of long segments (standalone lora_shrink); with
    S = 3 the batch averages 80 tokens per slot, so the call halves its k split."""
    import torch
    W = small_case(401, T=0, S=S, k=1024, slices=[256, 128], Rmax=32, segments=[70, 20, 150])
    mod = W.modules[0]
    pool = make_pool(rx, W, mod)
    R, ids = make_routing(rx, W)
    u = torch.full((2, W.T, 32), float("nan"), device="cuda")
    rx.shrink(pool, R, to_device(mod.x, "bf16"), u)
    torch.cuda.synchronize()
    u_ref, mask = O.shrink_per_token(to_f64(mod.x, "bf16"), oracle_adapters(W, mod), mod.slices, W.ids, W.S, 32)
    ug = u.double().cpu().numpy()
    assert not np.isnan(ug[mask]).any()
    assert np.abs(ug[mask] - u_ref[mask]).max() / np.abs(u_ref[mask]).max() < 1e-4
    pool.close(); R.close()


@pytest.mark.parametrize("case", ["max-slots", "max-in-features"])
def test_largest_pool_shapes(rx, case):
    """The largest shapes the boundary admits: 1024 slots (no rank-ordered dispatch,
    slot-table entries loaded per unit instead of held lane-wise, the workgroup
    routing kernel with a 1025-key histogram), and in_features = 65536 (16 k splits
    of 8 chunk steps each in the decode shrink)."""
    import torch
    if case == "max-slots":
        ranks = {s: 1 + (s * 7) % 16 for s in range(0, 1024, 3)}
        W = small_case(801, T=700, S=1024, k=512, slices=[256, 64], Rmax=16, ranks=ranks, invalid=4)
    else:
        W = small_case(802, T=0, S=3, k=65536, slices=[128], Rmax=8, segments=[1, 3, 20, 2])
    mod = W.modules[0]
    _log(f"{case}: T={W.T} S={W.S} k={mod.k} slices={mod.slices}")
    ads = oracle_adapters(W, mod)
    ref = O.lora_apply(to_f64(mod.x, "bf16"), np.zeros((W.T, sum(mod.slices))), ads, mod.slices, W.ids, W.S, "bf16",
                       max_rank=W.Rmax)
    y = _run_linear(rx, W, mod, np.zeros((W.T, sum(mod.slices)), dtype=np.float32), "f32")
    err = check_close(from_device(y), ref, "bf16", f"delta ({case})")
    _log(f"  normwise rel err {err:.2e}")
