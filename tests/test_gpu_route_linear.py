"""lora_route_linear (routing built inside the shrink launch for small batches)
against lora_build_routing + lora_linear and against the oracle, through the C ABI.

Bars: the routing outputs bit-exact against the oracle's counting sort; y bitwise
identical to the two-call path (same kernels' arithmetic on the same sorted
positions) and within the oracle tolerances.
"""
import os

import numpy as np
import pytest

import oracle.lora_oracle as O
from synthetic import small_case

from lora_cases import bits, check_close, from_device, make_pool, oracle_adapters, to_device, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rx():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import rank_adapter_gemm_build_amd as m
    return m


def _log(msg):
    print(msg, flush=True)


CASES = [
    # seed, T, S, k, slices, Rmax, dtype, invalid, segments
    (31, 64, 8, 4096, [4096], 16, "bf16", 0, None),          # decode batch, 8 slots
    (32, 37, 5, 520, [136, 24], 16, "bf16", 3, None),        # ragged widths, invalid ids
    (33, 45, 6, 264, [40, 8, 16], 9, "f32", 2, None),        # fp32 pool, vector units only
    (34, 1, 1, 8, [8], 4, "f32", 0, None),                   # one token
    (35, 256, 64, 1024, [1024, 256, 256], 16, "bf16", 4, None),   # packed slices, 256 tokens
    (36, 256, 255, 512, [512], 16, "bf16", 9, None),         # most slots a launch routes itself
    (37, 0, 6, 1032, [520], 64, "bf16", 0, [1, 2, 3, 4, 17, 40, 90, 99]),  # long segments, 2+ tiles
    (38, 300, 9, 1024, [1024, 512], 24, "bf16", 5, None),    # above 256 tokens: two-call fallback
]


def _ids_tensor(W):
    import torch
    return torch.from_numpy(np.ascontiguousarray(W.ids, dtype=np.int32)).cuda()


def _two_calls(rx, W, mod, y0, ydt):
    import torch
    pool = make_pool(rx, W, mod)
    R = rx.Routing(0, max(W.T, 1), W.S)
    R.build(_ids_tensor(W))
    y = to_device(y0, ydt)
    rx.linear(pool, R, to_device(mod.x, W.dtype), y)
    torch.cuda.synchronize()
    q = R.query()
    pool.close(); R.close()
    return y, q


def _fused(rx, W, mod, y0, ydt):
    import torch
    pool = make_pool(rx, W, mod)
    R = rx.Routing(0, max(W.T, 1), W.S)
    ids = _ids_tensor(W)
    y = to_device(y0, ydt)
    rx.route_linear(pool, R, ids, to_device(mod.x, W.dtype), y)
    torch.cuda.synchronize()
    q = R.query()
    pool.close(); R.close()
    return y, q


@pytest.mark.parametrize("mode", ["default", "tiles", "slot", "all-mfma", "vector"])
@pytest.mark.parametrize("case", CASES, ids=[f"seed{c[0]}" for c in CASES])
def test_route_linear_matches_two_calls(rx, case, mode):
    seed, T, S, k, slices, Rmax, dtype, invalid, segments = case
    W = small_case(seed, T=T, S=S, k=k, slices=slices, Rmax=Rmax, dtype=dtype, invalid=invalid, segments=segments)
    mod = W.modules[0]
    _log(f"route_linear seed={seed} T={W.T} S={S} slices={slices} Rmax={Rmax} {dtype} mode={mode}")
    env = {"tiles": {"RAXLORA_SLOT_MODE": "0"}, "slot": {"RAXLORA_SLOT_MODE": "1"},
           "all-mfma": {"RAXLORA_MFMA_MIN_SEG": "1", "RAXLORA_SLOT_MODE": "0"},
           "vector": {"RAXLORA_DISABLE_MFMA": "1"}}.get(mode, {})
    os.environ.update(env)
    try:
        D = sum(slices)
        yz = np.zeros((W.T, D), dtype=np.float32)
        y_ref, q_ref = _two_calls(rx, W, mod, yz, "f32")
        y_got, q_got = _fused(rx, W, mod, yz, "f32")
        # onto a base output in the pool dtype
        yb_ref, _ = _two_calls(rx, W, mod, mod.y_base, dtype)
        yb_got, _ = _fused(rx, W, mod, mod.y_base, dtype)
    finally:
        for key in env:
            os.environ.pop(key, None)
    ref = O.route_by_counting(list(W.ids), S)
    for q in (q_got, q_ref):
        assert np.array_equal(q["counts"], ref.counts)
        assert np.array_equal(q["seg_offsets"], ref.seg_offsets)
        assert np.array_equal(q["sorted_ids"], ref.sorted_ids)
        assert np.array_equal(q["active_slots"], ref.active_slots)
        assert q["num_active"] == ref.num_active and q["n_invalid"] == ref.n_invalid
    assert np.array_equal(bits(y_got), bits(y_ref)), "delta differs from build_routing + linear"
    assert np.array_equal(bits(yb_got), bits(yb_ref)), "y differs from build_routing + linear"
    ads = oracle_adapters(W, mod)
    x64 = to_f64(mod.x, dtype)
    delta = O.lora_apply(x64, np.zeros((W.T, D)), ads, slices, W.ids, S, dtype, max_rank=Rmax)
    err = check_close(from_device(y_got), delta, dtype, "delta")
    _log(f"  bitwise equal to the two-call path; error vs oracle {err:.2e}")


def test_route_linear_then_linear_other_module(rx):
    """The routing a fused call leaves behind serves the next module's lora_linear."""
    import torch
    W = small_case(41, T=200, S=16, k=1024, slices=[1024], Rmax=16, dtype="bf16", invalid=1)
    W2 = small_case(42, T=200, S=16, k=512, slices=[256, 256], Rmax=16, dtype="bf16")
    W2.ids = W.ids
    m1, m2 = W.modules[0], W2.modules[0]
    ids = _ids_tensor(W)
    outs = []
    for fused in (False, True):
        p1, p2 = make_pool(rx, W, m1), make_pool(rx, W2, m2)
        R = rx.Routing(0, W.T, W.S)
        y1 = to_device(m1.y_base, "bf16")
        y2 = to_device(m2.y_base, "bf16")
        if fused:
            rx.route_linear(p1, R, ids, to_device(m1.x, "bf16"), y1)
        else:
            R.build(ids)
            rx.linear(p1, R, to_device(m1.x, "bf16"), y1)
        rx.linear(p2, R, to_device(m2.x, "bf16"), y2)
        torch.cuda.synchronize()
        outs.append((bits(y1), bits(y2)))
        p1.close(); p2.close(); R.close()
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    ads = oracle_adapters(W2, m2)
    ref = O.lora_apply(to_f64(m2.x, "bf16"), to_f64(m2.y_base, "bf16"), ads, m2.slices, W.ids, W.S, "bf16",
                       max_rank=16)
    check_close(O.bf16_bits_to_f64(outs[1][1]), ref, "bf16", "second module")


def test_route_linear_no_lora_and_errors(rx):
    import torch
    W = small_case(43, T=50, S=4, k=256, slices=[128], Rmax=8, dtype="bf16")
    mod = W.modules[0]
    pool = make_pool(rx, W, mod)
    R = rx.Routing(0, W.T, W.S)
    x = to_device(mod.x, "bf16")
    y = to_device(mod.y_base, "bf16")
    none = torch.full((W.T,), -1, dtype=torch.int32, device="cuda")
    rx.route_linear(pool, R, none, x, y)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y), mod.y_base), "no-LoRA batch changed y"
    assert R.query()["num_active"] == 0
    lib = rx.lib
    ids = _ids_tensor(W)
    st = lib.lora_route_linear(pool.handle, R.handle, None, W.T, x.data_ptr(), x.stride(0), y.data_ptr(),
                               y.stride(0), rx.LORA_BF16, None)
    assert st == rx.LORA_ERR_INVALID_ARG
    st = lib.lora_route_linear(pool.handle, R.handle, ids.data_ptr(), W.T + 1, x.data_ptr(), x.stride(0),
                               y.data_ptr(), y.stride(0), rx.LORA_BF16, None)
    assert st == rx.LORA_ERR_CAPACITY
    R2 = rx.Routing(0, W.T, W.S + 1)
    st = lib.lora_route_linear(pool.handle, R2.handle, ids.data_ptr(), W.T, x.data_ptr(), x.stride(0),
                               y.data_ptr(), y.stride(0), rx.LORA_BF16, None)
    assert st == rx.LORA_ERR_SHAPE
    pool.close(); R.close(); R2.close()


@pytest.mark.parametrize("num", [2, 4])
def test_route_linear_full_size_matches_two_calls(rx, num):
    """At the full decode workloads (the launch shapes bench.py times: T = 64 and 8
    slots; T = 256, 64 slots and the packed QKV / gate_up / down modules), the fused
    call of the first module and the following lora_linear calls are bitwise equal to
    lora_build_routing + lora_linear (itself checked against the oracle on sampled
    rows at these sizes)."""
    import torch
    from synthetic import workload
    W = workload(num)
    _log(f"workload {num}: T={W.T} S={W.S} modules={[m.name for m in W.modules]}")
    ids = _ids_tensor(W)
    outs = []
    for fused in (False, True):
        pools = [make_pool(rx, W, m) for m in W.modules]
        R = rx.Routing(0, W.T, W.S)
        ys = []
        for i, (m, p) in enumerate(zip(W.modules, pools)):
            y = to_device(m.y_base if m.y_base is not None else np.zeros((W.T, sum(m.slices)), np.float32),
                          "bf16" if m.y_base is not None else "f32")
            x = to_device(m.x, W.dtype)
            if i == 0 and fused:
                rx.route_linear(p, R, ids, x, y)
            else:
                if i == 0:
                    R.build(ids)
                rx.linear(p, R, x, y)
            ys.append(y)
        torch.cuda.synchronize()
        outs.append([bits(y) for y in ys])
        for p in pools:
            p.close()
        R.close()
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
