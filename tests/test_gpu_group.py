"""Grouped calls (lora_linear_group / lora_route_linear_group: several target modules
of one batch in one shrink and one expand launch) against the per-module calls and
the oracle, through the C ABI.

Bars: y of every module bitwise identical to lora_linear on that module alone (the
grouped launch runs each module's units as its own launch would); the routing
outputs bit-exact; the branch alone within the oracle tolerances on every row.
"""
import os

import numpy as np
import pytest

import oracle.lora_oracle as O
from synthetic import small_case, workload

from lora_cases import bits, check_close, make_pool, oracle_adapters, to_device, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rx():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import rank_adapter_gemm_build_amd as m
    return m


def _log(msg):
    print(msg, flush=True)


def _ids(W):
    import torch
    return torch.from_numpy(np.ascontiguousarray(W.ids, dtype=np.int32)).cuda()


def _module_outputs(W, zero_base):
    """Per module the starting y: the drawn base (storage dtype), or zeros in fp32."""
    out = []
    for m in W.modules:
        if zero_base or m.y_base is None:
            out.append((np.zeros((W.T, sum(m.slices)), np.float32), "f32"))
        else:
            out.append((m.y_base, W.dtype))
    return out


def _run(rx, W, pools, mode, zero_base):
    """y of every module after one step in `mode`: 'per-module' (route_linear on the
    first module, linear on the others), 'group' (route_linear_group), or 'group-built'
    (build, then linear_group)."""
    import torch
    ids = _ids(W)
    R = rx.Routing(0, W.T, W.S)
    xs = [to_device(m.x, W.dtype) for m in W.modules]
    ys = [to_device(a, dt) for a, dt in _module_outputs(W, zero_base)]
    if mode == "per-module":
        for i, (p, x, y) in enumerate(zip(pools, xs, ys)):
            if i == 0:
                rx.route_linear(p, R, ids, x, y)
            else:
                rx.linear(p, R, x, y)
    elif mode == "group":
        rx.route_linear_group(pools, R, ids, xs, ys)
    else:
        R.build(ids)
        rx.linear_group(pools, R, xs, ys)
    torch.cuda.synchronize()
    q = R.query()
    R.close()
    return [bits(y) for y in ys], [y for y in ys], q


def _group_case(seed, T, S, Rmax, dtype, mods, invalid=2, segments=None, rslora=False):
    """A batch with several modules (k, slices) sharing its ids and slots."""
    base = small_case(seed, T=T, S=S, k=mods[0][0], slices=mods[0][1], Rmax=Rmax, dtype=dtype, invalid=invalid,
                      segments=segments, rslora=rslora)
    for i, (k, slices) in enumerate(mods[1:]):
        other = small_case(seed + 100 * (i + 1), T=base.T, S=S, k=k, slices=slices, Rmax=Rmax, dtype=dtype,
                           ranks=base.ranks)
        m = other.modules[0]
        m.name = f"m{i + 1}"
        base.modules.append(m)
    return base


GROUP_CASES = [
    # seed, T, S, Rmax, dtype, modules (k, slices), segments
    (61, 64, 8, 16, "bf16", [(4096, [4096]), (4096, [1024, 1024]), (1024, [512])], None),       # decode, self-routed
    (62, 200, 40, 32, "bf16", [(520, [136, 24]), (264, [64]), (1032, [520, 264])], None),        # ragged, mixed k
    (63, 0, 6, 64, "bf16", [(1032, [520]), (512, [1024, 256])], [1, 2, 3, 4, 17, 40, 90, 99]),   # long segments
    (64, 300, 9, 24, "bf16", [(1024, [1024, 512]), (2048, [256])], None),                        # routing launch first
    (65, 45, 6, 9, "f32", [(264, [40, 8, 16]), (136, [24])], None),                               # fp32: vector units
    (66, 256, 255, 16, "bf16", [(512, [512]), (512, [256]), (256, [128]), (128, [128]), (128, [64]),
                                (64, [64]), (64, [32]), (32, [32])], None),                       # 8 modules, 255 slots
]


@pytest.mark.parametrize("mode", ["default", "tiles", "slot", "all-mfma", "vector"])
@pytest.mark.parametrize("case", GROUP_CASES, ids=[f"seed{c[0]}" for c in GROUP_CASES])
def test_group_matches_per_module_calls(rx, case, mode):
    seed, T, S, Rmax, dtype, mods, segments = case
    W = _group_case(seed, T, S, Rmax, dtype, mods, segments=segments)
    _log(f"group seed={seed} T={W.T} S={S} modules={[(m.k, m.slices) for m in W.modules]} {dtype} mode={mode}")
    env = {"tiles": {"RAXLORA_SLOT_MODE": "0"}, "slot": {"RAXLORA_SLOT_MODE": "1"},
           "all-mfma": {"RAXLORA_MFMA_MIN_SEG": "1", "RAXLORA_SLOT_MODE": "0"},
           "vector": {"RAXLORA_DISABLE_MFMA": "1"}}.get(mode, {})
    os.environ.update(env)
    try:
        pools = [make_pool(rx, W, m) for m in W.modules]
        ref_bits, _, q_ref = _run(rx, W, pools, "per-module", False)
        for form in ("group", "group-built"):
            got_bits, _, q = _run(rx, W, pools, form, False)
            for i, (a, b) in enumerate(zip(ref_bits, got_bits)):
                assert np.array_equal(a, b), f"{form}: module {i} differs from its own call"
            for key in ("counts", "seg_offsets", "sorted_ids", "active_slots"):
                assert np.array_equal(q[key], q_ref[key]), key
        # the branch alone against the oracle, every row of every module
        _, ys, _ = _run(rx, W, pools, "group", True)
        for m, y in zip(W.modules, ys):
            ref = O.lora_apply(to_f64(m.x, dtype), np.zeros((W.T, sum(m.slices))), oracle_adapters(W, m), m.slices,
                               W.ids, W.S, dtype, max_rank=W.Rmax)
            check_close(y.double().cpu().numpy(), ref, dtype, f"group seed={seed} {m.name} delta ({mode})")
        for p in pools:
            p.close()
    finally:
        for key in env:
            os.environ.pop(key, None)


@pytest.mark.parametrize("num", [4, 5])
def test_group_full_workloads(rx, num):
    """The multi-module workloads at full size in one grouped step (workload 4: 256
    tokens, the routing inside the grouped shrink; workload 5: 1024 tokens, the routing
    launch first): bitwise equal to the per-module calls, the branch alone within the
    tolerance of the oracle's grouped formulation on every row."""
    W = workload(num)
    _log(f"group workload {num}: T={W.T} S={W.S} modules={[m.name for m in W.modules]}")
    pools = [make_pool(rx, W, m) for m in W.modules]
    ref_bits, _, _ = _run(rx, W, pools, "per-module", False)
    got_bits, _, _ = _run(rx, W, pools, "group", False)
    for m, a, b in zip(W.modules, ref_bits, got_bits):
        assert np.array_equal(a, b), f"module {m.name} differs from its own call"
    _, ys, _ = _run(rx, W, pools, "group", True)
    for m, y in zip(W.modules, ys):
        ref = O.lora_apply_grouped(to_f64(m.x, W.dtype), np.zeros((W.T, sum(m.slices))), oracle_adapters(W, m),
                                   m.slices, W.ids, W.S, W.dtype)
        check_close(y.double().cpu().numpy(), ref, W.dtype, f"group workload {num} {m.name} delta, all rows")
    for p in pools:
        p.close()


def test_group_fp8_matches_per_module_calls(rx):
    """FP8 pools in one grouped step equal their per-module calls bitwise."""
    import torch
    W = _group_case(67, 96, 12, 32, "bf16", [(1024, [1024]), (2048, [512, 256])])
    _log("group FP8")
    pools = []
    for m in W.modules:
        p = rx.Pool(0, W.S, W.Rmax, m.k, m.slices, rx.LORA_FP8E4M3, W.T)
        for s, r in W.ranks.items():
            conv = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).float().clamp(-448, 448) \
                .to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            p.register(s, [conv(a) for a in m.A[s]], [conv(b) for b in m.B[s]], W.alpha[s], r)
        pools.append(p)
    ref_bits, _, _ = _run(rx, W, pools, "per-module", False)
    got_bits, _, _ = _run(rx, W, pools, "group", False)
    for a, b in zip(ref_bits, got_bits):
        assert np.array_equal(a, b)
    for p in pools:
        p.close()


def test_group_errors(rx):
    import torch
    W = _group_case(68, 16, 4, 8, "bf16", [(64, [32]), (64, [32])])
    pools = [make_pool(rx, W, m) for m in W.modules]
    R = rx.Routing(0, 16, 4)
    R.build(_ids(W))
    xs = [to_device(m.x, "bf16") for m in W.modules]
    ys = [to_device(m.y_base, "bf16") for m in W.modules]
    with pytest.raises(rx.LoraError) as e:
        rx.linear_group([pools[0], pools[0]], R, xs, ys)            # a pool twice: one workspace
    assert e.value.status == rx.LORA_ERR_INVALID_ARG
    other = rx.Pool(0, 5, 8, 64, [32], rx.LORA_BF16, 16)
    with pytest.raises(rx.LoraError) as e:
        rx.linear_group([pools[0], other], R, xs, ys)               # slot count differs
    assert e.value.status == rx.LORA_ERR_SHAPE
    wide = rx.Pool(0, 4, 40, 64, [32], rx.LORA_BF16, 16)
    with pytest.raises(rx.LoraError) as e:
        rx.linear_group([pools[0], wide], R, xs, ys)                # rank padding 32 vs 64
    assert e.value.status == rx.LORA_ERR_SHAPE
    f32 = rx.Pool(0, 4, 8, 64, [32], rx.LORA_F32, 16)
    with pytest.raises((rx.LoraError, TypeError)):
        rx.linear_group([pools[0], f32], R, xs, ys)                 # weight dtype differs
    lib = rx.lib
    import ctypes as C
    P = (C.c_void_p * 9)(*([pools[0].handle] * 9))
    X = (C.c_void_p * 9)(*([xs[0].data_ptr()] * 9))
    L = (C.c_int * 9)(*([64] * 9))
    Y = (C.c_void_p * 9)(*([ys[0].data_ptr()] * 9))
    LY = (C.c_int * 9)(*([32] * 9))
    assert lib.lora_linear_group(P, 9, R.handle, X, L, Y, LY, rx.LORA_BF16, None) == rx.LORA_ERR_SHAPE
    assert lib.lora_linear_group(P, 0, R.handle, X, L, Y, LY, rx.LORA_BF16, None) == rx.LORA_ERR_SHAPE
    assert lib.lora_linear_group(None, 1, R.handle, X, L, Y, LY, rx.LORA_BF16, None) == rx.LORA_ERR_INVALID_ARG
    torch.cuda.synchronize()
    for p in pools + [other, wide, f32]:
        p.close()
    R.close()
