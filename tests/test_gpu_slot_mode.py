"""Slot mode (both kernels slot-major: every segment on the matrix cores, the weight
fragments issued before any routing data has arrived) through the C ABI, against the
oracle and against the tile-list kernels.

Bars: the branch alone (base 0, fp32 output) and y on its base within the oracle
tolerances on every row; lora_route_linear (routing built inside the shrink launch)
bitwise equal to lora_build_routing + lora_linear; the allocation-free call and the
grouped calls bitwise equal to lora_linear; no-LoRA rows bitwise untouched.
"""
import os

import numpy as np
import pytest

import oracle.lora_oracle as O
from synthetic import small_case, workload

from lora_cases import bits, check_close, from_device, make_pool, make_routing, oracle_adapters, to_device, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rx():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import rank_adapter_gemm_build_amd as m
    return m


def _log(msg):
    print(msg, flush=True)


class _mode:
    """RAXLORA_SLOT_MODE for the calls made inside the block."""

    def __init__(self, value: str):
        self.value = value

    def __enter__(self):
        self.old = os.environ.get("RAXLORA_SLOT_MODE")
        os.environ["RAXLORA_SLOT_MODE"] = self.value

    def __exit__(self, *exc):
        if self.old is None:
            os.environ.pop("RAXLORA_SLOT_MODE", None)
        else:
            os.environ["RAXLORA_SLOT_MODE"] = self.old


CASES = [
    # seed, T, S, k, slices, Rmax, invalid, segments
    (801, 64, 8, 4096, [4096], 16, 0, None),                     # the decode workload's shape: 16 parts of 8 steps
    (802, 40, 5, 520, [136, 24], 9, 3, None),                    # ragged widths, 9 rows per slice, invalid ids
    (803, 0, 6, 8192, [1024], 24, 0, [1, 17, 29, 40, 3, 60]),    # parts of 16 steps; segments past one tile and
                                                                 # past the record's 28 token ids
    (804, 96, 12, 14336, [4096], 16, 0, None),                   # parts of 32 steps (the down projection's k)
    (805, 256, 64, 1024, [1024, 256, 256], 16, 4, None),         # packed slices, 256 tokens
    (806, 1, 1, 8, [8], 4, 0, None),                             # one token, k of one chunk
    (807, 0, 3, 2056, [200, 48], 64, 0, [200, 50]),              # one long segment, two rank steps
    (808, 80, 10, 16384, [512, 512], 96, 2, None),               # k at the slot-mode limit, three rank steps
]


def _ids(W):
    import torch
    return torch.from_numpy(np.ascontiguousarray(W.ids, dtype=np.int32)).cuda()


def _linear(rx, W, mod, y0, ydt, fused):
    import torch
    pool = make_pool(rx, W, mod)
    R = rx.Routing(0, max(W.T, 1), W.S)
    y = to_device(y0, ydt)
    if fused:
        rx.route_linear(pool, R, _ids(W), to_device(mod.x, W.dtype), y)
    else:
        R.build(_ids(W))
        rx.linear(pool, R, to_device(mod.x, W.dtype), y)
    torch.cuda.synchronize()
    pool.close(); R.close()
    return y


def _noalloc(rx, W, mod, y0):
    import torch
    pool = make_pool(rx, W, mod)
    R, _ = make_routing(rx, W)
    x = to_device(mod.x, W.dtype)
    y = to_device(y0, W.dtype)
    st = rx.lib.lora_linear_noalloc(pool.handle, R.handle, x.data_ptr(), x.stride(0), y.data_ptr(), y.stride(0),
                                    rx.LORA_BF16, None)
    assert st == 0, rx.lora_last_error()
    torch.cuda.synchronize()
    pool.close(); R.close()
    return y


@pytest.mark.parametrize("case", CASES, ids=[f"seed{c[0]}" for c in CASES])
def test_slot_mode_against_oracle(rx, case):
    seed, T, S, k, slices, Rmax, invalid, segments = case
    W = small_case(seed, T=T, S=S, k=k, slices=slices, Rmax=Rmax, invalid=invalid, segments=segments)
    mod = W.modules[0]
    D = sum(slices)
    _log(f"slot mode seed={seed} T={W.T} S={S} k={k} slices={slices} Rmax={Rmax} ranks={sorted(W.ranks.values())}")
    zero = np.zeros((W.T, D), dtype=np.float32)
    with _mode("1"):
        d_two = _linear(rx, W, mod, zero, "f32", fused=False)
        d_fused = _linear(rx, W, mod, zero, "f32", fused=True)
        y_two = _linear(rx, W, mod, mod.y_base, "bf16", fused=False)
        y_fused = _linear(rx, W, mod, mod.y_base, "bf16", fused=True)
        y_na = _noalloc(rx, W, mod, mod.y_base)
    with _mode("0"):
        d_tiles = _linear(rx, W, mod, zero, "f32", fused=False)
    assert np.array_equal(bits(d_fused), bits(d_two)), "route_linear differs from build_routing + linear"
    assert np.array_equal(bits(y_fused), bits(y_two)), "route_linear differs from build_routing + linear (y)"
    assert np.array_equal(bits(y_na), bits(y_two)), "lora_linear_noalloc differs from lora_linear"
    ads = oracle_adapters(W, mod)
    x64 = to_f64(mod.x, "bf16")
    delta = O.lora_apply(x64, np.zeros((W.T, D)), ads, slices, W.ids, S, "bf16", max_rank=Rmax)
    err = check_close(from_device(d_two), delta, "bf16", f"slot-mode delta seed={seed}")
    err_t = check_close(from_device(d_tiles), delta, "bf16", f"tile-list delta seed={seed}")
    ref = O.lora_apply(x64, to_f64(mod.y_base, "bf16"), ads, slices, W.ids, S, "bf16", max_rank=Rmax)
    check_close(from_device(y_two), ref, "bf16", f"slot-mode y seed={seed}")
    untouched = (W.ids < 0) | (W.ids >= S)
    assert np.array_equal(bits(y_two)[untouched], mod.y_base[untouched])
    _log(f"  delta error: slot mode {err:.2e}, tile lists {err_t:.2e}")


def test_slot_mode_noalloc_without_first_tile_rows(rx):
    """A slot-mode call whose partial sums fit the allocation-free call's array only
    without the first-tile rows (k = 32768: 16 parts, 3 slices, ranks padded to 256,
    256 tokens over 8 slots): that call keeps every row by sorted position and is
    still bitwise equal to lora_linear, whose pool workspace has the first-tile rows."""
    import torch
    W = small_case(831, T=256, S=8, k=32768, slices=[64, 64, 64], Rmax=256, ranks={0: 4, 3: 7, 6: 1})
    mod = W.modules[0]
    zero = np.zeros((W.T, sum(mod.slices)), dtype=np.float32)
    _log(f"slot mode, allocation-free call past its first-tile rows: T={W.T} S={W.S} k={mod.k}")
    with _mode("1"):
        d_lin = _linear(rx, W, mod, zero, "f32", fused=False)
        pool = make_pool(rx, W, mod)
        R, _ = make_routing(rx, W)
        x = to_device(mod.x, W.dtype)
        d_na = to_device(zero, "f32")
        st = rx.lib.lora_linear_noalloc(pool.handle, R.handle, x.data_ptr(), x.stride(0), d_na.data_ptr(),
                                        d_na.stride(0), rx.LORA_F32, None)
        assert st == 0, rx.lora_last_error()
        torch.cuda.synchronize()
        pool.close(); R.close()
    assert np.array_equal(bits(d_na), bits(d_lin))
    delta = O.lora_apply(to_f64(mod.x, "bf16"), np.zeros(zero.shape), oracle_adapters(W, mod), mod.slices, W.ids, W.S,
                         "bf16", max_rank=W.Rmax)
    check_close(from_device(d_lin), delta, "bf16", "slot-mode delta, k = 32768, three slices")


def test_slot_mode_untouched_rows_and_columns(rx):
    """No-LoRA rows, an empty slot, a zero-scale slot and a missing slice stay
    bit-identical in slot mode."""
    import torch
    W = small_case(811, T=120, S=6, k=512, slices=[64, 128, 32], Rmax=8, invalid=4)
    mod = W.modules[0]
    mod.A[2][1] = None; mod.B[2][1] = None           # slot 2: slice 1 missing
    with _mode("1"):
        pool = make_pool(rx, W, mod)
        pool.unregister(3)                             # slot 3 empty
        pool.register(4, mod.A[4], mod.B[4], W.alpha[4], W.ranks[4], adapter_scale=0.0)   # slot 4 scale 0
        R, ids = make_routing(rx, W)
        y = to_device(mod.y_base, "bf16")
        rx.linear(pool, R, to_device(mod.x, "bf16"), y)
        torch.cuda.synchronize()
    got, base = bits(y), mod.y_base
    keys = np.where((W.ids >= 0) & (W.ids < W.S), W.ids, W.S)
    for key in (W.S, 3, 4):
        rows = keys == key
        assert np.array_equal(got[rows], base[rows]), key
    rows = keys == 2
    assert np.array_equal(got[rows][:, 64:192], base[rows][:, 64:192])
    assert not np.array_equal(got[rows][:, :64], base[rows][:, :64])
    ranks = dict(W.ranks)
    ranks.pop(3)
    ads = oracle_adapters(W, mod, ranks=ranks)
    ads[4] = O.Adapter(rank=ads[4].rank, A=ads[4].A, B=ads[4].B, alpha=ads[4].alpha, rslora=False, adapter_scale=0.0)
    ref = O.lora_apply(to_f64(mod.x, "bf16"), to_f64(mod.y_base, "bf16"), ads, mod.slices, W.ids, W.S, "bf16",
                       max_rank=W.Rmax)
    check_close(from_device(y), ref, "bf16", "slot-mode y with missing slice, empty and zero-scale slots")
    pool.close(); R.close()


def test_slot_mode_group_equals_per_module(rx):
    """A grouped call in slot mode (every module eligible) is bitwise equal to its
    per-module calls, with the routing built inside the grouped shrink and before it."""
    import torch
    T, S = 160, 24
    W = small_case(821, T=T, S=S, k=1024, slices=[1024, 256, 256], Rmax=16, invalid=2)
    W2 = small_case(822, T=T, S=S, k=1024, slices=[1536, 1536], Rmax=16, ranks=dict(W.ranks))
    W3 = small_case(823, T=T, S=S, k=3072, slices=[1024], Rmax=16, ranks=dict(W.ranks))
    W2.ids = W.ids; W3.ids = W.ids
    mods = [W.modules[0], W2.modules[0], W3.modules[0]]
    with _mode("1"):
        pools = [make_pool(rx, w, m) for w, m in zip((W, W2, W3), mods)]
        ids = _ids(W)
        xs = [to_device(m.x, "bf16") for m in mods]
        outs = {}
        for form in ("per-module", "group", "group-built"):
            R = rx.Routing(0, T, S)
            ys = [torch.zeros((T, sum(m.slices)), dtype=torch.float32, device="cuda") for m in mods]
            if form == "per-module":
                R.build(ids)
                for p, x, y in zip(pools, xs, ys):
                    rx.linear(p, R, x, y)
            elif form == "group":
                rx.route_linear_group(pools, R, ids, xs, ys)
            else:
                R.build(ids)
                rx.linear_group(pools, R, xs, ys)
            torch.cuda.synchronize()
            outs[form] = [bits(y) for y in ys]
            if form == "per-module":
                ref_ys = [from_device(y) for y in ys]
            R.close()
    for form in ("group", "group-built"):
        for i, (a, b) in enumerate(zip(outs["per-module"], outs[form])):
            assert np.array_equal(a, b), f"{form}: module {i} differs from its own call"
    for w, m, got in zip((W, W2, W3), mods, ref_ys):
        ref = O.lora_apply(to_f64(m.x, "bf16"), np.zeros((T, sum(m.slices))), oracle_adapters(w, m), m.slices,
                           W.ids, S, "bf16", max_rank=16)
        check_close(got, ref, "bf16", f"slot-mode group module k={m.k} slices={m.slices}")
    for p in pools:
        p.close()


@pytest.mark.parametrize("num,mode", [(2, "0"), (4, "1")])
def test_workloads_in_the_other_mode(rx, num, mode):
    """Full-size workloads in the mode they do not take by default: the decode
    workload (slot mode by default) through the tile-list kernels, the packed
    three-module workload (tile lists by default) in slot mode; the branch alone on
    every row of every module against the oracle's grouped formulation."""
    import torch
    W = workload(num)
    with _mode(mode):
        R, ids = make_routing(rx, W)
        for mod in W.modules:
            _log(f"workload {num} module {mod.name} (RAXLORA_SLOT_MODE={mode})")
            pool = make_pool(rx, W, mod)
            d0 = torch.zeros((W.T, sum(mod.slices)), dtype=torch.float32, device="cuda")
            rx.linear(pool, R, to_device(mod.x, W.dtype), d0)
            torch.cuda.synchronize()
            ref0 = O.lora_apply_grouped(to_f64(mod.x, W.dtype), np.zeros(tuple(d0.shape)), oracle_adapters(W, mod),
                                        mod.slices, W.ids, W.S, W.dtype)
            check_close(d0.double().cpu().numpy(), ref0, W.dtype,
                        f"workload {num} {mod.name} delta (RAXLORA_SLOT_MODE={mode})")
            pool.close()
        R.close()
