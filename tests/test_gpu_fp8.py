"""FP8 (e4m3) adapter pools against the oracle's FP8 path, through the C ABI.

Bars: registration bit-exact (stored bytes, and the scale fold against the
oracle's fold); an exact-integer case bit-exact; random cases within the bf16
tolerance (normwise relative error <= 2e-2 on the delta and on y) against the
float64 definition on the clamped-and-rounded activations; the fused
route-and-apply call bitwise equal to routing + lora_linear.  Inputs are drawn
with numpy and put on the e4m3 grid by torch's float8_e4m3fn conversion.
"""
import numpy as np
import pytest

import oracle.lora_oracle as O

from lora_cases import bits, check_close, from_device, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rx():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert hasattr(torch, "float8_e4m3fn")
    import rank_adapter_gemm_build_amd as m
    return m


def _log(msg):
    print(msg, flush=True)


def _fp8_bytes(vals):
    """e4m3 bit patterns of float values (clamped to the finite range) by torch."""
    import torch
    v = np.clip(np.asarray(vals, dtype=np.float64), -448.0, 448.0)
    return torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _bf16(a):
    return O.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def _case(seed, T, S, k, slices, Rmax, integer=False, big_x=True):
    rng = np.random.default_rng(seed)
    ranks = {s: int(rng.choice([r for r in (1, 2, 4, 8, 16, 32, 64) if r <= Rmax])) for s in range(S) if s != 1}
    A, B = {}, {}
    for s, r in ranks.items():
        if integer:
            A[s] = [_fp8_bytes(rng.integers(-2, 3, size=(r, k))) for _ in slices]
            B[s] = [_fp8_bytes(rng.integers(-2, 3, size=(d, r))) for d in slices]
        else:
            A[s] = [_fp8_bytes(rng.standard_normal((r, k)) * 0.5) for _ in slices]
            B[s] = [_fp8_bytes(rng.standard_normal((d, r)) / np.sqrt(r)) for d in slices]
    ids = rng.integers(0, S, size=T).astype(np.int32)
    ids[rng.random(T) < 0.1] = -1
    if T > 3:
        ids[:2] = [S + 2, -5]                      # invalid ids: no LoRA
    if integer:
        x = _bf16(rng.integers(-4, 5, size=(T, k)))
    else:
        xv = rng.standard_normal((T, k)) * 8.0
        if big_x:                                  # past the FP8 range: clamped to +-448
            xv.flat[rng.choice(xv.size, size=min(40, xv.size), replace=False)] = rng.choice([-1000.0, 460.0, 600.0, -449.0], 40)
            xv.flat[rng.choice(xv.size, size=min(40, xv.size), replace=False)] = rng.standard_normal(40) * 1e-3
        x = _bf16(xv)
    alpha = {s: float(2 * r) for s, r in ranks.items()}   # scale 2: exact folds
    return ranks, A, B, ids, x, alpha


def _pool(rx, S, Rmax, k, slices, T, ranks, A, B, alpha, premultiply=False, rslora=False):
    pool = rx.Pool(0, S, Rmax, k, slices, rx.LORA_FP8E4M3, T)
    for s, r in ranks.items():
        pool.register(s, A[s], B[s], alpha[s], r, rslora, premultiply=premultiply)
    return pool


def _oracle(ranks, A, B, ids, x, alpha, S, slices, Rmax, y_base, premultiply=False, rslora=False):
    ads = {s: O.Adapter(rank=r, A=[O.fp8_e4m3_decode(a) for a in A[s]], B=[O.fp8_e4m3_decode(b) for b in B[s]],
                        alpha=alpha[s], rslora=rslora, premultiply=premultiply) for s, r in ranks.items()}
    return O.lora_apply_fp8(O.bf16_bits_to_f64(x), y_base, ads, slices, ids, S, max_rank=Rmax)


def _run(rx, pool, ids, x, y0, ydt):
    import torch
    R = rx.Routing(0, len(ids), pool.S)
    R.build(torch.from_numpy(ids).cuda())
    y = to_device(y0, ydt)
    rx.linear(pool, R, to_device(x, "bf16"), y)
    torch.cuda.synchronize()
    R.close()
    return y


@pytest.mark.parametrize("premultiply,rslora", [(False, False), (True, False), (True, True)])
def test_fp8_registration_bit_exact(rx, premultiply, rslora):
    k, slices, Rmax, S = 264, [40, 16], 16, 3
    ranks, A, B, ids, x, alpha = _case(3, 8, S, k, slices, Rmax)
    pool = _pool(rx, S, Rmax, k, slices, 8, ranks, A, B, alpha, premultiply, rslora)
    for s, r in ranks.items():
        sc = O.lora_scale(alpha[s], r, rslora)
        for n, d in enumerate(slices):
            Ag, Bt = pool.read_slot(s, n)
            assert np.array_equal(Ag[:r], A[s][n]) and not Ag[r:].any()
            want = O.fp8_fold_scale(O.fp8_e4m3_decode(B[s][n]), sc) if premultiply else O.fp8_e4m3_decode(B[s][n])
            got = O.fp8_e4m3_decode(Bt[:r].T)
            assert np.array_equal(got, want), (s, n)
            assert not Bt[r:].any()
    pool.close()


@pytest.mark.parametrize("mode", ["default", "tiles", "slot", "vector", "all-mfma"])
def test_fp8_exact_integer_case(rx, mode):
    """Small integers everywhere: every product and partial sum is exact in fp32, so
    the fp32 output equals the definition exactly, on the vector units, the matrix
    cores and the default split between them."""
    import os
    T, S, k, slices, Rmax = 70, 5, 512, [256, 64], 40
    ranks, A, B, ids, x, alpha = _case(11, T, S, k, slices, Rmax, integer=True)
    env = {"tiles": {"RAXLORA_SLOT_MODE": "0"}, "slot": {"RAXLORA_SLOT_MODE": "1"},
           "vector": {"RAXLORA_DISABLE_MFMA": "1"},
           "all-mfma": {"RAXLORA_MFMA_MIN_SEG": "1", "RAXLORA_SLOT_MODE": "0"}}.get(mode, {})
    os.environ.update(env)
    try:
        pool = _pool(rx, S, Rmax, k, slices, T, ranks, A, B, alpha)
        D = sum(slices)
        y = _run(rx, pool, ids, x, np.zeros((T, D), dtype=np.float32), "f32")
    finally:
        for key in env:
            os.environ.pop(key, None)
    ref = _oracle(ranks, A, B, ids, x, alpha, S, slices, Rmax, np.zeros((T, D)))
    assert np.array_equal(from_device(y), ref)
    pool.close()


@pytest.mark.parametrize("mode", ["default", "slot", "vector"])
def test_fp8_every_bf16_activation_converts_exactly(rx, mode):
    """Every bf16 bit pattern of x but the NaNs (set to 0) through the activation
    conversion: with A and B one-hot (token t's rank-space value j is its x column j)
    and scale 1, the fp32 branch of token t column d is e4m3(clamp(x[t][d])) exactly,
    on the matrix cores (tile lists and slot mode) and on the vector units; +-inf and
    everything past +-448 give +-448."""
    import os
    T, k, r = 256, 256, 256
    pat = np.arange(T * k, dtype=np.uint32).astype(np.uint16).reshape(T, k)
    f = (pat.astype(np.uint32) << 16).view(np.float32)
    x = np.where(np.isnan(f), np.uint16(0), pat).astype(np.uint16)
    eye = np.eye(r, dtype=np.float64)
    A = {0: [_fp8_bytes(eye)]}
    B = {0: [_fp8_bytes(eye)]}
    ranks, alpha, ids = {0: r}, {0: float(r)}, np.zeros(T, dtype=np.int32)
    env = {"slot": {"RAXLORA_SLOT_MODE": "1"}, "vector": {"RAXLORA_DISABLE_MFMA": "1"}}.get(mode, {})
    os.environ.update(env)
    try:
        pool = _pool(rx, 1, r, k, [k], T, ranks, A, B, alpha)
        y = _run(rx, pool, ids, x, np.zeros((T, k), dtype=np.float32), "f32")
    finally:
        for key in env:
            os.environ.pop(key, None)
    ref = _oracle(ranks, A, B, ids, x, alpha, 1, [k], r, np.zeros((T, k)))
    got = from_device(y)
    assert np.array_equal(got, ref)
    xf = O.bf16_bits_to_f64(x)
    assert np.array_equal(got, O.fp8_quantize(xf))                       # the conversion alone
    assert np.all(got[np.isinf(xf)] == np.sign(xf[np.isinf(xf)]) * 448.0)
    pool.close()


@pytest.mark.parametrize("seed,T,S,k,slices,Rmax,premultiply", [
    (21, 37, 5, 520, [136, 24], 16, False),
    (22, 64, 8, 4096, [4096], 16, False),
    (23, 130, 4, 2056, [1544], 64, True),
    (24, 300, 9, 1024, [1024, 512], 32, False),
    (25, 256, 64, 4096, [4096, 1024, 1024], 16, True),
])
def test_fp8_matches_oracle(rx, seed, T, S, k, slices, Rmax, premultiply):
    _log(f"fp8 seed={seed} T={T} S={S} k={k} slices={slices} Rmax={Rmax} pre={premultiply}")
    ranks, A, B, ids, x, alpha = _case(seed, T, S, k, slices, Rmax)
    pool = _pool(rx, S, Rmax, k, slices, T, ranks, A, B, alpha, premultiply)
    D = sum(slices)
    y = _run(rx, pool, ids, x, np.zeros((T, D), dtype=np.float32), "f32")
    ref = _oracle(ranks, A, B, ids, x, alpha, S, slices, Rmax, np.zeros((T, D)), premultiply)
    err = check_close(from_device(y), ref, "bf16", "delta")
    yb = _bf16(np.random.default_rng(seed).standard_normal((T, D)))
    y2 = _run(rx, pool, ids, x, yb, "bf16")
    ref2 = _oracle(ranks, A, B, ids, x, alpha, S, slices, Rmax, O.bf16_bits_to_f64(yb), premultiply)
    check_close(from_device(y2), ref2, "bf16", "y")
    keys = np.where((ids >= 0) & (ids < S), ids, S)
    assert np.array_equal(bits(y2)[keys == S], yb[keys == S])
    _log(f"  normwise rel err {err:.2e}")
    pool.close()


def test_fp8_route_linear_matches_two_calls(rx):
    import torch
    T, S, k, slices, Rmax = 200, 16, 1024, [512, 512], 16
    ranks, A, B, ids, x, alpha = _case(31, T, S, k, slices, Rmax)
    pool = _pool(rx, S, Rmax, k, slices, T, ranks, A, B, alpha)
    yb = _bf16(np.random.default_rng(31).standard_normal((T, sum(slices))))
    y1 = _run(rx, pool, ids, x, yb, "bf16")
    R = rx.Routing(0, T, S)
    y2 = to_device(yb, "bf16")
    rx.route_linear(pool, R, torch.from_numpy(ids).cuda(), to_device(x, "bf16"), y2)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y1), bits(y2))
    pool.close(); R.close()


@pytest.mark.parametrize("num", [2, 4])
def test_fp8_full_workload_sampled_rows(rx, num):
    """The decode workloads at full size with every A and B put on the e4m3 grid (as
    the bench's FP8 measurement does), in the launch configuration it times (fused
    call for the first module); sampled rows against the oracle's FP8 path."""
    import torch
    from synthetic import workload
    W = workload(num)
    rng = np.random.default_rng(900 + num)
    ids = torch.from_numpy(np.ascontiguousarray(W.ids, dtype=np.int32)).cuda()
    R = rx.Routing(0, W.T, W.S)
    keys = np.where((W.ids >= 0) & (W.ids < W.S), W.ids, W.S)
    rows = np.array(sorted(set(rng.choice(W.T, size=min(40, W.T), replace=False).tolist())
                           | set(np.nonzero(keys == keys[0])[0].tolist())))
    for i, mod in enumerate(W.modules):
        _log(f"fp8 workload {num} module {mod.name} k={mod.k} slices={mod.slices}")
        A = {s: [_fp8_bytes(O.bf16_bits_to_f64(a)) for a in mod.A[s]] for s in W.ranks}
        B = {s: [_fp8_bytes(O.bf16_bits_to_f64(b)) for b in mod.B[s]] for s in W.ranks}
        pool = rx.Pool(0, W.S, W.Rmax, mod.k, mod.slices, rx.LORA_FP8E4M3, W.T)
        for s, r in W.ranks.items():
            pool.register(s, A[s], B[s], W.alpha[s], r, W.rslora, W.adapter_scale)
        yb = mod.y_base if mod.y_base is not None else _bf16(rng.standard_normal((W.T, sum(mod.slices))))
        y = to_device(yb, "bf16")
        if i == 0:
            rx.route_linear(pool, R, ids, to_device(mod.x, "bf16"), y)
        else:
            rx.linear(pool, R, to_device(mod.x, "bf16"), y)
        torch.cuda.synchronize()
        ads = {s: O.Adapter(rank=r, A=[O.fp8_e4m3_decode(a) for a in A[s]], B=[O.fp8_e4m3_decode(b) for b in B[s]],
                            alpha=W.alpha[s], rslora=W.rslora, adapter_scale=W.adapter_scale)
               for s, r in W.ranks.items()}
        ref = O.lora_apply_fp8(O.bf16_bits_to_f64(mod.x)[rows], O.bf16_bits_to_f64(yb)[rows], ads, mod.slices,
                               W.ids[rows], W.S, max_rank=W.Rmax)
        check_close(from_device(y)[rows], ref, "bf16", f"fp8 workload {num} {mod.name}")
        pool.close()
    R.close()
