"""The LoRA call joined to a base projection on another stream, and the decode step
captured in a HIP graph (torch.cuda.CUDAGraph), through the C ABI.

Bars: every result bitwise equal to the plain single-stream eager calls on the same
inputs (same kernels, same arithmetic) and within the bf16 tolerance of the CPU
oracle; graph replays checked one by one, with eager work between them.
"""
import numpy as np
import pytest

import oracle.lora_oracle as O
from synthetic import small_case, workload

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


def _ids(W):
    import torch
    return torch.from_numpy(np.ascontiguousarray(W.ids, dtype=np.int32)).cuda()


# T <= 256 takes the routing inside the shrink launch; 300 the separate routing launch
@pytest.mark.parametrize("T", [64, 300])
@pytest.mark.parametrize("prebuilt", [False, True])
def test_join_waits_for_the_base_output(rx, T, prebuilt):
    """The base stream is held back (a 1 ms spin) before it writes y; the LoRA stream's
    expand must still see that write: y ends as base + LoRA, bitwise the serial result."""
    import torch
    W = small_case(51, T=T, S=8, k=1024, slices=[512, 256], Rmax=16, dtype="bf16", invalid=2)
    mod = W.modules[0]
    _log(f"join T={T} prebuilt={prebuilt}")
    pool = make_pool(rx, W, mod)
    x = to_device(mod.x, "bf16")
    ybase = to_device(mod.y_base, "bf16")
    ids = _ids(W)
    # serial reference: base written, then the plain call
    R0 = rx.Routing(0, T, W.S)
    y_ref = ybase.clone()
    rx.route_linear(pool, R0, ids, x, y_ref)
    torch.cuda.synchronize()
    # joined: base output written late on stream A, LoRA on stream B
    R = rx.Routing(0, T, W.S)
    if prebuilt:
        R.build(ids)
        torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    y = torch.zeros_like(ybase)
    torch.cuda.synchronize()
    ready = torch.cuda.Event()
    with torch.cuda.stream(sa):
        torch.cuda._sleep(2_000_000)
        y.copy_(ybase)
        ready.record(sa)
    rx.linear_join(pool, R, x, y, ready, stream=sb, ids=None if prebuilt else ids)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y), bits(y_ref)), "joined result differs from the serial one"
    ref = O.lora_apply(to_f64(mod.x, "bf16"), to_f64(mod.y_base, "bf16"), oracle_adapters(W, mod), mod.slices,
                       W.ids, W.S, "bf16", max_rank=W.Rmax)
    check_close(from_device(y), ref, "bf16", f"joined call T={T} vs oracle")
    # without an event: the plain call
    y2 = ybase.clone()
    torch.cuda.synchronize()
    rx.linear_join(pool, R, x, y2, None, ids=None if prebuilt else ids)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y2), bits(y_ref))
    pool.close(); R.close(); R0.close()


@pytest.mark.parametrize("fused", [True, False])
def test_graph_capture_replays(rx, fused):
    """Routing + two modules captured once, replayed 4 times; between replays the same
    pools and routing object serve an eager call on another batch, so each replay
    must rebuild the routing it reads."""
    import torch
    W = small_case(52, T=96, S=12, k=1024, slices=[1024], Rmax=16, dtype="bf16", invalid=1)
    W2 = small_case(53, T=96, S=12, k=512, slices=[512, 256], Rmax=16, dtype="bf16")
    other = small_case(54, T=80, S=12, k=1024, slices=[1024], Rmax=16, dtype="bf16")
    m1, m2 = W.modules[0], W2.modules[0]
    p1, p2 = make_pool(rx, W, m1), make_pool(rx, W2, m2)
    x1, x2 = to_device(m1.x, "bf16"), to_device(m2.x, "bf16")
    yb1, yb2 = to_device(m1.y_base, "bf16"), to_device(m2.y_base, "bf16")
    ids = _ids(W)
    R = rx.Routing(0, 128, W.S)
    _log(f"graph fused={fused}")

    def step(y1, y2):
        if fused:
            rx.route_linear(p1, R, ids, x1, y1)
        else:
            R.build(ids)
            rx.linear(p1, R, x1, y1)
        rx.linear(p2, R, x2, y2)

    # eager reference, itself checked against the oracle
    r1, r2 = yb1.clone(), yb2.clone()
    step(r1, r2)
    torch.cuda.synchronize()
    ref1, ref2 = bits(r1), bits(r2)
    # both modules run on the one routing of W's ids (W2 supplies the second module's
    # adapters and input only)
    oracle_y = [O.lora_apply(to_f64(m_.x, "bf16"), to_f64(m_.y_base, "bf16"), oracle_adapters(W_, m_), m_.slices,
                             W.ids, W.S, "bf16", max_rank=W_.Rmax) for W_, m_ in ((W, m1), (W2, m2))]
    for n_, (o, r_) in enumerate(zip(oracle_y, (r1, r2))):
        check_close(from_device(r_), o, "bf16", f"graph fused={fused} eager module {n_ + 1} vs oracle")
    # capture (after a warm-up call on a side stream, as torch asks)
    g1, g2 = yb1.clone(), yb2.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(yb1.clone(), yb2.clone())
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(g1, g2)
    torch.cuda.synchronize()
    ox, oy = to_device(other.modules[0].x, "bf16"), to_device(other.modules[0].y_base, "bf16")
    oids = _ids(other)
    for rep in range(4):
        g1.copy_(yb1)
        g2.copy_(yb2)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(g1), ref1), f"replay {rep}: first module differs from eager"
        assert np.array_equal(bits(g2), ref2), f"replay {rep}: second module differs from eager"
        check_close(from_device(g1), oracle_y[0], "bf16", f"graph fused={fused} replay {rep} module 1 vs oracle")
        check_close(from_device(g2), oracle_y[1], "bf16", f"graph fused={fused} replay {rep} module 2 vs oracle")
        # eager work on the same objects with another batch between replays
        rx.route_linear(p1, R, oids, ox, oy.clone())
        torch.cuda.synchronize()
    p1.close(); p2.close(); R.close()


def test_join_with_the_base_gemm_at_the_decode_workload(rx):
    """The deployment form at the full decode workload (64 tokens, 8 slots,
    k = d = 4096, r = 16): the base projection y = x W0^T runs as a torch GEMM on one
    stream, the routing and shrink on another, and the expand waits for the GEMM's
    event.  y is checked against the oracle on the GEMM's own base output, and
    against the merged-weight form x (W0 + s B A)^T."""
    import torch
    W = workload(2)
    mod = W.modules[0]
    _log("join with the base GEMM, decode workload")
    pool = make_pool(rx, W, mod)
    R = rx.Routing(0, W.T, W.S)
    x = to_device(mod.x, "bf16")
    W0T = to_device(mod.W0, "bf16").t().contiguous()
    ids = _ids(W)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    y = torch.empty((W.T, sum(mod.slices)), dtype=torch.bfloat16, device="cuda")
    base = torch.empty_like(y)
    torch.cuda.synchronize()
    ready = torch.cuda.Event()
    with torch.cuda.stream(sa):
        torch.mm(x, W0T, out=y)
        ready.record(sa)
    rx.linear_join(pool, R, x, y, ready, stream=sb, ids=ids)
    torch.cuda.synchronize()
    torch.mm(x, W0T, out=base)          # the base output alone, for the oracle's input
    torch.cuda.synchronize()
    ads = oracle_adapters(W, mod)
    x64 = to_f64(mod.x, "bf16")
    ref = O.lora_apply(x64, from_device(base), ads, mod.slices, W.ids, W.S, "bf16", max_rank=W.Rmax)
    check_close(from_device(y), ref, "bf16", "joined to the base GEMM vs oracle")
    merged = O.merged_apply(x64, to_f64(mod.W0, "bf16"), ads, mod.slices, W.ids, W.S, "bf16")
    check_close(from_device(y), merged, "bf16", "joined to the base GEMM vs merged-weight form")
    pool.close(); R.close()


def test_graph_of_the_joined_step(rx):
    """The joined form captured in a HIP graph: the base GEMM on a forked stream, the
    routing and shrink on the capturing stream, the expand joined to the GEMM's event.
    Replayed 3 times with eager work between: each replay bitwise equal to the eager
    serial step (GEMM, then the fused call on one stream) and within the bf16
    tolerance of the oracle on that base output."""
    import torch
    W = small_case(57, T=64, S=8, k=1024, slices=[1024], Rmax=16, dtype="bf16", invalid=1)
    mod = W.modules[0]
    _log("graph of the joined step")
    pool = make_pool(rx, W, mod)
    R = rx.Routing(0, W.T, W.S)
    x = to_device(mod.x, "bf16")
    rng = np.random.default_rng(5)
    W0T = (torch.from_numpy(rng.standard_normal((mod.k, 1024)).astype(np.float32)) / 32.0).to(torch.bfloat16).cuda()
    ids = _ids(W)
    # eager serial reference
    y_ref = torch.mm(x, W0T)
    base = y_ref.clone()
    rx.route_linear(pool, R, ids, x, y_ref)
    torch.cuda.synchronize()
    ref_bits = bits(y_ref)
    ref = O.lora_apply(to_f64(mod.x, "bf16"), from_device(base), oracle_adapters(W, mod), mod.slices, W.ids, W.S,
                       "bf16", max_rank=W.Rmax)
    check_close(from_device(y_ref), ref, "bf16", "eager serial step vs oracle")
    y = torch.empty_like(y_ref)
    fa = torch.cuda.Stream()
    ev = torch.cuda.Event()
    warm = torch.cuda.Stream()
    warm.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(warm):
        torch.mm(x, W0T, out=y)
        rx.route_linear(pool, R, ids, x, y)
    torch.cuda.current_stream().wait_stream(warm)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cs = torch.cuda.current_stream()
        fa.wait_stream(cs)
        with torch.cuda.stream(fa):
            torch.mm(x, W0T, out=y)
            ev.record(fa)
        rx.linear_join(pool, R, x, y, ev, stream=cs, ids=ids)
        cs.wait_stream(fa)
    torch.cuda.synchronize()
    other = small_case(58, T=40, S=8, k=1024, slices=[1024], Rmax=16, dtype="bf16")
    ox, oy, oids = to_device(other.modules[0].x, "bf16"), to_device(other.modules[0].y_base, "bf16"), _ids(other)
    for rep in range(3):
        y.fill_(0.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(y), ref_bits), f"replay {rep} differs from the eager serial step"
        check_close(from_device(y), ref, "bf16", f"graph of the joined step, replay {rep} vs oracle")
        rx.route_linear(pool, R, oids, ox, oy.clone())
        torch.cuda.synchronize()
    pool.close(); R.close()
