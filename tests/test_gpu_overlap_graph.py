"""The LoRA call joined to a base projection on another stream, and the decode step
captured in a HIP graph (torch.cuda.CUDAGraph), through the C ABI.

Bars: every result bitwise equal to the plain single-stream eager calls on the same
inputs (same kernels, same arithmetic); graph replays checked one by one, with
eager work between them.
"""
import numpy as np
import pytest

from synthetic import small_case

from lora_cases import bits, make_pool, to_device

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

    # eager reference
    r1, r2 = yb1.clone(), yb2.clone()
    step(r1, r2)
    torch.cuda.synchronize()
    ref1, ref2 = bits(r1), bits(r2)
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
        # eager work on the same objects with another batch between replays
        rx.route_linear(p1, R, oids, ox, oy.clone())
        torch.cuda.synchronize()
    p1.close(); p2.close(); R.close()
