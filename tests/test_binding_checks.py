"""The Python binding rejects tensors the kernels would misread, before any call into
the library (no GPU needed: the dtype, shape and stride rules are checked before
the device rule, and a host tensor fails the device rule)."""
import numpy as np
import pytest
import torch

import rank_adapter_gemm_build_amd as rx


def _pool(wdtype=rx.LORA_BF16, k=64, slices=(32, 16), Rmax=8, embedding=False):
    p = object.__new__(rx.Pool)
    p.device, p.S, p.Rmax, p.k = 0, 4, Rmax, k
    p.slices = list(slices)
    p.D = sum(p.slices)
    p.wdtype, p.max_tokens, p.embedding = wdtype, 64, embedding
    p.handle = 0
    return p


def _routing(T=8):
    r = object.__new__(rx.Routing)
    r.device, r.max_tokens, r.S, r.T, r.handle = 0, 64, 4, T, 0
    return r


def _no_library_call(monkeypatch):
    def refuse(*a, **k):
        raise AssertionError("the library was called")
    for name in ("lora_linear", "lora_shrink", "lora_expand", "lora_route_linear", "lora_register_adapter",
                 "lora_build_routing", "lora_embedding", "lora_linear_join", "lora_route_linear_join"):
        monkeypatch.setattr(rx, name, refuse)


BF = torch.bfloat16


@pytest.mark.parametrize("make_x,make_y,err", [
    (lambda: torch.zeros(8, 64, dtype=torch.float32), lambda: torch.zeros(8, 48, dtype=BF), TypeError),   # x dtype
    (lambda: torch.zeros(8, 64, dtype=BF), lambda: torch.zeros(8, 48, dtype=torch.float16), TypeError),   # y dtype
    (lambda: torch.zeros(7, 64, dtype=BF), lambda: torch.zeros(8, 48, dtype=BF), ValueError),   # x rows < T
    (lambda: torch.zeros(8, 64, dtype=BF), lambda: torch.zeros(7, 48, dtype=BF), ValueError),   # y rows < T
    (lambda: torch.zeros(8, 56, dtype=BF), lambda: torch.zeros(8, 48, dtype=BF), ValueError),   # x width != k
    (lambda: torch.zeros(8, 64, dtype=BF), lambda: torch.zeros(8, 40, dtype=BF), ValueError),   # y width < D
    (lambda: torch.zeros(64, 8, dtype=BF).t(), lambda: torch.zeros(8, 48, dtype=BF), ValueError),   # column stride
    (lambda: torch.zeros(64, dtype=BF), lambda: torch.zeros(8, 48, dtype=BF), ValueError),   # not 2-D
    (lambda: torch.zeros(8, 64, dtype=BF), lambda: torch.zeros(8, 48, dtype=BF), ValueError),   # host tensors
])
def test_linear_rejects_bad_tensors(monkeypatch, make_x, make_y, err):
    _no_library_call(monkeypatch)
    with pytest.raises(err):
        rx.linear(_pool(), _routing(8), make_x(), make_y())


def test_linear_accepts_f32_output_and_wide_rows(monkeypatch):
    """y may be float32 and wider than D (a strided view into a bigger buffer): only the
    device rule remains, and it fails for host tensors."""
    _no_library_call(monkeypatch)
    with pytest.raises(ValueError, match="cuda:0"):
        rx.linear(_pool(), _routing(8), torch.zeros(8, 64, dtype=BF), torch.zeros(8, 64, dtype=torch.float32))


@pytest.mark.parametrize("ids,err", [
    (torch.zeros(8, dtype=torch.int64), TypeError),          # torch's default integer dtype
    (torch.zeros(8, dtype=torch.int16), TypeError),
    (torch.zeros(4, 2, dtype=torch.int32), ValueError),      # not 1-D
    (torch.zeros(16, dtype=torch.int32)[::2], ValueError),   # not contiguous
    (torch.zeros(8, dtype=torch.int32), ValueError),         # host tensor
    (np.zeros(8, dtype=np.int32), TypeError),                # not a tensor
])
def test_ids_rejected(monkeypatch, ids, err):
    _no_library_call(monkeypatch)
    with pytest.raises(err):
        rx.route_linear(_pool(), _routing(), ids, torch.zeros(8, 64, dtype=BF), torch.zeros(8, 48, dtype=BF))
    with pytest.raises(err):
        _routing().build(ids)


@pytest.mark.parametrize("u,err", [
    (torch.zeros(2, 8, 8, dtype=BF), TypeError),
    (torch.zeros(2, 8, 4), ValueError),              # Rmax is 8
    (torch.zeros(1, 8, 8), ValueError),              # two slices
    (torch.zeros(2, 8, 16)[:, :, :8], ValueError),   # not contiguous
    (torch.zeros(2, 8, 8), ValueError),              # host tensor
])
def test_u_rejected(monkeypatch, u, err):
    _no_library_call(monkeypatch)
    with pytest.raises(err):
        rx.expand(_pool(), _routing(8), u, torch.zeros(8, 48, dtype=BF))


def test_fp8_pool_takes_bf16_activations(monkeypatch):
    _no_library_call(monkeypatch)
    with pytest.raises(TypeError):
        rx.linear(_pool(rx.LORA_FP8E4M3), _routing(8), torch.zeros(8, 64, dtype=torch.uint8),
                  torch.zeros(8, 48, dtype=BF))


def test_embedding_pool_rejects_activations_and_short_vocab_ids(monkeypatch):
    _no_library_call(monkeypatch)
    with pytest.raises(ValueError):
        rx.linear(_pool(embedding=True, slices=(48,)), _routing(8), torch.zeros(8, 64, dtype=BF),
                  torch.zeros(8, 48, dtype=BF))
    with pytest.raises(ValueError):
        rx.embedding(_pool(), _routing(8), torch.zeros(8, dtype=torch.int32), torch.zeros(8, 48, dtype=BF))
    with pytest.raises(TypeError):
        rx.embedding(_pool(embedding=True, slices=(48,)), _routing(8), torch.zeros(8, dtype=torch.int64),
                     torch.zeros(8, 48, dtype=BF))


@pytest.mark.parametrize("A,B,err", [
    ([np.zeros((4, 64), np.float32), np.zeros((4, 64), np.uint16)],
     [np.zeros((32, 4), np.uint16), np.zeros((16, 4), np.uint16)], TypeError),      # A dtype
    ([np.zeros((4, 64), np.uint16), np.zeros((4, 64), np.uint16)],
     [np.zeros((32, 4), np.uint16), np.zeros((16, 5), np.uint16)], ValueError),     # B not [d, rank]
    ([np.zeros((4, 56), np.uint16), None],
     [np.zeros((32, 4), np.uint16), None], ValueError),                             # A not [rank, k]
    ([np.zeros((4, 64), np.uint16), None],
     [np.zeros((32, 4), np.uint16), np.zeros((16, 4), np.uint16)], ValueError),     # half-missing slice
    ([np.zeros((4, 64), np.uint16)],
     [np.zeros((32, 4), np.uint16)], ValueError),                                   # one slice of two
    ([np.zeros((64, 4), np.uint16).T, None],
     [np.zeros((32, 4), np.uint16), None], ValueError),                             # not contiguous
])
def test_register_rejects_bad_weights(monkeypatch, A, B, err):
    _no_library_call(monkeypatch)
    with pytest.raises(err):
        _pool().register(0, A, B, 8.0, 4)
