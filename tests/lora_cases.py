"""Helpers shared by the GPU tests: move seeded workloads onto the GPU through the
binding, and turn them into oracle inputs (test infrastructure)."""
from __future__ import annotations

import os

import numpy as np

import oracle.lora_oracle as O
from synthetic import Workload

BF16_TOL = 2e-2      # normwise relative error, bf16 storage with fp32 accumulation
F32_TOL = 1e-4       # max-abs error, fp32


def to_f64(a, dtype: str) -> np.ndarray:
    return O.bf16_bits_to_f64(a) if dtype == "bf16" else np.asarray(a, dtype=np.float64)


def oracle_adapters(W: Workload, mod, premultiply=False, ranks=None):
    ads = {}
    for s, r in (ranks or W.ranks).items():
        A = [None if a is None else to_f64(a, W.dtype) for a in mod.A[s]]
        B = [None if b is None else to_f64(b, W.dtype) for b in mod.B[s]]
        ads[s] = O.Adapter(rank=r, A=A, B=B, alpha=W.alpha[s], rslora=W.rslora,
                           adapter_scale=W.adapter_scale, premultiply=premultiply)
    return ads


def torch_dtype(dtype: str):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_device(a: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def from_device(t) -> np.ndarray:
    """Exact float64 values of a device tensor (bf16 or fp32)."""
    import torch
    if t.dtype == torch.bfloat16:
        return O.bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.double().cpu().numpy()


def bits(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy().view(np.uint32)


def make_pool(rx, W: Workload, mod, premultiply=False, max_tokens=None, device_src=False):
    wdt = rx.LORA_BF16 if W.dtype == "bf16" else rx.LORA_F32
    pool = rx.Pool(0, W.S, W.Rmax, mod.k, mod.slices, wdt, max_tokens or max(W.T, 1))
    for s, r in W.ranks.items():
        A, B = mod.A[s], mod.B[s]
        if device_src:
            A = [None if a is None else to_device(a, W.dtype) for a in A]
            B = [None if b is None else to_device(b, W.dtype) for b in B]
        pool.register(s, A, B, W.alpha[s], r, W.rslora, W.adapter_scale, premultiply=premultiply)
    return pool


def make_routing(rx, W: Workload, max_tokens=None):
    import torch
    R = rx.Routing(0, max_tokens or max(W.T, 1), W.S)
    ids = torch.from_numpy(np.ascontiguousarray(W.ids, dtype=np.int32)).cuda()
    R.build(ids)
    return R, ids


def y_base_of(W: Workload, mod) -> np.ndarray:
    """Base output in the storage format: y_base as drawn, or X W0^T rounded."""
    if mod.y_base is not None:
        return mod.y_base
    x = to_f64(mod.x, W.dtype)
    w0 = to_f64(mod.W0, W.dtype)
    yb = x @ w0.T
    if W.dtype == "bf16":
        return O.f32_to_bf16_bits(yb.astype(np.float32))
    return yb.astype(np.float32)


def normwise_rel(got: np.ndarray, ref: np.ndarray) -> float:
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / den) if den > 0 else float(np.abs(got).max())


# Measured errors of this session, printed as a table at the end of the run
# (tests/conftest.py): (test, what, measure, value, bar).
MEASURED = []


def record_error(what: str, measure: str, value: float, bar: float) -> None:
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    MEASURED.append((test, what, measure, float(value), float(bar)))


def check_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str) -> float:
    if dtype == "f32":
        err = float(np.abs(got - ref).max()) if got.size else 0.0
        record_error(what, "max-abs", err, F32_TOL)
        assert err <= F32_TOL, f"{what}: max-abs error {err:.3e} > {F32_TOL}"
    else:
        err = normwise_rel(got, ref) if got.size else 0.0
        record_error(what, "normwise-rel", err, BF16_TOL)
        assert err <= BF16_TOL, f"{what}: normwise relative error {err:.3e} > {BF16_TOL}"
    return err
