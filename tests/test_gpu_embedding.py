"""Embedding LoRA (lora_embedding on a pool from lora_embedding_pool_create) against
the oracle and against lora_linear on one-hot inputs, through the C ABI.

Bars: the hand-worked case exact (integers, fp32); random cases within the oracle
tolerances (fp32 max-abs <= 1e-4, bf16 normwise relative <= 2e-2); bitwise equal to
the linear branch on one-hot rows (the shrink of a one-hot row is exact, so both
paths hand the expand the same rank-space values).
"""
import json
import os

import numpy as np
import pytest

import oracle.lora_oracle as O

from lora_cases import bits, check_close, from_device, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rx():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import rank_adapter_gemm_build_amd as m
    return m


def _log(msg):
    print(msg, flush=True)


def _bf16(a):
    return O.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def _draw(seed, S, V, d, Rmax, T, dtype, p_nolora=0.15, bad_vocab=3):
    rng = np.random.default_rng(seed)
    ranks = {s: int(rng.choice([r for r in (1, 4, 8, 16, 32, 64) if r <= Rmax])) for s in range(S) if s != 1}
    A, B = {}, {}
    for s, r in ranks.items():
        a = rng.standard_normal((r, V)) * 0.5
        b = rng.standard_normal((d, r)) / np.sqrt(r)
        A[s] = _bf16(a) if dtype == "bf16" else a.astype(np.float32)
        B[s] = _bf16(b) if dtype == "bf16" else b.astype(np.float32)
    ids = rng.integers(0, S, size=T).astype(np.int32)
    ids[rng.random(T) < p_nolora] = -1
    vocab = rng.integers(0, V, size=T).astype(np.int32)
    vocab[rng.choice(T, size=min(bad_vocab, T), replace=False)] = [V, -1, V + 100][:min(bad_vocab, T)]
    yb = rng.standard_normal((T, d))
    yb = _bf16(yb) if dtype == "bf16" else yb.astype(np.float32)
    alpha = {s: float(2 * r) for s, r in ranks.items()}
    return ranks, A, B, ids, vocab, yb, alpha


def _f64(a, dtype):
    return O.bf16_bits_to_f64(a) if dtype == "bf16" else np.asarray(a, dtype=np.float64)


def _embed_pool(rx, S, Rmax, V, d, dtype, T, ranks, A, B, alpha):
    wdt = rx.LORA_BF16 if dtype == "bf16" else rx.LORA_F32
    pool = rx.Pool(0, S, Rmax, V, [d], wdt, T, embedding=True)
    for s, r in ranks.items():
        pool.register(s, [A[s]], [B[s]], alpha[s], r)
    return pool


def test_embedding_golden(rx):
    """The hand-worked case, with the output padded to 8 columns (zero rows of B)."""
    import torch
    with open(os.path.join(os.path.dirname(__file__), "golden", "embedding_case.json")) as f:
        g = json.load(f)
    d = 8
    Bp = np.zeros((d, g["rank"]), dtype=np.float32)
    Bp[:g["d"]] = np.array(g["B"], dtype=np.float32)
    yb = np.zeros((len(g["vocab_ids"]), d), dtype=np.float32)
    yb[:, :g["d"]] = np.array(g["y_base"], dtype=np.float32)
    pool = rx.Pool(0, g["S"], 4, g["vocab"], [d], rx.LORA_F32, 8, embedding=True)
    pool.register(0, [np.array(g["A"], dtype=np.float32)], [Bp], g["alpha"], g["rank"])
    R = rx.Routing(0, 8, g["S"])
    R.build(torch.tensor(g["slot_ids"], dtype=torch.int32, device="cuda"))
    y = to_device(yb, "f32")
    rx.embedding(pool, R, torch.tensor(g["vocab_ids"], dtype=torch.int32, device="cuda"), y)
    torch.cuda.synchronize()
    got = from_device(y)
    assert np.array_equal(got[:, :g["d"]], np.array(g["y"], dtype=np.float64))
    assert np.array_equal(got[:, g["d"]:], np.zeros((len(g["vocab_ids"]), d - g["d"])))
    pool.close(); R.close()


@pytest.mark.parametrize("dtype,T,S,V,d,Rmax", [("bf16", 37, 6, 1000, 512, 16), ("bf16", 300, 6, 32000, 1024, 64),
                                                ("f32", 45, 5, 777, 264, 8), ("bf16", 64, 8, 32000, 4096, 16)])
def test_embedding_matches_oracle(rx, dtype, T, S, V, d, Rmax):
    import torch
    _log(f"embedding {dtype} T={T} S={S} V={V} d={d} Rmax={Rmax}")
    ranks, A, B, ids, vocab, yb, alpha = _draw(70 + T, S, V, d, Rmax, T, dtype)
    pool = _embed_pool(rx, S, Rmax, V, d, dtype, T, ranks, A, B, alpha)
    R = rx.Routing(0, T, S)
    R.build(torch.from_numpy(ids).cuda())
    ads = {s: O.Adapter(rank=r, A=[_f64(A[s], dtype)], B=[_f64(B[s], dtype)], alpha=alpha[s])
           for s, r in ranks.items()}
    vt = torch.from_numpy(vocab).cuda()
    # delta alone (base 0, fp32 output), then onto a base in the pool dtype
    y0 = to_device(np.zeros((T, d), dtype=np.float32), "f32")
    rx.embedding(pool, R, vt, y0)
    y = to_device(yb, dtype)
    rx.embedding(pool, R, vt, y)
    torch.cuda.synchronize()
    ref0 = O.embedding_apply(vocab, np.zeros((T, d)), ads, V, ids, S, dtype)
    check_close(from_device(y0), ref0, dtype, "delta")
    ref = O.embedding_apply(vocab, _f64(yb, dtype), ads, V, ids, S, dtype)
    check_close(from_device(y), ref, dtype, "y")
    rows = ids < 0   # no-LoRA rows bit-untouched
    assert np.array_equal(bits(y)[rows], (yb.view(np.uint32) if dtype == "f32" else yb)[rows])
    pool.close(); R.close()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_embedding_equals_linear_on_one_hot_rows(rx, dtype):
    import torch
    T, S, V, d, Rmax = 90, 7, 1024, 1024, 16
    ranks, A, B, ids, vocab, yb, alpha = _draw(81, S, V, d, Rmax, T, dtype, bad_vocab=0)
    wdt = rx.LORA_BF16 if dtype == "bf16" else rx.LORA_F32
    emb = _embed_pool(rx, S, Rmax, V, d, dtype, T, ranks, A, B, alpha)
    lin = rx.Pool(0, S, Rmax, V, [d], wdt, T)
    for s, r in ranks.items():
        lin.register(s, [A[s]], [B[s]], alpha[s], r)
    onehot = np.zeros((T, V), dtype=np.float32)
    onehot[np.arange(T), vocab] = 1.0
    x = to_device(_bf16(onehot) if dtype == "bf16" else onehot, dtype)
    R = rx.Routing(0, T, S)
    R.build(torch.from_numpy(ids).cuda())
    y1 = to_device(yb, dtype)
    rx.embedding(emb, R, torch.from_numpy(vocab).cuda(), y1)
    y2 = to_device(yb, dtype)
    rx.linear(lin, R, x, y2)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y1), bits(y2))
    emb.close(); lin.close(); R.close()


def test_embedding_pool_errors(rx):
    import torch
    emb = rx.Pool(0, 2, 8, 100, [64], rx.LORA_BF16, 16, embedding=True)
    lin = rx.Pool(0, 2, 8, 128, [64], rx.LORA_BF16, 16)
    R = rx.Routing(0, 16, 2)
    R.build(torch.zeros(4, dtype=torch.int32, device="cuda"))
    x = torch.zeros((4, 128), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(4, dtype=torch.int32, device="cuda")
    lib = rx.lib
    assert lib.lora_linear(emb.handle, R.handle, x.data_ptr(), 128, y.data_ptr(), 64, rx.LORA_BF16, None) == \
        rx.LORA_ERR_INVALID_ARG
    assert lib.lora_embedding(lin.handle, R.handle, v.data_ptr(), y.data_ptr(), 64, rx.LORA_BF16, None) == \
        rx.LORA_ERR_INVALID_ARG
    assert lib.lora_embedding(emb.handle, R.handle, None, y.data_ptr(), 64, rx.LORA_BF16, None) == \
        rx.LORA_ERR_INVALID_ARG
    emb.close(); lin.close(); R.close()


@pytest.mark.parametrize("T,S", [(64, 8), (256, 200), (300, 9), (1, 1)])
def test_route_embedding_matches_two_calls(rx, T, S):
    """lora_route_embedding (routing inside the gather launch up to 256 tokens; the
    separate routing launch above) against lora_build_routing + lora_embedding:
    routing outputs and y bitwise equal."""
    import torch
    V, d, Rmax = 5000, 512, 32
    ranks, A, B, ids, vocab, yb, alpha = _draw(90 + T, S, V, d, Rmax, T, "bf16")
    pool = _embed_pool(rx, S, Rmax, V, d, "bf16", T, ranks, A, B, alpha)
    it, vt = torch.from_numpy(ids).cuda(), torch.from_numpy(vocab).cuda()
    R1, R2 = rx.Routing(0, T, S), rx.Routing(0, T, S)
    y1, y2 = to_device(yb, "bf16"), to_device(yb, "bf16")
    R1.build(it)
    rx.embedding(pool, R1, vt, y1)
    rx.route_embedding(pool, R2, it, vt, y2)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y1), bits(y2))
    q1, q2 = R1.query(), R2.query()
    for key in ("counts", "seg_offsets", "sorted_ids", "active_slots"):
        assert np.array_equal(q1[key], q2[key])
    assert q1["n_invalid"] == q2["n_invalid"] and q1["num_active"] == q2["num_active"]
    pool.close(); R1.close(); R2.close()
