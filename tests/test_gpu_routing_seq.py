"""lora_build_routing_seq (sequences of several tokens) against the oracle's
sequence-to-token expansion, bit-exact, through the C ABI; and lora_linear on such a
routing against the same call on the per-token ids."""
import json
import os

import numpy as np
import pytest

import oracle.lora_oracle as O
from synthetic import small_case

from lora_cases import bits, make_pool, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rx():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import rank_adapter_gemm_build_amd as m
    return m


def _check(rx, seq_ids, S, p, max_tokens=None):
    import torch
    Q = len(seq_ids)
    T = Q * p
    R = rx.Routing(0, max_tokens or max(T, 1), S)
    t = torch.tensor(np.asarray(seq_ids, dtype=np.int32), device="cuda") if Q else torch.empty(0, dtype=torch.int32,
                                                                                             device="cuda")
    R.build_seq(t, p)
    got = R.query()
    ref = O.route_tokens_per_seq(list(seq_ids), S, p)
    assert np.array_equal(got["counts"], ref.counts)
    assert np.array_equal(got["seg_offsets"], ref.seg_offsets)
    assert np.array_equal(got["sorted_ids"], ref.sorted_ids)
    assert np.array_equal(got["active_slots"], ref.active_slots)
    assert got["num_active"] == ref.num_active and got["n_invalid"] == ref.n_invalid
    R.close()


def test_routing_seq_golden(rx):
    with open(os.path.join(os.path.dirname(__file__), "golden", "routing_seq_cases.json")) as f:
        for c in json.load(f)["cases"]:
            _check(rx, c["seq_ids"], c["S"], c["tokens_per_seq"])


# the one-wave kernel (T <= 128, S < 128), the workgroup kernel with each wave's ids
# held in registers, and (large T) re-read per batch
@pytest.mark.parametrize("Q,p,S,seed", [(1, 1, 1, 0), (16, 5, 8, 1), (32, 4, 127, 2), (40, 7, 16, 3),
                                        (300, 3, 64, 4), (1000, 4, 200, 5), (9000, 4, 64, 6)])
def test_routing_seq_random(rx, Q, p, S, seed):
    rng = np.random.default_rng(seed)
    seq = rng.integers(-1, S, size=Q)
    seq[rng.random(Q) < 0.05] = S + 3   # a few invalid ids
    print(f"Q={Q} p={p} S={S} T={Q * p}", flush=True)
    _check(rx, seq.tolist(), S, p)


def test_routing_seq_errors(rx):
    import torch
    R = rx.Routing(0, 10, 4)
    ids = torch.zeros(4, dtype=torch.int32, device="cuda")
    lib = rx.lib
    assert lib.lora_build_routing_seq(R.handle, ids.data_ptr(), 4, 3, None) == rx.LORA_ERR_CAPACITY
    assert lib.lora_build_routing_seq(R.handle, ids.data_ptr(), 4, 0, None) == rx.LORA_ERR_SHAPE
    assert lib.lora_build_routing_seq(R.handle, None, 2, 2, None) == rx.LORA_ERR_INVALID_ARG
    R.close()


def test_linear_on_sequence_routing(rx):
    """y from a routing built per sequence equals y from the per-token ids, bitwise."""
    import torch
    Q, p = 24, 4
    W = small_case(61, T=Q * p, S=6, k=1024, slices=[512, 512], Rmax=16, dtype="bf16")
    rng = np.random.default_rng(61)
    seq = rng.integers(-1, W.S, size=Q).astype(np.int32)
    W.ids = np.repeat(seq, p)
    mod = W.modules[0]
    pool = make_pool(rx, W, mod)
    x = to_device(mod.x, "bf16")
    outs = []
    for per_seq in (True, False):
        R = rx.Routing(0, W.T, W.S)
        if per_seq:
            R.build_seq(torch.from_numpy(seq).cuda(), p)
        else:
            R.build(torch.from_numpy(W.ids).cuda())
        y = to_device(mod.y_base, "bf16")
        rx.linear(pool, R, x, y)
        torch.cuda.synchronize()
        outs.append(bits(y))
        R.close()
    assert np.array_equal(outs[0], outs[1])
    pool.close()
