"""lora_linear_noalloc (the allocation-free variant of lora_linear, whose k-split
partials live in the library's fixed scratch array) against lora_linear, through the
C ABI: bitwise equal on two calls in a row, the second with a smaller batch (the
scratch keeps the first call's contents), and within the oracle tolerance; a call
that needs more scratch than the array holds fails with CAPACITY."""
import numpy as np
import pytest

import oracle.lora_oracle as O
from synthetic import small_case

from lora_cases import bits, check_close, from_device, make_pool, oracle_adapters, to_device, to_f64

pytestmark = pytest.mark.gpu


def _call(rx, fn, pool, R, x, y):
    st = fn(pool.handle, R.handle, x.data_ptr(), x.stride(0), y.data_ptr(), y.stride(0), rx.LORA_BF16, None)
    assert st == 0, rx.lora_last_error()


def _case_pair(rx, W):
    import torch
    mod = W.modules[0]
    pool = make_pool(rx, W, mod)
    R = rx.Routing(0, W.T, W.S)
    R.build(torch.from_numpy(np.ascontiguousarray(W.ids, dtype=np.int32)).cuda())
    x = to_device(mod.x, "bf16")
    y_ref = to_device(mod.y_base, "bf16")
    y_na = to_device(mod.y_base, "bf16")
    _call(rx, rx.lib.lora_linear, pool, R, x, y_ref)
    _call(rx, rx.lib.lora_linear_noalloc, pool, R, x, y_na)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y_na), bits(y_ref)), "noalloc differs from lora_linear"
    ref = O.lora_apply(to_f64(mod.x, "bf16"), to_f64(mod.y_base, "bf16"), oracle_adapters(W, mod), mod.slices,
                       W.ids, W.S, "bf16", max_rank=W.Rmax)
    check_close(from_device(y_na), ref, "bf16", f"lora_linear_noalloc T={W.T} vs oracle")
    pool.close()
    R.close()


def test_noalloc_equals_linear_twice_then_smaller():
    import rank_adapter_gemm_build_amd as rx
    print("noalloc: 256 tokens, packed slices, then 37 tokens", flush=True)
    big = small_case(71, T=256, S=64, k=4096, slices=[4096, 1024, 1024], Rmax=16, invalid=3)
    _case_pair(rx, big)
    small = small_case(72, T=37, S=5, k=520, slices=[136, 24], Rmax=32, invalid=2)
    _case_pair(rx, small)
    long_segments = small_case(73, T=0, S=6, k=1032, slices=[520], Rmax=64, segments=[1, 2, 3, 4, 17, 40, 90, 99])
    _case_pair(rx, long_segments)


def test_noalloc_rejects_a_batch_beyond_the_scratch():
    import torch
    import rank_adapter_gemm_build_amd as rx
    print("noalloc: capacity error", flush=True)
    S, T, k = 4, 4096, 4096
    pool = rx.Pool(0, S, 64, k, [1024, 1024, 1024], rx.LORA_BF16, T)
    R = rx.Routing(0, T, S)
    R.build(torch.zeros(T, dtype=torch.int32, device="cuda"))
    x = torch.zeros((T, k), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((T, 3072), dtype=torch.bfloat16, device="cuda")
    # 4 k splits (4096 tokens on one slot halve the 8) x 3 slices x 4096 tokens x 64 ranks x 4 B = 12 MiB fits;
    # with max_lora_rank 96 (96 ranks per row) the call needs 18 MiB and does not
    st = rx.lib.lora_linear_noalloc(pool.handle, R.handle, x.data_ptr(), k, y.data_ptr(), 3072, rx.LORA_BF16, None)
    assert st == 0, rx.lora_last_error()
    wide = rx.Pool(0, S, 96, k, [1024, 1024, 1024], rx.LORA_BF16, T)
    st = rx.lib.lora_linear_noalloc(wide.handle, R.handle, x.data_ptr(), k, y.data_ptr(), 3072, rx.LORA_BF16, None)
    assert st == rx.LORA_ERR_CAPACITY, rx.lora_last_error()
    assert "scratch" in rx.lora_last_error()
    torch.cuda.synchronize()
    pool.close(); wide.close(); R.close()
