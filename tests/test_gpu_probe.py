"""The bandwidth probe (diagnostics) computes what it states: the read-and-write form
writes, for each 16-byte chunk j of dst, the xor of the chunks j, n + j, 2n + j, ...
of src (n = chunks written); sizes it cannot serve are refused before a launch."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def test_probe_read_write_form():
    import torch
    import rank_adapter_gemm_build_amd as rx
    rng = np.random.default_rng(3)
    ratio, n = 4, 3000
    src = rng.integers(0, 2 ** 32, size=(ratio * n, 4), dtype=np.uint32)
    s = torch.from_numpy(src.view(np.int32)).cuda()
    d = torch.zeros((n, 4), dtype=torch.int32, device="cuda")
    st = rx.lib.lora_bandwidth_probe(s.data_ptr(), s.numel() * 4, d.data_ptr(), d.numel() * 4, ratio, None)
    assert st == 0, rx.lora_last_error()
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(src.reshape(ratio, n, 4), axis=0)
    assert np.array_equal(d.cpu().numpy().view(np.uint32), want)
    # the read form: one word per thread, into a destination of at least 4 MiB
    big = torch.zeros(1 << 20, dtype=torch.int32, device="cuda")
    assert rx.lib.lora_bandwidth_probe(s.data_ptr(), s.numel() * 4, big.data_ptr(), big.numel() * 4, 0, None) == 0
    assert rx.lib.lora_bandwidth_probe(s.data_ptr(), s.numel() * 4, d.data_ptr(), d.numel() * 4, 0, None) == \
        rx.LORA_ERR_SHAPE
    assert rx.lib.lora_bandwidth_probe(s.data_ptr(), s.numel() * 4, d.data_ptr(), 16, ratio, None) == rx.LORA_ERR_SHAPE
    torch.cuda.synchronize()
