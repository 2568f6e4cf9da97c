"""C-ABI checks that need no GPU: exported symbols, constants, the pure scale
function, and argument validation (which runs before any HIP call)."""
import ctypes as C
import json
import os
import re

import numpy as np
import pytest

import rank_adapter_gemm_build_amd as rx
import oracle.lora_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "raxlora.h")


def _header_text():
    with open(HEADER) as f:
        return f.read()


def _declared_functions():
    text = re.sub(r"/\*.*?\*/", "", _header_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(lora_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert len(names) >= 16
    lib = C.CDLL(rx.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in raxlora.h but not exported"
    assert set(names) == set(rx.SIGNATURES), "binding signatures out of sync with the header"


def test_header_constants_match_binding():
    text = _header_text()
    defs = dict(re.findall(r"#define\s+(LORA_\w+)\s+\(?(-?\w+)\)?", text))
    for code, name in rx.STATUS.items():
        assert int(defs[name]) == code, name
    assert int(defs["LORA_SRC_DEVICE"].rstrip("u")) == rx.LORA_SRC_DEVICE
    assert int(defs["LORA_PREMULTIPLY"].rstrip("u")) == rx.LORA_PREMULTIPLY
    for n in ("LORA_MAX_SLICES", "LORA_MAX_SLOTS", "LORA_MAX_RANK", "LORA_MAX_IN_FEATURES"):
        assert int(defs[n]) == getattr(rx, n)


def test_status_strings():
    for code, name in rx.STATUS.items():
        assert rx.lora_status_string(code) == name
    assert rx.lora_status_string(-1234) == "LORA_ERR_UNKNOWN"


def test_scale_matches_oracle_golden():
    with open(os.path.join(ROOT, "tests", "golden", "scale_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        got = np.float32(rx.lora_compute_scale(c["alpha"], c["rank"], c["rslora"], c["adapter_scale"]))
        want = O.lora_scale(c["alpha"], c["rank"], c["rslora"], c["adapter_scale"])
        assert got.view(np.uint32) == np.float32(want).view(np.uint32), c


def test_scale_matches_oracle_random():
    rng = np.random.default_rng(0)
    for _ in range(3000):
        alpha = float(np.float32(rng.choice([0.0, rng.uniform(-64, 64), float(rng.integers(1, 129))])))
        rank = int(rng.integers(1, 257))
        rs = bool(rng.integers(0, 2))
        sc = float(np.float32(rng.choice([1.0, 0.0, rng.uniform(-4, 4)])))
        got = np.float32(rx.lora_compute_scale(alpha, rank, rs, sc))
        assert got.view(np.uint32) == np.float32(O.lora_scale(alpha, rank, rs, sc)).view(np.uint32)


@pytest.mark.parametrize("args,code", [
    ((1.0, 0, 0, 1.0), rx.LORA_ERR_RANK),
    ((float("nan"), 4, 0, 1.0), rx.LORA_ERR_INVALID_ARG),
    ((1.0, 4, 0, float("inf")), rx.LORA_ERR_INVALID_ARG),
    ((3e38, 1, 0, 3e38), rx.LORA_ERR_INVALID_ARG),   # overflows float
])
def test_scale_errors(args, code):
    out = C.c_float()
    assert rx.lib.lora_compute_scale(*args, C.byref(out)) == code
    assert rx.lora_last_error()
    assert rx.lib.lora_compute_scale(1.0, 4, 0, 1.0, None) == rx.LORA_ERR_INVALID_ARG


def _pool_create(*args):
    h = C.c_void_p()
    dev, S, R, k, slices, dt, T = args
    arr = (C.c_int * max(1, len(slices)))(*slices) if slices is not None else None
    return rx.lib.lora_pool_create(C.byref(h), dev, S, R, k, arr, len(slices or []), dt, T), h


@pytest.mark.parametrize("args,code", [
    ((0, 0, 16, 512, [512], rx.LORA_BF16, 8), rx.LORA_ERR_SHAPE),          # max_slots 0
    ((0, 1025, 16, 512, [512], rx.LORA_BF16, 8), rx.LORA_ERR_SHAPE),       # too many slots
    ((0, 4, 0, 512, [512], rx.LORA_BF16, 8), rx.LORA_ERR_SHAPE),           # rank 0
    ((0, 4, 257, 512, [512], rx.LORA_BF16, 8), rx.LORA_ERR_SHAPE),         # rank above the limit
    ((0, 4, 16, 0, [512], rx.LORA_BF16, 8), rx.LORA_ERR_SHAPE),            # k 0
    ((0, 4, 16, 512, [], rx.LORA_BF16, 8), rx.LORA_ERR_SHAPE),             # no slices
    ((0, 4, 16, 512, [512] * 9, rx.LORA_BF16, 8), rx.LORA_ERR_SHAPE),      # too many slices
    ((0, 4, 16, 512, [512, 0], rx.LORA_BF16, 8), rx.LORA_ERR_SHAPE),       # empty slice
    ((0, 4, 16, 512, [512], rx.LORA_BF16, 0), rx.LORA_ERR_SHAPE),          # max_tokens 0
    ((0, 4, 16, 512, [512], 7, 8), rx.LORA_ERR_DTYPE),                     # dtype
    ((0, 4, 16, 500, [512], rx.LORA_BF16, 8), rx.LORA_ERR_ALIGN),          # k % 8
    ((0, 4, 16, 512, [512, 100], rx.LORA_BF16, 8), rx.LORA_ERR_ALIGN),     # width % 8
    ((0, 4, 16, 70000, [512], rx.LORA_BF16, 8), rx.LORA_ERR_SHAPE),        # k above the limit
])
def test_pool_create_validation(args, code):
    st, h = _pool_create(*args)
    assert st == code, (rx.STATUS.get(st), rx.lora_last_error())
    assert h.value is None
    assert rx.lora_last_error()


def test_null_arguments_rejected_without_device():
    h = C.c_void_p()
    assert rx.lib.lora_pool_create(None, 0, 4, 16, 512, (C.c_int * 1)(512), 1, rx.LORA_BF16, 8) == rx.LORA_ERR_INVALID_ARG
    assert rx.lib.lora_pool_create(C.byref(h), 0, 4, 16, 512, None, 1, rx.LORA_BF16, 8) == rx.LORA_ERR_INVALID_ARG
    assert rx.lib.lora_routing_create(None, 0, 8, 4) == rx.LORA_ERR_INVALID_ARG
    assert rx.lib.lora_routing_create(C.byref(h), 0, 0, 4) == rx.LORA_ERR_SHAPE
    assert rx.lib.lora_routing_create(C.byref(h), 0, 8, 0) == rx.LORA_ERR_SHAPE
    assert rx.lib.lora_routing_create(C.byref(h), 0, 8, 2000) == rx.LORA_ERR_SHAPE
    pp = (C.c_void_p * 1)(None)
    assert rx.lib.lora_register_adapter(None, 0, pp, pp, 1.0, 4, 0, 1.0, 0, None) == rx.LORA_ERR_INVALID_ARG
    assert rx.lib.lora_unregister_adapter(None, 0, None) == rx.LORA_ERR_INVALID_ARG
    assert rx.lib.lora_pool_slot_info(None, 0, None, None, None, None, None) == rx.LORA_ERR_INVALID_ARG
    assert rx.lib.lora_pool_read_slot(None, 0, 0, None, None) == rx.LORA_ERR_INVALID_ARG
    assert rx.lib.lora_build_routing(None, None, 0, None) == rx.LORA_ERR_INVALID_ARG
    assert rx.lib.lora_routing_query(None, None, None, None, None, None, None) == rx.LORA_ERR_INVALID_ARG
    assert rx.lib.lora_shrink(None, None, None, 8, None, None) == rx.LORA_ERR_INVALID_ARG
    assert rx.lib.lora_expand(None, None, None, None, 8, rx.LORA_BF16, None) == rx.LORA_ERR_INVALID_ARG
    assert rx.lib.lora_linear(None, None, None, 8, None, 8, rx.LORA_BF16, None) == rx.LORA_ERR_INVALID_ARG
    assert rx.lib.lora_route_linear(None, None, None, 0, None, 8, None, 8, rx.LORA_BF16, None) == rx.LORA_ERR_INVALID_ARG
    assert rx.lib.lora_linear_join(None, None, None, 8, None, 8, rx.LORA_BF16, None, None) == rx.LORA_ERR_INVALID_ARG
    assert rx.lib.lora_route_linear_join(None, None, None, 0, None, 8, None, 8, rx.LORA_BF16, None, None) == \
        rx.LORA_ERR_INVALID_ARG
    assert rx.lib.lora_build_routing_seq(None, None, 0, 1, None) == rx.LORA_ERR_INVALID_ARG
    assert rx.lib.lora_embedding_pool_create(None, 0, 4, 16, 100, 64, rx.LORA_BF16, 8) == rx.LORA_ERR_INVALID_ARG
    assert rx.lib.lora_embedding(None, None, None, None, 8, rx.LORA_BF16, None) == rx.LORA_ERR_INVALID_ARG
    assert rx.lib.lora_route_embedding(None, None, None, 0, None, None, 8, rx.LORA_BF16, None) == \
        rx.LORA_ERR_INVALID_ARG
    assert rx.lib.lora_bandwidth_probe(None, 1 << 20, None, 1 << 22, 0, None) == rx.LORA_ERR_INVALID_ARG
    assert rx.lib.lora_linear_noalloc(None, None, None, 8, None, 8, rx.LORA_BF16, None) == rx.LORA_ERR_INVALID_ARG
    assert rx.lib.lora_linear_group(None, 1, None, None, None, None, None, rx.LORA_BF16, None) == \
        rx.LORA_ERR_INVALID_ARG
    assert rx.lib.lora_route_linear_group(None, 1, None, None, 0, None, None, None, None, rx.LORA_BF16, None) == \
        rx.LORA_ERR_INVALID_ARG
    assert rx.lib.lora_index_checks(None, None, 0) == rx.LORA_ERR_INVALID_ARG
    assert rx.lib.lora_pool_destroy(None) == rx.LORA_OK
    assert rx.lib.lora_routing_destroy(None) == rx.LORA_OK


def test_dtype_enum_matches_binding():
    text = re.sub(r"/\*.*?\*/", "", _header_text(), flags=re.S)
    enum = re.search(r"typedef enum \{([^}]*)\} lora_dtype;", text).group(1)
    vals = dict((k.strip(), int(v)) for k, v in re.findall(r"(LORA_\w+)\s*=\s*(\d+)", enum))
    assert vals == {"LORA_F32": rx.LORA_F32, "LORA_BF16": rx.LORA_BF16, "LORA_FP8E4M3": rx.LORA_FP8E4M3}


@pytest.mark.parametrize("args,code", [
    ((0, 4, 16, 100, 64, rx.LORA_FP8E4M3, 8), rx.LORA_ERR_DTYPE),   # FP8 embedding pools are not offered
    ((0, 4, 16, 100, 60, rx.LORA_BF16, 8), rx.LORA_ERR_ALIGN),      # output width % 8
    ((0, 4, 0, 100, 64, rx.LORA_BF16, 8), rx.LORA_ERR_SHAPE),       # rank 0
    ((0, 4, 16, 0, 64, rx.LORA_BF16, 8), rx.LORA_ERR_SHAPE),        # empty vocabulary
])
def test_embedding_pool_create_validation(args, code):
    h = C.c_void_p()
    st = rx.lib.lora_embedding_pool_create(C.byref(h), *args)
    assert st == code, (rx.STATUS.get(st), rx.lora_last_error())
    assert h.value is None


def test_valid_create_reports_missing_device():
    """On a machine without a GPU, a well-formed create fails with NO_DEVICE (a
    real error path); where a GPU exists the same call succeeds."""
    st, h = _pool_create(0, 4, 16, 512, [512], rx.LORA_BF16, 8)
    if st == rx.LORA_OK:
        rx.lora_pool_destroy(h.value)
        pytest.skip("a GPU is present")
    assert st in (rx.LORA_ERR_NO_DEVICE, rx.LORA_ERR_HIP), rx.lora_last_error()
    st2 = rx.lib.lora_routing_create(C.byref(C.c_void_p()), 0, 8, 4)
    assert st2 in (rx.LORA_ERR_NO_DEVICE, rx.LORA_ERR_HIP)


def test_index_checks_off_in_the_release_build():
    """The release library reports its index checks as compiled out, without touching a
    device."""
    assert rx.index_checks() == (False, 0)
