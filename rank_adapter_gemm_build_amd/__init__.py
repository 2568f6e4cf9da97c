"""Python binding of libraxlora.so, the gfx950 batched multi-adapter LoRA library.

Argument marshalling only: every step of the computation runs in the HIP kernels
behind the C ABI (include/raxlora.h).  The module-level functions carry the C names
and take raw integers for pointers and streams; the small ``Pool`` / ``Routing``
classes accept torch tensors and numpy arrays and pass their addresses.  There is
no fallback: importing fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
# RAXLORA_LIBRARY: the path of another build of the same library (the index-checking
# variant, libraxlora_debug.so) to load instead
LIB_PATH = os.environ.get("RAXLORA_LIBRARY") or os.path.join(_HERE, "libraxlora.so")

LORA_F32, LORA_BF16, LORA_FP8E4M3 = 0, 1, 2
LORA_SRC_DEVICE, LORA_PREMULTIPLY = 1, 2
LORA_MAX_SLICES, LORA_MAX_SLOTS, LORA_MAX_RANK, LORA_MAX_IN_FEATURES = 8, 1024, 256, 65536
LORA_MAX_GROUP = 8
LORA_NOALLOC_SCRATCH_BYTES = 16 << 20

STATUS = {
    0: "LORA_OK", -1: "LORA_ERR_INVALID_ARG", -2: "LORA_ERR_SHAPE", -3: "LORA_ERR_DTYPE",
    -4: "LORA_ERR_RANK", -5: "LORA_ERR_SLOT", -6: "LORA_ERR_CAPACITY", -7: "LORA_ERR_HIP",
    -8: "LORA_ERR_OOM", -9: "LORA_ERR_NO_DEVICE", -10: "LORA_ERR_ALIGN", -11: "LORA_ERR_STATE",
}
globals().update({name: code for code, name in STATUS.items()})

# every symbol declared in include/raxlora.h, with (restype, argtypes)
_P, _I, _F, _U, _VP = C.c_void_p, C.c_int, C.c_float, C.c_uint, C.c_void_p
SIGNATURES = {
    "lora_last_error": (C.c_char_p, []),
    "lora_status_string": (C.c_char_p, [_I]),
    "lora_compute_scale": (_I, [_F, _I, _I, _F, C.POINTER(C.c_float)]),
    "lora_pool_create": (_I, [C.POINTER(_P), _I, _I, _I, _I, C.POINTER(C.c_int), _I, _I, _I]),
    "lora_pool_destroy": (_I, [_P]),
    "lora_register_adapter": (_I, [_P, _I, C.POINTER(_VP), C.POINTER(_VP), _F, _I, _I, _F, _U, _VP]),
    "lora_unregister_adapter": (_I, [_P, _I, _VP]),
    "lora_pool_slot_info": (_I, [_P, _I, C.POINTER(C.c_int), C.POINTER(C.c_float), C.POINTER(C.c_uint32),
                                 C.POINTER(C.c_uint64), C.POINTER(C.c_uint64)]),
    "lora_pool_read_slot": (_I, [_P, _I, _I, _VP, _VP]),
    "lora_routing_create": (_I, [C.POINTER(_P), _I, _I, _I]),
    "lora_routing_destroy": (_I, [_P]),
    "lora_build_routing": (_I, [_P, _VP, _I, _VP]),
    "lora_routing_query": (_I, [_P, _VP, _VP, _VP, _VP, C.POINTER(C.c_int), C.POINTER(C.c_int)]),
    "lora_shrink": (_I, [_P, _P, _VP, _I, _VP, _VP]),
    "lora_expand": (_I, [_P, _P, _VP, _VP, _I, _I, _VP]),
    "lora_linear": (_I, [_P, _P, _VP, _I, _VP, _I, _I, _VP]),
    "lora_route_linear": (_I, [_P, _P, _VP, _I, _VP, _I, _VP, _I, _I, _VP]),
    "lora_build_routing_seq": (_I, [_P, _VP, _I, _I, _VP]),
    "lora_embedding_pool_create": (_I, [C.POINTER(_P), _I, _I, _I, _I, _I, _I, _I]),
    "lora_embedding": (_I, [_P, _P, _VP, _VP, _I, _I, _VP]),
    "lora_route_embedding": (_I, [_P, _P, _VP, _I, _VP, _VP, _I, _I, _VP]),
    "lora_linear_join": (_I, [_P, _P, _VP, _I, _VP, _I, _I, _VP, _VP]),
    "lora_route_linear_join": (_I, [_P, _P, _VP, _I, _VP, _I, _VP, _I, _I, _VP, _VP]),
    "lora_bandwidth_probe": (_I, [_VP, C.c_uint64, _VP, C.c_uint64, _I, _VP]),
    "lora_index_checks": (_I, [C.POINTER(C.c_int), C.POINTER(C.c_uint64), _I]),
    "lora_linear_noalloc": (_I, [_P, _P, _VP, _I, _VP, _I, _I, _VP]),
    "lora_linear_group": (_I, [C.POINTER(_P), _I, _P, C.POINTER(_VP), C.POINTER(C.c_int), C.POINTER(_VP),
                               C.POINTER(C.c_int), _I, _VP]),
    "lora_route_linear_group": (_I, [C.POINTER(_P), _I, _P, _VP, _I, C.POINTER(_VP), C.POINTER(C.c_int),
                                     C.POINTER(_VP), C.POINTER(C.c_int), _I, _VP]),
    "lora_timing_enable": (_I, [_I]),
    "lora_timing_report": (_I, [C.POINTER(C.c_double), C.POINTER(C.c_int), _I]),
    "lora_timing_kernel_name": (C.c_char_p, [_I]),
}

KERNEL_NAMES = ["routing", "shrink", "expand", "finish_u", "gather"]


def _load():
    # The library binds to the HIP runtime already in the process.  PyTorch ships its
    # own libamdhip64 (same soname); loading it first makes it the one runtime that
    # torch's memory and streams and these kernels share.  Loading ours first would
    # leave two runtimes in the process, and the second one finds no device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m rank_adapter_gemm_build_amd.build` "
                          "(or __graft_entry__.build())")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    return lib


lib = _load()


class LoraError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.lora_last_error().decode(errors="replace")
        super().__init__(f"{where}: {STATUS.get(status, status)}: {msg}")


def _check(status: int, where: str) -> None:
    if status != 0:
        raise LoraError(status, where)


# ------------------------------------------------------------- C-named calls
def lora_last_error() -> str:
    return lib.lora_last_error().decode(errors="replace")


def lora_status_string(status: int) -> str:
    return lib.lora_status_string(status).decode()


def lora_compute_scale(alpha: float, rank: int, rslora: bool, adapter_scale: float = 1.0) -> float:
    out = C.c_float()
    _check(lib.lora_compute_scale(alpha, rank, int(bool(rslora)), adapter_scale, C.byref(out)),
           "lora_compute_scale")
    return out.value


def lora_embedding_pool_create(device: int, max_slots: int, max_lora_rank: int, vocab: int, d: int, wdtype: int,
                               max_tokens: int) -> int:
    h = C.c_void_p()
    _check(lib.lora_embedding_pool_create(C.byref(h), device, max_slots, max_lora_rank, vocab, d, wdtype, max_tokens),
           "lora_embedding_pool_create")
    return h.value


def lora_embedding(pool: int, routing: int, vocab_ids: int, y: int, ldy: int, ydtype: int, stream: int = 0) -> None:
    _check(lib.lora_embedding(pool, routing, vocab_ids or None, y or None, ldy, ydtype, stream or None),
           "lora_embedding")


def lora_pool_create(device: int, max_slots: int, max_lora_rank: int, in_features: int,
                     slice_out: Sequence[int], wdtype: int, max_tokens: int) -> int:
    h = C.c_void_p()
    arr = (C.c_int * len(slice_out))(*slice_out)
    _check(lib.lora_pool_create(C.byref(h), device, max_slots, max_lora_rank, in_features, arr,
                                len(slice_out), wdtype, max_tokens), "lora_pool_create")
    return h.value


def lora_pool_destroy(pool: int) -> None:
    _check(lib.lora_pool_destroy(pool), "lora_pool_destroy")


def lora_register_adapter(pool: int, slot: int, a_ptrs: Sequence[int], b_ptrs: Sequence[int], alpha: float,
                          rank: int, rslora: bool, adapter_scale: float, flags: int, stream: int = 0) -> None:
    n = len(a_ptrs)
    A = (C.c_void_p * n)(*[p or None for p in a_ptrs])
    B = (C.c_void_p * n)(*[p or None for p in b_ptrs])
    _check(lib.lora_register_adapter(pool, slot, A, B, alpha, rank, int(bool(rslora)), adapter_scale,
                                     flags, stream or None), "lora_register_adapter")


def lora_unregister_adapter(pool: int, slot: int, stream: int = 0) -> None:
    _check(lib.lora_unregister_adapter(pool, slot, stream or None), "lora_unregister_adapter")


def lora_pool_slot_info(pool: int, slot: int):
    r, s, m, a, b = C.c_int(), C.c_float(), C.c_uint32(), C.c_uint64(), C.c_uint64()
    _check(lib.lora_pool_slot_info(pool, slot, C.byref(r), C.byref(s), C.byref(m), C.byref(a), C.byref(b)),
           "lora_pool_slot_info")
    return {"rank": r.value, "scale": s.value, "slice_mask": m.value, "a_offset": a.value, "bt_offset": b.value}


def lora_pool_read_slot(pool: int, slot: int, slice_: int, a_host: int, bt_host: int) -> None:
    _check(lib.lora_pool_read_slot(pool, slot, slice_, a_host or None, bt_host or None), "lora_pool_read_slot")


def lora_routing_create(device: int, max_tokens: int, max_slots: int) -> int:
    h = C.c_void_p()
    _check(lib.lora_routing_create(C.byref(h), device, max_tokens, max_slots), "lora_routing_create")
    return h.value


def lora_routing_destroy(routing: int) -> None:
    _check(lib.lora_routing_destroy(routing), "lora_routing_destroy")


def lora_build_routing(routing: int, ids_ptr: int, T: int, stream: int = 0) -> None:
    _check(lib.lora_build_routing(routing, ids_ptr or None, T, stream or None), "lora_build_routing")


def lora_routing_query(routing: int, counts: int, seg_offsets: int, sorted_ids: int, active_slots: int):
    na, ni = C.c_int(), C.c_int()
    _check(lib.lora_routing_query(routing, counts or None, seg_offsets or None, sorted_ids or None,
                                  active_slots or None, C.byref(na), C.byref(ni)), "lora_routing_query")
    return na.value, ni.value


def lora_shrink(pool: int, routing: int, x: int, ldx: int, u: int, stream: int = 0) -> None:
    _check(lib.lora_shrink(pool, routing, x or None, ldx, u or None, stream or None), "lora_shrink")


def lora_expand(pool: int, routing: int, u: int, y: int, ldy: int, ydtype: int, stream: int = 0) -> None:
    _check(lib.lora_expand(pool, routing, u or None, y or None, ldy, ydtype, stream or None), "lora_expand")


def lora_linear(pool: int, routing: int, x: int, ldx: int, y: int, ldy: int, ydtype: int, stream: int = 0) -> None:
    _check(lib.lora_linear(pool, routing, x or None, ldx, y or None, ldy, ydtype, stream or None), "lora_linear")


def lora_route_linear(pool: int, routing: int, ids: int, T: int, x: int, ldx: int, y: int, ldy: int, ydtype: int,
                      stream: int = 0) -> None:
    _check(lib.lora_route_linear(pool, routing, ids or None, T, x or None, ldx, y or None, ldy, ydtype,
                                 stream or None), "lora_route_linear")


def lora_linear_join(pool: int, routing: int, x: int, ldx: int, y: int, ldy: int, ydtype: int, stream: int,
                     y_ready: int) -> None:
    _check(lib.lora_linear_join(pool, routing, x or None, ldx, y or None, ldy, ydtype, stream or None,
                                y_ready or None), "lora_linear_join")


def lora_route_linear_join(pool: int, routing: int, ids: int, T: int, x: int, ldx: int, y: int, ldy: int,
                           ydtype: int, stream: int, y_ready: int) -> None:
    _check(lib.lora_route_linear_join(pool, routing, ids or None, T, x or None, ldx, y or None, ldy, ydtype,
                                      stream or None, y_ready or None), "lora_route_linear_join")


def index_checks(reset: bool = False):
    """(enabled, failed checks) of the index-checking build (lora_index_checks); (False,
    0) for the release build.  Synchronises the device."""
    en, n = C.c_int(), C.c_uint64()
    _check(lib.lora_index_checks(C.byref(en), C.byref(n), int(bool(reset))), "lora_index_checks")
    return bool(en.value), int(n.value)


def lora_timing_enable(on: bool) -> None:
    _check(lib.lora_timing_enable(int(bool(on))), "lora_timing_enable")


def lora_timing_report():
    """{kernel name: (total milliseconds, launches)} since the last report."""
    n = len(KERNEL_NAMES)
    ms = (C.c_double * n)()
    cnt = (C.c_int * n)()
    _check(lib.lora_timing_report(ms, cnt, n), "lora_timing_report")
    return {lib.lora_timing_kernel_name(i).decode(): (ms[i], cnt[i]) for i in range(n)}


# --------------------------------------------------------- tensor-level helpers
def _ptr(t) -> int:
    """Address of a torch tensor or numpy array (None -> 0)."""
    if t is None:
        return 0
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    return t.ctypes.data


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


class Pool:
    """One target module's adapter slots (owns the device pool)."""

    def __init__(self, device: int, max_slots: int, max_lora_rank: int, in_features: int,
                 slice_out: Sequence[int], wdtype: int, max_tokens: int, embedding: bool = False):
        """embedding: a token-embedding pool (in_features = vocabulary size, one slice;
        see lora_embedding_pool_create)."""
        self.device, self.S, self.Rmax, self.k = device, max_slots, max_lora_rank, in_features
        self.slices = list(slice_out)
        self.D = sum(self.slices)
        self.wdtype, self.max_tokens, self.embedding = wdtype, max_tokens, embedding
        if embedding:
            if len(self.slices) != 1:
                raise ValueError("an embedding pool has one slice")
            self.handle = lora_embedding_pool_create(device, max_slots, max_lora_rank, in_features, self.slices[0],
                                                     wdtype, max_tokens)
        else:
            self.handle = lora_pool_create(device, max_slots, max_lora_rank, in_features, slice_out, wdtype,
                                           max_tokens)

    def register(self, slot: int, A_slices, B_slices, alpha: float, rank: int, rslora: bool = False,
                 adapter_scale: float = 1.0, premultiply: bool = False, device_src: Optional[bool] = None,
                 stream=None) -> None:
        """A_slices[n] [rank, k], B_slices[n] [d_n, rank] (None for a missing slice), host
        numpy arrays or device tensors of the pool dtype (bf16 as torch.bfloat16 or uint16;
        FP8 as torch.float8_e4m3fn or uint8; an embedding pool's A is [rank, vocab])."""
        A_slices, B_slices = list(A_slices), list(B_slices)
        if len(A_slices) != len(self.slices) or len(B_slices) != len(self.slices):
            raise ValueError(f"the pool has {len(self.slices)} slices: give one A and one B per slice (None if missing)")
        arrs = [a for a in A_slices + B_slices if a is not None]
        if device_src is None:
            device_src = any(getattr(a, "is_cuda", False) for a in arrs)
        for n, (a, b) in enumerate(zip(A_slices, B_slices)):
            if (a is None) != (b is None):
                raise ValueError(f"slice {n}: give both A and B, or neither")
            if a is None:
                continue
            for t, shape, what in ((a, (rank, self.k), "A"), (b, (self.slices[n], rank), "B")):
                if tuple(t.shape) != shape:
                    raise ValueError(f"slice {n}: {what} must have shape {shape} (got {tuple(t.shape)})")
                if _weight_dtype(t) != self.wdtype:
                    raise TypeError(f"slice {n}: {what} must be {_DT_NAMES[self.wdtype]} (got {t.dtype})")
        for a in arrs:
            if getattr(a, "is_cuda", False) != device_src:
                raise ValueError("all slices must live on the same side (host or device)")
            if device_src and a.device.index != self.device:
                raise ValueError(f"device slices must be on cuda:{self.device}")
            if hasattr(a, "is_contiguous") and not a.is_contiguous():
                raise ValueError("slices must be contiguous")
            if not hasattr(a, "is_contiguous") and not a.flags["C_CONTIGUOUS"]:
                raise ValueError("slices must be contiguous")
        flags = (LORA_SRC_DEVICE if device_src else 0) | (LORA_PREMULTIPLY if premultiply else 0)
        lora_register_adapter(self.handle, slot, [_ptr(a) for a in A_slices], [_ptr(b) for b in B_slices],
                              alpha, rank, rslora, adapter_scale, flags,
                              _stream(stream) if device_src else (_stream(stream) if stream is not None else 0))

    def unregister(self, slot: int, stream=None) -> None:
        lora_unregister_adapter(self.handle, slot, _stream(stream))

    def slot_info(self, slot: int):
        return lora_pool_slot_info(self.handle, slot)

    def read_slot(self, slot: int, slice_: int):
        import numpy as np
        dt = {LORA_BF16: np.uint16, LORA_FP8E4M3: np.uint8}.get(self.wdtype, np.float32)
        A = np.zeros((self.k, self.Rmax) if self.embedding else (self.Rmax, self.k), dtype=dt)
        Bt = np.zeros((self.Rmax, self.slices[slice_]), dtype=dt)
        lora_pool_read_slot(self.handle, slot, slice_, A.ctypes.data, Bt.ctypes.data)
        return A, Bt

    def close(self) -> None:
        if self.handle:
            lora_pool_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Routing:
    """Fixed-address routing metadata for batches of up to max_tokens tokens."""

    def __init__(self, device: int, max_tokens: int, max_slots: int):
        self.device, self.max_tokens, self.S = device, max_tokens, max_slots
        self.handle = lora_routing_create(device, max_tokens, max_slots)
        self.T = -1

    def build(self, ids, stream=None) -> None:
        """ids: device int32 tensor [T]."""
        T = _check_ids(ids, self.device, "ids")
        lora_build_routing(self.handle, _ptr(ids) if T else 0, T, _stream(stream))
        self.T = T

    def build_seq(self, seq_ids, tokens_per_seq: int, stream=None) -> None:
        """seq_ids: device int32 tensor [num_seqs], one slot per sequence of
        tokens_per_seq consecutive tokens (see lora_build_routing_seq)."""
        n = _check_ids(seq_ids, self.device, "seq_ids")
        _check(lib.lora_build_routing_seq(self.handle, _ptr(seq_ids) if n else None, n, int(tokens_per_seq),
                                          _stream(stream) or None), "lora_build_routing_seq")
        self.T = n * int(tokens_per_seq)

    def query(self):
        import numpy as np
        counts = np.zeros(self.S + 1, dtype=np.int32)
        offs = np.zeros(self.S + 2, dtype=np.int32)
        sorted_ids = np.zeros(max(self.T, 1), dtype=np.int32)
        active = np.zeros(self.S, dtype=np.int32)
        na, ni = lora_routing_query(self.handle, counts.ctypes.data, offs.ctypes.data, sorted_ids.ctypes.data,
                                    active.ctypes.data)
        return {"counts": counts, "seg_offsets": offs, "sorted_ids": sorted_ids[:self.T],
                "active_slots": active[:na], "num_active": na, "n_invalid": ni}

    def close(self) -> None:
        if self.handle:
            lora_routing_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _dt(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return LORA_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return LORA_BF16
    if t.dtype in (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8)):
        return LORA_FP8E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _weight_dtype(a) -> int:
    """Pool dtype code of a weight array: a torch tensor or a numpy array."""
    if hasattr(a, "data_ptr"):
        return _dt(a)
    import numpy as np
    dt = np.dtype(a.dtype)
    if dt == np.float32:
        return LORA_F32
    if dt in (np.dtype(np.uint16), np.dtype(np.int16)):
        return LORA_BF16
    if dt == np.dtype(np.uint8):
        return LORA_FP8E4M3
    raise TypeError(f"unsupported weight dtype {dt}")


def _act(pool) -> int:
    """dtype of the activations x a pool takes: bf16 for FP8 pools, else the pool's."""
    return LORA_BF16 if pool.wdtype == LORA_FP8E4M3 else pool.wdtype


# ----------------------------------------------------------- argument checks
# The kernels address raw pointers, so a tensor of the wrong dtype, device, shape or
# stride would be read (or written) out of bounds.  These checks run before any call
# into the library; the dtype, shape and stride checks come before the device check,
# so every rule can be exercised without a GPU.
_DT_NAMES = {LORA_F32: "float32", LORA_BF16: "bfloat16", LORA_FP8E4M3: "float8 e4m3 (uint8)"}


def _check_on_device(t, device: int, what: str) -> None:
    if not getattr(t, "is_cuda", False) or t.device.index != device:
        raise ValueError(f"{what} must be a tensor on cuda:{device}")


def _check_ids(t, device: int, what: str) -> int:
    """An int32 vector of token (or sequence) ids on the object's GPU; returns its length."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch tensor")
    if t.dtype != torch.int32:
        raise TypeError(f"{what} must be int32 (got {t.dtype}): the kernels read 4-byte ids")
    if t.dim() != 1 or (t.numel() > 1 and t.stride(0) != 1):
        raise ValueError(f"{what} must be a contiguous 1-D tensor")
    if t.numel():
        _check_on_device(t, device, what)
    return int(t.numel())


def _check_matrix(t, device: int, rows: int, cols: int, dtypes, what: str, exact_cols: bool = True) -> None:
    """A row-major [>= rows, cols] tensor (unit column stride) of one of the dtypes."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch tensor")
    dt = _dt(t)
    if dt not in dtypes:
        raise TypeError(f"{what} must be {' or '.join(_DT_NAMES[d] for d in dtypes)} (got {t.dtype})")
    if t.dim() != 2:
        raise ValueError(f"{what} must be 2-D (got shape {tuple(t.shape)})")
    if (t.shape[1] != cols) if exact_cols else (t.shape[1] < cols):
        raise ValueError(f"{what} must have {'' if exact_cols else 'at least '}{cols} columns (got {t.shape[1]})")
    if t.shape[0] < rows:
        raise ValueError(f"{what} has {t.shape[0]} rows, the batch has {rows} tokens")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{what} must have unit column stride (got stride {t.stride()})")
    if t.shape[0] > 1 and t.stride(0) < t.shape[1]:
        raise ValueError(f"{what}: row stride {t.stride(0)} is below its width {t.shape[1]}")


def _on_device(device: int, **tensors) -> None:
    """The device rule, checked after every other rule of a call."""
    for what, t in tensors.items():
        _check_on_device(t, device, what)


def _routing_tokens(routing) -> int:
    return max(int(getattr(routing, "T", 0)), 0)


def _check_x(pool, rows: int, x) -> None:
    if pool.embedding:
        raise ValueError("an embedding pool takes vocabulary ids (embedding), not activations")
    _check_matrix(x, pool.device, rows, pool.k, (_act(pool),), "x")


def _check_y(pool, rows: int, y) -> None:
    _check_matrix(y, pool.device, rows, pool.D, (_act(pool), LORA_F32), "y", exact_cols=False)


def _check_u(pool, rows: int, u) -> None:
    import torch
    if not isinstance(u, torch.Tensor):
        raise TypeError("u must be a torch tensor")
    if u.dtype != torch.float32:
        raise TypeError(f"u must be float32 (got {u.dtype})")
    want = (len(pool.slices), rows, pool.Rmax)
    if tuple(u.shape) != want:
        raise ValueError(f"u must have shape {want} (got {tuple(u.shape)})")
    if not u.is_contiguous():
        raise ValueError("u must be contiguous")


def shrink(pool: Pool, routing: Routing, x, u, stream=None) -> None:
    """u [N, T, Rmax] fp32 = per-token A_slot x (see lora_shrink)."""
    T = _routing_tokens(routing)
    _check_x(pool, T, x)
    _check_u(pool, T, u)
    _on_device(pool.device, x=x, u=u)
    lora_shrink(pool.handle, routing.handle, _ptr(x), x.stride(0), _ptr(u), _stream(stream))


def expand(pool: Pool, routing: Routing, u, y, stream=None) -> None:
    """y += s B_slot u in place (see lora_expand)."""
    T = _routing_tokens(routing)
    _check_u(pool, T, u)
    _check_y(pool, T, y)
    _on_device(pool.device, u=u, y=y)
    lora_expand(pool.handle, routing.handle, _ptr(u), _ptr(y), y.stride(0), _dt(y), _stream(stream))


def linear(pool: Pool, routing: Routing, x, y, stream=None) -> None:
    """y += s B_slot (A_slot x) in place onto the caller's base output (see lora_linear)."""
    T = _routing_tokens(routing)
    _check_x(pool, T, x)
    _check_y(pool, T, y)
    _on_device(pool.device, x=x, y=y)
    lora_linear(pool.handle, routing.handle, _ptr(x), x.stride(0), _ptr(y), y.stride(0), _dt(y), _stream(stream))


def route_linear(pool: Pool, routing: Routing, ids, x, y, stream=None) -> None:
    """routing.build(ids) then linear(pool, routing, x, y), in one fewer launch for small
    batches (see lora_route_linear)."""
    T = _check_ids(ids, routing.device, "ids")
    _check_x(pool, T, x)
    _check_y(pool, T, y)
    _on_device(pool.device, x=x, y=y)
    lora_route_linear(pool.handle, routing.handle, _ptr(ids) if T else 0, T, _ptr(x), x.stride(0), _ptr(y),
                      y.stride(0), _dt(y), _stream(stream))
    routing.T = T


def linear_join(pool: Pool, routing: Routing, x, y, y_ready, stream=None, ids=None) -> None:
    """linear (or route_linear when ids is given) whose expand waits for the torch
    event y_ready, recorded after the base output was written into y on another
    stream (see lora_linear_join / lora_route_linear_join)."""
    T = _routing_tokens(routing) if ids is None else _check_ids(ids, routing.device, "ids")
    _check_x(pool, T, x)
    _check_y(pool, T, y)
    _on_device(pool.device, x=x, y=y)
    ev = y_ready.cuda_event if y_ready is not None else 0
    if ids is None:
        lora_linear_join(pool.handle, routing.handle, _ptr(x), x.stride(0), _ptr(y), y.stride(0), _dt(y),
                         _stream(stream), ev)
    else:
        lora_route_linear_join(pool.handle, routing.handle, _ptr(ids) if T else 0, T, _ptr(x), x.stride(0), _ptr(y),
                               y.stride(0), _dt(y), _stream(stream), ev)
        routing.T = T


def embedding(pool: Pool, routing: Routing, vocab_ids, y, stream=None) -> None:
    """y += s B_slot A_slot[:, vocab_id] per LoRA token (see lora_embedding)."""
    if not pool.embedding:
        raise ValueError("embedding() needs a pool made with embedding=True")
    T = _routing_tokens(routing)
    if _check_ids(vocab_ids, pool.device, "vocab_ids") < T:
        raise ValueError(f"vocab_ids has fewer than the batch's {T} tokens")
    _check_y(pool, T, y)
    _on_device(pool.device, y=y)
    lora_embedding(pool.handle, routing.handle, _ptr(vocab_ids), _ptr(y), y.stride(0), _dt(y), _stream(stream))


def route_embedding(pool: Pool, routing: Routing, slot_ids, vocab_ids, y, stream=None) -> None:
    """routing.build(slot_ids) then embedding(pool, routing, vocab_ids, y), in one fewer
    launch for small batches (see lora_route_embedding)."""
    if not pool.embedding:
        raise ValueError("route_embedding() needs a pool made with embedding=True")
    T = _check_ids(slot_ids, routing.device, "slot_ids")
    if _check_ids(vocab_ids, pool.device, "vocab_ids") != T:
        raise ValueError("slot_ids and vocab_ids must have one entry per token")
    _check_y(pool, T, y)
    _on_device(pool.device, y=y)
    _check(lib.lora_route_embedding(pool.handle, routing.handle, _ptr(slot_ids) if T else None, T,
                                    _ptr(vocab_ids) if T else None, _ptr(y), y.stride(0), _dt(y),
                                    _stream(stream) or None), "lora_route_embedding")
    routing.T = T


def _group_arrays(pools, xs, ys):
    n = len(pools)
    P = (C.c_void_p * n)(*[p.handle for p in pools])
    X = (C.c_void_p * n)(*[_ptr(x) or None for x in xs])
    LX = (C.c_int * n)(*[x.stride(0) for x in xs])
    Y = (C.c_void_p * n)(*[_ptr(y) or None for y in ys])
    LY = (C.c_int * n)(*[y.stride(0) for y in ys])
    return n, P, X, LX, Y, LY


def _check_group(pools, xs, ys, T):
    if not (len(pools) == len(xs) == len(ys)) or not 1 <= len(pools) <= LORA_MAX_GROUP:
        raise ValueError(f"give 1..{LORA_MAX_GROUP} pools with one x and one y each")
    dts = {_dt(y) for y in ys}
    if len(dts) != 1:
        raise TypeError("every y of a grouped call has the same dtype")
    for p, x, y in zip(pools, xs, ys):
        _check_x(p, T, x)
        _check_y(p, T, y)
    for p, x, y in zip(pools, xs, ys):
        _on_device(p.device, x=x, y=y)


def linear_group(pools, routing: Routing, xs, ys, stream=None) -> None:
    """linear(pools[m], routing, xs[m], ys[m]) for every m, in one shrink and one expand
    launch (see lora_linear_group)."""
    _check_group(pools, xs, ys, _routing_tokens(routing))
    n, P, X, LX, Y, LY = _group_arrays(pools, xs, ys)
    _check(lib.lora_linear_group(P, n, routing.handle, X, LX, Y, LY, _dt(ys[0]), _stream(stream) or None),
           "lora_linear_group")


def route_linear_group(pools, routing: Routing, ids, xs, ys, stream=None) -> None:
    """routing.build(ids) then linear_group(pools, routing, xs, ys); for batches of up to
    256 tokens the routing is built inside the grouped shrink launch (see
    lora_route_linear_group)."""
    T = _check_ids(ids, routing.device, "ids")
    _check_group(pools, xs, ys, T)
    n, P, X, LX, Y, LY = _group_arrays(pools, xs, ys)
    _check(lib.lora_route_linear_group(P, n, routing.handle, _ptr(ids) if T else None, T, X, LX, Y, LY, _dt(ys[0]),
                                       _stream(stream) or None), "lora_route_linear_group")
    routing.T = T
