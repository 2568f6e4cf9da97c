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
LIB_PATH = os.path.join(_HERE, "libraxlora.so")

LORA_F32, LORA_BF16, LORA_FP8E4M3 = 0, 1, 2
LORA_SRC_DEVICE, LORA_PREMULTIPLY = 1, 2
LORA_MAX_SLICES, LORA_MAX_SLOTS, LORA_MAX_RANK, LORA_MAX_IN_FEATURES = 8, 1024, 256, 65536

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
        numpy arrays or device tensors of the pool dtype (bf16 as torch.bfloat16 or uint16)."""
        arrs = [a for a in list(A_slices) + list(B_slices) if a is not None]
        if device_src is None:
            device_src = any(getattr(a, "is_cuda", False) for a in arrs)
        for a in arrs:
            if getattr(a, "is_cuda", False) != device_src:
                raise ValueError("all slices must live on the same side (host or device)")
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
        T = int(ids.numel())
        lora_build_routing(self.handle, _ptr(ids) if T else 0, T, _stream(stream))
        self.T = T

    def build_seq(self, seq_ids, tokens_per_seq: int, stream=None) -> None:
        """seq_ids: device int32 tensor [num_seqs], one slot per sequence of
        tokens_per_seq consecutive tokens (see lora_build_routing_seq)."""
        n = int(seq_ids.numel())
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


def _act(pool) -> int:
    """dtype of the activations x a pool takes: bf16 for FP8 pools, else the pool's."""
    return LORA_BF16 if pool.wdtype == LORA_FP8E4M3 else pool.wdtype


def shrink(pool: Pool, routing: Routing, x, u, stream=None) -> None:
    """u [N, T, Rmax] fp32 = per-token A_slot x (see lora_shrink)."""
    if _dt(x) != _act(pool):
        raise TypeError("x dtype must be the pool's activation dtype")
    lora_shrink(pool.handle, routing.handle, _ptr(x), x.stride(0), _ptr(u), _stream(stream))


def expand(pool: Pool, routing: Routing, u, y, stream=None) -> None:
    """y += s B_slot u in place (see lora_expand)."""
    lora_expand(pool.handle, routing.handle, _ptr(u), _ptr(y), y.stride(0), _dt(y), _stream(stream))


def linear(pool: Pool, routing: Routing, x, y, stream=None) -> None:
    """y += s B_slot (A_slot x) in place onto the caller's base output (see lora_linear)."""
    if _dt(x) != _act(pool):
        raise TypeError("x dtype must be the pool's activation dtype")
    lora_linear(pool.handle, routing.handle, _ptr(x), x.stride(0), _ptr(y), y.stride(0), _dt(y), _stream(stream))


def route_linear(pool: Pool, routing: Routing, ids, x, y, stream=None) -> None:
    """routing.build(ids) then linear(pool, routing, x, y), in one fewer launch for small
    batches (see lora_route_linear)."""
    if _dt(x) != _act(pool):
        raise TypeError("x dtype must be the pool's activation dtype")
    T = int(ids.numel())
    lora_route_linear(pool.handle, routing.handle, _ptr(ids) if T else 0, T, _ptr(x), x.stride(0), _ptr(y),
                      y.stride(0), _dt(y), _stream(stream))
    routing.T = T


def linear_join(pool: Pool, routing: Routing, x, y, y_ready, stream=None, ids=None) -> None:
    """linear (or route_linear when ids is given) whose expand waits for the torch
    event y_ready, recorded after the base output was written into y on another
    stream (see lora_linear_join / lora_route_linear_join)."""
    if _dt(x) != _act(pool):
        raise TypeError("x dtype must be the pool's activation dtype")
    ev = y_ready.cuda_event if y_ready is not None else 0
    if ids is None:
        lora_linear_join(pool.handle, routing.handle, _ptr(x), x.stride(0), _ptr(y), y.stride(0), _dt(y),
                         _stream(stream), ev)
    else:
        T = int(ids.numel())
        lora_route_linear_join(pool.handle, routing.handle, _ptr(ids) if T else 0, T, _ptr(x), x.stride(0), _ptr(y),
                               y.stride(0), _dt(y), _stream(stream), ev)
        routing.T = T


def embedding(pool: Pool, routing: Routing, vocab_ids, y, stream=None) -> None:
    """y += s B_slot A_slot[:, vocab_id] per LoRA token (see lora_embedding)."""
    lora_embedding(pool.handle, routing.handle, _ptr(vocab_ids), _ptr(y), y.stride(0), _dt(y), _stream(stream))


def route_embedding(pool: Pool, routing: Routing, slot_ids, vocab_ids, y, stream=None) -> None:
    """routing.build(slot_ids) then embedding(pool, routing, vocab_ids, y), in one fewer
    launch for small batches (see lora_route_embedding)."""
    T = int(slot_ids.numel())
    _check(lib.lora_route_embedding(pool.handle, routing.handle, _ptr(slot_ids) if T else None, T,
                                    _ptr(vocab_ids) if T else None, _ptr(y), y.stride(0), _dt(y),
                                    _stream(stream) or None), "lora_route_embedding")
    routing.T = T
