"""Python binding of libmoe (ctypes).

Argument marshalling only: every step of the layer runs in the HIP kernels of
libmoe.so; PyTorch provides device memory, pinned host memory and streams.
The function names match the C ABI in include/moe.h.  Importing this module
fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
MOE_E_INVALID = -1
MOE_E_UNSUPPORTED = -2
MOE_E_HIP = -3
MOE_E_WORKSPACE = -4
MOE_E_POOL = -5

MOE_F16 = 1
MOE_BF16 = 2
MOE_F32 = 3

_DTYPES = {torch.float16: MOE_F16, torch.bfloat16: MOE_BF16, torch.float32: MOE_F32}

# every symbol include/moe.h declares
EXPORTS = (
    "moe_blob_bytes", "moe_workspace_bytes", "moe_route", "moe_expert_ffn", "moe_combine",
    "moe_permute", "moe_layer_forward", "moe_pool_create", "moe_pool_destroy",
    "moe_pool_get_stats", "moe_pool_reset_stats", "moe_lfu_replay", "moe_set_tuning",
    "moe_pool_set_policy", "moe_cache_replay", "moe_pool_fail_copy",
    "moe_set_profile_events", "moe_workspace_timeouts", "moe_status_string",
    "moe_layer_forward_noalloc", "moe_store_stride", "moe_store_open", "moe_store_read",
    "moe_store_get_stats", "moe_store_close", "moe_pool_create_store", "moe_block_forward",
    "moe_block_workspace_bytes", "moe_read_probe",
)

MOE_STORE_DIRECT = 1
MOE_STORE_MMAP = 2


class MoEError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


class moe_qmat(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("meta", ctypes.c_void_p),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32), ("bits", ctypes.c_int32)]


class moe_bank(ctypes.Structure):
    _fields_ = [("blobs", ctypes.c_void_p), ("E", ctypes.c_int32), ("D", ctypes.c_int32),
                ("F", ctypes.c_int32)]


class moe_pool_stats(ctypes.Structure):
    _fields_ = [("lookups", ctypes.c_uint64), ("hits", ctypes.c_uint64),
                ("misses", ctypes.c_uint64), ("evictions", ctypes.c_uint64),
                ("bytes_h2d", ctypes.c_uint64)]


class moe_store_stats(ctypes.Structure):
    _fields_ = [("blobs", ctypes.c_uint64), ("bytes", ctypes.c_uint64), ("ns", ctypes.c_uint64),
                ("errors", ctypes.c_uint64), ("last_errno", ctypes.c_uint64),
                ("bounced", ctypes.c_uint64)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m quantized_mixture_experts_moe_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    P = ctypes.POINTER
    sig = {
        "moe_blob_bytes": (sz, [i32, i32]),
        "moe_workspace_bytes": (sz, [i32, i32, i32, i32, i32, i32]),
        "moe_route": (i32, [vp, i32, i32, P(moe_qmat), vp, i32, vp, vp, vp, vp, sz, vp]),
        "moe_expert_ffn": (i32, [vp, i32, i32, P(moe_bank), vp, i32, vp, vp, sz, vp]),
        "moe_combine": (i32, [vp, vp, vp, i32, i32, i32, vp, i32, vp]),
        "moe_permute": (i32, [vp, i32, i32, i32, vp, vp, vp, vp, vp]),
        "moe_layer_forward": (i32, [vp, i32, i32, P(moe_qmat), vp, i32, P(moe_bank),
                                    P(moe_bank), vp, i32, vp, i32, vp, vp, vp, sz, vp]),
        "moe_layer_forward_noalloc": (i32, [vp, i32, i32, P(moe_qmat), vp, i32, P(moe_bank),
                                            P(moe_bank), vp, i32, vp, vp, vp]),
        "moe_block_forward": (i32, [vp, i32, i32, vp, vp, ctypes.c_float, P(moe_qmat), vp, i32,
                                    P(moe_bank), P(moe_bank), vp, i32, vp, i32, vp, vp, vp, vp,
                                    sz, vp]),
        "moe_block_workspace_bytes": (sz, [i32, i32, i32, i32, i32, i32]),
        "moe_pool_create": (i32, [P(vp), i32, i32, i32, i32, i32, vp]),
        "moe_store_stride": (sz, [i32, i32]),
        "moe_store_open": (i32, [P(vp), ctypes.c_char_p, i32, i32, i32, i32, i32, i32]),
        "moe_store_read": (i32, [vp, i32, vp, i32, vp, sz]),
        "moe_store_get_stats": (i32, [vp, P(moe_store_stats)]),
        "moe_store_close": (i32, [vp]),
        "moe_pool_create_store": (i32, [P(vp), i32, vp, sz]),
        "moe_pool_destroy": (i32, [vp]),
        "moe_pool_get_stats": (i32, [vp, P(moe_pool_stats)]),
        "moe_pool_reset_stats": (i32, [vp]),
        "moe_lfu_replay": (i32, [i32, i32, i32, i32, vp, vp]),
        "moe_pool_set_policy": (i32, [vp, i32]),
        "moe_pool_fail_copy": (i32, [vp, i32]),
        "moe_cache_replay": (i32, [i32, i32, i32, i32, i32, vp, vp]),
        "moe_set_tuning": (i32, [ctypes.c_char_p, i32]),
        "moe_set_profile_events": (i32, [vp, i32]),
        "moe_workspace_timeouts": (i32, [vp, sz, P(ctypes.c_uint32), vp]),
        "moe_status_string": (ctypes.c_char_p, [i32]),
        "moe_read_probe": (i32, [vp, sz, vp, i32, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.moe_status_string(status).decode()


def _check(status: int, what: str) -> None:
    if status != MOE_OK:
        raise MoEError(status, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def moe_blob_bytes(D: int, F: int) -> int:
    return int(lib.moe_blob_bytes(D, F))


def moe_workspace_bytes(T: int, k: int, E: int, D: int, F: int, F_shared: int) -> int:
    return int(lib.moe_workspace_bytes(T, k, E, D, F, F_shared))


def moe_block_workspace_bytes(T: int, k: int, E: int, D: int, F: int, F_shared: int) -> int:
    return int(lib.moe_block_workspace_bytes(T, k, E, D, F, F_shared))


def moe_read_probe(buf: torch.Tensor, sink: torch.Tensor, blocks: int, stream=None) -> None:
    """Streaming read of the whole device buffer (measurement helper)."""
    _check(lib.moe_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), blocks,
                              _stream(stream)), "moe_read_probe")


def moe_set_tuning(key: str, value: int) -> None:
    _check(lib.moe_set_tuning(key.encode(), value), "moe_set_tuning")


class ProfileEvents:
    """Timing-event pairs the library records around its expert phase."""

    def __init__(self, n_pairs: int):
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_pairs)]
        for e in self.events:  # create the underlying hipEvent
            e.record()
        torch.cuda.synchronize()
        self._arr = (ctypes.c_void_p * len(self.events))(*[e.cuda_event for e in self.events])
        self.n = n_pairs

    def __enter__(self):
        _check(lib.moe_set_profile_events(ctypes.cast(self._arr, ctypes.c_void_p), self.n),
               "moe_set_profile_events")
        return self

    def __exit__(self, *exc):
        lib.moe_set_profile_events(None, 0)

    def elapsed_ms(self, count: int):
        return [self.events[2 * i].elapsed_time(self.events[2 * i + 1]) for i in range(count)]


# --------------------------------------------------------------------------
# device-resident weights
# --------------------------------------------------------------------------
class DeviceQMat:
    """An affine-quantised matrix in HBM (codes + meta tensors)."""

    def __init__(self, codes: np.ndarray, meta: np.ndarray, rows: int, cols: int, bits: int,
                 device="cuda"):
        self.codes = torch.from_numpy(np.ascontiguousarray(codes).view(np.uint8).reshape(-1)).to(device)
        self.meta = torch.from_numpy(np.ascontiguousarray(meta).view(np.int32).reshape(-1)).to(device)
        self.struct = moe_qmat(self.codes.data_ptr(), self.meta.data_ptr(), rows, cols, bits)
        self.rows, self.cols, self.bits = rows, cols, bits


class DeviceBank:
    """E expert blobs in HBM and the device array of their addresses."""

    def __init__(self, blobs: torch.Tensor, D: int, F: int):
        # blobs: uint8 device tensor [E, blob_bytes] (rows 256-byte aligned)
        assert blobs.dim() == 2 and blobs.dtype == torch.uint8 and blobs.is_cuda
        nb = moe_blob_bytes(D, F)
        assert blobs.shape[1] == nb and nb % 256 == 0
        self.blobs = blobs
        E = blobs.shape[0]
        addrs = [blobs.data_ptr() + e * blobs.stride(0) for e in range(E)]
        self.table = torch.tensor(np.array(addrs, dtype=np.uint64).view(np.int64),
                                  device=blobs.device)
        self.struct = moe_bank(self.table.data_ptr(), E, D, F)
        self.E, self.D, self.F = E, D, F

    @classmethod
    def from_numpy(cls, blobs: np.ndarray, D: int, F: int, device="cuda"):
        arr = np.ascontiguousarray(blobs).reshape(-1, moe_blob_bytes(D, F))
        return cls(torch.from_numpy(arr).to(device), D, F)


class Workspace:
    """Zero-filled device scratch for calls up to the given sizes (block:
    sized for moe_block_forward)."""

    def __init__(self, T, k, E, D, F, F_shared, device="cuda", block=False):
        n = (moe_block_workspace_bytes if block else moe_workspace_bytes)(T, k, E, D, F, F_shared)
        if n == 0:
            raise ValueError("invalid workspace sizes")
        self.buf = torch.zeros(n, dtype=torch.uint8, device=device)
        self.nbytes = n

    def timeouts(self, stream=None) -> int:
        """Device-side waits that timed out since the buffer was zero-filled
        (blocks the host until the stream's work is done)."""
        c = ctypes.c_uint32(0)
        _check(lib.moe_workspace_timeouts(_ptr(self.buf), self.nbytes, ctypes.byref(c),
                                          _stream(stream)), "moe_workspace_timeouts")
        return int(c.value)


def _x_dtype(x: torch.Tensor) -> int:
    dt = _DTYPES.get(x.dtype)
    if dt not in (MOE_F16, MOE_BF16):
        raise TypeError("x must be float16 or bfloat16")
    return dt


# --------------------------------------------------------------------------
# the ABI calls
# --------------------------------------------------------------------------
def moe_route(x: torch.Tensor, router: DeviceQMat, k: int, ids: torch.Tensor, gates: torch.Tensor,
              ws: Workspace, logit_bias: Optional[torch.Tensor] = None,
              logits: Optional[torch.Tensor] = None, stream=None) -> None:
    T = x.shape[0]
    _check(lib.moe_route(_ptr(x), _x_dtype(x), T, ctypes.byref(router.struct), _ptr(logit_bias),
                         k, _ptr(ids), _ptr(gates), _ptr(logits), _ptr(ws.buf), ws.nbytes,
                         _stream(stream)), "moe_route")


def moe_expert_ffn(x: torch.Tensor, bank: DeviceBank, ids: Optional[torch.Tensor], k: int,
                   y: torch.Tensor, ws: Workspace, stream=None) -> None:
    T = x.shape[0]
    _check(lib.moe_expert_ffn(_ptr(x), _x_dtype(x), T, ctypes.byref(bank.struct), _ptr(ids), k,
                              _ptr(y), _ptr(ws.buf), ws.nbytes, _stream(stream)),
           "moe_expert_ffn")


def moe_combine(y: torch.Tensor, gates: torch.Tensor, y_shared: Optional[torch.Tensor],
                out: torch.Tensor, stream=None) -> None:
    T, k, D = y.shape
    _check(lib.moe_combine(_ptr(y), _ptr(gates), _ptr(y_shared), T, k, D, _ptr(out),
                           _DTYPES[out.dtype], _stream(stream)), "moe_combine")


def moe_permute(ids: torch.Tensor, E: int, counts: torch.Tensor, offsets: torch.Tensor,
                perm: torch.Tensor, inv: torch.Tensor, stream=None) -> None:
    T, k = ids.shape
    _check(lib.moe_permute(_ptr(ids), T, k, E, _ptr(counts), _ptr(offsets), _ptr(perm),
                           _ptr(inv), _stream(stream)), "moe_permute")


def moe_layer_forward(x: torch.Tensor, router: DeviceQMat, k: int, routed: Optional[DeviceBank],
                      shared: Optional[DeviceBank], out: torch.Tensor, ws: Workspace,
                      logit_bias: Optional[torch.Tensor] = None, pool: Optional["Pool"] = None,
                      layer: int = 0, ids_out: Optional[torch.Tensor] = None,
                      gates_out: Optional[torch.Tensor] = None, stream=None) -> None:
    T = x.shape[0]
    _check(lib.moe_layer_forward(
        _ptr(x), _x_dtype(x), T, ctypes.byref(router.struct), _ptr(logit_bias), k,
        ctypes.byref(routed.struct) if routed is not None else None,
        ctypes.byref(shared.struct) if shared is not None else None,
        pool.handle if pool is not None else None, layer, _ptr(out), _DTYPES[out.dtype],
        _ptr(ids_out), _ptr(gates_out), _ptr(ws.buf), ws.nbytes, _stream(stream)),
        "moe_layer_forward")


def moe_block_forward(x: torch.Tensor, w_pre: torch.Tensor, w_post: torch.Tensor, eps: float,
                      router: DeviceQMat, k: int, routed: Optional[DeviceBank],
                      shared: Optional[DeviceBank], out: torch.Tensor, ws: Workspace,
                      logit_bias: Optional[torch.Tensor] = None, pool: Optional["Pool"] = None,
                      layer: int = 0, u_out: Optional[torch.Tensor] = None,
                      ids_out: Optional[torch.Tensor] = None,
                      gates_out: Optional[torch.Tensor] = None, stream=None) -> None:
    T = x.shape[0]
    _check(lib.moe_block_forward(
        _ptr(x), _x_dtype(x), T, _ptr(w_pre), _ptr(w_post), float(eps),
        ctypes.byref(router.struct), _ptr(logit_bias), k,
        ctypes.byref(routed.struct) if routed is not None else None,
        ctypes.byref(shared.struct) if shared is not None else None,
        pool.handle if pool is not None else None, layer, _ptr(out), _DTYPES[out.dtype],
        _ptr(u_out), _ptr(ids_out), _ptr(gates_out), _ptr(ws.buf), ws.nbytes, _stream(stream)),
        "moe_block_forward")


def moe_layer_forward_noalloc(x: torch.Tensor, router: DeviceQMat, k: int, routed: DeviceBank,
                              shared: Optional[DeviceBank], out: torch.Tensor,
                              logit_bias: Optional[torch.Tensor] = None,
                              ids_out: Optional[torch.Tensor] = None,
                              gates_out: Optional[torch.Tensor] = None, stream=None) -> None:
    """moe_layer_forward (resident experts) on the library's own fixed
    scratch array: nothing is allocated."""
    T = x.shape[0]
    _check(lib.moe_layer_forward_noalloc(
        _ptr(x), _x_dtype(x), T, ctypes.byref(router.struct), _ptr(logit_bias), k,
        ctypes.byref(routed.struct), ctypes.byref(shared.struct) if shared is not None else None,
        _ptr(out), _DTYPES[out.dtype], _ptr(ids_out), _ptr(gates_out), _stream(stream)),
        "moe_layer_forward_noalloc")


def moe_cache_replay(policy: int, slots: int, E: int, ids: np.ndarray) -> np.ndarray:
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    n, k = ids.shape
    ev = np.zeros((n, k, 4), dtype=np.int32)
    _check(lib.moe_cache_replay(policy, slots, E, k, n, ids.ctypes.data_as(ctypes.c_void_p),
                                ev.ctypes.data_as(ctypes.c_void_p)), "moe_cache_replay")
    return ev


def moe_lfu_replay(slots: int, E: int, ids: np.ndarray) -> np.ndarray:
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    n, k = ids.shape
    ev = np.zeros((n, k, 4), dtype=np.int32)
    _check(lib.moe_lfu_replay(slots, E, k, n, ids.ctypes.data_as(ctypes.c_void_p),
                              ev.ctypes.data_as(ctypes.c_void_p)), "moe_lfu_replay")
    return ev


def moe_store_stride(D: int, F: int) -> int:
    return int(lib.moe_store_stride(D, F))


class Store:
    """Expert blobs of every layer in one file, read by bounded-parallel pread
    (moe_store_open).  flags: 0 buffered, MOE_STORE_DIRECT, MOE_STORE_MMAP."""

    def __init__(self, path: str, n_layers: int, E: int, D: int, F: int, flags: int = 1,
                 threads: int = 16):
        h = ctypes.c_void_p()
        _check(lib.moe_store_open(ctypes.byref(h), path.encode(), n_layers, E, D, F, flags,
                                  threads), "moe_store_open")
        self.handle = h
        self.n_layers, self.E, self.D, self.F = n_layers, E, D, F
        self.stride = moe_store_stride(D, F)

    def read(self, layer: int, experts: Sequence[int], dst: Sequence[int], chunk: int = 0) -> None:
        """Read blobs into host buffers at the given addresses (each >= stride)."""
        ids = (ctypes.c_int32 * len(experts))(*[int(e) for e in experts])
        ptrs = (ctypes.c_void_p * len(dst))(*[int(d) for d in dst])
        _check(lib.moe_store_read(self.handle, layer, ctypes.cast(ids, ctypes.c_void_p),
                                  len(experts), ctypes.cast(ptrs, ctypes.c_void_p), chunk),
               "moe_store_read")

    def stats(self) -> dict:
        st = moe_store_stats()
        _check(lib.moe_store_get_stats(self.handle, ctypes.byref(st)), "moe_store_get_stats")
        return {f: int(getattr(st, f)) for f, _ in moe_store_stats._fields_}

    def close(self) -> None:
        if self.handle:
            lib.moe_store_close(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Pool:
    """HBM expert slot pool over pinned host blobs (moe_pool_create)."""

    def __init__(self, host_blobs: Sequence[torch.Tensor], n_layers: int, slots: int, E: int,
                 D: int, F: int):
        # host_blobs: pinned uint8 tensors; one [E, blob] tensor per layer
        assert len(host_blobs) == n_layers
        nb = moe_blob_bytes(D, F)
        addrs = []
        for t in host_blobs:
            assert t.is_pinned() and t.shape == (E, nb)
            addrs.extend(t.data_ptr() + e * t.stride(0) for e in range(E))
        self._keep = list(host_blobs)
        arr = (ctypes.c_void_p * len(addrs))(*addrs)
        h = ctypes.c_void_p()
        _check(lib.moe_pool_create(ctypes.byref(h), n_layers, slots, E, D, F,
                                   ctypes.cast(arr, ctypes.c_void_p)),
               "moe_pool_create")
        self.handle = h

    @classmethod
    def from_store(cls, store: "Store", slots: int, chunk: int = 0) -> "Pool":
        """A pool whose misses are read from the store (moe_pool_create_store)."""
        self = cls.__new__(cls)
        self._keep = [store]
        h = ctypes.c_void_p()
        _check(lib.moe_pool_create_store(ctypes.byref(h), slots, store.handle, chunk),
               "moe_pool_create_store")
        self.handle = h
        return self

    def set_policy(self, policy: int) -> None:
        """0: least frequently used (default), 1: least recently used."""
        _check(lib.moe_pool_set_policy(self.handle, policy), "moe_pool_set_policy")

    def fail_copy(self, after: int) -> None:
        """Test hook: let `after` copies through, then fail one (-1 clears)."""
        _check(lib.moe_pool_fail_copy(self.handle, after), "moe_pool_fail_copy")

    def stats(self) -> dict:
        st = moe_pool_stats()
        _check(lib.moe_pool_get_stats(self.handle, ctypes.byref(st)), "moe_pool_get_stats")
        return {f: int(getattr(st, f)) for f, _ in moe_pool_stats._fields_}

    def reset_stats(self) -> None:
        _check(lib.moe_pool_reset_stats(self.handle), "moe_pool_reset_stats")

    def close(self) -> None:
        if self.handle:
            lib.moe_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
