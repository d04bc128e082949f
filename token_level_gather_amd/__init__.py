"""Python binding of the MI355X sparse KV assembly library (``libkvs.so``).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch supplies device memory and streams.  The binding loads the
in-tree ``libkvs.so`` and raises if it is missing; there is no fallback.

Names follow the C ABI in ``include/kvs.h``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# KVS_LIB selects another build of the same library (e.g. the host-sanitizer
# build of the CPU tests); the default is the in-tree libkvs.so
LIB_PATH = os.environ.get("KVS_LIB") or os.path.join(HERE, "libkvs.so")
# the build with device-side bounds checks (a debugging aid; Pool(library=...))
CHECKED_LIB_PATH = os.path.join(HERE, "libkvs_checked.so")

KVS_OK = 0
KVS_EINVAL = -22
KVS_ENOMEM = -12
KVS_ERANGE = -34
KVS_EDUP = -17
KVS_ECORRUPT = -74
KVS_EBOUNDS = -14
KVS_EHIP_BASE = -1000

HEADS, HEAD_DIM, V_DIM = 16, 576, 512
ROW_BYTES = HEAD_DIM * 2
KERNEL_NAMES = ("diff_lru", "gather", "attention", "combine", "assemble")
KVS_FLAG_HITS_FIRST = 1
KVS_FLAG_PADDED_TOPK = 2
KVS_FLAG_DIRECT_HOT = 4
KVS_FLAG_CHECK = 8
KVS_FLAG_SEPARATE_ATTENTION = 16
PROBE_SINK_WORDS = 65536
# accesses checked by the device-checked build (kvs_step_stats.fault_site)
KVS_SITE_LRU_ORDER = 1
KVS_SITE_SLOT_TOKEN = 2
KVS_SITE_DIFF_LIST = 3
KVS_SITE_MISS = 4
KVS_SITE_HIT = 5
KVS_SITE_ROW_SLOT = 6
KVS_SITE_APPEND = 7

# Every exported symbol of include/kvs.h.
EXPORTS = (
    "kvs_query_sizes", "kvs_host_alloc", "kvs_host_free", "kvs_create_pool", "kvs_publish",
    "kvs_step", "kvs_free_request", "kvs_sync_status", "kvs_debug_read_state",
    "kvs_profile_begin", "kvs_profile_end", "kvs_release", "kvs_strerror",
    "kvs_graph_capture", "kvs_graph_launch", "kvs_graph_destroy", "kvs_publish_device",
    "kvs_append", "kvs_probe_host_read", "kvs_step_static", "kvs_probe_hit_copy",
)
STATIC_SCRATCH_BYTES = 32 << 20


class kvs_config(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("layers", ctypes.c_int32), ("context", ctypes.c_int64),
        ("slots", ctypes.c_int32), ("topk", ctypes.c_int32), ("heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("v_dim", ctypes.c_int32), ("scale", ctypes.c_float),
        ("attn_splits", ctypes.c_int32), ("fetch_blocks", ctypes.c_int32),
        ("hit_blocks", ctypes.c_int32), ("flags", ctypes.c_int32),
    ]


class kvs_sizes(ctypes.Structure):
    _fields_ = [
        ("host_pool_bytes", ctypes.c_uint64), ("hot_bytes", ctypes.c_uint64),
        ("meta_bytes", ctypes.c_uint64), ("cbuf_bytes", ctypes.c_uint64),
        ("scratch_bytes", ctypes.c_uint64), ("attn_splits", ctypes.c_int32),
        ("fetch_blocks", ctypes.c_int32),
    ]


class kvs_buffers(ctypes.Structure):
    _fields_ = [
        ("host_pool", ctypes.c_void_p), ("hot", ctypes.c_void_p), ("meta", ctypes.c_void_p),
        ("cbuf", ctypes.c_void_p), ("scratch", ctypes.c_void_p),
        ("host_pool_bytes", ctypes.c_uint64), ("hot_bytes", ctypes.c_uint64),
        ("meta_bytes", ctypes.c_uint64), ("cbuf_bytes", ctypes.c_uint64),
        ("scratch_bytes", ctypes.c_uint64),
    ]


class kvs_step_stats(ctypes.Structure):
    _fields_ = [
        ("unit_steps", ctypes.c_int64), ("hits", ctypes.c_int64), ("misses", ctypes.c_int64),
        ("evictions", ctypes.c_int64), ("host_bytes", ctypes.c_int64), ("status", ctypes.c_int32),
        ("fault_site", ctypes.c_int32), ("fault_index", ctypes.c_int64),
    ]


_I32P = ctypes.POINTER(ctypes.c_int32)


class kvs_unit_state(ctypes.Structure):
    _fields_ = [
        ("tok2slot", _I32P), ("slot2tok", _I32P), ("last_used", _I32P), ("lru_order", _I32P),
        ("slot_of", _I32P), ("miss_pos", _I32P), ("victims", _I32P), ("evicted", _I32P),
        ("counts", _I32P), ("row_slot", _I32P), ("step", ctypes.c_int32),
    ]


class kvs_kernel_times(ctypes.Structure):
    _fields_ = [("steps", ctypes.c_int32), ("launches", ctypes.c_int32 * len(KERNEL_NAMES)),
                ("ms_total", ctypes.c_float * len(KERNEL_NAMES))]


class KvsError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {strerror(code)} ({code})")


_libs = {}


def lib() -> ctypes.CDLL:
    """Load libkvs.so (built by ``__graft_entry__.build()``); raise if it is absent."""
    return load_library(LIB_PATH)


def load_library(path: str) -> ctypes.CDLL:
    """Load a build of the library (once per path) and declare its signatures."""
    path = os.path.abspath(path)
    if path in _libs:
        return _libs[path]
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build() "
                          "(python -m token_level_gather_amd._build)")
    # torch ships its own HIP runtime under the same soname; importing torch
    # first makes the library bind to that one, so the process has a single
    # HIP runtime (a library loaded before torch pulls in the system runtime,
    # and torch's then finds no device)
    import torch  # noqa: F401
    L = ctypes.CDLL(path)
    vp, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
    sig = {
        "kvs_query_sizes": [ctypes.POINTER(kvs_config), ctypes.POINTER(kvs_sizes)],
        "kvs_host_alloc": [u64, ctypes.POINTER(vp)],
        "kvs_host_free": [vp],
        "kvs_create_pool": [ctypes.POINTER(kvs_config), ctypes.POINTER(kvs_buffers), vp,
                            ctypes.POINTER(vp)],
        "kvs_publish": [vp, i32, i32, i64, i64, vp],
        "kvs_publish_device": [vp, i32, i32, i64, i64, vp, vp],
        "kvs_append": [vp, i32, vp, vp, vp],
        "kvs_probe_host_read": [vp, u64, vp, vp],
        "kvs_probe_hit_copy": [vp, i32, vp],
        "kvs_step": [vp, i32, vp, vp, vp, vp, vp],
        "kvs_step_static": [vp, i32, vp, vp, vp, vp, vp],
        "kvs_free_request": [vp, i32, vp],
        "kvs_sync_status": [vp, vp, ctypes.POINTER(kvs_step_stats)],
        "kvs_debug_read_state": [vp, i32, i32, vp, ctypes.POINTER(kvs_unit_state)],
        "kvs_profile_begin": [vp, i32, ctypes.c_uint32],
        "kvs_profile_end": [vp, ctypes.POINTER(kvs_kernel_times)],
        "kvs_release": [vp],
        "kvs_graph_capture": [vp, i32, vp, vp, vp, vp, ctypes.POINTER(vp)],
        "kvs_graph_launch": [vp, vp],
        "kvs_graph_destroy": [vp],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.kvs_strerror.argtypes = [ctypes.c_int]
    L.kvs_strerror.restype = ctypes.c_char_p
    _libs[path] = L
    return L


def strerror(code: int) -> str:
    return lib().kvs_strerror(int(code)).decode()


def _check(rc: int, what: str) -> int:
    if rc != KVS_OK:
        raise KvsError(rc, what)
    return rc


def make_config(batch, layers, context, slots, topk, scale=None, attn_splits=0, fetch_blocks=0,
                hit_blocks=0, flags=0, heads=HEADS, head_dim=HEAD_DIM, v_dim=V_DIM) -> kvs_config:
    if scale is None:
        scale = 1.0 / float(np.sqrt(head_dim))
    return kvs_config(batch, layers, context, slots, topk, heads, head_dim, v_dim, scale,
                      attn_splits, fetch_blocks, hit_blocks, flags)


def query_sizes(cfg: kvs_config) -> kvs_sizes:
    out = kvs_sizes()
    _check(lib().kvs_query_sizes(ctypes.byref(cfg), ctypes.byref(out)), "kvs_query_sizes")
    return out


class HostPool:
    """Pinned host memory from kvs_host_alloc, viewed as numpy uint16 [B][L][N][576]."""

    def __init__(self, batch, layers, context):
        self.shape = (batch, layers, context, HEAD_DIM)
        self.nbytes = batch * layers * context * ROW_BYTES
        ptr = ctypes.c_void_p()
        _check(lib().kvs_host_alloc(self.nbytes, ctypes.byref(ptr)), "kvs_host_alloc")
        self.ptr = ptr.value
        buf = (ctypes.c_uint16 * (self.nbytes // 2)).from_address(self.ptr)
        self.array = np.ctypeslib.as_array(buf).reshape(self.shape)

    def free(self):
        if self.ptr:
            self.array = None
            lib().kvs_host_free(self.ptr)
            self.ptr = None


def probe_host_read(host_ptr: int, nbytes: int, sink, stream=None) -> None:
    """Enqueue the zero-copy host-read probe (measurement helper): ``sink`` is a
    contiguous device tensor of PROBE_SINK_WORDS 4-byte words."""
    if not sink.is_cuda or sink.numel() * sink.element_size() < 4 * PROBE_SINK_WORDS:
        raise ValueError("sink must be a device tensor of PROBE_SINK_WORDS 4-byte words")
    _check(lib().kvs_probe_host_read(host_ptr, nbytes, sink.data_ptr(), _stream_ptr(stream)),
           "kvs_probe_host_read")


def _stream_ptr(stream, device=None) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


class Pool:
    """One pool of B requests x L layers: hot buffers, maps and the host pool.

    Device buffers are torch tensors on ``device`` (default: the current HIP
    device); the host pool is pinned memory from kvs_host_alloc
    (``self.host.array`` is its numpy view).  ``step`` enqueues one layer's
    fetch + write-back + attention.  Calls without a stream use ``device``'s
    current stream; when that is the default (NULL) stream, ``device`` must be
    the current device (the library rejects a stream of another device).
    ``close()`` (or leaving a ``with`` block) releases the
    pool and frees a host pool the pool allocated itself.
    """

    def __init__(self, batch, layers, context, slots, topk, scale=None, attn_splits=0,
                 fetch_blocks=0, hit_blocks=0, flags=0, host: Optional[HostPool] = None,
                 device=None, stream=None, library: Optional[ctypes.CDLL] = None):
        import torch
        self._lib = library if library is not None else lib()
        self.cfg = make_config(batch, layers, context, slots, topk, scale, attn_splits,
                               fetch_blocks, hit_blocks, flags)
        self.sizes = query_sizes(self.cfg)
        self.B, self.L, self.N, self.S, self.K = batch, layers, context, slots, topk
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None \
            else torch.device(device)
        self._owns_host = host is None
        self.host = host if host is not None else HostPool(batch, layers, context)
        if self.host.nbytes < self.sizes.host_pool_bytes:
            raise KvsError(KVS_ENOMEM, "host pool")

        def dev(nbytes):
            return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=self.device)

        self.hot = dev(self.sizes.hot_bytes)
        self.meta = dev(self.sizes.meta_bytes)
        self.cbuf = dev(self.sizes.cbuf_bytes)
        self.scratch = dev(self.sizes.scratch_bytes)
        bufs = kvs_buffers(self.host.ptr, self.hot.data_ptr(), self.meta.data_ptr(),
                           self.cbuf.data_ptr(), self.scratch.data_ptr(), self.host.nbytes,
                           self.hot.numel(), self.meta.numel(), self.cbuf.numel(),
                           self.scratch.numel())
        handle = ctypes.c_void_p()
        with torch.cuda.device(self.device):   # the library binds the pool to the current device
            rc = self._lib.kvs_create_pool(ctypes.byref(self.cfg), ctypes.byref(bufs),
                                       _stream_ptr(stream, self.device), ctypes.byref(handle))
        _check(rc,
               "kvs_create_pool")
        self.handle = handle

    # -- lifecycle --------------------------------------------------------
    def publish(self, req, layer, first_tok, rows: np.ndarray):
        rows = np.ascontiguousarray(rows, dtype=np.uint16)
        assert rows.ndim == 2 and rows.shape[1] == HEAD_DIM
        _check(self._lib.kvs_publish(self.handle, req, layer, first_tok, rows.shape[0],
                                 rows.ctypes.data), "kvs_publish")

    def publish_device(self, req, layer, first_tok, rows, stream=None):
        """rows: contiguous device tensor [n][576] of 2-byte elements."""
        if not rows.is_cuda or rows.dim() != 2 or rows.shape[1] != HEAD_DIM \
                or rows.element_size() != 2 or not rows.is_contiguous():
            raise ValueError("expected a contiguous device tensor [n][576] of bf16")
        _check(self._lib.kvs_publish_device(self.handle, req, layer, first_tok, rows.shape[0],
                                        rows.data_ptr(), _stream_ptr(stream, self.device)),
               "kvs_publish_device")

    def append(self, layer, rows, pos, stream=None):
        """rows [B][576] bf16 and pos [B] int64 (-1 = nothing to append), device."""
        self._check_dev(rows, (self.B, HEAD_DIM), 2)
        self._check_dev(pos, (self.B,), 8)
        _check(self._lib.kvs_append(self.handle, layer, rows.data_ptr(), pos.data_ptr(),
                                _stream_ptr(stream, self.device)), "kvs_append")

    def step(self, layer, topk, q, out, lse=None, stream=None):
        """topk [B][K] int32, q [B][16][576] bf16/uint16, out [B][16][512] bf16 (device)."""
        self._check_dev(topk, (self.B, self.K), 4)
        self._check_dev(q, (self.B, HEADS, HEAD_DIM), 2)
        self._check_dev(out, (self.B, HEADS, V_DIM), 2)
        lse_ptr = None
        if lse is not None:
            self._check_dev(lse, (self.B, HEADS), 4)
            lse_ptr = lse.data_ptr()
        _check(self._lib.kvs_step(self.handle, layer, topk.data_ptr(), q.data_ptr(), out.data_ptr(),
                              lse_ptr, _stream_ptr(stream, self.device)), "kvs_step")

    def step_static(self, layer, topk, q, out, lse=None, stream=None):
        """kvs_step_static: ``step`` with the library's static per-GPU scratch."""
        self._check_dev(topk, (self.B, self.K), 4)
        self._check_dev(q, (self.B, HEADS, HEAD_DIM), 2)
        self._check_dev(out, (self.B, HEADS, V_DIM), 2)
        lse_ptr = None
        if lse is not None:
            self._check_dev(lse, (self.B, HEADS), 4)
            lse_ptr = lse.data_ptr()
        _check(self._lib.kvs_step_static(self.handle, layer, topk.data_ptr(), q.data_ptr(),
                                     out.data_ptr(), lse_ptr, _stream_ptr(stream, self.device)),
               "kvs_step_static")

    def free_request(self, req, stream=None):
        _check(self._lib.kvs_free_request(self.handle, req, _stream_ptr(stream, self.device)),
               "kvs_free_request")

    def sync_status(self, stream=None):
        """Returns (status code, kvs_step_stats); the status is cleared."""
        st = kvs_step_stats()
        rc = self._lib.kvs_sync_status(self.handle, _stream_ptr(stream, self.device),
                                   ctypes.byref(st))
        if rc not in (KVS_OK, KVS_ERANGE, KVS_EDUP, KVS_ECORRUPT, KVS_EBOUNDS):
            raise KvsError(rc, "kvs_sync_status")
        return rc, st

    def probe_hit_copy(self, layer, stream=None):
        """kvs_probe_hit_copy (measurement helper): the index copy of the last
        step's hits alone, reading layer ``layer``'s hot rows."""
        _check(self._lib.kvs_probe_hit_copy(self.handle, layer, _stream_ptr(stream, self.device)),
               "kvs_probe_hit_copy")

    def read_state(self, req, layer, stream=None) -> dict:
        arr = {
            "tok2slot": np.empty(self.N, np.int32), "slot2tok": np.empty(self.S, np.int32),
            "last_used": np.empty(self.S, np.int32), "lru_order": np.empty(self.S, np.int32),
            "slot_of": np.empty(self.K, np.int32), "miss_pos": np.empty(self.K, np.int32),
            "victims": np.empty(self.K, np.int32), "evicted": np.empty(self.K, np.int32),
            "counts": np.empty(4, np.int32), "row_slot": np.empty(self.K, np.int32),
        }
        st = kvs_unit_state(*[a.ctypes.data_as(_I32P) for a in arr.values()], 0)
        _check(self._lib.kvs_debug_read_state(self.handle, req, layer, _stream_ptr(stream, self.device),
                                          ctypes.byref(st)), "kvs_debug_read_state")
        arr["step"] = int(st.step)
        return arr

    def profile_begin(self, max_steps, kernels=KERNEL_NAMES):
        """Bracket every launch of the named kernels with HIP events."""
        mask = 0
        for k in kernels:
            mask |= 1 << KERNEL_NAMES.index(k)
        _check(self._lib.kvs_profile_begin(self.handle, max_steps, mask), "kvs_profile_begin")

    def profile_end(self) -> dict:
        t = kvs_kernel_times()
        _check(self._lib.kvs_profile_end(self.handle, ctypes.byref(t)), "kvs_profile_end")
        return {"steps": t.steps,
                "launches": {n: t.launches[i] for i, n in enumerate(KERNEL_NAMES)},
                **{n: t.ms_total[i] for i, n in enumerate(KERNEL_NAMES)}}

    def capture(self, layer, topk, q, out, lse=None) -> "StepGraph":
        """Capture one step of `layer` over these fixed buffers into a HIP graph."""
        self._check_dev(topk, (self.B, self.K), 4)
        self._check_dev(q, (self.B, HEADS, HEAD_DIM), 2)
        self._check_dev(out, (self.B, HEADS, V_DIM), 2)
        if lse is not None:
            self._check_dev(lse, (self.B, HEADS), 4)
        import torch
        g = ctypes.c_void_p()
        with torch.cuda.device(self.device):   # the capture stream is made on the current device
            rc = self._lib.kvs_graph_capture(self.handle, layer, topk.data_ptr(), q.data_ptr(),
                                         out.data_ptr(), None if lse is None else lse.data_ptr(),
                                         ctypes.byref(g))
        _check(rc, "kvs_graph_capture")
        return StepGraph(g, (topk, q, out, lse), self.device, self._lib)

    def release(self):
        if self.handle:
            _check(self._lib.kvs_release(self.handle), "kvs_release")
            self.handle = None

    def close(self):
        """Release the pool and free the host pool if this pool allocated it."""
        self.release()
        if self._owns_host and self.host.ptr:
            self.host.free()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
        return False

    # -- helpers ----------------------------------------------------------
    def _check_dev(self, t, shape, itemsize):
        if not t.is_cuda or tuple(t.shape) != shape or t.element_size() != itemsize \
                or not t.is_contiguous():
            raise ValueError(f"expected a contiguous device tensor {shape} of {itemsize}-byte "
                             f"elements, got {tuple(t.shape)} {t.dtype} on {t.device}")


class StepGraph:
    """A captured kvs_step; launch() replays it on a stream of the pool's device."""

    def __init__(self, handle, keep_alive, device=None, library=None):
        self._lib = library if library is not None else lib()
        self.handle = handle
        self._keep = keep_alive
        self.device = device

    def launch(self, stream=None):
        _check(self._lib.kvs_graph_launch(self.handle, _stream_ptr(stream, self.device)),
               "kvs_graph_launch")

    def destroy(self):
        if self.handle:
            _check(self._lib.kvs_graph_destroy(self.handle), "kvs_graph_destroy")
            self.handle = None
