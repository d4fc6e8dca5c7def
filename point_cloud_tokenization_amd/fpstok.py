"""ctypes binding of libfpstok (include/fpstok.h).

Argument marshalling only: PyTorch supplies device memory and the current
HIP stream; every step of the tokenizer runs in the library's gfx950 kernels.
The library must have been built (``__graft_entry__.build()`` or
``python -m point_cloud_tokenization_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfpstok.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "fpstok.h")

OK, EINVAL, EWORKSPACE, EUNSUPPORTED, EHIP, EDEVICE = 0, 1, 2, 3, 4, 5
VORONOI, KNN = 0, 1
F32, F16, BF16 = 0, 1, 2  # fpstok_dtype
MAX_PATCHES, MAX_K, MAX_LLOYD = 1024, 64, 1000
NOALLOC_MAX_WORKSPACE = 64 << 20  # FPSTOK_NOALLOC_MAX_WORKSPACE


class FpstokError(RuntimeError):
    def __init__(self, status, where, detail):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (where, _STATUS.get(status, status), detail))


_STATUS = {OK: "ok", EINVAL: "invalid argument", EWORKSPACE: "workspace too small",
           EUNSUPPORTED: "unsupported", EHIP: "HIP runtime error",
           EDEVICE: "device-side failure"}


class Batch(ctypes.Structure):
    _fields_ = [("coords", ctypes.c_void_p), ("features", ctypes.c_void_p),
                ("offsets", ctypes.c_void_p), ("num_events", ctypes.c_int64),
                ("num_points", ctypes.c_int64), ("num_features", ctypes.c_int32),
                ("charge_col", ctypes.c_int32), ("max_event_points", ctypes.c_int64),
                ("coords_dtype", ctypes.c_int32), ("features_dtype", ctypes.c_int32)]


class Params(ctypes.Structure):
    _fields_ = [("num_patches", ctypes.c_int32), ("k", ctypes.c_int32),
                ("lloyd_iters", ctypes.c_int32), ("assign_mode", ctypes.c_int32),
                ("pool_weighted", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded libfpstok (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libfpstok.so is not built (%s); run __graft_entry__.build()"
                               % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        B, Pp = ctypes.POINTER(Batch), ctypes.POINTER(Params)
        L.fpstok_workspace_size.argtypes = [B, Pp]
        L.fpstok_workspace_size.restype = sz
        L.fpstok_sample.argtypes = [B, Pp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.fpstok_assign.argtypes = [B, Pp, vp, vp, vp, vp, sz, vp]
        L.fpstok_knn.argtypes = [B, Pp, vp, vp, vp, vp, sz, vp]
        L.fpstok_lloyd.argtypes = [B, Pp, vp, vp, vp, vp, sz, vp]
        L.fpstok_pool.argtypes = [B, Pp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.fpstok_tokenize.argtypes = [B, Pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.fpstok_tokenize_noalloc.argtypes = [B, Pp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.fpstok_validate.argtypes = [B, vp]
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        L.fpstok_pack.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp, vp]
        L.fpstok_unpack.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp]
        L.fpstok_pool_backward.argtypes = [B, Pp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.fpstok_random_start.argtypes = [vp, i64, ctypes.c_uint64, ctypes.c_uint64, vp, vp]
        L.fpstok_device_status.argtypes = [vp, sz, vp]
        L.fpstok_debug_set_spin_limit.argtypes = [ctypes.c_uint32]
        L.fpstok_debug_set_spin_limit.restype = None
        L.fpstok_upcast.argtypes = [vp, i64, i32, vp, vp]
        for f in ("fpstok_sample", "fpstok_assign", "fpstok_knn", "fpstok_lloyd",
                  "fpstok_pool", "fpstok_tokenize", "fpstok_validate", "fpstok_pack",
                  "fpstok_unpack", "fpstok_pool_backward", "fpstok_random_start",
                  "fpstok_device_status", "fpstok_tokenize_noalloc", "fpstok_upcast"):
            getattr(L, f).restype = ctypes.c_int
        L.fpstok_status_string.argtypes = [ctypes.c_int]
        L.fpstok_status_string.restype = ctypes.c_char_p
        L.fpstok_last_error.argtypes = []
        L.fpstok_last_error.restype = ctypes.c_char_p
        L.fpstok_version.argtypes = []
        L.fpstok_version.restype = ctypes.c_int
        _lib = L
    return _lib


def declared_functions():
    """Names of the functions include/fpstok.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fpstok_[a-z_]+)\s*\(", text)))


def _check(rc, where):
    if rc != OK:
        raise FpstokError(rc, where, lib().fpstok_last_error().decode())


def version():
    return lib().fpstok_version()


# ------------------------------------------------------------ tensor helpers

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, name, dev=None):
    import torch

    if t is None:
        raise ValueError("%s is required" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if dev is not None and t.device != dev:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, dev))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _dtype_code(t, name):
    import torch

    codes = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
    if t.dtype not in codes:
        raise TypeError("%s must be float32, float16 or bfloat16, got %s" % (name, t.dtype))
    return codes[t.dtype]


def make_batch(coords, offsets, features=None, charge_col=-1, max_event_points=0):
    """A Batch struct over the given tensors (which the caller keeps alive).
    coords and features may each be float32, float16 or bfloat16; the library
    upcasts 16-bit inputs exactly to float32 before using them.
    max_event_points: optional host-side bound on the pulses of any event (0:
    unknown); see fpstok_batch in include/fpstok.h."""
    import torch

    cd = _dtype_code(coords, "coords")
    _need(coords, coords.dtype, "coords")
    _need(offsets, torch.int64, "offsets", coords.device)
    if coords.dim() != 2 or coords.shape[1] != 4:
        raise ValueError("coords must be [N,4]")
    C, fd = 0, F32
    if features is not None:
        fd = _dtype_code(features, "features")
        _need(features, features.dtype, "features", coords.device)
        if features.dim() != 2 or features.shape[0] != coords.shape[0]:
            raise ValueError("features must be [N,C]")
        C = features.shape[1]
    bt = Batch(coords.data_ptr(), features.data_ptr() if features is not None else None,
               offsets.data_ptr(), offsets.numel() - 1, coords.shape[0], C, charge_col,
               int(max_event_points), cd, fd)
    return bt


def upcast(src, out, stream=None):
    """out[i] = float32 value of the float16 / bfloat16 src[i] (exact)."""
    import torch

    code = _dtype_code(src, "src")
    if code == F32:
        raise TypeError("src must be float16 or bfloat16")
    _need(src, src.dtype, "src")
    _need(out, torch.float32, "out", src.device)
    if out.numel() != src.numel():
        raise ValueError("out must have as many elements as src")
    _check(lib().fpstok_upcast(_ptr(src), src.numel(), code, _ptr(out),
                               _stream_handle(stream)), "fpstok_upcast")


def make_params(num_patches=128, k=16, lloyd_iters=0, assign_mode=VORONOI, pool_weighted=1):
    return Params(num_patches, k, lloyd_iters, assign_mode, pool_weighted)


def workspace_size(bt, pr):
    return lib().fpstok_workspace_size(ctypes.byref(bt), ctypes.byref(pr))


def alloc_workspace(bt, pr, device):
    import torch

    n = workspace_size(bt, pr)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


# ----------------------------------------------------------- the five calls

def sample(bt, pr, centroid_idx, centroids, token_count, assign, ws, start_idx=None,
           stream=None):
    _check(lib().fpstok_sample(ctypes.byref(bt), ctypes.byref(pr), _ptr(start_idx),
                               _ptr(centroid_idx), _ptr(centroids), _ptr(token_count),
                               _ptr(assign), _ptr(ws), ws.numel(), _stream_handle(stream)),
           "fpstok_sample")


def assign(bt, pr, centroids, token_count, out, ws, stream=None):
    _check(lib().fpstok_assign(ctypes.byref(bt), ctypes.byref(pr), _ptr(centroids),
                               _ptr(token_count), _ptr(out), _ptr(ws), ws.numel(),
                               _stream_handle(stream)), "fpstok_assign")


def knn(bt, pr, centroids, token_count, knn_idx, ws, stream=None):
    _check(lib().fpstok_knn(ctypes.byref(bt), ctypes.byref(pr), _ptr(centroids),
                            _ptr(token_count), _ptr(knn_idx), _ptr(ws), ws.numel(),
                            _stream_handle(stream)), "fpstok_knn")


def lloyd(bt, pr, centroids, token_count, assign_, ws, stream=None):
    _check(lib().fpstok_lloyd(ctypes.byref(bt), ctypes.byref(pr), _ptr(centroids),
                              _ptr(token_count), _ptr(assign_), _ptr(ws), ws.numel(),
                              _stream_handle(stream)), "fpstok_lloyd")


def pool(bt, pr, token_count, assign_, knn_idx, pooled, cell_count, ws, stream=None):
    _check(lib().fpstok_pool(ctypes.byref(bt), ctypes.byref(pr), _ptr(token_count),
                             _ptr(assign_), _ptr(knn_idx), _ptr(pooled), _ptr(cell_count),
                             _ptr(ws), ws.numel(), _stream_handle(stream)), "fpstok_pool")


def pool_backward(bt, pr, token_count, assign_, knn_idx, pooled, grad_pooled, grad_features,
                  ws, stream=None):
    """fpstok_pool_backward: gradient of the pooling with respect to the features."""
    _check(lib().fpstok_pool_backward(ctypes.byref(bt), ctypes.byref(pr), _ptr(token_count),
                                      _ptr(assign_), _ptr(knn_idx), _ptr(pooled),
                                      _ptr(grad_pooled), _ptr(grad_features), _ptr(ws),
                                      ws.numel(), _stream_handle(stream)), "fpstok_pool_backward")


def random_start(offsets, start_idx, seed, step=0, stream=None):
    """fpstok_random_start: a random FPS start per event into start_idx [B]
    int32 (offsets [B+1] int64), from Philox4x32-10 with the given seed and
    step."""
    import torch

    _need(offsets, torch.int64, "offsets")
    _need(start_idx, torch.int32, "start_idx")
    B = offsets.numel() - 1
    _check(lib().fpstok_random_start(_ptr(offsets), B, int(seed) & (2**64 - 1),
                                     int(step) & (2**64 - 1), _ptr(start_idx),
                                     _stream_handle(stream)), "fpstok_random_start")


def pack(token_count, rows, packed, doc_id, cu_seqlens, stream=None):
    """fpstok_pack on device tensors: token_count [B] int32, rows [B,P,D]
    float32; packed [B*P,D] float32, doc_id [B*P] int32 (or None) and
    cu_seqlens [B+1] int32 are written."""
    import torch

    B, P, D = rows.shape
    _need(token_count, torch.int32, "token_count")
    _need(rows, torch.float32, "rows")
    _need(packed, torch.float32, "packed")
    _need(cu_seqlens, torch.int32, "cu_seqlens")
    if doc_id is not None:
        _need(doc_id, torch.int32, "doc_id")
    _check(lib().fpstok_pack(B, P, D, _ptr(token_count), _ptr(rows), _ptr(packed), _ptr(doc_id),
                             _ptr(cu_seqlens), _stream_handle(stream)), "fpstok_pack")


def unpack(token_count, cu_seqlens, packed, rows, stream=None):
    """fpstok_unpack: rows [B,P,D] float32 from the packed rows."""
    import torch

    B, P, D = rows.shape
    for t, dt, name in ((token_count, torch.int32, "token_count"),
                        (cu_seqlens, torch.int32, "cu_seqlens"),
                        (packed, torch.float32, "packed"), (rows, torch.float32, "rows")):
        _need(t, dt, name)
    _check(lib().fpstok_unpack(B, P, D, _ptr(token_count), _ptr(cu_seqlens), _ptr(packed),
                               _ptr(rows), _stream_handle(stream)), "fpstok_unpack")


def tokenize_call(bt, pr, centroid_idx, centroids, token_count, assign_, knn_idx, pooled,
                  cell_count, ws, start_idx=None, stream=None):
    """fpstok_tokenize: the whole tokenizer in one call."""
    _check(lib().fpstok_tokenize(ctypes.byref(bt), ctypes.byref(pr), _ptr(start_idx),
                                 _ptr(centroid_idx), _ptr(centroids), _ptr(token_count),
                                 _ptr(assign_), _ptr(knn_idx), _ptr(pooled), _ptr(cell_count),
                                 _ptr(ws), ws.numel(), _stream_handle(stream)), "fpstok_tokenize")


def tokenize_noalloc_call(bt, pr, centroid_idx, centroids, token_count, assign_, knn_idx,
                          pooled, cell_count, start_idx=None, stream=None):
    """fpstok_tokenize_noalloc: the whole tokenizer with the library's fixed
    scratch region as its workspace (no allocation)."""
    _check(lib().fpstok_tokenize_noalloc(ctypes.byref(bt), ctypes.byref(pr), _ptr(start_idx),
                                         _ptr(centroid_idx), _ptr(centroids), _ptr(token_count),
                                         _ptr(assign_), _ptr(knn_idx), _ptr(pooled),
                                         _ptr(cell_count), _stream_handle(stream)),
           "fpstok_tokenize_noalloc")


def validate(bt, stream=None):
    _check(lib().fpstok_validate(ctypes.byref(bt), _stream_handle(stream)), "fpstok_validate")


def device_status(ws, stream=None):
    """fpstok_device_status: raises FpstokError (status EDEVICE) if a bounded
    wait between workgroups gave up in the last sample / tokenize call on the
    workspace tensor `ws`.  Synchronizes the stream."""
    _check(lib().fpstok_device_status(_ptr(ws), ws.numel(), _stream_handle(stream)),
           "fpstok_device_status")


def debug_set_spin_limit(polls):
    """Testing only: polls before a wait between workgroups gives up (0: the
    default)."""
    lib().fpstok_debug_set_spin_limit(int(polls))


# ------------------------------------------------------------- convenience

def offsets_from_batch_ids(batch_ids, num_events):
    """CSR offsets [B+1] from sorted per-pulse event ids (device-side; pass
    num_events to avoid a host sync)."""
    import torch

    counts = torch.bincount(batch_ids, minlength=num_events)
    off = torch.zeros(num_events + 1, dtype=torch.int64, device=batch_ids.device)
    torch.cumsum(counts, 0, out=off[1:])
    return off


class Tokenizer:
    """Preallocated outputs and workspace for one batch shape; call() runs the
    whole tokenizer (sample -> [Lloyd] -> [kNN] -> pool) on the current
    stream without host synchronization."""

    def __init__(self, coords, features, offsets, num_patches=128, assign_mode="voronoi", k=16,
                 lloyd_iters=0, pool="charge", charge_col=-1, max_event_points=0):
        import torch

        self.mode = {"voronoi": VORONOI, "knn": KNN}[assign_mode]
        self.coords, self.features, self.offsets = coords, features, offsets
        self.bt = make_batch(coords, offsets, features, charge_col, max_event_points)
        self.pr = make_params(num_patches, k, lloyd_iters, self.mode,
                              1 if pool == "charge" else 0)
        dev = coords.device
        B, N, P = offsets.numel() - 1, coords.shape[0], num_patches
        C = features.shape[1]
        self.out = dict(
            centroid_idx=torch.empty((B, P), dtype=torch.int32, device=dev),
            centroids=torch.empty((B, P, 4), dtype=torch.float32, device=dev),
            token_count=torch.empty(B, dtype=torch.int32, device=dev),
            # the Voronoi slots are computed in Voronoi mode and for Lloyd
            assign=torch.empty(N, dtype=torch.int32, device=dev)
            if self.mode == VORONOI or lloyd_iters > 0 else None,
            knn_idx=torch.empty((B, P, k), dtype=torch.int32, device=dev)
            if self.mode == KNN else None,
            pooled=torch.empty((B, P, C), dtype=torch.float32, device=dev),
            cell_count=torch.empty((B, P), dtype=torch.int32, device=dev),
        )
        self.ws = alloc_workspace(self.bt, self.pr, dev)
        # the call's fixed arguments, marshalled once; only the stream is
        # looked up per call (torch's current stream on this device)
        o = self.out
        self._fn = lib().fpstok_tokenize
        self._head = (ctypes.byref(self.bt), ctypes.byref(self.pr))
        self._tail = (_ptr(o["centroid_idx"]), _ptr(o["centroids"]), _ptr(o["token_count"]),
                      _ptr(o["assign"]), _ptr(o["knn_idx"]), _ptr(o["pooled"]),
                      _ptr(o["cell_count"]), _ptr(self.ws), self.ws.numel())
        self._dev = dev.index if dev.index is not None else torch.cuda.current_device()
        self._raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)

    def __call__(self, start_idx=None, stream=None):
        """fpstok_tokenize on the preallocated buffers."""
        if stream is None and self._raw_stream is not None:
            rc = self._fn(*self._head, _ptr(start_idx), *self._tail,
                          ctypes.c_void_p(self._raw_stream(self._dev)))
            if rc != OK:
                _check(rc, "fpstok_tokenize")
            return self.out
        o = self.out
        tokenize_call(self.bt, self.pr, o["centroid_idx"], o["centroids"], o["token_count"],
                      o["assign"], o["knn_idx"], o["pooled"], o["cell_count"], self.ws,
                      start_idx, stream)
        return o

    def check(self, stream=None):
        """Raise if the last call's outputs are not valid (fpstok_device_status;
        synchronizes)."""
        device_status(self.ws, stream)

    def stepwise(self, start_idx=None, stream=None):
        """The same result through the five separate calls."""
        o = self.out
        sample(self.bt, self.pr, o["centroid_idx"], o["centroids"], o["token_count"],
               o["assign"], self.ws, start_idx, stream)
        if self.pr.lloyd_iters > 0:
            lloyd(self.bt, self.pr, o["centroids"], o["token_count"], o["assign"], self.ws,
                  stream)
        if self.mode == KNN:
            knn(self.bt, self.pr, o["centroids"], o["token_count"], o["knn_idx"], self.ws,
                stream)
        pool(self.bt, self.pr, o["token_count"], o["assign"], o["knn_idx"], o["pooled"],
             o["cell_count"], self.ws, stream)
        return o


def tokenize(coords, features, offsets=None, batch_ids=None, num_events=None, num_patches=128,
             assign_mode="voronoi", k=16, lloyd_iters=0, pool="charge", charge_col=-1,
             start_idx=None, stream=None):
    """Tokenize one batch: returns a dict of device tensors (centroid_idx,
    centroids, token_count, assign, knn_idx or None, pooled, cell_count)."""
    if offsets is None:
        if batch_ids is None or num_events is None:
            raise ValueError("give offsets, or batch_ids with num_events")
        offsets = offsets_from_batch_ids(batch_ids, num_events)
    t = Tokenizer(coords, features, offsets, num_patches, assign_mode, k, lloyd_iters, pool,
                  charge_col)
    return t(start_idx, stream)
