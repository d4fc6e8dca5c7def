"""Oracle for the FPS tokenizer -- TEST INFRASTRUCTURE ONLY.

A plain, slow, single-threaded C implementation (``fpstok_oracle.c``) of what
the tokenizer computes, wrapped with ctypes for numpy arrays.  It decides the
correct answer in the parity tests.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it; the GPU library and
its Python binding never do, and the two share no code.

Parity pins: every function here is pinned in ``tests/test_oracle_pins.py``
against brute force on tiny events, hand-derived closed forms and invariants
(see that module's docstring).  No function is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fpstok_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_fpstok.so")

# -ffp-contract=off: no fused multiply-add, every float32 operation rounded on
# its own; no -ffast-math; x86-64 computes float in SSE (no excess precision).
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc; returns the path of the shared library."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        i32 = ctypes.c_int32
        lib.oracle_sample.argtypes = [P, P, i64, i32, P, P, P, P, P]
        lib.oracle_assign.argtypes = [P, P, i64, i32, P, P, P]
        lib.oracle_knn.argtypes = [P, P, i64, i32, i32, P, P, P]
        lib.oracle_lloyd.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, P, P]
        lib.oracle_pool.argtypes = [P, P, i64, i32, i32, i32, i32, i32, i32, P, P, P, P, P]
        lib.oracle_tokenize.argtypes = [P, P, P, i64, i32, i32, i32, i32, i32, i32, i32, P,
                                        P, P, P, P, P, P, P]
        lib.oracle_pack.argtypes = [P, i64, i32, i32, P, P, P, P]
        lib.oracle_unpack.argtypes = [P, i64, i32, i32, P, P, P]
        lib.oracle_pool_backward.argtypes = [P, P, i64, i32, i32, i32, i32, i32, i32, P, P, P,
                                             P, P, P]
        lib.oracle_philox4x32_10.argtypes = [P, P, P]
        lib.oracle_philox4x32_10.restype = None
        lib.oracle_random_start.argtypes = [P, i64, ctypes.c_uint64, ctypes.c_uint64, P]
        lib.oracle_upcast.argtypes = [P, i64, i32, P]
        for f in ("oracle_sample", "oracle_assign", "oracle_knn", "oracle_lloyd",
                  "oracle_pool", "oracle_tokenize", "oracle_pack", "oracle_unpack",
                  "oracle_pool_backward", "oracle_random_start", "oracle_upcast"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a, cols):
    a = np.ascontiguousarray(a, dtype=np.float32)
    if a.ndim != 2 or a.shape[1] != cols:
        raise ValueError("expected [N,%d] float32" % cols)
    return a


def _offs(offsets):
    o = np.ascontiguousarray(offsets, dtype=np.int64)
    if o.ndim != 1 or o.size < 1 or o[0] != 0 or np.any(np.diff(o) < 0):
        raise ValueError("offsets must be non-decreasing, start at 0")
    return o


def _check(rc, what):
    if rc != 0:
        raise RuntimeError("oracle %s failed with code %d" % (what, rc))


def sample(coords, offsets, P, start_idx=None, with_assign=True):
    """FPS / pass-through for every event.  Returns (centroid_idx [B,P] i32,
    centroids [B,P,4] f32, token_count [B] i32, assign [N] i32 or None)."""
    x = _f32(coords, 4)
    o = _offs(offsets)
    B = o.size - 1
    if o[-1] != x.shape[0]:
        raise ValueError("offsets[-1] != N")
    sel = np.empty((B, P), np.int32)
    cen = np.empty((B, P, 4), np.float32)
    tc = np.empty(B, np.int32)
    asg = np.empty(x.shape[0], np.int32) if with_assign else None
    st = None if start_idx is None else np.ascontiguousarray(start_idx, dtype=np.int32)
    _check(_load().oracle_sample(_ptr(x), _ptr(o), B, P, _ptr(st), _ptr(sel), _ptr(cen),
                                 _ptr(tc), _ptr(asg)), "sample")
    return sel, cen, tc, asg


def assign(coords, offsets, P, centroids, token_count):
    """Nearest-centroid slot of every pulse ([N] int32)."""
    x = _f32(coords, 4)
    o = _offs(offsets)
    B = o.size - 1
    cen = np.ascontiguousarray(centroids, dtype=np.float32).reshape(B, P, 4)
    tc = np.ascontiguousarray(token_count, dtype=np.int32)
    out = np.empty(x.shape[0], np.int32)
    _check(_load().oracle_assign(_ptr(x), _ptr(o), B, P, _ptr(cen), _ptr(tc), _ptr(out)),
           "assign")
    return out


def knn(coords, offsets, P, k, centroids, token_count):
    """k nearest pulses of each token ([B,P,k] int32, -1 padded)."""
    x = _f32(coords, 4)
    o = _offs(offsets)
    B = o.size - 1
    cen = np.ascontiguousarray(centroids, dtype=np.float32).reshape(B, P, 4)
    tc = np.ascontiguousarray(token_count, dtype=np.int32)
    out = np.empty((B, P, k), np.int32)
    _check(_load().oracle_knn(_ptr(x), _ptr(o), B, P, k, _ptr(cen), _ptr(tc), _ptr(out)),
           "knn")
    return out


def lloyd(coords, features, offsets, P, L, centroids, token_count, assign_in, charge_col):
    """L Lloyd rounds; returns new (centroids, assign) (inputs are not modified)."""
    x = _f32(coords, 4)
    o = _offs(offsets)
    B = o.size - 1
    f = np.ascontiguousarray(features, dtype=np.float32)
    C = f.shape[1] if f.ndim == 2 else 0
    cen = np.array(centroids, dtype=np.float32, copy=True).reshape(B, P, 4)
    asg = np.array(assign_in, dtype=np.int32, copy=True)
    tc = np.ascontiguousarray(token_count, dtype=np.int32)
    _check(_load().oracle_lloyd(_ptr(x), _ptr(f), _ptr(o), B, C, charge_col, P, L, _ptr(cen),
                                _ptr(tc), _ptr(asg)), "lloyd")
    return cen, asg


def pool(features, offsets, P, token_count, mode=0, assign=None, knn_idx=None, k=1,
         weighted=True, charge_col=-1):
    """Per-token (weighted) mean of the features; returns (pooled [B,P,C] f32,
    cell_count [B,P] i32)."""
    f = np.ascontiguousarray(features, dtype=np.float32)
    o = _offs(offsets)
    B = o.size - 1
    C = f.shape[1]
    tc = np.ascontiguousarray(token_count, dtype=np.int32)
    a = None if assign is None else np.ascontiguousarray(assign, dtype=np.int32)
    kn = None if knn_idx is None else np.ascontiguousarray(knn_idx, dtype=np.int32)
    if mode == 0 and a is None:
        raise ValueError("Voronoi pooling needs assign")
    if mode == 1 and kn is None:
        raise ValueError("kNN pooling needs knn_idx")
    out = np.empty((B, P, C), np.float32)
    cnt = np.empty((B, P), np.int32)
    _check(_load().oracle_pool(_ptr(f), _ptr(o), B, C, charge_col, P, mode, k, int(weighted),
                               _ptr(tc), _ptr(a), _ptr(kn), _ptr(out), _ptr(cnt)), "pool")
    return out, cnt


def tokenize(coords, features, offsets, P=128, mode=0, k=16, L=0, weighted=True,
             charge_col=-1, start_idx=None):
    """The whole tokenizer; returns a dict of numpy arrays."""
    x = _f32(coords, 4)
    f = np.ascontiguousarray(features, dtype=np.float32)
    o = _offs(offsets)
    B = o.size - 1
    C = f.shape[1]
    N = x.shape[0]
    out = dict(
        centroid_idx=np.empty((B, P), np.int32),
        centroids=np.empty((B, P, 4), np.float32),
        token_count=np.empty(B, np.int32),
        assign=np.empty(N, np.int32),
        knn_idx=np.empty((B, P, k), np.int32) if mode == 1 else None,
        pooled=np.empty((B, P, C), np.float32),
        cell_count=np.empty((B, P), np.int32),
    )
    st = None if start_idx is None else np.ascontiguousarray(start_idx, dtype=np.int32)
    _check(_load().oracle_tokenize(
        _ptr(x), _ptr(f), _ptr(o), B, C, charge_col, P, mode, k, L, int(weighted), _ptr(st),
        _ptr(out["centroid_idx"]), _ptr(out["centroids"]), _ptr(out["token_count"]),
        _ptr(out["assign"]), _ptr(out["knn_idx"]), _ptr(out["pooled"]),
        _ptr(out["cell_count"])), "tokenize")
    return out


def pack(token_count, rows):
    """Tokens of every event packed event after event (next to the path:
    variable-length attention).  rows [B,P,D]; returns (packed [sum T, D] f32,
    doc_id [sum T] i32, cu_seqlens [B+1] i32)."""
    r = np.ascontiguousarray(rows, dtype=np.float32)
    if r.ndim != 3:
        raise ValueError("rows must be [B,P,D]")
    B, P, D = r.shape
    tc = np.ascontiguousarray(token_count, dtype=np.int32)
    total = int(np.clip(tc, 0, P).sum()) if B else 0
    packed = np.empty((max(total, 0), D), np.float32)
    doc = np.empty(max(total, 0), np.int32)
    cu = np.empty(B + 1, np.int32)
    _check(_load().oracle_pack(_ptr(tc), B, P, D, _ptr(r), _ptr(packed), _ptr(doc), _ptr(cu)),
           "pack")
    return packed, doc, cu


def unpack(token_count, cu_seqlens, packed, P):
    """Inverse of pack: rows [B,P,D], zero beyond each event's tokens."""
    tc = np.ascontiguousarray(token_count, dtype=np.int32)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    pk = np.ascontiguousarray(packed, dtype=np.float32)
    B = tc.size
    D = pk.shape[1] if pk.ndim == 2 else 0
    rows = np.empty((B, P, D), np.float32)
    _check(_load().oracle_unpack(_ptr(tc), B, P, D, _ptr(cu), _ptr(pk), _ptr(rows)), "unpack")
    return rows


def pool_backward(features, offsets, P, token_count, pooled, grad_pooled, mode=0, assign=None,
                  knn_idx=None, k=1, weighted=True, charge_col=-1):
    """Gradient of pool() with respect to the features ([N,C] f32), given the
    gradient of the loss with respect to its output and the output itself."""
    f = np.ascontiguousarray(features, dtype=np.float32)
    o = _offs(offsets)
    B = o.size - 1
    C = f.shape[1]
    tc = np.ascontiguousarray(token_count, dtype=np.int32)
    a = None if assign is None else np.ascontiguousarray(assign, dtype=np.int32)
    kn = None if knn_idx is None else np.ascontiguousarray(knn_idx, dtype=np.int32)
    if mode == 0 and a is None:
        raise ValueError("Voronoi mode needs assign")
    if mode == 1 and kn is None:
        raise ValueError("kNN mode needs knn_idx")
    pm = np.ascontiguousarray(pooled, dtype=np.float32).reshape(B, P, C)
    g = np.ascontiguousarray(grad_pooled, dtype=np.float32).reshape(B, P, C)
    out = np.empty((f.shape[0], C), np.float32)
    _check(_load().oracle_pool_backward(_ptr(f), _ptr(o), B, C, charge_col, P, mode, k,
                                        int(weighted), _ptr(tc), _ptr(a), _ptr(kn), _ptr(pm),
                                        _ptr(g), _ptr(out)), "pool_backward")
    return out


def philox4x32_10(counter, key):
    """One block of Philox4x32-10 (4 words) for a 4-word counter and 2-word key."""
    c = np.ascontiguousarray(counter, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.empty(4, np.uint32)
    _load().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def random_start(offsets, seed, step=0):
    """A random FPS start per event ([B] int32) from Philox4x32-10."""
    o = _offs(offsets)
    B = o.size - 1
    out = np.empty(B, np.int32)
    _check(_load().oracle_random_start(_ptr(o), B, int(seed) & (2**64 - 1),
                                       int(step) & (2**64 - 1), _ptr(out)), "random_start")
    return out


F16, BF16 = 1, 2


def upcast(bits, dtype):
    """The float32 values of 16-bit inputs given as their bit patterns (any
    shape of uint16): dtype F16 (IEEE binary16) or BF16 (bfloat16).  Exact:
    every such value is a float32 value.  Low-precision coordinates or
    features go through this, then through the float32 functions above."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, np.float32)
    _check(_load().oracle_upcast(_ptr(b), b.size, int(dtype), _ptr(out)), "upcast")
    return out
