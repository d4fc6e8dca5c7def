"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/fpstok.h declares, and rejects invalid arguments on
the host before touching the device (no compute call is made here)."""
import ctypes
import os

import pytest

from point_cloud_tokenization_amd import build as fbuild
from point_cloud_tokenization_amd import fpstok as F


@pytest.fixture(scope="module")
def L():
    if fbuild.is_stale():
        fbuild.build()
    return F.lib()


def test_exports_every_declared_symbol(L):
    names = F.declared_functions()
    assert len(names) >= 10
    for name in ["fpstok_sample", "fpstok_assign", "fpstok_knn", "fpstok_lloyd", "fpstok_pool"]:
        assert name in names
    for name in names:
        assert hasattr(L, name), name


def test_only_the_abi_is_exported(L):
    import subprocess

    out = subprocess.run(["nm", "-D", "--defined-only", F.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted({ln.split()[-1] for ln in out.splitlines()
                       if " T " in ln and ln.split()[-1].startswith("fpstok_")})
    assert exported == F.declared_functions()


def test_version_and_strings(L):
    assert L.fpstok_version() == 3
    assert L.fpstok_status_string(0) == b"ok"
    assert L.fpstok_status_string(2) == b"workspace too small"
    assert L.fpstok_status_string(99) == b"unknown status"


def _bt(B=3, N=100, coords=0x10000, offsets=0x20000, features=0x30000, C=6, q=5, cd=F.F32,
        fd=F.F32):
    return F.Batch(coords, features, offsets, B, N, C, q, 0, cd, fd)


def test_batch_struct_matches_the_header():
    """coords, features, offsets, B, N, C, charge_col, max_event_points,
    coords_dtype, features_dtype: 64 bytes, the dtypes last."""
    assert ctypes.sizeof(F.Batch) == 64
    assert F.Batch.coords_dtype.offset == 56 and F.Batch.features_dtype.offset == 60


def test_workspace_size(L):
    pr = F.make_params()
    assert F.workspace_size(_bt(B=0, N=0), pr) == 0
    a = F.workspace_size(_bt(B=4, N=4250), pr)
    b = F.workspace_size(_bt(B=4, N=8500), pr)
    assert a > 12 * 4250 and b > a and a % 256 == 0
    assert L.fpstok_workspace_size(None, None) == 0
    # 16-bit inputs add their float32 copies: N*4 floats of coordinates, N*C
    # of features (each rounded up to 256 bytes)
    up = lambda n: (n + 255) // 256 * 256
    assert F.workspace_size(_bt(B=4, N=4250, cd=F.F16), pr) == a + up(4250 * 16)
    assert F.workspace_size(_bt(B=4, N=4250, fd=F.BF16), pr) == a + up(4250 * 6 * 4)
    assert F.workspace_size(_bt(B=4, N=4250, cd=F.BF16, fd=F.F16), pr) == \
        a + up(4250 * 16) + up(4250 * 24)


FAKE = ctypes.c_void_p(0x40000)


def _sample(L, bt, pr, ws_bytes=1 << 30, cidx=FAKE, cen=FAKE, tc=FAKE, ws=FAKE):
    return L.fpstok_sample(ctypes.byref(bt), ctypes.byref(pr), None, cidx, cen, tc, None, ws,
                           ws_bytes, None)


@pytest.mark.parametrize("mutate,expect", [
    (lambda bt, pr: setattr(pr, "num_patches", 0), F.EINVAL),
    (lambda bt, pr: setattr(pr, "num_patches", 1025), F.EINVAL),
    (lambda bt, pr: setattr(pr, "assign_mode", 7), F.EINVAL),
    (lambda bt, pr: (setattr(pr, "assign_mode", 1), setattr(pr, "k", 0)), F.EINVAL),
    (lambda bt, pr: (setattr(pr, "assign_mode", 1), setattr(pr, "k", 65)), F.EINVAL),
    (lambda bt, pr: setattr(pr, "lloyd_iters", -1), F.EINVAL),
    (lambda bt, pr: setattr(pr, "pool_weighted", 2), F.EINVAL),
    (lambda bt, pr: setattr(bt, "num_events", -1), F.EINVAL),
    (lambda bt, pr: setattr(bt, "num_points", -5), F.EINVAL),
    (lambda bt, pr: setattr(bt, "num_points", 1 << 31), F.EUNSUPPORTED),
    (lambda bt, pr: setattr(bt, "offsets", None), F.EINVAL),
    (lambda bt, pr: setattr(bt, "coords", None), F.EINVAL),
    (lambda bt, pr: setattr(bt, "coords", 0x10004), F.EINVAL),  # misaligned
    (lambda bt, pr: setattr(bt, "coords_dtype", 3), F.EINVAL),
    (lambda bt, pr: setattr(bt, "coords_dtype", -1), F.EINVAL),
    (lambda bt, pr: setattr(bt, "features_dtype", 3), F.EINVAL),
    # 16-bit coordinates need 8-byte alignment only
    (lambda bt, pr: (setattr(bt, "coords_dtype", F.F16), setattr(bt, "coords", 0x10004)),
     F.EINVAL),
])
def test_sample_rejects_bad_arguments(L, mutate, expect):
    bt, pr = _bt(), F.make_params()
    mutate(bt, pr)
    assert _sample(L, bt, pr) == expect
    assert L.fpstok_last_error() != b""


def test_upcast_rejects_bad_arguments(L):
    assert L.fpstok_upcast(FAKE, -1, F.F16, FAKE, None) == F.EINVAL
    assert L.fpstok_upcast(FAKE, 4, F.F32, FAKE, None) == F.EINVAL
    assert L.fpstok_upcast(FAKE, 4, 3, FAKE, None) == F.EINVAL
    assert L.fpstok_upcast(None, 4, F.F16, FAKE, None) == F.EINVAL
    assert L.fpstok_upcast(FAKE, 4, F.BF16, None, None) == F.EINVAL
    assert L.fpstok_upcast(ctypes.c_void_p(0x40001), 4, F.BF16, FAKE, None) == F.EINVAL
    assert L.fpstok_upcast(FAKE, 4, F.BF16, ctypes.c_void_p(0x40002), None) == F.EINVAL
    assert L.fpstok_upcast(None, 0, F.F16, None, None) == F.OK  # nothing to do


def test_validate_rejects_unknown_dtypes(L):
    assert L.fpstok_validate(ctypes.byref(_bt(B=0, N=0, cd=5)), None) == F.EINVAL
    assert L.fpstok_validate(ctypes.byref(_bt(B=0, N=0, fd=-2)), None) == F.EINVAL


def test_sample_rejects_missing_outputs_and_workspace(L):
    bt, pr = _bt(), F.make_params()
    assert _sample(L, bt, pr, cidx=None) == F.EINVAL
    assert _sample(L, bt, pr, cen=ctypes.c_void_p(0x40004)) == F.EINVAL
    need = F.workspace_size(bt, pr)
    assert _sample(L, bt, pr, ws_bytes=need - 1) == F.EWORKSPACE
    assert _sample(L, bt, pr, ws=None) == F.EWORKSPACE
    assert _sample(L, bt, pr, ws=ctypes.c_void_p(0x40010)) == F.EINVAL  # not 256-aligned


def test_empty_batch_is_a_noop(L):
    bt, pr = _bt(B=0, N=0, coords=None, offsets=None, features=None), F.make_params()
    assert _sample(L, bt, pr, cidx=None, cen=None, tc=None, ws=None, ws_bytes=0) == F.OK
    assert L.fpstok_knn(ctypes.byref(bt), ctypes.byref(F.make_params(k=4)), None, None, None,
                        None, 0, None) == F.OK
    assert L.fpstok_lloyd(ctypes.byref(bt), ctypes.byref(pr), None, None, None, None, 0,
                          None) == F.OK
    assert L.fpstok_pool(ctypes.byref(bt), ctypes.byref(pr), None, None, None, None, None, None,
                         0, None) == F.OK
    assert L.fpstok_assign(ctypes.byref(bt), ctypes.byref(pr), None, None, None, None, 0,
                           None) == F.OK


def test_other_calls_reject_bad_arguments(L):
    bt, pr = _bt(), F.make_params()
    b, p = ctypes.byref(bt), ctypes.byref(pr)
    # knn: k must be in range even in Voronoi-mode params
    assert L.fpstok_knn(b, ctypes.byref(F.make_params(k=0)), FAKE, FAKE, FAKE, FAKE, 1 << 30,
                        None) == F.EINVAL
    assert L.fpstok_knn(b, ctypes.byref(F.make_params(k=4)), None, FAKE, FAKE, FAKE, 1 << 30,
                        None) == F.EINVAL
    # assign: missing output
    assert L.fpstok_assign(b, p, FAKE, FAKE, None, FAKE, 1 << 30, None) == F.EINVAL
    # lloyd: charge column out of range
    bad = _bt(q=6)
    assert L.fpstok_lloyd(ctypes.byref(bad), ctypes.byref(F.make_params(lloyd_iters=2)), FAKE,
                          FAKE, FAKE, FAKE, 1 << 30, None) == F.EINVAL
    # lloyd with L = 0 is a no-op even with NULL buffers
    assert L.fpstok_lloyd(b, p, None, None, None, None, 0, None) == F.OK
    # pool: Voronoi needs assign, kNN needs knn_idx, features required
    assert L.fpstok_pool(b, p, FAKE, None, None, FAKE, None, FAKE, 1 << 30, None) == F.EINVAL
    knnp = ctypes.byref(F.make_params(assign_mode=1, k=4))
    assert L.fpstok_pool(b, knnp, FAKE, None, None, FAKE, None, FAKE, 1 << 30, None) == F.EINVAL
    nof = _bt(features=None)
    assert L.fpstok_pool(ctypes.byref(nof), p, FAKE, FAKE, None, FAKE, None, FAKE, 1 << 30,
                         None) == F.EINVAL
    assert L.fpstok_pool(ctypes.byref(_bt(C=0)), p, FAKE, FAKE, None, FAKE, None, FAKE, 1 << 30,
                         None) == F.EINVAL


def test_noalloc_rejects_batches_beyond_its_scratch_region(L):
    """The size check comes before any HIP call: a batch whose workspace is
    larger than the fixed region is refused with nothing enqueued."""
    pr = F.make_params(num_patches=1024)
    big = _bt(B=100, N=3_000_000)
    assert F.workspace_size(big, pr) > F.NOALLOC_MAX_WORKSPACE
    args = (None, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None)
    assert L.fpstok_tokenize_noalloc(ctypes.byref(big), ctypes.byref(pr), *args) == \
        F.EUNSUPPORTED
    assert b"scratch region" in L.fpstok_last_error()
    # argument errors are still found first
    assert L.fpstok_tokenize_noalloc(ctypes.byref(big), ctypes.byref(pr), None, None, FAKE, FAKE,
                                     FAKE, None, FAKE, None, None) == F.EINVAL
    empty = _bt(B=0, N=0)
    assert L.fpstok_tokenize_noalloc(ctypes.byref(empty), ctypes.byref(pr), *args) == F.OK


def test_device_status_rejects_bad_workspace(L):
    assert L.fpstok_device_status(None, 1 << 20, None) == F.EINVAL
    assert L.fpstok_last_error() != b""
    assert L.fpstok_device_status(FAKE, 255, None) == F.EINVAL
    assert L.fpstok_status_string(F.EDEVICE) == b"device-side failure"


def test_validate_rejects_null_batch(L):
    assert L.fpstok_validate(None, None) == F.EINVAL
    bt = _bt(B=0, N=0)
    assert L.fpstok_validate(ctypes.byref(bt), None) == F.OK


def test_python_binding_refuses_cpu_tensors():
    import torch

    x = torch.zeros((4, 4), dtype=torch.float32)
    off = torch.tensor([0, 4], dtype=torch.int64)
    with pytest.raises(ValueError):
        F.make_batch(x, off)
    with pytest.raises(TypeError):
        F.make_batch(x.double(), off)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(F, "LIB_PATH", os.path.join(str(tmp_path), "missing.so"))
    monkeypatch.setattr(F, "_lib", None)
    with pytest.raises(RuntimeError):
        F.lib()
