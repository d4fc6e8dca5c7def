"""GPU parity for 16-bit inputs (float16 coordinates, bfloat16 features and
the other way round): the library upcasts them exactly to float32, so every
output equals the oracle run on the upcast values (the oracle's own upcast,
pinned exhaustively on the CPU) and equals, bit for bit, the library's float32
path given those same float32 values.  Pull Request #923 ("Add Neptune
point-transformer backbone") lists low-precision tests among what it adds, and
its review settles that FPS runs in float32 whatever the input dtype."""
import numpy as np
import pytest

from point_cloud_tokenization_amd import synth
from tests.gpu_util import assert_close_scaled, log, member_scale, to_dev, to_np

pytestmark = pytest.mark.gpu

F16, BF16 = 1, 2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from point_cloud_tokenization_amd import fpstok as F

    F.lib()


def _bits(a, dtype):
    """uint16 bit patterns of float32 array `a` rounded to `dtype` (torch's
    round-to-nearest-even on the CPU; the rounding itself is not under test)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
    t = t.to(torch.float16 if dtype == F16 else torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _dev16(bits, dtype):
    import torch

    t = to_dev(bits.view(np.int16))
    return t.view(torch.float16 if dtype == F16 else torch.bfloat16)


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_upcast_every_bit_pattern(oracle_mod, dtype):
    import torch
    from point_cloud_tokenization_amd import fpstok as F

    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    src = _dev16(bits, dtype)
    out = torch.empty(bits.size, dtype=torch.float32, device="cuda:0")
    F.upcast(src, out)
    torch.cuda.synchronize()
    got = to_np(out)
    ref = oracle_mod.upcast(bits, dtype)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.array_equal(np.signbit(got[nan]), np.signbit(ref[nan]))
    log("upcast dtype=%d: %d values bit-exact, %d NaN" % (dtype, int((~nan).sum()),
                                                          int(nan.sum())))


def _run(x, f, off, P, mode, k, L, weighted, stepwise=False):
    from point_cloud_tokenization_amd import fpstok as F

    tok = F.Tokenizer(x, f, off, num_patches=P, assign_mode="knn" if mode else "voronoi", k=k,
                      lloyd_iters=L, pool="charge" if weighted else "mean",
                      charge_col=synth.CHARGE_COL)
    out = tok.stepwise() if stepwise else tok()
    tok.check()
    return {key: to_np(v) for key, v in out.items() if v is not None}


@pytest.mark.parametrize("name", ["tiny_uniform", "icecube_b64_voronoi", "icecube_b64_knn16",
                                  "icecube_b256_lloyd3"])
@pytest.mark.parametrize("cd,fd", [(F16, BF16), (BF16, F16)])
@pytest.mark.parametrize("stepwise", [False, True])
def test_tokenize_low_precision(oracle_mod, name, cd, fd, stepwise):
    w = synth.WORKLOADS[name]
    b = synth.make_batch(name, synth.parity_seed(name, 0))
    P, mode, k, L, wt, q = w["P"], w["mode"], w["k"], w["L"], w["weighted"], synth.CHARGE_COL
    log("low-precision case %s coords=%d features=%d stepwise=%d" % (name, cd, fd, stepwise))
    cb, fb = _bits(b["coords"], cd), _bits(b["features"], fd)
    x32, f32 = oracle_mod.upcast(cb, cd), oracle_mod.upcast(fb, fd)
    assert np.isfinite(x32).all() and (f32[:, q] >= 0).all()
    off = to_dev(b["offsets"])
    got = _run(_dev16(cb, cd), _dev16(fb, fd), off, P, mode, k, L, wt, stepwise)
    # the float32 path on the same values, bit for bit
    same = _run(to_dev(x32), to_dev(f32), off, P, mode, k, L, wt, stepwise)
    assert got.keys() == same.keys()
    for key in got:
        assert np.array_equal(got[key].view(np.uint8), same[key].view(np.uint8)), key
    # and the oracle on the upcast values
    ref = oracle_mod.tokenize(x32, f32, b["offsets"], P=P, mode=mode, k=k, L=L, weighted=wt,
                              charge_col=q)
    for key in ("token_count", "centroid_idx", "cell_count"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    if mode == 0 or L > 0:
        np.testing.assert_array_equal(got["assign"], ref["assign"])
    if mode == 1:
        np.testing.assert_array_equal(got["knn_idx"], ref["knn_idx"])
    wv = f32[:, q] if wt else np.ones(x32.shape[0], np.float32)
    scale = member_scale(f32, b["offsets"], P, wv, mode, assign=ref["assign"],
                         knn_idx=ref["knn_idx"])
    assert_close_scaled(got["pooled"], ref["pooled"], scale, "pooled")
    cscale = member_scale(x32, b["offsets"], P, f32[:, q], 0, assign=ref["assign"])
    assert_close_scaled(got["centroids"], ref["centroids"], cscale, "centroids")


def test_pool_backward_takes_16_bit_features(oracle_mod):
    """The gradient call reads bfloat16 features through the same upcast;
    its float32 gradient equals the float32 call's bit for bit."""
    import torch
    from point_cloud_tokenization_amd import fpstok as F

    b = synth.make_batch("icecube_b64_voronoi", synth.parity_seed("icecube_b64_voronoi", 1))
    fb = _bits(b["features"], BF16)
    f32 = oracle_mod.upcast(fb, BF16)
    x, off = to_dev(b["coords"]), to_dev(b["offsets"])
    grads = []
    for feats in (_dev16(fb, BF16), to_dev(f32)):
        tok = F.Tokenizer(x, feats, off, num_patches=128, charge_col=synth.CHARGE_COL)
        o = tok()
        gp = torch.ones_like(o["pooled"])
        gf = torch.empty(f32.shape, dtype=torch.float32, device="cuda:0")
        F.pool_backward(tok.bt, tok.pr, o["token_count"], o["assign"], None, o["pooled"], gp, gf,
                        tok.ws)
        tok.check()
        grads.append(to_np(gf))
    assert np.array_equal(grads[0].view(np.uint32), grads[1].view(np.uint32))
