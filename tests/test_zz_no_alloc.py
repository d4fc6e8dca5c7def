"""fpstok_tokenize_noalloc (the library's fixed scratch region as workspace)
against fpstok_tokenize (a caller workspace) through the C ABI: two calls in
a row on one GPU, the second on a smaller batch, in every mode, and once with
float16 coordinates and bfloat16 features (their float32 copies staged in the
scratch region too); every output must be identical (same kernels, same
inputs)."""
import numpy as np
import pytest

from point_cloud_tokenization_amd import synth

pytestmark = pytest.mark.gpu


def _outputs(b, P, mode, k, dev):
    import torch

    B = b["offsets"].size - 1
    N, C = b["features"].shape
    mk = lambda shape, dt: torch.full(shape, -77, dtype=dt, device=dev)  # noqa: E731
    return dict(centroid_idx=mk((B, P), torch.int32), centroids=mk((B, P, 4), torch.float32),
                token_count=mk((B,), torch.int32), assign=mk((N,), torch.int32),
                knn_idx=mk((B, P, k), torch.int32) if mode == 1 else None,
                pooled=mk((B, P, C), torch.float32), cell_count=mk((B, P), torch.int32))


def _run(b, P, mode, k, L, noalloc, half=False):
    import torch

    from point_cloud_tokenization_amd import fpstok as F

    dev = torch.device("cuda:0")
    x = torch.from_numpy(b["coords"]).to(dev)
    f = torch.from_numpy(b["features"]).to(dev)
    off = torch.from_numpy(b["offsets"]).to(dev)
    if half:
        x, f = x.to(torch.float16), f.to(torch.bfloat16)
    bt = F.make_batch(x, off, f, synth.CHARGE_COL, int(np.diff(b["offsets"]).max()))
    pr = F.make_params(P, k, L, mode, 1)
    o = _outputs(b, P, mode, k, dev)
    args = (o["centroid_idx"], o["centroids"], o["token_count"], o["assign"], o["knn_idx"],
            o["pooled"], o["cell_count"])
    if noalloc:
        F.tokenize_noalloc_call(bt, pr, *args)
    else:
        ws = F.alloc_workspace(bt, pr, dev)
        F.tokenize_call(bt, pr, *args, ws)
        F.device_status(ws)
    torch.cuda.synchronize()
    return {key: v.cpu().numpy() for key, v in o.items() if v is not None}


@pytest.mark.parametrize("first,second,mode,k,L,half", [
    ("icecube_highE_b512", "icecube_b64_voronoi", 0, 16, 0, False),
    ("icecube_b256_lloyd3", "tiny_uniform", 0, 16, 2, False),
    ("icecube_b64_knn16", "tiny_uniform", 1, 16, 0, False),
    ("icecube_b256_lloyd3", "icecube_b64_knn16", 1, 8, 1, False),
    ("icecube_b256_lloyd3", "icecube_b64_voronoi", 0, 16, 1, True),
])
def test_noalloc_matches_workspace_call(first, second, mode, k, L, half):
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    for name in (first, second):  # the second batch is the smaller one
        b = synth.make_batch(name, synth.parity_seed(name, 3))
        P = synth.WORKLOADS[name]["P"]
        print("no-alloc case %s P=%d mode=%d k=%d L=%d half=%d" % (name, P, mode, k, L, half),
              flush=True)
        ref = _run(b, P, mode, k, L, noalloc=False, half=half)
        got = _run(b, P, mode, k, L, noalloc=True, half=half)
        for key in ref:
            np.testing.assert_array_equal(got[key], ref[key], err_msg="%s %s" % (name, key))
