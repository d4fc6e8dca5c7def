"""GPU parity: every libfpstok call, through the C ABI, against the oracle on
the same seeded inputs.  Indices bit-exact; float outputs within the scaled
1e-5 tolerance of tests/gpu_util.py."""
import numpy as np
import pytest

from point_cloud_tokenization_amd import synth
from tests.gpu_util import check_pipeline, log, run_pipeline, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from point_cloud_tokenization_amd import fpstok as F

    F.lib()  # fails loudly when the library was not built


def _params(name):
    w = synth.WORKLOADS[name]
    return dict(P=w["P"], mode=w["mode"], k=w["k"], L=w["L"], weighted=w["weighted"],
                charge_col=synth.CHARGE_COL)


@pytest.mark.parametrize("name,r", [(n, r) for n in synth.WORKLOAD_ORDER for r in range(5)])
def test_workloads(oracle_mod, name, r):
    b = synth.make_batch(name, synth.parity_seed(name, r))
    st = check_pipeline(oracle_mod, b, label="%s/r%d" % (name, r), **_params(name))
    log("exact fractions %s" % st)


@pytest.mark.parametrize("mode,k,L", [(0, 16, 0), (1, 16, 0), (1, 64, 2), (0, 1, 2)])
def test_edge_sizes(oracle_mod, mode, k, L):
    ns = [0, 1, 2, 127, 128, 129, 255, 256, 257, 300, 511, 512, 513, 1023, 1024, 1025, 2047,
          2049, 3071, 3073, 4095, 4096, 4097, 6000, 0, 5]
    b = synth.uniform_events(ns, 77 + mode + L, C=6)
    check_pipeline(oracle_mod, b, P=128, mode=mode, k=k, L=L, label="edge sizes")


@pytest.mark.parametrize("P", [128, 256])
def test_lloyd_wide_bitmaps(oracle_mod, P):
    """Lloyd updates of events between 1025 and 2048 pulses, sorted by slot
    through bitmaps of 9 to 16 128-bit words per slot (kept in the rows'
    upper half), the sizes around both ends of that form, with the slot
    count at and below the bitmaps' capacity, and on a tie-rich grid."""
    ns = [1024, 1025, 1100, 1500, 1900, 2047, 2048, 700]
    b = synth.icecube_events(ns, 640 + P, C=6)
    check_pipeline(oracle_mod, b, P=P, mode=0, L=3, label="lloyd wide bitmaps P=%d" % P)
    g = synth.grid_events([1030, 2040], 650 + P, C=6, side=2)
    check_pipeline(oracle_mod, g, P=P, mode=0, L=2, label="lloyd wide bitmaps grid P=%d" % P)


@pytest.mark.parametrize("P", [1, 2, 7, 64, 256, 1024])
def test_num_patches_range(oracle_mod, P):
    ns = [P - 1 if P > 1 else 0, P, P + 1, 3 * P + 5, 3000]
    b = synth.icecube_events(ns, 100 + P, C=6)
    check_pipeline(oracle_mod, b, P=P, mode=0, L=1, label="P=%d" % P)
    check_pipeline(oracle_mod, b, P=P, mode=1, k=min(64, P + 3), label="P=%d knn" % P)


@pytest.mark.parametrize("side", [1, 2, 3])
def test_tie_rich_grids(oracle_mod, side):
    ns = [10, 130, 600, 2500, 5000]
    b = synth.grid_events(ns, 200 + side, C=6, side=side)
    check_pipeline(oracle_mod, b, P=128, mode=0, L=2, label="grid side %d" % side)
    check_pipeline(oracle_mod, b, P=128, mode=1, k=16, label="grid side %d knn" % side)


def test_identical_clouds(oracle_mod):
    # 400 and 700 pulses: 2 and 3 per lane, the all-zero maximum inside the
    # hand-scheduled loop's exchange
    b = synth.identical_events([5, 129, 400, 700, 1000, 4500], 9, C=6)
    check_pipeline(oracle_mod, b, P=128, mode=0, L=2, label="identical")
    check_pipeline(oracle_mod, b, P=128, mode=1, k=64, label="identical knn")


def test_start_idx_and_unit_charge(oracle_mod):
    b = synth.icecube_events([50, 700, 2000, 3300], 31, C=6)
    n = np.diff(b["offsets"])
    rng = np.random.default_rng(0)
    st = np.array([rng.integers(0, max(1, m)) for m in n], np.int32)
    check_pipeline(oracle_mod, b, P=128, mode=0, L=3, start_idx=st, label="start_idx")
    check_pipeline(oracle_mod, b, P=128, mode=1, k=16, charge_col=-1, label="unit charge")
    check_pipeline(oracle_mod, b, P=128, mode=0, weighted=False, label="plain mean")


def test_large_events(oracle_mod):
    b = synth.icecube_events([60000, 9000, 150], 5, C=6)
    check_pipeline(oracle_mod, b, P=256, mode=0, label="large events")


@pytest.mark.parametrize("n,P", [(691, 128), (5000, 128), (84240, 256)])
def test_single_event_batches(oracle_mod, n, P):
    """A batch of one event: one workgroup, a gang of 2 and a gang of 21
    workgroups with nothing else in the launch (the shape the bench times
    for the critical path); stepwise and fused."""
    b = synth.icecube_events([n], 600 + n % 97, C=6)
    check_pipeline(oracle_mod, b, P=P, mode=0, label="one event n=%d" % n)
    _tokenize_vs_oracle(oracle_mod, b, P, label="one event n=%d fused" % n)


def test_wide_features(oracle_mod):
    b = synth.icecube_events([400, 3000, 20], 8, C=21)
    check_pipeline(oracle_mod, b, P=128, mode=0, L=1, label="C=21")
    check_pipeline(oracle_mod, b, P=128, mode=1, k=8, label="C=21 knn")


def test_standalone_assign(oracle_mod):
    """fpstok_assign is the plain argmin for every event, including events
    with n <= P and centroids that are not pulses."""
    import torch

    from point_cloud_tokenization_amd import fpstok as F

    b = synth.uniform_events([3, 100, 1500, 0, 4000], 13, C=6)
    P = 64
    rng = np.random.default_rng(1)
    B = b["offsets"].size - 1
    cen = rng.uniform(-1, 1, (B, P, 4)).astype(np.float32)
    tc = np.array([3, 64, 64, 0, 17], np.int32)
    x, off = to_dev(b["coords"]), to_dev(b["offsets"])
    bt = F.make_batch(x, off)
    pr = F.make_params(P)
    ws = F.alloc_workspace(bt, pr, x.device)
    out = torch.empty(b["coords"].shape[0], dtype=torch.int32, device=x.device)
    F.assign(bt, pr, to_dev(cen), to_dev(tc), out, ws)
    np.testing.assert_array_equal(to_np(out), oracle_mod.assign(b["coords"], b["offsets"], P,
                                                                cen, tc))


def test_empty_batches(oracle_mod):
    b = synth.uniform_events([0, 0, 0], 1, C=6)
    check_pipeline(oracle_mod, b, P=16, mode=0, label="all empty")
    check_pipeline(oracle_mod, b, P=16, mode=1, k=4, label="all empty knn")


def test_repeatable_bit_for_bit():
    b = synth.make_batch("icecube_b256_lloyd3", 5)
    r1 = run_pipeline(b, 128, 0, 16, 3, True, 5)
    r2 = run_pipeline(b, 128, 0, 16, 3, True, 5)
    for key in r1:
        assert np.array_equal(r1[key], r2[key]), key


def test_gang_and_streaming_paths(oracle_mod):
    """Events split over several workgroups (4096 < n <= 262144) and one
    beyond that (single-workgroup streaming path)."""
    b = synth.icecube_events([4097, 8193, 20000, 262144, 300], 17, C=6)
    check_pipeline(oracle_mod, b, P=256, mode=0, label="gangs")
    b = synth.uniform_events([270000, 5000], 18, C=6)
    check_pipeline(oracle_mod, b, P=64, mode=0, label="streaming")


@pytest.mark.parametrize("P", [128, 300])
def test_candidate_list_overflow(oracle_mod, P):
    """More candidates above the bound than the lists hold: a workgroup's
    64-entry list, a shard's 63 published entries, the gang's 256 entries.
    Every lane holds one far pulse and copies of the seed (stride = pulses
    per lane; 400-768 pulses: the exchange inside the hand-scheduled loop,
    2 and 3 per lane).  With P = 300 the far pulses run out and the all-zero
    rule takes over, in single workgroups and in gangs."""
    ns = [200, 256, 400, 512, 700, 768, 1024, 2048, 4096, 8192, 20000]
    strides = [2, 2, 2, 2, 3, 3, 4, 8, 16, 16, 16]
    b = synth.seed_copies_events(ns, 31 + P, C=6, strides=strides)
    check_pipeline(oracle_mod, b, P=P, mode=0, label="overflow P=%d" % P)
    _tokenize_vs_oracle(oracle_mod, b, P, label="overflow fused P=%d" % P)


def test_graph_replay_matches_eager(oracle_mod):
    """The whole tokenizer captured in a HIP graph: every replay (with eager
    work and synchronizations in between) equals the eager result."""
    import torch

    from point_cloud_tokenization_amd import fpstok as F

    cases = [(name, hint) for name in ("icecube_b64_voronoi", "icecube_b64_knn16",
                                       "icecube_b256_lloyd3") for hint in (False, True)]
    for name, hint in cases:
        b = synth.make_batch(name, 77)
        w = synth.WORKLOADS[name]
        x, f, off = to_dev(b["coords"]), to_dev(b["features"]), to_dev(b["offsets"])
        tok = F.Tokenizer(x, f, off, num_patches=w["P"],
                          assign_mode="knn" if w["mode"] == 1 else "voronoi", k=w["k"],
                          lloyd_iters=w["L"], pool="charge", charge_col=5,
                          max_event_points=int(np.diff(b["offsets"]).max()) if hint else 0)
        ref = {k_: (to_np(v) if v is not None else None) for k_, v in tok().items()}
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            tok()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            tok()
        for rep in range(4):
            for v in tok.out.values():
                if v is not None:
                    v.fill_(-7)
            scratch = torch.randn(1000, device=x.device).sum()  # eager work in between
            g.replay()
            torch.cuda.synchronize()
            float(scratch)
            for k_, v in tok.out.items():
                if v is not None:
                    assert np.array_equal(to_np(v), ref[k_]), (name, hint, rep, k_)
        log("graph replay ok: %s hint=%s" % (name, hint))


def _tokenize_vs_oracle(oracle_mod, b, P, mode=0, k=16, L=0, weighted=True, charge_col=5,
                        stepwise=False, label="", max_event_points=0):
    """fpstok_tokenize (or the five calls) against oracle.tokenize."""
    from point_cloud_tokenization_amd import fpstok as F
    from tests.gpu_util import assert_close_scaled, member_scale

    log("tokenize case %s: B=%d N=%d P=%d mode=%d L=%d stepwise=%d" % (
        label, b["offsets"].size - 1, b["coords"].shape[0], P, mode, L, stepwise))
    x, f, off = to_dev(b["coords"]), to_dev(b["features"]), to_dev(b["offsets"])
    tok = F.Tokenizer(x, f, off, num_patches=P, assign_mode="knn" if mode else "voronoi", k=k,
                      lloyd_iters=L, pool="charge" if weighted else "mean", charge_col=charge_col,
                      max_event_points=max_event_points)
    out = tok.stepwise() if stepwise else tok()
    tok.check()  # no bounded wait between workgroups gave up
    got = {key: to_np(v) for key, v in out.items() if v is not None}
    ref = oracle_mod.tokenize(b["coords"], b["features"], b["offsets"], P=P, mode=mode, k=k, L=L,
                              weighted=weighted, charge_col=charge_col)
    for key in ("token_count", "centroid_idx", "cell_count"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key + " " + label)
    if mode == 0 or L > 0:
        np.testing.assert_array_equal(got["assign"], ref["assign"], err_msg="assign " + label)
    if mode == 1:
        np.testing.assert_array_equal(got["knn_idx"], ref["knn_idx"], err_msg="knn " + label)
    w = b["features"][:, charge_col] if (weighted and charge_col >= 0) else \
        np.ones(b["coords"].shape[0], np.float32)
    scale = member_scale(b["features"], b["offsets"], P, w, mode, assign=ref["assign"],
                         knn_idx=ref["knn_idx"])
    assert_close_scaled(got["pooled"], ref["pooled"], scale, "pooled " + label)
    cw = b["features"][:, charge_col] if charge_col >= 0 else np.ones(b["coords"].shape[0],
                                                                       np.float32)
    cscale = member_scale(b["coords"], b["offsets"], P, cw, 0, assign=ref["assign"])
    assert_close_scaled(got["centroids"], ref["centroids"], cscale, "centroids " + label)


@pytest.mark.parametrize("name,r", [(n, r) for n in synth.WORKLOAD_ORDER for r in range(5)])
def test_tokenize_workloads(oracle_mod, name, r):
    w = synth.WORKLOADS[name]
    b = synth.make_batch(name, synth.parity_seed(name, r))
    _tokenize_vs_oracle(oracle_mod, b, w["P"], w["mode"], w["k"], w["L"], w["weighted"], 5,
                        label=name)


def test_fused_lds_pooling(oracle_mod):
    """Single-workgroup events whose feature rows are staged in LDS during
    FPS: the bitmap slot sort and the LDS pooling, on both sides of their
    limits (1024 pulses; (n + 1) * C staged floats of at most 6144) and for
    every column count the LDS pooling specialises (1..8, more in passes),
    charge-weighted, unit-charge and plain mean."""
    ns = [129, 255, 256, 257, 640, 1023, 1024, 1025]
    for C in (1, 3, 6, 8, 9, 13):
        b = synth.icecube_events(ns, 300 + C, C=C)
        cc = synth.CHARGE_COL if C > synth.CHARGE_COL else -1
        _tokenize_vs_oracle(oracle_mod, b, 128, charge_col=cc, label="lds C=%d" % C)
        _tokenize_vs_oracle(oracle_mod, b, 128, weighted=False, charge_col=cc,
                            label="lds mean C=%d" % C)
    b = synth.icecube_events([1024, 700, 65, 513], 331, C=6)
    _tokenize_vs_oracle(oracle_mod, b, 64, charge_col=-1, label="lds P=64 unit charge")
    _tokenize_vs_oracle(oracle_mod, b, 256, label="lds P=256")


def test_pool_chunk_combines(oracle_mod):
    """Standalone Voronoi pooling over 4096-pulse chunks: every chunk sorted
    by slot, one-chunk events written directly, chunks of larger events
    written as records that the combine kernel adds in chunk order; P <= 256
    with rows of up to 6 columns (rows sorted into LDS by the persistent
    kernel, 1 and 6 columns) and the gather kernel otherwise (7 and 16
    columns, P > 256)."""
    ns = [4096, 4097, 8192, 12289, 16384, 16385, 40000, 300]
    for C, P in ((6, 128), (6, 256), (1, 200), (7, 64), (16, 128), (3, 300)):
        b = synth.icecube_events(ns, 400 + C + P, C=C)
        cc = synth.CHARGE_COL if C > synth.CHARGE_COL else -1
        check_pipeline(oracle_mod, b, P=P, charge_col=cc, label="pool chunks C=%d P=%d" % (C, P))
    b = synth.icecube_events([70000, 20000], 431, C=6)
    check_pipeline(oracle_mod, b, P=256, weighted=False, label="pool chunks plain mean")


def test_pool_many_rounds(oracle_mod):
    """More pooling chunks than compute units: the persistent sorting kernel
    takes them in rounds, in serpentine order, over a list whose partial
    chunks the planner sorted into length bands (partial chunks of every
    length, full chunks and multi-chunk events among them), stepwise and
    fused."""
    rng = np.random.default_rng(512)
    ns = [int(n) for n in rng.integers(1, 4096, 900)] + [4096, 9000, 20000, 0, 1]
    b = synth.icecube_events(ns, 512, C=6)
    check_pipeline(oracle_mod, b, P=128, label="pool many rounds")
    _tokenize_vs_oracle(oracle_mod, b, 128, label="fused many rounds")


def test_fused_sorted_pooling_widths(oracle_mod):
    """The fused kernel's pooling of events and gang shards through 1024-pulse
    sub-chunks sorted into LDS (P <= 256, rows of up to 6 columns), for every
    row width, weighted by a column, by unit charge and as plain means, at
    sub-chunk boundaries and with gangs; direct mode too (a bound of 4096)."""
    ns = [1025, 2048, 3000, 4096, 9000, 600, 1024]
    for C, cc in ((1, 0), (2, -1), (3, 1), (5, 4)):
        b = synth.icecube_events(ns, 700 + C, C=C)
        _tokenize_vs_oracle(oracle_mod, b, 256, charge_col=cc, label="fused sorted C=%d" % C)
    b = synth.icecube_events(ns, 710, C=6)
    _tokenize_vs_oracle(oracle_mod, b, 100, weighted=False, label="fused sorted plain P=100")
    d = synth.icecube_events([1025, 2047, 4096, 300], 711, C=4)
    _tokenize_vs_oracle(oracle_mod, d, 200, charge_col=2, label="fused sorted direct",
                        max_event_points=4096)


def test_tokenize_fused_edges(oracle_mod):
    """The fused Voronoi kernel on every path: pass-through, one workgroup,
    gangs (cooperative pooling across shards) and the streaming fallback."""
    b = synth.icecube_events([0, 3, 128, 129, 700, 4096, 4097, 9000, 30001, 50], 23, C=6)
    _tokenize_vs_oracle(oracle_mod, b, 128, label="fused edges")
    _tokenize_vs_oracle(oracle_mod, b, 256, weighted=False, label="fused edges plain mean")
    b = synth.grid_events([20000, 700], 24, C=11, side=2)
    _tokenize_vs_oracle(oracle_mod, b, 64, label="fused tie-rich gang C=11")
    b = synth.uniform_events([270000, 600], 25, C=6)
    _tokenize_vs_oracle(oracle_mod, b, 32, label="fused streaming")
    b = synth.icecube_events([800, 12000, 90], 26, C=6)
    _tokenize_vs_oracle(oracle_mod, b, 128, mode=1, k=16, L=1, stepwise=True, label="stepwise")


def test_knn_fused_pooling(oracle_mod):
    """fpstok_tokenize in kNN mode pools each list inside the kNN kernel:
    empty and one-pulse events, events at and around P, k above n, k = 1
    and the largest k, plain and unit-charge means, rows wider than a wave
    (C = 70: two column rounds), with and without the event-size bound."""
    ns = [0, 1, 5, 127, 128, 129, 300, 1000, 4097, 0, 40]
    b = synth.icecube_events(ns, 61, C=6)
    m = int(np.diff(b["offsets"]).max())
    for k, hint in ((16, 0), (16, m), (1, m), (64, 0)):
        _tokenize_vs_oracle(oracle_mod, b, 128, mode=1, k=k, label="knn fused k=%d hint=%d" % (k, hint),
                            max_event_points=hint)
    _tokenize_vs_oracle(oracle_mod, b, 128, mode=1, k=16, weighted=False,
                        label="knn fused plain mean", max_event_points=m)
    _tokenize_vs_oracle(oracle_mod, b, 128, mode=1, k=16, charge_col=-1,
                        label="knn fused unit charge", max_event_points=m)
    w = synth.icecube_events([0, 3, 200, 700], 62, C=70)
    _tokenize_vs_oracle(oracle_mod, w, 64, mode=1, k=16, label="knn fused C=70",
                        max_event_points=700)
    _tokenize_vs_oracle(oracle_mod, w, 64, mode=1, k=16, L=2, label="knn fused C=70 Lloyd")


def test_max_event_points_hint(oracle_mod):
    """The work-list-free path: a correct bound (every event within one
    workgroup) and a bound that is too small (events above 4096 pulses fall
    back to the one-workgroup streaming FPS), fused and stepwise."""
    for name in ("icecube_b64_voronoi", "tiny_uniform", "icecube_b256_lloyd3"):
        w = synth.WORKLOADS[name]
        b = synth.make_batch(name, synth.parity_seed(name, 2))
        m = int(np.diff(b["offsets"]).max())
        _tokenize_vs_oracle(oracle_mod, b, w["P"], w["mode"], w["k"], w["L"], w["weighted"], 5,
                            label=name + " hint", max_event_points=m)
        check_pipeline(oracle_mod, b, P=w["P"], mode=w["mode"], k=w["k"], L=w["L"],
                       label=name + " hint stepwise", max_event_points=m)
    b = synth.icecube_events([0, 3, 129, 700, 4096, 4097, 9000, 50], 27, C=6)
    _tokenize_vs_oracle(oracle_mod, b, 128, label="hint too small", max_event_points=100)
    _tokenize_vs_oracle(oracle_mod, b, 128, mode=1, k=16, L=1, stepwise=True,
                        label="hint too small stepwise", max_event_points=100)
    check_pipeline(oracle_mod, b, P=128, L=2, label="hint too small sample", max_event_points=5)
    _tokenize_vs_oracle(oracle_mod, b, 128, label="hint above one workgroup",
                        max_event_points=9000)
    # a bound that rules out events of more than one pooling chunk: no
    # combine kernel, and an event of ten chunks that breaks the bound is
    # summed whole by its first chunk's workgroup
    b = synth.icecube_events([40000, 300, 5000], 28, C=6)
    check_pipeline(oracle_mod, b, P=128, label="hint too small, 10-chunk event",
                   max_event_points=100)
    check_pipeline(oracle_mod, b, P=256, weighted=False, label="hint 16384", max_event_points=16384)
