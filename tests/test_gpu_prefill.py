"""GPU parity of the prefill kernel (M > 16) against the CPU oracle.

The prefill kernel works on 256 x 256 output tiles in K stages of 64; these
cases put M and N on both sides of the tile edges (ragged row and column
tails), mix every width inside one layer, and check the special cases that
must be bit-exact: integer closed form, power-of-two scales, one-hot rows,
zero input, determinism, no writes outside y.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import assert_within, note, to_dev, y_to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def exq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_bitrate_quantized_amd as m
    return m


def make_layer(exq, W, widths):
    q, s = exq.exq_pack(W, widths)
    codes, s_ref, q_ref = oracle.reference_layer(W, widths)
    np.testing.assert_array_equal(q, q_ref)
    np.testing.assert_array_equal(s, s_ref)
    N, K = W.shape
    layer = exq.Layer(K, N, widths, q, s)
    # exq_gemm serves M <= 64 with the decode kernel by default; these tests
    # are about the prefill kernel, so it is chosen for every M from 17 on.
    for M in range(17, 65):
        exq.exq_set_variant(layer.handle, M, exq.VARIANT_PREFILL)
    return layer, oracle.dequant(codes, s_ref, widths)


@pytest.mark.parametrize("N", [64, 320, 512])
def test_tile_edges_every_width(exq, N):
    widths = [2, 3, 4, 5, 6, 8, 4, 3, 2]
    K = 128 * len(widths)
    W = synth.weight(synth.seed_for("pf-edges", N), N, K)
    layer, w_ref = make_layer(exq, W, widths)
    for M in (17, 255, 256, 257, 520):
        x = synth.activations(synth.seed_for("pf-edges-x", N, M), M, K)
        note("prefill edges N=%d M=%d" % (N, M))
        y = y_to_np(layer.gemm(to_dev(x)))
        y_ref, bnd = oracle.gemm(x, w_ref)
        assert_within(y, y_ref, bnd, "prefill N=%d M=%d" % (N, M))
    layer.close()


@pytest.mark.parametrize("b", [2, 3, 4, 5, 6, 8])
def test_uniform_width(exq, b):
    K, N, M = 384, 256, 300
    W = synth.weight(synth.seed_for("pf-uniform", b), N, K)
    layer, w_ref = make_layer(exq, W, [b] * (K // 128))
    x = synth.activations(synth.seed_for("pf-uniform-x", b), M, K)
    note("prefill uniform b=%d" % b)
    y = y_to_np(layer.gemm(to_dev(x)))
    y_ref, bnd = oracle.gemm(x, w_ref)
    assert_within(y, y_ref, bnd, "prefill b=%d" % b)
    layer.close()


def test_integer_closed_form(exq):
    """All 8-bit, scales exactly 1, x in {-1,0,1}: y is the integer matmul, bit-exact."""
    rng = np.random.default_rng(23)
    K, N, M = 384, 320, 300
    Wi = rng.integers(-127, 128, size=(N, K))
    Wi[:, ::128] = 127
    layer, _ = make_layer(exq, Wi.astype(np.float32), [8, 8, 8])
    x = rng.integers(-1, 2, size=(M, K)).astype(np.float16)
    note("prefill closed form")
    y = y_to_np(layer.gemm(to_dev(x)))
    np.testing.assert_array_equal(y, (x.astype(np.int64) @ Wi.T).astype(np.float16))
    layer.close()


@pytest.mark.parametrize("b", [2, 3, 4, 5, 6, 8])
def test_power_of_two_scales_exact(exq, b):
    rng = np.random.default_rng(300 + b)
    qmax = (1 << (b - 1)) - 1
    K, N, M = 256, 256, 270
    e = rng.integers(-6, 3, size=(N, 2))
    Q = rng.integers(-qmax, qmax + 1, size=(N, K))
    Q[:, 0] = qmax
    Q[:, 128] = -qmax
    W = (Q * np.repeat(2.0 ** e, 128, axis=1)).astype(np.float32)
    layer, _ = make_layer(exq, W, [b, b])
    x = rng.integers(-2, 3, size=(M, K)).astype(np.float16)
    note("prefill pow2 b=%d" % b)
    y = y_to_np(layer.gemm(to_dev(x)))
    ref = x.astype(np.float64) @ W.astype(np.float64).T
    np.testing.assert_array_equal(y, ref.astype(np.float16))
    layer.close()


def test_one_hot_zero_determinism_guard(exq):
    widths = [3, 5, 2, 8, 6]
    K, N = 640, 320
    W = synth.weight(synth.seed_for("pf-special"), N, K)
    layer, w_ref = make_layer(exq, W, widths)
    M = 300
    note("prefill one-hot")
    ks = np.arange(M) * 7 % K
    x = np.zeros((M, K), dtype=np.float16)
    x[np.arange(M), ks] = 1.0
    y = y_to_np(layer.gemm(to_dev(x)))
    np.testing.assert_array_equal(y.view(np.uint16), w_ref[ks])
    note("prefill zero input")
    y = y_to_np(layer.gemm(to_dev(np.zeros((M, K), dtype=np.float16))))
    assert np.all(y == 0)
    note("prefill determinism and guard bands")
    x = to_dev(synth.activations(synth.seed_for("pf-guard"), M, K))
    pad = 8192
    buf = torch.full((M * N + 2 * pad,), -12345, dtype=torch.int16, device="cuda")
    out = buf[pad:pad + M * N].view(torch.float16).view(M, N)
    layer.gemm(x, out=out)
    first = y_to_np(out).copy()
    layer.gemm(x, out=out)
    np.testing.assert_array_equal(y_to_np(out), first)
    bb = buf.cpu().numpy()
    assert np.all(bb[:pad] == -12345) and np.all(bb[pad + M * N:] == -12345)
    layer.close()


def test_long_k(exq):
    """K = 28672 (224 groups), the longest accumulation of the workloads, on a column sample."""
    K, N, M = 28672, 256, 64
    G = K // 128
    W = synth.weight(synth.seed_for("pf-longk"), N, K)
    widths = synth.widths_mixed(G, synth.group_sq_norms(W), synth.seed_for("pf-longk-w"))
    layer, w_ref = make_layer(exq, W, widths)
    x = synth.activations(synth.seed_for("pf-longk-x"), M, K)
    note("prefill long K")
    y = y_to_np(layer.gemm(to_dev(x)))
    y_ref, bnd = oracle.gemm(x, w_ref)
    assert_within(y, y_ref, bnd, "prefill K=%d" % K)
    layer.close()


def test_prefill_plan_matches_oracle_and_is_repeatable(exq):
    """Several linears, different K and N, one launch at M > 16."""
    specs = [(384, 320, [3, 4, 5]), (1024, 128, [2] * 6 + [8, 6]), (256, 512, [6, 2])]
    layers, refs = [], []
    for i, (K, N, widths) in enumerate(specs):
        W = synth.weight(synth.seed_for("pf-plan", i), N, K)
        layer, w_ref = make_layer(exq, W, widths)
        layers.append(layer)
        refs.append(w_ref)
    for M in (17, 300):
        xs_h = [synth.activations(synth.seed_for("pf-plan-x", i, M), M, l.K) for i, l in enumerate(layers)]
        xs = [to_dev(x) for x in xs_h]
        ys = [torch.empty((M, l.N), dtype=torch.float16, device="cuda") for l in layers]
        note("prefill plan M=%d" % M)
        plan = exq.Plan(layers, xs, ys, M)
        plan.run()
        got = [y_to_np(y).copy() for y in ys]
        for x, g, w_ref, l in zip(xs_h, got, refs, layers):
            y_ref, bnd = oracle.gemm(x, w_ref)
            assert_within(g, y_ref, bnd, "prefill plan M=%d N=%d" % (M, l.N))
        plan.run()
        for y, g in zip(ys, got):
            np.testing.assert_array_equal(y_to_np(y), g)
        plan.close()
    for l in layers:
        l.close()


@pytest.mark.parametrize("col_tiles,pieces", [(320, 4), (384, 2)])
def test_prefill_plan_tiles_cut_along_k(exq, col_tiles, pieces):
    """A prefill plan whose XCD queues end on a partial round cuts that
    round's tiles along K: 320 (384) column tiles of one row tile give each
    of the 8 XCD queues 40 (48) tiles, so with 32 compute units per XCD the
    last 8 (16) tiles of each queue are cut into 4 (2) pieces, the last piece
    to finish adding them in K order.  Every output is checked against the
    oracle on a sample of rows (all columns), repeated launches (the arrival
    counters reset) give identical bits, and the uncut single-linear kernel
    agrees within the bound."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the cut layout below assumes 32 compute units per XCD")
    widths = [2, 3, 4, 8]
    K, N, M = 128 * len(widths), 256 * col_tiles, 256
    W = synth.weight(synth.seed_for("kcut", col_tiles), N, K)
    layer, w_ref = make_layer(exq, W, widths)
    x = synth.activations(synth.seed_for("kcut-x", col_tiles), M, K)
    xd = to_dev(x)
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    plan = exq.Plan([layer], [xd], [y], M)
    try:
        note("prefill plan cut along K: %d column tiles, %d pieces" % (col_tiles, pieces))
        plan.run()
        first = y_to_np(y).copy()
        for _ in range(2):
            plan.run()
            np.testing.assert_array_equal(y_to_np(y).view(np.uint16), first.view(np.uint16))
        rows = np.array([0, 1, 37, 128, 200, 254, 255])
        y_ref, bnd = oracle.gemm(x[rows], w_ref)
        assert_within(first[rows], y_ref, bnd, "plan cut along K")
        single = y_to_np(layer.gemm(xd))
        y_ref_s, bnd_s = oracle.gemm(x[rows], w_ref)
        assert_within(single[rows], y_ref_s, bnd_s, "single-linear prefill")
        both = np.abs(first.astype(np.float64) - single.astype(np.float64))
        assert float(both.max()) < 1.0
    finally:
        plan.close()
        layer.close()
