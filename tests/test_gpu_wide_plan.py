"""Decode plans large enough for the high-occupancy kernel, against the oracle.

A decode plan at M <= 4 with at least 4 workgroups (64-column tiles) per
compute unit runs a second instance of the plan kernel: four 8-wave
workgroups per CU with shallower pipelines.  These plans hold enough tiles
for it on any device of up to 256 CUs (1024 or more tiles) while keeping K
small for the oracle: every output is checked, at M = 1, 2 and 4, with and
without the zero-point edge structure (zero-code weights under large
activations), with fp16 and with quantized group scales, and a second run
must repeat the first bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import assert_within, note, to_dev, y_to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

WIDTHS = [2, 3, 4, 5, 6, 8]


@pytest.fixture(scope="module")
def exq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_bitrate_quantized_amd as m
    return m


def edge_case(rng, M, N, K):
    """(W, x): per group, each column's one non-zero weight sits on one of 4
    'hot' positions and every other code is the zero point; each row has one
    activation of 3e4 on a position off the hot ones and tiny ones elsewhere,
    so the large activations meet only zero-code weights."""
    W = np.zeros((N, K), dtype=np.float32)
    x = rng.uniform(-1e-3, 1e-3, size=(M, K)).astype(np.float32)
    for g in range(K // 128):
        hot = rng.choice(128, size=4, replace=False)
        rest = np.setdiff1d(np.arange(128), hot)
        k0 = 128 * g + hot[rng.integers(0, 4, size=N)]
        W[np.arange(N), k0] = rng.choice([-1.0, 1.0], size=N) * rng.uniform(1.0, 10.0, size=N)
        x[np.arange(M), 128 * g + rng.choice(rest, size=M)] = rng.choice([-1.0, 1.0], size=M) * 3.0e4
    return W, x.astype(np.float16)


@pytest.mark.parametrize("M", [1, 2, 4])
@pytest.mark.parametrize("edge", [False, True], ids=["normal", "zero-point-edge"])
@pytest.mark.parametrize("qs", [False, True], ids=["fp16-scales", "quantized-scales"])
def test_large_decode_plan(exq, M, edge, qs):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rng = np.random.default_rng(7 * M + edge + 100 * qs)
    N = 8192
    count = max(8, -(-4 * cus // (N // 64)))   # at least 4 tiles per CU
    layers, refs, xs_h = [], [], []
    for i in range(count):
        G = 1 + i % 6
        K = 128 * G
        widths = [WIDTHS[(i + g) % 6] for g in range(G)]
        if edge:
            W, x_edge = edge_case(rng, M, N, K)
        else:
            W = synth.weight(synth.seed_for("wide-plan", M, i), N, K)
        if qs:
            q, qsc, ref = exq.exq_pack_qs(W, widths)
            codes, R, qs_o, s_ref = oracle.quantize_qs(W, widths)
            np.testing.assert_array_equal(qsc, qs_o)
            np.testing.assert_array_equal(ref, R)
            layers.append(exq.Layer(K, N, widths, q, qsc, ref=ref))
        else:
            q, s = exq.exq_pack(W, widths)
            codes, s_ref, q_ref = oracle.reference_layer(W, widths)
            np.testing.assert_array_equal(q, q_ref)
            layers.append(exq.Layer(K, N, widths, q, s))
        refs.append(oracle.dequant(codes, s_ref, widths))
        xs_h.append(x_edge if edge else synth.activations(synth.seed_for("wide-plan-x", M, i), M, K))
    xs = [to_dev(x) for x in xs_h]
    ys = [torch.empty((M, N), dtype=torch.float16, device="cuda") for _ in layers]
    note("wide plan: %d linears x %d tiles, M=%d edge=%d qs=%d (%d CUs)" % (count, N // 64, M, edge, qs, cus))
    plan = exq.Plan(layers, xs, ys, M)
    try:
        plan.run()
        got = [y_to_np(y).copy() for y in ys]
        for i, (x, w_ref, g) in enumerate(zip(xs_h, refs, got)):
            y_ref, bnd = oracle.gemm(x, w_ref)
            assert_within(g, y_ref, bnd, "wide plan linear %d M=%d edge=%d qs=%d" % (i, M, edge, qs))
        plan.run()
        for y, g in zip(ys, got):
            np.testing.assert_array_equal(y_to_np(y), g)
    finally:
        plan.close()
        for l in layers:
            l.close()
