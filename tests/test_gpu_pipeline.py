"""Decode pipelines at every run length, against the oracle.

A wave streams its share of a layer's width-sorted groups as runs of equal
width, pipelined a fixed number of groups deep (1 to 4 in flight, by width
and layout).  A run executes whole rounds of that depth, then its last
partial round step by step; in the 16-row layout (M = 5..16) runs of widths up
to 6 bits stage each group's activations in a two-slot LDS ring, 8-bit runs
keep them in registers.  A layer of 8r groups of one width gives every one of
the 8 waves a run of exactly r groups, so r = 1..7 ends the runs on every
position of every round and on both ring slots.  Two widths in one layer
give each wave two runs back to back (the second starting while loads of the
first's last round may still be in flight).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import assert_within, note, to_dev, y_to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MS = [1, 4, 5, 16]


@pytest.fixture(scope="module")
def exq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_bitrate_quantized_amd as m
    return m


def check_layer(exq, widths, N, tag):
    K = 128 * len(widths)
    W = synth.weight(synth.seed_for("pipeline", tag), N, K)
    q, s = exq.exq_pack(W, widths)
    codes, s_ref, q_ref = oracle.reference_layer(W, widths)
    np.testing.assert_array_equal(q, q_ref)
    w_ref = oracle.dequant(codes, s_ref, widths)
    layer = exq.Layer(K, N, widths, q, s)
    try:
        for M in MS:
            x = synth.activations(synth.seed_for("pipeline-x", tag, M), M, K)
            note("pipeline %s K=%d N=%d M=%d" % (tag, K, N, M))
            y = y_to_np(layer.gemm(to_dev(x)))
            y_ref, bnd = oracle.gemm(x, w_ref)
            assert_within(y, y_ref, bnd, "pipeline %s M=%d" % (tag, M))
            # The same layer as a one-entry plan (64-column tiles).
            xd = to_dev(x)
            yd = torch.empty((M, N), dtype=torch.float16, device="cuda")
            plan = exq.Plan([layer], [xd], [yd], M)
            try:
                plan.run()
                assert_within(y_to_np(yd), y_ref, bnd, "pipeline %s plan M=%d" % (tag, M))
            finally:
                plan.close()
    finally:
        layer.close()


@pytest.mark.parametrize("r", [1, 2, 3, 4, 5, 7])
@pytest.mark.parametrize("b", [2, 3, 4, 6, 8])
def test_run_of_every_length(exq, b, r):
    check_layer(exq, [b] * (8 * r), 128, "b%d-r%d" % (b, r))


@pytest.mark.parametrize("r1,b1,r2,b2", [(1, 2, 2, 3), (3, 2, 1, 6), (5, 3, 3, 8), (2, 6, 5, 8), (7, 2, 4, 4)])
def test_two_runs_per_wave(exq, r1, b1, r2, b2):
    check_layer(exq, [b1] * (8 * r1) + [b2] * (8 * r2), 192, "b%dr%d-b%dr%d" % (b1, r1, b2, r2))
