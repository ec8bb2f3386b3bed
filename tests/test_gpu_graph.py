"""HIP-graph capture of the library's launches, through the C-ABI.

exq_gemm (decode and prefill row counts), exq_gemm_gated and exq_plan_run
(decode and prefill plans) are captured once with torch.cuda.graph and
replayed three times.  Before each replay the captured input buffers get new
values and eager work runs on the same stream; each replay's output must equal,
bit for bit, an eager call on the same inputs (a kernel's summation order does
not depend on how it was launched), and the eager call is within the oracle's
bound.  No entry point records a memset or an allocation, so the graphs hold
kernel nodes only.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import assert_within, note, to_dev, y_to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SHAPES = ((640, 384, [2, 5, 3, 8, 4]), (1024, 512, [6, 2, 2, 3, 4, 5, 8, 3]), (256, 192, [3, 6]))


@pytest.fixture(scope="module")
def exq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_bitrate_quantized_amd as m
    return m


@pytest.fixture(scope="module")
def layers(exq):
    out = []
    for i, (K, N, widths) in enumerate(SHAPES):
        W = synth.weight(synth.seed_for("graph", i), N, K)
        q, s = exq.exq_pack(W, widths)
        codes, s_ref, _ = oracle.reference_layer(W, widths)
        out.append((exq.Layer(K, N, widths, q, s), oracle.dequant(codes, s_ref, widths)))
    yield out
    for l, _ in out:
        l.close()


def inputs(tag, M, K, rep):
    return synth.activations(synth.seed_for("graph-x", tag, M, K, rep), M, K)


def capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def replays(g, xs_dev, fill, eager, outs, what):
    """Three replays: new inputs, eager reference, unrelated eager work, replay, compare."""
    for rep in range(3):
        new = fill(rep)
        for xd, xh in zip(xs_dev, new):
            xd.copy_(to_dev(xh))
        want = [y_to_np(y).copy() for y in eager()]
        for o in outs:
            o.fill_(float("nan"))
        junk = torch.randn(256, 256, device="cuda") @ torch.randn(256, 256, device="cuda")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        del junk
        for o, w in zip(outs, want):
            np.testing.assert_array_equal(y_to_np(o), w, err_msg="%s replay %d" % (what, rep))
        yield new, want


@pytest.mark.parametrize("M", [1, 5, 40, 300])
def test_gemm_in_graph(exq, layers, M):
    for i, (layer, w_ref) in enumerate(layers):
        note("graph gemm layer %d M=%d" % (i, M))
        x = to_dev(inputs("gemm", M, layer.K, -1))
        y = torch.empty((M, layer.N), dtype=torch.float16, device="cuda")
        g = capture(lambda: layer.gemm(x, out=y))
        fill = lambda rep: [inputs("gemm", M, layer.K, rep)]
        eager = lambda: [layer.gemm(x)]
        for new, want in replays(g, [x], fill, eager, [y], "gemm layer %d M=%d" % (i, M)):
            y_ref, bnd = oracle.gemm(new[0], w_ref)
            assert_within(want[0], y_ref, bnd, "eager gemm layer %d M=%d" % (i, M))
        del g


@pytest.mark.parametrize("M", [1, 16, 300])
def test_gated_in_graph(exq, layers, M):
    gate, up = layers[1][0], layers[1][0]
    note("graph gated M=%d" % M)
    x = to_dev(inputs("gated", M, gate.K, -1))
    h = torch.empty((M, gate.N), dtype=torch.float16, device="cuda")
    g = capture(lambda: exq.gemm_gated(x, gate, up, out=h))
    fill = lambda rep: [inputs("gated", M, gate.K, rep)]
    eager = lambda: [exq.gemm_gated(x, gate, up)]
    for _ in replays(g, [x], fill, eager, [h], "gated M=%d" % M):
        pass
    del g


@pytest.mark.parametrize("M", [1, 3, 16, 300])
def test_plan_in_graph(exq, layers, M):
    note("graph plan M=%d" % M)
    xs = [to_dev(inputs("plan", M, l.K, -1)) for l, _ in layers]
    ys = [torch.empty((M, l.N), dtype=torch.float16, device="cuda") for l, _ in layers]
    plan = exq.Plan([l for l, _ in layers], xs, ys, M)
    g = capture(plan.run)
    fill = lambda rep: [inputs("plan", M, l.K, rep) for l, _ in layers]

    def eager():
        plan.run()
        return [y.clone() for y in ys]

    for new, want in replays(g, xs, fill, eager, ys, "plan M=%d" % M):
        for xh, w, (l, w_ref) in zip(new, want, layers):
            y_ref, bnd = oracle.gemm(xh, w_ref)
            assert_within(w, y_ref, bnd, "eager plan M=%d K=%d" % (M, l.K))
    del g
    plan.close()
