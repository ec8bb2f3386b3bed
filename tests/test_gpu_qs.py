"""GPU parity of layers stored with quantized group scales (4-bit codes and a
column reference): dequantization bit-exact against the oracle's expansion,
and every kernel path -- decode with both tile widths, decode slices, prefill,
decode and prefill plans, the gated pair -- within the matmul bound."""
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


def qs_layer(exq, N, K, widths, tag):
    W = synth.weight(synth.seed_for("gpu-qs", tag), N, K).copy()
    W[1] = 0.0
    q, qs, ref = exq.exq_pack_qs(W, widths)
    codes, R, qs_o, scales = oracle.quantize_qs(W, widths)
    np.testing.assert_array_equal(qs, qs_o)
    np.testing.assert_array_equal(ref, R)
    return exq.Layer(K, N, widths, q, qs, ref=ref), oracle.dequant(codes, scales, widths)


@pytest.mark.parametrize("N", [320, 16384])
def test_qs_dequant_and_gemm(exq, N):
    widths = [2, 3, 4, 5, 6, 8, 2, 2]
    K = 128 * len(widths)
    lay, w_ref = qs_layer(exq, N, K, widths, "n%d" % N)
    note("qs dequant N=%d" % N)
    np.testing.assert_array_equal(lay.dequant().cpu().numpy().view(np.uint16), w_ref)
    for M in (1, 5, 16, 40, 300):
        x = synth.activations(synth.seed_for("gpu-qs-x", N, M), M, K)
        note("qs gemm N=%d M=%d" % (N, M))
        y = y_to_np(lay.gemm(to_dev(x)))
        y_ref, bnd = oracle.gemm(x, w_ref)
        assert_within(y, y_ref, bnd, "qs N=%d M=%d" % (N, M))
    lay.close()


def test_qs_plans_and_gated(exq):
    specs = [(1024, 1024, [2, 3, 2, 2, 6, 8, 2, 3]), (768, 2048, [3, 2, 4, 5, 2, 2])]
    layers, refs = [], []
    for i, (K, N, widths) in enumerate(specs):
        l, w = qs_layer(exq, N, K, widths, "plan%d" % i)
        layers.append(l)
        refs.append(w)
    for M in (1, 16, 300):
        xs_h = [synth.activations(synth.seed_for("gpu-qs-plan-x", i, M), M, l.K) for i, l in enumerate(layers)]
        xs = [to_dev(x) for x in xs_h]
        ys = [torch.empty((M, l.N), dtype=torch.float16, device="cuda") for l in layers]
        note("qs plan M=%d" % M)
        plan = exq.Plan(layers, xs, ys, M)
        plan.run()
        for x, y, w, l in zip(xs_h, ys, refs, layers):
            y_ref, bnd = oracle.gemm(x, w)
            assert_within(y_to_np(y), y_ref, bnd, "qs plan M=%d N=%d" % (M, l.N))
        plan.close()
    # a decode plan needs one scale storage for all its linears
    W = synth.weight(synth.seed_for("gpu-qs-mixed"), 1024, 1024)
    plain = exq.Layer.from_weight(W, [2] * 8)
    x1 = [to_dev(synth.activations(1, 1, 1024)) for _ in range(2)]
    y1 = [torch.empty((1, 1024), dtype=torch.float16, device="cuda") for _ in range(2)]
    with pytest.raises(exq.ExqError):
        exq.Plan([layers[0], plain], x1, y1, 1)
    # gated pair with quantized scales
    g, wg = qs_layer(exq, 1024, 1024, [2, 3, 4, 2, 2, 6, 8, 2], "gate")
    u, wu = qs_layer(exq, 1024, 1024, [3, 3, 2, 5, 2, 2, 2, 4], "up")
    for M in (1, 16, 100):
        x = synth.activations(synth.seed_for("gpu-qs-gated-x", M), M, 1024)
        note("qs gated M=%d" % M)
        h = y_to_np(exq.gemm_gated(to_dev(x), g, u))
        h_ref, allow = oracle.gated(x, wg, wu)
        ok, worst = oracle.within_allowance(h, h_ref, allow)
        assert ok, "qs gated M=%d worst %.3f" % (M, worst)
    with pytest.raises(exq.ExqError):
        exq.gemm_gated(to_dev(synth.activations(2, 1, 1024)), g, plain)
    for l in layers + [plain, g, u]:
        l.close()


def test_qs_70b_down_m1(exq):
    """The longest linear of the 70B block (down, 28672 -> 8192) with quantized scales, every output at M = 1."""
    from synth import workloads
    spec = [s for s in workloads.linears(3) if s.name == "down"][0]
    W = workloads.make_weight(spec)
    widths = workloads.make_widths(spec, W)
    q, qs, ref = exq.exq_pack_qs(W, widths)
    codes, R, qs_o, scales = oracle.quantize_qs(W, widths)
    np.testing.assert_array_equal(qs, qs_o)
    lay = exq.Layer(spec.K, spec.N, widths, q, qs, ref=ref)
    w_ref = oracle.dequant(codes, scales, widths)
    x = synth.activations(synth.seed_for("gpu-qs-down-x"), 1, spec.K)
    note("qs 70B down M=1")
    y = y_to_np(lay.gemm(to_dev(x)))
    y_ref, bnd = oracle.gemm(x, w_ref)
    assert_within(y, y_ref, bnd, "qs down")
    lay.close()
