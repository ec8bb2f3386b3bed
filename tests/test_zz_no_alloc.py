"""exq_gemm_noalloc, the allocation-free variant of exq_gemm, through the C-ABI.

It must give exq_gemm's results: for a quantized-scale layer at prefill row
counts it expands the group scales into the library's static device scratch
on every call instead of a per-layer allocation.  Two calls in a row share
that scratch (the second with a smaller layer and fewer rows); both must
equal exq_gemm bit for bit and meet the oracle's bound.  Decode row counts
and fp16-scale layers take exq_gemm's own launches.  A layer whose scales do
not fit the scratch is refused before any launch.
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


def qs_case(exq, tag, K, N, widths, M):
    W = synth.weight(synth.seed_for("noalloc", tag), N, K)
    codes, ref, qscale, scales = oracle.quantize_qs(W, widths)
    layer = exq.Layer.from_weight(W, widths, quantized_scales=True)
    x = synth.activations(synth.seed_for("noalloc-x", tag, M), M, K)
    return layer, x, oracle.dequant(codes, scales, widths)


def test_noalloc_matches_gemm_two_calls_in_a_row(exq):
    big = qs_case(exq, "big", 1024, 512, [2, 3, 4, 5, 6, 8, 3, 2], 300)
    small = qs_case(exq, "small", 512, 256, [3, 5, 2, 8], 100)
    xs = [to_dev(c[1]) for c in (big, small)]
    ys = [torch.full((c[1].shape[0], c[0].N), -1.0, dtype=torch.float16, device="cuda") for c in (big, small)]
    note("noalloc: two calls in a row (M=300 then M=100)")
    for (layer, x, _), xd, yd in zip((big, small), xs, ys):
        exq.exq_gemm_noalloc(xd.data_ptr(), x.shape[0], layer.handle, yd.data_ptr())
    got = [y_to_np(y).copy() for y in ys]
    note("noalloc: exq_gemm on the same inputs")
    for (layer, x, w_ref), xd, g in zip((big, small), xs, got):
        want = y_to_np(layer.gemm(xd))
        np.testing.assert_array_equal(g.view(np.uint16), want.view(np.uint16))
        y_ref, bnd = oracle.gemm(x, w_ref)
        assert_within(g, y_ref, bnd, "noalloc M=%d" % x.shape[0])
        layer.close()


@pytest.mark.parametrize("M", [1, 5, 40, 300])
def test_noalloc_fp16_scales_and_decode_rows(exq, M):
    """fp16-scale layers at every kernel choice, and a quantized-scale layer at decode rows."""
    widths = [2, 8, 4, 3]
    K, N = 128 * len(widths), 320
    W = synth.weight(synth.seed_for("noalloc-f16"), N, K)
    for qs in (False, True):
        layer = exq.Layer.from_weight(W, widths, quantized_scales=qs)
        x = to_dev(synth.activations(synth.seed_for("noalloc-f16-x", M), M, K))
        y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        note("noalloc M=%d qs=%d" % (M, qs))
        exq.exq_gemm_noalloc(x.data_ptr(), M, layer.handle, y.data_ptr())
        got = y_to_np(y).copy()
        np.testing.assert_array_equal(got.view(np.uint16), y_to_np(layer.gemm(x)).view(np.uint16))
        layer.close()


def test_noalloc_rejects_scales_beyond_the_scratch(exq):
    G, N, M = 64, 131584, 300          # 2 * G * N = 16.8 MB > 16 MiB
    K = 128 * G
    widths = np.full(G, 2, dtype=np.uint8)
    q = torch.zeros(exq.exq_packed_bytes(K, N, widths), dtype=torch.uint8, device="cuda")
    qs = torch.zeros(G * N // 2, dtype=torch.uint8, device="cuda")
    ref = torch.zeros(N, dtype=torch.int16, device="cuda")
    h = exq.exq_layer_create_qs(K, N, widths, q.data_ptr(), qs.data_ptr(), ref.data_ptr())
    x = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    y = torch.zeros((M, N), dtype=torch.float16, device="cuda")
    try:
        with pytest.raises(exq.ExqError) as ei:
            exq.exq_gemm_noalloc(x.data_ptr(), M, h, y.data_ptr())
        assert ei.value.status == exq.EXQ_ERR_UNSUPPORTED
    finally:
        exq.exq_layer_destroy(h)
