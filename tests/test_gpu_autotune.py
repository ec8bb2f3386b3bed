"""Per-shape kernel choice: every choice exq_gemm can be given meets the
oracle's bound and is deterministic; exq_autotune keeps one of them and
exq_gemm then reproduces that choice's output bit for bit."""
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


def layer(exq, K, N, widths, tag):
    W = synth.weight(synth.seed_for("tune", tag), N, K)
    codes, s, q = oracle.reference_layer(W, widths)
    return exq.Layer(K, N, widths, q, s), oracle.dequant(codes, s, widths)


@pytest.mark.parametrize("K,N", [(1024, 1024), (2048, 16384)])
def test_every_variant_matches_oracle(exq, K, N):
    G = K // 128
    lay, w_ref = layer(exq, K, N, ([2, 3, 4, 5, 6, 8] * 3)[:G], "v%d" % N)
    for M in (1, 7, 16, 24, 40):
        x = synth.activations(synth.seed_for("tune-x", N, M), M, K)
        y_ref, bnd = oracle.gemm(x, w_ref)
        variants = [exq.VARIANT_DEFAULT, exq.VARIANT_DECODE16, exq.VARIANT_DECODE64]
        if M > 16:
            variants.append(exq.VARIANT_PREFILL)
        for v in variants:
            exq.exq_set_variant(lay.handle, M, v)
            note("variant %d K=%d N=%d M=%d" % (v, K, N, M))
            xd = to_dev(x)
            y1 = y_to_np(lay.gemm(xd)).copy()
            assert_within(y1, y_ref, bnd, "variant %d M=%d" % (v, M))
            np.testing.assert_array_equal(y_to_np(lay.gemm(xd)), y1)
        exq.exq_set_variant(lay.handle, M, exq.VARIANT_DEFAULT)
    lay.close()


def test_autotune_keeps_a_choice(exq):
    K, N = 2048, 4096
    lay, w_ref = layer(exq, K, N, [2, 3, 3, 2, 6, 8, 2, 4, 5, 2, 2, 3, 3, 2, 2, 2], "auto")
    for M in (1, 16, 32):
        x = synth.activations(synth.seed_for("tune-auto-x", M), M, K)
        xd = to_dev(x)
        y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        note("autotune M=%d" % M)
        choice, times = exq.exq_autotune(xd.data_ptr(), M, lay.handle, y.data_ptr(), warmup=2, reps=12)
        assert choice in ((1, 2, 3) if M > 16 else (1, 2))
        assert len(times) == (3 if M > 16 else 2) and all(t > 0 for t in times)
        assert times[choice - 1] == min(times)
        tuned = y_to_np(y).copy()
        y_ref, bnd = oracle.gemm(x, w_ref)
        assert_within(tuned, y_ref, bnd, "autotuned M=%d" % M)
        np.testing.assert_array_equal(y_to_np(lay.gemm(xd)), tuned)          # exq_gemm now uses the choice
        exq.exq_set_variant(lay.handle, M, choice)
        np.testing.assert_array_equal(y_to_np(lay.gemm(xd)), tuned)
    lay.close()


def test_variant_arguments(exq):
    lay, _ = layer(exq, 256, 128, [2, 3], "args")
    for args in ((0, 1), (65, 1), (8, 3), (20, 4), (20, -1)):
        with pytest.raises(exq.ExqError):
            exq.exq_set_variant(lay.handle, *args)
    x = torch.zeros((4, 256), dtype=torch.float16, device="cuda")
    y = torch.zeros((4, 128), dtype=torch.float16, device="cuda")
    with pytest.raises(exq.ExqError):
        exq.exq_autotune(x.data_ptr(), 4, lay.handle, y.data_ptr(), reps=0)
    with pytest.raises(exq.ExqError):
        exq.exq_autotune(x.data_ptr(), 65, lay.handle, y.data_ptr())
    lay.close()
