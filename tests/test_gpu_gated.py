"""GPU parity of the fused gate/up product h = SiLU(x Wg^T) * (x Wu^T) against
the CPU oracle's exact h_ref and per-output allowance: both decode tilings
(16 and 64 columns), decode and prefill row counts, the 70B feed-forward
shapes, determinism, guard bands and argument errors."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import note, to_dev, y_to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def exq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_bitrate_quantized_amd as m
    return m


def pair(exq, K, N, widths_g, widths_u, tag):
    out = []
    for i, widths in enumerate((widths_g, widths_u)):
        W = synth.weight(synth.seed_for("gated", tag, i), N, K)
        codes, s, q = oracle.reference_layer(W, widths)
        out.append((exq.Layer(K, N, widths, q, s), oracle.dequant(codes, s, widths)))
    return out


def check(h, x, wg, wu, what):
    h_ref, allow = oracle.gated(x, wg, wu)
    ok, worst = oracle.within_allowance(h, h_ref, allow)
    assert ok, "%s: worst error / allowance %.3f" % (what, worst)


@pytest.mark.parametrize("N", [320, 16384])   # 16-column tiles below 256 tiles of 64, else 64-column tiles
def test_gated_matches_oracle(exq, N):
    K = 640
    (lg, wg), (lu, wu) = pair(exq, K, N, [2, 3, 4, 5, 6], [8, 6, 2, 2, 3], "n%d" % N)
    for M in (1, 2, 5, 16, 17, 40):
        x = synth.activations(synth.seed_for("gated-x", N, M), M, K)
        note("gated N=%d M=%d" % (N, M))
        h = y_to_np(exq.gemm_gated(to_dev(x), lg, lu))
        check(h, x, wg, wu, "N=%d M=%d" % (N, M))
    lg.close()
    lu.close()


def test_gated_prefill_tile_edges(exq):
    K, N = 384, 320
    (lg, wg), (lu, wu) = pair(exq, K, N, [3, 4, 6], [5, 2, 8], "pf")
    for M in (255, 257):
        x = synth.activations(synth.seed_for("gated-pf-x", M), M, K)
        note("gated prefill M=%d" % M)
        h = y_to_np(exq.gemm_gated(to_dev(x), lg, lu))
        check(h, x, wg, wu, "prefill M=%d" % M)
    lg.close()
    lu.close()


@pytest.mark.parametrize("M", [1, 16])
def test_gated_70b_feed_forward(exq, M):
    """The 70B gate/up pair (8192 -> 28672) at 2.55 bpw, every output."""
    from synth import workloads
    specs = [s for s in workloads.linears(3) if s.name in ("gate", "up")]
    layers, w_hats = [], []
    for spec in specs:
        W = workloads.make_weight(spec)
        widths = workloads.make_widths(spec, W)
        codes, s, q = oracle.reference_layer(W, widths)
        layers.append(exq.Layer(spec.K, spec.N, widths, q, s))
        w_hats.append(oracle.dequant(codes, s, widths))
    x = synth.activations(synth.seed_for("gated-70b-x", M), M, specs[0].K)
    note("gated 70B feed-forward M=%d" % M)
    h = y_to_np(exq.gemm_gated(to_dev(x), layers[0], layers[1]))
    check(h, x, w_hats[0], w_hats[1], "70B M=%d" % M)
    for l in layers:
        l.close()


def test_gated_deterministic_and_guarded(exq):
    K, N, M = 512, 1024, 16
    (lg, _), (lu, _) = pair(exq, K, N, [2, 2, 3, 8], [6, 5, 4, 3], "guard")
    x = to_dev(synth.activations(synth.seed_for("gated-guard-x"), M, K))
    pad = 4096
    for m in (3, M):
        note("gated guard bands M=%d" % m)
        buf = torch.full((m * N + 2 * pad,), -12345, dtype=torch.int16, device="cuda")
        out = buf[pad:pad + m * N].view(torch.float16).view(m, N)
        exq.gemm_gated(x[:m].contiguous(), lg, lu, out=out)
        first = y_to_np(out).copy()
        exq.gemm_gated(x[:m].contiguous(), lg, lu, out=out)
        np.testing.assert_array_equal(y_to_np(out), first)
        bb = buf.cpu().numpy()
        assert np.all(bb[:pad] == -12345) and np.all(bb[pad + m * N:] == -12345)
    lg.close()
    lu.close()


def test_gated_rejects_bad_arguments(exq):
    (lg, _), (lu, _) = pair(exq, 256, 128, [2, 3], [4, 5], "bad")
    other = exq.Layer.from_weight(synth.weight(synth.seed_for("gated-other"), 192, 256), [2, 3])
    x = torch.zeros((4, 256), dtype=torch.float16, device="cuda")
    h = torch.zeros((4, 128), dtype=torch.float16, device="cuda")
    with pytest.raises(exq.ExqError):
        exq.exq_gemm_gated(x.data_ptr(), 4, lg.handle, other.handle, h.data_ptr())
    with pytest.raises(exq.ExqError):
        exq.exq_gemm_gated(x.data_ptr(), 0, lg.handle, lu.handle, h.data_ptr())
    with pytest.raises(exq.ExqError):
        exq.exq_gemm_gated(x.data_ptr(), 4, lg.handle, lu.handle, x.data_ptr())
    for l in (lg, lu, other):
        l.close()
