"""Pins of the oracle's gated product h = SiLU(x Wg^T) * (x Wu^T) and of its
allowance, against closed forms and brute force rather than against itself."""
import math

import numpy as np

import oracle
import synth


def _w_hat(values):
    """fp16 bits of an array of values exactly representable in fp16."""
    a = np.asarray(values, dtype=np.float64)
    h = a.astype(np.float16)
    assert np.array_equal(h.astype(np.float64), a)
    return h.view(np.uint16)


def test_silu_closed_forms():
    # logistic(ln 3) = 3/4 exactly, so SiLU(+-ln 3) = +-ln 3 * (3/4 or 1/4).
    ln3 = math.log(3.0)
    np.testing.assert_allclose(oracle.silu([ln3, -ln3]), [0.75 * ln3, -0.25 * ln3], rtol=1e-15)
    assert oracle.silu(0.0) == 0.0
    # SiLU(t) - SiLU(-t) = t for every t (logistic(t) + logistic(-t) = 1).
    t = np.linspace(-30, 30, 2001)
    np.testing.assert_allclose(oracle.silu(t) - oracle.silu(-t), t, atol=1e-12)
    # Limits: SiLU(t) -> t for large t, -> 0 from below for very negative t.
    assert oracle.silu(800.0) == 800.0
    v = oracle.silu(-800.0)
    assert v == 0.0 and math.copysign(1.0, v) == -1.0


def test_silu_slope_bound_holds():
    t = np.linspace(-40, 40, 800001)
    d = np.diff(oracle.silu(t)) / np.diff(t)
    assert 1.09 < d.max() < oracle.SILU_SLOPE_BOUND
    assert -0.11 < d.min() < 0
    assert abs(t[np.argmax(d)] - 2.3994) < 1e-3


def test_gated_one_hot_rows():
    """x = e_k picks row k of each W_hat: h = SiLU(wg[k]) * wu[k] exactly in fp64."""
    wg = _w_hat([[0.0, 2.0, -2.0, 20.0], [1.0, -1.0, 0.5, -24.0]])
    wu = _w_hat([[3.0, 0.5, -1.0, 2.0], [-2.0, 4.0, 8.0, 1.0]])
    x = np.eye(2, dtype=np.float16)
    h, allow = oracle.gated(x, wg, wu)
    ln = lambda t: t / (1 + math.exp(-t))
    expect = [[0.0, ln(2.0) * 0.5, ln(-2.0) * -1.0, ln(20.0) * 2.0], [ln(1.0) * -2.0, ln(-1.0) * 4.0, ln(0.5) * 8.0,
                                                                     ln(-24.0) * 1.0]]
    np.testing.assert_allclose(h, expect, rtol=1e-14, atol=0)
    assert np.all(allow > 0)


def test_gated_sign_identity():
    """h(Wg) - h(-Wg) = g * u with g, u the (separately pinned) matmuls."""
    rng = np.random.default_rng(5)
    K, N, M = 256, 24, 3
    wg = rng.normal(0, 0.05, size=(K, N)).astype(np.float16)
    wu = rng.normal(0, 0.05, size=(K, N)).astype(np.float16)
    x = rng.normal(0, 1, size=(M, K)).astype(np.float16)
    h1, _ = oracle.gated(x, wg.view(np.uint16), wu.view(np.uint16))
    h2, _ = oracle.gated(x, (-wg).view(np.uint16), wu.view(np.uint16))
    g, _ = oracle.gemm(x, wg.view(np.uint16))
    u, _ = oracle.gemm(x, wu.view(np.uint16))
    np.testing.assert_allclose(h1 - h2, g * u, rtol=1e-12, atol=1e-14)


def test_allowance_covers_worst_perturbations():
    """Brute force: products moved anywhere within their matmul tolerance, SiLU
    evaluated in fp32 and the result rounded to fp16, stay within the allowance;
    and the allowance is not slack by orders of magnitude."""
    rng = np.random.default_rng(11)
    K, N, M = 384, 64, 4
    W = synth.weight(synth.seed_for("gated-pin", 0), 2 * N, K)
    codes, s, _ = oracle.reference_layer(W, [2, 6, 3])
    w = oracle.dequant(codes, s, [2, 6, 3])
    wg, wu = np.ascontiguousarray(w[:, :N]), np.ascontiguousarray(w[:, N:])
    x = synth.activations(synth.seed_for("gated-pin-x", 0), M, K)
    h, allow = oracle.gated(x, wg, wu)
    g, bg = oracle.gemm(x, wg)
    u, bu = oracle.gemm(x, wu)
    eg, eu = 2e-3 * bg + 1e-5, 2e-3 * bu + 1e-5
    worst = 0.0
    for sg in (-1.0, -0.5, 0.0, 0.5, 1.0):
        for su in (-1.0, 0.0, 1.0):
            gp = (g + sg * eg).astype(np.float32)
            up = (u + su * eu).astype(np.float32)
            hp = (gp / (np.float32(1) + np.exp(-gp)) * up).astype(np.float16).astype(np.float64)
            worst = max(worst, float(np.max(np.abs(hp - h) / allow)))
    assert worst <= 1.0
    assert worst > 0.05
