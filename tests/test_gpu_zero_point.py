"""GPU parity at the method's edge: weights whose code is the zero point under
large activations.

Each (group, column) of W holds one non-zero weight; every other code of the
group is the zero point z = 2^(b-1) (w_hat = 0).  Every row of x is zero at
the positions where any column has its non-zero weight, and elsewhere in the
group holds one large activation (about 3e4) among many tiny ones (about
1e-3).  So x*w_hat is zero term by term (variant "exact zero") or, with tiny
activations on the non-zero weights (variant "tiny"), y_ref and
B = sum|x*w_hat| are small while sum|x| is huge.  A kernel that multiplies
the codes c and removes z * sum(x) afterwards rounds two large sums of the
same activations separately; its error scales with z * sum|x| and misses
the stated bound |y - y_ref| <= 2e-3 * B + 1e-5 by orders of magnitude.  A
kernel that forms (c - z) exactly before its multiply-accumulate computes
products that are exact zeros there.

Every kernel path is covered through the C-ABI: the 4x4x4 decode with 16-
and 64-column tiles (M = 1 and 4), the 16-row MFMA decode (M = 16), 16-row
slices (M = 40), decode plans, the fused gate/up product, quantized group
scales, and the prefill kernel (M = 300).
"""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import assert_within, note, to_dev, y_to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

WIDTHS = [2, 3, 4, 5, 6, 8]
N = 128
K = 128 * len(WIDTHS)


@pytest.fixture(scope="module")
def exq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_bitrate_quantized_amd as m
    return m


def edge_case(seed: int, M: int, tiny_on_weights: bool, n_cols: int = N):
    """(W fp32 [N][K], x fp16 [M][K]) of the module docstring's structure."""
    rng = np.random.default_rng(seed)
    W = np.zeros((n_cols, K), dtype=np.float32)
    x = np.zeros((M, K), dtype=np.float32)
    for g in range(len(WIDTHS)):
        base = 128 * g
        hot = rng.choice(128, size=4, replace=False)          # where the non-zero weights sit
        rest = np.setdiff1d(np.arange(128), hot)
        k0 = hot[rng.integers(0, 4, size=n_cols)]
        W[np.arange(n_cols), base + k0] = rng.choice([-1.0, 1.0], size=n_cols) * rng.uniform(100.0, 1000.0, size=n_cols)
        for m in range(M):
            x[m, base + rest] = rng.uniform(-1e-3, 1e-3, size=rest.size)
            big = rng.choice(rest)
            x[m, base + big] = rng.choice([-1.0, 1.0]) * rng.uniform(2.0e4, 3.2e4)
            if tiny_on_weights:
                x[m, base + hot] = rng.uniform(-1e-3, 1e-3, size=hot.size)
    return W, x.astype(np.float16)


def reference(W):
    codes, s, q = oracle.reference_layer(W, WIDTHS)
    return codes, s, q, oracle.dequant(codes, s, WIDTHS)


def check(y, x, w_ref, exact_zero: bool, what: str):
    y_ref, bnd = oracle.gemm(x, w_ref)
    if exact_zero:
        assert np.all(y_ref == 0) and np.all(bnd == 0), "the inputs must make every product zero"
        assert np.all(y.astype(np.float64) == 0), "%s: %d nonzero outputs, max |y| %g" % (
            what, np.count_nonzero(y), float(np.max(np.abs(y.astype(np.float64)))))
    assert_within(y, y_ref, bnd, what)


CASES = [  # (M, variant forced through exq_set_variant or None for the default rule)
    (1, "decode16"), (1, "decode64"), (4, "decode16"), (4, "decode64"), (16, "decode16"), (16, "decode64"),
    (7, None), (40, None), (300, None),
]


@pytest.mark.parametrize("tiny", [False, True], ids=["exact-zero", "tiny"])
@pytest.mark.parametrize("M,variant", CASES)
def test_zero_code_weights_under_large_activations(exq, M, variant, tiny):
    W, x = edge_case(1000 + M, M, tiny)
    codes, s, q, w_ref = reference(W)
    layer = exq.Layer(K, N, WIDTHS, q, s)
    try:
        if variant is not None:
            exq.exq_set_variant(layer.handle, M, {"decode16": exq.VARIANT_DECODE16,
                                                  "decode64": exq.VARIANT_DECODE64}[variant])
        note("zero-point edge M=%d %s tiny=%d" % (M, variant, tiny))
        y = y_to_np(layer.gemm(to_dev(x)))
        check(y, x, w_ref, not tiny, "M=%d %s" % (M, variant))
    finally:
        layer.close()


@pytest.mark.parametrize("tiny", [False, True], ids=["exact-zero", "tiny"])
@pytest.mark.parametrize("M", [1, 3, 16])
def test_zero_code_weights_plan(exq, M, tiny):
    """Two linears in one decode plan (64-column tiles), each on its own x."""
    layers, xs, ys, refs = [], [], [], []
    for i in range(2):
        W, x = edge_case(2000 + 10 * M + i, M, tiny)
        codes, s, q, w_ref = reference(W)
        layers.append(exq.Layer(K, N, WIDTHS, q, s))
        xs.append(to_dev(x))
        ys.append(torch.empty((M, N), dtype=torch.float16, device="cuda"))
        refs.append((x, w_ref))
    plan = exq.Plan(layers, xs, ys, M)
    try:
        note("zero-point edge plan M=%d tiny=%d" % (M, tiny))
        plan.run()
        for i, (x, w_ref) in enumerate(refs):
            check(y_to_np(ys[i]), x, w_ref, not tiny, "plan M=%d linear %d" % (M, i))
    finally:
        plan.close()
        for l in layers:
            l.close()


@pytest.mark.parametrize("M", [1, 4, 16])
def test_zero_code_weights_gated(exq, M):
    """gate and up both of the edge structure on one x: h = SiLU(g) * u."""
    Wg, x = edge_case(3000 + M, M, True)
    Wu = (np.float32(-0.7) * Wg).astype(np.float32)   # non-zero where gate's are: on tiny activations
    _, sg, qg, wg = reference(Wg)
    _, su, qu, wu = reference(Wu)
    lg, lu = exq.Layer(K, N, WIDTHS, qg, sg), exq.Layer(K, N, WIDTHS, qu, su)
    try:
        note("zero-point edge gated M=%d" % M)
        h = y_to_np(exq.gemm_gated(to_dev(x), lg, lu))
        h_ref, allow = oracle.gated(x, wg, wu)
        ok, worst = oracle.within_allowance(h, h_ref, allow)
        assert ok, "gated M=%d: worst error / allowance %.3f" % (M, worst)
    finally:
        lg.close()
        lu.close()


@pytest.mark.parametrize("M", [1, 16])
def test_zero_code_weights_quantized_scales(exq, M):
    """The same structure packed with quantized group scales (4-bit codes)."""
    W, x = edge_case(4000 + M, M, False)
    codes, ref, qscale, scales = oracle.quantize_qs(W, WIDTHS)
    q = oracle.pack(codes, WIDTHS)
    w_ref = oracle.dequant(codes, scales, WIDTHS)
    layer = exq.Layer(K, N, WIDTHS, q, qscale, ref=ref)
    try:
        note("zero-point edge quantized scales M=%d" % M)
        y = y_to_np(layer.gemm(to_dev(x)))
        check(y, x, w_ref, True, "qs M=%d" % M)
    finally:
        layer.close()
