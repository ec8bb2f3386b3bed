"""GPU parity of the HIP path against the CPU oracle, through the C-ABI.

Bar: packed bytes, scales and dequantized weights bit-exact; matmul outputs
within |y - y_ref| <= 2e-3 * sum|x*w| + 1e-5 per output; special cases
(zero, one-hot, integer closed form, power-of-two scales, doubling) bit-exact.
"""
import os

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import assert_within, note, sample_cols, to_dev, y_to_np

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
    np.testing.assert_array_equal(s, s_ref)
    np.testing.assert_array_equal(q, q_ref)
    N, K = W.shape
    return exq.Layer(K, N, widths, q, s), codes, s_ref, q_ref


def full_check(exq, W, widths, Ms, tag):
    N, K = W.shape
    layer, codes, s_ref, q_ref = make_layer(exq, W, widths)
    note("%s dequant K=%d N=%d" % (tag, K, N))
    wd = layer.dequant().cpu().numpy().view(np.uint16)
    w_ref = oracle.dequant(codes, s_ref, widths)
    np.testing.assert_array_equal(wd, w_ref)
    worst = 0.0
    for M in Ms:
        x = synth.activations(synth.seed_for(tag, "x", M), M, K)
        note("%s gemm M=%d" % (tag, M))
        y = y_to_np(layer.gemm(to_dev(x)))
        y_ref, bnd = oracle.gemm(x, w_ref)
        worst = max(worst, assert_within(y, y_ref, bnd, "%s M=%d" % (tag, M)))
    layer.close()
    return worst


# ------------------------------------------------------------ small shapes

SMALL_WIDTHS = [2, 3, 4, 5, 6, 8, 3]


def test_small_layer_every_width_ragged_M(exq):
    W = synth.weight(synth.seed_for("small"), 192, 128 * len(SMALL_WIDTHS))
    full_check(exq, W, SMALL_WIDTHS, [1, 2, 3, 4, 5, 7, 8, 9, 12, 13, 16, 17, 33], "small")


@pytest.mark.parametrize("b", [2, 3, 4, 5, 6, 8])
def test_single_group_each_width(exq, b):
    W = synth.weight(synth.seed_for("single", b), 64, 128)
    full_check(exq, W, [b], [1, 6], "single-b%d" % b)


@pytest.mark.parametrize("widths", [
    [2, 2, 3, 8, 2, 4, 2, 6, 5, 2, 3, 2, 2, 3, 2, 2, 2, 2, 3, 2],   # 20 groups, every width
    [8, 3, 2],                                                    # fewer groups than waves
    [2] * 40 + [3] * 9 + [6, 8, 4, 5],                            # long runs, one wave per width
    [5, 6, 8, 8, 6, 5, 4, 3, 2, 8, 8, 8, 8],                      # wide groups dominate
])
def test_wave_chunking(exq, widths):
    W = synth.weight(synth.seed_for("chunks", *widths), 320, 128 * len(widths))
    full_check(exq, W, widths, [1, 4, 16], "chunks%d" % len(widths))


def test_zero_and_one_hot_and_doubling(exq):
    widths = [3, 5, 2, 8]
    W = synth.weight(synth.seed_for("special"), 128, 512)
    layer, codes, s_ref, q_ref = make_layer(exq, W, widths)
    w_ref = oracle.dequant(codes, s_ref, widths)
    note("special: zero input")
    for M in (1, 3, 16, 20):
        y = y_to_np(layer.gemm(to_dev(np.zeros((M, 512), dtype=np.float16))))
        assert np.all(y == 0)
    note("special: one-hot rows")
    ks = np.array([0, 1, 127, 128, 200, 255, 256, 300, 383, 384, 450, 511, 5, 77, 131, 260])
    x = np.zeros((16, 512), dtype=np.float16)
    x[np.arange(16), ks] = 1.0
    y = y_to_np(layer.gemm(to_dev(x)))
    np.testing.assert_array_equal(y.view(np.uint16), w_ref[ks])
    note("special: y(2x) == 2 y(x)")
    for M in (1, 7):
        x = synth.activations(synth.seed_for("dbl", M), M, 512)
        y1 = y_to_np(layer.gemm(to_dev(x)))
        y2 = y_to_np(layer.gemm(to_dev((x.astype(np.float32) * 2).astype(np.float16))))
        # exact where y is an fp16 normal (fp16 rounding commutes with doubling there)
        normal = np.abs(y1.astype(np.float32)) >= 2.0 ** -13
        np.testing.assert_array_equal(y2[normal], (y1[normal].astype(np.float32) * 2).astype(np.float16))
        assert np.all(np.abs(y2[~normal].astype(np.float64) - 2 * y1[~normal].astype(np.float64)) <= 2.0 ** -24)
    layer.close()


def test_integer_closed_form_all_8bit_unit_scale(exq):
    """All 8-bit, every scale exactly 1, x in {-1,0,1}: y is the integer matmul, bit-exact."""
    rng = np.random.default_rng(17)
    K, N = 384, 128
    Wi = rng.integers(-127, 128, size=(N, K))
    Wi[:, ::128] = 127                      # max |w| = 127 in every (group, column): scale 1
    W = Wi.astype(np.float32)
    layer, codes, s_ref, _ = make_layer(exq, W, [8, 8, 8])
    assert np.all(s_ref == 0x3C00)
    for M in (1, 4, 16, 40):
        x = rng.integers(-1, 2, size=(M, K)).astype(np.float16)
        note("closed form M=%d" % M)
        y = y_to_np(layer.gemm(to_dev(x)))
        ref = (x.astype(np.int64) @ Wi.T).astype(np.float16)
        np.testing.assert_array_equal(y, ref)
    layer.close()


@pytest.mark.parametrize("b", [2, 3, 4, 5, 6, 8])
def test_power_of_two_scales_exact(exq, b):
    rng = np.random.default_rng(100 + b)
    qmax = (1 << (b - 1)) - 1
    K, N = 256, 64
    e = rng.integers(-6, 3, size=(N, 2))
    Q = rng.integers(-qmax, qmax + 1, size=(N, K))
    Q[:, 0] = qmax
    Q[:, 128] = -qmax
    W = (Q * np.repeat(2.0 ** e, 128, axis=1)).astype(np.float32)
    layer, _, s_ref, _ = make_layer(exq, W, [b, b])
    np.testing.assert_array_equal(s_ref.view(np.float16).astype(np.float64), (2.0 ** e).T)
    for M in (1, 5, 30):
        x = rng.integers(-2, 3, size=(M, K)).astype(np.float16)
        note("pow2 b=%d M=%d" % (b, M))
        y = y_to_np(layer.gemm(to_dev(x)))
        ref = x.astype(np.float64) @ W.astype(np.float64).T
        np.testing.assert_array_equal(y, ref.astype(np.float16))
    layer.close()


def test_determinism_and_guard_bands(exq):
    widths = [2, 3, 2, 8, 2, 2, 4, 2]
    K, N = 1024, 256
    W = synth.weight(synth.seed_for("guard"), N, K)
    layer, *_ = make_layer(exq, W, widths)
    for M in (1, 16, 24):
        x = to_dev(synth.activations(synth.seed_for("guard-x", M), M, K))
        pad = 4096
        buf = torch.full((M * N + 2 * pad,), -12345, dtype=torch.int16, device="cuda")
        out = buf[pad:pad + M * N].view(torch.float16).view(M, N)
        note("guard M=%d" % M)
        layer.gemm(x, out=out)
        first = y_to_np(out).copy()
        layer.gemm(x, out=out)
        np.testing.assert_array_equal(y_to_np(out), first)
        b = buf.cpu().numpy()
        assert np.all(b[:pad] == -12345) and np.all(b[pad + M * N:] == -12345)
    layer.close()


def test_plan_matches_oracle_and_is_repeatable(exq):
    specs = [(256, 64, [2, 3]), (512, 192, [8, 2, 6, 5]), (1024, 128, [2] * 7 + [4]), (384, 320, [3, 3, 4])]
    layers, refs = [], []
    for i, (K, N, widths) in enumerate(specs):
        W = synth.weight(synth.seed_for("plan", i), N, K)
        layer, codes, s_ref, _ = make_layer(exq, W, widths)
        layers.append(layer)
        refs.append(oracle.dequant(codes, s_ref, widths))
    for M in (1, 3, 16):
        xs_h = [synth.activations(synth.seed_for("plan-x", i, M), M, l.K) for i, l in enumerate(layers)]
        xs = [to_dev(x) for x in xs_h]
        ys = [torch.empty((M, l.N), dtype=torch.float16, device="cuda") for l in layers]
        note("plan M=%d" % M)
        plan = exq.Plan(layers, xs, ys, M)
        plan.run()
        got = [y_to_np(y).copy() for y in ys]
        for x, g, w_ref, l in zip(xs_h, got, refs, layers):
            y_ref, bnd = oracle.gemm(x, w_ref)
            assert_within(g, y_ref, bnd, "plan M=%d N=%d" % (M, l.N))
        plan.run()
        for y, g in zip(ys, got):
            np.testing.assert_array_equal(y_to_np(y), g)
        plan.close()
    for l in layers:
        l.close()


def test_plan_with_shared_input(exq):
    """q/k/v-style: several linears of one K read the same x in one plan launch."""
    specs = [(640, 192, [2, 3, 8, 2, 5]), (640, 64, [6, 2, 2, 4, 3]), (640, 64, [3, 3, 2, 2, 2])]
    layers, refs = [], []
    for i, (K, N, widths) in enumerate(specs):
        W = synth.weight(synth.seed_for("plan-shared", i), N, K)
        layer, codes, s_ref, _ = make_layer(exq, W, widths)
        layers.append(layer)
        refs.append(oracle.dequant(codes, s_ref, widths))
    for M in (1, 7, 16):
        x_h = synth.activations(synth.seed_for("plan-shared-x", M), M, 640)
        x = to_dev(x_h)
        ys = [torch.empty((M, l.N), dtype=torch.float16, device="cuda") for l in layers]
        note("plan with shared input M=%d" % M)
        plan = exq.Plan(layers, [x] * len(layers), ys, M)
        plan.run()
        for y, w_ref, l in zip(ys, refs, layers):
            y_ref, bnd = oracle.gemm(x_h, w_ref)
            assert_within(y_to_np(y), y_ref, bnd, "shared-input plan M=%d N=%d" % (M, l.N))
        plan.close()
    for l in layers:
        l.close()


def test_runtime_errors_on_device(exq):
    W = synth.weight(synth.seed_for("err"), 64, 256)
    layer, *_ = make_layer(exq, W, [2, 4])
    x = to_dev(np.zeros((2, 256), dtype=np.float16))
    with pytest.raises(exq.ExqError) as ei:
        exq.exq_gemm(x.data_ptr(), 0, layer.handle, x.data_ptr() + 4096)
    assert ei.value.status == exq.EXQ_ERR_INVALID_ARG
    with pytest.raises(exq.ExqError) as ei:   # y overlaps x
        exq.exq_gemm(x.data_ptr(), 2, layer.handle, x.data_ptr() + 64)
    assert ei.value.status == exq.EXQ_ERR_INVALID_ARG
    with pytest.raises(exq.ExqError):
        exq.exq_gemm(x.data_ptr() + 2, 1, layer.handle, x.data_ptr() + 4096)
    layer.close()


def test_seeded_random_shapes(exq):
    """A seeded sweep of shapes, widths and row counts across the three kernel
    paths (4x4x4 decode, 16-row MFMA decode, prefill), against the oracle."""
    rng = np.random.default_rng(20261203)
    for case in range(24):
        G = int(rng.integers(1, 13))
        K, N = 128 * G, 64 * int(rng.integers(1, 10))
        widths = [int(b) for b in rng.choice([2, 3, 4, 5, 6, 8], size=G)]
        M = int(rng.choice([1, 2, 3, 4, 5, 8, 11, 16, 17, 40, 64, 65, 129, 300]))
        W = synth.weight(synth.seed_for("random-shapes", case), N, K)
        layer, codes, s_ref, _ = make_layer(exq, W, widths)
        x = synth.activations(synth.seed_for("random-shapes-x", case), M, K)
        note("random shape %d: K=%d N=%d M=%d widths=%s" % (case, K, N, M, widths))
        y = y_to_np(layer.gemm(to_dev(x)))
        y_ref, bnd = oracle.gemm(x, oracle.dequant(codes, s_ref, widths))
        assert_within(y, y_ref, bnd, "random shape %d (K=%d N=%d M=%d)" % (case, K, N, M))
        layer.close()


def test_seeded_random_plans(exq):
    """Seeded plans of 1-5 linears of random shapes and widths, decode and
    prefill row counts, against the oracle and repeatable bit for bit."""
    rng = np.random.default_rng(31)
    for case in range(8):
        count = int(rng.integers(1, 6))
        M = int(rng.choice([1, 3, 6, 16, 20, 256, 300]))
        layers, refs, xs_h = [], [], []
        for i in range(count):
            G = int(rng.integers(1, 9))
            K, N = 128 * G, 64 * int(rng.integers(1, 7))
            widths = [int(b) for b in rng.choice([2, 3, 4, 5, 6, 8], size=G)]
            W = synth.weight(synth.seed_for("random-plan", case, i), N, K)
            layer, codes, s_ref, _ = make_layer(exq, W, widths)
            layers.append(layer)
            refs.append(oracle.dequant(codes, s_ref, widths))
            xs_h.append(synth.activations(synth.seed_for("random-plan-x", case, i), M, K))
        xs = [to_dev(x) for x in xs_h]
        ys = [torch.empty((M, l.N), dtype=torch.float16, device="cuda") for l in layers]
        note("random plan %d: %d linears, M=%d" % (case, count, M))
        plan = exq.Plan(layers, xs, ys, M)
        plan.run()
        got = [y_to_np(y).copy() for y in ys]
        for x, g, w_ref, l in zip(xs_h, got, refs, layers):
            y_ref, bnd = oracle.gemm(x, w_ref)
            assert_within(g, y_ref, bnd, "random plan %d M=%d N=%d" % (case, M, l.N))
        plan.run()
        for y, g in zip(ys, got):
            np.testing.assert_array_equal(y_to_np(y), g)
        plan.close()
        for l in layers:
            l.close()


def test_plan_rejects_bad_arguments(exq):
    """exq_plan_create validates before it allocates: an empty list, M < 1, a
    misaligned buffer, an output overlapping an input or another output, and a
    decode plan mixing fp16 and quantized scale storage are INVALID_ARG; the
    corrected arguments make plans."""
    W = synth.weight(synth.seed_for("plan-err"), 128, 256)
    a, *_ = make_layer(exq, W, [3, 5])
    b = exq.Layer.from_weight(W, [3, 5], quantized_scales=True)
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    x0 = buf.data_ptr()
    y0, y1 = x0 + 32768, x0 + 49152

    def expect(handles, xs, ys, M):
        with pytest.raises(exq.ExqError) as ei:
            exq.exq_plan_create(handles, xs, ys, M)
        assert ei.value.status == exq.EXQ_ERR_INVALID_ARG

    expect([], [], [], 1)
    expect([a.handle], [x0], [y0], 0)
    expect([a.handle], [x0 + 2], [y0], 1)                        # misaligned x
    expect([a.handle], [x0], [x0 + 256], 2)                      # y overlaps x
    expect([a.handle, a.handle], [x0, x0], [y0, y0 + 128], 2)    # outputs overlap
    expect([a.handle, b.handle], [x0, x0], [y0, y1], 1)          # decode plan, two scale storages
    for handles, M in (([a.handle, a.handle], 2), ([a.handle, b.handle], 20), ([b.handle, b.handle], 1)):
        exq.exq_plan_destroy(exq.exq_plan_create(handles, [x0, x0], [y0, y1], M))
    a.close()
    b.close()


def test_plan_validates_every_entry_before_expanding_scales(exq):
    """A prefill plan whose first entry has quantized scales and whose second
    entry is invalid fails with INVALID_ARG before the first entry's fp16
    scales are expanded (an 8 MiB device allocation and a kernel launch).
    The device's free memory shows the expansion: a valid plan over the same
    layer allocates it (the control), the failed one does not."""
    G, N, M = 64, 65536, 20
    K = 128 * G
    widths = np.full(G, 2, dtype=np.uint8)
    q = torch.zeros(exq.exq_packed_bytes(K, N, widths), dtype=torch.uint8, device="cuda")
    qs = torch.zeros(G * N // 2, dtype=torch.uint8, device="cuda")
    ref = torch.zeros(N, dtype=torch.int16, device="cuda")
    W = synth.weight(synth.seed_for("plan-err-2"), 128, 256)
    a, *_ = make_layer(exq, W, [3, 5])
    big = [exq.exq_layer_create_qs(K, N, widths, q.data_ptr(), qs.data_ptr(), ref.data_ptr()) for _ in range(2)]
    xb = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    yb = torch.zeros((M, N), dtype=torch.float16, device="cuda")
    xa = torch.zeros((M, 256), dtype=torch.float16, device="cuda")
    ya = torch.zeros((M, 128), dtype=torch.float16, device="cuda")
    torch.cuda.synchronize()
    expansion = 2 * G * N
    try:
        note("plan validation order: control")
        free0 = torch.cuda.mem_get_info()[0]
        exq.exq_plan_destroy(exq.exq_plan_create([big[0], a.handle], [xb.data_ptr(), xa.data_ptr()],
                                                 [yb.data_ptr(), ya.data_ptr()], M))
        torch.cuda.synchronize()
        free1 = torch.cuda.mem_get_info()[0]
        if free0 - free1 < expansion:
            pytest.skip("the device's free-memory counter does not show an %d-byte allocation" % expansion)
        note("plan validation order: misaligned second entry")
        with pytest.raises(exq.ExqError) as ei:
            exq.exq_plan_create([big[1], a.handle], [xb.data_ptr(), xa.data_ptr() + 2],
                                [yb.data_ptr(), ya.data_ptr()], M)
        assert ei.value.status == exq.EXQ_ERR_INVALID_ARG
        torch.cuda.synchronize()
        free2 = torch.cuda.mem_get_info()[0]
        assert free1 - free2 < expansion, "the failed call allocated %d bytes" % (free1 - free2)
    finally:
        for h in big:
            exq.exq_layer_destroy(h)
        a.close()


def test_n_multiple_of_16(exq):
    """N = 80 (a multiple of 16, not of 64): decode (16-column tiles), prefill,
    gated and dequant match the oracle; the 64-column choices report
    UNSUPPORTED; prefill plans take it, decode plans refuse it."""
    K, N = 640, 80
    widths = [2, 8, 3, 6, 5]
    W = synth.weight(synth.seed_for("n80"), N, K)
    layer, codes, s_ref, q_ref = make_layer(exq, W, widths)
    w_ref = oracle.dequant(codes, s_ref, widths)
    try:
        note("N=80 dequant")
        np.testing.assert_array_equal(layer.dequant().cpu().numpy().view(np.uint16), w_ref)
        for M in (1, 4, 5, 16, 33, 300):
            x = synth.activations(synth.seed_for("n80-x", M), M, K)
            note("N=80 gemm M=%d" % M)
            y = y_to_np(layer.gemm(to_dev(x)))
            y_ref, bnd = oracle.gemm(x, w_ref)
            assert_within(y, y_ref, bnd, "N=80 M=%d" % M)
        with pytest.raises(exq.ExqError) as ei:
            exq.exq_set_variant(layer.handle, 4, exq.VARIANT_DECODE64)
        assert ei.value.status == exq.EXQ_ERR_UNSUPPORTED
        x = to_dev(synth.activations(synth.seed_for("n80-tune"), 4, K))
        y = torch.empty((4, N), dtype=torch.float16, device="cuda")
        note("N=80 autotune M=4")
        choice, times = exq.exq_autotune(x.data_ptr(), 4, layer.handle, y.data_ptr(), None, 2, 5)
        assert choice == exq.VARIANT_DECODE16 and times[1] == -1.0
        exq.exq_set_variant(layer.handle, 4, exq.VARIANT_DEFAULT)
        # gated pair of N = 80
        W2 = synth.weight(synth.seed_for("n80-up"), N, K)
        up, c2, s2, _ = make_layer(exq, W2, widths)
        w2 = oracle.dequant(c2, s2, widths)
        for M in (1, 16, 300):
            x = synth.activations(synth.seed_for("n80-g", M), M, K)
            note("N=80 gated M=%d" % M)
            h = y_to_np(exq.gemm_gated(to_dev(x), layer, up))
            h_ref, allow = oracle.gated(x, w_ref, w2)
            ok, worst = oracle.within_allowance(h, h_ref, allow)
            assert ok, "N=80 gated M=%d: %.3f" % (M, worst)
        # plans
        for M, ok_expected in ((1, False), (16, False), (40, True)):
            xs = [to_dev(synth.activations(synth.seed_for("n80-p", M, i), M, K)) for i in range(2)]
            ys = [torch.empty((M, N), dtype=torch.float16, device="cuda") for _ in range(2)]
            if not ok_expected:
                with pytest.raises(exq.ExqError) as ei:
                    exq.Plan([layer, up], xs, ys, M)
                assert ei.value.status == exq.EXQ_ERR_UNSUPPORTED
                continue
            note("N=80 prefill plan M=%d" % M)
            p = exq.Plan([layer, up], xs, ys, M)
            p.run()
            for i, wr in enumerate((w_ref, w2)):
                y_ref, bnd = oracle.gemm(xs[i].cpu().numpy(), wr)
                assert_within(y_to_np(ys[i]), y_ref, bnd, "N=80 plan M=%d entry %d" % (M, i))
            p.close()
        up.close()
    finally:
        layer.close()
