"""The five synthetic workloads at full size on the GPU, against the oracle.

Packed bytes, scales and W_hat are compared bit for bit (W_hat for every
linear of configs 1-4).  Outputs are compared on every column for configs 1,
2 and 3 (every M), on every column of 64 seeded rows (plus the first and
last) for config 4, and on seeded column samples for the 560 linears of
config 5, the oracle computing each from packed storage or from W itself.
"""
import numpy as np
import pytest

import oracle
from synth import workloads
from tests.gpu_helpers import assert_within, note, sample_cols, to_dev, y_to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def exq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_bitrate_quantized_amd as m
    return m


def check_linear(exq, spec, Ms, ncols=256, nrows=None, dequant=True):
    note("cfg%d %s K=%d N=%d: generate + pack" % (spec.config, spec.name, spec.K, spec.N))
    W = workloads.make_weight(spec)
    widths = workloads.make_widths(spec, W)
    q, s = exq.exq_pack(W, widths)
    codes, s_ref, q_ref = oracle.reference_layer(W, widths)
    np.testing.assert_array_equal(s, s_ref)
    np.testing.assert_array_equal(q, q_ref)
    del W
    layer = exq.Layer(spec.K, spec.N, widths, q, s)
    if dequant:
        note("cfg%d %s dequant" % (spec.config, spec.name))
        wd = layer.dequant().cpu().numpy().view(np.uint16)
        np.testing.assert_array_equal(wd, oracle.dequant(codes, s_ref, widths))
        del wd
    del codes
    cols = sample_cols(spec.N, ncols, spec.w_seed() & 0xFFFF)
    worst = 0.0
    for M in Ms:
        x = workloads.make_x(spec, M)
        note("cfg%d %s gemm M=%d" % (spec.config, spec.name, M))
        y = y_to_np(layer.gemm(to_dev(x)))
        rows = np.arange(M)
        if nrows is not None and M > nrows:
            rng = np.random.default_rng(M)
            rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, nrows, replace=False)]))
        y_ref, bnd = oracle.gemm_packed_cols(x[rows], q_ref, s_ref, widths, spec.K, spec.N, cols)
        worst = max(worst, assert_within(y[np.ix_(rows, cols)], y_ref, bnd, "cfg%d %s M=%d" % (spec.config, spec.name, M)))
    layer.close()
    return worst


def test_cfg1_uniform_4bit_4096(exq):
    spec = workloads.linears(1)[0]
    check_linear(exq, spec, workloads.M_VALUES[1], ncols=spec.N)


def test_cfg2_mixed_8192(exq):
    spec = workloads.linears(2)[0]
    check_linear(exq, spec, workloads.M_VALUES[2], ncols=spec.N)


@pytest.mark.parametrize("idx", range(7))
def test_cfg3_block_linear(exq, idx):
    spec = workloads.linears(3)[idx]
    check_linear(exq, spec, workloads.M_VALUES[3], ncols=spec.N)


@pytest.mark.parametrize("idx", range(7))
def test_cfg4_prefill_linear(exq, idx):
    spec = workloads.linears(4)[idx]
    check_linear(exq, spec, workloads.M_VALUES[4], ncols=spec.N, nrows=64)


CFG5_SAMPLE = (0, 6, 37 * 7 + 4, 79 * 7 + 1)


@pytest.mark.parametrize("idx", CFG5_SAMPLE)
def test_cfg5_stack_sample(exq, idx):
    spec = workloads.linears(5)[idx]
    check_linear(exq, spec, workloads.M_VALUES[5], ncols=128, dequant=False)


def test_cfg5_every_linear(exq):
    """Configuration 5 in full: every one of the 560 linears at M = 1 and
    M = 16, each on a column sample whose reference the
    oracle derives from W itself (its own quantizer, dequantization and fp64
    matmul on those columns: the quantizer works per (group, column))."""
    specs = workloads.linears(5)
    wbuf = None
    worst = 0.0
    for i, spec in enumerate(specs):
        if i % 70 == 0:
            note("cfg5 sweep: linear %d/%d" % (i, len(specs)))
        if wbuf is None or wbuf.size < spec.N * spec.K:
            wbuf = np.empty(spec.N * spec.K, dtype=np.float32)
        W = wbuf[: spec.N * spec.K].reshape(spec.N, spec.K)
        workloads.make_weight(spec, out=W)
        widths = workloads.make_widths(spec, W)
        q, s = exq.exq_pack(W, widths)
        layer = exq.Layer(spec.K, spec.N, widths, q, s)
        cols = sample_cols(spec.N, 64, spec.w_seed() & 0xFFFF)
        codes_c, scales_c = oracle.quantize(W[cols], widths)
        w_ref = oracle.dequant(codes_c, scales_c, widths)
        for M in (1, 16):
            x = workloads.make_x(spec, M)
            y = y_to_np(layer.gemm(to_dev(x)))
            y_ref, bnd = oracle.gemm(x, w_ref)
            worst = max(worst, assert_within(y[:, cols], y_ref, bnd, "cfg5 %s M=%d" % (spec.name, M)))
        layer.close()
    note("cfg5 sweep done, worst error / tolerance %.3f" % worst)


@pytest.mark.parametrize("M", [1, 16])
def test_cfg3_block_as_one_plan(exq, M):
    """The seven linears of a 70B-shaped block as one decode plan (the launch
    bench.py times), every output checked against the oracle (its own packed
    layer, bit-exact with the library's)."""
    specs = workloads.linears(3)
    layers, refs, xs_h = [], [], []
    for spec in specs:
        W = workloads.make_weight(spec)
        widths = workloads.make_widths(spec, W)
        q, s = exq.exq_pack(W, widths)
        _, s_ref, q_ref = oracle.reference_layer(W, widths)
        np.testing.assert_array_equal(q, q_ref)
        refs.append((q_ref, s_ref, widths))
        layers.append(exq.Layer(spec.K, spec.N, widths, q, s))
        xs_h.append(workloads.make_x(spec, M))
        del W
    xs = [to_dev(x) for x in xs_h]
    ys = [torch.empty((M, l.N), dtype=torch.float16, device="cuda") for l in layers]
    note("cfg3 block plan M=%d" % M)
    plan = exq.Plan(layers, xs, ys, M)
    plan.run()
    for spec, x, y, (q, s, widths) in zip(specs, xs_h, ys, refs):
        cols = np.arange(spec.N, dtype=np.int64)
        y_ref, bnd = oracle.gemm_packed_cols(x, q, s, widths, spec.K, spec.N, cols)
        assert_within(y_to_np(y), y_ref, bnd, "cfg3 plan %s M=%d" % (spec.name, M))
    plan.close()
    for l in layers:
        l.close()


def test_cfg4_block_as_one_plan(exq):
    """The seven linears of a 70B-shaped block at M = 2048 as one prefill plan
    (the launch bench.py times, with the tiles of each XCD's last round cut
    along K), every column of a row sample against the oracle, and the same
    bits on a second and third run."""
    specs = workloads.linears(4)
    M = workloads.M_VALUES[4][0]
    rng = np.random.default_rng(M)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 32, replace=False)]))
    layers, refs, xs_h = [], [], []
    for spec in specs:
        note("cfg4 plan %s: generate + pack" % spec.name)
        W = workloads.make_weight(spec)
        widths = workloads.make_widths(spec, W)
        q, s = exq.exq_pack(W, widths)
        codes, s_ref, q_ref = oracle.reference_layer(W, widths)
        np.testing.assert_array_equal(s, s_ref)
        np.testing.assert_array_equal(q, q_ref)
        del W, codes
        layers.append(exq.Layer(spec.K, spec.N, widths, q, s))
        refs.append((q_ref, s_ref, widths, np.arange(spec.N, dtype=np.int64)))
        xs_h.append(workloads.make_x(spec, M))
    xs = [to_dev(x) for x in xs_h]
    ys = [torch.empty((M, l.N), dtype=torch.float16, device="cuda") for l in layers]
    note("cfg4 block plan M=%d" % M)
    plan = exq.Plan(layers, xs, ys, M)
    plan.run()
    first = [y_to_np(y).copy() for y in ys]
    for spec, x, g, (q, s, widths, cols) in zip(specs, xs_h, first, refs):
        y_ref, bnd = oracle.gemm_packed_cols(x[rows], q, s, widths, spec.K, spec.N, cols)
        assert_within(g[np.ix_(rows, cols)], y_ref, bnd, "cfg4 plan %s" % spec.name)
    for _ in range(2):
        plan.run()
        for y, g in zip(ys, first):
            np.testing.assert_array_equal(y_to_np(y), g)
    plan.close()
    for l in layers:
        l.close()
