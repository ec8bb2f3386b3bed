"""Pins of the CPU oracle against things other than itself.

* fp16 rounding: numpy's float64 -> float16 cast (correctly rounded, ties to even).
* bit layout: bijection of the address function, brute-force enumeration of
  every code at every position and width (round trip), and byte-for-byte
  agreement with an independently written pure-Python layout walker.
* dequantization: every (width, code) under special scales against numpy.
* matmul: integer closed form, power-of-two scales, one-hot rows, math.fsum.
* quantizer: round-to-nearest invariants and degenerate groups.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from oracle import bitref

WIDTHS = (2, 3, 4, 5, 6, 8)


def np_f16_bits(v):
    with np.errstate(over="ignore"):
        return int(np.array([v], dtype=np.float64).astype(np.float16).view(np.uint16)[0])


# ------------------------------------------------------------------ fp16

def test_f16_from_double_matches_numpy():
    rng = np.random.default_rng(1)
    vals = list(rng.standard_normal(20000) * 10.0 ** rng.uniform(-9, 5, 20000))
    # exact ties between neighbours, in the normal and subnormal ranges
    for e in range(-24, 16):
        for m in (0, 1, 2, 1023, 1024, 2045, 2046, 2047):
            vals.append((2048 + 2 * m + 1) * 2.0 ** (e - 12))
    vals += [(2 * m + 1) * 2.0 ** -25 for m in range(0, 1030, 7)]
    vals += [0.0, -0.0, 65504.0, 65519.999, 65520.0, 70000.0, 2.0 ** -24, 2.0 ** -25,
             2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 6.1e-5, -6.1e-5, 1e-30]
    for v in vals:
        assert oracle.f16_from_double(v) == np_f16_bits(v), v


def test_f16_to_double_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    for h in range(0, 65536, 1):
        got = oracle.f16_to_double(h)
        r = ref[h]
        if math.isnan(r):
            assert math.isnan(got)
        else:
            assert got == r and math.copysign(1, got) == math.copysign(1, r), h


# ---------------------------------------------------------------- layout

@pytest.mark.parametrize("b", WIDTHS)
def test_address_function_is_a_bijection(b):
    seen = {}
    for k in range(128):
        total = 0
        for plane in (0, 1):
            dw, bit, w = oracle.field_position(b, k, plane)
            if w == 0:
                continue
            assert 0 <= dw < 4 * b
            assert bit >= 0 and bit + w <= 32
            for i in range(w):
                key = (dw, bit + i)
                assert key not in seen
                seen[key] = (k, total + i)
            total += w
        assert total == b
    assert len(seen) == 128 * b


@pytest.mark.parametrize("b", WIDTHS)
def test_brute_force_every_code_every_position(b):
    """Column t holds code (i + t) mod 2^b at position i: every code at every position."""
    n = 1 << b
    codes = np.array([[(i + t) % n for i in range(128)] for t in range(n)], dtype=np.uint8)
    widths = [b]
    q = oracle.pack(codes, widths)
    assert q.size == 16 * b * n
    np.testing.assert_array_equal(oracle.unpack(q, 128, n, widths), codes)
    np.testing.assert_array_equal(q, bitref.pack(codes, widths))
    np.testing.assert_array_equal(bitref.unpack(q, 128, n, widths), codes)


def test_multi_group_layout_and_size_invariant():
    rng = np.random.default_rng(7)
    widths = np.array([2, 3, 4, 5, 6, 8, 3, 2], dtype=np.uint8)
    K, N = 128 * widths.size, 16
    codes = np.zeros((N, K), dtype=np.uint8)
    for g, b in enumerate(widths):
        codes[:, 128 * g:128 * (g + 1)] = rng.integers(0, 1 << int(b), size=(N, 128))
    q = oracle.pack(codes, widths)
    assert q.size == sum(int(b) * 128 * N // 8 for b in widths) == oracle.packed_bytes(K, N, widths)
    np.testing.assert_array_equal(q, bitref.pack(codes, widths))
    np.testing.assert_array_equal(oracle.unpack(q, K, N, widths), codes)
    # a group's block is contiguous and starts at 16*N*P_g
    P = np.concatenate([[0], np.cumsum(widths.astype(int))])
    for g in range(widths.size):
        sub = codes.copy()
        sub[:, 128 * g:128 * (g + 1)] = 0
        q2 = oracle.pack(sub, widths)
        diff = np.nonzero(q != q2)[0]
        if diff.size:
            assert diff.min() >= 16 * N * P[g] and diff.max() < 16 * N * P[g + 1]


# --------------------------------------------------------------- dequant

def _scale_set():
    rng = np.random.default_rng(3)
    fixed = [0x3C00, 0x0400, 0x0001, 0x0155, 0x03FF, 0x7BFF, 0x0000, 0x2E66]
    rand = list(rng.integers(0, 0x7C00, size=1000))
    return np.array(fixed + rand, dtype=np.uint16)


@pytest.mark.parametrize("b", WIDTHS)
def test_dequant_every_code_against_numpy(b):
    scales = _scale_set()
    N = scales.size
    z = 1 << (b - 1)
    for c0 in range(0, 1 << b, 37 if b == 8 else 1):
        codes = np.full((N, 128), c0, dtype=np.uint8)
        codes[:, 1] = (c0 + 1) % (1 << b)
        wh = oracle.dequant(codes, scales.reshape(1, N), [b])
        sv = scales.view(np.float16).astype(np.float64)
        for col in (0, 1):
            c = int(codes[0, col])
            with np.errstate(over="ignore"):
                ref = ((c - z) * sv).astype(np.float16).view(np.uint16)
            np.testing.assert_array_equal(wh[col], ref)


# ------------------------------------------------------------------ gemm

def test_gemm_integer_closed_form_all_8bit_unit_scales():
    rng = np.random.default_rng(11)
    M, K, N = 5, 384, 64
    codes = rng.integers(0, 256, size=(N, K)).astype(np.uint8)
    scales = np.full((K // 128, N), 0x3C00, dtype=np.uint16)
    wh = oracle.dequant(codes, scales, [8] * (K // 128))
    x = rng.integers(-1, 2, size=(M, K)).astype(np.float16)
    y, bnd = oracle.gemm(x, wh)
    ref = x.astype(np.int64) @ (codes.astype(np.int64).T - 128)
    np.testing.assert_array_equal(y, ref.astype(np.float64))
    np.testing.assert_array_equal(bnd, np.abs(x.astype(np.int64)) @ np.abs(codes.astype(np.int64).T - 128))


@pytest.mark.parametrize("b", WIDTHS)
def test_gemm_power_of_two_scales_every_width(b):
    rng = np.random.default_rng(b)
    M, K, N = 3, 256, 32
    codes = rng.integers(0, 1 << b, size=(N, K)).astype(np.uint8)
    e = rng.integers(-8, 4, size=(2, N))
    scales = (2.0 ** e).astype(np.float16).view(np.uint16)
    wh = oracle.dequant(codes, scales, [b, b])
    x = rng.integers(-3, 4, size=(M, K)).astype(np.float16)
    y, _ = oracle.gemm(x, wh)
    z = 1 << (b - 1)
    wexact = (codes.astype(np.float64).T - z) * np.repeat(2.0 ** e, 128, axis=0)
    np.testing.assert_array_equal(y, x.astype(np.float64) @ wexact)


def test_gemm_one_hot_rows_return_weights():
    rng = np.random.default_rng(5)
    K, N = 256, 48
    widths = [3, 6]
    W = synth.weight(synth.seed_for("onehot"), N, K)
    codes, scales = oracle.quantize(W, widths)
    wh = oracle.dequant(codes, scales, widths)
    ks = rng.choice(K, size=8, replace=False)
    x = np.zeros((8, K), dtype=np.float16)
    x[np.arange(8), ks] = 1.0
    y, _ = oracle.gemm(x, wh)
    np.testing.assert_array_equal(y, wh[ks].view(np.float16).astype(np.float64))


def test_gemm_against_fsum():
    rng = np.random.default_rng(9)
    M, K, N = 3, 256, 8
    x = rng.standard_normal((M, K)).astype(np.float16)
    wh = (rng.standard_normal((K, N)) * 0.02).astype(np.float16).view(np.uint16)
    y, bnd = oracle.gemm(x, wh)
    wf = wh.view(np.float16).astype(np.float64)
    xf = x.astype(np.float64)
    for m in range(M):
        for n in range(N):
            exact = math.fsum(xf[m, k] * wf[k, n] for k in range(K))
            assert abs(y[m, n] - exact) <= K * 2.0 ** -53 * bnd[m, n]
            assert bnd[m, n] == pytest.approx(math.fsum(abs(xf[m, k] * wf[k, n]) for k in range(K)), rel=1e-15)


def test_gemm_packed_cols_matches_dequant_route():
    s = synth.seed_for("packedcols")
    K, N, M = 512, 96, 4
    widths = np.array([2, 8, 3, 5], dtype=np.uint8)
    W = synth.weight(s, N, K)
    codes, scales, q = oracle.reference_layer(W, widths)
    x = synth.activations(s + 1, M, K)
    y_full, b_full = oracle.gemm(x, oracle.dequant(codes, scales, widths))
    cols = [0, 5, 17, 95, 64]
    y, b = oracle.gemm_packed_cols(x, q, scales, widths, K, N, cols)
    np.testing.assert_array_equal(y, y_full[:, cols])
    np.testing.assert_array_equal(b, b_full[:, cols])


# -------------------------------------------------------------- quantizer

@pytest.mark.parametrize("b", WIDTHS)
def test_quantizer_round_to_nearest_invariants(b):
    s = synth.seed_for("rtn", b)
    K, N = 512, 64
    W = synth.weight(s, N, K)
    widths = [b] * (K // 128)
    codes, scales = oracle.quantize(W, widths)
    z, qmax = 1 << (b - 1), (1 << (b - 1)) - 1
    assert codes.min() >= 1 and codes.max() <= (1 << b) - 1
    wh = oracle.dequant(codes, scales, widths).view(np.float16).astype(np.float64).T  # [N][K]
    sv = np.repeat(scales.view(np.float16).astype(np.float64).T, 128, axis=1)  # [N][K]
    amax = np.abs(W.reshape(N, -1, 128)).max(axis=2)
    np.testing.assert_array_equal(scales, (amax.T / np.float32(qmax)).astype(np.float32).astype(np.float16).view(np.uint16))
    inside = np.abs(W / sv) <= qmax
    ulp = np.spacing(np.abs(wh).astype(np.float16)).astype(np.float64)
    err = np.abs(W.astype(np.float64) - wh)
    assert np.all(err[inside] <= sv[inside] / 2 + ulp[inside] / 2 + 1e-12)
    # the group maximum maps to +-qmax
    arg = np.abs(W.reshape(N, -1, 128)).argmax(axis=2)
    for n in range(N):
        for g in range(K // 128):
            c = int(codes[n, 128 * g + arg[n, g]])
            assert abs(c - z) == qmax


def test_quantizer_degenerate_groups():
    W = np.zeros((4, 256), dtype=np.float32)
    W[1, 5] = -0.5          # one nonzero: it becomes -qmax, the rest zero
    W[2, 130] = 1e-9        # scale underflows to fp16 zero -> all codes z
    widths = [3, 4]
    codes, scales = oracle.quantize(W, widths)
    assert scales[0, 0] == 0 and np.all(codes[0, :128] == 4)
    assert codes[1, 5] == 4 - 3 and np.all(np.delete(codes[1, :128], 5) == 4)
    assert scales[1, 2] == 0 and np.all(codes[2, 128:] == 8)
    wh = oracle.dequant(codes, scales, widths)
    assert np.all(wh.view(np.float16)[np.arange(256) != 5] == 0)


@pytest.mark.parametrize("b", WIDTHS)
def test_quantizer_ties_round_to_even(b):
    """Weights that put w/s exactly on a .5 tie, positive and negative, at every
    width: the codes must follow ties-to-even (the quantizer reading R3), which
    the distance inequality above cannot tell from ties-away-from-zero.  The
    expected codes come from numpy's own rint (round-half-even) on fp32, a
    route that shares nothing with the oracle's C code; the library packer is
    held to the same codes."""
    import mixed_bitrate_quantized_amd as exq
    z, qmax = 1 << (b - 1), (1 << (b - 1)) - 1
    s = np.float32(0.125)                               # a power of two: max|w| / qmax is exact
    ties = (np.arange(-qmax, qmax, dtype=np.float32) + np.float32(0.5)) * s   # w / s = -qmax + .5 .. qmax - .5
    N, K = 16, 256
    W = np.empty((N, K), dtype=np.float32)
    for n in range(N):
        for g in range(K // 128):
            blk = np.resize(np.roll(ties, 7 * n + 3 * g), 127)
            top = qmax * s if (n + g) % 2 == 0 else -qmax * s   # the group maximum, either sign
            W[n, 128 * g:128 * g + 128] = np.concatenate([[top], blk]).astype(np.float32)
    widths = [b] * (K // 128)
    codes, scales = oracle.quantize(W, widths)
    assert np.all(scales.view(np.float16) == np.float16(s))
    s16 = np.repeat(scales.view(np.float16).astype(np.float32).T, 128, axis=1)
    r = np.float32(W) / s16
    assert np.all(np.abs(r[:, 1::128] - np.floor(r[:, 1::128])) == 0.5)   # genuinely ties
    want = (np.clip(np.rint(r), -qmax, qmax) + z).astype(np.uint8)
    np.testing.assert_array_equal(codes, want)
    # ties-away-from-zero would differ on every other tie
    away = (np.clip(np.sign(r) * np.floor(np.abs(r) + 0.5), -qmax, qmax) + z).astype(np.uint8)
    assert np.count_nonzero(away != want) >= N * (K // 128) * 127 // 3
    q_lib, s_lib = exq.exq_pack(W, widths)
    np.testing.assert_array_equal(s_lib, scales)
    np.testing.assert_array_equal(oracle.unpack(q_lib, K, N, widths), want)
