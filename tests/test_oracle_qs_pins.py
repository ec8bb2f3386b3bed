"""Pins of the quantized-group-scale rule (oracle.quantize_qs) against an
independent numpy evaluation of each step, closed cases and invariants, and
the library's host packer against the oracle."""
import numpy as np
import pytest

import oracle
import synth

WIDTHS = [2, 3, 4, 5, 6, 8]


def nibbles(qs, N):
    """q[g][n] from the byte layout: low nibble even columns, high nibble odd."""
    G = qs.shape[0]
    q = np.empty((G, N), dtype=np.int64)
    q[:, 0::2] = qs & 15
    q[:, 1::2] = qs >> 4
    return q


def scale_np(R, q, b):
    """fp16 bits of fp32(t * fp32(1/qmax)) rounded to fp16, t = R (q+1)^2 / 256."""
    t = (np.float32(R) * np.float32((q + 1) ** 2) * np.float32(1 / 256)).astype(np.float32)
    inv = np.float32(1) / np.float32(2 ** (b - 1) - 1)
    return np.float16(np.float32(t * inv)).view(np.uint16)


def group_err_np(w, b, s16):
    """(codes, squared error) of the round-to-nearest rule at fp16 scale s16."""
    qmax = 2 ** (b - 1) - 1
    s = np.uint16(s16).view(np.float16).astype(np.float32)
    if s == 0:
        q = np.zeros_like(w)
    else:
        q = np.clip(np.rint((w / s).astype(np.float32)), -qmax, qmax)
    wh = np.float16(np.float32(q) * s).astype(np.float64)
    return (q + 2 ** (b - 1)).astype(np.uint8), float(np.sum((w.astype(np.float64) - wh) ** 2))


def test_qs_rule_against_numpy():
    N, K = 48, 768
    W = synth.weight(synth.seed_for("qs-pin"), N, K).copy()
    W[5] = 0.0                                   # an all-zero column
    W[9, 130] = 0.9                              # an outlier: one group far above the rest
    codes, R, qs, scales = oracle.quantize_qs(W, WIDTHS)
    q = nibbles(qs, N)
    for n in range(N):
        r16 = np.float16(np.abs(W[n]).max()).view(np.uint16)
        assert R[n] == r16
        Rf = np.uint16(R[n]).view(np.float16).astype(np.float32)
        for g, b in enumerate(WIDTHS):
            w = W[n, 128 * g:128 * g + 128]
            if Rf == 0:
                assert q[g, n] == 0 and scales[g, n] == 0
                assert np.all(codes[n, 128 * g:128 * g + 128] == 2 ** (b - 1))
                continue
            amax = np.float32(np.abs(w).max())
            qc = int(min(max(np.ceil(np.float32(16) * np.sqrt(np.float32(amax / Rf))), 1), 16)) - 1
            assert q[g, n] in (qc, qc - 1)
            c_hi, e_hi = group_err_np(w, b, scale_np(Rf, qc, b))
            if qc >= 1:
                c_lo, e_lo = group_err_np(w, b, scale_np(Rf, qc - 1, b))
                want = qc - 1 if e_lo < e_hi else qc
            else:
                want = qc
            assert q[g, n] == want
            assert scales[g, n] == scale_np(Rf, want, b)
            c_want = c_lo if want == qc - 1 else c_hi
            np.testing.assert_array_equal(codes[n, 128 * g:128 * g + 128], c_want)
            # qc covers the range: no code of the group is clipped at scale(qc)
            s_hi = np.uint16(scale_np(Rf, qc, b)).view(np.float16).astype(np.float32)
            assert amax / s_hi <= (2 ** (b - 1) - 1) * (1 + 2 ** -9)


def test_qs_closed_cases():
    """Groups whose range is R (k/16)^2 land on code k - 1 exactly (the smallest
    covering code), and scale(15) at 2 bits is R itself."""
    N, K = 16, 16 * 128
    R = 0.5
    W = np.zeros((N, K), dtype=np.float32)
    for n in range(N):
        for g in range(16):
            W[n, 128 * g] = R * ((g + 1) / 16) ** 2 if g != 15 else R
    widths = [2] * 16
    codes, Rb, qs, scales = oracle.quantize_qs(W, widths)
    q = nibbles(qs, N)
    assert np.all(Rb == np.float16(R).view(np.uint16))
    for g in range(16):
        # the chosen code is g or g - 1 (the lower one only if it quantizes better)
        assert np.all((q[g] == g) | (q[g] == g - 1))
    assert np.all(scales[15][q[15] == 15] == np.float16(R).view(np.uint16))


def test_nibble_layout_covers_every_code_and_parity():
    """A crafted layer puts every code 0..15 on even and on odd columns; the
    bytes decode back to the codes the oracle chose, nibble by nibble."""
    N, K = 32, 128 * 2
    W = np.zeros((N, K), dtype=np.float32)
    for n in range(N):
        W[n, 0] = 1.0                               # group 0 sets R = 1
        W[n, 128] = ((n % 16) + 1) ** 2 / 256.0     # group 1 range = R ((k)/16)^2, k = n % 16 + 1
    codes, R, qs, scales = oracle.quantize_qs(W, [8, 8])
    q = nibbles(qs, N)
    seen = {(int(q[1, n]), n % 2) for n in range(N)}
    assert len({c for c, _ in seen}) >= 12                       # nearly every code occurs
    assert {p for _, p in seen} == {0, 1}
    for n in range(N):
        byte = qs[1, n // 2]
        assert ((byte >> (4 * (n % 2))) & 15) == q[1, n]


def test_library_packer_matches_oracle():
    exq = pytest.importorskip("mixed_bitrate_quantized_amd")
    for i, (N, K, widths) in enumerate(((64, 768, WIDTHS), (192, 1024, [8, 2, 2, 3, 6, 2, 5, 4]))):
        W = synth.weight(synth.seed_for("qs-lib", i), N, K).copy()
        W[7] = 0.0
        W[11, 3] = 1.5
        q, qs, ref = exq.exq_pack_qs(W, widths)
        codes, R, qs_o, _ = oracle.quantize_qs(W, widths)
        np.testing.assert_array_equal(q, oracle.pack(codes, widths))
        np.testing.assert_array_equal(qs, qs_o)
        np.testing.assert_array_equal(ref, R)
    with pytest.raises(exq.ExqError):
        exq.exq_pack_qs(np.zeros((3, 128), dtype=np.float32), [2])   # odd N
