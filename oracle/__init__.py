"""TEST INFRASTRUCTURE ONLY: the CPU oracle for the mixed-bitrate quantized matmul.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The library under
``mixed_bitrate_quantized_amd`` never does, and shares no code with it.

The arithmetic lives in ``exq_oracle.c`` (plain C, scalar loops, double
precision, built with ``gcc -O2`` and no fast-math); ``bitref.py`` is an
independent pure-Python statement of the same bit layout used to cross-check
it.  Every function here is pinned by ``tests/test_oracle_pins.py``.

Parity pins and what they catch:
  * brute-force code enumeration at every width and position (pack/unpack
    round trip) and a bijection check of the bit address function;
  * the pure-Python layout reader/writer agreeing byte for byte;
  * fp16 rounding against ``numpy.float16`` (a correctly rounded library cast);
  * dequantization of every (width, code) under special scales against numpy;
  * the integer closed form (all 8-bit, unit scales, x in {-1,0,1}), one-hot
    rows and ``math.fsum`` for the matmul;
  * round-to-nearest invariants for the quantizer.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

GROUP = 128
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    src = os.path.join(_HERE, "exq_oracle.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
                               "-ffp-contract=off", src, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.oracle_f16_from_double.argtypes = [ctypes.c_double]
    lib.oracle_f16_from_double.restype = ctypes.c_uint16
    lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_double.restype = ctypes.c_double
    lib.oracle_field_position.argtypes = [i32, i32, i32, vp, vp]
    lib.oracle_field_position.restype = i32
    lib.oracle_packed_bytes.argtypes = [i32, i32, vp]
    lib.oracle_packed_bytes.restype = ctypes.c_uint64
    lib.oracle_pack.argtypes = [vp, i32, i32, vp, vp]
    lib.oracle_unpack.argtypes = [vp, i32, i32, vp, vp]
    lib.oracle_quantize.argtypes = [vp, i32, i32, vp, vp, vp]
    lib.oracle_quantize_qs.argtypes = [vp, i32, i32, vp, vp, vp, vp, vp]
    lib.oracle_dequant.argtypes = [vp, vp, i32, i32, vp, vp]
    lib.oracle_gemm.argtypes = [vp, i32, vp, i32, i32, vp, vp]
    lib.oracle_gemm.restype = None
    lib.oracle_gemm_packed_cols.argtypes = [vp, i32, vp, vp, vp, i32, i32, vp, i64, vp, vp]
    for f in (lib.oracle_pack, lib.oracle_unpack, lib.oracle_quantize, lib.oracle_dequant,
              lib.oracle_gemm_packed_cols):
        f.restype = i32
    _lib = lib
    return lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a: np.ndarray) -> int:
    return a.ctypes.data


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError("oracle %s failed (code %d)" % (what, rc))


def f16_from_double(v: float) -> int:
    return int(_load().oracle_f16_from_double(float(v)))


def f16_to_double(h: int) -> float:
    return float(_load().oracle_f16_to_double(int(h) & 0xFFFF))


def field_position(b: int, k: int, plane: int):
    """(column-local dword, bit offset, field width) of a code's plane field."""
    lib = _load()
    dw, bit = ctypes.c_int(0), ctypes.c_int(0)
    w = lib.oracle_field_position(b, k, plane, ctypes.addressof(dw), ctypes.addressof(bit))
    return dw.value, bit.value, w


def packed_bytes(K: int, N: int, widths) -> int:
    w = _c(widths, np.uint8)
    return int(_load().oracle_packed_bytes(K, N, _p(w)))


def quantize(W: np.ndarray, widths):
    """codes uint8 [N][K], scales fp16 bits uint16 [G][N] from W fp32 [N][K]."""
    W = _c(W, np.float32)
    N, K = W.shape
    w = _c(widths, np.uint8)
    codes = np.empty((N, K), dtype=np.uint8)
    scales = np.empty((K // GROUP, N), dtype=np.uint16)
    _check(_load().oracle_quantize(_p(W), K, N, _p(w), _p(codes), _p(scales)), "quantize")
    return codes, scales


def quantize_qs(W: np.ndarray, widths):
    """Quantized group scales: (codes uint8 [N][K], column range reference R fp16 bits [N],
    qscale bytes [G][N/2], expanded scales fp16 bits [G][N]) from W fp32 [N][K] (see exq_oracle.c)."""
    W = _c(W, np.float32)
    N, K = W.shape
    w = _c(widths, np.uint8)
    G = K // GROUP
    codes = np.empty((N, K), dtype=np.uint8)
    ref = np.empty(N, dtype=np.uint16)
    qscale = np.zeros((G, N // 2), dtype=np.uint8)
    scales = np.empty((G, N), dtype=np.uint16)
    _check(_load().oracle_quantize_qs(_p(W), K, N, _p(w), _p(codes), _p(ref), _p(qscale), _p(scales)),
           "quantize_qs")
    return codes, ref, qscale, scales


def pack(codes: np.ndarray, widths) -> np.ndarray:
    codes = _c(codes, np.uint8)
    N, K = codes.shape
    w = _c(widths, np.uint8)
    out = np.empty(packed_bytes(K, N, w), dtype=np.uint8)
    _check(_load().oracle_pack(_p(codes), K, N, _p(w), _p(out)), "pack")
    return out


def unpack(qweight: np.ndarray, K: int, N: int, widths) -> np.ndarray:
    q = _c(qweight, np.uint8)
    w = _c(widths, np.uint8)
    codes = np.empty((N, K), dtype=np.uint8)
    _check(_load().oracle_unpack(_p(q), K, N, _p(w), _p(codes)), "unpack")
    return codes


def dequant(codes: np.ndarray, scales: np.ndarray, widths) -> np.ndarray:
    """w_hat fp16 bits uint16 [K][N]."""
    codes = _c(codes, np.uint8)
    N, K = codes.shape
    s = _c(scales, np.uint16)
    w = _c(widths, np.uint8)
    out = np.empty((K, N), dtype=np.uint16)
    _check(_load().oracle_dequant(_p(codes), _p(s), K, N, _p(w), _p(out)), "dequant")
    return out


def gemm(x: np.ndarray, w_hat: np.ndarray):
    """(y_ref, bound) in float64 [M][N] from x fp16 [M][K] and w_hat fp16 bits [K][N]."""
    x = _c(np.asarray(x, dtype=np.float16).view(np.uint16), np.uint16)
    wh = _c(w_hat, np.uint16)
    M, K = x.shape
    K2, N = wh.shape
    assert K == K2
    y = np.empty((M, N), dtype=np.float64)
    bnd = np.empty((M, N), dtype=np.float64)
    _load().oracle_gemm(_p(x), M, _p(wh), K, N, _p(y), _p(bnd))
    return y, bnd


def gemm_packed_cols(x: np.ndarray, qweight: np.ndarray, scales: np.ndarray, widths, K: int, N: int, cols):
    """(y_ref, bound) [M][len(cols)] straight from EXQ1 storage, for the given output columns."""
    x = _c(np.asarray(x, dtype=np.float16).view(np.uint16), np.uint16)
    M = x.shape[0]
    q = _c(qweight, np.uint8)
    s = _c(scales, np.uint16)
    w = _c(widths, np.uint8)
    c = _c(cols, np.int64)
    y = np.empty((M, c.size), dtype=np.float64)
    bnd = np.empty((M, c.size), dtype=np.float64)
    _check(_load().oracle_gemm_packed_cols(_p(x), M, _p(q), _p(s), _p(w), K, N, _p(c), c.size,
                                           _p(y), _p(bnd)), "gemm_packed_cols")
    return y, bnd


# Bound on |SiLU'(t)| over all t: SiLU'(t) = s(t) (1 + t (1 - s(t))) with s the
# logistic function peaks at 1.0998 (t = 2.3994) and bottoms at -0.0998.
SILU_SLOPE_BOUND = 1.1


def silu(t):
    """SiLU(t) = t / (1 + e^-t) in float64, elementwise (e^-t overflowing to inf gives the signed-zero limit)."""
    t = np.asarray(t, dtype=np.float64)
    with np.errstate(over="ignore"):
        return t / (1.0 + np.exp(-t))


def gated(x: np.ndarray, w_gate_hat: np.ndarray, w_up_hat: np.ndarray, rel: float = 2e-3, abs_: float = 1e-5):
    """(h_ref, allowance) float64 [M][N] for h = SiLU(x Wg_hat^T) * (x Wu_hat^T).

    h_ref uses the exact (fp64) products g, u of the fp16 inputs.  A result
    whose two products each meet the matmul tolerance (E = rel * sum|x w| +
    abs_) and that evaluates SiLU(g) * u in fp32 and rounds it to fp16 is
    within
        1.1 E_g (|u| + E_u) + |SiLU(g)| E_u + 2^-10 (|h| + those terms) + 1e-7
    of h_ref: the first two terms bound |SiLU(g') u' - SiLU(g) u| for
    |g' - g| <= E_g, |u' - u| <= E_u by the mean value theorem, the third
    the fp32 evaluation and the fp16 rounding (relative 2^-11), the last the
    fp16 subnormal spacing."""
    g, bg = gemm(x, w_gate_hat)
    u, bu = gemm(x, w_up_hat)
    eg, eu = rel * bg + abs_, rel * bu + abs_
    s = silu(g)
    h = s * u
    terms = SILU_SLOPE_BOUND * eg * (np.abs(u) + eu) + np.abs(s) * eu
    return h, terms + 2.0 ** -10 * (np.abs(h) + terms) + 1e-7


def within_allowance(y: np.ndarray, y_ref: np.ndarray, allowance: np.ndarray):
    """(ok, worst ratio of error to allowance) for a per-output allowance."""
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - y_ref)
    ratio = err / allowance
    worst = float(np.max(ratio)) if ratio.size else 0.0
    return bool(np.all(err <= allowance) and np.all(np.isfinite(y))), worst


ALLOC_WIDTHS = (2, 3, 4, 5, 6, 8)


def group_errors(W: np.ndarray) -> np.ndarray:
    """float64 [G][6]: sum over each group's N x 128 weights of (w - w_hat)^2 at each
    width, w_hat from this oracle's own quantize and dequant."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    G = K // GROUP
    err = np.empty((G, len(ALLOC_WIDTHS)), dtype=np.float64)
    for j, b in enumerate(ALLOC_WIDTHS):
        widths = [b] * G
        codes, scales = quantize(W, widths)
        w_hat = dequant(codes, scales, widths).view(np.float16).astype(np.float64)   # [K][N]
        d = W.astype(np.float64).T - w_hat
        err[:, j] = (d * d).reshape(G, GROUP, N).sum(axis=(1, 2))
    return err


def allocate_exact(err, size, budget: int, min_width=None):
    """(minimum total error, widths) of min sum_g err[g][j_g] subject to
    sum_g ALLOC_WIDTHS[j_g] * size[g] <= budget and ALLOC_WIDTHS[j_g] >= min_width[g],
    by dynamic programming over the exact cost spent; None if infeasible."""
    err = np.asarray(err, dtype=np.float64)
    G = err.shape[0]
    size = np.broadcast_to(np.asarray(size, dtype=np.int64), (G,))
    dp = np.full(budget + 1, np.inf)
    dp[0] = 0.0
    choice = np.full((G, budget + 1), -1, dtype=np.int8)
    for g in range(G):
        new = np.full(budget + 1, np.inf)
        for j, b in enumerate(ALLOC_WIDTHS):
            if min_width is not None and b < min_width[g]:
                continue
            c = int(b * size[g])
            if c > budget:
                continue
            cand = np.full(budget + 1, np.inf)
            cand[c:] = dp[: budget + 1 - c] + err[g, j]
            better = cand < new
            new[better] = cand[better]
            choice[g, better] = j
        dp = new
    c = int(np.argmin(dp))
    if not np.isfinite(dp[c]):
        return None
    total = float(dp[c])
    widths = [0] * G
    for g in range(G - 1, -1, -1):
        j = int(choice[g, c])
        widths[g] = ALLOC_WIDTHS[j]
        c -= ALLOC_WIDTHS[j] * int(size[g])
    return total, widths


def reference_layer(W: np.ndarray, widths):
    """Oracle's own quantize + pack of a layer: (codes, scales, qweight)."""
    codes, scales = quantize(W, widths)
    return codes, scales, pack(codes, widths)


def within_tolerance(y: np.ndarray, y_ref: np.ndarray, bound: np.ndarray, rel: float = 2e-3, abs_: float = 1e-5):
    """Per-output check |y - y_ref| <= rel * sum|x*w| + abs_ (the stated matmul tolerance).

    Returns (ok, worst ratio of error to allowance)."""
    err = np.abs(np.asarray(y, dtype=np.float64) - y_ref)
    allow = rel * bound + abs_
    ratio = err / allow
    bad = ~np.isfinite(np.asarray(y, dtype=np.float64))
    worst = float(np.max(ratio)) if ratio.size else 0.0
    return bool(np.all(err <= allow) and not bad.any()), worst
