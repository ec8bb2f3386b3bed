"""Seeded synthetic inputs shared by the test oracle and the GPU path.

This module generates the inputs of a quantized linear layer -- fp32 weights,
fp16 activations and the per-group bit widths -- and nothing else.  It holds
none of the quantizer, packer, dequantizer or matmul arithmetic; both the
oracle and the library receive its outputs as plain arrays.

Workload shapes are Llama-3-70B's decoder-block linears (the pages name the
model, not its shapes): hidden 8192, 64 query heads and 8 key/value heads of
dimension 128, MLP width 28672.  The pages (promptquorum.com "ExLlamaV2
explained", EXL2 section) describe widths 2/3/4/5/6/8 mixed toward a target
average such as 2.55 bits per weight, with more important weight columns kept
at higher precision; the schedules below stand in for the calibration-driven
allocation, which needs trained weights.
"""
from __future__ import annotations

import ctypes
import hashlib
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_libsynth.so")
_lib = None

GROUP = 128
WIDTHS = (2, 3, 4, 5, 6, 8)

# Llama-3-70B decoder block linears as (name, K = in features, N = out features).
BLOCK_SHAPES = (
    ("q", 8192, 8192),
    ("k", 8192, 1024),
    ("v", 8192, 1024),
    ("o", 8192, 8192),
    ("gate", 8192, 28672),
    ("up", 8192, 28672),
    ("down", 28672, 8192),
)
N_BLOCKS_70B = 80


def build(force: bool = False) -> str:
    """Compile the generator's C source into synth/_libsynth.so."""
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", src, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    u64, i64, f32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_float
    vp = ctypes.c_void_p
    lib.synth_init.restype = None
    lib.synth_philox4x32_10.argtypes = [vp, vp, vp]
    lib.synth_fill_normal.argtypes = [u64, u64, u64, f32, vp]
    lib.synth_fill_u32.argtypes = [u64, u64, u64, vp]
    lib.synth_fill_rows.argtypes = [u64, i64, vp, i64, f32, vp]
    lib.synth_group_sq_norms.argtypes = [vp, i64, i64, i64, vp]
    lib.synth_quantile_table.restype = ctypes.POINTER(ctypes.c_float)
    lib.synth_init()
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def seed_for(*parts) -> int:
    """Stable 64-bit seed from a tuple of labels (config, linear index, tensor)."""
    h = hashlib.blake2b("/".join(str(p) for p in parts).encode(), digest_size=8)
    return int.from_bytes(h.digest(), "little")


def philox4x32_10(ctr, key) -> tuple:
    lib = _load()
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    lib.synth_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return tuple(int(v) for v in out)


def quantile_table() -> np.ndarray:
    lib = _load()
    return np.ctypeslib.as_array(lib.synth_quantile_table(), shape=(65537,)).copy()


def normal(seed: int, count: int, sigma: float = 1.0, first: int = 0, out: np.ndarray | None = None) -> np.ndarray:
    lib = _load()
    if out is None:
        out = np.empty(count, dtype=np.float32)
    assert out.dtype == np.float32 and out.size == count
    lib.synth_fill_normal(seed, first, count, sigma, _ptr(out))
    return out


def uniform_u32(seed: int, count: int, first: int = 0) -> np.ndarray:
    lib = _load()
    out = np.empty(count, dtype=np.uint32)
    lib.synth_fill_u32(seed, first, count, _ptr(out))
    return out


def weight(seed: int, N: int, K: int, sigma: float = 0.02, out: np.ndarray | None = None) -> np.ndarray:
    """W fp32 [N][K] row-major, iid N(0, sigma^2) (sigma is the standard deviation)."""
    if out is None:
        out = np.empty((N, K), dtype=np.float32)
    normal(seed, N * K, sigma, out=out.reshape(-1))
    return out


def weight_rows(seed: int, K: int, rows, sigma: float = 0.02) -> np.ndarray:
    """Rows `rows` of the matrix `weight(seed, N, K)` without generating the rest."""
    lib = _load()
    r = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((r.size, K), dtype=np.float32)
    lib.synth_fill_rows(seed, K, _ptr(r), r.size, sigma, _ptr(out))
    return out


def activations(seed: int, M: int, K: int) -> np.ndarray:
    """x fp16 [M][K]: N(0, 1) drawn in fp32, then rounded to fp16 (ties to even)."""
    return normal(seed, M * K, 1.0).astype(np.float16).reshape(M, K)


def group_sq_norms(W: np.ndarray, group: int = GROUP) -> np.ndarray:
    lib = _load()
    N, K = W.shape
    out = np.empty(K // group, dtype=np.float64)
    lib.synth_group_sq_norms(_ptr(W), N, K, group, _ptr(out))
    return out


def _permutation(seed: int, n: int) -> np.ndarray:
    """Seeded Fisher-Yates permutation of range(n)."""
    words = uniform_u32(seed, max(n, 1))
    p = np.arange(n)
    for i in range(n - 1, 0, -1):
        j = int(words[i]) % (i + 1)
        p[i], p[j] = p[j], p[i]
    return p


def widths_uniform(G: int, b: int) -> np.ndarray:
    return np.full(G, b, dtype=np.uint8)


def widths_mixed(G: int, sq_norms: np.ndarray, seed: int, bpw: float = 2.55, forced_frac: float = 0.05) -> np.ndarray:
    """Mixed widths averaging `bpw` code bits per weight, important groups kept high.

    The ceil(forced_frac * G) groups with the largest norm (ties: lower index)
    are forced to >= 6 bits: the largest gets 8, the rest 6.  Among the others
    a seeded permutation gives one group each 3, 4 and 5 bits; the remainder
    start at 2 bits and seeded 2->3 upgrades are applied until the width sum
    equals round(bpw * G).
    """
    target = int(round(bpw * G))
    w = np.full(G, 2, dtype=np.int64)
    order = sorted(range(G), key=lambda g: (-float(sq_norms[g]), g))
    F = int(math.ceil(forced_frac * G))
    forced = order[:F]
    for r, g in enumerate(forced):
        w[g] = 8 if r == 0 else 6
    rest = [g for g in range(G) if g not in set(forced)]
    perm = [rest[i] for i in _permutation(seed, len(rest))]
    for b, g in zip((3, 4, 5), perm[:3]):
        w[g] = b
    pool = perm[3:]
    need = target - int(w.sum())
    if need < 0 or need > len(pool):
        raise ValueError("cannot reach %.3f bpw with G=%d" % (bpw, G))
    for g in pool[:need]:
        w[g] = 3
    assert int(w.sum()) == target
    return w.astype(np.uint8)


def widths_mixed_4p0(G: int, seed: int) -> np.ndarray:
    """Widths from {3,4,5,6} summing to exactly 4*G with every width present.

    Counts: n6 = round(G/8), n5 = round(G/4), n3 = n5 + 2*n6 (so the sum is 4G),
    n4 = the rest; placed by a seeded permutation.
    """
    n6 = int(round(G / 8))
    n5 = int(round(G / 4))
    n3 = n5 + 2 * n6
    n4 = G - n3 - n5 - n6
    if min(n3, n4, n5, n6) < 1:
        raise ValueError("G=%d too small for the 4.0 bpw schedule" % G)
    flat = np.array([3] * n3 + [4] * n4 + [5] * n5 + [6] * n6, dtype=np.uint8)
    w = flat[_permutation(seed, G)]
    assert int(w.astype(np.int64).sum()) == 4 * G
    return w


def layer_widths(kind: str, G: int, seed: int, W: np.ndarray | None = None) -> np.ndarray:
    if kind == "u4":
        return widths_uniform(G, 4)
    if kind == "mixed2.55":
        assert W is not None
        return widths_mixed(G, group_sq_norms(W), seed)
    if kind == "mixed4.0":
        return widths_mixed_4p0(G, seed)
    if kind.startswith("u"):
        return widths_uniform(G, int(kind[1:]))
    raise ValueError(kind)
