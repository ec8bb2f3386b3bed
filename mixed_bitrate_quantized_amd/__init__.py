"""Python binding of libexq: mixed-bitrate (EXL2-style) quantized linears on MI355X.

Argument marshalling only.  Every step of the path -- packing, dequantization
and the matmul -- runs in libexq (host C++ and gfx950 HIP kernels); PyTorch
is used for device memory and streams.  The library is loaded from this
directory; importing the package fails loudly when it is missing and cannot
be built, and there is no fallback path.

The C entry points keep their names (``exq_pack``, ``exq_layer_create``,
``exq_gemm``, ...); see ``include/exq.h`` for argument meaning, layout,
ownership and errors.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libexq.so")
GROUP = 128
MAX_DECODE_M = 16

EXQ_OK, EXQ_ERR_INVALID_ARG, EXQ_ERR_UNSUPPORTED, EXQ_ERR_HIP, EXQ_ERR_OOM = range(5)


class ExqError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str):
        super().__init__("%s failed: %s (%s)" % (what, _status_name(status), detail))
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        from . import build as _b
        _b.build()
    # PyTorch ships its own HIP runtime.  Importing it first makes libexq bind
    # to that already-loaded runtime instead of loading a second copy from
    # the ROCm install, so device pointers and streams from torch and from
    # libexq belong to one runtime.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.exq_status_string.argtypes = [i32]
    lib.exq_status_string.restype = ctypes.c_char_p
    lib.exq_last_error.argtypes = []
    lib.exq_last_error.restype = ctypes.c_char_p
    lib.exq_packed_bytes.argtypes = [i32, i32, i32, vp]
    lib.exq_packed_bytes.restype = u64
    lib.exq_pack.argtypes = [vp, i32, i32, i32, vp, vp, vp]
    lib.exq_layer_create.argtypes = [i32, i32, i32, vp, vp, vp, ctypes.POINTER(vp)]
    lib.exq_layer_destroy.argtypes = [vp]
    lib.exq_layer_destroy.restype = None
    lib.exq_gemm.argtypes = [vp, i32, vp, vp, vp]
    lib.exq_gemm_noalloc.argtypes = [vp, i32, vp, vp, vp]
    lib.exq_dequant.argtypes = [vp, vp, vp]
    lib.exq_plan_create.argtypes = [i32, vp, vp, vp, i32, ctypes.POINTER(vp)]
    lib.exq_plan_run.argtypes = [vp, vp]
    lib.exq_plan_destroy.argtypes = [vp]
    lib.exq_plan_destroy.restype = None
    lib.exq_stream_read.argtypes = [vp, u64, vp, i32, vp]
    lib.exq_gemm_gated.argtypes = [vp, i32, vp, vp, vp, vp]
    lib.exq_group_errors.argtypes = [vp, i32, i32, i32, vp]
    lib.exq_pack_qs.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
    lib.exq_layer_create_qs.argtypes = [i32, i32, i32, vp, vp, vp, vp, ctypes.POINTER(vp)]
    lib.exq_trimmed_mean.argtypes = [vp, i32]
    lib.exq_trimmed_mean.restype = ctypes.c_double
    lib.exq_autotune.argtypes = [vp, i32, vp, vp, vp, i32, i32, vp, vp]
    lib.exq_set_variant.argtypes = [vp, i32, i32]
    lib.exq_allocate_widths.argtypes = [vp, vp, i32, ctypes.c_int64, vp, ctypes.c_uint64, ctypes.c_int64, vp, vp]
    for f in (lib.exq_pack, lib.exq_layer_create, lib.exq_gemm, lib.exq_gemm_noalloc, lib.exq_dequant, lib.exq_plan_create,
              lib.exq_plan_run, lib.exq_stream_read, lib.exq_gemm_gated, lib.exq_group_errors,
              lib.exq_allocate_widths, lib.exq_autotune, lib.exq_set_variant, lib.exq_pack_qs,
              lib.exq_layer_create_qs):
        f.restype = i32
    return lib


lib = _load()

# Symbols include/exq.h declares (checked by the tests).
EXPORTED = (
    "exq_status_string", "exq_last_error", "exq_packed_bytes", "exq_pack", "exq_layer_create",
    "exq_layer_destroy", "exq_gemm", "exq_dequant", "exq_plan_create", "exq_plan_run", "exq_plan_destroy",
    "exq_stream_read", "exq_gemm_gated", "exq_group_errors", "exq_allocate_widths", "exq_trimmed_mean",
    "exq_autotune", "exq_set_variant", "exq_pack_qs", "exq_layer_create_qs", "exq_gemm_noalloc",
)

VARIANT_DEFAULT, VARIANT_DECODE16, VARIANT_DECODE64, VARIANT_PREFILL = 0, 1, 2, 3


def _status_name(s: int) -> str:
    return lib.exq_status_string(s).decode()


def _check(status: int, what: str):
    if status != EXQ_OK:
        raise ExqError(status, what, lib.exq_last_error().decode())


def _np_ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _stream_ptr(stream) -> int | None:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return int(stream)


# ------------------------------------------------------------- entry points

def exq_status_string(status: int) -> str:
    return _status_name(status)


def exq_packed_bytes(K: int, N: int, widths, group_size: int = GROUP) -> int:
    w = np.ascontiguousarray(widths, dtype=np.uint8)
    return int(lib.exq_packed_bytes(K, N, group_size, _np_ptr(w)))


def exq_pack(W: np.ndarray, widths, group_size: int = GROUP):
    """Host quantize + pack.  W fp32 [N][K] -> (qweight uint8 bytes, scales fp16 bits uint16 [G][N])."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    w = np.ascontiguousarray(widths, dtype=np.uint8)
    nbytes = exq_packed_bytes(K, N, w, group_size)
    if nbytes == 0:
        _check(lib.exq_pack(_np_ptr(W), K, N, group_size, _np_ptr(w), None, None), "exq_pack")
    q = np.empty(nbytes, dtype=np.uint8)
    s = np.empty((K // group_size, N), dtype=np.uint16)
    _check(lib.exq_pack(_np_ptr(W), K, N, group_size, _np_ptr(w), _np_ptr(q), _np_ptr(s)), "exq_pack")
    return q, s


def exq_pack_qs(W: np.ndarray, widths, group_size: int = GROUP):
    """Host quantize + pack with quantized group scales.  W fp32 [N][K] ->
    (qweight uint8 bytes, 4-bit scale codes uint8 [G][N/2], column references fp16 bits uint16 [N])."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    w = np.ascontiguousarray(widths, dtype=np.uint8)
    nbytes = exq_packed_bytes(K, N, w, group_size)
    if nbytes == 0:
        _check(lib.exq_pack_qs(_np_ptr(W), K, N, group_size, _np_ptr(w), None, None, None), "exq_pack_qs")
    q = np.empty(nbytes, dtype=np.uint8)
    qs = np.empty((K // group_size, N // 2), dtype=np.uint8)
    ref = np.empty(N, dtype=np.uint16)
    _check(lib.exq_pack_qs(_np_ptr(W), K, N, group_size, _np_ptr(w), _np_ptr(q), _np_ptr(qs), _np_ptr(ref)),
           "exq_pack_qs")
    return q, qs, ref


def exq_layer_create_qs(K: int, N: int, widths, d_qweight: int, d_qscale: int, d_ref: int,
                        group_size: int = GROUP) -> int:
    w = np.ascontiguousarray(widths, dtype=np.uint8)
    h = ctypes.c_void_p()
    _check(lib.exq_layer_create_qs(K, N, group_size, _np_ptr(w), d_qweight, d_qscale, d_ref, ctypes.byref(h)),
           "exq_layer_create_qs")
    return h.value


def exq_layer_create(K: int, N: int, widths, d_qweight: int, d_scales: int, group_size: int = GROUP) -> int:
    w = np.ascontiguousarray(widths, dtype=np.uint8)
    h = ctypes.c_void_p()
    _check(lib.exq_layer_create(K, N, group_size, _np_ptr(w), d_qweight, d_scales, ctypes.byref(h)),
           "exq_layer_create")
    return h.value


def exq_layer_destroy(handle: int) -> None:
    lib.exq_layer_destroy(handle)


def exq_gemm(x_ptr: int, M: int, handle: int, y_ptr: int, stream=None) -> None:
    _check(lib.exq_gemm(x_ptr, M, handle, y_ptr, _stream_ptr(stream)), "exq_gemm")


def exq_gemm_noalloc(x_ptr: int, M: int, handle: int, y_ptr: int, stream=None) -> None:
    _check(lib.exq_gemm_noalloc(x_ptr, M, handle, y_ptr, _stream_ptr(stream)), "exq_gemm_noalloc")


def exq_gemm_gated(x_ptr: int, M: int, gate: int, up: int, h_ptr: int, stream=None) -> None:
    _check(lib.exq_gemm_gated(x_ptr, M, gate, up, h_ptr, _stream_ptr(stream)), "exq_gemm_gated")


def exq_group_errors(W: np.ndarray) -> np.ndarray:
    """Squared weight error of every group at every width: float64 [K/128][6] from W fp32 [N][K]."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    err = np.empty((K // 128, 6), dtype=np.float64)
    _check(lib.exq_group_errors(_np_ptr(W), K, N, 128, _np_ptr(err)), "exq_group_errors")
    return err


def exq_allocate_widths(err: np.ndarray, size, budget: int, min_width=None, seed: int = 0, iterations: int = 0):
    """(widths uint8 [G], total error) minimizing sum err[g][b_g] with sum b_g * size[g] <= budget."""
    err = np.ascontiguousarray(err, dtype=np.float64)
    G = err.shape[0]
    size = np.ascontiguousarray(np.broadcast_to(np.asarray(size, dtype=np.int32), (G,)))
    mw = None if min_width is None else np.ascontiguousarray(min_width, dtype=np.uint8)
    out = np.empty(G, dtype=np.uint8)
    total = ctypes.c_double()
    _check(lib.exq_allocate_widths(_np_ptr(err), _np_ptr(size), G, int(budget), None if mw is None else _np_ptr(mw),
                                   int(seed) & ((1 << 64) - 1), int(iterations), _np_ptr(out), ctypes.byref(total)),
           "exq_allocate_widths")
    return out, total.value


def exq_trimmed_mean(samples) -> float:
    s = np.ascontiguousarray(samples, dtype=np.float32)
    return lib.exq_trimmed_mean(_np_ptr(s), s.size)


def exq_autotune(x_ptr: int, M: int, handle: int, y_ptr: int, stream=None, warmup: int = 20, reps: int = 200):
    """(chosen variant, trimmed-mean microseconds per candidate from DECODE16 on)."""
    choice = ctypes.c_int()
    times = np.zeros(3, dtype=np.float32)
    _check(lib.exq_autotune(x_ptr, M, handle, y_ptr, _stream_ptr(stream), warmup, reps, ctypes.byref(choice),
                            _np_ptr(times)), "exq_autotune")
    return choice.value, times[: 3 if M > 16 else 2].tolist()


def exq_set_variant(handle: int, M: int, variant: int) -> None:
    _check(lib.exq_set_variant(handle, M, variant), "exq_set_variant")


def exq_dequant(handle: int, w_ptr: int, stream=None) -> None:
    _check(lib.exq_dequant(handle, w_ptr, _stream_ptr(stream)), "exq_dequant")


def exq_plan_create(handles, x_ptrs, y_ptrs, M: int) -> int:
    n = len(handles)
    H = (ctypes.c_void_p * n)(*handles)
    X = (ctypes.c_void_p * n)(*x_ptrs)
    Y = (ctypes.c_void_p * n)(*y_ptrs)
    p = ctypes.c_void_p()
    _check(lib.exq_plan_create(n, H, X, Y, M, ctypes.byref(p)), "exq_plan_create")
    return p.value


def exq_plan_run(plan: int, stream=None) -> None:
    _check(lib.exq_plan_run(plan, _stream_ptr(stream)), "exq_plan_run")


def exq_stream_read(buf_ptr: int, nbytes: int, sink_ptr: int, sink_words: int, stream=None) -> None:
    _check(lib.exq_stream_read(buf_ptr, nbytes, sink_ptr, sink_words, _stream_ptr(stream)), "exq_stream_read")


def exq_plan_destroy(plan: int) -> None:
    lib.exq_plan_destroy(plan)


# ------------------------------------------------------------ conveniences

class Layer:
    """A packed layer resident on the GPU: owns its torch buffers and the handle."""

    def __init__(self, K: int, N: int, widths, qweight: np.ndarray, scales: np.ndarray, device="cuda", ref=None):
        """fp16 scales [G][N]; or, with `ref` (fp16 bits [N]), 4-bit scale codes [G][N/2] in `scales`."""
        import torch
        self.K, self.N = K, N
        self.widths = np.ascontiguousarray(widths, dtype=np.uint8)
        self.qweight = torch.from_numpy(np.ascontiguousarray(qweight)).to(device)
        if ref is None:
            self.scales = torch.from_numpy(np.ascontiguousarray(scales).view(np.int16)).to(device)
            self.ref = None
            self.handle = exq_layer_create(K, N, self.widths, self.qweight.data_ptr(), self.scales.data_ptr())
        else:
            self.scales = torch.from_numpy(np.ascontiguousarray(scales, dtype=np.uint8)).to(device)
            self.ref = torch.from_numpy(np.ascontiguousarray(ref).view(np.int16)).to(device)
            self.handle = exq_layer_create_qs(K, N, self.widths, self.qweight.data_ptr(), self.scales.data_ptr(),
                                              self.ref.data_ptr())

    @classmethod
    def from_weight(cls, W: np.ndarray, widths, device="cuda", quantized_scales: bool = False):
        N, K = W.shape
        if quantized_scales:
            q, qs, ref = exq_pack_qs(W, widths)
            return cls(K, N, widths, q, qs, device, ref=ref)
        q, s = exq_pack(W, widths)
        return cls(K, N, widths, q, s, device)

    @property
    def packed_bytes(self) -> int:
        return int(self.qweight.numel())

    def gemm(self, x, out=None, stream=None):
        """x: torch fp16 [M][K] on the GPU -> y fp16 [M][N]."""
        import torch
        assert x.dtype == torch.float16 and x.is_contiguous() and x.shape[-1] == self.K
        M = x.shape[0]
        if out is None:
            out = torch.empty((M, self.N), dtype=torch.float16, device=x.device)
        exq_gemm(x.data_ptr(), M, self.handle, out.data_ptr(), stream)
        return out

    def dequant(self, stream=None):
        import torch
        w = torch.empty((self.K, self.N), dtype=torch.float16, device=self.qweight.device)
        exq_dequant(self.handle, w.data_ptr(), stream)
        return w

    def close(self):
        if self.handle:
            exq_layer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def gemm_gated(x, gate: "Layer", up: "Layer", out=None, stream=None):
    """x: torch fp16 [M][K] on the GPU -> h = SiLU(x gate^T) * (x up^T), fp16 [M][N]."""
    import torch
    assert x.dtype == torch.float16 and x.is_contiguous() and x.shape[-1] == gate.K
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, gate.N), dtype=torch.float16, device=x.device)
    exq_gemm_gated(x.data_ptr(), M, gate.handle, up.handle, out.data_ptr(), stream)
    return out


class Plan:
    """Independent linears bound to fixed x/y buffers, run as one launch."""

    def __init__(self, layers, xs, ys, M: int):
        self.layers, self.xs, self.ys = list(layers), list(xs), list(ys)  # keep buffers alive
        self.handle = exq_plan_create([l.handle for l in self.layers], [x.data_ptr() for x in self.xs],
                                      [y.data_ptr() for y in self.ys], M)

    def run(self, stream=None):
        exq_plan_run(self.handle, stream)

    def close(self):
        if self.handle:
            exq_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
