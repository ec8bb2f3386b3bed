"""C-ABI library on the CPU: symbols, status codes, argument validation and the host packer.

No test here launches a kernel; the packer is host code and is compared with
the oracle's own quantizer and packer bit for bit.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import mixed_bitrate_quantized_amd as exq
import oracle
import synth
from synth import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    text = open(os.path.join(ROOT, "include", "exq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(exq_[a-z_]+)\s*\(", text)))


def test_library_exports_every_header_symbol():
    syms = header_symbols()
    assert "exq_gemm" in syms and "exq_pack" in syms and len(syms) >= 10
    lib = ctypes.CDLL(exq.LIB_PATH)
    for s in syms:
        assert hasattr(lib, s), s
    assert sorted(exq.EXPORTED) == syms


def test_status_strings():
    assert exq.exq_status_string(0) == "EXQ_OK"
    assert exq.exq_status_string(1) == "EXQ_ERR_INVALID_ARG"
    assert exq.exq_status_string(2) == "EXQ_ERR_UNSUPPORTED"
    assert exq.exq_status_string(3) == "EXQ_ERR_HIP"
    assert exq.exq_status_string(4) == "EXQ_ERR_OOM"


def test_packed_bytes_invariant():
    w = np.array([2, 3, 4, 5, 6, 8, 2], dtype=np.uint8)
    assert exq.exq_packed_bytes(128 * 7, 192, w) == sum(int(b) * 128 * 192 // 8 for b in w)
    assert exq.exq_packed_bytes(100, 64, w) == 0          # K not a multiple of 128
    assert exq.exq_packed_bytes(128, 64, [7]) == 0          # unsupported width
    assert exq.exq_packed_bytes(128, 64, [4], group_size=64) == 0


def _expect(status, fn, *args):
    with pytest.raises(exq.ExqError) as ei:
        fn(*args)
    assert ei.value.status == status


def test_pack_rejects_bad_input():
    W = np.zeros((64, 256), dtype=np.float32)
    _expect(exq.EXQ_ERR_INVALID_ARG, exq.exq_pack, W, [2, 9])
    _expect(exq.EXQ_ERR_UNSUPPORTED, exq.exq_pack, W, [2, 2, 2, 2], 64)
    W2 = W.copy()
    W2[3, 7] = np.nan
    _expect(exq.EXQ_ERR_INVALID_ARG, exq.exq_pack, W2, [2, 2])
    W3 = W.copy()
    W3[0, 0] = 1e5          # 2-bit scale 1e5 overflows fp16
    _expect(exq.EXQ_ERR_INVALID_ARG, exq.exq_pack, W3, [2, 2])


def test_layer_and_gemm_validation_before_any_launch():
    w = np.array([4, 4], dtype=np.uint8)
    fake = 0x10000  # never dereferenced: every case fails validation first
    _expect(exq.EXQ_ERR_INVALID_ARG, exq.exq_layer_create, 256, 72, w, fake, fake)      # N % 16
    _expect(exq.EXQ_ERR_INVALID_ARG, exq.exq_layer_create, 200, 64, w, fake, fake)      # K % 128
    _expect(exq.EXQ_ERR_UNSUPPORTED, exq.exq_layer_create, 256, 64, [4, 4, 4, 4], fake, fake, 64)
    _expect(exq.EXQ_ERR_INVALID_ARG, exq.exq_layer_create, 256, 64, [4, 7], fake, fake)
    _expect(exq.EXQ_ERR_INVALID_ARG, exq.exq_layer_create, 256, 64, w, 0, fake)
    _expect(exq.EXQ_ERR_INVALID_ARG, exq.exq_layer_create, 256, 64, w, fake + 4, fake)  # misaligned
    _expect(exq.EXQ_ERR_INVALID_ARG, exq.exq_gemm, fake, 1, 0, fake + 4096, 0)          # NULL layer
    _expect(exq.EXQ_ERR_INVALID_ARG, exq.exq_dequant, 0, fake, 0)
    _expect(exq.EXQ_ERR_INVALID_ARG, exq.exq_plan_run, 0, 0)
    _expect(exq.EXQ_ERR_INVALID_ARG, exq.exq_plan_create, [], [], [], 1)


@pytest.mark.parametrize("widths", [
    [2, 3, 4, 5, 6, 8],
    [8, 8, 8],
    [3, 2, 2, 3, 5, 2, 6],
])
def test_host_packer_matches_oracle_bit_for_bit(widths):
    s = synth.seed_for("packer", *widths)
    K, N = 128 * len(widths), 192
    W = synth.weight(s, N, K)
    W[5, :] = 0.0                     # an all-zero row: scale 0 everywhere
    W[7, 3] = 0.5                     # one large value in a group
    q, sc = exq.exq_pack(W, widths)
    codes, sc_ref, q_ref = oracle.reference_layer(W, widths)
    np.testing.assert_array_equal(sc, sc_ref)
    np.testing.assert_array_equal(q, q_ref)


def test_host_packer_matches_oracle_on_a_workload_layer():
    spec = workloads.linears(2)[0]
    W = workloads.make_weight(spec)[:128]       # 128 rows of the 8192 x 8192 layer
    widths = workloads.make_widths(spec, workloads.make_weight(spec))
    q, sc = exq.exq_pack(W, widths)
    _, sc_ref, q_ref = oracle.reference_layer(W, widths)
    np.testing.assert_array_equal(sc, sc_ref)
    np.testing.assert_array_equal(q, q_ref)
    assert q.size == exq.exq_packed_bytes(spec.K, 128, widths)


def test_split_planner_balances_bytes():
    """The split plan is internal; check it indirectly through the byte model."""
    spec = workloads.linears(3)[6]          # down: K = 28672
    W = workloads.make_weight(spec)
    widths = workloads.make_widths(spec, W)
    assert int(widths.astype(int).sum()) == round(2.55 * spec.G)


def test_trimmed_mean_definition():
    """The autotune statistic: mean of the sorted samples between the 5/16 and
    11/16 quantiles (for 16k samples exactly sorted[5k:11k])."""
    import numpy as np
    import mixed_bitrate_quantized_amd as exq
    rng = np.random.default_rng(2)
    for k in (1, 3, 12):
        s = rng.normal(size=16 * k).astype(np.float32)
        expect = np.sort(s)[5 * k:11 * k].astype(np.float64).mean()
        assert abs(exq.exq_trimmed_mean(s) - expect) < 1e-6
        assert abs(exq.exq_trimmed_mean(rng.permutation(s)) - expect) < 1e-6
        # outliers in the top and bottom 5/16 do not move it
        t = s.copy()
        o = np.argsort(t)
        t[o[-1]] = 1e9
        t[o[0]] = -1e9
        assert abs(exq.exq_trimmed_mean(t) - expect) < 1e-6
    assert exq.exq_trimmed_mean([4.0]) == 4.0
    assert exq.exq_trimmed_mean([2.0, 6.0]) == 4.0
    assert exq.exq_trimmed_mean([]) == -1.0


def test_xcd_blocks_partition_every_tile_grid(tmp_path):
    """The prefill launches' XCD blocks (xcd_block in the internal header):
    for every grid up to 40 x 120 tiles the 8 blocks cover each tile once."""
    import shutil
    import subprocess
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    header = os.path.join(os.path.dirname(exq.__file__), "csrc", "exq_internal.h")
    src = tmp_path / "xcd_blocks.cpp"
    src.write_text('''#include "%s"
#include <cstdio>
#include <vector>
int main() {
    for (int R = 1; R <= 40; ++R)
        for (int C = 1; C <= 120; ++C) {
            std::vector<int> seen(R * C, 0);
            for (int b = 0; b < 8; ++b) {
                const exq::XcdBlock x = exq::xcd_block(R, C, b);
                if (x.nr < 0 || x.nc < 0) return 1;
                for (int r = x.r0; r < x.r0 + x.nr; ++r)
                    for (int c = x.c0; c < x.c0 + x.nc; ++c) {
                        if (r < 0 || r >= R || c < 0 || c >= C) return 2;
                        ++seen[r * C + c];
                    }
            }
            for (int v : seen)
                if (v != 1) return 3;
        }
    return 0;
}
''' % header)
    exe = tmp_path / "xcd_blocks"
    subprocess.run([cxx, "-std=c++17", "-O1", "-o", str(exe), str(src)], check=True)
    assert subprocess.run([str(exe)]).returncode == 0


def test_layer_create_accepts_n_multiple_of_16():
    """N = 80 and 96 pass validation (a multiple of 16 is served); without a GPU
    the metadata allocation is what fails, never argument validation."""
    w = np.array([4, 4], dtype=np.uint8)
    for N in (80, 96, 16):
        h = ctypes.c_void_p()
        st = exq.lib.exq_layer_create(256, N, 128, w.ctypes.data, 0x10000, 0x10000, ctypes.byref(h))
        assert st in (exq.EXQ_OK, exq.EXQ_ERR_OOM, exq.EXQ_ERR_HIP), (N, st)
        if st == exq.EXQ_OK:
            exq.exq_layer_destroy(h.value)


def test_layer_size_limits_are_unsupported():
    """Valid shapes beyond the layer limits fail with EXQ_ERR_UNSUPPORTED
    before anything is allocated: 65536 or more 16-byte words per column
    (16-bit word offsets), and 2 GiB or more of packed words (32-bit buffer
    offsets)."""
    fake = 0x10000  # never dereferenced
    _expect(exq.EXQ_ERR_UNSUPPORTED, exq.exq_layer_create, 128 * 8192, 16, np.full(8192, 8, np.uint8), fake, fake)
    _expect(exq.EXQ_ERR_UNSUPPORTED, exq.exq_layer_create, 128 * 2048, 32768, np.full(2048, 2, np.uint8), fake, fake)
