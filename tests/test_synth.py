"""Seeded input generators: published RNG vectors, normal sampler, width schedules."""
import collections
import math
import os
import statistics

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kat_rows():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            v = [int(t, 16) for t in line.split()]
            rows.append((v[0:4], v[4:6], tuple(v[6:10])))
    return rows


@pytest.mark.parametrize("ctr,key,expect", _kat_rows())
def test_philox_known_answers(ctr, key, expect):
    assert synth.philox4x32_10(ctr, key) == expect


def test_quantile_table_matches_python_inverse_cdf():
    t = synth.quantile_table()
    nd = statistics.NormalDist()
    for j in (1, 7, 100, 1000, 20000, 32767, 32769, 50000, 65535):
        assert abs(float(t[j]) - nd.inv_cdf(j / 65536)) < 1e-6
    assert t[32768] == 0.0
    assert np.all(np.diff(t) > 0)
    np.testing.assert_array_equal(t, -t[::-1])


def test_normal_moments_and_cdf():
    z = synth.normal(synth.seed_for("moments"), 1 << 22)
    assert abs(float(z.mean())) < 2e-3
    assert abs(float(z.std()) - 1.0) < 2e-3
    nd = statistics.NormalDist()
    for q in (-2.0, -1.0, 0.0, 0.5, 1.5, 3.0):
        emp = float(np.mean(z < q))
        assert abs(emp - nd.cdf(q)) < 1.5e-3


def test_counter_based_slices_agree():
    s = synth.seed_for("slices")
    full = synth.normal(s, 1000, 0.02)
    part = synth.normal(s, 37, 0.02, first=501)
    np.testing.assert_array_equal(full[501:538], part)
    W = synth.weight(s, 10, 100)
    rows = synth.weight_rows(s, 100, [3, 7])
    np.testing.assert_array_equal(W[[3, 7]], rows)


def test_activations_are_fp16_of_normal():
    s = synth.seed_for("x")
    x = synth.activations(s, 2, 4096)
    assert x.dtype == np.float16
    ref = synth.normal(s, 2 * 4096).reshape(2, 4096)
    np.testing.assert_array_equal(x, ref.astype(np.float16))


@pytest.mark.parametrize("G,expect", [
    (64, {8: 1, 6: 3, 5: 1, 4: 1, 3: 12, 2: 46}),
    (224, {8: 1, 6: 11, 5: 1, 4: 1, 3: 68, 2: 142}),
])
def test_mixed_255_schedule(G, expect):
    rng = np.random.default_rng(G)
    norms = rng.random(G)
    w = synth.widths_mixed(G, norms, synth.seed_for("sched", G))
    assert dict(collections.Counter(w.tolist())) == expect
    assert int(w.astype(int).sum()) == round(2.55 * G)
    F = math.ceil(0.05 * G)
    top = np.argsort(-norms, kind="stable")[:F]
    assert w[top[0]] == 8
    assert all(w[g] >= 6 for g in top)
    assert sum(1 for g in range(G) if w[g] >= 6) == F


def test_mixed_255_schedule_from_weights():
    s = synth.seed_for("sched-w")
    W = synth.weight(s, 256, 8192)
    norms = synth.group_sq_norms(W)
    ref = np.array([float(np.sum(W[:, 128 * g:128 * (g + 1)].astype(np.float64) ** 2)) for g in range(64)])
    np.testing.assert_allclose(norms, ref, rtol=1e-12)
    w = synth.layer_widths("mixed2.55", 64, s, W)
    assert int(w.astype(int).sum()) == 163


@pytest.mark.parametrize("G", [64, 224])
def test_mixed_4p0_schedule(G):
    w = synth.widths_mixed_4p0(G, synth.seed_for("4p0", G))
    assert set(w.tolist()) == {3, 4, 5, 6}
    assert int(w.astype(int).sum()) == 4 * G


def test_seeds_are_stable():
    assert synth.seed_for("cfg", 3, "W") == synth.seed_for("cfg", 3, "W")
    assert synth.seed_for("cfg", 3, "W") != synth.seed_for("cfg", 4, "W")
