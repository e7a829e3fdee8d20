"""The seeded generators: same seed, same bytes; the recipe's shapes and
value ranges; every quantisation group reaches the E4M3 maximum."""
import numpy as np

import workloads as W


def test_deterministic_and_shaped():
    w = W.WORKLOADS["decode_64x512x4096"]
    a, b = W.make_workload(w), W.make_workload(w)
    for k in ("A", "a_s", "B", "b_s"):
        assert np.array_equal(a[k], b[k])
    assert a["A"].shape == (64, 4096) and a["a_s"].shape == (64, 32)
    assert a["B"].shape == (512, 4096) and a["b_s"].shape == (4, 32)
    assert a["A"].dtype == np.uint8 and a["a_s"].dtype == np.float32


def test_no_nan_codes_and_groups_hit_max():
    d = W.make_inputs(24, 300, 512, seed=9)
    for codes in (d["A"], d["B"]):
        assert not np.isin(codes, [0x7F, 0xFF]).any()
    # each 1x128 activation group and each 128x128 weight block holds a +-448 code
    ga = (d["A"] & 0x7F).reshape(24, 4, 128).max(axis=2)
    assert np.all(ga == 0x7E)
    B = np.zeros((384, 512), np.uint8)
    B[:300] = d["B"] & 0x7F
    gb = B.reshape(3, 128, 4, 128).max(axis=(1, 3))
    assert np.all(gb == 0x7E)
    assert np.all(d["a_s"] > 0) and np.all(d["b_s"] > 0)


def test_outlier_rows():
    w = W.WORKLOADS["prefill_16384x4096x4096"]
    d = W.make_inputs(2000, 256, 256, seed=w.seed, outlier_frac=w.outlier_frac)
    n = len(d["outliers"])
    assert 5 <= n <= 40
    med = np.median(d["a_s"])
    assert np.all(d["a_s"][d["outliers"]].mean(axis=1) > 4 * med)


def test_exact_inputs_are_integers_and_powers_of_two():
    d = W.make_exact_inputs(8, 130, 256, seed=1)
    from tests._cases import torch_decode
    assert np.array_equal(torch_decode(d["A"]), d["Ai"].astype(np.float64))
    assert np.array_equal(torch_decode(d["B"]), d["Bi"].astype(np.float64))
    assert np.array_equal(d["a_s"], np.exp2(d["u"]).astype(np.float32))
    assert d["b_s"].shape == (2, 2)


def test_reshaped_workload_draws_from_its_base_seeds():
    # bench.py --N/--K renames a workload "<name>:N<n>:K<k>"; its sweep points
    # must still find a seed (that of the base workload's sweep point)
    import dataclasses
    w = W.WORKLOADS["small_16x512x256"]
    w2 = dataclasses.replace(w, name=w.name + ":N1536:K256", N=1536)
    assert W.sweep_seed(w2, 32) == W.sweep_seed(w, 32)
    d = W.make_workload(w2, 32)
    assert d["A"].shape == (32, 256) and d["B"].shape == (1536, 256)
