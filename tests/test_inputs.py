"""The seeded synthetic workloads: shapes, dtypes, reproducibility and the
structure each one is meant to carry (gate outliers, f16 rounding)."""
import numpy as np

from tiled_dense_gemm_matmul_amd import inputs


def test_shapes_and_dtypes():
    c1, c2, c3, c4 = inputs.cfg1(), inputs.cfg2(), inputs.cfg3(), inputs.cfg4()
    assert c1["X"].shape == (128, 768) and c1["W"].shape == (768, 768)
    assert c2["X"].shape == (512, 768) and c2["R"].shape == (512, 768)
    assert c3["G"].shape == (512, 3072) and c3["W"].shape == (3072, 768) and c3["R"].shape == (512, 768)
    assert c4["W_lm"].shape == (768, 16384) and c4["W_lm"].dtype == np.float16
    assert c4["W_gu"].shape == (768, 3072) and c4["W_gu"].dtype == np.float16
    for c in (c1, c2, c3, c4):
        for k, v in c.items():
            assert v.flags.c_contiguous
            assert v.dtype in (np.float32, np.float16), k


def test_reproducible():
    a, b = inputs.cfg3(), inputs.cfg3()
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert not np.array_equal(inputs.cfg1()["X"][:4], inputs.cfg2()["X"][:4])


def test_gate_outliers():
    G = inputs.cfg3()["G"]
    big = np.abs(G) == 80.0
    assert int(big.sum()) == 15728  # floor(0.01 * 512 * 3072)
    pos, neg = int((G == 80.0).sum()), int((G == -80.0).sum())
    assert pos + neg == 15728 and abs(pos - neg) < 500
    assert np.abs(G[~big]).max() < 8.0


def test_weight_statistics_and_f16_rounding():
    c4 = inputs.cfg4()
    rng = np.random.default_rng(3)
    rng.standard_normal((512, 768), dtype=np.float32)
    w32 = rng.standard_normal((768, 16384), dtype=np.float32) * np.float32(0.02)
    assert np.array_equal(w32.astype(np.float16).view(np.uint16), c4["W_lm"].view(np.uint16))
    assert abs(float(w32.std()) - 0.02) < 1e-4
    # round-to-nearest-even: every f16 is the closest binary16 to its draw
    sample = w32.reshape(-1)[:20000].astype(np.float64)
    h = c4["W_lm"].reshape(-1)[:20000]
    up = np.nextafter(h, np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(h, np.float16(-np.inf)).astype(np.float64)
    err = np.abs(h.astype(np.float64) - sample)
    assert np.all(err <= np.abs(up - sample)) and np.all(err <= np.abs(dn - sample))
    # a fraction of the weights land on binary16 subnormals (|w| < 2^-14)
    sub = np.abs(c4["W_lm"].astype(np.float32)) < 2.0 ** -14
    assert 0.001 < sub.mean() < 0.005


def test_random_case_integer_exactness():
    c = inputs.random_case(5, 33, 3072, 20, integer=True, residual=True)
    assert np.abs(c["X"]).max() <= 8 and np.abs(c["W"]).max() <= 8
    # every partial sum stays below 2^24, so fp32 accumulation is exact
    assert 3072 * 64 + 8 < 2 ** 24
