"""The seeded input generators: known answers, determinism, slicing, moments."""
import math

import numpy as np
import torch

import synthetic
from conftest import GOLDEN


def test_philox_known_answers():
    with open(GOLDEN + "/philox_kat.txt") as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        v = [int(h, 16) for h in r]
        np.testing.assert_array_equal(synthetic.philox(v[0:4], v[4:6]), np.array(v[6:10], np.uint32))


def test_slices_agree_and_keys_differ():
    a = synthetic.normal_f32(5, "w", 1001)
    b = synthetic.normal_f32(5, "w", 500, start=501)
    np.testing.assert_array_equal(a[501:], b)
    assert not np.array_equal(a, synthetic.normal_f32(6, "w", 1001))
    assert not np.array_equal(a, synthetic.normal_f32(5, "v", 1001))
    rb, rm = synthetic.normal_rows(5, "w", 4, 64, 0.5, bf16=True, mxfp4=True)
    np.testing.assert_array_equal(rb.reshape(-1), synthetic.normal_bf16(5, "w", 256, 0.5))
    np.testing.assert_array_equal(rm, synthetic.mxfp4_quantize(synthetic.normal_f32(5, "w", 256, 0.5).reshape(4, 64)))


def test_moments():
    z = synthetic.normal_f32(1, "m", 1 << 20).astype(np.float64)
    assert abs(z.mean()) < 5 / math.sqrt(1 << 20)
    assert abs(z.var() - 1) < 0.01
    assert abs(np.mean(z ** 4) - 3) < 0.05
    u = synthetic.uniform_f32(1, "u", 1 << 20, 0.0, 1.0).astype(np.float64)
    assert u.min() >= 0 and u.max() < 1 and abs(u.mean() - 0.5) < 0.002


def test_bf16_rne_matches_torch():
    v = synthetic.normal_f32(2, "r", 100000, 3.0)
    ours = synthetic.f32_to_bf16(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_zipf_bias():
    b = synthetic.zipf_bias(256).astype(np.float64)
    w = np.exp(b / 1.5)
    assert abs(w.sum() - 1) < 1e-5
    assert np.all(np.diff(b) < 0)
    np.testing.assert_allclose(w[0] / w[1], 2 ** 1.2, rtol=1e-5)


def test_presets_shapes():
    p = synthetic.PRESETS["c0"]
    prm = synthetic.layer_params(p)
    assert prm["router_w"].shape == (8, 64) and prm["w1"].shape == (8, 128, 64) and prm["w2"].shape == (8, 64, 128)
    assert abs(prm["w1"].std() - 1 / 8) < 0.01
    s = synthetic.small()
    prm = synthetic.layer_params(s, formats=("bf16", "mxfp4"))
    assert prm["w1"].shape == (s.n, 2 * s.F, s.L) and prm["w1"].dtype == np.uint16
    assert prm["w1@mxfp4"].size == s.n * 2 * s.F * s.L // 2 + s.n * 2 * s.F * s.L // 32
    x = synthetic.inputs(s)
    assert x.shape == (s.T, s.d)
    c = synthetic.Preset(**dict(s.cfg(), chunks=7, T=77))
    np.testing.assert_array_equal(synthetic.inputs(c, chunk=3), x[33:44])
