"""Host-side checks of the seeded input generators."""
import numpy as np
import torch

from dynamic_head_composition_amd import workloads as wl


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-6, 6, 100000),
                        np.array([0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8], np.float32)])
    ours = wl.bf16_bits(x.astype(np.float32))
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_seeded_and_deterministic():
    a = wl.make_workload(512, 2, 16, seed=5)
    b = wl.make_workload(512, 2, 16, seed=5)
    for f in ("q", "k", "v", "c", "g", "doc", "do"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = wl.make_workload(512, 2, 16, seed=6)
    assert not np.array_equal(a.q, c.q)


def test_values_representable_in_bf16():
    w = wl.make_workload(300, 3, 64, seed=1)
    for f in ("q", "k", "v", "do"):
        x = getattr(w, f)
        assert np.array_equal(wl.round_bf16(x), x)


def test_rms_rows():
    w = wl.make_workload(200, 2, 128, seed=2, dtype="f32")
    rms = np.sqrt(np.mean(w.q.astype(np.float64) ** 2, axis=-1))
    np.testing.assert_allclose(rms, 1.0, rtol=1e-5)


def test_document_streams():
    rng = np.random.default_rng(3)
    doc = wl.geometric_docs(rng, 200000, 1024)
    assert doc.shape == (200000,) and doc[0] == 0
    steps = np.diff(doc)
    assert set(np.unique(steps)) <= {0, 1}
    lengths = np.bincount(doc)
    assert 700 < lengths[:-1].mean() < 1400
    doc = wl.uniform_docs(np.random.default_rng(4), 100000, 8, 256)
    lengths = np.bincount(doc)
    assert lengths[:-1].min() >= 8 and lengths.max() <= 256


def test_config_recipes():
    w0 = wl.config_workload(0)
    assert (w0.T, w0.H, w0.d, w0.dtype, w0.window) == (256, 2, 16, "f32", 112)
    assert np.array_equal(w0.doc, np.array([0] * 100 + [1] * 156))
    assert np.all((w0.g >= 0.5) & (w0.g <= 1.5))
    w3 = wl.config_workload(3, T=4096)
    onehot = np.sum(w3.c == 1.0, axis=1) == 1
    assert 0.75 < onehot.mean() < 0.85
    assert np.all(w3.g == 1.0)
    w4 = wl.config_workload(4, T=4096)
    neg = w4.c <= -4.0
    assert 0.07 < neg.mean() < 0.13
    assert np.all((w4.g >= 0) & (w4.g <= 2))


def test_mudd_workload_seeded_shapes_and_dtypes():
    a = wl.make_mudd_workload(40, 96, 3, 5, seed=3)
    b = wl.make_mudd_workload(40, 96, 3, 5, seed=3)
    assert len(a.xs) == 5 and len(a.dys) == 3 and a.a.shape == (40, 3, 5)
    for u, v in zip(a.xs + a.dys + [a.a], b.xs + b.dys + [b.a]):
        assert u.dtype == np.float32 and np.array_equal(u, v)
    for x in a.xs + a.dys:
        assert x.shape == (40, 96) and np.array_equal(wl.round_bf16(x), x)
    assert (a.a < 0).any() and (a.a > 0).any()  # weights of both signs
    c = wl.make_mudd_workload(40, 96, 3, 5, seed=4)
    assert not np.array_equal(a.xs[0], c.xs[0])
    s = a.slice(10, 20)
    assert s.T == 10 and np.array_equal(s.xs[2], a.xs[2][10:20]) and np.array_equal(s.a, a.a[10:20])


def test_mudd_workload_f32_not_rounded():
    w = wl.make_mudd_workload(16, 8, 1, 2, dtype="f32", seed=1)
    assert not all(np.array_equal(wl.round_bf16(x), x) for x in w.xs)
