"""Seeded input generators: determinism, shapes, value structure (no GPU)."""
import numpy as np

import synth


def test_deterministic_and_shaped():
    a = synth.prefill_smoke(0)
    b = synth.prefill_smoke(0)
    assert np.array_equal(a.q8, b.q8) and np.array_equal(a.k8, b.k8)
    assert np.array_equal(a.w, b.w) and np.array_equal(a.k_scale, b.k_scale)
    assert a.q8.shape == (64, 64, 128) and a.k8.shape == (8192, 128)
    assert a.row_start.tolist() == [0] * 64
    assert a.row_end.tolist() == list(range(8129, 8193))
    assert a.pairs == sum(range(8129, 8193))
    c = synth.prefill_smoke(1)
    assert not np.array_equal(a.k8, c.k8)


def test_no_nan_codes_and_scale_recipe():
    a = synth.random_case("g", 8, 3000, seed=3)
    for arr in (a.q8, a.k8):
        assert not np.any((arr & 0x7F) == 0x7F)
    # amax/448 recipe: every key row reaches |code| = 448 (0x7E / 0xFE) somewhere
    assert np.all(np.any((a.k8 & 0x7F) == 0x7E, axis=1))
    assert np.all(a.k_scale > 0) and np.all(a.q_scale > 0)
    assert abs(float(a.w.std()) - 0.125) < 0.02


def test_adversarial_structure():
    ties = synth.causal_case("t", 4, 20000, seed=1, key_mode="ties16")
    assert np.unique(ties.k8, axis=0).shape[0] == 16
    dec = synth.causal_case("d", 2, 20000, seed=1, key_mode="decoy")
    lattice = np.arange(synth.SAMPLE_OFFSET, 20000, synth.SAMPLE_STRIDE)
    # decoys (x8) sit on every other lattice point: their scale is ~8x typical
    assert np.median(dec.k_scale[lattice[::2]]) > 5 * np.median(dec.k_scale)
    out = synth.causal_case("o", 2, 20000, seed=1, key_mode="outlier")
    heavy = np.nonzero(out.k_scale > 5 * np.median(out.k_scale))[0]
    assert synth.OUTLIER_KEYS - 100 <= heavy.size <= synth.OUTLIER_KEYS
    assert not np.any((heavy - synth.SAMPLE_OFFSET) % synth.SAMPLE_STRIDE == 0)
    # one block ending at the first row's last position, inside every row
    assert heavy.max() <= out.row_end.min() - 1
    assert heavy.max() - heavy.min() < synth.OUTLIER_KEYS * 1.01 + 10


def test_paged_decode_layout():
    lens = synth.paged_decode_lens(0)
    assert lens.shape == (16,) and lens.min() >= 1 and lens.max() <= 65536
    assert np.sum(lens <= 2048) >= 4
    c = synth.decode_case("p", [100, 1, 64, 129], seed=2, max_pages=8)
    used = c.page_table[c.page_table >= 0]
    assert sorted(used.tolist()) == list(range(c.k_cache.shape[0]))
    assert c.page_table[0].tolist()[:2] != [-1, -1] and c.page_table[0, 2] == -1


def test_adversarial_rows_split_as_configured():
    """2048 rows at the last positions of 163840 keys: half ties, a quarter
    split between the off-lattice outlier block and the on-lattice decoys
    (the underflow/repair quarter), the rest plain; every row appears once."""
    import inspect
    src = inspect.getsource(synth.adversarial)
    assert "1024" in src and "256" in src and "512" in src
    # row counts and disjoint positions without generating the keys
    N = 163840
    pos = np.arange(N - 2048, N)
    parts = [pos[:1024], pos[1024:1280], pos[1280:1536], pos[1536:]]
    assert sum(p.size for p in parts) == 2048
    assert np.array_equal(np.concatenate(parts), pos)


def test_random_codes_case_has_no_nan_codes():
    c = synth.random_codes_case("rc", 5000, [0, 10], [100, 5000], seed=3)
    assert not np.any((c.k8 & 0x7F) == 0x7F)
    assert c.k8.shape == (5000, 128) and c.q8.shape == (2, 64, 128)
    assert np.all(c.k_scale > 0)
