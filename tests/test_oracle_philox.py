"""Pins of the oracle's Philox4x32-10 against published known-answer vectors."""
import os

import numpy as np

from oracle import philox4x32_10, uniforms24, accept_uniforms
from conftest import GOLDEN


def _kat():
    rows = []
    with open(os.path.join(GOLDEN, "philox_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(t, 16) for t in line.split()])
    return np.array(rows, dtype=np.uint64)


def test_known_answer_vectors():
    kat = _kat()
    out = philox4x32_10(kat[:, 0:4], kat[:, 4:6])
    assert np.array_equal(out.astype(np.uint64), kat[:, 6:10])


def test_uniform_map_endpoints():
    u = uniforms24(np.array([0, 0xFF, 0x100, 0xFFFFFFFF], dtype=np.uint32))
    assert u[0] == 0.0 and u[1] == 0.0
    assert u[2] == 2.0 ** -24
    assert u[3] == 1.0 - 2.0 ** -24           # strictly below one
    assert np.all(u == u.astype(np.float32))   # exact in binary32


def test_accept_uniform_counter_layout():
    # position i, trial b, offset, tag 0; word 0 -> u, word 1 -> u'
    seed, b, k, off = 0x1234_5678_9ABC, 7, 5, 3
    u, u2 = accept_uniforms(seed, b, k, offset=off)
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], dtype=np.uint64)
    for i in range(k + 1):
        w = philox4x32_10(np.array([i, b, off, 0], dtype=np.uint64), key)
        assert u[i] == (int(w[0]) >> 8) * 2.0 ** -24
        assert u2[i] == (int(w[1]) >> 8) * 2.0 ** -24


def test_uniforms_look_uniform():
    u, u2 = accept_uniforms(42, 0, 4095)
    allu = np.concatenate([u, u2])
    assert abs(allu.mean() - 0.5) < 0.02
    hist = np.histogram(allu, bins=16, range=(0, 1))[0]
    expected = allu.size / 16
    chi2 = ((hist - expected) ** 2 / expected).sum()
    assert chi2 < 45.0      # dof 15, p ~ 1e-4
