"""Pins of the top-p selection oracle (oracle/select.py): brute force over all
subsets on tiny inputs, closed forms, invariants, and the mass against a library
softmax."""
import itertools

import numpy as np
import pytest
import torch

from oracle import select as OS
from oracle.attention import bf16_bits_to_f64


def _brute(mass, p):
    """Shortest set with mass >= p*total; among the shortest, the one that takes
    larger masses first and, for equal masses, lower positions (compare the sets'
    mass-ordered sequences lexicographically)."""
    n = len(mass)
    tot = sum(mass)
    for k in range(1, n + 1):
        best = None
        for c in itertools.combinations(range(n), k):
            if sum(mass[i] for i in c) >= p * tot - 1e-15:
                key = sorted(((-mass[i], i) for i in c))
                if best is None or key < best[0]:
                    best = (key, c)
        if best:
            return sorted(best[1])
    return list(range(n))


@pytest.mark.parametrize("seed", range(40))
def test_top_p_equals_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 9))
    mass = list(rng.choice([0.05, 0.1, 0.2, 0.3, 0.5, 1.0], size=n))  # many ties
    for p in (0.1, 0.5, 0.77, 0.9, 1.0):
        assert list(OS.top_p(mass, p)) == _brute(mass, p), (mass, p)


def test_top_p_closed_forms():
    n = 100
    uniform = np.full(n, 1.0 / n)
    for p in (0.01, 0.25, 0.5, 0.999, 1.0):
        k = int(np.ceil(p * n - 1e-9))
        assert list(OS.top_p(uniform, p)) == list(range(max(k, 1)))  # ties: lowest positions
    peaked = np.full(n, 0.2 / (n - 1))
    peaked[37] = 0.8
    assert list(OS.top_p(peaked, 0.8)) == [37]
    assert list(OS.top_p(peaked, 0.5)) == [37]
    assert list(OS.top_p(peaked, 0.81)) == [0, 1, 2, 3, 4, 37]  # 0.8 + 5 x 0.2/99
    assert list(OS.top_p(peaked, 1.0)) == list(range(n))


def test_top_p_permutation_invariance():
    rng = np.random.default_rng(5)
    mass = rng.random(300) ** 4
    perm = rng.permutation(300)
    a = OS.top_p(mass, 0.9)
    b = OS.top_p(mass[perm], 0.9)
    assert sorted(perm[b]) == list(a)


def test_key_mass_matches_library_softmax():
    rng = np.random.default_rng(1)
    G, N, D = 4, 57, 64
    qb = (rng.standard_normal((G, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    kb = (rng.standard_normal((N, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    m = OS.key_mass(qb, kb, 0.125)
    q = torch.from_numpy(bf16_bits_to_f64(qb))
    k = torch.from_numpy(bf16_bits_to_f64(kb))
    ref = torch.softmax(0.125 * q @ k.T, dim=1).mean(dim=0).numpy()
    assert np.max(np.abs(m - ref)) < 1e-15
    assert abs(m.sum() - 1.0) < 1e-12
