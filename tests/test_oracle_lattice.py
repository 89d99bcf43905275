"""Pins of the oracle's lattice quantisers.

The HyperQuant explainer (technical summary, Methodology 2) names the lattices
E8, D4, A2 and Z, their integer embedding (E8_int inside Z^8) and their lower
normalised second moment G than scalar quantisation.  The oracle is pinned by
brute-force enumeration of lattice points near each input, by membership and
translation invariants, and by the empirical G against the closed forms of
Conway & Sloane (SPLAG ch. 2, 20).
"""
import itertools

import numpy as np
import pytest

SQ3 = np.sqrt(3.0)


def members(lat, x):
    x = np.asarray(x, np.int64)
    if lat == 0:
        return np.ones(x.shape[0], bool)
    if lat == 1:
        return (x[:, 0] - x[:, 1]) % 2 == 0
    if lat == 2:
        return x.sum(1) % 2 == 0
    same = np.all((x - x[:, :1]) % 2 == 0, axis=1)
    return same & (x.sum(1) % 4 == 0)


def real_point(lat, x):
    x = np.asarray(x, np.float64)
    if lat == 1:
        return np.stack([x[:, 0], x[:, 1] * SQ3], 1)
    return x


def brute_candidates(lat, u):
    """All lattice points of the integer embedding within the covering radius
    (plus margin) of u, by enumeration."""
    u = np.asarray(u, np.float64)
    if lat == 0:
        return np.arange(np.floor(u[0]) - 1, np.ceil(u[0]) + 2)[:, None]
    if lat == 1:
        ii = np.arange(np.floor(u[0]) - 2, np.ceil(u[0]) + 3)
        jj = np.arange(np.floor(u[1] / SQ3) - 2, np.ceil(u[1] / SQ3) + 3)
        c = np.array(list(itertools.product(ii, jj)))
        return c[members(1, c)]
    if lat == 2:
        axes = [np.arange(np.round(v) - 1, np.round(v) + 2) for v in u]
        c = np.array(list(itertools.product(*axes)))
        return c[members(2, c)]
    out = []
    for par in (0, 1):  # the two cosets of 2D8 in 2E8, each coordinate within 2
        axes = []
        for v in u:
            lo, hi = int(np.floor(v - 2.0)), int(np.ceil(v + 2.0))
            axes.append([c for c in range(lo, hi + 1) if (c - par) % 2 == 0 and abs(c - v) <= 2.0 + 1e-9])
        c = np.array(list(itertools.product(*axes)), np.int64)
        out.append(c[c.sum(1) % 4 == 0])
    return np.concatenate(out)


def sqdist(lat, x, u):
    return np.sum((real_point(lat, np.atleast_2d(x)) - np.asarray(u, np.float64)) ** 2, axis=1)


def make_inputs(lat, rng, n):
    d = {0: 1, 1: 2, 2: 4, 3: 8}[lat]
    parts = [
        rng.standard_normal((n, d)) * 3.0,
        rng.standard_normal((n // 4, d)) * 200.0,
        np.round(rng.standard_normal((n // 4, d)) * 4.0) * 0.5,  # half-integers: ties
        np.round(rng.standard_normal((n // 8, d)) * 4.0),  # integers
        np.zeros((1, d)),
        np.full((1, d), 0.5),
        np.full((1, d), 1.0),
    ]
    return np.concatenate(parts).astype(np.float32)


@pytest.mark.parametrize("lat,tol_rel", [(0, 0.0), (1, 1e-6), (2, 0.0), (3, 2e-6)])
def test_nearest_point_equals_brute_force(orc, lat, tol_rel):
    """The decoders take their decisions in fp32; the tolerance is the fp32
    rounding of the compared distances (zero for Z and D4, whose decisions
    are exact comparisons of exact values)."""
    rng = np.random.default_rng(100 + lat)
    u = make_inputs(lat, rng, 400 if lat == 3 else 2000)
    x = orc.nearest(lat, u)
    assert np.all(members(lat, x)), "decoder returned a non-lattice point"
    for r in range(u.shape[0]):
        c = brute_candidates(lat, u[r])
        best = np.min(sqdist(lat, c, u[r]))
        got = sqdist(lat, x[r], u[r])[0]
        scale = 1.0 + float(np.max(np.abs(u[r]))) if lat == 1 else 8.0
        assert got <= best + tol_rel * scale + 1e-12, (lat, u[r], x[r], got, best)


@pytest.mark.parametrize("lat", [0, 1, 2, 3])
def test_translation_equivariance_away_from_ties(orc, lat):
    rng = np.random.default_rng(200 + lat)
    d = {0: 1, 1: 2, 2: 4, 3: 8}[lat]
    n = 300
    # inputs on a 2^-8 grid so that u + lambda is exact in fp32
    u = (np.round(rng.uniform(-6, 6, (n, d)) * 256) / 256).astype(np.float32)
    lam = orc.nearest(lat, (rng.standard_normal((n, d)) * 10).astype(np.float32))
    if lat == 1:
        # only shifts along the first axis, (2a, 0), keep u + lambda exact in fp32
        lam[:, 0] = 2 * (lam[:, 0] // 2)
        lam[:, 1] = 0
    assert np.all(members(lat, lam))
    shifted = (u.astype(np.float64) + real_point(lat, lam)).astype(np.float32)
    x0 = orc.nearest(lat, u)
    x1 = orc.nearest(lat, shifted)
    checked = 0
    for r in range(n):
        c = brute_candidates(lat, u[r])
        ds = np.sort(sqdist(lat, c, u[r]))
        if ds.size > 1 and ds[1] - ds[0] < 1e-3:
            continue  # near tie: several correct answers
        assert np.array_equal(x1[r], x0[r] + lam[r]), (u[r], lam[r])
        checked += 1
    assert checked > n // 3


G_CLOSED = {
    0: 1.0 / 12.0,
    1: 5.0 / (36.0 * SQ3),
    2: 13.0 / (120.0 * np.sqrt(2.0)),
    3: 929.0 / 12960.0,
}


@pytest.mark.parametrize("lat", [0, 1, 2, 3])
def test_empirical_normalised_second_moment(orc, lat):
    """G = E||e||^2 / (d V^(2/d)) for inputs uniform over a whole period of a
    sublattice (so the error is uniform over the Voronoi cell)."""
    rng = np.random.default_rng(300 + lat)
    d = {0: 1, 1: 2, 2: 4, 3: 8}[lat]
    n = 1_000_000 // d
    if lat == 0:
        period, vol = np.array([1.0]), 1.0
    elif lat == 1:
        period, vol = np.array([2.0, 2.0 * SQ3]), 2.0 * SQ3
    elif lat == 2:
        period, vol = np.full(4, 2.0), 2.0
    else:
        period, vol = np.full(8, 4.0), 256.0
    u = (rng.random((n, d)) * period).astype(np.float32)
    x = orc.nearest(lat, u)
    e2 = np.sum((real_point(lat, x) - u.astype(np.float64)) ** 2, axis=1)
    norm = d * vol ** (2.0 / d)
    g = e2.mean() / norm
    se = e2.std() / np.sqrt(n) / norm
    assert abs(g - G_CLOSED[lat]) < max(5 * se, 1e-4 * G_CLOSED[lat])
    assert abs(g - G_CLOSED[lat]) < 0.005 * G_CLOSED[lat]


def test_lattices_beat_scalar(orc):
    assert G_CLOSED[3] < G_CLOSED[2] < G_CLOSED[1] < G_CLOSED[0]


@pytest.mark.parametrize("lat", [0, 1, 2, 3])
def test_embed_matches_real_point(orc, lat):
    rng = np.random.default_rng(400 + lat)
    d = {0: 1, 1: 2, 2: 4, 3: 8}[lat]
    x = orc.nearest(lat, (rng.standard_normal((100, d)) * 20).astype(np.float32))
    assert np.allclose(orc.embed(lat, x), real_point(lat, x), rtol=1e-7, atol=0)
