"""Pins of the oracle's Haar-rotation variant (the QJL rotation the HyperQuant
explainer compares with the RHT for the KV cache; Methodology 1 and 4).

  * Q is orthogonal to fp32 rounding;
  * Q is Haar distributed: over many seeds the trace has mean 0 and second
    moment 1, and a column's entries have fourth moment 3 / (n (n + 2)), the
    values for the uniform measure on O(n) and on the sphere
    [Diaconis and Shahshahani, J. Appl. Prob. 31A (1994)];
  * the codec with Q: codes equal the nearest points of Q x / alpha computed
    independently in fp64 (all but the rare coordinates within rounding of a
    decision boundary), so orientation (Q, not Q^T) and scale (1/alpha) are
    those of the definition; decode stays within the covering radius; with
    subtractive dither the MSE per scalar is alpha^2 G V^(2/d); the rate
    calibration lands within 0.002 bps.
"""
import numpy as np
import pytest

from test_oracle_codec import DIMS, RCOV2, VOL, gaussian_tiles
from test_oracle_lattice import G_CLOSED

SEED = 0x5EED0001


@pytest.fixture(scope="module")
def orc():
    from oracle import oracle as O
    O.lib()
    return O


def test_haar_is_orthogonal_and_seeded(orc):
    q = orc.haar(SEED).astype(np.float64)
    assert np.abs(q.T @ q - np.eye(128)).max() <= 2 * 2.0 ** -24
    assert np.abs(q @ q.T - np.eye(128)).max() <= 2 * 2.0 ** -24
    assert np.array_equal(orc.haar(SEED), orc.haar(SEED))
    assert not np.array_equal(orc.haar(SEED), orc.haar(SEED + 1))


def test_haar_moments(orc):
    n, seeds = 128, 400
    tr, q4 = [], []
    for s in range(seeds):
        q = orc.haar(1000 + s).astype(np.float64)
        tr.append(np.trace(q))
        q4.append(np.mean(q[:, 0] ** 4))
    tr = np.array(tr)
    assert abs(tr.mean()) < 4 / np.sqrt(seeds)              # E tr Q = 0, sd 1
    assert abs(np.mean(tr ** 2) - 1.0) < 4 * np.sqrt(2 / seeds)  # E (tr Q)^2 = 1
    want = 3.0 / (n * (n + 2))
    q4 = np.array(q4)
    assert abs(q4.mean() - want) < 4 * q4.std() / np.sqrt(seeds)


@pytest.mark.parametrize("lat", [0, 2, 3])
def test_codes_are_nearest_points_of_q_x(orc, lat):
    rng = np.random.default_rng(3000 + lat)
    x = gaussian_tiles(rng, 200)
    alpha = 0.004
    st, w, off, k = orc.encode(lat, SEED, alpha, x, rot=1)
    assert st == 0
    q = orc.haar(SEED).astype(np.float64)
    u = (x.astype(np.float64) @ q.T) / alpha
    want = orc.nearest(lat, u.astype(np.float32).reshape(-1, DIMS[lat])).reshape(x.shape)
    got = np.stack([orc.parse_tile(lat, w, int(off[t]), int(off[t + 1]), int(k[t]))[1] for t in range(200)])
    assert (got == want).mean() > 0.999
    # the other orientation and the RHT's scale give other codes
    ut = (x.astype(np.float64) @ q) / alpha
    wt = orc.nearest(lat, ut.astype(np.float32).reshape(-1, DIMS[lat])).reshape(x.shape)
    assert (got == wt).mean() < 0.9
    us = u / np.sqrt(128.0)
    ws = orc.nearest(lat, us.astype(np.float32).reshape(-1, DIMS[lat])).reshape(x.shape)
    assert (got == ws).mean() < 0.9


@pytest.mark.parametrize("lat", [0, 1, 2, 3])
def test_haar_round_trip_within_covering_radius(orc, lat):
    rng = np.random.default_rng(3100 + lat)
    x = gaussian_tiles(rng, 128)
    alpha = 0.004
    st, w, off, k = orc.encode(lat, SEED, alpha, x, rot=1)
    assert st == 0
    st, y = orc.decode(lat, SEED, alpha, w, off, k, rot=1)
    assert st == 0
    err = np.linalg.norm(y.reshape(x.shape).astype(np.float64) - x, axis=1)
    bound = np.sqrt(RCOV2[lat] * 128 / DIMS[lat]) * alpha
    assert np.all(err <= bound * (1 + 1e-5) + 1e-6 * np.linalg.norm(x, axis=1))
    assert err.mean() < 0.2 * np.linalg.norm(x, axis=1).mean()


@pytest.mark.parametrize("lat", [2, 3])
def test_haar_dithered_distortion_closed_form(orc, lat):
    rng = np.random.default_rng(3200 + lat)
    x = (rng.standard_normal((2000, 128)) * 0.7).astype(np.float32)
    alpha = 0.05
    st, w, off, k = orc.encode(lat, SEED, alpha, x, dithered=True, tile_base=99, rot=1)
    assert st == 0
    st, y = orc.decode(lat, SEED, alpha, w, off, k, dithered=True, tile_base=99, rot=1)
    assert st == 0
    e2 = np.mean((y.reshape(x.shape).astype(np.float64) - x) ** 2, axis=1) / alpha ** 2
    want = G_CLOSED[lat] * VOL[lat] ** (2.0 / DIMS[lat])
    assert abs(e2.mean() - want) < 5 * e2.std() / np.sqrt(e2.size)


def test_haar_calibration_hits_the_rate(orc):
    rng = np.random.default_rng(3300)
    x = (rng.standard_normal((512, 128))).astype(np.float32)
    st, alpha, rate, it = orc.calibrate(2, SEED, 2.0, x, dithered=True, rot=1)
    assert st == 0 and abs(rate - 2.0) <= 0.002
    st, bits = orc.total_bits(2, SEED, alpha, x, dithered=True, rot=1)
    assert st == 0 and abs(bits / x.size - rate) < 1e-12
