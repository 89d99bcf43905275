"""Pins of the oracle's Haar-rotation variant (the QJL rotation the HyperQuant
explainer compares with the RHT for the KV cache; Methodology 1 and 4).

  * Q is orthogonal to fp32 rounding, and is the orthogonal factor of the
    seeded Gaussian matrix by an independent QR (LAPACK Householder);
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


def test_haar_is_the_qr_factor_of_its_gaussian_matrix(orc):
    """Q is the orthogonal factor, with a positive diagonal of R, of the
    seeded Gaussian matrix G (Gram-Schmidt on its columns): against LAPACK's
    Householder QR (numpy.linalg.qr, an independent algorithm) of the same G,
    the fp64 factors agree to ~1e-13, so the oracle's fp32 Q must equal the
    rounded LAPACK Q except where rounding sits on a boundary (one ulp).  G:
    Box-Muller pairs from Philox4x32-10 counters (p, 0, 0, "HAAR") under the
    seed's key, row-major.  libhq's Q is compared with this one bit for bit
    elsewhere, so the pin covers both."""
    key = np.array([SEED & 0xFFFFFFFF, SEED >> 32], dtype=np.uint32)
    r = np.stack([orc.philox(np.array([p, 0, 0, 0x48414152], dtype=np.uint32), key) for p in range(128 * 64)])
    u1 = (r[:, 0].astype(np.float64) + 1.0) / 2.0**32
    u2 = r[:, 1].astype(np.float64) / 2.0**32
    rad, ang = np.sqrt(-2.0 * np.log(u1)), 2.0 * np.pi * u2
    g = np.empty(128 * 128)
    g[0::2], g[1::2] = rad * np.cos(ang), rad * np.sin(ang)
    qn, rn = np.linalg.qr(g.reshape(128, 128))
    qn = qn * np.sign(np.diag(rn))[None, :]
    qo = orc.haar(SEED)
    q32 = qn.astype(np.float32)
    diff = np.abs(qo.astype(np.float64) - qn)
    ulp = np.spacing(np.abs(q32)).astype(np.float64)
    assert np.all(diff <= ulp), diff.max()
    assert np.mean(qo == q32) > 0.999, np.mean(qo == q32)
    # a transposed or sign-flipped recipe is far off
    assert np.abs(qo.astype(np.float64) - qn.T).max() > 0.1
    assert np.abs(qo.astype(np.float64) + qn).max() > 0.1


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


@pytest.mark.parametrize("lat", [2, 3])
def test_haar_scores_equal_query_dot_decoded_key(orc, lat):
    """alpha <Q q, u_hat> (the rotated-domain score) equals q . k_hat with
    k_hat the Haar decoder's fp32 reconstruction, to its rounding."""
    rng = np.random.default_rng(3400 + lat)
    H, S, qph = 2, 30, 3
    kx = rng.standard_normal((H * S, 128)).astype(np.float32)
    q = rng.standard_normal((H * qph, 128)).astype(np.float32)
    alpha = 0.4
    st, w, off, k = orc.encode(lat, SEED, alpha, kx, dithered=True, tile_base=70, rot=1)
    assert st == 0
    st, sc = orc.kv_scores(lat, SEED, alpha, w, off, k, H, S, 70, q, qph, rot=1)
    assert st == 0
    st, y = orc.decode(lat, SEED, alpha, w, off, k, dithered=True, tile_base=70, rot=1)
    khat = y.reshape(H, S, 128).astype(np.float64)
    want = np.einsum("hgi,hsi->hgs", q.reshape(H, qph, 128).astype(np.float64), khat).reshape(H * qph, S)
    scale = np.linalg.norm(q, axis=1)[:, None] * np.linalg.norm(khat.reshape(H * S, 128), axis=1).reshape(H, S).repeat(qph, 0)
    assert np.all(np.abs(sc - want) <= 1e-5 * scale)
    # and not the RHT's scores
    st, sr = orc.kv_scores(lat, SEED, alpha, w, off, k, H, S, 70, q, qph, rot=0)
    assert np.abs(sr - want).max() > 1e-2 * scale.max()


def test_haar_attention_one_key_and_uniform(orc):
    """With the Haar rotation: one key gives its value's reconstruction; scale 0
    gives the mean of the values' reconstructions."""
    rng = np.random.default_rng(3500)
    H, S, qph, lat, ak, av = 2, 20, 2, 3, 0.5, 0.4
    kx = rng.standard_normal((H * S, 128)).astype(np.float32)
    vx = rng.standard_normal((H * S, 128)).astype(np.float32)
    q = rng.standard_normal((H * qph, 128)).astype(np.float32)
    st, kw, ko, kk = orc.encode(lat, SEED, ak, kx, dithered=True, tile_base=0, rot=1)
    st2, vw, vo, vk = orc.encode(lat, SEED, av, vx, dithered=True, tile_base=H * S, rot=1)
    assert st == 0 and st2 == 0
    st, vd = orc.decode(lat, SEED, av, vw, vo, vk, dithered=True, tile_base=H * S, rot=1)
    vd = vd.reshape(H, S, 128).astype(np.float64)
    tol = 256 * 2.0 ** -24 * np.abs(vd).max()
    st, o = orc.kv_attention(lat, SEED, ak, (kw, ko, kk), 0, av, (vw, vo, vk), H * S, H, S, q, qph, 0.0, rot=1)
    assert st == 0
    np.testing.assert_allclose(o.reshape(H, qph, 128), np.repeat(vd.mean(axis=1)[:, None, :], qph, axis=1),
                               rtol=0, atol=tol)
    # one key per head: the streams of keys 0 and S (first of each head), as 1-tile heads
    for h in range(H):
        t = h * S
        ks = (kw, ko[t:t + 2], kk[t:t + 1])
        vs = (vw, vo[t:t + 2], vk[t:t + 1])
        st, o1 = orc.kv_attention(lat, SEED, ak, ks, t, av, vs, H * S + t, 1, 1, q[h * qph:(h + 1) * qph], qph, 0.3,
                                  rot=1)
        assert st == 0
        np.testing.assert_allclose(o1, np.repeat(vd[h, 0][None, :], qph, axis=0), rtol=0, atol=tol)
