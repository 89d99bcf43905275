"""Pins of bit-stripping, zigzag and Rice coding in the oracle.

The HyperQuant explainer (technical summary, Methodology 3) states that the
lattice membership constraints fix some bits of each integer code vector,
which are removed losslessly, and that the remaining symbols are Rice coded,
a variable-length code optimal for geometric sources.  Pins used here:
  * stripping is a bijection between the lattice and Z^d (x {0,1} for the E8
    coset bit): exactly log2(index) bits are removed and nothing is lost;
  * zigzag is a bijection Z -> N ordered by magnitude;
  * Rice(k) on a geometric source with theta^(2^k) = 1/2 costs exactly k + 2
    bits per symbol on average (Golomb 1966; Gallager & Van Voorhis 1975);
  * the chosen k minimises the tile length, which is convex in k;
  * hand-derived records of the stated layout (tests/golden/layout_records.json);
  * parse(write(codes)) = codes.
"""
import json
import os

import numpy as np
import pytest

from test_oracle_lattice import members

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DIMS = {0: 1, 1: 2, 2: 4, 3: 8}


@pytest.mark.parametrize("lat", [0, 1, 2, 3])
def test_strip_is_a_bijection(orc, lat):
    rng = np.random.default_rng(500 + lat)
    d = DIMS[lat]
    # arbitrary symbols -> unstrip gives lattice points -> strip gives them back
    sym = rng.integers(-1000, 1000, (3000, d)).astype(np.int32)
    raw = rng.integers(0, 2, 3000).astype(np.int32) if lat == 3 else np.zeros(3000, np.int32)
    x = orc.unstrip(lat, sym, raw)
    assert np.all(members(lat, x))
    sym2, raw2 = orc.strip(lat, x)
    assert np.array_equal(sym2, sym) and np.array_equal(raw2, raw)
    # arbitrary lattice points -> strip -> unstrip gives them back
    pts = orc.nearest(lat, (rng.standard_normal((3000, d)) * 50).astype(np.float32))
    s, r = orc.strip(lat, pts)
    assert np.array_equal(orc.unstrip(lat, s, r), pts)


@pytest.mark.parametrize("lat,index_bits", [(0, 0), (1, 1), (2, 1), (3, 8)])
def test_strip_removes_log2_index_bits(orc, lat, index_bits):
    """On large lattice points the symbols are smaller than the codes by
    log2(index of the embedding in Z^d) bits per vector in total, counting
    the raw E8 coset bit as one bit kept: 2E8 has index 2^8, D4 and the A2
    checkerboard 2, Z 1."""
    rng = np.random.default_rng(550 + lat)
    d = DIMS[lat]
    x = orc.nearest(lat, (rng.uniform(2.0**14, 2.0**15, (4000, d)) * rng.choice([-1, 1], (4000, d))).astype(np.float32))
    sym, raw = orc.strip(lat, x)
    removed = np.sum(np.log2(np.abs(x.astype(np.float64)) / np.abs(sym.astype(np.float64))), axis=1)
    kept_raw = 1.0 if lat == 3 else 0.0
    assert abs(removed.mean() - kept_raw - index_bits) < 0.01


def test_zigzag_bijection(orc):
    vals = list(range(-1000, 1001))
    ms = [orc.zigzag(v) for v in vals]
    assert sorted(ms) == list(range(2001))
    for v, m in zip(vals, ms):
        assert orc.unzigzag(m) == v
    # ordered by magnitude, non-negative first
    by_m = [orc.unzigzag(m) for m in range(9)]
    assert [abs(v) for v in by_m] == sorted(abs(v) for v in by_m)
    assert orc.zigzag(2**20 + 2) < 2**22 and orc.zigzag(-(2**20 + 2)) < 2**22


@pytest.mark.parametrize("k", [0, 1, 3, 5])
def test_rice_length_on_geometric_source(orc, k):
    """theta^(2^k) = 1/2: remainder uniform on k bits, quotient geometric(1/2),
    mean length k + 2 bits per symbol exactly."""
    rng = np.random.default_rng(600 + k)
    theta = 0.5 ** (1.0 / 2**k)
    n_tiles = 4000
    m = (rng.geometric(1.0 - theta, n_tiles * 128) - 1).astype(np.uint32).reshape(n_tiles, 128)
    lens = np.array([orc.rice_len(m[t], k, 0) for t in range(n_tiles)], np.float64) / 128.0
    se = lens.std() / np.sqrt(n_tiles)
    assert abs(lens.mean() - (k + 2)) < 5 * se
    # with the raw E8 bits added the length grows by exactly 16
    assert orc.rice_len(m[0], k, 16) == orc.rice_len(m[0], k, 0) + 16


def test_kstar_is_the_smallest_minimiser_and_matches_the_convexity_rule(orc):
    """L(k+1) - L(k) = 128 - S(k), S(k) = sum ceil((m >> k) / 2) non-increasing,
    so the smallest minimiser is min{k : S(k) <= 128}."""
    rng = np.random.default_rng(700)
    for t in range(600):
        scale = 2.0 ** rng.uniform(-2, 20)
        m = np.minimum(np.abs(rng.standard_normal(128) * scale), 2**21).astype(np.uint32)
        if t % 7 == 0:
            m[:] = rng.integers(0, 3)  # constant tiles: ties between k values
        kstar = orc.rice_kstar(m, 16 if t % 2 else 0)
        S = [int(np.sum((m.astype(np.int64) >> k) + 1 >> 1)) for k in range(23)]
        rule = next(k for k in range(23) if S[k] <= 128)
        assert kstar == rule
        lens = [orc.rice_len(m, k, 0) for k in range(23)]
        assert lens[kstar] == min(lens) and all(l > lens[kstar] for l in lens[:kstar])


def _golden_codes(rec):
    codes = np.full(128, rec.get("codes_default", 0), np.int32)
    for i, v in rec.get("codes_sparse", {}).items():
        codes[int(i)] = v
    for vi, vec in rec.get("codes_vectors", {}).items():
        codes[8 * int(vi):8 * int(vi) + 8] = vec
    return codes


def test_hand_derived_records(orc):
    with open(os.path.join(GOLDEN, "layout_records.json")) as f:
        recs = json.load(f)["records"]
    lat_of = {"Z": 0, "A2": 1, "D4": 2, "E8": 3}
    for rec in recs:
        lat = lat_of[rec["lattice"]]
        codes = _golden_codes(rec)
        words, L, k = orc.write_record_codes(lat, codes)
        want = [int(h, 16) for h in rec["words"]]
        assert (L, k) == (rec["length"], rec["k"]), rec["name"]
        assert words[:len(want)].tolist() == want, rec["name"]
        assert not words[len(want):].any()
        st, back = orc.parse_tile(lat, words, 0, L, k)
        assert st == 0 and np.array_equal(back, codes)


@pytest.mark.parametrize("lat", [0, 1, 2, 3])
def test_parse_inverts_write_at_any_offset(orc, lat):
    rng = np.random.default_rng(800 + lat)
    d = DIMS[lat]
    for t in range(200):
        scale = 2.0 ** rng.uniform(-3, 12)
        codes = orc.nearest(lat, (rng.standard_normal((128 // d, d)) * scale).astype(np.float32)).reshape(-1)
        off = int(rng.integers(0, 200))
        words, L, k = orc.write_record_codes(lat, codes, n_words=200, off=off)
        st, back = orc.parse_tile(lat, words, off, off + L, k)
        assert st == 0 and np.array_equal(back, codes)
        # the bits before the record are untouched
        assert int(words[off >> 5]) & ((1 << (off & 31)) - 1) == 0
