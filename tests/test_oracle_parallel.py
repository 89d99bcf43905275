"""The oracle's multi-threaded whole-tensor passes equal its serial loops.

The parallel encode runs each tile's steps on OpenMP threads, scans the
record lengths serially and ORs record bits in atomically; the parallel
decode and rate passes are per-tile.  None of that may change a bit of the
output, the status, or the calibrated alpha, which is what this file checks
(all lattices, plain and dithered, RHT and Haar, bf16 and fp32 input, and
the error paths)."""
import numpy as np
import pytest

SEED = 0x5EED0001


def inputs(rng, n_tiles, bf16):
    x = rng.standard_normal((n_tiles, 128)) * rng.uniform(0.005, 0.05, (n_tiles, 1))
    x[rng.random(x.shape) < 0.01] *= 30.0
    x = x.astype(np.float32)
    if bf16:
        b = x.view(np.uint32).astype(np.uint64)
        return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    return x


@pytest.mark.parametrize("lat", [0, 1, 2, 3])
@pytest.mark.parametrize("dithered", [False, True])
def test_parallel_encode_decode_equal_serial(orc, lat, dithered):
    rng = np.random.default_rng(70 + 2 * lat + int(dithered))
    x = inputs(rng, 3001, bf16=bool(lat & 1))
    alpha = 0.004
    res = {}
    for nt in (1, 7):
        with orc.threads(nt):
            st, w, off, k = orc.encode(lat, SEED, alpha, x, dithered=dithered, tile_base=77)
            assert st == 0
            st2, y = orc.decode(lat, SEED, alpha, w, off, k, dithered=dithered, tile_base=77, out_dtype=orc.BF16)
            assert st2 == 0
            st3, tb = orc.total_bits(lat, SEED, alpha, x, dithered=dithered, tile_base=77)
            assert st3 == 0
        res[nt] = (w, off, k, y, tb)
    for a, b in zip(res[1], res[7]):
        assert np.array_equal(a, b)
    assert res[1][4] == int(res[1][1][-1])


def test_parallel_haar_and_calibration_equal_serial(orc):
    rng = np.random.default_rng(90)
    x = inputs(rng, 700, bf16=False)
    out = {}
    for nt in (1, 5):
        with orc.threads(nt):
            st, a, r, it = orc.calibrate(3, SEED, 4.0, x)
            assert st == 0
            st, w, off, k = orc.encode(2, SEED, 0.01, x, dithered=True, tile_base=5, rot=1)
            assert st == 0
            st, y = orc.decode(2, SEED, 0.01, w, off, k, dithered=True, tile_base=5, rot=1)
            assert st == 0
        out[nt] = (a, r, it, w, off, k, y)
    for a, b in zip(out[1], out[5]):
        assert np.array_equal(np.asarray(a), np.asarray(b))


def test_parallel_statuses_equal_serial(orc):
    rng = np.random.default_rng(91)
    x = inputs(rng, 500, bf16=False)
    bad = x.copy()
    bad[123, 5] = np.nan
    bad[400, 0] = np.inf
    alpha = 0.004
    for nt in (1, 4):
        with orc.threads(nt):
            st, *_ = orc.encode(3, SEED, alpha, bad)
            assert st == orc.ERR_NONFINITE
            st, _ = orc.total_bits(3, SEED, alpha, bad)
            assert st == orc.ERR_NONFINITE
            st, *_ = orc.encode(3, SEED, 1e-9, x)  # step too fine
            assert st == orc.ERR_RANGE
            st, w, off, k = orc.encode(3, SEED, alpha, x, cap_words=1000)  # too small
            assert st == orc.ERR_CAPACITY
    # a record that does not parse: the same status, and zeros for it, either way
    with orc.threads(1):
        st, w, off, k = orc.encode(3, SEED, alpha, x)
    k2 = k.copy()
    k2[17] = 30
    ys = []
    for nt in (1, 6):
        with orc.threads(nt):
            st, y = orc.decode(3, SEED, alpha, w, off, k2)
            assert st == orc.ERR_CORRUPT
            ys.append(y)
    assert np.array_equal(ys[0], ys[1])
    assert np.all(ys[0].reshape(-1, 128)[17] == 0)


def test_parallel_gemv_equals_serial(orc):
    """The product over rows on several threads: the same sums (each row's
    in the same order) and the same status for a record that does not parse."""
    rng = np.random.default_rng(92)
    rows, cols = 37, 640
    x = inputs(rng, rows * cols // 128, bf16=True)
    v = rng.standard_normal((3, cols)).astype(np.float32)
    with orc.threads(1):
        st, w, off, k = orc.encode(3, SEED, 0.004, x)
        assert st == 0
    k2 = k.copy()
    k2[50] = 30
    out = {}
    for nt in (1, 7):
        with orc.threads(nt):
            out[nt] = (orc.gemv(3, SEED, 0.004, w, off, k, rows, cols, v),
                       orc.gemv(3, SEED, 0.004, w, off, k2, rows, cols, v))
    (s1, y1), (c1, z1) = out[1]
    (s7, y7), (c7, z7) = out[7]
    assert s1 == s7 == 0 and c1 == c7 == orc.ERR_CORRUPT
    assert np.array_equal(y1, y7) and np.array_equal(z1, z7)
