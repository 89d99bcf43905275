"""GPU parity of the matrix-core products (hq_gemm) against the oracle's fp64
product with the reconstructed weights, for 1 to 64 vectors.

Bound, per output y[j][r] (u = 2^-24, first order, a-posteriori where the
operands are known exactly; derived from the operations the kernels perform):
  * the rotated blocks x~ = H D x_b are the fp32 butterfly of the decoder,
    the same additions as the oracle's fp32 transform (pinned bit for bit by
    the encode parity), so their error against the exact H D x_b is known and
    enters as |c_dec sum_c U[r][c] (x~32 - x~)[j][c]| with U the integer codes;
  * the split into bf16 pieces: x~ = hi + lo + e, |e| <= 2^-16 |x~|;
    U = Uh + Ul + f, |f| <= 2^-16 |U| (0 below 2^16); the dropped lo*Ul is at
    most 2^-16 |x~ U|: together 3 2^-16 sum_c |x~||U| (plus 2^-120 per code for
    bf16 pieces below the normal range);
  * fp32 accumulation: each MFMA adds 16 products and the accumulator (at most
    17 roundings), a wave chains 6 of them per column block over `per` blocks,
    then 3 adds over the waves, the splits in order, one multiply by c_dec:
    D = 102 per + splits + 3 roundings on sum_c |x~||U|.
The test allows 1.25 times c_dec times the sum, plus u |y|.
"""
import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

SEED = 0x5EED0001
U_ = 2.0 ** -24


@pytest.fixture(scope="module")
def hq():
    import lattice_vq_entropy_amd as hq
    assert torch.cuda.is_available()
    hq.lib()
    return hq


@pytest.fixture(scope="module")
def orc():
    from oracle import oracle as O
    O.lib()
    return O


def host_bits(x: torch.Tensor) -> np.ndarray:
    x = x.detach().contiguous().cpu()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16).reshape(-1)
    return x.numpy().reshape(-1)


def hadamard(n=128):
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def split_shape(rows, cols):
    """Column blocks per work-group and the number of splits (as the library chooses them)."""
    nblk, ntn = cols // 128, -(-rows // 32)
    want = 1 if ntn >= 2048 else -(-2048 // ntn)
    want = max(1, min(want, nblk))
    per = -(-nblk // want)
    return per, -(-nblk // per)


def bound(orc, lat, alpha, stream, rows, cols, x, yref, row_ids=None):
    ow, oo, ok = stream
    nblk = cols // 128
    st, uh = orc.dequant_rotated_many(lat, SEED, ow, oo, ok, rows * nblk)
    assert st == 0
    U = uh.astype(np.float64).reshape(rows, cols)
    sg = orc.signs(SEED)
    hd = hadamard() * sg.astype(np.float64)[None, :]
    nb = x.shape[0]
    x32 = np.zeros((nb, cols))
    x64 = np.zeros((nb, cols))
    for j in range(nb):
        for b in range(nblk):
            blk = x[j, 128 * b:128 * (b + 1)].astype(np.float32)
            x32[j, 128 * b:128 * (b + 1)] = orc.fwht(sg * blk).astype(np.float64)
            x64[j, 128 * b:128 * (b + 1)] = hd @ blk.astype(np.float64)
    _, c_dec = orc.scales(alpha)
    per, splits = split_shape(rows if row_ids is None else row_ids[1], cols)
    D = 102 * per + splits + 3
    rot = np.abs((x32 - x64) @ U.T)
    A = np.abs(x32) @ np.abs(U).T
    tiny = 2.0 ** -120 * np.abs(U).sum(axis=1)[None, :]
    return 1.25 * c_dec * (rot + (3 * 2.0 ** -16 + D * U_) * A + tiny) + U_ * np.abs(yref) + 1e-30


def run(hq, orc, lat, w: torch.Tensor, x: np.ndarray, alpha: float):
    rows, cols = w.shape
    st, ow, oo, ok = orc.encode(lat, SEED, alpha, host_bits(w))
    assert st == 0
    st, yo = orc.gemv(lat, SEED, alpha, ow, oo, ok, rows, cols, x)
    assert st == 0
    plan = hq.Plan(lat, 4.0, SEED).set_alpha(alpha)
    ws = plan.workspace(rows * cols // 128)
    enc = hq.encode(plan, w.cuda(), ws)
    assert hq.status_sync(ws) == hq.OK
    gws = hq.gemm_workspace(rows, cols, x.shape[0])
    y = hq.gemm(plan, enc, rows, cols, torch.from_numpy(x).cuda(), gws)
    assert hq.status_sync(gws) == hq.OK
    y = y.cpu().numpy().astype(np.float64)
    b = bound(orc, lat, alpha, (ow, oo, ok), rows, cols, x, yo)
    err = np.abs(y - yo)
    assert np.all(err <= b), f"max err/bound {float((err / b).max()):.3f} at {np.unravel_index(np.argmax(err / b), b.shape)}"
    return y, yo, b, (ow, oo, ok)


@pytest.mark.parametrize("rows,cols,nb", [(1, 128, 1), (33, 384, 5), (70, 4224, 33), (64, 1152, 64),
                                          (100, 640, 32), (31, 256, 2)])
def test_gemm_shapes(hq, orc, rows, cols, nb):
    """One tile; row counts off and on multiples of 32; 1, 2, 3, 5, 9 and 33
    column blocks; one and two 32-vector tiles (33 and 64 vectors)."""
    g = torch.Generator().manual_seed(rows * 1000 + cols + nb)
    w = (torch.randn(rows, cols, generator=g) * 0.03).to(torch.bfloat16)
    x = torch.randn(nb, cols, generator=g).numpy().astype(np.float32)
    run(hq, orc, 3, w, x, 0.004)


@pytest.mark.parametrize("lat", [0, 2])
def test_gemm_other_lattices(hq, orc, lat):
    g = torch.Generator().manual_seed(91 + lat)
    w = (torch.randn(45, 512, generator=g) * 0.03).to(torch.bfloat16)
    x = torch.randn(7, 512, generator=g).numpy().astype(np.float32)
    run(hq, orc, lat, w, x, 0.004)


@pytest.mark.parametrize("case", range(6))
def test_gemm_random_shapes(hq, orc, case):
    """Seeded random cases: Z, D4 or E8, 1-150 rows, 1-24 column blocks,
    1-64 vectors, weights and vectors of random scale."""
    rng = np.random.default_rng(31000 + case)
    lat = int(rng.choice([0, 2, 3]))
    rows, cols, nb = int(rng.integers(1, 151)), 128 * int(rng.integers(1, 25)), int(rng.integers(1, 65))
    g = torch.Generator().manual_seed(31000 + case)
    w = (torch.randn(rows, cols, generator=g) * float(rng.uniform(0.005, 0.5))).to(torch.bfloat16)
    x = (torch.randn(nb, cols, generator=g) * float(rng.uniform(0.1, 10.0))).numpy().astype(np.float32)
    alpha = float(np.float32(float(w.float().pow(2).mean().sqrt()) * float(rng.uniform(0.05, 0.5))))
    run(hq, orc, lat, w, x, alpha)


def test_gemm_large_codes(hq, orc):
    """Codes of 2^16 and more (alpha far below the data's scale), where the
    code's bf16 split is inexact and the 2^-16 term carries the error."""
    g = torch.Generator().manual_seed(17)
    w = (torch.randn(40, 256, generator=g)).to(torch.bfloat16)
    x = torch.randn(3, 256, generator=g).numpy().astype(np.float32)
    y, yo, b, (ow, oo, ok) = run(hq, orc, 0, w, x, 2e-5)
    st, uh = orc.dequant_rotated_many(0, SEED, ow, oo, ok, 80)
    assert np.abs(uh).max() >= 2 ** 16


def test_gemm_bound_sees_a_missing_tile(hq, orc):
    """The bound is tighter than the effect of leaving out one tile: the
    oracle's product with one record corrupted (counted as zero) differs from
    the full product by more than the bound in that row."""
    g = torch.Generator().manual_seed(23)
    rows, cols, nb = 33, 1024, 4
    w = (torch.randn(rows, cols, generator=g) * 0.03).to(torch.bfloat16)
    x = torch.randn(nb, cols, generator=g).numpy().astype(np.float32)
    y, yo, b, (ow, oo, ok) = run(hq, orc, 3, w, x, 0.004)
    for t in (0, 5 * 8 + 3, rows * 8 - 1):
        k2 = ok.copy()
        k2[t] = 23  # beyond any Rice parameter: the record no longer parses
        st, y2 = orc.gemv(3, SEED, 0.004, ow, oo, k2, rows, cols, x)
        assert st == 5
        r = t // 8
        assert (np.abs(y2[:, r] - yo[:, r]) > b[:, r]).all()


def test_gemm_weight_4096x4096(hq, orc):
    """The whole 4096x4096 workload matrix (E8, alpha for 4 bps from the
    high-resolution formula), 16 vectors, every output against the oracle."""
    from lattice_vq_entropy_amd import workloads as W
    w = W.c2("cpu")
    sigma = float(w.float().pow(2).mean().sqrt())
    alpha = float(np.float32(math.sqrt(2 * math.pi * math.e) * sigma / (2.0 * 2.0 ** 4)))
    x = torch.randn(16, 4096, generator=torch.Generator().manual_seed(4097)).numpy().astype(np.float32)
    run(hq, orc, 3, w, x, alpha)


def test_gemm_weight_8192x28672_all_rows(hq, orc):
    """The 8192x28672 workload matrix (E8, alpha for 4 bps from the
    high-resolution formula), 32 vectors: all 8192 x 32 outputs against the
    oracle's product (on all host threads; rows are independent, so its sums
    are the single-thread ones)."""
    import os
    from lattice_vq_entropy_amd import workloads as W
    threads = max(1, min(16, os.cpu_count() or 1))
    w = W.c4("cpu")
    rows, cols = w.shape
    sigma = float(w.float().pow(2).mean().sqrt())
    alpha = float(np.float32(math.sqrt(2 * math.pi * math.e) * sigma / (2.0 * 2.0 ** 4)))
    x = torch.randn(32, cols, generator=torch.Generator().manual_seed(28673)).numpy().astype(np.float32)
    print(f"gemm 8192x28672 x 32: oracle on {threads} threads", flush=True)
    with orc.threads(threads):
        run(hq, orc, 3, w, x, alpha)
    del w


def test_gemm_arguments(hq):
    import ctypes as C
    L = hq.lib()
    D = C.c_void_p(4096)
    p = hq.Plan("A2", 4.0, 1).set_alpha(0.5)
    assert L.hq_gemm(p.handle, D, 8, D, D, 2, 256, D, 1, D, D, None) == hq.ERR_ARG   # A2
    q = hq.Plan("E8", 4.0, 1).set_alpha(0.5)
    assert L.hq_gemm(q.handle, D, 8, D, D, 2, 256, D, 65, D, D, None) == hq.ERR_ARG  # nb > 64
    assert L.hq_gemm(q.handle, D, 8, D, D, 2, 200, D, 1, D, D, None) == hq.ERR_ARG   # cols % 128
    assert L.hq_gemm(q.handle, D, 8, D, D, 0, 256, D, 1, D, D, None) == hq.OK
