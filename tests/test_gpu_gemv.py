"""GPU parity of the fused decode + matrix-vector product (hq_gemv) against
the oracle's fp64 product with the reconstructed weights.

Bound, per output y[j][r] (u = 2^-24, first order, derived from the fp32
operations the kernels perform in a fixed order):
  * the rotated blocks H D x_b are 7 butterfly levels of fp32 adds: each entry
    is off by at most 7u ||x_b||_1, which moves the tile's contribution
    c_dec <u_hat_b, .> by at most 7u c_dec ||u_hat_b||_1 ||x_b||_1
    <= 7u ||w_b||_2 ||x_b||_1   (||u_hat||_1 <= sqrt(128) ||u_hat||_2 and
    ||w_b||_2 = c_dec sqrt(128) ||u_hat_b||_2 for the reconstructed row piece w_b);
  * each tile's dot product is an 8-term fma chain per lane and a 4-level
    lane tree, 12 roundings, and the row sum over the nblk tiles is
    ceil(nblk/64) sequential adds per lane, a 4-level tree and 3 adds, then one
    multiply by c_dec: (12 + ceil(nblk/64) + 8) u c_dec sum_b |u_hat_b| . |H D x_b|
    <= (20 + ceil(nblk/64)) u sum_b ||w_b||_2 ||x_b||_2 (Cauchy-Schwarz,
    ||H D x_b||_2 = sqrt(128) ||x_b||_2).
The test allows 1.25 times the sum.  ||w_b||_2 comes from the oracle's decode.
"""
import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

SEED = 0x5EED0001
U = 2.0 ** -24


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


def bound(orc, lat, alpha, ow, oo, ok, rows, cols, x):
    st, wd = orc.decode(lat, SEED, alpha, ow, oo, ok)
    assert st == 0
    nblk = cols // 128
    wn = np.linalg.norm(wd.reshape(rows, nblk, 128).astype(np.float64), axis=2)        # [rows, nblk]
    xb = x.reshape(x.shape[0], nblk, 128).astype(np.float64)
    x2, x1 = np.linalg.norm(xb, axis=2), np.abs(xb).sum(axis=2)                          # [nb, nblk]
    chain = 20 + math.ceil(nblk / 64)
    return 1.25 * U * (chain * (x2 @ wn.T) + 7.0 * (x1 @ wn.T)) + 1e-30                  # [nb, rows]


def check(hq, orc, lat, w: torch.Tensor, x: np.ndarray, alpha: float):
    rows, cols = w.shape
    st, ow, oo, ok = orc.encode(lat, SEED, alpha, host_bits(w))
    assert st == 0
    st, yo = orc.gemv(lat, SEED, alpha, ow, oo, ok, rows, cols, x)
    assert st == 0
    plan = hq.Plan(lat, 4.0, SEED).set_alpha(alpha)
    ws = plan.workspace(rows * cols // 128)
    enc = hq.encode(plan, w.cuda(), ws)
    assert hq.status_sync(ws) == hq.OK
    gws = hq.gemv_workspace(rows, cols, x.shape[0])
    y = hq.gemv(plan, enc, rows, cols, torch.from_numpy(x).cuda(), gws)
    assert hq.status_sync(gws) == hq.OK
    y = y.cpu().numpy().astype(np.float64)
    b = bound(orc, lat, alpha, ow, oo, ok, rows, cols, x)
    err = np.abs(y - yo)
    assert np.all(err <= b), f"max err/bound {float((err / b).max()):.3f} at {np.unravel_index(np.argmax(err / b), b.shape)}"
    return float((err / b).max())


@pytest.mark.parametrize("rows,cols,nb", [(1, 128, 1), (3, 256, 2), (5, 384, 3), (40, 4096, 1), (33, 4224, 4),
                                          (7, 1152, 16), (70, 640, 5)])
def test_gemv_shapes(hq, orc, rows, cols, nb):
    """One row of one tile; rows of 2, 3, 9 and 5 blocks (the block index taken
    by a modulo per tile); 32 blocks (a chunk is a row); 33 blocks (chunks
    straddle rows); up to 16 vectors."""
    g = torch.Generator().manual_seed(rows * 1000 + cols + nb)
    w = (torch.randn(rows, cols, generator=g) * 0.03).to(torch.bfloat16)
    x = (torch.randn(nb, cols, generator=g)).numpy().astype(np.float32)
    check(hq, orc, 3, w, x, 0.004)


@pytest.mark.parametrize("lat", [0, 1, 2])
def test_gemv_other_lattices(hq, orc, lat):
    g = torch.Generator().manual_seed(77 + lat)
    w = (torch.randn(21, 512, generator=g) * 0.03).to(torch.bfloat16)
    x = torch.randn(2, 512, generator=g).numpy().astype(np.float32)
    check(hq, orc, lat, w, x, 0.004)


def test_gemv_weight_4096x4096(hq, orc):
    """The whole 4096x4096 workload matrix at the calibrated 4-bps alpha, one
    vector, every output against the oracle."""
    from lattice_vq_entropy_amd import workloads as W
    w = W.c2("cpu")
    plan = hq.Plan(3, 4.0, SEED)
    ws = plan.workspace(w.numel() // 128)
    alpha, rate = plan.calibrate(w.cuda(), ws)
    x = torch.randn(1, 4096, generator=torch.Generator().manual_seed(4096)).numpy().astype(np.float32)
    check(hq, orc, 3, w, x, alpha)


def test_gemv_weight_8192x28672_all_rows(hq, orc):
    """The 8192x28672 workload matrix (E8, calibrated 4 bps), one vector, every
    one of the 8192 outputs against the oracle's product (the oracle encodes
    the whole matrix and multiplies it on all host threads; rows are
    independent, so its sums are the single-thread ones)."""
    import os
    from lattice_vq_entropy_amd import workloads as W
    threads = max(1, min(16, os.cpu_count() or 1))
    w = W.c4("cuda")
    rows, cols = w.shape
    plan = hq.Plan(3, 4.0, SEED)
    ws = plan.workspace(w.numel() // 128)
    alpha, rate = plan.calibrate(w, ws)
    enc = hq.encode(plan, w, ws)
    assert hq.status_sync(ws) == hq.OK
    x = torch.randn(1, cols, generator=torch.Generator().manual_seed(28672)).numpy().astype(np.float32)
    gws = hq.gemv_workspace(rows, cols, 1)
    y = hq.gemv(plan, enc, rows, cols, torch.from_numpy(x).cuda(), gws)
    assert hq.status_sync(gws) == hq.OK
    y = y.cpu().numpy().astype(np.float64)
    wh = host_bits(w)
    del w, enc, ws
    torch.cuda.empty_cache()
    print(f"gemv 8192x28672: oracle on {threads} threads", flush=True)
    with orc.threads(threads):
        st, ow, oo, ok = orc.encode(3, SEED, alpha, wh)
        assert st == 0
        st, yo = orc.gemv(3, SEED, alpha, ow, oo, ok, rows, cols, x)
        assert st == 0
        b = bound(orc, 3, alpha, ow, oo, ok, rows, cols, x)
    err = np.abs(y - yo)
    assert np.all(err <= b), f"max err/bound {float((err / b).max()):.3f} at {np.unravel_index(np.argmax(err / b), b.shape)}"


def test_gemv_corrupt_record(hq, orc):
    g = torch.Generator().manual_seed(9)
    w = (torch.randn(4, 256, generator=g) * 0.03).to(torch.bfloat16).cuda()
    plan = hq.Plan(3, 4.0, SEED).set_alpha(0.004)
    ws = plan.workspace(8)
    enc = hq.encode(plan, w, ws)
    assert hq.status_sync(ws) == hq.OK
    enc.k[3] = (int(enc.k[3].item()) + 1) % 23
    gws = hq.gemv_workspace(4, 256, 1)
    hq.gemv(plan, enc, 4, 256, torch.ones(1, 256, device="cuda"), gws)
    assert hq.status_sync(gws) == hq.ERR_CORRUPT
