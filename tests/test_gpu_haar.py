"""GPU parity of the Haar-rotation variant (hq_plan_set_rotation kind 1)
against the oracle (rotation 1): both compute u = fl32(t c_enc) with t the fp32
fma chain of Q[i][j] x_j in index order, so the words, offsets, Rice
parameters and the fp32/bf16 reconstructions (the chain of Q[j][i] u_j, times
alpha) are bit for bit equal."""
import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

SEED = 0x5EED0001


@pytest.fixture(scope="module")
def hq():
    import lattice_vq_entropy_amd as hq
    assert torch.cuda.is_available(), "GPU tests need a GPU"
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


def haar_plan(hq, lat, alpha=None, bps=4.0):
    p = hq.Plan(lat, bps, SEED).set_rotation(1)
    if alpha is not None:
        p.set_alpha(alpha)
    return p


def parity(hq, orc, lat, x, alpha, dithered=False, tile_base=0):
    plan = haar_plan(hq, lat, alpha)
    n = x.numel() // 128
    ws = plan.workspace(n)
    enc = hq.encode(plan, x.cuda(), ws, dithered=dithered, tile_base=tile_base)
    assert hq.status_sync(ws) == hq.OK
    torch.cuda.synchronize()
    st, ow, oo, ok = orc.encode(lat, SEED, alpha, host_bits(x), dithered=dithered, tile_base=tile_base, rot=1)
    assert st == 0
    offsets = enc.offsets.cpu().numpy().view(np.uint64)
    assert np.array_equal(offsets, oo), f"offsets differ at {np.flatnonzero(offsets != oo)[:8]}"
    assert np.array_equal(enc.k.cpu().numpy()[:n], ok)
    words = enc.words.cpu().numpy().view(np.uint32)[: ow.size]
    assert np.array_equal(words, ow), f"words differ at {np.flatnonzero(words != ow)[:8]}"
    for dt, code in ((torch.float32, 0), (torch.bfloat16, 1)):
        y = hq.decode(plan, enc, ws, out_dtype=dt)
        assert hq.status_sync(ws) == hq.OK
        st, oy = orc.decode(lat, SEED, alpha, ow, oo, ok, dithered=dithered, tile_base=tile_base, out_dtype=code,
                            rot=1)
        assert st == 0
        g = host_bits(y)
        if code == 0:
            g, o = g.view(np.float32), oy.view(np.float32)
        else:
            g, o = (g.astype(np.uint32) << 16).view(np.float32), (oy.astype(np.uint32) << 16).view(np.float32)
        bad = np.flatnonzero(g != o)
        assert bad.size == 0, f"decode differs at {bad[:8]}: {g[bad[:4]]} vs {o[bad[:4]]}"
    return plan, enc, ws


@pytest.mark.parametrize("lat", [0, 1, 2, 3])
@pytest.mark.parametrize("dithered", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_haar_parity(hq, orc, lat, dithered, dtype):
    """Ragged sizes (a chunk and a bit), all lattices, bf16 and fp32 input."""
    g = torch.Generator().manual_seed(lat * 100 + dithered * 10 + (dtype == torch.float32))
    n = 1000 + 37 * lat
    x = torch.randn(n, 128, generator=g) * 0.03
    mask = torch.rand(n, 128, generator=g) < 0.01
    x = torch.where(mask, x * 20.0, x).to(dtype)
    parity(hq, orc, lat, x, 0.004, dithered=dithered, tile_base=555 if dithered else 0)


@pytest.mark.parametrize("n", [1, 31, 33, 300])
def test_haar_small_sizes(hq, orc, n):
    g = torch.Generator().manual_seed(n)
    x = (torch.randn(n, 128, generator=g) * 0.03).to(torch.bfloat16)
    parity(hq, orc, 3, x, 0.004)


def test_haar_kv_workload_shape(hq, orc):
    """A head of the 8x8x32768 KV workload's shape (1 x 1 x 32768 x 128 keys, N(0,1) with
    4 outlier channels x50), D4 at about 2 bps with dither: every tile."""
    g = torch.Generator().manual_seed(77)
    k = torch.randn(32768, 128, generator=g)
    ch = torch.randperm(128, generator=g)[:4]
    k[:, ch] *= 50.0
    k = k.to(torch.bfloat16)
    sigma = float(k.float().pow(2).mean().sqrt())
    alpha = float(np.float32(math.sqrt(2 * math.pi * math.e) * sigma / (2 ** 0.25 * 2.0 ** 2)))
    parity(hq, orc, 2, k, alpha, dithered=True, tile_base=1 << 20)


@pytest.mark.parametrize("lat,bps,dithered", [(3, 4.0, False), (2, 2.0, True)])
def test_haar_calibrate_matches_oracle(hq, orc, lat, bps, dithered):
    g = torch.Generator().manual_seed(int(bps * 10) + lat)
    x = (torch.randn(700, 128, generator=g) * 0.05).to(torch.bfloat16)
    plan = haar_plan(hq, lat, bps=bps)
    ws = plan.workspace(700)
    alpha, rate = plan.calibrate(x.cuda(), ws, dithered=dithered, tile_base=3)
    st, oa, orate, it = orc.calibrate(lat, SEED, bps, host_bits(x), dithered=dithered, tile_base=3, rot=1)
    assert st == 0
    assert alpha == oa and abs(rate - orate) < 1e-12, (alpha, oa, rate, orate)


def test_haar_append_and_container(hq, orc):
    g = torch.Generator().manual_seed(5)
    x = (torch.randn(500, 128, generator=g) * 0.03).to(torch.bfloat16)
    plan = haar_plan(hq, 3, 0.004)
    words, offsets, k = hq.alloc_stream(plan, 500, "cuda")
    ws = plan.workspace(500)
    enc = hq.encode(plan, x[:200].cuda(), ws, out=(words, offsets, k), dithered=True, tile_base=9)
    enc = hq.append(plan, enc, x[200:].cuda(), ws)
    assert hq.status_sync(ws) == hq.OK
    torch.cuda.synchronize()
    st, ow, oo, ok = orc.encode(3, SEED, 0.004, host_bits(x), dithered=True, tile_base=9, rot=1)
    assert np.array_equal(enc.offsets.cpu().numpy().view(np.uint64), oo)
    assert np.array_equal(enc.words.cpu().numpy().view(np.uint32)[: ow.size], ow)
    data = hq.save(plan, enc, ws)
    assert data[:64] == orc.header(3, SEED, 0.004, 4.0, True, True, 9, 500, int(oo[-1]), rot=1)
    plan2, enc2 = hq.load(data)
    assert plan2.rotation()[0] == 1
    ws2 = plan2.workspace(500)
    y = hq.decode(plan2, enc2, ws2, out_dtype=torch.float32)
    assert hq.status_sync(ws2) == hq.OK
    st, oy = orc.decode(3, SEED, 0.004, ow, oo, ok, dithered=True, tile_base=9, rot=1)
    assert np.array_equal(host_bits(y).view(np.float32), oy.view(np.float32))


def test_haar_rejected_by_fused_paths_and_reset(hq):
    import ctypes as C
    L = hq.lib()
    D = C.c_void_p(4096)
    p = haar_plan(hq, 3, 0.004)
    assert L.hq_kv_scores(p.handle, D, 8, D, D, 1, 1, 0, D, 4, D, D, None) == hq.ERR_ARG
    assert L.hq_gemv(p.handle, D, 8, D, D, 2, 256, D, 1, D, D, None) == hq.ERR_ARG
    assert L.hq_gemm(p.handle, D, 8, D, D, 2, 256, D, 1, D, D, None) == hq.ERR_ARG
    a32 = float(np.float32(0.004))
    assert p.get()[1] == np.float32(1.0 / a32) and p.get()[2] == np.float32(a32)  # c_enc = 1/alpha, c_dec = alpha
    p.set_rotation(0)
    assert p.rotation()[0] == 0 and p.get()[1] == np.float32(1.0 / (a32 * math.sqrt(128.0)))
