"""Full-size GPU parity on the workload shapes, by sampled tiles.

Each workload is encoded (and decoded) whole on the GPU with the calibrated
alpha, exactly as the benchmark runs it.  The oracle then encodes and decodes
a sample of tiles on its own (first, last, chunk-boundary and random tiles):
each sampled tile's record bits, Rice parameter and length must equal the
oracle's bit for bit, and its reconstruction must equal the oracle's.  Global
stream properties (offsets start at 0 and grow by the record lengths, the
unused bits of the last word are zero, the achieved rate is within 0.002 bps
of the target) are checked on the whole stream.
"""
import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

SEED = 0x5EED0001
N_SAMPLE = 192


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


def sample_tiles(n_tiles, rng):
    fixed = [0, 1, 31, 32, 33, n_tiles // 2, n_tiles - 33, n_tiles - 32, n_tiles - 2, n_tiles - 1]
    rnd = rng.choice(n_tiles, size=N_SAMPLE - len(fixed), replace=False).tolist()
    return sorted(set(t for t in fixed + rnd if 0 <= t < n_tiles))


def record_value(words: np.ndarray, start: int, length: int) -> int:
    w0, w1 = start >> 5, (start + length + 31) >> 5
    val = int.from_bytes(words[w0:w1].astype("<u4").tobytes(), "little")
    return (val >> (start & 31)) & ((1 << length) - 1)


def check_stream(hq, orc, lat, x2d: torch.Tensor, plan, bps, dithered=False, tile_base=0, out_dtype=torch.bfloat16,
                 seed=0):
    """Encode + decode x on the GPU, compare sampled tiles with the oracle."""
    n = x2d.numel() // 128
    ws = plan.workspace(n)
    enc = hq.encode(plan, x2d, ws, dithered=dithered, tile_base=tile_base)
    assert hq.status_sync(ws) == hq.OK
    y = hq.decode(plan, enc, ws, out_dtype=out_dtype)
    assert hq.status_sync(ws) == hq.OK
    torch.cuda.synchronize()
    alpha = plan.alpha
    offsets = enc.offsets.cpu().numpy().view(np.uint64)
    total = int(offsets[-1])
    words = enc.words[: (total + 31) // 32].cpu().numpy().view(np.uint32)
    kk = enc.k[:n].cpu().numpy()
    lens = np.diff(offsets.astype(np.int64))
    assert offsets[0] == 0 and np.all(lens > 0)
    if total % 32:
        assert int(words[-1]) >> (total % 32) == 0
    assert abs(total / (n * 128) - bps) <= 0.002, total / (n * 128)
    rng = np.random.default_rng(seed)
    tiles = sample_tiles(n, rng)
    xt = x2d.view(n, 128)[torch.tensor(tiles, device=x2d.device)]
    xh = host_bits(xt).reshape(len(tiles), -1)
    yt = y.view(n, 128)[torch.tensor(tiles, device=y.device)].cpu()
    code = 0 if out_dtype == torch.float32 else 1
    for i, t in enumerate(tiles):
        st, ow, oo, ok = orc.encode(lat, SEED, alpha, xh[i], dithered=dithered, tile_base=tile_base + t)
        assert st == 0
        L = int(oo[1])
        assert int(kk[t]) == int(ok[0]), f"tile {t}: k"
        assert int(lens[t]) == L, f"tile {t}: length"
        assert record_value(words, int(offsets[t]), L) == record_value(ow, 0, L), f"tile {t}: record bits"
        st, oy = orc.decode(lat, SEED, alpha, ow, oo, ok, dithered=dithered, tile_base=tile_base + t, out_dtype=code)
        assert st == 0
        if code == 1:
            g = (yt[i].view(torch.int16).numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
            o = (oy.astype(np.uint32) << 16).view(np.float32)
        else:
            g, o = yt[i].numpy(), oy
        assert np.array_equal(g, o), f"tile {t}: reconstruction"
    return enc, ws


def calibrated_plan(hq, lat, bps, x2d, dithered=False, tile_base=0):
    plan = hq.Plan(lat, bps, SEED)
    ws = plan.workspace(x2d.numel() // 128)
    alpha, rate = plan.calibrate(x2d, ws, dithered=dithered, tile_base=tile_base)
    assert abs(rate - bps) <= 0.002
    return plan


@pytest.mark.parametrize("bps", [3.0, 4.0, 5.0])
def test_weight_4096x4096_e8(hq, orc, bps):
    from lattice_vq_entropy_amd import workloads as W
    x = W.c2("cuda")
    plan = calibrated_plan(hq, 3, bps, x)
    check_stream(hq, orc, 3, x, plan, bps, seed=int(bps))


@pytest.mark.parametrize("lat,bps", [(1, 3.0), (1, 5.0), (0, 3.0), (0, 5.0), (3, 4.0)])
def test_weight_8192x28672(hq, orc, lat, bps):
    from lattice_vq_entropy_amd import workloads as W
    x = W.c4("cuda")
    plan = calibrated_plan(hq, lat, bps, x)
    check_stream(hq, orc, lat, x, plan, bps, seed=lat * 10 + int(bps))
    del x
    torch.cuda.empty_cache()


def test_above_65536_chunks(hq, orc):
    """More than 64 blocks of 1024 chunks of 32 tiles (2.1 M tiles, E8 at
    4 bps): the block totals become prefixes in a launch of their own before
    the placement; by sampled tiles."""
    n = 65536 * 32 + 5000
    g = torch.Generator(device="cuda").manual_seed(65537)
    x = (torch.randn(n, 128, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    plan = calibrated_plan(hq, 3, 4.0, x)
    check_stream(hq, orc, 3, x, plan, 4.0, seed=65537)
    del x
    torch.cuda.empty_cache()


def test_kv_8x8x32768_d4_dithered(hq, orc):
    """K and V of one layer, D4 at 2 bps with subtractive dither; plus the
    per-vector bias check of q . k_hat on 4096 random queries."""
    from lattice_vq_entropy_amd import workloads as W
    k, v, q = W.c3("cuda")
    for i, t in enumerate((k, v)):
        plan = calibrated_plan(hq, 2, 2.0, t, dithered=True, tile_base=0)
        enc, ws = check_stream(hq, orc, 2, t, plan, 2.0, dithered=True, tile_base=0, seed=100 + i)
    # bias of q . k_hat - q . k over all keys of one head, for 4096 queries:
    # the mean error per query is zero within its standard error
    plan = calibrated_plan(hq, 2, 2.0, k, dithered=True)
    ws = plan.workspace(k.numel() // 128)
    enc = hq.encode(plan, k, ws, dithered=True)
    khat = hq.decode(plan, enc, ws, out_dtype=torch.float32).view(8, 8, 32768, 128)
    assert hq.status_sync(ws) == hq.OK
    kh = k[0, 0].float()
    err = (q @ (khat[0, 0] - kh).T)  # [4096 queries, 32768 keys]
    mean = err.mean(dim=1)
    se = err.std(dim=1) / math.sqrt(err.shape[1])
    z = (mean / se).abs()
    assert float(z.max()) < 6.0, float(z.max())  # 4096 queries: max |z| of N(0,1) is ~4
    del k, v, khat, err
    torch.cuda.empty_cache()


def test_kv_1x8x131072_e8_scores(hq, orc):
    """Long-context K and V, E8 at 1.7 bps with dither; fused q . k_hat for
    32 query heads (4 per KV head) against all keys, without materialising
    k_hat, compared with the oracle's fp64 scores on sampled keys."""
    from lattice_vq_entropy_amd import workloads as W
    k, v, q = W.c5("cuda")
    heads, seq, qph = 8, 131072, 4
    plan = calibrated_plan(hq, 3, 1.7, k, dithered=True)
    enc, ws = check_stream(hq, orc, 3, k, plan, 1.7, dithered=True, seed=200)
    sc = hq.kv_scores(plan, enc, heads, seq, q, qph, ws)
    assert hq.status_sync(ws) == hq.OK
    sc = sc.cpu().numpy()
    alpha = plan.alpha
    _, _, c_dec = plan.get()
    qh = q.cpu().numpy()
    kb = host_bits(k).reshape(heads * seq, 128)
    rng = np.random.default_rng(7)
    for t in rng.choice(heads * seq, size=64, replace=False).tolist() + [0, heads * seq - 1]:
        h, s = divmod(t, seq)
        st, ow, oo, ok = orc.encode(3, SEED, alpha, kb[t], dithered=True, tile_base=t)
        st, osc = orc.kv_scores(3, SEED, alpha, ow, oo, ok, 1, 1, t, qh[h * qph:(h + 1) * qph], qph)
        assert st == 0
        st, uh = orc.dequant_rotated(3, SEED, ow, 0, int(oo[1]), int(ok[0]), dithered=True, tile_id=t)
        bound = 1e-5 * c_dec * np.linalg.norm(qh[h * qph:(h + 1) * qph].astype(np.float64), axis=1) * \
            math.sqrt(128.0) * np.linalg.norm(uh.astype(np.float64))
        got = sc[h * qph:(h + 1) * qph, s].astype(np.float64)
        assert np.all(np.abs(got - osc[:, 0]) <= bound), (t, got, osc[:, 0])
    # V is decoded plainly
    planv = calibrated_plan(hq, 3, 1.7, v, dithered=True, tile_base=heads * seq)
    check_stream(hq, orc, 3, v, planv, 1.7, dithered=True, tile_base=heads * seq, seed=201)
    del k, v
    torch.cuda.empty_cache()
