"""GPU side of the serialized form: compact side information packed and
unpacked on the device (bytes equal to the oracle's packing of the oracle's
own offsets and Rice parameters), and save/load round trips whose decode is
bit for bit the oracle's decode."""
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


def encoded(hq, lat, x, alpha, dithered=False, tile_base=0, bps=4.0):
    plan = hq.Plan(lat, bps, SEED).set_alpha(alpha)
    ws = plan.workspace(x.numel() // 128)
    enc = hq.encode(plan, x.cuda(), ws, dithered=dithered, tile_base=tile_base)
    assert hq.status_sync(ws) == hq.OK
    return plan, enc, ws


@pytest.mark.parametrize("lat,n,dithered", [(3, 4096, False), (2, 1000, True), (0, 33, False), (1, 1, True)])
def test_side_pack_matches_oracle(hq, orc, lat, n, dithered):
    g = torch.Generator().manual_seed(n + lat)
    x = (torch.randn(n, 128, generator=g) * 0.03).to(torch.bfloat16)
    plan, enc, ws = encoded(hq, lat, x, 0.004, dithered, 11)
    side = hq.side_pack(enc, ws)
    assert hq.status_sync(ws) == hq.OK
    st, ow, oo, ok = orc.encode(lat, SEED, 0.004, host_bits(x), dithered=dithered, tile_base=11)
    assert st == 0
    st, oside = orc.side_pack(oo, ok)
    assert st == 0
    nb = len(oside)
    assert side[:nb].cpu().numpy().tobytes() == oside
    o2, k2 = hq.side_unpack(side, n)
    torch.cuda.synchronize()
    assert np.array_equal(o2.cpu().numpy().view(np.uint64), oo)
    assert np.array_equal(k2.cpu().numpy()[:n], ok)


def test_side_pack_capacity(hq):
    """Records of about 2200 bits (Z, alpha 4e-5 on unit data): a chunk spans
    more than 2^16 bits and cannot be packed."""
    x = torch.randn(64, 128, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    plan, enc, ws = encoded(hq, 0, x, 4e-5, bps=16.0)
    assert enc.total_bits() > 2 * 65536
    hq.side_pack(enc, ws)
    assert hq.status_sync(ws) == hq.ERR_CAPACITY


@pytest.mark.parametrize("compact", [True, False])
@pytest.mark.parametrize("lat,dithered", [(3, False), (2, True)])
def test_save_load_round_trip(hq, orc, lat, dithered, compact):
    g = torch.Generator().manual_seed(lat * 7 + compact)
    n = 777
    x = (torch.randn(n, 128, generator=g) * 0.03).to(torch.bfloat16)
    plan, enc, ws = encoded(hq, lat, x, 0.004, dithered, 123 if dithered else 0)
    data = hq.save(plan, enc, ws, compact_side=compact)
    st, ow, oo, ok = orc.encode(lat, SEED, 0.004, host_bits(x), dithered=dithered, tile_base=123 if dithered else 0)
    assert st == 0
    head = orc.header(lat, SEED, 0.004, 4.0, dithered, compact, 123 if dithered else 0, n, int(oo[-1]))
    assert data[:64] == head
    plan2, enc2 = hq.load(data, extra_tiles=64)
    assert enc2.n_tiles == n and enc2.dithered == dithered and enc2.tile_base == (123 if dithered else 0)
    ws2 = plan2.workspace(n + 64)
    y = hq.decode(plan2, enc2, ws2, out_dtype=torch.bfloat16)
    assert hq.status_sync(ws2) == hq.OK
    st, oy = orc.decode(lat, SEED, 0.004, ow, oo, ok, dithered=dithered, tile_base=123 if dithered else 0, out_dtype=1)
    assert st == 0
    g16 = host_bits(y)
    nz = (oy & 0x7FFF) != 0  # a zero of either sign (its sign is left to the operation order)
    assert np.array_equal(g16[nz], oy[nz]) and np.all((g16[~nz] & 0x7FFF) == 0)
    # the loaded stream keeps growing: append 64 tiles, compare with one encode of all
    x2 = (torch.randn(64, 128, generator=g) * 0.03).to(torch.bfloat16)
    enc3 = hq.append(plan2, enc2, x2.cuda(), ws2)
    assert hq.status_sync(ws2) == hq.OK
    torch.cuda.synchronize()
    st, ow3, oo3, ok3 = orc.encode(lat, SEED, 0.004, host_bits(torch.cat([x, x2])), dithered=dithered,
                                   tile_base=123 if dithered else 0)
    assert np.array_equal(enc3.offsets.cpu().numpy().view(np.uint64), oo3)
    assert np.array_equal(enc3.words.cpu().numpy().view(np.uint32)[: ow3.size], ow3)
