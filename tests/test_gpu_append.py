"""GPU parity of hq_append / hq_kv_append (through the C ABI): a stream built
by appending pieces must be the stream that one encode of the concatenated
input gives, bit for bit (records are independent and abut, so the oracle's
encode of the whole input is the definition), for every lattice, with and
without dither (tile ids continue across pieces)."""
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


def stream_of(enc):
    torch.cuda.synchronize()
    n = enc.n_tiles
    offsets = enc.offsets.cpu().numpy().view(np.uint64)
    words = enc.words.cpu().numpy().view(np.uint32)[: (int(offsets[n]) + 31) // 32]
    return words, offsets, enc.k.cpu().numpy()[:n]


def build_by_appending(hq, plan, x, pieces, dithered, tile_base=0, dtype=torch.bfloat16):
    """Encode the first piece into buffers with room for all, append the rest."""
    n_all = x.numel() // 128
    xs = torch.split(x.view(n_all, 128), pieces)
    words, offsets, k = hq.alloc_stream(plan, n_all, x.device)
    ws = plan.workspace(max(pieces))
    enc = hq.encode(plan, xs[0].contiguous(), ws, out=(words, offsets, k), dithered=dithered, tile_base=tile_base)
    for xp in xs[1:]:
        enc = hq.append(plan, enc, xp.contiguous(), ws)
    assert hq.status_sync(ws) == hq.OK
    assert enc.n_tiles == n_all
    return enc


def check(hq, orc, lat, x, pieces, dithered, alpha, tile_base=0):
    plan = hq.Plan(lat, 4.0, SEED).set_alpha(alpha)
    enc = build_by_appending(hq, plan, x.cuda(), pieces, dithered, tile_base)
    gw, go, gk = stream_of(enc)
    st, ow, oo, ok = orc.encode(lat, SEED, alpha, host_bits(x), dithered=dithered, tile_base=tile_base)
    assert st == 0
    assert np.array_equal(go, oo), f"offsets differ at {np.flatnonzero(go != oo)[:8]}"
    assert np.array_equal(gk, ok)
    assert np.array_equal(gw, ow), f"words differ at {np.flatnonzero(gw != ow)[:8]}"
    return plan, enc, (ow, oo, ok)


@pytest.mark.parametrize("lat", [0, 1, 2, 3])
@pytest.mark.parametrize("dithered", [False, True])
def test_append_equals_one_encode(hq, orc, lat, dithered):
    """40 pieces of 1 to 70 tiles (inside a chunk, across chunks, whole chunks)."""
    g = torch.Generator().manual_seed(100 * lat + dithered)
    rng = np.random.default_rng(100 * lat + dithered)
    pieces = [int(p) for p in rng.choice([1, 2, 3, 5, 31, 32, 33, 64, 70], size=40)]
    x = (torch.randn(sum(pieces), 128, generator=g) * 0.03).to(torch.bfloat16)
    check(hq, orc, lat, x, pieces, dithered, alpha=0.004, tile_base=777 if dithered else 0)


def test_append_at_word_boundaries(hq, orc):
    """Records whose lengths are multiples of 32 (Z, k = 0, all symbols 0: 128
    ones of unary) put every append on a word boundary; then one unaligned."""
    x = torch.zeros(9, 128, dtype=torch.bfloat16)
    x[8, :3] = 1.0
    plan, enc, (ow, oo, ok) = check(hq, orc, 0, x, [1, 1, 2, 4, 1], False, alpha=1.0)
    assert all(int(oo[t]) % 32 == 0 for t in range(9))
    g = torch.Generator().manual_seed(5)
    y = torch.cat([x, (torch.randn(5, 128, generator=g)).to(torch.bfloat16)])
    check(hq, orc, 0, y, [9, 1, 1, 3], False, alpha=0.3)


def test_append_large_pieces_and_decode(hq, orc):
    """A piece of 300000 tiles (more than 8192 chunks: the scan launch) after
    one of 1000, then 7; the decode of the whole stream equals the oracle's."""
    g = torch.Generator().manual_seed(3)
    pieces = [1000, 300000, 7]
    x = (torch.randn(sum(pieces), 128, generator=g) * 0.02).to(torch.bfloat16)
    plan, enc, (ow, oo, ok) = check(hq, orc, 3, x, pieces, True, alpha=0.0031, tile_base=5)
    ws = plan.workspace(enc.n_tiles)
    y = hq.decode(plan, enc, ws, out_dtype=torch.bfloat16)
    assert hq.status_sync(ws) == hq.OK
    st, oy = orc.decode(3, SEED, 0.0031, ow, oo, ok, dithered=True, tile_base=5, out_dtype=1)
    assert st == 0
    g16 = host_bits(y)
    nz = (oy & 0x7FFF) != 0  # a zero of either sign (its sign is left to the operation order)
    assert np.array_equal(g16[nz], oy[nz]) and np.all((g16[~nz] & 0x7FFF) == 0)


def test_append_keeps_the_existing_stream(hq):
    """An append writes no word below the one holding the existing stream's
    end bit, keeps that word's bits below it, and nothing past its own end."""
    g = torch.Generator().manual_seed(11)
    plan = hq.Plan(3, 4.0, SEED).set_alpha(0.004)
    x = (torch.randn(300, 128, generator=g) * 0.03).to(torch.bfloat16).cuda()
    words, offsets, k = hq.alloc_stream(plan, 300, x.device)
    sentinel = -0x21524111
    words.fill_(sentinel)
    ws = plan.workspace(300)
    enc = hq.encode(plan, x[:77].contiguous(), ws, out=(words, offsets, k))
    assert hq.status_sync(ws) == hq.OK
    before = words.clone()
    B = enc.total_bits()
    enc = hq.append(plan, enc, x[77:].contiguous(), ws)
    assert hq.status_sync(ws) == hq.OK
    assert torch.equal(words[: B // 32], before[: B // 32])
    if B % 32:
        mask = (1 << (B % 32)) - 1
        assert (int(words[B // 32]) & mask) == (int(before[B // 32]) & mask)
    end = enc.used_words()
    assert bool((words[end:] == sentinel).all())


def test_append_capacity_error(hq):
    """An append that does not fit cap_words reports HQ_ERR_CAPACITY."""
    plan = hq.Plan(3, 4.0, SEED).set_alpha(0.004)
    x = (torch.randn(40, 128) * 0.03).to(torch.bfloat16).cuda()
    words, offsets, k = hq.alloc_stream(plan, 40, x.device)
    ws = plan.workspace(40)
    enc = hq.encode(plan, x[:20].contiguous(), ws, out=(words, offsets, k))
    assert hq.status_sync(ws) == hq.OK
    used = enc.used_words()
    small = (words[: used + 3], offsets, k)
    enc2 = hq.Encoded(small[0], offsets[:21], k[:20], 20, storage=small)
    hq.append(plan, enc2, x[20:].contiguous(), ws)
    assert hq.status_sync(ws) == hq.ERR_CAPACITY
    # an encode of several chunks into too few words also fails, and the
    # workspace stays usable: encodes on it equal encodes on a fresh one
    x = (torch.randn(300, 128) * 0.03).to(torch.bfloat16).cuda()
    w3, o3, k3 = hq.alloc_stream(plan, 300, x.device)
    ws = plan.workspace(300)
    hq.encode(plan, x, ws, out=(w3[:100], o3, k3))
    assert hq.status_sync(ws) == hq.ERR_CAPACITY
    for n in (300, 40, 7, 300):
        e1 = hq.encode(plan, x[:n].contiguous(), ws)
        assert hq.status_sync(ws) == hq.OK
        wsf = plan.workspace(n)
        e2 = hq.encode(plan, x[:n].contiguous(), wsf)
        assert hq.status_sync(wsf) == hq.OK
        assert torch.equal(e1.offsets, e2.offsets)
        assert torch.equal(e1.words[: e1.used_words()], e2.words[: e2.used_words()])
