"""Compact workspaces: staging slots sized from the plan's rate, and the
chunks that do not fit them.

A plan with a compact workspace stages each chunk's bits in a slot sized from
its rate (2.5 bits per scalar to spare); a chunk whose bits do not fit is
encoded again by the placement, from its input, straight into the stream.
These tests run compact plans whose nominal rate is far below the rate that
their alpha gives, so that staged and re-encoded chunks alternate, and compare
the whole stream (offsets, k, words) and the decode with the oracle, through
the C ABI: every lattice, plain and dithered, bf16 and fp32 input, the Haar
rotation, an append whose first chunk is re-encoded, more than 8192 chunks
(the two-level offset scan), and against the default full-size slots and the
noalloc entry point.
"""
import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

SEED = 0x5EED0001
NU = {0: 1.0, 1: math.sqrt(2 * math.sqrt(3)), 2: 2 ** 0.25, 3: 2.0}  # cell scale of each lattice


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


def host_bits(x):
    x = x.detach().contiguous().cpu()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16).reshape(-1)
    return x.numpy().reshape(-1)


def stream_of(enc):
    torch.cuda.synchronize()
    n = enc.n_tiles
    offsets = enc.offsets.cpu().numpy().view(np.uint64)[: n + 1].copy()
    words = enc.words.cpu().numpy().view(np.uint32)[: (int(offsets[n]) + 31) // 32].copy()
    return words, offsets, enc.k.cpu().numpy()[:n].copy()


def first_unstaged_bits(bps):
    """The smallest chunk bit count that is not staged, from the slot rule the
    library documents: a slot of 128 (bps + 2.5) + 8 words in whole uint4;
    a chunk is staged when its blocks ((A >> 5) + 5) >> 2 leave one block
    of the slot free, i.e. when A < (slot - 5) * 32."""
    w = int(bps * 128 + 2.5 * 128 + 8) + 1
    slot = min((w + 3) & ~3, 2968)
    return (slot - 5) * 32


def chunk_bits(offsets):
    n = len(offsets) - 1
    ends = list(range(32, n, 32)) + [n]
    starts = list(range(0, n, 32))
    return np.array([int(offsets[e]) - int(offsets[s]) for s, e in zip(starts, ends)])


def rows_input(rows, cols, seed, dtype=torch.bfloat16):
    """Rows of Gaussian data with per-row scales over a factor of 30, so the
    per-chunk rate spreads over about 5 bits per scalar."""
    g = torch.Generator().manual_seed(seed)
    sig = torch.exp(torch.empty(rows, 1).uniform_(math.log(0.002), math.log(0.06), generator=g))
    return (torch.randn(rows, cols, generator=g) * sig).to(dtype)


def compare(hq, orc, plan, lat, alpha, x, dithered=False, tile_base=0, rot=0, decode=True):
    n = x.numel() // 128
    ws = plan.workspace(n)
    enc = hq.encode(plan, x.cuda(), ws, dithered=dithered, tile_base=tile_base)
    assert hq.status_sync(ws) == hq.OK
    gw, go, gk = stream_of(enc)
    st, ow, oo, ok = orc.encode(lat, SEED, alpha, host_bits(x), dithered=dithered, tile_base=tile_base, rot=rot)
    assert st == 0
    assert np.array_equal(go, oo), f"offsets differ at {np.flatnonzero(go != oo)[:8]}"
    assert np.array_equal(gk, ok)
    assert np.array_equal(gw, ow), f"words differ at {np.flatnonzero(gw != ow)[:8]}"
    if decode:
        y = hq.decode(plan, enc, ws, out_dtype=torch.float32)
        assert hq.status_sync(ws) == hq.OK
        st, oy = orc.decode(lat, SEED, alpha, ow, oo, ok, dithered=dithered, tile_base=tile_base, out_dtype=0,
                            rot=rot)
        assert st == 0
        g32 = host_bits(y).view(np.uint32)
        nz = (oy.view(np.uint32) & 0x7FFFFFFF) != 0
        assert np.array_equal(g32[nz], oy.view(np.uint32)[nz])
    return go


def assert_mixed(offsets, nominal_bps):
    cb = chunk_bits(offsets)
    over = int((cb >= first_unstaged_bits(nominal_bps)).sum())
    print(f"chunks: {len(cb)}, re-encoded by the placement: {over}", flush=True)
    assert 0 < over < len(cb), (over, len(cb))


@pytest.mark.parametrize("lat", [0, 1, 2, 3])
@pytest.mark.parametrize("dithered", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_staged_and_reencoded_chunks_equal_oracle(hq, orc, lat, dithered, dtype):
    print(f"staging: lattice {lat} dithered {dithered} {dtype}", flush=True)
    x = rows_input(67, 1024, 300 + 8 * lat + 2 * dithered + (dtype == torch.float32), dtype)  # 536 tiles
    alpha = float(np.float32(0.0042 / NU[lat]))  # per-row rates of about 1 to 6 bits per scalar
    plan = hq.Plan(lat, 0.5, SEED).set_compact_workspace().set_alpha(alpha)  # nominal 0.5 bps: slots for about 3 bps
    go = compare(hq, orc, plan, lat, alpha, x, dithered=dithered, tile_base=11 if dithered else 0)
    assert_mixed(go, 0.5)


def test_haar_reencoded_chunks_equal_oracle(hq, orc):
    x = rows_input(40, 1024, 320)
    alpha = float(np.float32(0.0042 / NU[2]))
    plan = hq.Plan(2, 0.5, SEED).set_compact_workspace().set_rotation(1).set_alpha(alpha)
    go = compare(hq, orc, plan, 2, alpha, x, dithered=True, tile_base=3, rot=1)
    assert_mixed(go, 0.5)


def test_more_than_8192_chunks_with_reencoded_chunks(hq, orc):
    """9375 chunks: the offsets of the placement come from the block scan."""
    x = rows_input(37500, 1024, 321)
    alpha = 0.0021
    plan = hq.Plan(3, 0.5, SEED).set_compact_workspace().set_alpha(alpha)
    go = compare(hq, orc, plan, 3, alpha, x, decode=False)
    assert_mixed(go, 0.5)


def test_append_with_reencoded_chunks(hq, orc):
    """A stream built by appending pieces (the first chunk of a piece starts
    inside a word of the existing stream) equals one encode of the whole."""
    x = rows_input(48, 1024, 322)  # 384 tiles
    alpha = float(np.float32(0.0042 / NU[1]))
    plan = hq.Plan(1, 0.5, SEED).set_compact_workspace().set_alpha(alpha)
    n_all = x.numel() // 128
    pieces = [37, 100, 1, 64, 182]
    xs = torch.split(x.view(n_all, 128).cuda(), pieces)
    words, offsets, k = hq.alloc_stream(plan, n_all)
    ws = plan.workspace(max(pieces))
    enc = hq.encode(plan, xs[0].contiguous(), ws, out=(words, offsets, k))
    for xp in xs[1:]:
        enc = hq.append(plan, enc, xp.contiguous(), ws)
    assert hq.status_sync(ws) == hq.OK
    gw, go, gk = stream_of(enc)
    st, ow, oo, ok = orc.encode(1, SEED, alpha, host_bits(x))
    assert st == 0
    assert np.array_equal(go, oo) and np.array_equal(gk, ok) and np.array_equal(gw, ow)
    assert_mixed(go, 0.5)


def test_compact_equals_full_slots_and_noalloc(hq):
    """The same plan with full-size slots (every chunk staged), with a compact
    workspace (some chunks re-encoded), and hq_encode_noalloc (full-size
    slots): the same streams."""
    x = rows_input(64, 1024, 323).cuda()
    n = x.numel() // 128
    full = hq.Plan(0, 0.5, SEED).set_alpha(0.0042)
    comp = hq.Plan(0, 0.5, SEED).set_compact_workspace().set_alpha(0.0042)
    assert comp.workspace_bytes(n) < full.workspace_bytes(n) / 3
    ws_f, ws_c = full.workspace(n), comp.workspace(n)
    a = stream_of(hq.encode(full, x, ws_f))
    b = stream_of(hq.encode(comp, x, ws_c))
    status = hq.status_block()
    c = stream_of(hq.encode_noalloc(comp, x, status, out=hq.alloc_stream(comp, n)))
    assert hq.status_sync(ws_f) == hq.OK and hq.status_sync(ws_c) == hq.OK and hq.status_sync(status) == hq.OK
    assert_mixed(b[1], 0.5)
    for p, q, r in zip(a, b, c):
        assert np.array_equal(p, q) and np.array_equal(p, r)


def test_reencoded_chunks_respect_the_capacity(hq):
    """Re-encoded chunks write no word at or past cap_words: with the buffer
    filled with a sentinel and cap_words below the stream's need, the encode
    reports HQ_ERR_CAPACITY and every word from cap_words on keeps the
    sentinel; with cap_words equal to the need, the words past it do."""
    x = rows_input(24, 1024, 324).cuda()  # 192 tiles, 6 chunks
    plan = hq.Plan(3, 0.5, SEED).set_compact_workspace().set_alpha(0.0021)
    n = x.numel() // 128
    ws = plan.workspace(n)
    ref = hq.encode(plan, x, ws)
    assert hq.status_sync(ws) == hq.OK
    need = ref.used_words()
    assert_mixed(stream_of(ref)[1], 0.5)
    sentinel = -0x21524111
    words, offsets, k = hq.alloc_stream(plan, n)
    for cap in (need - 1, need // 2, need // 3 + 5):
        words.fill_(sentinel)
        hq.encode(plan, x, ws, out=(words, offsets, k), cap_words=cap)
        assert hq.status_sync(ws) == hq.ERR_CAPACITY
        assert bool((words[cap:] == sentinel).all()), f"words past cap_words = {cap} written"
    words.fill_(sentinel)
    hq.encode(plan, x, ws, out=(words, offsets, k), cap_words=need)
    assert hq.status_sync(ws) == hq.OK
    assert torch.equal(words[:need], ref.words[:need]) and bool((words[need:] == sentinel).all())
