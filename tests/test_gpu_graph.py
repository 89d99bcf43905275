"""Encodes captured in a HIP graph and launches of mixed sizes on one
workspace, through the C ABI.

A graph of hq_encode + hq_decode is replayed nine times over three inputs,
with eager encodes of a smaller and a larger tensor on the same workspace
between the replays: every replay must equal the eager encode and decode of
its input bit for bit (the codec records no memset, and nothing a launch
leaves in the workspace may leak into the next).  Launches of 4096, 5, 4096, 1 and 300 chunks in a
row on one workspace must each equal the oracle.
"""
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


def host_input(x):
    x = x.detach().contiguous().cpu()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16).reshape(-1)
    return x.numpy().reshape(-1)


def stream_of(enc):
    torch.cuda.synchronize()
    total = enc.total_bits()
    return (enc.words[: (total + 31) // 32].cpu().numpy().view(np.uint32).copy(),
            enc.offsets.cpu().numpy().view(np.uint64).copy(), enc.k[: enc.n_tiles].cpu().numpy().copy())


def same(a, b):
    return all(np.array_equal(p, q) for p, q in zip(a, b))


def test_graph_replays_equal_eager_with_other_encodes_between(hq):
    from lattice_vq_entropy_amd import workloads as W
    print("graph replays: E8 4 bps, 2048x4096 bf16 (2048 chunks), encode + decode, eager encodes between", flush=True)
    plan = hq.Plan(3, 4.0, SEED).set_alpha(0.0031)
    xs = [W.c2("cuda", rows=2048, cols=4096, seed=40 + i) for i in range(3)]
    small = W.c2("cuda", rows=24, cols=1024, seed=50)    # 6 chunks
    big = W.c2("cuda", rows=4096, cols=4096, seed=51)    # 4096 chunks
    n = xs[0].numel() // 128
    ws = plan.workspace(big.numel() // 128)
    refs, ref_ys = [], []
    for x in xs:
        e = hq.encode(plan, x, ws)
        refs.append(stream_of(e))
        ref_ys.append(hq.decode(plan, e, ws))
    ref_small = stream_of(hq.encode(plan, small, ws))
    ref_big = stream_of(hq.encode(plan, big, ws))
    assert hq.status_sync(ws) == hq.OK
    xin = xs[0].clone()
    out = hq.alloc_stream(plan, n)
    ybuf = torch.empty(n * 128, dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            enc = hq.encode(plan, xin, ws, out=out, stream=side)
            y = hq.decode(plan, enc, ws, out=ybuf, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(9):
        i = rep % 3
        xin.copy_(xs[i])
        g.replay()
        got = stream_of(enc)
        assert same(got, refs[i]), f"replay {rep} (input {i}) differs from the eager encode"
        assert torch.equal(y.view(torch.int16), ref_ys[i].view(torch.int16)), f"replay {rep}: decode differs"
        # eager work on the same workspace between replays: smaller and larger launches
        if rep % 2:
            assert same(stream_of(hq.encode(plan, small, ws)), ref_small)
        else:
            assert same(stream_of(hq.encode(plan, big, ws)), ref_big)
    assert hq.status_sync(ws) == hq.OK


def test_mixed_launch_sizes_on_one_workspace(hq, orc):
    """Launch sizes 4096, 5, 4096, 1, 300 chunks on one workspace: each stream
    equals the oracle's (what a larger launch left in the workspace past a
    smaller one's chunks is never read)."""
    from lattice_vq_entropy_amd import workloads as W
    plan = hq.Plan(2, 3.0, SEED).set_alpha(0.002)
    shapes = [(4096, 4096), (20, 1024), (4096, 4096), (1, 1024), (1200, 1024)]
    ws = plan.workspace(4096 * 4096 // 128)
    for i, (r, c) in enumerate(shapes):
        print(f"stale records: launch {i}, {r}x{c} bf16", flush=True)
        x = W.c2("cuda", rows=r, cols=c, seed=60 + i)
        got = stream_of(hq.encode(plan, x, ws))
        assert hq.status_sync(ws) == hq.OK
        st, ow, oo, ok = orc.encode(2, SEED, 0.002, host_input(x))
        assert st == 0
        assert same(got, (ow, oo, ok)), f"launch {i} ({r}x{c}) differs from the oracle"


def test_graph_of_single_chunk_encodes_and_appends(hq, orc):
    """Encodes of at most 32 tiles are one launch: a graph of an encode of 20
    tiles followed by two appends of 12 and 3 tiles (the appends start inside
    a word of the existing stream), replayed over three inputs, equals the
    oracle's encode of the 35 tiles every time."""
    plan = hq.Plan(1, 4.0, SEED).set_alpha(0.004)
    g = torch.Generator().manual_seed(77)
    xs = [(torch.randn(35, 128, generator=g) * 0.03).to(torch.bfloat16) for _ in range(3)]
    xin = xs[0].clone().cuda()
    words, offsets, k = hq.alloc_stream(plan, 35)
    ws = plan.workspace(20)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(gr, stream=side):
            enc = hq.encode(plan, xin[:20], ws, out=(words, offsets, k), stream=side)
            enc = hq.append(plan, enc, xin[20:32], ws, stream=side)
            enc = hq.append(plan, enc, xin[32:], ws, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(6):
        i = rep % 3
        xin.copy_(xs[i].cuda())
        gr.replay()
        got = stream_of(enc)
        st, ow, oo, ok = orc.encode(1, SEED, 0.004, host_input(xs[i]))
        assert st == 0
        assert same(got, (ow, oo, ok)), f"replay {rep} (input {i}) differs from the oracle"
    assert hq.status_sync(ws) == hq.OK
