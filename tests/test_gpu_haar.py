"""GPU parity of the Haar-rotation variant (hq_plan_set_rotation kind 1)
against the oracle (rotation 1): both compute u = fl32(t c_enc) with t the fp32
fma chain of Q[i][j] x_j in index order, so the words, offsets, Rice
parameters and the fp32/bf16 reconstructions (the chain of Q[j][i] u_j, times
alpha) are bit for bit equal.  The fused KV scores and attention with a Haar
plan are checked against the oracle's fp64 results within a-posteriori
rounding bounds (below)."""
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
    assert L.hq_kv_scores(p.handle, D, 8, D, D, 1, 1, 0, C.c_void_p(4100), 4, D, D, None) == hq.ERR_ARG  # q unaligned
    r = hq.Plan(3, 4.0, SEED).set_alpha(0.004)
    assert L.hq_kv_attention(p.handle, D, 8, D, D, 0, r.handle, D, 8, D, D, 0, 1, 1, D, 1, 1.0, D, D,
                             None) == hq.ERR_ARG  # rotation kinds differ
    assert L.hq_gemv(p.handle, D, 8, D, D, 2, 256, D, 1, D, D, None) == hq.ERR_ARG
    assert L.hq_gemm(p.handle, D, 8, D, D, 2, 256, D, 1, D, D, None) == hq.ERR_ARG
    a32 = float(np.float32(0.004))
    assert p.get()[1] == np.float32(1.0 / a32) and p.get()[2] == np.float32(a32)  # c_enc = 1/alpha, c_dec = alpha
    p.set_rotation(0)
    assert p.rotation()[0] == 0 and p.get()[1] == np.float32(1.0 / (a32 * math.sqrt(128.0)))


# ---------------------------------------------------------------------------
# Fused KV paths with the Haar rotation.  The queries are rotated by the same
# fp32 chain as the keys (q~_i = chain over j of Q[i][j] q_j), the scores are
# alpha_K <q~, u_hat_K>, and the attention's rotated-domain result
# a = alpha_V sum_j p_j u_hat_V,j / L is rotated back by the chain of
# Q[j][m] a_j.  The oracle forms Q q, the scores and the softmax in fp64 from
# the same fp32 Q and u_hat.  Bounds (u = 2^-24, first order, a-posteriori at
# the exact intermediate values; 1.25 times for the second-order terms):
#   * rotation chain of output i: u sum_k |S_ik|, S_ik = sum_{j<=k} Q[i][j] q_j;
#   * the score's dot product: fma chains of 8 within each of 16 lanes, a
#     4-level tree over the lanes, one multiply by alpha (as for the RHT);
#   * the attention's weights and sums: as for the RHT (module
#     test_gpu_attention), and the back rotation adds sum_k |Q[k][m]| e_k of
#     the rotated-domain errors e plus its own chain's u sum_k |T_mk|.
# ---------------------------------------------------------------------------
U = 2.0 ** -24


def chain_err(m: np.ndarray, x: np.ndarray):
    """y = m x in fp64 and, per output, u times the sum of the |partial sums|
    of the fp32 fma chain over the columns in index order."""
    part = np.cumsum(m.astype(np.float64) * x.astype(np.float64)[None, :], axis=1)
    return part[:, -1], U * np.abs(part).sum(axis=1)


def haar_encode_both(hq, orc, lat, alpha, x, tile_base, bps=2.0):
    st, w, o, kk = orc.encode(lat, SEED, alpha, host_bits(x), dithered=True, tile_base=tile_base, rot=1)
    assert st == 0
    plan = haar_plan(hq, lat, alpha, bps)
    ws = plan.workspace(x.numel() // 128)
    enc = hq.encode(plan, x.cuda(), ws, dithered=True, tile_base=tile_base)
    assert hq.status_sync(ws) == hq.OK
    torch.cuda.synchronize()
    assert np.array_equal(enc.offsets.cpu().numpy().view(np.uint64), o)
    assert np.array_equal(enc.k.cpu().numpy()[: enc.n_tiles], kk)
    assert np.array_equal(enc.words.cpu().numpy().view(np.uint32)[: w.size], w)
    return plan, enc, (w, o, kk)


def score_bound(orc, lat, alpha, stream, tile_base, n_heads, seq, q, qph):
    st, uh = orc.dequant_rotated_many(lat, SEED, *stream, n_heads * seq, dithered=True, tile_base=tile_base)
    assert st == 0
    Q = orc.haar(SEED)
    out = np.zeros((n_heads * qph, seq))
    for h in range(n_heads):
        u = uh[h * seq:(h + 1) * seq].astype(np.float64)
        for g in range(qph):
            qt, re = chain_err(Q, q[h * qph + g])
            part = np.cumsum((u * qt[None, :]).reshape(seq, 16, 8), axis=2)
            s = alpha * (u @ qt)
            d = alpha * (np.abs(u) @ re + U * np.abs(part).sum(axis=(1, 2)) + 4 * U * np.abs(part[:, :, -1]).sum(axis=1))
            out[h * qph + g] = 1.25 * (d + U * np.abs(s))
    return out


@pytest.mark.parametrize("lat,heads,seq,qph", [(3, 2, 1000, 4), (2, 1, 33, 16), (3, 3, 3, 5), (1, 1, 64, 1)])
def test_haar_kv_scores(hq, orc, lat, heads, seq, qph):
    """Fused scores with a Haar plan: 2 heads of 1000 keys (32 chunks, ragged),
    16 queries per head, more queries than keys per head (a workspace sized
    for the queries), one query."""
    from lattice_vq_entropy_amd import workloads as W
    k, _, q = W.c5("cpu", heads=heads, seq=seq, q_per_head=qph, seed=seq * 7 + qph)
    alpha = float(np.float32(0.9 * float(k.float().pow(2).mean().sqrt()) / 4.0))
    plan, enc, stream = haar_encode_both(hq, orc, lat, alpha, k, 4321)
    ws = torch.zeros(hq.lib().hq_kv_scores_workspace_bytes(plan.handle, heads, seq, qph), dtype=torch.uint8,
                     device="cuda")
    sc = hq.kv_scores(plan, enc, heads, seq, q.cuda(), qph, ws)
    assert hq.status_sync(ws) == hq.OK
    st, ref = orc.kv_scores(lat, SEED, alpha, *stream, heads, seq, 4321, q.numpy(), qph, rot=1)
    assert st == 0
    b = score_bound(orc, lat, alpha, stream, 4321, heads, seq, q.numpy(), qph)
    err = np.abs(sc.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= b), f"max err/bound {float((err / b).max()):.3f}"
    # the bound is far below the scores' spread (a wrong rotation or key would show)
    assert b.max() < 1e-4 * np.abs(ref).max()


def attn_bound(orc, lat, sk, kb, ak, sv, vb, av, n_heads, seq, q, qph, scale):
    st, uk = orc.dequant_rotated_many(lat, SEED, *sk, n_heads * seq, dithered=True, tile_base=kb)
    st2, uv = orc.dequant_rotated_many(lat, SEED, *sv, n_heads * seq, dithered=True, tile_base=vb)
    assert st == 0 and st2 == 0
    Q = orc.haar(SEED).astype(np.float64)
    G = -(-seq // 256)
    K = 132 + -(-G // 8)
    out = np.zeros((n_heads * qph, 128))
    for h in range(n_heads):
        ukh = uk[h * seq:(h + 1) * seq].astype(np.float64)
        uvh = uv[h * seq:(h + 1) * seq].astype(np.float64)
        for g in range(qph):
            qt, re = chain_err(Q, q[h * qph + g])
            part = np.cumsum((ukh * qt[None, :]).reshape(seq, 16, 8), axis=2)
            s = scale * ak * (ukh @ qt)
            d = abs(scale * ak) * (np.abs(ukh) @ re + U * np.abs(part).sum(axis=(1, 2)) +
                                   4 * U * np.abs(part[:, :, -1]).sum(axis=1)) + 2 * U * np.abs(s)
            M = s.max()
            p = np.exp(s - M)
            L = p.sum()
            eta = d + 8 * U + 3 * U * (M - s)
            eta[p < 2.0 ** -125] = 1.0
            a = (p @ uvh) / L
            e = (p * eta) @ np.abs(uvh - a[None, :]) / L + K * U * (p @ np.abs(uvh)) / L + (K + 2) * U * np.abs(a)
            _, rb = chain_err(Q.T, av * a)
            out[h * qph + g] = 1.25 * (av * (np.abs(Q).T @ e) + rb)
    return out


@pytest.mark.parametrize("lat,heads,seq,qph,scale", [
    (3, 2, 1000, 4, 128 ** -0.5),   # 4 groups, the last ragged
    (2, 1, 2061, 16, 128 ** -0.5),  # 9 groups, 4 query work-groups
    (3, 1, 300, 3, 0.0),            # scale 0: the mean of the values
    (3, 1, 400, 2, 4.0),            # sharp softmax
    (0, 2, 1, 3, 0.3),              # one key per head: that value
])
def test_haar_kv_attention(hq, orc, lat, heads, seq, qph, scale):
    from lattice_vq_entropy_amd import workloads as W
    k, v, q = W.c5("cpu", heads=heads, seq=seq, q_per_head=qph, seed=seq * 3 + qph)
    ak = float(np.float32(0.9 * float(k.float().pow(2).mean().sqrt()) / 4.0))
    av = float(np.float32(0.9 * float(v.float().pow(2).mean().sqrt()) / 4.0))
    pk, ek, sk = haar_encode_both(hq, orc, lat, ak, k, 0)
    pv, ev, sv = haar_encode_both(hq, orc, lat, av, v, heads * seq)
    ws = hq.attention_workspace(heads, seq, qph)
    out = hq.kv_attention(pk, ek, pv, ev, heads, seq, q.cuda(), qph, scale, ws)
    assert hq.status_sync(ws) == hq.OK
    out = out.cpu().numpy().astype(np.float64)
    st, ref = orc.kv_attention(lat, SEED, ak, sk, 0, av, sv, heads * seq, heads, seq, q.numpy(), qph, scale, rot=1)
    assert st == 0
    b = attn_bound(orc, lat, sk, 0, ak, sv, heads * seq, av, heads, seq, q.numpy(), qph, scale)
    err = np.abs(out - ref)
    assert np.all(err <= b), f"max err/bound {float((err / b).max()):.3f} at {np.unravel_index(np.argmax(err / b), b.shape)}"
    # and it is not the RHT's result for the same streams
    st, rr = orc.kv_attention(lat, SEED, ak, sk, 0, av, sv, heads * seq, heads, seq, q.numpy(), qph, scale, rot=0)
    assert np.abs(rr - ref).max() > 100 * b.max()


def test_haar_attention_bound_sees_a_missing_key(orc):
    """The Haar bound fails a result that leaves out the last key where the
    weights are spread (the oracle over the other keys, same records)."""
    from lattice_vq_entropy_amd import workloads as W
    lat, heads, seq, qph, scale = 3, 1, 900, 2, 0.004
    k, v, q = W.c5("cpu", heads=heads, seq=seq, q_per_head=qph, seed=4243)
    ak = float(np.float32(0.9 * float(k.float().pow(2).mean().sqrt()) / 4.0))
    av = float(np.float32(0.9 * float(v.float().pow(2).mean().sqrt()) / 4.0))
    st, w, o, kk = orc.encode(lat, SEED, ak, host_bits(k), dithered=True, tile_base=0, rot=1)
    st2, w2, o2, kk2 = orc.encode(lat, SEED, av, host_bits(v), dithered=True, tile_base=seq, rot=1)
    assert st == 0 and st2 == 0
    st, ref = orc.kv_attention(lat, SEED, ak, (w, o, kk), 0, av, (w2, o2, kk2), seq, heads, seq, q.numpy(), qph,
                               scale, rot=1)
    assert st == 0
    b = attn_bound(orc, lat, (w, o, kk), 0, ak, (w2, o2, kk2), seq, av, heads, seq, q.numpy(), qph, scale)
    st, ref2 = orc.kv_attention(lat, SEED, ak, (w, o[:seq], kk[:seq - 1]), 0, av, (w2, o2[:seq], kk2[:seq - 1]),
                                seq, heads, seq - 1, q.numpy(), qph, scale, rot=1)
    assert st == 0
    assert np.all((np.abs(ref2 - ref) > b).any(axis=1))
