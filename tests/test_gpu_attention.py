"""GPU parity of the fused attention over compressed keys and values
(hq_kv_attention) against the oracle's fp64 softmax(scale q . k_hat) v_hat.

Both sides read the same streams: the oracle encodes K and V itself, and the
GPU's encode of the same inputs is checked bit-exact against that first.  Both
form the same fp32 u_hat (dequantised code minus dither).  The bound, per
output coordinate of query (h, g), is derived from the fp32 operations the
kernels perform (u = 2^-24, first order):

  * scores: H D q is 7 butterfly levels (each entry off by <= 7u ||q||_1), the
    dot product with u_hat_j an 8-term fma chain and a 4-level lane tree (12
    roundings), then two multiplies by c_dec_K * scale:
      d_j <= |scale| c_K (7u ||q||_1 ||u_j||_1 + 12u sum_i |(H D q)_i| |u_ji|) + 3u |s_j|;
  * weights e^(s_j - M) are formed as e^(s_j - m_group) e^(m_group - M): the
    maxima are exact maxima of the computed scores, so score errors move a
    weight by a factor within e^(+-2 max d); each exponential is the hardware
    2^x of (argument * log2 e), 2 ulp (4u) plus 3u per unit of the argument,
    whose two arguments sum to M - s_j <= R, the score range; one multiply;
    weights below 2^-126 may flush to zero (at most seq of them):
      eta = 2 max_j d_j + 8u + 3u R + u + seq 2^-126;
  * a relative perturbation eta of every weight moves the normalised sum
    a_i = sum_j p_j u_ji / sum_j p_j by at most 2 eta max_j |u_ji|; the sums
    themselves are K = 24 + ceil(G/2) roundings deep (per lane 2 per chunk of
    up to 8 chunks, 2 row and 3 wave adds, the combine's product, ceil(G/2)
    sequential terms over the G groups of 256 keys, one add), for the
    numerator and the denominator alike: 2Ku max_j |u_ji|; times c_V / L: 2u;
  * the output D H (c_V a) is 7 butterfly levels: 7u c_V sum_k |a_k|, and
    each output sums 128 propagated coordinate errors.
  So |out - ref| <= c_V (2 eta + (2K + 9) u) sum_k max_j |u_V,jk|; the tests
allow 1.25 times that for the second-order terms.
"""
import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

SEED = 0x5EED0001
U = 2.0 ** -24
NU = {0: 1.0, 1: math.sqrt(2 * math.sqrt(3)), 2: 2 ** 0.25, 3: 2.0}


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


def alpha_for(lat, x: torch.Tensor, bps):
    sigma = float(x.float().pow(2).mean().sqrt())
    return float(np.float32(math.sqrt(2 * math.pi * math.e) * sigma / (NU[lat] * 2.0 ** bps)))


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


def bound(orc, lat, stream_k, kb, alpha_k, stream_v, vb, alpha_v, n_heads, seq, q, qph, scale):
    """Per query row, the bound of the module docstring (broadcast over the 128 outputs)."""
    st, uk = orc.dequant_rotated_many(lat, SEED, *stream_k, n_heads * seq, dithered=True, tile_base=kb)
    st2, uv = orc.dequant_rotated_many(lat, SEED, *stream_v, n_heads * seq, dithered=True, tile_base=vb)
    _, ck = orc.scales(alpha_k)
    _, cv = orc.scales(alpha_v)
    hd = hadamard() * orc.signs(SEED).astype(np.float64)[None, :]  # H D
    G = -(-seq // 256)
    K = 24 + -(-G // 2)
    out = np.zeros(n_heads * qph)
    for h in range(n_heads):
        ukh = uk[h * seq:(h + 1) * seq].astype(np.float64)
        uvh = uv[h * seq:(h + 1) * seq].astype(np.float64)
        vsum = np.abs(uvh).max(axis=0).sum()
        for g in range(qph):
            qr = q[h * qph + g].astype(np.float64)
            qt = hd @ qr
            s = scale * ck * (ukh @ qt)
            d = abs(scale) * ck * (7 * U * np.abs(qr).sum() * np.abs(ukh).sum(axis=1) +
                                   12 * U * (np.abs(ukh) @ np.abs(qt))) + 3 * U * np.abs(s)
            R = float(s.max() - s.min())
            eta = 2 * d.max() + 8 * U + 3 * U * R + U + seq * 2.0 ** -126
            out[h * qph + g] = 1.25 * cv * (2 * eta + (2 * K + 9) * U) * vsum
    return np.maximum(st, st2), out


def encode_both(hq, orc, lat, alpha, x, tile_base, bps):
    """The oracle's stream, and the GPU's encode of the same input checked bit-exact against it."""
    st, w, o, kk = orc.encode(lat, SEED, alpha, host_bits(x), dithered=True, tile_base=tile_base)
    assert st == 0
    plan = hq.Plan(lat, bps, SEED).set_alpha(alpha)
    ws = plan.workspace(x.numel() // 128)
    enc = hq.encode(plan, x.cuda(), ws, dithered=True, tile_base=tile_base)
    assert hq.status_sync(ws) == hq.OK
    torch.cuda.synchronize()
    n = enc.n_tiles
    gw = enc.words.cpu().numpy().view(np.uint32)[: (enc.total_bits() + 31) // 32]
    assert np.array_equal(enc.offsets.cpu().numpy().view(np.uint64), o)
    assert np.array_equal(enc.k.cpu().numpy()[:n], kk)
    assert np.array_equal(gw, w)
    return plan, enc, (w, o, kk)


def run_case(hq, orc, lat, bps, heads, seq, qph, scale, data_seed, kb=0, vb=None):
    from lattice_vq_entropy_amd import workloads as W
    k, v, q = W.c5("cpu", heads=heads, seq=seq, q_per_head=qph, seed=data_seed)
    vb = heads * seq if vb is None else vb
    ak, av = alpha_for(lat, k, bps), alpha_for(lat, v, bps)
    pk, ek, sk = encode_both(hq, orc, lat, ak, k, kb, bps)
    pv, ev, sv = encode_both(hq, orc, lat, av, v, vb, bps)
    ws = hq.attention_workspace(heads, seq, qph)
    out = hq.kv_attention(pk, ek, pv, ev, heads, seq, q.cuda(), qph, scale, ws)
    assert hq.status_sync(ws) == hq.OK
    out = out.cpu().numpy().astype(np.float64)
    st, ref = orc.kv_attention(lat, SEED, ak, sk, kb, av, sv, vb, heads, seq, q.numpy(), qph, scale)
    assert st == 0
    st, b = bound(orc, lat, sk, kb, ak, sv, vb, av, heads, seq, q.numpy(), qph, scale)
    assert st == 0
    assert np.isfinite(out).all()
    err = np.abs(out - ref)
    ratio = err / b[:, None]
    assert np.all(ratio <= 1.0), f"max err/bound {ratio.max():.3f} at {np.unravel_index(np.argmax(ratio), ratio.shape)}"
    return out, ref, dict(pk=pk, ek=ek, pv=pv, ev=ev, q=q, ws=ws, sv=sv, av=av)


@pytest.mark.parametrize("lat,bps,heads,seq,qph,scale", [
    (3, 1.7, 2, 1000, 4, 128 ** -0.5),     # 4 groups of 256 keys, the last ragged (232 keys, last chunk 8)
    (3, 1.7, 1, 256, 4, 128 ** -0.5),      # exactly one group
    (3, 1.7, 1, 257, 5, 128 ** -0.5),      # one key in the second group; a second work-group of 1 query
    (3, 1.7, 3, 31, 2, 128 ** -0.5),       # less than one chunk of 32 keys
    (3, 1.7, 2, 2061, 16, 128 ** -0.5),    # 9 groups, 16 queries per head (4 query work-groups)
    (3, 1.7, 1, 700, 3, 0.0),              # scale 0: the plain mean of the values
    (3, 1.7, 1, 300, 1, -0.2),             # negative scale
    (3, 1.7, 1, 400, 4, 4.0),              # sharp softmax: weights underflow
    (2, 2.0, 2, 700, 3, 128 ** -0.5),      # D4 at 2 bps
    (1, 3.0, 1, 600, 4, 128 ** -0.5),      # A2
    (0, 3.0, 1, 600, 4, 128 ** -0.5),      # Z
])
def test_attention_matches_oracle(hq, orc, lat, bps, heads, seq, qph, scale):
    run_case(hq, orc, lat, bps, heads, seq, qph, scale, data_seed=seq * 31 + qph)


def test_attention_one_key_is_that_value(hq, orc):
    """With one key the softmax weight is 1: the output is the value's
    reconstruction, which the oracle's decode gives independently."""
    out, ref, c = run_case(hq, orc, 3, 1.7, 2, 1, 3, 128 ** -0.5, data_seed=5)
    st, vh = orc.decode(3, SEED, c["av"], *c["sv"], dithered=True, tile_base=2, out_dtype=0)
    assert st == 0
    vh = vh.view(np.float32).reshape(2, 128).astype(np.float64)
    for h in range(2):
        assert np.allclose(ref[h * 3:(h + 1) * 3], vh[h][None, :], rtol=1e-6, atol=1e-7)
        assert np.allclose(out[h * 3:(h + 1) * 3], vh[h][None, :], rtol=1e-5, atol=1e-6)


def test_attention_tile_bases_and_determinism(hq, orc):
    """Keys and values at other tile ids (other dither streams), and two calls
    on one workspace give the same bits."""
    out, ref, c = run_case(hq, orc, 3, 1.7, 2, 333, 4, 128 ** -0.5, data_seed=8, kb=12345, vb=999999)
    again = hq.kv_attention(c["pk"], c["ek"], c["pv"], c["ev"], 2, 333, c["q"].cuda(), 4, 128 ** -0.5, c["ws"])
    assert hq.status_sync(c["ws"]) == hq.OK
    assert np.array_equal(again.cpu().numpy().astype(np.float64), out)


def test_attention_corrupt_key_record(hq, orc):
    """A key record whose Rice parameter is changed no longer parses: both sides
    count it as a zero vector and report a corrupt stream."""
    from lattice_vq_entropy_amd import workloads as W
    heads, seq, qph, scale = 1, 300, 2, 128 ** -0.5
    k, v, q = W.c5("cpu", heads=heads, seq=seq, q_per_head=qph, seed=77)
    ak, av = alpha_for(3, k, 1.7), alpha_for(3, v, 1.7)
    pk, ek, sk = encode_both(hq, orc, 3, ak, k, 0, 1.7)
    pv, ev, sv = encode_both(hq, orc, 3, av, v, seq, 1.7)
    w, o, kk = sk
    kk = kk.copy()
    kk[123] = (int(kk[123]) + 1) % 23
    ek.k[123] = int(kk[123])
    ws = hq.attention_workspace(heads, seq, qph)
    out = hq.kv_attention(pk, ek, pv, ev, heads, seq, q.cuda(), qph, scale, ws)
    assert hq.status_sync(ws) == hq.ERR_CORRUPT
    st, ref = orc.kv_attention(3, SEED, ak, (w, o, kk), 0, av, sv, seq, heads, seq, q.numpy(), qph, scale)
    assert st == 5
    st, b = bound(orc, 3, (w, o, kk), 0, ak, sv, seq, av, heads, seq, q.numpy(), qph, scale)
    err = np.abs(out.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= b[:, None])


def test_attention_1x8x131072_e8(hq, orc):
    """The long-context workload: K and V of 8 heads x 131072 tokens, E8 at
    1.7 bps with dither, 32 queries (4 per head); every head on the GPU, heads
    0 and 7 against the oracle, which encodes those heads itself (tile ids as
    in the whole-layer streams)."""
    from lattice_vq_entropy_amd import workloads as W
    heads, seq, qph, scale = 8, 131072, 4, 128 ** -0.5
    k, v, q = W.c5("cpu")
    ak, av = alpha_for(3, k, 1.7), alpha_for(3, v, 1.7)
    vb = heads * seq
    pk = hq.Plan(3, 1.7, SEED).set_alpha(ak)
    pv = hq.Plan(3, 1.7, SEED).set_alpha(av)
    ws = pk.workspace(heads * seq)
    ek = hq.encode(pk, k.cuda(), ws, dithered=True, tile_base=0)
    ev = hq.encode(pv, v.cuda(), ws, dithered=True, tile_base=vb)
    assert hq.status_sync(ws) == hq.OK
    aws = hq.attention_workspace(heads, seq, qph)
    out = hq.kv_attention(pk, ek, pv, ev, heads, seq, q.cuda(), qph, scale, aws)
    assert hq.status_sync(aws) == hq.OK
    out = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(out).all()
    kb16, vb16 = host_bits(k).reshape(heads, seq * 128), host_bits(v).reshape(heads, seq * 128)
    qn = q.numpy()
    for h in (0, 7):
        st, w, o, kk = orc.encode(3, SEED, ak, kb16[h], dithered=True, tile_base=h * seq)
        assert st == 0
        st, w2, o2, kk2 = orc.encode(3, SEED, av, vb16[h], dithered=True, tile_base=vb + h * seq)
        assert st == 0
        qh = qn[h * qph:(h + 1) * qph]
        st, ref = orc.kv_attention(3, SEED, ak, (w, o, kk), h * seq, av, (w2, o2, kk2), vb + h * seq, 1, seq, qh,
                                   qph, scale)
        assert st == 0
        st, b = bound(orc, 3, (w, o, kk), h * seq, ak, (w2, o2, kk2), vb + h * seq, av, 1, seq, qh, qph, scale)
        assert st == 0
        err = np.abs(out[h * qph:(h + 1) * qph] - ref)
        assert np.all(err <= b[:, None]), (h, float((err / b[:, None]).max()))
    del k, v, ek, ev
    torch.cuda.empty_cache()
