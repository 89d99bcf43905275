"""GPU parity of the fused attention over compressed keys and values
(hq_kv_attention) against the oracle's fp64 softmax(scale q . k_hat) v_hat.

Both sides read the same streams: the oracle encodes K and V itself, and the
GPU's encode of the same inputs is checked bit-exact against that first.  Both
form the same fp32 u_hat (dequantised code minus dither).  The bound is a
first-order, a-posteriori one: it follows the fp32 operations the kernels
perform, in their order, and evaluates each rounding's worst case at the exact
(fp64) intermediate values of this input (u = 2^-24):

  * scores s_j = scale c_K <H D q, u_j>.  The rotated query q~ is the fp32
    butterfly of Methodology 1's H in Sylvester order, smallest stride first,
    the same additions as the oracle's fp32 transform (which the encode parity
    pins bit for bit), so its error against the exact H D q is known exactly
    and enters as |scale c_K <q~ - H D q, u_j>|.  The dot product is an fma
    chain over the 8 coordinates 8v..8v+7 of each of 16 lanes (error at most u
    times the sum of the |partial sums|) and a 4-level tree over the lanes (at
    most 4u sum_v |lane sum|), then two multiplies (2u |s_j|): d_j.
  * weights p_j = e^(s_j - M): a factor shared by all weights cancels in the
    normalised sum, so only e^(d_j) and the two hardware exponentials per
    weight count (2 ulp each plus 3u per unit of their arguments, which add up
    to M - s_j): eta_j = d_j + 8u + 3u (M - s_j); a weight that may flush to
    zero (p_j < 2^-125) counts with eta_j = 1.
  * the rotated-domain result a_k = sum_j p_j u_jk / L moves by
    sum_j p_j eta_j |u_jk - a_k| / L; the sums are K = 132 + ceil(G/8)
    roundings deep (in a group of 256 keys each thread adds coordinate k of
    half the keys, up to 128 fma terms, and the two halves are added; then
    ceil(G/8) fma terms over every 8th of the G groups and a 3-level tree over
    the 8 slices; the weight sums are shallower): K u sum_j p_j |u_jk| / L for
    the numerator, K u |a_k| for the denominator, 2u |a_k| for c_V / L and the
    product.  Each output of D H (c_V a) adds all 128 of these errors.
  * the inverse butterfly of c_V a adds, for output m, u times the sum of the
    |intermediate values| at every level that feed m.
The tests allow 1.25 times the sum, for the second-order terms.
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


def cone_sum(x: np.ndarray) -> np.ndarray:
    """For the butterfly of x (Sylvester order, strides 1..64): per output m,
    the sum over levels of |intermediate values| that output m depends on."""
    y = x.astype(np.float64).copy()
    out = np.zeros(128)
    for lvl in range(1, 8):
        h = 1 << (lvl - 1)
        y = y.reshape(-1, 2, h)
        y = np.stack([y[:, 0] + y[:, 1], y[:, 0] - y[:, 1]], axis=1).reshape(128)
        span = 1 << lvl  # after this level, output m depends on positions p = m mod span
        out += np.tile(np.abs(y).reshape(128 // span, span).sum(axis=0), 128 // span)
    return out


def bound(orc, lat, stream_k, kb, alpha_k, stream_v, vb, alpha_v, n_heads, seq, q, qph, scale):
    """Per output, the bound of the module docstring: [n_heads*qph, 128]."""
    st, uk = orc.dequant_rotated_many(lat, SEED, *stream_k, n_heads * seq, dithered=True, tile_base=kb)
    st2, uv = orc.dequant_rotated_many(lat, SEED, *stream_v, n_heads * seq, dithered=True, tile_base=vb)
    _, ck = orc.scales(alpha_k)
    _, cv = orc.scales(alpha_v)
    sg = orc.signs(SEED)
    hd = hadamard() * sg.astype(np.float64)[None, :]  # H D
    G = -(-seq // 256)
    K = 132 + -(-G // 8)
    out = np.zeros((n_heads * qph, 128))
    for h in range(n_heads):
        ukh = uk[h * seq:(h + 1) * seq].astype(np.float64)
        uvh = uv[h * seq:(h + 1) * seq].astype(np.float64)
        for g in range(qph):
            q32 = q[h * qph + g].astype(np.float32)
            qt = hd @ q32.astype(np.float64)
            qt32 = orc.fwht(sg * q32).astype(np.float64)
            prod = (ukh * qt32[None, :]).reshape(seq, 16, 8)
            part = np.cumsum(prod, axis=2)
            s = scale * ck * (ukh @ qt)
            d = abs(scale * ck) * (np.abs(ukh @ (qt32 - qt)) + U * np.abs(part).sum(axis=(1, 2)) +
                                   4 * U * np.abs(part[:, :, -1]).sum(axis=1)) + 2 * U * np.abs(s)
            M = s.max()
            p = np.exp(s - M)
            L = p.sum()
            eta = d + 8 * U + 3 * U * (M - s)
            eta[p < 2.0 ** -125] = 1.0
            a = (p @ uvh) / L
            e = (p * eta) @ np.abs(uvh - a[None, :]) / L + K * U * (p @ np.abs(uvh)) / L + (K + 2) * U * np.abs(a)
            out[h * qph + g] = 1.25 * cv * (e.sum() + U * cone_sum(a))
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
    ratio = err / b
    assert np.all(ratio <= 1.0), f"max err/bound {ratio.max():.3f} at {np.unravel_index(np.argmax(ratio), ratio.shape)}"
    return out, ref, dict(pk=pk, ek=ek, pv=pv, ev=ev, q=q, ws=ws, sv=sv, av=av)


@pytest.mark.parametrize("lat,bps,heads,seq,qph,scale", [
    (3, 1.7, 2, 1000, 4, 128 ** -0.5),     # 4 groups of 256 keys, the last ragged (232 keys, last chunk 8)
    (3, 1.7, 1, 256, 4, 128 ** -0.5),      # exactly one group
    (3, 1.7, 1, 257, 5, 128 ** -0.5),      # one key in the second group; a second work-group of 1 query
    (3, 1.7, 3, 31, 2, 128 ** -0.5),       # less than one chunk of 32 keys
    (3, 1.7, 2, 2061, 16, 128 ** -0.5),    # 9 groups, 16 queries per head (4 query work-groups)
    (3, 1.7, 1, 700, 3, 0.0),              # scale 0: the plain mean of the values
    (3, 1.7, 1, 900, 2, 0.004),            # mild scale: every key carries weight
    (3, 1.7, 1, 300, 1, -0.2),             # negative scale
    (3, 1.7, 1, 400, 4, 4.0),              # sharp softmax: weights underflow
    (2, 2.0, 2, 700, 3, 128 ** -0.5),      # D4 at 2 bps
    (1, 3.0, 1, 600, 4, 128 ** -0.5),      # A2
    (0, 3.0, 1, 600, 4, 128 ** -0.5),      # Z
])
def test_attention_matches_oracle(hq, orc, lat, bps, heads, seq, qph, scale):
    run_case(hq, orc, lat, bps, heads, seq, qph, scale, data_seed=seq * 31 + qph)


@pytest.mark.parametrize("case", range(6))
def test_attention_random_shapes(hq, orc, case):
    """Seeded random cases: any lattice, 1-3 heads, 1-1299 keys, 1-16 queries
    per head, scales from 0 to sharp and negative, random tile ids."""
    rng = np.random.default_rng(97000 + 2 * case)
    lat = int(rng.integers(0, 4))
    heads, seq, qph = int(rng.integers(1, 4)), int(rng.integers(1, 1300)), int(rng.integers(1, 17))
    scale = float(rng.choice([0.0, 0.004, 128 ** -0.5, 0.5, -0.3]))
    bps = float(rng.uniform(1.5, 4.0))
    run_case(hq, orc, lat, bps, heads, seq, qph, scale, data_seed=97000 + 2 * case,
             kb=int(rng.integers(0, 1 << 20)), vb=int(rng.integers(1 << 20, 1 << 21)))


@pytest.mark.parametrize("scale,first", [(0.0, False), (0.004, False), (0.004, True)])
def test_attention_bound_sees_a_missing_key(orc, scale, first):
    """The bound is tight enough to fail a result that leaves out one key (the
    last, or the first) where the weights are spread: the oracle over the
    other keys (same records, same tile ids) differs from the full result by
    more than the bound somewhere in every query."""
    from lattice_vq_entropy_amd import workloads as W
    lat, heads, seq, qph = 3, 1, 900, 2
    k, v, q = W.c5("cpu", heads=heads, seq=seq, q_per_head=qph, seed=4242)
    ak, av = alpha_for(lat, k, 1.7), alpha_for(lat, v, 1.7)
    st, w, o, kk = orc.encode(lat, SEED, ak, host_bits(k), dithered=True, tile_base=0)
    st2, w2, o2, kk2 = orc.encode(lat, SEED, av, host_bits(v), dithered=True, tile_base=seq)
    assert st == 0 and st2 == 0
    st, ref = orc.kv_attention(lat, SEED, ak, (w, o, kk), 0, av, (w2, o2, kk2), seq, heads, seq, q.numpy(), qph, scale)
    assert st == 0
    st, b = bound(orc, lat, (w, o, kk), 0, ak, (w2, o2, kk2), seq, av, heads, seq, q.numpy(), qph, scale)
    assert st == 0
    if first:  # keys 1..seq-1: their offsets and Rice parameters, tile ids from 1
        ks, vs, kb, vb = (w, o[1:], kk[1:]), (w2, o2[1:], kk2[1:]), 1, seq + 1
    else:      # keys 0..seq-2
        ks, vs, kb, vb = (w, o[:seq], kk[:seq - 1]), (w2, o2[:seq], kk2[:seq - 1]), 0, seq
    st, ref2 = orc.kv_attention(lat, SEED, ak, ks, kb, av, vs, vb, heads, seq - 1, q.numpy(), qph, scale)
    assert st == 0
    assert np.all((np.abs(ref2 - ref) > b).any(axis=1))


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
    assert np.all(err <= b)


def test_attention_1x8x131072_e8(hq, orc):
    """The long-context workload: K and V of 8 heads x 131072 tokens, E8 at
    1.7 bps with dither, 32 queries (4 per head); every head on the GPU and
    every head against the oracle, which encodes each head itself (tile ids
    as in the whole-layer streams)."""
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
    import os
    threads = max(1, min(16, os.cpu_count() or 1))
    for h in range(heads):
        print(f"attention 1x8x131072: head {h} against the oracle", flush=True)
        with orc.threads(threads):
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
        assert np.all(err <= b), (h, float((err / b).max()))
    del k, v, ek, ev
    torch.cuda.empty_cache()
