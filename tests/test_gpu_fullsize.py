"""Full-size GPU parity on the workload shapes: whole streams.

Each workload is calibrated, encoded and decoded whole on the GPU with the
calibration's alpha, exactly as the benchmark runs it.  The oracle, on up to
16 host threads, calibrates, encodes and decodes the same input bytes on its
own.  Bit-exact: the calibrated alpha (fp32) and rate, every offset, every
Rice parameter, every stream word (the unused bits of the last word are zero)
and every decoded element.  The fused long-context scores are compared with
the oracle's fp64 scores on every key within the fp32 bound.
"""
import math
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

SEED = 0x5EED0001
THREADS = max(1, min(16, os.cpu_count() or 1))


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


def say(label, what):
    print(f"[{label}] {what}", flush=True)


def whole_stream(hq, orc, lat, x2d: torch.Tensor, bps, dithered=False, tile_base=0, out_dtype=torch.bfloat16,
                 label="", rot=0, compact=False):
    """Calibrate, encode and decode x on the GPU and in the oracle; compare
    everything bit for bit.  rot: the Haar rotation instead of the RHT;
    compact: a compact workspace.  Returns (plan, Encoded, workspace)."""
    n = x2d.numel() // 128
    plan = hq.Plan(lat, bps, SEED)
    if rot:
        plan.set_rotation(rot)
    if compact:
        plan.set_compact_workspace()
    ws = plan.workspace(n)
    say(label, f"{n} tiles: GPU calibration")
    a_gpu, r_gpu = plan.calibrate(x2d, ws, dithered=dithered, tile_base=tile_base)
    xh = host_bits(x2d)
    say(label, f"oracle calibration on {THREADS} threads")
    with orc.threads(THREADS):
        st, a_orc, r_orc, _ = orc.calibrate(lat, SEED, bps, xh, dithered=dithered, tile_base=tile_base, rot=rot)
    assert st == 0
    assert np.float32(a_gpu) == np.float32(a_orc), (a_gpu, a_orc)
    assert r_gpu == r_orc, (r_gpu, r_orc)
    assert abs(r_gpu - bps) <= 0.002
    say(label, f"alpha {a_gpu:.9g} equal, rate {r_gpu:.5f}; GPU encode + decode")
    enc = hq.encode(plan, x2d, ws, dithered=dithered, tile_base=tile_base)
    assert hq.status_sync(ws) == hq.OK
    y = hq.decode(plan, enc, ws, out_dtype=out_dtype)
    assert hq.status_sync(ws) == hq.OK
    torch.cuda.synchronize()
    offsets = enc.offsets.cpu().numpy().view(np.uint64)
    total = int(offsets[-1])
    words = enc.words[: (total + 31) // 32].cpu().numpy().view(np.uint32)
    kk = enc.k[:n].cpu().numpy()
    code = 0 if out_dtype == torch.float32 else 1
    yh = y.cpu()
    yh = yh.numpy() if code == 0 else yh.view(torch.int16).numpy().view(np.uint16)
    del y
    say(label, "oracle encode + decode")
    with orc.threads(THREADS):
        st, ow, oo, ok = orc.encode(lat, SEED, a_orc, xh, dithered=dithered, tile_base=tile_base, rot=rot)
        assert st == 0
        st, oy = orc.decode(lat, SEED, a_orc, ow, oo, ok, dithered=dithered, tile_base=tile_base, out_dtype=code,
                            rot=rot)
        assert st == 0
    assert np.array_equal(offsets, oo), "offsets"
    assert np.array_equal(kk, ok), "Rice parameters"
    assert words.size == ow.size and np.array_equal(words, ow), "stream words"
    if total % 32:
        assert int(words[-1]) >> (total % 32) == 0
    if code == 1:  # compared as values: the sign of an exact zero is unspecified
        g = (yh.astype(np.uint32) << 16).view(np.float32)
        o = (oy.astype(np.uint32) << 16).view(np.float32)
    else:
        g, o = yh, oy
    assert np.array_equal(g, o), "reconstruction"
    say(label, f"whole stream equal: {total} bits, {words.size} words, {n} tiles")
    return plan, enc, ws


@pytest.mark.parametrize("bps", [3.0, 4.0, 5.0])
def test_weight_4096x4096_e8(hq, orc, bps):
    from lattice_vq_entropy_amd import workloads as W
    x = W.c2("cuda")
    whole_stream(hq, orc, 3, x, bps, label=f"4096x4096 E8 {bps}")


@pytest.mark.parametrize("lat,bps", [(1, 3.0), (1, 5.0), (0, 3.0), (0, 5.0), (3, 4.0)])
def test_weight_8192x28672(hq, orc, lat, bps):
    from lattice_vq_entropy_amd import workloads as W
    x = W.c4("cuda")
    whole_stream(hq, orc, lat, x, bps, label=f"8192x28672 lattice {lat} {bps}")
    del x
    torch.cuda.empty_cache()


def test_above_65536_chunks(hq, orc):
    """More than 64 blocks of 1024 chunks of 32 tiles (2.1 M tiles, E8 at
    4 bps): the block totals become prefixes in a launch of their own before
    the placement."""
    n = 65536 * 32 + 5000
    g = torch.Generator(device="cuda").manual_seed(65537)
    x = (torch.randn(n, 128, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    whole_stream(hq, orc, 3, x, 4.0, label="2.1M tiles E8 4")
    del x
    torch.cuda.empty_cache()


@pytest.mark.parametrize("which", ["K", "V"])
def test_kv_8x8x32768_d4_dithered(hq, orc, which):
    """K or V of one layer, D4 at 2 bps with subtractive dither."""
    from lattice_vq_entropy_amd import workloads as W
    k, v, q = W.c3("cuda")
    t = k if which == "K" else v
    del q
    whole_stream(hq, orc, 2, t, 2.0, dithered=True, tile_base=0, label=f"KV 8x8x32768 {which} D4 2")
    del k, v, t
    torch.cuda.empty_cache()


def test_kv_8x8x32768_k_haar(hq, orc):
    """The K tensor of one layer with the Haar rotation instead of the RHT
    (D4, 2 bps, dither): alpha, offsets, k, words and reconstruction of the
    whole stream equal the oracle's."""
    from lattice_vq_entropy_amd import workloads as W
    k, v, q = W.c3("cuda")
    del v, q
    whole_stream(hq, orc, 2, k, 2.0, dithered=True, tile_base=0, label="KV 8x8x32768 K D4 2 Haar", rot=1)
    del k
    torch.cuda.empty_cache()


def test_weight_4096x4096_e8_compact_workspace(hq, orc):
    """The headline weight (E8, 4 bps) with a compact workspace: the same
    whole-stream equality (no chunk there exceeds its rate-sized slot)."""
    from lattice_vq_entropy_amd import workloads as W
    whole_stream(hq, orc, 3, W.c2("cuda"), 4.0, label="4096x4096 E8 4 compact", compact=True)


def test_kv_8x8x32768_bias(hq):
    """Per-query bias of q . k_hat - q . k over all keys of one head, for 4096
    queries: the mean error per query is zero within its standard error."""
    from lattice_vq_entropy_amd import workloads as W
    k, v, q = W.c3("cuda")
    plan = hq.Plan(2, 2.0, SEED)
    ws = plan.workspace(k.numel() // 128)
    plan.calibrate(k, ws, dithered=True)
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
    k_hat, compared with the oracle's fp64 scores for every key and query,
    each within its fp32 bound."""
    from lattice_vq_entropy_amd import workloads as W
    k, v, q = W.c5("cuda")
    heads, seq, qph = 8, 131072, 4
    plan, enc, ws = whole_stream(hq, orc, 3, k, 1.7, dithered=True, label="KV 1x8x131072 K E8 1.7")
    sc = hq.kv_scores(plan, enc, heads, seq, q, qph, ws)
    assert hq.status_sync(ws) == hq.OK
    sc = sc.cpu().numpy().astype(np.float64)
    alpha = plan.alpha
    _, _, c_dec = plan.get()
    qh = q.cpu().numpy()
    # the GPU stream, equal to the oracle's word for word (whole_stream checked it)
    torch.cuda.synchronize()
    n = heads * seq
    offs = enc.offsets.cpu().numpy().view(np.uint64)[: n + 1]
    words = enc.words.cpu().numpy().view(np.uint32)[: (int(offs[n]) + 31) // 32]
    kk = enc.k.cpu().numpy()[:n]
    del k, v, enc, ws
    torch.cuda.empty_cache()
    say("KV 1x8x131072 K E8 1.7", "scores: the oracle on every key")
    st, osc = orc.kv_scores(3, SEED, alpha, words, offs, kk, heads, seq, 0, qh, qph)
    assert st == 0
    st, uh = orc.dequant_rotated_many(3, SEED, words, offs, kk, n, dithered=True)
    assert st == 0
    un = np.linalg.norm(uh.reshape(heads, seq, 128).astype(np.float64), axis=2)          # [heads, seq]
    qn = np.linalg.norm(qh.reshape(heads, qph, 128).astype(np.float64), axis=2)           # [heads, qph]
    bound = 1e-5 * c_dec * math.sqrt(128.0) * (qn[:, :, None] * un[:, None, :]).reshape(heads * qph, seq)
    err = np.abs(sc - osc.reshape(heads * qph, seq))
    assert np.all(err <= bound), f"max err/bound {float((err / bound).max()):.3f}"


def test_kv_1x8x131072_e8_values(hq, orc):
    """The long-context values, decoded plainly (tile ids after the keys')."""
    from lattice_vq_entropy_amd import workloads as W
    k, v, q = W.c5("cuda")
    del k, q
    whole_stream(hq, orc, 3, v, 1.7, dithered=True, tile_base=8 * 131072, label="KV 1x8x131072 V E8 1.7")
    del v
    torch.cuda.empty_cache()
