"""Host-side checks of the libhq C ABI (no GPU needed): the library loads,
exports every function include/hq.h declares, and validates its arguments on
the host before touching a device."""
import ctypes as C

import pytest


@pytest.fixture(scope="module")
def hq():
    import lattice_vq_entropy_amd as hq
    hq.lib()
    return hq


def test_every_declared_function_is_exported(hq):
    names = hq.header_functions()
    assert len(names) >= 14
    L = hq.lib()
    for n in names:
        assert hasattr(L, n), n


def test_plan_lifecycle_and_constants(hq):
    p = hq.Plan("E8", 4.0, 0x5EED0001)
    with pytest.raises(hq.HQError) as e:
        p.get()
    assert e.value.code == hq.ERR_NOALPHA
    p.set_alpha(0.0057)
    a, ce, cd = p.get()
    assert a == pytest.approx(0.0057, rel=1e-7)
    assert ce * a * 128 ** 0.5 == pytest.approx(1.0, rel=1e-6)
    assert cd / a * 128 ** 0.5 == pytest.approx(1.0, rel=1e-6)
    # c_enc/c_dec are the same fp32 constants the oracle derives
    from oracle import oracle as O
    assert (ce, cd) == O.scales(a)


def test_sizes(hq):
    p = hq.Plan("E8", 4.0, 1)
    assert p.bound_words(1) == (16 + 128 * 23 + 31) // 32
    assert p.bound_words(1000) == (1000 * (16 + 128 * 23) + 31) // 32
    assert hq.Plan("Z", 4.0, 1).bound_words(32) == 32 * 128 * 23 // 32
    assert p.workspace_bytes(1) >= 256 + 16
    assert p.workspace_bytes(4096) >= 256 + 128 * 16
    # full-size staging slots by default; a compact workspace follows the
    # plan's rate: under half the bf16 bytes of the tiles at 4 bps, full-size
    # slots from about 21 bps
    n = 131072
    full = p.workspace_bytes(n)
    assert full > 1.4 * 256 * n
    assert hq.Plan("E8", 1.0, 1).workspace_bytes(n) == full
    c = lambda bps: hq.Plan("E8", bps, 1).set_compact_workspace().workspace_bytes(n)
    assert c(4.0) < 0.5 * 256 * n
    assert c(1.0) < c(4.0) < c(8.0) < full
    assert c(22.0) == c(1e6) == full
    assert p.set_compact_workspace(False).workspace_bytes(n) == full
    assert L_compact_arg_error(hq, p)


def L_compact_arg_error(hq, p):
    return hq.lib().hq_plan_set_compact_workspace(p.handle, 2) == hq.ERR_ARG and \
        hq.lib().hq_plan_set_compact_workspace(None, 1) == hq.ERR_ARG


def test_argument_errors_are_synchronous(hq):
    L = hq.lib()
    h = C.c_void_p(0)
    assert L.hq_plan(7, 128, 4.0, 1, C.byref(h)) == hq.ERR_ARG
    assert L.hq_plan(3, 64, 4.0, 1, C.byref(h)) == hq.ERR_ARG
    assert L.hq_plan(3, 128, -1.0, 1, C.byref(h)) == hq.ERR_ARG
    p = hq.Plan("D4", 2.0, 1)
    assert L.hq_plan_set_alpha(p.handle, 0.0) == hq.ERR_ARG
    assert L.hq_plan_set_alpha(p.handle, float("nan")) == hq.ERR_ARG
    # no alpha yet
    assert L.hq_encode(p.handle, None, 1, 4, None, 0, None, None, None, None) == hq.ERR_NOALPHA
    p.set_alpha(0.5)
    # null workspace / pointers, bad dtype
    assert L.hq_encode(p.handle, None, 1, 4, None, 0, None, None, None, None) == hq.ERR_ARG
    assert L.hq_encode(p.handle, None, 5, 4, None, 0, None, None, C.c_void_p(256), None) == hq.ERR_ARG
    # stream words 16-byte aligned, offsets 8-byte aligned
    A = C.c_void_p(4096)
    assert L.hq_encode(p.handle, A, 1, 4, C.c_void_p(4100), 64, A, A, A, None) == hq.ERR_ARG
    assert L.hq_encode(p.handle, A, 1, 4, A, 64, C.c_void_p(4100), A, A, None) == hq.ERR_ARG
    assert L.hq_decode(p.handle, None, 0, None, None, 4, None, 0, None, None) == hq.ERR_ARG
    assert L.hq_kv_scores(p.handle, None, 0, None, None, 1, 1, 0, None, 17, None, None, None) == hq.ERR_ARG
    D = C.c_void_p(4096)
    assert L.hq_append(p.handle, D, 1, 4, D, 8, None, D, 2, D, None) == hq.ERR_ARG       # no offsets
    assert L.hq_kv_append(p.handle, D, 1, 4, 0, D, 8, D, None, 2, D, None) == hq.ERR_ARG  # no k
    assert L.hq_append(p.handle, D, 1, 0, D, 8, D, D, 2, D, None) == hq.OK              # nothing to append
    assert L.hq_status_sync(None, None) == hq.ERR_ARG
    # the allocation-free encode: size limit and status block checked on the host
    big = hq.NOALLOC_MAX_TILES + 1
    assert L.hq_encode_noalloc(p.handle, A, 1, big, A, 64, A, A, A, None) == hq.ERR_ARG
    assert L.hq_encode_noalloc(p.handle, A, 1, 4, A, 64, A, A, None, None) == hq.ERR_ARG
    assert L.hq_encode_noalloc(p.handle, A, 1, 4, A, 64, A, A, C.c_void_p(4100), None) == hq.ERR_ARG
    assert L.hq_encode_noalloc(None, A, 1, 4, A, 64, A, A, A, None) == hq.ERR_ARG
    assert hq.status_str(hq.ERR_CORRUPT) == "corrupt stream"
    # matrix-vector products: shape and batch limits, null and misaligned pointers
    D = C.c_void_p(4096)
    assert L.hq_gemv(p.handle, D, 8, D, D, 2, 200, D, 1, D, D, None) == hq.ERR_ARG    # cols % 128
    assert L.hq_gemv(p.handle, D, 8, D, D, 2, 256, D, 0, D, D, None) == hq.ERR_ARG    # nb = 0
    assert L.hq_gemv(p.handle, D, 8, D, D, 2, 256, D, 17, D, D, None) == hq.ERR_ARG   # nb > 16
    assert L.hq_gemv(p.handle, D, 8, D, D, 2, 256, None, 1, D, D, None) == hq.ERR_ARG
    assert L.hq_gemv(p.handle, D, 8, D, D, 2, 256, C.c_void_p(4100), 1, D, D, None) == hq.ERR_ARG
    assert L.hq_gemv(p.handle, D, 8, D, D, 0, 256, D, 1, D, D, None) == hq.OK         # no rows: nothing to do
    q = hq.Plan("E8", 4.0, 1)
    assert L.hq_gemv(q.handle, D, 8, D, D, 2, 256, D, 1, D, D, None) == hq.ERR_NOALPHA
    # workspace: header, the rotated vectors (256-byte aligned), one fp32 per tile and vector
    assert L.hq_gemv_workspace_bytes(3, 256, 2) == 256 + 2048 + 4 * 2 * 3 * 2
    # attention: both plans with alpha, same lattice and seed; qph 1..16; finite scale; pointers
    pv = hq.Plan("E8", 4.0, 1).set_alpha(0.5)
    pk = hq.Plan("E8", 2.0, 1).set_alpha(0.25)
    args = lambda pk_, pv_, n_heads=2, seq=300, qd=D, qph=4, scale=0.1, ws=D: (
        pk_.handle, D, 8, D, D, 0, pv_.handle, D, 8, D, D, 600, n_heads, seq, qd, qph, scale, D, ws, None)
    A = L.hq_kv_attention
    assert A(*args(pk, hq.Plan("E8", 4.0, 1))) == hq.ERR_NOALPHA
    assert A(*args(pk, hq.Plan("E8", 4.0, 2).set_alpha(0.5))) == hq.ERR_ARG       # another seed
    assert A(*args(pk, hq.Plan("D4", 4.0, 1).set_alpha(0.5))) == hq.ERR_ARG       # another lattice
    assert A(*args(pk, pv, qph=0)) == hq.ERR_ARG
    assert A(*args(pk, pv, qph=17)) == hq.ERR_ARG
    assert A(*args(pk, pv, scale=float("inf"))) == hq.ERR_ARG
    assert A(*args(pk, pv, scale=float("nan"))) == hq.ERR_ARG
    assert A(*args(pk, pv, qd=None)) == hq.ERR_ARG
    assert A(*args(pk, pv, seq=0)) == hq.ERR_ARG
    assert A(*args(pk, pv, ws=C.c_void_p(4104))) == hq.ERR_ARG                      # misaligned workspace
    assert A(*args(pk, pv, n_heads=0)) == hq.OK                                      # no heads: nothing to do
    # workspace: header, then per head, group of 256 keys and query the maximum, the sum and 128 values,
    # then (256-byte aligned) 128 floats per query for the dense rotation's queries and result
    al = lambda b: (b + 255) // 256 * 256
    # scores with the RHT: the codec workspace of the keys' tiles
    assert L.hq_kv_scores_workspace_bytes(pk.handle, 2, 300, 4) == pk.workspace_bytes(600)
    assert L.hq_kv_attention_workspace_bytes(2, 300, 4) == al(256 + 4 * 2 * 2 * 4 * 130) + 512 * 8
    assert L.hq_kv_attention_workspace_bytes(8, 131072, 4) == al(256 + 4 * 8 * 512 * 4 * 130) + 512 * 32
