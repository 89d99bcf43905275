"""The serialized form of a stream (host side, no GPU): CRC-32, the 64-byte
container header and the compact side information, in the oracle and in
libhq's host calls.

The pages define no container; the layout is the library's own (documented in
include/hq.h).  The oracle writes it from that specification with its own
code; pins: the CRC-32 check value of the IEEE 802.3 / ISO-HDLC definition,
the documented byte positions, round trips through an independent big-integer
reader, and single-bit corruption detection."""
import ctypes as C
import struct

import numpy as np
import pytest


@pytest.fixture(scope="module")
def orc():
    from oracle import oracle as O
    O.lib()
    return O


@pytest.fixture(scope="module")
def hq():
    import lattice_vq_entropy_amd as hq
    hq.lib()
    return hq


def test_crc32_check_values(orc):
    # the catalogued check value of CRC-32 (IEEE 802.3, reflected 0x04C11DB7)
    assert orc.crc32(b"123456789") == 0xCBF43926
    assert orc.crc32(b"") == 0
    # one trailing zero byte changes the value; the complement convention
    # makes the CRC of data + its own little-endian CRC a constant residue
    d = b"HyperQuant"
    c = orc.crc32(d)
    assert orc.crc32(d + struct.pack("<I", c)) == 0x2144DF1C


def test_header_layout(orc):
    h = orc.header(3, 0x5EED0001, 0.0031, 4.0, True, True, 777, 131072, 67108864)
    assert len(h) == 64 and h[:4] == b"HQS1"
    ver, lat, flags, tile = struct.unpack_from("<HBBI", h, 4)
    assert (ver, lat, flags, tile) == (1, 3, 3, 128)
    alpha, bps, z0 = struct.unpack_from("<ffI", h, 12)
    assert alpha == np.float32(0.0031) and bps == 4.0 and z0 == 0
    assert struct.unpack_from("<QQQQ", h, 24) == (0x5EED0001, 777, 131072, 67108864)
    assert struct.unpack_from("<I", h, 56)[0] == 0
    assert struct.unpack_from("<I", h, 60)[0] == orc.crc32(h[:60])


@pytest.mark.parametrize("lat,dith,compact,alpha,bps", [(3, False, True, 0.0031, 4.0), (2, True, False, 0.25, 2.0),
                                                         (0, True, True, 1.5, 3.0), (1, False, False, 7e-4, 5.0)])
def test_library_header_matches_oracle(hq, orc, lat, dith, compact, alpha, bps):
    L = hq.lib()
    p = hq.Plan(lat, bps, 0xABCDEF0123).set_alpha(alpha)
    buf = C.create_string_buffer(64)
    assert L.hq_header_write(p.handle, int(dith), 99, 4097, 123456, int(compact), buf) == hq.OK
    assert buf.raw == orc.header(lat, 0xABCDEF0123, alpha, bps, dith, compact, 99, 4097, 123456)
    info = hq.header_read(buf.raw)
    assert (info.lattice, info.dithered, info.compact_side, info.tile) == (lat, int(dith), int(compact), 128)
    assert (info.seed, info.tile_base, info.n_tiles, info.total_bits) == (0xABCDEF0123, 99, 4097, 123456)
    assert info.alpha == np.float32(alpha) and info.bps == np.float32(bps)
    q = hq.Plan.from_header(buf.raw)
    assert q.get() == p.get() and q.lattice == lat and q.seed == 0xABCDEF0123


def test_header_corruption_is_detected(hq, orc):
    L = hq.lib()
    h = bytearray(orc.header(3, 1, 0.5, 4.0, False, True, 0, 10, 5000))
    info = hq.HeaderInfo()
    assert L.hq_header_read(C.create_string_buffer(bytes(h), 64), C.byref(info)) == hq.OK
    for byte in range(64):
        for bit in (0, 5):
            g = bytearray(h)
            g[byte] ^= 1 << bit
            assert L.hq_header_read(C.create_string_buffer(bytes(g), 64), C.byref(info)) == hq.ERR_CORRUPT
    p = hq.Plan(3, 4.0, 1)  # no alpha
    assert L.hq_header_write(p.handle, 0, 0, 1, 1, 1, C.create_string_buffer(64)) == hq.ERR_NOALPHA


def read_side(data: bytes, n: int):
    """An independent reader of the compact side information (big integers)."""
    offsets, ks = np.zeros(n + 1, np.uint64), np.zeros(n, np.uint8)
    for c in range((n + 31) // 32):
        rec = data[96 * c: 96 * (c + 1)]
        base = int.from_bytes(rec[0:8], "little")
        kbits = int.from_bytes(rec[72:92], "little")
        assert rec[92:96] == bytes(4)
        for j in range(32):
            t = 32 * c + j
            end = base + int.from_bytes(rec[8 + 2 * j: 10 + 2 * j], "little")
            if t < n:
                offsets[t + 1] = end
                ks[t] = (kbits >> (5 * j)) & 31
                if j == 0:
                    offsets[t] = base
            else:
                assert end == base and (kbits >> (5 * j)) & 31 == 0
    return offsets, ks


@pytest.mark.parametrize("n", [1, 31, 32, 33, 100])
def test_side_pack_round_trip(orc, n):
    rng = np.random.default_rng(n)
    lengths = rng.integers(128, 2100, size=n)
    offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(np.uint64) + 5
    k = rng.integers(0, 23, size=n).astype(np.uint8)
    st, side = orc.side_pack(offsets, k)
    assert st == 0 and len(side) == 96 * ((n + 31) // 32)
    o2, k2 = read_side(side, n)
    assert np.array_equal(o2, offsets) and np.array_equal(k2, k)


def test_side_pack_capacity(orc):
    offsets = np.array([0, 2000, 70000, 70100], np.uint64)  # the second record ends 70000 bits in
    st, _ = orc.side_pack(offsets, np.array([3, 4, 5], np.uint8))
    assert st == 4


def test_side_abi(hq):
    L = hq.lib()
    assert L.hq_side_bytes(0) == 0 and L.hq_side_bytes(1) == 96 and L.hq_side_bytes(33) == 192
    D = C.c_void_p(4096)
    assert L.hq_side_pack(None, D, 4, D, D, None) == hq.ERR_ARG
    assert L.hq_side_pack(D, D, 4, C.c_void_p(4104), D, None) == hq.ERR_ARG  # misaligned side
    assert L.hq_side_unpack(D, 4, None, D, None) == hq.ERR_ARG
    assert L.hq_side_pack(D, D, 0, D, D, None) == hq.OK


def test_header_rotation_flag(hq, orc):
    h = orc.header(2, 7, 0.25, 2.0, True, True, 0, 10, 5000, rot=1)
    assert h[7] == 1 | 2 | 4
    info = hq.header_read(h)
    assert info.rotation == 1 and info.dithered == 1 and info.compact_side == 1
    assert hq.header_read(orc.header(2, 7, 0.25, 2.0, True, True, 0, 10, 5000)).rotation == 0


@pytest.mark.parametrize("seed", [0x5EED0001, 1, 2 ** 63 + 5])
def test_library_haar_matrix_equals_oracle(hq, orc, seed):
    """Two implementations of the Haar recipe (Philox normals, Gram-Schmidt in
    double, fp32 rounding) give the same matrix bit for bit."""
    kind, q = hq.Plan("D4", 2.0, seed).rotation()
    assert kind == 0
    assert np.array_equal(q.view(np.uint32), orc.haar(seed).view(np.uint32))
