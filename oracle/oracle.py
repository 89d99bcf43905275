"""ctypes front end of the plain-C HyperQuant oracle (``hq_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  The product path
(``lattice_vq_entropy_amd``) never imports it and shares no code with it.

Every function is a thin marshalling wrapper: all arithmetic of the method
lives in ``hq_oracle.c``.  Source names used in comments are defined in
``hq_oracle.h``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "hq_oracle.c")
# ORC_SANITIZE=1: a separate AddressSanitizer + UndefinedBehaviorSanitizer
# build (load it with gcc's libasan preloaded, e.g.
#   ORC_SANITIZE=1 LD_PRELOAD=$(gcc -print-file-name=libasan.so) \
#   ASAN_OPTIONS=detect_leaks=0 python -m pytest tests -m "not gpu" -k oracle)
SANITIZE = os.environ.get("ORC_SANITIZE") == "1"
LIB = os.path.join(HERE, "liboracle_san.so" if SANITIZE else "liboracle.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]

Z, A2, D4, E8 = 0, 1, 2, 3
F32, BF16 = 0, 1
OK, ERR_ARG, ERR_NONFINITE, ERR_RANGE, ERR_CAPACITY, ERR_CORRUPT = 0, 1, 2, 3, 4, 5
LATTICES = {"Z": Z, "A2": A2, "D4": D4, "E8": E8}
DIM = {Z: 1, A2: 2, D4: 4, E8: 8}
RAW_BITS = {Z: 0, A2: 0, D4: 0, E8: 16}
TILE = 128
MAX_RECORD_BITS = {Z: 128 * 23, A2: 128 * 23, D4: 128 * 23, E8: 16 + 128 * 23}

# -O2 without -ffast-math and with contraction off: each fp32 operation is one
# IEEE binary32 operation in source order.
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11",
          "-D_GNU_SOURCE", "-Wall", "-Wextra", "-Wno-unused-parameter", "-fopenmp"]


def build(force: bool = False) -> str:
    """Compile liboracle.so next to its source (gcc)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, *(SAN_FLAGS if SANITIZE else []), "-o", tmp, SRC, "-lm"], check=True)
        os.replace(tmp, LIB)
    return LIB


_lib = None
_p = C.c_void_p
_u64 = C.c_uint64
_u32 = C.c_uint32
_f = C.c_float
_i = C.c_int


def lib():
    global _lib
    if _lib is None:
        build()
        L = C.CDLL(LIB)
        sig = {
            "orc_philox4x32_10": (None, [_p, _p, _p]),
            "orc_signs": (None, [_u64, _p]),
            "orc_fwht128": (None, [_p]),
            "orc_rht_forward": (None, [_p, _p, _f, _p]),
            "orc_nearest": (None, [_i, _p, _p]),
            "orc_embed": (None, [_i, _p, _p]),
            "orc_nearest_many": (None, [_i, _u64, _p, _p]),
            "orc_write_record_codes": (_u64, [_i, _p, _p, _u64, _p]),
            "orc_strip": (None, [_i, _p, _p, _p]),
            "orc_unstrip": (None, [_i, _p, _i, _p]),
            "orc_zigzag": (_u32, [C.c_int32]),
            "orc_unzigzag": (C.c_int32, [_u32]),
            "orc_rice_len": (_u64, [_p, _i, _i]),
            "orc_rice_kstar": (_i, [_p, _i]),
            "orc_dither": (None, [_i, _u64, _u64, _p]),
            "orc_scales": (None, [_f, _p, _p]),
            "orc_quantize_tile": (_i, [_i, _u64, _f, _p, _i, _u64, _p]),
            "orc_encode": (_i, [_i, _u64, _f, _p, _i, _u64, _i, _u64, _p, _u64, _p, _p]),
            "orc_total_bits": (_i, [_i, _u64, _f, _p, _i, _u64, _i, _u64, _p]),
            "orc_parse_tile": (_i, [_i, _p, _u64, _u64, _i, _p]),
            "orc_decode": (_i, [_i, _u64, _f, _p, _p, _p, _u64, _i, _u64, _p, _i]),
            "orc_dequant_rotated": (_i, [_i, _u64, _p, _u64, _u64, _i, _i, _u64, _p]),
            "orc_dequant_rotated_many": (_i, [_i, _u64, _p, _p, _p, _u64, _i, _u64, _p]),
            "orc_kv_scores": (_i, [_i, _u64, _f, _p, _p, _p, _u32, _u64, _u64, _p, _u32, _p]),
            "orc_calibrate": (_i, [_i, _u64, _f, _p, _i, _u64, _i, _u64, _p, _p, _p]),
            "orc_haar": (None, [_u64, _p]),
            "orc_kv_scores_r": (_i, [_i, _u64, _f, _i, _p, _p, _p, _u32, _u64, _u64, _p, _u32, _p]),
            "orc_kv_attention_r": (_i, [_i, _u64, _i, _f, _p, _p, _p, _u64, _f, _p, _p, _p, _u64, _u32, _u64, _p,
                                        _u32, _f, _p]),
            "orc_encode_r": (_i, [_i, _u64, _f, _i, _p, _i, _u64, _i, _u64, _p, _u64, _p, _p]),
            "orc_total_bits_r": (_i, [_i, _u64, _f, _i, _p, _i, _u64, _i, _u64, _p]),
            "orc_decode_r": (_i, [_i, _u64, _f, _i, _p, _p, _p, _u64, _i, _u64, _p, _i]),
            "orc_calibrate_r": (_i, [_i, _u64, _f, _i, _p, _i, _u64, _i, _u64, _p, _p, _p]),
            "orc_crc32": (C.c_uint32, [_p, C.c_size_t]),
            "orc_set_threads": (None, [_i]),
            "orc_get_threads": (_i, []),
            "orc_header_write": (None, [_i, _u64, _f, _f, _i, _i, _u64, _u64, _u64, _p]),
            "orc_header_write_r": (None, [_i, _u64, _f, _f, _i, _i, _i, _u64, _u64, _u64, _p]),
            "orc_side_pack": (_i, [_p, _p, _u64, _p]),
            "orc_gemv": (_i, [_i, _u64, _f, _p, _p, _p, _u64, _u64, _p, _u32, _p]),
            "orc_kv_attention": (_i, [_i, _u64, _f, _p, _p, _p, _u64, _f, _p, _p, _p, _u64, _u32, _u64, _p,
                                      _u32, _f, _p]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.c_void_p)


def _as_input(x: np.ndarray):
    """fp32 array, or bf16 bit patterns as uint16; returns (array, dtype code)."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError("oracle input must be float32 or bf16 bit patterns (uint16)")


# --------------------------------------------------------------------------- #
# primitives
# --------------------------------------------------------------------------- #
def philox(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.zeros(4, np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def signs(seed: int) -> np.ndarray:
    s = np.zeros(TILE, np.float32)
    lib().orc_signs(seed, _ptr(s))
    return s


def fwht(v: np.ndarray) -> np.ndarray:
    out = np.ascontiguousarray(v, dtype=np.float32).copy()
    lib().orc_fwht128(_ptr(out))
    return out


def rht_forward(x: np.ndarray, s: np.ndarray, c_enc: float) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    s = np.ascontiguousarray(s, dtype=np.float32)
    u = np.zeros(TILE, np.float32)
    lib().orc_rht_forward(_ptr(x), _ptr(s), c_enc, _ptr(u))
    return u


def nearest(lat: int, u: np.ndarray) -> np.ndarray:
    """Nearest points of a batch of vectors u[..., dim] (loops in C per vector)."""
    u = np.ascontiguousarray(u, dtype=np.float32).reshape(-1, DIM[lat])
    out = np.zeros(u.shape, np.int32)
    lib().orc_nearest_many(lat, u.shape[0], _ptr(u), _ptr(out))
    return out


def write_record_codes(lat: int, codes: np.ndarray, n_words: int = 96, off: int = 0):
    """(words, length, k) of one tile record written at bit ``off``."""
    codes = np.ascontiguousarray(codes, dtype=np.int32)
    assert codes.size == TILE
    words = np.zeros(n_words, np.uint32)
    k = C.c_int(0)
    L = lib().orc_write_record_codes(lat, _ptr(codes), _ptr(words), off, C.byref(k))
    return words, int(L), k.value


def embed(lat: int, x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.int32).reshape(-1, DIM[lat])
    out = np.zeros(x.shape, np.float32)
    L = lib()
    for r in range(x.shape[0]):
        L.orc_embed(lat, x[r].ctypes.data_as(C.c_void_p), out[r].ctypes.data_as(C.c_void_p))
    return out


def strip(lat: int, x: np.ndarray):
    x = np.ascontiguousarray(x, dtype=np.int32).reshape(-1, DIM[lat])
    sym = np.zeros(x.shape, np.int32)
    raw = np.zeros(x.shape[0], np.int32)
    L = lib()
    rb = C.c_int(0)
    for r in range(x.shape[0]):
        L.orc_strip(lat, x[r].ctypes.data_as(C.c_void_p), sym[r].ctypes.data_as(C.c_void_p), C.byref(rb))
        raw[r] = rb.value
    return sym, raw


def unstrip(lat: int, sym: np.ndarray, raw: np.ndarray) -> np.ndarray:
    sym = np.ascontiguousarray(sym, dtype=np.int32).reshape(-1, DIM[lat])
    out = np.zeros(sym.shape, np.int32)
    L = lib()
    for r in range(sym.shape[0]):
        L.orc_unstrip(lat, sym[r].ctypes.data_as(C.c_void_p), int(raw[r]), out[r].ctypes.data_as(C.c_void_p))
    return out


def zigzag(v: int) -> int:
    return int(lib().orc_zigzag(int(v)))


def unzigzag(m: int) -> int:
    return int(lib().orc_unzigzag(int(m)))


def rice_len(m: np.ndarray, k: int, raw_bits: int) -> int:
    m = np.ascontiguousarray(m, dtype=np.uint32)
    assert m.size == TILE
    return int(lib().orc_rice_len(_ptr(m), k, raw_bits))


def rice_kstar(m: np.ndarray, raw_bits: int) -> int:
    m = np.ascontiguousarray(m, dtype=np.uint32)
    assert m.size == TILE
    return int(lib().orc_rice_kstar(_ptr(m), raw_bits))


def dither(lat: int, seed: int, tile_id: int) -> np.ndarray:
    d = np.zeros(TILE, np.float32)
    lib().orc_dither(lat, seed, tile_id, _ptr(d))
    return d


def scales(alpha: float):
    ce, cd = C.c_float(0), C.c_float(0)
    lib().orc_scales(alpha, C.byref(ce), C.byref(cd))
    return ce.value, cd.value


def quantize_tile(lat: int, seed: int, alpha: float, x: np.ndarray, dithered=False, tile_id=0):
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.zeros(TILE, np.int32)
    st = lib().orc_quantize_tile(lat, seed, alpha, _ptr(x), int(dithered), tile_id, _ptr(codes))
    return st, codes


# --------------------------------------------------------------------------- #
# whole-tensor codec
# --------------------------------------------------------------------------- #
def bound_words(lat: int, n_tiles: int) -> int:
    return (n_tiles * MAX_RECORD_BITS[lat] + 31) // 32


def set_threads(n: int) -> None:
    """Host threads of the whole-tensor encode, decode, rate and calibration
    passes (1: the plain serial loops; the results do not depend on it)."""
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return int(lib().orc_get_threads())


class threads:
    """with threads(n): ... -- the oracle on n host threads inside the block."""

    def __init__(self, n: int):
        self.n, self.prev = int(n), None

    def __enter__(self):
        self.prev = get_threads()
        set_threads(self.n)
        return self

    def __exit__(self, *exc):
        set_threads(self.prev)
        return False


def encode(lat: int, seed: int, alpha: float, x: np.ndarray, dithered=False, tile_base=0,
           cap_words: int | None = None, rot: int = 0):
    """Returns (status, words, offsets, k).  x: fp32 or bf16 bits, size % 128 == 0.
    rot: 0 the RHT, 1 the Haar rotation."""
    xa, dt = _as_input(x)
    n_tiles = xa.size // TILE
    assert xa.size == n_tiles * TILE
    cap = bound_words(lat, n_tiles) if cap_words is None else cap_words
    words = np.zeros(max(cap, 1), np.uint32)
    offsets = np.zeros(n_tiles + 1, np.uint64)
    k = np.zeros(max(n_tiles, 1), np.uint8)
    st = lib().orc_encode_r(lat, seed, alpha, rot, _ptr(xa), dt, n_tiles, int(dithered), tile_base,
                            _ptr(words), cap, _ptr(offsets), _ptr(k))
    nwords = (int(offsets[-1]) + 31) // 32
    return st, words[:min(nwords, cap)], offsets, k[:n_tiles]


def total_bits(lat: int, seed: int, alpha: float, x: np.ndarray, dithered=False, tile_base=0, rot: int = 0):
    xa, dt = _as_input(x)
    n_tiles = xa.size // TILE
    bits = C.c_uint64(0)
    st = lib().orc_total_bits_r(lat, seed, alpha, rot, _ptr(xa), dt, n_tiles, int(dithered), tile_base,
                                C.byref(bits))
    return st, bits.value


def parse_tile(lat: int, words: np.ndarray, off: int, end: int, k: int):
    words = np.ascontiguousarray(words, dtype=np.uint32)
    codes = np.zeros(TILE, np.int32)
    st = lib().orc_parse_tile(lat, _ptr(words), off, end, k, _ptr(codes))
    return st, codes


def decode(lat: int, seed: int, alpha: float, words, offsets, k, dithered=False, tile_base=0,
           out_dtype=F32, rot: int = 0):
    words = np.ascontiguousarray(words, dtype=np.uint32)
    if words.size == 0:
        words = np.zeros(1, np.uint32)
    offsets = np.ascontiguousarray(offsets, dtype=np.uint64)
    k = np.ascontiguousarray(k, dtype=np.uint8)
    n_tiles = offsets.size - 1
    y = np.zeros(n_tiles * TILE, np.float32 if out_dtype == F32 else np.uint16)
    st = lib().orc_decode_r(lat, seed, alpha, rot, _ptr(words), _ptr(offsets),
                            _ptr(k if k.size else np.zeros(1, np.uint8)), n_tiles,
                            int(dithered), tile_base, _ptr(y), out_dtype)
    return st, y


def dequant_rotated(lat: int, seed: int, words, off: int, end: int, k: int, dithered=False,
                    tile_id=0):
    words = np.ascontiguousarray(words, dtype=np.uint32)
    uh = np.zeros(TILE, np.float32)
    st = lib().orc_dequant_rotated(lat, seed, _ptr(words), off, end, k, int(dithered), tile_id,
                                   _ptr(uh))
    return st, uh


def dequant_rotated_many(lat: int, seed: int, words, offsets, k, n: int, dithered=False, tile_base=0):
    """u_hat of tiles 0..n-1 of a stream, [n, 128] fp32 (zeros where a record does not parse)."""
    words = np.ascontiguousarray(words, dtype=np.uint32)
    offsets = np.ascontiguousarray(offsets, dtype=np.uint64)
    k = np.ascontiguousarray(k, dtype=np.uint8)
    assert offsets.size >= n + 1 and k.size >= n
    uh = np.zeros(n * TILE, np.float32)
    st = lib().orc_dequant_rotated_many(lat, seed, _ptr(words), _ptr(offsets), _ptr(k), n, int(dithered),
                                        tile_base, _ptr(uh))
    return st, uh.reshape(n, TILE)


def kv_scores(lat: int, seed: int, alpha: float, words, offsets, k, n_heads: int,
              tiles_per_head: int, tile_base: int, q: np.ndarray, qph: int, rot: int = 0):
    words = np.ascontiguousarray(words, dtype=np.uint32)
    offsets = np.ascontiguousarray(offsets, dtype=np.uint64)
    k = np.ascontiguousarray(k, dtype=np.uint8)
    q = np.ascontiguousarray(q, dtype=np.float32)
    assert q.size == n_heads * qph * TILE
    scores = np.zeros(n_heads * qph * tiles_per_head, np.float64)
    st = lib().orc_kv_scores_r(lat, seed, alpha, rot, _ptr(words), _ptr(offsets), _ptr(k), n_heads,
                               tiles_per_head, tile_base, _ptr(q), qph, _ptr(scores))
    return st, scores.reshape(n_heads * qph, tiles_per_head)


def gemv(lat: int, seed: int, alpha: float, words, offsets, k, rows: int, cols: int, x: np.ndarray):
    """y = W_hat x in fp64 for nb fp32 vectors x [nb, cols]; returns (status, y [nb, rows])."""
    words = np.ascontiguousarray(words, dtype=np.uint32)
    offsets = np.ascontiguousarray(offsets, dtype=np.uint64)
    k = np.ascontiguousarray(k, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, cols)
    nb = x.shape[0]
    y = np.zeros(nb * rows, np.float64)
    st = lib().orc_gemv(lat, seed, alpha, _ptr(words), _ptr(offsets), _ptr(k), rows, cols, _ptr(x), nb, _ptr(y))
    return st, y.reshape(nb, rows)


def kv_attention(lat: int, seed: int, alpha_k: float, kstream, k_tile_base: int, alpha_v: float, vstream,
                 v_tile_base: int, n_heads: int, seq: int, q: np.ndarray, qph: int, scale: float, rot: int = 0):
    """softmax(scale q . k_hat) v_hat per query in fp64; streams are (words, offsets, k).
    Returns (status, out [n_heads*qph, 128])."""
    kw, ko, kk = (np.ascontiguousarray(a, dtype=d) for a, d in zip(kstream, (np.uint32, np.uint64, np.uint8)))
    vw, vo, vk = (np.ascontiguousarray(a, dtype=d) for a, d in zip(vstream, (np.uint32, np.uint64, np.uint8)))
    q = np.ascontiguousarray(q, dtype=np.float32)
    assert q.size == n_heads * qph * TILE
    out = np.zeros(n_heads * qph * TILE, np.float64)
    st = lib().orc_kv_attention_r(lat, seed, rot, alpha_k, _ptr(kw), _ptr(ko), _ptr(kk), k_tile_base, alpha_v,
                                  _ptr(vw), _ptr(vo), _ptr(vk), v_tile_base, n_heads, seq, _ptr(q), qph, scale,
                                  _ptr(out))
    return st, out.reshape(n_heads * qph, TILE)


def calibrate(lat: int, seed: int, bps: float, x: np.ndarray, dithered=False, tile_base=0, rot: int = 0):
    xa, dt = _as_input(x)
    n_tiles = xa.size // TILE
    a, r, it = C.c_float(0), C.c_double(0), C.c_int(0)
    st = lib().orc_calibrate_r(lat, seed, bps, rot, _ptr(xa), dt, n_tiles, int(dithered), tile_base,
                               C.byref(a), C.byref(r), C.byref(it))
    return st, a.value, r.value, it.value


def haar(seed: int) -> np.ndarray:
    """The Haar rotation of a seed: fp32 [128, 128], u = Q x."""
    q = np.zeros(TILE * TILE, np.float32)
    lib().orc_haar(seed, _ptr(q))
    return q.reshape(TILE, TILE)


def crc32(data: bytes) -> int:
    buf = np.frombuffer(bytes(data), np.uint8).copy() if len(data) else np.zeros(1, np.uint8)
    return int(lib().orc_crc32(_ptr(buf), len(data)))


def header(lat: int, seed: int, alpha: float, bps: float, dithered: bool, compact: bool, tile_base: int,
           n_tiles: int, total_bits: int, rot: int = 0) -> bytes:
    out = np.zeros(64, np.uint8)
    lib().orc_header_write_r(lat, seed, alpha, bps, int(dithered), int(compact), rot, tile_base, n_tiles, total_bits,
                             _ptr(out))
    return out.tobytes()


def side_pack(offsets, k):
    """(status, bytes) of the compact side information of a stream's offsets [n+1] and k [n]."""
    offsets = np.ascontiguousarray(offsets, dtype=np.uint64)
    k = np.ascontiguousarray(k, dtype=np.uint8)
    n = offsets.size - 1
    out = np.zeros(max(96 * ((n + 31) // 32), 1), np.uint8)
    st = lib().orc_side_pack(_ptr(offsets), _ptr(k if k.size else np.zeros(1, np.uint8)), n, _ptr(out))
    return st, out[: 96 * ((n + 31) // 32)].tobytes()
