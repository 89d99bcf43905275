"""Python binding of libhq, the HyperQuant per-tile lattice codec for MI355X.

Argument marshalling only: every step of the codec runs in the HIP kernels of
``libhq.so`` (built by ``lattice_vq_entropy_amd/build.py``), called through its
C ABI (``include/hq.h``).  PyTorch supplies device memory and the stream.
The binding raises if the library is missing; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes as C
import os
import re

import torch  # noqa: F401  (loads the HIP runtime libhq links against)

HERE = os.path.dirname(os.path.abspath(__file__))
# HQ_SANITIZE=1 loads the host-sanitized build (build.py --sanitize)
LIB_PATH = os.path.join(HERE, "libhq_san.so" if os.environ.get("HQ_SANITIZE") == "1" else "libhq.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "hq.h")

Z, A2, D4, E8 = 0, 1, 2, 3
LATTICES = {"Z": Z, "A2": A2, "D4": D4, "E8": E8}
F32, BF16 = 0, 1
OK, ERR_ARG, ERR_NONFINITE, ERR_RANGE, ERR_CAPACITY, ERR_CORRUPT, ERR_DEVICE, ERR_NOALPHA = range(8)
TILE = 128


class HQError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        super().__init__(f"libhq: {status_str(code)} (code {code}){': ' + what if what else ''}")


_lib = None
_p, _u64, _u32, _f, _i = C.c_void_p, C.c_uint64, C.c_uint32, C.c_float, C.c_int

_SIGNATURES = {
    "hq_plan": (_i, [_i, _i, _f, _u64, C.POINTER(_p)]),
    "hq_plan_set_alpha": (_i, [_p, _f]),
    "hq_plan_get": (_i, [_p, C.POINTER(_f), C.POINTER(_f), C.POINTER(_f)]),
    "hq_plan_destroy": (None, [_p]),
    "hq_workspace_bytes": (C.c_size_t, [_p, _u64]),
    "hq_plan_set_compact_workspace": (_i, [_p, _i]),
    "hq_encode_bound_words": (_u64, [_p, _u64]),
    "hq_calibrate": (_i, [_p, _p, _i, _u64, _i, _u64, _p, _p, C.POINTER(_f), C.POINTER(C.c_double)]),
    "hq_encode": (_i, [_p, _p, _i, _u64, _p, _u64, _p, _p, _p, _p]),
    "hq_encode_noalloc": (_i, [_p, _p, _i, _u64, _p, _u64, _p, _p, _p, _p]),
    "hq_decode": (_i, [_p, _p, _u64, _p, _p, _u64, _p, _i, _p, _p]),
    "hq_kv_encode": (_i, [_p, _p, _i, _u64, _u64, _p, _u64, _p, _p, _p, _p]),
    "hq_kv_decode": (_i, [_p, _p, _u64, _p, _p, _u64, _u64, _p, _i, _p, _p]),
    "hq_kv_scores_workspace_bytes": (C.c_size_t, [_p, _u32, _u64, _u32]),
    "hq_kv_scores": (_i, [_p, _p, _u64, _p, _p, _u32, _u64, _u64, _p, _u32, _p, _p, _p]),
    "hq_gemv_workspace_bytes": (C.c_size_t, [_u64, _u64, _u32]),
    "hq_gemv": (_i, [_p, _p, _u64, _p, _p, _u64, _u64, _p, _u32, _p, _p, _p]),
    "hq_gemm_workspace_bytes": (C.c_size_t, [_u64, _u64, _u32]),
    "hq_gemm": (_i, [_p, _p, _u64, _p, _p, _u64, _u64, _p, _u32, _p, _p, _p]),
    "hq_append": (_i, [_p, _p, _i, _u64, _p, _u64, _p, _p, _u64, _p, _p]),
    "hq_kv_append": (_i, [_p, _p, _i, _u64, _u64, _p, _u64, _p, _p, _u64, _p, _p]),
    "hq_kv_attention_workspace_bytes": (C.c_size_t, [_u32, _u64, _u32]),
    "hq_kv_attention": (_i, [_p, _p, _u64, _p, _p, _u64, _p, _p, _u64, _p, _p, _u64, _u32, _u64, _p, _u32, C.c_float,
                             _p, _p, _p]),
    "hq_rotation_bytes": (C.c_size_t, []),
    "hq_plan_set_rotation": (_i, [_p, _i, _p, _p]),
    "hq_plan_get_rotation": (_i, [_p, C.POINTER(_i), _p]),
    "hq_side_bytes": (C.c_size_t, [_u64]),
    "hq_side_pack": (_i, [_p, _p, _u64, _p, _p, _p]),
    "hq_side_unpack": (_i, [_p, _u64, _p, _p, _p]),
    "hq_header_write": (_i, [_p, _i, _u64, _u64, _u64, _i, _p]),
    "hq_header_read": (_i, [_p, _p]),
    "hq_plan_from_header": (_i, [_p, C.POINTER(_p)]),
    "hq_status_sync": (_i, [_p, _p]),
    "hq_status_str": (C.c_char_p, [_i]),
}

HEADER_BYTES = 64


class HeaderInfo(C.Structure):
    """hq_header_info."""
    _fields_ = [("lattice", C.c_int), ("dithered", C.c_int), ("compact_side", C.c_int), ("tile", C.c_int),
                ("rotation", C.c_int), ("alpha", C.c_float), ("bps", C.c_float), ("seed", C.c_uint64), ("tile_base", C.c_uint64),
                ("n_tiles", C.c_uint64), ("total_bits", C.c_uint64)]


def header_functions() -> list[str]:
    """Names of the functions declared in include/hq.h."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(hq_\w+)\s*\(", text, re.M)))


def lib():
    """The loaded libhq (ctypes), raising when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python lattice_vq_entropy_amd/build.py` (no fallback exists)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_str(code: int) -> str:
    try:
        return lib().hq_status_str(code).decode()
    except Exception:  # library missing
        return f"status {code}"


def _check(code: int, what: str = ""):
    if code != OK:
        raise HQError(code, what)


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _dptr(t: torch.Tensor | None):
    if t is None:
        return C.c_void_p(0)
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("expected a contiguous device tensor")
    return C.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("input must be float32 or bfloat16")


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _need(t: torch.Tensor, nbytes: int, what: str):
    """Raise ValueError (instead of a device out-of-bounds access) when the
    buffer t holds fewer than nbytes bytes."""
    if _nbytes(t) < nbytes:
        raise ValueError(f"{what}: {_nbytes(t)} bytes, {nbytes} needed")


WS_HEADER_BYTES = 256  # the status word and counters at the start of every workspace


def _n_tiles(t: torch.Tensor) -> int:
    if t.numel() % TILE:
        raise ValueError("the number of elements must be a multiple of 128")
    return t.numel() // TILE


class Plan:
    """hq_plan: lattice, target bps, seed; alpha set by set_alpha or calibrate."""

    def __init__(self, lattice, bps: float, seed: int, tile: int = TILE):
        lat = LATTICES[lattice] if isinstance(lattice, str) else int(lattice)
        h = C.c_void_p(0)
        _check(lib().hq_plan(lat, tile, float(bps), int(seed), C.byref(h)), "hq_plan")
        self._h = h
        self.lattice, self.bps, self.seed = lat, float(bps), int(seed)
        self.rot = 0

    @classmethod
    def from_header(cls, header: bytes) -> "Plan":
        """hq_plan_from_header: the plan recorded in a 64-byte container header."""
        info = header_read(header)
        buf = C.create_string_buffer(bytes(header[:HEADER_BYTES]), HEADER_BYTES)
        h = C.c_void_p(0)
        _check(lib().hq_plan_from_header(buf, C.byref(h)), "hq_plan_from_header")
        self = cls.__new__(cls)
        self._h = h
        self.lattice, self.bps, self.seed = int(info.lattice), float(info.bps), int(info.seed)
        self.rot = 0
        return self

    def __del__(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.hq_plan_destroy(self._h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def set_rotation(self, kind: int, device="cuda", stream=None):
        """hq_plan_set_rotation: 0 the RHT, 1 the Haar rotation (its device copy is
        held by this object for the plan's life)."""
        buf = None
        if kind == 1:
            buf = torch.empty(int(lib().hq_rotation_bytes()), dtype=torch.uint8, device=device)
        _check(lib().hq_plan_set_rotation(self._h, int(kind), _dptr(buf), _stream(stream) if buf is not None
                                          else C.c_void_p(0)), "hq_plan_set_rotation")
        self._rot_buf = buf
        self.rot = int(kind)
        return self

    def rotation(self):
        """(kind, the Haar matrix of the plan's seed as fp32 [128, 128])."""
        import numpy as np
        kind = C.c_int(0)
        q = np.zeros(TILE * TILE, np.float32)
        _check(lib().hq_plan_get_rotation(self._h, C.byref(kind), q.ctypes.data_as(C.c_void_p)),
               "hq_plan_get_rotation")
        return kind.value, q.reshape(TILE, TILE)

    def set_compact_workspace(self, on: bool = True):
        """hq_plan_set_compact_workspace: staging slots sized from the plan's rate
        (a chunk that does not fit is encoded again by the placement)."""
        _check(lib().hq_plan_set_compact_workspace(self._h, int(bool(on))), "hq_plan_set_compact_workspace")
        return self

    def set_alpha(self, alpha: float):
        _check(lib().hq_plan_set_alpha(self._h, float(alpha)), "hq_plan_set_alpha")
        return self

    def get(self):
        a, ce, cd = C.c_float(0), C.c_float(0), C.c_float(0)
        _check(lib().hq_plan_get(self._h, C.byref(a), C.byref(ce), C.byref(cd)), "hq_plan_get")
        return a.value, ce.value, cd.value

    @property
    def alpha(self) -> float:
        return self.get()[0]

    def workspace_bytes(self, n_tiles: int) -> int:
        return int(lib().hq_workspace_bytes(self._h, n_tiles))

    def bound_words(self, n_tiles: int) -> int:
        return int(lib().hq_encode_bound_words(self._h, n_tiles))

    def decode_workspace_bytes(self, n_tiles: int) -> int:
        """Bytes a decode of n_tiles reads and writes in its workspace: the
        status header, and with the Haar rotation the rotated tiles."""
        return self.workspace_bytes(n_tiles) if self.rot else WS_HEADER_BYTES

    def workspace(self, n_tiles: int, device="cuda") -> torch.Tensor:
        """A zero-filled workspace (the zero fill is required once)."""
        return torch.zeros(self.workspace_bytes(n_tiles), dtype=torch.uint8, device=device)

    def calibrate(self, x: torch.Tensor, ws: torch.Tensor, dithered: bool = False, tile_base: int = 0,
                  stream=None):
        a, r = C.c_float(0), C.c_double(0)
        _check(lib().hq_calibrate(self._h, _dptr(x), _dtype_code(x), _n_tiles(x), int(dithered), tile_base,
                                  _dptr(ws), _stream(stream), C.byref(a), C.byref(r)), "hq_calibrate")
        return a.value, r.value


class Encoded:
    """Bitstream, per-tile bit offsets and Rice parameters of one encode."""

    def __init__(self, words, offsets, k, n_tiles, tile_base=0, dithered=False, storage=None):
        self.words, self.offsets, self.k = words, offsets, k
        self.n_tiles, self.tile_base, self.dithered = n_tiles, tile_base, dithered
        # the whole buffers (offsets and k may have room for appended tiles)
        self.storage = storage if storage is not None else (words, offsets, k)

    def total_bits(self) -> int:
        return int(self.offsets[-1].item())

    def used_words(self) -> int:
        return (self.total_bits() + 31) // 32


def alloc_stream(plan: Plan, n_tiles: int, device="cuda"):
    words = torch.empty(max(plan.bound_words(n_tiles), 1), dtype=torch.int32, device=device)
    offsets = torch.empty(n_tiles + 1, dtype=torch.int64, device=device)
    k = torch.empty(max(n_tiles, 1), dtype=torch.uint8, device=device)
    return words, offsets, k


def encode(plan: Plan, x: torch.Tensor, ws: torch.Tensor, out=None, dithered: bool = False,
           tile_base: int = 0, cap_words: int | None = None, stream=None) -> Encoded:
    """hq_encode / hq_kv_encode (asynchronous; check hq_status_sync for data errors)."""
    n = _n_tiles(x)
    words, offsets, k = out if out is not None else alloc_stream(plan, n, x.device)
    cap = _nbytes(words) // 4 if cap_words is None else cap_words
    if cap > _nbytes(words) // 4:
        raise ValueError(f"cap_words {cap} exceeds the {_nbytes(words) // 4} words of the stream buffer")
    _need(offsets, 8 * (n + 1), "offsets")
    _need(k, n, "k")
    _need(ws, plan.workspace_bytes(n), "workspace")
    if dithered:
        rc = lib().hq_kv_encode(plan.handle, _dptr(x), _dtype_code(x), n, tile_base, _dptr(words), cap,
                                _dptr(offsets), _dptr(k), _dptr(ws), _stream(stream))
    else:
        rc = lib().hq_encode(plan.handle, _dptr(x), _dtype_code(x), n, _dptr(words), cap, _dptr(offsets),
                             _dptr(k), _dptr(ws), _stream(stream))
    _check(rc, "encode")
    return Encoded(words, offsets[:n + 1], k[:max(n, 1)], n, tile_base, dithered, storage=(words, offsets, k))


NOALLOC_MAX_TILES = 32768  # HQ_NOALLOC_MAX_TILES
STATUS_BLOCK_BYTES = 256


def status_block(device="cuda") -> torch.Tensor:
    """A zero-filled status block for encode_noalloc (read with status_sync/check)."""
    return torch.zeros(STATUS_BLOCK_BYTES, dtype=torch.uint8, device=device)


def encode_noalloc(plan: Plan, x: torch.Tensor, status: torch.Tensor, out, cap_words: int | None = None,
                   stream=None) -> Encoded:
    """hq_encode_noalloc: hq_encode with the library's static device scratch as
    its workspace (nothing is allocated by the call; out = (words, offsets, k)
    must be given).  Data errors land in the status block."""
    n = _n_tiles(x)
    words, offsets, k = out
    cap = _nbytes(words) // 4 if cap_words is None else cap_words
    if cap > _nbytes(words) // 4:
        raise ValueError(f"cap_words {cap} exceeds the {_nbytes(words) // 4} words of the stream buffer")
    _need(offsets, 8 * (n + 1), "offsets")
    _need(k, n, "k")
    _need(status, STATUS_BLOCK_BYTES, "status block")
    rc = lib().hq_encode_noalloc(plan.handle, _dptr(x), _dtype_code(x), n, _dptr(words), cap, _dptr(offsets),
                                 _dptr(k), _dptr(status), _stream(stream))
    _check(rc, "encode_noalloc")
    return Encoded(words, offsets[:n + 1], k[:max(n, 1)], n, 0, False, storage=(words, offsets, k))


def append(plan: Plan, enc: Encoded, x: torch.Tensor, ws: torch.Tensor, stream=None) -> Encoded:
    """hq_append / hq_kv_append: the tiles of enc followed by those of x, in enc's buffers
    (allocate them with room, e.g. alloc_stream(plan, capacity_tiles), and encode into them)."""
    n, n_prev = _n_tiles(x), enc.n_tiles
    words, offsets, k = enc.storage
    if _nbytes(offsets) < 8 * (n_prev + n + 1) or _nbytes(k) < n_prev + n:
        raise ValueError("the stream's buffers have no room for the appended tiles")
    _need(ws, plan.workspace_bytes(n), "workspace")
    if enc.dithered:
        rc = lib().hq_kv_append(plan.handle, _dptr(x), _dtype_code(x), n, enc.tile_base + n_prev, _dptr(words),
                                words.numel(), _dptr(offsets), _dptr(k), n_prev, _dptr(ws), _stream(stream))
    else:
        rc = lib().hq_append(plan.handle, _dptr(x), _dtype_code(x), n, _dptr(words), words.numel(), _dptr(offsets),
                             _dptr(k), n_prev, _dptr(ws), _stream(stream))
    _check(rc, "append")
    m = n_prev + n
    return Encoded(words, offsets[:m + 1], k[:max(m, 1)], m, enc.tile_base, enc.dithered, storage=enc.storage)


def decode(plan: Plan, enc: Encoded, ws: torch.Tensor, out: torch.Tensor | None = None,
           out_dtype=torch.bfloat16, stream=None) -> torch.Tensor:
    """hq_decode / hq_kv_decode into a [n_tiles*128] tensor."""
    n = enc.n_tiles
    y = out if out is not None else torch.empty(n * TILE, dtype=out_dtype, device=enc.words.device)
    code = _dtype_code(y)
    if y.numel() < n * TILE:
        raise ValueError(f"output of {y.numel()} elements, {n * TILE} needed")
    _need(enc.offsets, 8 * (n + 1), "offsets")
    _need(enc.k, n, "k")
    _need(ws, plan.decode_workspace_bytes(n), "workspace")
    if enc.dithered:
        rc = lib().hq_kv_decode(plan.handle, _dptr(enc.words), _nbytes(enc.words) // 4, _dptr(enc.offsets),
                                _dptr(enc.k), n, enc.tile_base, _dptr(y), code, _dptr(ws), _stream(stream))
    else:
        rc = lib().hq_decode(plan.handle, _dptr(enc.words), _nbytes(enc.words) // 4, _dptr(enc.offsets), _dptr(enc.k),
                             n, _dptr(y), code, _dptr(ws), _stream(stream))
    _check(rc, "decode")
    return y


def kv_scores(plan: Plan, enc: Encoded, n_heads: int, tiles_per_head: int, q: torch.Tensor, qph: int,
              ws: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """hq_kv_scores: fp32 [n_heads*qph, tiles_per_head] = q . k_hat without materialising k_hat."""
    if q.dtype != torch.float32 or q.numel() != n_heads * qph * TILE:
        raise ValueError("q must be fp32 [n_heads*qph, 128]")
    need = int(lib().hq_kv_scores_workspace_bytes(plan.handle, n_heads, tiles_per_head, qph))
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace of {ws.numel() * ws.element_size()} bytes, {need} needed")
    s = out if out is not None else torch.empty(n_heads * qph, tiles_per_head, dtype=torch.float32,
                                                device=q.device)
    _need(s, 4 * n_heads * qph * tiles_per_head, "scores")
    _need(enc.offsets, 8 * (n_heads * tiles_per_head + 1), "offsets")
    rc = lib().hq_kv_scores(plan.handle, _dptr(enc.words), _nbytes(enc.words) // 4, _dptr(enc.offsets), _dptr(enc.k),
                            n_heads, tiles_per_head, enc.tile_base, _dptr(q), qph, _dptr(s), _dptr(ws),
                            _stream(stream))
    _check(rc, "kv_scores")
    return s


def gemv_workspace(rows: int, cols: int, nb: int = 1, device="cuda") -> torch.Tensor:
    """A zero-filled workspace for hq_gemv (the zero fill is required once)."""
    n = int(lib().hq_gemv_workspace_bytes(rows, cols, nb))
    return torch.zeros(n, dtype=torch.uint8, device=device)


def gemv(plan: Plan, enc: Encoded, rows: int, cols: int, x: torch.Tensor, ws: torch.Tensor,
         out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """hq_gemv: fp32 [nb, rows] = x W_hat^T for the compressed rows x cols matrix (x fp32 [nb, cols])."""
    if x.dtype != torch.float32 or not x.is_contiguous() or x.numel() % cols:
        raise ValueError("x must be contiguous fp32 [nb, cols]")
    if enc.dithered:
        raise ValueError("matrix-vector products take an undithered weight stream")
    nb = x.numel() // cols
    y = out if out is not None else torch.empty(nb, rows, dtype=torch.float32, device=x.device)
    _need(y, 4 * nb * rows, "y")
    _need(ws, int(lib().hq_gemv_workspace_bytes(rows, cols, nb)), "workspace")
    rc = lib().hq_gemv(plan.handle, _dptr(enc.words), _nbytes(enc.words) // 4, _dptr(enc.offsets), _dptr(enc.k),
                       rows, cols, _dptr(x), nb, _dptr(y), _dptr(ws), _stream(stream))
    _check(rc, "gemv")
    return y


def gemm_workspace(rows: int, cols: int, nb: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace for hq_gemm (the zero fill is required once)."""
    n = int(lib().hq_gemm_workspace_bytes(rows, cols, nb))
    return torch.zeros(n, dtype=torch.uint8, device=device)


def gemm(plan: Plan, enc: Encoded, rows: int, cols: int, x: torch.Tensor, ws: torch.Tensor,
         out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """hq_gemm: fp32 [nb, rows] = x W_hat^T on the matrix cores (x fp32 [nb, cols], nb <= 64)."""
    if x.dtype != torch.float32 or not x.is_contiguous() or x.numel() % cols:
        raise ValueError("x must be contiguous fp32 [nb, cols]")
    if enc.dithered:
        raise ValueError("matrix products take an undithered weight stream")
    nb = x.numel() // cols
    y = out if out is not None else torch.empty(nb, rows, dtype=torch.float32, device=x.device)
    _need(y, 4 * nb * rows, "y")
    _need(ws, int(lib().hq_gemm_workspace_bytes(rows, cols, nb)), "workspace")
    rc = lib().hq_gemm(plan.handle, _dptr(enc.words), _nbytes(enc.words) // 4, _dptr(enc.offsets), _dptr(enc.k),
                       rows, cols, _dptr(x), nb, _dptr(y), _dptr(ws), _stream(stream))
    _check(rc, "gemm")
    return y


def attention_workspace(n_heads: int, seq: int, qph: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace for hq_kv_attention (the zero fill is required once)."""
    n = int(lib().hq_kv_attention_workspace_bytes(n_heads, seq, qph))
    return torch.zeros(n, dtype=torch.uint8, device=device)


def kv_attention(plan_k: Plan, enc_k: Encoded, plan_v: Plan, enc_v: Encoded, n_heads: int, seq: int,
                 q: torch.Tensor, qph: int, scale: float, ws: torch.Tensor, out: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
    """hq_kv_attention: fp32 [n_heads*qph, 128] = softmax(scale q . k_hat) v_hat per query, without
    materialising k_hat or v_hat (both streams dithered, seq tiles per head)."""
    if q.dtype != torch.float32 or q.numel() != n_heads * qph * TILE:
        raise ValueError("q must be fp32 [n_heads*qph, 128]")
    if not (enc_k.dithered and enc_v.dithered):
        raise ValueError("attention takes dithered key and value streams")
    if enc_k.n_tiles < n_heads * seq or enc_v.n_tiles < n_heads * seq:
        raise ValueError("the streams hold fewer than n_heads*seq tiles")
    o = out if out is not None else torch.empty(n_heads * qph, TILE, dtype=torch.float32, device=q.device)
    _need(o, 4 * n_heads * qph * TILE, "out")
    _need(ws, int(lib().hq_kv_attention_workspace_bytes(n_heads, seq, qph)), "workspace")
    rc = lib().hq_kv_attention(plan_k.handle, _dptr(enc_k.words), _nbytes(enc_k.words) // 4, _dptr(enc_k.offsets),
                               _dptr(enc_k.k), enc_k.tile_base, plan_v.handle, _dptr(enc_v.words),
                               _nbytes(enc_v.words) // 4, _dptr(enc_v.offsets), _dptr(enc_v.k), enc_v.tile_base,
                               n_heads, seq, _dptr(q), qph, scale, _dptr(o), _dptr(ws), _stream(stream))
    _check(rc, "kv_attention")
    return o


def side_pack(enc: Encoded, ws: torch.Tensor, stream=None) -> torch.Tensor:
    """hq_side_pack: the compact side information of enc (uint8, 96 bytes per 32 tiles)."""
    n = enc.n_tiles
    side = torch.empty(max(int(lib().hq_side_bytes(n)), 16), dtype=torch.uint8, device=enc.words.device)
    _check(lib().hq_side_pack(_dptr(enc.offsets), _dptr(enc.k), n, _dptr(side), _dptr(ws), _stream(stream)),
           "side_pack")
    return side


def side_unpack(side: torch.Tensor, n_tiles: int, stream=None):
    """hq_side_unpack: (offsets int64 [n+1], k uint8 [n]) from compact side information."""
    offsets = torch.empty(n_tiles + 1, dtype=torch.int64, device=side.device)
    k = torch.empty(max(n_tiles, 1), dtype=torch.uint8, device=side.device)
    _check(lib().hq_side_unpack(_dptr(side), n_tiles, _dptr(offsets), _dptr(k), _stream(stream)), "side_unpack")
    return offsets, k


def header_write(plan: Plan, enc: Encoded, compact_side: bool = True) -> bytes:
    """hq_header_write for enc (synchronises to read its total bit count)."""
    buf = C.create_string_buffer(HEADER_BYTES)
    _check(lib().hq_header_write(plan.handle, int(enc.dithered), enc.tile_base, enc.n_tiles, enc.total_bits(),
                                 int(compact_side), buf), "header_write")
    return buf.raw


def header_read(header: bytes) -> HeaderInfo:
    if len(header) < HEADER_BYTES:
        raise ValueError("a container header is 64 bytes")
    info = HeaderInfo()
    buf = C.create_string_buffer(bytes(header[:HEADER_BYTES]), HEADER_BYTES)
    _check(lib().hq_header_read(buf, C.byref(info)), "header_read")
    return info


def save(plan: Plan, enc: Encoded, ws: torch.Tensor, compact_side: bool = True) -> bytes:
    """The stream as one self-describing byte string: the 64-byte header, the
    side information (compact, or uint64 offsets then uint8 k padded to 8
    bytes), then the used stream words."""
    head = header_write(plan, enc, compact_side)
    if compact_side:
        side = side_pack(enc, ws)
        check(ws)
        side_b = side[: int(lib().hq_side_bytes(enc.n_tiles))].cpu().numpy().tobytes()
    else:
        n = enc.n_tiles
        kb = enc.k[:n].cpu().numpy().tobytes()
        side_b = enc.offsets.cpu().numpy().tobytes() + kb + bytes(-len(kb) % 8)
    words = enc.words[: enc.used_words()].cpu().numpy().tobytes()
    return head + side_b + words


def load(data: bytes, device="cuda", extra_tiles: int = 0):
    """(plan, Encoded) from save()'s bytes; extra_tiles leaves room to append."""
    import numpy as np
    info = header_read(data)
    plan = Plan.from_header(data)
    if info.rotation:
        plan.set_rotation(1, device=device)
    n, total = int(info.n_tiles), int(info.total_bits)
    pos = HEADER_BYTES
    words = torch.zeros(max(plan.bound_words(n + extra_tiles), 1), dtype=torch.int32, device=device)
    offsets = torch.empty(n + extra_tiles + 1, dtype=torch.int64, device=device)
    k = torch.empty(max(n + extra_tiles, 1), dtype=torch.uint8, device=device)
    if info.compact_side:
        nb = int(lib().hq_side_bytes(n))
        side = torch.empty(max(nb, 16), dtype=torch.uint8, device=device)
        side[:nb].copy_(torch.from_numpy(np.frombuffer(data, np.uint8, nb, pos).copy()))
        o, kk = side_unpack(side, n)
        offsets[: n + 1].copy_(o)
        k[:n].copy_(kk[:n])
        pos += nb
    else:
        offsets[: n + 1].copy_(torch.from_numpy(np.frombuffer(data, np.int64, n + 1, pos).copy()))
        pos += 8 * (n + 1)
        k[:n].copy_(torch.from_numpy(np.frombuffer(data, np.uint8, n, pos).copy()))
        pos += n + (-n % 8)
    nw = (total + 31) // 32
    words[:nw].copy_(torch.from_numpy(np.frombuffer(data, np.int32, nw, pos).copy()))
    enc = Encoded(words, offsets[: n + 1], k[: max(n, 1)], n, int(info.tile_base), bool(info.dithered),
                  storage=(words, offsets, k))
    return plan, enc


def status_sync(ws: torch.Tensor, stream=None) -> int:
    """hq_status_sync: synchronise and return (and clear) the recorded data error."""
    return int(lib().hq_status_sync(_dptr(ws), _stream(stream)))


def check(ws: torch.Tensor, stream=None):
    _check(status_sync(ws, stream), "device status")
