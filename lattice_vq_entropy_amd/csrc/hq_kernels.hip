// hq_kernels.hip -- HIP kernels of the HyperQuant per-tile codec for gfx950.
//
// encode_k  : RHT -> (dither) -> nearest point -> strip -> zigzag -> Rice k ->
//             tile lengths -> scan within the chunk -> LDS bit assembly -> the
//             chunk's bits staged in the workspace, its bit count recorded.
//             [HQ Methodology 1-4]
// blocksum_k, blockscan_k (large tensors only): bit counts of blocks of 1024
//             chunks, and their exclusive prefixes.
// place_k   : each chunk's global bit offset from the counts before it, then
//             its staged bits funnel-shifted into the stream with aligned
//             16-byte stores; per-tile offsets.  No work-group waits on
//             another: the stream-ordered launches are the only
//             synchronisation.
// decode_k  : per tile, remainders at fixed positions and the unary section by
//             a 16-lane popcount scan and in-word select, then unstrip,
//             (dither), inverse RHT, scale, bf16/fp32 stores; or, in score
//             mode, dot products of the dequantised rotated key with the head's
//             rotated queries (q . k_hat = c_dec <H D q, u_hat>).
//
// One work-group of 256 threads owns a chunk of kChunkTiles consecutive tiles
// and walks them in passes of 16 tiles (four per wave, one per DPP row).
#include "hq_device.h"
#include "hq_kernels.h"
#include "hq_ws.h"

namespace hq {

__device__ __forceinline__ void set_status(WsHeader* ws, int code) { atomicOr(&ws->status, 1u << code); }

// One lane's 8 input coordinates of one tile, as loaded (raw bits).
template <bool BF16> struct InVec;
template <> struct InVec<true> { uint4 w; };
template <> struct InVec<false> { uint4 w0, w1; };

// 16 bytes from global memory; NT: a non-temporal (streaming) load, for data
// read once per launch (measured: it leaves the L2 to what is reused).
template <bool NT>
__device__ __forceinline__ uint4 load16(const uint32_t* p) {
  if constexpr (NT)
    return make_uint4(__builtin_nontemporal_load(p), __builtin_nontemporal_load(p + 1), __builtin_nontemporal_load(p + 2),
                      __builtin_nontemporal_load(p + 3));
  else
    return *reinterpret_cast<const uint4*>(p);
}

// NT: the encode reads its input once (the length-only passes of the
// calibration re-read it, and keep the normal loads)
template <bool BF16, bool NT = false>
__device__ __forceinline__ InVec<BF16> load_in(const void* x, uint64_t t, int v, bool valid) {
  InVec<BF16> in;
  if constexpr (BF16) {
    in.w = make_uint4(0u, 0u, 0u, 0u);
    if (valid) in.w = load16<NT>(reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(x) + t * kTile + 8 * v));
  } else {
    in.w0 = in.w1 = make_uint4(0u, 0u, 0u, 0u);
    if (valid) {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(reinterpret_cast<const float*>(x) + t * kTile + 8 * v);
      in.w0 = load16<NT>(p);
      in.w1 = load16<NT>(p + 4);
    }
  }
  return in;
}

template <bool BF16>
__device__ __forceinline__ bool lane_nonfinite(const void* x, uint64_t t, int v) {
  bool nf = false;
  if constexpr (BF16) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(x) + t * kTile + 8 * v;
#pragma unroll
    for (int i = 0; i < 8; ++i) nf |= (p[i] & 0x7F80u) == 0x7F80u;
  } else {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(x) + t * kTile + 8 * v;
#pragma unroll
    for (int i = 0; i < 8; ++i) nf |= (p[i] & 0x7F800000u) == 0x7F800000u;
  }
  return nf;
}

// 16 bytes to global memory with non-temporal (streaming) stores: outputs
// that the next launch reads, so the writing launch leaves them out of its L2
// (measured: the launch that follows starts sooner).
__device__ __forceinline__ void store_nt4(uint32_t* p, uint32_t x, uint32_t y, uint32_t z, uint32_t w) {
  __builtin_nontemporal_store(x, p);
  __builtin_nontemporal_store(y, p + 1);
  __builtin_nontemporal_store(z, p + 2);
  __builtin_nontemporal_store(w, p + 3);
}

// OR a value of up to 64 bits into the LDS bit stream s at bit P (stream bit
// P is bit P % 32 of s[P / 32]).
__device__ __forceinline__ void lds_or64(uint32_t* s, uint32_t P, uint64_t val) {
  const uint32_t w = P >> 5, sh = P & 31;
  const uint64_t lo = val << sh;                      // words w, w + 1
  const uint32_t x2 = (uint32_t)((val >> 32) << sh >> 32);  // word w + 2
  atomicOr(&s[w], (uint32_t)lo);
  atomicOr(&s[w + 1], (uint32_t)(lo >> 32));
  if (x2) atomicOr(&s[w + 2], x2);
}

// ===========================================================================
// Encode
// ===========================================================================
// Per-lane constants of a plan: butterfly signs, the scale with the lane sign
// folded in, and the sign bits of D for the lane's 8 coordinates.
template <bool BF16>
struct LaneConst {
  FwhtSigns fs;
  float scale;
  uint32_t sm;  // lane_signs16 (bf16) or lane_signs32 (fp32)
  __device__ __forceinline__ LaneConst(const EncArgs& a, int v) {
    fs = fwht_signs(v);
    scale = fs.lane_sign * a.c_enc;
    sm = BF16 ? lane_signs16(a.sl16, v) : lane_signs32(a.sl32, v);
  }
  // the lane's 8 coordinates with the signs of D applied, as fp32
  __device__ __forceinline__ void apply(const InVec<BF16>& in, float xv[8]) const {
    if constexpr (BF16) {
      const uint32_t ww[4] = {in.w.x, in.w.y, in.w.z, in.w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t s = ww[i] ^ ((sm << i) & 0x80008000u);  // sign bits 15 and 31 of the pair
        xv[2 * i] = __builtin_bit_cast(float, s << 16);
        xv[2 * i + 1] = __builtin_bit_cast(float, s & 0xFFFF0000u);
      }
    } else {
      const uint32_t ww[8] = {in.w0.x, in.w0.y, in.w0.z, in.w0.w, in.w1.x, in.w1.y, in.w1.z, in.w1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) xv[i] = __builtin_bit_cast(float, ww[i] ^ ((sm << i) & 0x80000000u));
    }
  }
};

// One tile's symbols as seen by one lane, and the tile's Rice parameter and
// record length.
struct TileSyms {
  uint32_t w[8];  // 2 m + 1 for the zigzag symbols m of the lane's coordinates
  uint32_t k;     // Rice parameter of the tile
  uint32_t L;     // record length of the tile (bits); 0 for a tile past the end
  uint32_t U;     // unary bits of the lane's 8 symbols
  bool odd;       // E8 coset bit of the lane's vector
};

// RHT -> (dither) -> nearest point -> strip -> zigzag -> Rice k for tile t,
// held by the 16-lane row of the calling lane.  Every lane of the wave calls
// it (ballots).  A tile past the end has zero input and L = 0.
template <int L, bool DITHER, bool BF16, bool PRE>
__device__ __forceinline__ void tile_front(const EncArgs& a, const LaneConst<BF16>& lc, const InVec<BF16>& in,
                                           uint64_t t, bool valid, int v, int r, int grp, TileSyms& ts) {
  constexpr uint32_t RAW = Lat<L>::raw;
  float d[8];  // the dither first: its own nearest-point search then runs with only the input in flight
  if constexpr (DITHER) dither_lane<L>(a.key0, a.key1, a.tile_base + t, v, d);
  float u[8];
  if constexpr (PRE) {  // already rotated (the Haar matrix): only the scale
    const uint32_t ww[8] = {in.w0.x, in.w0.y, in.w0.z, in.w0.w, in.w1.x, in.w1.y, in.w1.z, in.w1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) u[i] = __builtin_bit_cast(float, ww[i]) * a.c_enc;
  } else {
    lc.apply(in, u);
    fwht_tile(u, lc.fs);
#pragma unroll
    for (int i = 0; i < 8; ++i) u[i] = u[i] * lc.scale;
  }
  if constexpr (DITHER) {
#pragma unroll
    for (int i = 0; i < 8; ++i) u[i] = u[i] + d[i];
  }
  // out of range or not finite: the largest |u| by IEEE maximum (NaN wins),
  // one compare per lane instead of eight
  float umax = __builtin_elementwise_maximum(__builtin_fabsf(u[0]), __builtin_fabsf(u[1]));
#pragma unroll
  for (int i = 2; i < 8; ++i) umax = __builtin_elementwise_maximum(umax, __builtin_fabsf(u[i]));
  const bool bad = !(umax < kRangeLimit);
  quantize_syms<L>(u, ts.w, ts.odd);
  const uint64_t bad_mask = __ballot(bad);
  if (bad_mask) {
    // a tile with a non-finite input or a coordinate beyond the range: record
    // the error and code it as zeros (the output is unspecified then)
    const bool tile_bad = ((bad_mask >> (grp * 16)) & 0xFFFFull) != 0;
    bool nf = false;
    if (tile_bad && valid) {
      if constexpr (PRE) nf = a.x0_bf16 ? lane_nonfinite<true>(a.x0, t, v) : lane_nonfinite<false>(a.x0, t, v);
      else nf = lane_nonfinite<BF16>(a.x, t, v);
    }
    const bool tile_nf = ((__ballot(nf) >> (grp * 16)) & 0xFFFFull) != 0;
    if (tile_bad) {
      if (r == 0 && valid) set_status(a.ws, tile_nf ? 2 : 3);
#pragma unroll
      for (int i = 0; i < 8; ++i) ts.w[i] = 1u;  // m = 0
      ts.odd = false;
    }
  }
  // Rice parameter: the smallest k with S(k) = sum ceil((m >> k)/2) <= 128
  // minimises the tile length.  From M = sum m: S(k) <= 128 once
  // M <= 2^(k+7) (at kA) and S(k) > 128 while M >= 3*2^(k+7), so the answer
  // is one of kA-2, kA-1, kA; S(k) = A_k - A_(k+1) with A_j = sum m >> j.
  // With w = 2m + 1: the row sum of w is 2M + 128, and m >> j = w >> (j + 1).
  const uint32_t S2 = row_sum_u32(((ts.w[0] + ts.w[1]) + (ts.w[2] + ts.w[3])) + ((ts.w[4] + ts.w[5]) + (ts.w[6] + ts.w[7])));
  // M > 128 iff 2M + 128 > 384; then ceil(log2 M) = 32 - clz(M - 1) = 31 - clz(2M - 2)
  const uint32_t kA = S2 <= 384u ? 0u : 24u - (uint32_t)__builtin_clz(S2 - 130u);
  const uint32_t c1 = (kA >= 2u ? kA - 2u : 0u) + 1u;
  uint32_t a0 = 0, a1 = 0, a2 = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a0 += ts.w[i] >> c1;
    a1 += ts.w[i] >> (c1 + 1u);
    a2 += ts.w[i] >> (c1 + 2u);
  }
  const uint32_t c = c1 - 1u;
  const uint32_t tot = row_sum_u32(a0 | (a1 << 10) | (a2 << 20));  // A_c <= 512
  const uint32_t A0 = tot & 1023u, A1 = (tot >> 10) & 1023u, A2 = tot >> 20;
  uint32_t Ak, ak;
  if (A0 - A1 <= 128u) { ts.k = c; Ak = A0; ak = a0; }
  else if (A1 - A2 <= 128u) { ts.k = c + 1u; Ak = A1; ak = a1; }
  else { ts.k = c + 2u; Ak = A2; ak = a2; }
  ts.U = ak + 8u;
  ts.L = valid ? RAW + 128u * (1u + ts.k) + Ak : 0u;
}

// Assemble one tile's record at local bit tb of the zero-filled LDS stream s.  Every lane of the wave calls it (ballot,
// permutes); only lanes of valid tiles write.  vaddr: byte address, for a lane permute, of the lane in the same row
// that holds vector r.
template <int L>
__device__ __forceinline__ void tile_pack(uint32_t* s, uint32_t tb, const TileSyms& ts, int v, int r, int vaddr,
                                          int grp, bool valid) {
  constexpr uint32_t RAW = Lat<L>::raw;
  const uint32_t k = ts.k, k1 = k + 1u;  // m >> j = w >> (j + 1); the low k bits of m are bits 1..k of w
  uint32_t raw16 = 0;
  if constexpr (RAW > 0) {
    // bit v of a tile's field is the coset bit of vector v, held by lane v(r):
    // lanes 4..7 and 12..15 of each row hold their vectors in reverse order,
    // so the bits of every high nibble are reversed (scalar work on the ballot)
    uint64_t bm = __ballot(ts.odd);
    uint64_t hi = bm & 0xF0F0F0F0F0F0F0F0ull;
    hi = ((hi >> 1) & 0x5555555555555555ull) | ((hi & 0x5555555555555555ull) << 1);
    hi = ((hi >> 2) & 0x3333333333333333ull) | ((hi & 0x3333333333333333ull) << 2);
    bm = (bm & 0x0F0F0F0F0F0F0F0Full) | hi;
    raw16 = (uint32_t)(bm >> (grp * 16)) & 0xFFFFu;
    // lane 0 of a row (vector 0) writes the field together with its remainders
    // when they fit one 64-bit value (1 <= k <= 6), else on its own
    if (valid && r == 0 && (k == 0 || k > 6)) lds_or64(s, tb, raw16);
  }
  // exclusive scan of the unary lengths in vector order
  const uint32_t Uv = (uint32_t)__builtin_amdgcn_ds_bpermute(vaddr, (int)ts.U);
  const uint32_t incl = row_scan_u32(Uv);
  const uint32_t excl = (uint32_t)__builtin_amdgcn_ds_bpermute(vaddr, (int)(incl - Uv));
  if (!valid) return;
  if (k != 0) {
    const uint32_t rpos = tb + RAW + __umul24(8u * (uint32_t)v, k);
    if (k <= 8) {
      uint32_t lo = __builtin_amdgcn_ubfe(ts.w[0], 1, k), hi = __builtin_amdgcn_ubfe(ts.w[4], 1, k);
#pragma unroll
      for (int j = 1; j < 4; ++j) {
        lo |= __builtin_amdgcn_ubfe(ts.w[j], 1, k) << (j * k);
        hi |= __builtin_amdgcn_ubfe(ts.w[4 + j], 1, k) << (j * k);
      }
      uint64_t val = (uint64_t)lo | ((uint64_t)hi << (4 * k));
      uint32_t pos = rpos;
      if (RAW > 0 && r == 0 && k <= 6) {  // rpos = tb + RAW for vector 0
        val = (val << RAW) | raw16;
        pos = tb;
      }
      lds_or64(s, pos, val);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) lds_or64(s, rpos + j * k, __builtin_amdgcn_ubfe(ts.w[j], 1, k));
    }
  }
  const uint32_t upos = tb + RAW + 128u * k + excl;
  if (ts.U <= 64u) {
    // built from the last code back: V_j = ((V_(j+1) << 1) | 1) << q_j
    uint64_t msk = 1ull << (ts.w[7] >> k1);
#pragma unroll
    for (int j = 6; j >= 0; --j) {
      uint64_t t;
      asm("v_lshl_add_u64 %0, %1, 1, 1" : "=v"(t) : "v"(msk));  // (msk << 1) + 1 in one instruction
      msk = t << (ts.w[j] >> k1);
    }
    lds_or64(s, upos, msk);
  } else {
    uint32_t pos = upos;
    for (int j = 0; j < 8; ++j) {
      pos += ts.w[j] >> k1;
      atomicOr(&s[pos >> 5], 1u << (pos & 31));
      pos += 1;
    }
  }
}

// Sum of a 32-bit value over the 64 lanes; every lane receives it.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
  x = row_sum_u32(x);
  return __builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16) + __builtin_amdgcn_readlane(x, 32) +
         __builtin_amdgcn_readlane(x, 48);
}

// One chunk's records assembled in LDS by the whole work-group (256 threads):
// per pass of 16 tiles, front, tile lengths, offsets within the chunk,
// packing into the zero-filled s_stage.  Per tile slot: s_lo the chunk-local
// bit offset, s_k the Rice parameter.  Returns the chunk's bit count
// (work-group uniform); s_stage is complete when it returns.  NT: the input is
// read once per launch (non-temporal loads).
template <int L, bool DITHER, int IN, bool NT>
__device__ __forceinline__ uint32_t pack_chunk(const EncArgs& a, uint32_t chunk, uint32_t* s_stage, uint32_t* s_len,
                                               uint32_t* s_lo, uint32_t* s_k) {
  constexpr bool BF16 = IN == 1, PRE = IN == 2;  // input: fp32, bf16, or fp32 already rotated
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, grp = lane >> 4, r = lane & 15;
  const int v = lane_vector(r);
  const int pslot = wv * 4 + grp;
  const LaneConst<BF16> lc(a, v);
  const uint64_t t_first = (uint64_t)chunk * kChunkTiles;
  InVec<BF16> in[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const uint64_t t = t_first + p * 16 + pslot;
    in[p] = load_in<BF16, NT>(a.x, t, v, t < a.n_tiles);
  }
  for (int i = tid; i < kSlotWords / 4; i += 256) reinterpret_cast<uint4*>(s_stage)[i] = make_uint4(0u, 0u, 0u, 0u);
  // lane permute addresses: the row's lane of slot pslot, and of vector r
  const int paddr = ((lane & ~15) | pslot) << 2, vaddr = ((lane & ~15) | v) << 2;
  uint32_t base = 0;  // wave-uniform bit offset of the current pass
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int slot = p * 16 + pslot;
    const uint64_t t = t_first + slot;
    const bool valid = t < a.n_tiles;
    TileSyms ts;
    tile_front<L, DITHER, BF16, PRE>(a, lc, in[p], t, valid, v, r, grp, ts);
    if (r == 0) {
      s_len[slot] = ts.L;
      s_k[slot] = ts.k;
    }
    __syncthreads();
    // offsets within the pass: every row scans the pass's 16 lengths
    const uint32_t len = s_len[p * 16 + r];
    const uint32_t incl = row_scan_u32(len);
    const uint32_t tb = base + (uint32_t)__builtin_amdgcn_ds_bpermute(paddr, (int)(incl - len));
    if (r == 0) s_lo[slot] = tb;
    base += __builtin_amdgcn_readlane(incl, 15);
    tile_pack<L>(s_stage, tb, ts, v, r, vaddr, grp, valid);
  }
  __syncthreads();
  return base;  // >= 256: every chunk holds a tile
}

// Placement (step 3): chunks per work-group (one per wave), and the chunk
// count up to which each work-group sums the counts before its own.
constexpr uint32_t kSelfScanChunks = 8192;
constexpr uint32_t kPlaceChunks = 4;

// Stream words of one chunk from its bits in LDS, by the whole work-group:
// the chunk's bits go to stream bits [E, E + A) with a funnel shift, stream
// word first + i (i < nw) = (s[i] : s[i - 1]) >> (32 - sh), s[-1] holding the
// 32 stream bits before the chunk, in aligned 16-byte groups: thread q writes
// stream words g .. g + 3 with g = first - al + 4 q, i.e. i = li .. li + 3,
// li = 4 q - al, from s[li - 1 .. li + 3] (li - 1 >= -4: s has 4 words before
// it; li + 3 <= nw + 2 <= 2963).  The last chunk also writes its partial last
// word; the others leave it to the chunk after them.
__device__ __forceinline__ void put_chunk_words(uint32_t* words, uint64_t cap_words, const uint32_t* s, uint64_t E,
                                                uint32_t A, bool last, uint32_t tid) {
  const uint64_t E1 = E + A, first = E >> 5;
  const uint32_t sh = (uint32_t)(E & 31);
  const uint64_t endw = last ? (E1 + 31) >> 5 : E1 >> 5;
  const uint64_t stop = endw < cap_words ? endw : cap_words;
  const uint32_t nw = stop > first ? (uint32_t)(stop - first) : 0u;
  const uint32_t al = (uint32_t)(first & 3u);
  for (uint32_t q = tid; 4u * q < nw + al; q += 256u) {
    const int32_t li = (int32_t)(4u * q) - (int32_t)al;
    const uint32_t* src = s + li - 1;
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = sh ? __builtin_amdgcn_alignbit(src[e + 1], src[e], 32 - sh) : src[e + 1];
    uint32_t* dst = words + (first - al) + 4u * q;
    if (li >= 0 && li + 3 < (int32_t)nw) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (li + e >= 0 && li + e < (int32_t)nw) dst[e] = o[e];
    }
  }
}

// Whole uint4 blocks of a chunk's staging: its used words and at least one
// zero word after them.  A chunk is staged when one more block still fits its
// slot (slot_words, a multiple of 4: place_k's loads reach one block past the
// staged ones); otherwise place_k encodes it again.
__device__ __forceinline__ uint32_t staged_blocks(uint32_t A) { return ((A >> 5) + 2u + 3u) >> 2; }
__device__ __forceinline__ bool is_staged(uint32_t A, uint32_t slot_words) { return staged_blocks(A) < (slot_words >> 2); }

// Encode, step 1 of 3: one chunk of kChunkTiles tiles per work-group, chunk =
// blockIdx.x: its records in LDS (pack_chunk), then its bits to its staging
// slot when they fit, its bit count to agg, its last 32 bits to tailw, and per
// tile the chunk-local bit offset and k.  No work-group waits on another.
// direct (a tensor of one chunk): the chunk's stream offset is the stream's
// start, so the work-group writes the stream words, offsets and k itself and
// steps 2 and 3 are not launched.  LEN_ONLY: the chunk's bit count only.
template <int L, bool DITHER, int IN, bool LEN_ONLY>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(IN == 1 ? 8 : 1))) void encode_k(EncArgs a) {
  constexpr bool BF16 = IN == 1, PRE = IN == 2;
  // s_buf[3]: the 32 stream bits before the chunk (direct mode); then the chunk's bits
  __shared__ __align__(16) uint32_t s_buf[LEN_ONLY ? 8 : 4 + kSlotWords];
  __shared__ uint32_t s_len[kChunkTiles], s_lo[kChunkTiles], s_k[kChunkTiles];
  uint32_t* const s_stage = s_buf + 4;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const uint32_t chunk = blockIdx.x;
  const uint64_t t_first = (uint64_t)chunk * kChunkTiles;

  if constexpr (LEN_ONLY) {
    const int grp = lane >> 4, r = lane & 15, v = lane_vector(r), pslot = wv * 4 + grp;
    const LaneConst<BF16> lc(a, v);
    InVec<BF16> in[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const uint64_t t = t_first + p * 16 + pslot;
      in[p] = load_in<BF16, false>(a.x, t, v, t < a.n_tiles);
    }
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int slot = p * 16 + pslot;
      const uint64_t t = t_first + slot;
      TileSyms ts;
      tile_front<L, DITHER, BF16, PRE>(a, lc, in[p], t, t < a.n_tiles, v, r, grp, ts);
      if (r == 0) s_len[slot] = ts.L;
    }
    __syncthreads();
    if (wv == 0) {
      const uint32_t A = wave_sum_u32(lane < kChunkTiles ? s_len[lane] : 0u);
      if (lane == 0) a.partials[chunk] = A;
    }
  } else {
    const uint32_t A = pack_chunk<L, DITHER, IN, true>(a, chunk, s_stage, s_len, s_lo, s_k);
    if (a.direct) {
      // the only chunk: its stream offset is B, so its words, offsets and k
      // go out from here and no placement launch follows
      const uint64_t E = a.base ? *a.base : 0ull, E1 = E + A;
      if (tid == 0) {  // appending: the existing bits below B in its last word
        uint32_t t2 = 0u;
        if ((E & 31) && (E >> 5) < a.cap_words) t2 = a.words[E >> 5] << (32u - (uint32_t)(E & 31));
        s_buf[3] = t2;
      }
      __syncthreads();
      if (tid == 0 && (E1 + 31) / 32 > a.cap_words) set_status(a.ws, 4);
      if (tid < kChunkTiles) {
        const uint64_t t = t_first + tid;
        if (t < a.n_tiles) {
          a.offsets[t] = E + s_lo[tid];
          a.kout[t] = (uint8_t)s_k[tid];
          if (t == a.n_tiles - 1) a.offsets[a.n_tiles] = E1;
        }
      }
      put_chunk_words(a.words, a.cap_words, s_stage, E, A, true, tid);
      return;
    }
    const uint32_t n4 = staged_blocks(A);
    if (is_staged(A, a.slot_words)) {
      uint4* dst = reinterpret_cast<uint4*>(a.stage + (uint64_t)chunk * a.slot_words);
      for (uint32_t i = tid; i < n4; i += 256) {
        const uint4 q = reinterpret_cast<const uint4*>(s_stage)[i];
        store_nt4(&dst[i].x, q.x, q.y, q.z, q.w);
      }
    }
    if (tid < kChunkTiles) {
      const uint64_t t = t_first + tid;
      if (t < a.n_tiles) {
        a.loc[t] = s_lo[tid];
        a.kout[t] = (uint8_t)s_k[tid];
      }
    }
    if (tid == 0) {
      a.agg[chunk] = A;
      const uint32_t b = A - 32u, w = b >> 5, sh = b & 31;
      a.tailw[chunk] = sh ? __builtin_amdgcn_alignbit(s_stage[w + 1], s_stage[w], sh) : s_stage[w];
    }
  }
}

// Encode, step 2 of 3 (more than kSelfScanChunks chunks), first part: per
// block of 1024 chunks (one work-group, four counts per thread) the chunks'
// exclusive offsets within the block, Eloc[c] (32-bit: at most 1024 * 94720
// bits), and the block's total T[b].
constexpr uint32_t kScanBlock = 1024;
__global__ __launch_bounds__(256) void blocksum_k(const uint32_t* agg, uint32_t n, uint32_t* Eloc, uint64_t* T) {
  __shared__ uint32_t s_w[4];
  const uint32_t tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, i = blockIdx.x * kScanBlock + 4u * tid;
  uint4 g = make_uint4(0u, 0u, 0u, 0u);
  if (i < n) g = *reinterpret_cast<const uint4*>(agg + i);  // agg is padded to 64 entries
  if (i + 1 >= n) g.y = 0u;
  if (i + 2 >= n) g.z = 0u;
  if (i + 3 >= n) g.w = 0u;
  const uint32_t t = g.x + g.y + g.z + g.w;
  uint32_t x = t;  // inclusive scan over the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if ((int)lane >= o) x += y;
  }
  if (lane == 63) s_w[wv] = x;
  __syncthreads();
  uint32_t run = x - t;
#pragma unroll
  for (uint32_t w = 0; w < 3; ++w) run += w < wv ? s_w[w] : 0u;
  if (i < n) {
    const uint4 e = make_uint4(run, run + g.x, run + g.x + g.y, run + g.x + g.y + g.z);
    *reinterpret_cast<uint4*>(Eloc + i) = e;  // Eloc is padded like agg
  }
  if (tid == 0) T[blockIdx.x] = (uint64_t)s_w[0] + s_w[1] + s_w[2] + s_w[3];
}

// Encode, step 2 of 3, second part (above 64 blocks; up to 64 the placement
// sums the totals itself): the block totals T[0..nb) replaced in place by
// their exclusive prefix sums, by one work-group of 1024 threads (1024 blocks
// per round, a carry between rounds).
__global__ __launch_bounds__(1024) void blockscan_k(uint64_t* T, uint32_t nb) {
  __shared__ uint64_t s_w[16];
  __shared__ uint64_t s_carry;
  const uint32_t tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) s_carry = 0;
  for (uint32_t base = 0; base < nb; base += 1024u) {  // (uniform)
    const uint32_t i = base + tid;
    const uint64_t t = i < nb ? T[i] : 0ull;
    uint64_t x = t;  // inclusive scan over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint64_t y = __shfl_up(x, o);
      if ((int)lane >= o) x += y;
    }
    if (lane == 63) s_w[wv] = x;
    __syncthreads();  // (also: s_carry of the previous round is final)
    uint64_t run = s_carry + x - t;
#pragma unroll
    for (uint32_t w = 0; w < 15; ++w) run += w < wv ? s_w[w] : 0ull;
    if (i < nb) T[i] = run;
    __syncthreads();  // every thread has read s_w and s_carry
    if (tid == 1023) s_carry = run + t;
  }
}

// place_k's second part for plans with a compact workspace: the chunks of
// the work-group that were not staged, encoded again by the whole work-group
// and written straight into the stream (E: the calling wave's chunk offset).
template <int L, bool DITHER, int IN>
__device__ __forceinline__ void place_unstaged(const EncArgs& a, uint32_t cg, uint64_t E, uint64_t B) {
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wv = tid >> 6;
  // chunks that were not staged, after the staged ones so that only E is
  // live here (uniform: every wave reads the same four counts)
  uint32_t redo = 0;
#pragma unroll
  for (uint32_t w = 0; w < kPlaceChunks; ++w)
    if (cg + w < a.n_chunks && !is_staged(a.agg[cg + w], a.slot_words)) redo |= 1u << w;
  if (redo) {
    __shared__ __align__(16) uint32_t s_buf[4 + kSlotWords];
    __shared__ uint32_t s_len[kChunkTiles], s_lo[kChunkTiles], s_k[kChunkTiles];
    __shared__ unsigned long long s_E[kPlaceChunks];
    if (lane == 0) s_E[wv] = E;
    __syncthreads();
    for (uint32_t w = 0; w < kPlaceChunks; ++w) {  // (uniform)
      if (!((redo >> w) & 1u)) continue;
      const uint32_t c = cg + w;
      const uint32_t A2 = pack_chunk<L, DITHER, IN, false>(a, c, s_buf + 4, s_len, s_lo, s_k);
      if (tid == 0) {  // the 32 stream bits before the chunk
        uint32_t t2 = 0u;
        if (c > 0) t2 = a.tailw[c - 1];
        else if ((B & 31) && (B >> 5) < a.cap_words) t2 = a.words[B >> 5] << (32u - (uint32_t)(B & 31));
        s_buf[3] = t2;
      }
      __syncthreads();
      put_chunk_words(a.words, a.cap_words, s_buf + 4, s_E[w], A2, c == a.n_chunks - 1, tid);
      __syncthreads();  // before s_buf is filled again
    }
  }
}

// Encode, step 3 of 3: one chunk per wave, kPlaceChunks chunks per
// work-group.  The chunk's staged bits go to stream bits [B + E[c], B + E[c+1])
// with a funnel shift, four words per lane (the first kSpecIters uint4 of
// staging loads issued with the offset loads, before they arrive); the word
// shared with the predecessor takes the predecessor's last 32 bits, recorded
// by step 1, so every stream word is written exactly once.  B is 0, or when
// appending to an existing stream its end bit: then the first chunk's first
// word keeps the existing bits below B.  Also the per-tile offsets, and the
// capacity check.  E[c] is formed here: up to kSelfScanChunks chunks
// (SELF_SCAN) the work-group sums the bit counts of the chunks before its
// first (all reads of one small array that the L2 serves) and each wave adds
// those of the work-group's chunks before its own, so step 2 is skipped; above
// that as the bits of the blocks of 1024 chunks before its own (step 2) plus
// the counts in its block before it.  REDO (plans with a compact workspace,
// whose slots are sized from the plan's rate with a margin): a chunk that did
// not fit its slot (rare) is encoded again here by the whole work-group, from
// its input, straight into the stream.  That path needs the encode's
// registers, which costs the common path a tighter register budget, so plans
// with full-size slots (every chunk fits) run the instance without it.
template <int L, bool DITHER, int IN, bool SELF_SCAN, bool REDO>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(REDO ? 8 : 1))) void place_k(EncArgs a) {
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wv = tid >> 6;
  const uint32_t cg = blockIdx.x * kPlaceChunks;  // the work-group's first chunk
  const uint32_t chunk = cg + wv;
  const bool live = chunk < a.n_chunks;  // (wave-uniform)
  const uint32_t sb = a.slot_words >> 2;  // uint4 blocks per slot
  const uint32_t* st = a.stage + (uint64_t)chunk * a.slot_words;
  // SELF_SCAN: the counts [0, cg) as uint4 (the count array is padded to 64
  // entries), loaded first so that summing them waits for these loads only;
  // only the rounds of 1024 that hold counts below cg are loaded, and lanes
  // past cg in the last one read entry 0
  constexpr uint32_t kR = SELF_SCAN ? kSelfScanChunks / 1024 : 1;
  uint4 g[kR];
  if constexpr (SELF_SCAN) {
#pragma unroll
    for (uint32_t j = 0; j < kR; ++j) {  // (the round tests are work-group uniform)
      const uint32_t i = 4u * tid + 1024u * j;
      g[j] = make_uint4(0u, 0u, 0u, 0u);
      if (1024u * (j + 1) <= cg) g[j] = *reinterpret_cast<const uint4*>(a.agg + i);
      else if (1024u * j < cg) g[j] = *reinterpret_cast<const uint4*>(a.agg + (i < cg ? i : 0u));
    }
  }
  // staging reads: in round j lane l holds the uint4 blocks 64 j + l - 1 and
  // 64 j + l of the chunk's staged words; the first kSpecIters rounds are read
  // before the chunk's offset is known (enough below about 6 bits per scalar)
  constexpr uint32_t kSpecIters = 3;
  const uint4* st4 = reinterpret_cast<const uint4*>(st);
  uint4 u0[kSpecIters], u1[kSpecIters];
#pragma unroll
  for (uint32_t j = 0; j < kSpecIters; ++j) {  // (within the slot)
    const uint32_t q = lane + 64u * j;
    u1[j] = live && q < sb ? st4[q] : make_uint4(0u, 0u, 0u, 0u);
    u0[j] = (live && q && q <= sb) ? st4[q - 1u] : make_uint4(0u, 0u, 0u, 0u);
  }
  const uint64_t B = a.base ? *a.base : 0ull;  // work-group uniform
  uint32_t tw = 0u;                            // wave uniform
  if (live) {
    if (chunk > 0) tw = a.tailw[chunk - 1];
    else if ((B & 31) && (B >> 5) < a.cap_words) tw = a.words[B >> 5] << (32u - (uint32_t)(B & 31));  // bits below B
    // (B past the capacity fails the capacity check below)
  }
  if (lane == 0) u0[0].w = tw;  // staged word -1: the bits before the chunk's first
  const uint64_t t = (uint64_t)chunk * kChunkTiles + lane;
  const bool tl = live && lane < kChunkTiles && t < a.n_tiles;
  const uint32_t lc = tl ? a.loc[t] : 0u;
  const uint32_t A = live ? a.agg[chunk] : 0u;
  uint64_t E;
  if constexpr (SELF_SCAN) {
    __shared__ uint32_t s_part[4];
    // rounds wholly below cg add all four counts; only the round holding cg
    // masks (the tests are work-group uniform, so no VALU is spent on rounds
    // that were not loaded)
    uint32_t part = 0;
#pragma unroll
    for (uint32_t j = 0; j < kR; ++j) {
      if (1024u * (j + 1) <= cg) {
        part += g[j].x + g[j].y + g[j].z + g[j].w;
      } else if (1024u * j < cg) {
        const uint32_t i = 4u * tid + 1024u * j;
        part += (i < cg ? g[j].x : 0u) + (i + 1 < cg ? g[j].y : 0u) + (i + 2 < cg ? g[j].z : 0u) +
                (i + 3 < cg ? g[j].w : 0u);
      }
    }
    // (the wave total is formed by every lane: a lane-0-only branch would
    // leave the other rows' sums unfinished when read across lanes)
    const uint32_t wsum = wave_sum_u32(part);
    if (lane == 0) s_part[wv] = wsum;
    __syncthreads();
    uint32_t before = 0;  // the work-group's chunks before this wave's (all below n_chunks when live)
    for (uint32_t w = 0; w < wv; ++w) before += live ? a.agg[cg + w] : 0u;
    E = B + s_part[0] + s_part[1] + s_part[2] + s_part[3] + before;  // at most 8192 * 94720 bits
  } else {  // the block's prefix plus the offset within the block (uniform loads)
    uint64_t pre = 0;
    if (a.block_totals) {  // at most 64 blocks: lane b adds the total of block b before this one
      const uint32_t b = chunk >> 10;
      pre = lane < b && live ? a.blockpre[lane] : 0ull;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) pre += __shfl_xor(pre, o);
    } else if (live) {
      pre = a.blockpre[chunk >> 10];
    }
    E = live ? B + pre + a.eloc[chunk] : 0ull;
  }
  if (live) {
    const uint64_t E1 = E + A;
    if (lane == 0 && chunk == a.n_chunks - 1 && (E1 + 31) / 32 > a.cap_words) atomicOr(&a.ws->status, 1u << 4);
    if (tl) {
      a.offsets[t] = E + lc;
      if (t == a.n_tiles - 1) a.offsets[a.n_tiles] = E1;
    }
    const bool last = chunk == a.n_chunks - 1;
    const uint64_t first = E >> 5;
    const uint32_t sh = (uint32_t)(E & 31);
    const uint64_t endw = last ? (E1 + 31) >> 5 : E1 >> 5;
    const uint64_t stop = endw < a.cap_words ? endw : a.cap_words;
    const uint32_t nw = stop > first ? (uint32_t)(stop - first) : 0u;
    // stream words first + i (i < nw) = (s[i] : s[i - 1]) >> (32 - sh), in
    // 16-byte aligned groups: lane l of round j writes words g .. g + 3 with
    // g = first - al + 4 (64 j + l), i.e. i = li .. li + 3, li = 4 (64 j + l) - al;
    // its staged words s[li - 1 .. li + 3] are entries 3 - al .. 7 - al of the
    // two blocks it holds.  Blocks read past the spec rounds have li < nw, so
    // 4 q <= nw + 2 <= (A >> 5) + 4, q <= staged_blocks(A) < slot_words / 4:
    // inside the slot.
    const uint32_t al = (uint32_t)(first & 3u);  // (wave uniform)
    auto group = [&](uint32_t j, const uint4& b0, const uint4& b1) {
      const uint32_t q = lane + 64u * j;
      const int32_t li = (int32_t)(4u * q) - (int32_t)al;
      uint32_t w[5];
      if (al == 0) {  // (uniform)
        w[0] = b0.w; w[1] = b1.x; w[2] = b1.y; w[3] = b1.z; w[4] = b1.w;
      } else if (al == 1) {
        w[0] = b0.z; w[1] = b0.w; w[2] = b1.x; w[3] = b1.y; w[4] = b1.z;
      } else if (al == 2) {
        w[0] = b0.y; w[1] = b0.z; w[2] = b0.w; w[3] = b1.x; w[4] = b1.y;
      } else {
        w[0] = b0.x; w[1] = b0.y; w[2] = b0.z; w[3] = b0.w; w[4] = b1.x;
      }
      uint32_t o[4];
  #pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = sh ? __builtin_amdgcn_alignbit(w[e + 1], w[e], 32 - sh) : w[e + 1];
      uint32_t* dst = a.words + (first - al) + 4u * q;
      if (li >= 0 && li + 3 < (int32_t)nw) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
      } else {
  #pragma unroll
        for (int e = 0; e < 4; ++e)
          if (li + e >= 0 && li + e < (int32_t)nw) dst[e] = o[e];
      }
    };
    if (is_staged(A, a.slot_words)) {  // else its words come from place_unstaged
  #pragma unroll
      for (uint32_t j = 0; j < kSpecIters; ++j)
        if ((int32_t)(4u * (lane + 64u * j)) - (int32_t)al < (int32_t)nw) group(j, u0[j], u1[j]);
      for (uint32_t j = kSpecIters; 256u * j < nw + al; ++j) {
        const uint32_t q = lane + 64u * j;
        if ((int32_t)(4u * q) - (int32_t)al < (int32_t)nw) group(j, st4[q - 1u], st4[q]);
      }
    }
  }
  if constexpr (REDO) place_unstaged<L, DITHER, IN>(a, cg, E, B);  // (full-size slots: every chunk was staged)
}

// ===========================================================================
// Decode
// ===========================================================================
// position of the j-th (0-based) set bit of w; w has more than j set bits
__device__ __forceinline__ uint32_t select_bit(uint32_t w, uint32_t j) {
  uint32_t pos = 0, c;
  c = __builtin_popcount(w & 0xFFFFu);
  if (j >= c) { j -= c; w >>= 16; pos += 16; }
  c = __builtin_popcount(w & 0xFFu);
  if (j >= c) { j -= c; w >>= 8; pos += 8; }
  c = __builtin_popcount(w & 0xFu);
  if (j >= c) { j -= c; w >>= 4; pos += 4; }
  c = __builtin_popcount(w & 0x3u);
  if (j >= c) { j -= c; w >>= 2; pos += 2; }
  c = w & 1u;
  if (j >= c) pos += 1;
  return pos;
}

// The same from a table in LDS: lut[8 b + i] = position of the i-th set bit
// of the byte b.  The byte holding bit j is found from the popcounts of the
// low 8, 16 and 24 bits.
struct SelectLut {
  uint8_t v[256][8];
};
constexpr SelectLut make_select_lut() {
  SelectLut t{};
  for (int b = 0; b < 256; ++b) {
    int n = 0;
    for (int i = 0; i < 8; ++i)
      if ((b >> i) & 1) t.v[b][n++] = (uint8_t)i;
  }
  return t;
}
__constant__ SelectLut kSelectLut = make_select_lut();

__device__ __forceinline__ uint32_t select_bit_lut(uint32_t w, uint32_t j, const uint8_t* lut) {
  const uint32_t c0 = __builtin_popcount(w & 0xFFu), c1 = __builtin_popcount(w & 0xFFFFu),
                 c2 = __builtin_popcount(w & 0xFFFFFFu);
  const uint32_t bi = (uint32_t)(j >= c0) + (uint32_t)(j >= c1) + (uint32_t)(j >= c2);
  const uint32_t before = bi == 0 ? 0u : bi == 1 ? c0 : bi == 2 ? c1 : c2;
  return 8u * bi + lut[8u * __builtin_amdgcn_ubfe(w, 8u * bi, 8u) + (j - before)];
}

// Lattice coordinates of the lane's 8 symbols (inverse zigzag and unstrip),
// as fp32 real-space points.  With s = sext(bit 0 of m), 2*unzigzag(m) is
// m ^ s, so a halved coordinate plus the raw bit is one v_xad_u32.
template <int L>
__device__ __forceinline__ void dequant_lane(const uint32_t m[8], uint32_t raw, float p[8]) {
  uint32_t t[8];  // 2 * unzigzag(m)
#pragma unroll
  for (int j = 0; j < 8; ++j) t[j] = m[j] ^ (uint32_t)__builtin_amdgcn_sbfe((int)m[j], 0, 1);
  if constexpr (L == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = (float)((int32_t)t[j] >> 1);
  } else if constexpr (L == 1) {
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const int32_t jj = (int32_t)t[j + 1] >> 1;              // j
      const int32_t ii = (int32_t)(t[j] + ((uint32_t)jj & 1u));  // i = 2 i' + (j & 1)
      p[j] = (float)ii;
      p[j + 1] = (float)jj * kSqrt3;
    }
  } else if constexpr (L == 2) {
#pragma unroll
    for (int h = 0; h < 8; h += 4) {
      const uint32_t par = ((t[h] ^ t[h + 1] ^ t[h + 2]) >> 1) & 1u;  // parity of x0 + x1 + x2
#pragma unroll
      for (int j = 0; j < 3; ++j) p[h + j] = (float)((int32_t)t[h + j] >> 1);
      p[h + 3] = (float)(int32_t)(t[h + 3] + par);
    }
  } else {
    // x_i = 2 y_i + b; y_7 = 2 z_7 + parity(y_0 + ... + y_6), bit 1 of x_i = bit 0 of y_i
    uint32_t x[8];
#pragma unroll
    for (int j = 0; j < 7; ++j) x[j] = t[j] + raw;
    const uint32_t par = ((x[0] ^ x[1] ^ x[2] ^ x[3] ^ x[4] ^ x[5] ^ x[6]) >> 1) & 1u;
    x[7] = ((t[7] + par) << 1) + raw;
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = (float)(int32_t)x[j];
  }
}

// General segment starts (any unary length): count ones per word 16 words
// at a time, scan, select rank 8v-1 for every vector v.  Writes ust[1..15].
__device__ __forceinline__ uint32_t unary_starts_general(const uint32_t* s, uint32_t ustart, uint32_t uend, int r,
                                                         uint32_t* ust) {
  const uint32_t wA = ustart >> 5, wB = (uend - 1u) >> 5, nW = wB - wA + 1u;
  uint32_t rank_base = 0;
  for (uint32_t it = 0; it < nW; it += 16) {
    const uint32_t wi = wA + it + (uint32_t)r;
    uint32_t word = (it + (uint32_t)r < nW) ? s[wi] : 0u;
    if (wi == wA) word &= ~0u << (ustart & 31);
    if (wi == wB && (uend & 31)) word &= (1u << (uend & 31)) - 1u;
    const uint32_t cnt = __builtin_popcount(word);
    const uint32_t incl = row_scan_u32(cnt);
    const uint32_t ex = incl - cnt + rank_base;
    uint32_t R = ((ex + 8u) & ~7u) - 1u;  // smallest rank = 7 mod 8 that is >= ex
    while (R < ex + cnt && R < 120u) {
      ust[(R + 1u) >> 3] = wi * 32u + select_bit(word, R - ex) + 1u;
      R += 8u;
    }
    rank_base += row_sum_u32(cnt);
  }
  return rank_base;
}

// Parse the lane's 8 symbols of one tile record held in LDS (record at local
// bit base, length Lb, Rice parameter k) and return the dequantised
// real-space lattice coordinates.  Returns false when the record is corrupt
// (the outcome is uniform over the 16 lanes of the tile).  ust: 16 words of
// LDS per tile.
template <int L>
__device__ __forceinline__ bool parse_lane(const uint32_t* s, uint32_t base, uint32_t Lb, uint32_t k, int v, int r,
                                           int lane, uint32_t* ust, float p[8], const uint8_t* sel_lut = nullptr) {
  constexpr uint32_t RAW = Lat<L>::raw;
  uint32_t raw = 0;
  if constexpr (RAW > 0) {
    const uint32_t f = __builtin_amdgcn_alignbit(s[(base >> 5) + 1], s[base >> 5], base & 31);
    raw = (f >> v) & 1u;
  }
  // remainders: 8 fields of k bits at fixed positions
  uint32_t rem[8];
  const uint32_t rpos = base + RAW + __umul24(8u * (uint32_t)v, k);
  if (k <= 7) {
    const uint32_t w = rpos >> 5, sh = rpos & 31;
    const uint32_t w0 = s[w], w1 = s[w + 1], w2 = s[w + 2];
    const uint32_t lo = __builtin_amdgcn_alignbit(w1, w0, sh);
    const uint32_t hi = __builtin_amdgcn_alignbit(w2, w1, sh);
    const uint32_t h4 = __builtin_amdgcn_alignbit(hi, lo, 4 * k);  // fields 4..7 (4k < 32)
#pragma unroll
    for (int j = 0; j < 4; ++j) rem[j] = __builtin_amdgcn_ubfe(lo, j * k, k);
#pragma unroll
    for (int j = 0; j < 4; ++j) rem[4 + j] = __builtin_amdgcn_ubfe(h4, j * k, k);
  } else {
    const uint32_t mask = (1u << k) - 1u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t P = rpos + j * k;
      rem[j] = __builtin_amdgcn_alignbit(s[(P >> 5) + 1], s[P >> 5], P & 31) & mask;
    }
  }
  // unary section [ustart, uend): 128 ones; lane v's 8 codes start after the
  // (8v)-th one.  The record parses only if the section holds 128 ones and
  // the last one is its last bit.
  const uint32_t ustart = base + RAW + 128u * k, uend = base + Lb;
  const uint32_t wA = ustart >> 5, nW = ((uend - 1u) >> 5) - wA + 1u;
  const uint32_t lastbit = (s[(uend - 1u) >> 5] >> ((uend - 1u) & 31)) & 1u;
  uint32_t start;
  bool ok = lastbit != 0;
  if (nW <= 16) {
    // one word per lane: the ones of ranks [E, I) lie in word r
    uint32_t word = (uint32_t)r < nW ? s[wA + r] : 0u;
    if (r == 0) word &= ~0u << (ustart & 31);
    if ((uint32_t)r == nW - 1 && (uend & 31)) word &= (1u << (uend & 31)) - 1u;
    const uint32_t c = __builtin_popcount(word);
    const uint32_t I = row_scan_u32(c);
    if (r == 15) ok &= I == 128u;
    if (((__ballot(!ok) >> (lane & ~15)) & 0xFFFFull) != 0) return false;
    // Word r holds the first one of vector u's codes minus one, the one of
    // rank 8u - 1, for u in [vlo, vhi] (at most 4 of them, u = 1..15): it
    // records itself and its E for those u (the rest of the writes go to the
    // unused entry 0).  With 128 ones every entry 1..15 is written once.
    const uint32_t E = I - c;
    const uint32_t vlo = (E + 8u) >> 3, vhi = min(I >> 3, 15u);
    const uint32_t ent = (uint32_t)r | (E << 8);
#pragma unroll
    for (uint32_t j = 0; j < 4; ++j) {
      const uint32_t u = vlo + j;
      ust[u <= vhi ? u : 0u] = ent;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    start = ustart;
    if (v > 0) {
      const uint32_t e = ust[v];
      const uint32_t wr = e & 15u;
      uint32_t wd = s[wA + wr];
      if (wr == 0) wd &= ~0u << (ustart & 31);
      const uint32_t j = 8u * (uint32_t)v - 1u - (e >> 8);  // rank of the one within the word
      start = (wA + wr) * 32u + (sel_lut ? select_bit_lut(wd, j, sel_lut) : select_bit(wd, j)) + 1u;
    }
  } else {
    ok &= unary_starts_general(s, ustart, uend, r, ust) == 128u;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (((__ballot(!ok) >> (lane & ~15)) & 0xFFFFull) != 0) return false;
    start = v == 0 ? ustart : ust[v];
  }
  // the lane's 8 unary codes: q zeros then a one, from start
  uint32_t m[8];
  const uint32_t qlim = kMLimit >> k;
  {
    const uint32_t w = min(start >> 5, (uint32_t)kStageWords - 2u), sh = start & 31;
    uint32_t win = __builtin_amdgcn_alignbit(s[w + 1], s[w], sh);
    if (__builtin_popcount(win) >= 8) {
      // all 8 codes inside the 32-bit window: q < 32 <= qlim for k <= 17
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t q = (uint32_t)__builtin_ctz(win);
        m[j] = (q << k) | rem[j];
        win = (win >> q) >> 1;
      }
      if (k > 17u) {
        // a quotient of up to 31 may reach 2^22 only for k > 17
        uint32_t qmax = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) qmax = max(qmax, m[j] >> k);
        ok &= qmax < qlim;
      }
    } else {
      uint32_t pos = start;
      const uint32_t wlim = (uend >> 5) + 1u;  // the staging buffer holds words up to here
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t st = pos;
        uint32_t ww = s[min(pos >> 5, wlim)] >> (pos & 31);
        while (ww == 0u && pos < uend) {
          pos = (pos | 31u) + 1u;
          ww = s[min(pos >> 5, wlim)];
        }
        pos += (uint32_t)__builtin_ctz(ww | 0x80000000u);
        const uint32_t q = pos - st;
        ok &= pos < uend && q < qlim;
        m[j] = (q << k) | rem[j];
        pos += 1;
      }
    }
  }
  if (((__ballot(!ok) >> (lane & ~15)) & 0xFFFFull) != 0) return false;
  dequant_lane<L>(m, raw, p);
  return true;
}

// Stream words [w_first, w_end) of a chunk into LDS from the 16-byte
// boundary below its first record (s_stage[i] = word w_first + i), in whole
// uint4 loads, all issued before the LDS stores.  The words after w_end in
// the last group are what the buffer holds there (the next records' bits):
// a record never reads past its own end, and the checks that decide whether
// a record parses mask them off.  A group that would leave the buffer (only
// at the stream's end) is read word by word.  One zero group follows the
// span.  Every thread of the work-group calls it, after s_off[0..nt] is
// visible; returns whether the span is sane (work-group uniform).
template <bool NT = false>  // NT: the stream is read once per launch (a plain decode)
__device__ __forceinline__ bool stage_chunk(const uint32_t* words, uint64_t n_words, const uint64_t* s_off,
                                            uint32_t nt, uint32_t* s_stage, uint64_t& w_first, int tid) {
  const uint64_t o_first = s_off[0], o_end = s_off[nt];
  w_first = (o_first >> 5) & ~3ull;
  const uint64_t w_end = (o_end + 31) >> 5;
  const bool span_ok = o_end >= o_first && (w_end - w_first) <= (uint64_t)kStageWords - 8 && w_end <= n_words;
  if (span_ok) {
    const uint32_t n4 = (uint32_t)((w_end - w_first + 3) >> 2);
    const uint64_t full4 = (n_words - w_first) >> 2;  // groups wholly inside the buffer
    const uint32_t* src = words + w_first;
    uint4* dst = reinterpret_cast<uint4*>(s_stage);
    uint4 q[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const uint32_t i4 = (uint32_t)tid + 256u * j;
      q[j] = make_uint4(0u, 0u, 0u, 0u);
      if (i4 < n4) {
        if ((uint64_t)i4 < full4) {
          q[j] = load16<NT>(src + 4u * i4);
        } else {  // the buffer ends inside this group: its words below n_words
          const uint64_t left = n_words - w_first - 4ull * i4;  // 1..3
          q[j].x = src[4u * i4];
          if (left > 1) q[j].y = src[4u * i4 + 1];
          if (left > 2) q[j].z = src[4u * i4 + 2];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const uint32_t i4 = (uint32_t)tid + 256u * j;
      if (i4 < n4) dst[i4] = q[j];
    }
    if (tid == 0) dst[n4] = make_uint4(0u, 0u, 0u, 0u);
  }
  return span_ok;
}

// Per tile of a chunk, what a lane needs to parse its record, from one thread
// per tile after the offsets and Rice parameters are in LDS: the record's
// bit in the staged span, its length, k, and whether it is sane (k <= 22,
// length between the shortest and the longest possible record, span staged).
template <int L>
__device__ __forceinline__ void tile_records(const uint64_t* s_off, const uint32_t* s_k, uint32_t nt, uint64_t w_first,
                                             bool span_ok, uint4* s_rec, int tid) {
  constexpr uint32_t RAW = Lat<L>::raw;
  constexpr uint32_t MAXREC = RAW + 128u * 23u;
  if (tid < (int)nt) {
    const uint64_t o0 = s_off[tid], o1 = s_off[tid + 1];
    const uint32_t k = s_k[tid];
    const uint64_t Lr = o1 - o0;  // wraps past MAXREC when o1 < o0
    const bool ok = span_ok && k <= (uint32_t)kKMax && Lr >= RAW + 128u * (1u + k) && Lr <= MAXREC;
    s_rec[tid] = make_uint4((uint32_t)(o0 - 32 * w_first), (uint32_t)Lr, k, ok ? 1u : 0u);
  }
}

template <int L, bool DITHER, int OUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OUT == kOutScores ? 1 : 8))) void decode_k(DecArgs a) {
  __shared__ __align__(16) uint32_t s_stage[kStageWords];
  __shared__ uint64_t s_off[kChunkTiles + 1];
  __shared__ uint32_t s_k[kChunkTiles];
  __shared__ uint32_t s_ust[16][16];
  __shared__ uint4 s_rec[kChunkTiles];  // per tile: record bit, length, k, sane
  __shared__ float s_q[OUT == kOutScores ? 16 : 1][kTile];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, grp = lane >> 4, r = lane & 15;
  const int v = lane_vector(r);
  const FwhtSigns fs = fwht_signs(v);

  uint64_t t_first, t_limit, head = 0;
  if constexpr (OUT == kOutScores) {
    head = blockIdx.y;
    t_first = head * a.tiles_per_head + (uint64_t)blockIdx.x * kChunkTiles;
    t_limit = (head + 1) * a.tiles_per_head;
  } else {
    t_first = (uint64_t)blockIdx.x * kChunkTiles;
    t_limit = a.n_tiles;
  }
  const uint32_t nt = (uint32_t)((t_limit - t_first) < (uint64_t)kChunkTiles ? (t_limit - t_first) : kChunkTiles);
  uint32_t blk0 = 0;  // matrix-vector mode, nblk >= 32: block of the chunk's first tile
  if constexpr (OUT == kOutGemv) blk0 = a.nblk >= 32u ? (uint32_t)t_first % a.nblk : 0u;

  if (tid <= (int)nt) s_off[tid] = a.offsets[t_first + tid];
  if (tid < (int)nt) s_k[tid] = a.kin[t_first + tid];
  // the bit-select table (not with the scores' query block: LDS)
  constexpr bool kLut = OUT != kOutScores;
  __shared__ uint2 s_sel[kLut ? 256 : 1];
  if constexpr (kLut) s_sel[tid] = reinterpret_cast<const uint2*>(&kSelectLut)[tid];
  if constexpr (OUT == kOutScores) {
    // rotate the head's queries: q~ = H D q, one query per 16-lane row (with
    // a dense rotation the queries arrive rotated: q~ = Q q)
    const int g = wv * 4 + grp;
    if (g < (int)a.qph) {
      const float* qp = a.q + ((head * a.qph + g) * kTile + 8 * v);
      if (a.q_rot) {
#pragma unroll
        for (int i = 0; i < 8; ++i) s_q[g][8 * v + i] = qp[i];
      } else {
        const uint32_t sm = lane_signs32(a.sl32, v);
        float xq[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) xq[i] = __builtin_bit_cast(float, fbits(qp[i]) ^ ((sm << i) & 0x80000000u));
        fwht_tile(xq, fs);
#pragma unroll
        for (int i = 0; i < 8; ++i) s_q[g][8 * v + i] = xq[i] * fs.lane_sign;
      }
    }
  }
  __syncthreads();
  uint64_t w_first;
  const bool span_ok =
      stage_chunk<OUT == kOutF32 || OUT == kOutBf16 || OUT == kOutRot>(a.words, a.n_words, s_off, nt, s_stage, w_first, tid);
  tile_records<L>(s_off, s_k, nt, w_first, span_ok, s_rec, tid);
  __syncthreads();

  // output scale: the lane sign and c_dec, then the signs of D (bf16: on the
  // packed pairs after rounding, which is symmetric in the sign; fp32: folded
  // into eight per-coordinate scales)
  const float cs = fs.lane_sign * a.c_dec;
  const uint32_t sm = OUT == kOutBf16 ? lane_signs16(a.sl16, v) : lane_signs32(a.sl32, v);
  float sc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sc[i] = OUT == kOutF32 ? __builtin_bit_cast(float, fbits(cs) ^ ((sm << i) & 0x80000000u)) : cs;

#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int pslot = wv * 4 + grp;
    const int slot = p * 16 + pslot;
    const bool valid = slot < (int)nt;
    const uint64_t t = t_first + slot;
    // pv is written by a successful parse.  Without dither, slots past the
    // end and corrupt records (both rare) take zeros in a branch of their own,
    // so the common path spends no moves on them; the dithered variants keep
    // the zero start (fewer live registers there).
    float pv[8];
    if constexpr (DITHER) {
#pragma unroll
      for (int i = 0; i < 8; ++i) pv[i] = 0.0f;
    }
    bool good = false;
    if (valid) {
      const uint4 rec = s_rec[slot];
      if (rec.w) good = parse_lane<L>(s_stage, rec.x, rec.y, rec.z, v, r, lane, s_ust[pslot], pv,
                                          kLut ? reinterpret_cast<const uint8_t*>(s_sel) : nullptr);
      if (!good && r == 0) set_status(a.ws, 5);
      if constexpr (DITHER) {
        if (!good) {
#pragma unroll
          for (int i = 0; i < 8; ++i) pv[i] = 0.0f;
        } else {
          float d[8];
          dither_lane<L>(a.key0, a.key1, a.tile_base + t, v, d);
#pragma unroll
          for (int i = 0; i < 8; ++i) pv[i] = pv[i] - d[i];
        }
      }
    }
    if constexpr (!DITHER) {
      if (!good) {
#pragma unroll
        for (int i = 0; i < 8; ++i) pv[i] = 0.0f;
      }
    }
    if constexpr (OUT == kOutGemv) {
      // tile t covers 128-column block t mod nblk of its row: the dot product
      // with each vector's rotated block (the rows of a tile share validity)
      if (valid) {
        const uint32_t tt = (uint32_t)t;  // n_tiles < 2^32
        const uint32_t blk = a.nblk >= 32u ? (blk0 + (uint32_t)slot >= a.nblk ? blk0 + (uint32_t)slot - a.nblk
                                                                                : blk0 + (uint32_t)slot)
                                           : tt % a.nblk;
        const float* xb = a.xr + (uint64_t)blk * kTile + 8 * v;
        for (uint32_t j = 0; j < a.nb; ++j) {
          const float4 x0 = *reinterpret_cast<const float4*>(xb + (uint64_t)j * a.nblk * kTile);
          const float4 x1 = *reinterpret_cast<const float4*>(xb + (uint64_t)j * a.nblk * kTile + 4);
          const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
          float acc = 0.0f;
#pragma unroll
          for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(xv[i], pv[i], acc);
          acc = row_sum_f32(acc);
          if (r == 0) a.dots[(uint64_t)tt * a.nb + j] = acc;
        }
      }
    } else if constexpr (OUT == kOutScores) {
      if (valid) {
        const uint64_t sidx = t - head * a.tiles_per_head;
        for (uint32_t g = 0; g < a.qph; ++g) {
          float acc = 0.0f;
#pragma unroll
          for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(s_q[g][8 * v + i], pv[i], acc);
          acc = row_sum_f32(acc);
          if (r == 0) a.scores[(head * a.qph + g) * a.tiles_per_head + sidx] = acc * a.c_dec;
        }
      }
    } else if constexpr (OUT == kOutRot) {
      // the dequantised tile in the rotated domain (a dense inverse rotation follows)
      if (valid) {
        float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.y) + t * kTile + 8 * v);
        dst[0] = make_float4(pv[0], pv[1], pv[2], pv[3]);
        dst[1] = make_float4(pv[4], pv[5], pv[6], pv[7]);
      }
    } else {
      fwht_tile(pv, fs);
      if (valid) {
        float o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = pv[i] * sc[i];
        if constexpr (OUT == kOutBf16) {
          typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
          typedef float f32x2_t __attribute__((ext_vector_type(2)));
          uint32_t pk[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f32x2_t f = {o[2 * i], o[2 * i + 1]};
            pk[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t)) ^ ((sm << i) & 0x80008000u);
          }
          store_nt4(reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(a.y) + t * kTile + 8 * v), pk[0], pk[1],
                    pk[2], pk[3]);
        } else {
          uint32_t* dst = reinterpret_cast<uint32_t*>(reinterpret_cast<float*>(a.y) + t * kTile + 8 * v);
          store_nt4(dst, __builtin_bit_cast(uint32_t, o[0]), __builtin_bit_cast(uint32_t, o[1]),
                    __builtin_bit_cast(uint32_t, o[2]), __builtin_bit_cast(uint32_t, o[3]));
          store_nt4(dst + 4, __builtin_bit_cast(uint32_t, o[4]), __builtin_bit_cast(uint32_t, o[5]),
                    __builtin_bit_cast(uint32_t, o[6]), __builtin_bit_cast(uint32_t, o[7]));
        }
      }
    }
  }
}

// Largest |x| of a calibration input, as the bit pattern of |x| (fp32
// layout; bf16 values shifted up): for finite values the unsigned order of
// these patterns is the numeric order, and a NaN or an infinity gives a
// pattern >= 0x7F800000.  A maximum is exact and independent of the order
// of evaluation.  One partial per work-group (no same-address atomics).
__device__ __forceinline__ uint32_t absmax_u4(const uint4& w, int bf16) {
  const uint32_t q[4] = {w.x, w.y, w.z, w.w};
  uint32_t m = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (bf16)  // the pair's high and low values, each as |x| in the fp32 layout
      m = max(m, max(q[j] & 0x7FFF0000u, (q[j] << 16) & 0x7FFF0000u));
    else
      m = max(m, q[j] & 0x7FFFFFFFu);
  }
  return m;
}

__global__ __launch_bounds__(256) void absmax_k(const void* x, int bf16, uint64_t n, uint32_t* partials) {
  __shared__ uint32_t s_w[4];
  const uint4* p = reinterpret_cast<const uint4*>(x);
  const uint64_t n4 = bf16 ? n / 8 : n / 4;  // n is a multiple of 128
  const uint64_t stride = (uint64_t)gridDim.x * 256u;
  uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + 3 * stride < n4; i += 4 * stride) {
    const uint4 w0 = p[i], w1 = p[i + stride], w2 = p[i + 2 * stride], w3 = p[i + 3 * stride];
    acc = max(acc, max(max(absmax_u4(w0, bf16), absmax_u4(w1, bf16)), max(absmax_u4(w2, bf16), absmax_u4(w3, bf16))));
  }
  for (; i < n4; i += stride) acc = max(acc, absmax_u4(p[i], bf16));
  for (int o = 32; o >= 1; o >>= 1) acc = max(acc, (uint32_t)__shfl_xor((int)acc, o));
  if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) partials[blockIdx.x] = max(max(s_w[0], s_w[1]), max(s_w[2], s_w[3]));
}

__global__ __launch_bounds__(1024) void reduce_max_k(const uint32_t* p, uint32_t n, uint32_t* out) {
  __shared__ uint32_t s[1024];
  const uint32_t tid = threadIdx.x;
  uint32_t acc = 0u;
  for (uint32_t i = tid; i < n; i += 1024u) acc = max(acc, p[i]);
  s[tid] = acc;
  __syncthreads();
  for (int w = 512; w >= 1; w >>= 1) {
    if ((int)tid < w) s[tid] = max(s[tid], s[tid + w]);
    __syncthreads();
  }
  if (tid == 0) *out = s[0];
}

// One work-group of 1024 threads sums p[0..n) in a fixed order (eight loads
// in flight per thread).
template <typename T>
__global__ __launch_bounds__(1024) void reduce_k(const T* p, uint32_t n, T* out) {
  __shared__ T s[1024];
  const uint32_t tid = threadIdx.x;
  T acc = 0;
  uint32_t i = tid;
  for (; i + 7u * 1024u < n; i += 8u * 1024u) {
    T v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = p[i + 1024u * j];
    acc += ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
  }
  for (; i < n; i += 1024u) acc += p[i];
  s[tid] = acc;
  __syncthreads();
  for (int w = 512; w >= 1; w >>= 1) {
    if ((int)tid < w) s[tid] += s[tid + w];
    __syncthreads();
  }
  if (tid == 0) *out = s[0];
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int L, bool DITHER, int IN>
static hipError_t launch_encode_t(EncArgs a, bool len_only, hipStream_t st) {
  const dim3 grid(a.n_chunks);
  if (len_only) {
    hipLaunchKernelGGL((encode_k<L, DITHER, IN, true>), grid, dim3(256), 0, st, a);
    hipLaunchKernelGGL(reduce_k<unsigned long long>, dim3(1), dim3(1024), 0, st,
                       (const unsigned long long*)a.partials, a.n_chunks, &a.ws->bits);
    return hipGetLastError();
  }
  a.direct = a.n_chunks == 1;  // one chunk: encode_k writes the stream itself
  hipLaunchKernelGGL((encode_k<L, DITHER, IN, false>), grid, dim3(256), 0, st, a);
  if (a.direct) return hipGetLastError();
  const bool self_scan = a.n_chunks <= kSelfScanChunks;
  // step 2 (two-level): Eloc (u32 per chunk, padded to a multiple of 4) at
  // the start of the E region, the block prefixes (u64) after it
  uint32_t* eloc = reinterpret_cast<uint32_t*>(a.E);
  uint64_t* blockpre = a.E + ((a.n_chunks + 3) / 4) * 2;
  if (!self_scan) {
    const uint32_t nb = (a.n_chunks + kScanBlock - 1) / kScanBlock;
    hipLaunchKernelGGL(blocksum_k, dim3(nb), dim3(256), 0, st, (const uint32_t*)a.agg, a.n_chunks, eloc, blockpre);
    // up to 64 blocks the placement sums the totals itself (one launch fewer)
    if (nb > 64) hipLaunchKernelGGL(blockscan_k, dim3(1), dim3(1024), 0, st, blockpre, nb);
  }
  a.block_totals = !self_scan && (a.n_chunks + kScanBlock - 1) / kScanBlock <= 64;
  a.eloc = eloc;
  a.blockpre = blockpre;
  const dim3 pgrid((a.n_chunks + kPlaceChunks - 1) / kPlaceChunks);
  // rate-sized slots take the placement that can encode a chunk again; with
  // full-size slots every chunk is staged and the lean one runs
  const bool redo = a.slot_words < (uint32_t)kSlotWords;
  if (self_scan) {
    if (redo) hipLaunchKernelGGL((place_k<L, DITHER, IN, true, true>), pgrid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((place_k<L, DITHER, IN, true, false>), pgrid, dim3(256), 0, st, a);
  } else {
    if (redo) hipLaunchKernelGGL((place_k<L, DITHER, IN, false, true>), pgrid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((place_k<L, DITHER, IN, false, false>), pgrid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_encode(int lat, bool dither, int in, bool len_only, const EncArgs& a, hipStream_t st) {
#define HQ_ENC(LL)                                                                        \
  if (lat == LL) {                                                                        \
    if (dither) return in == 1   ? launch_encode_t<LL, true, 1>(a, len_only, st)          \
                       : in == 2 ? launch_encode_t<LL, true, 2>(a, len_only, st)          \
                                 : launch_encode_t<LL, true, 0>(a, len_only, st);         \
    return in == 1   ? launch_encode_t<LL, false, 1>(a, len_only, st)                     \
           : in == 2 ? launch_encode_t<LL, false, 2>(a, len_only, st)                     \
                     : launch_encode_t<LL, false, 0>(a, len_only, st);                    \
  }
  HQ_ENC(0) HQ_ENC(1) HQ_ENC(2) HQ_ENC(3)
#undef HQ_ENC
  return hipErrorInvalidValue;
}

template <int L, bool DITHER>
static hipError_t launch_decode_t(const DecArgs& a, int out, dim3 grid, hipStream_t st) {
  if (out == kOutBf16) hipLaunchKernelGGL((decode_k<L, DITHER, kOutBf16>), grid, dim3(256), 0, st, a);
  else if (out == kOutF32) hipLaunchKernelGGL((decode_k<L, DITHER, kOutF32>), grid, dim3(256), 0, st, a);
  else if (out == kOutRot) hipLaunchKernelGGL((decode_k<L, DITHER, kOutRot>), grid, dim3(256), 0, st, a);
  else if constexpr (DITHER) hipLaunchKernelGGL((decode_k<L, true, kOutScores>), grid, dim3(256), 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode(int lat, bool dither, int out, const DecArgs& a, dim3 grid, hipStream_t st) {
#define HQ_DEC(LL)                                                                        \
  if (lat == LL) return dither ? launch_decode_t<LL, true>(a, out, grid, st)              \
                               : launch_decode_t<LL, false>(a, out, grid, st);
  HQ_DEC(0) HQ_DEC(1) HQ_DEC(2) HQ_DEC(3)
#undef HQ_DEC
  return hipErrorInvalidValue;
}

// ===========================================================================
// Attention over compressed keys and values
// ===========================================================================
// A copy of x that the compiler cannot see through: values derived from it
// inside a loop are recomputed there instead of being hoisted and held in
// registers for the whole loop.
__device__ __forceinline__ int opaque_int(int x) {
  int y;
  asm volatile("v_mov_b32 %0, %1" : "=v"(y) : "v"(x));
  return y;
}

// Parse the lane's 8 values of chunk slot `slot` from the staged stream and
// subtract the tile's dither: u_hat in the rotated domain; zeros for a record
// that does not parse (status 5) or a slot past the end.
template <int L>
__device__ __forceinline__ void attn_parse(const uint32_t* s_stage, const uint64_t* s_off, const uint32_t* s_k,
                                           uint64_t w_first, bool span_ok, bool valid, int slot, uint64_t tile_id,
                                           uint32_t key0, uint32_t key1, int v, int r, int lane, uint32_t* ust,
                                           WsHeader* ws, float pv[8], const uint8_t* sel_lut) {
  constexpr uint32_t RAW = Lat<L>::raw;
  constexpr uint32_t MAXREC = RAW + 128u * 23u;
#pragma unroll
  for (int i = 0; i < 8; ++i) pv[i] = 0.0f;
  if (!valid) return;
  const uint64_t o0 = s_off[slot], o1 = s_off[slot + 1];
  const uint32_t k = s_k[slot];
  const uint64_t Lr = o1 - o0;
  const bool ok = span_ok && k <= (uint32_t)kKMax && Lr >= RAW + 128u * (1u + k) && Lr <= MAXREC;
  bool good = false;
  if (ok) good = parse_lane<L>(s_stage, (uint32_t)(o0 - 32 * w_first), (uint32_t)Lr, k, v, r, lane, ust, pv, sel_lut);
  if (!good) {
    if (r == 0) set_status(ws, 5);
#pragma unroll
    for (int i = 0; i < 8; ++i) pv[i] = 0.0f;
  } else {
    float d[8];
    dither_lane<L>(key0, key1, tile_id, v, d);
#pragma unroll
    for (int i = 0; i < 8; ++i) pv[i] = pv[i] - d[i];
  }
}

// Attention, step 1: one KV head (blockIdx.y), up to kAttnQ of its queries
// (blockIdx.z) and a group of up to kAttnChunks chunks of 32 keys (blockIdx.x).
// Phase 1: every key's score s = scale * c_dec_K <H D q, u_hat_K> for the
// queries (rotated once) into LDS.  Then per query the group maximum m, the
// weights e^(s - m) and their sum l.  Phase 2: the values' u_hat_V weighted
// and summed in the rotated domain: each pass's 16 parsed vectors go through
// LDS, and thread (i, half) adds coordinate i of the keys of its half of the
// pass for every query, so the running sums take 4 registers per thread.
// Writes per query (m, l, 128 weighted sums).  All sums run in a fixed order.
template <int L>
__global__ __launch_bounds__(256) void attn_k(AttnArgs a) {
  constexpr uint32_t kKeys = kAttnChunks * kChunkTiles;  // keys per group
  static_assert(kAttnQ == 4, "one float4 of weights per key");
  __shared__ __align__(16) uint32_t s_stage[kStageWords];
  __shared__ uint64_t s_off[kChunkTiles + 1];
  __shared__ uint32_t s_k[kChunkTiles];
  __shared__ uint32_t s_ust[16][16];
  __shared__ __align__(16) float s_qv[16][kTile];  // rotated queries (phase 1), a pass's values (phase 2)
  __shared__ float4 s_w[kKeys];                    // per key: the queries' scores, then weights
  __shared__ float s_ml[2][4][kAttnQ];            // per wave: maximum, then sum
  __shared__ uint2 s_sel[256];                     // bit-select table

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, grp = lane >> 4, r = lane & 15;
  const int v = lane_vector(r);
  const FwhtSigns fs = fwht_signs(v);
  const uint64_t head = blockIdx.y;
  const uint64_t s_first = (uint64_t)blockIdx.x * kKeys;  // first key of the group
  const uint32_t nkeys = (uint32_t)(a.seq - s_first < (uint64_t)kKeys ? a.seq - s_first : kKeys);
  const uint32_t nch = (nkeys + kChunkTiles - 1) / kChunkTiles;
  const uint32_t q0 = blockIdx.z * kAttnQ;  // first query of this work-group
  const uint32_t nq = a.qph - q0 < kAttnQ ? a.qph - q0 : kAttnQ;
  float* s_wf = reinterpret_cast<float*>(s_w);
  float (*s_q)[kTile] = s_qv;
  float (*s_v)[kTile] = s_qv;
  s_sel[tid] = reinterpret_cast<const uint2*>(&kSelectLut)[tid];  // visible after the first barrier below

  if (wv == 0 && grp < (int)nq) {  // rotate the queries: q~ = H D q (row-uniform branch)
    const float* qp = a.q + ((head * a.qph + q0 + grp) * kTile + 8 * v);
    if (a.q_rot) {  // a dense rotation: the queries arrive rotated, q~ = Q q
#pragma unroll
      for (int i = 0; i < 8; ++i) s_q[grp][8 * v + i] = qp[i];
    } else {
      const uint32_t sm = lane_signs32(a.sl32, v);
      float xq[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) xq[i] = __builtin_bit_cast(float, fbits(qp[i]) ^ ((sm << i) & 0x80000000u));
      fwht_tile(xq, fs);
#pragma unroll
      for (int i = 0; i < 8; ++i) s_q[grp][8 * v + i] = xq[i] * fs.lane_sign;
    }
  } else if (wv == 0) {  // unused query rows score zero
#pragma unroll
    for (int i = 0; i < 8; ++i) s_q[grp][8 * v + i] = 0.0f;
  }
  const float kscale = a.ck * a.scale;

  // ---- phase 1: scores
#pragma unroll 1
  for (uint32_t cc = 0; cc < nch; ++cc) {
    // lane indices from an opaque copy of the thread index: what the parse
    // derives from them is recomputed per chunk instead of held across the loop
    const int tid = opaque_int(threadIdx.x), lane = tid & 63, wv = tid >> 6, grp = lane >> 4, r = lane & 15;
    const int v = lane_vector(r), pslot = wv * 4 + grp;
    const uint64_t s0 = s_first + cc * kChunkTiles;
    const uint32_t nt = (uint32_t)(a.seq - s0 < (uint64_t)kChunkTiles ? a.seq - s0 : kChunkTiles);
    const uint64_t t_first = head * a.seq + s0;
    __syncthreads();  // the previous chunk's span is parsed
    if (tid <= (int)nt) s_off[tid] = a.ko[t_first + tid];
    if (tid < (int)nt) s_k[tid] = a.kk[t_first + tid];
    __syncthreads();
    uint64_t w_first;
    const bool span_ok = stage_chunk(a.kw, a.kn, s_off, nt, s_stage, w_first, tid);
    __syncthreads();
#pragma unroll 1
    for (int p = 0; p < kPasses; ++p) {
      const int slot = p * 16 + pslot;
      const bool valid = slot < (int)nt;
      float pv[8];
      attn_parse<L>(s_stage, s_off, s_k, w_first, span_ok, valid, slot, a.ktb + t_first + slot, a.key0, a.key1, v, r,
                    lane, s_ust[pslot], a.ws, pv,
                    reinterpret_cast<const uint8_t*>(s_sel));
#pragma unroll
      for (int g = 0; g < (int)kAttnQ; ++g) {
        float d = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) d = __builtin_fmaf(s_q[g][8 * v + i], pv[i], d);
        d = row_sum_f32(d);
        if (r == 0 && valid) s_wf[(cc * kChunkTiles + slot) * kAttnQ + g] = d * kscale;
      }
    }
  }
  __syncthreads();
  // ---- group maximum, weights e^(s - m) (zero past the last key), their sum (thread i: key i)
  const float4 s4 = tid < (int)nkeys ? s_w[tid] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  const float sg[kAttnQ] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
  for (int g = 0; g < (int)kAttnQ; ++g) {
    float mx = tid < (int)nkeys ? sg[g] : -__builtin_inff();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, o));
    if (lane == 0) s_ml[0][wv][g] = mx;
  }
  __syncthreads();
  float mgrp[kAttnQ], wt[kAttnQ];
#pragma unroll
  for (int g = 0; g < (int)kAttnQ; ++g) {
    mgrp[g] = __builtin_fmaxf(__builtin_fmaxf(s_ml[0][0][g], s_ml[0][1][g]), __builtin_fmaxf(s_ml[0][2][g], s_ml[0][3][g]));
    wt[g] = tid < (int)nkeys ? __expf(sg[g] - mgrp[g]) : 0.0f;
    float l = wt[g];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) l += __shfl_xor(l, o);
    if (lane == 0) s_ml[1][wv][g] = l;
  }
  s_w[tid] = make_float4(wt[0], wt[1], wt[2], wt[3]);  // 256 threads, kKeys = 256 keys

  // ---- phase 2: weighted value sums
  float acc[kAttnQ] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 1
  for (uint32_t cc = 0; cc < nch; ++cc) {
    // lane indices from an opaque copy of the thread index: what the parse
    // derives from them is recomputed per chunk instead of held across the loop
    const int tid = opaque_int(threadIdx.x), lane = tid & 63, wv = tid >> 6, grp = lane >> 4, r = lane & 15;
    const int v = lane_vector(r), pslot = wv * 4 + grp;
    const uint64_t s0 = s_first + cc * kChunkTiles;
    const uint32_t nt = (uint32_t)(a.seq - s0 < (uint64_t)kChunkTiles ? a.seq - s0 : kChunkTiles);
    const uint64_t t_first = head * a.seq + s0;
    __syncthreads();  // weights visible; the previous chunk's span is parsed
    if (tid <= (int)nt) s_off[tid] = a.vo[t_first + tid];
    if (tid < (int)nt) s_k[tid] = a.vk[t_first + tid];
    __syncthreads();
    uint64_t w_first;
    const bool span_ok = stage_chunk(a.vw, a.vn, s_off, nt, s_stage, w_first, tid);
    __syncthreads();
#pragma unroll 1
    for (int p = 0; p < kPasses; ++p) {
      const int slot = p * 16 + pslot;
      const bool valid = slot < (int)nt;
      float pv[8];
      attn_parse<L>(s_stage, s_off, s_k, w_first, span_ok, valid, slot, a.vtb + t_first + slot, a.key0, a.key1, v, r,
                    lane, s_ust[pslot], a.ws, pv,
                    reinterpret_cast<const uint8_t*>(s_sel));
      float4* vr = reinterpret_cast<float4*>(&s_v[pslot][8 * v]);  // zeros past the last key
      vr[0] = make_float4(pv[0], pv[1], pv[2], pv[3]);
      vr[1] = make_float4(pv[4], pv[5], pv[6], pv[7]);
      __syncthreads();
      const int ci = tid & (kTile - 1), half = tid >> 7;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = half * 8 + j;
        const float4 w = s_w[cc * kChunkTiles + p * 16 + row];  // zero past the last key
        const float x = s_v[row][ci];
        acc[0] = __builtin_fmaf(w.x, x, acc[0]);
        acc[1] = __builtin_fmaf(w.y, x, acc[1]);
        acc[2] = __builtin_fmaf(w.z, x, acc[2]);
        acc[3] = __builtin_fmaf(w.w, x, acc[3]);
      }
      __syncthreads();  // s_v is rewritten by the next pass
    }
  }
  // the two halves' sums (the value staging area is free)
  const int ci = tid & (kTile - 1), half = tid >> 7;
  float* s_red = &s_v[0][0];  // [kAttnQ][kTile]
  if (half == 1) {
#pragma unroll
    for (int g = 0; g < (int)kAttnQ; ++g) s_red[g * kTile + ci] = acc[g];
  }
  __syncthreads();
  float* part = a.part + ((head * a.n_groups + blockIdx.x) * a.qph + q0) * kAttnPart;
  if (half == 0) {
#pragma unroll
    for (int g = 0; g < (int)kAttnQ; ++g)
      if (g < (int)nq) part[g * kAttnPart + 2 + ci] = acc[g] + s_red[g * kTile + ci];
  }
  if (tid < (int)nq) {
    float mg = mgrp[0];
#pragma unroll
    for (int g = 1; g < (int)kAttnQ; ++g) mg = tid == g ? mgrp[g] : mg;
    part[tid * kAttnPart] = mg;
    part[tid * kAttnPart + 1] = ((s_ml[1][0][tid] + s_ml[1][1][tid]) + s_ml[1][2][tid]) + s_ml[1][3][tid];
  }
}

// Attention, step 2: one work-group of 1024 threads per query combines the
// groups of its head: M = max m_c, L = sum l_c e^(m_c - M), A = sum acc_c
// e^(m_c - M).  Thread (slice, i) sums coordinate i over the groups c = slice
// mod 8 in order; the 8 slices are then added as a fixed pairwise tree.  The
// output out = D H (c_dec_V A / L) is formed by one 16-lane row (with a dense
// rotation, c_dec_V A / L is written to rot_out and rotated back by rot_k).
__global__ __launch_bounds__(1024) void attn_combine_k(AttnArgs a) {
  __shared__ float s_red[16];
  __shared__ float s_a[8][kTile];
  __shared__ float s_l[8];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const uint32_t hg = blockIdx.x, head = hg / a.qph, g = hg % a.qph;
  const uint32_t stride = a.qph * kAttnPart;
  const float* P = a.part + ((uint64_t)head * a.n_groups * a.qph + g) * kAttnPart;
  float mx = -__builtin_inff();
  for (uint32_t c = (uint32_t)tid; c < a.n_groups; c += 1024u) mx = __builtin_fmaxf(mx, P[(uint64_t)c * stride]);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, o));
  if (lane == 0) s_red[wv] = mx;
  __syncthreads();
  float M = s_red[0];
#pragma unroll
  for (int w = 1; w < 16; ++w) M = __builtin_fmaxf(M, s_red[w]);
  const uint32_t i = (uint32_t)tid & 127u, slice = (uint32_t)tid >> 7;
  float acc = 0.0f, ls = 0.0f;
  constexpr int kB = 16;  // groups whose loads are issued together
#pragma unroll 1
  for (uint32_t c0 = slice; c0 < a.n_groups; c0 += 8u * kB) {
    float gm[kB], gl[kB], gx[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const uint32_t c = c0 + 8u * b;
      const bool in = c < a.n_groups;
      const float* pc = P + (uint64_t)(in ? c : a.n_groups - 1u) * stride;  // loads stay in bounds
      const float m = pc[0], l = pc[1], x = pc[2 + i];
      gm[b] = in ? m : -__builtin_inff();  // weight e^(-inf) = 0 past the last group
      gl[b] = in ? l : 0.0f;
      gx[b] = in ? x : 0.0f;
    }
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const float e = __expf(gm[b] - M);
      acc = __builtin_fmaf(e, gx[b], acc);
      ls = __builtin_fmaf(e, gl[b], ls);
    }
  }
  s_a[slice][i] = acc;
  if (i == 0) s_l[slice] = ls;
  __syncthreads();
  if (wv == 0) {  // row 0 of wave 0 transforms and stores; the other rows follow along
    const int r = lane & 15, v = lane_vector(r);
    const FwhtSigns fs = fwht_signs(v);
    const float l = ((s_l[0] + s_l[1]) + (s_l[2] + s_l[3])) + ((s_l[4] + s_l[5]) + (s_l[6] + s_l[7]));
    const float f = a.cv / l;
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = 8 * v + j;
      x[j] = (((s_a[0][c] + s_a[1][c]) + (s_a[2][c] + s_a[3][c])) + ((s_a[4][c] + s_a[5][c]) + (s_a[6][c] + s_a[7][c]))) *
             f;
    }
    if (a.rot_out) {  // a dense rotation: c_dec_V A / L goes to its inverse rotation (Q^T) instead
      if (lane < 16) {
        float4* o = reinterpret_cast<float4*>(a.rot_out + (uint64_t)hg * kTile + 8 * v);
        o[0] = make_float4(x[0], x[1], x[2], x[3]);
        o[1] = make_float4(x[4], x[5], x[6], x[7]);
      }
      return;
    }
    fwht_tile(x, fs);
    const uint32_t sm = lane_signs32(a.sl32, v);
    if (lane < 16) {
      float* o = a.out + (uint64_t)hg * kTile + 8 * v;
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = __builtin_bit_cast(float, fbits(x[j] * fs.lane_sign) ^ ((sm << j) & 0x80000000u));
    }
  }
}

hipError_t launch_attention(int lat, const AttnArgs& a, uint32_t n_heads, hipStream_t st) {
  const dim3 grid(a.n_groups, n_heads, (a.qph + kAttnQ - 1) / kAttnQ);
  if (lat == 0) hipLaunchKernelGGL(attn_k<0>, grid, dim3(256), 0, st, a);
  else if (lat == 1) hipLaunchKernelGGL(attn_k<1>, grid, dim3(256), 0, st, a);
  else if (lat == 2) hipLaunchKernelGGL(attn_k<2>, grid, dim3(256), 0, st, a);
  else if (lat == 3) hipLaunchKernelGGL(attn_k<3>, grid, dim3(256), 0, st, a);
  else return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_combine_k, dim3(n_heads * a.qph), dim3(1024), 0, st, a);
  return hipGetLastError();
}

// Matrix-vector products, step 1: the vectors' 128-column blocks rotated as
// the weights were, xr = H D x (exact signs, unnormalised transform), one block
// per 16-lane row, stored in natural coordinate order.
__global__ __launch_bounds__(256) void rotx_k(GemvArgs g) {
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 15;
  const int v = lane_vector(r);
  const uint32_t q = blockIdx.x * 16u + (uint32_t)(tid >> 4);  // block of all nb vectors
  const bool ok = q < g.nb * g.nblk;
  const uint32_t j = ok ? q / g.nblk : 0u, blk = ok ? q % g.nblk : 0u;
  const uint64_t base = ((uint64_t)j * g.nblk + blk) * kTile + 8 * v;
  float xv[8];
  const float4 x0 = *reinterpret_cast<const float4*>(g.x + base);
  const float4 x1 = *reinterpret_cast<const float4*>(g.x + base + 4);
  xv[0] = x0.x; xv[1] = x0.y; xv[2] = x0.z; xv[3] = x0.w;
  xv[4] = x1.x; xv[5] = x1.y; xv[6] = x1.z; xv[7] = x1.w;
  const uint32_t sm = lane_signs32(g.sl32, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) xv[i] = __builtin_bit_cast(float, fbits(xv[i]) ^ ((sm << i) & 0x80000000u));
  const FwhtSigns fs = fwht_signs(v);
  fwht_tile(xv, fs);  // every lane of the row takes part (cross-lane stages)
  if (ok) {
    float4* dst = reinterpret_cast<float4*>(g.xr + base);
    dst[0] = make_float4(xv[0] * fs.lane_sign, xv[1] * fs.lane_sign, xv[2] * fs.lane_sign, xv[3] * fs.lane_sign);
    dst[1] = make_float4(xv[4] * fs.lane_sign, xv[5] * fs.lane_sign, xv[6] * fs.lane_sign, xv[7] * fs.lane_sign);
  }
}

// Matrix-vector products, step 3: y[j][r] = c_dec * sum over the row's blocks
// of the tile dot products, one wave per (vector, row): lane l adds blocks l,
// l + 64, ... in order, then a fixed tree over the lanes.
__global__ __launch_bounds__(256) void rowsum_k(GemvArgs g) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t q = __builtin_amdgcn_readfirstlane(blockIdx.x * 4u + (threadIdx.x >> 6));
  if (q >= g.nb * g.rows) return;  // the whole wave
  const uint32_t j = q / g.rows, row = q % g.rows;
  const float* d = g.dots + (uint64_t)row * g.nblk * g.nb + j;
  float acc = 0.0f;
  for (uint32_t b = lane; b < g.nblk; b += 64u) acc += d[(uint64_t)b * g.nb];
  acc = row_sum_f32(acc);
  const int ai = __builtin_bit_cast(int, acc);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ai, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ai, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ai, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ai, 48));
  const float tot3 = ((r0 + r1) + r2) + r3;
  if (lane == 0) g.y[(uint64_t)j * g.rows + row] = tot3 * g.c_dec;
}

hipError_t launch_gemv(int lat, const DecArgs& d, const GemvArgs& g, hipStream_t st) {
  const uint32_t nq = g.nb * g.nblk;
  hipLaunchKernelGGL(rotx_k, dim3((nq + 15u) / 16u), dim3(256), 0, st, g);
  const dim3 grid((uint32_t)((d.n_tiles + kChunkTiles - 1) / kChunkTiles));
  if (lat == 0) hipLaunchKernelGGL((decode_k<0, false, kOutGemv>), grid, dim3(256), 0, st, d);
  else if (lat == 1) hipLaunchKernelGGL((decode_k<1, false, kOutGemv>), grid, dim3(256), 0, st, d);
  else if (lat == 2) hipLaunchKernelGGL((decode_k<2, false, kOutGemv>), grid, dim3(256), 0, st, d);
  else if (lat == 3) hipLaunchKernelGGL((decode_k<3, false, kOutGemv>), grid, dim3(256), 0, st, d);
  else return hipErrorInvalidValue;
  const uint32_t nw = g.nb * g.rows;
  hipLaunchKernelGGL(rowsum_k, dim3((nw + 3u) / 4u), dim3(256), 0, st, g);
  return hipGetLastError();
}

// ===========================================================================
// Matrix products Y = X W_hat^T with matrix cores
// ===========================================================================
// Each tile adds c_dec <u_hat, H D x_b> to its row's products, so Y is c_dec
// times the product of the rotated vectors (nb x cols) with the rotated codes
// U (rows x cols, integers for Z, D4 and E8), a dense contraction: bf16 MFMA
// 32x32x16 with fp32 accumulation.  Both operands are split into two bf16
// pieces, x~ = hi + lo (+ at most 2^-16 |x~|) and u = Uh + Ul (exact below
// 2^16), and hi Uh + hi Ul + lo Uh is accumulated (products of bf16 values
// are exact in fp32).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void split_bf16(const float x[8], uint4& hi, uint4& lo) {
  const f32x8_t f = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  const bf16x8_t h = __builtin_convertvector(f, bf16x8_t);
  const f32x8_t hf = __builtin_convertvector(h, f32x8_t);
  const bf16x8_t l = __builtin_convertvector(f - hf, bf16x8_t);  // x - hi is exact in fp32
  hi = __builtin_bit_cast(uint4, h);
  lo = __builtin_bit_cast(uint4, l);
}

// Step 1: the vectors' blocks rotated as the weights were (x~ = H D x, the
// butterfly of the decoder) and split; vector rows nb..nbp-1 are zero.
__global__ __launch_bounds__(256) void rotx_split_k(GemmArgs g) {
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 15;
  const int v = lane_vector(r);
  const uint32_t q = blockIdx.x * 16u + (uint32_t)(tid >> 4);  // (vector, block) of nbp x nblk
  const bool ok = q < g.nbp * g.nblk;
  const uint32_t j = ok ? q / g.nblk : 0u, blk = ok ? q % g.nblk : 0u;
  const bool in = ok && j < g.nb;
  const uint64_t src = ((uint64_t)(in ? j : 0u) * g.nblk + blk) * kTile + 8 * v;
  float xv[8];
  const float4 x0 = *reinterpret_cast<const float4*>(g.x + src);
  const float4 x1 = *reinterpret_cast<const float4*>(g.x + src + 4);
  xv[0] = x0.x; xv[1] = x0.y; xv[2] = x0.z; xv[3] = x0.w;
  xv[4] = x1.x; xv[5] = x1.y; xv[6] = x1.z; xv[7] = x1.w;
  const uint32_t sm = lane_signs32(g.sl32, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) xv[i] = __builtin_bit_cast(float, fbits(xv[i]) ^ ((sm << i) & 0x80000000u));
  const FwhtSigns fs = fwht_signs(v);
  fwht_tile(xv, fs);  // every lane of the row takes part (cross-lane stages)
#pragma unroll
  for (int i = 0; i < 8; ++i) xv[i] = in ? xv[i] * fs.lane_sign : 0.0f;
  if (ok) {
    uint4 hi, lo;
    split_bf16(xv, hi, lo);
    const uint64_t dst = ((uint64_t)j * g.nblk + blk) * kTile + 8 * v;
    const uint64_t piece = (uint64_t)g.nbp * g.nblk * kTile;
    *reinterpret_cast<uint4*>(g.xp + dst) = hi;
    *reinterpret_cast<uint4*>(g.xp + piece + dst) = lo;
  }
}

// Step 2: one work-group per 32 weight rows (blockIdx.x) and split of the
// column blocks (blockIdx.y).  Per block: the 32 tiles (one per row) are
// parsed, one per 16-lane row slot in two passes, each record staged in the
// slot's own LDS area; their codes, split, go to LDS as the B operand; then
// wave w accumulates K steps 2w and 2w+1 of the block for every 32-vector M
// tile.  The four waves' sums are added in a fixed order at the end.
template <int L, int NMT>
__global__ __launch_bounds__(256) void gemm_k(GemmArgs g) {
  constexpr uint32_t RAW = Lat<L>::raw;
  constexpr uint32_t MAXREC = RAW + 128u * 23u;
  constexpr int kBS = kTile + 8;  // B row stride (bf16): conflict-free 16-byte reads
  __shared__ __align__(16) uint32_t s_rec[16][kGemmRecWords];
  __shared__ uint32_t s_ust[16][16];
  __shared__ uint64_t s_o[33];
  __shared__ uint64_t s_o1[32];
  __shared__ uint32_t s_k[32];
  __shared__ __align__(16) uint16_t s_B[2][32][kBS];
  __shared__ uint2 s_sel[256];  // bit-select table

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  s_sel[tid] = reinterpret_cast<const uint2*>(&kSelectLut)[tid];
  const uint32_t r0 = blockIdx.x * 32u;
  const uint32_t b_lo = blockIdx.y * g.per;
  const uint32_t b_hi = b_lo + g.per < g.nblk ? b_lo + g.per : g.nblk;
  f32x16_t acc0 = {}, acc1 = {};
  const uint64_t piece = (uint64_t)g.nbp * g.nblk * kTile;
  // the 32 tiles' offsets and Rice parameters, loaded one block ahead
  const bool row_in = tid < 32 && r0 + tid < g.rows;
  const uint64_t t_row = (uint64_t)(r0 + (tid & 31)) * g.nblk;
  uint64_t nx_o = 0, nx_o1 = 0;
  uint32_t nx_k = 0;
  if (row_in && b_lo < b_hi) {
    nx_o = g.offsets[t_row + b_lo];
    nx_o1 = g.offsets[t_row + b_lo + 1];
    nx_k = g.k[t_row + b_lo];
  }

#pragma unroll 1
  for (uint32_t b = b_lo; b < b_hi; ++b) {
    if (tid < 32) {
      s_o[tid] = nx_o;
      s_o1[tid] = nx_o1;
      s_k[tid] = nx_k;
    }
    __syncthreads();  // (also: the previous block's B operand is consumed)
    if (row_in && b + 1 < b_hi) {
      nx_o = g.offsets[t_row + b + 1];
      nx_o1 = g.offsets[t_row + b + 2];
      nx_k = g.k[t_row + b + 1];
    }
    // lane indices from an opaque copy of the thread index: what the parse
    // derives from them is recomputed per block instead of held across the loop
    const int tid = opaque_int(threadIdx.x), lane = tid & 63, wv = tid >> 6, grp = lane >> 4, r = lane & 15;
    const int v = lane_vector(r), pslot = wv * 4 + grp;
#pragma unroll 1
    for (int p = 0; p < 2; ++p) {
      const int i = p * 16 + pslot;  // tile row within the 32
      const bool valid = r0 + (uint32_t)i < g.rows;
      const uint64_t o0 = s_o[i], o1 = s_o1[i];
      const uint32_t kk = s_k[i];
      const uint64_t Lr = o1 - o0;
      const uint64_t w_first = o0 >> 5, w_end = (o1 + 31) >> 5;
      const bool ok = valid && o1 >= o0 && kk <= (uint32_t)kKMax && Lr >= RAW + 128u * (1u + kk) && Lr <= MAXREC &&
                      w_end <= g.n_words;
      const uint32_t n = ok ? (uint32_t)(w_end - w_first) : 0u;  // <= 94
      uint32_t* sr = s_rec[pslot];
#pragma unroll
      for (int q = 0; q < (int)kGemmRecWords / 16; ++q) {
        const uint32_t w = (uint32_t)r + 16u * q;
        sr[w] = w < n ? g.words[w_first + w] : 0u;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = 0.0f;
      bool good = false;
      if (ok) good = parse_lane<L>(sr, (uint32_t)(o0 & 31u), (uint32_t)Lr, kk, v, r, lane, s_ust[pslot],
                                   pv, reinterpret_cast<const uint8_t*>(s_sel));
      if (valid && !good) {
        if (r == 0) set_status(g.ws, 5);
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = 0.0f;
      }
      uint4 hi, lo;
      split_bf16(pv, hi, lo);
      *reinterpret_cast<uint4*>(&s_B[0][i][8 * v]) = hi;
      *reinterpret_cast<uint4*>(&s_B[1][i][8 * v]) = lo;
    }
    __syncthreads();
    // matrix cores: B[k][j] = code k of row r0 + j (lane j + 32 (k / 8), element k % 8)
    const int bj = lane & 31, bk = 8 * (lane >> 5);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int k0 = 16 * (2 * wv + st);
      const bf16x8_t Bh = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(&s_B[0][bj][k0 + bk]));
      const bf16x8_t Bl = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(&s_B[1][bj][k0 + bk]));
      // A[i][k] = x~ of vector 32 mt + i (lane i + 32 (k / 8), element k % 8)
      const uint64_t ai = (uint64_t)bj * g.nblk * kTile + (uint64_t)b * kTile + k0 + bk;
      {
        const bf16x8_t Ah = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(g.xp + ai));
        const bf16x8_t Al = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(g.xp + piece + ai));
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ah, Bh, acc0, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ah, Bl, acc0, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Al, Bh, acc0, 0, 0, 0);
      }
      if constexpr (NMT > 1) {
        const uint64_t a1 = ai + (uint64_t)32 * g.nblk * kTile;
        const bf16x8_t Ah = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(g.xp + a1));
        const bf16x8_t Al = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(g.xp + piece + a1));
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ah, Bh, acc1, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ah, Bl, acc1, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Al, Bh, acc1, 0, 0, 0);
      }
    }
  }
  // the four waves' sums, per M tile, through LDS (the B area is free):
  // D[i][j] sits in lane j + 32 ((i / 4) % 2), register 4 (i / 8) + i % 4
  float* s_red = reinterpret_cast<float*>(&s_B[0][0][0]);  // [4 waves][32][32]
#pragma unroll
  for (uint32_t mt = 0; mt < (uint32_t)NMT; ++mt) {
    const f32x16_t a = mt == 0 ? acc0 : acc1;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int i = 8 * (q / 4) + 4 * (lane >> 5) + (q % 4), j = lane & 31;
      s_red[(wv * 32 + i) * 32 + j] = a[q];
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + 256 * e, i = idx >> 5, j = idx & 31;
      const float sum = ((s_red[(0 * 32 + i) * 32 + j] + s_red[(1 * 32 + i) * 32 + j]) + s_red[(2 * 32 + i) * 32 + j]) +
                        s_red[(3 * 32 + i) * 32 + j];
      const uint32_t m = 32u * mt + (uint32_t)i, row = r0 + (uint32_t)j;
      if (row < g.rows) {
        if (g.splits == 1) {
          if (m < g.nb) g.y[(uint64_t)m * g.rows + row] = sum * g.c_dec;
        } else {
          g.part[((uint64_t)blockIdx.y * g.nbp + m) * g.rows + row] = sum;
        }
      }
    }
  }
}

// Step 3 (more than one split): y = c_dec * (the splits' sums in order).
__global__ __launch_bounds__(256) void gemm_sum_k(GemmArgs g) {
  const uint64_t q = (uint64_t)blockIdx.x * 256u + threadIdx.x;
  if (q >= (uint64_t)g.nb * g.rows) return;
  const uint64_t stride = (uint64_t)g.nbp * g.rows;
  float s = g.part[q];
  for (uint32_t sp = 1; sp < g.splits; ++sp) s += g.part[sp * stride + q];
  g.y[q] = s * g.c_dec;
}

hipError_t launch_gemm(int lat, const GemmArgs& g, hipStream_t st) {
  const uint32_t nq = g.nbp * g.nblk;
  hipLaunchKernelGGL(rotx_split_k, dim3((nq + 15u) / 16u), dim3(256), 0, st, g);
  const dim3 grid((g.rows + 31u) / 32u, g.splits);
  const bool two = g.nbp > 32u;
  if (lat == 0) {
    if (two) hipLaunchKernelGGL((gemm_k<0, 2>), grid, dim3(256), 0, st, g);
    else hipLaunchKernelGGL((gemm_k<0, 1>), grid, dim3(256), 0, st, g);
  } else if (lat == 2) {
    if (two) hipLaunchKernelGGL((gemm_k<2, 2>), grid, dim3(256), 0, st, g);
    else hipLaunchKernelGGL((gemm_k<2, 1>), grid, dim3(256), 0, st, g);
  } else if (lat == 3) {
    if (two) hipLaunchKernelGGL((gemm_k<3, 2>), grid, dim3(256), 0, st, g);
    else hipLaunchKernelGGL((gemm_k<3, 1>), grid, dim3(256), 0, st, g);
  } else {
    return hipErrorInvalidValue;
  }
  if (g.splits > 1) {
    const uint64_t n = (uint64_t)g.nb * g.rows;
    hipLaunchKernelGGL(gemm_sum_k, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, st, g);
  }
  return hipGetLastError();
}

// ===========================================================================
// Dense rotation (the Haar matrix): y_i = fl32(t_i * scale) with t_i the fp32
// fma chain over j = 0..127 of M[i][j] x_j, in index order, for every tile.
// Persistent work-groups of 512 threads, one per CU: the matrix (as Mt[j][i],
// 64 KB) is loaded into LDS once; per round of kRotTiles = 128 tiles the
// inputs go to LDS transposed (Xt[j][t], 64 KB), and thread (coordinates
// 4c..4c+3, tiles 8g..8g+7) keeps 32 chains.  Per step it reads one float4 of
// Mt (32 distinct per half-wave) and two of Xt (the same for a half-wave: a
// broadcast): 48 bytes of LDS per 32 fma, so the vector ALUs, not the LDS,
// bound it.
// ===========================================================================
constexpr uint32_t kRotTiles = 128;
__global__ __launch_bounds__(512) void rot_k(RotArgs a) {
  __shared__ __align__(16) float s_m[kTile * kTile];      // Mt[128][128]
  __shared__ __align__(16) float s_x[kTile * kRotTiles];  // Xt[128][128]
  const uint32_t tid = threadIdx.x;
  for (uint32_t i = tid; i < kTile * kTile / 4; i += 512u)
    reinterpret_cast<float4*>(s_m)[i] = reinterpret_cast<const float4*>(a.mt)[i];
  const uint64_t n_rounds = (a.n_tiles + kRotTiles - 1) / kRotTiles;
  const uint32_t c4 = 4u * (tid & 31u), g8 = 8u * (tid >> 5);
  for (uint64_t rd = blockIdx.x; rd < n_rounds; rd += gridDim.x) {
    // inputs: thread -> tile tid / 4, coordinates 32 (tid % 4) .. + 31
    {
      const uint32_t tt = tid >> 2, j0 = 32u * (tid & 3u);
      const uint64_t t = rd * kRotTiles + tt;
      float xv[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) xv[e] = 0.0f;
      if (t < a.n_tiles) {
        if (a.in_bf16) {
          const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.x) + t * kTile + j0);
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const uint4 w = p[h];
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              xv[8 * h + 2 * e] = __builtin_bit_cast(float, ww[e] << 16);
              xv[8 * h + 2 * e + 1] = __builtin_bit_cast(float, ww[e] & 0xFFFF0000u);
            }
          }
        } else {
          const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.x) + t * kTile + j0);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float4 f = p[e];
            xv[4 * e] = f.x; xv[4 * e + 1] = f.y; xv[4 * e + 2] = f.z; xv[4 * e + 3] = f.w;
          }
        }
      }
      __syncthreads();  // (the matrix is in; the previous round's inputs are consumed)
#pragma unroll
      for (int e = 0; e < 32; ++e) s_x[(j0 + e) * kRotTiles + tt] = xv[e];
    }
    __syncthreads();
    float acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[i][k] = 0.0f;
#pragma unroll 2
    for (uint32_t j = 0; j < kTile; ++j) {
      const float4 m = *reinterpret_cast<const float4*>(s_m + j * kTile + c4);
      const float4 x0 = *reinterpret_cast<const float4*>(s_x + j * kRotTiles + g8);
      const float4 x1 = *reinterpret_cast<const float4*>(s_x + j * kRotTiles + g8 + 4u);
      const float mv[4] = {m.x, m.y, m.z, m.w}, xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[i][k] = __builtin_fmaf(mv[i], xw[k], acc[i][k]);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint64_t t = rd * kRotTiles + g8 + (uint32_t)k;
      if (t >= a.n_tiles) continue;
      const float o0 = acc[0][k] * a.scale, o1 = acc[1][k] * a.scale, o2 = acc[2][k] * a.scale,
                  o3 = acc[3][k] * a.scale;
      if (a.out_bf16) {
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        typedef float f32x2_t __attribute__((ext_vector_type(2)));
        const f32x2_t f01 = {o0, o1}, f23 = {o2, o3};
        const uint2 pk = make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(f01, bf16x2_t)),
                                    __builtin_bit_cast(uint32_t, __builtin_convertvector(f23, bf16x2_t)));
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.y) + t * kTile + c4) = pk;
      } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.y) + t * kTile + c4) = make_float4(o0, o1, o2, o3);
      }
    }
  }
}

hipError_t launch_rot(const RotArgs& a, hipStream_t st) {
  const uint64_t n_rounds = (a.n_tiles + kRotTiles - 1) / kRotTiles;
  const uint32_t grid = (uint32_t)(n_rounds < 256 ? n_rounds : 256);  // one work-group per CU (128 KB of LDS)
  hipLaunchKernelGGL(rot_k, dim3(grid), dim3(512), 0, st, a);
  return hipGetLastError();
}

// ===========================================================================
// Compact side information: per chunk of 32 tiles a 96-byte record
//   [0, 8)   uint64 bit offset of the chunk's first record
//   [8, 72)  uint16 end of record j minus that offset, j = 0..31
//   [72, 92) the 32 Rice parameters, 5 bits each, LSB first
//   [92, 96) zero
// (entries past the last tile are zero): 3 bytes per tile instead of 9.
// ===========================================================================
__global__ __launch_bounds__(256) void side_pack_k(const uint64_t* offsets, const uint8_t* kin, uint64_t n,
                                                   uint8_t* side, WsHeader* ws) {
  __shared__ uint32_t s_kw[8][5];
  const uint32_t tid = threadIdx.x, j = tid & 31u, cl = tid >> 5;
  const uint64_t t = (uint64_t)blockIdx.x * 256u + tid, c = t >> 5;
  const uint64_t n_chunks = (n + 31) >> 5;
  if (tid < 40) (&s_kw[0][0])[tid] = 0u;
  __syncthreads();
  const bool in_chunk = c < n_chunks, valid = t < n;
  uint8_t* rec = side + c * 96u;
  if (in_chunk) {
    const uint64_t base = offsets[c << 5];
    const uint64_t delta = valid ? offsets[t + 1] - base : 0ull;
    if (valid && delta > 0xFFFFull) set_status(ws, 4);
    reinterpret_cast<uint16_t*>(rec + 8)[j] = (uint16_t)delta;
    if (j == 0) *reinterpret_cast<uint64_t*>(rec) = base;
    const uint32_t kk = valid ? (uint32_t)kin[t] & 31u : 0u, p = 5u * j;
    atomicOr(&s_kw[cl][p >> 5], kk << (p & 31u));
    if ((p & 31u) > 27u) atomicOr(&s_kw[cl][(p >> 5) + 1u], kk >> (32u - (p & 31u)));
  }
  __syncthreads();
  if (in_chunk && j < 6) reinterpret_cast<uint32_t*>(rec + 72)[j] = j < 5 ? s_kw[cl][j] : 0u;
}

__global__ __launch_bounds__(256) void side_unpack_k(const uint8_t* side, uint64_t n, uint64_t* offsets,
                                                     uint8_t* kout) {
  const uint64_t t = (uint64_t)blockIdx.x * 256u + threadIdx.x;
  if (t >= n) return;
  const uint32_t j = (uint32_t)(t & 31u);
  const uint8_t* rec = side + (t >> 5) * 96u;
  const uint64_t base = *reinterpret_cast<const uint64_t*>(rec);
  const uint16_t* d = reinterpret_cast<const uint16_t*>(rec + 8);
  offsets[t] = j == 0 ? base : base + d[j - 1];
  if (t == n - 1) offsets[n] = base + d[j];
  const uint32_t* kw = reinterpret_cast<const uint32_t*>(rec + 72);
  const uint32_t p = 5u * j;
  uint32_t kk = kw[p >> 5] >> (p & 31u);
  if ((p & 31u) > 27u) kk |= kw[(p >> 5) + 1u] << (32u - (p & 31u));
  kout[t] = (uint8_t)(kk & 31u);
}

hipError_t launch_side(bool pack, const uint64_t* offsets_in, const uint8_t* k_in, const uint8_t* side_in,
                       uint64_t n, uint8_t* side_out, uint64_t* offsets_out, uint8_t* k_out, WsHeader* ws,
                       hipStream_t st) {
  const dim3 grid((uint32_t)((n + 255) / 256));
  if (pack) hipLaunchKernelGGL(side_pack_k, grid, dim3(256), 0, st, offsets_in, k_in, n, side_out, ws);
  else hipLaunchKernelGGL(side_unpack_k, grid, dim3(256), 0, st, side_in, n, offsets_out, k_out);
  return hipGetLastError();
}

// One uint64 written by a kernel (the offsets[0] = 0 of an empty stream): a
// launch instead of hipMemsetAsync, so that a captured graph holds no memset
// node.
__global__ void set_u64_k(uint64_t* p, uint64_t v) { *p = v; }

hipError_t launch_set_u64(uint64_t* p, uint64_t v, hipStream_t st) {
  hipLaunchKernelGGL(set_u64_k, dim3(1), dim3(1), 0, st, p, v);
  return hipGetLastError();
}

hipError_t launch_absmax(const void* x, bool bf16, uint64_t n, uint32_t* partials, uint32_t max_blocks, uint32_t* out,
                         hipStream_t st) {
  uint64_t blocks = (n + 255) / 256;
  if (blocks > max_blocks) blocks = max_blocks;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(absmax_k, dim3((uint32_t)blocks), dim3(256), 0, st, x, bf16 ? 1 : 0, n, partials);
  hipLaunchKernelGGL(reduce_max_k, dim3(1), dim3(1024), 0, st, (const uint32_t*)partials, (uint32_t)blocks, out);
  return hipGetLastError();
}

}  // namespace hq
