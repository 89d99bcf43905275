// hq_kernels.hip -- HIP kernels of the HyperQuant per-tile codec for gfx950.
//
// encode_k  : RHT -> (dither) -> nearest point -> strip -> zigzag -> Rice k ->
//             tile lengths -> work-group scan -> single-pass decoupled look-back
//             for the global bit offset -> LDS bit assembly -> coalesced stores.
//             [HQ Methodology 1-4; decoupled look-back after Merrill & Garland,
//             "Single-pass Parallel Prefix Scan with Decoupled Look-back", 2016]
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

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Load the lane's 8 coordinates of tile t (fp32 or bf16), signs of D applied.
template <bool BF16>
__device__ __forceinline__ void load_lane(const void* x, uint64_t t, int v, const uint32_t smask[8], float xv[8]) {
  if constexpr (BF16) {
    const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + t * kTile + 8 * v);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t s = ww[i] ^ smask[i];  // sign bits 15 and 31 of the pair
      xv[2 * i] = bf16_lo(s);
      xv[2 * i + 1] = bf16_hi(s);
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(x) + t * kTile + 8 * v);
    const uint4 w0 = p[0], w1 = p[1];
    const uint32_t ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) xv[i] = __builtin_bit_cast(float, ww[i] ^ smask[i]);
  }
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

// OR a value of up to 64 bits into the LDS bit stream at bit P (stream word i
// lives at s[1 + i]; s[0] holds the predecessor's tail).
__device__ __forceinline__ void lds_or64(uint32_t* s, uint32_t P, uint32_t lo, uint32_t hi) {
  const uint32_t w = 1 + (P >> 5), sh = P & 31;
  if (sh == 0) {
    if (lo) atomicOr(&s[w], lo);
    if (hi) atomicOr(&s[w + 1], hi);
  } else {
    const uint32_t x0 = lo << sh;
    const uint32_t x1 = __builtin_amdgcn_alignbit(hi, lo, 32 - sh);
    const uint32_t x2 = hi >> (32 - sh);
    if (x0) atomicOr(&s[w], x0);
    if (x1) atomicOr(&s[w + 1], x1);
    if (x2) atomicOr(&s[w + 2], x2);
  }
}

__device__ __forceinline__ uint32_t rev4(uint32_t n) {
  return ((n & 1u) << 3) | ((n & 2u) << 1) | ((n & 4u) >> 1) | ((n & 8u) >> 3);
}

// ===========================================================================
// Encode
// ===========================================================================
// Per-lane constants of a plan: butterfly signs, the scale with the lane
// sign folded in, and the sign bits of D for the lane's 8 coordinates.
template <bool BF16>
struct LaneConst {
  FwhtSigns fs;
  float scale;
  uint32_t smask[8];
  __device__ __forceinline__ LaneConst(const uint32_t sgn[4], int v, float c) {
    fs = fwht_signs(v);
    scale = fs.lane_sign * c;
    const uint32_t sbyte = (sgn[v >> 2] >> ((v & 3) * 8)) & 0xFFu;
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        smask[i] = (((sbyte >> (2 * i)) & 1u) << 15) | (((sbyte >> (2 * i + 1)) & 1u) << 31);
#pragma unroll
      for (int i = 4; i < 8; ++i) smask[i] = 0;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) smask[i] = ((sbyte >> i) & 1u) << 31;
    }
  }
};

// One tile's symbols as seen by one lane, and the tile's Rice parameter and
// record length.
struct TileSyms {
  uint32_t m[8];  // zigzag symbols of the lane's coordinates
  uint32_t raw;   // E8 coset bit of the lane's vector
  uint32_t k;     // Rice parameter of the tile
  uint32_t L;     // record length of the tile (bits)
  uint32_t ulen;  // unary bits of the lane's 8 symbols
};

// RHT -> (dither) -> nearest point -> strip -> zigzag -> Rice k for tile t,
// held by the 16-lane row of the calling lane.  Every lane of the wave calls
// it (it uses ballots); invalid tiles yield zero symbols.
template <int L, bool DITHER, bool BF16>
__device__ __forceinline__ void tile_front(const EncArgs& a, const LaneConst<BF16>& lc, uint64_t t, bool valid,
                                           int v, int r, int grp, TileSyms& ts) {
  constexpr uint32_t RAW = Lat<L>::raw;
  float xv[8];
  if (valid) {
    load_lane<BF16>(a.x, t, v, lc.smask, xv);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) xv[i] = 0.0f;
  }
  fwht_tile(xv, lc.fs);
  float u[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) u[i] = xv[i] * lc.scale;
  if constexpr (DITHER) {
    float d[8];
    dither_lane<L>(a.key0, a.key1, a.tile_base + t, v, d);
#pragma unroll
    for (int i = 0; i < 8; ++i) u[i] = u[i] + d[i];
  }
  bool bad = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) bad |= !(__builtin_fabsf(u[i]) < kRangeLimit);
  const uint64_t bad_mask = __ballot(bad);
  if (bad_mask) {
    const bool tile_bad = ((bad_mask >> (grp * 16)) & 0xFFFFull) != 0;
    bool nf = false;
    if (tile_bad && valid) nf = lane_nonfinite<BF16>(a.x, t, v);
    const bool tile_nf = ((__ballot(nf) >> (grp * 16)) & 0xFFFFull) != 0;
    if (tile_bad) {
      if (r == 0 && valid) set_status(a.ws, tile_nf ? 2 : 3);
#pragma unroll
      for (int i = 0; i < 8; ++i) u[i] = 0.0f;
    }
  }
  int32_t sym[8];
  quantize_lane<L>(u, sym, ts.raw);
  uint32_t lsum = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    ts.m[i] = valid ? zigzag(sym[i]) : 0u;
    lsum += ts.m[i];
  }
  // Rice parameter: the smallest k with S(k) = sum ceil((m >> k)/2) <= 128
  // minimises the tile length.  From M = sum m: S(k) <= 128 once
  // M <= 2^(k+7) (at kA) and S(k) > 128 while M >= 3*2^(k+7), so the answer
  // is one of kA-2, kA-1, kA; S(k) = A_k - A_(k+1) with A_j = sum m >> j.
  const uint32_t M = row_sum_u32(lsum);
  const int kA = M <= 128u ? 0 : (32 - __builtin_clz(M - 1u)) - 7;
  const int c = kA >= 2 ? kA - 2 : 0;
  uint32_t a0 = 0, a1 = 0, a2 = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t tt = ts.m[i] >> c;
    a0 += tt;
    a1 += tt >> 1;
    a2 += tt >> 2;
  }
  const uint32_t tot = row_sum_u32(a0 | (a1 << 10) | (a2 << 20));  // A_c <= 512
  const uint32_t A0 = tot & 1023u, A1 = (tot >> 10) & 1023u, A2 = tot >> 20;
  uint32_t Ak, ak;
  if (A0 - A1 <= 128u) { ts.k = c; Ak = A0; ak = a0; }
  else if (A1 - A2 <= 128u) { ts.k = c + 1; Ak = A1; ak = a1; }
  else { ts.k = c + 2; Ak = A2; ak = a2; }
  ts.ulen = ak + 8u;
  ts.L = valid ? RAW + 128u * (1u + ts.k) + Ak : 0u;
}

// Assemble one tile's record at local bit tb of the LDS stream s (stream word
// i at s[1 + i]).  Every lane of the wave calls it (ballot, shuffles); only
// lanes of valid tiles write.
template <int L>
__device__ __forceinline__ void tile_pack(uint32_t* s, uint32_t tb, const TileSyms& ts, int v, int r, int lane,
                                          int grp, bool valid) {
  constexpr uint32_t RAW = Lat<L>::raw;
  const uint32_t k = ts.k;
  if constexpr (RAW > 0) {
    const uint64_t bm = __ballot((ts.raw & 1u) != 0);
    const uint32_t g16 = (uint32_t)(bm >> (grp * 16)) & 0xFFFFu;
    // bit v of the field is the coset bit of vector v, held by lane v(r)
    const uint32_t raw16 = (g16 & 0x0F0Fu) | (rev4((g16 >> 4) & 0xFu) << 4) | (rev4((g16 >> 12) & 0xFu) << 12);
    if (valid && r == 0) lds_or64(s, tb, raw16, 0u);
  }
  // exclusive scan of the unary lengths in vector order
  const uint32_t U = ts.ulen;
  const int rowbase = lane & ~15;
  const uint32_t Uv = (uint32_t)__shfl((int)U, rowbase | lane_vector(r));
  const uint32_t incl = row_scan_u32(Uv);
  const uint32_t exv = incl - Uv;
  const uint32_t excl = (uint32_t)__shfl((int)exv, rowbase | lane_vector(r));
  if (!valid) return;
  const uint32_t rpos = tb + RAW + 8u * (uint32_t)v * k;
  if (k != 0) {
    const uint32_t mask = (1u << k) - 1u;
    if (k <= 8) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) lo |= (ts.m[j] & mask) << (j * k);
#pragma unroll
      for (int j = 4; j < 8; ++j) hi |= (ts.m[j] & mask) << ((j - 4) * k);
      const uint64_t R = (uint64_t)lo | ((uint64_t)hi << (4 * k));
      lds_or64(s, rpos, (uint32_t)R, (uint32_t)(R >> 32));
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) lds_or64(s, rpos + j * k, ts.m[j] & mask, 0u);
    }
  }
  const uint32_t upos = tb + RAW + 128u * k + excl;
  if (U <= 64u) {
    uint64_t msk = 0;
    uint32_t pos = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pos += ts.m[j] >> k;
      msk |= 1ull << pos;
      pos += 1;
    }
    lds_or64(s, upos, (uint32_t)msk, (uint32_t)(msk >> 32));
  } else {
    uint32_t pos = upos;
    for (int j = 0; j < 8; ++j) {
      pos += ts.m[j] >> k;
      atomicOr(&s[1 + (pos >> 5)], 1u << (pos & 31));
      pos += 1;
    }
  }
}

// Exclusive scan of the kChunkTiles lengths in ln[] into lo[0..kChunkTiles]
// (lo[kChunkTiles] = chunk total); wave 0 only.
__device__ __forceinline__ void chunk_scan(const uint32_t* ln, uint32_t* lo, int tid, int lane) {
  uint32_t l = tid < kChunkTiles ? ln[tid] : 0u;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(l, o);
    if (lane >= o) l += y;
  }
  if (tid < kChunkTiles) lo[tid + 1] = l;
  if (tid == 0) lo[0] = 0;
}

// Look-back control words (LDS) written by wave 0 for the whole work-group.
enum : uint32_t { kLbDone = 0, kLbAdvance = 1, kLbRetry = 2, kLbFallback = 3 };

// One chunk per work-group, chunk = blockIdx.x.  The single pass computes the
// chunk's symbols and lengths, publishes its bit total (aggregate), packs its
// bits in LDS, publishes its last 32 bits (tail), looks back over the
// predecessors' descriptors for its exclusive bit offset, then stores.
//
// Forward progress needs no assumption about dispatch order or residency:
// when a predecessor's descriptor stays unready for a.lookback_spins rounds
// (one round: device-coherent loads of 256 descriptors and a short sleep),
// the work-group recomputes that chunk's aggregate itself (and its tail if it
// is the immediate predecessor), as in the "decoupled fallback" single-pass
// scan.  All inter-work-group words carry the call's epoch, so relaxed
// device-scope atomics suffice and no same-address atomic is used.
template <int L, bool DITHER, bool BF16, bool LEN_ONLY>
__global__ __launch_bounds__(256) void encode_k(EncArgs a) {
  __shared__ uint32_t s_stage[kStageWords + 1];
  __shared__ uint32_t s_tbuf[kMaxRecordWords + 4];  // fallback: one tile's record
  __shared__ uint32_t s_len[kChunkTiles], s_lo[kChunkTiles + 1], s_k[kChunkTiles];
  __shared__ uint32_t s_len2[kChunkTiles], s_lo2[kChunkTiles + 1];
  __shared__ uint32_t s_ctl[4];
  __shared__ uint64_t s_ctl64[2];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, grp = lane >> 4, r = lane & 15;
  const int v = lane_vector(r);
  const LaneConst<BF16> lc(a.sgn, v, a.c_enc);
  const uint32_t chunk = blockIdx.x;
  const uint32_t epoch = a.epoch;
  const uint64_t t_first = (uint64_t)chunk * kChunkTiles;

  TileSyms ts[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int slot = p * 16 + wv * 4 + grp;
    const uint64_t t = t_first + slot;
    const bool valid = t < a.n_tiles;
    tile_front<L, DITHER, BF16>(a, lc, t, valid, v, r, grp, ts[p]);
    if (r == 0) {
      s_len[slot] = ts[p].L;
      s_k[slot] = ts[p].k;
    }
  }
  __syncthreads();
  if (wv == 0) chunk_scan(s_len, s_lo, tid, lane);
  __syncthreads();
  const uint32_t A = s_lo[kChunkTiles];

  if constexpr (LEN_ONLY) {
    if (tid == 0) a.partials[chunk] = A;
  } else {
    const uint64_t ep = (uint64_t)epoch << kDescEpochShift;
    if (tid == 0)
      __hip_atomic_store(&a.desc[chunk], (chunk == 0 ? kDescFlagIncl : kDescFlagAgg) | ep | (uint64_t)A,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t nz = ((A + 31u) >> 5) + 2u;
    for (uint32_t i = tid; i < nz; i += 256) s_stage[1 + i] = 0u;
    __syncthreads();
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int slot = p * 16 + wv * 4 + grp;
      tile_pack<L>(s_stage, s_lo[slot], ts[p], v, r, lane, grp, t_first + slot < a.n_tiles);
    }
    __syncthreads();
    if (tid == 0) {
      const uint32_t b = A - 32u;  // A >= 128: every chunk holds a tile
      const uint32_t w = 1 + (b >> 5), sh = b & 31;
      const uint32_t tailv = sh ? __builtin_amdgcn_alignbit(s_stage[w + 1], s_stage[w], sh) : s_stage[w];
      __hip_atomic_store(&a.tail[chunk], ((uint64_t)epoch << 32) | tailv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_ctl[1] = 0;  // predecessor tail not yet known
    }

    // ---- look-back (work-group-wide loop; wave 0 reads 256 descriptors) ----
    uint64_t excl = 0;
    int64_t j = (int64_t)chunk - 1;
    int spins = 0;
    while (j >= 0) {
      if (wv == 0) {
        uint64_t val[4];
        bool rdy[4], isP[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t idx = j - 4 * lane - q;
          const uint64_t d = idx >= 0 ? __hip_atomic_load(&a.desc[idx], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
          const uint32_t dep = (uint32_t)(d >> kDescEpochShift) & 0xFFFFFFu;
          const uint64_t flag = d >> 62;
          rdy[q] = idx < 0 || (flag != 0 && dep == epoch);
          isP[q] = idx < 0 || (rdy[q] && flag == 2);
          val[q] = idx >= 0 ? (d & kDescValueMask) : 0ull;
        }
        // first stop (inclusive or unready descriptor), newest first
        int qs = 4;
#pragma unroll
        for (int q = 3; q >= 0; --q) qs = (isP[q] || !rdy[q]) ? q : qs;
        uint64_t before = 0, all4 = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (q < qs) before += val[q];
          all4 += val[q];
        }
        const uint64_t bs = __ballot(qs < 4);
        const int fl = bs ? __builtin_ctzll(bs) : 64;
        uint64_t contrib = lane < fl ? all4 : (lane == fl ? before : 0ull);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) contrib += __shfl_xor(contrib, o);
        if (lane == (fl < 64 ? fl : 0)) {
          uint32_t ctl;
          uint64_t add = contrib;
          if (fl == 64) {
            ctl = kLbAdvance;
          } else if (isP[qs < 4 ? qs : 0] && qs < 4) {
            ctl = kLbDone;
            add += val[qs];
          } else {
            ctl = spins < (int)a.lookback_spins ? kLbRetry : kLbFallback;
            s_ctl64[1] = (uint64_t)(j - 4 * fl - qs);  // the unready chunk
          }
          s_ctl[0] = ctl;
          s_ctl64[0] = add;
        }
      }
      __syncthreads();
      const uint32_t ctl = s_ctl[0];
      const uint64_t add = s_ctl64[0];
      const int64_t jf = (int64_t)s_ctl64[1];
      __syncthreads();
      if (ctl == kLbDone) {
        excl += add;
        break;
      }
      if (ctl == kLbAdvance) {
        excl += add;
        j -= 256;
        continue;
      }
      if (ctl == kLbRetry) {
        ++spins;
        __builtin_amdgcn_s_sleep(2);
        continue;
      }
      // Fallback: compute chunk jf's aggregate here (and, for the immediate
      // predecessor, its last 32 bits), then continue below it.
      const uint64_t tf = (uint64_t)jf * kChunkTiles;  // a full chunk: jf < chunk
      for (uint32_t i = tid; i < kMaxRecordWords + 4; i += 256) s_tbuf[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int p = 0; p < kPasses; ++p) {
        const int slot = p * 16 + wv * 4 + grp;
        TileSyms fsy;
        tile_front<L, DITHER, BF16>(a, lc, tf + slot, true, v, r, grp, fsy);
        if (r == 0) s_len2[slot] = fsy.L;
        if (jf == (int64_t)chunk - 1 && p == kPasses - 1 && wv == 3) {
          tile_pack<L>(s_tbuf, 0u, fsy, v, r, lane, grp, grp == 3);  // slot kChunkTiles-1
          if (grp == 3 && r == 0) s_ctl[2] = fsy.L;
        }
      }
      __syncthreads();
      if (wv == 0) chunk_scan(s_len2, s_lo2, tid, lane);
      __syncthreads();
      excl += add + s_lo2[kChunkTiles];
      if (jf == (int64_t)chunk - 1 && tid == 0) {
        const uint32_t Lt = s_ctl[2], b = Lt - 32u;
        const uint32_t w = 1 + (b >> 5), sh = b & 31;
        s_stage[0] = sh ? __builtin_amdgcn_alignbit(s_tbuf[w + 1], s_tbuf[w], sh) : s_tbuf[w];
        s_ctl[1] = 1;
      }
      j = jf - 1;
      spins = 0;
      __syncthreads();
    }
    if (tid == 0) {
      if (chunk > 0)
        __hip_atomic_store(&a.desc[chunk], kDescFlagIncl | ep | (excl + A), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_ctl64[0] = excl;
      if (chunk == 0) {
        s_stage[0] = 0;
      } else if (s_ctl[1] == 0) {
        // the predecessor is running (it published its descriptor itself) and
        // publishes its tail before its own look-back
        uint64_t tw;
        while (((tw = __hip_atomic_load(&a.tail[chunk - 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) >> 32) !=
               (uint64_t)epoch)
          __builtin_amdgcn_s_sleep(1);
        s_stage[0] = (uint32_t)tw;
      }
    }
    __syncthreads();

    const uint64_t E = s_ctl64[0];
    if (tid < kChunkTiles) {
      const uint64_t t = t_first + tid;
      if (t < a.n_tiles) {
        a.offsets[t] = E + s_lo[tid];
        a.kout[t] = (uint8_t)s_k[tid];
        if (t == a.n_tiles - 1) a.offsets[a.n_tiles] = E + s_lo[tid + 1];
      }
    }
    const bool last = t_first + kChunkTiles >= a.n_tiles;
    const uint64_t first = E >> 5;
    const uint32_t sh = (uint32_t)(E & 31);
    const uint64_t endw = last ? (E + A + 31) >> 5 : (E + A) >> 5;
    if (tid == 0 && endw > a.cap_words) set_status(a.ws, 4);
    const uint64_t stop = endw < a.cap_words ? endw : a.cap_words;
    for (uint64_t w = first + tid; w < stop; w += 256) {
      const uint32_t i = (uint32_t)(w - first);
      a.words[w] = sh ? __builtin_amdgcn_alignbit(s_stage[1 + i], s_stage[i], 32 - sh) : s_stage[1 + i];
    }
  }
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
// (the verdict is uniform over the 16 lanes of the tile).  ust: 16 words of
// LDS per tile; tb: 16 bytes of LDS per tile.
template <int L>
__device__ __forceinline__ bool parse_lane(const uint32_t* s, uint32_t base, uint32_t Lb, uint32_t k, int v, int r,
                                           int lane, uint32_t* ust, uint8_t* tb, float p[8]) {
  constexpr uint32_t RAW = Lat<L>::raw;
  uint32_t raw = 0;
  if constexpr (RAW > 0) {
    const uint32_t f = __builtin_amdgcn_alignbit(s[(base >> 5) + 1], s[base >> 5], base & 31);
    raw = (f >> v) & 1u;
  }
  // remainders: 8 fields of k bits at fixed positions
  uint32_t rem[8];
  const uint32_t rpos = base + RAW + 8u * (uint32_t)v * k;
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
  // (8v)-th one
  const uint32_t ustart = base + RAW + 128u * k, uend = base + Lb;
  const uint32_t wA = ustart >> 5, nW = ((uend - 1u) >> 5) - wA + 1u;
  uint32_t start;
  bool ok = true;
  if (nW <= 16) {
    // one word per lane: inclusive one-counts I_r, kept as bytes in LDS
    uint32_t word = (uint32_t)r < nW ? s[wA + r] : 0u;
    if (r == 0) word &= ~0u << (ustart & 31);
    if ((uint32_t)r == nW - 1 && (uend & 31)) word &= (1u << (uend & 31)) - 1u;
    const uint32_t I = row_scan_u32(__builtin_popcount(word));
    if (r == 15) ok = I == 128u;
    tb[r] = (uint8_t)(I < 127u ? I : 127u);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint4 T = *reinterpret_cast<const uint4*>(tb);
    start = ustart;
    if (v > 0) {
      // word holding rank R = 8v-1: the number of words with I_w <= R, by a
      // packed-byte compare (byte 0x80 + R - I_w keeps bit 7 iff I_w <= R;
      // 7 <= R <= 119 and I_w <= 127, so no byte borrows)
      const uint32_t R = 8u * (uint32_t)v - 1u;
      const uint32_t key = (R * 0x01010101u) | 0x80808080u;
      const uint32_t wsel = __builtin_popcount((key - T.x) & 0x80808080u) + __builtin_popcount((key - T.y) & 0x80808080u) +
                            __builtin_popcount((key - T.z) & 0x80808080u) + __builtin_popcount((key - T.w) & 0x80808080u);
      const uint32_t q4 = wsel == 0 ? 0u : wsel - 1u;  // byte index of I_(w-1)
      const uint32_t Td = q4 < 4 ? T.x : q4 < 8 ? T.y : q4 < 12 ? T.z : T.w;
      const uint32_t Iprev = wsel == 0 ? 0u : __builtin_amdgcn_ubfe(Td, 8 * (q4 & 3), 8);
      uint32_t wd = s[wA + min(wsel, 15u)];
      if (wsel == 0) wd &= ~0u << (ustart & 31);
      start = (wA + wsel) * 32u + select_bit(wd, R - Iprev) + 1u;
    }
  } else {
    ok = unary_starts_general(s, ustart, uend, r, ust) == 128u;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    start = v == 0 ? ustart : ust[v];
  }
  const uint32_t lastbit = (s[(uend - 1u) >> 5] >> ((uend - 1u) & 31)) & 1u;
  ok &= lastbit != 0;
  if (((__ballot(!ok) >> (lane & ~15)) & 0xFFFFull) != 0) return false;
  // the lane's 8 unary codes: q zeros then a one, from start
  uint32_t m[8];
  const uint32_t qlim = kMLimit >> k;
  {
    const uint32_t w = min(start >> 5, (uint32_t)kStageWords - 2u), sh = start & 31;
    uint32_t win = __builtin_amdgcn_alignbit(s[w + 1], s[w], sh);
    if (__builtin_popcount(win) >= 8) {
      uint32_t prev = 0, qmax = 0;  // prev: bit after the previous one
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t pos = (uint32_t)__builtin_ctz(win);
        const uint32_t q = pos - prev;  // < 32
        qmax = max(qmax, q);
        m[j] = (q << k) | rem[j];
        prev = pos + 1;
        win &= win - 1u;
      }
      ok &= qmax < qlim;
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

template <int L, bool DITHER, int OUT>
__global__ __launch_bounds__(256) void decode_k(DecArgs a) {
  constexpr uint32_t RAW = Lat<L>::raw;
  constexpr uint32_t MAXREC = RAW + 128u * 23u;
  __shared__ uint32_t s_stage[kStageWords];
  __shared__ uint64_t s_off[kChunkTiles + 1];
  __shared__ uint32_t s_k[kChunkTiles];
  __shared__ uint32_t s_ust[16][16];
  __shared__ uint4 s_tb[16];  // per tile of a pass: 16 one-count bytes
  __shared__ float s_q[OUT == kOutScores ? 16 : 1][kTile];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, grp = lane >> 4, r = lane & 15;
  const int v = lane_vector(r);
  const FwhtSigns fs = fwht_signs(v);
  const uint32_t sbyte = (a.sgn[v >> 2] >> ((v & 3) * 8)) & 0xFFu;

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

  if (tid <= (int)nt) s_off[tid] = a.offsets[t_first + tid];
  if (tid < (int)nt) s_k[tid] = a.kin[t_first + tid];
  if constexpr (OUT == kOutScores) {
    // rotate the head's queries: q~ = H D q, one query per 16-lane row
    const int g = wv * 4 + grp;
    if (g < (int)a.qph) {
      const float* qp = a.q + ((head * a.qph + g) * kTile + 8 * v);
      float xq[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) xq[i] = ((sbyte >> i) & 1u) ? -qp[i] : qp[i];
      fwht_tile(xq, fs);
#pragma unroll
      for (int i = 0; i < 8; ++i) s_q[g][8 * v + i] = xq[i] * fs.lane_sign;
    }
  }
  __syncthreads();
  const uint64_t w_first = s_off[0] >> 5;
  const uint64_t w_end = (s_off[nt] + 31) >> 5;
  const bool span_ok = s_off[nt] >= s_off[0] && (w_end - w_first) <= (uint64_t)kStageWords - 4 && w_end <= a.n_words;
  if (span_ok) {
    const uint32_t n = (uint32_t)(w_end - w_first);
    for (uint32_t i = tid; i < n; i += 256) s_stage[i] = a.words[w_first + i];
    for (uint32_t i = n + tid; i < n + 4; i += 256) s_stage[i] = 0u;
  }
  __syncthreads();

  float sc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sc[i] = (((sbyte >> i) & 1u) ? -fs.lane_sign : fs.lane_sign) * a.c_dec;

#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int pslot = wv * 4 + grp;
    const int slot = p * 16 + pslot;
    const bool valid = slot < (int)nt;
    const uint64_t t = t_first + slot;
    float pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) pv[i] = 0.0f;
    if (valid) {
      const uint64_t o0 = s_off[slot], o1 = s_off[slot + 1];
      const uint32_t k = s_k[slot];
      const uint64_t Lr = o1 - o0;
      const bool ok = span_ok && o1 >= o0 && k <= (uint32_t)kKMax && Lr >= RAW + 128u * (1u + k) && Lr <= MAXREC;
      bool good = false;
      if (ok) good = parse_lane<L>(s_stage, (uint32_t)(o0 - 32 * w_first), (uint32_t)Lr, k, v, r, lane, s_ust[pslot],
                                       reinterpret_cast<uint8_t*>(&s_tb[pslot]), pv);
      if (!good) {
        if (r == 0) set_status(a.ws, 5);
#pragma unroll
        for (int i = 0; i < 8; ++i) pv[i] = 0.0f;
      } else if constexpr (DITHER) {
        float d[8];
        dither_lane<L>(a.key0, a.key1, a.tile_base + t, v, d);
#pragma unroll
        for (int i = 0; i < 8; ++i) pv[i] = pv[i] - d[i];
      }
    }
    if constexpr (OUT == kOutScores) {
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
            pk[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
          }
          *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.y) + t * kTile + 8 * v) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        } else {
          uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<float*>(a.y) + t * kTile + 8 * v);
          dst[0] = make_uint4(__builtin_bit_cast(uint32_t, o[0]), __builtin_bit_cast(uint32_t, o[1]),
                              __builtin_bit_cast(uint32_t, o[2]), __builtin_bit_cast(uint32_t, o[3]));
          dst[1] = make_uint4(__builtin_bit_cast(uint32_t, o[4]), __builtin_bit_cast(uint32_t, o[5]),
                              __builtin_bit_cast(uint32_t, o[6]), __builtin_bit_cast(uint32_t, o[7]));
        }
      }
    }
  }
}

// Sum of squares (fp64) for the calibration start point: one partial per
// work-group (no same-address atomics), reduced in a fixed order.
__global__ __launch_bounds__(256) void sumsq_k(const void* x, int bf16, uint64_t n, double* partials) {
  __shared__ double s_w[4];
  double acc = 0.0;
  for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (uint64_t)gridDim.x * 256) {
    float f = bf16 ? __builtin_bit_cast(float, (uint32_t)reinterpret_cast<const uint16_t*>(x)[i] << 16)
                   : reinterpret_cast<const float*>(x)[i];
    acc += (double)f * (double)f;
  }
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) partials[blockIdx.x] = (s_w[0] + s_w[1]) + (s_w[2] + s_w[3]);
}

template <typename T>
__global__ __launch_bounds__(256) void reduce_k(const T* p, uint32_t n, T* out) {
  __shared__ T s[256];
  T acc = 0;
  for (uint32_t i = threadIdx.x; i < n; i += 256) acc += p[i];
  s[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) s[threadIdx.x] += s[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = s[0];
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int L, bool DITHER, bool BF16>
static hipError_t launch_encode_t(EncArgs a, bool len_only, hipStream_t st) {
  const dim3 grid(a.n_chunks);
  if (len_only) {
    hipLaunchKernelGGL((encode_k<L, DITHER, BF16, true>), grid, dim3(256), 0, st, a);
    hipLaunchKernelGGL(reduce_k<unsigned long long>, dim3(1), dim3(256), 0, st,
                       (const unsigned long long*)a.partials, a.n_chunks, &a.ws->bits);
  } else {
    hipLaunchKernelGGL((encode_k<L, DITHER, BF16, false>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_encode(int lat, bool dither, bool bf16, bool len_only, const EncArgs& a, hipStream_t st) {
#define HQ_ENC(LL)                                                                        \
  if (lat == LL) {                                                                        \
    if (dither) return bf16 ? launch_encode_t<LL, true, true>(a, len_only, st)            \
                            : launch_encode_t<LL, true, false>(a, len_only, st);          \
    return bf16 ? launch_encode_t<LL, false, true>(a, len_only, st)                       \
                : launch_encode_t<LL, false, false>(a, len_only, st);                     \
  }
  HQ_ENC(0) HQ_ENC(1) HQ_ENC(2) HQ_ENC(3)
#undef HQ_ENC
  return hipErrorInvalidValue;
}

template <int L, bool DITHER>
static hipError_t launch_decode_t(const DecArgs& a, int out, dim3 grid, hipStream_t st) {
  if (out == kOutBf16) hipLaunchKernelGGL((decode_k<L, DITHER, kOutBf16>), grid, dim3(256), 0, st, a);
  else if (out == kOutF32) hipLaunchKernelGGL((decode_k<L, DITHER, kOutF32>), grid, dim3(256), 0, st, a);
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

hipError_t launch_sumsq(const void* x, bool bf16, uint64_t n, double* partials, uint32_t max_blocks, double* out,
                        hipStream_t st) {
  uint64_t blocks = (n + 255) / 256;
  if (blocks > max_blocks) blocks = max_blocks;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(sumsq_k, dim3((uint32_t)blocks), dim3(256), 0, st, x, bf16 ? 1 : 0, n, partials);
  hipLaunchKernelGGL(reduce_k<double>, dim3(1), dim3(256), 0, st, (const double*)partials, (uint32_t)blocks, out);
  return hipGetLastError();
}

}  // namespace hq
