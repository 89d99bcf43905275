// hq_device.h -- device building blocks of the HyperQuant tile codec on gfx950.
//
// Sources cited in this directory:
//   [HQ] "HyperQuant: A Rate-Distortion-Optimal Quantization Pipeline for Large
//        Language and Diffusion Models", gist.science explainer pages,
//        technical summary: Methodology 1 (per-tile RHT), 2 (lattice
//        quantization), 3 (bit-stripping and Rice coding), 4 (KV bias
//        correction); and the paper's abstract page, items (i)-(iv).
//   [Philox] Salmon et al., "Parallel random numbers: as easy as 1, 2, 3", SC'11.
//   [SPLAG] Conway & Sloane, "Sphere Packings, Lattices and Groups", ch. 20.
//
// Lane mapping.  A tile of 128 coordinates lives in 16 lanes of one DPP row,
// 8 consecutive coordinates per lane, so one 16-byte bf16 load per lane and one
// E8 vector (two D4, four A2, eight Z) per lane.  Lane r of the row holds
// lattice vector v(r) = r ^ (bit2(r) ? 3 : 0), coordinates 8v..8v+7.  With that
// permutation the four cross-lane butterfly stages of the Walsh-Hadamard
// transform (vector-index bits 0..3) pair lane r with r^1, r^2, r^7 and r^8,
// which are the DPP patterns quad_perm[1,0,3,2], quad_perm[2,3,0,1],
// row_half_mirror and row_ror:8.  Each stage is one v_fmac_f32 with a DPP
// source per value: new = partner * c + own with c = +-1, which is exact
// (the product is exact, one rounding) and equals the textbook a+b / a-b up to
// a per-lane sign (-1)^popcount(v) that the final scale absorbs.
//
// All fp32 arithmetic that decides a lattice code follows the oracle's order:
// no contraction (-ffp-contract=off), explicit fmaf only where the product is
// exact, round-to-nearest-even throughout, denormals kept.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hq {

constexpr int kTile = 128;
constexpr int kKMax = 22;
constexpr uint32_t kMLimit = 1u << 22;
constexpr float kRangeLimit = 1048576.0f;  // 2^20
constexpr float kSqrt3 = 1.7320508075688772f;
constexpr float kInv2Sqrt3 = 0.28867513459481287f;
constexpr uint32_t kTagDither = 0x44495448u;  // "DITH"

template <int L> struct Lat;
template <> struct Lat<0> { static constexpr int dim = 1, raw = 0; };  // Z
template <> struct Lat<1> { static constexpr int dim = 2, raw = 0; };  // A2
template <> struct Lat<2> { static constexpr int dim = 4, raw = 0; };  // D4
template <> struct Lat<3> { static constexpr int dim = 8, raw = 16; }; // E8 (2E8)

__device__ __forceinline__ int lane_vector(int r) { return r ^ (((r >> 2) & 1) ? 3 : 0); }

// ---------------------------------------------------------------------------
// DPP helpers
// ---------------------------------------------------------------------------
template <int CTRL> __device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i within 8
constexpr int kDppRor8 = 0x128;        // lane i <-> i^8 within 16
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;

// Sum over the 16 lanes of a row; every lane receives the total.
__device__ __forceinline__ uint32_t row_sum_u32(uint32_t x) {
  x += dpp_u32<kDppXor1>(x);
  x += dpp_u32<kDppXor2>(x);
  x += dpp_u32<kDppHalfMirror>(x);
  x += dpp_u32<kDppRor8>(x);
  return x;
}

__device__ __forceinline__ float row_sum_f32(float x) {
  x += __builtin_bit_cast(float, dpp_u32<kDppXor1>(__builtin_bit_cast(uint32_t, x)));
  x += __builtin_bit_cast(float, dpp_u32<kDppXor2>(__builtin_bit_cast(uint32_t, x)));
  x += __builtin_bit_cast(float, dpp_u32<kDppHalfMirror>(__builtin_bit_cast(uint32_t, x)));
  x += __builtin_bit_cast(float, dpp_u32<kDppRor8>(__builtin_bit_cast(uint32_t, x)));
  return x;
}

// Inclusive prefix sum over the 16 lanes of a row, in lane order.
__device__ __forceinline__ uint32_t row_scan_u32(uint32_t x) {
  // row_shr with bound_ctrl reads zero from lanes shifted in from outside the row
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kDppShr1, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kDppShr2, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kDppShr4, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kDppShr8, 0xF, 0xF, true);
  return x;
}

// ---------------------------------------------------------------------------
// Walsh-Hadamard transform of one tile held as 8 values per lane
// [HQ Methodology 1: H_n of RHT_n(x) = H_n D x, Sylvester order, stages of
// stride 1, 2, ..., 64].  On return the values carry the per-lane sign
// (-1)^popcount(v); callers fold it into their scale.
// ---------------------------------------------------------------------------
#define HQ_DPP_STAGE(CTRL)                                                       \
  asm volatile(                                                                  \
      "s_nop 1\n\t"                                                              \
      "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
      "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
      "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
      "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
      "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
      "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
      "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
      "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
      "s_nop 1"                                                                  \
      : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]),  \
        "+v"(x[6]), "+v"(x[7])                                                   \
      : "v"(c))

// Lanes of a 16-lane row whose vector index v(r) has bit s set (s = 0..3), and
// those where popcount(v(r)) is odd, repeated over the four rows of a wave.
constexpr uint64_t kLaneBit0 = 0x5A5A5A5A5A5A5A5Aull;
constexpr uint64_t kLaneBit1 = 0x3C3C3C3C3C3C3C3Cull;
constexpr uint64_t kLaneBit2 = 0xF0F0F0F0F0F0F0F0ull;
constexpr uint64_t kLaneBit3 = 0xFF00FF00FF00FF00ull;
constexpr uint64_t kLaneOdd = 0x6996699669966996ull;

// +1 in the lanes outside the lane mask, -1 inside it.  Built at its use (the
// asm is not hoisted or merged), so it holds a register only for one stage.
__device__ __forceinline__ float lane_sign_of(uint64_t mask) {
  float c;
  asm volatile("v_cndmask_b32_e64 %0, 1.0, -1.0, %1" : "=v"(c) : "s"(mask));
  return c;
}

// The lane's word of a 4-word lane-layout table (word v >> 2; the lane masks
// of vector bits 2 and 3 are constants).
__device__ __forceinline__ uint32_t lane_word4(const uint32_t W[4], int v) {
  const uint32_t lo = (v & 4) ? W[1] : W[0];
  const uint32_t hi = (v & 4) ? W[3] : W[2];
  return (v & 8) ? hi : lo;
}
// Signs of D for the lane's 8 coordinates from the host's lane layouts: bf16
// pairs, bit 15 - i = coordinate 2i and bit 31 - i = coordinate 2i + 1 (so
// pair i's flips are (sm << i) & 0x80008000); fp32, bit 31 - i = coordinate i.
__device__ __forceinline__ uint32_t lane_signs16(const uint32_t sl16[4], int v) {
  return (lane_word4(sl16, v) << (4 * (v & 3))) & 0xF000F000u;
}
__device__ __forceinline__ uint32_t lane_signs32(const uint32_t sl32[4], int v) {
  return (lane_word4(sl32, v) << (8 * (v & 3))) & 0xFF000000u;
}

struct FwhtSigns {
  float lane_sign;  // (-1)^popcount(v)
};

__device__ __forceinline__ FwhtSigns fwht_signs(int v) {
  FwhtSigns s;
  s.lane_sign = (__builtin_popcount(v) & 1) ? -1.0f : 1.0f;
  return s;
}

// Cross-lane stage s pairs lane r with the lane holding vector v ^ 2^s; the
// sign c = -1 where bit s of v is set.
__device__ __forceinline__ void fwht_tile(float x[8], const FwhtSigns&) {
  // in-lane strides 1, 2, 4 (index bits 0..2): plain butterflies
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i & h) continue;
      float a = x[i], b = x[i + h];
      x[i] = a + b;
      x[i + h] = a - b;
    }
  }
  float c;
  c = lane_sign_of(kLaneBit0); HQ_DPP_STAGE("quad_perm:[1,0,3,2]");  // stride 8
  c = lane_sign_of(kLaneBit1); HQ_DPP_STAGE("quad_perm:[2,3,0,1]");  // stride 16
  c = lane_sign_of(kLaneBit2); HQ_DPP_STAGE("row_half_mirror");      // stride 32
  c = lane_sign_of(kLaneBit3); HQ_DPP_STAGE("row_ror:8");            // stride 64
}

// ---------------------------------------------------------------------------
// Philox4x32-10 [Philox]
// ---------------------------------------------------------------------------
__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // one 32x32 -> 64-bit product each (a single v_mad_u64_u32 instead of a
    // separate low and high multiply)
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0], p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
    k0 += 0x9E3779B9u; k1 += 0xBB67AE85u;
  }
}

// ---------------------------------------------------------------------------
// Nearest points [HQ Methodology 2; SPLAG ch. 20] in the integer embeddings
// Z, A2 checkerboard {(i,j): i = j mod 2} with real point (i, j sqrt3),
// D4 = {x in Z^4: sum even}, 2E8.  Rounding to the nearest integer (ties to
// even) is the fp32 add of 1.5*2^23: for |h| < 2^22 the sum r has ulp 1, so it
// holds rint(h) exactly, read as r - 1.5*2^23 or, as an integer, as
// bits(r) - bits(1.5*2^23); the parity of rint(h) is bit 0 of bits(r).
// ---------------------------------------------------------------------------
constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
constexpr uint32_t kMagicBits = 0x4B400000u;

__device__ __forceinline__ uint32_t fbits(float f) { return __builtin_bit_cast(uint32_t, f); }

// a ^ b ^ c in one instruction
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// x - c + [lane in plus] - [lane in minus]: one add with carry-in and one
// subtract with borrow-in, the lane masks being wave-wide (scalar) values.
// c is held in a vector register (one scalar operand per instruction).
__device__ __forceinline__ int32_t add_sub_lane(uint32_t x, uint32_t c, uint64_t plus, uint64_t minus) {
  uint32_t t, r;
  uint64_t co;
  asm("v_addc_co_u32_e64 %0, %1, %2, 0, %3" : "=v"(t), "=s"(co) : "v"(x), "s"(plus));
  if (__builtin_constant_p(c) && c == 0u)
    asm("v_subb_co_u32_e64 %0, %1, %2, 0, %3" : "=v"(r), "=s"(co) : "v"(t), "s"(minus));
  else
    asm("v_subb_co_u32_e64 %0, %1, %2, %3, %4" : "=v"(r), "=s"(co) : "v"(t), "v"(c), "s"(minus));
  return (int32_t)r;
}

__device__ __forceinline__ uint32_t zigzag(int32_t v) {
  return ((uint32_t)v << 1) ^ (uint32_t)(v >> 31);
}

// The encoder keeps every symbol m as w = 2 m + 1; for m = zigzag(y) that is
// |4y + 1|.  From y held with an even bias, yb = y + B (|4y + 1| < 2^24 and
// 4B + 2^24 < 2^32 taken mod 2^32), it is one shift-or and one absolute
// difference against fourB = 4B mod 2^32.
__device__ __forceinline__ uint32_t zz1_biased(uint32_t yb, uint32_t fourB) {
  const uint32_t t = (yb << 2) | 1u;
  uint32_t r;
  asm("v_sad_u32 %0, %1, %2, 0" : "=v"(r) : "v"(t), "s"(fourB));
  return r;
}
// the same from an unbiased y
__device__ __forceinline__ uint32_t zz1(int32_t y) {
  const int32_t t = (int32_t)(((uint32_t)y << 2) | 1u);
  return (uint32_t)max(t, -t);
}
constexpr uint32_t kFourMagic = 4u * kMagicBits;  // mod 2^32
constexpr uint32_t kTwoMagic = 2u * kMagicBits;
__device__ __forceinline__ int32_t unzigzag(uint32_t m) {
  return (int32_t)(m >> 1) ^ -(int32_t)(m & 1u);
}

// D4: round every coordinate; when the sum is odd, move the first coordinate of
// largest |u - f| by 1 toward u (upward iff u - f >= 0).  e = u - f is exact.
// The decisions are wave-wide lane masks (ballots), combined with scalar
// logic, and applied as carry/borrow.  Every lane of the wave (or of the
// active set) must call it.
// x is returned as rint bits - cm: cm = kMagicBits gives the integers, cm = 0
// the integers biased by kMagicBits.
__device__ __forceinline__ void d4_core(const float u[4], int32_t x[4], uint32_t cm) {
  float e[4];
  uint32_t rb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float r = u[i] + kMagic;
    rb[i] = fbits(r);
    e[i] = u[i] - (r - kMagic);
  }
  const uint64_t ODD = __ballot(((rb[0] ^ rb[1] ^ rb[2] ^ rb[3]) & 1u) != 0);
  const float emax = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(e[0]), __builtin_fabsf(e[1])),
                                     __builtin_fmaxf(__builtin_fabsf(e[2]), __builtin_fabsf(e[3])));
  uint64_t seen = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint64_t HIT = __ballot(__builtin_fabsf(e[i]) == emax);
    const uint64_t UP = __ballot(e[i] >= 0.0f);
    const uint64_t FJ = ODD & HIT & ~seen;
    seen |= HIT;
    x[i] = add_sub_lane(rb[i], cm, FJ & UP, FJ & ~UP);
  }
}

// A2: best of the two rectangular cosets (ties even).
__device__ __forceinline__ float a2_dist(float u0, float u1, int32_t i, int32_t j) {
  float e0 = u0 - (float)i;
  float t = (float)j * kSqrt3;
  float e1 = u1 - t;
  return e0 * e0 + e1 * e1;
}

__device__ __forceinline__ void np_a2_codes(float u0, float u1, int32_t& i, int32_t& j) {
  float w0 = u0 * 0.5f, w1 = u1 * kInv2Sqrt3;
  int32_t ie = 2 * (int32_t)__builtin_rintf(w0), je = 2 * (int32_t)__builtin_rintf(w1);
  int32_t io = 2 * (int32_t)__builtin_floorf(w0) + 1, jo = 2 * (int32_t)__builtin_floorf(w1) + 1;
  float de = a2_dist(u0, u1, ie, je), dd = a2_dist(u0, u1, io, jo);
  bool even = de <= dd;
  i = even ? ie : io;
  j = even ? je : jo;
}

// 2E8 = 2D8 u (2D8 + 1), returned as halves y (x = 2y + b, b = 1 for the odd
// coset).  With h = u/2, ye = rint(h) and d = u - 2 ye (exact, |d| <= 1; as
// fma(2, M - r, u) it is never -0), floor(h) = ye - [d < 0], and the halved
// squared-distance difference of the parity-fixed even and odd candidates is
//   (sum |d_i| - 4) + [sum ye odd] 2 (1 - max |d|) - [sum floor(h) odd] 2 min |d|,
// evaluated in fp32 in this order (sum sequential); even wins ties.  The fix
// moves the first coordinate of largest |u - c| by 2 toward u: for the even
// coset the first argmax of |d|, upward iff d >= 0; for the odd coset the
// first argmin of |d|, upward iff d < 0 or d = 1 (d = 1 at the argmin means
// every |d_i| = 1, i.e. min |d| = 1).  Every adjustment of ye is -1, 0 or +1:
// a borrow and a carry on the integer.
// (y is returned as in d4_core: cm = kMagicBits unbiased, cm = 0 biased.)
__device__ __forceinline__ void e8_core(const float u[8], int32_t y[8], bool& odd, uint32_t cm) {
  float d[8];
  uint32_t rb[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float r = __builtin_fmaf(u[i], 0.5f, kMagic);  // u/2 is exact: one rounding
    rb[i] = fbits(r);
    d[i] = __builtin_fmaf(2.0f, kMagic - r, u[i]);
  }
  float S = __builtin_fabsf(d[0]), amax = S, amin = S;
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    const float ai = __builtin_fabsf(d[i]);
    S = S + ai;
    amax = __builtin_fmaxf(amax, ai);
    amin = __builtin_fminf(amin, ai);
  }
  // wave-wide lane masks; the logic below is scalar
  uint64_t NEG[8], PN = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    NEG[i] = __ballot(d[i] < 0.0f);
    PN ^= NEG[i];  // parity of the number of negative d
  }
  const uint32_t xr = xor3(xor3(rb[0], rb[1], rb[2]), xor3(rb[3], rb[4], rb[5]), rb[6] ^ rb[7]);
  const uint64_t PE = __ballot((xr & 1u) != 0);
  const uint64_t PO = PE ^ PN;
  const bool pe = __builtin_amdgcn_inverse_ballot_w64(PE);
  const bool po = __builtin_amdgcn_inverse_ballot_w64(PO);
  float delta = S - 4.0f;
  const float t1 = __builtin_fmaf(2.0f, 1.0f - amax, delta);  // delta + 2 (1 - max): exact product
  delta = pe ? t1 : delta;
  const float t2 = __builtin_fmaf(-2.0f, amin, delta);  // delta - 2 min: exact product
  delta = po ? t2 : delta;
  const bool even = delta <= 0.0f;
  odd = !even;
  const float target = even ? amax : amin;
  const uint64_t EVEN = __ballot(even);
  const uint64_t FIX = (EVEN & PE) | (~EVEN & PO);
  const uint64_t ODDUP = ~EVEN & __ballot(amin == 1.0f);
  uint64_t seen = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint64_t HIT = __ballot(__builtin_fabsf(d[i]) == target);
    const uint64_t FJ = FIX & HIT & ~seen;
    seen |= HIT;
    const uint64_t DOWN = ~EVEN & NEG[i];                    // floor(h) = ye - 1
    const uint64_t UP = (EVEN & ~NEG[i]) | DOWN | ODDUP;     // direction of the fix
    const uint64_t P = FJ & UP & ~DOWN;
    const uint64_t Q = (DOWN & ~FJ) | (FJ & ~UP);
    y[i] = add_sub_lane(rb[i], cm, P, Q);
  }
}

// Codes of one lattice vector from its symbols (inverse of the strip), as
// real-space fp32 coordinates of the embedding.
template <int L> __device__ __forceinline__ void unstrip_embed(const int32_t* sym, uint32_t raw, float* p);

template <> __device__ __forceinline__ void unstrip_embed<0>(const int32_t* sym, uint32_t, float* p) {
  p[0] = (float)sym[0];
}
template <> __device__ __forceinline__ void unstrip_embed<1>(const int32_t* sym, uint32_t, float* p) {
  int32_t j = sym[1];
  int32_t i = 2 * sym[0] + (j & 1);
  p[0] = (float)i;
  p[1] = (float)j * kSqrt3;
}
template <> __device__ __forceinline__ void unstrip_embed<2>(const int32_t* sym, uint32_t, float* p) {
  int32_t par = (sym[0] + sym[1] + sym[2]) & 1;
  p[0] = (float)sym[0]; p[1] = (float)sym[1]; p[2] = (float)sym[2];
  p[3] = (float)(2 * sym[3] + par);
}
template <> __device__ __forceinline__ void unstrip_embed<3>(const int32_t* sym, uint32_t raw, float* p) {
  int32_t par = 0;
#pragma unroll
  for (int i = 0; i < 7; ++i) par += sym[i];
  par &= 1;
  int32_t b = (int32_t)raw;
#pragma unroll
  for (int i = 0; i < 7; ++i) p[i] = (float)(2 * sym[i] + b);
  p[7] = (float)(2 * (2 * sym[7] + par) + b);
}

// Quantise the lane's 8 values [HQ Methodology 2] and strip them
// [Methodology 3]: the symbols as w = 2 zigzag(sym) + 1, and for E8 the coset
// bit.  Symbols: Z x; A2 (i - (j & 1)) >> 1 and j; D4 x0, x1, x2,
// (x3 - parity(x0+x1+x2)) >> 1; E8 the halves y_0..y_6 and y_7 >> 1 (the sum
// of the halves is even).  Z, D4 and E8 work on integers biased by kMagicBits
// (even, so parities and halvings carry over).
template <int L>
__device__ __forceinline__ void quantize_syms(const float u[8], uint32_t w[8], bool& odd) {
  odd = false;
  if constexpr (L == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = zz1_biased(fbits(u[i] + kMagic), kFourMagic);
  } else if constexpr (L == 1) {
#pragma unroll
    for (int h = 0; h < 8; h += 2) {
      int32_t i, j;
      np_a2_codes(u[h], u[h + 1], i, j);
      w[h] = zz1((i - (j & 1)) >> 1);
      w[h + 1] = zz1(j);
    }
  } else if constexpr (L == 2) {
#pragma unroll
    for (int h = 0; h < 8; h += 4) {
      int32_t x[4];
      d4_core(&u[h], x, 0u);
      const uint32_t p = ((uint32_t)x[0] ^ (uint32_t)x[1] ^ (uint32_t)x[2]) & 1u;
      w[h] = zz1_biased((uint32_t)x[0], kFourMagic);
      w[h + 1] = zz1_biased((uint32_t)x[1], kFourMagic);
      w[h + 2] = zz1_biased((uint32_t)x[2], kFourMagic);
      w[h + 3] = zz1_biased(((uint32_t)x[3] - p) >> 1, kTwoMagic);
    }
  } else {
    int32_t y[8];
    e8_core(u, y, odd, 0u);
#pragma unroll
    for (int i = 0; i < 7; ++i) w[i] = zz1_biased((uint32_t)y[i], kFourMagic);
    w[7] = zz1_biased((uint32_t)y[7] >> 1, kTwoMagic);
  }
}

// Subtractive dither of the lane's 8 coordinates [HQ Methodology 4]:
// tau uniform over one period of an integer sublattice, d = tau - Q(tau).
// Philox block j = coordinate/4 of tile id T: counter (j, lo32 T, hi32 T, "DITH").
template <int L>
__device__ __forceinline__ void dither_lane(uint32_t k0, uint32_t k1, uint64_t tile_id, int v, float d[8]) {
  float f[8];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    uint32_t c[4] = {(uint32_t)(2 * v + b), (uint32_t)tile_id, (uint32_t)(tile_id >> 32), kTagDither};
    philox4x32_10(c, k0, k1);
#pragma unroll
    for (int q = 0; q < 4; ++q) f[4 * b + q] = (float)(c[q] >> 8) * 0x1p-24f;
  }
  float tau[8];
  if constexpr (L == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) d[i] = f[i] - __builtin_rintf(f[i]);
  } else if constexpr (L == 1) {
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      tau[i] = 2.0f * f[i];
      tau[i + 1] = f[i + 1] * (2.0f * kSqrt3);
      int32_t ci, cj;
      np_a2_codes(tau[i], tau[i + 1], ci, cj);
      d[i] = tau[i] - (float)ci;
      d[i + 1] = tau[i + 1] - (float)cj * kSqrt3;
    }
  } else if constexpr (L == 2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) tau[i] = 2.0f * f[i];
    int32_t x[8];
    d4_core(&tau[0], &x[0], kMagicBits);
    d4_core(&tau[4], &x[4], kMagicBits);
#pragma unroll
    for (int i = 0; i < 8; ++i) d[i] = tau[i] - (float)x[i];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) tau[i] = 4.0f * f[i];
    int32_t y[8];
    bool odd;
    e8_core(tau, y, odd, kMagicBits);
#pragma unroll
    for (int i = 0; i < 8; ++i) d[i] = tau[i] - (float)(2 * y[i] + (odd ? 1 : 0));
  }
}

}  // namespace hq
