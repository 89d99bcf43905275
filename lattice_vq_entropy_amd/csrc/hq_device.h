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

struct FwhtSigns {
  float c0, c1, c2, c3;  // +1 / -1 per cross-lane stage: bit s of the lane's vector
  float lane_sign;       // (-1)^popcount(v)
};

__device__ __forceinline__ FwhtSigns fwht_signs(int v) {
  FwhtSigns s;
  s.c0 = (v & 1) ? -1.0f : 1.0f;
  s.c1 = (v & 2) ? -1.0f : 1.0f;
  s.c2 = (v & 4) ? -1.0f : 1.0f;
  s.c3 = (v & 8) ? -1.0f : 1.0f;
  s.lane_sign = (__builtin_popcount(v) & 1) ? -1.0f : 1.0f;
  return s;
}

__device__ __forceinline__ void fwht_tile(float x[8], const FwhtSigns& fs) {
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
  c = fs.c0; HQ_DPP_STAGE("quad_perm:[1,0,3,2]");  // stride 8
  c = fs.c1; HQ_DPP_STAGE("quad_perm:[2,3,0,1]");  // stride 16
  c = fs.c2; HQ_DPP_STAGE("row_half_mirror");      // stride 32
  c = fs.c3; HQ_DPP_STAGE("row_ror:8");            // stride 64
}

// ---------------------------------------------------------------------------
// Philox4x32-10 [Philox]
// ---------------------------------------------------------------------------
__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint32_t lo0 = 0xD2511F53u * c[0], hi0 = __umulhi(0xD2511F53u, c[0]);
    uint32_t lo1 = 0xCD9E8D57u * c[2], hi1 = __umulhi(0xCD9E8D57u, c[2]);
    uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
    k0 += 0x9E3779B9u; k1 += 0xBB67AE85u;
  }
}

// ---------------------------------------------------------------------------
// Nearest points [HQ Methodology 2; SPLAG ch. 20] in the integer embeddings
// Z, A2 checkerboard {(i,j): i = j mod 2} with real point (i, j sqrt3),
// D4 = {x in Z^4: sum even}, 2E8.  Outputs are the stripped symbols
// [HQ Methodology 3] of each vector directly, and for E8 the raw coset bit.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void np_z(const float* u, int32_t* sym) {
  sym[0] = (int32_t)__builtin_rintf(u[0]);
}

// D4: round, fix the parity on the first coordinate of largest error; symbols
// x0, x1, x2 and (x3 - parity(x0+x1+x2)) >> 1.
__device__ __forceinline__ void np_d4(const float* u, int32_t* sym) {
  float f[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __builtin_rintf(u[i]);
  int32_t xi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xi[i] = (int32_t)f[i];
  int32_t s = xi[0] + xi[1] + xi[2] + xi[3];
  if (s & 1) {
    float e[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) e[i] = __builtin_fabsf(u[i] - f[i]);
    int j = 0;
    float w = e[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) if (e[i] > w) { w = e[i]; j = i; }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i == j) xi[i] += (u[i] - f[i] >= 0.0f) ? 1 : -1;
  }
  int32_t p = (xi[0] + xi[1] + xi[2]) & 1;
  sym[0] = xi[0]; sym[1] = xi[1]; sym[2] = xi[2];
  sym[3] = (xi[3] - p) >> 1;
}

// A2: best of the two rectangular cosets; symbols (i - (j & 1)) >> 1 and j.
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

__device__ __forceinline__ void np_a2(const float* u, int32_t* sym) {
  int32_t i, j;
  np_a2_codes(u[0], u[1], i, j);
  sym[0] = (i - (j & 1)) >> 1;
  sym[1] = j;
}

// 2E8 = 2D8 u (2D8 + 1).  With h = u/2, ye = rint(h), yo = floor(h) and
// a_i = |u_i - 2 ye_i| (exact), the halved squared-distance difference of the
// parity-fixed even and odd candidates is
//   (sum a_i - 4) + [sum ye odd] 2 (1 - max a) - [sum yo odd] 2 min a,
// evaluated in fp32 in this order (sum sequential); even wins ties.  The fix
// moves the first coordinate of largest |u - c| by 2 toward u.  Symbols: the
// halves y_i = (x_i - b) / 2 with y_7's redundant low bit dropped, i.e. y_7 >> 1
// (the sum of the halves is even), and the raw coset bit b.
__device__ __forceinline__ void np_e8(const float* u, int32_t* sym, uint32_t& raw) {
  float ye[8], yo[8], a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float h = u[i] * 0.5f;
    ye[i] = __builtin_rintf(h);
    yo[i] = __builtin_floorf(h);
    a[i] = __builtin_fabsf(__builtin_fmaf(-2.0f, ye[i], u[i]));  // exact
  }
  float S = a[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) S = S + a[i];
  float sye = ye[0], syo = yo[0];  // integer-valued sums: exact in fp32
#pragma unroll
  for (int i = 1; i < 8; ++i) { sye = sye + ye[i]; syo = syo + yo[i]; }
  int pe = (int32_t)sye & 1, po = (int32_t)syo & 1;
  float amax = a[0], amin = a[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) { amax = __builtin_fmaxf(amax, a[i]); amin = __builtin_fminf(amin, a[i]); }
  float delta = S - 4.0f;
  if (pe) delta = delta + 2.0f * (1.0f - amax);
  if (po) delta = delta - 2.0f * amin;
  bool even = delta <= 0.0f;
  float target = even ? amax : amin;
  int fix = even ? pe : po;
  // first coordinate attaining the target
  int j = 7;
#pragma unroll
  for (int i = 6; i >= 0; --i) j = (a[i] == target) ? i : j;
  int32_t y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = (int32_t)(even ? ye[i] : yo[i]);
  if (fix) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i != j) continue;
      // even: direction of u - 2ye; odd: of u - (2yo + 1)
      float c = even ? 2.0f * ye[i] : __builtin_fmaf(2.0f, yo[i], 1.0f);
      y[i] += (u[i] - c >= 0.0f) ? 1 : -1;
    }
  }
#pragma unroll
  for (int i = 0; i < 7; ++i) sym[i] = y[i];
  sym[7] = y[7] >> 1;
  raw = even ? 0u : 1u;
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

// Quantise the 8 values of one lane to symbols (and raw bits for E8).
template <int L> __device__ __forceinline__ void quantize_lane(const float u[8], int32_t sym[8], uint32_t& raw) {
  raw = 0;
  if constexpr (L == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) np_z(&u[i], &sym[i]);
  } else if constexpr (L == 1) {
#pragma unroll
    for (int i = 0; i < 8; i += 2) np_a2(&u[i], &sym[i]);
  } else if constexpr (L == 2) {
    np_d4(&u[0], &sym[0]);
    np_d4(&u[4], &sym[4]);
  } else {
    np_e8(u, sym, raw);
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
    int32_t s[8];
    np_d4(&tau[0], &s[0]);
    np_d4(&tau[4], &s[4]);
    float p[8];
    unstrip_embed<2>(&s[0], 0, &p[0]);
    unstrip_embed<2>(&s[4], 0, &p[4]);
#pragma unroll
    for (int i = 0; i < 8; ++i) d[i] = tau[i] - p[i];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) tau[i] = 4.0f * f[i];
    int32_t s[8];
    uint32_t raw;
    np_e8(tau, s, raw);
    float p[8];
    unstrip_embed<3>(s, raw, p);
#pragma unroll
    for (int i = 0; i < 8; ++i) d[i] = tau[i] - p[i];
  }
}

__device__ __forceinline__ uint32_t zigzag(int32_t v) {
  return ((uint32_t)v << 1) ^ (uint32_t)(v >> 31);
}
__device__ __forceinline__ int32_t unzigzag(uint32_t m) {
  return (int32_t)(m >> 1) ^ -(int32_t)(m & 1u);
}

}  // namespace hq
