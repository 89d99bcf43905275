/*
 * hq_oracle.c -- plain, slow CPU reference of the HyperQuant per-tile codec.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the package smoke check and
 * the benchmark's CPU-baseline leg; never by the product path.  It shares no
 * code with the HIP library.  Source citations use the short names defined in
 * hq_oracle.h ([HQ-explainer], [HQ-abstract], [Philox], [SPLAG]).
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (no -ffast-math, no -march):
 * every fp32 operation below is one IEEE-754 binary32 operation rounded to
 * nearest-even, in the order written.  Where floating point decides an integer
 * (a lattice code), the HIP path takes the same decision in the same precision
 * and order, which is what makes codes and bitstreams comparable bit for bit.
 */
#include "hq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define N 128                 /* tile length [HQ-explainer, Methodology 1] */
#define KMAX 22               /* largest Rice parameter (reading: |u| < 2^20) */
#define RANGE_LIMIT 1048576.0f /* 2^20: codes stay below 2^21 */
#define M_LIMIT (1u << 22)    /* largest zigzag symbol a valid stream holds */

/* Host threads for whole-tensor encode, decode and rate passes (1: the plain
 * serial loops).  With more, the per-tile steps run on that many OpenMP
 * threads; see the parallel section below.  The results do not depend on it. */
static int g_threads = 1;
void orc_set_threads(int n) { g_threads = n > 0 ? n : 1; }
int orc_get_threads(void) { return g_threads; }

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 [Philox]: ten rounds of two 32x32->64 multiplies with the   */
/* published multipliers, the key bumped by the published Weyl constants.    */
/* ------------------------------------------------------------------------ */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)M0 * c0;
    uint64_t p1 = (uint64_t)M1 * c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += W0; k1 += W1;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Counter tags (reading): the sign vector uses counter (0,0,0,"SIGN"); the
 * dither block j of tile id T uses counter (j, lo32(T), hi32(T), "DITH"). */
#define TAG_SIGN 0x5349474Eu
#define TAG_DITH 0x44495448u

/* D of RHT_n(x) = H_n D x [HQ-explainer, Methodology 1]: one random sign per
 * coordinate, shared by every tile of a plan (reading: the "cheap +-1 sign
 * diagonal" per-layer rotation of Methodology 4 is this D). */
void orc_signs(uint64_t seed, float s[128]) {
  uint32_t ctr[4] = {0u, 0u, 0u, TAG_SIGN};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t r[4];
  orc_philox4x32_10(ctr, key, r);
  for (int i = 0; i < N; ++i) s[i] = ((r[i >> 5] >> (i & 31)) & 1u) ? -1.0f : 1.0f;
}

/* H_n of Methodology 1: the Walsh-Hadamard matrix in Sylvester order,
 * applied by the textbook butterfly, smallest stride first. */
void orc_fwht128(float v[128]) {
  for (int h = 1; h < N; h <<= 1) {
    for (int i = 0; i < N; ++i) {
      if (i & h) continue;
      float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
}

/* The orthonormal scale 1/sqrt(n) and the lattice scale alpha of
 * Methodology 2 ("integer implementation ... scale alpha") are folded into one
 * fp32 constant each way, computed in double and rounded once. */
void orc_scales(float alpha, float *c_enc, float *c_dec) {
  *c_enc = (float)(1.0 / ((double)alpha * sqrt(128.0)));
  *c_dec = (float)((double)alpha / sqrt(128.0));
}

void orc_rht_forward(const float x[128], const float s[128], float c_enc, float u[128]) {
  float v[N];
  for (int i = 0; i < N; ++i) v[i] = s[i] * x[i];
  orc_fwht128(v);
  for (int i = 0; i < N; ++i) u[i] = v[i] * c_enc;
}

/* ------------------------------------------------------------------------ */
/* The second rotation of Methodology 1: a Haar-uniform random orthogonal   */
/* 128 x 128 matrix Q (the "QJL" rotation the explainer compares with the   */
/* RHT for the KV cache; paper abstract, item (i)).  Reading of the recipe:  */
/* the QR factor with positive diagonal R of a matrix of independent        */
/* standard normals is Haar distributed [Mezzadri, Notices AMS 54 (2007)].  */
/*   G[i][j] = g[128 i + j]; pair p = 0..8191 of g from Philox4x32-10       */
/*   (counter (p, 0, 0, "HAAR"), key = seed): u1 = (r0 + 1) / 2^32,        */
/*   u2 = r1 / 2^32, g[2p] = sqrt(-2 ln u1) cos(2 pi u2), g[2p+1] = ... sin  */
/*   (Box-Muller), in double;                                               */
/*   Q = Gram-Schmidt of the columns of G (modified form, dot products and  */
/*   updates in index order, double), which gives R_jj > 0; rounded to fp32. */
/* The rotated tile is u = Q x / alpha, computed as u_i = fl32(t_i c_enc)   */
/* with t_i the fp32 fma chain over j = 0..127 of Q[i][j] x_j and            */
/* c_enc = fp32(1 / alpha) (Q is orthonormal: no 1/sqrt(n)); the inverse is */
/* x_i = fl32(t'_i c_dec), t'_i the fp32 fma chain of Q[j][i] u_j, c_dec =  */
/* alpha.                                                                   */
/* ------------------------------------------------------------------------ */
#define ORC_TAG_HAAR 0x48414152u /* "HAAR" */

void orc_haar(uint64_t seed, float q32[128 * 128]) {
  double *g = (double *)malloc(sizeof(double) * N * N);
  double *q = (double *)malloc(sizeof(double) * N * N);
  double v[N];
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  for (uint32_t p = 0; p < N * N / 2; ++p) {
    const uint32_t ctr[4] = {p, 0u, 0u, ORC_TAG_HAAR};
    uint32_t r[4];
    orc_philox4x32_10(ctr, key, r);
    const double u1 = ((double)r[0] + 1.0) / 4294967296.0;
    const double u2 = (double)r[1] / 4294967296.0;
    const double rad = sqrt(-2.0 * log(u1)), ang = 6.283185307179586 * u2;
    g[2 * p] = rad * cos(ang);
    g[2 * p + 1] = rad * sin(ang);
  }
  for (int j = 0; j < N; ++j) {
    for (int i = 0; i < N; ++i) v[i] = g[i * N + j];
    for (int c = 0; c < j; ++c) {
      double r = 0.0;
      for (int i = 0; i < N; ++i) r = r + q[i * N + c] * v[i];
      for (int i = 0; i < N; ++i) v[i] = v[i] - r * q[i * N + c];
    }
    double nrm = 0.0;
    for (int i = 0; i < N; ++i) nrm = nrm + v[i] * v[i];
    nrm = sqrt(nrm);
    for (int i = 0; i < N; ++i) q[i * N + j] = v[i] / nrm;
  }
  for (int i = 0; i < N * N; ++i) q32[i] = (float)q[i];
  free(g);
  free(q);
}

/* The rotation of a plan: the RHT (signs s, c_enc = 1/(alpha sqrt n)) or the
 * Haar matrix (c_enc = 1/alpha). */
typedef struct {
  int haar;
  float s[N];
  float c_enc, c_dec;
  float *q; /* haar: 128 x 128, row-major */
} rot_ctx;

static int ctx_init(rot_ctx *r, int rot, uint64_t seed, float alpha) {
  r->haar = rot;
  r->q = NULL;
  if (rot == 0) {
    orc_signs(seed, r->s);
    orc_scales(alpha, &r->c_enc, &r->c_dec);
    return ORC_OK;
  }
  if (rot != 1) return ORC_ERR_ARG;
  r->q = (float *)malloc(sizeof(float) * N * N);
  if (!r->q) return ORC_ERR_ARG;
  orc_haar(seed, r->q);
  r->c_enc = (float)(1.0 / (double)alpha);
  r->c_dec = alpha;
  return ORC_OK;
}

static void ctx_free(rot_ctx *r) { free(r->q); }

static void ctx_forward(const rot_ctx *r, const float x[N], float u[N]) {
  if (!r->haar) {
    orc_rht_forward(x, r->s, r->c_enc, u);
    return;
  }
  for (int i = 0; i < N; ++i) {
    float t = 0.0f;
    for (int j = 0; j < N; ++j) t = fmaf(r->q[i * N + j], x[j], t);
    u[i] = t * r->c_enc;
  }
}

static void ctx_inverse(const rot_ctx *r, float v[N]) {
  if (!r->haar) {
    orc_fwht128(v);
    for (int i = 0; i < N; ++i) v[i] = r->s[i] * (v[i] * r->c_dec);
    return;
  }
  float out[N];
  for (int i = 0; i < N; ++i) {
    float t = 0.0f;
    for (int j = 0; j < N; ++j) t = fmaf(r->q[j * N + i], v[j], t);
    out[i] = t * r->c_dec;
  }
  memcpy(v, out, sizeof(out));
}

/* ------------------------------------------------------------------------ */
/* Nearest points [HQ-explainer, Methodology 2; SPLAG ch. 20]               */
/* Integer embeddings (reading): Z; D4 = {x in Z^4 : sum even};             */
/* E8 as 2E8 = {x in Z^8 : all x_i of one parity, sum = 0 mod 4}            */
/* (the E^8_int subset Z^8 of Methodology 2); A2 as the checkerboard        */
/* {(i,j) : i = j mod 2} whose real point is (i, j*sqrt3).                  */
/* ------------------------------------------------------------------------ */
static const float S3 = 1.7320508075688772f;        /* fp32(sqrt 3) */
static const float K3 = 0.28867513459481287f;       /* fp32(1/(2 sqrt 3)) */

static int lat_dim(int lat) {
  switch (lat) {
    case ORC_Z: return 1;
    case ORC_A2: return 2;
    case ORC_D4: return 4;
    case ORC_E8: return 8;
    default: return 0;
  }
}

static void nearest_z(const float *u, int32_t *x) { x[0] = (int32_t)rintf(u[0]); }

/* D4: round every coordinate; if the sum is odd, re-round the coordinate with
 * the largest rounding error (first such index) the other way. */
static void nearest_d4(const float *u, int32_t *x) {
  float f[4];
  int32_t sum = 0;
  for (int i = 0; i < 4; ++i) { f[i] = rintf(u[i]); sum += (int32_t)f[i]; }
  if (sum & 1) {
    int j = 0;
    float worst = fabsf(u[0] - f[0]);
    for (int i = 1; i < 4; ++i) {
      float e = fabsf(u[i] - f[i]);
      if (e > worst) { worst = e; j = i; }
    }
    f[j] += (u[j] - f[j] >= 0.0f) ? 1.0f : -1.0f;
  }
  for (int i = 0; i < 4; ++i) x[i] = (int32_t)f[i];
}

/* 2E8 = 2D8 u (2D8 + 1).  Even candidate: nearest even integers e_i, parity
 * fixed on the coordinate with the largest |u_i - e_i|.  Odd candidate:
 * nearest odd integers o_i, parity fixed on the coordinate with the largest
 * |u_i - o_i| = 1 - |u_i - e_i|, i.e. the smallest a_i.  With a_i = |u_i - e_i|
 * (exact in fp32) the squared distances satisfy
 *   (D_even - D_odd)/2 = (sum a_i - 4) + [even fix] 2(1 - max a) - [odd fix] 2 min a,
 * which is evaluated in fp32 in exactly this order; even wins ties. */
static void nearest_e8(const float *u, int32_t *x) {
  float ye[8], yo[8], a[8];
  int32_t sye = 0, syo = 0;
  for (int i = 0; i < 8; ++i) {
    float h = u[i] * 0.5f;
    ye[i] = rintf(h);
    yo[i] = floorf(h);
    a[i] = fabsf(u[i] - 2.0f * ye[i]);
    sye += (int32_t)ye[i];
    syo += (int32_t)yo[i];
  }
  float S = a[0];
  for (int i = 1; i < 8; ++i) S = S + a[i];
  int jmax = 0, jmin = 0;
  for (int i = 1; i < 8; ++i) {
    if (a[i] > a[jmax]) jmax = i;
    if (a[i] < a[jmin]) jmin = i;
  }
  int pe = sye & 1, po = syo & 1;
  float delta = S - 4.0f;
  if (pe) delta = delta + 2.0f * (1.0f - a[jmax]);
  if (po) delta = delta - 2.0f * a[jmin];
  int32_t c[8];
  if (delta <= 0.0f) {
    for (int i = 0; i < 8; ++i) c[i] = 2 * (int32_t)ye[i];
    if (pe) c[jmax] += (u[jmax] - (float)c[jmax] >= 0.0f) ? 2 : -2;
  } else {
    for (int i = 0; i < 8; ++i) c[i] = 2 * (int32_t)yo[i] + 1;
    if (po) c[jmin] += (u[jmin] - (float)c[jmin] >= 0.0f) ? 2 : -2;
  }
  for (int i = 0; i < 8; ++i) x[i] = c[i];
}

/* A2: the real lattice {(i, j sqrt3) : i = j mod 2} is the union of two
 * rectangular cosets, rounded independently; the closer one wins (ties even). */
static float a2_dist(const float *u, int32_t i, int32_t j) {
  float e0 = u[0] - (float)i;
  float t = (float)j * S3;
  float e1 = u[1] - t;
  return e0 * e0 + e1 * e1;
}

static void nearest_a2(const float *u, int32_t *x) {
  float w0 = u[0] * 0.5f, w1 = u[1] * K3;
  int32_t ie = 2 * (int32_t)rintf(w0), je = 2 * (int32_t)rintf(w1);
  int32_t io = 2 * (int32_t)floorf(w0) + 1, jo = 2 * (int32_t)floorf(w1) + 1;
  float de = a2_dist(u, ie, je), dd = a2_dist(u, io, jo);
  if (de <= dd) { x[0] = ie; x[1] = je; }
  else { x[0] = io; x[1] = jo; }
}

void orc_nearest(int lat, const float *u, int32_t *x) {
  switch (lat) {
    case ORC_Z: nearest_z(u, x); break;
    case ORC_A2: nearest_a2(u, x); break;
    case ORC_D4: nearest_d4(u, x); break;
    case ORC_E8: nearest_e8(u, x); break;
    default: break;
  }
}

void orc_nearest_many(int lat, uint64_t n_vectors, const float *u, int32_t *x) {
  int d = lat_dim(lat);
  for (uint64_t r = 0; r < n_vectors; ++r) orc_nearest(lat, &u[r * (uint64_t)d], &x[r * (uint64_t)d]);
}

void orc_embed(int lat, const int32_t *x, float *p) {
  int d = lat_dim(lat);
  if (lat == ORC_A2) {
    p[0] = (float)x[0];
    p[1] = (float)x[1] * S3;
    return;
  }
  for (int i = 0; i < d; ++i) p[i] = (float)x[i];
}

/* ------------------------------------------------------------------------ */
/* Bit-stripping [HQ-explainer, Methodology 3]: the membership constraints   */
/* fix log2(index) bits of every code vector; they are removed before        */
/* coding.  E8: the common parity b (kept as one raw bit), then the halves   */
/* y_i = (x_i - b)/2 whose sum is even, so y_7's low bit is dropped.  D4:    */
/* x_3's low bit equals the parity of x_0+x_1+x_2.  A2: i's low bit equals   */
/* j's; i (real step 2 once stripped) and j (real step sqrt3) then have      */
/* nearly equal spread, so one Rice parameter fits both.  (Shifts below are  */
/* arithmetic, i.e. floor division.)                                         */
/* ------------------------------------------------------------------------ */
void orc_strip(int lat, const int32_t *x, int32_t *sym, int *raw_bit) {
  *raw_bit = 0;
  switch (lat) {
    case ORC_Z: sym[0] = x[0]; break;
    case ORC_A2: sym[0] = (x[0] - (x[1] & 1)) >> 1; sym[1] = x[1]; break;
    case ORC_D4: {
      int32_t p = (x[0] + x[1] + x[2]) & 1;
      sym[0] = x[0]; sym[1] = x[1]; sym[2] = x[2];
      sym[3] = (x[3] - p) >> 1;
      break;
    }
    case ORC_E8: {
      int32_t b = x[0] & 1, y[8], p = 0;
      for (int i = 0; i < 8; ++i) y[i] = (x[i] - b) >> 1;
      for (int i = 0; i < 7; ++i) p += y[i];
      p &= 1;
      for (int i = 0; i < 7; ++i) sym[i] = y[i];
      sym[7] = (y[7] - p) >> 1;
      *raw_bit = b;
      break;
    }
    default: break;
  }
}

void orc_unstrip(int lat, const int32_t *sym, int raw_bit, int32_t *x) {
  switch (lat) {
    case ORC_Z: x[0] = sym[0]; break;
    case ORC_A2: x[0] = 2 * sym[0] + (sym[1] & 1); x[1] = sym[1]; break;
    case ORC_D4: {
      int32_t p = (sym[0] + sym[1] + sym[2]) & 1;
      x[0] = sym[0]; x[1] = sym[1]; x[2] = sym[2];
      x[3] = 2 * sym[3] + p;
      break;
    }
    case ORC_E8: {
      int32_t y[8], p = 0;
      for (int i = 0; i < 7; ++i) { y[i] = sym[i]; p += sym[i]; }
      p &= 1;
      y[7] = 2 * sym[7] + p;
      for (int i = 0; i < 8; ++i) x[i] = 2 * y[i] + raw_bit;
      break;
    }
    default: break;
  }
}

/* Signed to unsigned for Rice coding (reading: zigzag). */
uint32_t orc_zigzag(int32_t v) { return v >= 0 ? 2u * (uint32_t)v : 2u * (uint32_t)(-(int64_t)v) - 1u; }
int32_t orc_unzigzag(uint32_t m) { return (m & 1u) ? -(int32_t)((m + 1u) >> 1) : (int32_t)(m >> 1); }

/* Rice coding [HQ-explainer, Methodology 3]: symbol m costs a k-bit remainder
 * plus a unary quotient (m >> k zeros and a terminating one).  One k per tile,
 * the smallest minimiser of the tile length (reading). */
uint64_t orc_rice_len(const uint32_t m[128], int k, int raw_bits) {
  uint64_t L = (uint64_t)raw_bits + (uint64_t)N * (uint64_t)(1 + k);
  for (int i = 0; i < N; ++i) L += (uint64_t)(m[i] >> k);
  return L;
}

int orc_rice_kstar(const uint32_t m[128], int raw_bits) {
  int best = 0;
  uint64_t bestL = orc_rice_len(m, 0, raw_bits);
  for (int k = 1; k <= KMAX; ++k) {
    uint64_t L = orc_rice_len(m, k, raw_bits);
    if (L < bestL) { bestL = L; best = k; }
  }
  return best;
}

/* ------------------------------------------------------------------------ */
/* Subtractive dither [HQ-explainer, Methodology 4]: U ~ Uniform(V(Lambda)). */
/* Construction (reading): tau uniform over one period of an integer         */
/* sublattice (4Z^8 in 2E8, 2Z^4 in D4, 2Z x 2sqrt3 Z in A2, Z), then        */
/* d = tau - Q(tau), which is uniform over the Voronoi cell.  Uniforms are   */
/* 24-bit: f = (r >> 8) * 2^-24 from Philox block j = coordinate / 4.        */
/* ------------------------------------------------------------------------ */
void orc_dither(int lat, uint64_t seed, uint64_t tile_id, float d[128]) {
  float f[N];
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  for (uint32_t j = 0; j < N / 4; ++j) {
    uint32_t ctr[4] = {j, (uint32_t)tile_id, (uint32_t)(tile_id >> 32), TAG_DITH};
    uint32_t r[4];
    orc_philox4x32_10(ctr, key, r);
    for (int c = 0; c < 4; ++c) f[4 * j + c] = (float)(r[c] >> 8) * 0x1p-24f;
  }
  int dim = lat_dim(lat);
  for (int v = 0; v < N / dim; ++v) {
    float tau[8], p[8];
    int32_t q[8];
    for (int c = 0; c < dim; ++c) {
      float fv = f[v * dim + c];
      switch (lat) {
        case ORC_Z: tau[c] = fv; break;
        case ORC_D4: tau[c] = 2.0f * fv; break;
        case ORC_E8: tau[c] = 4.0f * fv; break;
        case ORC_A2: tau[c] = (c == 0) ? 2.0f * fv : fv * (2.0f * S3); break;
        default: tau[c] = 0.0f; break;
      }
    }
    orc_nearest(lat, tau, q);
    orc_embed(lat, q, p);
    for (int c = 0; c < dim; ++c) d[v * dim + c] = tau[c] - p[c];
  }
}

/* ------------------------------------------------------------------------ */
/* Tile quantiser: RHT -> (dither) -> nearest point, range-checked.          */
/* ------------------------------------------------------------------------ */
static float load_elem(const void *x, int dtype, uint64_t i) {
  if (dtype == ORC_BF16) {
    uint32_t b = (uint32_t)((const uint16_t *)x)[i] << 16;
    float f;
    memcpy(&f, &b, 4);
    return f;
  }
  return ((const float *)x)[i];
}

static int quantize_tile_s(int lat, uint64_t seed, const rot_ctx *r,
                           const float x[128], int dithered, uint64_t tile_id,
                           int32_t codes[128]) {
  for (int i = 0; i < N; ++i)
    if (!isfinite(x[i])) return ORC_ERR_NONFINITE;
  float u[N];
  ctx_forward(r, x, u);
  if (dithered) {
    float d[N];
    orc_dither(lat, seed, tile_id, d);
    for (int i = 0; i < N; ++i) u[i] = u[i] + d[i];
  }
  for (int i = 0; i < N; ++i)
    if (!(fabsf(u[i]) < RANGE_LIMIT)) return ORC_ERR_RANGE;
  int dim = lat_dim(lat);
  for (int v = 0; v < N / dim; ++v) orc_nearest(lat, &u[v * dim], &codes[v * dim]);
  return ORC_OK;
}

int orc_quantize_tile(int lat, uint64_t seed, float alpha, const float x[128],
                      int dithered, uint64_t tile_id, int32_t codes[128]) {
  if (lat_dim(lat) == 0 || !(alpha > 0.0f) || !isfinite(alpha)) return ORC_ERR_ARG;
  rot_ctx r;
  ctx_init(&r, 0, seed, alpha);
  return quantize_tile_s(lat, seed, &r, x, dithered, tile_id, codes);
}

/* Codes of a tile -> zigzag symbols (vector-major) and raw bits. */
static int tile_symbols(int lat, const int32_t codes[128], uint32_t m[128], uint32_t *raw) {
  int dim = lat_dim(lat);
  *raw = 0;
  for (int v = 0; v < N / dim; ++v) {
    int32_t sym[8];
    int rb;
    orc_strip(lat, &codes[v * dim], sym, &rb);
    for (int c = 0; c < dim; ++c) m[v * dim + c] = orc_zigzag(sym[c]);
    if (lat == ORC_E8) *raw |= (uint32_t)rb << v;
  }
  return lat == ORC_E8 ? 16 : 0;
}

/* ------------------------------------------------------------------------ */
/* Stream layout (reading; parity unpinned by the pages):                    */
/*   record of tile t at bits [off[t], off[t+1]):                            */
/*     [raw bits (E8: bit v = coset bit of vector v)]                        */
/*     [128 remainders of k bits, symbol order, each LSB first]              */
/*     [128 unary quotients: q zeros then a one, symbol order]               */
/*   stream bit P is bit (P & 31) of uint32 word P >> 5; records abut.       */
/* ------------------------------------------------------------------------ */
static void put_bit(uint32_t *w, uint64_t pos) { w[pos >> 5] |= 1u << (pos & 31); }
/* the same when several threads write records that share a boundary word */
static void put_bit_atomic(uint32_t *w, uint64_t pos) {
  __atomic_fetch_or(&w[pos >> 5], 1u << (pos & 31), __ATOMIC_RELAXED);
}
static int get_bit(const uint32_t *w, uint64_t pos) { return (int)((w[pos >> 5] >> (pos & 31)) & 1u); }

static void write_record_with(void (*put)(uint32_t *, uint64_t), uint32_t *words, uint64_t off, int raw_bits,
                              uint32_t raw, const uint32_t m[128], int k) {
  uint64_t p = off;
  for (int b = 0; b < raw_bits; ++b, ++p)
    if ((raw >> b) & 1u) put(words, p);
  for (int i = 0; i < N; ++i)
    for (int b = 0; b < k; ++b, ++p)
      if ((m[i] >> b) & 1u) put(words, p);
  for (int i = 0; i < N; ++i) {
    p += m[i] >> k;
    put(words, p);
    ++p;
  }
}

static void write_record(uint32_t *words, uint64_t off, int raw_bits, uint32_t raw,
                         const uint32_t m[128], int k) {
  write_record_with(put_bit, words, off, raw_bits, raw, m, k);
}

static int encode_par(int lat, uint64_t seed, const rot_ctx *r, const void *x, int dtype, uint64_t n_tiles,
                      int dithered, uint64_t tile_base, uint32_t *words, uint64_t cap_words, uint64_t *offsets,
                      uint8_t *k);
static int total_bits_par(int lat, uint64_t seed, const rot_ctx *r, const void *x, int dtype, uint64_t n_tiles,
                          int dithered, uint64_t tile_base, uint64_t *bits);
static int decode_par(int lat, uint64_t seed, const rot_ctx *r, const uint32_t *words, const uint64_t *offsets,
                      const uint8_t *k, uint64_t n_tiles, int dithered, uint64_t tile_base, void *y, int dtype);

uint64_t orc_write_record_codes(int lat, const int32_t codes[128], uint32_t *words,
                                uint64_t off, int *k_out) {
  uint32_t m[N], raw;
  int raw_bits = tile_symbols(lat, codes, m, &raw);
  int kt = orc_rice_kstar(m, raw_bits);
  write_record(words, off, raw_bits, raw, m, kt);
  *k_out = kt;
  return orc_rice_len(m, kt, raw_bits);
}

int orc_encode(int lat, uint64_t seed, float alpha, const void *x, int dtype,
               uint64_t n_tiles, int dithered, uint64_t tile_base,
               uint32_t *words, uint64_t cap_words, uint64_t *offsets, uint8_t *k) {
  return orc_encode_r(lat, seed, alpha, 0, x, dtype, n_tiles, dithered, tile_base, words, cap_words,
                      offsets, k);
}

int orc_encode_r(int lat, uint64_t seed, float alpha, int rot, const void *x, int dtype,
                 uint64_t n_tiles, int dithered, uint64_t tile_base,
                 uint32_t *words, uint64_t cap_words, uint64_t *offsets, uint8_t *k) {
  if (lat_dim(lat) == 0 || !(alpha > 0.0f) || !isfinite(alpha)) return ORC_ERR_ARG;
  if (dtype != ORC_F32 && dtype != ORC_BF16) return ORC_ERR_ARG;
  rot_ctx r;
  if (ctx_init(&r, rot, seed, alpha) != ORC_OK) return ORC_ERR_ARG;
  if (g_threads > 1) {
    int st = encode_par(lat, seed, &r, x, dtype, n_tiles, dithered, tile_base, words, cap_words, offsets, k);
    ctx_free(&r);
    return st;
  }
  int status = ORC_OK;
  uint64_t off = 0, zeroed = 0; /* words [0, zeroed) have been cleared */
  offsets[0] = 0;
  for (uint64_t t = 0; t < n_tiles; ++t) {
    float xt[N];
    int32_t codes[N];
    uint32_t m[N], raw;
    for (int i = 0; i < N; ++i) xt[i] = load_elem(x, dtype, t * N + (uint64_t)i);
    int st = quantize_tile_s(lat, seed, &r, xt, dithered, tile_base + t, codes);
    if (st != ORC_OK) {
      ctx_free(&r);
      return st;
    }
    int raw_bits = tile_symbols(lat, codes, m, &raw);
    int kt = orc_rice_kstar(m, raw_bits);
    uint64_t L = orc_rice_len(m, kt, raw_bits);
    k[t] = (uint8_t)kt;
    uint64_t end = off + L;
    if (status == ORC_OK && (end + 31) / 32 <= cap_words) {
      uint64_t wend = (end + 31) / 32;
      for (; zeroed < wend; ++zeroed) words[zeroed] = 0u;
      write_record(words, off, raw_bits, raw, m, kt);
    } else {
      status = ORC_ERR_CAPACITY;
    }
    off = end;
    offsets[t + 1] = off;
  }
  ctx_free(&r);
  return status;
}

int orc_total_bits(int lat, uint64_t seed, float alpha, const void *x, int dtype,
                   uint64_t n_tiles, int dithered, uint64_t tile_base, uint64_t *bits) {
  return orc_total_bits_r(lat, seed, alpha, 0, x, dtype, n_tiles, dithered, tile_base, bits);
}

int orc_total_bits_r(int lat, uint64_t seed, float alpha, int rot, const void *x, int dtype,
                     uint64_t n_tiles, int dithered, uint64_t tile_base, uint64_t *bits) {
  if (lat_dim(lat) == 0 || !(alpha > 0.0f) || !isfinite(alpha)) return ORC_ERR_ARG;
  rot_ctx r;
  if (ctx_init(&r, rot, seed, alpha) != ORC_OK) return ORC_ERR_ARG;
  if (g_threads > 1) {
    int st = total_bits_par(lat, seed, &r, x, dtype, n_tiles, dithered, tile_base, bits);
    ctx_free(&r);
    return st;
  }
  uint64_t total = 0;
  for (uint64_t t = 0; t < n_tiles; ++t) {
    float xt[N];
    int32_t codes[N];
    uint32_t m[N], raw;
    for (int i = 0; i < N; ++i) xt[i] = load_elem(x, dtype, t * N + (uint64_t)i);
    int st = quantize_tile_s(lat, seed, &r, xt, dithered, tile_base + t, codes);
    if (st != ORC_OK) {
      ctx_free(&r);
      return st;
    }
    int raw_bits = tile_symbols(lat, codes, m, &raw);
    total += orc_rice_len(m, orc_rice_kstar(m, raw_bits), raw_bits);
  }
  ctx_free(&r);
  *bits = total;
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Decoder: parse the record, invert strip and zigzag, dequantise, inverse   */
/* RHT (H is symmetric with H H = nI, so the inverse is the same butterfly   */
/* followed by c_dec and D).                                                  */
/* A record is corrupt when k > 22, when it is longer than the longest valid */
/* record, when its unary section holds fewer than 128 ones before the end,  */
/* when the 128th one is not its last bit, or when a symbol reaches 2^22.    */
/* ------------------------------------------------------------------------ */
int orc_parse_tile(int lat, const uint32_t *words, uint64_t off, uint64_t end, int k,
                   int32_t codes[128]) {
  int dim = lat_dim(lat);
  if (dim == 0) return ORC_ERR_ARG;
  int raw_bits = lat == ORC_E8 ? 16 : 0;
  if (k < 0 || k > KMAX) return ORC_ERR_CORRUPT;
  if (end < off) return ORC_ERR_CORRUPT;
  uint64_t L = end - off;
  if (L > (uint64_t)raw_bits + (uint64_t)N * (KMAX + 1)) return ORC_ERR_CORRUPT;
  if (L < (uint64_t)raw_bits + (uint64_t)N * (uint64_t)(k + 1)) return ORC_ERR_CORRUPT;
  uint64_t p = off;
  uint32_t raw = 0, m[N];
  for (int b = 0; b < raw_bits; ++b, ++p) raw |= (uint32_t)get_bit(words, p) << b;
  for (int i = 0; i < N; ++i) {
    uint32_t r = 0;
    for (int b = 0; b < k; ++b, ++p) r |= (uint32_t)get_bit(words, p) << b;
    m[i] = r;
  }
  for (int i = 0; i < N; ++i) {
    uint64_t q = 0;
    while (p < end && !get_bit(words, p)) { ++q; ++p; }
    if (p >= end) return ORC_ERR_CORRUPT;
    ++p;
    uint64_t mv = (q << k) | m[i];
    if (mv >= M_LIMIT) return ORC_ERR_CORRUPT;
    m[i] = (uint32_t)mv;
  }
  if (p != end) return ORC_ERR_CORRUPT;
  for (int v = 0; v < N / dim; ++v) {
    int32_t sym[8];
    for (int c = 0; c < dim; ++c) sym[c] = orc_unzigzag(m[v * dim + c]);
    orc_unstrip(lat, sym, lat == ORC_E8 ? (int)((raw >> v) & 1u) : 0, &codes[v * dim]);
  }
  return ORC_OK;
}

static void dequant_codes(int lat, uint64_t seed, const int32_t codes[128], int dithered,
                          uint64_t tile_id, float uh[128]) {
  int dim = lat_dim(lat);
  for (int v = 0; v < N / dim; ++v) orc_embed(lat, &codes[v * dim], &uh[v * dim]);
  if (dithered) {
    float d[N];
    orc_dither(lat, seed, tile_id, d);
    for (int i = 0; i < N; ++i) uh[i] = uh[i] - d[i];
  }
}

int orc_dequant_rotated(int lat, uint64_t seed, const uint32_t *words, uint64_t off,
                        uint64_t end, int k, int dithered, uint64_t tile_id, float uh[128]) {
  int32_t codes[N];
  int st = orc_parse_tile(lat, words, off, end, k, codes);
  if (st != ORC_OK) return st;
  dequant_codes(lat, seed, codes, dithered, tile_id, uh);
  return ORC_OK;
}

/* The rotated-domain values of n consecutive tiles (tile t has id tile_base +
 * t), a loop over orc_dequant_rotated; a tile that does not parse is left
 * zero and its status returned (the first such). */
int orc_dequant_rotated_many(int lat, uint64_t seed, const uint32_t *words, const uint64_t *offsets,
                             const uint8_t *k, uint64_t n, int dithered, uint64_t tile_base, float *uh) {
  int status = ORC_OK;
  for (uint64_t t = 0; t < n; ++t) {
    int st = orc_dequant_rotated(lat, seed, words, offsets[t], offsets[t + 1], k[t], dithered, tile_base + t,
                                 &uh[t * N]);
    if (st != ORC_OK) {
      memset(&uh[t * N], 0, sizeof(float) * N);
      if (status == ORC_OK) status = st;
    }
  }
  return status;
}

static uint16_t f32_to_bf16_rne(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu)) return (uint16_t)((b >> 16) | 0x40u);
  uint32_t bias = 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)((b + bias) >> 16);
}

int orc_decode(int lat, uint64_t seed, float alpha, const uint32_t *words,
               const uint64_t *offsets, const uint8_t *k, uint64_t n_tiles,
               int dithered, uint64_t tile_base, void *y, int dtype) {
  return orc_decode_r(lat, seed, alpha, 0, words, offsets, k, n_tiles, dithered, tile_base, y, dtype);
}

int orc_decode_r(int lat, uint64_t seed, float alpha, int rot, const uint32_t *words,
                 const uint64_t *offsets, const uint8_t *k, uint64_t n_tiles,
                 int dithered, uint64_t tile_base, void *y, int dtype) {
  if (lat_dim(lat) == 0 || !(alpha > 0.0f) || !isfinite(alpha)) return ORC_ERR_ARG;
  if (dtype != ORC_F32 && dtype != ORC_BF16) return ORC_ERR_ARG;
  rot_ctx r;
  if (ctx_init(&r, rot, seed, alpha) != ORC_OK) return ORC_ERR_ARG;
  if (g_threads > 1) {
    int st = decode_par(lat, seed, &r, words, offsets, k, n_tiles, dithered, tile_base, y, dtype);
    ctx_free(&r);
    return st;
  }
  int status = ORC_OK;
  for (uint64_t t = 0; t < n_tiles; ++t) {
    int32_t codes[N];
    float v[N];
    int st = orc_parse_tile(lat, words, offsets[t], offsets[t + 1], (int)k[t], codes);
    if (st != ORC_OK) {
      status = st;
      for (int i = 0; i < N; ++i) v[i] = 0.0f;
    } else {
      dequant_codes(lat, seed, codes, dithered, tile_base + t, v);
      ctx_inverse(&r, v);
    }
    for (int i = 0; i < N; ++i) {
      if (dtype == ORC_BF16) ((uint16_t *)y)[t * N + (uint64_t)i] = f32_to_bf16_rne(v[i]);
      else ((float *)y)[t * N + (uint64_t)i] = v[i];
    }
  }
  ctx_free(&r);
  return status;
}

/* ------------------------------------------------------------------------ */
/* The same whole-tensor passes on g_threads host threads (OpenMP), for      */
/* large tensors.  Each tile's steps are those of the serial loops; the      */
/* exclusive scan of the record lengths stays serial; records are written    */
/* in parallel, a bit at a time with an atomic OR (every stream bit has one  */
/* writer and OR commutes, so no word depends on the order of the writes).   */
/* Status: the serial encoder and rate pass stop at the first failing tile,  */
/* so these report the first failing tile's status too; the serial decoder   */
/* keeps the last failing tile's status, and so does decode_par.  Statuses,  */
/* and the outputs of every call that succeeds (and every decode), therefore */
/* equal the serial functions'; a failing encode's outputs are unspecified.  */
/* ------------------------------------------------------------------------ */
static int encode_par(int lat, uint64_t seed, const rot_ctx *r, const void *x, int dtype, uint64_t n_tiles,
                      int dithered, uint64_t tile_base, uint32_t *words, uint64_t cap_words, uint64_t *offsets,
                      uint8_t *k) {
  uint32_t *m = (uint32_t *)malloc(sizeof(uint32_t) * N * (n_tiles ? n_tiles : 1));
  uint32_t *raw = (uint32_t *)malloc(sizeof(uint32_t) * (n_tiles ? n_tiles : 1));
  uint64_t *len = (uint64_t *)malloc(sizeof(uint64_t) * (n_tiles ? n_tiles : 1));
  int *tst = (int *)malloc(sizeof(int) * (n_tiles ? n_tiles : 1));
  if (!m || !raw || !len || !tst) {
    free(m); free(raw); free(len); free(tst);
    return ORC_ERR_ARG;
  }
  const int raw_bits = lat == ORC_E8 ? 16 : 0;
#pragma omp parallel for num_threads(g_threads) schedule(static)
  for (int64_t ti = 0; ti < (int64_t)n_tiles; ++ti) {
    const uint64_t t = (uint64_t)ti;
    float xt[N];
    int32_t codes[N];
    for (int i = 0; i < N; ++i) xt[i] = load_elem(x, dtype, t * N + (uint64_t)i);
    tst[t] = quantize_tile_s(lat, seed, r, xt, dithered, tile_base + t, codes);
    if (tst[t] != ORC_OK) continue;
    tile_symbols(lat, codes, &m[t * N], &raw[t]);
    const int kt = orc_rice_kstar(&m[t * N], raw_bits);
    k[t] = (uint8_t)kt;
    len[t] = orc_rice_len(&m[t * N], kt, raw_bits);
  }
  int status = ORC_OK;
  for (uint64_t t = 0; t < n_tiles; ++t)
    if (tst[t] != ORC_OK) { status = tst[t]; break; }
  if (status == ORC_OK) {
    offsets[0] = 0;
    uint64_t n_fit = 0; /* records written: those whose last word fits, a prefix of the tiles */
    for (uint64_t t = 0; t < n_tiles; ++t) {
      offsets[t + 1] = offsets[t] + len[t];
      if ((offsets[t + 1] + 31) / 32 <= cap_words && n_fit == t) n_fit = t + 1;
    }
    if (n_fit < n_tiles) status = ORC_ERR_CAPACITY;
    const uint64_t wend = (offsets[n_fit] + 31) / 32;
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int64_t w = 0; w < (int64_t)wend; ++w) words[w] = 0u;
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int64_t ti = 0; ti < (int64_t)n_fit; ++ti) {
      const uint64_t t = (uint64_t)ti;
      write_record_with(put_bit_atomic, words, offsets[t], raw_bits, raw[t], &m[t * N], (int)k[t]);
    }
  }
  free(m); free(raw); free(len); free(tst);
  return status;
}

static int total_bits_par(int lat, uint64_t seed, const rot_ctx *r, const void *x, int dtype, uint64_t n_tiles,
                          int dithered, uint64_t tile_base, uint64_t *bits) {
  int *tst = (int *)malloc(sizeof(int) * (n_tiles ? n_tiles : 1));
  if (!tst) return ORC_ERR_ARG;
  const int raw_bits = lat == ORC_E8 ? 16 : 0;
  uint64_t total = 0;
#pragma omp parallel for num_threads(g_threads) schedule(static) reduction(+ : total)
  for (int64_t ti = 0; ti < (int64_t)n_tiles; ++ti) {
    const uint64_t t = (uint64_t)ti;
    float xt[N];
    int32_t codes[N];
    uint32_t m[N], raw;
    for (int i = 0; i < N; ++i) xt[i] = load_elem(x, dtype, t * N + (uint64_t)i);
    tst[t] = quantize_tile_s(lat, seed, r, xt, dithered, tile_base + t, codes);
    if (tst[t] != ORC_OK) continue;
    tile_symbols(lat, codes, m, &raw);
    total += orc_rice_len(m, orc_rice_kstar(m, raw_bits), raw_bits);
  }
  int status = ORC_OK;
  for (uint64_t t = 0; t < n_tiles; ++t)
    if (tst[t] != ORC_OK) { status = tst[t]; break; }
  free(tst);
  if (status == ORC_OK) *bits = total;
  return status;
}

static int decode_par(int lat, uint64_t seed, const rot_ctx *r, const uint32_t *words, const uint64_t *offsets,
                      const uint8_t *k, uint64_t n_tiles, int dithered, uint64_t tile_base, void *y, int dtype) {
  int *tst = (int *)malloc(sizeof(int) * (n_tiles ? n_tiles : 1));
  if (!tst) return ORC_ERR_ARG;
#pragma omp parallel for num_threads(g_threads) schedule(static)
  for (int64_t ti = 0; ti < (int64_t)n_tiles; ++ti) {
    const uint64_t t = (uint64_t)ti;
    int32_t codes[N];
    float v[N];
    tst[t] = orc_parse_tile(lat, words, offsets[t], offsets[t + 1], (int)k[t], codes);
    if (tst[t] != ORC_OK) {
      for (int i = 0; i < N; ++i) v[i] = 0.0f;
    } else {
      dequant_codes(lat, seed, codes, dithered, tile_base + t, v);
      ctx_inverse(r, v);
    }
    for (int i = 0; i < N; ++i) {
      if (dtype == ORC_BF16) ((uint16_t *)y)[t * N + (uint64_t)i] = f32_to_bf16_rne(v[i]);
      else ((float *)y)[t * N + (uint64_t)i] = v[i];
    }
  }
  int status = ORC_OK;
  for (uint64_t t = 0; t < n_tiles; ++t)
    if (tst[t] != ORC_OK) status = tst[t];
  free(tst);
  return status;
}

/* ------------------------------------------------------------------------ */
/* Attention scores against compressed keys, in fp64:                        */
/* q . k_hat = q . (D H u_hat c_dec) = c_dec <H D q, u_hat>  (H symmetric).  */
/* ------------------------------------------------------------------------ */
static void fwht128_f64(double v[128]) {
  for (int h = 1; h < N; h <<= 1)
    for (int i = 0; i < N; ++i) {
      if (i & h) continue;
      double a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
}

int orc_kv_scores(int lat, uint64_t seed, float alpha, const uint32_t *words,
                  const uint64_t *offsets, const uint8_t *k, uint32_t n_heads,
                  uint64_t tiles_per_head, uint64_t tile_base, const float *q,
                  uint32_t qph, double *scores) {
  return orc_kv_scores_r(lat, seed, alpha, 0, words, offsets, k, n_heads, tiles_per_head, tile_base, q, qph,
                         scores);
}

/* With the Haar rotation (rot = 1): q . k_hat = q . (alpha Q^T u_hat) =
 * alpha <Q q, u_hat>, in fp64. */
int orc_kv_scores_r(int lat, uint64_t seed, float alpha, int rot, const uint32_t *words,
                    const uint64_t *offsets, const uint8_t *k, uint32_t n_heads,
                    uint64_t tiles_per_head, uint64_t tile_base, const float *q,
                    uint32_t qph, double *scores) {
  if (lat_dim(lat) == 0 || !(alpha > 0.0f) || qph == 0) return ORC_ERR_ARG;
  rot_ctx rc;
  if (ctx_init(&rc, rot, seed, alpha) != ORC_OK) return ORC_ERR_ARG;
  const float c_dec = rc.c_dec;
  uint32_t nq = n_heads * qph;
  double *qt = (double *)malloc(sizeof(double) * (size_t)nq * N);
  if (!qt) {
    ctx_free(&rc);
    return ORC_ERR_ARG;
  }
  for (uint32_t r = 0; r < nq; ++r) {
    const float *qr = &q[(size_t)r * N];
    if (rot == 0) {
      for (int i = 0; i < N; ++i) qt[(size_t)r * N + i] = (double)rc.s[i] * (double)qr[i];
      fwht128_f64(&qt[(size_t)r * N]);
    } else {
      for (int i = 0; i < N; ++i) {
        double acc = 0.0;
        for (int j = 0; j < N; ++j) acc += (double)rc.q[i * N + j] * (double)qr[j];
        qt[(size_t)r * N + i] = acc;
      }
    }
  }
  int status = ORC_OK;
  for (uint32_t h = 0; h < n_heads; ++h) {
    for (uint64_t j = 0; j < tiles_per_head; ++j) {
      uint64_t t = (uint64_t)h * tiles_per_head + j;
      int32_t codes[N];
      double uh[N];
      int st = orc_parse_tile(lat, words, offsets[t], offsets[t + 1], (int)k[t], codes);
      if (st != ORC_OK) {
        status = st;
        for (int i = 0; i < N; ++i) uh[i] = 0.0;
      } else {
        int dim = lat_dim(lat);
        float p[N], d[N];
        for (int v = 0; v < N / dim; ++v) orc_embed(lat, &codes[v * dim], &p[v * dim]);
        orc_dither(lat, seed, tile_base + t, d); /* keys are always dithered */
        for (int i = 0; i < N; ++i) uh[i] = (double)p[i] - (double)d[i];
      }
      for (uint32_t g = 0; g < qph; ++g) {
        const double *qr = &qt[((size_t)h * qph + g) * N];
        double acc = 0.0;
        for (int i = 0; i < N; ++i) acc += qr[i] * uh[i];
        scores[((size_t)h * qph + g) * tiles_per_head + j] = (double)c_dec * acc;
      }
    }
  }
  ctx_free(&rc);
  free(qt);
  return status;
}

/* ------------------------------------------------------------------------ */
/* Attention over compressed keys and values, in fp64, by the plain          */
/* definition: for each query q_{h,g} (qph queries per KV head h),           */
/*   s_t = scale * q . k_hat_t,  p = softmax(s) over the seq keys of head h, */
/*   out = sum_t p_t v_hat_t,                                                */
/* with k_hat and v_hat the decoder's reconstructions D (c_dec H u_hat) of   */
/* the dithered KV streams [HQ-explainer, Methodology 1 and 4] taken in real */
/* arithmetic (fp64, no fp32 rounding of the reconstructions).  Keys of head */
/* h are tiles h*seq + s of the K stream (tile ids k_tile_base + that), the  */
/* values likewise in the V stream; the two plans share lattice and seed and */
/* have their own alpha.  The softmax subtracts the maximum score.  Corrupt  */
/* records count as zero vectors and set the status.                         */
/* ------------------------------------------------------------------------ */
static void recon_f64(int lat, uint64_t seed, const rot_ctx *rc, float c_dec, const uint32_t *words,
                      const uint64_t *offsets, const uint8_t *k, uint64_t t, uint64_t tile_id, double w[128],
                      int *status) {
  int32_t codes[N];
  int st = orc_parse_tile(lat, words, offsets[t], offsets[t + 1], (int)k[t], codes);
  if (st != ORC_OK) {
    *status = st;
    for (int i = 0; i < N; ++i) w[i] = 0.0;
    return;
  }
  float uh[N];
  dequant_codes(lat, seed, codes, 1, tile_id, uh);
  if (!rc->haar) {
    for (int i = 0; i < N; ++i) w[i] = (double)uh[i];
    fwht128_f64(w);
    for (int i = 0; i < N; ++i) w[i] = (double)rc->s[i] * ((double)c_dec * w[i]);
  } else { /* alpha Q^T u_hat */
    for (int i = 0; i < N; ++i) {
      double acc = 0.0;
      for (int j = 0; j < N; ++j) acc += (double)rc->q[j * N + i] * (double)uh[j];
      w[i] = (double)c_dec * acc;
    }
  }
}

int orc_kv_attention(int lat, uint64_t seed, float alpha_k, const uint32_t *kw, const uint64_t *ko,
                     const uint8_t *kk, uint64_t k_tile_base, float alpha_v, const uint32_t *vw,
                     const uint64_t *vo, const uint8_t *vk, uint64_t v_tile_base, uint32_t n_heads,
                     uint64_t seq, const float *q, uint32_t qph, float scale, double *out) {
  return orc_kv_attention_r(lat, seed, 0, alpha_k, kw, ko, kk, k_tile_base, alpha_v, vw, vo, vk, v_tile_base,
                            n_heads, seq, q, qph, scale, out);
}

int orc_kv_attention_r(int lat, uint64_t seed, int rot, float alpha_k, const uint32_t *kw, const uint64_t *ko,
                       const uint8_t *kk, uint64_t k_tile_base, float alpha_v, const uint32_t *vw,
                       const uint64_t *vo, const uint8_t *vk, uint64_t v_tile_base, uint32_t n_heads,
                       uint64_t seq, const float *q, uint32_t qph, float scale, double *out) {
  if (lat_dim(lat) == 0 || !(alpha_k > 0.0f) || !(alpha_v > 0.0f) || qph == 0 || seq == 0) return ORC_ERR_ARG;
  rot_ctx rk, rv;
  if (ctx_init(&rk, rot, seed, alpha_k) != ORC_OK) return ORC_ERR_ARG;
  if (ctx_init(&rv, rot, seed, alpha_v) != ORC_OK) {
    ctx_free(&rk);
    return ORC_ERR_ARG;
  }
  const float ck = rk.c_dec, cv = rv.c_dec;
  double *sc = (double *)malloc(sizeof(double) * (size_t)seq * qph);
  if (!sc) {
    ctx_free(&rk);
    ctx_free(&rv);
    return ORC_ERR_ARG;
  }
  int status = ORC_OK;
  for (uint32_t h = 0; h < n_heads; ++h) {
    for (uint64_t j = 0; j < seq; ++j) {
      const uint64_t t = (uint64_t)h * seq + j;
      double kh[N];
      recon_f64(lat, seed, &rk, ck, kw, ko, kk, t, k_tile_base + t, kh, &status);
      for (uint32_t g = 0; g < qph; ++g) {
        const float *qr = &q[((size_t)h * qph + g) * N];
        double acc = 0.0;
        for (int i = 0; i < N; ++i) acc += (double)qr[i] * kh[i];
        sc[(size_t)g * seq + j] = (double)scale * acc;
      }
    }
    for (uint32_t g = 0; g < qph; ++g) {
      double *o = &out[((size_t)h * qph + g) * N];
      const double *sg = &sc[(size_t)g * seq];
      double m = sg[0];
      for (uint64_t j = 1; j < seq; ++j) m = sg[j] > m ? sg[j] : m;
      double l = 0.0;
      for (int i = 0; i < N; ++i) o[i] = 0.0;
      for (uint64_t j = 0; j < seq; ++j) {
        const double pj = exp(sg[j] - m);
        l += pj;
        double vh[N];
        recon_f64(lat, seed, &rv, cv, vw, vo, vk, (uint64_t)h * seq + j, v_tile_base + (uint64_t)h * seq + j, vh,
                  &status);
        for (int i = 0; i < N; ++i) o[i] += pj * vh[i];
      }
      for (int i = 0; i < N; ++i) o[i] /= l;
    }
  }
  ctx_free(&rk);
  ctx_free(&rv);
  free(sc);
  return status;
}

/* ------------------------------------------------------------------------ */
/* Matrix-vector products with a compressed weight matrix, in fp64, by the    */
/* plain definition y = W_hat x.  The weights are rows x cols with tiles of   */
/* 128 along each row (tile t = r * (cols / 128) + b holds row r, columns     */
/* 128 b .. 128 b + 127), as encoded by orc_encode without dither.  W_hat of  */
/* a tile is the decoder's reconstruction D (c_dec H u_hat) [HQ-explainer,    */
/* Methodology 1: the inverse of the orthonormal RHT] taken in real           */
/* arithmetic: H u_hat and the products are fp64 (exact for the integer       */
/* codes of Z, D4 and E8), with no fp32 rounding of the weights.  x holds nb  */
/* fp32 vectors [nb][cols]; y[j][r] = sum_c W_hat[r][c] x[j][c].  A tile that */
/* does not parse counts as zeros and sets the status.                        */
/* ------------------------------------------------------------------------ */
int orc_gemv(int lat, uint64_t seed, float alpha, const uint32_t *words, const uint64_t *offsets,
             const uint8_t *k, uint64_t rows, uint64_t cols, const float *x, uint32_t nb, double *y) {
  if (lat_dim(lat) == 0 || !(alpha > 0.0f) || nb == 0 || cols == 0 || cols % N) return ORC_ERR_ARG;
  float s[N], c_enc, c_dec;
  orc_signs(seed, s);
  orc_scales(alpha, &c_enc, &c_dec);
  const uint64_t nblk = cols / N;
  for (uint64_t i = 0; i < (uint64_t)nb * rows; ++i) y[i] = 0.0;
  int status = ORC_OK;
  /* rows are independent: with g_threads > 1 they are shared out among host
   * threads; each row's sums are formed in the same order either way (the only
   * error a tile can give is ORC_ERR_CORRUPT, so the status is the same too) */
#pragma omp parallel for num_threads(g_threads) schedule(dynamic, 8) if (g_threads > 1)
  for (int64_t ri = 0; ri < (int64_t)rows; ++ri) {
    const uint64_t r = (uint64_t)ri;
    for (uint64_t b = 0; b < nblk; ++b) {
      const uint64_t t = r * nblk + b;
      int32_t codes[N];
      int st = orc_parse_tile(lat, words, offsets[t], offsets[t + 1], (int)k[t], codes);
      if (st != ORC_OK) {
#pragma omp atomic write
        status = st;
        continue;
      }
      float uh[N];
      dequant_codes(lat, seed, codes, 0, t, uh);
      double w[N];
      for (int i = 0; i < N; ++i) w[i] = (double)uh[i];
      fwht128_f64(w);
      for (int i = 0; i < N; ++i) w[i] = (double)s[i] * ((double)c_dec * w[i]);
      for (uint32_t j = 0; j < nb; ++j) {
        const float *xj = &x[(size_t)j * cols + b * N];
        double acc = 0.0;
        for (int i = 0; i < N; ++i) acc += w[i] * (double)xj[i];
        y[(size_t)j * rows + r] += acc;
      }
    }
  }
  return status;
}

/* ------------------------------------------------------------------------ */
/* Rate calibration [HQ-explainer, Methodology 3: achieved rate within about */
/* 0.01 bps of the target].  Mechanism (reading): start from the             */
/* high-resolution estimate alpha0 = sqrt(2 pi e) sigma / (nu 2^R), with     */
/* sigma the RMS of the tensor and nu the per-dimension cell edge of the     */
/* embedding (Z 1, A2 sqrt(2 sqrt3), D4 2^(1/4), 2E8 2); bracket the target  */
/* in log2(alpha) from exact integers that contain log2 alpha0 (the binary   */
/* exponent of max |x|, ceil(log2 N) and floor(bps): see below), widen it by */
/* 4 while it does not hold the target, then bisect on the exact payload rate */
/* until it is within 0.002 bps, at most 40 times.  The fp32 alpha with the  */
/* closest rate wins; ties go to the larger alpha.                           */
/* ------------------------------------------------------------------------ */
static double rate_at(int lat, uint64_t seed, float a, int rot, const void *x, int dtype,
                      uint64_t n_tiles, int dithered, uint64_t tile_base, int *st) {
  uint64_t bits = 0;
  *st = orc_total_bits_r(lat, seed, a, rot, x, dtype, n_tiles, dithered, tile_base, &bits);
  if (*st == ORC_ERR_RANGE) return INFINITY; /* step too fine: treat as too many bits */
  return (double)bits / ((double)n_tiles * (double)N);
}

int orc_calibrate(int lat, uint64_t seed, float bps, const void *x, int dtype,
                  uint64_t n_tiles, int dithered, uint64_t tile_base,
                  float *alpha_out, double *bps_out, int *iters_out) {
  return orc_calibrate_r(lat, seed, bps, 0, x, dtype, n_tiles, dithered, tile_base, alpha_out, bps_out,
                         iters_out);
}

int orc_calibrate_r(int lat, uint64_t seed, float bps, int rot, const void *x, int dtype,
                    uint64_t n_tiles, int dithered, uint64_t tile_base,
                    float *alpha_out, double *bps_out, int *iters_out) {
  if (lat_dim(lat) == 0 || n_tiles == 0 || !(bps > 0.0f)) return ORC_ERR_ARG;
  /* The bracket starts from exact integers only -- the binary exponent of
   * max |x|, ceil(log2 N) and floor(bps) -- so that any implementation that
   * evaluates the rate exactly takes the same bisection path (a start from
   * the RMS would depend on how its sum of squares was rounded).  With
   * sigma = RMS(x) in [max/sqrt N, max] and the high-resolution estimate
   * alpha ~ sqrt(2 pi e) sigma / (nu 2^R), nu in [1, 2], the estimate lies in
   * [2^(eA - R - eN/2 + 1.05), 2^(eA - R + 3.05)]: the bracket below holds
   * it with 4 octaves to spare at the bottom and about one at the top, and
   * widens by 4 octaves at a time while it does not hold the target. */
  float amax = 0.0f;
  uint64_t n = n_tiles * (uint64_t)N;
  for (uint64_t i = 0; i < n; ++i) {
    float v = fabsf(load_elem(x, dtype, i));
    if (!isfinite(v)) return ORC_ERR_NONFINITE;
    if (v > amax) amax = v;
  }
  if (!(amax > 0.0f)) return ORC_ERR_ARG;
  int eA1;
  frexp((double)amax, &eA1); /* amax = f 2^eA1, f in [0.5, 1): floor(log2 amax) = eA1 - 1 */
  int eN = 0;                /* ceil(log2 n) */
  while ((1ull << eN) < n) ++eN;
  const double eA = (double)(eA1 - 1), Rf = floor((double)bps);
  double target = (double)bps;
  double lo = eA - Rf - 4.0 - (double)((eN + 1) / 2), hi = eA - Rf + 4.0;
  int st, iters = 0;
  float best_a = 0.0f;
  double best_r = 0.0, best_err = INFINITY;
#define CONSIDER(A, R)                                                        \
  do {                                                                        \
    double e_ = fabs((R) - target);                                           \
    if (e_ < best_err || (e_ == best_err && (A) > best_a)) {                  \
      best_err = e_; best_a = (A); best_r = (R);                              \
    }                                                                         \
  } while (0)
  for (int g = 0; g < 16; ++g) { /* lo must give a rate >= target */
    float a = (float)exp2(lo);
    double r = rate_at(lat, seed, a, rot, x, dtype, n_tiles, dithered, tile_base, &st);
    ++iters;
    if (st != ORC_OK && st != ORC_ERR_RANGE) return st;
    if (st == ORC_OK) CONSIDER(a, r);
    if (r >= target) break;
    lo -= 4.0;
  }
  for (int g = 0; g < 16; ++g) { /* hi must give a rate <= target */
    float a = (float)exp2(hi);
    double r = rate_at(lat, seed, a, rot, x, dtype, n_tiles, dithered, tile_base, &st);
    ++iters;
    if (st != ORC_OK && st != ORC_ERR_RANGE) return st;
    if (st == ORC_OK) CONSIDER(a, r);
    if (r <= target) break;
    hi += 4.0;
  }
  for (int it = 0; it < 40 && best_err > 0.002; ++it) {
    double mid = 0.5 * (lo + hi);
    float a = (float)exp2(mid);
    double r = rate_at(lat, seed, a, rot, x, dtype, n_tiles, dithered, tile_base, &st);
    ++iters;
    if (st != ORC_OK && st != ORC_ERR_RANGE) return st;
    if (st == ORC_OK) CONSIDER(a, r);
    if (r > target) lo = mid;
    else hi = mid;
  }
#undef CONSIDER
  if (!(best_a > 0.0f)) return ORC_ERR_RANGE;
  *alpha_out = best_a;
  *bps_out = best_r;
  if (iters_out) *iters_out = iters;
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Serialized form of a stream.  The pages define none: the stream, its      */
/* offsets and Rice parameters and the plan are the whole state [HQ-explainer,*/
/* Methodology 3: the side information of each tile is its offset and k].    */
/* These write the library's container layout from its specification: the   */
/* 64-byte header and the compact side information (96 bytes per 32 tiles). */
/* ------------------------------------------------------------------------ */

/* CRC-32 of IEEE 802.3, bit by bit: reflected polynomial 0xEDB88320,
 * register preset to all ones, final complement. */
uint32_t orc_crc32(const uint8_t *p, size_t n) {
  uint32_t c = 0xFFFFFFFFu;
  for (size_t i = 0; i < n; ++i) {
    c ^= p[i];
    for (int b = 0; b < 8; ++b) c = (c >> 1) ^ (0xEDB88320u & (0u - (c & 1u)));
  }
  return ~c;
}

static void le_store(uint8_t *p, uint64_t v, int n) {
  for (int i = 0; i < n; ++i) p[i] = (uint8_t)((v >> (8 * i)) & 0xFFu);
}

/* magic "HQS1", version 1, lattice, flags (1 dithered, 2 compact side),
 * tile 128, alpha and bps as fp32 bits, seed, tile base, tile count, total
 * bits, CRC-32 of bytes 0..59 at 60; reserved fields zero. */
void orc_header_write_r(int lat, uint64_t seed, float alpha, float bps, int dithered, int compact, int rot,
                        uint64_t tile_base, uint64_t n_tiles, uint64_t total_bits, uint8_t out[64]);

void orc_header_write(int lat, uint64_t seed, float alpha, float bps, int dithered, int compact, uint64_t tile_base,
                      uint64_t n_tiles, uint64_t total_bits, uint8_t out[64]) {
  orc_header_write_r(lat, seed, alpha, bps, dithered, compact, 0, tile_base, n_tiles, total_bits, out);
}

/* flags bit 2: the Haar rotation */
void orc_header_write_r(int lat, uint64_t seed, float alpha, float bps, int dithered, int compact, int rot,
                        uint64_t tile_base, uint64_t n_tiles, uint64_t total_bits, uint8_t out[64]) {
  uint32_t ab, bb;
  memset(out, 0, 64);
  memcpy(&ab, &alpha, 4);
  memcpy(&bb, &bps, 4);
  out[0] = 'H'; out[1] = 'Q'; out[2] = 'S'; out[3] = '1';
  le_store(out + 4, 1, 2);
  out[6] = (uint8_t)lat;
  out[7] = (uint8_t)((dithered ? 1 : 0) + (compact ? 2 : 0) + (rot ? 4 : 0));
  le_store(out + 8, 128, 4);
  le_store(out + 12, ab, 4);
  le_store(out + 16, bb, 4);
  le_store(out + 24, seed, 8);
  le_store(out + 32, tile_base, 8);
  le_store(out + 40, n_tiles, 8);
  le_store(out + 48, total_bits, 8);
  le_store(out + 60, orc_crc32(out, 60), 4);
}

/* Per chunk of 32 tiles: the chunk's first offset (8 bytes), each tile's end
 * offset minus it (2 bytes each), the 32 Rice parameters as 5-bit fields
 * (bit 5j + b of the 160-bit field is bit b of k of tile j), 4 zero bytes.
 * Entries past the last tile stay zero.  Returns ORC_ERR_CAPACITY when a
 * difference does not fit 16 bits. */
int orc_side_pack(const uint64_t *offsets, const uint8_t *k, uint64_t n, uint8_t *out) {
  const uint64_t chunks = (n + 31) / 32;
  int status = ORC_OK;
  memset(out, 0, (size_t)(96 * chunks));
  for (uint64_t c = 0; c < chunks; ++c) {
    uint8_t *rec = out + 96 * c;
    const uint64_t base = offsets[32 * c];
    le_store(rec, base, 8);
    for (uint64_t j = 0; j < 32 && 32 * c + j < n; ++j) {
      const uint64_t t = 32 * c + j;
      const uint64_t d = offsets[t + 1] - base;
      if (d > 65535u) status = ORC_ERR_CAPACITY;
      le_store(rec + 8 + 2 * j, d & 0xFFFFu, 2);
      for (int b = 0; b < 5; ++b) {
        const uint64_t bit = 5 * j + (uint64_t)b;
        if ((k[t] >> b) & 1u) rec[72 + bit / 8] |= (uint8_t)(1u << (bit % 8));
      }
    }
  }
  return status;
}
