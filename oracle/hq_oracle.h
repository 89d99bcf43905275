/*
 * hq_oracle.h -- plain, slow CPU reference of the HyperQuant per-tile codec.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the CPU-baseline leg of the benchmark may load or call this library.  The
 * product path (libhq, the HIP kernels and their Python binding) never does;
 * it shares no code, header, table or constant with this file.
 *
 * Sources cited in this directory:
 *   [HQ-explainer] "HyperQuant: A Rate-Distortion-Optimal Quantization
 *       Pipeline for Large Language and Diffusion Models", gist.science
 *       explainer pages (zh/nl/pt), technical summary; sections are named
 *       Methodology 1 (per-tile RHT), 2 (lattice quantization),
 *       3 (bit-stripping and Rice coding), 4 (KV-cache bias correction).
 *   [HQ-abstract] the paper's abstract page (layerthelatestinalattice.com),
 *       items (i)-(iv).
 *   [Philox] Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
 *       1, 2, 3", SC'11 -- the Philox4x32-10 generator.
 *   [SPLAG] Conway & Sloane, "Sphere Packings, Lattices and Groups", ch. 20
 *       (fast decoders for Z^n, D_n, E8 and A2).
 *
 * Parity status: every function below is pinned by a "not gpu" test (closed
 * form, brute force, invariant or published known-answer vector) except the
 * bit layout of the stream (symbol order, zigzag, field order, word order,
 * counter layout), which the pages leave open.  That layout is "parity
 * unpinned": it is fixed only by the readings stated with each function and
 * by round-trip tests.
 */
#ifndef HQ_ORACLE_H
#define HQ_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_Z = 0, ORC_A2 = 1, ORC_D4 = 2, ORC_E8 = 3 };
enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum {
  ORC_OK = 0, ORC_ERR_ARG = 1, ORC_ERR_NONFINITE = 2, ORC_ERR_RANGE = 3,
  ORC_ERR_CAPACITY = 4, ORC_ERR_CORRUPT = 5, ORC_ERR_DEVICE = 6, ORC_ERR_NOALPHA = 7
};

/* Philox4x32-10 block: out = Philox(ctr, key) [Philox]. */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* The 128 diagonal signs of D (+1/-1) for a plan seed. */
void orc_signs(uint64_t seed, float s[128]);

/* Unnormalised fast Walsh-Hadamard transform of 128 fp32 values in place,
 * natural (Sylvester) order, stages h = 1, 2, ..., 64. */
void orc_fwht128(float v[128]);

/* Forward RHT of one tile: u = c_enc * H (D x), fp32. */
void orc_rht_forward(const float x[128], const float s[128], float c_enc, float u[128]);

/* Nearest point of one lattice vector (dimension 1, 2, 4 or 8) in the integer
 * embedding of the lattice.  u has dim(lat) entries; x receives the codes. */
void orc_nearest(int lat, const float *u, int32_t *x);

void orc_nearest_many(int lat, uint64_t n_vectors, const float *u, int32_t *x);

/* Real-space coordinates of a code vector (A2: (i, j*sqrt3); others: x). */
void orc_embed(int lat, const int32_t *x, float *p);

/* Bit-stripping of one code vector: symbols (dim entries) and the raw coset
 * bit (E8 only; 0 otherwise).  Unstripping inverts it. */
void orc_strip(int lat, const int32_t *x, int32_t *sym, int *raw_bit);
void orc_unstrip(int lat, const int32_t *sym, int raw_bit, int32_t *x);

uint32_t orc_zigzag(int32_t v);
int32_t orc_unzigzag(uint32_t m);

/* Rice length of a tile for parameter k, and the smallest minimising k. */
uint64_t orc_rice_len(const uint32_t m[128], int k, int raw_bits);
int orc_rice_kstar(const uint32_t m[128], int raw_bits);

/* Subtractive dither of one tile: 128 values, uniform over the Voronoi cell of
 * the lattice (integer-embedding scale), from (seed, tile id). */
void orc_dither(int lat, uint64_t seed, uint64_t tile_id, float d[128]);

/* Scale constants of a plan: c_enc = fp32(1/(alpha*sqrt(128))),
 * c_dec = fp32(alpha/sqrt(128)). */
void orc_scales(float alpha, float *c_enc, float *c_dec);

/* Quantise one tile to lattice codes (128 int32, vector-major) after the RHT
 * and optional dither.  Returns an ORC_ status. */
int orc_quantize_tile(int lat, uint64_t seed, float alpha, const float x[128],
                      int dithered, uint64_t tile_id, int32_t codes[128]);

/* Write one tile's record for given codes at bit off of words (which must be
 * zero there); returns its length in bits and the chosen k. */
uint64_t orc_write_record_codes(int lat, const int32_t codes[128], uint32_t *words,
                                uint64_t off, int *k_out);

/* Encode n_tiles tiles of x (fp32 or bf16 bit patterns, row-major, 128 per
 * tile) into a bitstream.  words: cap_words uint32; offsets: n_tiles+1 uint64
 * bit offsets; k: n_tiles bytes.  Returns an ORC_ status. */
int orc_encode(int lat, uint64_t seed, float alpha, const void *x, int dtype,
               uint64_t n_tiles, int dithered, uint64_t tile_base,
               uint32_t *words, uint64_t cap_words, uint64_t *offsets, uint8_t *k);

/* Total payload bits of an encode (no stores).  Returns an ORC_ status. */
int orc_total_bits(int lat, uint64_t seed, float alpha, const void *x, int dtype,
                   uint64_t n_tiles, int dithered, uint64_t tile_base, uint64_t *bits);

/* Parse one tile's record back into its 128 lattice codes. */
int orc_parse_tile(int lat, const uint32_t *words, uint64_t off, uint64_t end, int k,
                   int32_t codes[128]);

/* Decode n_tiles tiles into y (fp32 or bf16).  Returns an ORC_ status. */
int orc_decode(int lat, uint64_t seed, float alpha, const uint32_t *words,
               const uint64_t *offsets, const uint8_t *k, uint64_t n_tiles,
               int dithered, uint64_t tile_base, void *y, int dtype);

/* Dequantised tile in the rotated domain, fp32: u_hat = embed(codes) - d. */
int orc_dequant_rotated(int lat, uint64_t seed, const uint32_t *words, uint64_t off,
                        uint64_t end, int k, int dithered, uint64_t tile_id, float uh[128]);
int orc_dequant_rotated_many(int lat, uint64_t seed, const uint32_t *words, const uint64_t *offsets,
                             const uint8_t *k, uint64_t n, int dithered, uint64_t tile_base, float *uh);

/* Fused-score reference in fp64: scores[h*qph+g][s] =
 * c_dec * < H D q_{h,g}, u_hat_{h,s} >. */
int orc_kv_scores(int lat, uint64_t seed, float alpha, const uint32_t *words,
                  const uint64_t *offsets, const uint8_t *k, uint32_t n_heads,
                  uint64_t tiles_per_head, uint64_t tile_base, const float *q,
                  uint32_t qph, double *scores);

/* Attention over dithered compressed keys and values, fp64: out[(h*qph+g)*128
 * + i] = sum_t softmax_t(scale * q_{h,g} . k_hat_{h,t}) v_hat_{h,t}[i]. */
int orc_kv_attention(int lat, uint64_t seed, float alpha_k, const uint32_t *kw, const uint64_t *ko,
                     const uint8_t *kk, uint64_t k_tile_base, float alpha_v, const uint32_t *vw,
                     const uint64_t *vo, const uint8_t *vk, uint64_t v_tile_base, uint32_t n_heads,
                     uint64_t seq, const float *q, uint32_t qph, float scale, double *out);

/* Matrix-vector products with a compressed (undithered) weight matrix, fp64:
 * y[j][r] = sum_c W_hat[r][c] x[j][c] with W_hat the reconstruction
 * D (c_dec H u_hat) in real arithmetic; tiles of 128 along the rows. */
int orc_gemv(int lat, uint64_t seed, float alpha, const uint32_t *words, const uint64_t *offsets,
             const uint8_t *k, uint64_t rows, uint64_t cols, const float *x, uint32_t nb, double *y);

/* Rate calibration: bisection on log2(alpha) for the payload rate
 * (bits per scalar).  Returns an ORC_ status. */
/* Host threads of the whole-tensor encode, decode and rate passes (default
 * 1: the plain serial loops).  With n > 1 they run the per-tile steps on n
 * OpenMP threads (the length scan stays serial, record bits are ORed in
 * atomically); statuses and the outputs of successful calls do not depend
 * on n.  Not thread-safe against concurrent codec calls. */
void orc_set_threads(int n);
int orc_get_threads(void);

/* Haar rotation variant (rot = 1; rot = 0 is the RHT): the matrix and the
 * codec calls with a rotation argument. */
void orc_haar(uint64_t seed, float q32[128 * 128]);
int orc_encode_r(int lat, uint64_t seed, float alpha, int rot, const void *x, int dtype,
                 uint64_t n_tiles, int dithered, uint64_t tile_base,
                 uint32_t *words, uint64_t cap_words, uint64_t *offsets, uint8_t *k);
int orc_total_bits_r(int lat, uint64_t seed, float alpha, int rot, const void *x, int dtype,
                     uint64_t n_tiles, int dithered, uint64_t tile_base, uint64_t *bits);
int orc_decode_r(int lat, uint64_t seed, float alpha, int rot, const uint32_t *words,
                 const uint64_t *offsets, const uint8_t *k, uint64_t n_tiles,
                 int dithered, uint64_t tile_base, void *y, int dtype);
int orc_calibrate_r(int lat, uint64_t seed, float bps, int rot, const void *x, int dtype,
                    uint64_t n_tiles, int dithered, uint64_t tile_base,
                    float *alpha_out, double *bps_out, int *iters_out);
int orc_kv_scores_r(int lat, uint64_t seed, float alpha, int rot, const uint32_t *words,
                    const uint64_t *offsets, const uint8_t *k, uint32_t n_heads,
                    uint64_t tiles_per_head, uint64_t tile_base, const float *q,
                    uint32_t qph, double *scores);
int orc_kv_attention_r(int lat, uint64_t seed, int rot, float alpha_k, const uint32_t *kw, const uint64_t *ko,
                       const uint8_t *kk, uint64_t k_tile_base, float alpha_v, const uint32_t *vw,
                       const uint64_t *vo, const uint8_t *vk, uint64_t v_tile_base, uint32_t n_heads,
                       uint64_t seq, const float *q, uint32_t qph, float scale, double *out);
uint32_t orc_crc32(const uint8_t *p, size_t n);
void orc_header_write(int lat, uint64_t seed, float alpha, float bps, int dithered, int compact, uint64_t tile_base,
                      uint64_t n_tiles, uint64_t total_bits, uint8_t out[64]);
void orc_header_write_r(int lat, uint64_t seed, float alpha, float bps, int dithered, int compact, int rot,
                        uint64_t tile_base, uint64_t n_tiles, uint64_t total_bits, uint8_t out[64]);
int orc_side_pack(const uint64_t *offsets, const uint8_t *k, uint64_t n, uint8_t *out);
int orc_calibrate(int lat, uint64_t seed, float bps, const void *x, int dtype,
                  uint64_t n_tiles, int dithered, uint64_t tile_base,
                  float *alpha_out, double *bps_out, int *iters_out);

#ifdef __cplusplus
}
#endif
#endif
