/*
 * hq.h -- C ABI of libhq, the HyperQuant per-tile lattice codec for MI355X
 * (gfx950).
 *
 * The operation is the data-free post-training codec of "HyperQuant: A
 * Rate-Distortion-Optimal Quantization Pipeline for Large Language and
 * Diffusion Models" (gist.science explainer pages, technical summary,
 * Methodology 1-4; the paper's abstract page, items (i)-(iv)):
 *   encode: per 128-wide tile, the randomized Hadamard transform
 *           u = H_n D x / (alpha sqrt n)                       (Methodology 1)
 *           nearest point of u in the integer embedding of E8, D4, A2 or Z
 *                                                               (Methodology 2)
 *           bit-stripping of the membership-fixed bits, Rice coding of the
 *           remaining symbols with one k per tile                (Methodology 3)
 *           for KV: subtractive dither U ~ Uniform(V(lattice)) added before
 *           and subtracted after quantisation                    (Methodology 4)
 *   decode: the inverse of each step.
 *
 * Conventions (all entry points):
 *   - Pointers named x, y, words, offsets, k, q, scores and ws are DEVICE
 *     pointers owned by the caller, 16-byte aligned.  The library never
 *     allocates device memory.  `stream` is a hipStream_t (NULL = null stream).
 *   - Calls are asynchronous on `stream` except hq_calibrate and
 *     hq_status_sync, which synchronise it.
 *   - Argument errors return synchronously (HQ_ERR_ARG, HQ_ERR_NOALPHA).
 *     Data errors found on the device (non-finite input, range, capacity,
 *     corrupt stream) are recorded in the workspace and returned by
 *     hq_status_sync; the outputs of the failing call are then unspecified.
 *     When several data errors occur, the lowest code is reported.
 *   - Workspace: a device buffer of hq_workspace_bytes() bytes (about 12 KB
 *     per 32 tiles: it holds each chunk's staged bits between the launches of
 *     one encode; about 3.5 KB at 4 bits per scalar for a plan with a compact
 *     workspace, hq_plan_set_compact_workspace), 16-byte aligned, zero-filled
 *     by the caller once before its first use.  One workspace must not be used by two calls that can run
 *     concurrently (e.g. on two streams).
 *   - No call waits on another work-group's progress; encode is one launch
 *     for at most 32 tiles (one chunk: its offset is the stream's start, so
 *     the packing launch writes the stream itself), two stream-ordered
 *     launches (pack per chunk, then placement, which sums the bit counts of
 *     the chunks before its own) up to 8192 chunks of 32 tiles, and three
 *     above (the bit counts of blocks of 1024 chunks between them; placement
 *     then adds the totals of the blocks before its own and its own block's
 *     counts), four above 65536 chunks (the block totals turned into prefixes
 *     by a launch of their own).  Encode and decode allocate nothing and can
 *     be captured in a HIP graph.
 *   - Tensors are row-major; every 128 consecutive elements form one tile
 *     (weights: tiles along rows; KV [B, H, S, 128]: one tile per vector).
 *   - Stream layout: record of tile t at bits [offsets[t], offsets[t+1]):
 *     [E8 only: 16 raw coset bits, bit v for lattice vector v]
 *     [128 Rice remainders of k[t] bits, symbol order, LSB first]
 *     [128 unary quotients, q zeros then a one].
 *     Stream bit P is bit P%32 of 32-bit word P/32; records abut; offsets[0]
 *     = 0; the unused bits of the last word are zero; words beyond it are
 *     not written.  The stream is not self-describing: decoding needs the
 *     same plan (lattice, seed, alpha).
 */
#ifndef HQ_H
#define HQ_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* (The last enumerator of each enum only gives the type the range of a 32-bit
 * int, so that an out-of-range value a caller passes is a checked argument
 * error, not undefined behaviour in the library.) */
typedef enum { HQ_Z = 0, HQ_A2 = 1, HQ_D4 = 2, HQ_E8 = 3, HQ_LATTICE_INT_RANGE_ = 0x7FFFFFFF } hq_lattice;
typedef enum { HQ_F32 = 0, HQ_BF16 = 1, HQ_DTYPE_INT_RANGE_ = 0x7FFFFFFF } hq_dtype;
typedef enum {
  HQ_OK = 0,
  HQ_ERR_ARG = 1,        /* bad argument (null pointer, tile != 128, size) */
  HQ_ERR_NONFINITE = 2,  /* NaN or Inf in the input */
  HQ_ERR_RANGE = 3,      /* a scaled coordinate reached 2^20: alpha too small */
  HQ_ERR_CAPACITY = 4,   /* the stream does not fit cap_words */
  HQ_ERR_CORRUPT = 5,    /* a record does not parse (decode) */
  HQ_ERR_DEVICE = 6,     /* a HIP runtime call failed */
  HQ_ERR_NOALPHA = 7,    /* the plan has no alpha yet */
  HQ_STATUS_INT_RANGE_ = 0x7FFFFFFF
} hq_status;

typedef struct hq_plan_s* hq_plan_t;

/* Create a plan [Methodology 1-2]: lattice, tile length (must be 128), target
 * rate in bits per scalar (used by hq_calibrate), seed of the random signs of
 * D and of the dither stream.  alpha is unset until hq_plan_set_alpha or
 * hq_calibrate.  The plan is host memory owned by the library. */
hq_status hq_plan(hq_lattice lattice, int tile, float bps, uint64_t seed, hq_plan_t* out);

/* The rotation of Methodology 1 [and the Haar-uniform "QJL" rotation the
 * explainer compares it with for the KV cache]: kind 0 = the RHT H D (the
 * default), kind 1 = a Haar-distributed random orthogonal Q made from the
 * plan's seed (Gram-Schmidt of Philox/Box-Muller normals in double, rounded to
 * fp32).  With Q: u = fl32(t c_enc), t_i the fp32 fma chain over j of
 * Q[i][j] x_j in index order, c_enc = fp32(1/alpha); decode x = fl32(t'
 * alpha), t' the chain of Q[j][i] u_j.  Kind 1 needs dev_buf: hq_rotation_bytes()
 * bytes of caller-owned device memory, 16-byte aligned, kept for the plan's
 * life (the call uploads Q^T and Q and synchronises stream).  Encode, decode,
 * their KV and append variants, calibration, hq_kv_scores and hq_kv_attention
 * follow the plan (the two fused KV paths rotate the queries with Q, and the
 * attention rotates its result back with Q^T, by the same fp32 chains);
 * hq_gemv and hq_gemm (which fold the RHT into the vectors) return
 * HQ_ERR_ARG for a Haar plan.  The workspace of a Haar plan is larger
 * (hq_workspace_bytes counts 512 bytes per tile more).
 * hq_plan_get_rotation: the kind, and if q is not NULL the Haar matrix of the
 * plan's seed (128 x 128 fp32, row-major, host memory; computed on the host,
 * whatever the current kind). */
size_t hq_rotation_bytes(void);
hq_status hq_plan_set_rotation(hq_plan_t plan, int kind, void* dev_buf, void* stream);
hq_status hq_plan_get_rotation(hq_plan_t plan, int* kind, float* q);

/* Fix the lattice scale alpha (> 0, finite) [Methodology 2]. */
hq_status hq_plan_set_alpha(hq_plan_t plan, float alpha);

/* Read back alpha and the fp32 scale constants c_enc = 1/(alpha sqrt 128),
 * c_dec = alpha/sqrt 128 (any output pointer may be NULL). */
hq_status hq_plan_get(hq_plan_t plan, float* alpha, float* c_enc, float* c_dec);

void hq_plan_destroy(hq_plan_t plan);

/* Workspace bytes for calls on up to n_tiles tiles. */
size_t hq_workspace_bytes(hq_plan_t plan, uint64_t n_tiles);

/* Staging slots of the plan's encodes (hq_workspace_bytes follows the mode:
 * set it before sizing a workspace; 0 or 1, else HQ_ERR_ARG).  0, the
 * default: each chunk of 32 tiles is staged in a slot that holds its longest
 * possible record bits, 11.9 KB per chunk (1.45x the bytes of its bf16
 * input).  1, compact: slots of 128 (bps + 2.5) + 8 words in whole uint4,
 * bps being the plan's rate (the workspace then takes 3.5 KB per chunk at
 * 4 bps, 0.43x the bf16 input); a chunk whose bits do not fit its slot is encoded again by the
 * placement launch, from its input, straight into the stream, so the result
 * is the same whatever the data.  The placement of a compact plan carries
 * that path and runs about 10 % slower on the measured weights. */
hq_status hq_plan_set_compact_workspace(hq_plan_t plan, int on);

/* Words that always suffice for the stream of n_tiles tiles (the longest
 * record is 16 + 128*23 bits for E8, 128*23 otherwise). */
uint64_t hq_encode_bound_words(hq_plan_t plan, uint64_t n_tiles);

/* Rate calibration [Methodology 3: the achieved rate lands within about 0.01
 * bps of the target]: bisection on log2(alpha) for the payload rate of x,
 * stopping within 0.002 bps (at most 40 steps after bracketing).  Sets the
 * plan's alpha.  dithered/tile_base select the KV dither stream.  Synchronous. */
hq_status hq_calibrate(hq_plan_t plan, const void* x, hq_dtype dtype, uint64_t n_tiles,
                       int dithered, uint64_t tile_base, void* ws, void* stream,
                       float* alpha_out, double* bps_out);

/* Encode n_tiles tiles of x (fp32 or bf16) [Methodology 1-3].
 * words: cap_words uint32 (see hq_encode_bound_words), 16-byte aligned;
 * offsets: n_tiles+1 uint64 bit offsets, 8-byte aligned; k: n_tiles uint8
 * Rice parameters.  Only words [0, ceil(offsets[n_tiles] / 32)) are written,
 * and none at or past cap_words (a stream that does not fit reports
 * HQ_ERR_CAPACITY). */
hq_status hq_encode(hq_plan_t plan, const void* x, hq_dtype dtype, uint64_t n_tiles,
                    uint32_t* words, uint64_t cap_words, uint64_t* offsets, uint8_t* k,
                    void* ws, void* stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: hq_encode
 * with its workspace in the library's own static device scratch instead of a
 * caller's buffer.  The scratch is one fixed array per GPU (the codec
 * workspace of HQ_NOALLOC_MAX_TILES tiles, about 12 MB), created with the
 * library's device code on each GPU that runs the call and held until the
 * process ends; the call itself allocates nothing.
 * Arguments as hq_encode, except: no ws; status is a caller-owned device
 * block of 256 bytes, 16-byte aligned, zero-filled once, where data errors
 * are recorded (read and clear it with hq_status_sync(status, stream)).
 * n_tiles above HQ_NOALLOC_MAX_TILES, and plans with the Haar rotation,
 * return HQ_ERR_ARG.  Every call on one GPU uses that GPU's one scratch, which
 * keeps the last call's contents: calls that overlap on one GPU (on two
 * streams, or from two threads without ordering) race; calls ordered on one
 * stream do not.  The result equals hq_encode's bit for bit. */
#define HQ_NOALLOC_MAX_TILES 32768u
hq_status hq_encode_noalloc(hq_plan_t plan, const void* x, hq_dtype dtype, uint64_t n_tiles, uint32_t* words,
                            uint64_t cap_words, uint64_t* offsets, uint8_t* k, void* status, void* stream);

/* Append n_tiles tiles of x to a stream that holds n_prev tiles: the new
 * records start at bit offsets[n_prev] (read on the device, so the call stays
 * asynchronous), the existing bits below it are kept, and offsets[n_prev ..
 * n_prev + n_tiles] and k[n_prev .. n_prev + n_tiles - 1] are written.  The
 * result is the stream that one hq_encode of both inputs, concatenated, would
 * give [Methodology 3: records are independent and abut].  cap_words counts
 * from word 0.  n_prev = 0 is hq_encode.  hq_kv_append: the dithered variant;
 * tile_base is the tile id of the first appended tile (for a continued KV
 * stream, the previous tile_base + n_prev). */
hq_status hq_append(hq_plan_t plan, const void* x, hq_dtype dtype, uint64_t n_tiles, uint32_t* words,
                    uint64_t cap_words, uint64_t* offsets, uint8_t* k, uint64_t n_prev, void* ws,
                    void* stream);
hq_status hq_kv_append(hq_plan_t plan, const void* x, hq_dtype dtype, uint64_t n_tiles,
                       uint64_t tile_base, uint32_t* words, uint64_t cap_words, uint64_t* offsets,
                       uint8_t* k, uint64_t n_prev, void* ws, void* stream);

/* Decode n_tiles tiles into y (fp32 or bf16): the inverse of each encode step
 * [Methodology 3: parse each record and restore the stripped bits;
 * Methodology 2: the lattice point in real coordinates (A2: (i, j sqrt 3)),
 * scaled by alpha; Methodology 1: the transposed transform D H^T / sqrt n,
 * H symmetric, so x_hat = D (c_dec H u_hat) with c_dec = alpha / sqrt 128].
 * y: n_tiles * 128 elements, 16-byte aligned, row-major like the input.
 * n_words is the number of readable words at `words` (at least
 * ceil(offsets[n_tiles] / 32)); records whose span leaves [0, n_words) are
 * reported as HQ_ERR_CORRUPT instead of being read.  bf16 output rounds the
 * fp32 value to nearest even.  ws: the codec workspace (its status word). */
hq_status hq_decode(hq_plan_t plan, const uint32_t* words, uint64_t n_words,
                    const uint64_t* offsets, const uint8_t* k, uint64_t n_tiles, void* y,
                    hq_dtype out_dtype, void* ws, void* stream);

/* KV variants with subtractive dither [Methodology 4]: the dither of tile t
 * is drawn from (seed, tile_base + t) by Philox4x32-10, so appended tokens
 * keep their own stream. */
hq_status hq_kv_encode(hq_plan_t plan, const void* x, hq_dtype dtype, uint64_t n_tiles,
                       uint64_t tile_base, uint32_t* words, uint64_t cap_words,
                       uint64_t* offsets, uint8_t* k, void* ws, void* stream);
hq_status hq_kv_decode(hq_plan_t plan, const uint32_t* words, uint64_t n_words,
                       const uint64_t* offsets, const uint8_t* k, uint64_t n_tiles,
                       uint64_t tile_base, void* y, hq_dtype out_dtype, void* ws, void* stream);

/* Attention scores against dithered compressed keys, without materialising
 * them [Methodology 4: the dithered KV quantiser keeps every inner product
 * q . k_hat unbiased; Methodology 1: the rotation is orthogonal, so
 * q . k_hat = <R q, R k_hat> is taken in the rotated domain, where the
 * decoder's k_hat is c_dec u_hat before its inverse transform]:
 * scores[(h*qph + g)*tiles_per_head + s] = q_{h,g} . k_hat_{h,s}
 * = c_dec <H D q_{h,g}, u_hat_{h,s}> for the keys of n_heads heads stored as
 * tiles h*tiles_per_head + s of one encode (tile ids tile_base + that).
 * With a Haar plan, = alpha <Q q_{h,g}, u_hat_{h,s}> (Q orthogonal): the
 * queries are rotated first, by a launch of their own, into the workspace.
 * q: fp32 [n_heads*qph][128] (16-byte aligned for a Haar plan); scores: fp32
 * [n_heads*qph][tiles_per_head].  1 <= qph <= 16.  ws: at least
 * hq_kv_scores_workspace_bytes(plan, n_heads, tiles_per_head, qph) bytes
 * (the codec workspace of the n_heads * tiles_per_head tiles suffices unless a
 * Haar plan has qph > tiles_per_head), zero-filled once, 16-byte aligned for a
 * Haar plan.  n_words: readable words at `words`, as for hq_decode.
 * Corrupt records score 0 and set HQ_ERR_CORRUPT. */
size_t hq_kv_scores_workspace_bytes(hq_plan_t plan, uint32_t n_heads, uint64_t tiles_per_head, uint32_t qph);
hq_status hq_kv_scores(hq_plan_t plan, const uint32_t* words, uint64_t n_words,
                       const uint64_t* offsets, const uint8_t* k, uint32_t n_heads,
                       uint64_t tiles_per_head, uint64_t tile_base, const float* q,
                       uint32_t qph, float* scores, void* ws, void* stream);

/* Matrix-vector products with a compressed weight matrix, without
 * materialising it: y[j*rows + r] = sum_c W_hat[r][c] x[j*cols + c] for nb
 * vectors, W_hat being the decoder's reconstruction of a rows x cols matrix
 * encoded by hq_encode (no dither) with tiles of 128 along each row (tile
 * r*(cols/128) + b holds columns 128b..128b+127 of row r).  Each tile adds
 * c_dec <u_hat, H D x_b> [Methodology 1: W_hat = D (c_dec H u_hat), H
 * symmetric], so the weights are never inverse-transformed.  x: fp32
 * [nb][cols], 16-byte aligned; y: fp32 [nb][rows]; cols a multiple of 128;
 * 1 <= nb <= 16; rows * cols / 128 and nb * rows below 2^32.  ws: at least
 * hq_gemv_workspace_bytes(rows, cols, nb) bytes, 16-byte aligned, zero-filled
 * once (a hq_workspace_bytes workspace of the same tiles is not enough in
 * general).  Three stream-ordered launches: rotate the vectors' blocks, one
 * dot product per tile and vector, fixed-order row sums.  Corrupt records
 * count as zeros and set HQ_ERR_CORRUPT. */
size_t hq_gemv_workspace_bytes(uint64_t rows, uint64_t cols, uint32_t nb);
hq_status hq_gemv(hq_plan_t plan, const uint32_t* words, uint64_t n_words,
                  const uint64_t* offsets, const uint8_t* k, uint64_t rows, uint64_t cols,
                  const float* x, uint32_t nb, float* y, void* ws, void* stream);

/* Matrix products with a compressed weight matrix on the matrix cores, for
 * 1 to 64 vectors: y[j*rows + r] = sum_c W_hat[r][c] x[j*cols + c], W_hat as
 * for hq_gemv (undithered Z, D4 or E8 stream; A2, whose codes are not
 * integers, returns HQ_ERR_ARG).  Per 128-column block, c_dec <u_hat, H D x_b>
 * [Methodology 1] for all vectors and 32 rows at a time is a dense product of
 * the rotated vectors with the integer codes: both are split into two bf16
 * pieces (x~ = hi + lo to within 2^-16 |x~|; codes exactly below 2^16) and
 * hi*Uh + hi*Ul + lo*Uh is accumulated in fp32 by bf16 MFMA, so the result is
 * within a few 2^-16 of the products' magnitudes plus fp32 accumulation.  The
 * column blocks are split over work-groups and the splits summed in a fixed
 * order (deterministic).  x: fp32 [nb][cols], 16-byte aligned; y: fp32
 * [nb][rows]; ws: hq_gemm_workspace_bytes(rows, cols, nb) bytes, 16-byte
 * aligned, zero-filled once.  Two or three stream-ordered launches.  Corrupt
 * records count as zeros and set HQ_ERR_CORRUPT. */
size_t hq_gemm_workspace_bytes(uint64_t rows, uint64_t cols, uint32_t nb);
hq_status hq_gemm(hq_plan_t plan, const uint32_t* words, uint64_t n_words,
                  const uint64_t* offsets, const uint8_t* k, uint64_t rows, uint64_t cols,
                  const float* x, uint32_t nb, float* y, void* ws, void* stream);

/* Attention of n_heads * qph queries over compressed keys and values, without
 * materialising them [Methodology 4: the dithered KV cache; Methodology 1:
 * the RHT is orthogonal, so q . k_hat = c_dec_K <H D q, u_hat_K> and
 * sum_j p_j v_hat_j = D (c_dec_V H sum_j p_j u_hat_V,j)]:
 *   out[h*qph + g] = sum_s softmax_s(scale * q_{h,g} . k_hat_{h,s}) v_hat_{h,s}
 * for the keys and values of head h stored as tiles h*seq + s of one
 * hq_kv_encode each (tile ids k_tile_base + that and v_tile_base + that).
 * plan_k and plan_v hold each stream's alpha and must share lattice, seed and
 * rotation kind.  With Haar plans the scores are alpha_K <Q q, u_hat_K> and
 * the output Q^T (alpha_V sum_j p_j u_hat_V,j / L): two more launches rotate
 * the queries (into the workspace) and the result.
 * q: fp32 [n_heads*qph][128] (finite); out: fp32 [n_heads*qph][128] (both
 * 16-byte aligned for Haar plans);
 * 1 <= qph <= 16; scale finite.  The weighted sums are formed in the rotated
 * domain by work-groups of 256 keys (maximum, weights e^(s - m) and their sum
 * per group) and combined per query in a fixed order, so results are
 * deterministic.  ws: at least hq_kv_attention_workspace_bytes(n_heads, seq,
 * qph) bytes, 16-byte aligned, zero-filled once.  Two stream-ordered
 * launches (four with Haar plans).  Records that do not parse count as zero vectors (score
 * scale * 0) and set HQ_ERR_CORRUPT. */
size_t hq_kv_attention_workspace_bytes(uint32_t n_heads, uint64_t seq, uint32_t qph);
hq_status hq_kv_attention(hq_plan_t plan_k, const uint32_t* k_words, uint64_t k_n_words,
                          const uint64_t* k_offsets, const uint8_t* k_k, uint64_t k_tile_base,
                          hq_plan_t plan_v, const uint32_t* v_words, uint64_t v_n_words,
                          const uint64_t* v_offsets, const uint8_t* v_k, uint64_t v_tile_base,
                          uint32_t n_heads, uint64_t seq, const float* q, uint32_t qph, float scale,
                          float* out, void* ws, void* stream);

/* Compact side information [Methodology 3: the offsets and Rice parameters
 * are the side information of the stream]: per chunk of 32 tiles one 96-byte
 * record, 3 bytes per tile instead of 9:
 *   bytes [0, 8)   uint64 bit offset of the chunk's first record
 *   bytes [8, 72)  uint16 end of the chunk's record j minus that offset
 *   bytes [72, 92) the chunk's 32 Rice parameters, 5 bits each, LSB first
 *   bytes [92, 96) zero
 * Entries past the last tile are zero.  side: hq_side_bytes(n_tiles) bytes,
 * 16-byte aligned, device memory.  hq_side_pack reads offsets[0..n_tiles]
 * and k; a chunk whose records span 2^16 bits or more (about 16 bits per
 * scalar) cannot be packed and sets HQ_ERR_CAPACITY in ws.  hq_side_unpack
 * writes offsets[0..n_tiles] and k[0..n_tiles-1].  Both asynchronous. */
size_t hq_side_bytes(uint64_t n_tiles);
hq_status hq_side_pack(const uint64_t* offsets, const uint8_t* k, uint64_t n_tiles, void* side,
                       void* ws, void* stream);
hq_status hq_side_unpack(const void* side, uint64_t n_tiles, uint64_t* offsets, uint8_t* k,
                         void* stream);

/* Container header: 64 bytes in HOST memory that make a stream
 * self-describing (the plan, the KV tile base, sizes), little-endian:
 *   0 magic "HQS1" | 4 version u16 = 1 | 6 lattice u8 | 7 flags u8 (bit 0
 *   dithered, bit 1 compact side information, bit 2 Haar rotation) | 8 tile
 *   u32 = 128 | 12 alpha
 *   f32 | 16 target bps f32 | 20 zero u32 | 24 seed u64 | 32 tile_base u64 |
 *   40 n_tiles u64 | 48 total bits u64 | 56 zero u32 | 60 CRC-32 (IEEE 802.3)
 *   of bytes 0..59.
 * hq_header_read returns HQ_ERR_CORRUPT for a wrong magic, version, checksum
 * or field; hq_plan_from_header makes the plan (alpha set) that decodes the
 * stream (for a Haar rotation, hq_plan_set_rotation must follow). */
#define HQ_HEADER_BYTES 64
typedef struct {
  hq_lattice lattice;
  int dithered, compact_side, tile;
  int rotation;  /* 1: the Haar rotation (hq_plan_set_rotation) */
  float alpha, bps;
  uint64_t seed, tile_base, n_tiles, total_bits;
} hq_header_info;
hq_status hq_header_write(hq_plan_t plan, int dithered, uint64_t tile_base, uint64_t n_tiles,
                          uint64_t total_bits, int compact_side, void* out);
hq_status hq_header_read(const void* in, hq_header_info* info);
hq_status hq_plan_from_header(const void* in, hq_plan_t* out);

/* Synchronise stream, return the lowest data error recorded in ws since the
 * last call, and clear it. */
hq_status hq_status_sync(void* ws, void* stream);

const char* hq_status_str(hq_status status);

#ifdef __cplusplus
}
#endif
#endif
