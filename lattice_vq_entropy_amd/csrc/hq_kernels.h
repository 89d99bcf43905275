// hq_kernels.h -- kernel argument blocks and launchers (internal to libhq).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hq_ws.h"

namespace hq {

constexpr int kOutF32 = 0, kOutBf16 = 1, kOutScores = 2, kOutGemv = 3, kOutRot = 4;

struct EncArgs {
  const void* x;
  uint64_t n_tiles;
  uint32_t* words;
  uint64_t cap_words;
  uint64_t* offsets;
  uint8_t* kout;
  // signs of D in the two lane layouts (sign_layouts on the host): for bf16
  // pairs and for fp32 values
  uint32_t sl16[4], sl32[4];
  float c_enc;
  uint32_t key0, key1;
  uint64_t tile_base;
  WsHeader* ws;
  uint32_t n_chunks;
  uint32_t* agg;     // bits per chunk
  uint64_t* E;       // chunk bit offsets, n_chunks + 1
  uint32_t* loc;     // chunk-local bit offset per tile
  uint32_t* tailw;   // last 32 stream bits of each chunk
  uint32_t* stage;   // slot_words staging words per chunk
  uint32_t slot_words;  // a multiple of 4, at most kSlotWords
  unsigned long long* partials;  // length-only pass: bits per chunk
  const uint64_t* base;  // append: the existing stream's end bit (device), else null
  const void* x0;        // pre-rotated input (x is the rotated tiles): the original, for error kinds
  int x0_bf16;
  // placement above the self-scan limit: chunk offsets within blocks of 1024,
  // and the bits of the blocks before each block (or, at most 64 blocks, the
  // blocks' own totals: block_totals)
  const uint32_t* eloc;
  const uint64_t* blockpre;
  int block_totals;
  int direct;  // one chunk: encode_k writes the stream itself (set by the launcher)
};

struct DecArgs {
  const uint32_t* words;
  uint64_t n_words;
  const uint64_t* offsets;
  const uint8_t* kin;
  uint64_t n_tiles;
  void* y;
  uint32_t sl16[4], sl32[4];  // as in EncArgs
  float c_dec;
  uint32_t key0, key1;
  uint64_t tile_base;
  WsHeader* ws;
  const float* q;
  float* scores;
  uint32_t qph;
  uint64_t tiles_per_head;
  int q_rot;  // the queries are already rotated (dense rotation: Q q), else H D q is formed here
  // matrix-vector mode: rotated vector blocks H D x (nb x cols fp32), per-tile
  // dot products (n_tiles x nb fp32), vectors per call, 128-column blocks per row
  const float* xr;
  float* dots;
  uint32_t nb;
  uint32_t nblk;
};

struct GemvArgs {
  const float* x;   // nb x cols
  float* xr;        // nb x cols: H D x per 128-column block
  const float* dots;
  float* y;         // nb x rows
  uint32_t rows, nblk, nb;
  uint32_t sl32[4];
  float c_dec;
};

// in: 0 fp32 tiles, 1 bf16 tiles, 2 fp32 tiles already rotated (scaled by c_enc here)
hipError_t launch_encode(int lat, bool dither, int in, bool len_only, const EncArgs& a, hipStream_t st);
hipError_t launch_decode(int lat, bool dither, int out, const DecArgs& a, dim3 grid, hipStream_t st);
// Attention over compressed keys and values (both dithered, one lattice and
// seed): per work-group one KV head, kAttnQ of its queries and kAttnChunks
// chunks of 32 keys.
constexpr uint32_t kAttnChunks = 8;
constexpr uint32_t kAttnQ = 4;  // queries per work-group
constexpr uint32_t kAttnPart = 2 + 128;  // per (head, group, query): max, sum, 128 weighted values
struct AttnArgs {
  const uint32_t* kw; uint64_t kn; const uint64_t* ko; const uint8_t* kk; uint64_t ktb; float ck;
  const uint32_t* vw; uint64_t vn; const uint64_t* vo; const uint8_t* vk; uint64_t vtb; float cv;
  uint32_t sl32[4];
  uint32_t key0, key1;
  const float* q;
  int q_rot;          // the queries are already rotated (dense rotation: Q q)
  float* rot_out;     // dense rotation: c_dec_V A / L per query, for rot_k with Q^T (else null)
  uint32_t qph;
  float scale;
  uint64_t seq;
  uint32_t n_groups;  // work-groups per head
  float* part;        // [n_heads][n_groups][qph][kAttnPart]
  float* out;         // [n_heads * qph][128]
  WsHeader* ws;
};

hipError_t launch_gemv(int lat, const DecArgs& d, const GemvArgs& g, hipStream_t st);

// Matrix products with MFMA: up to kGemmMaxVec vectors; weights in tiles of
// 32 rows x one 128-column block per step.
constexpr uint32_t kGemmMaxVec = 64;
constexpr uint32_t kGemmRecWords = 96;  // staging per tile: a record spans at most 94 words
struct GemmArgs {
  const uint32_t* words; uint64_t n_words; const uint64_t* offsets; const uint8_t* k;
  WsHeader* ws;
  const float* x;        // nb x cols
  uint16_t* xp;          // bf16 pieces [2][nbp][cols] of H D x per block: hi, then lo
  float* part;           // [splits][nbp][rows] when splits > 1
  float* y;              // nb x rows
  uint32_t rows, nblk, nb, nbp, splits, per;  // per: column blocks per split
  uint32_t sl32[4];
  float c_dec;
};
hipError_t launch_gemm(int lat, const GemmArgs& g, hipStream_t st);
hipError_t launch_attention(int lat, const AttnArgs& a, uint32_t n_heads, hipStream_t st);
// Dense rotation of tiles: y = fl32(fma-chain(M x) * scale) per tile, M given
// as Mt[j][i] (128 x 128 fp32, device).
struct RotArgs {
  const void* x; int in_bf16;
  void* y; int out_bf16;
  const float* mt;
  float scale;
  uint64_t n_tiles;
};
hipError_t launch_rot(const RotArgs& a, hipStream_t st);
hipError_t launch_side(bool pack, const uint64_t* offsets_in, const uint8_t* k_in, const uint8_t* side_in,
                       uint64_t n, uint8_t* side_out, uint64_t* offsets_out, uint8_t* k_out, WsHeader* ws,
                       hipStream_t st);
hipError_t launch_absmax(const void* x, bool bf16, uint64_t n, uint32_t* partials, uint32_t max_blocks, uint32_t* out,
                         hipStream_t st);
hipError_t launch_set_u64(uint64_t* p, uint64_t v, hipStream_t st);

}  // namespace hq
