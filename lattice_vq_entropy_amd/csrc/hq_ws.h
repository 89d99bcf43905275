// hq_ws.h -- layout of the caller-owned workspace shared by libhq's host code
// and kernels.  The caller zero-fills it once when allocating it; afterwards
// the kernels keep it consistent themselves (no per-call memset).
#pragma once
#include <stdint.h>

namespace hq {

struct WsHeader {
  uint32_t ticket;        // next chunk ticket of the running encode
  uint32_t done;          // work-groups of the running encode that finished
  uint32_t epoch;         // encode calls completed; tags look-back descriptors
  uint32_t status;        // bit (1 << code) for every error seen since the last sync
  unsigned long long bits;  // total payload bits of a length-only pass
  double sumsq;             // sum of squares of a calibration input
  uint32_t pad[56];
};
static_assert(sizeof(WsHeader) == 256, "workspace header is 256 bytes");

constexpr int kChunkTiles = 32;           // tiles per work-group
constexpr int kPasses = kChunkTiles / 16; // 16 tiles per pass (4 per wave)
constexpr int kMaxRecordWords = 93;       // ceil((16 + 128*23) / 32)
constexpr int kStageWords = kChunkTiles * kMaxRecordWords + 4;

// Look-back descriptor: [63:62] flag (1 aggregate, 2 inclusive prefix),
// [61:38] epoch (24 bits), [37:0] bit count.
constexpr uint64_t kDescFlagAgg = 1ull << 62;
constexpr uint64_t kDescFlagIncl = 2ull << 62;
constexpr int kDescEpochShift = 38;
constexpr uint64_t kDescValueMask = (1ull << 38) - 1;

inline uint64_t ws_chunks(uint64_t n_tiles) { return (n_tiles + kChunkTiles - 1) / kChunkTiles; }
inline uint64_t ws_bytes(uint64_t n_tiles) {
  uint64_t c = ws_chunks(n_tiles);
  return sizeof(WsHeader) + ((c * 16 + 255) & ~uint64_t(255));
}

}  // namespace hq
