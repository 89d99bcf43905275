// hq_ws.h -- layout of the caller-owned workspace shared by libhq's host code
// and kernels.  The caller zero-fills it once when allocating it (the status
// word must start clear); everything else is written before it is read within
// each call.
#pragma once
#include <stdint.h>

namespace hq {

struct WsHeader {
  uint32_t reserved0[3];
  uint32_t status;          // bit (1 << code) for every error seen since the last sync
  unsigned long long bits;  // total payload bits of a length-only pass
  double sumsq;             // sum of squares of a calibration input
  uint32_t pad[56];
};
static_assert(sizeof(WsHeader) == 256, "workspace header is 256 bytes");

constexpr int kChunkTiles = 32;            // tiles per work-group
constexpr int kPasses = kChunkTiles / 16;  // 16 tiles per pass (4 per wave)
constexpr int kMaxRecordWords = 93;        // ceil((16 + 128*23) / 32)
// staging words per chunk: the longest chunk (32 * 2960 bits = 2960 words),
// one zero word after it, rounded up to whole uint4
constexpr int kSlotWords = 2964;
// decode: LDS words holding one chunk's stream span
constexpr int kStageWords = kChunkTiles * kMaxRecordWords + 4;

inline uint64_t ws_chunks(uint64_t n_tiles) { return (n_tiles + kChunkTiles - 1) / kChunkTiles; }
inline uint64_t ws_align(uint64_t b) { return (b + 255) & ~uint64_t(255); }

// Regions after the header: agg (u32 per chunk), E (u64 per chunk + 1; the
// length-only pass keeps its per-chunk partials here), loc (u32 per tile
// slot), tailw (u32 per chunk), staging (kSlotWords u32 per chunk).  Each
// region starts on 256 bytes.
struct WsLayout {
  uint64_t agg, E, loc, tailw, stage, bytes;
};
inline WsLayout ws_layout(uint64_t n_tiles) {
  const uint64_t c = ws_chunks(n_tiles);
  WsLayout L;
  L.agg = sizeof(WsHeader);
  L.E = L.agg + ws_align(4 * c);  // 64 counts a block: the scan reads whole uint4
  L.loc = L.E + ws_align(8 * (c + 1));
  L.tailw = L.loc + ws_align(4 * c * kChunkTiles);
  L.stage = L.tailw + ws_align(4 * c);
  L.bytes = L.stage + 4 * c * (uint64_t)kSlotWords;
  return L;
}
inline uint64_t ws_bytes(uint64_t n_tiles) { return ws_layout(n_tiles).bytes; }

}  // namespace hq
