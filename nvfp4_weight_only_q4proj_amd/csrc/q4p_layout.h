// q4p_layout.h — sizes of the packed weight layout (host and device).
// The byte layout inside a tile is described in q4p_device.h.
#pragma once

#include <stdint.h>

namespace q4p {

constexpr int kTileN = 16;            // weight rows per tile
constexpr int kTileK = 128;           // k per tile: eight 16-element scale blocks
constexpr int kTileCodeBytes = 1024;  // 16 x 128 e2m1 codes
constexpr int kTileScaleBytes = 128;  // 16 x 8 e4m3 scales

constexpr int64_t n_tiles(int64_t N) { return (N + kTileN - 1) / kTileN; }
constexpr int64_t k_tiles(int64_t K) { return (K + kTileK - 1) / kTileK; }

}  // namespace q4p
