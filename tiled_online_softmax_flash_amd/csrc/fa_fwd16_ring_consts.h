// Launch geometry of the LDS-ring kernel, shared with the host dispatcher.
#pragma once

namespace fa {
constexpr int kRingBlockRows = 256;  // query rows per workgroup
constexpr int kRingRowBlocks = 1;    // 32-row blocks per wave: 8 waves of 32 rows, two per SIMD
// threads of a 256-row workgroup whose waves hold rb 32-row blocks each
constexpr int ring_threads(int rb) { return 64 * (kRingBlockRows / (32 * rb)); }
}  // namespace fa
