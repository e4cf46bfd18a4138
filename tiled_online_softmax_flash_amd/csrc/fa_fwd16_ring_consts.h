// Launch geometry of the LDS-ring kernel, shared with the host dispatcher.
#pragma once

namespace fa {
constexpr int kRingBlockRows = 256;  // 8 waves x 32 query rows
constexpr int kRingThreads = 512;
}  // namespace fa
