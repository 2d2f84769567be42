// Compile-time shape constants shared by host and device code.  Internal header.
#pragma once

namespace hhr {

constexpr int kD = 128;    // head_dim
constexpr int kNW = 4;     // 32-bit words per 128-bit code (appendix Table 4 of HHR: 128 bits)
constexpr int kMaxNW = 8;  // widest code: 256 bits (HHR appendix Figure 10 sweeps the width)
constexpr int kPS = 16;    // page size
constexpr int kWave = 64;  // CDNA wavefront width
constexpr int kMaxG = 16;  // query heads per KV head

// Split-K attention partial of one (b, g, chunk, query head): o~[128], m, l,
// padded so that each partial starts on a 16-byte boundary.
constexpr int kPartStride = kD + 4;

// Fine top-k distance chunks: 64 kept pages (1024 candidates) per workgroup.
constexpr int kHamChunkPages = 64;
constexpr int ham_chunks(int pages) { return (pages + kHamChunkPages - 1) / kHamChunkPages; }
// Candidates per cumulative H histogram block, and blocks per (b, g).
constexpr int kCumBlock = 256;
constexpr int ham_cum_blocks(int p_max) { return (p_max * kPS + kCumBlock - 1) / kCumBlock; }

}  // namespace hhr
