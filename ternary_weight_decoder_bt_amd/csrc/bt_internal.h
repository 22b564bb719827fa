// Internal definitions shared by the host half (bt_host.cpp) and the device half
// (bt_kernels.hip) of libbt. Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "bt.h"

namespace bt {

constexpr int kTileN = 16;          // weight rows per repacked tile (one MFMA N block)
constexpr int kStepK = 64;          // K per matrix-core step (16x16x64 int8)
constexpr int kSuperK = 256;        // K per 128-bit load per lane (four steps)
constexpr int kGemvWaves = 4;       // waves per GEMV workgroup, one tile each
constexpr int kQuantThreads = 256;  // threads per quantized row

constexpr uint32_t kPlanMagicQuant = 0x42545141u;   // "AQTB"
constexpr uint32_t kPlanMagicGemv = 0x42544d47u;    // "GMTB"

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// One GEMV problem as the kernel sees it. The single-matrix call passes it by
// value; a grouped plan stores an array of them in device memory.
struct GemvDesc {
    const int8_t* xq;
    const float* xscale;
    const int32_t* xsum;
    const uint8_t* w;       // repacked tiles
    float* y;
    int32_t* acc;           // may be null
    int32_t* ws;            // split-K partial sums, M x (tiles*16); null when chunks == 1
    uint32_t* cnt;          // split-K arrival counters, one per tile
    float w_scale;
    int32_t M, N, K;
    int32_t tiles;          // ceil(N / 16)
    int32_t chunks;         // K-splits per tile
    int32_t steps_per_chunk;  // 256-wide K steps per chunk (the last chunk may be shorter)
    int32_t full_steps;     // K / 256
    int32_t half_step;      // 1 if K % 256 == 128 (one trailing 128-wide step)
    int64_t block_begin;    // first workgroup of this problem in a grouped launch
    int64_t blocks;         // workgroups of this problem
};

struct QuantDesc {
    const float* x;
    int8_t* xq;
    float* xscale;
    int32_t* xsum;
    int64_t M, K;
    int64_t row_begin;      // first workgroup (= row) of this problem in a grouped launch
};

struct PlanHeader {
    uint32_t magic;
    int32_t count;
    int64_t total_blocks;
};

// Split-K policy of a single GEMV call; also sizes its workspace.
void gemv_shape(int64_t M, int64_t N, int64_t K, GemvDesc* d);
size_t gemv_workspace_bytes(const GemvDesc& d);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace bt
