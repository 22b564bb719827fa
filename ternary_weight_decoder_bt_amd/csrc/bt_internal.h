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
constexpr uint32_t kPlanMagicGemvFused = 0x42544646u;   // "FFTB"
constexpr uint32_t kPlanMagicRepack = 0x4254504bu;      // "KPTB"
constexpr uint32_t kPlanMagicGemm = 0x42544d4du;        // "MMTB"
constexpr uint32_t kPlanMagicTern = 0x42545454u;        // "TTTB"

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Largest K of the ternary matmul: |acc| <= 127 * K stays below 2^24, so
// every accumulator is exact in int32 and converts to fp32 exactly, and every
// byte offset the kernels form inside one tile's buffer (at most 128 rows of
// K int8, or 4 * K weight bytes per 16-row tile) fits their 32-bit offsets.
constexpr int64_t kMaxK = BT_MAX_K;

// GEMV tuning: weight steps (1 KB per wave) loaded per batch, and the LDS
// slice that holds one workgroup's int8 activations (M rows x its K range).
constexpr int kGemvBatch = 6;
constexpr int kGemvLdsBytes = 40960;
constexpr int kGemvFillWaves = 1024;   // waves that keep every compute unit streaming
// Single calls with fewer workgroups than this split each tile's 16 weight rows
// over up to kGemvRowPartsMax workgroups (see gemv_shape).
constexpr int kGemvFillBlocks = 256;
constexpr int kGemvRowPartsMax = 2;
constexpr int kGemvGroupedTilesPerWave = 2;

// Epilogue on the fp32 output (all optional): bias add, ReLU, per-output
// layer scale, residual add, in that order.
struct EpiArgs {
    const float* bias;      // [N] or null
    const float* gamma;     // [N] or null
    const float* res;       // M x N or null (may be the output buffer itself)
    int32_t relu;
    int32_t pad_;
};

// One GEMV problem as the kernel sees it. The single-matrix call passes it by
// value; a grouped plan stores an array of them in device memory.
// Arguments of the prefill GEMM launches (bt_gemm.hip).
struct GemmArgs {
    const int8_t* xq;
    const float* xscale;
    const int32_t* xsum;
    const uint8_t* w;
    float* y;
    int32_t* acc;
    float w_scale;
    int32_t M, N, K, tiles, steps;   // steps: 256-wide stages (Kp / 256)
    int32_t m_tiles, n_tiles, per_xcd;
    int32_t group_m;        // token-row bands per group of the tile order (tile_coords)
    EpiArgs epi;
    int32_t splits, sps;    // K ranges per tile and stages per range (1, all: no split)
    int32_t* ws;            // split K: one M x N int32 slice of partial sums per range
    int64_t ws_slice;       // int32 elements from one slice to the next
    int32_t slots;          // grouped persistent launch: this problem's workgroups per XCD
    int32_t slot_begin;     // and the first of them (workgroup id / 8)
};

struct GemvDesc {
    const float* x;         // fused quantization: fp32 activations (else null)
    int8_t* xq;             // unfused: input. fused: optional output (written once)
    float* xscale;          // same
    int32_t* xsum;          // same
    const uint8_t* w;       // repacked tiles
    float* y;
    int32_t* acc;           // may be null
    int32_t* ws;            // split-K partial sums, M x (tiles*16); null when chunks == 1
    uint32_t* cnt;          // split-K arrival counters, one per tile
    float w_scale;
    int32_t M, N, K;
    int32_t tiles;          // ceil(N / 16)
    int32_t steps;          // ceil(K / 256): 1 KB weight loads per tile
    int32_t chunks;         // K-splits per tile
    int32_t steps_per_chunk;
    int32_t tiles_per_wave;
    int32_t lds_row;        // bytes per activation row in LDS (steps_per_chunk*256 + 16)
    int32_t slices;         // chunks > 1: 1 = each chunk stores its partial sums in its
                            // own M x N slice of ws and a second launch adds them (single
                            // calls); 0 = atomics into ws, last chunk finishes (plans)
    int32_t waves_per_tile; // 1, 2 or 4: a tile's K range within a chunk is split over
                            // this many waves of one workgroup (tiles_per_wave is then 1)
    int32_t row_parts;      // 1, 2 or 4: a tile's 16 weight rows are split over this many
                            // workgroups, each loading and storing its 16 / row_parts rows
    int32_t pad_;
    int64_t groups;         // workgroups per chunk = ceil(tiles / (4 * tiles_per_wave)) * row_parts
    int64_t block_begin;    // first workgroup of this problem in a grouped launch
    int64_t blocks;         // workgroups of this problem = groups * chunks
    EpiArgs epi;            // zero: no epilogue
};

struct QuantDesc {
    const float* x;
    int8_t* xq;
    float* xscale;
    int32_t* xsum;
    int64_t M, K;
    int64_t row_begin;      // first workgroup of this problem in a grouped launch
};

// Quantization of rows short enough for one wave each (the row in registers,
// four rows per 256-thread workgroup); longer rows take a workgroup each.
constexpr bool quant_wave_rows(int64_t K) { return K % 4 == 0 && K <= 2048; }

struct RepackDesc {
    const uint8_t* packed;
    uint8_t* out;
    int32_t N, K;
    int32_t steps;          // ceil(K / 256): 1 KB output blocks per 16-row tile
    int32_t pad_;
    int64_t block_begin;    // first output block of this tensor in a grouped launch
    int64_t blocks;         // ceil(N / 16) * steps
};

// One tensor of a grouped ternarization: its first-pass workgroups write
// `nparts` partial sums of |w| to `partials`, its second-pass workgroups code
// and pack it. part_begin / pack_begin: its first workgroup of each launch.
struct TernDesc {
    const float* w;
    uint8_t* packed;
    float* scale;
    double* partials;
    int64_t N, K;
    float eps;
    int32_t nparts;
    int32_t pack_blocks;
    int32_t pad_;
    int64_t part_begin;
    int64_t pack_begin;
};

struct PlanHeader {
    uint32_t magic;
    int32_t count;
    int64_t total_blocks;
};

// Work split of a GEMV: K is split only where the activations do not fit one
// workgroup's LDS slice.
void gemv_shape(int64_t M, int64_t N, int64_t K, bool grouped, bool split_rows, GemvDesc* d);
size_t gemv_workspace_bytes(const GemvDesc& d);          // plans: atomics + counters
size_t gemv_partial_bytes(const GemvDesc& d);
size_t gemv_single_workspace_bytes(const GemvDesc& d);   // single calls: slices + d, row sums

// GEMM shape choice (M > 16), made from the shape alone so that the host can
// size the workspace: the persistent kernel (128 x 256 tiles) when there are
// at least as many such tiles as resident workgroup slots, else the tiled
// kernel with the tile shape of least estimated time (128 x 128, 128 x 96 or
// 64 x 64), with K split into `splits` ranges of `sps` stages when there are
// fewer tiles than compute units (partial sums meet in an int32 workspace).
constexpr int kGemmSlots = 512;   // resident workgroups (two per compute unit)
// 64-wide K steps the small-matrix I8_S kernel holds per weight tile: ceil(K/64)
// rounded up to a power of two (1, 2, 4 or 8).
inline int i8_stream_steps(int64_t K) {
    const int64_t s = (K + 63) / 64;
    return s <= 1 ? 1 : s <= 2 ? 2 : s <= 4 ? 4 : 8;
}
struct GemmChoice {
    int kind;        // 0 persistent, 1 tiled 128 x 256, 2 tiled 128 x 128, 3 tiled 64 x 64,
                     // 4 small int8 weight matrix held in LDS (i8_stream_kernel),
                     // 5 tiled 128 x 96
    int splits;      // K ranges (kinds 2, 3, 5), else 1
    int sps;         // stages per range (stage = 256-wide K for ternary, 128 for int8)
    int64_t tiles;   // output tiles of the chosen kind
};
GemmChoice gemm_choice(int64_t M, int64_t N, int64_t K, bool int8_weights, bool persistent_ok);
size_t gemm_workspace_bytes(const GemmChoice& c, int64_t M, int64_t N);
inline size_t gemm_slice_bytes(int64_t M, int64_t N) {
    return (size_t(M) * size_t(N) * sizeof(int32_t) + 255) & ~size_t(255);
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The persistent GEMM's output tiles (kPersistBM token rows x kPersistBN
// weight rows), the XCDs a launch spreads them over, and the resident
// workgroup slots of one XCD (two per compute unit, 32 compute units).
constexpr int kPersistBM = 128;
constexpr int kPersistBN = 256;
constexpr int kXcds = 8;
constexpr int kSlotsPerXcd = kGemmSlots / kXcds;
// grouped GEMM plans: target 128-element pieces of K per K range of a split
// projection (one layer at M = 512: ranges of 14 pieces 43.0-43.8 us, of 12
// 44.4-44.7 us, of 18 44.2-44.4 us, of 24 46.6-46.7 us)
constexpr int kPlanSplitStages = 16;

// Token-row bands per tile group of the GEMM's tile order: as many as one
// XCD's share of the tiles spans, so that share is one compact block.
inline int32_t gemm_group_m(int32_t m_tiles, int32_t n_tiles, int64_t tiles_per_xcd) {
    const int64_t gm = ceil_div(tiles_per_xcd, n_tiles);
    return int32_t(gm < 1 ? 1 : gm > m_tiles ? m_tiles : gm);
}

// bt_gemm.hip: the prefill GEMM for M > 16 (shape dispatch, split K and its
// reduction launch), and that reduction alone for a split single-call GEMV
// (same slice layout).
bt_status gemm_dispatch(GemmArgs g, bool int8_weights, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);
bt_status gemm_reduce_slices(const GemmArgs& g, hipStream_t stream);
// A grouped GEMM plan's launch (plan_dev: the plan's device copy).
bt_status gemm_grouped_launch(const PlanHeader* hdr, const void* plan_dev, hipStream_t stream);

}  // namespace bt
