// Prefill GEMM of libbt for gfx950 (CDNA4), M > 16 tokens: the ternary x INT8
// product of "VibeVoice-ASR-BitNet Technical Report" sections 2.2.2 and 2.4.2
// (Figure 4) on v_mfma_i32_16x16x64_i8, and the same kernel for int8 weights
// (the I8_S product). The repacked weight layout and the code-offset identity
// (weights enter as codes w + 1; the epilogue subtracts the per-token sum of
// q) are described at the top of bt_kernels.hip.
//
// Prefill GEMM for M > 16. A workgroup of WGM x WGN waves computes a
// (WA*WGM) x (WW*WGN) tile of y (token rows x weight rows); each wave owns a
// WA x WW sub-tile held as (WA/16) x (WW/16) MFMA accumulators.
//
// K advances in stages (256 wide for ternary weights, 128 for int8 weights).
// The workgroup's activation rows for a
// stage (BM x KS int8) are copied from global memory straight into one of NS
// LDS buffers (buffer_load ... lds: no staging registers), while another
// buffer feeds the matrix cores. Rows past M, and columns past K, read as
// zero through the buffer bounds. In LDS a row's 16-byte chunks are stored
// XOR-swizzled, so the 16 rows an MFMA fragment read touches fall in 16
// different bank groups. Each wave keeps its WW/16 weight tiles' packed words
// for the coming stages in registers (one load per tile and lane) and unpacks
// each 16-element word right before the WA/16 MFMAs that use it.
//
// Workgroup order: consecutive workgroup ids go to different XCDs, so ids are
// remapped to give each XCD a compact block of output tiles (a group of
// token-row bands, walked down the bands first): its activation rows and
// weight tiles stay in that XCD's L2.

#include <hip/hip_runtime.h>

#include <math.h>
#include <string.h>

#include <algorithm>
#include <type_traits>

#include "bt_device.h"

#pragma clang fp contract(off)

namespace {

using bt::GemmArgs;

using bt::kXcds;

// Scheduling hint for the code just before it: interleave its kLoads vector
// loads with the MFMAs, one load followed by G MFMAs (the LDS copies and the
// fragment reads touch different stage arrays, so the order is free).
template <int kLoads, int G>
__device__ __forceinline__ void sched_loads_among_mfma() {
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one vector-memory read
        __builtin_amdgcn_sched_group_barrier(0x008, G, 0);   // G matrix-core ops
    }
}

// Output tile (mt, nt) of linear tile index L. Tiles are ordered in groups of
// group_m token-row bands; inside a group they run down the bands first. The
// tiles that run at the same time on one XCD (consecutive indices) then form
// a compact block whose activation rows and weight tiles both stay in that
// XCD's L2, instead of one band's row that sweeps every weight tile through it.
__device__ __forceinline__ void tile_coords(const GemmArgs& g, int L, int& mt, int& nt) {
    const int per_group = g.group_m * g.n_tiles;
    const int grp = L / per_group;
    const int first_m = grp * g.group_m;
    const int gm = min(g.m_tiles - first_m, g.group_m);
    const int r = L - grp * per_group;
    mt = first_m + r % gm;
    nt = r / gm;
}

__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, int8_t* lds_wave_base,
                                          uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (BT_LDS void*)lds_wave_base, 16, int(voff),
                                              int(soff), 0, 0);
}

// vmcnt(n) with the other counters left alone (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Epilogue of a full 16 x 64 output block of one wave (token rows mb..mb+15,
// columns nb..nb+63) given in the MFMA layout: lane l holds v[t] = columns
// 16t + 4(l/16) .. +3 of row l%16. Stored straight, every store instruction
// would write 16 rows x 64 bytes (half cache lines). Instead the block passes
// through the wave's own 4 KB of LDS (16-byte slots XOR-swizzled by row, so
// both the writes and the reads are conflict-free) and is stored row-wise:
// 16 lanes write 256 contiguous bytes of one row, whole cache lines.
// A wave's bias and layer-scale values for its 64 columns nb.. in the MFMA
// layout (columns nb + 16t + 4(l/16) .. +3), loaded once per tile.
struct EpiCols {
    v4f bias[4];
    v4f gamma[4];
};

__device__ __forceinline__ EpiCols epi_cols_load(const EpiArgs& e, int64_t nb, int lane) {
    EpiCols c;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int64_t n = nb + 16 * t + 4 * (lane >> 4);
        c.bias[t] = e.bias ? gld<v4f>(e.bias + n) : v4f{0.0f, 0.0f, 0.0f, 0.0f};
        c.gamma[t] = e.gamma ? gld<v4f>(e.gamma + n) : v4f{1.0f, 1.0f, 1.0f, 1.0f};
    }
    return c;
}

// The epilogue's column steps run in the MFMA layout, its residual add in the
// row layout (16-byte residual loads of whole rows).
__device__ __forceinline__ void gemm_store_block_rows(const v4f (&v)[4], float* ep, float* y,
                                                      int64_t ldy, int64_t mb, int64_t nb,
                                                      int lane, const EpiArgs& e,
                                                      const EpiCols& ec) {
    const int rl = lane & 15;
    const int cq = lane >> 4;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        v4f vt = v[t];
        if (e.bias) vt = vt + ec.bias[t];
        if (e.relu) {
            vt.x = vt.x > 0.0f ? vt.x : 0.0f;
            vt.y = vt.y > 0.0f ? vt.y : 0.0f;
            vt.z = vt.z > 0.0f ? vt.z : 0.0f;
            vt.w = vt.w > 0.0f ? vt.w : 0.0f;
        }
        if (e.gamma) vt = ec.gamma[t] * vt;
        lds_st<v4f>(ep + rl * 64 + (((4 * t + cq) ^ rl) * 4), vt);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 4 * j + cq;
        const int c = lane & 15;
        v4f row = lds_ld<v4f>(ep + r * 64 + ((c ^ r) * 4));
        const int64_t o = (mb + r) * ldy + nb + 4 * c;
        if (e.res) row = gld<v4f>(e.res + o) + row;
        __builtin_nontemporal_store(row, (BT_GLOBAL v4f*)(y + o));
    }
}

// Weight registers of one tile and stage for int8 weights: one 16-byte
// fragment per 64-wide step.
template <int NK>
struct W8Frag {
    v4u k[NK];
};

// kW8: the I8_S product (int8 weights, repacked by bt_repack_int8): the
// fragments go to the matrix cores as loaded and no row-sum correction applies.
template <int WA, int WW, int WGM, int WGN, int KS, int NS, bool kW8 = false>
__global__ __launch_bounds__(64 * WGM * WGN) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_kernel(GemmArgs g) {
    constexpr int BM = WA * WGM;
    constexpr int BN = WW * WGN;
    constexpr int NW = WGM * WGN;
    constexpr int TA = WA / 16;    // MFMA blocks along tokens per wave
    constexpr int TW = WW / 16;    // MFMA blocks (16-row weight tiles) per wave
    constexpr int NK = KS / 64;    // 64-wide MFMA steps per stage
    constexpr int CPR = KS / 16;   // 16-byte chunks per activation row per stage
    constexpr int kStage = BM * KS;                   // LDS bytes per activation stage
    constexpr int kDmaPerWave = BM * CPR / 64 / NW;   // 1 KB copies per wave per stage
    constexpr int kLoads = TW + kDmaPerWave;          // vector-memory ops per wave and stage
    // the stage's loads spread over the first three quarters of its MFMAs
    // (measured: +7-18% at 128 x 128 tiles; at 64 x 64 tiles a burst is better)
    constexpr int kMfmaPerStage = TA * TW * NK;
    constexpr bool kSpreadLoads = WA >= 64;
    constexpr int kLoadGap = kMfmaPerStage * 3 / 4 / kLoads > 0 ? kMfmaPerStage * 3 / 4 / kLoads : 1;
    static_assert(KS == 128 || KS == 256, "stage width");
    static_assert(WA % 16 == 0 && WW % 16 == 0, "wave tile");
    static_assert(NS >= 2 && (NS - 2) * kLoads < 64, "pipeline depth");
    static_assert(kDmaPerWave * 64 * NW == BM * CPR, "A stage must split evenly over waves");
    // One LDS array per pipeline stage: the copy that fills one stage and the
    // fragment reads of another then touch different objects, which lets the
    // compiler see that a read need not wait for every copy still in flight
    // (with one array it waits for all of them before each stage's reads).
    static_assert(NS <= 4, "at most four stage buffers");
    __shared__ __attribute__((aligned(16))) int8_t As0[kStage];
    __shared__ __attribute__((aligned(16))) int8_t As1[kStage];
    __shared__ __attribute__((aligned(16))) int8_t As2[NS > 2 ? kStage : 16];
    __shared__ __attribute__((aligned(16))) int8_t As3[NS > 3 ? kStage : 16];
    auto stage_buf = [&](int buf) -> int8_t* {
        return buf == 0 ? As0 : buf == 1 ? As1 : buf == 2 ? As2 : As3;
    };
    // After the main loop the stage buffers are idle (a barrier makes sure):
    // the row-wise epilogue's blocks live in the first one.
    constexpr bool kRowStores = WW == 64;   // row-wise epilogue through LDS
    float* const Ep = reinterpret_cast<float*>(As0);
    static_assert(!kRowStores || kStage >= NW * 16 * 64 * 4,
                  "epilogue blocks fit the first stage buffer");

    // Swizzled LDS slot of logical chunk c of row r: the 16 rows an MFMA
    // fragment read serves at once land in 16 distinct 4-bank groups.
    auto slot_of = [](int r, int c) {
        return KS == 256 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7));
    };

    // work unit = (tile, K range); a unit's ranges sit next to each other so
    // they run on the same XCD and share its L2
    const int xcd = blockIdx.x % kXcds;
    const int unit = xcd * g.per_xcd + blockIdx.x / kXcds;
    if (unit >= g.m_tiles * g.n_tiles * g.splits) return;
    const int tile_id = unit / g.splits;
    const int split = unit - tile_id * g.splits;
    int mt, nt;
    tile_coords(g, tile_id, mt, nt);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wm = wave / WGN;
    const int wn = wave - wm * WGN;
    const int64_t m0 = int64_t(mt) * BM;
    const int n0 = nt * BN;
    const int t0 = min(n0 / bt::kTileN + wn * (WW / bt::kTileN), g.tiles - 1);
    // a tile's 256-wide step is 1 KB of 2-bit codes, or 4 KB of int8 weights
    const uint32_t tile_bytes = uint32_t(g.steps) * (kW8 ? 4096u : 1024u);
    const int nst = (g.K + KS - 1) / KS;
    const int sb = split * g.sps;                 // first stage of this K range
    const int lst = min(g.sps, nst - sb);         // its stages

    // This wave's weight tiles as one buffer. The tile is part of the
    // per-lane (VGPR) offset, which the buffer's range check sees, so tiles
    // past N read as zero; the scalar offset only selects the stage. Per
    // stage a lane needs KS/64 words of its 16 bytes in a tile's 256-wide
    // step: all 16 bytes (KS = 256) or the matching 8-byte half (KS = 128).
    const __amdgpu_buffer_rsrc_t wrsrc = make_rsrc(
        g.w + int64_t(t0) * tile_bytes,
        uint32_t(min(WW / bt::kTileN, g.tiles - t0)) * tile_bytes);
    using BVec = typename std::conditional<
        kW8, W8Frag<NK>, typename std::conditional<KS == 256, v4u, v2u>::type>::type;
    // A stage past K (padding of the pipeline) reads zeros: bit 31 set in
    // its per-lane offsets puts them out of range (buffers here stay below
    // 2^31 bytes and the scalar offset below 2^30, so the sum cannot wrap),
    // and no byte is fetched. The masks are ORed in, never branched on: a
    // branch around the loads would make the compiler's wait counts
    // conservative.
    constexpr uint32_t kNowhere = 0x80000000u;
    auto load_b = [&](BVec (&b)[TW], int s, uint32_t pad) {
#pragma unroll
        for (int t = 0; t < TW; ++t) {
            const uint32_t voff = (uint32_t(lane) * 16u + uint32_t(t) * tile_bytes) | pad;
            if constexpr (kW8) {
                // int8: 64-wide steps of 1 KB, NK of them per stage
#pragma unroll
                for (int kk = 0; kk < NK; ++kk)
                    b[t].k[kk] = buf_ld16u(wrsrc, voff, uint32_t(s * NK + kk) * 1024u);
            } else if constexpr (KS == 256) {
                b[t] = buf_ld16u(wrsrc, voff, uint32_t(s) * 1024u);
            } else {
                const uint32_t koff = uint32_t(s >> 1) * 1024u + uint32_t(s & 1) * 8u;
                b[t] = __builtin_bit_cast(
                    v2u, __builtin_amdgcn_raw_buffer_load_b64(wrsrc, int(voff), int(koff), 0));
            }
        }
    };

    // The workgroup's activation rows as one buffer; rows past M read as zero
    // (the row is part of the per-lane offset, which the range check sees).
    const uint32_t arows = uint32_t(min(int64_t(BM), int64_t(g.M) - m0));
    const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(g.xq + m0 * g.K, arows * uint32_t(g.K));
    // Copy j of this wave fills LDS slots p = (wave*kDmaPerWave + j)*64 + lane:
    // row r = p / CPR, slot p % CPR, logical chunk c = slot_of^-1 (an XOR, its
    // own inverse). The row advances by 64/CPR per copy; the swizzle repeats
    // every 4 copies, so four per-lane chunk offsets serve all copies.
    constexpr int RPC = 64 / CPR;   // rows per copy
    const int r0 = wave * kDmaPerWave * RPC + lane / CPR;
    uint32_t avoff[4];
    uint32_t ccol[4];    // byte offset of this lane's chunk inside a stage
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = r0 + RPC * q;
        const int c = slot_of(r, lane % CPR);
        avoff[q] = uint32_t(r0) * uint32_t(g.K) + uint32_t(c) * 16u;
        ccol[q] = uint32_t(c) * 16u;
    }
    auto load_a = [&](int buf, int s, uint32_t pad) {
        const uint32_t kcol = uint32_t(s) * KS;
        // bytes of K left in this stage: a chunk past K (K % 16 == 0, so a
        // chunk is wholly in or out) must read zero, not the next row
        const uint32_t left = uint32_t(g.K) > kcol ? uint32_t(g.K) - kcol : 0u;
#pragma unroll
        for (int j = 0; j < kDmaPerWave; ++j) {
            const uint32_t voff = (avoff[j & 3] + uint32_t(RPC * j) * uint32_t(g.K)) | pad |
                                  (ccol[j & 3] >= left ? kNowhere : 0u);
            lds_dma16(arsrc, stage_buf(buf) + (wave * kDmaPerWave + j) * 1024, voff, kcol);
        }
    };

    // The MFMA runs transposed: A = weight fragment, B = activation fragment,
    // so C[n][m] and a lane holds 4 consecutive weight rows (outputs n) of one
    // token m, which the epilogue writes as one 16-byte store.
    v4i acc[TA][TW];
#pragma unroll
    for (int i = 0; i < TA; ++i)
#pragma unroll
        for (int t = 0; t < TW; ++t) acc[i][t] = v4i{0, 0, 0, 0};

    // fragment reads: row (wm*WA + 16i + lane%16), logical chunk 4kk + lane/16
    const int afrag = (wm * WA + (lane & 15)) * KS;
    int aslot[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) aslot[kk] = slot_of(lane & 15, 4 * kk + (lane >> 4)) * 16;

    // Software pipeline over NS stage buffers: the loads of stage s + NS - 1
    // go out while stage s is consumed, so each load has NS - 1 stages of
    // MFMAs to land. Stage s uses LDS buffer s % NS and weight registers
    // b[s % NS]; the loop is unrolled by NS so both indices are static. The
    // stage count is padded to a multiple of NS with stages that read zeros,
    // so every stage issues the same loads and every wait count is a
    // constant (conditional issues would make the compiler's own counts
    // conservative and stall on loads just issued).
    BVec b[NS][TW];
    auto issue = [&](int buf, BVec (&bn)[TW], int ls) {
        const uint32_t pad = ls < lst ? 0u : kNowhere;
        load_b(bn, sb + ls, pad);   // weights first: the stage wait then covers both
        load_a(buf, sb + ls, pad);
    };
    auto consume = [&](int buf, const BVec (&bc)[TW]) {
        const int8_t* abuf = stage_buf(buf) + afrag;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            v4i af[TA];
#pragma unroll
            for (int i = 0; i < TA; ++i) af[i] = lds_ld<v4i>(abuf + i * 16 * KS + aslot[kk]);
#pragma unroll
            for (int t = 0; t < TW; ++t) {
                v4i bf;
                if constexpr (kW8)
                    bf = __builtin_bit_cast(v4i, bc[t].k[kk]);
                else
                    bf = unpack16(bc[t][kk]);
#pragma unroll
                for (int i = 0; i < TA; ++i) acc[i][t] = mfma16x16x64(bf, af[i], acc[i][t]);
            }
        }
    };

    const int nst_pad = (lst + NS - 1) / NS * NS;
#pragma unroll
    for (int p = 0; p < NS - 1; ++p) issue(p, b[p], p);
    for (int s0 = 0; s0 < nst_pad; s0 += NS) {
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            // Stage s0 + u: its loads have landed once at most the NS - 2
            // later stages' are in flight; the barrier then also tells every
            // wave that all are done with buffer (u - 1) % NS, refilled next.
            __builtin_amdgcn_sched_barrier(0);
            wait_vmcnt<(NS - 2) * kLoads>();
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            const int nb = (u + NS - 1) % NS;   // static once unrolled
            issue(nb, b[nb], s0 + u + NS - 1);
            if constexpr (kSpreadLoads) {
                consume(u, b[u]);
                sched_loads_among_mfma<kLoads, kLoadGap>();
            } else {
                asm volatile("" ::: "memory");
                consume(u, b[u]);
            }
        }
    }
    // the padding loads still in flight write zeros into LDS: let them land,
    // and let every wave finish reading the stages, before LDS is reused
    wait_vmcnt<0>();
    __syncthreads();

    // Split K: this range's partial sums go to its own slice of the
    // workspace; splitk_reduce_kernel, launched next, adds the slices and
    // stores the output (the kernel boundary orders the two, with no fence).
    if (g.splits > 1) {
        int32_t* slice = g.ws + split * g.ws_slice;
        const bool vec = (g.N & 3) == 0;
#pragma unroll
        for (int i = 0; i < TA; ++i) {
            const int64_t mm = m0 + wm * WA + 16 * i + (lane & 15);
            if (mm >= g.M) continue;
#pragma unroll
            for (int t = 0; t < TW; ++t) {
                const int n = n0 + wn * WW + 16 * t + 4 * (lane >> 4);
                if (vec && n + 3 < g.N) {
                    gst<v4i>(slice + mm * g.N + n, acc[i][t]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < g.N) gst<int32_t>(slice + mm * g.N + n + r, acc[i][t][r]);
                }
            }
        }
        return;
    }

    // epilogue: acc[i][t][r] = C[n = n0 + wn*WW + 16t + 4(l/16) + r][m = m0 + wm*WA + 16i + l%16]
    const int nq = n0 + wn * WW + 4 * (lane >> 4);
    const bool full = m0 + BM <= g.M && n0 + BN <= g.N && (g.N & 3) == 0;
    // 128 x 96 tiles (two waves of 48 columns side by side): a tile row is three
    // 128-byte lines, the middle one half in each wave. The workgroup puts each
    // 16-row block together in LDS and stores it as whole rows, so every line is
    // written once and whole (direct stores wrote 1.35-1.41x the output bytes;
    // o at M = 4096 13.9 -> 12.95 us).
    constexpr bool kWgRows = WGN == 2 && WW == 48 && !kW8;
    if constexpr (kWgRows) {
        if (full && !g.acc) {
            constexpr int kRowB = BN * 4;          // bytes of one output row of the tile
            constexpr int kRowP = kRowB + 16;      // padded LDS row stride
            constexpr int kBlk = 16 * kRowP;       // one wm group's 16 rows
            static_assert(kStage >= WGM * kBlk, "epilogue rows fit the first stage buffer");
            char* blk = reinterpret_cast<char*>(As0) + wm * kBlk;
#pragma unroll
            for (int i = 0; i < TA; ++i) {
                const int64_t mb = m0 + wm * WA + 16 * i;
                const int32_t qs = gld<int32_t>(g.xsum + mb + (lane & 15));
                const float rs = gld<float>(g.xscale + mb + (lane & 15)) * g.w_scale;
#pragma unroll
                for (int t = 0; t < TW; ++t) {
                    const v4i a = acc[i][t] - qs;
                    const v4f v = {float(a.x) * rs, float(a.y) * rs, float(a.z) * rs,
                                   float(a.w) * rs};
                    const int col = wn * WW + 16 * t + 4 * (lane >> 4);
                    lds_st<v4f>(blk + (lane & 15) * kRowP + col * 4, v);
                }
                __syncthreads();
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    const int o = wn * (16 * kRowB / 2) + j * 1024 + lane * 16;
                    const int r = o / kRowB;
                    const int cb = o - r * kRowB;
                    v4f v = lds_ld<v4f>(blk + r * kRowP + cb);
                    const int64_t row = mb + r;
                    const int n = n0 + cb / 4;
                    v = epi_col4(g.epi, v, n);
                    if (g.epi.res) v = gld<v4f>(g.epi.res + row * g.N + n) + v;
                    __builtin_nontemporal_store(v, (BT_GLOBAL v4f*)(g.y + row * g.N + n));
                }
                __syncthreads();
            }
            return;
        }
    }
    if (kRowStores && full && !g.acc) {
        float* ep = Ep + wave * (16 * 64);
        const EpiCols ec = epi_cols_load(g.epi, n0 + wn * WW, lane);
#pragma unroll
        for (int i = 0; i < TA; ++i) {
            const int64_t mb = m0 + wm * WA + 16 * i;
            const int32_t qs = kW8 ? 0 : gld<int32_t>(g.xsum + mb + (lane & 15));
            const float rs = gld<float>(g.xscale + mb + (lane & 15)) * g.w_scale;
            v4f v[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const v4i a = acc[i][t] - qs;
                v[t] = v4f{float(a.x) * rs, float(a.y) * rs, float(a.z) * rs, float(a.w) * rs};
            }
            gemm_store_block_rows(v, ep, g.y, g.N, mb, n0 + wn * WW, lane, g.epi, ec);
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < TA; ++i) {
        const int64_t mm = m0 + wm * WA + 16 * i + (lane & 15);
        if (!full && mm >= g.M) continue;
        const int32_t qs = kW8 ? 0 : gld<int32_t>(g.xsum + mm);
        const float rs = gld<float>(g.xscale + mm) * g.w_scale;
        float* yrow = g.y + mm * g.N;
        int32_t* arow = g.acc ? g.acc + mm * g.N : nullptr;
#pragma unroll
        for (int t = 0; t < TW; ++t) {
            const int n = nq + 16 * t;
            const v4i a = acc[i][t] - qs;
            v4f yv = {float(a.x) * rs, float(a.y) * rs, float(a.z) * rs, float(a.w) * rs};
            if (full) {
                yv = epi_col4(g.epi, yv, n);
                if (g.epi.res) yv = gld<v4f>(g.epi.res + mm * g.N + n) + yv;
                __builtin_nontemporal_store(yv, (BT_GLOBAL v4f*)(yrow + n));
                if (arow) __builtin_nontemporal_store(a, (BT_GLOBAL v4i*)(arow + n));
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (n + r < g.N) {
                        float v = epi_col(g.epi, yv[r], n + r);
                        if (g.epi.res) v = g.epi.res[mm * g.N + n + r] + v;
                        gst<float>(yrow + n + r, v);
                        if (arow) gst<int32_t>(arow + n + r, a[r]);
                    }
                }
            }
        }
    }
}

// Persistent prefill GEMM (without the fused epilogue: a call that asks for
// one runs gemm_kernel, which has the registers for it). A workgroup of NW
// waves side by side along N
// owns a WA x (WW*NW) output tile at a time and walks a run of tiles: the
// tiles of one XCD's contiguous band, taken round-robin by that XCD's
// workgroups (consecutive tiles share token rows, which stay in the XCD's
// L2). Its stage pipeline runs straight across tile boundaries: while the
// last stages of a tile are consumed, the first stages of the next tile are
// already being loaded, so a tile costs no start-up latency and the epilogue
// of one tile overlaps the loads of the next. Stages per tile are padded to a
// multiple of NS with stages that read zeros (a buffer's range check turns
// their loads into no-ops), which keeps every stage's wait count constant.
//
// The body serves two launches: one problem over the whole grid
// (gemm_persistent_kernel), or many independent problems in one grid
// (gemm_persistent_grouped_kernel), where each problem owns `per_wg`
// workgroup slots in every XCD and a workgroup walks only its problem's tiles.
// `slot` is the workgroup's slot among its problem's slots of one XCD. `lda`
// is the byte stride of the activation rows: g.K, or more when g views one
// K range of a wider problem. Without y (g.y null) only acc is stored.
template <int WA, int WW, int NW, int KS, int NS>
__device__ __forceinline__ void gemm_persistent_body(const GemmArgs& g, int slot, int per_wg,
                                                     int lda) {
    constexpr int BM = WA;
    constexpr int BN = WW * NW;
    constexpr int TA = WA / 16;
    constexpr int TW = WW / 16;
    constexpr int NK = KS / 64;
    constexpr int CPR = KS / 16;
    constexpr int kStage = BM * KS;
    constexpr int kDmaPerWave = BM * CPR / 64 / NW;
    constexpr int kLoads = TW + kDmaPerWave;
    static_assert(KS == 128 || KS == 256, "stage width");
    static_assert(WA % 16 == 0 && WW % 16 == 0, "wave tile");
    static_assert(NS >= 2 && (NS - 2) * kLoads < 64, "pipeline depth");
    static_assert(kDmaPerWave * 64 * NW == BM * CPR, "A stage must split evenly over waves");
    // One LDS array per pipeline stage: the copy that fills one stage and the
    // fragment reads of another then touch different objects, which lets the
    // compiler see that a read need not wait for every copy still in flight
    // (with one array it waits for all of them before each stage's reads).
    static_assert(NS <= 4, "at most four stage buffers");
    __shared__ __attribute__((aligned(16))) int8_t As0[kStage];
    __shared__ __attribute__((aligned(16))) int8_t As1[kStage];
    __shared__ __attribute__((aligned(16))) int8_t As2[NS > 2 ? kStage : 16];
    __shared__ __attribute__((aligned(16))) int8_t As3[NS > 3 ? kStage : 16];
    auto stage_buf = [&](int buf) -> int8_t* {
        return buf == 0 ? As0 : buf == 1 ? As1 : buf == 2 ? As2 : As3;
    };
    constexpr bool kRowStores = WW == 64;   // row-wise epilogue through LDS
    __shared__ __attribute__((aligned(16))) float Ep[kRowStores ? NW * 16 * 64 : 4];

    auto slot_of = [](int r, int c) {
        return KS == 256 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7));
    };

    // this workgroup's tiles: first, first + per_wg, ... below hi
    const int xcd = blockIdx.x % kXcds;
    const int total = g.m_tiles * g.n_tiles;
    const int lo = xcd * g.per_xcd;
    const int hi = min(lo + g.per_xcd, total);
    const int first = lo + slot;
    if (first >= hi) return;
    const int count = (hi - first + per_wg - 1) / per_wg;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const uint32_t tile_bytes = uint32_t(g.steps) * 1024u;
    const int nst = (g.K + KS - 1) / KS;
    const int nst_pad = (nst + NS - 1) / NS * NS;

    // Buffers of a tile: its token rows and this wave's weight tiles. Rows
    // past M and weight tiles past N read as zero (range check).
    auto tile_rsrc = [&](int tile_id, __amdgpu_buffer_rsrc_t& ra, __amdgpu_buffer_rsrc_t& rw) {
        int mt, nt;
        tile_coords(g, tile_id, mt, nt);
        const int64_t m0 = int64_t(mt) * BM;
        const int t0 = min(nt * (BN / bt::kTileN) + wave * TW, g.tiles - 1);
        ra = make_rsrc(g.xq + m0 * lda, uint32_t(min(int64_t(BM), int64_t(g.M) - m0)) * uint32_t(lda));
        rw = make_rsrc(g.w + int64_t(t0) * tile_bytes, uint32_t(min(TW, g.tiles - t0)) * tile_bytes);
    };

    constexpr uint32_t kNowhere = 0x80000000u;
    using BVec = typename std::conditional<KS == 256, v4u, v2u>::type;
    auto load_b = [&](BVec (&b)[TW], __amdgpu_buffer_rsrc_t rw, int s, uint32_t pad) {
        const uint32_t koff = KS == 256 ? uint32_t(s) * 1024u
                                        : uint32_t(s >> 1) * 1024u + uint32_t(s & 1) * 8u;
#pragma unroll
        for (int t = 0; t < TW; ++t) {
            const uint32_t voff = (uint32_t(lane) * 16u + uint32_t(t) * tile_bytes) | pad;
            if constexpr (KS == 256)
                b[t] = buf_ld16u(rw, voff, koff);
            else
                b[t] = __builtin_bit_cast(
                    v2u, __builtin_amdgcn_raw_buffer_load_b64(rw, int(voff), int(koff), 0));
        }
    };
    constexpr int RPC = 64 / CPR;
    const int r0 = wave * kDmaPerWave * RPC + lane / CPR;
    uint32_t avoff[4];
    uint32_t ahigh[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = r0 + RPC * q;
        const int c = slot_of(r, lane % CPR);
        avoff[q] = uint32_t(r0) * uint32_t(lda) + uint32_t(c) * 16u;
        ahigh[q] = c >= 8 ? kNowhere : 0u;
    }
    const bool tail128 = KS == 256 && (g.K & 255) != 0;
    auto load_a = [&](int buf, __amdgpu_buffer_rsrc_t ra, int s, uint32_t pad) {
        const uint32_t kcol = uint32_t(s) * KS;
        const uint32_t tail = (tail128 && s == nst - 1) ? 0xffffffffu : 0u;
#pragma unroll
        for (int j = 0; j < kDmaPerWave; ++j) {
            const uint32_t voff = (avoff[j & 3] + uint32_t(RPC * j) * uint32_t(lda)) | pad |
                                  (ahigh[j & 3] & tail);
            lds_dma16(ra, stage_buf(buf) + (wave * kDmaPerWave + j) * 1024, voff, kcol);
        }
    };

    v4i acc[TA][TW];
#pragma unroll
    for (int i = 0; i < TA; ++i)
#pragma unroll
        for (int t = 0; t < TW; ++t) acc[i][t] = v4i{0, 0, 0, 0};
    const int afrag = (lane & 15) * KS;
    int aslot[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) aslot[kk] = slot_of(lane & 15, 4 * kk + (lane >> 4)) * 16;
    // Per 64-wide step: the TW weight fragments unpacked once, then the TA
    // activation fragments in two halves, each half through all TW weight
    // tiles (half the activation registers of reading all TA up front).
    static_assert(TA % 2 == 0, "two halves of activation fragments");
    auto consume = [&](int buf, const BVec (&bc)[TW]) {
        const int8_t* abuf = stage_buf(buf) + afrag;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            v4i bf[TW];
#pragma unroll
            for (int t = 0; t < TW; ++t) bf[t] = unpack16(bc[t][kk]);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                v4i af[TA / 2];
#pragma unroll
                for (int i = 0; i < TA / 2; ++i)
                    af[i] = lds_ld<v4i>(abuf + (h * TA / 2 + i) * 16 * KS + aslot[kk]);
#pragma unroll
                for (int t = 0; t < TW; ++t)
#pragma unroll
                    for (int i = 0; i < TA / 2; ++i)
                        acc[h * TA / 2 + i][t] = mfma16x16x64(bf[t], af[i], acc[h * TA / 2 + i][t]);
            }
        }
    };

    BVec b[NS][TW];
    __amdgpu_buffer_rsrc_t ra_cur, rw_cur, ra_nxt, rw_nxt;
    tile_rsrc(first, ra_cur, rw_cur);
#pragma unroll
    for (int p = 0; p < NS - 1; ++p) {
        const uint32_t pad = p < nst ? 0u : kNowhere;
        load_b(b[p], rw_cur, p, pad);
        load_a(p, ra_cur, p, pad);
    }

    for (int k = 0; k < count; ++k) {
        const int tile_id = first + k * per_wg;
        const bool has_next = k + 1 < count;
        tile_rsrc(has_next ? tile_id + per_wg : tile_id, ra_nxt, rw_nxt);
        int mt, nt;
        tile_coords(g, tile_id, mt, nt);
        const int64_t m0 = int64_t(mt) * BM;
        const int n0 = nt * BN;

        // the epilogue's per-token row sums and scales, fetched early
        int32_t qs[TA];
        float rs[TA];
#pragma unroll
        for (int i = 0; i < TA; ++i) {
            const int64_t mc = min(m0 + 16 * i + (lane & 15), int64_t(g.M) - 1);
            qs[i] = gld<int32_t>(g.xsum + mc);
            rs[i] = gld<float>(g.xscale + mc) * g.w_scale;
        }

        for (int s0 = 0; s0 < nst_pad; s0 += NS) {
#pragma unroll
            for (int u = 0; u < NS; ++u) {
                // stage s0 + u: wait for its loads (the NS - 2 later stages'
                // may stay in flight), then a barrier, after which every wave
                // is also done with buffer (u - 1) % NS, refilled next
                __builtin_amdgcn_sched_barrier(0);
                wait_vmcnt<(NS - 2) * kLoads>();
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                const int nb = (u + NS - 1) % NS;   // static once unrolled
                const int tgt = s0 + u + NS - 1;
                const bool in_cur = tgt < nst_pad;
                const int st = in_cur ? tgt : tgt - nst_pad;
                const bool valid = st < nst && (in_cur || has_next);
                const uint32_t pad = valid ? 0u : kNowhere;
                load_b(b[nb], in_cur ? rw_cur : rw_nxt, st, pad);
                load_a(nb, in_cur ? ra_cur : ra_nxt, st, pad);
                consume(u, b[u]);
                // spread the stage's loads over its matrix-core work (one per
                // eight MFMAs) rather than issuing them in one burst: a burst
                // fills the vector-memory queue and stalls the wave (+10% measured)
                sched_loads_among_mfma<kLoads, 8>();
            }
        }

        // epilogue: acc[i][t][r] = C[n = n0 + wave*WW + 16t + 4(l/16) + r][m = m0 + 16i + l%16]
        const int nq = n0 + wave * WW + 4 * (lane >> 4);
        const bool full = m0 + BM <= g.M && n0 + BN <= g.N && (g.N & 3) == 0;
        const bool rows = kRowStores && full && !g.acc;
#pragma unroll
        for (int i = 0; i < TA; ++i) {
            const int64_t mm = m0 + 16 * i + (lane & 15);
            if (rows) {
                v4f v[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const v4i a = acc[i][t] - qs[i];
                    const float r = rs[i];
                    v[t] = v4f{float(a.x) * r, float(a.y) * r, float(a.z) * r, float(a.w) * r};
                }
                gemm_store_block_rows(v, Ep + wave * (16 * 64), g.y, g.N, m0 + 16 * i,
                                      n0 + wave * WW, lane, EpiArgs{}, EpiCols{});
            } else if (full || mm < g.M) {
                float* yrow = g.y + mm * g.N;
                int32_t* arow = g.acc ? g.acc + mm * g.N : nullptr;
#pragma unroll
                for (int t = 0; t < TW; ++t) {
                    const int n = nq + 16 * t;
                    const v4i a = acc[i][t] - qs[i];
                    const float r = rs[i];
                    const v4f yv = {float(a.x) * r, float(a.y) * r, float(a.z) * r, float(a.w) * r};
                    if (full) {
                        if (g.y) __builtin_nontemporal_store(yv, (BT_GLOBAL v4f*)(yrow + n));
                        if (arow) __builtin_nontemporal_store(a, (BT_GLOBAL v4i*)(arow + n));
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if (n + e < g.N) {
                                if (g.y) gst<float>(yrow + n + e, yv[e]);
                                if (arow) gst<int32_t>(arow + n + e, a[e]);
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < TW; ++t) acc[i][t] = v4i{0, 0, 0, 0};
        }
        ra_cur = ra_nxt;
        rw_cur = rw_nxt;
    }
    // the padding loads still in flight write zeros into LDS: let them land
    // before the workgroup can exit
    wait_vmcnt<0>();
}

template <int WA, int WW, int NW, int KS, int NS>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_persistent_kernel(GemmArgs g) {
    gemm_persistent_body<WA, WW, NW, KS, NS>(g, int(blockIdx.x) / kXcds,
                                             int(gridDim.x) / kXcds, g.K);
}

// Many problems in one launch: the problem owning slot blockIdx.x / 8 (one
// lane per descriptor compares its first slot, a ballot counts them), then
// that problem's persistent walk. Descriptors are ordered by first slot.
// A problem split along K (splits > 1) has g.slots slots per K range, range r
// after range r - 1; a workgroup of range r walks the problem viewed as that
// range alone (activations and weights offset to its first stage, K its
// length, the full row stride) and stores the raw int32 partial sums in the
// range's slice of g.ws, with row sums read from the zeros after the slices
// and no y; splitk_reduce_kernel, launched next, adds the slices.
template <int WA, int WW, int NW, int KS, int NS>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_persistent_grouped_kernel(const GemmArgs* __restrict__ descs, int32_t count) {
    const int slot = int(blockIdx.x) / kXcds;
    const int lane = threadIdx.x & 63;
    int p = -1;
    for (int base = 0; base < count; base += 64) {
        const int i = base + lane;
        const int begin = i < count ? descs[i].slot_begin : INT32_MAX;
        p += int(__popcll(__ballot(begin <= slot)));
    }
    p = __builtin_amdgcn_readfirstlane(p);
    GemmArgs g = descs[p];
    const int lda = g.K;
    int local = slot - g.slot_begin;
    if (g.splits > 1) {
        // ranges are counted in 128-element pieces of K (sps is even, so a
        // range starts on a 256-wide weight step; the last may end half-way
        // through one, which the body's K tail handles)
        const int r = local / g.slots;
        local -= r * g.slots;
        const int base = r * g.sps;                 // first 128-element piece of the range
        const int pieces = (g.K + 127) / 128;
        g.xq += int64_t(base) * 128;
        g.w += int64_t(base / 2) * 1024;            // two pieces per 1 KB weight step
        g.K = min(g.sps, pieces - base) * 128;
        g.acc = g.ws + int64_t(r) * g.ws_slice;
        g.xsum = g.ws + int64_t(g.splits) * g.ws_slice;
        g.y = nullptr;
    }
    gemm_persistent_body<WA, WW, NW, KS, NS>(g, local, g.slots, lda);
}

// Launch of the tiled GEMM for one tile shape (the shape itself is chosen on
// the host, gemm_choice): one workgroup per (tile, K range), numbered so that
// an XCD's workgroups take one compact block of tiles.
template <int WA, int WW, int WGM, int WGN, int KS, int NS, bool kW8 = false>
bt_status launch_gemm(GemmArgs g, hipStream_t stream) {
    constexpr int BM = WA * WGM;
    constexpr int BN = WW * WGN;
    g.m_tiles = int32_t(bt::ceil_div(g.M, BM));
    g.n_tiles = int32_t(bt::ceil_div(g.N, BN));
    if (g.splits <= 1) {
        g.splits = 1;
        g.sps = int32_t(bt::ceil_div(g.K, KS));
    }
    const int64_t total = int64_t(g.m_tiles) * g.n_tiles * g.splits;
    g.per_xcd = int32_t(bt::ceil_div(total, kXcds));
    g.group_m = bt::gemm_group_m(g.m_tiles, g.n_tiles, bt::ceil_div(g.per_xcd, g.splits));
    const int64_t grid = int64_t(g.per_xcd) * kXcds;
    if (grid > (int64_t(1) << 31) - 1) return BT_ERR_SHAPE;
    (void)hipGetLastError();
    hipLaunchKernelGGL((gemm_kernel<WA, WW, WGM, WGN, KS, NS, kW8>), dim3(unsigned(grid)),
                       dim3(64 * WGM * WGN), 0, stream, g);
    return hipGetLastError() == hipSuccess ? BT_OK : BT_ERR_DEVICE;
}

// The persistent kernel's shape: waves of 128 tokens x 64 weight rows, four
// side by side (tiles of 128 x 256), 256-wide K stages in two buffers (64 KB of
// LDS, plus 16 KB for the epilogue: two workgroups fill a compute unit's 160
// KB), two workgroups per compute unit. Measured on the long-prefill stack's
// grouped launch against 128-wide stages in three buffers: 4.51-4.54 ->
// 4.41-4.42 ms (fewer waits and barriers per MFMA).
constexpr int kPersistWA = bt::kPersistBM;
constexpr int kPersistNW = bt::kPersistBN / 64;
constexpr int kPersistKS = 256;
constexpr int kPersistNS = 2;
constexpr int kPersistWgsPerCu = 2;

// Compute units of the current device (queried on every call: the host keeps
// no state between calls).
int device_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        return 256;
    return n;
}

template <int WA, int WW, int NW, int KS, int NS>
bt_status launch_gemm_persistent(GemmArgs g, hipStream_t stream) {
    constexpr int BM = WA;
    constexpr int BN = WW * NW;
    g.splits = 1;   // a single launch walks whole tiles
    g.m_tiles = int32_t(bt::ceil_div(g.M, BM));
    g.n_tiles = int32_t(bt::ceil_div(g.N, BN));
    const int64_t total = int64_t(g.m_tiles) * g.n_tiles;
    if (total > (int64_t(1) << 31) - 1) return BT_ERR_SHAPE;
    g.per_xcd = int32_t(bt::ceil_div(total, kXcds));
    g.group_m = bt::gemm_group_m(g.m_tiles, g.n_tiles, g.per_xcd);
    // one workgroup per resident slot, a multiple of the XCD count, and no
    // more than there are tiles in an XCD's band
    const int64_t slots = int64_t(device_cus()) * kPersistWgsPerCu / kXcds;
    const int64_t per_xcd_wgs = std::max<int64_t>(1, std::min<int64_t>(slots, g.per_xcd));
    (void)hipGetLastError();
    hipLaunchKernelGGL((gemm_persistent_kernel<WA, WW, NW, KS, NS>),
                       dim3(unsigned(per_xcd_wgs * kXcds)), dim3(64 * NW), 0, stream, g);
    return hipGetLastError() == hipSuccess ? BT_OK : BT_ERR_DEVICE;
}

// A grouped GEMM plan (bt_matmul_plan_build with M > 16): the host copy sizes
// the grid (every problem's slots, in every XCD), the device copy feeds the
// kernel.
bt_status launch_gemm_grouped(const bt::PlanHeader* hdr, const GemmArgs* dev_descs,
                              hipStream_t stream) {
    const int64_t grid = hdr->total_blocks * kXcds;
    if (grid < 1 || grid > (int64_t(1) << 31) - 1) return BT_ERR_SHAPE;
    (void)hipGetLastError();
    hipLaunchKernelGGL((gemm_persistent_grouped_kernel<kPersistWA, 64, kPersistNW, kPersistKS, kPersistNS>),
                       dim3(unsigned(grid)), dim3(64 * kPersistNW), 0, stream, dev_descs,
                       hdr->count);
    return hipGetLastError() == hipSuccess ? BT_OK : BT_ERR_DEVICE;
}

// Split K, second launch: output element (m, n .. n+3) = the sum of its
// partial sums over the K ranges (exact int32), then the same rescale and
// epilogue as the GEMM kernels: one thread per 4 consecutive outputs.
template <bool kW8>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs g) {
    const int64_t quads = int64_t(g.M) * ((g.N + 3) / 4);
    for (int64_t qd = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; qd < quads;
         qd += int64_t(gridDim.x) * blockDim.x) {
        const int64_t m = qd / ((g.N + 3) / 4);
        const int n = int((qd - m * ((g.N + 3) / 4)) * 4);
        const int64_t o = m * g.N + n;
        const int32_t qs = kW8 ? 0 : gld<int32_t>(g.xsum + m);
        const float rs = gld<float>(g.xscale + m) * g.w_scale;
        if ((g.N & 3) == 0) {
            // up to eight slices' loads in flight at once, then their sum
            v4i a = gld<v4i>(g.ws + o);
            for (int sp0 = 1; sp0 < g.splits; sp0 += 8) {
                v4i p[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    p[j] = sp0 + j < g.splits ? gld<v4i>(g.ws + (sp0 + j) * g.ws_slice + o)
                                              : v4i{0, 0, 0, 0};
                a += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
            }
            a -= qs;
            v4f y = {float(a.x) * rs, float(a.y) * rs, float(a.z) * rs, float(a.w) * rs};
            y = epi_col4(g.epi, y, n);
            if (g.epi.res) y = gld<v4f>(g.epi.res + o) + y;
            __builtin_nontemporal_store(y, (BT_GLOBAL v4f*)(g.y + o));
            if (g.acc) gst<v4i>(g.acc + o, a);
        } else {
            for (int r = 0; r < 4 && n + r < g.N; ++r) {
                int32_t a = gld<int32_t>(g.ws + o + r);
                for (int sp = 1; sp < g.splits; ++sp) a += gld<int32_t>(g.ws + sp * g.ws_slice + o + r);
                a -= qs;
                float y = epi_col(g.epi, float(a) * rs, n + r);
                if (g.epi.res) y = g.epi.res[o + r] + y;
                g.y[o + r] = y;
                if (g.acc) g.acc[o + r] = a;
            }
        }
    }
}

template <bool kW8>
bt_status launch_splitk_reduce(const GemmArgs& g, hipStream_t stream) {
    const int64_t quads = int64_t(g.M) * ((g.N + 3) / 4);
    const int64_t grid = std::min<int64_t>(bt::ceil_div(quads, 256), int64_t(1) << 20);
    hipLaunchKernelGGL(splitk_reduce_kernel<kW8>, dim3(unsigned(grid)), dim3(256), 0, stream, g);
    return hipGetLastError() == hipSuccess ? BT_OK : BT_ERR_DEVICE;
}

// I8_S product for a small weight matrix and many tokens (the tokenizer's early
// stages: N x K int8 of at most 64 KB, K <= 512, M up to hundreds of thousands).
// Every workgroup first copies the whole repacked matrix, [tile][64-wide step]
// in 1 KB pieces, into LDS. Each wave then streams blocks of 16 tokens: one
// 16-byte activation fragment per lane and 64-wide step, prefetched a block
// ahead, meets the 16-row weight tiles held in LDS, four tiles per pass, and
// the fp32 rows go out at once. Per token these shapes read K + 4 bytes and
// write 4 N, so the output bytes bound them; the generic GEMM's 128-token
// tiles with one K stage each spend their time in start-up and epilogue.
template <int NK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NK >= 8 ? 2 : 4))) void i8_stream_kernel(GemmArgs g) {
    extern __shared__ __attribute__((aligned(16))) int8_t wl[];
    constexpr uint32_t kNowhere = 0x80000000u;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int tiles = g.tiles;
    // after the weights: each wave's 4 KB for turning 16 x 64 output blocks into rows
    float* const ep = reinterpret_cast<float*>(wl + int64_t(tiles) * NK * 1024) + (tid >> 6) * 1024;
    const int64_t steps64 = int64_t(g.steps) * 4;   // 64-wide steps per repacked tile
    for (int i = tid; i < tiles * NK * 64; i += 256) {
        const int tk = i >> 6;
        const int t = tk / NK;
        const int kk = tk - t * NK;
        lds_st<v4u>(wl + int64_t(i) * 16,
                    gld<v4u>(g.w + (int64_t(t) * steps64 + kk) * 1024 + (i & 63) * 16));
    }
    __syncthreads();

    const int64_t nblocks = (int64_t(g.M) + 15) / 16;
    const int64_t stride = int64_t(gridDim.x) * 4;
    int64_t b = int64_t(blockIdx.x) * 4 + (tid >> 6);
    // rows past M and K chunks past K read as zero (M * K < 2^31 is checked on the host)
    const __amdgpu_buffer_rsrc_t ar = make_rsrc(g.xq, uint32_t(int64_t(g.M) * g.K));
    const int ml = lane & 15;
    const uint32_t kq = 16u * uint32_t(lane >> 4);
    auto load_a = [&](v4u (&a)[NK], int64_t blk) {
        const int64_t m = blk * 16 + ml;
        const uint32_t base = m < g.M ? uint32_t(m) * uint32_t(g.K) : kNowhere;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            const uint32_t k = 64u * kk + kq;
            a[kk] = buf_ld16u(ar, k < uint32_t(g.K) ? base + k : kNowhere, 0);
        }
    };
    auto load_s = [&](int64_t blk) {
        return gld<float>(g.xscale + min(blk * 16 + ml, int64_t(g.M) - 1));
    };
    v4u a_cur[NK], a_nxt[NK];
    load_a(a_cur, b);
    float s_cur = load_s(b);
    const bool vec = (g.N & 3) == 0;
    for (; b < nblocks; b += stride) {
        load_a(a_nxt, b + stride);
        const float s_nxt = load_s(b + stride);
        const int64_t m = b * 16 + ml;
        const float rs = s_cur * g.w_scale;
        const bool full_rows = (b + 1) * 16 <= int64_t(g.M) && vec && !g.acc;
        for (int p = 0; p < tiles; p += 4) {
            v4i acc[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[t] = v4i{0, 0, 0, 0};
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                const v4i af = __builtin_bit_cast(v4i, a_cur[kk]);
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    if (p + t < tiles)
                        acc[t] = mfma16x16x64(
                            lds_ld<v4i>(wl + (int64_t(p + t) * NK + kk) * 1024 + lane * 16), af,
                            acc[t]);
            }
            // acc[t][r] = C[n = 16(p+t) + 4(l/16) + r][token m]
            if (full_rows && 16 * (p + 4) <= g.N) {
                // a whole 16 x 64 block: rows go out 256 contiguous bytes at a time
                const EpiCols ec = epi_cols_load(g.epi, 16 * p, lane);
                v4f v[4];
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    v[t] = v4f{float(acc[t].x) * rs, float(acc[t].y) * rs, float(acc[t].z) * rs,
                               float(acc[t].w) * rs};
                gemm_store_block_rows(v, ep, g.y, g.N, b * 16, 16 * p, lane, g.epi, ec);
                continue;
            }
            if (m < g.M) {
                float* yrow = g.y + m * g.N;
                int32_t* arow = g.acc ? g.acc + m * g.N : nullptr;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    if (p + t >= tiles) continue;
                    const int n = 16 * (p + t) + 4 * (lane >> 4);
                    const v4i a = acc[t];
                    v4f yv = {float(a.x) * rs, float(a.y) * rs, float(a.z) * rs, float(a.w) * rs};
                    if (vec && n + 3 < g.N) {
                        yv = epi_col4(g.epi, yv, n);
                        if (g.epi.res) yv = gld<v4f>(g.epi.res + m * g.N + n) + yv;
                        __builtin_nontemporal_store(yv, (BT_GLOBAL v4f*)(yrow + n));
                        if (arow) __builtin_nontemporal_store(a, (BT_GLOBAL v4i*)(arow + n));
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            if (n + r < g.N) {
                                float v = epi_col(g.epi, yv[r], n + r);
                                if (g.epi.res) v = g.epi.res[m * g.N + n + r] + v;
                                gst<float>(yrow + n + r, v);
                                if (arow) gst<int32_t>(arow + n + r, a[r]);
                            }
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) a_cur[kk] = a_nxt[kk];
        s_cur = s_nxt;
    }
}

template <int NK>
bt_status launch_i8_stream(GemmArgs g, hipStream_t stream) {
    g.tiles = int32_t(bt::ceil_div(g.N, bt::kTileN));
    const size_t lds = size_t(g.tiles) * NK * 1024 + 4 * 4096;
    const int64_t nblocks = bt::ceil_div(g.M, 16);
    const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(6, int64_t(163840 / lds)));
    const int64_t wgs = std::max<int64_t>(
        1, std::min<int64_t>(bt::ceil_div(nblocks, 4), int64_t(device_cus()) * per_cu));
    (void)hipGetLastError();
    hipLaunchKernelGGL(i8_stream_kernel<NK>, dim3(unsigned(wgs)), dim3(256), lds, stream, g);
    return hipGetLastError() == hipSuccess ? BT_OK : BT_ERR_DEVICE;
}

// Runs the kernel gemm_choice picked for the shape; with split K, each range
// writes its own slice of the workspace and a second launch adds the slices.
bt_status dispatch_gemm(GemmArgs g, bool int8_weights, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
    const bt::GemmChoice c =
        bt::gemm_choice(g.M, g.N, g.K, int8_weights, !epi_any(g.epi));
    g.splits = 1;
    if (c.splits > 1) {
        const size_t need = bt::gemm_workspace_bytes(c, g.M, g.N);
        if (!workspace || workspace_bytes < need) return BT_ERR_WORKSPACE;
        if (!bt::aligned16(workspace)) return BT_ERR_ALIGN;
        g.splits = c.splits;
        g.sps = c.sps;
        g.ws = static_cast<int32_t*>(workspace);
        g.ws_slice = int64_t(bt::gemm_slice_bytes(g.M, g.N) / sizeof(int32_t));
    }
    bt_status st;
    if (int8_weights && c.kind == 4) {
        const int nk = bt::i8_stream_steps(g.K);
        return nk == 1 ? launch_i8_stream<1>(g, stream)
             : nk == 2 ? launch_i8_stream<2>(g, stream)
             : nk == 4 ? launch_i8_stream<4>(g, stream)
                       : launch_i8_stream<8>(g, stream);
    }
    if (int8_weights) {
        st = c.kind == 3   ? launch_gemm<32, 32, 2, 2, 128, 2, true>(g, stream)
             : c.kind == 2 ? launch_gemm<64, 64, 2, 2, 128, 2, true>(g, stream)
                           : launch_gemm<128, 64, 1, 4, 128, 2, true>(g, stream);
        if (st == BT_OK && g.splits > 1) st = launch_splitk_reduce<true>(g, stream);
        return st;
    }
    if (c.kind == 0)
        return launch_gemm_persistent<kPersistWA, 64, kPersistNW, kPersistKS, kPersistNS>(g, stream);
    st = c.kind == 3   ? launch_gemm<32, 32, 2, 2, 256, 2>(g, stream)
         : c.kind == 5 ? launch_gemm<64, 48, 2, 2, 256, 2>(g, stream)
         : c.kind == 2 ? launch_gemm<64, 64, 2, 2, 256, 2>(g, stream)
                       : launch_gemm<128, 64, 1, 4, 128, 2>(g, stream);
    if (st == BT_OK && g.splits > 1) st = launch_splitk_reduce<false>(g, stream);
    return st;
}

}  // namespace

namespace bt {

bt_status gemm_dispatch(GemmArgs g, bool int8_weights, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
    return dispatch_gemm(g, int8_weights, workspace, workspace_bytes, stream);
}

bt_status gemm_reduce_slices(const GemmArgs& g, hipStream_t stream) {
    return launch_splitk_reduce<false>(g, stream);
}

bt_status gemm_grouped_launch(const PlanHeader* hdr, const void* plan_dev, hipStream_t stream) {
    const auto* descs = reinterpret_cast<const GemmArgs*>(static_cast<const char*>(plan_dev) +
                                                          sizeof(PlanHeader));
    bt_status st = launch_gemm_grouped(hdr, descs, stream);
    // projections split along K: one more launch each adds the slices (the
    // kernel boundary orders it after every range's partial sums)
    const auto* host = reinterpret_cast<const GemmArgs*>(hdr + 1);
    for (int32_t i = 0; st == BT_OK && i < hdr->count; ++i)
        if (host[i].splits > 1) st = launch_splitk_reduce<false>(host[i], stream);
    return st;
}

}  // namespace bt
