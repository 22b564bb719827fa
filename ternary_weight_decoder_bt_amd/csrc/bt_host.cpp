// Host half of libbt: status strings, the canonical 2-bit format, argument
// checks shared with the device half, and plan building for grouped launches.
// Nothing in this file touches the GPU.

#include <string.h>

#include <algorithm>
#include <cmath>
#include <limits>

#include "bt_internal.h"

using bt::ceil_div;

extern "C" const char* bt_status_string(bt_status s) {
    switch (s) {
        case BT_OK: return "ok";
        case BT_ERR_NULL: return "a required pointer is NULL";
        case BT_ERR_SHAPE: return "invalid shape (M, N, K >= 1, K % 128 == 0 and K <= 131072 required)";
        case BT_ERR_VALUE: return "invalid value (weight outside {-1,0,1}, code 3, or non-finite scale)";
        case BT_ERR_ALIGN: return "device pointer not 16-byte aligned";
        case BT_ERR_DEVICE: return "HIP runtime error";
        case BT_ERR_WORKSPACE: return "workspace missing or too small";
    }
    return "unknown status";
}

static bool valid_nk(int64_t N, int64_t K) {
    if (N < 1 || K < 1 || K % BT_GROUP_K) return false;
    // every byte count and int32 index the kernels form must fit
    if (N > (int64_t(1) << 30) || K > bt::kMaxK) return false;
    const int64_t padded = ceil_div(N, bt::kTileN) * bt::kTileN;
    return padded <= std::numeric_limits<int64_t>::max() / (K + bt::kSuperK);
}

extern "C" size_t bt_packed_bytes(int64_t N, int64_t K) {
    return valid_nk(N, K) ? size_t(N) * size_t(K) / 4 : 0;
}

extern "C" size_t bt_repacked_bytes(int64_t N, int64_t K) {
    if (!valid_nk(N, K)) return 0;
    return size_t(ceil_div(N, bt::kTileN) * bt::kTileN) *
           size_t(ceil_div(K, bt::kSuperK) * bt::kSuperK) / 4;
}

// Canonical layout (blog post "Paper 說支援 ARM，我大概是第一個真的去編譯的人",
// second postscript: 128-element groups; technical report section 2.2.2: 2-bit
// codes). Byte b of group g holds the codes of elements 32s + b, s = 0..3, at
// bits 2s..2s+1; code = w + 1.
extern "C" bt_status bt_pack_ternary(const int8_t* w, int64_t N, int64_t K, uint8_t* packed) {
    if (!w || !packed) return BT_ERR_NULL;
    if (!valid_nk(N, K)) return BT_ERR_SHAPE;
    const size_t total = size_t(N) * size_t(K);
    uint8_t bad = 0;
    for (size_t i = 0; i < total; ++i) bad |= uint8_t(uint8_t(w[i] + 1) > 2);
    if (bad) return BT_ERR_VALUE;
    const int64_t groups = K / BT_GROUP_K;
    for (int64_t n = 0; n < N; ++n) {
        const int8_t* row = w + n * K;
        uint8_t* out = packed + n * (K / 4);
        for (int64_t g = 0; g < groups; ++g) {
            const int8_t* src = row + g * BT_GROUP_K;
            for (int b = 0; b < 32; ++b) {
                out[g * 32 + b] = uint8_t((src[b] + 1) | ((src[32 + b] + 1) << 2) |
                                          ((src[64 + b] + 1) << 4) | ((src[96 + b] + 1) << 6));
            }
        }
    }
    return BT_OK;
}

extern "C" bt_status bt_unpack_ternary(const uint8_t* packed, int64_t N, int64_t K, int8_t* w) {
    if (!w || !packed) return BT_ERR_NULL;
    if (!valid_nk(N, K)) return BT_ERR_SHAPE;
    const size_t bytes = size_t(N) * size_t(K) / 4;
    for (size_t i = 0; i < bytes; ++i) {
        const uint8_t v = packed[i];
        // a pair equal to 0b11 has both of its bits set
        if ((v & (v >> 1) & 0x55u) != 0) return BT_ERR_VALUE;
    }
    const int64_t groups = K / BT_GROUP_K;
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t* in = packed + n * (K / 4);
        int8_t* row = w + n * K;
        for (int64_t g = 0; g < groups; ++g) {
            for (int s = 0; s < 4; ++s)
                for (int b = 0; b < 32; ++b)
                    row[g * BT_GROUP_K + 32 * s + b] = int8_t(((in[g * 32 + b] >> (2 * s)) & 3) - 1);
        }
    }
    return BT_OK;
}

namespace bt {

// Work split of a GEMV. Each wave streams tiles_per_wave 16-row tiles over one
// K chunk; a workgroup (4 waves) first stages its chunk of the M activation
// rows (and a zero row) in LDS, so a chunk is at most
// kGemvLdsBytes / (256 (M + 1)) steps; K is split only for that. (Splitting
// K further for parallelism was measured to lose: the cross-workgroup
// synchronization it needs costs more than the extra workgroups gain.)
void gemv_shape(int64_t M, int64_t N, int64_t K, bool grouped, bool split_rows, GemvDesc* d) {
    memset(d, 0, sizeof(*d));
    d->M = int32_t(M);
    d->N = int32_t(N);
    d->K = int32_t(K);
    d->tiles = int32_t(ceil_div(N, kTileN));
    d->steps = int32_t(ceil_div(K, kSuperK));
    d->tiles_per_wave = grouped ? kGemvGroupedTilesPerWave : 1;
    // M activation rows plus one zero row per chunk
    const int64_t lds_steps = std::max<int64_t>(1, kGemvLdsBytes / ((M + 1) * kSuperK));
    int64_t chunks = ceil_div(d->steps, lds_steps);
    const int64_t spc = ceil_div(d->steps, chunks);
    chunks = ceil_div(d->steps, spc);
    d->chunks = int32_t(chunks);
    d->steps_per_chunk = int32_t(spc);
    d->lds_row = int32_t(spc * kSuperK + 16);
    // A single call with few tiles leaves most compute units idle and each wave
    // streaming a long K range: split every tile's K range over 2 or 4 waves of
    // its workgroup instead (partial sums meet in LDS), while each wave keeps
    // at least one 256-element step.
    d->waves_per_tile = 1;
    if (!grouped) {
        while (d->waves_per_tile < kGemvWaves && d->tiles * d->waves_per_tile < kGemvFillWaves &&
               spc >= 2 * d->waves_per_tile)
            d->waves_per_tile *= 2;
    }
    d->groups = ceil_div(d->tiles, int64_t(kGemvWaves / d->waves_per_tile) * d->tiles_per_wave);
    // A single call on quantized rows that still has few workgroups (one per
    // tile of down, o or qkv at M = 1): split each tile's 16 weight rows over 2
    // workgroups. Each loads only its rows' bytes, so the weights stream
    // through twice as many compute units, and each stores only its rows, so
    // nothing has to be combined across workgroups (down at M = 1: 5.40 ->
    // 5.24 us, qkv 4.17 -> 3.89 us). Fused calls keep whole tiles: there each
    // extra workgroup would quantize the token rows once more, and the
    // measured chain of fused calls did not gain.
    d->row_parts = 1;
    if (!grouped && split_rows) {
        while (d->row_parts < kGemvRowPartsMax && d->groups * chunks * d->row_parts * 2 <= kGemvFillBlocks)
            d->row_parts *= 2;
    }
    d->groups *= d->row_parts;
    d->blocks = d->groups * chunks;
}

size_t gemv_partial_bytes(const GemvDesc& d) {
    return (size_t(d.M) * size_t(d.tiles) * kTileN * sizeof(int32_t) + 255) & ~size_t(255);
}

size_t gemv_single_workspace_bytes(const GemvDesc& d) {
    if (d.chunks <= 1) return 0;
    return gemm_slice_bytes(d.M, d.N) * size_t(d.chunks) +
           ((size_t(d.M) * 8 + 255) & ~size_t(255));
}

size_t gemv_workspace_bytes(const GemvDesc& d) {
    if (d.chunks <= 1) return 0;
    return gemv_partial_bytes(d) + ((size_t(d.tiles) * sizeof(uint32_t) + 255) & ~size_t(255));
}

GemmChoice gemm_choice(int64_t M, int64_t N, int64_t K, bool int8_weights, bool persistent_ok) {
    GemmChoice c{1, 1, 0, 0};
    // int8 weights of at most 64 KB with K <= 512: held whole in LDS, tokens streamed
    if (int8_weights && K <= 512 && ceil_div(N, kTileN) * i8_stream_steps(K) <= 64 &&
        M * K < (int64_t(1) << 31)) {
        c.kind = 4;
        c.tiles = ceil_div(M, 16);
        return c;
    }
    const int64_t wide = ceil_div(M, 128) * ceil_div(N, 256);
    if (wide >= kGemmSlots) {
        c.kind = persistent_ok && !int8_weights ? 0 : 1;
        c.tiles = wide;
        return c;
    }
    // The tile shape with the least estimated time: the rounds of the resident
    // workgroup slots its tiles need (a last round, or a whole launch, of at
    // most one workgroup per compute unit takes about two thirds of the time
    // of one with two), times the tile's area over its measured relative
    // efficiency (64 x 64: 0.6, 128 x 96: 0.89, 128 x 128: 1; int8 weights have
    // no 128 x 96 kernel). Measured at M = 150 ... 6144 on the decoder's and
    // the tokenizer's shapes, it picks the fastest shape, or one within 5% of
    // it, in every case.
    struct Cand { int kind; int64_t bm, bn; double eff; };
    const Cand cands[3] = {{2, 128, 128, 1.0}, {5, 128, 96, 0.89}, {3, 64, 64, 0.6}};
    double best = 0.0;
    for (const Cand& k : cands) {
        if (int8_weights && k.kind == 5) continue;
        const int64_t t = ceil_div(M, k.bm) * ceil_div(N, k.bn);
        const int64_t full = t / kGemmSlots, rem = t % kGemmSlots;
        const double rounds =
            double(full) + (rem == 0 ? 0.0 : rem <= kGemmSlots / 2 ? 0.66 : 1.0);
        const double est = rounds * double(k.bm * k.bn) / k.eff;
        if (c.tiles == 0 || est < best) {
            best = est;
            c.kind = k.kind;
            c.tiles = t;
        }
    }
    // Fewer tiles than compute units: split K into ranges that fill the
    // compute units about once more, of at most 16 stages each where K is
    // long, within one round of slots. The ranges' slices cost (splits + 1)
    // M x N int32 of traffic, so the split is taken for a small output or a
    // long K only. Measured: 12-30% faster at M = 150 ... 512 with K = 8192,
    // 8960; a split of a 6000 x 512 output over K = 2048 was 30% slower.
    const int64_t nst = ceil_div(K, int8_weights ? 128 : 256);
    int64_t splits = 1;
    if (c.tiles < kGemmSlots / 2 && nst >= 8) {
        int64_t s = std::max({int64_t(2), ceil_div(192, c.tiles), ceil_div(nst, 16)});
        s = std::min({s, int64_t(kGemmSlots) / c.tiles, nst / 4});
        if (s >= 2 && (M * N <= (int64_t(1) << 20) || K >= 1000 * (s + 1))) splits = s;
    }
    const int64_t sps = ceil_div(nst, std::max<int64_t>(splits, 1));
    c.sps = int(sps);
    c.splits = int(ceil_div(nst, sps));
    return c;
}

size_t gemm_workspace_bytes(const GemmChoice& c, int64_t M, int64_t N) {
    if (c.splits <= 1) return 0;
    return gemm_slice_bytes(M, N) * size_t(c.splits);
}

}  // namespace bt

extern "C" size_t bt_matmul_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || !valid_nk(N, K)) return 0;
    if (M > BT_GEMV_MAX_M)
        return bt::gemm_workspace_bytes(bt::gemm_choice(M, N, K, false, true), M, N);
    bt::GemvDesc d;
    bt::gemv_shape(M, N, K, false, true, &d);
    return bt::gemv_single_workspace_bytes(d);
}

extern "C" size_t bt_int8_matmul_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || bt_int8_repacked_bytes(N, K) == 0) return 0;
    return bt::gemm_workspace_bytes(bt::gemm_choice(M, N, K, true, false), M, N);
}

// ------------------------------------------------------------------ plans

extern "C" size_t bt_int8_repacked_bytes(int64_t N, int64_t K) {
    // K % 32 == 0 (whole 16-byte fragments, the report's 32-element I8_S
    // blocks) and 127 * 128 * K < 2^31
    if (N < 1 || K < 32 || K % 32 != 0 || K > 131072 || N > (int64_t(1) << 31) - 16)
        return 0;
    return size_t(bt::ceil_div(N, bt::kTileN) * bt::kTileN) * size_t(bt::ceil_div(K, bt::kSuperK) * bt::kSuperK);
}

extern "C" size_t bt_repack_plan_bytes(int32_t count) {
    if (count < 1) return 0;
    return sizeof(bt::PlanHeader) + size_t(count) * sizeof(bt::RepackDesc);
}

extern "C" bt_status bt_repack_plan_build(const bt_repack_desc* descs, int32_t count,
                                          void* plan_host, size_t plan_bytes) {
    if (!descs || !plan_host) return BT_ERR_NULL;
    if (count < 1) return BT_ERR_SHAPE;
    if (plan_bytes < bt_repack_plan_bytes(count)) return BT_ERR_WORKSPACE;
    for (int32_t i = 0; i < count; ++i) {
        const bt_repack_desc& r = descs[i];
        if (!r.packed_dev || !r.wdev) return BT_ERR_NULL;
        if (!valid_nk(r.N, r.K)) return BT_ERR_SHAPE;
        if (!bt::aligned16(r.packed_dev) || !bt::aligned16(r.wdev)) return BT_ERR_ALIGN;
    }
    auto* hdr = static_cast<bt::PlanHeader*>(plan_host);
    auto* out = reinterpret_cast<bt::RepackDesc*>(hdr + 1);
    int64_t blocks = 0;
    for (int32_t i = 0; i < count; ++i) {
        const bt_repack_desc& r = descs[i];
        const int64_t steps = bt::ceil_div(r.K, bt::kSuperK);
        const int64_t nb = bt::ceil_div(r.N, bt::kTileN) * steps;
        out[i] = bt::RepackDesc{r.packed_dev, static_cast<uint8_t*>(r.wdev), int32_t(r.N),
                                int32_t(r.K), int32_t(steps), 0, blocks, nb};
        blocks += nb;
    }
    hdr->magic = bt::kPlanMagicRepack;
    hdr->count = count;
    hdr->total_blocks = blocks;
    return BT_OK;
}

extern "C" size_t bt_quant_plan_bytes(int32_t count) {
    if (count < 1) return 0;
    return sizeof(bt::PlanHeader) + size_t(count) * sizeof(bt::QuantDesc);
}

extern "C" bt_status bt_quant_plan_build(const bt_quant_desc* descs, int32_t count,
                                         void* plan_host, size_t plan_bytes) {
    if (!descs || !plan_host) return BT_ERR_NULL;
    if (count < 1) return BT_ERR_SHAPE;
    if (plan_bytes < bt_quant_plan_bytes(count)) return BT_ERR_WORKSPACE;
    // everything is checked, the grid size included, before the plan is written
    auto quant_blocks = [](const bt_quant_desc& q) {
        return bt::quant_wave_rows(q.K) ? ceil_div(q.M, bt::kQuantThreads / 64) : q.M;
    };
    int64_t total = 0;
    for (int32_t i = 0; i < count; ++i) {
        const bt_quant_desc& q = descs[i];
        if (!q.x || !q.xq || !q.xscale || !q.xsum) return BT_ERR_NULL;
        if (q.M < 1 || q.K < 1 || q.K > (int64_t(1) << 30) || q.M > (int64_t(1) << 31))
            return BT_ERR_SHAPE;
        if (!bt::aligned16(q.x) || !bt::aligned16(q.xq) || !bt::aligned16(q.xscale) ||
            !bt::aligned16(q.xsum))
            return BT_ERR_ALIGN;
        total += quant_blocks(q);
    }
    if (total > (int64_t(1) << 31) - 1) return BT_ERR_SHAPE;
    auto* hdr = static_cast<bt::PlanHeader*>(plan_host);
    auto* out = reinterpret_cast<bt::QuantDesc*>(hdr + 1);
    int64_t blocks = 0;
    for (int32_t i = 0; i < count; ++i) {
        const bt_quant_desc& q = descs[i];
        out[i] = bt::QuantDesc{q.x, q.xq, q.xscale, q.xsum, q.M, q.K, blocks};
        blocks += quant_blocks(q);
    }
    hdr->magic = bt::kPlanMagicQuant;
    hdr->count = count;
    hdr->total_blocks = blocks;
    return BT_OK;
}

static_assert(sizeof(bt::GemmArgs) <= sizeof(bt::GemvDesc), "a plan entry holds either kind");

extern "C" size_t bt_matmul_plan_bytes(int32_t count) {
    if (count < 1) return 0;
    return sizeof(bt::PlanHeader) + size_t(count) * sizeof(bt::GemvDesc);
}

// A projection of a grouped GEMM plan (M > BT_GEMV_MAX_M): quantized inputs
// only (quantization is not fused into the GEMM).
static bt_status check_gemm_desc(const bt_matmul_desc& m) {
    if (!m.wdev || !m.y || !m.xq || !m.xscale || !m.xsum) return BT_ERR_NULL;
    if (m.M <= BT_GEMV_MAX_M || m.M > (int64_t(1) << 31) - 1 || !valid_nk(m.N, m.K))
        return BT_ERR_SHAPE;
    if (!bt::aligned16(m.xq) || !bt::aligned16(m.xscale) || !bt::aligned16(m.xsum) ||
        !bt::aligned16(m.wdev) || !bt::aligned16(m.y) || (m.acc && !bt::aligned16(m.acc)))
        return BT_ERR_ALIGN;
    if (m.x) return BT_ERR_VALUE;
    if (!std::isfinite(m.w_scale)) return BT_ERR_VALUE;
    // output tiles and this projection's workgroups must fit the kernel's int32 indexes
    const int64_t tiles = ceil_div(m.M, bt::kPersistBM) * ceil_div(m.N, bt::kPersistBN);
    if (tiles > (int64_t(1) << 31) - 1) return BT_ERR_SHAPE;
    return BT_OK;
}

// K ranges of a projection in a grouped GEMM plan: 1, unless it has fewer
// output tiles than a quarter of the resident workgroup slots and a K of at
// least two ranges of kPlanSplitStages 128-element pieces; then ranges of at
// most about that many pieces (an even number: a range starts on a 1 KB weight
// step), at most one range-tile per compute unit. A plan's other projections
// at K = 1536 have 12 pieces per tile, so a range of a split projection takes
// about as long as one of their tiles (one layer at M = 512: down's 24 tiles of
// 70 pieces become 5 ranges of 14 pieces over the same 24 tiles).
struct PlanSplit { int64_t splits, sps; };
static PlanSplit gemm_plan_split(const bt_matmul_desc& m) {
    const int64_t tiles = ceil_div(m.M, bt::kPersistBM) * ceil_div(m.N, bt::kPersistBN);
    const int64_t nst = ceil_div(m.K, 128);
    if (tiles >= bt::kGemmSlots / 4 || nst < 2 * bt::kPlanSplitStages) return {1, nst};
    const int64_t s = std::max<int64_t>(
        2, std::min<int64_t>(ceil_div(nst, bt::kPlanSplitStages), (bt::kGemmSlots / 2) / tiles));
    const int64_t sps = (ceil_div(nst, s) + 1) & ~int64_t(1);
    return {ceil_div(nst, sps), sps};
}

// Workgroup slots per XCD a projection of a grouped GEMM plan takes: as many as
// its single launch would use (the resident slots of an XCD, or fewer when it
// has fewer tiles there), for each of its K ranges.
static int64_t gemm_plan_range_slots(const bt_matmul_desc& m) {
    const int64_t tiles = ceil_div(m.M, bt::kPersistBM) * ceil_div(m.N, bt::kPersistBN);
    return std::min<int64_t>(bt::kSlotsPerXcd, ceil_div(tiles, bt::kXcds));
}
static int64_t gemm_plan_slots(const bt_matmul_desc& m) {
    return gemm_plan_range_slots(m) * gemm_plan_split(m).splits;
}

// Workspace of a grouped GEMM plan's projection split along K: one M x N int32
// slice of partial sums per K range, then M int32 zeros (the ranges' row sums).
static size_t gemm_plan_ws_bytes(const bt_matmul_desc& m) {
    const PlanSplit sp = gemm_plan_split(m);
    if (sp.splits <= 1) return 0;
    return bt::gemm_slice_bytes(m.M, m.N) * size_t(sp.splits) + bt::gemm_slice_bytes(m.M, 1);
}

// Grouped GEMM plan: every projection runs the persistent GEMM's walk over its
// own 128 x 256 output tiles with as many workgroups per XCD as its single
// launch would use (the 64 resident slots of an XCD, or fewer when it has
// fewer tiles there), one projection after another in the grid: the
// dispatcher starts a projection's workgroups as the previous one's finish,
// so the XCDs' resident workgroups mostly share one projection's activation
// rows in their L2, and no launch ends in a tail. Projections with the same K
// run back to back, the longest K first (stable sort), so the longest walks
// (e.g. down's K ranges) are not left for the end of the grid. Measured on
// MI355X, long prefill M=4096 (28 layers x 4 projections, separate
// activations): 5.23 ms per stack as 112 single launches, 4.60 ms grouped in
// decoder order, 4.43 ms grouped by K (longest K first or last: the same);
// one layer at M=512 (down split into 5 K ranges): longest K first 41.0-42.7
// us against 42.8-44.0 us last;
// slots shared out in proportion to work, with every projection resident at
// once, took 5.46 ms (the activation rows of many projections thrash the L2).
// A projection split along K (gemm_plan_split) takes its slots once per K
// range, ranges one after another; its workspace slices and zeros are carved
// from the plan's workspace in descriptor order.
static bt_status build_gemm_plan(const bt_matmul_desc* descs, int32_t count, void* workspace,
                                 void* plan_host) {
    // descriptors already checked (check_gemm_desc), total slots within range,
    // workspace large enough
    auto* hdr = static_cast<bt::PlanHeader*>(plan_host);
    auto* out = reinterpret_cast<bt::GemmArgs*>(hdr + 1);
    char* ws = static_cast<char*>(workspace);
    for (int32_t i = 0; i < count; ++i) {
        const bt_matmul_desc& m = descs[i];
        bt::GemmArgs g;
        memset(&g, 0, sizeof(g));
        g.xq = m.xq;
        g.xscale = m.xscale;
        g.xsum = m.xsum;
        g.w = static_cast<const uint8_t*>(m.wdev);
        g.y = m.y;
        g.acc = m.acc;
        g.w_scale = m.w_scale;
        g.M = int32_t(m.M);
        g.N = int32_t(m.N);
        g.K = int32_t(m.K);
        g.tiles = int32_t(ceil_div(m.N, bt::kTileN));
        g.steps = int32_t(ceil_div(m.K, bt::kSuperK));
        g.m_tiles = int32_t(ceil_div(m.M, bt::kPersistBM));
        g.n_tiles = int32_t(ceil_div(m.N, bt::kPersistBN));
        const int64_t tiles = int64_t(g.m_tiles) * g.n_tiles;
        g.per_xcd = int32_t(ceil_div(tiles, bt::kXcds));
        g.group_m = bt::gemm_group_m(g.m_tiles, g.n_tiles, g.per_xcd);
        const PlanSplit sp = gemm_plan_split(m);
        g.splits = int32_t(sp.splits);
        g.sps = int32_t(sp.sps);
        if (sp.splits > 1) {
            g.ws = reinterpret_cast<int32_t*>(ws);
            g.ws_slice = int64_t(bt::gemm_slice_bytes(m.M, m.N) / sizeof(int32_t));
            ws += gemm_plan_ws_bytes(m);
        }
        g.slots = int32_t(gemm_plan_range_slots(m));   // per K range
        out[i] = g;
    }
    std::stable_sort(out, out + count,
                     [](const bt::GemmArgs& a, const bt::GemmArgs& b) { return a.K > b.K; });
    int64_t slot = 0;
    for (int32_t i = 0; i < count; ++i) {
        out[i].slot_begin = int32_t(slot);
        slot += int64_t(out[i].slots) * out[i].splits;
    }
    hdr->magic = bt::kPlanMagicGemm;
    hdr->count = count;
    hdr->total_blocks = slot;   // slots per XCD; the grid is 8 x this
    return BT_OK;
}

static bt_status check_matmul_desc(const bt_matmul_desc& m, bool fused) {
    if (!m.wdev || !m.y) return BT_ERR_NULL;
    if (fused ? !m.x : (!m.xq || !m.xscale || !m.xsum)) return BT_ERR_NULL;
    if (m.M < 1 || m.M > BT_GEMV_MAX_M || !valid_nk(m.N, m.K)) return BT_ERR_SHAPE;
    if ((m.xq && !bt::aligned16(m.xq)) || (m.xscale && !bt::aligned16(m.xscale)) ||
        (m.xsum && !bt::aligned16(m.xsum)) || (m.x && !bt::aligned16(m.x)) ||
        !bt::aligned16(m.wdev) || !bt::aligned16(m.y) || (m.acc && !bt::aligned16(m.acc)))
        return BT_ERR_ALIGN;
    if (!std::isfinite(m.w_scale)) return BT_ERR_VALUE;
    return BT_OK;
}

extern "C" size_t bt_matmul_plan_workspace_bytes(const bt_matmul_desc* descs, int32_t count) {
    if (!descs || count < 1) return 0;
    size_t total = 0;
    if (descs[0].M > BT_GEMV_MAX_M) {
        for (int32_t i = 0; i < count; ++i) {
            if (check_gemm_desc(descs[i]) != BT_OK) return 0;
            total += gemm_plan_ws_bytes(descs[i]);
        }
        return total;
    }
    for (int32_t i = 0; i < count; ++i) {
        if (descs[i].M < 1 || descs[i].M > BT_GEMV_MAX_M || !valid_nk(descs[i].N, descs[i].K))
            return 0;
        bt::GemvDesc d;
        bt::gemv_shape(descs[i].M, descs[i].N, descs[i].K, true, false, &d);
        total += bt::gemv_workspace_bytes(d);
    }
    return total;
}

extern "C" bt_status bt_matmul_plan_build(const bt_matmul_desc* descs, int32_t count,
                                          void* workspace, size_t workspace_bytes,
                                          void* plan_host, size_t plan_bytes) {
    if (!descs || !plan_host) return BT_ERR_NULL;
    if (count < 1) return BT_ERR_SHAPE;
    if (plan_bytes < bt_matmul_plan_bytes(count)) return BT_ERR_WORKSPACE;
    if (descs[0].M > BT_GEMV_MAX_M) {
        // a GEMM plan: every projection has M > BT_GEMV_MAX_M; everything is
        // checked before the plan is written
        int64_t slots = 0;
        for (int32_t i = 0; i < count; ++i) {
            const bt_status st = check_gemm_desc(descs[i]);
            if (st != BT_OK) return st;
            slots += gemm_plan_slots(descs[i]);
        }
        if (slots * bt::kXcds > (int64_t(1) << 31) - 1) return BT_ERR_SHAPE;
        const size_t need = bt_matmul_plan_workspace_bytes(descs, count);
        if (need) {
            if (!workspace || workspace_bytes < need) return BT_ERR_WORKSPACE;
            if (!bt::aligned16(workspace)) return BT_ERR_ALIGN;
        }
        return build_gemm_plan(descs, count, workspace, plan_host);
    }
    const bool fused = descs[0].x != nullptr;
    for (int32_t i = 0; i < count; ++i) {
        if ((descs[i].x != nullptr) != fused) return BT_ERR_VALUE;   // all fused or none
        const bt_status st = check_matmul_desc(descs[i], fused);
        if (st != BT_OK) return st;
    }
    const size_t need = bt_matmul_plan_workspace_bytes(descs, count);
    if (need) {
        if (!workspace || workspace_bytes < need) return BT_ERR_WORKSPACE;
        if (!bt::aligned16(workspace)) return BT_ERR_ALIGN;
    }
    int64_t total_blocks = 0;
    for (int32_t i = 0; i < count; ++i) {
        bt::GemvDesc d;
        bt::gemv_shape(descs[i].M, descs[i].N, descs[i].K, true, false, &d);
        total_blocks += d.blocks;
    }
    if (total_blocks > int64_t(1) << 31) return BT_ERR_SHAPE;   // nothing written yet
    auto* hdr = static_cast<bt::PlanHeader*>(plan_host);
    auto* out = reinterpret_cast<bt::GemvDesc*>(hdr + 1);
    char* ws = static_cast<char*>(workspace);
    for (int32_t i = 0; i < count; ++i) {
        const bt_matmul_desc& m = descs[i];
        bt::GemvDesc d;
        bt::gemv_shape(m.M, m.N, m.K, true, false, &d);
        d.x = m.x;
        d.xq = const_cast<int8_t*>(m.xq);
        d.xscale = const_cast<float*>(m.xscale);
        d.xsum = const_cast<int32_t*>(m.xsum);
        d.w = static_cast<const uint8_t*>(m.wdev);
        d.y = m.y;
        d.acc = m.acc;
        d.w_scale = m.w_scale;
        if (d.chunks > 1) {
            d.ws = reinterpret_cast<int32_t*>(ws);
            d.cnt = reinterpret_cast<uint32_t*>(ws + bt::gemv_partial_bytes(d));
            ws += bt::gemv_workspace_bytes(d);
        }
        out[i] = d;
    }
    // Longest workgroups first: the grid drains in dispatch order, so the
    // long-K projections (e.g. down, 8960 wide) must not be the tail.
    std::stable_sort(out, out + count, [](const bt::GemvDesc& a, const bt::GemvDesc& b) {
        return int64_t(a.steps_per_chunk) * a.tiles_per_wave >
               int64_t(b.steps_per_chunk) * b.tiles_per_wave;
    });
    int64_t blocks = 0;
    for (int32_t i = 0; i < count; ++i) {
        out[i].block_begin = blocks;
        blocks += out[i].blocks;
    }
    hdr->magic = fused ? bt::kPlanMagicGemvFused : bt::kPlanMagicGemv;
    hdr->count = count;
    hdr->total_blocks = blocks;
    return BT_OK;
}
