// Offline ternarization of full-precision weights on the device: fp32 W ->
// canonical 2-bit codes + the per-tensor scale.
//
// "VibeVoice-ASR-BitNet Technical Report", section 2.2.2: the decoder's weights
// are quantized to ternary following the BitNet approach of its reference [11]
// ("The era of 1-bit LLMs"), whose absmean quantizer divides each weight by the
// tensor's mean |w| (plus eps), rounds to the nearest integer and clips to
// [-1, 1]. The scale gamma multiplies the codes back.
//
// Two launches, because every code depends on the mean over the whole tensor:
//   1. absmean_partial_kernel: each of B workgroups sums |w| over a fixed
//      strided share of the tensor in fp64 and writes one partial.
//   2. ternarize_pack_kernel: every workgroup adds the B partials in one fixed
//      order (so all of them, and every call, see the same S), forms
//      gamma = fl32(S / (N K)) and delta = fl32(gamma + eps), and codes and
//      packs its share of the tensor: round_half_away(w / delta) clipped to
//      [-1, 1] is +-1 exactly where |w / delta| >= 1/2.
// Both passes stream the fp32 tensor with 16-byte loads; the second writes one
// 32-bit word (16 codes) per 4 x 16-byte loads. A grouped plan runs the same two
// passes for many tensors, one launch per pass.

#include <hip/hip_runtime.h>

#include <math.h>

#include <algorithm>
#include <cstring>

#include "bt_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxPartials = 1024;      // B: workgroups of the first pass
constexpr int kPackBlocks = 2048;       // workgroups of the second pass (grid-stride)
constexpr int kUnroll = 4;              // 16-byte loads in flight per thread per iteration

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Sum of v over the workgroup in a fixed order (lanes, then waves).
__device__ __forceinline__ double block_sum(double v, double* red) {
    v = wave_sum(v);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) s += red[w];
    __syncthreads();
    return s;
}

__device__ __forceinline__ double abs_sum4(v4f v) {
    return (double(fabsf(v.x)) + double(fabsf(v.y))) + (double(fabsf(v.z)) + double(fabsf(v.w)));
}

// Partial sum `b` of the tensor's `nparts`: the 16-byte vectors b*256 + t +
// j*(nparts*256) for the workgroup's threads t, each in fp64, added in a fixed
// order (per thread, then lanes, then waves).
__device__ __forceinline__ void absmean_partial_body(const v4f* __restrict__ w, int64_t nvec,
                                                     int32_t b, int32_t nparts,
                                                     double* __restrict__ partials,
                                                     double* red) {
    const int64_t stride = int64_t(nparts) * kThreads;
    double s = 0.0;
    int64_t i = int64_t(b) * kThreads + threadIdx.x;
    for (; i + (kUnroll - 1) * stride < nvec; i += kUnroll * stride) {
        v4f v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(w + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) s += abs_sum4(v[u]);
    }
    for (; i < nvec; i += stride) s += abs_sum4(__builtin_nontemporal_load(w + i));
    s = block_sum(s, red);
    if (threadIdx.x == 0) partials[b] = s;
}

__global__ __launch_bounds__(kThreads) void absmean_partial_kernel(const v4f* __restrict__ w,
                                                                   int64_t nvec,
                                                                   double* __restrict__ partials) {
    __shared__ double red[kThreads / 64];
    absmean_partial_body(w, nvec, int32_t(blockIdx.x), int32_t(gridDim.x), partials, red);
}

// Packed field of one weight: code w + 1 of its ternary value.
__device__ __forceinline__ uint32_t code_of(float w, float delta) {
    const float t = w / delta;                     // IEEE division (correctly rounded)
    return fabsf(t) >= 0.5f ? (t > 0.0f ? 2u : 0u) : 1u;
}

// Word j of the packed tensor: bytes 4c .. 4c+3 of 128-element group g of row n
// (c = j mod 8). Byte b of a group holds elements 128g + 32s + b at bits 2s.
// Workgroup `b` of the `nblocks` that code and pack one tensor: every one adds
// the partial sums in the same order, so all see the same gamma.
__device__ __forceinline__ void ternarize_pack_body(const float* __restrict__ w, int64_t N,
                                                    int64_t K, float eps,
                                                    const double* __restrict__ partials,
                                                    int32_t nparts,
                                                    uint32_t* __restrict__ packed,
                                                    float* __restrict__ scale, int32_t b,
                                                    int32_t nblocks, double* red) {
    double s = 0.0;
    for (int p = threadIdx.x; p < nparts; p += kThreads) s += partials[p];
    s = block_sum(s, red);
    const float gamma = float(s / double(N * K));
    const float delta = gamma + eps;
    if (b == 0 && threadIdx.x == 0) *scale = gamma;

    const int64_t words_per_row = K / 16;
    const int64_t words = N * words_per_row;
    const int64_t stride = int64_t(nblocks) * kThreads;
    for (int64_t j = int64_t(b) * kThreads + threadIdx.x; j < words; j += stride) {
        const int64_t n = j / words_per_row;
        const int64_t wj = j - n * words_per_row;
        const float* src = w + n * K + (wj >> 3) * 128 + (wj & 7) * 4;
        v4f v[4];
#pragma unroll
        for (int p = 0; p < 4; ++p)
            v[p] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(src + 32 * p));
        uint32_t word = 0;
        if (delta != 0.0f) {   // delta == 0 only for an all-zero tensor: every code is 1
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                word |= code_of(v[p].x, delta) << (2 * p);
                word |= code_of(v[p].y, delta) << (8 + 2 * p);
                word |= code_of(v[p].z, delta) << (16 + 2 * p);
                word |= code_of(v[p].w, delta) << (24 + 2 * p);
            }
        } else {
            word = 0x55555555u;
        }
        packed[j] = word;
    }
}

__global__ __launch_bounds__(kThreads) void ternarize_pack_kernel(
    const float* __restrict__ w, int64_t N, int64_t K, float eps,
    const double* __restrict__ partials, int32_t nparts, uint32_t* __restrict__ packed,
    float* __restrict__ scale) {
    __shared__ double red[kThreads / 64];
    ternarize_pack_body(w, N, K, eps, partials, nparts, packed, scale, int32_t(blockIdx.x),
                        int32_t(gridDim.x), red);
}

// Many tensors per launch: the workgroup's tensor is the last whose first
// workgroup (part_begin, or pack_begin) is at or before it, found with one lane
// per descriptor and a ballot; then the single kernels' bodies with the
// tensor's own workgroup count, so every tensor gets the same partial sums,
// gamma and bytes as from bt_ternarize.
template <bool kPack>
__device__ __forceinline__ int tern_desc_of(const bt::TernDesc* __restrict__ descs,
                                            int32_t count, int64_t blk) {
    const int lane = threadIdx.x & 63;
    int p = -1;
    for (int base = 0; base < count; base += 64) {
        const int i = base + lane;
        const int64_t begin =
            i < count ? (kPack ? descs[i].pack_begin : descs[i].part_begin) : INT64_MAX;
        p += int(__popcll(__ballot(begin <= blk)));
    }
    return __builtin_amdgcn_readfirstlane(p);
}

__global__ __launch_bounds__(kThreads) void absmean_partial_grouped_kernel(
    const bt::TernDesc* __restrict__ descs, int32_t count) {
    __shared__ double red[kThreads / 64];
    const int64_t blk = blockIdx.x;
    const bt::TernDesc& d = descs[tern_desc_of<false>(descs, count, blk)];
    absmean_partial_body(reinterpret_cast<const v4f*>(d.w), d.N * d.K / 4,
                         int32_t(blk - d.part_begin), d.nparts, d.partials, red);
}

__global__ __launch_bounds__(kThreads) void ternarize_pack_grouped_kernel(
    const bt::TernDesc* __restrict__ descs, int32_t count) {
    __shared__ double red[kThreads / 64];
    const int64_t blk = blockIdx.x;
    const bt::TernDesc& d = descs[tern_desc_of<true>(descs, count, blk)];
    ternarize_pack_body(d.w, d.N, d.K, d.eps, d.partials, d.nparts,
                        reinterpret_cast<uint32_t*>(d.packed), d.scale,
                        int32_t(blk - d.pack_begin), d.pack_blocks, red);
}

int32_t partial_blocks(int64_t N, int64_t K) {
    const int64_t nvec = N * K / 4;
    return int32_t(std::min<int64_t>(kMaxPartials, bt::ceil_div(nvec, int64_t(kThreads) * 8)));
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + nb && pb < pa + na;
}

}  // namespace

extern "C" size_t bt_ternarize_workspace_bytes(int64_t N, int64_t K) {
    if (bt_packed_bytes(N, K) == 0) return 0;
    return (size_t(partial_blocks(N, K)) * sizeof(double) + 255) & ~size_t(255);
}

namespace {

// bt_ternarize's argument rules for one tensor with its workspace region.
bt_status check_ternarize(const float* w, int64_t N, int64_t K, float eps, const uint8_t* packed,
                          const float* scale, const void* workspace, size_t workspace_bytes) {
    if (!w || !packed || !scale) return BT_ERR_NULL;
    const size_t pbytes = bt_packed_bytes(N, K);
    if (pbytes == 0) return BT_ERR_SHAPE;
    if (!isfinite(eps) || eps < 0.0f) return BT_ERR_VALUE;
    if (!bt::aligned16(w) || !bt::aligned16(packed) || !bt::aligned16(scale) ||
        (workspace && !bt::aligned16(workspace)))
        return BT_ERR_ALIGN;
    const size_t need = bt_ternarize_workspace_bytes(N, K);
    if (!workspace || workspace_bytes < need) return BT_ERR_WORKSPACE;
    const size_t wbytes = size_t(N) * size_t(K) * sizeof(float);
    if (overlaps(w, wbytes, packed, pbytes) || overlaps(w, wbytes, workspace, need) ||
        overlaps(packed, pbytes, workspace, need) || overlaps(scale, 4, w, wbytes) ||
        overlaps(scale, 4, packed, pbytes) || overlaps(scale, 4, workspace, need))
        return BT_ERR_VALUE;
    return BT_OK;
}

unsigned pack_blocks_of(int64_t N, int64_t K) {
    const int64_t words = int64_t(bt_packed_bytes(N, K) / 4);
    return unsigned(std::min<int64_t>(kPackBlocks, bt::ceil_div(words, kThreads)));
}

}  // namespace

extern "C" bt_status bt_ternarize(const float* w, int64_t N, int64_t K, float eps,
                                  uint8_t* packed, float* scale, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    const bt_status st = check_ternarize(w, N, K, eps, packed, scale, workspace, workspace_bytes);
    if (st != BT_OK) return st;
    const int32_t nparts = partial_blocks(N, K);
    const unsigned pack_blocks = pack_blocks_of(N, K);
    auto* partials = static_cast<double*>(workspace);
    (void)hipGetLastError();
    hipLaunchKernelGGL(absmean_partial_kernel, dim3(unsigned(nparts)), dim3(kThreads), 0, stream,
                       reinterpret_cast<const v4f*>(w), int64_t(N) * K / 4, partials);
    hipLaunchKernelGGL(ternarize_pack_kernel, dim3(pack_blocks), dim3(kThreads), 0, stream, w, N,
                       K, eps, partials, nparts, reinterpret_cast<uint32_t*>(packed), scale);
    return hipGetLastError() == hipSuccess ? BT_OK : BT_ERR_DEVICE;
}

// ------------------------------------------------------------ grouped plans

extern "C" size_t bt_ternarize_plan_bytes(int32_t count) {
    if (count < 1) return 0;
    return sizeof(bt::PlanHeader) + size_t(count) * sizeof(bt::TernDesc);
}

extern "C" size_t bt_ternarize_plan_workspace_bytes(const bt_ternarize_desc* descs,
                                                    int32_t count) {
    if (!descs || count < 1) return 0;
    size_t total = 0;
    for (int32_t i = 0; i < count; ++i) {
        const size_t b = bt_ternarize_workspace_bytes(descs[i].N, descs[i].K);
        if (b == 0) return 0;
        total += b;
    }
    return total;
}

extern "C" bt_status bt_ternarize_plan_build(const bt_ternarize_desc* descs, int32_t count,
                                             void* workspace, size_t workspace_bytes,
                                             void* plan_host, size_t plan_bytes) {
    if (!descs || !plan_host) return BT_ERR_NULL;
    if (count < 1) return BT_ERR_SHAPE;
    if (plan_bytes < bt_ternarize_plan_bytes(count)) return BT_ERR_WORKSPACE;
    for (int32_t i = 0; i < count; ++i)
        if (bt_packed_bytes(descs[i].N, descs[i].K) == 0) return BT_ERR_SHAPE;
    const size_t need = bt_ternarize_plan_workspace_bytes(descs, count);
    if (!workspace || workspace_bytes < need) return BT_ERR_WORKSPACE;
    // every tensor by bt_ternarize's rules, with its own slice of the workspace
    char* ws = static_cast<char*>(workspace);
    for (int32_t i = 0; i < count; ++i) {
        const bt_ternarize_desc& d = descs[i];
        const size_t b = bt_ternarize_workspace_bytes(d.N, d.K);
        const bt_status st = check_ternarize(d.w, d.N, d.K, d.eps, d.packed, d.scale, ws, b);
        if (st != BT_OK) return st;
        ws += b;
    }
    // no tensor's outputs may meet another tensor's input or outputs, and the
    // workspace meets no tensor's buffers
    for (int32_t i = 0; i < count; ++i) {
        const bt_ternarize_desc& a = descs[i];
        const size_t pa = bt_packed_bytes(a.N, a.K);
        const size_t wa = size_t(a.N) * size_t(a.K) * sizeof(float);
        if (overlaps(workspace, need, a.w, wa) || overlaps(workspace, need, a.packed, pa) ||
            overlaps(workspace, need, a.scale, 4))
            return BT_ERR_VALUE;
        for (int32_t j = 0; j < count; ++j) {
            if (i == j) continue;
            const bt_ternarize_desc& b = descs[j];
            const size_t pb = bt_packed_bytes(b.N, b.K);
            const size_t wb = size_t(b.N) * size_t(b.K) * sizeof(float);
            if (overlaps(a.packed, pa, b.w, wb) || overlaps(a.packed, pa, b.packed, pb) ||
                overlaps(a.packed, pa, b.scale, 4) || overlaps(a.scale, 4, b.w, wb) ||
                overlaps(a.scale, 4, b.scale, 4))
                return BT_ERR_VALUE;
        }
    }
    int64_t parts = 0, packs = 0;
    for (int32_t i = 0; i < count; ++i) {
        parts += partial_blocks(descs[i].N, descs[i].K);
        packs += pack_blocks_of(descs[i].N, descs[i].K);
    }
    if (parts > (int64_t(1) << 31) - 1 || packs > (int64_t(1) << 31) - 1) return BT_ERR_SHAPE;
    // checked: write the plan
    auto* hdr = static_cast<bt::PlanHeader*>(plan_host);
    auto* out = reinterpret_cast<bt::TernDesc*>(hdr + 1);
    ws = static_cast<char*>(workspace);
    parts = packs = 0;
    for (int32_t i = 0; i < count; ++i) {
        const bt_ternarize_desc& d = descs[i];
        bt::TernDesc t;
        memset(&t, 0, sizeof(t));
        t.w = d.w;
        t.packed = d.packed;
        t.scale = d.scale;
        t.partials = reinterpret_cast<double*>(ws);
        t.N = d.N;
        t.K = d.K;
        t.eps = d.eps;
        t.nparts = partial_blocks(d.N, d.K);
        t.pack_blocks = int32_t(pack_blocks_of(d.N, d.K));
        t.part_begin = parts;
        t.pack_begin = packs;
        parts += t.nparts;
        packs += t.pack_blocks;
        ws += bt_ternarize_workspace_bytes(d.N, d.K);
        out[i] = t;
    }
    hdr->magic = bt::kPlanMagicTern;
    hdr->count = count;
    hdr->total_blocks = parts;   // first launch; the second's is the last pack_begin + its blocks
    return BT_OK;
}

extern "C" bt_status bt_ternarize_grouped(const void* plan_host, const void* plan_dev,
                                          hipStream_t stream) {
    if (!plan_host || !plan_dev) return BT_ERR_NULL;
    const auto* hdr = static_cast<const bt::PlanHeader*>(plan_host);
    if (hdr->magic != bt::kPlanMagicTern || hdr->count < 1 || hdr->total_blocks < 1)
        return BT_ERR_VALUE;
    if (!bt::aligned16(plan_dev)) return BT_ERR_ALIGN;
    const auto* host = reinterpret_cast<const bt::TernDesc*>(hdr + 1);
    const bt::TernDesc& last = host[hdr->count - 1];
    const int64_t packs = last.pack_begin + last.pack_blocks;
    const auto* descs = reinterpret_cast<const bt::TernDesc*>(
        static_cast<const char*>(plan_dev) + sizeof(bt::PlanHeader));
    (void)hipGetLastError();
    hipLaunchKernelGGL(absmean_partial_grouped_kernel, dim3(unsigned(hdr->total_blocks)),
                       dim3(kThreads), 0, stream, descs, hdr->count);
    hipLaunchKernelGGL(ternarize_pack_grouped_kernel, dim3(unsigned(packs)), dim3(kThreads), 0,
                       stream, descs, hdr->count);
    return hipGetLastError() == hipSuccess ? BT_OK : BT_ERR_DEVICE;
}
