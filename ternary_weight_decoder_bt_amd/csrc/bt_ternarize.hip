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
// 32-bit word (16 codes) per 4 x 16-byte loads.

#include <hip/hip_runtime.h>

#include <math.h>

#include <algorithm>

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

__global__ __launch_bounds__(kThreads) void absmean_partial_kernel(const v4f* __restrict__ w,
                                                                   int64_t nvec,
                                                                   double* __restrict__ partials) {
    __shared__ double red[kThreads / 64];
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    double s = 0.0;
    int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    for (; i + (kUnroll - 1) * stride < nvec; i += kUnroll * stride) {
        v4f v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(w + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) s += abs_sum4(v[u]);
    }
    for (; i < nvec; i += stride) s += abs_sum4(__builtin_nontemporal_load(w + i));
    s = block_sum(s, red);
    if (threadIdx.x == 0) partials[blockIdx.x] = s;
}

// Packed field of one weight: code w + 1 of its ternary value.
__device__ __forceinline__ uint32_t code_of(float w, float delta) {
    const float t = w / delta;                     // IEEE division (correctly rounded)
    return fabsf(t) >= 0.5f ? (t > 0.0f ? 2u : 0u) : 1u;
}

// Word j of the packed tensor: bytes 4c .. 4c+3 of 128-element group g of row n
// (c = j mod 8). Byte b of a group holds elements 128g + 32s + b at bits 2s.
__global__ __launch_bounds__(kThreads) void ternarize_pack_kernel(
    const float* __restrict__ w, int64_t N, int64_t K, float eps,
    const double* __restrict__ partials, int32_t nparts, uint32_t* __restrict__ packed,
    float* __restrict__ scale) {
    __shared__ double red[kThreads / 64];
    double s = 0.0;
    for (int p = threadIdx.x; p < nparts; p += kThreads) s += partials[p];
    s = block_sum(s, red);
    const float gamma = float(s / double(N * K));
    const float delta = gamma + eps;
    if (blockIdx.x == 0 && threadIdx.x == 0) *scale = gamma;

    const int64_t words_per_row = K / 16;
    const int64_t words = N * words_per_row;
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    for (int64_t j = int64_t(blockIdx.x) * kThreads + threadIdx.x; j < words; j += stride) {
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

extern "C" bt_status bt_ternarize(const float* w, int64_t N, int64_t K, float eps,
                                  uint8_t* packed, float* scale, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
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
    const int32_t nparts = partial_blocks(N, K);
    const int64_t words = int64_t(pbytes / 4);
    const unsigned pack_blocks =
        unsigned(std::min<int64_t>(kPackBlocks, bt::ceil_div(words, kThreads)));
    auto* partials = static_cast<double*>(workspace);
    (void)hipGetLastError();
    hipLaunchKernelGGL(absmean_partial_kernel, dim3(unsigned(nparts)), dim3(kThreads), 0, stream,
                       reinterpret_cast<const v4f*>(w), int64_t(N) * K / 4, partials);
    hipLaunchKernelGGL(ternarize_pack_kernel, dim3(pack_blocks), dim3(kThreads), 0, stream, w, N,
                       K, eps, partials, nparts, reinterpret_cast<uint32_t*>(packed), scale);
    return hipGetLastError() == hipSuccess ? BT_OK : BT_ERR_DEVICE;
}
