// Device half of libbt for gfx950 (CDNA4): weight repack, per-token INT8
// quantization, the decode GEMV (M <= 16) and the prefill GEMM (M > 16).
//
// Method ("VibeVoice-ASR-BitNet Technical Report", sections 2.2.2 and 2.4.2,
// Figure 4): ternary weights stored as 2-bit codes are unpacked to INT8 and
// multiplied with per-token INT8 activations; products are summed exactly in
// integers and then rescaled to fp32.
//
// How it maps to the matrix cores: every contraction here runs on
// v_mfma_i32_16x16x64_i8 (A = 16 tokens x 64 K of activations, B = 64 K x 16
// weight rows, C = 16 x 16 int32). Weights enter the MFMA as their codes
// c = w + 1 in {0, 1, 2}; since sum_k q*w = sum_k q*c - sum_k q, the epilogue
// subtracts the per-token sum of q. That keeps the unpack to one shift and one
// AND per 4 weights, with no per-byte subtraction.
//
// Repacked weight layout (written by repack_kernel, read by both matmuls):
//   K is padded to Kp = ceil(K/256)*256 and N to a multiple of 16 (padding
//   holds zero weights; the activation side is zero there too);
//   tile t = 16 consecutive rows, 4*Kp bytes, stored contiguously;
//   inside a tile, 256-wide K steps S of 1 KB: lane l (row 16t + l%16,
//   K quarter l/16) owns bytes [16l, 16l+16) = four 32-bit words, word jj
//   holding K = 256S + 64jj + 16(l/16) + e, e = 0..15, with element e in
//   byte e%4 at bits 2*(e/4). So one 128-bit load per lane yields the B
//   fragments of four MFMA steps, and unpacking word jj is
//   (word >> 2s) & 0x03030303 for s = 0..3.

#include <hip/hip_runtime.h>

#include <float.h>
#include <math.h>

#include <string.h>

#include <algorithm>
#include <type_traits>

#include "bt_internal.h"

#pragma clang fp contract(off)

namespace {

using bt::GemvDesc;
using bt::QuantDesc;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr uint32_t kLow2 = 0x03030303u;

__device__ __forceinline__ v4i unpack16(uint32_t p) {
    v4i b;
    b[0] = int(p & kLow2);
    b[1] = int((p >> 2) & kLow2);
    b[2] = int((p >> 4) & kLow2);
    b[3] = int((p >> 6) & kLow2);
    return b;
}

__device__ __forceinline__ v4i mfma16x16x64(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Pointers held in descriptors are generic; these casts make the compiler
// emit global_* / ds_* instructions instead of flat_* ones (flat accesses
// also count against the LDS wait counter and serialize the two queues).
#define BT_GLOBAL __attribute__((address_space(1)))
#define BT_LDS __attribute__((address_space(3)))

template <typename T>
__device__ __forceinline__ T gld(const void* p) {
    return *(const BT_GLOBAL T*)p;
}

// Streaming load for data read exactly once (the weights).
template <typename T>
__device__ __forceinline__ T gld_stream(const void* p) {
    return __builtin_nontemporal_load((const BT_GLOBAL T*)p);
}

template <typename T>
__device__ __forceinline__ void gst(void* p, T v) {
    *(BT_GLOBAL T*)p = v;
}

// Buffer resources (base and size in SGPRs): a load takes a per-lane VGPR
// offset plus a scalar offset, and any byte past the size reads as zero.
constexpr int kBufferFlags = 0x00020000;   // gfx9 buffer resource word 3

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), kBufferFlags);
}

__device__ __forceinline__ v4u buf_ld16u(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(r, int(voff), int(soff), 0));
}

template <typename T>
__device__ __forceinline__ T lds_ld(const void* p) {
    return *(const BT_LDS T*)p;
}

template <typename T>
__device__ __forceinline__ void lds_st(void* p, T v) {
    *(BT_LDS T*)p = v;
}

// ---------------------------------------------------------------- epilogue
//
// The fused epilogues of the technical report's section 2.4.1 on the fp32
// output y = fl32(fl32(acc) * fl32(d * s_w)): bias add, ReLU (a non-positive
// value becomes +0), layer scale, residual add; each one fp32 operation.

using bt::EpiArgs;

__host__ __device__ __forceinline__ bool epi_any(const EpiArgs& e) {
    return e.bias || e.gamma || e.res || e.relu;
}

// bias, ReLU and layer scale on one value of output column n
__device__ __forceinline__ float epi_col(const EpiArgs& e, float y, int64_t n) {
    if (e.bias) y = y + e.bias[n];
    if (e.relu) y = y > 0.0f ? y : 0.0f;
    if (e.gamma) y = e.gamma[n] * y;
    return y;
}

// the same on four consecutive columns n .. n+3 (n % 4 == 0, 16-byte loads)
__device__ __forceinline__ v4f epi_col4(const EpiArgs& e, v4f y, int64_t n) {
    if (e.bias) y = y + gld<v4f>(e.bias + n);
    if (e.relu) {
        y.x = y.x > 0.0f ? y.x : 0.0f;
        y.y = y.y > 0.0f ? y.y : 0.0f;
        y.z = y.z > 0.0f ? y.z : 0.0f;
        y.w = y.w > 0.0f ? y.w : 0.0f;
    }
    if (e.gamma) y = gld<v4f>(e.gamma + n) * y;
    return y;
}

// ------------------------------------------------------------------ repack

// One wave per 1 KB output block (16-row tile t, 256-wide step S); lane l
// writes its 16 bytes, the four words jj = 0..3 of row r = 16t + l%16 at
// K = 256S + 64jj + 16q + e (q = l/16, e = 0..15). In the canonical layout
// those 16 elements are the 16 consecutive bytes starting at byte
// 32(jj/2) + 16(q%2) of the row's 64-byte piece for step S, at bit pair
// 2(jj%2) + q/2. So a lane reads two 16-byte chunks of its row (jj = 0, 1
// share one, jj = 2, 3 the other) and the wave reads its 16 rows' pieces
// whole; padding rows and columns get code 1 (weight 0).
// The two canonical 16-byte chunks lane l needs for output block blk (zero
// where the block is padding; `valid` says which halves are real).
struct RepackIn {
    uint4 c[2];
    bool valid[2];
};

__device__ __forceinline__ RepackIn repack_load(const uint8_t* __restrict__ packed, int32_t N,
                                                int32_t K, int32_t steps, int64_t blk, int lane) {
    const int r = lane & 15;
    const int q = lane >> 4;
    const int64_t t = blk / steps;
    const int32_t S = int32_t(blk - t * steps);
    const int64_t n = t * bt::kTileN + r;
    RepackIn in;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t k0 = int64_t(bt::kSuperK) * S + 128 * h;   // group 2S + h
        in.valid[h] = n < N && k0 < K;
        in.c[h] = in.valid[h] ? *reinterpret_cast<const uint4*>(packed + n * (K / 4) + k0 / 4 +
                                                                16 * (q & 1))
                              : uint4{0, 0, 0, 0};
    }
    return in;
}

__device__ __forceinline__ void repack_store(const RepackIn& in, uint8_t* __restrict__ out,
                                             int64_t blk, int lane) {
    const int q = lane >> 4;
    uint32_t w[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint4 c = in.c[h];
#pragma unroll
        for (int jl = 0; jl < 2; ++jl) {
            const int sh = 2 * (2 * jl + (q >> 1));
            w[2 * h + jl] = in.valid[h] ? ((c.x >> sh) & kLow2) | (((c.y >> sh) & kLow2) << 2) |
                                              (((c.z >> sh) & kLow2) << 4) |
                                              (((c.w >> sh) & kLow2) << 6)
                                        : 0x55555555u;   // padding: code 1 = weight 0
        }
    }
    *reinterpret_cast<uint4*>(out + blk * 1024 + lane * 16) = uint4{w[0], w[1], w[2], w[3]};
}

#ifndef BT_REPACK_PER_WAVE
#define BT_REPACK_PER_WAVE 8
#endif
constexpr int kRepackPerWave = BT_REPACK_PER_WAVE;   // output blocks a wave handles per pass

__global__ __launch_bounds__(256) void repack_kernel(const uint8_t* __restrict__ packed, int32_t N,
                                                     int32_t K, int32_t steps, int64_t blocks,
                                                     uint8_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t waves = (int64_t(gridDim.x) * blockDim.x) >> 6;
    for (int64_t b0 = ((int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6) * kRepackPerWave;
         b0 < blocks; b0 += waves * kRepackPerWave) {
        RepackIn in[kRepackPerWave];
#pragma unroll
        for (int u = 0; u < kRepackPerWave; ++u)
            in[u] = repack_load(packed, N, K, steps, min(b0 + u, blocks - 1), lane);
#pragma unroll
        for (int u = 0; u < kRepackPerWave; ++u)
            if (b0 + u < blocks) repack_store(in[u], out, b0 + u, lane);
    }
}

// Many tensors in one launch: a wave takes runs of global output blocks and
// finds each block's tensor with one lane per descriptor (64 offsets compared
// at once, counted with a ballot) instead of a chain of dependent loads.
__global__ __launch_bounds__(256) void repack_grouped_kernel(
    const bt::RepackDesc* __restrict__ descs, int32_t count, int64_t total_blocks) {
    const int lane = threadIdx.x & 63;
    const int64_t waves = (int64_t(gridDim.x) * blockDim.x) >> 6;
    for (int64_t b0 = ((int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6) * kRepackPerWave;
         b0 < total_blocks; b0 += waves * kRepackPerWave) {
        int idx[kRepackPerWave];
#pragma unroll
        for (int u = 0; u < kRepackPerWave; ++u) idx[u] = -1;
        for (int base = 0; base < count; base += 64) {
            const int i = base + lane;
            const int64_t begin = i < count ? descs[i].block_begin : INT64_MAX;
#pragma unroll
            for (int u = 0; u < kRepackPerWave; ++u)
                idx[u] += __popcll(__ballot(begin <= min(b0 + u, total_blocks - 1)));
        }
        RepackIn in[kRepackPerWave];
#pragma unroll
        for (int u = 0; u < kRepackPerWave; ++u) {
            const bt::RepackDesc& d = descs[idx[u]];
            in[u] = repack_load(d.packed, d.N, d.K, d.steps,
                                min(b0 + u, total_blocks - 1) - d.block_begin, lane);
        }
#pragma unroll
        for (int u = 0; u < kRepackPerWave; ++u) {
            if (b0 + u < total_blocks) {
                const bt::RepackDesc& d = descs[idx[u]];
                repack_store(in[u], d.out, b0 + u - d.block_begin, lane);
            }
        }
    }
}

// Int8 weights (the I8_S product) in the same tile order: 16-row tiles, K
// padded to Kp = ceil(K/256)*256, each 64-wide step one 1 KB block in which
// lane l holds the 16 bytes of row l%16 at K = 64S + 16(l/16) .. +15, the
// fragment one matrix-core step reads. One wave per 1 KB block; padding is 0.
__global__ __launch_bounds__(256) void repack_int8_kernel(const int8_t* __restrict__ w, int32_t N,
                                                          int32_t K, int32_t steps64,
                                                          int64_t blocks,
                                                          int8_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    for (int64_t blk = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6; blk < blocks;
         blk += (int64_t(gridDim.x) * blockDim.x) >> 6) {
        const int64_t t = blk / steps64;
        const int32_t S = int32_t(blk - t * steps64);
        const int64_t n = t * bt::kTileN + (lane & 15);
        const int64_t k = int64_t(64) * S + 16 * (lane >> 4);
        v4u v = {0u, 0u, 0u, 0u};
        if (n < N && k < K) v = gld<v4u>(w + n * K + k);   // K % 16 == 0: whole 16 bytes
        gst<v4u>(out + blk * 1024 + lane * 16, v);
    }
}

// ---------------------------------------------------------------- quantize

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Round half away from zero, exactly: v - trunc(v) is exact in fp32 for every
// |v| < 2^23, so the comparison with 1/2 sees the true fraction.
__device__ __forceinline__ int quant1(float v) {
    const float t = truncf(v);
    const float f = v - t;
    float r = (fabsf(f) >= 0.5f) ? t + copysignf(1.0f, v) : t;
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return int(r);
}

__device__ __forceinline__ int pack4(int a, int b, int c, int d) {
    return (a & 0xff) | ((b & 0xff) << 8) | ((c & 0xff) << 16) | (int(uint32_t(d) << 24));
}

constexpr int kQuantRegs = 9;    // float4 per thread kept in registers: K <= 9216

struct QuantShared {
    float fmax[bt::kQuantThreads / 64];
    int isum[bt::kQuantThreads / 64];
};

__device__ __forceinline__ float block_max(float v, QuantShared& sh) {
    v = wave_max(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sh.fmax[w] = v;
    __syncthreads();
    float r = sh.fmax[0];
#pragma unroll
    for (int i = 1; i < bt::kQuantThreads / 64; ++i) r = fmaxf(r, sh.fmax[i]);
    return r;
}

__device__ __forceinline__ int block_sum(int v, QuantShared& sh) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sh.isum[w] = v;
    __syncthreads();
    int r = 0;
#pragma unroll
    for (int i = 0; i < bt::kQuantThreads / 64; ++i) r += sh.isum[i];
    return r;
}

// One workgroup quantizes one row: absmax, then scale, round and clamp, then
// the row sum of q. With K % 4 == 0 and K <= 9216 the row stays in registers
// between the two passes; otherwise the second pass re-reads it.
__device__ void quantize_row(const float* __restrict__ x, int64_t K, int8_t* __restrict__ q,
                             float* xscale, int32_t* xsum, QuantShared& sh) {
    const int tid = threadIdx.x;
    constexpr int T = bt::kQuantThreads;
    float amax = 0.0f;
    int s = 0;
    const bool vec = (K % 4) == 0;
    const int64_t K4 = K >> 2;
    if (vec && K4 <= int64_t(kQuantRegs) * T) {
        float4 v[kQuantRegs];
#pragma unroll
        for (int i = 0; i < kQuantRegs; ++i) {
            const int64_t idx = tid + int64_t(i) * T;
            if (idx < K4) {
                v[i] = reinterpret_cast<const float4*>(x)[idx];
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)),
                                         fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
            }
        }
        amax = block_max(amax, sh);
        float inv = 127.0f / amax;
        const bool dead = !(inv <= FLT_MAX);
        if (dead) inv = 0.0f;
#pragma unroll
        for (int i = 0; i < kQuantRegs; ++i) {
            const int64_t idx = tid + int64_t(i) * T;
            if (idx < K4) {
                const int a = quant1(v[i].x * inv), b = quant1(v[i].y * inv);
                const int c = quant1(v[i].z * inv), d = quant1(v[i].w * inv);
                reinterpret_cast<int*>(q)[idx] = pack4(a, b, c, d);
                s += a + b + c + d;
            }
        }
        s = block_sum(s, sh);
        if (tid == 0) {
            *xscale = dead ? 0.0f : amax / 127.0f;
            if (xsum) *xsum = s;
        }
        return;
    }
    for (int64_t i = tid; i < K; i += T) amax = fmaxf(amax, fabsf(x[i]));
    amax = block_max(amax, sh);
    float inv = 127.0f / amax;
    const bool dead = !(inv <= FLT_MAX);
    if (dead) inv = 0.0f;
    for (int64_t i = tid; i < K; i += T) {
        const int a = quant1(x[i] * inv);
        q[i] = int8_t(a);
        s += a;
    }
    s = block_sum(s, sh);
    if (tid == 0) {
        *xscale = dead ? 0.0f : amax / 127.0f;
        if (xsum) *xsum = s;
    }
}

__global__ __launch_bounds__(bt::kQuantThreads) void quantize_kernel(const float* __restrict__ x,
                                                                     int64_t K,
                                                                     int8_t* __restrict__ xq,
                                                                     float* __restrict__ xscale,
                                                                     int32_t* __restrict__ xsum) {
    __shared__ QuantShared sh;
    const int64_t m = blockIdx.x;
    quantize_row(x + m * K, K, xq + m * K, xscale + m, xsum ? xsum + m : nullptr, sh);
}

// Short rows (K <= 2048, K % 4 == 0): one wave per row, four rows per
// workgroup, the row held in registers and reduced with cross-lane shuffles
// only (no LDS, no barrier). Same arithmetic as quantize_row.
constexpr int kWaveRowRegs = 8;   // float4 per lane: K <= 64 * 8 * 4 = 2048

__global__ __launch_bounds__(bt::kQuantThreads) void quantize_wave_rows_kernel(
    const float* __restrict__ x, int64_t M, int64_t K, int8_t* __restrict__ xq,
    float* __restrict__ xscale, int32_t* __restrict__ xsum) {
    const int lane = threadIdx.x & 63;
    const int64_t m = int64_t(blockIdx.x) * (bt::kQuantThreads / 64) + (threadIdx.x >> 6);
    if (m >= M) return;
    const int64_t K4 = K >> 2;
    const float* xr = x + m * K;
    v4f v[kWaveRowRegs];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < kWaveRowRegs; ++j) {
        const int64_t i = lane + 64 * j;
        v[j] = i < K4 ? gld<v4f>(xr + 4 * i) : v4f{0.0f, 0.0f, 0.0f, 0.0f};
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)),
                                 fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
    }
    amax = wave_max(amax);
    float inv = 127.0f / amax;
    const bool dead = !(inv <= FLT_MAX);
    if (dead) inv = 0.0f;
    int s = 0;
    int* qr = reinterpret_cast<int*>(xq + m * K);
#pragma unroll
    for (int j = 0; j < kWaveRowRegs; ++j) {
        const int64_t i = lane + 64 * j;
        if (i < K4) {
            const int a = quant1(v[j].x * inv), b = quant1(v[j].y * inv);
            const int c = quant1(v[j].z * inv), d = quant1(v[j].w * inv);
            gst<int>(qr + i, pack4(a, b, c, d));
            s += a + b + c + d;
        }
    }
    s = wave_sum(s);
    if (lane == 0) {
        gst<float>(xscale + m, dead ? 0.0f : amax / 127.0f);
        if (xsum) gst<int32_t>(xsum + m, s);
    }
}

// ----------------------------------- RMS normalization fused with quantization
//
// "rms_norm_scaled" (technical report section 2.4.1: RMS normalization with a
// scale parameter) feeding the per-token INT8 quantization (section 2.2.2), in
// one pass over x: h = fl32(fl32(x * r) * g) with r = fl32(1 / fl32(sqrt(fl32(
// ms + eps)))), ms = fl32(S / K), S the sum of squares in fp64 (each fp32
// square is exact in fp64, so only the additions round); a row whose r is not
// finite gets r = 0. h is then quantized exactly as quantize_row does, and the
// normalized row is never written to memory.

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ double sumsq4(v4f v) {
    const double a = v.x, b = v.y, c = v.z, d = v.w;
    return ((a * a + b * b) + c * c) + d * d;
}

__device__ __forceinline__ float rms_factor(double S, int64_t K, float eps) {
    const float ms = float(S / double(K));
    const float r = 1.0f / sqrtf(ms + eps);
    return r <= FLT_MAX ? r : 0.0f;   // not finite (or NaN) -> 0
}

struct RmsShared {
    double s[bt::kQuantThreads / 64];
    QuantShared q;
};

__device__ __forceinline__ double block_sum_f64(double v, RmsShared& sh) {
    v = wave_sum_f64(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sh.s[w] = v;
    __syncthreads();
    double r = sh.s[0];
#pragma unroll
    for (int i = 1; i < bt::kQuantThreads / 64; ++i) r += sh.s[i];
    return r;
}

// One wave per row (K % 4 == 0, K <= 2048), rows in registers.
__global__ __launch_bounds__(bt::kQuantThreads) void rmsnorm_quantize_wave_rows_kernel(
    const float* __restrict__ x, const float* __restrict__ g, float eps, int64_t M, int64_t K,
    int8_t* __restrict__ xq, float* __restrict__ xscale, int32_t* __restrict__ xsum) {
    const int lane = threadIdx.x & 63;
    const int64_t m = int64_t(blockIdx.x) * (bt::kQuantThreads / 64) + (threadIdx.x >> 6);
    if (m >= M) return;
    const int64_t K4 = K >> 2;
    const float* xr = x + m * K;
    v4f v[kWaveRowRegs];
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < kWaveRowRegs; ++j) {
        const int64_t i = lane + 64 * j;
        v[j] = i < K4 ? gld<v4f>(xr + 4 * i) : v4f{0.0f, 0.0f, 0.0f, 0.0f};
        ss += sumsq4(v[j]);
    }
    const float r = rms_factor(wave_sum_f64(ss), K, eps);
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < kWaveRowRegs; ++j) {
        const int64_t i = lane + 64 * j;
        if (i < K4) {
            v[j] = (v[j] * r) * gld<v4f>(g + 4 * i);
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)),
                                     fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
        }
    }
    amax = wave_max(amax);
    float inv = 127.0f / amax;
    const bool dead = !(inv <= FLT_MAX);
    if (dead) inv = 0.0f;
    int s = 0;
    int* qr = reinterpret_cast<int*>(xq + m * K);
#pragma unroll
    for (int j = 0; j < kWaveRowRegs; ++j) {
        const int64_t i = lane + 64 * j;
        if (i < K4) {
            const int a = quant1(v[j].x * inv), b = quant1(v[j].y * inv);
            const int c = quant1(v[j].z * inv), d = quant1(v[j].w * inv);
            gst<int>(qr + i, pack4(a, b, c, d));
            s += a + b + c + d;
        }
    }
    s = wave_sum(s);
    if (lane == 0) {
        gst<float>(xscale + m, dead ? 0.0f : amax / 127.0f);
        if (xsum) gst<int32_t>(xsum + m, s);
    }
}

// One workgroup per row: the row in registers when K % 4 == 0 and K <= 9216,
// else three passes over x and g (sum of squares, absmax of h, quantize).
__global__ __launch_bounds__(bt::kQuantThreads) void rmsnorm_quantize_kernel(
    const float* __restrict__ x, const float* __restrict__ g, float eps, int64_t K,
    int8_t* __restrict__ xq, float* __restrict__ xscale, int32_t* __restrict__ xsum) {
    __shared__ RmsShared sh;
    const int64_t m = blockIdx.x;
    const float* xr = x + m * K;
    int8_t* qrow = xq + m * K;
    const int tid = threadIdx.x;
    constexpr int T = bt::kQuantThreads;
    const int64_t K4 = K >> 2;
    float amax = 0.0f;
    int s = 0;
    if ((K & 3) == 0 && K4 <= int64_t(kQuantRegs) * T) {
        v4f v[kQuantRegs];
        double ss = 0.0;
#pragma unroll
        for (int i = 0; i < kQuantRegs; ++i) {
            const int64_t idx = tid + int64_t(i) * T;
            v[i] = idx < K4 ? gld<v4f>(xr + 4 * idx) : v4f{0.0f, 0.0f, 0.0f, 0.0f};
            ss += sumsq4(v[i]);
        }
        const float r = rms_factor(block_sum_f64(ss, sh), K, eps);
#pragma unroll
        for (int i = 0; i < kQuantRegs; ++i) {
            const int64_t idx = tid + int64_t(i) * T;
            if (idx < K4) {
                v[i] = (v[i] * r) * gld<v4f>(g + 4 * idx);
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)),
                                         fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
            }
        }
        amax = block_max(amax, sh.q);
        float inv = 127.0f / amax;
        if (!(inv <= FLT_MAX)) inv = 0.0f;
#pragma unroll
        for (int i = 0; i < kQuantRegs; ++i) {
            const int64_t idx = tid + int64_t(i) * T;
            if (idx < K4) {
                const int a = quant1(v[i].x * inv), b = quant1(v[i].y * inv);
                const int c = quant1(v[i].z * inv), d = quant1(v[i].w * inv);
                reinterpret_cast<int*>(qrow)[idx] = pack4(a, b, c, d);
                s += a + b + c + d;
            }
        }
    } else {
        double ss = 0.0;
        for (int64_t k = tid; k < K; k += T) {
            const double a = xr[k];
            ss += a * a;
        }
        const float r = rms_factor(block_sum_f64(ss, sh), K, eps);
        for (int64_t k = tid; k < K; k += T) amax = fmaxf(amax, fabsf((xr[k] * r) * g[k]));
        amax = block_max(amax, sh.q);
        float inv = 127.0f / amax;
        if (!(inv <= FLT_MAX)) inv = 0.0f;
        for (int64_t k = tid; k < K; k += T) {
            const int a = quant1(((xr[k] * r) * g[k]) * inv);
            qrow[k] = int8_t(a);
            s += a;
        }
    }
    s = block_sum(s, sh.q);
    if (tid == 0) {
        const bool dead = !(127.0f / amax <= FLT_MAX);
        xscale[m] = dead ? 0.0f : amax / 127.0f;
        if (xsum) xsum[m] = s;
    }
}

__global__ __launch_bounds__(bt::kQuantThreads) void quantize_grouped_kernel(
    const QuantDesc* __restrict__ descs, int32_t count) {
    __shared__ QuantShared sh;
    const int64_t b = blockIdx.x;
    int lo = 0, hi = count - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (descs[mid].row_begin <= b) lo = mid; else hi = mid - 1;
    }
    const QuantDesc d = descs[lo];
    const int64_t m = b - d.row_begin;
    quantize_row(d.x + m * d.K, d.K, d.xq + m * d.K, d.xscale + m, d.xsum + m, sh);
}

// -------------------------------------------------------------------- GEMV
//
// A workgroup is 4 waves. It first copies its K chunk of the M activation rows
// into LDS (zero beyond K), then each wave streams tiles_per_wave 16-row weight
// tiles through the matrix cores. A wave's work is a sequence of items (tile,
// batch of up to kB 1 KB steps); the loads of item i+1 are issued before item
// i is consumed, so every wave keeps up to 2*kB KB of weights in flight.
//
// MFMA operands per 64-wide K step: lane l holds A = q[l%16][16(l/16)..+15]
// (zero for tokens >= M) from LDS and B = the unpacked codes of tile row l%16
// at the same K; the C fragment holds tokens 4(l/16)+i, output row l%16.

constexpr int kB = bt::kGemvBatch;

struct GemvBatch {
    v4u w[kB];
};

// Loads steps sb .. sb+kB-1 of a tile, clamping the step to `last` (a repeated
// step is a cache hit and is never consumed): no branches, so the compiler
// can count the loads in flight exactly.
__device__ __forceinline__ void gemv_issue(GemvBatch& b, const uint8_t* wt, int sb, int last,
                                           int lane) {
#pragma unroll
    for (int u = 0; u < kB; ++u) {
        const int st = min(sb + u, last);
#if BT_GEMV_NONTEMPORAL
        b.w[u] = gld_stream<v4u>(wt + int64_t(st) * 1024 + lane * 16);
#else
        b.w[u] = gld<v4u>(wt + int64_t(st) * 1024 + lane * 16);
#endif
    }
}

__device__ __forceinline__ v4i gemv_consume(const GemvBatch& b, int n, const int8_t* a, v4i c) {
#pragma unroll
    for (int u = 0; u < kB; ++u) {
        if (u < n) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                c = mfma16x16x64(lds_ld<v4i>(a + u * 256 + 64 * jj), unpack16(b.w[u][jj]), c);
        }
    }
    return c;
}

struct GemvShared {
    QuantShared red;
    float wmax[BT_GEMV_MAX_M][bt::kGemvWaves];   // fused prologue: per-wave |x| maxima
    float d[BT_GEMV_MAX_M];                       // per-token scale d_m
    int32_t qs[bt::kGemvWaves][BT_GEMV_MAX_M];    // per-token sum of q, as per-wave parts
};

__device__ __forceinline__ int32_t gemv_row_sum(const GemvShared& sh, int m) {
    int32_t s = sh.qs[0][m];
#pragma unroll
    for (int w = 1; w < bt::kGemvWaves; ++w) s += sh.qs[w][m];
    return s;
}

// Epilogue of one tile. With K split into chunks, partial sums meet in the
// workspace (int32 addition is exact in any order) and the last chunk to
// arrive reads the total, clears the workspace and finishes the tile.
__device__ __forceinline__ void gemv_finish(const GemvDesc& d, int64_t tile, v4i c, int lane,
                                            const GemvShared& sh, int chunk) {
    const int kq = lane >> 4;
    const int64_t n = tile * bt::kTileN + (lane & 15);
    if (d.chunks > 1 && d.slices) {
        // this chunk's partial sums into its own slice; a second launch adds
        // the slices and finishes (no cross-workgroup synchronization here)
        const int64_t slice = ((int64_t(d.M) * d.N * 4 + 255) & ~int64_t(255)) / 4;
        if (n < d.N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int mm = 4 * kq + i;
                if (mm < d.M) gst<int32_t>(d.ws + chunk * slice + int64_t(mm) * d.N + n, c[i]);
            }
        }
        return;
    }
    if (d.chunks > 1) {
        const int64_t ldw = int64_t(d.tiles) * bt::kTileN;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int mm = 4 * kq + i;
            if (mm < d.M) atomicAdd(d.ws + mm * ldw + n, c[i]);
        }
        __threadfence();
        uint32_t prev = 0;
        if (lane == 0) prev = atomicAdd(d.cnt + tile, 1u);
        prev = __shfl(prev, 0, 64);
        if (prev != uint32_t(d.chunks - 1)) return;
        __threadfence();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int mm = 4 * kq + i;
            if (mm < d.M) c[i] = atomicExch(d.ws + mm * ldw + n, 0);
        }
        if (lane == 0) atomicExch(d.cnt + tile, 0u);
    }
    if (n < d.N) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int mm = 4 * kq + i;
            if (mm < d.M) {
                const int32_t qsum = gemv_row_sum(sh, mm);
                const float dm = sh.d[mm];
                const int32_t acc = c[i] - qsum;
                const float rs = dm * d.w_scale;
                const int64_t o = int64_t(mm) * d.N + n;
                float v = epi_col(d.epi, float(acc) * rs, n);
                if (d.epi.res) v = d.epi.res[o] + v;
                gst<float>(d.y + o, v);
                if (d.acc) gst<int32_t>(d.acc + o, acc);
            }
        }
    }
}

// Fused quantization prologue: each workgroup quantizes the whole of every
// token row (the row sum of q and the scale need all of it), keeps its own K
// chunk in LDS, and the first workgroup of the problem also writes q, d and
// the row sums out when asked to. The arithmetic is quantize_row's exactly.
// Rows up to kFusedRegs*1024 elements are read once into registers; token 0
// is read before the first weight loads go out, so its data is not queued
// behind them. Longer rows are read twice (absmax, then quantize).
constexpr int kFusedRegs = 2;   // float4 per thread: K <= 2048 in one read
constexpr int kGemvThreads = 64 * bt::kGemvWaves;

struct FusedRow {
    v4f v[kFusedRegs];
};

__device__ __forceinline__ void gemv_load_row(FusedRow& r, const GemvDesc& d, int m) {
    const int64_t K4 = d.K >> 2;
    const float* xr = d.x + int64_t(m) * d.K;
#pragma unroll
    for (int j = 0; j < kFusedRegs; ++j) {
        // clamped, branch-free: lanes past the row re-read its last float4
        // and their values are never used
        const int64_t i = min(int64_t(threadIdx.x) + int64_t(j) * kGemvThreads, K4 - 1);
        r.v[j] = gld<v4f>(xr + 4 * i);
    }
}

__device__ __forceinline__ int gemv_quant_store(v4f v, float inv, int64_t k, int m, bool writer,
                                                const GemvDesc& d, int64_t kbeg, int64_t kend,
                                                int8_t* lds) {
    const int a = quant1(v.x * inv), b = quant1(v.y * inv);
    const int c = quant1(v.z * inv), e = quant1(v.w * inv);
    const int packed = pack4(a, b, c, e);
    if (k >= kbeg && k < kend) lds_st<int>(lds + m * d.lds_row + (k - kbeg), packed);
    if (writer && d.xq) gst<int>(d.xq + int64_t(m) * d.K + k, packed);
    return a + b + c + e;
}

// One short row held in registers: a barrier joins the four wave maxima; the
// row sum is left as four wave parts that the caller's barrier publishes.
__device__ __forceinline__ void gemv_quant_short_row(const FusedRow& r, int m, const GemvDesc& d,
                                                     bool writer, int64_t kbeg, int64_t kend,
                                                     int8_t* lds, GemvShared& sh) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int64_t K4 = d.K >> 2;
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < kFusedRegs; ++j) {
        const int64_t i = tid + int64_t(j) * kGemvThreads;
        if (i < K4)
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(r.v[j].x), fabsf(r.v[j].y)),
                                     fmaxf(fabsf(r.v[j].z), fabsf(r.v[j].w))));
    }
    amax = wave_max(amax);
    if ((tid & 63) == 0) sh.wmax[m][wave] = amax;
    __syncthreads();
    amax = sh.wmax[m][0];
#pragma unroll
    for (int w = 1; w < bt::kGemvWaves; ++w) amax = fmaxf(amax, sh.wmax[m][w]);
    float inv = 127.0f / amax;
    const bool dead = !(inv <= FLT_MAX);
    if (dead) inv = 0.0f;
    int s = 0;
#pragma unroll
    for (int j = 0; j < kFusedRegs; ++j) {
        const int64_t i = tid + int64_t(j) * kGemvThreads;
        if (i < K4) s += gemv_quant_store(r.v[j], inv, 4 * i, m, writer, d, kbeg, kend, lds);
    }
    s = wave_sum(s);
    if ((tid & 63) == 0) sh.qs[wave][m] = s;
    if (tid == 0) {
        const float dm = dead ? 0.0f : amax / 127.0f;
        sh.d[m] = dm;
        if (writer && d.xscale) gst<float>(d.xscale + m, dm);
    }
}

// All token rows. `r0` holds token 0 when the rows are short. Ends with the
// barrier that publishes q, d and the row-sum parts; the writer then stores
// the row sums.
__device__ __forceinline__ void gemv_quantize_rows(const GemvDesc& d, const FusedRow& r0,
                                                   bool writer, int64_t kbeg, int64_t kend,
                                                   int8_t* lds, GemvShared& sh) {
    const int tid = threadIdx.x;
    constexpr int T = kGemvThreads;
    const int64_t K4 = d.K >> 2;   // K % 128 == 0
    if (K4 <= int64_t(kFusedRegs) * T) {
        gemv_quant_short_row(r0, 0, d, writer, kbeg, kend, lds, sh);
        for (int m = 1; m < d.M; ++m) {
            FusedRow r;
            gemv_load_row(r, d, m);
            gemv_quant_short_row(r, m, d, writer, kbeg, kend, lds, sh);
        }
    } else {
        for (int m = 0; m < d.M; ++m) {
            const float* xr = d.x + int64_t(m) * d.K;
            float amax = 0.0f;
            for (int64_t i = tid; i < K4; i += T) {
                const v4f v = gld<v4f>(xr + 4 * i);
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
            }
            amax = block_max(amax, sh.red);
            float inv = 127.0f / amax;
            const bool dead = !(inv <= FLT_MAX);
            if (dead) inv = 0.0f;
            int s = 0;
            for (int64_t i = tid; i < K4; i += T)
                s += gemv_quant_store(gld<v4f>(xr + 4 * i), inv, 4 * i, m, writer, d, kbeg, kend, lds);
            s = block_sum(s, sh.red);
            if (tid < bt::kGemvWaves) sh.qs[tid][m] = tid == 0 ? s : 0;
            if (tid == 0) {
                const float dm = dead ? 0.0f : amax / 127.0f;
                sh.d[m] = dm;
                if (writer && d.xscale) gst<float>(d.xscale + m, dm);
            }
            __syncthreads();   // the reduction slots are reused by the next row
        }
    }
    __syncthreads();
    if (writer && d.xsum && tid < d.M) gst<int32_t>(d.xsum + tid, gemv_row_sum(sh, tid));
}

template <bool kFused, bool kWaveSplit>
__device__ __forceinline__ void gemv_block(const GemvDesc& d, int64_t local_block, int8_t* lds,
                                           GemvShared& sh) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int chunk = int(local_block / d.groups);
    const int64_t g = local_block - int64_t(chunk) * d.groups;
    const int s0 = chunk * d.steps_per_chunk;
    const int s1 = min(s0 + d.steps_per_chunk, d.steps);
    const int nsteps = s1 - s0;
    // With waves_per_tile > 1, wave `wave` takes sub-range `sub` of its tile's
    // steps [s0, s1) (possibly empty: its loads are then clamped repeats of a
    // valid step, never consumed).
    const int wpt = kWaveSplit ? d.waves_per_tile : 1;
    const int sub = wave & (wpt - 1);
    const int sps_w = (nsteps + wpt - 1) / wpt;
    const int ws0 = min(s0 + sub * sps_w, s1);
    const int ws1 = min(ws0 + sps_w, s1);
    const int nsteps_w = ws1 - ws0;
    const int nb = max(1, (nsteps_w + kB - 1) / kB);
    const int total = d.tiles_per_wave * nb;
    const int tile_stride = bt::kGemvWaves / wpt;
    const int64_t tile0 = g * (int64_t(tile_stride) * d.tiles_per_wave) + wave / wpt;
    const int64_t tile_bytes = int64_t(d.steps) * 1024;

    // Items are (tile, batch of kB steps). Two items are loaded back to back
    // (2*kB KB in flight per wave), then consumed. Loads are unconditional:
    // a tile past N or a step past the chunk is clamped to a valid address and
    // its data is never consumed.
    auto issue = [&](GemvBatch& b, int idx) {
        const int r = idx / nb;
        const int bb = idx - r * nb;
        const int64_t t = min(tile0 + int64_t(tile_stride) * r, int64_t(d.tiles) - 1);
        gemv_issue(b, d.w + t * tile_bytes, ws0 + bb * kB, ws1 - 1, lane);
    };

    // The first weight batches go out before the activations are staged, so
    // their latency overlaps the staging. Fused: token 0's activations go out
    // first, and the second batch waits until the rows are quantized (the
    // registers it needs hold the activations until then).
    FusedRow r0;
    if (kFused) gemv_load_row(r0, d, 0);
    GemvBatch b0, b1;
    issue(b0, 0);
    if (!kFused) issue(b1, min(1, total - 1));

    // Stage this chunk of the M token rows in LDS rows 0..M-1 (zero past K)
    // and a zero row M, which the lanes of tokens >= M read instead.
    const int64_t kbeg = int64_t(s0) * bt::kSuperK;
    const int64_t kend = int64_t(s1) * bt::kSuperK;
    const int pieces = nsteps * (bt::kSuperK / 16);
    if (kFused) {
        for (int i = tid; i < (d.M + 1) * pieces; i += 64 * bt::kGemvWaves) {
            const int m = i / pieces;
            const int col = (i - m * pieces) * 16;
            if (m == d.M || kbeg + col >= d.K) lds_st<v4i>(lds + m * d.lds_row + col, v4i{0, 0, 0, 0});
        }
        gemv_quantize_rows(d, r0, chunk == 0 && g == 0, kbeg, kend, lds, sh);
        issue(b1, min(1, total - 1));
    } else {
        for (int i = tid; i < (d.M + 1) * pieces; i += 64 * bt::kGemvWaves) {
            const int m = i / pieces;
            const int col = (i - m * pieces) * 16;
            v4i v = {0, 0, 0, 0};
            if (m < d.M && kbeg + col < d.K) v = gld<v4i>(d.xq + int64_t(m) * d.K + kbeg + col);
            lds_st<v4i>(lds + m * d.lds_row + col, v);
        }
        // the epilogue's per-token scale and row sum, read once
        if (tid < d.M) {
            sh.d[tid] = gld<float>(d.xscale + tid);
            sh.qs[0][tid] = gld<int32_t>(d.xsum + tid);
#pragma unroll
            for (int w = 1; w < bt::kGemvWaves; ++w) sh.qs[w][tid] = 0;
        }
        __syncthreads();
    }

    const int am = min(lane & 15, d.M);
    const int8_t* abase = lds + am * d.lds_row + 16 * (lane >> 4);
    v4i cur = {0, 0, 0, 0};
    auto consume = [&](const GemvBatch& b, int idx) {
        const int r = idx / nb;
        const int bb = idx - r * nb;
        const int64_t t = tile0 + int64_t(tile_stride) * r;
        if (t >= d.tiles) return;
        cur = gemv_consume(b, min(kB, nsteps_w - bb * kB), abase + (ws0 - s0 + bb * kB) * 256,
                           cur);
        if (bb == nb - 1 && wpt == 1) {
            gemv_finish(d, t, cur, lane, sh, chunk);
            cur = v4i{0, 0, 0, 0};
        }
    };

    // Two items are in flight, then consumed. The scheduling barriers keep the
    // unpacking of batch 1 below the use of batch 0.
    for (int idx = 0; idx < total; idx += 2) {
        if (idx > 0) {
            issue(b0, idx);
            __builtin_amdgcn_sched_barrier(0);
            issue(b1, min(idx + 1, total - 1));
        }
        __builtin_amdgcn_sched_barrier(0);
        consume(b0, idx);
        __builtin_amdgcn_sched_barrier(0);
        if (idx + 1 < total) consume(b1, idx + 1);
    }
    if (kWaveSplit && wpt > 1) {
        // the sub-range sums of each tile meet in LDS (over the activations,
        // which every wave has finished reading), then its first wave finishes
        __syncthreads();
        v4i* part = reinterpret_cast<v4i*>(lds);
        part[wave * 64 + lane] = cur;
        __syncthreads();
        if (sub == 0 && tile0 < d.tiles) {
            for (int s = 1; s < wpt; ++s) cur += part[(wave + s) * 64 + lane];
            gemv_finish(d, tile0, cur, lane, sh, chunk);
        }
    }
}

// Single calls: waves_per_tile may split a tile's K range over the workgroup.
template <bool kFused>
__global__ __launch_bounds__(64 * bt::kGemvWaves) __attribute__((amdgpu_waves_per_eu(4))) void gemv_kernel(GemvDesc d) {
    extern __shared__ __attribute__((aligned(16))) int8_t gemv_lds[];
    __shared__ GemvShared sh;
    gemv_block<kFused, true>(d, blockIdx.x, gemv_lds, sh);
}

template <bool kFused>
__global__ __launch_bounds__(64 * bt::kGemvWaves) __attribute__((amdgpu_waves_per_eu(5))) void gemv_grouped_kernel(
    const GemvDesc* __restrict__ descs, int32_t count) {
    extern __shared__ __attribute__((aligned(16))) int8_t gemv_lds[];
    __shared__ GemvShared sh;
    const int64_t b = blockIdx.x;
    int lo = 0, hi = count - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (descs[mid].block_begin <= b) lo = mid; else hi = mid - 1;
    }
    const GemvDesc d = descs[lo];
    gemv_block<kFused, false>(d, b - d.block_begin, gemv_lds, sh);
}

size_t gemv_lds_bytes(const GemvDesc& d) {
    const size_t rows = size_t(d.M + 1) * size_t(d.lds_row);
    // waves_per_tile > 1 reuses the activation space for the waves' partial sums
    return d.waves_per_tile > 1 ? std::max(rows, size_t(bt::kGemvWaves) * 64 * 16) : rows;
}

// -------------------------------------------------------------------- GEMM
//
// Prefill GEMM for M > 16. A workgroup of WGM x WGN waves computes a
// (WA*WGM) x (WW*WGN) tile of y (token rows x weight rows); each wave owns a
// WA x WW sub-tile held as (WA/16) x (WW/16) MFMA accumulators.
//
// K advances in 256-wide stages. The workgroup's activation rows for a stage
// (BM x 256 int8) are copied from global memory straight into one of two LDS
// buffers (buffer_load ... lds: no staging registers), while the other
// buffer feeds the matrix cores. Rows past M, and columns past K, read as
// zero through the buffer bounds. In LDS a row's sixteen 16-byte chunks are
// stored XOR-swizzled (chunk c of row r at slot c ^ (r % 16)), so the 16 rows
// an MFMA fragment read touches fall in 16 different bank groups. Each wave
// keeps its WW/16 weight tiles' packed words for the next stage in registers
// (one 128-bit load per tile and lane) and unpacks each 16-element word right
// before the WA/16 MFMAs that use it.
//
// Workgroup order: consecutive workgroup ids go to different XCDs, so ids are
// remapped to give each XCD a contiguous band of output tiles (whole rows of
// tiles along N): the activation rows of a band stay in that XCD's L2.

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
};

constexpr int kXcds = 8;

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
    static_assert(KS == 128 || KS == 256, "stage width");
    static_assert(WA % 16 == 0 && WW % 16 == 0, "wave tile");
    static_assert(NS >= 2 && (NS - 2) * kLoads < 64, "pipeline depth");
    static_assert(kDmaPerWave * 64 * NW == BM * CPR, "A stage must split evenly over waves");
    __shared__ __attribute__((aligned(16))) int8_t As[NS * kStage];
    // After the main loop the stage buffers are idle (a barrier makes sure):
    // the row-wise epilogue's blocks live in them.
    constexpr bool kRowStores = WW == 64;   // row-wise epilogue through LDS
    float* const Ep = reinterpret_cast<float*>(As);
    static_assert(NS * kStage >= NW * 16 * 64 * 4, "epilogue blocks fit the stage buffers");

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
            lds_dma16(arsrc, As + buf * kStage + (wave * kDmaPerWave + j) * 1024, voff, kcol);
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
    const int8_t* afrag = As + (wm * WA + (lane & 15)) * KS;
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
        const int8_t* abuf = afrag + buf * kStage;
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
            asm volatile("" ::: "memory");
            consume(u, b[u]);
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
template <int WA, int WW, int NW, int KS, int NS>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_persistent_kernel(GemmArgs g) {
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
    __shared__ __attribute__((aligned(16))) int8_t As[NS * kStage];
    constexpr bool kRowStores = WW == 64;   // row-wise epilogue through LDS
    __shared__ __attribute__((aligned(16))) float Ep[kRowStores ? NW * 16 * 64 : 4];

    auto slot_of = [](int r, int c) {
        return KS == 256 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7));
    };

    // this workgroup's tiles: first, first + per_wg, ... below hi
    const int xcd = blockIdx.x % kXcds;
    const int per_wg = int(gridDim.x) / kXcds;
    const int total = g.m_tiles * g.n_tiles;
    const int lo = xcd * g.per_xcd;
    const int hi = min(lo + g.per_xcd, total);
    const int first = lo + int(blockIdx.x) / kXcds;
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
        ra = make_rsrc(g.xq + m0 * g.K, uint32_t(min(int64_t(BM), int64_t(g.M) - m0)) * uint32_t(g.K));
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
        avoff[q] = uint32_t(r0) * uint32_t(g.K) + uint32_t(c) * 16u;
        ahigh[q] = c >= 8 ? kNowhere : 0u;
    }
    const bool tail128 = KS == 256 && (g.K & 255) != 0;
    auto load_a = [&](int buf, __amdgpu_buffer_rsrc_t ra, int s, uint32_t pad) {
        const uint32_t kcol = uint32_t(s) * KS;
        const uint32_t tail = (tail128 && s == nst - 1) ? 0xffffffffu : 0u;
#pragma unroll
        for (int j = 0; j < kDmaPerWave; ++j) {
            const uint32_t voff = (avoff[j & 3] + uint32_t(RPC * j) * uint32_t(g.K)) | pad |
                                  (ahigh[j & 3] & tail);
            lds_dma16(ra, As + buf * kStage + (wave * kDmaPerWave + j) * 1024, voff, kcol);
        }
    };

    v4i acc[TA][TW];
#pragma unroll
    for (int i = 0; i < TA; ++i)
#pragma unroll
        for (int t = 0; t < TW; ++t) acc[i][t] = v4i{0, 0, 0, 0};
    const int8_t* afrag = As + (lane & 15) * KS;
    int aslot[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) aslot[kk] = slot_of(lane & 15, 4 * kk + (lane >> 4)) * 16;
    auto consume = [&](int buf, const BVec (&bc)[TW]) {
        const int8_t* abuf = afrag + buf * kStage;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            v4i af[TA];
#pragma unroll
            for (int i = 0; i < TA; ++i) af[i] = lds_ld<v4i>(abuf + i * 16 * KS + aslot[kk]);
#pragma unroll
            for (int t = 0; t < TW; ++t) {
                const v4i bf = unpack16(bc[t][kk]);
#pragma unroll
                for (int i = 0; i < TA; ++i) acc[i][t] = mfma16x16x64(bf, af[i], acc[i][t]);
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
                asm volatile("" ::: "memory");
                consume(u, b[u]);
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
                        __builtin_nontemporal_store(yv, (BT_GLOBAL v4f*)(yrow + n));
                        if (arow) __builtin_nontemporal_store(a, (BT_GLOBAL v4i*)(arow + n));
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if (n + e < g.N) {
                                gst<float>(yrow + n + e, yv[e]);
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

#ifndef BT_GEMM_WA
#define BT_GEMM_WA 128
#endif
#ifndef BT_GEMM_WW
#define BT_GEMM_WW 64
#endif
#ifndef BT_GEMM_WGM
#define BT_GEMM_WGM 1
#endif
#ifndef BT_GEMM_WGN
#define BT_GEMM_WGN 4
#endif
#ifndef BT_GEMM_KS
#define BT_GEMM_KS 128
#endif
#ifndef BT_GEMM_NS
#define BT_GEMM_NS 2
#endif


#ifndef BT_GEMM_GROUPED
#define BT_GEMM_GROUPED 1
#endif

// Token-row bands per tile group: as many as one XCD's share of the tiles
// spans, so that share is one compact block of the output.
int32_t gemm_group_m(int32_t m_tiles, int32_t n_tiles, int64_t tiles_per_xcd) {
    if (!BT_GEMM_GROUPED) return 1;
    const int64_t gm = bt::ceil_div(tiles_per_xcd, n_tiles);
    return int32_t(std::max<int64_t>(1, std::min<int64_t>(m_tiles, gm)));
}

// Shape dispatch of the GEMM: the default tile, or a 128 x 128 tile (waves of
// 64 x 64) when the default leaves fewer than two workgroups per compute unit
// (e.g. 4096 x 1536 outputs).
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
    g.group_m = gemm_group_m(g.m_tiles, g.n_tiles, bt::ceil_div(g.per_xcd, g.splits));
    const int64_t grid = int64_t(g.per_xcd) * kXcds;
    if (grid > (int64_t(1) << 31) - 1) return BT_ERR_SHAPE;
    (void)hipGetLastError();
    hipLaunchKernelGGL((gemm_kernel<WA, WW, WGM, WGN, KS, NS, kW8>), dim3(unsigned(grid)),
                       dim3(64 * WGM * WGN), 0, stream, g);
    return hipGetLastError() == hipSuccess ? BT_OK : BT_ERR_DEVICE;
}

#ifndef BT_GEMM_PERSISTENT
#define BT_GEMM_PERSISTENT 1
#endif
#ifndef BT_GEMM_P_WA
#define BT_GEMM_P_WA 128
#endif
#ifndef BT_GEMM_P_NW
#define BT_GEMM_P_NW 4
#endif
#ifndef BT_GEMM_P_NS
#define BT_GEMM_P_NS 3
#endif
#ifndef BT_GEMM_P_WGS_PER_CU
#define BT_GEMM_P_WGS_PER_CU 2
#endif

// Compute units of the current device, read once per device.
int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

template <int WA, int WW, int NW, int KS, int NS>
bt_status launch_gemm_persistent(GemmArgs g, hipStream_t stream) {
    constexpr int BM = WA;
    constexpr int BN = WW * NW;
    g.m_tiles = int32_t(bt::ceil_div(g.M, BM));
    g.n_tiles = int32_t(bt::ceil_div(g.N, BN));
    const int64_t total = int64_t(g.m_tiles) * g.n_tiles;
    if (total > (int64_t(1) << 31) - 1) return BT_ERR_SHAPE;
    g.per_xcd = int32_t(bt::ceil_div(total, kXcds));
    g.group_m = gemm_group_m(g.m_tiles, g.n_tiles, g.per_xcd);
    // one workgroup per resident slot, a multiple of the XCD count, and no
    // more than there are tiles in an XCD's band
    const int64_t slots = int64_t(device_cus()) * BT_GEMM_P_WGS_PER_CU / kXcds;
    const int64_t per_xcd_wgs = std::max<int64_t>(1, std::min<int64_t>(slots, g.per_xcd));
    (void)hipGetLastError();
    hipLaunchKernelGGL((gemm_persistent_kernel<WA, WW, NW, KS, NS>),
                       dim3(unsigned(per_xcd_wgs * kXcds)), dim3(64 * NW), 0, stream, g);
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
            v4i a = gld<v4i>(g.ws + o);
            for (int sp = 1; sp < g.splits; ++sp) a += gld<v4i>(g.ws + sp * g.ws_slice + o);
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

// Runs the kernel gemm_choice picked for the shape; with split K, binds the
// workspace (partial sums, then one counter per tile).
bt_status dispatch_gemm(GemmArgs g, bool int8_weights, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
    const bt::GemmChoice c =
        bt::gemm_choice(g.M, g.N, g.K, int8_weights, BT_GEMM_PERSISTENT && !epi_any(g.epi));
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
    if (int8_weights) {
        st = c.kind == 2 ? launch_gemm<64, 64, 2, 2, 128, 2, true>(g, stream)
                         : launch_gemm<128, 64, 1, 4, 128, 2, true>(g, stream);
        if (st == BT_OK && g.splits > 1) st = launch_splitk_reduce<true>(g, stream);
        return st;
    }
#if BT_GEMM_PERSISTENT
    if (c.kind == 0)
        return launch_gemm_persistent<BT_GEMM_P_WA, 64, BT_GEMM_P_NW, 128, BT_GEMM_P_NS>(g, stream);
#endif
    st = c.kind == 2 ? launch_gemm<64, 64, 2, 2, 256, 2>(g, stream)
                     : launch_gemm<128, 64, 1, 4, 128, 2>(g, stream);
    if (st == BT_OK && g.splits > 1) st = launch_splitk_reduce<false>(g, stream);
    return st;
}

bt_status launched() {
    return hipGetLastError() == hipSuccess ? BT_OK : BT_ERR_DEVICE;
}

bool nk_ok(int64_t N, int64_t K) { return bt_repacked_bytes(N, K) != 0; }

}  // namespace

// ===================================================================== C ABI

extern "C" bt_status bt_repack_ternary(const uint8_t* packed_dev, int64_t N, int64_t K, void* wdev,
                                       hipStream_t stream) {
    if (!packed_dev || !wdev) return BT_ERR_NULL;
    if (!nk_ok(N, K)) return BT_ERR_SHAPE;
    if (!bt::aligned16(packed_dev) || !bt::aligned16(wdev)) return BT_ERR_ALIGN;
    const int64_t steps = bt::ceil_div(K, bt::kSuperK);
    const int64_t blocks = bt::ceil_div(N, bt::kTileN) * steps;   // 1 KB output blocks
    const int64_t grid = std::min<int64_t>(bt::ceil_div(blocks, 4 * kRepackPerWave), int64_t(1) << 20);
    (void)hipGetLastError();
    hipLaunchKernelGGL(repack_kernel, dim3(unsigned(grid)), dim3(256), 0, stream, packed_dev,
                       int32_t(N), int32_t(K), int32_t(steps), blocks,
                       static_cast<uint8_t*>(wdev));
    return launched();
}

extern "C" bt_status bt_repack_ternary_grouped(const void* plan_host, const void* plan_dev,
                                               hipStream_t stream) {
    if (!plan_host || !plan_dev) return BT_ERR_NULL;
    const auto* hdr = static_cast<const bt::PlanHeader*>(plan_host);
    if (hdr->magic != bt::kPlanMagicRepack || hdr->count < 1 || hdr->total_blocks < 1)
        return BT_ERR_VALUE;
    if (!bt::aligned16(plan_dev)) return BT_ERR_ALIGN;
    const auto* descs = reinterpret_cast<const bt::RepackDesc*>(
        static_cast<const char*>(plan_dev) + sizeof(bt::PlanHeader));
    const int64_t grid = std::min<int64_t>(bt::ceil_div(hdr->total_blocks, 4 * kRepackPerWave),
                                           int64_t(1) << 20);
    (void)hipGetLastError();
    hipLaunchKernelGGL(repack_grouped_kernel, dim3(unsigned(grid)), dim3(256), 0, stream, descs,
                       hdr->count, hdr->total_blocks);
    return launched();
}

extern "C" bt_status bt_quantize_act(const float* x, int64_t M, int64_t K, int8_t* xq,
                                     float* xscale, int32_t* xsum, hipStream_t stream) {
    if (!x || !xq || !xscale) return BT_ERR_NULL;
    if (M < 1 || K < 1 || M > (int64_t(1) << 31) - 1 || K > (int64_t(1) << 30))
        return BT_ERR_SHAPE;
    if (!bt::aligned16(x) || !bt::aligned16(xq) || !bt::aligned16(xscale) ||
        (xsum && !bt::aligned16(xsum)))
        return BT_ERR_ALIGN;
    (void)hipGetLastError();
    if (K % 4 == 0 && K / 4 <= 64 * kWaveRowRegs) {
        const int64_t rows_per_wg = bt::kQuantThreads / 64;
        hipLaunchKernelGGL(quantize_wave_rows_kernel, dim3(unsigned(bt::ceil_div(M, rows_per_wg))),
                           dim3(bt::kQuantThreads), 0, stream, x, M, K, xq, xscale, xsum);
    } else {
        hipLaunchKernelGGL(quantize_kernel, dim3(unsigned(M)), dim3(bt::kQuantThreads), 0, stream,
                           x, K, xq, xscale, xsum);
    }
    return launched();
}

extern "C" bt_status bt_rmsnorm_quantize(const float* x, const float* g, float eps, int64_t M,
                                         int64_t K, int8_t* xq, float* xscale, int32_t* xsum,
                                         hipStream_t stream) {
    if (!x || !g || !xq || !xscale) return BT_ERR_NULL;
    if (M < 1 || K < 1 || M > (int64_t(1) << 31) - 1 || K > (int64_t(1) << 30))
        return BT_ERR_SHAPE;
    if (!bt::aligned16(x) || !bt::aligned16(g) || !bt::aligned16(xq) || !bt::aligned16(xscale) ||
        (xsum && !bt::aligned16(xsum)))
        return BT_ERR_ALIGN;
    if (!isfinite(eps) || eps < 0.0f) return BT_ERR_VALUE;
    (void)hipGetLastError();
    if (K % 4 == 0 && K / 4 <= 64 * kWaveRowRegs) {
        const int64_t rows_per_wg = bt::kQuantThreads / 64;
        hipLaunchKernelGGL(rmsnorm_quantize_wave_rows_kernel,
                           dim3(unsigned(bt::ceil_div(M, rows_per_wg))), dim3(bt::kQuantThreads),
                           0, stream, x, g, eps, M, K, xq, xscale, xsum);
    } else {
        hipLaunchKernelGGL(rmsnorm_quantize_kernel, dim3(unsigned(M)), dim3(bt::kQuantThreads), 0,
                           stream, x, g, eps, K, xq, xscale, xsum);
    }
    return launched();
}

// Fills the split-K workspace pointers of a single-call GEMV.
// A single call whose activations need more than one LDS slice splits K:
// the chunks' partial sums go to slices of the workspace, and after them the
// fused path's scales and row sums when the caller does not keep them.
static bt_status gemv_bind_workspace(GemvDesc& d, void* workspace, size_t workspace_bytes) {
    const size_t need = bt::gemv_single_workspace_bytes(d);
    if (!need) return BT_OK;
    if (!workspace || workspace_bytes < need) return BT_ERR_WORKSPACE;
    if (!bt::aligned16(workspace)) return BT_ERR_ALIGN;
    d.slices = 1;
    d.ws = static_cast<int32_t*>(workspace);
    return BT_OK;
}

// Second launch of a split single-call GEMV: adds the chunks' slices, then
// the rescale and epilogue (the GEMM's split-K reduction, which shares the
// slice layout).
static bt_status gemv_reduce(const GemvDesc& d, hipStream_t stream) {
    GemmArgs g;
    memset(&g, 0, sizeof(g));
    g.xscale = d.xscale;
    g.xsum = d.xsum;
    g.y = d.y;
    g.acc = d.acc;
    g.w_scale = d.w_scale;
    g.M = d.M;
    g.N = d.N;
    g.K = d.K;
    g.epi = d.epi;
    g.splits = d.chunks;
    g.ws = d.ws;
    g.ws_slice = int64_t(bt::gemm_slice_bytes(d.M, d.N) / sizeof(int32_t));
    return launch_splitk_reduce<false>(g, stream);
}

extern "C" bt_status bt_ternary_matmul_fused(int64_t M, int64_t N, int64_t K, const float* x,
                                             const void* wdev, float w_scale, float* y,
                                             int32_t* acc, int8_t* xq, float* xscale,
                                             int32_t* xsum, void* workspace,
                                             size_t workspace_bytes, hipStream_t stream) {
    if (!x || !wdev || !y) return BT_ERR_NULL;
    if (M < 1 || M > BT_GEMV_MAX_M || !nk_ok(N, K)) return BT_ERR_SHAPE;
    if (!bt::aligned16(x) || !bt::aligned16(wdev) || !bt::aligned16(y) ||
        (acc && !bt::aligned16(acc)) || (xq && !bt::aligned16(xq)) ||
        (xscale && !bt::aligned16(xscale)) || (xsum && !bt::aligned16(xsum)))
        return BT_ERR_ALIGN;
    if (!isfinite(w_scale)) return BT_ERR_VALUE;
    GemvDesc d;
    bt::gemv_shape(M, N, K, false, &d);
    const bt_status st = gemv_bind_workspace(d, workspace, workspace_bytes);
    if (st != BT_OK) return st;
    d.x = x;
    d.xq = xq;
    d.xscale = xscale;
    d.xsum = xsum;
    d.w = static_cast<const uint8_t*>(wdev);
    d.y = y;
    d.acc = acc;
    d.w_scale = w_scale;
    if (d.chunks > 1) {
        // the second launch needs the scales and row sums: keep them in the
        // workspace, after the slices, when the caller does not
        char* scratch = reinterpret_cast<char*>(d.ws) + bt::gemm_slice_bytes(M, N) * d.chunks;
        if (!d.xscale) d.xscale = reinterpret_cast<float*>(scratch);
        if (!d.xsum) d.xsum = reinterpret_cast<int32_t*>(scratch + 4 * M);
    }
    (void)hipGetLastError();
    hipLaunchKernelGGL(gemv_kernel<true>, dim3(unsigned(d.blocks)), dim3(64 * bt::kGemvWaves),
                       gemv_lds_bytes(d), stream, d);
    const bt_status st2 = launched();
    if (st2 != BT_OK || d.chunks <= 1) return st2;
    return gemv_reduce(d, stream);
}

// Checks an epilogue against the output it is applied to and converts it.
static bt_status epilogue_args(const bt_epilogue* epi, int64_t M, int64_t N, const float* y,
                               EpiArgs* out) {
    memset(out, 0, sizeof(*out));
    if (!epi) return BT_OK;
    if (!bt::aligned16(epi->bias) || !bt::aligned16(epi->layer_scale) ||
        !bt::aligned16(epi->residual))
        return BT_ERR_ALIGN;
    if (epi->residual && epi->residual != y) {
        // the residual is the output itself, or disjoint from it
        const uintptr_t r0 = reinterpret_cast<uintptr_t>(epi->residual);
        const uintptr_t y0 = reinterpret_cast<uintptr_t>(y);
        const uintptr_t bytes = uintptr_t(M) * uintptr_t(N) * sizeof(float);
        if (r0 < y0 + bytes && y0 < r0 + bytes) return BT_ERR_VALUE;
    }
    out->bias = epi->bias;
    out->gamma = epi->layer_scale;
    out->res = epi->residual;
    out->relu = epi->relu ? 1 : 0;
    return BT_OK;
}

static bt_status matmul_impl(int64_t M, int64_t N, int64_t K, const int8_t* xq,
                             const float* xscale, const int32_t* xsum, const void* wdev,
                             float w_scale, const bt_epilogue* epi, float* y, int32_t* acc,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!xq || !xscale || !xsum || !wdev || !y) return BT_ERR_NULL;
    if (M < 1 || M > (int64_t(1) << 31) - 1 || !nk_ok(N, K)) return BT_ERR_SHAPE;
    if (!bt::aligned16(xq) || !bt::aligned16(xscale) || !bt::aligned16(xsum) ||
        !bt::aligned16(wdev) || !bt::aligned16(y) || (acc && !bt::aligned16(acc)))
        return BT_ERR_ALIGN;
    if (!isfinite(w_scale)) return BT_ERR_VALUE;
    EpiArgs e;
    const bt_status est = epilogue_args(epi, M, N, y, &e);
    if (est != BT_OK) return est;
    if (M <= BT_GEMV_MAX_M) {
        GemvDesc d;
        bt::gemv_shape(M, N, K, false, &d);
        const bt_status st = gemv_bind_workspace(d, workspace, workspace_bytes);
        if (st != BT_OK) return st;
        d.xq = const_cast<int8_t*>(xq);
        d.xscale = const_cast<float*>(xscale);
        d.xsum = const_cast<int32_t*>(xsum);
        d.w = static_cast<const uint8_t*>(wdev);
        d.y = y;
        d.acc = acc;
        d.w_scale = w_scale;
        d.epi = e;
        (void)hipGetLastError();
        hipLaunchKernelGGL(gemv_kernel<false>, dim3(unsigned(d.blocks)), dim3(64 * bt::kGemvWaves),
                           gemv_lds_bytes(d), stream, d);
        const bt_status lst = launched();
        if (lst != BT_OK || d.chunks <= 1) return lst;
        return gemv_reduce(d, stream);
    }
    GemmArgs g;
    memset(&g, 0, sizeof(g));
    g.epi = e;
    g.xq = xq;
    g.xscale = xscale;
    g.xsum = xsum;
    g.w = static_cast<const uint8_t*>(wdev);
    g.y = y;
    g.acc = acc;
    g.w_scale = w_scale;
    g.M = int32_t(M);
    g.N = int32_t(N);
    g.K = int32_t(K);
    g.tiles = int32_t(bt::ceil_div(N, bt::kTileN));
    g.steps = int32_t(bt::ceil_div(K, bt::kSuperK));
    return dispatch_gemm(g, false, workspace, workspace_bytes, stream);
}

extern "C" bt_status bt_ternary_matmul(int64_t M, int64_t N, int64_t K, const int8_t* xq,
                                       const float* xscale, const int32_t* xsum, const void* wdev,
                                       float w_scale, float* y, int32_t* acc, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
    return matmul_impl(M, N, K, xq, xscale, xsum, wdev, w_scale, nullptr, y, acc, workspace,
                       workspace_bytes, stream);
}

extern "C" bt_status bt_ternary_matmul_epilogue(int64_t M, int64_t N, int64_t K, const int8_t* xq,
                                                const float* xscale, const int32_t* xsum,
                                                const void* wdev, float w_scale,
                                                const bt_epilogue* epi, float* y, int32_t* acc,
                                                void* workspace, size_t workspace_bytes,
                                                hipStream_t stream) {
    return matmul_impl(M, N, K, xq, xscale, xsum, wdev, w_scale, epi, y, acc, workspace,
                       workspace_bytes, stream);
}

// ------------------------------------------------------------------ I8_S

static bool i8_nk_ok(int64_t N, int64_t K) { return bt_int8_repacked_bytes(N, K) != 0; }

extern "C" bt_status bt_repack_int8(const int8_t* w_dev, int64_t N, int64_t K, void* wdev,
                                    hipStream_t stream) {
    if (!w_dev || !wdev) return BT_ERR_NULL;
    if (!i8_nk_ok(N, K)) return BT_ERR_SHAPE;
    if (!bt::aligned16(w_dev) || !bt::aligned16(wdev)) return BT_ERR_ALIGN;
    const int64_t steps64 = bt::ceil_div(K, bt::kSuperK) * (bt::kSuperK / 64);
    const int64_t blocks = bt::ceil_div(N, bt::kTileN) * steps64;
    const int64_t grid = std::min<int64_t>(bt::ceil_div(blocks, 4), int64_t(1) << 20);
    (void)hipGetLastError();
    hipLaunchKernelGGL(repack_int8_kernel, dim3(unsigned(grid)), dim3(256), 0, stream, w_dev,
                       int32_t(N), int32_t(K), int32_t(steps64), blocks,
                       static_cast<int8_t*>(wdev));
    return launched();
}

extern "C" bt_status bt_int8_matmul(int64_t M, int64_t N, int64_t K, const int8_t* xq,
                                    const float* xscale, const void* w8dev, float w_scale,
                                    const bt_epilogue* epi, float* y, int32_t* acc,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!xq || !xscale || !w8dev || !y) return BT_ERR_NULL;
    if (M < 1 || M > (int64_t(1) << 31) - 1 || !i8_nk_ok(N, K)) return BT_ERR_SHAPE;
    if (!bt::aligned16(xq) || !bt::aligned16(xscale) || !bt::aligned16(w8dev) ||
        !bt::aligned16(y) || (acc && !bt::aligned16(acc)))
        return BT_ERR_ALIGN;
    if (!isfinite(w_scale)) return BT_ERR_VALUE;
    GemmArgs g;
    memset(&g, 0, sizeof(g));
    const bt_status est = epilogue_args(epi, M, N, y, &g.epi);
    if (est != BT_OK) return est;
    g.xq = xq;
    g.xscale = xscale;
    g.xsum = nullptr;
    g.w = static_cast<const uint8_t*>(w8dev);
    g.y = y;
    g.acc = acc;
    g.w_scale = w_scale;
    g.M = int32_t(M);
    g.N = int32_t(N);
    g.K = int32_t(K);
    g.tiles = int32_t(bt::ceil_div(N, bt::kTileN));
    g.steps = int32_t(bt::ceil_div(K, bt::kSuperK));
    return dispatch_gemm(g, true, workspace, workspace_bytes, stream);
}

extern "C" bt_status bt_quantize_act_grouped(const void* plan_host, const void* plan_dev,
                                             hipStream_t stream) {
    if (!plan_host || !plan_dev) return BT_ERR_NULL;
    const auto* hdr = static_cast<const bt::PlanHeader*>(plan_host);
    if (hdr->magic != bt::kPlanMagicQuant || hdr->count < 1) return BT_ERR_VALUE;
    if (!bt::aligned16(plan_dev)) return BT_ERR_ALIGN;
    const auto* descs = reinterpret_cast<const QuantDesc*>(static_cast<const char*>(plan_dev) +
                                                           sizeof(bt::PlanHeader));
    (void)hipGetLastError();
    hipLaunchKernelGGL(quantize_grouped_kernel, dim3(unsigned(hdr->total_blocks)),
                       dim3(bt::kQuantThreads), 0, stream, descs, hdr->count);
    return launched();
}

extern "C" bt_status bt_ternary_matmul_grouped(const void* plan_host, const void* plan_dev,
                                               hipStream_t stream) {
    if (!plan_host || !plan_dev) return BT_ERR_NULL;
    const auto* hdr = static_cast<const bt::PlanHeader*>(plan_host);
    const bool fused = hdr->magic == bt::kPlanMagicGemvFused;
    if ((!fused && hdr->magic != bt::kPlanMagicGemv) || hdr->count < 1) return BT_ERR_VALUE;
    if (!bt::aligned16(plan_dev)) return BT_ERR_ALIGN;
    const auto* host_descs = reinterpret_cast<const GemvDesc*>(hdr + 1);
    size_t lds = 0;
    for (int32_t i = 0; i < hdr->count; ++i) lds = std::max(lds, gemv_lds_bytes(host_descs[i]));
    const auto* descs = reinterpret_cast<const GemvDesc*>(static_cast<const char*>(plan_dev) +
                                                          sizeof(bt::PlanHeader));
    (void)hipGetLastError();
    if (fused)
        hipLaunchKernelGGL(gemv_grouped_kernel<true>, dim3(unsigned(hdr->total_blocks)),
                           dim3(64 * bt::kGemvWaves), lds, stream, descs, hdr->count);
    else
        hipLaunchKernelGGL(gemv_grouped_kernel<false>, dim3(unsigned(hdr->total_blocks)),
                           dim3(64 * bt::kGemvWaves), lds, stream, descs, hdr->count);
    return launched();
}
