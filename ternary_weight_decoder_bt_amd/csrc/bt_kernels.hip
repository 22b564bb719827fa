// Device half of libbt for gfx950 (CDNA4): weight repack, per-token INT8
// quantization (plain and fused with RMS normalization), the decode GEMV
// (M <= 16) and the C ABI of the device entry points. The prefill GEMM
// (M > 16) is in bt_gemm.hip, the offline ternarization in bt_ternarize.hip.
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
#include <mutex>
#include <type_traits>

#include "bt_device.h"

#pragma clang fp contract(off)

namespace {

using bt::GemmArgs;
using bt::GemvDesc;
using bt::QuantDesc;

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

constexpr int kRepackPerWave = 8;   // output blocks a wave handles per pass

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

// Row m quantized by one wave (K % 4 == 0, K <= 2048).
__device__ __forceinline__ void quantize_wave_row(const float* __restrict__ x, int64_t K,
                                                  int64_t m, int8_t* __restrict__ xq,
                                                  float* __restrict__ xscale,
                                                  int32_t* __restrict__ xsum) {
    const int lane = threadIdx.x & 63;
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

__global__ __launch_bounds__(bt::kQuantThreads) void quantize_wave_rows_kernel(
    const float* __restrict__ x, int64_t M, int64_t K, int8_t* __restrict__ xq,
    float* __restrict__ xscale, int32_t* __restrict__ xsum) {
    const int64_t m = int64_t(blockIdx.x) * (bt::kQuantThreads / 64) + (threadIdx.x >> 6);
    if (m >= M) return;
    quantize_wave_row(x, K, m, xq, xscale, xsum);
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

// Many quantizations in one launch. A workgroup finds its problem with one
// lane per descriptor (first workgroups compared at once, counted with a
// ballot), then quantizes four rows, one per wave, where the rows are short
// (K % 4 == 0, K <= 2048), else one row with the whole workgroup.
__global__ __launch_bounds__(bt::kQuantThreads) void quantize_grouped_kernel(
    const QuantDesc* __restrict__ descs, int32_t count) {
    __shared__ QuantShared sh;
    const int64_t b = blockIdx.x;
    const int lane = threadIdx.x & 63;
    int p = -1;
    for (int base = 0; base < count; base += 64) {
        const int i = base + lane;
        const int64_t begin = i < count ? descs[i].row_begin : INT64_MAX;
        p += int(__popcll(__ballot(begin <= b)));
    }
    p = __builtin_amdgcn_readfirstlane(p);
    const QuantDesc d = descs[p];
    const int64_t local = b - d.row_begin;
    if (bt::quant_wave_rows(d.K)) {
        const int64_t m = local * (bt::kQuantThreads / 64) + (threadIdx.x >> 6);
        if (m < d.M) quantize_wave_row(d.x, d.K, m, d.xq, d.xscale, d.xsum);
        return;
    }
    quantize_row(d.x + local * d.K, d.K, d.xq + local * d.K, d.xscale + local,
                 d.xsum + local, sh);
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
// `wl` is the lane whose 16 bytes this lane loads: itself, or with row parts a
// lane of the same K piece in the workgroup's own rows (two lanes then read one
// address, which costs one fetch).
__device__ __forceinline__ void gemv_issue(GemvBatch& b, const uint8_t* wt, int sb, int last,
                                           int wl) {
#pragma unroll
    for (int u = 0; u < kB; ++u) {
        const int st = min(sb + u, last);
        b.w[u] = gld_stream<v4u>(wt + int64_t(st) * 1024 + wl * 16);
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
// arrive reads the total, clears the workspace and finishes the tile. Every
// access to the shared words (partial sums and arrival counters) is an atomic,
// performed where all compute units and XCDs see it; a chunk waits until its
// additions have completed before it counts itself in, and the last chunk
// reads the totals with atomics after its count came back. No fence is needed:
// a device-scope fence would add a write-back and invalidation of the L2 for
// plain stores, which none of this uses, and costs more than the whole
// product for a 16-token batch (measured: the down projection 16.5 -> 1.4 us
// per layer without it).
__device__ __forceinline__ void gemv_finish(const GemvDesc& d, int64_t tile, v4i c, int lane,
                                            const GemvShared& sh, int chunk, bool own_row) {
    // With row parts (single calls only), a lane outside the workgroup's rows
    // holds a copy of another row's sums and stores nothing. Plans never split
    // rows, so every lane of a plan's wave reaches the atomics below.
    if (!own_row) return;
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
        // the additions complete (are performed) before the count goes out
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0);
        asm volatile("" ::: "memory");
        uint32_t prev = 0;
        if (lane == 0) prev = atomicAdd(d.cnt + tile, 1u);
        prev = __shfl(prev, 0, 64);
        if (prev != uint32_t(d.chunks - 1)) return;
        asm volatile("" ::: "memory");
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
// Rows up to R*1024 elements (R float4 per thread) are read once into
// registers; token 0 is read before the first weight loads go out, so its
// data is not queued behind them (a wave's vector loads return in order).
// Longer rows are read twice (absmax, then quantize). Grouped launches hold
// R = 2 (K <= 2048); single calls take R = 9 for rows up to 9216 elements.
constexpr int kFusedRegs = 2;       // grouped launches: K <= 2048 in one read
constexpr int kFusedRegsLong = 9;   // single calls with 2048 < K <= 9216
constexpr int kGemvThreads = 64 * bt::kGemvWaves;

template <int R>
struct FusedRow {
    v4f v[R];
};

template <int R>
__device__ __forceinline__ void gemv_load_row(FusedRow<R>& r, const GemvDesc& d, int m) {
    const int64_t K4 = d.K >> 2;
    const float* xr = d.x + int64_t(m) * d.K;
#pragma unroll
    for (int j = 0; j < R; ++j) {
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
template <int R>
__device__ __forceinline__ void gemv_quant_short_row(const FusedRow<R>& r, int m, const GemvDesc& d,
                                                     bool writer, int64_t kbeg, int64_t kend,
                                                     int8_t* lds, GemvShared& sh) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int64_t K4 = d.K >> 2;
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < R; ++j) {
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
    for (int j = 0; j < R; ++j) {
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
template <int R>
__device__ __forceinline__ void gemv_quantize_rows(const GemvDesc& d, const FusedRow<R>& r0,
                                                   bool writer, int64_t kbeg, int64_t kend,
                                                   int8_t* lds, GemvShared& sh) {
    const int tid = threadIdx.x;
    constexpr int T = kGemvThreads;
    const int64_t K4 = d.K >> 2;   // K % 128 == 0
    if (K4 <= int64_t(R) * T) {
        gemv_quant_short_row(r0, 0, d, writer, kbeg, kend, lds, sh);
        for (int m = 1; m < d.M; ++m) {
            FusedRow<R> r;
            gemv_load_row(r, d, m);
            gemv_quant_short_row(r, m, d, writer, kbeg, kend, lds, sh);
        }
    } else {
        // Long rows, read twice (absmax, then quantize), kLongBatch float4 per
        // thread in flight at a time: loads at clamped indices, unconditional,
        // so each batch costs one round trip rather than one per float4.
        constexpr int kLongBatch = 4;
        for (int m = 0; m < d.M; ++m) {
            const float* xr = d.x + int64_t(m) * d.K;
            float amax = 0.0f;
            for (int64_t i0 = tid; i0 < K4; i0 += int64_t(kLongBatch) * T) {
                v4f v[kLongBatch];
#pragma unroll
                for (int u = 0; u < kLongBatch; ++u)
                    v[u] = gld<v4f>(xr + 4 * min(i0 + int64_t(u) * T, K4 - 1));
#pragma unroll
                for (int u = 0; u < kLongBatch; ++u)
                    if (i0 + int64_t(u) * T < K4)
                        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)),
                                                 fmaxf(fabsf(v[u].z), fabsf(v[u].w))));
            }
            amax = block_max(amax, sh.red);
            float inv = 127.0f / amax;
            const bool dead = !(inv <= FLT_MAX);
            if (dead) inv = 0.0f;
            int s = 0;
            for (int64_t i0 = tid; i0 < K4; i0 += int64_t(kLongBatch) * T) {
                v4f v[kLongBatch];
#pragma unroll
                for (int u = 0; u < kLongBatch; ++u)
                    v[u] = gld<v4f>(xr + 4 * min(i0 + int64_t(u) * T, K4 - 1));
#pragma unroll
                for (int u = 0; u < kLongBatch; ++u) {
                    const int64_t i = i0 + int64_t(u) * T;
                    if (i < K4)
                        s += gemv_quant_store(v[u], inv, 4 * i, m, writer, d, kbeg, kend, lds);
                }
            }
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

// Activation pieces (16 bytes of one token row) a thread of a single call
// loads into registers before the weight loads go out: with the weights first,
// every staging load would wait for them (in-order return) and each further
// round of staging loads would add a round trip. Four cover a whole row of up
// to 16384 elements.
constexpr int kEarlyPieces = 4;

template <bool kFused, bool kWaveSplit, int R>
__device__ __forceinline__ void gemv_block(const GemvDesc& d, int64_t local_block, int8_t* lds,
                                           GemvShared& sh) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int chunk = int(local_block / d.groups);
    const int64_t gp = local_block - int64_t(chunk) * d.groups;
    // row part `part` of the tiles of workgroup group g: weight rows
    // [part * rp, (part + 1) * rp) of each 16-row tile
    // (grouped launches never split rows: their count is fixed at 1 here)
    const int parts = kWaveSplit ? d.row_parts : 1;
    const int64_t g = gp / parts;
    const int part = int(gp - g * parts);
    const int rp = bt::kTileN / parts;
    const int wl = (lane & ~15) | (part * rp + (lane & 15) % rp);
    const bool own_row = (lane & 15) / rp == part;
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
        gemv_issue(b, d.w + t * tile_bytes, ws0 + bb * kB, ws1 - 1, wl);
    };

    // The first weight batches go out before the activations are staged, so
    // their latency overlaps the staging. Fused: token 0's activations go out
    // first, and the second batch waits until the rows are quantized (the
    // registers it needs hold the activations until then).
    // Stage this chunk of the M token rows in LDS rows 0..M-1 (zero past K)
    // and a zero row M, which the lanes of tokens >= M read instead.
    const int64_t kbeg = int64_t(s0) * bt::kSuperK;
    const int64_t kend = int64_t(s1) * bt::kSuperK;
    const int pieces = nsteps * (bt::kSuperK / 16);
    const int real_pieces = d.M * pieces;
    // single calls: the first pieces of the unfused activations go out before
    // the weights (addresses clamped into the row, so the loads are
    // unconditional; a piece past the rows or past K is stored as zero)
    constexpr bool kEarly = kWaveSplit && !kFused;
    v4i early[kEarly ? kEarlyPieces : 1];
    float early_d = 0.0f;
    int32_t early_qs = 0;
    if constexpr (kEarly) {
#pragma unroll
        for (int j = 0; j < kEarlyPieces; ++j) {
            const int i = min(tid + j * kGemvThreads, real_pieces - 1);
            const int m = i / pieces;
            const int64_t col = min(int64_t(i - m * pieces) * 16, int64_t(d.K) - kbeg - 16);
            early[j] = gld<v4i>(d.xq + int64_t(m) * d.K + kbeg + col);
        }
        // the epilogue's per-token scale and row sum, too
        early_d = gld<float>(d.xscale + min(tid, d.M - 1));
        early_qs = gld<int32_t>(d.xsum + min(tid, d.M - 1));
        // keep these loads ahead of the weights' (the compiler may not sink them)
        __builtin_amdgcn_sched_barrier(0);
    }
    FusedRow<R> r0;
    if (kFused) gemv_load_row(r0, d, 0);
    // Single calls: keep token 0's loads ahead of the weights' (left to itself,
    // the compiler issued the long-row kernel's weight loads first, and the row
    // then waited for them); grouped launches already keep this order.
    if constexpr (kFused && kWaveSplit) __builtin_amdgcn_sched_barrier(0);
    GemvBatch b0, b1;
    issue(b0, 0);
    if (!kFused) issue(b1, min(1, total - 1));
    if constexpr (kEarly) __builtin_amdgcn_sched_barrier(0);

    if (kFused) {
        for (int i = tid; i < (d.M + 1) * pieces; i += 64 * bt::kGemvWaves) {
            const int m = i / pieces;
            const int col = (i - m * pieces) * 16;
            if (m == d.M || kbeg + col >= d.K) lds_st<v4i>(lds + m * d.lds_row + col, v4i{0, 0, 0, 0});
        }
        gemv_quantize_rows(d, r0, chunk == 0 && gp == 0, kbeg, kend, lds, sh);
        issue(b1, min(1, total - 1));
    } else {
        int first = 0;
        if constexpr (kEarly) {
#pragma unroll
            for (int j = 0; j < kEarlyPieces; ++j) {
                const int i = tid + j * kGemvThreads;
                if (i < real_pieces) {
                    const int m = i / pieces;
                    const int col = (i - m * pieces) * 16;
                    lds_st<v4i>(lds + m * d.lds_row + col,
                                kbeg + col < d.K ? early[j] : v4i{0, 0, 0, 0});
                }
            }
            first = kEarlyPieces * kGemvThreads;
            for (int i = tid; i < pieces; i += kGemvThreads)   // the zero row M
                lds_st<v4i>(lds + d.M * d.lds_row + i * 16, v4i{0, 0, 0, 0});
        }
        const int staged = kEarly ? real_pieces : (d.M + 1) * pieces;
        for (int i = first + tid; i < staged; i += kGemvThreads) {
            const int m = i / pieces;
            const int col = (i - m * pieces) * 16;
            v4i v = {0, 0, 0, 0};
            if (m < d.M && kbeg + col < d.K) v = gld<v4i>(d.xq + int64_t(m) * d.K + kbeg + col);
            lds_st<v4i>(lds + m * d.lds_row + col, v);
        }
        // the epilogue's per-token scale and row sum, read once
        if (tid < d.M) {
            sh.d[tid] = kEarly ? early_d : gld<float>(d.xscale + tid);
            sh.qs[0][tid] = kEarly ? early_qs : gld<int32_t>(d.xsum + tid);
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
            gemv_finish(d, t, cur, lane, sh, chunk, own_row);
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
            gemv_finish(d, tile0, cur, lane, sh, chunk, own_row);
        }
    }
}

// Single calls: waves_per_tile may split a tile's K range over the workgroup;
// R float4 per thread hold a fused call's token row.
template <bool kFused, int R = kFusedRegs>
__global__ __launch_bounds__(64 * bt::kGemvWaves) __attribute__((amdgpu_waves_per_eu(R > kFusedRegs ? 2 : 4))) void gemv_kernel(GemvDesc d) {
    extern __shared__ __attribute__((aligned(16))) int8_t gemv_lds[];
    __shared__ GemvShared sh;
    gemv_block<kFused, true, R>(d, blockIdx.x, gemv_lds, sh);
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
    gemv_block<kFused, false, kFusedRegs>(d, b - d.block_begin, gemv_lds, sh);
}

size_t gemv_lds_bytes(const GemvDesc& d) {
    const size_t rows = size_t(d.M + 1) * size_t(d.lds_row);
    // waves_per_tile > 1 reuses the activation space for the waves' partial sums
    return d.waves_per_tile > 1 ? std::max(rows, size_t(bt::kGemvWaves) * 64 * 16) : rows;
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
    return bt::gemm_reduce_slices(g, stream);
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
    bt::gemv_shape(M, N, K, false, false, &d);
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
    if (K > 4 * kFusedRegs * kGemvThreads && K <= 4 * kFusedRegsLong * kGemvThreads)
        hipLaunchKernelGGL((gemv_kernel<true, kFusedRegsLong>), dim3(unsigned(d.blocks)),
                           dim3(64 * bt::kGemvWaves), gemv_lds_bytes(d), stream, d);
    else
        hipLaunchKernelGGL((gemv_kernel<true, kFusedRegs>), dim3(unsigned(d.blocks)),
                           dim3(64 * bt::kGemvWaves), gemv_lds_bytes(d), stream, d);
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

// Argument checks of bt_ternary_matmul (everything but the workspace).
static bt_status matmul_check(int64_t M, int64_t N, int64_t K, const int8_t* xq,
                              const float* xscale, const int32_t* xsum, const void* wdev,
                              float w_scale, const float* y, const int32_t* acc) {
    if (!xq || !xscale || !xsum || !wdev || !y) return BT_ERR_NULL;
    if (M < 1 || M > (int64_t(1) << 31) - 1 || !nk_ok(N, K)) return BT_ERR_SHAPE;
    if (!bt::aligned16(xq) || !bt::aligned16(xscale) || !bt::aligned16(xsum) ||
        !bt::aligned16(wdev) || !bt::aligned16(y) || (acc && !bt::aligned16(acc)))
        return BT_ERR_ALIGN;
    if (!isfinite(w_scale)) return BT_ERR_VALUE;
    return BT_OK;
}

static bt_status matmul_impl(int64_t M, int64_t N, int64_t K, const int8_t* xq,
                             const float* xscale, const int32_t* xsum, const void* wdev,
                             float w_scale, const bt_epilogue* epi, float* y, int32_t* acc,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const bt_status cst = matmul_check(M, N, K, xq, xscale, xsum, wdev, w_scale, y, acc);
    if (cst != BT_OK) return cst;
    EpiArgs e;
    const bt_status est = epilogue_args(epi, M, N, y, &e);
    if (est != BT_OK) return est;
    if (M <= BT_GEMV_MAX_M) {
        GemvDesc d;
        bt::gemv_shape(M, N, K, false, true, &d);
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
    return bt::gemm_dispatch(g, false, workspace, workspace_bytes, stream);
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

// ------------------------------------------- allocation-free matmul entry point
//
// For callers that cannot allocate (code under graph capture, serving loops,
// harnesses that forbid it): bt_ternary_matmul with the split-K workspace
// taken from a fixed device array of this library instead of the caller.
// Each GPU holds its own copy of the array (from the library's load until the
// process ends); its address on a device is looked up once, with that device
// current, and kept. Nothing in it has to start at zero: every K range writes
// its whole partial-sum slice before the reduction launch reads it, so the
// previous call's contents do no harm. Calls that overlap in time on one GPU
// (different streams without ordering) share the array and race.
constexpr size_t kScratchBytes = BT_NOALLOC_SCRATCH_BYTES;
constexpr int kScratchDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

struct ScratchSlot {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchSlot scratch_slots[kScratchDevices];

// The device address of `scratch` on the current device.
bt_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices)
        return BT_ERR_DEVICE;
    ScratchSlot& slot = scratch_slots[dev];
    std::call_once(slot.once, [&slot] {
        void* p = nullptr;
        slot.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        slot.ptr = p;
    });
    if (slot.err != hipSuccess || !slot.ptr) return BT_ERR_DEVICE;
    *out = slot.ptr;
    return BT_OK;
}

}  // namespace

extern "C" bt_status bt_ternary_matmul_noalloc(int64_t M, int64_t N, int64_t K, const int8_t* xq,
                                               const float* xscale, const int32_t* xsum,
                                               const void* wdev, float w_scale, float* y,
                                               int32_t* acc, hipStream_t stream) {
    const bt_status cst = matmul_check(M, N, K, xq, xscale, xsum, wdev, w_scale, y, acc);
    if (cst != BT_OK) return cst;
    const size_t need = bt_matmul_workspace_bytes(M, N, K);
    if (need > kScratchBytes) return BT_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need) {
        const bt_status st = scratch_address(&ws);
        if (st != BT_OK) return st;
    }
    return matmul_impl(M, N, K, xq, xscale, xsum, wdev, w_scale, nullptr, y, acc, ws,
                       ws ? kScratchBytes : 0, stream);
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
    return bt::gemm_dispatch(g, true, workspace, workspace_bytes, stream);
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
    if (hdr->magic == bt::kPlanMagicGemm && hdr->count >= 1) {
        if (!bt::aligned16(plan_dev)) return BT_ERR_ALIGN;
        return bt::gemm_grouped_launch(hdr, plan_dev, stream);
    }
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
