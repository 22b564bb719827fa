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
//   tile t = 16 consecutive rows, 4*K bytes, stored contiguously;
//   inside a tile, 256-wide K steps S of 1 KB: lane l (row 16t + l%16,
//   K quarter l/16) owns bytes [16l, 16l+16) = four 32-bit words, word jj
//   holding K = 256S + 64jj + 16(l/16) + e, e = 0..15, with element e in
//   byte e%4 at bits 2*(e/4). A trailing 128-wide step (K % 256 == 128) is
//   512 B with 8 bytes per lane. So one 128-bit load per lane yields the
//   B fragments of four MFMA steps, and unpacking word jj is
//   (word >> 2s) & 0x03030303 for s = 0..3.

#include <hip/hip_runtime.h>

#include <float.h>
#include <math.h>

#include <algorithm>

#include "bt_internal.h"

#pragma clang fp contract(off)

namespace {

using bt::GemvDesc;
using bt::QuantDesc;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

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

// ------------------------------------------------------------------ repack

// One thread per output word. Word (tile t, step S, lane l, word jj) gathers
// the 16 codes of row 16t + l%16 at K = k0 .. k0+15, k0 = 256S + 64jj + 16(l/16).
// In the canonical layout those 16 elements share one bit pair (k0 % 128) / 32
// of 16 consecutive bytes starting at byte 32*(k0/128) + k0 % 32 of the row.
__global__ __launch_bounds__(256) void repack_kernel(const uint8_t* __restrict__ packed, int32_t N,
                                                     int32_t K, int64_t total_words,
                                                     uint32_t* __restrict__ out) {
    const int32_t full = K / bt::kSuperK;
    for (int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; gid < total_words;
         gid += int64_t(gridDim.x) * blockDim.x) {
        const int64_t t = gid / K;
        const int32_t d = int32_t(gid - t * K);
        const int32_t S = d >> 8;
        const int32_t rem = d & 255;
        int32_t lane, jj;
        if (S < full) {
            lane = rem >> 2;
            jj = rem & 3;
        } else {
            lane = rem >> 1;
            jj = rem & 1;
        }
        const int64_t n = t * bt::kTileN + (lane & 15);
        const int32_t k0 = bt::kSuperK * S + bt::kStepK * jj + 16 * (lane >> 4);
        uint32_t word = 0x55555555u;   // padding rows: code 1 = weight 0
        if (n < N) {
            const uint8_t* row = packed + n * (K / 4);
            const uint4 c = *reinterpret_cast<const uint4*>(row + 32 * (k0 >> 7) + (k0 & 31));
            const int sh = 2 * ((k0 & 127) >> 5);
            word = ((c.x >> sh) & kLow2) | (((c.y >> sh) & kLow2) << 2) |
                   (((c.z >> sh) & kLow2) << 4) | (((c.w >> sh) & kLow2) << 6);
        }
        out[gid] = word;
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

constexpr int kQuantRegs = 16;   // float4 per thread kept in registers: K <= 16384

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
// the row sum of q. With K % 4 == 0 and K <= 16384 the row stays in registers
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

constexpr int kGemvInFlight = 8;   // 1 KB weight loads in flight per wave

// One wave computes one 16-row tile over one K chunk. The A fragment of lane l
// is q[l%16][64j + 16(l/16) .. +15] (zero for tokens >= M); the B fragment is
// the unpacked word of that lane. The C fragment holds tokens 4(l/16)+i,
// output row l%16 of the tile.
__device__ __forceinline__ void gemv_wave(const GemvDesc& d, int64_t local_block) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t wg_per_chunk = (d.tiles + bt::kGemvWaves - 1) / bt::kGemvWaves;
    const int chunk = int(local_block / wg_per_chunk);
    const int tile = int(local_block - int64_t(chunk) * wg_per_chunk) * bt::kGemvWaves + wave;
    if (tile >= d.tiles) return;
    const int steps = d.full_steps + d.half_step;
    const int s0 = chunk * d.steps_per_chunk;
    const int s1 = min(s0 + d.steps_per_chunk, steps);
    const int s1_full = min(s1, d.full_steps);

    const uint8_t* wt = d.w + int64_t(tile) * 4 * d.K;
    const int am = lane & 15;
    const int kq = lane >> 4;
    const bool arow = am < d.M;
    const int8_t* xrow = d.xq + int64_t(am) * d.K + 16 * kq;
    v4i c = {0, 0, 0, 0};

    int S = s0;
    for (; S < s1_full; S += kGemvInFlight) {
        v4u w[kGemvInFlight];
#pragma unroll
        for (int u = 0; u < kGemvInFlight; ++u)
            if (S + u < s1_full)
                w[u] = __builtin_nontemporal_load(
                    reinterpret_cast<const v4u*>(wt + int64_t(S + u) * 1024 + lane * 16));
#pragma unroll
        for (int u = 0; u < kGemvInFlight; ++u) {
            if (S + u < s1_full) {
                const uint32_t ww[4] = {w[u][0], w[u][1], w[u][2], w[u][3]};
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    v4i a = {0, 0, 0, 0};
                    if (arow)
                        a = *reinterpret_cast<const v4i*>(xrow + int64_t(S + u) * 256 + 64 * jj);
                    c = mfma16x16x64(a, unpack16(ww[jj]), c);
                }
            }
        }
    }
    if (s1 > d.full_steps) {   // this chunk ends with the trailing 128-wide step
        S = d.full_steps;
        const v2u w = __builtin_nontemporal_load(
            reinterpret_cast<const v2u*>(wt + int64_t(S) * 1024 + lane * 8));
        const uint32_t ww[2] = {w[0], w[1]};
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            v4i a = {0, 0, 0, 0};
            if (arow) a = *reinterpret_cast<const v4i*>(xrow + int64_t(S) * 256 + 64 * jj);
            c = mfma16x16x64(a, unpack16(ww[jj]), c);
        }
    }

    const int n_local = lane & 15;
    const int n = tile * bt::kTileN + n_local;
    if (d.chunks > 1) {
        // Split K: add this chunk's partial sums (int32 addition is exact in
        // any order), and let the last chunk to arrive finish the tile.
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
                const int32_t acc = c[i] - d.xsum[mm];
                const float rs = d.xscale[mm] * d.w_scale;
                d.y[int64_t(mm) * d.N + n] = float(acc) * rs;
                if (d.acc) d.acc[int64_t(mm) * d.N + n] = acc;
            }
        }
    }
}

__global__ __launch_bounds__(64 * bt::kGemvWaves) void gemv_kernel(GemvDesc d) {
    gemv_wave(d, blockIdx.x);
}

__global__ __launch_bounds__(64 * bt::kGemvWaves) void gemv_grouped_kernel(
    const GemvDesc* __restrict__ descs, int32_t count) {
    const int64_t b = blockIdx.x;
    int lo = 0, hi = count - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (descs[mid].block_begin <= b) lo = mid; else hi = mid - 1;
    }
    const GemvDesc d = descs[lo];
    gemv_wave(d, b - d.block_begin);
}

// -------------------------------------------------------------------- GEMM

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kALds = bt::kSuperK + 16;   // padded LDS row: 16 lanes hit distinct banks

struct GemmArgs {
    const int8_t* xq;
    const float* xscale;
    const int32_t* xsum;
    const uint8_t* w;
    float* y;
    int32_t* acc;
    float w_scale;
    int32_t M, N, K, tiles, full_steps, half_step;
};

// 128 x 128 output tile per workgroup, 4 waves as 2 x 2, each wave 64 x 64 =
// 4 x 4 MFMA blocks. Per 256-wide K step the activation tile (128 x 256 int8)
// is staged in LDS and each wave loads the packed words of its four 16-row
// weight tiles straight from global memory (one 128-bit load per tile).
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) int8_t As[kBM * kALds];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int64_t m0 = int64_t(blockIdx.y) * kBM;
    const int n0 = blockIdx.x * kBN;
    const int t0 = n0 / bt::kTileN + wn * 4;

    v4i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    const int steps = g.full_steps + g.half_step;
    for (int S = 0; S < steps; ++S) {
        const bool half = S >= g.full_steps;
        uint4 wb[4];
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) {
            const int t = t0 + tn;
            wb[tn] = uint4{0, 0, 0, 0};
            if (t < g.tiles) {
                const uint8_t* base = g.w + int64_t(t) * 4 * g.K + int64_t(S) * 1024;
                if (!half) {
                    wb[tn] = *reinterpret_cast<const uint4*>(base + lane * 16);
                } else {
                    const uint2 h = *reinterpret_cast<const uint2*>(base + lane * 8);
                    wb[tn].x = h.x;
                    wb[tn].y = h.y;
                }
            }
        }
        const int kw = half ? 128 : 256;
        const int cpr = kw / 16;   // 16-byte chunks per row
        __syncthreads();
        for (int ch = tid; ch < kBM * cpr; ch += 256) {
            const int r = ch / cpr;
            const int col = (ch - r * cpr) * 16;
            const int64_t gm = m0 + r;
            int4 v = {0, 0, 0, 0};
            if (gm < g.M)
                v = *reinterpret_cast<const int4*>(g.xq + gm * g.K + int64_t(S) * 256 + col);
            *reinterpret_cast<int4*>(As + r * kALds + col) = v;
        }
        __syncthreads();
        const int nj = half ? 2 : 4;
        for (int jj = 0; jj < nj; ++jj) {
            v4i bf[4];
#pragma unroll
            for (int tn = 0; tn < 4; ++tn) {
                const uint32_t word = jj == 0 ? wb[tn].x : jj == 1 ? wb[tn].y : jj == 2 ? wb[tn].z : wb[tn].w;
                bf[tn] = unpack16(word);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const v4i af = *reinterpret_cast<const v4i*>(
                    As + (wm * 64 + 16 * i + (lane & 15)) * kALds + 64 * jj + 16 * (lane >> 4));
#pragma unroll
                for (int tn = 0; tn < 4; ++tn) acc[i][tn] = mfma16x16x64(af, bf[tn], acc[i][tn]);
            }
        }
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t mm = m0 + wm * 64 + 16 * i + 4 * (lane >> 4) + r;
            if (mm >= g.M) continue;
            const int32_t qs = g.xsum[mm];
            const float rs = g.xscale[mm] * g.w_scale;
#pragma unroll
            for (int tn = 0; tn < 4; ++tn) {
                const int n = n0 + wn * 64 + 16 * tn + (lane & 15);
                if (n < g.N) {
                    const int32_t a = acc[i][tn][r] - qs;
                    g.y[mm * g.N + n] = float(a) * rs;
                    if (g.acc) g.acc[mm * g.N + n] = a;
                }
            }
        }
    }
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
    const int64_t tiles = bt::ceil_div(N, bt::kTileN);
    const int64_t words = tiles * K;
    const int64_t blocks = std::min<int64_t>(bt::ceil_div(words, 256), int64_t(1) << 20);
    (void)hipGetLastError();
    hipLaunchKernelGGL(repack_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, packed_dev,
                       int32_t(N), int32_t(K), words, static_cast<uint32_t*>(wdev));
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
    hipLaunchKernelGGL(quantize_kernel, dim3(unsigned(M)), dim3(bt::kQuantThreads), 0, stream, x, K,
                       xq, xscale, xsum);
    return launched();
}

extern "C" bt_status bt_ternary_matmul(int64_t M, int64_t N, int64_t K, const int8_t* xq,
                                       const float* xscale, const int32_t* xsum, const void* wdev,
                                       float w_scale, float* y, int32_t* acc, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
    if (!xq || !xscale || !xsum || !wdev || !y) return BT_ERR_NULL;
    if (M < 1 || M > (int64_t(1) << 31) - 1 || !nk_ok(N, K)) return BT_ERR_SHAPE;
    if (!bt::aligned16(xq) || !bt::aligned16(xscale) || !bt::aligned16(xsum) ||
        !bt::aligned16(wdev) || !bt::aligned16(y) || (acc && !bt::aligned16(acc)))
        return BT_ERR_ALIGN;
    if (!isfinite(w_scale)) return BT_ERR_VALUE;
    if (M <= BT_GEMV_MAX_M) {
        GemvDesc d;
        bt::gemv_shape(M, N, K, &d);
        const size_t need = bt::gemv_workspace_bytes(d);
        if (need) {
            if (!workspace || workspace_bytes < need) return BT_ERR_WORKSPACE;
            if (!bt::aligned16(workspace)) return BT_ERR_ALIGN;
            const size_t partial =
                (size_t(d.M) * size_t(d.tiles) * bt::kTileN * sizeof(int32_t) + 255) & ~size_t(255);
            d.ws = static_cast<int32_t*>(workspace);
            d.cnt = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + partial);
        }
        d.xq = xq;
        d.xscale = xscale;
        d.xsum = xsum;
        d.w = static_cast<const uint8_t*>(wdev);
        d.y = y;
        d.acc = acc;
        d.w_scale = w_scale;
        (void)hipGetLastError();
        hipLaunchKernelGGL(gemv_kernel, dim3(unsigned(d.blocks)), dim3(64 * bt::kGemvWaves), 0,
                           stream, d);
        return launched();
    }
    GemmArgs g;
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
    g.full_steps = int32_t(K / bt::kSuperK);
    g.half_step = int32_t((K % bt::kSuperK) != 0);
    const int64_t gy = bt::ceil_div(M, kBM);
    if (gy > 65535) return BT_ERR_SHAPE;
    (void)hipGetLastError();
    hipLaunchKernelGGL(gemm_kernel, dim3(unsigned(bt::ceil_div(N, kBN)), unsigned(gy)), dim3(256), 0,
                       stream, g);
    return launched();
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
    if (hdr->magic != bt::kPlanMagicGemv || hdr->count < 1) return BT_ERR_VALUE;
    if (!bt::aligned16(plan_dev)) return BT_ERR_ALIGN;
    const auto* descs = reinterpret_cast<const GemvDesc*>(static_cast<const char*>(plan_dev) +
                                                          sizeof(bt::PlanHeader));
    (void)hipGetLastError();
    hipLaunchKernelGGL(gemv_grouped_kernel, dim3(unsigned(hdr->total_blocks)),
                       dim3(64 * bt::kGemvWaves), 0, stream, descs, hdr->count);
    return launched();
}
