// Hardware ceilings measured on the part itself: the int8 matrix-core issue
// rate (v_mfma_i32_16x16x64_i8, the instruction the ternary matmul uses) with
// the shader clock it ran at, and plain streaming-read bandwidth. Declared in
// include/bt_ceilings.h; a library of its own, not part of the matmul path.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "bt_ceilings.h"

namespace {

typedef int32_t v4i __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;   // independent accumulators per wave

// Eight independent dependency chains per wave and several waves per SIMD:
// enough instructions in flight that the matrix core, not their latency, sets
// the rate. Operands live in registers; nothing is loaded inside the loop.
// The occupancy attribute keeps the accumulators in ordinary registers (the
// instruction's VGPR form): without it the compiler placed them in AGPRs and
// shuffled them between iterations, halving the measured rate.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4)))
void mfma_issue_kernel(int iters, int32_t a_word,
                                                         int32_t b_word, int32_t* out,
                                                         int64_t* clocks) {
    const v4i a = {a_word, a_word, a_word, a_word};
    const v4i b = {b_word, b_word, b_word, b_word};
    v4i c[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) c[j] = v4i{0, 0, 0, 0};
    const bool rec = blockIdx.x == 0 && threadIdx.x == 0;
    int64_t t0 = 0, w0 = 0;
    if (rec) {
        t0 = clock64();
        w0 = wall_clock64();
    }
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < kChains; ++j)
            c[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c[j], 0, 0, 0);
    }
    if (rec) {
        clocks[0] = t0;
        clocks[1] = w0;
        clocks[2] = clock64();
        clocks[3] = wall_clock64();
    }
    uint32_t s = 0;   // wrapping sum
#pragma unroll
    for (int j = 0; j < kChains; ++j)
        s += uint32_t(c[j].x) + uint32_t(c[j].y) + uint32_t(c[j].z) + uint32_t(c[j].w);
    out[int64_t(blockIdx.x) * 256 + threadIdx.x] = int32_t(s);
}

// Grid-stride streaming read, eight 16-byte non-temporal loads in flight per
// thread; the XOR of everything a wave read goes out so that no load is dead.
__global__ __launch_bounds__(256) void stream_read_kernel(const v4u* __restrict__ p, int64_t n,
                                                          v4u* __restrict__ out) {
    constexpr int U = 8;
    v4u acc = {0, 0, 0, 0};
    const int64_t stride = int64_t(gridDim.x) * 256;
    int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    // every index in the unrolled body is at most i + (U - 1) * stride < n
    for (; i + (U - 1) * stride < n; i += U * stride) {
        v4u v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    for (; i < n; i += stride) acc ^= __builtin_nontemporal_load(p + i);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        acc.x ^= uint32_t(__shfl_xor(int(acc.x), off));
        acc.y ^= uint32_t(__shfl_xor(int(acc.y), off));
        acc.z ^= uint32_t(__shfl_xor(int(acc.z), off));
        acc.w ^= uint32_t(__shfl_xor(int(acc.w), off));
    }
    if ((threadIdx.x & 63) == 0) out[int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6)] = acc;
}

int launch_status() { return hipGetLastError() == hipSuccess ? 0 : 5; }

}  // namespace

extern "C" int btc_mfma_i8_issue(int blocks, int iters, int8_t a_byte, int8_t b_byte,
                                 int32_t* out, int64_t* clocks, hipStream_t stream) {
    if (!out || !clocks) return 1;
    if (blocks < 1 || blocks > 65536 || iters < 1 || iters > (1 << 20)) return 2;
    const uint32_t ab = uint32_t(uint8_t(a_byte)) * 0x01010101u;
    const uint32_t bb = uint32_t(uint8_t(b_byte)) * 0x01010101u;
    (void)hipGetLastError();
    hipLaunchKernelGGL(mfma_issue_kernel, dim3(blocks), dim3(256), 0, stream, iters, int32_t(ab),
                       int32_t(bb), out, clocks);
    return launch_status();
}

extern "C" int btc_wall_clock_khz(int device) {
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, device) != hipSuccess) return -1;
    return khz;
}

extern "C" int btc_stream_read(const void* p, int64_t bytes, int blocks, uint32_t* out,
                               hipStream_t stream) {
    if (!p || !out) return 1;
    if (bytes < 16 || bytes % 16 != 0 || bytes > (int64_t(1) << 40) || blocks < 1 ||
        blocks > 65536 || reinterpret_cast<uintptr_t>(p) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(out) % 16 != 0)
        return 2;
    (void)hipGetLastError();
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, stream,
                       static_cast<const v4u*>(p), bytes / 16, reinterpret_cast<v4u*>(out));
    return launch_status();
}
