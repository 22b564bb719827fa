// Device helpers shared by the HIP sources of libbt (gfx950): vector types,
// the 2-bit unpack, the int8 matrix-core step, global / buffer / LDS access
// wrappers and the fp32 epilogue's per-column steps. Every translation unit
// gets its own copy (unnamed namespace).
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "bt_internal.h"

// every fp32 step is its own rounding (no fused multiply-add)
#pragma clang fp contract(off)

namespace {

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

}  // namespace
