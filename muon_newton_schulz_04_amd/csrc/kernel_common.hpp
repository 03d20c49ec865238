// Device helpers shared by the libmuon kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_types.hpp"

namespace muon {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Two floats rounded to bf16 (nearest even) and packed, lo in bits 0..15: one
// two-wide conversion, which gfx950 does in one v_cvt_pk_bf16_f32.
typedef float f32x2_cvt __attribute__((ext_vector_type(2)));
typedef bf16 bf16x2_cvt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_cvt f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_cvt));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Wave-wide sum with a fixed butterfly order (deterministic).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Block-wide sum for 256 threads; every thread gets the same value.
// Deterministic: fixed per-wave butterfly, then waves summed in index order.
__device__ __forceinline__ float block_sum_256(float v, float* red /* >= 4 floats of LDS */) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float t = ((red[0] + red[1]) + red[2]) + red[3];
    return t;
}

}  // namespace muon
