// nosa_device.h -- small device helpers for gfx950 (wave64) kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nosa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ---- element conversions -------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float32 -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ float load_elem(const void *p, size_t i);
template <> __device__ __forceinline__ float load_elem<float>(const void *p, size_t i) {
    return ((const float *)p)[i];
}
template <> __device__ __forceinline__ float load_elem<uint16_t>(const void *p, size_t i) {
    return __uint_as_float((uint32_t)((const uint16_t *)p)[i] << 16);
}

template <typename T> __device__ __forceinline__ void store_elem(void *p, size_t i, float x);
template <> __device__ __forceinline__ void store_elem<float>(void *p, size_t i, float x) {
    ((float *)p)[i] = x;
}
template <> __device__ __forceinline__ void store_elem<uint16_t>(void *p, size_t i, float x) {
    ((uint16_t *)p)[i] = f32_to_bf16_rne(x);
}

// ---- cross-lane moves ----------------------------------------------------------------
// DPP controls (gfx9 encoding).
enum : int {
    kDppQuadXor1 = 0xB1,       // quad_perm [1,0,3,2]
    kDppQuadXor2 = 0x4E,       // quad_perm [2,3,0,1]
    kDppRowRor4 = 0x124,       // rotate right by 4 within a 16-lane row
    kDppRowRor8 = 0x128,       // rotate right by 8 within a 16-lane row (= lane ^ 8)
    kDppRowMirror = 0x140,     // lane i <- lane 15 - i within a row
    kDppRowHalfMirror = 0x141  // lane i <- lane 7 - i within each half row
};

template <int CTRL> __device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float xor_lane(float x, int mask) { return __shfl_xor(x, mask, 64); }

// Compiler-level ordering of LDS traffic between lanes of one wave.  The hardware executes a
// wave's LDS instructions in order, so only code motion has to be prevented.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Monotone map of float32 onto uint32 (larger float -> larger key), with -0 folded onto +0.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u << 1) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Number of active lanes below this one in a 64-bit lane mask.
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Agent-scope load: reads data published by other workgroups after an acquire fence.
__device__ __forceinline__ float load_agent(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Inclusive sum over the threads of a 256-thread workgroup, in thread order.
// Every thread of the workgroup must call it (it contains barriers).
__device__ __forceinline__ int block_incl_scan256(int v, int *ws4) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    if (lane == 63) ws4[w] = v;
    __syncthreads();
    int add = 0;
    for (int i = 0; i < w; ++i) add += ws4[i];
    __syncthreads();
    return v + add;
}

}  // namespace nosa
