// kda_device.h -- device-side helpers shared by the libkda kernels (gfx950).
//
// Wave64 DPP reductions, bf16 <-> f32 conversion and MFMA vector types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- bf16 -----
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Two floats to packed bf16 (low half = a), round to nearest even, on the
// hardware converter (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{a, b}), b2));
}

// hi + lo split of two floats: hi = bf16(x), lo = bf16(x - hi); packed pairs.
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
    hi = pack_bf16(a, b);
    lo = pack_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// Element loaders: float or bf16 (carried as uint16_t) to float.
template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float* p) { return *p; }
    static __device__ __forceinline__ f32x4 load4(const float* p) {
        return *reinterpret_cast<const f32x4*>(p);
    }
    static __device__ __forceinline__ void store(float* p, float x) { *p = x; }
};
template <> struct Elem<uint16_t> {
    static __device__ __forceinline__ float load(const uint16_t* p) { return bf16_bits_to_f32(*p); }
    static __device__ __forceinline__ f32x4 load4(const uint16_t* p) {
        const u16x4 b = *reinterpret_cast<const u16x4*>(p);
        return f32x4{bf16_bits_to_f32(b[0]), bf16_bits_to_f32(b[1]), bf16_bits_to_f32(b[2]),
                     bf16_bits_to_f32(b[3])};
    }
    static __device__ __forceinline__ void store(uint16_t* p, float x) { *p = f32_to_bf16_bits(x); }
};

// ----------------------------------------------------------------- DPP -----
// GFX9 DPP controls: quad_perm(1,0,3,2) swaps neighbours, quad_perm(2,3,0,1)
// swaps pairs, row_half_mirror reverses each group of 8 lanes.
constexpr int DPP_QUAD_XOR1 = 0xB1;
constexpr int DPP_QUAD_XOR2 = 0x4E;
constexpr int DPP_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of 8 lanes; every lane of the group gets the sum.
__device__ __forceinline__ float sum8(float x) {
    x += dpp_mov<DPP_QUAD_XOR1>(x);
    x += dpp_mov<DPP_QUAD_XOR2>(x);
    x += dpp_mov<DPP_HALF_MIRROR>(x);
    return x;
}

// Sum over each aligned group of 16 lanes (a DPP row).
__device__ __forceinline__ float sum16(float x) {
    x = sum8(x);
    x += dpp_mov<DPP_ROW_MIRROR>(x);
    return x;
}

// Workgroup barrier that orders LDS only.  __syncthreads() also orders global
// memory, which makes every wave wait for its outstanding global loads and
// stores (the next chunk's prefetch, the output stores) at each barrier.
__device__ __forceinline__ void block_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace kda
