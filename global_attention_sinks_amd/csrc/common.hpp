// Device-side helpers shared by the gfx950 kernels of the attention hot path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mimo {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kDqk = 192;     // q/k head dim
constexpr int kDv = 128;      // v head dim
constexpr int kRope = 64;     // rotated dims (first 64)
constexpr int kPairs = 32;    // rotate-half pairs: dim i with dim i + 32

// Rotary frequencies as fixed-point turns: turn[i] = theta_i / (2 pi) * 2^64,
// theta_i = base^(-2i/64).  The angle of pair i at position p in turns is then
// (p * turn[i]) mod 2^64, exact in integer arithmetic for any position, so the
// only rounding is the final conversion of a value in [-1/2, 1/2) turn.
struct RopeTurns {
    uint64_t turn[kPairs];
};

__device__ __forceinline__ void rope_sincos(uint64_t turn, int64_t pos, float &s, float &c) {
    uint64_t t = (uint64_t)pos * turn;
    float r = (float)(int32_t)(uint32_t)(t >> 32) * 2.3283064365386963e-10f;   // 2^-32
    s = __builtin_amdgcn_sinf(r);   // hardware sin/cos take revolutions
    c = __builtin_amdgcn_cosf(r);
}

// Same angle from a turn count already reduced mod 2^64 (fixed point, 64 fraction bits).
__device__ __forceinline__ void turn_sincos(uint64_t t, float &s, float &c) {
    float r = (float)(int32_t)(uint32_t)(t >> 32) * 2.3283064365386963e-10f;
    s = __builtin_amdgcn_sinf(r);
    c = __builtin_amdgcn_cosf(r);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    f32x2 v = {lo, hi};
    bf16x2 b = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Rotate 8 consecutive pairs: x holds dims [i0, i0+8) of the first half and y
// the partner dims [i0+32, i0+40); angles are those of pairs i0..i0+7.
__device__ __forceinline__ void rope_rotate8(u32x4 &x, u32x4 &y, const RopeTurns &rt, int i0,
                                             int64_t pos) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        float s0, c0, s1, c1;
        rope_sincos(rt.turn[i0 + 2 * w], pos, s0, c0);
        rope_sincos(rt.turn[i0 + 2 * w + 1], pos, s1, c1);
        float x0 = bf_lo(x[w]), x1 = bf_hi(x[w]);
        float y0 = bf_lo(y[w]), y1 = bf_hi(y[w]);
        x[w] = pack_bf16(x0 * c0 - y0 * s0, x1 * c1 - y1 * s1);
        y[w] = pack_bf16(y0 * c0 + x0 * s0, y1 * c1 + x1 * s1);
    }
}

// Cross-lane helpers (wave64).
__device__ __forceinline__ float max_xor32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ u32x4 ldg128(const uint16_t *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ void stg128(uint16_t *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

}  // namespace mimo
