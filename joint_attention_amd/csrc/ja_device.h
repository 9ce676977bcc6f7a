// Device-side types and helpers shared by the gfx950 kernels of joint_attn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "joint_attn.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx2 __attribute__((ext_vector_type(2)));

namespace ja {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Workgroups of one launch are handed to the 8 XCDs round-robin (id % 8).  Renumber
// them so each XCD receives one contiguous range of logical tiles: neighbouring tiles
// (same batch-head, so the same K/V) then run on one XCD and share its L2.
__device__ inline int xcd_remap(int bid, int total) {
    const int q = total >> 3, r = total & 7;
    const int x = bid & 7, k = bid >> 3;
    const int base = x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
    return base + k;
}

// Exchange with the other half of the wave: returns {x of lanes 0..31, x of lanes
// 32..63} in some order in every lane; callers only use symmetric combinations.
__device__ inline void halves(float x, float& a, float& b) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

__device__ inline float wave_halves_max(float x) {
    float a, b;
    halves(x, a, b);
    return fmaxf(a, b);
}

__device__ inline float wave_halves_sum(float x) {
    float a, b;
    halves(x, a, b);
    return a + b;
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace ja
