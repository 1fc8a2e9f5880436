// Device-side helpers shared by the kvc kernels: element conversions with
// IEEE round-to-nearest-even and cross-lane reductions for 64-wide waves.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc_kernels.h"

namespace kvc {

// ---- conversions -----------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ float f16_to_f32(uint32_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// bfloat16 keeps the high half of the binary32 pattern: add 0x7FFF plus the
// lowest kept bit, then shift (round to nearest, ties to even; overflow carries
// into the exponent and yields infinity). NaN -> quiet NaN 0x7FC0 with its sign.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) & 0x8000u) | 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// binary16 via the hardware conversion, which rounds to nearest-even in the
// default rounding mode and keeps binary16 subnormals; NaN -> 0x7E00 with sign.
__device__ __forceinline__ uint32_t f32_to_f16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) & 0x8000u) | 0x7E00u;
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// Value of x after storing it as dtype DT (identity for F32).
template <int DT>
__device__ __forceinline__ float round_as(float x) {
    if constexpr (DT == F32) return x;
    else if constexpr (DT == BF16) return bf16_to_f32(f32_to_bf16_rne(x));
    else return f16_to_f32(f32_to_f16_rne(x));
}

// Load 8 consecutive elements of dtype DT (16-byte aligned for 16-bit types,
// 32-byte aligned for F32) as float32 (exact).
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float (&o)[8]) {
    if constexpr (DT == F32) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
        float4 a = p[0], b = p[1];
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    } else {
        uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
        uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (DT == BF16) {
                o[2 * i] = bf16_to_f32(ws[i] & 0xFFFFu);
                o[2 * i + 1] = bf16_to_f32(ws[i] >> 16);
            } else {
                o[2 * i] = f16_to_f32(ws[i] & 0xFFFFu);
                o[2 * i + 1] = f16_to_f32(ws[i] >> 16);
            }
        }
    }
}

// Round 8 float32 values to dtype DT and store them.
template <int DT>
__device__ __forceinline__ void store8(void* base, int64_t elem, const float (&v)[8]) {
    if constexpr (DT == F32) {
        float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + elem);
        p[0] = make_float4(v[0], v[1], v[2], v[3]);
        p[1] = make_float4(v[4], v[5], v[6], v[7]);
    } else {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t lo, hi;
            if constexpr (DT == BF16) {
                lo = f32_to_bf16_rne(v[2 * i]);
                hi = f32_to_bf16_rne(v[2 * i + 1]);
            } else {
                lo = f32_to_f16_rne(v[2 * i]);
                hi = f32_to_f16_rne(v[2 * i + 1]);
            }
            w[i] = lo | (hi << 16);
        }
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + elem) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// Rotary position embedding of 8 pairs, elements i0 + e (x1[e]) and
// i0 + e + D/2 (x2[e]) of one head vector at position pos, with the pairs'
// frequencies f[e] (the "rotate half" pairing): angle = pos * f[e] in float64,
// y1 = x1 cos - x2 sin, y2 = x2 cos + x1 sin, each product and the sum rounded
// in float64 (no fused multiply-add), then rounded to float32.
__device__ __forceinline__ void rope8(const float (&x1)[8], const float (&x2)[8], int64_t pos, const double* f,
                                      float (&y1)[8], float (&y2)[8]) {
#pragma clang fp contract(off)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const double ang = static_cast<double>(pos) * f[e];
        double sn, cs;
        sincos(ang, &sn, &cs);
        const double a = static_cast<double>(x1[e]) * cs;
        const double b = static_cast<double>(x2[e]) * sn;
        const double c = static_cast<double>(x2[e]) * cs;
        const double d = static_cast<double>(x1[e]) * sn;
        y1[e] = static_cast<float>(a - b);
        y2[e] = static_cast<float>(c + d);
    }
}

// Hardware base-2 exponential (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- cross-lane reductions --------------------------------------------------
// DPP row operations act within rows of 16 lanes. quad_perm [1,0,3,2] and
// [2,3,0,1] exchange with lanes 1 and 2 away; after those a whole quad holds
// one value, so row_half_mirror (lane i <-> 7 - i) pairs quad 0 with quad 1,
// and row_mirror (i <-> 15 - i) pairs the two 8-lane halves; row_ror:n rotates
// a row (lane i gets lane i - n, mod 16). Distances 16 and 32 use gfx950's
// v_permlane16_swap / v_permlane32_swap (VALU, no LDS traffic): applied to
// (x, x) they return, in each lane, x of that lane and of the lane 16 (32)
// away, in an order that depends on the lane.

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

constexpr int kDppXor1 = 0xB1;        // quad_perm(1,0,3,2)
constexpr int kDppXor2 = 0x4E;        // quad_perm(2,3,0,1)
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppRor4 = 0x124;
constexpr int kDppRor8 = 0x128;

// op(x, x of the lane D away), D = 16 or 32; op is commutative.
template <int D, bool MAX>
__device__ __forceinline__ float xor_op(float x) {
    static_assert(D == 16 || D == 32, "lane swap distance");
    const uint32_t u = __float_as_uint(x);
    float a, b;
    if constexpr (D == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        a = __uint_as_float(r[0]);
        b = __uint_as_float(r[1]);
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        a = __uint_as_float(r[0]);
        b = __uint_as_float(r[1]);
    }
    return MAX ? fmaxf(a, b) : a + b;
}

// Sum (or max) over the lanes that share lane % N (N = 4..64, power of two):
// across the 64 / N aligned groups of N lanes. Every lane gets the result.
template <int N, bool MAX>
__device__ __forceinline__ float across_groups(float x) {
    static_assert(N >= 4 && N <= 64, "group width");
    if constexpr (N == 4) x = MAX ? fmaxf(x, dpp_f<kDppRor4>(x)) : x + dpp_f<kDppRor4>(x);
    if constexpr (N <= 8) x = MAX ? fmaxf(x, dpp_f<kDppRor8>(x)) : x + dpp_f<kDppRor8>(x);
    if constexpr (N <= 16) x = xor_op<16, MAX>(x);
    if constexpr (N <= 32) x = xor_op<32, MAX>(x);
    return x;
}

// In-place sums of M independent values over aligned groups of N lanes
// (N in 1..16). The steps go across all M values before the next step, so a
// DPP read never directly follows the write it depends on.
template <int N, int M>
__device__ __forceinline__ void group_sum_n(float (&x)[M]) {
    if constexpr (N >= 2) {
#pragma unroll
        for (int i = 0; i < M; ++i) x[i] += dpp_f<kDppXor1>(x[i]);
    }
    if constexpr (N >= 4) {
#pragma unroll
        for (int i = 0; i < M; ++i) x[i] += dpp_f<kDppXor2>(x[i]);
    }
    if constexpr (N >= 8) {
#pragma unroll
        for (int i = 0; i < M; ++i) x[i] += dpp_f<kDppHalfMirror>(x[i]);
    }
    if constexpr (N >= 16) {
#pragma unroll
        for (int i = 0; i < M; ++i) x[i] += dpp_f<kDppMirror>(x[i]);
    }
    static_assert(N <= 16, "group_sum_n works inside one 16-lane DPP row");
}

// Sum over aligned groups of N lanes (N in 1..64, power of two); every lane of
// a group gets the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (N >= 2) x += dpp_f<kDppXor1>(x);
    if constexpr (N >= 4) x += dpp_f<kDppXor2>(x);
    if constexpr (N >= 8) x += dpp_f<kDppHalfMirror>(x);
    if constexpr (N >= 16) x += dpp_f<kDppMirror>(x);
    if constexpr (N >= 32) x = xor_op<16, false>(x);
    if constexpr (N >= 64) x = xor_op<32, false>(x);
    return x;
}

}  // namespace kvc
