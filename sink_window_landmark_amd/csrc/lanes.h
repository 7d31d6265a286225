// Wave-level lane exchanges for gfx950, shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "swl_internal.h"

namespace swl {

// Lane exchanges without LDS.  The partner of a lane at bit B is the lane
// index xor 1, 2, 7, 15, 16, 32 for B = 0 .. 5: DPP quad permutes, the 8- and
// 16-lane mirrors, then the gfx950 permlane swaps across rows.  The masks
// are linearly independent with top bit B, which is all that sums over a
// whole group of lanes need (for a sum that must keep the lanes below bit B
// apart, use xor_sum).
template <int C>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), C, 0xF, 0xF, false));
}
template <int B>
struct DppCtl;
template <> struct DppCtl<0> { static constexpr int v = 0xB1; };    // quad_perm 1,0,3,2
template <> struct DppCtl<1> { static constexpr int v = 0x4E; };    // quad_perm 2,3,0,1
template <> struct DppCtl<2> { static constexpr int v = 0x141; };   // row_half_mirror
template <> struct DppCtl<3> { static constexpr int v = 0x140; };   // row_mirror

// the two halves of a permlane swap of (a, b), as floats
template <int B>
__device__ __forceinline__ void pl_swap(float a, float b, float& r0, float& r1)
{
    static_assert(B == 4 || B == 5, "cross-row swaps only");
    if constexpr (B == 4) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        r0 = __uint_as_float(r[0]);
        r1 = __uint_as_float(r[1]);
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        r0 = __uint_as_float(r[0]);
        r1 = __uint_as_float(r[1]);
    }
}

// x plus (or max with) the partner's x at bit B
template <int B>
__device__ __forceinline__ float pair_sum(float x)
{
    if constexpr (B <= 3) {
        return x + dpp<DppCtl<B>::v>(x);
    } else {
        float r0, r1;
        pl_swap<B>(x, x, r0, r1);   // lanes of both halves see (lower x, upper x)
        return r0 + r1;
    }
}
template <int B>
__device__ __forceinline__ float pair_max(float x)
{
    if constexpr (B <= 3) {
        return fmaxf(x, dpp<DppCtl<B>::v>(x));
    } else {
        float r0, r1;
        pl_swap<B>(x, x, r0, r1);
        return fmaxf(r0, r1);
    }
}
// One reduce-scatter step: lanes with bit B clear get lo + the partner's lo,
// lanes with it set hi + the partner's hi.
template <int B>
__device__ __forceinline__ float pair_split(float lo, float hi, int lane)
{
    if constexpr (B <= 3) {
        const float a = lo + dpp<DppCtl<B>::v>(lo), b = hi + dpp<DppCtl<B>::v>(hi);
        return (lane >> B) & 1 ? b : a;
    } else {
        float r0, r1;
        pl_swap<B>(lo, hi, r0, r1);   // (own lo, partner lo) below, (partner hi, own hi) above
        return r0 + r1;
    }
}
// x plus the x of lane ^ (1 << B) exactly (the lanes below bit B kept apart)
template <int B>
__device__ __forceinline__ float xor_sum(float x)
{
    if constexpr (B <= 1 || B >= 4) return pair_sum<B>(x);
    else return x + __shfl_xor(x, 1 << B, 64);
}

// the x of lane ^ (1 << B), exactly
template <int B>
__device__ __forceinline__ float xor_get(float x, int lane)
{
    if constexpr (B <= 1) {
        return dpp<DppCtl<B>::v>(x);
    } else if constexpr (B <= 3) {
        return __shfl_xor(x, 1 << B, 64);
    } else {
        float r0, r1;
        pl_swap<B>(x, x, r0, r1);   // (lower x, upper x) in every lane
        return (lane >> B) & 1 ? r0 : r1;
    }
}

__device__ __forceinline__ float wsum(float x)
{
    x = pair_sum<0>(x);
    x = pair_sum<1>(x);
    x = pair_sum<2>(x);
    x = pair_sum<3>(x);
    x = pair_sum<4>(x);
    return pair_sum<5>(x);
}

__device__ __forceinline__ float wmax(float x)
{
    x = pair_max<0>(x);
    x = pair_max<1>(x);
    x = pair_max<2>(x);
    x = pair_max<3>(x);
    x = pair_max<4>(x);
    return pair_max<5>(x);
}

// Sum of x over aligned groups of 16 lanes.
__device__ __forceinline__ float sum16(float x)
{
    x = pair_sum<0>(x);
    x = pair_sum<1>(x);
    x = pair_sum<2>(x);
    return pair_sum<3>(x);
}

// Sum and maximum of x over aligned groups of 32 lanes.
__device__ __forceinline__ float sum32(float x)
{
    x = pair_sum<0>(x);
    x = pair_sum<1>(x);
    x = pair_sum<2>(x);
    x = pair_sum<3>(x);
    return pair_sum<4>(x);
}

__device__ __forceinline__ float max32(float x)
{
    x = pair_max<0>(x);
    x = pair_max<1>(x);
    x = pair_max<2>(x);
    x = pair_max<3>(x);
    return pair_max<4>(x);
}

// value_exp_of over group g's block maxima (far_score), evaluated by every
// lane of the calling wave (all 64 lanes must call it).
__device__ __forceinline__ int value_exp(const KParams& p, int g)
{
    float x = 0.f;
    for (int i = threadIdx.x & 63; i < p.vm_n; i += 64) x = fmaxf(x, p.vmax[(int64_t)g * VM_SLOTS + i]);
    x = wmax(x);
    return __builtin_amdgcn_readfirstlane(value_exp_of(x));   // the same in every lane
}

}  // namespace swl
