// kv4_common.h -- device helpers shared by the libkv4 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "kv4_device_types.h"
#include "kv4_launch.h"

namespace kv4 {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { FMT_INT4_PROT = 0, FMT_INT8 = 1, FMT_BF16 = 2 };

// One launch of `kernel` with its argument struct; the timer's events, when set, are stamped from
// the launch's own dispatch.
template <typename Arg>
inline hipError_t launch_kernel(void (*kernel)(Arg), dim3 grid, dim3 block, hipStream_t stream,
                                const KernelTimer& tm, const Arg& a)
{
    if (tm.start || tm.stop)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, tm.start, tm.stop, 0, a);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------------------------

template <int Begin, int End, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    if constexpr (Begin < End) {
        f(std::integral_constant<int, Begin>{});
        static_for<Begin + 1, End>(f);
    }
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float as_float(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ u16x2 as_u16x2(uint32_t u) { return __builtin_bit_cast(u16x2, u); }
__device__ __forceinline__ uint32_t as_uint(float f) { return __builtin_bit_cast(uint32_t, f); }

__device__ __forceinline__ float f16_bits_to_float(uint32_t bits16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

__device__ __forceinline__ uint16_t f16_bits(_Float16 h) { return __builtin_bit_cast(uint16_t, h); }

// Largest fp16 <= x (x finite, within the fp16 range); zero results are +0.
__device__ __forceinline__ uint32_t f16_round_down(float x)
{
    _Float16 h = (_Float16)x; // round to nearest even
    uint32_t b = f16_bits(h);
    if ((float)h > x) {
        if (b & 0x8000u)
            b = b + 1u;          // negative: one step away from zero
        else if (b == 0u)
            b = 0x8001u;         // +0 above a tiny negative x
        else
            b = b - 1u;          // positive: one step toward zero
    }
    if (b == 0x8000u) b = 0u;
    return b;
}

// Smallest fp16 >= x; zero results are +0.
__device__ __forceinline__ uint32_t f16_round_up(float x)
{
    _Float16 h = (_Float16)x;
    uint32_t b = f16_bits(h);
    if ((float)h < x) {
        if (b & 0x8000u)
            b = b - 1u;          // negative: one step toward zero (0x8001 -> -0)
        else
            b = b + 1u;          // non-negative: one step away from zero
    }
    if (b == 0x8000u) b = 0u;
    return b;
}

// Value of lane (lane ^ 1).
__device__ __forceinline__ float dpp_xor1(float x)
{
    return as_float((uint32_t)__builtin_amdgcn_mov_dpp((int)as_uint(x), 0xB1, 0xF, 0xF, false));
}

// Value of lane l ^ M of x within each row of 16 lanes (M = 1, 2, 4, 8), by DPP moves (no LDS
// access): 1 and 2 are quad permutations; 4 is row_half_mirror (l ^ 7) followed by quad_perm
// [3,2,1,0] (l ^ 3); 8 rotates the row by 8.
template <int M>
__device__ __forceinline__ float lane_xor_row(float x)
{
    static_assert(M == 1 || M == 2 || M == 4 || M == 8, "a partner inside the row");
    const int v = (int)as_uint(x);
    int r;
    if constexpr (M == 1) {
        r = __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);
    } else if constexpr (M == 2) {
        r = __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);
    } else if constexpr (M == 4) {
        const int t = __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);
        r = __builtin_amdgcn_mov_dpp(t, 0x1B, 0xF, 0xF, false);
    } else {
        r = __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false);
    }
    return as_float((uint32_t)r);
}

// Value of lane l ^ 16 within each half of the wave (ds_swizzle in bit mode, and-mask 0x1F,
// xor-mask 0x10: no address computation).
__device__ __forceinline__ float lane_xor16(float x)
{
    return as_float((uint32_t)__builtin_amdgcn_ds_swizzle((int)as_uint(x), 0x401F));
}

// Value of lane l ^ M for a power of two M < 64 (every lane active).
template <int M>
__device__ __forceinline__ float lane_xor(float x)
{
    if constexpr (M <= 8)
        return lane_xor_row<M>(x);
    else if constexpr (M == 16)
        return lane_xor16(x);
    else
        return __shfl_xor(x, M, 64);
}

// One butterfly of a Hadamard stage across lanes l and l ^ M: x + x' on the lane without bit M,
// x' - x on the lane with it (x' the partner's value).  sgn is +1 or -1 to match; an fma with a
// factor of +-1 rounds once, exactly like the add or the subtract it replaces.
template <int M>
__device__ __forceinline__ float butterfly_xor(float x, float sgn)
{
    return fmaf(sgn, x, lane_xor<M>(x));
}

// x[l] + x[l ^ 32] and max(x[l], x[l ^ 32]).  v_permlane32_swap of x with itself leaves the two
// values of the pair, one in each result, on every lane; a sum or max of the two is the same bits
// whichever result holds which.
__device__ __forceinline__ float add_xor32(float x)
{
    const int v = (int)as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return as_float((uint32_t)r[0]) + as_float((uint32_t)r[1]);
}

__device__ __forceinline__ float max_xor32(float x)
{
    const int v = (int)as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return fmaxf(as_float((uint32_t)r[0]), as_float((uint32_t)r[1]));
}

// LDS written by some lanes of a wave and then read by other lanes of the same wave: the LDS
// queue of a wave is in order; this keeps the compiler from moving accesses across it.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ bool is_protected(int t, int L, int S, int R)
{
    if (t < S) return t < L;
    int lo = L - R;
    if (lo < S) lo = S;
    return t >= lo && t < L;
}

__device__ __forceinline__ half4_t to_half4(uint32_t lo, uint32_t hi)
{
    return __builtin_bit_cast(half4_t, (u32x2){lo, hi});
}

__device__ __forceinline__ short4_t to_short4(uint32_t lo, uint32_t hi)
{
    return __builtin_bit_cast(short4_t, (u32x2){lo, hi});
}

template <int ABID>
__device__ __forceinline__ float4_t mfma_h(half4_t a, half4_t b, float4_t c)
{
    // 16 blocks of 4x4x4; A of block ABID is broadcast to all 16 blocks
    return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, 4, ABID, 0);
}

// A of block ABID of each half wave (blocks 0..7, 8..15) is broadcast to the blocks of that half
template <int ABID>
__device__ __forceinline__ float4_t mfma_h_half(half4_t a, half4_t b, float4_t c)
{
    return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, 3, ABID, 0);
}

template <int ABID>
__device__ __forceinline__ float4_t mfma_bf(short4_t a, short4_t b, float4_t c)
{
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, b, c, 4, ABID, 0);
}

// DPP move of x with control CTRL; lanes of rows outside ROWMASK keep their own value.
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ float dpp_keep(float x)
{
    const int v = (int)as_uint(x);
    return as_float((uint32_t)__builtin_amdgcn_update_dpp(v, v, CTRL, ROWMASK, 0xF, false));
}

// Max / sum over the 64 lanes with DPP row operations and the gfx9 row broadcasts; the result is
// read from lane 63 and is wave-uniform.  The summation order is fixed.
__device__ __forceinline__ float wave_max_u(float x)
{
    x = fmaxf(x, dpp_keep<0xB1>(x));       // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp_keep<0x4E>(x));       // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp_keep<0x141>(x));      // row_half_mirror
    x = fmaxf(x, dpp_keep<0x140>(x));      // row_mirror: every lane holds its row's max
    x = fmaxf(x, dpp_keep<0x142, 0xA>(x)); // row_bcast:15 into rows 1, 3
    x = fmaxf(x, dpp_keep<0x143, 0xC>(x)); // row_bcast:31 into rows 2, 3
    return as_float((uint32_t)__builtin_amdgcn_readlane((int)as_uint(x), 63));
}

// DPP move of x with control CTRL; lanes of rows outside ROWMASK read 0.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_or_zero(float x)
{
    return as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_uint(x), CTRL, ROWMASK, 0xF, false));
}

__device__ __forceinline__ float wave_sum_u(float x)
{
    x = x + dpp_keep<0xB1>(x);
    x = x + dpp_keep<0x4E>(x);
    x = x + dpp_keep<0x141>(x);
    x = x + dpp_keep<0x140>(x);            // every lane holds its row's sum
    x = x + dpp_or_zero<0x142, 0xA>(x);    // rows 1, 3 add the previous row
    x = x + dpp_or_zero<0x143, 0xC>(x);    // rows 2, 3 add rows 0 + 1
    return as_float((uint32_t)__builtin_amdgcn_readlane((int)as_uint(x), 63));
}

} // namespace kv4
