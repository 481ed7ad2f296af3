// kv4_kernels.hip -- gfx950 kernels of libkv4.
//
//   append_kernel        fused block-FWHT + token-wise quantization + nibble packing + paged store,
//                        plus the INT8 copy of protected positions ("SAW-INT4: System-Aware 4-Bit
//                        KV-Cache Quantization for Real-World LLM Serving", Abstract: fused
//                        rotation-quantization written into paged layouts; "KV4-RL: Unlocking
//                        Faster Asynchronous Rollouts for RLVR with INT4 KV Cache Quantization",
//                        Abstract: INT8 protection of sinks and recent context).
//   decode_split_kernel  split-KV flash-decode over the paged INT4 pages and the INT8 slots
//                        (fused attention over the quantized cache, SAW-INT4 Abstract).
//   merge_kernel         log-sum-exp merge of the split partials and the inverse rotation.
//
// Build with -ffp-contract=off: the append's binary32 steps must stay single IEEE operations.
// Where the decode wants a fused multiply-add it calls fmaf explicitly.
#include <hip/hip_runtime.h>
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

__device__ __forceinline__ float as_float(uint32_t u) { return __builtin_bit_cast(float, u); }
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
    return as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_uint(x), 0xB1, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
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

template <int ABID>
__device__ __forceinline__ float4_t mfma_bf(short4_t a, short4_t b, float4_t c)
{
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, b, c, 4, ABID, 0);
}

// ---------------------------------------------------------------------------------------------
// append
// ---------------------------------------------------------------------------------------------
// One wave per (task, kv head).  Lane l handles row l/2 (rows 0..15: K of page slot 0..15,
// rows 16..31: V of slot 0..15) and half l%2 of its D dims.

template <int N>
__device__ __forceinline__ void fwht_in_lane(float (&y)[N], int b)
{
    // stages h = 1, 2, 4, ... while h < b and h < N, in that order; butterflies (a+c, a-c)
#pragma unroll
    for (int h = 1; h < N; h <<= 1) {
        if (h < b) {
#pragma unroll
            for (int i = 0; i < N; i++) {
                if ((i & h) == 0) {
                    float a0 = y[i], c0 = y[i + h];
                    y[i] = a0 + c0;
                    y[i + h] = a0 - c0;
                }
            }
        }
    }
}

// Last stage h = N when b == 2N: partner lane holds the other half of the row.
template <int N>
__device__ __forceinline__ void fwht_across_pair(float (&y)[N], int half)
{
    const uint32_t sgn = half ? 0x80000000u : 0u;
#pragma unroll
    for (int i = 0; i < N; i++) {
        float own = y[i];
        float partner = dpp_xor1(own);
        // half 0: own(dim i) + partner(dim i+N); half 1: partner(dim i) - own(dim i+N)
        y[i] = partner + as_float(as_uint(own) ^ sgn);
    }
}

struct QuantParams {
    uint32_t s_bits, z_bits;
    float zf, inv;
};

// Token-wise scale / zero of one row from its exact min and max; Q = 15 or 255.
__device__ __forceinline__ QuantParams quant_params(float mn, float mx, float Qf)
{
    QuantParams p;
    p.z_bits = f16_round_down(mn);
    p.zf = f16_bits_to_float(p.z_bits);
    float r = mx - p.zf;
    float t = r / Qf;
    p.s_bits = f16_round_up(t);
    float sf = f16_bits_to_float(p.s_bits);
    p.inv = (sf != 0.0f) ? 1.0f / sf : 0.0f; // s == 0: every code is 0
    return p;
}

template <int D, int FMT>
__global__ __launch_bounds__(64) void append_kernel(AppendArgs a)
{
    constexpr int N = D / 2;
    // V rows staged for the dim-major V layout: INT4 packed rows [16][D/2], INT8 rows [16][D],
    // bf16 rows [16][D] x 2 B
    __shared__ __align__(16) uint8_t lds[16 * D * 2];
    uint8_t* lds_v4 = lds;            // [16][D/2]
    uint8_t* lds_v8 = lds + 16 * D;   // [16][D]

    const int lane = threadIdx.x;
    const AppendTask tk = a.tasks[blockIdx.x];
    const int h = blockIdx.y;
    const int rho = lane >> 1, half = lane & 1;
    const bool is_v = rho >= kPageSize;
    const int slot = rho & (kPageSize - 1);
    const int s0 = tk.t0 & (kPageSize - 1);
    const int s1 = s0 + tk.n;
    const bool active = slot >= s0 && slot < s1;
    const int t = tk.t0 - s0 + slot;
    if (lane == 0 && h == 0 && (tk.flags & kTaskNewPage)) a.bt[tk.bt_index] = tk.page;
    uint8_t* pb = a.pool + ((int64_t)tk.page * a.hkv + h) * a.page_block;

    u32x4 raw[N / 8];
    if (active) {
        const uint16_t* src = (is_v ? a.v : a.k) + ((int64_t)(tk.row0 + slot - s0) * a.hkv + h) * D + half * N;
#pragma unroll
        for (int q = 0; q < N / 8; q++) raw[q] = *(const u32x4*)(src + 8 * q);
    } else {
#pragma unroll
        for (int q = 0; q < N / 8; q++) raw[q] = (u32x4){0u, 0u, 0u, 0u};
    }

    if constexpr (FMT == FMT_BF16) {
        uint16_t* lds_bf = (uint16_t*)lds; // [16][D]
        if (active) {
            if (!is_v) {
#pragma unroll
                for (int q = 0; q < N / 8; q++) *(u32x4*)(pb + (half * (N / 8) + q) * 256 + slot * 16) = raw[q];
            } else {
#pragma unroll
                for (int q = 0; q < N / 8; q++) *(u32x4*)(lds_bf + slot * D + half * N + 8 * q) = raw[q];
            }
        }
        __syncthreads();
        // dim-major V: [D][16 slots x bf16]
#pragma unroll
        for (int dd = 0; dd < D / 64; dd++) {
            const int d = dd * 64 + lane;
            uint32_t* dst = (uint32_t*)(pb + 32 * D + d * 32);
            uint32_t w[8];
#pragma unroll
            for (int j = 0; j < 8; j++) w[j] = (tk.n < 16) ? dst[j] : 0u;
            for (int s = s0; s < s1; s++) {
                uint32_t v = lds_bf[s * D + d];
                int sh = (s & 1) * 16;
#pragma unroll
                for (int j = 0; j < 8; j++)
                    if (j == (s >> 1)) w[j] = (w[j] & ~(0xFFFFu << sh)) | (v << sh);
            }
#pragma unroll
            for (int j = 0; j < 8; j += 4) *(u32x4*)(dst + j) = (u32x4){w[j], w[j + 1], w[j + 2], w[j + 3]};
        }
        return;
    } else {
        // ---- rotate ----
        float y[N];
#pragma unroll
        for (int q = 0; q < N / 8; q++) {
#pragma unroll
            for (int j = 0; j < 4; j++) {
                y[8 * q + 2 * j] = as_float(raw[q][j] << 16);
                y[8 * q + 2 * j + 1] = as_float(raw[q][j] & 0xFFFF0000u);
            }
        }
        fwht_in_lane<N>(y, a.block);
        if (a.block == D) fwht_across_pair<N>(y, half);
        if (a.block > 1) {
#pragma unroll
            for (int i = 0; i < N; i++) y[i] = y[i] * a.cb;
        }
        // ---- row min / max ----
        float mn = y[0], mx = y[0];
#pragma unroll
        for (int i = 1; i < N; i++) {
            mn = fminf(mn, y[i]);
            mx = fmaxf(mx, y[i]);
        }
        mn = fminf(mn, dpp_xor1(mn));
        mx = fmaxf(mx, dpp_xor1(mx));

        const bool prot = (FMT == FMT_INT4_PROT) && active && is_protected(t, tk.len_new, a.sinks, a.recent);

        if constexpr (FMT == FMT_INT4_PROT) {
            // ---- INT4 codes, natural nibble order: byte k = code[2k] | code[2k+1] << 4 ----
            const QuantParams qp = quant_params(mn, mx, 15.0f);
            uint32_t pk[N / 8];
#pragma unroll
            for (int q = 0; q < N / 8; q++) {
                uint32_t e = 0, o = 0;
                float u0 = (y[8 * q + 0] - qp.zf) * qp.inv, u1 = (y[8 * q + 1] - qp.zf) * qp.inv;
                float u2 = (y[8 * q + 2] - qp.zf) * qp.inv, u3 = (y[8 * q + 3] - qp.zf) * qp.inv;
                float u4 = (y[8 * q + 4] - qp.zf) * qp.inv, u5 = (y[8 * q + 5] - qp.zf) * qp.inv;
                float u6 = (y[8 * q + 6] - qp.zf) * qp.inv, u7 = (y[8 * q + 7] - qp.zf) * qp.inv;
                e = __builtin_amdgcn_cvt_pk_u8_f32(u0, 0, e);
                e = __builtin_amdgcn_cvt_pk_u8_f32(u2, 1, e);
                e = __builtin_amdgcn_cvt_pk_u8_f32(u4, 2, e);
                e = __builtin_amdgcn_cvt_pk_u8_f32(u6, 3, e);
                o = __builtin_amdgcn_cvt_pk_u8_f32(u1, 0, o);
                o = __builtin_amdgcn_cvt_pk_u8_f32(u3, 1, o);
                o = __builtin_amdgcn_cvt_pk_u8_f32(u5, 2, o);
                o = __builtin_amdgcn_cvt_pk_u8_f32(u7, 3, o);
                pk[q] = e | (o << 4);
            }
            if (active) {
                if (!is_v) {
                    // K: [D/32 chunks][16 slots][16 B]; this half covers chunks half*N/32 ..
#pragma unroll
                    for (int c = 0; c < N / 32; c++)
                        *(u32x4*)(pb + (half * (N / 32) + c) * 256 + slot * 16) =
                            (u32x4){pk[4 * c], pk[4 * c + 1], pk[4 * c + 2], pk[4 * c + 3]};
                } else {
#pragma unroll
                    for (int c = 0; c < N / 32; c++)
                        *(u32x4*)(lds_v4 + slot * (D / 2) + half * (N / 2) + 16 * c) =
                            (u32x4){pk[4 * c], pk[4 * c + 1], pk[4 * c + 2], pk[4 * c + 3]};
                }
                if (half == 0)
                    *(uint32_t*)(pb + 16 * D + slot * 8 + (is_v ? 4 : 0)) = qp.s_bits | (qp.z_bits << 16);
            }
        }

        // ---- INT8 codes: protected positions (INT4_PROT) or every position (INT8 format) ----
        const bool want8 = (FMT == FMT_INT8) ? active : prot;
        if (__ballot(want8) != 0ull) {
            const QuantParams qp = quant_params(mn, mx, 255.0f);
            uint32_t cb8[N / 4];
#pragma unroll
            for (int q = 0; q < N / 4; q++) {
                uint32_t w = 0;
                w = __builtin_amdgcn_cvt_pk_u8_f32((y[4 * q + 0] - qp.zf) * qp.inv, 0, w);
                w = __builtin_amdgcn_cvt_pk_u8_f32((y[4 * q + 1] - qp.zf) * qp.inv, 1, w);
                w = __builtin_amdgcn_cvt_pk_u8_f32((y[4 * q + 2] - qp.zf) * qp.inv, 2, w);
                w = __builtin_amdgcn_cvt_pk_u8_f32((y[4 * q + 3] - qp.zf) * qp.inv, 3, w);
                cb8[q] = w;
            }
            if (want8) {
                uint8_t* tb;
                int s8;
                if (FMT == FMT_INT8) {
                    tb = pb;
                    s8 = slot;
                } else {
                    const int u = (t < a.sinks) ? t : a.sinks + t % a.recent;
                    tb = a.int8_pool + (((int64_t)tk.seq * a.hkv + h) * a.int8_tiles + (u >> 4)) * a.int8_tile;
                    s8 = u & 15;
                }
                if (!is_v) {
                    // K8: [D/16 chunks][16 slots][16 B]; this half covers chunks half*N/16 ..
#pragma unroll
                    for (int c = 0; c < N / 16; c++)
                        *(u32x4*)(tb + (half * (N / 16) + c) * 256 + s8 * 16) =
                            (u32x4){cb8[4 * c], cb8[4 * c + 1], cb8[4 * c + 2], cb8[4 * c + 3]};
                } else {
#pragma unroll
                    for (int c = 0; c < N / 16; c++)
                        *(u32x4*)(lds_v8 + slot * D + half * N + 16 * c) =
                            (u32x4){cb8[4 * c], cb8[4 * c + 1], cb8[4 * c + 2], cb8[4 * c + 3]};
                }
                if (half == 0) *(uint32_t*)(tb + 32 * D + s8 * 8 + (is_v ? 4 : 0)) = qp.s_bits | (qp.z_bits << 16);
            }
        }
        __syncthreads();

        // ---- dim-major V stores: lane = dim ----
#pragma unroll
        for (int dd = 0; dd < D / 64; dd++) {
            const int d = dd * 64 + lane;
            if constexpr (FMT == FMT_INT4_PROT) {
                // [D][8 B]: nibble s = slot s
                u32x2* dst = (u32x2*)(pb + 8 * D + d * 8);
                u32x2 w = (tk.n < 16) ? *dst : (u32x2){0u, 0u};
                for (int s = s0; s < s1; s++) {
                    uint32_t nib = (lds_v4[s * (D / 2) + (d >> 1)] >> ((d & 1) * 4)) & 0xFu;
                    int sh = (s & 7) * 4;
                    if (s < 8)
                        w.x = (w.x & ~(0xFu << sh)) | (nib << sh);
                    else
                        w.y = (w.y & ~(0xFu << sh)) | (nib << sh);
                }
                *dst = w;
                // INT8 copies of protected positions: one byte per (position, dim)
                for (int s = s0; s < s1; s++) {
                    const int ts = tk.t0 - s0 + s;
                    if (!is_protected(ts, tk.len_new, a.sinks, a.recent)) continue;
                    const int u = (ts < a.sinks) ? ts : a.sinks + ts % a.recent;
                    uint8_t* tb = a.int8_pool + (((int64_t)tk.seq * a.hkv + h) * a.int8_tiles + (u >> 4)) * a.int8_tile;
                    tb[16 * D + d * 16 + (u & 15)] = lds_v8[s * D + d];
                }
            } else {
                // INT8 format: [D][16 B], byte s = slot s
                u32x4* dst = (u32x4*)(pb + 16 * D + d * 16);
                u32x4 w = (tk.n < 16) ? *dst : (u32x4){0u, 0u, 0u, 0u};
                for (int s = s0; s < s1; s++) {
                    uint32_t v = lds_v8[s * D + d];
                    int sh = (s & 3) * 8;
#pragma unroll
                    for (int j = 0; j < 4; j++)
                        if (j == (s >> 2)) w[j] = (w[j] & ~(0xFFu << sh)) | (v << sh);
                }
                *dst = w;
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------------------------
// One wave per contiguous range of global steps.  A step of a (sequence, kv head) unit covers
//   INT4:  4 pages = 64 positions (lane = position); K codes feed the B operand of
//          v_mfma_f32_4x4x4f16 as fp16 subnormal patterns (value code * 2^-24), the rotated,
//          power-of-two-normalised query (split hi + lo fp16) is the broadcast A operand;
//          scores are s * (q . code) + z * sum(q), so K is never dequantised element-wise.
//   INT8:  32 protection slots (or 2 INT8 pages), lanes 0..31.
//   BF16:  1 page = 16 positions, lanes 0..15.
// PV uses the same 4x4x4 MFMA with lane = output dim: V codes (dim-major in the page) are the B
// operand and p*s (hi + lo fp16, exchanged through LDS) the broadcast A operand; the zero-point
// term sum_t p_t z_t is accumulated per lane and added once.

constexpr int kLdsQBytes = 4 * 128 * 4; // rotated query, G x D fp32
constexpr int kLdsPBytes = 64 * 16;     // per-step probability exchange
constexpr int kLdsPerWave = kLdsQBytes + kLdsPBytes;

struct UnitState {
    float m[4], lsum[4], zsum[4];
    float F[4], sumq[4];
};

template <int D, int G, int FMT>
struct DecodeWave {
    static constexpr int NHV = D / 64;    // output dims per lane
    static constexpr int NPAIR = D / 32;  // A-operand VGPR pairs for INT4 / INT8 steps
    static constexpr int NPAIR_BF = D / 64;

    const DecodeArgs& a;
    const int lane;
    uint8_t* lds_q;
    uint8_t* lds_p;

    half4_t A4[NPAIR], A8[NPAIR];
    short4_t Abf[NPAIR_BF];
    float4_t acc[NHV];
    UnitState st;

    __device__ DecodeWave(const DecodeArgs& args, int ln, uint8_t* lq, uint8_t* lp)
        : a(args), lane(ln), lds_q(lq), lds_p(lp) {}

    // ---- query prologue ----
    __device__ void prologue(const DecodeUnit& U, bool need4, bool need8)
    {
        const uint16_t* qrow = a.q + ((int64_t)U.entry * (a.hkv * G) + U.head * G) * D;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            st.m[i] = -INFINITY;
            st.lsum[i] = 0.f;
            st.zsum[i] = 0.f;
        }
#pragma unroll
        for (int hv = 0; hv < NHV; hv++) acc[hv] = (float4_t){0.f, 0.f, 0.f, 0.f};

        if constexpr (FMT == FMT_BF16) {
            // raw bf16 query (no rotation); A step m = dims 4m..4m+3, pair m/16, quad m%16
            const int s = lane >> 2, i = lane & 3;
#pragma unroll
            for (int v = 0; v < NPAIR_BF; v++) {
                const int m = 16 * v + s;
                uint32_t lo = 0, hi = 0;
                if (i < G) {
                    const uint32_t* src = (const uint32_t*)(qrow + i * D + 4 * m);
                    lo = src[0];
                    hi = src[1];
                }
                Abf[v] = to_short4(lo, hi);
            }
#pragma unroll
            for (int i2 = 0; i2 < 4; i2++) {
                st.F[i2] = a.scale_log2;
                st.sumq[i2] = 0.f;
            }
            return;
        } else {
            // lane holds dims lane + 64*j of each head
            float qv[G][NHV];
#pragma unroll
            for (int i = 0; i < G; i++)
#pragma unroll
                for (int j = 0; j < NHV; j++) qv[i][j] = as_float((uint32_t)qrow[i * D + 64 * j + lane] << 16);
            for (int hh = 1; hh < a.block; hh <<= 1) {
                if (hh < 64) {
#pragma unroll
                    for (int i = 0; i < G; i++)
#pragma unroll
                        for (int j = 0; j < NHV; j++) {
                            float other = __shfl_xor(qv[i][j], hh, 64);
                            qv[i][j] = (lane & hh) ? other - qv[i][j] : qv[i][j] + other;
                        }
                } else {
#pragma unroll
                    for (int i = 0; i < G; i++) {
                        float a0 = qv[i][0], a1 = qv[NHV > 1 ? i : i][NHV > 1 ? 1 : 0];
                        qv[i][0] = a0 + a1;
                        if constexpr (NHV > 1) qv[i][1] = a0 - a1;
                    }
                }
            }
            float* lq = (float*)lds_q;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                if (i < G) {
                    float mx = 0.f;
#pragma unroll
                    for (int j = 0; j < NHV; j++) {
                        qv[i][j] = qv[i][j] * a.cb;
                        mx = fmaxf(mx, fabsf(qv[i][j]));
                    }
                    mx = wave_max(mx);
                    int e = 0;
                    if (mx > 0.f) frexpf(mx, &e);
                    const int eq = (mx > 0.f) ? 15 - e : 0; // max |q| * 2^eq in [2^14, 2^15)
                    float sq = 0.f;
#pragma unroll
                    for (int j = 0; j < NHV; j++) {
                        qv[i][j] = ldexpf(qv[i][j], eq);
                        sq += qv[i][j];
                        lq[i * D + 64 * j + lane] = qv[i][j];
                    }
                    st.sumq[i] = wave_sum(sq);
                    st.F[i] = a.scale_log2 * ldexpf(1.0f, -eq);
                } else {
                    st.sumq[i] = 0.f;
                    st.F[i] = 0.f;
                }
            }
            wave_lds_sync();
            const int s = lane >> 2, i = lane & 3;
            if (need4) {
                // step m = 16c + 4wd + 2gp + hl; pair c, quad s = m % 16
                const int hl = s & 1, gp = (s >> 1) & 1, wd = s >> 2;
#pragma unroll
                for (int c = 0; c < NPAIR; c++) {
                    const int u = 4 * c + wd;
                    const int d0 = 8 * u + 2 * gp; // dims d0, d0+4, d0+1, d0+5
                    float x[4] = {0.f, 0.f, 0.f, 0.f};
                    if (i < G) {
                        x[0] = lq[i * D + d0];
                        x[1] = lq[i * D + d0 + 4];
                        x[2] = lq[i * D + d0 + 1] * 0.0625f;
                        x[3] = lq[i * D + d0 + 5] * 0.0625f;
                    }
                    _Float16 r[4];
#pragma unroll
                    for (int k = 0; k < 4; k++) {
                        _Float16 hi16 = (_Float16)x[k];
                        r[k] = hl ? (_Float16)(x[k] - (float)hi16) : hi16;
                    }
                    A4[c] = (half4_t){r[0], r[1], r[2], r[3]};
                }
            }
            if (need8) {
                // step m = 2u + hl (dims 4u..4u+3); pair m/16, quad s = m % 16
                const int hl = s & 1;
#pragma unroll
                for (int v = 0; v < NPAIR; v++) {
                    const int u = 8 * v + (s >> 1);
                    float x[4] = {0.f, 0.f, 0.f, 0.f};
                    if (i < G) {
#pragma unroll
                        for (int k = 0; k < 4; k++) x[k] = lq[i * D + 4 * u + k];
                    }
                    _Float16 r[4];
#pragma unroll
                    for (int k = 0; k < 4; k++) {
                        _Float16 hi16 = (_Float16)x[k];
                        r[k] = hl ? (_Float16)(x[k] - (float)hi16) : hi16;
                    }
                    A8[v] = (half4_t){r[0], r[1], r[2], r[3]};
                }
            }
            wave_lds_sync();
        }
    }

    // ---- online softmax over one step's scores (sc: -inf for masked lanes) ----
    // quantized formats: e' = score + log2(s_V) bounds the PV operand p*s_V by 2^15.
    __device__ __forceinline__ void softmax_update(const float (&sc)[4], float lg, bool valid, float sV, float zV,
                                                   float (&pt)[4])
    {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            if (i >= G) {
                pt[i] = 0.f;
                continue;
            }
            float ep = (FMT == FMT_BF16) ? sc[i] : sc[i] + lg;
            if (!valid) ep = -INFINITY;
            const float mt = wave_max(ep);
            const float mnew = fmaxf(st.m[i], mt);
            if (mnew > st.m[i]) {
                const float alpha = (st.m[i] == -INFINITY) ? 0.f : exp2f(st.m[i] - mnew);
#pragma unroll
                for (int hv = 0; hv < NHV; hv++) acc[hv][i] *= alpha;
                st.lsum[i] *= alpha;
                st.zsum[i] *= alpha;
                st.m[i] = mnew;
            }
            const float mref = (st.m[i] == -INFINITY) ? 0.f : st.m[i];
            float p = 0.f;
            if (valid) p = exp2f(sc[i] - mref + ((FMT == FMT_BF16) ? 0.f : 15.f));
            st.lsum[i] += p;
            if (FMT != FMT_BF16) {
                if (valid) st.zsum[i] = fmaf(p, zV, st.zsum[i]);
                pt[i] = valid ? p * sV : 0.f;
            } else {
                pt[i] = p;
            }
        }
    }

    // fp16 hi/lo of the PV operand, exchanged so that quad st holds step st's 4 positions:
    // lds_p[st][head][hi k0..k3 | lo k0..k3]
    __device__ __forceinline__ void exchange_h(const float (&pt)[4], int st_w, int kk, float fs, bool writer,
                                               half4_t& Ahi, half4_t& Alo)
    {
        uint16_t* L16 = (uint16_t*)lds_p;
        if (writer) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float x = pt[i] * fs;
                const _Float16 hi = (_Float16)x;
                const _Float16 lo = (_Float16)(x - (float)hi);
                L16[(st_w * 4 + i) * 8 + kk] = f16_bits(hi);
                L16[(st_w * 4 + i) * 8 + 4 + kk] = f16_bits(lo);
            }
        }
        wave_lds_sync();
        const u32x4 v = *(const u32x4*)(lds_p + lane * 16);
        Ahi = to_half4(v.x, v.y);
        Alo = to_half4(v.z, v.w);
        wave_lds_sync();
    }

    // ---- INT4 step: pages p_first .. p_first+3 of the INT4 range ----
    __device__ void int4_step(const DecodeUnit& U, int p_first, int p_end)
    {
        const int npg = min(kInt4StepPages, p_end - p_first);
        const int pj = lane >> 4, t16 = lane & 15;
        const int pos = (p_first + pj) * kPageSize + t16;
        const bool have = pj < npg;
        const bool valid = have && pos >= a.sinks && pos < U.len - a.recent;
        const int32_t* btr = a.bt + (int64_t)U.seq * a.max_pps;
        const int64_t hoff = (int64_t)U.head * a.page_block;

        u32x4 kc[D / 32];
        u32x2 szl = (u32x2){0u, 0u};
        if (have) {
            const uint8_t* pbl = a.pool + (int64_t)btr[p_first + pj] * a.hkv * a.page_block + hoff;
#pragma unroll
            for (int c = 0; c < D / 32; c++) kc[c] = *(const u32x4*)(pbl + c * 256 + t16 * 16);
            szl = *(const u32x2*)(pbl + 16 * D + t16 * 8);
        } else {
#pragma unroll
            for (int c = 0; c < D / 32; c++) kc[c] = (u32x4){0u, 0u, 0u, 0u};
        }
        u32x2 vc[kInt4StepPages][NHV];
#pragma unroll
        for (int q = 0; q < kInt4StepPages; q++) {
            if (q < npg) {
                const uint8_t* pbq = a.pool + (int64_t)btr[p_first + q] * a.hkv * a.page_block + hoff;
#pragma unroll
                for (int hv = 0; hv < NHV; hv++) vc[q][hv] = *(const u32x2*)(pbq + 8 * D + (64 * hv + lane) * 8);
            } else {
#pragma unroll
                for (int hv = 0; hv < NHV; hv++) vc[q][hv] = (u32x2){0u, 0u};
            }
        }

        // QK: steps m = 16c + 4wd + 2gp + hl
        float4_t S = (float4_t){0.f, 0.f, 0.f, 0.f};
        static_for<0, D / 32>([&](auto C) {
            static_for<0, 4>([&](auto WD) {
                const uint32_t w = kc[C][(int)WD];
                const uint32_t w8 = w >> 8;
                const half4_t B0 = to_half4(w & 0x000F000Fu, w & 0x00F000F0u);
                const half4_t B1 = to_half4(w8 & 0x000F000Fu, w8 & 0x00F000F0u);
                constexpr int m0 = (4 * C + WD) * 4;
                S = mfma_h<(m0 + 0) % 16>(A4[C], B0, S);
                S = mfma_h<(m0 + 1) % 16>(A4[C], B0, S);
                S = mfma_h<(m0 + 2) % 16>(A4[C], B1, S);
                S = mfma_h<(m0 + 3) % 16>(A4[C], B1, S);
            });
        });

        const float sK = f16_bits_to_float(szl.x & 0xFFFFu), zK = f16_bits_to_float(szl.x >> 16);
        const float sV = f16_bits_to_float(szl.y & 0xFFFFu), zV = f16_bits_to_float(szl.y >> 16);
        const float sK24 = sK * 16777216.0f;
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; i++) sc[i] = valid ? st.F[i] * fmaf(S[i], sK24, zK * st.sumq[i]) : -INFINITY;
        const float lg = (sV > 0.f) ? __log2f(sV) : -24.f;
        float pt[4];
        softmax_update(sc, lg, valid, sV, zV, pt);

        // exchange: position t16 = 8wd + n -> PV step 4pj + 2wd + (n>>1 & 1), slot kk
        const int n = t16 & 7, wd = t16 >> 3;
        const int st_w = pj * 4 + wd * 2 + ((n >> 1) & 1);
        const int kk = ((n >> 2) & 1) | ((n & 1) << 1);
        half4_t Ahi, Alo;
        exchange_h(pt, st_w, kk, (n & 1) ? 0.0625f : 1.0f, true, Ahi, Alo);

        static_for<0, kInt4StepPages>([&](auto PJ) {
            static_for<0, 2>([&](auto WD) {
                static_for<0, NHV>([&](auto HV) {
                    const uint32_t w = vc[PJ][HV][(int)WD];
                    const uint32_t w8 = w >> 8;
                    const half4_t B0 = to_half4(w & 0x000F000Fu, w & 0x00F000F0u);
                    const half4_t B1 = to_half4(w8 & 0x000F000Fu, w8 & 0x00F000F0u);
                    constexpr int s0 = PJ * 4 + WD * 2;
                    acc[HV] = mfma_h<s0>(Ahi, B0, acc[HV]);
                    acc[HV] = mfma_h<s0>(Alo, B0, acc[HV]);
                    acc[HV] = mfma_h<s0 + 1>(Ahi, B1, acc[HV]);
                    acc[HV] = mfma_h<s0 + 1>(Alo, B1, acc[HV]);
                });
            });
        });
    }

    // ---- INT8 step: 32 slots (protection segment) or 2 pages (INT8 format) ----
    __device__ void int8_step(const DecodeUnit& U, int j)
    {
        const bool lane_ok = lane < 32;
        const int sl = lane & 31;
        const uint8_t* tile_base[2] = {nullptr, nullptr};
        const int32_t* btr = a.bt + (int64_t)U.seq * a.max_pps;
        bool tile_ok[2];
        int pos = -1;
        bool valid = false;
        if constexpr (FMT == FMT_INT4_PROT) {
            const uint8_t* seg = a.int8_pool + ((int64_t)U.seq * a.hkv + U.head) * a.int8_tiles * a.int8_tile;
#pragma unroll
            for (int tt = 0; tt < 2; tt++) {
                const int tile = 2 * j + tt;
                tile_ok[tt] = tile < a.int8_tiles;
                tile_base[tt] = seg + (int64_t)tile * a.int8_tile;
            }
            const int u = kInt8StepSlots * j + sl;
            const int L = U.len;
            if (lane_ok && u < a.sinks + a.recent) {
                if (u < a.sinks) {
                    valid = u < L;
                } else {
                    const int jr = u - a.sinks;
                    const int back = L - 1 - jr;
                    if (back >= 0) {
                        const int tpos = L - 1 - back % a.recent;
                        valid = tpos >= a.sinks;
                    }
                }
            }
        } else {
            const int npages = (U.len + kPageSize - 1) / kPageSize;
#pragma unroll
            for (int tt = 0; tt < 2; tt++) {
                const int pg = 2 * j + tt;
                tile_ok[tt] = pg < npages;
                tile_base[tt] = tile_ok[tt] ? a.pool + (int64_t)btr[pg] * a.hkv * a.page_block +
                                                  (int64_t)U.head * a.page_block
                                            : a.pool;
            }
            pos = (2 * j + (sl >> 4)) * kPageSize + (sl & 15);
            valid = lane_ok && pos < U.len;
        }
        const int my_tile = sl >> 4, s8 = sl & 15;
        const bool have = lane_ok && (my_tile == 0 ? tile_ok[0] : tile_ok[1]);
        const uint8_t* tb = my_tile == 0 ? tile_base[0] : tile_base[1];

        u32x4 k8[D / 16];
        u32x2 szl = (u32x2){0u, 0u};
        if (have) {
#pragma unroll
            for (int c = 0; c < D / 16; c++) k8[c] = *(const u32x4*)(tb + c * 256 + s8 * 16);
            szl = *(const u32x2*)(tb + 32 * D + s8 * 8);
        } else {
#pragma unroll
            for (int c = 0; c < D / 16; c++) k8[c] = (u32x4){0u, 0u, 0u, 0u};
        }
        u32x4 v8[2][NHV];
#pragma unroll
        for (int tt = 0; tt < 2; tt++) {
#pragma unroll
            for (int hv = 0; hv < NHV; hv++)
                v8[tt][hv] = tile_ok[tt] ? *(const u32x4*)(tile_base[tt] + 16 * D + (64 * hv + lane) * 16)
                                         : (u32x4){0u, 0u, 0u, 0u};
        }

        // QK: word (c, wd) holds dims 4u..4u+3, u = 4c + wd; steps m = 2u + hl
        float4_t S = (float4_t){0.f, 0.f, 0.f, 0.f};
        static_for<0, D / 16>([&](auto C) {
            static_for<0, 4>([&](auto WD) {
                const uint32_t w = k8[C][(int)WD];
                const half4_t B = to_half4(__builtin_amdgcn_perm(0u, w, 0x0C010C00u),
                                           __builtin_amdgcn_perm(0u, w, 0x0C030C02u));
                constexpr int u = 4 * C + WD;
                S = mfma_h<(2 * u) % 16>(A8[(2 * u) / 16], B, S);
                S = mfma_h<(2 * u + 1) % 16>(A8[(2 * u + 1) / 16], B, S);
            });
        });

        const float sK = f16_bits_to_float(szl.x & 0xFFFFu), zK = f16_bits_to_float(szl.x >> 16);
        const float sV = f16_bits_to_float(szl.y & 0xFFFFu), zV = f16_bits_to_float(szl.y >> 16);
        const float sK24 = sK * 16777216.0f;
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; i++) sc[i] = valid ? st.F[i] * fmaf(S[i], sK24, zK * st.sumq[i]) : -INFINITY;
        const float lg = (sV > 0.f) ? __log2f(sV) : -24.f;
        float pt[4];
        softmax_update(sc, lg, valid, sV, zV, pt);

        half4_t Ahi, Alo;
        exchange_h(pt, sl >> 2, sl & 3, 1.0f, lane_ok, Ahi, Alo);

        static_for<0, 2>([&](auto TT) {
            static_for<0, 4>([&](auto Q) {
                static_for<0, NHV>([&](auto HV) {
                    const uint32_t w = v8[TT][HV][(int)Q];
                    const half4_t B = to_half4(__builtin_amdgcn_perm(0u, w, 0x0C010C00u),
                                               __builtin_amdgcn_perm(0u, w, 0x0C030C02u));
                    constexpr int s0 = 4 * TT + Q;
                    acc[HV] = mfma_h<s0>(Ahi, B, acc[HV]);
                    acc[HV] = mfma_h<s0>(Alo, B, acc[HV]);
                });
            });
        });
    }

    // ---- BF16 step: one page, lanes 0..15 ----
    __device__ void bf16_step(const DecodeUnit& U, int pg)
    {
        const int32_t* btr = a.bt + (int64_t)U.seq * a.max_pps;
        const uint8_t* pb = a.pool + (int64_t)btr[pg] * a.hkv * a.page_block + (int64_t)U.head * a.page_block;
        const int nvalid = min(kPageSize, U.len - pg * kPageSize);
        const bool valid = lane < nvalid;
        u32x4 kr[D / 8];
        if (lane < kPageSize) {
#pragma unroll
            for (int c = 0; c < D / 8; c++) kr[c] = *(const u32x4*)(pb + c * 256 + lane * 16);
        } else {
#pragma unroll
            for (int c = 0; c < D / 8; c++) kr[c] = (u32x4){0u, 0u, 0u, 0u};
        }
        u32x4 vv[NHV][2];
#pragma unroll
        for (int hv = 0; hv < NHV; hv++) {
#pragma unroll
            for (int q = 0; q < 2; q++) vv[hv][q] = *(const u32x4*)(pb + 32 * D + (64 * hv + lane) * 32 + 16 * q);
        }
        if (nvalid < kPageSize) {
            // positions >= L hold unspecified bytes: clear them so that 0 * garbage cannot be NaN
#pragma unroll
            for (int hv = 0; hv < NHV; hv++)
#pragma unroll
                for (int q = 0; q < 2; q++)
#pragma unroll
                    for (int k = 0; k < 4; k++) {
                        const int s_lo = 8 * q + 2 * k;
                        uint32_t m = 0u;
                        if (s_lo < nvalid) m |= 0x0000FFFFu;
                        if (s_lo + 1 < nvalid) m |= 0xFFFF0000u;
                        vv[hv][q][k] &= m;
                    }
        }

        float4_t S = (float4_t){0.f, 0.f, 0.f, 0.f};
        static_for<0, D / 8>([&](auto C) {
            constexpr int m0 = 2 * C;
            S = mfma_bf<m0 % 16>(Abf[m0 / 16], to_short4(kr[C].x, kr[C].y), S);
            S = mfma_bf<(m0 + 1) % 16>(Abf[(m0 + 1) / 16], to_short4(kr[C].z, kr[C].w), S);
        });
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; i++) sc[i] = valid ? st.F[i] * S[i] : -INFINITY;
        float pt[4];
        softmax_update(sc, 0.f, valid, 1.f, 0.f, pt);

        // bf16 hi/lo exchange (truncation split; hi + lo carries 16 significant bits)
        uint16_t* L16 = (uint16_t*)lds_p;
        if (lane < kPageSize) {
            const int stw = lane >> 2, kk = lane & 3;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint32_t hb = as_uint(pt[i]) & 0xFFFF0000u;
                const float lo = pt[i] - as_float(hb);
                L16[(stw * 4 + i) * 8 + kk] = (uint16_t)(hb >> 16);
                L16[(stw * 4 + i) * 8 + 4 + kk] = (uint16_t)(as_uint(lo) >> 16);
            }
        }
        wave_lds_sync();
        const u32x4 pv = *(const u32x4*)(lds_p + lane * 16);
        const short4_t Ahi = to_short4(pv.x, pv.y), Alo = to_short4(pv.z, pv.w);
        wave_lds_sync();
        static_for<0, 4>([&](auto ST) {
            static_for<0, NHV>([&](auto HV) {
                const u32x4 w = vv[HV][ST / 2];
                const short4_t B = (ST % 2 == 0) ? to_short4(w.x, w.y) : to_short4(w.z, w.w);
                acc[HV] = mfma_bf<ST>(Ahi, B, acc[HV]);
                acc[HV] = mfma_bf<ST>(Alo, B, acc[HV]);
            });
        });
    }

    __device__ void epilogue(int64_t pidx)
    {
#pragma unroll
        for (int i = 0; i < G; i++) {
            const float l = wave_sum(st.lsum[i]);
            const float z = (FMT == FMT_BF16) ? 0.f : wave_sum(st.zsum[i]);
            float* po = a.part_o + (pidx * G + i) * D;
#pragma unroll
            for (int hv = 0; hv < NHV; hv++) {
                const float v = (FMT == FMT_BF16) ? acc[hv][i] : fmaf(acc[hv][i], 16777216.0f, z);
                po[64 * hv + lane] = v;
            }
            if (lane == 0) {
                float mref = st.m[i];
                if (mref != -INFINITY && FMT != FMT_BF16) mref -= 15.f;
                a.part_ml[(pidx * G + i) * 2 + 0] = mref;
                a.part_ml[(pidx * G + i) * 2 + 1] = l;
            }
        }
    }
};

template <int D, int G, int FMT>
__global__ __launch_bounds__(64 * kWavesPerBlock) void decode_split_kernel(DecodeArgs a)
{
    __shared__ __align__(16) uint8_t lds_all[kWavesPerBlock][kLdsPerWave];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + wv;
    if (w >= a.n_waves) return;
    const int64_t T = a.total_steps, W = a.n_waves;
    int64_t s = w * T / W;
    const int64_t s_end = (w + 1) * T / W;
    if (s >= s_end) return;
    int lo = 0, hi = a.n_units - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.units[mid].step_begin <= s)
            lo = mid;
        else
            hi = mid - 1;
    }
    int u = lo;
    DecodeWave<D, G, FMT> dw(a, lane, lds_all[wv], lds_all[wv] + kLdsQBytes);
    while (s < s_end) {
        const DecodeUnit U = a.units[u];
        const int64_t ue = (u + 1 < a.n_units) ? a.units[u + 1].step_begin : T;
        const int k0 = (int)(s - U.step_begin);
        const int k1 = (int)((s_end < ue ? s_end : ue) - U.step_begin);
        int n8 = 0, p0 = 0, p1 = 0;
        if constexpr (FMT == FMT_INT4_PROT) {
            n8 = (a.sinks + a.recent > 0) ? (a.sinks + a.recent + kInt8StepSlots - 1) / kInt8StepSlots : 0;
            const int lo4 = a.sinks, hi4 = U.len - a.recent;
            if (hi4 > lo4) {
                p0 = lo4 / kPageSize;
                p1 = (hi4 - 1) / kPageSize + 1;
            }
        }
        const bool need8 = (FMT == FMT_INT8) || (FMT == FMT_INT4_PROT && k0 < n8);
        const bool need4 = (FMT == FMT_INT4_PROT) && k1 > n8;
        dw.prologue(U, need4, need8);
        for (int k = k0; k < k1; k++) {
            if constexpr (FMT == FMT_INT4_PROT) {
                if (k < n8)
                    dw.int8_step(U, k);
                else
                    dw.int4_step(U, p0 + kInt4StepPages * (k - n8), p1);
            } else if constexpr (FMT == FMT_INT8) {
                dw.int8_step(U, k);
            } else {
                dw.bf16_step(U, k);
            }
        }
        dw.epilogue(w + u);
        s = U.step_begin + k1;
        u++;
    }
}

// ---------------------------------------------------------------------------------------------
// merge: one block of D threads per unit
// ---------------------------------------------------------------------------------------------

__device__ __forceinline__ int64_t wave_of_step(int64_t step, int64_t T, int64_t W)
{
    int64_t w = ((step + 1) * W - 1) / T;
    return w < W - 1 ? w : W - 1;
}

template <int D, int G, bool ROT>
__global__ __launch_bounds__(D) void merge_kernel(DecodeArgs a)
{
    __shared__ float buf[D];
    const int u = blockIdx.x;
    const int d = threadIdx.x;
    const DecodeUnit U = a.units[u];
    const int64_t T = a.total_steps, W = a.n_waves;
    const int64_t sb = U.step_begin;
    const int64_t se = (u + 1 < a.n_units) ? a.units[u + 1].step_begin : T;
    const int64_t w0 = wave_of_step(sb, T, W), w1 = wave_of_step(se - 1, T, W);
    for (int i = 0; i < G; i++) {
        float M = -INFINITY;
        for (int64_t w = w0; w <= w1; w++) M = fmaxf(M, a.part_ml[((w + u) * G + i) * 2]);
        float Ls = 0.f, O = 0.f;
        if (M != -INFINITY) {
            for (int64_t w = w0; w <= w1; w++) {
                const float mw = a.part_ml[((w + u) * G + i) * 2];
                if (mw == -INFINITY) continue;
                const float f = exp2f(mw - M);
                Ls = fmaf(a.part_ml[((w + u) * G + i) * 2 + 1], f, Ls);
                O = fmaf(a.part_o[((w + u) * G + i) * D + d], f, O);
            }
        }
        float r = (Ls > 0.f) ? O / Ls : 0.f;
        if (ROT && a.block > 1) {
            buf[d] = r;
            for (int hh = 1; hh < a.block; hh <<= 1) {
                __syncthreads();
                const float other = buf[d ^ hh];
                const float mine = buf[d];
                __syncthreads();
                buf[d] = (d & hh) ? other - mine : mine + other;
            }
            __syncthreads();
            r = buf[d] * a.cb;
            __syncthreads();
        }
        a.out[((int64_t)U.entry * (a.hkv * G) + U.head * G + i) * D + d] = r;
    }
}

// ---------------------------------------------------------------------------------------------
// launches
// ---------------------------------------------------------------------------------------------

hipError_t launch_append(int d, int format, int n_tasks, const AppendArgs& a, hipStream_t stream)
{
    if (n_tasks <= 0) return hipSuccess;
    dim3 grid((unsigned)n_tasks, (unsigned)a.hkv), block(64);
#define KV4_APPEND_CASE(DD, FF)                                                          \
    if (d == DD && format == FF) {                                                       \
        hipLaunchKernelGGL((append_kernel<DD, FF>), grid, block, 0, stream, a);          \
        return hipGetLastError();                                                        \
    }
    KV4_APPEND_CASE(64, 0)
    KV4_APPEND_CASE(64, 1)
    KV4_APPEND_CASE(64, 2)
    KV4_APPEND_CASE(128, 0)
    KV4_APPEND_CASE(128, 1)
    KV4_APPEND_CASE(128, 2)
#undef KV4_APPEND_CASE
    return hipErrorInvalidValue;
}

template <int D, int G, int F>
static hipError_t launch_split_t(const DecodeArgs& a, hipStream_t stream)
{
    const unsigned blocks = (unsigned)((a.n_waves + kWavesPerBlock - 1) / kWavesPerBlock);
    hipLaunchKernelGGL((decode_split_kernel<D, G, F>), dim3(blocks), dim3(64 * kWavesPerBlock), 0, stream, a);
    return hipGetLastError();
}

template <int D, int G, int F>
static hipError_t launch_merge_t(const DecodeArgs& a, hipStream_t stream)
{
    hipLaunchKernelGGL((merge_kernel<D, G, F != FMT_BF16>), dim3((unsigned)a.n_units), dim3(D), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_decode_split(int d, int g, int format, const DecodeArgs& a, hipStream_t stream)
{
    if (a.n_units <= 0) return hipSuccess;
#define KV4_DEC_CASE(DD, GG, FF) \
    if (d == DD && g == GG && format == FF) return launch_split_t<DD, GG, FF>(a, stream);
#define KV4_DEC_G(DD, FF) KV4_DEC_CASE(DD, 1, FF) KV4_DEC_CASE(DD, 2, FF) KV4_DEC_CASE(DD, 4, FF)
    KV4_DEC_G(64, 0)
    KV4_DEC_G(64, 1)
    KV4_DEC_G(64, 2)
    KV4_DEC_G(128, 0)
    KV4_DEC_G(128, 1)
    KV4_DEC_G(128, 2)
#undef KV4_DEC_G
#undef KV4_DEC_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_decode_merge(int d, int g, int format, const DecodeArgs& a, hipStream_t stream)
{
    if (a.n_units <= 0) return hipSuccess;
#define KV4_DEC_CASE(DD, GG, FF) \
    if (d == DD && g == GG && format == FF) return launch_merge_t<DD, GG, FF>(a, stream);
#define KV4_DEC_G(DD, FF) KV4_DEC_CASE(DD, 1, FF) KV4_DEC_CASE(DD, 2, FF) KV4_DEC_CASE(DD, 4, FF)
    KV4_DEC_G(64, 0)
    KV4_DEC_G(64, 1)
    KV4_DEC_G(64, 2)
    KV4_DEC_G(128, 0)
    KV4_DEC_G(128, 1)
    KV4_DEC_G(128, 2)
#undef KV4_DEC_G
#undef KV4_DEC_CASE
    return hipErrorInvalidValue;
}

} // namespace kv4
