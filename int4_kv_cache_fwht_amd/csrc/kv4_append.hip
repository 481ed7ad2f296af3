// kv4_append.hip -- fused block-FWHT + token-wise quantization + nibble packing + paged store, plus
// the INT8 copy of protected positions.  Sources: "SAW-INT4: System-Aware 4-Bit KV-Cache
// Quantization for Real-World LLM Serving", Abstract (a fused rotation-quantization kernel writing
// into paged KV layouts); "KV4-RL: Unlocking Faster Asynchronous Rollouts for RLVR with INT4 KV
// Cache Quantization", Abstract (INT8 protection of attention sinks and recent context).
//
// Build with -ffp-contract=off: every binary32 step here must stay a single IEEE operation so that
// codes and scales match the oracle bit for bit.
#include "kv4_common.h"

namespace kv4 {

// ---------------------------------------------------------------------------------------------
// append
// ---------------------------------------------------------------------------------------------
// One wave per (task, kv head).  Lane l handles row l/2 (rows 0..15: K of page slot 0..15,
// rows 16..31: V of slot 0..15): with Q = D/4 and h = l%2, its values are dims Q h .. Q h + Q - 1
// and D/2 + Q h .. D/2 + Q h + Q - 1.  A rotate-half RoPE pair (i, i + D/2) then sits in one lane;
// the butterfly stages of span < Q run inside each quarter block, span Q pairs the lanes l and
// l ^ 1, and span D/2 pairs the lane's two quarter blocks.

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

// The stage whose pairs span the lane pair: the partner lane holds the other value of each pair.
// Half 0 (dim i) takes own + partner, half 1 (dim i + span) partner - own: one DPP move and one
// fma with a factor of +-1 per value (rounded once, like the add or subtract it replaces).
template <int N>
__device__ __forceinline__ void fwht_across_pair(float (&y)[N], int half)
{
    const float sgn = half ? -1.f : 1.f;
#pragma unroll
    for (int i = 0; i < N; i++) y[i] = butterfly_xor<1>(y[i], sgn);
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

// ROT: 0 no rotation (block 1, and the BF16 format), 2 the full block (block == D: every stage,
// with no test between them), 1 any other block (stages tested against the block at run time).
template <int D, int FMT, int ROT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(FMT == FMT_INT4_PROT ? 4 : 1))) void append_kernel(AppendArgs a)
{
    constexpr int N = D / 2; // values per lane
    constexpr int Q = D / 4; // dims per quarter block
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
    // dim of the lane's value i
    auto dimof = [&](int i) { return i < Q ? Q * half + i : D / 2 + Q * half + (i - Q); };

    u32x4 raw[N / 8];
    if (active) {
        const uint16_t* src = (is_v ? a.v : a.k) + ((int64_t)(tk.row0 + slot - s0) * a.hkv + h) * D;
#pragma unroll
        for (int q = 0; q < N / 8; q++) raw[q] = *(const u32x4*)(src + dimof(8 * q));
    } else {
#pragma unroll
        for (int q = 0; q < N / 8; q++) raw[q] = (u32x4){0u, 0u, 0u, 0u};
    }
    // fused RoPE: the key row's cos / sin table values for its dims Q h + j (j < Q), loaded with
    // the rows so that their latency overlaps
    const bool rope = FMT != FMT_BF16 && a.rope_cos != nullptr && !is_v;
    float4_t rc[FMT != FMT_BF16 ? Q / 4 : 1], rs[FMT != FMT_BF16 ? Q / 4 : 1];
    if constexpr (FMT != FMT_BF16) {
        if (rope) {
            const int tr = active ? t : 0;
            const float* cr = a.rope_cos + (int64_t)tr * N + Q * half;
            const float* sr = a.rope_sin + (int64_t)tr * N + Q * half;
#pragma unroll
            for (int q = 0; q < Q / 4; q++) {
                rc[q] = *(const float4_t*)(cr + 4 * q);
                rs[q] = *(const float4_t*)(sr + 4 * q);
            }
        }
    }

    if constexpr (FMT == FMT_BF16) {
        uint16_t* lds_bf = (uint16_t*)lds; // [16][D]
        if (active) {
            if (!is_v) {
                // K: [D/8 chunks][16 slots][16 B]
#pragma unroll
                for (int q = 0; q < N / 8; q++) *(u32x4*)(pb + (dimof(8 * q) / 8) * 256 + slot * 16) = raw[q];
            } else {
#pragma unroll
                for (int q = 0; q < N / 8; q++) *(u32x4*)(lds_bf + slot * D + dimof(8 * q)) = raw[q];
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
        // bf16 -> fp32 by pairs of 8-value groups (q in the first quarter block, q + Q/8 in the
        // second), each pair followed by the fused RoPE of its key values: the pair (i, i + D/2)
        // is values j and j + Q of the lane (i = Q h + j); binary32,
        // (x_i c - x_{i+D/2} s, x_{i+D/2} c + x_i s) with the caller's table row of t
        float y[N];
#pragma unroll
        for (int q = 0; q < Q / 8; q++) {
#pragma unroll
            for (int k = 0; k < 2; k++) {
                const int g8 = q + k * (Q / 8);
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    y[8 * g8 + 2 * j] = as_float(raw[g8][j] << 16);
                    y[8 * g8 + 2 * j + 1] = as_float(raw[g8][j] & 0xFFFF0000u);
                }
            }
            if (rope) {
#pragma unroll
                for (int j = 8 * q; j < 8 * q + 8; j++) {
                    const float c = rc[j / 4][j % 4], sn = rs[j / 4][j % 4];
                    const float x0 = y[j], x1 = y[Q + j];
                    y[j] = x0 * c - x1 * sn;
                    y[Q + j] = x1 * c + x0 * sn;
                }
            }
        }
        // stages h = 1, 2, ..., b/2 in that order: h < Q inside each quarter block, h = Q across
        // the lane pair, h = D/2 between the lane's two quarter blocks.  With the block a run-time
        // value, every stage is a branch and the 64 values are copied into place at each join; the
        // full block (the usual case) has the stages unconditional.
        if constexpr (ROT != 0) {
            const int b = (ROT == 2) ? D : a.block;
            fwht_in_lane<N>(y, b < Q ? b : Q);
            if (b > Q) fwht_across_pair<N>(y, half);
            if (b > D / 2) {
#pragma unroll
                for (int i = 0; i < Q; i++) {
                    const float a0 = y[i], c0 = y[i + Q];
                    y[i] = a0 + c0;
                    y[i + Q] = a0 - c0;
                }
            }
            if (b > 1) {
#pragma unroll
                for (int i = 0; i < N; i++) y[i] = y[i] * a.cb;
            }
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

        // ---- INT8 codes: protected positions (INT4_PROT), every position (INT8 format), and every
        // position when the INT4 codes are re-quantized from the INT8 round trip ----
        const bool want8 = (FMT == FMT_INT8) ? active : prot;
        const bool requant = (FMT == FMT_INT4_PROT) && a.requant != 0;
        const bool any8 = __ballot(want8) != 0ull; // some row of the page gets INT8 codes
        QuantParams qp8 = {};
        uint32_t cb8[N / 4];
        if (requant || any8) {
            qp8 = quant_params(mn, mx, 255.0f);
#pragma unroll
            for (int q = 0; q < N / 4; q++) {
                uint32_t w = 0;
                w = __builtin_amdgcn_cvt_pk_u8_f32((y[4 * q + 0] - qp8.zf) * qp8.inv, 0, w);
                w = __builtin_amdgcn_cvt_pk_u8_f32((y[4 * q + 1] - qp8.zf) * qp8.inv, 1, w);
                w = __builtin_amdgcn_cvt_pk_u8_f32((y[4 * q + 2] - qp8.zf) * qp8.inv, 2, w);
                w = __builtin_amdgcn_cvt_pk_u8_f32((y[4 * q + 3] - qp8.zf) * qp8.inv, 3, w);
                cb8[q] = w;
            }
        }

        if constexpr (FMT == FMT_INT4_PROT) {
            if (requant) {
                // the INT4 copy quantizes the INT8 round trip x8 = fl32(s8 * code8 + z8) (the
                // product is exact, so the fma rounds once, like product-then-sum)
                const float s8 = f16_bits_to_float(qp8.s_bits);
#pragma unroll
                for (int i = 0; i < N; i++) y[i] = fmaf(s8, (float)((cb8[i / 4] >> (8 * (i % 4))) & 0xFFu), qp8.zf);
                mn = y[0];
                mx = y[0];
#pragma unroll
                for (int i = 1; i < N; i++) {
                    mn = fminf(mn, y[i]);
                    mx = fmaxf(mx, y[i]);
                }
                mn = fminf(mn, dpp_xor1(mn));
                mx = fmaxf(mx, dpp_xor1(mx));
            }
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
                // K: [D/32 chunks][16 slots][16 B]; V staged as packed rows [16][D/2]
                if constexpr (Q >= 32) {
#pragma unroll
                    for (int c = 0; c < N / 32; c++) {
                        const int d0 = dimof(32 * c);
                        const u32x4 w = {pk[4 * c], pk[4 * c + 1], pk[4 * c + 2], pk[4 * c + 3]};
                        if (!is_v)
                            *(u32x4*)(pb + (d0 / 32) * 256 + slot * 16) = w;
                        else
                            *(u32x4*)(lds_v4 + slot * (D / 2) + d0 / 2) = w;
                    }
                } else {
#pragma unroll
                    for (int c = 0; c < N / 16; c++) {
                        const int d0 = dimof(16 * c);
                        const u32x2 w = {pk[2 * c], pk[2 * c + 1]};
                        if (!is_v)
                            *(u32x2*)(pb + (d0 / 32) * 256 + slot * 16 + (d0 % 32) / 2) = w;
                        else
                            *(u32x2*)(lds_v4 + slot * (D / 2) + d0 / 2) = w;
                    }
                }
                if (half == 0)
                    *(uint32_t*)(pb + 16 * D + slot * 8 + (is_v ? 4 : 0)) = qp.s_bits | (qp.z_bits << 16);
            }
        }

        // ---- INT8 stores ----
        {
            const QuantParams& qp = qp8;
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
                // the tile is two blocks of 16D + 128 bytes; block x holds K dims x*D/2 .. as
                // [D/32 chunks of 16 dims][16 slots][16 B]
                constexpr int BB = 16 * D + 128;
#pragma unroll
                for (int c = 0; c < N / 16; c++) {
                    const int d0 = dimof(16 * c);
                    const u32x4 w = {cb8[4 * c], cb8[4 * c + 1], cb8[4 * c + 2], cb8[4 * c + 3]};
                    if (!is_v)
                        *(u32x4*)(tb + (d0 / (D / 2)) * BB + ((d0 % (D / 2)) / 16) * 256 + s8 * 16) = w;
                    else
                        *(u32x4*)(lds_v8 + slot * D + d0) = w;
                }
                // scales: a copy in each block (block `half` from this lane)
                *(uint32_t*)(tb + half * BB + 16 * D + s8 * 8 + (is_v ? 4 : 0)) = qp.s_bits | (qp.z_bits << 16);
            }
        }
        __syncthreads();

        if constexpr (FMT == FMT_INT4_PROT) {
            // ---- dim-major V, [D][8 B] with nibble s = slot s: lane l < D/2 takes dims 2l and
            // 2l + 1 (byte l of every staged row) and writes their 16 B at once ----
            if (lane < D / 2) {
                uint32_t e0 = 0u, e1 = 0u, o0 = 0u, o1 = 0u; // dim 2l: slots 0-7, 8-15; dim 2l + 1: the same
#pragma unroll
                for (int s = 0; s < kPageSize; s++) {
                    const uint32_t b = lds_v4[s * (D / 2) + lane];
                    const uint32_t lo = b & 0xFu, hi = b >> 4;
                    if (s < 8) {
                        e0 |= lo << (4 * s);
                        o0 |= hi << (4 * s);
                    } else {
                        e1 |= lo << (4 * (s - 8));
                        o1 |= hi << (4 * (s - 8));
                    }
                }
                u32x4* dst = (u32x4*)(pb + 8 * D + 16 * lane);
                if (tk.n < kPageSize) {
                    // a partial page keeps the nibbles of the slots outside [s0, s1) (the staged
                    // rows of those slots were not written)
                    const uint64_t m = (((uint64_t)1 << (4 * tk.n)) - 1u) << (4 * s0);
                    const uint32_t mlo = (uint32_t)m, mhi = (uint32_t)(m >> 32);
                    const u32x4 old = *dst;
                    e0 = (old.x & ~mlo) | (e0 & mlo);
                    e1 = (old.y & ~mhi) | (e1 & mhi);
                    o0 = (old.z & ~mlo) | (o0 & mlo);
                    o1 = (old.w & ~mhi) | (o1 & mhi);
                }
                *dst = (u32x4){e0, e1, o0, o1};
            }
            // ---- INT8 copies of protected positions (pages that hold one): one byte per
            // (position, dim), lane = dim ----
            if (any8) {
#pragma unroll
                for (int dd = 0; dd < D / 64; dd++) {
                    const int d = dd * 64 + lane;
                    for (int s = s0; s < s1; s++) {
                        const int ts = tk.t0 - s0 + s;
                        if (!is_protected(ts, tk.len_new, a.sinks, a.recent)) continue;
                        const int u = (ts < a.sinks) ? ts : a.sinks + ts % a.recent;
                        uint8_t* tb = a.int8_pool + (((int64_t)tk.seq * a.hkv + h) * a.int8_tiles + (u >> 4)) * a.int8_tile;
                        // V of slot u % 16: block (u % 16) / 8, [D][8 B], byte (u % 8)
                        tb[((u >> 3) & 1) * (16 * D + 128) + 8 * D + d * 8 + (u & 7)] = lds_v8[s * D + d];
                    }
                }
            }
        } else {
            // ---- dim-major V stores (INT8 format): lane = dim ----
#pragma unroll
            for (int dd = 0; dd < D / 64; dd++) {
                const int d = dd * 64 + lane;
                // INT8 format: block x = slot / 8 holds V as [D][8 B], byte j = slot 8x + j
                u32x2* dst0 = (u32x2*)(pb + 8 * D + d * 8);
                u32x2* dst1 = (u32x2*)(pb + (16 * D + 128) + 8 * D + d * 8);
                u32x4 w = (tk.n < 16) ? (u32x4){(*dst0).x, (*dst0).y, (*dst1).x, (*dst1).y} : (u32x4){0u, 0u, 0u, 0u};
                for (int s = s0; s < s1; s++) {
                    uint32_t v = lds_v8[s * D + d];
                    int sh = (s & 3) * 8;
#pragma unroll
                    for (int j = 0; j < 4; j++)
                        if (j == (s >> 2)) w[j] = (w[j] & ~(0xFFu << sh)) | (v << sh);
                }
                *dst0 = (u32x2){w[0], w[1]};
                *dst1 = (u32x2){w[2], w[3]};
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// append of single positions (INT4_PROT): one wave per (task, kv head) for a task that writes one
// position.  Lane l holds dims PL*(l % 32) .. +PL-1 of the K row (l < 32) or the V row (l >= 32):
// the butterfly stages of span < PL run in the lane, the others pair lanes l and l ^ (span / PL)
// of the same row (same stage order and arithmetic as the page-task kernel, so the results are
// the same bits).  The V nibbles of the slot are merged into their bytes with a read-modify-write
// whose loads are issued together with the row loads.
// ---------------------------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(64) void append_token_kernel(AppendArgs a)
{
    constexpr int PL = D / 32; // dims per lane
    AppendTask tk;
    // task e from the argument block, read in place from the kernarg segment before the test of
    // n_arg (the loads do not wait for it).  With an uploaded task list the grid can exceed the
    // kArgEntries entries of the block, so the index is clamped into it; those values are unused.
    const int e = blockIdx.x;
    const int ea = e < kArgEntries ? e : 0;
    const __attribute__((address_space(4))) char* ka =
        (const __attribute__((address_space(4))) char*)__builtin_amdgcn_kernarg_segment_ptr();
    const int32_t pg = ((const __attribute__((address_space(4))) int32_t*)(ka + offsetof(AppendArgs, arg_page)))[ea];
    const int32_t aseq = ((const __attribute__((address_space(4))) int32_t*)(ka + offsetof(AppendArgs, arg_seq)))[ea];
    const int32_t at0 = ((const __attribute__((address_space(4))) int32_t*)(ka + offsetof(AppendArgs, arg_t0)))[ea];
    if (a.n_arg > 0) {
        // the host passes an argument plan only when every sequence of the call writes exactly
        // one position, so the sequence's length after the call is t0 + 1
        tk.seq = aseq;
        tk.t0 = at0;
        tk.page = pg & 0x7FFFFFFF;
        tk.flags = pg < 0 ? kTaskNewPage : 0;
        tk.n = 1;
        tk.row0 = e;
        tk.len_new = tk.t0 + 1;
        tk.bt_index = tk.seq * a.max_pps + tk.t0 / kPageSize;
    } else {
        tk = a.tasks[blockIdx.x];
    }
    const int h = blockIdx.y;
    const int lane = threadIdx.x;
    const int row = lane >> 5; // 0: K, 1: V
    const int l32 = lane & 31;
    const int d0 = PL * l32;
    const int slot = tk.t0 & (kPageSize - 1);
    if (lane == 0 && h == 0 && (tk.flags & kTaskNewPage)) a.bt[tk.bt_index] = tk.page;
    uint8_t* pb = a.pool + ((int64_t)tk.page * a.hkv + h) * a.page_block;

    // row values and the V bytes that hold this slot's nibbles (loaded by all lanes, used by V)
    const uint16_t* src = (row ? a.v : a.k) + ((int64_t)tk.row0 * a.hkv + h) * D + d0;
    uint16_t raw[PL];
#pragma unroll
    for (int j = 0; j < PL; j++) raw[j] = src[j];
    uint8_t* vbyte = pb + 8 * D + d0 * 8 + (slot >> 1);
    uint8_t old[PL];
#pragma unroll
    for (int j = 0; j < PL; j++) old[j] = vbyte[8 * j];
    // fused RoPE table values of the lane's dims (lanes l and l ^ 16 hold the pairs (i, i + D/2)),
    // loaded with the row
    const bool rope = a.rope_cos != nullptr;
    float rcv[PL], rsv[PL];
    if (rope) {
        const float* cr = a.rope_cos + (int64_t)tk.t0 * (D / 2) + PL * (l32 & 15);
        const float* sr = a.rope_sin + (int64_t)tk.t0 * (D / 2) + PL * (l32 & 15);
#pragma unroll
        for (int j = 0; j < PL; j++) {
            rcv[j] = cr[j];
            rsv[j] = sr[j];
        }
    }

    float y[PL];
#pragma unroll
    for (int j = 0; j < PL; j++) y[j] = as_float((uint32_t)raw[j] << 16);
    // fused RoPE of the key row: lanes l and l ^ 16 hold the pairs (i, i + D/2)
    if (rope) {
#pragma unroll
        for (int j = 0; j < PL; j++) {
            const float own = y[j];
            const float other = lane_xor16(own);
            const float oc = own * rcv[j], os = other * rsv[j];
            const float r = (l32 & 16) ? oc + os : oc - os;
            y[j] = row == 0 ? r : own;
        }
    }
    // stages h = 1, 2, ... < b in order
#pragma unroll
    for (int hh = 1; hh < PL; hh <<= 1) {
        if (hh < a.block) {
#pragma unroll
            for (int i = 0; i < PL; i++) {
                if ((i & hh) == 0) {
                    const float a0 = y[i], c0 = y[i + hh];
                    y[i] = a0 + c0;
                    y[i + hh] = a0 - c0;
                }
            }
        }
    }
    // then the stages h = PL * M < b across lanes: partner lane l ^ M (M <= 16 stays in the row's
    // 32 lanes), DPP moves and one swizzle instead of LDS permutes
    static_for<0, 5>([&](auto S) {
        constexpr int M = 1 << S;
        if (M * PL < a.block) {
            const float sgn = (l32 & M) ? -1.f : 1.f;
#pragma unroll
            for (int i = 0; i < PL; i++) y[i] = butterfly_xor<M>(y[i], sgn);
        }
    });
    if (a.block > 1) {
#pragma unroll
        for (int i = 0; i < PL; i++) y[i] = y[i] * a.cb;
    }
    // row min / max over the 32 lanes of the row
    float mn = y[0], mx = y[0];
#pragma unroll
    for (int i = 1; i < PL; i++) {
        mn = fminf(mn, y[i]);
        mx = fmaxf(mx, y[i]);
    }
    static_for<0, 5>([&](auto S) {
        constexpr int M = 1 << S;
        mn = fminf(mn, lane_xor<M>(mn));
        mx = fmaxf(mx, lane_xor<M>(mx));
    });

    // ---- INT8 codes: protected position, or INT4 re-quantized from the INT8 round trip ----
    const int t = tk.t0;
    const bool prot = is_protected(t, tk.len_new, a.sinks, a.recent);
    QuantParams qp8 = {};
    uint32_t c8[PL];
    if (prot || a.requant != 0) {
        qp8 = quant_params(mn, mx, 255.0f);
#pragma unroll
        for (int i = 0; i < PL; i++) c8[i] = __builtin_amdgcn_cvt_pk_u8_f32((y[i] - qp8.zf) * qp8.inv, 0, 0u);
    }
    if (a.requant != 0) {
        // x8 = fl32(s8 * code8 + z8): the product is exact, so the fma rounds once
        const float s8f = f16_bits_to_float(qp8.s_bits);
#pragma unroll
        for (int i = 0; i < PL; i++) y[i] = fmaf(s8f, (float)c8[i], qp8.zf);
        mn = y[0];
        mx = y[0];
#pragma unroll
        for (int i = 1; i < PL; i++) {
            mn = fminf(mn, y[i]);
            mx = fmaxf(mx, y[i]);
        }
        static_for<0, 5>([&](auto S) {
            constexpr int M = 1 << S;
            mn = fminf(mn, lane_xor<M>(mn));
            mx = fmaxf(mx, lane_xor<M>(mx));
        });
    }

    // ---- INT4 page copy ----
    {
        const QuantParams qp = quant_params(mn, mx, 15.0f);
        uint32_t c[PL];
#pragma unroll
        for (int i = 0; i < PL; i++) c[i] = __builtin_amdgcn_cvt_pk_u8_f32((y[i] - qp.zf) * qp.inv, 0, 0u);
        if (row == 0) {
            // K: [D/32 chunks][16 slots][16 B], byte k of a chunk = dims 2k (low), 2k+1 (high)
            uint8_t* dst = pb + (d0 / 32) * 256 + slot * 16 + (d0 % 32) / 2;
#pragma unroll
            for (int i = 0; i < PL; i += 2) dst[i / 2] = (uint8_t)(c[i] | (c[i + 1] << 4));
        } else {
            // V: [D dims][8 B], nibble s = slot s
#pragma unroll
            for (int j = 0; j < PL; j++) {
                const uint32_t b = (slot & 1) ? ((old[j] & 0x0Fu) | (c[j] << 4)) : ((old[j] & 0xF0u) | c[j]);
                vbyte[8 * j] = (uint8_t)b;
            }
        }
        if (l32 == 0) *(uint32_t*)(pb + 16 * D + slot * 8 + row * 4) = qp.s_bits | (qp.z_bits << 16);
    }

    // ---- INT8 copy when the position is protected ----
    if (prot) {
        const QuantParams& qp = qp8;
        const int u = (t < a.sinks) ? t : a.sinks + t % a.recent;
        uint8_t* tb = a.int8_pool + (((int64_t)tk.seq * a.hkv + h) * a.int8_tiles + (u >> 4)) * a.int8_tile;
        const int s8 = u & 15;
        const uint32_t (&c)[PL] = c8;
        constexpr int BB = 16 * D + 128; // the tile's two blocks
        if (row == 0) {
            // K of dims half x = d0 / (D/2): [D/32 chunks][16 slots][16 B], one byte per dim
            const int x = d0 / (D / 2), dx = d0 % (D / 2);
            uint8_t* dst = tb + x * BB + (dx / 16) * 256 + s8 * 16 + dx % 16;
#pragma unroll
            for (int i = 0; i < PL; i++) dst[i] = (uint8_t)c[i];
        } else {
            // V of slot s8: block s8 / 8, [D dims][8 B], byte s8 % 8
            uint8_t* dst = tb + (s8 >> 3) * BB + 8 * D + d0 * 8 + (s8 & 7);
#pragma unroll
            for (int j = 0; j < PL; j++) dst[8 * j] = (uint8_t)c[j];
        }
        if (l32 == 0) {
#pragma unroll
            for (int x = 0; x < 2; x++) *(uint32_t*)(tb + x * BB + 16 * D + s8 * 8 + row * 4) = qp.s_bits | (qp.z_bits << 16);
        }
    }
}

hipError_t launch_append_token(int d, int n_tasks, const AppendArgs& a, hipStream_t stream, const KernelTimer& tm)
{
    if (n_tasks <= 0) return hipSuccess;
    dim3 grid((unsigned)n_tasks, (unsigned)a.hkv), block(64);
    if (d == 64) return launch_kernel(append_token_kernel<64>, grid, block, stream, tm, a);
    if (d == 128) return launch_kernel(append_token_kernel<128>, grid, block, stream, tm, a);
    return hipErrorInvalidValue;
}

hipError_t launch_append(int d, int format, int n_tasks, const AppendArgs& a, hipStream_t stream,
                         const KernelTimer& tm)
{
    if (n_tasks <= 0) return hipSuccess;
    dim3 grid((unsigned)n_tasks, (unsigned)a.hkv), block(64);
#define KV4_APPEND_CASE(DD, FF)                                                                     \
    if (d == DD && format == FF) {                                                                  \
        if (FF == FMT_BF16 || a.block <= 1)                                                         \
            return launch_kernel(append_kernel<DD, FF, 0>, grid, block, stream, tm, a);             \
        if (FF != FMT_BF16 && a.block == DD)                                                        \
            return launch_kernel(append_kernel<DD, FF, FF == FMT_BF16 ? 0 : 2>, grid, block, stream, tm, a); \
        return launch_kernel(append_kernel<DD, FF, FF == FMT_BF16 ? 0 : 1>, grid, block, stream, tm, a); \
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

} // namespace kv4
