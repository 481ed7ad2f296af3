// kv4_mq.hip -- causal multi-query attention over the paged INT4 cache with INT8 sink/recent
// slots: several query positions per sequence (its last n positions: a prefill chunk, or the
// tokens of a multi-token decode step), each attending the positions up to its own.
// Sources: "SAW-INT4: System-Aware 4-Bit KV-Cache Quantization for Real-World LLM Serving",
// Abstract (fused attention over a paged INT4 cache after a block-diagonal Hadamard rotation);
// "KV4-RL: Unlocking Faster Asynchronous Rollouts for RLVR with INT4 KV Cache Quantization",
// Abstract (sinks and recent context read from INT8).
//
// A wave takes 16 query rows -- (query position, query head) pairs that share one kv head -- and
// a chunk of that (sequence, kv head)'s steps.  A step is 32 positions: two INT8 tiles (the
// protection slots, first) or two INT4 pages.  Both products run on v_mfma_f32_16x16x32_f16:
//   S^T = K Q^T:  the A operand is 16 positions' key codes as fp16 subnormal patterns (value
//                 code * 2^-24, exact; INT4 odd elements times 16); the B operand the rotated
//                 query rows, scaled by a power of two to below 2^14 (INT4 odd elements divided by
//                 16) and split into hi + lo fp16.  A score is s_K (q . code) + z_K sum(q).
//   O += P' V:    the A operand is p * s_V (hi + lo fp16), the B operand the value codes (stored
//                 dim-major) centred as fp16 integers (code - 8; INT8: - 128);
//                 sum_t p_t (z_V,t + 8 s_V,t) is accumulated per lane.
// Positions are assigned to the S^T rows so that the accumulator of lane l holds the scores of
// query row l % 16 for 8 consecutive positions of the step -- exactly the positions whose p * s_V
// lane l supplies to the PV operand, and whose value codes are one 4-byte (INT4) or 8-byte (INT8)
// run of each dim row.  The two products therefore need no exchange between lanes.
//
// Softmax reference: per query row, the running maximum of score + (exponent field of s_V, the
// largest over a lane's positions); it is raised only when a step exceeds it by more than kMqTau
// (then the accumulators are rescaled).  This bounds p * s_V * 2^27 below 2^14, inside the fp16
// range, whatever the value scales.
#include "kv4_common.cuh"

namespace kv4 {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

constexpr float kMqTau = 1.f;
constexpr float kPScale = 134217728.f; // 2^27

template <typename T>
__device__ __forceinline__ T mq_uniform(const T* p)
{
    return *(const __attribute__((address_space(4))) T*)p;
}

__device__ __forceinline__ float4_t mfma16x32(u32x4 a, u32x4 b, float4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c,
                                                  0, 0, 0);
}

// Eight INT4 key codes, nibble i = element i, one per 16-bit half in the element order
// (0, 4, 1, 5, 2, 6, 3, 7); as fp16 these are the subnormal patterns code * 2^-24, the odd
// elements multiplied by 16 (at most 240 * 2^-24, still exact): four ands and one shift.  The
// query operand carries the 1/16 of those elements.
__device__ __forceinline__ u32x4 spread_int4_x16(uint32_t w)
{
    const uint32_t w8 = w >> 8;
    return (u32x4){w & 0x000F000Fu, w & 0x00F000F0u, w8 & 0x000F000Fu, w8 & 0x00F000F0u};
}

// Eight INT8 codes (bytes of w0 = elements 0..3, of w1 = elements 4..7), same order.
__device__ __forceinline__ u32x4 spread_int8(uint32_t w0, uint32_t w1)
{
    return (u32x4){__builtin_amdgcn_perm(w1, w0, 0x0C040C00u), __builtin_amdgcn_perm(w1, w0, 0x0C050C01u),
                   __builtin_amdgcn_perm(w1, w0, 0x0C060C02u), __builtin_amdgcn_perm(w1, w0, 0x0C070C03u)};
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Spread value codes (code in the low bits of each half) -> code - MID as fp16 integers, MID = 8
// (INT4) or 128 (INT8): 0x6400 | code is the fp16 value 1024 + code, and one packed fp16
// subtraction of 1024 + MID is exact.  Centred codes keep the PV accumulators at the scale of the
// result: with raw codes they would hold about sum p (s_V * code midpoint), which the zero-point
// term then cancels, and the MFMA accumulation error of that large sum showed in the output at
// the 1e-4 level.  (The score path has no such cancellation; its key codes stay raw.)
template <int MID>
__device__ __forceinline__ u32x4 centre(u32x4 x)
{
    const half2_t off = {(_Float16)(-(1024 + MID)), (_Float16)(-(1024 + MID))};
    u32x4 r;
#pragma unroll
    for (int s = 0; s < 4; s++)
        r[s] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, x[s] | 0x64006400u) + off);
    return r;
}

// Eight INT4 value codes in the spread order, centred: (nibble | 0x6400) is the fp16 value
// 1024 + code, less 1024 + MID in one packed fp16 subtraction.  k6400 holds 0x64006400 in a
// vector register, so that mask-and-or is one v_and_or_b32 (two literals cannot share it).
template <int MID>
__device__ __forceinline__ u32x4 spread_centre_int4(uint32_t w, uint32_t k6400)
{
    const half2_t off = {(_Float16)(-(1024 + MID)), (_Float16)(-(1024 + MID))};
    u32x4 r;
#pragma unroll
    for (int s = 0; s < 4; s++)
        r[s] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, ((w >> (4 * s)) & 0x000F000Fu) | k6400) + off);
    return r;
}

// A pair of fp16 values times 16 (exact: the values stay below 2^14).
__device__ __forceinline__ uint32_t pair_x16(uint32_t v)
{
    const half2_t k16 = {(_Float16)16.f, (_Float16)16.f};
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, v) * k16);
}

// Query operand registers 1 and 3 (the odd elements) times 16, for key codes without that factor.
// The elements pass through pair_x16 by value: hipcc's bit cast of a vector-element lvalue (q[1])
// reads element 0.
__device__ __forceinline__ u32x4 odd_x16(u32x4 q)
{
    return (u32x4){q[0], pair_x16(q[1]), q[2], pair_x16(q[3])};
}

// hi + lo fp16 of eight floats, same element order as the spreads.
__device__ __forceinline__ void split_hilo(const float (&x)[8], u32x4& hi, u32x4& lo)
{
#pragma unroll
    for (int s = 0; s < 4; s++) {
        const _Float16 h0 = (_Float16)x[s], h1 = (_Float16)x[s + 4];
        const _Float16 l0 = (_Float16)(x[s] - (float)h0), l1 = (_Float16)(x[s + 4] - (float)h1);
        hi[s] = (uint32_t)f16_bits(h0) | ((uint32_t)f16_bits(h1) << 16);
        lo[s] = (uint32_t)f16_bits(l0) | ((uint32_t)f16_bits(l1) << 16);
    }
}

// hi + lo fp16 of eight floats (same element order), hi truncated toward zero: the residual
// x - hi is exact in fp32 and its own fp16 truncation leaves about 2^-20 of x.
__device__ __forceinline__ void split_hilo_rtz(const float (&x)[8], u32x4& hi, u32x4& lo)
{
#pragma unroll
    for (int s = 0; s < 4; s++) {
        const half2_t h = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(x[s], x[s + 4]));
        const float r0 = fmaf((float)h[0], -1.f, x[s]), r1 = fmaf((float)h[1], -1.f, x[s + 4]);
        hi[s] = __builtin_bit_cast(uint32_t, h);
        lo[s] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(r0, r1));
    }
}

__device__ __forceinline__ float lo_half(uint32_t d) { return (float)__builtin_bit_cast(half2_t, d)[0]; }
__device__ __forceinline__ float hi_half(uint32_t d) { return (float)__builtin_bit_cast(half2_t, d)[1]; }

__device__ __forceinline__ u32x4 ld16(const uint8_t* p) { return *(const u32x4*)p; }
__device__ __forceinline__ u32x2 ld8(const uint8_t* p) { return *(const u32x2*)p; }
__device__ __forceinline__ uint32_t ld4(const uint8_t* p) { return *(const uint32_t*)p; }

// The call entry that holds `key`: the last entry whose first task (GRP false) or first merge
// group (GRP true) is <= key (both increase along the entries).  Lane l reads entry l of each round
// of 64 and a ballot counts them: one load per round instead of a chain of dependent scalar loads.
template <bool GRP>
__device__ __forceinline__ int mq_find_entry(const MqArgs& a, int key, int lane)
{
    int cnt = 0;
    for (int e0 = 0; e0 < a.n_entries; e0 += 64) {
        const int e = e0 + lane;
        const int v = e < a.n_entries ? (GRP ? a.entries[e].grp0 : a.entries[e].task0) : 0x7FFFFFFF;
        cnt += __builtin_popcountll(__ballot(v <= key));
        if (__ballot(v > key) != 0ull) break;
    }
    return cnt - 1;
}

template <typename T>
__device__ __forceinline__ const T* pick(bool c, const T* x, const T* y)
{
    return c ? x : y;
}

template <int D, int G, int FMT>
struct MqWave {
    static constexpr int KS = D / 32;   // k-steps of S^T = INT4 key-code dwords per tile and lane
    static constexpr int NCB = D / 16;  // 16-dim column blocks of the output
    static constexpr int DPL = D / 4;   // query dims per lane in the prologue
    static constexpr int QT = kMqRows / G;
    static constexpr int IB = 16 * D + 128; // bytes of an INT4 page block / an INT8 tile block

    // One step's operands for this lane.  INT8 buffers hold twice the key and value bytes.
    template <bool IS8>
    struct Buf {
        uint32_t k[2][IS8 ? 2 * KS : KS];
        uint32_t v[NCB][IS8 ? 2 : 1];
        uint32_t sc[16];
    };

    const MqArgs& a;
    const int lane, n, g;
    int seq, L, head, pos_r;
    int first_pos;       // position of the row tile's first query (wave-uniform)
    int lo4, hi4;        // INT4_PROT: INT4-read positions [S, L - R)
    int ring_base, ring_mod; // INT4_PROT: first recent position and its residue mod R
    const uint8_t* t8;   // INT4_PROT: this (sequence, kv head)'s INT8 tiles
    const int32_t* btrow;
    const uint8_t* hbase; // the pool at this kv head's block of page 0
    uint32_t pstride;     // bytes from one page to the next (all kv heads' blocks)
    int p0, p1;          // INT4 page range (INT4_PROT) or page count (INT8 format: p1)
    float m_ref = -__builtin_inff(), lsum = 0.f, zsum = 0.f, Ar = 0.f, Br = 0.f;
    uint32_t k6400;      // 0x64006400 in a vector register (identity DPP move: not a literal)
    u32x4 qhi[KS], qlo[KS];
    float4_t acc[NCB];

    __device__ MqWave(const MqArgs& args, int l)
        : a(args), lane(l), n(l & 15), g(l >> 4),
          k6400((uint32_t)__builtin_amdgcn_update_dpp(0, 0x64006400, 0xE4, 0xF, 0xF, false))
    {
    }

    // Rotated, scaled query row n: dims DPL*g .. DPL*g + DPL - 1 held by this lane.
    __device__ void prologue(const MqEntry& e, int rt)
    {
        const int jq = rt * QT + n / G, gi = n % G;
        const bool row_ok = jq < e.nq;
        pos_r = row_ok ? e.len - e.nq + jq : -1;
        first_pos = e.len - e.nq + rt * QT;
        const uint16_t* qp = a.q + ((int64_t)(e.qrow0 + (row_ok ? jq : 0)) * a.hq + head * G + gi) * D + DPL * g;
        float x[DPL];
#pragma unroll
        for (int c = 0; c < DPL / 8; c++) {
            const u32x4 u = ld16((const uint8_t*)(qp + 8 * c));
#pragma unroll
            for (int j = 0; j < 4; j++) {
                x[8 * c + 2 * j] = row_ok ? as_float(u[j] << 16) : 0.f;
                x[8 * c + 2 * j + 1] = row_ok ? as_float(u[j] & 0xFFFF0000u) : 0.f;
            }
        }
        // FWHT over blocks of `block` dims: in-lane stages, then across the lanes of the row
#pragma unroll
        for (int h = 1; h < DPL; h <<= 1) {
            if (h < a.block) {
#pragma unroll
                for (int i = 0; i < DPL; i++) {
                    if (i & h) continue;
                    const float u = x[i], w = x[i + h];
                    x[i] = u + w;
                    x[i + h] = u - w;
                }
            }
        }
        static_for<0, 2>([&](auto ST) {
            constexpr int MASK = 16 << ST;
            if ((DPL << ST) < a.block) {
                const float sgn = (lane & MASK) ? -1.f : 1.f;
#pragma unroll
                for (int i = 0; i < DPL; i++) x[i] = butterfly_xor<MASK>(x[i], sgn);
            }
        });
        float sum = 0.f, mx = 0.f;
#pragma unroll
        for (int i = 0; i < DPL; i++) {
            x[i] *= a.cb;
            sum += x[i];
            mx = fmaxf(mx, fabsf(x[i]));
        }
        sum += lane_xor16(sum);
        sum = add_xor32(sum);
        mx = fmaxf(mx, lane_xor16(mx));
        mx = max_xor32(mx);
        const int E = __builtin_amdgcn_frexp_expf(mx); // mx < 2^E
        // q 2^(14-E): below 2^14, so that the fp16 hi and lo parts stay normal; the odd elements of
        // each group of 8 are divided by 16 (their INT4 key codes arrive multiplied by 16)
#pragma unroll
        for (int j = 0; j < KS; j++) {
            float y[8];
#pragma unroll
            for (int i = 0; i < 8; i++) y[i] = __builtin_ldexpf(x[8 * j + i], 14 - E - ((i & 1) ? 4 : 0));
            split_hilo(y, qhi[j], qlo[j]);
        }
        // score (log2 units) = Ar * s_K * acc + Br * z_K, acc = 2^-24 sum(q 2^(14-E) * code)
        Ar = __builtin_ldexpf(a.scale_log2, 24 + E - 14);
        Br = a.scale_log2 * sum;
#pragma unroll
        for (int c = 0; c < NCB; c++) acc[c] = (float4_t){0.f, 0.f, 0.f, 0.f};
    }

    // INT4 page pair of unit step s (s >= n8): pages p0 + 2 (s - n8) and the next (clamped).
    __device__ void load4(Buf<false>& b, int s) const
    {
        const int pi = p0 + 2 * (s - a.n8);
        const uint32_t pa = (uint32_t)mq_uniform(btrow + pi);
        const uint32_t pb = (uint32_t)mq_uniform(btrow + (pi + 1 < p1 ? pi + 1 : pi));
        // the lane picks its page id first: one 32x32 -> 64-bit multiply-add per pointer
        const int kslot = 8 * ((n >> 2) & 1) + (n & 3);
        const uint8_t* kp = hbase + (uint64_t)(n < 8 ? pa : pb) * pstride + kslot * 16;
        const uint8_t* vp = hbase + (uint64_t)(g < 2 ? pa : pb) * pstride;
        if constexpr (D == 128) {
            kp += 256 * g;
#pragma unroll
            for (int t = 0; t < 2; t++) {
                const u32x4 w = ld16(kp + 64 * t);
#pragma unroll
                for (int j = 0; j < 4; j++) b.k[t][j] = w[j];
            }
        } else {
            kp += 256 * (g >> 1) + 8 * (g & 1);
#pragma unroll
            for (int t = 0; t < 2; t++) {
                const u32x2 w = ld8(kp + 64 * t);
                b.k[t][0] = w[0];
                b.k[t][1] = w[1];
            }
        }
#pragma unroll
        for (int c = 0; c < NCB; c++) b.v[c][0] = ld4(vp + 8 * D + (16 * c + n) * 8 + 4 * (g & 1));
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const u32x4 w = ld16(vp + 16 * D + 64 * (g & 1) + 16 * j);
#pragma unroll
            for (int i = 0; i < 4; i++) b.sc[4 * j + i] = w[i];
        }
    }

    // Two INT8 tiles: ta (positions of the lane's key rows < 8) and tb.
    __device__ void load8(Buf<true>& b, const uint8_t* A, const uint8_t* B) const
    {
        const int kslot = 8 * ((n >> 2) & 1) + (n & 3);
        const uint8_t* kp = pick(n < 8, A, B) + IB * (g >> 1) + kslot * 16;
        const uint8_t* vp = pick(g < 2, A, B);
        if constexpr (D == 128) {
            kp += 512 * (g & 1);
#pragma unroll
            for (int t = 0; t < 2; t++) {
#pragma unroll
                for (int c = 0; c < 2; c++) {
                    const u32x4 w = ld16(kp + 64 * t + 256 * c);
#pragma unroll
                    for (int j = 0; j < 4; j++) b.k[t][4 * c + j] = w[j];
                }
            }
        } else {
            kp += 256 * (g & 1);
#pragma unroll
            for (int t = 0; t < 2; t++) {
                const u32x4 w = ld16(kp + 64 * t);
#pragma unroll
                for (int j = 0; j < 4; j++) b.k[t][j] = w[j];
            }
        }
#pragma unroll
        for (int c = 0; c < NCB; c++) {
            const u32x2 w = ld8(vp + IB * (g & 1) + 8 * D + (16 * c + n) * 8);
            b.v[c][0] = w[0];
            b.v[c][1] = w[1];
        }
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const u32x4 w = ld16(vp + 16 * D + 64 * (g & 1) + 16 * j);
#pragma unroll
            for (int i = 0; i < 4; i++) b.sc[4 * j + i] = w[i];
        }
    }

    __device__ void load8_step(Buf<true>& b, int s) const
    {
        if (FMT == FMT_INT8) {
            const int pa = mq_uniform(btrow + 2 * s);
            const int pb = mq_uniform(btrow + (2 * s + 1 < p1 ? 2 * s + 1 : 2 * s));
            load8(b, a.pool + ((int64_t)pa * a.hkv + head) * a.page_block,
                  a.pool + ((int64_t)pb * a.hkv + head) * a.page_block);
        } else {
            const int tb = 2 * s + 1 < a.int8_tiles ? 2 * s + 1 : 2 * s;
            load8(b, t8 + (int64_t)(2 * s) * a.int8_tile, t8 + (int64_t)tb * a.int8_tile);
        }
    }

    // Position of the lane's step element t (0..7) and whether this wave may read it at all.
    template <bool IS8>
    __device__ __forceinline__ void positions(int s, int (&pos)[8]) const
    {
        const int k0 = 8 * g;
        if (!IS8) {
            const int base = 16 * (p0 + 2 * (s - a.n8)) + k0;
#pragma unroll
            for (int t = 0; t < 8; t++) {
                const int p = base + t;
                pos[t] = (p >= lo4 && p < hi4) ? p : 0x7FFFFFFF;
            }
        } else if (FMT == FMT_INT8) {
            const int base = 32 * s + k0;
#pragma unroll
            for (int t = 0; t < 8; t++) pos[t] = base + t < L ? base + t : 0x7FFFFFFF;
        } else {
            const int base = 32 * s + k0;
#pragma unroll
            for (int t = 0; t < 8; t++) {
                const int u = base + t;
                int p = 0x7FFFFFFF;
                if (u < a.sinks) {
                    p = u < L ? u : 0x7FFFFFFF;
                } else if (u < a.sinks + a.recent) {
                    int r = (u - a.sinks) - ring_mod;
                    if (r < 0) r += a.recent;
                    const int q = ring_base + r;
                    p = q < L ? q : 0x7FFFFFFF;
                }
                pos[t] = p;
            }
        }
    }

    // One step.  FULL: every position of the step is readable and at or before every row's own
    // position (wave-uniform), so no per-position test is made.
    template <bool IS8, bool FULL>
    __device__ void compute(const Buf<IS8>& b, int s)
    {
        constexpr int MID = IS8 ? 128 : 8;
        int pos[8];
        if (!FULL) positions<IS8>(s, pos);
        // S^T for the two tiles
        float4_t sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KS; j++) {
            const u32x4 ka = IS8 ? spread_int8(b.k[0][2 * j], b.k[0][2 * j + 1]) : spread_int4_x16(b.k[0][j]);
            const u32x4 kb = IS8 ? spread_int8(b.k[1][2 * j], b.k[1][2 * j + 1]) : spread_int4_x16(b.k[1][j]);
            const u32x4 qh = IS8 ? odd_x16(qhi[j]) : qhi[j];
            const u32x4 ql = IS8 ? odd_x16(qlo[j]) : qlo[j];
            sa = mfma16x32(ka, qh, sa);
            sb = mfma16x32(kb, qh, sb);
            sa = mfma16x32(ka, ql, sa);
            sb = mfma16x32(kb, ql, sb);
        }
        // fp16 scales enter the fp32 arithmetic as fma operands (v_fma_mix_f32: no conversions).
        // The reference bound uses one exponent per lane: the largest s_V of the lane's readable
        // positions (positive fp16 patterns order like their values), so st + e_lane bounds
        // st + log2 s_V + 1 for each of them.
        float st[8];
        bool ok[8];
        float smax = -__builtin_inff();
        uint32_t svmax = 0;
#pragma unroll
        for (int t = 0; t < 8; t++) {
            const float r = t < 4 ? sa[t] : sb[t - 4];
            const uint32_t d0 = b.sc[2 * t], d1 = b.sc[2 * t + 1];
            st[t] = fmaf(lo_half(d0), r * Ar, fmaf(hi_half(d0), Br, 0.f));
            ok[t] = FULL || pos[t] <= pos_r;
            smax = ok[t] ? fmaxf(smax, st[t]) : smax;
            svmax = ok[t] ? max(svmax, d1 & 0xFFFFu) : svmax;
        }
        float wmax = smax + (float)(svmax >> 10);
        wmax = fmaxf(wmax, lane_xor16(wmax));
        wmax = max_xor32(wmax);
        const bool need = wmax > m_ref + kMqTau;
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float f = need ? __builtin_amdgcn_exp2f(m_ref - wmax) : 1.f;
            if (need) m_ref = wmax;
            lsum *= f;
            zsum *= f;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float fr = __shfl(f, 4 * g + i, 64);
#pragma unroll
                for (int c = 0; c < NCB; c++) acc[c][i] *= fr;
            }
        }
        // p is carried as p * 2^27 (lsum, zsum too; undone in finish): P = p * 2^27 * s_V is then
        // one fma, and P < 2^14 by the reference rule
        float P[8];
        const float m27 = m_ref - 27.f;
#pragma unroll
        for (int t = 0; t < 8; t++) {
            const uint32_t d1 = b.sc[2 * t + 1];
            // unread slots hold unspecified bytes (their scales may be inf / NaN): select, never
            // multiply them by zero
            const float p = ok[t] ? __builtin_amdgcn_exp2f(st[t] - m27) : 0.f;
            lsum += p;
            zsum = ok[t] ? fmaf(p, fmaf(lo_half(d1), (float)MID, hi_half(d1)), zsum) : zsum;
            P[t] = ok[t] ? fmaf(lo_half(d1), p, 0.f) : 0.f;
        }
        u32x4 phi, plo;
        split_hilo_rtz(P, phi, plo);
#pragma unroll
        for (int c = 0; c < NCB; c++) {
            const u32x4 bv = IS8 ? centre<MID>(spread_int8(b.v[c][0], b.v[c][1]))
                                 : spread_centre_int4<MID>(b.v[c][0], k6400);
            acc[c] = mfma16x32(phi, bv, acc[c]);
            acc[c] = mfma16x32(plo, bv, acc[c]);
        }
    }

    // INT8 steps [s0, s1): a few per task (the protection slots), one buffer.
    __device__ void run8(int s0, int s1)
    {
        for (int s = s0; s < s1; s++) {
            Buf<true> b;
            load8_step(b, s);
            compute<true, false>(b, s);
        }
    }

    // INT4 step s covers positions [16 (p0 + 2 (s - n8)), +32): all readable and not after the
    // tile's first row (the smallest row position)?
    __device__ __forceinline__ bool interior(int s) const
    {
        const int base = kPageSize * (p0 + 2 * (s - a.n8));
        return base >= lo4 && base + kMqStepSlots <= hi4 && base + kMqStepSlots - 1 <= first_pos;
    }

    __device__ __forceinline__ void step4(const Buf<false>& b, int s)
    {
        if (interior(s))
            compute<false, true>(b, s);
        else
            compute<false, false>(b, s);
    }

    // INT4 steps [s0, s1) with the next step's loads in flight during each step; a load past the
    // end repeats the last step's addresses and is not used.
    __device__ void run4(int s0, int s1)
    {
        if (s0 >= s1) return;
        Buf<false> b0, b1;
        load4(b0, s0);
        for (int s = s0; s < s1; s += 2) {
            load4(b1, s + 1 < s1 ? s + 1 : s);
            step4(b0, s);
            if (s + 1 >= s1) break;
            load4(b0, s + 2 < s1 ? s + 2 : s + 1);
            step4(b1, s + 1);
        }
    }

    __device__ void finish(int task)
    {
        lsum += lane_xor16(lsum);
        lsum = add_xor32(lsum);
        zsum += lane_xor16(zsum);
        zsum = add_xor32(zsum);
        if (g == 0) {
            float* ml = a.part_ml + ((int64_t)task * kMqRows + n) * 2;
            ml[0] = m_ref;
            ml[1] = lsum * (1.f / kPScale);
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int row = 4 * g + i;
            const float z = __shfl(zsum, row, 64);
            float* o = a.part_o + ((int64_t)task * kMqRows + row) * D + n;
#pragma unroll
            for (int c = 0; c < NCB; c++) o[16 * c] = (acc[c][i] + z) * (1.f / kPScale);
        }
    }
};

template <int D, int G, int FMT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void mq_split_kernel(MqArgs a)
{
    const int wave = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (wave >= a.tasks) return;
    const int lane = (int)(threadIdx.x & 63);
    const int lo = mq_find_entry<false>(a, wave, lane);
    MqEntry e;
    e.seq = mq_uniform(&a.entries[lo].seq);
    e.len = mq_uniform(&a.entries[lo].len);
    e.nq = mq_uniform(&a.entries[lo].nq);
    e.qrow0 = mq_uniform(&a.entries[lo].qrow0);
    e.task0 = mq_uniform(&a.entries[lo].task0);
    e.steps = mq_uniform(&a.entries[lo].steps);
    e.nch = mq_uniform(&a.entries[lo].nch);
    const int nrt = (e.nq * G + kMqRows - 1) / kMqRows;
    int local = wave - e.task0;
    const int head = local / (e.nch * nrt);
    local -= head * e.nch * nrt;
    const int chunk = local / nrt;
    const int rt = local - chunk * nrt;

    MqWave<D, G, FMT> W(a, lane);
    W.seq = e.seq;
    W.L = e.len;
    W.head = head;
    W.btrow = a.bt + (int64_t)e.seq * a.max_pps;
    W.hbase = a.pool + (int64_t)head * a.page_block;
    W.pstride = (uint32_t)(a.hkv * a.page_block);
    if (FMT == FMT_INT4_PROT) {
        W.lo4 = a.sinks;
        W.hi4 = e.len - a.recent;
        W.p0 = a.sinks / kPageSize;
        W.p1 = W.hi4 > W.lo4 ? (W.hi4 - 1) / kPageSize + 1 : W.p0;
        W.ring_base = e.len - a.recent > a.sinks ? e.len - a.recent : a.sinks;
        W.ring_mod = a.recent > 0 ? W.ring_base % a.recent : 0;
        W.t8 = a.int8_pool + ((int64_t)e.seq * a.hkv + head) * a.int8_tiles * a.int8_tile;
    } else {
        W.lo4 = W.hi4 = W.p0 = W.ring_base = W.ring_mod = 0;
        W.p1 = (e.len + kPageSize - 1) / kPageSize;
        W.t8 = nullptr;
    }
    W.prologue(e, rt);
    const int s0 = chunk * a.spc;
    const int s1 = s0 + a.spc < e.steps ? s0 + a.spc : e.steps;
    const int n8 = FMT == FMT_INT8 ? e.steps : a.n8;
    W.run8(s0, s1 < n8 ? s1 : n8);
    if (FMT == FMT_INT4_PROT) W.run4(s0 > n8 ? s0 : n8, s1);
    W.finish(wave);
}

template <int D, int G, bool ROT>
__global__ __launch_bounds__(256) void mq_merge_kernel(MqArgs a)
{
    constexpr int DPM = D / 64;
    constexpr int QT = kMqRows / G;
    const int wave = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (wave >= a.groups * kMqRows) return;
    const int lane = (int)(threadIdx.x & 63);
    const int grp = wave / kMqRows, r = wave % kMqRows;
    const int lo = mq_find_entry<true>(a, grp, lane);
    const int nq = mq_uniform(&a.entries[lo].nq);
    const int qrow0 = mq_uniform(&a.entries[lo].qrow0);
    const int task0 = mq_uniform(&a.entries[lo].task0);
    const int grp0 = mq_uniform(&a.entries[lo].grp0);
    const int nch = mq_uniform(&a.entries[lo].nch);
    const int nrt = (nq * G + kMqRows - 1) / kMqRows;
    const int local = grp - grp0;
    const int head = local / nrt, rt = local - head * nrt;
    const int jq = rt * QT + r / G, gi = r % G;
    if (jq >= nq) return;
    // chunk c's partial of this row sits in task slot T(c); lane c of a round of 64 holds its
    // (m, l), one vector load per round
    const int64_t T0 = (int64_t)task0 + (int64_t)head * nch * nrt + rt; // T(c) = T0 + c nrt
    float M = -__builtin_inff();
    for (int c0 = 0; c0 < nch; c0 += 64) {
        const int c = c0 + lane;
        M = fmaxf(M, c < nch ? a.part_ml[((T0 + (int64_t)c * nrt) * kMqRows + r) * 2] : -__builtin_inff());
    }
    M = wave_max_u(M);
    float l = 0.f, o[DPM];
#pragma unroll
    for (int k = 0; k < DPM; k++) o[k] = 0.f;
    for (int c0 = 0; c0 < nch; c0 += 64) {
        const int c = c0 + lane;
        const float* mlc = a.part_ml + ((T0 + (int64_t)c * nrt) * kMqRows + r) * 2;
        const float m = c < nch ? mlc[0] : -__builtin_inff();
        const float lc = c < nch ? mlc[1] : 0.f;
        const float wgt = exp2f(m - M);
        l += wave_sum_u(wgt * lc);
        // the outputs in chunk order, each weight read from its lane; the loads of 8 chunks are
        // issued before the first of them is used (8 keeps 8 waves per SIMD)
        const int cn = __builtin_amdgcn_readfirstlane(nch - c0 < 64 ? nch - c0 : 64);
        // chunk c's outputs: a wave-uniform base plus the lane's offset
        const float* obase = a.part_o + (T0 * kMqRows + r) * D;
        const int64_t ostride = (int64_t)nrt * kMqRows * D;
        for (int cb = 0; cb < cn; cb += 8) {
            float pv[8][DPM];
#pragma unroll
            for (int k = 0; k < 8; k++) {
                const float* po = obase + (int64_t)(c0 + cb + k) * ostride;
#pragma unroll
                for (int q = 0; q < DPM; q++) pv[k][q] = cb + k < cn ? po[lane * DPM + q] : 0.f;
            }
#pragma unroll
            for (int k = 0; k < 8; k++) {
                if (cb + k < cn) {
                    const float w = as_float((uint32_t)__builtin_amdgcn_readlane((int)as_uint(wgt), cb + k));
#pragma unroll
                    for (int q = 0; q < DPM; q++) o[q] = fmaf(w, pv[k][q], o[q]);
                }
            }
        }
    }
    const float inv = 1.f / l;
#pragma unroll
    for (int k = 0; k < DPM; k++) o[k] *= inv;
    if (ROT) {
        // o H_bd (Sylvester H is symmetric, so this is also o H_bd^T), stages h = 1, 2, ..., b/2
        if (DPM == 2 && a.block > 1) {
            const float u = o[0], w = o[DPM - 1];
            o[0] = u + w;
            o[DPM - 1] = u - w;
        }
        static_for<0, 6>([&](auto S) {
            constexpr int M = 1 << S;
            if (M * DPM < a.block) {
                const float sgn = (lane & M) ? -1.f : 1.f;
#pragma unroll
                for (int k = 0; k < DPM; k++) o[k] = butterfly_xor<M>(o[k], sgn);
            }
        });
#pragma unroll
        for (int k = 0; k < DPM; k++) o[k] *= a.cb;
    }
    float* out = a.out + ((int64_t)(qrow0 + jq) * a.hq + head * G + gi) * D + lane * DPM;
#pragma unroll
    for (int k = 0; k < DPM; k++) out[k] = o[k];
}

template <int D, int G, int FMT>
hipError_t split_dispatch(const MqArgs& a, hipStream_t stream, const KernelTimer& tm)
{
    const int blocks = (a.tasks + 3) / 4;
    return launch_kernel(mq_split_kernel<D, G, FMT>, dim3(blocks), dim3(256), stream, tm, a);
}

template <int D, int G>
hipError_t merge_dispatch(const MqArgs& a, hipStream_t stream, const KernelTimer& tm)
{
    const int64_t waves = (int64_t)a.groups * kMqRows;
    const int blocks = (int)((waves + 3) / 4);
    return launch_kernel(mq_merge_kernel<D, G, true>, dim3(blocks), dim3(256), stream, tm, a);
}

template <int D, int G, int FMT>
hipError_t split_residency(int* bpc)
{
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(bpc, mq_split_kernel<D, G, FMT>, 256, 0);
}

} // namespace

template <int FMT>
hipError_t split_by_shape(int d, int g, const MqArgs& a, hipStream_t st, const KernelTimer& tm)
{
    if (d == 128 && g == 4) return split_dispatch<128, 4, FMT>(a, st, tm);
    if (d == 128 && g == 2) return split_dispatch<128, 2, FMT>(a, st, tm);
    if (d == 128 && g == 1) return split_dispatch<128, 1, FMT>(a, st, tm);
    if (d == 64 && g == 4) return split_dispatch<64, 4, FMT>(a, st, tm);
    if (d == 64 && g == 2) return split_dispatch<64, 2, FMT>(a, st, tm);
    if (d == 64 && g == 1) return split_dispatch<64, 1, FMT>(a, st, tm);
    return hipErrorInvalidValue;
}

template <int FMT>
hipError_t residency_by_shape(int d, int g, int* bpc)
{
    if (d == 128 && g == 4) return split_residency<128, 4, FMT>(bpc);
    if (d == 128 && g == 2) return split_residency<128, 2, FMT>(bpc);
    if (d == 128 && g == 1) return split_residency<128, 1, FMT>(bpc);
    if (d == 64 && g == 4) return split_residency<64, 4, FMT>(bpc);
    if (d == 64 && g == 2) return split_residency<64, 2, FMT>(bpc);
    if (d == 64 && g == 1) return split_residency<64, 1, FMT>(bpc);
    return hipErrorInvalidValue;
}

hipError_t launch_mq_split(int d, int g, int format, const MqArgs& a, hipStream_t stream, const KernelTimer& tm)
{
    if (a.tasks <= 0) return hipSuccess;
    if (format == FMT_INT4_PROT) return split_by_shape<FMT_INT4_PROT>(d, g, a, stream, tm);
    if (format == FMT_INT8) return split_by_shape<FMT_INT8>(d, g, a, stream, tm);
    return hipErrorInvalidValue;
}

hipError_t launch_mq_merge(int d, int g, const MqArgs& a, hipStream_t stream, const KernelTimer& tm)
{
    if (a.groups <= 0) return hipSuccess;
    if (d == 128 && g == 4) return merge_dispatch<128, 4>(a, stream, tm);
    if (d == 128 && g == 2) return merge_dispatch<128, 2>(a, stream, tm);
    if (d == 128 && g == 1) return merge_dispatch<128, 1>(a, stream, tm);
    if (d == 64 && g == 4) return merge_dispatch<64, 4>(a, stream, tm);
    if (d == 64 && g == 2) return merge_dispatch<64, 2>(a, stream, tm);
    if (d == 64 && g == 1) return merge_dispatch<64, 1>(a, stream, tm);
    return hipErrorInvalidValue;
}

hipError_t mq_split_residency(int d, int g, int format, int* blocks_per_cu)
{
    *blocks_per_cu = 0;
    if (format == FMT_INT4_PROT) return residency_by_shape<FMT_INT4_PROT>(d, g, blocks_per_cu);
    if (format == FMT_INT8) return residency_by_shape<FMT_INT8>(d, g, blocks_per_cu);
    return hipSuccess;
}

} // namespace kv4
