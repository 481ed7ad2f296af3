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
#include "kv4_common.h"

namespace kv4 {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

constexpr float kMqTau = 1.f;
constexpr float kPScale = 134217728.f; // 2^27
// INT4 steps are staged in LDS: each step's two page blocks are copied by global_load_lds_dwordx4
// (no VGPRs while in flight) into a ring of kMqStages stage buffers per wave, kMqStages - 1 steps
// ahead of the step being computed.
constexpr int kMqStages = 3;

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding: vmcnt bits 3:0 and 15:14)
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x0F70);
}

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

// Eight INT4 value codes in the spread order, centred.  A nibble in bits 0-3 of a half,
// or'ed with 0x6400, is the fp16 value 1024 + code, less 1024 + MID in one packed fp16
// subtraction; a nibble left in bits 4-7 gives 1024 + 16 code, and (1024 + 16 code) / 16 - 64 - MID
// is one packed fp16 fma.  Both are exact (integers below 2^11), so one shift serves four
// codes.  k6400 holds 0x64006400 in a vector register, so that mask-and-or is one v_and_or_b32
// (two literals cannot share it).
template <int MID>
__device__ __forceinline__ u32x4 spread_centre_int4(uint32_t w, uint32_t k6400)
{
    const half2_t off = {(_Float16)(-(1024 + MID)), (_Float16)(-(1024 + MID))};
    const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const half2_t off16 = {(_Float16)(-(64 + MID)), (_Float16)(-(64 + MID))};
    const uint32_t w8 = w >> 8;
    const half2_t e0 = __builtin_bit_cast(half2_t, (w & 0x000F000Fu) | k6400);
    const half2_t o0 = __builtin_bit_cast(half2_t, (w & 0x00F000F0u) | k6400);
    const half2_t e1 = __builtin_bit_cast(half2_t, (w8 & 0x000F000Fu) | k6400);
    const half2_t o1 = __builtin_bit_cast(half2_t, (w8 & 0x00F000F0u) | k6400);
    return (u32x4){__builtin_bit_cast(uint32_t, e0 + off),
                   __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(o0, sixteenth, off16)),
                   __builtin_bit_cast(uint32_t, e1 + off),
                   __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(o1, sixteenth, off16))};
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
// x - hi is exact in fp32 and its own fp16 truncation leaves about 2^-20 of x.  m1 is -1 held in a
// vector register, so that each residual stays one v_fma_mix_f32 reading hi's fp16 half (with a
// literal -1 the compiler turns the fma into a conversion and a subtraction).
__device__ __forceinline__ void split_hilo_rtz(const float (&x)[8], u32x4& hi, u32x4& lo, float m1)
{
#pragma unroll
    for (int s = 0; s < 4; s++) {
        const half2_t h = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(x[s], x[s + 4]));
        const float r0 = fmaf((float)h[0], m1, x[s]), r1 = fmaf((float)h[1], m1, x[s + 4]);
        hi[s] = __builtin_bit_cast(uint32_t, h);
        lo[s] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(r0, r1));
    }
}

__device__ __forceinline__ float lo_half(uint32_t d) { return (float)__builtin_bit_cast(half2_t, d)[0]; }
__device__ __forceinline__ float hi_half(uint32_t d) { return (float)__builtin_bit_cast(half2_t, d)[1]; }

__device__ __forceinline__ u32x4 ld16(const uint8_t* p) { return *(const u32x4*)p; }
__device__ __forceinline__ u32x2 ld8(const uint8_t* p) { return *(const u32x2*)p; }

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
    static constexpr int CPB = (IB + 1023) / 1024; // 1 KB copy instructions per page block
    static constexpr int SB = 1024 * CPB;          // LDS bytes of a staged page block (padded)
    static constexpr int STAGE = 2 * SB;           // LDS bytes of one staged INT4 step (two blocks)
    static constexpr int RING = kMqStages * STAGE; // a wave's own stage ring
    // Workgroup-shared INT4 steps (the four waves take four row tiles of one chunk): one stage ring
    // for the workgroup, and each wave spreads a quarter of a step's operands into LDS for all four.
    static constexpr int NOPS = NCB;               // shared operands of a step: the value blocks
    static constexpr int QOPS = NOPS / 4;          // operands a wave spreads
    static constexpr int NCOPY = 2 * CPB;          // copy instructions of a step
    static constexpr int PERW = (NCOPY + 3) / 4;   // copies a wave issues per step
    static constexpr int SH_STAGES = 6;            // shared ring: steps k .. k + 5 of a pair iteration
    static constexpr int SH_RING = SH_STAGES * STAGE;
    static constexpr int SPR = NOPS * 64 * 16;     // one step's spread operands
    static constexpr int SH_AREAS = 4;             // operand areas: steps k .. k + 3
    static constexpr int SH_LDS = SH_RING + SH_AREAS * SPR;
    static_assert(NOPS % 4 == 0, "the operands split evenly over four waves");

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
    float m_ref = -__builtin_inff(), lsum = 0.f, zsum = 0.f, Ar = 0.f, Bu = 0.f;
    __attribute__((address_space(3))) uint8_t* ring; // kMqStages INT4 stage buffers (the wave's or the workgroup's)
    __attribute__((address_space(3))) uint8_t* spr;  // shared steps: the spread operands [NOPS][64 lanes][16 B]
    int wv = 0;          // shared steps: wave index in the workgroup
    uint32_t k6400;      // 0x64006400 in a vector register (identity DPP move: not a literal)
    float m1;            // -1 in a vector register (the same)
    u32x4 qhi[KS], qlo[KS];
    float4_t acc[NCB];

    __device__ MqWave(const MqArgs& args, int l)
        : a(args), lane(l), n(l & 15), g(l >> 4),
          k6400((uint32_t)__builtin_amdgcn_update_dpp(0, 0x64006400, 0xE4, 0xF, 0xF, false)),
          m1(as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)0xBF800000u, 0xE4, 0xF, 0xF, false)))
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
        // score (log2 units) = Ar * (s_K * acc + Bu * z_K), acc = 2^-24 sum(q 2^(14-E) * code):
        // a step keeps the bracket (st) and applies Ar once per position, in the exponent's fma
        Ar = __builtin_ldexpf(a.scale_log2, 24 + E - 14);
        Bu = __builtin_ldexpf(sum, 14 - 24 - E);
#pragma unroll
        for (int c = 0; c < NCB; c++) acc[c] = (float4_t){0.f, 0.f, 0.f, 0.f};
    }

    // Page ids of INT4 step s (s >= n8): pages p0 + 2 (s - n8) and the next (clamped to the last).
    __device__ __forceinline__ void step_pages(int s, uint32_t& pa, uint32_t& pb) const
    {
        // wave-uniform by construction; readfirstlane lets the compiler see it, so that the block
        // table is read with scalar loads (a vector load here would make the loop wait on vmcnt)
        const int pi = __builtin_amdgcn_readfirstlane(p0 + 2 * (s - a.n8));
        const int pj = __builtin_amdgcn_readfirstlane(pi + 1 < p1 ? pi + 1 : pi);
        pa = (uint32_t)mq_uniform(btrow + pi);
        pb = (uint32_t)mq_uniform(btrow + pj);
    }

    // Copies the two page blocks of a step into stage buffer st: CPB instructions per block, each
    // moving 16 bytes per lane with every lane active, so that a step is always 2 * CPB
    // instructions.  In the last one, the lanes past the block's end re-read its last 128 bytes
    // into the padding of the staged block (read inside the block, never used).
    __device__ __forceinline__ void stage_copy(uint32_t pa, uint32_t pb, int st) const
    {
        __attribute__((address_space(3))) uint8_t* dst = ring + st * STAGE;
#pragma unroll
        for (int x = 0; x < 2; x++) {
            const uint8_t* src = hbase + (uint64_t)(x ? pb : pa) * pstride;
#pragma unroll
            for (int i = 0; i < CPB; i++) {
                int off = 1024 * i + 16 * lane;
                if (1024 * (i + 1) > IB) off = off < IB ? off : IB - 128 + 16 * (lane & 7);
                __builtin_amdgcn_global_load_lds((const void*)(src + off),
                                                 (__attribute__((address_space(3))) void*)(dst + x * SB + 1024 * i), 16,
                                                 0, 0);
            }
        }
    }

    // The operands of an INT4 step from stage buffer st (page A block, then page B block).
    __device__ __forceinline__ void stage_read(Buf<false>& b, int st) const
    {
        const __attribute__((address_space(3))) uint8_t* base = ring + st * STAGE;
        const int kslot = 8 * ((n >> 2) & 1) + (n & 3);
        const __attribute__((address_space(3))) uint8_t* kp = base + (n < 8 ? 0 : SB) + kslot * 16;
        const __attribute__((address_space(3))) uint8_t* vp = base + (g < 2 ? 0 : SB);
        if constexpr (D == 128) {
            kp += 256 * g;
#pragma unroll
            for (int t = 0; t < 2; t++) {
                const u32x4 w = *(const __attribute__((address_space(3))) u32x4*)(kp + 64 * t);
#pragma unroll
                for (int j = 0; j < 4; j++) b.k[t][j] = w[j];
            }
        } else {
            kp += 256 * (g >> 1) + 8 * (g & 1);
#pragma unroll
            for (int t = 0; t < 2; t++) {
                const u32x2 w = *(const __attribute__((address_space(3))) u32x2*)(kp + 64 * t);
                b.k[t][0] = w[0];
                b.k[t][1] = w[1];
            }
        }
#pragma unroll
        for (int c = 0; c < NCB; c++)
            b.v[c][0] = *(const __attribute__((address_space(3))) uint32_t*)(vp + 8 * D + (16 * c + n) * 8 + 4 * (g & 1));
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const u32x4 w = *(const __attribute__((address_space(3))) u32x4*)(vp + 16 * D + 64 * (g & 1) + 16 * j);
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
        // positions (positive fp16 patterns order like their values), so Ar st + e_lane bounds
        // Ar st + log2 s_V + 1 for each of them (Ar > 0: the largest st gives the largest score).
        float st[8];
        bool ok[8];
        float smax = -__builtin_inff();
        uint32_t svmax = 0;
#pragma unroll
        for (int t = 0; t < 8; t++) {
            const float r = t < 4 ? sa[t] : sb[t - 4];
            const uint32_t d0 = b.sc[2 * t], d1 = b.sc[2 * t + 1];
            st[t] = fmaf(lo_half(d0), r, fmaf(hi_half(d0), Bu, 0.f));
            ok[t] = FULL || pos[t] <= pos_r;
            smax = ok[t] ? fmaxf(smax, st[t]) : smax;
            if (!FULL) svmax = ok[t] ? max(svmax, d1 & 0xFFFFu) : svmax;
        }
        if (FULL) {
            // every slot read: the largest s_V pattern by 16-bit maxima of the low halves
            u16x2 mv = as_u16x2(b.sc[1]);
#pragma unroll
            for (int t = 1; t < 8; t++) mv = __builtin_elementwise_max(mv, as_u16x2(b.sc[2 * t + 1]));
            svmax = mv.x;
        }
        float wmax = fmaf(smax, Ar, (float)(svmax >> 10));
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
            const float p = ok[t] ? __builtin_amdgcn_exp2f(fmaf(st[t], Ar, -m27)) : 0.f;
            lsum += p;
            zsum = ok[t] ? fmaf(p, fmaf(lo_half(d1), (float)MID, hi_half(d1)), zsum) : zsum;
            P[t] = ok[t] ? fmaf(lo_half(d1), p, 0.f) : 0.f;
        }
        u32x4 phi, plo;
        split_hilo_rtz(P, phi, plo, m1);
#pragma unroll
        for (int c = 0; c < NCB; c++) {
            const u32x4 bv = IS8 ? centre<MID>(spread_int8(b.v[c][0], b.v[c][1]))
                                 : spread_centre_int4<MID>(b.v[c][0], k6400);
            acc[c] = mfma16x32(phi, bv, acc[c]);
            acc[c] = mfma16x32(plo, bv, acc[c]);
        }
    }

    // S^T of a step for the two tiles of 16 positions
    template <bool IS8, typename KOp>
    __device__ __forceinline__ void qk(KOp kop, float4_t& sa, float4_t& sb) const
    {
        sa = (float4_t){0.f, 0.f, 0.f, 0.f};
        sb = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KS; j++) {
            const u32x4 ka = kop(0, j);
            const u32x4 kb = kop(1, j);
            const u32x4 qh = IS8 ? odd_x16(qhi[j]) : qhi[j];
            const u32x4 ql = IS8 ? odd_x16(qlo[j]) : qlo[j];
            sa = mfma16x32(ka, qh, sa);
            sb = mfma16x32(kb, qh, sb);
            sa = mfma16x32(ka, ql, sa);
            sb = mfma16x32(kb, ql, sb);
        }
    }

    // The rest of a step, from its S^T: scores, online softmax, O += P' V (the arithmetic of
    // compute() after its products, for operands that come from the workgroup's shared area).
    template <bool IS8, bool FULL, typename VOp>
    __device__ __forceinline__ void softmax_pv(const float4_t& sa, const float4_t& sb, VOp vop,
                                               const uint32_t (&sc)[16], int s)
    {
        constexpr int MID = IS8 ? 128 : 8;
        int pos[8];
        if (!FULL) positions<IS8>(s, pos);
        // fp16 scales enter the fp32 arithmetic as fma operands (v_fma_mix_f32: no conversions).
        // The reference bound uses one exponent per lane: the largest s_V of the lane's readable
        // positions (positive fp16 patterns order like their values), so Ar st + e_lane bounds
        // Ar st + log2 s_V + 1 for each of them (Ar > 0: the largest st gives the largest score).
        float st[8];
        bool ok[8];
        float smax = -__builtin_inff();
        uint32_t svmax = 0;
#pragma unroll
        for (int t = 0; t < 8; t++) {
            const float r = t < 4 ? sa[t] : sb[t - 4];
            const uint32_t d0 = sc[2 * t], d1 = sc[2 * t + 1];
            st[t] = fmaf(lo_half(d0), r, fmaf(hi_half(d0), Bu, 0.f));
            ok[t] = FULL || pos[t] <= pos_r;
            smax = ok[t] ? fmaxf(smax, st[t]) : smax;
            if (!FULL) svmax = ok[t] ? max(svmax, d1 & 0xFFFFu) : svmax;
        }
        if (FULL) {
            // every slot read: the largest s_V pattern by 16-bit maxima of the low halves
            u16x2 mv = as_u16x2(sc[1]);
#pragma unroll
            for (int t = 1; t < 8; t++) mv = __builtin_elementwise_max(mv, as_u16x2(sc[2 * t + 1]));
            svmax = mv.x;
        }
        float wmax = fmaf(smax, Ar, (float)(svmax >> 10));
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
            const uint32_t d1 = sc[2 * t + 1];
            // unread slots hold unspecified bytes (their scales may be inf / NaN): select, never
            // multiply them by zero
            const float p = ok[t] ? __builtin_amdgcn_exp2f(fmaf(st[t], Ar, -m27)) : 0.f;
            lsum += p;
            zsum = ok[t] ? fmaf(p, fmaf(lo_half(d1), (float)MID, hi_half(d1)), zsum) : zsum;
            P[t] = ok[t] ? fmaf(lo_half(d1), p, 0.f) : 0.f;
        }
        u32x4 phi, plo;
        split_hilo_rtz(P, phi, plo, m1);
#pragma unroll
        for (int c = 0; c < NCB; c++) {
            const u32x4 bv = vop(c);
            acc[c] = mfma16x32(phi, bv, acc[c]);
            acc[c] = mfma16x32(plo, bv, acc[c]);
        }
    }

    // INT8 steps [s0, s1): a few per task (the protection slots), one buffer.
    // (one buffer: a second one would not fit the register budget of 2 waves per SIMD)
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

    // INT4 steps [s0, s1) through the LDS ring: the copies of the next kMqStages - 1 steps are in
    // flight while a step is computed.  Every iteration issues exactly one step's copies (past the
    // end they repeat the last step and are never read), so the wait for the oldest one is a fixed
    // count.  A stage is refilled only in the iteration after its operands were read (and used).
    __device__ void run4(int s0, int s1)
    {
        if (s0 >= s1) return;
        constexpr int PER = 2 * CPB; // copy instructions per step
        uint32_t pa, pb;
#pragma unroll
        for (int j = 0; j < kMqStages - 1; j++) {
            step_pages(min(s0 + j, s1 - 1), pa, pb);
            stage_copy(pa, pb, j);
        }
        step_pages(min(s0 + kMqStages - 1, s1 - 1), pa, pb);
        int st = 0;
        for (int s = s0; s < s1; s++) {
            __builtin_amdgcn_sched_barrier(0);
            stage_copy(pa, pb, st == 0 ? kMqStages - 1 : st - 1);
            step_pages(min(s + kMqStages, s1 - 1), pa, pb);
            wait_vmcnt<(kMqStages - 1) * PER>();
            __builtin_amdgcn_sched_barrier(0);
            Buf<false> b;
            stage_read(b, st);
            step4(b, s);
            st = st + 1 == kMqStages ? 0 : st + 1;
        }
        wait_vmcnt<0>();
    }

    // ---- INT4 steps shared by the four waves of a workgroup (row tiles 4k .. 4k + 3 of one
    // (entry, kv head, chunk)): the same pages, the same steps [s0, s1), the same barriers. ----

    // The copies of a step into the workgroup's stage st: wave wv issues copies wv and wv + 4 of the
    // step's NCOPY (the last one repeated where the count runs out: the same bytes to the same
    // place), so every wave issues PERW copies per step.
    __device__ __forceinline__ void stage_copy_sh(uint32_t pa, uint32_t pb, int st) const
    {
        __attribute__((address_space(3))) uint8_t* dst = ring + st * STAGE;
#pragma unroll
        for (int m = 0; m < PERW; m++) {
            const int k = min(wv + 4 * m, NCOPY - 1);
            const int x = k / CPB, i = k - x * CPB;
            const uint8_t* src = hbase + (uint64_t)(x ? pb : pa) * pstride;
            int off = 1024 * i + 16 * lane;
            if (1024 * (i + 1) > IB) off = off < IB ? off : IB - 128 + 16 * (lane & 7);
            __builtin_amdgcn_global_load_lds((const void*)(src + off),
                                             (__attribute__((address_space(3))) void*)(dst + x * SB + 1024 * i), 16, 0,
                                             0);
        }
    }

    // This wave's quarter of the step's value operands (column blocks QOPS wv ..), spread from
    // stage st into operand area buf (each lane's code words sit where stage_read finds them).
    // The key operands stay per wave: their spread costs 5 VALU per 8 codes against 11 for the
    // centred values, for the same LDS bytes.
    __device__ __forceinline__ void spread_quarter(int st, int buf) const
    {
        const __attribute__((address_space(3))) uint8_t* vp =
            ring + st * STAGE + (g < 2 ? 0 : SB) + 8 * D + (16 * QOPS * wv + n) * 8 + 4 * (g & 1);
        __attribute__((address_space(3))) u32x4* dst =
            (__attribute__((address_space(3))) u32x4*)(spr + buf * SPR) + (QOPS * wv) * 64 + lane;
        uint32_t w[QOPS];
#pragma unroll
        for (int q = 0; q < QOPS; q++) w[q] = *(const __attribute__((address_space(3))) uint32_t*)(vp + 128 * q);
#pragma unroll
        for (int q = 0; q < QOPS; q++) dst[q * 64] = spread_centre_int4<8>(w[q], k6400);
    }

    // S^T of the step in stage st (its key codes, spread by this wave)
    __device__ __forceinline__ void qk_sh(int st, float4_t& sa, float4_t& sb) const
    {
        uint32_t kw[2][KS];
        const int kslot = 8 * ((n >> 2) & 1) + (n & 3);
        const __attribute__((address_space(3))) uint8_t* kp = ring + st * STAGE + (n < 8 ? 0 : SB) + kslot * 16;
        if constexpr (D == 128) {
            kp += 256 * g;
#pragma unroll
            for (int t = 0; t < 2; t++) {
                const u32x4 w = *(const __attribute__((address_space(3))) u32x4*)(kp + 64 * t);
#pragma unroll
                for (int j = 0; j < 4; j++) kw[t][j] = w[j];
            }
        } else {
            kp += 256 * (g >> 1) + 8 * (g & 1);
#pragma unroll
            for (int t = 0; t < 2; t++) {
                const u32x2 w = *(const __attribute__((address_space(3))) u32x2*)(kp + 64 * t);
                kw[t][0] = w[0];
                kw[t][1] = w[1];
            }
        }
        qk<false>([&](int t, int j) { return spread_int4_x16(kw[t][j]); }, sa, sb);
    }

    // Step s: S^T from its key codes in stage st, then the softmax and P V with the scales from
    // stage st and the value operands from area buf.
    __device__ __forceinline__ void compute_sh(int st, int buf, int s)
    {
        float4_t sa, sb;
        qk_sh(st, sa, sb);
        const __attribute__((address_space(3))) uint8_t* vp = ring + st * STAGE + (g < 2 ? 0 : SB);
        uint32_t sc[16];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const u32x4 w = *(const __attribute__((address_space(3))) u32x4*)(vp + 16 * D + 64 * (g & 1) + 16 * j);
#pragma unroll
            for (int i = 0; i < 4; i++) sc[4 * j + i] = w[i];
        }
        // the value operands are read here, ahead of the products and branches that precede
        // their use, so that their LDS latency is covered
        const __attribute__((address_space(3))) u32x4* op =
            (const __attribute__((address_space(3))) u32x4*)(spr + buf * SPR) + lane;
        u32x4 vv[NCB];
#pragma unroll
        for (int c = 0; c < NCB; c++) vv[c] = op[c * 64];
        auto vop = [&](int c) { return vv[c]; };
        if (interior(s))
            softmax_pv<false, true>(sa, sb, vop, sc, s);
        else
            softmax_pv<false, false>(sa, sb, vop, sc, s);
    }

    // s_waitcnt vmcnt(N) lgkmcnt(0), then the workgroup barrier, as one statement the compiler
    // does not move memory accesses across (a fence would also wait for the copies in flight).
    template <int N>
    __device__ __forceinline__ static void barrier_vm()
    {
        static_assert(N == 0 || N == 2 || N == 4, "the counts the step loop uses");
        if constexpr (N == 0)
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        else if constexpr (N == 2)
            asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }

    // Steps in pairs, one barrier per pair, with the spread one pair ahead of the products (the
    // four waves then meet every other step, so a wave that runs late on one step can catch up on
    // the next).  Before the iteration for steps k, k + 1 (offsets from s0) the ring holds steps
    // k .. k + 3 (k + 2, k + 3 possibly in flight, the only copies in flight) and operand areas
    // k % 4, (k + 1) % 4 hold steps k, k + 1 spread.  Iteration: wait for this wave's copies;
    // barrier (every copy of k + 2, k + 3 has landed, both areas are complete, and every wave is
    // done with steps k - 2, k - 1: their stages and areas are free); copy steps k + 4, k + 5 into
    // the freed stages; spread this wave's quarter of steps k + 2, k + 3; compute steps k, k + 1.
    // Past s1 - 1 the copies repeat the last step and their spreads are never read.  [s0, s1) is
    // the same for the four waves, so every wave passes the same barriers.
    __device__ void run4_sh(int s0, int s1)
    {
        if (s0 >= s1) return;
        const int n = s1 - s0;
        uint32_t pa, pb, qa, qb;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            step_pages(min(s0 + j, s1 - 1), pa, pb);
            stage_copy_sh(pa, pb, j);
        }
        step_pages(min(s0 + 4, s1 - 1), pa, pb);
        step_pages(min(s0 + 5, s1 - 1), qa, qb);
        __builtin_amdgcn_sched_barrier(0);
        barrier_vm<2 * PERW>();
        __builtin_amdgcn_sched_barrier(0);
        spread_quarter(0, 0);
        spread_quarter(1, 1);
        int sk = 0; // k % SH_STAGES
        for (int k = 0; k < n; k += 2) {
            __builtin_amdgcn_sched_barrier(0);
            barrier_vm<0>();
            __builtin_amdgcn_sched_barrier(0);
            const int s4 = sk + 4 < SH_STAGES ? sk + 4 : sk + 4 - SH_STAGES;
            const int s2 = sk + 2 < SH_STAGES ? sk + 2 : sk + 2 - SH_STAGES;
            stage_copy_sh(pa, pb, s4);
            stage_copy_sh(qa, qb, s4 + 1);
            step_pages(min(s0 + k + 6, s1 - 1), pa, pb);
            step_pages(min(s0 + k + 7, s1 - 1), qa, qb);
            spread_quarter(s2, (k + 2) & 3);
            spread_quarter(s2 + 1, (k + 3) & 3);
            compute_sh(sk, k & 3, s0 + k);
            if (k + 1 < n) compute_sh(sk + 1, (k + 1) & 3, s0 + k + 1);
            sk = s2;
        }
        __builtin_amdgcn_sched_barrier(0);
        barrier_vm<0>();
    }

    // The task's partial into slot `task`; or, when the row tile is one chunk (e.nch == 1), the
    // output rows themselves: what the merge does with a single partial (divide by l, the inverse
    // rotation, the scale fl32(1/sqrt(b))), with the stages across the lane's 16-lane row (dims
    // 16 c + n: h < 16) and then across its column blocks (h >= 16).
    __device__ void finish(int task, const MqEntry& e, int rt)
    {
        lsum += lane_xor16(lsum);
        lsum = add_xor32(lsum);
        zsum += lane_xor16(zsum);
        zsum = add_xor32(zsum);
        if (e.nch == 1) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int row = 4 * g + i;
                const float z = __shfl(zsum, row, 64);
                const float inv = 1.f / (__shfl(lsum, row, 64) * (1.f / kPScale));
                float x[NCB];
#pragma unroll
                for (int c = 0; c < NCB; c++) x[c] = ((acc[c][i] + z) * (1.f / kPScale)) * inv;
                static_for<0, 4>([&](auto S) {
                    constexpr int M = 1 << S;
                    if (M < a.block) {
                        const float sgn = (lane & M) ? -1.f : 1.f;
#pragma unroll
                        for (int c = 0; c < NCB; c++) x[c] = butterfly_xor<M>(x[c], sgn);
                    }
                });
#pragma unroll
                for (int hc = 1; hc < NCB; hc <<= 1) {
                    if (16 * hc < a.block) {
#pragma unroll
                        for (int c = 0; c < NCB; c++) {
                            if (c & hc) continue;
                            const float u = x[c], w = x[c + hc];
                            x[c] = u + w;
                            x[c + hc] = u - w;
                        }
                    }
                }
                const int jq = rt * QT + row / G, gi = row % G;
                if (jq < e.nq) {
                    float* out = a.out + ((int64_t)(e.qrow0 + jq) * a.hq + head * G + gi) * D + n;
#pragma unroll
                    for (int c = 0; c < NCB; c++) out[16 * c] = x[c] * a.cb;
                }
            }
            return;
        }
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

// Workgroup order for the XCDs.  Tasks run with the row tile fastest, so the 16 row tiles of a
// (sequence, kv head, chunk) -- four consecutive workgroups -- read the same pages.  Workgroups are
// dispatched to the 8 XCDs of the chip in turn (b on XCD b % 8), each with its own L2; this
// bijection of [0, 32 floor(n / 32)) gives each group of four consecutive task blocks one XCD, so
// that their re-reads of the pages hit the same L2.  The last n % 32 blocks keep their order.
__device__ __forceinline__ int xcd_grouped_block(int b, int nb)
{
    const int full = nb / 32 * 32;
    if (b >= full) return b;
    const int xcd = b & 7, slot = b >> 3;
    return (slot >> 2) * 32 + xcd * 4 + (slot & 3);
}

// The task's wave: entry, kv head, chunk and row tile of task `wave`, then its steps.  SH: the
// INT4 steps are shared by the workgroup's four waves (tasks 4k .. 4k + 3: row tiles of one
// chunk), through `ring` (the workgroup's stage ring) and `spr` (its operand area).
template <int D, int G, int FMT, bool SH>
__device__ __forceinline__ void mq_split_task(const MqArgs& a, int wave, int lane, int wv,
                                              __attribute__((address_space(3))) uint8_t* ring,
                                              __attribute__((address_space(3))) uint8_t* spr)
{
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
    W.ring = ring;
    W.spr = spr;
    W.wv = wv;
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
    const int s0 = chunk * a.spc;
    const int s1 = s0 + a.spc < e.steps ? s0 + a.spc : e.steps;
    const int n8 = FMT == FMT_INT8 ? e.steps : a.n8;
    W.prologue(e, rt);
    W.run8(s0, s1 < n8 ? s1 : n8);
    if (FMT == FMT_INT4_PROT) {
        if constexpr (SH)
            W.run4_sh(s0 > n8 ? s0 : n8, s1);
        else
            W.run4(s0 > n8 ? s0 : n8, s1);
    }
    W.finish(wave, e, rt);
}

template <int D, int G, int FMT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void mq_split_kernel(MqArgs a)
{
    const int wave = xcd_grouped_block((int)blockIdx.x, (int)gridDim.x) * 4 + (int)(threadIdx.x >> 6);
    if (wave >= a.tasks) return;
    const int lane = (int)(threadIdx.x & 63);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    __shared__ __align__(16) uint8_t mq_ring[4][MqWave<D, G, FMT>::RING];
    mq_split_task<D, G, FMT, false>(a, wave, lane, wv, (__attribute__((address_space(3))) uint8_t*)mq_ring[wv], nullptr);
}

// Workgroup-shared INT4 steps: launched only when every entry's row-tile count is a multiple of 4,
// so that a.tasks is too and the four waves of a workgroup take row tiles 4k .. 4k + 3 of one
// (entry, kv head, chunk): all four run the same steps and pass the same barriers, and no wave of
// a launched workgroup leaves early.
template <int D, int G, int FMT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void mq_split_shared_kernel(MqArgs a)
{
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wave = xcd_grouped_block((int)blockIdx.x, (int)gridDim.x) * 4 + wv;
    const int lane = (int)(threadIdx.x & 63);
    __shared__ __align__(16) uint8_t mq_sh[MqWave<D, G, FMT>::SH_LDS];
    __attribute__((address_space(3))) uint8_t* base = (__attribute__((address_space(3))) uint8_t*)mq_sh;
    mq_split_task<D, G, FMT, true>(a, wave, lane, wv, base, base + MqWave<D, G, FMT>::SH_RING);
}

// Merge waves: one per (row tile, RQ of its rows); lane l holds output dims DPM l .. DPM l + DPM - 1.
// With RQ > 1 the rows share the wave's entry lookup and their loads are issued together, which
// pays once one row per wave would take several rounds of resident waves (many row tiles); with
// few tiles one row per wave keeps more rows in flight.  Row r's chunk partials are merged in chunk
// order (log-sum-exp against their maximum), then the inverse FWHT is applied and the row stored.
constexpr int kMqMergeWideWaves = 16384; // one-row waves from which RQ = 4 is used

template <int D, int G, bool ROT, int RQ>
__global__ __launch_bounds__(256) void mq_merge_kernel(MqArgs a)
{
    constexpr int DPM = D / 64;
    constexpr int QT = kMqRows / G;
    constexpr int NC = 8; // chunk count of the one-round-trip path
    const int wave = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (wave >= a.groups * (kMqRows / RQ)) return;
    const int lane = (int)(threadIdx.x & 63);
    const int grp = wave / (kMqRows / RQ), r0 = (wave % (kMqRows / RQ)) * RQ;
    const int lo = mq_find_entry<true>(a, grp, lane);
    const int nq = mq_uniform(&a.entries[lo].nq);
    const int qrow0 = mq_uniform(&a.entries[lo].qrow0);
    const int task0 = mq_uniform(&a.entries[lo].task0);
    const int grp0 = mq_uniform(&a.entries[lo].grp0);
    const int nch = mq_uniform(&a.entries[lo].nch);
    if (nch == 1) return; // the split kernel wrote these rows from their single partial
    const int nrt = (nq * G + kMqRows - 1) / kMqRows;
    const int local = grp - grp0;
    const int head = local / nrt, rt = local - head * nrt;
    if (rt * QT + r0 / G >= nq) return; // every row of the wave lies past the entry's queries
    // chunk c's partials of the tile sit in task slot T(c) = T0 + c nrt: (m, l) of row r at
    // part_ml[(T(c) kMqRows + r) 2], its output at part_o[(T(c) kMqRows + r) D]
    const int64_t T0 = (int64_t)task0 + (int64_t)head * nch * nrt + rt;
    const int64_t cstride = (int64_t)nrt * kMqRows; // rows from one chunk's slot to the next
    float l[RQ], o[RQ][DPM];
#pragma unroll
    for (int q = 0; q < RQ; q++) {
        l[q] = 0.f;
#pragma unroll
        for (int k = 0; k < DPM; k++) o[q][k] = 0.f;
    }
    if (nch <= NC) {
        // every (m, l) and every output row of the RQ rows loaded before the first is used; lane c
        // holds chunk c's (m, l), chunks past nch repeat the last one's outputs and get weight 0
        float mj[RQ], lj[RQ], pv[NC][RQ][DPM];
#pragma unroll
        for (int q = 0; q < RQ; q++) {
            const float* mlc = a.part_ml + ((T0 * kMqRows + r0 + q) + (int64_t)lane * cstride) * 2;
            mj[q] = lane < nch ? mlc[0] : -__builtin_inff();
            lj[q] = lane < nch ? mlc[1] : 0.f;
        }
#pragma unroll
        for (int c = 0; c < NC; c++) {
            const float* po = a.part_o + ((T0 * kMqRows + r0) + (int64_t)(c < nch ? c : nch - 1) * cstride) * D + lane * DPM;
#pragma unroll
            for (int q = 0; q < RQ; q++)
#pragma unroll
                for (int k = 0; k < DPM; k++) pv[c][q][k] = po[q * D + k];
        }
#pragma unroll
        for (int q = 0; q < RQ; q++) {
            const float M = wave_max_u(mj[q]);
            const float wgt = exp2f(mj[q] - M);
            l[q] = wave_sum_u(wgt * lj[q]);
#pragma unroll
            for (int c = 0; c < NC; c++) {
                if (c < nch) {
                    const float w = as_float((uint32_t)__builtin_amdgcn_readlane((int)as_uint(wgt), c));
#pragma unroll
                    for (int k = 0; k < DPM; k++) o[q][k] = fmaf(w, pv[c][q][k], o[q][k]);
                }
            }
        }
    } else {
#pragma unroll
        for (int q = 0; q < RQ; q++) {
            const int r = r0 + q;
            float M = -__builtin_inff();
            for (int c0 = 0; c0 < nch; c0 += 64) {
                const int c = c0 + lane;
                M = fmaxf(M, c < nch ? a.part_ml[((T0 * kMqRows + r) + (int64_t)c * cstride) * 2] : -__builtin_inff());
            }
            M = wave_max_u(M);
            for (int c0 = 0; c0 < nch; c0 += 64) {
                const int c = c0 + lane;
                const float* mlc = a.part_ml + ((T0 * kMqRows + r) + (int64_t)c * cstride) * 2;
                const float m = c < nch ? mlc[0] : -__builtin_inff();
                const float lc = c < nch ? mlc[1] : 0.f;
                const float wgt = exp2f(m - M);
                l[q] += wave_sum_u(wgt * lc);
                // the outputs in chunk order, each weight read from its lane; the loads of 8 chunks
                // are issued before the first of them is used
                const int cn = __builtin_amdgcn_readfirstlane(nch - c0 < 64 ? nch - c0 : 64);
                const float* obase = a.part_o + (T0 * kMqRows + r) * D;
                for (int cb = 0; cb < cn; cb += 8) {
                    float pw[8][DPM];
#pragma unroll
                    for (int k = 0; k < 8; k++) {
                        const float* po = obase + (int64_t)(c0 + cb + k) * cstride * D;
#pragma unroll
                        for (int d = 0; d < DPM; d++) pw[k][d] = cb + k < cn ? po[lane * DPM + d] : 0.f;
                    }
#pragma unroll
                    for (int k = 0; k < 8; k++) {
                        if (cb + k < cn) {
                            const float w = as_float((uint32_t)__builtin_amdgcn_readlane((int)as_uint(wgt), cb + k));
#pragma unroll
                            for (int d = 0; d < DPM; d++) o[q][d] = fmaf(w, pw[k][d], o[q][d]);
                        }
                    }
                }
            }
        }
    }
#pragma unroll
    for (int q = 0; q < RQ; q++) {
        const int r = r0 + q;
        const int jq = rt * QT + r / G, gi = r % G;
        if (jq >= nq) continue; // (wave-uniform)
        float x[DPM];
        const float inv = 1.f / l[q];
#pragma unroll
        for (int k = 0; k < DPM; k++) x[k] = o[q][k] * inv;
        if (ROT) {
            // x H_bd (Sylvester H is symmetric, so this is also x H_bd^T), stages h = 1, 2, ..., b/2
            if (DPM == 2 && a.block > 1) {
                const float u = x[0], w = x[DPM - 1];
                x[0] = u + w;
                x[DPM - 1] = u - w;
            }
            static_for<0, 6>([&](auto S) {
                constexpr int M = 1 << S;
                if (M * DPM < a.block) {
                    const float sgn = (lane & M) ? -1.f : 1.f;
#pragma unroll
                    for (int k = 0; k < DPM; k++) x[k] = butterfly_xor<M>(x[k], sgn);
                }
            });
#pragma unroll
            for (int k = 0; k < DPM; k++) x[k] *= a.cb;
        }
        float* out = a.out + ((int64_t)(qrow0 + jq) * a.hq + head * G + gi) * D + lane * DPM;
#pragma unroll
        for (int k = 0; k < DPM; k++) out[k] = x[k];
    }
}

template <int D, int G, int FMT>
hipError_t split_dispatch(const MqArgs& a, hipStream_t stream, const KernelTimer& tm)
{
    const int blocks = (a.tasks + 3) / 4;
    if (FMT == FMT_INT4_PROT && a.share) {
        if (a.tasks % 4 != 0) return hipErrorInvalidValue; // the shared kernel needs whole workgroups
        return launch_kernel(mq_split_shared_kernel<D, G, FMT>, dim3(blocks), dim3(256), stream, tm, a);
    }
    return launch_kernel(mq_split_kernel<D, G, FMT>, dim3(blocks), dim3(256), stream, tm, a);
}

template <int D, int G>
hipError_t merge_dispatch(const MqArgs& a, hipStream_t stream, const KernelTimer& tm)
{
    if ((int64_t)a.groups * kMqRows >= kMqMergeWideWaves) {
        const int blocks = (int)(((int64_t)a.groups * (kMqRows / 4) + 3) / 4);
        return launch_kernel(mq_merge_kernel<D, G, true, 4>, dim3(blocks), dim3(256), stream, tm, a);
    }
    const int blocks = (int)(((int64_t)a.groups * kMqRows + 3) / 4);
    return launch_kernel(mq_merge_kernel<D, G, true, 1>, dim3(blocks), dim3(256), stream, tm, a);
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
