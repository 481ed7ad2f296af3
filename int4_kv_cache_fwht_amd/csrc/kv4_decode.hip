// kv4_decode.hip -- GQA decode attention over the paged INT4 cache with INT8 sink/recent slots:
// split-KV flash-decode kernel, then a log-sum-exp merge that also applies the inverse rotation.
// Source: "SAW-INT4: System-Aware 4-Bit KV-Cache Quantization for Real-World LLM Serving",
// Abstract (fused attention over a paged INT4 cache after a block-diagonal Hadamard rotation);
// "KV4-RL: Unlocking Faster Asynchronous Rollouts for RLVR with INT4 KV Cache Quantization",
// Abstract (sinks and recent context read from INT8).
//
// Work split: the (sequence, kv head) units are laid end to end as a global range of steps and
// every wave takes an equal contiguous share of it (balanced for any length mix), writing one
// partial (reference max, sum, output) per unit it touches.  A step covers
//   INT4:  4 pages = 64 positions, lane = position.  The K codes are the B operand of
//          v_mfma_f32_4x4x4f16 as fp16 subnormal patterns (value code * 2^-24, exact); the
//          rotated, power-of-two-normalised query split into hi + lo fp16 is the A operand,
//          broadcast from one lane quad to all 16 blocks (CBSZ = 4, ABID = quad).  A score is
//          s * (q . code) + z * sum(q): keys are never dequantised element by element.
//   INT8:  32 protection slots (or 2 INT8 pages), lanes 0..31, same scheme with byte codes.
//   BF16:  1 page = 16 positions, lanes 0..15, raw bf16 operands.
// PV runs on the same MFMA with lane = output dim: V codes (dim-major in the page) are the B
// operand and p*s (split hi + lo fp16 after an fp32 exchange through LDS) is broadcast; the
// zero-point term sum_t p_t z_t is accumulated per lane and added once per unit.
//
// Latency hiding: the next step's loads are issued before the current step's arithmetic
// (ping-pong buffers).  Every load of a step is issued unconditionally -- indices past the end are
// clamped onto the last valid page, whose lines the same step already reads, and the duplicated
// positions are masked -- so that the waitcnt counters never have to drain the prefetch.  Page ids
// and the plan are read with scalar loads (a separate counter) one step ahead.
#include "kv4_common.cuh"

namespace kv4 {

constexpr int kLdsQBytes = 4 * 128 * 4; // rotated query, G x D fp32
constexpr int kLdsPBytes = 64 * 16;     // per-step probability exchange (fp32)
constexpr int kLdsPerWave = kLdsQBytes + kLdsPBytes;
// Running max: a full reduction (and rescale) happens only when some score exceeds the current
// reference by more than kTau; p * s_V = 2^(score + log2 s_V - m + kPOffset) <= 2^(kPOffset + kTau)
// = 2^15 keeps the fp16 PV operand in range.
constexpr float kTau = 1.f;
constexpr float kPOffset = 14.f;

// Wave-uniform read through the constant address space: a scalar load (lgkmcnt), so it never
// waits on the vector loads in flight.  Only for memory no kernel of this launch writes (the block
// table and the plan); the scalar cache is invalidated at every dispatch.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* p)
{
    return *(const __attribute__((address_space(4))) T*)p;
}

__device__ __forceinline__ DecodeUnit ld_unit(const DecodeUnit* units, int u)
{
    DecodeUnit r;
    r.seq = ld_uniform(&units[u].seq);
    r.len = ld_uniform(&units[u].len);
    r.entry = ld_uniform(&units[u].entry);
    r.head = ld_uniform(&units[u].head);
    r.step_begin = ld_uniform(&units[u].step_begin);
    return r;
}

// s_waitcnt vmcnt(0), other counters untouched (gfx9 encoding)
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int D, int G, int FMT>
struct DecodeWave {
    static constexpr int NHV = D / 64;   // output dims per lane
    static constexpr int NPAIR = D / 32; // A-operand VGPR pairs of the INT4 / INT8 query sets
    static constexpr int NPAIR_BF = D / 64;
    static constexpr int NQ = (FMT == FMT_BF16) ? 2 * NPAIR_BF : G * NHV; // raw query registers

    struct Int4Data {
        u32x4 kc[D / 32];
        u32x2 sz;
        u32x2 vc[kInt4StepPages][NHV];
    };
    struct Int8Data {
        u32x4 k8[D / 16];
        u32x2 sz;
        u32x4 v8[2][NHV];
    };

    const DecodeArgs& a;
    const int lane;
    uint8_t* lds_q;
    uint8_t* lds_p;

    half4_t A4[NPAIR], A8[NPAIR];
    short4_t Abf[NPAIR_BF];
    float4_t acc[NHV][2]; // two accumulation chains per output half
    float m[4], lsum[4], zsum[4], F[4], sumq[4];

    __device__ DecodeWave(const DecodeArgs& args, int ln, uint8_t* lq, uint8_t* lp)
        : a(args), lane(ln), lds_q(lq), lds_p(lp) {}

    // ---- query: raw loads (issued first), then rotate / normalise / split into A operands ----
    __device__ __forceinline__ void load_q(const DecodeUnit& U, uint32_t (&qr)[NQ])
    {
        const uint16_t* qrow = a.q + ((int64_t)U.entry * (a.hkv * G) + U.head * G) * D;
        if constexpr (FMT == FMT_BF16) {
            // A step m = dims 4m..4m+3 of head lane&3, pair m/16, quad m%16
            const int s = lane >> 2, i = lane & 3;
            const int ic = i < G ? i : 0;
#pragma unroll
            for (int v = 0; v < NPAIR_BF; v++) {
                const uint32_t* src = (const uint32_t*)(qrow + ic * D + 4 * (16 * v + s));
                qr[2 * v] = src[0];
                qr[2 * v + 1] = src[1];
            }
        } else {
#pragma unroll
            for (int i = 0; i < G; i++)
#pragma unroll
                for (int j = 0; j < NHV; j++) qr[i * NHV + j] = qrow[i * D + 64 * j + lane];
        }
    }

    __device__ void prologue(const uint32_t (&qr)[NQ], bool need4, bool need8)
    {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            m[i] = -INFINITY;
            lsum[i] = 0.f;
            zsum[i] = 0.f;
        }
#pragma unroll
        for (int hv = 0; hv < NHV; hv++) acc[hv][0] = acc[hv][1] = (float4_t){0.f, 0.f, 0.f, 0.f};

        if constexpr (FMT == FMT_BF16) {
            const bool live = (lane & 3) < G;
#pragma unroll
            for (int v = 0; v < NPAIR_BF; v++) Abf[v] = to_short4(live ? qr[2 * v] : 0u, live ? qr[2 * v + 1] : 0u);
#pragma unroll
            for (int i2 = 0; i2 < 4; i2++) {
                F[i2] = a.scale_log2;
                sumq[i2] = 0.f;
            }
        } else {
            // lane holds dims lane + 64*j of each head; block FWHT in fp32 (any stage order)
            float qv[G][NHV];
#pragma unroll
            for (int i = 0; i < G; i++)
#pragma unroll
                for (int j = 0; j < NHV; j++) qv[i][j] = as_float(qr[i * NHV + j] << 16);
            for (int hh = 1; hh < a.block && hh < 64; hh <<= 1) {
#pragma unroll
                for (int i = 0; i < G; i++)
#pragma unroll
                    for (int j = 0; j < NHV; j++) {
                        const float other = __shfl_xor(qv[i][j], hh, 64);
                        qv[i][j] = (lane & hh) ? other - qv[i][j] : qv[i][j] + other;
                    }
            }
            if constexpr (NHV > 1) {
                if (a.block > 64) {
#pragma unroll
                    for (int i = 0; i < G; i++) {
                        const float a0 = qv[i][0], a1 = qv[i][1];
                        qv[i][0] = a0 + a1;
                        qv[i][1] = a0 - a1;
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
                    mx = wave_max_u(mx);
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
                    sumq[i] = wave_sum_u(sq);
                    F[i] = a.scale_log2 * ldexpf(1.0f, -eq);
                } else {
                    sumq[i] = 0.f;
                    F[i] = 0.f;
                }
            }
            wave_lds_sync();
            const int s = lane >> 2, i = lane & 3;
            if (need4) {
                // INT4 step m = 16c + 4wd + 2gp + hl: pair c, quad m % 16; the dims of word
                // u = 4c + wd are fed in the order (8u, 8u+4, 8u+1, 8u+5) (gp 0) or
                // (8u+2, 8u+6, 8u+3, 8u+7) (gp 1); the odd dims arrive multiplied by 16.
                const int hl = s & 1, gp = (s >> 1) & 1, wd = s >> 2;
#pragma unroll
                for (int c = 0; c < NPAIR; c++) {
                    const int d0 = 8 * (4 * c + wd) + 2 * gp;
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
                        const _Float16 hi16 = (_Float16)x[k];
                        r[k] = hl ? (_Float16)(x[k] - (float)hi16) : hi16;
                    }
                    A4[c] = (half4_t){r[0], r[1], r[2], r[3]};
                }
            }
            if (need8) {
                // INT8 step m = 2u + hl (dims 4u..4u+3): pair m / 16, quad m % 16
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
                        const _Float16 hi16 = (_Float16)x[k];
                        r[k] = hl ? (_Float16)(x[k] - (float)hi16) : hi16;
                    }
                    A8[v] = (half4_t){r[0], r[1], r[2], r[3]};
                }
            }
            wave_lds_sync();
        }
    }

    // ---- online softmax over one step: sc[i] are log2-domain scores (-inf where masked) ----
    // Quantized formats track the max of score + log2(s_V) (see kTau / kPOffset).
    __device__ __forceinline__ void softmax_step(const float (&sc)[4], float lg, bool valid, float sVv, float zVv,
                                                 float (&pt)[4])
    {
        float ep[4];
        bool over = false;
#pragma unroll
        for (int i = 0; i < G; i++) {
            ep[i] = valid ? ((FMT == FMT_BF16) ? sc[i] : sc[i] + lg) : -INFINITY;
            over |= ep[i] > m[i] + kTau;
        }
        if (__builtin_amdgcn_ballot_w64(over) != 0) {
            float mnew[4];
#pragma unroll
            for (int i = 0; i < G; i++) mnew[i] = fmaxf(m[i], wave_max_u(ep[i]));
#pragma unroll
            for (int i = 0; i < G; i++) {
                if (mnew[i] > m[i]) {
                    const float alpha = (m[i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[i] - mnew[i]);
#pragma unroll
                    for (int hv = 0; hv < NHV; hv++) {
                        acc[hv][0][i] *= alpha;
                        acc[hv][1][i] *= alpha;
                    }
                    lsum[i] *= alpha;
                    zsum[i] *= alpha;
                    m[i] = mnew[i];
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            if (i < G) {
                const float off = (m[i] == -INFINITY) ? 0.f : ((FMT == FMT_BF16) ? -m[i] : kPOffset - m[i]);
                const float p = valid ? __builtin_amdgcn_exp2f(sc[i] + off) : 0.f;
                lsum[i] += p;
                if (FMT != FMT_BF16) {
                    zsum[i] = fmaf(p, zVv, zsum[i]);
                    pt[i] = p * sVv;
                } else {
                    pt[i] = p;
                }
            } else {
                pt[i] = 0.f;
            }
        }
    }

    // PV operand exchange: writer lane stores its fp32 values at lds_p[st][head][slot]; reader
    // lane (4 st + head) gets the 4 slots of PV step st and splits them into fp16 hi + lo
    // (slots 2, 3 scaled by 1/16 when the V codes of those slots arrive multiplied by 16).
    __device__ __forceinline__ void exchange_h(const float (&pt)[4], int st_w, int kk, bool writer, bool odd16,
                                               half4_t& Ahi, half4_t& Alo)
    {
        float* L32 = (float*)lds_p;
        if (writer) {
#pragma unroll
            for (int i = 0; i < 4; i++) L32[(st_w * 4 + i) * 4 + kk] = pt[i];
        }
        wave_lds_sync();
        float4_t v = *(const float4_t*)(L32 + lane * 4);
        wave_lds_sync();
        if (odd16) {
            v.z *= 0.0625f;
            v.w *= 0.0625f;
        }
        const auto h01 = __builtin_amdgcn_cvt_pkrtz(v.x, v.y);
        const auto h23 = __builtin_amdgcn_cvt_pkrtz(v.z, v.w);
        const auto l01 = __builtin_amdgcn_cvt_pkrtz(v.x - (float)h01[0], v.y - (float)h01[1]);
        const auto l23 = __builtin_amdgcn_cvt_pkrtz(v.z - (float)h23[0], v.w - (float)h23[1]);
        Ahi = to_half4(__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23));
        Alo = to_half4(__builtin_bit_cast(uint32_t, l01), __builtin_bit_cast(uint32_t, l23));
    }

    // ================================ INT4 steps ================================
    // page ids of the step whose first page is p_first (clamped to the last INT4 page)
    __device__ __forceinline__ void int4_ids(const DecodeUnit& U, int p_first, int p_end, int32_t (&id)[4])
    {
        const int32_t* btr = a.bt + (int64_t)U.seq * a.max_pps;
        const int last = p_end - 1;
#pragma unroll
        for (int q = 0; q < kInt4StepPages; q++) id[q] = ld_uniform(btr + min(p_first + q, last));
    }

    __device__ __forceinline__ void int4_load(const DecodeUnit& U, const int32_t (&id)[4], Int4Data& dd)
    {
        const int pj = lane >> 4, t16 = lane & 15;
        const int64_t stride = (int64_t)a.hkv * a.page_block;
        const int64_t hoff = (int64_t)U.head * a.page_block;
        const int32_t my_id = pj == 0 ? id[0] : pj == 1 ? id[1] : pj == 2 ? id[2] : id[3];
        const uint8_t* pbl = a.pool + (int64_t)my_id * stride + hoff;
#pragma unroll
        for (int c = 0; c < D / 32; c++) dd.kc[c] = *(const u32x4*)(pbl + c * 256 + t16 * 16);
        dd.sz = *(const u32x2*)(pbl + 16 * D + t16 * 8);
#pragma unroll
        for (int q = 0; q < kInt4StepPages; q++) {
            const uint8_t* pbq = a.pool + (int64_t)id[q] * stride + hoff;
#pragma unroll
            for (int hv = 0; hv < NHV; hv++) dd.vc[q][hv] = *(const u32x2*)(pbq + 8 * D + (64 * hv + lane) * 8);
        }
    }

    // QK + softmax + exchange; returns the PV A operands
    __device__ __forceinline__ void int4_qk(const DecodeUnit& U, int p_first, int p_end, const Int4Data& dd,
                                            half4_t& Ahi, half4_t& Alo)
    {
        const int npg = min(kInt4StepPages, p_end - p_first);
        const int pj = lane >> 4, t16 = lane & 15;
        const int pos = (p_first + pj) * kPageSize + t16;
        const bool valid = pj < npg && pos >= a.sinks && pos < U.len - a.recent;

        // steps m = 16c + 4wd + 2gp + hl; two accumulation chains
        float4_t S2[2];
        S2[0] = S2[1] = (float4_t){0.f, 0.f, 0.f, 0.f};
        static_for<0, D / 32>([&](auto C) {
            static_for<0, 4>([&](auto WD) {
                const uint32_t w = dd.kc[C][(int)WD];
                const uint32_t w8 = w >> 8;
                const half4_t B0 = to_half4(w & 0x000F000Fu, w & 0x00F000F0u);
                const half4_t B1 = to_half4(w8 & 0x000F000Fu, w8 & 0x00F000F0u);
                constexpr int m0 = (4 * C + WD) * 4;
                constexpr int ch = WD & 1;
                S2[ch] = mfma_h<(m0 + 0) % 16>(A4[C], B0, S2[ch]);
                S2[ch] = mfma_h<(m0 + 1) % 16>(A4[C], B0, S2[ch]);
                S2[ch] = mfma_h<(m0 + 2) % 16>(A4[C], B1, S2[ch]);
                S2[ch] = mfma_h<(m0 + 3) % 16>(A4[C], B1, S2[ch]);
            });
        });
        const float4_t S = S2[0] + S2[1];

        const float sK = f16_bits_to_float(dd.sz.x & 0xFFFFu), zK = f16_bits_to_float(dd.sz.x >> 16);
        const float sV = f16_bits_to_float(dd.sz.y & 0xFFFFu), zV = f16_bits_to_float(dd.sz.y >> 16);
        const float sK24 = sK * 16777216.0f;
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; i++) sc[i] = valid ? F[i] * fmaf(S[i], sK24, zK * sumq[i]) : -INFINITY;
        const float lg = (sV > 0.f) ? __builtin_amdgcn_logf(sV) : -24.f;
        float pt[4];
        softmax_step(sc, lg, valid, valid ? sV : 0.f, valid ? zV : 0.f, pt);

        // position t16 = 8wd + n feeds PV step 4pj + 2wd + ((n >> 1) & 1), slot kk
        const int n = t16 & 7, wd = t16 >> 3;
        const int st_w = pj * 4 + wd * 2 + ((n >> 1) & 1);
        const int kk = ((n >> 2) & 1) | ((n & 1) << 1);
        exchange_h(pt, st_w, kk, true, true, Ahi, Alo);
    }

    __device__ __forceinline__ void int4_pv(const Int4Data& dd, const half4_t& Ahi, const half4_t& Alo)
    {
        // pages past the range carry zero probabilities: their (duplicated) codes add nothing
        static_for<0, kInt4StepPages>([&](auto PJ) {
            static_for<0, 2>([&](auto WD) {
                static_for<0, NHV>([&](auto HV) {
                    const uint32_t w = dd.vc[PJ][HV][(int)WD];
                    const uint32_t w8 = w >> 8;
                    const half4_t B0 = to_half4(w & 0x000F000Fu, w & 0x00F000F0u);
                    const half4_t B1 = to_half4(w8 & 0x000F000Fu, w8 & 0x00F000F0u);
                    constexpr int s0 = PJ * 4 + WD * 2;
                    acc[HV][WD] = mfma_h<s0>(Ahi, B0, acc[HV][WD]);
                    acc[HV][WD] = mfma_h<s0>(Alo, B0, acc[HV][WD]);
                    acc[HV][WD] = mfma_h<s0 + 1>(Ahi, B1, acc[HV][WD]);
                    acc[HV][WD] = mfma_h<s0 + 1>(Alo, B1, acc[HV][WD]);
                });
            });
        });
    }

    // ================================ INT8 steps ================================
    // Tile bases of INT8 step j (clamped to existing tiles / pages).
    __device__ __forceinline__ void int8_bases(const DecodeUnit& U, int j, const uint8_t* (&tb)[2])
    {
        if constexpr (FMT == FMT_INT4_PROT) {
            const uint8_t* seg = a.int8_pool + ((int64_t)U.seq * a.hkv + U.head) * a.int8_tiles * a.int8_tile;
#pragma unroll
            for (int tt = 0; tt < 2; tt++) tb[tt] = seg + (int64_t)min(2 * j + tt, a.int8_tiles - 1) * a.int8_tile;
        } else {
            const int npages = (U.len + kPageSize - 1) / kPageSize;
            const int32_t* btr = a.bt + (int64_t)U.seq * a.max_pps;
#pragma unroll
            for (int tt = 0; tt < 2; tt++)
                tb[tt] = a.pool + (int64_t)ld_uniform(btr + min(2 * j + tt, npages - 1)) * a.hkv * a.page_block +
                         (int64_t)U.head * a.page_block;
        }
    }

    __device__ __forceinline__ void int8_load(const uint8_t* const (&tb)[2], Int8Data& dd)
    {
        const int sl = lane & 31;
        // per-lane offset from tile 0 (keeps the access a global-memory load)
        const int64_t d01 = tb[1] - tb[0];
        const uint8_t* t = tb[0] + ((sl >> 4) ? d01 : (int64_t)0);
        const int s8 = sl & 15;
#pragma unroll
        for (int c = 0; c < D / 16; c++) dd.k8[c] = *(const u32x4*)(t + c * 256 + s8 * 16);
        dd.sz = *(const u32x2*)(t + 32 * D + s8 * 8);
#pragma unroll
        for (int tt = 0; tt < 2; tt++)
#pragma unroll
            for (int hv = 0; hv < NHV; hv++) dd.v8[tt][hv] = *(const u32x4*)(tb[tt] + 16 * D + (64 * hv + lane) * 16);
    }

    __device__ __forceinline__ void int8_compute(const DecodeUnit& U, int j, const Int8Data& dd)
    {
        const bool lane_ok = lane < 32;
        const int sl = lane & 31;
        bool valid = false;
        if constexpr (FMT == FMT_INT4_PROT) {
            const int u = kInt8StepSlots * j + sl;
            const int L = U.len;
            if (lane_ok && u < a.sinks + a.recent) {
                if (u < a.sinks) {
                    valid = u < L;
                } else {
                    const int back = L - 1 - (u - a.sinks);
                    if (back >= 0) valid = (L - 1 - back % a.recent) >= a.sinks;
                }
            }
        } else {
            const int pos = (2 * j + (sl >> 4)) * kPageSize + (sl & 15);
            valid = lane_ok && pos < U.len;
        }

        // QK: word (c, wd) holds dims 4u..4u+3 (u = 4c + wd); steps m = 2u + hl
        float4_t S4[4];
#pragma unroll
        for (int c = 0; c < 4; c++) S4[c] = (float4_t){0.f, 0.f, 0.f, 0.f};
        static_for<0, D / 16>([&](auto C) {
            static_for<0, 4>([&](auto WD) {
                const uint32_t w = dd.k8[C][(int)WD];
                const half4_t B = to_half4(__builtin_amdgcn_perm(0u, w, 0x0C010C00u),
                                           __builtin_amdgcn_perm(0u, w, 0x0C030C02u));
                constexpr int u = 4 * C + WD;
                S4[WD] = mfma_h<(2 * u) % 16>(A8[(2 * u) / 16], B, S4[WD]);
                S4[WD] = mfma_h<(2 * u + 1) % 16>(A8[(2 * u + 1) / 16], B, S4[WD]);
            });
        });
        const float4_t S = (S4[0] + S4[1]) + (S4[2] + S4[3]);

        const float sK = f16_bits_to_float(dd.sz.x & 0xFFFFu), zK = f16_bits_to_float(dd.sz.x >> 16);
        const float sV = f16_bits_to_float(dd.sz.y & 0xFFFFu), zV = f16_bits_to_float(dd.sz.y >> 16);
        const float sK24 = sK * 16777216.0f;
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; i++) sc[i] = valid ? F[i] * fmaf(S[i], sK24, zK * sumq[i]) : -INFINITY;
        const float lg = (sV > 0.f) ? __builtin_amdgcn_logf(sV) : -24.f;
        float pt[4];
        softmax_step(sc, lg, valid, valid ? sV : 0.f, valid ? zV : 0.f, pt);

        half4_t Ahi, Alo;
        exchange_h(pt, sl >> 2, sl & 3, lane_ok, false, Ahi, Alo);

        // tiles past the range carry zero probabilities
        static_for<0, 2>([&](auto TT) {
            static_for<0, 4>([&](auto Q) {
                static_for<0, NHV>([&](auto HV) {
                    const uint32_t w = dd.v8[TT][HV][(int)Q];
                    const half4_t B = to_half4(__builtin_amdgcn_perm(0u, w, 0x0C010C00u),
                                               __builtin_amdgcn_perm(0u, w, 0x0C030C02u));
                    constexpr int s0 = 4 * TT + Q;
                    acc[HV][TT] = mfma_h<s0>(Ahi, B, acc[HV][TT]);
                    acc[HV][TT] = mfma_h<s0>(Alo, B, acc[HV][TT]);
                });
            });
        });
    }

    // ================================ BF16 steps ================================
    __device__ void bf16_step(const DecodeUnit& U, int pg)
    {
        const int32_t* btr = a.bt + (int64_t)U.seq * a.max_pps;
        const uint8_t* pb =
            a.pool + (int64_t)ld_uniform(btr + pg) * a.hkv * a.page_block + (int64_t)U.head * a.page_block;
        const int nvalid = min(kPageSize, U.len - pg * kPageSize);
        const bool valid = lane < nvalid;
        u32x4 kr[D / 8];
        const int t16 = lane & 15;
#pragma unroll
        for (int c = 0; c < D / 8; c++) kr[c] = *(const u32x4*)(pb + c * 256 + t16 * 16);
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
                        uint32_t msk = 0u;
                        if (s_lo < nvalid) msk |= 0x0000FFFFu;
                        if (s_lo + 1 < nvalid) msk |= 0xFFFF0000u;
                        vv[hv][q][k] &= msk;
                    }
        }

        float4_t S4[2];
        S4[0] = S4[1] = (float4_t){0.f, 0.f, 0.f, 0.f};
        static_for<0, D / 8>([&](auto C) {
            constexpr int m0 = 2 * C;
            S4[C % 2] = mfma_bf<m0 % 16>(Abf[m0 / 16], to_short4(kr[C].x, kr[C].y), S4[C % 2]);
            S4[C % 2] = mfma_bf<(m0 + 1) % 16>(Abf[(m0 + 1) / 16], to_short4(kr[C].z, kr[C].w), S4[C % 2]);
        });
        const float4_t S = S4[0] + S4[1];
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; i++) sc[i] = valid ? F[i] * S[i] : -INFINITY;
        float pt[4];
        softmax_step(sc, 0.f, valid, 1.f, 0.f, pt);

        // fp32 exchange; reader splits into bf16 hi (truncation) + bf16 lo (16 significant bits)
        float* L32 = (float*)lds_p;
        if (lane < kPageSize) {
#pragma unroll
            for (int i = 0; i < 4; i++) L32[((lane >> 2) * 4 + i) * 4 + (lane & 3)] = pt[i];
        }
        wave_lds_sync();
        const float4_t v = *(const float4_t*)(L32 + lane * 4);
        wave_lds_sync();
        uint32_t hb[4], lb[4];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            hb[k] = as_uint(v[k]) & 0xFFFF0000u;
            lb[k] = as_uint(v[k] - as_float(hb[k]));
        }
        const short4_t Ahi = to_short4(__builtin_amdgcn_perm(hb[1], hb[0], 0x07060302u),
                                       __builtin_amdgcn_perm(hb[3], hb[2], 0x07060302u));
        const short4_t Alo = to_short4(__builtin_amdgcn_perm(lb[1], lb[0], 0x07060302u),
                                       __builtin_amdgcn_perm(lb[3], lb[2], 0x07060302u));
        static_for<0, 4>([&](auto ST) {
            static_for<0, NHV>([&](auto HV) {
                const u32x4 w = vv[HV][ST / 2];
                const short4_t B = (ST % 2 == 0) ? to_short4(w.x, w.y) : to_short4(w.z, w.w);
                acc[HV][ST % 2] = mfma_bf<ST>(Ahi, B, acc[HV][ST % 2]);
                acc[HV][ST % 2] = mfma_bf<ST>(Alo, B, acc[HV][ST % 2]);
            });
        });
    }

    __device__ void epilogue(int64_t pidx)
    {
#pragma unroll
        for (int i = 0; i < G; i++) {
            const float l = wave_sum_u(lsum[i]);
            const float z = (FMT == FMT_BF16) ? 0.f : wave_sum_u(zsum[i]);
            float* po = a.part_o + (pidx * G + i) * D;
#pragma unroll
            for (int hv = 0; hv < NHV; hv++) {
                const float o = acc[hv][0][i] + acc[hv][1][i];
                po[64 * hv + lane] = (FMT == FMT_BF16) ? o : fmaf(o, 16777216.0f, z);
            }
            if (lane == 0) {
                float mref = m[i];
                if (mref != -INFINITY && FMT != FMT_BF16) mref -= kPOffset;
                a.part_ml[(pidx * G + i) * 2 + 0] = mref;
                a.part_ml[(pidx * G + i) * 2 + 1] = l;
            }
        }
    }

    // ---- one unit's steps [k0, k1) ----
    __device__ void run_unit(const DecodeUnit& U, int k0, int k1)
    {
        uint32_t qr[NQ];
        load_q(U, qr);
        if constexpr (FMT == FMT_BF16) {
            prologue(qr, false, false);
            for (int k = k0; k < k1; k++) bf16_step(U, k);
            return;
        } else {
            int n8 = 0, p0 = 0, p1 = 0;
            if constexpr (FMT == FMT_INT4_PROT) {
                n8 = (a.sinks + a.recent > 0) ? (a.sinks + a.recent + kInt8StepSlots - 1) / kInt8StepSlots : 0;
                const int lo4 = a.sinks, hi4 = U.len - a.recent;
                if (hi4 > lo4) {
                    p0 = lo4 / kPageSize;
                    p1 = (hi4 - 1) / kPageSize + 1;
                }
            } else {
                n8 = k1; // every step of the INT8 format is an INT8 step
            }
            const int e8 = min(k1, n8); // INT8 steps are [k0, e8), INT4 steps [max(k0, n8), k1)
            int k = k0;
            Int4Data a4, b4;
            int32_t ida[4], idb[4];
            if (k < e8) {
                // INT8 steps (a few per unit in the INT4 format): one buffer, no prefetch
                Int8Data a8;
                const uint8_t* tba[2];
                int8_bases(U, k, tba);
                int8_load(tba, a8);
                prologue(qr, k1 > n8, true);
                while (true) {
                    int8_compute(U, k, a8);
                    if (++k >= e8) break;
                    int8_bases(U, k, tba);
                    int8_load(tba, a8);
                }
                if (k >= k1) return;
                int4_ids(U, p0, p1, ida);
                int4_load(U, ida, a4);
            } else {
                int4_ids(U, p0 + kInt4StepPages * (k - n8), p1, ida);
                int4_load(U, ida, a4);
                prologue(qr, true, false);
            }
            // INT4 steps [k, k1): ping-pong; page ids one step ahead of the data
            int kn = min(k + 1, k1 - 1);
            int4_ids(U, p0 + kInt4StepPages * (kn - n8), p1, idb);
            while (true) {
                half4_t Ahi, Alo;
                int4_load(U, idb, b4); // step k + 1 (or step k again at the end: cached lines)
                int4_qk(U, p0 + kInt4StepPages * (k - n8), p1, a4, Ahi, Alo);
                kn = min(k + 2, k1 - 1);
                int4_ids(U, p0 + kInt4StepPages * (kn - n8), p1, ida);
                int4_pv(a4, Ahi, Alo);
                if (++k >= k1) break;
                int4_load(U, ida, a4);
                int4_qk(U, p0 + kInt4StepPages * (k - n8), p1, b4, Ahi, Alo);
                kn = min(k + 2, k1 - 1);
                int4_ids(U, p0 + kInt4StepPages * (kn - n8), p1, idb);
                int4_pv(b4, Ahi, Alo);
                if (++k >= k1) break;
            }
            wait_vm_all();
        }
    }
};

template <int D, int G, int FMT>
__global__ __launch_bounds__(64 * kWavesPerBlock) __attribute__((amdgpu_waves_per_eu(3)))
void decode_split_kernel(DecodeArgs a)
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
        if (ld_uniform(&a.units[mid].step_begin) <= s)
            lo = mid;
        else
            hi = mid - 1;
    }
    int u = lo;
    DecodeWave<D, G, FMT> dw(a, lane, lds_all[wv], lds_all[wv] + kLdsQBytes);
    while (s < s_end) {
        const DecodeUnit U = ld_unit(a.units, u);
        const int64_t ue = (u + 1 < a.n_units) ? ld_uniform(&a.units[u + 1].step_begin) : T;
        const int k0 = (int)(s - U.step_begin);
        const int k1 = (int)((s_end < ue ? s_end : ue) - U.step_begin);
        dw.run_unit(U, k0, k1);
        dw.epilogue(w + u);
        s = U.step_begin + k1;
        u++;
    }
}

// ---------------------------------------------------------------------------------------------
// merge: one block of G x D threads per unit; thread (i, d) merges head i, dim d
// ---------------------------------------------------------------------------------------------

__device__ __forceinline__ int64_t wave_of_step(int64_t step, int64_t T, int64_t W)
{
    const int64_t w = ((step + 1) * W - 1) / T;
    return w < W - 1 ? w : W - 1;
}

template <int D, int G, bool ROT>
__global__ __launch_bounds__(G * D) void merge_kernel(DecodeArgs a)
{
    __shared__ float buf[G * D];
    const int u = blockIdx.x;
    const int i = threadIdx.x / D, d = threadIdx.x % D;
    const DecodeUnit U = ld_unit(a.units, u);
    const int64_t T = a.total_steps, W = a.n_waves;
    const int64_t sb = U.step_begin;
    const int64_t se = (u + 1 < a.n_units) ? ld_uniform(&a.units[u + 1].step_begin) : T;
    const int64_t w0 = wave_of_step(sb, T, W), w1 = wave_of_step(se - 1, T, W);
    const int n = (int)(w1 - w0 + 1);
    const float* ml = a.part_ml + ((w0 + u) * G + i) * 2;
    const float* po = a.part_o + ((w0 + u) * G + i) * D + d;
    float M = -INFINITY;
    for (int j = 0; j < n; j++) M = fmaxf(M, ml[(int64_t)j * G * 2]);
    float Ls = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll 4
        for (int j = 0; j < n; j++) {
            const float mw = ml[(int64_t)j * G * 2];
            const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
            Ls = fmaf(ml[(int64_t)j * G * 2 + 1], f, Ls);
            O = fmaf(po[(int64_t)j * G * D], f, O);
        }
    }
    float r = (Ls > 0.f) ? O / Ls : 0.f;
    if (ROT && a.block > 1) {
        float* bh = buf + i * D;
        bh[d] = r;
        for (int hh = 1; hh < a.block; hh <<= 1) {
            __syncthreads();
            const float other = bh[d ^ hh];
            const float mine = bh[d];
            __syncthreads();
            bh[d] = (d & hh) ? other - mine : mine + other;
        }
        __syncthreads();
        r = bh[d] * a.cb;
    }
    a.out[((int64_t)U.entry * (a.hkv * G) + U.head * G + i) * D + d] = r;
}

// ---------------------------------------------------------------------------------------------
// launches
// ---------------------------------------------------------------------------------------------

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
    hipLaunchKernelGGL((merge_kernel<D, G, F != FMT_BF16>), dim3((unsigned)a.n_units), dim3(G * D), 0, stream, a);
    return hipGetLastError();
}

#define KV4_DEC_DISPATCH(FN)                                                                        \
    if (a.n_units <= 0) return hipSuccess;                                                          \
    if (d == 64 && g == 1 && format == 0) return FN<64, 1, 0>(a, stream);                           \
    if (d == 64 && g == 2 && format == 0) return FN<64, 2, 0>(a, stream);                           \
    if (d == 64 && g == 4 && format == 0) return FN<64, 4, 0>(a, stream);                           \
    if (d == 64 && g == 1 && format == 1) return FN<64, 1, 1>(a, stream);                           \
    if (d == 64 && g == 2 && format == 1) return FN<64, 2, 1>(a, stream);                           \
    if (d == 64 && g == 4 && format == 1) return FN<64, 4, 1>(a, stream);                           \
    if (d == 64 && g == 1 && format == 2) return FN<64, 1, 2>(a, stream);                           \
    if (d == 64 && g == 2 && format == 2) return FN<64, 2, 2>(a, stream);                           \
    if (d == 64 && g == 4 && format == 2) return FN<64, 4, 2>(a, stream);                           \
    if (d == 128 && g == 1 && format == 0) return FN<128, 1, 0>(a, stream);                         \
    if (d == 128 && g == 2 && format == 0) return FN<128, 2, 0>(a, stream);                         \
    if (d == 128 && g == 4 && format == 0) return FN<128, 4, 0>(a, stream);                         \
    if (d == 128 && g == 1 && format == 1) return FN<128, 1, 1>(a, stream);                         \
    if (d == 128 && g == 2 && format == 1) return FN<128, 2, 1>(a, stream);                         \
    if (d == 128 && g == 4 && format == 1) return FN<128, 4, 1>(a, stream);                         \
    if (d == 128 && g == 1 && format == 2) return FN<128, 1, 2>(a, stream);                         \
    if (d == 128 && g == 2 && format == 2) return FN<128, 2, 2>(a, stream);                         \
    if (d == 128 && g == 4 && format == 2) return FN<128, 4, 2>(a, stream);                         \
    return hipErrorInvalidValue;

hipError_t launch_decode_split(int d, int g, int format, const DecodeArgs& a, hipStream_t stream)
{
    KV4_DEC_DISPATCH(launch_split_t)
}

hipError_t launch_decode_merge(int d, int g, int format, const DecodeArgs& a, hipStream_t stream)
{
    KV4_DEC_DISPATCH(launch_merge_t)
}

#undef KV4_DEC_DISPATCH

} // namespace kv4
