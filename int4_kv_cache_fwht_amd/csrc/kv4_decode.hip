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
//   INT8:  32 slots (2 tiles), lane = slot within each half wave; the two half waves take the two
//          halves of the head dimension, the A operand is broadcast per half (CBSZ = 3) and the
//          two partial scores are added across halves.
//   BF16:  1 page = 16 positions, lanes 0..15, raw bf16 operands.
// PV runs on the same MFMA with lane = output dim: V codes (dim-major in the page) are the B
// operand and p*s (split hi + lo fp16 after an fp32 exchange through LDS) is broadcast; the
// zero-point term sum_t p_t z_t is accumulated per lane and added once per unit.
//
// Latency hiding (quantized formats): a unit's INT8 and INT4 steps run as one pipeline.  An INT8
// tile is stored as two blocks shaped like an INT4 page block, so both step types issue the same
// 13 vector loads (4 x 16 B of K, 8 B of scales, 8 x 8 B of V) into the same registers and only
// the four block addresses differ: the next step's loads are always in flight during the current
// step's arithmetic and the wait counters never drain them.  Loads past the end repeat the last
// step's addresses (cached lines) and are never used.  Page ids are read with scalar loads (their
// own counter) two steps ahead.
#include "kv4_common.h"

#include <mutex>

namespace kv4 {

// Device scratch of the allocation-free decode entry point: the split kernel's partials live here
// instead of in a caller workspace.  One copy per GPU, held until the process ends.  Host code
// never uses the array's name as an address: decode_scratch() looks up each device's copy once
// (with that device current) and every later use goes through the pointer it returns.
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};
} // namespace

hipError_t decode_scratch(void** ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

constexpr int kLdsQBytes = 4 * 128 * 4; // rotated query, G x D fp32 (raw bf16 query first)
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

// A field of the kernel's own argument block, read in place from the kernarg segment.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(4))) T* kernarg_field(size_t offset)
{
    return (const __attribute__((address_space(4))) T*)((const __attribute__((address_space(4))) char*)
                                                            __builtin_amdgcn_kernarg_segment_ptr() + offset);
}

// Global steps of one (entry, kv head) unit at length L, the start charge included (the host
// planner's rule).
template <int FMT>
__device__ __forceinline__ int unit_steps_dev(const DecodeArgs& a, int L, int n8)
{
    if (FMT == FMT_INT4_PROT) {
        const int lo = a.sinks, hi = L - a.recent;
        const int pages = hi > lo ? (hi - 1) / kPageSize + 1 - lo / kPageSize : 0;
        return kUnitStartSteps + n8 + (pages + kInt4StepPages - 1) / kInt4StepPages;
    }
    const int pages = (L + kPageSize - 1) / kPageSize;
    if (FMT == FMT_INT8) return kUnitStartSteps + (pages + kInt8StepPages - 1) / kInt8StepPages;
    return kUnitStartSteps + pages;
}

// Argument plan held in registers: lane l holds entries l + 64 j (first global step, sequence id,
// length), loaded in one batch of vector loads; a wave looks entries up with readlane.
struct EntryRegs {
    int32_t step[kArgEntries / 64], seq[kArgEntries / 64], len[kArgEntries / 64];
};

// Lane l of register j of x (j, l wave-uniform): every register is read at lane l first and the
// scalar results are selected, so the register array is never indexed at run time.
template <int N>
__device__ __forceinline__ int32_t lane_pick(const int32_t (&x)[N], int j, int l)
{
    int32_t r = __builtin_amdgcn_readlane(x[0], l);
#pragma unroll
    for (int i = 1; i < N; i++) {
        const int32_t v = __builtin_amdgcn_readlane(x[i], l);
        r = (j == i) ? v : r;
    }
    return r;
}

__device__ __forceinline__ EntryRegs load_entries(const DecodeArgs& a, int lane)
{
    const auto* stp = kernarg_field<int32_t>(offsetof(DecodeArgs, arg_step));
    const auto* seqp = kernarg_field<int32_t>(offsetof(DecodeArgs, arg_seq));
    const auto* lenp = kernarg_field<int32_t>(offsetof(DecodeArgs, arg_len));
    EntryRegs r;
#pragma unroll
    for (int j = 0; j < kArgEntries / 64; j++) {
        const int e = 64 * j + lane;
        const int ec = e < a.n_arg ? e : 0;
        r.step[j] = e < a.n_arg ? stp[ec] : 0x7FFFFFFF;
        r.seq[j] = seqp[ec];
        r.len[j] = lenp[ec];
    }
    return r;
}

// Unit u of the argument plan (entries in registers) and the end of its step range.
template <int FMT>
__device__ __forceinline__ void arg_unit(const DecodeArgs& a, const EntryRegs& er, int n8, int u, DecodeUnit& U,
                                         int64_t& ue)
{
    const int e = u / a.hkv, h = u - e * a.hkv;
    const int j = e >> 6, l = e & 63;
    U.seq = lane_pick(er.seq, j, l);
    U.len = lane_pick(er.len, j, l);
    U.entry = e;
    U.head = h;
    const int st = unit_steps_dev<FMT>(a, U.len, n8);
    U.step_begin = (int64_t)lane_pick(er.step, j, l) + (int64_t)h * st;
    ue = U.step_begin + st;
}

// The unit of the argument plan that holds global step s.
template <int FMT>
__device__ __forceinline__ int arg_first_unit(const DecodeArgs& a, const EntryRegs& er, int n8, int64_t s)
{
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < kArgEntries / 64; j++) cnt += __builtin_popcountll(__ballot(er.step[j] <= s));
    const int e = cnt - 1;
    const int j = e >> 6, l = e & 63;
    const int len = lane_pick(er.len, j, l);
    const int ex = lane_pick(er.step, j, l);
    return e * a.hkv + (int)((s - ex) / unit_steps_dev<FMT>(a, len, n8));
}

// Unit u of the argument plan read with scalar loads (the merge kernel's single lookup).
template <int FMT>
__device__ __forceinline__ void arg_unit_scalar(const DecodeArgs& a, int n8, int u, DecodeUnit& U, int64_t& ue)
{
    const int e = u / a.hkv, h = u - e * a.hkv;
    U.seq = kernarg_field<int32_t>(offsetof(DecodeArgs, arg_seq))[e];
    U.len = kernarg_field<int32_t>(offsetof(DecodeArgs, arg_len))[e];
    U.entry = e;
    U.head = h;
    const int st = unit_steps_dev<FMT>(a, U.len, n8);
    U.step_begin = (int64_t)kernarg_field<int32_t>(offsetof(DecodeArgs, arg_step))[e] + (int64_t)h * st;
    ue = U.step_begin + st;
}

// s_waitcnt vmcnt(0), other counters untouched (gfx9 encoding)
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Identity DPP move: keeps a wave-uniform value in a vector register (frees scalar registers).
__device__ __forceinline__ float in_vgpr(float x)
{
    return as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_uint(x), 0xE4, 0xF, 0xF, false));
}

// Block indices of one step (page ids or INT8 tile indices), wave-uniform.
struct Ids {
    int32_t i0, i1, i2, i3;
};

template <int D, int G, int FMT>
struct DecodeWave {
    static constexpr int NHV = D / 64;   // output dims per lane
    static constexpr int NPAIR = D / 32; // A-operand VGPR pairs of the INT4 / INT8 query sets
    static constexpr int NPAIR_BF = D / 64;
    static constexpr int NK = D / 32;    // 16-byte K pieces per lane and step
    static constexpr int NV = 4 * NHV;   // 8-byte V pieces per lane and step
    static constexpr int QLANES = G * D / 8;

    // One step's data for the quantized formats.
    //   INT4: k[c] = 16 B piece c of the lane's slot (dims 32c..32c+31), sz = its scales,
    //         v[q * NHV + hv] = 8 B of dim 64 hv + lane in page q.
    //   INT8: k[c] = dims D/2 * half + 16c .. +15 of the lane's slot (half = lane / 32, slot =
    //         lane % 32), sz = its scales, v[q * NHV + hv] = slots 16 (q % 2) + 8 (q / 2) .. +7 of
    //         dim 64 hv + lane.
    struct Buf {
        u32x4 k[NK];
        u32x2 sz;
        u32x2 v[NV];
    };

    const DecodeArgs& a;
    const int lane;
    uint8_t* lds_q;
    uint8_t* lds_p;
    const int64_t w;     // wave index (partial slot of unit u is w + u)
    const int64_t s_end; // one past the wave's last global step
    const int n8;        // INT8 steps at the start of an INT4_PROT unit

    EntryRegs er; // argument plan (a.n_arg > 0)
    // Issue-priority feedback between the two waves that share a SIMD (both in this workgroup).
    // The arbiter favours the older wave, which with equal work would finish well before the
    // younger one and leave the younger to run its last steps alone. Each wave publishes its step
    // count in LDS (prog[own]) and takes the higher priority while it is not ahead of
    // prog[partner]; own == partner (no partner) keeps it at the higher one.
    int* prog = nullptr;
    int own = 0, partner = 0;
    int done = 0;
    half4_t A4[NPAIR], A8[NPAIR];
    short4_t Abf[NPAIR_BF];
    float4_t acc[NHV][2]; // two accumulation chains per output half
    float m[4], mt[4], lsum[4], zsum[4], F[4], sumq[4]; // mt = m + kTau, the rescale threshold

    __device__ DecodeWave(const DecodeArgs& args, int ln, uint8_t* lq, uint8_t* lp, int64_t wi, int64_t se)
        : a(args), lane(ln), lds_q(lq), lds_p(lp), w(wi), s_end(se),
          n8((FMT == FMT_INT4_PROT && args.sinks + args.recent > 0)
                 ? (args.sinks + args.recent + kInt8StepSlots - 1) / kInt8StepSlots
                 : 0)
    {
    }

    __device__ __forceinline__ void reset_state()
    {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            m[i] = -INFINITY;
            mt[i] = -INFINITY;
            lsum[i] = 0.f;
            zsum[i] = 0.f;
        }
#pragma unroll
        for (int hv = 0; hv < NHV; hv++) acc[hv][0] = acc[hv][1] = (float4_t){0.f, 0.f, 0.f, 0.f};
    }

    // ---- query prologue of a unit (quantized formats): rotate, normalise, split into A operands ----
    __device__ void prologue_q(const u32x4& qraw)
    {
        reset_state();
        // raw bf16 rows through LDS into the layout "lane holds dims lane + 64 j of each head"
        uint16_t* raw = (uint16_t*)lds_q;
        if (lane < QLANES) *(u32x4*)(raw + 8 * lane) = qraw;
        wave_lds_sync();
        float qv[G][NHV];
#pragma unroll
        for (int i = 0; i < G; i++)
#pragma unroll
            for (int j = 0; j < NHV; j++) qv[i][j] = as_float((uint32_t)raw[i * D + 64 * j + lane] << 16);
        wave_lds_sync();
        // block FWHT in fp32 (any stage order); partner lane l ^ H by DPP, swizzle or permute
        static_for<0, 6>([&](auto S) {
            constexpr int H = 1 << S;
            if (H < a.block) {
                const float sgn = (lane & H) ? -1.f : 1.f;
#pragma unroll
                for (int i = 0; i < G; i++)
#pragma unroll
                    for (int j = 0; j < NHV; j++) qv[i][j] = butterfly_xor<H>(qv[i][j], sgn);
            }
        });
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
                sumq[i] = in_vgpr(wave_sum_u(sq));
                F[i] = in_vgpr(a.scale_log2 * ldexpf(1.0f, -eq));
            } else {
                sumq[i] = 0.f;
                F[i] = 0.f;
            }
        }
        wave_lds_sync();
        const int i = lane & 3;
        if (FMT == FMT_INT4_PROT) {
            // INT4 step m = 16c + 4wd + 2gp + hl: pair c, quad m % 16 (all 16 blocks); the dims of
            // word u = 4c + wd are fed in the order (8u, 8u+4, 8u+1, 8u+5) (gp 0) or
            // (8u+2, 8u+6, 8u+3, 8u+7) (gp 1); the odd dims arrive multiplied by 16.
            const int s = lane >> 2;
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
        if (FMT == FMT_INT8 || n8 > 0) {
            // INT8 step m = 8v + s of half h (lane = 32h + 4s + i): pair v, block s of the half;
            // word u = m / 2 holds dims h*D/2 + 4u .. +3, hl = m % 2
            const int h = lane >> 5, s = (lane >> 2) & 7;
#pragma unroll
            for (int v = 0; v < NPAIR; v++) {
                const int mm = 8 * v + s, u = mm >> 1, hl = mm & 1;
                const int d0 = h * (D / 2) + 4 * u;
                float x[4] = {0.f, 0.f, 0.f, 0.f};
                if (i < G) {
#pragma unroll
                    for (int k = 0; k < 4; k++) x[k] = lq[i * D + d0 + k];
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

    // ---- online softmax over one step: sc[i] are log2-domain scores (-inf where masked) ----
    // Quantized formats track the max of score + log2(s_V) (see kTau / kPOffset).
    __device__ __forceinline__ void softmax_step(const float (&sc)[4], float lg, bool valid, float sVv, float zVv,
                                                 float (&pt)[4])
    {
        // every caller passes sc = -inf on invalid lanes: their ep is -inf and their p is 0
        float ep[4];
        bool over = false;
#pragma unroll
        for (int i = 0; i < G; i++) {
            ep[i] = (FMT == FMT_BF16) ? sc[i] : sc[i] + lg;
            over |= ep[i] > mt[i];
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
                    m[i] = in_vgpr(mnew[i]);
                    mt[i] = in_vgpr(mnew[i] + kTau);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            if (i < G) {
                const float off = (m[i] == -INFINITY) ? 0.f : ((FMT == FMT_BF16) ? -m[i] : kPOffset - m[i]);
                const float p = __builtin_amdgcn_exp2f(sc[i] + off);
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
        done++;
        if (lane == 0) __hip_atomic_store(prog + own, done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        wave_lds_sync();
        float4_t v = *(const float4_t*)(L32 + lane * 4);
        const int other = __hip_atomic_load(prog + partner, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        wave_lds_sync();
        if (done <= __builtin_amdgcn_readfirstlane(other))
            __builtin_amdgcn_s_setprio(1);
        else
            __builtin_amdgcn_s_setprio(0);
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

    // ================================ steps of one unit ================================
    __device__ __forceinline__ bool is_int8_step(int k) const { return FMT == FMT_INT8 || k < n8; }

    // INT4 pages [p0, p1) of the positions [S, L - R) read from INT4 (empty when L <= S + R)
    __device__ __forceinline__ int int4_p1(int len) const
    {
        const int hi4 = len - a.recent;
        return hi4 > a.sinks ? (hi4 - 1) / kPageSize + 1 : 0;
    }

    // Block indices of step k: INT4 = 4 page ids (clamped to the last INT4 page); INT8 format =
    // the 2 pages' ids and INT8 protection = the 2 tile indices, each listed twice (tile j % 2,
    // block j / 2 of the tile).
    __device__ __forceinline__ Ids step_ids(const DecodeUnit& U, int k, int p1) const
    {
        const int32_t* btr = a.bt + (int64_t)U.seq * a.max_pps;
        Ids id;
        if (FMT == FMT_INT8) {
            const int last = (U.len + kPageSize - 1) / kPageSize - 1;
            id.i0 = ld_uniform(btr + min(2 * k, last));
            id.i1 = ld_uniform(btr + min(2 * k + 1, last));
            id.i2 = id.i0;
            id.i3 = id.i1;
        } else if (k < n8) {
            id.i0 = min(2 * k, a.int8_tiles - 1);
            id.i1 = min(2 * k + 1, a.int8_tiles - 1);
            id.i2 = id.i0;
            id.i3 = id.i1;
        } else {
            const int p_first = a.sinks / kPageSize + kInt4StepPages * (k - n8);
            const int last = p1 - 1;
            id.i0 = ld_uniform(btr + min(p_first, last));
            id.i1 = ld_uniform(btr + min(p_first + 1, last));
            id.i2 = ld_uniform(btr + min(p_first + 2, last));
            id.i3 = ld_uniform(btr + min(p_first + 3, last));
        }
        return id;
    }

    // The step's 14 vector loads.  Both step types read four blocks of 16D + 128 bytes shaped
    // alike: INT4 = the 4 pages; INT8 = block j / 2 of tile j % 2 (tile half j / 2 of the dims for
    // K, slots 16 (j % 2) + 8 (j / 2) .. +7 for V).  Only the four block addresses differ, so the
    // loads are the same instructions for both.
    __device__ __forceinline__ void load_step(const DecodeUnit& U, int k, const Ids& id, Buf& b) const
    {
        const bool t8 = is_int8_step(k);
        const uint8_t* base;
        int64_t stride;
        if (FMT == FMT_INT4_PROT && t8) {
            base = a.int8_pool + ((int64_t)U.seq * a.hkv + U.head) * a.int8_tiles * a.int8_tile;
            stride = a.int8_tile;
        } else {
            base = a.pool + (int64_t)U.head * a.page_block;
            stride = (int64_t)a.hkv * a.page_block;
        }
        const int64_t hb = t8 ? (int64_t)(16 * D + 128) : 0;
        const uint8_t* pg0 = base + (int64_t)id.i0 * stride;
        const uint8_t* pg1 = base + (int64_t)id.i1 * stride;
        const uint8_t* pg2 = base + (int64_t)id.i2 * stride + hb;
        const uint8_t* pg3 = base + (int64_t)id.i3 * stride + hb;
        // K and scales: slot lane % 16 of block lane / 16
        const int kb = lane >> 4;
        const uint8_t* pk = kb == 0 ? pg0 : kb == 1 ? pg1 : kb == 2 ? pg2 : pg3;
        const uint32_t t16 = (uint32_t)(lane & 15);
        // one fixed issue order (K, scales, V) everywhere, so that the wait counts agree on every
        // path into the pipeline loop.  The cache lines are read once per launch: nontemporal
        // loads keep them from displacing other lines (on MI355X the split kernel streams 8-11%
        // faster with them).
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c2 = 0; c2 < NK; c2++) b.k[c2] = __builtin_nontemporal_load((const u32x4*)(pk + t16 * 16 + c2 * 256));
        b.sz = __builtin_nontemporal_load((const u32x2*)(pk + 16 * D + t16 * 8));
        // V: dim 64 hv + lane of block q
#pragma unroll
        for (int hv = 0; hv < NHV; hv++) {
            const uint32_t vo = 8 * D + 512 * hv + (uint32_t)lane * 8u;
            b.v[0 * NHV + hv] = __builtin_nontemporal_load((const u32x2*)(pg0 + vo));
            b.v[1 * NHV + hv] = __builtin_nontemporal_load((const u32x2*)(pg1 + vo));
            b.v[2 * NHV + hv] = __builtin_nontemporal_load((const u32x2*)(pg2 + vo));
            b.v[3 * NHV + hv] = __builtin_nontemporal_load((const u32x2*)(pg3 + vo));
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // ================================ INT4 steps ================================
    // QK + softmax + exchange; returns the PV A operands
    __device__ __forceinline__ void int4_qk(const DecodeUnit& U, int k, int p1, const Buf& b, half4_t& Ahi,
                                            half4_t& Alo)
    {
        const int p_first = a.sinks / kPageSize + kInt4StepPages * (k - n8);
        const int npg = min(kInt4StepPages, p1 - p_first);
        const int pj = lane >> 4, t16 = lane & 15;
        const int pos = (p_first + pj) * kPageSize + t16;
        const bool valid = pj < npg && pos >= a.sinks && pos < U.len - a.recent;

        // steps m = 16c + 4wd + 2gp + hl; two accumulation chains
        float4_t S2[2];
        S2[0] = S2[1] = (float4_t){0.f, 0.f, 0.f, 0.f};
        static_for<0, NK>([&](auto C) {
            static_for<0, 4>([&](auto WD) {
                const uint32_t wv = b.k[C][(int)WD];
                const uint32_t w8 = wv >> 8;
                const half4_t B0 = to_half4(wv & 0x000F000Fu, wv & 0x00F000F0u);
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

        const float sK = f16_bits_to_float(b.sz.x & 0xFFFFu), zK = f16_bits_to_float(b.sz.x >> 16);
        const float sV = f16_bits_to_float(b.sz.y & 0xFFFFu), zV = f16_bits_to_float(b.sz.y >> 16);
        const float sK24 = sK * 16777216.0f;
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; i++) sc[i] = valid ? F[i] * fmaf(S[i], sK24, zK * sumq[i]) : -INFINITY;
        // finite on invalid lanes (unspecified scale bits), so that their ep = sc + lg stays -inf
        const float lg = (valid && sV > 0.f) ? __builtin_amdgcn_logf(sV) : -24.f;
        float pt[4];
        softmax_step(sc, lg, valid, valid ? sV : 0.f, valid ? zV : 0.f, pt);

        // position t16 = 8wd + n feeds PV step 4pj + 2wd + ((n >> 1) & 1), slot kk
        const int n = t16 & 7, wd = t16 >> 3;
        const int st_w = pj * 4 + wd * 2 + ((n >> 1) & 1);
        const int kk = ((n >> 2) & 1) | ((n & 1) << 1);
        exchange_h(pt, st_w, kk, true, true, Ahi, Alo);
    }

    __device__ __forceinline__ void int4_pv(const Buf& b, const half4_t& Ahi, const half4_t& Alo)
    {
        // pages past the range carry zero probabilities: their (duplicated) codes add nothing
        static_for<0, kInt4StepPages>([&](auto PJ) {
            static_for<0, 2>([&](auto WD) {
                static_for<0, NHV>([&](auto HV) {
                    const uint32_t wv = b.v[PJ * NHV + HV][(int)WD];
                    const uint32_t w8 = wv >> 8;
                    const half4_t B0 = to_half4(wv & 0x000F000Fu, wv & 0x00F000F0u);
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
    __device__ __forceinline__ void int8_qk(const DecodeUnit& U, int k, const Buf& b, half4_t& Ahi, half4_t& Alo)
    {
        const bool lane_ok = lane < 32;
        const int sl = lane & 31;
        bool valid = false;
        if constexpr (FMT == FMT_INT4_PROT) {
            const int u = kInt8StepSlots * k + sl;
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
            const int pos = (2 * k + (sl >> 4)) * kPageSize + (sl & 15);
            valid = lane_ok && pos < U.len;
        }

        // QK over the lane's half of the dims: word (c, wd) holds dims h*D/2 + 4u .. +3 with
        // u = 4c + wd; steps m = 2u + hl use pair c, block 2wd + hl of the half
        float4_t S4[4];
#pragma unroll
        for (int q = 0; q < 4; q++) S4[q] = (float4_t){0.f, 0.f, 0.f, 0.f};
        static_for<0, NK>([&](auto C) {
            static_for<0, 4>([&](auto WD) {
                const uint32_t wv = b.k[C][(int)WD];
                const half4_t B = to_half4(__builtin_amdgcn_perm(0u, wv, 0x0C010C00u),
                                           __builtin_amdgcn_perm(0u, wv, 0x0C030C02u));
                S4[WD] = mfma_h_half<2 * WD>(A8[C], B, S4[WD]);
                S4[WD] = mfma_h_half<2 * WD + 1>(A8[C], B, S4[WD]);
            });
        });
        float4_t S = (S4[0] + S4[1]) + (S4[2] + S4[3]);
#pragma unroll
        for (int i = 0; i < 4; i++) S[i] = add_xor32(S[i]);

        const float sK = f16_bits_to_float(b.sz.x & 0xFFFFu), zK = f16_bits_to_float(b.sz.x >> 16);
        const float sV = f16_bits_to_float(b.sz.y & 0xFFFFu), zV = f16_bits_to_float(b.sz.y >> 16);
        const float sK24 = sK * 16777216.0f;
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; i++) sc[i] = valid ? F[i] * fmaf(S[i], sK24, zK * sumq[i]) : -INFINITY;
        // finite on invalid lanes (unspecified scale bits), so that their ep = sc + lg stays -inf
        const float lg = (valid && sV > 0.f) ? __builtin_amdgcn_logf(sV) : -24.f;
        float pt[4];
        softmax_step(sc, lg, valid, valid ? sV : 0.f, valid ? zV : 0.f, pt);
        exchange_h(pt, sl >> 2, sl & 3, lane_ok, false, Ahi, Alo);
    }

    __device__ __forceinline__ void int8_pv(const Buf& b, const half4_t& Ahi, const half4_t& Alo)
    {
        // v[q * NHV + hv] word w holds slots 16 (q % 2) + 8 (q / 2) + 4 w .. +3 of dim 64 hv + lane:
        // PV step 4 (q % 2) + 2 (q / 2) + w.  Tiles past the range carry zero probabilities.
        static_for<0, 4>([&](auto Q) {
            static_for<0, 2>([&](auto WW) {
                static_for<0, NHV>([&](auto HV) {
                    const uint32_t wv = b.v[Q * NHV + HV][(int)WW];
                    const half4_t B = to_half4(__builtin_amdgcn_perm(0u, wv, 0x0C010C00u),
                                               __builtin_amdgcn_perm(0u, wv, 0x0C030C02u));
                    constexpr int s0 = 4 * (Q % 2) + 2 * (Q / 2) + WW;
                    acc[HV][Q % 2] = mfma_h<s0>(Ahi, B, acc[HV][Q % 2]);
                    acc[HV][Q % 2] = mfma_h<s0>(Alo, B, acc[HV][Q % 2]);
                });
            });
        });
    }

    // arithmetic of step k on buffer b
    __device__ __forceinline__ void compute_qk(const DecodeUnit& U, int k, int p1, const Buf& b, half4_t& Ahi,
                                               half4_t& Alo)
    {
        if (is_int8_step(k))
            int8_qk(U, k, b, Ahi, Alo);
        else
            int4_qk(U, k, p1, b, Ahi, Alo);
    }

    __device__ __forceinline__ void compute_pv(int k, const Buf& b, const half4_t& Ahi, const half4_t& Alo)
    {
        if (is_int8_step(k))
            int8_pv(b, Ahi, Alo);
        else
            int4_pv(b, Ahi, Alo);
    }

    // ---- one unit's steps [k0, k1) (quantized formats): INT8 and INT4 steps in one pipeline ----
    // The wave walks its n steps from a rotation r that a multiplicative hash of the wave index
    // picks (step i of the walk is k0 + (i + r) mod n): waves with equal slices of one long
    // sequence would otherwise stream addresses a fixed stride apart in lock step, which some
    // strides map onto few memory channels.  The online softmax takes the steps in any order.
    __device__ void run_unit(const DecodeUnit& U, int k0, int k1)
    {
        const int p1 = (FMT == FMT_INT4_PROT) ? int4_p1(U.len) : 0;
        const int n = k1 - k0;
        const int r = (int)(((uint32_t)w * 2654435761u >> 8) % (uint32_t)n);
        // walk index i (clamped to the last: the trailing prefetch re-reads cached lines) -> step
        auto at = [&](int i) {
            i = min(i, n - 1) + r;
            return k0 + (i >= n ? i - n : i);
        };
        Ids id = step_ids(U, at(0), p1);
        // query rows of the unit (issued first: the prologue waits for them only): lane l holds
        // 8 bf16 of head l / (D/8), dims 8 (l % (D/8)) .. +7
        const uint16_t* pq = a.q + ((int64_t)U.entry * (a.hkv * G) + U.head * G) * D + 8 * min(lane, QLANES - 1);
        const u32x4 qraw = *(const u32x4*)pq;
        Buf A, B;
        load_step(U, at(0), id, A);
        id = step_ids(U, at(1), p1);
        prologue_q(qraw);
        int i = 0;
        while (true) {
            half4_t Ahi, Alo;
            load_step(U, at(i + 1), id, B);
            compute_qk(U, at(i), p1, A, Ahi, Alo);
            id = step_ids(U, at(i + 2), p1);
            compute_pv(at(i), A, Ahi, Alo);
            if (++i >= n) break;
            load_step(U, at(i + 1), id, A);
            compute_qk(U, at(i), p1, B, Ahi, Alo);
            id = step_ids(U, at(i + 2), p1);
            compute_pv(at(i), B, Ahi, Alo);
            if (++i >= n) break;
        }
    }

    // unit u and the end of its step range, from the argument plan or the uploaded one
    __device__ __forceinline__ void unit_at(int u, DecodeUnit& U, int64_t& ue) const
    {
        if (a.n_arg > 0) {
            arg_unit<FMT>(a, er, n8, u, U, ue);
        } else {
            U = ld_unit(a.units, u);
            ue = (u + 1 < a.n_units) ? ld_uniform(&a.units[u + 1].step_begin) : a.total_steps;
        }
    }

    // Work steps [k0, k1) of unit U inside the wave's slice [s, s_end): the unit's global range
    // [step_begin, ue) opens with kUnitStartSteps steps without work (empty when the slice covers
    // only those).
    __device__ __forceinline__ void unit_slice(const DecodeUnit& U, int64_t ue, int64_t s, int& k0, int& k1) const
    {
        const int64_t wb = U.step_begin + kUnitStartSteps;
        k0 = (int)(s > wb ? s - wb : 0);
        k1 = (int)((s_end < ue ? s_end : ue) - wb);
    }

    // The waves holding a unit's first and last work step (global steps step_begin +
    // kUnitStartSteps and ue - 1, inside this wave's slice [s, s_end) from s on) record
    // themselves: the merge reads the unit's partials w0 + u .. w1 + u.
    __device__ __forceinline__ void mark_unit(const DecodeUnit& U, int64_t ue, int64_t s, int u) const
    {
        const int64_t wb = U.step_begin + kUnitStartSteps;
        if (lane == 0) {
            if (wb >= s && wb < s_end) a.unit_waves[2 * u] = (int32_t)w;
            if (ue - 1 >= s && ue - 1 < s_end) a.unit_waves[2 * u + 1] = (int32_t)w;
        }
    }

    // ---- the wave's steps [s, s_end), starting in unit u (quantized formats) ----
    __device__ void run(int u, int64_t s)
    {
        while (s < s_end) {
            DecodeUnit U;
            int64_t ue;
            unit_at(u, U, ue);
            int k0, k1;
            unit_slice(U, ue, s, k0, k1);
            mark_unit(U, ue, s, u);
            if (k1 > k0) {
                run_unit(U, k0, k1);
                epilogue(w + u);
            }
            s = ue;
            u++;
        }
        wait_vm_all();
    }

    // ================================ BF16 baseline ================================
    // q: lane (4 s + i) holds dims 4m..4m+3 of head i for A step m = 16 v + s, pair v
    __device__ __forceinline__ void prologue_bf16(const DecodeUnit& U)
    {
        reset_state();
        const uint16_t* qrow = a.q + ((int64_t)U.entry * (a.hkv * G) + U.head * G) * D;
        const int s = lane >> 2, i = lane & 3;
        const bool live = i < G;
        const int ic = live ? i : 0;
#pragma unroll
        for (int v = 0; v < NPAIR_BF; v++) {
            const uint32_t* src = (const uint32_t*)(qrow + ic * D + 4 * (16 * v + s));
            const uint32_t lo = src[0], hi = src[1];
            Abf[v] = to_short4(live ? lo : 0u, live ? hi : 0u);
        }
#pragma unroll
        for (int i2 = 0; i2 < 4; i2++) {
            F[i2] = a.scale_log2;
            sumq[i2] = 0.f;
        }
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
        for (int c = 0; c < D / 8; c++) kr[c] = __builtin_nontemporal_load((const u32x4*)(pb + c * 256 + t16 * 16));
        u32x4 vv[NHV][2];
#pragma unroll
        for (int hv = 0; hv < NHV; hv++) {
#pragma unroll
            for (int q = 0; q < 2; q++)
                vv[hv][q] = __builtin_nontemporal_load((const u32x4*)(pb + 32 * D + (64 * hv + lane) * 32 + 16 * q));
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

    // ---- the wave's steps [s, s_end) for the BF16 format (one page per step, no prefetch) ----
    __device__ void run_bf16(int u, int64_t s)
    {
        while (s < s_end) {
            DecodeUnit U;
            int64_t ue;
            unit_at(u, U, ue);
            int k0, k1;
            unit_slice(U, ue, s, k0, k1);
            mark_unit(U, ue, s, u);
            if (k1 > k0) {
                prologue_bf16(U);
                for (int k = k0; k < k1; k++) bf16_step(U, k);
                epilogue(w + u);
            }
            s = ue;
            u++;
        }
    }
};

// The global steps [s, e) of wave w: round 1 (w < n_waves1) shares the first steps1 steps in equal
// slices, round 2 the remaining ones.  Round-2 workgroups come after every round-1 workgroup in
// dispatch order, so the hardware hands them to the compute units that finish round 1 first.
__device__ __forceinline__ void wave_slice(const DecodeArgs& a, int64_t w, int64_t& s, int64_t& e)
{
    if (w < a.n_waves1) {
        s = w * a.steps1 / a.n_waves1;
        e = (w + 1) * a.steps1 / a.n_waves1;
    } else {
        const int64_t j = w - a.n_waves1, W2 = a.n_waves - a.n_waves1, T2 = a.total_steps - a.steps1;
        s = a.steps1 + j * T2 / W2;
        e = a.steps1 + (j + 1) * T2 / W2;
    }
}

template <int D, int G, int FMT>
__global__ __launch_bounds__(64 * kWavesPerBlock) __attribute__((amdgpu_waves_per_eu(2)))
void decode_split_kernel(DecodeArgs a)
{
    __shared__ __align__(16) uint8_t lds_all[kWavesPerBlock][kLdsPerWave];
    __shared__ int lds_simd[kWavesPerBlock], lds_prog[kWavesPerBlock];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // SIMD of this wave (HW_ID bits 5:4); the partner is the other wave of the workgroup on it
    const int simd = __builtin_amdgcn_readfirstlane(((int)__builtin_amdgcn_s_getreg((31 << 11) | 4) >> 4) & 3);
    if (lane == 0) {
        lds_simd[wv] = simd;
        lds_prog[wv] = 0;
    }
    __syncthreads();
    int partner = wv;
#pragma unroll
    for (int i = kWavesPerBlock - 1; i >= 0; i--)
        if (i != wv && lds_simd[i] == simd) partner = i;
    partner = __builtin_amdgcn_readfirstlane(partner);
    const int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + wv;
    if (w >= a.n_waves) return;
    int64_t s, s_end;
    wave_slice(a, w, s, s_end);
    if (s >= s_end) return;
    DecodeWave<D, G, FMT> dw(a, lane, lds_all[wv], lds_all[wv] + kLdsQBytes, w, s_end);
    dw.prog = lds_prog;
    dw.own = wv;
    dw.partner = partner;
    int lo = 0;
    if (a.n_arg > 0) {
        dw.er = load_entries(a, lane);
        lo = arg_first_unit<FMT>(a, dw.er, dw.n8, s);
    } else {
        int hi = a.n_units - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (ld_uniform(&a.units[mid].step_begin) <= s)
                lo = mid;
            else
                hi = mid - 1;
        }
    }
    if constexpr (FMT == FMT_BF16)
        dw.run_bf16(lo, s);
    else
        dw.run(lo, s);
}

// ---------------------------------------------------------------------------------------------
// merge: one wave per (unit, q head) -- lane holds dims lane + 64 j -- combines the unit's partials
// in wave order (log-sum-exp against their common maximum), then applies the inverse rotation
// (H is symmetric: the same FWHT and the fl32(1/sqrt(b)) scale) in registers
// ---------------------------------------------------------------------------------------------

// OUT16: the output rows are bf16 (round to nearest even of the fp32 result) at a.out.
template <int D, int G, int FMT, bool OUT16 = false>
__global__ __launch_bounds__(64 * G) void merge_kernel(DecodeArgs a)
{
    constexpr int NHV = D / 64;
    constexpr bool ROT = FMT != FMT_BF16;
    const int u = blockIdx.x;
    const int i = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    DecodeUnit U;
    if (a.n_arg > 0) {
        const int n8 = (FMT == FMT_INT4_PROT && a.sinks + a.recent > 0)
                           ? (a.sinks + a.recent + kInt8StepSlots - 1) / kInt8StepSlots
                           : 0;
        int64_t ue;
        arg_unit_scalar<FMT>(a, n8, u, U, ue);
    } else {
        U = ld_unit(a.units, u);
    }
    // the first and last wave holding work steps of the unit (after its start charge), as the
    // split kernel recorded them
    const int64_t w0 = ld_uniform(a.unit_waves + 2 * u), w1 = ld_uniform(a.unit_waves + 2 * u + 1);
    const int n = (int)(w1 - w0 + 1);
    // partial j of this unit sits at index w0 + u + j.  Lane j of a round of 64 holds partial
    // j's (m, l): one vector load per round instead of a scalar load (and its wait) per partial.
    const float* ml = a.part_ml + ((w0 + u) * G + i) * 2;
    const float* po = a.part_o + ((w0 + u) * G + i) * D + lane;
    float M = -INFINITY;
    float Ls = 0.f, O[NHV];
#pragma unroll
    for (int hv = 0; hv < NHV; hv++) O[hv] = 0.f;
    // the usual case: every (m, l) and every output row are loaded before any is used (one memory
    // round trip; rows past n repeat the last partial and get weight 0).  Same sums in the same
    // order as the general loop below.  NP = 4, 8 or 16 loads, the fewest that cover n.
    auto fast = [&](auto NPC) {
        constexpr int NP = decltype(NPC)::value;
        const float mj = lane < n ? ml[(int64_t)lane * G * 2] : -INFINITY;
        const float lj = lane < n ? ml[(int64_t)lane * G * 2 + 1] : 0.f;
        float pv[NP][NHV];
#pragma unroll
        for (int k = 0; k < NP; k++)
#pragma unroll
            for (int hv = 0; hv < NHV; hv++) pv[k][hv] = po[(int64_t)(k < n ? k : n - 1) * G * D + 64 * hv];
        M = wave_max_u(mj);
        if (M != -INFINITY) {
            const float fj = (mj == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mj - M);
            Ls = wave_sum_u(fj * lj);
#pragma unroll
            for (int k = 0; k < NP; k++) {
                if (k < n) {
                    const float f = as_float((uint32_t)__builtin_amdgcn_readlane((int)as_uint(fj), k));
#pragma unroll
                    for (int hv = 0; hv < NHV; hv++) O[hv] = fmaf(pv[k][hv], f, O[hv]);
                }
            }
        }
    };
    if (n >= 1 && n <= 16) {
        if (n <= 4)
            fast(std::integral_constant<int, 4>{});
        else if (n <= 8)
            fast(std::integral_constant<int, 8>{});
        else
            fast(std::integral_constant<int, 16>{});
        M = -INFINITY; // the general loop below is skipped
    } else {
        for (int j0 = 0; j0 < n; j0 += 64) {
            const int j = j0 + lane;
            M = fmaxf(M, j < n ? ml[(int64_t)j * G * 2] : -INFINITY);
        }
        M = wave_max_u(M);
    }
    if (M != -INFINITY) {
        for (int j0 = 0; j0 < n; j0 += 64) {
            const int j = j0 + lane;
            const float mj = j < n ? ml[(int64_t)j * G * 2] : -INFINITY;
            const float lj = j < n ? ml[(int64_t)j * G * 2 + 1] : 0.f;
            const float fj = (mj == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mj - M);
            Ls += wave_sum_u(fj * lj);
            // the outputs in partial order, each weight read from its lane; the loads of 16
            // partials are issued before the first of them is used
            const int jn = __builtin_amdgcn_readfirstlane(n - j0 < 64 ? n - j0 : 64);
            for (int jb = 0; jb < jn; jb += 16) {
                float pv[16][NHV];
#pragma unroll
                for (int k = 0; k < 16; k++)
#pragma unroll
                    for (int hv = 0; hv < NHV; hv++)
                        pv[k][hv] = jb + k < jn ? po[(int64_t)(j0 + jb + k) * G * D + 64 * hv] : 0.f;
#pragma unroll
                for (int k = 0; k < 16; k++) {
                    if (jb + k < jn) {
                        const float f = as_float((uint32_t)__builtin_amdgcn_readlane((int)as_uint(fj), jb + k));
#pragma unroll
                        for (int hv = 0; hv < NHV; hv++) O[hv] = fmaf(pv[k][hv], f, O[hv]);
                    }
                }
            }
        }
    }
    float r[NHV];
#pragma unroll
    for (int hv = 0; hv < NHV; hv++) r[hv] = (Ls > 0.f) ? O[hv] / Ls : 0.f;
    if (ROT && a.block > 1) {
        static_for<0, 6>([&](auto S) {
            constexpr int H = 1 << S;
            if (H < a.block) {
                const float sgn = (lane & H) ? -1.f : 1.f;
#pragma unroll
                for (int hv = 0; hv < NHV; hv++) r[hv] = butterfly_xor<H>(r[hv], sgn);
            }
        });
        if constexpr (NHV > 1) {
            if (a.block > 64) {
                const float a0 = r[0], a1 = r[1];
                r[0] = a0 + a1;
                r[1] = a0 - a1;
            }
        }
#pragma unroll
        for (int hv = 0; hv < NHV; hv++) r[hv] = r[hv] * a.cb;
    }
    const int64_t oi = ((int64_t)U.entry * (a.hkv * G) + U.head * G + i) * D + lane;
    if constexpr (OUT16) {
        uint16_t* o = (uint16_t*)a.out + oi;
#pragma unroll
        for (int hv = 0; hv < NHV; hv++) {
            const uint32_t x = as_uint(r[hv]);
            o[64 * hv] = (uint16_t)((x + 0x7FFFu + ((x >> 16) & 1u)) >> 16);
        }
    } else {
        float* o = a.out + oi;
#pragma unroll
        for (int hv = 0; hv < NHV; hv++) o[64 * hv] = r[hv];
    }
}

// ---------------------------------------------------------------------------------------------
// launches
// ---------------------------------------------------------------------------------------------

template <int D, int G, int F>
static hipError_t launch_split_t(const DecodeArgs& a, hipStream_t stream, const KernelTimer& tm)
{
    const unsigned blocks = (unsigned)((a.n_waves + kWavesPerBlock - 1) / kWavesPerBlock);
    return launch_kernel(decode_split_kernel<D, G, F>, dim3(blocks), dim3(64 * kWavesPerBlock), stream, tm, a);
}

template <int D, int G, int F>
static hipError_t launch_merge_t(const DecodeArgs& a, hipStream_t stream, const KernelTimer& tm)
{
    return launch_kernel(merge_kernel<D, G, F>, dim3((unsigned)a.n_units), dim3(64 * G), stream, tm, a);
}

template <int D, int G, int F>
static hipError_t launch_merge16_t(const DecodeArgs& a, hipStream_t stream, const KernelTimer& tm)
{
    return launch_kernel(merge_kernel<D, G, F, true>, dim3((unsigned)a.n_units), dim3(64 * G), stream, tm, a);
}

#define KV4_DEC_DISPATCH(FN)                                                                        \
    if (a.n_units <= 0) return hipSuccess;                                                          \
    if (d == 64 && g == 1 && format == 0) return FN<64, 1, 0>(a, stream, tm);                       \
    if (d == 64 && g == 2 && format == 0) return FN<64, 2, 0>(a, stream, tm);                       \
    if (d == 64 && g == 4 && format == 0) return FN<64, 4, 0>(a, stream, tm);                       \
    if (d == 64 && g == 1 && format == 1) return FN<64, 1, 1>(a, stream, tm);                       \
    if (d == 64 && g == 2 && format == 1) return FN<64, 2, 1>(a, stream, tm);                       \
    if (d == 64 && g == 4 && format == 1) return FN<64, 4, 1>(a, stream, tm);                       \
    if (d == 64 && g == 1 && format == 2) return FN<64, 1, 2>(a, stream, tm);                       \
    if (d == 64 && g == 2 && format == 2) return FN<64, 2, 2>(a, stream, tm);                       \
    if (d == 64 && g == 4 && format == 2) return FN<64, 4, 2>(a, stream, tm);                       \
    if (d == 128 && g == 1 && format == 0) return FN<128, 1, 0>(a, stream, tm);                     \
    if (d == 128 && g == 2 && format == 0) return FN<128, 2, 0>(a, stream, tm);                     \
    if (d == 128 && g == 4 && format == 0) return FN<128, 4, 0>(a, stream, tm);                     \
    if (d == 128 && g == 1 && format == 1) return FN<128, 1, 1>(a, stream, tm);                     \
    if (d == 128 && g == 2 && format == 1) return FN<128, 2, 1>(a, stream, tm);                     \
    if (d == 128 && g == 4 && format == 1) return FN<128, 4, 1>(a, stream, tm);                     \
    if (d == 128 && g == 1 && format == 2) return FN<128, 1, 2>(a, stream, tm);                     \
    if (d == 128 && g == 2 && format == 2) return FN<128, 2, 2>(a, stream, tm);                     \
    if (d == 128 && g == 4 && format == 2) return FN<128, 4, 2>(a, stream, tm);                     \
    return hipErrorInvalidValue;

hipError_t launch_decode_split(int d, int g, int format, const DecodeArgs& a, hipStream_t stream,
                               const KernelTimer& tm)
{
    KV4_DEC_DISPATCH(launch_split_t)
}

template <int D, int G, int F>
static hipError_t residency_t(int* blocks_per_cu)
{
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, decode_split_kernel<D, G, F>,
                                                        64 * kWavesPerBlock, 0);
}

hipError_t decode_split_residency(int d, int g, int format, int* blocks_per_cu)
{
#define KV4_RES_CASE(DD, GG, FF) \
    if (d == DD && g == GG && format == FF) return residency_t<DD, GG, FF>(blocks_per_cu);
    KV4_RES_CASE(64, 1, 0) KV4_RES_CASE(64, 2, 0) KV4_RES_CASE(64, 4, 0)
    KV4_RES_CASE(64, 1, 1) KV4_RES_CASE(64, 2, 1) KV4_RES_CASE(64, 4, 1)
    KV4_RES_CASE(64, 1, 2) KV4_RES_CASE(64, 2, 2) KV4_RES_CASE(64, 4, 2)
    KV4_RES_CASE(128, 1, 0) KV4_RES_CASE(128, 2, 0) KV4_RES_CASE(128, 4, 0)
    KV4_RES_CASE(128, 1, 1) KV4_RES_CASE(128, 2, 1) KV4_RES_CASE(128, 4, 1)
    KV4_RES_CASE(128, 1, 2) KV4_RES_CASE(128, 2, 2) KV4_RES_CASE(128, 4, 2)
#undef KV4_RES_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_decode_merge(int d, int g, int format, const DecodeArgs& a, hipStream_t stream,
                               const KernelTimer& tm)
{
    KV4_DEC_DISPATCH(launch_merge_t)
}

hipError_t launch_decode_merge_bf16(int d, int g, int format, const DecodeArgs& a, hipStream_t stream,
                                    const KernelTimer& tm)
{
    KV4_DEC_DISPATCH(launch_merge16_t)
}

#undef KV4_DEC_DISPATCH

} // namespace kv4
