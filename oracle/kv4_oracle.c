/*
 * kv4_oracle.c -- plain, slow CPU oracle for the INT4 KV cache with block-diagonal Hadamard
 * rotation and INT8 sink/recent protection.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call this file;
 * only the tests, the smoke check and the benchmark's CPU-baseline leg use it.  It shares no
 * code, header, table or constant with the HIP library.
 *
 * What it follows (sources are the pages' own text; none prints formulas, so each step below
 * is the plainest reading of the prose, written out):
 *   - "SAW-INT4: System-Aware 4-Bit KV-Cache Quantization for Real-World LLM Serving",
 *     Abstract: token-wise INT4 quantization after a block-diagonal Hadamard rotation, written
 *     into a paged KV-cache layout; fused attention over that cache.
 *   - "KV4-RL: Unlocking Faster Asynchronous Rollouts for RLVR with INT4 KV Cache Quantization",
 *     Abstract: calibration-free INT4 KV quantization with selective INT8 protection of attention
 *     sinks and recent context; a bounded number of protected positions.
 *   - "KV Cache Quantization" topic page, item 5 (KV4-RL blurb): the full context is stored in
 *     INT4 and only the sinks and recent context are additionally held in INT8.
 *
 * Arithmetic rules: every float step is a single IEEE binary32 operation with round-to-nearest-
 * even (build with -O2 -ffp-contract=off, no fast-math, SSE arithmetic), denormals kept.
 * Attention is evaluated in binary64 on the exactly dequantized values.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* Status values returned by the oracle (its own numbering, independent of the library's). */
enum {
    KV4O_OK = 0,
    KV4O_INVALID_ARGUMENT = 1,
    KV4O_OUT_OF_PAGES = 2,
    KV4O_SEQ_STATE = 3,
    KV4O_PRECONDITION = 7 /* non-finite input or a rotated value outside the fp16 range */
};

/* Storage formats. */
enum { KV4O_FMT_INT4_PROT = 0, KV4O_FMT_INT8 = 1, KV4O_FMT_BF16 = 2 };

/* ------------------------------------------------------------------------------------------ */
/* Scalar definitions                                                                          */
/* ------------------------------------------------------------------------------------------ */

/* bfloat16 is by definition the upper half of a binary32 pattern, so widening is exact. */
static float bf16_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Value of an IEEE binary16 bit pattern (finite patterns only), evaluated from the format's
 * definition: subnormal m * 2^-24, normal (1024 + m) * 2^(e - 25). */
double kv4o_fp16_value(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int e = (bits >> 10) & 0x1f;
    int m = bits & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else
        v = ldexp((double)(1024 + m), e - 25);
    return sign ? -v : v;
}

/* Bit pattern of a value that is exactly representable in binary16 (caller guarantees it). */
static uint16_t fp16_bits_of_exact(double v)
{
    uint16_t sign = 0;
    if (v < 0) {
        sign = 0x8000;
        v = -v;
    }
    if (v == 0)
        return sign;
    if (v < ldexp(1.0, -14)) /* subnormal: integer multiple of 2^-24 */
        return (uint16_t)(sign | (uint16_t)ldexp(v, 24));
    int ex;
    frexp(v, &ex); /* v = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1; /* floor(log2 v) */
    double mant = ldexp(v, -e) - 1.0; /* in [0, 1) */
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)ldexp(mant, 10));
}

/* Spacing of the binary16 grid on the binade that holds |x| (|x| > 0). */
static double fp16_spacing(double ax)
{
    if (ax < ldexp(1.0, -14))
        return ldexp(1.0, -24);
    int ex;
    frexp(ax, &ex);
    return ldexp(1.0, (ex - 1) - 10);
}

/* Largest binary16 value <= x, as a bit pattern; a zero input gives +0.
 * Returns 0 on success, -1 if x lies outside [-65504, 65504] or is not finite. */
int kv4o_fp16_round_down(float xf, uint16_t* out)
{
    double x = (double)xf;
    if (!isfinite(x) || x > 65504.0 || x < -65504.0)
        return -1;
    if (x == 0) {
        *out = 0;
        return 0;
    }
    double ax = fabs(x);
    double q = fp16_spacing(ax);
    double v;
    if (x > 0)
        v = floor(x / q) * q; /* exact: x is binary32 and q a power of two */
    else
        v = -ceil(ax / q) * q; /* may step to the next binade's first value, which is representable */
    if (v == 0) {
        *out = 0;
        return 0;
    }
    *out = fp16_bits_of_exact(v);
    return 0;
}

/* Smallest binary16 value >= x (mirror image of round-down); a zero input gives +0. */
int kv4o_fp16_round_up(float xf, uint16_t* out)
{
    if (xf == 0.0f) {
        *out = 0;
        return 0;
    }
    uint16_t b;
    if (kv4o_fp16_round_down(-xf, &b) != 0)
        return -1;
    if (b == 0) {
        *out = 0;
        return 0;
    }
    *out = (uint16_t)(b ^ 0x8000);
    return 0;
}

/* Round half to even, by definition (no reliance on the current rounding mode). */
static float round_half_even(float u)
{
    float f = floorf(u);
    float d = u - f; /* exact for |u| < 2^23 */
    if (d > 0.5f)
        return f + 1.0f;
    if (d < 0.5f)
        return f;
    return (fmodf(f, 2.0f) == 0.0f) ? f : f + 1.0f;
}

/* ------------------------------------------------------------------------------------------ */
/* Rotation: block-diagonal Hadamard (SAW-INT4, Abstract)                                      */
/* ------------------------------------------------------------------------------------------ */

/* 1/sqrt(b) rounded once to binary32. */
float kv4o_rotation_scale(int b)
{
    return (float)(1.0 / sqrt((double)b));
}

/* In-place rotation of an n-vector: for each block of b consecutive entries, the fast
 * Walsh-Hadamard transform with stages h = 1, 2, 4, ..., b/2 in that order; each stage replaces
 * every pair (i, i+h) (bit h of i clear) by (a + c, a - c) in binary32; after the last stage,
 * each entry is multiplied once by fl32(1/sqrt(b)).  b = 1 leaves the vector unchanged.
 * The resulting map is x -> x * H_bd with H_b[i][k] = (-1)^popcount(i & k) / sqrt(b). */
void kv4o_fwht_f32(float* y, int n, int b)
{
    if (b <= 1)
        return;
    float cb = kv4o_rotation_scale(b);
    for (int j0 = 0; j0 < n; j0 += b) {
        float* blk = y + j0;
        for (int h = 1; h < b; h <<= 1) {
            for (int i0 = 0; i0 < b; i0 += 2 * h) {
                for (int i = i0; i < i0 + h; i++) {
                    float a = blk[i];
                    float c = blk[i + h];
                    blk[i] = a + c;
                    blk[i + h] = a - c;
                }
            }
        }
        for (int i = 0; i < b; i++)
            blk[i] = blk[i] * cb;
    }
}

/* Rotary position embedding of one bf16 key row at one position, rotate-half pairing: for
 * i < n/2 the pair (x_i, x_{i+n/2}) with c = cos_row[i], s = sin_row[i] becomes
 *   (fl32(fl32(x_i c) - fl32(x_{i+n/2} s)),  fl32(fl32(x_{i+n/2} c) + fl32(x_i s))).
 * The tables are the caller's (the pages apply the Hadamard transform to keys after RoPE and
 * leave RoPE itself to the model). */
void kv4o_rope_bf16(const uint16_t* x, int n, const float* cos_row, const float* sin_row, float* out)
{
    int half = n / 2;
    for (int i = 0; i < half; i++) {
        float a = bf16_to_float(x[i]), b = bf16_to_float(x[i + half]);
        float c = cos_row[i], s = sin_row[i];
        float ac = a * c, bs = b * s, bc = b * c, as = a * s;
        out[i] = ac - bs;
        out[i + half] = bc + as;
    }
}

/* bf16 row -> rotated binary32 row. */
void kv4o_rotate_bf16(const uint16_t* x, int n, int b, float* y)
{
    for (int i = 0; i < n; i++)
        y[i] = bf16_to_float(x[i]);
    kv4o_fwht_f32(y, n, b);
}

/* ------------------------------------------------------------------------------------------ */
/* Token-wise asymmetric quantization (SAW-INT4 Abstract; KV4-RL Abstract: calibration-free)    */
/* ------------------------------------------------------------------------------------------ */

/* One group = one token's rotated n-vector for one kv head (K and V separately).
 *   mn, mx     = exact min / max of the group
 *   z          = fp16 round-down of mn          (zero offset, a real value: x^ = s*code + z)
 *   r          = fl32(mx - z)
 *   t          = fl32(r / Q)                     (correctly rounded division)
 *   s          = fp16 round-up of t
 *   s == 0     -> every code is 0
 *   otherwise  inv = fl32(1 / s), u = fl32(fl32(y - z) * inv), code = clamp(rne(u), 0, Q)
 * Q = 15 for INT4, 255 for INT8.  Returns 0, or -1 on a precondition violation. */
int kv4o_quantize(const float* y, int n, int Q, uint8_t* codes, uint16_t* s_bits, uint16_t* z_bits)
{
    float mn = y[0], mx = y[0];
    for (int i = 0; i < n; i++) {
        if (!isfinite(y[i]))
            return -1;
        if (y[i] < mn)
            mn = y[i];
        if (y[i] > mx)
            mx = y[i];
    }
    uint16_t zb, sb;
    if (kv4o_fp16_round_down(mn, &zb) != 0 || mx > 65504.0f)
        return -1;
    float zf = (float)kv4o_fp16_value(zb);
    float r = mx - zf;
    float t = r / (float)Q;
    if (kv4o_fp16_round_up(t, &sb) != 0)
        return -1;
    float sf = (float)kv4o_fp16_value(sb);
    *s_bits = sb;
    *z_bits = zb;
    if (sf == 0.0f) {
        for (int i = 0; i < n; i++)
            codes[i] = 0;
        return 0;
    }
    float inv = 1.0f / sf;
    for (int i = 0; i < n; i++) {
        float diff = y[i] - zf;
        float u = diff * inv;
        float c = round_half_even(u);
        if (c < 0.0f)
            c = 0.0f;
        if (c > (float)Q)
            c = (float)Q;
        codes[i] = (uint8_t)c;
    }
    return 0;
}

/* Exact dequantized value s*code + z (binary64 holds it exactly: both terms are integer
 * multiples of 2^-24 below 2^25 in magnitude). */
static double dequant(uint8_t code, uint16_t s_bits, uint16_t z_bits)
{
    return kv4o_fp16_value(s_bits) * (double)code + kv4o_fp16_value(z_bits);
}

/* Nibble packing of INT4 codes: byte k = code[2k] | code[2k+1] << 4. */
void kv4o_pack_int4(const uint8_t* codes, int n, uint8_t* out)
{
    for (int k = 0; k < n / 2; k++)
        out[k] = (uint8_t)((codes[2 * k] & 0xf) | ((codes[2 * k + 1] & 0xf) << 4));
}

/* ------------------------------------------------------------------------------------------ */
/* Protected set (KV4-RL Abstract; topic page item 5)                                          */
/* ------------------------------------------------------------------------------------------ */

/* Prot(L) = {t < min(S, L)} u {max(S, L - R) <= t < L}. */
int kv4o_is_protected(int t, int L, int S, int R)
{
    if (t < 0 || t >= L)
        return 0;
    if (t < S)
        return 1;
    int lo = L - R;
    if (lo < S)
        lo = S;
    return t >= lo;
}

/* INT8 slot of a protected position: sinks first (slot t for t < S), then a ring of R slots
 * (slot S + t mod R). */
int kv4o_int8_slot(int t, int S, int R)
{
    if (t < S)
        return t;
    return S + (t % R);
}

/* ------------------------------------------------------------------------------------------ */
/* Cache model: FIFO page allocator, block tables, INT4 pages, INT8 sink/ring slots             */
/* ------------------------------------------------------------------------------------------ */

typedef struct kv4o_cache {
    int hq, hkv, d, P, num_pages, max_seqs, max_pps, S, R, b, fmt;
    int requant; /* eviction rule: 0 dual write, 1 INT4 codes from the INT8 round trip */
    int* len;  /* [max_seqs] */
    int* bt;   /* [max_seqs][max_pps] */
    int* fifo; /* circular free list of capacity num_pages */
    int fifo_head, fifo_count;
    /* per token-slot storage, one code per byte (logical, unpacked), indexed by
     * (page, head, slot-in-page, kv) with kv 0 = K, 1 = V */
    uint8_t* codes;  /* [num_pages][hkv][P][2][d] : INT4 codes (fmt 0) or INT8 codes (fmt 1) */
    uint16_t* sz;    /* [num_pages][hkv][P][2][2] : (s, z) fp16 bits */
    uint16_t* bf;    /* [num_pages][hkv][P][2][d] : bf16 bits (fmt 2) */
    uint8_t* filled; /* [num_pages][P] : 1 once the slot holds a token's data */
    /* INT8 protection slots (fmt 0 only) */
    uint8_t* c8;  /* [max_seqs][hkv][S+R][2][d] */
    uint16_t* s8; /* [max_seqs][hkv][S+R][2][2] */
    int* tok8;    /* [max_seqs][S+R] : token currently held by the slot, -1 if none */
} kv4o_cache;

static size_t page_idx(const kv4o_cache* c, int page, int h, int slot, int kv)
{
    return ((((size_t)page * c->hkv + h) * c->P + slot) * 2 + kv);
}

static size_t seg_idx(const kv4o_cache* c, int seq, int h, int slot, int kv)
{
    return ((((size_t)seq * c->hkv + h) * (c->S + c->R) + slot) * 2 + kv);
}

void kv4o_destroy(kv4o_cache* c)
{
    if (!c)
        return;
    free(c->len);
    free(c->bt);
    free(c->fifo);
    free(c->codes);
    free(c->sz);
    free(c->bf);
    free(c->filled);
    free(c->c8);
    free(c->s8);
    free(c->tok8);
    free(c);
}

/* Returns NULL on an invalid configuration or allocation failure. */
kv4o_cache* kv4o_create(int hq, int hkv, int d, int P, int num_pages, int max_seqs, int max_pps, int S, int R,
                        int b, int fmt)
{
    if (hq <= 0 || hkv <= 0 || hq % hkv || d <= 0 || d % 2 || P <= 0 || num_pages < 0 || max_seqs <= 0 ||
        max_pps <= 0 || S < 0 || R < 0 || b <= 0 || (b & (b - 1)) || d % b || fmt < 0 || fmt > 2)
        return NULL;
    kv4o_cache* c = (kv4o_cache*)calloc(1, sizeof *c);
    if (!c)
        return NULL;
    c->hq = hq;
    c->hkv = hkv;
    c->d = d;
    c->P = P;
    c->num_pages = num_pages;
    c->max_seqs = max_seqs;
    c->max_pps = max_pps;
    c->S = S;
    c->R = R;
    c->b = b;
    c->fmt = fmt;
    c->len = (int*)calloc((size_t)max_seqs, sizeof(int));
    c->bt = (int*)malloc((size_t)max_seqs * max_pps * sizeof(int));
    c->fifo = (int*)malloc(((size_t)num_pages + 1) * sizeof(int));
    size_t slots = (size_t)num_pages * hkv * P * 2;
    c->filled = (uint8_t*)calloc((size_t)num_pages * P + 1, 1);
    if (fmt == KV4O_FMT_BF16) {
        c->bf = (uint16_t*)calloc(slots * d + 1, sizeof(uint16_t));
    } else {
        c->codes = (uint8_t*)calloc(slots * d + 1, 1);
        c->sz = (uint16_t*)calloc(slots * 2 + 1, sizeof(uint16_t));
    }
    size_t nseg = (size_t)max_seqs * hkv * (S + R) * 2;
    if (fmt == KV4O_FMT_INT4_PROT) {
        c->c8 = (uint8_t*)calloc(nseg * d + 1, 1);
        c->s8 = (uint16_t*)calloc(nseg * 2 + 1, sizeof(uint16_t));
        c->tok8 = (int*)malloc(((size_t)max_seqs * (S + R) + 1) * sizeof(int));
    }
    if (!c->len || !c->bt || !c->fifo || !c->filled || (fmt == KV4O_FMT_BF16 ? !c->bf : (!c->codes || !c->sz)) ||
        (fmt == KV4O_FMT_INT4_PROT && (!c->c8 || !c->s8 || !c->tok8))) {
        kv4o_destroy(c);
        return NULL;
    }
    for (size_t i = 0; i < (size_t)max_seqs * max_pps; i++)
        c->bt[i] = -1;
    if (c->tok8)
        for (size_t i = 0; i < (size_t)max_seqs * (S + R); i++)
            c->tok8[i] = -1;
    /* the free list starts as 0, 1, ..., num_pages - 1 */
    for (int i = 0; i < num_pages; i++)
        c->fifo[i] = i;
    c->fifo_head = 0;
    c->fifo_count = num_pages;
    return c;
}

/* Selects the INT8 -> INT4 eviction rule (INT4_PROT only; before the first append).
 *   0: dual write -- a position's INT4 code is quantized from its rotated values when appended.
 *   1: re-quantization -- a position that leaves the recent window moves from INT8 to INT4 by
 *      quantizing its INT8 copy's dequantized row ([KV4]: tokens leaving the window move from
 *      INT8 to INT4).  That row depends on the position alone, so the INT4 code is computed when
 *      the position is appended (for every position, so that a prefill equals single appends). */
int kv4o_set_eviction(kv4o_cache* c, int mode)
{
    if (mode < 0 || mode > 1 || (mode == 1 && c->fmt != KV4O_FMT_INT4_PROT))
        return KV4O_INVALID_ARGUMENT;
    for (int i = 0; i < c->max_seqs; i++)
        if (c->len[i] != 0)
            return KV4O_SEQ_STATE;
    c->requant = mode;
    return KV4O_OK;
}

static int fifo_pop(kv4o_cache* c)
{
    int p = c->fifo[c->fifo_head];
    c->fifo_head = (c->fifo_head + 1) % c->num_pages;
    c->fifo_count--;
    return p;
}

static void fifo_push(kv4o_cache* c, int page)
{
    int tail = (c->fifo_head + c->fifo_count) % c->num_pages;
    c->fifo[tail] = page;
    c->fifo_count++;
}

int kv4o_free_pages(const kv4o_cache* c) { return c->fifo_count; }

int kv4o_seq_length(const kv4o_cache* c, int seq)
{
    if (seq < 0 || seq >= c->max_seqs)
        return -1;
    return c->len[seq];
}

/* Copies the sequence's block table (ceil(L/P) entries) into pages; returns the count or -1. */
int kv4o_block_table(const kv4o_cache* c, int seq, int* pages, int cap)
{
    if (seq < 0 || seq >= c->max_seqs)
        return -1;
    int n = (c->len[seq] + c->P - 1) / c->P;
    for (int j = 0; j < n && j < cap; j++)
        pages[j] = c->bt[(size_t)seq * c->max_pps + j];
    return n;
}

/* Releases a sequence: its pages go to the back of the free list in block-table order and its
 * length becomes 0. */
int kv4o_seq_free(kv4o_cache* c, int seq)
{
    if (seq < 0 || seq >= c->max_seqs)
        return KV4O_INVALID_ARGUMENT;
    int n = (c->len[seq] + c->P - 1) / c->P;
    for (int j = 0; j < n; j++) {
        int p = c->bt[(size_t)seq * c->max_pps + j];
        for (int s = 0; s < c->P; s++)
            c->filled[(size_t)p * c->P + s] = 0;
        fifo_push(c, p);
        c->bt[(size_t)seq * c->max_pps + j] = -1;
    }
    if (c->tok8)
        for (int u = 0; u < c->S + c->R; u++)
            c->tok8[(size_t)seq * (c->S + c->R) + u] = -1;
    c->len[seq] = 0;
    return KV4O_OK;
}

/* Writes one token (all heads, K and V) at position t of seq; L_new is the length after the
 * call, which decides INT8 protection.  k, v: [hkv][d] bf16 bits, or NULL (allocation only).
 * rope_cos / rope_sin: NULL, or this position's table rows [d/2]: the key rows then get RoPE
 * (kv4o_rope_bf16) before the Hadamard rotation. */
static int write_token(kv4o_cache* c, int seq, int t, int L_new, const uint16_t* k, const uint16_t* v,
                       const float* rope_cos, const float* rope_sin)
{
    int page = c->bt[(size_t)seq * c->max_pps + t / c->P];
    int slot = t % c->P;
    if (!k || !v)
        return KV4O_OK;
    float* y = (float*)malloc((size_t)c->d * 2 * sizeof(float));
    uint8_t* c8row = (uint8_t*)malloc((size_t)c->d);
    if (!y || !c8row) {
        free(y);
        free(c8row);
        return KV4O_INVALID_ARGUMENT;
    }
    float* x8 = y + c->d;
    int rc = KV4O_OK;
    for (int h = 0; h < c->hkv && rc == KV4O_OK; h++) {
        for (int kv = 0; kv < 2 && rc == KV4O_OK; kv++) {
            const uint16_t* x = (kv == 0 ? k : v) + (size_t)h * c->d;
            size_t pi = page_idx(c, page, h, slot, kv);
            if (c->fmt == KV4O_FMT_BF16) {
                memcpy(c->bf + pi * c->d, x, (size_t)c->d * sizeof(uint16_t));
                continue;
            }
            if (kv == 0 && rope_cos) {
                kv4o_rope_bf16(x, c->d, rope_cos, rope_sin, y);
                kv4o_fwht_f32(y, c->d, c->b);
            } else {
                kv4o_rotate_bf16(x, c->d, c->b, y);
            }
            int Q = (c->fmt == KV4O_FMT_INT8) ? 255 : 15;
            if (c->requant) {
                /* INT4 from the INT8 round trip: x8 = fl32(s8 * code8 + z8) (the product is exact) */
                uint16_t s8b, z8b;
                if (kv4o_quantize(y, c->d, 255, c8row, &s8b, &z8b) != 0) {
                    rc = KV4O_PRECONDITION;
                    break;
                }
                float s8f = (float)kv4o_fp16_value(s8b), z8f = (float)kv4o_fp16_value(z8b);
                for (int i = 0; i < c->d; i++) {
                    float prod = s8f * (float)c8row[i];
                    x8[i] = prod + z8f;
                }
                if (kv4o_quantize(x8, c->d, 15, c->codes + pi * c->d, &c->sz[pi * 2], &c->sz[pi * 2 + 1]) != 0) {
                    rc = KV4O_PRECONDITION;
                    break;
                }
            } else if (kv4o_quantize(y, c->d, Q, c->codes + pi * c->d, &c->sz[pi * 2], &c->sz[pi * 2 + 1]) != 0) {
                rc = KV4O_PRECONDITION;
                break;
            }
            if (c->fmt == KV4O_FMT_INT4_PROT && kv4o_is_protected(t, L_new, c->S, c->R)) {
                int u = kv4o_int8_slot(t, c->S, c->R);
                size_t si = seg_idx(c, seq, h, u, kv);
                if (kv4o_quantize(y, c->d, 255, c->c8 + si * c->d, &c->s8[si * 2], &c->s8[si * 2 + 1]) != 0) {
                    rc = KV4O_PRECONDITION;
                    break;
                }
                c->tok8[(size_t)seq * (c->S + c->R) + u] = t;
            }
        }
    }
    free(y);
    free(c8row);
    if (rc == KV4O_OK)
        c->filled[(size_t)page * c->P + slot] = 1;
    return rc;
}

static int append_rows(kv4o_cache* c, int n_seqs, const int* seq_ids, const int* n_new, const uint16_t* k_new,
                       const uint16_t* v_new, const float* rope_cos, const float* rope_sin, int rope_positions);

/* Appends n_new[i] tokens to seq_ids[i], for i in call order.  Rows of k_new / v_new are ordered
 * by (call order, ascending position), each row [hkv][d] bf16.  All-or-nothing on page
 * shortage: if the free list cannot cover every new page of the call, nothing changes. */
int kv4o_append(kv4o_cache* c, int n_seqs, const int* seq_ids, const int* n_new, const uint16_t* k_new,
                const uint16_t* v_new)
{
    return append_rows(c, n_seqs, seq_ids, n_new, k_new, v_new, NULL, NULL, 0);
}

/* The same with pre-RoPE keys: the key row of position t gets RoPE with table rows
 * rope_cos[t], rope_sin[t] ([rope_positions][d/2] binary32) before the Hadamard rotation.  Every
 * new position must be < rope_positions.  The RoPE output is not rounded to bf16: the cache
 * stores the rotation of the binary32 RoPE output. */
int kv4o_append_rope(kv4o_cache* c, int n_seqs, const int* seq_ids, const int* n_new, const uint16_t* k_new,
                     const uint16_t* v_new, const float* rope_cos, const float* rope_sin, int rope_positions)
{
    if (!rope_cos || !rope_sin || rope_positions < 0)
        return KV4O_INVALID_ARGUMENT;
    return append_rows(c, n_seqs, seq_ids, n_new, k_new, v_new, rope_cos, rope_sin, rope_positions);
}

static int append_rows(kv4o_cache* c, int n_seqs, const int* seq_ids, const int* n_new, const uint16_t* k_new,
                       const uint16_t* v_new, const float* rope_cos, const float* rope_sin, int rope_positions)
{
    if (n_seqs < 0)
        return KV4O_INVALID_ARGUMENT;
    long needed = 0;
    for (int i = 0; i < n_seqs; i++) {
        int s = seq_ids[i];
        if (s < 0 || s >= c->max_seqs || n_new[i] < 0)
            return KV4O_INVALID_ARGUMENT;
        for (int j = 0; j < i; j++)
            if (seq_ids[j] == s)
                return KV4O_INVALID_ARGUMENT;
        long L0 = c->len[s], L1 = L0 + n_new[i];
        if (L1 > (long)c->max_pps * c->P)
            return KV4O_SEQ_STATE;
        if (rope_cos && L1 > rope_positions)
            return KV4O_INVALID_ARGUMENT;
        needed += (L1 + c->P - 1) / c->P - (L0 + c->P - 1) / c->P;
    }
    if (needed > c->fifo_count)
        return KV4O_OUT_OF_PAGES;
    size_t row = 0;
    size_t row_elems = (size_t)c->hkv * c->d;
    for (int i = 0; i < n_seqs; i++) {
        int s = seq_ids[i];
        int L0 = c->len[s], L1 = L0 + n_new[i];
        for (int t = L0; t < L1; t++, row++) {
            if (t % c->P == 0)
                c->bt[(size_t)s * c->max_pps + t / c->P] = fifo_pop(c);
            size_t half = (size_t)c->d / 2;
            int rc = write_token(c, s, t, L1, k_new ? k_new + row * row_elems : NULL,
                                 v_new ? v_new + row * row_elems : NULL, rope_cos ? rope_cos + (size_t)t * half : NULL,
                                 rope_sin ? rope_sin + (size_t)t * half : NULL);
            if (rc != KV4O_OK)
                return rc;
        }
        c->len[s] = L1;
    }
    return KV4O_OK;
}

/* Logical contents of a page slot: codes [d], (s, z) bits; bf16 format returns the bits in
 * bf_out instead.  Returns 0, or -1 if the position is not stored. */
int kv4o_get_page_token(const kv4o_cache* c, int seq, int t, int h, int kv, uint8_t* codes, uint16_t* sz,
                        uint16_t* bf_out, int* page_out)
{
    if (seq < 0 || seq >= c->max_seqs || t < 0 || t >= c->len[seq] || h < 0 || h >= c->hkv || kv < 0 || kv > 1)
        return -1;
    int page = c->bt[(size_t)seq * c->max_pps + t / c->P];
    int slot = t % c->P;
    if (!c->filled[(size_t)page * c->P + slot])
        return -1;
    size_t pi = page_idx(c, page, h, slot, kv);
    if (page_out)
        *page_out = page;
    if (c->fmt == KV4O_FMT_BF16) {
        if (bf_out)
            memcpy(bf_out, c->bf + pi * c->d, (size_t)c->d * sizeof(uint16_t));
        return 0;
    }
    if (codes)
        memcpy(codes, c->codes + pi * c->d, (size_t)c->d);
    if (sz) {
        sz[0] = c->sz[pi * 2];
        sz[1] = c->sz[pi * 2 + 1];
    }
    return 0;
}

/* Logical contents of a whole page for kv head h: codes [P][2][d] (or bf16 bits [P][2][d] for the
 * bf16 format, in bf_out), scales [P][2][2], filled [P].  Returns 0, or -1 on a bad index. */
int kv4o_get_page(const kv4o_cache* c, int page, int h, uint8_t* codes, uint16_t* sz, uint16_t* bf_out,
                  uint8_t* filled)
{
    if (page < 0 || page >= c->num_pages || h < 0 || h >= c->hkv)
        return -1;
    size_t p0 = page_idx(c, page, h, 0, 0);
    size_t n = (size_t)c->P * 2;
    if (c->fmt == KV4O_FMT_BF16) {
        if (bf_out)
            memcpy(bf_out, c->bf + p0 * c->d, n * c->d * sizeof(uint16_t));
    } else {
        if (codes)
            memcpy(codes, c->codes + p0 * c->d, n * c->d);
        if (sz)
            memcpy(sz, c->sz + p0 * 2, n * 2 * sizeof(uint16_t));
    }
    if (filled)
        memcpy(filled, c->filled + (size_t)page * c->P, (size_t)c->P);
    return 0;
}

/* Logical contents of INT8 slot u of (seq, h, kv); token_out gets the token held (-1: none). */
int kv4o_get_int8_slot(const kv4o_cache* c, int seq, int u, int h, int kv, uint8_t* codes, uint16_t* sz,
                       int* token_out)
{
    if (c->fmt != KV4O_FMT_INT4_PROT || seq < 0 || seq >= c->max_seqs || u < 0 || u >= c->S + c->R || h < 0 ||
        h >= c->hkv || kv < 0 || kv > 1)
        return -1;
    size_t si = seg_idx(c, seq, h, u, kv);
    if (codes)
        memcpy(codes, c->c8 + si * c->d, (size_t)c->d);
    if (sz) {
        sz[0] = c->s8[si * 2];
        sz[1] = c->s8[si * 2 + 1];
    }
    if (token_out)
        *token_out = c->tok8[(size_t)seq * (c->S + c->R) + u];
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Decode attention (binary64)                                                                 */
/* ------------------------------------------------------------------------------------------ */

/* Exact block-diagonal Hadamard applied to a binary64 row: out = x * H_bd (H is symmetric, so
 * this is also x * H_bd^T).  Written as the plain matrix-vector product. */
static void hadamard_f64(const double* x, int n, int b, double* out)
{
    double sc = 1.0 / sqrt((double)b);
    for (int j0 = 0; j0 < n; j0 += b) {
        for (int k = 0; k < b; k++) {
            double acc = 0.0;
            for (int i = 0; i < b; i++) {
                double sgn = (__builtin_popcount((unsigned)(i & k)) & 1) ? -1.0 : 1.0;
                acc += x[j0 + i] * sgn;
            }
            out[j0 + k] = acc * sc;
        }
    }
}

/* Dequantized K and V rows (rotated domain for the quantized formats, raw bf16 values for the
 * bf16 format) that decode reads for position t of seq at length L: the INT8 slot when t is in
 * Prot(L) (INT4_PROT format), otherwise the page copy. */
static int fetch_kv(const kv4o_cache* c, int seq, int t, int L, int h, double* kout, double* vout)
{
    int d = c->d;
    if (c->fmt == KV4O_FMT_INT4_PROT && kv4o_is_protected(t, L, c->S, c->R)) {
        int u = kv4o_int8_slot(t, c->S, c->R);
        if (c->tok8[(size_t)seq * (c->S + c->R) + u] != t)
            return -1;
        for (int kv = 0; kv < 2; kv++) {
            size_t si = seg_idx(c, seq, h, u, kv);
            double* o = kv ? vout : kout;
            for (int i = 0; i < d; i++)
                o[i] = dequant(c->c8[si * d + i], c->s8[si * 2], c->s8[si * 2 + 1]);
        }
        return 0;
    }
    int page = c->bt[(size_t)seq * c->max_pps + t / c->P];
    int slot = t % c->P;
    if (page < 0 || !c->filled[(size_t)page * c->P + slot])
        return -1;
    for (int kv = 0; kv < 2; kv++) {
        size_t pi = page_idx(c, page, h, slot, kv);
        double* o = kv ? vout : kout;
        if (c->fmt == KV4O_FMT_BF16) {
            for (int i = 0; i < d; i++)
                o[i] = (double)bf16_to_float(c->bf[pi * d + i]);
        } else {
            for (int i = 0; i < d; i++)
                o[i] = dequant(c->codes[pi * d + i], c->sz[pi * 2], c->sz[pi * 2 + 1]);
        }
    }
    return 0;
}

/* All L dequantized rows of (seq, h): k_out, v_out [L][d] binary64. */
int kv4o_dequant_seq(const kv4o_cache* c, int seq, int h, double* k_out, double* v_out)
{
    if (seq < 0 || seq >= c->max_seqs || h < 0 || h >= c->hkv)
        return KV4O_INVALID_ARGUMENT;
    int L = c->len[seq];
    for (int t = 0; t < L; t++)
        if (fetch_kv(c, seq, t, L, h, k_out + (size_t)t * c->d, v_out + (size_t)t * c->d) != 0)
            return KV4O_SEQ_STATE;
    return KV4O_OK;
}

/* One (sequence, kv head) unit: the G query heads that share kv head h (query head g reads kv
 * head g / G), for nq query rows.  Query row r sits at position p = L - nq + r of the sequence
 * (length L) and attends positions 0 .. p; every position is read from the copy that decode
 * reads at length L (the INT8 slot when it is in Prot(L), else its page).  nq = 1 is decode
 * attention over all L positions.  q: [nq][hq][d] bf16 bits of this sequence; out: [nq][hq][d]
 * binary64. */
static int attend_unit(const kv4o_cache* c, int seq, int h, int nq, const uint16_t* q, double scale, double* out)
{
    int d = c->d, G = c->hq / c->hkv, L = c->len[seq];
    int rotated = (c->fmt != KV4O_FMT_BF16);
    double* kb = (double*)malloc((size_t)L * d * sizeof(double));
    double* vb = (double*)malloc((size_t)L * d * sizeof(double));
    double* e = (double*)malloc((size_t)L * sizeof(double));
    double* qr = (double*)malloc((size_t)d * 3 * sizeof(double));
    if (!kb || !vb || !e || !qr) {
        free(kb);
        free(vb);
        free(e);
        free(qr);
        return KV4O_INVALID_ARGUMENT;
    }
    int rc = kv4o_dequant_seq(c, seq, h, kb, vb);
    for (int r = 0; r < nq && rc == KV4O_OK; r++) {
        int n = L - nq + r + 1; /* positions attended by row r */
        for (int gi = 0; gi < G; gi++) {
            int g = h * G + gi;
            const uint16_t* qrow = q + ((size_t)r * c->hq + g) * d;
            double* orow = out + ((size_t)r * c->hq + g) * d;
            double* qd = qr;
            double* qrot = qr + d;
            double* o = qr + 2 * d;
            for (int i = 0; i < d; i++)
                qd[i] = (double)bf16_to_float(qrow[i]);
            if (rotated)
                hadamard_f64(qd, d, c->b, qrot);
            else
                memcpy(qrot, qd, (size_t)d * sizeof(double));
            double m = -INFINITY;
            for (int t = 0; t < n; t++) {
                double acc = 0.0;
                for (int i = 0; i < d; i++)
                    acc += qrot[i] * kb[(size_t)t * d + i];
                e[t] = scale * acc;
                if (e[t] > m)
                    m = e[t];
            }
            double l = 0.0;
            for (int t = 0; t < n; t++) {
                e[t] = exp(e[t] - m);
                l += e[t];
            }
            for (int i = 0; i < d; i++) {
                double acc = 0.0;
                for (int t = 0; t < n; t++)
                    acc += e[t] * vb[(size_t)t * d + i];
                o[i] = acc / l;
            }
            if (rotated)
                hadamard_f64(o, d, c->b, orow);
            else
                memcpy(orow, o, (size_t)d * sizeof(double));
        }
    }
    free(kb);
    free(vb);
    free(e);
    free(qr);
    return rc;
}

typedef struct {
    const kv4o_cache* c;
    int n_seqs;
    const int* seq_ids;
    const int* n_q;     /* query rows per sequence (NULL: one each) */
    const size_t* row0; /* first query row of each sequence */
    const uint16_t* q;
    double scale;
    double* out;
    int next; /* shared work counter, guarded by lock */
    int rc;
    pthread_mutex_t lock;
} decode_job;

static void* decode_worker(void* arg)
{
    decode_job* job = (decode_job*)arg;
    const kv4o_cache* c = job->c;
    size_t per_seq = (size_t)c->hq * c->d;
    for (;;) {
        pthread_mutex_lock(&job->lock);
        int w = job->next++;
        pthread_mutex_unlock(&job->lock);
        if (w >= job->n_seqs * c->hkv)
            break;
        int i = w / c->hkv, h = w % c->hkv;
        int nq = job->n_q ? job->n_q[i] : 1;
        size_t r0 = job->row0 ? job->row0[i] : (size_t)i;
        int rc = attend_unit(c, job->seq_ids[i], h, nq, job->q + r0 * per_seq, job->scale, job->out + r0 * per_seq);
        if (rc != KV4O_OK) {
            pthread_mutex_lock(&job->lock);
            job->rc = rc;
            pthread_mutex_unlock(&job->lock);
        }
    }
    return NULL;
}

static int run_attend(const kv4o_cache* c, int n_seqs, const int* seq_ids, const int* n_q, const uint16_t* q,
                      double scale, double* out, int n_threads, int* threads_used)
{
    if (n_seqs < 0)
        return KV4O_INVALID_ARGUMENT;
    size_t* row0 = (size_t*)malloc(((size_t)n_seqs + 1) * sizeof(size_t));
    if (!row0)
        return KV4O_INVALID_ARGUMENT;
    row0[0] = 0;
    for (int i = 0; i < n_seqs; i++) {
        int s = seq_ids[i];
        int nq = n_q ? n_q[i] : 1;
        if (s < 0 || s >= c->max_seqs || nq < 1) {
            free(row0);
            return KV4O_INVALID_ARGUMENT;
        }
        for (int j = 0; j < i; j++)
            if (seq_ids[j] == s) {
                free(row0);
                return KV4O_INVALID_ARGUMENT;
            }
        if (c->len[s] < nq) {
            free(row0);
            return KV4O_SEQ_STATE;
        }
        row0[i + 1] = row0[i] + (size_t)nq;
    }
    if (scale <= 0)
        scale = 1.0 / sqrt((double)c->d);
    if (n_threads <= 0)
        n_threads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (n_threads < 1)
        n_threads = 1;
    if (n_threads > n_seqs * c->hkv)
        n_threads = n_seqs * c->hkv > 0 ? n_seqs * c->hkv : 1;
    decode_job job;
    job.c = c;
    job.n_seqs = n_seqs;
    job.seq_ids = seq_ids;
    job.n_q = n_q;
    job.row0 = row0;
    job.q = q;
    job.scale = scale;
    job.out = out;
    job.next = 0;
    job.rc = KV4O_OK;
    pthread_mutex_init(&job.lock, NULL);
    pthread_t* th = (pthread_t*)malloc((size_t)n_threads * sizeof(pthread_t));
    int started = 0;
    for (int i = 1; th && i < n_threads; i++)
        if (pthread_create(&th[started], NULL, decode_worker, &job) == 0)
            started++;
    decode_worker(&job);
    for (int i = 0; i < started; i++)
        pthread_join(th[i], NULL);
    free(th);
    free(row0);
    pthread_mutex_destroy(&job.lock);
    if (threads_used)
        *threads_used = started + 1;
    return job.rc;
}

/* Decode attention for a batch: q [n_seqs][hq][d] bf16 bits, out [n_seqs][hq][d] binary64.
 * scale <= 0 selects 1/sqrt(d).  Every listed sequence must have length >= 1.  Work is spread
 * over n_threads threads (0: all online processors); *threads_used reports the count. */
int kv4o_decode(const kv4o_cache* c, int n_seqs, const int* seq_ids, const uint16_t* q, double scale, double* out,
                int n_threads, int* threads_used)
{
    return run_attend(c, n_seqs, seq_ids, NULL, q, scale, out, n_threads, threads_used);
}

/* Causal attention of several query rows per sequence over the cache as it stands: the n_q[i]
 * rows of sequence seq_ids[i] (length L, 1 <= n_q[i] <= L) sit at positions L - n_q[i] .. L - 1
 * and row r attends positions 0 .. L - n_q[i] + r, each read from the copy decode reads at
 * length L.  q: [sum n_q][hq][d] bf16 bits, rows of a sequence consecutive, sequences in call
 * order; out: the same shape, binary64. */
int kv4o_attend_multi(const kv4o_cache* c, int n_seqs, const int* seq_ids, const int* n_q, const uint16_t* q,
                      double scale, double* out, int n_threads, int* threads_used)
{
    return run_attend(c, n_seqs, seq_ids, n_q, q, scale, out, n_threads, threads_used);
}
