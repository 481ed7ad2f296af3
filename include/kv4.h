/*
 * kv4.h -- C ABI of libkv4: a paged KV cache stored as token-wise asymmetric INT4 of
 * block-Hadamard-rotated keys and values, with attention-sink and recent-window positions also
 * held in INT8, plus GQA decode attention over it.  Hand-written HIP kernels for gfx950.
 *
 * Sources (the pages describe the method in prose only):
 *   [SAW]  "SAW-INT4: System-Aware 4-Bit KV-Cache Quantization for Real-World LLM Serving",
 *          Abstract -- token-wise INT4 quantization after a block-diagonal Hadamard rotation,
 *          a fused rotation+quantization write into a paged KV-cache layout, fused attention.
 *   [KV4]  "KV4-RL: Unlocking Faster Asynchronous Rollouts for RLVR with INT4 KV Cache
 *          Quantization", Abstract -- calibration-free INT4 KV with selective INT8 protection of
 *          attention sinks and recent context, over a bounded number of positions.
 *   [TOP5] "KV Cache Quantization" topic page, item 5 -- the full context is stored in INT4 and
 *          only sinks and recent context are (additionally) held in INT8.
 *
 * Conventions for every entry point
 *   - Pointers marked (host) are read during the call only; pointers marked (device) are device
 *     memory on the cache's device, owned by the caller, and must stay valid until the stream
 *     work enqueued by the call has finished.  The library never frees caller memory.
 *   - Calls validate every argument and update the handle's host state synchronously, then
 *     enqueue device work on `stream` and return; results are valid in stream order.
 *   - A call that returns an error other than KV4_ERR_HIP has changed nothing.  After
 *     KV4_ERR_HIP the cache state is undefined.  kv4_last_error() gives the detail.
 *   - A handle is not thread-safe.  Calls that touch the same sequences from different streams
 *     must be ordered by the caller.
 */
#ifndef KV4_H
#define KV4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kv4_status {
    KV4_OK = 0,
    KV4_ERR_INVALID_ARGUMENT = 1,   /* malformed argument (bad id, negative count, duplicate id, ...) */
    KV4_ERR_OUT_OF_PAGES = 2,       /* the free list cannot cover the call; nothing changed */
    KV4_ERR_SEQ_STATE = 3,          /* sequence would exceed max_pages_per_seq, or decode of length 0 */
    KV4_ERR_WORKSPACE_TOO_SMALL = 4,/* workspace smaller than the size query reports */
    KV4_ERR_UNSUPPORTED = 5,        /* valid configuration with no kernel instantiation */
    KV4_ERR_HIP = 6                 /* a HIP runtime call failed; state undefined */
} kv4_status;

typedef enum kv4_format {
    KV4_FORMAT_INT4_PROT = 0, /* INT4 pages for every token + INT8 sink/recent slots ([KV4], [TOP5]) */
    KV4_FORMAT_INT8 = 1,      /* every token INT8 in pages, same rotation and quantizer (baseline) */
    KV4_FORMAT_BF16 = 2       /* raw bf16 pages, no rotation, no quantization (baseline) */
} kv4_format;

/* How a position that leaves the recent window reaches its INT4 copy (INT4_PROT only). */
typedef enum kv4_eviction {
    KV4_EVICT_DUAL_WRITE = 0, /* INT4 code quantized from the rotated values at append ([TOP5]) */
    KV4_EVICT_REQUANT = 1     /* INT4 code re-quantized from the INT8 copy ([KV4]: tokens leaving the
                                 window move from INT8 to INT4); see kv4_append */
} kv4_eviction;

typedef struct kv4_config {
    int32_t num_q_heads;       /* Hq; Hq % Hkv == 0 and G = Hq / Hkv in {1, 2, 4} */
    int32_t num_kv_heads;      /* Hkv >= 1 */
    int32_t head_dim;          /* D in {64, 128} */
    int32_t page_size;         /* P; must be 16 */
    int32_t num_pages;         /* pages in the pool (each holds P tokens of every kv head) */
    int32_t max_seqs;          /* sequence ids are 0 .. max_seqs-1 */
    int32_t max_pages_per_seq; /* block-table row length */
    int32_t num_sinks;         /* S >= 0 INT8-protected leading positions (INT4_PROT only) */
    int32_t num_recent;        /* R >= 0 INT8-protected trailing positions (INT4_PROT only) */
    int32_t hadamard_block;    /* b: power of two dividing D; 1 = no rotation ("plain INT4") */
    int32_t format;            /* kv4_format */
    int32_t eviction;          /* kv4_eviction; must be KV4_EVICT_DUAL_WRITE for INT8 / BF16 */
} kv4_config;

/*
 * Device buffer sizes for a configuration.  Documented memory layout (part of the ABI; tests
 * read the pools through it).  Every block below is 128-byte aligned; base pointers must be
 * 256-byte aligned.  "chunk" interleaving puts 16 consecutive slots' 16-byte pieces side by side.
 *
 * INT4_PROT page block, per (page, kv head), page_block_bytes = 16*D + 128:
 *   [0, 8D)        K codes  [D/32 chunks][16 slots][16 B]; the 16 B piece c of slot t holds
 *                  dims 32c..32c+31 of token t, byte k = code[2k] | code[2k+1] << 4
 *   [8D, 16D)      V codes  [D dims][8 B]; byte k of dim d = code(slot 2k) | code(slot 2k+1) << 4
 *   [16D, 16D+128) scales   [16 slots][4 x fp16] = (K scale, K zero, V scale, V zero)
 * INT8 tile (INT4_PROT protection slots and INT8-format pages), int8_tile_bytes = 32*D + 256:
 *   two blocks x = 0, 1 of 16*D + 128 bytes each, shaped like an INT4 page block; block x holds
 *   [0, 8D)        K codes  [D/32 chunks][16 slots][16 B]; piece c of slot t = dims
 *                  x*D/2 + 16c .. x*D/2 + 16c + 15 of token t, one byte each
 *   [8D, 16D)      V codes  [D dims][8 B]; byte j of dim d = code of slot 8x + j
 *   [16D, 16D+128) scales   [16 slots][4 x fp16] as above (the same in both blocks)
 * BF16 page block, page_block_bytes = 64*D:
 *   [0, 32D)       K        [D/8 chunks][16 slots][8 x bf16]
 *   [32D, 64D)     V        [D dims][16 slots x bf16]
 *
 * page_pool  : [num_pages][Hkv][page_block_bytes]     (INT8 format: page block = INT8 tile)
 * int8_pool  : [max_seqs][Hkv][int8_tiles][int8_tile_bytes], INT4_PROT only; slot u of a sequence
 *              is tile u/16, slot u%16.  Sink position t < S sits in slot t; a recent position
 *              t >= S sits in ring slot S + (t mod R).
 * block_table: int32 [max_seqs][max_pages_per_seq]; entry j of a sequence is the page holding its
 *              positions 16j .. 16j+15.  Entries beyond ceil(L/16) are unspecified.
 * Slots outside the current protected set and page slots >= L hold unspecified bytes.
 * Codes and scales follow the quantizer described at kv4_append.
 */
typedef struct kv4_buffer_sizes {
    size_t page_pool;
    size_t int8_pool;
    size_t block_table;
    size_t page_block_bytes;
    size_t int8_tile_bytes;
    int32_t int8_tiles; /* ceil((S + R) / 16) for INT4_PROT, else 0 */
} kv4_buffer_sizes;

typedef struct kv4_buffers {
    void* page_pool;      /* (device) page_pool bytes */
    void* int8_pool;      /* (device) int8_pool bytes; may be NULL when int8_pool == 0 */
    int32_t* block_table; /* (device) block_table bytes */
} kv4_buffers;

typedef struct kv4_cache* kv4_cache_t;

/* Sizes of the caller-allocated device buffers for `cfg`.  Errors: INVALID_ARGUMENT for a
 * malformed config (b not a power of two, D % b != 0, Hq % Hkv != 0, negative counts, an unknown
 * eviction rule or KV4_EVICT_REQUANT outside INT4_PROT),
 * UNSUPPORTED for a valid config without a kernel (P != 16, D not in {64,128}, G not in {1,2,4}). */
kv4_status kv4_buffer_sizes_query(const kv4_config* cfg, kv4_buffer_sizes* out);

/* Creates a cache over caller-allocated buffers on the current HIP device.  All sequences start
 * empty; the free list is 0, 1, ..., num_pages-1.  The buffers' initial contents do not matter. */
kv4_status kv4_cache_create(const kv4_config* cfg, const kv4_buffers* bufs, kv4_cache_t* out);

/* Destroys the handle (host state only).  Waits for the handle's own staging copies. */
kv4_status kv4_cache_destroy(kv4_cache_t h);

/* Device workspace needed by kv4_append for this argument list (host arrays). */
kv4_status kv4_append_workspace_size(kv4_cache_t h, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_new,
                                     size_t* bytes);

/*
 * Append n_new[i] new positions to sequence seq_ids[i] for each i (ids distinct).
 *   k_new, v_new (device): bf16 [sum(n_new)][Hkv][D], rows ordered by (call order, ascending
 *   position).  K is taken as given (post-RoPE); no position encoding is applied here.
 * Per call: if the free list holds fewer pages than the call needs, KV4_ERR_OUT_OF_PAGES and no
 * change.  Otherwise pages are popped from the front of the free list, sequences in call order,
 * positions ascending, and written into the block table.
 * Per new position t (sequence length becomes L = L_old + n_new) and kv head, K and V separately
 * ([SAW] rotation and token-wise quantization; [KV4]/[TOP5] protection):
 *   y    = FWHT of each b-block of the bf16 row, stages h = 1, 2, ..., b/2 in binary32
 *          (each butterfly (a, c) -> (a + c, a - c)), then one multiply by fl32(1/sqrt(b))
 *   z    = largest fp16 <= min(y);  s = smallest fp16 >= fl32(fl32(max(y) - z) / Q)
 *   code = round-half-even(fl32(fl32(y - z) * fl32(1/s))), 0 when s == 0   (no FMA contraction)
 *   INT4 (Q = 15) is written to the page for every position; when t is in
 *   Prot(L) = {t < min(S, L)} u {max(S, L - R) <= t < L} the INT8 code (Q = 255, same y) is also
 *   written to the position's sink or ring slot.  A position that later leaves Prot is read from
 *   its INT4 page copy.  Zero results of z and s are stored as +0.
 *   eviction = KV4_EVICT_DUAL_WRITE: the INT4 code is quantized from y (nothing is re-quantized).
 *   eviction = KV4_EVICT_REQUANT: the INT4 code is quantized from the INT8 round trip
 *   x8 = fl32(s8 * code8 + z8) of y (the move from INT8 to INT4 of a position leaving the window,
 *   computed when the position is appended: x8 depends on the position alone, and doing it for
 *   every position keeps a prefill equal to single appends).
 * INT8 format: Q = 255 in pages for every position.  BF16 format: bf16 rows copied.
 * Preconditions not checked per element: inputs finite, |y| <= 65504.
 * Errors: INVALID_ARGUMENT, OUT_OF_PAGES, SEQ_STATE (length would exceed max_pages_per_seq * P),
 * WORKSPACE_TOO_SMALL, HIP.
 */
kv4_status kv4_append(kv4_cache_t h, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_new,
                      const void* k_new, const void* v_new, void* workspace, size_t ws_bytes,
                      void* stream /* hipStream_t; NULL = null stream */);

/*
 * kv4_append with keys given before RoPE: the append applies RoPE to each key row and then
 * everything kv4_append does (the pages apply the Hadamard transform to keys after RoPE; this
 * fuses the two so the post-RoPE keys never go to memory).  For position t and i < D/2, with
 * c = rope_cos[t][i], s = rope_sin[t][i] (binary32, caller-owned device tables [rope_positions][D/2]):
 *   (x_i, x_{i+D/2}) -> (fl32(fl32(x_i c) - fl32(x_{i+D/2} s)), fl32(fl32(x_{i+D/2} c) + fl32(x_i s)))
 * (rotate-half pairing).  The binary32 result is rotated and quantized as is (no bf16 rounding in
 * between).  Values are unchanged.  Every new position must be < rope_positions.
 * Formats: INT4_PROT and INT8 (BF16: UNSUPPORTED).  Other errors as kv4_append.
 */
kv4_status kv4_append_rope(kv4_cache_t h, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_new,
                           const void* k_new, const void* v_new, const float* rope_cos, const float* rope_sin,
                           int32_t rope_positions, void* workspace, size_t ws_bytes,
                           void* stream /* hipStream_t */);

/* Releases a sequence: length -> 0, its pages go to the back of the free list in block-table
 * order.  Host state only.  Error: INVALID_ARGUMENT for a bad id. */
kv4_status kv4_seq_free(kv4_cache_t h, int32_t seq_id);

/* Device workspace needed by kv4_decode_attention for any call with up to n_seqs sequences. */
kv4_status kv4_decode_workspace_size(kv4_cache_t h, int32_t n_seqs, size_t* bytes);

/*
 * Decode attention for n_seqs sequences (ids distinct, every length L >= 1).  [SAW] Abstract:
 * attention fused over the paged INT4 layout of block-Hadamard-rotated keys and values (the query
 * is rotated once and the output un-rotated once, since H is orthogonal); [KV4] Abstract and
 * [TOP5]: the attention-sink and recent-context positions are read from their INT8 copies, every
 * other position from INT4.
 *
 *   q   (device) bf16 [n_seqs][Hq][D], row i for seq_ids[i];
 *   out (device) fp32 [n_seqs][Hq][D].
 * Query head g reads kv head g / G.  Over all L positions t (the INT8 slot when t is in Prot(L),
 * otherwise the INT4 page copy; INT8 / BF16 formats read their pages):
 *   out[g] = sum_t softmax_t(scale * <q_g H, k^_t>) v^_t H^T
 * where k^, v^ are the dequantized rotated rows (s*code + z) and H the block-diagonal Hadamard
 * (identity for BF16).  scale <= 0 selects 1/sqrt(D).
 * Errors: INVALID_ARGUMENT, SEQ_STATE (length 0), WORKSPACE_TOO_SMALL, HIP.
 */
kv4_status kv4_decode_attention(kv4_cache_t h, int32_t n_seqs, const int32_t* seq_ids, const void* q,
                                float scale, float* out, void* workspace, size_t ws_bytes,
                                void* stream /* hipStream_t */);

/* Device workspace needed by kv4_multi_query_attention for exactly this argument list and the
 * cache's current lengths (query it for the call it is meant for).  Errors as for the call. */
kv4_status kv4_multi_query_workspace_size(kv4_cache_t h, int32_t n_seqs, const int32_t* seq_ids,
                                          const int32_t* n_q, size_t* bytes);

/*
 * Causal attention of several query positions per sequence over the cache as it stands (a
 * prefill chunk attending the cache after the chunk's own append, or the tokens of a multi-token
 * decode step).  The pages define no such call; it extends the fused attention of [SAW] with the
 * reading stated here.  For each i (ids distinct, length L >= n_q[i] >= 1), the n_q[i] query rows
 * of sequence seq_ids[i] sit at positions L - n_q[i] .. L - 1, and row r attends positions
 * 0 .. L - n_q[i] + r, each read from the copy decode reads at length L (the INT8 slot when the
 * position is in Prot(L), else its INT4 page copy):
 *   out[row][g] = sum_{t <= pos(row)} softmax_t(scale * <q_g H, k^_t>) v^_t H^T
 * n_q[i] = 1 for every i is decode attention.
 *   q   (device) bf16 [sum n_q][Hq][D]: the rows of a sequence consecutive in ascending position,
 *       sequences in call order;
 *   out (device) fp32, the same shape and order.
 * Formats: INT4_PROT and INT8 (BF16: UNSUPPORTED).  scale <= 0 selects 1/sqrt(D).
 * Errors: INVALID_ARGUMENT, SEQ_STATE (length 0 or n_q > L), UNSUPPORTED, WORKSPACE_TOO_SMALL, HIP.
 */
kv4_status kv4_multi_query_attention(kv4_cache_t h, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_q,
                                     const void* q, float scale, float* out, void* workspace, size_t ws_bytes,
                                     void* stream /* hipStream_t */);

/* kv4_decode_attention with bf16 output: out (device) bf16 [n_seqs][Hq][D], each value the
 * round-to-nearest-even of the fp32 result kv4_decode_attention returns for the same call (for
 * the next layer of a model that runs in bf16).  Same arguments, workspace and errors. */
kv4_status kv4_decode_attention_bf16(kv4_cache_t h, int32_t n_seqs, const int32_t* seq_ids, const void* q,
                                     float scale, void* out, void* workspace, size_t ws_bytes,
                                     void* stream /* hipStream_t */);

/*
 * kv4_decode_attention for callers that cannot allocate memory during the call (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same computation,
 * kernels and result bits as kv4_decode_attention with its automatic wave count, but the
 * split-KV partials live in a device scratch array that the library holds, one per GPU, of
 * 16 MiB, kept until the process ends (its address is looked up once per device by
 * kv4_cache_create).  The call allocates nothing, host or device, and records no profiling events.
 *   q (device) bf16 [n_seqs][Hq][D], out (device) fp32 [n_seqs][Hq][D], as kv4_decode_attention.
 * Limits: n_seqs <= 256 (UNSUPPORTED beyond), and the call's partials (about (W + n_seqs * Hkv) *
 * G * (D + 2) * 4 bytes, W = the split's wave count) must fit the 16 MiB (WORKSPACE_TOO_SMALL).
 * Nothing in the scratch needs clearing between calls: every partial the merge reads is written by
 * the same call.  All calls on one GPU share that GPU's scratch: calls that may overlap (on
 * different streams, or from several handles or threads) race and must be ordered by the caller.
 * Other errors as kv4_decode_attention.
 */
kv4_status kv4_decode_attention_noalloc(kv4_cache_t h, int32_t n_seqs, const int32_t* seq_ids, const void* q,
                                        float scale, float* out, void* stream /* hipStream_t */);

/* Host-state queries. */
kv4_status kv4_seq_length(kv4_cache_t h, int32_t seq_id, int32_t* len);
kv4_status kv4_block_table(kv4_cache_t h, int32_t seq_id, int32_t* pages /* host */, int32_t cap, int32_t* n);
kv4_status kv4_free_pages(kv4_cache_t h, int32_t* n);

/* Tuning: number of waves the decode split kernel launches (0 = automatic). */
kv4_status kv4_set_decode_waves(kv4_cache_t h, int32_t waves);
/* Tuning: a second round of round2_waves decode split waves that share the last
 * (1000 - round1_permille) / 1000 of the call's steps (0 = one round).  The results do not depend
 * on it beyond rounding order. */
kv4_status kv4_set_decode_rounds(kv4_cache_t h, int32_t round2_waves, int32_t round1_permille);
/* Tuning: multi-query calls of the INT4+INT8 format in which every sequence has a multiple of 4
 * row tiles (n_q * (hq / hkv) / 16 rounded up) let the four waves of a workgroup, which take
 * four row tiles of the same pages, share each step's staged pages and spread operands
 * (enable != 0, the default); 0 gives every wave its own.  The results are the same bits either
 * way. */
kv4_status kv4_set_mq_share(kv4_cache_t h, int32_t enable);

/* Kernel timing (measurement of the hot path).  When enabled, each kernel a call launches on its
 * stream stamps a pair of HIP events from its own dispatch (start, stop), so a duration is that
 * kernel's execution alone; kv4_profile_read waits for them and returns the summed durations.
 * Enabling (or disabling) resets the totals.  Off by default. */
typedef struct kv4_profile {
    int64_t append_launches;
    double append_ms;  /* append kernels */
    int64_t decode_launches;
    double split_ms;   /* decode split-KV kernels */
    double merge_ms;   /* decode merge + inverse-rotation kernels */
    int64_t mq_launches;
    double mq_split_ms;  /* multi-query split kernels */
    double mq_merge_ms;  /* multi-query merge + inverse-rotation kernels */
} kv4_profile;
kv4_status kv4_profile_enable(kv4_cache_t h, int32_t enable);
kv4_status kv4_profile_read(kv4_cache_t h, kv4_profile* out);
/* Per-launch durations (ms, launch order) of one kernel kind since profiling was enabled: kind 0
 * append, 1 decode split, 2 decode merge, 3 multi-query split, 4 multi-query merge.  Writes up to
 * cap values to ms (host) and the number collected to *n.  Waits for the events. */
kv4_status kv4_profile_durations(kv4_cache_t h, int32_t kind, float* ms, int32_t cap, int32_t* n);

/*
 * HBM ceiling probe (measurement; no cache involved): the practical streaming bandwidth of the
 * device that the cache kernels' achieved bytes per second are compared with, beside the published
 * peak.  Runs `reps` back-to-back launches on `stream` of
 *   mode 0: a streaming read of `bytes` from src (16-byte loads); each lane of the grid stores one
 *           folded word to dst, so dst (device) must hold blocks * 1024 bytes;
 *   mode 1: a copy of `bytes` from src to dst (device, non-overlapping);
 * each launch stamping its own start / stop events, waits for them and writes each launch's
 * duration in ms to ms[0 .. reps) (host).  blocks: workgroups of 256 lanes, 0 = 8 per compute unit.
 * bytes must be a positive multiple of 16, pointers 16-byte aligned, on the current device.
 * Errors: INVALID_ARGUMENT, HIP.
 */
kv4_status kv4_hbm_probe(int32_t mode, const void* src, void* dst, size_t bytes, int32_t blocks, int32_t reps,
                         float* ms, void* stream /* hipStream_t */);

const char* kv4_status_string(kv4_status s);
/* Detail of the last error on h (or of the last handle-less error when h is NULL). */
const char* kv4_last_error(kv4_cache_t h);

#ifdef __cplusplus
}
#endif

#endif /* KV4_H */
