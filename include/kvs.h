/*
 * kvs.h -- C ABI of the MI355X (gfx950) paged GQA decode + block-scoring library.
 *
 * What the library computes, per decode step:
 *
 *  1. Paged decode attention.  For every sequence s, layer l and query head h,
 *     the step's query attends over all n_s cached positions of the sequence.
 *     Position t lives in physical block block_table[s][t / 16] at slot t % 16
 *     ("KV cache offload" architecture post, "Top row": fixed-size blocks and a
 *     per-sequence table from logical positions to physical block ids).  Query
 *     head h reads KV head h / 8 (GQA Per-Head Scoring Streams, panel 1:
 *     Q0-Q7 -> KV-head 0 ... Q56-Q63 -> KV-head 7).  out = softmax(scale q.K) V
 *     (KV-Cache Offloading for LLM Inference -- Visual Reference, Sec. 2,
 *     Diagram 2.2).  No mask other than the sequence length; no rotary encoding.
 *
 *  2. Block mass.  In the same step the probability mass that every
 *     (layer, query head) puts on each 16-token block is summed into one fp32
 *     number per (sequence, logical block): the 640 (layer, KV-head) streams of
 *     the 80-layer model reduced to one score per block (GQA Per-Head Scoring
 *     Streams, panel 2).  The sum over streams is this library's reading of the
 *     page's unnamed aggregation.
 *
 *  3. Scoring.  Per (sequence, block) record: normalise the mass by the
 *     sequence's largest block mass, EMA/LRFU update
 *     E <- alpha m_hat + (1 - alpha) E (Visual Reference Sec. 11, Diagram 11.1),
 *     touch count += 1, touch timestamp = step, priority
 *     P = w_R (b+1)/nb + w_E E + w_N anchor (Sec. 12, Diagram 12.1) and tier
 *     0 if P >= t_high, 1 if P >= t_low, else 2 (Sec. 12, Diagram 12.2).
 *
 * Conventions for every entry point:
 *  - Device pointers are caller-owned device memory.  The library allocates
 *    nothing, frees nothing and keeps no device state between calls.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *    compute call only enqueues work on that stream; results are valid once the
 *    stream reaches them.  Only kvs_device_status() synchronises.
 *  - Return value: KVS_OK (0) or a negative kvs_status.  Every argument that can
 *    be checked on the host is checked before anything is enqueued; on error
 *    nothing is launched and kvs_last_error() holds a message (thread-local).
 *  - Errors only visible in device data (a physical block id outside the pool,
 *    a sequence longer than its table row, inconsistent record offsets, a step
 *    that does not advance) never cause an out-of-bounds access: the offending
 *    block, sequence or record is skipped and a bit is OR-ed into a sticky
 *    status word at the start of the workspace (read it with
 *    kvs_device_status()).
 *  - Calls on different streams are safe when their outputs and workspaces are
 *    disjoint.
 */
#ifndef KVS_H
#define KVS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KVS_OK = 0,
    KVS_E_NULL = -1,       /* a required pointer is NULL */
    KVS_E_SHAPE = -2,      /* head shape other than 64 / 8 / 128 / 16, or num_layers outside [1, 65535] */
    KVS_E_RANGE = -3,      /* a count or index argument is out of range */
    KVS_E_ALIGN = -4,      /* a tensor is not 16-byte aligned */
    KVS_E_WORKSPACE = -5,  /* workspace smaller than the matching *_workspace_bytes() */
    KVS_E_POLICY = -6,     /* alpha not in (0, 1], a negative weight, cut points not 0 <= t_low <= t_high */
    KVS_E_HIP = -7         /* the HIP runtime reported an error while enqueuing */
} kvs_status;

/* Sticky device status bits (kvs_device_status). */
#define KVS_DEV_BAD_BLOCK_ID   0x1u  /* a table entry outside [0, pool_blocks): block skipped */
#define KVS_DEV_BAD_SEQ_LEN    0x2u  /* seq_len < 0 or > 16 * max_blocks_per_seq: sequence skipped */
#define KVS_DEV_BAD_OFFSETS    0x4u  /* meta_offsets inconsistent with seq_lens / total_blocks */
#define KVS_DEV_STALE_STEP     0x8u  /* step <= a record's touch timestamp: record left unchanged */
#define KVS_DEV_POOL_EXHAUSTED 0x10u /* kvs_append_kv: no free block, table row full or no record
                                        capacity for a sequence that needed a block: not appended;
                                        kvs_kivi_advance: no free quantised block (or no room on
                                        the fp16 free stack): boundary not moved */

/* Model head shape.  The kernels support num_q_heads 64, num_kv_heads 8,
 * head_dim 128, block_tokens 16 and 1 <= num_layers <= 65535 (Visual Reference
 * Sec. 1, Architecture Parameters). */
typedef struct {
    int32_t num_layers;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_tokens;
} kvs_shape;

/* Scoring parameters.  The pages call every one of these uncalibrated and
 * illustrative (Visual Reference Sec. 12), so all are runtime values.
 * Defaults from the pages: w_recency 0.25, w_ema 0.55, w_anchor 0.20,
 * t_low 0.3, t_high 0.6; alpha 0.05 (simulated optimum) or 0.15 (specified),
 * Sec. 11. */
typedef struct {
    double alpha;
    double w_recency;
    double w_ema;
    double w_anchor;
    double t_low;
    double t_high;
} kvs_policy;

/* The 64-byte per-block record (GQA Per-Head Scoring Streams, "Per-block state
 * (64 bytes)": 16 B identity key, 8 B score, 8 B touch timestamp, 4 B touch
 * count, reserved).  The library keeps the tier label, an anchor flag and the
 * last priority inside the reserved bytes. */
typedef struct {
    uint64_t key[2];       /*  0: identity {seq_id, logical block index}; survives eviction */
    double   score;        /* 16: EMA/LRFU score E, starts at 0 */
    uint64_t t_touch;      /* 24: step of the last touch; UINT64_MAX = never touched */
    uint32_t touch_count;  /* 32: decode steps that read the block */
    uint8_t  tier;         /* 36: 0 pinned HBM, 1 evictable HBM, 2 CXL; 0xFF = unclassified */
    uint8_t  flags;        /* 37: bit 0 = anchor-zone block */
    uint16_t reserved0;    /* 38 */
    double   priority;     /* 40: last P; 0 before the first classification */
    uint8_t  reserved1[16];/* 48 */
} kvs_block_meta;

#define KVS_NEVER_TOUCHED  UINT64_MAX
#define KVS_UNCLASSIFIED   0xFFu
#define KVS_FLAG_ANCHOR    0x1u

/* ---- host-only helpers (no GPU needed) ---------------------------------- */

/* KV bytes of one token: 2 (K and V) x layers x KV heads x head_dim x 2 B
 * (Visual Reference Sec. 3, Diagram 3.1).  0 if shape is NULL. */
size_t kvs_bytes_per_token(const kvs_shape* shape);

/* Bytes of one physical block: block_tokens x kvs_bytes_per_token(). */
size_t kvs_block_bytes(const kvs_shape* shape);

/* sizeof(kvs_block_meta) (64).  When offsets != NULL and n >= 9, writes the byte
 * offsets of key, score, t_touch, touch_count, tier, flags, reserved0,
 * priority, reserved1. */
size_t kvs_meta_layout(size_t* offsets, int n);

/* Stored K/V formats, one per decode entry point. */
#define KVS_KV_FP16 0   /* kvs_decode_step: fp16 values */
#define KVS_KV_E4M3 1   /* kvs_decode_step_e4m3: FP8 E4M3 codes */
#define KVS_KV_KIVI2 2  /* kvs_decode_step_kivi: 2-bit KIVI blocks + fp16 residual */

/* Blocks per split used for this problem when split_blocks == 0 is passed (a
 * power of two in [16, 1024] -- at most 512 for KVS_KV_E4M3 and 128 for
 * KVS_KV_KIVI2 -- chosen from the sizes and the stored format kv_format, one of
 * KVS_KV_*, so that the launch keeps enough reads in flight); otherwise
 * split_blocks itself if valid (for KVS_KV_KIVI2 it must also be even).  0 if
 * any argument is invalid. */
int32_t kvs_decode_split_blocks(const kvs_shape* shape, int32_t kv_format, int32_t batch,
                                int32_t max_blocks_per_seq, int32_t layer_begin,
                                int32_t layer_end, int32_t split_blocks);

/* Workspace bytes the decode entry point of format kv_format needs for these
 * sizes (0 on invalid input).  The workspace holds a 256-byte status header,
 * the per-split softmax statistics and partial outputs, and the
 * per-(layer, head, block) mass partials: about
 * 4 x 64 x (layer_end - layer_begin) x total_blocks bytes. */
size_t kvs_decode_workspace_bytes(const kvs_shape* shape, int32_t kv_format, int32_t batch,
                                  int32_t max_blocks_per_seq, int64_t total_blocks,
                                  int32_t layer_begin, int32_t layer_end,
                                  int32_t split_blocks);

/* Bytes of one quantised (KIVI 2-bit) block: num_layers x 2 x 8 x 768, 3/16
 * of an fp16 block.  0 if shape is NULL. */
size_t kvs_kivi_block_bytes(const kvs_shape* shape);

/* Workspace bytes kvs_score_update needs (status header + per-chunk maxima). */
size_t kvs_score_workspace_bytes(int32_t batch, int32_t max_blocks_per_seq);

/* A fixed English name for a kvs_status code ("unknown status" for any other
 * value).  The string is static: the caller does not free it. */
const char* kvs_status_string(int code);
/* The message of this host thread's last status-returning call: its error
 * if it failed, "" if it succeeded (a thread-local buffer of at most 511
 * characters; the size helpers above return no status and leave it alone).
 * The pointer stays valid for the thread's life; the next status-returning
 * call on the thread rewrites the text. */
const char* kvs_last_error(void);

/* Measurement hook.  With both events non-NULL (hipEvent_t passed as void*),
 * every later kvs_decode_step call on this host thread records `before` on its
 * stream just before the paged decode kernel and `after` just after it, so a
 * caller can time that kernel alone.  kvs_set_decode_events(NULL, NULL) turns
 * it off.  Returns KVS_E_NULL when exactly one event is NULL. */
int kvs_set_decode_events(void* before, void* after);

/* ---- device entry points ------------------------------------------------- */

/* Bandwidth probe: the achievable-HBM reference that throughput figures are
 * compared with (the pages measure achievable streaming bandwidth with a plain
 * copy of large buffers, median of several runs: Visual Reference Sec. 4 and 9,
 * measurement notes).  Not part of the decode path.
 *  mode 0 (read):  reads `bytes` from src, each wave 8 KiB chunks of 1 KiB
 *                  non-temporal loads, two chunks in flight, with the grid
 *                  sweeping the buffer front to back; every lane folds what it
 *                  read into one 32-bit word written to dst (dst must hold
 *                  grid x 256 words, 2,048 x 256 for grid 0: the library
 *                  cannot check this and writes past a shorter dst).
 *  mode 1 (copy):  copies `bytes` from src to dst.
 * bytes must be a non-zero multiple of 16; src and dst 16-byte aligned;
 * grid = number of 256-lane work-groups (0 = library choice). */
int kvs_stream_probe(const void* src, void* dst, size_t bytes, int mode, int32_t grid,
                     void* stream);

/* Zero the 256-byte status header of a workspace (decode or score).  Call once
 * after allocating a workspace.  Enqueues one small kernel. */
int kvs_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* Waits for `stream`, copies the sticky status word of `workspace` to *bits and
 * clears it.  The only synchronising call. */
int kvs_device_status(void* workspace, void* stream, uint32_t* bits);

/* One paged GQA decode step plus block mass, for layers [layer_begin, layer_end).
 *
 *  q             fp16 [batch][num_layers][64][128], device, 16-B aligned.
 *  kv_pool       fp16 [pool_blocks][num_layers][2][8][16][128], device, 16-B
 *                aligned.  Index [p][l][0] holds keys, [p][l][1] values; slot
 *                o of block p is position 16 b + o of every sequence whose
 *                table maps logical block b to p.
 *  block_table   int32 [batch][max_blocks_per_seq], device: physical block id
 *                of each logical block.  Entries past a sequence's end are not read.
 *  seq_lens      int32 [batch], device: tokens per sequence (0 allowed).
 *  meta_offsets  int32 [batch + 1], device: record index of (s, b) is
 *                meta_offsets[s] + b.  meta_offsets[s+1] - meta_offsets[s] is the
 *                sequence's record capacity: it must be >= ceil(seq_lens[s] / 16)
 *                and <= max_blocks_per_seq, and meta_offsets[batch] <= total_blocks.
 *                (Equal to ceil(seq_lens[s] / 16) for a cache that does not grow;
 *                larger when kvs_append_kv will grow the sequence.)
 *  total_blocks  host copy of the number of records.
 *  scale         softmax scale (1/sqrt(128) for the pages' model).
 *  out           fp16 [batch][num_layers][64][128], device: rows of layers in
 *                range are overwritten; other rows are not touched.
 *  block_mass    fp32 [total_blocks], device: sum over layers in range, all 64
 *                query heads and the block's tokens of the softmax probability.
 *                accumulate == 0 overwrites, 1 adds (for per-layer-range calls).
 *  split_blocks  blocks per split-K work item; 0 = library choice.  Must match
 *                the value given to kvs_decode_workspace_bytes.
 *  workspace     device scratch of kvs_decode_workspace_bytes() bytes, 256-B
 *                aligned, status header zeroed once by kvs_workspace_init().
 * A wave of the decode serves one KV head, or two adjacent ones (2 i, 2 i + 1)
 * when the records cover at least 3/4 of batch x splits x split_blocks (the
 * sequences fill their splits).  The results are the same bit for bit either
 * way, except that with two heads per wave a NaN among the values a sequence
 * reads from one head also makes those channels NaN in the other head's output
 * rows.
 */
int kvs_decode_step(const kvs_shape* shape,
                    const void* q,
                    const void* kv_pool, int64_t pool_blocks,
                    const int32_t* block_table, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, const int32_t* meta_offsets,
                    int32_t batch, int64_t total_blocks,
                    int32_t layer_begin, int32_t layer_end,
                    float scale,
                    void* out, float* block_mass, int accumulate,
                    int32_t split_blocks,
                    void* workspace, size_t workspace_bytes,
                    void* stream);

/* Bytes of the library-owned scratch kvs_decode_step_noalloc uses (32 MiB). */
#define KVS_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* kvs_decode_step without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It allocates nothing (no hipMalloc, hipFree or allocating
 * library routine).  The split statistics, partial outputs and mass partials
 * live in a file-scope device array of KVS_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends; its address is
 * looked up once per device on the first call there (make that first call
 * outside graph capture).  Arguments, results and rules are those of
 * kvs_decode_step, except:
 *  status  uint32, device, 4-B aligned, caller-owned: the sticky device-data
 *          bits kvs_device_status() would report for a workspace are OR-ed in
 *          here; the caller clears it.
 * A call whose sizes need more than KVS_NOALLOC_SCRATCH_BYTES (see
 * kvs_decode_workspace_bytes with KVS_KV_FP16) returns KVS_E_WORKSPACE before
 * anything is enqueued: split such a step into layer ranges (accumulate = 1).
 * Every call on one GPU shares that GPU's scratch, which keeps the last call's
 * contents (each call writes every part it later reads): calls that overlap
 * on one GPU -- on different streams or from different host threads without
 * ordering -- race and give wrong results. */
int kvs_decode_step_noalloc(const kvs_shape* shape,
                            const void* q,
                            const void* kv_pool, int64_t pool_blocks,
                            const int32_t* block_table, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, const int32_t* meta_offsets,
                            int32_t batch, int64_t total_blocks,
                            int32_t layer_begin, int32_t layer_end,
                            float scale,
                            void* out, float* block_mass, int accumulate,
                            int32_t split_blocks,
                            uint32_t* status,
                            void* stream);

/* The same step over a pool of FP8 E4M3 codes: kv_pool is uint8
 * [pool_blocks][num_layers][2][8][16][128] holding OCP E4M3 codes with no scale
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 encodes
 * m * 2^-9; 0x7F / 0xFF are NaN), half the bytes of the fp16 pool (Fitting a
 * Million Tokens, Sec. 02: FP8 E4M3 KV, no calibration).  Every code is
 * dequantised exactly to fp16 inside the kernel; q, out, the block mass and all
 * other arguments, sizes and rules are those of kvs_decode_step (the workspace
 * of kvs_decode_workspace_bytes serves both).  One wave serves KV heads 2 i
 * and 2 i + 1 together; each query head's arithmetic is that of a decode with
 * one head per wave, except that a NaN code among the values a sequence reads
 * from one of the two heads also makes the other head's output rows NaN (its
 * product with that head's zero weights). */
int kvs_decode_step_e4m3(const kvs_shape* shape,
                         const void* q,
                         const void* kv_pool, int64_t pool_blocks,
                         const int32_t* block_table, int32_t max_blocks_per_seq,
                         const int32_t* seq_lens, const int32_t* meta_offsets,
                         int32_t batch, int64_t total_blocks,
                         int32_t layer_begin, int32_t layer_end,
                         float scale,
                         void* out, float* block_mass, int accumulate,
                         int32_t split_blocks,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/* ---- KIVI-style 2-bit KV (Fitting a Million Tokens, Sec. 02) --------------
 * Asymmetric 2-bit quantisation in groups of 32 elements: zero point z = the
 * group minimum, scale s = fp16(fp32(fp32(max - min) / 3)), code =
 * clamp(rint(fp32(fp32(x - z) / s)), 0, 3) (code 0 when s == 0), read back as
 * z + code * s.  Keys are grouped per channel over 32 consecutive tokens (two
 * 16-token blocks), values per token over 32 consecutive channels.  The newest
 * tokens stay fp16: tokens [0, quant_len) of a sequence are quantised, with
 * quant_len a multiple of 32 given by kvs_kivi_quant_len (the pages' residual
 * window of ~128 tokens: residual_tokens = 128).
 *
 * Quantised block format, uint8 [kivi_blocks][num_layers][2][8][768]: per
 * layer 8 key tiles then 8 value tiles of 768 bytes, one per KV head.  Bytes
 * [0, 512) of a tile hold the block's 16 x 128 codes as 64 little-endian
 * 8-byte entries; entry l = 16 j + c is two 32-bit words holding four sets
 * S = 0..3 of 8 codes, set S in word S / 2, code m of the set at bits
 * 4 m + 2 (S % 2).
 *   key tile:   entry (j, c) is token c; set S, code m is channel 32 S + 8 j + m.
 *   value tile: set S, code m is token 4 j + (m % 4) of channel
 *               16 (2 S + m / 4) + c.
 * Bytes [512, 768): 64 fp16 scales then 64 fp16 zero points.
 *   key tile:   the 32-token group of an even/odd block pair; channels 0..63
 *               in the even block, 64..127 in the odd one, at index d % 64.
 *   value tile: token t, channel group g at index 16 g + t.
 * A 32-token pair is two blocks with logical indices 2 p and 2 p + 1; the
 * two may be any physical blocks of the quantised pool. */

/* The window rule: quantised tokens of a seq_len-token sequence whose newest
 * residual_tokens tokens stay fp16, i.e. the largest multiple of 32 that
 * leaves at least residual_tokens tokens (0 below residual_tokens + 32):
 * max(0, floor((seq_len - residual_tokens) / 32) * 32).  kvs_kivi_advance
 * applies the same rule on the device.  Host only; -1 if an argument is
 * negative. */
int32_t kvs_kivi_quant_len(int32_t seq_len, int32_t residual_tokens);

/* Quantise 32-token pairs of fp16 blocks into quantised blocks.
 *  kv_pool     fp16 pool as for kvs_decode_step (read only).
 *  kivi_pool   quantised pool, uint8 [kivi_blocks][num_layers][2][8][768].
 *  pairs       int32 [n_pairs][4], device: {fp16 block of tokens 0..15, fp16
 *              block of tokens 16..31, destination block for tokens 0..15,
 *              destination block for tokens 16..31}.  Pairs whose ids fall
 *              outside the pools are skipped and raise KVS_DEV_BAD_BLOCK_ID.
 *              Destination blocks of different pairs must differ.
 *  workspace   >= 256 bytes with a status header zeroed by kvs_workspace_init.
 * Every layer and KV head of each pair is quantised.  Inputs must be finite. */
int kvs_kivi_quantize(const kvs_shape* shape,
                      const void* kv_pool, int64_t pool_blocks,
                      void* kivi_pool, int64_t kivi_blocks,
                      const int32_t* pairs, int32_t n_pairs,
                      void* workspace, size_t workspace_bytes,
                      void* stream);

/* Workspace bytes kvs_kivi_advance needs for `batch` sequences (status header,
 * job list). */
size_t kvs_kivi_advance_workspace_bytes(int32_t batch);

/* Move KIVI quantisation boundaries forward after appends: the fp16 residual
 * window is where keys wait until 32 tokens form a whole group (Fitting a
 * Million Tokens, Sec. 02).  For each sequence s, in batch order, with
 * kvs_kivi_quant_len(seq_lens[s], residual_tokens) > quant_lens[s]: the fp16 blocks of
 * logical blocks quant_lens[s] / 16 and + 1 (ids in kv_pool) are quantised
 * into two blocks taken from the top of the KIVI free stack (the first such
 * sequence takes kivi_free[top - 1] for its even block and kivi_free[top - 2]
 * for its odd one, the next the two below); those table entries then hold the
 * KIVI ids, quant_lens[s] grows by 32, and the two fp16 ids are pushed onto
 * fp16_free (the stack kvs_append_kv pops), pair by pair in batch order.  At
 * most one pair per sequence per call, so a call after every append keeps
 * quant_lens[s] == max(0, floor((seq_lens[s] - residual_tokens) / 32) * 32).
 * With too few KIVI ids, later sequences are left unchanged and
 * KVS_DEV_POOL_EXHAUSTED is raised; bad lengths raise KVS_DEV_BAD_SEQ_LEN, ids
 * outside the pools KVS_DEV_BAD_BLOCK_ID.  Tops and stacks are device int32;
 * a top outside [0, capacity] is clamped into it (KVS_DEV_BAD_OFFSETS).  The
 * fp16 blocks of a sequence's residual window must be its own (not shared with
 * another sequence's table): they are pushed onto fp16_free once quantised.
 * Calls that overlap on one stream order race. */
int kvs_kivi_advance(const kvs_shape* shape,
                     const void* kv_pool, int64_t pool_blocks,
                     void* kivi_pool, int64_t kivi_blocks,
                     int32_t* block_table, int32_t max_blocks_per_seq,
                     const int32_t* seq_lens, int32_t* quant_lens, int32_t batch,
                     int32_t residual_tokens,
                     const int32_t* kivi_free, int32_t kivi_free_capacity, int32_t* kivi_free_top,
                     int32_t* fp16_free, int32_t fp16_free_capacity, int32_t* fp16_free_top,
                     void* workspace, size_t workspace_bytes,
                     void* stream);

/* The decode step of kvs_decode_step over a KIVI cache: for sequence s, block
 * table entries b < quant_lens[s] / 16 are ids in kivi_pool (quantised blocks,
 * pairs 2p, 2p + 1 holding one 32-token key group), and entries from
 * quant_lens[s] / 16 on are ids in kv_pool (fp16 residual blocks).
 * quant_lens: int32 [batch], device; each a multiple of 32 in [0, seq_lens[s]],
 * else the sequence is skipped and KVS_DEV_BAD_SEQ_LEN raised.  The result is
 * attention over the read-back values z + code * s of the quantised tokens and
 * the fp16 values of the rest.  split_blocks must be 0 or even.  Workspace:
 * kvs_decode_workspace_bytes(..., KVS_KV_KIVI2, ...).  Other arguments, outputs
 * and rules as kvs_decode_step. */
int kvs_decode_step_kivi(const kvs_shape* shape,
                         const void* q,
                         const void* kv_pool, int64_t pool_blocks,
                         const void* kivi_pool, int64_t kivi_blocks,
                         const int32_t* block_table, int32_t max_blocks_per_seq,
                         const int32_t* seq_lens, const int32_t* quant_lens,
                         const int32_t* meta_offsets,
                         int32_t batch, int64_t total_blocks,
                         int32_t layer_begin, int32_t layer_end,
                         float scale,
                         void* out, float* block_mass, int accumulate,
                         int32_t split_blocks,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/* Initialise records [0, total_blocks): key = {seq_ids[s], b}, score 0,
 * t_touch = KVS_NEVER_TOUCHED, touch_count 0, tier = KVS_UNCLASSIFIED,
 * flags = KVS_FLAG_ANCHOR when b < anchor_blocks, priority 0, reserved 0.
 * seq_ids: uint64 [batch], device.  anchor_blocks >= 0. */
int kvs_meta_init(kvs_block_meta* meta, const int32_t* meta_offsets,
                  const uint64_t* seq_ids, int32_t batch,
                  int32_t max_blocks_per_seq, int64_t total_blocks,
                  int32_t anchor_blocks, void* stream);

/* seq_lens (int32 [batch], device) in kvs_score_update, kvs_classify and
 * kvs_evict_candidates: when non-NULL, only the first ceil(seq_lens[s] / 16)
 * records of each sequence's capacity are live (and nb below is that count);
 * when NULL, every record of the capacity is live. */

/* One scoring step over every record of every sequence in the batch:
 * m_hat = block_mass / max over the sequence's blocks (0 if that max is 0),
 * E <- alpha m_hat + (1 - alpha) E_prev in fp64, where E_prev is the stored
 * score decayed by (1 - alpha)^(step - t_touch - 1) for a record whose last
 * touch is older than the previous step (input 0 on untouched steps;
 * RETRACTIONS, Sec. 3), touch_count += 1, t_touch = step.
 * With classify != 0 also priority and tier (as kvs_classify).  A record whose
 * t_touch is not KVS_NEVER_TOUCHED and >= step is left unchanged
 * (KVS_DEV_STALE_STEP).  workspace: kvs_score_workspace_bytes() bytes. */
int kvs_score_update(kvs_block_meta* meta, const float* block_mass,
                     const int32_t* meta_offsets, const int32_t* seq_lens, int32_t batch,
                     int32_t max_blocks_per_seq, int64_t total_blocks,
                     uint64_t step, const kvs_policy* policy, int classify,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Priority and tier of every record from its current score, without touching
 * it: P = w_recency (b + 1) / nb + w_ema score + w_anchor [flags & ANCHOR],
 * tier = 0 if P >= t_high, 1 if P >= t_low, else 2, where b is the record's
 * logical block and nb its sequence's record count.  Writes priority and tier
 * into the records and, when tiers_out != NULL, tier into tiers_out[record]. */
int kvs_classify(kvs_block_meta* meta, const int32_t* meta_offsets, const int32_t* seq_lens,
                 int32_t batch, int32_t max_blocks_per_seq, int64_t total_blocks,
                 const kvs_policy* policy, uint8_t* tiers_out, void* stream);

/* Workspace bytes kvs_evict_candidates needs (status header + per-chunk partials). */
size_t kvs_evict_workspace_bytes(int32_t batch, int32_t max_blocks_per_seq);

/* Eviction candidate of each sequence at step `now`: the record with the lowest
 * decayed score, where a record's score decays by (1 - alpha) on every step
 * after its last touch (RETRACTIONS, Sec. 3; GQA Per-Head Scoring Streams,
 * panel 3: one ordering per sequence, the coldest block is the candidate).
 * The order is taken on the key K = ln score + t_touch * (-ln(1 - alpha)),
 * which orders records exactly as their decayed scores at any time; a zero
 * score (never attended) ranks lowest.  Ties go to the lowest logical block.
 *  active          uint8 [batch], device, nullable: sequences with 0 get no
 *                  candidate (out_block -1, out_key +inf).
 *  exclude_pinned  1: tier-0 records are never candidates.
 *  out_block       int32 [batch], device: logical block, or -1 if none.
 *  out_key         double [batch], device: the candidate's K, or +inf.
 * Records with t_touch > now are skipped (KVS_DEV_STALE_STEP).  alpha in (0, 1).
 * workspace: kvs_evict_workspace_bytes() bytes, 256-B aligned, header zeroed
 * once by kvs_workspace_init(). */
int kvs_evict_candidates(const kvs_block_meta* meta, const int32_t* meta_offsets,
                         const int32_t* seq_lens, const uint8_t* active, int32_t batch,
                         int32_t max_blocks_per_seq,
                         int64_t total_blocks, uint64_t now, double alpha, int exclude_pinned,
                         int32_t* out_block, double* out_key, void* workspace,
                         size_t workspace_bytes, void* stream);

/* kvs_decode_step over an fp16 pool, with pairs of sequences that share
 * blocks (a prefix cache's refcounted blocks, KV cache offload post, "Top
 * row") decoded by one wave: each block the two hold at the same logical
 * position is read from HBM once and scored for both.  Outputs, block mass
 * and every other argument, size and rule are those of kvs_decode_step, and
 * the results are bit-identical to it whatever the pairing.
 *  pair_role  int32 [batch], device: pair_role[a] = b together with
 *             pair_role[b] = -2 - a links sequences a and b (a != b); -1 marks
 *             an unpaired sequence.  Entries whose partner does not link back
 *             are treated as unpaired.  A split of a linked pair is decoded
 *             jointly when both sequences hold its first block as the same
 *             physical block; other splits are decoded separately.
 *  split_blocks  at most 512 (a paired work-group holds both sequences' mass
 *             partials in LDS); 0 chooses as kvs_decode_split_blocks does for
 *             KVS_KV_FP16, capped at 512.  The workspace must fit
 *             kvs_decode_workspace_bytes(..., KVS_KV_FP16, ..., that split).
 * KVS_E_NULL when pair_role is NULL; KVS_E_RANGE for a split above 512. */
int kvs_decode_step_paired(const kvs_shape* shape,
                           const void* q,
                           const void* kv_pool, int64_t pool_blocks,
                           const int32_t* block_table, int32_t max_blocks_per_seq,
                           const int32_t* seq_lens, const int32_t* pair_role,
                           const int32_t* meta_offsets,
                           int32_t batch, int64_t total_blocks,
                           int32_t layer_begin, int32_t layer_end,
                           float scale,
                           void* out, float* block_mass, int accumulate,
                           int32_t split_blocks,
                           void* workspace, size_t workspace_bytes,
                           void* stream);

/* kvs_decode_step_paired over an FP8 E4M3 pool: the decode of
 * kvs_decode_step_e4m3 with pairs of sequences that share blocks decoded by one
 * wave, one block per step as in kvs_decode_step_paired.  The results are
 * bit-identical to kvs_decode_step_e4m3 whatever the pairing (for finite
 * codes: see the NaN note there).
 * pair_role, split_blocks (at most 512; 0 chooses as kvs_decode_split_blocks
 * does for KVS_KV_E4M3, capped at 256) and every other argument as in
 * kvs_decode_step_paired; the workspace must fit
 * kvs_decode_workspace_bytes(..., KVS_KV_E4M3, ..., that split). */
int kvs_decode_step_e4m3_paired(const kvs_shape* shape,
                                const void* q,
                                const void* kv_pool, int64_t pool_blocks,
                                const int32_t* block_table, int32_t max_blocks_per_seq,
                                const int32_t* seq_lens, const int32_t* pair_role,
                                const int32_t* meta_offsets,
                                int32_t batch, int64_t total_blocks,
                                int32_t layer_begin, int32_t layer_end,
                                float scale,
                                void* out, float* block_mass, int accumulate,
                                int32_t split_blocks,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/* Workspace bytes kvs_append_kv needs (status header + two words per sequence). */
size_t kvs_append_workspace_bytes(int32_t batch);

/* Append one token per sequence to the paged cache (the write that precedes
 * each decode step: generation adds one key and one value per layer per KV head,
 * Fitting a Million Tokens, Sec. 01; fixed-size blocks from a block manager's
 * pool, KV cache offload post, "Top row").  For every sequence s in batch order:
 * the token goes to position t = seq_lens[s], logical block t / 16, slot t % 16.
 * When t % 16 == 0 a block is taken from the top of the free stack -- the k-th
 * sequence (in batch order) that needs one takes free_stack[*free_top - 1 - k] --
 * block_table[s][t / 16] is set and the block's record at meta_offsets[s] + t / 16
 * is created fresh (as kvs_meta_init).  K and V of the token are written to the
 * slot for every layer and KV head; nothing else in the pool changes.  Then
 * seq_lens[s] += 1 and finally *free_top decreases by the blocks taken.
 *  kv_elem_bytes  2: the pool holds fp16 values, 1: E4M3 codes.  k_new and v_new
 *                 are [batch][num_layers][8][128] elements of that format (no
 *                 rounding happens here), device, 16-byte aligned.
 *  free_stack     int32 [free_capacity], device; entries [0, *free_top) are free.
 *  free_top       int32, device, in / out; a value outside [0, free_capacity] is
 *                 clamped into it (KVS_DEV_BAD_OFFSETS).
 *  seq_lens       int32 [batch], device, in / out.
 * A sequence that needs a block when none is left, whose table row or record
 * capacity is full, is left unchanged (KVS_DEV_POOL_EXHAUSTED).  The partial
 * tail block a token is written into must belong to that sequence alone: the
 * library keeps no reference counts, so a tail block shared with another
 * table (a shared prefix that ends inside a block) would change under it.
 * Shared prefixes therefore cover whole blocks.
 * workspace: kvs_append_workspace_bytes() bytes. */
int kvs_append_kv(const kvs_shape* shape, int kv_elem_bytes,
                  const void* k_new, const void* v_new,
                  void* kv_pool, int64_t pool_blocks,
                  int32_t* block_table, int32_t max_blocks_per_seq,
                  int32_t* seq_lens,
                  const int32_t* free_stack, int32_t free_capacity, int32_t* free_top,
                  kvs_block_meta* meta, const int32_t* meta_offsets, const uint64_t* seq_ids,
                  int32_t anchor_blocks, int32_t batch, int64_t total_blocks,
                  void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVS_H */
