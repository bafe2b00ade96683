/*
 * mab.h -- C ABI of the mixed-batch attention library for a paged,
 * block-quantized KV cache (AMD Instinct MI355X, gfx950).
 *
 * Source of the operations: the MBufo page "自研RDNA高併發推論引擎 以AI Max+ 395為範例"
 * (lcz.me, topic 2938).
 *   - Section 1 ("高併發（架構差異）"): the rows of one bounded prefill chunk and
 *     all due single-token decode rows share one ForwardBatch and one attention
 *     kernel, so the prefill tick also emits every decoder's token.
 *   - Section 2 ("提供更多壓縮精度（成本差異）"), KV modes table: q8 keeps one f16
 *     scale per 32 elements (34-byte blocks); the 4-bit modes pack 32 values into
 *     18-byte blocks; blocked modes are bit-exact at the codec level.
 *   - Section 2, occupancy table ("佔用"): bytes per position 1088 (q8) and 576
 *     (K4V4) at 4 KV heads x 128 dims.
 *
 * Conventions for every function below:
 *   - Pointers without a "_host" suffix are DEVICE pointers (HIP device memory
 *     of the current device); "_host" pointers are host memory read during the
 *     call only.  The library allocates nothing, keeps no state between calls,
 *     never synchronizes the stream and never prints, aborts or throws.
 *   - "stream" is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     on it and the call returns at once; results are ready when the stream
 *     reaches that point.  Calls on one stream run in order.
 *   - Errors detectable on the host are returned as a non-zero status before
 *     anything is enqueued (see mab_status_string).  Device arrays must hold
 *     the same values as their host mirrors; block-table entries must be valid
 *     page ids in [0, num_pages) for every page a sequence uses.  Violating
 *     either is undefined behaviour on the device (not detected).
 *
 * Data layout (all little-endian, tightly packed, C order):
 *   block   : 32 consecutive head_dim values of one token and one KV head:
 *             bytes [0,2) = fp16 scale d; then the codes.
 *             q8 (34 B): 32 two's-complement int8 codes.
 *             q4 (18 B): 16 bytes, byte j = code 2j (low nibble) | code 2j+1
 *                        (high nibble), two's-complement nibbles.
 *             f16 (64 B): the unquantized mode of the same table: the 32
 *                        values as little-endian IEEE halves, no scale.
 *             value = code * d.  Encoding: s = fl32(max|x| / Q) (Q = 127 or 7,
 *             IEEE binary32 divide), code = clamp(rint_even(fl32(x / s)), -Q, Q),
 *             d = fp16 round-to-nearest-even of s (no flush); all-zero block:
 *             d = +0, codes 0.
 *   pool    : uint8 [num_pages][num_kv_heads][page_size][head_dim/32][B],
 *             one pool for K (k_format) and one for V (v_format).
 *   token t of sequence s lives in page block_table[s*max_pages_per_seq + t/page_size],
 *             slot t % page_size.
 *   q       : fp16 [num_rows][num_q_heads][head_dim]
 *   k_new/v_new : fp16 [num_rows][num_kv_heads][head_dim]
 *   out     : fp32 [num_rows][num_q_heads][head_dim]
 *   batch   : the rows of sequence s are [q_start[s], q_start[s+1]); row i of s
 *             sits at position prefix_len[s] + i and attends keys 0 .. that
 *             position of s (full over the cached prefix, causal inside the
 *             rows of s).  A decode row is a sequence with one row; its
 *             context is prefix_len + 1.  Query head h reads KV head
 *             h / (num_q_heads / num_kv_heads).
 *
 * Supported shapes (others return MAB_ERR_UNSUPPORTED or MAB_ERR_SHAPE):
 *   head_dim in {64, 128}; num_q_heads % num_kv_heads == 0 with a group of at
 *   most 8 query heads per KV head; page_size a positive multiple of 16;
 *   1 <= rows per sequence; num_seqs <= 4096; all buffers 16-byte aligned;
 *   k_format and v_format both MAB_KV_F16 or neither.
 */
#ifndef MAB_H
#define MAB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum {
  MAB_OK = 0,
  MAB_ERR_NULL = 1,        /* a required pointer is NULL                       */
  MAB_ERR_SHAPE = 2,       /* a layout or batch field breaks a stated rule     */
  MAB_ERR_UNSUPPORTED = 3, /* well-formed but outside the supported shapes     */
  MAB_ERR_WORKSPACE = 4,   /* workspace smaller than attention_workspace_bytes */
  MAB_ERR_ALIGN = 5,       /* a device buffer is not 16-byte aligned           */
  MAB_ERR_HIP = 6,         /* the HIP runtime refused a kernel launch          */
  MAB_ERR_QUOTA = 7,       /* mab_sched_submit: the client's pending cap is full */
  MAB_ERR_SCRATCH = 8      /* mixed_attention_fwd_noalloc: the batch needs more
                              than MAB_NOALLOC_SCRATCH_BYTES of workspace      */
};

/* KV block formats (MBufo page, section 2 modes table and occupancy table). */
enum {
  MAB_KV_Q8 = 1,  /* 34-byte block: fp16 scale + 32 x int8            */
  MAB_KV_Q4 = 2,  /* 18-byte block: fp16 scale + 16 bytes of 32 x int4 */
  MAB_KV_F16 = 3  /* 64-byte block: 32 x fp16, unquantized (K and V both f16 only) */
};

/* Shape of the cache and of the attention heads. */
typedef struct mab_kv_layout {
  int32_t num_q_heads;  /* Hq                                    */
  int32_t num_kv_heads; /* Hkv; Hq % Hkv == 0                    */
  int32_t head_dim;     /* D                                     */
  int32_t page_size;    /* tokens per page                       */
  int32_t num_pages;    /* pages in each pool                    */
  int32_t k_format;     /* MAB_KV_Q8, MAB_KV_Q4 or MAB_KV_F16    */
  int32_t v_format;     /* same; f16 only together with f16      */
  int32_t reserved;     /* must be 0                             */
} mab_kv_layout;

/* Batch flags.
 *
 * MAB_BATCH_INVARIANT: every decode and verify row (a sequence of at most 16
 * rows) gives bit-identical outputs whatever else shares the batch, as the
 * MBufo page's three-numbers table (greedy output bit-identical) and the
 * fairness part of its section 1 (a prompt checked by hash alone and under
 * load) ask of a serving engine.  Without it, the keys of all decode rows are
 * cut into equal ranges per wave across the whole batch, so a row's split
 * points, and with them its fp32 rounding (within 1e-3 of the output), depend
 * on the other rows; with it, each row's keys are cut into pieces of
 * MAB_INVARIANT_PIECE_KEYS from its own first key and each piece runs on its
 * own wave.  Prefill-chunk rows are batch-independent either way: their key
 * splits depend only on their own tile count and the device's compute-unit
 * count.  The grouping of a verify row's tokens depends only on its own
 * length and the layout.  Cost on one MI355X: about +26% on a batch of 16
 * short decode rows, +25% on 4-token verify rows, nothing on single long
 * rows. */
enum { MAB_BATCH_INVARIANT = 1 };
#define MAB_INVARIANT_PIECE_KEYS 512

/* One ForwardBatch: chunk rows and decode rows together (MBufo page, section 1). */
typedef struct mab_batch {
  int32_t num_seqs;          /* S                                                 */
  int32_t num_rows;          /* total query rows = q_start[S]                     */
  int32_t max_pages_per_seq; /* row stride of block_table                         */
  int32_t flags;             /* 0, or MAB_BATCH_INVARIANT                         */
  const int32_t* q_start;         /* device [S+1], q_start[0] = 0, non-decreasing */
  const int32_t* prefix_len;      /* device [S], cached positions before the rows */
  const int32_t* block_table;     /* device [S * max_pages_per_seq] page ids      */
  const int32_t* q_start_host;    /* host mirror of q_start                       */
  const int32_t* prefix_len_host; /* host mirror of prefix_len                    */
} mab_batch;

/* Bytes of one 32-value block of `format` (34, 18 or 64); 0 for an unknown format. */
int32_t kv_block_bytes(int32_t format);

/* Bytes of one pool of `format` for `layout`:
 * num_pages * num_kv_heads * page_size * (head_dim/32) * kv_block_bytes(format).
 * Returns -1 if the layout is invalid. */
int64_t kv_pool_bytes(const mab_kv_layout* layout, int32_t format);

/* Device workspace that mixed_attention_fwd needs for this batch (split-K
 * partial results and small per-row tables).  Computed from the host mirrors
 * and the current device's compute-unit count (the work is cut to fill that
 * device), so query it on the device the call will run on.
 * Returns a negative status (-MAB_ERR_*) if the layout or batch is invalid. */
int64_t attention_workspace_bytes(const mab_kv_layout* layout, const mab_batch* batch);

/* kv_append_quant: quantize the step's new keys and values into the cache.
 *
 * Operation (MBufo page, section 2 modes table, codec as in the header
 * comment): for every row i of sequence s, every KV head g and every 32-value
 * block b, encode k_new[row][g][32b .. 32b+31] into the k_format block at
 * position prefix_len[s] + i of sequence s, and likewise v_new into the
 * v_format pool.  Bytes written are bit-identical to the stated encoding.
 * Only the blocks of the batch's rows are written; nothing else in the pools
 * changes.  Call it before mixed_attention_fwd in the same step: attention
 * reads every key, the rows' own included, from the cache.
 *
 * k_new, v_new : device fp16 [num_rows][Hkv][D], read only.
 * k_pool, v_pool : device pools (layout above), written in place.
 * Rows of one call must not target the same position twice. */
int32_t kv_append_quant(const mab_kv_layout* layout, const mab_batch* batch,
                        const void* k_new, const void* v_new,
                        void* k_pool, void* v_pool, void* stream);

/* mixed_attention_fwd: one attention step of a mixed batch over the cache.
 *
 * Operation (MBufo page, section 1: chunk and decode rows in one ForwardBatch
 * and one attention kernel): for each row r of sequence s at position
 * t = prefix_len[s] + (r - q_start[s]) and each query head h with KV head
 * g = h / (Hq/Hkv),
 *     z_j = sm_scale * <q[r][h], K_hat[s][j][g]>,  j = 0 .. t
 *     out[r][h] = sum_j softmax(z)_j * V_hat[s][j][g]
 * where K_hat, V_hat are the dequantized cache blocks.  Arithmetic: fp16
 * operands on the matrix cores with fp32 accumulation, fp32 online softmax,
 * split-K over key ranges merged by log-sum-exp in fixed order.  The result
 * is deterministic (bit-identical run to run) and independent of the
 * physical page ids.  Sequences of more than 16 rows (prefill chunks) get
 * results that are also bit-identical whatever else shares the batch.  Shorter
 * sequences (decode rows, and verify rows of 2-16 tokens, which run on the
 * decode path in groups of 16/G rows, G = Hq/Hkv, or of 32/G rows over
 * quantized pools when the sequence has more than 16/G rows) have their key
 * ranges cut according to the whole batch, so they may differ in the last
 * bits (within 1e-3 at unit-scale values) between different batches.
 *
 * q          : device fp16 [num_rows][Hq][D], read only.
 * k_pool, v_pool : device pools, read only.
 * sm_scale   : softmax scale (typically 1/sqrt(D)); must be positive and
 *              finite (MAB_ERR_UNSUPPORTED otherwise).
 * out        : device fp32 [num_rows][Hq][D], fully written.
 * workspace  : device scratch of at least attention_workspace_bytes() bytes,
 *              owned by the caller; contents need not be initialized and are
 *              clobbered.  Concurrent calls need distinct workspaces. */
int32_t mixed_attention_fwd(const mab_kv_layout* layout, const mab_batch* batch,
                            const void* q, const void* k_pool, const void* v_pool,
                            float sm_scale, float* out,
                            void* workspace, int64_t workspace_bytes, void* stream);

/* mixed_attention_fwd_timed: mixed_attention_fwd (same operation, arguments,
 * results and errors) that also times its attention kernel, for measurement:
 * kernel_start and kernel_stop are hipEvent_t handles (created by the caller,
 * on the stream's device) that take the attention kernel's own start and end
 * timestamps (the kernel is launched through hipExtLaunchKernel), so that
 * hipEventElapsedTime(kernel_start, kernel_stop) is that kernel's execution
 * time, without the merge kernels of the same call.  Either handle may be
 * NULL (not recorded).  A call that returns an error before enqueueing
 * anything records neither. */
int32_t mixed_attention_fwd_timed(const mab_kv_layout* layout, const mab_batch* batch,
                                  const void* q, const void* k_pool, const void* v_pool,
                                  float sm_scale, float* out,
                                  void* workspace, int64_t workspace_bytes, void* stream,
                                  void* kernel_start, void* kernel_stop);

/* mixed_attention_fwd_noalloc: mixed_attention_fwd for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same operation, arguments, results and
 * determinism as mixed_attention_fwd; the workspace is instead a fixed array
 * of MAB_NOALLOC_SCRATCH_BYTES owned by the library, one per device, which
 * each device that runs the call holds until the process ends.  The call
 * allocates nothing (the array's device address is looked up once per
 * device, on the first call with that device current).
 *
 * The caller still owns q, the pools and out.  A batch whose
 * attention_workspace_bytes() exceeds MAB_NOALLOC_SCRATCH_BYTES returns
 * MAB_ERR_SCRATCH before anything is enqueued.  The array needs no
 * initialisation and keeps whatever the last call left in it.  Every call on
 * one device shares that device's array: calls that may overlap on one
 * device (several streams, several host threads) race and give undefined
 * results; serialise them, or use mixed_attention_fwd with distinct
 * workspaces. */
#define MAB_NOALLOC_SCRATCH_BYTES (128LL << 20)
int32_t mixed_attention_fwd_noalloc(const mab_kv_layout* layout, const mab_batch* batch,
                                    const void* q, const void* k_pool, const void* v_pool,
                                    float sm_scale, float* out, void* stream);

/* Static English text for a status code (never NULL). */
const char* mab_status_string(int32_t status);

/* mab_debug_status: the device-side check of page ids (the block table's
 * values, which the host cannot see).
 *
 * With MAB_DEBUG=1 in the environment of the calling process (read at each
 * kv_append_quant / mixed_attention_fwd call), every page id the kernels read
 * from the block table is checked against [0, num_pages); an id outside it
 * sets a flag on the current device and page 0 is read or written instead,
 * so the kernels never leave the pools (the results of the affected rows are
 * then meaningless).  Without MAB_DEBUG=1 page ids are trusted and an invalid
 * one is undefined behaviour.
 *
 * Returns 1 if the flag is set, 0 if not, or -MAB_ERR_HIP if the device could
 * not be read.  reset != 0 clears the flag after reading.  Synchronous: waits
 * for all work on the current device first (every stream).  A debugging aid:
 * the pages define no error reporting of their own. */
int32_t mab_debug_status(int32_t reset);

/* ------------------------------------------------------------------------
 * Measurement probes.  No passage of the pages defines them: they measure
 * what this device reaches on plain work, the realism lines beside the
 * roofline fractions of the attention calls.  Both enqueue one kernel on
 * `stream` and return at once.
 * ---------------------------------------------------------------------- */

/* Reads `bytes` (a multiple of 16, >= 16) of device memory at `buf` (16-byte
 * aligned) once, with 16-byte non-temporal loads, eight 256-thread
 * work-groups per compute unit, sixteen loads in flight per thread.  `sink`:
 * 16 bytes of device memory (16-byte aligned), practically never written.  Time it
 * with events on `stream`; bytes / time is the device's stream-read rate.
 * Returns MAB_OK, MAB_ERR_NULL, MAB_ERR_SHAPE, MAB_ERR_ALIGN or MAB_ERR_HIP. */
int32_t mab_probe_stream_read(const void* buf, int64_t bytes, void* sink, void* stream);

/* Runs `iters` (>= 1) rounds of eight independent 16x16x32 fp16 matrix-core
 * products per wave, two 4-wave work-groups per compute unit.  `sink`: 16
 * bytes of device memory (16-byte aligned), practically never written.
 * Returns the flops enqueued (2*16*16*32 per product), or a negative status. */
int64_t mab_probe_mfma_f16(int32_t iters, void* sink, void* stream);

/* ------------------------------------------------------------------------
 * Step scheduler and batch builder (host only; no device memory).
 *
 * Decides each engine tick's rows and writes the tick's batch descriptor,
 * following the scheduler rules of the MBufo page, section 1: the table of
 * scheduler guarantees and the fairness part (SRTF, starving-decode
 * preemption, near-done gate).
 *
 *  - Admission: pending requests take free session slots, clients taking
 *    turns (FIFO within a client).  A request reserves its KV pages,
 *    ceil((prompt_len + token_limit - 1) / page_size), at admission: the
 *    lowest-numbered free pages.  Admission stops at the first request that
 *    does not fit.
 *  - Decode first: while some decoder is due, a tick is a decode step over
 *    the due decoders in queue order.  Otherwise it is a merged step: one
 *    prefill chunk slice of at most prefill_chunk tokens plus the decoders
 *    at the head of the queue.  Either way a tick serves at most
 *    max_decode_rows decoders.
 *  - Served decoders move to the back of the queue (PopDecoder rotation).
 *    After a merged step every resident decoder is due
 *    (MarkAllDecodersDue).
 *  - The chunk goes to the prefill that needs the fewest chunk slices to
 *    finish, ceil(remaining / prefill_chunk), the earliest request among
 *    equal counts (SRTF): a prefill with one slice left goes before every
 *    longer one.  While a request waits for a slot and some decoder is within
 *    near_done_gate tokens of its limit, prefills with more than one slice
 *    left get no chunk.
 *
 * Positions: a chunk row covers prompt positions [prefix, prefix + q_len).
 * A decoder that has produced g tokens feeds token g: one row with
 * prefix_len = prompt_len + g - 1.  The last chunk of a prompt yields the
 * request's first token.  A request that has produced token_limit tokens is
 * finished, and its slot and pages are released at the end of that tick.
 * ---------------------------------------------------------------------- */

typedef struct mab_sched_config {
  int32_t sessions;               /* resident requests at most (session slots), >= 1      */
  int32_t prefill_chunk;          /* tokens of one prefill chunk slice at most, >= 1      */
  int32_t max_pending_per_client; /* waiting requests per client at most, >= 1           */
  int32_t near_done_gate;         /* tokens left that make a decoder "near done", >= 0   */
  int32_t max_decode_rows;        /* decoders served per tick at most; 0: sessions       */
  int32_t page_size;              /* tokens per KV page (the layout's page_size), >= 1    */
  int32_t num_pages;              /* pages in the pool (the layout's num_pages), >= 1     */
  int32_t max_pages_per_seq;      /* block-table row width, >= 1                          */
} mab_sched_config;

typedef struct mab_sched mab_sched; /* opaque; owned by the caller via create/destroy */

typedef struct mab_step_info {
  int32_t kind;     /* 0: nothing to run, 1: decode step, 2: merged step      */
  int32_t num_seqs; /* sequences written to the step arrays                   */
  int32_t num_rows; /* query rows = q_start[num_seqs]                         */
  int32_t pending;  /* requests still waiting for a slot after this tick      */
} mab_step_info;

/* Creates a scheduler with every page free.  *out receives it (NULL on
 * error).  Returns MAB_ERR_NULL or MAB_ERR_SHAPE (a field out of range). */
int32_t mab_sched_create(const mab_sched_config* cfg, mab_sched** out);

/* Frees a scheduler (NULL is allowed). */
void mab_sched_destroy(mab_sched* s);

/* Queues a request: client id >= 0, prompt_len >= 1 tokens, token_limit >= 1
 * tokens to produce.  *request_id receives its id (0, 1, 2, ... in submit
 * order) or -1.  MAB_ERR_SHAPE: a field out of range, positions past int32
 * (prompt_len + token_limit - 1 > INT32_MAX), or a request that could never
 * fit (more pages than max_pages_per_seq or num_pages).
 * MAB_ERR_QUOTA: the client already has max_pending_per_client requests
 * waiting. */
int32_t mab_sched_submit(mab_sched* s, int32_t client, int32_t prompt_len, int32_t token_limit,
                         int64_t* request_id);

/* Runs one tick: admission, then the step's choice, then the state update
 * (the step is taken as run).  Host arrays of `capacity` sequences, capacity
 * >= max_decode_rows + 1 (MAB_ERR_SHAPE otherwise):
 *   request_id[capacity], prefix_len[capacity], emit[capacity],
 *   finished[capacity], q_start[capacity + 1],
 *   block_table[capacity * max_pages_per_seq] (row-major, padded with -1).
 * Sequences are the decoders in the order served (q_len 1), then the chunk
 * slice if any.  emit[i] = 1 when row i's step yields a token of its request,
 * finished[i] = 1 when that request is done.  q_start, prefix_len and
 * block_table are the mab_batch fields of the step (copy them to the device
 * for kv_append_quant and mixed_attention_fwd).  kind 0 writes only
 * q_start[0] = 0. */
int32_t mab_sched_step(mab_sched* s, mab_step_info* info, int64_t* request_id, int32_t* q_start,
                       int32_t* prefix_len, int32_t* block_table, int32_t* emit, int32_t* finished,
                       int32_t capacity);

#ifdef __cplusplus
}
#endif

#endif /* MAB_H */
