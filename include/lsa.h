/*
 * liblsa -- the per-decode-step hot path of Lookahead Sparse Attention (LSA)
 * and of the KV swap around it, for AMD Instinct MI355X (gfx950).
 *
 * One decode step is: score every compressed indexer key with the memory
 * indexers (lsa_score), keep the query-critical chunks (lsa_select), stage
 * them into a bounded slot pool managed as an LRU over a larger cold pool
 * (lsa_stage), and attend over a sliding window plus the staged entries
 * (lsa_attend).  lsa_decode_step chains the four for a stack of sparse layers.
 *
 * Sources (cited by title and section; the pages are public web text):
 *   [P1] PocketLLM, "FlashMemory 1M 上下文显存优化使用文档": overview (two-tier
 *        KV cache), configuration flags, GPU_CHUNKS / PINNED_MIB tuning
 *        (closed-form sizing), expected logs, troubleshooting (errors 1-4,
 *        swap auto-disable), technical details (architecture, memory layout,
 *        GgufKvSwapLayerState, swap-in and store flows).
 *   [P2] article on "FlashMemory-DeepSeek-V4: Lightning Index Ultra-Long
 *        Context via Lookahead Sparse Attention": LSA section (memory indexer
 *        queries vs compressed indexer keys; sigmoid threshold selector), the
 *        placement section (three indexers, OR-mode routing).
 *   [P4] "KVSwap：大模型推理中的KV缓存优化技术": §2.2 grouped KV prediction,
 *        §2.3 low-rank K, §3.2 ring buffer of 400 groups.
 *
 * Conventions for every entry point:
 *   - Pointers documented "device" are HBM addresses on the current HIP device
 *     (e.g. torch tensors' data_ptr()); "host" pointers are ordinary CPU memory.
 *     The caller owns every pointer it passes; liblsa owns only what its own
 *     *_create functions allocate (context workspace, pool tables, cold pools).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns; outputs are valid once that stream has synchronised.
 *     Counts produced on the device stay on the device.
 *   - Every call returns an lsa_status.  On failure nothing is enqueued and
 *     lsa_last_error() (thread-local) holds a one-line explanation.
 *   - No entry point calls hipMalloc/hipFree on the step path, except that a
 *     context grows its workspace the first time a larger problem is seen
 *     (lsa_ctx_reserve pre-sizes it).
 *   - Scores must not be NaN.  Arguments outside the documented ranges return
 *     LSA_ERR_INVALID_ARG, unsupported shapes LSA_ERR_UNSUPPORTED.
 */
#ifndef LSA_H
#define LSA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LSA_ABI_VERSION 7
#define LSA_MAX_LAYERS 64
#define LSA_MAX_BATCH 64

typedef enum lsa_status {
    LSA_OK = 0,
    LSA_ERR_INVALID_ARG = 1,
    LSA_ERR_SLOTS_LT_TOPK = 2,   /* [P1] error 2: GPU_CHUNKS must be >= index_topk */
    LSA_ERR_PINNED_CAP = 3,      /* [P1] error 3: pinned cache exceeds cap */
    LSA_ERR_NOT_STORED = 4,      /* [P1] error 4: selected chunk before it was stored */
    LSA_ERR_HIP = 5,             /* a HIP runtime call failed */
    LSA_ERR_NO_MEMORY = 6,       /* device or pinned allocation failed */
    LSA_ERR_UNSUPPORTED = 7      /* a valid shape this build has no kernel for */
} lsa_status;

/* Key-only formats.  [P1] technical details (memory layout and known limits):
 * the indexer keys are fp4 today, and fp8/int8 keys are the way to shrink the
 * resident key cache.
 *   LSA_FP8_E4M3  OCP E4M3: 1 sign, 4 exponent bits with bias 7, 3 mantissa
 *                 bits, subnormals, no infinities, codes 0x7F / 0xFF NaN.
 *   LSA_MXFP4     OCP MX FP4: E2M1 codes (1 sign, 2 exponent bits with bias 1,
 *                 1 mantissa bit: +-{0, .5, 1, 1.5, 2, 3, 4, 6}), two per byte,
 *                 element 2i in bits 0-3 of byte i.
 *   LSA_MXINT8    OCP MX INT8: two's-complement int8 codes with an implicit
 *                 scale of 2^-6 (value code/64).
 * The MX formats carry one E8M0 scale (unsigned byte s, value 2^(s-127); 255
 * is NaN and not allowed) per 32 consecutive elements of a key. */
typedef enum lsa_dtype {
    LSA_F32 = 0, LSA_BF16 = 1, LSA_F16 = 2, LSA_FP8_E4M3 = 3, LSA_MXFP4 = 4, LSA_MXINT8 = 5
} lsa_dtype;
typedef enum lsa_ensemble { LSA_ENSEMBLE_MAX = 0, LSA_ENSEMBLE_MEAN = 1 } lsa_ensemble;
typedef enum lsa_select_mode { LSA_SELECT_TOPK = 0, LSA_SELECT_THRESHOLD = 1 } lsa_select_mode;
typedef enum lsa_cold_kind { LSA_COLD_HBM = 0, LSA_COLD_HOST = 1 } lsa_cold_kind;

typedef void* lsa_stream_t; /* hipStream_t */

/* ----------------------------------------------------------- closed forms --
 * [P1] PINNED_MIB tuning: compressed_cap = (context_length + ratio - 1) / ratio;
 * required pinned bytes = sum over sparse layers of compressed_cap * kv_dim *
 * sizeof(element).  [P1] expected logs: max_capacity = window + gpu_chunks.
 * Invalid arguments (ctx < 0, ratio <= 0, ...) give 0 / -1. */
int64_t  lsa_compressed_cap(int64_t ctx, int32_t ratio);
uint64_t lsa_pinned_bytes(int64_t ctx, const int32_t* ratios /* host [n_layers] */,
                          int32_t n_layers, int32_t kv_dim, lsa_dtype dtype);
int32_t  lsa_max_capacity(int32_t window, int32_t gpu_chunks);
/* [P1] PINNED_MIB: LSA_ERR_PINNED_CAP, with "required_mib=X cap_mib=Y" in
 * lsa_last_error(), when the layers' pinned bytes exceed cap_bytes. */
lsa_status lsa_check_pinned(int64_t ctx, const int32_t* ratios, int32_t n_layers, int32_t kv_dim,
                            lsa_dtype dtype, uint64_t cap_bytes);
/* logit threshold used by threshold selection: the largest float t_f with
 * t_f <= ln(tau / (1 - tau)); an entry passes when score > t_f, i.e. exactly
 * when sigmoid(score) > tau over the reals.  NaN for tau outside (0, 1). */
float lsa_threshold_logit(double tau);

const char* lsa_status_string(lsa_status s);
const char* lsa_last_error(void);
int32_t     lsa_abi_version(void);

/* ---------------------------------------------------------------- context --
 * Owns the device workspace of lsa_select / lsa_attend / lsa_decode_step and
 * optional per-kernel timing events.  One context per device and thread of
 * use; calls on one context must not overlap.  `device` becomes current. */
typedef struct lsa_ctx lsa_ctx;
lsa_status lsa_ctx_create(lsa_ctx** out, int32_t device);
void       lsa_ctx_destroy(lsa_ctx* ctx);
lsa_status lsa_ctx_reserve(lsa_ctx* ctx, uint64_t bytes);

/* Kernel timing: when on, lsa_decode_step / lsa_score / lsa_attend record HIP
 * events around their launches on the launch stream.  lsa_ctx_timing_read
 * waits for the last event, returns for each kernel kind (LSA_K_*) the summed
 * milliseconds and launch count since the previous read, and resets them.
 * LSA_K_STAGE covers the LRU update together with the copy of missed rows;
 * LSA_K_GATHER is kept for layout and reads 0. */
enum { LSA_K_SCORE = 0, LSA_K_SELECT = 1, LSA_K_STAGE = 2, LSA_K_GATHER = 3,
       LSA_K_ATTEND = 4, LSA_K_COMBINE = 5, LSA_K_COUNT = 6 };
lsa_status lsa_ctx_set_timing(lsa_ctx* ctx, int32_t on);
lsa_status lsa_ctx_timing_read(lsa_ctx* ctx, double* ms /* host [LSA_K_COUNT] */,
                               int64_t* launches /* host [LSA_K_COUNT] */);

/* Cache policy of the indexer keys in the step calls of this context
 * (lsa_decode_step, lsa_decode_step_noalloc, lsa_lookahead_prime,
 * lsa_lookahead_step).  [P1] limitations and future work, items 1-2: the keys of
 * the whole context stay in device memory and every step reads all of them.
 * non_temporal = 0 (the default): the default policy, so that keys read again
 * at the next step may still be in the last-level cache (a loop over one
 * indexer layer).  non_temporal != 0: the non-temporal policy, which lsa_score
 * always uses; it streams keys that other work evicts between steps (a model's
 * other layers) faster and keeps them from displacing what the caches hold.
 * Scores, selections and outputs do not depend on it.  Takes effect at the
 * next call; LSA_ERR_INVALID_ARG for a NULL ctx. */
lsa_status lsa_ctx_set_key_policy(lsa_ctx* ctx, int32_t non_temporal);

/* ------------------------------------------------------------- projection --
 * [P1] architecture overview: the decode token's hidden state (hidden[4096])
 * feeds the three scorers.  Each indexer i maps it linearly to its query heads
 * and head weights, the (q, w) that lsa_score takes:
 *     q[b,i,h,t] = sum_c wq[i,h,t,c] * hidden[b,c]
 *     w[b,i,h]   = sum_c ww[i,h,c]   * hidden[b,c]
 * Accumulation is fp32 in an unspecified order, so the result is exact
 * whenever every partial sum is representable in fp32.
 *   hidden  device f32 [batch][d_model], finite, 16-byte aligned
 *   wq      device [n_idx][heads][dk][d_model], w_dtype LSA_F32 or LSA_BF16
 *   ww      device [n_idx][heads][d_model], same dtype
 *   q       device f32 [batch][n_idx][heads][dk]
 *   w       device f32 [batch][n_idx][heads]
 * Supported: d_model a multiple of 8 and at most 16384; 1 <= batch <=
 * LSA_MAX_BATCH; n_idx * heads * (dk + 1) < 2^31.  Weight rows are read once
 * per four sequences. */
lsa_status lsa_project(const float* hidden, int32_t batch, int32_t d_model, const void* wq, const void* ww,
                       lsa_dtype w_dtype, int32_t n_idx, int32_t heads, int32_t dk, float* q, float* w,
                       lsa_stream_t stream);

/* ------------------------------------------------------------------ score --
 * [P1] architecture: 3 scorers read the shared indexer keys and are combined
 * by an ensemble (FLASHMEMORY_ENSEMBLE=max|mean); [P2] LSA section: memory
 * indexer queries are matched against the compressed indexer keys by dot
 * product.  For every sequence b and valid entry j < n_valid[b]:
 *     s_i[j]   = sum_h w[b,i,h] * ReLU( q[b,i,h,:] . keys[b,j,:] )   (fp32)
 *     score[j] = max_i s_i[j]                (LSA_ENSEMBLE_MAX), or
 *                fl(sum_i s_i[j]) / n_idx    (LSA_ENSEMBLE_MEAN: the float s_i added
 *                                             in double in indexer order, rounded
 *                                             once to float, one IEEE division)
 * with -0 written as +0.  Accumulation is fp32 in an unspecified order, so the
 * result is exact whenever every partial sum is representable in fp32.  Keys
 * of every dtype enter as their exact values (an fp8 code decodes exactly, an
 * MX element is its code times its block scale), and each product with the
 * fp32 query is exact before the accumulation.
 *   keys   device [batch][n_keys][dk] elements, rows contiguous, key_dtype
 *          LSA_F32, LSA_BF16, LSA_FP8_E4M3 (one byte per element), LSA_MXFP4
 *          (dk/2 bytes per key) or LSA_MXINT8 (dk bytes); NaN codes are not
 *          allowed
 *   key_scales  device u8 [batch][n_keys][dk/32] E8M0 block scales for the MX
 *          dtypes, with 2 <= s <= 252 (every scaled element then is a bf16
 *          normal or zero); ignored (may be NULL) otherwise
 *   n_valid host [batch] (0 <= n_valid[b] <= n_keys) or NULL for n_keys each
 *   q      device f32 [batch][n_idx][heads][dk]
 *   w      device f32 [batch][n_idx][heads]
 *   scores device f32 [batch][n_keys]; entries j >= n_valid[b] are not written
 * Supported: dk in {32, 64, 128} (64 or 128 for LSA_MXFP4); 1 <= n_idx <= 4; 1 <= heads <= 8;
 * 1 <= batch <= LSA_MAX_BATCH; n_keys * dk * sizeof(key) < 2^32 per sequence.
 * The keys are read with the non-temporal cache policy (one pass that streams
 * them); the step calls, which read the same keys at every step, read them with
 * the default policy so that they may stay in the last-level cache.  The
 * scores do not depend on the policy. */
lsa_status lsa_score(const void* keys, lsa_dtype key_dtype, const uint8_t* key_scales, int32_t batch, int64_t n_keys,
                     const int64_t* n_valid, int32_t dk, const float* q, const float* w,
                     int32_t n_idx, int32_t heads, lsa_ensemble ensemble, float* scores,
                     lsa_stream_t stream);

/* ----------------------------------------------------------------- select --
 * [P1] "global top-k (512 chunks)" with index_topk = global_keep_cap; [P2]
 * Recall / Threshold Selector: recall entries whose sigmoid(score) exceeds
 * tau.  Order: higher score first, lower index first among equal scores
 * (+0 and -0 are equal).
 *   LSA_SELECT_TOPK:      the first min(k, n_valid) entries of that order;
 *   LSA_SELECT_THRESHOLD: the entries with sigmoid(score) > tau (computed as
 *                         score > lsa_threshold_logit(tau)); if more than k
 *                         pass, the first k of them in the order.
 *   scores device f32 [n_seg][n_keys]; n_valid host [n_seg] or NULL (for
 *          n_seg > LSA_MAX_BATCH the values must all be equal)
 *   sel    device i32 [n_seg][k]: selected indices ascending, then -1 padding
 *   count  device i32 [n_seg]: number selected
 * Supported: 1 <= k <= 4096, n_seg >= 1, n_keys <= 2^31 - 1 and
 * ceil(n_keys / 32768) * k <= 32768; tau in (0, 1) for threshold mode. */
lsa_status lsa_select(lsa_ctx* ctx, const float* scores, int32_t n_seg, int64_t n_keys,
                      const int64_t* n_valid, lsa_select_mode mode, int32_t k, double tau,
                      int32_t* sel, int32_t* count, lsa_stream_t stream);

/* ------------------------------------------------------------------ pools --
 * [P1] technical details, GgufKvSwapLayerState and swap-in flow: per sparse
 * layer, all compressed rows live in a cold pool ([P1]: pinned host; here also
 * HBM) and `gpu_chunks` GPU slots stage the selected ones, managed as an LRU.
 * One pool serves one sparse layer for `batch` independent sequences.
 *
 * kv_buf is the caller's device buffer [batch][lsa_pool_rows(desc)][kv_dim]
 * (sequence b at element offset b * kv_stride_b): rows 0..window-1 hold the
 * sliding window (the caller writes them), the rest are slots.  A layer with
 * compressed_cap <= gpu_chunks is fully resident ([P1] troubleshooting,
 * swap auto-disable): its rows window + j hold entry j and nothing swaps.
 *
 * lsa_pool_create errors: gpu_chunks < topk without allow_topk_reduction ->
 * LSA_ERR_SLOTS_LT_TOPK ([P1] error 2); a host cold pool above
 * pinned_cap_bytes (0 = no cap) -> LSA_ERR_PINNED_CAP ([P1] error 3).
 * With allow_topk_reduction and gpu_chunks < topk, at most gpu_chunks chunks
 * may be staged per step ([P1] TEST_ALLOW_TOPK_REDUCTION). */
typedef struct lsa_pool_desc {
    int64_t ctx;                /* context length in tokens */
    int32_t ratio;              /* this layer's compression ratio (a multiple of the source ratio) */
    int32_t window;             /* sliding-window rows, [P1]: 128 */
    int32_t gpu_chunks;         /* staging slots S, [P1]: 512 or 1024; S >= 1, and S <= 4096 when it swaps */
    int32_t topk;               /* index_topk the selection may produce, <= 1024 */
    int32_t kv_dim;             /* D, [P1]: 512 */
    int32_t batch;              /* sequences, 1 <= batch <= LSA_MAX_BATCH */
    lsa_dtype dtype;            /* row storage: LSA_F32, LSA_BF16 or LSA_F16 */
    lsa_cold_kind cold;         /* where the full store lives */
    uint64_t pinned_cap_bytes;  /* [P1] PINNED_MIB, 0 = unlimited */
    int32_t allow_topk_reduction;
    void* kv_buf;               /* device, caller-owned */
    int64_t kv_stride_b;        /* elements between sequences of kv_buf */
    /* Optional caller-owned cold store (LSA_COLD_HBM only): when non-NULL the
       pool allocates none and uses cold_buf + b * cold_stride_b (bytes) as the
       [cap][kv_dim] rows of sequence b.  Several pools may share one store. */
    void* cold_buf;
    int64_t cold_stride_b;      /* bytes between sequences of cold_buf */
} lsa_pool_desc;

typedef struct lsa_pool_stats_t {
    uint64_t hits, misses;      /* [P1] gguf_kv_swap_stats hits= misses= */
    uint64_t h2d_bytes;         /* rows moved cold -> slots */
    uint64_t d2h_bytes;         /* rows stored into the pool */
    int64_t compressed_cap;
    int32_t swap_enabled;       /* 0: fully resident ([P1] gguf_kv_swap=0 reason=...) */
    int32_t resident;           /* slots in use, summed over sequences */
} lsa_pool_stats_t;

typedef struct lsa_pool lsa_pool;
/* rows per sequence that kv_buf must hold: window + (swap ? gpu_chunks : cap) */
int64_t    lsa_pool_rows(const lsa_pool_desc* desc);
lsa_status lsa_pool_create(lsa_pool** out, const lsa_pool_desc* desc);
void       lsa_pool_destroy(lsa_pool* pool);
/* [P1] store flow: copy `count` rows (host or device memory, [count][kv_dim]
 * in the pool dtype) into entries first..first+count-1 of sequence b and mark
 * them stored; a staged copy of such an entry is refreshed.  Asynchronous. */
lsa_status lsa_pool_store(lsa_pool* pool, int32_t b, int64_t first, int64_t count,
                          const void* rows, lsa_stream_t stream);
/* Host address of the pinned cold pool of sequence b (LSA_COLD_HOST only),
 * [cap][kv_dim]; rows written there directly must be declared with
 * lsa_pool_mark_stored. NULL otherwise. */
void*      lsa_pool_host_rows(lsa_pool* pool, int32_t b);
lsa_status lsa_pool_mark_stored(lsa_pool* pool, int32_t b, int64_t first, int64_t count,
                                lsa_stream_t stream);
/* empty every slot (stored rows stay stored) and zero hits/misses/h2d. */
lsa_status lsa_pool_reset(lsa_pool* pool, lsa_stream_t stream);
/* Adaptive GPU_CHUNKS ([P1] limitations, future work: the staging capacity
 * adjusted from the runtime LRU hit rate; [P1] troubleshooting: a miss rate
 * above 50 % or more than 10 MB of H2D per step calls for more GPU_CHUNKS).
 * The capacity is the number of slots a swapping pool may use, 1..gpu_chunks
 * (gpu_chunks: the slots its kv_buf holds; a new pool uses all of them).
 * Growing makes the next slots usable (a miss takes the lowest unused slot).
 * Shrinking to C evicts the least recently used entries until at most C
 * remain, then moves every remaining entry whose slot is >= C, with its row,
 * to the lowest vacated slot below C (both in ascending slot order); the LRU
 * order is kept.  Enqueued on `stream`.  Call it between lsa_decode_step
 * calls, or re-prime the lookahead schedule after it (staged steps and
 * captured graphs keep the old slots).  A capacity below topk returns
 * LSA_ERR_SLOTS_LT_TOPK unless the pool allows top-k reduction.  Resident
 * pools keep every row and ignore the capacity. */
lsa_status lsa_pool_set_capacity(lsa_pool* pool, int32_t capacity, lsa_stream_t stream);
int32_t    lsa_pool_capacity(const lsa_pool* pool);
/* KVSwap article §3.2 (rolling buffer): replacement by LRU weighted with the
 * entries' importance scores, and a prefetch trigger at 70 % buffer
 * utilisation.  For a swapping pool:
 *   recency_weight w (percent, 0..100): the eviction candidates of a step
 *     (entries resident when it starts and not selected by it) are evicted in
 *     ascending w*a + (100-w)*c, ties to the smaller a, where a is the
 *     candidate's recency rank (0 = least recently used) and c its importance
 *     rank (0 = lowest score of the step's scorer for that entry, equal scores
 *     ranked by a).  100 is plain LRU.  Below 100 the stage needs the step's
 *     scores of the pool's own entries: the pool's ratio must be the scored
 *     source ratio (lsa_decode_step passes its scores, lsa_kvswap_step its
 *     low-rank scores, lsa_stage its `importance`).
 *   high_water h (percent, 1..100): after a step the pool keeps at most
 *     max(floor(h * capacity / 100), the step's entries) slots in use,
 *     evicting further candidates in the same order, so the next step's misses
 *     first take the freed slots (the lowest free slot first).  100 is off.
 * Policies beyond plain LRU need gpu_chunks <= 1024.  Takes effect from the
 * next stage; a pool that used them keeps taking free slots from anywhere
 * below its capacity. */
lsa_status lsa_pool_set_replacement(lsa_pool* pool, int32_t recency_weight, int32_t high_water);
/* The adaptive policy, over the steps since the previous call (or reset):
 * with h hits, m misses and x bytes of H2D in `steps` steps, grow by `step`
 * slots (up to max_capacity) when m/(h+m) > grow_miss_rate or x/steps >
 * grow_h2d_bytes_per_step; else shrink by `step` (down to min_capacity) when
 * m/(h+m) < shrink_miss_rate; no lookups, no change.  Synchronises `stream`
 * (it reads the counters); writes the resulting capacity to *capacity. */
typedef struct lsa_adapt_policy {
    double grow_miss_rate;            /* [P1]: 0.5 */
    double grow_h2d_bytes_per_step;   /* [P1]: 10 MB */
    double shrink_miss_rate;          /* 0 never shrinks */
    int32_t step;
    int32_t min_capacity, max_capacity;
} lsa_adapt_policy;
lsa_status lsa_pool_adapt(lsa_pool* pool, const lsa_adapt_policy* policy, int32_t steps, int32_t* capacity,
                          lsa_stream_t stream);
/* Synchronises `stream`, then reports counters.  Returns LSA_ERR_NOT_STORED
 * ([P1] error 4) if a stage since the last call found an entry that was never
 * stored in a sequence's list (that stage left the sequence's slot table, LRU
 * order and counters unchanged and wrote an empty row list, so its attention
 * output is zero), and LSA_ERR_INVALID_ARG if a list held an entry outside
 * [0, compressed_cap).  The flags are cleared once reported.  The stage runs on
 * the device and the step calls return before it does, so this is where the
 * error surfaces. */
lsa_status lsa_pool_stats(lsa_pool* pool, lsa_pool_stats_t* out, lsa_stream_t stream);
/* Test hook ([P1] KV_SWAP_VALIDATE): copies the slot table of sequence b to
 * host: slot_logical [gpu_chunks] (-1 = unused) and lru [gpu_chunks] (slot ids
 * from most to least recently used); returns the number of used slots in
 * *n_used.  Synchronises `stream`. */
lsa_status lsa_pool_state(lsa_pool* pool, int32_t b, int32_t* slot_logical, int32_t* lru,
                          int32_t* n_used, lsa_stream_t stream);

/* ------------------------------------------------------------------ stage --
 * [P1] swap-in flow: for the chunks selected on the ratio-src_ratio source
 * layer, map them to this pool's ratio (entry j -> floor(j * src_ratio /
 * ratio), duplicates removed, ascending), keep the complete ones (entry m with
 * m < floor(n_valid[b] * src_ratio / ratio): the tokens of a chunk that is not
 * complete yet all lie in the sliding window), then per entry: a hit moves it
 * to the LRU front; a miss takes the lowest unused slot, else evicts the least
 * recently used one, and its row is copied cold -> slot.  [P1] error 4: if the
 * list of sequence b holds an entry that was never stored, nothing of b
 * changes, n_rows[b] = 0 and the pool's error flag is set (lsa_pool_stats).  Hits are handled
 * before misses, each in ascending order, so no selected chunk is evicted in
 * the step that selects it.  Writes the physical row list the attention reads:
 * phys[b][0..window-1] = 0..window-1, then window + slot of each entry in
 * ascending entry order; n_rows[b] = window + entries.
 *   sel   device i32 [batch][sel_stride] ascending source-layer indices
 *   count device i32 [batch]
 *   n_valid host [batch] valid source-layer entries per sequence, or NULL
 *         (every chunk complete)
 *   importance device f32 [batch][compressed_cap]: the step's score of every
 *         entry, for a pool whose replacement weighs importance (its ratio must
 *         equal src_ratio); NULL otherwise
 *   phys  device i32 [batch][phys_stride], phys_stride >= window + sel_stride
 *   n_rows device i32 [batch]
 * sel_stride must not exceed the pool's gpu_chunks when it swaps (it is the
 * most entries a step can stage), nor 1024. */
lsa_status lsa_stage(lsa_pool* pool, const int32_t* sel, const int32_t* count, int32_t sel_stride,
                     int32_t src_ratio, const int64_t* n_valid, const float* importance, int32_t* phys,
                     int32_t phys_stride, int32_t* n_rows, lsa_stream_t stream);

/* ----------------------------------------------------------------- attend --
 * [P1] overview "Two-tier KV cache" and indexed_cached_attention (window +
 * selected): per sequence b and head h, with rows r = phys[b][0..n_rows[b]-1]
 * of kv (each row serves as key and value):
 *     out[b,h,:] = sum_r softmax_r(scale * q[b,h,:] . kv[r,:]) * kv[r,:]
 * accumulated in fp32; out = 0 when n_rows[b] == 0.  The split over rows
 * depends only on n_rows[b], so the result does not depend on which physical
 * rows hold the entries (swap on and off give identical bits).
 *   q    device f32 [batch][hq][kv_dim];  out device f32 [batch][hq][kv_dim]
 *   kv   device [batch] x rows x kv_dim (dtype F32 or BF16), sequence b at
 *        element offset b * kv_stride_b
 *   kv_rows rows per sequence of kv: phys entries outside [0, kv_rows) read
 *        as zero rows (a malformed list cannot read past the buffer)
 *   phys device i32 [batch][phys_stride]; n_rows device i32 [batch], values
 *        clamped to [0, phys_stride]
 * Supported: 1 <= hq <= 16, kv_dim in {128, 256, 512}, 1 <= batch <= LSA_MAX_BATCH,
 * phys_stride <= 5120.
 * When the whole grid of 32-row splits fits on the GPU at once, the splits
 * merge in the same launch through counters in the context (calls on one
 * context must not overlap, as for its workspace); a merge that waits longer
 * than about a second (a split that never ran) writes NaN, and so does every
 * later one-launch attention of that context. */
lsa_status lsa_attend(lsa_ctx* ctx, const float* q, const void* kv, lsa_dtype dtype,
                      int64_t kv_stride_b, int64_t kv_rows, const int32_t* phys,
                      int32_t phys_stride, const int32_t* n_rows, int32_t batch, int32_t hq,
                      int32_t kv_dim, float scale, float* out, lsa_stream_t stream);

/* ------------------------------------------------------------ decode step --
 * [P1] architecture overview: score once on the shared source layer, one
 * global selection, then for every sparse layer the swap-in and the attention
 * over window + selected.  All layers' pools must share `batch`. */
typedef struct lsa_step_desc {
    /* scoring of the shared source layer (see lsa_score) */
    const void* keys; lsa_dtype key_dtype; const uint8_t* key_scales; int64_t n_keys; const int64_t* n_valid;
    int32_t dk;
    const float* q_idx; const float* w_idx; int32_t n_idx; int32_t heads; lsa_ensemble ensemble;
    /* selection (see lsa_select); k is lowered to the smallest swapping pool's
       gpu_chunks when that pool allows top-k reduction */
    lsa_select_mode mode; int32_t k; double tau; int32_t src_ratio;
    float* scores;              /* device f32 [batch][n_keys] */
    int32_t* sel;               /* device i32 [batch][k] */
    int32_t* count;             /* device i32 [batch] */
    /* sparse layers */
    int32_t n_layers;           /* 1..LSA_MAX_LAYERS ([P1]: 41 sparse layers share one selection);
                                   the lookahead schedule needs n_layers * batch <= 1024 */
    lsa_pool* const* pools;     /* host [n_layers] */
    const float* q_attn;        /* device f32 [n_layers][batch][hq][kv_dim] */
    float* out;                 /* device f32 [n_layers][batch][hq][kv_dim] */
    int32_t* phys;              /* device i32 [n_layers][batch][window + k] or NULL (workspace) */
    int32_t* n_rows;            /* device i32 [n_layers][batch] or NULL (workspace) */
    int32_t hq; float scale; int32_t batch;
} lsa_step_desc;
lsa_status lsa_decode_step(lsa_ctx* ctx, const lsa_step_desc* step, lsa_stream_t stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same step
 * as lsa_decode_step (same kernels, same results, bit for bit), but its scratch
 * (select histogram and candidates, attention partials, row lists, miss lists)
 * lives in a static device array of LSA_STATIC_SCRATCH_BYTES that every GPU
 * the library runs on holds until the process ends; the call allocates and
 * frees nothing (no hipMalloc / hipFree, no events, no timing).  A step needing
 * more scratch than that returns LSA_ERR_UNSUPPORTED and enqueues nothing.
 * ctx's device must be current.  Every call on one GPU shares that GPU's
 * array and it keeps the last call's contents (the call clears what must start
 * at zero), so calls that overlap on one GPU -- on different streams or from
 * different threads -- race; the row lists are those of the last call (pass
 * phys / n_rows to keep them elsewhere). */
#define LSA_STATIC_SCRATCH_BYTES (32u << 20)
lsa_status lsa_decode_step_noalloc(lsa_ctx* ctx, const lsa_step_desc* step, lsa_stream_t stream);

/* [P2] LSA section: the memory indexer is triggered periodically, and each
 * prediction covers the chunks of the coming short decoding window.  A step of
 * that window on which the indexer does not fire attends over the rows the
 * last lsa_decode_step staged: no scoring, selection or staging (the indexer
 * query and weights of `step` are not read), and the pools' counters and LRU
 * order stay as they are.  `step` must have the shapes of that lsa_decode_step
 * (its q_attn and out are this step's); when it passed no phys / n_rows, the
 * rows live in the context workspace, and a call in between on the same
 * context that needs a larger workspace loses them (pass phys / n_rows then).
 * A (layer, sequence) whose last stage failed with [P1] error 4 has an empty
 * row list and gets a zero output. */
lsa_status lsa_decode_attend(lsa_ctx* ctx, const lsa_step_desc* step, lsa_stream_t stream);

/* ------------------------------------------------------ lookahead schedule --
 * [P2] LSA section: the memory indexer predicts, ahead of time, which chunks
 * the coming decoding window will use, and only those are recalled to the GPU;
 * [P1] limitations and future work: global scoring runs synchronously in the
 * reference and overlapping it is listed as future work.
 * Here the prediction for the next step overlaps the current step:
 *   lsa_lookahead_prime(ctx, d, s): score d->q_idx / d->w_idx, select and stage
 *     every layer on stream s: the rows of the first step (their missed rows
 *     are copied by the first lsa_lookahead_step).
 *   lsa_lookahead_step(ctx, d, s): for the current step, copy its missed rows
 *     into their slots and attend d->q_attn over its staged rows (writing
 *     d->out); for the NEXT step, score d->q_idx / d->w_idx (the indexer query
 *     that predicts it), select and stage.  Three launches on s: the row copy
 *     beside the key scan (which also builds the selection's histogram and
 *     candidate lists), the attention splits beside the selection's final
 *     pass, the attention merge beside the stage.
 * The outputs equal lsa_decode_step's when step t's call carries the indexer
 * query of step t+1: every kernel body is the same, and the stage of step t+1
 * runs after step t's attention has finished.
 * d->phys / d->n_rows, when given, hold two buffers: [2][n_layers][batch][window + k]
 * and [2][n_layers][batch]; the context alternates between them (the rows of
 * the coming step are in buffer lsa_lookahead_buffer(ctx)).  Calls that
 * overlap on one context race; a captured step replays correctly only in the
 * order it was captured. */
lsa_status lsa_lookahead_prime(lsa_ctx* ctx, const lsa_step_desc* step, lsa_stream_t stream);
lsa_status lsa_lookahead_step(lsa_ctx* ctx, const lsa_step_desc* step, lsa_stream_t stream);
int32_t    lsa_lookahead_buffer(const lsa_ctx* ctx);
/* The periodic indexer in the lookahead schedule ([P2] LSA section): with a
 * period of D steps, steps D*j .. D*j + D-1 attend over the rows of prediction
 * j.  The last step of a window calls lsa_lookahead_step, which attends and
 * predicts the next window (its q_idx / w_idx are the indexer query of that
 * window); the other steps call lsa_lookahead_attend, which only attends (and,
 * on the first step of a window, copies the window's missed rows into their
 * slots).  The outputs equal lsa_decode_step on the first step of each window
 * and lsa_decode_attend on the others. */
lsa_status lsa_lookahead_attend(lsa_ctx* ctx, const lsa_step_desc* step, lsa_stream_t stream);

/* ---------------------------------------------------------------- KVSwap --
 * KVSwap article, sections 2.2-2.3 and 3.2: keys of a head group are kept as
 * low-rank factors K ~ U diag(S) V^T; the group's query scores every position,
 * the top positions are staged into a bounded slot buffer and each head of the
 * group attends over full-precision K and V rows of those positions.
 * A segment is one head group of one sequence and layer; rows of the slot
 * buffer hold [K of the group's heads | V of the group's heads].
 *
 * lsa_score_lowrank: for every segment s and position t < T,
 *     scores[s][t] = q[s] . (U[s] diag(S[s]) V[s]^T)[t,:] = U[s][t,:] . p[s],
 *     p[s] = diag(S[s]) V[s]^T q[s]     (fp32 accumulation)
 *   U device f16 [n_seg][T][rank], S device f32 [n_seg][rank],
 *   V device f16 [n_seg][C][rank], q device f32 [n_seg][C],
 *   scores device f32 [n_seg][T].  rank in {16, 32, 64}; 1 <= C <= 4096;
 *   T * rank * 2 < 4 GiB; n_seg <= 65535.  Uses the context workspace
 *   (n_seg * rank floats). */
lsa_status lsa_score_lowrank(lsa_ctx* ctx, const void* U, lsa_dtype factor_dtype, int32_t n_seg, int64_t T,
                             int32_t rank, const float* S, const void* V, int32_t C, const float* q,
                             float* scores, lsa_stream_t stream);

/* lsa_attend_kv: for segment s and head h < heads, over rows
 * r = phys[s][0..n_rows[s]-1] of the segment's slot rows,
 *     out[s,h,:] = sum_r softmax_r(scale * q[s,h,:] . K_h[r,:]) * V_h[r,:]
 * with K_h[r,:] = row r elements [h*dh, (h+1)*dh) and V_h[r,:] = row r
 * elements [(heads+h)*dh, (heads+h+1)*dh); fp32 accumulation; out = 0 when
 * n_rows[s] == 0.
 *   q   device f32 [n_seg][heads][dh];  out device f32 [n_seg][heads][dh]
 *   kv  device, dtype F16 or BF16, segment s at element offset s * kv_stride_seg,
 *       kv_rows rows of 2 * heads * dh elements; phys entries outside
 *       [0, kv_rows) read as zero rows
 *   phys device i32 [n_seg][phys_stride]; n_rows device i32 [n_seg], clamped
 *       to [0, phys_stride]
 * Supported: 1 <= heads <= 8, dh in {64, 128}, phys_stride <= 4096 and
 * (heads + 2) * phys_stride <= 16384. */
lsa_status lsa_attend_kv(lsa_ctx* ctx, const float* q, const void* kv, lsa_dtype dtype, int64_t kv_stride_seg,
                         int64_t kv_rows, int32_t heads, int32_t head_dim, const int32_t* phys,
                         int32_t phys_stride, const int32_t* n_rows, int32_t n_seg, float scale, float* out,
                         lsa_stream_t stream);

/* lsa_kvswap_step: one decode step of the KVSwap variant over n_pools pools of
 * `batch` sequences each (segment s = pool * batch + b): lsa_score_lowrank over
 * all segments, top-k per segment (lsa_select rules: ties to the lowest
 * position, output ascending), lsa_stage of every pool (window 0, positions
 * used as entries directly), then lsa_attend_kv over the staged rows.
 * Every pool must have window 0, ratio 1, compressed_cap == T, the same batch,
 * dtype and kv_dim == 2 * heads * head_dim, and their kv_buf must be laid out
 * back to back: pool p's kv_buf == pool 0's + p * batch * kv_stride_b elements.
 * The stage of all pools is one launch: each call copies the pools' stage
 * descriptors to the device (a stream-ordered copy from one of two pinned host
 * buffers of the context) and first waits on the host until the copy from that
 * buffer two calls back has completed; the first call allocates them.  The call
 * is therefore not meant for stream capture. */
typedef struct lsa_kvswap_desc {
    const void* U; const float* S; const void* V; lsa_dtype factor_dtype;
    int64_t T; int32_t rank;
    const float* q;             /* device f32 [n_seg][heads * head_dim] */
    int32_t heads, head_dim;
    int32_t k;                  /* positions kept per segment, <= 1024 */
    float* scores;              /* device f32 [n_seg][T], or NULL: then each segment is
                                   scored and its top-k taken in one workgroup and no
                                   score is written (T <= 32768, k <= 1024; not with a
                                   pool whose recency weight is below 100, which reads
                                   the scores: LSA_ERR_INVALID_ARG) */
    int32_t* sel;               /* device i32 [n_seg][k] */
    int32_t* count;             /* device i32 [n_seg] */
    int32_t n_pools;
    lsa_pool* const* pools;     /* host [n_pools] */
    int32_t* phys;              /* device i32 [n_seg][k] */
    int32_t* n_rows;            /* device i32 [n_seg] */
    float scale;
    float* out;                 /* device f32 [n_seg][heads][head_dim] */
} lsa_kvswap_desc;
lsa_status lsa_kvswap_step(lsa_ctx* ctx, const lsa_kvswap_desc* d, lsa_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* LSA_H */
