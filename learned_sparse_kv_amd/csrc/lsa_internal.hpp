// Internal declarations shared by the liblsa HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lsa.h"

namespace lsa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ------------------------------------------------------------ device helpers
// Buffer resource for raw buffer loads: reads at byte offsets >= num_records
// return zero, which is how ragged tails are padded without branches.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_records) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_records,
                                             0x00020000);
}

// The builtin returns four uint32 lanes; keep that type (assigning it to a
// float vector would convert values instead of moving bits).
__device__ inline uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// The same with the non-temporal cache policy (NT): for data read once per
// launch that no later kernel reads again soon, so it does not displace what
// the caches hold.
__device__ inline uint4 buffer_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 2);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ inline float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ inline float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }

// Order-preserving map of a float to uint32 (larger float -> larger key);
// -0 is first turned into +0 so the two compare equal.
__device__ inline uint32_t order_key(float x) {
    x = x + 0.0f;
    const uint32_t b = __float_as_uint(x);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes of a wave, in six DPP adds: shifts by
// 1, 2, 4 and 8 lanes within each 16-lane row (a lane with no source adds 0),
// then lane 15's total into rows 1 and 3 and lane 31's total into rows 2 and
// 3.  No LDS permute, so a scan costs a few VALU latencies.
__device__ inline int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return v;
}

__device__ inline int wave_sum(int v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    return v;
}

// Adds 1 to hist[dg] for every active lane of the wave; the lanes sharing the
// first active lane's value are added with one atomic (clustered keys would
// otherwise serialise on one LDS address).  Call with the whole wave.
__device__ inline void hist_add(uint32_t* hist, bool act, uint32_t dg) {
    const uint64_t am = __ballot(act);
    if (am) {
        const int lane = threadIdx.x & 63;
        const int first = __ffsll((unsigned long long)am) - 1;
        const uint32_t d0 = __shfl(dg, first, 64);
        const uint64_t same = __ballot(act && dg == d0);
        if (lane == first) atomicAdd(&hist[d0], (uint32_t)__popcll(same));
        if (act && dg != d0) atomicAdd(&hist[dg], 1u);
    }
}

// Exclusive block-wide prefix sum for blockDim.x == NT (multiple of 64);
// `smem` needs NT/64 ints.  Returns the exclusive prefix; *total = sum.
template <int NT>
__device__ inline int block_excl_scan(int v, int* smem, int* total) {
    static_assert(NT % 64 == 0 && NT <= 4096, "whole waves, at most 64");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    constexpr int NW = NT / 64;
    const int incl = wave_incl_scan(v);
    if (lane == 63) smem[wave] = incl;
    __syncthreads();
    // every wave scans the wave totals itself (one LDS read per lane), so the
    // block needs no serial pass and no third barrier phase
    const int wt = wave_incl_scan(lane < NW ? smem[lane] : 0);
    const int before = __builtin_amdgcn_readlane(wt, wave > 0 ? wave - 1 : 0);
    *total = __builtin_amdgcn_readlane(wt, NW - 1);
    __syncthreads();   // smem is free again for the caller's next scan
    return (wave > 0 ? before : 0) + incl - v;
}

// ------------------------------------------------------------------ launchers
constexpr int kSelBins = 2048;        // 11-bit key histogram of the long-segment path
constexpr int kSelShift = 21;         // bin = order_key(score) >> kSelShift
constexpr int kSelKeepCap = 8192;     // entries (above + in the boundary bucket) resolved in LDS
constexpr int kSelColBlk = 1024;      // entries per candidate list block of the histogram path
constexpr int kSelFinalBlocks = 4096; // list blocks per segment whose starts the final selection keeps in LDS
constexpr int kSelSingle = 32768;     // segments up to this length use one workgroup
// sparse layers per stage / attention launch: a step with more layers issues
// these launches per group of this many layers (their arguments stay small)
constexpr int kLaunchLayers = 16;
// (layer, sequence) segments the lookahead schedule's row copy handles in one launch
constexpr int kCopyMaxSegs = 1024;

// Query/weight projection of the hidden state (lsa_project.hip).
struct ProjectArgs {
    const float* hidden;    // [batch][d_model]
    const void* wq;         // [q_rows][d_model]
    const void* ww;         // [w_rows][d_model]
    float* q;               // [batch][q_rows]
    float* w;               // [batch][w_rows]
    int32_t d_model, q_rows, w_rows;
};
hipError_t launch_project(const ProjectArgs& a, int w_dtype, int batch, int n_cu, hipStream_t s);

struct ScoreArgs {
    const void* keys;
    const uint8_t* scales;    // MX keys: E8M0 per 32 elements, [batch][n_keys][dk/32]
    const float* q;
    const float* w;
    float* scores;
    int64_t n_keys;
    int32_t batch, n_idx, heads, ensemble;
    int32_t n_valid[LSA_MAX_BATCH];
    int32_t tile_start[LSA_MAX_BATCH + 1];   // prefix of 32-key tiles per sequence
};
// stream_keys: load the keys with the non-temporal cache policy (lsa_score, a
// pass that reads them once); the decode steps, which read the same keys at every
// step, leave them to the caches
hipError_t launch_fm_score(const ScoreArgs& a, int key_dtype, int dk, int n_cu, hipStream_t s, bool stream_keys);
// What the score waves write for the select as they score: the histogram
// (hist set: [n_seg][kSelBins], zero on entry), or the candidate lists
// (blk_count set; see the select's pre = 1): per 256-entry sub-block the
// entries of bin >= guess[seq] (in threshold mode no higher than the
// threshold's bin) passing the threshold, in index order, with their order keys.
struct ScoreHistArgs {
    uint32_t* hist;
    int32_t mode;
    float t_f;
    int32_t* blk_count;         // [n_seg][4 * nblk]
    int32_t* blk_idx;           // [n_seg][4 * nblk][256]
    uint32_t* blk_key;          // [n_seg][4 * nblk][256]
    const int32_t* guess;       // [n_seg]
    int32_t nblk;               // 1024-entry blocks per sequence
};
// the grid of the list-writing score launch (one workgroup per CU at most,
// a multiple of the batch)
int score_lists_grid(const ScoreArgs& a, int n_cu);
// fm_score with the select's candidate lists: fp32 and bf16 keys
hipError_t launch_fm_score_lists(const ScoreArgs& a, const ScoreHistArgs& h, int key_dtype, int dk, int n_cu,
                                 hipStream_t s, bool stream_keys);

struct SelectArgs {
    const float* scores;
    int64_t n_keys;
    int32_t n_seg, k, stride, mode;   // k: most entries kept; stride: row length of sel
    float t_f;                  // threshold mode: pass if score > t_f
    int32_t n_valid_uniform;    // used when has_n_valid == 0
    int32_t has_n_valid;
    int32_t n_valid[LSA_MAX_BATCH];
    int32_t* sel;
    int32_t* count;
    int32_t path;               // 0: one workgroup per segment, 1: histogram path
    int32_t e1;                 // path 0: keys per thread
    int32_t nblk;               // path 1: 1024-entry blocks per segment
    // path 1 workspace.  hist is zero on entry and left zero on exit.
    uint32_t* hist;             // [n_seg][kSelBins]
    int32_t* blk_count;         // [n_seg][nblk] entries each block kept
    int32_t* blk_idx;           // [n_seg][nblk][1024] kept indices (top bit: boundary bucket)
    uint32_t* blk_key;          // [n_seg][nblk][1024] their keys
    // pre = 1: the score launch wrote the block lists: every entry of bin
    // >= guess (passing the threshold), unmarked, in index order, and no
    // histogram; the final selection takes b* from the listed entries when they
    // number at least the K chosen, and scans the scores otherwise
    int32_t pre;
    int32_t blk_stride;         // entries per block list (0: kSelColBlk)
    // when set, the final selection writes the bin the next step's lists start
    // at: this step's b*, or one bin lower when b* and above hold fewer than
    // 1.5 times the entries chosen (and, from a histogram, the lower bin keeps
    // the lists short)
    int32_t* guess_out;         // [n_seg]
};
// Fills the shape fields; returns false when out of range.  *zero_bytes is the
// size of the zero-initialised region (hist + counters), *ws_bytes the rest.
bool select_plan(SelectArgs* a, size_t* zero_bytes, size_t* ws_bytes);
void select_bind(SelectArgs* a, void* zero_region, void* ws);
hipError_t launch_fm_select(const SelectArgs& a, hipStream_t s);

struct StageLayer {
    int32_t* slot_of;           // [batch][cap] slot or -1
    int32_t* logical_of;        // [batch][S] entry or -1
    int32_t* lru;               // [batch][S] slot ids, most recent first
    int32_t* meta;              // [batch][4]: used slots, not-stored flag
    uint64_t* stats;            // [batch][4]: hits, misses, h2d bytes
    const uint8_t* ready;       // [batch][cap]
    // bit b: every entry of sequence b is marked stored (the stage then skips
    // its ready lookups; the flags are only ever set, never cleared)
    uint64_t all_ready;
    const int32_t* sel;         // [batch][sel_stride]
    const int32_t* count;       // [batch]
    int32_t* phys;              // [batch][phys_stride]
    int32_t* n_rows;            // [batch]
    const void* cold;           // cold rows, sequence b at b * cold_stride_b bytes
    void* kv;                   // kv_buf
    int64_t cap, cold_stride_b, kv_stride_b_bytes;
    int32_t ratio, src_ratio, S, window, swap, sel_stride, phys_stride, row_bytes;
    int32_t cap_slots;          // slots the pool may use (adaptive capacity), <= S
    // defer_copy: instead of copying missed rows, write src[b][r] = cold entry
    // of list row r for a miss, -1 otherwise; the attention then reads the
    // missed rows from the cold pool and fills their slots
    int32_t defer_copy;
    int32_t* src;               // [batch][phys_stride]
    // optional: seg_cold[b] = address of sequence b's cold rows (written by the
    // stage, so a later kernel can find a missed row without the pool)
    uint64_t* seg_cold;         // [batch]
    // optional: the misses of a deferring stage as a compact list,
    // miss[b][rank] = {address of the cold row, address of its slot row}, and
    // n_miss[b] = their number (0 for a resident layer)
    uint64_t* miss;             // [batch][phys_stride][2]
    int32_t* n_miss;            // [batch]
    // replacement beyond plain LRU (S <= 1024 only): general = 1 takes free
    // slots from anywhere below cap_slots, evicts candidates in the order that
    // weighs recency (recency_w percent) against importance (imp[b][entry],
    // the step's scores; read when recency_w < 100), and frees slots down to
    // max(hw_slots, the step's entries) after the step
    int32_t general, recency_w, hw_slots;
    int64_t imp_stride;
    const float* imp;
};
struct StageArgs {
    int32_t n_layers, batch;
    // valid source entries per sequence: a layer uses its chunks below
    // floor(src_valid[b] * src_ratio / ratio), the complete ones
    int32_t src_valid[LSA_MAX_BATCH];
    StageLayer L[kLaunchLayers];
};
hipError_t launch_kv_stage(const StageArgs& a, hipStream_t s);
// the stage of n_layers layers (descriptors in device memory) as one launch
// small: every layer has S <= 512 slots and sel_stride <= 512 (512-thread workgroups)
hipError_t launch_kv_stage_table(const StageLayer* layers, int n_layers, int batch, bool small, hipStream_t s);
// copy the rows a deferred stage recorded in src[] from the cold pool into their slots
hipError_t launch_fetch_missed(const StageArgs& a, int phys_stride, hipStream_t s);
// the select's last launch alone (path 1: the final kernel; path 0: the whole select)
hipError_t launch_fm_select_final(const SelectArgs& a, hipStream_t s);
// copy the rows of entries [first, first+count) of sequence b that are staged
// from the cold pool into their slots
// shrink every sequence of a swapping pool to `capacity` slots (tables + rows)
hipError_t launch_pool_shrink(const StageLayer& L, int batch, int capacity, hipStream_t s);
hipError_t launch_refresh_staged(const StageLayer& L, int b, int64_t first, int64_t count,
                                 hipStream_t s);

struct AttendLayer {
    const float* q;             // [batch][hq][D]
    const void* kv;
    const int32_t* phys;
    const int32_t* n_rows;
    float* out;                 // [batch][hq][D]
    int64_t kv_stride_b;        // elements
    int64_t kv_rows;            // rows per sequence; phys entries outside read as zero rows
    int32_t phys_stride;
    // optional (deferred staging): list row r with src[b][r] >= 0 is read from
    // cold entry src and written into kv row phys[b][r]
    const int32_t* src;
    void* kv_w;                 // writable alias of kv
    const void* cold;
    int64_t cold_stride_b;      // bytes
    int64_t cold_rows;          // entries per sequence of the cold pool
};
struct AttendArgs {
    int32_t n_layers, batch, hq, D, dtype, max_splits;
    float scale;
    float* part_acc;            // [layer][b][split][16][D]
    float* part_ml;             // [layer][b][split][2][16]
    // one-launch form (split and merge together): its counters (kAttendSyncWords,
    // zero between launches; nullptr: always two launches) and the CUs that
    // decide whether the whole grid can be resident at once
    uint32_t* sync;
    int32_t n_cu;
    AttendLayer L[kLaunchLayers];
};
constexpr int kAttendRows = 32;
// counters of the one-launch attention: one 128-byte line per (layer,
// sequence) pair and one for the error word, so the waits of different pairs
// never poll the line another pair counts on
constexpr int kAttendSyncStride = 32;
constexpr int kAttendSyncWords = kAttendSyncStride * (1 + kLaunchLayers * LSA_MAX_BATCH);
constexpr int kAttendMaxRows = 5120;    // longest row list (window + entries) of one attention
size_t attend_workspace_bytes(int n_layers, int batch, int D, int max_rows);
hipError_t launch_lsa_attend(const AttendArgs& a, hipStream_t s, hipEvent_t mid = nullptr);
// the split launch alone (its merge runs elsewhere)
hipError_t launch_attend_splits(const AttendArgs& a, hipStream_t s);
// fused launches of the lookahead schedule.  launch_la_fetch_score scores and,
// in the same launch, copies the rows in the miss lists of `ca` (a deferring
// stage's output, laid out back to back over (layer, sequence)) into their slots.
// With hist_for (a path-1 select with one segment per sequence, see
// la_fused_hist), the score launch also builds that select's histogram, and,
// when guess is set and the blocks fit, its candidate lists from bin guess[seq]
// on (*lists = true; the final selection then runs with pre = 1).
// The missed rows a deferring stage listed for a step: the lists and counts of
// every (layer, sequence) segment lie back to back, segment s = layer * batch + b.
struct CopyArgs {
    const uint64_t* miss;     // [n_seg][phys_stride][2]: cold row address, slot row address
    const int32_t* n_miss;    // [n_seg]
    int32_t n_seg, phys_stride, row_bytes;
};
// n_seg = 0: the rows were copied already (the launch only scores).
hipError_t launch_la_fetch_score(const ScoreArgs& sa, const CopyArgs& ca, int key_dtype, int dk, int n_cu,
                                 const SelectArgs* hist_for, const int32_t* guess, bool* lists, hipStream_t s,
                                 bool stream_keys);
bool la_fused_hist(const ScoreArgs& sa, const SelectArgs& se, int n_cu);
// select histogram (unless hist_done) and collect (unless se.pre) of step t+1,
// then its final selection beside the attention splits of step t (short
// segments: the splits, then the one-kernel select)
hipError_t launch_la_select_split(const AttendArgs& aa, const SelectArgs& se, bool hist_done, hipStream_t s);
// the stage of step t+1 beside the split merge of step t
hipError_t launch_la_stage_combine(const StageArgs& ga, const AttendArgs& aa, hipStream_t s);

}  // namespace lsa

namespace lsa {

// --------------------------------------------------------- KVSwap variant
__device__ inline float f16_to_f32(uint16_t bits) { return (float)__builtin_bit_cast(_Float16, bits); }

struct LowrankArgs {
    const uint16_t* U;      // [n_seg][T][rank] f16
    const float* S;         // [n_seg][rank]
    const uint16_t* V;      // [n_seg][C][rank] f16
    const float* q;         // [n_seg][C]
    float* p;               // [n_seg][rank] workspace: S * (V^T q)
    float* scores;          // [n_seg][T]
    int64_t T;
    int32_t n_seg, rank, C;
    int32_t rows_per_block;
};
hipError_t launch_lowrank_score(const LowrankArgs& a, hipStream_t s, hipEvent_t mid = nullptr);
// the score and the top-k of every segment in one launch, no scores written
// (a.scores and a.p unused): sel [n_seg][k] ascending, count [n_seg]
bool lowrank_select_fits(int64_t T, int rank, int k);
// one workgroup per CU (at most n_cu), each taking every grid-th segment
hipError_t launch_lowrank_select(const LowrankArgs& a, int k, int32_t* sel, int32_t* count, int n_cu,
                                 hipStream_t s);

struct AttendKVArgs {
    const float* q;         // [n_seg][heads * head_dim]
    const void* kv;         // segment s rows at element s * kv_stride_seg; row = [K heads | V heads]
    int64_t kv_stride_seg;  // elements
    int64_t kv_rows;
    const int32_t* phys;    // [n_seg][phys_stride]
    const int32_t* n_rows;  // [n_seg]
    float* out;             // [n_seg][heads][head_dim]
    int32_t phys_stride, n_seg, heads, head_dim, dtype;
    float scale;
    // optional (deferred staging): list row i with src[s][i] >= 0 is read from
    // cold row src of the segment's cold store (address seg_cold[s]) and
    // written into its slot row phys[s][i]
    const int32_t* src;         // [n_seg][phys_stride]
    const uint64_t* seg_cold;   // [n_seg]
    int64_t cold_rows;          // rows of each segment's cold store
};
constexpr int kAttendKVMaxRows = 4096;
hipError_t launch_attend_kv(const AttendKVArgs& a, hipStream_t s);
// stage (kv_stage's 512-thread form, descriptors layers[n_seg / batch]) and
// attention of each segment in one workgroup: heads 1, 2, 4 or 8, head_dim 64
// or 128, phys_stride (the selection stride) and every pool's slots <= 512
bool stage_attend_kv_fits(int heads, int head_dim, int phys_stride, int max_slots);
hipError_t launch_stage_attend_kv(const StageLayer* layers, int batch, const AttendKVArgs& a, hipStream_t s);

}  // namespace lsa
