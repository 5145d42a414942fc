// kv_stage: ratio map + LRU slot assignment + gather of missed rows.
//
// [P1] technical details, swap-in flow of gguf_kv_swap_in_selected: each
// selected logical chunk is looked up in the slot table; a hit is moved to the
// LRU front and counted; a miss evicts the LRU back, takes its slot, has its
// row copied from the cold pool, and is counted; then every chunk's index is
// rewritten to the physical row window + slot.  [P1] store flow / error 4: a
// chunk that was never stored must not be selected.  [P1] troubleshooting: a
// layer whose compressed_cap <= gpu_chunks does not swap (rows = window + j).
//
// Readings shared with the CPU oracle: a source chunk j maps to chunk
// floor(j * src_ratio / ratio) of this layer (duplicates dropped), and a layer
// chunk is only used once it is complete, i.e. once the valid source entries
// cover all of its tokens (the tokens of an incomplete chunk are all inside
// the sliding window); hits are handled before misses, each in ascending chunk
// order; a miss takes the lowest never-used slot before it evicts.  A step
// whose list holds a chunk that was never stored ([P1] error 4) changes
// nothing: the pool's tables and counters stay as they were, the row list is
// empty (so the attention writes zeros) and the pool's error flag is set.
//
// Design (gfx950): one 1024-thread workgroup per (layer, sequence) replaces
// the host-side std::list walk with prefix sums.  The LRU list is kept as an
// array `lru` of used slots, most recent first.  With h hits and m misses in
// a step, the page's sequential loop leaves the list as
//     [misses, last processed first] [hits, last processed first]
//     [untouched slots in their old order, minus the evicted ones]
// and the evicted slots are exactly the last (m - free) untouched entries of
// the old list, taken from the back.  Slots are handed out lowest-first and
// never freed, so the unused ones are always used..S-1.  The same workgroup
// then copies its missed rows cold -> slot (HBM cold pools, or pinned host
// memory read directly over PCIe, so no host round trip sits in the step).
#include "lsa_internal.hpp"

namespace lsa {

namespace {
namespace stage_k {

constexpr int kNT = 1024;
constexpr int kMaxSlots = 4096;
constexpr int kSmallNT = 512;   // threads and slots of the small-pool form

// Copies `chunks` 16-byte chunks (cpr per row) of the rows src_row[m] of
// `cold` to rows dst_row_off + dst_row[m] of `kv`, eight chunks in flight per
// thread.  The loads are unconditional (a chunk past the end re-reads the last
// one) and the batch is held in named registers; only the stores are
// predicated.
template <int NT>
__device__ inline void copy_rows(const char* cold, char* kv, int row_bytes, int chunks, int cpr, const int* src_row,
                                 const int* dst_row, int dst_row_off) {
    const int tid = threadIdx.x;
    auto addr = [&](int c, int64_t& from, int64_t& to) {
        const int cc = c < chunks ? c : chunks - 1;
        const int m = cc / cpr, off = (cc - m * cpr) * 16;
        from = (int64_t)src_row[m] * row_bytes + off;
        to = (int64_t)(dst_row_off + dst_row[m]) * row_bytes + off;
    };
    for (int c0 = 0; c0 < chunks; c0 += NT * 8) {
        int64_t f0, f1, f2, f3, f4, f5, f6, f7, t0, t1, t2, t3, t4, t5, t6, t7;
        addr(c0 + 0 * NT + tid, f0, t0);
        addr(c0 + 1 * NT + tid, f1, t1);
        addr(c0 + 2 * NT + tid, f2, t2);
        addr(c0 + 3 * NT + tid, f3, t3);
        addr(c0 + 4 * NT + tid, f4, t4);
        addr(c0 + 5 * NT + tid, f5, t5);
        addr(c0 + 6 * NT + tid, f6, t6);
        addr(c0 + 7 * NT + tid, f7, t7);
        const uint4 v0 = *reinterpret_cast<const uint4*>(cold + f0);
        const uint4 v1 = *reinterpret_cast<const uint4*>(cold + f1);
        const uint4 v2 = *reinterpret_cast<const uint4*>(cold + f2);
        const uint4 v3 = *reinterpret_cast<const uint4*>(cold + f3);
        const uint4 v4 = *reinterpret_cast<const uint4*>(cold + f4);
        const uint4 v5 = *reinterpret_cast<const uint4*>(cold + f5);
        const uint4 v6 = *reinterpret_cast<const uint4*>(cold + f6);
        const uint4 v7 = *reinterpret_cast<const uint4*>(cold + f7);
        if (c0 + 0 * NT + tid < chunks) *reinterpret_cast<uint4*>(kv + t0) = v0;
        if (c0 + 1 * NT + tid < chunks) *reinterpret_cast<uint4*>(kv + t1) = v1;
        if (c0 + 2 * NT + tid < chunks) *reinterpret_cast<uint4*>(kv + t2) = v2;
        if (c0 + 3 * NT + tid < chunks) *reinterpret_cast<uint4*>(kv + t3) = v3;
        if (c0 + 4 * NT + tid < chunks) *reinterpret_cast<uint4*>(kv + t4) = v4;
        if (c0 + 5 * NT + tid < chunks) *reinterpret_cast<uint4*>(kv + t5) = v5;
        if (c0 + 6 * NT + tid < chunks) *reinterpret_cast<uint4*>(kv + t6) = v6;
        if (c0 + 7 * NT + tid < chunks) *reinterpret_cast<uint4*>(kv + t7) = v7;
    }
}

// One (sequence b, layer) of the stage; a workgroup of NT threads, at most MS
// slots per sequence (NT >= the selection stride, and >= the slots for the
// rolling buffer).
// src_valid: valid entries of sequence b in the source layer; this layer's
// complete chunks are the first floor(src_valid * src_ratio / ratio).
template <int NT = kNT, int MS = kMaxSlots>
__device__ __forceinline__ void kv_stage_body(const StageLayer& L, const int b, const int src_valid) {
    const int tid = threadIdx.x;

    __shared__ int s_scan[NT / 64 + 1];
    __shared__ int s_sel[NT];
    __shared__ int s_slot[NT];     // slot of s_sel[i] before this step (-1: none)
    __shared__ int s_victim[NT];
    __shared__ int s_order[MS];
    __shared__ int s_logical[MS];   // logical_of before this step
    __shared__ uint8_t s_hit[MS];
    __shared__ int s_mlog[NT];     // missed entries and their slots, by miss rank
    __shared__ int s_mslot[NT];

    // Loads come in two dependent rounds: the selection together with the LRU
    // state (order, slot occupants, used count), then the slot-table entry and
    // ready flag of each source entry's chunk.  The tables are not written
    // before they are read below.
    const bool sw = L.swap != 0;
    int32_t* slot_of = L.slot_of + (int64_t)b * L.cap;
    int32_t* logical_of = L.logical_of + (int64_t)b * L.S;
    int32_t* lru = L.lru + (int64_t)b * L.S;
    const int S = L.S;
    const int32_t* sel = L.sel + (int64_t)b * L.sel_stride;
    const int n_src_raw = L.count[b];
    const int sv = tid < L.sel_stride ? sel[tid] : 0;
    const int sp = (tid >= 1 && tid <= L.sel_stride) ? sel[tid - 1] : 0;
    int n_used = 0;
    if (sw) {
        n_used = L.meta[b * 4 + 0];
        for (int i = tid; i < S; i += NT) {
            s_order[i] = lru[i];
            s_logical[i] = logical_of[i];
            s_hit[i] = 0;
        }
    }

    // 1. source selection -> this layer's ascending unique chunk list
    const int n_src = n_src_raw < 0 ? 0 : (n_src_raw > L.sel_stride ? L.sel_stride : n_src_raw);
    const int64_t complete = (int64_t)(src_valid < 0 ? 0 : src_valid) * L.src_ratio / L.ratio;
    bool keep = false;
    int m = -1;
    if (tid < n_src) {
        m = (int)((int64_t)sv * L.src_ratio / L.ratio);
        keep = (tid == 0 || m != (int)((int64_t)sp * L.src_ratio / L.ratio)) && m < complete;
    }
    int my_slot = -1;
    uint8_t my_rdy = 1;
    if (keep && m >= 0 && m < L.cap) {
        my_rdy = ((L.all_ready >> b) & 1) ? 1 : L.ready[(int64_t)b * L.cap + m];
        if (sw) my_slot = slot_of[m];
    }
    // wait for the two table loads here, on every lane: consumed only under
    // `keep`, they would otherwise leave the compiler waiting for all memory
    // operations (the stores below included) before each later store
    asm volatile("" ::"v"(my_slot), "v"((int)my_rdy));
    // one scan counts the kept chunks and the never-stored ones among them
    const bool unstored = keep && my_rdy == 0;
    int tot0;
    const int packed0 = block_excl_scan<NT>((keep ? 1 : 0) | (unstored ? 1 << 16 : 0), s_scan, &tot0);
    const int pos = packed0 & 0xFFFF;
    const int n_l = tot0 & 0xFFFF;
    if ((tot0 >> 16) != 0) {   // uniform: [P1] error 4, the step changes nothing
        if (tid == 0) {
            atomicOr(&L.meta[b * 4 + 1], 1);
            L.n_rows[b] = 0;
            if (L.n_miss) L.n_miss[b] = 0;
        }
        return;
    }
    if (keep) {
        s_sel[pos] = m;
        s_slot[pos] = my_slot;
    }
    __syncthreads();

    int32_t* phys = L.phys + (int64_t)b * L.phys_stride;
    for (int r = tid; r < L.window; r += NT) phys[r] = r;
    if (tid == 0) L.n_rows[b] = L.window + n_l;
    // entries outside [0, cap) (a malformed selection) are flagged and read
    // window row 0 instead, so no access leaves the pool's buffers
    int l = tid < n_l ? s_sel[tid] : -1;
    if (tid < n_l && (l < 0 || l >= L.cap)) {
        atomicOr(&L.meta[b * 4 + 1], 2);
        phys[L.window + tid] = 0;
        l = -1;
    }

    if (L.seg_cold && tid == 0)
        L.seg_cold[b] = (uint64_t)(static_cast<const char*>(L.cold) + b * L.cold_stride_b);
    if (L.n_miss && tid == 0) L.n_miss[b] = 0;   // a swapping layer overwrites it below
    int32_t* src = L.defer_copy ? L.src + (int64_t)b * L.phys_stride : nullptr;
    if (src) {
        for (int r = tid; r < L.window; r += NT) src[r] = -1;
        if (tid < n_l) src[L.window + tid] = -1;
    }
    if (!sw) {
        if (l >= 0) phys[L.window + tid] = L.window + l;
        return;
    }

    // 2. hits and misses, ranked in ascending chunk order
    int slot = l >= 0 ? s_slot[tid] : -1;
    const bool hit = slot >= 0;
    const bool miss = l >= 0 && !hit;
    if (hit) s_hit[slot] = 1;
    int tot;
    const int packed = block_excl_scan<NT>((hit ? 1 : 0) | (miss ? 1 << 16 : 0), s_scan, &tot);
    const int hit_rank = packed & 0xFFFF, miss_rank = packed >> 16;
    const int n_hit = tot & 0xFFFF, n_miss = tot >> 16;
    int new_used;
    if (!L.general) {
        const int free_slots = L.cap_slots - n_used;   // slots [n_used, capacity) are unused
        const int n_evict = n_miss > free_slots ? n_miss - free_slots : 0;

        // 3. untouched used slots in old list order; the last n_evict are evicted
        constexpr int kPer = MS / NT;
        bool untouched[kPer];
        int c_untouched = 0;
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int p = tid * kPer + q;
            untouched[q] = p < n_used && s_hit[s_order[p]] == 0;
            c_untouched += untouched[q] ? 1 : 0;
        }
        int n_untouched;
        int before = block_excl_scan<NT>(c_untouched, s_scan, &n_untouched);
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            if (!untouched[q]) continue;
            const int p = tid * kPer + q;
            const int after = n_untouched - before - 1;
            if (after < n_evict) {
                s_victim[after] = s_order[p];           // victim 0 = least recently used
            } else {
                lru[n_miss + n_hit + before] = s_order[p];
            }
            ++before;
        }
        __syncthreads();

        // 4. slots for the misses; the evicted chunks leave the table
        if (miss) slot = miss_rank < free_slots ? n_used + miss_rank : s_victim[miss_rank - free_slots];
        int old = -1;
        if (tid < n_evict) old = s_logical[s_victim[tid]];
        __syncthreads();
        if (old >= 0) slot_of[old] = -1;
        new_used = n_used + (n_miss < free_slots ? n_miss : free_slots);
    } else {
        // [P4] rolling-buffer reading (gpu_chunks <= NT): free slots may lie
        // anywhere below the capacity; the candidates (untouched used slots) are
        // evicted in ascending recency_w * a + (100 - recency_w) * c, a = recency
        // rank (0 = least recent), c = importance rank (0 = lowest score, ties by
        // a), ties by a; then the high-water mark frees the next candidates down
        // to max(hw_slots, this step's entries).  Thread t handles LRU position t,
        // slot t and candidate t.
        __shared__ int s_free[NT];
        __shared__ int s_cand[NT];     // candidate slots by recency rank
        __shared__ float s_cimp[NT];
        __shared__ int s_cprio[NT];
        const bool fr = tid < L.cap_slots && tid < S && s_logical[tid] < 0;
        int n_free;
        const int fpos = block_excl_scan<NT>(fr ? 1 : 0, s_scan, &n_free);
        if (fr) s_free[fpos] = tid;
        const int uslot = tid < n_used ? s_order[tid] : -1;
        const bool cand = uslot >= 0 && s_hit[uslot] == 0;
        int n_cand;
        const int cpos = block_excl_scan<NT>(cand ? 1 : 0, s_scan, &n_cand);
        if (cand) s_cand[n_cand - cpos - 1] = uslot;
        __syncthreads();
        if (L.recency_w < 100) {
            // an entry past the complete ones (valid entries shrank) ranks lowest
            float my_imp = 0.0f;
            if (tid < n_cand) {
                const int e = s_logical[s_cand[tid]];
                my_imp = e < complete ? L.imp[(int64_t)b * L.imp_stride + e] : -INFINITY;
            }
            s_cimp[tid] = my_imp;
            __syncthreads();
            int c = 0;
            if (tid < n_cand)
                for (int j = 0; j < n_cand; ++j) {
                    const float o = s_cimp[j];
                    c += (o < my_imp || (o == my_imp && j < tid)) ? 1 : 0;
                }
            const int prio = L.recency_w * tid + (100 - L.recency_w) * c;
            s_cprio[tid] = prio;
            __syncthreads();
            int v = 0;
            if (tid < n_cand)
                for (int j = 0; j < n_cand; ++j) {
                    const int o = s_cprio[j];
                    v += (o < prio || (o == prio && j < tid)) ? 1 : 0;
                }
            if (tid < n_cand) s_victim[v] = s_cand[tid];
        } else if (tid < n_cand) {
            s_victim[tid] = s_cand[tid];
        }
        __syncthreads();
        const int n_ev_miss = n_miss > n_free ? n_miss - n_free : 0;
        const int kept = n_hit + n_miss + (n_cand - n_ev_miss);
        const int limit = L.hw_slots > n_hit + n_miss ? L.hw_slots : n_hit + n_miss;
        int n_extra = kept > limit ? kept - limit : 0;
        if (n_extra > n_cand - n_ev_miss) n_extra = n_cand - n_ev_miss;
        const int n_ev = n_ev_miss + n_extra;
        int old = -1;
        if (tid < n_ev) {
            old = s_logical[s_victim[tid]];
            s_hit[s_victim[tid]] = 2;                  // evicted
        }
        if (miss) slot = miss_rank < n_free ? s_free[miss_rank] : s_victim[miss_rank - n_free];
        __syncthreads();
        if (old >= 0) slot_of[old] = -1;
        if (tid >= n_ev_miss && tid < n_ev) logical_of[s_victim[tid]] = -1;
        // the candidates that stay, in their old order, after the misses and hits
        const bool stays = cand && s_hit[uslot] != 2;
        int n_stay;
        const int spos = block_excl_scan<NT>(stays ? 1 : 0, s_scan, &n_stay);
        if (stays) lru[n_miss + n_hit + spos] = uslot;
        new_used = n_hit + n_miss + n_stay;
    }
    if (miss) {
        slot_of[l] = slot;
        logical_of[slot] = l;
        s_mlog[miss_rank] = l;
        s_mslot[miss_rank] = slot;
        lru[n_miss - 1 - miss_rank] = slot;
        if (src) src[L.window + tid] = l;
        if (L.miss) {
            uint64_t* e = L.miss + ((int64_t)b * L.phys_stride + miss_rank) * 2;
            e[0] = (uint64_t)(static_cast<const char*>(L.cold) + b * L.cold_stride_b + (int64_t)l * L.row_bytes);
            e[1] = (uint64_t)(static_cast<char*>(L.kv) + b * L.kv_stride_b_bytes +
                              (int64_t)(L.window + slot) * L.row_bytes);
        }
    }
    if (hit) lru[n_miss + n_hit - 1 - hit_rank] = slot;
    if (l >= 0) phys[L.window + tid] = L.window + slot;
    if (tid == 0) {
        L.meta[b * 4 + 0] = new_used;
        uint64_t* st = L.stats + (int64_t)b * 4;
        st[0] += (uint64_t)n_hit;
        st[1] += (uint64_t)n_miss;
        st[2] += (uint64_t)n_miss * (uint64_t)L.row_bytes;
        if (L.n_miss) L.n_miss[b] = n_miss;
    }
    if (src) return;   // the attention reads the missed rows and fills their slots
    __syncthreads();

    // 5. copy the missed rows cold -> slot (pinned host rows are read over PCIe
    //    directly); kBatch 16-byte loads per thread are in flight at a time
    const int cpr = L.row_bytes / 16;
    const int chunks = n_miss * cpr;
    const char* cold = static_cast<const char*>(L.cold) + b * L.cold_stride_b;
    char* kv = static_cast<char*>(L.kv) + b * L.kv_stride_b_bytes;
    copy_rows<NT>(cold, kv, L.row_bytes, chunks, cpr, s_mlog, s_mslot, L.window);
}

__global__ __launch_bounds__(kNT) void kv_stage_kernel(const StageArgs a) {
    kv_stage_body(a.L[blockIdx.y], blockIdx.x, a.src_valid[blockIdx.x]);
}

// Any number of layers in one launch: their descriptors come from device
// memory (copied to registers once, so the body's stores cannot alias them).
// Pools of at most 512 slots with at most 512 entries per selection (KVSwap's
// 400-slot buffers) take 512-thread workgroups with a quarter of the LDS, so
// four fit on a CU instead of two.
template <int NT, int MS>
__global__ __launch_bounds__(NT) void kv_stage_table_kernel(const StageLayer* Ls) {
    const StageLayer L = Ls[blockIdx.y];
    kv_stage_body<NT, MS>(L, blockIdx.x, 0x7FFFFFFF);
}

__global__ __launch_bounds__(256) void refresh_staged_kernel(const StageLayer L, int b, int64_t first, int64_t count) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t i = (int64_t)blockIdx.x * 4 + wave;
    if (i >= count) return;
    const int64_t l = first + i;
    const int slot = L.slot_of[(int64_t)b * L.cap + l];
    if (slot < 0) return;
    const char* src = static_cast<const char*>(L.cold) + b * L.cold_stride_b + l * L.row_bytes;
    char* dst = static_cast<char*>(L.kv) + b * L.kv_stride_b_bytes + (int64_t)(L.window + slot) * L.row_bytes;
    for (int off = lane * 16; off < L.row_bytes; off += 64 * 16)
        *reinterpret_cast<uint4*>(dst + off) = *reinterpret_cast<const uint4*>(src + off);
}

// Shrink of a swapping pool to C usable slots ([P1] future work: adaptive
// GPU_CHUNKS; the procedure is the oracle's reading).  The first C entries of
// the LRU list (the most recent) stay and the rest leave the slot table; every
// staying entry in a slot >= C moves, with its row, to the lowest vacated slot
// below C (a free slot or one whose entry left), both taken in ascending slot
// order; the LRU list keeps its order with the new slot ids.  Used slots may
// lie anywhere below S (a high-water mark leaves free slots between them).
// One workgroup per sequence; thread t ranks slots kPer*t .. kPer*t + kPer - 1.
__global__ __launch_bounds__(kNT) void pool_shrink_kernel(const StageLayer L, const int C) {
    const int b = blockIdx.x, tid = threadIdx.x;
    int32_t* slot_of = L.slot_of + (int64_t)b * L.cap;
    int32_t* logical_of = L.logical_of + (int64_t)b * L.S;
    int32_t* lru = L.lru + (int64_t)b * L.S;
    const int n_used = L.meta[b * 4 + 0];
    const int S = L.S;
    if (n_used > S) return;   // uniform: every thread read the same count
    __shared__ int s_scan[kNT / 64 + 1];
    __shared__ int s_lru[kMaxSlots];     // LRU list before (slot ids)
    __shared__ int s_log[kMaxSlots];     // occupant of each slot before
    __shared__ int s_new[kMaxSlots];     // new slot of each old slot, -1 if it leaves
    __shared__ uint8_t s_keep[kMaxSlots];
    __shared__ int s_vac[kMaxSlots];     // vacated slots below C, by rank
    __shared__ int s_high[kMaxSlots];    // staying slots >= C, by rank
    for (int i = tid; i < S; i += kNT) {
        s_keep[i] = 0;
        s_log[i] = logical_of[i];
    }
    __syncthreads();
    for (int p = tid; p < n_used; p += kNT) {
        const int sl = lru[p];
        s_lru[p] = sl;
        if (p < C && sl >= 0 && sl < S) s_keep[sl] = 1;
    }
    __syncthreads();
    constexpr int kPer = kMaxSlots / kNT;
    int c_vac = 0, c_high = 0;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int sl = tid * kPer + q;
        if (sl < S) {
            c_vac += (sl < C && !s_keep[sl]) ? 1 : 0;
            c_high += (sl >= C && s_keep[sl]) ? 1 : 0;
        }
    }
    int n_vac, n_high;
    int r_vac = block_excl_scan<kNT>(c_vac, s_scan, &n_vac);
    int r_high = block_excl_scan<kNT>(c_high, s_scan, &n_high);
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int sl = tid * kPer + q;
        if (sl >= S) continue;
        s_new[sl] = (sl < C && s_keep[sl]) ? sl : -1;
        if (sl < C && !s_keep[sl]) s_vac[r_vac++] = sl;
        if (sl >= C && s_keep[sl]) s_high[r_high++] = sl;
    }
    __syncthreads();
    // at most C entries stay, so n_high <= n_vac; the min only keeps a damaged
    // table from indexing past the ranked lists
    const int n_move = n_high < n_vac ? n_high : n_vac;
    for (int r = tid; r < n_move; r += kNT) s_new[s_high[r]] = s_vac[r];
    __syncthreads();
    for (int sl = tid; sl < S; sl += kNT) {
        const int l = s_log[sl];
        if (l >= 0 && l < L.cap) slot_of[l] = s_new[sl];
        if (!s_keep[sl] || sl >= C) logical_of[sl] = -1;
    }
    __syncthreads();
    for (int r = tid; r < n_move; r += kNT) logical_of[s_vac[r]] = s_log[s_high[r]];
    for (int p = tid; p < n_used; p += kNT) {
        const int sl = s_lru[p];
        lru[p] = (p < C && sl >= 0 && sl < S) ? s_new[sl] : -1;
    }
    // rows of the moved entries: slot row s_high[r] -> slot row s_vac[r]
    const int cpr = L.row_bytes / 16;
    char* kv = static_cast<char*>(L.kv) + b * L.kv_stride_b_bytes;
    // eight 16-byte chunks per thread in flight before their stores
    const int n_chunks = n_move * cpr;
    for (int i0 = 0; i0 < n_chunks; i0 += 8 * kNT) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * kNT + tid;
            if (i < n_chunks) {
                const int r = i / cpr, c = i - r * cpr;
                v[u] = *reinterpret_cast<const uint4*>(kv + (int64_t)(L.window + s_high[r]) * L.row_bytes + c * 16);
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * kNT + tid;
            if (i < n_chunks) {
                const int r = i / cpr, c = i - r * cpr;
                *reinterpret_cast<uint4*>(kv + (int64_t)(L.window + s_vac[r]) * L.row_bytes + c * 16) = v[u];
            }
        }
    }
    if (tid == 0) L.meta[b * 4 + 0] = n_used < C ? n_used : C;
}

// Copies the rows a stage recorded as missed (src[b][r] >= 0: cold entry of
// list row r) from the cold pool into their slots.  One workgroup per 32 list
// rows of one (layer, sequence); every load of a batch is issued before any
// store, so reads of pinned host rows keep many PCIe requests in flight.
constexpr int kFetchRows = 32;
constexpr int kFetchNT = 256;
__device__ __forceinline__ void fetch_missed_body(const StageArgs& a, const int bx, const int by, const int bz) {
    const StageLayer& L = a.L[bz];
    const int b = by, r0 = bx * kFetchRows;
    if (!L.swap || r0 >= L.phys_stride) return;
    __shared__ int s_src[kFetchRows], s_dst[kFetchRows];
    __shared__ int s_n;
    const int tid = threadIdx.x;
    if (tid == 0) s_n = 0;
    __syncthreads();
    if (tid < kFetchRows) {
        const int r = r0 + tid;
        const int n = L.n_rows[b];
        const int sr = (r < n && r < L.phys_stride) ? L.src[(int64_t)b * L.phys_stride + r] : -1;
        const int ph = (r < n && r < L.phys_stride) ? L.phys[(int64_t)b * L.phys_stride + r] : -1;
        // only rows the stage itself recorded: a cold entry below cap and a slot row
        if (sr >= 0 && sr < L.cap && ph >= L.window && ph < L.window + L.S) {
            const int i = atomicAdd(&s_n, 1);
            s_src[i] = sr;
            s_dst[i] = ph;
        }
    }
    __syncthreads();
    const int cpr = L.row_bytes / 16;
    const int chunks = s_n * cpr;
    const char* cold = static_cast<const char*>(L.cold) + b * L.cold_stride_b;
    char* kv = static_cast<char*>(L.kv) + b * L.kv_stride_b_bytes;
    copy_rows<kFetchNT>(cold, kv, L.row_bytes, chunks, cpr, s_src, s_dst, 0);
}

__global__ __launch_bounds__(kFetchNT) void fetch_missed_kernel(const StageArgs a) {
    fetch_missed_body(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

}  // namespace stage_k
#ifndef LSA_BODIES_ONLY
using namespace stage_k;
#endif
}  // namespace

#ifndef LSA_BODIES_ONLY
hipError_t launch_fetch_missed(const StageArgs& a, int phys_stride, hipStream_t s) {
    const dim3 grid((unsigned)((phys_stride + kFetchRows - 1) / kFetchRows), a.batch, a.n_layers);
    hipLaunchKernelGGL(fetch_missed_kernel, grid, dim3(kFetchNT), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_kv_stage(const StageArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(kv_stage_kernel, dim3(a.batch, a.n_layers), dim3(kNT), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_kv_stage_table(const StageLayer* layers, int n_layers, int batch, bool small, hipStream_t s) {
    if (n_layers < 1 || n_layers > 65535 || batch < 1) return hipErrorInvalidValue;
    if (small)
        hipLaunchKernelGGL((kv_stage_table_kernel<kSmallNT, kSmallNT>), dim3(batch, n_layers), dim3(kSmallNT), 0, s,
                           layers);
    else
        hipLaunchKernelGGL((kv_stage_table_kernel<kNT, kMaxSlots>), dim3(batch, n_layers), dim3(kNT), 0, s, layers);
    return hipGetLastError();
}

hipError_t launch_pool_shrink(const StageLayer& L, int batch, int capacity, hipStream_t s) {
    if (L.S > kMaxSlots || capacity < 1 || capacity > L.S) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pool_shrink_kernel, dim3(batch), dim3(kNT), 0, s, L, capacity);
    return hipGetLastError();
}

hipError_t launch_refresh_staged(const StageLayer& L, int b, int64_t first, int64_t count, hipStream_t s) {
    if (count <= 0) return hipSuccess;
    const dim3 grid((unsigned)((count + 3) / 4));
    hipLaunchKernelGGL(refresh_staged_kernel, grid, dim3(256), 0, s, L, b, first, count);
    return hipGetLastError();
}

#endif  // LSA_BODIES_ONLY

}  // namespace lsa
