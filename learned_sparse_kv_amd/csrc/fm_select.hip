// fm_select: top-k / sigmoid-threshold selection of compressed entries.
//
// [P1] "global top-k (512 chunks)", index_topk = global_keep_cap = 512;
// [P2] Recall / Threshold Selector: entries whose sigmoid(score) exceeds a
// threshold are recalled.  Order: score descending, index ascending on ties.
// Threshold mode keeps score > t_f (t_f = largest float <= logit(tau), worked
// out on the host), then caps at k by the same order.  Output: the chosen
// indices in ascending order, -1 padding, and the count.
//
// Design (gfx950).  Scores become order-preserving 32-bit keys (-0 folded
// into +0).  Two paths:
//
// * Segments of at most 32768 entries: one 1024-thread workgroup holds the
//   keys in registers (contiguous indices per thread, so thread order is index
//   order), finds the K-th largest key T with three radix passes (12, 10 and
//   10 bits) over LDS histograms -- the last two over the first pass's
//   boundary bin, compacted into LDS -- and compacts {key > T} plus the
//   lowest-indexed keys equal to T with two block scans.  The atomics of the
//   last two passes are pre-aggregated per wave (the lanes sharing the first
//   active lane's digit add with one atomic), which removes the contention of
//   clustered digits.
//
// * Longer segments: (1) every 4096-entry block builds an 11-bit key histogram
//   in LDS and adds it to a per-segment global histogram; (2) every 1024-entry
//   block finds the boundary bucket b* holding the K-th largest key from that
//   histogram and keeps, in index order (block scan, no atomics), its entries
//   in buckets >= b*; (3) one workgroup per segment gathers the kept entries in
//   block order -- which is global index order -- resolves b* over the 21 key
//   bits below the bucket (a radix pass over 11 bits, then the last 10 by ranking
//   the few keys of the bin found, or by a second radix pass), and places {above b*} +
//   {candidates > T} + {the first candidates equal to T}: ties fall to the
//   lowest index because the list is in index order, and the output is
//   already ascending.  If more than 8192 entries are kept, step (3) falls back
//   to an exact streaming select over the whole segment.  Step (3) leaves the
//   histogram zeroed for the next call.
#include "lsa_internal.hpp"

namespace lsa {

namespace {
namespace select_k {

constexpr int kNT = 1024;
constexpr int kNW = kNT / 64;
constexpr int kBlk = 4096;          // entries per block of the histogram kernel
constexpr int kColBlk = kSelColBlk;   // entries per block of the collect kernel
constexpr int kMaxBlocks = kSelFinalBlocks;   // collect blocks whose lists the final kernel gathers in LDS
constexpr int kBlkThreads = 256;

struct KthShared {
    uint32_t hist[256];
    int scan[kNW + 1];
    uint32_t digit;
    int above;
};

__device__ inline int seg_valid(const SelectArgs& a, int seg) {
    return a.has_n_valid ? a.n_valid[seg] : a.n_valid_uniform;
}

// Given a 256-bin histogram of the digits of the still-tied keys, finds the
// digit d holding the rem-th largest key; sh.digit = d, sh.above = keys with a
// larger digit.  Threads tid < 256 own digit 255 - tid.
__device__ inline void find_digit(const uint32_t* hist, int rem, KthShared& sh) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t d = 255u - (uint32_t)(tid & 255);
    const int cnt = tid < 256 ? (int)hist[d] : 0;
    const int incl = wave_incl_scan(cnt);
    if (tid < 256 && lane == 63) sh.scan[wave] = incl;
    __syncthreads();
    if (tid < 256) {
        int off = 0;
        for (int w = 0; w < wave; ++w) off += sh.scan[w];
        const int ge = off + incl;
        if (ge >= rem && ge - cnt < rem) {
            sh.digit = d;
            sh.above = ge - cnt;
        }
    }
    __syncthreads();
}

// Over hist[0, NB) taken from the top bin down: the bin holding the rem-th
// largest entry (1 <= rem <= the histogram's total); *bin = it, *above =
// entries in the bins above it.  Thread t of the NT owns bins NB-1-PER*t-i.
template <int NB, int NT>
__device__ void find_bin(const uint32_t* hist, int rem, int* scan, int* out, int* bin, int* above) {
    constexpr int PER = NB / NT;
    static_assert(PER >= 1 && NB % NT == 0, "bins per thread");
    const int t = threadIdx.x;
    int c[PER];
    int local = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        c[i] = (int)hist[NB - 1 - PER * t - i];
        local += c[i];
    }
    int tot;
    int run = block_excl_scan<NT>(local, scan, &tot);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        if (run < rem && run + c[i] >= rem) {
            out[0] = NB - 1 - PER * t - i;
            out[1] = run;
        }
        run += c[i];
    }
    __syncthreads();
    *bin = out[0];
    *above = out[1];
    __syncthreads();
}

constexpr int kWideBins = 4096;   // first digit: key bits 31..20 (sign, exponent, 3 mantissa bits)
constexpr int kWideCand = 4096;   // keys of the first digit's boundary bin resolved from LDS

struct KthWide {
    uint32_t hist[kWideBins];
    uint32_t cand[kWideCand];
    int scan[kNW + 1];
    int out[2];
};

// K-th largest key among the valid ones (1 <= K <= #valid): T, and the number
// of keys equal to T that belong to the top K.  Three radix passes of 12, 10
// and 10 bits.  The first runs over every entry with 4096 bins, which spread
// float keys far better than the top byte (sign and 7 exponent bits: a dozen
// bins, so the histogram atomics serialised).  The keys of its boundary bin
// are then compacted into LDS (when they fit) and the last two passes run over
// them alone.
// key[e] == 0 marks an entry that takes no part (no float maps to order key 0).
// pre: the first pass's histogram (key >> 20 over the valid keys), when the
// caller has already built it (outside sh); otherwise it is built here.
template <int E>
__device__ void block_kth(const uint32_t (&key)[E], int K, KthWide& sh, uint32_t* T_out, int* need_eq_out,
                          const uint32_t* pre = nullptr) {
    const int tid = threadIdx.x;
    if (!pre) {
        for (int i = tid; i < kWideBins; i += kNT) sh.hist[i] = 0u;
        __syncthreads();
        // plain atomics: over 4096 bins a wave's lanes rarely share one, so the
        // per-wave pre-aggregation (a cross-lane read per entry) costs more than
        // the collisions it saves (304 against 352 us for 4096 x 32768 entries);
        // all-equal keys are the worst case, about twice as slow as pre-aggregated
#pragma unroll
        for (int e = 0; e < E; ++e)
            if ((key[e] != 0u)) atomicAdd(&sh.hist[key[e] >> 20], 1u);
        __syncthreads();
    }
    const uint32_t* h0 = pre ? pre : sh.hist;
    int bin, above;
    find_bin<kWideBins, kNT>(h0, K, sh.scan, sh.out, &bin, &above);
    const uint32_t d0 = (uint32_t)bin;
    const int c0 = (int)h0[d0];
    int rem = K - above;
    __syncthreads();   // every thread has read c0 before the histogram is cleared
    uint32_t d1;
    if (c0 <= kWideCand) {
        int mine = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) mine += ((key[e] != 0u) && (key[e] >> 20) == d0) ? 1 : 0;
        int tot;
        int off = block_excl_scan<kNT>(mine, sh.scan, &tot);
#pragma unroll
        for (int e = 0; e < E; ++e)
            if ((key[e] != 0u) && (key[e] >> 20) == d0) sh.cand[off++] = key[e] & 0xFFFFFu;
        for (int i = tid; i < 1024; i += kNT) sh.hist[i] = 0u;
        __syncthreads();
        for (int p0 = 0; p0 < c0; p0 += kNT) {
            const int p = p0 + tid;
            const bool act = p < c0;
            hist_add(sh.hist, act, act ? sh.cand[p] >> 10 : 0u);
        }
        __syncthreads();
        find_bin<1024, kNT>(sh.hist, rem, sh.scan, sh.out, &bin, &above);
        d1 = (uint32_t)bin;
        rem -= above;
        for (int i = tid; i < 1024; i += kNT) sh.hist[i] = 0u;
        __syncthreads();
        for (int p0 = 0; p0 < c0; p0 += kNT) {
            const int p = p0 + tid;
            const bool act = p < c0 && (sh.cand[p] >> 10) == d1;
            hist_add(sh.hist, act, act ? sh.cand[p] & 1023u : 0u);
        }
        __syncthreads();
    } else {
        // too many keys in the boundary bin: the same two passes over the registers
        for (int i = tid; i < 1024; i += kNT) sh.hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e) hist_add(sh.hist, (key[e] != 0u) && (key[e] >> 20) == d0, (key[e] >> 10) & 1023u);
        __syncthreads();
        find_bin<1024, kNT>(sh.hist, rem, sh.scan, sh.out, &bin, &above);
        d1 = (uint32_t)bin;
        rem -= above;
        for (int i = tid; i < 1024; i += kNT) sh.hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e)
            hist_add(sh.hist, (key[e] != 0u) && (key[e] >> 10) == ((d0 << 10) | d1), key[e] & 1023u);
        __syncthreads();
    }
    find_bin<1024, kNT>(sh.hist, rem, sh.scan, sh.out, &bin, &above);
    *T_out = (d0 << 20) | (d1 << 10) | (uint32_t)bin;
    *need_eq_out = rem - above;
}

// Writes the chosen entries (all keys > T, plus the first need_eq equal to T
// in thread order = index order) in index order; thread t holds entries
// base .. base + E - 1.  The choice is made twice (counted, then written) so
// that no per-entry flags stay live across the scans.
template <int E>
__device__ void block_choose(const uint32_t (&key)[E], uint32_t T, int need_eq, int* scan, int64_t base,
                             int32_t* out_sel, int stride) {
    int c_eq = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) c_eq += ((key[e] != 0u) && key[e] == T) ? 1 : 0;
    int tot;
    const int r0 = block_excl_scan<kNT>(c_eq, scan, &tot);
    int c_sel = 0, r = r0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const bool gt = (key[e] != 0u) && key[e] > T;
        const bool eq = (key[e] != 0u) && key[e] == T;
        c_sel += (gt || (eq && r < need_eq)) ? 1 : 0;
        r += eq ? 1 : 0;
    }
    int pos = block_excl_scan<kNT>(c_sel, scan, &tot);
    r = r0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const bool gt = (key[e] != 0u) && key[e] > T;
        const bool eq = (key[e] != 0u) && key[e] == T;
        if ((gt || (eq && r < need_eq)) && pos < stride) out_sel[pos++] = (int32_t)(base + e);
        r += eq ? 1 : 0;
    }
}

template <int E>
__device__ inline void load_scores(const float* sc, int64_t base, int n_valid, float (&x)[E], bool (&v)[E]) {
    const bool vec = E >= 4 && (((uintptr_t)(sc + base)) & 15u) == 0 && base + E <= n_valid;
    if (vec) {
#pragma unroll
        for (int e = 0; e < E; e += 4) {
            const f32x4 q = *reinterpret_cast<const f32x4*>(sc + base + e);
            x[e] = q[0];
            x[e + 1] = q[1];
            x[e + 2] = q[2];
            x[e + 3] = q[3];
        }
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = true;
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            v[e] = base + e < n_valid;
            x[e] = v[e] ? sc[base + e] : 0.0f;
        }
    }
}

// ---------------------------------------------------------------- path 0
// two workgroups per CU (eight waves per SIMD): one's passes overlap the
// other's score loads
template <int E>
__global__ __launch_bounds__(kNT, 8) void select_single(const SelectArgs a) {
    __shared__ KthWide sh;
    const int tid = threadIdx.x;
    const int seg = blockIdx.x;
    const int n_valid = seg_valid(a, seg);
    const int64_t base = (int64_t)tid * E;
    const float* sc = a.scores + (int64_t)seg * a.n_keys;

    float x[E];
    bool valid[E];
    load_scores<E>(sc, base, n_valid, x, valid);
    // order key 0 (no float has it) marks entries past n_valid or below the threshold
    uint32_t key[E];
    int c_valid = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if (a.mode == LSA_SELECT_THRESHOLD) valid[e] = valid[e] && (x[e] > a.t_f);
        key[e] = valid[e] ? order_key(x[e]) : 0u;
        c_valid += valid[e] ? 1 : 0;
    }
    int n_ok;
    block_excl_scan<kNT>(c_valid, sh.scan, &n_ok);
    const int K = n_ok < a.k ? n_ok : a.k;
    int32_t* out_sel = a.sel + (int64_t)seg * a.stride;
    if (K == 0) {
        for (int i = tid; i < a.stride; i += kNT) out_sel[i] = -1;
        if (tid == 0) a.count[seg] = 0;
        return;
    }
    uint32_t T;
    int need_eq;
    block_kth<E>(key, K, sh, &T, &need_eq);
    block_choose<E>(key, T, need_eq, sh.scan, base, out_sel, a.stride);
    for (int i = K + tid; i < a.stride; i += kNT) out_sel[i] = -1;
    if (tid == 0) a.count[seg] = K;
}

// ---------------------------------------------------------------- path 1
__device__ inline bool entry(const SelectArgs& a, const float* sc, int64_t j, int n_valid, uint32_t* key) {
    bool v = j < n_valid;
    const float x = v ? sc[j] : 0.0f;
    if (a.mode == LSA_SELECT_THRESHOLD) v = v && (x > a.t_f);
    *key = order_key(x);
    return v;
}

template <int NT>
__device__ __forceinline__ void sel_hist_body(const SelectArgs& a, const int bx, const int by) {
    constexpr int PER = kBlk / NT;
    __shared__ uint32_t h[kSelBins];
    const int tid = threadIdx.x, seg = by;
    const int64_t base = (int64_t)bx * kBlk;
    const int n_valid = seg_valid(a, seg);
    const float* sc = a.scores + (int64_t)seg * a.n_keys;
    // all loads first: one memory latency per block instead of one per entry
    float x[PER];
#pragma unroll
    for (int it = 0; it < PER; ++it) {
        const int64_t j = base + it * NT + tid;
        x[it] = j < n_valid ? sc[j] : 0.0f;
    }
    for (int i = tid; i < kSelBins; i += NT) h[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int it = 0; it < PER; ++it) {
        const int64_t j = base + it * NT + tid;
        bool v = j < n_valid;
        if (a.mode == LSA_SELECT_THRESHOLD) v = v && (x[it] > a.t_f);
        hist_add(h, v, order_key(x[it]) >> kSelShift);
    }
    __syncthreads();
    uint32_t* g = a.hist + (int64_t)seg * kSelBins;
    for (int i = tid; i < kSelBins; i += NT) {
        const uint32_t c = h[i];
        if (c) atomicAdd(&g[i], c);
    }
}

__global__ __launch_bounds__(kBlkThreads) void sel_hist_kernel(const SelectArgs a) {
    sel_hist_body<kBlkThreads>(a, blockIdx.x, blockIdx.y);
}

// From the segment histogram: out[0] = boundary bucket b* (-1 if nothing is
// chosen), out[1] = entries in buckets above b*, out[2] = valid entries.
template <int NT>
__device__ void find_boundary(const uint32_t* g, int k, int* s_scan, int* out) {
    constexpr int PER = kSelBins / NT;
    const int t = threadIdx.x;
    uint32_t c[PER];
    int local = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        c[i] = g[kSelBins - 1 - PER * t - i];
        local += (int)c[i];
    }
    int total;
    int run = block_excl_scan<NT>(local, s_scan, &total);
    const int K = total < k ? total : k;
    if (t == 0) {
        out[0] = -1;
        out[1] = 0;
        out[2] = total;
    }
    __syncthreads();
    if (K > 0) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (run < K && run + (int)c[i] >= K) {
                out[0] = kSelBins - 1 - PER * t - i;
                out[1] = run;
            }
            run += (int)c[i];
        }
    }
    __syncthreads();
}

// Every 1024-entry block keeps, in index order, its entries in buckets >= b*
// (those above b* are chosen for sure; those in b* are the candidates), with
// their keys; the top index bit marks a candidate.
__device__ __forceinline__ void sel_collect_body(const SelectArgs& a, const int bx, const int by) {
    constexpr int PER = kColBlk / kBlkThreads;   // 4 consecutive entries per thread
    __shared__ int s_scan[kBlkThreads / 64 + 1];
    __shared__ int s_b[3];
    const int tid = threadIdx.x, seg = by, blk = bx;
    const int n_valid = seg_valid(a, seg);
    const float* sc = a.scores + (int64_t)seg * a.n_keys;
    const int64_t base = (int64_t)blk * kColBlk + tid * PER;
    float x[PER];
    bool v[PER];
    load_scores<PER>(sc, base, n_valid, x, v);
    find_boundary<kBlkThreads>(a.hist + (int64_t)seg * kSelBins, a.k, s_scan, s_b);
    const int bstar = s_b[0];
    uint32_t key[PER];
    int keep[PER];
    int c = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        if (a.mode == LSA_SELECT_THRESHOLD) v[e] = v[e] && (x[e] > a.t_f);
        key[e] = order_key(x[e]);
        const int bin = (int)(key[e] >> kSelShift);
        keep[e] = (bstar >= 0 && v[e] && bin >= bstar) ? (bin == bstar ? 2 : 1) : 0;
        c += keep[e] ? 1 : 0;
    }
    int tot;
    int pos = block_excl_scan<kBlkThreads>(c, s_scan, &tot);
    const int64_t ob = ((int64_t)seg * a.nblk + blk) * kColBlk;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        if (!keep[e]) continue;
        a.blk_idx[ob + pos] = (int32_t)(base + e) | (keep[e] == 2 ? (int32_t)0x80000000 : 0);
        a.blk_key[ob + pos] = key[e];
        ++pos;
    }
    if (tid == 0) a.blk_count[(int64_t)seg * a.nblk + blk] = tot;
}

__global__ __launch_bounds__(kBlkThreads) void sel_collect_kernel(const SelectArgs a) {
    sel_collect_body(a, blockIdx.x, blockIdx.y);
}

// Exact selection straight from the scores by one workgroup: four radix passes
// over the whole segment, then an index-ordered compaction.  Used when the
// boundary bucket overflows the candidate list.
template <int NT>
__device__ uint32_t stream_select(const SelectArgs& a, const float* sc, int n_valid, int K, KthShared& sh,
                                  int32_t* out_sel) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0, mask = 0;
    int rem = K;
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        if (tid < 256) sh.hist[tid] = 0u;
        __syncthreads();
        for (int64_t c = 0; c < n_valid; c += NT) {
            uint32_t key;
            const bool v = entry(a, sc, c + tid, n_valid, &key);
            hist_add(sh.hist, v && (key & mask) == prefix, (key >> shift) & 255u);
        }
        __syncthreads();
        find_digit(sh.hist, rem, sh);
        prefix |= sh.digit << shift;
        mask |= 255u << shift;
        rem -= sh.above;
        __syncthreads();
    }
    const uint32_t T = prefix;
    const int need_eq = rem;
    constexpr int E = 8;
    int run_eq = 0, run_out = 0;
    for (int64_t c = 0; c < n_valid; c += (int64_t)NT * E) {
        uint32_t key[E];
        bool v[E];
        int c_eq = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            v[e] = entry(a, sc, c + (int64_t)tid * E + e, n_valid, &key[e]);
            c_eq += (v[e] && key[e] == T) ? 1 : 0;
        }
        int tot_eq;
        int r = run_eq + block_excl_scan<NT>(c_eq, sh.scan, &tot_eq);
        bool take[E];
        int c_take = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const bool eq = v[e] && key[e] == T;
            take[e] = (v[e] && key[e] > T) || (eq && r < need_eq);
            r += eq ? 1 : 0;
            c_take += take[e] ? 1 : 0;
        }
        int tot_take;
        int pos = run_out + block_excl_scan<NT>(c_take, sh.scan, &tot_take);
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (take[e] && pos < a.stride) out_sel[pos++] = (int32_t)(c + (int64_t)tid * E + e);
        run_eq += tot_eq;
        run_out += tot_take;
    }
    return T;
}

// One workgroup of NT threads per segment: gathers the blocks' kept entries (global index
// order), resolves the boundary bucket with a radix pass over key bits 20..10
// and then bits 9..0 -- by ranking the members of the bin found when they are
// few, else by a second radix pass -- and writes the chosen indices (already
// ascending).
constexpr int kFewMembers = 64;
template <int NT, int MAXB = kMaxBlocks>
__device__ __forceinline__ void sel_final_body(const SelectArgs& a, const int seg) {
    __shared__ KthShared sh;
    __shared__ int s_b[3];
    __shared__ int32_t s_idx[kSelKeepCap];
    __shared__ uint32_t s_key[kSelKeepCap];
    __shared__ int s_start[MAXB + 1];
    __shared__ uint32_t s_h2[2048];
    __shared__ uint32_t s_few[kFewMembers];
    __shared__ int s_few_n, s_few_t[2];
    const int tid = threadIdx.x;
    uint32_t* g = a.hist + (int64_t)seg * kSelBins;
    // the blocks' counts are loaded before the histogram is scanned (thread t
    // owns blocks [t*PB, (t+1)*PB)), so the two reads overlap
    const int nb = a.nblk;
    const int stride = a.blk_stride ? a.blk_stride : kColBlk;   // entries per block list
    const int PB = (nb + NT - 1) / NT;
    constexpr int kPB = (MAXB + NT - 1) / NT;   // PB <= kPB whenever nb <= MAXB
    const int32_t* cnt = a.blk_count + (int64_t)seg * nb;
    // counts stay in registers for the block offsets below (no second read)
    int c_own[kPB];
    int mine = 0;
#pragma unroll
    for (int q = 0; q < kPB; ++q) {
        const int bi = tid * PB + q;
        c_own[q] = (q < PB && bi < nb) ? cnt[bi] : 0;
        mine += c_own[q];
    }
    int32_t* out_sel = a.sel + (int64_t)seg * a.stride;
    // pre: the lists hold every entry of bin >= the guess (every passing entry
    // in threshold mode), so the boundary bin b* comes from the listed entries
    // themselves; otherwise from the segment's histogram
    const bool pre = a.pre != 0;
    int K = 0, bstar = 0, above = 0, gn = 0;
    if (!pre) {
        find_boundary<NT>(g, a.k, sh.scan, s_b);
        const int total = s_b[2];
        K = total < a.k ? total : a.k;
        bstar = s_b[0];
        above = s_b[1];
        if (K == 0) mine = 0;
    }
    // pre: the listed entries' bins are counted as they are gathered
    if (pre)
        for (int i = tid; i < kSelBins; i += NT) s_h2[i] = 0u;
    // block offsets; n_keep = listed entries
    int n_keep;
    int off = block_excl_scan<NT>(mine, sh.scan, &n_keep);
    if (pre) {
        const int nv = seg_valid(a, seg);
        const int avail = a.mode == LSA_SELECT_THRESHOLD ? n_keep : nv;
        K = avail < a.k ? avail : a.k;
    }
    // with lists from the score launch the guess held if they list K entries
    const bool in_lds = K > 0 && n_keep <= kSelKeepCap && nb <= MAXB && (!pre || n_keep >= K);
    if (in_lds) {
        // every block's first position in the gathered list
#pragma unroll
        for (int q = 0; q < kPB; ++q) {
            const int bi = tid * PB + q;
            if (q < PB && bi < nb) s_start[bi] = off;
            off += c_own[q];
        }
        if (tid == 0) s_start[nb] = n_keep;
        __syncthreads();
        // all threads copy: entry p belongs to the last block starting at or before p.
        // A thread's entries are all loaded before any is stored, so the gather
        // costs one memory round trip however many entries each thread takes.
        constexpr int kGather = (kSelKeepCap + NT - 1) / NT;
        int32_t g_idx[kGather];
        uint32_t g_key[kGather];
#pragma unroll
        for (int i = 0; i < kGather; ++i) {
            const int p = tid + i * NT;
            if (p < n_keep) {
                int lo = 0, hi = nb - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (s_start[mid] <= p) lo = mid; else hi = mid - 1;
                }
                const int64_t src = ((int64_t)seg * nb + lo) * stride + (p - s_start[lo]);
                g_idx[i] = a.blk_idx[src];
                g_key[i] = a.blk_key[src];
            }
        }
#pragma unroll
        for (int i = 0; i < kGather; ++i) {
            const int p = tid + i * NT;
            if (p < n_keep) {
                s_idx[p] = g_idx[i];
                s_key[p] = g_key[i];
                if (pre) atomicAdd(&s_h2[g_key[i] >> kSelShift], 1u);
            }
        }
        __syncthreads();
        if (pre) {
            // b* and the count above it from the listed bins' histogram; entries
            // listed below b* stay in place (every later pass tests the bin)
            find_boundary<NT>(s_h2, K, sh.scan, s_b);
            bstar = s_b[0];
            above = s_b[1];
            const int at_b = above + (int)s_h2[bstar];
            // the next step's guess: b*, or one bin lower when b* and above hold
            // fewer than 1.5 times the entries chosen
            gn = (2 * at_b < 3 * K && bstar > 0) ? bstar - 1 : bstar;
            __syncthreads();   // s_h2 is read before the passes below reuse it
        }
        // bits 20..0 of the candidates' keys (bucket b* fixes the rest): a radix
        // pass over bits 20..10, then bits 9..0 of the candidates in the bin found
        const int need = K - above;
        for (int i = tid; i < 2048; i += NT) s_h2[i] = 0u;
        __syncthreads();
        // (plain atomics: 2048 bins spread these digits; see select_single)
        for (int p0 = 0; p0 < n_keep; p0 += NT) {
            const int p = p0 + tid;
            if (p < n_keep && (int)(s_key[p] >> kSelShift) == bstar) atomicAdd(&s_h2[(s_key[p] >> 10) & 2047u], 1u);
        }
        __syncthreads();
        int bin, bin_above;
        find_bin<2048, NT>(s_h2, need, sh.scan, s_b, &bin, &bin_above);
        const uint32_t d1 = (uint32_t)bin;
        const int rem = need - bin_above;
        const int c_d1 = (int)s_h2[d1];   // candidates in bin d1; 1 <= rem <= c_d1
        uint32_t low_T;
        int need_eq;
        __syncthreads();   // every thread has read c_d1 before s_h2 or the counter changes
        if (c_d1 <= kFewMembers) {   // uniform
            // few keys share bin d1 (the usual case): rank them against each other
            // instead of a second histogram pass.  Each member counts the members
            // above and equal to it; the one whose range holds rank rem gives T's
            // low bits and how many keys equal to T are taken.
            if (tid == 0) s_few_n = 0;
            __syncthreads();
            for (int p0 = 0; p0 < n_keep; p0 += NT) {
                const int p = p0 + tid;
                if (p < n_keep && (int)(s_key[p] >> kSelShift) == bstar && ((s_key[p] >> 10) & 2047u) == d1)
                    s_few[atomicAdd(&s_few_n, 1)] = s_key[p] & 1023u;
            }
            __syncthreads();
            if (tid < c_d1) {
                const uint32_t me = s_few[tid];
                int gt = 0, eq = 0;
                for (int i = 0; i < c_d1; ++i) {
                    const uint32_t o = s_few[i];
                    gt += o > me ? 1 : 0;
                    eq += o == me ? 1 : 0;
                }
                if (gt < rem && rem <= gt + eq) {   // every such member writes the same pair
                    s_few_t[0] = (int)me;
                    s_few_t[1] = rem - gt;
                }
            }
            __syncthreads();
            low_T = (uint32_t)s_few_t[0];
            need_eq = s_few_t[1];
        } else {
            for (int i = tid; i < 1024; i += NT) s_h2[i] = 0u;
            __syncthreads();
            for (int p0 = 0; p0 < n_keep; p0 += NT) {
                const int p = p0 + tid;
                const bool act = p < n_keep && (int)(s_key[p] >> kSelShift) == bstar && ((s_key[p] >> 10) & 2047u) == d1;
                hist_add(s_h2, act, p < n_keep ? s_key[p] & 1023u : 0u);
            }
            __syncthreads();
            find_bin<1024, NT>(s_h2, rem, sh.scan, s_b, &bin, &bin_above);
            low_T = (uint32_t)bin;
            need_eq = rem - bin_above;
        }
        const uint32_t T = ((uint32_t)bstar << kSelShift) | (d1 << 10) | low_T;
        // index-ordered placement with one scan: thread t takes entries [t*E2, t*E2 + E2);
        // an entry above T (every entry above b*, and candidates > T; listed
        // entries below b* are below T and take no place) goes to
        // (entries above T before it) + min(candidates equal to T before it, need_eq),
        // and the first need_eq candidates equal to T fill in between
        const int E2 = (n_keep + NT - 1) / NT;   // <= kSelKeepCap / NT
        const int q0 = tid * E2;
        int c_gt = 0, c_eq = 0;
        for (int e = 0; e < E2; ++e) {
            const int p = q0 + e;
            if (p >= n_keep) break;
            const int32_t raw = s_idx[p];
            const uint32_t k2 = s_key[p];
            if (k2 > T) ++c_gt;
            else if (k2 == T) ++c_eq;
        }
        int tot;
        const int packed = block_excl_scan<NT>(c_gt | (c_eq << 16), sh.scan, &tot);
        int n_gt = packed & 0xFFFF, n_eq = packed >> 16;
        for (int e = 0; e < E2; ++e) {
            const int p = q0 + e;
            if (p >= n_keep) break;
            const int32_t raw = s_idx[p];
            const uint32_t k2 = s_key[p];
            if (k2 > T) {
                const int pos = n_gt + (n_eq < need_eq ? n_eq : need_eq);
                if (pos < a.stride) out_sel[pos] = raw & 0x7FFFFFFF;
                ++n_gt;
            } else if (k2 == T) {
                if (n_eq < need_eq && n_gt + n_eq < a.stride) out_sel[n_gt + n_eq] = raw & 0x7FFFFFFF;
                ++n_eq;
            }
        }
    } else if (pre && K > 0) {
        // the guess failed (too few listed, or too many): the exact scan; the
        // next step's lists start one bin below this step's K-th key
        const uint32_t T = stream_select<NT>(a, a.scores + (int64_t)seg * a.n_keys, seg_valid(a, seg), K, sh, out_sel);
        const int bt = (int)(T >> kSelShift);
        gn = bt > 0 ? bt - 1 : 0;
    } else if (K > 0) {
        stream_select<NT>(a, a.scores + (int64_t)seg * a.n_keys, seg_valid(a, seg), K, sh, out_sel);
    }
    for (int i = K + tid; i < a.stride; i += NT) out_sel[i] = -1;
    if (tid == 0) {
        a.count[seg] = K;
        if (a.guess_out) {
            if (!pre && K > 0) {
                // from the histogram: b*, or one bin lower when b* and above hold
                // fewer than 1.5 times the entries chosen and the lower bin
                // keeps the lists within half the LDS list
                const int at_b = above + (int)g[bstar];
                gn = bstar;
                if (2 * at_b < 3 * K && bstar > 0 && at_b + (int)g[bstar - 1] <= kSelKeepCap / 2) gn = bstar - 1;
            }
            a.guess_out[seg] = gn;   // no entry chosen: the lists start at bin 0
        }
    }
    if (!pre) {
        __syncthreads();
        for (int i = tid; i < kSelBins; i += NT) g[i] = 0u;
    }
}

__global__ __launch_bounds__(kNT) void sel_final_kernel(const SelectArgs a) {
    sel_final_body<kNT>(a, blockIdx.x);
}

int next_pow2(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

}  // namespace select_k
#ifndef LSA_BODIES_ONLY
using namespace select_k;
#endif
}  // namespace

#ifndef LSA_BODIES_ONLY
bool select_plan(SelectArgs* a, size_t* zero_bytes, size_t* ws_bytes) {
    if (a->k > 4096) return false;
    if (a->n_keys <= kSelSingle) {
        a->path = 0;
        a->e1 = next_pow2((int)((a->n_keys + kNT - 1) / kNT));
        if (a->e1 < 1) a->e1 = 1;
        a->nblk = 0;
        *zero_bytes = 0;
        *ws_bytes = 0;
        return true;
    }
    a->path = 1;
    a->e1 = 0;
    a->nblk = (int)((a->n_keys + kColBlk - 1) / kColBlk);
    *zero_bytes = (size_t)a->n_seg * kSelBins * 4;
    const size_t nb = (size_t)a->n_seg * a->nblk;
    // counts for four lists per block: the score launch's lists cover a
    // quarter block each
    *ws_bytes = nb * 16 + 256 + nb * kColBlk * 8 + 256;
    return true;
}

void select_bind(SelectArgs* a, void* zero_region, void* ws) {
    if (a->path != 1) return;
    a->hist = static_cast<uint32_t*>(zero_region);
    char* w = static_cast<char*>(ws);
    const size_t nb = (size_t)a->n_seg * a->nblk;
    a->blk_count = reinterpret_cast<int32_t*>(w);
    w += (nb * 16 + 255) / 256 * 256;
    a->blk_idx = reinterpret_cast<int32_t*>(w);
    a->blk_key = reinterpret_cast<uint32_t*>(w + nb * kColBlk * 4);
}

hipError_t launch_fm_select_final(const SelectArgs& a, hipStream_t s) {
    if (a.path == 0) return launch_fm_select(a, s);
    hipLaunchKernelGGL(sel_final_kernel, dim3(a.n_seg), dim3(kNT), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_fm_select(const SelectArgs& a, hipStream_t s) {
    if (a.path == 0) {
        const dim3 grid(a.n_seg), block(kNT);
        switch (a.e1) {
            case 1: hipLaunchKernelGGL(select_single<1>, grid, block, 0, s, a); break;
            case 2: hipLaunchKernelGGL(select_single<2>, grid, block, 0, s, a); break;
            case 4: hipLaunchKernelGGL(select_single<4>, grid, block, 0, s, a); break;
            case 8: hipLaunchKernelGGL(select_single<8>, grid, block, 0, s, a); break;
            case 16: hipLaunchKernelGGL(select_single<16>, grid, block, 0, s, a); break;
            case 32: hipLaunchKernelGGL(select_single<32>, grid, block, 0, s, a); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    const dim3 gh((unsigned)((a.n_keys + kBlk - 1) / kBlk), a.n_seg);
    hipLaunchKernelGGL(sel_hist_kernel, gh, dim3(kBlkThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sel_collect_kernel, dim3(a.nblk, a.n_seg), dim3(kBlkThreads), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sel_final_kernel, dim3(a.n_seg), dim3(kNT), 0, s, a);
    return hipGetLastError();
}

#endif  // LSA_BODIES_ONLY

}  // namespace lsa
