// fm_select: top-k / sigmoid-threshold selection of compressed entries.
//
// [P1] "global top-k (512 chunks)", index_topk = global_keep_cap = 512;
// [P2] Recall / Threshold Selector: entries whose sigmoid(score) exceeds a
// threshold are recalled.  Order: score descending, index ascending on ties.
// Threshold mode keeps score > t_f (t_f = largest float <= logit(tau), worked
// out on the host), then caps at k by the same order.  Output: the chosen
// indices in ascending order, -1 padding, and the count.
//
// Design (gfx950): scores become order-preserving 32-bit keys (-0 folded into
// +0).  A 1024-thread workgroup holds up to 32768 keys in registers (E per
// thread, contiguous indices per thread so thread order is index order) and
// finds the K-th largest key T by four 8-bit radix passes over LDS
// histograms (one histogram per wave; each wave first adds the lanes that
// share the first active lane's digit with one atomic, which takes the
// contention out of the clustered high digits).  The chosen set is every key
// > T plus the lowest-indexed (K - #greater) keys equal to T: two block
// scans (ties by index, then output positions) compact it in index order.
// Long segments run two stages: blocks of 1024*E entries emit their own
// top-k candidates in index order; one workgroup per segment then selects
// from the concatenated candidates.  The global top-k is always inside the
// union of per-block top-k sets, so the result is exact.
#include "lsa_internal.hpp"

namespace lsa {

namespace {

constexpr int kNT = 1024;
constexpr int kNW = kNT / 64;

struct SelShared {
    uint32_t hist[kNW][256];
    int scan[kNW + 1];
    uint32_t digit;
    int above;
};

// K-th largest key among the valid ones (1 <= K <= #valid).  Returns T and the
// number of keys equal to T that belong to the top K.
template <int E>
__device__ void block_kth(const uint32_t (&key)[E], const bool (&valid)[E], int K, SelShared& sh,
                          uint32_t* T_out, int* need_eq_out) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t prefix = 0, mask = 0;
    int rem = K;
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int i = tid; i < kNW * 256; i += kNT) (&sh.hist[0][0])[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const bool act = valid[e] && (key[e] & mask) == prefix;
            const uint32_t dg = (key[e] >> shift) & 255u;
            const uint64_t am = __ballot(act);
            if (am) {
                const int first = __ffsll((unsigned long long)am) - 1;
                const uint32_t d0 = __shfl(dg, first, 64);
                const uint64_t same = __ballot(act && dg == d0);
                if (lane == first) atomicAdd(&sh.hist[wave][d0], (uint32_t)__popcll(same));
                if (act && dg != d0) atomicAdd(&sh.hist[wave][dg], 1u);
            }
        }
        __syncthreads();
        // thread tid < 256 owns digit 255 - tid, so an inclusive scan over tid
        // counts the keys whose digit is >= that digit
        const uint32_t d = 255u - (uint32_t)(tid & 255);
        int cnt = 0;
        if (tid < 256) {
#pragma unroll
            for (int w = 0; w < kNW; ++w) cnt += (int)sh.hist[w][d];
        }
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
        prefix |= sh.digit << shift;
        mask |= 255u << shift;
        rem -= sh.above;
        __syncthreads();
    }
    *T_out = prefix;
    *need_eq_out = rem;
}

// Marks the chosen keys (all > T, plus the first need_eq equal to T in index
// order) and returns each chosen key's output position in index order.
template <int E>
__device__ void block_choose(const uint32_t (&key)[E], const bool (&valid)[E], uint32_t T, int need_eq,
                             SelShared& sh, bool (&take)[E], int* pos0) {
    int c_eq = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) c_eq += (valid[e] && key[e] == T) ? 1 : 0;
    int tot;
    int r = block_excl_scan<kNT>(c_eq, sh.scan, &tot);
    int c_sel = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const bool gt = valid[e] && key[e] > T;
        const bool eq = valid[e] && key[e] == T;
        take[e] = gt || (eq && r < need_eq);
        r += eq ? 1 : 0;
        c_sel += take[e] ? 1 : 0;
    }
    *pos0 = block_excl_scan<kNT>(c_sel, sh.scan, &tot);
}

template <int E>
__global__ __launch_bounds__(kNT) void select_stage1(const SelectArgs a) {
    __shared__ SelShared sh;
    const int tid = threadIdx.x;
    const int seg = blockIdx.y, blk = blockIdx.x;
    const int n_valid = a.has_n_valid ? a.n_valid[seg] : a.n_valid_uniform;
    const int64_t base = (int64_t)blk * (kNT * E) + (int64_t)tid * E;
    const float* sc = a.scores + (int64_t)seg * a.n_keys;

    uint32_t key[E];
    bool valid[E];
    int c_valid = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int64_t j = base + e;
        bool v = j < n_valid;
        const float x = v ? sc[j] : 0.0f;
        if (a.mode == LSA_SELECT_THRESHOLD) v = v && (x > a.t_f);
        key[e] = order_key(x);
        valid[e] = v;
        c_valid += v ? 1 : 0;
    }
    int n_ok;
    block_excl_scan<kNT>(c_valid, sh.scan, &n_ok);
    const int K = n_ok < a.k ? n_ok : a.k;

    const bool final_stage = a.nblk == 1;
    int32_t* out_sel = a.sel + (int64_t)seg * a.stride;
    if (K == 0) {
        if (final_stage) {
            for (int i = tid; i < a.stride; i += kNT) out_sel[i] = -1;
            if (tid == 0) a.count[seg] = 0;
        } else if (tid == 0) {
            a.cand_n[seg * a.nblk + blk] = 0;
        }
        return;
    }
    uint32_t T;
    int need_eq;
    block_kth<E>(key, valid, K, sh, &T, &need_eq);
    bool take[E];
    int pos;
    block_choose<E>(key, valid, T, need_eq, sh, take, &pos);
    if (final_stage) {
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (take[e] && pos < a.stride) out_sel[pos++] = (int32_t)(base + e);
        for (int i = K + tid; i < a.stride; i += kNT) out_sel[i] = -1;
        if (tid == 0) a.count[seg] = K;
    } else {
        const int64_t cb = ((int64_t)seg * a.nblk + blk) * a.k;
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (take[e] && pos < a.k) {
                a.cand_key[cb + pos] = key[e];
                a.cand_idx[cb + pos] = (int32_t)(base + e);
                ++pos;
            }
        if (tid == 0) a.cand_n[seg * a.nblk + blk] = K;
    }
}

template <int E>
__global__ __launch_bounds__(kNT) void select_stage2(const SelectArgs a) {
    __shared__ SelShared sh;
    const int tid = threadIdx.x;
    const int seg = blockIdx.x;
    const int slots = a.nblk * a.k;
    const int64_t cb = (int64_t)seg * slots;

    uint32_t key[E];
    int32_t idx[E];
    bool valid[E];
    int c_valid = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int p = tid * E + e;
        bool v = p < slots;
        if (v) v = (p % a.k) < a.cand_n[seg * a.nblk + p / a.k];
        key[e] = v ? a.cand_key[cb + p] : 0u;
        idx[e] = v ? a.cand_idx[cb + p] : 0;
        valid[e] = v;
        c_valid += v ? 1 : 0;
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
    block_kth<E>(key, valid, K, sh, &T, &need_eq);
    bool take[E];
    int pos;
    block_choose<E>(key, valid, T, need_eq, sh, take, &pos);
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (take[e] && pos < a.stride) out_sel[pos++] = idx[e];
    for (int i = K + tid; i < a.stride; i += kNT) out_sel[i] = -1;
    if (tid == 0) a.count[seg] = K;
}

int next_pow2(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

hipError_t launch_s1(const SelectArgs& a, hipStream_t s) {
    const dim3 grid(a.nblk, a.n_seg), block(kNT);
    switch (a.e1) {
        case 1: hipLaunchKernelGGL(select_stage1<1>, grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL(select_stage1<2>, grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL(select_stage1<4>, grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL(select_stage1<8>, grid, block, 0, s, a); break;
        case 16: hipLaunchKernelGGL(select_stage1<16>, grid, block, 0, s, a); break;
        case 32: hipLaunchKernelGGL(select_stage1<32>, grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_s2(const SelectArgs& a, hipStream_t s) {
    const dim3 grid(a.n_seg), block(kNT);
    switch (a.e2) {
        case 1: hipLaunchKernelGGL(select_stage2<1>, grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL(select_stage2<2>, grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL(select_stage2<4>, grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL(select_stage2<8>, grid, block, 0, s, a); break;
        case 16: hipLaunchKernelGGL(select_stage2<16>, grid, block, 0, s, a); break;
        case 32: hipLaunchKernelGGL(select_stage2<32>, grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

// Chooses the stage shapes; returns 0 when the problem is out of range.
size_t select_workspace_bytes(int n_seg, int64_t n_keys, int k, int* nblk, int* e1, int* e2) {
    if (n_keys <= 32768) {
        *nblk = 1;
        *e1 = next_pow2((int)((n_keys + kNT - 1) / kNT));
        if (*e1 < 1) *e1 = 1;
        *e2 = 0;
        return 1;
    }
    int E = 8;
    int64_t nb = (n_keys + (int64_t)kNT * E - 1) / ((int64_t)kNT * E);
    while (nb * k > 32768 && E < 32) {
        E *= 2;
        nb = (n_keys + (int64_t)kNT * E - 1) / ((int64_t)kNT * E);
    }
    if (nb * k > 32768) return 0;
    *nblk = (int)nb;
    *e1 = E;
    *e2 = next_pow2((int)((nb * k + kNT - 1) / kNT));
    return (size_t)n_seg * nb * k * 8 + (size_t)n_seg * nb * 4 + 256;
}

hipError_t launch_fm_select(const SelectArgs& a, hipStream_t s) {
    hipError_t e = launch_s1(a, s);
    if (e != hipSuccess || a.nblk == 1) return e;
    return launch_s2(a, s);
}

}  // namespace lsa
