// lsa_attend: decode attention over the sliding window plus the staged
// compressed entries, every row used as both key and value.
//
// [P1] overview "Two-tier KV cache" and per-layer indexed_cached_attention
// (window + selected), reading d_kv_cache[physical_id]:
//   out[h,:] = sum_r softmax_r(scale * q[h,:] . kv[phys[r],:]) * kv[phys[r],:]
//
// Design (gfx950): flash-decode split over rows.  All heads share the rows
// (MQA-like), so a workgroup of 8 waves issues every load of one 32-row tile
// at once, stages it in LDS, and computes the 16-head x 32-row score block and
// the 16-head x D output block with v_mfma_f32_16x16x4f32: QK^T splits the rows
// over 2 waves and the D (contraction) dimension over 4, the softmax runs on
// 32 lanes per head, PV splits D over the 8 waves.  Each split
// writes its running max, softmax denominator and unnormalised output; a
// second kernel merges the splits in split order.  Split s always covers list
// rows [32 s, 32 s + 32), so the arithmetic depends only on the list length
// and the row contents -- not on which physical rows hold them.
#include "lsa_internal.hpp"

namespace lsa {

namespace {
namespace attend_k {

constexpr int kR = kAttendRows;   // rows per split
constexpr int kThreads = 512;
constexpr int kMaxSplits = kAttendMaxRows / kAttendRows;

template <typename KT>
__device__ inline float ld_elem(const char* p);
template <>
__device__ inline float ld_elem<float>(const char* p) { return *reinterpret_cast<const float*>(p); }
template <>
__device__ inline float ld_elem<uint16_t>(const char* p) {
    return __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(p)) << 16);
}

template <typename KT>
__device__ inline void unpack(const uint4& u, float* out);
template <>
__device__ inline void unpack<float>(const uint4& u, float* out) {
    out[0] = __uint_as_float(u.x);
    out[1] = __uint_as_float(u.y);
    out[2] = __uint_as_float(u.z);
    out[3] = __uint_as_float(u.w);
}
template <>
__device__ inline void unpack<uint16_t>(const uint4& u, float* out) {
    out[0] = bf16_lo(u.x);
    out[1] = bf16_hi(u.x);
    out[2] = bf16_lo(u.y);
    out[3] = bf16_hi(u.y);
    out[4] = bf16_lo(u.z);
    out[5] = bf16_hi(u.z);
    out[6] = bf16_lo(u.w);
    out[7] = bf16_hi(u.w);
}

template <int D, typename KT>
constexpr int tile_bytes() { return kR * (D * (int)sizeof(KT) + 16); }

// Stores and loads of data that another workgroup reads or wrote in the same
// launch: agent-scope relaxed atomics, which the L2 of every XCD passes through
// to the device's coherence point (no whole-cache write-back or invalidate).
__device__ __forceinline__ void st_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// tile: LDS of tile_bytes<D, KT>() bytes, 16-byte aligned, from the caller.
// Returns whether the split holds rows (false: it returned before any work);
// *n_out is the clamped row count.  COH: the partials are stored with agent
// scope, for a merge in the same launch.
template <int D, typename KT, bool COH = false>
__device__ __forceinline__ bool attend_split_body(const AttendArgs& a, const int bx, const int by, const int bz,
                                                  char* tile, int* n_out = nullptr) {
    constexpr int RB = D * (int)sizeof(KT);          // row bytes
    constexpr int LS = RB + 16;                      // LDS row stride
    constexpr int CPR = RB / 16;                     // 16-byte chunks per row
    constexpr int LOADS = kR * CPR / kThreads;       // 16-byte row loads per thread
    constexpr int RSTEP = kThreads / CPR;            // rows covered by one round of loads
    constexpr int QK_STEPS = D / 16;                 // per lane: a quarter of D over 4 k-lanes
    constexpr int PER_READ = 16 / (int)sizeof(KT);
    constexpr int NB = D / 128;                      // 16-wide output blocks per wave in PV
    static_assert(LOADS >= 1 && (kR * CPR) % kThreads == 0, "tile must split evenly");

    __shared__ float sS[4][16][kR];
    __shared__ float sP[16][kR + 1];   // padded: the PV reads of one row of P hit 16 banks
    __shared__ int s_ph[kR];
    __shared__ int s_src[kR];

    const AttendLayer& L = a.L[bz];
    const int b = by, split = bx;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r0 = split * kR;
    // scores: S[h][r] = q[h] . row[r]; wave = (row block nb, quarter kq of D).  The
    // query loads go first, unconditionally (a head past hq reads head 0 and is
    // zeroed after), so they overlap the row-list round trip instead of waiting
    // behind the row loads
    const int nb = wave & 1, kq = wave >> 1;
    const int h = lane & 15, g = lane >> 4;
    const int e0 = kq * (D / 4) + g * QK_STEPS;
    f32x4 q4[QK_STEPS / 4];
    {
        const float* qp = L.q + ((int64_t)b * a.hq + (h < a.hq ? h : 0)) * D + e0;
#pragma unroll
        for (int s = 0; s < QK_STEPS; s += 4) q4[s / 4] = *reinterpret_cast<const f32x4*>(qp + s);
    }
    // the row count and this split's row list load together (one memory round trip)
    int p = -1, sr = -1;
    if (tid < kR && r0 + tid < L.phys_stride) {
        p = L.phys[(int64_t)b * L.phys_stride + r0 + tid];
        if (L.src) sr = L.src[(int64_t)b * L.phys_stride + r0 + tid];
    }
    int n = L.n_rows[b];
    n = n < 0 ? 0 : (n > L.phys_stride ? L.phys_stride : n);
    if (n_out) *n_out = n;
    if (r0 >= n) return false;   // uniform
    const int cnt = n - r0 < kR ? n - r0 : kR;
    const int pair = bz * a.batch + b;
    // wait for the row list here, on every lane: loaded under a branch, it would
    // otherwise make the compiler wait for every outstanding load before each
    // row load that reuses its registers, one round trip per row load
    asm volatile("" ::"v"(p), "v"(sr));

    if (tid < kR) {
        if (tid >= cnt) p = sr = -1;
        s_ph[tid] = (p >= 0 && p < L.kv_rows) ? p : -1;
        s_src[tid] = (sr >= 0 && sr < L.cold_rows && s_ph[tid] >= 0) ? sr : -1;
    }
    __syncthreads();
    // every row load of the tile is issued before any is used; a row staged
    // in this step comes from the cold pool and is written into its slot
    const char* kvb = static_cast<const char*>(L.kv) + (int64_t)b * L.kv_stride_b * (int64_t)sizeof(KT);
    const char* cb = static_cast<const char*>(L.cold) + (int64_t)b * L.cold_stride_b;
    const int cc = tid % CPR, rr = tid / CPR;
    uint4 v[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int r = rr + i * RSTEP;
        const int p = s_ph[r], sr = s_src[r];
        const char* from = sr >= 0 ? cb + (int64_t)sr * RB : kvb + (int64_t)p * RB;
        v[i] = p >= 0 ? *reinterpret_cast<const uint4*>(from + cc * 16) : make_uint4(0u, 0u, 0u, 0u);
    }
    if (L.src) {
        char* kvw = static_cast<char*>(L.kv_w) + (int64_t)b * L.kv_stride_b * (int64_t)sizeof(KT);
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int r = rr + i * RSTEP;
            if (s_src[r] >= 0) *reinterpret_cast<uint4*>(kvw + (int64_t)s_ph[r] * RB + cc * 16) = v[i];
        }
    }
    float qa[QK_STEPS];
#pragma unroll
    for (int s = 0; s < QK_STEPS; ++s) qa[s] = h < a.hq ? q4[s / 4][s % 4] : 0.0f;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) *reinterpret_cast<uint4*>(tile + (rr + i * RSTEP) * LS + cc * 16) = v[i];
    __syncthreads();
    {
        const char* rowp = tile + (nb * 16 + h) * LS + e0 * (int)sizeof(KT);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int rd = 0; rd < QK_STEPS / PER_READ; ++rd) {
            float kb[PER_READ];
            unpack<KT>(*reinterpret_cast<const uint4*>(rowp + rd * 16), kb);
#pragma unroll
            for (int e = 0; e < PER_READ; ++e)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[rd * PER_READ + e], kb[e], acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) sS[kq][4 * g + r][nb * 16 + h] = acc[r];
    }
    __syncthreads();

    // softmax over this split's rows: 32 lanes per head, fixed-pattern reductions
    float* ml = a.part_ml + ((int64_t)pair * a.max_splits + split) * 32;
    {
        const int hh = tid >> 5, r = tid & 31;
        const bool in = r < cnt;
        const float z = in ? (((sS[0][hh][r] + sS[1][hh][r]) + sS[2][hh][r]) + sS[3][hh][r]) * a.scale : -INFINITY;
        float m = z;
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 32));
        const float p = in ? expf(z - m) : 0.0f;
        float l = p;
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) l += __shfl_xor(l, o, 32);
        sP[hh][r] = p;
        if (r == 0) {
            if (COH) {
                st_agent(ml + hh, m);
                st_agent(ml + 16 + hh, l);
            } else {
                ml[hh] = m;
                ml[16 + hh] = l;
            }
        }
    }
    __syncthreads();

    // unnormalised output O[h][d] = sum_r P[h][r] row[r][d]; wave = D/8 columns
    {
        const int d0 = wave * (D / 8);
        f32x4 acc[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        // step s takes rows (s & 3) + 4 g + 16 (s >> 2): the four k-lanes read rows
        // four apart, 16 LDS banks apart with the row padding
#pragma unroll
        for (int s = 0; s < kR / 4; ++s) {
            const int r = (s & 3) + 4 * g + 16 * (s >> 2);
            const float pa = sP[h][r];
            const char* rp = tile + r * LS;
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const float vb = ld_elem<KT>(rp + (d0 + 16 * i + h) * (int)sizeof(KT));
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa, vb, acc[i], 0, 0, 0);
            }
        }
        float* po = a.part_acc + ((int64_t)pair * a.max_splits + split) * 16 * D;
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float* dst = po + (4 * g + r) * D + d0 + 16 * i + h;
                if (COH)
                    st_agent(dst, acc[i][r]);
                else
                    *dst = acc[i][r];
            }
    }
    return true;
}

template <int D, typename KT>
__global__ __launch_bounds__(kThreads, 2) void attend_split_kernel(const AttendArgs a) {
    __shared__ __attribute__((aligned(16))) char tile[tile_bytes<D, KT>()];
    attend_split_body<D, KT>(a, blockIdx.x, blockIdx.y, blockIdx.z, tile);
}

// One workgroup of NT threads per (layer, sequence, NT/256 consecutive
// 32-column slices of D): the splits' maxima and denominators are staged in
// LDS with one parallel load, every thread then merges two outputs over the
// splits in split order.
constexpr int kCombCols = 32;
constexpr int kSpec = 24;   // splits whose outputs are loaded before the row count is known (768 rows)

// The merge weights of every head from the splits' maxima and denominators
// (s_ml, split s at s * 32: 16 maxima, then 16 denominators):
// w[s][h] = exp(m_s - M_h) with M_h = max_s m_s, inv[h] = 1 / sum_s w[s][h] l_s,
// the sum taken in split order.  Every thread of the workgroup (NT) takes part:
// each finds its head's maximum and the weights of a share of the splits, then
// 16 threads add the denominators.  Both merges use it, so they agree bit for
// bit.  Starts and ends with the workgroup in step (s_ml written before).
// (LDS reads go eight at a time, on clamped indices, so their latencies overlap.)
template <int NT>
__device__ __forceinline__ void merge_weights(const float* s_ml, const int ns, float* s_w, float* s_inv) {
    const int tid = threadIdx.x, hh = tid & 15;
    float M = -INFINITY;
    for (int s0 = 0; s0 < ns; s0 += 8) {
        float m[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) m[u] = s_ml[(s0 + u < ns ? s0 + u : ns - 1) * 32 + hh];
#pragma unroll
        for (int u = 0; u < 8; ++u) M = fmaxf(M, m[u]);
    }
    for (int s = tid >> 4; s < ns; s += NT / 16) s_w[s * 16 + hh] = expf(s_ml[s * 32 + hh] - M);
    __syncthreads();
    if (tid < 16) {
        float den = 0.0f;
        for (int s0 = 0; s0 < ns; s0 += 8) {
            float w[8], l[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int sv = s0 + u < ns ? s0 + u : ns - 1;
                w[u] = s_w[sv * 16 + tid];
                l[u] = s_ml[sv * 32 + 16 + tid];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s0 + u < ns) den = __builtin_fmaf(w[u], l[u], den);
        }
        s_inv[tid] = 1.0f / den;
    }
    __syncthreads();
}

template <int D, int NT = 256>
__device__ __forceinline__ void attend_combine_body(const AttendArgs& a, const int bx, const int by, const int bz) {
    static_assert(NT % 256 == 0, "whole slices per workgroup");
    __shared__ float s_ml[kMaxSplits * 32];
    __shared__ float s_w[kMaxSplits][16];   // exp(m_s - M_h)
    __shared__ float s_inv[16];             // 1 / sum_s exp(m_s - M_h) l_s
    const AttendLayer& L = a.L[bz];
    const int b = by;
    const int tid = threadIdx.x;
    const int pair = bz * a.batch + b;
    const int slice = bx * (NT / 256) + (tid >> 8);
    const int d0 = slice * kCombCols;
    // thread -> (head h, columns d0 + c and d0 + c + 16)
    const int h = (tid & 255) >> 4, c = tid & 15;
    const bool mine = h < a.hq && d0 < D;
    // the row count, every split's maxima and denominators, and this thread's
    // outputs of the first kSpec splits are loaded at once (entries past the
    // row count are read but not used), so a list of up to kSpec splits merges
    // in one memory round trip
    // (every load below is unconditional, on a clamped index, and all are issued
    // before the first is used: a load under a branch would make the compiler
    // wait for everything outstanding at the join)
    const float* po = a.part_acc + (int64_t)pair * a.max_splits * 16 * D + (int64_t)(mine ? h : 0) * D + (mine ? d0 : 0);
    float x0[kSpec], x1[kSpec];
#pragma unroll
    for (int j = 0; j < kSpec; ++j) {
        const int jj = j < a.max_splits ? j : a.max_splits - 1;
        x0[j] = po[(int64_t)jj * 16 * D + c];
        x1[j] = po[(int64_t)jj * 16 * D + c + 16];
    }
    const float* ml = a.part_ml + (int64_t)pair * a.max_splits * 32;
    constexpr int kMlPer = (kMaxSplits * 32 + NT - 1) / NT;
    const int n_ml = a.max_splits * 32;
    float mlv[kMlPer];
#pragma unroll
    for (int q = 0; q < kMlPer; ++q) {
        const int i = tid + q * NT;
        mlv[q] = ml[i < n_ml ? i : n_ml - 1];
    }
#pragma unroll
    for (int q = 0; q < kMlPer; ++q)
        if (tid + q * NT < n_ml) s_ml[tid + q * NT] = mlv[q];
#pragma unroll
    for (int j = 0; j < kSpec; ++j) {
        const bool in = mine && j < a.max_splits;
        x0[j] = in ? x0[j] : 0.0f;
        x1[j] = in ? x1[j] : 0.0f;
    }
    int n = L.n_rows[b];
    n = n < 0 ? 0 : (n > L.phys_stride ? L.phys_stride : n);
    const int ns = (n + kR - 1) / kR;
    __syncthreads();
    merge_weights<NT>(s_ml, ns, &s_w[0][0], s_inv);
    if (!mine) return;
    float* out = L.out + ((int64_t)b * a.hq + h) * D + d0;
    if (ns == 0) {
        out[c] = 0.0f;
        out[c + 16] = 0.0f;
        return;
    }
    float n0 = 0.0f, n1 = 0.0f;
#pragma unroll
    for (int j = 0; j < kSpec; ++j) {
        if (j < ns) {
            const float f = s_w[j][h];
            n0 = __builtin_fmaf(f, x0[j], n0);
            n1 = __builtin_fmaf(f, x1[j], n1);
        }
    }
    // longer lists: the remaining splits, eight loads in flight at a time
    for (int s0 = kSpec; s0 < ns; s0 += 8) {
        float y0[8], y1[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool in = s0 + j < ns;
            y0[j] = in ? po[(int64_t)(s0 + j) * 16 * D + c] : 0.0f;
            y1[j] = in ? po[(int64_t)(s0 + j) * 16 * D + c + 16] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (s0 + j < ns) {
                const float f = s_w[s0 + j][h];
                n0 = __builtin_fmaf(f, y0[j], n0);
                n1 = __builtin_fmaf(f, y1[j], n1);
            }
        }
    }
    out[c] = n0 * s_inv[h];
    out[c + 16] = n1 * s_inv[h];
}

template <int D>
__global__ __launch_bounds__(256) void attend_combine_kernel(const AttendArgs a) {
    attend_combine_body<D>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

// ---- one launch: every split merges a share of the columns once all splits
// of its (layer, sequence) have stored their partials.
//
// The splits of one (layer, sequence) count themselves on an arrival counter
// and wait for it to reach the number of live splits; the last to leave resets
// the counters.  Waiting is safe because the host launches this form only when
// every workgroup of the grid can be resident at once (the ones that wait
// never keep a missing one from starting).  The wait is bounded: a workgroup
// that gives up writes NaN to its columns and sets the sticky error word, and
// from then on every launch on these counters writes NaN (a failed wait leaves
// them counted).
constexpr uint32_t kSpinLimit = 1u << 20;

// LDS of the merge (maxima and denominators, weights, inverses), in the tile
// buffer once the split is done with it
constexpr int kMergeLds = kMaxSplits * 32 * 4 + kMaxSplits * 16 * 4 + 16 * 4;

// 16-byte loads of partials another workgroup of the launch stored: buffer
// loads with the device-scope cache policy (SC1), which the XCD's L2 does not
// answer from a line it may hold from before.
constexpr int kCpolDevice = 16;
__device__ __forceinline__ f32x4 ld4_agent(__amdgpu_buffer_rsrc_t r, const uint32_t off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolDevice);
    return f32x4{__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3])};
}

// The merge in the launch.  Column slices of 32 go to the live splits in
// turn: split s merges slices s, s + ns, s + 2 ns, ..., four at a time, one per
// 128-thread quarter, each thread four columns of one head.  Same arithmetic, in
// the same order, as attend_combine_body.  A thread's first kPre splits load
// together with every split's maxima and denominators: one memory round trip
// for lists of up to kPre splits.
template <int D>
__device__ __forceinline__ void attend_merge_share(const AttendArgs& a, const AttendLayer& L, const int b,
                                                   const int pair, const int split, const int ns, const bool ok,
                                                   char* lds) {
    constexpr int NSL = D / kCombCols;
    constexpr int kPre = 20;
    float* s_ml = reinterpret_cast<float*>(lds);   // [ns][32]
    float* s_w = s_ml + kMaxSplits * 32;            // [ns][16]
    float* s_inv = s_w + kMaxSplits * 16;           // [16]
    const int tid = threadIdx.x;
    if (split >= NSL) return;   // uniform: no slice for this split
    const int quarter = tid >> 7, h = (tid & 127) >> 3, c = (tid & 7) * 4;
    int j = split + quarter * ns;
    const bool mine = j < NSL && h < a.hq;
    const int d0 = (j < NSL ? j : split) * kCombCols;   // clamped: every load stays in range
    const int hh = h < a.hq ? h : 0;
    const __amdgpu_buffer_rsrc_t rp =
        make_rsrc(a.part_acc + (int64_t)pair * a.max_splits * 16 * D, (uint32_t)(a.max_splits * 16 * D * 4));
    f32x4 y[kPre];
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
        const int sv = u < ns ? u : ns - 1;
        y[u] = ld4_agent(rp, (uint32_t)(((sv * 16 + hh) * D + d0 + c) * 4));
    }
    const float* ml = a.part_ml + (int64_t)pair * a.max_splits * 32;
    const int n_ml = ns * 32;
    const float m0 = ld_agent(ml + (tid < n_ml ? tid : 0));
    const float m1 = ld_agent(ml + (tid + kThreads < n_ml ? tid + kThreads : 0));
    if (tid < n_ml) s_ml[tid] = m0;
    if (tid + kThreads < n_ml) s_ml[tid + kThreads] = m1;
    for (int i = tid + 2 * kThreads; i < n_ml; i += kThreads) s_ml[i] = ld_agent(ml + i);
    __syncthreads();
    merge_weights<kThreads>(s_ml, ns, s_w, s_inv);
    if (!mine) return;
    const float inv = s_inv[h];
    float* out = L.out + ((int64_t)b * a.hq + h) * D;
    f32x4 n = {0.f, 0.f, 0.f, 0.f};
    float fw[kPre];
#pragma unroll
    for (int u = 0; u < kPre; ++u) fw[u] = s_w[(u < ns ? u : ns - 1) * 16 + h];
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
        if (u < ns) {
#pragma unroll
            for (int e = 0; e < 4; ++e) n[e] = __builtin_fmaf(fw[u], y[u][e], n[e]);
        }
    }
    for (int from = kPre;; from = 0) {
        // the remaining splits of slice j, eight loads in flight
        for (int s0 = from; s0 < ns; s0 += 8) {
            f32x4 z[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int sv = s0 + u < ns ? s0 + u : ns - 1;
                z[u] = ld4_agent(rp, (uint32_t)(((sv * 16 + h) * D + j * kCombCols + c) * 4));
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (s0 + u < ns) {
                    const float f = s_w[(s0 + u) * 16 + h];
#pragma unroll
                    for (int e = 0; e < 4; ++e) n[e] = __builtin_fmaf(f, z[u][e], n[e]);
                }
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) out[j * kCombCols + c + e] = ok ? n[e] * inv : __builtin_nanf("");
        // short lists (fewer than NSL / 4 splits): the quarter's further slices
        j += 4 * ns;
        if (j >= NSL) break;
        n = f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

// sync: [0] sticky error word, then per (layer, sequence) pair p, at word
// kAttendSyncStride * (1 + p): arrivals, departures; all zero between launches.
template <int D, typename KT>
__device__ __forceinline__ void attend_fused_body(const AttendArgs& a, const int bx, const int by, const int bz,
                                                  char* lds) {
    int n = 0;
    if (!attend_split_body<D, KT, true>(a, bx, by, bz, lds, &n)) {
        // an empty list: split 0 writes the zero output
        if (n == 0 && bx == 0) {
            float* out = a.L[bz].out + (int64_t)by * a.hq * D;
            for (int i = threadIdx.x; i < a.hq * D; i += kThreads) out[i] = 0.0f;
        }
        return;
    }
    const int ns = (n + kR - 1) / kR;
    const int pair = bz * a.batch + by;
    uint32_t* err = a.sync;
    uint32_t* arrive = a.sync + kAttendSyncStride * (1 + pair);
    uint32_t* depart = arrive + 1;
    __shared__ int s_ok;
    // every partial store of this workgroup has completed before it counts
    // itself; the count is a release and the wait ends with an acquire, so the
    // partials are ordered before the merge's loads in the memory model too (the
    // SC1 accesses leave no dirty line for the release to write back: measured,
    // the fences cost nothing next to relaxed atomics)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        int ok = __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0;
        if (ok) {
            __hip_atomic_fetch_add(arrive, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            uint32_t spins = 0;
            while (__hip_atomic_load(arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)ns) {
                __builtin_amdgcn_s_sleep(8);
                if (++spins == kSpinLimit) {
                    ok = 0;
                    __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
            if (ok && __hip_atomic_fetch_add(depart, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                          (uint32_t)ns - 1) {
                __hip_atomic_store(arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(depart, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        s_ok = ok;
    }
    __syncthreads();
    attend_merge_share<D>(a, a.L[bz], by, pair, bx, ns, s_ok != 0, lds);
}

template <int D, typename KT>
constexpr int fused_kernel_lds() {
    return tile_bytes<D, KT>() > kMergeLds ? tile_bytes<D, KT>() : kMergeLds;
}

template <int D, typename KT>
__global__ __launch_bounds__(kThreads, 2) void attend_fused_kernel(const AttendArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[fused_kernel_lds<D, KT>()];
    attend_fused_body<D, KT>(a, blockIdx.x, blockIdx.y, blockIdx.z, lds);
}

// Workgroups of attend_fused_kernel<D, KT> one CU holds at once (0: unknown).
template <int D, typename KT>
int fused_per_cu() {
    static int per_cu = -1;
    if (per_cu < 0) {
        int nb = 0;
        per_cu = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, attend_fused_kernel<D, KT>, kThreads, 0) ==
                         hipSuccess
                     ? nb
                     : 0;
    }
    return per_cu;
}

template <int D, typename KT>
hipError_t launch_t(const AttendArgs& a, hipStream_t s, hipEvent_t mid) {
    const int64_t grid = (int64_t)a.max_splits * a.batch * a.n_layers;
    if (a.sync && grid <= (int64_t)a.n_cu * fused_per_cu<D, KT>()) {
        hipLaunchKernelGGL((attend_fused_kernel<D, KT>), dim3(a.max_splits, a.batch, a.n_layers), dim3(kThreads), 0,
                           s, a);
        hipError_t e = hipGetLastError();
        if (e == hipSuccess && mid) e = hipEventRecord(mid, s);
        return e;
    }
    const dim3 g1(a.max_splits, a.batch, a.n_layers);
    hipLaunchKernelGGL((attend_split_kernel<D, KT>), g1, dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (mid) {
        e = hipEventRecord(mid, s);
        if (e != hipSuccess) return e;
    }
    const dim3 g2(D / kCombCols, a.batch, a.n_layers);
    hipLaunchKernelGGL((attend_combine_kernel<D>), g2, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace attend_k
#ifndef LSA_BODIES_ONLY
using namespace attend_k;
#endif
}  // namespace

#ifndef LSA_BODIES_ONLY
size_t attend_workspace_bytes(int n_layers, int batch, int D, int max_rows) {
    const size_t splits = (size_t)((max_rows + kR - 1) / kR);
    return (size_t)n_layers * batch * splits * (16 * (size_t)D + 32) * sizeof(float);
}

template <int D, typename KT>
hipError_t launch_splits_t(const AttendArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((attend_split_kernel<D, KT>), dim3(a.max_splits, a.batch, a.n_layers), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_attend_splits(const AttendArgs& a, hipStream_t s) {
    if (a.max_splits == 0) return hipSuccess;
    if (a.dtype == LSA_F32) {
        if (a.D == 128) return launch_splits_t<128, float>(a, s);
        if (a.D == 256) return launch_splits_t<256, float>(a, s);
        if (a.D == 512) return launch_splits_t<512, float>(a, s);
    } else if (a.dtype == LSA_BF16) {
        if (a.D == 128) return launch_splits_t<128, uint16_t>(a, s);
        if (a.D == 256) return launch_splits_t<256, uint16_t>(a, s);
        if (a.D == 512) return launch_splits_t<512, uint16_t>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_lsa_attend(const AttendArgs& a, hipStream_t s, hipEvent_t mid) {
    if (a.max_splits == 0) return hipSuccess;
    if (a.dtype == LSA_F32) {
        if (a.D == 128) return launch_t<128, float>(a, s, mid);
        if (a.D == 256) return launch_t<256, float>(a, s, mid);
        if (a.D == 512) return launch_t<512, float>(a, s, mid);
    } else if (a.dtype == LSA_BF16) {
        if (a.D == 128) return launch_t<128, uint16_t>(a, s, mid);
        if (a.D == 256) return launch_t<256, uint16_t>(a, s, mid);
        if (a.D == 512) return launch_t<512, uint16_t>(a, s, mid);
    }
    return hipErrorInvalidValue;
}

#endif  // LSA_BODIES_ONLY

}  // namespace lsa
