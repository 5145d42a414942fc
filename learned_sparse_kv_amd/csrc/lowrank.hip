// KVSwap grouped low-rank key prediction.
//
// KVSwap article, section 2.3 (low-rank K and its reconstruction): a head
// group's keys over all positions are kept as factors K ~ U diag(S) V^T, with
// U [T][rank] per position; section 2.2 (grouped prediction): the group's
// query is scored against every position and the top entries are loaded.
// The score of position t is q . K[t,:] = U[t,:] . p with p = diag(S) V^T q,
// so the reconstruction is never formed: one small projection per group
// (rank x C) and then a scan over U at 2 * rank bytes per position.
//
// Design (gfx950): the scan is a plain HBM stream (64 bytes per position at
// rank 32, four flops per byte), so it runs on VALU with coalesced 16-byte
// buffer loads: rank/8 lanes cover one row, a wave covers 64*8/rank rows per
// load, and the partial dots are combined across those lanes.  The projection
// p is computed once per group by a separate small launch rather than being
// repeated by every block of the scan.
#include "lsa_internal.hpp"
#define LSA_BODIES_ONLY
#include "fm_select.hip"
#undef LSA_BODIES_ONLY

namespace lsa {

namespace {

constexpr int kThreads = 256;

// p = diag(S) V^T q of one segment (V [C][R] f16, q [C], S [R], in global
// memory or LDS): threads t < 256 (every thread of the workgroup calls this)
// sum rank index t % R over the columns c = t / R + 256/R * i, then the first R
// threads add the 256/R partial sums in order and write p_out[x].  red: 256
// floats of LDS.
template <int R>
__device__ __forceinline__ void lowrank_p_from(const uint16_t* V, const float* q, const int C, const float* S,
                                               float* red, float* p_out) {
    constexpr int kParts = 256 / R;
    const int tid = threadIdx.x;
    const int x = tid % R, part = tid / R;
    if (tid < 256) {
        float acc = 0.0f;
        for (int c = part; c < C; c += kParts) acc += f16_to_f32(V[c * R + x]) * q[c];
        red[tid] = acc;
    }
    __syncthreads();
    if (tid < R) {
        float t = 0.0f;
#pragma unroll
        for (int i = 0; i < kParts; ++i) t += red[i * R + x];
        p_out[x] = S[x] * t;
    }
}

template <int R>
__device__ __forceinline__ void lowrank_p_body(const LowrankArgs& a, const int s, float* red, float* p_out) {
    lowrank_p_from<R>(a.V + (int64_t)s * a.C * R, a.q + (int64_t)s * a.C, a.C, a.S + (int64_t)s * R, red, p_out);
}

// One lane's part of a row's score (eight f16 of U against its eight values
// of p), summed over the row's R/8 lanes: DPP quad permutes for lane
// distances 1 and 2 (no LDS permute), a shuffle for 4.
template <int R>
__device__ __forceinline__ float row_score(const uint4& v, const float (&p)[8]) {
    constexpr int kLpr = R / 8;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float d = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        d += p[2 * e] * f16_to_f32((uint16_t)(w[e] & 0xFFFF));
        d += p[2 * e + 1] * f16_to_f32((uint16_t)(w[e] >> 16));
    }
    if constexpr (kLpr >= 2)
        d += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(d), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    if constexpr (kLpr >= 4)
        d += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(d), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    if constexpr (kLpr >= 8) d += __shfl_xor(d, 4, 64);
    return d;
}

// LDS_VQ: V and q of segment blockIdx.x first go into LDS (16-byte buffer loads
// straight to LDS, one round trip; dynamic LDS of vq_bytes(C)), and p is then
// summed from there in the same order, instead of from 64 rounds of 2- and
// 4-byte loads per thread that each wait a full memory latency.
__host__ __device__ inline int vq_v_bytes(int C, int R) { return (C * R * 2 + 1023) / 1024 * 1024; }
__host__ __device__ inline int vq_bytes(int C, int R) { return vq_v_bytes(C, R) + (C * 4 + 1023) / 1024 * 1024; }

template <int R, bool LDS_VQ>
__global__ __launch_bounds__(kThreads) void lowrank_p_kernel(const LowrankArgs a) {
    __shared__ float red[kThreads];
    const int s = blockIdx.x;
    float* p_out = a.p + (int64_t)s * R;
    if constexpr (LDS_VQ) {
        extern __shared__ __attribute__((aligned(1024))) char vq[];
        const int C = a.C, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int v_bytes = vq_v_bytes(C, R), all = vq_bytes(C, R);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.V + (int64_t)s * C * R, (uint32_t)(C * R * 2));
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + (int64_t)s * C, (uint32_t)(C * 4));
        for (int c = wave; c < all / 1024; c += kThreads / 64) {
            const bool in_v = c * 1024 < v_bytes;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(in_v ? rv : rq, (__attribute__((address_space(3))) void*)(vq + c * 1024),
                                                     16, (in_v ? c * 1024 : c * 1024 - v_bytes) + lane * 16, 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        lowrank_p_from<R>(reinterpret_cast<const uint16_t*>(vq), reinterpret_cast<const float*>(vq + v_bytes), C,
                          a.S + (int64_t)s * R, red, p_out);
    } else {
        lowrank_p_body<R>(a, s, red, p_out);
    }
}

template <int R>
__global__ __launch_bounds__(kThreads) void lowrank_scan_kernel(const LowrankArgs a) {
    constexpr int kLpr = R / 8;             // lanes per row, 8 halves (16 bytes) each
    constexpr int kRpw = 64 / kLpr;         // rows per wave load
    constexpr int kRpb = 4 * kRpw;          // rows per block load
    constexpr int kUnroll = 8;
    const int s = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % kLpr;
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = a.p[(int64_t)s * R + sub * 8 + e];
    const uint32_t row_bytes = R * 2;
    const __amdgpu_buffer_rsrc_t ru = make_rsrc(a.U + (int64_t)s * a.T * R, (uint32_t)(a.T * row_bytes));
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scores + (int64_t)s * a.T, (uint32_t)(a.T * 4));
    const int64_t first = (int64_t)blockIdx.x * a.rows_per_block;
    const int64_t last = first + a.rows_per_block < a.T ? first + a.rows_per_block : a.T;
    for (int64_t base = first; base < last; base += kRpb * kUnroll) {
        uint4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t row = base + u * kRpb + wave * kRpw + lane / kLpr;
            // rows past the end read as zero (offsets stay below 2^32: T * row_bytes < 4 GiB);
            // U is read once per step, so its lines are not kept
            v[u] = buffer_load16_nt(ru, (uint32_t)(row < a.T ? row : a.T) * row_bytes + sub * 16);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const float d = row_score<R>(v[u], p);
            const int64_t row = base + u * kRpb + wave * kRpw + lane / kLpr;
            // one lane per row stores; rows past the end and the other lanes are dropped
            const uint32_t off = (sub == 0 && row < last) ? (uint32_t)row * 4u : 0xFFFFFFF0u;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(d + 0.0f), rs, off, 0, 0);
        }
    }
}

// Score and top-k of a segment in one workgroup, the scores never leaving
// the CU: p as lowrank_p_kernel, the scan as lowrank_scan_kernel (the same
// arithmetic, so the same bits), each row's score into LDS (one padding word
// per 32, so that a thread's E consecutive entries sit in distinct banks), then
// the top-k of the one-workgroup select (fm_select, select_single) over the
// E entries each thread takes from LDS: the same choice, ties to the lowest
// position, output ascending.  T <= kFuseMaxT; the LDS of the scores is
// reused by the select once they are in registers.
//
// One workgroup per CU, each taking segments blockIdx.x, blockIdx.x + grid, ...
// The select reads and writes only the first 33 KB of the LDS, so before it
// starts, the workgroup has the first batch of its next segment's U rows (64
// KB) copied from HBM into the LDS above that (buffer loads straight to LDS);
// the CU's memory traffic then goes on while it selects, and the next scan
// takes its first batch from the LDS.
constexpr int kFuseMaxT = 32768;

template <int R, int E>
__global__ __launch_bounds__(select_k::kNT) void lowrank_select_kernel(const LowrankArgs a, const int k,
                                                                       int32_t* sel, int32_t* count) {
    constexpr int NT = select_k::kNT;
    // four 16-byte loads in flight per lane (16 waves): 2.67 ms per 32K step, against 2.80 / 2.70 /
    // 2.72 / 2.72 with 2 / 3 / 6 / 8
    constexpr int kLpr = R / 8, kRpw = 64 / kLpr, kRpb = (NT / 64) * kRpw, kUnroll = 4;
    constexpr int kBatch = kRpb * kUnroll;          // rows per batch: NT * kUnroll 16-byte pieces
    constexpr int kPreBytes = NT * kUnroll * 16;    // 64 KB
    constexpr int kPreOff = (int)((sizeof(select_k::KthWide) + 1023) / 1024 * 1024);
    __shared__ union FuseLds {
        float sc[kFuseMaxT + kFuseMaxT / 32];
        select_k::KthWide sh;
        float red[256];
    } u;
    static_assert(kPreOff + kPreBytes <= (int)sizeof(FuseLds), "prefetch region inside the score LDS");
    __shared__ float s_p[R];
    // the select's first histogram (key bits 31..20), counted as the scores are made
    __shared__ uint32_t s_hist[select_k::kWideBins];
    char* const pre = reinterpret_cast<char*>(&u) + kPreOff;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, sub = lane % kLpr;
    const int T = (int)a.T, C = a.C;
    const uint32_t row_bytes = R * 2;
    // V and q of a segment are copied into the LDS above the U copy when they fit
    // (C <= 525 at rank 32), so p is summed from LDS rather than from 64 rounds
    // of small loads, each waiting behind the other CUs' U streams
    constexpr int kVqOff = kPreOff + kPreBytes;
    const int v_bytes = (C * R * 2 + 1023) / 1024 * 1024, q_bytes = (C * 4 + 1023) / 1024 * 1024;
    const bool vq_lds = kVqOff + v_bytes + q_bytes <= (int)sizeof(FuseLds);
    uint16_t* const Vl = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(&u) + kVqOff);
    float* const ql = reinterpret_cast<float*>(reinterpret_cast<char*>(&u) + kVqOff + v_bytes);
    auto copy_vq = [&](int seg) {
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.V + (int64_t)seg * C * R, (uint32_t)(C * R * 2));
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + (int64_t)seg * C, (uint32_t)(C * 4));
        for (int c = wave; c < v_bytes / 1024; c += NT / 64)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(
                reinterpret_cast<char*>(Vl) + c * 1024), 16, c * 1024 + lane * 16, 0, 0, 0);
        for (int c = wave; c < q_bytes / 1024; c += NT / 64)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (__attribute__((address_space(3))) void*)(
                reinterpret_cast<char*>(ql) + c * 1024), 16, c * 1024 + lane * 16, 0, 0, 0);
    };
    bool have_pre = false;
    for (int s = blockIdx.x; s < a.n_seg; s += gridDim.x) {
        if (vq_lds && !have_pre) copy_vq(s);   // later segments' were copied during the previous select
        for (int i = tid; i < select_k::kWideBins; i += NT) s_hist[i] = 0u;
        __builtin_amdgcn_s_waitcnt(0);   // this wave's copies have landed
        __syncthreads();   // every wave's copies are in LDS
        if (vq_lds)
            lowrank_p_from<R>(Vl, ql, C, a.S + (int64_t)s * R, u.red, s_p);
        else
            lowrank_p_body<R>(a, s, u.red, s_p);
        __syncthreads();   // p is in LDS (red read)
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = s_p[sub * 8 + e];
        auto take = [&](const uint4 (&v)[kUnroll], int base) {
#pragma unroll
            for (int uu = 0; uu < kUnroll; ++uu) {
                const float d = row_score<R>(v[uu], p);
                const int row = base + uu * kRpb + wave * kRpw + lane / kLpr;
                if (sub == 0 && row < T) {
                    u.sc[row + (row >> 5)] = d + 0.0f;
                    atomicAdd(&s_hist[order_key(d + 0.0f) >> 20], 1u);
                }
            }
        };
        int base0 = 0;
        if (have_pre) {
            // the first batch from the LDS (rows past T read as zero there and are dropped)
            uint4 v[kUnroll];
#pragma unroll
            for (int uu = 0; uu < kUnroll; ++uu) {
                const int row = uu * kRpb + wave * kRpw + lane / kLpr;
                v[uu] = *reinterpret_cast<const uint4*>(pre + row * row_bytes + sub * 16);
            }
            __syncthreads();   // red is read (p) and the prefetched rows are in registers
            take(v, 0);
            base0 = kBatch;
        } else {
            __syncthreads();   // red is read before the scores overwrite it
        }
        const __amdgpu_buffer_rsrc_t ru = make_rsrc(a.U + (int64_t)s * a.T * R, (uint32_t)(a.T * row_bytes));
        for (int base = base0; base < T; base += kBatch) {
            uint4 v[kUnroll];
#pragma unroll
            for (int uu = 0; uu < kUnroll; ++uu) {
                const int row = base + uu * kRpb + wave * kRpw + lane / kLpr;
                // rows past the end read as zero; U is read once per step, so its lines are not kept
                v[uu] = buffer_load16_nt(ru, (uint32_t)(row < T ? row : T) * row_bytes + sub * 16);
            }
            take(v, base);
        }
        __syncthreads();
        // thread t takes entries t*E .. t*E + E - 1 (order key 0: past the segment)
        uint32_t key[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int j = tid * E + e;
            key[e] = j < T ? order_key(u.sc[j + (j >> 5)]) : 0u;
        }
        __syncthreads();   // the scores are in registers: the LDS is the select's and the prefetch's from here
        const int s_next = s + (int)gridDim.x;
        have_pre = s_next < a.n_seg;
        if (have_pre) {
            const __amdgpu_buffer_rsrc_t rn =
                make_rsrc(a.U + (int64_t)s_next * a.T * R, (uint32_t)(a.T * row_bytes));
            // wave w copies the 1 KB pieces w, w + 16, ... of the batch, lane l the 16 bytes at 16 l
            for (int c = wave; c < kPreBytes / 1024; c += NT / 64)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rn, (__attribute__((address_space(3))) void*)(pre + c * 1024), 16, c * 1024 + lane * 16, 0, 0, 2);
            if (vq_lds) copy_vq(s_next);
        }
        // every position of the segment is an entry (T >= 1), so K = min(k, T) >= 1
        const int K = T < k ? T : k;
        int32_t* out_sel = sel + (int64_t)s * k;
        uint32_t Tk;
        int need_eq;
        select_k::block_kth<E>(key, K, u.sh, &Tk, &need_eq, s_hist);
        select_k::block_choose<E>(key, Tk, need_eq, u.sh.scan, (int64_t)tid * E, out_sel, k);
        for (int i = K + tid; i < k; i += NT) out_sel[i] = -1;
        if (tid == 0) count[s] = K;
        __syncthreads();   // the select's LDS is free before the next segment's p
    }
}

template <int R>
hipError_t launch_r(const LowrankArgs& a, hipStream_t s, hipEvent_t mid) {
    const int vq = vq_bytes(a.C, R);
    if (vq <= 64 * 1024)
        hipLaunchKernelGGL((lowrank_p_kernel<R, true>), dim3(a.n_seg), dim3(kThreads), (size_t)vq, s, a);
    else
        hipLaunchKernelGGL((lowrank_p_kernel<R, false>), dim3(a.n_seg), dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (mid) (void)hipEventRecord(mid, s);
    const int64_t blocks = (a.T + a.rows_per_block - 1) / a.rows_per_block;
    hipLaunchKernelGGL((lowrank_scan_kernel<R>), dim3((unsigned)blocks, a.n_seg), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int R>
hipError_t launch_rs(const LowrankArgs& a, int E, int k, int32_t* sel, int32_t* count, int n_cu, hipStream_t s) {
    const dim3 grid(a.n_seg < n_cu ? a.n_seg : n_cu), block(select_k::kNT);
    switch (E) {
        case 1: hipLaunchKernelGGL((lowrank_select_kernel<R, 1>), grid, block, 0, s, a, k, sel, count); break;
        case 2: hipLaunchKernelGGL((lowrank_select_kernel<R, 2>), grid, block, 0, s, a, k, sel, count); break;
        case 4: hipLaunchKernelGGL((lowrank_select_kernel<R, 4>), grid, block, 0, s, a, k, sel, count); break;
        case 8: hipLaunchKernelGGL((lowrank_select_kernel<R, 8>), grid, block, 0, s, a, k, sel, count); break;
        case 16: hipLaunchKernelGGL((lowrank_select_kernel<R, 16>), grid, block, 0, s, a, k, sel, count); break;
        case 32: hipLaunchKernelGGL((lowrank_select_kernel<R, 32>), grid, block, 0, s, a, k, sel, count); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool lowrank_select_fits(int64_t T, int rank, int k) {
    return T >= 1 && T <= kFuseMaxT && k >= 1 && k <= select_k::kNT && (rank == 16 || rank == 32 || rank == 64);
}

hipError_t launch_lowrank_select(const LowrankArgs& a, int k, int32_t* sel, int32_t* count, int n_cu,
                                 hipStream_t s) {
    if (a.n_seg == 0) return hipSuccess;
    if (!lowrank_select_fits(a.T, a.rank, k) || n_cu < 1) return hipErrorInvalidValue;
    int E = 1;
    while ((int64_t)E * select_k::kNT < a.T) E *= 2;
    if (a.rank == 16) return launch_rs<16>(a, E, k, sel, count, n_cu, s);
    if (a.rank == 32) return launch_rs<32>(a, E, k, sel, count, n_cu, s);
    return launch_rs<64>(a, E, k, sel, count, n_cu, s);
}

hipError_t launch_lowrank_score(const LowrankArgs& a, hipStream_t s, hipEvent_t mid) {
    if (a.T == 0 || a.n_seg == 0) return hipSuccess;
    if (a.rank == 16) return launch_r<16>(a, s, mid);
    if (a.rank == 32) return launch_r<32>(a, s, mid);
    if (a.rank == 64) return launch_r<64>(a, s, mid);
    return hipErrorInvalidValue;
}

}  // namespace lsa
