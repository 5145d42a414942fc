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

namespace lsa {

namespace {

constexpr int kThreads = 256;

template <int R>
__global__ __launch_bounds__(kThreads) void lowrank_p_kernel(const LowrankArgs a) {
    constexpr int kParts = kThreads / R;
    __shared__ float red[kThreads];
    const int s = blockIdx.x;
    const int x = threadIdx.x % R, part = threadIdx.x / R;
    const uint16_t* V = a.V + (int64_t)s * a.C * R;
    const float* q = a.q + (int64_t)s * a.C;
    float acc = 0.0f;
    for (int c = part; c < a.C; c += kParts) acc += f16_to_f32(V[(int64_t)c * R + x]) * q[c];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (part == 0) {
        float t = 0.0f;
#pragma unroll
        for (int i = 0; i < kParts; ++i) t += red[i * R + x];
        a.p[(int64_t)s * R + x] = a.S[(int64_t)s * R + x] * t;
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
            const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
            float d = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                d += p[2 * e] * f16_to_f32((uint16_t)(w[e] & 0xFFFF));
                d += p[2 * e + 1] * f16_to_f32((uint16_t)(w[e] >> 16));
            }
            // sum over the row's kLpr lanes: DPP quad permutes for lane distances 1
            // and 2 (no LDS permute), a shuffle for 4
            if constexpr (kLpr >= 2)
                d += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(d), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
            if constexpr (kLpr >= 4)
                d += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(d), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
            if constexpr (kLpr >= 8) d += __shfl_xor(d, 4, 64);
            const int64_t row = base + u * kRpb + wave * kRpw + lane / kLpr;
            // one lane per row stores; rows past the end and the other lanes are dropped
            const uint32_t off = (sub == 0 && row < last) ? (uint32_t)row * 4u : 0xFFFFFFF0u;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(d + 0.0f), rs, off, 0, 0);
        }
    }
}

template <int R>
hipError_t launch_r(const LowrankArgs& a, hipStream_t s, hipEvent_t mid) {
    hipLaunchKernelGGL((lowrank_p_kernel<R>), dim3(a.n_seg), dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (mid) (void)hipEventRecord(mid, s);
    const int64_t blocks = (a.T + a.rows_per_block - 1) / a.rows_per_block;
    hipLaunchKernelGGL((lowrank_scan_kernel<R>), dim3((unsigned)blocks, a.n_seg), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lowrank_score(const LowrankArgs& a, hipStream_t s, hipEvent_t mid) {
    if (a.T == 0 || a.n_seg == 0) return hipSuccess;
    if (a.rank == 16) return launch_r<16>(a, s, mid);
    if (a.rank == 32) return launch_r<32>(a, s, mid);
    if (a.rank == 64) return launch_r<64>(a, s, mid);
    return hipErrorInvalidValue;
}

}  // namespace lsa
