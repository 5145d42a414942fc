// lsa_project: the memory indexers' query heads and head weights, projected
// from the decode token's hidden state.
//
// [P1] architecture overview: the token's hidden state (hidden[4096]) feeds
// the three scorers.  Each indexer i maps it linearly to its H query heads of
// dk values and its H head weights:
//   q[b,i,h,:] = Wq[i,h] . hidden[b]        (Wq[i,h] is dk x d_model)
//   w[b,i,h]   = Ww[i,h,:] . hidden[b]
// so that lsa_score can take (q, w) of the same step.
//
// Design (gfx950): a batched GEMV -- up to four hidden vectors against
// n_idx*H*(dk+1) weight rows -- bound by reading the weights from HBM once,
// so it stays off the matrix cores.  Each wave owns one weight row.  Lane l
// reads the row's 16-byte chunks l, l+64, l+128, ... through a buffer
// resource clamped to the row (so a ragged row end reads zeros) together with
// the hidden elements those chunks multiply (from L1/L2: every wave of the
// launch reads the same few KB), all loads of a 4096-wide row issued before
// the first use, so a row costs one memory latency; there is no LDS stage and
// no barrier.  The wave sums its lanes with a butterfly of cross-lane adds.
// More than four vectors run as several launches, each reading the weights
// again.
#include "lsa_internal.hpp"

namespace lsa {

namespace {
namespace project_k {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
// 16-byte weight chunks per lane in flight: a whole 4096-wide row for one or
// two vectors, half of it for three or four (the matching hidden elements sit
// in registers beside them)
template <typename WT, int NB>
constexpr int kInFlight = (sizeof(WT) == 4 ? 16 : 8) / (NB > 2 ? 2 : 1);

// 16 bytes of weights times the matching hidden elements
template <typename WT>
struct Chunk;
template <>
struct Chunk<float> {
    static constexpr int kElems = 4;
    static constexpr int kHid = 1;   // 16-byte hidden loads per chunk
    __device__ static inline float dot(const uint4& u, const uint4* h) {
        float s = __uint_as_float(u.x) * __uint_as_float(h[0].x);
        s += __uint_as_float(u.y) * __uint_as_float(h[0].y);
        s += __uint_as_float(u.z) * __uint_as_float(h[0].z);
        s += __uint_as_float(u.w) * __uint_as_float(h[0].w);
        return s;
    }
};
template <>
struct Chunk<uint16_t> {
    static constexpr int kElems = 8;
    static constexpr int kHid = 2;
    __device__ static inline float dot(const uint4& u, const uint4* h) {
        float s = bf16_lo(u.x) * __uint_as_float(h[0].x);
        s += bf16_hi(u.x) * __uint_as_float(h[0].y);
        s += bf16_lo(u.y) * __uint_as_float(h[0].z);
        s += bf16_hi(u.y) * __uint_as_float(h[0].w);
        s += bf16_lo(u.z) * __uint_as_float(h[1].x);
        s += bf16_hi(u.z) * __uint_as_float(h[1].y);
        s += bf16_lo(u.w) * __uint_as_float(h[1].z);
        s += bf16_hi(u.w) * __uint_as_float(h[1].w);
        return s;
    }
};

template <typename WT, int NB>
__global__ __launch_bounds__(kThreads) void project_kernel(const ProjectArgs a) {
    constexpr int kF = kInFlight<WT, NB>;
    constexpr int kH = Chunk<WT>::kHid;
    const int lane = threadIdx.x & 63;
    const int row_bytes = a.d_model * (int)sizeof(WT);
    __amdgpu_buffer_rsrc_t rh[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) rh[b] = make_rsrc(a.hidden + (int64_t)b * a.d_model, (uint32_t)a.d_model * 4u);
    const int n_chunks = row_bytes / 16;
    // rows wave, wave + all waves, ...; uniform per wave, so a row's buffer
    // resource stays in scalar registers
    const int n_waves = gridDim.x * kWaves;
    for (int row = __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + (threadIdx.x >> 6));
         row < a.q_rows + a.w_rows; row += n_waves) {
    const char* wrow = row < a.q_rows
        ? static_cast<const char*>(a.wq) + (int64_t)row * row_bytes
        : static_cast<const char*>(a.ww) + (int64_t)(row - a.q_rows) * row_bytes;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(wrow, (uint32_t)row_bytes);

    float acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = 0.0f;
    for (int c0 = 0; c0 < n_chunks; c0 += 64 * kF) {
        // a round's weight chunks and their hidden elements, all loaded before use
        // (past the row end both read as zero)
        uint4 u[kF], h[kF][NB][kH];
#pragma unroll
        for (int k = 0; k < kF; ++k) u[k] = buffer_load16(r, (uint32_t)(c0 + lane + 64 * k) * 16u);
#pragma unroll
        for (int k = 0; k < kF; ++k) {
            const uint32_t e0 = (uint32_t)(c0 + lane + 64 * k) * Chunk<WT>::kElems * 4u;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int x = 0; x < kH; ++x) h[k][b][x] = buffer_load16(rh[b], e0 + 16u * x);
        }
#pragma unroll
        for (int k = 0; k < kF; ++k)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[b] += Chunk<WT>::dot(u[k], h[k][b]);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) acc[b] += __shfl_xor(acc[b], d, 64);
    }
    if (lane == 0) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (row < a.q_rows) a.q[(int64_t)b * a.q_rows + row] = acc[b];
            else a.w[(int64_t)b * a.w_rows + (row - a.q_rows)] = acc[b];
        }
    }
    }
}

constexpr int kGridPerCu = 2;   // workgroups per CU (1, 2, 4 and 8 time within 0.5 us)

template <typename WT>
hipError_t launch_t(const ProjectArgs& a0, int batch, int n_cu, hipStream_t s) {
    const int rows = a0.q_rows + a0.w_rows;
    int g = (rows + kWaves - 1) / kWaves;
    if (g > n_cu * kGridPerCu) g = n_cu * kGridPerCu;
    const dim3 grid((unsigned)g), block(kThreads);
    for (int b0 = 0; b0 < batch;) {
        const int nb = batch - b0 < 4 ? batch - b0 : 4;   // vectors per launch
        ProjectArgs a = a0;
        a.hidden = a0.hidden + (int64_t)b0 * a0.d_model;
        a.q = a0.q + (int64_t)b0 * a0.q_rows;
        a.w = a0.w + (int64_t)b0 * a0.w_rows;
        switch (nb) {
            case 1: hipLaunchKernelGGL((project_kernel<WT, 1>), grid, block, 0, s, a); break;
            case 2: hipLaunchKernelGGL((project_kernel<WT, 2>), grid, block, 0, s, a); break;
            case 3: hipLaunchKernelGGL((project_kernel<WT, 3>), grid, block, 0, s, a); break;
            default: hipLaunchKernelGGL((project_kernel<WT, 4>), grid, block, 0, s, a); break;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        b0 += nb;
    }
    return hipSuccess;
}

}  // namespace project_k
}  // namespace

hipError_t launch_project(const ProjectArgs& a, int w_dtype, int batch, int n_cu, hipStream_t s) {
    if (w_dtype == LSA_F32) return project_k::launch_t<float>(a, batch, n_cu, s);
    if (w_dtype == LSA_BF16) return project_k::launch_t<uint16_t>(a, batch, n_cu, s);
    return hipErrorInvalidValue;
}

}  // namespace lsa
