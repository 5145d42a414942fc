// fm_score: every memory-indexer query against every compressed indexer key,
// fused with the per-head ReLU, head weights and the max/mean ensemble.
//
// [P1] architecture: three scorers read the one shared indexer key cache and
// are combined by max or mean; [P2] LSA section: indexer queries are matched
// against compressed indexer keys by dot product.  Score of entry j:
//   s_i[j] = sum_h w[i,h] * ReLU(q[i,h,:] . key[j,:]),  e[j] = max_i / mean_i s_i[j].
//
// Design (gfx950): the key scan is the only O(context) traffic of a decode
// step, so keys are read from HBM exactly once, in coalesced 16-byte buffer
// loads (out-of-range tails read as zero), and every query is applied to a
// key while it sits in LDS.  The (n_idx*H <= 32) x dk query block stays in
// registers as the A operand of v_mfma_f32_32x32x2f32; a wave multiplies it by
// 32 keys at a time (B operand), so one MFMA chain yields all 32x32 dot
// products of its tile.  Query row i of the MFMA is indexer i/8, head i%8;
// with that layout each lane's 16 accumulators hold 4 heads of each of 4
// indexers for one key, so the ReLU/weight/head-sum/ensemble epilogue is
// in-lane plus one cross-half exchange.  The k dimension is permuted so that a
// lane reads one contiguous half-row from LDS (lane half 0 takes elements
// 0..dk/2-1, half 1 the rest); A uses the same permutation, so the products
// are unchanged.  LDS rows are padded by 16 bytes so that 8 consecutive rows
// start in different bank groups.
// Every wave works on its own 32-key tiles and LDS region with wave-scope
// fences only -- no workgroup barriers -- and issues the next tile's loads
// before the MFMAs of the current one, so one wave's memory phase overlaps
// another's MFMAs.  The grid is one 4-wave workgroup per CU (fewer when the
// scan is short), which keeps every wave's share of tiles equal.
#include "lsa_internal.hpp"

namespace lsa {

namespace {
namespace score_k {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTile = 32;          // keys per wave tile

template <int DK, typename KT>
struct Cfg {
    static constexpr int kRowBytes = DK * (int)sizeof(KT);
    static constexpr int kLdsStride = kRowBytes + 16;
    static constexpr int kTileBytes = kTile * kRowBytes;
    static constexpr int kLoads = kTileBytes / (64 * 16);      // 16-byte loads per lane
    static constexpr int kHalf = DK / 2;                     // MFMA k-steps
    static constexpr int kHalfBytes = kHalf * (int)sizeof(KT);
    static constexpr int kReads = kHalfBytes / 16;           // ds_read_b128 per lane
    static_assert(kTileBytes % (64 * 16) == 0, "tile must split into 16-byte loads");
    static_assert(kHalfBytes % 16 == 0, "half row must be 16-byte aligned");
};

template <typename KT>
__device__ inline void unpack16(const uint4& u, float* out);

template <>
__device__ inline void unpack16<float>(const uint4& u, float* out) {
    out[0] = __uint_as_float(u.x);
    out[1] = __uint_as_float(u.y);
    out[2] = __uint_as_float(u.z);
    out[3] = __uint_as_float(u.w);
}

template <>
__device__ inline void unpack16<uint16_t>(const uint4& u, float* out) {
    out[0] = bf16_lo(u.x);
    out[1] = bf16_hi(u.x);
    out[2] = bf16_lo(u.y);
    out[3] = bf16_hi(u.y);
    out[4] = bf16_lo(u.z);
    out[5] = bf16_hi(u.z);
    out[6] = bf16_lo(u.w);
    out[7] = bf16_hi(u.w);
}

template <int DK, typename KT>
__device__ __forceinline__ void fm_score_body(const ScoreArgs& a, const int bx, const int gx) {
    using C = Cfg<DK, KT>;
    constexpr int kPerRead = 16 / (int)sizeof(KT);
    __shared__ __attribute__((aligned(16))) char lds[kWaves][kTile * C::kLdsStride];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keeps tile state in SGPRs
    const int col = lane & 31;      // key within the tile (B/D column); query row for A
    const int half = lane >> 5;     // which half of dk this lane feeds

    const int total = a.tile_start[a.batch];
    const int stride = gx * kWaves;
    int t = bx * kWaves + wave;
    if (t >= total) return;

    auto seq_of = [&](int tile) {
        int b = 0;
        while (tile >= a.tile_start[b + 1]) ++b;
        return b;
    };
    const char* kbase = static_cast<const char*>(a.keys);
    auto load_tile = [&](int tile, uint4 (&dst)[C::kLoads]) {
        const int b = seq_of(tile);
        const __amdgpu_buffer_rsrc_t r = make_rsrc(kbase + (int64_t)b * a.n_keys * C::kRowBytes,
                                                   (uint32_t)a.n_valid[b] * (uint32_t)C::kRowBytes);
        const uint32_t base = (uint32_t)(tile - a.tile_start[b]) * (uint32_t)C::kTileBytes;
#pragma unroll
        for (int i = 0; i < C::kLoads; ++i) dst[i] = buffer_load16(r, base + (uint32_t)(i * 64 + lane) * 16u);
    };

    int cur_b = -1;
    float qa[C::kHalf];
    float wr[16];
    char* my = lds[wave];
    uint4 pre[C::kLoads];
    load_tile(t, pre);

    while (t < total) {
        const int b = seq_of(t);
        if (b != cur_b) {
            cur_b = b;
            // A operand: query row `col` (indexer col/8, head col%8), elements half*DK/2 + s
            const int g = col >> 3, hd = col & 7;
            const bool qv = g < a.n_idx && hd < a.heads;
            const float* qrow = a.q + (((int64_t)b * a.n_idx + (qv ? g : 0)) * a.heads + (qv ? hd : 0)) * DK + half * C::kHalf;
#pragma unroll
            for (int s = 0; s < C::kHalf; s += 4) {
                f32x4 v = qv ? *reinterpret_cast<const f32x4*>(qrow + s) : f32x4{0.f, 0.f, 0.f, 0.f};
                qa[s] = v[0];
                qa[s + 1] = v[1];
                qa[s + 2] = v[2];
                qa[s + 3] = v[3];
            }
            // epilogue weights: accumulator r is query row 8*(r/4) + 4*half + r%4
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gi = r >> 2, hi = 4 * half + (r & 3);
                wr[r] = (gi < a.n_idx && hi < a.heads) ? a.w[((int64_t)b * a.n_idx + gi) * a.heads + hi] : 0.0f;
            }
        }
        const int tile_in_seq = t - a.tile_start[b];

#pragma unroll
        for (int i = 0; i < C::kLoads; ++i) {
            const int off = (i * 64 + lane) * 16;
            *reinterpret_cast<uint4*>(my + (off / C::kRowBytes) * C::kLdsStride + off % C::kRowBytes) = pre[i];
        }
        // the wave's LDS writes are visible to all its lanes past this point
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        const int t_next = t + stride;
        if (t_next < total) load_tile(t_next, pre);

        // 32 keys x 32 query rows, k = DK
        f32x16 acc = {};
        const char* myrow = my + col * C::kLdsStride + half * C::kHalfBytes;
#pragma unroll
        for (int rd = 0; rd < C::kReads; ++rd) {
            const uint4 u = *reinterpret_cast<const uint4*>(myrow + rd * 16);
            float kb[kPerRead];
            unpack16<KT>(u, kb);
#pragma unroll
            for (int e = 0; e < kPerRead; ++e)
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[rd * kPerRead + e], kb[e], acc, 0, 0, 0);
        }
        // all lanes' LDS reads of this tile are done before the next tile is written
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // epilogue: per indexer, this lane's 4 heads; then the other half's 4 heads
        float s[4];
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
            float v = 0.0f;
#pragma unroll
            for (int c = 0; c < 4; ++c) v += wr[4 * gi + c] * fmaxf(acc[4 * gi + c], 0.0f);
            s[gi] = v;
        }
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) s[gi] = (s[gi] + __shfl_xor(s[gi], 32, 64)) + 0.0f;
        float e;
        if (a.ensemble == LSA_ENSEMBLE_MAX) {
            e = s[0];
            for (int gi = 1; gi < a.n_idx; ++gi) e = fmaxf(e, s[gi]);
        } else {
            float sum = s[0];
            for (int gi = 1; gi < a.n_idx; ++gi) sum += s[gi];
            e = sum / (float)a.n_idx;
        }
        const int key = tile_in_seq * kTile + col;
        if (half == 0 && key < a.n_valid[b]) a.scores[(int64_t)b * a.n_keys + key] = e + 0.0f;

        t = t_next;
    }
}

template <int DK, typename KT>
__global__ __launch_bounds__(kThreads, 2) void fm_score_kernel(const ScoreArgs a) {
    fm_score_body<DK, KT>(a, blockIdx.x, gridDim.x);
}

template <int DK, typename KT>
hipError_t launch_t(const ScoreArgs& a, int n_cu, hipStream_t s) {
    const int total = a.tile_start[a.batch];
    if (total == 0) return hipSuccess;
    int grid = (total + kWaves - 1) / kWaves;
    if (grid > n_cu) grid = n_cu;
    hipLaunchKernelGGL((fm_score_kernel<DK, KT>), dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace score_k
#ifndef LSA_BODIES_ONLY
using namespace score_k;
#endif
}  // namespace

#ifndef LSA_BODIES_ONLY
hipError_t launch_fm_score(const ScoreArgs& a, int key_dtype, int dk, int n_cu, hipStream_t s) {
    if (key_dtype == LSA_F32) {
        if (dk == 32) return launch_t<32, float>(a, n_cu, s);
        if (dk == 64) return launch_t<64, float>(a, n_cu, s);
        if (dk == 128) return launch_t<128, float>(a, n_cu, s);
    } else if (key_dtype == LSA_BF16) {
        if (dk == 32) return launch_t<32, uint16_t>(a, n_cu, s);
        if (dk == 64) return launch_t<64, uint16_t>(a, n_cu, s);
        if (dk == 128) return launch_t<128, uint16_t>(a, n_cu, s);
    }
    return hipErrorInvalidValue;
}

#endif  // LSA_BODIES_ONLY

}  // namespace lsa
