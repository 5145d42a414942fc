// Fused launches of the lookahead schedule.
//
// [P2] LSA section: the memory indexer predicts, ahead of time, the chunks the
// coming decoding window needs, and only those are recalled to the GPU; [P1]
// limitations / future work: the reference scores synchronously, and
// overlapping the global scoring is listed as the way to remove that cost.
//
// One lookahead step t runs on a single stream as five launches:
//   A  fm_score of step t+1, each workgroup with one extra wave that copies a
//      share of step t's missed rows into their slots
//   B  [attention splits of step t                    | select histogram t+1]
//   C  [attention combine of step t                   | select collect t+1]
//   D  select of step t+1 (final)
//   E  stage of step t+1 (LRU; records its misses for the next A)
// Design (gfx950): independent work of two steps shares one launch
// ("horizontal fusion"): in A every score workgroup carries a copy wave, whose
// PCIe reads run beside the key scan on their own load counter; in B and C the
// first blocks of the launch run one body and the rest the other.  So the row
// copies overlap the key scan and the attention overlaps the selection without
// extra streams, events or host launches.  Every body is the same code the separate kernels run, so the
// results are those of the synchronous step.  Stage t+1 runs after the
// attention of step t has finished (stream order), so it may evict any row
// not selected for t+1.
#define LSA_BODIES_ONLY
#include "fm_score.hip"
#include "fm_select.hip"
#include "kv_stage.hip"
#include "lsa_attend.hip"
#undef LSA_BODIES_ONLY

namespace lsa {

namespace {

struct Split {
    int n0;        // blocks of the first body
    int x, y;      // its grid (x fastest), z = n0 / (x * y)
    int x2;        // second body's x extent (y = rest)
};

// The copy wave of a score workgroup: copies the missed rows recorded in the
// list rows wg, wg + n_wg, wg + 2 n_wg, ... of the flattened (layer, sequence,
// row) space from the cold pool into their slots.  Its misses go to LDS in
// rank order, then every lane copies 16-byte chunks of them, kCopyInFlight
// loads at a time (loads unconditional on clamped indices, stores predicated,
// so the batch stays in registers).  The wave has its own load counter, so the
// score waves never wait on its loads; on a pinned-host cold pool the PCIe
// reads still slow down while the score streams keys from HBM (measured: the
// fused launch takes about the score time plus the fetch time).
#ifndef LSA_COPY_IN_FLIGHT
#define LSA_COPY_IN_FLIGHT 4
#endif
constexpr int kCopyInFlight = LSA_COPY_IN_FLIGHT;

struct CopyRow {
    int64_t from;   // byte offset in the layer's cold pool
    int64_t to;     // byte offset in the layer's KV buffer
    int layer, row_bytes;
};

__device__ inline void copy_wave(const StageArgs& ga, int phys_stride, int wg, int n_wg, CopyRow* rows) {
    const int lane = threadIdx.x & 63;
    const int per_layer = ga.batch * phys_stride;
    const int total = ga.n_layers * per_layer;
    for (int k0 = 0; wg + k0 * n_wg < total; k0 += 64) {
        const int i = wg + (k0 + lane) * n_wg;
        bool miss = false;
        CopyRow cr{0, 0, 0, 0};
        if (i < total) {
            const int layer = i / per_layer, b = (i / phys_stride) % ga.batch, r = i % phys_stride;
            const StageLayer& L = ga.L[layer];
            if (L.swap && r < L.n_rows[b]) {
                const int sr = L.src[(int64_t)b * phys_stride + r];
                const int ph = L.phys[(int64_t)b * phys_stride + r];
                if (sr >= 0 && sr < L.cap && ph >= L.window && ph < L.window + L.S) {
                    miss = true;
                    cr.from = b * L.cold_stride_b + (int64_t)sr * L.row_bytes;
                    cr.to = b * L.kv_stride_b_bytes + (int64_t)ph * L.row_bytes;
                    cr.layer = layer;
                    cr.row_bytes = L.row_bytes;
                }
            }
        }
        const uint64_t m = __ballot(miss);
        const int n = __popcll(m);
        if (n == 0) continue;
        if (miss) rows[__popcll(m & ((1ull << lane) - 1ull))] = cr;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int cpr = rows[0].row_bytes / 16;   // one row size per step (every layer shares kv_dim)
        const int chunks = n * cpr;
        // source and destination of chunk c (clamped to the last chunk)
        auto at = [&](int c, const char*& from, char*& to) {
            const int cc = c < chunks ? c : chunks - 1;
            const int j = cc / cpr, off = (cc - j * cpr) * 16;
            const CopyRow& r = rows[j];
            from = static_cast<const char*>(ga.L[r.layer].cold) + r.from + off;
            to = static_cast<char*>(ga.L[r.layer].kv) + r.to + off;
        };
        for (int c0 = 0; c0 < chunks; c0 += 64 * kCopyInFlight) {
            // kCopyInFlight chunks per lane in flight
            const char* f[kCopyInFlight];
            char* to[kCopyInFlight];
            uint4 v[kCopyInFlight];
#pragma unroll
            for (int u = 0; u < kCopyInFlight; ++u) at(c0 + u * 64 + lane, f[u], to[u]);
#pragma unroll
            for (int u = 0; u < kCopyInFlight; ++u) v[u] = *reinterpret_cast<const uint4*>(f[u]);
#pragma unroll
            for (int u = 0; u < kCopyInFlight; ++u)
                if (c0 + u * 64 + lane < chunks) *reinterpret_cast<uint4*>(to[u]) = v[u];
        }
        // the next pass may reuse the list entries
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// Workgroup = 4 score waves (fm_score) + 1 copy wave.
template <int DK, typename KT>
__global__ __launch_bounds__(320, 1) void la_score_copy(const ScoreArgs sa, const StageArgs ga, const int phys_stride) {
    __shared__ CopyRow s_rows[64];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (wave == 4) {
        copy_wave(ga, phys_stride, blockIdx.x, gridDim.x, s_rows);
        return;
    }
    score_k::fm_score_body<DK, KT>(sa, blockIdx.x, gridDim.x);
}

template <int D, typename KT>
__global__ __launch_bounds__(512, 2) void la_attend_hist(const AttendArgs aa, const SelectArgs se, const Split sp) {
    const int b = blockIdx.x;
    if (b < sp.n0) {
        attend_k::attend_split_body<D, KT>(aa, b % sp.x, (b / sp.x) % sp.y, b / (sp.x * sp.y));
        return;
    }
    const int h = b - sp.n0;
    select_k::sel_hist_body<512>(se, h % sp.x2, h / sp.x2);
}

template <int D>
__global__ __launch_bounds__(256) void la_combine_collect(const AttendArgs aa, const SelectArgs se, const Split sp) {
    const int b = blockIdx.x;
    if (b < sp.n0) {
        attend_k::attend_combine_body<D>(aa, b % sp.x, (b / sp.x) % sp.y, b / (sp.x * sp.y));
        return;
    }
    const int h = b - sp.n0;
    select_k::sel_collect_body(se, h % sp.x2, h / sp.x2);
}

template <int DK, typename KT>
hipError_t launch_a(const ScoreArgs& sa, const StageArgs& ga, int phys_stride, int n_cu, hipStream_t s) {
    const int total = sa.tile_start[sa.batch];
    int grid = (total + score_k::kWaves - 1) / score_k::kWaves;
    if (grid > n_cu) grid = n_cu;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL((la_score_copy<DK, KT>), dim3(grid), dim3(320), 0, s, sa, ga, phys_stride);
    return hipGetLastError();
}

template <int D, typename KT>
hipError_t launch_b(const AttendArgs& aa, const SelectArgs& se, hipStream_t s) {
    Split sp{};
    sp.x = aa.max_splits;
    sp.y = aa.batch;
    sp.n0 = aa.max_splits * aa.batch * aa.n_layers;
    int nh = 0;
    if (se.path == 1) {
        sp.x2 = (int)((se.n_keys + select_k::kBlk - 1) / select_k::kBlk);
        nh = sp.x2 * se.n_seg;
    }
    if (sp.n0 + nh == 0) return hipSuccess;
    hipLaunchKernelGGL((la_attend_hist<D, KT>), dim3(sp.n0 + nh), dim3(512), 0, s, aa, se, sp);
    return hipGetLastError();
}

template <int D>
hipError_t launch_c(const AttendArgs& aa, const SelectArgs& se, hipStream_t s) {
    Split sp{};
    sp.x = D / attend_k::kCombCols;
    sp.y = aa.batch;
    sp.n0 = sp.x * aa.batch * aa.n_layers;
    int nc = 0;
    if (se.path == 1) {
        sp.x2 = se.nblk;
        nc = se.nblk * se.n_seg;
    }
    if (sp.n0 + nc == 0) return hipSuccess;
    hipLaunchKernelGGL((la_combine_collect<D>), dim3(sp.n0 + nc), dim3(256), 0, s, aa, se, sp);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_la_fetch_score(const ScoreArgs& sa, const StageArgs& ga, int phys_stride, int key_dtype, int dk,
                                 int n_cu, hipStream_t s) {
    if (key_dtype == LSA_F32) {
        if (dk == 32) return launch_a<32, float>(sa, ga, phys_stride, n_cu, s);
        if (dk == 64) return launch_a<64, float>(sa, ga, phys_stride, n_cu, s);
        if (dk == 128) return launch_a<128, float>(sa, ga, phys_stride, n_cu, s);
    } else if (key_dtype == LSA_BF16) {
        if (dk == 32) return launch_a<32, uint16_t>(sa, ga, phys_stride, n_cu, s);
        if (dk == 64) return launch_a<64, uint16_t>(sa, ga, phys_stride, n_cu, s);
        if (dk == 128) return launch_a<128, uint16_t>(sa, ga, phys_stride, n_cu, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_la_attend_hist(const AttendArgs& aa, const SelectArgs& se, hipStream_t s) {
    if (aa.max_splits == 0) return hipErrorInvalidValue;
    if (aa.dtype == LSA_F32) {
        if (aa.D == 128) return launch_b<128, float>(aa, se, s);
        if (aa.D == 256) return launch_b<256, float>(aa, se, s);
        if (aa.D == 512) return launch_b<512, float>(aa, se, s);
    } else if (aa.dtype == LSA_BF16) {
        if (aa.D == 128) return launch_b<128, uint16_t>(aa, se, s);
        if (aa.D == 256) return launch_b<256, uint16_t>(aa, se, s);
        if (aa.D == 512) return launch_b<512, uint16_t>(aa, se, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_la_combine_collect(const AttendArgs& aa, const SelectArgs& se, hipStream_t s) {
    if (aa.D == 128) return launch_c<128>(aa, se, s);
    if (aa.D == 256) return launch_c<256>(aa, se, s);
    if (aa.D == 512) return launch_c<512>(aa, se, s);
    return hipErrorInvalidValue;
}

}  // namespace lsa
