// Fused launches of the lookahead schedule.
//
// [P2] LSA section: the memory indexer predicts, ahead of time, the chunks the
// coming decoding window needs, and only those are recalled to the GPU; [P1]
// limitations / future work: the reference scores synchronously, and
// overlapping the global scoring is listed as the way to remove that cost.
//
// One lookahead step t runs on a single stream as three launches:
//   A  fm_score of step t+1, each workgroup with one extra wave that copies a
//      share of step t's missed rows into their slots (the score waves also
//      build the select's histogram and write its candidate lists)
//   (B select histogram of step t+1, only when A cannot: segments that are not
//      one per sequence, or fewer score workgroups than sequences)
//   (C select collect of step t+1, only when A did not write the lists)
//   D  [attention splits of step t                    | final select of step t+1]
//   E  [stage of step t+1 (LRU; records its misses)   | split merge of step t]
// Design (gfx950): independent work of two steps shares one launch
// ("horizontal fusion"): in A every score workgroup carries a copy wave, whose
// PCIe reads run beside the key scan on their own load counter; in D and E the
// first blocks of the launch run one body and the rest the other.  The final
// select (one workgroup per segment) and the stage (one per layer and
// sequence) leave most CUs idle, so the attention of step t fills them.  Every
// body is the same code the separate kernels run, so the results are those of
// the synchronous step.  The stage of step t+1 runs after the attention splits
// of step t have read their rows (stream order), and the stage itself moves no
// row (the next A copies them), so it may evict any row not selected for t+1.
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

typedef __attribute__((address_space(1))) u32x4 global_u32x4;

// 16-byte chunks each copy lane has in flight per pass.  One is fastest on the
// 1M-context workload (72.4 us per step against 73.7 / 75.7 / 76.7 us for 2 / 4 /
// 8): with 256 copy waves it keeps 256 KB of PCIe reads outstanding, which the
// link drains at its full rate, while deeper queues sit in the memory path in
// front of the score waves' key loads and slow both.
constexpr int kCopyInFlight = 1;

// The copy wave of a score workgroup.  All missed rows of the step are split
// into 16-byte chunks, numbered row by row in segment order, and lane `lane`
// of copy wave `wg` (of n_wg) takes chunks wg*64 + lane + u*G for G = 64*n_wg:
// every copy lane of the launch gets the same share, whatever the miss count of
// its own rows, so the PCIe reads stay spread evenly over the launch.  A chunk finds its segment by binary search of the prefix of the miss
// counts (in LDS).  Loads are unconditional on a clamped chunk index and stores
// are predicated, so a pass stays in registers.  The wave has its own load
// counter: the score waves never wait on its reads.
__device__ inline void copy_wave(const CopyArgs& ca, const int wg, const int n_wg, int* s_pre) {
    const int lane = threadIdx.x & 63;
    // exclusive prefix of the per-segment miss counts
    int carry = 0;
    for (int s0 = 0; s0 < ca.n_seg; s0 += 64) {
        const int sg = s0 + lane;
        const int c = sg < ca.n_seg ? ca.n_miss[sg] : 0;
        int v = c;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(v, d, 64);
            if (lane >= d) v += o;
        }
        if (sg < ca.n_seg) s_pre[sg] = carry + v - c;
        carry += __shfl(v, 63, 64);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    const int shift = __builtin_ctz((unsigned)(ca.row_bytes / 16));   // row_bytes / 16 is a power of two
    const int cpr_mask = (ca.row_bytes / 16) - 1;
    const int chunks = carry << shift;
    const int G = n_wg * 64;
    for (int base = wg * 64; base < chunks; base += G * kCopyInFlight) {
        uint64_t from[kCopyInFlight], to[kCopyInFlight];
#pragma clang loop unroll(full)
        for (int u = 0; u < kCopyInFlight; ++u) {
            int c = base + lane + u * G;
            c = c < chunks ? c : chunks - 1;
            const int m = c >> shift;                    // missed row, in segment order
            // last segment starting at or before m: a fixed-step binary search
            int lo = 0;
#pragma clang loop unroll(full)
            for (int step = kCopyMaxSegs / 2; step > 0; step >>= 1)
                if (lo + step < ca.n_seg && s_pre[lo + step] <= m) lo += step;
            const uint64_t* e = ca.miss + ((int64_t)lo * ca.phys_stride + (m - s_pre[lo])) * 2;
            const uint64_t off = (uint64_t)(c & cpr_mask) * 16u;
            from[u] = e[0] + off;
            to[u] = e[1] + off;
        }
        // global (not generic) accesses: their completion counts in order, so all
        // loads of the pass are issued before the first wait
        u32x4 v[kCopyInFlight];
#pragma clang loop unroll(full)
        for (int u = 0; u < kCopyInFlight; ++u) v[u] = *reinterpret_cast<const global_u32x4*>(from[u]);
#pragma clang loop unroll(full)
        for (int u = 0; u < kCopyInFlight; ++u)
            if (base + lane + u * G < chunks) *reinterpret_cast<global_u32x4*>(to[u]) = v[u];
    }
}

// Workgroup = 4 score waves (fm_score) + 1 copy wave.  With HIST the score
// waves also count their scores into an LDS histogram; the last of them to
// finish adds it to the segment's histogram (its PCIe-bound copy wave
// usually ends later, so the flush costs no time).  With CAND they also write
// the select's candidate lists (score_k::CandOut).
template <int DK, typename KT, bool HIST, bool CAND, bool NT>
__global__ __launch_bounds__(320, 1) void la_score_copy(const ScoreArgs sa, const CopyArgs ca, const ScoreHistArgs ha) {
    static_assert(!(HIST && CAND), "the lists replace the histogram");
    __shared__ int s_pre[kCopyMaxSegs];
    __shared__ uint32_t s_hist[HIST ? kSelBins : 1];
    __shared__ int s_done;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (HIST) {
        for (int i = threadIdx.x; i < kSelBins; i += 320) s_hist[i] = 0u;
        if (threadIdx.x == 0) s_done = 0;
        __syncthreads();
    }
    if (wave == 4) {
        copy_wave(ca, blockIdx.x, gridDim.x, s_pre);
        return;
    }
    const score_k::CandOut co{ha.blk_idx, ha.blk_key, ha.blk_count, ha.guess, ha.nblk,
                              ha.mode == LSA_SELECT_THRESHOLD ? 1 : 0, ha.t_f};
    score_k::fm_score_body<DK, KT, HIST, CAND, NT>(sa, blockIdx.x, gridDim.x, s_hist, ha.mode, ha.t_f, &co);
    if (HIST) score_k::score_hist_flush(sa, s_hist, &s_done, ha.hist);
}

// Launch D: the attention splits of step t beside the final selection of step
// t+1 (path 1: one 512-thread workgroup per segment).  Both wait long on few
// dependent memory reads, so neither lengthens the other.  The selection
// workgroups come first in the grid, so they are dispatched first: the splits'
// workgroups start over a few microseconds, and the selection's one long chain
// of dependent phases should not wait behind them.
constexpr int kFinMaxBlocks = 1024;   // collect blocks per segment (1M entries); more take the exact fallback

template <int D, typename KT>
__global__ __launch_bounds__(512, 1) void la_final_split(const AttendArgs aa, const SelectArgs se, const Split sp) {
    __shared__ __attribute__((aligned(16))) char tile[attend_k::tile_bytes<D, KT>()];
    const int n_sel = (int)gridDim.x - sp.n0;   // one workgroup per segment
    const int b = blockIdx.x;
    if (b < n_sel) {
        select_k::sel_final_body<512, kFinMaxBlocks>(se, b);
        return;
    }
    const int a = b - n_sel;
    attend_k::attend_split_body<D, KT>(aa, a % sp.x, (a / sp.x) % sp.y, a / (sp.x * sp.y), tile);
}

// Launch E: the stage of step t+1 (one 1024-thread workgroup per (layer,
// sequence)) beside the split merge of step t (four 32-column slices per
// workgroup).
template <int D>
__global__ __launch_bounds__(1024, 1) void la_stage_combine(const StageArgs ga, const AttendArgs aa, const Split sp) {
    const int b = blockIdx.x;
    if (b < sp.n0) {
        stage_k::kv_stage_body(ga.L[b / ga.batch], b % ga.batch, ga.src_valid[b % ga.batch]);
        return;
    }
    const int h = b - sp.n0;
    attend_k::attend_combine_body<D, 1024>(aa, h % sp.x2, (h / sp.x2) % aa.batch, h / (sp.x2 * aa.batch));
}

// The score launch's grid: one workgroup per CU at most; with the histogram
// and several sequences, whole workgroups per sequence.
int la_score_grid(const ScoreArgs& sa, bool hist, int n_cu) {
    const int total = sa.tile_start[sa.batch];
    int grid = (total + score_k::kWaves - 1) / score_k::kWaves;
    if (grid > n_cu) grid = n_cu;
    if (grid < 1) grid = 1;
    if (hist && sa.batch > 1) grid -= grid % sa.batch;
    return grid;
}

template <int DK, typename KT, bool NT>
void launch_a_nt(const ScoreArgs& sa, const CopyArgs& ca, const ScoreHistArgs& ha, int grid, hipStream_t s) {
    if (ha.blk_count)
        hipLaunchKernelGGL((la_score_copy<DK, KT, false, true, NT>), dim3(grid), dim3(320), 0, s, sa, ca, ha);
    else if (ha.hist)
        hipLaunchKernelGGL((la_score_copy<DK, KT, true, false, NT>), dim3(grid), dim3(320), 0, s, sa, ca, ha);
    else
        hipLaunchKernelGGL((la_score_copy<DK, KT, false, false, NT>), dim3(grid), dim3(320), 0, s, sa, ca, ha);
}

template <int DK, typename KT>
hipError_t launch_a(const ScoreArgs& sa, const CopyArgs& ca, const ScoreHistArgs& ha, int n_cu, hipStream_t s,
                    bool stream_keys) {
    const int grid = la_score_grid(sa, ha.hist != nullptr || ha.blk_count != nullptr, n_cu);
    if (grid < 1) return hipErrorInvalidValue;
    if (stream_keys)
        launch_a_nt<DK, KT, true>(sa, ca, ha, grid, s);
    else
        launch_a_nt<DK, KT, false>(sa, ca, ha, grid, s);
    return hipGetLastError();
}

template <int D, typename KT>
hipError_t launch_d(const AttendArgs& aa, const SelectArgs& se, bool hist_done, hipStream_t s) {
    Split sp{};
    sp.x = aa.max_splits;
    sp.y = aa.batch;
    sp.n0 = aa.max_splits * aa.batch * aa.n_layers;
    if (se.path == 1) {
        // hist (unless the score launch built it) and collect, then the final
        // selection beside the attention splits
        hipError_t e = hipSuccess;
        if (!hist_done && !se.pre) {
            hipLaunchKernelGGL(select_k::sel_hist_kernel,
                               dim3((unsigned)((se.n_keys + select_k::kBlk - 1) / select_k::kBlk), se.n_seg),
                               dim3(select_k::kBlkThreads), 0, s, se);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        if (!se.pre) {
            hipLaunchKernelGGL(select_k::sel_collect_kernel, dim3(se.nblk, se.n_seg), dim3(select_k::kBlkThreads), 0, s,
                               se);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL((la_final_split<D, KT>), dim3(sp.n0 + se.n_seg), dim3(512), 0, s, aa, se, sp);
        return hipGetLastError();
    }
    // short segments: the attention splits, then the one-kernel selection
    if (sp.n0 > 0) {
        hipLaunchKernelGGL((attend_k::attend_split_kernel<D, KT>), dim3(aa.max_splits, aa.batch, aa.n_layers),
                           dim3(attend_k::kThreads), 0, s, aa);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_fm_select(se, s);
}

template <int D>
hipError_t launch_e(const StageArgs& ga, const AttendArgs& aa, hipStream_t s) {
    Split sp{};
    sp.n0 = ga.batch * ga.n_layers;
    sp.x2 = (D / attend_k::kCombCols + 3) / 4;
    const int nc = sp.x2 * aa.batch * aa.n_layers;
    hipLaunchKernelGGL((la_stage_combine<D>), dim3(sp.n0 + nc), dim3(1024), 0, s, ga, aa, sp);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_la_fetch_score(const ScoreArgs& sa, const CopyArgs& ca, int key_dtype, int dk, int n_cu,
                                 const SelectArgs* hist_for, const int32_t* guess, bool* lists, hipStream_t s,
                                 bool stream_keys) {
    const int cpr = ca.row_bytes / 16;
    if (ca.n_seg < 0 || ca.n_seg > kCopyMaxSegs || (ca.n_seg && (!ca.miss || !ca.n_miss)) || ca.row_bytes % 16 != 0 ||
        cpr < 1 || (cpr & (cpr - 1)) != 0)
        return hipErrorInvalidValue;
    ScoreHistArgs ha{};
    *lists = false;
    if (hist_for) {
        if (!la_fused_hist(sa, *hist_for, n_cu)) return hipErrorInvalidValue;
        ha.mode = hist_for->mode;
        ha.t_f = hist_for->t_f;
        // the candidate lists in place of the histogram when their sub-blocks
        // fit the final selection's block table
        const int G = la_score_grid(sa, true, n_cu) / sa.batch;
        if (guess && G > 0 && hist_for->nblk * score_k::kWaves <= kFinMaxBlocks) {
            ha.blk_count = hist_for->blk_count;
            ha.blk_idx = hist_for->blk_idx;
            ha.blk_key = hist_for->blk_key;
            ha.guess = guess;
            ha.nblk = hist_for->nblk;
            *lists = true;
        } else {
            ha.hist = hist_for->hist;
        }
    }
    if (key_dtype == LSA_F32) {
        if (dk == 32) return launch_a<32, float>(sa, ca, ha, n_cu, s, stream_keys);
        if (dk == 64) return launch_a<64, float>(sa, ca, ha, n_cu, s, stream_keys);
        if (dk == 128) return launch_a<128, float>(sa, ca, ha, n_cu, s, stream_keys);
    } else if (key_dtype == LSA_BF16) {
        if (dk == 32) return launch_a<32, uint16_t>(sa, ca, ha, n_cu, s, stream_keys);
        if (dk == 64) return launch_a<64, uint16_t>(sa, ca, ha, n_cu, s, stream_keys);
        if (dk == 128) return launch_a<128, uint16_t>(sa, ca, ha, n_cu, s, stream_keys);
    } else if (key_dtype == LSA_FP8_E4M3) {
        if (dk == 32) return launch_a<32, uint8_t>(sa, ca, ha, n_cu, s, stream_keys);
        if (dk == 64) return launch_a<64, uint8_t>(sa, ca, ha, n_cu, s, stream_keys);
        if (dk == 128) return launch_a<128, uint8_t>(sa, ca, ha, n_cu, s, stream_keys);
    } else if (key_dtype == LSA_MXFP4) {
        if (dk == 64) return launch_a<64, score_k::mxfp4_tag>(sa, ca, ha, n_cu, s, stream_keys);
        if (dk == 128) return launch_a<128, score_k::mxfp4_tag>(sa, ca, ha, n_cu, s, stream_keys);
    } else if (key_dtype == LSA_MXINT8) {
        if (dk == 32) return launch_a<32, score_k::mxint8_tag>(sa, ca, ha, n_cu, s, stream_keys);
        if (dk == 64) return launch_a<64, score_k::mxint8_tag>(sa, ca, ha, n_cu, s, stream_keys);
        if (dk == 128) return launch_a<128, score_k::mxint8_tag>(sa, ca, ha, n_cu, s, stream_keys);
    }
    return hipErrorInvalidValue;
}

bool la_fused_hist(const ScoreArgs& sa, const SelectArgs& se, int n_cu) {
    // one select segment per sequence, and at least one workgroup of score waves
    // per sequence: the grid (capped at one workgroup per CU, then rounded down
    // to a multiple of the batch, as launch_a does) must keep one per sequence
    const int tiles = sa.tile_start[sa.batch];
    int grid = (tiles + score_k::kWaves - 1) / score_k::kWaves;
    if (grid > n_cu) grid = n_cu;
    return se.path == 1 && se.n_seg == sa.batch && se.hist != nullptr && grid >= sa.batch;
}

hipError_t launch_la_select_split(const AttendArgs& aa, const SelectArgs& se, bool hist_done, hipStream_t s) {
    if (aa.max_splits == 0) return hipErrorInvalidValue;
    if (aa.dtype == LSA_F32) {
        if (aa.D == 128) return launch_d<128, float>(aa, se, hist_done, s);
        if (aa.D == 256) return launch_d<256, float>(aa, se, hist_done, s);
        if (aa.D == 512) return launch_d<512, float>(aa, se, hist_done, s);
    } else if (aa.dtype == LSA_BF16) {
        if (aa.D == 128) return launch_d<128, uint16_t>(aa, se, hist_done, s);
        if (aa.D == 256) return launch_d<256, uint16_t>(aa, se, hist_done, s);
        if (aa.D == 512) return launch_d<512, uint16_t>(aa, se, hist_done, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_la_stage_combine(const StageArgs& ga, const AttendArgs& aa, hipStream_t s) {
    if (ga.batch != aa.batch || ga.n_layers != aa.n_layers) return hipErrorInvalidValue;
    if (aa.D == 128) return launch_e<128>(ga, aa, s);
    if (aa.D == 256) return launch_e<256>(ga, aa, s);
    if (aa.D == 512) return launch_e<512>(ga, aa, s);
    return hipErrorInvalidValue;
}

}  // namespace lsa
