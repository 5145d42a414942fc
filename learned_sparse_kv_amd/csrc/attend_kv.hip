// Per-head attention of the KVSwap variant over separate K and V rows.
//
// KVSwap article, section 2.2 (grouped loading: the heads of a group share one
// selection) and section 3.2 (the selected entries sit in a bounded buffer):
// for segment s (one head group of one sequence and layer) and each head h of
// the group, with rows r = phys[s][0..n-1] of the staging buffer,
//     out[s,h,:] = sum_r softmax_r(scale * q[s,h,:] . K_h[r,:]) * V_h[r,:]
// where a row holds the keys of all the group's heads followed by their values.
//
// Design (gfx950): one workgroup per segment and one wave per head.  A head's
// key and value slices of a row are head_dim * 2 bytes each; head_dim*2/16
// lanes load one with 16-byte buffer loads, so a wave load covers 4 (dh 128)
// or 8 (dh 64) rows and reads each row slice exactly once.  The K and V slices
// of a batch of rows are loaded together and the softmax is taken in the same
// pass with a running maximum per lane group (rescaled once per batch), so a
// wave waits on memory once per batch instead of once per pass; the lane
// groups are combined in a fixed order at the end.  The work per row is a few
// flops per byte: an HBM stream, not a contraction worth MFMA (M = 1 per head).
#include "lsa_internal.hpp"
#define LSA_BODIES_ONLY
#include "kv_stage.hip"
#undef LSA_BODIES_ONLY

namespace lsa {

namespace {

template <typename T>
__device__ inline void unpack8(const uint4& u, float* f);

template <>
__device__ inline void unpack8<uint16_t>(const uint4& u, float* f) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = f16_to_f32((uint16_t)(w[e] & 0xFFFF));
        f[2 * e + 1] = f16_to_f32((uint16_t)(w[e] >> 16));
    }
}

struct Bf16 {};
template <>
__device__ inline void unpack8<Bf16>(const uint4& u, float* f) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = bf16_lo(w[e]);
        f[2 * e + 1] = bf16_hi(w[e]);
    }
}

// LDS words of the body: the row list (2 per row), and with WPH > 1 the
// partial results of the waves after the first of each head
__host__ __device__ inline int attend_kv_lds_words(int phys_stride, int heads, int dh, int wph) {
    return 2 * phys_stride + (wph > 1 ? heads * (wph - 1) * (dh / 8) * 10 : 0);
}

// Segment s; WPH waves per head (wave w: head w / WPH, rows of every WPH-th
// batch from w % WPH), the workgroup's waves = heads * WPH.  The waves of a
// head are combined in order by the first.  The reads of n_rows and seg_cold
// are vector loads, so a stage that has just written them in this workgroup
// is seen.
template <int DH, typename ET, int WPH>
__device__ __forceinline__ void attend_kv_body(const AttendKVArgs& a, const int s, int32_t* lds) {
    constexpr int kLpr = DH * 2 / 16;       // lanes per row slice
    constexpr int kRpi = 64 / kLpr;         // rows per wave load
    constexpr int kUnroll = 4;              // rows per lane group per batch (K and V: 8 loads in flight)
    // LDS: per list row its slot byte offset and cold row (-1: none)
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = wv / WPH, part = wv % WPH;
    const int sub = lane % kLpr, rg = lane / kLpr;
    int n = __hip_atomic_load(a.n_rows + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    n = n < 0 ? 0 : (n > a.phys_stride ? a.phys_stride : n);
    float* out = a.out + ((int64_t)s * a.heads + h) * DH;
    if (n == 0) {   // uniform over the workgroup
        if (part == 0 && lane < kLpr)
            for (int e = 0; e < 8; ++e) out[lane * 8 + e] = 0.0f;
        return;
    }
    uint32_t* s_off = reinterpret_cast<uint32_t*>(lds);
    int32_t* s_src = lds + a.phys_stride;

    const uint32_t row_bytes = (uint32_t)(2 * a.heads * DH * 2);
    const uint32_t nrec = (uint32_t)a.kv_rows * row_bytes;
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(static_cast<const char*>(a.kv) + a.kv_stride_seg * 2 * s, nrec);
    const int32_t* ph = a.phys + (int64_t)s * a.phys_stride;
    const int32_t* srcs = a.src ? a.src + (int64_t)s * a.phys_stride : nullptr;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int32_t p = ph[i];
        // rows outside [0, kv_rows) read as zero (offset past the buffer)
        s_off[i] = ((uint32_t)p < (uint32_t)a.kv_rows) ? (uint32_t)p * row_bytes : nrec;
        s_src[i] = srcs ? srcs[i] : -1;
    }
    __syncthreads();

    const uint32_t k_off = (uint32_t)(h * DH * 2 + sub * 16);
    const uint32_t v_off = (uint32_t)((a.heads + h) * DH * 2 + sub * 16);
    // deferred staging: a missed row is read from the cold store and this
    // head's K and V slices are written into its slot.  Every lane issues both
    // the slot loads and the cold loads; the ones it does not need are pointed
    // past their buffer, read zero and move no data, so the loads of a batch
    // stay branch-free and in flight together.  The cold reads and the slot
    // writes are non-temporal: neither is read again in this step, and kept
    // lines would only push out what the next launches stream (32K KVSwap
    // step 2.60 -> 2.58 ms, most of it in the next step's score).
    const uint32_t cold_rec = srcs ? (uint32_t)a.cold_rows * row_bytes : 0u;
    const uint64_t cold_base =
        srcs ? __hip_atomic_load(a.seg_cold + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) : 0ull;
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(srcs ? reinterpret_cast<const void*>(cold_base) : a.kv, cold_rec);
    auto load_batch = [&](int i0, uint4* kk, uint4* vv) {
        int32_t c[kUnroll];
        uint32_t off[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int i = i0 + u * kRpi + rg;
            off[u] = i < n ? s_off[i] : nrec;
            c[u] = i < n ? s_src[i] : -1;
        }
        if (!srcs) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                kk[u] = buffer_load16(r, off[u] + k_off);
                vv[u] = buffer_load16(r, off[u] + v_off);
            }
            return;
        }
        uint4 wk[kUnroll], wv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const bool cold = (uint32_t)c[u] < (uint32_t)a.cold_rows;
            const uint32_t so = cold ? nrec : off[u];
            const uint32_t co = cold ? (uint32_t)c[u] * row_bytes : cold_rec;
            kk[u] = buffer_load16(r, so + k_off);
            vv[u] = buffer_load16(r, so + v_off);
            wk[u] = buffer_load16_nt(rc, co + k_off);
            wv[u] = buffer_load16_nt(rc, co + v_off);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const bool cold = (uint32_t)c[u] < (uint32_t)a.cold_rows;
            kk[u] = make_uint4(kk[u].x | wk[u].x, kk[u].y | wk[u].y, kk[u].z | wk[u].z, kk[u].w | wk[u].w);
            vv[u] = make_uint4(vv[u].x | wv[u].x, vv[u].y | wv[u].y, vv[u].z | wv[u].z, vv[u].w | wv[u].w);
            // the slot writes go past the buffer (dropped) unless this row was missed
            const uint32_t wo = (cold && off[u] < nrec) ? off[u] : nrec;
            const u32x4 dk = {kk[u].x, kk[u].y, kk[u].z, kk[u].w};
            const u32x4 dv = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
            __builtin_amdgcn_raw_buffer_store_b128(dk, r, wo == nrec ? nrec : wo + k_off, 0, 2);
            __builtin_amdgcn_raw_buffer_store_b128(dv, r, wo == nrec ? nrec : wo + v_off, 0, 2);
        }
    };

    float qv[8];
    {
        const float* qh = a.q + ((int64_t)s * a.heads + h) * DH + sub * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = qh[e];
    }

    // one pass with a running maximum: lane group rg takes rows i = rg (mod
    // kRpi) and keeps its own maximum m, sum l and PV sums acc; each batch
    // rescales them once by exp(m_old - m_new)
    float m = -INFINITY, l = 0.0f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int i0 = part * kRpi * kUnroll; i0 < n; i0 += WPH * kRpi * kUnroll) {
        uint4 kk[kUnroll], vv[kUnroll];
        load_batch(i0, kk, vv);
        float z[kUnroll];
        float mb = m;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float f[8];
            unpack8<ET>(kk[u], f);
            float d = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) d += qv[e] * f[e];
#pragma unroll
            for (int o = 1; o < kLpr; o <<= 1) d += __shfl_xor(d, o, 64);
            const int i = i0 + u * kRpi + rg;
            z[u] = i < n ? a.scale * d : -INFINITY;
            mb = fmaxf(mb, z[u]);
        }
        // a group with no row yet keeps m = -inf; 0 then stands in for the
        // maximum so that every exponent below is -inf (weight 0), not NaN
        const float mu = mb == -INFINITY ? 0.0f : mb;
        const float corr = expf(m - mu);
        l *= corr;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= corr;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const float pz = expf(z[u] - mu);
            l += pz;
            float f[8];
            unpack8<ET>(vv[u], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += pz * f[e];
        }
        m = mb;
    }
    // combine the lane groups: each to the wave's maximum, then summed
    float mw = m;
#pragma unroll
    for (int o = kLpr; o < 64; o <<= 1) mw = fmaxf(mw, __shfl_xor(mw, o, 64));
    // a group with no row has m = -inf (weight 0); a wave with no row at all (WPH > 1, short
    // lists) has mw = -inf too and keeps l = 0, sums 0
    const float g = mw == -INFINITY ? 0.0f : expf(m - mw);
    l *= g;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= g;
#pragma unroll
    for (int o = kLpr; o < 64; o <<= 1) {
        l += __shfl_xor(l, o, 64);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
    }
    if constexpr (WPH > 1) {
        // the other waves of this head hand their (m, l, sums) to the first, which
        // takes them in wave order
        float* comb = reinterpret_cast<float*>(lds + 2 * a.phys_stride) + (h * (WPH - 1)) * kLpr * 10;
        if (part > 0 && lane < kLpr) {
            float* c = comb + ((part - 1) * kLpr + lane) * 10;
            c[0] = mw;
            c[1] = l;
#pragma unroll
            for (int e = 0; e < 8; ++e) c[2 + e] = acc[e];
        }
        __syncthreads();
        if (part > 0) return;
        if (lane < kLpr) {
            float mt = mw;
            for (int q = 1; q < WPH; ++q) mt = fmaxf(mt, comb[((q - 1) * kLpr + lane) * 10]);
            // a wave with no row has m = -inf (weight 0); mt is finite (n >= 1)
            const float g0 = expf(mw - mt);
            l *= g0;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] *= g0;
            for (int q = 1; q < WPH; ++q) {
                const float* c = comb + ((q - 1) * kLpr + lane) * 10;
                const float gq = expf(c[0] - mt);
                l += c[1] * gq;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += c[2 + e] * gq;
            }
        }
    }
    if (lane < kLpr) {
        const float inv_l = 1.0f / l;
#pragma unroll
        for (int e = 0; e < 8; ++e) out[lane * 8 + e] = acc[e] * inv_l;
    }
}

template <int DH, typename ET>
__global__ __launch_bounds__(512) void attend_kv_kernel(const AttendKVArgs a) {
    extern __shared__ int32_t lds[];
    attend_kv_body<DH, ET, 1>(a, blockIdx.x, lds);
}

// KVSwap section 3.2 then section 2.2 for one segment per workgroup: the
// segment's stage (the 512-thread form of kv_stage, pools of at most 512
// slots), then its attention with 8 / heads waves per head.  The stage's
// chain of dependent rounds then overlaps the attention streams of the other
// workgroups on the CU instead of taking a launch of its own.
template <int DH, typename ET, int WPH>
__global__ __launch_bounds__(512) void stage_attend_kv_kernel(const StageLayer* Ls, const int batch,
                                                              const AttendKVArgs a) {
    extern __shared__ int32_t lds[];
    const int s = blockIdx.x;
    {
        const StageLayer L = Ls[s / batch];
        stage_k::kv_stage_body<stage_k::kSmallNT, stage_k::kSmallNT>(L, s % batch, 0x7FFFFFFF);
    }
    __syncthreads();   // the stage's tables, row list and miss sources are written
    attend_kv_body<DH, ET, WPH>(a, s, lds);
}

template <int DH>
hipError_t launch_dh(const AttendKVArgs& a, hipStream_t s) {
    const size_t lds = (size_t)attend_kv_lds_words(a.phys_stride, a.heads, DH, 1) * sizeof(int32_t);
    if (a.dtype == LSA_F16)
        hipLaunchKernelGGL((attend_kv_kernel<DH, uint16_t>), dim3(a.n_seg), dim3(64 * a.heads), lds, s, a);
    else if (a.dtype == LSA_BF16)
        hipLaunchKernelGGL((attend_kv_kernel<DH, Bf16>), dim3(a.n_seg), dim3(64 * a.heads), lds, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <int DH, int WPH>
hipError_t launch_sa(const StageLayer* layers, int batch, const AttendKVArgs& a, hipStream_t s) {
    const size_t lds = (size_t)attend_kv_lds_words(a.phys_stride, a.heads, DH, WPH) * sizeof(int32_t);
    const dim3 grid(a.n_seg), block(64 * a.heads * WPH);
    if (a.dtype == LSA_F16)
        hipLaunchKernelGGL((stage_attend_kv_kernel<DH, uint16_t, WPH>), grid, block, lds, s, layers, batch, a);
    else if (a.dtype == LSA_BF16)
        hipLaunchKernelGGL((stage_attend_kv_kernel<DH, Bf16, WPH>), grid, block, lds, s, layers, batch, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <int DH>
hipError_t launch_sa_dh(const StageLayer* layers, int batch, const AttendKVArgs& a, hipStream_t s) {
    switch (a.heads) {
        case 1: return launch_sa<DH, 8>(layers, batch, a, s);
        case 2: return launch_sa<DH, 4>(layers, batch, a, s);
        case 4: return launch_sa<DH, 2>(layers, batch, a, s);
        case 8: return launch_sa<DH, 1>(layers, batch, a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_attend_kv(const AttendKVArgs& a, hipStream_t s) {
    if (a.n_seg == 0) return hipSuccess;
    if (a.head_dim == 64) return launch_dh<64>(a, s);
    if (a.head_dim == 128) return launch_dh<128>(a, s);
    return hipErrorInvalidValue;
}

bool stage_attend_kv_fits(int heads, int head_dim, int phys_stride, int max_slots) {
    return (heads == 1 || heads == 2 || heads == 4 || heads == 8) && (head_dim == 64 || head_dim == 128) &&
           phys_stride >= 1 && phys_stride <= stage_k::kSmallNT && max_slots <= stage_k::kSmallNT;
}

hipError_t launch_stage_attend_kv(const StageLayer* layers, int batch, const AttendKVArgs& a, hipStream_t s) {
    if (a.n_seg == 0) return hipSuccess;
    if (batch < 1 || a.n_seg % batch != 0) return hipErrorInvalidValue;
    if (a.head_dim == 64) return launch_sa_dh<64>(layers, batch, a, s);
    if (a.head_dim == 128) return launch_sa_dh<128>(layers, batch, a, s);
    return hipErrorInvalidValue;
}

}  // namespace lsa
