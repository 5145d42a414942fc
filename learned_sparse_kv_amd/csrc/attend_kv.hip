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

template <int DH, typename ET>
__global__ __launch_bounds__(512) void attend_kv_kernel(const AttendKVArgs a) {
    constexpr int kLpr = DH * 2 / 16;       // lanes per row slice
    constexpr int kRpi = 64 / kLpr;         // rows per wave load
    constexpr int kUnroll = 4;              // rows per lane group per batch (K and V: 8 loads in flight)
    // LDS: per list row its slot byte offset and cold row (-1: none)
    extern __shared__ int32_t lds[];
    const int s = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int h = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = lane % kLpr, rg = lane / kLpr;
    int n = a.n_rows[s];
    n = n < 0 ? 0 : (n > a.phys_stride ? a.phys_stride : n);
    float* out = a.out + ((int64_t)s * a.heads + h) * DH;
    if (n == 0) {   // uniform over the workgroup
        if (lane < kLpr)
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
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(srcs ? reinterpret_cast<const void*>(a.seg_cold[s]) : a.kv, cold_rec);
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
    for (int i0 = 0; i0 < n; i0 += kRpi * kUnroll) {
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
    const float g = expf(m - mw);   // mw is finite (n >= 1); a group with no row has m = -inf, weight 0
    l *= g;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= g;
#pragma unroll
    for (int o = kLpr; o < 64; o <<= 1) {
        l += __shfl_xor(l, o, 64);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
    }
    if (lane < kLpr) {
        const float inv_l = 1.0f / l;
#pragma unroll
        for (int e = 0; e < 8; ++e) out[lane * 8 + e] = acc[e] * inv_l;
    }
}

template <int DH>
hipError_t launch_dh(const AttendKVArgs& a, hipStream_t s) {
    const size_t lds = (size_t)2 * a.phys_stride * sizeof(int32_t);
    if (a.dtype == LSA_F16)
        hipLaunchKernelGGL((attend_kv_kernel<DH, uint16_t>), dim3(a.n_seg), dim3(64 * a.heads), lds, s, a);
    else if (a.dtype == LSA_BF16)
        hipLaunchKernelGGL((attend_kv_kernel<DH, Bf16>), dim3(a.n_seg), dim3(64 * a.heads), lds, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attend_kv(const AttendKVArgs& a, hipStream_t s) {
    if (a.n_seg == 0) return hipSuccess;
    if (a.head_dim == 64) return launch_dh<64>(a, s);
    if (a.head_dim == 128) return launch_dh<128>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace lsa
