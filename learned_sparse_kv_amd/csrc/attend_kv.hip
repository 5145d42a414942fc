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
// key (and later value) slice of a row is head_dim * 2 bytes; head_dim*2/16
// lanes load it with 16-byte buffer loads, so a wave load covers 4 (dh 128) or
// 8 (dh 64) rows and reads each row slice exactly once.  Pass 1 forms the
// scaled dots into LDS, the softmax is taken over LDS, pass 2 accumulates
// p_i * V rows per lane group and the groups are combined in a fixed order.
// The work per row is a few flops per byte: an HBM stream, not a contraction
// worth MFMA (M = 1 per head).
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
    constexpr int kUnroll = 4;
    // LDS: per list row its slot byte offset and cold row (-1: none), then per head the scores
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
    float* z = reinterpret_cast<float*>(lds + 2 * a.phys_stride) + h * a.phys_stride;

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

    // deferred staging: a missed row is read from the cold store and this
    // head's K (pass 1) or V (pass 2) slice is written into its slot.  Every
    // lane issues both a slot load and a cold load; the one it does not need
    // is pointed past its buffer, reads zero and moves no data, so the loads of
    // a batch stay branch-free and in flight together.
    const uint32_t cold_rec = srcs ? (uint32_t)a.cold_rows * row_bytes : 0u;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(srcs ? reinterpret_cast<const void*>(a.seg_cold[s]) : a.kv, cold_rec);
    auto load_batch = [&](int i0, uint32_t slice, uint4* v) {
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
            for (int u = 0; u < kUnroll; ++u) v[u] = buffer_load16(r, off[u] + slice);
            return;
        }
        uint4 w[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const bool cold = (uint32_t)c[u] < (uint32_t)a.cold_rows;
            v[u] = buffer_load16(r, (cold ? nrec : off[u]) + slice);
            w[u] = buffer_load16(rc, cold ? (uint32_t)c[u] * row_bytes + slice : cold_rec);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const bool cold = (uint32_t)c[u] < (uint32_t)a.cold_rows;
            v[u] = make_uint4(v[u].x | w[u].x, v[u].y | w[u].y, v[u].z | w[u].z, v[u].w | w[u].w);
            const u32x4 d = {v[u].x, v[u].y, v[u].z, v[u].w};
            // the slot write goes past the buffer (dropped) unless this row was missed
            __builtin_amdgcn_raw_buffer_store_b128(d, r, (cold && off[u] < nrec) ? off[u] + slice : nrec, 0, 0);
        }
    };

    float qv[8];
    {
        const float* qh = a.q + ((int64_t)s * a.heads + h) * DH + sub * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = qh[e];
    }
    const uint32_t k_off = (uint32_t)(h * DH * 2 + sub * 16);
    const uint32_t v_off = (uint32_t)((a.heads + h) * DH * 2 + sub * 16);

    // pass 1: z_i = scale * q . K_i
    for (int i0 = 0; i0 < n; i0 += kRpi * kUnroll) {
        uint4 kv[kUnroll];
        load_batch(i0, k_off, kv);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float f[8];
            unpack8<ET>(kv[u], f);
            float d = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) d += qv[e] * f[e];
#pragma unroll
            for (int o = 1; o < kLpr; o <<= 1) d += __shfl_xor(d, o, 64);
            const int i = i0 + u * kRpi + rg;
            if (sub == 0 && i < n) z[i] = a.scale * d;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // softmax over the n scores of this head
    float m = -INFINITY;
    for (int i = lane; i < n; i += 64) m = fmaxf(m, z[i]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float l = 0.0f;
    for (int i = lane; i < n; i += 64) {
        const float pz = expf(z[i] - m);
        z[i] = pz;
        l += pz;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o, 64);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // pass 2: sum_i p_i V_i, rows i = rg (mod kRpi) per lane group
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < n; i0 += kRpi * kUnroll) {
        uint4 vv[kUnroll];
        load_batch(i0, v_off, vv);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int i = i0 + u * kRpi + rg;
            const float pi = i < n ? z[i] : 0.0f;
            float f[8];
            unpack8<ET>(vv[u], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += pi * f[e];
        }
    }
#pragma unroll
    for (int o = kLpr; o < 64; o <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
    if (lane < kLpr) {
        const float inv_l = 1.0f / l;
#pragma unroll
        for (int e = 0; e < 8; ++e) out[lane * 8 + e] = acc[e] * inv_l;
    }
}

template <int DH>
hipError_t launch_dh(const AttendKVArgs& a, hipStream_t s) {
    const size_t lds = (size_t)(a.heads + 2) * a.phys_stride * sizeof(float);
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
