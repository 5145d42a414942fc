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
// Every wave works on its own 32-key tiles (tiles wave, wave + 4*grid, ...)
// and its own two LDS tile buffers, with wave-scope fences only -- no
// workgroup barriers.  The tile loop is software-pipelined: while the MFMA
// chain reads tile t from one buffer, each of its 16-byte read steps also
// writes one piece of tile t+1 (held in registers) into the other buffer and
// issues the load of the same piece of tile t+2, so a full tile of loads stays
// in flight under the MFMAs and no separate copy phase remains.  On gfx950 a
// wave's VALU instructions do not overlap its own f32 MFMAs (measured: each
// adds its issue time to the chain), so the loop keeps VALU work to the
// epilogue: integer-max ReLU, head weights, a permlane32 swap for the other
// half's heads, and the ensemble.  Tiles are taken per sequence, so the
// queries, weights and buffer resources stay fixed in the inner loop; with
// several sequences the waves split into one group per sequence, so each
// wave's pipeline and query set-up start once.  The
// grid is one 4-wave workgroup per CU (two for fp8 keys; fewer when the scan
// is short), which keeps every wave's share of tiles equal.
#include "lsa_internal.hpp"

namespace lsa {

namespace {
namespace score_k {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kSub = 32;           // keys per MFMA block (the B operand's columns)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Key storage formats: float, uint16_t (bf16 bits), uint8_t (fp8 E4M3), and
// the two OCP MX formats, which carry one E8M0 scale per 32 elements of a key.
struct mxfp4_tag {};    // E2M1 codes, two per byte, element 2i in the low nibble
struct mxint8_tag {};   // int8 codes with an implicit 2^-6
template <typename KT>
struct KeyFmt {
    static constexpr int kBits = 8 * (int)sizeof(KT);
    static constexpr bool kMX = false;
};
template <>
struct KeyFmt<mxfp4_tag> {
    static constexpr int kBits = 4;
    static constexpr bool kMX = true;
};
template <>
struct KeyFmt<mxint8_tag> {
    static constexpr int kBits = 8;
    static constexpr bool kMX = true;
};

// A wave tile is kNSub blocks of 32 keys: 32 fp32 keys (128 * DK bytes), 64
// keys of every narrower format.  The 64-key tile of the one-byte and fp4
// formats keeps a wave within 256 registers, so two waves share a SIMD (one's
// decode VALU runs under the other's MFMAs) and the score waves of the fused
// score+copy launch (five waves per workgroup) need no spills.
template <int DK, typename KT>
struct Cfg {
    static constexpr int kBits = KeyFmt<KT>::kBits;
    static constexpr bool kMX = KeyFmt<KT>::kMX;
    static constexpr int kNSub = kBits == 32 ? 1 : 2;
    static constexpr int kTile = kSub * kNSub;               // keys per wave tile
    static constexpr int kRowBytes = DK * kBits / 8;
    static constexpr int kLdsStride = kRowBytes + 16;
    static constexpr int kTileBytes = kTile * kRowBytes;
    static constexpr int kLoads = kTileBytes / (64 * 16);      // 16-byte loads per lane
    static constexpr int kHalf = DK / 2;                     // elements of a key row per lane
    static constexpr int kHalfBytes = kRowBytes / 2;
    static constexpr int kReads = kHalfBytes / 16;           // ds_read_b128 per lane and block
    static constexpr int kSteps = kNSub * kReads;            // read steps per tile
    static_assert(kTileBytes % (64 * 16) == 0, "tile must split into 16-byte loads");
    static_assert(kHalfBytes % 16 == 0, "half row must be 16-byte aligned");
    static_assert(kSteps == kLoads, "one tile load per read step");
};

// Exact split of an fp32 value into three bf16 parts, x = hi + mid + lo: hi
// keeps the top 8 significant bits, mid the next 8 of the remainder, and the
// remainder after that has at most 8 significant bits, so it is exact in bf16.
__device__ inline void split3(float x, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
    const uint32_t u = __float_as_uint(x);
    const float r1 = x - __uint_as_float(u & 0xFFFF0000u);
    const uint32_t u1 = __float_as_uint(r1);
    const float r2 = r1 - __uint_as_float(u1 & 0xFFFF0000u);
    hi = (uint16_t)(u >> 16);
    mid = (uint16_t)(u1 >> 16);
    lo = (uint16_t)(__float_as_uint(r2) >> 16);
}

__device__ inline bf16x8 as_bf16x8(const uint4& u) {
    return __builtin_bit_cast(bf16x8, u);
}

// max(x, 0) for finite x in one integer max: a set sign bit makes the pattern
// a negative int32 (-0 becomes +0)
__device__ inline float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Buffer resource of one tile: base at the tile, records = bytes of the
// sequence's valid keys from there on, so every read of the tile stays inside
// the sequence and rows >= n_valid read as zero.  A sequence has
// ceil(n_valid / keys per tile) tiles, so a tile's first row is valid: tile_off < seq_bytes.
__device__ inline __amdgpu_buffer_rsrc_t tile_rsrc(const char* seq, uint32_t seq_bytes, uint32_t tile_off) {
    return make_rsrc(seq + tile_off, seq_bytes - tile_off);
}

__device__ inline void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The query block as the MFMA's A operand: for fp32 keys the fp32 values for
// v_mfma_f32_32x32x2f32; for bf16 and fp8 keys each value split exactly into
// three bf16 parts (hi, mid, lo) for v_mfma_f32_32x32x16_bf16, so every product
// with a key (exact in bf16) is the exact product with the fp32 query.
template <int DK, bool F32>
struct QOperand;
template <int DK>
struct QOperand<DK, true> {
    float v[DK / 2];
};
template <int DK>
struct QOperand<DK, false> {
    bf16x8 hi[DK / 16], mid[DK / 16], lo[DK / 16];
};

// Two fp8 (OCP E4M3) codes -> their exact bf16 values, packed, in one
// instruction (scale 1): every E4M3 value, subnormals included, is a bf16
// normal or zero, so the conversion does not round.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
template <bool HIGH_PAIR>
__device__ inline uint32_t fp8x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HIGH_PAIR));
}

// Two fp4 (E2M1) codes of byte SEL of w, times the scale, as packed bf16: exact
// while the scaled values are bf16 normals or zero.
template <int SEL>
__device__ inline uint32_t fp4x2_to_bf16x2(uint32_t w, float scale) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, SEL));
}

// Two int8 codes (bytes 2K and 2K+1 of w) times sf, as packed bf16.  A code c
// is taken as the unsigned byte of c + 128 (the sign bit flipped), so
// (c + 128) * sf - 128 * sf = c * sf in one fused multiply-add with no
// rounding (sf is a power of two); the product has at most 8 significant bits
// and so is exact in bf16.
template <int K>
__device__ inline uint32_t i8x2_to_bf16x2(uint32_t w, float sf, float off) {
    const uint32_t x = w ^ 0x80808080u;
    const float f0 = fmaf((float)((x >> (16 * K)) & 0xFFu), sf, off);
    const float f1 = fmaf((float)((x >> (16 * K + 8)) & 0xFFu), sf, off);
    return __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
}

// The E8M0 scale bytes of one key (DK/32 of them), as the low bytes of a word.
template <int DK>
__device__ inline uint32_t load_scales(__amdgpu_buffer_rsrc_t r, int key) {
    const uint32_t off = (uint32_t)key * (DK / 32);
    if constexpr (DK == 128) return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    else if constexpr (DK == 64) return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
    else return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

// 2^(s-127) for an E8M0 byte s >= 1
__device__ inline float e8m0(uint32_t s) { return __uint_as_float(s << 23); }

// With HIST, every stored score that the select would count (a valid entry;
// in threshold mode one above t_f) is also added to the LDS histogram `hist`
// of 11-bit key tops -- the select's first pass -- so a caller can skip it.
// Candidate lists written by the score launch (the lookahead schedule's
// select): per sub-block of kCandSub consecutive entries, in index order, the
// entries of bin >= guess[seq] that pass the threshold, with their order keys.
// The workgroups split evenly over the sequences (the grid is a multiple of the
// batch) and each takes whole 1024-entry blocks; its waves take one quarter of
// them each, a run of consecutive tiles, so each wave writes the lists of its
// own sub-blocks as it goes.
constexpr int kCandSub = kSelColBlk / kWaves;   // 256
struct CandOut {
    int32_t* idx;            // [n_seg][nsb][kCandSub]
    uint32_t* key;           // [n_seg][nsb][kCandSub]
    int32_t* count;          // [n_seg][nsb]
    const int32_t* guess;    // [n_seg]
    int32_t nblk;            // 1024-entry blocks per sequence
    int32_t thr;             // threshold mode: an entry also needs score > t_f
    float t_f;
};

// The 1024-entry blocks of workgroup bx of gx: returns the first, *seq the
// sequence and *n their number (0 when the sequence has fewer blocks than
// workgroups).
__device__ inline int cand_blocks(const ScoreArgs& a, const int bx, const int gx, const int nblk, int* seq, int* n) {
    const int G = gx / a.batch;
    *seq = bx / G;
    const int j = bx - *seq * G;
    const int per = (nblk + G - 1) / G;
    const int first = j * per;
    const int last = first + per < nblk ? first + per : nblk;
    *n = last > first ? last - first : 0;
    return first;
}

// A 16-byte key load; NT: with the non-temporal cache policy.
template <bool NT>
__device__ __forceinline__ uint4 key_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (NT) return buffer_load16_nt(r, off);
    else return buffer_load16(r, off);
}

// NT: the keys are loaded with the non-temporal policy (a pass that streams
// them once); without it they may stay in the caches for the next step's pass.
template <int DK, typename KT, bool HIST = false, bool CAND = false, bool NT = false>
__device__ __forceinline__ void fm_score_body(const ScoreArgs& a, const int bx, const int gx, uint32_t* hist = nullptr,
                                              const int hist_mode = 0, const float hist_t_f = 0.0f,
                                              const CandOut* co = nullptr) {
    using C = Cfg<DK, KT>;
    constexpr bool kF32 = C::kBits == 32;
    constexpr int kSteps = C::kSteps;
    constexpr int kTile = C::kTile;
    static_assert(1024 % C::kRowBytes == 0, "a 64-lane load covers whole rows");
    constexpr int kBuf = kTile * C::kLdsStride;
    constexpr int kLoadStride = (1024 / C::kRowBytes) * C::kLdsStride;   // LDS bytes per 64-lane load
    constexpr int kSubBytes = kSub * C::kLdsStride;                     // LDS bytes per 32-key block
    __shared__ __attribute__((aligned(16))) char lds[kWaves][2][kBuf];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: keeps tile state in SGPRs
    const int col = lane & 31;      // key within a 32-key block (B/D column); query row for A
    const int half = lane >> 5;     // which half of dk this lane feeds
    int total = a.tile_start[a.batch];
    int stride = gx * kWaves;
    int t = bx * kWaves + wave;
    // CAND: this wave's sequence, first sub-block and sub-block count, the list
    // bin and key threshold, and the running list of the current sub-block
    int c_seq = 0, c_sb = 0, c_nsb = 0, c_guess = 0, c_run = 0, c_cur = 0;
    uint32_t c_tkey = 0;
    if constexpr (CAND) {
        int nb;
        const int b0 = cand_blocks(a, bx, gx, co->nblk, &c_seq, &nb);
        c_guess = co->guess[c_seq];
        c_tkey = co->thr ? order_key(co->t_f) : 0u;
        // threshold mode lists every passing entry: the guess goes no higher
        // than the threshold's own bin
        if (co->thr && (int)(c_tkey >> kSelShift) < c_guess) c_guess = (int)(c_tkey >> kSelShift);
        constexpr int kTpb = kSelColBlk / kTile;    // tiles per block
        const int tw = nb * (kTpb / kWaves);        // tiles per wave: nb sub-blocks
        const int ts = a.tile_start[c_seq], te = a.tile_start[c_seq + 1];
        const int lo_w = ts + b0 * kTpb + wave * tw;
        t = lo_w < te ? lo_w : te;
        total = lo_w + tw < te ? lo_w + tw : te;
        stride = 1;
        c_sb = b0 * kWaves + wave * nb;
        c_nsb = nb;
        c_cur = c_sb;
    } else if (a.batch > 1 && stride >= a.batch) {
        // several sequences: the waves split into one equal group per sequence, so
        // a wave's tiles all lie in one sequence and its load pipeline (and query
        // set-up) starts once, not once per sequence; the waves left over idle
        const int per = stride / a.batch;
        const int bq = t / per;
        if (bq >= a.batch) return;
        t = a.tile_start[bq] + (t - bq * per);
        total = a.tile_start[bq + 1];
        stride = per;
    }

    const char* kbase = static_cast<const char*>(a.keys);
    const __amdgpu_buffer_rsrc_t zero_r = make_rsrc(kbase, 0u);     // every read returns zero
    // LDS byte offset of this lane's 16-byte piece of load i: woff + i * kLoadStride
    const int woff = (lane * 16 / C::kRowBytes) * C::kLdsStride + (lane * 16) % C::kRowBytes;
    const int roff = col * C::kLdsStride + half * C::kHalfBytes;
    // byte offset of load i of a tile: vo[i / 4] + (i % 4) * 1024 (the constant goes to the
    // instruction's offset field)
    uint32_t vo[(kSteps + 3) / 4];
#pragma unroll
    for (int k = 0; k < (kSteps + 3) / 4; ++k) vo[k] = (uint32_t)lane * 16u + (uint32_t)k * 4096u;
    char* const my0 = lds[wave][0];

    int b = 0;
    while (t < total) {
        // one run of this wave's tiles that belong to sequence b
        while (t >= a.tile_start[b + 1]) ++b;
        // a run ends at the sequence's last tile, or at the workgroup's (CAND)
        const int lo = a.tile_start[b], hi = a.tile_start[b + 1] < total ? a.tile_start[b + 1] : total;
        const int nv = a.n_valid[b];
        const char* const seq = kbase + (int64_t)b * a.n_keys * C::kRowBytes;
        const uint32_t seq_bytes = (uint32_t)nv * (uint32_t)C::kRowBytes;
        // scores of keys >= n_valid, and every store of lane half 1 (offset 2^31), are dropped
        const __amdgpu_buffer_rsrc_t so = make_rsrc(a.scores + (int64_t)b * a.n_keys, (uint32_t)nv * 4u);
        // MX keys: the scale words of this lane's key in each 32-key block of tile t
        // (sc_cur) and of tile t + stride (sc_nxt); keys >= n_valid read zero
        __amdgpu_buffer_rsrc_t srs = zero_r;
        uint32_t sc_cur[C::kNSub], sc_nxt[C::kNSub];
        if constexpr (C::kMX) {
            srs = make_rsrc(a.scales + (int64_t)b * a.n_keys * (DK / 32), (uint32_t)nv * (uint32_t)(DK / 32));
#pragma unroll
            for (int j = 0; j < C::kNSub; ++j) {
                sc_cur[j] = load_scales<DK>(srs, (t - lo) * kTile + j * kSub + col);
                sc_nxt[j] = load_scales<DK>(srs, (t + stride - lo) * kTile + j * kSub + col);
            }
        }

        // prologue: tile t into LDS buffer 0, tile t + stride in flight in registers; the
        // queries and weights load behind the first tile
        uint4 pre[kSteps];
        const __amdgpu_buffer_rsrc_t r0 = tile_rsrc(seq, seq_bytes, (uint32_t)(t - lo) * (uint32_t)C::kTileBytes);
#pragma unroll
        for (int i = 0; i < kSteps; ++i) pre[i] = key_load16<NT>(r0, vo[i >> 2] + (uint32_t)(i & 3) * 1024u);
        __builtin_amdgcn_sched_barrier(0);
        // A operand: query row `col` (indexer col/8, head col%8), elements half*DK/2 + e
        QOperand<DK, kF32> qa;
        {
            const int g = col >> 3, hd = col & 7;
            const bool qv = g < a.n_idx && hd < a.heads;
            const float* qrow = a.q + (((int64_t)b * a.n_idx + (qv ? g : 0)) * a.heads + (qv ? hd : 0)) * DK + half * C::kHalf;
            if constexpr (kF32) {
#pragma unroll
                for (int e = 0; e < C::kHalf; e += 4) {
                    const f32x4 v = qv ? *reinterpret_cast<const f32x4*>(qrow + e) : f32x4{0.f, 0.f, 0.f, 0.f};
                    qa.v[e] = v[0];
                    qa.v[e + 1] = v[1];
                    qa.v[e + 2] = v[2];
                    qa.v[e + 3] = v[3];
                }
            } else {
#pragma unroll
                for (int blk = 0; blk < C::kHalf / 8; ++blk) {
                    uint32_t wh[4], wm[4], wl[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const f32x2 v = qv ? *reinterpret_cast<const f32x2*>(qrow + 8 * blk + 2 * p) : f32x2{0.f, 0.f};
                        uint16_t h0, m0, l0, h1, m1, l1;
                        split3(v[0], h0, m0, l0);
                        split3(v[1], h1, m1, l1);
                        wh[p] = (uint32_t)h0 | ((uint32_t)h1 << 16);
                        wm[p] = (uint32_t)m0 | ((uint32_t)m1 << 16);
                        wl[p] = (uint32_t)l0 | ((uint32_t)l1 << 16);
                    }
                    qa.hi[blk] = as_bf16x8(make_uint4(wh[0], wh[1], wh[2], wh[3]));
                    qa.mid[blk] = as_bf16x8(make_uint4(wm[0], wm[1], wm[2], wm[3]));
                    qa.lo[blk] = as_bf16x8(make_uint4(wl[0], wl[1], wl[2], wl[3]));
                }
            }
        }
        // epilogue weights: accumulator r is query row 8*(r/4) + 4*half + r%4
        float wr[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int gi = r >> 2, hi_ = 4 * half + (r & 3);
            wr[r] = (gi < a.n_idx && hi_ < a.heads) ? a.w[((int64_t)b * a.n_idx + gi) * a.heads + hi_] : 0.0f;
        }

        __builtin_amdgcn_sched_barrier(0);
        {
#pragma unroll
            for (int i = 0; i < kSteps; ++i) *reinterpret_cast<uint4*>(my0 + woff + i * kLoadStride) = pre[i];
            const int tn = t + stride;
            const __amdgpu_buffer_rsrc_t rn =
                tn < hi ? tile_rsrc(seq, seq_bytes, (uint32_t)(tn - lo) * (uint32_t)C::kTileBytes) : zero_r;
#pragma unroll
            for (int i = 0; i < kSteps; ++i) pre[i] = key_load16<NT>(rn, vo[i >> 2] + (uint32_t)(i & 3) * 1024u);
        }
        wave_sync();

        int cur = 0;
        for (; t < hi; t += stride) {
            // LDS buffer `cur` holds tile t; `pre` holds tile t + stride (in flight).  Each
            // MFMA step also moves one piece of `pre` into the other buffer and refills it
            // with tile t + 2*stride, so loads stay in flight under the MFMA chain.
            const int t2 = t + 2 * stride;
            const __amdgpu_buffer_rsrc_t r2 =
                t2 < hi ? tile_rsrc(seq, seq_bytes, (uint32_t)(t2 - lo) * (uint32_t)C::kTileBytes) : zero_r;
            const char* rd = my0 + cur * kBuf + roff;
            char* wrb = my0 + (cur ^ 1) * kBuf + woff;
            uint32_t sc_n2[C::kNSub];
            if constexpr (C::kMX) {
#pragma unroll
                for (int j = 0; j < C::kNSub; ++j) sc_n2[j] = load_scales<DK>(srs, (t2 - lo) * kTile + j * kSub + col);
            }

            f32x16 acc[C::kNSub];
#pragma unroll
            for (int j = 0; j < C::kNSub; ++j) acc[j] = f32x16{};
            uint4 u = *reinterpret_cast<const uint4*>(rd);
#pragma unroll
            for (int s = 0; s < kSteps; ++s) {
                // step s reads 16 bytes of key block j = s / kReads at read rr = s % kReads
                const int j = s / C::kReads, rr = s % C::kReads;
                const int sn = s + 1;
                const uint4 un = sn < kSteps
                    ? *reinterpret_cast<const uint4*>(rd + (sn / C::kReads) * kSubBytes + (sn % C::kReads) * 16)
                    : u;
                *reinterpret_cast<uint4*>(wrb + s * kLoadStride) = pre[s];
                pre[s] = key_load16<NT>(r2, vo[s >> 2] + (uint32_t)(s & 3) * 1024u);
                if constexpr (kF32) {
                    const float kb[4] = {__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                                         __uint_as_float(u.w)};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(qa.v[rr * 4 + e], kb[e], acc[j], 0, 0, 0);
                } else if constexpr (C::kBits == 16) {
                    const bf16x8 kb = as_bf16x8(u);
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa.hi[rr], kb, acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa.mid[rr], kb, acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa.lo[rr], kb, acc[j], 0, 0, 0);
                } else if constexpr (__is_same(KT, mxfp4_tag)) {
                    // 32 fp4 codes of one MX block (index half*DK/64 + rr): elements of
                    // blocks 4*rr .. 4*rr + 3
                    const float sf = e8m0((sc_cur[j] >> (8 * (half * (DK / 64) + rr))) & 0xFFu);
                    const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const bf16x8 km = as_bf16x8(make_uint4(fp4x2_to_bf16x2<0>(uw[m], sf), fp4x2_to_bf16x2<1>(uw[m], sf),
                                                               fp4x2_to_bf16x2<2>(uw[m], sf), fp4x2_to_bf16x2<3>(uw[m], sf)));
                        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa.hi[4 * rr + m], km, acc[j], 0, 0, 0);
                        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa.mid[4 * rr + m], km, acc[j], 0, 0, 0);
                        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa.lo[4 * rr + m], km, acc[j], 0, 0, 0);
                    }
                } else if constexpr (__is_same(KT, mxint8_tag)) {
                    // 16 int8 codes, half of MX block (half*DK/2 + 16*rr) / 32: elements of
                    // blocks 2*rr and 2*rr + 1
                    const float sf = e8m0((sc_cur[j] >> (8 * ((half * (DK / 2) + 16 * rr) / 32))) & 0xFFu) * (1.0f / 64.0f);
                    const float off = -128.0f * sf;
                    const bf16x8 k0 = as_bf16x8(make_uint4(i8x2_to_bf16x2<0>(u.x, sf, off), i8x2_to_bf16x2<1>(u.x, sf, off),
                                                           i8x2_to_bf16x2<0>(u.y, sf, off), i8x2_to_bf16x2<1>(u.y, sf, off)));
                    const bf16x8 k1 = as_bf16x8(make_uint4(i8x2_to_bf16x2<0>(u.z, sf, off), i8x2_to_bf16x2<1>(u.z, sf, off),
                                                           i8x2_to_bf16x2<0>(u.w, sf, off), i8x2_to_bf16x2<1>(u.w, sf, off)));
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa.hi[2 * rr], k0, acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa.mid[2 * rr], k0, acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa.lo[2 * rr], k0, acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa.hi[2 * rr + 1], k1, acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa.mid[2 * rr + 1], k1, acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa.lo[2 * rr + 1], k1, acc[j], 0, 0, 0);
                } else {
                    // 16 fp8 codes: elements of blocks 2*rr and 2*rr + 1
                    const bf16x8 k0 = as_bf16x8(make_uint4(fp8x2_to_bf16x2<false>(u.x), fp8x2_to_bf16x2<true>(u.x),
                                                           fp8x2_to_bf16x2<false>(u.y), fp8x2_to_bf16x2<true>(u.y)));
                    const bf16x8 k1 = as_bf16x8(make_uint4(fp8x2_to_bf16x2<false>(u.z), fp8x2_to_bf16x2<true>(u.z),
                                                           fp8x2_to_bf16x2<false>(u.w), fp8x2_to_bf16x2<true>(u.w)));
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa.hi[2 * rr], k0, acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa.mid[2 * rr], k0, acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa.lo[2 * rr], k0, acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa.hi[2 * rr + 1], k1, acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa.mid[2 * rr + 1], k1, acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa.lo[2 * rr + 1], k1, acc[j], 0, 0, 0);
                }
                u = un;
                __builtin_amdgcn_sched_barrier(0);
            }
            // the other buffer is complete and this one's reads are done
            wave_sync();

#pragma unroll
            for (int j = 0; j < C::kNSub; ++j) {
                // epilogue: per indexer, this lane's 4 heads; then the other half's 4 heads
                float sv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int gi = 0; gi < 4; ++gi) {
                    if (gi >= a.n_idx) break;   // uniform
                    float v = 0.0f;
#pragma unroll
                    for (int c = 0; c < 4; ++c) v += wr[4 * gi + c] * relu(acc[j][4 * gi + c]);
                    // lanes 0..31 receive lane l+32's value in r[1]
                    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
                    sv[gi] = (v + __uint_as_float(r[1])) + 0.0f;
                }
                float e;
                if (a.ensemble == LSA_ENSEMBLE_MAX) {
                    e = sv[0];
                    if (a.n_idx > 1) e = fmaxf(e, sv[1]);
                    if (a.n_idx > 2) e = fmaxf(e, sv[2]);
                    if (a.n_idx > 3) e = fmaxf(e, sv[3]);
                } else {
                    // mean ensemble: the float indexer scores are added in
                    // double, in indexer order (exact unless their exponents
                    // lie more than 27 apart), rounded once to float, and
                    // divided once by n_idx in IEEE single precision
                    double sum = (double)sv[0];
                    if (a.n_idx > 1) sum += (double)sv[1];
                    if (a.n_idx > 2) sum += (double)sv[2];
                    if (a.n_idx > 3) sum += (double)sv[3];
                    e = (float)sum / (float)a.n_idx;
                }
                const int key = (t - lo) * kTile + j * kSub + col;
                const uint32_t off = half ? 0x80000000u : (uint32_t)key * 4u;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(e + 0.0f), so, off, 0, 0);
                if (HIST) {
                    const float ev = e + 0.0f;
                    if (half == 0 && key < nv && (hist_mode != LSA_SELECT_THRESHOLD || ev > hist_t_f))
                        atomicAdd(&hist[order_key(ev) >> kSelShift], 1u);
                }
                if (CAND) {
                    // the 32 keys of this block lie in one sub-block; a new one
                    // closes the list of the last (its count written by lane 0)
                    const int sb = key / kCandSub;   // uniform over the lanes that matter
                    const int sbu = __builtin_amdgcn_readfirstlane(sb);
                    if (sbu != c_cur) {
                        if (lane == 0) co->count[(int64_t)c_seq * (co->nblk * kWaves) + c_cur] = c_run;
                        c_cur = sbu;
                        c_run = 0;
                    }
                    const uint32_t ok = order_key(e);
                    const bool cand = half == 0 && key < nv && (int)(ok >> kSelShift) >= c_guess && (!co->thr || ok > c_tkey);
                    const uint64_t bal = __ballot(cand);
                    if (cand) {
                        const int pos = c_run + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
                        const int64_t at = ((int64_t)c_seq * (co->nblk * kWaves) + sbu) * kCandSub + pos;
                        co->idx[at] = key;
                        co->key[at] = ok;
                    }
                    c_run += __popcll(bal);
                }
            }
            cur ^= 1;
            if constexpr (C::kMX) {
#pragma unroll
                for (int j = 0; j < C::kNSub; ++j) {
                    sc_cur[j] = sc_nxt[j];
                    sc_nxt[j] = sc_n2[j];
                }
            }
        }
    }
    if constexpr (CAND) {
        // the current sub-block's count, and zero for the wave's sub-blocks past
        // the sequence's valid entries (they had no tile)
        if (lane == 0) {
            for (int sb = c_cur; sb < c_sb + c_nsb; ++sb)
                co->count[(int64_t)c_seq * (co->nblk * kWaves) + sb] = sb == c_cur ? c_run : 0;
        }
    }
}

// The end of a workgroup's score waves that count their scores into s_hist
// (HIST): each counts itself finished on s_done (zero on entry) after its LDS
// adds, and the last one adds the non-zero bins to its sequence's histogram
// (with several sequences the grid is a multiple of the batch and every wave
// of a workgroup scores one sequence).
__device__ inline void score_hist_flush(const ScoreArgs& a, const uint32_t* s_hist, int* s_done, uint32_t* hist) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    const int lane = threadIdx.x & 63;
    int prev = 0;
    if (lane == 0) prev = atomicAdd(s_done, 1);
    prev = __shfl(prev, 0, 64);
    if (prev != kWaves - 1) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const int seg = a.batch > 1 ? (int)(blockIdx.x / (gridDim.x / a.batch)) : 0;
    uint32_t* gh = hist + (size_t)seg * kSelBins;
    for (int i = lane; i < kSelBins; i += 64) {
        const uint32_t c = s_hist[i];
        if (c) atomicAdd(&gh[i], c);
    }
}

// workgroups per CU: two for the one-byte and fp4 formats (registers and LDS
// fit two), else one
template <typename KT>
constexpr int kWgPerCu = KeyFmt<KT>::kBits <= 8 ? 2 : 1;

template <int DK, typename KT, bool NT>
__global__ __launch_bounds__(kThreads, kWgPerCu<KT>) void fm_score_kernel(const ScoreArgs a) {
    fm_score_body<DK, KT, false, false, NT>(a, blockIdx.x, gridDim.x);
}

// fm_score that also writes the select's candidate lists (one workgroup per
// CU, as the lists' schedule assumes)
template <int DK, typename KT, bool NT>
__global__ __launch_bounds__(kThreads, 1) void fm_score_lists_kernel(const ScoreArgs a, const ScoreHistArgs h) {
    const CandOut co{h.blk_idx, h.blk_key, h.blk_count, h.guess, h.nblk, h.mode == LSA_SELECT_THRESHOLD ? 1 : 0, h.t_f};
    fm_score_body<DK, KT, false, true, NT>(a, blockIdx.x, gridDim.x, nullptr, h.mode, h.t_f, &co);
}

template <int DK, typename KT>
hipError_t launch_lists_t(const ScoreArgs& a, const ScoreHistArgs& h, int n_cu, hipStream_t s, bool stream_keys) {
    const int grid = score_lists_grid(a, n_cu);
    if (grid < a.batch || grid < 1) return hipErrorInvalidValue;
    if (stream_keys)
        hipLaunchKernelGGL((fm_score_lists_kernel<DK, KT, true>), dim3(grid), dim3(kThreads), 0, s, a, h);
    else
        hipLaunchKernelGGL((fm_score_lists_kernel<DK, KT, false>), dim3(grid), dim3(kThreads), 0, s, a, h);
    return hipGetLastError();
}

template <int DK, typename KT>
hipError_t launch_t(const ScoreArgs& a, int n_cu, hipStream_t s, bool stream_keys) {
    const int total = a.tile_start[a.batch];
    if (total == 0) return hipSuccess;
    int grid = (total + kWaves - 1) / kWaves;
    if (grid > n_cu * kWgPerCu<KT>) grid = n_cu * kWgPerCu<KT>;
    if (stream_keys)
        hipLaunchKernelGGL((fm_score_kernel<DK, KT, true>), dim3(grid), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((fm_score_kernel<DK, KT, false>), dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace score_k
#ifndef LSA_BODIES_ONLY
using namespace score_k;
#endif
}  // namespace

#ifndef LSA_BODIES_ONLY
int score_lists_grid(const ScoreArgs& a, int n_cu) {
    int grid = (a.tile_start[a.batch] + score_k::kWaves - 1) / score_k::kWaves;
    if (grid > n_cu) grid = n_cu;
    if (grid < 1) grid = 1;
    if (a.batch > 1) grid -= grid % a.batch;
    return grid;
}

hipError_t launch_fm_score_lists(const ScoreArgs& a, const ScoreHistArgs& h, int key_dtype, int dk, int n_cu,
                                 hipStream_t s, bool stream_keys) {
    if (key_dtype == LSA_F32) {
        if (dk == 32) return launch_lists_t<32, float>(a, h, n_cu, s, stream_keys);
        if (dk == 64) return launch_lists_t<64, float>(a, h, n_cu, s, stream_keys);
        if (dk == 128) return launch_lists_t<128, float>(a, h, n_cu, s, stream_keys);
    } else if (key_dtype == LSA_BF16) {
        if (dk == 32) return launch_lists_t<32, uint16_t>(a, h, n_cu, s, stream_keys);
        if (dk == 64) return launch_lists_t<64, uint16_t>(a, h, n_cu, s, stream_keys);
        if (dk == 128) return launch_lists_t<128, uint16_t>(a, h, n_cu, s, stream_keys);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fm_score(const ScoreArgs& a, int key_dtype, int dk, int n_cu, hipStream_t s, bool stream_keys) {
    if (key_dtype == LSA_F32) {
        if (dk == 32) return launch_t<32, float>(a, n_cu, s, stream_keys);
        if (dk == 64) return launch_t<64, float>(a, n_cu, s, stream_keys);
        if (dk == 128) return launch_t<128, float>(a, n_cu, s, stream_keys);
    } else if (key_dtype == LSA_BF16) {
        if (dk == 32) return launch_t<32, uint16_t>(a, n_cu, s, stream_keys);
        if (dk == 64) return launch_t<64, uint16_t>(a, n_cu, s, stream_keys);
        if (dk == 128) return launch_t<128, uint16_t>(a, n_cu, s, stream_keys);
    } else if (key_dtype == LSA_FP8_E4M3) {
        if (dk == 32) return launch_t<32, uint8_t>(a, n_cu, s, stream_keys);
        if (dk == 64) return launch_t<64, uint8_t>(a, n_cu, s, stream_keys);
        if (dk == 128) return launch_t<128, uint8_t>(a, n_cu, s, stream_keys);
    } else if (key_dtype == LSA_MXFP4) {
        if (dk == 64) return launch_t<64, mxfp4_tag>(a, n_cu, s, stream_keys);
        if (dk == 128) return launch_t<128, mxfp4_tag>(a, n_cu, s, stream_keys);
    } else if (key_dtype == LSA_MXINT8) {
        if (dk == 32) return launch_t<32, mxint8_tag>(a, n_cu, s, stream_keys);
        if (dk == 64) return launch_t<64, mxint8_tag>(a, n_cu, s, stream_keys);
        if (dk == 128) return launch_t<128, mxint8_tag>(a, n_cu, s, stream_keys);
    }
    return hipErrorInvalidValue;
}

#endif  // LSA_BODIES_ONLY

}  // namespace lsa
