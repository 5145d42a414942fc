// liblsa host side: the C ABI of include/lsa.h -- argument validation, the
// page's closed forms and error conditions, context workspace, slot pools,
// per-kernel timing, and the decode-step composition.  All arithmetic of the
// step runs in the kernels of fm_score.hip, fm_select.hip, kv_stage.hip and
// lsa_attend.hip.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "lsa_internal.hpp"

using namespace lsa;

namespace {

thread_local std::string g_err;

lsa_status fail(lsa_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

#define HIPTRY(call)                                                                     \
    do {                                                                                 \
        hipError_t e_ = (call);                                                          \
        if (e_ != hipSuccess) return fail(LSA_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
    } while (0)

int elem_bytes(lsa_dtype d) { return d == LSA_F32 ? 4 : d == LSA_FP8_E4M3 ? 1 : 2; }
bool row_dtype_ok(lsa_dtype d) { return d == LSA_F32 || d == LSA_BF16 || d == LSA_F16; }

int n_cu_current() {
    static int cache[128] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 128) return 256;
    if (!cache[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ------------------------------------------------------ static scratch
// The scratch of lsa_decode_step_noalloc: one static device array, of which
// every GPU the library runs on holds its own copy (at its own address) until
// the process ends.  Host code never passes `scratch` itself to a kernel (on
// the host the name is only a stand-in); it uses the device address that
// hipGetSymbolAddress returns, looked up once per device with that device
// current and kept in g_scratch_addr.
static __device__ __align__(256) char scratch[LSA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 128;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch` (device `dev` must
// be current).  NULL with an error when the lookup fails.
lsa_status scratch_address(int dev, void** out) {
    *out = nullptr;
    if (dev < 0 || dev >= kMaxDevices) return LSA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return LSA_ERR_HIP;
        }
        g_scratch_addr[dev] = ptr;
    }
    *out = g_scratch_addr[dev];
    return LSA_OK;
}

// Clears n words (a plain fill kernel, so a captured step records no memset).
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

}  // namespace

// ------------------------------------------------------------------ context
struct lsa_ctx {
    int device = 0;
    void* scratch = nullptr;    // this device's copy of the static scratch (device address)
    lsa_status scratch_status = LSA_OK;
    int n_cu = 256;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    void* zero = nullptr;       // select histogram: zero between calls
    size_t zero_bytes = 0;
    bool timing = false;
    // the step calls load the indexer keys non-temporally (lsa_ctx_set_key_policy)
    bool stream_keys = false;
    struct Pending {
        int kind;
        hipEvent_t a, b;
    };
    std::vector<Pending> pending;
    std::vector<hipEvent_t> spare;
    // lookahead schedule: which of the two row-list buffers holds the rows of
    // the coming step
    int la_cur = 0;
    // whether the missed rows of buffer la_cur have been copied into their
    // slots (by an attention of the window the last prediction serves)
    bool la_fetched = false;
    // KVSwap stage: every pool's stage descriptor goes to the device in one copy
    // and the stage of all pools runs as one launch.  Two (pinned host, device)
    // table pairs alternate; a pair is reused only once the stage launch that
    // read it two calls back has completed
    StageLayer* kv_layers_dev[2] = {nullptr, nullptr};
    StageLayer* kv_layers_host[2] = {nullptr, nullptr};
    hipEvent_t kv_layers_done[2] = {nullptr, nullptr};
    int kv_layers_cap = 0;
    int kv_layers_next = 0;
    // lookahead schedule: per sequence, the select bin from which the next
    // step's score launch lists candidates (written by each step's final
    // selection; a wrong guess only costs the exact fallback)
    int32_t* sel_guess = nullptr;   // device [LSA_MAX_BATCH]
    // counters of the one-launch attention (AttendArgs::sync), in the same
    // allocation; zero between launches
    uint32_t* att_sync = nullptr;
};

namespace {

// The table pair the next KVSwap stage uses (n descriptors), grown on first
// use.  The device table is written by a stream-ordered copy from the pinned
// host table, so every step's stage reads its own descriptors; the host waits
// until the stage that read the pair two calls back has completed, so neither
// table is overwritten while a launch may still read it (also across streams).
lsa_status kv_layer_buffer(lsa_ctx* c, int n, StageLayer** host, StageLayer** dev) {
    if (n > c->kv_layers_cap) {
        HIPTRY(hipDeviceSynchronize());
        for (int i = 0; i < 2; ++i) {
            if (c->kv_layers_dev[i]) (void)hipFree(c->kv_layers_dev[i]);
            if (c->kv_layers_host[i]) (void)hipHostFree(c->kv_layers_host[i]);
            c->kv_layers_dev[i] = nullptr;
            c->kv_layers_host[i] = nullptr;
        }
        c->kv_layers_cap = 0;
        const size_t bytes = (size_t)n * sizeof(StageLayer);
        for (int i = 0; i < 2; ++i) {
            if (hipMalloc(reinterpret_cast<void**>(&c->kv_layers_dev[i]), bytes) != hipSuccess)
                return fail(LSA_ERR_NO_MEMORY, "KVSwap stage table: hipMalloc of %zu bytes failed", bytes);
            if (hipHostMalloc(reinterpret_cast<void**>(&c->kv_layers_host[i]), bytes, hipHostMallocDefault) != hipSuccess)
                return fail(LSA_ERR_NO_MEMORY, "KVSwap stage table: hipHostMalloc of %zu bytes failed", bytes);
            if (!c->kv_layers_done[i]) HIPTRY(hipEventCreateWithFlags(&c->kv_layers_done[i], hipEventDisableTiming));
            HIPTRY(hipEventRecord(c->kv_layers_done[i], nullptr));
        }
        c->kv_layers_cap = n;
    }
    const int slot = c->kv_layers_next;
    HIPTRY(hipEventSynchronize(c->kv_layers_done[slot]));
    *host = c->kv_layers_host[slot];
    *dev = c->kv_layers_dev[slot];
    return LSA_OK;
}

lsa_status ws_ensure(lsa_ctx* c, size_t bytes) {
    if (bytes <= c->ws_bytes) return LSA_OK;
    size_t want = align_up(bytes, (size_t)1 << 20);
    if (c->ws) {
        HIPTRY(hipDeviceSynchronize());
        HIPTRY(hipFree(c->ws));
        c->ws = nullptr;
        c->ws_bytes = 0;
    }
    if (hipMalloc(&c->ws, want) != hipSuccess) {
        (void)hipGetLastError();
        c->ws = nullptr;
        return fail(LSA_ERR_NO_MEMORY, "workspace allocation of %zu bytes failed", want);
    }
    c->ws_bytes = want;
    return LSA_OK;
}

// The zero region is left zeroed by the kernels that use it; a new or grown
// region is zeroed here.
lsa_status zero_ensure(lsa_ctx* c, size_t bytes) {
    if (bytes <= c->zero_bytes) return LSA_OK;
    size_t want = align_up(bytes, (size_t)1 << 16);
    if (c->zero) {
        HIPTRY(hipDeviceSynchronize());
        HIPTRY(hipFree(c->zero));
        c->zero = nullptr;
        c->zero_bytes = 0;
    }
    if (hipMalloc(&c->zero, want) != hipSuccess) {
        (void)hipGetLastError();
        c->zero = nullptr;
        return fail(LSA_ERR_NO_MEMORY, "select workspace allocation of %zu bytes failed", want);
    }
    HIPTRY(hipMemset(c->zero, 0, want));
    HIPTRY(hipDeviceSynchronize());
    c->zero_bytes = want;
    return LSA_OK;
}

hipEvent_t ev_take(lsa_ctx* c) {
    if (!c->spare.empty()) {
        hipEvent_t e = c->spare.back();
        c->spare.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Records an event before construction and one at end(); nothing when timing is off.
struct Timed {
    lsa_ctx* c;
    int kind;
    hipStream_t s;
    hipEvent_t a = nullptr;
    Timed(lsa_ctx* c_, int kind_, hipStream_t s_) : c(c_), kind(kind_), s(s_) {
        if (c && c->timing) {
            a = ev_take(c);
            if (a) (void)hipEventRecord(a, s);
        }
    }
    void end() {
        if (!a) return;
        hipEvent_t b = ev_take(c);
        if (!b) return;
        (void)hipEventRecord(b, s);
        c->pending.push_back({kind, a, b});
        a = nullptr;
    }
};

}  // namespace

// ------------------------------------------------------------------- pools
struct lsa_pool {
    lsa_pool_desc d;
    int device = 0;
    int64_t cap = 0;
    int swap = 0;
    int row_bytes = 0;
    int64_t rows_per_seq = 0;
    void* tables = nullptr;
    int32_t* slot_of = nullptr;
    int32_t* logical_of = nullptr;
    int32_t* lru = nullptr;
    int32_t* meta = nullptr;
    uint64_t* stats = nullptr;
    uint8_t* ready = nullptr;
    void* cold_dev = nullptr;   // device address of the cold pool (HBM, or mapped pinned host)
    void* cold_host = nullptr;  // host address when pinned
    int64_t cold_stride_b = 0;  // bytes
    bool cold_owned = false;    // false: the caller's cold_buf
    uint64_t d2h_bytes = 0;
    int32_t capacity = 0;       // slots a swapping pool may use (adaptive GPU_CHUNKS), <= gpu_chunks
    int32_t recency_w = 100;    // replacement weighting, percent (100 = plain LRU)
    int32_t high_water = 100;   // percent of the capacity kept in use at most after a step
    bool general = false;       // set once a policy beyond plain LRU was used: free slots may have holes
    uint64_t last_hits = 0, last_misses = 0, last_h2d = 0;   // counters at the last lsa_pool_adapt
    // per sequence: entries [0, ready_prefix[b]) are marked stored (host-side
    // bookkeeping of the ready flags, which are only ever set)
    int64_t ready_prefix[LSA_MAX_BATCH] = {};
};

extern "C" {

// ------------------------------------------------------------ closed forms
int64_t lsa_compressed_cap(int64_t ctx, int32_t ratio) {
    if (ctx < 0 || ratio <= 0) return -1;
    return (ctx + ratio - 1) / ratio;
}

uint64_t lsa_pinned_bytes(int64_t ctx, const int32_t* ratios, int32_t n_layers, int32_t kv_dim,
                          lsa_dtype dtype) {
    if (!ratios || n_layers < 0 || kv_dim <= 0 || ctx < 0) return 0;
    uint64_t tot = 0;
    for (int32_t l = 0; l < n_layers; ++l) {
        const int64_t cap = lsa_compressed_cap(ctx, ratios[l]);
        if (cap < 0) return 0;
        tot += (uint64_t)cap * (uint64_t)kv_dim * (uint64_t)elem_bytes(dtype);
    }
    return tot;
}

int32_t lsa_max_capacity(int32_t window, int32_t gpu_chunks) {
    if (window < 0 || gpu_chunks < 0) return -1;
    return window + gpu_chunks;
}

lsa_status lsa_check_pinned(int64_t ctx, const int32_t* ratios, int32_t n_layers, int32_t kv_dim,
                            lsa_dtype dtype, uint64_t cap_bytes) {
    if (!ratios || n_layers <= 0 || kv_dim <= 0 || ctx < 0)
        return fail(LSA_ERR_INVALID_ARG, "lsa_check_pinned: invalid arguments");
    const uint64_t need = lsa_pinned_bytes(ctx, ratios, n_layers, kv_dim, dtype);
    if (need > cap_bytes)
        return fail(LSA_ERR_PINNED_CAP, "pinned cache exceeds cap: required_mib=%llu cap_mib=%llu",
                    (unsigned long long)((need + (1u << 20) - 1) >> 20),
                    (unsigned long long)(cap_bytes >> 20));
    return LSA_OK;
}

float lsa_threshold_logit(double tau) {
    if (!(tau > 0.0 && tau < 1.0)) return NAN;
    const double t = log(tau / (1.0 - tau));
    float tf = (float)t;
    if ((double)tf > t) tf = nextafterf(tf, -INFINITY);
    return tf;
}

const char* lsa_status_string(lsa_status s) {
    switch (s) {
        case LSA_OK: return "ok";
        case LSA_ERR_INVALID_ARG: return "invalid argument";
        case LSA_ERR_SLOTS_LT_TOPK: return "gpu_chunks must be >= index_topk";
        case LSA_ERR_PINNED_CAP: return "pinned cache exceeds cap";
        case LSA_ERR_NOT_STORED: return "selected chunk before it was stored";
        case LSA_ERR_HIP: return "HIP runtime error";
        case LSA_ERR_NO_MEMORY: return "out of memory";
        case LSA_ERR_UNSUPPORTED: return "unsupported shape";
    }
    return "unknown status";
}

const char* lsa_last_error(void) { return g_err.c_str(); }
int32_t lsa_abi_version(void) { return LSA_ABI_VERSION; }

// ----------------------------------------------------------------- context
lsa_status lsa_ctx_create(lsa_ctx** out, int32_t device) {
    if (!out) return fail(LSA_ERR_INVALID_ARG, "lsa_ctx_create: out is NULL");
    *out = nullptr;
    int n = 0;
    HIPTRY(hipGetDeviceCount(&n));
    if (device < 0 || device >= n) return fail(LSA_ERR_INVALID_ARG, "device %d of %d", device, n);
    HIPTRY(hipSetDevice(device));
    lsa_ctx* c = new lsa_ctx;
    c->device = device;
    c->n_cu = n_cu_current();
    // the static scratch's device address, looked up once per device (only the
    // allocation-free step needs it, so a failed lookup fails only that call)
    c->scratch_status = scratch_address(device, &c->scratch);
    const size_t small = LSA_MAX_BATCH * sizeof(int32_t) + kAttendSyncWords * sizeof(uint32_t);
    if (hipMalloc(reinterpret_cast<void**>(&c->sel_guess), small) != hipSuccess) {
        delete c;
        return fail(LSA_ERR_NO_MEMORY, "lsa_ctx_create: %zu bytes of device memory", small);
    }
    c->att_sync = reinterpret_cast<uint32_t*>(c->sel_guess + LSA_MAX_BATCH);
    if (hipMemset(c->sel_guess, 0, small) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        (void)hipFree(c->sel_guess);
        delete c;
        return fail(LSA_ERR_HIP, "lsa_ctx_create: clearing the select guesses and attention counters failed");
    }
    *out = c;
    return LSA_OK;
}

void lsa_ctx_destroy(lsa_ctx* c) {
    if (!c) return;
    (void)hipDeviceSynchronize();
    if (c->ws) (void)hipFree(c->ws);
    if (c->zero) (void)hipFree(c->zero);
    if (c->sel_guess) (void)hipFree(c->sel_guess);
    for (auto& p : c->pending) {
        (void)hipEventDestroy(p.a);
        (void)hipEventDestroy(p.b);
    }
    for (auto e : c->spare) (void)hipEventDestroy(e);
    for (int i = 0; i < 2; ++i) {
        if (c->kv_layers_dev[i]) (void)hipFree(c->kv_layers_dev[i]);
        if (c->kv_layers_host[i]) (void)hipHostFree(c->kv_layers_host[i]);
        if (c->kv_layers_done[i]) (void)hipEventDestroy(c->kv_layers_done[i]);
    }
    delete c;
}

lsa_status lsa_ctx_reserve(lsa_ctx* c, uint64_t bytes) {
    if (!c) return fail(LSA_ERR_INVALID_ARG, "ctx is NULL");
    return ws_ensure(c, (size_t)bytes);
}

lsa_status lsa_ctx_set_timing(lsa_ctx* c, int32_t on) {
    if (!c) return fail(LSA_ERR_INVALID_ARG, "ctx is NULL");
    c->timing = on != 0;
    return LSA_OK;
}

lsa_status lsa_ctx_set_key_policy(lsa_ctx* c, int32_t non_temporal) {
    if (!c) return fail(LSA_ERR_INVALID_ARG, "ctx is NULL");
    c->stream_keys = non_temporal != 0;
    return LSA_OK;
}

lsa_status lsa_ctx_timing_read(lsa_ctx* c, double* ms, int64_t* launches) {
    if (!c || !ms || !launches) return fail(LSA_ERR_INVALID_ARG, "lsa_ctx_timing_read: NULL argument");
    for (int k = 0; k < LSA_K_COUNT; ++k) {
        ms[k] = 0.0;
        launches[k] = 0;
    }
    if (!c->pending.empty()) HIPTRY(hipEventSynchronize(c->pending.back().b));
    for (auto& p : c->pending) {
        float t = 0.f;
        HIPTRY(hipEventElapsedTime(&t, p.a, p.b));
        ms[p.kind] += t;
        launches[p.kind] += 1;
        c->spare.push_back(p.a);
        c->spare.push_back(p.b);
    }
    c->pending.clear();
    return LSA_OK;
}

}  // extern "C"

// ------------------------------------------------------------------ score
namespace {

bool mx_dtype(lsa_dtype d) { return d == LSA_MXFP4 || d == LSA_MXINT8; }

// bytes of one key row of dk elements
uint64_t key_row_bytes(lsa_dtype d, int32_t dk) {
    if (d == LSA_MXFP4) return (uint64_t)dk / 2;
    if (d == LSA_MXINT8) return (uint64_t)dk;
    return (uint64_t)dk * (uint64_t)elem_bytes(d);
}

lsa_status score_args(const void* keys, lsa_dtype key_dtype, const uint8_t* key_scales, int32_t batch,
                      int64_t n_keys, const int64_t* n_valid, int32_t dk, const float* q, const float* w,
                      int32_t n_idx, int32_t heads, lsa_ensemble ens, float* scores, ScoreArgs* a) {
    if (batch < 1 || batch > LSA_MAX_BATCH) return fail(LSA_ERR_INVALID_ARG, "batch %d not in [1, %d]", batch, LSA_MAX_BATCH);
    if (n_keys < 0 || n_keys > INT32_MAX) return fail(LSA_ERR_INVALID_ARG, "n_keys %lld out of range", (long long)n_keys);
    if (!keys || !q || !w || !scores) return fail(LSA_ERR_INVALID_ARG, "lsa_score: NULL pointer");
    if (ens != LSA_ENSEMBLE_MAX && ens != LSA_ENSEMBLE_MEAN) return fail(LSA_ERR_INVALID_ARG, "ensemble %d", (int)ens);
    if (dk <= 0 || n_idx <= 0 || heads <= 0) return fail(LSA_ERR_INVALID_ARG, "dk, n_idx and heads must be positive");
    if (key_dtype != LSA_F32 && key_dtype != LSA_BF16 && key_dtype != LSA_FP8_E4M3 && !mx_dtype(key_dtype))
        return fail(LSA_ERR_UNSUPPORTED, "key dtype %d (supported: F32, BF16, FP8_E4M3, MXFP4, MXINT8)",
                    (int)key_dtype);
    if (dk != 32 && dk != 64 && dk != 128) return fail(LSA_ERR_UNSUPPORTED, "dk %d (supported: 32, 64, 128)", dk);
    if (key_dtype == LSA_MXFP4 && dk == 32) return fail(LSA_ERR_UNSUPPORTED, "MXFP4 keys need dk 64 or 128");
    if (mx_dtype(key_dtype) && !key_scales) return fail(LSA_ERR_INVALID_ARG, "MX keys need key_scales");
    if (n_idx > 4 || heads > 8) return fail(LSA_ERR_UNSUPPORTED, "n_idx %d x heads %d (supported: <= 4 x <= 8)", n_idx, heads);
    if ((uint64_t)n_keys * key_row_bytes(key_dtype, dk) >= ((uint64_t)1 << 32))
        return fail(LSA_ERR_UNSUPPORTED, "a sequence's keys exceed 4 GiB");
    memset(a, 0, sizeof(*a));
    a->keys = keys;
    a->scales = mx_dtype(key_dtype) ? key_scales : nullptr;
    a->q = q;
    a->w = w;
    a->scores = scores;
    a->n_keys = n_keys;
    a->batch = batch;
    a->n_idx = n_idx;
    a->heads = heads;
    a->ensemble = ens;
    // keys per wave tile: 32 fp32 keys, 64 of every narrower format
    const int64_t tile_keys = key_dtype == LSA_F32 ? 32 : 64;
    int tiles = 0;
    for (int b = 0; b < batch; ++b) {
        const int64_t nv = n_valid ? n_valid[b] : n_keys;
        if (nv < 0 || nv > n_keys) return fail(LSA_ERR_INVALID_ARG, "n_valid[%d] = %lld not in [0, n_keys]", b, (long long)nv);
        a->n_valid[b] = (int32_t)nv;
        a->tile_start[b] = tiles;
        tiles += (int)((nv + tile_keys - 1) / tile_keys);
    }
    a->tile_start[batch] = tiles;
    return LSA_OK;
}

lsa_status select_setup(lsa_ctx* c, const float* scores, int32_t n_seg, int64_t n_keys, const int64_t* n_valid,
                        lsa_select_mode mode, int32_t k, int32_t stride, double tau, int32_t* sel, int32_t* count,
                        SelectArgs* a, size_t* zero_need, size_t* ws_need) {
    if (!scores || !sel || !count) return fail(LSA_ERR_INVALID_ARG, "lsa_select: NULL pointer");
    if (n_seg < 1) return fail(LSA_ERR_INVALID_ARG, "n_seg %d", n_seg);
    if (n_keys < 0 || n_keys > INT32_MAX) return fail(LSA_ERR_INVALID_ARG, "n_keys out of range");
    if (mode != LSA_SELECT_TOPK && mode != LSA_SELECT_THRESHOLD) return fail(LSA_ERR_INVALID_ARG, "mode %d", (int)mode);
    if (k < 1 || k > 4096) return fail(LSA_ERR_INVALID_ARG, "k %d not in [1, 4096]", k);
    if (mode == LSA_SELECT_THRESHOLD && !(tau > 0.0 && tau < 1.0))
        return fail(LSA_ERR_INVALID_ARG, "tau %g not in (0, 1)", tau);
    memset(a, 0, sizeof(*a));
    a->scores = scores;
    a->n_keys = n_keys;
    a->n_seg = n_seg;
    a->k = k;
    a->stride = stride;
    a->mode = mode;
    a->t_f = mode == LSA_SELECT_THRESHOLD ? lsa_threshold_logit(tau) : 0.0f;
    a->sel = sel;
    a->count = count;
    a->n_valid_uniform = (int32_t)n_keys;
    if (n_valid) {
        bool uniform = true;
        for (int s = 0; s < n_seg; ++s) {
            if (n_valid[s] < 0 || n_valid[s] > n_keys)
                return fail(LSA_ERR_INVALID_ARG, "n_valid[%d] = %lld not in [0, n_keys]", s, (long long)n_valid[s]);
            uniform = uniform && n_valid[s] == n_valid[0];
        }
        if (uniform) {
            a->n_valid_uniform = (int32_t)n_valid[0];
        } else {
            if (n_seg > LSA_MAX_BATCH)
                return fail(LSA_ERR_UNSUPPORTED, "per-segment n_valid needs n_seg <= %d", LSA_MAX_BATCH);
            a->has_n_valid = 1;
            for (int s = 0; s < n_seg; ++s) a->n_valid[s] = (int32_t)n_valid[s];
        }
    }
    (void)c;
    if (!select_plan(a, zero_need, ws_need)) return fail(LSA_ERR_UNSUPPORTED, "selection shape out of range");
    return LSA_OK;
}

StageLayer stage_layer(const lsa_pool* p, const int32_t* sel, const int32_t* count, int32_t sel_stride,
                       int32_t src_ratio, int32_t* phys, int32_t phys_stride, int32_t* n_rows,
                       const float* imp = nullptr, int64_t imp_stride = 0) {
    StageLayer L;
    memset(&L, 0, sizeof(L));
    L.slot_of = p->slot_of;
    L.logical_of = p->logical_of;
    L.lru = p->lru;
    L.meta = p->meta;
    L.stats = p->stats;
    L.ready = p->ready;
    L.all_ready = 0;
    for (int b = 0; b < p->d.batch && b < 64; ++b)
        if (p->ready_prefix[b] >= p->cap) L.all_ready |= 1ull << b;
    L.sel = sel;
    L.count = count;
    L.phys = phys;
    L.n_rows = n_rows;
    L.cold = p->cold_dev;
    L.kv = p->d.kv_buf;
    L.cap = p->cap;
    L.cold_stride_b = p->cold_stride_b;
    L.kv_stride_b_bytes = p->d.kv_stride_b * (int64_t)elem_bytes(p->d.dtype);
    L.ratio = p->d.ratio;
    L.src_ratio = src_ratio;
    L.S = p->d.gpu_chunks;
    L.cap_slots = p->capacity;
    L.window = p->d.window;
    L.swap = p->swap;
    L.sel_stride = sel_stride;
    L.phys_stride = phys_stride;
    L.row_bytes = p->row_bytes;
    L.general = p->general ? 1 : 0;
    L.recency_w = p->recency_w;
    L.hw_slots = p->high_water < 100 ? (int32_t)((int64_t)p->high_water * p->capacity / 100) : INT32_MAX;
    L.imp = imp;
    L.imp_stride = imp_stride;
    return L;
}

// A pool that weighs its replacement needs the step's scores of its own entries:
// its ratio must be the source ratio (entries = scored entries).
lsa_status stage_importance_check(const lsa_pool* p, const float* imp, int32_t src_ratio, int l) {
    if (!p->swap || p->recency_w >= 100) return LSA_OK;
    if (!imp) return fail(LSA_ERR_INVALID_ARG, "pool %d weighs importance in its replacement: the step's scores "
                                               "are needed", l);
    if (p->d.ratio != src_ratio)
        return fail(LSA_ERR_UNSUPPORTED, "pool %d weighs importance in its replacement but its ratio %d is not the "
                                         "scored source ratio %d", l, p->d.ratio, src_ratio);
    return LSA_OK;
}

// valid source entries per sequence (NULL: unbounded, every chunk complete)
lsa_status fill_src_valid(StageArgs* a, const int64_t* n_valid) {
    for (int b = 0; b < a->batch; ++b) {
        const int64_t v = n_valid ? n_valid[b] : (int64_t)INT32_MAX;
        if (v < 0) return fail(LSA_ERR_INVALID_ARG, "n_valid[%d] = %lld < 0", b, (long long)v);
        a->src_valid[b] = (int32_t)(v > INT32_MAX ? INT32_MAX : v);
    }
    return LSA_OK;
}

lsa_status stage_check(const lsa_pool* p, int32_t sel_stride, int32_t src_ratio, int32_t phys_stride) {
    if (sel_stride < 1 || sel_stride > 1024) return fail(LSA_ERR_INVALID_ARG, "sel_stride %d not in [1, 1024]", sel_stride);
    if (p->swap && sel_stride > p->capacity)
        return fail(LSA_ERR_SLOTS_LT_TOPK, "a step may select %d chunks but the pool uses %d slots",
                    sel_stride, p->capacity);
    if (src_ratio < 1 || p->d.ratio % src_ratio != 0)
        return fail(LSA_ERR_INVALID_ARG, "pool ratio %d is not a multiple of src_ratio %d", p->d.ratio, src_ratio);
    if (phys_stride < p->d.window + sel_stride)
        return fail(LSA_ERR_INVALID_ARG, "phys_stride %d < window + sel_stride (%d)", phys_stride, p->d.window + sel_stride);
    return LSA_OK;
}


// attention split + combine, timed as two intervals when timing is on
lsa_status attend_timed(lsa_ctx* ctx, const AttendArgs& a, hipStream_t s) {
    Timed t(ctx, LSA_K_ATTEND, s);
    hipEvent_t mid = t.a ? ev_take(ctx) : nullptr;
    HIPTRY(launch_lsa_attend(a, s, mid));
    if (mid) {
        ctx->pending.push_back({LSA_K_ATTEND, t.a, mid});
        t.a = nullptr;
        hipEvent_t e = ev_take(ctx);
        if (e) {
            (void)hipEventRecord(e, s);
            ctx->pending.push_back({LSA_K_COMBINE, mid, e});
        }
    } else {
        t.end();
    }
    return LSA_OK;
}

}  // namespace

extern "C" {

lsa_status lsa_project(const float* hidden, int32_t batch, int32_t d_model, const void* wq, const void* ww,
                       lsa_dtype w_dtype, int32_t n_idx, int32_t heads, int32_t dk, float* q, float* w,
                       lsa_stream_t stream) {
    if (!hidden || !wq || !ww || !q || !w) return fail(LSA_ERR_INVALID_ARG, "lsa_project: NULL pointer");
    if (batch < 1 || batch > LSA_MAX_BATCH) return fail(LSA_ERR_INVALID_ARG, "batch %d not in [1, %d]", batch, LSA_MAX_BATCH);
    if (n_idx < 1 || heads < 1 || dk < 1) return fail(LSA_ERR_INVALID_ARG, "n_idx, heads and dk must be positive");
    if (w_dtype != LSA_F32 && w_dtype != LSA_BF16)
        return fail(LSA_ERR_UNSUPPORTED, "weight dtype %d (supported: F32, BF16)", (int)w_dtype);
    if (d_model < 8 || d_model % 8 != 0 || d_model > 16384)
        return fail(LSA_ERR_UNSUPPORTED, "d_model %d (supported: multiples of 8 up to 16384)", d_model);
    if ((int64_t)n_idx * heads * (dk + 1) >= ((int64_t)1 << 31))
        return fail(LSA_ERR_UNSUPPORTED, "too many projection rows");
    if (((uintptr_t)hidden & 15) != 0) return fail(LSA_ERR_INVALID_ARG, "hidden must be 16-byte aligned");
    ProjectArgs a;
    a.hidden = hidden;
    a.wq = wq;
    a.ww = ww;
    a.q = q;
    a.w = w;
    a.d_model = d_model;
    a.q_rows = n_idx * heads * dk;
    a.w_rows = n_idx * heads;
    HIPTRY(launch_project(a, w_dtype, batch, n_cu_current(), (hipStream_t)stream));
    return LSA_OK;
}

lsa_status lsa_score(const void* keys, lsa_dtype key_dtype, const uint8_t* key_scales, int32_t batch, int64_t n_keys,
                     const int64_t* n_valid, int32_t dk, const float* q, const float* w, int32_t n_idx,
                     int32_t heads, lsa_ensemble ensemble, float* scores, lsa_stream_t stream) {
    ScoreArgs a;
    lsa_status st = score_args(keys, key_dtype, key_scales, batch, n_keys, n_valid, dk, q, w, n_idx, heads, ensemble,
                               scores, &a);
    if (st != LSA_OK) return st;
    HIPTRY(launch_fm_score(a, key_dtype, dk, n_cu_current(), (hipStream_t)stream, true));
    return LSA_OK;
}

lsa_status lsa_select(lsa_ctx* ctx, const float* scores, int32_t n_seg, int64_t n_keys, const int64_t* n_valid,
                      lsa_select_mode mode, int32_t k, double tau, int32_t* sel, int32_t* count,
                      lsa_stream_t stream) {
    if (!ctx) return fail(LSA_ERR_INVALID_ARG, "ctx is NULL");
    SelectArgs a;
    size_t need = 0, zneed = 0;
    lsa_status st = select_setup(ctx, scores, n_seg, n_keys, n_valid, mode, k, k, tau, sel, count, &a, &zneed, &need);
    if (st != LSA_OK) return st;
    st = zero_ensure(ctx, zneed);
    if (st != LSA_OK) return st;
    st = ws_ensure(ctx, need);
    if (st != LSA_OK) return st;
    select_bind(&a, ctx->zero, ctx->ws);
    Timed t(ctx, LSA_K_SELECT, (hipStream_t)stream);
    HIPTRY(launch_fm_select(a, (hipStream_t)stream));
    t.end();
    return LSA_OK;
}

// ------------------------------------------------------------------- pools
int64_t lsa_pool_rows(const lsa_pool_desc* d) {
    if (!d) return -1;
    const int64_t cap = lsa_compressed_cap(d->ctx, d->ratio);
    if (cap < 0 || d->window < 0 || d->gpu_chunks < 1) return -1;
    return d->window + (cap > d->gpu_chunks ? d->gpu_chunks : cap);
}

void lsa_pool_destroy(lsa_pool* p) {
    if (!p) return;
    (void)hipDeviceSynchronize();
    if (p->tables) (void)hipFree(p->tables);
    if (p->cold_host) (void)hipHostFree(p->cold_host);
    else if (p->cold_dev && p->cold_owned) (void)hipFree(p->cold_dev);
    delete p;
}

lsa_status lsa_pool_create(lsa_pool** out, const lsa_pool_desc* d) {
    if (!out || !d) return fail(LSA_ERR_INVALID_ARG, "lsa_pool_create: NULL argument");
    *out = nullptr;
    if (d->ctx < 0 || d->ratio < 1) return fail(LSA_ERR_INVALID_ARG, "ctx %lld, ratio %d", (long long)d->ctx, d->ratio);
    if (d->window < 0 || d->window > 4096) return fail(LSA_ERR_INVALID_ARG, "window %d not in [0, 4096]", d->window);
    if (d->gpu_chunks < 1) return fail(LSA_ERR_INVALID_ARG, "gpu_chunks %d < 1", d->gpu_chunks);
    if (d->topk < 1 || d->topk > 1024) return fail(LSA_ERR_INVALID_ARG, "topk %d not in [1, 1024]", d->topk);
    if (d->batch < 1 || d->batch > LSA_MAX_BATCH) return fail(LSA_ERR_INVALID_ARG, "batch %d", d->batch);
    if (!row_dtype_ok(d->dtype)) return fail(LSA_ERR_UNSUPPORTED, "row dtype %d", (int)d->dtype);
    if (d->kv_dim < 8 || (d->kv_dim * elem_bytes(d->dtype)) % 16 != 0)
        return fail(LSA_ERR_UNSUPPORTED, "kv_dim %d: rows must be a multiple of 16 bytes", d->kv_dim);
    if (d->cold != LSA_COLD_HBM && d->cold != LSA_COLD_HOST) return fail(LSA_ERR_INVALID_ARG, "cold kind %d", (int)d->cold);
    if (!d->kv_buf) return fail(LSA_ERR_INVALID_ARG, "kv_buf is NULL");
    const int64_t cap = lsa_compressed_cap(d->ctx, d->ratio);
    if (cap > INT32_MAX) return fail(LSA_ERR_UNSUPPORTED, "compressed_cap %lld", (long long)cap);
    const int swap = cap > d->gpu_chunks ? 1 : 0;
    if (swap && d->gpu_chunks > 4096)
        return fail(LSA_ERR_UNSUPPORTED, "a swapping pool supports at most 4096 gpu_chunks (got %d)", d->gpu_chunks);
    const int64_t rows = lsa_pool_rows(d);
    if (d->batch > 1 && d->kv_stride_b < rows * d->kv_dim)
        return fail(LSA_ERR_INVALID_ARG, "kv_stride_b %lld < rows * kv_dim (%lld)", (long long)d->kv_stride_b,
                    (long long)(rows * d->kv_dim));
    if (swap && d->gpu_chunks < d->topk && !d->allow_topk_reduction)
        return fail(LSA_ERR_SLOTS_LT_TOPK, "gpu_chunks (%d) must be >= index_topk (%d)", d->gpu_chunks, d->topk);
    const int row_bytes = d->kv_dim * elem_bytes(d->dtype);
    const uint64_t cold_bytes = swap ? (uint64_t)d->batch * (uint64_t)cap * (uint64_t)row_bytes : 0;
    if (d->cold_buf && d->cold != LSA_COLD_HBM)
        return fail(LSA_ERR_INVALID_ARG, "a caller-owned cold_buf must be device memory (LSA_COLD_HBM)");
    if (d->cold_buf && d->batch > 1 && d->cold_stride_b < cap * (int64_t)row_bytes)
        return fail(LSA_ERR_INVALID_ARG, "cold_stride_b %lld < compressed_cap * row bytes (%lld)",
                    (long long)d->cold_stride_b, (long long)(cap * (int64_t)row_bytes));
    if (swap && d->cold == LSA_COLD_HOST && d->pinned_cap_bytes && cold_bytes > d->pinned_cap_bytes)
        return fail(LSA_ERR_PINNED_CAP, "pinned cache exceeds cap: required_mib=%llu cap_mib=%llu",
                    (unsigned long long)((cold_bytes + (1u << 20) - 1) >> 20),
                    (unsigned long long)(d->pinned_cap_bytes >> 20));

    lsa_pool* p = new lsa_pool;
    p->d = *d;
    HIPTRY(hipGetDevice(&p->device));
    p->cap = cap;
    p->swap = swap;
    p->row_bytes = row_bytes;
    p->rows_per_seq = rows;
    p->capacity = d->gpu_chunks;
    const int64_t B = d->batch, S = swap ? d->gpu_chunks : 1, C = cap;
    const size_t sz_slot = align_up((size_t)(swap ? B * C : 1) * 4, 256);
    const size_t sz_lo = align_up((size_t)(B * S) * 4, 256);
    const size_t sz_meta = align_up((size_t)B * 16, 256);
    const size_t sz_stats = align_up((size_t)B * 32, 256);
    const size_t sz_ready = align_up((size_t)(B * C), 256);
    const size_t total = sz_slot + 2 * sz_lo + sz_meta + sz_stats + sz_ready;
    if (hipMalloc(&p->tables, total) != hipSuccess) {
        (void)hipGetLastError();
        delete p;
        return fail(LSA_ERR_NO_MEMORY, "pool tables (%zu bytes)", total);
    }
    char* t = static_cast<char*>(p->tables);
    p->slot_of = reinterpret_cast<int32_t*>(t); t += sz_slot;
    p->logical_of = reinterpret_cast<int32_t*>(t); t += sz_lo;
    p->lru = reinterpret_cast<int32_t*>(t); t += sz_lo;
    p->meta = reinterpret_cast<int32_t*>(t); t += sz_meta;
    p->stats = reinterpret_cast<uint64_t*>(t); t += sz_stats;
    p->ready = reinterpret_cast<uint8_t*>(t);
    hipError_t e = hipMemset(p->tables, 0, total);
    if (e == hipSuccess) e = hipMemset(p->slot_of, 0xFF, sz_slot + 2 * sz_lo);
    if (e == hipSuccess && swap) {
        p->cold_stride_b = (int64_t)C * row_bytes;
        if (d->cold_buf) {
            p->cold_dev = d->cold_buf;
            if (d->batch > 1) p->cold_stride_b = d->cold_stride_b;
        } else if (d->cold == LSA_COLD_HBM) {
            e = hipMalloc(&p->cold_dev, cold_bytes);
            p->cold_owned = true;
        } else {
            e = hipHostMalloc(&p->cold_host, cold_bytes, hipHostMallocDefault);
            if (e == hipSuccess) e = hipHostGetDevicePointer(&p->cold_dev, p->cold_host, 0);
        }
        if (e != hipSuccess) {
            (void)hipGetLastError();
            lsa_pool_destroy(p);
            return fail(LSA_ERR_NO_MEMORY, "cold pool of %llu bytes (%s)", (unsigned long long)cold_bytes,
                        d->cold == LSA_COLD_HBM ? "HBM" : "pinned host");
        }
    }
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        lsa_pool_destroy(p);
        return fail(LSA_ERR_HIP, "pool initialisation: %s", hipGetErrorString(e));
    }
    *out = p;
    return LSA_OK;
}

void* lsa_pool_host_rows(lsa_pool* p, int32_t b) {
    if (!p || !p->cold_host || b < 0 || b >= p->d.batch) return nullptr;
    return static_cast<char*>(p->cold_host) + (int64_t)b * p->cold_stride_b;
}

static lsa_status mark_ready(lsa_pool* p, int32_t b, int64_t first, int64_t count, hipStream_t s) {
    HIPTRY(hipMemsetAsync(p->ready + (int64_t)b * p->cap + first, 1, (size_t)count, s));
    if (first <= p->ready_prefix[b] && first + count > p->ready_prefix[b]) p->ready_prefix[b] = first + count;
    if (p->swap) {
        StageLayer L = stage_layer(p, nullptr, nullptr, 1, 1, nullptr, 0, nullptr);
        HIPTRY(launch_refresh_staged(L, b, first, count, s));
    }
    p->d2h_bytes += (uint64_t)count * (uint64_t)p->row_bytes;
    return LSA_OK;
}

lsa_status lsa_pool_store(lsa_pool* p, int32_t b, int64_t first, int64_t count, const void* rows,
                          lsa_stream_t stream) {
    if (!p) return fail(LSA_ERR_INVALID_ARG, "pool is NULL");
    if (b < 0 || b >= p->d.batch || first < 0 || count < 0 || first + count > p->cap)
        return fail(LSA_ERR_INVALID_ARG, "store of entries [%lld, %lld) of sequence %d outside [0, %lld)",
                    (long long)first, (long long)(first + count), b, (long long)p->cap);
    if (count == 0) return LSA_OK;
    if (!rows) return fail(LSA_ERR_INVALID_ARG, "rows is NULL");
    hipStream_t s = (hipStream_t)stream;
    const size_t bytes = (size_t)count * p->row_bytes;
    void* dst;
    if (p->swap) {
        char* base = static_cast<char*>(p->cold_host ? p->cold_host : p->cold_dev);
        dst = base + (int64_t)b * p->cold_stride_b + first * p->row_bytes;
    } else {
        dst = static_cast<char*>(p->d.kv_buf) +
              ((int64_t)b * p->d.kv_stride_b + (p->d.window + first) * (int64_t)p->d.kv_dim) * elem_bytes(p->d.dtype);
    }
    HIPTRY(hipMemcpyAsync(dst, rows, bytes, hipMemcpyDefault, s));
    return mark_ready(p, b, first, count, s);
}

lsa_status lsa_pool_mark_stored(lsa_pool* p, int32_t b, int64_t first, int64_t count, lsa_stream_t stream) {
    if (!p) return fail(LSA_ERR_INVALID_ARG, "pool is NULL");
    if (b < 0 || b >= p->d.batch || first < 0 || count < 0 || first + count > p->cap)
        return fail(LSA_ERR_INVALID_ARG, "entries [%lld, %lld) outside [0, %lld)", (long long)first,
                    (long long)(first + count), (long long)p->cap);
    if (count == 0) return LSA_OK;
    return mark_ready(p, b, first, count, (hipStream_t)stream);
}

lsa_status lsa_pool_reset(lsa_pool* p, lsa_stream_t stream) {
    if (!p) return fail(LSA_ERR_INVALID_ARG, "pool is NULL");
    hipStream_t s = (hipStream_t)stream;
    const int64_t B = p->d.batch;
    if (p->swap) {
        HIPTRY(hipMemsetAsync(p->slot_of, 0xFF, (size_t)(B * p->cap) * 4, s));
        HIPTRY(hipMemsetAsync(p->logical_of, 0xFF, (size_t)(B * p->d.gpu_chunks) * 4, s));
    }
    HIPTRY(hipMemsetAsync(p->meta, 0, (size_t)B * 16, s));
    HIPTRY(hipMemsetAsync(p->stats, 0, (size_t)B * 32, s));
    p->last_hits = p->last_misses = p->last_h2d = 0;
    return LSA_OK;
}

lsa_status lsa_pool_set_capacity(lsa_pool* p, int32_t capacity, lsa_stream_t stream) {
    if (!p) return fail(LSA_ERR_INVALID_ARG, "pool is NULL");
    if (capacity < 1 || capacity > p->d.gpu_chunks)
        return fail(LSA_ERR_INVALID_ARG, "capacity %d not in [1, gpu_chunks = %d]", capacity, p->d.gpu_chunks);
    if (p->swap && capacity < p->d.topk && !p->d.allow_topk_reduction)
        return fail(LSA_ERR_SLOTS_LT_TOPK, "capacity (%d) must be >= index_topk (%d)", capacity, p->d.topk);
    if (p->swap && capacity < p->capacity) {
        const StageLayer L = stage_layer(p, nullptr, nullptr, 1, 1, nullptr, 0, nullptr);
        HIPTRY(launch_pool_shrink(L, p->d.batch, capacity, (hipStream_t)stream));
    }
    p->capacity = capacity;
    return LSA_OK;
}

int32_t lsa_pool_capacity(const lsa_pool* p) { return p ? p->capacity : -1; }

lsa_status lsa_pool_set_replacement(lsa_pool* p, int32_t recency_weight, int32_t high_water) {
    if (!p) return fail(LSA_ERR_INVALID_ARG, "pool is NULL");
    if (recency_weight < 0 || recency_weight > 100 || high_water < 1 || high_water > 100)
        return fail(LSA_ERR_INVALID_ARG, "recency_weight %d not in [0, 100] or high_water %d not in [1, 100]",
                    recency_weight, high_water);
    if (p->swap && (recency_weight < 100 || high_water < 100) && p->d.gpu_chunks > 1024)
        return fail(LSA_ERR_UNSUPPORTED, "a replacement beyond plain LRU needs gpu_chunks <= 1024 (got %d)",
                    p->d.gpu_chunks);
    p->recency_w = recency_weight;
    p->high_water = high_water;
    if (recency_weight < 100 || high_water < 100) p->general = true;
    return LSA_OK;
}

lsa_status lsa_pool_adapt(lsa_pool* p, const lsa_adapt_policy* pol, int32_t steps, int32_t* capacity,
                          lsa_stream_t stream) {
    if (!p || !pol) return fail(LSA_ERR_INVALID_ARG, "lsa_pool_adapt: NULL argument");
    if (pol->step < 1 || pol->min_capacity < 1 || pol->max_capacity > p->d.gpu_chunks ||
        pol->min_capacity > pol->max_capacity || steps < 0)
        return fail(LSA_ERR_INVALID_ARG, "policy: step %d, capacity bounds [%d, %d] (gpu_chunks %d), steps %d",
                    pol->step, pol->min_capacity, pol->max_capacity, p->d.gpu_chunks, steps);
    if (p->swap && pol->min_capacity < p->d.topk && !p->d.allow_topk_reduction)
        return fail(LSA_ERR_SLOTS_LT_TOPK, "policy min_capacity (%d) must be >= index_topk (%d)", pol->min_capacity,
                    p->d.topk);
    HIPTRY(hipStreamSynchronize((hipStream_t)stream));
    const int B = p->d.batch;
    std::vector<uint64_t> st((size_t)B * 4);
    HIPTRY(hipMemcpy(st.data(), p->stats, st.size() * 8, hipMemcpyDeviceToHost));
    uint64_t hits = 0, misses = 0, h2d = 0;
    for (int b = 0; b < B; ++b) {
        hits += st[b * 4 + 0];
        misses += st[b * 4 + 1];
        h2d += st[b * 4 + 2];
    }
    const uint64_t h = hits - p->last_hits, m = misses - p->last_misses, x = h2d - p->last_h2d;
    p->last_hits = hits;
    p->last_misses = misses;
    p->last_h2d = h2d;
    int32_t c = p->capacity;
    if (h + m > 0) {
        const double miss_rate = (double)m / (double)(h + m);
        const double h2d_per_step = (double)x / (double)(steps > 0 ? steps : 1);
        if (miss_rate > pol->grow_miss_rate || h2d_per_step > pol->grow_h2d_bytes_per_step)
            c = std::min(pol->max_capacity, c + pol->step);
        else if (miss_rate < pol->shrink_miss_rate)
            c = std::max(pol->min_capacity, c - pol->step);
    }
    if (c != p->capacity) {
        lsa_status r = lsa_pool_set_capacity(p, c, stream);
        if (r != LSA_OK) return r;
    }
    if (capacity) *capacity = p->capacity;
    return LSA_OK;
}

lsa_status lsa_pool_stats(lsa_pool* p, lsa_pool_stats_t* out, lsa_stream_t stream) {
    if (!p || !out) return fail(LSA_ERR_INVALID_ARG, "lsa_pool_stats: NULL argument");
    HIPTRY(hipStreamSynchronize((hipStream_t)stream));
    const int B = p->d.batch;
    std::vector<uint64_t> st((size_t)B * 4);
    std::vector<int32_t> meta((size_t)B * 4);
    HIPTRY(hipMemcpy(st.data(), p->stats, st.size() * 8, hipMemcpyDeviceToHost));
    HIPTRY(hipMemcpy(meta.data(), p->meta, meta.size() * 4, hipMemcpyDeviceToHost));
    memset(out, 0, sizeof(*out));
    int flags = 0;
    for (int b = 0; b < B; ++b) {
        out->hits += st[b * 4 + 0];
        out->misses += st[b * 4 + 1];
        out->h2d_bytes += st[b * 4 + 2];
        out->resident += meta[b * 4 + 0];
        flags |= meta[b * 4 + 1];
        meta[b * 4 + 1] = 0;
    }
    out->d2h_bytes = p->d2h_bytes;
    out->compressed_cap = p->cap;
    out->swap_enabled = p->swap;
    if (flags) {
        HIPTRY(hipMemcpy(p->meta, meta.data(), meta.size() * 4, hipMemcpyHostToDevice));
        if (flags & 2) return fail(LSA_ERR_INVALID_ARG, "a step selected an entry outside [0, compressed_cap)");
        return fail(LSA_ERR_NOT_STORED, "selected chunk before it was stored");
    }
    return LSA_OK;
}

lsa_status lsa_pool_state(lsa_pool* p, int32_t b, int32_t* slot_logical, int32_t* lru, int32_t* n_used,
                          lsa_stream_t stream) {
    if (!p || !slot_logical || !lru || !n_used) return fail(LSA_ERR_INVALID_ARG, "lsa_pool_state: NULL argument");
    if (b < 0 || b >= p->d.batch) return fail(LSA_ERR_INVALID_ARG, "sequence %d", b);
    HIPTRY(hipStreamSynchronize((hipStream_t)stream));
    const int S = p->d.gpu_chunks;
    if (!p->swap) {
        for (int i = 0; i < S; ++i) slot_logical[i] = -1;
        *n_used = 0;
        return LSA_OK;
    }
    int32_t meta[4];
    HIPTRY(hipMemcpy(meta, p->meta + b * 4, 16, hipMemcpyDeviceToHost));
    HIPTRY(hipMemcpy(slot_logical, p->logical_of + (int64_t)b * S, (size_t)S * 4, hipMemcpyDeviceToHost));
    HIPTRY(hipMemcpy(lru, p->lru + (int64_t)b * S, (size_t)S * 4, hipMemcpyDeviceToHost));
    *n_used = meta[0];
    return LSA_OK;
}

// ------------------------------------------------------------------- stage
lsa_status lsa_stage(lsa_pool* p, const int32_t* sel, const int32_t* count, int32_t sel_stride, int32_t src_ratio,
                     const int64_t* n_valid, const float* importance, int32_t* phys, int32_t phys_stride,
                     int32_t* n_rows, lsa_stream_t stream) {
    if (!p || !sel || !count || !phys || !n_rows) return fail(LSA_ERR_INVALID_ARG, "lsa_stage: NULL argument");
    lsa_status st = stage_check(p, sel_stride, src_ratio, phys_stride);
    if (st != LSA_OK) return st;
    st = stage_importance_check(p, importance, src_ratio, 0);
    if (st != LSA_OK) return st;
    StageArgs a;
    memset(&a, 0, sizeof(a));
    a.n_layers = 1;
    a.batch = p->d.batch;
    st = fill_src_valid(&a, n_valid);
    if (st != LSA_OK) return st;
    a.L[0] = stage_layer(p, sel, count, sel_stride, src_ratio, phys, phys_stride, n_rows, importance, p->cap);
    hipStream_t s = (hipStream_t)stream;
    HIPTRY(launch_kv_stage(a, s));
    return LSA_OK;
}

// ------------------------------------------------------------------ attend
lsa_status lsa_attend(lsa_ctx* ctx, const float* q, const void* kv, lsa_dtype dtype, int64_t kv_stride_b,
                      int64_t kv_rows, const int32_t* phys, int32_t phys_stride, const int32_t* n_rows,
                      int32_t batch, int32_t hq, int32_t kv_dim, float scale, float* out, lsa_stream_t stream) {
    if (!ctx || !q || !kv || !phys || !n_rows || !out) return fail(LSA_ERR_INVALID_ARG, "lsa_attend: NULL argument");
    if (batch < 1 || batch > LSA_MAX_BATCH) return fail(LSA_ERR_INVALID_ARG, "batch %d", batch);
    if (hq < 1 || phys_stride < 1 || kv_rows < 0 || !isfinite(scale))
        return fail(LSA_ERR_INVALID_ARG, "hq %d, phys_stride %d, kv_rows %lld, scale %g", hq, phys_stride,
                    (long long)kv_rows, (double)scale);
    if (batch > 1 && kv_stride_b < kv_rows * kv_dim) return fail(LSA_ERR_INVALID_ARG, "kv_stride_b < kv_rows * kv_dim");
    if (!row_dtype_ok(dtype)) return fail(LSA_ERR_UNSUPPORTED, "row dtype %d", (int)dtype);
    if (hq > 16 || (kv_dim != 128 && kv_dim != 256 && kv_dim != 512))
        return fail(LSA_ERR_UNSUPPORTED, "hq %d, kv_dim %d (supported: hq <= 16, kv_dim 128/256/512)", hq, kv_dim);
    if (phys_stride > kAttendMaxRows)
        return fail(LSA_ERR_UNSUPPORTED, "phys_stride %d > %d rows", phys_stride, kAttendMaxRows);
    AttendArgs a;
    memset(&a, 0, sizeof(a));
    a.n_layers = 1;
    a.batch = batch;
    a.hq = hq;
    a.D = kv_dim;
    a.dtype = dtype;
    a.max_splits = (phys_stride + kAttendRows - 1) / kAttendRows;
    a.scale = scale;
    const size_t need = attend_workspace_bytes(1, batch, kv_dim, phys_stride);
    lsa_status st = ws_ensure(ctx, need);
    if (st != LSA_OK) return st;
    a.part_acc = static_cast<float*>(ctx->ws);
    a.part_ml = a.part_acc + (size_t)batch * a.max_splits * 16 * kv_dim;
    a.sync = ctx->att_sync;
    a.n_cu = ctx->n_cu;
    a.L[0] = AttendLayer{q, kv, phys, n_rows, out, kv_stride_b, kv_rows, phys_stride, nullptr, nullptr, nullptr, 0, 0};
    return attend_timed(ctx, a, (hipStream_t)stream);
}

// ------------------------------------------------------------- decode step
}  // extern "C"

namespace {

// Everything one decode step launches, validated and bound to the workspace.
// n_buf row-list buffers are laid out (2 for the lookahead schedule).
struct StepPlan {
    // with a fixed scratch buffer (the allocation-free entry point) the select's
    // zero region is cleared by a fill kernel at the start of every call
    uint32_t* zero_clear = nullptr;
    size_t zero_clear_words = 0;
    ScoreArgs sa;
    SelectArgs se;
    // the layers in groups of kLaunchLayers, one stage / attention launch each;
    // phys / n_rows / src point at buffer 0
    static constexpr int kMaxGroups = (LSA_MAX_LAYERS + kLaunchLayers - 1) / kLaunchLayers;
    StageArgs ga[kMaxGroups];
    AttendArgs aa[kMaxGroups];
    int n_groups = 0;
    int B = 0, D = 0, W = 0, L = 0, k_eff = 0, phys_stride = 0;
    StageLayer& stage(int l) { return ga[l / kLaunchLayers].L[l % kLaunchLayers]; }
    AttendLayer& attend(int l) { return aa[l / kLaunchLayers].L[l % kLaunchLayers]; }
    int32_t* phys = nullptr;     // [n_buf][L][B][phys_stride]
    int32_t* n_rows = nullptr;   // [n_buf][L][B]
    int32_t* srcs = nullptr;     // [n_buf][L][B][phys_stride]
    uint64_t* miss = nullptr;    // [n_buf][L][B][phys_stride][2]
    int32_t* n_miss = nullptr;   // [n_buf][L][B]
};

// fixed / fixed_bytes: bind the workspace to this buffer instead of the
// context's (nothing is allocated; too small a buffer is an error)
lsa_status step_plan(lsa_ctx* ctx, const lsa_step_desc* d, int n_buf, StepPlan* P, char* fixed = nullptr,
                     size_t fixed_bytes = 0) {
    if (!ctx || !d) return fail(LSA_ERR_INVALID_ARG, "decode step: NULL argument");
    if (d->n_layers < 1 || d->n_layers > LSA_MAX_LAYERS)
        return fail(LSA_ERR_INVALID_ARG, "n_layers %d not in [1, %d]", d->n_layers, LSA_MAX_LAYERS);
    if (!d->pools || !d->q_attn || !d->out || !d->scores || !d->sel || !d->count)
        return fail(LSA_ERR_INVALID_ARG, "decode step: NULL pointer in the step");
    const lsa_pool* p0 = d->pools[0];
    if (!p0) return fail(LSA_ERR_INVALID_ARG, "pool 0 is NULL");
    const int B = d->batch, D = p0->d.kv_dim, W = p0->d.window;
    const lsa_dtype dt = p0->d.dtype;
    if (d->hq < 1 || d->hq > 16) return fail(LSA_ERR_UNSUPPORTED, "hq %d (supported 1..16)", d->hq);
    if (D != 128 && D != 256 && D != 512) return fail(LSA_ERR_UNSUPPORTED, "kv_dim %d", D);
    if (dt != LSA_F32 && dt != LSA_BF16) return fail(LSA_ERR_UNSUPPORTED, "row dtype %d (supported: F32, BF16)", (int)dt);
    if (!isfinite(d->scale)) return fail(LSA_ERR_INVALID_ARG, "scale");
    int k_eff = d->k;
    for (int l = 0; l < d->n_layers; ++l) {
        const lsa_pool* p = d->pools[l];
        if (!p) return fail(LSA_ERR_INVALID_ARG, "pool %d is NULL", l);
        if (p->d.batch != B || p->d.kv_dim != D || p->d.window != W || p->d.dtype != dt)
            return fail(LSA_ERR_INVALID_ARG, "pool %d: batch, kv_dim, window and dtype must match the step", l);
        if (p->swap && p->capacity < k_eff) {
            if (!p->d.allow_topk_reduction)
                return fail(LSA_ERR_SLOTS_LT_TOPK, "pool %d: gpu_chunks (%d) must be >= index_topk (%d)", l,
                            p->capacity, d->k);
            k_eff = p->capacity;
        }
    }
    lsa_status st = score_args(d->keys, d->key_dtype, d->key_scales, B, d->n_keys, d->n_valid, d->dk, d->q_idx,
                               d->w_idx, d->n_idx, d->heads, d->ensemble, d->scores, &P->sa);
    if (st != LSA_OK) return st;
    size_t sel_need = 0, sel_zero = 0;
    st = select_setup(ctx, d->scores, B, d->n_keys, d->n_valid, d->mode, k_eff, d->k, d->tau, d->sel, d->count, &P->se,
                      &sel_zero, &sel_need);
    if (st != LSA_OK) return st;
    const int phys_stride = W + d->k;
    if (phys_stride > kAttendMaxRows)
        return fail(LSA_ERR_UNSUPPORTED, "window + k = %d > %d rows", phys_stride, kAttendMaxRows);
    for (int l = 0; l < d->n_layers; ++l) {
        st = stage_check(d->pools[l], k_eff, d->src_ratio, phys_stride);
        if (st != LSA_OK) return st;
        st = stage_importance_check(d->pools[l], d->scores, d->src_ratio, l);
        if (st != LSA_OK) return st;
    }
    const int L = d->n_layers;
    // workspace: select candidates | attend partials | phys | n_rows | src | miss lists | miss counts
    const size_t off_att = align_up(sel_need, 256);
    const size_t att_bytes = attend_workspace_bytes(L, B, D, phys_stride);
    const size_t off_phys = off_att + align_up(att_bytes, 256);
    const size_t phys_bytes = d->phys ? 0 : align_up((size_t)n_buf * L * B * phys_stride * 4, 256);
    const size_t off_nrows = off_phys + phys_bytes;
    const size_t nrows_bytes = d->n_rows ? 0 : align_up((size_t)n_buf * L * B * 4, 256);
    const size_t off_src = off_nrows + nrows_bytes;
    const size_t src_bytes = align_up((size_t)n_buf * L * B * phys_stride * 4, 256);
    const size_t off_miss = off_src + src_bytes;
    const size_t miss_bytes = align_up((size_t)n_buf * L * B * phys_stride * 16, 256);
    const size_t off_nmiss = off_miss + miss_bytes;
    const size_t nmiss_bytes = align_up((size_t)n_buf * L * B * 4, 256);
    const size_t ws_total = off_nmiss + nmiss_bytes;
    char* ws;
    void* zero;
    // zero region: the select's histogram
    const size_t zero_need = align_up(sel_zero, 256);
    uint32_t* att_sync = ctx->att_sync;
    if (fixed) {
        // the attention's counters sit in the cleared region too, so every call
        // starts them at zero whatever an earlier call on the device left
        const size_t zero_al = zero_need + align_up(kAttendSyncWords * sizeof(uint32_t), 256);
        if (zero_al + ws_total > fixed_bytes)
            return fail(LSA_ERR_UNSUPPORTED, "the step needs %zu bytes of scratch; the static scratch holds %zu",
                        zero_al + ws_total, fixed_bytes);
        zero = fixed;
        att_sync = reinterpret_cast<uint32_t*>(fixed + zero_need);
        ws = fixed + zero_al;
        P->zero_clear = reinterpret_cast<uint32_t*>(fixed);
        P->zero_clear_words = zero_al / 4;
    } else {
        st = zero_ensure(ctx, zero_need);
        if (st != LSA_OK) return st;
        st = ws_ensure(ctx, ws_total);
        if (st != LSA_OK) return st;
        ws = static_cast<char*>(ctx->ws);
        zero = ctx->zero;
    }
    select_bind(&P->se, zero, ws);
    P->phys = d->phys ? d->phys : reinterpret_cast<int32_t*>(ws + off_phys);
    P->n_rows = d->n_rows ? d->n_rows : reinterpret_cast<int32_t*>(ws + off_nrows);
    P->srcs = reinterpret_cast<int32_t*>(ws + off_src);
    P->miss = reinterpret_cast<uint64_t*>(ws + off_miss);
    P->n_miss = reinterpret_cast<int32_t*>(ws + off_nmiss);
    P->B = B;
    P->D = D;
    P->W = W;
    P->L = L;
    P->k_eff = k_eff;
    P->phys_stride = phys_stride;

    P->n_groups = (L + kLaunchLayers - 1) / kLaunchLayers;
    const int max_splits = (phys_stride + kAttendRows - 1) / kAttendRows;
    float* acc_base = reinterpret_cast<float*>(ws + off_att);
    float* ml_base = acc_base + (size_t)L * B * max_splits * 16 * D;
    for (int g = 0; g < P->n_groups; ++g) {
        const int l0 = g * kLaunchLayers;
        const int nl = std::min(kLaunchLayers, L - l0);
        StageArgs& ga = P->ga[g];
        memset(&ga, 0, sizeof(ga));
        ga.n_layers = nl;
        ga.batch = B;
        for (int b = 0; b < B; ++b) ga.src_valid[b] = P->sa.n_valid[b];
        AttendArgs& aa = P->aa[g];
        memset(&aa, 0, sizeof(aa));
        aa.n_layers = nl;
        aa.batch = B;
        aa.hq = d->hq;
        aa.D = D;
        aa.dtype = dt;
        aa.max_splits = max_splits;
        aa.scale = d->scale;
        aa.part_acc = acc_base + (size_t)l0 * B * max_splits * 16 * D;
        aa.part_ml = ml_base + (size_t)l0 * B * max_splits * 32;
        aa.sync = att_sync;
        aa.n_cu = ctx->n_cu;
    }
    for (int l = 0; l < L; ++l) {
        const lsa_pool* p = d->pools[l];
        int32_t* ph = P->phys + (size_t)l * B * phys_stride;
        int32_t* nr = P->n_rows + (size_t)l * B;
        int32_t* sr = P->srcs + (size_t)l * B * phys_stride;
        StageLayer& sl = P->stage(l);
        sl = stage_layer(p, d->sel, d->count, d->k, d->src_ratio, ph, phys_stride, nr, d->scores, d->n_keys);
        sl.defer_copy = 1;
        sl.src = sr;
        sl.miss = P->miss + (size_t)l * B * phys_stride * 2;
        sl.n_miss = P->n_miss + (size_t)l * B;
        P->attend(l) = AttendLayer{d->q_attn + (size_t)l * B * d->hq * D, p->d.kv_buf, ph, nr,
                                   d->out + (size_t)l * B * d->hq * D, p->d.kv_stride_b, p->rows_per_seq, phys_stride,
                                   nullptr, p->d.kv_buf, p->cold_dev, p->cold_stride_b, p->cap};
    }
    return LSA_OK;
}

// The missed rows of row-list buffer `buf` as the lookahead copy reads them
// (n_seg = 0: nothing to copy).
CopyArgs plan_copy(const StepPlan& P, int buf, bool copy) {
    const size_t per_buf = (size_t)P.L * P.B;
    return CopyArgs{P.miss + buf * per_buf * P.phys_stride * 2, P.n_miss + buf * per_buf,
                    copy ? P.L * P.B : 0, P.phys_stride, P.D * (P.aa[0].dtype == LSA_F32 ? 4 : 2)};
}

// a swapping layer's missed rows are read from the cold pool by the attention,
// which also fills their slots
void plan_attention_fetches(StepPlan* P, const lsa_step_desc* d) {
    for (int l = 0; l < P->L; ++l)
        if (d->pools[l]->swap) P->attend(l).src = P->stage(l).src;
}

lsa_status attend_groups(lsa_ctx* ctx, const StepPlan& P, hipStream_t s) {
    for (int g = 0; g < P.n_groups; ++g) {
        lsa_status st = attend_timed(ctx, P.aa[g], s);
        if (st != LSA_OK) return st;
    }
    return LSA_OK;
}

// Point the stage and attention of a plan at row-list buffer `buf`.
void plan_use_buffer(StepPlan* P, int buf) {
    const size_t per_buf = (size_t)P->L * P->B;
    for (int l = 0; l < P->L; ++l) {
        int32_t* ph = P->phys + (buf * per_buf + (size_t)l * P->B) * P->phys_stride;
        int32_t* nr = P->n_rows + buf * per_buf + (size_t)l * P->B;
        StageLayer& sl = P->stage(l);
        sl.phys = ph;
        sl.n_rows = nr;
        sl.src = P->srcs + (buf * per_buf + (size_t)l * P->B) * P->phys_stride;
        sl.miss = P->miss + (buf * per_buf + (size_t)l * P->B) * P->phys_stride * 2;
        sl.n_miss = P->n_miss + buf * per_buf + (size_t)l * P->B;
        P->attend(l).phys = ph;
        P->attend(l).n_rows = nr;
    }
}

// Whether the score launch can write the select's histogram and candidate
// lists: the long-segment select with one segment per sequence, fp32 or bf16
// keys, a workgroup per sequence at least, and list blocks that fit the final
// selection's table.
bool score_lists_fit(const ScoreArgs& sa, const SelectArgs& se, lsa_dtype key_dtype, int n_cu) {
    return (key_dtype == LSA_F32 || key_dtype == LSA_BF16) && se.path == 1 && se.n_seg == sa.batch &&
           sa.tile_start[sa.batch] > 0 && score_lists_grid(sa, n_cu) >= sa.batch && se.nblk * 4 <= kSelFinalBlocks;
}

lsa_status launch_predict(lsa_ctx* ctx, const StepPlan& P, const lsa_step_desc* d, hipStream_t s, bool fetch) {
    if (score_lists_fit(P.sa, P.se, d->key_dtype, ctx->n_cu)) {
        // score, histogram and candidate lists in one launch (the lists from
        // the bin the previous step's final selection left), then the final
        // selection, which checks that bin against this step's boundary
        const ScoreHistArgs h{nullptr, P.se.mode, P.se.t_f, P.se.blk_count, P.se.blk_idx, P.se.blk_key,
                              ctx->sel_guess, P.se.nblk};
        {
            Timed t(ctx, LSA_K_SCORE, s);
            HIPTRY(launch_fm_score_lists(P.sa, h, d->key_dtype, d->dk, ctx->n_cu, s, ctx->stream_keys));
            t.end();
        }
        SelectArgs se = P.se;
        se.pre = 1;
        se.nblk = P.se.nblk * 4;
        se.blk_stride = kSelColBlk / 4;
        se.guess_out = ctx->sel_guess;
        Timed t(ctx, LSA_K_SELECT, s);
        HIPTRY(launch_fm_select_final(se, s));
        t.end();
    } else {
        {
            Timed t(ctx, LSA_K_SCORE, s);
            HIPTRY(launch_fm_score(P.sa, d->key_dtype, d->dk, ctx->n_cu, s, ctx->stream_keys));
            t.end();
        }
        SelectArgs se = P.se;
        se.guess_out = ctx->sel_guess;
        Timed t(ctx, LSA_K_SELECT, s);
        HIPTRY(launch_fm_select(se, s));
        t.end();
    }
    for (int g = 0; g < P.n_groups; ++g) {
        Timed t(ctx, LSA_K_STAGE, s);
        HIPTRY(launch_kv_stage(P.ga[g], s));
        t.end();
    }
    if (fetch) {
        for (int g = 0; g < P.n_groups; ++g) {
            Timed t(ctx, LSA_K_GATHER, s);
            HIPTRY(launch_fetch_missed(P.ga[g], P.phys_stride, s));
            t.end();
        }
    }
    return LSA_OK;
}


}  // namespace

extern "C" {

lsa_status lsa_decode_step(lsa_ctx* ctx, const lsa_step_desc* d, lsa_stream_t stream) {
    StepPlan P;
    lsa_status st = step_plan(ctx, d, 1, &P);
    if (st != LSA_OK) return st;
    plan_attention_fetches(&P, d);
    hipStream_t s = (hipStream_t)stream;
    st = launch_predict(ctx, P, d, s, false);
    if (st != LSA_OK) return st;
    return attend_groups(ctx, P, s);
}

lsa_status lsa_decode_attend(lsa_ctx* ctx, const lsa_step_desc* d, lsa_stream_t stream) {
    StepPlan P;
    lsa_status st = step_plan(ctx, d, 1, &P);
    if (st != LSA_OK) return st;
    // the rows lsa_decode_step staged: its attention already filled the slots
    return attend_groups(ctx, P, (hipStream_t)stream);
}

lsa_status lsa_decode_step_noalloc(lsa_ctx* ctx, const lsa_step_desc* d, lsa_stream_t stream) {
    if (!ctx) return fail(LSA_ERR_INVALID_ARG, "ctx is NULL");
    if (!ctx->scratch)
        return fail(LSA_ERR_HIP, "device %d: the static scratch has no device address (lookup status %d)",
                    ctx->device, (int)ctx->scratch_status);
    int cur = -1;
    HIPTRY(hipGetDevice(&cur));
    if (cur != ctx->device)
        return fail(LSA_ERR_INVALID_ARG, "the context belongs to device %d but device %d is current", ctx->device, cur);
    StepPlan P;
    lsa_status st = step_plan(ctx, d, 1, &P, static_cast<char*>(ctx->scratch), LSA_STATIC_SCRATCH_BYTES);
    if (st != LSA_OK) return st;
    plan_attention_fetches(&P, d);
    hipStream_t s = (hipStream_t)stream;
    // the select's histogram region must start at zero; the array keeps whatever
    // the previous call on this device left in it
    if (P.zero_clear_words) {
        const size_t n = P.zero_clear_words;
        const unsigned grid = (unsigned)std::min<size_t>((n + 255) / 256, 1024);
        hipLaunchKernelGGL(zero_words_kernel, dim3(grid), dim3(256), 0, s, P.zero_clear, n);
        HIPTRY(hipGetLastError());
    }
    HIPTRY(launch_fm_score(P.sa, d->key_dtype, d->dk, ctx->n_cu, s, ctx->stream_keys));
    HIPTRY(launch_fm_select(P.se, s));
    for (int g = 0; g < P.n_groups; ++g) HIPTRY(launch_kv_stage(P.ga[g], s));
    for (int g = 0; g < P.n_groups; ++g) HIPTRY(launch_lsa_attend(P.aa[g], s));
    return LSA_OK;
}

int32_t lsa_lookahead_buffer(const lsa_ctx* ctx) { return ctx ? ctx->la_cur : 0; }

lsa_status lsa_lookahead_attend(lsa_ctx* ctx, const lsa_step_desc* d, lsa_stream_t stream) {
    StepPlan P;
    lsa_status st = step_plan(ctx, d, 2, &P);
    if (st != LSA_OK) return st;
    plan_use_buffer(&P, ctx->la_cur);
    // the first attention over a prediction's rows reads its missed rows from
    // the cold pools and fills their slots
    if (!ctx->la_fetched) plan_attention_fetches(&P, d);
    st = attend_groups(ctx, P, (hipStream_t)stream);
    if (st != LSA_OK) return st;
    ctx->la_fetched = true;
    return LSA_OK;
}

lsa_status lsa_lookahead_prime(lsa_ctx* ctx, const lsa_step_desc* d, lsa_stream_t stream) {
    StepPlan P;
    lsa_status st = step_plan(ctx, d, 2, &P);
    if (st != LSA_OK) return st;
    if (P.L * P.B > kCopyMaxSegs)
        return fail(LSA_ERR_UNSUPPORTED, "the lookahead schedule handles n_layers * batch <= %d (got %d)", kCopyMaxSegs,
                    P.L * P.B);
    ctx->la_cur = 0;
    ctx->la_fetched = false;
    plan_use_buffer(&P, 0);
    // the first step's rows are staged; its lookahead step copies the missed ones
    return launch_predict(ctx, P, d, (hipStream_t)stream, false);
}

// Step t (rows in buffer cur) and the prediction of step t+1 (into buffer
// nxt), as three or four launches on one stream; see lookahead.hip.
lsa_status lsa_lookahead_step(lsa_ctx* ctx, const lsa_step_desc* d, lsa_stream_t stream) {
    StepPlan P;
    lsa_status st = step_plan(ctx, d, 2, &P);
    if (st != LSA_OK) return st;
    if (P.L * P.B > kCopyMaxSegs)
        return fail(LSA_ERR_UNSUPPORTED, "the lookahead schedule handles n_layers * batch <= %d (got %d)", kCopyMaxSegs,
                    P.L * P.B);
    const int cur = ctx->la_cur, nxt = cur ^ 1;
    hipStream_t s = (hipStream_t)stream;
    plan_use_buffer(&P, cur);
    // the rows step t reads: its recorded misses are copied by the score launch
    // (unless an attention of the window already did)
    const CopyArgs ca = plan_copy(P, cur, !ctx->la_fetched);
    const bool fuse_hist = la_fused_hist(P.sa, P.se, ctx->n_cu);
    bool lists = false;
    {
        Timed t(ctx, LSA_K_SCORE, s);
        HIPTRY(launch_la_fetch_score(P.sa, ca, d->key_dtype, d->dk, ctx->n_cu, fuse_hist ? &P.se : nullptr,
                                     ctx->sel_guess, &lists, s, ctx->stream_keys));
        t.end();
    }
    {
        Timed t(ctx, LSA_K_SELECT, s);
        // with the lists written by the score launch the final selection checks
        // their guess and takes them in place of the collect pass
        SelectArgs se = P.se;
        if (lists) {
            // one list per quarter block
            se.pre = 1;
            se.nblk = P.se.nblk * 4;
            se.blk_stride = kSelColBlk / 4;
        }
        se.guess_out = ctx->sel_guess;
        HIPTRY(launch_la_select_split(P.aa[0], se, fuse_hist, s));
        for (int g = 1; g < P.n_groups; ++g) HIPTRY(launch_attend_splits(P.aa[g], s));
        t.end();
    }
    AttendArgs attend_cur[StepPlan::kMaxGroups];   // the merges of step t's splits
    for (int g = 0; g < P.n_groups; ++g) attend_cur[g] = P.aa[g];
    plan_use_buffer(&P, nxt);
    {
        Timed t(ctx, LSA_K_STAGE, s);
        for (int g = 0; g < P.n_groups; ++g) HIPTRY(launch_la_stage_combine(P.ga[g], attend_cur[g], s));
        t.end();
    }
    ctx->la_cur = nxt;
    ctx->la_fetched = false;
    return LSA_OK;
}

}  // extern "C"

// ------------------------------------------------------------------ KVSwap
namespace {

lsa_status lowrank_args(const void* U, lsa_dtype fdt, int32_t n_seg, int64_t T, int32_t rank, const float* S,
                        const void* V, int32_t C, const float* q, float* scores, LowrankArgs* a,
                        bool scores_optional = false) {
    if (!U || !S || !V || !q || (!scores && !scores_optional))
        return fail(LSA_ERR_INVALID_ARG, "lsa_score_lowrank: NULL pointer");
    if (fdt != LSA_F16) return fail(LSA_ERR_UNSUPPORTED, "factor dtype %d (supported: F16)", (int)fdt);
    if (n_seg < 0 || T < 0) return fail(LSA_ERR_INVALID_ARG, "n_seg %d, T %lld", n_seg, (long long)T);
    if (n_seg > 65535) return fail(LSA_ERR_UNSUPPORTED, "n_seg %d > 65535", n_seg);
    if (rank != 16 && rank != 32 && rank != 64) return fail(LSA_ERR_UNSUPPORTED, "rank %d (supported: 16, 32, 64)", rank);
    if (C < 1 || C > 4096) return fail(LSA_ERR_UNSUPPORTED, "C %d not in [1, 4096]", C);
    if ((uint64_t)T * (uint64_t)rank * 2u >= ((uint64_t)1 << 32)) return fail(LSA_ERR_UNSUPPORTED, "U of a segment exceeds 4 GiB");
    memset(a, 0, sizeof(*a));
    a->U = static_cast<const uint16_t*>(U);
    a->S = S;
    a->V = static_cast<const uint16_t*>(V);
    a->q = q;
    a->scores = scores;
    a->T = T;
    a->n_seg = n_seg;
    a->rank = rank;
    a->C = C;
    a->rows_per_block = 2048;
    return LSA_OK;
}

lsa_status attend_kv_args(const float* q, const void* kv, lsa_dtype dt, int64_t kv_stride_seg, int64_t kv_rows,
                          int32_t heads, int32_t dh, const int32_t* phys, int32_t phys_stride, const int32_t* n_rows,
                          int32_t n_seg, float scale, float* out, AttendKVArgs* a) {
    if (!q || !kv || !phys || !n_rows || !out) return fail(LSA_ERR_INVALID_ARG, "lsa_attend_kv: NULL pointer");
    if (dt != LSA_F16 && dt != LSA_BF16) return fail(LSA_ERR_UNSUPPORTED, "K/V dtype %d (supported: F16, BF16)", (int)dt);
    if (heads < 1 || heads > 8) return fail(LSA_ERR_UNSUPPORTED, "heads %d not in [1, 8]", heads);
    if (dh != 64 && dh != 128) return fail(LSA_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", dh);
    if (n_seg < 0 || phys_stride < 1 || phys_stride > kAttendKVMaxRows || kv_rows < 0 || !isfinite(scale))
        return fail(LSA_ERR_INVALID_ARG, "n_seg %d, phys_stride %d, kv_rows %lld", n_seg, phys_stride, (long long)kv_rows);
    if ((int64_t)(heads + 2) * phys_stride * 4 > 65536)
        return fail(LSA_ERR_UNSUPPORTED, "(heads + 2) * phys_stride = %d exceeds the 16384 words one workgroup keeps in LDS",
                    (heads + 2) * phys_stride);
    const int64_t row_elems = 2LL * heads * dh;
    if ((uint64_t)kv_rows * (uint64_t)row_elems * 2u >= ((uint64_t)1 << 32))
        return fail(LSA_ERR_UNSUPPORTED, "a segment's rows exceed 4 GiB");
    if (n_seg > 1 && kv_stride_seg < kv_rows * row_elems)
        return fail(LSA_ERR_INVALID_ARG, "kv_stride_seg %lld < kv_rows * row elements", (long long)kv_stride_seg);
    memset(a, 0, sizeof(*a));
    a->q = q;
    a->kv = kv;
    a->kv_stride_seg = kv_stride_seg;
    a->kv_rows = kv_rows;
    a->phys = phys;
    a->n_rows = n_rows;
    a->out = out;
    a->phys_stride = phys_stride;
    a->n_seg = n_seg;
    a->heads = heads;
    a->head_dim = dh;
    a->dtype = dt;
    a->scale = scale;
    return LSA_OK;
}

}  // namespace

extern "C" {

lsa_status lsa_score_lowrank(lsa_ctx* ctx, const void* U, lsa_dtype factor_dtype, int32_t n_seg, int64_t T,
                             int32_t rank, const float* S, const void* V, int32_t C, const float* q,
                             float* scores, lsa_stream_t stream) {
    if (!ctx) return fail(LSA_ERR_INVALID_ARG, "ctx is NULL");
    LowrankArgs a;
    lsa_status st = lowrank_args(U, factor_dtype, n_seg, T, rank, S, V, C, q, scores, &a);
    if (st != LSA_OK) return st;
    st = ws_ensure(ctx, align_up((size_t)n_seg * rank * 4, 256));
    if (st != LSA_OK) return st;
    a.p = static_cast<float*>(ctx->ws);
    hipStream_t s = (hipStream_t)stream;
    Timed t(ctx, LSA_K_SCORE, s);
    HIPTRY(launch_lowrank_score(a, s));
    t.end();
    return LSA_OK;
}

lsa_status lsa_attend_kv(lsa_ctx* ctx, const float* q, const void* kv, lsa_dtype dtype, int64_t kv_stride_seg,
                         int64_t kv_rows, int32_t heads, int32_t head_dim, const int32_t* phys,
                         int32_t phys_stride, const int32_t* n_rows, int32_t n_seg, float scale, float* out,
                         lsa_stream_t stream) {
    if (!ctx) return fail(LSA_ERR_INVALID_ARG, "ctx is NULL");
    AttendKVArgs a;
    lsa_status st = attend_kv_args(q, kv, dtype, kv_stride_seg, kv_rows, heads, head_dim, phys, phys_stride, n_rows,
                                   n_seg, scale, out, &a);
    if (st != LSA_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    Timed t(ctx, LSA_K_ATTEND, s);
    HIPTRY(launch_attend_kv(a, s));
    t.end();
    return LSA_OK;
}

lsa_status lsa_kvswap_step(lsa_ctx* ctx, const lsa_kvswap_desc* d, lsa_stream_t stream) {
    if (!ctx || !d) return fail(LSA_ERR_INVALID_ARG, "lsa_kvswap_step: NULL argument");
    if (d->n_pools < 1 || !d->pools || !d->pools[0]) return fail(LSA_ERR_INVALID_ARG, "no pools");
    if (!d->sel || !d->count || !d->phys || !d->n_rows || !d->out)
        return fail(LSA_ERR_INVALID_ARG, "lsa_kvswap_step: NULL pointer in the step");
    const lsa_pool* p0 = d->pools[0];
    const int B = p0->d.batch;
    const int64_t n_seg64 = (int64_t)d->n_pools * B;
    if (n_seg64 > INT32_MAX / 2) return fail(LSA_ERR_UNSUPPORTED, "too many segments");
    const int n_seg = (int)n_seg64;
    const int64_t row_elems = 2LL * d->heads * d->head_dim;
    const int eb = elem_bytes(p0->d.dtype);
    for (int i = 0; i < d->n_pools; ++i) {
        const lsa_pool* p = d->pools[i];
        if (!p) return fail(LSA_ERR_INVALID_ARG, "pool %d is NULL", i);
        if (p->d.batch != B || p->d.dtype != p0->d.dtype || p->d.kv_dim != row_elems || p->d.window != 0 ||
            p->d.ratio != 1 || p->cap != d->T || p->d.kv_stride_b != p0->d.kv_stride_b ||
            p->d.gpu_chunks != p0->d.gpu_chunks)
            return fail(LSA_ERR_INVALID_ARG,
                        "pool %d: needs window 0, ratio 1, compressed_cap T, kv_dim 2*heads*head_dim and the "
                        "batch, dtype, gpu_chunks and kv_stride_b of pool 0", i);
        const char* want = static_cast<const char*>(p0->d.kv_buf) + (int64_t)i * B * p0->d.kv_stride_b * eb;
        if (p->d.kv_buf != want) return fail(LSA_ERR_INVALID_ARG, "pool %d: kv_buf is not pool 0's + %d * batch * kv_stride_b", i, i);
        if (p->swap && p->capacity < d->k)
            return fail(LSA_ERR_SLOTS_LT_TOPK, "pool %d: gpu_chunks (%d) must be >= k (%d)", i, p->capacity, d->k);
    }
    // no scores buffer: score and top-k in one launch per step, the scores never
    // written (a pool that weighs importance needs them, so it needs the buffer)
    const bool fused = d->scores == nullptr;
    if (fused) {
        if (!lowrank_select_fits(d->T, d->rank, d->k))
            return fail(LSA_ERR_UNSUPPORTED, "without a scores buffer the step needs T <= 32768, rank 16/32/64 and "
                        "k <= 1024 (T %lld, rank %d, k %d)", (long long)d->T, d->rank, d->k);
        for (int i = 0; i < d->n_pools; ++i)
            if (d->pools[i]->swap && d->pools[i]->recency_w < 100)
                return fail(LSA_ERR_INVALID_ARG, "pool %d weighs importance (recency weight %d): the step needs "
                            "its scores buffer", i, d->pools[i]->recency_w);
    }
    LowrankArgs la;
    lsa_status st = lowrank_args(d->U, d->factor_dtype, n_seg, d->T, d->rank, d->S, d->V, d->heads * d->head_dim, d->q,
                                 d->scores, &la, fused);
    if (st != LSA_OK) return st;
    if (d->T > INT32_MAX || (uint64_t)d->T * (uint64_t)row_elems * (uint64_t)eb >= ((uint64_t)1 << 32))
        return fail(LSA_ERR_UNSUPPORTED, "T %lld: a sequence's cold rows must stay below 4 GiB", (long long)d->T);
    SelectArgs se;
    size_t sel_need = 0, sel_zero = 0;
    memset(&se, 0, sizeof(se));
    if (!fused) {
        st = select_setup(ctx, d->scores, n_seg, d->T, nullptr, LSA_SELECT_TOPK, d->k, d->k, 0.5, d->sel, d->count,
                          &se, &sel_zero, &sel_need);
        if (st != LSA_OK) return st;
        st = zero_ensure(ctx, sel_zero);
        if (st != LSA_OK) return st;
    } else if (!d->sel || !d->count) {
        return fail(LSA_ERR_INVALID_ARG, "lsa_kvswap_step: NULL sel or count");
    }
    for (int i = 0; i < d->n_pools; ++i) {
        st = stage_check(d->pools[i], d->k, 1, d->k);
        if (st != LSA_OK) return st;
    }
    AttendKVArgs ka;
    st = attend_kv_args(d->q, p0->d.kv_buf, p0->d.dtype, p0->d.kv_stride_b, p0->rows_per_seq, d->heads, d->head_dim,
                        d->phys, d->k, d->n_rows, n_seg, d->scale, d->out, &ka);
    if (st != LSA_OK) return st;
    // workspace: select candidates | p | src | seg_cold
    const size_t off_p = align_up(sel_need, 256);
    const size_t off_src = off_p + align_up((size_t)n_seg * d->rank * 4, 256);
    const size_t off_cold = off_src + align_up((size_t)n_seg * d->k * 4, 256);
    st = ws_ensure(ctx, off_cold + align_up((size_t)n_seg * 8, 256));
    if (st != LSA_OK) return st;
    char* ws = static_cast<char*>(ctx->ws);
    if (!fused) select_bind(&se, ctx->zero, ws);
    la.p = reinterpret_cast<float*>(ws + off_p);
    int32_t* srcs = reinterpret_cast<int32_t*>(ws + off_src);
    uint64_t* seg_cold = reinterpret_cast<uint64_t*>(ws + off_cold);
    // missed rows are read from the cold store by the attention, which also fills their slots
    ka.src = srcs;
    ka.seg_cold = seg_cold;
    ka.cold_rows = d->T;
    // the stage descriptors: the tables (and any allocation or wait they need)
    // are settled before the first launch, so a failure enqueues nothing
    StageLayer* host = nullptr;
    StageLayer* dev = nullptr;
    st = kv_layer_buffer(ctx, d->n_pools, &host, &dev);
    if (st != LSA_OK) return st;
    for (int i = 0; i < d->n_pools; ++i) {
        const size_t seg0 = (size_t)i * B;
        host[i] = stage_layer(d->pools[i], d->sel + seg0 * d->k, d->count + seg0, d->k, 1, d->phys + seg0 * d->k,
                              d->k, d->n_rows + seg0, fused ? nullptr : d->scores + seg0 * d->T, d->T);
        host[i].defer_copy = 1;
        host[i].src = srcs + seg0 * d->k;
        host[i].seg_cold = seg_cold + seg0;
    }
    bool small_pools = d->k <= 512;
    for (int i = 0; i < d->n_pools; ++i) small_pools = small_pools && host[i].S <= 512;

    hipStream_t s = (hipStream_t)stream;
    const int slot = ctx->kv_layers_next;
    HIPTRY(hipMemcpyAsync(dev, host, (size_t)d->n_pools * sizeof(StageLayer), hipMemcpyHostToDevice, s));
    if (fused) {
        Timed t(ctx, LSA_K_SCORE, s);
        HIPTRY(launch_lowrank_select(la, d->k, d->sel, d->count, ctx->n_cu, s));
        t.end();
    } else {
        {
            Timed t(ctx, LSA_K_SCORE, s);
            HIPTRY(launch_lowrank_score(la, s));
            t.end();
        }
        Timed t(ctx, LSA_K_SELECT, s);
        HIPTRY(launch_fm_select(se, s));
        t.end();
    }
    int max_slots = 0;
    for (int i = 0; i < d->n_pools; ++i) max_slots = host[i].S > max_slots ? host[i].S : max_slots;
    if (small_pools && stage_attend_kv_fits(d->heads, d->head_dim, d->k, max_slots)) {
        // each segment's stage and attention in one workgroup
        Timed t(ctx, LSA_K_ATTEND, s);
        HIPTRY(launch_stage_attend_kv(dev, B, ka, s));
        t.end();
        HIPTRY(hipEventRecord(ctx->kv_layers_done[slot], s));
        ctx->kv_layers_next = slot ^ 1;
        return LSA_OK;
    }
    {
        Timed t(ctx, LSA_K_STAGE, s);
        HIPTRY(launch_kv_stage_table(dev, d->n_pools, B, small_pools, s));
        t.end();
        // the pair is free again once this stage has run
        HIPTRY(hipEventRecord(ctx->kv_layers_done[slot], s));
        ctx->kv_layers_next = slot ^ 1;
    }
    {
        Timed t(ctx, LSA_K_ATTEND, s);
        HIPTRY(launch_attend_kv(ka, s));
        t.end();
    }
    return LSA_OK;
}

}  // extern "C"
