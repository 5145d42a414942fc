// Plain CPU oracle of the LSA decode hot path (score -> select -> stage ->
// attend) and of KVSwap's grouped low-rank prediction.
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
// or calls this file; only the test-suite, the package smoke check and the
// benchmark's CPU-baseline leg load it (through oracle/__init__.py).  It shares
// no code, header, table or constant with the HIP library.
//
// Every step is written the slow, obvious way: double accumulation, one entry
// at a time, std::stable_sort for ordering, and for the slot pool the literal
// structure of page 1 (a std::list LRU plus an unordered_map).  Each function
// names the passage of the source pages it follows.  The pages are:
//   [P1] "FlashMemory 1M 上下文显存优化使用文档" (PocketLLM performance doc)
//   [P2] article on "FlashMemory-DeepSeek-V4: Lightning Index Ultra-Long
//        Context via Lookahead Sparse Attention"
//   [P4] "KVSwap：大模型推理中的KV缓存优化技术"
// Where the pages leave a step open, the reading taken is stated inline.
//
// Build: g++ -std=c++17 -O2 -shared -fPIC lsa_oracle.cpp -o liblsa_oracle.so

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <list>
#include <numeric>
#include <set>
#include <unordered_map>
#include <vector>

namespace {

enum { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2, DT_FP8_E4M3 = 3, DT_MXFP4 = 4, DT_MXINT8 = 5 };
enum { ENS_MAX = 0, ENS_MEAN = 1 };
enum { SEL_TOPK = 0, SEL_THRESHOLD = 1 };
enum { ST_OK = 0, ST_NOT_STORED = 4 };

// IEEE binary16 -> double, from the format's definition (1 sign, 5 exponent
// bits with bias 15, 10 fraction bits; exponent 0 = subnormal).
double half_to_double(uint16_t h) {
    const int sign = h >> 15;
    const int expo = (h >> 10) & 31;
    const int frac = h & 1023;
    double v;
    if (expo == 0) {
        v = std::ldexp((double)frac, -24);
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = std::ldexp((double)(1024 + frac), expo - 25);
    }
    return sign ? -v : v;
}

// bfloat16 is the upper half of an IEEE binary32.
double bf16_to_double(uint16_t b) {
    const uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// OCP 8-bit E4M3 -> double, from the format's definition (1 sign, 4 exponent
// bits with bias 7, 3 fraction bits; exponent 0 = subnormal, frac * 2^-9; no
// infinities, and exponent 15 with fraction 7 is NaN).  [P1] technical details
// (known limits) names fp8 indexer keys as the next step after fp4.
double fp8_e4m3_to_double(uint8_t c) {
    const int sign = c >> 7;
    const int expo = (c >> 3) & 15;
    const int frac = c & 7;
    double v;
    if (expo == 0) {
        v = std::ldexp((double)frac, -9);
    } else if (expo == 15 && frac == 7) {
        v = NAN;
    } else {
        v = std::ldexp((double)(8 + frac), expo - 10);
    }
    return sign ? -v : v;
}

// OCP MX FP4 element (E2M1) -> double, from the format's definition: 1 sign,
// 2 exponent bits with bias 1, 1 mantissa bit; exponent 0 is subnormal
// (mantissa * 0.5); no infinities or NaN.
double e2m1_to_double(uint8_t nib) {
    const int sign = (nib >> 3) & 1;
    const int expo = (nib >> 1) & 3;
    const int man = nib & 1;
    const double v = expo == 0 ? 0.5 * man : std::ldexp(1.0 + 0.5 * man, expo - 1);
    return sign ? -v : v;
}

// OCP MX scale (E8M0) -> double: 2^(s - 127); 255 is NaN.
double e8m0_to_double(uint8_t s) { return s == 255 ? NAN : std::ldexp(1.0, (int)s - 127); }

double elem(const void* base, int dtype, int64_t i);

// Element t of key j (a row of dk elements) in key_dtype.  The MX formats
// ([P1] technical details: the reference's own keys are fp4) multiply each
// code by the E8M0 scale of its block of 32 consecutive elements
// (scales [.][dk/32]); MX INT8 codes carry an implicit 2^-6.
double key_elem(const void* keys, const uint8_t* scales, int dtype, int32_t dk, int64_t j, int32_t t) {
    if (dtype == DT_MXFP4) {
        const uint8_t byte = static_cast<const uint8_t*>(keys)[j * (dk / 2) + t / 2];
        const uint8_t nib = (t & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
        return e2m1_to_double(nib) * e8m0_to_double(scales[j * (dk / 32) + t / 32]);
    }
    if (dtype == DT_MXINT8) {
        const int8_t c = static_cast<const int8_t*>(keys)[j * dk + t];
        return (double)c / 64.0 * e8m0_to_double(scales[j * (dk / 32) + t / 32]);
    }
    return elem(keys, dtype, j * dk + t);
}

double elem(const void* base, int dtype, int64_t i) {
    if (dtype == DT_FP8_E4M3) return fp8_e4m3_to_double(((const uint8_t*)base)[i]);
    if (dtype == DT_F32) {
        float f;
        std::memcpy(&f, (const char*)base + 4 * i, 4);
        return f;
    }
    uint16_t h;
    std::memcpy(&h, (const char*)base + 2 * i, 2);
    return dtype == DT_BF16 ? bf16_to_double(h) : half_to_double(h);
}

// Total order of the selector: higher score first, lower index first among
// equal scores.  Reading: the pages give no tie rule; the lowest index wins.
// -0 and +0 compare equal here, so they tie.
struct ByScoreThenIndex {
    const float* e;
    bool operator()(int32_t a, int32_t b) const {
        if (e[a] != e[b]) return e[a] > e[b];
        return a < b;
    }
};

}  // namespace

extern "C" {

// ---------------------------------------------------------------- sizing ---
// [P1] "POCKETLLM_GGUF_KV_SWAP_PINNED_MIB" tuning section: per layer
// compressed_cap = (context_length + ratio - 1) / ratio and the pinned bytes
// are the sum over sparse layers of compressed_cap * kv_dim * sizeof(element).
int64_t oracle_compressed_cap(int64_t ctx, int32_t ratio) {
    return (ctx + ratio - 1) / ratio;
}

uint64_t oracle_pinned_bytes(int64_t ctx, const int32_t* ratios, int32_t n_layers,
                             int32_t kv_dim, int32_t elem_bytes) {
    uint64_t total = 0;
    for (int32_t l = 0; l < n_layers; ++l)
        total += (uint64_t)oracle_compressed_cap(ctx, ratios[l]) * (uint64_t)kv_dim *
                 (uint64_t)elem_bytes;
    return total;
}

// [P1] expected-log section: max_capacity = window(128) + gpu_chunks(512).
int32_t oracle_max_capacity(int32_t window, int32_t gpu_chunks) { return window + gpu_chunks; }

// [P1] troubleshooting, "gguf_kv_swap=0 reason=no_layer_with_compressed_cap_gt_gpu_chunks":
// a layer whose compressed_cap <= gpu_chunks is kept fully resident (no swap).
int32_t oracle_swap_enabled(int64_t cap, int32_t gpu_chunks) { return cap > gpu_chunks ? 1 : 0; }

// ------------------------------------------------------------ projection ---
// [P1] architecture overview: the decode token's hidden state (hidden[4096])
// feeds the three scorers.  Reading (the pages give no formula): every
// indexer i maps the hidden vector linearly to its H query heads and its H
// head weights,
//     q[i,h,t] = sum_c Wq[i,h,t,c] * hidden[c],   w[i,h] = sum_c Ww[i,h,c] * hidden[c],
// summed in double and rounded once to float.
// hidden: [B][d_model] f32; wq: [n_idx][H][dk][d_model] and ww: [n_idx][H][d_model]
// in w_dtype; q: [B][n_idx][H][dk]; w: [B][n_idx][H].
void oracle_project(const float* hidden, int32_t B, int32_t d_model, const void* wq, const void* ww,
                    int32_t w_dtype, int32_t n_idx, int32_t H, int32_t dk, float* q, float* w) {
    const int64_t q_rows = (int64_t)n_idx * H * dk, w_rows = (int64_t)n_idx * H;
    for (int32_t b = 0; b < B; ++b) {
        const float* x = hidden + (int64_t)b * d_model;
        for (int64_t r = 0; r < q_rows; ++r) {
            double acc = 0.0;
            for (int32_t c = 0; c < d_model; ++c) acc += elem(wq, w_dtype, r * d_model + c) * (double)x[c];
            q[(int64_t)b * q_rows + r] = (float)acc;
        }
        for (int64_t r = 0; r < w_rows; ++r) {
            double acc = 0.0;
            for (int32_t c = 0; c < d_model; ++c) acc += elem(ww, w_dtype, r * d_model + c) * (double)x[c];
            w[(int64_t)b * w_rows + r] = (float)acc;
        }
    }
}

// ----------------------------------------------------------------- score ---
// [P1] architecture overview: the hidden state feeds 3 scorers which read the
// shared indexer_kv_cache and are combined by an ensemble (max or mean).
// [P2] "LSA 让模型预判 KV chunk": memory-indexer queries are matched against the
// compressed indexer keys by dot-product similarity.
// Reading (the pages give no head formula): indexer i scores entry j as
//     s_i[j] = sum_h w[i,h] * ReLU( q[i,h,:] . key[j,:] )
// kept as a float; the max ensemble takes the largest s_i[j], the mean ensemble
// rounds the sum of the float s_i[j] to float and divides once by n_idx in
// IEEE single precision.  -0 is written as +0.
//
// keys: [n_valid][dk] elements in key_dtype (with key_scales [n_valid][dk/32]
// for the MX formats, else unused); q: [n_idx][H][dk]; w: [n_idx][H]; e: [n_valid].
void oracle_score(const void* keys, int32_t key_dtype, const uint8_t* key_scales, int64_t n_valid, int32_t dk,
                  const float* q, const float* w, int32_t n_idx, int32_t H,
                  int32_t ensemble, float* e) {
    std::vector<double> key(dk);
    std::vector<float> s(n_idx);
    for (int64_t j = 0; j < n_valid; ++j) {
        for (int32_t t = 0; t < dk; ++t) key[t] = key_elem(keys, key_scales, key_dtype, dk, j, t);
        for (int32_t i = 0; i < n_idx; ++i) {
            double acc = 0.0;
            for (int32_t h = 0; h < H; ++h) {
                const float* qh = q + ((int64_t)i * H + h) * dk;
                double d = 0.0;
                for (int32_t t = 0; t < dk; ++t) d += (double)qh[t] * key[t];
                const double relu = d > 0.0 ? d : 0.0;
                acc += (double)w[(int64_t)i * H + h] * relu;
            }
            s[i] = (float)acc + 0.0f;
        }
        float r;
        if (ensemble == ENS_MAX) {
            r = s[0];
            for (int32_t i = 1; i < n_idx; ++i)
                if (s[i] > r) r = s[i];
        } else {
            double sum = 0.0;
            for (int32_t i = 0; i < n_idx; ++i) sum += (double)s[i];
            const float sum_f = (float)sum;
            r = sum_f / (float)n_idx;
        }
        e[j] = r + 0.0f;
    }
}

// ---------------------------------------------------------------- select ---
// [P2] "Recall / Threshold Selector": an entry is recalled when the sigmoid of
// its score exceeds a threshold tau.  Over the reals sigmoid(e) > tau holds
// exactly when e > logit(tau) = ln(tau / (1 - tau)); for a float e that is
// e > t_f with t_f the largest float not above logit(tau).
float oracle_threshold_float(double tau) {
    const double t = std::log(tau / (1.0 - tau));
    float tf = (float)t;
    if ((double)tf > t) tf = std::nextafterf(tf, -INFINITY);
    return tf;
}

// Top-k mode: [P1] "global top-k (512 chunks)", index_topk = global_keep_cap.
// Threshold mode: [P2] sigmoid threshold, capped at k ([P1] log line
// "global_keep_cap=512").  Reading: when more than k entries pass, the first k
// of the total order are kept; fewer than k valid entries means all of them.
// The selected indices are returned in ascending order.
int32_t oracle_select(const float* e, int64_t n_valid, int32_t mode, int32_t k, double tau,
                      int32_t* sel) {
    std::vector<int32_t> order(n_valid);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), ByScoreThenIndex{e});

    std::vector<int32_t> chosen;
    if (mode == SEL_TOPK) {
        for (int64_t r = 0; r < n_valid && (int64_t)chosen.size() < k; ++r)
            chosen.push_back(order[r]);
    } else {
        const float tf = oracle_threshold_float(tau);
        std::vector<int32_t> pass;
        for (int64_t r = 0; r < n_valid; ++r)
            if (e[order[r]] > tf) pass.push_back(order[r]);
        for (size_t r = 0; r < pass.size() && (int64_t)chosen.size() < k; ++r)
            chosen.push_back(pass[r]);
    }
    std::sort(chosen.begin(), chosen.end());
    std::copy(chosen.begin(), chosen.end(), sel);
    return (int32_t)chosen.size();
}

// ------------------------------------------------------------- ratio map ---
// [P1] FlashMemory vs native indexer table and the log line "source_ratio=4":
// one global selection over the ratio-4 source layer is reused by every sparse
// layer, including the ratio-128 ones.  Reading (the pages do not say how):
// source entry j covers tokens [j*r_src, (j+1)*r_src), which lie in entry
// floor(j*r_src / r_layer) of a layer whose ratio is a multiple of r_src; the
// layer's list is the ascending set of those entries, duplicates removed.
// [P1] store flow: the compressor emits a layer's chunk once its r_layer
// tokens exist.  Reading: with src_valid source entries (tokens
// [0, src_valid*r_src) compressed), a layer entry m whose last token
// (m+1)*r_layer - 1 lies beyond them does not exist yet and is left out of the
// list; its tokens are all among the newest r_layer - 1 and so inside the
// 128-row sliding window.
int32_t oracle_ratio_map(const int32_t* sel, int32_t count, int32_t src_ratio,
                         int32_t layer_ratio, int64_t src_valid, int32_t* out) {
    std::set<int64_t> s;
    const int64_t tokens = src_valid * (int64_t)src_ratio;
    for (int32_t i = 0; i < count; ++i) {
        const int64_t m = (int64_t)sel[i] * src_ratio / layer_ratio;
        const int64_t last_token = (m + 1) * (int64_t)layer_ratio - 1;
        if (last_token < tokens) s.insert(m);
    }
    int32_t n = 0;
    for (int64_t v : s) out[n++] = (int32_t)v;
    return n;
}

// ----------------------------------------------------------------- stage ---
// [P1] "KV_SWAP 实现细节": the per-layer state is this struct, and swap-in of
// the selected logical IDs works per ID: a hit touches the entry (moves it to
// the LRU front) and counts a hit; a miss evicts the LRU back (pop_back),
// takes that slot, copies the host row into it and counts a miss; the ID is
// then rewritten to the physical row window + slot.  A selected chunk that was
// never stored is an error ("selected chunk before it was stored").
// Readings: (a) the doc gives no order among the IDs of one step: hits are
// processed first, then misses, each group in ascending logical order, so a
// step never evicts a chunk it selected; (b) while a slot was never used, a
// miss takes the lowest-numbered unused slot instead of evicting.
struct OracleSwapLayerState {
    int64_t compressed_cap;
    int32_t gpu_chunks;
    int32_t window;
    int64_t row_bytes;
    std::vector<uint8_t> host_ready;          // [compressed_cap]
    std::vector<int> gpu_slot_logical;        // [gpu_chunks], -1 = unused
    std::unordered_map<int, int> slot_by_logical;
    std::list<int> slot_lru;                  // slot ids, front = most recently used
    uint64_t hits = 0, misses = 0, h2d_bytes = 0, d2h_bytes = 0;
    int32_t capacity;                         // slots in use at most (adaptive GPU_CHUNKS)
    uint64_t last_hits = 0, last_misses = 0, last_h2d = 0;   // counters at the last adapt
    int32_t recency_weight = 100;             // replacement weighting, percent (100 = plain LRU)
    int32_t high_water = 100;                 // percent of the capacity kept in use at most after a step
};

void* oracle_pool_new(int64_t cap, int32_t gpu_chunks, int32_t window, int64_t row_bytes) {
    auto* p = new OracleSwapLayerState;
    p->compressed_cap = cap;
    p->gpu_chunks = gpu_chunks;
    p->window = window;
    p->row_bytes = row_bytes;
    p->host_ready.assign(cap, 0);
    p->gpu_slot_logical.assign(gpu_chunks, -1);
    p->capacity = gpu_chunks;
    return p;
}

void oracle_pool_free(void* pool) { delete static_cast<OracleSwapLayerState*>(pool); }

// [P1] store flow: the row is copied device-to-host and host_ready is set.
void oracle_pool_store(void* pool, int64_t first, int64_t count) {
    auto* p = static_cast<OracleSwapLayerState*>(pool);
    for (int64_t l = first; l < first + count; ++l) p->host_ready[l] = 1;
    p->d2h_bytes += (uint64_t)count * (uint64_t)p->row_bytes;
}

// [P4] §3.2 (rolling buffer): the replacement weighs LRU order with the
// entries' importance scores, and a prefetch is triggered at 70 % buffer
// utilisation.  The page gives neither formula.  Readings:
//  * the candidates for eviction are the entries resident when the step starts
//    and not selected by it.  Each gets a recency rank a (0 = least recently
//    used, in LRU order) and an importance rank c (0 = lowest importance -- the
//    step's prediction score of that entry --, equal scores ranked by a), and
//    candidates are evicted in ascending order of w*a + (100-w)*c, equal values
//    by a, where w is the recency weight in percent (100 = plain LRU);
//  * with a high-water mark h percent below 100, a step that leaves more than
//    max(floor(h * capacity / 100), its own entries) slots in use evicts the
//    next candidates in the same order down to that count: the freed slots are
//    where the next step's misses land, without an eviction.
// w and h are set per pool; with both at 100 the stage below is the page's
// plain LRU loop.
void oracle_pool_set_replacement(void* pool, int32_t recency_weight, int32_t high_water) {
    auto* p = static_cast<OracleSwapLayerState*>(pool);
    p->recency_weight = recency_weight;
    p->high_water = high_water;
}

// sel: ascending unique logical IDs of this layer (n of them).
// importance: the step's score of every logical ID ([compressed_cap]); read
// only when the pool weighs its replacement (may be NULL otherwise).
// phys: [window + n]; rows 0..window-1 are the window, then one row per ID.
// miss_logical / miss_slot: [n]; the misses in processing order.
// Returns 0, or 4 when a selected ID was never stored (nothing is changed then).
int32_t oracle_pool_stage(void* pool, const int32_t* sel, int32_t n, const float* importance, int32_t* phys,
                          int32_t* miss_logical, int32_t* miss_slot, int32_t* n_miss) {
    auto* p = static_cast<OracleSwapLayerState*>(pool);
    for (int32_t i = 0; i < n; ++i)
        if (!p->host_ready[sel[i]]) return ST_NOT_STORED;
    for (int32_t r = 0; r < p->window; ++r) phys[r] = r;
    *n_miss = 0;
    if (p->compressed_cap <= p->gpu_chunks) {   // swap disabled: fully resident
        for (int32_t i = 0; i < n; ++i) phys[p->window + i] = p->window + sel[i];
        return ST_OK;
    }
    // eviction order of this step's candidates (resident and not selected)
    std::set<int32_t> selected(sel, sel + n);
    std::vector<int> cand;                      // slots, least recently used first
    for (auto it = p->slot_lru.rbegin(); it != p->slot_lru.rend(); ++it)
        if (!selected.count(p->gpu_slot_logical[*it])) cand.push_back(*it);
    std::vector<int> evict_order(cand.size());
    std::iota(evict_order.begin(), evict_order.end(), 0);   // indices into cand = recency ranks
    if (p->recency_weight < 100) {
        std::vector<int> by_imp(cand.size());
        std::iota(by_imp.begin(), by_imp.end(), 0);
        std::stable_sort(by_imp.begin(), by_imp.end(), [&](int x, int y) {
            return importance[p->gpu_slot_logical[cand[x]]] < importance[p->gpu_slot_logical[cand[y]]];
        });
        std::vector<int64_t> prio(cand.size());
        for (size_t c = 0; c < by_imp.size(); ++c) {
            const int a = by_imp[c];
            prio[a] = (int64_t)p->recency_weight * a + (int64_t)(100 - p->recency_weight) * (int64_t)c;
        }
        std::stable_sort(evict_order.begin(), evict_order.end(), [&](int x, int y) { return prio[x] < prio[y]; });
    }
    size_t next_victim = 0;
    std::vector<int32_t> missed;
    for (int32_t i = 0; i < n; ++i) {           // hits, ascending
        auto it = p->slot_by_logical.find(sel[i]);
        if (it == p->slot_by_logical.end()) {
            missed.push_back(sel[i]);
            continue;
        }
        const int slot = it->second;
        p->slot_lru.remove(slot);
        p->slot_lru.push_front(slot);
        p->hits++;
    }
    for (int32_t l : missed) {                  // misses, ascending
        int slot = -1;
        for (int s = 0; s < p->capacity; ++s)
            if (p->gpu_slot_logical[s] < 0) { slot = s; break; }
        if (slot < 0) {
            slot = cand[evict_order[next_victim++]];
            p->slot_lru.remove(slot);
            p->slot_by_logical.erase(p->gpu_slot_logical[slot]);
        }
        p->gpu_slot_logical[slot] = l;
        p->slot_by_logical[l] = slot;
        p->slot_lru.push_front(slot);
        p->misses++;
        p->h2d_bytes += (uint64_t)p->row_bytes;
        miss_logical[*n_miss] = l;
        miss_slot[*n_miss] = slot;
        (*n_miss)++;
    }
    // the high-water mark: free slots for the next step's misses
    if (p->high_water < 100) {
        const int64_t limit = std::max<int64_t>((int64_t)p->high_water * p->capacity / 100, n);
        while ((int64_t)p->slot_lru.size() > limit && next_victim < cand.size()) {
            const int slot = cand[evict_order[next_victim++]];
            p->slot_lru.remove(slot);
            p->slot_by_logical.erase(p->gpu_slot_logical[slot]);
            p->gpu_slot_logical[slot] = -1;
        }
    }
    for (int32_t i = 0; i < n; ++i) phys[p->window + i] = p->window + p->slot_by_logical[sel[i]];
    return ST_OK;
}

// [P1] limitations, future work: adaptive GPU_CHUNKS, the staging capacity
// adjusted from the runtime LRU hit rate.  The pages give no procedure.
// Reading: the capacity is the number of slots the pool may use (at most
// gpu_chunks).  Growing makes more slots available (a miss still takes the
// lowest unused slot).  Shrinking to C evicts least recently used entries
// (pop_back) until at most C remain, then moves every remaining entry whose
// slot is >= C to the lowest vacated slot below C, taking both lists in
// ascending slot order; its row moves with it and the LRU order is unchanged.
// A pool whose swap is disabled ignores the capacity.
void oracle_pool_set_capacity(void* pool, int32_t C) {
    auto* p = static_cast<OracleSwapLayerState*>(pool);
    p->capacity = C;
    if (p->compressed_cap <= p->gpu_chunks) return;
    while ((int32_t)p->slot_lru.size() > C) {
        const int slot = p->slot_lru.back();
        p->slot_lru.pop_back();
        p->slot_by_logical.erase(p->gpu_slot_logical[slot]);
        p->gpu_slot_logical[slot] = -1;
    }
    std::vector<int> high, vacated;
    for (int s = C; s < p->gpu_chunks; ++s)
        if (p->gpu_slot_logical[s] >= 0) high.push_back(s);
    for (int s = 0; s < C; ++s)
        if (p->gpu_slot_logical[s] < 0) vacated.push_back(s);
    for (size_t i = 0; i < high.size(); ++i) {
        const int from = high[i], to = vacated[i];
        const int l = p->gpu_slot_logical[from];
        p->gpu_slot_logical[to] = l;
        p->gpu_slot_logical[from] = -1;
        p->slot_by_logical[l] = to;
        for (int& e : p->slot_lru)
            if (e == from) e = to;
    }
}

int32_t oracle_pool_capacity(void* pool) { return static_cast<OracleSwapLayerState*>(pool)->capacity; }

// [P1] troubleshooting: a miss rate above 50 % or more than 10 MB of H2D per
// step calls for a larger GPU_CHUNKS; [P1] tuning: a smaller one saves memory
// at more misses.  Reading of the adaptive policy: over the steps since the
// last call, grow by `step` slots (up to max_c) when the miss rate exceeds
// grow_miss or the H2D bytes per step exceed grow_h2d; otherwise shrink by
// `step` (down to min_c) when the miss rate is below shrink_miss; no lookups,
// no change.  Returns the new capacity.
int32_t oracle_pool_adapt(void* pool, double grow_miss, double grow_h2d, double shrink_miss, int32_t step,
                          int32_t min_c, int32_t max_c, int32_t steps) {
    auto* p = static_cast<OracleSwapLayerState*>(pool);
    const uint64_t h = p->hits - p->last_hits, m = p->misses - p->last_misses, x = p->h2d_bytes - p->last_h2d;
    p->last_hits = p->hits;
    p->last_misses = p->misses;
    p->last_h2d = p->h2d_bytes;
    int32_t C = p->capacity;
    if (h + m > 0) {
        const double miss_rate = (double)m / (double)(h + m);
        const double h2d_per_step = (double)x / (double)(steps > 0 ? steps : 1);
        if (miss_rate > grow_miss || h2d_per_step > grow_h2d)
            C = std::min(max_c, C + step);
        else if (miss_rate < shrink_miss)
            C = std::max(min_c, C - step);
    }
    if (C != p->capacity) oracle_pool_set_capacity(pool, C);
    return C;
}

// stats: hits, misses, h2d_bytes, d2h_bytes
void oracle_pool_stats(void* pool, uint64_t* out) {
    auto* p = static_cast<OracleSwapLayerState*>(pool);
    out[0] = p->hits;
    out[1] = p->misses;
    out[2] = p->h2d_bytes;
    out[3] = p->d2h_bytes;
}

// slot_logical: [gpu_chunks] logical ID held by each slot (-1 unused);
// lru: slot ids from most to least recently used; returns their number.
int32_t oracle_pool_state(void* pool, int32_t* slot_logical, int32_t* lru) {
    auto* p = static_cast<OracleSwapLayerState*>(pool);
    for (int s = 0; s < p->gpu_chunks; ++s) slot_logical[s] = p->gpu_slot_logical[s];
    int32_t n = 0;
    for (int s : p->slot_lru) lru[n++] = s;
    return n;
}

// ---------------------------------------------------------------- attend ---
// [P1] "Two-tier KV cache" and the per-layer sparse attention
// (indexed_cached_attention over window + selected): one decode query per head
// attends over the window rows and then the selected compressed entries.
// Readings: each compressed entry serves as both key and value (kv_dim 512);
// softmax(scale * q.row) with no mask and no sink; rows are taken in list order
// (window 0..W-1, then the selected entries in ascending logical order), read
// from the full store by logical ID -- staging only moves rows, so this is also
// the answer with swapping switched off.  With no rows the output is 0.
//
// q: [Hq][D] f32; window: [W][D]; store: [cap][D] (kv_dtype); sel: [n]; out: [Hq][D].
void oracle_attend(const float* q, int32_t Hq, int32_t D, const void* window, int32_t W,
                   const void* store, int32_t kv_dtype, const int32_t* sel, int32_t n,
                   float scale, float* out) {
    const int32_t rows = W + n;
    std::vector<double> kv((size_t)rows * D);
    for (int32_t r = 0; r < rows; ++r)
        for (int32_t d = 0; d < D; ++d)
            kv[(size_t)r * D + d] = r < W ? elem(window, kv_dtype, (int64_t)r * D + d)
                                          : elem(store, kv_dtype, (int64_t)sel[r - W] * D + d);
    std::vector<double> z(rows);
    for (int32_t h = 0; h < Hq; ++h) {
        if (rows == 0) {
            for (int32_t d = 0; d < D; ++d) out[(size_t)h * D + d] = 0.0f;
            continue;
        }
        double m = -INFINITY;
        for (int32_t r = 0; r < rows; ++r) {
            double dot = 0.0;
            for (int32_t d = 0; d < D; ++d) dot += (double)q[(size_t)h * D + d] * kv[(size_t)r * D + d];
            z[r] = (double)scale * dot;
            m = std::max(m, z[r]);
        }
        double den = 0.0;
        for (int32_t r = 0; r < rows; ++r) {
            z[r] = std::exp(z[r] - m);
            den += z[r];
        }
        for (int32_t d = 0; d < D; ++d) {
            double num = 0.0;
            for (int32_t r = 0; r < rows; ++r) num += z[r] * kv[(size_t)r * D + d];
            out[(size_t)h * D + d] = (float)(num / den);
        }
    }
}

// ------------------------------------------------------- KVSwap variant ---
// [P4] §2.3.1-2.3.2: K is kept as low-rank factors K ~ U diag(S) V^T and
// rebuilt on demand (reconstruct_K = U @ diag(S) @ V.T); §2.2.1: the
// prediction scores are q @ K^T followed by top-k with k = MG = 400; §2.2.2:
// heads are grouped (G = 4) and a group shares one selection.
// Reading: a group's key at position t is the concatenation of its heads'
// keys (width C = G * head_dim); its query is the concatenation of the heads'
// queries; score[t] = q . K[t,:] with K[t,:] = sum_x U[t,x] S[x] V[:,x].
//
// U: [T][r] f16; S: [r] f32; V: [C][r] f16; q: [C] f32; score: [T].
void oracle_lowrank_score(const uint16_t* U, int64_t T, int32_t r, const float* S,
                          const uint16_t* V, int32_t C, const float* q, float* score) {
    std::vector<double> krow(C);
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t c = 0; c < C; ++c) {
            double k = 0.0;
            for (int32_t x = 0; x < r; ++x)
                k += half_to_double(U[t * r + x]) * (double)S[x] * half_to_double(V[(int64_t)c * r + x]);
            krow[c] = k;
        }
        double dot = 0.0;
        for (int32_t c = 0; c < C; ++c) dot += (double)q[c] * krow[c];
        score[t] = (float)dot + 0.0f;
    }
}

// Per-head attention of the KVSwap variant over separate full-precision K and
// V rows of the selected positions (no window).  K, V: position p of this head
// starts at element p * row_stride; q: [dh]; out: [dh].
void oracle_attend_kv(const float* q, int32_t dh, const void* K, const void* V, int32_t kv_dtype,
                      int64_t row_stride, const int32_t* pos, int32_t n, float scale, float* out) {
    if (n == 0) {
        for (int32_t d = 0; d < dh; ++d) out[d] = 0.0f;
        return;
    }
    std::vector<double> z(n);
    double m = -INFINITY;
    for (int32_t i = 0; i < n; ++i) {
        double dot = 0.0;
        for (int32_t d = 0; d < dh; ++d)
            dot += (double)q[d] * elem(K, kv_dtype, (int64_t)pos[i] * row_stride + d);
        z[i] = (double)scale * dot;
        m = std::max(m, z[i]);
    }
    double den = 0.0;
    for (int32_t i = 0; i < n; ++i) {
        z[i] = std::exp(z[i] - m);
        den += z[i];
    }
    for (int32_t d = 0; d < dh; ++d) {
        double num = 0.0;
        for (int32_t i = 0; i < n; ++i) num += z[i] * elem(V, kv_dtype, (int64_t)pos[i] * row_stride + d);
        out[d] = (float)(num / den);
    }
}

}  // extern "C"
