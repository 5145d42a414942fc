// Drives every entry point of the CPU oracle on small random inputs, built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_oracle_sanitize.py.
// Any out-of-bounds access, use after free, leak, signed overflow or misaligned
// access aborts the run.  Test infrastructure only.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "../oracle/lsa_oracle.cpp"

namespace {
std::mt19937 rng(12345);
float grid() { return (float)((int)(rng() % 17) - 8) / 8.0f; }
int below(int n) { return (int)(rng() % (unsigned)n); }
}  // namespace

int main() {
    // sizing
    const int32_t ratios[3] = {4, 128, 4};
    volatile uint64_t sink = oracle_pinned_bytes(8192, ratios, 3, 512, 4) + oracle_compressed_cap(1000, 7) +
                             oracle_max_capacity(128, 512) + oracle_swap_enabled(16, 8);
    (void)sink;
    // projection
    const int B = 2, dm = 32, ni = 2, H = 3, dk = 8;
    std::vector<float> hid(B * dm), wq(ni * H * dk * dm), ww(ni * H * dm), q(B * ni * H * dk), w(B * ni * H);
    for (auto& x : hid) x = grid();
    for (auto& x : wq) x = grid();
    for (auto& x : ww) x = grid();
    oracle_project(hid.data(), B, dm, wq.data(), ww.data(), 0, ni, H, dk, q.data(), w.data());
    // score in every key format
    const int N = 300;
    std::vector<float> keys(N * dk);
    for (auto& x : keys) x = grid();
    std::vector<uint8_t> codes(N * dk), scales(N * (dk / 32 + 1));
    for (auto& c : codes) c = (uint8_t)below(120);
    for (auto& s : scales) s = (uint8_t)(120 + below(8));
    std::vector<float> e(N);
    for (int ens = 0; ens < 2; ++ens) {
        oracle_score(keys.data(), 0, nullptr, N, dk, q.data(), w.data(), ni, H, ens, e.data());
        oracle_score(codes.data(), 3, nullptr, N, dk, q.data(), w.data(), ni, H, ens, e.data());
    }
    const int dk32 = 32;
    std::vector<float> q32(ni * H * dk32), w32(ni * H);
    for (auto& x : q32) x = grid();
    for (auto& x : w32) x = grid();
    std::vector<uint8_t> c4(N * dk32 / 2), c8(N * dk32), sc(N);
    for (auto& c : c4) c = (uint8_t)below(256);
    for (auto& c : c8) c = (uint8_t)below(128);
    for (auto& s : sc) s = (uint8_t)(124 + below(3));
    oracle_score(c4.data(), 4, sc.data(), N, dk32, q32.data(), w32.data(), ni, H, 0, e.data());
    oracle_score(c8.data(), 5, sc.data(), N, dk32, q32.data(), w32.data(), ni, H, 1, e.data());
    // select and the ratio map
    std::vector<int32_t> sel(64), lsel(64);
    int32_t n = oracle_select(e.data(), N, 0, 64, 0.5, sel.data());
    n = oracle_select(e.data(), N, 1, 64, 0.7, sel.data());
    n = oracle_select(e.data(), N, 0, 40, 0.5, sel.data());
    const int32_t nl = oracle_ratio_map(sel.data(), n, 4, 128, N, lsel.data());
    (void)oracle_threshold_float(0.3);
    // pools: plain, weighted with a high-water mark, capacity changes
    for (int mode = 0; mode < 3; ++mode) {
        const int cap = 200, S = 48, W = 4;
        void* p = oracle_pool_new(cap, S, W, 64);
        oracle_pool_store(p, 0, 150);
        if (mode == 1) oracle_pool_set_replacement(p, 50, 70);
        if (mode == 2) oracle_pool_set_replacement(p, 0, 40);
        std::vector<float> imp(cap);
        std::vector<int32_t> phys(W + 64), ml(64), ms(64), sl(S), lru(S);
        int32_t nm = 0;
        for (int step = 0; step < 40; ++step) {
            std::vector<int32_t> s;
            for (int j = 0; j < cap && (int)s.size() < 40; ++j)
                if (below(4) == 0) s.push_back(j);
            for (auto& x : imp) x = grid();
            (void)oracle_pool_stage(p, s.data(), (int32_t)s.size(), imp.data(), phys.data(), ml.data(), ms.data(), &nm);
            if (step == 20) oracle_pool_set_capacity(p, 40);
            if (step == 25) oracle_pool_set_capacity(p, 48);
            if (step == 30) (void)oracle_pool_adapt(p, 0.5, 1e7, 0.1, 4, 40, 48, 10);
            if (step == 35) oracle_pool_store(p, 150, 50);
            (void)oracle_pool_state(p, sl.data(), lru.data());
        }
        uint64_t st[4];
        oracle_pool_stats(p, st);
        oracle_pool_free(p);
    }
    // attention (rows and none), KVSwap score and attention
    const int D = 16, Hq = 3, Wn = 5;
    std::vector<float> qa(Hq * D), win(Wn * D), store(N * D), out(Hq * D);
    for (auto& x : qa) x = grid();
    for (auto& x : win) x = grid();
    for (auto& x : store) x = grid();
    oracle_attend(qa.data(), Hq, D, win.data(), Wn, store.data(), 0, lsel.data(), nl, 0.25f, out.data());
    oracle_attend(qa.data(), Hq, D, win.data(), 0, store.data(), 0, lsel.data(), 0, 0.25f, out.data());
    const int T = 100, r = 8, C = 16;
    std::vector<uint16_t> U(T * r), V(C * r), kv(T * 2 * C);
    for (auto& x : U) x = (uint16_t)(0x3000 + below(0x400));
    for (auto& x : V) x = (uint16_t)(0x3000 + below(0x400));
    for (auto& x : kv) x = (uint16_t)(0x3000 + below(0x400));
    std::vector<float> S(r), qg(C), score(T), o(C);
    for (auto& x : S) x = grid();
    for (auto& x : qg) x = grid();
    oracle_lowrank_score(U.data(), T, r, S.data(), V.data(), C, qg.data(), score.data());
    std::vector<int32_t> pos(20);
    for (auto& x : pos) x = below(T);
    oracle_attend_kv(qg.data(), C, kv.data(), kv.data() + C, 2, 2 * C, pos.data(), 20, 0.25f, o.data());
    std::printf("oracle sanitize run ok\n");
    return 0;
}
