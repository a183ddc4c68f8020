// Host-code check of libspectra under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Built by tests/test_host_sanitizers.py from this file and the library's host source
// (spectra_host.cpp: layout validation, sizes, float64 calibration with its blocked products,
// eigen-solver, robust pairs and value correction) with -fsanitize=address,undefined; the HIP
// launchers are not part of it.  It calls every host entry point on small seeded problems (and
// on invalid arguments) and checks the returned status and a few invariants; an out-of-bounds
// access, use of uninitialised heap memory through a bad index, integer overflow or other
// undefined behaviour aborts the run with the sanitizer's report.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "../../include/spectra.h"

static int failures = 0;
#define CHECK(cond)                                                                        \
    do {                                                                                   \
        if (!(cond)) {                                                                     \
            std::printf("FAILED %s:%d: %s (%s)\n", __FILE__, __LINE__, #cond, spectra_last_error()); \
            ++failures;                                                                    \
        }                                                                                  \
    } while (0)

struct Problem {
    int d, kv, dh;
    std::vector<double> G, WK, WV, rows;
};

static Problem make_problem(int d, int kv, int dh, int n_rows, unsigned seed) {
    Problem p{d, kv, dh, {}, {}, {}, {}};
    std::mt19937_64 rng(seed);
    std::normal_distribution<double> nd;
    p.rows.resize((size_t)n_rows * d);
    for (int r = 0; r < n_rows; ++r)
        for (int i = 0; i < d; ++i) p.rows[(size_t)r * d + i] = nd(rng) / std::sqrt(1.0 + i);   // decaying spread
    p.G.assign((size_t)d * d, 0.0);
    for (int r = 0; r < n_rows; ++r)
        for (int i = 0; i < d; ++i)
            for (int j = 0; j < d; ++j) p.G[(size_t)i * d + j] += p.rows[(size_t)r * d + i] * p.rows[(size_t)r * d + j] / n_rows;
    p.WK.resize((size_t)d * kv * dh);
    p.WV.resize((size_t)d * kv * dh);
    for (auto& x : p.WK) x = nd(rng) / std::sqrt((double)d);
    for (auto& x : p.WV) x = nd(rng) / std::sqrt((double)d);
    return p;
}

// One calibration; returns its status.  Outputs are sized exactly as the header states.
static spectra_status calibrate(const Problem& p, spectra_calib_params prm, bool with_rows, int* r_act_k = nullptr,
                                std::vector<uint8_t>* wk_out = nullptr) {
    const int R = prm.n_seg * prm.seg_rank, seg_cols = p.kv * p.dh / prm.n_seg;
    const int groups = prm.seg_rank / prm.group_size;
    std::vector<double> dk((size_t)R * p.d), dv((size_t)R * p.d), uk((size_t)R * seg_cols), uv((size_t)R * seg_cols);
    std::vector<uint8_t> wk((size_t)prm.n_seg * groups), wv((size_t)prm.n_seg * groups);
    std::vector<double> sk(R), sv(R), tk(prm.n_seg), tv(prm.n_seg);
    std::vector<int32_t> ek(prm.n_seg), ev(prm.n_seg);
    spectra_calib_out out{dk.data(), dv.data(), uk.data(), uv.data(), wk.data(), wv.data(), sk.data(), sv.data(),
                          tk.data(), tv.data(), ek.data(), ev.data(), 0, 0};
    if (with_rows) {
        prm.rows = p.rows.data();
        prm.n_rows = (int64_t)(p.rows.size() / p.d);
    }
    const spectra_status st = spectra_calibrate(prm.robust ? nullptr : p.G.data(), p.WK.data(), p.WV.data(), p.d,
                                                p.kv, p.dh, &prm, &out);
    if (st == SPECTRA_OK) {
        int act = 0;
        for (int g = 0; g < prm.n_seg * groups; ++g) {
            CHECK(wk[g] <= 8 && wv[g] <= 8);
            act += wk[g] > 0;
        }
        CHECK(out.r_act_k == act * prm.group_size);
        for (int s = 0; s < prm.n_seg; ++s)
            for (int i = 1; i < prm.seg_rank; ++i) CHECK(sk[(size_t)s * prm.seg_rank + i] <= sk[(size_t)s * prm.seg_rank + i - 1] * (1 + 1e-9) + 1e-300);
        if (r_act_k) *r_act_k = out.r_act_k;
        if (wk_out) *wk_out = wk;
    }
    return st;
}

static spectra_calib_params params(int n_seg, int rank, int g, double budget) {
    spectra_calib_params p{};
    p.n_seg = n_seg;
    p.seg_rank = rank;
    p.group_size = g;
    p.budget_bits = budget;
    p.scale_bits = 16;
    p.max_width = 8;
    p.rank_rule = SPECTRA_RANK_FIXED;
    return p;
}

int main() {
    const Problem p = make_problem(48, 2, 16, 300, 7);
    // joint latent, water-filled, several budgets and group sizes
    for (double budget : {1.0, 2.0, 4.0, 8.0})
        for (int g : {1, 2, 4, 8, 16}) CHECK(calibrate(p, params(1, 32, g, budget), false) == SPECTRA_OK);
    // per-head segments, fixed width with an energy rank reported
    {
        spectra_calib_params q = params(2, 12, 2, 0.0);
        q.fixed_width = 4;
        q.energy = 0.95;
        CHECK(calibrate(p, q, false) == SPECTRA_OK);
    }
    // rank rules
    {
        spectra_calib_params q = params(1, 32, 4, 3.0);
        q.rank_rule = SPECTRA_RANK_ENERGY;
        q.energy = 0.9;
        CHECK(calibrate(p, q, false) == SPECTRA_OK);
        q.rank_rule = SPECTRA_RANK_GAP;
        q.gap_ratio = 1.5;
        CHECK(calibrate(p, q, false) == SPECTRA_OK);
    }
    // outlier-robust pairs and the value-latent correction (both read the rows)
    {
        spectra_calib_params q = params(2, 16, 4, 2.0);
        q.robust = 1;
        CHECK(calibrate(p, q, true) == SPECTRA_OK);
        q.robust = 0;
        q.value_correction = 1;
        CHECK(calibrate(p, q, true) == SPECTRA_OK);
        q.robust = 1;
        CHECK(calibrate(p, q, true) == SPECTRA_OK);
    }
    // invalid arguments come back as errors, nothing is written
    {
        spectra_calib_params q = params(3, 32, 4, 2.0);              // 3 does not divide 2 heads
        CHECK(calibrate(p, q, false) == SPECTRA_EINVAL);
        q = params(1, 30, 4, 2.0);                                     // 4 does not divide 30
        CHECK(calibrate(p, q, false) == SPECTRA_EINVAL);
        q = params(1, 64, 4, 2.0);                                     // rank above the segment width
        CHECK(calibrate(p, q, false) == SPECTRA_EINVAL);
        q = params(1, 32, 4, 2.0);
        q.robust = 1;                                                  // robust without rows
        CHECK(calibrate(p, q, false) == SPECTRA_EINVAL);
        q = params(1, 32, 4, 2.0);
        q.rank_rule = SPECTRA_RANK_GAP;                                // ratio must exceed 1
        q.gap_ratio = 1.0;
        CHECK(calibrate(p, q, false) == SPECTRA_EINVAL);
        Problem bad = p;
        bad.G[5] = NAN;
        CHECK(calibrate(bad, params(1, 32, 4, 2.0), false) == SPECTRA_ENUMERIC);
    }
    // layouts and sizes from a calibration, then invalid layouts
    {
        int rk = 0;
        std::vector<uint8_t> w;
        CHECK(calibrate(p, params(1, 32, 16, 4.0), false, &rk, &w) == SPECTRA_OK);
        spectra_layout L{48, 4, 2, 16, 1, 32, 16, w.data(), w.data()};
        size_t bb = 0, cb = 0;
        CHECK(spectra_block_bytes(&L, SPECTRA_TENSOR_K, &bb) == SPECTRA_OK && bb > 0);
        CHECK(spectra_cache_bytes(&L, SPECTRA_TENSOR_V, 3, 1000, &cb) == SPECTRA_OK && cb == 3 * 8 * bb);
        CHECK(spectra_block_bytes(&L, 2, &bb) == SPECTRA_EINVAL);
        const uint8_t wide[2] = {9, 4};
        spectra_layout L2{48, 4, 2, 16, 1, 32, 16, wide, wide};
        CHECK(spectra_block_bytes(&L2, SPECTRA_TENSOR_K, &bb) == SPECTRA_EINVAL);
        spectra_layout L3{48, 3, 2, 16, 1, 32, 16, w.data(), w.data()};   // 3 query heads over 2 KV heads
        CHECK(spectra_block_bytes(&L3, SPECTRA_TENSOR_K, &bb) == SPECTRA_EINVAL);
        CHECK(spectra_cache_bytes(&L, SPECTRA_TENSOR_K, -1, 10, &cb) == SPECTRA_EINVAL);
        CHECK(spectra_cache_bytes(nullptr, SPECTRA_TENSOR_K, 1, 10, &cb) == SPECTRA_EINVAL);
    }
    std::printf("%s: %d failures\n", failures ? "FAIL" : "OK", failures);
    return failures ? 1 : 0;
}
