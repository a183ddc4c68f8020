// Host side of libspectra: argument validation, sizes, error reporting and the float64
// calibration ("SPECTRA" technical summary, SPECTRA pipeline stages 1-2).
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <limits>
#include <string>
#include <vector>

#include "spectra_internal.h"

namespace spectra {

static thread_local std::string g_err;
static thread_local void* g_ev_before = nullptr;
static thread_local void* g_ev_after = nullptr;

spectra_status fail(spectra_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

void clear_error() { g_err.clear(); }

void take_timing_events(void** before, void** after) {
    *before = g_ev_before;
    *after = g_ev_after;
    g_ev_before = g_ev_after = nullptr;
}

spectra_status make_layout(const spectra_layout* L, LayoutInfo* o) {
    if (!L) return fail(SPECTRA_EINVAL, "layout is NULL");
    if (L->d_model <= 0 || L->n_q_heads <= 0 || L->n_kv_heads <= 0 || L->d_head <= 0)
        return fail(SPECTRA_EINVAL, "layout: non-positive dimension");
    if (L->n_q_heads % L->n_kv_heads)
        return fail(SPECTRA_EINVAL, "layout: n_q_heads %d not a multiple of n_kv_heads %d",
                    L->n_q_heads, L->n_kv_heads);
    if (L->n_seg <= 0 || L->n_kv_heads % L->n_seg || L->n_seg > kMaxSeg)
        return fail(SPECTRA_EINVAL, "layout: n_seg %d must divide n_kv_heads %d (max %d)",
                    L->n_seg, L->n_kv_heads, kMaxSeg);
    if (L->group_size <= 0 || L->seg_rank <= 0 || L->seg_rank % L->group_size)
        return fail(SPECTRA_EINVAL, "layout: group_size %d must divide seg_rank %d",
                    L->group_size, L->seg_rank);
    const int seg_cols = L->n_kv_heads * L->d_head / L->n_seg;
    if (L->seg_rank > seg_cols)
        return fail(SPECTRA_EINVAL, "layout: seg_rank %d exceeds segment width %d", L->seg_rank, seg_cols);
    if (!L->widths_k || !L->widths_v) return fail(SPECTRA_EINVAL, "layout: widths are NULL");
    std::memset(o, 0, sizeof *o);
    o->d_model = L->d_model;
    o->n_q = L->n_q_heads;
    o->n_kv = L->n_kv_heads;
    o->d_head = L->d_head;
    o->n_seg = L->n_seg;
    o->seg_rank = L->seg_rank;
    o->g = L->group_size;
    o->n_groups = L->seg_rank / L->group_size;
    o->seg_cols = seg_cols;
    o->kv_per_seg = L->n_kv_heads / L->n_seg;
    o->q_per_kv = L->n_q_heads / L->n_kv_heads;
    for (int t = 0; t < 2; ++t) {
        const uint8_t* w = t == 0 ? L->widths_k : L->widths_v;
        TensorInfo& ti = o->t[t];
        int n = 0;
        int64_t codes = 0;
        for (int s = 0; s < L->n_seg; ++s) {
            ti.seg_chunk0[s] = n;
            for (int k = 0; k < o->n_groups; ++k) {
                int b = w[s * o->n_groups + k];
                if (b > 8) return fail(SPECTRA_EINVAL, "layout: width %d > 8", b);
                if (b == 0) continue;
                if (n >= kMaxC) return fail(SPECTRA_ENOTSUP, "layout: more than %d non-empty groups", kMaxC);
                ti.width[n] = (uint8_t)b;
                ti.seg[n] = (uint8_t)s;
                codes += 16LL * o->g * b;
                ++n;
            }
        }
        ti.seg_chunk0[L->n_seg] = n;
        ti.n_chunks = n;
        ti.r_act = n * o->g;
        ti.codes_bytes = (int32_t)codes;
        int64_t bb = codes + (int64_t)n * kBT * 2;
        if (bb > (1LL << 30)) return fail(SPECTRA_ENOTSUP, "layout: block too large");
        ti.block_bytes = (int32_t)bb;
    }
    return SPECTRA_OK;
}

// ------------------------------------------------------------------ dense helpers (fp64)

// C[m x n] = A[m x k] * B[k x n], row-major.  Blocks of 16 rows of C share each row of B
// (loaded once per block, not once per row), in column slabs of 512 that keep the block's rows
// of C in cache; every element sums its k products in ascending order.
static void matmul(int m, int n, int k, const double* A, const double* B, double* C) {
    constexpr int RB = 16, CB = 512;
#pragma omp parallel for schedule(dynamic, 1)
    for (int i0 = 0; i0 < m; i0 += RB) {
        const int i1 = std::min(m, i0 + RB);
        for (int i = i0; i < i1; ++i) std::fill(C + (size_t)i * n, C + (size_t)i * n + n, 0.0);
        for (int j0 = 0; j0 < n; j0 += CB) {
            const int j1 = std::min(n, j0 + CB);
            for (int p = 0; p < k; ++p) {
                const double* b = B + (size_t)p * n;
                for (int i = i0; i < i1; ++i) {
                    const double a = A[(size_t)i * k + p];
                    if (a == 0.0) continue;
                    double* c = C + (size_t)i * n;
                    for (int j = j0; j < j1; ++j) c[j] += a * b[j];
                }
            }
        }
    }
}
// C[m x n] = A^T B with A [k x m], B [k x n], row-major; the same blocking (row p of A gives
// the block's 16 multipliers, read contiguously), k products summed in ascending order.
static void matmul_tn(int m, int n, int k, const double* A, const double* B, double* C) {
    constexpr int RB = 16, CB = 512;
#pragma omp parallel for schedule(dynamic, 1)
    for (int i0 = 0; i0 < m; i0 += RB) {
        const int i1 = std::min(m, i0 + RB);
        for (int i = i0; i < i1; ++i) std::fill(C + (size_t)i * n, C + (size_t)i * n + n, 0.0);
        for (int j0 = 0; j0 < n; j0 += CB) {
            const int j1 = std::min(n, j0 + CB);
            for (int p = 0; p < k; ++p) {
                const double* b = B + (size_t)p * n;
                const double* ap = A + (size_t)p * m;
                for (int i = i0; i < i1; ++i) {
                    const double a = ap[i];
                    if (a == 0.0) continue;
                    double* c = C + (size_t)i * n;
                    for (int j = j0; j < j1; ++j) c[j] += a * b[j];
                }
            }
        }
    }
}

// Symmetric eigen-decomposition of A (n x n, row-major, overwritten):
// Householder reduction to tridiagonal form, then implicit symmetric QR steps with the
// Wilkinson shift, accumulating the orthogonal factors (Golub & Van Loan, Matrix
// Computations, sections 8.3.1-8.3.3).  Returns eigenvalues `lam` (unsorted) and
// eigenvectors as the columns of Z (n x n row-major).  false if QR did not converge.
static bool sym_eig(int n, std::vector<double>& A, std::vector<double>& lam, std::vector<double>& Z) {
    auto a = [&](int i, int j) -> double& { return A[(size_t)i * n + j]; };
    std::vector<std::vector<double>> hv(std::max(0, n - 2));
    std::vector<double> hbeta(std::max(0, n - 2), 0.0);
    std::vector<double> p(n), w(n);
    for (int k = 0; k + 2 < n; ++k) {
        const int m = n - k - 1;
        std::vector<double>& v = hv[k];
        v.assign(m, 0.0);
        double nrm2 = 0.0;
        for (int i = 0; i < m; ++i) {
            v[i] = a(k + 1 + i, k);
            nrm2 += v[i] * v[i];
        }
        const double nrm = std::sqrt(nrm2);
        double beta = 0.0;
        if (nrm > 0.0) {
            const double alpha = v[0] > 0 ? -nrm : nrm;   // P x = alpha e1
            v[0] -= alpha;
            double vv = 0.0;
            for (int i = 0; i < m; ++i) vv += v[i] * v[i];
            beta = vv > 0 ? 2.0 / vv : 0.0;
            if (beta != 0.0) {
                // p = beta B v,  w = p - (beta/2)(p.v) v,  B -= v w^T + w v^T
#pragma omp parallel for schedule(static)
                for (int i = 0; i < m; ++i) {
                    const double* row = &A[(size_t)(k + 1 + i) * n + k + 1];
                    double s = 0.0;
                    for (int j = 0; j < m; ++j) s += row[j] * v[j];
                    p[i] = beta * s;
                }
                double pv = 0.0;
                for (int i = 0; i < m; ++i) pv += p[i] * v[i];
                const double K = 0.5 * beta * pv;
                for (int i = 0; i < m; ++i) w[i] = p[i] - K * v[i];
#pragma omp parallel for schedule(static)
                for (int i = 0; i < m; ++i) {
                    double* row = &A[(size_t)(k + 1 + i) * n + k + 1];
                    const double vi = v[i], wi = w[i];
                    for (int j = 0; j < m; ++j) row[j] -= vi * w[j] + wi * v[j];
                }
            }
            a(k + 1, k) = a(k, k + 1) = alpha;
            for (int i = 1; i < m; ++i) a(k + 1 + i, k) = a(k, k + 1 + i) = 0.0;
        }
        hbeta[k] = beta;
    }
    std::vector<double> d(n), e(std::max(1, n - 1), 0.0);
    for (int i = 0; i < n; ++i) d[i] = a(i, i);
    for (int i = 0; i + 1 < n; ++i) e[i] = a(i + 1, i);
    // Q = H_0 H_1 ... H_{n-3}, accumulated backwards.
    Z.assign((size_t)n * n, 0.0);
    for (int i = 0; i < n; ++i) Z[(size_t)i * n + i] = 1.0;
    for (int k = n - 3; k >= 0; --k) {
        if (hbeta[k] == 0.0) continue;
        const int m = n - k - 1;
        const std::vector<double>& v = hv[k];
        const double beta = hbeta[k];
        // Z[k+1:, k+1:] = (I - beta v v^T) Z[k+1:, k+1:]
        std::vector<double> t(m, 0.0);
        for (int i = 0; i < m; ++i) {
            const double vi = v[i];
            if (vi == 0.0) continue;
            const double* row = &Z[(size_t)(k + 1 + i) * n + k + 1];
            for (int j = 0; j < m; ++j) t[j] += vi * row[j];
        }
#pragma omp parallel for schedule(static)
        for (int i = 0; i < m; ++i) {
            double* row = &Z[(size_t)(k + 1 + i) * n + k + 1];
            const double f = beta * v[i];
            for (int j = 0; j < m; ++j) row[j] -= f * t[j];
        }
    }
    // Implicit symmetric QR on (d, e).
    const double eps = std::numeric_limits<double>::epsilon();
    std::vector<double> rc, rs;
    std::vector<int> rk;
    long iters = 0;
    const long max_iters = 60L * n + 100;
    int hi = n - 1;
    while (hi > 0) {
        if (std::fabs(e[hi - 1]) <= eps * (std::fabs(d[hi - 1]) + std::fabs(d[hi]))) {
            e[hi - 1] = 0.0;
            --hi;
            continue;
        }
        int lo = hi - 1;
        while (lo > 0 && std::fabs(e[lo - 1]) > eps * (std::fabs(d[lo - 1]) + std::fabs(d[lo]))) --lo;
        if (++iters > max_iters) return false;
        const double dl = 0.5 * (d[hi - 1] - d[hi]);
        const double eh = e[hi - 1];
        const double den = dl + (dl >= 0 ? 1.0 : -1.0) * std::hypot(dl, eh);
        const double mu = d[hi] - eh * eh / den;
        double x = d[lo] - mu, z = e[lo];
        rc.clear(); rs.clear(); rk.clear();
        for (int k = lo; k < hi; ++k) {
            double c, s;
            if (z == 0.0) { c = 1.0; s = 0.0; }
            else if (std::fabs(z) > std::fabs(x)) { const double tau = -x / z; s = 1.0 / std::sqrt(1 + tau * tau); c = s * tau; }
            else { const double tau = -z / x; c = 1.0 / std::sqrt(1 + tau * tau); s = c * tau; }
            if (k > lo) e[k - 1] = c * x - s * z;
            const double ak = d[k], bk = e[k], ck = d[k + 1];
            d[k] = ak * c * c - 2 * bk * c * s + ck * s * s;
            d[k + 1] = ak * s * s + 2 * bk * c * s + ck * c * c;
            e[k] = (ak - ck) * c * s + bk * (c * c - s * s);
            if (k + 1 < hi) {
                z = -s * e[k + 1];
                e[k + 1] = c * e[k + 1];
                x = e[k];
            }
            rc.push_back(c); rs.push_back(s); rk.push_back(k);
        }
        const int nr = (int)rk.size();
#pragma omp parallel for schedule(static) if (n >= 256)
        for (int i = 0; i < n; ++i) {
            double* row = &Z[(size_t)i * n];
            for (int r = 0; r < nr; ++r) {
                const int k = rk[r];
                const double zk = row[k], zk1 = row[k + 1];
                row[k] = rc[r] * zk - rs[r] * zk1;
                row[k + 1] = rs[r] * zk + rc[r] * zk1;
            }
        }
    }
    lam = d;
    return true;
}

// Widths at water level theta: b_k = number of breakpoints v_k 2^-(2j-1) (j = 1..maxw) that
// are >= theta, i.e. clamp(floor(1/2 log2(v_k/theta) + 1/2), 0, maxw) without log rounding.
// Median of a (copied) sample; the mean of the two middle values for an even count.
static double median_of(std::vector<double>& a) {
    const size_t n = a.size(), h = n / 2;
    std::nth_element(a.begin(), a.begin() + h, a.end());
    const double hi = a[h];
    if (n % 2) return hi;
    const double lo = *std::max_element(a.begin(), a.begin() + h);
    return 0.5 * (lo + hi);
}

// Outlier-robust eigen-pairs of the projected calibration rows Y = rows W_s (n x m), in the
// form sym_eig returns them (values `lam`, eigenvector j = column j of the row-major m x m Z).
// Directions: eigenvectors of the spatial-sign second moment S = mean over the rows with
// y != 0 of y y^T / |y|^2, placed in descending order of S's eigenvalues (so that ties in the
// variances below keep that order under the caller's stable sort).  Values: the median over
// all rows of (y . u)^2 divided by the median of chi-squared(1), (Phi^-1(3/4))^2.
static bool robust_pairs(const double* rows, int64_t n, int d, int m, const std::vector<double>& Ws,
                         std::vector<double>& lam, std::vector<double>& Z) {
    constexpr double kChi2Median1 = 0.45493642311957272;
    std::vector<double> Y((size_t)n * m);
    matmul((int)n, m, d, rows, Ws.data(), Y.data());
    std::vector<double> Yn(Y);
    int64_t nz = 0;
#pragma omp parallel for schedule(static) reduction(+ : nz)
    for (int64_t i = 0; i < n; ++i) {
        double* y = &Yn[(size_t)i * m];
        double s = 0;
        for (int j = 0; j < m; ++j) s += y[j] * y[j];
        if (s > 0) {
            const double inv = 1.0 / std::sqrt(s);
            for (int j = 0; j < m; ++j) y[j] *= inv;
            ++nz;
        }
    }
    std::vector<double> S((size_t)m * m, 0.0);
    if (nz > 0) {
        matmul_tn(m, m, (int)n, Yn.data(), Yn.data(), S.data());
        for (double& x : S) x /= (double)nz;
    }
    for (int i = 0; i < m; ++i)
        for (int j = i + 1; j < m; ++j) {
            const double v = 0.5 * (S[(size_t)i * m + j] + S[(size_t)j * m + i]);
            S[(size_t)i * m + j] = S[(size_t)j * m + i] = v;
        }
    std::vector<double> mu, U;
    if (!sym_eig(m, S, mu, U)) return false;
    std::vector<int> order(m);
    for (int i = 0; i < m; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return mu[a] > mu[b]; });
    Z.assign((size_t)m * m, 0.0);
    for (int c = 0; c < m; ++c)
        for (int i = 0; i < m; ++i) Z[(size_t)i * m + c] = U[(size_t)i * m + order[c]];
    std::vector<double>().swap(Yn);
    std::vector<double> Pj((size_t)n * m);               // projections y . u_c
    matmul((int)n, m, m, Y.data(), Z.data(), Pj.data());
    lam.assign(m, 0.0);
#pragma omp parallel
    {
        std::vector<double> p((size_t)n);
#pragma omp for schedule(dynamic, 4)
        for (int c = 0; c < m; ++c) {
            for (int64_t r = 0; r < n; ++r) {
                const double x = Pj[(size_t)r * m + c];
                p[r] = x * x;
            }
            lam[c] = median_of(p) / kChi2Median1;
        }
    }
    return true;
}

// float32 -> fp16 round-to-nearest-even, back in float32, for finite x >= 0; values at or
// above the largest fp16 number (65504) give 65504.  fp16 keeps 11 significant bits down to
// 2^-14 and a fixed quantum of 2^-24 below it; every scaling here is by a power of two (exact).
static float fp16_round(float x) {
    if (x >= 65504.0f) return 65504.0f;
    if (x < 6.103515625e-05f) return std::nearbyint(x * 16777216.0f) / 16777216.0f;
    int e;
    (void)std::frexp(x, &e);                          // x = m 2^e, m in [0.5, 1)
    const float q = std::ldexp(1.0f, e - 11);
    return std::nearbyint(x / q) * q;
}

// The encoder's per-token group quantiser (cache layout of include/spectra.h), float32 as
// written there, returning the dequantised values: s = fp16(A 2^(1-b)), A = max_j |c_j|;
// u_j = clamp(rint(c_j / s + (2^b-1)/2), 0, 2^b - 1) (0 when s = 0); c^_j = s (u_j - (2^b-1)/2).
static void quant_dequant_group(const float* c, int g, int b, double* out) {
    float A = 0.0f;
    for (int j = 0; j < g; ++j) A = std::max(A, std::fabs(c[j]));
    const float s = fp16_round(std::ldexp(A, 1 - b));
    const float h = 0.5f * (float)((1 << b) - 1);
    const float umax = (float)((1 << b) - 1);
    for (int j = 0; j < g; ++j) {
        float u = 0.0f;
        if (s != 0.0f) {
            const float x = c[j] / s;
            u = std::min(std::max(std::nearbyint(x + h), 0.0f), umax);
        }
        out[j] = (double)s * ((double)u - (double)h);
    }
}

// Cholesky solve of the symmetric positive definite N X = R (N n x n, R n x m, row-major;
// N overwritten by its factor, R by X).  False when N is not positive definite.
static bool chol_solve(int n, int m, std::vector<double>& N, std::vector<double>& R) {
    for (int j = 0; j < n; ++j) {
        double d = N[(size_t)j * n + j];
        for (int k = 0; k < j; ++k) d -= N[(size_t)j * n + k] * N[(size_t)j * n + k];
        if (!(d > 0)) return false;
        const double l = std::sqrt(d);
        N[(size_t)j * n + j] = l;
        for (int i = j + 1; i < n; ++i) {
            double v = N[(size_t)i * n + j];
            for (int k = 0; k < j; ++k) v -= N[(size_t)i * n + k] * N[(size_t)j * n + k];
            N[(size_t)i * n + j] = v / l;
        }
    }
#pragma omp parallel for schedule(static)
    for (int c = 0; c < m; ++c) {
        for (int i = 0; i < n; ++i) {                  // L y = r
            double v = R[(size_t)i * m + c];
            for (int k = 0; k < i; ++k) v -= N[(size_t)i * n + k] * R[(size_t)k * m + c];
            R[(size_t)i * m + c] = v / N[(size_t)i * n + i];
        }
        for (int i = n - 1; i >= 0; --i) {             // L^T x = y
            double v = R[(size_t)i * m + c];
            for (int k = i + 1; k < n; ++k) v -= N[(size_t)k * n + i] * R[(size_t)k * m + c];
            R[(size_t)i * m + c] = v / N[(size_t)i * n + i];
        }
    }
    return true;
}

// Value-latent correction of one segment (spectra_calibrate): C = rows W_down_s (wdt holds
// W_down_s^T, nc x d), C^ = the encoder's quantisation of C in float32 with the active widths
// wa (group size g), F = (C^T C^)^-1 C^T C, and wu (nc x sc) <- F wu.
static bool value_correction(const double* rows, int64_t n, int d, const double* wdt, int nc,
                             const std::vector<int>& wa, int g, double* wu, int sc) {
    std::vector<double> Wd((size_t)d * nc);
    for (int i = 0; i < d; ++i)
        for (int c = 0; c < nc; ++c) Wd[(size_t)i * nc + c] = wdt[(size_t)c * d + i];
    std::vector<double> C((size_t)n * nc), Ch((size_t)n * nc);
    matmul((int)n, nc, d, rows, Wd.data(), C.data());
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        std::vector<float> c32(g);
        for (size_t k = 0; k < wa.size(); ++k) {
            const double* src = &C[(size_t)r * nc + k * g];
            for (int j = 0; j < g; ++j) c32[j] = (float)src[j];
            quant_dequant_group(c32.data(), g, wa[k], &Ch[(size_t)r * nc + k * g]);
        }
    }
    std::vector<double> N((size_t)nc * nc), R((size_t)nc * nc);
    matmul_tn(nc, nc, (int)n, Ch.data(), Ch.data(), N.data());
    matmul_tn(nc, nc, (int)n, Ch.data(), C.data(), R.data());
    if (!chol_solve(nc, nc, N, R)) return false;
    std::vector<double> out((size_t)nc * sc);
    matmul(nc, sc, nc, R.data(), wu, out.data());
    std::copy(out.begin(), out.end(), wu);
    return true;
}

static void widths_at(const std::vector<double>& v, double theta, int maxw, std::vector<int>& w) {
    w.assign(v.size(), 0);
    for (size_t k = 0; k < v.size(); ++k) {
        if (!(v[k] > 0)) continue;
        int b = 0;
        for (int j = 1; j <= maxw; ++j)
            if (std::ldexp(v[k], -(2 * j - 1)) >= theta) b = j;
        w[k] = b;
    }
}

static long long alloc_cost(const std::vector<int>& w, int g, int sb) {
    long long c = 0;
    for (int b : w) if (b > 0) c += (long long)g * b + sb;
    return c;
}

// Reverse water-filling: lower the level through the breakpoints (largest first) while the
// cost stays within R; returns the level of the last accepted breakpoint (inf if none).
static double water_fill(const std::vector<double>& v, int g, long long R, int sb, int maxw,
                         std::vector<int>& widths) {
    std::vector<double> bp;
    for (double x : v)
        if (x > 0)
            for (int j = 1; j <= maxw; ++j) bp.push_back(std::ldexp(x, -(2 * j - 1)));
    std::sort(bp.begin(), bp.end(), [](double a, double b) { return a > b; });
    bp.erase(std::unique(bp.begin(), bp.end()), bp.end());
    double theta = std::numeric_limits<double>::infinity();
    widths.assign(v.size(), 0);
    std::vector<int> w;
    for (double t : bp) {
        widths_at(v, t, maxw, w);
        if (alloc_cost(w, g, sb) > R) break;
        theta = t;
        widths = w;
    }
    return theta;
}

}  // namespace spectra

using namespace spectra;

extern "C" {

const char* spectra_last_error(void) { return g_err.c_str(); }

const char* spectra_version(void) { return "spectra-mi355x 0.1"; }

void spectra_set_timing_events(void* before, void* after) {
    if (before && after) { g_ev_before = before; g_ev_after = after; }
    else { g_ev_before = g_ev_after = nullptr; }
}

spectra_status spectra_block_bytes(const spectra_layout* layout, int32_t tensor, size_t* bytes) {
    clear_error();
    LayoutInfo li;
    spectra_status st = make_layout(layout, &li);
    if (st) return st;
    if (tensor != 0 && tensor != 1) return fail(SPECTRA_EINVAL, "tensor must be 0 (K) or 1 (V)");
    if (!bytes) return fail(SPECTRA_EINVAL, "bytes is NULL");
    *bytes = (size_t)li.t[tensor].block_bytes;
    return SPECTRA_OK;
}

spectra_status spectra_cache_bytes(const spectra_layout* layout, int32_t tensor, int32_t batch,
                                   int64_t cap_tokens, size_t* bytes) {
    clear_error();
    LayoutInfo li;
    spectra_status st = make_layout(layout, &li);
    if (st) return st;
    if (tensor != 0 && tensor != 1) return fail(SPECTRA_EINVAL, "tensor must be 0 (K) or 1 (V)");
    if (!bytes) return fail(SPECTRA_EINVAL, "bytes is NULL");
    if (batch < 0 || cap_tokens < 0) return fail(SPECTRA_EINVAL, "negative batch or capacity");
    const int64_t nblk = (cap_tokens + kBT - 1) / kBT;
    *bytes = (size_t)batch * (size_t)nblk * (size_t)li.t[tensor].block_bytes;
    return SPECTRA_OK;
}

spectra_status spectra_calibrate(const double* G, const double* W_K, const double* W_V,
                                 int32_t d_model, int32_t n_kv_heads, int32_t d_head,
                                 const spectra_calib_params* P, spectra_calib_out* out) {
    clear_error();
    if (!W_K || !W_V || !P || !out || (!G && !P->robust)) return fail(SPECTRA_EINVAL, "calibrate: NULL argument");
    if ((P->robust || P->value_correction) && !P->rows)
        return fail(SPECTRA_EINVAL, "calibrate: robust calibration and value correction need the calibration rows");
    if (d_model <= 0 || n_kv_heads <= 0 || d_head <= 0) return fail(SPECTRA_EINVAL, "calibrate: bad dims");
    if (P->n_seg <= 0 || n_kv_heads % P->n_seg) return fail(SPECTRA_EINVAL, "calibrate: n_seg must divide n_kv_heads");
    const int seg_cols = n_kv_heads * d_head / P->n_seg;
    if (P->group_size <= 0 || P->seg_rank <= 0 || P->seg_rank % P->group_size || P->seg_rank > seg_cols)
        return fail(SPECTRA_EINVAL, "calibrate: need group_size | seg_rank <= segment width");
    if (P->rank_rule < SPECTRA_RANK_FIXED || P->rank_rule > SPECTRA_RANK_GAP)
        return fail(SPECTRA_EINVAL, "calibrate: unknown rank rule %d", (int)P->rank_rule);
    if (P->rank_rule == SPECTRA_RANK_ENERGY && !(P->energy > 0 && P->energy <= 1))
        return fail(SPECTRA_EINVAL, "calibrate: the energy rank rule needs 0 < energy <= 1");
    if (P->rank_rule == SPECTRA_RANK_GAP && !(P->gap_ratio > 1))
        return fail(SPECTRA_EINVAL, "calibrate: the spectral-gap rank rule needs gap_ratio > 1");
    if (P->max_width < 1 || P->max_width > 8 || P->fixed_width > 8 || P->scale_bits < 0)
        return fail(SPECTRA_EINVAL, "calibrate: bad width parameters");
    if (!out->w_down_t_k || !out->w_down_t_v || !out->w_up_k || !out->w_up_v || !out->widths_k ||
        !out->widths_v || !out->sigma2_k || !out->sigma2_v)
        return fail(SPECTRA_EINVAL, "calibrate: NULL output array");
    if (P->rows && P->n_rows < 1) return fail(SPECTRA_EINVAL, "calibrate: rows given with n_rows < 1");
    const bool robust = P->robust != 0;
    const size_t dd = (size_t)d_model * d_model, dn = (size_t)d_model * n_kv_heads * d_head;
    if (P->rows) {
        const size_t nr = (size_t)P->n_rows * d_model;
        for (size_t i = 0; i < nr; ++i)
            if (!std::isfinite(P->rows[i])) return fail(SPECTRA_ENUMERIC, "calibrate: rows not finite");
    }
    if (!robust)
        for (size_t i = 0; i < dd; ++i) if (!std::isfinite(G[i])) return fail(SPECTRA_ENUMERIC, "calibrate: G not finite");
    for (size_t i = 0; i < dn; ++i)
        if (!std::isfinite(W_K[i]) || !std::isfinite(W_V[i])) return fail(SPECTRA_ENUMERIC, "calibrate: W not finite");

    const int n_all = n_kv_heads * d_head;
    const int groups = P->seg_rank / P->group_size;
    const long long R = (long long)std::floor(P->budget_bits * seg_cols + 1e-9);
    std::vector<double> GW(robust ? 0 : (size_t)d_model * n_all);
    for (int t = 0; t < 2; ++t) {
        const double* W = t == 0 ? W_K : W_V;
        double* wd = t == 0 ? out->w_down_t_k : out->w_down_t_v;
        double* wu = t == 0 ? out->w_up_k : out->w_up_v;
        uint8_t* wid = t == 0 ? out->widths_k : out->widths_v;
        double* sig = t == 0 ? out->sigma2_k : out->sigma2_v;
        double* th = t == 0 ? out->theta_k : out->theta_v;
        int32_t* er = t == 0 ? out->energy_rank_k : out->energy_rank_v;
        if (!robust) matmul(d_model, n_all, d_model, G, W, GW.data());   // G W (all columns)
        int row = 0;
        for (int s = 0; s < P->n_seg; ++s) {
            const int c0 = s * seg_cols;
            // M = W_s^T (G W)_s
            std::vector<double> Ws((size_t)d_model * seg_cols);
            for (int i = 0; i < d_model; ++i)
                for (int j = 0; j < seg_cols; ++j) Ws[(size_t)i * seg_cols + j] = W[(size_t)i * n_all + c0 + j];
            std::vector<double> lam, Z;
            if (robust) {
                if (!robust_pairs(P->rows, P->n_rows, d_model, seg_cols, Ws, lam, Z))
                    return fail(SPECTRA_ENUMERIC, "calibrate: eigen-solver did not converge");
            } else {
                std::vector<double> GWs((size_t)d_model * seg_cols);
                for (int i = 0; i < d_model; ++i)
                    for (int j = 0; j < seg_cols; ++j) GWs[(size_t)i * seg_cols + j] = GW[(size_t)i * n_all + c0 + j];
                std::vector<double> M((size_t)seg_cols * seg_cols);
                matmul_tn(seg_cols, seg_cols, d_model, Ws.data(), GWs.data(), M.data());
                for (int i = 0; i < seg_cols; ++i)
                    for (int j = i + 1; j < seg_cols; ++j) {
                        const double m = 0.5 * (M[(size_t)i * seg_cols + j] + M[(size_t)j * seg_cols + i]);
                        M[(size_t)i * seg_cols + j] = M[(size_t)j * seg_cols + i] = m;
                    }
                if (!sym_eig(seg_cols, M, lam, Z)) return fail(SPECTRA_ENUMERIC, "calibrate: eigen-solver did not converge");
            }
            std::vector<int> order(seg_cols);
            for (int i = 0; i < seg_cols; ++i) order[i] = i;
            std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return lam[a] > lam[b]; });
            // eigenvector columns in order, canonical sign (largest |entry| positive, first on ties)
            std::vector<double> V((size_t)seg_cols * P->seg_rank);
            for (int c = 0; c < P->seg_rank; ++c) {
                const int src = order[c];
                int arg = 0;
                double best = -1;
                for (int i = 0; i < seg_cols; ++i) {
                    const double m = std::fabs(Z[(size_t)i * seg_cols + src]);
                    if (m > best) { best = m; arg = i; }
                }
                const double sg = Z[(size_t)arg * seg_cols + src] < 0 ? -1.0 : 1.0;
                for (int i = 0; i < seg_cols; ++i) V[(size_t)i * P->seg_rank + c] = sg * Z[(size_t)i * seg_cols + src];
                sig[(size_t)s * P->seg_rank + c] = lam[src];
            }
            // energy rank: smallest r whose leading eigenvalues (negative round-off as zero)
            // hold the share `energy` of the total; 1 when the total is zero
            int erank = -1;
            if (P->energy > 0) {
                double tot = 0, acc = 0;
                for (int i = 0; i < seg_cols; ++i) tot += std::max(0.0, lam[order[i]]);
                erank = 1;
                if (tot > 0) {
                    erank = seg_cols;
                    for (int i = 0; i < seg_cols; ++i) {
                        acc += std::max(0.0, lam[order[i]]);
                        if (acc / tot >= P->energy - 1e-15) { erank = i + 1; break; }
                    }
                }
            }
            if (er) er[s] = erank;
            // rank cap of the rule, in whole groups
            int cap = P->seg_rank;
            if (P->rank_rule == SPECTRA_RANK_ENERGY) {
                cap = std::min(cap, erank);
            } else if (P->rank_rule == SPECTRA_RANK_GAP) {
                double best = 0;
                int at = -1;
                for (int i = 0; i + 1 < P->seg_rank; ++i) {
                    const double a = std::max(lam[order[i]], 1e-300), b = std::max(lam[order[i + 1]], 1e-300);
                    if (a / b > best) { best = a / b; at = i; }
                }
                if (at >= 0 && best >= P->gap_ratio) cap = at + 1;
            }
            const int cap_groups = (cap + P->group_size - 1) / P->group_size;
            std::vector<int> w;
            double theta = std::numeric_limits<double>::quiet_NaN();
            if (P->fixed_width > 0) {
                w.assign(cap_groups, P->fixed_width);
            } else {
                std::vector<double> v(cap_groups, 0.0);
                for (int k = 0; k < cap_groups; ++k) {
                    double acc = 0;
                    for (int j = 0; j < P->group_size; ++j) acc += sig[(size_t)s * P->seg_rank + k * P->group_size + j];
                    v[k] = acc / P->group_size;
                }
                theta = water_fill(v, P->group_size, R, P->scale_bits, P->max_width, w);
            }
            w.resize(groups, 0);                          // groups past the cap: no bits
            if (th) th[s] = theta;
            std::vector<int> cols;                       // active latent columns in order
            for (int k = 0; k < groups; ++k) {
                wid[s * groups + k] = (uint8_t)w[k];
                if (w[k] > 0)
                    for (int j = 0; j < P->group_size; ++j) cols.push_back(k * P->group_size + j);
            }
            const int nc = (int)cols.size();
            // w_down_t row = (W_s V[:, c])^T ; w_up row = V[:, c]^T
#pragma omp parallel for schedule(dynamic, 8)
            for (int ci = 0; ci < nc; ++ci) {
                const int c = cols[ci];
                double* dst = wd + (size_t)(row + ci) * d_model;
                for (int i = 0; i < d_model; ++i) {
                    double acc = 0;
                    const double* wr = &Ws[(size_t)i * seg_cols];
                    for (int q = 0; q < seg_cols; ++q) acc += wr[q] * V[(size_t)q * P->seg_rank + c];
                    dst[i] = acc;
                }
                for (int q = 0; q < seg_cols; ++q) wu[(size_t)(row + ci) * seg_cols + q] = V[(size_t)q * P->seg_rank + c];
            }
            if (t == 1 && P->value_correction && nc > 0) {
                std::vector<int> wa;                         // widths of the active groups, in order
                for (int k = 0; k < groups; ++k)
                    if (w[k] > 0) wa.push_back(w[k]);
                if (!value_correction(P->rows, P->n_rows, d_model, wd + (size_t)row * d_model, nc, wa,
                                      P->group_size, wu + (size_t)row * seg_cols, seg_cols))
                    return fail(SPECTRA_ENUMERIC, "calibrate: value correction: dequantised latents are rank-deficient");
            }
            row += nc;
        }
        (t == 0 ? out->r_act_k : out->r_act_v) = row;
    }
    return SPECTRA_OK;
}

}  // extern "C"
