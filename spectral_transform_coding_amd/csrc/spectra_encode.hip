// Encode: down-project, quantise per token in groups, bit-pack and append (gfx950).
//
// "SPECTRA" technical summary, SPECTRA pipeline stage 3: each token is projected down, quantised
// per token and appended to the latent cache; stage 2: adjacent coordinates share one width
// per group, and zero-width groups are absent from W_down and the cache.
//
// One workgroup computes a 128-token x 128-column tile of C = X W_down (bfloat16 inputs on the
// matrix cores with float32 accumulation, or float32 inputs on the vector ALUs), then, in the
// same launch, for every (token, group) of the tile:
//   A = max_j |c_j|,  s = fp16(A 2^(1-b)) (65504 on overflow),
//   u_j = clamp(rint_even(c_j / s + (2^b-1)/2), 0, 2^b-1)   (u = 0 when s = 0),
// stores s, and packs the codes into the cache words they occupy (plain store when the tile
// holds every code of the word, atomic OR when the word is shared with other tokens).
#include <hip/hip_runtime.h>
#include <type_traits>
#include <cmath>
#include <cstring>

#include "spectra_device.h"

namespace spectra {

// Sequence of flattened row `row` (rows are sequence-major, n_new per sequence): a 32-bit
// division whenever the row index fits in 31 bits (every realistic batch), 64-bit otherwise.
__device__ __forceinline__ int row_seq(int64_t row, int n_new) {
    return row < (int64_t)0x7FFFFFFF ? (int)row / n_new : (int)(row / n_new);
}


constexpr int kTM = 128, kTN = 128, kTK = 32;

template <typename DT> struct GemmSmem;
template <> struct GemmSmem<uint16_t> { uint16_t A[kTM][kTK + 8]; uint16_t B[kTN][kTK + 8]; };
template <> struct GemmSmem<float> { float A[kTM][kTK + 1]; float B[kTN][kTK + 1]; };
struct EpiSmem {
    float lat[kTM][kTN + 1];
    uint8_t cds[kTM][kTN];
};
constexpr int kEncodeLds = sizeof(EpiSmem);
static_assert(sizeof(GemmSmem<float>) <= sizeof(EpiSmem), "LDS union");

// float32 quantisation of one code, exactly as specified (no contraction).
__device__ __forceinline__ uint32_t quant_code(float c, float s, int b) {
#pragma clang fp contract(off)
    if (s == 0.0f) return 0u;
    const float h = 0.5f * (float)((1u << b) - 1u);
    const float x = __fdiv_rn(c, s) + h;
    float r = __builtin_rintf(x);
    r = fminf(fmaxf(r, 0.0f), (float)((1u << b) - 1u));
    return (uint32_t)r;
}

// The same code for a whole group, with the division replaced by an exact equivalent: with
// r = RN(1/s) and q0 = RN(c r), the residual c - q0 s is exact in one fused multiply-add and
// RN(q0 + (c - q0 s) r) = RN(c / s) (Markstein's correction step; checked exhaustively for every
// float32 significand of c against every 11-bit significand of s, which covers every fp16
// scale; quotients below 2^-28 in magnitude, where intermediates may be subnormal, do not move
// c / s + h off h).  s = 0 gives r = 0 and h = -inf, hence code 0.
struct QuantGroup {
    float s, r, h, top;
};
__device__ __forceinline__ QuantGroup quant_group(_Float16 s16, int b) {
    const float s = (float)s16;
    QuantGroup g;
    g.s = s;
    g.r = s == 0.0f ? 0.0f : __fdiv_rn(1.0f, s);
    g.top = (float)((1u << b) - 1u);
    g.h = s == 0.0f ? -__builtin_inff() : 0.5f * g.top;
    return g;
}
__device__ __forceinline__ uint32_t quant_div(float c, const QuantGroup& g) {
    const float q0 = __fmul_rn(c, g.r);
    const float t = __fmaf_rn(__fmaf_rn(-q0, g.s, c), g.r, q0);
    const float x = __fadd_rn(t, g.h);
    return (uint32_t)fminf(fmaxf(__builtin_rintf(x), 0.0f), g.top);
}

// bf16 tile product on the matrix cores: wave w covers rows 64 (w>>1) .. +64 and columns
// 64 (w&1) .. +64 of the tile as 2 x 2 blocks of 32 x 32.
__device__ __forceinline__ void gemm_tile_bf16(GemmSmem<uint16_t>& sm, const uint16_t* __restrict__ x,
                                               const uint16_t* __restrict__ w, int d, int64_t row0,
                                               int64_t M, int col0, int N, EpiSmem& epi) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wr = wv >> 1, wc = wv & 1;
    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};
    uint4 ra[2], rb[2];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int idx = tid + 256 * r, row = idx >> 2, kq = idx & 3;
            const int64_t gr = row0 + row;
            ra[r] = gr < M ? *reinterpret_cast<const uint4*>(x + gr * d + k0 + 8 * kq) : make_uint4(0, 0, 0, 0);
            const int gc = col0 + row;
            rb[r] = gc < N ? *reinterpret_cast<const uint4*>(w + (int64_t)gc * d + k0 + 8 * kq) : make_uint4(0, 0, 0, 0);
        }
    };
    fetch(0);
    for (int k0 = 0; k0 < d; k0 += kTK) {
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int idx = tid + 256 * r, row = idx >> 2, kq = idx & 3;
            *reinterpret_cast<uint4*>(&sm.A[row][8 * kq]) = ra[r];
            *reinterpret_cast<uint4*>(&sm.B[row][8 * kq]) = rb[r];
        }
        __syncthreads();
        if (k0 + kTK < d) fetch(k0 + kTK);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8_t a[2], bb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint4 va = *reinterpret_cast<const uint4*>(&sm.A[64 * wr + 32 * i + (lane & 31)][16 * ks + 8 * (lane >> 5)]);
                const uint4 vb = *reinterpret_cast<const uint4*>(&sm.B[64 * wc + 32 * i + (lane & 31)][16 * ks + 8 * (lane >> 5)]);
                __builtin_memcpy(&a[i], &va, 16);
                __builtin_memcpy(&bb[i], &vb, 16);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bb[j], acc[i][j], 0, 0, 0);
        }
    }
    __syncthreads();   // the epilogue buffer overlays the operand tiles
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int a = 0; a < 16; ++a) {
                const int r = 64 * wr + 32 * i + 8 * (a >> 2) + 4 * (lane >> 5) + (a & 3);
                const int c = 64 * wc + 32 * j + (lane & 31);
                epi.lat[r][c] = acc[i][j][a];
            }
}

// float32 tile product on the vector ALUs: thread t covers rows 8 (t/16) .. +8 and columns
// 8 (t%16) .. +8; each output is a float32 fused multiply-add chain in increasing k.
__device__ __forceinline__ void gemm_tile_f32(GemmSmem<float>& sm, const float* __restrict__ x,
                                              const float* __restrict__ w, int d, int64_t row0,
                                              int64_t M, int col0, int N, EpiSmem& epi) {
    const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
    float acc[8][8];
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[r][c] = 0.0f;
    for (int k0 = 0; k0 < d; k0 += kTK) {
        __syncthreads();
        for (int idx = tid; idx < kTM * kTK / 4; idx += 256) {
            const int row = idx >> 3, kq = idx & 7;
            const int64_t gr = row0 + row;
            const float4 va = gr < M ? *reinterpret_cast<const float4*>(x + gr * d + k0 + 4 * kq) : make_float4(0, 0, 0, 0);
            const int gc = col0 + row;
            const float4 vb = gc < N ? *reinterpret_cast<const float4*>(w + (int64_t)gc * d + k0 + 4 * kq) : make_float4(0, 0, 0, 0);
            sm.A[row][4 * kq] = va.x; sm.A[row][4 * kq + 1] = va.y; sm.A[row][4 * kq + 2] = va.z; sm.A[row][4 * kq + 3] = va.w;
            sm.B[row][4 * kq] = vb.x; sm.B[row][4 * kq + 1] = vb.y; sm.B[row][4 * kq + 2] = vb.z; sm.B[row][4 * kq + 3] = vb.w;
        }
        __syncthreads();
        for (int kk = 0; kk < kTK; ++kk) {
            float a[8], b[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) a[r] = sm.A[8 * tr + r][kk];
#pragma unroll
            for (int c = 0; c < 8; ++c) b[c] = sm.B[8 * tc + c][kk];
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[r][c] = __builtin_fmaf(a[r], b[c], acc[r][c]);
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) epi.lat[8 * tr + r][8 * tc + c] = acc[r][c];
}

// Packs the codes cds[r rs + c cs] (tile rows r = tokens row0 + r, columns col0 + c) into
// every 32-bit word of the (sequence, block, group) code chunks the tile touches: a plain store
// when the tile holds every code of the word, an atomic OR when the word is shared with tokens
// outside the tile.
// ORs a b-bit code of (slot tau, coordinate j) into a code chunk's words (the positions it
// occupies, as read_code reads them); the bits must be zero before.
__device__ __forceinline__ void or_code(int kind, int g, int b, uint32_t* w, int tau, int j, uint32_t code) {
    if (g != 16) {
        const int bit = (tau * g + j) * b, wi = bit >> 5, off = bit & 31;
        atomicOr(w + wi, code << off);
        if (off + b > 32) atomicOr(w + wi + 1, code >> (32 - off));
        return;
    }
    int L, T, e;
    run_of(kind, tau, j, &L, &T, &e);
    const int gam = (4 * T + (e >> 1)) * b;
    const int wi = 64 * (gam >> 4) + L, off = gam & 15, sh = 16 * (e & 1);
    atomicOr(w + wi, ((code << off) & 0xFFFFu) << sh);   // this stream's half-word only
    if (off + b > 16) atomicOr(w + wi + 64, (code >> (16 - off)) << sh);
}

// Tokens per (sequence, tile) up to which pack_tile ORs codes one by one instead of building
// whole chunk words.
constexpr int kPackCodeTokens = 16;

__device__ __forceinline__ void pack_tile(const LayoutInfo& li, const Positions& start, int n_new, int64_t row0, int64_t row_end,
                          int col0, int ncol, const uint8_t* cds, int rs, int cs, uint8_t* __restrict__ cache_k,
                          uint8_t* __restrict__ cache_v, int64_t seq_bytes_k, int64_t seq_bytes_v, int tid,
                          int nthreads) {
    const int g = li.g;
    const int rk = li.t[0].r_act;
    // code p of a chunk is token p / g, coordinate p % g: shifts when g is a power of two
    const bool g_pow2 = (g & (g - 1)) == 0;
    const int g_log = __builtin_ctz((unsigned)g);
    const int sb_lo = row_seq(row0, n_new), sb_hi = row_seq(row_end - 1, n_new);
    for (int sb = sb_lo; sb <= sb_hi; ++sb) {
        const int64_t i_lo = max(row0, (int64_t)sb * n_new) - (int64_t)sb * n_new;
        const int64_t i_hi = min(row_end, (int64_t)(sb + 1) * n_new) - (int64_t)sb * n_new;
        const int64_t p_lo = start.v[sb] + i_lo, p_hi = start.v[sb] + i_hi;    // positions [p_lo, p_hi)
        const int64_t r_base = (int64_t)sb * n_new - start.v[sb] - row0;       // tile row of position pos: r_base + pos
        if (p_hi - p_lo <= kPackCodeTokens) {
            // few tokens (appends): each code's bits are ORed into the word(s) that hold them,
            // one thread per (token, column); walking whole chunks for them cost 19 us per call
            for (int idx = tid; idx < (int)(p_hi - p_lo) * ncol; idx += nthreads) {
                const int64_t pos = p_lo + idx / ncol;
                const int c = idx % ncol, col = col0 + c;
                const uint32_t code = cds[(r_base + pos) * rs + (int64_t)c * cs];
                if (code == 0) continue;
                const int kind = col < rk ? 0 : 1;
                const int lc = col - (kind ? rk : 0), chunk = lc / g, j = lc % g;
                const TensorInfo& ti = li.t[kind];
                uint32_t* words = reinterpret_cast<uint32_t*>(
                    (kind ? cache_v + sb * seq_bytes_v : cache_k + sb * seq_bytes_k) + (pos / kBT) * ti.block_bytes +
                    chunk_code_offset(ti, g, chunk));
                or_code(kind, g, ti.width[chunk], words, (int)(pos % kBT), j, code);
            }
            continue;
        }
        // word wi of the chunk of (block blk, group at tile column c0): built from the tile's codes,
        // stored when the tile covers all of its codes, ORed in when it covers some
        auto build_word = [&](int64_t blk, int c0, int wi) {
            const int col = col0 + c0;
            const int kind = col < rk ? 0 : 1;
            const int chunk = (col - (kind ? rk : 0)) / g;
            const TensorInfo& ti = li.t[kind];
            const int b = ti.width[chunk];
            if (wi >= 4 * g * b) return;
            uint32_t* words = reinterpret_cast<uint32_t*>(
                (kind ? cache_v + sb * seq_bytes_v : cache_k + sb * seq_bytes_k) + blk * ti.block_bytes +
                chunk_code_offset(ti, g, chunk));
            uint32_t word = 0;
            int covered = 0, total = 0;
            // tokens tau of this block that the tile holds, and the tile row of token 0
            const int tau_lo = (int)max<int64_t>(p_lo - blk * kBT, 0);
            const int tau_hi = (int)min<int64_t>(p_hi - blk * kBT, kBT);
            const int r_blk = (int)(r_base + blk * kBT);
            // one code whose bits start at bit c0b of its stream, into the word part that holds
            // stream bits [w0b, w0b + width) at word bit `base`
            auto take = [&](int tau, int j, int c0b, int w0b, int width, int base) {
                ++total;
                if (tau < tau_lo || tau >= tau_hi) return;
                const int r = r_blk + tau;
                const uint32_t code = cds[(int64_t)r * rs + (int64_t)(c0 + j) * cs];
                const int sh = c0b - w0b;
                uint32_t part = sh >= 0 ? (code << sh) : (code >> (-sh));
                if (width < 32) part &= (1u << width) - 1u;
                word |= part << base;
                ++covered;
            };
            if (g == 16) {
                const int L = wi & 63, kw = wi >> 6;     // chunk word 64 kw + L
                for (int sg = 0; sg < 2; ++sg) {
                    const int ia = (16 * kw) / b, ib = (16 * kw + 15) / b;
                    for (int i = ia; i <= ib; ++i) {
                        int tau, j;
                        run_inv(kind, L, i >> 2, 2 * (i & 3) + sg, &tau, &j);
                        take(tau, j, i * b, 16 * kw, 16, 16 * sg);
                    }
                }
            } else {
                const int bit0 = 32 * wi;
                const int pa = bit0 / b, pb = (bit0 + 31) / b;
                if (g_pow2)
                    for (int p = pa; p <= pb; ++p) take(p >> g_log, p & (g - 1), p * b, bit0, 32, 0);
                else
                    for (int p = pa; p <= pb; ++p) take(p / g, p % g, p * b, bit0, 32, 0);
            }
            if (covered == total) words[wi] = word;
            else if (covered > 0) atomicOr(words + wi, word);
        };
        // A (block, group) chunk holds 4 g b words, at most 4 g 8 = 32 g.  When that is fewer than
        // the threads (g < 16 with 512 threads), one flat range over (block, group, word) keeps
        // every thread busy (slots past a narrower width idle); otherwise the threads take one
        // chunk's words at a time.
        const int64_t blk_lo = p_lo / kBT;
        const int nblk = (int)((p_hi - 1) / kBT - blk_lo + 1);
        const int ngr = ncol / g, wmax = 32 * g;
        if (wmax < nthreads) {
            for (int idx = tid; idx < nblk * ngr * wmax; idx += nthreads) {
                const int t = idx / wmax;
                build_word(blk_lo + t / ngr, (t % ngr) * g, idx % wmax);
            }
        } else {
            for (int64_t blk = blk_lo; blk < blk_lo + nblk; ++blk)
                for (int c0 = 0; c0 < ncol; c0 += g)
                    for (int wi = tid; wi < wmax; wi += nthreads) build_word(blk, c0, wi);
        }
    }
}

// Quantises a tile of float32 latents lat[r * ls + c] (tile rows r = tokens row0 + r < row_end,
// columns col0 + c < col0 + ncol, whole groups), stores every (token, group) scale into its scale
// chunk and packs the codes into the cache (codes staged in cds[r * cs + c]); optionally copies
// the latents to latent_out [M x N].  Any group size; all `nthreads` threads of the workgroup
// take part, and the caller has made lat visible to them.
__device__ void quantise_tile(const LayoutInfo& li, const Positions& start, int n_new, int64_t row0, int64_t row_end,
                              int col0, int ncol, const float* lat, int ls, uint8_t* cds, int cs,
                              uint8_t* __restrict__ cache_k, uint8_t* __restrict__ cache_v, int64_t seq_bytes_k,
                              int64_t seq_bytes_v, float* __restrict__ latent_out, int tid, int nthreads) {
    const int g = li.g;
    const int rk = li.t[0].r_act, N = li.t[0].r_act + li.t[1].r_act;
    const int nrow = (int)(row_end - row0);
    if (latent_out)
        for (int idx = tid; idx < nrow * ncol; idx += nthreads) {
            const int r = idx / ncol, c = idx % ncol;
            latent_out[(row0 + r) * N + col0 + c] = lat[r * ls + c];
        }
    // ---- scales and codes of every (token, group) of the tile
    const int gpt = ncol / g;
    // token positions: when the tile's rows belong to one sequence (the usual case), row row0 + r
    // is position p0 + r of sequence sb0, with no division per row
    const int sb0 = row_seq(row0, n_new);
    const int64_t p0 = start.v[sb0] + (row0 - (int64_t)sb0 * n_new);
    const bool one_seq = row_seq(row_end - 1, n_new) == sb0;
    if (nrow * gpt < nthreads && (g & (g - 1)) == 0 && g <= 64 && ncol % g == 0 && nthreads % 64 == 0) {
        // fewer (token, group) pairs than threads (appends): one thread per element.  A group's
        // g elements sit in g consecutive lanes of one wave (ncol is a multiple of g), its
        // maximum is a log2(g)-step lane exchange, and the group's first lane stores the scale.
        // (One-token append of the 128k workload 18.1 -> 17.2 us; on large tiles the thread per
        // pair below is faster: per-head prefill 206 against 227 us.)
        for (int base = 0; base < nrow * ncol; base += nthreads) {
            const int idx = base + tid;
            const bool ok = idx < nrow * ncol;
            const int r = ok ? idx / ncol : 0, c = ok ? idx % ncol : 0;
            const float v = ok ? lat[r * ls + c] : 0.0f;
            float A = fabsf(v);
            for (int o = 1; o < g; o <<= 1) A = fmaxf(A, __shfl_xor(A, o));
            if (!ok) continue;
            const int col = col0 + (c & ~(g - 1));
            const int kind = col < rk ? 0 : 1;
            const int chunk = (col - (kind ? rk : 0)) / g;
            const int b = li.t[kind].width[chunk];
            const float s32 = A * __uint_as_float((uint32_t)(128 - b) << 23);   // A * 2^(1-b), exact
            _Float16 s16 = (_Float16)s32;                                        // round to nearest even
            if (__builtin_isinf((float)s16)) s16 = (_Float16)65504.0f;
            cds[r * cs + c] = (uint8_t)quant_code(v, (float)s16, b);
            if ((c & (g - 1)) == 0) {
                const int64_t row = row0 + r;
                const int sb = one_seq ? sb0 : row_seq(row, n_new);
                const int64_t pos = one_seq ? p0 + r : start.v[sb] + (row - (int64_t)sb * n_new);
                const TensorInfo& ti = li.t[kind];
                uint8_t* blk =
                    (kind ? cache_v + sb * seq_bytes_v : cache_k + sb * seq_bytes_k) + (pos / kBT) * ti.block_bytes;
                uint16_t bits;
                __builtin_memcpy(&bits, &s16, 2);
                reinterpret_cast<uint16_t*>(blk + ti.codes_bytes + 256 * chunk)[scale_index(kind, li.g, (int)(pos % kBT))] =
                    bits;
            }
        }
    } else
    for (int idx = tid; idx < nrow * gpt; idx += nthreads) {
        const int r = idx / gpt, c0 = (idx % gpt) * g;
        const int col = col0 + c0;
        const int kind = col < rk ? 0 : 1;
        const int chunk = (col - (kind ? rk : 0)) / g;
        const int b = li.t[kind].width[chunk];
        float A = 0.0f;
        for (int j = 0; j < g; ++j) A = fmaxf(A, fabsf(lat[r * ls + c0 + j]));
        const float s32 = A * __uint_as_float((uint32_t)(128 - b) << 23);   // A * 2^(1-b), exact
        _Float16 s16 = (_Float16)s32;                                        // round to nearest even
        if (__builtin_isinf((float)s16)) s16 = (_Float16)65504.0f;
        const float s = (float)s16;
        for (int j = 0; j < g; ++j) cds[r * cs + c0 + j] = (uint8_t)quant_code(lat[r * ls + c0 + j], s, b);
        const int64_t row = row0 + r;
        const int sb = one_seq ? sb0 : row_seq(row, n_new);
        const int64_t pos = one_seq ? p0 + r : start.v[sb] + (row - (int64_t)sb * n_new);
        const TensorInfo& ti = li.t[kind];
        uint8_t* blk = (kind ? cache_v + sb * seq_bytes_v : cache_k + sb * seq_bytes_k) + (pos / kBT) * ti.block_bytes;
        uint16_t bits;
        __builtin_memcpy(&bits, &s16, 2);
        reinterpret_cast<uint16_t*>(blk + ti.codes_bytes + 256 * chunk)[scale_index(kind, li.g, (int)(pos % kBT))] = bits;
    }
    __syncthreads();
    // ---- pack
    pack_tile(li, start, n_new, row0, row_end, col0, ncol, cds, cs, 1, cache_k, cache_v, seq_bytes_k, seq_bytes_v,
              tid, nthreads);
}

template <typename DT>
__global__ __launch_bounds__(256) void encode_kernel(LayoutInfo li, Positions start, int batch, int n_new,
                                                     const DT* __restrict__ x, const DT* __restrict__ w,
                                                     uint8_t* __restrict__ cache_k, uint8_t* __restrict__ cache_v,
                                                     int64_t seq_bytes_k, int64_t seq_bytes_v,
                                                     float* __restrict__ latent_out) {
    extern __shared__ __align__(16) unsigned char smem[];
    EpiSmem& epi = *reinterpret_cast<EpiSmem*>(smem);
    GemmSmem<DT>& gs = *reinterpret_cast<GemmSmem<DT>*>(smem);
    const int tid = threadIdx.x;
    const int N = li.t[0].r_act + li.t[1].r_act;
    const int64_t M = (int64_t)batch * n_new;
    const int col0 = blockIdx.x * kTN;
    const int64_t row0 = (int64_t)blockIdx.y * kTM;
    const int64_t row_end = min(M, row0 + kTM);

    if constexpr (sizeof(DT) == 2)
        gemm_tile_bf16(gs, x, w, li.d_model, row0, M, col0, N, epi);
    else
        gemm_tile_f32(gs, x, w, li.d_model, row0, M, col0, N, epi);
    __syncthreads();

    quantise_tile(li, start, n_new, row0, row_end, col0, min(kTN, N - col0), &epi.lat[0][0], kTN + 1, &epi.cds[0][0], kTN,
                  cache_k, cache_v, seq_bytes_k, seq_bytes_v, latent_out, tid, 256);
}


// ------------------------------------------------------------------ few-row encode (appends)
//
// One workgroup computes a 16-token x 16-column tile of C = X W_down over the whole of d_model,
// so that a short append (a few tokens per call, as in decoding) spreads W_down over
// N / 16 workgroups instead of streaming it through a handful of large tiles; the tile is then
// quantised and packed by quantise_tile.
//   bf16: the four waves take the 32-wide k steps round-robin, one 16x16x32 matrix-core product
//         each (X rows as the first operand: lane l holds row l % 16 and k 8 (l / 16) .. + 8),
//         eight steps' operands loaded before their products; the four partial tiles are summed
//         in LDS in wave order;
//   fp32: 32-wide k steps of X and W staged in LDS; thread (r, c) keeps one fused multiply-add
//         chain in increasing k for its output.
constexpr int kSR = 16, kSC = 16, kSK = 32;
struct SmallSmem {
    float part[4][kSR][kSC];            // bf16: per-wave partial tiles
    float xs[kSR][kSK + 1], ws[kSC][kSK + 1];   // fp32: staged k step
    float lat[kSR][kSC + 1];
    uint8_t cds[kSR][kSC];
};

template <typename DT>
__global__ __launch_bounds__(256) void encode_small_kernel(LayoutInfo li, Positions start, int batch, int n_new,
                                                           const DT* __restrict__ x, const DT* __restrict__ w,
                                                           uint8_t* __restrict__ cache_k, uint8_t* __restrict__ cache_v,
                                                           int64_t seq_bytes_k, int64_t seq_bytes_v,
                                                           float* __restrict__ latent_out) {
    __shared__ __align__(16) SmallSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int d = li.d_model;
    const int N = li.t[0].r_act + li.t[1].r_act;
    const int64_t M = (int64_t)batch * n_new;
    const int col0 = blockIdx.x * kSC;
    const int64_t row0 = (int64_t)blockIdx.y * kSR;
    const int64_t row_end = min(M, row0 + kSR);
    const int ncol = min(kSC, N - col0);
    if constexpr (sizeof(DT) == 2) {
        const int r = lane & 15, kq = lane >> 4;
        const bool rok = row0 + r < M, cok = col0 + r < N;
        const uint16_t* xr = x + (rok ? row0 + r : 0) * d + 8 * kq;
        const uint16_t* wr = w + (int64_t)(cok ? col0 + r : 0) * d + 8 * kq;
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
        const int nk = d / kSK;
        // the wave's k steps are wv, wv + 4, ...; kSD of them are loaded before any product (W
        // comes from HBM once per call: the loads in flight hide its latency)
        constexpr int kSD = 8;
        int ks = wv;
        for (; ks + 4 * (kSD - 1) < nk; ks += 4 * kSD) {
            uint4 a[kSD], b[kSD];
#pragma unroll
            for (int u = 0; u < kSD; ++u) {
                const int k0 = (ks + 4 * u) * kSK;
                a[u] = rok ? *reinterpret_cast<const uint4*>(xr + k0) : make_uint4(0, 0, 0, 0);
                b[u] = cok ? *reinterpret_cast<const uint4*>(wr + k0) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < kSD; ++u) {
                bf16x8_t av, bv;
                __builtin_memcpy(&av, &a[u], 16);
                __builtin_memcpy(&bv, &b[u], 16);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
            }
        }
        for (; ks < nk; ks += 4) {
            const int k0 = ks * kSK;
            uint4 a0 = rok ? *reinterpret_cast<const uint4*>(xr + k0) : make_uint4(0, 0, 0, 0);
            uint4 b0 = cok ? *reinterpret_cast<const uint4*>(wr + k0) : make_uint4(0, 0, 0, 0);
            bf16x8_t av, bv;
            __builtin_memcpy(&av, &a0, 16);
            __builtin_memcpy(&bv, &b0, 16);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
        }
        // output: column lane % 16, rows 4 (lane / 16) .. + 4
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.part[wv][4 * kq + e][r] = acc[e];
        __syncthreads();
        {
            const int rr = tid >> 4, cc = tid & 15;
            sm.lat[rr][cc] = ((sm.part[0][rr][cc] + sm.part[1][rr][cc]) + sm.part[2][rr][cc]) + sm.part[3][rr][cc];
        }
    } else {
        const int rr = tid >> 4, cc = tid & 15;
        float acc = 0.0f;
        // k steps in batches of kSF: a batch's operands are all requested before its first step
        // is staged, so a call waits for memory once per batch, not once per step
        constexpr int kSF = 8, kPer = kSR * kSK / 256;       // elements per thread, operand and step
        for (int kb = 0; kb < d; kb += kSF * kSK) {
            float xr[kSF][kPer], wr[kSF][kPer];
#pragma unroll
            for (int f = 0; f < kSF; ++f) {
                const int k0 = min(kb + f * kSK, d - kSK);   // past the end: a repeat, never used
#pragma unroll
                for (int e = 0; e < kPer; ++e) {
                    const int i = tid + 256 * e, rw = i / kSK, kk = i % kSK;
                    xr[f][e] = row0 + rw < M ? (float)x[(row0 + rw) * d + k0 + kk] : 0.0f;
                    wr[f][e] = col0 + rw < N ? (float)w[(int64_t)(col0 + rw) * d + k0 + kk] : 0.0f;
                }
            }
#pragma unroll
            for (int f = 0; f < kSF; ++f) {
                if (kb + f * kSK >= d) break;
                __syncthreads();
#pragma unroll
                for (int e = 0; e < kPer; ++e) {
                    const int i = tid + 256 * e, rw = i / kSK, kk = i % kSK;
                    sm.xs[rw][kk] = xr[f][e];
                    sm.ws[rw][kk] = wr[f][e];
                }
                __syncthreads();
#pragma unroll 8
                for (int kk = 0; kk < kSK; ++kk) acc = __builtin_fmaf(sm.xs[rr][kk], sm.ws[cc][kk], acc);
            }
        }
        sm.lat[rr][cc] = acc;
    }
    __syncthreads();
    quantise_tile(li, start, n_new, row0, row_end, col0, ncol, &sm.lat[0][0], kSC + 1, &sm.cds[0][0], kSC, cache_k,
                  cache_v, seq_bytes_k, seq_bytes_v, latent_out, tid, 256);
}


// --------------------------------------------------------------- matrix-core encode (bf16)
//
// One workgroup (8 waves) computes a 256-token x 256-column tile of C = X W_down on the matrix
// cores (bf16 products, fp32 accumulation) and quantises and packs it in the same launch:
//   * k advances in steps of 32; operand pieces go from memory straight into LDS (16-byte
//     direct loads, four per thread and step, no registers), kEStages steps deep: while step s
//     is multiplied, steps s+1 .. s+kEStages-1 are in flight, and one barrier per step publishes
//     the next step's buffer and frees the oldest one.  The loop is bound by that operand
//     traffic from L2 (each 256 x 256 tile reads 4 MB), not by the matrix cores or the LDS;
//   * wave (wr, wc) owns rows 128 wr .. +128 and columns 64 wc .. +64: 4 x 2 accumulators of
//     32 x 32, each holding a block of C transposed (W_down rows are the first operand), so that
//     a lane holds one token and eight columns of each of two groups;
//   * epilogue (g = 16): the group maximum is seven in-lane maxima and one exchange with the lane
//     32 apart (the group's other eight columns); the scale and its reciprocal are formed once
//     per lane and group, the codes take a multiply and two fused multiply-adds each (see
//     quant_div); scales and codes go to LDS, then the tile's code words are packed;
//   * epilogue (g = 2, 4, 8): quantise_tile in passes of 128 x 128;
//   * the products of 32-column blocks past the end of W_down are skipped (a narrow W_down, such
//     as 96 columns, leaves most of its one column tile empty).
constexpr int kEM = 256, kEN = 256, kEK = 32, kEStages = 4;
constexpr int kEStageBytes = (kEM + kEN) * kEK * 2;                   // A and B tiles of one step
constexpr int kEP = kEK / 8;                                         // 16-byte pieces per row
constexpr int kERowsPerLoad = 64 / kEP;                              // rows per 1 KB wave load
constexpr int kELoads = kEK / 16;                                    // loads per thread, operand and step
static_assert(kEP == 4 || kEP == 8, "k step");
// Operand tiles in LDS: rows of 2 kEK bytes; piece c of row r is stored at position
// c ^ ((r / (16 / kEP)) % kEP), so that an operand read (one piece of 16 consecutive rows per
// 16 lanes) hits 16 distinct groups of four banks.  A direct load fills 1 KB per wave
// instruction, lane i at byte 16 i: lane i fetches the piece that belongs at that position.
__device__ __forceinline__ int enc_swz(int r) { return (r >> (kEP == 8 ? 1 : 2)) & (kEP - 1); }
__device__ __forceinline__ int enc_pos(int r, int c) { return 2 * kEK * r + 16 * (c ^ enc_swz(r)); }
constexpr int kCdsRow = kEN + 8;                                      // code tile: bytes per token (8-aligned)
constexpr int kEpiLds = kEM * kCdsRow + (kEN / 16) * kEM * 2 + 2 * (kEN / 16) * 4;     // codes, scales, groups
constexpr int kEncodeMfmaLds = kEStages * kEStageBytes > kEpiLds ? kEStages * kEStageBytes : kEpiLds;
static_assert(kEncodeMfmaLds <= 160 * 1024, "encode LDS");

typedef uint32_t u32x4e_t __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) unsigned char lds_u8;

// s_waitcnt with vmcnt = n (0..15) and the other counters unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 16, "vmcnt");
    __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Workgroup barrier without a memory fence: a fenced barrier would wait for every direct load
// in flight.  The caller waits for what the other waves must see (wait_vmcnt, lgkmcnt) first;
// the empty asm with a memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void bare_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);                              // lgkmcnt(0)
    __asm__ __volatile__("s_barrier" ::: "memory");
}

// Run words of one lane run from its 32 codes cd[8 T + e]: code e of quarter T belongs to pair
// i = 4 T + e / 2 at stream bits [i B, i B + B) of stream e % 2, and run word k holds stream bits
// [16 k, 16 k + 16) of stream 0 in its low half and of stream 1 in its high half.
template <int B>
__device__ __forceinline__ void run_words(const uint32_t (&cd)[32], uint32_t (&wd)[8]) {
    uint32_t s0[4] = {0, 0, 0, 0}, s1[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int w = (i * B) >> 5, off = (i * B) & 31;
        s0[w] |= cd[2 * i] << off;
        s1[w] |= cd[2 * i + 1] << off;
        if (off + B > 32) {
            s0[w + 1] |= cd[2 * i] >> (32 - off);
            s1[w + 1] |= cd[2 * i + 1] >> (32 - off);
        }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int q = k >> 1, sh = 16 * (k & 1);
        wd[k] = k < B ? ((s0[q] >> sh) & 0xFFFFu) | (((s1[q] >> sh) & 0xFFFFu) << 16) : 0u;
    }
}

__global__ __launch_bounds__(512, 1) void encode_mfma_kernel(LayoutInfo li, Positions start, int batch, int n_new,
                                                          const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ w,
                                                          uint8_t* __restrict__ cache_k, uint8_t* __restrict__ cache_v,
                                                          int64_t seq_bytes_k, int64_t seq_bytes_v,
                                                          float* __restrict__ latent_out, int n_col_tiles) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wv >> 2, wc = wv & 3;
    const int d = li.d_model;
    const int rk = li.t[0].r_act, N = li.t[0].r_act + li.t[1].r_act;
    const int64_t M = (int64_t)batch * n_new;
    // column tiles of one row tile run on one XCD (workgroup id mod 8), so X is fetched from HBM
    // once and re-read from that XCD's L2
    const int id = blockIdx.x;
    const int xcd = id & 7, slot = id >> 3;
    const int col_tile = slot % n_col_tiles;
    const int64_t row_tile = (int64_t)(slot / n_col_tiles) * 8 + xcd;
    const int col0 = col_tile * kEN;
    const int64_t row0 = row_tile * kEM;
    if (row0 >= M) return;
    const int64_t row_end = min(M, row0 + kEM);

    // stage t: A tile (256 rows x 32 bf16, swizzled) at kEStageBytes t, B tile 16 KB after it
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8*)smem;
    // direct loads of this thread: load j of each operand fills the 1 KB at byte
    // 1024 (kELoads wv + j) of the tile; lane i gets row kERowsPerLoad (kELoads wv + j) + i / kEP,
    // position i % kEP, hence piece (i % kEP) ^ enc_swz(row).  Rows past the matrix re-read its
    // last row (their results are never stored).
    const uint16_t* pa[kELoads];
    const uint16_t* pb[kELoads];
#pragma unroll
    for (int j = 0; j < kELoads; ++j) {
        const int r = kERowsPerLoad * (kELoads * wv + j) + lane / kEP;
        const int c = (lane % kEP) ^ enc_swz(r);
        pa[j] = x + min(row0 + r, M - 1) * d + 8 * c;
        pb[j] = w + (int64_t)min(col0 + r, N - 1) * d + 8 * c;
    }
    // a wave whose B rows all lie past the end of W_down (a narrow W_down, such as 96 columns)
    // loads no B pieces: no product reads those rows (their 32-column blocks are skipped)
    const bool bload = col0 + kERowsPerLoad * kELoads * wv < N;
    auto issue = [&](int step, int stage) {
        const int k0 = step * kEK;
        const uint32_t base = lds0 + stage * kEStageBytes + 1024 * kELoads * wv;
#pragma unroll
        for (int j = 0; j < kELoads; ++j)
            __builtin_amdgcn_global_load_lds(pa[j] + k0, (lds_u8*)(uintptr_t)(base + 1024 * j), 16, 0, 0);
        if (bload) {
#pragma unroll
            for (int j = 0; j < kELoads; ++j)
                __builtin_amdgcn_global_load_lds(pb[j] + k0, (lds_u8*)(uintptr_t)(base + kEM * kEK * 2 + 1024 * j), 16,
                                                 0, 0);
        }
    };
    const int nk = d / kEK;
    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i][0] = acc[i][1] = f32x16_t{};
    // 32-column blocks of this wave that hold columns of W_down (the last column tile of a
    // narrow W_down is mostly padding: its products are skipped; the operand loads stay regular)
    const int ncol_tile = min(kEN, N - col0);
    const bool cj0 = 64 * wc < ncol_tile, cj1 = 64 * wc + 32 < ncol_tile;

    // prologue: steps 0 .. kEStages-2 in flight; wait for step 0
#pragma unroll
    for (int t = 0; t < kEStages - 1; ++t) issue(min(t, nk - 1), t);
    if (bload) wait_vmcnt<2 * kELoads * (kEStages - 2)>();
    else wait_vmcnt<kELoads * (kEStages - 2)>();
    bare_barrier();
    // step s: issue step s + kEStages - 1 into the stage read at step s - 1 (every wave has
    // passed the barrier after it), multiply step s, wait for step s + 1 (the last
    // 2 kELoads (kEStages - 2) loads of this thread may stay in flight, kELoads (kEStages - 2)
    // for a wave without B loads) and pass the barrier.
    // Loads past the end re-read the last step into a stage that is never read again, which
    // keeps the counts regular.
    // The k loop is compiled twice: without column guards for tiles whose 32-column blocks all
    // hold columns (straight-line products, operand reads overlapping them), and with them.
    auto k_loop = [&](auto full) {
        constexpr bool kFull = decltype(full)::value;
        for (int step = 0; step < nk; ++step) {
            issue(min(step + kEStages - 1, nk - 1), (step + kEStages - 1) % kEStages);
            const unsigned char* st = smem + (step % kEStages) * kEStageBytes;
            bf16x8_t av[kEK / 16][4], bv[kEK / 16][2];
#pragma unroll
            for (int ks = 0; ks < kEK / 16; ++ks) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const u32x4e_t t = *reinterpret_cast<const u32x4e_t*>(
                        st + enc_pos(128 * wr + 32 * i + (lane & 31), 2 * ks + (lane >> 5)));
                    __builtin_memcpy(&av[ks][i], &t, 16);
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const u32x4e_t t = *reinterpret_cast<const u32x4e_t*>(
                        st + kEM * kEK * 2 + enc_pos(64 * wc + 32 * j + (lane & 31), 2 * ks + (lane >> 5)));
                    __builtin_memcpy(&bv[ks][j], &t, 16);
                }
            }
            // all of the step's operand reads are in flight before its first product (only that
            // one waits for the LDS latency; the others' operands land under earlier products)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < kEK / 16; ++ks)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        if (kFull || (j == 0 ? cj0 : cj1))
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[ks][j], av[ks][i], acc[i][j], 0, 0, 0);
            if (bload) wait_vmcnt<2 * kELoads * (kEStages - 2)>();          // loads per step: A and B
            else wait_vmcnt<kELoads * (kEStages - 2)>();                    // A only
            bare_barrier();
        }
    };
    if (cj0 && cj1) k_loop(std::true_type{});
    else k_loop(std::false_type{});
    // the trailing loads write LDS that the epilogue reuses: all of them land first
    wait_vmcnt<0>();
    __syncthreads();

    if (li.g != 16) {
        // ---- group sizes other than 16 (2, 4, 8): the tile is quantised and packed by
        // quantise_tile in passes of 128 tokens x 128 columns; in each pass the two waves that
        // hold those accumulators put them into an LDS tile lat[128][129] first
        float* lat = reinterpret_cast<float*>(smem);
        uint8_t* cds_g = smem + 128 * 129 * 4;
        for (int rh = 0; rh < 2; ++rh) {
            const int64_t pr0 = row0 + 128 * rh;
            if (pr0 >= row_end) break;
            for (int ch = 0; ch < 2; ++ch) {
                const int pc0 = col0 + 128 * ch;
                const int pnc = min(128, N - pc0);
                if (pnc <= 0) break;
                __syncthreads();                       // the previous pass is done with lat and cds
                if (wr == rh && (wc >> 1) == ch) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 2; ++j)
#pragma unroll
                            for (int a = 0; a < 16; ++a)
                                lat[(32 * i + (lane & 31)) * 129 + 64 * (wc & 1) + 32 * j + 8 * (a >> 2) + 4 * (lane >> 5) +
                                    (a & 3)] = acc[i][j][a];
                }
                __syncthreads();
                quantise_tile(li, start, n_new, pr0, min(row_end, pr0 + 128), pc0, pnc, lat, 129, cds_g, 128, cache_k,
                              cache_v, seq_bytes_k, seq_bytes_v, latent_out, tid, 512);
            }
        }
        return;
    }

    // ---- epilogue: accumulator (i, j), element a of lane l holds C at tile row (token)
    // 128 wr + 32 i + l % 32 and tile column 64 wc + 32 j + 8 (a / 4) + 4 (l / 32) + a % 4.
    // Elements 0..7 and 8..15 are eight columns of the groups 4 wc + 2 j and 4 wc + 2 j + 1; the
    // lane 32 apart holds the other eight.  Codes go to a row-major tile cds[token][column]
    // (rows of kCdsRow bytes), four columns per 32-bit LDS write.
    uint8_t* cds = smem;
    const int ncol = min(kEN, N - col0);
    const int nrow = (int)(row_end - row0);
    // token positions: when the tile's rows belong to one sequence (the usual case), row row0 + rl
    // is position p0 + rl of sequence sb0, with no division per row
    const int sb0 = row_seq(row0, n_new);
    const int64_t p0 = start.v[sb0] + (row0 - (int64_t)sb0 * n_new);
    const bool one_seq = row_seq(row_end - 1, n_new) == sb0;
    // scales are collected in LDS (sct[group][token]) and written after the tile is done: as
    // whole 16-byte pieces of the scale chunks for a block-aligned tile of one sequence, else
    // entry by entry (the per-element code stays small: the epilogue is unrolled 128 times)
    const bool aligned = one_seq && p0 % kBT == 0;
    uint16_t* sct = reinterpret_cast<uint16_t*>(smem + kEM * kCdsRow);
    // per group of the tile: width and code offset in its block (read by the packing loop)
    int* gtab = reinterpret_cast<int*>(smem + kEM * kCdsRow + (kEN / 16) * kEM * 2);
    if (tid < kEN / 16 && 16 * tid < ncol) {
        const int col = col0 + 16 * tid;
        const int kind = col < rk ? 0 : 1;
        const int chunk = (col - (kind ? rk : 0)) >> 4;
        const TensorInfo& ti = li.t[kind];
        int coff = 0;
        for (int c = 0; c < chunk; ++c) coff += 256 * ti.width[c];
        gtab[2 * tid] = ti.width[chunk];
        gtab[2 * tid + 1] = coff;
    }
    __syncthreads();
    // one accumulator block at a time (explicit instances keep every register index constant)
    auto epi_block = [&](const f32x16_t& blkacc, int i, int j) {
        const int rl = 128 * wr + 32 * i + (lane & 31);                      // token in the tile
        const bool row_ok = rl < nrow;
#pragma unroll
        for (int hg = 0; hg < 2; ++hg) {
            const int gi = 4 * wc + 2 * j + hg;                               // group in the tile
            const bool grp_ok = 16 * gi < ncol;
            const int b = grp_ok ? gtab[2 * gi] : 1;
            float m = fabsf(blkacc[8 * hg]);
#pragma unroll
            for (int a = 1; a < 8; ++a) m = fmaxf(m, fabsf(blkacc[8 * hg + a]));
            const auto mx = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
            const float A = fmaxf(__uint_as_float(mx[0]), __uint_as_float(mx[1]));
            _Float16 s16 = (_Float16)(A * __uint_as_float((uint32_t)(128 - b) << 23));   // A 2^(1-b), exact; RNE
            if (__builtin_isinf((float)s16)) s16 = (_Float16)65504.0f;
            QuantGroup qg = quant_group(s16, b);
            uint16_t bits;
            __builtin_memcpy(&bits, &s16, 2);
            // both lanes of the pair hold the scale and write the same entry; entries of rows
            // past the end are never read
            sct[gi * kEM + rl] = bits;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                uint32_t packed = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) packed |= quant_div(blkacc[8 * hg + 4 * q + e], qg) << (8 * e);
                const int cl = 16 * gi + 8 * q + 4 * (lane >> 5);            // first of 4 columns
                // rows past the end hold zeros: a block's last words are packed whole
                *reinterpret_cast<uint32_t*>(cds + rl * kCdsRow + cl) = row_ok ? packed : 0u;
                if (latent_out && row_ok && grp_ok) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) latent_out[(row0 + rl) * N + col0 + cl + e] = blkacc[8 * hg + 4 * q + e];
                }
            }
        }
    };
    epi_block(acc[0][0], 0, 0); epi_block(acc[0][1], 0, 1);
    epi_block(acc[1][0], 1, 0); epi_block(acc[1][1], 1, 1);
    epi_block(acc[2][0], 2, 0); epi_block(acc[2][1], 2, 1);
    epi_block(acc[3][0], 3, 0); epi_block(acc[3][1], 3, 1);
    __syncthreads();

    // ---- pack.  Fast path: the tile's tokens are one sequence's positions p0 .. p0 + nrow with
    // p0 on a block boundary, so every code word of the tile's blocks belongs to this tile (words
    // past the last token hold zeros, as in a fresh cache): thread items are lane runs
    // (block, group, run L), each assembled from its 32 codes and stored as b plain words.
    if (!aligned) {
        for (int it = tid; it < 16 * nrow; it += 512) {
            const int gr = it / nrow, rl = it % nrow;
            const int col = col0 + 16 * gr;
            if (col >= col0 + ncol) continue;
            const int kind = col < rk ? 0 : 1;
            const int chunk = (col - (kind ? rk : 0)) >> 4;
            const TensorInfo& ti = li.t[kind];
            const int64_t row = row0 + rl;
            const int sb = one_seq ? sb0 : row_seq(row, n_new);
            const int64_t pos = one_seq ? p0 + rl : start.v[sb] + (row - (int64_t)sb * n_new);
            uint8_t* blk = (kind ? cache_v + sb * seq_bytes_v : cache_k + sb * seq_bytes_k) + (pos / kBT) * ti.block_bytes;
            reinterpret_cast<uint16_t*>(blk + ti.codes_bytes + 256 * chunk)[scale_index(kind, 16, (int)(pos % kBT))] =
                sct[gr * kEM + rl];
        }
        pack_tile(li, start, n_new, row0, row_end, col0, ncol, cds, kCdsRow, 1, cache_k, cache_v, seq_bytes_k,
                  seq_bytes_v, tid, 512);
        return;
    }
    const int nb = (nrow + kBT - 1) / kBT;
    const int ngr = (ncol + 15) / 16;
    // scales: 16-byte piece q (entries 8 q .. 8 q + 7) of the scale chunk of (block bi, group gr);
    // entry E holds slot E (V) or slot 32 (E % 4) + pi(E / 4) (K).  In the last, partial block
    // only the entries of this tile's tokens are written.
    for (int item = tid; item < nb * ngr * 16; item += 512) {
        const int q = item & 15, gr = (item >> 4) % ngr, bi = (item >> 4) / ngr;
        const int col = col0 + 16 * gr;
        const int kind = col < rk ? 0 : 1;
        const int chunk = (col - (kind ? rk : 0)) >> 4;
        const TensorInfo& ti = li.t[kind];
        uint16_t* dst = reinterpret_cast<uint16_t*>((kind ? cache_v + sb0 * seq_bytes_v : cache_k + sb0 * seq_bytes_k) +
                                                    (p0 / kBT + bi) * ti.block_bytes + ti.codes_bytes + 256 * chunk) + 8 * q;
        uint16_t v[8];
        int tau[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int E = 8 * q + e;
            tau[e] = kind == 0 ? 32 * (E & 3) + quarter_token(E >> 2) : E;
            v[e] = sct[gr * kEM + kBT * bi + tau[e]];
        }
        if (kBT * (bi + 1) <= nrow) {
            uint4 w4;
            w4.x = v[0] | ((uint32_t)v[1] << 16);
            w4.y = v[2] | ((uint32_t)v[3] << 16);
            w4.z = v[4] | ((uint32_t)v[5] << 16);
            w4.w = v[6] | ((uint32_t)v[7] << 16);
            *reinterpret_cast<uint4*>(dst) = w4;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (kBT * bi + tau[e] < nrow) dst[e] = v[e];
        }
    }
    for (int item = tid; item < nb * ngr * 64; item += 512) {
        const int L = item & 63, gr = (item >> 6) % ngr, bi = (item >> 6) / ngr;
        const int col = col0 + 16 * gr;
        const int kind = col < rk ? 0 : 1;
        const int chunk = (col - (kind ? rk : 0)) >> 4;
        const TensorInfo& ti = li.t[kind];
        const int b = gtab[2 * gr], coff = gtab[2 * gr + 1];
        // codes of the run: quarter T, e = 0..7
        uint32_t cd[32];                                     // codes (T, e) at 8 T + e
        if (kind == 0) {        // K: token 32 T + pi(m) (m = L % 32), coordinates 8 (L / 32) + e
            const uint8_t* cbase = cds + (kBT * bi + quarter_token(L & 31)) * kCdsRow + 16 * gr + 8 * (L >> 5);
#pragma unroll
            for (int T = 0; T < 4; ++T) {
                const uint2 v8 = *reinterpret_cast<const uint2*>(cbase + 32 * T * kCdsRow);   // 8-byte aligned
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    cd[8 * T + e] = (v8.x >> (8 * e)) & 0xFFu;
                    cd[8 * T + 4 + e] = (v8.y >> (8 * e)) & 0xFFu;
                }
            }
        } else {                // V: coordinate L % 16, tokens 32 T + 8 (L / 16) + e
            const uint8_t* cbase = cds + (kBT * bi + 8 * (L >> 4)) * kCdsRow + 16 * gr + (L & 15);
#pragma unroll
            for (int T = 0; T < 4; ++T)
#pragma unroll
                for (int e = 0; e < 8; ++e) cd[8 * T + e] = cbase[(32 * T + e) * kCdsRow];
        }
        uint32_t wd[8];
        switch (b) {                                         // b is the same for the whole wave
            case 1: run_words<1>(cd, wd); break;
            case 2: run_words<2>(cd, wd); break;
            case 3: run_words<3>(cd, wd); break;
            case 4: run_words<4>(cd, wd); break;
            case 5: run_words<5>(cd, wd); break;
            case 6: run_words<6>(cd, wd); break;
            case 7: run_words<7>(cd, wd); break;
            default: run_words<8>(cd, wd); break;
        }
        uint32_t* words = reinterpret_cast<uint32_t*>((kind ? cache_v + sb0 * seq_bytes_v : cache_k + sb0 * seq_bytes_k) +
                                                      (p0 / kBT + bi) * ti.block_bytes + coff);
        const bool full = kBT * (bi + 1) <= nrow;
#pragma unroll
        for (int kw = 0; kw < 8; ++kw) {
            if (kw < b) {
                if (full) words[64 * kw + L] = wd[kw];
                else atomicOr(words + 64 * kw + L, wd[kw]);  // block shared with later tokens
            }
        }
    }
}

}  // namespace spectra

using namespace spectra;

extern "C" spectra_status spectra_encode_append(const spectra_layout* layout, spectra_dtype dtype, const void* x,
                                                int32_t batch, int32_t n_new, const void* w_down_t, void* cache_k,
                                                void* cache_v, int64_t cap_tokens, const int32_t* start_pos,
                                                float* latent_out, void* stream) {
    clear_error();
    LayoutInfo li;
    spectra_status st = make_layout(layout, &li);
    if (st) return st;
    if (dtype != SPECTRA_F32 && dtype != SPECTRA_BF16) return fail(SPECTRA_ENOTSUP, "encode: unknown dtype %d", (int)dtype);
    if (batch <= 0 || n_new < 0) return fail(SPECTRA_EINVAL, "encode: batch must be positive, n_new non-negative");
    if (batch > kMaxB) return fail(SPECTRA_ENOTSUP, "encode: batch %d > %d", batch, kMaxB);
    if (!x || !w_down_t || !cache_k || !cache_v || !start_pos) return fail(SPECTRA_EINVAL, "encode: NULL pointer argument");
    if (li.d_model % kTK) return fail(SPECTRA_ENOTSUP, "encode: d_model %d not a multiple of %d", li.d_model, kTK);
    if (kTN % li.g) return fail(SPECTRA_ENOTSUP, "encode: group size %d does not divide %d", li.g, kTN);
    Positions sp;
    std::memset(&sp, 0, sizeof sp);
    for (int b = 0; b < batch; ++b) {
        if (start_pos[b] < 0 || (int64_t)start_pos[b] + n_new > cap_tokens)
            return fail(SPECTRA_ECAPACITY, "encode: positions [%d, %lld) of sequence %d exceed capacity %lld", start_pos[b],
                        (long long)start_pos[b] + n_new, b, (long long)cap_tokens);
        sp.v[b] = start_pos[b];
    }
    const int N = li.t[0].r_act + li.t[1].r_act;
    const int64_t M = (int64_t)batch * n_new;
    if (M == 0 || N == 0) return SPECTRA_OK;
    const int64_t nblk = (cap_tokens + kBT - 1) / kBT;
    const int64_t sbk = nblk * li.t[0].block_bytes, sbv = nblk * li.t[1].block_bytes;
    dim3 grid((N + kTN - 1) / kTN, (unsigned)((M + kTM - 1) / kTM));
    hipStream_t s = (hipStream_t)stream;
    constexpr int64_t kSmallEncodeRows = 64;           // bf16 or fp32
    constexpr int64_t kSmallEncodeF32 = 1 << 16;       // fp32: rows x columns
    // few rows (appends while decoding) or a small float32 problem: 16 x 16 tiles over all of d_model
    if (kSC % li.g == 0 && li.d_model % kSK == 0 &&
        (M <= kSmallEncodeRows || (dtype == SPECTRA_F32 && M * N <= kSmallEncodeF32))) {
        const dim3 gs((N + kSC - 1) / kSC, (unsigned)((M + kSR - 1) / kSR));
        if (dtype == SPECTRA_BF16)
            hipLaunchKernelGGL(encode_small_kernel<uint16_t>, gs, dim3(256), 0, s, li, sp, batch, n_new,
                               (const uint16_t*)x, (const uint16_t*)w_down_t, (uint8_t*)cache_k, (uint8_t*)cache_v,
                               sbk, sbv, latent_out);
        else
            hipLaunchKernelGGL(encode_small_kernel<float>, gs, dim3(256), 0, s, li, sp, batch, n_new, (const float*)x,
                               (const float*)w_down_t, (uint8_t*)cache_k, (uint8_t*)cache_v, sbk, sbv, latent_out);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(SPECTRA_EHIP, "encode: %s", hipGetErrorString(e));
        return SPECTRA_OK;
    }
    const bool mfma_path = dtype == SPECTRA_BF16 && kSC % li.g == 0 && li.d_model % kEK == 0;
    if (mfma_path ? !reserve_lds((const void*)encode_mfma_kernel, kEncodeMfmaLds)
                  : !reserve_lds(dtype == SPECTRA_BF16 ? (const void*)encode_kernel<uint16_t> : (const void*)encode_kernel<float>, kEncodeLds))
        return fail(SPECTRA_EHIP, "encode: cannot reserve %d bytes of LDS", mfma_path ? kEncodeMfmaLds : kEncodeLds);
    if (mfma_path) {
        const int nct = (N + kEN - 1) / kEN;
        const int64_t nrt = (M + kEM - 1) / kEM;
        const int64_t nrt8 = (nrt + 7) / 8 * 8;                // row tiles padded to whole XCD rounds
        hipLaunchKernelGGL(encode_mfma_kernel, dim3((unsigned)(nrt8 * nct)), dim3(512), kEncodeMfmaLds, s, li, sp, batch,
                           n_new, (const uint16_t*)x, (const uint16_t*)w_down_t, (uint8_t*)cache_k, (uint8_t*)cache_v,
                           sbk, sbv, latent_out, nct);
    } else if (dtype == SPECTRA_BF16)
        hipLaunchKernelGGL(encode_kernel<uint16_t>, grid, dim3(256), kEncodeLds, s, li, sp, batch, n_new,
                           (const uint16_t*)x, (const uint16_t*)w_down_t, (uint8_t*)cache_k, (uint8_t*)cache_v, sbk, sbv,
                           latent_out);
    else
        hipLaunchKernelGGL(encode_kernel<float>, grid, dim3(256), kEncodeLds, s, li, sp, batch, n_new, (const float*)x,
                           (const float*)w_down_t, (uint8_t*)cache_k, (uint8_t*)cache_v, sbk, sbv, latent_out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SPECTRA_EHIP, "encode: %s", hipGetErrorString(e));
    return SPECTRA_OK;
}
