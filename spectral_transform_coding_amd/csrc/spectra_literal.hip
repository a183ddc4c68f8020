// Literal decode of libspectra (gfx950): keys and values are rebuilt from the packed latent
// and attended, the order in which the SPECTRA pipeline's stage 3 states the decode.  The
// product path (spectra_decode_attn) computes the same attention in latent space; this path
// exists to measure what that saves, and is checked against the same float64 attention.
//
//   lift    K^ = C^_K W_up_K, V^ = C^_V W_up_V for every cached token (matrix cores, f16
//           operands, float32 accumulation), written to the workspace in float32;
//   attend  split-K online softmax of each query head over K^, V^ (float32 VALU);
//   merge   the splits of each query head.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>

#include "spectra_device.h"

namespace spectra {

constexpr int kLitRMax = 512;            // latent rank per segment
constexpr int kLitQ = 8;                 // query heads per key/value head
constexpr int kLitDh = 256;              // head dimension
constexpr int kLitTile = 64;             // tokens per attention tile (one per lane)

static int lit_rank_pad(const LayoutInfo& li) {
    int r = 0;
    for (int t = 0; t < 2; ++t)
        for (int s = 0; s < li.n_seg; ++s) r = std::max(r, li.g * (li.t[t].seg_chunk0[s + 1] - li.t[t].seg_chunk0[s]));
    return std::max(16, (r + 15) / 16 * 16);
}

// W_up of one tensor as fp16 terms in k-blocks of 8 per segment: wt[0][s][k / 8][n][k % 8] =
// fp16(W[row0_s + k, n]), wt[1][...] = fp16(W - fp16(W)) (zero for bf16 weights), zero for k at
// or past the segment's rank (grid-stride over n_seg x seg_cols x RP).  A 32x32x16 product's
// B operand (8 consecutive k of 32 consecutive columns) is then one contiguous 512-byte run.
template <typename DT>
__global__ __launch_bounds__(256) void literal_wt_kernel(LayoutInfo li, int kind, const DT* __restrict__ w, int RP,
                                                          _Float16* __restrict__ wt) {
    const TensorInfo& T = li.t[kind];
    const int64_t total = (int64_t)li.n_seg * li.seg_cols * RP;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
        const int e = (int)(idx % 8);
        const int n = (int)((idx / 8) % li.seg_cols);
        const int kb = (int)((idx / (8 * li.seg_cols)) % (RP / 8));
        const int s = (int)(idx / ((int64_t)RP * li.seg_cols));
        const int k = 8 * kb + e;
        const int rs = li.g * (T.seg_chunk0[s + 1] - T.seg_chunk0[s]);
        const float v = k < rs ? load_f32(w, (int64_t)(li.g * T.seg_chunk0[s] + k) * li.seg_cols + n) : 0.0f;
        const _Float16 hi = (_Float16)v;
        wt[idx] = hi;
        wt[total + idx] = (_Float16)(v - (float)hi);
    }
}

// Lift (grid: half cache blocks, sequence, tensor; 512 threads).  For each segment the 64
// tokens' dequantised latents C^_s (thread = one latent column, rows in batches of 8 whose code
// words and scales are all requested before any is used; the column's chunk, width and offsets
// from a table in LDS) are staged in LDS as fp16 hi = fp16(c), and for keys also
// lo = fp16(c - hi) (scores amplify key errors through the softmax; value errors enter
// linearly); wave w then computes column tiles 2p, 2p + 1 (32 columns each) for
// p = w, w + 8, ... over the 64 tokens with 32x32x16 f16 products: A = latent terms from LDS,
// B = 16-byte pieces of the k-blocked W_up terms read from memory (L2-resident), the W lo term
// only for float32 weights.  Output rows = the tokens' rows of out
// [batch][rows_per_seq][n_kv d_head], float32.
// Words of (slot tau, coordinate j)'s b-bit code in a chunk (the cache layout of read_code):
// its code is ((w[i0] >> sh) >> off | (w[i1] >> sh) << (lim - off)) & mask, the second word
// read whole whatever the code's position (it is inside the block: the next chunk or the
// scale chunks follow every chunk), so that a batch of codes needs no branch.
struct LitCode {
    int i0, i1, off, sh, lim;
};
__device__ __forceinline__ LitCode lit_code_at(int kind, int g, int b, int tau, int j) {
    LitCode c;
    if (g != 16) {
        const int bit = (tau * g + j) * b;
        c.i0 = bit >> 5;
        c.i1 = c.i0 + 1;
        c.off = bit & 31;
        c.sh = 0;
        c.lim = 32;
    } else {
        int L, T, e;
        run_of(kind, tau, j, &L, &T, &e);
        const int gam = (4 * T + (e >> 1)) * b;
        c.i0 = 64 * (gam >> 4) + L;
        c.i1 = c.i0 + 64;
        c.off = gam & 15;
        c.sh = 16 * (e & 1);
        c.lim = 16;
    }
    return c;
}
__device__ __forceinline__ uint32_t lit_code(const LitCode& c, uint32_t w0, uint32_t w1, int b) {
    const uint32_t hm = c.lim == 16 ? 0xFFFFu : 0xFFFFFFFFu;
    const uint32_t lo = ((w0 >> c.sh) & hm) >> c.off;
    const uint32_t hi = c.off + b > c.lim ? ((w1 >> c.sh) & hm) << (c.lim - c.off) : 0u;
    return (lo | hi) & ((1u << b) - 1u);
}

template <bool LO>
__global__ __launch_bounds__(512) void literal_lift_kernel(LayoutInfo li, Positions ctx, const uint8_t* __restrict__ cache_k,
                                                           const uint8_t* __restrict__ cache_v, int64_t seq_bytes_k,
                                                           int64_t seq_bytes_v, const _Float16* __restrict__ wt_k,
                                                           const _Float16* __restrict__ wt_v, int RP,
                                                           float* __restrict__ kh, float* __restrict__ vh,
                                                           int64_t rows_per_seq) {
    const int blk = blockIdx.x >> 1, half = blockIdx.x & 1, b = blockIdx.y, kind = blockIdx.z;
    if ((int64_t)blk * kBT + 64 * half >= ctx.v[b]) return;
    const TensorInfo& T = li.t[kind];
    const uint8_t* bp = (kind ? cache_v + (int64_t)b * seq_bytes_v : cache_k + (int64_t)b * seq_bytes_k) +
                        (int64_t)blk * T.block_bytes;
    const _Float16* wt = kind ? wt_v : wt_k;
    const int64_t wt_terms = (int64_t)li.n_seg * li.seg_cols * RP;
    const int ncols = li.n_kv * li.d_head;
    float* out = (kind ? vh : kh) + ((int64_t)b * rows_per_seq + (int64_t)blk * kBT + 64 * half) * ncols;
    const int KP = RP + 8;                            // LDS row stride (halves): rows 16-byte aligned
    extern __shared__ __align__(16) unsigned char smem[];
    _Float16* cl = reinterpret_cast<_Float16*>(smem);                  // hi terms [64][KP]
    _Float16* cll = cl + 64 * KP;                                       // lo terms [64][KP] (keys)
    int* coff = reinterpret_cast<int*>(cll + 64 * KP);                  // code offset of each chunk
    int* ctab = coff + kMaxC;                                           // [3][RP] per latent column
    const bool alo = kind == 0;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, m = lane & 31, kh2 = lane >> 5;
    if (tid == 0) {
        int o = 0;
        for (int c = 0; c < T.n_chunks; ++c) {
            coff[c] = o;
            o += 16 * li.g * T.width[c];
        }
    }
    for (int s = 0; s < li.n_seg; ++s) {
        const int c0 = T.seg_chunk0[s], rs = li.g * (T.seg_chunk0[s + 1] - c0);
        const int rp = (rs + 15) / 16 * 16;
        __syncthreads();                              // offsets written; previous segment consumed
        // column table: code chunk offset, width | coordinate << 8, scale chunk offset
        for (int i = tid; i < rs; i += 512) {
            const int c = c0 + i / li.g;
            ctab[i] = coff[c];
            ctab[RP + i] = T.width[c] | ((i % li.g) << 8);
            ctab[2 * RP + i] = T.codes_bytes + 256 * c;
        }
        __syncthreads();
        // thread -> column i = tid % rp, rows r0, r0 + rpp, ... (rpp = 512 / rp rows per pass)
        const int rpp = rp ? 512 / rp : 0, ci = rp ? tid % rp : 0, r0 = rp ? tid / rp : 0;
        if (r0 < rpp) {                               // none for a segment without active groups
            const bool live = ci < rs;
            const int co = live ? ctab[ci] : 0, wj = live ? ctab[RP + ci] : 1, so = live ? ctab[2 * RP + ci] : 0;
            const int bw = wj & 0xFF, jj = wj >> 8;
            const float hoff = 0.5f * (float)((1u << bw) - 1u);
            const uint32_t* w = reinterpret_cast<const uint32_t*>(bp + co);
            const uint16_t* sp = reinterpret_cast<const uint16_t*>(bp + so);
            for (int rb = r0; rb < 64; rb += 8 * rpp) {
                uint32_t w0[8], w1[8];
                uint16_t sb[8];
                LitCode cd[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int r = rb + rpp * u, tau = 64 * half + r;
                    cd[u] = LitCode{0, 0, 0, 0, 32};
                    w0[u] = w1[u] = 0u;
                    sb[u] = 0;
                    if (live && r < 64) {
                        cd[u] = lit_code_at(kind, li.g, bw, tau, jj);
                        w0[u] = w[cd[u].i0];
                        w1[u] = w[cd[u].i1];
                        sb[u] = sp[scale_index(kind, li.g, tau)];
                    }
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int r = rb + rpp * u;
                    if (r >= 64) break;
                    const float v = live ? f16_bits_to_f32(sb[u]) * ((float)lit_code(cd[u], w0[u], w1[u], bw) - hoff) : 0.0f;
                    const _Float16 hi = (_Float16)v;
                    cl[r * KP + ci] = hi;
                    cll[r * KP + ci] = (_Float16)(v - (float)hi);
                }
            }
        }
        __syncthreads();
        const _Float16* ws = wt + (int64_t)s * li.seg_cols * RP;
        for (int p = wv; 64 * p < li.seg_cols; p += 8) {
            const int nb = 64 * p, ntl = std::min(2, (li.seg_cols - nb) / 32);
            f32x16_t acc[2][2];
#pragma unroll
            for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = f32x16_t{};
            // B operands of kKB k-steps are requested together (the transposed terms were written
            // by another XCD's kernel: they come from beyond this XCD's L2)
            constexpr int kKB = 4;
            for (int kb0 = 0; kb0 < rp; kb0 += 16 * kKB) {
                half8_t bh[kKB][2], bl[kKB][2];
#pragma unroll
                for (int u = 0; u < kKB; ++u) {
                    const int k0 = std::min(kb0 + 16 * u, rp - 16);          // in range; unused past rp
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int n = nb + 32 * std::min(j, ntl - 1) + m;   // a valid column
                        const _Float16* src = ws + ((int64_t)(k0 / 8 + kh2) * li.seg_cols + n) * 8;
                        bh[u][j] = *reinterpret_cast<const half8_t*>(src);
                        if constexpr (LO) bl[u][j] = *reinterpret_cast<const half8_t*>(src + wt_terms);
                    }
                }
#pragma unroll
                for (int u = 0; u < kKB; ++u) {
                    const int k0 = kb0 + 16 * u;
                    if (k0 >= rp) break;
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const int ao = (32 * i + m) * KP + k0 + 8 * kh2;
                        const half8_t a = *reinterpret_cast<const half8_t*>(cl + ao);
                        const half8_t al = *reinterpret_cast<const half8_t*>(cll + ao);
#pragma unroll
                        for (int j = 0; j < 2; ++j) {
                            if (j < ntl) {
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bh[u][j], acc[i][j], 0, 0, 0);
                                if (alo) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, bh[u][j], acc[i][j], 0, 0, 0);
                                if constexpr (LO)
                                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bl[u][j], acc[i][j], 0, 0, 0);
                            }
                        }
                    }
                }
            }
            // acc[i][j][4 r + e]: token 32 i + 8 r + 4 kh2 + e of the 64, column nb + 32 j + m
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    if (j >= ntl) continue;
#pragma unroll
                    for (int t = 0; t < 16; ++t) {
                        const int row = 32 * i + 8 * (t >> 2) + 4 * kh2 + (t & 3);
                        out[(int64_t)row * ncols + s * li.seg_cols + nb + 32 * j + m] = acc[i][j][t];
                    }
                }
        }
    }
}

// Attend (grid: splits, key/value head, sequence; 256 threads).  Per 64-token tile the keys are
// staged in LDS with 16-byte loads (a thread's loads of a round all issued before any store),
// rows past the context as zeros; thread pairs (token, head) form the scores; wave w then
// takes head w (w + 4, ...): tile maximum and sum over its 64 lanes, base-2 online softmax with
// one running maximum and sum per head (scores scaled by qscale = softmax_scale log2 e); the
// values are staged the same way and thread pairs (head, dimension) accumulate the output.
// Partials pm, pl [batch][splits][n_q], po [batch][splits][n_q][d_head].  Dynamic LDS:
// 64 (d_head + 4) + q_per_kv (d_head + 64) + 3 q_per_kv floats.
constexpr int kLitOut = kLitQ * kLitDh / 256;      // (head, dimension) pairs per thread
__device__ __forceinline__ void lit_stage(float* xt, int ld, const float* src, int64_t ncols, int64_t row0,
                                          int64_t rows_valid, int dh, int tid) {
    const int n4 = dh / 4, items = kLitTile * n4;
    for (int base = 0; base < items; base += 256 * 8) {
        f32x4_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int idx = base + tid + 256 * u, r = idx / n4, c = idx % n4;
            v[u] = f32x4_t{0, 0, 0, 0};
            if (idx < items && r < rows_valid) v[u] = *reinterpret_cast<const f32x4_t*>(src + (row0 + r) * ncols + 4 * c);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int idx = base + tid + 256 * u, r = idx / n4, c = idx % n4;
            if (idx < items) *reinterpret_cast<f32x4_t*>(xt + r * ld + 4 * c) = v[u];
        }
    }
}
__global__ __launch_bounds__(256) void literal_attn_kernel(LayoutInfo li, Positions ctx, const float* __restrict__ q,
                                                           float qscale, const float* __restrict__ kh,
                                                           const float* __restrict__ vh, int64_t rows_per_seq,
                                                           int split_tokens, int n_splits, float* __restrict__ pm,
                                                           float* __restrict__ pl, float* __restrict__ po) {
    const int split = blockIdx.x, kv = blockIdx.y, b = blockIdx.z, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int dh = li.d_head, nq = li.q_per_kv, ncols = li.n_kv * dh, h0 = kv * nq, ld = dh + 4;
    const int64_t t0 = (int64_t)split * split_tokens;
    const int64_t t1 = std::min<int64_t>(ctx.v[b], t0 + split_tokens);
    if (t0 >= t1) return;
    extern __shared__ __align__(16) float lsm[];
    float* xt = lsm;                                  // [64][ld] keys, then values
    float* qs = xt + kLitTile * ld;                   // [nq][dh] scaled query
    float* ps = qs + nq * dh;                         // [nq][64] scores, then probabilities
    float* mh = ps + nq * kLitTile;                   // [nq] running maximum
    float* lh = mh + nq;                              // [nq] running sum
    float* al = lh + nq;                              // [nq] this tile's rescale factor
    for (int i = tid; i < nq * dh; i += 256) qs[i] = q[((int64_t)b * li.n_q + h0) * dh + i] * qscale;
    if (tid < nq) {
        mh[tid] = -INFINITY;
        lh[tid] = 0.0f;
    }
    float o[kLitOut];
#pragma unroll
    for (int k = 0; k < kLitOut; ++k) o[k] = 0.0f;   // fixed (head, dimension) pairs per thread
    const float* kb = kh + (int64_t)b * rows_per_seq * ncols + kv * dh;
    const float* vb = vh + (int64_t)b * rows_per_seq * ncols + kv * dh;
    for (int64_t tile = t0; tile < t1; tile += kLitTile) {
        const int64_t nvalid = std::min<int64_t>(kLitTile, t1 - tile);
        __syncthreads();                              // previous tile's values and factors consumed
        lit_stage(xt, ld, kb, ncols, tile, nvalid, dh, tid);
        __syncthreads();
        for (int pr = tid; pr < nq * kLitTile; pr += 256) {
            const int t = pr % kLitTile, h = pr / kLitTile;
            float sc = 0.0f;
#pragma unroll 4
            for (int d = 0; d < dh; d += 4) {
                const f32x4_t x = *reinterpret_cast<const f32x4_t*>(xt + t * ld + d);
                const f32x4_t y = *reinterpret_cast<const f32x4_t*>(qs + h * dh + d);
                sc += x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
            }
            ps[h * kLitTile + t] = t < nvalid ? sc : -INFINITY;
        }
        __syncthreads();
        for (int h = wv; h < nq; h += 4) {
            const float s = ps[h * kLitTile + lane];
            float mt = s;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) mt = fmaxf(mt, __shfl_xor(mt, off));
            const float mold = mh[h];
            const float mn = fmaxf(mold, mt);          // finite: the tile holds a valid token
            const float p = s == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(s - mn);
            float ls = p;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) ls += __shfl_xor(ls, off);
            ps[h * kLitTile + lane] = p;
            if (lane == 0) {
                const float a = __builtin_amdgcn_exp2f(mold - mn);   // 0 while mold = -inf
                al[h] = a;
                lh[h] = lh[h] * a + ls;
                mh[h] = mn;
            }
        }
        lit_stage(xt, ld, vb, ncols, tile, nvalid, dh, tid);   // keys were consumed before the barrier above
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kLitOut; ++k) {
            const int pr = tid + 256 * k;
            if (pr >= nq * dh) break;
            const int h = pr / dh, d = pr % dh;
            float acc = o[k] * al[h];
#pragma unroll 8
            for (int t = 0; t < kLitTile; ++t) acc += ps[h * kLitTile + t] * xt[t * ld + d];
            o[k] = acc;
        }
    }
    __syncthreads();
    const int64_t base = ((int64_t)b * n_splits + split) * li.n_q + h0;
    if (tid < nq) {
        pm[base + tid] = mh[tid];
        pl[base + tid] = lh[tid];
    }
#pragma unroll
    for (int k = 0; k < kLitOut; ++k) {
        const int pr = tid + 256 * k;
        if (pr >= nq * dh) break;
        po[(base + pr / dh) * dh + pr % dh] = o[k];
    }
}

// Merge (grid: query head, sequence; 256 threads): M = max_s m_s, L = sum_s 2^(m_s - M) l_s,
// o[d] = sum_s 2^(m_s - M) o_s[d] / L (zero for an empty context).
__global__ __launch_bounds__(256) void literal_merge_kernel(LayoutInfo li, Positions ctx, const float* __restrict__ pm,
                                                            const float* __restrict__ pl, const float* __restrict__ po,
                                                            int split_tokens, int n_splits, float* __restrict__ out) {
    const int h = blockIdx.x, b = blockIdx.y, dh = li.d_head;
    const int ns = ctx.v[b] <= 0 ? 0 : (ctx.v[b] + split_tokens - 1) / split_tokens;
    const int64_t base = (int64_t)b * n_splits * li.n_q + h;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, pm[base + (int64_t)s * li.n_q]);
    float L = 0.0f;
    for (int s = 0; s < ns; ++s) L += __builtin_amdgcn_exp2f(pm[base + (int64_t)s * li.n_q] - M) * pl[base + (int64_t)s * li.n_q];
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    for (int d = threadIdx.x; d < dh; d += 256) {
        float acc = 0.0f;
        for (int s = 0; s < ns; ++s)
            acc += __builtin_amdgcn_exp2f(pm[base + (int64_t)s * li.n_q] - M) * po[(base + (int64_t)s * li.n_q) * dh + d];
        out[((int64_t)b * li.n_q + h) * dh + d] = acc * inv;
    }
}

// Query in float32 for the attend kernel (bf16 or float32 input).
template <typename DT>
__global__ __launch_bounds__(256) void literal_q_kernel(const DT* __restrict__ q, int64_t n, float* __restrict__ qf) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) qf[i] = load_f32(q, i);
}

struct LitPlan {
    int RP;
    int64_t rows_per_seq;
    int split_tokens, n_splits;
    size_t off_kh, off_vh, off_wk, off_wv, off_q, off_pm, off_pl, off_po, total;
};

static size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

// With for_size the split partials are sized for the largest split count any context up to
// max_ctx can take (a shorter context can take more, shorter splits), so that a workspace sized
// for max_ctx serves every shorter context too.
static LitPlan lit_plan(const LayoutInfo& li, int B, int64_t max_ctx, bool for_size = false) {
    LitPlan p{};
    p.RP = lit_rank_pad(li);
    const int64_t blocks = std::max<int64_t>(1, (max_ctx + kBT - 1) / kBT);
    p.rows_per_seq = blocks * kBT;
    // about 2048 one-wave workgroups in the attend kernel, splits of whole 64-token tiles
    const int64_t tiles = std::max<int64_t>(1, (max_ctx + kLitTile - 1) / kLitTile);
    const int64_t units = (int64_t)B * li.n_kv;
    const int64_t per_seq = std::min<int64_t>(tiles, std::max<int64_t>(1, (2048 + units - 1) / units));
    const int64_t tps = (tiles + per_seq - 1) / per_seq;
    p.split_tokens = (int)(tps * kLitTile);
    p.n_splits = (int)((tiles + tps - 1) / tps);
    const size_t splits = for_size ? (size_t)per_seq : (size_t)p.n_splits;   // ceil(n / ceil(n / k)) <= k
    const size_t ncols = (size_t)li.n_kv * li.d_head;
    const size_t wterms = (size_t)li.n_seg * li.seg_cols * p.RP * 2;
    size_t o = 0;
    p.off_kh = o; o += a256((size_t)B * p.rows_per_seq * ncols * 4);
    p.off_vh = o; o += a256((size_t)B * p.rows_per_seq * ncols * 4);
    p.off_wk = o; o += a256(wterms * 2);
    p.off_wv = o; o += a256(wterms * 2);
    p.off_q = o;  o += a256((size_t)B * li.n_q * li.d_head * 4);
    p.off_pm = o; o += a256((size_t)B * splits * li.n_q * 4);
    p.off_pl = o; o += a256((size_t)B * splits * li.n_q * 4);
    p.off_po = o; o += a256((size_t)B * splits * li.n_q * li.d_head * 4);
    p.total = o;
    return p;
}

static spectra_status lit_hip_check(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SPECTRA_EHIP, "%s: %s", what, hipGetErrorString(e));
    return SPECTRA_OK;
}

// Shape limits of the literal path (reported as ENOTSUP).
static spectra_status lit_supported(const LayoutInfo& li) {
    if (li.q_per_kv > kLitQ) return fail(SPECTRA_ENOTSUP, "literal decode: more than %d query heads per key/value head", kLitQ);
    if (li.d_head > kLitDh || li.d_head % 4) return fail(SPECTRA_ENOTSUP, "literal decode: d_head must be a multiple of 4 up to %d", kLitDh);
    if (li.seg_cols % 32) return fail(SPECTRA_ENOTSUP, "literal decode: segment width %d not a multiple of 32", li.seg_cols);
    if (lit_rank_pad(li) > kLitRMax) return fail(SPECTRA_ENOTSUP, "literal decode: segment rank above %d", kLitRMax);
    return SPECTRA_OK;
}

}  // namespace spectra

using namespace spectra;

extern "C" {

spectra_status spectra_decode_literal_workspace_bytes(const spectra_layout* layout, int32_t batch, int64_t max_ctx,
                                                      size_t* bytes) {
    clear_error();
    LayoutInfo li;
    spectra_status st = make_layout(layout, &li);
    if (st) return st;
    if (!bytes) return fail(SPECTRA_EINVAL, "literal workspace: NULL output");
    if (batch <= 0 || max_ctx < 0) return fail(SPECTRA_EINVAL, "literal workspace: bad batch or context");
    if ((st = lit_supported(li))) return st;
    *bytes = lit_plan(li, batch, max_ctx, true).total;
    return SPECTRA_OK;
}

spectra_status spectra_decode_attn_literal(const spectra_layout* layout, spectra_dtype dtype, const void* q,
                                           const void* cache_k, const void* cache_v, int64_t cap_tokens,
                                           int32_t batch, const int32_t* ctx_len, const void* w_up_k,
                                           const void* w_up_v, float softmax_scale, float* out, void* workspace,
                                           size_t workspace_bytes, void* stream) {
    clear_error();
    LayoutInfo li;
    spectra_status st = make_layout(layout, &li);
    if (st) return st;
    if (dtype != SPECTRA_F32 && dtype != SPECTRA_BF16) return fail(SPECTRA_ENOTSUP, "literal decode: unknown dtype %d", (int)dtype);
    if (batch <= 0) return fail(SPECTRA_EINVAL, "literal decode: batch must be positive");
    if (batch > kMaxB) return fail(SPECTRA_ENOTSUP, "literal decode: batch %d > %d", batch, kMaxB);
    if (!q || !cache_k || !cache_v || !ctx_len || !w_up_k || !w_up_v || !out || !workspace)
        return fail(SPECTRA_EINVAL, "literal decode: NULL pointer argument");
    if (cap_tokens <= 0) return fail(SPECTRA_EINVAL, "literal decode: capacity must be positive");
    if ((st = lit_supported(li))) return st;
    Positions ctx;
    std::memset(&ctx, 0, sizeof ctx);
    int64_t max_ctx = 0;
    for (int b = 0; b < batch; ++b) {
        if (ctx_len[b] < 0 || ctx_len[b] > cap_tokens)
            return fail(SPECTRA_ECAPACITY, "literal decode: ctx_len[%d] = %d outside [0, %lld]", b, ctx_len[b],
                        (long long)cap_tokens);
        ctx.v[b] = ctx_len[b];
        max_ctx = std::max<int64_t>(max_ctx, ctx_len[b]);
    }
    const LitPlan p = lit_plan(li, batch, max_ctx);
    if (workspace_bytes < p.total)
        return fail(SPECTRA_ECAPACITY, "literal decode: workspace %zu bytes < %zu needed", workspace_bytes, p.total);
    hipStream_t s = (hipStream_t)stream;
    unsigned char* ws = (unsigned char*)workspace;
    float* kh = (float*)(ws + p.off_kh);
    float* vh = (float*)(ws + p.off_vh);
    _Float16* wk = (_Float16*)(ws + p.off_wk);
    _Float16* wv = (_Float16*)(ws + p.off_wv);
    float* qf = (float*)(ws + p.off_q);
    float* pm = (float*)(ws + p.off_pm);
    float* pl = (float*)(ws + p.off_pl);
    float* po = (float*)(ws + p.off_po);
    const bool bf = dtype == SPECTRA_BF16;
    const int64_t wterms = (int64_t)li.n_seg * li.seg_cols * p.RP;
    const unsigned wgrid = (unsigned)std::min<int64_t>(4096, (wterms + 255) / 256);
    const int64_t nq = (int64_t)batch * li.n_q * li.d_head;
    if (bf) {
        hipLaunchKernelGGL(literal_wt_kernel<uint16_t>, dim3(wgrid), dim3(256), 0, s, li, 0, (const uint16_t*)w_up_k, p.RP, wk);
        hipLaunchKernelGGL(literal_wt_kernel<uint16_t>, dim3(wgrid), dim3(256), 0, s, li, 1, (const uint16_t*)w_up_v, p.RP, wv);
        hipLaunchKernelGGL(literal_q_kernel<uint16_t>, dim3((unsigned)((nq + 255) / 256)), dim3(256), 0, s,
                           (const uint16_t*)q, nq, qf);
    } else {
        hipLaunchKernelGGL(literal_wt_kernel<float>, dim3(wgrid), dim3(256), 0, s, li, 0, (const float*)w_up_k, p.RP, wk);
        hipLaunchKernelGGL(literal_wt_kernel<float>, dim3(wgrid), dim3(256), 0, s, li, 1, (const float*)w_up_v, p.RP, wv);
        hipLaunchKernelGGL(literal_q_kernel<float>, dim3((unsigned)((nq + 255) / 256)), dim3(256), 0, s,
                           (const float*)q, nq, qf);
    }
    if ((st = lit_hip_check("literal decode: weights"))) return st;
    if (max_ctx > 0) {
        const int64_t nblk_cap = (cap_tokens + kBT - 1) / kBT;
        const int lds = 2 * 64 * (p.RP + 8) * 2 + kMaxC * 4 + 3 * p.RP * 4;
        const void* fn = bf ? (const void*)literal_lift_kernel<false> : (const void*)literal_lift_kernel<true>;
        if (!reserve_lds(fn, lds)) return fail(SPECTRA_EHIP, "literal decode: cannot reserve %d bytes of LDS", lds);
        const dim3 g((unsigned)(2 * ((max_ctx + kBT - 1) / kBT)), batch, 2);
        if (bf)
            hipLaunchKernelGGL(literal_lift_kernel<false>, g, dim3(512), lds, s, li, ctx, (const uint8_t*)cache_k,
                               (const uint8_t*)cache_v, nblk_cap * li.t[0].block_bytes, nblk_cap * li.t[1].block_bytes,
                               wk, wv, p.RP, kh, vh, p.rows_per_seq);
        else
            hipLaunchKernelGGL(literal_lift_kernel<true>, g, dim3(512), lds, s, li, ctx, (const uint8_t*)cache_k,
                               (const uint8_t*)cache_v, nblk_cap * li.t[0].block_bytes, nblk_cap * li.t[1].block_bytes,
                               wk, wv, p.RP, kh, vh, p.rows_per_seq);
        if ((st = lit_hip_check("literal decode: lift"))) return st;
        const int alds = (kLitTile * (li.d_head + 4) + li.q_per_kv * (li.d_head + kLitTile) + 3 * li.q_per_kv) * 4;
        if (!reserve_lds((const void*)literal_attn_kernel, alds))
            return fail(SPECTRA_EHIP, "literal decode: cannot reserve %d bytes of LDS", alds);
        hipLaunchKernelGGL(literal_attn_kernel, dim3(p.n_splits, li.n_kv, batch), dim3(256), alds, s, li, ctx, qf,
                           softmax_scale * 1.4426950408889634f, kh, vh, p.rows_per_seq, p.split_tokens, p.n_splits,
                           pm, pl, po);
        if ((st = lit_hip_check("literal decode: attend"))) return st;
    }
    hipLaunchKernelGGL(literal_merge_kernel, dim3(li.n_q, batch), dim3(256), 0, s, li, ctx, pm, pl, po,
                       p.split_tokens, p.n_splits, out);
    return lit_hip_check("literal decode: merge");
}

}  // extern "C"
