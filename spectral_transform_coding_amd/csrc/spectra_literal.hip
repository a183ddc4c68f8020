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

// W_up of one tensor, transposed per segment into fp16 terms: wt[0][s][n][k] = fp16(W[row0_s + k, n]),
// wt[1][...] = fp16(W - fp16(W)) (zero for bf16 weights), zero for k at or past the segment's
// rank (grid-stride over n_seg x seg_cols x RP).
template <typename DT>
__global__ __launch_bounds__(256) void literal_wt_kernel(LayoutInfo li, int kind, const DT* __restrict__ w, int RP,
                                                          _Float16* __restrict__ wt) {
    const TensorInfo& T = li.t[kind];
    const int64_t total = (int64_t)li.n_seg * li.seg_cols * RP;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
        const int k = (int)(idx % RP);
        const int n = (int)((idx / RP) % li.seg_cols);
        const int s = (int)(idx / ((int64_t)RP * li.seg_cols));
        const int rs = li.g * (T.seg_chunk0[s + 1] - T.seg_chunk0[s]);
        const float v = k < rs ? load_f32(w, (int64_t)(li.g * T.seg_chunk0[s] + k) * li.seg_cols + n) : 0.0f;
        const _Float16 hi = (_Float16)v;
        wt[idx] = hi;
        wt[total + idx] = (_Float16)(v - (float)hi);
    }
}

// Lift (grid: half cache blocks, sequence, tensor; 256 threads).  For each segment the 64
// tokens' dequantised latents C^_s are staged in LDS as fp16 hi = fp16(c), and for keys also
// lo = fp16(c - hi) (scores amplify key errors through the softmax; value errors enter
// linearly); wave w then computes column tiles 2p, 2p + 1 (32 columns each) for
// p = w, w + 4, ... over the 64 tokens with 32x32x16 f16 products: A = latent terms from LDS,
// B = 16-byte pieces of the transposed W_up terms read from memory (L2-resident), the W lo term
// only for float32 weights.  Output rows = the tokens' rows of out
// [batch][rows_per_seq][n_kv d_head], float32.
template <bool LO>
__global__ __launch_bounds__(256) void literal_lift_kernel(LayoutInfo li, Positions ctx, const uint8_t* __restrict__ cache_k,
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
        for (int idx = tid; idx < 64 * rp; idx += 256) {
            const int r = idx / rp, i = idx % rp;
            float v = 0.0f;
            if (i < rs) {
                const int c = c0 + i / li.g;
                v = dequant_at(T, kind, li.g, bp, c, coff[c], 64 * half + r, i % li.g);
            }
            const _Float16 hi = (_Float16)v;
            cl[r * KP + i] = hi;
            cll[r * KP + i] = (_Float16)(v - (float)hi);
        }
        __syncthreads();
        const _Float16* ws = wt + (int64_t)s * li.seg_cols * RP;
        for (int p = wv; 64 * p < li.seg_cols; p += 4) {
            const int nb = 64 * p, ntl = std::min(2, (li.seg_cols - nb) / 32);
            f32x16_t acc[2][2];
#pragma unroll
            for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = f32x16_t{};
            for (int k0 = 0; k0 < rp; k0 += 16) {
                half8_t bh[2], bl[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int n = nb + 32 * std::min(j, ntl - 1) + m;   // a valid column
                    const _Float16* src = ws + (int64_t)n * RP + k0 + 8 * kh2;
                    bh[j] = *reinterpret_cast<const half8_t*>(src);
                    if constexpr (LO) bl[j] = *reinterpret_cast<const half8_t*>(src + wt_terms);
                }
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int ao = (32 * i + m) * KP + k0 + 8 * kh2;
                    const half8_t a = *reinterpret_cast<const half8_t*>(cl + ao);
                    const half8_t al = *reinterpret_cast<const half8_t*>(cll + ao);
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        if (j < ntl) {
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bh[j], acc[i][j], 0, 0, 0);
                            if (alo) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, bh[j], acc[i][j], 0, 0, 0);
                            if constexpr (LO)
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bl[j], acc[i][j], 0, 0, 0);
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

// Attend (grid: splits, key/value head, sequence; one wave).  Lane t takes token t of each
// 64-token tile: its scores for the key/value head's query heads from the tile's keys staged in
// LDS; per head the wave keeps one running maximum and sum (base-2 online softmax, scores
// scaled by qscale = softmax_scale log2 e); lane l then accumulates dimensions l + 64 i of the
// output from the tile's values and probabilities.  Rows past the context are staged as zeros.
// Partials pm, pl [batch][splits][n_q], po [batch][splits][n_q][d_head].
__global__ __launch_bounds__(64) void literal_attn_kernel(LayoutInfo li, Positions ctx, const float* __restrict__ q,
                                                          float qscale, const float* __restrict__ kh,
                                                          const float* __restrict__ vh, int64_t rows_per_seq,
                                                          int split_tokens, int n_splits, float* __restrict__ pm,
                                                          float* __restrict__ pl, float* __restrict__ po) {
    const int split = blockIdx.x, kv = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
    const int dh = li.d_head, nq = li.q_per_kv, ncols = li.n_kv * dh, h0 = kv * nq;
    const int64_t t0 = (int64_t)split * split_tokens;
    const int64_t t1 = std::min<int64_t>(ctx.v[b], t0 + split_tokens);
    if (t0 >= t1) return;
    __shared__ float qs[kLitQ][kLitDh];
    __shared__ float xt[kLitTile][kLitDh + 1];
    __shared__ float ps[kLitQ][kLitTile];
    for (int i = lane; i < nq * dh; i += 64) qs[i / dh][i % dh] = q[((int64_t)b * li.n_q + h0 + i / dh) * dh + i % dh] * qscale;
    float mh[kLitQ], lh[kLitQ], al[kLitQ], o[kLitQ][kLitDh / 64];
#pragma unroll
    for (int h = 0; h < kLitQ; ++h) {
        mh[h] = -INFINITY;
        lh[h] = 0.0f;
#pragma unroll
        for (int i = 0; i < kLitDh / 64; ++i) o[h][i] = 0.0f;
    }
    const float* kb = kh + (int64_t)b * rows_per_seq * ncols + kv * dh;
    const float* vb = vh + (int64_t)b * rows_per_seq * ncols + kv * dh;
    for (int64_t tile = t0; tile < t1; tile += kLitTile) {
        __syncthreads();                              // previous tile's values consumed
        for (int r = 0; r < kLitTile; ++r)
            for (int d = lane; d < dh; d += 64) xt[r][d] = tile + r < t1 ? kb[(tile + r) * ncols + d] : 0.0f;
        __syncthreads();
        const bool ok = tile + lane < t1;
        float sc[kLitQ];
#pragma unroll
        for (int h = 0; h < kLitQ; ++h) sc[h] = 0.0f;
        for (int d = 0; d < dh; ++d) {
            const float k = xt[lane][d];
#pragma unroll
            for (int h = 0; h < kLitQ; ++h)
                if (h < nq) sc[h] += qs[h][d] * k;
        }
#pragma unroll
        for (int h = 0; h < kLitQ; ++h) {
            if (h >= nq) break;
            const float s = ok ? sc[h] : -INFINITY;
            float mt = s;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) mt = fmaxf(mt, __shfl_xor(mt, off));
            const float mn = fmaxf(mh[h], mt);        // finite: the tile holds a valid token
            al[h] = __builtin_amdgcn_exp2f(mh[h] - mn);   // 0 while mh = -inf
            const float p = ok ? __builtin_amdgcn_exp2f(s - mn) : 0.0f;
            float ls = p;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) ls += __shfl_xor(ls, off);
            lh[h] = lh[h] * al[h] + ls;
            mh[h] = mn;
            ps[h][lane] = p;
        }
        __syncthreads();                              // keys consumed, probabilities visible
        for (int r = 0; r < kLitTile; ++r)
            for (int d = lane; d < dh; d += 64) xt[r][d] = tile + r < t1 ? vb[(tile + r) * ncols + d] : 0.0f;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kLitDh / 64; ++i) {
            const int d = lane + 64 * i;
            if (d >= dh) break;
#pragma unroll
            for (int h = 0; h < kLitQ; ++h) {
                if (h >= nq) break;
                float acc = o[h][i] * al[h];
                for (int r = 0; r < kLitTile; ++r) acc += ps[h][r] * xt[r][d];
                o[h][i] = acc;
            }
        }
    }
    const int64_t base = ((int64_t)b * n_splits + split) * li.n_q + h0;
    for (int h = 0; h < nq; ++h) {
        if (lane == 0) {
            pm[base + h] = mh[h];
            pl[base + h] = lh[h];
        }
#pragma unroll
        for (int i = 0; i < kLitDh / 64; ++i) {
            const int d = lane + 64 * i;
            if (d < dh) po[(base + h) * dh + d] = o[h][i];
        }
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

static LitPlan lit_plan(const LayoutInfo& li, int B, int64_t max_ctx) {
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
    const size_t ncols = (size_t)li.n_kv * li.d_head;
    const size_t wterms = (size_t)li.n_seg * li.seg_cols * p.RP * 2;
    size_t o = 0;
    p.off_kh = o; o += a256((size_t)B * p.rows_per_seq * ncols * 4);
    p.off_vh = o; o += a256((size_t)B * p.rows_per_seq * ncols * 4);
    p.off_wk = o; o += a256(wterms * 2);
    p.off_wv = o; o += a256(wterms * 2);
    p.off_q = o;  o += a256((size_t)B * li.n_q * li.d_head * 4);
    p.off_pm = o; o += a256((size_t)B * p.n_splits * li.n_q * 4);
    p.off_pl = o; o += a256((size_t)B * p.n_splits * li.n_q * 4);
    p.off_po = o; o += a256((size_t)B * p.n_splits * li.n_q * li.d_head * 4);
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
    if (li.d_head > kLitDh) return fail(SPECTRA_ENOTSUP, "literal decode: d_head > %d", kLitDh);
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
    *bytes = lit_plan(li, batch, max_ctx).total;
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
        const int lds = 2 * 64 * (p.RP + 8) * 2 + kMaxC * 4;
        static int reserved[2] = {0, 0};
        const void* fn = bf ? (const void*)literal_lift_kernel<false> : (const void*)literal_lift_kernel<true>;
        if (reserved[bf] < lds) {
            if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
                return fail(SPECTRA_EHIP, "literal decode: cannot reserve %d bytes of LDS", lds);
            reserved[bf] = lds;
        }
        const dim3 g((unsigned)(2 * ((max_ctx + kBT - 1) / kBT)), batch, 2);
        if (bf)
            hipLaunchKernelGGL(literal_lift_kernel<false>, g, dim3(256), lds, s, li, ctx, (const uint8_t*)cache_k,
                               (const uint8_t*)cache_v, nblk_cap * li.t[0].block_bytes, nblk_cap * li.t[1].block_bytes,
                               wk, wv, p.RP, kh, vh, p.rows_per_seq);
        else
            hipLaunchKernelGGL(literal_lift_kernel<true>, g, dim3(256), lds, s, li, ctx, (const uint8_t*)cache_k,
                               (const uint8_t*)cache_v, nblk_cap * li.t[0].block_bytes, nblk_cap * li.t[1].block_bytes,
                               wk, wv, p.RP, kh, vh, p.rows_per_seq);
        if ((st = lit_hip_check("literal decode: lift"))) return st;
        hipLaunchKernelGGL(literal_attn_kernel, dim3(p.n_splits, li.n_kv, batch), dim3(64), 0, s, li, ctx, qf,
                           softmax_scale * 1.4426950408889634f, kh, vh, p.rows_per_seq, p.split_tokens, p.n_splits,
                           pm, pl, po);
        if ((st = lit_hip_check("literal decode: attend"))) return st;
    }
    hipLaunchKernelGGL(literal_merge_kernel, dim3(li.n_q, batch), dim3(256), 0, s, li, ctx, pm, pl, po,
                       p.split_tokens, p.n_splits, out);
    return lit_hip_check("literal decode: merge");
}

}  // extern "C"
