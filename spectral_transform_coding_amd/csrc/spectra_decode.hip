// Decode attention over the packed latent cache (gfx950).
//
// "SPECTRA" technical summary, SPECTRA pipeline stage 3: keys and values are rebuilt from the
// latent cache for standard attention.  Here the rebuild is folded into the query and the
// output (latent-space attention, "Significance" section):
//   scores  S[t,h] = c^K_t . q~_h,   q~_h = scale * log2(e) * W_upK[:, kv(h)] q_h
//   values  z_h    = sum_t p[t,h] c^V_t,   o_h = (z_h / l_h) W_upV[:, kv(h)]
// which equals softmax(scale K^ q) V^ with K^ = C^K W_upK, V^ = C^V W_upV.
//
// Kernels: absorb (q~ and its fp16 hi/lo matrix-core operands), decode_mfma (stream
// the cache, unpack, dequantise, scores and value accumulation on the matrix cores, split-K
// online softmax), decode_generic (same on the vector ALUs for layouts the fast kernel does
// not cover), merge_lift (merge splits, lift by W_upV), output projection (optional W_O').
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <hip/hiprtc.h>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <map>
#include <atomic>
#include <mutex>
#include <string>
#include <tuple>
#include <type_traits>
#include <vector>

#include "spectra_device.h"
#include "spectra_decode_mfma.h"

namespace spectra {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kFastMaxChunks = 32;     // non-empty groups per tensor (8 per wave and role)
constexpr int kMaxLds = 160 * 1024;                    // LDS per workgroup on gfx950
// Width sets the matrix-core kernel is compiled for (bit b = width b).  Water-filled widths of
// one layer span a few adjacent values; fewer compiled widths mean less code per block.
constexpr int kMaskHigh = 0x1E0;   // 5..8
constexpr int kMaskMid = 0x078;    // 3..6
constexpr int kMaskLow = 0x03E;    // 1..5
constexpr int kMaskAll = 0x1FE;    // 1..8
constexpr int kGenTile = 128;          // tokens per tile of the generic kernel
constexpr int kMaxSplits = 1024;       // splits per sequence (bounded by the planner's target)
constexpr int kGenMaxH = 16, kGenMaxR = 64, kGenMaxHR = 256;

// ----------------------------------------------------------------------------- planning

struct DecodePlan {
    bool fast;
    int n_hg;                          // matrix-core kernel: groups of up to 32 query heads
    int small;                         // small-rank kernel instance (small_id), 0 when not used
    bool fused;                        // small-rank decode in one launch (decode_small_fused_kernel)
    int64_t small_cost;                // the split-per-wave plan's rounds x (blocks per split + 1)
    int split_tokens, n_splits;
    int RK, RV;                        // widest segment latent (K, V)
    size_t off_qt, off_pm, off_pl, off_pz, off_ob, total;
};

static int seg_r(const LayoutInfo& li, int t, int s) {
    return li.g * (li.t[t].seg_chunk0[s + 1] - li.t[t].seg_chunk0[s]);
}

// The matrix-core kernel takes query heads in groups of 32 (one grid row per group: the cache
// is streamed once per group).
constexpr int kFastHeads = 32, kFastMaxHeads = 256;
static bool fast_ok(const LayoutInfo& li) {
    return li.g == 16 && li.n_seg == 1 && li.n_q <= kFastMaxHeads && li.t[0].n_chunks >= 1 &&
           li.t[1].n_chunks >= 1 && li.t[0].n_chunks <= kFastMaxChunks && li.t[1].n_chunks <= kFastMaxChunks;
}

static bool generic_ok(const LayoutInfo& li) {
    const int hs = li.n_q / li.n_seg;
    if (hs > kGenMaxH) return false;
    for (int s = 0; s < li.n_seg; ++s)
        if (seg_r(li, 0, s) > kGenMaxR || seg_r(li, 1, s) > kGenMaxR || hs * seg_r(li, 1, s) > kGenMaxHR)
            return false;
    return true;
}

// Small-rank kernel instances (query heads per segment <= H, rank per segment <= R, group size G;
// the bounds size the per-lane registers).  small_kind picks the cheapest instance that holds the
// layout (token-major code chunks, g != 16, a token's codes of a chunk within 32 bits and two
// consecutive tokens' within the 64 bits from their first word), or 0.
#define SPECTRA_SMALL_INSTANCES(X) X(8, 8, 2) X(5, 6, 2) X(8, 8, 4) X(2, 16, 4) X(8, 8, 8) X(2, 16, 8)
constexpr int small_id(int H, int R, int G) { return (H << 16) | (R << 8) | G; }
static int small_kind(const LayoutInfo& li) {
    if (li.g == 16) return 0;
    const int hs = li.n_q / li.n_seg;
    int r = 0, wmax = 0;
    for (int s = 0; s < li.n_seg; ++s) r = std::max(r, std::max(seg_r(li, 0, s), seg_r(li, 1, s)));
    for (int t = 0; t < 2; ++t)
        for (int c = 0; c < li.t[t].n_chunks; ++c) {
            const int gb = li.g * li.t[t].width[c];
            wmax = std::max(wmax, (int)li.t[t].width[c]);
            // a lane's two slots' codes must end within the 64 bits from their first word
            for (int lane = 0; lane < 64; ++lane)
                if (((2 * lane * gb) & 31) + 2 * gb > 64) return 0;
        }
    if (li.g * wmax > 32 || r < 1) return 0;
    int best = 0, best_cost = 1 << 30;
#define SPECTRA_SMALL_PICK(H, R, G) \
    if (li.g == G && hs <= H && r <= R && H * R < best_cost) { best = small_id(H, R, G); best_cost = H * R; }
    SPECTRA_SMALL_INSTANCES(SPECTRA_SMALL_PICK)
#undef SPECTRA_SMALL_PICK
    return best;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace offsets for `splits` splits per sequence.
static void plan_offsets(DecodePlan& p, const LayoutInfo& li, int B, int splits) {
    size_t o = 0;
    p.off_qt = o;  o += align256((size_t)B * li.n_q * std::max(p.RK, 1) * 4);
    p.off_pm = o;  o += align256((size_t)B * splits * li.n_q * 4);
    p.off_pl = o;  o += align256((size_t)B * splits * li.n_q * 4);
    p.off_pz = o;  o += align256((size_t)B * splits * li.n_q * std::max(p.RV, 1) * 4);
    p.off_ob = o;  o += align256((size_t)B * li.n_q * li.d_head * 4);
    p.total = o;
}

// small_slots: waves of the chosen small-rank instance the device holds at once (0: unknown,
// as when only the workspace size is asked for).  With for_size the offsets and total are those
// of the largest split count any context up to max_ctx can take, so that a workspace sized for
// max_ctx serves every shorter context too (a shorter context can take more, shorter splits).
static DecodePlan make_plan(const LayoutInfo& li, int B, int64_t max_ctx, int64_t small_slots = 0,
                            bool for_size = false) {
    DecodePlan p{};
    p.fast = fast_ok(li);
    p.n_hg = p.fast ? (li.n_q + kFastHeads - 1) / kFastHeads : 1;
    p.small = p.fast ? 0 : small_kind(li);
    p.RK = p.RV = 0;
    for (int s = 0; s < li.n_seg; ++s) {
        p.RK = std::max(p.RK, seg_r(li, 0, s));
        p.RV = std::max(p.RV, seg_r(li, 1, s));
    }
    // Splits: about one workgroup per compute unit for the matrix-core kernel (each split
    // writes a float32 partial of n_q x r_act, so fewer, longer splits cost less traffic), four
    // per compute unit for the generic kernel (one per sequence, segment and split).  The small
    // kernel's one-wave workgroups: at most 16384 in all (the workspace is sized for that); when
    // the number of waves the device holds at once is known, the count that minimises rounds x
    // (blocks per split + 1), the 1 standing for a split's fixed work (query load, lane merge,
    // partial stores), so that the last round of waves is not left mostly empty.
    const int64_t blocks = std::max<int64_t>(1, (max_ctx + kBT - 1) / kBT);
    const int64_t units = p.fast ? (int64_t)B * p.n_hg : (int64_t)B * li.n_seg;
    const int64_t target = p.fast ? 256 : p.small ? 16384 : 1024;
    int64_t per_seq = std::max<int64_t>(1, (target + units - 1) / units);
    per_seq = std::min(per_seq, blocks);
    // every context up to max_ctx takes at most this many splits: ceil(n / ceil(n / k)) <= k
    // for its own block count n, and its k is per_seq capped at n <= blocks
    const int64_t split_bound = per_seq;
    if (p.small && small_slots > 0) {
        int64_t best = per_seq, best_cost = INT64_MAX;
        for (int64_t ns = 1; ns <= per_seq; ++ns) {
            const int64_t bps = (blocks + ns - 1) / ns, ns_eff = (blocks + bps - 1) / bps;
            const int64_t cost = ((units * ns_eff + small_slots - 1) / small_slots) * (bps + 1);
            if (cost < best_cost) {
                best_cost = cost;
                best = ns;
            }
        }
        per_seq = best;
        p.small_cost = best_cost;
    }
    const int64_t bps = (blocks + per_seq - 1) / per_seq;
    p.split_tokens = (int)(bps * kBT);
    p.n_splits = (int)((blocks + bps - 1) / bps);
    plan_offsets(p, li, B, for_size ? (int)split_bound : p.n_splits);
    return p;
}

// ----------------------------------------------------------------- generic decode kernel


// One workgroup = one (split, sequence, segment); one token per thread for the scores, one
// (head, coordinate) pair per thread for the value accumulation; float32 throughout.
__global__ __launch_bounds__(256) void decode_generic_kernel(
    LayoutInfo li, Positions ctx, const uint8_t* __restrict__ cache_k,
    const uint8_t* __restrict__ cache_v, int64_t seq_bytes_k, int64_t seq_bytes_v,
    const float* __restrict__ qt, int RK, float* __restrict__ pm, float* __restrict__ pl,
    float* __restrict__ pz, int RV, int split_tokens, int n_splits) {
    const int split = blockIdx.x;
    const int b = blockIdx.y / li.n_seg, seg = blockIdx.y % li.n_seg;
    const int tid = threadIdx.x;
    const int64_t t0 = (int64_t)split * split_tokens;
    const int64_t t1 = min((int64_t)ctx.v[b], t0 + split_tokens);
    if (t0 >= t1) return;
    const int Hs = li.kv_per_seg * li.q_per_kv;
    const int h0 = seg * Hs;
    const TensorInfo& TK = li.t[0];
    const TensorInfo& TV = li.t[1];
    const int ck0 = TK.seg_chunk0[seg], ck1 = TK.seg_chunk0[seg + 1];
    const int cv0 = TV.seg_chunk0[seg], cv1 = TV.seg_chunk0[seg + 1];
    const int rk = li.g * (ck1 - ck0), rv = li.g * (cv1 - cv0);

    __shared__ float qs[kGenMaxH][kGenMaxR];
    __shared__ float cvt[kGenTile][kGenMaxR + 1];
    __shared__ float sbuf[kGenMaxH][kGenTile];
    __shared__ float m_s[kGenMaxH], l_s[kGenMaxH], a_s[kGenMaxH];
    __shared__ int64_t koff[kGenMaxR], voff[kGenMaxR];

    for (int i = tid; i < Hs * rk; i += blockDim.x)
        qs[i / rk][i % rk] = qt[((int64_t)b * li.n_q + h0 + i / rk) * RK + i % rk];
    for (int c = tid; c < ck1 - ck0; c += blockDim.x) koff[c] = chunk_code_offset(TK, li.g, ck0 + c);
    for (int c = tid; c < cv1 - cv0; c += blockDim.x) voff[c] = chunk_code_offset(TV, li.g, cv0 + c);
    if (tid < Hs) { m_s[tid] = -INFINITY; l_s[tid] = 0.0f; }
    float z = 0.0f;
    const int zh = tid / max(rv, 1), zi = tid % max(rv, 1);
    const bool zown = rv > 0 && tid < Hs * rv;
    __syncthreads();

    const uint8_t* seqk = cache_k + (int64_t)b * seq_bytes_k;
    const uint8_t* seqv = cache_v + (int64_t)b * seq_bytes_v;
    for (int64_t start = t0; start < t1; start += kGenTile) {
        const int64_t blk = start / kBT;
        const uint8_t* bk = seqk + blk * TK.block_bytes;
        const uint8_t* bv = seqv + blk * TV.block_bytes;
        if (tid < kGenTile) {
            const int64_t tok = start + tid;
            const int tau = (int)(tok - blk * kBT);
            float sc[kGenMaxH];
#pragma unroll
            for (int h = 0; h < kGenMaxH; ++h) sc[h] = 0.0f;
            if (tok < t1) {
                for (int c = 0; c < ck1 - ck0; ++c)
                    for (int j = 0; j < li.g; ++j) {
                        const float x = dequant_at(TK, 0, li.g, bk, ck0 + c, koff[c], tau, j);
#pragma unroll
                        for (int h = 0; h < kGenMaxH; ++h)
                            if (h < Hs) sc[h] += x * qs[h][c * li.g + j];
                    }
                for (int c = 0; c < cv1 - cv0; ++c)
                    for (int j = 0; j < li.g; ++j)
                        cvt[tid][c * li.g + j] = dequant_at(TV, 1, li.g, bv, cv0 + c, voff[c], tau, j);
            } else {
                for (int i = 0; i < rv; ++i) cvt[tid][i] = 0.0f;
            }
#pragma unroll
            for (int h = 0; h < kGenMaxH; ++h)
                if (h < Hs) sbuf[h][tid] = tok < t1 ? sc[h] : -INFINITY;
        }
        __syncthreads();
        if (tid < Hs) {
            float mx = m_s[tid];
            for (int t = 0; t < kGenTile; ++t) mx = fmaxf(mx, sbuf[tid][t]);
            a_s[tid] = __builtin_amdgcn_exp2f(m_s[tid] - mx);
            m_s[tid] = mx;
        }
        __syncthreads();
        for (int i = tid; i < Hs * kGenTile; i += blockDim.x) {
            const int h = i / kGenTile, t = i % kGenTile;
            sbuf[h][t] = __builtin_amdgcn_exp2f(sbuf[h][t] - m_s[h]);
        }
        __syncthreads();
        if (tid < Hs) {
            float s = 0.0f;
            for (int t = 0; t < kGenTile; ++t) s += sbuf[tid][t];
            l_s[tid] = l_s[tid] * a_s[tid] + s;
        }
        if (zown) {
            float acc = z * a_s[zh];
            for (int t = 0; t < kGenTile; ++t) acc += sbuf[zh][t] * cvt[t][zi];
            z = acc;
        }
        __syncthreads();
    }
    const int64_t pbase = ((int64_t)b * n_splits + split) * li.n_q + h0;
    if (tid < Hs) {
        pm[pbase + tid] = m_s[tid];
        pl[pbase + tid] = l_s[tid];
    }
    if (zown) pz[(pbase + zh) * RV + zi] = z;
}

// Small-rank decode (per-head or narrow latents, token-major code chunks): one wave per (split,
// sequence, segment); lane l owns the consecutive slots 2 l and 2 l + 1 of every 128-token block
// and keeps, per query head of the segment, its own sum and latent value accumulator against a
// reference maximum shared by the wave (online softmax that rescales only when the reference
// moves), so no step waits for another lane until the wave merges the lanes at the end.  Same
// partials (m, l, z) as the generic kernel.
//   SPECTRA technical summary, pipeline stage 3 (attention over the dequantised cache, here in
// latent space); the per-head segments follow the spectral-kv forum thread, Technical principle 1.
// Raw words of the lane's two slots in the segment's chunks: for chunk c, the two 32-bit words
// from the one holding the slots' first code bit (the host admits only widths whose 2 G codes
// then end within these 64 bits; the second word is read even when unused: it is still inside
// the block, in the next chunk or the scale chunks) and the two fp16 scales as one 32-bit word.
// Chunks past nc come with offset 0 and width 1 (in-bounds reads, unused).  All loads are issued
// before any is used.
template <int R, int G>
struct SmallRaw {
    uint32_t w0[R / G], w1[R / G];
    uint32_t s[R / G];
};
// Byte offsets in a block of this lane's code window and scale word, per chunk (loop-invariant).
template <int R, int G>
struct SmallOfs {
    int code[R / G], scale[R / G];
};
template <int R, int G>
__device__ __forceinline__ SmallOfs<R, G> small_offsets(const TensorInfo& T, int c0, int nc, const int (&ofs)[R / G],
                                                        const int (&wd)[R / G], int lane) {
    SmallOfs<R, G> o;
#pragma unroll
    for (int c = 0; c < R / G; ++c) {
        o.code[c] = ofs[c] + 4 * ((2 * lane * G * wd[c]) >> 5);
        o.scale[c] = T.codes_bytes + 256 * (c0 + (c < nc ? c : 0)) + 4 * lane;
    }
    return o;
}
// One block's words through a buffer resource on the (wave-uniform) block address, so a block
// costs no per-lane address arithmetic.
template <int R, int G>
__device__ __forceinline__ void small_load(const uint8_t* blk, int block_bytes, const SmallOfs<R, G>& o,
                                           SmallRaw<R, G>& raw) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blk), (short)0, block_bytes, kBufferWord3);
#pragma unroll
    for (int c = 0; c < R / G; ++c) {
        const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(r, o.code[c], 0, 2);
        raw.w0[c] = x[0];
        raw.w1[c] = x[1];
        raw.s[c] = __builtin_amdgcn_raw_buffer_load_b32(r, o.scale[c], 0, 2);
    }
}
// The dequantised latent of the lane's slot 2 lane + k (zeros past the segment's rank):
// s (u - (2^b - 1) / 2) as one fused multiply-add s u + (-s h), s h rounded to float32.
// G = 2: a funnel shift brings the lane's two-token code window (2 G b <= 32 bits, from bit
// (2 lane G b) mod 32 of the two words) into one 32-bit word, and each code is one bit-field
// extract.  Larger G: token k's G codes from a 64-bit shift of the two words.
template <int R, int G>
__device__ __forceinline__ void small_dequant(const SmallRaw<R, G>& raw, int nc, const int (&wd)[R / G], int lane,
                                              int k, float (&out)[R]) {
#pragma unroll
    for (int c = 0; c < R / G; ++c) {
        const int b = wd[c];
        const float s = c < nc ? f16_bits_to_f32((uint16_t)(raw.s[c] >> (16 * k))) : 0.0f;
        const float nsh = -s * (0.5f * (float)((1u << b) - 1u));
        if constexpr (G == 2) {
            const uint32_t x = __builtin_amdgcn_alignbit(raw.w1[c], raw.w0[c], (uint32_t)((2 * lane * G * b) & 31));
#pragma unroll
            for (int j = 0; j < G; ++j)
                out[c * G + j] =
                    __builtin_fmaf((float)__builtin_amdgcn_ubfe(x, (uint32_t)((k * G + j) * b), (uint32_t)b), s, nsh);
        } else {
            const int bit = ((2 * lane * G * b) & 31) + k * G * b;   // bit + G b <= 64
            const uint64_t xw = ((uint64_t)raw.w1[c] << 32) | raw.w0[c];
            const uint32_t x = (uint32_t)(xw >> bit);
            const uint32_t mask = (1u << b) - 1u;
#pragma unroll
            for (int j = 0; j < G; ++j) out[c * G + j] = __builtin_fmaf((float)((x >> (j * b)) & mask), s, nsh);
        }
    }
}

// One split of one (sequence, segment) by one wave: tokens [t0, t1) of the sequence (t0 < t1),
// scored against the wave's query latents q (zeros past the segment's heads and rank).  On return
// every lane holds the wave's merged partials: the reference maximum m (base 2), the sum l of
// 2^(s - m) and the accumulator z = sum 2^(s - m) c^V, per head.
template <int MAXH, int MAXR, int G>
__device__ __forceinline__ void small_split(const LayoutInfo& li, int seg, int Hs, int64_t t0, int64_t t1,
                                            const uint8_t* seqk, const uint8_t* seqv, const float (&q)[MAXH][MAXR],
                                            int lane, float (&m)[MAXH], float (&L)[MAXH], float (&zz)[MAXH][MAXR]) {
    const TensorInfo& TK = li.t[0];
    const TensorInfo& TV = li.t[1];
    constexpr int NC = MAXR / G;
    const int ck0 = TK.seg_chunk0[seg], nck = TK.seg_chunk0[seg + 1] - ck0;
    const int cv0 = TV.seg_chunk0[seg], ncv = TV.seg_chunk0[seg + 1] - cv0;
    int kofs[NC], kwd[NC], vofs[NC], vwd[NC];
    // the segment's chunks are consecutive: offsets from the first one's by the widths
    int ko_run = (int)chunk_code_offset(TK, G, ck0), vo_run = (int)chunk_code_offset(TV, G, cv0);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        kwd[c] = c < nck ? (int)TK.width[ck0 + c] : 1;
        vwd[c] = c < ncv ? (int)TV.width[cv0 + c] : 1;
        kofs[c] = c < nck ? ko_run : 0;
        vofs[c] = c < ncv ? vo_run : 0;
        ko_run += 16 * G * kwd[c];
        vo_run += 16 * G * vwd[c];
    }
    // Online softmax against one reference maximum per head shared by the wave (m): the first
    // block's wave maximum, raised only when a score passes it by more than 64 (weights stay
    // below 2^64, sums far from float32 overflow); then z and l are rescaled once.  No lane
    // rescales per block.  Weights of tokens 2^126 below the reference underflow to zero: their
    // share of the softmax is below float32 resolution anyway.
    float l[MAXH], z[MAXH][MAXR];
#pragma unroll
    for (int h = 0; h < MAXH; ++h) {
        m[h] = 0.0f;                                   // set from the first block's scores
        l[h] = 0.0f;
#pragma unroll
        for (int i = 0; i < MAXR; ++i) z[h][i] = 0.0f;
    }
    bool first = true;                                 // wave-uniform
    const SmallOfs<MAXR, G> ko = small_offsets<MAXR, G>(TK, ck0, nck, kofs, kwd, lane);
    const SmallOfs<MAXR, G> vo = small_offsets<MAXR, G>(TV, cv0, ncv, vofs, vwd, lane);
    // a block's words are all requested before any is used; latency is hidden by the other
    // waves on the SIMD (a one-block-ahead register ring measured slower: it costs occupancy)
    for (int64_t blk = t0 / kBT; blk * kBT < t1; ++blk) {
        SmallRaw<MAXR, G> ck_raw, cv_raw;
        small_load<MAXR, G>(seqk + blk * TK.block_bytes, TK.block_bytes, ko, ck_raw);
        small_load<MAXR, G>(seqv + blk * TV.block_bytes, TV.block_bytes, vo, cv_raw);
        // tokens of this block outside [t0, t1) (the split's first and last block only)
        const bool edge = blk * kBT < t0 || (blk + 1) * kBT > t1;
        float sc[2][MAXH], cvv[2][MAXR];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float ckk[MAXR];
            small_dequant<MAXR, G>(ck_raw, nck, kwd, lane, u, ckk);
            small_dequant<MAXR, G>(cv_raw, ncv, vwd, lane, u, cvv[u]);
            // scores relative to the reference: s - m
#pragma unroll
            for (int h = 0; h < MAXH; ++h) {
                float acc = -m[h];
#pragma unroll
                for (int i = 0; i < MAXR; ++i) acc += ckk[i] * q[h][i];
                sc[u][h] = acc;
            }
        }
        if (edge) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int64_t tok = blk * kBT + 2 * lane + u;
                if (tok < t0 || tok >= t1)
#pragma unroll
                    for (int h = 0; h < MAXH; ++h) sc[u][h] = -INFINITY;
            }
        }
        // reference maxima: set on the split's first block, raised when a score passes one by 64
        bool raise = first;
        if (!raise) {
            float over = -INFINITY;
#pragma unroll
            for (int h = 0; h < MAXH; ++h)
                if (h < Hs) over = fmaxf(over, fmaxf(sc[0][h], sc[1][h]));
            raise = __builtin_amdgcn_ballot_w64(over > 64.0f) != 0;
        }
        if (raise) {
#pragma unroll
            for (int h = 0; h < MAXH; ++h) {
                if (h >= Hs) break;
                // the block's scores themselves, then the new reference (masked tokens: -inf)
                const float s0 = sc[0][h] + m[h], s1 = sc[1][h] + m[h];
                float M = fmaxf(s0, s1);
                if (!first) M = fmaxf(M, m[h]);
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
                const float al = first ? 0.0f : __builtin_amdgcn_exp2f(m[h] - M);
                l[h] *= al;
#pragma unroll
                for (int i = 0; i < MAXR; ++i) z[h][i] *= al;
                sc[0][h] = s0 - M;
                sc[1][h] = s1 - M;
                m[h] = M;
            }
            first = false;
        }
#pragma unroll
        for (int h = 0; h < MAXH; ++h) {
            if (h >= Hs) break;
            const float pa = __builtin_amdgcn_exp2f(sc[0][h]), pb = __builtin_amdgcn_exp2f(sc[1][h]);
            l[h] += pa + pb;
#pragma unroll
            for (int i = 0; i < MAXR; ++i) z[h][i] = __builtin_fmaf(pb, cvv[1][i], __builtin_fmaf(pa, cvv[0][i], z[h][i]));
        }
    }
    // merge the lanes: every lane's sums share the wave's reference maximum m
#pragma unroll
    for (int h = 0; h < MAXH; ++h) {
        if (h >= Hs) break;
        float s = l[h];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
        L[h] = s;
#pragma unroll
        for (int i = 0; i < MAXR; ++i) {
            float x = z[h][i];
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
            zz[h][i] = x;
        }
    }
}

template <int MAXH, int MAXR, int G>
__global__ __launch_bounds__(64) void decode_small_kernel(
    LayoutInfo li, Positions ctx, const uint8_t* __restrict__ cache_k,
    const uint8_t* __restrict__ cache_v, int64_t seq_bytes_k, int64_t seq_bytes_v,
    const float* __restrict__ qt, int RK, float* __restrict__ pm, float* __restrict__ pl,
    float* __restrict__ pz, int RV, int split_tokens, int n_splits) {
    const int split = blockIdx.x;
    const int b = blockIdx.y / li.n_seg, seg = blockIdx.y % li.n_seg;
    const int lane = threadIdx.x;
    const int64_t t0 = (int64_t)split * split_tokens;
    const int64_t t1 = min((int64_t)ctx.v[b], t0 + split_tokens);
    if (t0 >= t1) return;
    const int Hs = li.kv_per_seg * li.q_per_kv, h0 = seg * Hs;
    const int rk = G * (li.t[0].seg_chunk0[seg + 1] - li.t[0].seg_chunk0[seg]);
    const int rv = G * (li.t[1].seg_chunk0[seg + 1] - li.t[1].seg_chunk0[seg]);
    float q[MAXH][MAXR];
#pragma unroll
    for (int h = 0; h < MAXH; ++h)
#pragma unroll
        for (int i = 0; i < MAXR; ++i)
            q[h][i] = (h < Hs && i < rk) ? qt[((int64_t)b * li.n_q + h0 + h) * RK + i] : 0.0f;
    float m[MAXH], L[MAXH], zz[MAXH][MAXR];
    small_split<MAXH, MAXR, G>(li, seg, Hs, t0, t1, cache_k + (int64_t)b * seq_bytes_k,
                               cache_v + (int64_t)b * seq_bytes_v, q, lane, m, L, zz);
    const int64_t pbase = ((int64_t)b * n_splits + split) * li.n_q + h0;
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < MAXH; ++h) {
            if (h >= Hs) break;
            pm[pbase + h] = m[h];
            pl[pbase + h] = L[h];
#pragma unroll
            for (int i = 0; i < MAXR; ++i)
                if (i < rv) pz[(pbase + h) * RV + i] = zz[h][i];
        }
    }
}

// The whole small-rank decode of one (sequence, segment) in one workgroup, when a sequence takes
// at most kSmallFusedWaves splits: wave w streams split w, and the workgroup also does the
// steps around the stream that otherwise take launches of their own.
//   1. query absorption (SPECTRA technical summary, pipeline stage 3: scores taken in latent
//      space): q~[h][i] = qscale sum_d q[b, h, d] W_upK[r0 + i, c0(h) + d], float32 sums of
//      the inputs' products, eight lanes per (head, coordinate) and a three-step lane sum;
//   2. the wave's split (small_split);
//   3. merge of the splits (online-softmax combination): M = max_w m_w, weights 2^(m_w - M)
//      (0 for empty splits), L = sum_w weight l_w, z = sum_w weight z_w / L (0 for an empty
//      context), in split order;
//   4. lift: out[b, h, d] = sum_i z[h][i] W_upV[r0 + i, c0(h) + d], float32.
constexpr int kSmallFusedWaves = 8;
template <typename DT, int MAXH, int MAXR, int G>
__global__ __launch_bounds__(64 * kSmallFusedWaves) void decode_small_fused_kernel(
    LayoutInfo li, Positions ctx, const DT* __restrict__ q, const DT* __restrict__ w_up_k,
    const DT* __restrict__ w_up_v, float qscale, const uint8_t* __restrict__ cache_k,
    const uint8_t* __restrict__ cache_v, int64_t seq_bytes_k, int64_t seq_bytes_v, int split_tokens,
    float* __restrict__ out) {
    const int b = blockIdx.x / li.n_seg, seg = blockIdx.x % li.n_seg;
    // the wave index is made wave-uniform (scalar), so the split's block loop stays scalar
    const int tid = threadIdx.x, lane = tid & 63, nt = blockDim.x, nw = nt >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int Hs = li.kv_per_seg * li.q_per_kv, h0 = seg * Hs, dh = li.d_head;
    const int rk = G * (li.t[0].seg_chunk0[seg + 1] - li.t[0].seg_chunk0[seg]);
    const int rv = G * (li.t[1].seg_chunk0[seg + 1] - li.t[1].seg_chunk0[seg]);
    const int r0k = G * li.t[0].seg_chunk0[seg], r0v = G * li.t[1].seg_chunk0[seg];
    __shared__ float qs[MAXH][MAXR];
    __shared__ float sm[kSmallFusedWaves][MAXH], sl[kSmallFusedWaves][MAXH];
    __shared__ float sz[kSmallFusedWaves][MAXH][MAXR];
    __shared__ float zf[MAXH][MAXR];

    // 1. absorption: lane j of a pair's eight takes d = j, j + 8, ... (eight lanes read 16
    //    consecutive bytes of a row), all of its loads requested before the first product (in
    //    batches of 16), so that the query and W_upK reads cost one memory round trip per batch
    const int npair = Hs * rk;
    for (int p0 = 0; p0 < npair; p0 += nt / 8) {
        const int p = p0 + tid / 8, j = tid & 7;
        float acc = 0.0f;
        if (p < npair) {
            const int h = p / rk, i = p % rk, head = h0 + h;
            const int c0 = ((head / li.q_per_kv) % li.kv_per_seg) * dh;
            const DT* qrow = q + ((int64_t)b * li.n_q + head) * dh;
            const DT* wrow = w_up_k + (int64_t)(r0k + i) * li.seg_cols + c0;
            const int nk = (dh - j + 7) / 8;                  // this lane's elements
            auto batch = [&](auto nb) __attribute__((always_inline)) {
                constexpr int NB = decltype(nb)::value;
                for (int k0 = 0; k0 < nk; k0 += NB) {
                    float qv[NB], wv[NB];
#pragma unroll
                    for (int e = 0; e < NB; ++e) {             // unconditional (clamped) loads
                        const int dd = j + 8 * min(k0 + e, nk - 1);
                        qv[e] = load_f32(qrow, dd);
                        wv[e] = load_f32(wrow, dd);
                    }
#pragma unroll
                    for (int e = 0; e < NB; ++e)
                        if (k0 + e < nk) acc += qv[e] * wv[e];
                }
            };
            if (nk <= 8) batch(std::integral_constant<int, 8>{});   // d_head up to 64: one batch of 8
            else batch(std::integral_constant<int, 16>{});
        }
        acc += __shfl_xor(acc, 1);
        acc += __shfl_xor(acc, 2);
        acc += __shfl_xor(acc, 4);
        if (p < npair && j == 0) qs[p / rk][p % rk] = acc * qscale;
    }
    __syncthreads();
    // every lane reads the same values: they go to scalar registers, as the split-per-wave
    // kernel's scalar loads of q~ do, leaving the vector registers to the stream
    float qr[MAXH][MAXR];
#pragma unroll
    for (int h = 0; h < MAXH; ++h)
#pragma unroll
        for (int i = 0; i < MAXR; ++i)
            qr[h][i] = (h < Hs && i < rk) ? __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(qs[h][i]))) : 0.0f;

    // 2. this wave's split
    const int64_t t0 = (int64_t)wave * split_tokens;
    const int64_t t1 = min((int64_t)ctx.v[b], t0 + split_tokens);
    if (t0 < t1) {
        float m[MAXH], L[MAXH], zz[MAXH][MAXR];
        small_split<MAXH, MAXR, G>(li, seg, Hs, t0, t1, cache_k + (int64_t)b * seq_bytes_k,
                                   cache_v + (int64_t)b * seq_bytes_v, qr, lane, m, L, zz);
        if (lane == 0) {
#pragma unroll
            for (int h = 0; h < MAXH; ++h) {
                if (h >= Hs) break;
                sm[wave][h] = m[h];
                sl[wave][h] = L[h];
#pragma unroll
                for (int i = 0; i < MAXR; ++i) sz[wave][h][i] = zz[h][i];
            }
        }
    } else if (lane < Hs) {
        sm[wave][lane] = -INFINITY;                    // an empty split: weight 0
        sl[wave][lane] = 0.0f;
    }
    __syncthreads();

    // 3. merge of the splits, one thread per (head, coordinate)
    for (int p = tid; p < Hs * rv; p += nt) {
        const int h = p / rv, i = p % rv;
        float M = -INFINITY;
        for (int w = 0; w < nw; ++w) M = fmaxf(M, sm[w][h]);
        float Ls = 0.0f, acc = 0.0f;
        for (int w = 0; w < nw; ++w) {
            if (sm[w][h] == -INFINITY) continue;
            const float wt = __builtin_amdgcn_exp2f(sm[w][h] - M);
            Ls += wt * sl[w][h];
            acc += wt * sz[w][h][i];
        }
        zf[h][i] = Ls > 0.0f ? acc / Ls : 0.0f;
    }
    __syncthreads();

    // 4. lift, consecutive threads on consecutive output columns (the column's MAXR W_upV
    //    entries requested before the first product)
    for (int o = tid; o < Hs * dh; o += nt) {
        const int h = o / dh, d = o % dh, head = h0 + h;
        const int c0 = ((head / li.q_per_kv) % li.kv_per_seg) * dh;
        const DT* wcol = w_up_v + (int64_t)r0v * li.seg_cols + c0 + d;
        float wv[MAXR];
#pragma unroll
        for (int i = 0; i < MAXR; ++i)             // rows clamped to the segment's (none when rv is 0)
            wv[i] = rv > 0 ? load_f32(wcol, (int64_t)min(i, rv - 1) * li.seg_cols) : 0.0f;
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < MAXR; ++i)
            if (i < rv) acc += zf[h][i] * wv[i];
        out[((int64_t)b * li.n_q + head) * dh + d] = acc;
    }
}

// ---------------------------------------------------------------------- combine splits

// One workgroup per (key/value head, group of its query heads, sequence), heads in passes of up
// to 8:
//   merge the splits of each head:  M = max_s m_s,  w_s = 2^(m_s - M),  L = sum_s w_s l_s,
//   z[r] = sum_s w_s z_s[r] / L  (zero for an empty context);
//   lift:  o[d] = sum_r z[r] W_upV[r0 + r, c0 + d], with W_upV's slice staged through LDS in
//   row chunks of 64 KB (16-byte loads, all in flight together).
constexpr int kMergeHeads = 8;
constexpr int kLiftChunkBytes = 65536;
constexpr int kMergeLds = kMergeHeads * 512 * 4 + kMergeHeads * kMaxSplits * 4 + kLiftChunkBytes + 2 * kMergeHeads * 512 * 4 + 64;

template <typename DT>
__global__ __launch_bounds__(256) void merge_lift_kernel(LayoutInfo li, Positions ctx,
                                                         const float* __restrict__ pm,
                                                         const float* __restrict__ pl,
                                                         const float* __restrict__ pz, int RV,
                                                         int n_splits, int split_tokens,
                                                         const DT* __restrict__ w_up,
                                                         float* __restrict__ out, int heads_per_wg) {
    const int groups = (li.q_per_kv + heads_per_wg - 1) / heads_per_wg;
    const int kv = blockIdx.x / groups, hg = blockIdx.x % groups, b = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int seg = kv / li.kv_per_seg;
    const int r0 = li.g * li.t[1].seg_chunk0[seg];
    const int rv = li.g * (li.t[1].seg_chunk0[seg + 1] - li.t[1].seg_chunk0[seg]);
    const int c0 = (kv % li.kv_per_seg) * li.d_head;
    const int dh = li.d_head;
    const int ctxb = ctx.v[b];
    const int ns = ctxb <= 0 ? 0 : (ctxb + split_tokens - 1) / split_tokens;
    extern __shared__ __align__(16) unsigned char smem[];
    float* zs = reinterpret_cast<float*>(smem);                           // [8][512]
    float* wts = zs + kMergeHeads * 512;                                  // [8][kMaxSplits]
    unsigned char* wch = reinterpret_cast<unsigned char*>(wts + kMergeHeads * kMaxSplits);   // W rows
    float* red = reinterpret_cast<float*>(wch + kLiftChunkBytes);         // [2][8][512] partial sums
    float* invl = red + 2 * kMergeHeads * 512;                            // [8]... (16 floats)

    const int rows_per_chunk = kLiftChunkBytes / (dh * (int)sizeof(DT));
    const int parts = dh <= 128 ? 2 : 1;                                  // r range split over halves
    const int hend = min(li.q_per_kv, (hg + 1) * heads_per_wg);
    for (int h0 = hg * heads_per_wg; h0 < hend; h0 += kMergeHeads) {
        const int nh = min(kMergeHeads, hend - h0);
        __syncthreads();
        // ---- split weights: wave hh (and hh + 4) handles head hh
        for (int hh = wv; hh < nh; hh += 4) {
            const int h = kv * li.q_per_kv + h0 + hh;
            const int64_t base = (int64_t)b * n_splits * li.n_q + h;
            float mx = -INFINITY;
            for (int sp = lane; sp < ns; sp += 64) mx = fmaxf(mx, pm[base + (int64_t)sp * li.n_q]);
            for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
            float ls = 0.0f;
            for (int sp = lane; sp < ns; sp += 64) {
                const float wgt = mx == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(pm[base + (int64_t)sp * li.n_q] - mx);
                wts[hh * kMaxSplits + sp] = wgt;
                ls += wgt * pl[base + (int64_t)sp * li.n_q];
            }
            for (int o = 32; o > 0; o >>= 1) ls += __shfl_xor(ls, o);
            if (lane == 0) invl[hh] = ls > 0.0f ? 1.0f / ls : 0.0f;
        }
        __syncthreads();
        // ---- merged latent values z[hh][r]: thread tid owns 4-float groups g = tid + 256 k of the
        // [nh][rv] block (rv a multiple of 4); four splits per round, so that up to 16 16-byte
        // loads per thread are in flight together.  Other rv: one float per item.
        if (rv % 4) {
            const int64_t sbase = (int64_t)b * n_splits * li.n_q + kv * li.q_per_kv + h0;
            for (int it = tid; it < nh * rv; it += 256) {
                const int hh = it / rv, r = it % rv;
                float acc = 0.0f;
                for (int sp = 0; sp < ns; ++sp)
                    acc += wts[hh * kMaxSplits + sp] * pz[(sbase + (int64_t)sp * li.n_q + hh) * RV + r];
                zs[hh * 512 + r] = acc * invl[hh];
            }
        } else {
            const int ngroups = nh * rv / 4;
            f32x4_t zacc[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) zacc[k] = f32x4_t{0, 0, 0, 0};
            const int64_t sbase = (int64_t)b * n_splits * li.n_q + kv * li.q_per_kv + h0;
            int goff[4], ghh[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int gi = min(tid + 256 * k, max(ngroups - 1, 0));   // past the end: re-read the last
                ghh[k] = (4 * gi) / rv;
                goff[k] = ghh[k] * RV + (4 * gi) % rv;
            }
            const int nsr = rv > 0 ? ns : 0;
            for (int sp0 = 0; sp0 < nsr; sp0 += 4) {
                f32x4_t x[4][4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int sp = min(sp0 + u, nsr - 1);
                    const float* pzs = pz + (sbase + (int64_t)sp * li.n_q) * RV;
#pragma unroll
                    for (int k = 0; k < 4; ++k) x[u][k] = *reinterpret_cast<const f32x4_t*>(pzs + goff[k]);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (sp0 + u >= nsr) break;
#pragma unroll
                    for (int k = 0; k < 4; ++k) zacc[k] += wts[ghh[k] * kMaxSplits + sp0 + u] * x[u][k];
                }
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int gi = tid + 256 * k;
                if (gi < ngroups) {
                    const f32x4_t zz = zacc[k] * invl[ghh[k]];
                    *reinterpret_cast<f32x4_t*>(zs + ghh[k] * 512 + (4 * gi) % rv) = zz;
                }
            }
        }
        // ---- lift: thread (d, part) accumulates the part-th share of each chunk's rows
        float acc[2][kMergeHeads];
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int hh = 0; hh < kMergeHeads; ++hh) acc[k][hh] = 0.0f;
        for (int rc = 0; rc < rv; rc += rows_per_chunk) {
            const int nr = min(rows_per_chunk, rv - rc);
            const int row_bytes = dh * (int)sizeof(DT);
            const int n16 = nr * row_bytes / 16;
            __syncthreads();                           // previous chunk consumed; z visible
            // stage rows rc .. rc + nr of the slice: 16-byte pieces, up to 16 per thread in flight
            for (int p0 = 0; p0 < n16; p0 += 256 * 16) {
                u32x4_t v[16];
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const int pidx = min(p0 + tid + 256 * k, n16 - 1);   // tail lanes re-read a valid piece
                    const int r = pidx / (row_bytes / 16), off = pidx % (row_bytes / 16);
                    v[k] = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const unsigned char*>(w_up) +
                                                             ((int64_t)(r0 + rc + r) * li.seg_cols + c0) * sizeof(DT) + 16 * off);
                }
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const int pidx = p0 + tid + 256 * k;
                    if (pidx < n16) reinterpret_cast<u32x4_t*>(wch)[pidx] = v[k];
                }
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int item = tid + 256 * k;
                if (item >= dh * parts) continue;
                const int d = item % dh, part = item / dh;
                const int half = (nr + parts - 1) / parts;
                const int rb = part * half, re = min(nr, rb + half);
                int r = rb;
                for (; r + 4 <= re; r += 4) {
                    const float w0 = load_f32(reinterpret_cast<const DT*>(wch), (int64_t)r * dh + d);
                    const float w1 = load_f32(reinterpret_cast<const DT*>(wch), (int64_t)(r + 1) * dh + d);
                    const float w2 = load_f32(reinterpret_cast<const DT*>(wch), (int64_t)(r + 2) * dh + d);
                    const float w3 = load_f32(reinterpret_cast<const DT*>(wch), (int64_t)(r + 3) * dh + d);
#pragma unroll
                    for (int hh = 0; hh < kMergeHeads; ++hh)
                        if (hh < nh) {
                            const float* z = zs + hh * 512 + rc + r;
                            acc[k][hh] += z[0] * w0 + z[1] * w1 + z[2] * w2 + z[3] * w3;
                        }
                }
                for (; r < re; ++r) {
                    const float wv_ = load_f32(reinterpret_cast<const DT*>(wch), (int64_t)r * dh + d);
#pragma unroll
                    for (int hh = 0; hh < kMergeHeads; ++hh)
                        if (hh < nh) acc[k][hh] += zs[hh * 512 + rc + r] * wv_;
                }
            }
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int item = tid + 256 * k;
            if (item >= dh * parts) continue;
            const int d = item % dh, part = item / dh;
#pragma unroll
            for (int hh = 0; hh < kMergeHeads; ++hh)
                if (hh < nh) red[(part * kMergeHeads + hh) * 512 + d] = acc[k][hh];
        }
        __syncthreads();
        for (int it = tid; it < nh * dh; it += 256) {
            const int hh = it / dh, d = it % dh;
            float o = red[hh * 512 + d];
            if (parts == 2) o += red[(kMergeHeads + hh) * 512 + d];
            const int h = kv * li.q_per_kv + h0 + hh;
            out[((int64_t)b * li.n_q + h) * dh + d] = o;
        }
    }
}

// ------------------------------------------------------------ small tiled products

// The three small products of the path, as 32 x 32 output tiles with k staged through LDS in
// steps of 128 (grid: column tiles, row tiles, key/value head):
//   absorb   q~[b,h,i] = qscale * sum_d q[b,h,d] W_upK[r0 + i, c0 + d]   (rows (b, h of kv))
//   lift     o[b,h,d]  = sum_r z[b,h,r] W_upV[r0 + r, c0 + d]
//   out_proj y[b,n]    = sum_k o[b,k] W_O[k, n]
// with r0 the segment's first latent row and c0 the head's first column in the segment.
enum { kAbsorb = 0, kLift = 1, kOutProj = 2 };

template <int MODE, typename DT>
__global__ __launch_bounds__(256) void tile_gemm_kernel(LayoutInfo li, int B, const void* __restrict__ a_ptr,
                                                        const DT* __restrict__ w, float* __restrict__ out,
                                                        int ld, float alpha) {
    const int kv = blockIdx.z, tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    int R, Kd, N, r0 = 0, c0 = 0;
    if constexpr (MODE == kOutProj) {
        R = B;
        Kd = li.n_q * li.d_head;
        N = li.d_model;
    } else {
        const TensorInfo& T = li.t[MODE == kAbsorb ? 0 : 1];
        const int seg = kv / li.kv_per_seg;
        const int rs = li.g * (T.seg_chunk0[seg + 1] - T.seg_chunk0[seg]);
        r0 = li.g * T.seg_chunk0[seg];
        c0 = (kv % li.kv_per_seg) * li.d_head;
        R = B * li.q_per_kv;
        Kd = MODE == kAbsorb ? li.d_head : rs;
        N = MODE == kAbsorb ? rs : li.d_head;
    }
    const int n0 = blockIdx.x * 32, row0 = blockIdx.y * 32;
    if (n0 >= N || row0 >= R) return;
    // global row index of tile row i: (sequence, query head) for the per-head products
    auto row_of = [&](int rr) -> int64_t {
        if constexpr (MODE == kOutProj) return rr;
        else return (int64_t)(rr / li.q_per_kv) * li.n_q + kv * li.q_per_kv + rr % li.q_per_kv;
    };
    // k in stages of 128; the next stage's loads are in flight while the current one computes
    constexpr int KS = 128;
    __shared__ float As[KS][33];
    __shared__ float Ws[KS][33];
    // Loads are unconditional at clamped (in-range) addresses and masked afterwards, so that all
    // of a stage's loads are in flight together.
    using AT = typename std::conditional<MODE == kAbsorb, DT, float>::type;
    AT ra[16];
    DT rw[16];
    uint32_t va = 0, vw = 0;
    auto load_stage = [&](int k0) {
        va = vw = 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int idx = tid + 256 * e;
            {
                const int k = idx & (KS - 1), rr = idx / KS;
                const bool ok = row0 + rr < R && k0 + k < Kd;
                va |= (uint32_t)ok << e;
                const int64_t row = row_of(min(row0 + rr, R - 1));
                const int kc = min(k0 + k, Kd - 1);
                if constexpr (MODE == kAbsorb) ra[e] = reinterpret_cast<const DT*>(a_ptr)[row * li.d_head + kc];
                else ra[e] = reinterpret_cast<const float*>(a_ptr)[row * ld + kc];
            }
            if constexpr (MODE == kAbsorb) {
                // W element (k, n) = W_upK[r0 + n, c0 + k]: contiguous along k
                const int kk = idx & (KS - 1), nn = idx / KS;
                vw |= (uint32_t)(n0 + nn < N && k0 + kk < Kd) << e;
                rw[e] = w[(int64_t)(r0 + min(n0 + nn, N - 1)) * li.seg_cols + c0 + min(k0 + kk, Kd - 1)];
            } else {
                const int nn = idx & 31, kk = idx >> 5;
                vw |= (uint32_t)(n0 + nn < N && k0 + kk < Kd) << e;
                const int nc = min(n0 + nn, N - 1), kc = min(k0 + kk, Kd - 1);
                if constexpr (MODE == kLift) rw[e] = w[(int64_t)(r0 + kc) * li.seg_cols + c0 + nc];
                else rw[e] = w[(int64_t)kc * N + nc];
            }
        }
    };
    auto to_f32 = [](auto v) -> float {
        if constexpr (std::is_same<decltype(v), uint16_t>::value) return bf16_to_f32(v);
        else return v;
    };
    float acc[2][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}};
    load_stage(0);
    for (int k0 = 0; k0 < Kd; k0 += KS) {
        __syncthreads();                               // the previous stage is consumed
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int idx = tid + 256 * e;
            As[idx & (KS - 1)][idx / KS] = (va >> e) & 1 ? to_f32(ra[e]) : 0.0f;
            const float x = (vw >> e) & 1 ? to_f32(rw[e]) : 0.0f;
            if constexpr (MODE == kAbsorb) Ws[idx & (KS - 1)][idx / KS] = x;
            else Ws[idx >> 5][idx & 31] = x;
        }
        __syncthreads();
        if (k0 + KS < Kd) load_stage(k0 + KS);
        const int kn = min(KS, Kd - k0);
#pragma unroll 8
        for (int k = 0; k < kn; ++k) {
            const float a0 = As[k][ty], a1 = As[k][ty + 16];
            const float w0 = Ws[k][tx], w1 = Ws[k][tx + 16];
            acc[0][0] += a0 * w0;
            acc[0][1] += a0 * w1;
            acc[1][0] += a1 * w0;
            acc[1][1] += a1 * w1;
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int rr = row0 + ty + 16 * i;
        if (rr >= R) continue;
        const int64_t row = row_of(rr);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + tx + 16 * j;
            if (n >= N) continue;
            if constexpr (MODE == kAbsorb) out[row * ld + n] = acc[i][j] * alpha;
            else if constexpr (MODE == kLift) out[row * li.d_head + n] = acc[i][j];
            else out[row * N + n] = acc[i][j];
        }
    }
}

// ------------------------------------------------- query absorption and merge + lift (lean)

// Eight consecutive elements of a row as float32 (16-byte aligned; bf16 = one 16-byte load).
__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
    const uint4 x = *reinterpret_cast<const uint4*>(p);
    const uint32_t u[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(u[i] << 16);
        v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
    const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Query absorption for one key/value head (grid: column tiles, row tiles, key/value head):
//   q~[b,h,i] = qscale * sum_d q[b,h,d] W_upK[r0 + i, c0 + d]
// rows (b, j) = query head kv q_per_kv + j of sequence b, columns i < the segment's active rank.
// 64 x 32 output tiles; d in chunks of 128 whose loads (16-byte row pieces; d_head and the W_upK
// row stride multiples of 8 elements) are all issued before the chunk is staged through LDS as
// float32, so that one memory round trip feeds the whole chunk; 256 threads, 4 x 2 outputs each.
// q~ goes to qt (float32), row (b, h) of length ldq.
template <typename DT>
__global__ __launch_bounds__(256) void absorb_kernel(LayoutInfo li, int B, const DT* __restrict__ q,
                                                     const DT* __restrict__ w, float* __restrict__ qt, int ldq,
                                                     float alpha) {
    constexpr int KC = 128;
    const int kv = blockIdx.z, tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const TensorInfo& T = li.t[0];
    const int seg = kv / li.kv_per_seg;
    const int r0 = li.g * T.seg_chunk0[seg];
    const int rk = li.g * (T.seg_chunk0[seg + 1] - T.seg_chunk0[seg]);
    const int c0 = (kv % li.kv_per_seg) * li.d_head;
    const int dh = li.d_head, R = B * li.q_per_kv;
    const int n0 = blockIdx.x * 32, row0 = blockIdx.y * 64;
    if (n0 >= rk || row0 >= R) return;
    __shared__ float As[KC][65];   // [d][row]
    __shared__ float Ws[KC][33];   // [d][column]
    float acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i][0] = acc[i][1] = 0.0f;
    // pieces of a chunk: A 64 rows x 16 pieces of 8 (4 per thread), W 32 columns x 16 (2 per thread)
    int64_t aoff[4], woff[2];
    int arow[4], ak[4], wcol[2], wk[2];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int pc = tid + 256 * e;
        arow[e] = pc >> 4;
        ak[e] = (pc & 15) * 8;
        const int row = min(row0 + arow[e], R - 1);
        aoff[e] = ((int64_t)(row / li.q_per_kv) * li.n_q + kv * li.q_per_kv + row % li.q_per_kv) * dh;
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int pc = tid + 256 * e;
        wcol[e] = pc >> 4;
        wk[e] = (pc & 15) * 8;
        woff[e] = (int64_t)(r0 + min(n0 + wcol[e], rk - 1)) * li.seg_cols + c0;
    }
    for (int k0 = 0; k0 < dh; k0 += KC) {
        float av[4][8], wv[2][8];
#pragma unroll
        for (int e = 0; e < 4; ++e) load8(q + aoff[e] + min(k0 + ak[e], dh - 8), av[e]);   // tail: masked below
#pragma unroll
        for (int e = 0; e < 2; ++e) load8(w + woff[e] + min(k0 + wk[e], dh - 8), wv[e]);
        __syncthreads();                               // previous chunk consumed
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool ok = k0 + ak[e] < dh && row0 + arow[e] < R;
#pragma unroll
            for (int i = 0; i < 8; ++i) As[ak[e] + i][arow[e]] = ok ? av[e][i] : 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const bool ok = k0 + wk[e] < dh && n0 + wcol[e] < rk;
#pragma unroll
            for (int i = 0; i < 8; ++i) Ws[wk[e] + i][wcol[e]] = ok ? wv[e][i] : 0.0f;
        }
        __syncthreads();
        const int kn = min(KC, dh - k0);
#pragma unroll 8
        for (int k = 0; k < kn; ++k) {
            float a[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[k][ty + 16 * i];
            const float b0 = Ws[k][tx], b1 = Ws[k][tx + 16];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[i][0] += a[i] * b0;
                acc[i][1] += a[i] * b1;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rr = row0 + ty + 16 * i;
        if (rr >= R) continue;
        const int bq = rr / li.q_per_kv, head = kv * li.q_per_kv + rr % li.q_per_kv;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + tx + 16 * j;
            if (n >= rk) continue;
            qt[((int64_t)bq * li.n_q + head) * ldq + n] = acc[i][j] * alpha;
        }
    }
}

// Query absorption on the matrix cores (bf16 inputs, d_head a multiple of 16 up to 256): each wave
// computes a 32 x 32 tile of q~ (rows (b, j), columns i) with bf16 32x32x16 products accumulated
// in float32 (the products of bf16 values are exact); its operands are 16-byte pieces of q rows
// and W_upK rows read straight from memory, all issued before the first product.  Workgroup: 4
// waves = 64 x 64 outputs (grid: column tiles, row tiles, key/value head).  Writes q~ to qt
// (float32, row (b, h) of length ldq): a store instruction covers 32 consecutive columns of two
// rows.
constexpr int kAbsorbMaxD = 256;
__global__ __launch_bounds__(256) void absorb_mfma_kernel(LayoutInfo li, int B, const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ w, float alpha,
                                                          float* __restrict__ qt, int ldq) {
    const int kv = blockIdx.z, lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const TensorInfo& T = li.t[0];
    const int seg = kv / li.kv_per_seg;
    const int r0 = li.g * T.seg_chunk0[seg];
    const int rk = li.g * (T.seg_chunk0[seg + 1] - T.seg_chunk0[seg]);
    const int c0 = (kv % li.kv_per_seg) * li.d_head;
    const int dh = li.d_head, R = B * li.q_per_kv;
    const int row0 = blockIdx.y * 64 + 32 * (wv >> 1), n0 = blockIdx.x * 64 + 32 * (wv & 1);
    if (n0 >= rk || row0 >= R) return;
    const int m = lane & 31, kh = lane >> 5;
    const int row = min(row0 + m, R - 1), col = min(n0 + m, rk - 1);
    const uint16_t* qa = q + ((int64_t)(row / li.q_per_kv) * li.n_q + kv * li.q_per_kv + row % li.q_per_kv) * dh + 8 * kh;
    const uint16_t* wb = w + (int64_t)(r0 + col) * li.seg_cols + c0 + 8 * kh;
    constexpr int KS = kAbsorbMaxD / 16;
    bf16x8_t a[KS], b[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        if (16 * k < dh) {
            a[k] = *reinterpret_cast<const bf16x8_t*>(qa + 16 * k);
            b[k] = *reinterpret_cast<const bf16x8_t*>(wb + 16 * k);
        }
    }
    f32x16_t acc = {};
#pragma unroll
    for (int k = 0; k < KS; ++k)
        if (16 * k < dh) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[k], acc, 0, 0, 0);
    // acc[4 i + j] holds row 8 i + 4 kh + j of the tile, column m
    const int n = n0 + m;
    if (n >= rk) return;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const int rr = row0 + 8 * (t >> 2) + 4 * kh + (t & 3);
        if (rr >= R) continue;
        const int bq = rr / li.q_per_kv, head = kv * li.q_per_kv + rr % li.q_per_kv;
        qt[((int64_t)bq * li.n_q + head) * ldq + n] = acc[t] * alpha;
    }
}

// Merge the splits of up to NH query heads of one key/value head and lift them by W_upV (grid:
// key/value head x ceil(q_per_kv / hpw) parts, sequence; 512 threads; d_head a power of two in
// [32, 256]); part p takes query heads p hpw .. min(q_per_kv, (p + 1) hpw) - 1, hpw <= NH:
//   M = max_s m_s,  L = sum_s 2^(m_s - M) l_s,  z[r] = sum_s 2^(m_s - M) z_s[r] / L  (0 if empty),
//   o[d] = sum_r z[r] W_upV[r0 + r, c0 + d].
// Thread (column pair dp, row part rp) keeps its ROWS rows of the W_upV slice in registers: the
// loads are issued first and land while the split weights and z are formed.  z is formed in one
// memory round trip when it fits: the (head, 4 rows) units (single rows when rv or RV is not a
// multiple of 4) times the splits are dealt to the 512 threads as S slices of consecutive
// splits, each thread holding its slice's partials in registers; the S slice sums are added in
// slice order.  Rank <= 512, d_head even with d_head / 2 dividing 512, W rows 4- (bf16) or
// 8-byte (fp32) aligned at 2 d.
template <typename DT, int NH, int ROWS>
__global__ __launch_bounds__(512) void merge_lift2_kernel(LayoutInfo li, Positions ctx, const float* __restrict__ pm,
                                                          const float* __restrict__ pl, const float* __restrict__ pz,
                                                          int RV, int n_splits, int split_tokens, int hpw,
                                                          const DT* __restrict__ w_up, float* __restrict__ out) {
    const int parts = (li.q_per_kv + hpw - 1) / hpw;
    const int kv = blockIdx.x / parts, part = blockIdx.x % parts, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int seg = kv / li.kv_per_seg;
    const int r0 = li.g * li.t[1].seg_chunk0[seg];
    const int rv = li.g * (li.t[1].seg_chunk0[seg + 1] - li.t[1].seg_chunk0[seg]);
    const int c0 = (kv % li.kv_per_seg) * li.d_head;
    const int dh = li.d_head, dpairs = dh >> 1, rparts = 512 / dpairs;
    const int rows_per = 4 * ((rv + 4 * rparts - 1) / (4 * rparts));   // a multiple of 4
    const int dp = tid % dpairs, rp = tid / dpairs;
    const int ctxb = ctx.v[b];
    const int ns = ctxb <= 0 ? 0 : (ctxb + split_tokens - 1) / split_tokens;
    const int h0 = kv * li.q_per_kv + part * hpw;
    const int nh = min(hpw, li.q_per_kv - part * hpw);                 // heads of this workgroup
    __shared__ __align__(16) float zs[NH][512 + 128];  // rows past rv (up to rparts rows_per) are 0
    __shared__ float hmax[NH], hinv[NH];
    __shared__ float red[1024 * NH];                   // [rparts][NH][dh] partial sums (rparts dh = 1024)
    __shared__ f32x4_t zpart[512];                     // [S][units] slice sums of z

    // ---- this thread's W_upV rows (clamped in-range addresses; rows past rv are not used)
    constexpr int WW = sizeof(DT) == 2 ? 1 : 2;       // 32-bit words per column pair
    uint32_t wr[ROWS][WW];
#pragma unroll
    for (int j = 0; j < ROWS; ++j) {
        const int r = min(rp * rows_per + j, max(rv - 1, 0));
        const DT* src = w_up + (int64_t)(r0 + r) * li.seg_cols + c0 + 2 * dp;
        if constexpr (WW == 1) wr[j][0] = *reinterpret_cast<const uint32_t*>(src);
        else {
            const uint2 x = *reinterpret_cast<const uint2*>(src);
            wr[j][0] = x.x;
            wr[j][1] = x.y;
        }
    }
    // ---- one-round z: unit ui (head uh, rows ur .. ur + V - 1) for splits sl cps .. sl cps + cps - 1
    constexpr int kPre = 16;
    const bool vec = (rv & 3) == 0 && (RV & 3) == 0;
    const int V = vec ? 4 : 1;
    const int units = nh * rv / V;
    const int S = units > 0 ? max(1, min(ns, 512 / units)) : 1;
    const int cps = (ns + S - 1) / S;
    const bool pre = units > 0 && units <= 512 && ns <= 64 && cps <= kPre;
    const int ui = pre ? tid % units : 0, sl = pre ? tid / units : S;
    const int uh = (V * ui) / rv, ur = (V * ui) % rv;
    const int64_t ubase = (int64_t)b * n_splits * li.n_q + h0 + uh;
    f32x4_t xs[kPre];
    if (pre && sl < S) {
#pragma unroll
        for (int u = 0; u < kPre; ++u) {
            if (u < cps) {
                const int sp = min(sl * cps + u, ns - 1);
                const float* src = pz + (ubase + (int64_t)sp * li.n_q) * RV + ur;
                xs[u] = vec ? *reinterpret_cast<const f32x4_t*>(src) : f32x4_t{*src, 0.0f, 0.0f, 0.0f};
            }
        }
    }
    __shared__ float wts[NH][64];                      // split weights 2^(m_s - M) when ns <= 64
    // ---- per-head maximum and normaliser (wave hh)
    if (wv < nh) {
        const int64_t base = (int64_t)b * n_splits * li.n_q + h0 + wv;
        float mx = -__builtin_inff(), ls = 0.0f;
        if (ns <= 64) {                                // one split per lane, one load round
            const float m_ = lane < ns ? pm[base + (int64_t)lane * li.n_q] : -__builtin_inff();
            const float l_ = lane < ns ? pl[base + (int64_t)lane * li.n_q] : 0.0f;
            mx = m_;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
            const float wgt = lane < ns ? __builtin_amdgcn_exp2f(m_ - mx) : 0.0f;
            wts[wv][lane] = wgt;
            ls = wgt * l_;
        } else {
            for (int sp = lane; sp < ns; sp += 64) mx = fmaxf(mx, pm[base + (int64_t)sp * li.n_q]);
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
            for (int sp = lane; sp < ns; sp += 64)
                ls += __builtin_amdgcn_exp2f(pm[base + (int64_t)sp * li.n_q] - mx) * pl[base + (int64_t)sp * li.n_q];
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) ls += __shfl_xor(ls, o);
        if (lane == 0) {
            hmax[wv] = mx;
            hinv[wv] = ls > 0.0f ? 1.0f / ls : 0.0f;
        }
    }
    __syncthreads();
    // ---- merged z
    if (pre) {
        if (sl < S) {
            f32x4_t acc = {0, 0, 0, 0};
#pragma unroll
            for (int u = 0; u < kPre; ++u)
                if (u < cps && sl * cps + u < ns) acc += wts[uh][sl * cps + u] * xs[u];
            zpart[sl * units + ui] = acc;
        }
        __syncthreads();
        for (int i = tid; i < units; i += 512) {
            f32x4_t acc = zpart[i];
            for (int s2 = 1; s2 < S; ++s2) acc += zpart[s2 * units + i];
            const int hh = (V * i) / rv, r = (V * i) % rv;
            const float inv = hinv[hh];
            zs[hh][r] = acc[0] * inv;
            if (vec) {
                zs[hh][r + 1] = acc[1] * inv;
                zs[hh][r + 2] = acc[2] * inv;
                zs[hh][r + 3] = acc[3] * inv;
            }
        }
    } else if (vec) {
        for (int gi = tid; gi < nh * rv / 4; gi += 512) {
            const int hh = (4 * gi) / rv, r = (4 * gi) % rv;
            const int64_t base = (int64_t)b * n_splits * li.n_q + h0 + hh;
            const float M = hmax[hh];
            f32x4_t acc = {0, 0, 0, 0};
            for (int sp0 = 0; sp0 < ns; sp0 += 8) {
                f32x4_t x[8];
                float wgt[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int sp = min(sp0 + u, ns - 1);
                    x[u] = *reinterpret_cast<const f32x4_t*>(pz + (base + (int64_t)sp * li.n_q) * RV + r);
                    wgt[u] = sp0 + u < ns ? __builtin_amdgcn_exp2f(pm[base + (int64_t)sp * li.n_q] - M) : 0.0f;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) acc += wgt[u] * x[u];
            }
            const float inv = hinv[hh];
            zs[hh][r] = acc[0] * inv;
            zs[hh][r + 1] = acc[1] * inv;
            zs[hh][r + 2] = acc[2] * inv;
            zs[hh][r + 3] = acc[3] * inv;
        }
    } else {
        for (int it = tid; it < nh * rv; it += 512) {
            const int hh = it / rv, r = it % rv;
            const int64_t base = (int64_t)b * n_splits * li.n_q + h0 + hh;
            float acc = 0.0f;
            for (int sp = 0; sp < ns; ++sp)
                acc += __builtin_amdgcn_exp2f(pm[base + (int64_t)sp * li.n_q] - hmax[hh]) *
                       pz[(base + (int64_t)sp * li.n_q) * RV + r];
            zs[hh][r] = acc * hinv[hh];
        }
    }
    // rows [rv, rparts rows_per) of every head, and all rows of the NH - nh unused heads: zeros
    const int used = rparts * rows_per, tail = used - rv;
    for (int it = tid; it < nh * tail; it += 512) zs[it / tail][rv + it % tail] = 0.0f;
    for (int it = tid; it < (NH - nh) * used; it += 512) zs[nh + it / used][it % used] = 0.0f;
    __syncthreads();
    // ---- lift: this thread's rows, all heads, columns 2 dp and 2 dp + 1; z is read four rows at
    // a time (rows_per is a multiple of 4 here, and z rows past rv are 0, so no row is masked)
    float a[NH][2];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) a[hh][0] = a[hh][1] = 0.0f;
#pragma unroll
    for (int j0 = 0; j0 < ROWS; j0 += 4) {
        if (j0 < rows_per) {
            f32x4_t z4[NH];
#pragma unroll
            for (int hh = 0; hh < NH; ++hh) z4[hh] = *reinterpret_cast<const f32x4_t*>(&zs[hh][rp * rows_per + j0]);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float w0, w1;
                if constexpr (WW == 1) {
                    w0 = __uint_as_float(wr[j0 + u][0] << 16);
                    w1 = __uint_as_float(wr[j0 + u][0] & 0xFFFF0000u);
                } else {
                    w0 = __uint_as_float(wr[j0 + u][0]);
                    w1 = __uint_as_float(wr[j0 + u][1]);
                }
#pragma unroll
                for (int hh = 0; hh < NH; ++hh) {
                    a[hh][0] += z4[hh][u] * w0;
                    a[hh][1] += z4[hh][u] * w1;
                }
            }
        }
    }
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
        red[(rp * NH + hh) * dh + 2 * dp] = a[hh][0];
        red[(rp * NH + hh) * dh + 2 * dp + 1] = a[hh][1];
    }
    __syncthreads();
    for (int it = tid; it < nh * dh; it += 512) {
        const int hh = it / dh, d = it % dh;
        float o = 0.0f;
        for (int q = 0; q < rparts; ++q) o += red[(q * NH + hh) * dh + d];
        out[((int64_t)b * li.n_q + h0 + hh) * dh + d] = o;
    }
}

// ------------------------------------------------------------------- unpack test hook

__global__ __launch_bounds__(256) void unpack_kernel(LayoutInfo li, int kind, const uint8_t* __restrict__ cache,
                                                     int64_t seq_bytes, int64_t pos0, int64_t n_tok,
                                                     float* __restrict__ out) {
    const TensorInfo& ti = li.t[kind];
    const int b = blockIdx.y;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n_tok * ti.r_act) return;
    const int64_t i = idx / ti.r_act;
    const int col = (int)(idx % ti.r_act);
    const int c = col / li.g, j = col % li.g;
    const int64_t pos = pos0 + i;
    const uint8_t* blk = cache + (int64_t)b * seq_bytes + (pos / kBT) * ti.block_bytes;
    out[((int64_t)b * n_tok + i) * ti.r_act + col] =
        dequant_at(ti, kind, li.g, blk, c, chunk_code_offset(ti, li.g, c), (int)(pos % kBT), j);
}

}  // namespace spectra

using namespace spectra;

// The small-rank instance the planner picks for this layout (0: another kernel runs).
static int small_kind_if_used(const LayoutInfo& li) { return fast_ok(li) ? 0 : small_kind(li); }

// Waves of small-rank instance `kind` the current device holds at once (compute units x
// resident one-wave workgroups per unit), cached per device and instance; 0 when unknown.
static int64_t small_slots(int kind) {
    if (!kind) return 0;
    static std::mutex mu;
    static std::map<std::pair<int, int>, int64_t> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lk(mu);
    const auto key = std::make_pair(dev, kind);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    const void* fn = nullptr;
    switch (kind) {
#define SPECTRA_SMALL_FN(H, R, G) case small_id(H, R, G): fn = (const void*)decode_small_kernel<H, R, G>; break;
        SPECTRA_SMALL_INSTANCES(SPECTRA_SMALL_FN)
#undef SPECTRA_SMALL_FN
        default: break;
    }
    int per_cu = 0, cus = 0;
    int64_t slots = 0;
    if (fn && hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 64, 0) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
        slots = (int64_t)per_cu * cus;
    else
        (void)hipGetLastError();                       // the split count falls back; no error left behind
    cache[key] = slots;
    return slots;
}

// Workgroups of `waves` waves of the one-launch small-rank kernel (instance `kind`, bf16 or
// float32 inputs) the current device holds at once, cached; 0 when unknown.
static int64_t small_fused_slots(int kind, bool bf, int waves) {
    static std::mutex mu;
    static std::map<std::tuple<int, int, bool, int>, int64_t> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lk(mu);
    const auto key = std::make_tuple(dev, kind, bf, waves);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    const void* fn = nullptr;
    switch (kind) {
#define SPECTRA_SMALL_FUSED_FN(H, R, G)                                                             \
    case small_id(H, R, G):                                                                          \
        fn = bf ? (const void*)decode_small_fused_kernel<uint16_t, H, R, G>                          \
                : (const void*)decode_small_fused_kernel<float, H, R, G>;                            \
        break;
        SPECTRA_SMALL_INSTANCES(SPECTRA_SMALL_FUSED_FN)
#undef SPECTRA_SMALL_FUSED_FN
        default: break;
    }
    int per_cu = 0, cus = 0;
    int64_t slots = 0;
    if (fn && hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 64 * waves, 0) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
        slots = (int64_t)per_cu * cus;
    else
        (void)hipGetLastError();
    cache[key] = slots;
    return slots;
}

// Small-rank layouts: one launch (absorption, every split of a (sequence, segment) in one
// workgroup, merge and lift) when a sequence's splits fit one workgroup and the estimate is no
// worse than the split-per-wave plan plus its two extra launches.  Both estimates count rounds
// of resident work x (blocks per split + 1); kSmallLaunchBlocks prices the absorption and merge
// launches and their gaps in block steps of one wave (about 20 us against 2.7 us per block on the
// per-head workload).  SPECTRA_SMALL_FUSED=0 keeps the split-per-wave plan.
constexpr int64_t kSmallLaunchBlocks = 7;
static void plan_small_fused(DecodePlan& p, const LayoutInfo& li, int B, int64_t max_ctx, bool bf) {
    p.fused = false;
    if (!p.small || p.small_cost <= 0) return;
    const char* env = std::getenv("SPECTRA_SMALL_FUSED");
    if (env && env[0] == '0') return;
    const int64_t blocks = std::max<int64_t>(1, (max_ctx + kBT - 1) / kBT);
    const int64_t units = (int64_t)B * li.n_seg;
    int64_t best_cost = INT64_MAX, best_bps = 0, best_ns = 0;
    for (int64_t ns = 1; ns <= std::min<int64_t>(kSmallFusedWaves, blocks); ++ns) {
        const int64_t bps = (blocks + ns - 1) / ns, ns_eff = (blocks + bps - 1) / bps;
        const int64_t slots = small_fused_slots(p.small, bf, (int)ns_eff);
        if (slots <= 0) continue;
        const int64_t cost = ((units + slots - 1) / slots) * (bps + 1);
        if (cost < best_cost) {
            best_cost = cost;
            best_bps = bps;
            best_ns = ns_eff;
        }
    }
    if (best_ns == 0 || best_cost > p.small_cost + kSmallLaunchBlocks) return;
    p.fused = true;
    p.split_tokens = (int)(best_bps * kBT);
    p.n_splits = (int)best_ns;
}

bool spectra::reserve_lds(const void* kernel, int bytes) {
    static std::mutex mu;
    static std::map<std::pair<int, const void*>, int> done;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    std::lock_guard<std::mutex> lk(mu);
    int& have = done[std::make_pair(dev, kernel)];
    if (have >= bytes) return true;
    if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess) return false;
    have = bytes;
    return true;
}

static spectra_status hip_check(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SPECTRA_EHIP, "%s: %s", what, hipGetErrorString(e));
    return SPECTRA_OK;
}

// ------------------------------------------------ run-time specialised decode kernels
//
// The stream kernel's slot loops are compiled once per layout with that layout's group widths
// as constants (the width-generic kernel branches on the width of every slot of every block).
// The source is this library's own device code (spectra_decode_mfma.h and the headers it
// needs), embedded at build time; hiprtc compiles it for the device's architecture, and the
// kernel is cached per (device, K widths, V widths) for the life of the process.
namespace spectra {
#include "spectra_jit_source.inc"   // kJitSource: the device headers as one string

struct JitKernel {
    hipModule_t mod;
    hipFunction_t fn;      // nullptr: compilation or loading failed; the ahead-of-time kernel runs
};
static std::mutex g_jit_mu;
static std::map<std::string, JitKernel> g_jit;
static int g_jit_mode = -1;            // -1: not yet read from SPECTRA_JIT
static std::atomic<int> g_key_split_all{0};   // spectra_set_key_split: 1 = every key group split
static int g_jit_count = 0;

static bool jit_on() {
    std::lock_guard<std::mutex> lk(g_jit_mu);
    if (g_jit_mode < 0) {
        const char* e = std::getenv("SPECTRA_JIT");
        g_jit_mode = (e && e[0] == '0') ? 0 : 1;
    }
    return g_jit_mode == 1;
}

// Specialised kernel for this layout's widths on the current device (compiled on first use).
// *fn = nullptr when the kernel cannot be compiled or loaded: the caller then runs the width-
// generic kernel compiled into the library (same results, bit for bit), and the failure is
// remembered so that later calls do not try again.  The lock is not held while compiling: two
// threads may compile the same layout at once, and the second to finish drops its module.
// With may_compile false only a kernel already compiled for this layout is returned (nullptr
// otherwise): compiling and loading a module allocates device memory.
static spectra_status jit_decode_kernel(const LayoutInfo& li, hipFunction_t* fn, bool may_compile = true) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SPECTRA_EHIP, "decode: hipGetDevice failed");
    int wt[2][kRoleWaves][kSlots] = {};
    int mask = 0;
    std::string key = std::to_string(dev) + "|S" + std::to_string(li.k_split);
    for (int t = 0; t < 2; ++t) {
        key += t ? "|V" : "|K";
        for (int c = 0; c < li.t[t].n_chunks; ++c) {
            const int w = li.t[t].width[c];
            wt[t][c % kRoleWaves][c / kRoleWaves] = w;
            mask |= 1 << w;
            key += (char)('0' + w);
        }
    }
    {
        std::lock_guard<std::mutex> lk(g_jit_mu);
        auto it = g_jit.find(key);
        if (it != g_jit.end()) {
            *fn = it->second.fn;
            return SPECTRA_OK;
        }
    }
    if (!may_compile) {
        *fn = nullptr;
        return SPECTRA_OK;
    }
    // remembers the outcome (a failure as fn = nullptr) and returns the cached function
    auto settle = [&](JitKernel k) {
        std::lock_guard<std::mutex> lk(g_jit_mu);
        auto ins = g_jit.emplace(key, k);
        if (!ins.second) {
            if (k.fn) (void)hipModuleUnload(k.mod);   // another thread finished first
        } else if (k.fn) {
            ++g_jit_count;
        }
        *fn = ins.first->second.fn;
        return SPECTRA_OK;
    };
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(SPECTRA_EHIP, "decode: hipGetDeviceProperties failed");
    std::string arch = prop.gcnArchName;
    arch = arch.substr(0, arch.find(':'));           // processor only (feature-generic code)
    std::string src = kJitSource;
    src += "\nstruct JitWidths {\n    static constexpr bool kStatic = true;\n    static constexpr bool kExactLoads = false;\n"
           "    static constexpr int kSplitGroups = " + std::to_string(li.k_split) + ";\n"
           "    static constexpr signed char kW[2][4][8] = {";
    for (int t = 0; t < 2; ++t) {
        src += t ? ", {" : "{";
        for (int w = 0; w < kRoleWaves; ++w) {
            src += w ? ", {" : "{";
            for (int i = 0; i < kSlots; ++i) src += (i ? ", " : "") + std::to_string(wt[t][w][i]);
            src += "}";
        }
        src += "}";
    }
    src += "};\n    static constexpr int width(int r, int w, int i) { return kW[r][w][i]; }\n};\n"
           "extern \"C\" __global__ __launch_bounds__(512, 1) void spectra_decode_jit(\n"
           "    spectra::LayoutInfo li, spectra::Positions ctx, const uint8_t* __restrict__ cache_k,\n"
           "    const uint8_t* __restrict__ cache_v, int64_t seq_bytes_k, int64_t seq_bytes_v,\n"
           "    const float* __restrict__ qt, float* __restrict__ pm, float* __restrict__ pl,\n"
           "    float* __restrict__ pz, int RV, int split_tokens, int n_splits) {\n"
           "    spectra::decode_mfma_body<" + std::to_string(mask) + ", JitWidths>(li, ctx, cache_k, cache_v, seq_bytes_k,\n"
           "        seq_bytes_v, qt, pm, pl, pz, RV, split_tokens, n_splits);\n}\n";
    hiprtcProgram prog;
    if (hiprtcCreateProgram(&prog, src.c_str(), "spectra_decode_jit.hip", 0, nullptr, nullptr) != HIPRTC_SUCCESS)
        return settle(JitKernel{nullptr, nullptr});
    const std::string arch_opt = "--offload-arch=" + arch;
    // block alignment of jump targets: the unrolled slot loops are sensitive to instruction
    // fetch alignment; packed fp32 instructions are kept out (plain float code only)
    const char* opts[] = {arch_opt.c_str(), "-O3", "-std=c++17", "-mllvm", "-align-all-nofallthru-blocks=6",
                          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"};
    const hiprtcResult cr = hiprtcCompileProgram(prog, (int)(sizeof opts / sizeof opts[0]), opts);
    if (cr != HIPRTC_SUCCESS) {
        hiprtcDestroyProgram(&prog);
        return settle(JitKernel{nullptr, nullptr});
    }
    size_t code_size = 0;
    hiprtcGetCodeSize(prog, &code_size);
    std::vector<char> code(code_size);
    hiprtcGetCode(prog, code.data());
    hiprtcDestroyProgram(&prog);
    JitKernel k{};
    if (hipModuleLoadData(&k.mod, code.data()) != hipSuccess) {
        (void)hipGetLastError();
        return settle(JitKernel{nullptr, nullptr});
    }
    if (hipModuleGetFunction(&k.fn, k.mod, "spectra_decode_jit") != hipSuccess) {
        (void)hipGetLastError();
        (void)hipModuleUnload(k.mod);
        return settle(JitKernel{nullptr, nullptr});
    }
    return settle(k);
}
// ------------------------------------------------ scratch of the no-allocation entry point
//
// spectra_decode_attn_noalloc takes its workspace from this array instead of the caller.  Each
// device that loads the library holds its own copy until the process ends.  Host code never
// uses the array's name as an address: its device address on the current device comes from
// hipGetSymbolAddress, looked up once per device and kept.
static __device__ __align__(256) unsigned char scratch[SPECTRA_NOALLOC_SCRATCH_BYTES];

static spectra_status scratch_pointer(void** out) {
    static std::mutex mu;
    static std::map<int, void*> ptrs;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SPECTRA_EHIP, "decode (no allocation): hipGetDevice failed");
    std::lock_guard<std::mutex> lk(mu);
    auto it = ptrs.find(dev);
    if (it == ptrs.end()) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(SPECTRA_EHIP, "decode (no allocation): scratch address on device %d: %s", dev,
                        hipGetErrorString(e));
        it = ptrs.emplace(dev, p).first;
    }
    *out = it->second;
    return SPECTRA_OK;
}

// The decode call behind both entry points.  noalloc: the workspace is the scratch array
// (workspace and workspace_bytes are ignored), and no specialised kernel is compiled (a cached
// one is used if this layout already has one).
static spectra_status decode_attn_impl(const spectra_layout* layout, spectra_dtype dtype, const void* q,
                                       const void* cache_k, const void* cache_v, int64_t cap_tokens,
                                       int32_t batch, const int32_t* ctx_len, const void* w_up_k,
                                       const void* w_up_v, float softmax_scale, const void* w_o,
                                       float* out, void* workspace, size_t workspace_bytes,
                                       void* stream, bool noalloc);

}  // namespace spectra

extern "C" {

spectra_status spectra_decode_workspace_bytes(const spectra_layout* layout, int32_t batch,
                                              int64_t max_ctx, size_t* bytes) {
    clear_error();
    LayoutInfo li;
    spectra_status st = make_layout(layout, &li);
    if (st) return st;
    if (!bytes) return fail(SPECTRA_EINVAL, "bytes is NULL");
    if (batch < 0 || max_ctx < 0) return fail(SPECTRA_EINVAL, "negative batch or context");
    *bytes = make_plan(li, std::max(batch, 1), max_ctx, 0, true).total;
    return SPECTRA_OK;
}

spectra_status spectra_decode_attn(const spectra_layout* layout, spectra_dtype dtype, const void* q,
                                   const void* cache_k, const void* cache_v, int64_t cap_tokens,
                                   int32_t batch, const int32_t* ctx_len, const void* w_up_k,
                                   const void* w_up_v, float softmax_scale, const void* w_o,
                                   float* out, void* workspace, size_t workspace_bytes,
                                   void* stream) {
    return decode_attn_impl(layout, dtype, q, cache_k, cache_v, cap_tokens, batch, ctx_len, w_up_k, w_up_v,
                            softmax_scale, w_o, out, workspace, workspace_bytes, stream, false);
}

spectra_status spectra_decode_attn_noalloc(const spectra_layout* layout, spectra_dtype dtype, const void* q,
                                           const void* cache_k, const void* cache_v, int64_t cap_tokens,
                                           int32_t batch, const int32_t* ctx_len, const void* w_up_k,
                                           const void* w_up_v, float softmax_scale, const void* w_o,
                                           float* out, void* stream) {
    return decode_attn_impl(layout, dtype, q, cache_k, cache_v, cap_tokens, batch, ctx_len, w_up_k, w_up_v,
                            softmax_scale, w_o, out, nullptr, SPECTRA_NOALLOC_SCRATCH_BYTES, stream, true);
}

}  // extern "C"

spectra_status spectra::decode_attn_impl(const spectra_layout* layout, spectra_dtype dtype, const void* q,
                                                const void* cache_k, const void* cache_v, int64_t cap_tokens,
                                                int32_t batch, const int32_t* ctx_len, const void* w_up_k,
                                                const void* w_up_v, float softmax_scale, const void* w_o,
                                                float* out, void* workspace, size_t workspace_bytes,
                                                void* stream, bool noalloc) {
    clear_error();
    LayoutInfo li;
    spectra_status st = make_layout(layout, &li);
    if (st) return st;
    li.k_split = g_key_split_all.load() ? li.t[0].n_chunks : split_query_groups(li.t[0].n_chunks);
    if (dtype != SPECTRA_F32 && dtype != SPECTRA_BF16) return fail(SPECTRA_ENOTSUP, "decode: unknown dtype %d", (int)dtype);
    if (batch <= 0) return fail(SPECTRA_EINVAL, "decode: batch must be positive");
    if (batch > kMaxB) return fail(SPECTRA_ENOTSUP, "decode: batch %d > %d", batch, kMaxB);
    if (!q || !cache_k || !cache_v || !ctx_len || !w_up_k || !w_up_v || !out || (!workspace && !noalloc))
        return fail(SPECTRA_EINVAL, "decode: NULL pointer argument");
    if (cap_tokens <= 0) return fail(SPECTRA_EINVAL, "decode: capacity must be positive");
    if (li.d_head > 512) return fail(SPECTRA_ENOTSUP, "decode: d_head > 512");
    Positions ctx;
    std::memset(&ctx, 0, sizeof ctx);
    int64_t max_ctx = 0;
    for (int b = 0; b < batch; ++b) {
        if (ctx_len[b] < 0 || ctx_len[b] > cap_tokens)
            return fail(SPECTRA_ECAPACITY, "decode: ctx_len[%d] = %d outside [0, %lld]", b, ctx_len[b], (long long)cap_tokens);
        ctx.v[b] = ctx_len[b];
        max_ctx = std::max<int64_t>(max_ctx, ctx_len[b]);
    }
    DecodePlan p = make_plan(li, batch, max_ctx, small_slots(small_kind_if_used(li)));
    plan_small_fused(p, li, batch, max_ctx, dtype == SPECTRA_BF16);
    if (!p.fast && !p.small && !generic_ok(li))
        return fail(SPECTRA_ENOTSUP, "decode: no kernel for this layout (group %d, segments %d, heads %d)", li.g, li.n_seg, li.n_q);
    if (p.RK > 512 || p.RV > 512) return fail(SPECTRA_ENOTSUP, "decode: segment latent wider than 512");
    if (p.n_splits > kMaxSplits) return fail(SPECTRA_ENOTSUP, "decode: %d splits > %d", p.n_splits, kMaxSplits);
    {
        const size_t es = dtype == SPECTRA_BF16 ? 2 : 4;
        if ((reinterpret_cast<uintptr_t>(w_up_v) & 15) || (li.seg_cols * es) % 16 || (li.d_head * es) % 16)
            return fail(SPECTRA_ENOTSUP, "decode: W_upV rows must start on 16-byte boundaries (d_head %d)", li.d_head);
    }
    if (noalloc && p.total > (size_t)SPECTRA_NOALLOC_SCRATCH_BYTES)
        return fail(SPECTRA_ECAPACITY, "decode (no allocation): this call needs %zu bytes of workspace, more than the "
                    "%zu-byte scratch the library holds per device; use spectra_decode_attn with a workspace",
                    p.total, (size_t)SPECTRA_NOALLOC_SCRATCH_BYTES);
    if (workspace_bytes < p.total)
        return fail(SPECTRA_ECAPACITY, "decode: workspace %zu bytes < %zu needed", workspace_bytes, p.total);
    if (noalloc && (st = scratch_pointer(&workspace))) return st;
    hipStream_t s = (hipStream_t)stream;
    unsigned char* ws = (unsigned char*)workspace;
    float* qt = (float*)(ws + p.off_qt);
    float* pm = (float*)(ws + p.off_pm);
    float* pl = (float*)(ws + p.off_pl);
    float* pz = (float*)(ws + p.off_pz);
    float* ob = (float*)(ws + p.off_ob);
    const int64_t nblk = (cap_tokens + kBT - 1) / kBT;
    const int64_t sbk = nblk * li.t[0].block_bytes, sbv = nblk * li.t[1].block_bytes;
    const float qscale = softmax_scale * kLog2e;
    const bool bf = dtype == SPECTRA_BF16;

    const int RKa = std::max(p.RK, 1), RVa = std::max(p.RV, 1);
    const dim3 g_abs((RKa + 31) / 32, (batch * li.q_per_kv + 31) / 32, li.n_kv);
    const size_t esz = bf ? 2 : 4;
    if (p.fused) {
        // the one-launch small-rank kernel absorbs the query itself
    } else if (bf && li.d_head % 16 == 0 && li.d_head <= kAbsorbMaxD && li.seg_cols % 8 == 0 &&
        reinterpret_cast<uintptr_t>(q) % 16 == 0 && reinterpret_cast<uintptr_t>(w_up_k) % 16 == 0) {
        const dim3 g_ab((RKa + 63) / 64, (batch * li.q_per_kv + 63) / 64, li.n_kv);
        hipLaunchKernelGGL(absorb_mfma_kernel, g_ab, dim3(256), 0, s, li, batch, (const uint16_t*)q,
                           (const uint16_t*)w_up_k, qscale, qt, RKa);
    } else if (li.d_head % 8 == 0 && li.seg_cols % 8 == 0 && reinterpret_cast<uintptr_t>(q) % 16 == 0 &&
        reinterpret_cast<uintptr_t>(w_up_k) % 16 == 0 && li.d_head * esz >= 16) {
        const dim3 g_ab((RKa + 31) / 32, (batch * li.q_per_kv + 63) / 64, li.n_kv);
        if (bf)
            hipLaunchKernelGGL(absorb_kernel<uint16_t>, g_ab, dim3(256), 0, s, li, batch, (const uint16_t*)q,
                               (const uint16_t*)w_up_k, qt, RKa, qscale);
        else
            hipLaunchKernelGGL(absorb_kernel<float>, g_ab, dim3(256), 0, s, li, batch, (const float*)q,
                               (const float*)w_up_k, qt, RKa, qscale);
    } else if (bf)
        hipLaunchKernelGGL((tile_gemm_kernel<kAbsorb, uint16_t>), g_abs, dim3(256), 0, s, li, batch, q,
                           (const uint16_t*)w_up_k, qt, RKa, qscale);
    else
        hipLaunchKernelGGL((tile_gemm_kernel<kAbsorb, float>), g_abs, dim3(256), 0, s, li, batch, q,
                           (const float*)w_up_k, qt, RKa, qscale);
    if ((st = hip_check("absorb"))) return st;
    // Timing events, when set, are stamped by the streaming kernel's own dispatch (the extended
    // launches take them), so they measure its execution alone, not the queue's packet gaps.
    void *ev0 = nullptr, *ev1 = nullptr;
    take_timing_events(&ev0, &ev1);
    const hipEvent_t e0 = (hipEvent_t)ev0, e1 = (hipEvent_t)ev1;
#define SPECTRA_TIMED_LAUNCH(KERN, GRID, BLOCK, LDS, ...)                                        \
    do {                                                                                         \
        if (e0) hipExtLaunchKernelGGL(KERN, GRID, BLOCK, LDS, s, e0, e1, 0u, __VA_ARGS__);      \
        else hipLaunchKernelGGL(KERN, GRID, BLOCK, LDS, s, __VA_ARGS__);                          \
    } while (0)
    float* const o = w_o ? ob : out;                   // the attention output before W_O'
    if (p.fast) {
        const int lds = kFastLds;
        // smallest compiled width set that holds every width of the layout
        int used = 0;
        for (int t = 0; t < 2; ++t)
            for (int c = 0; c < li.t[t].n_chunks; ++c) used |= 1 << li.t[t].width[c];
        const int masks[] = {kMaskHigh, kMaskMid, kMaskLow, kMaskAll};
        int mask = kMaskAll;
        for (int m : masks)
            if ((used & ~m) == 0) { mask = m; break; }
        auto kern = mask == kMaskHigh ? decode_mfma_kernel<kMaskHigh>
                  : mask == kMaskMid  ? decode_mfma_kernel<kMaskMid>
                  : mask == kMaskLow  ? decode_mfma_kernel<kMaskLow>
                                      : decode_mfma_kernel<kMaskAll>;
        if (!reserve_lds((const void*)kern, lds)) return fail(SPECTRA_EHIP, "decode: cannot reserve %d bytes of LDS", lds);
        hipFunction_t jf = nullptr;
        if (jit_on() && (st = jit_decode_kernel(li, &jf, !noalloc))) return st;
        constexpr unsigned kThreads = 64 * 2 * kRoleWaves;
        if (jf) {
            const uint8_t* ck8 = (const uint8_t*)cache_k;
            const uint8_t* cv8 = (const uint8_t*)cache_v;
            int split_tokens = p.split_tokens, n_splits = p.n_splits, rv = RVa;
            int64_t sk = sbk, sv = sbv;
            const float* qtc = qt;
            void* args[] = {&li, &ctx, &ck8, &cv8, &sk, &sv, &qtc, &pm, &pl, &pz, &rv, &split_tokens, &n_splits};
            // the extended launch takes its grid in work-items
            const hipError_t e =
                e0 ? hipExtModuleLaunchKernel(jf, (uint32_t)p.n_splits * kThreads, (uint32_t)batch, (uint32_t)p.n_hg,
                                              kThreads, 1, 1, lds, s, args, nullptr, e0, e1, 0)
                   : hipModuleLaunchKernel(jf, p.n_splits, batch, p.n_hg, kThreads, 1, 1, lds, s, args, nullptr);
            if (e != hipSuccess) return fail(SPECTRA_EHIP, "decode: launch of the specialised kernel failed");
        } else {
            SPECTRA_TIMED_LAUNCH(kern, dim3(p.n_splits, batch, p.n_hg), dim3(kThreads), lds, li, ctx,
                                 (const uint8_t*)cache_k, (const uint8_t*)cache_v, sbk, sbv, qt, pm, pl, pz,
                                 RVa, p.split_tokens, p.n_splits);
        }
        if ((st = hip_check("decode_mfma"))) return st;
    } else if (p.fused) {
        const dim3 gf(batch * li.n_seg), bfz(64 * p.n_splits);
#define SPECTRA_SMALL_FUSED(DT, H, R, G)                                                                    \
        SPECTRA_TIMED_LAUNCH((decode_small_fused_kernel<DT, H, R, G>), gf, bfz, 0, li, ctx, (const DT*)q,  \
                             (const DT*)w_up_k, (const DT*)w_up_v, qscale, (const uint8_t*)cache_k,        \
                             (const uint8_t*)cache_v, sbk, sbv, p.split_tokens, o)
        switch (p.small) {
#define SPECTRA_SMALL_FUSED_CASE(H, R, G)                                                 \
            case small_id(H, R, G):                                                      \
                if (bf) SPECTRA_SMALL_FUSED(uint16_t, H, R, G);                          \
                else SPECTRA_SMALL_FUSED(float, H, R, G);                                \
                break;
            SPECTRA_SMALL_INSTANCES(SPECTRA_SMALL_FUSED_CASE)
#undef SPECTRA_SMALL_FUSED_CASE
            default: return fail(SPECTRA_EINVAL, "decode: no small-rank instance %d", p.small);
        }
#undef SPECTRA_SMALL_FUSED
        if ((st = hip_check("decode_small_fused"))) return st;
        goto out_proj;
    } else if (p.small) {
        const dim3 gs(p.n_splits, batch * li.n_seg);
#define SPECTRA_SMALL(H, R, G) SPECTRA_TIMED_LAUNCH((decode_small_kernel<H, R, G>), gs, dim3(64), 0, li, ctx,        \
                                                    (const uint8_t*)cache_k, (const uint8_t*)cache_v, sbk, sbv, qt,   \
                                                    std::max(p.RK, 1), pm, pl, pz, std::max(p.RV, 1),                \
                                                    p.split_tokens, p.n_splits)
        switch (p.small) {
#define SPECTRA_SMALL_CASE(H, R, G) case small_id(H, R, G): SPECTRA_SMALL(H, R, G); break;
            SPECTRA_SMALL_INSTANCES(SPECTRA_SMALL_CASE)
#undef SPECTRA_SMALL_CASE
            default: return fail(SPECTRA_EINVAL, "decode: no small-rank instance %d", p.small);
        }
#undef SPECTRA_SMALL
        if ((st = hip_check("decode_small"))) return st;
    } else {
        SPECTRA_TIMED_LAUNCH(decode_generic_kernel, dim3(p.n_splits, batch * li.n_seg), dim3(256), 0, li, ctx,
                             (const uint8_t*)cache_k, (const uint8_t*)cache_v, sbk, sbv, qt, std::max(p.RK, 1),
                             pm, pl, pz, std::max(p.RV, 1), p.split_tokens, p.n_splits);
        if ((st = hip_check("decode_generic"))) return st;
    }
#undef SPECTRA_TIMED_LAUNCH
    // lean merge + lift when the shape fits it (one workgroup per key/value head and sequence)
    {
        const int dh = li.d_head, nh = li.q_per_kv;
        const size_t es = bf ? 2 : 4;
        const int rparts = (dh >= 32 && dh <= 256 && (dh & (dh - 1)) == 0) ? 512 / (dh / 2) : 0;
        const int rows = rparts ? 4 * ((RVa + 4 * rparts - 1) / (4 * rparts)) : 1 << 30;
        const int rmax = bf ? 64 : 32;                 // W rows held in registers per thread
        // about one workgroup per compute unit: halve the query heads per workgroup while there
        // are fewer (key/value head, part, sequence) triples than compute units (the W_upV slice
        // is then read once per part, from L2); at most 8 heads per workgroup
        int hpw = nh;
        while (hpw > 8 || (hpw > 1 && (int64_t)li.n_kv * batch * ((nh + hpw - 1) / hpw) < 256)) hpw = (hpw + 1) / 2;
        const bool fits = rparts && RVa <= 512 && rows <= rmax &&
                          (reinterpret_cast<uintptr_t>(w_up_v) % (2 * es)) == 0 && (li.seg_cols % 2) == 0;
        if (fits) {
            const int R = rows <= 32 ? 32 : 64;
            const dim3 g2(li.n_kv * ((nh + hpw - 1) / hpw), batch);
#define SPECTRA_ML2(DT, NH, RR) hipLaunchKernelGGL((merge_lift2_kernel<DT, NH, RR>), g2, dim3(512), 0, s, li, ctx, \
                                                   pm, pl, pz, RVa, p.n_splits, p.split_tokens, hpw,             \
                                                   (const DT*)w_up_v, o)
#define SPECTRA_ML2_NH(DT, RR) \
            switch (hpw) { case 1: SPECTRA_ML2(DT, 1, RR); break; case 2: SPECTRA_ML2(DT, 2, RR); break; \
                          case 3: case 4: SPECTRA_ML2(DT, 4, RR); break; default: SPECTRA_ML2(DT, 8, RR); break; }
            if (bf) {
                if (R == 32) { SPECTRA_ML2_NH(uint16_t, 32) } else { SPECTRA_ML2_NH(uint16_t, 64) }
            } else {
                SPECTRA_ML2_NH(float, 32)
            }
#undef SPECTRA_ML2_NH
#undef SPECTRA_ML2
            if ((st = hip_check("merge_lift"))) return st;
            goto out_proj;
        }
    }
    {
    {
        const void* mk = bf ? (const void*)merge_lift_kernel<uint16_t> : (const void*)merge_lift_kernel<float>;
        if (!reserve_lds(mk, kMergeLds)) return fail(SPECTRA_EHIP, "decode: cannot reserve %d bytes of LDS", kMergeLds);
    }
    // about one workgroup per compute unit: split each key/value head's query heads into groups
    int hpw = li.q_per_kv;
    while (hpw > 1 && (int64_t)li.n_kv * batch * ((li.q_per_kv + hpw - 1) / hpw) < 256) hpw = (hpw + 1) / 2;
    const dim3 g_ml(li.n_kv * ((li.q_per_kv + hpw - 1) / hpw), batch);
    if (bf)
        hipLaunchKernelGGL(merge_lift_kernel<uint16_t>, g_ml, dim3(256), kMergeLds, s, li, ctx, pm, pl,
                           pz, RVa, p.n_splits, p.split_tokens, (const uint16_t*)w_up_v, o, hpw);
    else
        hipLaunchKernelGGL(merge_lift_kernel<float>, g_ml, dim3(256), kMergeLds, s, li, ctx, pm, pl,
                           pz, RVa, p.n_splits, p.split_tokens, (const float*)w_up_v, o, hpw);
    if ((st = hip_check("merge_lift"))) return st;
    }
out_proj:
    if (w_o) {
        const dim3 g_out((li.d_model + 31) / 32, (batch + 31) / 32, 1);
        if (bf)
            hipLaunchKernelGGL((tile_gemm_kernel<kOutProj, uint16_t>), g_out, dim3(256), 0, s, li, batch, ob,
                               (const uint16_t*)w_o, out, li.n_q * li.d_head, 1.0f);
        else
            hipLaunchKernelGGL((tile_gemm_kernel<kOutProj, float>), g_out, dim3(256), 0, s, li, batch, ob,
                               (const float*)w_o, out, li.n_q * li.d_head, 1.0f);
        if ((st = hip_check("out_proj"))) return st;
    }
    return SPECTRA_OK;
}

extern "C" {

spectra_status spectra_unpack_dequant(const spectra_layout* layout, int32_t tensor, const void* cache,
                                      int64_t cap_tokens, int32_t batch, int64_t pos0, int64_t n_tok,
                                      float* out, void* stream) {
    clear_error();
    LayoutInfo li;
    spectra_status st = make_layout(layout, &li);
    if (st) return st;
    if (tensor != 0 && tensor != 1) return fail(SPECTRA_EINVAL, "unpack: tensor must be 0 or 1");
    if (!cache || !out) return fail(SPECTRA_EINVAL, "unpack: NULL pointer");
    if (batch <= 0 || pos0 < 0 || n_tok < 0) return fail(SPECTRA_EINVAL, "unpack: bad range");
    if (pos0 + n_tok > cap_tokens) return fail(SPECTRA_ECAPACITY, "unpack: range beyond capacity");
    const int64_t total = n_tok * li.t[tensor].r_act;
    if (total == 0) return SPECTRA_OK;
    const int64_t nblk = (cap_tokens + kBT - 1) / kBT;
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)((total + 255) / 256), batch), dim3(256), 0, (hipStream_t)stream,
                       li, (int)tensor, (const uint8_t*)cache, nblk * li.t[tensor].block_bytes, pos0, n_tok, out);
    return hip_check("unpack");
}

}  // extern "C"

extern "C" int spectra_set_jit(int mode) {
    using namespace spectra;
    (void)jit_on();                                   // reads SPECTRA_JIT once
    std::lock_guard<std::mutex> lk(g_jit_mu);
    const int prev = g_jit_mode;
    if (mode == 0 || mode == 1) g_jit_mode = mode;
    return prev;
}

extern "C" int spectra_set_key_split(int mode) {
    if (mode == 0 || mode == 1) return spectra::g_key_split_all.exchange(mode);
    return spectra::g_key_split_all.load();
}

extern "C" int spectra_jit_kernel_count(void) {
    std::lock_guard<std::mutex> lk(spectra::g_jit_mu);
    return spectra::g_jit_count;
}
