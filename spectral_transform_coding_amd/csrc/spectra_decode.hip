// Decode attention over the packed latent cache (gfx950).
//
// "SPECTRA" technical summary, SPECTRA pipeline stage 3: keys and values are rebuilt from the
// latent cache for standard attention.  Here the rebuild is folded into the query and the
// output (latent-space attention, "Significance" section):
//   scores  S[t,h] = c^K_t . q~_h,   q~_h = scale * log2(e) * W_upK[:, kv(h)] q_h
//   values  z_h    = sum_t p[t,h] c^V_t,   o_h = (z_h / l_h) W_upV[:, kv(h)]
// which equals softmax(scale K^ q) V^ with K^ = C^K W_upK, V^ = C^V W_upV.
//
// Kernels: absorb (q~), pack_q (fp16 hi/lo matrix-core operands of q~), decode_mfma (stream
// the cache, unpack, dequantise, scores and value accumulation on the matrix cores, split-K
// online softmax), decode_generic (same on the vector ALUs for layouts the fast kernel does
// not cover), combine (merge splits, lift by W_upV), output projection (optional W_O').
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstring>
#include <type_traits>

#include "spectra_device.h"

namespace spectra {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kFastWaves = 4;          // waves per workgroup of the matrix-core kernel
constexpr int kFastMaxChunks = 32;     // non-empty groups per tensor (8 per wave)
constexpr int kFastTail = 8192 + 512 + 1024;           // P operands, maxima, row sums
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
    int split_tokens, n_splits;
    int RK, RV;                        // widest segment latent (K, V)
    size_t off_qt, off_qhl, off_pm, off_pl, off_pz, off_zm, off_ob, total;
};

static int seg_r(const LayoutInfo& li, int t, int s) {
    return li.g * (li.t[t].seg_chunk0[s + 1] - li.t[t].seg_chunk0[s]);
}

static bool fast_ok(const LayoutInfo& li) {
    return li.g == 16 && li.n_seg == 1 && li.n_q <= 32 && li.t[0].n_chunks <= kFastMaxChunks &&
           li.t[1].n_chunks <= kFastMaxChunks;
}

static bool generic_ok(const LayoutInfo& li) {
    const int hs = li.n_q / li.n_seg;
    if (hs > kGenMaxH) return false;
    for (int s = 0; s < li.n_seg; ++s)
        if (seg_r(li, 0, s) > kGenMaxR || seg_r(li, 1, s) > kGenMaxR || hs * seg_r(li, 1, s) > kGenMaxHR)
            return false;
    return true;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static DecodePlan make_plan(const LayoutInfo& li, int B, int64_t max_ctx) {
    DecodePlan p{};
    p.fast = fast_ok(li);
    p.RK = p.RV = 0;
    for (int s = 0; s < li.n_seg; ++s) {
        p.RK = std::max(p.RK, seg_r(li, 0, s));
        p.RV = std::max(p.RV, seg_r(li, 1, s));
    }
    // Splits: about one workgroup per compute unit for the matrix-core kernel (each split
    // writes a float32 partial of n_q x r_act, so fewer, longer splits cost less traffic), four
    // per compute unit for the generic kernel (one per sequence, segment and split).
    const int64_t blocks = std::max<int64_t>(1, (max_ctx + kBT - 1) / kBT);
    const int64_t units = p.fast ? (int64_t)B : (int64_t)B * li.n_seg;
    const int64_t target = p.fast ? 256 : 1024;
    int64_t per_seq = std::max<int64_t>(1, (target + units - 1) / units);
    per_seq = std::min(per_seq, blocks);
    const int64_t bps = (blocks + per_seq - 1) / per_seq;
    p.split_tokens = (int)(bps * kBT);
    p.n_splits = (int)((blocks + bps - 1) / bps);
    size_t o = 0;
    p.off_qt = o;  o += align256((size_t)B * li.n_q * std::max(p.RK, 1) * 4);
    p.off_qhl = o; o += p.fast ? align256((size_t)B * std::max(li.t[0].n_chunks, 1) * 64 * 32) : 0;
    p.off_pm = o;  o += align256((size_t)B * p.n_splits * li.n_q * 4);
    p.off_pl = o;  o += align256((size_t)B * p.n_splits * li.n_q * 4);
    p.off_pz = o;  o += align256((size_t)B * p.n_splits * li.n_q * std::max(p.RV, 1) * 4);
    p.off_zm = o;  o += align256((size_t)B * li.n_q * std::max(p.RV, 1) * 4);
    p.off_ob = o;  o += align256((size_t)B * li.n_q * li.d_head * 4);
    p.total = o;
    return p;
}

// --------------------------------------------------------------- absorb and pack q~

// Matrix-core B operand of q~ per (sequence, K chunk), lane l = 32 H + n: head n, latent
// coordinates 16 c + 8 H + e (e = 0..7), as fp16 hi and lo = fp16(q~ - hi).
__global__ __launch_bounds__(64) void pack_q_kernel(LayoutInfo li, const float* __restrict__ qt,
                                                    int RK, half8_t* __restrict__ qhl) {
    const int c = blockIdx.x, b = blockIdx.y, l = threadIdx.x;
    const int n = l & 31, H = l >> 5;
    half8_t hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = n < li.n_q ? qt[((int64_t)b * li.n_q + n) * RK + 16 * c + 8 * H + e] : 0.0f;
        const _Float16 h = (_Float16)x;
        hi[e] = h;
        lo[e] = (_Float16)(x - (float)h);
    }
    const int64_t base = (((int64_t)b * li.t[0].n_chunks + c) * 64 + l) * 2;
    qhl[base] = hi;
    qhl[base + 1] = lo;
}

// ------------------------------------------------------------ matrix-core decode kernel

// Pair i (0..15) of a run of B-bit codes held in B words, as two fp16 values u - (2^B-1)/2.
// The pair's codes sit at the same offset in the low and high 16 bits; shifting them to bit 1
// of each half and OR-ing 0x6000 gives the fp16 numbers 512 + u (spacing 1/2 there), from
// which 512 + (2^B-1)/2 (representable) is subtracted exactly.
// v_and_or_b32 with the mask in a scalar register and the OR term in a vector register (gfx9
// VOP3 encodings take no literal constants).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t orv) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(orv));
    return r;
}

// Pair i (0..15) of a run of B-bit codes held in B words, as two fp16 values u - (2^B-1)/2.
// The pair's codes sit at the same offset in the low and high 16 bits; shifting them to bit 1
// of each half and OR-ing 0x6000 gives the fp16 numbers 512 + u (spacing 1/2 there), from
// which 512 + (2^B-1)/2 (representable) is subtracted exactly.  `magic` holds 0x60006000.
template <int B, int I>
__device__ __forceinline__ half2_t run_pair(const uint32_t (&w)[B], uint32_t magic) {
    constexpr int gam = I * B, k = gam >> 4, off = gam & 15;
    constexpr uint32_t M = (1u << B) - 1u;
    uint32_t bits;
    if constexpr (off + B <= 16) {
        uint32_t t;
        if constexpr (off >= 1) t = w[k] >> (off - 1);
        else t = w[k] << 1;
        bits = and_or(t, (M << 1) | (M << 17), magic);
    } else {
        constexpr int lo = 16 - off;             // bits in word k
        constexpr uint32_t Ml = (1u << lo) - 1u, Mh = (1u << (B - lo)) - 1u;
        const uint32_t a = and_or(w[k] >> (off - 1), (Ml << 1) | (Ml << 17), magic);
        bits = and_or(w[k + 1] << (lo + 1), (Mh << (lo + 1)) | (Mh << (lo + 17)), a);
    }
    half2_t x;
    __builtin_memcpy(&x, &bits, 4);
    const _Float16 cst = (_Float16)(512.0f + 0.5f * (float)M);
    const half2_t off2 = {cst, cst};
    return x - off2;
}

template <int B>
__device__ __forceinline__ void unpack_run(const uint32_t (&w)[B], uint32_t magic, half2_t (&u)[16]) {
    u[0] = run_pair<B, 0>(w, magic);   u[1] = run_pair<B, 1>(w, magic);
    u[2] = run_pair<B, 2>(w, magic);   u[3] = run_pair<B, 3>(w, magic);
    u[4] = run_pair<B, 4>(w, magic);   u[5] = run_pair<B, 5>(w, magic);
    u[6] = run_pair<B, 6>(w, magic);   u[7] = run_pair<B, 7>(w, magic);
    u[8] = run_pair<B, 8>(w, magic);   u[9] = run_pair<B, 9>(w, magic);
    u[10] = run_pair<B, 10>(w, magic); u[11] = run_pair<B, 11>(w, magic);
    u[12] = run_pair<B, 12>(w, magic); u[13] = run_pair<B, 13>(w, magic);
    u[14] = run_pair<B, 14>(w, magic); u[15] = run_pair<B, 15>(w, magic);
}

// K chunk: this lane's 32 codes (w8, first B words valid) are coordinates 8H..8H+7 of token
// pi(m) in each quarter T, sb[T] its scales.  c^ = s (u - h) rounded once to fp16; the query
// side carries the precision (q~ = hi + lo, two products), since score errors are amplified
// by the softmax while value errors enter linearly.
template <int B>
__device__ __forceinline__ void k_chunk(const uint32_t (&w8)[8], const uint32_t (&sb)[4], const half8_t qh,
                                        const half8_t ql, uint32_t magic, f32x16_t (&S)[4]) {
#pragma clang fp contract(off)
    uint32_t w[B];
#pragma unroll
    for (int i = 0; i < B; ++i) w[i] = w8[i];
    half2_t u[16];
    unpack_run<B>(w, magic, u);
    half8_t a[4];
#pragma unroll
    for (int T = 0; T < 4; ++T) {
        const uint16_t s16 = (uint16_t)sb[T];
        _Float16 sc;
        __builtin_memcpy(&sc, &s16, 2);
        const half2_t s2 = {sc, sc};
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) {
            const half2_t c2 = u[4 * T + pr] * s2;
            a[T][2 * pr] = c2[0];
            a[T][2 * pr + 1] = c2[1];
        }
    }
#pragma unroll
    for (int T = 0; T < 4; ++T) S[T] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[T], qh, S[T], 0, 0, 0);
#pragma unroll
    for (int T = 0; T < 4; ++T) S[T] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[T], ql, S[T], 0, 0, 0);
}

// Up to 8 words of this lane's run of a chunk in LDS (word w at chunk word 64 w + lane; reads
// past a short run stay inside the LDS allocation, which always follows a K block with at
// least 2 KB).
__device__ __forceinline__ void lds_run8(const unsigned char* chunk, int lane, uint32_t (&w8)[8]) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(chunk) + lane;
#pragma unroll
    for (int i = 0; i < 8; ++i) w8[i] = src[64 * i];
}

// V chunk: this lane's 32 codes (already in registers) are coordinate (lane & 15) of tokens
// 32T + 8q + e.  c^ rounded once to fp16; z^T[coords x heads] += C^T P on the matrix cores.
template <int B>
__device__ __forceinline__ void v_chunk(const uint32_t (&w8)[8], const uint4 (&vs)[4],
                                        const half8_t (&P)[4][2], uint32_t magic, f32x4_t (&Z)[2]) {
#pragma clang fp contract(off)
    uint32_t w[B];
#pragma unroll
    for (int i = 0; i < B; ++i) w[i] = w8[i];
    half2_t u[16];
    unpack_run<B>(w, magic, u);
#pragma unroll
    for (int T = 0; T < 4; ++T) {
        const uint32_t sp[4] = {vs[T].x, vs[T].y, vs[T].z, vs[T].w};
        half8_t a;
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) {
            half2_t s2;
            __builtin_memcpy(&s2, &sp[pr], 4);
            const half2_t c2 = u[4 * T + pr] * s2;
            a[2 * pr] = c2[0];
            a[2 * pr + 1] = c2[1];
        }
        Z[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, P[T][0], Z[0], 0, 0, 0);
        Z[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, P[T][1], Z[1], 0, 0, 0);
    }
}

// This lane's B words of a V chunk run, straight from global memory into registers.
template <int B>
__device__ __forceinline__ void v_load(const uint8_t* __restrict__ chunk, int lane, uint32_t (&w8)[8]) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(chunk) + lane;
#pragma unroll
    for (int i = 0; i < B; ++i) w8[i] = __builtin_nontemporal_load(src + 64 * i);
}

// Asynchronous copy of `bytes` (a multiple of 16) from global to LDS by the workgroup's four
// waves, 1 KB per wave instruction (each lane moves 16 bytes straight into LDS).  Wave wv
// issues copy_count(bytes, wv) instructions.
__device__ __forceinline__ void stage_copy(const uint8_t* __restrict__ src, unsigned char* dst, int bytes,
                                           int wv, int lane) {
    const int n1k = bytes >> 10;
    for (int c = wv; c < n1k; c += kFastWaves)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src + c * 1024 + lane * 16),
                                         (__attribute__((address_space(3))) void*)(dst + c * 1024), 16, 0, 0);
    const int rem = bytes - (n1k << 10);
    if (rem && wv == (n1k % kFastWaves) && lane * 16 < rem)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src + n1k * 1024 + lane * 16),
                                         (__attribute__((address_space(3))) void*)(dst + n1k * 1024), 16, 0, 0);
}

__device__ __forceinline__ int copy_count(int bytes, int wv) {
    const int n1k = bytes >> 10;
    return (n1k - wv + kFastWaves - 1) / kFastWaves + ((bytes & 1023) && wv == n1k % kFastWaves ? 1 : 0);
}

// s_waitcnt vmcnt(n), other counters untouched (gfx9 encoding: vmcnt bits [3:0] and [15:14]).
template <int N>
__device__ __forceinline__ void waitcnt_vm() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_vmcnt(int n) {   // n is wave-uniform, 0..31
    switch (n) {
#define SPECTRA_W(N) case N: waitcnt_vm<N>(); break;
        SPECTRA_W(0) SPECTRA_W(1) SPECTRA_W(2) SPECTRA_W(3) SPECTRA_W(4) SPECTRA_W(5) SPECTRA_W(6) SPECTRA_W(7)
        SPECTRA_W(8) SPECTRA_W(9) SPECTRA_W(10) SPECTRA_W(11) SPECTRA_W(12) SPECTRA_W(13) SPECTRA_W(14)
        SPECTRA_W(15) SPECTRA_W(16) SPECTRA_W(17) SPECTRA_W(18) SPECTRA_W(19) SPECTRA_W(20) SPECTRA_W(21)
        SPECTRA_W(22) SPECTRA_W(23) SPECTRA_W(24) SPECTRA_W(25) SPECTRA_W(26) SPECTRA_W(27) SPECTRA_W(28)
        SPECTRA_W(29) SPECTRA_W(30) SPECTRA_W(31)
#undef SPECTRA_W
        default: __builtin_amdgcn_s_waitcnt(0); break;
    }
}

// Writes / adds one 32x32 score tile partial (16 floats per lane) to / from LDS, lane-interleaved
// so that each 16-byte access of a wave is contiguous.
__device__ __forceinline__ void put_tile(float* base, int lane, const f32x16_t& v) {
    f32x4_t* d = reinterpret_cast<f32x4_t*>(base);
#pragma unroll
    for (int k = 0; k < 4; ++k) d[k * 64 + lane] = f32x4_t{v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]};
}
__device__ __forceinline__ void add_tile(const float* base, int lane, f32x16_t& v) {
    const f32x4_t* d = reinterpret_cast<const f32x4_t*>(base);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const f32x4_t x = d[k * 64 + lane];
        v[4 * k] += x[0]; v[4 * k + 1] += x[1]; v[4 * k + 2] += x[2]; v[4 * k + 3] += x[3];
    }
}

// One workgroup = one (split, sequence), four waves.  Per 128-token block:
//   * the K block is copied into LDS by DMA, double-buffered (block n+1 streams in while block
//     n is used); the V block's scales likewise; the V codes of block n are loaded by every
//     lane straight into registers at the start of block n and used after the K phase;
//   * wave w owns K chunks w, w+4, ... and V chunks w, w+4, ...; the score partials of the
//     four waves are summed by a two-round exchange through LDS (in the spent K buffer), after
//     which wave w holds the block's quarter T = w and runs its online softmax.
template <int WMASK>   // bit b set: code paths for width b are compiled in
__global__ __launch_bounds__(256, 1) void decode_mfma_kernel(
    LayoutInfo li, Positions ctx, const uint8_t* __restrict__ cache_k,
    const uint8_t* __restrict__ cache_v, int64_t seq_bytes_k, int64_t seq_bytes_v,
    const half8_t* __restrict__ qhl, float* __restrict__ pm, float* __restrict__ pl,
    float* __restrict__ pz, int RV, int split_tokens, int n_splits, int ex_separate) {
    const int split = blockIdx.x, b = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int64_t t0 = (int64_t)split * split_tokens;
    const int64_t t1 = min((int64_t)ctx.v[b], t0 + split_tokens);
    if (t0 >= t1) return;

    const TensorInfo& TK = li.t[0];
    const TensorInfo& TV = li.t[1];
    const int BK = TK.block_bytes, BV = TV.block_bytes;
    const int VS = TV.n_chunks * 256;                  // V scale bytes per block
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char* kbuf = smem;                        // [2][BK]
    unsigned char* vsbuf = smem + 2 * BK;              // [2][VS]
    unsigned char* tail = vsbuf + 2 * VS;
    float* ex_sep = reinterpret_cast<float*>(tail);    // 32 KB exchange when K blocks are small
    if (ex_separate) tail += 32768;
    half8_t* plds = reinterpret_cast<half8_t*>(tail);                             // [4 T][2][64]
    float* tmax = reinterpret_cast<float*>(tail + 8192);                           // [4][32]
    float* lred = tmax + 128;                                                       // [4][64]

    const int nk = TK.n_chunks, nv = TV.n_chunks;
    const int ldk = copy_count(BK, wv), ldvs = copy_count(VS, wv);
    int vc_off[8], kc_off[8], kw[8], vw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int ck = wv + 4 * i;
        int ok = 0, ov = 0;
        for (int c = 0; c < ck && c < nk; ++c) ok += 256 * TK.width[c];
        for (int c = 0; c < ck && c < nv; ++c) ov += 256 * TV.width[c];
        kc_off[i] = __builtin_amdgcn_readfirstlane(ok);
        vc_off[i] = __builtin_amdgcn_readfirstlane(ov);
        kw[i] = __builtin_amdgcn_readfirstlane(ck < nk ? (int)TK.width[ck] : 0);
        vw[i] = __builtin_amdgcn_readfirstlane(ck < nv ? (int)TV.width[ck] : 0);
    }
    // q~ operands of this wave's K chunks stay in registers
    half8_t qh[8], ql[8];
    const half8_t* qb = qhl + (int64_t)b * nk * 128;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = wv + 4 * i;
        if (c < nk) {
            qh[i] = qb[(c * 64 + lane) * 2];
            ql[i] = qb[(c * 64 + lane) * 2 + 1];
        } else {
            qh[i] = half8_t{};
            ql[i] = half8_t{};
        }
    }
    uint32_t magic = 0x60006000u;
    asm volatile("" : "+v"(magic));                    // keep the constant in a vector register

    const int n = lane & 31, H = lane >> 5;
    float m_run = -INFINITY, l_run = 0.0f;
    f32x4_t Z[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i) Z[i][0] = Z[i][1] = f32x4_t{0, 0, 0, 0};
    uint32_t vr[8][8];                                 // V code runs of this wave's chunks

    const uint8_t* seqk = cache_k + (int64_t)b * seq_bytes_k;
    const uint8_t* seqv = cache_v + (int64_t)b * seq_bytes_v;
    const int64_t blk0 = t0 / kBT, blk1 = (t1 + kBT - 1) / kBT;
    __builtin_amdgcn_s_waitcnt(0);                     // q~ operands are in registers
    stage_copy(seqk + blk0 * BK, kbuf, BK, wv, lane);
    stage_copy(seqv + blk0 * BV + TV.codes_bytes, vsbuf, VS, wv, lane);
    for (int64_t blk = blk0; blk < blk1; ++blk) {
        const int cur = (int)((blk - blk0) & 1);
        const bool more = blk + 1 < blk1;
        unsigned char* sK = kbuf + cur * BK;
        const unsigned char* sVs = vsbuf + cur * VS;
        __builtin_amdgcn_s_waitcnt(0);                 // K block and V scales of this block landed
        __syncthreads();                               // ... for every wave; previous buffers free
        // V codes of this block into registers, then the next block's copies (in this order:
        // the V phase waits only for the older V loads)
        {
            const uint8_t* bv = seqv + blk * BV;
#define SPECTRA_V_LOAD(BW)                                                                        \
            if constexpr ((WMASK >> BW) & 1) _Pragma("unroll") for (int i = 0; i < 8; ++i) {       \
                if (vw[i] == BW) v_load<BW>(bv + vc_off[i], lane, vr[i]);                          \
            }
            SPECTRA_V_LOAD(8) SPECTRA_V_LOAD(7) SPECTRA_V_LOAD(6) SPECTRA_V_LOAD(5)
            SPECTRA_V_LOAD(4) SPECTRA_V_LOAD(3) SPECTRA_V_LOAD(2) SPECTRA_V_LOAD(1)
#undef SPECTRA_V_LOAD
        }
        asm volatile("" ::: "memory");
        if (more) {
            stage_copy(seqk + (blk + 1) * BK, kbuf + (cur ^ 1) * BK, BK, wv, lane);
            stage_copy(seqv + (blk + 1) * BV + TV.codes_bytes, vsbuf + (cur ^ 1) * VS, VS, wv, lane);
        }
        const int lo_t = (int)(max(t0, blk * kBT) - blk * kBT);
        const int hi_t = (int)(min(t1, blk * kBT + kBT) - blk * kBT);

        // ---- partial scores over this wave's K chunks, all four quarters
        f32x16_t S[4];
#pragma unroll
        for (int T = 0; T < 4; ++T) S[T] = f32x16_t{};
        {
            // slot-major, the next slot's LDS reads in flight while this slot computes
            const int t = quarter_token(lane & 31);
            uint32_t kr[2][8], ks[2][4];
            auto kfetch = [&](int i, int buf) {
                const unsigned char* ch = sK + kc_off[i];
                const uint16_t* sc = reinterpret_cast<const uint16_t*>(sK + TK.codes_bytes + 256 * (wv + 4 * i));
                lds_run8(ch, lane, kr[buf]);
#pragma unroll
                for (int T = 0; T < 4; ++T) ks[buf][T] = sc[32 * T + t];
            };
            if (kw[0]) kfetch(0, 0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (i + 1 < 8 && kw[i + 1]) kfetch(i + 1, (i + 1) & 1);
#define SPECTRA_K_WIDTH(BW) \
                if constexpr ((WMASK >> BW) & 1) if (kw[i] == BW) k_chunk<BW>(kr[i & 1], ks[i & 1], qh[i], ql[i], magic, S);
                SPECTRA_K_WIDTH(8) SPECTRA_K_WIDTH(7) SPECTRA_K_WIDTH(6) SPECTRA_K_WIDTH(5)
                SPECTRA_K_WIDTH(4) SPECTRA_K_WIDTH(3) SPECTRA_K_WIDTH(2) SPECTRA_K_WIDTH(1)
#undef SPECTRA_K_WIDTH
            }
        }
        float* ex = ex_separate ? ex_sep : reinterpret_cast<float*>(sK);
        if (!ex_separate) __syncthreads();             // the exchange overwrites this K block

        // ---- exchange: round 1 with wave wv^2 (quarters of the other pair), round 2 with wv^1
        {
            const int p1 = wv ^ 2;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int T = p1 ^ k;                  // slot k of writer wv holds quarter (wv^2)^k
#pragma unroll
                for (int TT = 0; TT < 4; ++TT)
                    if (TT == T) put_tile(ex + (wv * 2 + k) * 1024, lane, S[TT]);
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int T = wv ^ k;                  // writer p1's slot k holds quarter wv^k
#pragma unroll
                for (int TT = 0; TT < 4; ++TT)
                    if (TT == T) add_tile(ex + (p1 * 2 + k) * 1024, lane, S[TT]);
            }
            __syncthreads();
            const int p2 = wv ^ 1;
#pragma unroll
            for (int TT = 0; TT < 4; ++TT)
                if (TT == p2) put_tile(ex + wv * 1024, lane, S[TT]);
            __syncthreads();
#pragma unroll
            for (int TT = 0; TT < 4; ++TT)
                if (TT == wv) add_tile(ex + p2 * 1024, lane, S[TT]);
        }

        // ---- this wave's quarter T = wv: masking, quarter maximum per head
        float sv[16];
#pragma unroll
        for (int a = 0; a < 16; ++a) {
            float v = 0.0f;
#pragma unroll
            for (int TT = 0; TT < 4; ++TT)
                if (TT == wv) v = S[TT][a];
            sv[a] = v;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int a = 0; a < 16; ++a) {
            const int tok = 32 * wv + 16 * H + a;
            if (tok < lo_t || tok >= hi_t) sv[a] = -INFINITY;
            mx = fmaxf(mx, sv[a]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (H == 0) tmax[wv * 32 + n] = mx;
        __syncthreads();
        const float M = fmaxf(fmaxf(tmax[n], tmax[32 + n]), fmaxf(tmax[64 + n], tmax[96 + n]));
        const float m_new = fmaxf(m_run, M);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // m_run = -inf gives 0
        m_run = m_new;
        float ps = 0.0f;
        half8_t pw[2];
#pragma unroll
        for (int a = 0; a < 16; ++a) {
            const float p = __builtin_amdgcn_exp2f(sv[a] - m_new);
            ps += p;
            pw[a >> 3][a & 7] = (_Float16)p;
        }
        l_run = l_run * alpha + ps;
        // P operand of the value products: quarter wv, head half n/16, lane 16 q + n%16
#pragma unroll
        for (int c = 0; c < 2; ++c) plds[(wv * 2 + (n >> 4)) * 64 + 16 * (2 * H + c) + (n & 15)] = pw[c];
        __syncthreads();                               // P visible

        // ---- rescale and accumulate values over this wave's V chunks
        wait_vmcnt(more ? ldk + ldvs : 0);             // this block's V codes are in registers
        const float a_lo = __shfl(alpha, lane & 15);
        const float a_hi = __shfl(alpha, 16 + (lane & 15));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            Z[i][0] *= a_lo;
            Z[i][1] *= a_hi;
        }
        half8_t P[4][2];
#pragma unroll
        for (int T = 0; T < 4; ++T) {
            P[T][0] = plds[(T * 2 + 0) * 64 + lane];
            P[T][1] = plds[(T * 2 + 1) * 64 + lane];
        }
        {
            const int q4 = lane >> 4;
            uint4 vs[2][4];
            auto vfetch = [&](int i, int buf) {
                const unsigned char* sc = sVs + 256 * (wv + 4 * i);
#pragma unroll
                for (int T = 0; T < 4; ++T) vs[buf][T] = *reinterpret_cast<const uint4*>(sc + 2 * (32 * T + 8 * q4));
            };
            if (vw[0]) vfetch(0, 0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (i + 1 < 8 && vw[i + 1]) vfetch(i + 1, (i + 1) & 1);
#define SPECTRA_V_WIDTH(BW) \
                if constexpr ((WMASK >> BW) & 1) if (vw[i] == BW) v_chunk<BW>(vr[i], vs[i & 1], P, magic, Z[i]);
                SPECTRA_V_WIDTH(8) SPECTRA_V_WIDTH(7) SPECTRA_V_WIDTH(6) SPECTRA_V_WIDTH(5)
                SPECTRA_V_WIDTH(4) SPECTRA_V_WIDTH(3) SPECTRA_V_WIDTH(2) SPECTRA_V_WIDTH(1)
#undef SPECTRA_V_WIDTH
            }
        }
    }

    // ---- partial results of this split
    __syncthreads();
    lred[wv * 64 + lane] = l_run;
    __syncthreads();
    const int64_t pbase = ((int64_t)b * n_splits + split) * li.n_q;
    if (wv == 0 && lane < 32 && lane < li.n_q) {
        float L = 0.0f;
        for (int w2 = 0; w2 < kFastWaves; ++w2) L += lred[w2 * 64 + lane] + lred[w2 * 64 + lane + 32];
        pm[pbase + lane] = m_run;
        pl[pbase + lane] = L;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (!vw[i]) continue;
        const int c = wv + 4 * i;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int head = 16 * hh + (lane & 15);
            if (head >= li.n_q) continue;
            float* dst = pz + (pbase + head) * RV + 16 * c + 4 * (lane >> 4);
            *reinterpret_cast<f32x4_t*>(dst) = Z[i][hh];
        }
    }
}

// ----------------------------------------------------------------- generic decode kernel

// Dequantised latent coordinate (chunk c, coordinate j) of slot tau of a block.
__device__ __forceinline__ float dequant_at(const TensorInfo& ti, int kind, int g, const uint8_t* blk,
                                            int c, int64_t code_off, int tau, int j) {
    const int bw = ti.width[c];
    const uint32_t u = read_code(kind, g, bw, blk + code_off, tau, j);
    const uint16_t sb = reinterpret_cast<const uint16_t*>(blk + ti.codes_bytes + 256 * c)[tau];
    const float s = f16_bits_to_f32(sb);
    return s * ((float)u - 0.5f * (float)((1u << bw) - 1u));
}

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

// ---------------------------------------------------------------------- combine splits

// Merge the splits of one (sequence, query head):  M = max_s m_s,  w_s = 2^(m_s - M),
// L = sum_s w_s l_s,  z[r] = sum_s w_s z_s[r] / L  (zero for an empty context).
__global__ __launch_bounds__(256) void merge_kernel(LayoutInfo li, Positions ctx,
                                                    const float* __restrict__ pm,
                                                    const float* __restrict__ pl,
                                                    const float* __restrict__ pz, int RV,
                                                    int n_splits, int split_tokens,
                                                    float* __restrict__ zm) {
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int seg = (h / li.q_per_kv) / li.kv_per_seg;
    const int rv = li.g * (li.t[1].seg_chunk0[seg + 1] - li.t[1].seg_chunk0[seg]);
    const int ctxb = ctx.v[b];
    const int ns = ctxb <= 0 ? 0 : (ctxb + split_tokens - 1) / split_tokens;
    const int64_t base = (int64_t)b * n_splits * li.n_q + h;
    __shared__ float wgt[kMaxSplits];
    __shared__ float red[8];
    float mx = -INFINITY;
    for (int sp = tid; sp < ns; sp += 256) mx = fmaxf(mx, pm[base + (int64_t)sp * li.n_q]);
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float ls = 0.0f;
    for (int sp = tid; sp < ns; sp += 256) {
        const float w = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(pm[base + (int64_t)sp * li.n_q] - M);
        wgt[sp] = w;
        ls += w * pl[base + (int64_t)sp * li.n_q];
    }
    for (int o = 32; o > 0; o >>= 1) ls += __shfl_xor(ls, o);
    if ((tid & 63) == 0) red[4 + (tid >> 6)] = ls;
    __syncthreads();
    const float L = red[4] + red[5] + red[6] + red[7];
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    for (int r = tid; r < rv; r += 256) {
        float acc = 0.0f;
#pragma unroll 8
        for (int sp = 0; sp < ns; ++sp) acc += wgt[sp] * pz[(base + (int64_t)sp * li.n_q) * RV + r];
        zm[((int64_t)b * li.n_q + h) * RV + r] = acc * inv;
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

static spectra_status hip_check(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SPECTRA_EHIP, "%s: %s", what, hipGetErrorString(e));
    return SPECTRA_OK;
}

extern "C" {

spectra_status spectra_decode_workspace_bytes(const spectra_layout* layout, int32_t batch,
                                              int64_t max_ctx, size_t* bytes) {
    clear_error();
    LayoutInfo li;
    spectra_status st = make_layout(layout, &li);
    if (st) return st;
    if (!bytes) return fail(SPECTRA_EINVAL, "bytes is NULL");
    if (batch < 0 || max_ctx < 0) return fail(SPECTRA_EINVAL, "negative batch or context");
    *bytes = make_plan(li, std::max(batch, 1), max_ctx).total;
    return SPECTRA_OK;
}

spectra_status spectra_decode_attn(const spectra_layout* layout, spectra_dtype dtype, const void* q,
                                   const void* cache_k, const void* cache_v, int64_t cap_tokens,
                                   int32_t batch, const int32_t* ctx_len, const void* w_up_k,
                                   const void* w_up_v, float softmax_scale, const void* w_o,
                                   float* out, void* workspace, size_t workspace_bytes,
                                   void* stream) {
    clear_error();
    LayoutInfo li;
    spectra_status st = make_layout(layout, &li);
    if (st) return st;
    if (dtype != SPECTRA_F32 && dtype != SPECTRA_BF16) return fail(SPECTRA_ENOTSUP, "decode: unknown dtype %d", (int)dtype);
    if (batch <= 0) return fail(SPECTRA_EINVAL, "decode: batch must be positive");
    if (batch > kMaxB) return fail(SPECTRA_ENOTSUP, "decode: batch %d > %d", batch, kMaxB);
    if (!q || !cache_k || !cache_v || !ctx_len || !w_up_k || !w_up_v || !out || !workspace)
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
    const DecodePlan p = make_plan(li, batch, max_ctx);
    if (!p.fast && !generic_ok(li))
        return fail(SPECTRA_ENOTSUP, "decode: no kernel for this layout (group %d, segments %d, heads %d)", li.g, li.n_seg, li.n_q);
    if (p.RK > 512 || p.RV > 512) return fail(SPECTRA_ENOTSUP, "decode: segment latent wider than 512");
    if (p.n_splits > kMaxSplits) return fail(SPECTRA_ENOTSUP, "decode: %d splits > %d", p.n_splits, kMaxSplits);
    if (workspace_bytes < p.total)
        return fail(SPECTRA_ECAPACITY, "decode: workspace %zu bytes < %zu needed", workspace_bytes, p.total);
    hipStream_t s = (hipStream_t)stream;
    unsigned char* ws = (unsigned char*)workspace;
    float* qt = (float*)(ws + p.off_qt);
    half8_t* qhl = (half8_t*)(ws + p.off_qhl);
    float* pm = (float*)(ws + p.off_pm);
    float* pl = (float*)(ws + p.off_pl);
    float* pz = (float*)(ws + p.off_pz);
    float* zm = (float*)(ws + p.off_zm);
    float* ob = (float*)(ws + p.off_ob);
    const int64_t nblk = (cap_tokens + kBT - 1) / kBT;
    const int64_t sbk = nblk * li.t[0].block_bytes, sbv = nblk * li.t[1].block_bytes;
    const float qscale = softmax_scale * kLog2e;
    const bool bf = dtype == SPECTRA_BF16;

    const int RKa = std::max(p.RK, 1), RVa = std::max(p.RV, 1);
    const dim3 g_abs((RKa + 31) / 32, (batch * li.q_per_kv + 31) / 32, li.n_kv);
    if (bf)
        hipLaunchKernelGGL((tile_gemm_kernel<kAbsorb, uint16_t>), g_abs, dim3(256), 0, s, li, batch, q,
                           (const uint16_t*)w_up_k, qt, RKa, qscale);
    else
        hipLaunchKernelGGL((tile_gemm_kernel<kAbsorb, float>), g_abs, dim3(256), 0, s, li, batch, q,
                           (const float*)w_up_k, qt, RKa, qscale);
    if ((st = hip_check("absorb"))) return st;
    void *ev0 = nullptr, *ev1 = nullptr;
    take_timing_events(&ev0, &ev1);
    if (p.fast) {
        if (li.t[0].n_chunks > 0) {
            hipLaunchKernelGGL(pack_q_kernel, dim3(li.t[0].n_chunks, batch), dim3(64), 0, s, li, qt, RKa, qhl);
            if ((st = hip_check("pack_q"))) return st;
        }
        const int BK = li.t[0].block_bytes, BV = li.t[1].block_bytes;
        const int VS = li.t[1].n_chunks * 256;
        const int ex_separate = BK < 32768 ? 1 : 0;    // the score exchange reuses a large K block
        const int lds = 2 * BK + 2 * VS + (ex_separate ? 32768 : 0) + kFastTail;
        if (lds > kMaxLds) return fail(SPECTRA_ENOTSUP, "decode: cache blocks of %d + %d bytes do not fit in LDS", BK, BV);
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
        static int lds_reserved[4] = {0, 0, 0, 0};
        const int mi = mask == kMaskHigh ? 0 : mask == kMaskMid ? 1 : mask == kMaskLow ? 2 : 3;
        if (lds > lds_reserved[mi]) {
            if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
                return fail(SPECTRA_EHIP, "decode: cannot reserve %d bytes of LDS", lds);
            lds_reserved[mi] = lds;
        }
        if (ev0) (void)hipEventRecord((hipEvent_t)ev0, s);
        hipLaunchKernelGGL(kern, dim3(p.n_splits, batch), dim3(256), lds, s, li, ctx,
                           (const uint8_t*)cache_k, (const uint8_t*)cache_v, sbk, sbv, qhl, pm, pl, pz,
                           std::max(p.RV, 1), p.split_tokens, p.n_splits, ex_separate);
        if (ev1) (void)hipEventRecord((hipEvent_t)ev1, s);
        if ((st = hip_check("decode_mfma"))) return st;
    } else {
        if (ev0) (void)hipEventRecord((hipEvent_t)ev0, s);
        hipLaunchKernelGGL(decode_generic_kernel, dim3(p.n_splits, batch * li.n_seg), dim3(256), 0, s, li, ctx,
                           (const uint8_t*)cache_k, (const uint8_t*)cache_v, sbk, sbv, qt, std::max(p.RK, 1),
                           pm, pl, pz, std::max(p.RV, 1), p.split_tokens, p.n_splits);
        if (ev1) (void)hipEventRecord((hipEvent_t)ev1, s);
        if ((st = hip_check("decode_generic"))) return st;
    }
    float* o = w_o ? ob : out;
    hipLaunchKernelGGL(merge_kernel, dim3(li.n_q, batch), dim3(256), 0, s, li, ctx, pm, pl, pz, RVa, p.n_splits,
                       p.split_tokens, zm);
    if ((st = hip_check("merge"))) return st;
    const dim3 g_lift((li.d_head + 31) / 32, (batch * li.q_per_kv + 31) / 32, li.n_kv);
    if (bf)
        hipLaunchKernelGGL((tile_gemm_kernel<kLift, uint16_t>), g_lift, dim3(256), 0, s, li, batch, zm,
                           (const uint16_t*)w_up_v, o, RVa, 1.0f);
    else
        hipLaunchKernelGGL((tile_gemm_kernel<kLift, float>), g_lift, dim3(256), 0, s, li, batch, zm,
                           (const float*)w_up_v, o, RVa, 1.0f);
    if ((st = hip_check("lift"))) return st;
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
