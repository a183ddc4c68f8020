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
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstring>
#include <type_traits>

#include "spectra_device.h"

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
    int split_tokens, n_splits;
    int RK, RV;                        // widest segment latent (K, V)
    size_t off_qt, off_qhl, off_pm, off_pl, off_pz, off_ob, total;
};

static int seg_r(const LayoutInfo& li, int t, int s) {
    return li.g * (li.t[t].seg_chunk0[s + 1] - li.t[t].seg_chunk0[s]);
}

static bool fast_ok(const LayoutInfo& li) {
    return li.g == 16 && li.n_seg == 1 && li.n_q <= 32 && li.t[0].n_chunks >= 1 &&
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
    p.off_ob = o;  o += align256((size_t)B * li.n_q * li.d_head * 4);
    p.total = o;
    return p;
}

// ------------------------------------------------------------ matrix-core decode kernel

// (x & mask) | orv: the compiler selects one v_and_or_b32 for it.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t orv) {
    return (x & mask) | orv;                           // v_and_or_b32
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

// K group operands: this lane's 32 codes (w8, first B words valid) are coordinates 8H..8H+7
// of token pi(m) in each quarter T, sb[T] (low 16 bits) their fp16 scales.  a[T] = c^ = s (u - h)
// rounded once to fp16; the query side carries the precision (q~ = hi + lo, two products),
// since score errors are amplified by the softmax while value errors enter linearly.
template <int B>
__device__ __forceinline__ void k_operands(const uint32_t (&w8)[8], const uint32_t (&sb)[4], uint32_t magic,
                                           half8_t (&a)[4]) {
#pragma clang fp contract(off)
    uint32_t w[B];
#pragma unroll
    for (int i = 0; i < B; ++i) w[i] = w8[i];
    half2_t u[16];
    unpack_run<B>(w, magic, u);
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
}

// V group operands: this lane's 32 codes are coordinate (lane & 15) of tokens 32T + 8q + e,
// vs[T] the eight tokens' fp16 scales.  a[T] = c^ rounded once to fp16.
template <int B>
__device__ __forceinline__ void v_operands(const uint32_t (&w8)[8], const uint4 (&vs)[4], uint32_t magic,
                                           half8_t (&a)[4]) {
#pragma clang fp contract(off)
    uint32_t w[B];
#pragma unroll
    for (int i = 0; i < B; ++i) w[i] = w8[i];
    half2_t u[16];
    unpack_run<B>(w, magic, u);
#pragma unroll
    for (int T = 0; T < 4; ++T) {
        const uint32_t sp[4] = {vs[T].x, vs[T].y, vs[T].z, vs[T].w};
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) {
            half2_t s2;
            __builtin_memcpy(&s2, &sp[pr], 4);
            const half2_t c2 = u[4 * T + pr] * s2;
            a[T][2 * pr] = c2[0];
            a[T][2 * pr + 1] = c2[1];
        }
    }
}

// Operands of a group of width bw (one of WMASK's widths): an if-else chain over the compiled
// widths whose last arm (the narrowest compiled width) is unconditional, so every path defines
// the operands.
template <int WMASK, int BW = 8>
__device__ __forceinline__ void k_operands_w(int bw, const uint32_t (&w8)[8], const uint32_t (&sb)[4],
                                             uint32_t magic, half8_t (&a)[4]) {
    if constexpr (BW >= 1) {
        if constexpr (!((WMASK >> BW) & 1)) k_operands_w<WMASK, BW - 1>(bw, w8, sb, magic, a);
        else if constexpr ((WMASK & ((1 << BW) - 1)) == 0) k_operands<BW>(w8, sb, magic, a);
        else if (bw == BW) k_operands<BW>(w8, sb, magic, a);
        else k_operands_w<WMASK, BW - 1>(bw, w8, sb, magic, a);
    }
}
template <int WMASK, int BW = 8>
__device__ __forceinline__ void v_operands_w(int bw, const uint32_t (&w8)[8], const uint4 (&vs)[4],
                                             uint32_t magic, half8_t (&a)[4]) {
    if constexpr (BW >= 1) {
        if constexpr (!((WMASK >> BW) & 1)) v_operands_w<WMASK, BW - 1>(bw, w8, vs, magic, a);
        else if constexpr ((WMASK & ((1 << BW) - 1)) == 0) v_operands<BW>(w8, vs, magic, a);
        else if (bw == BW) v_operands<BW>(w8, vs, magic, a);
        else v_operands_w<WMASK, BW - 1>(bw, w8, vs, magic, a);
    }
}

// s_waitcnt vmcnt(n), other counters untouched (gfx9 encoding: vmcnt bits [3:0] and [15:14]).
template <int N>
__device__ __forceinline__ void waitcnt_vm() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// n is wave-uniform.  Counts above 63 wait for 63: a wave never has more than 63 vector memory
// operations in flight (issue stalls at the counter's maximum), and they complete in order, so
// an operation followed by 64 or more later ones has completed.
__device__ __forceinline__ void wait_vmcnt(int n) {
    switch (n) {
#define SPECTRA_W(N) case N: waitcnt_vm<N>(); break;
        SPECTRA_W(0) SPECTRA_W(1) SPECTRA_W(2) SPECTRA_W(3) SPECTRA_W(4) SPECTRA_W(5) SPECTRA_W(6) SPECTRA_W(7)
        SPECTRA_W(8) SPECTRA_W(9) SPECTRA_W(10) SPECTRA_W(11) SPECTRA_W(12) SPECTRA_W(13) SPECTRA_W(14)
        SPECTRA_W(15) SPECTRA_W(16) SPECTRA_W(17) SPECTRA_W(18) SPECTRA_W(19) SPECTRA_W(20) SPECTRA_W(21)
        SPECTRA_W(22) SPECTRA_W(23) SPECTRA_W(24) SPECTRA_W(25) SPECTRA_W(26) SPECTRA_W(27) SPECTRA_W(28)
        SPECTRA_W(29) SPECTRA_W(30) SPECTRA_W(31) SPECTRA_W(32) SPECTRA_W(33) SPECTRA_W(34) SPECTRA_W(35)
        SPECTRA_W(36) SPECTRA_W(37) SPECTRA_W(38) SPECTRA_W(39) SPECTRA_W(40) SPECTRA_W(41) SPECTRA_W(42)
        SPECTRA_W(43) SPECTRA_W(44) SPECTRA_W(45) SPECTRA_W(46) SPECTRA_W(47) SPECTRA_W(48) SPECTRA_W(49)
        SPECTRA_W(50) SPECTRA_W(51) SPECTRA_W(52) SPECTRA_W(53) SPECTRA_W(54) SPECTRA_W(55) SPECTRA_W(56)
        SPECTRA_W(57) SPECTRA_W(58) SPECTRA_W(59) SPECTRA_W(60) SPECTRA_W(61) SPECTRA_W(62)
#undef SPECTRA_W
        default: waitcnt_vm<63>(); break;
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

// ------------------------------------------------------------ matrix-core decode kernel
//
// One workgroup = one (split, sequence), eight waves: waves 0-3 are key waves, 4-7 value
// waves, one of each per SIMD, so that one role's waits are covered by the other's work.
// Wave w of a role owns the groups ("slots") c = w, w + 4, ... of its tensor (at most 8).
//
// Codes go from HBM straight into registers: each slot keeps the b words of this lane's run
// (and, for keys, the lane's four scales), and right after a slot of block n is consumed the
// same registers are reloaded with block n + 1 (a one-block prefetch ring).  Value waves load
// their slots' fp16 scales (256 bytes per group and block) into registers one block ahead and
// store them to their own LDS area when the block starts.  Key waves keep their q~ operands in
// LDS.
//
// Key waves, block n: partial scores of their groups for the block's four 32-token quarters
// (two fp16 matrix-core products per tile: c^ times q~ hi and lo); three partial tiles go to
// LDS and the fourth is completed with the other waves' partials (barrier A), so key wave w
// holds the full scores of quarter w; block maxima per head (barrier B); then p = 2^(s - m),
// written to LDS as fp16 with the rescale factor 2^(m_old - m_new).
// Value waves process block n - 1 (from barrier A of block n on; they meet barrier B after
// their first slots) while the key waves work on block n: z = z * alpha + C^T P.
constexpr int kRoleWaves = 4;
constexpr int kSlots = 8;
constexpr int kQLds = kRoleWaves * kSlots * 2 * 64 * 16;  // [4 key waves][8 slots][hi, lo][64] half8
constexpr int kVsLds = kRoleWaves * 2048;                 // [4 value waves][8 slots][256 B]
constexpr int kExLds = kRoleWaves * 3 * 4096;             // [4 writers][3 tiles][1024 floats]
constexpr int kPLds = 2 * 8192;                           // [2 buffers][4 T][2 halves][64] half8
constexpr int kSmallLds = 4 * 32 * 4 + 2 * 32 * 4 + 4 * 64 * 4;   // maxima, rescale, row sums
constexpr int kFastLds = kQLds + kVsLds + kExLds + kPLds + kSmallLds;

struct SlotGeom {
    int off[kSlots];      // byte offset of the slot's code chunk in a block (0 for unused slots)
    int wd[kSlots];       // width (0: no group)
    int ns;               // slots in use (slots fill in order)
};

// Chunk offsets by one load per lane and a prefix sum across lanes (at most 32 chunks), then
// the wave's eight slots read out of the lanes.
__device__ __forceinline__ SlotGeom slot_geom(const TensorInfo& T, int w, int lane) {
    const int nc = T.n_chunks;
    const int k = lane & 31;
    const int wk = k < nc ? (int)T.width[k] : 0;
    int incl = 256 * wk;
#pragma unroll
    for (int d = 1; d < 32; d <<= 1) {
        const int t = __shfl_up(incl, d, 32);
        if (k >= d) incl += t;
    }
    const int excl = incl - 256 * wk;
    SlotGeom g;
    g.ns = 0;
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
        const int c = w + kRoleWaves * i;
        g.ns += c < nc ? 1 : 0;
        g.off[i] = c < nc ? __builtin_amdgcn_readlane(excl, c) : 0;
        g.wd[i] = c < nc ? __builtin_amdgcn_readlane(wk, c) : 0;
    }
    return g;
}

// This lane's run words of a slot (word k at chunk word 64 k + lane), HBM -> registers.  Every
// slot issues exactly eight loads, so that the number of loads in flight is a compile-time
// constant: the loads go through a buffer resource whose size is the chunk's 256 b bytes, and
// rows at or past the width (all rows of a slot without a group) fall outside it, which the
// hardware answers with zeros without touching memory.
constexpr int kBufferWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)
__device__ __forceinline__ void ring_load(const uint8_t* __restrict__ chunk, int bw, int lane, uint32_t (&w8)[8]) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(chunk), (short)0, 256 * bw, kBufferWord3);
#pragma unroll
    for (int k = 0; k < 8; ++k) w8[k] = __builtin_amdgcn_raw_buffer_load_b32(r, lane * 4 + 256 * k, 0, 2);
}

// Scales of a value wave's slots for one block, HBM -> registers (then LDS): lane l holds bytes
// 32 (l & 7) .. of slot l / 8's scale chunk (two 16-byte loads); slots without a group, and
// everything when `blk` is past the split (bytes = 0), read as zeros.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void value_scales(const uint8_t* __restrict__ blk, int bytes, const TensorInfo& T,
                                             int w, const SlotGeom& g, int lane, u32x4_t (&v)[2]) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blk), (short)0, bytes, kBufferWord3);
    const int s = lane >> 3;
    const int off = s < g.ns ? T.codes_bytes + 256 * (w + kRoleWaves * s) + 32 * (lane & 7) : bytes;
    v[0] = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
    v[1] = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 2);
}

// Ring waits.  Per slot and block a key wave issues kKeyOps loads (eight code words, one scale
// pair), a value wave kValOps (eight code words), plus kValDma scale loads per block for value
// waves (value_scales); every load is issued whether or not another block follows.  When slot i of block n is
// consumed, the loads issued after it are the later slots of block n, block n+1's scale loads
// and block n+1's earlier slots.
constexpr int kKeyOps = 9, kValOps = 8, kValDma = 2;
constexpr int kValueSlotsBeforeB = 2;   // value slots processed between barriers A and B
template <int PER, int DMA>
__device__ __forceinline__ void ring_wait() { waitcnt_vm<PER * (kSlots - 1) + DMA>(); }

// This lane's four K scales of a slot (entries 4m .. 4m+3 of the group's scale chunk); a
// resource of `bytes` = 0 returns zeros without a memory access.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2_t key_scales(const uint8_t* __restrict__ scale_chunk, int bytes, int m) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(scale_chunk), (short)0, bytes, kBufferWord3);
    return __builtin_amdgcn_raw_buffer_load_b64(r, 8 * m, 0, 2);
}

template <int WMASK>
__device__ __forceinline__ void key_role(const LayoutInfo& li, int b, int w, int lane, int64_t t0, int64_t t1,
                                         const uint8_t* __restrict__ seq, const half8_t* __restrict__ qhl,
                                         unsigned char* smem, float* __restrict__ pm,
                                         float* __restrict__ pl, int64_t pbase) {
    const TensorInfo& TK = li.t[0];
    const int BK = TK.block_bytes;
    const SlotGeom g = slot_geom(TK, w, lane);
    half8_t* qlds = reinterpret_cast<half8_t*>(smem) + w * kSlots * 128;
    float* ex = reinterpret_cast<float*>(smem + kQLds + kVsLds);
    half8_t* plds = reinterpret_cast<half8_t*>(smem + kQLds + kVsLds + kExLds);
    float* tmax = reinterpret_cast<float*>(smem + kQLds + kVsLds + kExLds + kPLds);
    float* alph = tmax + 128;
    float* lred = alph + 64;

    const half8_t* qb = qhl + (int64_t)b * TK.n_chunks * 128;
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
        const int c = w + kRoleWaves * i;
        if (g.wd[i]) {
            const bool head = (lane & 31) < li.n_q;     // lanes of absent heads hold zeros
            qlds[i * 128 + lane] = head ? qb[(c * 64 + lane) * 2] : half8_t{};
            qlds[i * 128 + 64 + lane] = head ? qb[(c * 64 + lane) * 2 + 1] : half8_t{};
        }
    }
    uint32_t magic = 0x60006000u;
    asm volatile("" : "+v"(magic));                    // keep the constant in a vector register
    const int n = lane & 31, H = lane >> 5;
    float m_run = -INFINITY, l_run = 0.0f;
    uint32_t cr[kSlots][8];
    u32x2_t sr[kSlots];

    const int blk0 = (int)(t0 / kBT), blk1 = (int)((t1 + kBT - 1) / kBT);
    const int t0i = (int)t0, t1i = (int)t1;
    __builtin_amdgcn_s_waitcnt(0);                     // q~ operands are in LDS
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
        ring_load(seq + (int64_t)blk0 * BK + g.off[i], g.wd[i], lane, cr[i]);
        sr[i] = key_scales(seq + (int64_t)blk0 * BK + TK.codes_bytes + 256 * (w + kRoleWaves * i), g.wd[i] ? 256 : 0, n);
        __builtin_amdgcn_sched_barrier(0);             // keep the ring's slot order
    }

    for (int blk = blk0; blk < blk1; ++blk) {
        const int cur = (blk - blk0) & 1;
        const bool more = blk + 1 < blk1;
        const uint8_t* nb = seq + (int64_t)(blk + 1) * BK;
        f32x16_t S[4];
#pragma unroll
        for (int T = 0; T < 4; ++T) S[T] = f32x16_t{};
#pragma unroll
        for (int i = 0; i < kSlots; ++i) {
            if (g.wd[i]) {
                const half8_t qh = qlds[i * 128 + lane], ql = qlds[i * 128 + 64 + lane];
                ring_wait<kKeyOps, 0>();
                const uint32_t ks[4] = {sr[i][0], sr[i][0] >> 16, sr[i][1], sr[i][1] >> 16};
                half8_t a[4];
                k_operands_w<WMASK>(g.wd[i], cr[i], ks, magic, a);
#pragma unroll
                for (int T = 0; T < 4; ++T) S[T] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[T], qh, S[T], 0, 0, 0);
#pragma unroll
                for (int T = 0; T < 4; ++T) S[T] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[T], ql, S[T], 0, 0, 0);
            }
            // next block (nothing is read past the split: sizes 0 return zeros)
            ring_load(nb + g.off[i], more ? g.wd[i] : 0, lane, cr[i]);
            sr[i] = key_scales(nb + TK.codes_bytes + 256 * (w + kRoleWaves * i), more && g.wd[i] ? 256 : 0, n);
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- scores of quarter w: own partial plus the other three waves' partials
#pragma unroll
        for (int T = 0; T < 4; ++T)
            if (T != w) put_tile(ex + (w * 3 + T - (T > w ? 1 : 0)) * 1024, lane, S[T]);
        __syncthreads();                               // A
        float sv[16];
#pragma unroll
        for (int T = 0; T < 4; ++T)
            if (T == w) {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (v != w) add_tile(ex + (v * 3 + w - (w > v ? 1 : 0)) * 1024, lane, S[T]);
#pragma unroll
                for (int a = 0; a < 16; ++a) sv[a] = S[T][a];
            }
        const int lo_t = max(t0i, blk * kBT) - blk * kBT;
        const int hi_t = min(t1i, blk * kBT + kBT) - blk * kBT;
        float mx = -INFINITY;
#pragma unroll
        for (int a = 0; a < 16; ++a) {
            const int tok = 32 * w + 16 * H + a;
            if (tok < lo_t || tok >= hi_t) sv[a] = -INFINITY;
            mx = fmaxf(mx, sv[a]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (H == 0) tmax[w * 32 + n] = mx;
        __syncthreads();                               // B
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
        // P operand of the value products: quarter w, head half n/16, lane 16 q + n%16
        half8_t* pb = plds + cur * 512;
#pragma unroll
        for (int c = 0; c < 2; ++c) pb[(w * 2 + (n >> 4)) * 64 + 16 * (2 * H + c) + (n & 15)] = pw[c];
        if (w == 0 && H == 0) alph[cur * 32 + n] = alpha;
    }
    lred[w * 64 + lane] = l_run;
    __syncthreads();                                   // F: last P visible, row sums written
    if (w == 0 && lane < 32 && lane < li.n_q) {
        float L = 0.0f;
        for (int v = 0; v < kRoleWaves; ++v) L += lred[v * 64 + lane] + lred[v * 64 + lane + 32];
        pm[pbase + lane] = m_run;
        pl[pbase + lane] = L;
    }
}

template <int WMASK>
__device__ __forceinline__ void value_role(const LayoutInfo& li, int w, int lane, int64_t t0, int64_t t1,
                                           const uint8_t* __restrict__ seq, unsigned char* smem,
                                           float* __restrict__ pz, int RV, int64_t pbase) {
    const TensorInfo& TV = li.t[1];
    const int BV = TV.block_bytes;
    const SlotGeom g = slot_geom(TV, w, lane);
    unsigned char* sc = smem + kQLds + w * 2048;
    const half8_t* plds = reinterpret_cast<const half8_t*>(smem + kQLds + kVsLds + kExLds);
    const float* alph = reinterpret_cast<const float*>(smem + kQLds + kVsLds + kExLds + kPLds) + 128;

    uint32_t magic = 0x60006000u;
    asm volatile("" : "+v"(magic));
    f32x4_t Z[kSlots][2];
#pragma unroll
    for (int i = 0; i < kSlots; ++i) Z[i][0] = Z[i][1] = f32x4_t{0, 0, 0, 0};
    uint32_t cr[kSlots][8];
    const int q4 = lane >> 4;

    const int blk0 = (int)(t0 / kBT), blk1 = (int)((t1 + kBT - 1) / kBT);
    u32x4_t vsr[2];
    value_scales(seq + (int64_t)blk0 * BV, BV, TV, w, g, lane, vsr);
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
        ring_load(seq + (int64_t)blk0 * BV + g.off[i], g.wd[i], lane, cr[i]);
        __builtin_amdgcn_sched_barrier(0);             // keep the ring's slot order
    }
    __syncthreads();                                   // A of the first block
    __syncthreads();                                   // B of the first block
    for (int blk = blk0; blk < blk1; ++blk) {
        const int cur = (blk - blk0) & 1;
        const bool more = blk + 1 < blk1;
        const uint8_t* nb = seq + (int64_t)(blk + 1) * BV;
        __syncthreads();                               // A of block blk+1, or F: P of blk visible
        // this block's scales (loaded before its kSlots * kValOps slot loads) -> this wave's LDS
        // area, then the next block's scales into the same registers
        waitcnt_vm<kSlots * kValOps - 1>();
        reinterpret_cast<u32x4_t*>(sc)[2 * lane] = vsr[0];
        reinterpret_cast<u32x4_t*>(sc)[2 * lane + 1] = vsr[1];
        value_scales(nb, more ? BV : 0, TV, w, g, lane, vsr);
        __builtin_amdgcn_sched_barrier(0);
        const unsigned char* scb = sc;

        const float a_lo = alph[cur * 32 + (lane & 15)];
        const float a_hi = alph[cur * 32 + 16 + (lane & 15)];
        if (__builtin_amdgcn_ballot_w64(a_lo != 1.0f || a_hi != 1.0f)) {   // some head's maximum moved
#pragma unroll
            for (int i = 0; i < kSlots; ++i) {
                Z[i][0] *= a_lo;
                Z[i][1] *= a_hi;
            }
        }
        half8_t P[4][2];
        const half8_t* pb = plds + cur * 512;
#pragma unroll
        for (int T = 0; T < 4; ++T) {
            P[T][0] = pb[(T * 2 + 0) * 64 + lane];
            P[T][1] = pb[(T * 2 + 1) * 64 + lane];
        }
#pragma unroll
        for (int i = 0; i < kSlots; ++i) {
            if (g.wd[i]) {
                uint4 vs[4];
#pragma unroll
                for (int T = 0; T < 4; ++T) vs[T] = *reinterpret_cast<const uint4*>(scb + 256 * i + 2 * (32 * T + 8 * q4));
                ring_wait<kValOps, kValDma>();
                half8_t a[4];
                v_operands_w<WMASK>(g.wd[i], cr[i], vs, magic, a);
#pragma unroll
                for (int T = 0; T < 4; ++T) {
                    Z[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[T], P[T][0], Z[i][0], 0, 0, 0);
                    Z[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[T], P[T][1], Z[i][1], 0, 0, 0);
                }
            }
            ring_load(nb + g.off[i], more ? g.wd[i] : 0, lane, cr[i]);   // next block (zeros past the split)
            __builtin_amdgcn_sched_barrier(0);
            // B of block blk+1: the key waves' short reduction runs while this wave works
            if (i == kValueSlotsBeforeB - 1 && more) __syncthreads();
        }
    }
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
        if (!g.wd[i]) continue;
        const int c = w + kRoleWaves * i;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int head = 16 * hh + (lane & 15);
            if (head >= li.n_q) continue;
            float* dst = pz + (pbase + head) * RV + 16 * c + 4 * (lane >> 4);
            *reinterpret_cast<f32x4_t*>(dst) = Z[i][hh];
        }
    }
}

template <int WMASK>   // bit b set: code paths for width b are compiled in
__global__ __launch_bounds__(512, 1) void decode_mfma_kernel(
    LayoutInfo li, Positions ctx, const uint8_t* __restrict__ cache_k,
    const uint8_t* __restrict__ cache_v, int64_t seq_bytes_k, int64_t seq_bytes_v,
    const half8_t* __restrict__ qhl, float* __restrict__ pm, float* __restrict__ pl,
    float* __restrict__ pz, int RV, int split_tokens, int n_splits) {
    const int split = blockIdx.x, b = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t0 = (int64_t)split * split_tokens;
    const int64_t t1 = min((int64_t)ctx.v[b], t0 + split_tokens);
    if (t0 >= t1) return;
    extern __shared__ __align__(16) unsigned char smem[];
    const int64_t pbase = ((int64_t)b * n_splits + split) * li.n_q;
    if (wid < kRoleWaves)
        key_role<WMASK>(li, b, wid, lane, t0, t1, cache_k + (int64_t)b * seq_bytes_k, qhl, smem, pm, pl, pbase);
    else
        value_role<WMASK>(li, wid - kRoleWaves, lane, t0, t1, cache_v + (int64_t)b * seq_bytes_v, smem, pz, RV, pbase);
}

// ----------------------------------------------------------------- generic decode kernel

// Dequantised latent coordinate (chunk c, coordinate j) of slot tau of a block.
__device__ __forceinline__ float dequant_at(const TensorInfo& ti, int kind, int g, const uint8_t* blk,
                                            int c, int64_t code_off, int tau, int j) {
    const int bw = ti.width[c];
    const uint32_t u = read_code(kind, g, bw, blk + code_off, tau, j);
    const uint16_t sb = reinterpret_cast<const uint16_t*>(blk + ti.codes_bytes + 256 * c)[scale_index(kind, g, tau)];
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
                                                        int ld, float alpha, half8_t* __restrict__ qhl) {
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
            if constexpr (MODE == kAbsorb) {
                const float v = acc[i][j] * alpha;
                out[row * ld + n] = v;
                if (qhl) {
                    // matrix-core operand of q~ (chunk n/16, lane 32 H + head, element e), hi and lo
                    const int head = (int)(row % li.n_q), bq = (int)(row / li.n_q);
                    const int c = n >> 4, H = (n >> 3) & 1, e = n & 7;
                    _Float16* dst = reinterpret_cast<_Float16*>(qhl) +
                                    ((((int64_t)bq * li.t[0].n_chunks + c) * 64 + 32 * H + head) * 2) * 8 + e;
                    const _Float16 hi = (_Float16)v;
                    dst[0] = hi;
                    dst[8] = (_Float16)(v - (float)hi);
                }
            }
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
    {
        const size_t es = dtype == SPECTRA_BF16 ? 2 : 4;
        if ((reinterpret_cast<uintptr_t>(w_up_v) & 15) || (li.seg_cols * es) % 16 || (li.d_head * es) % 16)
            return fail(SPECTRA_ENOTSUP, "decode: W_upV rows must start on 16-byte boundaries (d_head %d)", li.d_head);
    }
    if (workspace_bytes < p.total)
        return fail(SPECTRA_ECAPACITY, "decode: workspace %zu bytes < %zu needed", workspace_bytes, p.total);
    hipStream_t s = (hipStream_t)stream;
    unsigned char* ws = (unsigned char*)workspace;
    float* qt = (float*)(ws + p.off_qt);
    half8_t* qhl = (half8_t*)(ws + p.off_qhl);
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
    half8_t* qop = p.fast ? qhl : nullptr;            // the matrix-core kernel's q~ operands
    if (bf)
        hipLaunchKernelGGL((tile_gemm_kernel<kAbsorb, uint16_t>), g_abs, dim3(256), 0, s, li, batch, q,
                           (const uint16_t*)w_up_k, qt, RKa, qscale, qop);
    else
        hipLaunchKernelGGL((tile_gemm_kernel<kAbsorb, float>), g_abs, dim3(256), 0, s, li, batch, q,
                           (const float*)w_up_k, qt, RKa, qscale, qop);
    if ((st = hip_check("absorb"))) return st;
    void *ev0 = nullptr, *ev1 = nullptr;
    take_timing_events(&ev0, &ev1);
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
        static int lds_reserved[4] = {0, 0, 0, 0};
        const int mi = mask == kMaskHigh ? 0 : mask == kMaskMid ? 1 : mask == kMaskLow ? 2 : 3;
        if (lds > lds_reserved[mi]) {
            if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
                return fail(SPECTRA_EHIP, "decode: cannot reserve %d bytes of LDS", lds);
            lds_reserved[mi] = lds;
        }
        if (ev0) (void)hipEventRecord((hipEvent_t)ev0, s);
        hipLaunchKernelGGL(kern, dim3(p.n_splits, batch), dim3(64 * 2 * kRoleWaves), lds, s, li, ctx,
                           (const uint8_t*)cache_k, (const uint8_t*)cache_v, sbk, sbv, qhl, pm, pl, pz,
                           RVa, p.split_tokens, p.n_splits);
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
    static int merge_lds_reserved[2] = {0, 0};
    const int mi2 = bf ? 1 : 0;
    if (merge_lds_reserved[mi2] < kMergeLds) {
        const void* mk = bf ? (const void*)merge_lift_kernel<uint16_t> : (const void*)merge_lift_kernel<float>;
        if (hipFuncSetAttribute(mk, hipFuncAttributeMaxDynamicSharedMemorySize, kMergeLds) != hipSuccess)
            return fail(SPECTRA_EHIP, "decode: cannot reserve %d bytes of LDS", kMergeLds);
        merge_lds_reserved[mi2] = kMergeLds;
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
    if (w_o) {
        const dim3 g_out((li.d_model + 31) / 32, (batch + 31) / 32, 1);
        if (bf)
            hipLaunchKernelGGL((tile_gemm_kernel<kOutProj, uint16_t>), g_out, dim3(256), 0, s, li, batch, ob,
                               (const uint16_t*)w_o, out, li.n_q * li.d_head, 1.0f, nullptr);
        else
            hipLaunchKernelGGL((tile_gemm_kernel<kOutProj, float>), g_out, dim3(256), 0, s, li, batch, ob,
                               (const float*)w_o, out, li.n_q * li.d_head, 1.0f, nullptr);
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
