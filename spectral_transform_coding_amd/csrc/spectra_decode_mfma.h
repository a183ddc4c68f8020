// Matrix-core decode stream kernel of libspectra (gfx950): device code only.
//
// Included by spectra_decode.hip (compiled ahead of time with run-time slot widths) and embedded
// as source text for run-time compilation of kernels specialised to one layout's slot widths.
#pragma once

#include "spectra_device.h"

namespace spectra {

// ------------------------------------------------------------ matrix-core decode kernel

// (x & mask) | orv: the compiler selects one v_and_or_b32 for it.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t orv) {
    return (x & mask) | orv;                           // v_and_or_b32
}

// mg[o - 1]: the fp16 exponent pattern of 2^(10 - o) in both halves (o = 1..8), kept in vector
// registers.
__device__ __forceinline__ void magic_table(uint32_t (&mg)[8]) {
#pragma unroll
    for (int o = 1; o <= 8; ++o) {
        mg[o - 1] = (uint32_t)(25 - o) * 0x04000400u;
        asm volatile("" : "+v"(mg[o - 1]));
    }
}

// Pair i (0..15) of a run of B-bit codes held in B words, as two fp16 values u - (2^B-1)/2.
// The pair's codes sit at the same offset in the low and high 16 bits.  With the code at bit
// o >= 1 of each half, OR-ing the exponent of 2^(10-o) gives the fp16 numbers 2^(10-o) + u
// (bit o has weight 1 there; exact while o + B <= 10), from which 2^(10-o) + (2^B-1)/2
// (representable: the spacing there is 2^-o <= 1/2) is subtracted exactly.
//
// Shifts are shared: the pairs of a word that do not straddle into the next word are taken in
// order, and each shifted copy of the word (its first pair at bit 1) serves every following
// pair that still ends at or below bit 10 (B = 2: four pairs per shift, B = 3: three, B = 4:
// two; wider codes one).  A code that straddles two words is assembled at bit 1 from both.
// mg[o - 1] holds the exponent pattern of 2^(10-o) in both halves, (25 - o) * 0x04000400, in a
// vector register (v_and_or_b32 takes its mask from a scalar register, so the pattern must be
// in a vector one for the and-or to stay one instruction).
__host__ __device__ constexpr int run_anchor(int B, int I) {
    const int k = (I * B) >> 4;
    int a = -1;
    for (int J = 0; J <= I; ++J) {
        const int g = J * B;
        if ((g >> 4) != k || (g & 15) + B > 16) continue;   // another word's pair, or a straddle
        if (a < 0 || (g & 15) - a + 1 + B > 10) a = g & 15;
    }
    return a;
}
template <int B, int I>
__device__ __forceinline__ half2_t run_pair(const uint32_t (&w)[B], const uint32_t (&mg)[8]) {
    constexpr int gam = I * B, k = gam >> 4, off = gam & 15;
    constexpr uint32_t M = (1u << B) - 1u;
    constexpr bool whole = off + B <= 16;        // not straddling into word k + 1
    constexpr int a = whole ? run_anchor(B, I) : 0;
    constexpr int o = whole ? off - a + 1 : 1;   // bit of the code in each half
    uint32_t bits;
    if constexpr (whole) {
        static_assert(o >= 1 && o + B <= 10, "pair outside the exact range");
        uint32_t t;
        if constexpr (a >= 2) t = w[k] >> (a - 1);
        else if constexpr (a == 1) t = w[k];
        else t = w[k] << 1;
        bits = and_or(t, (M << o) | (M << (o + 16)), mg[o - 1]);
    } else {
        constexpr int lo = 16 - off;             // bits in word k
        constexpr uint32_t Ml = (1u << lo) - 1u, Mh = (1u << (B - lo)) - 1u;
        const uint32_t a = and_or(w[k] >> (off - 1), (Ml << 1) | (Ml << 17), mg[0]);
        bits = and_or(w[k + 1] << (lo + 1), (Mh << (lo + 1)) | (Mh << (lo + 17)), a);
    }
    half2_t x;
    __builtin_memcpy(&x, &bits, 4);
    const _Float16 cst = (_Float16)((float)(1 << (10 - o)) + 0.5f * (float)M);
    const half2_t off2 = {cst, cst};
    return x - off2;
}

template <int B>
__device__ __forceinline__ void unpack_run(const uint32_t (&w)[B], const uint32_t (&mg)[8], half2_t (&u)[16]) {
    u[0] = run_pair<B, 0>(w, mg);   u[1] = run_pair<B, 1>(w, mg);
    u[2] = run_pair<B, 2>(w, mg);   u[3] = run_pair<B, 3>(w, mg);
    u[4] = run_pair<B, 4>(w, mg);   u[5] = run_pair<B, 5>(w, mg);
    u[6] = run_pair<B, 6>(w, mg);   u[7] = run_pair<B, 7>(w, mg);
    u[8] = run_pair<B, 8>(w, mg);   u[9] = run_pair<B, 9>(w, mg);
    u[10] = run_pair<B, 10>(w, mg); u[11] = run_pair<B, 11>(w, mg);
    u[12] = run_pair<B, 12>(w, mg); u[13] = run_pair<B, 13>(w, mg);
    u[14] = run_pair<B, 14>(w, mg); u[15] = run_pair<B, 15>(w, mg);
}

// K group operands: this lane's 32 codes (w8, first B words valid) are coordinates 8H..8H+7
// of token pi(m) in each quarter T, sb[T] (low 16 bits) their fp16 scales.  a[T] = c^ = s (u - h)
// rounded once to fp16.  Score errors are amplified by the softmax (value errors enter
// linearly), so the leading, high-variance groups carry more precision on both sides: the query
// as q~ = hi + lo, and with LO the latent's residual al[T] = fp16(s (u - h) - a[T]) from one
// fused multiply-add: the product of the exact fp16 values u - h and s has at most 19
// significant bits, so the residual is exact whenever it lies in fp16's normal range (products
// of magnitude 2^-3 and up); below, fp16's subnormal spacing bounds its error by 2^-25.
//
// 1-bit groups: u - h = +-1/2, so c^ = +-fp16(s / 2) (round-to-nearest-even is symmetric, so this
// is the general path's product bit for bit).  The pair is built as the bit pattern of fp16(s / 2)
// with the sign bit set where the code is 0: the complemented code word, its bit moved to bit
// 15 / 31, through one v_and_or_b32 per pair.  The residual is zero (s / 2 differs from
// fp16(s / 2) by 0 or 2^-25, and fp16 rounds 2^-25 to 0), so al is zero and split slots of 1-bit
// groups skip the al q~ product.
template <int B, bool LO = false>
__device__ __forceinline__ void k_operands(const uint32_t (&w8)[8], const uint32_t (&sb)[4], const uint32_t (&mg)[8],
                                           half8_t (&a)[4], half8_t (&al)[4]) {
#pragma clang fp contract(off)
    if constexpr (B == 1) {
        const uint32_t w0 = ~w8[0];                      // sign bit = code 0
#pragma unroll
        for (int T = 0; T < 4; ++T) {
            const uint16_t s16 = (uint16_t)sb[T];
            _Float16 sc;
            __builtin_memcpy(&sc, &s16, 2);
            const half2_t h2 = half2_t{sc, sc} * half2_t{(_Float16)0.5f, (_Float16)0.5f};
            uint32_t hb;
            __builtin_memcpy(&hb, &h2, 4);
#pragma unroll
            for (int pr = 0; pr < 4; ++pr) {
                const int i = 4 * T + pr;                         // pair i: stream bit i of each half
                const uint32_t t = i < 15 ? w0 << (15 - i) : w0;
                const uint32_t bits = and_or(t, 0x80008000u, hb);
                half2_t x;
                __builtin_memcpy(&x, &bits, 4);
                a[T][2 * pr] = x[0];
                a[T][2 * pr + 1] = x[1];
                if constexpr (LO) {
                    al[T][2 * pr] = (_Float16)0.0f;
                    al[T][2 * pr + 1] = (_Float16)0.0f;
                }
            }
        }
        return;
    }
    uint32_t w[B];
#pragma unroll
    for (int i = 0; i < B; ++i) w[i] = w8[i];
    half2_t u[16];
    unpack_run<B>(w, mg, u);
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
            if constexpr (LO) {
                const half2_t l2 = __builtin_elementwise_fma(u[4 * T + pr], s2, -c2);
                al[T][2 * pr] = l2[0];
                al[T][2 * pr + 1] = l2[1];
            }
        }
    }
}

// V group operands: this lane's 32 codes are coordinate (lane & 15) of tokens 32T + 8q + e,
// vs[T] the eight tokens' fp16 scales.  a[T] = c^ rounded once to fp16.
// 1-bit groups: a[T] = +-s = 2 c^, the scale pair's bits with the sign of the complemented code
// (one v_and_or_b32 per pair, no multiply); the slot's accumulators are halved when the split
// ends.  The products p (+-s) are exact, so the float32 sums are exactly twice those of
// p (+-fp16(s / 2)) and halving them is exact: the same results bit for bit wherever s / 2 is
// an fp16 number (s >= 2^-13, or s's last significand bit zero), and the exact product below.
template <int B>
__device__ __forceinline__ void v_operands(const uint32_t (&w8)[8], const uint4 (&vs)[4], const uint32_t (&mg)[8],
                                           half8_t (&a)[4]) {
#pragma clang fp contract(off)
    if constexpr (B == 1) {
        const uint32_t w0 = ~w8[0];                      // sign bit = code 0
#pragma unroll
        for (int T = 0; T < 4; ++T) {
            const uint32_t sp[4] = {vs[T].x, vs[T].y, vs[T].z, vs[T].w};
#pragma unroll
            for (int pr = 0; pr < 4; ++pr) {
                const int i = 4 * T + pr;
                const uint32_t t = i < 15 ? w0 << (15 - i) : w0;
                const uint32_t bits = and_or(t, 0x80008000u, sp[pr]);   // scales are >= 0
                half2_t x;
                __builtin_memcpy(&x, &bits, 4);
                a[T][2 * pr] = x[0];
                a[T][2 * pr + 1] = x[1];
            }
        }
        return;
    }
    uint32_t w[B];
#pragma unroll
    for (int i = 0; i < B; ++i) w[i] = w8[i];
    half2_t u[16];
    unpack_run<B>(w, mg, u);
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
template <int WMASK, bool LO = false, int BW = 8>
__device__ __forceinline__ void k_operands_w(int bw, const uint32_t (&w8)[8], const uint32_t (&sb)[4],
                                             const uint32_t (&mg)[8], half8_t (&a)[4], half8_t (&al)[4]) {
    if constexpr (BW >= 1) {
        if constexpr (!((WMASK >> BW) & 1)) k_operands_w<WMASK, LO, BW - 1>(bw, w8, sb, mg, a, al);
        else if constexpr ((WMASK & ((1 << BW) - 1)) == 0) k_operands<BW, LO>(w8, sb, mg, a, al);
        else if (bw == BW) k_operands<BW, LO>(w8, sb, mg, a, al);
        else k_operands_w<WMASK, LO, BW - 1>(bw, w8, sb, mg, a, al);
    }
}
template <int WMASK, int BW = 8>
__device__ __forceinline__ void v_operands_w(int bw, const uint32_t (&w8)[8], const uint4 (&vs)[4],
                                             const uint32_t (&mg)[8], half8_t (&a)[4]) {
    if constexpr (BW >= 1) {
        if constexpr (!((WMASK >> BW) & 1)) v_operands_w<WMASK, BW - 1>(bw, w8, vs, mg, a);
        else if constexpr ((WMASK & ((1 << BW) - 1)) == 0) v_operands<BW>(w8, vs, mg, a);
        else if (bw == BW) v_operands<BW>(w8, vs, mg, a);
        else v_operands_w<WMASK, BW - 1>(bw, w8, vs, mg, a);
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
// One workgroup = one (split, sequence, group of up to 32 query heads: heads 32 z .. 32 z + 31 for
// grid row z), eight waves: waves 0-3 are key waves, 4-7 value
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

// Slot widths.  DynamicWidths reads them from the layout at run time (one kernel per width
// family, a branch per slot).  A specialised kernel passes a type with kStatic = true whose
// width(role, wave, slot) is a constant table: the slot loops then unroll into straight-line
// code with exactly b loads per slot and no width branches.
struct DynamicWidths {
    static constexpr bool kStatic = false;
    static constexpr bool kExactLoads = false;
    static constexpr int kSplitGroups = 0;
    static constexpr int width(int, int, int) { return 0; }
};

// Key groups whose scores take the split terms (c^ q~ = hi hi + hi lo + lo hi, three products);
// the others take hi hi alone (one product).  Groups are in energy order, so the score error of
// single fp16 terms comes mostly from the leading groups; but a heavy-tailed token (a large
// scale on every coordinate) carries it into the later groups too.  By default the leading three
// quarters of the groups (at least 4, at most all) are split: on the Llama-shaped workload with
// 1 % Student-t(3) rows this keeps every sequence's output within 1.2e-3 of float64 attention,
// where the leading quarter alone left 2.3e-3.  A token whose latent is about 100 times the
// others' can still move the output by up to 3e-3; spectra_set_key_split(1) splits every group
// (LayoutInfo::k_split, set per call by the host).
__host__ __device__ constexpr int split_query_groups(int n_chunks) {
    return (3 * n_chunks + 3) / 4 > 4 ? (3 * n_chunks + 3) / 4 : (n_chunks < 4 ? n_chunks : 4);
}
template <class WT, int ROLE, int W>
__device__ __forceinline__ int slot_width(const SlotGeom& g, int i) {
    if constexpr (WT::kStatic) return WT::width(ROLE, W, i);
    else return g.wd[i];
}
// Whether key slot i of wave w takes the split query.
template <class WT, int W>
__device__ __forceinline__ bool slot_split(int w, int i, int n_split) {
    if constexpr (WT::kStatic) return W + kRoleWaves * i < WT::kSplitGroups;
    else return w + kRoleWaves * i < n_split;
}

// This lane's run words of a slot (word k at chunk word 64 k + lane), HBM -> registers.  Every
// slot issues exactly eight loads, so that the number of loads in flight is a compile-time
// constant: the loads go through a buffer resource whose size is the chunk's 256 b bytes, and
// rows at or past the width (all rows of a slot without a group) fall outside it, which the
// hardware answers with zeros without touching memory.
// Word 3 of the buffer resource descriptor (CDNA3 / CDNA4 instruction set reference, buffer
// resource table): DATA_FORMAT (bits 18:15) = 4, 32-bit; every other field 0 (no swizzle, no
// thread-id add, no index stride; the destination selects and number format are not used by
// untyped loads).  With stride 0, NUM_RECORDS (word 2) is a byte count: an offset at or past it
// reads as zero without a memory access.
constexpr int kBufferWord3 = 0x00020000;
// With static widths (bw a constant) only the b words of the run are loaded.
template <bool STATIC>
__device__ __forceinline__ void ring_load(const uint8_t* __restrict__ chunk, int bw, int bytes_bw, int lane,
                                          uint32_t (&w8)[8]) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(chunk), (short)0, 256 * bytes_bw, kBufferWord3);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        if (!STATIC || k < bw) w8[k] = __builtin_amdgcn_raw_buffer_load_b32(r, lane * 4 + 256 * k, 0, 2);
        else w8[k] = 0;
    }
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
// With static widths the load counts differ per slot; the compiler's own waits are exact there
// (straight-line code), so no manual wait is issued.
template <int PER, int DMA, bool STATIC>
__device__ __forceinline__ void ring_wait() {
    if constexpr (!STATIC) waitcnt_vm<PER * (kSlots - 1) + DMA>();
}

// This lane's four K scales of a slot (entries 4m .. 4m+3 of the group's scale chunk); a
// resource of `bytes` = 0 returns zeros without a memory access.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2_t key_scales(const uint8_t* __restrict__ scale_chunk, int bytes, int m) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(scale_chunk), (short)0, bytes, kBufferWord3);
    return __builtin_amdgcn_raw_buffer_load_b64(r, 8 * m, 0, 2);
}

template <int WMASK, class WT, int W>
__device__ __forceinline__ void key_role(const LayoutInfo& li, int b, int h0, int w, int lane, int64_t t0, int64_t t1,
                                         const uint8_t* __restrict__ seq, const float* __restrict__ qt,
                                         unsigned char* smem, float* __restrict__ pm,
                                         float* __restrict__ pl, int64_t pbase) {
    const TensorInfo& TK = li.t[0];
    const int BK = TK.block_bytes;
    const SlotGeom g = slot_geom(TK, w, lane);
    const int n_split = li.k_split;
    half8_t* qlds = reinterpret_cast<half8_t*>(smem) + w * kSlots * 128;
    float* ex = reinterpret_cast<float*>(smem + kQLds + kVsLds);
    half8_t* plds = reinterpret_cast<half8_t*>(smem + kQLds + kVsLds + kExLds);
    float* tmax = reinterpret_cast<float*>(smem + kQLds + kVsLds + kExLds + kPLds);
    float* alph = tmax + 128;
    float* lred = alph + 64;

    constexpr bool kS = WT::kStatic && WT::kExactLoads;   // exact per-slot loads and waits
    // q~ operands of this wave's slots: lane (H, n) holds coordinates 8 H .. 8 H + 7 of chunk c for
    // head n, split into fp16 hi = fp16(v) and lo = fp16(v - hi) (q~ rows are 16 n_chunks long)
    const float* qb = qt + ((int64_t)b * li.n_q + h0 + (lane & 31)) * (16 * TK.n_chunks) + 8 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
        const int c = w + kRoleWaves * i;
        if (slot_width<WT, 0, W>(g, i)) {
            half8_t hi = {}, lo = {};
            if (h0 + (lane & 31) < li.n_q) {            // lanes of absent heads hold zeros
                const f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(qb + 16 * c);
                const f32x4_t v1 = *reinterpret_cast<const f32x4_t*>(qb + 16 * c + 4);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float v = e < 4 ? v0[e] : v1[e - 4];
                    hi[e] = (_Float16)v;
                    lo[e] = (_Float16)(v - (float)hi[e]);
                }
            }
            qlds[i * 128 + lane] = hi;
            qlds[i * 128 + 64 + lane] = lo;
        }
    }
    uint32_t mg[8];
    magic_table(mg);
    const int n = lane & 31, H = lane >> 5;
    float m_run = -__builtin_inff(), l_run = 0.0f;
    uint32_t cr[kSlots][8];
    u32x2_t sr[kSlots];

    const int blk0 = (int)(t0 / kBT), blk1 = (int)((t1 + kBT - 1) / kBT);
    const int t0i = (int)t0, t1i = (int)t1;
    __builtin_amdgcn_s_waitcnt(0);                     // q~ operands are in LDS
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
        const int bw = slot_width<WT, 0, W>(g, i);
        ring_load<kS>(seq + (int64_t)blk0 * BK + g.off[i], bw, bw, lane, cr[i]);
        if (!kS || bw) sr[i] = key_scales(seq + (int64_t)blk0 * BK + TK.codes_bytes + 256 * (w + kRoleWaves * i), bw ? 256 : 0, n);
        else sr[i] = u32x2_t{0, 0};
        __builtin_amdgcn_sched_barrier(0);             // keep the ring's slot order
    }

    for (int blk = blk0; blk < blk1; ++blk) {
        const int cur = (blk - blk0) & 1;
        const bool more = blk + 1 < blk1;
        const uint8_t* nb = seq + (int64_t)(blk + 1) * BK;
        f32x16_t S[4];
#pragma unroll
        for (int T = 0; T < 4; ++T) S[T] = f32x16_t{};
        // Software pipeline over the slots: slot i + 1's operands are unpacked while slot i's
        // products run (the wave's vector instructions issue between its own matrix
        // instructions instead of waiting behind a burst of them).
        half8_t an[4], anl[4] = {};
        {
            const int b0 = slot_width<WT, 0, W>(g, 0);
            if (b0) {
                ring_wait<kKeyOps, 0, kS>();
                const uint32_t ks[4] = {sr[0][0], sr[0][0] >> 16, sr[0][1], sr[0][1] >> 16};
                if (slot_split<WT, W>(w, 0, n_split)) k_operands_w<WMASK, true>(b0, cr[0], ks, mg, an, anl);
                else k_operands_w<WMASK>(b0, cr[0], ks, mg, an, anl);
            }
        }
#pragma unroll
        for (int i = 0; i < kSlots; ++i) {
            const int bw = slot_width<WT, 0, W>(g, i);
            half8_t a[4] = {an[0], an[1], an[2], an[3]};
            half8_t al[4] = {anl[0], anl[1], anl[2], anl[3]};
            const bool split = slot_split<WT, W>(w, i, n_split);
            half8_t qh = {}, ql = {};
            if (bw) {
                qh = qlds[i * 128 + lane];
                if (split) ql = qlds[i * 128 + 64 + lane];
            }
            if (i + 1 < kSlots) {
                const int bn = slot_width<WT, 0, W>(g, i + 1);
                if (bn) {
                    ring_wait<kKeyOps, 0, kS>();
                    const uint32_t ks[4] = {sr[i + 1][0], sr[i + 1][0] >> 16, sr[i + 1][1], sr[i + 1][1] >> 16};
                    if (slot_split<WT, W>(w, i + 1, n_split)) k_operands_w<WMASK, true>(bn, cr[i + 1], ks, mg, an, anl);
                    else k_operands_w<WMASK>(bn, cr[i + 1], ks, mg, an, anl);
                }
            }
            if (bw) {
#pragma unroll
                for (int T = 0; T < 4; ++T) S[T] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[T], qh, S[T], 0, 0, 0);
                if (split) {                               // c^ q~ = hi hi + hi lo + lo hi (lo lo dropped)
#pragma unroll
                    for (int T = 0; T < 4; ++T) S[T] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[T], ql, S[T], 0, 0, 0);
                    if (bw != 1) {                         // 1-bit groups: lo is zero
#pragma unroll
                        for (int T = 0; T < 4; ++T) S[T] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[T], qh, S[T], 0, 0, 0);
                    }
                }
            }
            // next block (nothing is read past the split: sizes 0 return zeros)
            ring_load<kS>(nb + g.off[i], bw, more ? bw : 0, lane, cr[i]);
            if (!kS || bw) sr[i] = key_scales(nb + TK.codes_bytes + 256 * (w + kRoleWaves * i), more && bw ? 256 : 0, n);
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
        float mx = -__builtin_inff();
        if (lo_t > 0 || hi_t < kBT) {                  // first or last block of the split only
#pragma unroll
            for (int a = 0; a < 16; ++a) {
                const int tok = 32 * w + 16 * H + a;
                if (tok < lo_t || tok >= hi_t) sv[a] = -__builtin_inff();
            }
        }
#pragma unroll
        for (int a = 0; a < 16; ++a) mx = fmaxf(mx, sv[a]);
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
    if (w == 0 && lane < 32 && h0 + lane < li.n_q) {
        float L = 0.0f;
        for (int v = 0; v < kRoleWaves; ++v) L += lred[v * 64 + lane] + lred[v * 64 + lane + 32];
        pm[pbase + h0 + lane] = m_run;
        pl[pbase + h0 + lane] = L;
    }
}

template <int WMASK, class WT, int W>
__device__ __forceinline__ void value_role(const LayoutInfo& li, int h0, int w, int lane, int64_t t0, int64_t t1,
                                           const uint8_t* __restrict__ seq, unsigned char* smem,
                                           float* __restrict__ pz, int RV, int64_t pbase) {
    const TensorInfo& TV = li.t[1];
    const int BV = TV.block_bytes;
    const SlotGeom g = slot_geom(TV, w, lane);
    unsigned char* sc = smem + kQLds + w * 2048;
    const half8_t* plds = reinterpret_cast<const half8_t*>(smem + kQLds + kVsLds + kExLds);
    const float* alph = reinterpret_cast<const float*>(smem + kQLds + kVsLds + kExLds + kPLds) + 128;

    uint32_t mg[8];
    magic_table(mg);
    f32x4_t Z[kSlots][2];
#pragma unroll
    for (int i = 0; i < kSlots; ++i) Z[i][0] = Z[i][1] = f32x4_t{0, 0, 0, 0};
    uint32_t cr[kSlots][8];
    const int q4 = lane >> 4;

    const int blk0 = (int)(t0 / kBT), blk1 = (int)((t1 + kBT - 1) / kBT);
    u32x4_t vsr[2];
    constexpr bool kS = WT::kStatic && WT::kExactLoads;
    value_scales(seq + (int64_t)blk0 * BV, BV, TV, w, g, lane, vsr);
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
        const int bw = slot_width<WT, 1, W>(g, i);
        ring_load<kS>(seq + (int64_t)blk0 * BV + g.off[i], bw, bw, lane, cr[i]);
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
        if constexpr (!kS) waitcnt_vm<kSlots * kValOps - 1>();
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
        if constexpr (kValueSlotsBeforeB == 0) {
            if (more) __syncthreads();                 // B of block blk+1
        }
        // software pipeline as in the key waves: slot i + 1 is unpacked under slot i's products
        half8_t an[4];
        {
            const int b0 = slot_width<WT, 1, W>(g, 0);
            if (b0) {
                uint4 vs[4];
#pragma unroll
                for (int T = 0; T < 4; ++T) vs[T] = *reinterpret_cast<const uint4*>(scb + 2 * (32 * T + 8 * q4));
                ring_wait<kValOps, kValDma, kS>();
                v_operands_w<WMASK>(b0, cr[0], vs, mg, an);
            }
        }
#pragma unroll
        for (int i = 0; i < kSlots; ++i) {
            const int bw = slot_width<WT, 1, W>(g, i);
            half8_t a[4] = {an[0], an[1], an[2], an[3]};
            if (i + 1 < kSlots) {
                const int bn = slot_width<WT, 1, W>(g, i + 1);
                if (bn) {
                    uint4 vs[4];
#pragma unroll
                    for (int T = 0; T < 4; ++T)
                        vs[T] = *reinterpret_cast<const uint4*>(scb + 256 * (i + 1) + 2 * (32 * T + 8 * q4));
                    ring_wait<kValOps, kValDma, kS>();
                    v_operands_w<WMASK>(bn, cr[i + 1], vs, mg, an);
                }
            }
            if (bw) {
#pragma unroll
                for (int T = 0; T < 4; ++T) {
                    Z[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[T], P[T][0], Z[i][0], 0, 0, 0);
                    Z[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[T], P[T][1], Z[i][1], 0, 0, 0);
                }
            }
            ring_load<kS>(nb + g.off[i], bw, more ? bw : 0, lane, cr[i]);   // next block (zeros past the split)
            __builtin_amdgcn_sched_barrier(0);
            // B of block blk+1: the key waves' short reduction runs while this wave works
            if (i == kValueSlotsBeforeB - 1 && more) __syncthreads();
        }
    }
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
        const int bw = slot_width<WT, 1, W>(g, i);
        if (!bw) continue;
        if ((WMASK & 2) && bw == 1) {                  // 1-bit slots accumulated 2 c^ (v_operands)
            Z[i][0] *= 0.5f;
            Z[i][1] *= 0.5f;
        }
        const int c = w + kRoleWaves * i;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int head = h0 + 16 * hh + (lane & 15);
            if (head >= li.n_q) continue;
            float* dst = pz + (pbase + head) * RV + 16 * c + 4 * (lane >> 4);
            *reinterpret_cast<f32x4_t*>(dst) = Z[i][hh];
        }
    }
}

// WMASK bit b set: code paths for width b are compiled in.  WT: slot widths (DynamicWidths, or a
// constant table of a specialised kernel).
template <int WMASK, class WT>
__device__ __forceinline__ void decode_mfma_body(
    LayoutInfo li, Positions ctx, const uint8_t* __restrict__ cache_k,
    const uint8_t* __restrict__ cache_v, int64_t seq_bytes_k, int64_t seq_bytes_v,
    const float* __restrict__ qt, float* __restrict__ pm, float* __restrict__ pl,
    float* __restrict__ pz, int RV, int split_tokens, int n_splits) {
    const int split = blockIdx.x, b = blockIdx.y, h0 = 32 * (int)blockIdx.z;   // head group
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t0 = (int64_t)split * split_tokens;
    const int64_t t1 = min((int64_t)ctx.v[b], t0 + split_tokens);
    if (t0 >= t1) return;
    extern __shared__ __align__(16) unsigned char smem[];
    const int64_t pbase = ((int64_t)b * n_splits + split) * li.n_q;
    const uint8_t* sk = cache_k + (int64_t)b * seq_bytes_k;
    const uint8_t* sv = cache_v + (int64_t)b * seq_bytes_v;
    if constexpr (!WT::kStatic) {
        if (wid < kRoleWaves) key_role<WMASK, WT, 0>(li, b, h0, wid, lane, t0, t1, sk, qt, smem, pm, pl, pbase);
        else value_role<WMASK, WT, 0>(li, h0, wid - kRoleWaves, lane, t0, t1, sv, smem, pz, RV, pbase);
    } else {
        switch (wid) {   // one straight-line body per wave (its own slot widths)
            case 0: key_role<WMASK, WT, 0>(li, b, h0, 0, lane, t0, t1, sk, qt, smem, pm, pl, pbase); break;
            case 1: key_role<WMASK, WT, 1>(li, b, h0, 1, lane, t0, t1, sk, qt, smem, pm, pl, pbase); break;
            case 2: key_role<WMASK, WT, 2>(li, b, h0, 2, lane, t0, t1, sk, qt, smem, pm, pl, pbase); break;
            case 3: key_role<WMASK, WT, 3>(li, b, h0, 3, lane, t0, t1, sk, qt, smem, pm, pl, pbase); break;
            case 4: value_role<WMASK, WT, 0>(li, h0, 0, lane, t0, t1, sv, smem, pz, RV, pbase); break;
            case 5: value_role<WMASK, WT, 1>(li, h0, 1, lane, t0, t1, sv, smem, pz, RV, pbase); break;
            case 6: value_role<WMASK, WT, 2>(li, h0, 2, lane, t0, t1, sv, smem, pz, RV, pbase); break;
            default: value_role<WMASK, WT, 3>(li, h0, 3, lane, t0, t1, sv, smem, pz, RV, pbase); break;
        }
    }
}

template <int WMASK>
__global__ __launch_bounds__(512, 1) void decode_mfma_kernel(
    LayoutInfo li, Positions ctx, const uint8_t* __restrict__ cache_k,
    const uint8_t* __restrict__ cache_v, int64_t seq_bytes_k, int64_t seq_bytes_v,
    const float* __restrict__ qt, float* __restrict__ pm, float* __restrict__ pl,
    float* __restrict__ pz, int RV, int split_tokens, int n_splits) {
    decode_mfma_body<WMASK, DynamicWidths>(li, ctx, cache_k, cache_v, seq_bytes_k, seq_bytes_v, qt, pm, pl, pz, RV,
                                           split_tokens, n_splits);
}

}  // namespace spectra
