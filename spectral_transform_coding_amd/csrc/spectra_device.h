// Device helpers shared by the encode and decode kernels of libspectra (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "spectra_internal.h"

namespace spectra {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
    return __uint_as_float(((uint32_t)v) << 16);
}

template <typename DT> __device__ __forceinline__ float load_f32(const DT* p, int64_t i);
template <> __device__ __forceinline__ float load_f32<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_f32<uint16_t>(const uint16_t* p, int64_t i) {
    return bf16_to_f32(p[i]);
}

// Code positions inside a group's code chunk (see the cache layout in include/spectra.h):
//   g != 16: code (tau, j) occupies chunk bits [(tau g + j) b, +b) (token-major bit stream);
//   g == 16: the chunk holds 64 runs L of b 32-bit words, word-major: word w of run L is
//     chunk word 64 w + L.  Run L holds, for each 32-token quarter T, 8 codes e = 0..7:
//     K -> coordinates 8H + e of token 32T + pi(m) (L = 32H + m), V -> coordinate j of token
//     32T + 8q + e (L = 16q + j).  Codes e and e + 1 form pair i = 4T + e/2; even e lives in
//     the low 16 bits of the run's words, odd e in the high 16 bits, at stream bits
//     [i b, i b + b) (stream bit gamma: run word gamma/16, bit gamma%16).

// pi(m): token of matrix-core row m inside a 32-token quarter (rows 8i + 4H + j of a 32x32
// accumulator hold tokens 16H + 4i + j).
__device__ __forceinline__ int quarter_token(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }
__device__ __forceinline__ int quarter_row(int t) { return 8 * ((t >> 2) & 3) + 4 * (t >> 4) + (t & 3); }

// Entry of a scale chunk that holds the scale of slot tau: slot order, except K with g == 16,
// where entry 4 pi^-1(t) + T holds slot 32 T + t (a K run's four scales are adjacent).
__device__ __forceinline__ int scale_index(int kind, int g, int tau) {
    return (g == 16 && kind == 0) ? 4 * quarter_row(tau & 31) + (tau >> 5) : tau;
}

// Run, quarter and e of (slot tau, coordinate j) for g == 16.
__device__ __forceinline__ void run_of(int kind, int tau, int j, int* L, int* T, int* e) {
    const int t = tau & 31;
    *T = tau >> 5;
    if (kind == 0) {
        *L = 32 * (j >> 3) + quarter_row(t);
        *e = j & 7;
    } else {
        *L = 16 * (t >> 3) + j;
        *e = t & 7;
    }
}

// (slot, coordinate) of run L, quarter T, code e for g == 16.
__device__ __forceinline__ void run_inv(int kind, int L, int T, int e, int* tau, int* j) {
    if (kind == 0) {
        *tau = 32 * T + quarter_token(L & 31);
        *j = 8 * (L >> 5) + e;
    } else {
        *tau = 32 * T + 8 * (L >> 4) + e;
        *j = L & 15;
    }
}

// Reads the b-bit code of (slot tau, coordinate j) from a code chunk (only words of the
// chunk itself).
__device__ __forceinline__ uint32_t read_code(int kind, int g, int b, const uint8_t* chunk, int tau, int j) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(chunk);
    const uint32_t mask = (1u << b) - 1u;
    if (g != 16) {
        const int64_t bit = (int64_t)(tau * g + j) * b;
        const int64_t wi = bit >> 5;
        const int off = (int)(bit & 31);
        uint32_t v = w[wi] >> off;
        if (off + b > 32) v |= w[wi + 1] << (32 - off);
        return v & mask;
    }
    int L, T, e;
    run_of(kind, tau, j, &L, &T, &e);
    const int gam = (4 * T + (e >> 1)) * b;
    const int wi = 64 * (gam >> 4) + L, off = gam & 15, sh = 16 * (e & 1);
    uint32_t v = ((w[wi] >> sh) & 0xFFFFu) >> off;     // this stream's half-word only
    if (off + b > 16) v |= ((w[wi + 64] >> sh) & 0xFFFFu) << (16 - off);
    return v & mask;
}

// Byte offset of chunk c's codes inside a block (device side): 16 g times the sum of the
// widths before it.  The widths are summed four per 32-bit word (one v_sad_u8 each) with the
// word loads unrolled, so that they are in flight together: a loop of dependent byte loads
// from the kernel arguments cost about 0.25 us per chunk.
__device__ __forceinline__ int64_t chunk_code_offset(const TensorInfo& t, int g, int c) {
    const uint32_t* w4 = reinterpret_cast<const uint32_t*>(t.width);   // width[] is 4-byte aligned
    uint32_t sum = 0;
    const int nw = c >> 2;
#pragma unroll 8
    for (int i = 0; i < nw; ++i) sum = __builtin_amdgcn_sad_u8(w4[i], 0u, sum);
    for (int i = 4 * nw; i < c; ++i) sum += t.width[i];
    return 16LL * g * (int64_t)sum;
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t v) {
    _Float16 h;
    __builtin_memcpy(&h, &v, 2);
    return (float)h;
}

// Dequantised latent coordinate (chunk c, coordinate j) of slot tau of a block.
__device__ __forceinline__ float dequant_at(const TensorInfo& ti, int kind, int g, const uint8_t* blk,
                                            int c, int64_t code_off, int tau, int j) {
    const int bw = ti.width[c];
    const uint32_t u = read_code(kind, g, bw, blk + code_off, tau, j);
    const uint16_t sb = reinterpret_cast<const uint16_t*>(blk + ti.codes_bytes + 256 * c)[scale_index(kind, g, tau)];
    const float s = f16_bits_to_f32(sb);
    return s * ((float)u - 0.5f * (float)((1u << bw) - 1u));
}

}  // namespace spectra
