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

// Position of (slot tau, coordinate j) in a group's code chunk.  For g == 16 the chunk is 64
// runs of 32 codes, one run per wave lane of the decode's matrix-core operands; otherwise
// token-major.
__device__ __forceinline__ int code_pos(int kind, int g, int tau, int j) {
    if (g != 16) return tau * g + j;
    const int T = tau >> 5, t = tau & 31;
    int L, e;
    if (kind == 0) {
        const int H = j >> 3;
        e = j & 7;
        const int m = 8 * ((t >> 2) & 3) + 4 * (t >> 4) + (t & 3);
        L = 32 * H + m;
    } else {
        const int q = t >> 3;
        e = t & 7;
        L = 16 * q + j;
    }
    return 32 * L + 8 * T + e;
}

// Inverse of code_pos: position p -> (tau, j).
__device__ __forceinline__ void code_pos_inv(int kind, int g, int p, int* tau, int* j) {
    if (g != 16) { *tau = p / g; *j = p - (p / g) * g; return; }
    const int L = p >> 5, eps = p & 31, T = eps >> 3, e = eps & 7;
    if (kind == 0) {
        const int H = L >> 5, m = L & 31;
        const int t = 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
        *tau = 32 * T + t;
        *j = 8 * H + e;
    } else {
        const int q = L >> 4;
        *tau = 32 * T + 8 * q + e;
        *j = L & 15;
    }
}

// Reads a `b`-bit field starting at bit `bit` of a chunk (b <= 8).  Reads at most the 32-bit
// word after the field's first word; a chunk is always followed by more block bytes.
__device__ __forceinline__ uint32_t read_field(const uint8_t* chunk, int64_t bit, int b) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(chunk);
    const int64_t wi = bit >> 5;
    const int off = (int)(bit & 31);
    uint32_t v = w[wi] >> off;
    if (off + b > 32) v |= w[wi + 1] << (32 - off);
    return v & ((1u << b) - 1u);
}

// Byte offset of chunk c's codes inside a block (device side).
__device__ __forceinline__ int64_t chunk_code_offset(const TensorInfo& t, int g, int c) {
    int64_t o = 0;
    for (int i = 0; i < c; ++i) o += 16LL * g * t.width[i];
    return o;
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t v) {
    _Float16 h;
    __builtin_memcpy(&h, &v, 2);
    return (float)h;
}

}  // namespace spectra
