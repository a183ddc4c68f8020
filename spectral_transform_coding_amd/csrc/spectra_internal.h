// Internal declarations shared by the host code and the HIP launchers of libspectra.
#pragma once

#include <cstdint>
#include <cstddef>

#include "../../include/spectra.h"

namespace spectra {

constexpr int kBT = SPECTRA_BLOCK_TOKENS;   // tokens per cache block
constexpr int kMaxB = SPECTRA_MAX_BATCH;
constexpr int kMaxC = SPECTRA_MAX_CHUNKS;
constexpr int kMaxSeg = 64;

// Per tensor (K or V): the non-empty groups ("chunks") in storage order.
struct TensorInfo {
    int32_t n_chunks;
    int32_t r_act;          // active latent columns = g * n_chunks
    int32_t block_bytes;    // one 128-token block
    int32_t codes_bytes;    // code chunks of a block; scale chunks follow
    int32_t seg_chunk0[kMaxSeg + 1];  // first chunk of each segment (prefix)
    uint8_t width[kMaxC];   // width of each chunk
    uint8_t seg[kMaxC];     // segment of each chunk
};
static_assert(__builtin_offsetof(TensorInfo, width) % 4 == 0 && kMaxC % 4 == 0,
              "width[] is read as 32-bit words");

// Everything a kernel needs to know about a layer's cache; passed by value as a kernel
// argument (plain data, no pointers).
struct LayoutInfo {
    int32_t d_model, n_q, n_kv, d_head;
    int32_t n_seg, seg_rank, g, n_groups;
    int32_t seg_cols, kv_per_seg, q_per_kv;
    int32_t k_split;        // decode: leading key groups with the two-term products (set per call)
    TensorInfo t[2];
};

struct Positions {           // per-sequence integers passed as a kernel argument
    int32_t v[kMaxB];
};

// Validates a public layout and derives LayoutInfo.  Sets the error message on failure.
spectra_status make_layout(const spectra_layout* L, LayoutInfo* out);

// Records a printf-style message for spectra_last_error() and returns `st`.
spectra_status fail(spectra_status st, const char* fmt, ...);
void clear_error();

// Byte offset of chunk c's codes inside a block.
inline int64_t code_offset(const TensorInfo& t, int g, int c) {
    int64_t o = 0;
    for (int i = 0; i < c; ++i) o += 16LL * g * t.width[i];
    return o;
}

// Raises `kernel`'s dynamic LDS limit to at least `bytes` on the current device (the attribute
// is per device; each (device, kernel) is set once, under a lock).  False if the runtime refuses.
bool reserve_lds(const void* kernel, int bytes);

// Timing hook (spectra_set_timing_events): returns and clears the pending events.
void take_timing_events(void** before, void** after);

}  // namespace spectra
