/*
 * spectra.h - C ABI of the latent KV-cache codec (libspectra.so, MI355X / gfx950).
 *
 * The codec follows "SPECTRA: Pushing the KV Cache Beyond the 2-Bit Cliff via Spectral
 * Transform Coding" (technical summary, SPECTRA pipeline stages 1-3):
 *   - calibration (host): an activation-Gram-weighted SVD of W_K and W_V gives an
 *     energy-ordered latent (W_down, W_up); reverse water-filling gives per-group widths;
 *   - encode (GPU): tokens are down-projected, quantised per token in groups and appended
 *     to a packed latent cache;
 *   - decode (GPU): the packed cache is streamed, dequantised and used for softmax attention.
 *
 * Conventions for every call:
 *   - All matrices are row-major.  "dev" pointers are device memory on the current HIP device,
 *     "host" pointers are host memory.  The caller owns every buffer; the library allocates
 *     no device memory and keeps no state besides a thread-local error message.
 *   - GPU calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream) and
 *     return after enqueueing.  Buffers must stay valid until that work finishes.
 *   - Arguments visible on the host are checked before anything is enqueued; on error nothing
 *     is enqueued and no buffer is touched.  Kernel launch failures return SPECTRA_EHIP.
 *   - No call prints, aborts or throws.  spectra_last_error() describes the last failure on
 *     the calling thread.
 */
#ifndef SPECTRA_H
#define SPECTRA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SPECTRA_OK = 0,
    SPECTRA_EINVAL = 1,    /* null pointer, inconsistent shape, width outside 0..8, ... */
    SPECTRA_ENOTSUP = 2,   /* valid request with no kernel for it (see each call) */
    SPECTRA_ECAPACITY = 3, /* positions beyond the cache capacity, or workspace too small */
    SPECTRA_EHIP = 4,      /* a HIP runtime call or kernel launch failed */
    SPECTRA_ENUMERIC = 5   /* calibration: non-finite input or eigen-solver failure */
} spectra_status;

typedef enum {
    SPECTRA_F32 = 0,       /* x, w_down_t, q, w_up, w_o are float32 */
    SPECTRA_BF16 = 1       /* ... are bfloat16 */
} spectra_dtype;

enum { SPECTRA_TENSOR_K = 0, SPECTRA_TENSOR_V = 1 };

/* Tokens per cache block; capacities are rounded up to a multiple of it. */
#define SPECTRA_BLOCK_TOKENS 128
/* Largest batch one call accepts (positions travel as kernel arguments). */
#define SPECTRA_MAX_BATCH 256
/* Largest number of non-empty groups per tensor. */
#define SPECTRA_MAX_CHUNKS 256

/*
 * One layer's codec shape, fixed after calibration.
 * Latent segments: n_seg = 1 puts one latent over all key/value heads; n_seg = n_kv_heads
 * gives every key/value head its own latent (per-head rank as in the spectral-kv thread,
 * "Technical principle 1").  Each segment has seg_rank latent coordinates in groups of
 * group_size adjacent coordinates sharing one width ("SPECTRA pipeline", stage 2, grouping).
 * widths_k / widths_v: host [n_seg * seg_rank / group_size], values 0..8; a 0-width group is
 * dropped from W_down, W_up and the cache.  r_act (active latent columns of a tensor) is
 * group_size times the number of non-zero widths.
 * Query head h uses key/value head h / (n_q_heads / n_kv_heads).
 */
typedef struct {
    int32_t d_model, n_q_heads, n_kv_heads, d_head;
    int32_t n_seg, seg_rank, group_size;
    const uint8_t* widths_k;
    const uint8_t* widths_v;
} spectra_layout;

/* ---------------------------------------------------------------- calibration (host) ---- */

typedef struct {
    int32_t n_seg, seg_rank, group_size;
    double budget_bits;    /* bits per original element, 16-bit group scales included:
                              R = floor(budget_bits * n_kv_heads * d_head / n_seg) per token,
                              tensor and segment */
    int32_t fixed_width;   /* > 0: every group gets this width and budget_bits is ignored */
    double energy;         /* > 0: also report the smallest rank reaching this energy share */
    int32_t scale_bits;    /* bits charged per non-empty group (16 for fp16 scales) */
    int32_t max_width;     /* 1..8 */
    int32_t rank_rule;     /* spectra_rank_rule: which leading groups may receive bits */
    double gap_ratio;      /* SPECTRA_RANK_GAP: smallest eigenvalue ratio that counts as a gap (> 1) */
    /* Calibration rows (host [n_rows x d_model], row-major, float64; NULL when unused), for
       the two options below (see spectra_calibrate), each of which needs them. */
    const double* rows;
    int64_t n_rows;
    int32_t robust;            /* != 0: outlier-robust eigen-pairs from the rows; G not read (may be NULL) */
    int32_t value_correction;  /* != 0: least-squares value-latent correction folded into W_up_V */
} spectra_calib_params;

/* Rank rules: the kept rank r_cap (at most seg_rank) is rounded up to whole groups; groups past it
 * get width 0 and the budget (or the fixed width) goes to the groups before it.
 *   SPECTRA_RANK_FIXED  r_cap = seg_rank.
 *   SPECTRA_RANK_ENERGY r_cap = the energy rank: the smallest r whose leading eigenvalues hold the
 *                       share `energy` of the segment's total (spectral-kv forum thread, Technical
 *                       principle 1: effective rank per head at a target energy such as 95 %);
 *                       requires 0 < energy <= 1.
 *   SPECTRA_RANK_GAP    r_cap = i for the largest ratio lambda_i / lambda_{i+1} over 1 <= i < seg_rank
 *                       (first on ties) when it reaches gap_ratio, else seg_rank.  This library's
 *                       reading of the ablation study's spectral-gap criterion for trimming the
 *                       estimated dimension ("Ablation, Statistical Inference, and Validation for
 *                       KV-Cache Compression", Core contributions 3); eigenvalues <= 0 count as
 *                       1e-300.  Requires gap_ratio > 1. */
typedef enum { SPECTRA_RANK_FIXED = 0, SPECTRA_RANK_ENERGY = 1, SPECTRA_RANK_GAP = 2 } spectra_rank_rule;

/* Host output arrays, all caller-allocated with the maximal sizes given
 * (R = n_seg * seg_rank, seg_cols = n_kv_heads * d_head / n_seg).  Only the first r_act rows
 * of w_down_t / w_up are written.  Nullable members are skipped when NULL. */
typedef struct {
    double* w_down_t_k;      /* [R x d_model]: row i = weights of active latent column i */
    double* w_down_t_v;
    double* w_up_k;          /* [R x seg_cols]: row i = reconstruction row of column i */
    double* w_up_v;
    uint8_t* widths_k;       /* [n_seg * seg_rank / group_size] */
    uint8_t* widths_v;
    double* sigma2_k;        /* [n_seg * seg_rank] eigenvalues, descending per segment */
    double* sigma2_v;
    double* theta_k;         /* [n_seg] water level per segment (nullable; NaN if fixed) */
    double* theta_v;
    int32_t* energy_rank_k;  /* [n_seg] (nullable; -1 unless params.energy > 0) */
    int32_t* energy_rank_v;
    int32_t r_act_k, r_act_v; /* written by the call */
} spectra_calib_out;

/*
 * spectra_calibrate - G-weighted SVD and water-filled widths, float64, synchronous.
 * "SPECTRA pipeline" stage 1 (transform weighted by G = E[h^T h], "Methodology", third
 * observation) and stage 2 (reverse water-filling over the latent coordinates' marginal
 * variances; adjacent coordinates grouped; zero-bit groups dropped).
 * For each tensor W in {W_K, W_V} and segment s: M = W_s^T G W_s, eigenvectors V in
 * descending eigenvalue order (largest-magnitude entry of each made positive),
 * V_r = first seg_rank columns, sigma^2 = their eigenvalues, group variance = mean of its
 * sigma^2, widths b_k = clamp(floor(1/2 log2(v_k/theta) + 1/2), 0, max_width) at the lowest
 * breakpoint theta = v_k 4^-(j-1/2) whose cost sum_{b_k>0}(g b_k + scale_bits) fits R.
 * W_down_s = W_s V_r[:, active], W_up_s = V_r[:, active]^T.
 *   G:   host [d_model x d_model] (symmetric positive semi-definite)
 *   W_K, W_V: host [d_model x n_kv_heads*d_head]
 * The rank rule (params.rank_rule, see spectra_rank_rule) limits the groups that take part.
 * Outlier-robust variant (params.robust != 0, rows given), for heavy-tailed calibration rows, whose
 * sample second moment the ablation study ("Ablation, Statistical Inference, and Validation
 * for KV-Cache Compression", performance in specific regimes) finds corrupted by outliers:
 * with Y = rows W_s (the segment's projected rows), the directions are the eigenvectors of the
 * spatial-sign second moment S = mean of y y^T / |y|^2 over the rows with y != 0 (a row's scale
 * drops out), and the variance along each direction u is the median over all rows of (y . u)^2
 * divided by 0.45493642311957 (the median of chi-squared with one degree of freedom, so that
 * Gaussian rows give their variance).  Directions are then ordered by these variances,
 * descending, and take the place of M's eigen-pairs in everything above; sigma^2 reports the
 * variances.  A common per-row scale mixture (Student-t rows) multiplies every variance by one
 * factor, which leaves widths and rank rules unchanged.
 * Value-latent correction (params.value_correction != 0, rows given): stage 1 of the pipeline
 * folds a closed-form correction of W_O into the weights but gives no formula.  Here, per
 * segment of V, the calibration rows' exact latents C = rows W_down_s and their dequantised
 * values C^ (C rounded to float32, quantised and dequantised as the encoder does with the
 * calibrated widths) give the least-squares map F = (C^T C^)^-1 C^T C, and W_up_s becomes
 * F W_up_s, so that a cached token's value is rebuilt as c^ F W_up.  With one segment per key/
 * value head this is a correction of the output projection's input; with a joint latent it
 * cannot be written on the head outputs, so it is folded into W_up_V.  Only W_up_V changes.
 * Errors: EINVAL (shapes, group_size not dividing seg_rank, seg_rank > segment width, unknown
 * rank rule, energy outside (0, 1] for SPECTRA_RANK_ENERGY, gap_ratio <= 1 for SPECTRA_RANK_GAP,
 * robust or value_correction without rows, rows given with n_rows < 1, G NULL without robust),
 * ENUMERIC (non-finite input, eigen-solver did not converge, dequantised latents of rank below
 * the active columns for the value correction).
 * Uses OpenMP threads.
 */
spectra_status spectra_calibrate(const double* G, const double* W_K, const double* W_V,
                                 int32_t d_model, int32_t n_kv_heads, int32_t d_head,
                                 const spectra_calib_params* params, spectra_calib_out* out);

/* ------------------------------------------------------------------------- sizes ---- */

/* Bytes of one tensor's cache (tensor = SPECTRA_TENSOR_K or _V) for `batch` sequences of
 * capacity cap_tokens (rounded up to whole 128-token blocks).  The buffer must be zero-filled
 * before the first append: the encoder ORs codes into words it shares with other tokens. */
spectra_status spectra_cache_bytes(const spectra_layout* layout, int32_t tensor, int32_t batch,
                                   int64_t cap_tokens, size_t* bytes);

/* Bytes of one 128-token block of a tensor's cache. */
spectra_status spectra_block_bytes(const spectra_layout* layout, int32_t tensor, size_t* bytes);

/* Workspace bytes spectra_decode_attn needs for `batch` sequences of at most max_ctx tokens.
 * The figure covers every context from 0 to max_ctx (a shorter context can be cut into more,
 * shorter splits), so one workspace sized at a cache's capacity serves every call on it. */
spectra_status spectra_decode_workspace_bytes(const spectra_layout* layout, int32_t batch,
                                              int64_t max_ctx, size_t* bytes);

/* -------------------------------------------------------------------------- encode ---- */

/*
 * spectra_encode_append - down-project, quantise per token and append ("SPECTRA pipeline",
 * stage 3: tokens are down-projected, quantised per token and appended to the latent cache).
 *   x:          dev [batch x n_new x d_model] (dtype); row (b, i) is token i of sequence b
 *   w_down_t:   dev [(r_act_k + r_act_v) x d_model] (dtype): K's active columns, then V's
 *   cache_k/v:  dev, spectra_cache_bytes(...) bytes for (batch, cap_tokens), zero-filled
 *   start_pos:  host [batch]; token i of sequence b goes to position start_pos[b] + i
 *   latent_out: dev [batch x n_new x (r_act_k + r_act_v)] float32, or NULL: the float32 latent
 *               the codes were computed from (test hook)
 * For every token and group: A = max|c_j|, s = fp16(A 2^(1-b)) (65504 on overflow),
 * u_j = clamp(rint_even(c_j / s + (2^b-1)/2), 0, 2^b-1) in float32 (u = 0 when s = 0).
 * Positions being written must hold no earlier codes (the words are ORed).
 * Errors: EINVAL, ECAPACITY (start_pos[b] + n_new > cap_tokens, or negative),
 * ENOTSUP (batch > SPECTRA_MAX_BATCH, d_model not a multiple of 32, too many groups), EHIP.
 */
spectra_status spectra_encode_append(const spectra_layout* layout, spectra_dtype dtype,
                                     const void* x, int32_t batch, int32_t n_new,
                                     const void* w_down_t, void* cache_k, void* cache_v,
                                     int64_t cap_tokens, const int32_t* start_pos,
                                     float* latent_out, void* stream);

/* -------------------------------------------------------------------------- decode ---- */

/*
 * spectra_decode_attn - attention of one query token per sequence over its packed cache.
 * "SPECTRA pipeline" stage 3: keys and values are rebuilt from the latent for standard
 * attention.  The result equals softmax(scale * K^ q) V^ per query head with
 * K^ = C^_K W_up_K and V^ = C^_V W_up_V on the first ctx_len[b] cached tokens; it is computed
 * in latent space (the query is absorbed into W_up_K, values are accumulated in the latent
 * and lifted by W_up_V once), which the "Significance" section names as the route that also
 * saves compute.
 *   q:        dev [batch x n_q_heads x d_head] (dtype)
 *   cache_k/v: dev caches of capacity cap_tokens
 *   ctx_len:  host [batch], 0 <= ctx_len[b] <= cap_tokens (0 gives a zero output row)
 *   w_up_k/v: dev [r_act x seg_cols] (dtype), segment rows in order
 *   w_o:      dev [(n_q_heads*d_head) x d_model] (dtype) or NULL; if given the output is
 *             y = concat_h(o_h) w_o (a corrected W_O folded into the weights)
 *   out:      dev float32 [batch x n_q_heads x d_head], or [batch x d_model] with w_o
 *   workspace: dev, at least spectra_decode_workspace_bytes(layout, batch, max ctx_len)
 * Error: within 2e-3 max relative error of float64 attention on the same cache.  Products on
 * the matrix cores take fp16 operands with float32 accumulation.  Scores: in the leading three
 * quarters of the key groups (energy order; at least four groups) both the dequantised latent
 * and the absorbed query are carried as two fp16 terms (hi + lo) and three products are summed
 * (hi hi + hi lo + lo hi); the remaining groups take one product of single fp16 terms.  Values:
 * dequantised latents and softmax weights as single fp16 terms.  Measured worst case about
 * 1.1e-3, on heavy-tailed (Student-t) rows through a calibrated transform, where large per-token
 * scales carry the rounding into every group; below 6e-4 on Gaussian rows, peaked attention
 * included; below 1e-3 with zero rows, subnormal scales and a token 30 times the others.  A
 * token 100 times the others reached 3.1e-3: spectra_set_key_split(1) splits every key group
 * (5.2e-4 there).  Requires |dequantised latent| < 65504.
 * Kernels by layout: group size 16 with one segment (a joint latent), 1-32 active groups per
 * tensor and up to 256 query heads: the matrix-core stream kernel (heads in groups of 32, each
 * group streaming the cache once); group sizes 2, 4, 8 with narrow segments (up to 8 query
 * heads and rank 8, or 2 heads and rank 16, per segment): the small-rank kernels (float32; the
 * whole call in one launch when a sequence takes at most 8 splits, else one wave per split with
 * separate absorption and merge launches; SPECTRA_SMALL_FUSED=0 in the environment forces the
 * latter); otherwise the float32 generic kernel (at most 16 query heads and rank 64 per segment).
 * Errors: EINVAL, ECAPACITY (ctx_len > cap_tokens, workspace too small), ENOTSUP
 * (batch > SPECTRA_MAX_BATCH or a shape no kernel covers), EHIP.
 */
spectra_status spectra_decode_attn(const spectra_layout* layout, spectra_dtype dtype,
                                   const void* q, const void* cache_k, const void* cache_v,
                                   int64_t cap_tokens, int32_t batch, const int32_t* ctx_len,
                                   const void* w_up_k, const void* w_up_v, float softmax_scale,
                                   const void* w_o, float* out, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Bytes of the scratch array spectra_decode_attn_noalloc draws its workspace from (per device). */
#define SPECTRA_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * spectra_decode_attn_noalloc - spectra_decode_attn for callers that cannot allocate memory:
 * code under HIP graph capture, tight serving loops, and harnesses that forbid allocation.
 * Same arguments, result and errors as spectra_decode_attn, without the workspace: the library
 * keeps one scratch array of SPECTRA_NOALLOC_SCRATCH_BYTES bytes per device (held until the
 * process ends) and the call allocates nothing (no hipMalloc or hipFree, no run-time kernel
 * compilation: a layout runs its specialised kernel only if an earlier spectra_decode_attn call
 * compiled one, else the width-generic kernel, with the same results).  A call whose workspace
 * (spectra_decode_workspace_bytes for its batch and longest context) exceeds the scratch returns
 * SPECTRA_ECAPACITY before anything is enqueued.  Every call on one device shares that device's
 * scratch, which keeps the last call's contents: calls that overlap on one device (concurrent
 * streams, or host threads) race and must be serialised by the caller.
 */
spectra_status spectra_decode_attn_noalloc(const spectra_layout* layout, spectra_dtype dtype,
                                           const void* q, const void* cache_k, const void* cache_v,
                                           int64_t cap_tokens, int32_t batch, const int32_t* ctx_len,
                                           const void* w_up_k, const void* w_up_v, float softmax_scale,
                                           const void* w_o, float* out, void* stream);

/*
 * spectra_decode_attn_literal - the same attention as spectra_decode_attn, computed in the
 * order the "SPECTRA pipeline" states for stage 3: keys and values are first rebuilt for every
 * cached token, K^ = C^_K W_up_K and V^ = C^_V W_up_V (float32, in the workspace), then each
 * query head attends over them (split-K online softmax, float32).  It exists to measure what
 * computing in latent space saves (the "Significance" section's point): rebuilding costs
 * 2 r_act n_kv d_head multiply-adds per token and tensor where the latent-space path needs
 * r_act n_q.  Arguments as for spectra_decode_attn, without w_o; out: dev float32
 * [batch x n_q_heads x d_head].
 *   workspace: dev, at least spectra_decode_literal_workspace_bytes(layout, batch, max ctx_len)
 *              (about 8 n_kv d_head bytes per token of the longest context and sequence).
 * Error: within 2e-3 max relative error of float64 attention on the same cache (latents
 * rounded once to fp16, W_up as two fp16 terms, float32 accumulation).
 * Errors: EINVAL, ECAPACITY (ctx_len > cap_tokens, workspace too small), ENOTSUP (batch >
 * SPECTRA_MAX_BATCH, more than 8 query heads per key/value head, d_head > 256, a segment
 * width not a multiple of 32 or a segment rank above 512), EHIP.
 */
spectra_status spectra_decode_literal_workspace_bytes(const spectra_layout* layout, int32_t batch,
                                                      int64_t max_ctx, size_t* bytes);
spectra_status spectra_decode_attn_literal(const spectra_layout* layout, spectra_dtype dtype,
                                           const void* q, const void* cache_k, const void* cache_v,
                                           int64_t cap_tokens, int32_t batch, const int32_t* ctx_len,
                                           const void* w_up_k, const void* w_up_v, float softmax_scale,
                                           float* out, void* workspace, size_t workspace_bytes,
                                           void* stream);

/*
 * spectra_set_jit - run-time specialisation of the decode stream kernel.  With it on (the
 * default; the environment variable SPECTRA_JIT=0 turns it off at start-up), the first
 * spectra_decode_attn call for a layout whose group widths have not been seen on the current
 * device compiles (hiprtc, a few seconds) a kernel with those widths as constants and caches it
 * for the life of the process; later calls reuse it.  Results are bit-identical to the
 * width-generic kernel compiled into the library, which runs when it is off.  Layouts the
 * matrix-core kernel does not cover are not affected.  mode: 1 on, 0 off, any other value
 * only queries.  Returns the previous setting (1 or 0).  A layout whose specialised kernel
 * cannot be compiled or loaded runs the width-generic kernel (the failure is remembered for the
 * process, and no error is reported).  Not thread-safe with respect to concurrent decode calls
 * that change it.
 */
int spectra_set_jit(int mode);

/*
 * spectra_set_key_split - precision of the decode's key scores on the matrix-core path.  The
 * absorbed query and the dequantised key latent are fp16 operands; in the "split" key groups
 * each is carried as two fp16 terms (hi + lo) and a score tile takes three products (hi hi +
 * hi lo + lo hi) with float32 accumulation ("SPECTRA: Pushing the KV Cache Beyond the 2-Bit
 * Cliff via Spectral Transform Coding", pipeline stage 3, the attention read out of the
 * compressed cache).  mode 0 (the default): the leading three quarters of the key groups in
 * energy order (at least 4) are split, which keeps the synthetic workloads, heavy-tailed rows
 * included, within 1.2e-3 of float64 attention.  mode 1: every key group is split; for caches
 * holding tokens whose latent is far beyond the calibration's scale (a token 100 times the
 * others moved the default's output by up to 3e-3), at about 6 % more decode time on the
 * Llama-shaped workload.  Any other value only queries.  Returns the previous mode.  Process-
 * wide; takes effect on the next spectra_decode_attn call (the specialised kernel is cached per
 * layout and mode).  Layouts outside the matrix-core kernel (float32 vector-ALU kernels) are
 * not affected.
 */
int spectra_set_key_split(int mode);

/* spectra_jit_kernel_count - specialised decode kernels compiled and loaded so far in this process. */
int spectra_jit_kernel_count(void);

/* ----------------------------------------------------------------------- test hooks ---- */

/*
 * spectra_unpack_dequant - dequantised latent rows read back from a packed cache:
 * out[b, i, :] = c^ of position pos0 + i of sequence b, active columns in order, float32
 * (c^ = s (u - (2^b-1)/2), exact).  out: dev [batch x n_tok x r_act(tensor)].
 * Errors: EINVAL, ECAPACITY (pos0 + n_tok > cap_tokens), EHIP.
 */
spectra_status spectra_unpack_dequant(const spectra_layout* layout, int32_t tensor,
                                      const void* cache, int64_t cap_tokens, int32_t batch,
                                      int64_t pos0, int64_t n_tok, float* out, void* stream);

/*
 * spectra_set_timing_events - if both are non-NULL, the next spectra_decode_attn call on this
 * thread launches its streaming kernel with hipEvent `before` and `after` attached to the
 * dispatch (hipExtLaunchKernel / hipExtModuleLaunchKernel), so that they carry the kernel's own
 * start and end times (for the one-launch small-rank kernel: the whole call's work); the setting
 * is then cleared.  Both must be created hipEvents with timing.
 * For measurement only.
 */
void spectra_set_timing_events(void* before, void* after);

/* Message describing the last error on the calling thread ("" if none). */
const char* spectra_last_error(void);

/* Library version string. */
const char* spectra_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPECTRA_H */
