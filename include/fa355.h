/*
 * fa355.h -- C ABI of libfa355: fused tiled scaled-dot-product attention for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (defined on the pages cited per entry point):
 *   S = scale * Q K^T, masked, P = softmax(S) row by row, O = P V,
 *   L = per-row natural-log logsumexp of the visible entries of S.
 * The N x N matrices S and P are never stored.
 *
 * Mask: key j is visible to query i iff
 *   (causal == 0 || j <= i) && (window < 0 || j >= i - window).
 * A window of W therefore admits W + 1 keys including the query's own
 * position; window = -1 disables it.  A query row with no visible key gets
 * O = 0 and L = -inf.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers (memory of the current HIP
 *    device); sizes are element counts.  Tensors are dense and row-major
 *    ("contiguous") in the layouts stated per call.
 *  - dtype FA_BF16: q/k/v/o/dO (and the caches) are bfloat16; FA_FP16:
 *    IEEE half precision; FA_FP32: float32.  lse, dq, dk, dv and all
 *    statistics are float32 in every case.  The 16-bit types run the same
 *    matrix-core kernels (fp16 inputs with an fp32 accumulator are the
 *    mixed-precision upgrade listed in "Build a FlashAttention Tiled
 *    Self-Attention Block from Scratch in Pure NumPy", Extending It).
 *  - Ownership: the caller owns every buffer, including workspaces.  The
 *    library never allocates, frees or synchronises; every call is
 *    asynchronous on `stream` (a hipStream_t, NULL = the default stream).
 *    Inputs are read only; outputs are fully overwritten; outputs must not
 *    alias inputs or each other.
 *  - Errors: a status is returned, nothing is thrown across the ABI.  Every
 *    argument check happens before any HIP call, so an error status other
 *    than FA_ERR_HIP means nothing was launched.  fa_last_error() returns a
 *    thread-local text describing the most recent failure on this thread.
 *  - scale is used as given (0 is legal and gives uniform weights); it must
 *    be finite.
 */
#ifndef FA355_H
#define FA355_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* null required pointer, dim <= 0, window < -1,
                             non-finite scale, bad block size, ...        */
  FA_ERR_UNSUPPORTED = 2, /* valid arguments with no kernel (dtype x d)    */
  FA_ERR_WORKSPACE = 3,   /* workspace pointer null or too small           */
  FA_ERR_HIP = 4          /* the HIP launch itself failed                  */
} fa_status;

typedef enum fa_dtype { FA_FP32 = 0, FA_BF16 = 1, FA_FP16 = 2 } fa_dtype;

/* Library version (major * 10000 + minor * 100 + patch). */
int fa_version(void);

/* Short constant text for a status code. */
const char* fa_status_str(fa_status status);

/* Thread-local description of the last failure ("" after a success). */
const char* fa_last_error(void);

/*
 * fa_fwd -- tiled forward pass with online softmax.
 *
 * Defined by "Building Flash Attention from Scratch in Pure NumPy",
 * Architecture Overview and Steps 2-3 (for each query tile walk the K/V
 * tiles keeping a running max m, a running sum l and an unnormalised O,
 * rescaled by exp(m_old - m_new); divide once at the end), with the causal
 * and sliding-window masks of "Build a FlashAttention-2 Inference Kernel
 * from Scratch in Pure Python", Steps 2-3.  Tiles that the mask hides
 * entirely are skipped, never loaded.
 *
 *   q, k, v : [B, H, N, d] inputs, dtype
 *   o       : [B, H, N, d] output, dtype
 *   lse     : [B, H, N] float32 output, L = m + ln(l) (natural log), or NULL
 *   causal  : 0 or 1;  window : -1 (off) or >= 0
 *
 * Supported: FA_BF16 and FA_FP16 with d in {64, 128} (MFMA kernels);
 * FA_FP32 with 1 <= d <= 256 (generic kernel).  Other d: FA_ERR_UNSUPPORTED.
 * Sizes: B*H <= 2^31-1 and B*H*N*d < 2^63; N need not be a tile multiple.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, float scale, int causal, int window,
                 fa_dtype dtype, void* stream);

/*
 * fa_fwd_ex -- fa_fwd with an explicit tile shape (0, 0 = automatic).
 *   FA_FP32: 1 <= block_q <= 64, 1 <= block_k <= 64 (any values, e.g. 4 x 4
 *            for the worked example "FlashAttention Algorithm > Worked
 *            Example", Setting Up the Example), with block_q * d and
 *            block_k * d <= 8192 and block_k * (d + 1) <= 8256; automatic: 64 x 64 for
 *            d <= 128, 32 x 32 above.
 *   FA_BF16, FA_FP16: block_q in {32, 64, 128, 256}, block_k = 64.
 * Any other pair: FA_ERR_INVALID_ARG.
 */
fa_status fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int N, int d, float scale, int causal, int window,
                    fa_dtype dtype, void* stream, int block_q, int block_k);

/*
 * fa_fwd_tune -- measure the forward's tile shapes on this problem and let
 * later automatic calls use the fastest.
 *
 * The tile shape chosen from measurement rather than fixed is the
 * "profiling-driven auto-tuning" upgrade of "Build a FlashAttention-2
 * Inference Kernel from Scratch in Pure Python", Extending It (there from
 * hardware counters; here from the HIP event timestamps of each candidate).
 * The NumPy page's roadmap (Extending It) asks for tile sizes justified by
 * the on-chip memory: every candidate fits gfx950's 160 KB of LDS.
 *
 * For each block_q in {32, 64, 128, 256} (block_k = 64) the forward runs
 * once to warm up and `reps` more times between two HIP events on
 * `stream`; the mean time per call goes to times_ms[i] (if non-NULL, 4
 * floats, candidate order as above) and the fastest block_q to
 * *best_block_q (if non-NULL).  That choice is remembered for the process
 * under the key (dtype, d, causal, window, B*H, N): fa_fwd (and fa_fwd_ex
 * with block_q = 0) then uses it instead of the built-in heuristic.  On
 * return o and lse hold the chosen tile's result for these inputs.
 *
 * Unlike every other call this one SYNCHRONISES `stream` and creates two
 * HIP events (released before it returns); it is meant for set-up, not the
 * hot loop.  The remembered table is guarded by a mutex.
 *
 * Arguments as fa_fwd, plus reps in [1, 1000].  FA_FP32: FA_ERR_UNSUPPORTED.
 */
fa_status fa_fwd_tune(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int N, int d, float scale, int causal, int window,
                      fa_dtype dtype, void* stream, int reps, int* best_block_q, float* times_ms);

/*
 * The block_q an automatic fa_fwd call uses for this problem: the one
 * fa_fwd_tune remembered (then *tuned = 1, if tuned is non-NULL), else the
 * built-in heuristic's (*tuned = 0).  Returns 0 for invalid arguments.
 */
int fa_fwd_auto_block_q(int B, int H, int N, int d, int causal, int window, fa_dtype dtype,
                        int* tuned);

/* Forget every remembered tile choice (automatic calls use the heuristic again). */
void fa_tune_reset(void);

/*
 * Save / restore the remembered tile choices, so that a process can start
 * with the choices an earlier one measured.  A row is 7 int64 values:
 * (dtype, d, causal, window, B*H, N, block_q).
 *
 * fa_tune_export writes up to max_rows rows to `rows` (host memory, 7 *
 * max_rows values) and returns the number of remembered choices (rows may
 * be NULL to query it).  fa_tune_import adds or replaces n_rows choices;
 * it checks every row first (16-bit dtype, d in {64, 128}, causal 0/1,
 * window >= -1, positive sizes, block_q a tuning candidate) and changes
 * nothing on FA_ERR_INVALID_ARG.
 */
int fa_tune_export(int64_t* rows, int max_rows);
fa_status fa_tune_import(const int64_t* rows, int n_rows);

/*
 * fa_decode_workspace_size -- bytes of workspace fa_decode needs for these
 * sizes and this split length (chunk = 0: enough for the automatic choice,
 * which may use shorter splits under a window, so size for any window).
 * Returns 0 for invalid sizes.
 */
size_t fa_decode_workspace_size(int S, int H, int Lmax, int d, int chunk);

/*
 * fa_decode -- one new query token per sequence against its KV cache,
 * split over the cache length ("split-K") and merged by logsumexp.
 *
 * Defined by "Build a FlashAttention Kernel with Online Softmax and KV Cache
 * in Pure Python", Steps 4-5: the new token's query attends to every cached
 * key including its own (the last valid row), so no causal mask is needed.
 * Each split produces a partial (m, l, o) by the online-softmax update of
 * "Building Flash Attention from Scratch in Pure NumPy", Step 2; a second
 * kernel merges the partials: M = max m_c, l = sum exp(m_c - M) l_c,
 * o = sum exp(m_c - M) o_c / l.
 *
 *   q        : [S, H, d] new queries, dtype
 *   kcache   : [S, H, Lmax, d] keys, dtype;  vcache: same for values
 *   seqlens  : [S] int32 device array, 1 <= seqlens[s] <= Lmax: rows
 *              0..seqlens[s]-1 of sequence s are valid (the last one is the
 *              new token's); other rows are never read.  Values outside
 *              [1, Lmax] are clamped into it on the device.
 *   o        : [S, H, d] output, dtype;  lse: [S, H] float32 output or NULL
 *   window   : -1 (off) or >= 0: only rows >= seqlens[s]-1-window are used
 *   chunk    : tokens per split, a positive multiple of 64, or 0 (auto)
 *   workspace: >= fa_decode_workspace_size(S, H, Lmax, d, chunk) bytes
 *
 * Supported: FA_BF16, FA_FP16 and FA_FP32 with d in {64, 128}.
 */
fa_status fa_decode(const void* q, const void* kcache, const void* vcache,
                    const int32_t* seqlens, void* o, float* lse,
                    int S, int H, int Lmax, int d, float scale, int window, int chunk,
                    void* workspace, size_t workspace_bytes, fa_dtype dtype, void* stream);

/*
 * fa_decode_paged -- fa_decode over a paged KV cache.
 *
 * The cache of "Build a FlashAttention Kernel with Online Softmax and KV
 * Cache in Pure Python", Step 2, grows token by token; here its rows live in
 * fixed-size pages drawn from a shared pool and found through a per-sequence
 * page table -- the paged KV cache listed as the first upgrade in "Build a
 * FlashAttention-2 Inference Kernel from Scratch in Pure Python", Extending
 * It -- so no sequence reserves Lmax rows.  The result is exactly fa_decode's
 * on the logical cache the table describes.
 *
 *   q, o, lse, seqlens, window, chunk : as in fa_decode
 *   k_pages     : [num_pages, H, page_size, d] key pool, dtype
 *   v_pages     : [num_pages, H, page_size, d] value pool, dtype
 *   block_table : [S, max_pages] int32 device array: logical token t of
 *                 sequence s is row t % page_size of page
 *                 block_table[s * max_pages + t / page_size].  Only the
 *                 entries covering tokens 0..seqlens[s]-1 are read.  An entry
 *                 outside [0, num_pages) hides the tokens it would hold
 *                 (used for pages evicted from a sliding window); nothing
 *                 outside the pool is ever read.
 *   page_size   : a positive multiple of 64 tokens
 *   max_pages   : table columns; seqlens[s] is clamped to
 *                 [1, max_pages * page_size]
 *   workspace   : >= fa_decode_workspace_size(S, H, max_pages * page_size,
 *                 d, chunk) bytes
 *
 * Supported: FA_BF16, FA_FP16 and FA_FP32 with d in {64, 128}.
 */
fa_status fa_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                          const int32_t* block_table, const int32_t* seqlens, void* o, float* lse,
                          int S, int H, int d, int num_pages, int page_size, int max_pages,
                          float scale, int window, int chunk,
                          void* workspace, size_t workspace_bytes, fa_dtype dtype, void* stream);

/*
 * fa_bwd_workspace_size -- bytes of workspace fa_bwd needs (0 if invalid).
 */
size_t fa_bwd_workspace_size(int B, int H, int N, int d);

/*
 * fa_bwd -- backward pass that recomputes P from the stored L.
 *
 * Defined by "Building Flash Attention from Scratch in Pure NumPy", Step 4:
 * D = rowsum(dO * O), then per K/V tile, over the query tiles it is visible
 * to, P = exp(S - L) is recomputed and
 *   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
 *   dQ = scale * dS K,  dK = scale * dS^T Q
 * (the page's dK/dQ lines are declared simplified; these are the exact
 * gradients through the softmax).
 *
 *   q, k, v, o, dO : [B, H, N, d] dtype (o and lse from fa_fwd)
 *   lse            : [B, H, N] float32
 *   dq, dk, dv     : [B, H, N, d] float32 outputs
 *   workspace      : >= fa_bwd_workspace_size(B, H, N, d) bytes
 *
 * Supported: FA_BF16 and FA_FP16 with d in {64, 128}.  No atomics: dq, dk and dv are
 * each written once, so repeated calls give identical bits.  P and dS are
 * rounded to the input type for the products that use them (fp32
 * accumulation): with FA_FP16 a |dP - D| above 65504 overflows, as for
 * any fp16 operand.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
                 const float* lse, float* dq, float* dk, float* dv,
                 int B, int H, int N, int d, float scale, int causal, int window,
                 void* workspace, size_t workspace_bytes, fa_dtype dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA355_H */
