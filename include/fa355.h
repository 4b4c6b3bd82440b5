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
 *            Example", Setting Up the Example) at any d <= 256, on the
 *            vector ALUs; or 128 x 32 at d = 64 and 128, on the matrix cores
 *            (float32 MFMA: float32 products and sums).  Automatic: 128 x 32
 *            at d = 64 and 128, 64 x 64 otherwise.
 *   FA_BF16, FA_FP16: block_q in {32, 64, 128} (1, 2 or 4 waves) with
 *            block_k in {32, 64}, or 128 at d = 64 (at d = 128 two 128-key
 *            score tiles exceed a wave's registers); or 256 x 64 (8 waves,
 *            two groups one phase apart, whose three LDS stages leave no
 *            room for 128-key tiles).  Automatic (block_q = 0): the tile
 *            fa_fwd_tune remembered for the problem, else the built-in
 *            choice (see fa_fwd_auto_block_q); a non-zero block_k then
 *            overrides the automatic key tile.
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
 * Candidates: the FA_FWD_TUNE_CANDIDATES tiles (block_q, block_k) = (32,
 * 32), (32, 64), (32, 128), (64, 32), (64, 64), (64, 128), (128, 32),
 * (128, 64), (128, 128) and (256, 64), in this order (the 128-key tiles
 * at d = 64 only).  Each runs once to warm up and `reps` more times
 * between two HIP events on `stream`; the mean time per call goes to
 * times_ms[i] (if non-NULL, one float per candidate, -1 for one skipped) and the fastest tile to *best_block_q / *best_block_k (each
 * if non-NULL).  That choice is remembered for the process under the key
 * (dtype, d, causal, window, B*H, N): fa_fwd (and fa_fwd_ex with block_q =
 * 0) then uses it instead of the built-in heuristic.  On return o and lse
 * hold the chosen tile's result for these inputs.
 *
 * Unlike every other call this one SYNCHRONISES `stream` and creates two
 * HIP events (released before it returns); it is meant for set-up, not the
 * hot loop.  The remembered table is guarded by a mutex.
 *
 * Arguments as fa_fwd, plus reps in [1, 1000].  FA_FP32: FA_ERR_UNSUPPORTED.
 */
#define FA_FWD_TUNE_CANDIDATES 10
fa_status fa_fwd_tune(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int N, int d, float scale, int causal, int window,
                      fa_dtype dtype, void* stream, int reps, int* best_block_q, int* best_block_k,
                      float* times_ms);

/*
 * The tile an automatic fa_fwd call uses for this problem: the one
 * fa_fwd_tune remembered (then *tuned = 1, if tuned is non-NULL), else the
 * built-in heuristic's (*tuned = 0): 32 x 32 under a window of at most 128
 * keys; 256 x 64 at d = 128 without a window when B * H * ceil(N / 256) >=
 * 256; otherwise 128 x 32 at d = 128 and 128 x 64 at d = 64 (FA_FP32:
 * 128 x 32 at d = 64 and 128, 64 x 64 otherwise).  Returns block_q and writes block_k to
 * *block_k (if non-NULL); returns 0 for invalid arguments.  (fa_fwd_ex with
 * block_q = 0 and a block_k other than 64 uses 128 rows where this would give
 * 256.)
 */
int fa_fwd_auto_block_q(int B, int H, int N, int d, int causal, int window, fa_dtype dtype,
                        int* block_k, int* tuned);

/*
 * Remembered tuning choices.  fa_fwd_tune, fa_decode_tune and fa_bwd_tune
 * each remember their fastest candidate for the problem they measured;
 * automatic calls on the same problem then use it.  A choice is a row of
 * FA_TUNE_ROW int64 values:
 *   (kind, dtype, d, causal, window, rows, n, value)
 * with, per kind,
 *   FA_TUNE_FWD_TILE    : rows = B * H, n = N, value = block_q * 1000 +
 *                         block_k
 *   FA_TUNE_DECODE_CHUNK: causal = 0, rows = S * H, n = Lmax, value = chunk
 *                         (dense, no-allocation and paged decode alike; for
 *                         the paged call Lmax = max_pages * page_size)
 *   FA_TUNE_BWD_DQ_ROWS : rows = B * H, n = N, value = query rows per
 *                         workgroup of the dQ kernel (128 or 256)
 * The table is process state guarded by a mutex.
 *
 * fa_tune_reset forgets every choice (automatic calls use the built-in
 * heuristics again).  fa_tune_export writes up to max_rows rows to `rows`
 * (host memory, FA_TUNE_ROW * max_rows values) and returns the number of
 * remembered choices (rows may be NULL to query it).  fa_tune_import adds
 * or replaces n_rows choices; it checks every row first (known kind,
 * 16-bit dtype, d in {64, 128}, causal 0/1 (0 for decode), window >= -1,
 * positive sizes, value a candidate of its kind) and changes nothing on
 * FA_ERR_INVALID_ARG.
 */
#define FA_TUNE_FWD_TILE 0
#define FA_TUNE_DECODE_CHUNK 1
#define FA_TUNE_BWD_DQ_ROWS 2
#define FA_TUNE_ROW 8
void fa_tune_reset(void);
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
 * fa_decode_tune -- measure the split length on this problem and let later
 * automatic decode calls (chunk = 0) use the fastest.
 *
 * The split length of the split-K decode ("Build a FlashAttention Kernel
 * with Online Softmax and KV Cache in Pure Python", Steps 4-5) chosen by
 * measurement: the "profiling-driven auto-tuning" upgrade of "Build a
 * FlashAttention-2 Inference Kernel from Scratch in Pure Python", Extending
 * It.  Candidates: FA_DECODE_TUNE_CANDIDATES splits of 256, 512, 1024, 2048
 * and 4096 tokens, skipping those shorter than the shortest automatic split
 * (so that fa_decode_workspace_size(S, H, Lmax, d, 0) stays enough for
 * every automatic call) and those that repeat the one-split case.  Each
 * runs once to warm up and `reps` more times between two HIP events on
 * `stream`; times_ms[i] (if non-NULL, FA_DECODE_TUNE_CANDIDATES floats in
 * the order above) gets the mean ms per call, or -1 for a skipped
 * candidate, and *best_chunk (if non-NULL) the fastest.  The choice is
 * remembered under (dtype, d, window, S * H, Lmax).  On return o and lse
 * hold the chosen split's result.
 *
 * Arguments as fa_decode (minus chunk), plus reps in [1, 1000]; the
 * workspace must hold fa_decode_workspace_size(S, H, Lmax, d, 0) bytes.
 * Like fa_fwd_tune it SYNCHRONISES `stream` and creates two HIP events.
 */
#define FA_DECODE_TUNE_CANDIDATES 5
fa_status fa_decode_tune(const void* q, const void* kcache, const void* vcache,
                         const int32_t* seqlens, void* o, float* lse,
                         int S, int H, int Lmax, int d, float scale, int window,
                         void* workspace, size_t workspace_bytes, fa_dtype dtype, void* stream,
                         int reps, int* best_chunk, float* times_ms);

/*
 * The split length an automatic decode call uses for this problem: the one
 * fa_decode_tune remembered (*tuned = 1), else the built-in choice
 * (*tuned = 0).  Returns 0 for invalid arguments.
 */
int fa_decode_auto_chunk(int S, int H, int Lmax, int d, int window, fa_dtype dtype, int* tuned);

/*
 * fa_decode_noalloc -- fa_decode that allocates nothing and takes no
 * workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same operation, arguments (minus the workspace), layouts, kernels and
 * results as fa_decode.  The split partials go to a static device array of
 * FA_DECODE_NOALLOC_SCRATCH_BYTES (32 MiB) that the library holds on every
 * device it runs on until the process ends; its address is looked up on the
 * first call on each device (that call must be made with the device
 * current).  The array needs no clearing between calls.
 *
 *   Limit: fa_decode_workspace_size(S, H, Lmax, d, chunk) must not exceed
 *   FA_DECODE_NOALLOC_SCRATCH_BYTES; larger requests return
 *   FA_ERR_WORKSPACE before any HIP call (e.g. d = 128 with splits of 1024
 *   tokens covers S * H * ceil(Lmax / 1024) up to 64,527 partials).
 *   `stream` must belong to the current device (else FA_ERR_HIP).
 *   Concurrency: every call on one device shares that device's array, so
 *   calls that can overlap on one device (different streams, or other host
 *   threads) race and give wrong results; serialise them.
 *
 * Supported: as fa_decode.
 */
#define FA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
fa_status fa_decode_noalloc(const void* q, const void* kcache, const void* vcache,
                            const int32_t* seqlens, void* o, float* lse,
                            int S, int H, int Lmax, int d, float scale, int window, int chunk,
                            fa_dtype dtype, void* stream);

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
 * fa_decode_check -- find the arguments that fa_decode, fa_decode_noalloc
 * and fa_decode_paged repair on the device instead of rejecting.  Those
 * calls read seqlens (and the page table) only on the device, so they cannot
 * return an error for them without synchronising: a length outside [1,
 * capacity] is clamped into it, and a table entry outside [0, num_pages)
 * leaves its page's tokens out (the argument readings of "Build a
 * FlashAttention Kernel with Online Softmax and KV Cache in Pure Python",
 * Step 4, and of the paged cache of "Build a FlashAttention-2 Inference
 * Kernel from Scratch in Pure Python", Extending It, extended to such input).
 * This call reports them, one int32 per sequence, so that a caller can check
 * its inputs on the stream before or after the decode:
 *   flags[s] = 0, or the OR of
 *     FA_CHECK_LENGTH (1): seqlens[s] < 1 or > capacity (capacity = Lmax
 *                          for a dense cache, max_pages * page_size for a
 *                          paged one);
 *     FA_CHECK_PAGE   (2): paged only -- an entry of block_table[s] outside
 *                          [0, num_pages) among the pages holding the tokens
 *                          the decode reads (with the window, if any, of the
 *                          decode call: pages before its first token are
 *                          never read).
 *
 *   seqlens     : [S] int32, device memory
 *   block_table : [S, max_pages] int32, device memory; NULL for a dense cache
 *                 (page_size, max_pages and num_pages are then ignored)
 *   Lmax        : dense cache length (ignored for a paged cache)
 *   window      : as in the decode call (-1 off)
 *   flags       : [S] int32, device memory, written
 *
 * Asynchronous on `stream`; allocates nothing.  S = 0 is a no-op.  Errors:
 * FA_ERR_INVALID_ARG for null pointers, S < 0, window < -1, non-positive
 * sizes, or max_pages * page_size above 2^31-1; FA_ERR_HIP if the launch fails.
 */
#define FA_CHECK_LENGTH 1
#define FA_CHECK_PAGE 2
fa_status fa_decode_check(const int32_t* seqlens, const int32_t* block_table, int S, int Lmax, int page_size,
                          int max_pages, int num_pages, int window, int32_t* flags, void* stream);

/*
 * fa_bwd_workspace_size -- bytes of workspace fa_bwd needs (0 if invalid):
 * D and L log2(e) of every query row (8 bytes per row).  With this much the
 * 16-bit backward forms dQ by recomputing S and dP.
 */
size_t fa_bwd_workspace_size(int B, int H, int N, int d);

/*
 * fa_bwd_workspace_size_ds -- bytes of workspace with which a 16-bit fa_bwd
 * call (d in {64, 128}) forms dQ from a stored dS instead (0 if invalid):
 * the above, 256-byte aligned, plus one 32 x 32 block of dS in the input type
 * (2 KB) per (query block, key block) pair holding a visible (query, key)
 * pair, per (batch, head) slice -- the lower triangle of blocks for causal
 * attention, a band of ceil(W / 32) + 1 blocks per query block with a causal
 * window of W keys, every block otherwise.  About B * H * N^2 bytes for
 * causal attention (0.54 GB at B = 2, H = 16, N = 4096), so it is the
 * caller's choice: fa_bwd takes this path whenever workspace_bytes is at
 * least this size, unless fa_bwd_tune measured a recompute kernel faster.
 * (It pays once the product kernel's grid of B * H * ceil(N / 128)
 * workgroups fills the chip; on small grids the recompute kernels lead.)
 */
size_t fa_bwd_workspace_size_ds(int B, int H, int N, int d, int causal, int window);

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
 *   workspace      : >= fa_bwd_workspace_size(B, H, N, d) bytes; with
 *                    >= fa_bwd_workspace_size_ds(...) bytes the 16-bit
 *                    backward takes the stored-dS path (below)
 *
 * Supported: FA_BF16 and FA_FP16 with d in {64, 128}, and FA_FP32 with any
 * 1 <= d <= 256.  No atomics: dq, dk and dv are each written once, so
 * repeated calls give identical bits.  For the 16-bit types P and dS are
 * rounded to the input type for the products that use them (fp32
 * accumulation): with FA_FP16 a |dP - D| above 65504 overflows, as for any
 * fp16 operand.  FA_FP32 keeps every step in float32 (float32 MFMA at
 * d = 64 and 128, vector-ALU FMAs at other d).
 *
 * How the 16-bit backward forms dQ (both ways give the same dv bits; dk and
 * dq agree to rounding order, D being summed by another kernel and dq formed
 * from the same terms in another order):
 *  - recompute: a dQ kernel in the forward's loop order (a workgroup owns
 *    query rows and walks the key tiles) recomputes S, P, dP and dS, and
 *    also stores D and L log2(e) for the dK / dV kernel that follows; seven
 *    matrix products per visible tile pair where the page's step has five;
 *  - stored dS: a small kernel forms D and L log2(e), the dK / dV kernel
 *    also writes each dS block it forms (rounded to the input type, as the
 *    products use it) into the workspace, and a product kernel forms
 *    dQ = scale * dS K from those blocks: five matrix products, plus one
 *    write and one read of the visible dS blocks.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
                 const float* lse, float* dq, float* dk, float* dv,
                 int B, int H, int N, int d, float scale, int causal, int window,
                 void* workspace, size_t workspace_bytes, fa_dtype dtype, void* stream);

/*
 * fa_bwd_tune -- measure the backward's ways of forming dQ on this problem
 * and let later fa_bwd calls use the fastest.
 *
 * Candidates (FA_BWD_TUNE_CANDIDATES, in this order): the recompute dQ kernel
 * with 128 query rows per workgroup (4 waves, two workgroups per CU), with
 * 256 (8 waves in two groups one phase apart, one workgroup per CU), and
 * FA_BWD_DQ_STORED, dQ from the stored dS (tried only when workspace_bytes
 * is at least fa_bwd_workspace_size_ds; its time is -1 otherwise).  Which is
 * fastest depends on how well each grid fills the chip and on the mask, so
 * the choice is measured: the "profiling-driven auto-tuning" upgrade of
 * "Build a FlashAttention-2 Inference Kernel from Scratch in Pure Python",
 * Extending It.  The whole backward runs once to warm up and `reps` more
 * times per candidate between two HIP events on `stream`; times_ms[i] (if
 * non-NULL, FA_BWD_TUNE_CANDIDATES floats) gets the mean ms per call and
 * *best_dq_rows (if non-NULL) the fastest (128, 256 or FA_BWD_DQ_STORED),
 * remembered under (dtype, d, causal, window, B * H, N).  On return dq, dk
 * and dv hold the chosen way's result.
 *
 * Arguments as fa_bwd (16-bit types only: the float32 backward has one
 * kernel and returns FA_ERR_UNSUPPORTED), plus reps in [1, 1000].  Like
 * fa_fwd_tune it SYNCHRONISES `stream` and creates two HIP events.
 */
#define FA_BWD_TUNE_CANDIDATES 3
#define FA_BWD_DQ_STORED 1
fa_status fa_bwd_tune(const void* q, const void* k, const void* v, const void* o, const void* dO,
                      const float* lse, float* dq, float* dk, float* dv,
                      int B, int H, int N, int d, float scale, int causal, int window,
                      void* workspace, size_t workspace_bytes, fa_dtype dtype, void* stream,
                      int reps, int* best_dq_rows, float* times_ms);

/*
 * How an fa_bwd call with workspace_bytes of workspace forms dQ for this
 * problem: 128 or 256 (the recompute kernel with that many query rows per
 * workgroup) or FA_BWD_DQ_STORED.  The choice fa_bwd_tune remembered
 * (*tuned = 1) when the workspace allows it; else (*tuned = 0) the stored dS
 * when workspace_bytes >= fa_bwd_workspace_size_ds, else the recompute
 * kernel whose grid fills the chip (256 rows once B * H * ceil(N / 256)
 * reaches 256 workgroups, else 128).  Returns 0 for invalid arguments and for
 * FA_FP32, whose backward has a single way.
 */
int fa_bwd_auto_dq_rows(int B, int H, int N, int d, int causal, int window, fa_dtype dtype,
                        size_t workspace_bytes, int* tuned);

#ifdef __cplusplus
}
#endif

#endif /* FA355_H */
