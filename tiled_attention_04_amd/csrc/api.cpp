// C ABI of libfa355 (declared in include/fa355.h): argument validation,
// kernel selection and launch on the caller's stream.  Every check runs
// before the first HIP call, so a non-HIP error means nothing was launched.
#include "fa355.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <tuple>

#include "fa_launch.h"

namespace {

thread_local char g_err[512] = "";

fa_status fail(fa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

fa_status done(hipError_t err, const char* what) {
  if (err != hipSuccess) return fail(FA_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
  g_err[0] = '\0';
  return FA_OK;
}

size_t elem_bytes(fa_dtype t) { return t == FA_FP32 ? 4 : 2; }

bool valid_dtype(int t) { return t == FA_FP32 || t == FA_BF16 || t == FA_FP16; }

fa::Elem elem_of(fa_dtype t) {
  return t == FA_BF16 ? fa::Elem::kBF16 : t == FA_FP16 ? fa::Elem::kF16 : fa::Elem::kF32;
}

const char* dtype_name(fa_dtype t) { return t == FA_BF16 ? "bf16" : t == FA_FP16 ? "fp16" : "float32"; }

constexpr long long kMaxThreadsPerLaunch = 0xFFFFFFFFLL;  // grid * block must fit 32 bits
constexpr long long kMaxBufferBytes = 0x7FFFFFFFLL;       // 32-bit buffer offsets per slice

// Checks common to the dense (forward / backward) calls.
fa_status check_dense(int B, int H, int N, int d, float scale, int causal, int window, int dtype) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0)
    return fail(FA_ERR_INVALID_ARG, "sizes must be positive (B=%d H=%d N=%d d=%d)", B, H, N, d);
  if ((long long)B * H > INT_MAX) return fail(FA_ERR_INVALID_ARG, "B*H exceeds 2^31-1");
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
  if (window < -1) return fail(FA_ERR_INVALID_ARG, "window must be -1 (off) or >= 0 (got %d)", window);
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite");
  if (!valid_dtype(dtype)) return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if ((long long)N * d * (long long)elem_bytes((fa_dtype)dtype) > kMaxBufferBytes)
    return fail(FA_ERR_UNSUPPORTED, "one (batch, head) slice of N*d exceeds 2 GiB");
  return FA_OK;
}

int auto_block_q(int B, int H, int N, int window) {
  // Prefer the 8-wave ping-pong kernel (256 query rows, one workgroup per
  // CU) while it still fills the 256 CUs of an MI355X -- except under a
  // sliding window, where the 4-wave kernel measured faster; then 4-wave
  // workgroups (two per CU); then smaller query tiles.
  const long long bh = (long long)B * H;
  if (window < 0 && bh * ((N + 255) / 256) >= 256) return 256;
  if (bh * ((N + 127) / 128) >= 512) return 128;
  if (bh * ((N + 63) / 64) >= 256) return 64;
  return 32;
}

// Tile choices measured by fa_fwd_tune, by problem: automatic calls with
// the same (dtype, d, causal, window, B*H, N) use them instead of the
// heuristic above.
using TuneKey = std::tuple<int, int, int, int, long long, int>;
std::mutex g_tune_mu;
std::map<TuneKey, int> g_tuned;

TuneKey tune_key(fa_dtype dtype, int d, int causal, int window, int B, int H, int N) {
  return TuneKey{(int)dtype, d, causal, window, (long long)B * H, N};
}

int tuned_block_q(const TuneKey& key) {
  std::lock_guard<std::mutex> lock(g_tune_mu);
  auto it = g_tuned.find(key);
  return it == g_tuned.end() ? 0 : it->second;
}

constexpr int kTuneCandidates[4] = {32, 64, 128, 256};

}  // namespace

extern "C" {

int fa_version(void) { return 100; }

const char* fa_status_str(fa_status status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
    case FA_ERR_HIP: return "FA_ERR_HIP";
  }
  return "FA_ERR_UNKNOWN";
}

const char* fa_last_error(void) { return g_err; }

fa_status fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                    int N, int d, float scale, int causal, int window, fa_dtype dtype, void* stream,
                    int block_q, int block_k) {
  if (!q || !k || !v || !o) return fail(FA_ERR_INVALID_ARG, "q, k, v and o must be non-null");
  fa_status st = check_dense(B, H, N, d, scale, causal, window, dtype);
  if (st != FA_OK) return st;
  const fa::Mask mask{causal, window};
  if (dtype == FA_FP32) {
    if (d > 256) return fail(FA_ERR_UNSUPPORTED, "float32 forward supports d <= 256 (got %d)", d);
    if (block_q == 0 && block_k == 0) block_q = block_k = d <= 128 ? 64 : 32;
    if (block_q < 1 || block_q > 64 || block_k < 1 || block_k > 64)
      return fail(FA_ERR_INVALID_ARG, "float32 tiles must be 1..64 x 1..64 (got %d x %d)", block_q, block_k);
    if (block_q * d > 8192 || block_k * d > 8192 || block_k * (d + 1) > 64 * 129)
      return fail(FA_ERR_INVALID_ARG, "float32 tiles of %d x %d rows do not fit LDS at d = %d", block_q,
                  block_k, d);
    const long long wgs = (long long)B * H * ((N + block_q - 1) / block_q);
    if (wgs * 256 > kMaxThreadsPerLaunch) return fail(FA_ERR_UNSUPPORTED, "grid too large");
    return done(fa::launch_fwd_fp32((const float*)q, (const float*)k, (const float*)v, (float*)o, lse,
                                    B, H, N, d, scale, mask, block_q, block_k, (hipStream_t)stream),
                "fa_fwd (float32)");
  }
  if (d != 64 && d != 128)
    return fail(FA_ERR_UNSUPPORTED, "%s forward supports d in {64, 128} (got %d)", dtype_name(dtype), d);
  if (block_q == 0) block_q = tuned_block_q(tune_key(dtype, d, causal, window, B, H, N));
  if (block_q == 0) block_q = auto_block_q(B, H, N, window);
  if (block_k == 0) block_k = 64;
  if ((block_q != 32 && block_q != 64 && block_q != 128 && block_q != 256) || block_k != 64)
    return fail(FA_ERR_INVALID_ARG, "16-bit tiles must be {32,64,128,256} x 64 (got %d x %d)", block_q, block_k);
  const long long wgs = (long long)B * H * ((N + block_q - 1) / block_q);
  if (wgs * 2 * block_q > kMaxThreadsPerLaunch) return fail(FA_ERR_UNSUPPORTED, "grid too large");
  return done(fa::launch_fwd_mfma(q, k, v, o, lse, B, H, N, d, scale, mask, block_q,
                                  dtype == FA_FP16, (hipStream_t)stream),
              dtype == FA_FP16 ? "fa_fwd (fp16)" : "fa_fwd (bf16)");
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int N, int d, float scale, int causal, int window, fa_dtype dtype, void* stream) {
  return fa_fwd_ex(q, k, v, o, lse, B, H, N, d, scale, causal, window, dtype, stream, 0, 0);
}

fa_status fa_fwd_tune(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                      int N, int d, float scale, int causal, int window, fa_dtype dtype, void* stream,
                      int reps, int* best_block_q, float* times_ms) {
  if (!q || !k || !v || !o) return fail(FA_ERR_INVALID_ARG, "q, k, v and o must be non-null");
  fa_status st = check_dense(B, H, N, d, scale, causal, window, dtype);
  if (st != FA_OK) return st;
  if (dtype == FA_FP32) return fail(FA_ERR_UNSUPPORTED, "tuning covers the 16-bit forward only");
  if (d != 64 && d != 128)
    return fail(FA_ERR_UNSUPPORTED, "%s forward supports d in {64, 128} (got %d)", dtype_name(dtype), d);
  if (reps < 1 || reps > 1000) return fail(FA_ERR_INVALID_ARG, "reps must be 1..1000 (got %d)", reps);
  for (int bq : kTuneCandidates) {  // every candidate's grid must be launchable
    const long long wgs = (long long)B * H * ((N + bq - 1) / bq);
    if (wgs * 2 * bq > kMaxThreadsPerLaunch) return fail(FA_ERR_UNSUPPORTED, "grid too large");
  }
  const hipStream_t s = (hipStream_t)stream;
  const fa::Mask mask{causal, window};
  const bool f16 = dtype == FA_FP16;
  hipEvent_t ev[2];
  hipError_t err = hipEventCreate(&ev[0]);
  if (err != hipSuccess) return done(err, "fa_fwd_tune (event)");
  err = hipEventCreate(&ev[1]);
  if (err != hipSuccess) {
    (void)hipEventDestroy(ev[0]);
    return done(err, "fa_fwd_tune (event)");
  }
  float best_ms = 0.f;
  int best = 0;
  for (int i = 0; i < 4 && err == hipSuccess; ++i) {
    const int bq = kTuneCandidates[i];
    err = fa::launch_fwd_mfma(q, k, v, o, lse, B, H, N, d, scale, mask, bq, f16, s);  // warm-up
    if (err == hipSuccess) err = hipEventRecord(ev[0], s);
    for (int r = 0; r < reps && err == hipSuccess; ++r)
      err = fa::launch_fwd_mfma(q, k, v, o, lse, B, H, N, d, scale, mask, bq, f16, s);
    if (err == hipSuccess) err = hipEventRecord(ev[1], s);
    if (err == hipSuccess) err = hipEventSynchronize(ev[1]);
    float ms = 0.f;
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, ev[0], ev[1]);
    ms /= (float)reps;
    if (times_ms) times_ms[i] = ms;
    if (err == hipSuccess && (best == 0 || ms < best_ms)) {
      best = bq;
      best_ms = ms;
    }
  }
  (void)hipEventDestroy(ev[0]);
  (void)hipEventDestroy(ev[1]);
  if (err != hipSuccess) return done(err, "fa_fwd_tune");
  {
    std::lock_guard<std::mutex> lock(g_tune_mu);
    g_tuned[tune_key(dtype, d, causal, window, B, H, N)] = best;
  }
  if (best_block_q) *best_block_q = best;
  // Leave o and lse holding the chosen tile's result.
  return done(fa::launch_fwd_mfma(q, k, v, o, lse, B, H, N, d, scale, mask, best, f16, s),
              "fa_fwd_tune");
}

int fa_fwd_auto_block_q(int B, int H, int N, int d, int causal, int window, fa_dtype dtype,
                        int* tuned) {
  if (tuned) *tuned = 0;
  if (check_dense(B, H, N, d, 0.f, causal, window, dtype) != FA_OK) return 0;
  if (dtype == FA_FP32) return 64;
  const int t = tuned_block_q(tune_key(dtype, d, causal, window, B, H, N));
  if (t != 0) {
    if (tuned) *tuned = 1;
    return t;
  }
  return auto_block_q(B, H, N, window);
}

void fa_tune_reset(void) {
  std::lock_guard<std::mutex> lock(g_tune_mu);
  g_tuned.clear();
}

int fa_tune_export(int64_t* rows, int max_rows) {
  std::lock_guard<std::mutex> lock(g_tune_mu);
  const int n = (int)g_tuned.size();
  if (!rows || max_rows <= 0) return n;
  int i = 0;
  for (const auto& kv : g_tuned) {
    if (i >= max_rows) break;
    int64_t* r = rows + 7 * (size_t)i;
    r[0] = std::get<0>(kv.first);  // dtype
    r[1] = std::get<1>(kv.first);  // d
    r[2] = std::get<2>(kv.first);  // causal
    r[3] = std::get<3>(kv.first);  // window
    r[4] = std::get<4>(kv.first);  // B * H
    r[5] = std::get<5>(kv.first);  // N
    r[6] = kv.second;              // block_q
    ++i;
  }
  return n;
}

fa_status fa_tune_import(const int64_t* rows, int n_rows) {
  if (n_rows < 0 || (n_rows > 0 && !rows)) return fail(FA_ERR_INVALID_ARG, "rows must hold n_rows >= 0 rows");
  for (int i = 0; i < n_rows; ++i) {  // validate everything before changing the table
    const int64_t* r = rows + 7 * (size_t)i;
    bool ok_bq = false;
    for (int bq : kTuneCandidates) ok_bq |= r[6] == bq;
    if ((r[0] != FA_BF16 && r[0] != FA_FP16) || (r[1] != 64 && r[1] != 128) || (r[2] != 0 && r[2] != 1) ||
        r[3] < -1 || r[3] > INT_MAX || r[4] <= 0 || r[4] > INT_MAX || r[5] <= 0 || r[5] > INT_MAX || !ok_bq)
      return fail(FA_ERR_INVALID_ARG, "tuning row %d is not a valid (dtype, d, causal, window, B*H, N, "
                  "block_q) entry", i);
  }
  std::lock_guard<std::mutex> lock(g_tune_mu);
  for (int i = 0; i < n_rows; ++i) {
    const int64_t* r = rows + 7 * (size_t)i;
    g_tuned[TuneKey{(int)r[0], (int)r[1], (int)r[2], (int)r[3], r[4], (int)r[5]}] = (int)r[6];
  }
  g_err[0] = '\0';
  return FA_OK;
}

size_t fa_decode_workspace_size(int S, int H, int Lmax, int d, int chunk) {
  if (S <= 0 || H <= 0 || Lmax <= 0 || d <= 0 || chunk < 0 || chunk % 64 != 0) return 0;
  if (chunk == 0) chunk = fa::decode_auto_chunk(S, H, Lmax, 0);  // the windowed choice: smallest splits, largest workspace
  return fa::decode_workspace_bytes(S, H, Lmax, d, chunk);
}

fa_status fa_decode(const void* q, const void* kcache, const void* vcache, const int32_t* seqlens,
                    void* o, float* lse, int S, int H, int Lmax, int d, float scale, int window,
                    int chunk, void* workspace, size_t workspace_bytes, fa_dtype dtype,
                    void* stream) {
  if (!q || !kcache || !vcache || !seqlens || !o)
    return fail(FA_ERR_INVALID_ARG, "q, kcache, vcache, seqlens and o must be non-null");
  if (S <= 0 || H <= 0 || Lmax <= 0 || d <= 0)
    return fail(FA_ERR_INVALID_ARG, "sizes must be positive (S=%d H=%d Lmax=%d d=%d)", S, H, Lmax, d);
  if ((long long)S * H > INT_MAX) return fail(FA_ERR_INVALID_ARG, "S*H exceeds 2^31-1");
  if (window < -1) return fail(FA_ERR_INVALID_ARG, "window must be -1 (off) or >= 0 (got %d)", window);
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite");
  if (chunk < 0 || chunk % 64 != 0)
    return fail(FA_ERR_INVALID_ARG, "chunk must be 0 (auto) or a positive multiple of 64 (got %d)", chunk);
  if (!valid_dtype(dtype)) return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "decode supports d in {64, 128} (got %d)", d);
  if ((long long)Lmax * d * (long long)elem_bytes(dtype) > kMaxBufferBytes)
    return fail(FA_ERR_UNSUPPORTED, "one (sequence, head) cache slice exceeds 2 GiB");
  if (chunk == 0) chunk = fa::decode_auto_chunk(S, H, Lmax, window);
  const long long nchunk = (Lmax + chunk - 1) / chunk;
  if (nchunk * S * H * 256 > kMaxThreadsPerLaunch) return fail(FA_ERR_UNSUPPORTED, "grid too large");
  const size_t need = fa::decode_workspace_bytes(S, H, Lmax, d, chunk);
  if (!workspace || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "decode needs %zu workspace bytes (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", null pointer");
  return done(fa::launch_decode(q, kcache, vcache, seqlens, o, lse, S, H, Lmax, d, scale, window, chunk,
                                workspace, elem_of(dtype), (hipStream_t)stream),
              "fa_decode");
}

fa_status fa_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                          const int32_t* block_table, const int32_t* seqlens, void* o, float* lse,
                          int S, int H, int d, int num_pages, int page_size, int max_pages,
                          float scale, int window, int chunk, void* workspace,
                          size_t workspace_bytes, fa_dtype dtype, void* stream) {
  if (!q || !k_pages || !v_pages || !block_table || !seqlens || !o)
    return fail(FA_ERR_INVALID_ARG, "q, k_pages, v_pages, block_table, seqlens and o must be non-null");
  if (S <= 0 || H <= 0 || d <= 0 || num_pages <= 0 || max_pages <= 0)
    return fail(FA_ERR_INVALID_ARG, "sizes must be positive (S=%d H=%d d=%d num_pages=%d max_pages=%d)",
                S, H, d, num_pages, max_pages);
  if (page_size <= 0 || page_size % 64 != 0)
    return fail(FA_ERR_INVALID_ARG, "page_size must be a positive multiple of 64 (got %d)", page_size);
  if ((long long)S * H > INT_MAX) return fail(FA_ERR_INVALID_ARG, "S*H exceeds 2^31-1");
  if ((long long)max_pages * page_size > INT_MAX)
    return fail(FA_ERR_INVALID_ARG, "max_pages * page_size exceeds 2^31-1");
  if (window < -1) return fail(FA_ERR_INVALID_ARG, "window must be -1 (off) or >= 0 (got %d)", window);
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite");
  if (chunk < 0 || chunk % 64 != 0)
    return fail(FA_ERR_INVALID_ARG, "chunk must be 0 (auto) or a positive multiple of 64 (got %d)", chunk);
  if (!valid_dtype(dtype)) return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "decode supports d in {64, 128} (got %d)", d);
  if ((long long)page_size * d * (long long)elem_bytes(dtype) > kMaxBufferBytes)
    return fail(FA_ERR_UNSUPPORTED, "one page of one head exceeds 2 GiB");
  const int Lmax = max_pages * page_size;
  if (chunk == 0) chunk = fa::decode_auto_chunk(S, H, Lmax, window);
  const long long nchunk = (Lmax + chunk - 1) / chunk;
  if (nchunk * S * H * 256 > kMaxThreadsPerLaunch) return fail(FA_ERR_UNSUPPORTED, "grid too large");
  const size_t need = fa::decode_workspace_bytes(S, H, Lmax, d, chunk);
  if (!workspace || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "paged decode needs %zu workspace bytes (got %zu%s)", need,
                workspace_bytes, workspace ? "" : ", null pointer");
  return done(fa::launch_decode_paged(q, k_pages, v_pages, block_table, seqlens, o, lse, S, H, d,
                                      num_pages, page_size, max_pages, scale, window, chunk, workspace,
                                      elem_of(dtype), (hipStream_t)stream),
              "fa_decode_paged");
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return 0;
  return fa::bwd_workspace_bytes(B, H, N, d);
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
                 const float* lse, float* dq, float* dk, float* dv, int B, int H, int N, int d,
                 float scale, int causal, int window, void* workspace, size_t workspace_bytes,
                 fa_dtype dtype, void* stream) {
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv)
    return fail(FA_ERR_INVALID_ARG, "every tensor pointer of fa_bwd must be non-null");
  fa_status st = check_dense(B, H, N, d, scale, causal, window, dtype);
  if (st != FA_OK) return st;
  if (dtype == FA_FP32) return fail(FA_ERR_UNSUPPORTED, "backward supports bf16 and fp16 inputs only");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "backward supports d in {64, 128} (got %d)", d);
  if ((long long)N * d * 4 > kMaxBufferBytes)
    return fail(FA_ERR_UNSUPPORTED, "one (batch, head) slice of the float32 gradients exceeds 2 GiB");
  const long long rows = (long long)B * H * N;
  const long long pre_rows_per_block = 2048 / d;  // 256 threads, d / 8 per row
  const long long pre_threads = (rows + pre_rows_per_block - 1) / pre_rows_per_block * 256;
  const long long main_threads = (long long)((N + 127) / 128) * B * H * 512;  // 128 keys per workgroup
  if (pre_threads > kMaxThreadsPerLaunch || main_threads > kMaxThreadsPerLaunch)
    return fail(FA_ERR_UNSUPPORTED, "grid too large");
  const size_t need = fa::bwd_workspace_bytes(B, H, N, d);
  if (!workspace || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "backward needs %zu workspace bytes (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", null pointer");
  return done(fa::launch_bwd_mfma(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale,
                                  fa::Mask{causal, window}, workspace, dtype == FA_FP16,
                                  (hipStream_t)stream),
              "fa_bwd");
}

}  // extern "C"
