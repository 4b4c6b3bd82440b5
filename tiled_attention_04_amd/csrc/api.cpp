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

// The built-in forward tile, as block_q * 1000 + block_k, from sweeps of
// every tile over shapes from 1 x 8 x 64 to 4 x 32 x 4096, d = 64 and 128,
// with and without windows (one MI355X):
//  * a window of at most 128 keys: 32 x 32 -- a tile of bq rows touches about
//    bq + W keys for W + 1 useful ones, and short tiles waste the least
//    (15-25% ahead of 128-row tiles at W = 128; from W = 256 on, 128-row
//    tiles lead again, by 25-44% at 2 x 16 x 4096);
//  * d = 128 without a window, while the 8-wave ping-pong kernel (256 query
//    rows, one workgroup per CU) still fills the 256 CUs: 256 x 64;
//  * otherwise the 4-wave kernel (two workgroups per CU) with 128 query rows
//    and 32-key tiles at d = 128, 64-key tiles at d = 64 -- ahead of 32- and
//    64-row tiles even when its grid leaves CUs idle (up to 4.7x at
//    1 x 8 x 1024 x 64, where one-wave workgroups each load every K/V tile
//    alone), and at d = 64 ahead of the ping-pong kernel too.
// Every choice measured within 15% of the fastest tile of its shape.
int auto_tile(int B, int H, int N, int d, int window) {
  const long long bh = (long long)B * H;
  if (window >= 0 && window <= 128) return 32032;
  if (d == 128 && window < 0 && bh * ((N + 255) / 256) >= 256) return 256064;
  return d == 128 ? 128032 : 128064;
}

// Choices measured by the tuning calls, by kind and problem: automatic calls
// with the same key use them instead of the built-in heuristics.  Key:
// (kind, dtype, d, causal, window, B*H or S*H, N or Lmax).
enum TuneKind {
  kTuneFwd = FA_TUNE_FWD_TILE,
  kTuneDecode = FA_TUNE_DECODE_CHUNK,
  kTuneBwd = FA_TUNE_BWD_DQ_ROWS
};
using TuneKey = std::tuple<int, int, int, int, int, long long, int>;
std::mutex g_tune_mu;
std::map<TuneKey, int> g_tuned;

TuneKey tune_key(TuneKind kind, fa_dtype dtype, int d, int causal, int window, long long rows, int n) {
  return TuneKey{(int)kind, (int)dtype, d, causal, window, rows, n};
}

int tuned_value(const TuneKey& key) {
  std::lock_guard<std::mutex> lock(g_tune_mu);
  auto it = g_tuned.find(key);
  return it == g_tuned.end() ? 0 : it->second;
}

void remember(const TuneKey& key, int value) {
  std::lock_guard<std::mutex> lock(g_tune_mu);
  g_tuned[key] = value;
}

// A forward tile is remembered as block_q * 1000 + block_k.
int tuned_tile(fa_dtype dtype, int d, int causal, int window, int B, int H, int N) {
  return tuned_value(tune_key(kTuneFwd, dtype, d, causal, window, (long long)B * H, N));
}

// The split length of an automatic decode call: the tuned one, else the
// heuristic.  (Tuning only tries splits at least as long as the shortest
// automatic one, so fa_decode_workspace_size(..., 0) stays enough.)
int auto_decode_chunk(fa_dtype dtype, int d, int window, int S, int H, int Lmax) {
  const int t = tuned_value(tune_key(kTuneDecode, dtype, d, 0, window, (long long)S * H, Lmax));
  return t != 0 ? t : fa::decode_auto_chunk(S, H, Lmax, window);
}

// How an fa_bwd call forms dQ: the tuned choice, else from the stored dS
// whenever the workspace holds it, else the recompute kernel the heuristic
// picks (also when the tuned choice is the stored dS but the workspace is
// too small for it).
int auto_dq_rows(fa_dtype dtype, int d, int causal, int window, int B, int H, int N, size_t workspace_bytes) {
  const bool room = workspace_bytes >= fa::bwd_workspace_bytes_ds(B, H, N, d, fa::Mask{causal, window});
  const int t = tuned_value(tune_key(kTuneBwd, dtype, d, causal, window, (long long)B * H, N));
  if (t == 128 || t == 256 || (t == fa::kDqStored && room)) return t;
  return room ? fa::kDqStored : fa::bwd_auto_dq_rows(B, H, N);
}

// One timing loop of a tuning call: a warm-up launch, then reps launches
// between two events; the mean ms per launch, or a negative value with err
// set on failure.
template <typename Launch>
float time_launches(hipEvent_t ev0, hipEvent_t ev1, hipStream_t s, int reps, hipError_t& err,
                    Launch&& launch) {
  err = launch();
  if (err == hipSuccess) err = hipEventRecord(ev0, s);
  for (int r = 0; r < reps && err == hipSuccess; ++r) err = launch();
  if (err == hipSuccess) err = hipEventRecord(ev1, s);
  if (err == hipSuccess) err = hipEventSynchronize(ev1);
  float ms = 0.f;
  if (err == hipSuccess) err = hipEventElapsedTime(&ms, ev0, ev1);
  return err == hipSuccess ? ms / (float)reps : -1.f;
}

// Two timing events, destroyed with the object.
struct EventPair {
  hipEvent_t ev[2] = {nullptr, nullptr};
  hipError_t err = hipSuccess;
  EventPair() {
    err = hipEventCreate(&ev[0]);
    if (err == hipSuccess) err = hipEventCreate(&ev[1]);
  }
  ~EventPair() {
    if (ev[0]) (void)hipEventDestroy(ev[0]);
    if (ev[1]) (void)hipEventDestroy(ev[1]);
  }
};

// Forward tiles (block_q, block_k) fa_fwd_tune measures, as block_q * 1000 +
// block_k: the 1-4 wave kernels with 32-, 64- and 128-key tiles, and the
// 8-wave ping-pong kernel (64-key tiles only: its three LDS stages would not
// fit 128).
constexpr int kTuneCandidates[FA_FWD_TUNE_CANDIDATES] = {32032,  32064,  32128,  64032,  64064,
                                                         64128,  128032, 128064, 128128, 256064};
// (128-key tiles at d = 64 only: at d = 128 they exceed the register file.)
bool valid_16bit_tile(int block_q, int block_k, int d) {
  if (block_k == 128 && d != 64) return false;
  for (int c : kTuneCandidates) {
    if (c == block_q * 1000 + block_k) return true;
  }
  return false;
}
constexpr int kDecodeTuneChunks[FA_DECODE_TUNE_CANDIDATES] = {256, 512, 1024, 2048, 4096};
constexpr int kDecodeTuneCount = FA_DECODE_TUNE_CANDIDATES;

// Checks of a dense decode call; on success `chunk` holds the split length
// the call will use (the automatic one when it was 0).
fa_status check_decode(const void* q, const void* kcache, const void* vcache, const int32_t* seqlens,
                       const void* o, int S, int H, int Lmax, int d, float scale, int window,
                       int& chunk, int dtype) {
  if (!q || !kcache || !vcache || !seqlens || !o)
    return fail(FA_ERR_INVALID_ARG, "q, kcache, vcache, seqlens and o must be non-null");
  if (S <= 0 || H <= 0 || Lmax <= 0 || d <= 0)
    return fail(FA_ERR_INVALID_ARG, "sizes must be positive (S=%d H=%d Lmax=%d d=%d)", S, H, Lmax, d);
  if ((long long)S * H > INT_MAX) return fail(FA_ERR_INVALID_ARG, "S*H exceeds 2^31-1");
  if (window < -1) return fail(FA_ERR_INVALID_ARG, "window must be -1 (off) or >= 0 (got %d)", window);
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite");
  if (chunk < 0 || chunk % 64 != 0)
    return fail(FA_ERR_INVALID_ARG, "chunk must be 0 (auto) or a positive multiple of 64 (got %d)", chunk);
  if (!valid_dtype(dtype)) return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "decode supports d in {64, 128} (got %d)", d);
  if ((long long)Lmax * d * (long long)elem_bytes((fa_dtype)dtype) > kMaxBufferBytes)
    return fail(FA_ERR_UNSUPPORTED, "one (sequence, head) cache slice exceeds 2 GiB");
  if (chunk == 0) chunk = auto_decode_chunk((fa_dtype)dtype, d, window, S, H, Lmax);
  const long long nchunk = (Lmax + chunk - 1) / chunk;
  if (nchunk * S * H * 256 > kMaxThreadsPerLaunch) return fail(FA_ERR_UNSUPPORTED, "grid too large");
  return FA_OK;
}

// Checks of a backward call (fa_bwd and fa_bwd_tune).
fa_status check_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
                    const float* lse, const float* dq, const float* dk, const float* dv, int B, int H,
                    int N, int d, float scale, int causal, int window, const void* workspace,
                    size_t workspace_bytes, fa_dtype dtype) {
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv)
    return fail(FA_ERR_INVALID_ARG, "every tensor pointer of fa_bwd must be non-null");
  fa_status st = check_dense(B, H, N, d, scale, causal, window, dtype);
  if (st != FA_OK) return st;
  if (dtype == FA_FP32) {
    if (d > 256) return fail(FA_ERR_UNSUPPORTED, "float32 backward supports d <= 256 (got %d)", d);
  } else if (d != 64 && d != 128) {
    return fail(FA_ERR_UNSUPPORTED, "%s backward supports d in {64, 128} (got %d)", dtype_name(dtype), d);
  }
  if ((long long)N * d * 4 > kMaxBufferBytes)
    return fail(FA_ERR_UNSUPPORTED, "one (batch, head) slice of the float32 gradients exceeds 2 GiB");
  // The largest grid: 256-thread workgroups over tiles of 128 query rows or
  // keys (16-bit), or bwd_fp32_tile(d) (float32).
  const int tile = dtype == FA_FP32 ? fa::bwd_fp32_tile(d) : 128;
  if ((long long)((N + tile - 1) / tile) * B * H * 256 > kMaxThreadsPerLaunch)
    return fail(FA_ERR_UNSUPPORTED, "grid too large");
  const size_t need = fa::bwd_workspace_bytes(B, H, N, d);
  if (!workspace || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "backward needs %zu workspace bytes (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", null pointer");
  return FA_OK;
}

}  // namespace

extern "C" {

static_assert(fa::kDqStored == FA_BWD_DQ_STORED, "stored-dS choice code");

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
    // 128 x 32 on the matrix cores at d = 64 and 128 (the automatic tile
    // there), any tile up to 64 x 64 on the vector ALUs.
    const bool mfma = d == 64 || d == 128;
    if (block_q == 0 && block_k == 0) {
      block_q = mfma ? 128 : 64;
      block_k = mfma ? 32 : 64;
    }
    const bool on_mfma = mfma && block_q == 128 && block_k == 32;
    if (!on_mfma && (block_q < 1 || block_q > 64 || block_k < 1 || block_k > 64))
      return fail(FA_ERR_INVALID_ARG, "float32 tiles must be 1..64 x 1..64, or 128 x 32 at d = 64 or 128 "
                  "(got %d x %d at d = %d)", block_q, block_k, d);
    const long long wgs = (long long)B * H * ((N + block_q - 1) / block_q);
    if (wgs * 256 > kMaxThreadsPerLaunch) return fail(FA_ERR_UNSUPPORTED, "grid too large");
    if (on_mfma)
      return done(fa::launch_fwd_fp32_mfma((const float*)q, (const float*)k, (const float*)v, (float*)o, lse,
                                           B, H, N, d, scale, mask, (hipStream_t)stream),
                  "fa_fwd (float32)");
    return done(fa::launch_fwd_fp32((const float*)q, (const float*)k, (const float*)v, (float*)o, lse,
                                    B, H, N, d, scale, mask, block_q, block_k, (hipStream_t)stream),
                "fa_fwd (float32)");
  }
  if (d != 64 && d != 128)
    return fail(FA_ERR_UNSUPPORTED, "%s forward supports d in {64, 128} (got %d)", dtype_name(dtype), d);
  if (block_q == 0) {  // the tuned tile, else the heuristic's
    int t = tuned_tile(dtype, d, causal, window, B, H, N);
    if (t == 0) t = auto_tile(B, H, N, d, window);
    block_q = t / 1000;
    if (block_k == 0) block_k = t % 1000;
    if (block_q == 256 && block_k != 64) block_q = 128;  // the ping-pong kernel has 64-key tiles only
  }
  if (block_k == 0) block_k = 64;
  if (!valid_16bit_tile(block_q, block_k, d))
    return fail(FA_ERR_INVALID_ARG, "16-bit tiles must be {32,64,128} x {32,64} (x 128 too at d = 64) or 256 x 64 "
                "(got %d x %d at d = %d)", block_q, block_k, d);
  const long long wgs = (long long)B * H * ((N + block_q - 1) / block_q);
  if (wgs * 2 * block_q > kMaxThreadsPerLaunch) return fail(FA_ERR_UNSUPPORTED, "grid too large");
  return done(fa::launch_fwd_mfma(q, k, v, o, lse, B, H, N, d, scale, mask, block_q, block_k,
                                  dtype == FA_FP16, (hipStream_t)stream),
              dtype == FA_FP16 ? "fa_fwd (fp16)" : "fa_fwd (bf16)");
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int N, int d, float scale, int causal, int window, fa_dtype dtype, void* stream) {
  return fa_fwd_ex(q, k, v, o, lse, B, H, N, d, scale, causal, window, dtype, stream, 0, 0);
}

fa_status fa_fwd_tune(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                      int N, int d, float scale, int causal, int window, fa_dtype dtype, void* stream,
                      int reps, int* best_block_q, int* best_block_k, float* times_ms) {
  if (!q || !k || !v || !o) return fail(FA_ERR_INVALID_ARG, "q, k, v and o must be non-null");
  fa_status st = check_dense(B, H, N, d, scale, causal, window, dtype);
  if (st != FA_OK) return st;
  if (dtype == FA_FP32) return fail(FA_ERR_UNSUPPORTED, "tuning covers the 16-bit forward only");
  if (d != 64 && d != 128)
    return fail(FA_ERR_UNSUPPORTED, "%s forward supports d in {64, 128} (got %d)", dtype_name(dtype), d);
  if (reps < 1 || reps > 1000) return fail(FA_ERR_INVALID_ARG, "reps must be 1..1000 (got %d)", reps);
  for (int c : kTuneCandidates) {  // every candidate's grid must be launchable
    const int bq = c / 1000;
    const long long wgs = (long long)B * H * ((N + bq - 1) / bq);
    if (wgs * 2 * bq > kMaxThreadsPerLaunch) return fail(FA_ERR_UNSUPPORTED, "grid too large");
  }
  const hipStream_t s = (hipStream_t)stream;
  const fa::Mask mask{causal, window};
  const bool f16 = dtype == FA_FP16;
  EventPair evs;
  if (evs.err != hipSuccess) return done(evs.err, "fa_fwd_tune (event)");
  hipError_t err = hipSuccess;
  float best_ms = 0.f;
  int best = 0;
  for (int i = 0; i < FA_FWD_TUNE_CANDIDATES && err == hipSuccess; ++i) {
    const int bq = kTuneCandidates[i] / 1000, bk = kTuneCandidates[i] % 1000;
    if (!valid_16bit_tile(bq, bk, d)) {
      if (times_ms) times_ms[i] = -1.f;
      continue;
    }
    const float ms = time_launches(evs.ev[0], evs.ev[1], s, reps, err, [&] {
      return fa::launch_fwd_mfma(q, k, v, o, lse, B, H, N, d, scale, mask, bq, bk, f16, s);
    });
    if (times_ms) times_ms[i] = ms;
    if (err == hipSuccess && (best == 0 || ms < best_ms)) {
      best = kTuneCandidates[i];
      best_ms = ms;
    }
  }
  if (err != hipSuccess) return done(err, "fa_fwd_tune");
  remember(tune_key(kTuneFwd, dtype, d, causal, window, (long long)B * H, N), best);
  if (best_block_q) *best_block_q = best / 1000;
  if (best_block_k) *best_block_k = best % 1000;
  // Leave o and lse holding the chosen tile's result.
  return done(fa::launch_fwd_mfma(q, k, v, o, lse, B, H, N, d, scale, mask, best / 1000, best % 1000, f16, s),
              "fa_fwd_tune");
}

int fa_fwd_auto_block_q(int B, int H, int N, int d, int causal, int window, fa_dtype dtype,
                        int* block_k, int* tuned) {
  if (tuned) *tuned = 0;
  if (block_k) *block_k = 0;
  if (check_dense(B, H, N, d, 0.f, causal, window, dtype) != FA_OK) return 0;
  if (dtype == FA_FP32) {
    const bool mfma = d == 64 || d == 128;
    if (block_k) *block_k = mfma ? 32 : 64;
    return mfma ? 128 : 64;
  }
  const int t = tuned_tile(dtype, d, causal, window, B, H, N);
  if (t != 0) {
    if (tuned) *tuned = 1;
    if (block_k) *block_k = t % 1000;
    return t / 1000;
  }
  const int a = auto_tile(B, H, N, d, window);
  if (block_k) *block_k = a % 1000;
  return a / 1000;
}

fa_status fa_decode_tune(const void* q, const void* kcache, const void* vcache, const int32_t* seqlens,
                         void* o, float* lse, int S, int H, int Lmax, int d, float scale, int window,
                         void* workspace, size_t workspace_bytes, fa_dtype dtype, void* stream, int reps,
                         int* best_chunk, float* times_ms) {
  int chunk0 = 0;  // (validates everything; chunk0 becomes the automatic choice)
  fa_status st = check_decode(q, kcache, vcache, seqlens, o, S, H, Lmax, d, scale, window, chunk0,
                              (int)dtype);
  if (st != FA_OK) return st;
  if (reps < 1 || reps > 1000) return fail(FA_ERR_INVALID_ARG, "reps must be 1..1000 (got %d)", reps);
  const int min_chunk = fa::decode_auto_chunk(S, H, Lmax, 0);
  const size_t need = fa::decode_workspace_bytes(S, H, Lmax, d, min_chunk);
  if (!workspace || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "decode tuning needs %zu workspace bytes, as for an automatic call "
                "(got %zu%s)", need, workspace_bytes, workspace ? "" : ", null pointer");
  const hipStream_t s = (hipStream_t)stream;
  EventPair evs;
  if (evs.err != hipSuccess) return done(evs.err, "fa_decode_tune (event)");
  hipError_t err = hipSuccess;
  float best_ms = 0.f;
  int best = 0;
  for (int i = 0; i < kDecodeTuneCount && err == hipSuccess; ++i) {
    const int c = kDecodeTuneChunks[i];
    // Splits shorter than the shortest automatic one would outgrow the
    // workspace an automatic call is promised; splits past the longest
    // cache repeat the one-split case.
    const bool ok = c >= min_chunk && (i == 0 || kDecodeTuneChunks[i - 1] < Lmax);
    if (!ok) {
      if (times_ms) times_ms[i] = -1.f;
      continue;
    }
    const float ms = time_launches(evs.ev[0], evs.ev[1], s, reps, err, [&] {
      return fa::launch_decode(q, kcache, vcache, seqlens, o, lse, S, H, Lmax, d, scale, window, c,
                               workspace, elem_of(dtype), s);
    });
    if (times_ms) times_ms[i] = ms;
    if (err == hipSuccess && (best == 0 || ms < best_ms)) {
      best = c;
      best_ms = ms;
    }
  }
  if (err != hipSuccess) return done(err, "fa_decode_tune");
  if (best == 0) best = min_chunk;  // (every candidate skipped: cannot happen, min_chunk <= 1024)
  remember(tune_key(kTuneDecode, dtype, d, 0, window, (long long)S * H, Lmax), best);
  if (best_chunk) *best_chunk = best;
  return done(fa::launch_decode(q, kcache, vcache, seqlens, o, lse, S, H, Lmax, d, scale, window, best,
                                workspace, elem_of(dtype), s),
              "fa_decode_tune");
}

int fa_decode_auto_chunk(int S, int H, int Lmax, int d, int window, fa_dtype dtype, int* tuned) {
  if (tuned) *tuned = 0;
  if (S <= 0 || H <= 0 || Lmax <= 0 || window < -1 || !valid_dtype(dtype) || (d != 64 && d != 128))
    return 0;
  const int t = tuned_value(tune_key(kTuneDecode, dtype, d, 0, window, (long long)S * H, Lmax));
  if (t != 0) {
    if (tuned) *tuned = 1;
    return t;
  }
  return fa::decode_auto_chunk(S, H, Lmax, window);
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
    int64_t* r = rows + FA_TUNE_ROW * (size_t)i;
    r[0] = std::get<0>(kv.first);  // kind
    r[1] = std::get<1>(kv.first);  // dtype
    r[2] = std::get<2>(kv.first);  // d
    r[3] = std::get<3>(kv.first);  // causal
    r[4] = std::get<4>(kv.first);  // window
    r[5] = std::get<5>(kv.first);  // B * H or S * H
    r[6] = std::get<6>(kv.first);  // N or Lmax
    r[7] = kv.second;              // block_q, chunk or dQ rows
    ++i;
  }
  return n;
}

fa_status fa_tune_import(const int64_t* rows, int n_rows) {
  if (n_rows < 0 || (n_rows > 0 && !rows)) return fail(FA_ERR_INVALID_ARG, "rows must hold n_rows >= 0 rows");
  for (int i = 0; i < n_rows; ++i) {  // validate everything before changing the table
    const int64_t* r = rows + FA_TUNE_ROW * (size_t)i;
    bool ok_value = false;
    if (r[0] == FA_TUNE_FWD_TILE) {
      ok_value = r[7] > 0 && r[7] <= INT_MAX && valid_16bit_tile((int)(r[7] / 1000), (int)(r[7] % 1000), (int)r[2]);
    } else if (r[0] == FA_TUNE_DECODE_CHUNK) {
      for (int c : kDecodeTuneChunks) ok_value |= r[7] == c;
      ok_value &= r[3] == 0;
    } else if (r[0] == FA_TUNE_BWD_DQ_ROWS) {
      ok_value = r[7] == 128 || r[7] == 256 || r[7] == FA_BWD_DQ_STORED;
    }
    if (!ok_value || (r[1] != FA_BF16 && r[1] != FA_FP16) || (r[2] != 64 && r[2] != 128) ||
        (r[3] != 0 && r[3] != 1) || r[4] < -1 || r[4] > INT_MAX || r[5] <= 0 || r[5] > INT_MAX ||
        r[6] <= 0 || r[6] > INT_MAX)
      return fail(FA_ERR_INVALID_ARG, "tuning row %d is not a valid (kind, dtype, d, causal, window, rows, "
                  "N, value) entry", i);
  }
  std::lock_guard<std::mutex> lock(g_tune_mu);
  for (int i = 0; i < n_rows; ++i) {
    const int64_t* r = rows + FA_TUNE_ROW * (size_t)i;
    g_tuned[TuneKey{(int)r[0], (int)r[1], (int)r[2], (int)r[3], (int)r[4], r[5], (int)r[6]}] = (int)r[7];
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
  const fa_status st = check_decode(q, kcache, vcache, seqlens, o, S, H, Lmax, d, scale, window, chunk,
                                    (int)dtype);
  if (st != FA_OK) return st;
  const size_t need = fa::decode_workspace_bytes(S, H, Lmax, d, chunk);
  if (!workspace || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "decode needs %zu workspace bytes (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", null pointer");
  return done(fa::launch_decode(q, kcache, vcache, seqlens, o, lse, S, H, Lmax, d, scale, window, chunk,
                                workspace, elem_of(dtype), (hipStream_t)stream),
              "fa_decode");
}

fa_status fa_decode_noalloc(const void* q, const void* kcache, const void* vcache,
                            const int32_t* seqlens, void* o, float* lse, int S, int H, int Lmax, int d,
                            float scale, int window, int chunk, fa_dtype dtype, void* stream) {
  static_assert(fa::kDecodeScratchBytes == FA_DECODE_NOALLOC_SCRATCH_BYTES,
                "the header states the scratch size");
  const fa_status st = check_decode(q, kcache, vcache, seqlens, o, S, H, Lmax, d, scale, window, chunk,
                                    (int)dtype);
  if (st != FA_OK) return st;
  const size_t need = fa::decode_workspace_bytes(S, H, Lmax, d, chunk);
  if (need > fa::kDecodeScratchBytes)
    return fail(FA_ERR_WORKSPACE,
                "fa_decode_noalloc: %d splits of %d tokens for %d x %d (sequence, head) pairs need %zu "
                "bytes of partials, above its %zu-byte static scratch (use fa_decode with a workspace, "
                "or longer splits)",
                (int)((Lmax + chunk - 1) / chunk), chunk, S, H, need, (size_t)fa::kDecodeScratchBytes);
  return done(fa::launch_decode_noalloc(q, kcache, vcache, seqlens, o, lse, S, H, Lmax, d, scale, window,
                                        chunk, elem_of(dtype), (hipStream_t)stream),
              "fa_decode_noalloc");
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
  if (chunk == 0) chunk = auto_decode_chunk(dtype, d, window, S, H, Lmax);
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

fa_status fa_decode_check(const int32_t* seqlens, const int32_t* block_table, int S, int Lmax, int page_size,
                          int max_pages, int num_pages, int window, int32_t* flags, void* stream) {
  if (!seqlens || !flags) return fail(FA_ERR_INVALID_ARG, "seqlens and flags must be non-null");
  if (S < 0) return fail(FA_ERR_INVALID_ARG, "S must be >= 0 (got %d)", S);
  if (window < -1) return fail(FA_ERR_INVALID_ARG, "window must be -1 (off) or >= 0 (got %d)", window);
  if (block_table) {
    if (page_size <= 0 || max_pages <= 0 || num_pages <= 0)
      return fail(FA_ERR_INVALID_ARG, "page_size, max_pages and num_pages must be positive (got %d, %d, %d)",
                  page_size, max_pages, num_pages);
    if ((long long)max_pages * page_size > INT_MAX)
      return fail(FA_ERR_INVALID_ARG, "max_pages * page_size exceeds 2^31-1");
  } else if (Lmax <= 0) {
    return fail(FA_ERR_INVALID_ARG, "Lmax must be positive for a dense cache (got %d)", Lmax);
  }
  return done(fa::launch_decode_check(seqlens, block_table, S, Lmax, page_size, max_pages, num_pages, window,
                                      flags, (hipStream_t)stream),
              "fa_decode_check");
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return 0;
  return fa::bwd_workspace_bytes(B, H, N, d);
}

size_t fa_bwd_workspace_size_ds(int B, int H, int N, int d, int causal, int window) {
  if (check_dense(B, H, N, d, 0.f, causal, window, FA_BF16) != FA_OK || (d != 64 && d != 128)) return 0;
  return fa::bwd_workspace_bytes_ds(B, H, N, d, fa::Mask{causal, window});
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
                 const float* lse, float* dq, float* dk, float* dv, int B, int H, int N, int d,
                 float scale, int causal, int window, void* workspace, size_t workspace_bytes,
                 fa_dtype dtype, void* stream) {
  const fa_status st = check_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, window,
                                 workspace, workspace_bytes, dtype);
  if (st != FA_OK) return st;
  if (dtype == FA_FP32) {  // matrix cores at d = 64 and 128, vector ALUs otherwise
    const auto launch = d == 64 || d == 128 ? fa::launch_bwd_fp32_mfma : fa::launch_bwd_fp32;
    return done(launch((const float*)q, (const float*)k, (const float*)v, (const float*)o, (const float*)dO, lse,
                       dq, dk, dv, B, H, N, d, scale, fa::Mask{causal, window}, workspace, (hipStream_t)stream),
                "fa_bwd (float32)");
  }
  return done(fa::launch_bwd_mfma(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale,
                                  fa::Mask{causal, window}, workspace, dtype == FA_FP16,
                                  auto_dq_rows(dtype, d, causal, window, B, H, N, workspace_bytes),
                                  (hipStream_t)stream),
              "fa_bwd");
}

fa_status fa_bwd_tune(const void* q, const void* k, const void* v, const void* o, const void* dO,
                      const float* lse, float* dq, float* dk, float* dv, int B, int H, int N, int d,
                      float scale, int causal, int window, void* workspace, size_t workspace_bytes,
                      fa_dtype dtype, void* stream, int reps, int* best_dq_rows, float* times_ms) {
  const fa_status st = check_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, window,
                                 workspace, workspace_bytes, dtype);
  if (st != FA_OK) return st;
  if (dtype == FA_FP32) return fail(FA_ERR_UNSUPPORTED, "the float32 backward has one kernel: nothing to tune");
  if (reps < 1 || reps > 1000) return fail(FA_ERR_INVALID_ARG, "reps must be 1..1000 (got %d)", reps);
  const hipStream_t s = (hipStream_t)stream;
  const fa::Mask mask{causal, window};
  EventPair evs;
  if (evs.err != hipSuccess) return done(evs.err, "fa_bwd_tune (event)");
  hipError_t err = hipSuccess;
  const int cand[FA_BWD_TUNE_CANDIDATES] = {128, 256, fa::kDqStored};
  const bool room = workspace_bytes >= fa::bwd_workspace_bytes_ds(B, H, N, d, mask);
  float best_ms = 0.f;
  int best = 0;
  for (int i = 0; i < FA_BWD_TUNE_CANDIDATES && err == hipSuccess; ++i) {
    if (cand[i] == fa::kDqStored && !room) {
      if (times_ms) times_ms[i] = -1.f;
      continue;
    }
    const float ms = time_launches(evs.ev[0], evs.ev[1], s, reps, err, [&] {
      return fa::launch_bwd_mfma(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, mask, workspace,
                                 dtype == FA_FP16, cand[i], s);
    });
    if (times_ms) times_ms[i] = ms;
    if (err == hipSuccess && (best == 0 || ms < best_ms)) {
      best = cand[i];
      best_ms = ms;
    }
  }
  if (err != hipSuccess) return done(err, "fa_bwd_tune");
  remember(tune_key(kTuneBwd, dtype, d, causal, window, (long long)B * H, N), best);
  if (best_dq_rows) *best_dq_rows = best;
  return done(fa::launch_bwd_mfma(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, mask, workspace,
                                  dtype == FA_FP16, best, s),
              "fa_bwd_tune");
}

int fa_bwd_auto_dq_rows(int B, int H, int N, int d, int causal, int window, fa_dtype dtype,
                        size_t workspace_bytes, int* tuned) {
  if (tuned) *tuned = 0;
  if (check_dense(B, H, N, d, 0.f, causal, window, dtype) != FA_OK || dtype == FA_FP32 ||
      (d != 64 && d != 128))
    return 0;
  const int choice = auto_dq_rows(dtype, d, causal, window, B, H, N, workspace_bytes);
  const int t = tuned_value(tune_key(kTuneBwd, dtype, d, causal, window, (long long)B * H, N));
  if (tuned) *tuned = t != 0 && t == choice;
  return choice;
}

}  // extern "C"
