// Internal launchers, one per kernel family.  Arguments have been validated by
// the C ABI layer (api.cpp) before any of these is called; each returns the
// HIP error of its launch(es).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Mask bounds shared by every kernel family: query i sees key j iff
// (!causal || j <= i) && (window < 0 || j >= i - window) && j < n_keys.
struct Mask {
  int causal;
  int window;
};

// Element type of q, k, v, o (and dO, the caches).
enum class Elem { kF32, kBF16, kF16 };

// Generic float32 forward, any 1 <= d <= 128, tiles 1..64 x 1..64.
hipError_t launch_fwd_fp32(const float* q, const float* k, const float* v, float* o, float* lse,
                           int B, int H, int N, int d, float scale, Mask mask, int block_q,
                           int block_k, hipStream_t stream);

// 16-bit MFMA forward (bf16, or fp16 when f16), d in {64, 128}, block_q in
// {32, 64, 128, 256}, block_k = 64.
hipError_t launch_fwd_mfma(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, int d, float scale, Mask mask, int block_q,
                           bool f16, hipStream_t stream);

// Split-K decode (+ merge), any Elem, d in {64, 128}.
size_t decode_workspace_bytes(int S, int H, int Lmax, int d, int chunk);
int decode_auto_chunk(int S, int H, int Lmax, int window);
hipError_t launch_decode(const void* q, const void* kc, const void* vc, const int32_t* seqlens,
                         void* o, float* lse, int S, int H, int Lmax, int d, float scale,
                         int window, int chunk, void* ws, Elem elem, hipStream_t stream);
hipError_t launch_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                               const int32_t* block_table, const int32_t* seqlens, void* o, float* lse,
                               int S, int H, int d, int num_pages, int page_size, int max_pages,
                               float scale, int window, int chunk, void* ws, Elem elem,
                               hipStream_t stream);

// 16-bit backward (bf16, or fp16 when f16): preprocess, dK/dV and dQ
// kernels, d in {64, 128}.
size_t bwd_workspace_bytes(int B, int H, int N, int d);
hipError_t launch_bwd_mfma(const void* q, const void* k, const void* v, const void* o,
                           const void* dO, const float* lse, float* dq, float* dk, float* dv,
                           int B, int H, int N, int d, float scale, Mask mask, void* ws, bool f16,
                           hipStream_t stream);

}  // namespace fa
