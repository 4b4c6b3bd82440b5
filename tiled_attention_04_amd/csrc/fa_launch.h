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

// Float32 forward on the matrix cores, d in {64, 128}: 128 query rows x
// 32 keys per tile (the automatic float32 tile at those head sizes).
hipError_t launch_fwd_fp32_mfma(const float* q, const float* k, const float* v, float* o, float* lse, int B,
                                int H, int N, int d, float scale, Mask mask, hipStream_t stream);

// Generic float32 forward, any 1 <= d <= 256, tiles 1..64 x 1..64.
hipError_t launch_fwd_fp32(const float* q, const float* k, const float* v, float* o, float* lse,
                           int B, int H, int N, int d, float scale, Mask mask, int block_q,
                           int block_k, hipStream_t stream);

// 16-bit MFMA forward (bf16, or fp16 when f16), d in {64, 128}, block_q in
// {32, 64, 128} with block_k in {32, 64, 128}, or block_q = 256 with
// block_k = 64.
hipError_t launch_fwd_mfma(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, int d, float scale, Mask mask, int block_q,
                           int block_k, bool f16, hipStream_t stream);

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

// The same dense decode with its partials in a static device array of
// kDecodeScratchBytes per device instead of a caller workspace (the caller
// has checked that decode_workspace_bytes fits).  No allocation; calls that
// overlap on one device race on the array.
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
// Per-sequence flags of the arguments the decode repairs on the device
// (bit 1: length outside [1, capacity]; bit 2: an absent page among those read).
hipError_t launch_decode_check(const int32_t* seqlens, const int32_t* block_table, int S, int Lmax,
                               int page_size, int max_pages, int num_pages, int window, int32_t* flags,
                               hipStream_t stream);
hipError_t launch_decode_noalloc(const void* q, const void* kc, const void* vc, const int32_t* seqlens,
                                 void* o, float* lse, int S, int H, int Lmax, int d, float scale,
                                 int window, int chunk, Elem elem, hipStream_t stream);

// 16-bit backward (bf16, or fp16 when f16), d in {64, 128}.  dq_rows picks
// how dQ is formed: by a kernel that recomputes S and dP, with 256 (8-wave
// ping-pong) or 128 (4 waves) query rows per workgroup, before the dK / dV
// kernel (bwd_auto_dq_rows is the built-in choice between them; workspace
// bwd_workspace_bytes); or kDqStored: the dK / dV kernel also stores dS and
// a product kernel forms dQ = scale dS K from it (workspace
// bwd_workspace_bytes_ds, which grows with the visible blocks of N x N).
constexpr int kDqStored = 1;
size_t bwd_workspace_bytes(int B, int H, int N, int d);
size_t bwd_workspace_bytes_ds(int B, int H, int N, int d, Mask mask);

// Float32 backward, any 1 <= d <= 256: the dQ kernel (which also leaves D of
// every query row in ws) then the dK / dV kernel, both over square tiles of
// bwd_fp32_tile(d) rows.  ws: at least B * H * N floats.
int bwd_fp32_tile(int d);
// Float32 backward on the matrix cores, d in {64, 128}: the dQ kernel (which
// also stores D and L log2(e) of every query row in ws) then the dK / dV
// kernel, 128 rows per workgroup.  ws: at least 2 * B * H * N floats.
hipError_t launch_bwd_fp32_mfma(const float* q, const float* k, const float* v, const float* o, const float* dO,
                                const float* lse, float* dq, float* dk, float* dv, int B, int H, int N, int d,
                                float scale, Mask mask, void* ws, hipStream_t stream);
hipError_t launch_bwd_fp32(const float* q, const float* k, const float* v, const float* o, const float* dO,
                           const float* lse, float* dq, float* dk, float* dv, int B, int H, int N, int d,
                           float scale, Mask mask, void* ws, hipStream_t stream);
int bwd_auto_dq_rows(int B, int H, int N);
hipError_t launch_bwd_mfma(const void* q, const void* k, const void* v, const void* o,
                           const void* dO, const float* lse, float* dq, float* dk, float* dv,
                           int B, int H, int N, int d, float scale, Mask mask, void* ws, bool f16,
                           int dq_rows, hipStream_t stream);

}  // namespace fa
