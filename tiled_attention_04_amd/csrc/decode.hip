// Single-token decode over a KV cache, split over the cache length and merged
// by logsumexp.
//
// Method: "Build a FlashAttention Kernel with Online Softmax and KV Cache in
// Pure Python", Steps 4-5 -- the new token's query attends to every valid
// cache row, its own included, so no mask is needed.  Each split runs the
// online-softmax update of "Building Flash Attention from Scratch in Pure
// NumPy", Step 2, over its rows and leaves a partial (m, l, o); the merge
// kernel combines the partials with the same rescaling identity.
//
// The work is a matrix-vector product per (sequence, head): about one flop
// per byte of K/V, so it is bound by HBM bandwidth, and it runs on the vector
// ALUs (a 1-row MFMA would waste 31 of 32 rows).  Design points:
//  * Every lane loads 16 bytes of a cache row; a group of D*elem/16 lanes
//    covers one row and a wave reads several rows per instruction, fully
//    coalesced.  Each lane keeps 8 rows of K and 8 of V in flight, so a
//    256-thread workgroup has 64 KB of loads outstanding.
//  * Loads go through a buffer resource sized to the valid rows of the
//    (sequence, head), so rows at or past seqlens[s] are never read (they
//    return zero and are masked), and no 64-bit address arithmetic is needed
//    per lane.
//  * q is pre-multiplied by scale*log2(e) in float32; scores are reduced
//    across the row's lanes with DPP; exponentials are exp2.
//  * Workgroups past the end of a sequence (the grid is sized from Lmax on
//    the host, since the lengths live on the device) exit at once.
#include "fa_common.h"
#include "fa_launch.h"

#include <mutex>

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 8;

// A 16-byte load of a cache row, marked non-temporal: every row is read once
// per call, so keeping it in the caches only evicts other data.  (Measured on
// the 64 x 32 ragged batch: 5.86 -> 6.61 TB/s dense, 5.47 -> 6.05 TB/s with a
// 1024-token window, 5.93 -> 6.52 TB/s paged; same values.)
constexpr int kCacheStream = 2;  // buffer-load cache policy: nt
__device__ __forceinline__ uint4 load_row16(rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kCacheStream));
}

template <typename T>
__device__ __forceinline__ void widen(const uint4& u, float (&x)[16 / sizeof(T)]);

template <>
__device__ __forceinline__ void widen<bf16>(const uint4& u, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = word(u, i);
    x[2 * i] = bf16_lo(w);
    x[2 * i + 1] = bf16_hi(w);
  }
}

template <>
__device__ __forceinline__ void widen<f16>(const uint4& u, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = word(u, i);
    x[2 * i] = f16_lo(w);
    x[2 * i + 1] = f16_hi(w);
  }
}

template <>
__device__ __forceinline__ void widen<float>(const uint4& u, float (&x)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = __builtin_bit_cast(float, word(u, i));
}

__device__ __forceinline__ void clamp_len(int& n, int Lmax) { n = n < 1 ? 1 : (n > Lmax ? Lmax : n); }

// Where the cache rows live.  Dense: [S][H][Lmax][D].  Paged: a pool of pages
// [num_pages][H][page_size][D]; token t of sequence s is row t % page_size of
// page table[s * max_pages + t / page_size].  A table entry outside
// [0, num_pages) hides the tokens it would hold (they are never read).
struct PagedCache {
  const int32_t* table;  // null: dense cache
  int page_size, max_pages, num_pages;
};

template <typename T, int D, bool PAGED>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(
    const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
    const int32_t* __restrict__ seqlens, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    int S, int H, int Lmax, int nchunk, int chunk, float scale_log2, int window, PagedCache pc) {
  constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte load
  constexpr int LPR = D / VEC;          // lanes per cache row
  constexpr int RPW = 64 / LPR;         // rows per wave instruction
  constexpr int GROUPS = kWaves * RPW;  // row groups in the workgroup
  constexpr int ROWS = kUnroll * RPW;   // rows per loop trip (at most 64)
  __shared__ float red_o[GROUPS][D];
  __shared__ float red_m[GROUPS], red_l[GROUPS];

  const int id = blockIdx.x;
  const int h = id % H;
  const int s = (id / H) % S;
  int n = seqlens[s];
  clamp_len(n, Lmax);
  const int lo = window >= 0 ? max(0, n - 1 - window) : 0;
  // With a window the grid covers only the splits a window can touch,
  // counted from the one holding its first row; without, all of them.
  const int c = id / (H * S) + (window >= 0 ? lo / chunk : 0);
  const int c_begin = c * chunk;
  if (c >= nchunk || c_begin >= n || c_begin + chunk <= lo) return;  // the merge skips this split too

  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // uniform: row ranges and pages per wave
  const int g = lane / LPR, e = lane % LPR;
  const size_t sh = (size_t)s * H + h;
  rsrc_t k_src, v_src;
  if constexpr (!PAGED) {  // one buffer over the valid rows of the (sequence, head) slice
    const size_t slice = sh * (size_t)Lmax * D;
    const uint32_t valid_bytes = (uint32_t)n * D * (uint32_t)sizeof(T);
    k_src = make_rsrc(kc + slice, valid_bytes);
    v_src = make_rsrc(vc + slice, valid_bytes);
  }

  float qv[VEC];
  widen<T>(*(const uint4*)(q + sh * D + e * VEC), qv);
#pragma unroll
  for (int i = 0; i < VEC; ++i) qv[i] *= scale_log2;

  // This wave's rows: a quarter of the split, clipped to [lo, n).  With pages
  // the loop trips start at multiples of ROWS (page sizes are multiples of
  // 64), so every trip reads a single page; rows before r_lo are masked.
  const int per_wave = chunk / kWaves;
  const int r_lo = max(lo, c_begin + w * per_wave);
  const int r_begin = PAGED ? (r_lo & ~(ROWS - 1)) : r_lo;
  const int r_end = min(n, c_begin + (w + 1) * per_wave);

  float m = kNegInf, l = 0.f;
  float acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.f;

  for (int r0 = r_begin; r0 < r_end; r0 += ROWS) {
    int row0 = r0;  // row of the trip's first row within its buffer
    bool page_ok = true;
    if constexpr (PAGED) {
      // The buffer covers the page's valid rows only: rows at or past n read
      // as zero (a stale row could hold NaN, and 0 * NaN is NaN).
      const int slot = r0 / pc.page_size;
      // (wave-uniform, so the buffer resource below lives in scalar registers)
      const int page = __builtin_amdgcn_readfirstlane(pc.table[(size_t)s * pc.max_pages + slot]);
      page_ok = (uint32_t)page < (uint32_t)pc.num_pages;
      const int rows_here = min(pc.page_size, n - slot * pc.page_size);
      const size_t pbase = ((size_t)(page_ok ? page : 0) * H + h) * (size_t)pc.page_size * D;
      const uint32_t pbytes = page_ok ? (uint32_t)rows_here * D * (uint32_t)sizeof(T) : 0u;
      k_src = make_rsrc(kc + pbase, pbytes);
      v_src = make_rsrc(vc + pbase, pbytes);
      row0 = r0 - slot * pc.page_size;
    }
    uint4 kr[kUnroll], vr[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t off = (uint32_t)((row0 + u * RPW + g) * D + e * VEC) * (uint32_t)sizeof(T);
      kr[u] = load_row16(k_src, off);
      vr[u] = load_row16(v_src, off);
    }
    // Every load of the trip is issued before any of them is used (left
    // alone, the compiler interleaves fp16 loads with their mixed-precision
    // FMAs and keeps far fewer bytes in flight).
    __builtin_amdgcn_sched_barrier(0);
    float sc[kUnroll];
    float mx = kNegInf;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float kx[VEC];
      widen<T>(kr[u], kx);
      float p = 0.f;
#pragma unroll
      for (int i = 0; i < VEC; ++i) p = __builtin_fmaf(qv[i], kx[i], p);
      p = group_sum<LPR>(p);
      const int row = r0 + u * RPW + g;
      const bool in = PAGED ? (row >= r_lo) & (row < r_end) & page_ok : row < r_end;
      sc[u] = in ? p : kNegInf;
      mx = fmaxf(mx, sc[u]);
    }
    const float m_new = fmaxf(m, mx);
    const float ref = m_new == kNegInf ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - ref);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] *= alpha;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float p = __builtin_amdgcn_exp2f(sc[u] - ref);
      l += p;
      float vx[VEC];
      widen<T>(vr[u], vx);
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] = __builtin_fmaf(p, vx[i], acc[i]);
    }
  }

  // Combine the row groups of the workgroup, then write this split's partial.
  const int gi = w * RPW + g;
#pragma unroll
  for (int i = 0; i < VEC; ++i) red_o[gi][e * VEC + i] = acc[i];
  if (e == 0) {
    red_m[gi] = m;
    red_l[gi] = l;
  }
  __syncthreads();
  if (t < D) {
    float M = kNegInf;
    for (int j = 0; j < GROUPS; ++j) M = fmaxf(M, red_m[j]);
    const float ref = M == kNegInf ? 0.f : M;
    float o = 0.f, L = 0.f;
    for (int j = 0; j < GROUPS; ++j) {
      const float a = __builtin_amdgcn_exp2f(red_m[j] - ref);
      o = __builtin_fmaf(a, red_o[j][t], o);
      L = __builtin_fmaf(a, red_l[j], L);
    }
    const size_t part = sh * nchunk + c;
    ws_o[part * D + t] = o;
    if (t == 0) {
      ws_ml[2 * part] = M;
      ws_ml[2 * part + 1] = L;
    }
  }
}

template <typename T>
__device__ __forceinline__ T from_float(float x);
template <>
__device__ __forceinline__ float from_float<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_float<bf16>(float x) { return (bf16)x; }
template <>
__device__ __forceinline__ f16 from_float<f16>(float x) { return (f16)x; }

// One workgroup of D threads per (sequence, head): M = max m_c,
// l = sum exp(m_c - M) l_c, o = sum exp(m_c - M) o_c / l, L = M ln2 + ln l.
template <typename T, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
    const int32_t* __restrict__ seqlens, T* __restrict__ o, float* __restrict__ lse, int H,
    int Lmax, int nchunk, int chunk, int window) {
  const int sh = blockIdx.x;
  const int s = sh / H;
  const int t = threadIdx.x;
  int n = seqlens[s];
  clamp_len(n, Lmax);
  const int lo = window >= 0 ? max(0, n - 1 - window) : 0;
  const int c0 = lo / chunk, c1 = (n - 1) / chunk;
  const size_t part0 = (size_t)sh * nchunk;
  float M = kNegInf;
  for (int c = c0; c <= c1; ++c) M = fmaxf(M, ws_ml[2 * (part0 + c)]);
  const float ref = M == kNegInf ? 0.f : M;
  float acc = 0.f, L = 0.f;
  for (int c = c0; c <= c1; ++c) {
    const float a = __builtin_amdgcn_exp2f(ws_ml[2 * (part0 + c)] - ref);
    L = __builtin_fmaf(a, ws_ml[2 * (part0 + c) + 1], L);
    acc = __builtin_fmaf(a, ws_o[(part0 + c) * D + t], acc);
  }
  o[(size_t)sh * D + t] = from_float<T>(L > 0.f ? acc / L : 0.f);
  if (t == 0 && lse != nullptr) lse[sh] = L > 0.f ? M * kLn2 + logf(L) : kNegInf;
}

template <typename T, int D>
hipError_t launch_t(const void* q, const void* kc, const void* vc, const int32_t* seqlens, void* o,
                    float* lse, int S, int H, int Lmax, float scale, int window, int chunk,
                    void* ws, PagedCache pc, hipStream_t stream) {
  const int nchunk = (Lmax + chunk - 1) / chunk;
  float* ws_o = (float*)ws;
  float* ws_ml = ws_o + (size_t)S * H * nchunk * D;
  // A window of W rows touches at most ceil(W / chunk) + 1 splits.
  const int nsplit = window >= 0 ? min(nchunk, (window + chunk) / chunk + 1) : nchunk;
  const long long grid = (long long)nsplit * S * H;
  if (pc.table)
    hipLaunchKernelGGL((decode_split_kernel<T, D, true>), dim3((unsigned)grid), dim3(kThreads), 0, stream,
                       (const T*)q, (const T*)kc, (const T*)vc, seqlens, ws_o, ws_ml, S, H, Lmax,
                       nchunk, chunk, scale * kLog2e, window, pc);
  else
    hipLaunchKernelGGL((decode_split_kernel<T, D, false>), dim3((unsigned)grid), dim3(kThreads), 0, stream,
                       (const T*)q, (const T*)kc, (const T*)vc, seqlens, ws_o, ws_ml, S, H, Lmax,
                       nchunk, chunk, scale * kLog2e, window, pc);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((unsigned)(S * H)), dim3(D), 0, stream,
                     ws_o, ws_ml, seqlens, (T*)o, lse, H, Lmax, nchunk, chunk, window);
  return hipGetLastError();
}

}  // namespace

int decode_auto_chunk(int S, int H, int Lmax, int window) {
  // Large splits keep the merge cheap; shrink them only when the grid would
  // otherwise hold fewer than ~4 workgroups per compute unit.  The cap:
  // 1024 tokens for full caches, 512 under a window (whose few splits per
  // sequence then balance better); measured on the 64 x 32 ragged batch,
  // 1024 against 512 is 1.2-1.9% faster without a window, 1.6% slower with
  // a 1024-token one.
  long long target = (long long)S * H * Lmax / 1024;
  int chunk = (int)(target / 64) * 64;
  const int cap = window >= 0 ? 512 : 1024;
  if (chunk > cap) chunk = cap;
  if (chunk < 64) chunk = 64;
  return chunk;
}

size_t decode_workspace_bytes(int S, int H, int Lmax, int d, int chunk) {
  const size_t nchunk = (size_t)((Lmax + chunk - 1) / chunk);
  return (size_t)S * H * nchunk * (size_t)(d + 2) * sizeof(float);
}

namespace {
template <typename T>
hipError_t dispatch_t(const void* q, const void* kc, const void* vc, const int32_t* seqlens, void* o,
                      float* lse, int S, int H, int Lmax, int d, float scale, int window, int chunk,
                      void* ws, PagedCache pc, hipStream_t stream) {
  if (d == 128)
    return launch_t<T, 128>(q, kc, vc, seqlens, o, lse, S, H, Lmax, scale, window, chunk, ws, pc, stream);
  return launch_t<T, 64>(q, kc, vc, seqlens, o, lse, S, H, Lmax, scale, window, chunk, ws, pc, stream);
}

hipError_t dispatch(const void* q, const void* kc, const void* vc, const int32_t* seqlens, void* o,
                    float* lse, int S, int H, int Lmax, int d, float scale, int window, int chunk,
                    void* ws, Elem elem, PagedCache pc, hipStream_t stream) {
  switch (elem) {
    case Elem::kBF16:
      return dispatch_t<bf16>(q, kc, vc, seqlens, o, lse, S, H, Lmax, d, scale, window, chunk, ws, pc, stream);
    case Elem::kF16:
      return dispatch_t<f16>(q, kc, vc, seqlens, o, lse, S, H, Lmax, d, scale, window, chunk, ws, pc, stream);
    default:
      return dispatch_t<float>(q, kc, vc, seqlens, o, lse, S, H, Lmax, d, scale, window, chunk, ws, pc, stream);
  }
}
}  // namespace

hipError_t launch_decode(const void* q, const void* kc, const void* vc, const int32_t* seqlens,
                         void* o, float* lse, int S, int H, int Lmax, int d, float scale,
                         int window, int chunk, void* ws, Elem elem, hipStream_t stream) {
  return dispatch(q, kc, vc, seqlens, o, lse, S, H, Lmax, d, scale, window, chunk, ws, elem,
                  PagedCache{nullptr, 0, 0, 0}, stream);
}

// ---------------------------------------------------------------------------
// Decode without a caller workspace, for callers that cannot allocate.  The
// split partials go to `scratch`, a fixed array in device memory: the loader
// places one copy on every device the library runs on, and it stays until the
// process ends.  Its device address is looked up once per device with
// hipGetSymbolAddress (in host code the array's name is only a stand-in, not
// an address a kernel can use) and kept in `g_scratch_ptr`.  Every call on a
// device shares that device's copy, so calls that overlap on one device race;
// nothing in it needs clearing, because the merge kernel reads only the
// partials its own split kernel wrote in the same call.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_ptr(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (stream != nullptr) {  // the partials must live on the stream's device
    int sdev = 0;
    err = hipStreamGetDevice(stream, &sdev);
    if (err != hipSuccess) return err;
    if (sdev != dev) return hipErrorInvalidDevice;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

hipError_t launch_decode_noalloc(const void* q, const void* kc, const void* vc, const int32_t* seqlens,
                                 void* o, float* lse, int S, int H, int Lmax, int d, float scale,
                                 int window, int chunk, Elem elem, hipStream_t stream) {
  void* ws = nullptr;
  const hipError_t err = scratch_ptr(stream, &ws);
  if (err != hipSuccess) return err;
  return dispatch(q, kc, vc, seqlens, o, lse, S, H, Lmax, d, scale, window, chunk, ws, elem,
                  PagedCache{nullptr, 0, 0, 0}, stream);
}

hipError_t launch_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                               const int32_t* block_table, const int32_t* seqlens, void* o, float* lse,
                               int S, int H, int d, int num_pages, int page_size, int max_pages,
                               float scale, int window, int chunk, void* ws, Elem elem,
                               hipStream_t stream) {
  return dispatch(q, k_pages, v_pages, seqlens, o, lse, S, H, max_pages * page_size, d, scale, window,
                  chunk, ws, elem, PagedCache{block_table, page_size, max_pages, num_pages}, stream);
}

namespace {

// One thread per sequence: the arguments the decode kernels repair on the
// device instead of rejecting (clamp_len above; table entries outside the
// pool), reported as flag bits.  For a paged cache only the pages that hold
// the tokens a call reads are examined (with a window, the pages before its
// first token are never read, so whatever they hold does no harm).
__global__ __launch_bounds__(256) void decode_check_kernel(const int32_t* __restrict__ seqlens,
                                                           PagedCache pc, int S, int Lmax, int window,
                                                           int32_t* __restrict__ flags) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= S) return;
  const int cap = pc.table ? pc.max_pages * pc.page_size : Lmax;
  int n = seqlens[s];
  int f = (n < 1 || n > cap) ? 1 : 0;
  if (pc.table) {
    clamp_len(n, cap);
    const int lo = window >= 0 ? max(0, n - 1 - window) : 0;
    const int32_t* row = pc.table + (size_t)s * pc.max_pages;
    for (int p = lo / pc.page_size; p <= (n - 1) / pc.page_size; ++p)
      if ((uint32_t)row[p] >= (uint32_t)pc.num_pages) f |= 2;
  }
  flags[s] = f;
}

}  // namespace

hipError_t launch_decode_check(const int32_t* seqlens, const int32_t* block_table, int S, int Lmax,
                               int page_size, int max_pages, int num_pages, int window, int32_t* flags,
                               hipStream_t stream) {
  if (S == 0) return hipSuccess;
  const PagedCache pc{block_table, page_size, max_pages, num_pages};
  hipLaunchKernelGGL(decode_check_kernel, dim3((unsigned)((S + 255) / 256)), dim3(256), 0, stream, seqlens, pc, S,
                     Lmax, window, flags);
  return hipGetLastError();
}

}  // namespace fa
