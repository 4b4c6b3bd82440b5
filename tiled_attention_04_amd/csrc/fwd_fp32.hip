// Generic float32 forward: any head size d <= 256 and any tile shape up to
// 64 x 64 whose tiles fit the LDS staging buffers (block_q * d and
// block_k * d at most 8192 floats: 64 x 64 tiles up to d = 128, 32 x 32 up
// to d = 256), including the 4 x 4 tiles of the worked example
// ("FlashAttention Algorithm > Worked Example", Setting Up the Example).
//
// One workgroup owns one query tile and walks the key/value tiles the mask
// leaves visible, keeping the running max m, running sum l and unnormalised
// output O of the online softmax ("Building Flash Attention from Scratch in
// Pure NumPy", Architecture Overview and Step 2).  Everything is staged in
// LDS and computed with plain float32 FMAs; this path is for exactness on
// small and odd shapes, the bf16 MFMA kernels are the fast path.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxTile = 64;
constexpr int kTileFloats = 8192;            // Q, V and O tiles: block * d floats at most
constexpr int kKFloats = kMaxTile * 129;     // K tile, rows padded by one float
constexpr int kSPitch = kMaxTile + 1;

__global__ __launch_bounds__(kThreads) void fwd_fp32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int N, int d, int BQ, int BK, int nqt,
    float scale, int causal, int window) {
  __shared__ float Qs[kTileFloats];
  __shared__ float Ks[kKFloats];
  __shared__ float Vs[kTileFloats];
  __shared__ float Os[kTileFloats];
  __shared__ float Ss[kMaxTile * kSPitch];
  __shared__ float m_row[kMaxTile], l_row[kMaxTile], a_row[kMaxTile];

  const int t = threadIdx.x;
  const int bh = blockIdx.x / nqt;
  const int q0 = (blockIdx.x % nqt) * BQ;
  const size_t base = (size_t)bh * (size_t)N * (size_t)d;
  const int nq = min(BQ, N - q0);
  const int kpitch = d + 1;

  for (int i = t; i < BQ * d; i += kThreads) {
    const int r = i / d, c = i % d;
    Qs[i] = r < nq ? q[base + (size_t)(q0 + r) * d + c] : 0.f;
    Os[i] = 0.f;
  }
  if (t < BQ) {
    m_row[t] = kNegInf;
    l_row[t] = 0.f;
  }

  // Key tiles that hold at least one visible key for this query tile.
  const int kmin = window >= 0 ? max(0, q0 - window) : 0;
  const int kmax = causal ? min(N - 1, q0 + nq - 1) : N - 1;
  for (int kt = kmin / BK; kt <= kmax / BK; ++kt) {
    const int k0 = kt * BK;
    const int nk = min(BK, N - k0);
    __syncthreads();  // readers of the previous tile are done
    for (int i = t; i < BK * d; i += kThreads) {
      const int r = i / d, c = i % d;
      const bool in = r < nk;
      const size_t g = base + (size_t)(k0 + r) * d + c;
      Ks[r * kpitch + c] = in ? k[g] : 0.f;
      Vs[i] = in ? v[g] : 0.f;
    }
    __syncthreads();
    // Scaled, masked scores of the tile.
    for (int i = t; i < BQ * BK; i += kThreads) {
      const int r = i / BK, c = i % BK;
      float acc = 0.f;
      for (int e = 0; e < d; ++e) acc = __builtin_fmaf(Qs[r * d + e], Ks[c * kpitch + e], acc);
      const int qi = q0 + r, kj = k0 + c;
      const bool vis = kj < N && (!causal || kj <= qi) && (window < 0 || kj >= qi - window);
      Ss[r * kSPitch + c] = vis ? acc * scale : kNegInf;
    }
    __syncthreads();
    // Online-softmax statistics, one thread per query row.
    if (t < BQ) {
      const float m_old = m_row[t];
      float mx = kNegInf;
      for (int c = 0; c < BK; ++c) mx = fmaxf(mx, Ss[t * kSPitch + c]);
      const float m_new = fmaxf(m_old, mx);
      const float ref = m_new == kNegInf ? 0.f : m_new;  // no key seen yet: any finite reference
      const float alpha = expf(m_old - ref);               // exp(-inf) = 0 while m_old is -inf
      float sum = 0.f;
      for (int c = 0; c < BK; ++c) {
        const float p = expf(Ss[t * kSPitch + c] - ref);
        Ss[t * kSPitch + c] = p;
        sum += p;
      }
      l_row[t] = alpha * l_row[t] + sum;
      m_row[t] = m_new;
      a_row[t] = alpha;
    }
    __syncthreads();
    // O <- alpha * O + P V.
    for (int i = t; i < BQ * d; i += kThreads) {
      const int r = i / d, c = i % d;
      float acc = Os[i] * a_row[r];
      for (int j = 0; j < BK; ++j) acc = __builtin_fmaf(Ss[r * kSPitch + j], Vs[j * d + c], acc);
      Os[i] = acc;
    }
  }
  __syncthreads();
  for (int i = t; i < nq * d; i += kThreads) {
    const int r = i / d;
    const float l = l_row[r];
    o[base + (size_t)q0 * d + i] = l > 0.f ? Os[i] / l : 0.f;
  }
  if (t < nq && lse != nullptr) {
    const float l = l_row[t];
    lse[(size_t)bh * N + q0 + t] = l > 0.f ? m_row[t] + logf(l) : kNegInf;
  }
}

}  // namespace

hipError_t launch_fwd_fp32(const float* q, const float* k, const float* v, float* o, float* lse,
                           int B, int H, int N, int d, float scale, Mask mask, int block_q,
                           int block_k, hipStream_t stream) {
  const int nqt = (N + block_q - 1) / block_q;
  const long long grid = (long long)nqt * B * H;
  hipLaunchKernelGGL(fwd_fp32_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, q, k, v, o,
                     lse, N, d, block_q, block_k, nqt, scale, mask.causal, mask.window);
  return hipGetLastError();
}

}  // namespace fa
