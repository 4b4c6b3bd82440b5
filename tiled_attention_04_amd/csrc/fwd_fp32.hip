// Generic float32 forward on the vector ALUs: any head size 1 <= d <= 256
// and any tile shape from 1 x 1 to 64 x 64 (block_q query rows x block_k
// keys), including the 4 x 4 tiles of the worked example ("FlashAttention
// Algorithm > Worked Example", Setting Up the Example).  The automatic
// float32 tile at d = 64 and 128 runs on the matrix cores instead
// (fwd_fp32_mfma.hip).
//
// One workgroup owns one query tile and walks the key/value tiles the mask
// leaves visible, keeping the running max m, running sum l and unnormalised
// output O of the online softmax ("Building Flash Attention from Scratch in
// Pure NumPy", Architecture Overview and Step 2) for each of its rows; the
// statistics move once per key tile of the caller's size, as the page's loop
// does, so every tile shape gives the same result up to rounding.  The
// arithmetic is plain float32 FMAs on LDS-staged tiles: the tiles sit in 64-row LDS
// buffers whatever the caller's tile, a 16 x 16 grid of threads holds 4 x 4
// scores each, a row's max and sum are butterflies over its 16 lanes, and
// the P V product accumulates one key at a time into registers.  Up to
// d = 128, K and V have their own buffers; above, V is staged into K's
// buffer once the scores of the tile are taken, so that 64-row tiles of
// 256 columns fit the LDS.
#include "fa_launch.h"
#include "fp32_tile.h"

namespace fa {
namespace {

using namespace fp32;

constexpr int kTB = 64;

template <int DM, bool kSharedKV>
__global__ __launch_bounds__(kThreads) void fwd_fp32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int N, int d, int BQ, int BK, int nqt,
    float scale, int causal, int window) {
  using F = Tile<kTB, DM>;
  constexpr int R = F::R, P = F::kPitch, SP = F::kSPitch;
  __shared__ __align__(16) float Qs[kTB * P];
  __shared__ __align__(16) float Ks[kTB * P];
  __shared__ __align__(16) float Vbuf[kSharedKV ? 4 : kTB * P];
  __shared__ float Ts[kTB * SP];
  float* Vs = kSharedKV ? Ks : Vbuf;

  const int t = threadIdx.x, ti = t >> 4, tj = t & 15;
  const int bh = blockIdx.x / nqt;
  const int q0 = (blockIdx.x - bh * nqt) * BQ;
  const size_t base = (size_t)bh * N * d;
  const int dpad = (d + 3) & ~3;
  const int nq = min(BQ, N - q0);

  stage<kTB, P>(Qs, q + base, q0, nq, d, dpad);

  float m_run[R], l_run[R];
  float4 oacc[R][F::kChunks];
#pragma unroll
  for (int a = 0; a < R; ++a) {
    m_run[a] = kNegInf;
    l_run[a] = 0.f;
  }
  zero<kTB, DM>(oacc);

  // Key tiles that hold at least one visible key for this query tile.
  const int kmin = window >= 0 ? max(0, q0 - window) : 0;
  const int kmax = causal ? min(N - 1, q0 + nq - 1) : N - 1;
  for (int kt = kmin / BK; kt <= kmax / BK; ++kt) {
    const int k0 = kt * BK;
    const int nk = min(BK, N - k0);
    __syncthreads();  // the previous tile's readers are done
    stage<kTB, P>(Ks, k + base, k0, nk, d, dpad);
    if constexpr (!kSharedKV) stage<kTB, P>(Vs, v + base, k0, nk, d, dpad);
    __syncthreads();
    float s[1][R][R];
    dot_blocks<kTB, DM, 1>(Qs, Ks, nullptr, nullptr, dpad, ti, tj, s);
#pragma unroll
    for (int a = 0; a < R; ++a) {
      const int i = ti + 16 * a;
      float x[R];
      float mx = kNegInf;
#pragma unroll
      for (int b = 0; b < R; ++b) {
        const int j = tj + 16 * b;
        const bool vis = i < nq && j < nk && visible(q0 + i, k0 + j, N, causal, window);
        x[b] = vis ? s[0][a][b] * scale : kNegInf;
        mx = fmaxf(mx, x[b]);
      }
      const float m_new = fmaxf(m_run[a], row_max16(mx));
      const float ref = m_new == kNegInf ? 0.f : m_new;  // no key seen yet: any finite reference
      const float alpha = expf(m_run[a] - ref);           // exp(-inf) = 0 while m is -inf
      float sum = 0.f;
#pragma unroll
      for (int b = 0; b < R; ++b) {
        const float p = expf(x[b] - ref);
        Ts[(tj + 16 * b) * SP + i] = p;  // [key][query]: the P V product walks keys
        sum += p;
      }
      l_run[a] = alpha * l_run[a] + row_sum16(sum);
      m_run[a] = m_new;
#pragma unroll
      for (int c = 0; c < F::kChunks; ++c) {
        oacc[a][c].x *= alpha;
        oacc[a][c].y *= alpha;
        oacc[a][c].z *= alpha;
        oacc[a][c].w *= alpha;
      }
    }
    if constexpr (kSharedKV) {
      __syncthreads();  // the scores are taken: K's buffer takes V
      stage<kTB, P>(Vs, v + base, k0, nk, d, dpad);
    }
    __syncthreads();
    accumulate<kTB, DM>(Ts, Vs, nk, dpad, ti, tj, oacc);
  }

  float inv[R];
#pragma unroll
  for (int a = 0; a < R; ++a) inv[a] = l_run[a] > 0.f ? 1.f / l_run[a] : 0.f;
  store_rows<kTB, DM>(o + base, oacc, inv, q0, nq, d, ti, tj);
  if (lse != nullptr && tj == 0) {
#pragma unroll
    for (int a = 0; a < R; ++a) {
      const int i = ti + 16 * a;
      if (i < nq) lse[(size_t)bh * N + q0 + i] = l_run[a] > 0.f ? m_run[a] + logf(l_run[a]) : kNegInf;
    }
  }
}

}  // namespace

hipError_t launch_fwd_fp32(const float* q, const float* k, const float* v, float* o, float* lse,
                           int B, int H, int N, int d, float scale, Mask mask, int block_q,
                           int block_k, hipStream_t stream) {
  const int nqt = (N + block_q - 1) / block_q;
  const unsigned grid = (unsigned)((long long)nqt * B * H);
  if (d <= 128)
    hipLaunchKernelGGL((fwd_fp32_kernel<128, false>), dim3(grid), dim3(kThreads), 0, stream, q, k, v, o, lse, N, d,
                       block_q, block_k, nqt, scale, mask.causal, mask.window);
  else
    hipLaunchKernelGGL((fwd_fp32_kernel<256, true>), dim3(grid), dim3(kThreads), 0, stream, q, k, v, o, lse, N, d,
                       block_q, block_k, nqt, scale, mask.causal, mask.window);
  return hipGetLastError();
}

}  // namespace fa
