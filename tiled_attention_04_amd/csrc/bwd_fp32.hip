// Float32 backward: dQ, dK and dV recomputed from the stored L for any head
// size 1 <= d <= 256 ("Building Flash Attention from Scratch in Pure NumPy",
// Step 4: D = rowsum(dO * O), P = exp(scale * Q K^T - L), dV = P^T dO,
// dP = dO V^T, dS = P * (dP - D), dQ = scale * dS K, dK = scale * dS^T Q).
//
// The vector-ALU float32 backward, for the head sizes the float32 MFMA
// kernels do not take (any d other than 64 and 128), with the 16-bit
// backward's two-kernel shape and no atomics.  The first kernel owns a tile
// of query rows: it forms D for them (kept in the workspace for the second)
// and walks the key tiles the mask leaves visible, accumulating dQ in
// registers.  The second owns a tile of keys and walks the query tiles that
// see them, accumulating dK and dV.  Everything is plain float32 FMAs on tiles
// staged in LDS, the head dimension padded to a multiple of 4 with zeros
// (which add exact zeros): 64 x 64 tiles with a 4 x 4 block of scores per
// thread for d <= 128, 32 x 32 tiles with 2 x 2 up to d = 256.  Every output
// is written once, so repeated calls give identical bits.
#include "fa_launch.h"
#include "fp32_tile.h"

namespace fa {
namespace {

using namespace fp32;

// L as the recompute uses it: a row that saw no key (L = -inf) gets P = 0.
__device__ inline float row_l(float L) { return L == kNegInf ? __builtin_inff() : L; }

// dQ for one tile of TB query rows, and D of those rows into Dws.
template <int TB, int DM>
__global__ __launch_bounds__(kThreads) void bwd_fp32_dq_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ o, const float* __restrict__ dO, const float* __restrict__ lse,
    float* __restrict__ Dws, float* __restrict__ dq, int N, int d, int nt, float scale, int causal,
    int window) {
  using F = Tile<TB, DM>;
  constexpr int R = F::R, P = F::kPitch, SP = F::kSPitch;
  __shared__ __align__(16) float Qs[TB * P];
  __shared__ __align__(16) float Gs[TB * P];
  __shared__ __align__(16) float Ks[TB * P];
  __shared__ __align__(16) float Vs[TB * P];
  __shared__ float Ts[TB * SP];
  __shared__ float Lr[TB], Dr[TB];

  const int t = threadIdx.x, ti = t >> 4, tj = t & 15;
  const int bh = blockIdx.x / nt;
  const int q0 = (blockIdx.x - bh * nt) * TB;
  const size_t base = (size_t)bh * N * d;
  const size_t rbase = (size_t)bh * N;
  const int dpad = (d + 3) & ~3;

  stage<TB, P>(Qs, q + base, q0, min(TB, N - q0), d, dpad);
  stage<TB, P>(Gs, dO + base, q0, min(TB, N - q0), d, dpad);
  __syncthreads();
  {
    // D_i = dO_i . O_i: G neighbouring lanes per row, then a butterfly.
    constexpr int G = kThreads / TB;
    const int r = t / G, part = t - r * G;
    const bool in = q0 + r < N;
    float acc = 0.f;
    if (in)
      for (int e = part; e < d; e += G) acc = __builtin_fmaf(Gs[r * P + e], o[base + (size_t)(q0 + r) * d + e], acc);
#pragma unroll
    for (int m = 1; m < G; m <<= 1) acc += __shfl_xor(acc, m);
    if (part == 0) {
      Dr[r] = acc;
      Lr[r] = row_l(in ? lse[rbase + q0 + r] : kNegInf);
      if (in) Dws[rbase + q0 + r] = acc;
    }
  }

  const int qlast = min(q0 + TB, N) - 1;
  const int kmin = window >= 0 ? max(0, q0 - window) : 0;
  const int kmax = causal ? qlast : N - 1;
  float4 acc[R][F::kChunks];
  zero<TB, DM>(acc);

  for (int kt = kmin / TB; kt <= kmax / TB; ++kt) {
    const int k0 = kt * TB;
    __syncthreads();  // the previous tile's readers are done (and Dr / Lr are written)
    stage<TB, P>(Ks, k + base, k0, min(TB, N - k0), d, dpad);
    stage<TB, P>(Vs, v + base, k0, min(TB, N - k0), d, dpad);
    __syncthreads();
    float sd[2][R][R];
    dot_blocks<TB, DM, 2>(Qs, Ks, Gs, Vs, dpad, ti, tj, sd);
    float (&s)[R][R] = sd[0];
    float (&dp)[R][R] = sd[1];
#pragma unroll
    for (int a = 0; a < R; ++a) {
      const int i = ti + 16 * a;
#pragma unroll
      for (int b = 0; b < R; ++b) {
        const int j = tj + 16 * b;
        float ds = 0.f;
        if (visible(q0 + i, k0 + j, N, causal, window)) {
          const float p = expf(__builtin_fmaf(s[a][b], scale, -Lr[i]));
          ds = p * (dp[a][b] - Dr[i]);
        }
        Ts[j * SP + i] = ds;  // [key][query]: the accumulation walks keys
      }
    }
    __syncthreads();
    accumulate<TB, DM>(Ts, Ks, min(TB, N - k0), dpad, ti, tj, acc);
  }
  float mul[R];
#pragma unroll
  for (int a = 0; a < R; ++a) mul[a] = scale;
  store_rows<TB, DM>(dq + base, acc, mul, q0, min(TB, N - q0), d, ti, tj);
}

// dK and dV for one tile of TB keys.
template <int TB, int DM>
__global__ __launch_bounds__(kThreads) void bwd_fp32_kv_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ Dws,
    float* __restrict__ dk, float* __restrict__ dv, int N, int d, int nt, float scale, int causal, int window) {
  using F = Tile<TB, DM>;
  constexpr int R = F::R, P = F::kPitch, SP = F::kSPitch;
  __shared__ __align__(16) float Qs[TB * P];
  __shared__ __align__(16) float Gs[TB * P];
  __shared__ __align__(16) float Ks[TB * P];
  __shared__ __align__(16) float Vs[TB * P];
  __shared__ float Ts[TB * SP];
  __shared__ float Lr[TB], Dr[TB];

  const int t = threadIdx.x, ti = t >> 4, tj = t & 15;
  const int bh = blockIdx.x / nt;
  const int k0 = (blockIdx.x - bh * nt) * TB;
  const size_t base = (size_t)bh * N * d;
  const size_t rbase = (size_t)bh * N;
  const int dpad = (d + 3) & ~3;

  stage<TB, P>(Ks, k + base, k0, min(TB, N - k0), d, dpad);
  stage<TB, P>(Vs, v + base, k0, min(TB, N - k0), d, dpad);

  const int klast = min(k0 + TB, N) - 1;
  const int qmin = causal ? k0 : 0;
  const int qmax = window >= 0 ? min(N - 1, klast + window) : N - 1;
  float4 ak[R][F::kChunks], av[R][F::kChunks];
  zero<TB, DM>(ak);
  zero<TB, DM>(av);

  for (int qt = qmin / TB; qt <= qmax / TB; ++qt) {
    const int q0 = qt * TB;
    __syncthreads();  // the previous tile's readers are done
    stage<TB, P>(Qs, q + base, q0, min(TB, N - q0), d, dpad);
    stage<TB, P>(Gs, dO + base, q0, min(TB, N - q0), d, dpad);
    if (t < TB) {
      const bool in = q0 + t < N;
      Lr[t] = row_l(in ? lse[rbase + q0 + t] : kNegInf);
      Dr[t] = in ? Dws[rbase + q0 + t] : 0.f;
    }
    __syncthreads();
    float sd[2][R][R];
    dot_blocks<TB, DM, 2>(Qs, Ks, Gs, Vs, dpad, ti, tj, sd);
    float (&s)[R][R] = sd[0];
    float (&dp)[R][R] = sd[1];
#pragma unroll
    for (int a = 0; a < R; ++a) {
      const int i = ti + 16 * a;
#pragma unroll
      for (int b = 0; b < R; ++b) {
        const int j = tj + 16 * b;
        float p = 0.f, ds = 0.f;
        if (visible(q0 + i, k0 + j, N, causal, window)) {
          p = expf(__builtin_fmaf(s[a][b], scale, -Lr[i]));
          ds = p * (dp[a][b] - Dr[i]);
        }
        Ts[i * SP + j] = p;  // [query][key]: the accumulation walks queries
        dp[a][b] = ds;
      }
    }
    const int nq = min(TB, N - q0);
    __syncthreads();
    accumulate<TB, DM>(Ts, Gs, nq, dpad, ti, tj, av);  // dV_j += P_ij dO_i
    __syncthreads();
#pragma unroll
    for (int a = 0; a < R; ++a)
#pragma unroll
      for (int b = 0; b < R; ++b) Ts[(ti + 16 * a) * SP + tj + 16 * b] = dp[a][b];
    __syncthreads();
    accumulate<TB, DM>(Ts, Qs, nq, dpad, ti, tj, ak);  // dK_j += dS_ij Q_i
  }
  float mul[R];
#pragma unroll
  for (int a = 0; a < R; ++a) mul[a] = scale;
  store_rows<TB, DM>(dk + base, ak, mul, k0, min(TB, N - k0), d, ti, tj);
#pragma unroll
  for (int a = 0; a < R; ++a) mul[a] = 1.f;
  store_rows<TB, DM>(dv + base, av, mul, k0, min(TB, N - k0), d, ti, tj);
}

template <int TB, int DM>
hipError_t launch_t(const float* q, const float* k, const float* v, const float* o, const float* dO,
                    const float* lse, float* dq, float* dk, float* dv, int B, int H, int N, int d,
                    float scale, Mask mask, float* Dws, hipStream_t stream) {
  const int nt = (N + TB - 1) / TB;
  const unsigned grid = (unsigned)((long long)nt * B * H);
  // dQ first: it also leaves D of every query row in the workspace.
  hipLaunchKernelGGL((bwd_fp32_dq_kernel<TB, DM>), dim3(grid), dim3(kThreads), 0, stream, q, k, v, o, dO, lse,
                     Dws, dq, N, d, nt, scale, mask.causal, mask.window);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((bwd_fp32_kv_kernel<TB, DM>), dim3(grid), dim3(kThreads), 0, stream, q, k, v, dO, lse,
                     Dws, dk, dv, N, d, nt, scale, mask.causal, mask.window);
  return hipGetLastError();
}

}  // namespace

int bwd_fp32_tile(int d) { return d <= 128 ? 64 : 32; }

hipError_t launch_bwd_fp32(const float* q, const float* k, const float* v, const float* o, const float* dO,
                           const float* lse, float* dq, float* dk, float* dv, int B, int H, int N, int d,
                           float scale, Mask mask, void* ws, hipStream_t stream) {
  float* Dws = (float*)ws;
  if (d <= 128) return launch_t<64, 128>(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, mask, Dws, stream);
  return launch_t<32, 256>(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, mask, Dws, stream);
}

}  // namespace fa
