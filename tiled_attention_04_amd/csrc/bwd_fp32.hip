// Float32 backward: dQ, dK and dV recomputed from the stored L for any head
// size 1 <= d <= 256 ("Building Flash Attention from Scratch in Pure NumPy",
// Step 4: D = rowsum(dO * O), P = exp(scale * Q K^T - L), dV = P^T dO,
// dP = dO V^T, dS = P * (dP - D), dQ = scale * dS K, dK = scale * dS^T Q).
//
// The float32 companion of the 16-bit MFMA backward, with the same two-kernel
// shape and no atomics.  The first kernel owns a tile of query rows: it forms
// D for them (kept in the workspace for the second) and walks the key tiles
// the mask leaves visible, accumulating dQ in registers.  The second owns a
// tile of keys and walks the query tiles that see them, accumulating dK and
// dV.  Everything is plain float32 FMAs on tiles staged in LDS, the head
// dimension padded to a multiple of 4 with zeros (which add exact zeros):
// 64 x 64 tiles with a 4 x 4 block of scores per thread for d <= 128,
// 32 x 32 tiles with 2 x 2 up to d = 256.  Every output is written once, so
// repeated calls give identical bits.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kThreads = 256;  // 16 x 16 threads over a score tile

template <int TB, int DM>
struct Fp32Tile {
  static constexpr int R = TB / 16;       // rows (and columns) of a thread's score block
  static constexpr int kPitch = DM + 4;   // floats per staged row: float4-aligned, rows 16 B apart mod 256 B
  static constexpr int kSPitch = TB + 1;  // pitch of the score tile
  static constexpr int kChunks = DM / 64; // float4 column chunks a thread accumulates per output row
  static_assert(kChunks >= 1 && R >= 1, "tile shape");
};

__device__ inline bool visible(int qi, int kj, int N, int causal, int window) {
  return qi < N && kj < N && (!causal || kj <= qi) && (window < 0 || kj >= qi - window);
}

// L as the recompute uses it: a row that saw no key (L = -inf) gets P = 0.
__device__ inline float row_l(float L) { return L == kNegInf ? __builtin_inff() : L; }

// Rows [r0, r0 + TB) of one [N, d] float32 slice into LDS with pitch P;
// columns d..dpad-1 and rows at or past N read as zero.
template <int TB, int P>
__device__ inline void stage(float* dst, const float* __restrict__ src, int r0, int N, int d, int dpad) {
  for (int i = threadIdx.x; i < TB * dpad; i += kThreads) {
    const int r = i / dpad, c = i - r * dpad;
    dst[r * P + c] = (r0 + r < N && c < d) ? src[(size_t)(r0 + r) * d + c] : 0.f;
  }
}

__device__ inline const float4& at4(const float* p) { return *reinterpret_cast<const float4*>(p); }

// s[a][b] = Q_i . K_j and dp[a][b] = dO_i . V_j for the thread's query rows
// i = ti + 16a and keys j = tj + 16b, summed in ascending head index.
template <int TB, int DM>
__device__ inline void score_block(const float* Qs, const float* Gs, const float* Ks, const float* Vs, int dpad,
                                   int ti, int tj, float (&s)[TB / 16][TB / 16], float (&dp)[TB / 16][TB / 16]) {
  constexpr int R = Fp32Tile<TB, DM>::R, P = Fp32Tile<TB, DM>::kPitch;
#pragma unroll
  for (int a = 0; a < R; ++a)
#pragma unroll
    for (int b = 0; b < R; ++b) s[a][b] = dp[a][b] = 0.f;
  for (int e = 0; e < dpad; e += 4) {
    float4 qv[R], gv[R];
#pragma unroll
    for (int a = 0; a < R; ++a) {
      qv[a] = at4(Qs + (ti + 16 * a) * P + e);
      gv[a] = at4(Gs + (ti + 16 * a) * P + e);
    }
#pragma unroll
    for (int b = 0; b < R; ++b) {
      const float4 kv = at4(Ks + (tj + 16 * b) * P + e);
      const float4 vv = at4(Vs + (tj + 16 * b) * P + e);
#pragma unroll
      for (int a = 0; a < R; ++a) {
        s[a][b] = __builtin_fmaf(qv[a].x, kv.x, s[a][b]);
        s[a][b] = __builtin_fmaf(qv[a].y, kv.y, s[a][b]);
        s[a][b] = __builtin_fmaf(qv[a].z, kv.z, s[a][b]);
        s[a][b] = __builtin_fmaf(qv[a].w, kv.w, s[a][b]);
        dp[a][b] = __builtin_fmaf(gv[a].x, vv.x, dp[a][b]);
        dp[a][b] = __builtin_fmaf(gv[a].y, vv.y, dp[a][b]);
        dp[a][b] = __builtin_fmaf(gv[a].z, vv.z, dp[a][b]);
        dp[a][b] = __builtin_fmaf(gv[a].w, vv.w, dp[a][b]);
      }
    }
  }
}

// acc[a][c] += sum over n < nrows of W[n][row_a] * X[n][chunk_c], where the
// thread's output rows are row_a = ti + 16a and its columns the float4 chunks
// tj + 16c (W: score tile, pitch TB + 1, indexed [n][row]; X: staged rows).
template <int TB, int DM>
__device__ inline void accumulate(const float* Ws, const float* Xs, int nrows, int dpad, int ti, int tj,
                                  float4 (&acc)[TB / 16][DM / 64]) {
  using F = Fp32Tile<TB, DM>;
  constexpr int R = F::R, C = F::kChunks, P = F::kPitch, SP = F::kSPitch;
  for (int n = 0; n < nrows; ++n) {
    float w[R];
#pragma unroll
    for (int a = 0; a < R; ++a) w[a] = Ws[n * SP + ti + 16 * a];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int e0 = 4 * (tj + 16 * c);
      if (e0 < dpad) {
        const float4 x = at4(Xs + n * P + e0);
#pragma unroll
        for (int a = 0; a < R; ++a) {
          acc[a][c].x = __builtin_fmaf(w[a], x.x, acc[a][c].x);
          acc[a][c].y = __builtin_fmaf(w[a], x.y, acc[a][c].y);
          acc[a][c].z = __builtin_fmaf(w[a], x.z, acc[a][c].z);
          acc[a][c].w = __builtin_fmaf(w[a], x.w, acc[a][c].w);
        }
      }
    }
  }
}

// Rows r0 + ti + 16a (< N) of one [N, d] float32 slice from acc * mul.
template <int TB, int DM>
__device__ inline void store_rows(float* __restrict__ dst, const float4 (&acc)[TB / 16][DM / 64], float mul,
                                  int r0, int N, int d, int ti, int tj) {
  using F = Fp32Tile<TB, DM>;
#pragma unroll
  for (int a = 0; a < F::R; ++a) {
    const int r = r0 + ti + 16 * a;
    if (r >= N) continue;
    float* row = dst + (size_t)r * d;
#pragma unroll
    for (int c = 0; c < F::kChunks; ++c) {
      const int e0 = 4 * (tj + 16 * c);
      const float vals[4] = {acc[a][c].x, acc[a][c].y, acc[a][c].z, acc[a][c].w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (e0 + u < d) row[e0 + u] = vals[u] * mul;
    }
  }
}

// dQ for one tile of TB query rows, and D of those rows into Dws.
template <int TB, int DM>
__global__ __launch_bounds__(kThreads) void bwd_fp32_dq_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ o, const float* __restrict__ dO, const float* __restrict__ lse,
    float* __restrict__ Dws, float* __restrict__ dq, int N, int d, int nt, float scale, int causal,
    int window) {
  using F = Fp32Tile<TB, DM>;
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

  stage<TB, P>(Qs, q + base, q0, N, d, dpad);
  stage<TB, P>(Gs, dO + base, q0, N, d, dpad);
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
#pragma unroll
  for (int a = 0; a < R; ++a)
#pragma unroll
    for (int c = 0; c < F::kChunks; ++c) acc[a][c] = make_float4(0.f, 0.f, 0.f, 0.f);

  for (int kt = kmin / TB; kt <= kmax / TB; ++kt) {
    const int k0 = kt * TB;
    __syncthreads();  // the previous tile's readers are done (and Dr / Lr are written)
    stage<TB, P>(Ks, k + base, k0, N, d, dpad);
    stage<TB, P>(Vs, v + base, k0, N, d, dpad);
    __syncthreads();
    float s[R][R], dp[R][R];
    score_block<TB, DM>(Qs, Gs, Ks, Vs, dpad, ti, tj, s, dp);
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
  store_rows<TB, DM>(dq + base, acc, scale, q0, N, d, ti, tj);
}

// dK and dV for one tile of TB keys.
template <int TB, int DM>
__global__ __launch_bounds__(kThreads) void bwd_fp32_kv_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ Dws,
    float* __restrict__ dk, float* __restrict__ dv, int N, int d, int nt, float scale, int causal, int window) {
  using F = Fp32Tile<TB, DM>;
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

  stage<TB, P>(Ks, k + base, k0, N, d, dpad);
  stage<TB, P>(Vs, v + base, k0, N, d, dpad);

  const int klast = min(k0 + TB, N) - 1;
  const int qmin = causal ? k0 : 0;
  const int qmax = window >= 0 ? min(N - 1, klast + window) : N - 1;
  float4 ak[R][F::kChunks], av[R][F::kChunks];
#pragma unroll
  for (int a = 0; a < R; ++a)
#pragma unroll
    for (int c = 0; c < F::kChunks; ++c) ak[a][c] = av[a][c] = make_float4(0.f, 0.f, 0.f, 0.f);

  for (int qt = qmin / TB; qt <= qmax / TB; ++qt) {
    const int q0 = qt * TB;
    __syncthreads();  // the previous tile's readers are done
    stage<TB, P>(Qs, q + base, q0, N, d, dpad);
    stage<TB, P>(Gs, dO + base, q0, N, d, dpad);
    if (t < TB) {
      const bool in = q0 + t < N;
      Lr[t] = row_l(in ? lse[rbase + q0 + t] : kNegInf);
      Dr[t] = in ? Dws[rbase + q0 + t] : 0.f;
    }
    __syncthreads();
    float s[R][R], dp[R][R];
    score_block<TB, DM>(Qs, Gs, Ks, Vs, dpad, ti, tj, s, dp);
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
  store_rows<TB, DM>(dk + base, ak, scale, k0, N, d, ti, tj);
  store_rows<TB, DM>(dv + base, av, 1.f, k0, N, d, ti, tj);
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
