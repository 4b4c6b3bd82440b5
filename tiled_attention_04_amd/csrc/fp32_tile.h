// Building blocks of the float32 kernels (forward and backward): square
// tiles of TB rows staged in LDS with the head dimension padded to a multiple
// of 4 (zeros, which add exact zeros), a 16 x 16 grid of threads over a
// TB x TB score tile with an R x R block of scores per thread (rows
// ti + 16a, columns tj + 16b), and row accumulators of TB x DM outputs with
// R rows and DM / 64 float4 column chunks (tj + 16c) per thread.  Everything
// is plain float32 FMAs; the float4 LDS reads of 16 different rows are 16 B
// apart modulo 256 B (row pitch DM + 4 floats), so each fills the banks once.
#pragma once

#include "fa_common.h"

namespace fa {
namespace fp32 {

constexpr int kThreads = 256;

template <int TB, int DM>
struct Tile {
  static constexpr int R = TB / 16;       // rows (and columns) of a thread's score block
  static constexpr int kPitch = DM + 4;   // floats per staged row
  static constexpr int kSPitch = TB + 1;  // pitch of a score tile in LDS
  static constexpr int kChunks = DM / 64; // float4 column chunks per accumulated row
  static_assert(kChunks >= 1 && R >= 1 && TB <= 64, "tile shape");
};

__device__ inline bool visible(int qi, int kj, int N, int causal, int window) {
  return qi < N && kj < N && (!causal || kj <= qi) && (window < 0 || kj >= qi - window);
}

__device__ inline const float4& at4(const float* p) { return *reinterpret_cast<const float4*>(p); }

// Rows [r0, r0 + nrows) of one [N, d] float32 slice into the first rows of a
// TB-row LDS tile (pitch P); columns d..dpad-1 and rows from nrows on are zero.
template <int TB, int P>
__device__ inline void stage(float* dst, const float* __restrict__ src, int r0, int nrows, int d, int dpad) {
  for (int i = threadIdx.x; i < TB * dpad; i += kThreads) {
    const int r = i / dpad, c = i - r * dpad;
    dst[r * P + c] = (r < nrows && c < d) ? src[(size_t)(r0 + r) * d + c] : 0.f;
  }
}

// s[p][a][b] = X_p[ti + 16a] . Y_p[tj + 16b] for NP pairs (X0, Y0), (X1, Y1)
// of staged tiles, summed in ascending head index.
template <int TB, int DM, int NP>
__device__ inline void dot_blocks(const float* X0, const float* Y0, const float* X1, const float* Y1, int dpad,
                                  int ti, int tj, float (&s)[NP][TB / 16][TB / 16]) {
  constexpr int R = Tile<TB, DM>::R, P = Tile<TB, DM>::kPitch;
  const float* X[2] = {X0, X1};
  const float* Y[2] = {Y0, Y1};
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int a = 0; a < R; ++a)
#pragma unroll
      for (int b = 0; b < R; ++b) s[p][a][b] = 0.f;
  for (int e = 0; e < dpad; e += 4) {
    float4 xv[NP][R];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int a = 0; a < R; ++a) xv[p][a] = at4(X[p] + (ti + 16 * a) * P + e);
#pragma unroll
    for (int b = 0; b < R; ++b) {
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const float4 y = at4(Y[p] + (tj + 16 * b) * P + e);
#pragma unroll
        for (int a = 0; a < R; ++a) {
          float acc = s[p][a][b];
          acc = __builtin_fmaf(xv[p][a].x, y.x, acc);
          acc = __builtin_fmaf(xv[p][a].y, y.y, acc);
          acc = __builtin_fmaf(xv[p][a].z, y.z, acc);
          acc = __builtin_fmaf(xv[p][a].w, y.w, acc);
          s[p][a][b] = acc;
        }
      }
    }
  }
}

// acc[a][c] += sum over n < nrows of W[n][row_a] * X[n][chunk_c]: the
// thread's output rows row_a = ti + 16a, its columns the float4 chunks
// tj + 16c (W: a score tile indexed [n][row]; X: staged rows).
template <int TB, int DM>
__device__ inline void accumulate(const float* Ws, const float* Xs, int nrows, int dpad, int ti, int tj,
                                  float4 (&acc)[TB / 16][DM / 64]) {
  using F = Tile<TB, DM>;
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

template <int TB, int DM>
__device__ inline void zero(float4 (&acc)[TB / 16][DM / 64]) {
#pragma unroll
  for (int a = 0; a < TB / 16; ++a)
#pragma unroll
    for (int c = 0; c < DM / 64; ++c) acc[a][c] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// Rows r0 + ti + 16a (for ti + 16a < nrows) of one [N, d] float32 slice from
// acc[a] * mul[a].
template <int TB, int DM>
__device__ inline void store_rows(float* __restrict__ dst, const float4 (&acc)[TB / 16][DM / 64],
                                  const float (&mul)[TB / 16], int r0, int nrows, int d, int ti, int tj) {
  using F = Tile<TB, DM>;
#pragma unroll
  for (int a = 0; a < F::R; ++a) {
    const int r = ti + 16 * a;
    if (r >= nrows) continue;
    float* row = dst + (size_t)(r0 + r) * d;
#pragma unroll
    for (int c = 0; c < F::kChunks; ++c) {
      const int e0 = 4 * (tj + 16 * c);
      const float vals[4] = {acc[a][c].x, acc[a][c].y, acc[a][c].z, acc[a][c].w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (e0 + u < d) row[e0 + u] = vals[u] * mul[a];
    }
  }
}

// Butterflies over the 16 lanes of one score row (lanes ti * 16 + tj).
__device__ inline float row_max16(float x) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}
__device__ inline float row_sum16(float x) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

}  // namespace fp32
}  // namespace fa
