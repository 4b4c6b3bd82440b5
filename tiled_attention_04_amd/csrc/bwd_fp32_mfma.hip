// Float32 backward on the matrix cores (v_mfma_f32_32x32x2_f32: float32
// products and sums), head sizes 64 and 128 ("Building Flash Attention from
// Scratch in Pure NumPy", Step 4: D = rowsum(dO * O), P = exp(scale Q K^T - L),
// dV = P^T dO, dP = dO V^T, dS = P * (dP - D), dQ = scale dS K,
// dK = scale dS^T Q).  The two-kernel shape of the 16-bit backward, no
// atomics: the dQ kernel first (it also stores D and L in log2 units for
// every query row), then the dK / dV kernel.
//
// In both kernels a lane keeps half of one row of each operand it contracts
// over the head dimension in registers (MFMA step j contracts head columns
// h * D / 2 + j of both operands, h the half-wave), and the 32 x 32 results
// come in the accumulator layout: one column per lane, 16 rows.  That layout
// is already the B operand of the second products, two rows per step taken
// from the register both half-waves hold, so P and dS never leave the lane:
//  * dQ kernel (a wave owns 32 query rows, Q and dO rows in registers):
//    S^T = K Q^T and dP^T = V dO^T hold one query and 16 keys per lane, and
//    dQ^T += K^T dS^T reads K's rows of those keys from LDS;
//  * dK / dV kernel (a wave owns 32 keys, K and V rows in registers):
//    S = Q K^T and dP = dO V^T hold one key and 16 queries per lane, and
//    dV^T += dO^T P, dK^T += Q^T dS read the rows of those queries from LDS.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;  // query rows (dQ) or keys (dK / dV) per workgroup
constexpr int kStep = 32;           // keys (dQ) or query rows (dK / dV) per step

template <int D>
struct B32 {
  static constexpr int H = D / 2;                      // head columns per half-wave
  static constexpr int CB = D / 32;                    // 32-row blocks of dQ^T, dK^T, dV^T
  static constexpr int RP = D + 4;                     // rows read 16 B at a time along the row
  static constexpr int XP = D + 8;                     // rows also read across (the half-waves 4 rows apart)
  static constexpr int LD = kStep * D / 4 / kThreads;  // float4 loads per thread per staged tile
};

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Half of row `row` of one [N, D] slice (columns h * D / 2 ..), zeros past N.
template <int D>
__device__ __forceinline__ void load_half_row(const float* __restrict__ slice, int row, int N, int h,
                                              float (&dst)[D / 2]) {
  const bool in = row < N;
  const float4* src = reinterpret_cast<const float4*>(slice + (size_t)(in ? row : 0) * D + h * (D / 2));
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const float4 x = in ? src[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    dst[4 * c] = x.x;
    dst[4 * c + 1] = x.y;
    dst[4 * c + 2] = x.z;
    dst[4 * c + 3] = x.w;
  }
}

// Two [kStep, D] row tiles of one slice from row r0 (rows past N zero):
// loaded into registers, then stored into LDS with pitches PA and PB.
template <int D>
struct TilePair {
  float4 a[B32<D>::LD], b[B32<D>::LD];
  __device__ __forceinline__ void load(const float* __restrict__ sa, const float* __restrict__ sb, int r0, int N) {
#pragma unroll
    for (int u = 0; u < B32<D>::LD; ++u) {
      const int i = threadIdx.x + kThreads * u, row = i / (D / 4), c4 = i - row * (D / 4);
      const bool in = r0 + row < N;
      const size_t off = (size_t)(in ? r0 + row : 0) * D + 4 * c4;
      a[u] = in ? *reinterpret_cast<const float4*>(sa + off) : make_float4(0.f, 0.f, 0.f, 0.f);
      b[u] = in ? *reinterpret_cast<const float4*>(sb + off) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  template <int PA, int PB>
  __device__ __forceinline__ void store(float* da, float* db) const {
#pragma unroll
    for (int u = 0; u < B32<D>::LD; ++u) {
      const int i = threadIdx.x + kThreads * u, row = i / (D / 4), c4 = i - row * (D / 4);
      *reinterpret_cast<float4*>(da + row * PA + 4 * c4) = a[u];
      *reinterpret_cast<float4*>(db + row * PB + 4 * c4) = b[u];
    }
  }
};

// Rows of the 32 x D result a lane holds in the accumulator layout (row
// `row`, columns 32 cb + c_row(r, h)) to one [N, D] slice, times mul.
template <int D>
__device__ __forceinline__ void store_row(float* __restrict__ slice, int row, int h, const f32x16 (&acc)[D / 32],
                                          float mul) {
  float* dst = slice + (size_t)row * D;
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<float4*>(dst + 32 * cb + 8 * g + 4 * h) =
          make_float4(acc[cb][4 * g] * mul, acc[cb][4 * g + 1] * mul, acc[cb][4 * g + 2] * mul,
                      acc[cb][4 * g + 3] * mul);
}

__device__ __forceinline__ bool visible(int qi, int kj, int N, int causal, int window) {
  return qi < N && kj < N && (!causal || kj <= qi) && (window < 0 || kj >= qi - window);
}

// dQ for 128 query rows, and D and L2 = L log2(e) of those rows.
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_f32_dq_kernel(const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
                       const float* __restrict__ o, const float* __restrict__ dO, const float* __restrict__ lse,
                       float* __restrict__ Dv, float* __restrict__ L2, float* __restrict__ dq, int BH, int N,
                       int nqt, float scale, float c_log2, int causal, int window) {
  using C = B32<D>;
  __shared__ __align__(16) float Ks[2][kStep * C::XP];
  __shared__ __align__(16) float Vs[2][kStep * C::RP];

  const int t = threadIdx.x;
  const int lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  int bh, qr;
  tile_order(blockIdx.x, BH, nqt, causal && window < 0, bh, qr);  // heaviest causal tile first
  const int qt = causal ? nqt - 1 - qr : qr;
  const int q0 = qt * kRows;
  const size_t base = (size_t)bh * (size_t)N * D;
  const int wq0 = q0 + 32 * w;
  const int my_q = wq0 + l32;
  const bool q_in = my_q < N;

  float qv[C::H], gv[C::H];
  load_half_row<D>(q + base, my_q, N, h, qv);
  load_half_row<D>(dO + base, my_q, N, h, gv);
  float Di, Li;
  {
    float ov[C::H];
    load_half_row<D>(o + base, my_q, N, h, ov);
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < C::H; ++j) acc = __builtin_fmaf(gv[j], ov[j], acc);
    Di = pair_sum(acc);
    const float L = q_in ? lse[(size_t)bh * N + my_q] : kNegInf;
    Li = L == kNegInf ? __builtin_inff() : L * kLog2e;  // a row without keys: every P is 0
  }

  const int q_last = min(q0 + kRows, N) - 1;
  const int kmin = window >= 0 ? max(0, q0 - window) : 0;
  const int kmax = causal ? q_last : N - 1;
  const int kt0 = kmin / kStep, kt1 = kmax / kStep + 1;

  f32x16 dqa[C::CB];
#pragma unroll
  for (int cb = 0; cb < C::CB; ++cb) dqa[cb] = f32x16{};
  TilePair<D> kvt;
  if (kt0 < kt1) {
    kvt.load(k + base, v + base, kt0 * kStep, N);
    kvt.template store<C::XP, C::RP>(Ks[0], Vs[0]);
  }
  __syncthreads();
  for (int kt = kt0; kt < kt1; ++kt) {
    const int buf = (kt - kt0) & 1;
    const bool more = kt + 1 < kt1;
    if (more) kvt.load(k + base, v + base, (kt + 1) * kStep, N);
    const int k0 = kt * kStep;
    const bool act = wq0 < N && !(causal && k0 > wq0 + 31) && !(window >= 0 && k0 + kStep - 1 < wq0 - window);
    if (act) {
      const float* Kb = Ks[buf];
      const float* Vb = Vs[buf];
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
      for (int c = 0; c < C::H / 4; ++c) {
        const float4 kk = *reinterpret_cast<const float4*>(Kb + l32 * C::XP + h * C::H + 4 * c);
        const float4 vv = *reinterpret_cast<const float4*>(Vb + l32 * C::RP + h * C::H + 4 * c);
        sacc = mfma_f32(kk.x, qv[4 * c], sacc);
        dpacc = mfma_f32(vv.x, gv[4 * c], dpacc);
        sacc = mfma_f32(kk.y, qv[4 * c + 1], sacc);
        dpacc = mfma_f32(vv.y, gv[4 * c + 1], dpacc);
        sacc = mfma_f32(kk.z, qv[4 * c + 2], sacc);
        dpacc = mfma_f32(vv.z, gv[4 * c + 2], dpacc);
        sacc = mfma_f32(kk.w, qv[4 * c + 3], sacc);
        dpacc = mfma_f32(vv.w, gv[4 * c + 3], dpacc);
      }
      // Lane: query my_q, keys k0 + c_row(r, h).
      const bool need_mask = (causal && k0 + kStep - 1 > wq0) || (window >= 0 && wq0 + 31 - k0 > window) ||
                             k0 + kStep > N || wq0 + 32 > N;
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c_log2, -Li));
        if (need_mask) p = visible(my_q, k0 + c_row(r, h), N, causal, window) ? p : 0.f;
        ds[r] = p * (dpacc[r] - Di);
      }
      // dQ^T += K^T dS^T: step j takes keys c_row(j, 0) and c_row(j, 1).
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float* krow = Kb + c_row(j, h) * C::XP + l32;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) dqa[cb] = mfma_f32(krow[32 * cb], ds[j], dqa[cb]);
      }
    }
    if (more) kvt.template store<C::XP, C::RP>(Ks[buf ^ 1], Vs[buf ^ 1]);  // its readers passed the last barrier
    __syncthreads();
  }
  if (q_in) {
    store_row<D>(dq + base, my_q, h, dqa, scale);
    if (h == 0) {
      Dv[(size_t)bh * N + my_q] = Di;
      L2[(size_t)bh * N + my_q] = Li;
    }
  }
}

// dK and dV for 128 keys.
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_f32_kv_kernel(const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
                       const float* __restrict__ dO, const float* __restrict__ Dv, const float* __restrict__ L2,
                       float* __restrict__ dk, float* __restrict__ dv, int BH, int N, int nkt, float scale,
                       float c_log2, int causal, int window) {
  using C = B32<D>;
  __shared__ __align__(16) float Qs[2][kStep * C::XP];
  __shared__ __align__(16) float Gs[2][kStep * C::XP];
  __shared__ float Ls[2][kStep], Ds[2][kStep];

  const int t = threadIdx.x;
  const int lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  int bh, kt;
  tile_order(blockIdx.x, BH, nkt, causal && window < 0, bh, kt);  // heaviest causal tile (kt = 0) first
  const int k0 = kt * kRows;
  const size_t base = (size_t)bh * (size_t)N * D;
  const int wk0 = k0 + 32 * w;
  const int my_key = wk0 + l32;

  float kv[C::H], vv[C::H];
  load_half_row<D>(k + base, my_key, N, h, kv);
  load_half_row<D>(v + base, my_key, N, h, vv);

  const int k_last = min(k0 + kRows, N) - 1;
  const int qmin = causal ? k0 : 0;
  const int qmax = window >= 0 ? min(N - 1, k_last + window) : N - 1;
  const int qt0 = qmin / kStep, qt1 = qmax / kStep + 1;
  const float* Lrow = L2 + (size_t)bh * N;
  const float* Drow = Dv + (size_t)bh * N;

  f32x16 dka[C::CB], dva[C::CB];
#pragma unroll
  for (int cb = 0; cb < C::CB; ++cb) {
    dka[cb] = f32x16{};
    dva[cb] = f32x16{};
  }
  TilePair<D> qgt;
  float ld = 0.f;  // L2 (t < 32) or D (32 <= t < 64) of one row of the next step
  auto load_ld = [&](int r0) {
    if (t < 2 * kStep) {
      const int row = r0 + (t & (kStep - 1));
      ld = row < N ? (t < kStep ? Lrow[row] : Drow[row]) : 0.f;
    }
  };
  auto store_ld = [&](int b) {
    if (t < kStep) Ls[b][t] = ld;
    else if (t < 2 * kStep) Ds[b][t - kStep] = ld;
  };
  if (qt0 < qt1) {
    qgt.load(q + base, dO + base, qt0 * kStep, N);
    load_ld(qt0 * kStep);
    qgt.template store<C::XP, C::XP>(Qs[0], Gs[0]);
    store_ld(0);
  }
  __syncthreads();
  for (int qt = qt0; qt < qt1; ++qt) {
    const int buf = (qt - qt0) & 1;
    const bool more = qt + 1 < qt1;
    if (more) {
      qgt.load(q + base, dO + base, (qt + 1) * kStep, N);
      load_ld((qt + 1) * kStep);
    }
    const int q0 = qt * kStep;
    const bool act = wk0 < N && !(causal && wk0 > q0 + kStep - 1) && !(window >= 0 && wk0 + 31 < q0 - window);
    if (act) {
      const float* Qb = Qs[buf];
      const float* Gb = Gs[buf];
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
      for (int c = 0; c < C::H / 4; ++c) {
        const float4 qq = *reinterpret_cast<const float4*>(Qb + l32 * C::XP + h * C::H + 4 * c);
        const float4 gg = *reinterpret_cast<const float4*>(Gb + l32 * C::XP + h * C::H + 4 * c);
        sacc = mfma_f32(qq.x, kv[4 * c], sacc);
        dpacc = mfma_f32(gg.x, vv[4 * c], dpacc);
        sacc = mfma_f32(qq.y, kv[4 * c + 1], sacc);
        dpacc = mfma_f32(gg.y, vv[4 * c + 1], dpacc);
        sacc = mfma_f32(qq.z, kv[4 * c + 2], sacc);
        dpacc = mfma_f32(gg.z, vv[4 * c + 2], dpacc);
        sacc = mfma_f32(qq.w, kv[4 * c + 3], sacc);
        dpacc = mfma_f32(gg.w, vv[4 * c + 3], dpacc);
      }
      // Lane: key my_key, queries q0 + c_row(r, h).
      const bool need_mask = (causal && wk0 + 31 > q0) || (window >= 0 && q0 + kStep - 1 - wk0 > window) ||
                             wk0 + 32 > N || q0 + kStep > N;
      float p[16], ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qrow = c_row(r, h);
        float x = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c_log2, -Ls[buf][qrow]));
        if (need_mask) x = visible(q0 + qrow, my_key, N, causal, window) ? x : 0.f;
        p[r] = x;
        ds[r] = x * (dpacc[r] - Ds[buf][qrow]);
      }
      // dV^T += dO^T P and dK^T += Q^T dS: step j takes query rows
      // c_row(j, 0) and c_row(j, 1).
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float* grow = Gb + c_row(j, h) * C::XP + l32;
        const float* qrow = Qb + c_row(j, h) * C::XP + l32;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) {
          dva[cb] = mfma_f32(grow[32 * cb], p[j], dva[cb]);
          dka[cb] = mfma_f32(qrow[32 * cb], ds[j], dka[cb]);
        }
      }
    }
    if (more) {  // that buffer's readers passed the last barrier
      qgt.template store<C::XP, C::XP>(Qs[buf ^ 1], Gs[buf ^ 1]);
      store_ld(buf ^ 1);
    }
    __syncthreads();
  }
  if (my_key < N) {
    store_row<D>(dk + base, my_key, h, dka, scale);
    store_row<D>(dv + base, my_key, h, dva, 1.f);
  }
}

template <int D>
hipError_t launch_t(const float* q, const float* k, const float* v, const float* o, const float* dO,
                    const float* lse, float* dq, float* dk, float* dv, int B, int H, int N, float scale,
                    Mask mask, void* ws, hipStream_t stream) {
  const long long rows = (long long)B * H * N;
  float* Dv = (float*)ws;
  float* L2 = Dv + rows;
  const int nt = (N + kRows - 1) / kRows;
  const unsigned grid = (unsigned)((long long)nt * B * H);
  const float c = scale * kLog2e;
  hipLaunchKernelGGL((bwd_f32_dq_kernel<D>), dim3(grid), dim3(kThreads), 0, stream, q, k, v, o, dO, lse, Dv, L2,
                     dq, B * H, N, nt, scale, c, mask.causal, mask.window);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((bwd_f32_kv_kernel<D>), dim3(grid), dim3(kThreads), 0, stream, q, k, v, dO, Dv, L2, dk, dv,
                     B * H, N, nt, scale, c, mask.causal, mask.window);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_fp32_mfma(const float* q, const float* k, const float* v, const float* o, const float* dO,
                                const float* lse, float* dq, float* dk, float* dv, int B, int H, int N, int d,
                                float scale, Mask mask, void* ws, hipStream_t stream) {
  if (d == 128) return launch_t<128>(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, scale, mask, ws, stream);
  return launch_t<64>(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, scale, mask, ws, stream);
}

}  // namespace fa
