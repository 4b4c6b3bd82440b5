// Float32 forward on the matrix cores (v_mfma_f32_32x32x2_f32: float32
// products, float32 accumulation), head sizes 64 and 128: the automatic
// float32 tile.  Same method as the 16-bit forward ("Building Flash Attention
// from Scratch in Pure NumPy", Architecture Overview and Step 2; "FlashAttention
// Algorithm", the online softmax): a workgroup of 4 waves owns 128 query
// rows, 32 per wave, and walks 32-key tiles of K and V staged in LDS (two
// buffers, the next tile's loads in flight during this tile's math).
//
// Per wave and tile: S^T = K Q^T on the matrix cores, the 32 x 32 result in
// the accumulator layout (lane l holds query l % 32 and 16 keys); the lane's
// Q row (half of the head columns per half-wave, the contraction order of
// both operands) stays in registers for the whole key walk.  The online
// softmax runs in log2 units on those 16 scores plus the other half-wave's
// 16 (one lane swap for the row max and sum), and P^T is already the B
// operand of O^T += V^T P^T: each MFMA step takes the two keys that the two
// half-waves hold in the same register, with the matching V rows read from
// LDS.  Every tile rescales O exactly (no lazy reference: this is the
// float32 path).
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBQ = 32 * kWaves;  // query rows per workgroup
constexpr int kBK = 32;           // keys per tile

template <int D>
struct F32Mfma {
  static constexpr int KP = D + 4;                   // K rows: float4 reads of 16 rows fill the banks once
  static constexpr int VP = D + 8;                   // V rows: the half-waves' rows (4 apart) 128 B apart mod 256 B
  static constexpr int H = D / 2;                    // head columns per half-wave
  static constexpr int CB = D / 32;                  // 32-row blocks of O^T
  static constexpr int LD = kBK * D / 4 / kThreads;  // float4 loads of K (and of V) per thread per tile
};

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_f32_mfma_kernel(const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
                         float* __restrict__ o, float* __restrict__ lse, int BH, int N, int nqt, float c_log2,
                         int causal, int window) {
  using C = F32Mfma<D>;
  __shared__ __align__(16) float Ks[2][kBK * C::KP];
  __shared__ __align__(16) float Vs[2][kBK * C::VP];

  const int t = threadIdx.x;
  const int lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);

  int bh, qr;
  tile_order(blockIdx.x, BH, nqt, causal && window < 0, bh, qr);  // heaviest causal tile first
  const int qt = causal ? nqt - 1 - qr : qr;
  const int q0 = qt * kBQ;
  const size_t base = (size_t)bh * (size_t)N * D;
  const int wq0 = q0 + 32 * w;  // this wave's queries wq0 .. wq0 + 31
  const int my_q = wq0 + l32;   // this lane's query
  const bool q_in = my_q < N;

  // The lane's half of its Q row: Q[my_q][h * H + j], j < H (zeros past N).
  float qv[C::H];
  {
    const float4* src = reinterpret_cast<const float4*>(q + base + (size_t)(q_in ? my_q : 0) * D + h * C::H);
#pragma unroll
    for (int c = 0; c < C::H / 4; ++c) {
      const float4 x = q_in ? src[c] : make_float4(0.f, 0.f, 0.f, 0.f);
      qv[4 * c] = x.x;
      qv[4 * c + 1] = x.y;
      qv[4 * c + 2] = x.z;
      qv[4 * c + 3] = x.w;
    }
  }

  // Key tiles that hold at least one visible key for this workgroup's rows.
  const int q_last = min(q0 + kBQ, N) - 1;
  const int kmin = window >= 0 ? max(0, q0 - window) : 0;
  const int kmax = causal ? q_last : N - 1;
  const int kt0 = kmin / kBK, kt1 = kmax / kBK + 1;

  // Tile staging: element u of thread t is float4 i = t + kThreads * u of
  // the tile's kBK x D / 4 float4s (rows past N read as zero).
  float4 kr[C::LD], vr[C::LD];
  auto load_tile = [&](int kt) {
    const int k0 = kt * kBK;
#pragma unroll
    for (int u = 0; u < C::LD; ++u) {
      const int i = t + kThreads * u, row = i / (D / 4), c4 = i - row * (D / 4);
      const bool in = k0 + row < N;
      const size_t off = base + (size_t)(in ? k0 + row : 0) * D + 4 * c4;
      kr[u] = in ? *reinterpret_cast<const float4*>(k + off) : make_float4(0.f, 0.f, 0.f, 0.f);
      vr[u] = in ? *reinterpret_cast<const float4*>(v + off) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < C::LD; ++u) {
      const int i = t + kThreads * u, row = i / (D / 4), c4 = i - row * (D / 4);
      *reinterpret_cast<float4*>(&Ks[buf][row * C::KP + 4 * c4]) = kr[u];
      *reinterpret_cast<float4*>(&Vs[buf][row * C::VP + 4 * c4]) = vr[u];
    }
  };

  float m_run = kNegInf, l_run = 0.f;  // log2 units
  f32x16 oacc[C::CB];
#pragma unroll
  for (int cb = 0; cb < C::CB; ++cb) oacc[cb] = f32x16{};

  if (kt0 < kt1) {
    load_tile(kt0);
    store_tile(0);
  }
  __syncthreads();
  for (int kt = kt0; kt < kt1; ++kt) {
    const int buf = (kt - kt0) & 1;
    const bool more = kt + 1 < kt1;
    if (more) load_tile(kt + 1);  // in flight during this tile's math
    const int k0 = kt * kBK;
    const bool act = wq0 < N && !(causal && k0 > wq0 + 31) && !(window >= 0 && k0 + kBK - 1 < wq0 - window);
    if (act) {
      const float* Kb = Ks[buf];
      const float* Vb = Vs[buf];
      // S^T = K Q^T: MFMA step j contracts head columns h * H + j of both.
      f32x16 sacc = f32x16{};
#pragma unroll
      for (int c = 0; c < C::H / 4; ++c) {
        const float4 kk = *reinterpret_cast<const float4*>(Kb + l32 * C::KP + h * C::H + 4 * c);
        sacc = mfma_f32(kk.x, qv[4 * c], sacc);
        sacc = mfma_f32(kk.y, qv[4 * c + 1], sacc);
        sacc = mfma_f32(kk.z, qv[4 * c + 2], sacc);
        sacc = mfma_f32(kk.w, qv[4 * c + 3], sacc);
      }
      const bool need_mask = (causal && k0 + kBK - 1 > wq0) || (window >= 0 && wq0 + 31 - k0 > window) ||
                             k0 + kBK > N || wq0 + 32 > N;
      float p[16];
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = sacc[r] * c_log2;
        if (need_mask) {
          const int kj = k0 + c_row(r, h);
          const bool vis = q_in && kj < N && (!causal || kj <= my_q) && (window < 0 || kj >= my_q - window);
          x = vis ? x : kNegInf;
        }
        p[r] = x;
        mx = fmaxf(mx, x);
      }
      const float m_new = fmaxf(m_run, pair_max(mx));
      const float ref = m_new == kNegInf ? 0.f : m_new;  // no visible key yet: any finite reference
      const float alpha = __builtin_amdgcn_exp2f(m_run - ref);
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = __builtin_amdgcn_exp2f(p[r] - ref);
        sum += p[r];
      }
      l_run = l_run * alpha + pair_sum(sum);
      m_run = m_new;
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb) oacc[cb] *= alpha;
      // O^T += V^T P^T: step j takes keys c_row(j, 0) and c_row(j, 1).
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float* vrow = Vb + c_row(j, h) * C::VP + l32;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) oacc[cb] = mfma_f32(vrow[32 * cb], p[j], oacc[cb]);
      }
    }
    if (more) store_tile(buf ^ 1);  // that buffer's readers passed the last barrier
    __syncthreads();
  }

  if (q_in) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* orow = o + base + (size_t)my_q * D;
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(orow + 32 * cb + 8 * g + 4 * h) =
            make_float4(oacc[cb][4 * g] * inv, oacc[cb][4 * g + 1] * inv, oacc[cb][4 * g + 2] * inv,
                        oacc[cb][4 * g + 3] * inv);
    if (h == 0 && lse != nullptr)
      lse[(size_t)bh * N + my_q] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : kNegInf;
  }
}

}  // namespace

hipError_t launch_fwd_fp32_mfma(const float* q, const float* k, const float* v, float* o, float* lse, int B,
                                int H, int N, int d, float scale, Mask mask, hipStream_t stream) {
  const int nqt = (N + kBQ - 1) / kBQ;
  const unsigned grid = (unsigned)((long long)nqt * B * H);
  const float c = scale * kLog2e;
  if (d == 128)
    hipLaunchKernelGGL((fwd_f32_mfma_kernel<128>), dim3(grid), dim3(kThreads), 0, stream, q, k, v, o, lse, B * H,
                       N, nqt, c, mask.causal, mask.window);
  else
    hipLaunchKernelGGL((fwd_f32_mfma_kernel<64>), dim3(grid), dim3(kThreads), 0, stream, q, k, v, o, lse, B * H,
                       N, nqt, c, mask.causal, mask.window);
  return hipGetLastError();
}

}  // namespace fa
