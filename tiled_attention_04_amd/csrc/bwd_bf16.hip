// bf16 backward that recomputes P from the stored logsumexp L.
//
// Method: "Building Flash Attention from Scratch in Pure NumPy", Step 4 --
// D = rowsum(dO * O) first, then an outer loop over key/value tiles and an
// inner loop over the query tiles that see them, recomputing P tile by tile.
// The page's own dK and dQ lines are declared simplified there; the kernels
// use the exact gradients through the softmax:
//   P = exp(S - L),  dV += P^T dO,  dP = dO V^T,  dS = P * (dP - D),
//   dK += scale * dS^T Q,  dQ += scale * dS K.
//
// Mapping onto CDNA4 (v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//  * bwd_pre: one 16-byte slice per lane, D reduced with DPP; it also zeroes
//    dq and stores L in log2 units so the main kernel needs one exp2 per score.
//  * bwd_main: a workgroup of 4 waves owns 128 keys (32 per wave) for its
//    whole life: the wave's K and V rows sit in registers as MFMA B operands
//    and its dK, dV accumulators in registers.  It walks the 64-row query
//    tiles that see those keys; each tile's Q and dO are staged in LDS both
//    row-major (A operands of S = Q K^T and dP = dO V^T) and transposed (B
//    operands of dK and dV), the transposed copies with the row order of the
//    accumulator layout so that P and dS feed the next MFMAs straight from
//    registers.  dS is also written to LDS so that dQ = dS K can be formed per
//    query row; dQ is accumulated in float32 with atomics.  The next query
//    tile is prefetched into registers while the current one is computed.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kBKV = 128;  // keys per workgroup
constexpr int kBQ = 64;    // queries per step

template <int W>
__device__ __forceinline__ int rm_off(int row, int chunk) {  // row-major [rows][W], swizzled
  return row * W + ((chunk ^ (row & 7)) << 3);
}

// Transposed [D][64] tile with the accumulator's row order (bits 2 and 3 of
// the row index swapped within each group of 16) and a chunk swizzle.
__device__ __forceinline__ int tpos(int u) { return (u & ~12) | ((u & 4) << 1) | ((u & 8) >> 1); }
__device__ __forceinline__ int t64_off(int c, int pos) {
  return c * kBQ + ((((pos >> 3) ^ ((c + (c >> 3)) & 7))) << 3) + (pos & 7);
}

// Two packed bf16 columns of four rows -> the 4 values of column cc.
__device__ __forceinline__ uint2 column4(const uint4 (&r)[4], int cc) {
  const uint32_t a0 = word(r[0], cc >> 1), a1 = word(r[1], cc >> 1);
  const uint32_t a2 = word(r[2], cc >> 1), a3 = word(r[3], cc >> 1);
  uint2 out;
  if (cc & 1) {
    out.x = (a0 >> 16) | (a1 & 0xffff0000u);
    out.y = (a2 >> 16) | (a3 & 0xffff0000u);
  } else {
    out.x = (a0 & 0xffffu) | (a1 << 16);
    out.y = (a2 & 0xffffu) | (a3 << 16);
  }
  return out;
}

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(
    const bf16* __restrict__ o, const bf16* __restrict__ dO, const float* __restrict__ lse,
    float* __restrict__ Dv, float* __restrict__ L2, float* __restrict__ dq, long long rows) {
  constexpr int LPR = D / 8;
  constexpr int RPB = kThreads / LPR;
  const int t = threadIdx.x;
  const long long row = (long long)blockIdx.x * RPB + t / LPR;
  const int e = t % LPR;
  float p = 0.f;
  if (row < rows) {
    const size_t off = (size_t)row * D + e * 8;
    const uint4 a = *(const uint4*)(o + off);
    const uint4 b = *(const uint4*)(dO + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p = __builtin_fmaf(bf16_lo(word(a, i)), bf16_lo(word(b, i)), p);
      p = __builtin_fmaf(bf16_hi(word(a, i)), bf16_hi(word(b, i)), p);
    }
    const float4 z = {0.f, 0.f, 0.f, 0.f};
    *(float4*)(dq + off) = z;
    *(float4*)(dq + off + 4) = z;
  }
  p = group_sum<LPR>(p);
  if (row < rows && e == 0) {
    Dv[row] = p;
    const float L = lse[row];
    L2[row] = L == kNegInf ? __builtin_inff() : L * kLog2e;  // row without keys: P = 0
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_main_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                     const bf16* __restrict__ v, const bf16* __restrict__ dO,
                     const float* __restrict__ Dv, const float* __restrict__ L2,
                     float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv,
                     int BH, int N, int nkt, float scale, float scale_log2, int causal, int window) {
  constexpr int KS = D / 16;
  constexpr int CB = D / 32;
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int QUNITS = (kBQ / 4) * CPR;     // 4-row x 16-byte units of a Q tile
  constexpr int KUNITS = (kBKV / 4) * CPR;
  __shared__ __attribute__((aligned(16))) bf16 Qs[kBQ * D];
  __shared__ __attribute__((aligned(16))) bf16 dOs[kBQ * D];
  __shared__ __attribute__((aligned(16))) bf16 Qt[D * kBQ];
  __shared__ __attribute__((aligned(16))) bf16 dOt[D * kBQ];
  __shared__ __attribute__((aligned(16))) bf16 Kt[D * kBKV];
  __shared__ __attribute__((aligned(16))) bf16 dSs[kBQ * kBKV];
  __shared__ __attribute__((aligned(16))) float Ls[kBQ];
  __shared__ __attribute__((aligned(16))) float Ds[kBQ];

  const int t = threadIdx.x;
  const int lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // uniform: keeps per-wave branches scalar

  int bh, kt;
  const int id = blockIdx.x;
  tile_order(id, BH, nkt, causal && window < 0, bh, kt);  // heaviest key tile (kt = 0) first
  const int k0 = kt * kBKV;
  const size_t base = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const rsrc_t q_src = make_rsrc(q + base, head_bytes);
  const rsrc_t k_src = make_rsrc(k + base, head_bytes);
  const rsrc_t v_src = make_rsrc(v + base, head_bytes);
  const rsrc_t do_src = make_rsrc(dO + base, head_bytes);
  const float* Lrow = L2 + (size_t)bh * N;
  const float* Drow = Dv + (size_t)bh * N;

  // This wave's 32 keys as B fragments: K[key][16 s + 8 h + 0..7], same for V.
  const int my_key = k0 + 32 * w + l32;
  bf16x8 kf[KS], vf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const uint32_t off = (uint32_t)(my_key * D + 16 * s + 8 * h) * 2u;
    kf[s] = as_bf16x8(load16(k_src, off));
    vf[s] = as_bf16x8(load16(v_src, off));
  }
  // K^T of the whole key tile in LDS (natural key order) for dQ = dS K.
  for (int i = t; i < KUNITS; i += kThreads) {
    const int co = i % CPR, kq = i / CPR;
    uint4 r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = load16(k_src, (uint32_t)((k0 + 4 * kq + e) * D + co * 8) * 2u);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const int c = co * 8 + cc;
      *(uint2*)(Kt + c * kBKV + ((((4 * kq) >> 3) ^ (c & 7)) << 3) + ((4 * kq) & 7)) = column4(r, cc);
    }
  }

  f32x16 dk_acc[CB], dv_acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    dk_acc[cb] = f32x16{};
    dv_acc[cb] = f32x16{};
  }

  // Query tiles that see at least one of this workgroup's keys.
  const int k_hi = k0 + kBKV - 1;
  const int qmin = causal ? k0 : 0;
  const int qmax = window >= 0 ? min(N - 1, k_hi + window) : N - 1;
  const int qt0 = qmin / kBQ, qt1 = qmax / kBQ + 1;

  // Prefetch registers for one query tile: 4 rows x 16 bytes of Q and dO.
  uint4 qr[4], dr[4];
  float lv = 0.f;
  auto prefetch = [&](int qt) {
    const int q0 = qt * kBQ;
    if (QUNITS >= kThreads || t < QUNITS) {
      const int co = t % CPR, qq = t / CPR;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t off = (uint32_t)((q0 + 4 * qq + e) * D + co * 8) * 2u;
        qr[e] = load16(q_src, off);
        dr[e] = load16(do_src, off);
      }
    }
    if (t < kBQ) lv = q0 + t < N ? Lrow[q0 + t] : __builtin_inff();
    else if (t < 2 * kBQ) lv = q0 + t - kBQ < N ? Drow[q0 + t - kBQ] : 0.f;
  };

  if (qt0 < qt1) prefetch(qt0);
  for (int qt = qt0; qt < qt1; ++qt) {
    const int q0 = qt * kBQ;
    __syncthreads();  // every read of the previous tile's LDS is done
    if (QUNITS >= kThreads || t < QUNITS) {
      const int co = t % CPR, qq = t / CPR;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        *(uint4*)(Qs + rm_off<D>(4 * qq + e, co)) = qr[e];
        *(uint4*)(dOs + rm_off<D>(4 * qq + e, co)) = dr[e];
      }
      const int pos = tpos(4 * qq);
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        *(uint2*)(Qt + t64_off(co * 8 + cc, pos)) = column4(qr, cc);
        *(uint2*)(dOt + t64_off(co * 8 + cc, pos)) = column4(dr, cc);
      }
    }
    if (t < kBQ) Ls[t] = lv;
    else if (t < 2 * kBQ) Ds[t - kBQ] = lv;
    __syncthreads();
    if (qt + 1 < qt1) prefetch(qt + 1);

    // S = Q K^T and dP = dO V^T for the tile's two 32-row blocks.
    f32x16 sacc[2], dpacc[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      sacc[qb] = f32x16{};
      dpacc[qb] = f32x16{};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 a = *(const bf16x8*)(Qs + rm_off<D>(qb * 32 + l32, 2 * s + h));
        sacc[qb] = mfma32(a, kf[s], sacc[qb]);
      }
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 a = *(const bf16x8*)(dOs + rm_off<D>(qb * 32 + l32, 2 * s + h));
        dpacc[qb] = mfma32(a, vf[s], dpacc[qb]);
      }
    }

    // P = exp2(S * scale * log2e - L2) and dS = P (dP - D), masked.
    const bool need_mask = (causal && q0 < k_hi) || (window >= 0 && q0 + kBQ - 1 - k0 > window) ||
                           (k_hi >= N) || (q0 + kBQ > N);
    uint32_t ppk[2][8], dspk[2][8];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 L4 = *(const float4*)(Ls + qb * 32 + 8 * g + 4 * h);
        const float4 D4 = *(const float4*)(Ds + qb * 32 + 8 * g + 4 * h);
        float pv[4], dsv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * g + i;
          const float Li = i == 0 ? L4.x : i == 1 ? L4.y : i == 2 ? L4.z : L4.w;
          const float Di = i == 0 ? D4.x : i == 1 ? D4.y : i == 2 ? D4.z : D4.w;
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][r], scale_log2, -Li));
          if (need_mask) {
            const int qrow = q0 + qb * 32 + 8 * g + 4 * h + i;
            const bool vis = my_key < N && qrow < N && (!causal || my_key <= qrow) &&
                             (window < 0 || my_key >= qrow - window);
            p = vis ? p : 0.f;
          }
          pv[i] = p;
          dsv[i] = p * (dpacc[qb][r] - Di);
        }
        ppk[qb][2 * g] = pack_bf16(pv[0], pv[1]);
        ppk[qb][2 * g + 1] = pack_bf16(pv[2], pv[3]);
        dspk[qb][2 * g] = pack_bf16(dsv[0], dsv[1]);
        dspk[qb][2 * g + 1] = pack_bf16(dsv[2], dsv[3]);
      }
    }

    // dV += P^T dO and dK += dS^T Q, 16 queries per step.
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 pw = {ppk[s >> 1][4 * (s & 1)], ppk[s >> 1][4 * (s & 1) + 1],
                        ppk[s >> 1][4 * (s & 1) + 2], ppk[s >> 1][4 * (s & 1) + 3]};
      const uint4 dw = {dspk[s >> 1][4 * (s & 1)], dspk[s >> 1][4 * (s & 1) + 1],
                        dspk[s >> 1][4 * (s & 1) + 2], dspk[s >> 1][4 * (s & 1) + 3]};
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int off = t64_off(cb * 32 + l32, 16 * s + 8 * h);
        dv_acc[cb] = mfma32(as_bf16x8(pw), *(const bf16x8*)(dOt + off), dv_acc[cb]);
        dk_acc[cb] = mfma32(as_bf16x8(dw), *(const bf16x8*)(Qt + off), dk_acc[cb]);
      }
    }

    // dS (bf16) to LDS in natural [query][key] order for dQ.
    {
      const int kl = 32 * w + l32;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = qb * 32 + c_row(r, h);
          const uint32_t pair = dspk[qb][r >> 1];
          const uint16_t bits = (r & 1) ? (uint16_t)(pair >> 16) : (uint16_t)(pair & 0xffffu);
          *(uint16_t*)(dSs + ql * kBKV + ((((kl >> 3) ^ (ql & 7))) << 3) + (kl & 7)) = bits;
        }
      }
    }
    __syncthreads();

    // dQ[64 x D] += dS K: wave w forms rows 32*(w/2).. and column blocks
    // 2*(w%2) + {0, 1} of D=128 (column block w%2 of D=64).
    {
      constexpr int NCB = CB / 2;
      const int qb = w >> 1;
      f32x16 dqacc[NCB];
#pragma unroll
      for (int j = 0; j < NCB; ++j) dqacc[j] = f32x16{};
#pragma unroll
      for (int s = 0; s < kBKV / 16; ++s) {
        const bf16x8 a = *(const bf16x8*)(dSs + rm_off<kBKV>(qb * 32 + l32, 2 * s + h));
#pragma unroll
        for (int j = 0; j < NCB; ++j) {
          const int c = (NCB * (w & 1) + j) * 32 + l32;
          const bf16x8 b = *(const bf16x8*)(Kt + c * kBKV + (((2 * s + h) ^ (c & 7)) << 3));
          dqacc[j] = mfma32(a, b, dqacc[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < NCB; ++j) {
        const int c = (NCB * (w & 1) + j) * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qrow = q0 + qb * 32 + c_row(r, h);
          if (qrow < N) unsafeAtomicAdd(dq + base + (size_t)qrow * D + c, scale * dqacc[j][r]);
        }
      }
    }
  }

  // dK = scale * dS^T Q, dV = P^T dO for this wave's 32 keys.
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int krow = k0 + 32 * w + c_row(r, h);
      if (krow < N) {
        const size_t off = base + (size_t)krow * D + cb * 32 + l32;
        dk[off] = scale * dk_acc[cb][r];
        dv[off] = dv_acc[cb][r];
      }
    }
  }
}

template <int D>
hipError_t launch_t(const void* q, const void* k, const void* v, const void* o, const void* dO,
                    const float* lse, float* dq, float* dk, float* dv, int B, int H, int N,
                    float scale, Mask mask, void* ws, hipStream_t stream) {
  const long long rows = (long long)B * H * N;
  float* Dv = (float*)ws;
  float* L2 = Dv + rows;
  constexpr int RPB = kThreads / (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(kThreads),
                     0, stream, (const bf16*)o, (const bf16*)dO, lse, Dv, L2, dq, rows);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int nkt = (N + kBKV - 1) / kBKV;
  const long long grid = (long long)nkt * B * H;
  hipLaunchKernelGGL((bwd_main_kernel<D>), dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dO, Dv, L2, dq, dk,
                     dv, B * H, N, nkt, scale, scale * kLog2e, mask.causal, mask.window);
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int N, int d) {
  (void)d;
  return (size_t)B * H * N * 2 * sizeof(float);
}

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const void* dO, const float* lse, float* dq, float* dk, float* dv,
                           int B, int H, int N, int d, float scale, Mask mask, void* ws,
                           hipStream_t stream) {
  if (d == 128) return launch_t<128>(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, scale, mask, ws, stream);
  return launch_t<64>(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, scale, mask, ws, stream);
}

}  // namespace fa
