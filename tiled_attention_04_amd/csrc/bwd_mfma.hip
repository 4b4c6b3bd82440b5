// 16-bit (bf16 or fp16) backward that recomputes P from the stored
// logsumexp L.  Every kernel is written once for the element type T.
//
// Method: "Building Flash Attention from Scratch in Pure NumPy", Step 4 --
// D = rowsum(dO * O) first, then an outer loop over key/value tiles and an
// inner loop over the query tiles that see them, recomputing P tile by tile.
// The page's own dK and dQ lines are declared simplified there; the kernels
// use the exact gradients through the softmax:
//   P = exp(S - L),  dV += P^T dO,  dP = dO V^T,  dS = P * (dP - D),
//   dK += scale * dS^T Q,  dQ += scale * dS K.
//
// Mapping onto CDNA4 (v_mfma_f32_32x32x16_bf16 / _f16, fp32 accumulation), three
// kernels on one stream:
//  * bwd_pre: one 16-byte slice per lane, D reduced with DPP; it also stores
//    L in log2 units so the other kernels need one exp2 per score.
//  * bwd_main: dK and dV, in the page's loop order (key/value tiles outer):
//    a workgroup of 8 waves owns a 128-key tile and walks the query tiles.
//  * bwd_dq: dQ, with the loops the other way round (a workgroup owns 128
//    query rows and walks the key tiles, as the forward does), recomputing
//    S, P, dP and dS; no atomics, so dQ is deterministic.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kThreads = 512;     // main kernel: 8 waves
constexpr int kPreThreads = 256;  // preprocessing kernel
constexpr int kBKV = 128;  // keys per workgroup
constexpr int kBQ = 64;    // queries per step

constexpr int kSchedVALU = 0x002, kSchedMFMA = 0x008, kSchedDSRead = 0x100;

// Scheduling pattern for a block of M MFMAs fed by R LDS reads, with V
// vector-ALU instructions of independent work placed after each MFMA: the
// first A reads go ahead, the rest are spread evenly over the MFMAs.  Keeps
// the compiler from hoisting every operand read (which runs out of registers
// at one wave per SIMD) while the reads still run ahead of their MFMAs.
template <int I, int M, int R, int A, int V, int SYNC>
__device__ __forceinline__ void interleave_step() {
  if constexpr (I < M) {
    constexpr int n = (I + 1) * (R - A) / M - I * (R - A) / M;
    __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, SYNC);
    if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(kSchedDSRead, n, SYNC);
    if constexpr (V > 0) __builtin_amdgcn_sched_group_barrier(kSchedVALU, V, SYNC);
    interleave_step<I + 1, M, R, A, V, SYNC>();
  }
}
template <int M, int R, int A, int V, int SYNC>
__device__ __forceinline__ void interleave() {
  __builtin_amdgcn_sched_group_barrier(kSchedDSRead, A, SYNC);
  interleave_step<0, M, R, A, V, SYNC>();
}

template <typename T, int D>
__global__ __launch_bounds__(kPreThreads) void bwd_pre_kernel(
    const T* __restrict__ o, const T* __restrict__ dO, const float* __restrict__ lse,
    float* __restrict__ Dv, float* __restrict__ L2, long long rows) {
  constexpr int LPR = D / 8;
  constexpr int RPB = kPreThreads / LPR;
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
      p = __builtin_fmaf(lo16<T>(word(a, i)), lo16<T>(word(b, i)), p);
      p = __builtin_fmaf(hi16<T>(word(a, i)), hi16<T>(word(b, i)), p);
    }
  }
  p = group_sum<LPR>(p);
  if (row < rows && e == 0) {
    Dv[row] = p;
    const float L = lse[row];
    L2[row] = L == kNegInf ? __builtin_inff() : L * kLog2e;  // row without keys: P = 0
  }
}

// Main backward kernel: dK and dV.  A workgroup of 8 waves (two per SIMD)
// owns 128 keys and walks the 64-row query tiles that see them.  Wave
// w = (kb, qb), kb = w % 4 and qb = w / 4:
//  * scores: S = Q K^T and dP = dO V^T for its 32 keys (block kb) and the
//    tile's query rows 32 qb .. 32 qb + 31; Q and dO come from LDS as MFMA A
//    operands, the wave's K and V rows stay in registers as B operands;
//  * P = exp2(S c - L2) and dS = P (dP - D) on the vector ALUs, written to LDS
//    (keys as rows) in the order of the MFMA A operand, so every wave reads
//    P^T and dS^T of a key block for all 64 queries with 16-byte reads;
//  * gradients: dV += P^T dO and dK += dS^T Q for the wave's key block and
//    half of the columns, over all 64 queries (B operands by transpose reads
//    of the row-major dO and Q tiles).
// Q, dO, L2 and D of the next query tile stream into LDS by direct loads
// while the current one is processed (two stages); K and V are read once.
// dQ is formed by its own kernel (below): accumulated here it would take one
// float atomic per query row, column and key tile, and those atomics cost
// about as much as all the rest of this kernel.
template <int D>
struct BwdTile {
  static constexpr int kQPitch = D == 128 ? 304 : 144;  // bytes per Q / dO row in LDS
  static constexpr int kSPitch = 144;                    // bytes per P^T / dS^T row (64 queries)
  static constexpr int kQBytes = kBQ * kQPitch;
  static constexpr int kSBytes = kBKV * kSPitch;
  static constexpr int kQBlocks = kQBytes / 1024;  // 1 KB per wave-wide direct load
  static_assert(kQBytes % 1024 == 0, "tiles must be whole 1 KB blocks");
};

template <typename T, int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_main_kernel(const T* __restrict__ q, const T* __restrict__ k,
                     const T* __restrict__ v, const T* __restrict__ dO,
                     const float* __restrict__ Dv, const float* __restrict__ L2,
                     float* __restrict__ dk, float* __restrict__ dv,
                     int BH, int N, int nkt, float scale, float scale_log2, int causal, int window) {
  using TL = BwdTile<D>;
  constexpr int NW = kThreads / 64;  // 8
  constexpr int KS = D / 16;         // 16-wide steps over the head dimension
  constexpr int CB = D / 32;         // 32-column blocks of the head dimension
  constexpr int NCB = CB / 2;        // column blocks of dK / dV per wave
  constexpr int QPER = (TL::kQBlocks + NW - 1) / NW;
  constexpr int QP = TL::kQPitch, SP = TL::kSPitch;
  // One LDS object per stage and matrix (the compiler then knows that direct
  // loads into one stage do not alias reads of the other).
  __shared__ __attribute__((aligned(1024))) char Q0[TL::kQBytes];
  __shared__ __attribute__((aligned(1024))) char Q1[TL::kQBytes];
  __shared__ __attribute__((aligned(1024))) char O0[TL::kQBytes];
  __shared__ __attribute__((aligned(1024))) char O1[TL::kQBytes];
  __shared__ __attribute__((aligned(1024))) char Pt[TL::kSBytes];
  __shared__ __attribute__((aligned(1024))) char dSt[TL::kSBytes];
  __shared__ __attribute__((aligned(256))) float LD0[2 * kBQ];  // L2 then D of a query tile
  __shared__ __attribute__((aligned(256))) float LD1[2 * kBQ];

  const int t = threadIdx.x;
  const int lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // uniform: keeps per-wave branches scalar
  __builtin_assume(w >= 0 && w < NW);
  const int kb = w & 3, qb = w >> 2;

  int bh, kt;
  tile_order(blockIdx.x, BH, nkt, causal && window < 0, bh, kt);  // heaviest key tile (kt = 0) first
  const int k0 = kt * kBKV;
  const size_t base = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;

  // This wave's 32 key and value rows as B operands of S and dP:
  // K[key][16 s + 8 h + 0..7] and V[key][16 s + 8 h + 0..7].
  const int my_key = k0 + 32 * kb + l32;
  vec8<T> kf[KS], vf[KS];
  {
    const rsrc_t k_src = make_rsrc(k + base, head_bytes);
    const rsrc_t v_src = make_rsrc(v + base, head_bytes);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kf[s] = as_vec8<T>(load16(k_src, (uint32_t)(my_key * D + 16 * s + 8 * h) * 2u));
      vf[s] = as_vec8<T>(load16(v_src, (uint32_t)(my_key * D + 16 * s + 8 * h) * 2u));
    }
  }

  // Query tiles that see at least one of this workgroup's keys.
  const int k_hi = k0 + kBKV - 1;
  const int qmin = causal ? k0 : 0;
  const int qmax = window >= 0 ? min(N - 1, k_hi + window) : N - 1;
  const int qt0 = qmin / kBQ, qt1 = qmax / kBQ + 1;

  // Direct-load source offsets of this lane (padding lanes read nothing).
  uint32_t qpre[QPER];
#pragma unroll
  for (int i = 0; i < QPER; ++i) qpre[i] = block_src<D>(w + i * NW, lane, QP);

  auto stage_q = [&] __device__ (auto st) -> char* { return decltype(st)::value == 0 ? Q0 : Q1; };
  auto stage_o = [&] __device__ (auto st) -> char* { return decltype(st)::value == 0 ? O0 : O1; };
  auto stage_ld = [&] __device__ (auto st) -> float* { return decltype(st)::value == 0 ? LD0 : LD1; };
  const float* Lrow = L2 + (size_t)bh * N;
  const float* Drow = Dv + (size_t)bh * N;
  // This wave's share of the direct loads of query tile qt into stage st:
  // Q and dO blocks, and (waves 0 and 1) the tile's 64 values of L2 / D.
  auto load_qtile = [&] __device__ (int qt, auto st) {
    const int q0 = qt * kBQ;
    const uint32_t bytes = (uint32_t)max(0, N - q0) * D * 2u;
    const rsrc_t qs = make_rsrc(q + base + (size_t)q0 * D, bytes);
    const rsrc_t os = make_rsrc(dO + base + (size_t)q0 * D, bytes);
    char* qd = stage_q(st);
    char* od = stage_o(st);
#pragma unroll
    for (int i = 0; i < QPER; ++i) {
      const int blk = w + i * NW;
      if (blk < TL::kQBlocks) {
        load_lds16(qs, qd + blk * 1024, qpre[i]);
        load_lds16(os, od + blk * 1024, qpre[i]);
      }
    }
    if (w < 2) {
      const rsrc_t ls = make_rsrc((w == 0 ? Lrow : Drow) + q0, (uint32_t)max(0, N - q0) * 4u);
      load_lds4(ls, stage_ld(st) + w * kBQ, (uint32_t)lane * 4u);
    }
  };

  using std::integral_constant;
  // Prologue: the first query tile resident.
  if (qt0 < qt1) load_qtile(qt0, integral_constant<int, 0>{});
  // The K and V rows above must be in flight together with this tile's
  // loads: left to itself the compiler issued them only after the wait
  // below, so the two round trips to memory ran one after the other.  An
  // empty asm that reads them here keeps them ahead of the wait.
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
  for (int s = 0; s < KS; ++s) asm volatile("" : "+v"(kf[s]), "+v"(vf[s]));
#endif
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  f32x16 dk_acc[NCB], dv_acc[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    dk_acc[c] = f32x16{};
    dv_acc[c] = f32x16{};
  }
  const int q_rd = (32 * qb + l32) * QP + 16 * h;       // A operands of S and dP
  const int s_wr = (32 * kb + l32) * SP + (32 * qb + 8 * h) * 2;  // this lane's P / dS pieces
  const int s_rd = (32 * kb + l32) * SP + 16 * h;       // A operands of dV / dK
  const int tr_q = tr_addr<QP>(lane);                   // B operands of dV / dK

  // One query tile in stage ST.
  auto tile = [&] __device__ (auto stage, int qt) {
    constexpr int ST = decltype(stage)::value;
    const char* Qs = stage_q(stage);
    const char* Os = stage_o(stage);
    const float* LD = stage_ld(stage);
    const int q0 = qt * kBQ;
    if (qt + 1 < qt1) load_qtile(qt + 1, integral_constant<int, ST ^ 1>{});
    const bool need_mask = (causal && q0 < k_hi) || (window >= 0 && q0 + kBQ - 1 - k0 > window) ||
                           (k_hi >= N) || (q0 + kBQ > N);

    // 1) S = Q K^T, then dP = dO V^T while P = exp2(S * scale * log2e - L2)
    //    (masked) is formed on the vector ALUs.
    f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; ++s)
      sacc = mfma32(*(const vec8<T>*)(Qs + q_rd + 32 * s), kf[s], sacc);
    interleave<KS, KS, 4, 0, 1>();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      dpacc = mfma32(*(const vec8<T>*)(Os + q_rd + 32 * s), vf[s], dpacc);
    float pv[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 L4 = *(const float4*)(LD + 32 * qb + 8 * g + 4 * h);
      pv[4 * g + 0] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[4 * g + 0], scale_log2, -L4.x));
      pv[4 * g + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[4 * g + 1], scale_log2, -L4.y));
      pv[4 * g + 2] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[4 * g + 2], scale_log2, -L4.z));
      pv[4 * g + 3] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[4 * g + 3], scale_log2, -L4.w));
    }
    // Hidden pairs get P = 0 (one branch around the whole tile: inside the
    // element loop the test would be evaluated on every tile).
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qrow = q0 + 32 * qb + c_row(r, h);
        const int lo = window >= 0 ? qrow - window : 0;
        const int hi = min(causal ? qrow : N - 1, N - 1);
        const bool vis = (qrow < N) & ((uint32_t)(my_key - lo) <= (uint32_t)(hi - lo));
        pv[r] = vis ? pv[r] : 0.f;
      }
    }
    uint32_t ppk[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) ppk[j] = pack2<T>(pv[2 * j], pv[2 * j + 1]);
    interleave<KS, KS, 4, 6, 2>();
    __builtin_amdgcn_sched_barrier(0);
    uint32_t dspk[8];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 D4 = *(const float4*)(LD + kBQ + 32 * qb + 8 * g + 4 * h);
      dspk[2 * g] = pack2<T>(pv[4 * g] * (dpacc[4 * g] - D4.x), pv[4 * g + 1] * (dpacc[4 * g + 1] - D4.y));
      dspk[2 * g + 1] = pack2<T>(pv[4 * g + 2] * (dpacc[4 * g + 2] - D4.z),
                                  pv[4 * g + 3] * (dpacc[4 * g + 3] - D4.w));
    }
    // P^T and dS^T rows: this lane's key, its 16 queries in A-operand order.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      *(uint4*)(Pt + s_wr + 32 * j) = uint4{ppk[4 * j], ppk[4 * j + 1], ppk[4 * j + 2], ppk[4 * j + 3]};
      *(uint4*)(dSt + s_wr + 32 * j) = uint4{dspk[4 * j], dspk[4 * j + 1], dspk[4 * j + 2], dspk[4 * j + 3]};
    }
    // LDS writes done, then the barrier; direct loads stay in flight.
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // 2) dV += P^T dO and dK += dS^T Q over the tile's 64 queries (16 per
    //    step) for this wave's column blocks.
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const vec8<T> pa = *(const vec8<T>*)(Pt + s_rd + 32 * s);
      const vec8<T> da = *(const vec8<T>*)(dSt + s_rd + 32 * s);
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        const int off = tr_q + 16 * s * QP + 64 * (NCB * qb + c);
        dv_acc[c] = mfma32(pa, read_tr8<QP, T>(Os + off), dv_acc[c]);
        dk_acc[c] = mfma32(da, read_tr8<QP, T>(Qs + off), dk_acc[c]);
      }
    }
    interleave<8 * NCB, 8 + 16 * NCB, 4, 0, 3>();
    __builtin_amdgcn_sched_barrier(0);

    // The next tile's direct loads have landed; after the barrier no wave
    // reads this stage, P^T or dS^T any more.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  for (int qt = qt0; qt < qt1; qt += 2) {
    tile(integral_constant<int, 0>{}, qt);
    if (qt + 1 >= qt1) break;
    tile(integral_constant<int, 1>{}, qt + 1);
  }

  // dK = scale * dS^T Q, dV = P^T dO for key block kb and this wave's column
  // blocks; rows past N fall outside the buffers and are dropped.
  const rsrc_t dk_dst = make_rsrc(dk + base, (uint32_t)N * D * 4u);
  const rsrc_t dv_dst = make_rsrc(dv + base, (uint32_t)N * D * 4u);
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t off =
          ((uint32_t)(k0 + 32 * kb + c_row(r, h)) * D + 32 * (NCB * qb + c) + l32) * 4u;
      store_f32(dk_dst, off, scale * dk_acc[c][r]);
      store_f32(dv_dst, off, dv_acc[c][r]);
    }
  }
}

// Store this wave's 32 x D block of dQ (rows r0 .. r0 + 31 of the slice,
// rows at or past N dropped), scaled, through `stage`: 32 * (2 D + 16) bytes
// of LDS that only this wave uses, half of the columns at a time.  In the
// accumulator layout a lane holds 16-byte pieces of 32 different rows, so
// storing from it directly splits every store instruction into 32 pieces of
// 32 bytes; read back row by row from LDS each store instruction writes
// whole half-rows of 2 D bytes.
template <int D, int CB>
__device__ __forceinline__ void store_dq_rows(const f32x16 (&dqa)[CB], float scale, char* stage,
                                              float* __restrict__ dq_slice, int r0, int N, int lane) {
  constexpr int P = 2 * D + 16;
  constexpr int HB = CB / 2;          // 32-column blocks per half
  constexpr int CPR = 2 * D / 16;     // 16-byte chunks per half row
  constexpr int RPP = 64 / CPR;       // half rows per wave-wide read
  const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int c = 0; c < HB; ++c)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& a = dqa[half * HB + c];
        *(float4*)(stage + l32 * P + (32 * c + 8 * g + 4 * h) * 4) =
            float4{scale * a[4 * g], scale * a[4 * g + 1], scale * a[4 * g + 2], scale * a[4 * g + 3]};
      }
#pragma unroll
    for (int i = 0; i < 32 / RPP; ++i) {
      const int row = i * RPP + lane / CPR, ch = lane % CPR;
      const uint4 u = *(const uint4*)(stage + row * P + ch * 16);
      if (r0 + row < N)
        *(uint4*)((char*)(dq_slice + (size_t)(r0 + row) * D + half * (D / 2)) + ch * 16) = u;
    }
  }
}

// dQ kernel: dQ = scale * dS K without atomics.  A workgroup of 4 waves owns
// 128 query rows (32 per wave, one per lane pair as in the forward kernels)
// and walks the 64-key tiles they see, recomputing per tile
//   S^T = K Q^T,  dP^T = V dO^T   (Q and dO rows in registers as B operands,
//                                  K and V rows from LDS as A operands),
//   P^T = exp2(S^T * scale * log2e - L2),  dS^T = P^T (dP^T - D)
//                                 (L2 and D: one value per lane),
//   dQ^T += K^T dS^T              (K^T by transpose reads of the K tile, dS^T
//                                  packed to T straight from the
//                                  accumulators, as P in the forward).
// K and V tiles are double-buffered in LDS and filled by direct loads.
constexpr int kDqBK = 64;   // keys per tile
constexpr int kDqThreads = 256;

template <int D>
struct DqTile {
  static constexpr int kKPitch = D == 128 ? 304 : 144;  // K rows: 16-byte and transpose reads
  static constexpr int kVPitch = 2 * D + 16;             // V rows: 16-byte reads
  static constexpr int kKBytes = kDqBK * kKPitch;
  static constexpr int kVBytes = kDqBK * kVPitch;
  static constexpr int kKBlocks = kKBytes / 1024;
  static constexpr int kVBlocks = kVBytes / 1024;
  static_assert(kKBytes % 1024 == 0 && kVBytes % 1024 == 0, "tiles must be whole 1 KB blocks");
  // Two waves' dQ half-blocks (32 rows of 2 D + 16 bytes each) fit a tile.
  static_assert(2 * 32 * (2 * D + 16) <= kKBytes && 2 * 32 * (2 * D + 16) <= kVBytes, "dQ staging");
};

// (d = 128 may run one wave per SIMD: this kernel serves grids too small for
// the ping-pong kernel below, under two workgroups per CU anyway, and held to
// two waves per SIMD its registers spilled to scratch -- 21-27% slower.
// d = 64 fits two waves per SIMD and is faster so.)
template <typename T, int D>
__global__ __launch_bounds__(kDqThreads) __attribute__((amdgpu_waves_per_eu(D == 128 ? 1 : 2, 2)))
void bwd_dq_kernel(const T* __restrict__ q, const T* __restrict__ k,
                   const T* __restrict__ v, const T* __restrict__ dO,
                   const float* __restrict__ Dv, const float* __restrict__ L2,
                   float* __restrict__ dq, int BH, int N, int nqt, float scale, float scale_log2,
                   int causal, int window) {
  using TL = DqTile<D>;
  constexpr int NW = kDqThreads / 64;
  constexpr int BQ = 32 * NW;
  constexpr int KS = D / 16;
  constexpr int CB = D / 32;
  constexpr int KPER = (TL::kKBlocks + NW - 1) / NW;
  constexpr int VPER = (TL::kVBlocks + NW - 1) / NW;
  constexpr int KP = TL::kKPitch, VP = TL::kVPitch;
  __shared__ __attribute__((aligned(1024))) char Kb0[TL::kKBytes];
  __shared__ __attribute__((aligned(1024))) char Kb1[TL::kKBytes];
  __shared__ __attribute__((aligned(1024))) char Vb0[TL::kVBytes];
  __shared__ __attribute__((aligned(1024))) char Vb1[TL::kVBytes];

  const int t = threadIdx.x;
  const int lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  __builtin_assume(w >= 0 && w < NW);

  int bh, qr;
  tile_order(blockIdx.x, BH, nqt, causal && window < 0, bh, qr);
  const int qt = causal ? nqt - 1 - qr : qr;  // causal: the longest rows first
  const int q0 = qt * BQ;
  const size_t base = (size_t)bh * (size_t)N * D;
  const int qi = q0 + 32 * w + l32;  // this lane's query row

  // Q and dO rows of this lane as B fragments: [qi][16 s + 8 h + 0..7]
  // (rows past N read as zero), and the row's L2 and D.
  vec8<T> qf[KS], of[KS];
  {
    const rsrc_t q_src = make_rsrc(q + base, (uint32_t)N * D * 2u);
    const rsrc_t o_src = make_rsrc(dO + base, (uint32_t)N * D * 2u);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint32_t off = (uint32_t)(qi * D + 16 * s + 8 * h) * 2u;
      qf[s] = as_vec8<T>(load16(q_src, off));
      of[s] = as_vec8<T>(load16(o_src, off));
    }
  }
  const bool row_ok = qi < N;
  const float Li = row_ok ? L2[(size_t)bh * N + qi] : 0.f;
  const float Di = row_ok ? Dv[(size_t)bh * N + qi] : 0.f;

  // Key tiles holding at least one key visible to this query tile, and the
  // keys this lane's row sees.
  const int q_hi = q0 + BQ - 1;
  const int kmin = window >= 0 ? max(0, q0 - window) : 0;
  const int kmax = causal ? min(N - 1, q_hi) : N - 1;
  const int kt0 = kmin / kDqBK, kt1 = kmax / kDqBK + 1;
  const int key_lo = window >= 0 ? qi - window : 0;
  const int key_hi = causal ? min(qi, N - 1) : N - 1;

  uint32_t kpre[KPER], vpre[VPER];
#pragma unroll
  for (int i = 0; i < KPER; ++i) kpre[i] = block_src<D>(w + i * NW, lane, KP);
#pragma unroll
  for (int i = 0; i < VPER; ++i) vpre[i] = block_src<D>(w + i * NW, lane, VP);
  auto load_kv = [&] __device__ (int kt, char* kd, char* vd) {
    const int k0 = kt * kDqBK;
    const uint32_t bytes = (uint32_t)max(0, N - k0) * D * 2u;
    const rsrc_t ks = make_rsrc(k + base + (size_t)k0 * D, bytes);
    const rsrc_t vs = make_rsrc(v + base + (size_t)k0 * D, bytes);
#pragma unroll
    for (int i = 0; i < KPER; ++i)
      if (w + i * NW < TL::kKBlocks) load_lds16(ks, kd + (w + i * NW) * 1024, kpre[i]);
#pragma unroll
    for (int i = 0; i < VPER; ++i)
      if (w + i * NW < TL::kVBlocks) load_lds16(vs, vd + (w + i * NW) * 1024, vpre[i]);
  };

  const int k_rd = l32 * KP + 16 * h;  // A operands of S^T (K rows)
  const int v_rd = l32 * VP + 16 * h;  // A operands of dP^T (V rows)
  const int k_tr = tr_addr<KP>(lane);  // A operands of dQ^T (K^T)

  f32x16 dqa[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) dqa[cb] = f32x16{};

  if (kt0 < kt1) load_kv(kt0, Kb0, Vb0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  auto tile = [&] __device__ (auto parity, int kt) {
    constexpr int P = decltype(parity)::value;
    const char* Kc = P ? Kb1 : Kb0;
    const char* Vc = P ? Vb1 : Vb0;
    if (kt + 1 < kt1) load_kv(kt + 1, P ? Kb0 : Kb1, P ? Vb0 : Vb1);
    const int k0 = kt * kDqBK;
    const bool need_mask = (k0 + kDqBK > N) || (causal && k0 + kDqBK - 1 > q0) ||
                           (window >= 0 && k0 < q_hi - window);

    // S^T and dP^T for the tile's two 32-key blocks.
    f32x16 sacc[2], dpacc[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      sacc[kb2] = f32x16{};
      dpacc[kb2] = f32x16{};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        sacc[kb2] = mfma32(*(const vec8<T>*)(Kc + k_rd + kb2 * 32 * KP + 32 * s), qf[s], sacc[kb2]);
        dpacc[kb2] = mfma32(*(const vec8<T>*)(Vc + v_rd + kb2 * 32 * VP + 32 * s), of[s], dpacc[kb2]);
      }
    }
    // dS^T = P^T (dP^T - D), P^T = exp2(S^T c - L2) with hidden keys at 0
    // (the mask is one branch around the whole tile: inside the element
    // loop it would be evaluated on every tile).
    // (P^T overwrites S^T in place.)
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sacc[kb2][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb2][r], scale_log2, -Li));
    if (need_mask) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb2 * 32 + c_row(r, h);
          sacc[kb2][r] = (uint32_t)(key - key_lo) <= (uint32_t)(key_hi - key_lo) ? sacc[kb2][r] : 0.f;
        }
    }
    uint32_t dspk[2][8];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; r += 2)
        dspk[kb2][r >> 1] = pack2<T>(sacc[kb2][r] * (dpacc[kb2][r] - Di),
                                      sacc[kb2][r + 1] * (dpacc[kb2][r + 1] - Di));
    // dQ^T += K^T dS^T, 16 keys per step.
#pragma unroll
    for (int s = 0; s < kDqBK / 16; ++s) {
      const uint4 dw = {dspk[s >> 1][4 * (s & 1)], dspk[s >> 1][4 * (s & 1) + 1],
                        dspk[s >> 1][4 * (s & 1) + 2], dspk[s >> 1][4 * (s & 1) + 3]};
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        dqa[cb] = mfma32(read_tr8<KP, T>(Kc + k_tr + 16 * s * KP + 64 * cb), as_vec8<T>(dw), dqa[cb]);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads of the next tile have landed
    __syncthreads();
  };

  for (int kt = kt0; kt < kt1; kt += 2) {
    tile(std::integral_constant<int, 0>{}, kt);
    if (kt + 1 >= kt1) break;
    tile(std::integral_constant<int, 1>{}, kt + 1);
  }

  // dQ row qi: element r of block cb is column 32 cb + c_row(r, h); four
  // consecutive columns per 16-byte store.
  // dQ through LDS (the loop's last barrier freed the K tiles): two waves
  // per tile.
  store_dq_rows<D, CB>(dqa, scale, (w < 2 ? Kb0 : Kb1) + (w & 1) * 32 * (2 * D + 16), dq + base,
                       q0 + 32 * w, N, lane);
}

// Ping-pong dQ kernel for long sequences: 8 waves, 256 query rows per
// workgroup, the same computation as bwd_dq_kernel.  The waves form two groups
// (by their order of arrival on a SIMD, one wave of each group per SIMD) that
// run the tile loop one phase apart with workgroup barriers between phases:
// while one group's waves form P and dS of tile j on the vector ALUs, the
// other group's waves issue their matrix work -- dQ of tile j, then S and dP
// of tile j+1 -- so every SIMD's matrix core has work while its vector ALU is
// busy.  K and V tiles sit in three LDS stages; every wave loads its share of
// tile j+2 while tiles j and j+1 are in use, and waits for its own loads just
// before the barrier that opens group 0's next matrix phase.
constexpr int kDqPPThreads = 512;

template <int D>
struct DqPPTile {
  static constexpr int kKPitch = D == 128 ? 304 : 144;  // K rows: 16-byte and transpose reads
  static constexpr int kVPitch = 2 * D + 16;             // V rows: 16-byte reads
  static constexpr int kKBytes = kDqBK * kKPitch;
  static constexpr int kVBytes = kDqBK * kVPitch;
  static constexpr int kKBlocks = kKBytes / 1024;
  static constexpr int kVBlocks = kVBytes / 1024;
  static_assert(kKBytes % 1024 == 0 && kVBytes % 1024 == 0, "tiles must be whole 1 KB blocks");
  // Two waves' dQ half-blocks (32 rows of 2 D + 16 bytes each) fit a tile.
  static_assert(2 * 32 * (2 * D + 16) <= kKBytes && 2 * 32 * (2 * D + 16) <= kVBytes, "dQ staging");
};

// Keeps the vector-ALU results of a phase on their side of the barrier that
// follows (compiler passes would otherwise sink the arithmetic next to its
// only users, the MFMAs of the next phase).
template <int CB>
__device__ __forceinline__ void pin_dq_phase(uint32_t (&ds)[2][8], f32x16 (&acc)[CB]) {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(ds[i][j]));
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) asm volatile("" : "+v"(acc[cb]));
#endif
}

template <typename T, int D>
__global__ __launch_bounds__(kDqPPThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_pp_kernel(const T* __restrict__ q, const T* __restrict__ k,
                      const T* __restrict__ v, const T* __restrict__ dO,
                      const float* __restrict__ Dv, const float* __restrict__ L2,
                      float* __restrict__ dq, int BH, int N, int nqt, float scale, float scale_log2,
                      int causal, int window) {
  using TL = DqPPTile<D>;
  constexpr int NW = kDqPPThreads / 64;
  constexpr int BQ = 32 * NW;
  constexpr int KS = D / 16;
  constexpr int CB = D / 32;
  constexpr int KPER = (TL::kKBlocks + NW - 1) / NW;
  constexpr int VPER = (TL::kVBlocks + NW - 1) / NW;
  constexpr int KP = TL::kKPitch, VP = TL::kVPitch;
  __shared__ __attribute__((aligned(1024))) char K0[TL::kKBytes];
  __shared__ __attribute__((aligned(1024))) char K1[TL::kKBytes];
  __shared__ __attribute__((aligned(1024))) char K2[TL::kKBytes];
  __shared__ __attribute__((aligned(1024))) char V0[TL::kVBytes];
  __shared__ __attribute__((aligned(1024))) char V1[TL::kVBytes];
  __shared__ __attribute__((aligned(1024))) char V2[TL::kVBytes];
  __shared__ int simd_slots[4];

  const int t = threadIdx.x;
  const int lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  __builtin_assume(w >= 0 && w < NW);

  int bh, qr;
  tile_order(blockIdx.x, BH, nqt, causal && window < 0, bh, qr);
  const int qt = causal ? nqt - 1 - qr : qr;  // causal: the longest rows first
  const int q0 = qt * BQ;
  const size_t base = (size_t)bh * (size_t)N * D;
  const int qi = q0 + 32 * w + l32;  // this lane's query row

  if (t < 4) simd_slots[t] = 0;
  __syncthreads();
  const int grp = wave_group(simd_slots, lane);

  // Q and dO rows of this lane as B fragments (rows past N read as zero), and
  // the row's L2 and D.
  vec8<T> qf[KS], of[KS];
  {
    const rsrc_t q_src = make_rsrc(q + base, (uint32_t)N * D * 2u);
    const rsrc_t o_src = make_rsrc(dO + base, (uint32_t)N * D * 2u);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint32_t off = (uint32_t)(qi * D + 16 * s + 8 * h) * 2u;
      qf[s] = as_vec8<T>(load16(q_src, off));
      of[s] = as_vec8<T>(load16(o_src, off));
    }
  }
  const bool row_ok = qi < N;
  const float Li = row_ok ? L2[(size_t)bh * N + qi] : 0.f;
  const float Di = row_ok ? Dv[(size_t)bh * N + qi] : 0.f;

  // Key tiles holding at least one key visible to this query tile, the keys
  // this lane's row sees, and the tiles that hold any key visible to this
  // wave's 32 rows (the others it skips).
  const int q_hi = q0 + BQ - 1;
  const int kmin = window >= 0 ? max(0, q0 - window) : 0;
  const int kmax = causal ? min(N - 1, q_hi) : N - 1;
  const int kt0 = kmin / kDqBK, kt1 = kmax / kDqBK + 1;
  const int key_lo = window >= 0 ? qi - window : 0;
  const int key_hi = causal ? min(qi, N - 1) : N - 1;
  const int wq0 = q0 + 32 * w, wq1 = wq0 + 31;
  const int wk_lo = window >= 0 ? max(0, wq0 - window) : 0;
  const int wk_hi = wq0 < N ? (causal ? min(N - 1, wq1) : N - 1) : -1;
  auto active = [&] __device__ (int tile) {
    const int k0 = tile * kDqBK;
    return k0 <= wk_hi && k0 + kDqBK - 1 >= wk_lo;
  };

  uint32_t kpre[KPER], vpre[VPER];
#pragma unroll
  for (int i = 0; i < KPER; ++i) kpre[i] = block_src<D>(w + i * NW, lane, KP);
#pragma unroll
  for (int i = 0; i < VPER; ++i) vpre[i] = block_src<D>(w + i * NW, lane, VP);
  auto kstage = [&] __device__ (auto st) -> char* {
    constexpr int S = decltype(st)::value;
    return S == 0 ? K0 : S == 1 ? K1 : K2;
  };
  auto vstage = [&] __device__ (auto st) -> char* {
    constexpr int S = decltype(st)::value;
    return S == 0 ? V0 : S == 1 ? V1 : V2;
  };
  auto load_share = [&] __device__ (int tile, auto st) {
    const int k0 = tile * kDqBK;
    const uint32_t bytes = (uint32_t)max(0, N - k0) * D * 2u;
    const rsrc_t ks = make_rsrc(k + base + (size_t)k0 * D, bytes);
    const rsrc_t vs = make_rsrc(v + base + (size_t)k0 * D, bytes);
    char* kd = kstage(st);
    char* vd = vstage(st);
#pragma unroll
    for (int i = 0; i < KPER; ++i)
      if (w + i * NW < TL::kKBlocks) load_lds16(ks, kd + (w + i * NW) * 1024, kpre[i]);
#pragma unroll
    for (int i = 0; i < VPER; ++i)
      if (w + i * NW < TL::kVBlocks) load_lds16(vs, vd + (w + i * NW) * 1024, vpre[i]);
  };

  const int k_rd = l32 * KP + 16 * h;  // A operands of S^T (K rows)
  const int v_rd = l32 * VP + 16 * h;  // A operands of dP^T (V rows)
  const int k_tr = tr_addr<KP>(lane);  // A operands of dQ^T (K^T)

  f32x16 dqa[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) dqa[cb] = f32x16{};
  f32x16 sc[2], dpc[2];  // S^T and dP^T of the tile in flight

  // S^T and dP^T of a tile (stage `st`) for its two 32-key blocks.
  auto scores = [&] __device__ (auto st) {
    const char* kn = kstage(st) + k_rd;
    const char* vn = vstage(st) + v_rd;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      sc[kb2] = f32x16{};
      dpc[kb2] = f32x16{};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        sc[kb2] = mfma32(*(const vec8<T>*)(kn + kb2 * 32 * KP + 32 * s), qf[s], sc[kb2]);
        dpc[kb2] = mfma32(*(const vec8<T>*)(vn + kb2 * 32 * VP + 32 * s), of[s], dpc[kb2]);
      }
    }
  };

  using std::integral_constant;
  const int nblk = (TL::kKBlocks - w + NW - 1) / NW + (TL::kVBlocks - w + NW - 1) / NW;
  load_share(kt0, integral_constant<int, 0>{});
  if (kt0 + 1 < kt1) load_share(kt0 + 1, integral_constant<int, 1>{});
  wait_vm(kt0 + 1 < kt1 ? nblk : 0);  // tile kt0 only; tile kt0+1 may still land
  barrier_keep_loads();
  if (active(kt0)) scores(integral_constant<int, 0>{});
  if (grp == 1) {  // group 1 runs one phase behind
    // Its shares of tile kt0+1 must have landed before group 0's first
    // matrix phase (the barrier below opens it); group 0 waits for its own
    // shares before that barrier in its first vector phase.
    wait_vm(0);
    barrier_keep_loads();
  }

  // Tile kt in stage ST: vector phase (P, dS of tile kt), barrier, matrix
  // phase (dQ of tile kt, S and dP of tile kt+1), barrier.
  auto tile_step = [&] __device__ (auto stage, int kt) {
    constexpr int ST = decltype(stage)::value;
    constexpr int STN = (ST + 1) % 3, STF = (ST + 2) % 3;
    const bool load_far = kt + 2 < kt1;
    // ---- vector phase (group 1 also issues its loads of tile kt+2 here)
    if (grp == 1 && load_far) load_share(kt + 2, integral_constant<int, STF>{});
    const bool act = active(kt), act_next = kt + 1 < kt1 && active(kt + 1);
    uint32_t dspk[2][8];
    if (act) {
      const int k0 = kt * kDqBK;
      // (P^T overwrites S^T in place.)
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sc[kb2][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb2][r], scale_log2, -Li));
      const bool need_mask = (k0 + kDqBK > N) || (causal && k0 + kDqBK - 1 > wq0) ||
                             (window >= 0 && k0 < wq1 - window);
      if (need_mask) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb2 * 32 + c_row(r, h);
            sc[kb2][r] = (uint32_t)(key - key_lo) <= (uint32_t)(key_hi - key_lo) ? sc[kb2][r] : 0.f;
          }
      }
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; r += 2)
          dspk[kb2][r >> 1] = pack2<T>(sc[kb2][r] * (dpc[kb2][r] - Di),
                                        sc[kb2][r + 1] * (dpc[kb2][r + 1] - Di));
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) dspk[i][j] = 0u;
    }
    pin_dq_phase<CB>(dspk, dqa);
    // Group 0's matrix phase (after this barrier) needs tile kt+1 whole;
    // group 1 waits for its loads at the end of its matrix phase instead.
    if (grp == 0) wait_vm(0);
    barrier_keep_loads();
    // ---- matrix phase (group 0 issues its loads of tile kt+2 here)
    if (grp == 0 && load_far) load_share(kt + 2, integral_constant<int, STF>{});
    if (act) {
      const char* kc = kstage(integral_constant<int, ST>{}) + k_tr;
#pragma unroll
      for (int s = 0; s < kDqBK / 16; ++s) {
        const uint4 dw = {dspk[s >> 1][4 * (s & 1)], dspk[s >> 1][4 * (s & 1) + 1],
                          dspk[s >> 1][4 * (s & 1) + 2], dspk[s >> 1][4 * (s & 1) + 3]};
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          dqa[cb] = mfma32(read_tr8<KP, T>(kc + 16 * s * KP + 64 * cb), as_vec8<T>(dw), dqa[cb]);
      }
    }
    if (act_next) scores(integral_constant<int, STN>{});
    if (grp == 1) wait_vm(0);
    barrier_keep_loads();
  };

  for (int kt = kt0; kt < kt1; kt += 3) {
    tile_step(integral_constant<int, 0>{}, kt);
    if (kt + 1 >= kt1) break;
    tile_step(integral_constant<int, 1>{}, kt + 1);
    if (kt + 2 >= kt1) break;
    tile_step(integral_constant<int, 2>{}, kt + 2);
  }
  if (grp == 0) barrier_keep_loads();  // match group 1's extra barrier

  // dQ through LDS (after the last barrier no wave reads the stages): two
  // waves per K stage, the last two in V stage 0.
  store_dq_rows<D, CB>(dqa, scale, (w < 2 ? K0 : w < 4 ? K1 : w < 6 ? K2 : V0) + (w & 1) * 32 * (2 * D + 16),
                       dq + base, q0 + 32 * w, N, lane);
}

template <typename T, int D>
hipError_t launch_t(const void* q, const void* k, const void* v, const void* o, const void* dO,
                    const float* lse, float* dq, float* dk, float* dv, int B, int H, int N,
                    float scale, Mask mask, void* ws, int dq_rows, hipStream_t stream) {
  const long long rows = (long long)B * H * N;
  float* Dv = (float*)ws;
  float* L2 = Dv + rows;
  constexpr int RPB = kPreThreads / (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(kPreThreads),
                     0, stream, (const T*)o, (const T*)dO, lse, Dv, L2, rows);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int nkt = (N + kBKV - 1) / kBKV;
  const long long grid = (long long)nkt * B * H;
  hipLaunchKernelGGL((bwd_main_kernel<T, D>), dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     (const T*)q, (const T*)k, (const T*)v, (const T*)dO, Dv, L2, dk, dv,
                     B * H, N, nkt, scale, scale * kLog2e, mask.causal, mask.window);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  // dQ: the ping-pong kernel (256 query rows per workgroup) or the 4-wave
  // kernel (128 rows).
  if (dq_rows == 256) {
    const int nqt = (N + 255) / 256;
    hipLaunchKernelGGL((bwd_dq_pp_kernel<T, D>), dim3((unsigned)((long long)nqt * B * H)), dim3(kDqPPThreads),
                       0, stream, (const T*)q, (const T*)k, (const T*)v, (const T*)dO, Dv,
                       L2, dq, B * H, N, nqt, scale, scale * kLog2e, mask.causal, mask.window);
  } else {
    constexpr int BQ = kDqThreads / 2;  // 32 query rows per wave
    const int nqt = (N + BQ - 1) / BQ;
    hipLaunchKernelGGL((bwd_dq_kernel<T, D>), dim3((unsigned)((long long)nqt * B * H)), dim3(kDqThreads), 0,
                       stream, (const T*)q, (const T*)k, (const T*)v, (const T*)dO, Dv, L2,
                       dq, B * H, N, nqt, scale, scale * kLog2e, mask.causal, mask.window);
  }
  return hipGetLastError();
}

}  // namespace

int bwd_auto_dq_rows(int B, int H, int N) {
  // The ping-pong dQ kernel while its grid (256 rows per workgroup, one per
  // CU) still fills the 256 CUs, else the 4-wave kernel.
  return (long long)B * H * ((N + 255) / 256) >= 256 ? 256 : 128;
}

size_t bwd_workspace_bytes(int B, int H, int N, int d) {
  (void)d;
  return (size_t)B * H * N * 2 * sizeof(float);
}

hipError_t launch_bwd_mfma(const void* q, const void* k, const void* v, const void* o,
                           const void* dO, const float* lse, float* dq, float* dk, float* dv,
                           int B, int H, int N, int d, float scale, Mask mask, void* ws, bool f16,
                           int dq_rows, hipStream_t stream) {
  if (dq_rows != 128 && dq_rows != 256) dq_rows = bwd_auto_dq_rows(B, H, N);
  if (f16) {
    if (d == 128)
      return launch_t<fa::f16, 128>(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, scale, mask, ws, dq_rows, stream);
    return launch_t<fa::f16, 64>(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, scale, mask, ws, dq_rows, stream);
  }
  if (d == 128)
    return launch_t<bf16, 128>(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, scale, mask, ws, dq_rows, stream);
  return launch_t<bf16, 64>(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, scale, mask, ws, dq_rows, stream);
}

}  // namespace fa
