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
// Mapping onto CDNA4 (v_mfma_f32_32x32x16_bf16 / _f16, fp32 accumulation).
// With a workspace that holds dS (the stored-dS path), three kernels on one
// stream: bwd_pre (D and L in log2 units), bwd_kv4 below, which also writes
// each dS block it forms, and bwd_dq_ds, dQ = scale dS K from those blocks
// -- the page's five products, nothing recomputed.  Otherwise (the recompute
// path) two kernels on one stream:
//  * bwd_dq4 (4 waves, two workgroups per CU) or bwd_dq_pp (8 waves in two
//    groups one phase apart, for grids that fill the chip): dQ, with the
//    loops the other way round (a workgroup owns 128 or 256 query rows and
//    walks the key tiles, as the forward does), recomputing S, P, dP and dS;
//    no atomics, so dQ is deterministic.  Owning every query row once, it also
//    forms the page's first step, D = rowsum(dO * O), and L in log2 units
//    for the next kernel.
//  * bwd_kv4: dK and dV, in the page's loop order (key/value tiles outer):
//    a workgroup of 4 waves owns a 128-key tile and walks the query tiles.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kBKV = 128;  // keys per dK / dV workgroup

// Where the dK / dV kernel leaves dS for the dQ product: one 32 x 32 block
// (2 KB) per (query block qb, key block kb) that holds a visible pair, at
// block index ds_block(qb, kb) of its (batch, head) slice:
//  * mode 1, causal without a window: the lower triangle, qb (qb + 1) / 2 + kb;
//  * mode 2, causal with a window of W keys: a band of A + 1 blocks per
//    query block, A = ceil(W / 32), slot kb - qb + A (kb >= qb - A for every
//    visible block);
//  * mode 0, otherwise: every block, qb nb + kb.
struct DsLayout {
  int mode;
  int nb;              // 32-row blocks per slice
  int A;               // band: ceil(window / 32)
  int width;           // band: blocks per query block
  long long per_head;  // blocks per slice
};

__host__ __device__ __forceinline__ long long ds_block(const DsLayout& L, int qb, int kb) {
  return L.mode == 1   ? (long long)qb * (qb + 1) / 2 + kb
         : L.mode == 2 ? (long long)qb * L.width + kb - qb + L.A
                       : (long long)qb * L.nb + kb;
}

// Byte offset of the dS blocks in the workspace: after D and L2 (two floats
// per query row), 256-byte aligned.
size_t ds_offset(long long rows) { return ((size_t)rows * 8u + 255u) / 256u * 256u; }

DsLayout ds_layout(int N, int causal, int window) {
  DsLayout L{};
  L.nb = (N + 31) / 32;
  if (causal && (window < 0 || (window + 31) / 32 >= L.nb)) {  // a window over the whole slice: triangle
    L.mode = 1;
    L.per_head = (long long)L.nb * (L.nb + 1) / 2;
  } else if (causal) {
    L.mode = 2;
    L.A = (window + 31) / 32;
    L.width = L.A + 1;
    L.per_head = (long long)L.nb * L.width;
  } else {
    L.mode = 0;
    L.per_head = (long long)L.nb * L.nb;
  }
  return L;
}


// dK / dV kernel with four waves and two workgroups per CU.  A workgroup owns
// 128 keys, 32 per wave, and walks the query tiles that see them 32 queries
// at a time.  Each wave forms S = Q K^T and dP = dO V^T for its own 32 keys
// and all 32 queries of the step, so P and dS never leave the wave: in the
// 32x32 accumulator layout a lane holds one key and 16 queries, which is
// already the A operand (keys x queries) of dV += P^T dO and dK += dS^T Q
// once the queries run in the accumulator's row order -- the order in which
// the transpose reads deliver the rows of the dO and Q tiles.  Without the
// exchange of P and dS there is one workgroup barrier per step (the query
// tile's stage recycling), and the two workgroups that share a CU (one wave
// of each per SIMD) run independently, so one's vector work, barriers and
// start-up overlap the other's matrix work.
//  * K: a 128-row tile in LDS (B operands of S, 16-byte reads), loaded once;
//    V: this wave's 32 rows in registers (B operands of dP);
//  * Q, dO, L2 and D of the next query tile stream into LDS by direct loads
//    while the current one is processed (two stages);
//  * a wave skips the steps in which every key it owns is hidden from every
//    query of the tile (the causal diagonal, a window's far edge).
constexpr int kKv4Threads = 256;
constexpr int kKv4BQ = 32;  // queries per step

template <int D>
struct Kv4Tile {
  static constexpr int kKPitch = 2 * D + 16;                 // K rows: 16-byte reads
  static constexpr int kQPitch = D == 128 ? 304 : 144;       // Q / dO rows: 16-byte and transpose reads
  static constexpr int kKBytes = kBKV * kKPitch;
  static constexpr int kQBytes = (kKv4BQ * kQPitch + 1023) / 1024 * 1024;
  static constexpr int kKBlocks = kKBytes / 1024;
  static constexpr int kQBlocks = kQBytes / 1024;
  static_assert(kKBytes % 1024 == 0, "K tile must be whole 1 KB blocks");
};

// block_src for a tile of `rows` rows: lanes past the last row or on row
// padding read zero.
template <int D>
__device__ __forceinline__ uint32_t block_src_rows(int blk, int lane, int pitch, int rows) {
  const int pos = blk * 1024 + lane * 16;
  const int row = pos / pitch, col = pos - row * pitch;
  return row < rows && col < D * 2 ? (uint32_t)(row * D * 2 + col) : 0x80000000u;
}

template <typename T, int D, bool DS>
__global__ __launch_bounds__(kKv4Threads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_kv4_kernel(const T* __restrict__ q, const T* __restrict__ k,
                    const T* __restrict__ v, const T* __restrict__ dO,
                    const float* __restrict__ Dv, const float* __restrict__ L2,
                    float* __restrict__ dk, float* __restrict__ dv, T* __restrict__ dsw, DsLayout lay,
                    int BH, int N, int nkt, float scale, float scale_log2, int causal, int window) {
  using TL = Kv4Tile<D>;
  constexpr int NW = kKv4Threads / 64;  // 4
  constexpr int KS = D / 16;            // 16-wide steps over the head dimension
  constexpr int CB = D / 32;            // 32-column blocks of dK / dV
  constexpr int KPER = (TL::kKBlocks + NW - 1) / NW;
  constexpr int QPER = (TL::kQBlocks + NW - 1) / NW;
  constexpr int KP = TL::kKPitch, QP = TL::kQPitch;
  __shared__ __attribute__((aligned(1024))) char Kt[TL::kKBytes];
  __shared__ __attribute__((aligned(1024))) char Q0[TL::kQBytes];
  __shared__ __attribute__((aligned(1024))) char Q1[TL::kQBytes];
  __shared__ __attribute__((aligned(1024))) char O0[TL::kQBytes];
  __shared__ __attribute__((aligned(1024))) char O1[TL::kQBytes];
  __shared__ __attribute__((aligned(256))) float LD0[128];  // L2 in [0, 64), D in [64, 128)
  __shared__ __attribute__((aligned(256))) float LD1[128];

  const int t = threadIdx.x;
  const int lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // uniform: keeps per-wave branches scalar
  __builtin_assume(w >= 0 && w < NW);

  int bh, kt;
  tile_order(blockIdx.x, BH, nkt, causal && window < 0, bh, kt);  // heaviest key tile (kt = 0) first
  const int k0 = kt * kBKV;
  const size_t base = (size_t)bh * (size_t)N * D;
  const int wk0 = k0 + 32 * w;           // this wave's keys: wk0 .. wk0 + 31
  const int wk1 = min(wk0 + 31, N - 1);  // the last of them that exists
  const int my_key = wk0 + l32;

  // K tile (rows past N read as zero) and this wave's V rows.
  {
    const rsrc_t k_src = make_rsrc(k + base + (size_t)k0 * D, (uint32_t)max(0, N - k0) * D * 2u);
#pragma unroll
    for (int i = 0; i < KPER; ++i) {
      const int blk = w + i * NW;
      if (blk < TL::kKBlocks) load_lds16(k_src, Kt + blk * 1024, block_src_rows<D>(blk, lane, KP, kBKV));
    }
  }
  vec8<T> vf[KS];
  {
    const rsrc_t v_src = make_rsrc(v + base, (uint32_t)N * D * 2u);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      vf[s] = as_vec8<T>(load16(v_src, (uint32_t)(my_key * D + 16 * s + 8 * h) * 2u));
  }

  // Query tiles that see at least one of this workgroup's keys.
  const int k_hi = k0 + kBKV - 1;
  const int qmin = causal ? k0 : 0;
  const int qmax = window >= 0 ? min(N - 1, k_hi + window) : N - 1;
  const int qt0 = qmin / kKv4BQ, qt1 = qmax / kKv4BQ + 1;

  uint32_t qpre[QPER];
#pragma unroll
  for (int i = 0; i < QPER; ++i) qpre[i] = block_src_rows<D>(w + i * NW, lane, QP, kKv4BQ);
  auto stage_q = [&] __device__ (auto st) -> char* { return decltype(st)::value == 0 ? Q0 : Q1; };
  auto stage_o = [&] __device__ (auto st) -> char* { return decltype(st)::value == 0 ? O0 : O1; };
  auto stage_ld = [&] __device__ (auto st) -> float* { return decltype(st)::value == 0 ? LD0 : LD1; };
  const float* Lrow = L2 + (size_t)bh * N;
  const float* Drow = Dv + (size_t)bh * N;
  // This wave's share of the direct loads of query tile qt into stage st.
  auto load_qtile = [&] __device__ (int qt, auto st) {
    const int q0 = qt * kKv4BQ;
    const uint32_t bytes = (uint32_t)max(0, N - q0) * D * 2u;
    const rsrc_t qs = make_rsrc(q + base + (size_t)q0 * D, bytes);
    const rsrc_t os = make_rsrc(dO + base + (size_t)q0 * D, bytes);
#pragma unroll
    for (int i = 0; i < QPER; ++i) {
      const int blk = w + i * NW;
      if (blk < TL::kQBlocks) {
        load_lds16(qs, stage_q(st) + blk * 1024, qpre[i]);
        load_lds16(os, stage_o(st) + blk * 1024, qpre[i]);
      }
    }
    if (w < 2) {
      const rsrc_t ls = make_rsrc((w == 0 ? Lrow : Drow) + q0, (uint32_t)max(0, N - q0) * 4u);
      load_lds4(ls, stage_ld(st) + w * 64, (uint32_t)lane * 4u);
    }
  };

  using std::integral_constant;
  if (qt0 < qt1) load_qtile(qt0, integral_constant<int, 0>{});
  // The V rows above must be in flight together with the tile's loads:
  // left to itself the compiler issued them only after the wait below, so
  // the two round trips to memory ran one after the other.  An empty asm
  // that reads them here keeps them ahead of the wait.
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
  for (int s = 0; s < KS; ++s) asm volatile("" : "+v"(vf[s]));
#endif
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  f32x16 dk_acc[CB], dv_acc[CB];
#pragma unroll
  for (int c = 0; c < CB; ++c) {
    dk_acc[c] = f32x16{};
    dv_acc[c] = f32x16{};
  }
  const int q_rd = l32 * QP + 16 * h;              // A operands of S and dP (Q, dO rows)
  const int k_rd = (32 * w + l32) * KP + 16 * h;   // B operands of S (K rows)
  const int tr_q = tr_addr<QP>(lane);              // B operands of dV / dK

  // With DS each step's dS block is stored at the start of the next step,
  // so that the stores complete during a whole step of work instead of
  // holding up the step's closing wait.
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  uint32_t dpend[8];
  char* pend = nullptr;
  auto store_pending = [&] __device__ () {
    if (pend) {
      __builtin_nontemporal_store(u32x4{dpend[0], dpend[1], dpend[2], dpend[3]}, (u32x4*)(pend + lane * 16));
      __builtin_nontemporal_store(u32x4{dpend[4], dpend[5], dpend[6], dpend[7]}, (u32x4*)(pend + 1024 + lane * 16));
    }
  };
  auto tile = [&] __device__ (auto stage, int qt) {
    constexpr int ST = decltype(stage)::value;
    const char* Qs = stage_q(stage);
    const char* Os = stage_o(stage);
    const float* LD = stage_ld(stage);
    const int q0 = qt * kKv4BQ;
    if (qt + 1 < qt1) load_qtile(qt + 1, integral_constant<int, ST ^ 1>{});
    if constexpr (DS) {
      store_pending();
      pend = nullptr;
    }
    const bool act = wk0 <= wk1 && !(causal && wk0 > q0 + kKv4BQ - 1) && !(window >= 0 && wk1 < q0 - window);
    if (act) {
      const bool need_mask = (causal && wk0 + 31 > q0) || (window >= 0 && q0 + kKv4BQ - 1 - wk0 > window) ||
                             (wk0 + 31 >= N) || (q0 + kKv4BQ > N);
      // S = Q K^T and dP = dO V^T, then P = exp2(S c - L2) and dS = P (dP - D)
      // on the vector ALUs, then dV += P^T dO and dK += dS^T Q, 16 queries
      // per MFMA step.  (The compiler's own instruction order measured
      // fastest here: with every register of the lane in use, explicit
      // interleaving patterns only delayed the operand reads.)
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        sacc = mfma32(*(const vec8<T>*)(Qs + q_rd + 32 * s), *(const vec8<T>*)(Kt + k_rd + 32 * s), sacc);
#pragma unroll
      for (int s = 0; s < KS; ++s)
        dpacc = mfma32(*(const vec8<T>*)(Os + q_rd + 32 * s), vf[s], dpacc);
      float pv[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 L4 = *(const float4*)(LD + 8 * g + 4 * h);
        pv[4 * g + 0] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[4 * g + 0], scale_log2, -L4.x));
        pv[4 * g + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[4 * g + 1], scale_log2, -L4.y));
        pv[4 * g + 2] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[4 * g + 2], scale_log2, -L4.z));
        pv[4 * g + 3] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[4 * g + 3], scale_log2, -L4.w));
      }
      // Hidden pairs get P = 0 (one branch around the whole step).
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qrow = q0 + c_row(r, h);
          const int lo = window >= 0 ? qrow - window : 0;
          const int hi = min(causal ? qrow : N - 1, N - 1);
          const bool vis = (qrow < N) & ((uint32_t)(my_key - lo) <= (uint32_t)(hi - lo));
          pv[r] = vis ? pv[r] : 0.f;
        }
      }
      uint32_t ppk[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) ppk[j] = pack2<T>(pv[2 * j], pv[2 * j + 1]);
      uint32_t dspk[8];
      auto form_ds = [&] __device__ () {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 D4 = *(const float4*)(LD + 64 + 8 * g + 4 * h);
          dspk[2 * g] = pack2<T>(pv[4 * g] * (dpacc[4 * g] - D4.x), pv[4 * g + 1] * (dpacc[4 * g + 1] - D4.y));
          dspk[2 * g + 1] = pack2<T>(pv[4 * g + 2] * (dpacc[4 * g + 2] - D4.z),
                                      pv[4 * g + 3] * (dpacc[4 * g + 3] - D4.w));
        }
      };
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const vec8<T> pa = as_vec8<T>(uint4{ppk[4 * s], ppk[4 * s + 1], ppk[4 * s + 2], ppk[4 * s + 3]});
#pragma unroll
        for (int c = 0; c < CB; ++c)
          dv_acc[c] = mfma32(pa, read_tr8<QP, T>(Os + tr_q + 16 * s * QP + 64 * c), dv_acc[c]);
      }
      form_ds();
      if constexpr (DS) {
        // The block is stored at the start of the next step.  The 32 x 32 dS
        // block of (query block qt, this wave's key block) holds in lane
        // order the lane's 16 values -- slots 16 h .. 16 h + 15 of its key's
        // row, slot 16 h + r for query c_row(r, h) --, the first eight at
        // 16 lane, the last eight at 1024 + 16 lane, so that each store
        // instruction writes 1 KB contiguous.  Written once and read once by
        // the next kernel: non-temporal stores.
        pend = (char*)(dsw + ((size_t)bh * (size_t)lay.per_head + (size_t)ds_block(lay, qt, wk0 >> 5)) * 1024);
#pragma unroll
        for (int j = 0; j < 8; ++j) dpend[j] = dspk[j];
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const vec8<T> da = as_vec8<T>(uint4{dspk[4 * s], dspk[4 * s + 1], dspk[4 * s + 2], dspk[4 * s + 3]});
#pragma unroll
        for (int c = 0; c < CB; ++c)
          dk_acc[c] = mfma32(da, read_tr8<QP, T>(Qs + tr_q + 16 * s * QP + 64 * c), dk_acc[c]);
      }
    }
    // The next tile's direct loads have landed (and, with DS, this step's
    // dS stores); after the barrier no wave reads this stage any more.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  for (int qt = qt0; qt < qt1; qt += 2) {
    tile(integral_constant<int, 0>{}, qt);
    if (qt + 1 >= qt1) break;
    tile(integral_constant<int, 1>{}, qt + 1);
  }

  if constexpr (DS) store_pending();
  // dK = scale * dS^T Q, dV = P^T dO for this wave's keys; rows past N fall
  // outside the buffers and are dropped.
  const rsrc_t dk_dst = make_rsrc(dk + base, (uint32_t)N * D * 4u);
  const rsrc_t dv_dst = make_rsrc(dv + base, (uint32_t)N * D * 4u);
#pragma unroll
  for (int c = 0; c < CB; ++c) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t off = ((uint32_t)(wk0 + c_row(r, h)) * D + 32 * c + l32) * 4u;
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

// Per-row constants of the backward for this lane's query row qi, formed by
// the dQ kernels (which own every query row once and hold its dO already):
// D = rowsum(dO * O) (the two lanes of a row each sum half of the columns)
// and L2 = L * log2(e) (+inf for a row without visible keys, so that every P
// of it is 0).  Stored for the dK / dV kernel, which runs after them.
// In three parts, so that the loads of O and L travel with the kernel's first
// K/V tile instead of taking a memory round trip of their own: issue the
// loads, form D and L2 once the first tile's wait has passed, store them at
// the end.
template <int KS>
struct RowConstants {
  uint4 o[KS];  // this lane's half of the O row, as the dO fragments
  float L;
};
template <int KS>
__device__ __forceinline__ void row_constants_load(RowConstants<KS>& rc, rsrc_t o_src, uint32_t row_off,
                                                   const float* __restrict__ lse, size_t row, bool row_ok) {
#pragma unroll
  for (int s = 0; s < KS; ++s) rc.o[s] = load16(o_src, row_off + 32u * s);
  rc.L = row_ok ? lse[row] : 0.f;
}
template <typename T, int KS>
__device__ __forceinline__ void row_constants_form(const RowConstants<KS>& rc, const vec8<T> (&of)[KS], float& Di,
                                                   float& Li) {
  float p = 0.f;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const uint4 b = __builtin_bit_cast(uint4, of[s]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p = __builtin_fmaf(lo16<T>(word(rc.o[s], i)), lo16<T>(word(b, i)), p);
      p = __builtin_fmaf(hi16<T>(word(rc.o[s], i)), hi16<T>(word(b, i)), p);
    }
  }
  Di = pair_sum(p);
  Li = rc.L == kNegInf ? __builtin_inff() : rc.L * kLog2e;
}
__device__ __forceinline__ void row_constants_store(float* __restrict__ Dv, float* __restrict__ L2, size_t row,
                                                    bool row_ok, int h, float Di, float Li) {
  if (row_ok && h == 0) {
    Dv[row] = Di;
    L2[row] = Li;
  }
}

constexpr int kDqBK = 64;  // keys per tile of the ping-pong dQ kernel

// dQ kernel with four waves and two workgroups per CU (the counterpart of
// bwd_kv4_kernel): a workgroup owns 128 query rows, 32 per wave (one per lane
// pair, Q and dO rows in registers as B operands, L2 and D one value per
// lane), and walks the keys that see them KB * 32 at a time (KB = 1 at
// d = 128, where two 32-key blocks would not fit two waves per SIMD; 2 at
// d = 64), recomputing
//   S^T = K Q^T,  dP^T = V dO^T        (K and V rows from LDS),
//   P^T = exp2(S^T c - L2),  dS^T = P^T (dP^T - D),
//   dQ^T += K^T dS^T                    (K^T by transpose reads, dS^T packed
//                                        straight from the accumulator).
// One workgroup barrier per step (the K / V stage recycling); a wave skips
// the steps whose keys are all hidden from its 32 rows.
constexpr int kDq4Threads = 256;

template <int D, int KB>
struct Dq4Tile {
  static constexpr int kBK = 32 * KB;                    // keys per step
  static constexpr int kKPitch = D == 128 ? 304 : 144;  // K rows: 16-byte and transpose reads
  static constexpr int kVPitch = 2 * D + 16;             // V rows: 16-byte reads
  static constexpr int kKBytes = (kBK * kKPitch + 1023) / 1024 * 1024;
  static constexpr int kVBytes = (kBK * kVPitch + 1023) / 1024 * 1024;
  static constexpr int kKBlocks = kKBytes / 1024;
  static constexpr int kVBlocks = kVBytes / 1024;
  // Each wave stages its dQ rows (32 rows of 2 D + 16 bytes) in one buffer.
  static_assert(32 * (2 * D + 16) <= kKBytes && 32 * (2 * D + 16) <= kVBytes, "dQ staging");
};

template <typename T, int D, int KB>
__global__ __launch_bounds__(kDq4Threads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq4_kernel(const T* __restrict__ q, const T* __restrict__ k,
                    const T* __restrict__ v, const T* __restrict__ dO,
                    const T* __restrict__ o, const float* __restrict__ lse,
                    float* __restrict__ Dv, float* __restrict__ L2,
                    float* __restrict__ dq, int BH, int N, int nqt, float scale, float scale_log2,
                    int causal, int window) {
  using TL = Dq4Tile<D, KB>;
  constexpr int BK = TL::kBK;
  constexpr int NW = kDq4Threads / 64;
  constexpr int BQ = 32 * NW;
  constexpr int KS = D / 16;
  constexpr int CB = D / 32;
  constexpr int KPER = (TL::kKBlocks + NW - 1) / NW;
  constexpr int VPER = (TL::kVBlocks + NW - 1) / NW;
  constexpr int KP = TL::kKPitch, VP = TL::kVPitch;
  __shared__ __attribute__((aligned(1024))) char K0[TL::kKBytes];
  __shared__ __attribute__((aligned(1024))) char K1[TL::kKBytes];
  __shared__ __attribute__((aligned(1024))) char V0[TL::kVBytes];
  __shared__ __attribute__((aligned(1024))) char V1[TL::kVBytes];

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
  // (rows past N read as zero), and the row's D and L2.
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
  RowConstants<KS> rc;
  row_constants_load<KS>(rc, make_rsrc(o + base, (uint32_t)N * D * 2u), (uint32_t)(qi * D + 8 * h) * 2u, lse,
                         (size_t)bh * N + qi, row_ok);
  float Li, Di;  // formed once the first tile's wait has passed

  // Key steps holding a key visible to any row of the workgroup, the keys
  // this lane's row sees, and those any row of this wave sees.
  const int q_hi = q0 + BQ - 1;
  const int kmin = window >= 0 ? max(0, q0 - window) : 0;
  const int kmax = causal ? min(N - 1, q_hi) : N - 1;
  const int kt0 = kmin / BK, kt1 = kmax / BK + 1;
  const int key_lo = window >= 0 ? qi - window : 0;
  const int key_hi = causal ? min(qi, N - 1) : N - 1;
  const int wq0 = q0 + 32 * w, wq1 = wq0 + 31;
  const int wk_lo = window >= 0 ? max(0, wq0 - window) : 0;
  const int wk_hi = wq0 < N ? (causal ? min(N - 1, wq1) : N - 1) : -1;

  uint32_t kpre[KPER], vpre[VPER];
#pragma unroll
  for (int i = 0; i < KPER; ++i) kpre[i] = block_src_rows<D>(w + i * NW, lane, KP, BK);
#pragma unroll
  for (int i = 0; i < VPER; ++i) vpre[i] = block_src_rows<D>(w + i * NW, lane, VP, BK);
  auto load_kv = [&] __device__ (int kt, char* kd, char* vd) {
    const int k0 = kt * BK;
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

  if (kt0 < kt1) load_kv(kt0, K0, V0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  row_constants_form<T, KS>(rc, of, Di, Li);

  auto tile = [&] __device__ (auto parity, int kt) {
    constexpr int P = decltype(parity)::value;
    const char* Kc = P ? K1 : K0;
    const char* Vc = P ? V1 : V0;
    if (kt + 1 < kt1) load_kv(kt + 1, P ? K0 : K1, P ? V0 : V1);
    const int k0 = kt * BK;
    if (k0 <= wk_hi && k0 + BK - 1 >= wk_lo) {
      const bool need_mask = (k0 + BK > N) || (causal && k0 + BK - 1 > wq0) || (window >= 0 && k0 < wq1 - window);
      f32x16 sc[KB], dpc[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        sc[kb] = f32x16{};
        dpc[kb] = f32x16{};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          sc[kb] = mfma32(*(const vec8<T>*)(Kc + k_rd + kb * 32 * KP + 32 * s), qf[s], sc[kb]);
          dpc[kb] = mfma32(*(const vec8<T>*)(Vc + v_rd + kb * 32 * VP + 32 * s), of[s], dpc[kb]);
        }
      }
      // P^T = exp2(S^T c - L2) (overwriting S^T), hidden keys at 0.
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sc[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][r], scale_log2, -Li));
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + c_row(r, h);
            sc[kb][r] = (uint32_t)(key - key_lo) <= (uint32_t)(key_hi - key_lo) ? sc[kb][r] : 0.f;
          }
      }
      uint32_t dspk[KB][8];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2)
          dspk[kb][r >> 1] = pack2<T>(sc[kb][r] * (dpc[kb][r] - Di), sc[kb][r + 1] * (dpc[kb][r + 1] - Di));
      // dQ^T += K^T dS^T, 16 keys per step.
#pragma unroll
      for (int s = 0; s < BK / 16; ++s) {
        const uint4 dw = {dspk[s >> 1][4 * (s & 1)], dspk[s >> 1][4 * (s & 1) + 1], dspk[s >> 1][4 * (s & 1) + 2],
                          dspk[s >> 1][4 * (s & 1) + 3]};
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          dqa[cb] = mfma32(read_tr8<KP, T>(Kc + k_tr + 16 * s * KP + 64 * cb), as_vec8<T>(dw), dqa[cb]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads of the next tile have landed
    __syncthreads();
  };

  for (int kt = kt0; kt < kt1; kt += 2) {
    tile(std::integral_constant<int, 0>{}, kt);
    if (kt + 1 >= kt1) break;
    tile(std::integral_constant<int, 1>{}, kt + 1);
  }

  // dQ through LDS (the loop's last barrier freed the stages): one buffer per
  // wave.
  store_dq_rows<D, CB>(dqa, scale, w == 0 ? K0 : w == 1 ? K1 : w == 2 ? V0 : V1, dq + base, q0 + 32 * w, N,
                       lane);
  row_constants_store(Dv, L2, (size_t)bh * N + qi, row_ok, h, Di, Li);
}

// Ping-pong dQ kernel for long sequences: 8 waves, 256 query rows per
// workgroup, the same computation as bwd_dq4_kernel.  The waves form two groups
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
#else
  (void)ds; (void)acc;
#endif
}

template <typename T, int D>
__global__ __launch_bounds__(kDqPPThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_pp_kernel(const T* __restrict__ q, const T* __restrict__ k,
                      const T* __restrict__ v, const T* __restrict__ dO,
                      const T* __restrict__ o, const float* __restrict__ lse,
                      float* __restrict__ Dv, float* __restrict__ L2,
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
  RowConstants<KS> rc;
  row_constants_load<KS>(rc, make_rsrc(o + base, (uint32_t)N * D * 2u), (uint32_t)(qi * D + 8 * h) * 2u, lse,
                         (size_t)bh * N + qi, row_ok);
  float Li, Di;  // formed once the first tile's wait has passed

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
  wait_vm(kt0 + 1 < kt1 ? nblk : 0);  // tile kt0 only (and O and L, issued before it); tile kt0+1 may still land
  row_constants_form<T, KS>(rc, of, Di, Li);
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
  row_constants_store(Dv, L2, (size_t)bh * N + qi, row_ok, h, Di, Li);
}


// D = rowsum(dO * O) and L2 = L log2(e) (+inf for a row without visible keys)
// of every query row, for the stored-dS backward (whose dK / dV kernel runs
// first): 8 lanes of 16 bytes per 64 columns, D / 8 lanes per row.
constexpr int kPreThreads = 256;

template <typename T, int D>
__global__ __launch_bounds__(kPreThreads)
void bwd_pre_kernel(const T* __restrict__ o, const T* __restrict__ dO, const float* __restrict__ lse,
                    float* __restrict__ Dv, float* __restrict__ L2, long long rows) {
  constexpr int LPR = D / 8;                   // lanes per row
  constexpr int RPB = kPreThreads / LPR;       // rows per workgroup
  const int t = threadIdx.x;
  const long long row = (long long)blockIdx.x * RPB + t / LPR;
  const int part = t % LPR;
  float p = 0.f;
  if (row < rows) {  // each element is read once: non-temporal loads
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const uint4 a = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4*)(o + (size_t)row * D + 8 * part)));
    const uint4 b = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4*)(dO + (size_t)row * D + 8 * part)));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p = __builtin_fmaf(lo16<T>(word(a, i)), lo16<T>(word(b, i)), p);
      p = __builtin_fmaf(hi16<T>(word(a, i)), hi16<T>(word(b, i)), p);
    }
  }
  p = group_sum<LPR>(p);
  if (row < rows && part == 0) {
    const float L = lse[row];
    Dv[row] = p;
    L2[row] = L == kNegInf ? __builtin_inff() : L * kLog2e;
  }
}

// dQ = scale * dS K from the dS blocks the dK / dV kernel stored: the
// product of "Building Flash Attention from Scratch in Pure NumPy", Step 4,
// with nothing recomputed.  Four waves own 128 query rows (32 each) and walk
// the key blocks their rows see, two 32-key blocks per step.  The kernel
// streams the dS blocks once from HBM: each wave keeps the dS blocks of its
// next four steps in flight in registers (non-temporal loads), and the
// workgroup's K rows (read by every query tile of the slice, mostly from L2)
// come through a ring of four LDS stages by direct loads.  (Loads retire in
// issue order, so the dS loads run no further ahead than the K stages: a
// wait for step i's K rows also waits for every dS load issued before
// them.)  Per block a wave copies its dS block into its own 2 KB of LDS,
// row-major by key (16-byte chunks swizzled), and forms
//   dQ^T += K^T dS^T
// with K^T and dS^T both from transpose reads (those of the dS tile give the
// queries as the accumulator's columns).  A wave skips the blocks that hold
// no pair visible to its rows (the dK / dV kernel never wrote them).
constexpr int kDsThreads = 256;
constexpr int kDsKB = 2;      // 32-key blocks per step
constexpr int kDsStages = 4;  // K stages, and steps of dS in flight per wave

// s_waitcnt on the vector-memory counter only, for any count up to 63 (the
// counter's width on gfx950: four low bits and two high bits of the
// immediate).
template <int N>
__device__ __forceinline__ void wait_vm_n() {
  static_assert(N >= 0 && N <= 63, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// The K rows of one step (kDsKB blocks of 32 keys), unpadded (2 D bytes per
// row), with the 16-byte chunks of each row permuted by an XOR with a
// function of the row, so that the transpose reads of four consecutive rows
// hit distinct LDS banks (unpadded rows 256 or 128 bytes apart would all
// start on the same bank).  16 KB per stage at d = 128, so that four stages
// fit two workgroups per CU.
template <int D>
struct DsTile {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kKBytes = 32 * kDsKB * kRowBytes;
  static constexpr int kKBlocks = kKBytes / 1024;
  static constexpr int kKPer = kKBlocks / 4;  // direct loads per wave and step
  static_assert(kKBlocks % 4 == 0, "K blocks per wave");
  // XOR applied to the 16-byte chunk index of row r: rows r .. r + 3 of a
  // transpose read then start 64 bytes apart modulo the 256-byte bank cycle.
  static __device__ __forceinline__ int chunk_xor(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

template <typename T, int D>
__global__ __launch_bounds__(kDsThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_ds_kernel(const T* __restrict__ k, const T* __restrict__ dsw, DsLayout lay,
                      float* __restrict__ dq, int BH, int N, int nqt, float scale, int causal, int window) {
  using TL = DsTile<D>;
  constexpr int NW = kDsThreads / 64;  // 4
  constexpr int BQ = 32 * NW;          // 128 query rows
  constexpr int CB = D / 32;
  constexpr int RB = TL::kRowBytes;
  constexpr int KPER = TL::kKPer;
  constexpr int KB = kDsKB;
  constexpr int S = kDsStages;
  // One LDS object per K stage, so that the compiler can tell the stages'
  // direct loads apart and wait only for the stage it reads.
  __shared__ __attribute__((aligned(1024))) char T0[TL::kKBytes];
  __shared__ __attribute__((aligned(1024))) char T1[TL::kKBytes];
  __shared__ __attribute__((aligned(1024))) char T2[TL::kKBytes];
  __shared__ __attribute__((aligned(1024))) char T3[TL::kKBytes];
  __shared__ __attribute__((aligned(1024))) char Sd[NW * 2048];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  __builtin_assume(w >= 0 && w < NW);

  int bh, qr;
  tile_order(blockIdx.x, BH, nqt, causal && window < 0, bh, qr);
  const int qt = causal ? nqt - 1 - qr : qr;  // causal: the longest rows first
  const int q0 = qt * BQ;
  const int wq0 = q0 + 32 * w;  // this wave's rows: wq0 .. wq0 + 31
  const int qb = wq0 >> 5;
  const size_t base = (size_t)bh * (size_t)N * D;
  const T* ds_slice = dsw + (size_t)bh * (size_t)lay.per_head * 1024;
  char* Sw = Sd + w * 2048;

  // Key blocks holding a key visible to any row of the workgroup, KB per step.
  const int kmin = window >= 0 ? max(0, q0 - window) : 0;
  const int kmax = causal ? min(N - 1, q0 + BQ - 1) : N - 1;
  const int kb0 = kmin >> 5, nsteps = ((kmax >> 5) + 1 - kb0 + KB - 1) / KB;
  // Whether key block kb holds a pair visible to this wave's rows -- the
  // test under which the dK / dV kernel stored the block.
  auto visible = [&] __device__ (int kb) {
    const int kk0 = kb * 32, kk1 = min(kk0 + 31, N - 1);
    return kk0 < N && wq0 < N && !(causal && kk0 > wq0 + 31) && !(window >= 0 && kk1 < wq0 - window);
  };

  // Source offset of this lane's 16 bytes in each of its K blocks: LDS
  // chunk c of row r holds K chunk c ^ chunk_xor(r).
  uint32_t kpre[KPER];
#pragma unroll
  for (int j = 0; j < KPER; ++j) {
    const int pos = (w + j * NW) * 1024 + lane * 16;
    const int r = pos / RB, c = (pos % RB) / 16;
    kpre[j] = (uint32_t)(r * RB + ((c ^ TL::chunk_xor(r)) * 16));
  }
  // Every wave issues the same loads per step -- KPER direct loads of K rows
  // and two 16-byte loads per dS block (steps past the end and blocks the
  // wave skips load through an empty buffer: zeros, no memory traffic) -- so
  // one wait count serves every step and wave, and the compiler's own count
  // of the loads in flight stays exact enough not to add waits of its own.
  constexpr int per_step = KPER + 2 * KB;
  auto load_k = [&] __device__ (int i, char* kd) {
    const int kb = kb0 + KB * i;
    const rsrc_t ks = make_rsrc(k + base + (size_t)kb * 32 * D, i < nsteps ? (uint32_t)max(0, N - kb * 32) * D * 2u : 0u);
#pragma unroll
    for (int j = 0; j < KPER; ++j) load_lds16(ks, kd + (w + j * NW) * 1024, kpre[j]);
  };
  auto load_ds = [&] __device__ (int i, uint4 (&r)[KB][2]) {
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      const int kb = kb0 + KB * i + b;
      const bool mine = i < nsteps && visible(kb);
      const rsrc_t ss = make_rsrc(ds_slice + (mine ? (size_t)ds_block(lay, qb, kb) * 1024 : 0), mine ? 2048u : 0u);
      // Each block is read once: non-temporal, as the decode reads its cache.
      r[b][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ss, (uint32_t)lane * 16u, 0, 2));
      r[b][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ss, 1024u + (uint32_t)lane * 16u, 0, 2));
    }
  };

  f32x16 acc[CB];
#pragma unroll
  for (int c = 0; c < CB; ++c) acc[c] = f32x16{};
  // Transpose-read addresses: row 4 (g / 2) + gi / 4 (plus 16 s, plus 8 in
  // the read's second half, plus 32 per block) and bytes 64 c + 32 (g & 1) +
  // 8 (gi & 3) of the logical tile, as tr_addr gives for a padded one; in
  // the swizzled tile the 64-byte block c of that row sits at block c ^ x,
  // x the row's chunk XOR / 4 (the same for all rows a lane reads).
  const int g = lane >> 4, gi = lane & 15;
  const int trow = 4 * (g >> 1) + (gi >> 2);
  const int tx = TL::chunk_xor(trow) / 4;
  int trk[CB];
#pragma unroll
  for (int c = 0; c < CB; ++c) trk[c] = trow * RB + 64 * (c ^ tx) + 32 * (g & 1) + 8 * (gi & 3);
  // The dS tile in LDS: 32 rows (keys) of 64 bytes (32 slots), row-major,
  // with the 16-byte chunk c of row r at chunk c ^ ((r / 4) & 3).  The
  // stored block is in the dK / dV kernel's lane order: this lane's two
  // 16-byte pieces are chunks 2 h and 2 h + 1 of the row of key lane % 32
  // (h = lane / 32), and with the swizzle the sixteen lanes of each write
  // pass hit distinct banks (unswizzled, keys 64 bytes apart collide four
  // ways).  The transpose reads (row 16 s + 8 half + 4 (g / 2) + gi / 4,
  // bytes 32 (g & 1) + 8 (gi & 3), as tr_addr gives) follow the same swizzle,
  // which moves whole 16-byte chunks, so each lane's 8 bytes stay whole.
  const int dkey = lane & 31, dh = lane >> 5, dsw_x = (dkey >> 2) & 3;
  const int ds_lds0 = dkey * 64 + 16 * ((2 * dh) ^ dsw_x);
  const int ds_lds1 = dkey * 64 + 16 * ((2 * dh + 1) ^ dsw_x);
  int trs[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int r = 16 * s + 8 * half + 4 * (g >> 1) + (gi >> 2);
      const int c = 2 * (g & 1) + ((gi & 3) >> 1);
      trs[s][half] = r * 64 + 16 * (c ^ ((r >> 2) & 3)) + 8 * (gi & 1);
    }
  auto read_ds = [&] __device__ (int s) -> vec8<T> {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Sw + trs[s][0]));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Sw + trs[s][1]));
    const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
    return as_vec8<T>(uint4{l2.x, l2.y, h2.x, h2.y});
  };
  uint4 dsr[S][KB][2];

  auto stage_k = [&] __device__ (auto st) -> char* {
    constexpr int X = decltype(st)::value;
    return X == 0 ? T0 : X == 1 ? T1 : X == 2 ? T2 : T3;
  };
  using std::integral_constant;
  // Issue order as if steps -4 .. -1 had run: dS of step 0, then (K of step
  // j, dS of step j + 1) for j = 0 .. 2.
  load_ds(0, dsr[0]);
  auto prologue = [&] __device__ (auto jj) {
    constexpr int J = decltype(jj)::value;
    __builtin_amdgcn_sched_barrier(0);
    load_k(J, stage_k(integral_constant<int, J>{}));
    __builtin_amdgcn_sched_barrier(0);
    load_ds(J + 1, dsr[J + 1]);
  };
  prologue(integral_constant<int, 0>{});
  prologue(integral_constant<int, 1>{});
  prologue(integral_constant<int, 2>{});

  // Step i: after the K rows of step i were issued came the dS of step
  // i + 1 and the loads of steps i + 1 and i + 2, so waiting down to that
  // many leaves K of step i (and the older dS of step i) landed; the barrier
  // makes every wave's K loads visible and retires every read of step
  // i - 1's stage, into which the K rows of step i + 3 go next.  Then, per
  // block of the step, this wave's dS block moves from registers to its LDS
  // block (LDS runs a wave's accesses in order, so the second block's write
  // follows the first block's reads) and the products; the registers take
  // the dS of step i + 4.
  auto step = [&] __device__ (auto sl, int i) {
    constexpr int X = decltype(sl)::value;  // K stage and register slot of step i
    wait_vm_n<2 * KB + (S - 2) * per_step>();
    barrier_keep_loads();
    load_k(i + S - 1, stage_k(integral_constant<int, (X + S - 1) % S>{}));
    __builtin_amdgcn_sched_barrier(0);  // the wait count assumes K's loads go first
    bool vis[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b) vis[b] = i < nsteps && visible(kb0 + KB * i + b);
    const char* Kt = stage_k(integral_constant<int, X>{});
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      if (vis[b]) {
        *(uint4*)(Sw + ds_lds0) = dsr[X][b][0];
        *(uint4*)(Sw + ds_lds1) = dsr[X][b][1];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const vec8<T> bo = read_ds(s);
#pragma unroll
          for (int c = 0; c < CB; ++c)
            acc[c] = mfma32(read_tr8<RB, T>(Kt + trk[c] + (32 * b + 16 * s) * RB), bo, acc[c]);
        }
      }
    }
    load_ds(i + S, dsr[X]);
  };
  // Whole rounds of four steps (those past the end do no work): with no
  // exit inside the round each register slot stays in its registers from
  // round to round, where exits between the steps made the compiler copy
  // slots at the loop's back edge and wait for their loads there.
  for (int i = 0; i < nsteps; i += S) {
    step(integral_constant<int, 0>{}, i);
    step(integral_constant<int, 1>{}, i + 1);
    step(integral_constant<int, 2>{}, i + 2);
    step(integral_constant<int, 3>{}, i + 3);
  }
  // dQ straight from the accumulators: the lane holds 16 columns of the row
  // of its slot, four runs of four, each one 16-byte store (the two halves
  // of the wave fill 32 contiguous bytes of a row; the rows' four runs of a
  // 32-column block complete whole 128-byte lines in L2).  This is a small
  // part of the kernel's traffic (dQ once against every visible dS block).
  // The empty loads past the end must land before the wave ends.
  const int slot = lane & 31, hh = lane >> 5;
  const int row = wq0 + c_row(slot & 15, slot >> 4);
  if (row < N) {
    float* dst = dq + base + (size_t)row * D;
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *(float4*)(dst + 32 * c + 8 * g4 + 4 * hh) =
            float4{scale * acc[c][4 * g4], scale * acc[c][4 * g4 + 1], scale * acc[c][4 * g4 + 2],
                   scale * acc[c][4 * g4 + 3]};
  }
  __builtin_amdgcn_s_waitcnt(0);
}

template <typename T, int D>
hipError_t launch_t(const void* q, const void* k, const void* v, const void* o, const void* dO,
                    const float* lse, float* dq, float* dk, float* dv, int B, int H, int N,
                    float scale, Mask mask, void* ws, int dq_rows, hipStream_t stream) {
  const long long rows = (long long)B * H * N;
  float* Dv = (float*)ws;
  float* L2 = Dv + rows;
  if (dq_rows == kDqStored) {
    // D and L2, then dK / dV (storing dS), then dQ as the product dS K.
    constexpr int RPB = kPreThreads / (D / 8);
    hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(kPreThreads), 0,
                       stream, (const T*)o, (const T*)dO, lse, Dv, L2, rows);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const DsLayout lay = ds_layout(N, mask.causal, mask.window);
    T* dsw = (T*)((char*)ws + ds_offset(rows));
    const int nkt = (N + kBKV - 1) / kBKV;
    hipLaunchKernelGGL((bwd_kv4_kernel<T, D, true>), dim3((unsigned)((long long)nkt * B * H)), dim3(kKv4Threads),
                       0, stream, (const T*)q, (const T*)k, (const T*)v, (const T*)dO, Dv, L2, dk, dv, dsw, lay,
                       B * H, N, nkt, scale, scale * kLog2e, mask.causal, mask.window);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int nqt = (N + 127) / 128;
    hipLaunchKernelGGL((bwd_dq_ds_kernel<T, D>), dim3((unsigned)((long long)nqt * B * H)), dim3(kDsThreads), 0,
                       stream, (const T*)k, (const T*)dsw, lay, dq, B * H, N, nqt, scale, mask.causal, mask.window);
    return hipGetLastError();
  }
  // dQ first: it also stores D and L2 of every query row, which the dK / dV
  // kernel reads.  dQ: the ping-pong kernel (256 query rows per workgroup) or
  // the 4-wave kernel (128 rows).
  if (dq_rows == 256) {
    const int nqt = (N + 255) / 256;
    hipLaunchKernelGGL((bwd_dq_pp_kernel<T, D>), dim3((unsigned)((long long)nqt * B * H)), dim3(kDqPPThreads),
                       0, stream, (const T*)q, (const T*)k, (const T*)v, (const T*)dO, (const T*)o, lse,
                       Dv, L2, dq, B * H, N, nqt, scale, scale * kLog2e, mask.causal, mask.window);
  } else {
    constexpr int BQ = kDq4Threads / 2;  // 32 query rows per wave
    const int nqt = (N + BQ - 1) / BQ;
    hipLaunchKernelGGL((bwd_dq4_kernel<T, D, D == 64 ? 2 : 1>), dim3((unsigned)((long long)nqt * B * H)),
                       dim3(kDq4Threads), 0, stream, (const T*)q, (const T*)k, (const T*)v, (const T*)dO,
                       (const T*)o, lse, Dv, L2, dq, B * H, N, nqt, scale, scale * kLog2e, mask.causal,
                       mask.window);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int nkt = (N + kBKV - 1) / kBKV;
  const long long grid = (long long)nkt * B * H;
  hipLaunchKernelGGL((bwd_kv4_kernel<T, D, false>), dim3((unsigned)grid), dim3(kKv4Threads), 0, stream,
                     (const T*)q, (const T*)k, (const T*)v, (const T*)dO, Dv, L2, dk, dv, (T*)nullptr, DsLayout{},
                     B * H, N, nkt, scale, scale * kLog2e, mask.causal, mask.window);
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

size_t bwd_workspace_bytes_ds(int B, int H, int N, int d, Mask mask) {
  (void)d;
  const long long rows = (long long)B * H * N;
  const DsLayout lay = ds_layout(N, mask.causal, mask.window);
  return ds_offset(rows) + (size_t)B * H * (size_t)lay.per_head * 2048u;
}

hipError_t launch_bwd_mfma(const void* q, const void* k, const void* v, const void* o,
                           const void* dO, const float* lse, float* dq, float* dk, float* dv,
                           int B, int H, int N, int d, float scale, Mask mask, void* ws, bool f16,
                           int dq_rows, hipStream_t stream) {
  if (dq_rows != 128 && dq_rows != 256 && dq_rows != kDqStored) dq_rows = bwd_auto_dq_rows(B, H, N);
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
