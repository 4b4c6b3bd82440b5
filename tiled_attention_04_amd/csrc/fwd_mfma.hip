// 16-bit (bf16 or fp16) forward on gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16 / _f16, fp32 accumulation).  Every kernel is
// written once for the element type T; the two types share tiles, LDS
// layouts and transpose reads and differ only in the MFMA opcode and the
// conversions.
//
// Method: "Building Flash Attention from Scratch in Pure NumPy", Architecture
// Overview and Steps 2-3 -- per query tile, walk the key/value tiles, keep the
// running row max m and sum l, rescale O by exp(m_old - m_new), add P V, and
// divide by l once at the end; the masks and the skipping of hidden tiles
// follow "Build a FlashAttention-2 Inference Kernel from Scratch in Pure
// Python", Steps 2-3 (causal, sliding window, masked entries set to -inf).
//
// Mapping onto CDNA4:
//  * A workgroup of NW waves owns BQ = 32*NW query rows; each wave owns 32.
//    Key/value tiles are BK = 64 rows (32, or at d = 64 also 128, on
//    request for the 1-4 wave kernels; the 8-wave ping-pong kernel's three
//    LDS stages leave room for 64 only).  They go from HBM straight into LDS
//    (buffer_load ... lds, 16 bytes per lane): no register staging and no
//    ALU work to place them.  K and V are double-buffered.
//  * Scores are computed transposed, S^T = K Q^T: K (from LDS) is the A
//    operand and the wave's Q rows, loaded once into registers, are the B
//    operand.  In the 32x32 accumulator layout every lane then holds one
//    query column (lane % 32) and 16 of its keys, so the row max needs a
//    single swap between the two 32-lane halves, the row sum is kept per lane
//    and combined once at the end, and the rescale of O is one scalar per lane.
//  * P (rounded to T) is already in the B-operand layout of O^T = V^T P^T.
//    The A operand V^T is read from the row-major V tile with the LDS
//    transpose read ds_read_b64_tr_b16, whose 16-lane groups deliver 4
//    consecutive keys of one column per lane; the two reads per MFMA step
//    pick the keys in the accumulator's row order.
//  * Software pipeline: while the VALU runs the softmax of tile j, the
//    matrix cores already compute the scores of tile j+1 (K runs one tile
//    ahead of V), and the loads of K_{j+2} and V_{j+1} are in flight.
//  * LDS rows are padded (K by 16 bytes, V by 64) so that the MFMA operand
//    reads hit distinct banks with affine (immediate-offset) addressing; the
//    direct loads skip the padding by giving those lanes an out-of-range
//    offset.
//  * The exponentials use exp2 with scale*log2(e) folded into one FMA; the
//    running max is taken on raw scores (a negative scale negates Q's bits
//    instead); the row sum is accumulated in fp32 (a sum of the T-rounded
//    P would cost L up to 2^-9 on rows with few keys).  L is converted back
//    to natural log.
//  * Workgroups are ordered so that all query tiles of one (batch, head) land
//    on the same XCD (the dispatcher deals workgroup ids round-robin over the
//    8 XCDs), heaviest causal tiles first, so K/V tiles are reused from that
//    XCD's L2.
#include "fa_common.h"
#include "fa_launch.h"

#include <type_traits>

namespace fa {
namespace {

constexpr int kBK = 64;

// LDS layout of one K and one V tile of BK key rows (BK = 32, 64 or 128),
// each rounded up to whole 1 KB direct-load blocks (a block's bytes past the
// tile's rows land in that padding and are never read).
template <int D, int BK = kBK>
struct Tile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kKPitch = kRowBytes + 16;  // bytes per K row in LDS
  static constexpr int kVPitch = kRowBytes + 64;  // bytes per V row in LDS
  static constexpr int kKBytes = (BK * kKPitch + 1023) / 1024 * 1024;
  static constexpr int kVBytes = (BK * kVPitch + 1023) / 1024 * 1024;
  static constexpr int kKBlocks = kKBytes / 1024;  // 1 KB per wave-wide direct load
  static constexpr int kVBlocks = kVBytes / 1024;
  static constexpr int kSmem = 2 * (kKBytes + kVBytes);
  static constexpr int kNB = BK / 32;  // 32-key blocks per tile
  static_assert(BK == 32 || BK == 64 || BK == 128, "key tiles of 32, 64 or 128 rows");
  // O staging: one wave's 32 rows of 2 D + 16 bytes fit each of the four
  // buffers, two waves' fit a K tile from 64 keys up.
  static_assert(32 * (2 * D + 16) <= kKBytes && 32 * (2 * D + 16) <= kVBytes, "O staging");
  static_assert(BK < 64 || (2 * 32 * (2 * D + 16) <= kKBytes && 2 * 32 * (2 * D + 16) <= kVBytes),
                "O staging");
};

// Issue this wave's share of the direct loads of one tile (rows k0.. of a
// [N][D] 16-bit matrix) into an LDS tile with `PITCH`-byte rows.
template <int D, int NW, int NBLK, int PITCH, bool PRE, int NPRE, typename T>
__device__ __forceinline__ void load_tile(const T* __restrict__ g, int k0, int N, char* lds_tile,
                                          const uint32_t (&pre)[NPRE], int w, int lane) {
  const rsrc_t src = make_rsrc(g + (size_t)k0 * D, (uint32_t)max(0, N - k0) * D * 2u);
#pragma unroll
  for (int i = 0; i < (NBLK + NW - 1) / NW; ++i) {
    const int blk = w + i * NW;
    if (NBLK % NW == 0 || blk < NBLK) {
      uint32_t off;
      if constexpr (PRE) off = pre[i];
      else off = block_src<D>(blk, lane, PITCH);
      load_lds16(src, lds_tile + blk * 1024, off);
    }
  }
}

// Reference shift of the exponentials, in log2 units (see softmax_tile).
constexpr float kTau = 8.f;

// Hide the scores of keys outside [lo, hi] (tile-relative) by setting them
// to -inf ("Build a FlashAttention-2 Inference Kernel from Scratch in Pure
// Python", Step 2).  Only tiles that straddle a mask boundary or the end of
// the sequence need this.
template <int NB>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[NB], int lo, int hi, int h) {
#pragma unroll
  for (int kb2 = 0; kb2 < NB; ++kb2) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rel = kb2 * 32 + c_row(r, h);
      s[kb2][r] = ((rel >= lo) & (rel <= hi)) ? s[kb2][r] : kNegInf;
    }
  }
}

// Bounds of a lane's partial sum (its 32 keys of the tile) for which the
// exponentials taken against the current reference are kept: above the cap
// some P could exceed 2^14; below the floor (with nothing accumulated yet)
// everything may have underflowed.
constexpr float kSumCap = 16384.f;
constexpr float kSumFloor = 0x1p-60f;
// fp16 keeps P in 5 exponent bits: below 2^-14 it is subnormal (absolute
// spacing 2^-24) and below 2^-25 it rounds to zero.  A reference far above
// the row's scores (the initial 0 against scores all near -20, say) would
// pass the floor above with every P subnormal or zero while l, summed in
// fp32, stays right: O would collapse towards 0.  For fp16 the fast path is
// therefore kept only while each lane's running sum against the reference
// (earlier tiles included) is at least 1/2, so the row's sum l is at least
// 1 and each P's rounding error, at most 2^-25 absolute, is at most 2^-25
// of l.  (A lane whose half of the row sums below 1/2 while the row as a
// whole is fine takes the exact path for nothing: a rare cost, and cheaper
// than a cross-lane sum on every tile, which pushed the 8-wave kernel's
// registers over its budget.)
constexpr float kLaneSumFloorF16 = 0.5f;

// One tile of the online softmax for this lane's query row ("Building Flash
// Attention from Scratch in Pure NumPy", Step 2): raw scores s (16 keys per
// 32-key block, in the accumulator's row order) -> P in T in pk, with the
// running reference m_ref (log2 units) and sum l_run updated and O rescaled
// by 2^(m_old - m_new) when the reference moves.
//
// The reference is lazy: P = 2^(x - ref) is first computed against the
// current reference (0 for a row that has none yet), and kept when every
// lane's partial sum lies in [kSumFloor, kSumCap] (for fp16: at most kSumCap,
// and the lane's running sum at least kLaneSumFloorF16) -- then no P exceeds
// 2^14 and none that matters has underflowed or lost precision, and the
// tile costs no max and no rescale.  Otherwise (a row's first scores, a jump of the running max, or
// keys all hidden so far) the wave takes the exact path: tile max, raise the
// reference when the max exceeds it by more than kTau, rescale l and O, and
// recompute P.  Rows that passed the test keep their reference and P.  O / l
// and L = ref + log2(l) do not depend on the reference.
// c = |scale| * log2(e), at least 1e-30 so that a hidden score (-inf) always
// gives exp2(-inf * c - ref) = 0 exactly.
//
// kBatched picks the instruction order of the exponentials: all 32 scaled
// scores, then all 32 exponentials, then four partial sums (independent
// instructions back to back), or one score, its exponential and a running
// sum at a time.  The batched order measured 2-4% faster in the kernels that
// run two workgroups per CU and 1-4% slower in the ping-pong kernel, whose
// softmax shares each SIMD with the other group's matrix work.
template <typename T, int CB, bool kBatched, int NB = 2>
__device__ __forceinline__ void softmax_tile(const f32x16 (&s)[NB], uint32_t (&pk)[NB][8],
                                             f32x16 (&oacc)[CB], float& m_ref, float& l_run,
                                             float c) {
  auto exps = [&](float ref) {
    if constexpr (kBatched) {
      constexpr int E = 16 * NB;  // scores per lane
      float x[E];
#pragma unroll
      for (int i = 0; i < E; ++i) x[i] = __builtin_fmaf(s[i >> 4][i & 15], c, -ref);
#pragma unroll
      for (int i = 0; i < E; ++i) x[i] = __builtin_amdgcn_exp2f(x[i]);
      float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < E; ++i) part[i & 3] += x[i];
#pragma unroll
      for (int i = 0; i < E / 2; ++i) pk[i >> 3][i & 7] = pack2<T>(x[2 * i], x[2 * i + 1]);
      return (part[0] + part[1]) + (part[2] + part[3]);
    } else {
      float sum = 0.f;
#pragma unroll
      for (int kb2 = 0; kb2 < NB; ++kb2) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb2][r], c, -ref));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb2][r + 1], c, -ref));
          pk[kb2][r >> 1] = pack2<T>(p0, p1);
          sum += p0 + p1;
        }
      }
      return sum;
    }
  };
  if (m_ref == kNegInf) m_ref = 0.f;
  const float fast = exps(m_ref);
  bool keep;
  if constexpr (std::is_same<T, f16>::value)
    keep = fast <= kSumCap && l_run + fast >= kLaneSumFloorF16;
  else
    keep = fast <= kSumCap && l_run + fast >= kSumFloor;
  if (__builtin_amdgcn_ballot_w64(!keep) == 0) {
    l_run += fast;
    return;
  }
  float mx = kNegInf;
#pragma unroll
  for (int kb2 = 0; kb2 < NB; ++kb2) {
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb2][r]);
  }
  mx = pair_max(mx);
  const float m_tile = mx == kNegInf ? kNegInf : mx * c;
  // Only rows that failed the test move (both lanes of a row agree), so a
  // row's result never depends on the other rows of the wave.  With nothing
  // accumulated in the row yet, any finite reference will do: take the max.
  const bool row_failed = pair_sum(keep ? 0.f : 1.f) != 0.f;
  const bool up = row_failed &&
                  (m_tile > m_ref + kTau || (pair_sum(l_run) == 0.f && m_tile != kNegInf));
  if (__builtin_amdgcn_ballot_w64(up) != 0) {
    const float alpha = up ? __builtin_amdgcn_exp2f(m_ref - m_tile) : 1.f;
    m_ref = up ? m_tile : m_ref;
    l_run *= alpha;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) oacc[cb] *= alpha;
  }
  l_run += exps(m_ref);
}

// Store this wave's 32 x D block of O (rows r0 .. r0 + 31 of the slice at
// o_slice; rows at or past N dropped), normalised by inv, through `stage`,
// a region of 32 * (2 D + 16) bytes of LDS that only this wave uses.  The
// accumulator layout gives each lane 8-byte pieces of 32 different rows, so
// storing from it directly splits every store instruction into 32 partial
// cache lines; written to LDS in that layout and read back row by row, each
// store instruction writes whole 2D-byte rows instead.  (Rows padded by 16
// bytes: 16-byte aligned reads, at most 2-way conflicts on the writes.)
template <typename T, int D, int CB>
__device__ __forceinline__ void store_o_rows(const f32x16 (&oacc)[CB], float inv, char* stage,
                                             T* __restrict__ o_slice, int r0, int N, int lane) {
  constexpr int P = 2 * D + 16;
  constexpr int CPR = D / 8;      // 16-byte chunks per row
  constexpr int RPP = 64 / CPR;   // rows per wave-wide read
  const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      uint2 st;
      st.x = pack2<T>(oacc[cb][4 * gq + 0] * inv, oacc[cb][4 * gq + 1] * inv);
      st.y = pack2<T>(oacc[cb][4 * gq + 2] * inv, oacc[cb][4 * gq + 3] * inv);
      *(uint2*)(stage + l32 * P + (cb * 32 + 8 * gq + 4 * h) * 2) = st;
    }
  }
#pragma unroll
  for (int i = 0; i < 32 / RPP; ++i) {
    const int row = i * RPP + lane / CPR, ch = lane % CPR;
    const uint4 u = *(const uint4*)(stage + row * P + ch * 16);
    if (r0 + row < N) *(uint4*)((char*)(o_slice + (size_t)(r0 + row) * D) + ch * 16) = u;
  }
}

// Scheduling groups (masks of __builtin_amdgcn_sched_group_barrier).
constexpr int kSchedVALU = 0x002, kSchedMFMA = 0x008, kSchedDSRead = 0x100;

// Interleave NS score MFMAs (one 16-byte K read each) with the softmax VALU
// work, then NP PV MFMAs (two transpose reads each), keeping the LDS reads a
// few MFMAs ahead of their use.
template <int NS, int NP>
__device__ __forceinline__ void schedule_pipeline() {
  constexpr int kAheadS = 4, kAheadP = 4, kValuPerMfma = 7;
  __builtin_amdgcn_sched_group_barrier(kSchedDSRead, kAheadS, 0);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
    if (i + kAheadS < NS) __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedVALU, kValuPerMfma, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2 * kAheadP, 0);
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
    if (i + kAheadP < NP) __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2, 0);
  }
}

template <typename T, int D, int NW, int BK>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW == 4 && BK < 128 ? 2 : 1)))
void fwd_mfma_kernel(const T* __restrict__ q, const T* __restrict__ k,
                     const T* __restrict__ v, T* __restrict__ o, float* __restrict__ lse,
                     int BH, int N, int nqt, float c_log2, int negate_q, int causal, int window) {
  using TL = Tile<D, BK>;
  constexpr int NB = TL::kNB;  // 32-key blocks per key tile
  constexpr int NT = 64 * NW;  // threads
  constexpr int BQ = 32 * NW;
  constexpr int KS = D / 16;  // MFMA steps over the head dimension
  constexpr int CB = D / 32;  // 32-column blocks of O
  constexpr bool PRE = NW == 4;  // keep the per-lane direct-load offsets in registers
  constexpr int KPER = PRE ? (TL::kKBlocks + NW - 1) / NW : 1;
  constexpr int VPER = PRE ? (TL::kVBlocks + NW - 1) / NW : 1;
  // Separate LDS objects per buffer: the compiler can then tell that the
  // buffers being read do not alias the ones the direct loads are filling,
  // and does not wait for those loads before every LDS read.
  __shared__ __attribute__((aligned(1024))) char Kb0[TL::kKBytes];
  __shared__ __attribute__((aligned(1024))) char Kb1[TL::kKBytes];
  __shared__ __attribute__((aligned(1024))) char Vb0[TL::kVBytes];
  __shared__ __attribute__((aligned(1024))) char Vb1[TL::kVBytes];

  const int t = threadIdx.x;
  const int lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // uniform: keeps per-wave branches scalar

  // Workgroup -> (batch*head, query tile).
  int bh, qr;
  const int id = blockIdx.x;
  tile_order(id, BH, nqt, causal && window < 0, bh, qr);
  const int qt = causal ? nqt - 1 - qr : qr;
  const int q0 = qt * BQ;
  const size_t base = (size_t)bh * (size_t)N * D;
  const T* kg = k + base;
  const T* vg = v + base;
  const int qi = q0 + 32 * w + l32;  // this lane's query row

  // Rows the direct loads may leave unwritten (past N) must hold finite values.
  for (int i = t; i < TL::kKBytes / 16; i += NT) {
    ((uint4*)Kb0)[i] = uint4{0u, 0u, 0u, 0u};
    ((uint4*)Kb1)[i] = uint4{0u, 0u, 0u, 0u};
  }
  for (int i = t; i < TL::kVBytes / 16; i += NT) {
    ((uint4*)Vb0)[i] = uint4{0u, 0u, 0u, 0u};
    ((uint4*)Vb1)[i] = uint4{0u, 0u, 0u, 0u};
  }

  uint32_t kpre[KPER], vpre[VPER];
  if constexpr (PRE) {
#pragma unroll
    for (int i = 0; i < KPER; ++i) kpre[i] = block_src<D>(w + i * NW, lane, TL::kKPitch);
#pragma unroll
    for (int i = 0; i < VPER; ++i) vpre[i] = block_src<D>(w + i * NW, lane, TL::kVPitch);
  }

  // Q rows of this wave as MFMA B fragments: Q[qi][16 s + 8 h + 0..7]
  // (rows >= N read as zero).  The loads are issued here together with the
  // first K/V tiles; the sign flip for a negative scale (S * scale =
  // (-S) * |scale|, exact in bf16 and fp16) is applied once they have landed,
  // without a branch: a branch on each loaded value made every load wait
  // for the one before it.
  const rsrc_t q_src = make_rsrc(q + base, (uint32_t)N * D * 2u);
  const uint32_t q_neg = negate_q ? 0x80008000u : 0u;
  uint4 q_raw[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) q_raw[s] = load16(q_src, (uint32_t)(qi * D + 16 * s + 8 * h) * 2u);
  vec8<T> qf[KS];

  // Key tiles holding at least one visible key for this query tile.
  const int q_hi = q0 + BQ - 1;
  const int kmin = window >= 0 ? max(0, q0 - window) : 0;
  const int kmax = causal ? min(N - 1, q_hi) : N - 1;
  const int kt0 = kmin / BK, kt1 = kmax / BK + 1;
  // Keys this lane's query row may see (the tail of the sequence included).
  const int key_lo = window >= 0 ? qi - window : 0;
  const int key_hi = causal ? min(qi, N - 1) : N - 1;

  // Per-lane LDS byte offsets of the MFMA operand reads.
  //  K (A of S^T): row l32 (+32 per key block), bytes 32 s + 16 h.
  const int k_rd = l32 * TL::kKPitch + 16 * h;
  //  V^T (A of O^T) via ds_read_b64_tr_b16: in 16-lane group g, lane i points
  //  at key row 4 (g/2) + i/4 and columns 16 (g%2) + 4 (i%4) of the step's
  //  16 keys; the second read of a step adds 8 key rows.
  const int g = lane >> 4, gi = lane & 15;
  const int v_rd = (4 * (g >> 1) + (gi >> 2)) * TL::kVPitch + (16 * (g & 1) + 4 * (gi & 3)) * 2;

  f32x16 oacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) oacc[cb] = f32x16{};
  float m_ref = kNegInf, l_run = 0.f;  // log2 units

  __syncthreads();  // LDS zeroed before any direct load lands
  load_tile<D, NW, TL::kKBlocks, TL::kKPitch, PRE>(kg, kt0 * BK, N, Kb0, kpre, w, lane);
  load_tile<D, NW, TL::kVBlocks, TL::kVPitch, PRE>(vg, kt0 * BK, N, Vb0, vpre, w, lane);
  if (kt0 + 1 < kt1)
    load_tile<D, NW, TL::kKBlocks, TL::kKPitch, PRE>(kg, (kt0 + 1) * BK, N, Kb1, kpre, w, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qf[s] = as_vec8<T>(uint4{q_raw[s].x ^ q_neg, q_raw[s].y ^ q_neg, q_raw[s].z ^ q_neg, q_raw[s].w ^ q_neg});

  // S^T = K Q^T of the first tile for its 32-key blocks.
  f32x16 s_a[NB];
#pragma unroll
  for (int kb2 = 0; kb2 < NB; ++kb2) {
    s_a[kb2] = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const vec8<T> a = *(const vec8<T>*)(Kb0 + k_rd + kb2 * 32 * TL::kKPitch + 32 * s);
      s_a[kb2] = mfma32(a, qf[s], s_a[kb2]);
    }
  }
  __syncthreads();  // every wave is done with K buffer 0 before it is refilled

  // One pipeline step for tile kt, whose parity selects the buffers at
  // compile time: K_{kt+1} is in the "next" K buffer, V_kt in the "current"
  // V buffer; S_kt is in s_cur and S_{kt+1} is written to s_next.
  auto step = [&](auto parity, f32x16 (&s_cur)[NB], f32x16 (&s_next)[NB], int kt) {
    constexpr int P = decltype(parity)::value;
    char* const k_next = P ? Kb0 : Kb1;
    char* const k_refill = P ? Kb1 : Kb0;
    char* const v_cur = P ? Vb1 : Vb0;
    char* const v_next = P ? Vb0 : Vb1;
    const bool has_next = kt + 1 < kt1;
    if (has_next) load_tile<D, NW, TL::kVBlocks, TL::kVPitch, PRE>(vg, (kt + 1) * BK, N, v_next, vpre, w, lane);
    if (kt + 2 < kt1) load_tile<D, NW, TL::kKBlocks, TL::kKPitch, PRE>(kg, (kt + 2) * BK, N, k_refill, kpre, w, lane);

    const int k0 = kt * BK;
    const bool need_mask = (k0 + BK > N) || (causal && k0 + BK - 1 > q0) ||
                           (window >= 0 && k0 < q_hi - window);
    if (need_mask) mask_tile(s_cur, key_lo - k0, key_hi - k0, h);

    // Scores of the next tile on the matrix cores (on the last tile they are
    // computed from whatever the buffer holds and discarded) ...
#pragma unroll
    for (int kb2 = 0; kb2 < NB; ++kb2) {
      s_next[kb2] = mfma32(*(const vec8<T>*)(k_next + k_rd + kb2 * 32 * TL::kKPitch), qf[0], f32x16{});
#pragma unroll
      for (int s = 1; s < KS; ++s) {
        const vec8<T> a = *(const vec8<T>*)(k_next + k_rd + kb2 * 32 * TL::kKPitch + 32 * s);
        s_next[kb2] = mfma32(a, qf[s], s_next[kb2]);
      }
    }

    // ... while the vector ALUs run the softmax of this one.
    uint32_t pk[NB][8];
    // (Batched exponentials hold all of a lane's scores at once: with
    // 128-key tiles that is 64 more live registers than the kernel has room
    // for.)
    softmax_tile<T, CB, (NB <= 2), NB>(s_cur, pk, oacc, m_ref, l_run, c_log2);

    // O^T += V^T P^T, 16 keys per step.
    const char* vt = v_cur + v_rd;
#pragma unroll
    for (int s = 0; s < 2 * NB; ++s) {
      const uint4 pw = {pk[s >> 1][4 * (s & 1) + 0], pk[s >> 1][4 * (s & 1) + 1],
                        pk[s >> 1][4 * (s & 1) + 2], pk[s >> 1][4 * (s & 1) + 3]};
      const vec8<T> pb = as_vec8<T>(pw);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const char* p = vt + 16 * s * TL::kVPitch + 64 * cb;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 * TL::kVPitch));
        const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
        const vec8<T> a = as_vec8<T>(uint4{l2.x, l2.y, h2.x, h2.y});
        oacc[cb] = mfma32(a, pb, oacc[cb]);
      }
    }

    // Instruction order for the region above: K operand reads run a few
    // MFMAs ahead, and each score MFMA is followed by a slice of the softmax
    // so that the matrix cores and the vector ALUs work at the same time; the
    // V^T reads likewise run ahead of the PV MFMAs.
    schedule_pipeline<NB * KS, 2 * NB * CB>();
    __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads have landed
    __syncthreads();
  };

  f32x16 s_b[NB];
  for (int kt = kt0; kt < kt1; kt += 2) {  // two tiles per trip: s_a and s_b swap roles
    step(std::integral_constant<int, 0>{}, s_a, s_b, kt);
    if (kt + 1 < kt1) step(std::integral_constant<int, 1>{}, s_b, s_a, kt + 1);
  }

  // Epilogue: O = O / l, L = m ln2 + ln l.
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  // O through LDS (the loop's last barrier freed the buffers): two waves per
  // K buffer, or with 32-key tiles one wave per buffer.
  char* const stage = BK >= 64 ? (w < 2 ? Kb0 : Kb1) + (w & 1) * 32 * (2 * D + 16)
                               : (w == 0 ? Kb0 : w == 1 ? Kb1 : w == 2 ? Vb0 : Vb1);
  store_o_rows<T, D, CB>(oacc, inv, stage, o + base, q0 + 32 * w, N, lane);
  if (qi < N && h == 0 && lse != nullptr)
    lse[(size_t)bh * N + qi] = l_tot > 0.f ? m_ref * kLn2 + logf(l_tot) : kNegInf;
}

// ---------------------------------------------------------------------------
// Ping-pong forward for long sequences: 8 waves, 256 query rows per workgroup.
//
// The waves form two groups of four that run the same tile loop half a step
// apart, separated by workgroup barriers: while one group issues its matrix
// work for tile j (P_j V_j and the scores of tile j+1), the other runs the
// softmax of its own tile j on the vector ALUs, then they swap.  Each SIMD
// hosts one wave of each group, so its matrix core and vector ALU are busy at
// the same time.  A wave keeps a single score buffer: the scores of tile j+1
// are written after the softmax of tile j has consumed them.  K/V tiles sit in
// three LDS stages (one workgroup per CU); tile j+2 is loaded while tiles j and
// j+1 are in use, and every wave loads its share of each tile.
//
// Barrier bookkeeping: group 0 runs  [softmax j] B [matrix j] B ...  and group
// 1 runs one barrier behind, so between consecutive barriers one group is in
// its matrix phase and the other in its softmax phase.  Every wave executes
// the same number of barriers, whichever group it is in.

// Scheduling of the matrix phase: NPV PV MFMAs with two transpose reads each,
// then NS score MFMAs with one K read each; operand reads run AHEAD MFMAs
// ahead.
template <int NPV, int NS>
__device__ __forceinline__ void schedule_matrix_phase() {
  constexpr int AHEAD = 4;
  __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2 * AHEAD, 1);
#pragma unroll
  for (int i = 0; i < NPV; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 1);
    if (i + AHEAD < NPV) __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2, 1);
    else __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 1);
  }
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 1);
    if (i + AHEAD < NS) __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 1);
  }
}

// Force values to be computed at this point of the program: an empty asm
// that reads and "writes" them keeps compiler passes from sinking their
// arithmetic past the barrier that follows (they would otherwise move next
// to their only users, the MFMAs of the other phase).
// (The asm only exists in the device pass: the host pass also parses device
// functions, and AMDGPU register constraints mean nothing there.)
template <int CB>
__device__ __forceinline__ void pin_softmax_results(uint32_t (&pk)[2][8], f32x16 (&oacc)[CB],
                                                    float& l_run, float& m_ref) {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(pk[i][j]));
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) asm volatile("" : "+v"(oacc[cb]));
  asm volatile("" : "+v"(l_run), "+v"(m_ref));
#else
  (void)pk; (void)oacc; (void)l_run; (void)m_ref;
#endif
}

// LDS stages of the ping-pong kernel (K and V each; 3 or 4).  Three keep the
// direct loads two tiles ahead, which hides their latency (111 KB of LDS for
// d = 128); four measured no faster.
#ifndef FA_PINGPONG_STAGES
#define FA_PINGPONG_STAGES 3
#endif
constexpr int kPingPongStages = FA_PINGPONG_STAGES;


template <typename T, int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_pingpong_kernel(const T* __restrict__ q, const T* __restrict__ k,
                         const T* __restrict__ v, T* __restrict__ o, float* __restrict__ lse,
                         int BH, int N, int nqt, float c_log2, int negate_q, int causal, int window) {
  using TL = Tile<D>;
  constexpr int NW = 8;
  constexpr int BQ = 32 * NW;
  constexpr int KS = D / 16;
  constexpr int CB = D / 32;
  constexpr int KPER = (TL::kKBlocks + NW - 1) / NW;
  constexpr int VPER = (TL::kVBlocks + NW - 1) / NW;
  constexpr int NS = kPingPongStages;  // LDS stages; loads run NS-1 tiles ahead
  static_assert(NS == 3 || NS == 4, "3 or 4 stages");
  // One LDS object per stage and matrix (see the alias note in fwd_mfma_kernel).
  __shared__ __attribute__((aligned(1024))) char K0[TL::kKBytes];
  __shared__ __attribute__((aligned(1024))) char K1[TL::kKBytes];
  __shared__ __attribute__((aligned(1024))) char K2[TL::kKBytes];
  __shared__ __attribute__((aligned(1024))) char K3[NS > 3 ? TL::kKBytes : 1];
  __shared__ __attribute__((aligned(1024))) char V0[TL::kVBytes];
  __shared__ __attribute__((aligned(1024))) char V1[TL::kVBytes];
  __shared__ __attribute__((aligned(1024))) char V2[TL::kVBytes];
  __shared__ __attribute__((aligned(1024))) char V3[NS > 3 ? TL::kVBytes : 1];
  __shared__ int simd_slots[4];

  const int t = threadIdx.x;
  const int lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // uniform: keeps per-wave branches scalar

  int bh, qr;
  const int id = blockIdx.x;
  tile_order(id, BH, nqt, causal && window < 0, bh, qr);
  const int qt = causal ? nqt - 1 - qr : qr;
  const int q0 = qt * BQ;
  const size_t base = (size_t)bh * (size_t)N * D;
  const T* kg = k + base;
  const T* vg = v + base;
  const int qi = q0 + 32 * w + l32;

  // (The stages need no clearing: a stage is read only after its tile has
  // landed, except for the scores of a tile past the end, which are dropped.)
  if (t < 4) simd_slots[t] = 0;
  __syncthreads();
  // Group = order of arrival of this wave on its SIMD (HW_ID bits 5:4), so
  // that each SIMD hosts one wave of each group when waves are spread evenly.
  const int grp = wave_group(simd_slots, lane);

  uint32_t kpre[KPER], vpre[VPER];
#pragma unroll
  for (int i = 0; i < KPER; ++i) kpre[i] = block_src<D>(w + i * NW, lane, TL::kKPitch);
#pragma unroll
  for (int i = 0; i < VPER; ++i) vpre[i] = block_src<D>(w + i * NW, lane, TL::kVPitch);
  const int k_nblk = (TL::kKBlocks - w + NW - 1) / NW;  // K / V blocks this wave loads per tile
  const int v_nblk = (TL::kVBlocks - w + NW - 1) / NW;
  constexpr int kVMin = TL::kVBlocks / NW;  // fewest V blocks of any wave
  static_assert(kVMin >= 1, "every wave loads a V block");

  // Q rows (sign-flipped after the prologue's wait, as in fwd_mfma_kernel).
  const rsrc_t q_src = make_rsrc(q + base, (uint32_t)N * D * 2u);
  const uint32_t q_neg = negate_q ? 0x80008000u : 0u;
  uint4 q_raw[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) q_raw[s] = load16(q_src, (uint32_t)(qi * D + 16 * s + 8 * h) * 2u);
  vec8<T> qf[KS];

  const int q_hi = q0 + BQ - 1;
  const int kmin = window >= 0 ? max(0, q0 - window) : 0;
  const int kmax = causal ? min(N - 1, q_hi) : N - 1;
  const int kt0 = kmin / kBK, kt1 = kmax / kBK + 1;
  const int key_lo = window >= 0 ? qi - window : 0;
  const int key_hi = causal ? min(qi, N - 1) : N - 1;
  const int wq0 = q0 + 32 * w, wq1 = wq0 + 31;
  // Keys visible to at least one row of this wave: tiles outside this range
  // (past a causal diagonal, before a window) are skipped by the wave, which
  // still takes part in the loads and barriers.
  const int wk_lo = window >= 0 ? max(0, wq0 - window) : 0;
  const int wk_hi = wq0 < N ? (causal ? min(N - 1, wq1) : N - 1) : -1;
  auto active = [&] __device__ (int tile) {
    const int k0 = tile * kBK;
    return k0 <= wk_hi && k0 + kBK - 1 >= wk_lo;
  };

  const int k_rd = l32 * TL::kKPitch + 16 * h;
  const int g = lane >> 4, gi = lane & 15;
  const int v_rd = (4 * (g >> 1) + (gi >> 2)) * TL::kVPitch + (16 * (g & 1) + 4 * (gi & 3)) * 2;

  auto kstage = [&] __device__ (auto st) -> char* {
    constexpr int S = decltype(st)::value;
    return S == 0 ? K0 : S == 1 ? K1 : S == 2 ? K2 : K3;
  };
  auto vstage = [&] __device__ (auto st) -> char* {
    constexpr int S = decltype(st)::value;
    return S == 0 ? V0 : S == 1 ? V1 : S == 2 ? V2 : V3;
  };
  // This wave's share of the direct loads of tile `tile` into stage st (K
  // blocks first, then V, so that a wait for K can leave V in flight).
  auto load_share = [&] __device__ (int tile, auto st) {
    const int k0 = tile * kBK;
    const rsrc_t ks = make_rsrc(kg + (size_t)k0 * D, (uint32_t)max(0, N - k0) * D * 2u);
    const rsrc_t vs = make_rsrc(vg + (size_t)k0 * D, (uint32_t)max(0, N - k0) * D * 2u);
    char* kd = kstage(st);
    char* vd = vstage(st);
#pragma unroll
    for (int i = 0; i < KPER; ++i) {
      const int blk = w + i * NW;
      if (blk < TL::kKBlocks)
        load_lds16(ks, kd + blk * 1024, kpre[i]);
    }
#pragma unroll
    for (int i = 0; i < VPER; ++i) {
      const int blk = w + i * NW;
      if (blk < TL::kVBlocks)
        load_lds16(vs, vd + blk * 1024, vpre[i]);
    }
  };

  f32x16 oacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) oacc[cb] = f32x16{};
  float m_ref = kNegInf, l_run = 0.f;
  f32x16 sc[2];  // scores of the tile in flight

  using std::integral_constant;
  // Loads of tile t by this wave (0 past the end).
  auto n_loads = [&] __device__ (int tile) { return tile < kt1 ? k_nblk + v_nblk : 0; };
  // Prologue: tiles kt0 .. kt0+NS-2 in flight, then the scores of tile kt0
  // as soon as Q and its K have landed.
  load_share(kt0, integral_constant<int, 0>{});
  if (kt0 + 1 < kt1) load_share(kt0 + 1, integral_constant<int, 1>{});
  if constexpr (NS > 3) {
    if (kt0 + 2 < kt1) load_share(kt0 + 2, integral_constant<int, 2>{});
    wait_vm(n_loads(kt0 + 2));
  } else {
    // Q and K of the first tile; its V and the second tile may still land.
    wait_vm(v_nblk + (kt0 + 1 < kt1 ? k_nblk + v_nblk : 0));
  }
  barrier_keep_loads();
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qf[s] = as_vec8<T>(uint4{q_raw[s].x ^ q_neg, q_raw[s].y ^ q_neg, q_raw[s].z ^ q_neg, q_raw[s].w ^ q_neg});
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2) {
    sc[kb2] = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; ++s)
      sc[kb2] = mfma32(*(const vec8<T>*)(K0 + k_rd + kb2 * 32 * TL::kKPitch + 32 * s), qf[s], sc[kb2]);
  }
  if (grp == 1) {  // group 1 runs one phase behind
    // Its shares of V of the first tile and K of the second must have landed
    // before group 0's first matrix phase (the barrier below opens it).
    if constexpr (NS == 3) wait_vm(kt0 + 1 < kt1 ? v_nblk : 0);
    barrier_keep_loads();
  }

  // One tile: softmax phase, barrier, matrix phase, barrier.  Stage of tile
  // kt is ST (compile time); tile kt+1 is in stage (ST+1)%NS and tile
  // kt+NS-1 is loaded into stage (ST+NS-1)%NS, the one tile kt-1 used.
  auto tile_step = [&] __device__ (auto stage, int kt) {
    constexpr int ST = decltype(stage)::value;
    constexpr int STN = (ST + 1) % NS, STF = (ST + NS - 1) % NS;
    const int far = kt + NS - 1;
    const bool load_far = far < kt1;
    // ---- softmax phase (group 1 also issues its loads of tile kt+NS-1 here)
    if (grp == 1 && load_far) load_share(far, integral_constant<int, STF>{});
    const bool act = active(kt), act_next = kt + 1 < kt1 && active(kt + 1);
    uint32_t pk[2][8];
    if (act) {
      const int k0 = kt * kBK;
      const bool need_mask = (k0 + kBK > N) || (causal && k0 + kBK - 1 > wq0) ||
                             (window >= 0 && k0 < wq1 - window);
      if (need_mask) mask_tile(sc, key_lo - k0, key_hi - k0, h);
      softmax_tile<T, CB, false>(sc, pk, oacc, m_ref, l_run, c_log2);
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) pk[i][j] = 0u;  // (P V adds nothing)
    }
    pin_softmax_results<CB>(pk, oacc, l_run, m_ref);
    // Group 0: tile kt+1's K must be resident for its matrix phase; its V
    // and the tiles after it may stay in flight.  With three stages the
    // count is the fewest V blocks any wave loads: loads complete in order
    // and V_{kt+1} was issued last, so waiting until that many remain covers
    // K_{kt+1} in every wave (a wave with one V block more waits for a load
    // issued a whole tile ago), and past the last tile there is nothing to
    // wait for.  A constant keeps the wait a single instruction (a count
    // known only at run time costs a chain of compares and branches).
    if (grp == 0) {
      if constexpr (NS == 3)
        wait_vm(kVMin);
      else
        wait_vm(n_loads(kt + 2) + (kt + 1 < kt1 ? v_nblk : 0));
    }
    barrier_keep_loads();
    // ---- matrix phase (group 0 issues its loads of tile kt+NS-1 here)
    if (grp == 0 && load_far) load_share(far, integral_constant<int, STF>{});
    {
      const char* vt = vstage(integral_constant<int, ST>{}) + v_rd;
      const char* kn = kstage(integral_constant<int, STN>{}) + k_rd;
      // P V of this tile, then the scores of tile kt+1.
      auto pv = [&] __device__ () {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint4 pw = {pk[s >> 1][4 * (s & 1) + 0], pk[s >> 1][4 * (s & 1) + 1],
                            pk[s >> 1][4 * (s & 1) + 2], pk[s >> 1][4 * (s & 1) + 3]};
          const vec8<T> pb = as_vec8<T>(pw);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            const char* p = vt + 16 * s * TL::kVPitch + 64 * cb;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 * TL::kVPitch));
            const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
            oacc[cb] = mfma32(as_vec8<T>(uint4{l2.x, l2.y, h2.x, h2.y}), pb, oacc[cb]);
          }
        }
      };
      auto qk = [&] __device__ () {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          sc[kb2] = mfma32(*(const vec8<T>*)(kn + kb2 * 32 * TL::kKPitch), qf[0], f32x16{});
#pragma unroll
          for (int s = 1; s < KS; ++s)
            sc[kb2] = mfma32(*(const vec8<T>*)(kn + kb2 * 32 * TL::kKPitch + 32 * s), qf[s], sc[kb2]);
        }
      };
      if (act || act_next) {  // (a wave past all its keys does no matrix work)
        pv();
        qk();
        schedule_matrix_phase<4 * CB, 2 * KS>();
      }
    }
    // Group 1: its K of tile kt+2 must have landed before group 0 needs it in
    // the next matrix phase; V_{kt+2} and later tiles may stay in flight
    // (the same constant count as above).
    if (grp == 1) {
      if constexpr (NS == 3)
        wait_vm(kVMin);
      else
        wait_vm(n_loads(kt + 3) + (kt + 2 < kt1 ? v_nblk : 0));
    }
    barrier_keep_loads();
  };

  for (int kt = kt0; kt < kt1; kt += NS) {
    tile_step(integral_constant<int, 0>{}, kt);
    if (kt + 1 >= kt1) break;
    tile_step(integral_constant<int, 1>{}, kt + 1);
    if (kt + 2 >= kt1) break;
    tile_step(integral_constant<int, 2>{}, kt + 2);
    if constexpr (NS > 3) {
      if (kt + 3 >= kt1) break;
      tile_step(integral_constant<int, 3 % NS>{}, kt + 3);
    }
  }
  if (grp == 0) barrier_keep_loads();  // match group 1's extra barrier

  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  // O through LDS (after the last barrier no wave reads the stages): two
  // waves per K stage, the last two in V stage 0.
  store_o_rows<T, D, CB>(oacc, inv, (w < 2 ? K0 : w < 4 ? K1 : w < 6 ? K2 : V0) + (w & 1) * 32 * (2 * D + 16),
                         o + base, q0 + 32 * w, N, lane);
  if (qi < N && h == 0 && lse != nullptr)
    lse[(size_t)bh * N + qi] = l_tot > 0.f ? m_ref * kLn2 + logf(l_tot) : kNegInf;
}


template <typename T, int D, int NW, int BK>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                  int N, float scale, Mask mask, hipStream_t stream) {
  constexpr int BQ = 32 * NW;
  const int nqt = (N + BQ - 1) / BQ;
  const long long grid = (long long)nqt * B * H;
  hipLaunchKernelGGL((fwd_mfma_kernel<T, D, NW, BK>), dim3((unsigned)grid), dim3(64 * NW), 0, stream,
                     (const T*)q, (const T*)k, (const T*)v, (T*)o, lse, B * H, N, nqt,
                     fmaxf(fabsf(scale) * kLog2e, 1e-30f), scale < 0.f ? 1 : 0, mask.causal,
                     mask.window);
  return hipGetLastError();
}

// 128-key tiles for d = 64 only: at d = 128 two 128-key score tiles, O and Q
// take more registers than a wave has, and the spills would put scratch
// memory (and its allocation) on the path.
template <typename T, int D, int NW>
hipError_t launch_bk(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                     int N, float scale, Mask mask, int block_k, hipStream_t stream) {
  if (block_k == 32) return launch<T, D, NW, 32>(q, k, v, o, lse, B, H, N, scale, mask, stream);
  if constexpr (D == 64) {
    if (block_k == 128) return launch<T, D, NW, 128>(q, k, v, o, lse, B, H, N, scale, mask, stream);
  }
  return launch<T, D, NW, 64>(q, k, v, o, lse, B, H, N, scale, mask, stream);
}

template <typename T, int D>
hipError_t launch_pingpong(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                           int H, int N, float scale, Mask mask, hipStream_t stream) {
  const int nqt = (N + 255) / 256;
  const long long grid = (long long)nqt * B * H;
  hipLaunchKernelGGL((fwd_pingpong_kernel<T, D>), dim3((unsigned)grid), dim3(512), 0, stream,
                     (const T*)q, (const T*)k, (const T*)v, (T*)o, lse, B * H, N, nqt,
                     fmaxf(fabsf(scale) * kLog2e, 1e-30f), scale < 0.f ? 1 : 0, mask.causal,
                     mask.window);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                    int N, int d, float scale, Mask mask, int block_q, int block_k, hipStream_t stream) {
  if (d == 128) {
    if (block_q == 256) return launch_pingpong<T, 128>(q, k, v, o, lse, B, H, N, scale, mask, stream);
    if (block_q == 128) return launch_bk<T, 128, 4>(q, k, v, o, lse, B, H, N, scale, mask, block_k, stream);
    if (block_q == 64) return launch_bk<T, 128, 2>(q, k, v, o, lse, B, H, N, scale, mask, block_k, stream);
    return launch_bk<T, 128, 1>(q, k, v, o, lse, B, H, N, scale, mask, block_k, stream);
  }
  if (block_q == 256) return launch_pingpong<T, 64>(q, k, v, o, lse, B, H, N, scale, mask, stream);
  if (block_q == 128) return launch_bk<T, 64, 4>(q, k, v, o, lse, B, H, N, scale, mask, block_k, stream);
  if (block_q == 64) return launch_bk<T, 64, 2>(q, k, v, o, lse, B, H, N, scale, mask, block_k, stream);
  return launch_bk<T, 64, 1>(q, k, v, o, lse, B, H, N, scale, mask, block_k, stream);
}

}  // namespace

hipError_t launch_fwd_mfma(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, int d, float scale, Mask mask, int block_q,
                           int block_k, bool f16, hipStream_t stream) {
  if (f16) return dispatch<fa::f16>(q, k, v, o, lse, B, H, N, d, scale, mask, block_q, block_k, stream);
  return dispatch<bf16>(q, k, v, o, lse, B, H, N, d, scale, mask, block_q, block_k, stream);
}

}  // namespace fa
