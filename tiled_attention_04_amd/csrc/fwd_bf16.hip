// bf16 forward on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16, fp32
// accumulation).
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
//    Key/value tiles are BK = 64 rows, double-buffered in LDS and prefetched
//    from HBM into registers one tile ahead.
//  * Scores are computed transposed, S^T = K Q^T: K (from LDS) is the A
//    operand and the wave's Q rows, loaded once into registers, are the B
//    operand.  In the 32x32 accumulator layout every lane then holds one
//    query column (lane % 32) and 16 of its keys, so the row max needs a
//    single swap between the two 32-lane halves, the row sum is kept per lane
//    and combined once at the end, and the rescale of O is one scalar per lane.
//  * P (rounded to bf16) is already in the B-operand layout of O^T = V^T P^T,
//    so it goes from the softmax straight into the second MFMA.  To make the
//    A operand (V^T) a single 16-byte LDS read per step, V is written to LDS
//    transposed, with the keys of every 16-key group permuted (bits 2 and 3
//    of the key index swapped) to match the accumulator's row order.
//  * LDS rows are XOR-swizzled in 16-byte chunks so that the MFMA operand
//    reads are free of bank conflicts.
//  * The exponentials use exp2 with scale*log2(e) folded into one multiply;
//    L is converted back to natural log on output.
//  * Workgroups are ordered so that all query tiles of one (batch, head) land
//    on the same XCD (the dispatcher deals workgroup ids round-robin over the
//    8 XCDs), heaviest causal tiles first, so K/V tiles are reused from that
//    XCD's L2.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kBK = 64;

// Row-major [rows][D] tile: 16-byte chunk c of row r is stored at chunk
// c ^ (r & 7) (D >= 64 so every row has at least 8 chunks).
template <int D>
__device__ __forceinline__ int rm_off(int row, int chunk) {
  return row * D + ((chunk ^ (row & 7)) << 3);
}

// Transposed [D][kBK] tile: key u of the tile sits at position vt_pos(u) of
// row c; 16-byte chunks of a row are swizzled with (c + c/8) & 7.
__device__ __forceinline__ int vt_pos(int u) { return (u & ~12) | ((u & 4) << 1) | ((u & 8) >> 1); }
__device__ __forceinline__ int vt_off(int c, int pos) {
  return c * kBK + ((((pos >> 3) ^ ((c + (c >> 3)) & 7))) << 3) + (pos & 7);
}

template <int D, int T>
struct TileIO {
  static constexpr int kChunksPerRow = D / 8;
  static constexpr int kKChunks = kBK * kChunksPerRow;         // 16-byte chunks of K
  static constexpr int kKPer = (kKChunks + T - 1) / T;
  static constexpr int kVUnits = (kBK / 4) * kChunksPerRow;      // 4 rows x 16 bytes of V
  static constexpr int kVPer = (kVUnits + T - 1) / T;

  uint4 kr[kKPer];
  uint4 vr[kVPer][4];

  // Tile rows k0.. of K and V into registers; rows >= N read as zero.
  __device__ __forceinline__ void load(rsrc_t kr_src, rsrc_t vr_src, int k0, int t) {
#pragma unroll
    for (int j = 0; j < kKPer; ++j) {
      const int i = t + j * T;
      if (kKChunks % T == 0 || i < kKChunks) {
        const int row = k0 + i / kChunksPerRow;
        kr[j] = load16(kr_src, (uint32_t)(row * D + (i % kChunksPerRow) * 8) * 2u);
      }
    }
#pragma unroll
    for (int j = 0; j < kVPer; ++j) {
      const int i = t + j * T;
      if (kVUnits % T == 0 || i < kVUnits) {
        const int co = i % kChunksPerRow;
        const int row0 = k0 + 4 * (i / kChunksPerRow);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          vr[j][e] = load16(vr_src, (uint32_t)((row0 + e) * D + co * 8) * 2u);
      }
    }
  }

  __device__ __forceinline__ void store(bf16* __restrict__ Ks, bf16* __restrict__ Vt, int t) const {
#pragma unroll
    for (int j = 0; j < kKPer; ++j) {
      const int i = t + j * T;
      if (kKChunks % T == 0 || i < kKChunks)
        *(uint4*)(Ks + rm_off<D>(i / kChunksPerRow, i % kChunksPerRow)) = kr[j];
    }
#pragma unroll
    for (int j = 0; j < kVPer; ++j) {
      const int i = t + j * T;
      if (kVUnits % T == 0 || i < kVUnits) {
        const int co = i % kChunksPerRow;
        const int pos = vt_pos(4 * (i / kChunksPerRow));
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
          const uint32_t a0 = word(vr[j][0], cc >> 1), a1 = word(vr[j][1], cc >> 1);
          const uint32_t a2 = word(vr[j][2], cc >> 1), a3 = word(vr[j][3], cc >> 1);
          uint2 out;
          if (cc & 1) {
            out.x = (a0 >> 16) | (a1 & 0xffff0000u);
            out.y = (a2 >> 16) | (a3 & 0xffff0000u);
          } else {
            out.x = (a0 & 0xffffu) | (a1 << 16);
            out.y = (a2 & 0xffffu) | (a3 << 16);
          }
          *(uint2*)(Vt + vt_off(co * 8 + cc, pos)) = out;
        }
      }
    }
  }
};

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW == 4 ? 2 : 1)))
void fwd_bf16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                     const bf16* __restrict__ v, bf16* __restrict__ o, float* __restrict__ lse,
                     int BH, int N, int nqt, float scale_log2, int causal, int window) {
  constexpr int T = 64 * NW;
  constexpr int BQ = 32 * NW;
  constexpr int KS = D / 16;  // MFMA steps over the head dimension
  constexpr int CB = D / 32;  // 32-column blocks of O
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][kBK * D];
  __shared__ __attribute__((aligned(16))) bf16 Vt[2][D * kBK];

  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6, h = lane >> 5, l32 = lane & 31;

  // Workgroup -> (batch*head, query tile).
  int bh, qr;
  const int id = blockIdx.x;
  if ((BH & 7) == 0) {
    const int xcd = id & 7, slot = id >> 3;
    bh = (slot / nqt) * 8 + xcd;
    qr = slot % nqt;
  } else {
    bh = id / nqt;
    qr = id % nqt;
  }
  const int qt = causal ? nqt - 1 - qr : qr;
  const int q0 = qt * BQ;
  const size_t base = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const rsrc_t k_src = make_rsrc(k + base, head_bytes);
  const rsrc_t v_src = make_rsrc(v + base, head_bytes);
  const rsrc_t q_src = make_rsrc(q + base, head_bytes);
  const int qi = q0 + 32 * w + l32;  // this lane's query row

  // Q rows of this wave as MFMA B fragments: Q[qi][16 s + 8 h + 0..7]
  // (rows >= N read as zero).
  bf16x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qf[s] = as_bf16x8(load16(q_src, (uint32_t)(qi * D + 16 * s + 8 * h) * 2u));

  // Key tiles holding at least one visible key for this query tile.
  const int q_hi = q0 + BQ - 1;
  const int kmin = window >= 0 ? max(0, q0 - window) : 0;
  const int kmax = causal ? min(N - 1, q_hi) : N - 1;
  const int kt0 = kmin / kBK, kt1 = kmax / kBK + 1;

  f32x16 oacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) oacc[cb] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;

  TileIO<D, T> io;
  io.load(k_src, v_src, kt0 * kBK, t);
  io.store(Ks[0], Vt[0], t);
  __syncthreads();

  for (int kt = kt0; kt < kt1; ++kt) {
    const int buf = (kt - kt0) & 1;
    const bool more = kt + 1 < kt1;
    if (more) io.load(k_src, v_src, (kt + 1) * kBK, t);
    const bf16* Kc = Ks[buf];
    const bf16* Vc = Vt[buf];

    // S^T = K Q^T for the tile's two 32-key blocks.
    f32x16 sacc[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      sacc[kb2] = f32x16{};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 a = *(const bf16x8*)(Kc + rm_off<D>(kb2 * 32 + l32, 2 * s + h));
        sacc[kb2] = mfma32(a, qf[s], sacc[kb2]);
      }
    }

    // Scale into log2 units and mask (only tiles that straddle a boundary).
    const int k0 = kt * kBK;
    const bool need_mask = (k0 + kBK > N) || (causal && k0 + kBK - 1 > q0) ||
                           (window >= 0 && k0 < q_hi - window);
    float mx = kNegInf;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = sacc[kb2][r] * scale_log2;
        if (need_mask) {
          const int key = k0 + kb2 * 32 + c_row(r, h);
          const bool vis = key < N && (!causal || key <= qi) && (window < 0 || key >= qi - window);
          x = vis ? x : kNegInf;
        }
        sacc[kb2][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, swap_halves(mx));
    const float m_new = fmaxf(m_run, mx);
    const float ref = m_new == kNegInf ? 0.f : m_new;  // nothing visible yet: any finite reference
    const float alpha = __builtin_amdgcn_exp2f(m_run - ref);
    m_run = m_new;

    uint32_t pk[2][8];
    float psum = 0.f;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(sacc[kb2][r] - ref);
        const float p1 = __builtin_amdgcn_exp2f(sacc[kb2][r + 1] - ref);
        psum += p0 + p1;
        pk[kb2][r >> 1] = pack_bf16(p0, p1);
      }
    }
    l_run = alpha * l_run + psum;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) oacc[cb] *= alpha;

    // O^T += V^T P^T, 16 keys per step.
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 pw = {pk[s >> 1][4 * (s & 1) + 0], pk[s >> 1][4 * (s & 1) + 1],
                        pk[s >> 1][4 * (s & 1) + 2], pk[s >> 1][4 * (s & 1) + 3]};
      const bf16x8 pb = as_bf16x8(pw);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const bf16x8 a = *(const bf16x8*)(Vc + vt_off(cb * 32 + l32, 16 * s + 8 * h));
        oacc[cb] = mfma32(a, pb, oacc[cb]);
      }
    }

    if (more) io.store(Ks[buf ^ 1], Vt[buf ^ 1], t);
    __syncthreads();
  }

  // Epilogue: O = O / l, L = m ln2 + ln l.
  const float l_tot = l_run + swap_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qi < N) {
    bf16* orow = o + base + (size_t)qi * D;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 st;
        st.x = pack_bf16(oacc[cb][4 * g + 0] * inv, oacc[cb][4 * g + 1] * inv);
        st.y = pack_bf16(oacc[cb][4 * g + 2] * inv, oacc[cb][4 * g + 3] * inv);
        *(uint2*)(orow + cb * 32 + 8 * g + 4 * h) = st;
      }
    }
    if (h == 0 && lse != nullptr)
      lse[(size_t)bh * N + qi] = l_tot > 0.f ? m_run * kLn2 + logf(l_tot) : kNegInf;
  }
}

template <int D, int NW>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                  int N, float scale, Mask mask, hipStream_t stream) {
  constexpr int BQ = 32 * NW;
  const int nqt = (N + BQ - 1) / BQ;
  const long long grid = (long long)nqt * B * H;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NW>), dim3((unsigned)grid), dim3(64 * NW), 0, stream,
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, lse, B * H, N, nqt,
                     scale * kLog2e, mask.causal, mask.window);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, int d, float scale, Mask mask, int block_q,
                           hipStream_t stream) {
  if (d == 128) {
    if (block_q == 128) return launch<128, 4>(q, k, v, o, lse, B, H, N, scale, mask, stream);
    if (block_q == 64) return launch<128, 2>(q, k, v, o, lse, B, H, N, scale, mask, stream);
    return launch<128, 1>(q, k, v, o, lse, B, H, N, scale, mask, stream);
  }
  if (block_q == 128) return launch<64, 4>(q, k, v, o, lse, B, H, N, scale, mask, stream);
  if (block_q == 64) return launch<64, 2>(q, k, v, o, lse, B, H, N, scale, mask, stream);
  return launch<64, 1>(q, k, v, o, lse, B, H, N, scale, mask, stream);
}

}  // namespace fa
