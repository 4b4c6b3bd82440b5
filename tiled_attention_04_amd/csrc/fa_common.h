// Device-side building blocks shared by the libfa355 kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------- bf16 ----

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Two floats -> packed bf16 pair (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// ---------------------------------------------------------------- fp16 ----

typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(f16, (uint16_t)w); }
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(f16, (uint16_t)(w >> 16));
}

// ------------------------------------------ 16-bit MFMA element types ----
// The matrix-core kernels are written once for T = bf16 or f16: both are
// 16-bit, so tiles, LDS layouts and transpose reads are identical; only the
// MFMA opcode and the float <-> T conversions differ.
template <typename T> struct Elem16;
template <> struct Elem16<bf16> { typedef bf16x8 v8; typedef bf16x2 v2; };
template <> struct Elem16<f16> { typedef f16x8 v8; typedef f16x2 v2; };
template <typename T> using vec8 = typename Elem16<T>::v8;

template <typename T>
__device__ __forceinline__ vec8<T> as_vec8(uint4 u) { return __builtin_bit_cast(vec8<T>, u); }

// Two floats -> packed pair of T (round to nearest even).
template <typename T>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, typename Elem16<T>::v2));
}

// Low / high element of a packed pair of T, widened to float (exact).
template <typename T> __device__ __forceinline__ float lo16(uint32_t w);
template <typename T> __device__ __forceinline__ float hi16(uint32_t w);
template <> __device__ __forceinline__ float lo16<bf16>(uint32_t w) { return bf16_lo(w); }
template <> __device__ __forceinline__ float hi16<bf16>(uint32_t w) { return bf16_hi(w); }
template <> __device__ __forceinline__ float lo16<f16>(uint32_t w) { return f16_lo(w); }
template <> __device__ __forceinline__ float hi16<f16>(uint32_t w) { return f16_hi(w); }

// 32-bit word i (compile-time after unrolling) of a 16-byte register value.
__device__ __forceinline__ uint32_t word(const uint4& u, int i) {
  return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w;
}

// ------------------------------------------------------- buffer loads ----
// A buffer resource covering `bytes` bytes from `base`: 16-byte loads at or
// past the end read as zero, so ragged tails need no branches.  Offsets are
// 32-bit byte offsets from `base`.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 load16(rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// One float to a buffer at a byte offset (dropped past the buffer's end).
// The value is first forced into a VGPR: a store whose data is an element
// of an accumulator vector held in AGPRs has been compiled to store the
// vector's first element for every index.
__device__ __forceinline__ void store_f32(rsrc_t r, uint32_t byte_off, float x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm("" : "+v"(x));
#endif
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), r, byte_off, 0, 0);
}

// ---------------------------------------------------------------- MFMA ----
// v_mfma_f32_32x32x16_bf16.  Operand layout (wave64):
//   A (32 x 16, row-major M x K): lane l holds A[l % 32][8 * (l / 32) + 0..7]
//   B (16 x 32, K x N):           lane l holds B[8 * (l / 32) + 0..7][l % 32]
//   C (32 x 32):                  lane l, element r holds
//                                 C[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32]
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_32x32x16_f16: the same operand and accumulator layouts.
__device__ __forceinline__ f32x16 mfma32(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Row index (within a 32 x 32 C block) of element r for a lane in half h.
__device__ __forceinline__ constexpr int c_row(int r, int h) { return 8 * (r / 4) + 4 * h + (r % 4); }

// --------------------------------------------------------- cross-lane ----

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of G lanes (G in {1,2,4,8,16,32,64}); every lane of
// the group receives the total.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (G >= 2) x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]
  if constexpr (G >= 4) x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]
  if constexpr (G >= 8) x += dpp<0x141>(x);   // row_half_mirror
  if constexpr (G >= 16) x += dpp<0x140>(x);  // row_mirror
  if constexpr (G >= 32) x += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
  if constexpr (G >= 64) x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32); }

// The two halves of the wave exchanged by one VALU lane swap
// (v_permlane32_swap): returns {value of lanes 0-31, value of lanes 32-63}
// as seen by lane l and lane l ^ 32 alike.  (The vector result is copied to
// scalars before any bit cast: casting its subscripted elements directly is
// miscompiled.)
__device__ __forceinline__ void wave_halves(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, x), false, false);
  const unsigned a = r[0], b = r[1];
  lo = __builtin_bit_cast(float, a);
  hi = __builtin_bit_cast(float, b);
}

// max / sum of x over lanes l and l ^ 32; both lanes get the same bits.
__device__ __forceinline__ float pair_max(float x) {
  float a, b;
  wave_halves(x, a, b);
  return a > b ? a : b;
}
__device__ __forceinline__ float pair_sum(float x) {
  float a, b;
  wave_halves(x, a, b);
  return a + b;
}

// Workgroup id -> (head slice bh, tile rank r) for a grid of BH * ntiles
// workgroups; rank 0 is dispatched first.  Consecutive ids go round-robin
// over the 8 XCDs of the chip and, when BH is a multiple of 8, every head
// stays on one XCD (its K/V are shared in that XCD's L2).  Each XCD walks
// its heads in groups, all ranks of a group before the next group, so only
// the group's heads are live in its L2:
//  * spread (for plain causal attention, where rank 0 is the most expensive
//    tile and the cost falls with the rank): groups of four heads, rank by
//    rank inside a group, so every group ends with its cheapest tiles and
//    the tail stays short (measured 2-3% faster than one group of all
//    heads, whose K/V leave the L2 between ranks, and than groups of two);
//  * grouped (work about the same for every tile): groups of two heads.
__device__ __forceinline__ void tile_order(int id, int BH, int ntiles, bool spread, int& bh, int& r) {
  if ((BH & 7) == 0) {
    const int xcd = id & 7, slot = id >> 3, nbh8 = BH >> 3;
    const int G = spread ? (nbh8 < 4 ? nbh8 : 4) : 2;  // heads per group and XCD
    const int full = nbh8 / G;        // groups of G heads; a last group may hold fewer
    int grp, hh;
    if (slot < full * G * ntiles) {
      grp = slot / (G * ntiles);
      const int rem = slot - grp * G * ntiles;
      r = rem / G;
      hh = rem - r * G;
    } else {
      const int rem = slot - full * G * ntiles, last = nbh8 - full * G;
      grp = full;
      r = rem / last;
      hh = rem - r * last;
    }
    bh = (grp * G + hh) * 8 + xcd;
  } else {
    r = id / BH;
    bh = id - r * BH;
  }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// One 16-byte (4-byte) direct load per lane from a buffer resource into LDS:
// lane l's bytes land at dst + 16 l (dst + 4 l); dst is wave-uniform.  Kept
// out of lambdas: the host pass rejects this builtin there and then silently
// drops the kernel.
__device__ __forceinline__ void load_lds16(rsrc_t src, char* dst, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void*)dst, 16, voffset, 0, 0, 0);
}
__device__ __forceinline__ void load_lds4(rsrc_t src, void* dst, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void*)dst, 4, voffset, 0, 0, 0);
}

// Global byte offset (within the tile) that lane `lane` of direct-load block
// `blk` must fetch, for a tile stored with `pitch` bytes per row; lanes that
// land on row padding get an offset past any buffer so they read zero.
template <int D>
__device__ __forceinline__ uint32_t block_src(int blk, int lane, int pitch) {
  const int pos = blk * 1024 + lane * 16;
  const int row = pos / pitch, col = pos - row * pitch;
  return col < D * 2 ? (uint32_t)(row * D * 2 + col) : 0x80000000u;
}

// V^T-style operand of one 32x32x16 MFMA from a row-major 16-bit tile in LDS:
// two transpose reads, 8 rows apart, at this lane's address a.
template <int PITCH, typename T = bf16>
__device__ __forceinline__ vec8<T> read_tr8(const char* a) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 8 * PITCH));
  const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
  return as_vec8<T>(uint4{l2.x, l2.y, h2.x, h2.y});
}

// This lane's transpose-read address in a row-major 16-bit tile with
// PITCH-byte rows.  With +16 s rows (a 16-row step) and +64 c bytes (a
// 32-column block) read_tr8 yields, in lane l, 8 rows of column 32 c + l % 32
// -- rows 16 s + {0..3, 8..11} in the lower half of the wave and
// 16 s + {4..7, 12..15} in the upper half, the row order of the 32x32 MFMA
// accumulator -- i.e. the operand "row block of 32, 16 along K" of an MFMA
// whose K dimension runs along the tile's rows.
template <int PITCH>
__device__ __forceinline__ int tr_addr(int lane) {
  const int g = lane >> 4, gi = lane & 15;
  return (4 * (g >> 1) + (gi >> 2)) * PITCH + (16 * (g & 1) + 4 * (gi & 3)) * 2;
}

// s_waitcnt on the vector-memory counter only: wait until at most n of this
// wave's vector loads (here: direct loads into LDS) are still in flight
// (n above 12 waits for 12).
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {  // the count is an immediate operand
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
    case 10: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
    case 11: __builtin_amdgcn_s_waitcnt(0x0F7B); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
  }
}

// Workgroup barrier that does not drain outstanding vector loads (unlike
// __syncthreads, whose release fence waits for every memory operation).  The
// "memory" clobber keeps LDS accesses on their side of it and the scheduling
// barriers keep all other instructions there too (the ping-pong phases rely
// on it).
__device__ __forceinline__ void barrier_keep_loads() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// The same, after this wave's LDS writes have completed (for data other
// waves read after the barrier).
__device__ __forceinline__ void barrier_after_lds_writes() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Ping-pong group of the calling wave: the order in which waves arrive on
// their SIMD (HW_ID bits 5:4), modulo 2, so that each SIMD hosts one wave of
// each group when the workgroup's waves are spread evenly.  `slots` is a
// zeroed per-SIMD counter in LDS.
__device__ __forceinline__ int wave_group(int* slots, int lane) {
  const int simd = __builtin_amdgcn_s_getreg((1 << 11) | (4 << 6) | 4) & 3;
  int slot = 0;
  if (lane == 0) slot = atomicAdd(&slots[simd], 1);
  return __builtin_amdgcn_readfirstlane(slot) & 1;
}

}  // namespace fa
