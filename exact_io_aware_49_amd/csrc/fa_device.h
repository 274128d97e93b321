// fa_device.h -- device-side types and helpers shared by the gfx950 kernels.
//
// Matrix-core conventions (CDNA3/CDNA4 MFMA, wave64), used by every kernel:
//   v_mfma_f32_32x32x16_bf16  C[32x32] += A[32x16] * B[16x32]
//     A operand: lane l holds row (l % 32) and 8 consecutive k-slots of half (l / 32).
//     B operand: lane l holds column (l % 32) and the same 8 k-slots.
//     C/D      : lane l, register r holds C[row][col] with col = l % 32 and
//                row = 8 * (r / 4) + 4 * (l / 32) + (r % 4).
//   Which physical k each (half, slot) denotes does not matter as long as A and
//   B use the same assignment, so kernels choose whatever k-order makes their
//   loads contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "fa_map.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef short shortx4 __attribute__((ext_vector_type(4)));

#define FA_LDS(T, p) ((__attribute__((address_space(3))) T *)(p))

// Calls f(std::integral_constant<int, I>{}) for I = 0 .. N-1 (compile-time loop).
template <int N, typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ floatx16 mfma32x32x16(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

// 16-byte loads/stores.
__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }
__device__ __forceinline__ void st8(void *p, u32x2 v) { *reinterpret_cast<u32x2 *>(p) = v; }

// Pack two floats into bf16 (round to nearest, ties to even), low half first:
// one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const floatx2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// lo + hi of a packed bf16 pair, accumulated in float32 (v_dot2c_f32_bf16 with (1, 1)).
__device__ __forceinline__ float add_bf16_pair(uint32_t pair, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
}

// Both halves of the wave exchange a value: returns {lanes 0..31 of x twice,
// lanes 32..63 of x twice} as (first, second); per lane, one of the two is its
// own value and the other its partner's (lane ^ 32).  v_permlane32_swap_b32.
__device__ __forceinline__ float max_with_partner(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_partner(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Eight floats -> bf16x8 operand.
__device__ __forceinline__ bf16x8 to_bf16x8(float f0, float f1, float f2, float f3, float f4, float f5,
                                            float f6, float f7) {
  u32x4 u;
  u[0] = pack_bf16x2(f0, f1);
  u[1] = pack_bf16x2(f2, f3);
  u[2] = pack_bf16x2(f4, f5);
  u[3] = pack_bf16x2(f6, f7);
  return as_bf16x8(u);
}

// 2^x on the transcendental unit (exact 0 for -inf).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Exchange a value with the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

// bf16 bit pattern of the low / high half of a 32-bit word, as float.
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Row index permutation used when loading the A operand of a score tile:
// swapping bits 2 and 3 of the row index makes C-register r of lane half h
// hold row 16 * (r / 8) + 8 * h + (r % 8), i.e. eight consecutive registers
// cover eight consecutive rows, which is the k-slot order the next product
// (scores times values) wants for its B operand.
__device__ __forceinline__ int swap_bits23(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// ---- staging of 4-row x 8-column bf16 blocks into LDS -----------------------
// A block is rows r0..r0+3, columns 8g..8g+7 of a row-major [nrows][ld] bf16
// matrix: four 16-byte vectors, one per row.  Rows >= nrows read as zero.
__device__ __forceinline__ void load_block4x8(u32x4 (&blk)[4], const __bf16 *base, int r0, int nrows, int ld,
                                              int g) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = r0 + u;
    blk[u] = (r < nrows) ? ld16(base + (size_t)r * ld + 8 * g) : u32x4{0, 0, 0, 0};
  }
}

// Row-major copy: lds[(lr0 + u) * stride + 8g .. +8) = row u of the block.
__device__ __forceinline__ void store_block_rows(__bf16 *lds, int stride, int lr0, int g, const u32x4 (&blk)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) st16(lds + (lr0 + u) * stride + 8 * g, blk[u]);
}

// Transposed copy: ldsT[(8g + e) * strideT + lr0 .. +4) = column e of the block
// (the four rows' values of column 8g+e), for e = 0..7.
__device__ __forceinline__ void store_block_transposed(__bf16 *ldsT, int strideT, int lr0, int g,
                                                       const u32x4 (&blk)[4]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t a0 = blk[0][p], a1 = blk[1][p], a2 = blk[2][p], a3 = blk[3][p];
    u32x2 lo, hi;
    // v_perm_b32 picks bytes from {src0 (bytes 4..7), src1 (bytes 0..3)}
    lo[0] = __builtin_amdgcn_perm(a1, a0, 0x05040100u);  // col 2p of rows 0,1
    lo[1] = __builtin_amdgcn_perm(a3, a2, 0x05040100u);  // col 2p of rows 2,3
    hi[0] = __builtin_amdgcn_perm(a1, a0, 0x07060302u);  // col 2p+1 of rows 0,1
    hi[1] = __builtin_amdgcn_perm(a3, a2, 0x07060302u);  // col 2p+1 of rows 2,3
    st8(ldsT + (8 * g + 2 * p) * strideT + lr0, lo);
    st8(ldsT + (8 * g + 2 * p + 1) * strideT + lr0, hi);
  }
}

// ---- direct global -> LDS loads ------------------------------------------
// A buffer resource over `bytes` bytes at `base`: loads at offsets >= bytes
// return zero, which is how rows past the end of a sequence read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from rsrc + voffset into LDS at lds_wave_base + 16 * lane
// (buffer_load_dwordx4 ... lds).  lds_wave_base must be wave-uniform.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, void *lds_wave_base, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, FA_LDS(void, lds_wave_base), 16, (int)voffset, 0, 0, 0);
}

// 4 bytes per lane into LDS at lds_wave_base + 4 * lane (buffer_load_dword ... lds).
__device__ __forceinline__ void load_lds4(__amdgpu_buffer_rsrc_t rsrc, void *lds_wave_base, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, FA_LDS(void, lds_wave_base), 4, (int)voffset, 0, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Chunk permutation for a row-major bf16 tile of d = 64, 128 or 256 columns that is
// read both as rows (16 consecutive rows, one 16-byte chunk each: the A operand
// of a 32x32x16 MFMA) and transposed (ds_read_b64_tr_b16: 4 consecutive rows x
// 4 chunks per 32 lanes).  physical chunk = logical chunk ^ swz_rt(row); both
// patterns then hit 64 distinct banks.  Rows 16 apart share a permutation.  At
// d >= 128 a row is a whole number of 256-byte bank cycles, so d = 256 uses the
// d = 128 pattern on its first 16 chunks (chunks 16..31 keep bit 4).
template <int D>
__device__ __forceinline__ int swz_rt(int r) {
  if constexpr (D == 32) return (r >> 2) & 3;  // four 64-byte rows per bank cycle
  return (D >= 128) ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Chunk permutations of a streamed K or V tile (physical chunk = logical
// chunk ^ swz(row)).  swz_k makes the score reads (16 consecutive rows, one
// 16-byte chunk each) hit distinct banks; swz_v does the same for the
// transposed value reads (4 rows x 4 chunks per 16 lanes).  At d >= 128 a row
// is a multiple of the 256-byte bank cycle, so d = 128 and d = 256 share them.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  if constexpr (D == 32) return (r >> 2) & 3;
  return (D >= 128) ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  if constexpr (D == 32) return (r >> 2) & 3;  // the 4 rows of a transposed read share a value
  return (D >= 128) ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)FA_LDS(const void, p);
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane j supplies the address
// of 4 consecutive bf16 of some row; lane i receives element (i % 4) of the
// rows supplied by lanes 4t + i / 4, t = 0..3 (in that order).  Used to read a
// transposed operand straight from a row-major LDS tile.
//
// Issued through inline asm: the compiler would otherwise wait for every
// outstanding global->LDS transfer before it (it cannot prove the transfer
// writes a different buffer).  The caller must therefore (1) only read LDS
// whose transfers are known complete (vmcnt(0) + barrier) and (2) call
// lds_wait() on the results before using them.
__device__ __forceinline__ u32x2 ds_read_tr16(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr) : "memory");
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_tr16_at(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field is 16 bits");
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}

// ds_read_b128 at addr + OFF, issued through inline asm (same contract as
// ds_read_tr16: the caller guarantees completed transfers and waits with
// lds_wait before use).
template <int OFF>
__device__ __forceinline__ u32x4 ds_read_b128_at(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field is 16 bits");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}

// max(a, b, c): the compiler forms v_max3_f32 from it.  (Not inline asm: the
// operands are often fresh matrix-core results, and only the compiler pads a
// read of those with the wait states the hardware needs.)
__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}

// s_waitcnt lgkmcnt(0) followed by empty asm statements that redefine each of
// the given registers: every later use reads the post-wait value.
template <typename T>
__device__ __forceinline__ void redefine(T &r) {
  asm volatile("" : "+v"(r));
}
template <typename... T>
__device__ __forceinline__ void lds_wait_all(T &...regs) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  (redefine(regs), ...);
}

// s_waitcnt lgkmcnt(0), with the given registers routed through it so that
// no use of them can be scheduled before the wait.
__device__ __forceinline__ void lds_wait(u32x2 &a, u32x2 &b, u32x2 &c, u32x2 &d) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}
__device__ __forceinline__ void lds_wait(u32x4 &a, u32x4 &b, u32x4 &c, u32x4 &d) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}
__device__ __forceinline__ void lds_wait(u32x4 &a, u32x4 &b) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void lds_wait(u32x4 &a) { asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a)); }
__device__ __forceinline__ void lds_wait(u32x2 &a, u32x2 &b, u32x4 &c) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c));
}
__device__ __forceinline__ void lds_wait(u32x2 &a, u32x2 &b) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b));
}

}  // namespace fa
