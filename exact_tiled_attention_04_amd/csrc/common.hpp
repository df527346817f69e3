// Device helpers shared by the attention kernels (gfx950 / CDNA4 only).
//
// MFMA operand layouts used throughout (wave64; verified on gfx950):
//   v_mfma_f32_32x32x16_bf16  C[32x32] += A[32x16] * B[16x32]
//     A: lane l holds A[l%32][8*(l/32) + e], e = 0..7
//     B: lane l holds B[8*(l/32) + e][l%32]
//     C: lane l, register r holds C[8*(r/4) + 4*(l/32) + r%4][l%32]
//   v_mfma_f32_16x16x32_bf16  C[16x16] += A[16x32] * B[32x16]
//     A: lane l holds A[l%16][8*(l/16) + e]
//     B: lane l holds B[8*(l/16) + e][l%16]
//     C: lane l, register r holds C[4*(l/16) + r][l%16]
//   ds_read_b64_tr_b16 (per group of 16 lanes): source lane s supplies the
//     address of 4 consecutive 16-bit values; they form row s/4, columns
//     4*(s%4)..4*(s%4)+3 of a 4x16 block, and lane j receives column j
//     (rows 0..3) of that block.  Pointing the four lanes of row r at
//     M[k0 + r][n0 .. n0 + 15] therefore hands lane j the values
//     M[k0 .. k0+3][n0 + j]: a column read of a row-major tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace eta {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// 2^x on the transcendental unit (inputs below -126 give 0, -inf gives 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Round-to-nearest-even pack of two floats into two bf16 (low = a).
__device__ __forceinline__ unsigned int pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(unsigned int, v);
}

__device__ __forceinline__ float bf16_bits_to_float(unsigned short h) {
  return __builtin_bit_cast(float, ((unsigned int)h) << 16);
}

// LDS transpose read of 4 bf16 (see header comment for the lane mapping).
// The pointer is cast straight to the LDS address space (not through an
// integer) so alias analysis still sees which LDS object it reads.
__device__ __forceinline__ s16x4 lds_read_tr(const void* lds_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)lds_ptr);
}

__device__ __forceinline__ bf16x8 join_tr(const s16x4& lo, const s16x4& hi) {
  u32x4 r;
  u32x2 a = __builtin_bit_cast(u32x2, lo);
  u32x2 b = __builtin_bit_cast(u32x2, hi);
  r[0] = a[0];
  r[1] = a[1];
  r[2] = b[0];
  r[3] = b[1];
  return __builtin_bit_cast(bf16x8, r);
}

// XOR swizzles of the 16-byte chunks of row-major bf16 tiles in LDS (64 banks
// of 4 bytes; a b128 access is served 16 lanes per cycle, a b64 transpose
// read 32 lanes per cycle).  The tiles are read two ways:
//   * row reads (MFMA A operand, ds_read_b128): lanes 0..15 read the same
//     chunk of 16 consecutive rows;
//   * transpose reads (ds_read_b64_tr_b16): 32 lanes read 4 consecutive rows,
//     64 contiguous bytes each.
// tile_swz<D> keeps both conflict-free for rows of D bf16:
//   D = 128 (256-byte rows): the two 2-bit halves of row % 16 swapped, so 16
//     consecutive rows land on 16 distinct chunks and 4 consecutive rows on 4
//     distinct 64-byte groups;
//   D = 64 (128-byte rows, two rows per bank line): row bit 1 moves to chunk
//     bit 2 and row bits 2..3 to chunk bits 0..1, so rows of equal parity
//     among 16 take 8 distinct chunks and rows r, r + 2 differ in chunk bit 2.
template <int D>
__device__ __forceinline__ int tile_swz(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Swizzle of the decode V tile, read only by transposes whose 32 lanes cover
// 8 consecutive rows at the same 32-byte column: the 8 rows must fall on 8
// distinct chunk pairs (D = 128) or, for rows of equal parity, 4 (D = 64).
template <int D>
__device__ __forceinline__ int decode_swz(int row) {
  if constexpr (D == 128) return ((row & 7) << 1) | ((row >> 3) & 1);
  else return (((row >> 1) & 3) << 1) | ((row >> 3) & 1);
}

// Value of lane (l ^ 32): the other half of the wave.
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, 64);
}

// v_permlane32_swap: exchanges lanes 32..63 of `a` with lanes 0..31 of `b`.
// Starting from a = b = x it leaves a = [x_lo | x_lo], b = [x_hi | x_hi], so
// every lane holds both x[l] and x[l ^ 32].  Written as inline assembly with
// both registers as outputs (the compiler builtin drops the second result);
// the s_nops cover the VALU-write / permlane-read hazards on either side.
__device__ __forceinline__ void permlane32_swap(unsigned& a, unsigned& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
// max / sum of lanes l and l ^ 32 without an LDS round trip.
__device__ __forceinline__ float halves_max(float x) {
  unsigned a = __builtin_bit_cast(unsigned, x), b = a;
  permlane32_swap(a, b);
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float halves_sum(float x) {
  unsigned a = __builtin_bit_cast(unsigned, x), b = a;
  permlane32_swap(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// Raw buffer resource over [base, base + bytes): loads past the end return
// zeros and stores past it are dropped, so ragged tiles need no branches.
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(buf_rsrc r, int voffset, int soffset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voffset, soffset, 0));
}
// The same load marked non-temporal (cache policy bit nt): for data read once
// and never again, such as a decode's K and V cache rows.  At 2 waves per
// SIMD of paged decode it raised the sustained read rate by 7-10% over the
// default policy.
__device__ __forceinline__ u32x4 buf_load16_nt(buf_rsrc r, int voffset, int soffset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voffset, soffset, 2));
}

// Direct global -> LDS copy of 16 bytes per lane (buffer_load_dwordx4 ... lds):
// lane l's bytes land at lds_base + 16 * l (lds_base wave-uniform); lanes
// whose offset is past the buffer range write zeros (both verified on gfx950).
// Completion is tracked by vmcnt, not lgkmcnt.
__device__ __forceinline__ void buf_load16_lds(buf_rsrc r, void* lds_base, int voffset,
                                               int soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base,
                                           16, voffset, soffset, 0, 0);
}

// Wait until every vector-memory operation of this wave (including direct
// LDS copies) has completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Stores a wave's 32 x D tile, held in the C layout of 32x32 MFMAs (lane
// (row l % 32, half l / 32) register r of block nb = column
// 32 nb + 8 (r / 4) + 4 (l / 32) + r % 4), times `mul`, in bf16 as whole rows:
// the tile goes through `stage` (32 * 2D bytes of LDS the wave alone uses,
// 16-byte chunk c of row r at chunk c ^ (r % chunks-per-row): conflict-free
// both ways), then each lane stores 16 bytes and every instruction writes
// whole rows.  Row r goes to dst + r * row_stride; rows >= rows_valid are
// skipped.  Storing the C layout directly writes 32 rows in 16-byte pieces
// per instruction, which measured slower.
template <int D>
__device__ __forceinline__ void store_tile_rows(const f32x16 (&acc)[D / 32], float mul,
                                                char* stage, __bf16* dst, size_t row_stride,
                                                int rows_valid, int lane) {
  constexpr int ROW = 2 * D;
  constexpr int CPR = ROW / 16;   // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;   // rows per store instruction
  const int li = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int c = 4 * nb + r4;  // chunk of columns 32 nb + 8 r4 .. + 7
      u32x2 w;
      w[0] = pack_bf16x2(acc[nb][4 * r4 + 0] * mul, acc[nb][4 * r4 + 1] * mul);
      w[1] = pack_bf16x2(acc[nb][4 * r4 + 2] * mul, acc[nb][4 * r4 + 3] * mul);
      *(u32x2*)(stage + li * ROW + ((c ^ (li & (CPR - 1))) * 16) + hh * 8) = w;
    }
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / CPR;
    const int c = lane % CPR;
    const u32x4 v = *(const u32x4*)(stage + r * ROW + ((c ^ (r & (CPR - 1))) * 16));
    if (r < rows_valid) *(u32x4*)(dst + (size_t)r * row_stride + c * 8) = v;
  }
}

// Wave-uniform "any lane true".
__device__ __forceinline__ bool wave_any(bool p) { return __any(p); }

}  // namespace eta
