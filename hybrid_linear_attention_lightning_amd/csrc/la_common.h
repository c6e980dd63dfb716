// la_common.h -- device helpers shared by the Lightning Attention HIP kernels
// (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// Layout helpers of the chunked prefill kernels (forward and fused backward).

__host__ __device__ constexpr int frag_base(int qb) {
  // number of 32-key P^T fragments that query blocks 0..qb-1 use (qb/2+1 each)
  return qb + ((qb & 1) ? (qb >> 1) * (qb >> 1) : (qb >> 1) * ((qb >> 1) - 1));
}

// Swizzle of the 16-byte chunk index of row r of a [C][D] bf16 tile.  It
// depends on r mod 16 only.  In a 64-bank model with 16 lanes served per
// pass, it keeps the row-fragment reads (16 rows x 16 B), the transposing
// reads and the 16-byte direct moves free of bank conflicts at D = 128; the
// K^T read in the state's feature order touches one 8-byte half of each
// chunk and is 2-way at D = 64.
template <int D>
__host__ __device__ constexpr int swz_of(int r) {
  if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  return ((r >> 1) & 1) | ((((r >> 1) ^ (r >> 2)) & 1) << 1) | (((r >> 3) & 1) << 2);
}

// two fp32 -> packed bf16x2 (lo in bits 0..15), round to nearest even; on
// gfx950 this is one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf2f(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// D = A(16x32) * B(32x16) + C on the matrix cores, bf16 inputs, fp32 accumulate.
// Lane l holds A[l%16][8*(l/16) .. +7], B[8*(l/16) .. +7][l%16] and
// D[4*(l/16) + r][l%16] for r = 0..3.
__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4_t lds_read16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i receives element (i % 4) of the 8-byte rows addressed by
// lanes 4r + i/4, for r = 0..3.  If lane i of a group points at row k0 + i/4,
// columns c0 + 4 (i % 4) .. +3 of a row-major bf16 tile, lane i receives the
// column c0 + i of rows k0 .. k0+3: a column fragment of a row-major tile.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2_t lds_read_tr8(const uint16_t* p) {
  const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, r);
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its outstanding global loads (which may be prefetching
// the next chunk, directly into LDS or into registers).
// Wait until at most N vector-memory operations of this wave are
// outstanding (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt
// and lgkmcnt left at their maxima, i.e. not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// x[i] + x[i ^ 16] and x[i] + x[i ^ 32] for lane i of the wave, through the
// gfx950 lane-swap instructions (vector ALU, no LDS): each swap returns the
// two halves of the exchanged pair, whose sum is the wanted one.
__device__ __forceinline__ float sum_lane_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_lane_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The value of x, hidden from the optimizer (an empty asm that "may change"
// it): keeps address arithmetic from being hoisted or folded across the
// point where it is called.  opaque_s keeps a wave-uniform value in an SGPR.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ uint32_t opaque_s(uint32_t x) {
  asm volatile("" : "+s"(x));
  return x;
}
// base + off bytes, for a wave-uniform base and a per-lane unsigned 32-bit
// byte offset: the operands of the scalar-base + 32-bit vector-offset form
// of the global memory instructions, which needs no 64-bit vector address
// arithmetic per access.  The offset passes through an empty asm at each
// use, so that its widening to 64 bits is not hoisted away from the access
// (the instruction form is chosen only where the widening is seen).
__device__ __forceinline__ const uint16_t* at_bytes(const uint16_t* base, uint32_t off) {
  asm volatile("" : "+v"(off));
  return reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(base) + off);
}
__device__ __forceinline__ uint16_t* at_bytes(uint16_t* base, uint32_t off) {
  asm volatile("" : "+v"(off));
  return reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(base) + off);
}
// Raw buffer resource (stride 0) over 2 GiB from base: the operand of the
// buffer memory instructions.  Dword 3 is the gfx9 format word for 32-bit
// elements.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff,
                                           0x00020000);
}
// Direct move of 16 bytes per lane, from the buffer at byte offset voff
// (per lane) into LDS: lane i writes the 16 bytes at lds + 16 i.
//  * The buffer form (buffer_load_dwordx4 ... lds) is used rather than the
//    global one: the compiler counts a pending global_load_lds among the
//    LDS-counter events as well, which turns every later LDS wait into a
//    wait for zero outstanding operations; a buffer load only counts as a
//    vector-memory operation.
//  * The loads are marked non-temporal (nt): every byte is read once, and
//    the streamed tiles need not stay in the caches (measured a few percent
//    faster on the 128K prefill, main pass and pre-pass).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds) {
  constexpr int kNonTemporal = 2;  // cache-policy bit nt
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)(uintptr_t)lds, 16, voff, 0, 0, kNonTemporal);
}
// x, known to be the same in every lane, as a scalar value
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// 2^x without the denormal-range fix-up of exp2f (v_exp_f32; results below
// 2^-126 flush to zero, which the decay factors tolerate).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Split four fp32 values into bf16 hi + lo parts (x ~= hi + lo to about 2^-16
// relative): the matrix cores then see 16 significant bits instead of 8.
// hi is x rounded to bf16; the residual x - hi is exact in fp32 and comes
// from one bf16 dot product per value (hi_pair . (-1, 0) + x), with both
// products exact, instead of unpacking hi and subtracting.
__device__ __forceinline__ void split4(f32x4_t x, u32x2_t& hi, u32x2_t& lo) {
  const uint32_t h0 = pack2(x[0], x[1]), h1 = pack2(x[2], x[3]);
  hi = u32x2_t{h0, h1};
  // (-1, 0) and (0, -1) as bf16 pairs, passed as opaque bit patterns: as
  // inline constants the packed pair would be encoded as the fp32 constant
  // -1.0, whose bf16 halves are (0, -1)
  const bf16x2_t neg_lo = __builtin_bit_cast(bf16x2_t, opaque_s(0x0000BF80u));
  const bf16x2_t neg_hi = __builtin_bit_cast(bf16x2_t, opaque_s(0xBF800000u));
  const bf16x2_t p0 = __builtin_bit_cast(bf16x2_t, h0), p1 = __builtin_bit_cast(bf16x2_t, h1);
  lo = u32x2_t{pack2(__builtin_amdgcn_fdot2_f32_bf16(p0, neg_lo, x[0], false),
                     __builtin_amdgcn_fdot2_f32_bf16(p0, neg_hi, x[1], false)),
               pack2(__builtin_amdgcn_fdot2_f32_bf16(p1, neg_lo, x[2], false),
                     __builtin_amdgcn_fdot2_f32_bf16(p1, neg_hi, x[3], false))};
}

}  // namespace la
