// Device helpers shared by the HIP kernels of the FLARE++ mixer (forward and backward): types,
// MFMA wrappers with their lane layouts, lane moves and 16-byte chunk conversions. Every function
// has internal linkage, one copy per translation unit.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace flarepp {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRmsEps = 1e-6f;


__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }
__device__ __forceinline__ float shfl(float v, int src) { return __shfl(v, src, 64); }

// Score MFMAs start from a zero accumulator, so the register allocator may place their destination
// on top of an A or B operand that dies there; the double-depth 16x16x32 bf16 form then returns
// wrong products. Operands that feed several score MFMAs are kept live until all of them have been
// issued: the MFMAs stay above a scheduling barrier that only they may not cross, and an empty asm
// statement below it uses the operands.
__device__ __forceinline__ void keep_live(const bf16x8& x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void keep_live(const bf16x4& x) { asm volatile("" ::"v"(x)); }
template <typename S>  // fp32 operand structs: one register per element
__device__ __forceinline__ void keep_live(const S& x) {
#pragma unroll
  for (int i = 0; i < (int)(sizeof(S) / sizeof(float)); i++) asm volatile("" ::"v"(x.v[i]));
}
// sched_barrier mask: VALU, SALU, memory and transcendental instructions may cross; MFMA may not.
constexpr int kAllButMfma = 0x7F6;

__device__ __forceinline__ f32x4 mfma_32k(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16k(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_4k(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// 32x32x16 bf16 (gfx950): lane l supplies row (l % 32) of A and column (l % 32) of B with
// k = 8 (l / 32) .. 8 (l / 32) + 7, and receives column (l % 32), rows 8 (v / 4) + 4 (l / 32) + v % 4
// (v = 0..15) of the 32x32 result.
__device__ __forceinline__ f32x16 mfma_32x32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_32x32_f16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void keep_live(const f32x16& x) { asm volatile("" ::"v"(x)); }
// The register allocator may place an MFMA's destination on top of an A or B operand that dies at
// that instruction, and the double-depth gfx950 MFMA forms then return wrong products. hold(acc, x)
// keeps x live past the MFMA that produced acc: an empty asm that reads x and rewrites acc, so it can
// only come after that MFMA, whatever order instruction selection and scheduling choose.
template <typename O>
__device__ __forceinline__ void hold(f32x16& acc, const O& x) {
  asm volatile("" : "+v"(acc) : "v"(x));
}
__device__ __forceinline__ void keep_live(const f16x8& x) { asm volatile("" ::"v"(x)); }
// bf16 -> fp16, rounding to nearest even (exact inside the fp16 range; overflow gives inf, which
// the range check of the zero-shift pass catches).
__device__ __forceinline__ f16x8 to_f16x8(bf16x8 x) {
  f16x8 r;
#pragma unroll
  for (int e = 0; e < 8; e++) r[e] = (f16)(float)x[e];
  return r;
}
// Row (or column) of the 32x32 result held in slot v by a lane of half h = l / 32.
__host__ __device__ constexpr int row32(int v, int h) { return 8 * (v >> 2) + 4 * h + (v & 3); }

// Sums of packed probabilities on the matrix unit. A bf16x8 operand of the 32x32x16 layout (lane l:
// index l % 32, eight k values) read as a 16x16x32 operand puts index i and i + 16 in the same
// 16-row, in the even and odd k-slices. Against this 0/1 selector (all ones in k-slices of the
// matching parity, columns 0-7 for even slices and 8-15 for odd ones) the 16x16x32 MFMA returns
// the sum over the k values of index i in row (or column) i % 16 of columns (rows) 0-7 when
// i < 16, and of columns (rows) 8-15 when i >= 16.
__device__ __forceinline__ bf16x8 sum_selector(int lane) {
  const bool one = (((lane >> 4) & 1) == 0) == ((lane & 15) < 8);
  const bf16 v = one ? (bf16)1.0f : (bf16)0.0f;
  return bf16x8{v, v, v, v, v, v, v, v};
}

// Transposed LDS read of 4 bf16 (ds_read_b64_tr_b16). Every lane addresses 8 bytes; within each
// group of 16 lanes, lane i receives as element j the element i % 4 of the 8 bytes addressed by
// group lane 4 j + i / 4. `p` points into LDS.
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* p) {
  lds_s16x4* q = (lds_s16x4*)(__attribute__((address_space(3))) char*)(p);
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(q));
}

template <typename T>
__device__ __forceinline__ float to_f(T x) { return (float)x; }

// Parts per routing query in the score MFMAs of the exact passes: bf16 keeps a hi/lo pair, fp32
// one exact value.
template <typename T>
constexpr int kQParts = sizeof(T) == 2 ? 2 : 1;
// Elements per routing-query row in the workspace: bf16 rows hold hi, lo and the fp16 query (the
// score operand of the zero-shift passes, stored as raw fp16 bits); fp32 rows hold the query.
template <typename T>
constexpr int kQRow = sizeof(T) == 2 ? 3 : 1;

// 16-byte global/LDS chunk.
typedef uint32_t Chunk __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ void chunk_to_float(const Chunk& c, float* out) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      out[2 * i] = __uint_as_float(c[i] << 16);
      out[2 * i + 1] = __uint_as_float(c[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; i++) out[i] = __uint_as_float(c[i]);
  }
}

template <typename T>
__device__ __forceinline__ Chunk float_to_chunk(const float* v) {
  Chunk c;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      bf16x2 p = {(bf16)v[2 * i], (bf16)v[2 * i + 1]};
      c[i] = __builtin_bit_cast(uint32_t, p);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; i++) c[i] = __float_as_uint(v[i]);
  }
  return c;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}

// Sum over aligned groups of N consecutive lanes (N = 1, 2, 4, 8) with DPP lane moves.
template <int DPP>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), DPP, 0xF, 0xF, false));
}
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp_move<0xB1>(v);   // quad_perm(1,0,3,2): lane ^ 1
  if constexpr (N >= 4) v += dpp_move<0x4E>(v);   // quad_perm(2,3,0,1): lane ^ 2
  if constexpr (N >= 8) v += dpp_move<0x141>(v);  // row_half_mirror: the other quad of 8 lanes
  return v;
}

}  // namespace
}  // namespace flarepp
