// Microbenchmarks behind the roofline denominators of the FLARE++ mixer's kernels on gfx950: the
// issue rate of v_exp_f32 (one per softmax score), of plain fp32 VALU work, of the 32x32x16 bf16
// matrix instruction, of their mixes (whether one pipe's work hides under another's), and the HBM
// stream rate. Built as its own library (libflarepp_microbench.so) so the mixer library carries no
// benchmark code; the benchmark script reaches it with --microbench.
//
// Every kernel runs a fixed number of loop iterations per lane over independent dependency chains
// (enough of them to cover each pipe's latency), on a grid of 4-wave workgroups that puts `wps`
// waves on every SIMD of the chip, and writes one value per lane so that nothing is dead code.
// Rates are instructions (or bytes) per second over the whole device, from HIP events around the
// launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device.h"

namespace {

using flarepp::bf16x8;
using flarepp::f32x16;

constexpr int kChains = 8;  // independent chains per lane

// Kinds. Per loop iteration and lane: kExp 8 exps; kFma 8 fmas; kExpFma 8 exps and 8 fmas;
// kMfma 4 MFMAs (32x32x16 bf16); kMfmaFma 4 MFMAs and 32 fmas; kMfmaExp 4 MFMAs and 16 exps;
// kMfmaExpFma 4 MFMAs, 16 exps and 16 fmas. kTile and kTileAgpr: the per-tile loop of the split-N
// partial kernels without LDS (one 32x32 tile of scores per iteration: two 32x32x16 fp16 score
// MFMAs for the next tile, 16 exps and 8 bf16 packs of this tile's scores, two 32x32x16 bf16 P.V
// MFMAs and two 16x16x32 row-sum MFMAs); kTile leaves the register form of every MFMA to the
// compiler, kTileAgpr keeps the P.V and row-sum accumulators in AGPRs. kTileLds reads the key and
// value operands from LDS tiles laid out as in the kernels; kTileWg16 runs it in 16-wave workgroups
// (4 waves per SIMD from one workgroup) and kTileWg16Sync adds a workgroup barrier every 8 tiles,
// as the kernels' 256-token stages do; kTileRand is kTileWg16Sync on pseudo-random keys and values
// (scores of a few units, as the mixer's workloads give; the others' nearly constant operands
// switch fewer bits, which lets the clock rise). kExpF16: 8 v_exp_f16 per iteration.
// kTileRandNoSum leaves the row sums out of kTileRand, kTileRandDot2 takes them with 8 v_dot2 per
// tile instead of the two row-sum MFMAs; kMfmaRand is kMfma on pseudo-random operands.
enum Kind {
  kExp = 0, kFma, kExpFma, kMfma, kMfmaFma, kMfmaExp, kMfmaExpFma, kTile, kTileAgpr, kTileLds, kTileWg16,
  kTileWg16Sync, kTileRand, kExpF16, kTileRandNoSum, kTileRandDot2, kMfmaRand, kNumCompute
};
// Row sums of a tile loop variant: on the matrix unit, left out, or on v_dot2.
enum SumMode { kSumMfma = 0, kSumNone, kSumDot2 };

using flarepp::f16x8;
using flarepp::f32x4;

// B operand of a 32x32x16 P.V MFMA from a row-major bf16 LDS tile with rows along k (the layout the
// kernels read their value tiles in): two transposed 8-byte reads per lane.
__device__ __forceinline__ bf16x8 flarepp_lds_rows32(const __bf16* tile, int stride, int r0, int lane) {
  const int i = lane & 15, cb = (lane >> 4) & 1, h = lane >> 5;
  const __bf16* p = tile + (r0 + 4 * h + (i >> 2)) * stride + 16 * cb + 4 * (i & 3);
  const flarepp::bf16x4 lo = flarepp::lds_read_tr4(p);
  const flarepp::bf16x4 hi = flarepp::lds_read_tr4(p + 8 * stride);
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 4; e++) {
    o[e] = lo[e];
    o[4 + e] = hi[e];
  }
  return o;
}

// The partial kernels' tile loop (see Kind). The MFMAs are written out so that each accumulator
// sits in the register file named by the variant (the compiler would pick its own); the score
// MFMAs of the next tile are issued a whole iteration before the exponentials read their results,
// as in the kernels, and the packs' results reach the P.V MFMAs after two wait states. Operands are
// made opaque to the compiler each iteration (empty asm) so that nothing is hoisted out of the loop.
// Pseudo-random value in [-1, 1) from an index (an integer hash).
__device__ __forceinline__ float hash_unit(uint32_t i) {
  i ^= i >> 16;
  i *= 0x7feb352du;
  i ^= i >> 15;
  i *= 0x846ca68bu;
  i ^= i >> 16;
  return (float)(int32_t)i * 0x1p-31f;
}

template <bool AGPR, bool LDS, int NW, bool SYNC, bool RAND = false, int SUM = kSumMfma>
__global__ __launch_bounds__(NW * 64) void tile_kernel(float* out, int iters, float seed) {
  const int lane_id = threadIdx.x + blockIdx.x * blockDim.x;
  const int lane = threadIdx.x & 63;
  // LDS tiles of 256 tokens as the kernels stage them: fp16 keys with rows of 40 halfwords, bf16
  // values with rows of 48.
  constexpr int RS = 40, VS = 48, STG = 256;
  __shared__ __align__(16) _Float16 ks[LDS ? STG * RS : 1];
  __shared__ __align__(16) __bf16 vs[LDS ? STG * VS : 1];
  if constexpr (LDS) {
    for (int i = threadIdx.x; i < STG * RS; i += NW * 64)
      ks[i] = (_Float16)(RAND ? 0.6f * hash_unit(i + 977u * blockIdx.x) : 0.001f * (i & 7));
    for (int i = threadIdx.x; i < STG * VS; i += NW * 64)
      vs[i] = (__bf16)(RAND ? hash_unit(i + 7919u * blockIdx.x + 12345u) : 0.01f * (i & 7));
    __syncthreads();
  }
  f16x8 k0, k1, q0, q1;
  bf16x8 v0, v1, sel;
#pragma unroll
  for (int e = 0; e < 8; e++) {
    k0[e] = (_Float16)(seed * 0.1f * e);
    k1[e] = (_Float16)(-seed * 0.1f * e);
    q0[e] = (_Float16)(RAND ? 0.6f * hash_unit(lane * 8 + e) : 0.05f * e);
    q1[e] = (_Float16)(RAND ? 0.6f * hash_unit(lane * 8 + e + 512) : 0.02f * e);
    v0[e] = (__bf16)(0.3f * e);
    v1[e] = (__bf16)(0.1f * e);
    sel[e] = (__bf16)1.0f;
  }
  f32x16 zw = {}, sa = {}, sb = {};
  f32x4 ls = {};
  float lsum = 0.f;
  // One tile: scores of the next tile into `nx`, exponentials and P.V of this tile's `cu`.
  auto tile = [&](f32x16& cu, f32x16& nx, int st) __attribute__((always_inline)) {
    if constexpr (LDS) {
      const _Float16* kr = ks + (32 * st + (lane & 31)) * RS + 8 * (lane >> 5);
      k0 = *reinterpret_cast<const f16x8*>(kr);
      k1 = *reinterpret_cast<const f16x8*>(kr + 16);
      v0 = flarepp_lds_rows32(vs, VS, 32 * st, lane);
      v1 = flarepp_lds_rows32(vs, VS, 32 * st + 16, lane);
    }
    asm volatile(
        "v_mfma_f32_32x32x16_f16 %0, %1, %3, 0\n\t"
        "v_mfma_f32_32x32x16_f16 %0, %2, %4, %0"
        : "=&v"(nx)
        : "v"(k0), "v"(k1), "v"(q0), "v"(q1));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int v = 0; v < 16; v++) cu[v] = __builtin_amdgcn_exp2f(cu[v]);
    bf16x8 p0, p1;
#pragma unroll
    for (int e = 0; e < 8; e++) {
      p0[e] = (__bf16)cu[e];
      p1[e] = (__bf16)cu[8 + e];
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (AGPR) {
      asm volatile(
          "s_nop 1\n\t"
          "v_mfma_f32_32x32x16_bf16 %0, %2, %4, %0\n\t"
          "v_mfma_f32_16x16x32_bf16 %1, %2, %6, %1\n\t"
          "v_mfma_f32_32x32x16_bf16 %0, %3, %5, %0\n\t"
          "v_mfma_f32_16x16x32_bf16 %1, %3, %6, %1"
          : "+a"(zw), "+a"(ls)
          : "v"(p0), "v"(p1), "v"(v0), "v"(v1), "v"(sel));
    } else if constexpr (SUM == kSumMfma) {
      asm volatile(
          "s_nop 1\n\t"
          "v_mfma_f32_32x32x16_bf16 %0, %2, %4, %0\n\t"
          "v_mfma_f32_16x16x32_bf16 %1, %2, %6, %1\n\t"
          "v_mfma_f32_32x32x16_bf16 %0, %3, %5, %0\n\t"
          "v_mfma_f32_16x16x32_bf16 %1, %3, %6, %1"
          : "+v"(zw), "+v"(ls)
          : "v"(p0), "v"(p1), "v"(v0), "v"(v1), "v"(sel));
    } else {
      asm volatile(
          "s_nop 1\n\t"
          "v_mfma_f32_32x32x16_bf16 %0, %1, %3, %0\n\t"
          "v_mfma_f32_32x32x16_bf16 %0, %2, %4, %0"
          : "+v"(zw)
          : "v"(p0), "v"(p1), "v"(v0), "v"(v1));
      if constexpr (SUM == kSumDot2) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int i = 0; i < 4; i++) {
          lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p0[2 * i], p0[2 * i + 1]}, one, lsum, false);
          lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p1[2 * i], p1[2 * i + 1]}, one, lsum, false);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // Two tiles per iteration, so the score buffers alternate without copies; 8 tiles per stage.
  for (int it = 0; it < iters; it += 2) {
    tile(sa, sb, it & 7);
    tile(sb, sa, (it + 1) & 7);
    if constexpr (SYNC) {
      if ((it & 7) == 6) __syncthreads();
    }
  }
  float r = ls[0] + ls[1] + ls[2] + ls[3] + lsum;
#pragma unroll
  for (int v = 0; v < 16; v++) r += zw[v] + sa[v];
  out[lane_id] = r;
}

template <int KIND>
__global__ __launch_bounds__(256) void compute_kernel(float* out, int iters, float seed) {
  const int lane_id = threadIdx.x + blockIdx.x * blockDim.x;
  float x[kChains], y[kChains];
#pragma unroll
  for (int i = 0; i < kChains; i++) {
    x[i] = seed * (float)(i + 1) + (float)(lane_id & 7) * 1e-3f;
    y[i] = 1.0f + 1e-3f * (float)i;
  }
  f32x16 acc[4];
  bf16x8 a = {}, b = {};
  if constexpr ((KIND >= kMfma && KIND <= kMfmaExpFma) || KIND == kMfmaRand) {
#pragma unroll
    for (int e = 0; e < 8; e++) {
      a[e] = (__bf16)(KIND == kMfmaRand ? hash_unit(lane_id * 16 + e) : seed + 0.01f * e);
      b[e] = (__bf16)(KIND == kMfmaRand ? hash_unit(lane_id * 16 + e + 8) : seed - 0.01f * e);
    }
#pragma unroll
    for (int j = 0; j < 4; j++) acc[j] = f32x16{};
  }
  for (int it = 0; it < iters; it++) {
    if constexpr ((KIND >= kMfma && KIND <= kMfmaExpFma) || KIND == kMfmaRand) {
#pragma unroll
      for (int j = 0; j < 4; j++) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    // x <- 2^(-x) converges to a fixed point near 0.64, so the exponentials stay finite.
    if constexpr (KIND == kExp || KIND == kExpFma) {
#pragma unroll
      for (int i = 0; i < kChains; i++) x[i] = __builtin_amdgcn_exp2f(-x[i]);
    }
    if constexpr (KIND == kMfmaExp || KIND == kMfmaExpFma) {
#pragma unroll
      for (int r = 0; r < 2; r++)
#pragma unroll
        for (int i = 0; i < kChains; i++) x[i] = __builtin_amdgcn_exp2f(-x[i]);
    }
    if constexpr (KIND == kExpF16) {
#pragma unroll
      for (int i = 0; i < kChains; i++) x[i] = (float)__builtin_exp2f16(-(_Float16)x[i]);
    }
    if constexpr (KIND == kFma || KIND == kExpFma) {
#pragma unroll
      for (int i = 0; i < kChains; i++) y[i] = __builtin_fmaf(y[i], 0.999f, 1e-3f);
    }
    if constexpr (KIND == kMfmaFma) {
#pragma unroll
      for (int r = 0; r < 4; r++)
#pragma unroll
        for (int i = 0; i < kChains; i++) y[i] = __builtin_fmaf(y[i], 0.999f, 1e-3f);
    }
    if constexpr (KIND == kMfmaExpFma) {
#pragma unroll
      for (int r = 0; r < 2; r++)
#pragma unroll
        for (int i = 0; i < kChains; i++) y[i] = __builtin_fmaf(y[i], 0.999f, 1e-3f);
    }
  }
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < kChains; i++) r += x[i] + y[i];
  if constexpr ((KIND >= kMfma && KIND <= kMfmaExpFma) || KIND == kMfmaRand) {
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int v = 0; v < 16; v++) r += acc[j][v];
  }
  out[lane_id] = r;
}

// Read `n16` 16-byte chunks and write them to `dst` (a device copy through the vector units),
// grid-strided; or read only (dst null) and fold them into one value per lane.
__global__ __launch_bounds__(256) void stream_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                     int64_t n16, float* out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t fold = 0;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    if (dst) {
      dst[i] = a;
      dst[i + stride] = b;
      dst[i + 2 * stride] = c;
      dst[i + 3 * stride] = d;
    } else {
      fold ^= a.x ^ b.y ^ c.z ^ d.w;
    }
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    if (dst) dst[i] = a; else fold ^= a.x;
  }
  if (!dst) out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = (float)fold;
}

// Each 16-byte chunk i of `src` (or, with src null, a value made from i) written to `copies`
// destinations dst + j n16: the traffic mix of a kernel that reads one tensor and writes several.
__global__ __launch_bounds__(256) void fan_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                  int64_t n16, int copies) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int64_t k = i + u * stride;
      v[u] = src ? src[k] : make_uint4((uint32_t)k, (uint32_t)(k >> 32), 1u, 2u);
    }
    for (int j = 0; j < copies; j++) {
#pragma unroll
      for (int u = 0; u < 4; u++) dst[i + u * stride + j * n16] = v[u];
    }
  }
  for (; i < n16; i += stride) {
    const uint4 v = src ? src[i] : make_uint4((uint32_t)i, (uint32_t)(i >> 32), 1u, 2u);
    for (int j = 0; j < copies; j++) dst[i + j * n16] = v;
  }
}

template <int KIND>
hipError_t launch_compute(int grid, float* out, int iters, hipStream_t st) {
  hipLaunchKernelGGL(compute_kernel<KIND>, dim3(grid), dim3(256), 0, st, out, iters, 0.5f);
  return hipGetLastError();
}

hipError_t launch_kind(int kind, int grid, float* out, int iters, hipStream_t st) {
  switch (kind) {
    case kExp: return launch_compute<kExp>(grid, out, iters, st);
    case kFma: return launch_compute<kFma>(grid, out, iters, st);
    case kExpFma: return launch_compute<kExpFma>(grid, out, iters, st);
    case kMfma: return launch_compute<kMfma>(grid, out, iters, st);
    case kMfmaFma: return launch_compute<kMfmaFma>(grid, out, iters, st);
    case kMfmaExp: return launch_compute<kMfmaExp>(grid, out, iters, st);
    case kMfmaExpFma: return launch_compute<kMfmaExpFma>(grid, out, iters, st);
    case kTile:
      hipLaunchKernelGGL((tile_kernel<false, false, 4, false>), dim3(grid), dim3(256), 0, st, out, iters, 0.5f);
      return hipGetLastError();
    case kTileAgpr:
      hipLaunchKernelGGL((tile_kernel<true, false, 4, false>), dim3(grid), dim3(256), 0, st, out, iters, 0.5f);
      return hipGetLastError();
    case kTileLds:
      hipLaunchKernelGGL((tile_kernel<false, true, 4, false>), dim3(grid), dim3(256), 0, st, out, iters, 0.5f);
      return hipGetLastError();
    // 16-wave workgroups: a quarter of the workgroups, the same waves per SIMD.
    case kTileWg16:
      hipLaunchKernelGGL((tile_kernel<false, true, 16, false>), dim3(grid / 4), dim3(1024), 0, st, out, iters, 0.5f);
      return hipGetLastError();
    case kTileWg16Sync:
      hipLaunchKernelGGL((tile_kernel<false, true, 16, true>), dim3(grid / 4), dim3(1024), 0, st, out, iters, 0.5f);
      return hipGetLastError();
    case kTileRand:
      hipLaunchKernelGGL((tile_kernel<false, true, 16, true, true>), dim3(grid / 4), dim3(1024), 0, st, out, iters, 0.5f);
      return hipGetLastError();
    case kExpF16: return launch_compute<kExpF16>(grid, out, iters, st);
    case kTileRandNoSum:
      hipLaunchKernelGGL((tile_kernel<false, true, 16, true, true, kSumNone>), dim3(grid / 4), dim3(1024), 0, st, out,
                         iters, 0.5f);
      return hipGetLastError();
    case kTileRandDot2:
      hipLaunchKernelGGL((tile_kernel<false, true, 16, true, true, kSumDot2>), dim3(grid / 4), dim3(1024), 0, st, out,
                         iters, 0.5f);
      return hipGetLastError();
    case kMfmaRand: return launch_compute<kMfmaRand>(grid, out, iters, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

extern "C" {

// Number of compute kinds (see the Kind list above; their names from flarepp_mb_kind_name).
int flarepp_mb_num_kinds(void) { return kNumCompute; }

const char* flarepp_mb_kind_name(int kind) {
  static const char* const names[kNumCompute] = {"exp", "fma", "exp+fma", "mfma", "mfma+fma", "mfma+exp",
                                                 "mfma+exp+fma", "tile", "tile_agpr_acc", "tile_lds", "tile_lds_wg16",
                                                 "tile_lds_wg16_sync8", "tile_lds_wg16_sync8_random", "exp_f16",
                                                 "tile_random_no_row_sums", "tile_random_dot2_row_sums",
                                                 "mfma_random"};
  return (kind >= 0 && kind < kNumCompute) ? names[kind] : nullptr;
}

// Runs compute kind `kind` with `iters` loop iterations per lane on `grid` 4-wave workgroups
// (grid = 256 CUs x 4 SIMDs x waves per SIMD / 4). `out` is a device buffer of grid * 256 floats.
// One warm-up launch, then `reps` timed launches; *ms receives the mean time per launch. Returns 0,
// or a HIP error code.
int flarepp_mb_compute(int kind, int grid, int iters, int reps, float* out, hipStream_t st, double* ms) {
  if (grid < 1 || iters < 1 || reps < 1 || !out || !ms) return (int)hipErrorInvalidValue;
  hipError_t e = launch_kind(kind, grid, out, iters, st);
  if (e != hipSuccess) return (int)e;
  hipEvent_t a, b;
  if ((e = hipEventCreate(&a)) != hipSuccess) return (int)e;
  if ((e = hipEventCreate(&b)) != hipSuccess) { (void)hipEventDestroy(a); return (int)e; }
  (void)hipEventRecord(a, st);
  for (int r = 0; r < reps && e == hipSuccess; r++) e = launch_kind(kind, grid, out, iters, st);
  (void)hipEventRecord(b, st);
  if (e == hipSuccess) e = hipEventSynchronize(b);
  float t = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&t, a, b);
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  *ms = (double)t / reps;
  return (int)e;
}

// Reads `bytes` (a multiple of 16) from `src` (null: writes only) and writes them `copies` (1-4)
// times, to dst, dst + bytes, ...; timing as flarepp_mb_compute.
int flarepp_mb_fanout(const void* src, void* dst, int64_t bytes, int copies, int grid, int reps, hipStream_t st,
                      double* ms) {
  if (!dst || bytes <= 0 || (bytes & 15) || copies < 1 || copies > 4 || grid < 1 || reps < 1 || !ms)
    return (int)hipErrorInvalidValue;
  const int64_t n16 = bytes / 16;
  const uint4* s = static_cast<const uint4*>(src);
  uint4* d = static_cast<uint4*>(dst);
  hipLaunchKernelGGL(fan_kernel, dim3(grid), dim3(256), 0, st, s, d, n16, copies);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  hipEvent_t a, b;
  if ((e = hipEventCreate(&a)) != hipSuccess) return (int)e;
  if ((e = hipEventCreate(&b)) != hipSuccess) { (void)hipEventDestroy(a); return (int)e; }
  (void)hipEventRecord(a, st);
  for (int r = 0; r < reps && e == hipSuccess; r++) {
    hipLaunchKernelGGL(fan_kernel, dim3(grid), dim3(256), 0, st, s, d, n16, copies);
    e = hipGetLastError();
  }
  (void)hipEventRecord(b, st);
  if (e == hipSuccess) e = hipEventSynchronize(b);
  float t = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&t, a, b);
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  *ms = (double)t / reps;
  return (int)e;
}

// Streams `bytes` (a multiple of 16) from `src` to `dst` (dst null: read only, `out` then takes
// grid * 256 floats) with `grid` 4-wave workgroups; timing as flarepp_mb_compute.
int flarepp_mb_stream(const void* src, void* dst, int64_t bytes, int grid, int reps, float* out, hipStream_t st,
                      double* ms) {
  if (!src || bytes <= 0 || (bytes & 15) || grid < 1 || reps < 1 || !ms || (!dst && !out))
    return (int)hipErrorInvalidValue;
  const int64_t n16 = bytes / 16;
  const uint4* s = static_cast<const uint4*>(src);
  uint4* d = static_cast<uint4*>(dst);
  hipLaunchKernelGGL(stream_kernel, dim3(grid), dim3(256), 0, st, s, d, n16, out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  hipEvent_t a, b;
  if ((e = hipEventCreate(&a)) != hipSuccess) return (int)e;
  if ((e = hipEventCreate(&b)) != hipSuccess) { (void)hipEventDestroy(a); return (int)e; }
  (void)hipEventRecord(a, st);
  for (int r = 0; r < reps && e == hipSuccess; r++) {
    hipLaunchKernelGGL(stream_kernel, dim3(grid), dim3(256), 0, st, s, d, n16, out);
    e = hipGetLastError();
  }
  (void)hipEventRecord(b, st);
  if (e == hipSuccess) e = hipEventSynchronize(b);
  float t = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&t, a, b);
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  *ms = (double)t / reps;
  return (int)e;
}

}  // extern "C"
