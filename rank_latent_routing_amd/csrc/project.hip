// Projections around the FLARE++ mixer ("FLARE++: Low-rank attention with attention-synthesized
// routing"): the synthesis keys of Section 3.2 Eq. 5, the routing keys and values before Eq. 8 with
// the learned-scale normalization N_a on the keys (Appendix C.2 lists where N_a and N0 apply), the
// head split and the output projection of Section 2, and the per-head seed normalization and gate
// logistic of Eq. 6-7.
//
// A projection is Out = X W^T with C <= 512 input channels (W in torch's Linear layout: row o holds
// output channel o). One wave owns one output group of 32 channels. The group's weight rows (32
// channels x C inputs) stay in registers for the whole kernel as the MFMA A operand; 32-token tiles
// of X, staged through LDS, are the B operand. Each B-operand read from LDS feeds one MFMA, which
// keeps the matrix unit below the LDS bandwidth's limit but above what the HBM traffic of the
// projection (X once, the outputs once) allows, so the kernel stays memory-bound. The product is the transposed tile (rows = channels,
// columns = tokens), so a lane holds 16 channels of one token: the per-head RMS of the routing keys
// is a sum over the lane's own values plus one exchange with lane + 32, and the head-split stores
// are runs of 4 channels.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "device.h"
#include "kernels.h"

namespace flarepp {
namespace {

typedef float f32x8 __attribute__((ext_vector_type(8)));

// One 32x32x16 step. bf16: one MFMA. fp32: eight 32x32x2 MFMAs; step e takes k = e from lanes 0-31
// and k = 8 + e from lanes 32-63, so both dtypes hold k = 8 (l / 32) + e in element e of lane l.
template <typename T>
struct PStep;
template <>
struct PStep<bf16> {
  using Op = bf16x8;
  __device__ static f32x16 mma(const Op& a, const Op& b, const f32x16& c) { return mfma_32x32(a, b, c); }
  __device__ static Op load(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
};
template <>
struct PStep<float> {
  using Op = f32x8;
  __device__ static f32x16 mma(const Op& a, const Op& b, const f32x16& c) {
    f32x16 r = c;
#pragma unroll
    for (int e = 0; e < 8; e++) r = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], r, 0, 0, 0);
    return r;
  }
  __device__ static Op load(const float* p) {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(p), hi = *reinterpret_cast<const f32x4*>(p + 4);
    return Op{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
};

// Four consecutive output elements from fp32 values (bf16: round to nearest even).
__device__ __forceinline__ void store4(bf16* p, const float* v) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const bf16x2 a = __builtin_convertvector((f32x2{v[0], v[1]}), bf16x2);
  const bf16x2 b = __builtin_convertvector((f32x2{v[2], v[3]}), bf16x2);
  *reinterpret_cast<bf16x4*>(p) = bf16x4{a[0], a[1], b[0], b[1]};
}
__device__ __forceinline__ void store4(float* p, const float* v) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
}

// Result row (output channel within the group) of slot v of a lane in half hh of the wave.
__device__ __forceinline__ int slot_row(int v, int hh) { return 8 * (v >> 2) + 4 * hh + (v & 3); }

// KS: k steps of 16 input channels the weight registers hold (C <= 16 KS); NW: waves per workgroup
// (8 at two waves per SIMD; 4 at one wave per SIMD, whose 512 registers hold the wider weight rows
// without spilling); FRONT: the three front-end projections (head-split outputs, N_a on the first)
// or the output projection (head-split input, row-major output).
template <typename T, int D, int KS, int NW, bool FRONT>
__global__ __launch_bounds__(NW * 64, NW / 4) void project_kernel(ProjArgs a) {
  using P = PStep<T>;
  using Op = typename P::Op;
  constexpr int NT = NW * 64;
  constexpr int TB = kProjTile;
  constexpr int CH = 16 / sizeof(T);                              // elements per 16-byte chunk
  constexpr int LQ = (KS * 16 / CH * TB + NT - 1) / NT;           // staged chunks per thread, at most
  extern __shared__ __align__(16) unsigned char smem[];
  const int C = a.C, CPR = C / CH, kc = C / 16, nch = a.nproj * C;
  T* xs = reinterpret_cast<T*>(smem);                             // two [TB][C] tiles
  float* tab = reinterpret_cast<float*>(xs + 2 * TB * C);         // biases [nch], then the key scale [D]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hh = lane >> 5, l32 = lane & 31;
  // Workgroups are dispatched round-robin over the 8 XCDs; renumber them so that consecutive logical
  // workgroups (the group blocks of one token range, which read the same X rows) share an XCD and
  // its L2. The grid is a multiple of 8.
  const int logical = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  if (logical >= a.nwg) return;  // whole workgroup, before any barrier
  const int gb = logical % a.ngb, r = logical / a.ngb;  // group block, token range
  const int b = r / a.nranges;
  const int t0 = (r % a.nranges) * a.tiles_per_wg;
  const int t1 = min(t0 + a.tiles_per_wg, a.ntiles);
  const int64_t N = a.N;

  // LDS rows: the 16-byte chunks of row `row` are permuted by an XOR with (row / rpb) mod xm, xm the
  // largest power of two (at most 16) dividing the chunks per row, so the 32 rows one B-operand read
  // touches spread over the banks and every XOR stays inside the row.
  const int xm = min(CPR & -CPR, 16), rpb = max(1, 16 / CPR);
  auto off = [&](int row, int chunk) { return row * C + ((chunk ^ ((row / rpb) & (xm - 1))) * CH); };

  for (int i = tid; i < nch; i += NT) {
    const int p = i / C;
    tab[i] = a.bias[p] ? to_f(reinterpret_cast<const T*>(a.bias[p])[i - p * C]) : 0.f;
  }
  if constexpr (FRONT)
    for (int i = tid; i < D; i += NT) tab[nch + i] = a.scale ? to_f(reinterpret_cast<const T*>(a.scale)[i]) : 1.f;

  // Weight rows of this wave's group: lane l holds output channel g0 + l % 32, inputs
  // 16 ks + 8 (l / 32) .. + 7 for every k step (zero past C and for channels past the last).
  const int g0 = 32 * (gb * NW + wave);
  Op wa[KS];
  {
    const int ch = g0 + l32;
    const bool ok = ch < nch;
    const int p = ok ? ch / C : 0;
    const T* wr = reinterpret_cast<const T*>(a.W[p]) + (int64_t)(ok ? ch - p * C : 0) * C + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
      Op w = Op{};
      if (ok && ks < kc) w = P::load(wr + 16 * ks);
      wa[ks] = w;
    }
  }

  // Staging of one token tile: chunk q of the tile goes to LDS offset lofs[i] (-1: none).
  Chunk ld[LQ];
  int lofs[LQ];
  const T* X = reinterpret_cast<const T*>(a.X);
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < LQ; i++) {
      const int q = tid + i * NT;
      Chunk v = {0u, 0u, 0u, 0u};
      int o = -1;
      if (q < TB * CPR) {
        int row, chunk;
        const T* src;
        if constexpr (FRONT) {  // X [B][N][C]: a tile is one contiguous run
          row = q / CPR;
          chunk = q - row * CPR;
          src = X + ((int64_t)b * N + (int64_t)t * TB + row) * C + chunk * CH;
        } else {  // Y [B][H][N][D]: per head, a tile is one contiguous run
          constexpr int CPH = D / CH;
          const int hd = q / (TB * CPH), rem = q - hd * (TB * CPH);
          row = rem / CPH;
          const int jd = rem - row * CPH;
          chunk = hd * CPH + jd;
          src = X + (((int64_t)b * a.H + hd) * N + (int64_t)t * TB + row) * D + jd * CH;
        }
        if ((int64_t)t * TB + row < N) v = *reinterpret_cast<const Chunk*>(src);
        o = off(row, chunk);
      }
      ld[i] = v;
      lofs[i] = o;
    }
  };
  auto store_tile = [&](T* buf) {
#pragma unroll
    for (int i = 0; i < LQ; i++)
      if (lofs[i] >= 0) *reinterpret_cast<Chunk*>(buf + lofs[i]) = ld[i];
  };

  // B operand of k step ks: token l % 32 of the tile, inputs 16 ks + 8 (l / 32) .. + 7.
  const int rsw = (l32 / rpb) & (xm - 1), rbase = l32 * C;
  auto read_b = [&](const T* buf, int ks) {
    if constexpr (sizeof(T) == 2) {
      return *reinterpret_cast<const bf16x8*>(buf + rbase + (((2 * ks + hh) ^ rsw) * CH));
    } else {
      const f32x4 lo = *reinterpret_cast<const f32x4*>(buf + rbase + (((4 * ks + 2 * hh) ^ rsw) * CH));
      const f32x4 hi = *reinterpret_cast<const f32x4*>(buf + rbase + (((4 * ks + 2 * hh + 1) ^ rsw) * CH));
      return Op{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };

  // N_a over one head's channels: the lane's values v[i0 .. i0 + nv) plus those of lane + 32; d0 is
  // the head's first channel within the group.
  auto normalize = [&](float* v, int i0, int nv, int d0) {
    float ss = 0.f;
    for (int i = i0; i < i0 + nv; i++) ss += v[i] * v[i];
    ss += shfl_xor(ss, 32);
    const float rr = rsqrtf(ss * (1.0f / D) + kRmsEps);
    for (int i = i0; i < i0 + nv; i++) v[i] *= rr * tab[nch + slot_row(i, hh) - d0];
  };

  auto epilogue = [&](int t, const f32x16& acc) {
    const int64_t n = (int64_t)t * TB + l32;
    const bool nok = n < N;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; i++) v[i] = acc[i] + tab[g0 + slot_row(i, hh)];
    if constexpr (FRONT) {
      // The group's heads: two of 16 channels (D = 16, slots 0-7 and 8-15) or one of 32.
#pragma unroll
      for (int s = 0; s < 32 / D; s++) {
        const int c0 = g0 + D * s;
        if (c0 >= nch) break;
        const int p = c0 / C, h = (c0 - p * C) / D;
        if (p == 0) normalize(v, 16 / (32 / D) * s, 16 / (32 / D), D * s);
        T* dst = reinterpret_cast<T*>(a.out[p]) + (((int64_t)b * a.H + h) * N + n) * D;
#pragma unroll
        for (int j = 4 / (32 / D) * s; j < 4 / (32 / D) * (s + 1); j++)
          if (nok) store4(dst + 8 * j + 4 * hh - D * s, v + 4 * j);
      }
    } else {
      T* dst = reinterpret_cast<T*>(a.out[0]) + ((int64_t)b * N + n) * C;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int c = g0 + 8 * j + 4 * hh;
        if (nok && c < C) store4(dst + c, v + 4 * j);
      }
    }
  };

  load_tile(t0);
  store_tile(xs);
  __syncthreads();
  for (int t = t0; t < t1; t++) {
    const int cur = (t - t0) & 1;
    const T* buf = xs + cur * TB * C;
    if (t + 1 < t1) load_tile(t + 1);
    if (g0 < nch) {  // whole wave: a group past the last channel only helps with the staging
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < KS; ks++) {
        if (ks < kc) {
          const Op xb = read_b(buf, ks);
          acc = P::mma(wa[ks], xb, acc);
          hold(acc, xb);
        }
      }
      epilogue(t, acc);
    }
    if (t + 1 < t1) store_tile(xs + (cur ^ 1) * TB * C);
    __syncthreads();
  }
}

// Synthesis seeds N_a(Qseed) (scale nq, Eq. 6) in the model dtype, and the gates g = sigmoid(gamma)
// (Eq. 7) in fp32. One thread per seed row.
template <typename T, int D>
__global__ __launch_bounds__(256) void block_params_kernel(BlockParamArgs a) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < a.H) a.g[i] = 1.0f / (1.0f + expf(-a.gamma[i]));
  if (i >= a.H * a.M) return;
  const T* q = reinterpret_cast<const T*>(a.Qseed) + (int64_t)i * D;
  const T* sc = reinterpret_cast<const T*>(a.nq);
  T* o = reinterpret_cast<T*>(a.Qs) + (int64_t)i * D;
  float x[D], ss = 0.f;
#pragma unroll
  for (int d = 0; d < D; d++) {
    x[d] = to_f(q[d]);
    ss += x[d] * x[d];
  }
  const float rr = rsqrtf(ss * (1.0f / D) + kRmsEps);
#pragma unroll
  for (int d = 0; d < D; d++) o[d] = (T)(x[d] * rr * (sc ? to_f(sc[d]) : 1.0f));
}

template <typename T, int D, bool FRONT>
hipError_t launch_project_t(const ProjArgs& a, int grid, hipStream_t st) {
  const int dtype = sizeof(T) == 2 ? 1 : 0;
  const size_t lds = proj_lds_bytes(dtype, a.C, a.nproj);
  const int C = a.C;
  auto go = [&](auto kernel, int nw) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(nw * 64), lds, st, a);
    return hipGetLastError();
  };
  if (C <= 64) return go(project_kernel<T, D, 4, 8, FRONT>, 8);
  if (C <= 128) return go(project_kernel<T, D, 8, 8, FRONT>, 8);
  if constexpr (sizeof(T) == 2) {
    if (C <= 256) return go(project_kernel<T, D, 16, 8, FRONT>, 8);
    return go(project_kernel<T, D, 32, 4, FRONT>, 4);
  } else {
    return go(project_kernel<T, D, 16, 4, FRONT>, 4);
  }
}

}  // namespace

int proj_waves(int dtype, int C) { return C <= (dtype == 1 ? 256 : 128) ? 8 : 4; }

size_t proj_lds_bytes(int dtype, int C, int nproj) {
  const size_t es = dtype == 1 ? 2 : 4;
  return 2 * (size_t)kProjTile * C * es + ((size_t)nproj * C + 32) * sizeof(float);
}

hipError_t launch_project(const ProjArgs& a, int dtype, int D, bool front, int grid, hipStream_t st) {
  if (dtype == 1) {
    if (D == 16) return front ? launch_project_t<bf16, 16, true>(a, grid, st) : launch_project_t<bf16, 16, false>(a, grid, st);
    return front ? launch_project_t<bf16, 32, true>(a, grid, st) : launch_project_t<bf16, 32, false>(a, grid, st);
  }
  if (D == 16) return front ? launch_project_t<float, 16, true>(a, grid, st) : launch_project_t<float, 16, false>(a, grid, st);
  return front ? launch_project_t<float, 32, true>(a, grid, st) : launch_project_t<float, 32, false>(a, grid, st);
}

hipError_t launch_block_params(const BlockParamArgs& a, int dtype, int D, hipStream_t st) {
  const int rows = a.H * a.M > a.H ? a.H * a.M : a.H;
  const dim3 grid((rows + 255) / 256);
  if (dtype == 1) {
    if (D == 16) hipLaunchKernelGGL((block_params_kernel<bf16, 16>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((block_params_kernel<bf16, 32>), grid, dim3(256), 0, st, a);
  } else {
    if (D == 16) hipLaunchKernelGGL((block_params_kernel<float, 16>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((block_params_kernel<float, 32>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace flarepp
