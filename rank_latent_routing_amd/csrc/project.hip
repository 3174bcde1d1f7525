// Projections around the FLARE++ mixer ("FLARE++: Low-rank attention with attention-synthesized
// routing"): the synthesis keys of Section 3.2 Eq. 5, the routing keys and values before Eq. 8 with
// the learned-scale normalization N_a on the keys (Appendix C.2 lists where N_a and N0 apply), the
// head split and the output projection of Section 3.1 ("Full self-attention"), and the per-head seed
// normalization and gate logistic of Eq. 6-7.
//
// A projection is Out = X W^T with C <= 512 input channels (W in torch's Linear layout: row o holds
// output channel o). One wave owns one output group of 32 channels. The group's weight rows (32
// channels x C inputs) stay in registers for the whole kernel as the MFMA A operand; 64-token tiles
// of X (two 32-token blocks), staged through LDS, are the B operand. Each B-operand read from LDS
// feeds one MFMA: that keeps the matrix unit below the LDS bandwidth's limit but above what the HBM
// traffic of the projection (X once, the outputs once) allows, so the kernel stays memory-bound.
// The product is the transposed tile (rows = channels, columns = tokens), so a lane holds 16
// channels of one token: the per-head RMS of the routing keys is a sum over the lane's own values
// plus one exchange with lane + 32, and the head-split stores are runs of 4 channels. The staging
// has no branches (clamped rows, a junk slot for idle threads), so the compiler's memory-counter
// waits follow the data instead of draining all outstanding stores each tile.
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

// KS: k steps of 16 input channels the weight registers hold (C <= 16 KS); NW: waves per workgroup;
// WPE: waves per SIMD the register budget allows (2: 256 registers; 1: 512, which hold the widest
// weight rows without spilling); FRONT: the three front-end projections (head-split outputs, N_a on
// the first) or the output projection (head-split input, row-major output).
template <typename T, int D, int KS, int NW, int WPE, bool FRONT>
__global__ __launch_bounds__(NW * 64, WPE) void project_kernel(ProjArgs a) {
  using P = PStep<T>;
  using Op = typename P::Op;
  constexpr int NT = NW * 64;
  constexpr int TB = kProjTile;
  constexpr int NB = TB / 32;                                     // 32-token blocks per tile
  constexpr int CH = 16 / sizeof(T);                              // elements per 16-byte chunk
  constexpr int LQ = (KS * 16 / CH * TB + NT - 1) / NT;           // staged chunks per thread, at most
  extern __shared__ __align__(16) unsigned char smem[];
  const int C = a.C, CPR = C / CH, kc = C / 16, nch = a.nproj * C;
  const int BUF = TB * C + CH;                                    // a [TB][C] tile and a junk chunk
  T* xs = reinterpret_cast<T*>(smem);                             // two buffers
  float* tab = reinterpret_cast<float*>(xs + 2 * BUF);            // biases [nch], then the key scale [D]

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so group indices are scalar
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
  // 16 ks + 8 (l / 32) .. + 7 for every k step; zero past C and for channels past the last, so the
  // padded k steps (ks >= C / 16) add nothing. Every lane loads an existing row (selects, no branches).
  const int g0 = 32 * (gb * NW + wave);
  Op wa[KS];
  {
    const int ch = g0 + l32;
    const bool ok = ch < nch;
    const int p = ok ? ch / C : 0;
    const void* wp = p == 0 ? a.W[0] : (p == 1 ? a.W[1] : a.W[2]);
    const T* wr = reinterpret_cast<const T*>(wp) + (int64_t)(ok ? ch - p * C : 0) * C + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
      const Op w = P::load(wr + 16 * min(ks, kc - 1));
      wa[ks] = (ok && ks < kc) ? w : Op{};
    }
  }

  // Staging of one token tile. Thread chunk i covers chunk q = tid + i NT of the tile (row, 16-byte
  // chunk); its global pointer for tile t0 and its LDS offset are fixed for the whole kernel, and a
  // tile further on is a uniform step of TB rows. Threads past the tile's chunks load row 0's first
  // chunk and write it to the junk chunk. Rows past N (only in a last, partial tile) are read clamped
  // to row N - 1: an output token depends on its own row only, and tokens past N are never stored.
  constexpr int RS = FRONT ? 0 : 1;  // row stride selector: X rows hold C elements, Y rows D
  const int64_t rstride = RS ? D : C;
  const T* src0[LQ];
  int lofs[LQ], lrow[LQ];
  {
    const T* X = reinterpret_cast<const T*>(a.X);
#pragma unroll
    for (int i = 0; i < LQ; i++) {
      const int q0 = tid + i * NT;
      const bool qok = q0 < TB * CPR;
      const int q = qok ? q0 : 0;
      int row, chunk;
      if constexpr (FRONT) {  // X [B][N][C]: a tile is one contiguous run
        row = q / CPR;
        chunk = q - row * CPR;
        src0[i] = X + ((int64_t)b * N + (int64_t)t0 * TB + row) * C + chunk * CH;
      } else {  // Y [B][H][N][D]: per head, a tile is one contiguous run
        constexpr int CPH = D / CH;
        const int hd = q / (TB * CPH), rem = q - hd * (TB * CPH);
        row = rem / CPH;
        const int jd = rem - row * CPH;
        chunk = hd * CPH + jd;
        src0[i] = X + (((int64_t)b * a.H + hd) * N + (int64_t)t0 * TB + row) * D + jd * CH;
      }
      lofs[i] = qok ? off(row, chunk) : TB * C;
      lrow[i] = row;
    }
  }
  Chunk ld[LQ];
  auto load_tile = [&](int t) {
    const int64_t step = (int64_t)(t - t0) * TB * rstride;
    const int64_t left = N - (int64_t)t * TB;  // rows of this tile that exist
    if (left >= TB) {
#pragma unroll
      for (int i = 0; i < LQ; i++) ld[i] = *reinterpret_cast<const Chunk*>(src0[i] + step);
    } else {
#pragma unroll
      for (int i = 0; i < LQ; i++) {
        const int back = max(lrow[i] - (int)(left - 1), 0);
        ld[i] = *reinterpret_cast<const Chunk*>(src0[i] + step - back * rstride);
      }
    }
  };
  auto store_tile = [&](T* buf) {
#pragma unroll
    for (int i = 0; i < LQ; i++) *reinterpret_cast<Chunk*>(buf + lofs[i]) = ld[i];
  };

  // B operand of k step ks of token block tb: token 32 tb + l % 32 of the tile, inputs
  // 16 ks + 8 (l / 32) .. + 7. Padded k steps re-read the last real one (their weights are zero).
  // The swizzle's XOR term is the same for rows r and r + 32 (32 / rpb is a multiple of xm).
  const int rsw = (l32 / rpb) & (xm - 1), rbase = l32 * C;
  auto read_b = [&](const T* buf, int ks0, int tb) {
    const int ks = min(ks0, kc - 1);
    const T* row = buf + rbase + tb * 32 * C;
    if constexpr (sizeof(T) == 2) {
      return *reinterpret_cast<const bf16x8*>(row + (((2 * ks + hh) ^ rsw) * CH));
    } else {
      const f32x4 lo = *reinterpret_cast<const f32x4*>(row + (((4 * ks + 2 * hh) ^ rsw) * CH));
      const f32x4 hi = *reinterpret_cast<const f32x4*>(row + (((4 * ks + 2 * hh + 1) ^ rsw) * CH));
      return Op{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };

  // Output. The result tile of a token block (32 tokens x the group's 32 channels) goes through a
  // per-wave LDS area (rows of 32 channels plus 16 bytes of padding against bank conflicts) and
  // leaves in 16-byte chunks in destination order: per head, the 32 token rows of D channels are one
  // contiguous run of the head-split output (front end); for the output projection each token's 32
  // channels are one run of its row. Chunk k = lane + 64 u of a lane has a fixed LDS offset, token
  // and destination offset; its head (front end) is 64 u / (chunks per head), the same for all lanes
  // since a head's chunks are a multiple of 64.
  constexpr int NH = FRONT ? 32 / D : 1;                          // heads per group
  constexpr int RSE = 32 + CH;                                    // LDS row stride, elements
  constexpr int NU = 32 * 32 / CH / 64;                           // chunks per lane
  T* ep = reinterpret_cast<T*>(tab + nch + 32) + wave * 32 * RSE;
  int ck_lds[NU], ck_tok[NU], ck_dst[NU];
  bool ck_ok[NU];
#pragma unroll
  for (int u = 0; u < NU; u++) {
    const int k = lane + 64 * u;
    if constexpr (FRONT) {
      constexpr int PH = 32 * D / CH;  // chunks per head
      const int sh = k / PH, rem = k - sh * PH, tok = rem / (D / CH), w = rem - tok * (D / CH);
      ck_tok[u] = tok;
      ck_lds[u] = tok * RSE + sh * D + w * CH;
      ck_dst[u] = tok * D + w * CH;
      ck_ok[u] = g0 + D * sh < nch;
    } else {
      const int tok = k / (32 / CH), cc = k - tok * (32 / CH);
      ck_tok[u] = tok;
      ck_lds[u] = tok * RSE + cc * CH;
      ck_dst[u] = tok * C + cc * CH;
      ck_ok[u] = g0 + cc * CH < C;
    }
  }
  // Per head of the group: output tensor, head index and whether it carries N_a (front end).
  T* hbase[NH];
  bool norm[NH], hok[NH];
#pragma unroll
  for (int sh = 0; sh < NH; sh++) {
    if constexpr (FRONT) {
      const int c0 = g0 + D * sh;
      hok[sh] = c0 < nch;
      const int pp = hok[sh] ? c0 / C : 0, h = hok[sh] ? (c0 - pp * C) / D : 0;
      norm[sh] = pp == 0;
      void* op = pp == 0 ? a.out[0] : (pp == 1 ? a.out[1] : a.out[2]);
      hbase[sh] = reinterpret_cast<T*>(op) + ((int64_t)b * a.H + h) * N * D;
    } else {
      hok[sh] = true;
      norm[sh] = false;
      hbase[sh] = reinterpret_cast<T*>(a.out[0]) + (int64_t)b * N * C + g0;
    }
  }
  const int64_t ostride = FRONT ? D : C;  // elements per token row of the output

  // N_a over one head's channels: the lane's values v[i0 .. i0 + nv) plus those of lane + 32; d0 is
  // the head's first channel within the group. The argument of the reciprocal square root is at
  // least the epsilon, so the hardware instruction needs no range handling.
  auto normalize = [&](float* v, int i0, int nv, int d0) {
    float ss = 0.f;
    for (int i = i0; i < i0 + nv; i++) ss += v[i] * v[i];
    ss += shfl_xor(ss, 32);
    const float rr = __builtin_amdgcn_rsqf(ss * (1.0f / D) + kRmsEps);
    for (int i = i0; i < i0 + nv; i++) v[i] *= rr * tab[nch + slot_row(i, hh) - d0];
  };

  auto epilogue = [&](int t, int tb, const f32x16& acc) {
    const int64_t n0 = (int64_t)t * TB + 32 * tb;  // first token of the block
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; i++) v[i] = acc[i];
#pragma unroll
    for (int sh = 0; sh < NH; sh++) {
      constexpr int NV = 16 / NH;  // slots per head
      if (hok[sh] && norm[sh]) normalize(v, NV * sh, NV, D * sh);
    }
    // Slots 4j .. 4j + 3 of the lane are channels 8j + 4 (l / 32) .. + 3 of token l % 32.
#pragma unroll
    for (int j = 0; j < 4; j++) store4(ep + l32 * RSE + 8 * j + 4 * hh, v + 4 * j);
#pragma unroll
    for (int u = 0; u < NU; u++) {
      constexpr int PH = FRONT ? 32 * D / CH : 64 * NU;  // chunks per head
      const Chunk c = *reinterpret_cast<const Chunk*>(ep + ck_lds[u]);
      if (ck_ok[u] && n0 + ck_tok[u] < N)
        *reinterpret_cast<Chunk*>(hbase[64 * u / PH] + n0 * ostride + ck_dst[u]) = c;
    }
  };

  __syncthreads();  // the bias and scale table
  // The group's biases as the accumulator's starting value: slot i of the lane is channel
  // g0 + slot_row(i, l / 32).
  f32x16 bias;
#pragma unroll
  for (int i = 0; i < 16; i++) bias[i] = tab[g0 + slot_row(i, hh)];

  load_tile(t0);
  store_tile(xs);
  __syncthreads();
  for (int t = t0; t < t1; t++) {
    const int cur = (t - t0) & 1;
    const T* buf = xs + cur * BUF;
    if (t + 1 < t1) load_tile(t + 1);
    const bool active = g0 < nch;  // whole wave: a group past the last channel only helps with the staging
    f32x16 acc[NB];
    if (active) {
      // LDS reads run PD k steps ahead of the MFMAs that use them (hold() orders the instruction
      // stream as written, so the distance is set here, not by the scheduler).
      constexpr int PD = sizeof(T) == 2 ? 4 : 2;
      Op xr[KS][NB];
#pragma unroll
      for (int ks = 0; ks < PD && ks < KS; ks++)
#pragma unroll
        for (int tb = 0; tb < NB; tb++) xr[ks][tb] = read_b(buf, ks, tb);
#pragma unroll
      for (int ks = 0; ks < KS; ks++) {
        if (ks + PD < KS) {
#pragma unroll
          for (int tb = 0; tb < NB; tb++) xr[ks + PD][tb] = read_b(buf, ks + PD, tb);
        }
#pragma unroll
        for (int tb = 0; tb < NB; tb++) {
          acc[tb] = P::mma(wa[ks], xr[ks][tb], ks == 0 ? bias : acc[tb]);
          hold(acc[tb], xr[ks][tb]);
        }
      }
    }
    // The next tile goes to LDS before this tile's results go out, so that waiting for its loads
    // does not also wait for those stores.
    if (t + 1 < t1) store_tile(xs + (cur ^ 1) * BUF);
    if (active) {
#pragma unroll
      for (int tb = 0; tb < NB; tb++) epilogue(t, tb, acc[tb]);
    }
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
  if (C <= 64) return go(project_kernel<T, D, 4, 8, 2, FRONT>, 8);
  if (C <= 128) return go(project_kernel<T, D, 8, 8, 2, FRONT>, 8);
  if constexpr (sizeof(T) == 2) {
    if (C <= 256) return go(project_kernel<T, D, 16, 8, 2, FRONT>, 8);
    return go(project_kernel<T, D, 32, 4, 1, FRONT>, 4);
  } else {
    return go(project_kernel<T, D, 16, 4, 1, FRONT>, 4);
  }
}

}  // namespace

int proj_waves(int dtype, int C) { return C <= (dtype == 1 ? 256 : 128) ? 8 : 4; }

size_t proj_lds_bytes(int dtype, int C, int nproj) {
  const size_t es = dtype == 1 ? 2 : 4;
  // Two staging buffers with their junk chunks, the bias and scale table, and each wave's output
  // transposition area (32 rows of 32 channels plus 16 bytes).
  return 2 * ((size_t)kProjTile * C * es + 16) + ((size_t)nproj * C + 32) * sizeof(float) +
         (size_t)proj_waves(dtype, C) * 32 * (32 * es + 16);
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
