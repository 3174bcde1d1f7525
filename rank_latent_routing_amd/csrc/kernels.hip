// HIP kernels of the FLARE++ mixer forward pass for gfx950 (CDNA4).
//
// Method: "FLARE++: Low-rank attention with attention-synthesized routing" (arXiv 2608.11519 v2),
// Section 3.2 Eq. 5-8 (one block: Appendix A.1 Eq. 11). Three softmax routing calls per
// (batch, head): synthesis and encode normalize over the N tokens, decode over the M latents.
//
// Kernel plan (one launch each, in stream order):
//   partial<SYNTH>  split-N online-softmax partials of the synthesis call; the RMS normalization
//                   of S is fused into the tile load and S serves as both keys and values.
//   merge_gate      log-sum-exp merge of the chunk partials (Appendix B.3 Eq. 29-33, chunks in the
//                   role of the pages' ranks) then Q = N0(Qf) + g Qd in fp32 (Eq. 7).
//   partial<ENC>    the same engine for the encode call, keys K, values V.
//   merge           log-sum-exp merge -> Z.
//   decode          Q and Z resident in LDS; every token's scores against all M latents, softmax
//                   over M, product with Z.
//
// Numerics. Every logit is computed directly in log2 units: the query operand of each call
// carries the factor c = log2(e)/sqrt(D) (folded into the normalized synthesis keys, and into Q
// when merge_gate casts it), so one v_exp_f32 per score evaluates exp(q.k/sqrt(D)). A softmax is
// invariant to the shift subtracted from its logits (Appendix B.3 Eq. 29). The kernels first use
// shift 0, which needs no running maximum, and check afterwards that it was exact: every row sum
// in [2^-80, 2^100] and finite accumulators mean no exponential overflowed and no term within
// 2^-24 of a row's largest was lost to underflow. Rows of a chunk (partials) or of a token group
// (decode) that fail are recomputed with exact running maxima (online softmax over token stages,
// or a two-pass maximum over the M latents).
//
// Routing queries in bf16 runs are carried as a pair hi + lo of bf16 values (hi = bf16(c q),
// lo = bf16(c q - hi)) and every score is the sum of two chained MFMAs, so the queries keep about
// 16 significant bits in the logits; the keys, values and probabilities are bf16 operands with fp32
// accumulation.
//
// MFMA layouts (checked on gfx950): for v_mfma_f32_16x16x{32,16}_bf16 and 16x16x4_f32, lane l
// supplies row (l % 16) of A and column (l % 16) of B with the k-slice selected by g = l / 16, and
// receives column (l % 16), rows 4g..4g+3 of the 16x16 result. Score tiles are computed with the
// keys as A so that the result lands with one latent per lane column and eight consecutive tokens
// per lane, which is exactly the A (or B) operand layout of the following P.V product: the
// probabilities never leave registers. The P.V operand that runs along tokens (values) or latents
// (Z) is read from a row-major LDS tile with ds_read_b64_tr_b16, whose 16-lane groups return
// lane i, element j = element (i mod 4) of the 8 bytes addressed by group lane 4j + i/4.
#include <hip/hip_runtime.h>
#include <cstdint>
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace flarepp {
namespace {

// v on lanes l and l ^ 32 combined, on every lane, through one swap of the wave's halves
// (v_permlane32_swap: the first result holds lanes 0-31 of v in both halves, the second lanes
// 32-63): no LDS permute and no lane-index arithmetic. Sums and maxima are commutative, so every
// lane gets exactly v_l + v_(l^32) (or the max), as a shfl_xor by 32 would give. The swap reads the
// partner lane whether or not it is active, so callers run it with all 64 lanes active (every use
// sits in wave-uniform control flow).
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// x0 - hi0 and x1 - hi1, where hp holds hi0 (low half) and hi1 (high half), the bf16 roundings of
// x0 and x1: one bf16 dot product per value (x + hi * -1 + other * 0), exact as x - hi is a float.
// The selectors (-1, 0) and (0, -1) sit in registers as literals: an inline-constant encoding of a
// packed bf16 operand need not place the value in the half the vector names.
typedef float residual2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t literal_u32(uint32_t v) {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
  return r;
}
__device__ __forceinline__ residual2_t bf16_residual2(uint32_t hp, float x0, float x1) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const b2 h = __builtin_bit_cast(b2, hp);
  const b2 m0 = __builtin_bit_cast(b2, literal_u32(0x0000bf80u));  // element 0: -1, element 1: 0
  const b2 m1 = __builtin_bit_cast(b2, literal_u32(0xbf800000u));  // element 0: 0, element 1: -1
  return residual2_t{__builtin_amdgcn_fdot2_f32_bf16(h, m0, x0, false),
                     __builtin_amdgcn_fdot2_f32_bf16(h, m1, x1, false)};
}

// A priori bounds on the logits (log2 units) of the zero-shift passes with fp16 score operands. The
// fp16 rounding of a computed score operand (the synthesis keys c N0(s), the routing queries c Q)
// moves a logit by at most 2^-11 of the bound, and the output's sensitivity to that error grows
// with the keys' and seeds' scales, so larger bounds take the exact passes, whose logits are
// exact up to fp32 accumulation. Synthesis: ||Qseed_m|| log2(e) (the keys have unit RMS); the
// benchmark workloads reach about 12. Encode and decode: ||c Q_m|| ||K_n||; the workloads reach
// about 14 (39 with the keys scaled by 4).
constexpr float kFastBound = 24.0f;
constexpr float kRouteBound = 20.0f;

__device__ __forceinline__ float sumsq_bf16x8(bf16x8 x) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const bf16x2 p = {x[2 * i], x[2 * i + 1]};
    s = __builtin_amdgcn_fdot2_f32_bf16(p, p, s, false);
  }
  return s;
}
// Maximum over the wave with DPP moves within each row of 16 lanes and reads of the four rows'
// results: no lane-address registers (which the compiler would otherwise keep live across the
// partial kernel's stage loop, between a reduction before it and one after it).
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_move<0xB1>(v));   // lane ^ 1
  v = fmaxf(v, dpp_move<0x4E>(v));   // lane ^ 2
  v = fmaxf(v, dpp_move<0x141>(v));  // the other quad of 8 lanes
  v = fmaxf(v, dpp_move<0x140>(v));  // the other half of 16 lanes
  const auto rd = [&](int l) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l)); };
  return fmaxf(fmaxf(rd(0), rd(16)), fmaxf(rd(32), rd(48)));
}

// The 16-bit operand of a P.V MFMA read as fp16 (the tile holds fp16 values); unused for fp32 tiles.
template <typename OctT>
__device__ __forceinline__ f16x8 as_f16x8(const OctT& o) {
  if constexpr (sizeof(OctT) == sizeof(f16x8)) return __builtin_bit_cast(f16x8, o);
  else return f16x8{};
}

__device__ __forceinline__ float sumsq_f16x8(f16x8 x) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const f16x2 p = {x[2 * i], x[2 * i + 1]};
    s = __builtin_amdgcn_fdot2(p, p, s, false);
  }
  return s;
}

// ------------------------------------------------------------------------------------------
// Per-dtype operand helpers. A "slice" is the D/4 consecutive elements of a row that one lane
// feeds to the score MFMA (k = g*D/4 ... g*D/4 + D/4 - 1). An "oct" is the 8 consecutive tokens
// (or latents) one lane feeds to the P.V MFMA.
template <typename T, int D>
struct Ops;

struct OpsBf16Common {
  using Oct = bf16x8;
  __device__ static Oct pack(f32x4 lo, f32x4 hi) {
    Oct r;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      r[i] = (bf16)lo[i];
      r[4 + i] = (bf16)hi[i];
    }
    return r;
  }
  // Sum of the eight (rounded) probabilities, two per v_dot2.
  __device__ static float osum(Oct p, float acc) {
    const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      bf16x2 q = {p[2 * i], p[2 * i + 1]};
      acc = __builtin_amdgcn_fdot2_f32_bf16(q, one, acc, false);
    }
    return acc;
  }
  __device__ static f32x4 pv(Oct a, Oct b, f32x4 c) { return mfma_32k(a, b, c); }
  // Oct of a row-major LDS tile along its rows: rows r0 + 8g .. r0 + 8g + 7 of column col0 + c
  // for lane (c, g), read with two transposed loads (rows r0 + 8g + 4h + j for h = 0, 1).
  __device__ static Oct load_oct_rows(const bf16* tile, int stride, int r0, int col0, int c, int g) {
    const bf16* p = tile + (r0 + 8 * g + (c >> 2)) * stride + col0 + 4 * (c & 3);
    const bf16x4 lo = lds_read_tr4(p);
    const bf16x4 hi = lds_read_tr4(p + 4 * stride);
    Oct o;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      o[i] = lo[i];
      o[4 + i] = hi[i];
    }
    return o;
  }
};

// B operand of a 32x32x16 P.V MFMA from a row-major bf16 LDS tile whose rows run along k: lane l
// (dims 16 cb + i, cb = (l / 16) % 2, i = l % 16, half h = l / 32) receives rows
// r0 + row32(e, h) (e = 0..7) of column col0 + 16 cb + i, read with two transposed loads.
__device__ __forceinline__ bf16x8 load_rows32(const bf16* tile, int stride, int r0, int col0, int lane) {
  const int i = lane & 15, cb = (lane >> 4) & 1, h = lane >> 5;
  const bf16* p = tile + (r0 + 4 * h + (i >> 2)) * stride + col0 + 16 * cb + 4 * (i & 3);
  const bf16x4 lo = lds_read_tr4(p);
  const bf16x4 hi = lds_read_tr4(p + 8 * stride);
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 4; e++) {
    o[e] = lo[e];
    o[4 + e] = hi[e];
  }
  return o;
}
// Eight consecutive slots (8 t .. 8 t + 7) of a 32x32 result as the bf16 A operand of the next
// 32x32x16 MFMA (k = rows 16 t .. 16 t + 15 of the result).
__device__ __forceinline__ bf16x8 pack32(const f32x16& x, int t) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; e++) r[e] = (bf16)x[8 * t + e];
  return r;
}

template <>
struct Ops<bf16, 32> : OpsBf16Common {
  using Slice = bf16x8;
  __device__ static Slice zero_slice() { return Slice{}; }
  __device__ static Slice load_slice(const bf16* row, int g) { return *reinterpret_cast<const bf16x8*>(row + 8 * g); }
  __device__ static f32x4 qk(Slice a, Slice b, f32x4 c) { return mfma_32k(a, b, c); }
  __device__ static float sumsq(Slice a) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) s += (float)a[i] * (float)a[i];
    return s;
  }
};

template <>
struct Ops<bf16, 16> : OpsBf16Common {
  using Slice = bf16x4;
  __device__ static Slice zero_slice() { return Slice{}; }
  __device__ static Slice load_slice(const bf16* row, int g) { return *reinterpret_cast<const bf16x4*>(row + 4 * g); }
  __device__ static f32x4 qk(Slice a, Slice b, f32x4 c) { return mfma_16k(a, b, c); }
  __device__ static float sumsq(Slice a) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) s += (float)a[i] * (float)a[i];
    return s;
  }
};

template <int D>
struct Ops<float, D> {
  struct Slice {
    float v[D / 4];
  };
  struct Oct {
    float v[8];
  };
  __device__ static Slice zero_slice() {
    Slice s;
#pragma unroll
    for (int i = 0; i < D / 4; i++) s.v[i] = 0.f;
    return s;
  }
  __device__ static Slice load_slice(const float* row, int g) {
    Slice s;
    const f32x4* p = reinterpret_cast<const f32x4*>(row + (D / 4) * g);
#pragma unroll
    for (int i = 0; i < D / 16; i++) {
      f32x4 t = p[i];
#pragma unroll
      for (int j = 0; j < 4; j++) s.v[4 * i + j] = t[j];
    }
    return s;
  }
  __device__ static f32x4 qk(const Slice& a, const Slice& b, f32x4 c) {
#pragma unroll
    for (int s = 0; s < D / 4; s++) c = mfma_4k(a.v[s], b.v[s], c);
    return c;
  }
  __device__ static float sumsq(const Slice& a) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < D / 4; i++) s += a.v[i] * a.v[i];
    return s;
  }
  __device__ static Oct pack(f32x4 lo, f32x4 hi) {
    Oct r;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      r.v[i] = lo[i];
      r.v[4 + i] = hi[i];
    }
    return r;
  }
  __device__ static float osum(const Oct& p, float acc) {
#pragma unroll
    for (int i = 0; i < 8; i++) acc += p.v[i];
    return acc;
  }
  __device__ static f32x4 pv(const Oct& a, const Oct& b, f32x4 c) {
#pragma unroll
    for (int j = 0; j < 8; j++) c = mfma_4k(a.v[j], b.v[j], c);
    return c;
  }
  // fp32 tiles read along their rows are stored transposed: a stored row is a source column.
  __device__ static Oct load_oct_rows(const float* tile_t, int stride, int r0, int col0, int c, int g) {
    const f32x4* q = reinterpret_cast<const f32x4*>(tile_t + (col0 + c) * stride + r0 + 8 * g);
    const f32x4 a = q[0], b = q[1];
    Oct o;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      o.v[j] = a[j];
      o.v[4 + j] = b[j];
    }
    return o;
  }
};


// LDS layout of a tile whose rows (tokens or latents) run along the k-range of a P.V operand:
// bf16 keeps the rows (read with transposed loads), fp32 stores the transpose. gfx950's LDS serves
// 64 banks of 4 bytes per cycle, 32 lanes of a transposed 8-byte read: for D = 32 those lanes read
// rows r0..r0+3 at bytes 0-31 and 32-63 of each, which unpadded 64-byte rows spread over all 256
// bytes (SQ_LDS_BANK_CONFLICT per 32x32 tile of the partial kernels: 10 with 96-byte rows, 1 with
// these). PAD: elements added per row (the decode keeps 16, which measured faster there).
constexpr int kDecodeZPad = 16;  // decode_wide_kernel's Z rows: 96 bytes
template <typename T, int D, int PAD = (D == 32 ? 0 : 8)>
struct RowTile {
  static constexpr bool kTransposed = sizeof(T) == 4;
  static constexpr int kRowStride = D + PAD;
  __host__ __device__ static constexpr int tstride(int rows) { return rows + 4; }
  __host__ __device__ static constexpr int elems(int rows) { return kTransposed ? D * tstride(rows) : rows * kRowStride; }
  __host__ __device__ static constexpr int stride(int rows) { return kTransposed ? tstride(rows) : kRowStride; }
};


// Store one 16-byte chunk (elements col .. col + 16/sizeof(T) - 1 of row `row`) into a RowTile.
template <typename T, int D, int PAD = (D == 32 ? 0 : 8)>
__device__ __forceinline__ void rowtile_store(T* tile, int rows, int row, int col, const Chunk& ck) {
  using RT = RowTile<T, D, PAD>;
  if constexpr (RT::kTransposed) {
    float x[4];
    chunk_to_float<T>(ck, x);
#pragma unroll
    for (int j = 0; j < 4; j++) tile[(col + j) * RT::tstride(rows) + row] = (T)x[j];
  } else {
    *reinterpret_cast<Chunk*>(tile + row * RT::kRowStride + col) = ck;
  }
}


// Token order inside a 32-token subtile: score MFMA `half` row r holds token 8*(r/4)+4*half+r%4,
// so that lane group g receives tokens 8g..8g+7 across the two halves.
__device__ __forceinline__ int perm_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

// ------------------------------------------------------------------------------------------
// Split-N partial kernel (synthesis and encode).
//
// Workgroup = NW waves; wave w owns latents [lat0, lat0 + LPW) as NLB blocks of 16. The workgroup
// streams its token chunk through LDS in stages of kStage tokens (double-buffered): a row-major key
// tile (A operand of the score MFMA) and a value RowTile (B operand of the P.V MFMA). Global loads
// run two stages ahead of the compute through two register sets. For each latent row the kernel
// accumulates the shift m, the sum l of exp2(logit - m) and the P.V product.
//
// A chunk is first streamed with shift 0 (no running maximum). That is exact whenever no
// exponential overflowed and every term that matters stayed a normal float, which the kernel checks
// afterwards on every row: l in [2^-80, 2^100] and a finite accumulator. If any row of the workgroup
// fails, the whole chunk is streamed again with exact running maxima (online softmax). bf16 runs
// with D = 32 take that first pass on fp16 score operands; with `hilo` set they take it with the
// bf16 keys against the hi/lo query pair instead, the logits of the exact pass and of the
// backward kernels, so that the normalizers they leave match those logits.
//
// HILO (bf16, the backward's recompute): the P.V product and the row sums take each probability as
// a pair hi + lo (hi = bf16(p), lo = bf16(p - hi)), and the synthesis call's values N0(s) likewise
// (a second value tile holds their lo parts): P.V = Phi.Vhi + Plo.Vhi + Phi.Vlo. The backward forms
// the row terms of the encode and synthesis calls from these Z and Qd against products that take
// every operand as a pair; single-bf16 P and N0(s) would leave those terms about 2^-8 off, which
// dominates the cotangents when a softmax row spans only a few tokens.
//
// Grid: x enumerates (chunk, latent group) so that the latent groups of one chunk land on the same
// XCD (workgroups are dealt to the 8 XCDs round-robin by x) and share its L2; y = b * H + h.
template <typename T, int D, int LPW, int NW, bool SYNTH, int STG, bool HILO>
__global__ __launch_bounds__(NW * 64) void partial_kernel(PartialArgs a) {
  static_assert(!HILO || sizeof(T) == 2, "hi/lo probabilities are for bf16 operands");
  constexpr int kStage = STG;  // tokens per LDS stage
  using O = Ops<T, D>;
  using Slice = typename O::Slice;
  using Oct = typename O::Oct;
  using VT = RowTile<T, D>;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  constexpr int NLB = LPW / 16;
  constexpr int NDB = D / 16;
  constexpr int NT = NW * 64;
  constexpr int CH = 16 / sizeof(T);    // elements per 16-byte chunk
  constexpr int CPR = D / CH;           // chunks per token row
  constexpr int NCH = kStage * CPR;     // chunks per stage per tensor
  constexpr int PER = (NCH + NT - 1) / NT;
  constexpr int RS = D + CH;            // key tile row stride (elements)
  constexpr int VE = VT::elems(kStage); // value tile elements per buffer
  constexpr int VSTR = VT::stride(kStage);

  extern __shared__ __align__(16) unsigned char smem[];
  T* ks = reinterpret_cast<T*>(smem);                   // [2][kStage][RS]
  T* vt = ks + 2 * kStage * RS;                          // [2][VE]
  T* vtl = vt + 2 * VE;                                  // HILO synthesis: value lo parts, [2][VE]
  // bf16 synthesis on the 16x16x32 path: the key tile holds the raw synthesis keys s (exact bf16)
  // and this array each token's factor c / rms(s), applied to the scores in fp32 (see store_set).
  constexpr bool kFactorKeys = SYNTH && sizeof(T) == 2;
  // bf16 synthesis (not the backward's HILO instance): the exact pass takes its probabilities and
  // values N0(s) in fp16. Both fit its range there (P <= 1 under the running maximum,
  // |N0(s)| <= sqrt(D)), and fp16 keeps 11 significant bits to bf16's 8: at large seed scales the
  // routing queries, and through them the routing logits, inherit the synthesis call's rounding.
  constexpr bool kF16Exact = SYNTH && sizeof(T) == 2 && !HILO;
  float* tf = reinterpret_cast<float*>(vt + (HILO && SYNTH ? 4 : 2) * VE);  // [2][kStage]
  int* fail_s = reinterpret_cast<int*>(tf + (kFactorKeys ? 2 * kStage : 0));  // one flag
  // Encode's zero-shift pass (the routing bound of kRouteBound): each wave's largest ||c Q_m||^2, and
  // per token row of a stage the largest ||K_n||^2 staged through it (kept in LDS, so no register
  // stays live across the pass).
  float* qred = reinterpret_cast<float*>(fail_s + 4);  // [NW]
  float* knmax = qred + NW;                            // [kStage]

  // (chunk, latent group) of this workgroup.
  int chunk_id, lg;
  if (a.nlg == 1) {
    chunk_id = blockIdx.x;
    lg = 0;
  } else {
    const int slot = blockIdx.x >> 3;
    lg = slot % a.nlg;
    chunk_id = (slot / a.nlg) * 8 + (blockIdx.x & 7);
  }
  if (chunk_id >= a.nchunk) return;  // padding workgroups of the XCD mapping (whole workgroup)

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int bh = blockIdx.y;
  const int64_t n_begin = (int64_t)chunk_id * a.chunk;
  const int64_t n_end = (n_begin + a.chunk < a.N) ? n_begin + a.chunk : a.N;
  const int nstage = (int)((n_end - n_begin + kStage - 1) / kStage);
  const int lat0 = (lg * NW + wave) * LPW;
  const bool active = lat0 < a.Mp;
  if (tid == 0) *fail_s = 0;
  for (int t = tid; t < kStage; t += NT) knmax[t] = 0.f;
  __syncthreads();

  const T* kbase = reinterpret_cast<const T*>(a.K) + (int64_t)bh * a.N * D;
  const T* vbase = reinterpret_cast<const T*>(a.V) + (int64_t)bh * a.N * D;
  // Synthesis queries are the seeds (one exact part); encode queries are the workspace hi/lo pair.
  constexpr int QP = SYNTH ? 1 : kQParts<T>;
  constexpr int QRS = SYNTH ? D : kQRow<T> * D;  // query row stride (elements)
  const T* qbase = reinterpret_cast<const T*>(a.Q) + (int64_t)(SYNTH ? bh % a.H : bh) * a.Mq * QRS;

  // Query operands (B of the score MFMA): lane (c, g) holds slice g of latent lat0 + 16 lb + c.
  Slice qb[NLB], qlo[NLB];
  auto load_queries = [&]() {
#pragma unroll
    for (int lb = 0; lb < NLB; lb++) {
      const int row = lat0 + 16 * lb + c;
      qb[lb] = (row < a.Mq) ? O::load_slice(qbase + (int64_t)row * QRS, g) : O::zero_slice();
      if constexpr (QP == 2) qlo[lb] = (row < a.Mq) ? O::load_slice(qbase + (int64_t)row * QRS + D, g) : O::zero_slice();
    }
  };
  // bf16 runs with D = 32 and whole 32-latent blocks per wave take the zero-shift pass with
  // 32x32x16 MFMAs on fp16 score operands (keys and queries in fp16, one MFMA per 16 dims) and bf16
  // probabilities and values; the exact pass keeps 16x16x32 bf16 MFMAs with hi/lo queries.
  constexpr bool kWide = sizeof(T) == 2 && D == 32 && LPW % 32 == 0;
  constexpr int NB = kWide ? LPW / 32 : 1;
  const int h32 = lane >> 5;
  // Wide query operands: lane l holds dims 16 kh + 8 h .. + 7 of latent lat0 + 32 nb + l % 32
  // (encode: the fp16 part of the workspace row; synthesis: the bf16 seeds converted).
  f16x8 qw[NB][2];
  if constexpr (kWide) {
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
      const int row = lat0 + 32 * nb + (lane & 31);
#pragma unroll
      for (int kh = 0; kh < 2; kh++) {
        if (row >= a.Mq) {
          qw[nb][kh] = f16x8{};
        } else if constexpr (SYNTH) {
          qw[nb][kh] = to_f16x8(*reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16*>(qbase) +
                                                                 (int64_t)row * QRS + 16 * kh + 8 * h32));
        } else {
          qw[nb][kh] = *reinterpret_cast<const f16x8*>(reinterpret_cast<const bf16*>(qbase) + (int64_t)row * QRS +
                                                       2 * D + 16 * kh + 8 * h32);
        }
      }
    }
    if constexpr (!SYNTH) {
      // The largest ||c Q_m||^2 of this wave's latents, for the routing bound of the zero-shift
      // pass: each lane reads a whole fp16 row (no lane exchange, whose address registers the
      // compiler would keep live across the stage loop).
      float q2 = 0.f;
#pragma unroll
      for (int nb = 0; nb < NB; nb++) {
        const int row = lat0 + 32 * nb + (lane & 31);
        if (row < a.Mq) {
          const f16x8* qr = reinterpret_cast<const f16x8*>(reinterpret_cast<const bf16*>(qbase) + (int64_t)row * QRS + 2 * D);
          float ss = 0.f;
#pragma unroll
          for (int k = 0; k < D / 8; k++) ss += sumsq_f16x8(qr[k]);
          q2 = fmaxf(q2, ss);
        }
      }
      q2 = wave_max_dpp(q2);
      if (lane == 0) qred[wave] = q2;
    }
  } else {
    load_queries();
  }
  const float c_scale = kLog2e * rsqrtf((float)D);

  f32x4 zacc[NLB][NDB];
  float lsum[NLB], mrow[NLB];

  // Two register sets of loaded chunks; set P holds stages of parity P.
  Chunk kr[2][PER], vr[2][PER];
  auto load_set = [&](auto P, int stage) {
    const int64_t s0 = n_begin + (int64_t)stage * kStage;
#pragma unroll
    for (int i = 0; i < PER; i++) {
      const int q = tid + i * NT;
      Chunk ck = {0u, 0u, 0u, 0u}, cv = {0u, 0u, 0u, 0u};
      if (q < NCH) {
        const int t = q / CPR, part = q % CPR;
        const int64_t n = s0 + t;
        if (n < n_end) {
          ck = *reinterpret_cast<const Chunk*>(kbase + n * D + part * CH);
          if constexpr (!SYNTH) cv = *reinterpret_cast<const Chunk*>(vbase + n * D + part * CH);
        }
      }
      kr[decltype(P)::value][i] = ck;
      vr[decltype(P)::value][i] = cv;
    }
  };
  // Store a register set into LDS buffer `buf`. F16 (bf16 runs of the wide zero-shift pass): the
  // key tile holds fp16 keys. F16V (bf16 synthesis, exact pass): the value tile holds N0(s) in fp16.
  // The encode's wide zero-shift pass also keeps the largest ||K_n||^2 per row (knmax).
  auto store_set = [&](auto P, int buf, auto F16, auto F16V) {
    constexpr bool f16keys = decltype(F16)::value && sizeof(T) == 2;
    constexpr bool f16vals = decltype(F16V)::value && sizeof(T) == 2;
    T* kdst = ks + buf * kStage * RS;
    T* vdst = vt + buf * VE;
#pragma unroll
    for (int i = 0; i < PER; i++) {
      const int q = tid + i * NT;
      if (q < NCH) {
        const int t = q / CPR, part = q % CPR;
        if constexpr (SYNTH) {
          // N0 of the synthesis key row (Section 3.2, Eq. 5): keys c*N0(s), values N0(s). The
          // row's CPR chunks sit in consecutive lanes, reduced with DPP.
          float x[CH];
          chunk_to_float<T>(kr[decltype(P)::value][i], x);
          float ss = 0.f;
#pragma unroll
          for (int j = 0; j < CH; j++) ss += x[j] * x[j];
          ss = group_sum<CPR>(ss);
          const float inv = rsqrtf(ss * (1.0f / D) + kRmsEps);  // v_rsq_f32 (1 ulp)
          float kx[CH];
#pragma unroll
          for (int j = 0; j < CH; j++) {
            x[j] *= inv;
            kx[j] = x[j] * c_scale;
          }
          if constexpr (f16keys) {
            f16x8 hk;
#pragma unroll
            for (int j = 0; j < 8; j++) hk[j] = (f16)kx[j];
            *reinterpret_cast<f16x8*>(kdst + t * RS + part * CH) = hk;
          } else if constexpr (kFactorKeys) {
            // c N0(s) = (c / rms(s)) s: the raw keys are exact bf16 MFMA operands and the factor
            // scales each token's scores in fp32. A bf16 copy of c N0(s) would carry a relative
            // error of 2^-9 into logits that grow with the seeds' scale (Appendix A.3, Eq. 14).
            *reinterpret_cast<Chunk*>(kdst + t * RS + part * CH) = kr[decltype(P)::value][i];
            if (part == 0) tf[buf * kStage + t] = inv * c_scale;
          } else {
            *reinterpret_cast<Chunk*>(kdst + t * RS + part * CH) = float_to_chunk<T>(kx);
          }
          if constexpr (f16vals) {
            f16x8 hv;
#pragma unroll
            for (int j = 0; j < 8; j++) hv[j] = (f16)x[j];
            rowtile_store<T, D>(vdst, kStage, t, part * CH, __builtin_bit_cast(Chunk, hv));
          } else {
            rowtile_store<T, D>(vdst, kStage, t, part * CH, float_to_chunk<T>(x));
          }
          if constexpr (HILO) {
            float xl[CH];
#pragma unroll
            for (int j = 0; j < CH; j++) xl[j] = x[j] - (float)(T)x[j];
            rowtile_store<T, D>(vtl + buf * VE, kStage, t, part * CH, float_to_chunk<T>(xl));
          }
        } else {
          if constexpr (f16keys) {
            const bf16x8 kb = __builtin_bit_cast(bf16x8, kr[decltype(P)::value][i]);
            *reinterpret_cast<f16x8*>(kdst + t * RS + part * CH) = to_f16x8(kb);
            // An LDS max without a returned value (non-negative floats order as their bits), so
            // no register waits for it in this loop, where every register is in use.
            const float k2 = group_sum<CPR>(sumsq_bf16x8(kb));
            if (part == 0) atomicMax(reinterpret_cast<unsigned*>(knmax) + t, __float_as_uint(k2));
          } else
            *reinterpret_cast<Chunk*>(kdst + t * RS + part * CH) = kr[decltype(P)::value][i];
          rowtile_store<T, D>(vdst, kStage, t, part * CH, vr[decltype(P)::value][i]);
        }
      }
    }
  };

  // One stage of compute on buffer `buf` (tokens s0 .. s0 + nvalid - 1).
  auto compute = [&](auto EXACT, int buf, int nvalid) {
    constexpr bool exact = decltype(EXACT)::value;
    const T* kt = ks + buf * kStage * RS;
    const T* vtt = vt + buf * VE;
    const T* vtlt = vtl + buf * VE;
    const int nsub = (nvalid + 31) / 32;
    for (int st = 0; st < nsub; st++) {
      const Slice ka0 = O::load_slice(kt + (32 * st + perm_row(c, 0)) * RS, g);
      const Slice ka1 = O::load_slice(kt + (32 * st + perm_row(c, 1)) * RS, g);
      f32x4 s0v[NLB], s1v[NLB];
#pragma unroll
      for (int lb = 0; lb < NLB; lb++) {
        s0v[lb] = O::qk(ka0, qb[lb], f32x4{0.f, 0.f, 0.f, 0.f});
        s1v[lb] = O::qk(ka1, qb[lb], f32x4{0.f, 0.f, 0.f, 0.f});
        if constexpr (QP == 2) {
          s0v[lb] = O::qk(ka0, qlo[lb], s0v[lb]);
          s1v[lb] = O::qk(ka1, qlo[lb], s1v[lb]);
        }
      }
      __builtin_amdgcn_sched_barrier(kAllButMfma);
      keep_live(ka0);
      keep_live(ka1);
      if constexpr (kFactorKeys) {
        // Lane group g holds tokens 32 st + 8 g + i (s0v[.][i]) and + 4 + i (s1v[.][i]).
        const f32x4* fp = reinterpret_cast<const f32x4*>(tf + buf * kStage + 32 * st + 8 * g);
        const f32x4 f0 = fp[0], f1 = fp[1];
#pragma unroll
        for (int lb = 0; lb < NLB; lb++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            s0v[lb][i] *= f0[i];
            s1v[lb][i] *= f1[i];
          }
      }
      // Tokens past the end of the chunk do not enter the softmax.
      if (32 * st + 32 > nvalid) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const bool ok0 = 32 * st + 8 * g + i < nvalid;
          const bool ok1 = 32 * st + 8 * g + 4 + i < nvalid;
#pragma unroll
          for (int lb = 0; lb < NLB; lb++) {
            if (!ok0) s0v[lb][i] = -INFINITY;
            if (!ok1) s1v[lb][i] = -INFINITY;
          }
        }
      }
      if constexpr (exact) {
#pragma unroll
        for (int lb = 0; lb < NLB; lb++) {
          float tm = fmaxf(fmaxf(fmaxf(s0v[lb][0], s0v[lb][1]), fmaxf(s0v[lb][2], s0v[lb][3])),
                           fmaxf(fmaxf(s1v[lb][0], s1v[lb][1]), fmaxf(s1v[lb][2], s1v[lb][3])));
          tm = fmaxf(tm, shfl_xor(tm, 16));
          tm = max_xor32(tm);
          const float mold = mrow[lb];
          const float mnew = fmaxf(mold, tm);
          const float alpha = (mnew == mold) ? 1.0f : exp2_fast(mold - mnew);
          const float shift = (mnew == -INFINITY) ? 0.0f : mnew;
          mrow[lb] = mnew;
          lsum[lb] *= alpha;
          // Accumulator row 4g+i of this block belongs to the latent held by lane column 4g+i.
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const float ai = shfl(alpha, 4 * g + i);
#pragma unroll
            for (int db = 0; db < NDB; db++) zacc[lb][db][i] *= ai;
          }
#pragma unroll
          for (int i = 0; i < 4; i++) {
            s0v[lb][i] = exp2_fast(s0v[lb][i] - shift);
            s1v[lb][i] = exp2_fast(s1v[lb][i] - shift);
          }
        }
      } else {
#pragma unroll
        for (int lb = 0; lb < NLB; lb++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            s0v[lb][i] = exp2_fast(s0v[lb][i]);
            s1v[lb][i] = exp2_fast(s1v[lb][i]);
          }
      }
      if constexpr (kF16Exact && exact) {
        f16x8 vh[NDB];
#pragma unroll
        for (int db = 0; db < NDB; db++)
          vh[db] = as_f16x8(O::load_oct_rows(vtt, VSTR, 32 * st, 16 * db, c, g));
#pragma unroll
        for (int lb = 0; lb < NLB; lb++) {
          f16x8 ph;
#pragma unroll
          for (int i = 0; i < 4; i++) {
            ph[i] = (f16)s0v[lb][i];
            ph[4 + i] = (f16)s1v[lb][i];
          }
          typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
          const f16x2 one = {(f16)1.0f, (f16)1.0f};
#pragma unroll
          for (int i = 0; i < 4; i++) lsum[lb] = __builtin_amdgcn_fdot2(f16x2{ph[2 * i], ph[2 * i + 1]}, one, lsum[lb], false);
#pragma unroll
          for (int db = 0; db < NDB; db++)
            zacc[lb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph, vh[db], zacc[lb][db], 0, 0, 0);
        }
        continue;
      }
      Oct vb[NDB];
#pragma unroll
      for (int db = 0; db < NDB; db++) vb[db] = O::load_oct_rows(vtt, VSTR, 32 * st, 16 * db, c, g);
      Oct vbl[HILO && SYNTH ? NDB : 1];
      if constexpr (HILO && SYNTH) {
#pragma unroll
        for (int db = 0; db < NDB; db++) vbl[db] = O::load_oct_rows(vtlt, VSTR, 32 * st, 16 * db, c, g);
      }
#pragma unroll
      for (int lb = 0; lb < NLB; lb++) {
        const Oct pa = O::pack(s0v[lb], s1v[lb]);
        lsum[lb] = O::osum(pa, lsum[lb]);
#pragma unroll
        for (int db = 0; db < NDB; db++) zacc[lb][db] = O::pv(pa, vb[db], zacc[lb][db]);
        if constexpr (HILO) {
          // Residuals s - bf16(s), two per packed word of pa (bf16_residual2).
          typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
          const u32x4 pw = __builtin_bit_cast(u32x4, pa);
          const residual2_t a0 = bf16_residual2(pw[0], s0v[lb][0], s0v[lb][1]);
          const residual2_t a1 = bf16_residual2(pw[1], s0v[lb][2], s0v[lb][3]);
          const residual2_t b0 = bf16_residual2(pw[2], s1v[lb][0], s1v[lb][1]);
          const residual2_t b1 = bf16_residual2(pw[3], s1v[lb][2], s1v[lb][3]);
          const f32x4 r0 = {a0[0], a0[1], a1[0], a1[1]}, r1 = {b0[0], b0[1], b1[0], b1[1]};
          const Oct pl = O::pack(r0, r1);
          lsum[lb] = O::osum(pl, lsum[lb]);
#pragma unroll
          for (int db = 0; db < NDB; db++) {
            zacc[lb][db] = O::pv(pl, vb[db], zacc[lb][db]);
            if constexpr (SYNTH) zacc[lb][db] = O::pv(pa, vbl[db], zacc[lb][db]);
          }
        }
      }
    }
  };

  // Zero-shift stage compute with 32x32x16 MFMAs (kWide): per 32-token sub-tile, the fp16 key rows
  // (A operand, token 32 st + l % 32) against each 32-latent block's fp16 queries, then the bf16
  // probabilities of result slots 8t .. 8t+7 (tokens row32(8t + e, h)) times the value rows of the
  // same tokens.
  f32x16 zw[NB];
  float lw[NB];
  // Row sums of the pipelined stages, accumulated on the matrix unit (see sum_selector).
  f32x4 ls4 = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16x8 sel = sum_selector(lane);
  auto compute_wide = [&](int buf, int nvalid) {
    if constexpr (kWide) {
      const bf16* kt = reinterpret_cast<const bf16*>(ks) + buf * kStage * RS;
      const bf16* vtt = reinterpret_cast<const bf16*>(vt) + buf * VE;
      const int nsub = (nvalid + 31) / 32;
      for (int st = 0; st < nsub; st++) {
        const bf16* krow = kt + (32 * st + (lane & 31)) * RS + 8 * h32;
        const f16x8 ka0 = *reinterpret_cast<const f16x8*>(krow);
        const f16x8 ka1 = *reinterpret_cast<const f16x8*>(krow + 16);
        f32x16 sw[NB];
#pragma unroll
        for (int nb = 0; nb < NB; nb++) {
          sw[nb] = mfma_32x32_f16(ka0, qw[nb][0], f32x16{});
          sw[nb] = mfma_32x32_f16(ka1, qw[nb][1], sw[nb]);
        }
        __builtin_amdgcn_sched_barrier(kAllButMfma);
        keep_live(ka0);
        keep_live(ka1);
        if (32 * st + 32 > nvalid) {
#pragma unroll
          for (int v = 0; v < 16; v++)
            if (32 * st + row32(v, h32) >= nvalid)
#pragma unroll
              for (int nb = 0; nb < NB; nb++) sw[nb][v] = -INFINITY;
        }
        const bf16x8 vb0 = load_rows32(vtt, VSTR, 32 * st, 0, lane);
        const bf16x8 vb1 = load_rows32(vtt, VSTR, 32 * st + 16, 0, lane);
#pragma unroll
        for (int nb = 0; nb < NB; nb++) {
#pragma unroll
          for (int v = 0; v < 16; v++) sw[nb][v] = exp2_fast(sw[nb][v]);
          const bf16x8 p0 = pack32(sw[nb], 0), p1 = pack32(sw[nb], 1);
          lw[nb] = O::osum(p1, O::osum(p0, lw[nb]));
          zw[nb] = mfma_32x32(p0, vb0, zw[nb]);
          zw[nb] = mfma_32x32(p1, vb1, zw[nb]);
          __builtin_amdgcn_sched_barrier(kAllButMfma);
          keep_live(p0);
          keep_live(p1);
        }
        keep_live(vb0);
        keep_live(vb1);
      }
    }
  };
  // Full stages of the wide zero-shift pass, software-pipelined over the 32-token sub-tiles. Step j
  // issues, in this order (each piece fenced so the scheduler keeps it):
  //   S1(j+1) | exp 0-3 (j) | S2(j+1) | exp 4-7 | pack/sum slots 0-7 | PV1(j) | exp 8-15 |
  //   pack/sum slots 8-15 | PV2(j)
  // where S1, S2 are the two fp16 score MFMAs of the next sub-tile and PV1, PV2 the bf16 P.V MFMAs
  // of this one, so every MFMA runs under vector work of the same wave. LDS operands are read one
  // step ahead. Sub-tiles go in pairs so no register copies are needed between steps.
  auto compute_wide_full = [&](int buf) {
    if constexpr (kWide && NB == 1) {
      constexpr int NS = kStage / 32;
      static_assert(NS % 2 == 0, "pairs of sub-tiles");
      const bf16* kt = reinterpret_cast<const bf16*>(ks) + buf * kStage * RS + (lane & 31) * RS + 8 * h32;
      const bf16* vtt = reinterpret_cast<const bf16*>(vt) + buf * VE;
      auto fence = []() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };
      struct KOp { f16x8 a, b; };
      struct VOp { bf16x8 a, b; };
      auto load_k = [&](int st) __attribute__((always_inline)) {
        return KOp{*reinterpret_cast<const f16x8*>(kt + 32 * st * RS), *reinterpret_cast<const f16x8*>(kt + 32 * st * RS + 16)};
      };
      auto load_v = [&](int st) __attribute__((always_inline)) {
        return VOp{load_rows32(vtt, VSTR, 32 * st, 0, lane), load_rows32(vtt, VSTR, 32 * st + 16, 0, lane)};
      };
      auto exps = [&](f32x16& x, int v0) __attribute__((always_inline)) {
#pragma unroll
        for (int v = 0; v < 4; v++) x[v0 + v] = exp2_fast(x[v0 + v]);
      };
      // Step st: scores of sub-tile st+1 into `nx` (keys `kn`, replaced by those of st+2 once the
      // score MFMAs are issued), probabilities and P.V of sub-tile st (`cu`).
      auto step = [&](int st, f32x16& cu, const VOp& vc, f32x16& nx, KOp& kn) __attribute__((always_inline)) {
        const bool has_next = st + 1 < NS;
        if (has_next) nx = mfma_32x32_f16(kn.a, qw[0][0], f32x16{});
        fence();
        exps(cu, 0);
        fence();
        if (has_next) nx = mfma_32x32_f16(kn.b, qw[0][1], nx);
        fence();
        keep_live(kn.a);
        keep_live(kn.b);
        if (st + 2 < NS) kn = load_k(st + 2);
        exps(cu, 4);
        const bf16x8 p0 = pack32(cu, 0);
        fence();
        zw[0] = mfma_32x32(p0, vc.a, zw[0]);
        ls4 = mfma_32k(p0, sel, ls4);
        fence();
        keep_live(p0);
        keep_live(vc.a);
        exps(cu, 8);
        exps(cu, 12);
        const bf16x8 p1 = pack32(cu, 1);
        fence();
        zw[0] = mfma_32x32(p1, vc.b, zw[0]);
        ls4 = mfma_32k(p1, sel, ls4);
        fence();
        keep_live(p1);
        keep_live(vc.b);
      };
      // Prologue: scores of sub-tile 0 and the keys of sub-tile 1. Step st reads the values of
      // sub-tile st at its start and the keys of sub-tile st+2 once its score MFMAs are issued.
      f32x16 sc[2];
      {
        const KOp k0 = load_k(0);
        sc[0] = mfma_32x32_f16(k0.a, qw[0][0], f32x16{});
        sc[0] = mfma_32x32_f16(k0.b, qw[0][1], sc[0]);
        fence();
        keep_live(k0.a);
        keep_live(k0.b);
      }
      KOp kn = load_k(1);
#pragma unroll
      for (int st = 0; st < NS; st++) {
        const VOp vc = load_v(st);
        step(st, sc[st & 1], vc, sc[(st + 1) & 1], kn);
      }
    }
  };

  auto run_chunk_wide = [&]() {
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
      lw[nb] = 0.f;
      zw[nb] = f32x16{};
    }
    ls4 = f32x4{0.f, 0.f, 0.f, 0.f};
    load_set(I0{}, 0);
    if (nstage > 1) load_set(I1{}, 1);
    store_set(I0{}, 0, std::true_type{}, std::false_type{});
    if (nstage > 2) load_set(I0{}, 2);
    __syncthreads();
    auto wstep = [&](auto P, int s) {
      if (s + 1 < nstage) store_set(P, (s + 1) & 1, std::true_type{}, std::false_type{});
      if (s + 3 < nstage) load_set(P, s + 3);
      if (active) {
        const int64_t left = n_end - (n_begin + (int64_t)s * kStage);
        if (NB == 1 && left >= kStage)
          compute_wide_full(s & 1);
        else
          compute_wide(s & 1, left < kStage ? (int)left : kStage);
      }
      __syncthreads();
    };
    for (int s = 0; s < nstage; s += 2) {
      wstep(I1{}, s);
      if (s + 1 < nstage) wstep(I0{}, s + 1);
    }
  };

  // Stage s: store stage s+1 (register set P = (s+1) % 2) into its buffer, refill set P with stage
  // s+3, compute stage s, barrier.
  auto step = [&](auto P, auto EXACT, int s) {
    if (s + 1 < nstage)
      store_set(P, (s + 1) & 1, std::false_type{}, std::integral_constant<bool, decltype(EXACT)::value && kF16Exact>{});
    if (s + 3 < nstage) load_set(P, s + 3);
    if (active) {
      const int64_t left = n_end - (n_begin + (int64_t)s * kStage);
      compute(EXACT, s & 1, left < kStage ? (int)left : kStage);
    }
    __syncthreads();
  };

  auto run_chunk = [&](auto EXACT) {
#pragma unroll
    for (int lb = 0; lb < NLB; lb++) {
      lsum[lb] = 0.f;
      mrow[lb] = decltype(EXACT)::value ? -INFINITY : 0.f;
#pragma unroll
      for (int db = 0; db < NDB; db++) zacc[lb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    load_set(I0{}, 0);
    if (nstage > 1) load_set(I1{}, 1);
    store_set(I0{}, 0, std::false_type{}, std::integral_constant<bool, decltype(EXACT)::value && kF16Exact>{});
    if (nstage > 2) load_set(I0{}, 2);
    __syncthreads();
    for (int s = 0; s < nstage; s += 2) {
      step(I1{}, EXACT, s);
      if (s + 1 < nstage) step(I0{}, EXACT, s + 1);
    }
  };

  // Synthesis logits are bounded a priori by ||Qseed_m|| log2(e) (the keys have unit RMS): seeds
  // far outside the zero-shift range go straight to the exact pass.
  bool exact = a.force_exact != 0;
  if constexpr (SYNTH) {
    float qss = 0.f;
    if constexpr (kWide) {
#pragma unroll
      for (int nb = 0; nb < NB; nb++) {
        float ss = 0.f;
#pragma unroll
        for (int kh = 0; kh < 2; kh++)
#pragma unroll
          for (int e = 0; e < 8; e++) ss += (float)qw[nb][kh][e] * (float)qw[nb][kh][e];
        ss = sum_xor32(ss);
        qss = fmaxf(qss, ss);
      }
    } else {
#pragma unroll
      for (int lb = 0; lb < NLB; lb++) {
        float ss = O::sumsq(qb[lb]);
        ss += shfl_xor(ss, 16);
        ss = sum_xor32(ss);
        qss = fmaxf(qss, ss);
      }
    }
    if (!__all(sqrtf(qss) * kLog2e * 1.01f <= kFastBound) && lane == 0) atomicOr(fail_s, 1);
    __syncthreads();
    exact = exact || *fail_s != 0;
  }
  const int64_t pbase = ((int64_t)bh * a.nchunk + chunk_id) * a.Mp;
  if constexpr (kWide) {
    if (!HILO && !exact && !a.hilo) {
      run_chunk_wide();
      if constexpr (NB == 1) {
        // Latent j = l % 32 sums to row j % 16, columns 0-7 (j < 16) or 8-15 (j >= 16): lane
        // 16 ((j % 16) / 4) + 8 (j / 16), slot j % 4. Counted once, on the half h = 0.
        const int j = lane & 31;
        const int src = 16 * ((j & 15) >> 2) + 8 * (j >> 4);
        const float s0 = shfl(ls4[0], src), s1 = shfl(ls4[1], src), s2 = shfl(ls4[2], src), s3 = shfl(ls4[3], src);
        const int slot = j & 3;
        const float lj = slot == 0 ? s0 : slot == 1 ? s1 : slot == 2 ? s2 : s3;
        if (h32 == 0) lw[0] += lj;
      }
      bool ok = true;
      if (active) {
#pragma unroll
        for (int nb = 0; nb < NB; nb++) {
          const float l = sum_xor32(lw[nb]);
          ok = ok && l >= 0x1p-80f && l <= 0x1p100f;
#pragma unroll
          for (int v = 0; v < 16; v++) ok = ok && fabsf(zw[nb][v]) <= 3.0e38f;
        }
      }
      if (!__all(ok) && lane == 0) atomicOr(fail_s, 1);
      __syncthreads();
      // Routing bound (kRouteBound) over every latent and token of the chunk: beyond it the chunk
      // takes the exact pass, whose logits use the hi/lo query pair.
      bool in_bound = true;
      if constexpr (!SYNTH) {
        float qm = 0.f, km = 0.f;
#pragma unroll
        for (int w = 0; w < NW; w++) qm = fmaxf(qm, qred[w]);
        for (int t = lane; t < kStage; t += 64) km = fmaxf(km, knmax[t]);
        in_bound = qm * wave_max_dpp(km) <= kRouteBound * kRouteBound;
      }
      if (*fail_s == 0 && in_bound) {
        if (!active) return;
#pragma unroll
        for (int nb = 0; nb < NB; nb++) {
          const float l = sum_xor32(lw[nb]);
          const int row = lat0 + 32 * nb + (lane & 31);
          if (h32 == 0 && row < a.Mp) {
            a.part_l[pbase + row] = l;
            a.part_m[pbase + row] = 0.f;
          }
#pragma unroll
          for (int v = 0; v < 16; v++) {
            const int r = lat0 + 32 * nb + row32(v, h32);
            if (r < a.Mp) a.part_acc[(pbase + r) * D + (lane & 31)] = zw[nb][v];
          }
        }
        return;
      }
      exact = true;
    }
    load_queries();
  }
  if (!exact) {
    run_chunk(std::false_type{});
    // Check every row of the zero-shift pass.
    bool ok = true;
    if (active) {
#pragma unroll
      for (int lb = 0; lb < NLB; lb++) {
        float l = lsum[lb];
        l += shfl_xor(l, 16);
        l = sum_xor32(l);
        ok = ok && l >= 0x1p-80f && l <= 0x1p100f;
#pragma unroll
        for (int db = 0; db < NDB; db++)
#pragma unroll
          for (int i = 0; i < 4; i++) ok = ok && fabsf(zacc[lb][db][i]) <= 3.0e38f;
      }
    }
    if (!__all(ok) && lane == 0) atomicOr(fail_s, 1);
    __syncthreads();
    exact = *fail_s != 0;
  }
  if (exact) run_chunk(std::true_type{});

  if (!active) return;
  // Partials of this chunk: l and m per latent, the P.V accumulator per latent and channel.
#pragma unroll
  for (int lb = 0; lb < NLB; lb++) {
    float l = lsum[lb];
    l += shfl_xor(l, 16);
    l = sum_xor32(l);
    const int row = lat0 + 16 * lb + c;
    if (g == 0 && row < a.Mp) {
      a.part_l[pbase + row] = l;
      a.part_m[pbase + row] = mrow[lb];
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r = lat0 + 16 * lb + 4 * g + i;
      if (r < a.Mp) {
#pragma unroll
        for (int db = 0; db < NDB; db++) a.part_acc[(pbase + r) * D + 16 * db + c] = zacc[lb][db][i];
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// Merge of the chunk partials (Appendix B.3, Eq. 30-33): m = max_c m_c, d = sum_c 2^(m_c - m) l_c,
// U = sum_c 2^(m_c - m) A_c, result U / d. With GATE, Q = N0(Qf) + g * Qd (Eq. 7) in fp32, cast
// with the factor c = log2(e)/sqrt(D) folded in; otherwise Z is cast unscaled. One thread per
// (latent, channel); rows in [M, Mout) are written as zeros.
template <typename T, int D, bool GATE>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  // Block: 256 / D latent rows x D channels. The chunk maxima and the normalizer of a row are
  // reduced across its D lanes (chunks strided over the lanes); the chunk weights 2^(m_c - m) go
  // through LDS to the accumulator pass, which streams the chunks with several loads in flight.
  constexpr int RPB = 256 / D;
  extern __shared__ float wsh[];  // [RPB][nchunk]
  const int bh = blockIdx.y;
  const int lr = threadIdx.x / D, d = threadIdx.x % D;
  const int row = blockIdx.x * RPB + lr;
  float* w = wsh + lr * a.nchunk;
  float res = 0.f, qd = 0.f;
  const int64_t base = (int64_t)bh * a.nchunk * a.Mp;
  const bool valid = row < a.M;
  float m = -INFINITY, den = 0.f;
  if (valid) {
    for (int ch = d; ch < a.nchunk; ch += D) m = fmaxf(m, a.part_m[base + (int64_t)ch * a.Mp + row]);
  }
#pragma unroll
  for (int o = 1; o < D; o <<= 1) m = fmaxf(m, shfl_xor(m, o));
  if (valid) {
    for (int ch = d; ch < a.nchunk; ch += D) {
      const int64_t o = base + (int64_t)ch * a.Mp + row;
      const float wc = exp2_fast(a.part_m[o] - m);
      w[ch] = wc;
      den += wc * a.part_l[o];
    }
  }
#pragma unroll
  for (int o = 1; o < D; o <<= 1) den += shfl_xor(den, o);
  if (a.lse && d == 0 && row < a.Mout) a.lse[(int64_t)bh * a.Mout + row] = valid ? m + log2f(den) : INFINITY;
  __syncthreads();
  if (valid) {
    const float* acc = a.part_acc + (base + row) * D + d;
    const int64_t cstride = (int64_t)a.Mp * D;
    float num0 = 0.f, num1 = 0.f, num2 = 0.f, num3 = 0.f;
    int ch = 0;
    for (; ch + 4 <= a.nchunk; ch += 4) {
      num0 += w[ch] * acc[(int64_t)ch * cstride];
      num1 += w[ch + 1] * acc[(int64_t)(ch + 1) * cstride];
      num2 += w[ch + 2] * acc[(int64_t)(ch + 2) * cstride];
      num3 += w[ch + 3] * acc[(int64_t)(ch + 3) * cstride];
    }
    for (; ch < a.nchunk; ch++) num0 += w[ch] * acc[(int64_t)ch * cstride];
    qd = ((num0 + num1) + (num2 + num3)) / den;
    res = qd;
  }
  if (row >= a.Mout) return;  // rows past M up to Mout are written as zeros below
  if constexpr (GATE) {
    // Without Qf the routing queries are Qd alone (simplified FLARE++, Appendix A.8 Eq. 20).
    const int h = bh % a.H;
    const bool fixed = a.Qf != nullptr;
    const float f = (fixed && row < a.M) ? to_f(reinterpret_cast<const T*>(a.Qf)[((int64_t)h * a.M + row) * D + d]) : 0.f;
    float ss = f * f;
#pragma unroll
    for (int m = 1; m < D; m <<= 1) ss += shfl_xor(ss, m);
    const float gv = fixed ? a.g[h] : 1.0f;
    res = (row < a.M) ? f / sqrtf(ss * (1.0f / D) + kRmsEps) + gv * qd : 0.f;
    if (a.dbg_qd && row < a.M) a.dbg_qd[((int64_t)bh * a.M + row) * D + d] = qd;
    if (a.dbg_out && row < a.M) a.dbg_out[((int64_t)bh * a.M + row) * D + d] = res;
    // c*Q as hi (and, for bf16, lo = the rounding residual of hi).
    const float cq = res * (kLog2e * rsqrtf((float)D));
    T* qo = reinterpret_cast<T*>(a.out) + ((int64_t)bh * a.Mout + row) * kQRow<T> * D + d;
    const T hi = (T)cq;
    qo[0] = hi;
    if constexpr (sizeof(T) == 2) {
      qo[D] = (T)(cq - to_f(hi));
      reinterpret_cast<f16*>(qo + 2 * D)[0] = (f16)cq;
    }
  } else {
    if (a.dbg_out && row < a.M) a.dbg_out[((int64_t)bh * a.M + row) * D + d] = res;
    reinterpret_cast<T*>(a.out)[((int64_t)bh * a.Mout + row) * D + d] = (T)res;
  }
}

// ------------------------------------------------------------------------------------------
// Plain FLARE (Section 3.1, Eq. 3): the routing-query rows of the workspace from the caller's
// fixed queries, c*Q in the same parts as the gate writes (bf16: hi, lo, fp16). One thread per
// (latent, channel) of every (b, h) block.
template <typename T, int D>
__global__ __launch_bounds__(256) void query_prep_kernel(QueryPrepArgs a) {
  const int bh = blockIdx.y;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int row = idx / D, d = idx % D;
  if (row >= a.Mout) return;
  const int h = bh % a.H;
  const float q = row < a.M ? to_f(reinterpret_cast<const T*>(a.Q)[((int64_t)h * a.M + row) * D + d]) : 0.f;
  const float cq = q * (kLog2e * rsqrtf((float)D));
  T* qo = reinterpret_cast<T*>(a.out) + ((int64_t)bh * a.Mout + row) * kQRow<T> * D + d;
  const T hi = (T)cq;
  qo[0] = hi;
  if constexpr (sizeof(T) == 2) {
    qo[D] = (T)(cq - to_f(hi));
    reinterpret_cast<f16*>(qo + 2 * D)[0] = (f16)cq;
  }
}

// ------------------------------------------------------------------------------------------
// Decode: every token's scores against all M routing queries, softmax over M, times Z
// (Eq. 8, second call). The workgroup keeps c*Q (row-major, A operand of the score MFMA, hi then lo
// per row) and Z (a RowTile: the A operand of the P.V MFMA runs along latents) in LDS; each wave
// takes groups of 16 * TB tokens whose K rows it reads straight from HBM as B operands.
template <typename T, int D, int NW, int TB>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeArgs a) {
  using O = Ops<T, D>;
  using Slice = typename O::Slice;
  using Oct = typename O::Oct;
  using ZT = RowTile<T, D>;
  constexpr int NDB = D / 16;
  constexpr int NT = NW * 64;
  constexpr int CH = 16 / sizeof(T);
  constexpr int CPR = D / CH;
  constexpr int QP = kQParts<T>;
  constexpr int RQ = QP * D + CH;  // a row holds the hi part then (bf16) the lo part
  constexpr int TG = 16 * TB;      // tokens per wave group

  extern __shared__ __align__(16) unsigned char smem[];
  const int Mp = a.Mp;  // multiple of 32
  T* qs = reinterpret_cast<T*>(smem);  // [Mp][RQ]
  T* zs = qs + Mp * RQ;                 // RowTile of Mp rows
  const int ZSTR = ZT::stride(Mp);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int bh = blockIdx.y;
  const T* qsrc = reinterpret_cast<const T*>(a.Q) + (int64_t)bh * Mp * kQRow<T> * D;
  const T* zsrc = reinterpret_cast<const T*>(a.Z) + (int64_t)bh * Mp * D;

  for (int q0 = 0; q0 < Mp * CPR; q0 += NT) {
    const int q = q0 + tid;
    if (q < Mp * CPR) {
      const int row = q / CPR, part = q % CPR;
      *reinterpret_cast<Chunk*>(qs + row * RQ + part * CH) =
          *reinterpret_cast<const Chunk*>(qsrc + (int64_t)row * kQRow<T> * D + part * CH);
      if constexpr (QP == 2)
        *reinterpret_cast<Chunk*>(qs + row * RQ + D + part * CH) =
            *reinterpret_cast<const Chunk*>(qsrc + (int64_t)row * kQRow<T> * D + D + part * CH);
      rowtile_store<T, D>(zs, Mp, row, part * CH, *reinterpret_cast<const Chunk*>(zsrc + (int64_t)row * D + part * CH));
    }
  }
  __syncthreads();

  const int64_t t_begin = (int64_t)blockIdx.x * a.tokens_per_wg;
  const int64_t t_end = (t_begin + a.tokens_per_wg < a.N) ? t_begin + a.tokens_per_wg : a.N;
  const T* kbase = reinterpret_cast<const T*>(a.K) + (int64_t)bh * a.N * D;
  T* obase = reinterpret_cast<T*>(a.out) + (int64_t)bh * a.N * D;
  const int nlb = Mp / 32;
  const bool ragged = (a.M & 31) != 0;

  for (int64_t base = t_begin + (int64_t)wave * TG; base < t_end; base += (int64_t)NW * TG) {
    Slice kb[TB];
#pragma unroll
    for (int t = 0; t < TB; t++) {
      const int64_t tok = base + 16 * t + c;
      kb[t] = (tok < a.N) ? O::load_slice(kbase + tok * D, g) : O::zero_slice();
    }

    // Scores of latent block lb for every token block t: lane (c, g) gets token 16t + c and
    // latents 32 lb + 8g .. 32 lb + 8g + 7 (s0[t]: first four, s1[t]: last four).
    auto scores_all = [&](int lb, f32x4* s0, f32x4* s1) {
      const Slice qa0 = O::load_slice(qs + (32 * lb + perm_row(c, 0)) * RQ, g);
      const Slice qa1 = O::load_slice(qs + (32 * lb + perm_row(c, 1)) * RQ, g);
      Slice ql0, ql1;
      if constexpr (QP == 2) {
        ql0 = O::load_slice(qs + (32 * lb + perm_row(c, 0)) * RQ + D, g);
        ql1 = O::load_slice(qs + (32 * lb + perm_row(c, 1)) * RQ + D, g);
      }
#pragma unroll
      for (int t = 0; t < TB; t++) {
        s0[t] = O::qk(qa0, kb[t], f32x4{0.f, 0.f, 0.f, 0.f});
        s1[t] = O::qk(qa1, kb[t], f32x4{0.f, 0.f, 0.f, 0.f});
        if constexpr (QP == 2) {
          s0[t] = O::qk(ql0, kb[t], s0[t]);
          s1[t] = O::qk(ql1, kb[t], s1[t]);
        }
      }
      __builtin_amdgcn_sched_barrier(kAllButMfma);
      keep_live(qa0);
      keep_live(qa1);
      if constexpr (QP == 2) {
        keep_live(ql0);
        keep_live(ql1);
      }
      if (ragged && lb == nlb - 1) {
#pragma unroll
        for (int t = 0; t < TB; t++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            if (32 * lb + 8 * g + i >= a.M) s0[t][i] = -INFINITY;
            if (32 * lb + 8 * g + 4 + i >= a.M) s1[t][i] = -INFINITY;
          }
      }
    };

    f32x4 yacc[TB][NDB];
    float lsum[TB];
    auto clear = [&]() {
#pragma unroll
      for (int t = 0; t < TB; t++) {
        lsum[t] = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; db++) yacc[t][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    };
    // Probabilities, their sums and the P.V product over all latent blocks, with the exponentials
    // shifted by `shift` (exact path) or unshifted (zero-shift path).
    float shift[TB];
    auto accumulate = [&](auto exact) {
      for (int lb = 0; lb < nlb; lb++) {
        Oct za[NDB];
#pragma unroll
        for (int db = 0; db < NDB; db++) za[db] = O::load_oct_rows(zs, ZSTR, 32 * lb, 16 * db, c, g);
        f32x4 s0[TB], s1[TB];
        scores_all(lb, s0, s1);
#pragma unroll
        for (int t = 0; t < TB; t++) {
#pragma unroll
          for (int i = 0; i < 4; i++) {
            if constexpr (decltype(exact)::value) {
              s0[t][i] = exp2_fast(s0[t][i] - shift[t]);
              s1[t][i] = exp2_fast(s1[t][i] - shift[t]);
            } else {
              s0[t][i] = exp2_fast(s0[t][i]);
              s1[t][i] = exp2_fast(s1[t][i]);
            }
          }
          const Oct pb = O::pack(s0[t], s1[t]);
          lsum[t] = O::osum(pb, lsum[t]);
#pragma unroll
          for (int db = 0; db < NDB; db++) yacc[t][db] = O::pv(za[db], pb, yacc[t][db]);
        }
        __builtin_amdgcn_sched_barrier(kAllButMfma);
#pragma unroll
        for (int db = 0; db < NDB; db++) keep_live(za[db]);
      }
    };

    // Zero-shift pass, then the check of every token's softmax over M (see the file header).
    clear();
    bool ok = a.force_exact == 0;
    if (ok) accumulate(std::false_type{});
#pragma unroll
    for (int t = 0; t < TB; t++) {
      float l = lsum[t];
      l += shfl_xor(l, 16);
      l = sum_xor32(l);
      ok = ok && l >= 0x1p-80f && l <= 0x1p100f;
#pragma unroll
      for (int db = 0; db < NDB; db++)
#pragma unroll
        for (int i = 0; i < 4; i++) ok = ok && fabsf(yacc[t][db][i]) <= 3.0e38f;
    }
    if (!__all(ok)) {
      // Two-pass maximum over the M latents for each token.
#pragma unroll
      for (int t = 0; t < TB; t++) shift[t] = -INFINITY;
      for (int lb = 0; lb < nlb; lb++) {
        f32x4 s0[TB], s1[TB];
        scores_all(lb, s0, s1);
#pragma unroll
        for (int t = 0; t < TB; t++)
          shift[t] = fmaxf(shift[t], fmaxf(fmaxf(fmaxf(s0[t][0], s0[t][1]), fmaxf(s0[t][2], s0[t][3])),
                                           fmaxf(fmaxf(s1[t][0], s1[t][1]), fmaxf(s1[t][2], s1[t][3]))));
      }
#pragma unroll
      for (int t = 0; t < TB; t++) {
        shift[t] = fmaxf(shift[t], shfl_xor(shift[t], 16));
        shift[t] = max_xor32(shift[t]);
      }
      clear();
      accumulate(std::true_type{});
    }

#pragma unroll
    for (int t = 0; t < TB; t++) {
      float l = lsum[t];
      l += shfl_xor(l, 16);
      l = sum_xor32(l);
      const float inv = 1.0f / l;
      const int64_t tok = base + 16 * t + c;
      if (tok < t_end) {
#pragma unroll
        for (int db = 0; db < NDB; db++) {
          T* dst = obase + tok * D + 16 * db + 4 * g;
          if constexpr (sizeof(T) == 2) {
            bf16x4 o;
#pragma unroll
            for (int i = 0; i < 4; i++) o[i] = (bf16)(yacc[t][db][i] * inv);
            *reinterpret_cast<bf16x4*>(dst) = o;
          } else {
            f32x4 o;
#pragma unroll
            for (int i = 0; i < 4; i++) o[i] = yacc[t][db][i] * inv;
            *reinterpret_cast<f32x4*>(dst) = o;
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// Decode for bf16 runs with D = 32 (Eq. 8, second call). The workgroup keeps the fp16 routing
// queries c*Q (A operand of the score MFMA, row-major) and Z (a RowTile: B operand of the P.V MFMA,
// read along latents) in LDS. Each wave takes groups of 32 * TB tokens; per latent block of 32 the
// scores of every token block come from 32x32x16 fp16 MFMAs (the keys converted to fp16 in
// registers) and land with one token per lane column and 16 latents per lane: exactly the B operand
// of the bf16 MFMA Z^T P, which yields Y^T with one token per lane column. Zero-shift pass, per-token range check, and for a group that fails an exact pass:
// two passes over the latents with running maxima, scores from bf16 keys and the hi/lo queries
// read from the workspace.
template <int NW, int TB, bool PREF = true>
__global__ __launch_bounds__(NW * 64) void decode_wide_kernel(DecodeArgs a) {
  constexpr int D = 32;
  constexpr int QHS = D + 8;  // fp16 query row stride in LDS (80 bytes: conflict-free row reads)
  using ZT = RowTile<bf16, D, kDecodeZPad>;
  constexpr int NT = NW * 64;
  constexpr int TG = 32 * TB;

  extern __shared__ __align__(16) unsigned char smem[];
  const int Mp = a.Mp;  // multiple of 32
  f16* qh = reinterpret_cast<f16*>(smem);                  // [Mp + 32][QHS]: a zero block at the end
  bf16* zs = reinterpret_cast<bf16*>(qh + (Mp + 32) * QHS);  // RowTile of Mp rows
  const int ZSTR = ZT::stride(Mp);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int bh = blockIdx.y;
  const bf16* qsrc = reinterpret_cast<const bf16*>(a.Q) + (int64_t)bh * Mp * kQRow<bf16> * D;
  const bf16* zsrc = reinterpret_cast<const bf16*>(a.Z) + (int64_t)bh * Mp * D;

  // Stage the queries and Z; keep the largest ||c Q_m||^2 (a row's four chunks sit in four
  // consecutive lanes) for the routing bound of the zero-shift pass.
  float q2 = 0.f;
  for (int q = tid; q < Mp * 4; q += NT) {
    const int row = q >> 2, part = q & 3;
    const Chunk qc = *reinterpret_cast<const Chunk*>(qsrc + (int64_t)row * kQRow<bf16> * D + 2 * D + part * 8);
    *reinterpret_cast<Chunk*>(qh + row * QHS + part * 8) = qc;
    q2 = fmaxf(q2, group_sum<4>(sumsq_f16x8(__builtin_bit_cast(f16x8, qc))));
    rowtile_store<bf16, D, kDecodeZPad>(zs, Mp, row, part * 8, *reinterpret_cast<const Chunk*>(zsrc + (int64_t)row * D + part * 8));
  }
  for (int q = tid; q < 32 * 4; q += NT) *reinterpret_cast<Chunk*>(qh + (Mp + (q >> 2)) * QHS + (q & 3) * 8) = Chunk{0u, 0u, 0u, 0u};
  float* qred = reinterpret_cast<float*>(zs + ZT::elems(Mp));  // [NW]
  q2 = wave_max_dpp(q2);
  if (lane == 0) qred[wave] = q2;
  __syncthreads();
  float qmax2 = 0.f;
#pragma unroll
  for (int w = 0; w < NW; w++) qmax2 = fmaxf(qmax2, qred[w]);

  const int64_t t_begin = (int64_t)blockIdx.x * a.tokens_per_wg;
  const int64_t t_end = (t_begin + a.tokens_per_wg < a.N) ? t_begin + a.tokens_per_wg : a.N;
  const bf16* kbase = reinterpret_cast<const bf16*>(a.K) + (int64_t)bh * a.N * D;
  bf16* obase = reinterpret_cast<bf16*>(a.out) + (int64_t)bh * a.N * D;
  const int nlb = Mp / 32;
  const bool ragged = (a.M & 31) != 0;

  // Key operands (B of the score MFMA): lane l holds dims 16 kh + 8 h .. + 7 of token
  // base + 32 tb + l % 32. The next wave group's keys are loaded while this one is computed.
  auto load_keys_at = [&](int64_t base, int tb, int kh) __attribute__((always_inline)) {
    const int64_t tok = base + 32 * tb + col;
    return tok < t_end ? *reinterpret_cast<const bf16x8*>(kbase + tok * D + 16 * kh + 8 * h) : bf16x8{};
  };
  const int64_t gstride = (int64_t)NW * TG;
  bf16x8 knext[TB][2];
  if constexpr (PREF) {
#pragma unroll
    for (int tb = 0; tb < TB; tb++)
#pragma unroll
      for (int kh = 0; kh < 2; kh++) knext[tb][kh] = load_keys_at(t_begin + (int64_t)wave * TG, tb, kh);
  }

  for (int64_t base = t_begin + (int64_t)wave * TG; base < t_end; base += gstride) {
    auto load_keys = [&](int tb, int kh) __attribute__((always_inline)) { return load_keys_at(base, tb, kh); };
    f16x8 kf[TB][2];
    // ||K_n||^2 of this lane's tokens (lanes l and l ^ 32 hold the two halves of a key).
    float k2[TB];
    if constexpr (PREF) {
#pragma unroll
      for (int tb = 0; tb < TB; tb++) {
        k2[tb] = sumsq_bf16x8(knext[tb][0]) + sumsq_bf16x8(knext[tb][1]);
#pragma unroll
        for (int kh = 0; kh < 2; kh++) kf[tb][kh] = to_f16x8(knext[tb][kh]);
      }
      if (base + gstride < t_end) {
#pragma unroll
        for (int tb = 0; tb < TB; tb++)
#pragma unroll
          for (int kh = 0; kh < 2; kh++) knext[tb][kh] = load_keys_at(base + gstride, tb, kh);
      }
    } else {
#pragma unroll
      for (int tb = 0; tb < TB; tb++) {
        const bf16x8 k0 = load_keys_at(base, tb, 0), k1 = load_keys_at(base, tb, 1);
        k2[tb] = sumsq_bf16x8(k0) + sumsq_bf16x8(k1);
        kf[tb][0] = to_f16x8(k0);
        kf[tb][1] = to_f16x8(k1);
      }
    }

    f32x16 yacc[TB];
    float lsum[TB], shift[TB];
    auto clear = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int tb = 0; tb < TB; tb++) {
        lsum[tb] = 0.f;
        yacc[tb] = f32x16{};
      }
    };
    // Latents past M do not enter the softmax.
    auto mask = [&](int lb, f32x16 (&sc)[TB]) __attribute__((always_inline)) {
      if (ragged && lb == nlb - 1) {
#pragma unroll
        for (int v = 0; v < 16; v++)
          if (32 * lb + row32(v, h) >= a.M)
#pragma unroll
            for (int tb = 0; tb < TB; tb++) sc[tb][v] = -INFINITY;
      }
    };
    auto scores_fast = [&](int lb, f32x16 (&sc)[TB]) __attribute__((always_inline)) {
      const f16* qrow = qh + (32 * lb + col) * QHS + 8 * h;
      const f16x8 qa0 = *reinterpret_cast<const f16x8*>(qrow);
      const f16x8 qa1 = *reinterpret_cast<const f16x8*>(qrow + 16);
#pragma unroll
      for (int tb = 0; tb < TB; tb++) {
        sc[tb] = mfma_32x32_f16(qa0, kf[tb][0], f32x16{});
        sc[tb] = mfma_32x32_f16(qa1, kf[tb][1], sc[tb]);
      }
      __builtin_amdgcn_sched_barrier(kAllButMfma);
      keep_live(qa0);
      keep_live(qa1);
      mask(lb, sc);
    };
    // Exact-pass scores: bf16 keys against the hi and lo query parts (four chained MFMAs).
    bf16x8 kb[TB][2];
    auto scores_exact = [&](int lb, f32x16 (&sc)[TB]) __attribute__((always_inline)) {
      const bf16* qrow = qsrc + (int64_t)(32 * lb + col) * kQRow<bf16> * D + 8 * h;
      const bf16x8 hi0 = *reinterpret_cast<const bf16x8*>(qrow);
      const bf16x8 hi1 = *reinterpret_cast<const bf16x8*>(qrow + 16);
      const bf16x8 lo0 = *reinterpret_cast<const bf16x8*>(qrow + D);
      const bf16x8 lo1 = *reinterpret_cast<const bf16x8*>(qrow + D + 16);
#pragma unroll
      for (int tb = 0; tb < TB; tb++) {
        sc[tb] = mfma_32x32(hi0, kb[tb][0], f32x16{});
        sc[tb] = mfma_32x32(hi1, kb[tb][1], sc[tb]);
        sc[tb] = mfma_32x32(lo0, kb[tb][0], sc[tb]);
        sc[tb] = mfma_32x32(lo1, kb[tb][1], sc[tb]);
      }
      __builtin_amdgcn_sched_barrier(kAllButMfma);
      keep_live(hi0);
      keep_live(hi1);
      keep_live(lo0);
      keep_live(lo1);
      mask(lb, sc);
    };
    // Probabilities (shifted by the token's maximum in the exact pass), their sums and P.V.
    auto accumulate = [&](auto EXACT) __attribute__((always_inline)) {
      for (int lb = 0; lb < nlb; lb++) {
        const bf16x8 zb0 = load_rows32(zs, ZSTR, 32 * lb, 0, lane);
        const bf16x8 zb1 = load_rows32(zs, ZSTR, 32 * lb + 16, 0, lane);
        f32x16 sc[TB];
        if constexpr (decltype(EXACT)::value)
          scores_exact(lb, sc);
        else
          scores_fast(lb, sc);
#pragma unroll
        for (int tb = 0; tb < TB; tb++) {
#pragma unroll
          for (int v = 0; v < 16; v++) {
            if constexpr (decltype(EXACT)::value)
              sc[tb][v] = exp2_fast(sc[tb][v] - shift[tb]);
            else
              sc[tb][v] = exp2_fast(sc[tb][v]);
          }
          const bf16x8 p0 = pack32(sc[tb], 0), p1 = pack32(sc[tb], 1);
          lsum[tb] = Ops<bf16, 32>::osum(p1, Ops<bf16, 32>::osum(p0, lsum[tb]));
          yacc[tb] = mfma_32x32(zb0, p0, yacc[tb]);
          yacc[tb] = mfma_32x32(zb1, p1, yacc[tb]);
          __builtin_amdgcn_sched_barrier(kAllButMfma);
          keep_live(p0);
          keep_live(p1);
        }
        keep_live(zb0);
        keep_live(zb1);
      }
    };

    // Zero-shift pass for one 32-token block, software-pipelined over the latent blocks as in the
    // partial kernels: step lb issues the score MFMAs of block lb+1 (the zero block past Mp after
    // the last) between fenced groups of block lb's exponentials and pack/sum work, then its P.V.
    // Token sums on the matrix unit (see sum_selector) when the register budget allows: with 12
    // waves, or with 16 waves and no key prefetch; otherwise they stay on v_dot2.
    constexpr bool kSumsOnMfma = NW <= 12 || !PREF;
    f32x4 ls4 = f32x4{0.f, 0.f, 0.f, 0.f};
    auto accumulate_fast_pipelined = [&]() __attribute__((always_inline)) {
      if constexpr (TB == 1) {
        // Selector as the A operand: lane l supplies row l % 16 of k-slice l / 16.
        const bf16x8 dsel = kSumsOnMfma ? sum_selector(lane) : bf16x8{};
        auto fence = []() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };
        struct QOp { f16x8 a, b; };
        // The lane's query row in block 0 as an LDS address; block lb adds a wave-uniform offset
        // (one 32-bit add per block instead of a generic-pointer multiply-add).
        typedef __attribute__((address_space(3))) const f16x8 lds_f16x8;
        typedef __attribute__((address_space(3))) const char lds_char;
        lds_char* const qlane = (lds_char*)(qh + col * QHS + 8 * h);
        auto load_q = [&](int lb) __attribute__((always_inline)) {
          lds_f16x8* qrow = (lds_f16x8*)(qlane + lb * (32 * QHS * (int)sizeof(f16)));
          return QOp{qrow[0], qrow[2]};
        };
        auto exps = [&](f32x16& x, int v0) __attribute__((always_inline)) {
#pragma unroll
          for (int v = 0; v < 4; v++) x[v0 + v] = exp2_fast(x[v0 + v]);
        };
        // qn holds the query operands of block lb+1 on entry and of block lb+2 on exit. mask: the
        // final latent block when M is not a multiple of 32, whose rows past M are masked (a
        // wave-uniform branch, so the other blocks pay no VALU for it).
        // FIRST: block 0, whose P.V product and token sums start from a zero accumulator (an inline
        // constant of the MFMA), so the accumulators need no clearing per wave group.
        auto step = [&](auto FIRST, bool mask, int lb, f32x16& cu, f32x16& nx, QOp& qn) __attribute__((always_inline)) {
          constexpr bool kFirst = decltype(FIRST)::value;
          const bf16x8 zb0 = load_rows32(zs, ZSTR, 32 * lb, 0, lane);
          const bf16x8 zb1 = load_rows32(zs, ZSTR, 32 * lb + 16, 0, lane);
          if (mask) {
#pragma unroll
            for (int v = 0; v < 16; v++)
              if (32 * lb + row32(v, h) >= a.M) cu[v] = -INFINITY;
          }
          nx = mfma_32x32_f16(qn.a, kf[0][0], f32x16{});
          fence();
          exps(cu, 0);
          fence();
          nx = mfma_32x32_f16(qn.b, kf[0][1], nx);
          fence();
          keep_live(qn.a);
          keep_live(qn.b);
          qn = load_q(lb + 2 <= nlb ? lb + 2 : nlb);
          exps(cu, 4);
          const bf16x8 p0 = pack32(cu, 0);
          if constexpr (!kSumsOnMfma) lsum[0] = Ops<bf16, 32>::osum(p0, lsum[0]);
          fence();
          yacc[0] = mfma_32x32(zb0, p0, kFirst ? f32x16{} : yacc[0]);
          if constexpr (kSumsOnMfma) ls4 = mfma_32k(dsel, p0, kFirst ? f32x4{} : ls4);
          fence();
          keep_live(p0);
          keep_live(zb0);
          exps(cu, 8);
          exps(cu, 12);
          const bf16x8 p1 = pack32(cu, 1);
          if constexpr (!kSumsOnMfma) lsum[0] = Ops<bf16, 32>::osum(p1, lsum[0]);
          fence();
          yacc[0] = mfma_32x32(zb1, p1, yacc[0]);
          if constexpr (kSumsOnMfma) ls4 = mfma_32k(dsel, p1, ls4);
          fence();
          keep_live(p1);
          keep_live(zb1);
        };
        f32x16 sa, sb;
        {
          const QOp q0 = load_q(0);
          sa = mfma_32x32_f16(q0.a, kf[0][0], f32x16{});
          sa = mfma_32x32_f16(q0.b, kf[0][1], sa);
          fence();
          keep_live(q0.a);
          keep_live(q0.b);
        }
        QOp qn = load_q(1);
        // Pairs of blocks (the scores alternate between sa and sb), then an odd last block.
        if (nlb >= 2) {
          step(std::true_type{}, false, 0, sa, sb, qn);
          step(std::false_type{}, ragged && nlb == 2, 1, sb, sa, qn);
          int lb = 2;
          for (; lb + 2 <= nlb; lb += 2) {
            step(std::false_type{}, false, lb, sa, sb, qn);
            step(std::false_type{}, ragged && lb + 2 == nlb, lb + 1, sb, sa, qn);
          }
          if (lb < nlb) step(std::false_type{}, ragged, lb, sa, sb, qn);
        } else {
          step(std::true_type{}, ragged, 0, sa, sb, qn);
        }
        if constexpr (kSumsOnMfma) {
          // Token t = l % 32 sums to column t % 16 of rows 0-7 (t < 16) or 8-15 (t >= 16): lane
          // t (t < 16) or t + 16, slot 0. Counted once, on the half h = 0.
          const float lt = shfl(ls4[0], col < 16 ? col : col + 16);
          lsum[0] = h == 0 ? lt : 0.f;
        }
      }
    };

    // The pipelined pass starts its accumulators from zero itself; the others are cleared.
#pragma unroll
    for (int tb = 0; tb < TB; tb++) lsum[tb] = 0.f;
    bool ok = a.force_exact == 0;
    // Routing bound (kRouteBound): a group holding a token beyond it takes the exact pass at once.
#pragma unroll
    for (int tb = 0; tb < TB; tb++) ok = ok && qmax2 * sum_xor32(k2[tb]) <= kRouteBound * kRouteBound;
    ok = __all(ok);
    if (ok) {
      if constexpr (TB == 1) {
        accumulate_fast_pipelined();
      } else {
        clear();
        accumulate(std::false_type{});
      }
    }

    // Within the routing bound every logit of the pass lies in [-kRouteBound, kRouteBound], so each
    // probability is within 2^+-kRouteBound and the row sum l of up to Mp of them within [2^-80,
    // 2^100]; a sum outside that range means a key beyond fp16 range (or NaN). The accumulator is
    // then at most 2^(kRouteBound + 10) max |Z|, finite for the inputs the library takes (it checks
    // no accumulator: where it would overflow, so would the exact pass's Z).
#pragma unroll
    for (int tb = 0; tb < TB; tb++) {
      const float l = sum_xor32(lsum[tb]);
      ok = ok && l >= 0x1p-80f && l <= 0x1p100f;
    }
    if (!__all(ok)) {
#pragma unroll
      for (int tb = 0; tb < TB; tb++)
#pragma unroll
        for (int kh = 0; kh < 2; kh++) kb[tb][kh] = load_keys(tb, kh);
#pragma unroll
      for (int tb = 0; tb < TB; tb++) shift[tb] = -INFINITY;
      for (int lb = 0; lb < nlb; lb++) {
        f32x16 sc[TB];
        scores_exact(lb, sc);
#pragma unroll
        for (int tb = 0; tb < TB; tb++)
#pragma unroll
          for (int v = 0; v < 16; v++) shift[tb] = fmaxf(shift[tb], sc[tb][v]);
      }
#pragma unroll
      for (int tb = 0; tb < TB; tb++) {
        shift[tb] = max_xor32(shift[tb]);
        if (shift[tb] == -INFINITY) shift[tb] = 0.f;
      }
      clear();
      accumulate(std::true_type{});
    }

    // Y = yacc / l. The P.V product is computed transposed (Z^T P), so result slot v of lane l
    // holds dim row32(v, h) of token l % 32 of its block: four runs of four consecutive dims, each
    // stored as one 8-byte write, and the token's sum is the lane's own (plus its partner l ^ 32).
#pragma unroll
    for (int tb = 0; tb < TB; tb++) {
      const float inv = __builtin_amdgcn_rcpf(sum_xor32(lsum[tb]));  // 1 ulp, then rounded to bf16
      const int64_t tok = base + 32 * tb + col;
      if (tok < t_end) {
#pragma unroll
        for (int gq = 0; gq < 4; gq++) {
          bf16x4 o;
#pragma unroll
          for (int i = 0; i < 4; i++) o[i] = (bf16)(yacc[tb][4 * gq + i] * inv);
          *reinterpret_cast<bf16x4*>(obase + tok * D + row32(4 * gq, h)) = o;
        }
      }
    }
  }
}

}  // namespace

// ------------------------------------------------------------------------------------------
// Launchers.

// Dynamic LDS above 64 KiB has to be allowed per kernel (gfx950 has 160 KiB per workgroup).
template <typename F>
static hipError_t allow_lds(F* fn, size_t lds) {
  if (lds <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

// LDS of the partial kernel: key tiles, value tiles (VLO: and their lo parts), the per-token key
// factors of bf16 synthesis (FK), one flag (in 16 bytes), a per-wave maximum (up to 16 waves) and a
// per-row maximum of a stage.
template <typename T, int D, int STG, bool VLO, bool FK>
static size_t partial_lds_t() {
  constexpr int CH = 16 / sizeof(T);
  return (size_t)(2 * STG * (D + CH) + (VLO ? 4 : 2) * RowTile<T, D>::elems(STG)) * sizeof(T) +
         (FK ? 2 * STG * sizeof(float) : 0) + 16 + (16 + STG) * sizeof(float);
}

template <typename T, int D, int LPW, int NW, bool SYNTH, int STG, bool HILO>
static hipError_t launch_partial_t(const PartialArgs& a, int grid_x, int grid_y, hipStream_t st) {
  const size_t lds = partial_lds_t<T, D, STG, HILO && SYNTH, SYNTH && sizeof(T) == 2>();
  hipError_t e = allow_lds(partial_kernel<T, D, LPW, NW, SYNTH, STG, HILO>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((partial_kernel<T, D, LPW, NW, SYNTH, STG, HILO>), dim3(grid_x, grid_y), dim3(NW * 64), lds, st, a);
  return hipGetLastError();
}

// bf16 calls with `hilo` set (the backward's recompute) take the hi/lo P.V instance.
template <typename T, int D, int LPW, int NW, bool SYNTH, int STG>
static hipError_t launch_partial_h(const PartialArgs& a, int grid_x, int grid_y, hipStream_t st) {
  if constexpr (sizeof(T) == 2)
    if (a.hilo) return launch_partial_t<T, D, LPW, NW, SYNTH, STG, true>(a, grid_x, grid_y, st);
  return launch_partial_t<T, D, LPW, NW, SYNTH, STG, false>(a, grid_x, grid_y, st);
}

// Partial-kernel variants (latents per wave, waves per workgroup, tokens per stage); see
// partial_plan_shape. The 16-wave variant is built for bf16 only (fp32 operands need more than the
// 128 registers per lane that 16 waves leave).
template <typename T, int D, bool SYNTH>
static hipError_t launch_partial_d(const PartialArgs& a, int plan, int gx, int gy, hipStream_t st) {
  switch (plan) {
    case 0: return launch_partial_h<T, D, 16, 4, SYNTH, 128>(a, gx, gy, st);
    case 1: return launch_partial_h<T, D, 32, 4, SYNTH, 128>(a, gx, gy, st);
    case 2: return launch_partial_h<T, D, 32, 8, SYNTH, 128>(a, gx, gy, st);
    case 3:
      if constexpr (sizeof(T) == 2) return launch_partial_h<T, D, 32, 16, SYNTH, 256>(a, gx, gy, st);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_partial(const PartialArgs& a, int dtype, int D, bool synth, int plan, int gx, int gy,
                          hipStream_t st) {
  if (dtype == 1) {
    if (D == 32) return synth ? launch_partial_d<bf16, 32, true>(a, plan, gx, gy, st) : launch_partial_d<bf16, 32, false>(a, plan, gx, gy, st);
    return synth ? launch_partial_d<bf16, 16, true>(a, plan, gx, gy, st) : launch_partial_d<bf16, 16, false>(a, plan, gx, gy, st);
  }
  if (D == 32) return synth ? launch_partial_d<float, 32, true>(a, plan, gx, gy, st) : launch_partial_d<float, 32, false>(a, plan, gx, gy, st);
  return synth ? launch_partial_d<float, 16, true>(a, plan, gx, gy, st) : launch_partial_d<float, 16, false>(a, plan, gx, gy, st);
}

template <typename T, int D, bool GATE>
static hipError_t launch_merge_t(const MergeArgs& a, int BH, hipStream_t st) {
  const int gx = (a.Mout * D + 255) / 256;
  const size_t lds = (size_t)(256 / D) * a.nchunk * sizeof(float);
  hipError_t e = allow_lds(merge_kernel<T, D, GATE>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((merge_kernel<T, D, GATE>), dim3(gx, BH), dim3(256), lds, st, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_query_prep_t(const QueryPrepArgs& a, int BH, hipStream_t st) {
  const int gx = (a.Mout * D + 255) / 256;
  hipLaunchKernelGGL((query_prep_kernel<T, D>), dim3(gx, BH), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_query_prep(const QueryPrepArgs& a, int dtype, int D, int BH, hipStream_t st) {
  if (dtype == 1) return D == 32 ? launch_query_prep_t<bf16, 32>(a, BH, st) : launch_query_prep_t<bf16, 16>(a, BH, st);
  return D == 32 ? launch_query_prep_t<float, 32>(a, BH, st) : launch_query_prep_t<float, 16>(a, BH, st);
}

hipError_t launch_merge(const MergeArgs& a, int dtype, int D, bool gate, int BH, hipStream_t st) {
  if (dtype == 1) {
    if (D == 32) return gate ? launch_merge_t<bf16, 32, true>(a, BH, st) : launch_merge_t<bf16, 32, false>(a, BH, st);
    return gate ? launch_merge_t<bf16, 16, true>(a, BH, st) : launch_merge_t<bf16, 16, false>(a, BH, st);
  }
  if (D == 32) return gate ? launch_merge_t<float, 32, true>(a, BH, st) : launch_merge_t<float, 32, false>(a, BH, st);
  return gate ? launch_merge_t<float, 16, true>(a, BH, st) : launch_merge_t<float, 16, false>(a, BH, st);
}

template <typename T, int D>
static size_t decode_lds_t(int Mp, int NW) {
  constexpr int CH = 16 / sizeof(T);
  return (size_t)(Mp * (kQParts<T> * D + CH) + RowTile<T, D>::elems(Mp)) * sizeof(T) + NW * sizeof(float);
}

template <typename T, int D, int NW, int TB>
static hipError_t launch_decode_t(const DecodeArgs& a, int gx, int gy, hipStream_t st) {
  const size_t lds = decode_lds_t<T, D>(a.Mp, NW);
  hipError_t e = allow_lds(decode_kernel<T, D, NW, TB>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_kernel<T, D, NW, TB>), dim3(gx, gy), dim3(NW * 64), lds, st, a);
  return hipGetLastError();
}

// Waves per workgroup and 16-token blocks per wave group: (8, 4), (12, 4) or (16, 2).
// fp32 runs use (8, 4) or (16, 2): four fp32 token blocks do not fit the register budget of 12 waves.
template <typename T, int D>
static hipError_t launch_decode_d(const DecodeArgs& a, int nw, int gx, int gy, hipStream_t st) {
  if (nw == 16) return launch_decode_t<T, D, 16, 2>(a, gx, gy, st);
  if constexpr (sizeof(T) == 2) {
    if (nw == 12) return launch_decode_t<T, D, 12, 4>(a, gx, gy, st);
  }
  if (nw != 8) return hipErrorInvalidValue;
  return launch_decode_t<T, D, 8, 4>(a, gx, gy, st);
}

static size_t decode_wide_lds(int Mp) {
  // fp16 query rows (and a zero block), the Z tile, and one float per wave (up to 16).
  return (size_t)(Mp + 32) * (32 + 8) * sizeof(_Float16) + (size_t)RowTile<bf16, 32, kDecodeZPad>::elems(Mp) * sizeof(bf16) +
         16 * sizeof(float);
}

template <int NW, int TB, bool PREF = true>
static hipError_t launch_decode_wide_t(const DecodeArgs& a, int gx, int gy, hipStream_t st) {
  const size_t lds = decode_wide_lds(a.Mp);
  hipError_t e = allow_lds(decode_wide_kernel<NW, TB, PREF>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_wide_kernel<NW, TB, PREF>), dim3(gx, gy), dim3(NW * 64), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, int D, int nw, int gx, int gy, hipStream_t st) {
  if (dtype == 1 && D == 32) {
    // 12 or 16 waves: one 32-token block per wave group with the pipelined zero-shift pass (16
    // waves: keys loaded at the group's start, leaving the registers for the token sums on the
    // matrix unit); 8 waves: two blocks per group, not pipelined.
    switch (nw) {
      case 8: return launch_decode_wide_t<8, 2>(a, gx, gy, st);
      case 12: return launch_decode_wide_t<12, 1>(a, gx, gy, st);
      case 16: return launch_decode_wide_t<16, 1, false>(a, gx, gy, st);
      default: return hipErrorInvalidValue;
    }
  }
  if (dtype == 1) return launch_decode_d<bf16, 16>(a, nw, gx, gy, st);
  return D == 32 ? launch_decode_d<float, 32>(a, nw, gx, gy, st) : launch_decode_d<float, 16>(a, nw, gx, gy, st);
}

size_t decode_lds_bytes(int dtype, int D, int Mp, int nw) {
  if (dtype == 1) return D == 32 ? decode_wide_lds(Mp) : decode_lds_t<bf16, 16>(Mp, nw);
  return D == 32 ? decode_lds_t<float, 32>(Mp, nw) : decode_lds_t<float, 16>(Mp, nw);
}


}  // namespace flarepp
