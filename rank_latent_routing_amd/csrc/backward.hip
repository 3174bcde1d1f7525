// HIP kernels of the FLARE++ mixer backward pass for gfx950 (CDNA4).
//
// Method: "FLARE++: Low-rank attention with attention-synthesized routing" (arXiv 2608.11519 v2).
// The mixer (Appendix A.1, Eq. 11) is three softmax routing calls (Section 3.2, Eq. 6 and Eq. 8)
// joined by the gate (Eq. 7) and the normalization N0 (Eq. 5). Its cotangents follow the SDPA
// backward of Appendix B.5 (Eq. 46-49) call by call, in reverse order: decode, encode, gate,
// synthesis, N0. For one call o = softmax(q k^T / sqrt(D)) v with cotangent do and probabilities P:
//   dP = do v^T,  c = rowsum(P * dP) = <do, o>,  dS = P * (dP - c),
//   dq = dS k / sqrt(D),  dk = dS^T q / sqrt(D),  dv = P^T do.
// The host first recomputes the synthesis and encode calls and keeps every softmax row's normalizer
// L in the logits' log2 units (the logits carry c = log2(e)/sqrt(D)), so that each probability here
// is one exponential of a known logit, P = 2^(l - L), with no running maximum.
//
// Kernels (32x32x16 MFMAs with bf16 operands and fp32 accumulation; fp32 runs issue eight 32x32x2
// fp32 MFMAs per 32x32x16 step, with the same lane layout):
//   center       Zc = Z - mean_m Z, the decode call's dP operand (the shift cancels in dP - c).
//   decode       per token: the normalizer L_n and c_n = sum_m P dP of its softmax over latents (one
//                online pass), then the decode call's part of dK (a second pass), in fp32.
//   latent-side  one per call: the latent-indexed cotangents, which sum over tokens (decode: dZ and
//                dQ; encode: dQ; synthesis: dQseed), split over token chunks like the forward
//                partials. Each wave owns 32 latents; the chunk's token tiles pass through LDS.
//   reduce       the chunk sums plus the latent-sized steps between the calls: <dZ, Z>, the gate
//                and N0 of Qf, and the batch sums of the shared parameters.
//   token-side   the token-indexed cotangents, which sum over latents: dK (adding the decode part)
//                and dV from the encode call, dS from the synthesis call and N0. The latent tensors
//                of one (batch, head) stay in LDS; each wave takes blocks of 32 tokens.
//
// Precision. The cotangents are sums in which rounding errors of the operands do not cancel while the
// terms themselves largely do (each dS = P (dP - c) sums to zero along its softmax, and the values of
// a call cluster). Every operand the kernels compute (P, dS, c*Q, Zc, dZ, G, c*N0(S)) therefore
// enters the matrix unit as a bf16 pair hi + lo (hi = bf16(x), lo = bf16(x - hi), about 16
// significant bits); a product of two pairs takes the three MFMAs hi.hi + hi.lo + lo.hi. The inputs
// K, V, S, dY and the seeds are exact bf16. Each c is formed from the operands its dP products see
// (the decode call's from its own P and dP, the encode call's as <dZ, Z> with dZ as carried, the
// synthesis call's as <G, Qd> likewise), and the recomputed forward takes the exact hi/lo path, so
// that its normalizers match the logits computed here; its P.V products take P (and the synthesis
// values N0(S)) as pairs too, so that Z and Qd, and with them those c, are as exact as the products
// here. The token-side kernels of bf16 runs take fp16 instead (11 significant bits against bf16's
// 8) where a product over latents carries no cancellation: single fp16 operands, scaled by powers
// of two into fp16's range, and fp16 pairs (about 22 bits) in place of the bf16 pairs elsewhere, so
// that their latent tensors still fit in LDS (see each kernel).
//
// Layout of the 32x32x16 MFMA C[i][j] += sum_k A[i][k] B[k][j]: lane l supplies row l % 32 of A and
// column l % 32 of B with k = 8 (l / 32) + e (e = 0..7) and receives column l % 32, rows
// row32(v, l / 32) (v = 0..15). The 16 result slots of a tile, taken eight at a time (split), are
// directly the B operand of a product that sums over the tile's rows; the matching A operand comes
// from LDS with transposed reads (krows), rows in the same row32 order.
#include <hip/hip_runtime.h>
#include <cstdint>
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace flarepp {
namespace {

typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr float kLn2 = 0.6931471805599453f;

// Rows of D elements in LDS whose 16-byte chunks are permuted by an XOR with (row / RPB) % CPR, where
// RPB rows span the 64 banks: the row reads of 32 lanes (32 rows, one chunk each) and the transposed
// reads (4 rows x 32 bytes per group of 16 lanes) then touch distinct banks.
template <typename T, int D>
struct Swz {
  static constexpr int CH = 16 / sizeof(T);      // elements per chunk
  static constexpr int CPR = D / CH;             // chunks per row
  static constexpr int RPB = 256 / (16 * CPR);   // rows per 256 bytes
  __device__ static int off(int row, int col) {
    return row * D + (((col / CH) ^ ((row / RPB) % CPR)) * CH) + (col % CH);
  }
};

// Position of latent (or token) m in a stats array laid out so that lane half h of a 32-block reads
// the 16 values of its result slots, rows row32(v, h), as one contiguous run.
__device__ __forceinline__ int stat_pos(int m) {
  const int r = m & 31;
  return (m & ~31) + 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
}

// Element offsets, inside one block of 32 tile rows, of what a lane reads: the row operand (row l % 32,
// dims 16 kk + 8 (l / 32) .. + 7; fp32 as two 4-element chunks) and the transposed A operand of one
// 16-row k block (bf16: the two 4 x 16 transposed reads; fp32: its eight elements). The swizzle's
// XOR term depends on a row only through (row / RPB) % CPR, the same in every block of 16 rows, so
// these offsets serve every block: block b of 32 rows starts 32 b D elements further, k block t of
// a 32-row block 16 t D further.
template <typename T, int D>
struct LaneOffs {
  int row[D / 16][2];
  int kr[8];
};
template <typename T, int D>
__device__ __forceinline__ LaneOffs<T, D> lane_offsets(int lane) {
  using S = Swz<T, D>;
  LaneOffs<T, D> o;
  const int hh = lane >> 5, l = lane & 31;
#pragma unroll
  for (int kk = 0; kk < D / 16; kk++) {
    o.row[kk][0] = S::off(l, 16 * kk + 8 * hh);
    o.row[kk][1] = S::off(l, 16 * kk + 8 * hh + 4);
  }
  if constexpr (sizeof(T) == 2) {
    const int i = lane & 15, cb = ((lane >> 4) & 1) & (D / 16 - 1);
    const int col = 16 * cb + 4 * (i & 3);
    o.kr[0] = S::off(4 * hh + (i >> 2), col);
    o.kr[1] = S::off(8 + 4 * hh + (i >> 2), col);
#pragma unroll
    for (int e = 2; e < 8; e++) o.kr[e] = 0;
  } else {
#pragma unroll
    for (int e = 0; e < 8; e++) o.kr[e] = S::off(row32(e, hh), l & (D - 1));
  }
  return o;
}

// Operands of one 32x32x16 step. Op holds the eight k values of a lane; Pair is an operand with its
// rounding residual (bf16) or the operand alone (fp32).
template <typename T>
struct Frag;

template <>
struct Frag<bf16> {
  using Op = bf16x8;
  static constexpr bool kLo = true;
  struct Pair {
    Op h, l;
  };
  __device__ static Op zero() { return Op{}; }
  __device__ static f32x16 mma(const Op& a, const Op& b, const f32x16& c) { return mfma_32x32(a, b, c); }
  // Eight values as a pair: hi = the upper 16 bits of each value (bf16 by truncation), lo = the exact
  // residual x - hi rounded to bf16; hi + lo keeps about 16 significant bits. Two values share one
  // byte permute (hi) and one packed conversion (lo).
  __device__ static Pair split8(const float* v) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint32_t b0 = __float_as_uint(v[2 * i]), b1 = __float_as_uint(v[2 * i + 1]);
      h[i] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
      const f32x2 r = {v[2 * i] - __uint_as_float(b0 & 0xffff0000u), v[2 * i + 1] - __uint_as_float(b1 & 0xffff0000u)};
      l[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
    }
    return Pair{__builtin_bit_cast(Op, h), __builtin_bit_cast(Op, l)};
  }
  // Slots 8t .. 8t + 7 of a result tile as a pair.
  __device__ static Pair split(const f32x16& x, int t) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; e++) v[e] = x[8 * t + e];
    return split8(v);
  }
  __device__ static void to_float(const Op& o, float* x) {
#pragma unroll
    for (int e = 0; e < 8; e++) x[e] = (float)o[e];
  }
  __device__ static Op gload(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
  // The row operand of 32-row block `blk` (lane offsets o), k block kk.
  template <int D>
  __device__ static Op row_at(const bf16* blk, const LaneOffs<bf16, D>& o, int kk) {
    return *reinterpret_cast<const bf16x8*>(blk + o.row[kk][0]);
  }
  // The transposed A operand of the 16-row k block starting at `blk`: lane l gets its rows row32(e,
  // l / 32) of column l % 32 (D = 16: column l % 16; the upper 16 result rows then repeat the lower
  // ones and are not used).
  template <int D>
  __device__ static Op krows_at(const bf16* blk, const LaneOffs<bf16, D>& o) {
    const bf16x4 lo = lds_read_tr4(blk + o.kr[0]);
    const bf16x4 hi = lds_read_tr4(blk + o.kr[1]);
    Op r;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      r[e] = lo[e];
      r[4 + e] = hi[e];
    }
    return r;
  }
};

template <>
struct Frag<float> {
  using Op = f32x8;
  static constexpr bool kLo = false;
  struct Pair {
    Op h;
  };
  __device__ static Op zero() { return Op{}; }
  // Step e covers k = e (lanes 0-31) and k = 8 + e (lanes 32-63) of the 32x32x16 layout.
  __device__ static f32x16 mma(const Op& a, const Op& b, const f32x16& c) {
    f32x16 r = c;
#pragma unroll
    for (int e = 0; e < 8; e++) r = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], r, 0, 0, 0);
    return r;
  }
  __device__ static Pair split(const f32x16& x, int t) {
    Pair p;
#pragma unroll
    for (int e = 0; e < 8; e++) p.h[e] = x[8 * t + e];
    return p;
  }
  __device__ static Pair split8(const float* v) {
    Pair p;
#pragma unroll
    for (int e = 0; e < 8; e++) p.h[e] = v[e];
    return p;
  }
  __device__ static void to_float(const Op& o, float* x) {
#pragma unroll
    for (int e = 0; e < 8; e++) x[e] = o[e];
  }
  __device__ static Op gload(const float* p) {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(p), hi = *reinterpret_cast<const f32x4*>(p + 4);
    return Op{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  template <int D>
  __device__ static Op row_at(const float* blk, const LaneOffs<float, D>& o, int kk) {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(blk + o.row[kk][0]);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(blk + o.row[kk][1]);
    return Op{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  template <int D>
  __device__ static Op krows_at(const float* blk, const LaneOffs<float, D>& o) {
    Op r;
#pragma unroll
    for (int e = 0; e < 8; e++) r[e] = blk[o.kr[e]];
    return r;
  }
};

// Products of pairs and exact operands (the lo.lo term of two pairs is below fp32 resolution).
template <typename F>
__device__ __forceinline__ f32x16 mma_ep(const typename F::Op& a, const typename F::Pair& b, f32x16 c) {
  if constexpr (F::kLo) c = F::mma(a, b.l, c);
  return F::mma(a, b.h, c);
}
template <typename F>
__device__ __forceinline__ f32x16 mma_pe(const typename F::Pair& a, const typename F::Op& b, f32x16 c) {
  if constexpr (F::kLo) c = F::mma(a.l, b, c);
  return F::mma(a.h, b, c);
}
template <typename F>
__device__ __forceinline__ f32x16 mma_pp(const typename F::Pair& a, const typename F::Pair& b, f32x16 c) {
  if constexpr (F::kLo) {
    c = F::mma(a.l, b.h, c);
    c = F::mma(a.h, b.l, c);
  }
  return F::mma(a.h, b.h, c);
}
template <typename F>
__device__ __forceinline__ void hold(f32x16& acc, const typename F::Pair& x) {
  hold(acc, x.h);
  if constexpr (F::kLo) hold(acc, x.l);
}
// Pair reads of two swizzled tiles (hi, lo) at a lane's precomputed offsets.
template <typename F, int D, typename T, typename O>
__device__ __forceinline__ typename F::Pair row_pair_at(const T* bh, const T* bl, const O& o, int kk) {
  typename F::Pair p;
  p.h = F::template row_at<D>(bh, o, kk);
  if constexpr (F::kLo) p.l = F::template row_at<D>(bl, o, kk);
  return p;
}
template <typename F, int D, typename T, typename O>
__device__ __forceinline__ typename F::Pair krows_pair_at(const T* bh, const T* bl, const O& o) {
  typename F::Pair p;
  p.h = F::template krows_at<D>(bh, o);
  if constexpr (F::kLo) p.l = F::template krows_at<D>(bl, o);
  return p;
}
template <typename F, typename T>
__device__ __forceinline__ typename F::Pair gload_pair(const T* h, const T* l, int64_t o) {
  typename F::Pair p;
  p.h = F::gload(h + o);
  if constexpr (F::kLo) p.l = F::gload(l + o);
  return p;
}
template <typename F>
__device__ __forceinline__ typename F::Pair zero_pair() {
  typename F::Pair p;
  p.h = F::zero();
  if constexpr (F::kLo) p.l = F::zero();
  return p;
}

// x as a dtype pair: hi = T(x), lo = T(x - hi) (fp32: lo unused).
template <typename T>
__device__ __forceinline__ void store_pair(T* hi, T* lo, int64_t o, float x) {
  const T h = (T)x;
  hi[o] = h;
  if constexpr (sizeof(T) == 2) lo[o] = (T)(x - to_f(h));
}
template <typename T>
__device__ __forceinline__ float pair_value(const T* hi, const T* lo, int64_t o) {
  if constexpr (sizeof(T) == 2) return to_f(hi[o]) + to_f(lo[o]);
  return to_f(hi[o]);
}

template <typename T>
__device__ __forceinline__ void store4(T* dst, float x0, float x1, float x2, float x3) {
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<bf16x4*>(dst) = bf16x4{(bf16)x0, (bf16)x1, (bf16)x2, (bf16)x3};
  } else {
    *reinterpret_cast<f32x4*>(dst) = f32x4{x0, x1, x2, x3};
  }
}
template <typename T>
__device__ __forceinline__ void load4(const T* src, float* x) {
  if constexpr (sizeof(T) == 2) {
    const bf16x4 v = *reinterpret_cast<const bf16x4*>(src);
#pragma unroll
    for (int i = 0; i < 4; i++) x[i] = (float)v[i];
  } else {
    const f32x4 v = *reinterpret_cast<const f32x4*>(src);
#pragma unroll
    for (int i = 0; i < 4; i++) x[i] = v[i];
  }
}

// Stats of 32 latents (stat_pos order) for lane half hh: the 16 values of its result slots.
__device__ __forceinline__ f32x16 load_stats16(const float* base, int hh) {
  f32x16 out;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(base + 16 * hh + 4 * q);
#pragma unroll
    for (int i = 0; i < 4; i++) out[4 * q + i] = v[i];
  }
  return out;
}

// Exponent s of the power of two 2^s that brings x (> 0) below 2^14 (x 2^s < 2^14 <= 2x 2^s), clamped
// to [-100, 100] so that 2^s and 2^-s stay normal floats; 0 for x = 0. The fp16 operands of the
// bf16 backward are scaled by such factors into fp16's range and the results scaled back exactly.
__device__ __forceinline__ int pow2_below_2e14(float x) {
  int e = 0;
  (void)frexpf(x, &e);  // x < 2^e
  return x > 0.f ? (14 - e < -100 ? -100 : 14 - e > 100 ? 100 : 14 - e) : 0;
}

// ------------------------------------------------------------------------------------------
// Latent-side kernel of one routing call (Appendix B.5, Eq. 46-49, the sums over tokens).
//
// Per 32-token x 32-latent tile of a wave, with the score tile C[token][latent] (lane = latent):
//   l = X_n . Qr_m (log2 units), P = 2^(l - L), dP = W_n . Wr_m, dS = P (dP - c),
//   acc1[d][m] += sum_n X[n][d] dS[n][m]        and, for decode, acc0[d][m] += sum_n W[n][d] P[n][m].
// L and c are per token for decode (softmax over latents) and per latent for encode and synthesis
// (softmax over tokens). Synthesis scores the normalized keys c*N0(S) (a pair) against the seeds and
// takes dP = (c*N0(S)) . (G/c); the host scales acc1 by 1/sqrt(D) (decode, encode) or ln 2
// (synthesis).
//
// Workgroup = NW waves, latent group of 32*NW latents; grid x enumerates (chunk, latent group) with
// the groups of one chunk on the same XCD, y = b * H + h. The token tiles of a chunk pass through
// LDS in stages of bwd_stage_t tokens, double-buffered, the next stage's global loads issued
// before the current stage's compute. Tokens past the chunk's end load as zeros and are masked out
// of P.
template <typename T, int D, int CALL, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void bwd_latent_kernel(BwdLatentArgs a) {
  using F = Frag<T>;
  using Op = typename F::Op;
  using Pair = typename F::Pair;
  using Sw = Swz<T, D>;
  constexpr int ST = bwd_stage_t(sizeof(T) == 2, NW);
  constexpr int KB = D / 16;
  constexpr int NT = NW * 64;
  constexpr int CH = 16 / sizeof(T), CPR = D / CH;
  constexpr int NCH = ST * CPR;  // chunks per tensor per stage
  constexpr bool DEC = CALL == kBwdDecode, SYN = CALL == kBwdSynthesis;
  // bf16 decode call: both products over tokens take single fp16 operands (no cancellation in
  // either sum): K and dY scaled per (batch, head) into fp16's range (by max |K| and by
  // max_n |dY_n|_1 >= max |dY|), in fp16 copies of the stage tiles; P as 2^14 P (the score product
  // starts from 14 - L); dS scaled per (batch, head) from the bound
  // |dP - c| <= 2 max_n |dY_n|_1 max |Zc| below 2^14. The maxima come from the token decode kernel's
  // waves. The stores take the factors out exactly.
  constexpr bool H16 = DEC && sizeof(T) == 2;
  // Stage tiles: X and W (decode, encode), or the hi and lo parts of c*N0(S) (synthesis).
  constexpr int NLOAD = SYN ? NCH : 2 * NCH;
  constexpr int PER = (NLOAD + NT - 1) / NT;
  constexpr int QRS = SYN ? D : kQRow<T> * D;  // elements per query row

  extern __shared__ __align__(16) unsigned char smem[];
  T* xs = reinterpret_cast<T*>(smem);                          // [2][ST * D]
  T* ws = xs + 2 * ST * D;                                     // [2][ST * D]: W, or the lo part of X
  float* tst = reinterpret_cast<float*>(ws + 2 * ST * D);      // [2][2][ST] decode token stats
  f16* xs16 = reinterpret_cast<f16*>(tst + 4 * ST);             // H16: [2][ST * D] 2^sk K
  f16* ws16 = xs16 + 2 * ST * D;                                // H16: [2][ST * D] 2^sy dY
  float* mred = reinterpret_cast<float*>(ws16 + 2 * ST * D);    // H16: [2][NW] maxima

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
  const int lane = tid & 63, wave = tid >> 6, hh = lane >> 5;
  const int bh = blockIdx.y;
  const int64_t n_begin = (int64_t)chunk_id * a.chunk;
  const int64_t n_end = (n_begin + a.chunk < a.N) ? n_begin + a.chunk : a.N;
  const int nstage = (int)((n_end - n_begin + ST - 1) / ST);
  const int lat0 = (lg * NW + wave) * 32;
  const bool active = lat0 < a.Mp;
  const int lrow = lat0 + (lane & 31);
  const float c_scale = kLog2e * rsqrtf((float)D);
  const LaneOffs<T, D> lofs = lane_offsets<T, D>(lane);

  const T* xbase = reinterpret_cast<const T*>(a.X) + (int64_t)bh * a.N * D;
  const T* wbase = SYN ? xbase : reinterpret_cast<const T*>(a.W) + (int64_t)bh * a.N * D;

  // Latent operands (B of the score and dP products): lane l holds dims 16 kk + 8 (l / 32) .. + 7 of
  // latent lrow. Synthesis: the seeds (exact); otherwise c*Q as a pair. Wr is always a pair.
  Pair qb[KB], wb[KB];
  float Ll = 0.f, Lc = 0.f;
#pragma unroll
  for (int kk = 0; kk < KB; kk++) {
    qb[kk] = zero_pair<F>();
    wb[kk] = zero_pair<F>();
  }
  if (active) {
    const int64_t wo = ((int64_t)bh * a.Mp + lrow) * D;
#pragma unroll
    for (int kk = 0; kk < KB; kk++) {
      if constexpr (SYN) {
        if (lrow < a.M)
          qb[kk].h = F::gload(reinterpret_cast<const T*>(a.Qr) + ((int64_t)(bh % a.H) * a.M + lrow) * D + 16 * kk + 8 * hh);
      } else {
        const T* q = reinterpret_cast<const T*>(a.Qr) + ((int64_t)bh * a.Mp + lrow) * QRS + 16 * kk + 8 * hh;
        qb[kk].h = F::gload(q);
        if constexpr (F::kLo) qb[kk].l = F::gload(q + D);
      }
      wb[kk] = gload_pair<F>(reinterpret_cast<const T*>(a.Wr), reinterpret_cast<const T*>(a.Wr_lo),
                             wo + 16 * kk + 8 * hh);
    }
    if constexpr (!DEC) {
      Ll = a.ll[(int64_t)bh * a.Mp + lrow];
      Lc = a.lc[(int64_t)bh * a.Mp + lrow];
    }
  }
  // Encode and synthesis: the lane's latent has one L and one c; the products start from them
  // (negated, in every slot), so they come out as l - L and dP - c.
  f32x16 negL, negC;
#pragma unroll
  for (int v = 0; v < 16; v++) {
    negL[v] = -Ll;
    negC[v] = -Lc;
  }

  // H16: per-(batch, head) scales 2^sk (K), 2^sy (dY) and 2^sd (dS, with P as 2^14 P).
  int sk = 0, sy = 0, sd = 0;
  if constexpr (H16) {
    float m[2] = {0.f, 0.f};
    const float* tm = a.tmax + (int64_t)bh * a.ntmax * 2;
    for (int i = tid; i < a.ntmax; i += NT) {
#pragma unroll
      for (int j = 0; j < 2; j++) m[j] = fmaxf(m[j], tm[2 * i + j]);
    }
#pragma unroll
    for (int j = 0; j < 2; j++) {
      m[j] = wave_max(m[j]);
      if (lane == 0) mred[j * NW + wave] = m[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; j++) {
      m[j] = 0.f;
      for (int w = 0; w < NW; w++) m[j] = fmaxf(m[j], mred[j * NW + w]);
    }
    sk = pow2_below_2e14(m[0]);
    sy = pow2_below_2e14(m[1]);  // |dY| <= |dY_n|_1
    sd = pow2_below_2e14(16384.f * 2.f * m[1] * a.zmax[bh]);
  }
  const float fk = ldexpf(1.f, sk), fy = ldexpf(1.f, sy), fd = ldexpf(1.f, sd);

  Chunk rg[PER];
  float tsl = 0.f, tsc = 0.f;
  auto load = [&](int stage) __attribute__((always_inline)) {
    const int64_t s0 = n_begin + (int64_t)stage * ST;
#pragma unroll
    for (int i = 0; i < PER; i++) {
      const int q = tid + i * NT;
      Chunk v = {0u, 0u, 0u, 0u};
      if (q < NLOAD) {
        const bool isw = !SYN && q >= NCH;
        const int qq = isw ? q - NCH : q;
        const int64_t n = s0 + qq / CPR;
        if (n < n_end) v = *reinterpret_cast<const Chunk*>((isw ? wbase : xbase) + n * D + (qq % CPR) * CH);
      }
      rg[i] = v;
    }
    if constexpr (DEC) {
      if (tid < ST) {
        const int64_t n = s0 + tid;
        tsl = n < n_end ? a.tl[(int64_t)bh * a.N + n] : INFINITY;
        tsc = n < n_end ? a.tc[(int64_t)bh * a.N + n] : 0.f;
      }
    }
  };
  auto store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PER; i++) {
      const int q = tid + i * NT;
      if constexpr (SYN) {
        // c * N0 of the synthesis key row (Section 3.2, Eq. 5) as a pair: the row's CPR chunks sit
        // in consecutive lanes.
        float x[CH];
        chunk_to_float<T>(rg[i], x);
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < CH; j++) ss += x[j] * x[j];
        ss = group_sum<CPR>(ss);
        const float sc = c_scale / sqrtf(ss * (1.0f / D) + kRmsEps);
        float hi[CH], lo[CH];
#pragma unroll
        for (int j = 0; j < CH; j++) {
          const float v = x[j] * sc;
          hi[j] = to_f((T)v);
          lo[j] = v - hi[j];
        }
        if (q < NLOAD) {
          const int o = buf * ST * D + Sw::off(q / CPR, (q % CPR) * CH);
          *reinterpret_cast<Chunk*>(xs + o) = float_to_chunk<T>(hi);
          if constexpr (F::kLo) *reinterpret_cast<Chunk*>(ws + o) = float_to_chunk<T>(lo);
        }
      } else {
        if (q < NLOAD) {
          const bool isw = q >= NCH;
          const int qq = isw ? q - NCH : q;
          const int o = buf * ST * D + Sw::off(qq / CPR, (qq % CPR) * CH);
          *reinterpret_cast<Chunk*>((isw ? ws : xs) + o) = rg[i];
          if constexpr (H16) {
            float x[CH];
            chunk_to_float<T>(rg[i], x);
            const float f = isw ? fy : fk;
            f16x8 h;
#pragma unroll
            for (int j = 0; j < CH; j++) h[j] = (f16)(x[j] * f);
            *reinterpret_cast<f16x8*>((isw ? ws16 : xs16) + o) = h;
          }
        }
      }
    }
    if constexpr (DEC) {
      if (tid < ST) {
        const int p = stat_pos(tid);
        // Negated: the decode products start from -L and -c (H16: 14 - L, so that P comes out as
        // 2^14 P).
        tst[(2 * buf) * ST + p] = (H16 ? 14.f : 0.f) - tsl;
        tst[(2 * buf + 1) * ST + p] = -tsc;
      }
    }
  };

  f32x16 acc0 = {}, acc1 = {};
  // MASKED: the chunk's last stage, whose tokens past nvalid are out of the softmax.
  // The 32-token sub-tiles go in pairs: the score and dP products of both are issued first; the
  // matrix unit then computes the second's while the vector unit exponentiates and splits the first.
  constexpr int NS = ST / 32;  // sub-tiles per stage
  constexpr int NPR = 2;       // sub-tiles per pair
  auto compute = [&](int buf, auto MASKED, int nvalid) __attribute__((always_inline)) {
    const T* xt = xs + buf * ST * D;
    const T* wt = ws + buf * ST * D;
#pragma unroll
    for (int g = 0; g < NS; g += NPR) {
    if (decltype(MASKED)::value && 32 * g >= nvalid) break;  // the rest of the last stage is empty
    f32x16 s_all[NPR], dp_all[NPR];
#pragma unroll
    for (int j = 0; j < NPR; j++) {
      const int sub = g + j;
      const int r0 = 32 * sub;
      // The products start from -L and -c: the tokens' (decode, negated in LDS) or the latent's.
      f32x16 s = negL, dp = negC;
      if constexpr (DEC) {
        s = load_stats16(tst + (2 * buf) * ST + r0, hh);
        dp = load_stats16(tst + (2 * buf + 1) * ST + r0, hh);
      }
      if constexpr (SYN) {
        Pair xa[KB];
#pragma unroll
        for (int kk = 0; kk < KB; kk++) {
          xa[kk] = row_pair_at<F, D>(xt + r0 * D, wt + r0 * D, lofs, kk);
          s = mma_pe<F>(xa[kk], qb[kk].h, s);
          dp = mma_pp<F>(xa[kk], wb[kk], dp);
        }
#pragma unroll
        for (int kk = 0; kk < KB; kk++) {
          hold<F>(s, xa[kk]);
          hold<F>(dp, xa[kk]);
        }
      } else {
        Op xa[KB], wa[KB];
#pragma unroll
        for (int kk = 0; kk < KB; kk++) {
          xa[kk] = F::template row_at<D>(xt + r0 * D, lofs, kk);
          wa[kk] = F::template row_at<D>(wt + r0 * D, lofs, kk);
          s = mma_ep<F>(xa[kk], qb[kk], s);
          dp = mma_ep<F>(wa[kk], wb[kk], dp);
        }
#pragma unroll
        for (int kk = 0; kk < KB; kk++) {
          hold(s, xa[kk]);
          hold(dp, wa[kk]);
        }
      }
      s_all[j] = s;
      dp_all[j] = dp;
    }
#pragma unroll
    for (int j = 0; j < NPR; j++) {
      const int r0 = 32 * (g + j);
      const f32x16& s = s_all[j];
      const f32x16& dp = dp_all[j];
      f32x16 P, dS;
#pragma unroll
      for (int v = 0; v < 16; v++) {
        float p = exp2_fast(s[v]);
        if constexpr (decltype(MASKED)::value)
          if (r0 + row32(v, hh) >= nvalid) p = 0.f;
        P[v] = p;
        dS[v] = H16 ? p * dp[v] * fd : p * dp[v];
      }
      if constexpr (H16) {
#pragma unroll
        for (int t = 0; t < 2; t++) {
          f16x8 dsk, pk;
#pragma unroll
          for (int e = 0; e < 8; e++) {
            dsk[e] = (f16)dS[8 * t + e];
            pk[e] = (f16)P[8 * t + e];
          }
          const f16x8 xk = __builtin_bit_cast(
              f16x8, F::template krows_at<D>(reinterpret_cast<const T*>(xs16 + buf * ST * D + (r0 + 16 * t) * D), lofs));
          acc1 = mfma_32x32_f16(xk, dsk, acc1);
          hold(acc1, xk);
          hold(acc1, dsk);
          const f16x8 wk = __builtin_bit_cast(
              f16x8, F::template krows_at<D>(reinterpret_cast<const T*>(ws16 + buf * ST * D + (r0 + 16 * t) * D), lofs));
          acc0 = mfma_32x32_f16(wk, pk, acc0);
          hold(acc0, wk);
          hold(acc0, pk);
        }
        continue;
      }
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const Pair dsp = F::split(dS, t);
        if constexpr (SYN) {
          const Pair xk = krows_pair_at<F, D>(xt + (r0 + 16 * t) * D, wt + (r0 + 16 * t) * D, lofs);
          acc1 = mma_pp<F>(xk, dsp, acc1);
          hold<F>(acc1, xk);
        } else {
          const Op xk = F::template krows_at<D>(xt + (r0 + 16 * t) * D, lofs);
          acc1 = mma_ep<F>(xk, dsp, acc1);
          hold(acc1, xk);
        }
        hold<F>(acc1, dsp);
        if constexpr (DEC) {
          const Op wk = F::template krows_at<D>(wt + (r0 + 16 * t) * D, lofs);
          const Pair pp = F::split(P, t);
          acc0 = mma_ep<F>(wk, pp, acc0);
          hold(acc0, wk);
          hold<F>(acc0, pp);
        }
      }
    }
    }
  };

  load(0);
  store(0);
  // Wait here for every global load so far (the latent operands above included). Without it the
  // compiler carries those loads into the loop as possibly outstanding and waits for them in the
  // middle of each stage's products, which also waits out the next stage's prefetch there
  // (vmcnt 0; lgkmcnt and expcnt left at their maxima).
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (int stage = 0; stage < nstage; stage++) {
    const int buf = stage & 1;
    if (stage + 1 < nstage) load(stage + 1);
    const int64_t left = n_end - (n_begin + (int64_t)stage * ST);
    if (active) {
      if (left < ST)
        compute(buf, std::true_type{}, (int)left);
      else
        compute(buf, std::false_type{}, ST);
    }
    if (stage + 1 < nstage) store(buf ^ 1);
    __syncthreads();
  }

  if (!active) return;
  // Result slot v of lane l: dim row32(v, l / 32) of latent lrow; four consecutive dims per store.
  // H16: less the factors 2^(sk + 14 + sd) (acc1) and 2^(sy + 14) (acc0).
  const int64_t prow = ((int64_t)bh * a.nchunk + chunk_id) * a.Mp + lrow;
  if constexpr (H16) {
    const float o1 = ldexpf(1.f, -(sk + 14 + sd)), o0 = ldexpf(1.f, -(sy + 14));
#pragma unroll
    for (int v = 0; v < 16; v++) {
      acc1[v] *= o1;
      acc0[v] *= o0;
    }
  }
#pragma unroll
  for (int gq = 0; gq < 4; gq++) {
    const int d0 = row32(4 * gq, hh);
    if (d0 < D) {
      *reinterpret_cast<f32x4*>(a.part1 + prow * D + d0) =
          f32x4{acc1[4 * gq], acc1[4 * gq + 1], acc1[4 * gq + 2], acc1[4 * gq + 3]};
      if constexpr (DEC)
        *reinterpret_cast<f32x4*>(a.part0 + prow * D + d0) =
            f32x4{acc0[4 * gq], acc0[4 * gq + 1], acc0[4 * gq + 2], acc0[4 * gq + 3]};
    }
  }
}

// ------------------------------------------------------------------------------------------
// Reductions. Each wave covers 64 consecutive (latent, channel) entries, 64 / D whole latent rows,
// so that a row's D channels sit in consecutive lanes for the row sums. With many chunks
// (BwdReduceArgs::split = 4) the four waves of a block share one such range, each summing a quarter
// of the chunk partials, and wave 0 adds the quarters in a fixed order and finishes the entries;
// with few (split = 1) each wave sums all chunks of its own range. Sums run with eight loads in
// flight, in an order fixed by the shapes alone, so the results are the same on every call.
template <int D>
__device__ __forceinline__ float row_sum(float v) {
#pragma unroll
  for (int o = 1; o < D; o <<= 1) v += shfl_xor(v, o);
  return v;
}

// p[c * stride] summed over c in [c0, c1): eight independent partial sums, combined pairwise.
__device__ __forceinline__ float strided_sum(const float* p, int64_t stride, int c0, int c1) {
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int c = c0;
  for (; c + 8 <= c1; c += 8) {
#pragma unroll
    for (int k = 0; k < 8; k++) s[k] += p[(int64_t)(c + k) * stride];
  }
#pragma unroll
  for (int k = 0; k < 7; k++)
    if (c + k < c1) s[k] += p[(int64_t)(c + k) * stride];
  return ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
}

// The same over the items j in [j0, j1) of runs of n items, run r starting at item (n + skip) r:
// item j sits at p[(j + (j / n) skip) * stride].
__device__ __forceinline__ float run_sum(const float* p, int64_t stride, int n, int skip, int j0, int j1) {
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int j = j0;
  for (; j + 8 <= j1; j += 8) {
#pragma unroll
    for (int k = 0; k < 8; k++) s[k] += p[(int64_t)(j + k + ((j + k) / n) * skip) * stride];
  }
#pragma unroll
  for (int k = 0; k < 7; k++)
    if (j + k < j1) s[k] += p[(int64_t)(j + k + ((j + k) / n) * skip) * stride];
  return ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
}

// How a reduction block's waves split the work: `part` of `split` parts of the chunks, for entry
// group `eg` of the block's 4 / split groups of 64 entries.
struct RedSplit {
  int part, eg, first;  // first: the wave's first entry
  __device__ RedSplit(int split) {
    const int wave = threadIdx.x >> 6, groups = 4 / split;
    part = wave / groups;
    eg = wave % groups;
    first = (blockIdx.x * groups + eg) * 64;
  }
  // The part [c0, c1) of n chunks this wave sums.
  __device__ int c0(int n, int split) const { return n * part / split; }
  __device__ int c1(int n, int split) const { return n * (part + 1) / split; }
};

// Adds the parts' values v of each lane's entry in a fixed order; the total is valid in the waves of
// part 0.
__device__ __forceinline__ float add_parts(float (*red)[64], float v, int split) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (split == 1) return v;
  red[wave][lane] = v;
  __syncthreads();
  return (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
}

// After the decode call: dZ = sum of the P^T dY partials (kept as a pair for the encode call), dQ_dec
// = sum of the dS^T K partials over sqrt(D), and the encode call's c_m = <dZ_m, Z_m> with dZ as the
// pair carries it.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_reduce_decode_kernel(BwdReduceArgs a) {
  __shared__ float red[2][4][64];
  const int bh = blockIdx.y;
  const RedSplit w(a.split);
  const int idx = w.first + (threadIdx.x & 63);
  const int row = idx / D, d = idx % D;
  const bool valid = row < a.M;
  const int64_t cs = (int64_t)a.Mp * D;
  const int64_t base = ((int64_t)bh * a.nchunk * a.Mp + row) * D + d;
  const int c0 = w.c0(a.nchunk, a.split), c1 = w.c1(a.nchunk, a.split);
  float z = valid ? strided_sum(a.part0 + base, cs, c0, c1) : 0.f;
  float q = valid ? strided_sum(a.part1 + base, cs, c0, c1) : 0.f;
  z = add_parts(red[0], z, a.split);
  q = add_parts(red[1], q, a.split);
  if (w.part != 0 || row >= a.Mp) return;  // whole rows
  q *= rsqrtf((float)D);
  const int64_t o = ((int64_t)bh * a.Mp + row) * D + d;
  T* zh = reinterpret_cast<T*>(a.dZop);
  T* zl = reinterpret_cast<T*>(a.dZop_lo);
  store_pair<T>(zh, zl, o, z);
  a.dZ32[o] = z;
  a.dQdec[o] = q;
  const float zr = pair_value<T>(zh, zl, o);
  const float e = row_sum<D>(valid ? zr * a.Z32[((int64_t)bh * a.M + row) * D + d] : 0.f);
  if (d == 0) a.ce[(int64_t)bh * a.Mp + row] = e;
}

// After the encode call: dQ = dQ_dec + dQ_enc; the gate Q = N0(Qf) + g Qd (Eq. 7) gives
// dQf = N0'(Qf)^T dQ (per (b, h), summed over the batch later), the gate's <dQ, Qd> and the
// synthesis call's cotangent G = g dQ (a pair G / c for the dP operand) with c_m = <G_m, Qd_m>
// (G as the pair carries it).
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_reduce_gate_kernel(BwdReduceArgs a) {
  __shared__ float red[4][64];
  const int bh = blockIdx.y, h = bh % a.H;
  const RedSplit w(a.split);
  const int idx = w.first + (threadIdx.x & 63);
  const int row = idx / D, d = idx % D;
  const bool valid = row < a.M;
  const int64_t cs = (int64_t)a.Mp * D;
  const int64_t base = ((int64_t)bh * a.nchunk * a.Mp + row) * D + d;
  float q = valid ? strided_sum(a.part1 + base, cs, w.c0(a.nchunk, a.split), w.c1(a.nchunk, a.split)) : 0.f;
  q = add_parts(red, q, a.split);
  if (w.part != 0 || row >= a.Mp) return;
  const int64_t o = ((int64_t)bh * a.Mp + row) * D + d;
  if (valid) q = a.dQdec[o] + q * rsqrtf((float)D);
  const float f = valid ? to_f(reinterpret_cast<const T*>(a.Qf)[((int64_t)h * a.M + row) * D + d]) : 0.f;
  const float ss = row_sum<D>(f * f);
  const float tq = row_sum<D>(f * q);
  const float r = 1.0f / sqrtf(ss * (1.0f / D) + kRmsEps);
  a.dQf_bh[o] = valid ? r * q - r * r * r * f * tq * (1.0f / D) : 0.f;
  const float qd = valid ? a.Qd32[((int64_t)bh * a.M + row) * D + d] : 0.f;
  const float rd = row_sum<D>(q * qd);
  const float gv = a.g[h];
  const float c_scale = kLog2e * rsqrtf((float)D);
  T* gh = reinterpret_cast<T*>(a.Gop);
  T* gl = reinterpret_cast<T*>(a.Gop_lo);
  store_pair<T>(gh, gl, o, valid ? gv * q / c_scale : 0.f);
  const float cg = row_sum<D>(pair_value<T>(gh, gl, o) * qd) * c_scale;
  if (d == 0) {
    a.cs[(int64_t)bh * a.Mp + row] = valid ? cg : 0.f;
    a.rowdot[(int64_t)bh * a.Mp + row] = valid ? rd : 0.f;
  }
}

// After the synthesis call: the cotangents of the parameters shared over the batch. dQseed is the
// sum over batch and chunks of the dS^T (c N0(S)) partials times ln 2 (= 1/(c sqrt(D))); dQf the batch
// sum of the per-(b, h) values; dg = sum over the batch of <dQ, Qd>. Grid x covers the M x D
// entries of one head (y); block 0 of each head also sums dg.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_reduce_synthesis_kernel(BwdReduceArgs a) {
  __shared__ float red[4][64];
  const int h = blockIdx.y;
  const RedSplit w(a.split);
  const int idx = w.first + (threadIdx.x & 63);
  const int row = idx / D, d = idx % D;
  if (blockIdx.x == 0) {
    __shared__ float part[4];
    float s = 0.f;
    for (int i = threadIdx.x; i < a.B * a.M; i += 256) {
      const int b = i / a.M, m = i % a.M;
      s += a.rowdot[(int64_t)(b * a.H + h) * a.Mp + m];
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) s += shfl_xor(s, o);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) a.dg[h] = (part[0] + part[1]) + (part[2] + part[3]);
  }
  const bool valid = row < a.M;
  const int64_t cs = (int64_t)a.Mp * D;
  // The partials of head h: nchunk chunks per batch element, the other heads' chunks in between.
  const int nb = a.B * a.nchunk;
  const float qs = add_parts(
      red, valid ? run_sum(a.part1 + ((int64_t)h * a.nchunk * a.Mp + row) * D + d, cs, a.nchunk,
                           (a.H - 1) * a.nchunk, w.c0(nb, a.split), w.c1(nb, a.split))
                 : 0.f, a.split);
  if (w.part != 0 || !valid) return;
  const float qf = strided_sum(a.dQf_bh + ((int64_t)h * a.Mp + row) * D + d, (int64_t)a.H * a.Mp * D, 0, a.B);
  const int64_t o = ((int64_t)h * a.M + row) * D + d;
  reinterpret_cast<T*>(a.dQseed)[o] = (T)(qs * kLn2);
  reinterpret_cast<T*>(a.dQf)[o] = (T)qf;
}

// ------------------------------------------------------------------------------------------
// Zc = Z - mean_m Z per (b, h), as a pair: one block per (b, h), the column sums through LDS. Each
// thread's rows go in batches of eight, loads ahead of the stores.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_center_kernel(BwdCenterArgs a) {
  constexpr int RPB = 256 / D;  // rows per pass
  __shared__ float part[256];
  const int bh = blockIdx.x;
  const int d = threadIdx.x % D, r0 = threadIdx.x / D;
  const float* z = a.Z32 + (int64_t)bh * a.M * D;
  const float s = strided_sum(z + (int64_t)r0 * D + d, (int64_t)RPB * D, 0, r0 < a.M ? (a.M - r0 + RPB - 1) / RPB : 0);
  part[threadIdx.x] = s;
  __syncthreads();
  float mean = 0.f;
  for (int r = 0; r < RPB; r++) mean += part[r * D + d];
  mean /= (float)a.M;
  T* oh = reinterpret_cast<T*>(a.Zc) + (int64_t)bh * a.Mp * D;
  T* ol = reinterpret_cast<T*>(a.Zc_lo) + (int64_t)bh * a.Mp * D;
  float mx = 0.f;
  for (int m0 = r0; m0 < a.Mp; m0 += 8 * RPB) {
    float zv[8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const int m = m0 + k * RPB;
      zv[k] = m < a.M ? z[(int64_t)m * D + d] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const int m = m0 + k * RPB;
      if (m < a.Mp) {
        const float zc = m < a.M ? zv[k] - mean : 0.f;
        store_pair<T>(oh, ol, (int64_t)m * D + d, zc);
        mx = fmaxf(mx, fabsf(zc));
      }
    }
  }
  if (a.zmax) {
    __syncthreads();  // every thread has read part[] above
    part[threadIdx.x] = mx;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if ((int)threadIdx.x < w) part[threadIdx.x] = fmaxf(part[threadIdx.x], part[threadIdx.x + w]);
      __syncthreads();
    }
    if (threadIdx.x == 0) a.zmax[bh] = part[0];
  }
}

// Latent tensors of one (batch, head) in LDS, block-major: for every block of 32 latent rows, the
// kernel's NTILE tiles follow each other (32 x D elements each, swizzled rows), so that a tile's
// position inside a block is a compile-time offset. Tile j gets rows of `stride` elements from src
// (rows >= rows_valid zero).
template <typename T, int D, int NT, int NTILE>
__device__ __forceinline__ void fill_blocked(T* lds, int j, const T* src, int stride, int rows_valid, int Mp) {
  using Sw = Swz<T, D>;
  constexpr int CH = 16 / sizeof(T), CPR = D / CH;
  for (int q = threadIdx.x; q < Mp * CPR; q += NT) {
    const int row = q / CPR, part = q % CPR;
    T* dst = lds + ((row >> 5) * NTILE + j) * 32 * D + Sw::off(row & 31, part * CH);
    *reinterpret_cast<Chunk*>(dst) =
        row < rows_valid ? *reinterpret_cast<const Chunk*>(src + (int64_t)row * stride + part * CH) : Chunk{0u, 0u, 0u, 0u};
  }
}
template <int NT>
__device__ __forceinline__ void fill_stats(float* sl, float* sc, const float* l, const float* c, int Mp,
                                           float c_factor = 1.f) {
  // Negated: the score and dP products start from -L and -c, so they come out as l - L and dP - c.
  for (int m = threadIdx.x; m < Mp; m += NT) {
    const int p = stat_pos(m);
    sl[p] = -l[m];
    sc[p] = -c[m] * c_factor;
  }
}

// ------------------------------------------------------------------------------------------
// Decode call, per token (Section 3.2 Eq. 8, the softmax over latents; Appendix B.5 for the
// cotangent). With l_nm = K_n . c Q_m and dP_nm = dY_n . Zc_m (c*Q and Zc as pairs):
//   pass 1 (shift 0 with a range check, else online with a running maximum per lane half):
//                                                     L_n = log2 sum_m 2^(l_nm),
//                                                     c_n = sum_m 2^(l_nm - L_n) dP_nm;
//   pass 2:  dK_dec,n = (1/sqrt(D)) sum_m P_nm (dP_nm - c_n) Q_m,  kept in fp32 for the encode kernel.
// LDS holds c*Q and Zc (pairs), and for bf16 c*Q in fp16 (the routing-query rows' third part).
// bf16: the dK product takes dS and c*Q as single fp16 operands (no cancellation in that sum). dS is
// scaled per token by a power of two 2^sh that keeps it below 2^14: |dP - c| <= 2 |dY_n|_1 max|Zc|,
// and the factor enters at no cost through the second pass's start value -L + sh; the store takes it
// out exactly.
template <typename T, int D, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_token_decode_kernel(BwdTokenArgs a) {
  using F = Frag<T>;
  using Op = typename F::Op;
  using Pair = typename F::Pair;
  constexpr int KB = D / 16;
  constexpr int NT = NW * 64;
  constexpr int NP = F::kLo ? 2 : 1;  // tiles per pair
  constexpr bool kH = F::kLo;

  // Block-major LDS (fill_blocked): per 32 latents, c*Q hi, [lo], Zc hi, [lo], [c*Q fp16].
  constexpr int NTILE = 2 * NP + (kH ? 1 : 0);
  constexpr int TQH = 0, TQL = 1, TZH = NP, TZL = NP + 1, TQ16 = 2 * NP;
  extern __shared__ __align__(16) unsigned char smem[];
  const int Mp = a.Mp;
  T* tiles = reinterpret_cast<T*>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), hh = lane >> 5;
  const int bh = blockIdx.y;
  {
    const T* qsrc = reinterpret_cast<const T*>(a.Qrows) + (int64_t)bh * Mp * kQRow<T> * D;
    const T* zsrc = reinterpret_cast<const T*>(a.Zc) + (int64_t)bh * Mp * D;
    fill_blocked<T, D, NT, NTILE>(tiles, TQH, qsrc, kQRow<T> * D, Mp, Mp);
    fill_blocked<T, D, NT, NTILE>(tiles, TZH, zsrc, D, Mp, Mp);
    if constexpr (F::kLo) {
      fill_blocked<T, D, NT, NTILE>(tiles, TQL, qsrc + D, kQRow<T> * D, Mp, Mp);
      fill_blocked<T, D, NT, NTILE>(tiles, TZL, reinterpret_cast<const T*>(a.Zc_lo) + (int64_t)bh * Mp * D, D, Mp, Mp);
      fill_blocked<T, D, NT, NTILE>(tiles, TQ16, qsrc + 2 * D, kQRow<T> * D, Mp, Mp);
    }
  }
  __syncthreads();
  const LaneOffs<T, D> lofs = lane_offsets<T, D>(lane);
  auto tile = [&](int lb, int j) __attribute__((always_inline)) { return tiles + (lb * NTILE + j) * 32 * D; };

  const int64_t t_begin = (int64_t)blockIdx.x * a.tokens_per_wg;
  const int64_t t_end = (t_begin + a.tokens_per_wg < a.N) ? t_begin + a.tokens_per_wg : a.N;
  const int nlb = Mp / 32;
  const bool ragged = (a.M & 31) != 0;
  const T* kbase = reinterpret_cast<const T*>(a.K) + (int64_t)bh * a.N * D;
  const T* ybase = reinterpret_cast<const T*>(a.dY) + (int64_t)bh * a.N * D;
  const float zmax = kH ? a.zmax[bh] : 0.f;
  // bf16: the largest |K| (as bf16 magnitude bits) and |dY_n|_1 of the wave's tokens, for the
  // scales of the decode call's latent-side fp16 products.
  uint32_t kmx = 0;
  float y1m = 0.f;

  for (int64_t base = t_begin + (int64_t)wave * 32; base < t_end; base += (int64_t)NW * 32) {
    const int64_t tok = base + (lane & 31);
    const bool valid = tok < t_end;
    Op kb[KB], yb[KB];
#pragma unroll
    for (int kk = 0; kk < KB; kk++) {
      const int64_t o = tok * D + 16 * kk + 8 * hh;
      kb[kk] = valid ? F::gload(kbase + o) : F::zero();
      yb[kk] = valid ? F::gload(ybase + o) : F::zero();
    }
    // Logits and dP of latent block lb (C[latent][token], lane = token), masked past M.
    // MASKED: the last block when M is not a multiple of 32 (peeled, so the other blocks carry no
    // mask instructions).
    auto scores = [&](int lb, f32x16& E, f32x16& dP, auto MASKED, const f32x16& e0, const f32x16& d0)
                      __attribute__((always_inline)) {
      Pair qa[KB], za[KB];
      E = e0;
      dP = d0;
#pragma unroll
      for (int kk = 0; kk < KB; kk++) {
        qa[kk] = row_pair_at<F, D>(tile(lb, TQH), tile(lb, TQL), lofs, kk);
        za[kk] = row_pair_at<F, D>(tile(lb, TZH), tile(lb, TZL), lofs, kk);
        E = mma_pe<F>(qa[kk], kb[kk], E);
        dP = mma_pe<F>(za[kk], yb[kk], dP);
      }
#pragma unroll
      for (int kk = 0; kk < KB; kk++) {
        hold<F>(E, qa[kk]);
        hold(E, kb[kk]);
        hold<F>(dP, za[kk]);
        hold(dP, yb[kk]);
      }
      if constexpr (decltype(MASKED)::value) {
#pragma unroll
        for (int v = 0; v < 16; v++)
          if (32 * lb + row32(v, hh) >= a.M) E[v] = -INFINITY;
      }
    };
    // Runs body(lb, MASKED) over the latent blocks, the ragged last one masked.
    auto over_blocks = [&](auto&& body) __attribute__((always_inline)) {
      for (int lb = 0; lb < nlb - 1; lb++) body(lb, std::false_type{});
      if (ragged)
        body(nlb - 1, std::true_type{});
      else
        body(nlb - 1, std::false_type{});
    };

    // The token's other 16 latents of every block are in lane l ^ 32. First pass with shift 0 (no
    // running maximum), exact whenever no exponential overflowed and the terms that matter stayed
    // normal floats: every token's sum in [2^-80, 2^100] and a finite u (the check of the forward
    // passes). A wave with any token outside it takes the pass with running maxima instead.
    float Ld = 0.f, cd = 0.f;
    bool done = false;
    if (!a.force_exact) {
      float l = 0.f, u = 0.f;
      over_blocks([&](int lb, auto MASKED) __attribute__((always_inline)) {
        f32x16 E, dP;
        scores(lb, E, dP, MASKED, f32x16{}, f32x16{});
#pragma unroll
        for (int v = 0; v < 16; v++) {
          const float p = exp2_fast(E[v]);
          l += p;
          u += p * dP[v];
        }
      });
      const float lt = l + shfl_xor(l, 32), ut = u + shfl_xor(u, 32);
      const bool ok = !valid || (lt >= 0x1p-80f && lt <= 0x1p100f && fabsf(ut) <= 3.0e38f);
      if (__all(ok)) {
        Ld = log2f(lt);
        cd = ut / lt;
        done = true;
      }
    }
    if (!done) {
      float mrun = -INFINITY, l = 0.f, u = 0.f;
      over_blocks([&](int lb, auto MASKED) __attribute__((always_inline)) {
        f32x16 E, dP;
        scores(lb, E, dP, MASKED, f32x16{}, f32x16{});
        float bm = E[0];
#pragma unroll
        for (int v = 1; v < 16; v++) bm = fmaxf(bm, E[v]);
        const float mn = fmaxf(mrun, bm);
        const float ms = mn == -INFINITY ? 0.f : mn;
        const float sc = exp2_fast(mrun - ms);
        l *= sc;
        u *= sc;
#pragma unroll
        for (int v = 0; v < 16; v++) {
          const float p = exp2_fast(E[v] - ms);
          l += p;
          u += p * dP[v];
        }
        mrun = mn;
      });
      const float mo = shfl_xor(mrun, 32), lo = shfl_xor(l, 32), uo = shfl_xor(u, 32);
      const float mt = fmaxf(mrun, mo);
      const float mts = mt == -INFINITY ? 0.f : mt;
      const float wa = exp2_fast(mrun - mts), wb = exp2_fast(mo - mts);
      const float lt = l * wa + lo * wb;
      Ld = mts + log2f(lt);
      cd = (u * wa + uo * wb) / lt;
    }
    if (valid && hh == 0) {
      a.tl[(int64_t)bh * a.N + tok] = Ld;
      a.tc[(int64_t)bh * a.N + tok] = cd;
    }

    // Second pass: the products start from the token's -L (+ sh) and -c (in every slot), so they
    // come out as l - L (+ sh) and dP - c.
    int sh = 0;
    if constexpr (kH) {
      float y1 = 0.f;
#pragma unroll
      for (int kk = 0; kk < KB; kk++)
#pragma unroll
        for (int e = 0; e < 8; e++) y1 += fabsf((float)yb[kk][e]);
#pragma unroll
      for (int kk = 0; kk < KB; kk++) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 kw = __builtin_bit_cast(u32x4, kb[kk]);
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const uint32_t m = kw[i] & 0x7fff7fffu;
          kmx = max(kmx, max(m & 0xffffu, m >> 16));
        }
      }
      y1 += shfl_xor(y1, 32);
      y1m = fmaxf(y1m, y1);
      sh = pow2_below_2e14(2.f * y1 * zmax);  // the bound >= |dP - c| of the token
    }
    f32x16 negL, negC;
#pragma unroll
    for (int v = 0; v < 16; v++) {
      negL[v] = (float)sh - Ld;
      negC[v] = -cd;
    }
    f32x16 accK = {};
    over_blocks([&](int lb, auto MASKED) __attribute__((always_inline)) {
      f32x16 E, dP;
      scores(lb, E, dP, MASKED, negL, negC);
      f32x16 dS;
#pragma unroll
      for (int v = 0; v < 16; v++) dS[v] = exp2_fast(E[v]) * dP[v];
#pragma unroll
      for (int t = 0; t < 2; t++) {
        if constexpr (kH) {
          const Op qk = F::template krows_at<D>(tile(lb, TQ16) + 16 * t * D, lofs);
          f16x8 sk;
#pragma unroll
          for (int e = 0; e < 8; e++) sk[e] = (f16)dS[8 * t + e];
          accK = mfma_32x32_f16(__builtin_bit_cast(f16x8, qk), sk, accK);
          hold(accK, qk);
          hold(accK, sk);
        } else {
          const Pair qk = krows_pair_at<F, D>(tile(lb, TQH) + 16 * t * D, tile(lb, TQL) + 16 * t * D, lofs);
          const Pair sk = F::split(dS, t);
          accK = mma_pp<F>(qk, sk, accK);
          hold<F>(accK, qk);
          hold<F>(accK, sk);
        }
      }
    });
    if (valid) {
      // dK_dec = (1/sqrt(D)) dS Q = ln 2 * dS (c*Q), less the factor 2^sh; slot v holds dim
      // row32(v, l / 32).
      const float os = ldexpf(kLn2, -sh);
      float* dk = a.dKdec + ((int64_t)bh * a.N + base) * D;
#pragma unroll
      for (int gq = 0; gq < 4; gq++) {
        const int d0 = row32(4 * gq, hh);
        if (d0 < D)
          *reinterpret_cast<f32x4*>(dk + (lane & 31) * D + d0) = f32x4{accK[4 * gq] * os, accK[4 * gq + 1] * os,
                                                    accK[4 * gq + 2] * os, accK[4 * gq + 3] * os};
      }
    }
  }
  if constexpr (kH) {
    const float km = wave_max(__uint_as_float(kmx << 16));
    y1m = wave_max(y1m);
    if (lane == 0) {
      float* o = a.tmax + (((int64_t)bh * gridDim.x + blockIdx.x) * NW + wave) * 2;
      o[0] = km;
      o[1] = y1m;
    }
  }
}

// Encode call, per token (Appendix B.5, the sums over latents): with P_mn = 2^(l_mn - L_m) and
// dP_mn = dZ_m . V_n,
//   dK_n = dK_dec,n + (1/sqrt(D)) sum_m P_mn (dP_mn - c_m) Q_m,   dV_n = sum_m P_mn dZ_m.
// LDS holds c*Q and dZ (pairs) and the per-latent L and c. Score tiles are C[latent][token]
// (lane = token); the products over latents are computed transposed, R[d][token], so that each lane
// ends with 16 dims of its own token. fp32 runs this kernel; bf16 runs bwd_token_encode_h_kernel
// below.
template <typename T, int D, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_token_encode_kernel(BwdTokenArgs a) {
  static_assert(sizeof(T) == 4, "bf16 runs bwd_token_encode_h_kernel");
  using F = Frag<T>;
  using Op = typename F::Op;
  using Pair = typename F::Pair;
  constexpr int KB = D / 16;
  constexpr int NT = NW * 64;

  // Block-major LDS (fill_blocked): per 32 latents, c*Q and dZ; then the stats.
  constexpr int NTILE = 2;
  constexpr int TQH = 0, TZH = 1;
  extern __shared__ __align__(16) unsigned char smem[];
  const int Mp = a.Mp;
  T* tiles = reinterpret_cast<T*>(smem);
  float* sl = reinterpret_cast<float*>(tiles + NTILE * Mp * D);  // [Mp] L_enc, stat_pos order
  float* sc = sl + Mp;                                            // [Mp] c_enc

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, hh = lane >> 5;
  const int bh = blockIdx.y;
  {
    const T* qsrc = reinterpret_cast<const T*>(a.Qrows) + (int64_t)bh * Mp * kQRow<T> * D;
    fill_blocked<T, D, NT, NTILE>(tiles, TQH, qsrc, kQRow<T> * D, Mp, Mp);
    fill_blocked<T, D, NT, NTILE>(tiles, TZH, reinterpret_cast<const T*>(a.dZop) + (int64_t)bh * Mp * D, D, Mp, Mp);
    fill_stats<NT>(sl, sc, a.lenc + (int64_t)bh * Mp, a.ce + (int64_t)bh * Mp, Mp);
  }
  __syncthreads();
  const LaneOffs<T, D> lofs = lane_offsets<T, D>(lane);
  auto tile = [&](int lb, int j) __attribute__((always_inline)) { return tiles + (lb * NTILE + j) * 32 * D; };

  const int64_t t_begin = (int64_t)blockIdx.x * a.tokens_per_wg;
  const int64_t t_end = (t_begin + a.tokens_per_wg < a.N) ? t_begin + a.tokens_per_wg : a.N;
  const int nlb = Mp / 32;
  const T* kbase = reinterpret_cast<const T*>(a.K) + (int64_t)bh * a.N * D;
  const T* vbase = reinterpret_cast<const T*>(a.V) + (int64_t)bh * a.N * D;

  for (int64_t base = t_begin + (int64_t)wave * 32; base < t_end; base += (int64_t)NW * 32) {
    const int64_t tok = base + (lane & 31);
    const bool valid = tok < t_end;
    Op kb[KB], vb[KB];
#pragma unroll
    for (int kk = 0; kk < KB; kk++) {
      const int64_t o = tok * D + 16 * kk + 8 * hh;
      kb[kk] = valid ? F::gload(kbase + o) : F::zero();
      vb[kk] = valid ? F::gload(vbase + o) : F::zero();
    }
    f32x16 accK = {}, accV = {};
    // One latent block.
    auto block = [&](int lb) __attribute__((always_inline)) {
      Pair qa[KB], za[KB];
      // Latents past M: zero rows of c*Q and dZ, L = +inf, c = 0, so P and dS vanish there. The
      // products start from -L and -c (negated in LDS): E = l - L, dP = dP - c.
      f32x16 E = load_stats16(sl + 32 * lb, hh), dP = load_stats16(sc + 32 * lb, hh);
#pragma unroll
      for (int kk = 0; kk < KB; kk++) {
        qa[kk] = row_pair_at<F, D>(tile(lb, TQH), tile(lb, TQH), lofs, kk);
        za[kk] = row_pair_at<F, D>(tile(lb, TZH), tile(lb, TZH), lofs, kk);
        E = mma_pe<F>(qa[kk], kb[kk], E);
        dP = mma_pe<F>(za[kk], vb[kk], dP);
      }
#pragma unroll
      for (int kk = 0; kk < KB; kk++) {
        hold<F>(E, qa[kk]);
        hold(E, kb[kk]);
        hold<F>(dP, za[kk]);
        hold(dP, vb[kk]);
      }
      f32x16 P, dS;
#pragma unroll
      for (int v = 0; v < 16; v++) {
        const float p = exp2_fast(E[v]);
        P[v] = p;
        dS[v] = p * dP[v];
      }
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const Pair qk = krows_pair_at<F, D>(tile(lb, TQH) + 16 * t * D, tile(lb, TQH) + 16 * t * D, lofs);
        const Pair sk = F::split(dS, t);
        accK = mma_pp<F>(qk, sk, accK);
        hold<F>(accK, qk);
        hold<F>(accK, sk);
        const Pair zk = krows_pair_at<F, D>(tile(lb, TZH) + 16 * t * D, tile(lb, TZH) + 16 * t * D, lofs);
        const Pair pk = F::split(P, t);
        accV = mma_pp<F>(zk, pk, accV);
        hold<F>(accV, zk);
        hold<F>(accV, pk);
      }
    };
    for (int lb = 0; lb < nlb; lb++) block(lb);
    if (valid) {
      // dK = dK_dec + (1/sqrt(D)) dS Q = dK_dec + ln 2 * dS (c*Q).
      const int64_t to = ((int64_t)bh * a.N + tok) * D;
      T* dk = reinterpret_cast<T*>(a.dK) + to;
      T* dv = reinterpret_cast<T*>(a.dV) + to;
#pragma unroll
      for (int gq = 0; gq < 4; gq++) {
        const int d0 = row32(4 * gq, hh);
        if (d0 < D) {
          const f32x4 kd = *reinterpret_cast<const f32x4*>(a.dKdec + to + d0);
          store4<T>(dk + d0, kd[0] + accK[4 * gq] * kLn2, kd[1] + accK[4 * gq + 1] * kLn2,
                    kd[2] + accK[4 * gq + 2] * kLn2, kd[3] + accK[4 * gq + 3] * kLn2);
          store4<T>(dv + d0, accV[4 * gq], accV[4 * gq + 1], accV[4 * gq + 2], accV[4 * gq + 3]);
        }
      }
    }
  }
}

// The encode call's token-side cotangents for bf16 inputs, with fp16 operands in place of the bf16
// pairs of the kernel above. fp16's 11 significant bits against bf16's 8 let single values replace
// pairs in the two products that sum over latents, and the fp16 pairs (22 bits) carry the score and
// dP products at the pairs' accuracy, so the four latent tiles fit in LDS as before:
//   c*Q as an fp16 pair: the workspace's bf16 pair hi + lo is exact in fp32 and splits exactly into
//     fp16 hi + lo, so the logits equal those of the recomputed forward (whose normalizers L are
//     used here) up to the order of the fp32 sums. The hi part alone is the dK product's operand.
//   dZ as an fp16 pair, scaled per (batch, head) by 2^g so that its largest element lies in
//     (2^13, 2^14]; c_m = <dZ_m, Z_m> is formed here from that pair, so that dP - c sees the very
//     operands of dP. The hi part alone is the dV product's operand.
//   K and V in fp16, exact for bf16 values of magnitude in [2^-14, 2^15). A 32-token group whose
//     largest |K| or |V| lies beyond 2^15 (or whose V all lie below 2^-6) takes them scaled by a power
//     of two and undoes the scale on the products (a wave-uniform branch, not taken by ordinary data).
//   P in fp16 as 2^14 P (the score product starts from 14 - L), at most 2^14.
//   dS in fp16, scaled per token by a power of two 2^sh that keeps it below 2^14, from the bound
//     |dP - c| = |dZ_m . (V_n - Z_m)| <= max_m |dZ_m|_1 (max |V_n| + max |Z|).
// The products over latents take one MFMA each per 32x32x16 step (three with pairs) and the pairs'
// splits are gone; the stores take the scale factors out exactly.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_token_encode_h_kernel(BwdTokenArgs a) {
  using F = Frag<bf16>;
  using Op = typename F::Op;
  constexpr int KB = D / 16;
  constexpr int NT = NW * 64;
  constexpr int CPR = D / 8;
  using Sw = Swz<bf16, D>;

  // Block-major LDS: per 32 latents, c*Q hi, c*Q lo, 2^g dZ hi, 2^g dZ lo (fp16); then the stats
  // (14 - L and -2^g c, stat_pos order) and per-wave maxima.
  constexpr int NTILE = 4;
  constexpr int TQH = 0, TQL = 1, TZH = 2, TZL = 3;
  extern __shared__ __align__(16) unsigned char smem[];
  const int Mp = a.Mp;
  f16* tiles = reinterpret_cast<f16*>(smem);
  float* sl = reinterpret_cast<float*>(tiles + NTILE * Mp * D);  // [Mp]
  float* sc = sl + Mp;                                            // [Mp]
  float* red = sc + Mp;                                           // [3][16]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, hh = lane >> 5;
  const int bh = blockIdx.y;
  auto tile = [&](int lb, int j) __attribute__((always_inline)) { return tiles + (lb * NTILE + j) * 32 * D; };
  auto tile_at = [&](int row, int j, int part) __attribute__((always_inline)) {
    return tiles + ((row >> 5) * NTILE + j) * 32 * D + Sw::off(row & 31, part * 8);
  };
  auto block_max = [&](float v, int slot) __attribute__((always_inline)) {
    v = wave_max(v);
    if (lane == 0) red[16 * slot + wave] = v;
    __syncthreads();
    float m = 0.f;
#pragma unroll
    for (int w = 0; w < NW; w++) m = fmaxf(m, red[16 * slot + w]);
    return m;
  };
  // Power of two 2^s with x 2^s < 2^14 (x > 0), clamped to the fp32 range of the factors.

  const float* dz = a.dZ32 + (int64_t)bh * Mp * D;
  const float* zz = a.Z32 + (int64_t)bh * a.M * D;
  int g = 0;
  float A1 = 0.f, ZM = 0.f;
  {
    const bf16* qsrc = reinterpret_cast<const bf16*>(a.Qrows) + (int64_t)bh * Mp * kQRow<bf16> * D;
    for (int q = tid; q < Mp * CPR; q += NT) {
      const int row = q / CPR, part = q % CPR;
      const bf16* r = qsrc + (int64_t)row * kQRow<bf16> * D + part * 8;
      float hv[8], lv[8];
      chunk_to_float<bf16>(*reinterpret_cast<const Chunk*>(r), hv);
      chunk_to_float<bf16>(*reinterpret_cast<const Chunk*>(r + D), lv);
      f16x8 oh, ol;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const float v = hv[e] + lv[e];
        const f16 h = (f16)v;
        oh[e] = h;
        ol[e] = (f16)(v - (float)h);
      }
      *reinterpret_cast<f16x8*>(tile_at(row, TQH, part)) = oh;
      *reinterpret_cast<f16x8*>(tile_at(row, TQL, part)) = ol;
    }
    float mx = 0.f;
    for (int i = tid; i < a.M * D; i += NT) mx = fmaxf(mx, fabsf(dz[i]));
    g = pow2_below_2e14(block_max(mx, 0));
    const float gs = ldexpf(1.f, g);
    float a1 = 0.f, zm = 0.f;
    for (int row = tid; row < Mp; row += NT) {
      const bool valid = row < a.M;
      float c = 0.f, n1 = 0.f;
#pragma unroll
      for (int part = 0; part < CPR; part++) {
        f16x8 oh, ol;
#pragma unroll
        for (int e = 0; e < 8; e++) {
          const int d = 8 * part + e;
          const float v = valid ? dz[(int64_t)row * D + d] * gs : 0.f;
          const f16 h = (f16)v, l = (f16)(v - (float)h);
          oh[e] = h;
          ol[e] = l;
          const float pv = (float)h + (float)l;
          const float zv = valid ? zz[(int64_t)row * D + d] : 0.f;
          c += pv * zv;
          n1 += fabsf(pv);
          zm = fmaxf(zm, fabsf(zv));
        }
        *reinterpret_cast<f16x8*>(tile_at(row, TZH, part)) = oh;
        *reinterpret_cast<f16x8*>(tile_at(row, TZL, part)) = ol;
      }
      a1 = fmaxf(a1, n1);
      const int p = stat_pos(row);
      sl[p] = 14.f - a.lenc[(int64_t)bh * Mp + row];
      sc[p] = -c;
    }
    A1 = block_max(a1, 1);
    ZM = block_max(zm, 2);
  }
  __syncthreads();
  const LaneOffs<bf16, D> lofs = lane_offsets<bf16, D>(lane);
  auto row16 = [&](int lb, int j, int kk) __attribute__((always_inline)) {
    return __builtin_bit_cast(f16x8, F::template row_at<D>(reinterpret_cast<const bf16*>(tile(lb, j)), lofs, kk));
  };
  auto krows16 = [&](int lb, int j, int t) __attribute__((always_inline)) {
    return __builtin_bit_cast(f16x8, F::template krows_at<D>(reinterpret_cast<const bf16*>(tile(lb, j) + 16 * t * D), lofs));
  };

  const int64_t t_begin = (int64_t)blockIdx.x * a.tokens_per_wg;
  const int64_t t_end = (t_begin + a.tokens_per_wg < a.N) ? t_begin + a.tokens_per_wg : a.N;
  const int nlb = Mp / 32;
  const bf16* kbase = reinterpret_cast<const bf16*>(a.K) + (int64_t)bh * a.N * D;
  const bf16* vbase = reinterpret_cast<const bf16*>(a.V) + (int64_t)bh * a.N * D;
  const float bound0 = 16384.f * A1;  // 2^14 max_m |2^g dZ_m|_1

  for (int64_t base = t_begin + (int64_t)wave * 32; base < t_end; base += (int64_t)NW * 32) {
    const int64_t tok = base + (lane & 31);
    const bool valid = tok < t_end;
    float kx[KB][8], vx[KB][8];
    float kmx = 0.f, vmx = 0.f;
#pragma unroll
    for (int kk = 0; kk < KB; kk++) {
      const int64_t o = tok * D + 16 * kk + 8 * hh;
      F::to_float(valid ? F::gload(kbase + o) : F::zero(), kx[kk]);
      F::to_float(valid ? F::gload(vbase + o) : F::zero(), vx[kk]);
#pragma unroll
      for (int e = 0; e < 8; e++) {
        kmx = fmaxf(kmx, fabsf(kx[kk][e]));
        vmx = fmaxf(vmx, fabsf(vx[kk][e]));
      }
    }
    vmx = fmaxf(vmx, shfl_xor(vmx, 32));  // the token's largest |V|
    // Wave-uniform scales of K and V (1 unless the group's values leave fp16's exact range).
    const float wk = wave_max(kmx), wv = wave_max(vmx);
    const int ek = wk >= 32768.f ? pow2_below_2e14(wk) : 0;
    const int ev = (wv >= 32768.f || (wv > 0.f && wv < 0x1p-6f)) ? pow2_below_2e14(wv) : 0;
    const bool rare = (ek | ev) != 0;
    const float fk = ldexpf(1.f, ek), fv = ldexpf(1.f, ev);
    if (rare) {
#pragma unroll
      for (int kk = 0; kk < KB; kk++)
#pragma unroll
        for (int e = 0; e < 8; e++) {
          kx[kk][e] *= fk;
          vx[kk][e] *= fv;
        }
    }
    f16x8 k16[KB], v16[KB];
#pragma unroll
    for (int kk = 0; kk < KB; kk++)
#pragma unroll
      for (int e = 0; e < 8; e++) {
        k16[kk][e] = (f16)kx[kk][e];
        v16[kk][e] = (f16)vx[kk][e];
      }
    const int sh = pow2_below_2e14(bound0 * (vmx + ZM));
    const float dsc = ldexpf(1.f, sh);
    const float ifk = ldexpf(1.f, -ek), ifv = ldexpf(1.f, -ev);

    f32x16 accK = {}, accV = {};
    auto block = [&](int lb) __attribute__((always_inline)) {
      f16x8 qh[KB], ql[KB], zh[KB], zl[KB];
      // The products start from 14 - L and -2^g c: E = l - L + 14, dP = 2^g (dP - c). With K or V
      // scaled by 2^ek or 2^ev, so are their start values, and the results are scaled back.
      f32x16 E = load_stats16(sl + 32 * lb, hh), dP = load_stats16(sc + 32 * lb, hh);
      if (rare) {
#pragma unroll
        for (int v = 0; v < 16; v++) {
          E[v] *= fk;
          dP[v] *= fv;
        }
      }
#pragma unroll
      for (int kk = 0; kk < KB; kk++) {
        qh[kk] = row16(lb, TQH, kk);
        ql[kk] = row16(lb, TQL, kk);
        zh[kk] = row16(lb, TZH, kk);
        zl[kk] = row16(lb, TZL, kk);
        E = mfma_32x32_f16(ql[kk], k16[kk], E);
        E = mfma_32x32_f16(qh[kk], k16[kk], E);
        dP = mfma_32x32_f16(zl[kk], v16[kk], dP);
        dP = mfma_32x32_f16(zh[kk], v16[kk], dP);
      }
#pragma unroll
      for (int kk = 0; kk < KB; kk++) {
        hold(E, qh[kk]);
        hold(E, ql[kk]);
        hold(E, k16[kk]);
        hold(dP, zh[kk]);
        hold(dP, zl[kk]);
        hold(dP, v16[kk]);
      }
      if (rare) {
#pragma unroll
        for (int v = 0; v < 16; v++) {
          E[v] *= ifk;
          dP[v] *= ifv;
        }
      }
      f16x8 pk[2], sk[2];
#pragma unroll
      for (int v = 0; v < 16; v++) {
        const float p = exp2_fast(E[v]);  // 2^14 P
        pk[v >> 3][v & 7] = (f16)p;
        sk[v >> 3][v & 7] = (f16)(p * dP[v] * dsc);
      }
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const f16x8 qk = krows16(lb, TQH, t);
        accK = mfma_32x32_f16(qk, sk[t], accK);
        hold(accK, qk);
        hold(accK, sk[t]);
        const f16x8 zk = krows16(lb, TZH, t);
        accV = mfma_32x32_f16(zk, pk[t], accV);
        hold(accV, zk);
        hold(accV, pk[t]);
      }
    };
    int lb = 0;
    for (; lb + 4 <= nlb; lb += 4) {
#pragma unroll
      for (int u = 0; u < 4; u++) block(lb + u);
    }
    for (; lb < nlb; lb++) block(lb);
    if (valid) {
      // dK = dK_dec + ln 2 * dS (c*Q) and dV = P^T dZ, less the factors 2^(14 + g + sh) and 2^(14 + g).
      const float ok = ldexpf(kLn2, -(14 + g + sh)), ov = ldexpf(1.f, -(14 + g));
      const int64_t to = ((int64_t)bh * a.N + tok) * D;
      bf16* dk = reinterpret_cast<bf16*>(a.dK) + to;
      bf16* dv = reinterpret_cast<bf16*>(a.dV) + to;
#pragma unroll
      for (int gq = 0; gq < 4; gq++) {
        const int d0 = row32(4 * gq, hh);
        if (d0 < D) {
          const f32x4 kd = *reinterpret_cast<const f32x4*>(a.dKdec + to + d0);
          store4<bf16>(dk + d0, kd[0] + accK[4 * gq] * ok, kd[1] + accK[4 * gq + 1] * ok,
                       kd[2] + accK[4 * gq + 2] * ok, kd[3] + accK[4 * gq + 3] * ok);
          store4<bf16>(dv + d0, accV[4 * gq] * ov, accV[4 * gq + 1] * ov, accV[4 * gq + 2] * ov,
                       accV[4 * gq + 3] * ov);
        }
      }
    }
  }
}

// Synthesis call and N0, per token (Section 3.2, Eq. 5-6): with the seeds Qseed as queries and the
// normalized keys Sn = N0(S) as keys and values,
//   dSn_n = (1/sqrt(D)) sum_m dS[m][n] Qseed_m + sum_m P[m][n] G_m,   dS = N0'(S)^T dSn,
// where N0'(s)^T u = r u - r^3 s mean(s * u), r = (mean(s^2) + eps)^(-1/2). LDS holds the seeds, G / c
// and the per-latent L and c of the call. fp32 runs this kernel; bf16 runs
// bwd_token_synthesis_h_kernel below.
template <typename T, int D, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_token_synthesis_kernel(BwdTokenArgs a) {
  static_assert(sizeof(T) == 4, "bf16 runs bwd_token_synthesis_h_kernel");
  using F = Frag<T>;
  using Op = typename F::Op;
  using Pair = typename F::Pair;
  constexpr int KB = D / 16;
  constexpr int NT = NW * 64;

  // Block-major LDS (fill_blocked): per 32 latents, the seeds (rows >= M zero) and G / c; then the
  // stats.
  constexpr int NTILE = 2;
  constexpr int TQS = 0, TGH = 1;
  extern __shared__ __align__(16) unsigned char smem[];
  const int Mp = a.Mp;
  T* tiles = reinterpret_cast<T*>(smem);
  float* sl = reinterpret_cast<float*>(tiles + NTILE * Mp * D);  // [Mp] L_syn, stat_pos order
  float* sc = sl + Mp;                                            // [Mp] c_syn

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, hh = lane >> 5;
  const int bh = blockIdx.y, h = bh % a.H;
  {
    fill_blocked<T, D, NT, NTILE>(tiles, TQS, reinterpret_cast<const T*>(a.Qseed) + (int64_t)h * a.M * D, D, a.M, Mp);
    fill_blocked<T, D, NT, NTILE>(tiles, TGH, reinterpret_cast<const T*>(a.Gop) + (int64_t)bh * Mp * D, D, Mp, Mp);
    fill_stats<NT>(sl, sc, a.lsyn + (int64_t)bh * Mp, a.cs + (int64_t)bh * Mp, Mp);
  }
  __syncthreads();
  const LaneOffs<T, D> lofs = lane_offsets<T, D>(lane);
  auto tile = [&](int lb, int j) __attribute__((always_inline)) { return tiles + (lb * NTILE + j) * 32 * D; };

  const int64_t t_begin = (int64_t)blockIdx.x * a.tokens_per_wg;
  const int64_t t_end = (t_begin + a.tokens_per_wg < a.N) ? t_begin + a.tokens_per_wg : a.N;
  const int nlb = Mp / 32;
  const float c_scale = kLog2e * rsqrtf((float)D);
  const T* sbase = reinterpret_cast<const T*>(a.S) + (int64_t)bh * a.N * D;

  for (int64_t base = t_begin + (int64_t)wave * 32; base < t_end; base += (int64_t)NW * 32) {
    const int64_t tok = base + (lane & 31);
    const bool valid = tok < t_end;
    // c * N0(S) of the lane's token as a pair: dims 16 kk + 8 (l / 32) .. + 7 here, the rest in
    // lane l ^ 32.
    float x[KB][8];
    float ss = 0.f;
#pragma unroll
    for (int kk = 0; kk < KB; kk++) {
      const Op raw = valid ? F::gload(sbase + tok * D + 16 * kk + 8 * hh) : F::zero();
      F::to_float(raw, x[kk]);
#pragma unroll
      for (int e = 0; e < 8; e++) ss += x[kk][e] * x[kk][e];
    }
    ss += shfl_xor(ss, 32);
    const float rn = 1.0f / sqrtf(ss * (1.0f / D) + kRmsEps);
    Pair sb[KB];
#pragma unroll
    for (int kk = 0; kk < KB; kk++) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; e++) y[e] = x[kk][e] * (rn * c_scale);
      sb[kk] = F::split8(y);
    }
    f32x16 accA = {}, accB = {};
    // One latent block.
    auto block = [&](int lb) __attribute__((always_inline)) {
      Op qa[KB];
      Pair ga[KB];
      // The products start from -L and -c (negated in LDS): A = l - L, dP = dP - c.
      f32x16 A = load_stats16(sl + 32 * lb, hh), dP = load_stats16(sc + 32 * lb, hh);
#pragma unroll
      for (int kk = 0; kk < KB; kk++) {
        qa[kk] = F::template row_at<D>(tile(lb, TQS), lofs, kk);
        ga[kk] = row_pair_at<F, D>(tile(lb, TGH), tile(lb, TGH), lofs, kk);
        A = mma_ep<F>(qa[kk], sb[kk], A);
        dP = mma_pp<F>(ga[kk], sb[kk], dP);
      }
#pragma unroll
      for (int kk = 0; kk < KB; kk++) {
        hold(A, qa[kk]);
        hold<F>(A, sb[kk]);
        hold<F>(dP, ga[kk]);
        hold<F>(dP, sb[kk]);
      }
      f32x16 P, dS;
#pragma unroll
      for (int v = 0; v < 16; v++) {
        const float p = exp2_fast(A[v]);
        P[v] = p;
        dS[v] = p * dP[v];
      }
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const Op qk = F::template krows_at<D>(tile(lb, TQS) + 16 * t * D, lofs);
        const Pair sk = F::split(dS, t);
        accA = mma_ep<F>(qk, sk, accA);
        hold(accA, qk);
        hold<F>(accA, sk);
        const Pair gk = krows_pair_at<F, D>(tile(lb, TGH) + 16 * t * D, tile(lb, TGH) + 16 * t * D, lofs);
        const Pair pk = F::split(P, t);
        accB = mma_pp<F>(gk, pk, accB);
        hold<F>(accB, gk);
        hold<F>(accB, pk);
      }
    };
    for (int lb = 0; lb < nlb; lb++) block(lb);
    // dSn in slot v: dim row32(v, l / 32) of the lane's token; with S at the same dims, the N0
    // backward needs one sum over the token's D dims (this lane's and lane l ^ 32's).
    const float s_scale = rsqrtf((float)D);
    float dsn[16], sv[16];
    float t = 0.f;
#pragma unroll
    for (int gq = 0; gq < 4; gq++) {
      const int d0 = row32(4 * gq, hh);
      float s4[4] = {0.f, 0.f, 0.f, 0.f};
      if (d0 < D && valid) load4<T>(sbase + tok * D + d0, s4);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int v = 4 * gq + i;
        dsn[v] = accA[v] * s_scale + accB[v] * c_scale;
        sv[v] = s4[i];
        if (d0 < D) t += sv[v] * dsn[v];
      }
    }
    t += shfl_xor(t, 32);
    if (valid) {
      T* ds = reinterpret_cast<T*>(a.dS) + ((int64_t)bh * a.N + tok) * D;
      const float r3 = rn * rn * rn * t * (1.0f / D);
#pragma unroll
      for (int gq = 0; gq < 4; gq++) {
        const int d0 = row32(4 * gq, hh);
        if (d0 < D) {
          const int v = 4 * gq;
          store4<T>(ds + d0, rn * dsn[v] - r3 * sv[v], rn * dsn[v + 1] - r3 * sv[v + 1],
                    rn * dsn[v + 2] - r3 * sv[v + 2], rn * dsn[v + 3] - r3 * sv[v + 3]);
        }
      }
    }
  }
}

// The synthesis call's token-side cotangent for bf16 inputs, with fp16 operands (as in the encode
// kernel above):
//   the seeds in fp16, exact for bf16 values of magnitude in [2^-14, 2^15) (a head with seeds of
//     2^15 or more takes them scaled by a power of two, and the products' start values alike);
//   c*N0(S) per token as the bf16 pair the recompute's logits used (hi truncated, lo rounded),
//     carried exactly by an fp16 pair, so the logits match the normalizers L;
//   G / c as an fp16 pair scaled per (batch, head) by 2^q so that its largest element lies in
//     (2^13, 2^14] (the bf16 pair hi + lo splits exactly), the dP operand; its hi part is the
//     operand of sum_m P G;
//   P in fp16 as 2^14 P (the score product starts from 14 - L), at most 2^14 and clear of fp16's
//     subnormals down to P = 2^-28;
//   dS in fp16 against the seeds, scaled per (batch, head) from the bound
//     |dP - c| = |G_m . (N0(s_n) - Qd_m)| <= max_m |G_m|_1 2 sqrt(D), which keeps it below 2^14.
// dP = G . c N0(S) keeps the pairs: near a one-hot synthesis row, dP - c is a difference of nearly
// equal terms.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_token_synthesis_h_kernel(BwdTokenArgs a) {
  using F = Frag<bf16>;
  using Op = typename F::Op;
  constexpr int KB = D / 16;
  constexpr int NT = NW * 64;
  constexpr int CPR = D / 8;
  using Sw = Swz<bf16, D>;

  // Block-major LDS: per 32 latents, the seeds (rows >= M zero), 2^q G / c hi and lo (fp16); then
  // the stats (14 - L and -2^q c, stat_pos order) and per-wave maxima.
  constexpr int NTILE = 3;
  constexpr int TQS = 0, TGH = 1, TGL = 2;
  extern __shared__ __align__(16) unsigned char smem[];
  const int Mp = a.Mp;
  f16* tiles = reinterpret_cast<f16*>(smem);
  float* sl = reinterpret_cast<float*>(tiles + NTILE * Mp * D);  // [Mp]
  float* sc = sl + Mp;                                            // [Mp]
  float* red = sc + Mp;                                           // [3][16]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, hh = lane >> 5;
  const int bh = blockIdx.y, h = bh % a.H;
  auto tile = [&](int lb, int j) __attribute__((always_inline)) { return tiles + (lb * NTILE + j) * 32 * D; };
  auto tile_at = [&](int row, int j, int part) __attribute__((always_inline)) {
    return tiles + ((row >> 5) * NTILE + j) * 32 * D + Sw::off(row & 31, part * 8);
  };
  auto block_max = [&](float v, int slot) __attribute__((always_inline)) {
    v = wave_max(v);
    if (lane == 0) red[16 * slot + wave] = v;
    __syncthreads();
    float m = 0.f;
#pragma unroll
    for (int w = 0; w < NW; w++) m = fmaxf(m, red[16 * slot + w]);
    return m;
  };

  const bf16* seeds = reinterpret_cast<const bf16*>(a.Qseed) + (int64_t)h * a.M * D;
  const bf16* gh = reinterpret_cast<const bf16*>(a.Gop) + (int64_t)bh * Mp * D;
  const bf16* gl = reinterpret_cast<const bf16*>(a.G_lo) + (int64_t)bh * Mp * D;
  int q = 0, es = 0;
  float A1 = 0.f;
  {
    float smx = 0.f, gmx = 0.f;
    for (int i = tid; i < a.M * D; i += NT) smx = fmaxf(smx, fabsf((float)seeds[i]));
    for (int i = tid; i < Mp * D; i += NT) gmx = fmaxf(gmx, fabsf((float)gh[i] + (float)gl[i]));
    smx = block_max(smx, 0);
    gmx = block_max(gmx, 1);
    es = smx >= 32768.f ? pow2_below_2e14(smx) : 0;
    q = pow2_below_2e14(gmx);
    const float fs = ldexpf(1.f, es), gs = ldexpf(1.f, q);
    float a1 = 0.f;
    for (int row = tid; row < Mp; row += NT) {
      float n1 = 0.f;
#pragma unroll
      for (int part = 0; part < CPR; part++) {
        float sv[8], hv[8], lv[8];
        if (row < a.M) chunk_to_float<bf16>(*reinterpret_cast<const Chunk*>(seeds + (int64_t)row * D + part * 8), sv);
        else {
#pragma unroll
          for (int e = 0; e < 8; e++) sv[e] = 0.f;
        }
        chunk_to_float<bf16>(*reinterpret_cast<const Chunk*>(gh + (int64_t)row * D + part * 8), hv);
        chunk_to_float<bf16>(*reinterpret_cast<const Chunk*>(gl + (int64_t)row * D + part * 8), lv);
        f16x8 os, oh, ol;
#pragma unroll
        for (int e = 0; e < 8; e++) {
          os[e] = (f16)(sv[e] * fs);
          const float v = (hv[e] + lv[e]) * gs;
          const f16 x = (f16)v;
          oh[e] = x;
          ol[e] = (f16)(v - (float)x);
          n1 += fabsf((float)oh[e] + (float)ol[e]);
        }
        *reinterpret_cast<f16x8*>(tile_at(row, TQS, part)) = os;
        *reinterpret_cast<f16x8*>(tile_at(row, TGH, part)) = oh;
        *reinterpret_cast<f16x8*>(tile_at(row, TGL, part)) = ol;
      }
      a1 = fmaxf(a1, n1);
      const int p = stat_pos(row);
      sl[p] = 14.f - a.lsyn[(int64_t)bh * Mp + row];
      sc[p] = -a.cs[(int64_t)bh * Mp + row] * gs;
    }
    A1 = block_max(a1, 2);
  }
  __syncthreads();
  const bool rare = es != 0;  // uniform over the workgroup
  const float fs = ldexpf(1.f, es), ifs = ldexpf(1.f, -es);
  // dS' = 2^14 P 2^q (dP - c) is at most 2^14 A1 2 log2(e); ksc keeps it below 2^14.
  const int ke = pow2_below_2e14(16384.f * A1 * (2.f * kLog2e));
  const float ksc = ldexpf(1.f, ke);
  const LaneOffs<bf16, D> lofs = lane_offsets<bf16, D>(lane);
  auto row16 = [&](int lb, int j, int kk) __attribute__((always_inline)) {
    return __builtin_bit_cast(f16x8, F::template row_at<D>(reinterpret_cast<const bf16*>(tile(lb, j)), lofs, kk));
  };
  auto krows16 = [&](int lb, int j, int t) __attribute__((always_inline)) {
    return __builtin_bit_cast(f16x8, F::template krows_at<D>(reinterpret_cast<const bf16*>(tile(lb, j) + 16 * t * D), lofs));
  };

  const int64_t t_begin = (int64_t)blockIdx.x * a.tokens_per_wg;
  const int64_t t_end = (t_begin + a.tokens_per_wg < a.N) ? t_begin + a.tokens_per_wg : a.N;
  const int nlb = Mp / 32;
  const float c_scale = kLog2e * rsqrtf((float)D);
  const bf16* sbase = reinterpret_cast<const bf16*>(a.S) + (int64_t)bh * a.N * D;

  for (int64_t base = t_begin + (int64_t)wave * 32; base < t_end; base += (int64_t)NW * 32) {
    const int64_t tok = base + (lane & 31);
    const bool valid = tok < t_end;
    // c * N0(S) of the lane's token: dims 16 kk + 8 (l / 32) .. + 7 here, the rest in lane l ^ 32;
    // rounded to the bf16 pair (hi by truncation, lo to nearest) and carried as an fp16 pair.
    float x[KB][8];
    float ss = 0.f;
#pragma unroll
    for (int kk = 0; kk < KB; kk++) {
      F::to_float(valid ? F::gload(sbase + tok * D + 16 * kk + 8 * hh) : F::zero(), x[kk]);
#pragma unroll
      for (int e = 0; e < 8; e++) ss += x[kk][e] * x[kk][e];
    }
    ss += shfl_xor(ss, 32);
    const float rn = 1.0f / sqrtf(ss * (1.0f / D) + kRmsEps);
    f16x8 sbh[KB], sbl[KB];
#pragma unroll
    for (int kk = 0; kk < KB; kk++)
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const float y = x[kk][e] * (rn * c_scale);
        const float yh = __uint_as_float(__float_as_uint(y) & 0xffff0000u);
        const float w = yh + (float)(bf16)(y - yh);
        const f16 wh = (f16)w;
        sbh[kk][e] = wh;
        sbl[kk][e] = (f16)(w - (float)wh);
      }
    f32x16 accA = {}, accB = {};
    auto block = [&](int lb) __attribute__((always_inline)) {
      f16x8 qa[KB], gha[KB], gla[KB];
      // The products start from 14 - L and -2^q c: A = l - L + 14, dP = 2^q (dP - c).
      f32x16 A = load_stats16(sl + 32 * lb, hh), dP = load_stats16(sc + 32 * lb, hh);
      if (rare) {
#pragma unroll
        for (int v = 0; v < 16; v++) A[v] *= fs;
      }
#pragma unroll
      for (int kk = 0; kk < KB; kk++) {
        qa[kk] = row16(lb, TQS, kk);
        gha[kk] = row16(lb, TGH, kk);
        gla[kk] = row16(lb, TGL, kk);
        A = mfma_32x32_f16(qa[kk], sbl[kk], A);
        A = mfma_32x32_f16(qa[kk], sbh[kk], A);
        dP = mfma_32x32_f16(gla[kk], sbh[kk], dP);
        dP = mfma_32x32_f16(gha[kk], sbl[kk], dP);
        dP = mfma_32x32_f16(gha[kk], sbh[kk], dP);
      }
#pragma unroll
      for (int kk = 0; kk < KB; kk++) {
        hold(A, qa[kk]);
        hold(A, sbh[kk]);
        hold(A, sbl[kk]);
        hold(dP, gha[kk]);
        hold(dP, gla[kk]);
        hold(dP, sbh[kk]);
        hold(dP, sbl[kk]);
      }
      if (rare) {
#pragma unroll
        for (int v = 0; v < 16; v++) A[v] *= ifs;
      }
      f16x8 pk[2], sk[2];
#pragma unroll
      for (int v = 0; v < 16; v++) {
        const float p = exp2_fast(A[v]);  // 2^14 P
        pk[v >> 3][v & 7] = (f16)p;
        sk[v >> 3][v & 7] = (f16)(p * dP[v] * ksc);
      }
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const f16x8 qk = krows16(lb, TQS, t);
        accA = mfma_32x32_f16(qk, sk[t], accA);
        hold(accA, qk);
        hold(accA, sk[t]);
        const f16x8 gk = krows16(lb, TGH, t);
        accB = mfma_32x32_f16(gk, pk[t], accB);
        hold(accB, gk);
        hold(accB, pk[t]);
      }
    };
    int lb = 0;
    for (; lb + 4 <= nlb; lb += 4) {
#pragma unroll
      for (int u = 0; u < 4; u++) block(lb + u);
    }
    for (; lb < nlb; lb++) block(lb);
    // dSn = (1/sqrt(D)) sum_m dS Qseed + c sum_m P (G / c), less the factors: accA carries
    // 2^(14 + q + ke + es), accB 2^(14 + q). Slot v holds dim row32(v, l / 32) of the lane's token;
    // with S at the same dims, the N0 backward needs one sum over the token's D dims (this lane's
    // and lane l ^ 32's).
    const float fa = ldexpf(rsqrtf((float)D), -(14 + q + ke + es)), fb = ldexpf(c_scale, -(14 + q));
    float dsn[16], sv[16];
    float t = 0.f;
#pragma unroll
    for (int gq = 0; gq < 4; gq++) {
      const int d0 = row32(4 * gq, hh);
      float s4[4] = {0.f, 0.f, 0.f, 0.f};
      if (d0 < D && valid) load4<bf16>(sbase + tok * D + d0, s4);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int v = 4 * gq + i;
        dsn[v] = accA[v] * fa + accB[v] * fb;
        sv[v] = s4[i];
        if (d0 < D) t += sv[v] * dsn[v];
      }
    }
    t += shfl_xor(t, 32);
    if (valid) {
      bf16* ds = reinterpret_cast<bf16*>(a.dS) + ((int64_t)bh * a.N + tok) * D;
      const float r3 = rn * rn * rn * t * (1.0f / D);
#pragma unroll
      for (int gq = 0; gq < 4; gq++) {
        const int d0 = row32(4 * gq, hh);
        if (d0 < D) {
          const int v = 4 * gq;
          store4<bf16>(ds + d0, rn * dsn[v] - r3 * sv[v], rn * dsn[v + 1] - r3 * sv[v + 1],
                       rn * dsn[v + 2] - r3 * sv[v + 2], rn * dsn[v + 3] - r3 * sv[v + 3]);
        }
      }
    }
  }
}

// Zero fill (a kernel rather than a memset node, so that the call can be captured in a graph).
__global__ __launch_bounds__(256) void bwd_zero_kernel(uint32_t* p, int64_t words) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < words) p[i] = 0u;
}

}  // namespace

// ------------------------------------------------------------------------------------------
// Launchers.

hipError_t launch_bwd_zero(void* p, size_t bytes, hipStream_t st) {
  const int64_t words = (int64_t)(bytes / 4);
  if (words == 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

template <typename F>
static hipError_t allow_lds_bwd(F* fn, size_t lds) {
  if (lds <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

template <typename T, int D>
static hipError_t launch_bwd_center_t(const BwdCenterArgs& a, int BH, hipStream_t st) {
  hipLaunchKernelGGL((bwd_center_kernel<T, D>), dim3(BH), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_center(const BwdCenterArgs& a, int dtype, int D, int BH, hipStream_t st) {
  if (dtype == 1) return D == 32 ? launch_bwd_center_t<bf16, 32>(a, BH, st) : launch_bwd_center_t<bf16, 16>(a, BH, st);
  return D == 32 ? launch_bwd_center_t<float, 32>(a, BH, st) : launch_bwd_center_t<float, 16>(a, BH, st);
}

template <typename T, int D, int CALL, int NW>
static hipError_t launch_bwd_latent_t(const BwdLatentArgs& a, int gx, int BH, hipStream_t st) {
  const size_t stage = (size_t)bwd_stage_t(sizeof(T) == 2, NW);
  const size_t lds = 4 * stage * D * sizeof(T) + (CALL == kBwdDecode ? 4 * stage * sizeof(float) : 0) +
                     (CALL == kBwdDecode && sizeof(T) == 2 ? 4 * stage * D * sizeof(f16) + 2 * NW * sizeof(float) : 0);
  hipError_t e = allow_lds_bwd(bwd_latent_kernel<T, D, CALL, NW>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_latent_kernel<T, D, CALL, NW>), dim3(gx, BH), dim3(NW * 64), lds, st, a);
  return hipGetLastError();
}

template <typename T, int D, int CALL>
static hipError_t launch_bwd_latent_c(const BwdLatentArgs& a, int nw, int gx, int BH, hipStream_t st) {
  return nw == 8 ? launch_bwd_latent_t<T, D, CALL, 8>(a, gx, BH, st) : launch_bwd_latent_t<T, D, CALL, 4>(a, gx, BH, st);
}

template <typename T, int D>
static hipError_t launch_bwd_latent_d(const BwdLatentArgs& a, int call, int nw, int gx, int BH, hipStream_t st) {
  switch (call) {
    case kBwdDecode: return launch_bwd_latent_c<T, D, kBwdDecode>(a, nw, gx, BH, st);
    case kBwdEncode: return launch_bwd_latent_c<T, D, kBwdEncode>(a, nw, gx, BH, st);
    default: return launch_bwd_latent_c<T, D, kBwdSynthesis>(a, nw, gx, BH, st);
  }
}

hipError_t launch_bwd_latent(const BwdLatentArgs& a, int dtype, int D, int call, int nw, int grid_x, int BH,
                             hipStream_t st) {
  if (dtype == 1)
    return D == 32 ? launch_bwd_latent_d<bf16, 32>(a, call, nw, grid_x, BH, st)
                   : launch_bwd_latent_d<bf16, 16>(a, call, nw, grid_x, BH, st);
  return D == 32 ? launch_bwd_latent_d<float, 32>(a, call, nw, grid_x, BH, st)
                 : launch_bwd_latent_d<float, 16>(a, call, nw, grid_x, BH, st);
}

template <typename T, int D>
static hipError_t launch_bwd_reduce_t(const BwdReduceArgs& a, int call, int BH, hipStream_t st) {
  // Four waves per range of 64 entries when there are 16 or more chunk partials per entry (the batch's
  // included for the synthesis call), else one.
  BwdReduceArgs r = a;
  if (call == kBwdSynthesis) {
    r.split = a.B * a.nchunk >= 16 ? 4 : 1;
    const int per_block = 64 * (4 / r.split);
    const unsigned gx = (unsigned)((a.M * D + per_block - 1) / per_block);
    hipLaunchKernelGGL((bwd_reduce_synthesis_kernel<T, D>), dim3(gx, a.H), dim3(256), 0, st, r);
    return hipGetLastError();
  }
  r.split = a.nchunk >= 16 ? 4 : 1;
  const unsigned gx = (unsigned)(a.Mp * D / (64 * (4 / r.split)));  // Mp is a multiple of 32, D of 16
  if (call == kBwdDecode)
    hipLaunchKernelGGL((bwd_reduce_decode_kernel<T, D>), dim3(gx, BH), dim3(256), 0, st, r);
  else
    hipLaunchKernelGGL((bwd_reduce_gate_kernel<T, D>), dim3(gx, BH), dim3(256), 0, st, r);
  return hipGetLastError();
}

hipError_t launch_bwd_reduce(const BwdReduceArgs& a, int dtype, int D, int call, int BH, hipStream_t st) {
  if (dtype == 1) return D == 32 ? launch_bwd_reduce_t<bf16, 32>(a, call, BH, st) : launch_bwd_reduce_t<bf16, 16>(a, call, BH, st);
  return D == 32 ? launch_bwd_reduce_t<float, 32>(a, call, BH, st) : launch_bwd_reduce_t<float, 16>(a, call, BH, st);
}

template <typename T, int D>
static size_t bwd_token_lds_t(int Mp, int kind) {
  constexpr size_t NP = sizeof(T) == 2 ? 2 : 1;  // tiles per pair
  const size_t tile = (size_t)Mp * D * sizeof(T), stats = 2 * (size_t)Mp * sizeof(float);
  switch (kind) {
    case kBwdTokDecode: return (2 * NP + (NP - 1)) * tile;  // bf16: c*Q in fp16 as well
    case kBwdTokEncode: return 2 * NP * tile + stats + (sizeof(T) == 2 ? 48 * sizeof(float) : 0);  // bf16: per-wave maxima
    default:  // seeds and G / c (bf16: both fp16, G / c as a pair; fp32: plain), stats, per-wave maxima
      return sizeof(T) == 2 ? 3 * tile + stats + 48 * sizeof(float) : 2 * tile + stats;
  }
}

size_t bwd_token_lds_bytes(int dtype, int D, int Mp, int kind) {
  if (dtype == 1) return D == 32 ? bwd_token_lds_t<bf16, 32>(Mp, kind) : bwd_token_lds_t<bf16, 16>(Mp, kind);
  return D == 32 ? bwd_token_lds_t<float, 32>(Mp, kind) : bwd_token_lds_t<float, 16>(Mp, kind);
}

// NW waves per workgroup (8 or 12) for every token-side kernel.
template <typename T, int D, int NW>
static hipError_t launch_bwd_token_t(const BwdTokenArgs& a, int kind, int gx, int BH, hipStream_t st) {
  const size_t lds = bwd_token_lds_t<T, D>(a.Mp, kind);
  auto go = [&](auto* fn, int nw) {
    hipError_t e = allow_lds_bwd(fn, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3(gx, BH), dim3(nw * 64), lds, st, a);
    return hipGetLastError();
  };
  switch (kind) {
    case kBwdTokDecode:
      // fp32 with 32 channels has no 12-wave instance (it would spill): it runs 8.
      if constexpr (std::is_same<T, float>::value && D == 32 && NW == 12) return hipErrorInvalidValue;
      else return go(bwd_token_decode_kernel<T, D, NW>, NW);
    case kBwdTokEncode:
      if constexpr (sizeof(T) == 2) return go(bwd_token_encode_h_kernel<D, NW>, NW);
      else return go(bwd_token_encode_kernel<T, D, NW>, NW);
    default:
      if constexpr (sizeof(T) == 2) return go(bwd_token_synthesis_h_kernel<D, NW>, NW);
      else return go(bwd_token_synthesis_kernel<T, D, NW>, NW);
  }
}

template <int NW>
static hipError_t launch_bwd_token_w(const BwdTokenArgs& a, int dtype, int D, int kind, int grid_x, int BH,
                                     hipStream_t st) {
  if (dtype == 1)
    return D == 32 ? launch_bwd_token_t<bf16, 32, NW>(a, kind, grid_x, BH, st)
                   : launch_bwd_token_t<bf16, 16, NW>(a, kind, grid_x, BH, st);
  return D == 32 ? launch_bwd_token_t<float, 32, NW>(a, kind, grid_x, BH, st)
                 : launch_bwd_token_t<float, 16, NW>(a, kind, grid_x, BH, st);
}

hipError_t launch_bwd_token(const BwdTokenArgs& a, int dtype, int D, int kind, int nw, int grid_x, int BH,
                            hipStream_t st) {
  if (nw == 12) return launch_bwd_token_w<12>(a, dtype, D, kind, grid_x, BH, st);
  if (nw != 8) return hipErrorInvalidValue;
  return launch_bwd_token_w<8>(a, dtype, D, kind, grid_x, BH, st);
}

}  // namespace flarepp
