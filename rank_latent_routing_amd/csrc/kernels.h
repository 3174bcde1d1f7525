// Internal interface between the host library (flarepp.cpp) and the HIP kernels (kernels.hip:
// forward; backward.hip: backward).
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace flarepp {

// Tokens per LDS stage of the split-N partial kernels (plans 0-2; plan 3 uses 2 * kStage).
constexpr int kStage = 128;
// Partial-kernel plans: {latents per wave, waves per workgroup, tokens per stage}.
struct PartialShape {
  int lpw, nw, stage;
};
inline PartialShape partial_plan_shape(int plan) {
  switch (plan) {
    case 0: return {16, 4, kStage};
    case 1: return {32, 4, kStage};
    case 2: return {32, 8, kStage};
    default: return {32, 16, 2 * kStage};
  }
}
// Waves per decode workgroup: 8, or 12 when the latent tensors in LDS allow one workgroup per CU
// (16 is also built for the other cases). Tokens per wave group: bf16 with D = 32, 32 * TB with
// TB = 2 (8 waves) or 1 (12 waves, the default); otherwise 16 * TB with TB = 4 (8, 12 waves) or 2
// (16 waves).
constexpr int kDecodeWaves = 8;
constexpr int kDecodeWavesWide = 12;
inline int decode_group_tokens(int dtype, int D, int nw) {
  if (dtype == 1 && D == 32) return nw == 8 ? 64 : 32;  // 12 waves: one 32-token block per group
  return nw == 16 ? 32 : 64;
}

// One split-N softmax pass (synthesis or encode) over [BH, N, D] keys/values.
struct PartialArgs {
  const void* K;   // keys [BH][N][D] (synthesis: the un-normalized synthesis keys S)
  const void* V;   // values [BH][N][D] (unused by synthesis: values are the normalized keys)
  const void* Q;   // query rows: synthesis Qseed [H][Mq][D]; encode c*Q [BH][Mq][R*D]
                   // (R = 3 parts hi, lo, fp16 for bf16; 1 for fp32)
  int H;           // heads (synthesis queries are indexed by bh % H)
  int Mq;          // rows per query block (rows >= Mq read as zero)
  int Mp;          // latent rows in the partial buffers (M rounded up to 16)
  int64_t N;       // tokens
  int64_t chunk;   // tokens per chunk, a multiple of the plan's stage
  int nchunk;      // chunks per (b, h)
  int nlg;         // latent groups per chunk (workgroups sharing one chunk's tokens)
  int force_exact; // skip the zero-shift pass (test hook)
  int hilo;        // bf16, D = 32: skip the fp16 wide zero-shift pass, so the logits use the hi/lo
                   // queries on every pass (the zero-shift one first, the exact one if it fails)
  float* part_acc; // [BH][nchunk][Mp][D]
  float* part_l;   // [BH][nchunk][Mp]
  float* part_m;   // [BH][nchunk][Mp]
};

// Log-sum-exp merge of the chunk partials, with or without the gate.
struct MergeArgs {
  const float* part_acc;
  const float* part_l;
  const float* part_m;
  int nchunk;
  int Mp;          // rows of the partial buffers
  int M;           // valid latents
  int Mout;        // rows of the output block per (b, h) (M rounded up to 32; extra rows zero)
  int H;
  const void* Qf;  // gate only: [H][M][D] dtype; null: Q = Qd (no fixed query, no gate)
  const float* g;  // gate only: [H] (unused when Qf is null)
  void* out;       // gate: c*Q [BH][Mout][R*D] (R parts as above); merge: Z [BH][Mout][D]
  float* dbg_qd;   // optional fp32 [BH][M][D] (gate only): Qd
  float* dbg_out;  // optional fp32 [BH][M][D]: Q (gate) or Z (merge)
  float* lse;      // optional [BH][Mout]: log2 of each row's softmax normalizer in the logits' log2
                   // units (rows >= M: +inf, so that 2^(logit - lse) = 0 there)
};

struct DecodeArgs {
  const void* K;   // [BH][N][D]
  const void* Q;   // c*Q rows [BH][Mp][R*D] (R = 3 parts hi, lo, fp16 for bf16; 1 for fp32)
  const void* Z;   // Z [BH][Mp][D]
  void* out;       // [BH][N][D]
  int64_t N;
  int M;
  int Mp;          // M rounded up to 32
  int64_t tokens_per_wg;
  int force_exact; // skip the zero-shift pass (test hook)
};

// Routing-query rows of the workspace from the caller's fixed queries (plain FLARE).
struct QueryPrepArgs {
  const void* Q;   // [H][M][D] dtype
  int H, M, Mout;  // rows per (b, h) block in the output; rows in [M, Mout) are zero
  void* out;       // c*Q rows [BH][Mout][R*D] as for the gate
};

// ---- Backward pass (backward.hip).
//
// Logits are in log2 units throughout: l = c q.k with c = log2(e)/sqrt(D), and every probability is
// 2^(l - L) with L the row's log2 normalizer. Computed bf16 operands travel as hi + lo pairs
// (hi = bf16(x), lo = bf16(x - hi)); "_lo" pointers hold the lo parts (unused for fp32).
enum BwdCall { kBwdDecode = 0, kBwdEncode = 1, kBwdSynthesis = 2 };

// Latent-side kernel of one routing call: the cotangents of the latent-indexed tensors, which sum
// over tokens, as per-chunk partials. Score logits X_n . Qr_m (X: K, or c*N0(S) for synthesis);
// dP = W_n . Wr_m (W: dY for decode with Wr = Zc, V for encode with Wr = dZ, c*N0(S) for synthesis
// with Wr = G/c).
struct BwdLatentArgs {
  const void* X;     // [BH][N][D] dtype: K (decode, encode) or S (synthesis, normalized in-kernel)
  const void* W;     // [BH][N][D] dtype: dY (decode) or V (encode); unused by synthesis
  const float* tl;   // decode: [BH][N] per-token log2 normalizer
  const float* tc;   // decode: [BH][N] per-token c = sum_m P dP
  const void* Qr;    // decode/encode: c*Q workspace rows [BH][Mp][R*D]; synthesis: Qseed [H][M][D]
  const void* Wr;    // [BH][Mp][D] dtype hi part: Zc (decode), dZ (encode), G/c (synthesis); rows >= M zero
  const void* Wr_lo; // the lo part
  const float* ll;   // encode/synthesis: [BH][Mp] per-latent log2 normalizer (rows >= M: +inf)
  const float* lc;   // encode/synthesis: [BH][Mp] per-latent <dZ, Z> or <G, Qd>, with dZ and G as the
                     // dP operand carries them (rows >= M: 0)
  float* part0;      // decode: [BH][nchunk][Mp][D] sum_n P dY
  float* part1;      // [BH][nchunk][Mp][D] sum_n dS X
  const float* tmax; // bf16 decode: [BH][ntmax][2] maxima of the token decode kernel's waves
  const float* zmax; // bf16 decode: [BH] largest |Zc| element
  int ntmax;
  int64_t N;
  int64_t chunk;     // tokens per chunk (a multiple of the stage)
  int nchunk, nlg, M, Mp, H;
};

// Sums of the latent-side partials and the latent-sized steps between the calls.
struct BwdReduceArgs {
  const float* part0;
  const float* part1;
  int nchunk, M, Mp, H, B;
  int split;          // waves per range of 64 entries (1 or 4), set by the launcher
  // decode -> encode
  const float* Z32;   // [BH][M][D] fp32 Z
  float* dZ32;        // [BH][Mp][D]
  void* dZop;         // [BH][Mp][D] dtype hi part of dZ
  void* dZop_lo;      // lo part
  float* ce;          // [BH][Mp]
  float* dQdec;       // [BH][Mp][D] (already scaled by 1/sqrt(D))
  // encode -> gate -> synthesis
  const void* Qf;     // [H][M][D] dtype
  const float* g;     // [H]
  const float* Qd32;  // [BH][M][D] fp32 Qd
  float* dQf_bh;      // [BH][Mp][D]
  void* Gop;          // [BH][Mp][D] dtype hi part of g dQ / c
  void* Gop_lo;       // lo part
  float* cs;          // [BH][Mp]: <g dQ, Qd>
  float* rowdot;      // [BH][Mp]: <dQ, Qd>
  // synthesis -> parameter cotangents
  void* dQseed;       // [H][M][D] dtype
  void* dQf;          // [H][M][D] dtype
  float* dg;          // [H]
};

// Token-side kernels: per-token quantities that sum over latents. Decode: the normalizer L_n of each
// token's softmax over latents, c_n = sum_m P_nm dP_nm, and the decode call's part of dK (fp32).
// Encode: dK (adding the decode part) and dV. Synthesis: dS.
struct BwdTokenArgs {
  const void* K; const void* V; const void* dY; const void* S;  // [BH][N][D] dtype
  float* tl; float* tc;  // decode per-token L and c (written by the decode kernel)
  float* dKdec;          // [BH][N][D] fp32: the decode call's dK (written by decode, read by encode)
  const void* Qrows;     // c*Q workspace rows [BH][Mp][R*D] (hi, lo parts)
  const void* Zc; const void* Zc_lo;      // [BH][Mp][D] dtype: Z minus its mean over latents
  float* tmax;  // bf16 decode: [BH][gridDim.x * NW][2] per-wave max |K| and max_n |dY_n|_1
  const float* zmax;                      // [BH] largest |Zc| element (bf16 decode's dK product)
  const void* dZop; const void* dZ_lo;    // [BH][Mp][D] dtype
  const float* lenc; const float* ce;     // [BH][Mp]
  const float* dZ32;                      // [BH][Mp][D] fp32 dZ (bf16 encode kernel's fp16 operands)
  const float* Z32;                       // [BH][M][D] fp32 Z of the forward
  const void* Qseed;                      // [H][M][D] dtype
  const void* Gop; const void* G_lo;      // [BH][Mp][D] dtype: G / c
  const float* lsyn; const float* cs;     // [BH][Mp]
  void* dK; void* dV; void* dS;           // [BH][N][D] dtype
  int64_t N;
  int64_t tokens_per_wg;
  int M, Mp, H;
  int force_exact;         // decode statistics: skip the zero-shift pass (test hook)
};
enum BwdTokenKind { kBwdTokDecode = 0, kBwdTokEncode = 1, kBwdTokSynthesis = 2 };

// Z centered over the latents, Zc_m = Z_m - mean_m Z_m, as the decode call's dP operand: the shift
// cancels in dP - c, and rounding then scales with the spread of Z rather than with its mean.
struct BwdCenterArgs {
  const float* Z32;  // [BH][M][D]
  void* Zc;          // [BH][Mp][D] dtype hi part (rows >= M zero)
  void* Zc_lo;       // lo part
  float* zmax;       // optional [BH]: the largest |Zc| element
  int M, Mp;
};

// Tokens per LDS stage of the latent-side kernel: bf16 runs 256 with 8-wave workgroups and 128
// with 4-wave ones, fp32 runs 64 (their operands take twice the registers).
constexpr int bwd_stage_t(bool bf16, int nw) { return bf16 ? (nw == 8 ? 256 : 128) : 64; }
inline int bwd_stage(int dtype, int nw) { return bwd_stage_t(dtype == 1, nw); }
inline int bwd_latent_waves(int Mp) { return Mp >= 256 ? 8 : 4; }
constexpr int kBwdTokenWaves = 8;       // smallest token-side workgroup (the token split is sized for it)
constexpr int kBwdTokenWavesWide = 12;  // token encode and synthesis kernels (8 also built)
// Token decode kernel: 12 waves (3 per SIMD, at most 168 registers per lane) for bf16; fp32 keeps
// 8, as its 32-channel instance would spill at 12 (no such instance is built).
inline int bwd_decode_waves(int dtype) { return dtype == 1 ? 12 : 8; }

hipError_t launch_bwd_center(const BwdCenterArgs& a, int dtype, int D, int BH, hipStream_t st);
hipError_t launch_bwd_latent(const BwdLatentArgs& a, int dtype, int D, int call, int nw, int grid_x, int BH,
                             hipStream_t st);
hipError_t launch_bwd_reduce(const BwdReduceArgs& a, int dtype, int D, int call, int BH, hipStream_t st);
hipError_t launch_bwd_token(const BwdTokenArgs& a, int dtype, int D, int kind, int nw, int grid_x, int BH,
                            hipStream_t st);
size_t bwd_token_lds_bytes(int dtype, int D, int Mp, int kind);
hipError_t launch_bwd_zero(void* p, size_t bytes, hipStream_t st);  // bytes: a multiple of 4

hipError_t launch_query_prep(const QueryPrepArgs& a, int dtype, int D, int BH, hipStream_t stream);
hipError_t launch_partial(const PartialArgs& a, int dtype, int D, bool synth, int plan, int grid_x,
                          int grid_y, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, int dtype, int D, bool gate, int BH, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int dtype, int D, int nw, int grid_x, int grid_y,
                         hipStream_t stream);
size_t decode_lds_bytes(int dtype, int D, int Mp, int nw);

// ---- Projections around the mixer (project.hip) ----------------------------------------------
// Out = X W^T per 32-token tile; each wave keeps the weight rows of its 32-channel output group in
// registers. Front end: X [B][N][C] -> K = N_a(X Wk^T + bk), V = X Wv^T + bv, S = X Ws^T + bs, each
// [B][H][N][D]. Output projection: Y [B][H][N][D] (heads concatenated) -> Y Wo^T + bo, [B][N][C].
constexpr int kProjTile = 64;   // tokens per LDS stage (two 32-token blocks)
struct ProjArgs {
  const void* X;        // front end: X [B][N][C]; output projection: Y [B][H][N][D]
  const void* W[3];     // [C][C] each, row o = the weights of output channel o (torch Linear layout)
  const void* bias[3];  // [C] or null
  const void* scale;    // front end: the key scale [D] of N_a (null: 1)
  void* out[3];         // front end: K, V, S [B][H][N][D]; output projection: out [B][N][C]
  int H, C;
  int nproj;            // 3 (front end) or 1
  int ngb;              // workgroups sharing one token range (one 32-channel group per wave)
  int64_t N;
  int ntiles;           // kProjTile-token tiles per batch element
  int tiles_per_wg;     // tiles per token range
  int nranges;          // token ranges per batch element
  int nwg;              // workgroups with work; the grid rounds it up to a multiple of 8
};
int proj_waves(int dtype, int C);  // waves per workgroup for channel width C
size_t proj_lds_bytes(int dtype, int C, int nproj);
hipError_t launch_project(const ProjArgs& a, int dtype, int D, bool front, int grid, hipStream_t st);

// Synthesis seeds N_a(Qseed) and gates sigmoid(gamma) for the block.
struct BlockParamArgs {
  const void* Qseed;    // [H][M][D]
  const void* nq;       // [D] seed scale or null (1)
  const float* gamma;   // [H] gate logits
  void* Qs;             // [H][M][D] out, the model dtype
  float* g;             // [H] out
  int H, M;
};
hipError_t launch_block_params(const BlockParamArgs& a, int dtype, int D, hipStream_t st);

}  // namespace flarepp
