// Internal interface between the host library (flarepp.cpp) and the HIP kernels (kernels.hip).
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
  const void* Qf;  // gate only: [H][M][D] dtype
  const float* g;  // gate only: [H]
  void* out;       // gate: c*Q [BH][Mout][R*D] (R parts as above); merge: Z [BH][Mout][D]
  float* dbg_qd;   // optional fp32 [BH][M][D] (gate only): Qd
  float* dbg_out;  // optional fp32 [BH][M][D]: Q (gate) or Z (merge)
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

hipError_t launch_query_prep(const QueryPrepArgs& a, int dtype, int D, int BH, hipStream_t stream);
hipError_t launch_partial(const PartialArgs& a, int dtype, int D, bool synth, int plan, int grid_x,
                          int grid_y, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, int dtype, int D, bool gate, int BH, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int dtype, int D, int nw, int grid_x, int grid_y,
                         hipStream_t stream);
size_t decode_lds_bytes(int dtype, int D, int Mp, int nw);
size_t partial_lds_bytes(int dtype, int D, int plan);

}  // namespace flarepp
