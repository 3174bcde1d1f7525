/*
 * flarepp.h - C ABI of the FLARE++ token mixer on MI355X (gfx950): the forward pass, its variants,
 * its backward pass, and the block of projections around it.
 *
 * Source: "FLARE++: Low-rank attention with attention-synthesized routing" (arXiv 2608.11519 v2),
 * Section 3.2, Eq. 5-8, restated as one block in Appendix A.1, Eq. 11. For each batch element b and
 * head h the mixer makes three softmax routing calls:
 *
 *   synthesis : Qd = softmax(Qseed . N0(S)^T / sqrt(D)) . N0(S)   softmax over the N tokens
 *                                                                   (Eq. 6 with the shared keys and
 *                                                                   values of Eq. 5 / Appendix A.6,
 *                                                                   Eq. 19)
 *   gate      : Q  = N0(Qf) + g . Qd                                (Eq. 7 / Appendix A.4, Eq. 15)
 *   encode    : Z  = softmax(Q . K^T / sqrt(D)) . V                 softmax over the N tokens (Eq. 8)
 *   decode    : Y  = softmax(K . Q^T / sqrt(D)) . Z                 softmax over the M latents (Eq. 8;
 *                                                                   the decode factor is the softmax
 *                                                                   of the transposed scores, Eq. 4)
 *
 * N0 is RMS normalization without a learned scale over the head dimension D (Section 3.2):
 * N0(x) = x / sqrt(mean(x^2) + 1e-6). The pages give no epsilon; 1e-6 is this library's constant.
 * The learned-scale normalizations of the pages (on the seeds and on the routing keys) are the
 * caller's: Qseed and K are taken as already normalized. The gate value g is passed directly
 * (the pages parameterize it as a sigmoid of a learned logit). The N x N mixing matrix
 * W_dec . W_enc (rank <= M, Eq. 9) is never formed.
 *
 * Layouts (all row-major and contiguous, element type given by `dtype`):
 *   K, V, S, out : [B, H, N, D]   (S = synthesis keys before normalization)
 *   Qseed, Qf    : [H, M, D]      shared over the batch
 *   g            : [H] float32    gate values, normally in [0, 1]
 * All pointers are device pointers on the current HIP device. Every tensor pointer must be 16-byte
 * aligned. `out` must not overlap any input. Inputs are read-only.
 *
 * Supported: dtype FLAREPP_FP32 or FLAREPP_BF16 (out has the input dtype; accumulation is fp32),
 * D in {16, 32}, 1 <= M <= 512, N >= 0, B >= 0, H >= 0, B*H <= 65535, gfx950 devices only.
 * B*H*N == 0 is a valid call that does nothing.
 *
 * Semantics: every call is asynchronous on `stream` (no host synchronization, no device-to-host
 * copies). Results are deterministic: no atomics, fixed reduction order. Calls on different
 * streams may run concurrently when each has its own workspace. Validation happens before anything
 * is enqueued, so a call that returns an error has enqueued nothing. Errors raised while kernels
 * run surface at the caller's next synchronization of `stream`, as in HIP. No C++ exception or
 * abort crosses this interface. Inputs holding NaN or Inf give NaN outputs; finite inputs whose
 * values exceed about 1e22 in magnitude may overflow the fp32 accumulators.
 *
 * The entry points that take a caller's workspace (the *_ws ones, flarepp_mix_backward_ws,
 * flarepp_block_ws) enqueue kernel launches only: no allocation, memset, copy or synchronization.
 * A caller may capture them in a HIP graph and replay it; every replay recomputes everything from
 * the inputs, so the workspace needs no clearing between replays. The entry points without a
 * workspace argument allocate theirs stream-ordered (hipMallocAsync / hipFreeAsync on `stream`).
 */
#ifndef FLAREPP_H
#define FLAREPP_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum flarepp_status {
  FLAREPP_OK = 0,
  FLAREPP_INVALID_ARGUMENT = 1, /* null pointer, negative size, size overflow, bad workspace size */
  FLAREPP_UNSUPPORTED = 2,      /* D not in {16,32}, M outside [1,512], unknown dtype, B*H too
                                   large, or a device that is not gfx950 */
  FLAREPP_MISALIGNED = 3,       /* a tensor pointer that is not 16-byte aligned */
  FLAREPP_OUT_OF_MEMORY = 4,    /* workspace allocation failed */
  FLAREPP_LAUNCH_FAILED = 5,    /* a kernel launch was rejected by the runtime */
  FLAREPP_DEVICE_ERROR = 6,     /* the HIP runtime reported an error while querying the device */
  FLAREPP_SCRATCH_TOO_SMALL = 7 /* flarepp_mix_noalloc: the problem needs more workspace than the
                                   static scratch holds (FLAREPP_NOALLOC_SCRATCH_BYTES) */
};

/* Element types of K, V, S, Qseed, Qf and out. */
enum flarepp_dtype { FLAREPP_FP32 = 0, FLAREPP_BF16 = 1 };

/*
 * Full mixer forward (Eq. 11): out[b,h] = decode(encode(gate(synthesis(Qseed[h], S[b,h]), Qf[h],
 * g[h]), K[b,h], V[b,h])). The library allocates its workspace with hipMallocAsync on `stream`
 * and frees it with hipFreeAsync on the same stream.
 */
int flarepp_mix(const void* K, const void* V, const void* S, const void* Qseed, const void* Qf,
                const float* g, int B, int H, int64_t N, int M, int D, int dtype, void* out,
                hipStream_t stream);

/* Bytes of device workspace that flarepp_mix_ws and flarepp_mix_debug need for these sizes, or 0
 * when the sizes are invalid or unsupported (or when B*H*N == 0). */
size_t flarepp_workspace_bytes(int B, int H, int64_t N, int M, int D, int dtype);

/*
 * Same as flarepp_mix, with a caller-owned device workspace of at least
 * flarepp_workspace_bytes(...) bytes, 256-byte aligned. The workspace holds the per-chunk
 * online-softmax partials of the two token-axis softmaxes (the log-sum-exp merge of Appendix B,
 * Eq. 29-33, applied across token chunks of one GPU) and the latent tensors Q and Z. Its contents
 * need no initialization and are dead after the call's kernels finish.
 */
int flarepp_mix_ws(const void* K, const void* V, const void* S, const void* Qseed, const void* Qf,
                   const float* g, int B, int H, int64_t N, int M, int D, int dtype, void* out,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): flarepp_mix with its workspace in a static device array of
 * FLAREPP_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it runs on until the
 * process ends. The call allocates nothing (no hipMalloc, hipFree or allocating library routine) and
 * otherwise behaves as flarepp_mix_ws. A problem whose workspace, flarepp_workspace_bytes(...),
 * exceeds the scratch returns FLAREPP_SCRATCH_TOO_SMALL and enqueues nothing; 32 MiB holds every
 * shape up to the 1M-token one (B=1, H=8, N=2^20, M=512, D=32: about 18 MiB). All calls on one GPU
 * share that GPU's scratch: calls that overlap on one GPU (other streams, other threads) race, so a
 * caller serializes them, for instance on one stream.
 */
#define FLAREPP_NOALLOC_SCRATCH_BYTES (32u << 20)
int flarepp_mix_noalloc(const void* K, const void* V, const void* S, const void* Qseed, const void* Qf,
                        const float* g, int B, int H, int64_t N, int M, int D, int dtype, void* out,
                        hipStream_t stream);

/*
 * flarepp_mix_ws that also exports the per-(b,h) latent stages as fp32 device arrays of shape
 * [B, H, M, D] before any cast to `dtype`: Qd (synthesis output, Eq. 6), Q (gated routing queries,
 * Eq. 7) and Z (encoder output, Eq. 8). Any of the three may be NULL.
 */
int flarepp_mix_debug(const void* K, const void* V, const void* S, const void* Qseed,
                      const void* Qf, const float* g, int B, int H, int64_t N, int M, int D,
                      int dtype, void* out, float* Qd, float* Q, float* Z, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * Plain FLARE (Section 3.1, Eq. 3), the fixed-query special case of the mixer: for each (b, h),
 * out = softmax_M(K Q^T / sqrt(D)) softmax_N(Q K^T / sqrt(D)) V with the caller's latent queries
 * Q [H, M, D] used as given (no normalization, no synthesis, no gate), shared over the batch.
 * Layouts, support, semantics and errors as for flarepp_mix; Q must not overlap `out`. The library
 * allocates its workspace stream-ordered (flarepp_flare) or takes the caller's
 * (flarepp_flare_ws, at least flarepp_workspace_bytes(B, H, N, M, D, dtype) bytes, 256-byte
 * aligned).
 */
int flarepp_flare(const void* K, const void* V, const void* Q, int B, int H, int64_t N, int M, int D,
                  int dtype, void* out, hipStream_t stream);
int flarepp_flare_ws(const void* K, const void* V, const void* Q, int B, int H, int64_t N, int M,
                     int D, int dtype, void* out, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/*
 * Simplified FLARE++ (Appendix A.8, Eq. 20): the routing queries are the synthesized correction
 * alone, Q = SDPA(Qseed, Sk, Sv), with no fixed query and no gate; then Z = SDPA(Q, K, V) and
 * out = SDPA(K, Q, Z) as in Eq. 8. Sk and Sv are the synthesis keys and the separate synthesis
 * values [B, H, N, D], used as given: the learned-scale normalization the pages apply to the seeds
 * and the synthesis keys is the caller's, as for flarepp_mix's Qseed and K. Qseed [H, M, D] is
 * shared over the batch. Layouts, support, semantics and errors as for flarepp_mix; out must not
 * overlap any input. Workspace: stream-ordered (flarepp_mix_simplified) or the caller's
 * (flarepp_mix_simplified_ws, at least flarepp_workspace_bytes(B, H, N, M, D, dtype) bytes, 256-byte
 * aligned).
 */
int flarepp_mix_simplified(const void* K, const void* V, const void* Sk, const void* Sv,
                           const void* Qseed, int B, int H, int64_t N, int M, int D, int dtype,
                           void* out, hipStream_t stream);
int flarepp_mix_simplified_ws(const void* K, const void* V, const void* Sk, const void* Sv,
                              const void* Qseed, int B, int H, int64_t N, int M, int D, int dtype,
                              void* out, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * Backward pass of flarepp_mix: given the same inputs and the cotangent dY of `out`
 * ([B, H, N, D], dtype), writes the cotangents of every input (Appendix B.5, Eq. 46-49 applied to
 * the decode, encode and synthesis calls of Section 3.2 Eq. 6 and Eq. 8 in reverse order, through
 * the gate of Eq. 7 and the normalization N0 of Eq. 5):
 *   dK, dV, dS  [B, H, N, D] dtype  (dK sums the encode and decode calls' contributions);
 *   dQseed, dQf [H, M, D]    dtype  (summed over the batch, as the seeds and Qf are shared);
 *   dg          [H]          fp32   (the cotangent of the gate value g, summed over the batch).
 * The forward pass is recomputed inside the call (nothing has to be kept from flarepp_mix).
 * Accumulation is fp32. In bf16 runs the operands the library computes (probabilities, score
 * cotangents, the routing queries, Z, dZ and the other latent cotangents) enter the matrix unit as
 * pairs hi + lo (bf16, or fp16 in the token-side kernels; at least 16 significant bits) wherever a
 * product's terms cancel, and as single fp16 values (11 bits) scaled by powers of two into fp16's
 * range where they do not: the token-side products over latents and the decode call's products over
 * tokens. Support as for flarepp_mix. Every output is written fully and must not
 * overlap any other argument buffer; inputs are read-only. With B*H*N == 0 the shared parameters'
 * cotangents are set to zero. Deterministic (no atomics), asynchronous on `stream`.
 * flarepp_mix_backward allocates its workspace stream-ordered; flarepp_mix_backward_ws takes the
 * caller's: at least flarepp_backward_workspace_bytes(B, H, N, M, D, dtype) bytes (0 for invalid
 * sizes), 256-byte aligned. It holds per-token statistics and, for bf16, the decode call's part of
 * dK in fp32, so it grows with B*H*N*D.
 */
size_t flarepp_backward_workspace_bytes(int B, int H, int64_t N, int M, int D, int dtype);
int flarepp_mix_backward(const void* K, const void* V, const void* S, const void* Qseed, const void* Qf,
                         const float* g, const void* dY, int B, int H, int64_t N, int M, int D,
                         int dtype, void* dK, void* dV, void* dS, void* dQseed, void* dQf, float* dg,
                         hipStream_t stream);
int flarepp_mix_backward_ws(const void* K, const void* V, const void* S, const void* Qseed,
                            const void* Qf, const float* g, const void* dY, int B, int H, int64_t N,
                            int M, int D, int dtype, void* dK, void* dV, void* dS, void* dQseed,
                            void* dQf, float* dg, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * The same backward in two calls, the way a training step runs it (the pages' backward takes the
 * log-normalizers and outputs its forward kept, Appendix B.3 and B.5):
 *
 * flarepp_mix_forward_saved runs the mixer forward and keeps, in the caller's workspace, the state
 * the backward starts from: both token-axis calls computed with hi/lo query logits and hi/lo P.V
 * products (as the backward's own recompute computes them), the routing-query rows, Z and Qd in
 * fp32, and the synthesis and encode calls' per-latent log2 normalizers. It writes `out` like
 * flarepp_mix (the same bars; its latent stages carry more bits). The workspace is at least
 * flarepp_backward_workspace_bytes(B, H, N, M, D, dtype) bytes, 256-byte aligned.
 *
 * flarepp_mix_backward_saved then writes the cotangents as flarepp_mix_backward_ws does, bit for
 * bit, without recomputing that state: the workspace must hold what flarepp_mix_forward_saved left
 * for the same inputs and sizes, untouched since (the library cannot check this; other contents
 * give wrong cotangents, not a fault). It only reads that state, so several cotangents dY can follow
 * one forward_saved. Both calls only enqueue kernels (no allocation) and may be captured in a HIP
 * graph. Arguments, support and errors as for flarepp_mix and flarepp_mix_backward_ws.
 */
int flarepp_mix_forward_saved(const void* K, const void* V, const void* S, const void* Qseed, const void* Qf,
                              const float* g, int B, int H, int64_t N, int M, int D, int dtype, void* out,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);
int flarepp_mix_backward_saved(const void* K, const void* V, const void* S, const void* Qseed, const void* Qf,
                               const float* g, const void* dY, int B, int H, int64_t N, int M, int D, int dtype,
                               void* dK, void* dV, void* dS, void* dQseed, void* dQf, float* dg, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * The block around the mixer: the feature projections in front of it, the per-head normalizations
 * and the output projection (Section 3.2: the synthesis keys of Eq. 5, the routing keys and values
 * before Eq. 8, the seeds and the gate of Eq. 6-7; Appendix C.2 for which tensors carry the learned-
 * scale normalization N_a; Section 3.1, "Full self-attention", for the head split and the output
 * projection).
 *
 * Layouts (row-major, contiguous, element type `dtype` unless stated):
 *   X, out         : [B, N, C] with C = H * D; head h owns channels h*D .. h*D + D - 1
 *   Wk, Wv, Ws, Wo : [C, C], row o holding the input weights of output channel o (the layout of
 *                    torch.nn.Linear's weight): a projection computes x . W^T + b, so the pages'
 *                    matrix W_K is Wk transposed
 *   bk, bv, bs, bo : [C] biases, or NULL for none
 *   nk, nq         : [D] learned scales of N_a on the routing keys and on the seeds (one vector
 *                    shared by all heads), or NULL for a unit scale
 *   gamma          : [H] float32 gate logits; the gate is g = 1 / (1 + exp(-gamma))
 * N_a(x) = x / sqrt(mean(x^2) + 1e-6) * scale over each head's D channels, in fp32.
 * Support: dtype FLAREPP_FP32 or FLAREPP_BF16, D in {16, 32}, C <= 512 (bf16) or C <= 256 (fp32),
 * N <= 2^35, B <= 65535, gfx950. Tensor pointers 16-byte aligned (biases and scales: aligned to
 * their element). Outputs must not overlap any input or each other. Products accumulate in fp32;
 * outputs are rounded once to `dtype` (bf16: to nearest even).
 *
 * flarepp_project writes K = N_a(X Wk^T + bk) with scale nk, V = X Wv^T + bv and S = X Ws^T + bs,
 * each [B, H, N, D] (S un-normalized: the mixer applies N0 to it), ready for flarepp_mix.
 * flarepp_out_project writes out[b, n] = concat_h(Y[b, h, n]) Wo^T + bo for Y [B, H, N, D].
 * B*H*N == 0 does nothing.
 */
int flarepp_project(const void* X, const void* Wk, const void* Wv, const void* Ws, const void* bk,
                    const void* bv, const void* bs, const void* nk, int B, int H, int64_t N, int D,
                    int dtype, void* K, void* V, void* S, hipStream_t stream);
int flarepp_out_project(const void* Y, const void* Wo, const void* bo, int B, int H, int64_t N, int D,
                        int dtype, void* out, hipStream_t stream);

/*
 * The whole block: flarepp_project, then the mixer (flarepp_mix) with the seeds N_a(Qseed) (scale
 * nq, rounded to dtype) and the gates sigmoid(gamma), then flarepp_out_project of its output. Qseed
 * and Qf are [H, M, D] as for flarepp_mix (Qf is normalized by the mixer with N0). Support: the
 * union of the mixer's and the projections' conditions (1 <= M <= 512, B*H <= 65535). flarepp_block
 * allocates its workspace stream-ordered; flarepp_block_ws takes the caller's, at least
 * flarepp_block_workspace_bytes(B, H, N, M, D, dtype) bytes (0 for invalid sizes), 256-byte aligned.
 * It holds K, V, S and the mixer output (4 B H N D elements) besides the mixer's own workspace.
 */
size_t flarepp_block_workspace_bytes(int B, int H, int64_t N, int M, int D, int dtype);
int flarepp_block(const void* X, const void* Wk, const void* Wv, const void* Ws, const void* Wo,
                  const void* bk, const void* bv, const void* bs, const void* bo, const void* Qseed,
                  const void* Qf, const float* gamma, const void* nq, const void* nk, int B, int H,
                  int64_t N, int M, int D, int dtype, void* out, hipStream_t stream);
int flarepp_block_ws(const void* X, const void* Wk, const void* Wv, const void* Ws, const void* Wo,
                     const void* bk, const void* bv, const void* bs, const void* bo, const void* Qseed,
                     const void* Qf, const float* gamma, const void* nq, const void* nk, int B, int H,
                     int64_t N, int M, int D, int dtype, void* out, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/* Test hook: while enabled (non-zero), every call skips the zero-shift pass and computes all three
 * softmaxes with exact running maxima (the path the library otherwise takes only for rows whose
 * zero-shift result fails its range check). Results agree with the default path to rounding.
 * Process-wide; returns the previous setting. */
int flarepp_debug_force_exact(int enable);

/* Kernel timing. While enabled, every mixer call records a HIP event pair around each of its
 * kernels on the call's stream. flarepp_timing_read synchronizes those events, adds their elapsed
 * times per kernel into ms[0..n-1] and launch counts into counts[0..n-1] (n <= number of kernel
 * kinds, see flarepp_kernel_name), clears the record and returns the number of kernel kinds.
 * Timing state is per process; concurrent timed calls from several threads are not supported. */
int flarepp_timing_enable(int enable);
int flarepp_timing_read(double* ms, long long* counts, int n);
/* Name of kernel kind `i` (0 <= i < number of kinds), NULL otherwise. */
const char* flarepp_kernel_name(int i);

/* Human-readable text of a status code. Never NULL. */
const char* flarepp_strerror(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int flarepp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLAREPP_H */
