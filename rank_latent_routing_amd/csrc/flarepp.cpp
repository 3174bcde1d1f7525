// Host side of the FLARE++ mixer library: argument validation, launch planning, workspace layout,
// the C ABI declared in include/flarepp.h, and optional per-kernel event timing.
//
// The mixer (arXiv 2608.11519 v2, Appendix A.1 Eq. 11) runs as five kernels on the caller's
// stream: synthesis partials, merge + gate, encode partials, merge, decode. The two token-axis
// softmaxes are split over token chunks whose online-softmax partials are combined with the
// log-sum-exp merge of Appendix B.3 (Eq. 29-33), chunks standing in for the pages' ranks.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "flarepp.h"
#include "kernels.h"

namespace {

using flarepp::kStage;

constexpr int kVersion = 400;  // 0.4.0
constexpr int kNumKinds = 19;
const char* const kKindNames[kNumKinds] = {"synthesis_partial", "merge_gate", "encode_partial",
                                           "merge", "decode", "query_prep",
                                           "bwd_center", "bwd_token_decode", "bwd_latent_decode",
                                           "bwd_reduce_decode", "bwd_latent_encode", "bwd_reduce_gate",
                                           "bwd_latent_synthesis", "bwd_reduce_synthesis",
                                           "bwd_token_encode", "bwd_token_synthesis", "project",
                                           "out_project", "block_params"};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Launch-plan overrides for tuning sweeps (read once per process).
int env_int(const char* name, int fallback) {
  const char* v = std::getenv(name);
  if (!v || !*v) return fallback;
  char* end = nullptr;
  const long x = std::strtol(v, &end, 10);
  return (end && *end == 0 && x > 0 && x < (1 << 30)) ? (int)x : fallback;
}
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Launch plan and workspace layout for one problem shape. The same function serves
// flarepp_workspace_bytes and the launches, so both always agree.
struct Plan {
  int BH = 0;
  int H = 0;
  int Mp16 = 0, Mp32 = 0;
  int part_plan = 0;  // kernel variant, see flarepp::partial_plan_shape
  int nlg = 1;        // latent groups (workgroups per chunk)
  int64_t chunk = 0;
  int nchunk = 0;
  int part_gx = 0;    // grid x of the partial kernels
  int dec_nw = 8;     // waves per decode workgroup
  int dec_gx = 0;
  int64_t dec_tpw = 0;
  size_t off_acc = 0, off_l = 0, off_m = 0, off_q = 0, off_z = 0, total = 0;
};

// hilo: the plan of the backward's recompute and of the saved forward, whose partial kernels take the
// hi/lo instance.
Plan make_plan(int B, int H, int64_t N, int M, int D, int dtype, bool hilo = false) {
  Plan p;
  p.BH = B * H;
  p.H = H;
  p.Mp16 = (M + 15) / 16 * 16;
  p.Mp32 = (M + 31) / 32 * 32;
  // Partial-kernel variant: latents per wave x waves per workgroup, and latent groups per chunk.
  if (p.Mp16 <= 64) p.part_plan = 0;
  else if (p.Mp16 <= 128) p.part_plan = 1;
  else if (p.Mp16 <= 256 || dtype == FLAREPP_FP32) p.part_plan = 2;
  else p.part_plan = 3;  // bf16, M > 256: one 16-wave workgroup per chunk, 256-token stages
  const int plan_env = env_int("FLAREPP_PARTIAL_PLAN", -1);
  if (plan_env >= 0 && plan_env <= 3 && !(plan_env == 3 && dtype == FLAREPP_FP32)) p.part_plan = plan_env;
  const flarepp::PartialShape ps = flarepp::partial_plan_shape(p.part_plan);
  p.nlg = (int)ceil_div(p.Mp16, (int64_t)ps.lpw * ps.nw);
  // Workgroups over the token chunks: 256 for 16-wave groups (1 per CU), and for the 8-wave groups of
  // the plain forward (2 per CU); 512 otherwise. Fewer chunks make the merges cheaper, which
  // outweighs the partials' lower occupancy down to these counts. Measured per call: 1M-token
  // workload 2.04 -> 2.02 ms (against 512), M = 256 (8-wave) 0.219 -> 0.200 ms (512 against 1024 and
  // 2048) and 0.214-0.222 -> 0.204-0.210 ms (256 against 512, same box; the hi/lo instances there
  // took 103 + 93 us at 512 and 112 + 99 us at 256), M = 128 (4-wave) 0.174 -> 0.161 ms (512
  // against 1024 and 2048; 256 took 0.174), M = 64 (4-wave) 0.068 -> 0.059 ms (512; 256 took 0.071).
  const int64_t target =
      env_int("FLAREPP_PARTIAL_WORKGROUPS", ps.nw == 16 || (ps.nw == 8 && !hilo) ? 256 : 512);
  int64_t nchunk = ceil_div(target, (int64_t)p.BH * p.nlg);
  nchunk = nchunk < 1 ? 1 : nchunk;
  // At most 2048 chunks: the merge keeps a row block's chunk weights in LDS (16 rows x 2048 x 4 B).
  int64_t max_chunks = ceil_div(N, (int64_t)ps.stage);
  if (max_chunks > 2048) max_chunks = 2048;
  if (nchunk > max_chunks) nchunk = max_chunks;
  p.chunk = ceil_div(ceil_div(N, nchunk), (int64_t)ps.stage) * ps.stage;
  p.nchunk = (int)ceil_div(N, p.chunk);
  // With several latent groups, grid x holds 8 chunks per XCD slot row (see partial_kernel).
  p.part_gx = p.nlg == 1 ? p.nchunk : (int)(ceil_div(p.nchunk, 8) * 8 * p.nlg);
  // Decode: wider workgroups when Q and Z need more than half of the CU's LDS.
  p.dec_nw = flarepp::decode_lds_bytes(dtype, D, p.Mp32, flarepp::kDecodeWaves) > 80 * 1024
                 ? flarepp::kDecodeWavesWide : flarepp::kDecodeWaves;
  const int nw_env = env_int("FLAREPP_DECODE_WAVES", 0);
  if (nw_env == 8 || nw_env == 12 || nw_env == 16) p.dec_nw = nw_env;
  if (dtype == FLAREPP_FP32 && p.dec_nw == 12) p.dec_nw = 16;  // no 12-wave fp32 variant
  if (dtype == FLAREPP_BF16 && D == 32 && nw_env == 0) p.dec_nw = 16;  // pipelined 16-wave variant
  const int64_t group = flarepp::decode_group_tokens(dtype, D, p.dec_nw);
  const int64_t dec_target = env_int("FLAREPP_DECODE_WORKGROUPS", p.dec_nw == 8 ? 512 : 256);
  int64_t gx = ceil_div(dec_target, p.BH);
  const int64_t max_gx = ceil_div(N, group * p.dec_nw);
  if (gx > max_gx) gx = max_gx;
  if (gx < 1) gx = 1;
  p.dec_tpw = ceil_div(ceil_div(N, gx), group) * group;
  p.dec_gx = (int)ceil_div(N, p.dec_tpw);

  const size_t es = dtype == FLAREPP_BF16 ? 2 : 4;
  const size_t nrow = (size_t)p.BH * p.nchunk * p.Mp16;
  size_t off = 0;
  p.off_acc = off; off = align256(off + nrow * D * sizeof(float));
  p.off_l = off;   off = align256(off + nrow * sizeof(float));
  p.off_m = off;   off = align256(off + nrow * sizeof(float));
  const size_t qparts = dtype == FLAREPP_BF16 ? 3 : 1;  // bf16 routing queries: hi, lo and fp16
  p.off_q = off;   off = align256(off + (size_t)p.BH * p.Mp32 * qparts * D * es);
  p.off_z = off;   off = align256(off + (size_t)p.BH * p.Mp32 * D * es);
  p.total = off;
  return p;
}

std::atomic<int> g_force_exact{0};

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Size-only validation. Returns OK, or the status to report. Sets *empty when B*H*N == 0.
int validate_sizes(int B, int H, int64_t N, int M, int D, int dtype, bool* empty) {
  *empty = false;
  if (dtype != FLAREPP_FP32 && dtype != FLAREPP_BF16) return FLAREPP_UNSUPPORTED;
  if (B < 0 || H < 0 || N < 0 || M < 1) return FLAREPP_INVALID_ARGUMENT;
  if (D != 16 && D != 32) return FLAREPP_UNSUPPORTED;
  if (M > 512) return FLAREPP_UNSUPPORTED;
  if ((int64_t)B * H > 65535) return FLAREPP_UNSUPPORTED;
  // Element counts must stay far from int64 overflow (the kernels index with int64).
  if (N > ((int64_t)1 << 40) || (int64_t)B * H * N > ((int64_t)1 << 50)) return FLAREPP_INVALID_ARGUMENT;
  if ((int64_t)B * H * N == 0) *empty = true;
  return FLAREPP_OK;
}

// Device check, cached per device ordinal.
int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FLAREPP_DEVICE_ERROR;
  static std::mutex mu;
  static std::vector<int> cache;  // 0 unknown, 1 gfx950, 2 other
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FLAREPP_DEVICE_ERROR;
    cache[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
  }
  return cache[dev] == 1 ? FLAREPP_OK : FLAREPP_UNSUPPORTED;
}

// ---- per-kernel event timing
struct Timing {
  std::mutex mu;
  bool enabled = false;
  struct Rec { int kind; hipEvent_t a, b; };
  std::vector<Rec> pending;
  std::vector<hipEvent_t> pool;
  hipEvent_t get() {
    if (!pool.empty()) { hipEvent_t e = pool.back(); pool.pop_back(); return e; }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
Timing& timing() {
  static Timing t;
  return t;
}

template <typename F>
hipError_t run_kernel(int kind, hipStream_t st, F&& launch) {
  Timing& t = timing();
  if (!t.enabled) return launch();
  std::lock_guard<std::mutex> lock(t.mu);
  hipEvent_t a = t.get(), b = t.get();
  if (a) (void)hipEventRecord(a, st);
  hipError_t e = launch();
  if (b) (void)hipEventRecord(b, st);
  if (a && b) t.pending.push_back({kind, a, b});
  return e;
}

int validate_pointers(const void* K, const void* V, const void* S, const void* Qseed, const void* Qf,
                      const float* g, int B, int H, int64_t N, int M, int D, int dtype, const void* out) {
  if (!K || !V || !S || !Qseed || !Qf || !g || !out) return FLAREPP_INVALID_ARGUMENT;
  const void* ptrs[] = {K, V, S, Qseed, Qf, g, out};
  for (const void* p : ptrs)
    if ((uintptr_t)p & 15) return FLAREPP_MISALIGNED;
  const size_t es = dtype == FLAREPP_BF16 ? 2 : 4;
  const size_t nbig = (size_t)B * H * N * D * es, nq = (size_t)H * M * D * es;
  if (overlaps(out, nbig, K, nbig) || overlaps(out, nbig, V, nbig) || overlaps(out, nbig, S, nbig) ||
      overlaps(out, nbig, Qseed, nq) || overlaps(out, nbig, Qf, nq) || overlaps(out, nbig, g, H * sizeof(float)))
    return FLAREPP_INVALID_ARGUMENT;
  return FLAREPP_OK;
}

// Softmax normalizers the forward kernels leave for the backward pass (log2 units; null: not kept).
struct Saved {
  float* lsyn = nullptr;  // [BH][Mp32] synthesis, per latent
  float* lenc = nullptr;  // [BH][Mp32] encode, per latent
  bool hilo = false;      // split-N partials with hi/lo query logits on every pass (the backward's)
  bool no_decode = false; // stop after the encode merge
};

// Encode partials, merge and decode on the routing-query rows already in the workspace.
int enqueue_routing(const void* K, const void* V, int64_t N, int M, int D, int dtype, void* out, float* dZ,
                    void* ws, const Plan& p, hipStream_t st, const Saved& sv = Saved());

int enqueue(const void* K, const void* V, const void* S, const void* Qseed, const void* Qf, const float* g,
            int B, int H, int64_t N, int M, int D, int dtype, void* out, float* dQd, float* dQ, float* dZ,
            void* ws, const Plan& p, hipStream_t st, const Saved& sv = Saved()) {
  char* w = static_cast<char*>(ws);
  float* acc = reinterpret_cast<float*>(w + p.off_acc);
  float* pl = reinterpret_cast<float*>(w + p.off_l);
  float* pm = reinterpret_cast<float*>(w + p.off_m);
  void* qbuf = w + p.off_q;
  const int gx_part = p.part_gx;
  (void)B;

  flarepp::PartialArgs pa{};
  pa.K = S; pa.V = S; pa.Q = Qseed; pa.H = H; pa.Mq = M; pa.Mp = p.Mp16; pa.N = N;
  pa.chunk = p.chunk; pa.nchunk = p.nchunk; pa.nlg = p.nlg; pa.part_acc = acc;
  pa.force_exact = g_force_exact.load() ? 1 : 0; pa.hilo = sv.hilo ? 1 : 0; pa.part_l = pl; pa.part_m = pm;
  if (run_kernel(0, st, [&] { return flarepp::launch_partial(pa, dtype, D, true, p.part_plan, gx_part, p.BH, st); }) != hipSuccess)
    return FLAREPP_LAUNCH_FAILED;

  flarepp::MergeArgs ma{};
  ma.part_acc = acc; ma.part_l = pl; ma.part_m = pm; ma.nchunk = p.nchunk; ma.Mp = p.Mp16; ma.M = M;
  ma.Mout = p.Mp32; ma.H = H; ma.Qf = Qf; ma.g = g; ma.out = qbuf; ma.dbg_qd = dQd; ma.dbg_out = dQ;
  ma.lse = sv.lsyn;
  if (run_kernel(1, st, [&] { return flarepp::launch_merge(ma, dtype, D, true, p.BH, st); }) != hipSuccess)
    return FLAREPP_LAUNCH_FAILED;

  return enqueue_routing(K, V, N, M, D, dtype, out, dZ, ws, p, st, sv);
}

int enqueue_routing(const void* K, const void* V, int64_t N, int M, int D, int dtype, void* out, float* dZ,
                    void* ws, const Plan& p, hipStream_t st, const Saved& sv) {
  char* w = static_cast<char*>(ws);
  float* acc = reinterpret_cast<float*>(w + p.off_acc);
  float* pl = reinterpret_cast<float*>(w + p.off_l);
  float* pm = reinterpret_cast<float*>(w + p.off_m);
  void* qbuf = w + p.off_q;
  void* zbuf = w + p.off_z;

  flarepp::PartialArgs pa{};
  pa.K = K; pa.V = V; pa.Q = qbuf; pa.H = p.H; pa.Mq = p.Mp32; pa.Mp = p.Mp16; pa.N = N;
  pa.chunk = p.chunk; pa.nchunk = p.nchunk; pa.nlg = p.nlg; pa.part_acc = acc;
  pa.force_exact = g_force_exact.load() ? 1 : 0; pa.hilo = sv.hilo ? 1 : 0; pa.part_l = pl; pa.part_m = pm;
  if (run_kernel(2, st, [&] { return flarepp::launch_partial(pa, dtype, D, false, p.part_plan, p.part_gx, p.BH, st); }) != hipSuccess)
    return FLAREPP_LAUNCH_FAILED;

  flarepp::MergeArgs ma{};
  ma.part_acc = acc; ma.part_l = pl; ma.part_m = pm; ma.nchunk = p.nchunk; ma.Mp = p.Mp16; ma.M = M;
  ma.Mout = p.Mp32; ma.H = p.H; ma.Qf = nullptr; ma.g = nullptr; ma.out = zbuf; ma.dbg_qd = nullptr; ma.dbg_out = dZ;
  ma.lse = sv.lenc;
  if (run_kernel(3, st, [&] { return flarepp::launch_merge(ma, dtype, D, false, p.BH, st); }) != hipSuccess)
    return FLAREPP_LAUNCH_FAILED;
  if (sv.no_decode) return FLAREPP_OK;

  flarepp::DecodeArgs da{};
  da.K = K; da.Q = qbuf; da.Z = zbuf; da.out = out; da.N = N; da.M = M; da.Mp = p.Mp32; da.tokens_per_wg = p.dec_tpw;
  da.force_exact = pa.force_exact;
  if (run_kernel(4, st, [&] { return flarepp::launch_decode(da, dtype, D, p.dec_nw, p.dec_gx, p.BH, st); }) != hipSuccess)
    return FLAREPP_LAUNCH_FAILED;
  return FLAREPP_OK;
}

int mix_common(const void* K, const void* V, const void* S, const void* Qseed, const void* Qf, const float* g,
               int B, int H, int64_t N, int M, int D, int dtype, void* out, float* dQd, float* dQ, float* dZ,
               void* ws, size_t ws_bytes, bool own_ws, hipStream_t st) {
  bool empty = false;
  int rc = validate_sizes(B, H, N, M, D, dtype, &empty);
  if (rc != FLAREPP_OK || empty) return rc;
  rc = validate_pointers(K, V, S, Qseed, Qf, g, B, H, N, M, D, dtype, out);
  if (rc != FLAREPP_OK) return rc;
  const Plan p = make_plan(B, H, N, M, D, dtype);
  if (!own_ws) {
    if (!ws || ws_bytes < p.total) return FLAREPP_INVALID_ARGUMENT;
    if ((uintptr_t)ws & 255) return FLAREPP_MISALIGNED;
  }
  rc = check_device();
  if (rc != FLAREPP_OK) return rc;
  if (own_ws) {
    if (hipMallocAsync(&ws, p.total, st) != hipSuccess) {
      (void)hipGetLastError();
      return FLAREPP_OUT_OF_MEMORY;
    }
  }
  rc = enqueue(K, V, S, Qseed, Qf, g, B, H, N, M, D, dtype, out, dQd, dQ, dZ, ws, p, st);
  if (own_ws) (void)hipFreeAsync(ws, st);
  return rc;
}

// ---- The mixer without allocation (flarepp_mix_noalloc)
//
// Its workspace is this file-scope device array: every GPU the library runs on holds one copy of it
// from the module's load until the process ends, at an address of its own. The host never uses the
// array's name as a device address; it looks the address up once per device and passes that
// pointer to the kernels, as the other entry points pass their workspace. The workspace needs no
// clearing: the kernels write every entry they later read. Calls that overlap on one GPU share the
// array and race.
__device__ __align__(256) unsigned char scratch[FLAREPP_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on the current device, looked up on the first call per device (with
// that device current) and kept.
int noalloc_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return FLAREPP_DEVICE_ERROR;
  }
  static std::mutex mu;
  static std::vector<void*> ptrs;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)ptrs.size() <= dev) ptrs.resize(dev + 1, nullptr);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return FLAREPP_DEVICE_ERROR;
    }
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return FLAREPP_OK;
}

int mix_noalloc_common(const void* K, const void* V, const void* S, const void* Qseed, const void* Qf,
                       const float* g, int B, int H, int64_t N, int M, int D, int dtype, void* out, hipStream_t st) {
  bool empty = false;
  int rc = validate_sizes(B, H, N, M, D, dtype, &empty);
  if (rc != FLAREPP_OK || empty) return rc;
  rc = validate_pointers(K, V, S, Qseed, Qf, g, B, H, N, M, D, dtype, out);
  if (rc != FLAREPP_OK) return rc;
  const Plan p = make_plan(B, H, N, M, D, dtype);
  if (p.total > (size_t)FLAREPP_NOALLOC_SCRATCH_BYTES) return FLAREPP_SCRATCH_TOO_SMALL;
  rc = check_device();
  if (rc != FLAREPP_OK) return rc;
  void* ws = nullptr;
  rc = noalloc_scratch(&ws);
  if (rc != FLAREPP_OK) return rc;
  return enqueue(K, V, S, Qseed, Qf, g, B, H, N, M, D, dtype, out, nullptr, nullptr, nullptr, ws, p, st);
}

int flare_common(const void* K, const void* V, const void* Q, int B, int H, int64_t N, int M, int D, int dtype,
                 void* out, void* ws, size_t ws_bytes, bool own_ws, hipStream_t st) {
  bool empty = false;
  int rc = validate_sizes(B, H, N, M, D, dtype, &empty);
  if (rc != FLAREPP_OK || empty) return rc;
  if (!K || !V || !Q || !out) return FLAREPP_INVALID_ARGUMENT;
  const void* ptrs[] = {K, V, Q, out};
  for (const void* p : ptrs)
    if ((uintptr_t)p & 15) return FLAREPP_MISALIGNED;
  const size_t es = dtype == FLAREPP_BF16 ? 2 : 4;
  const size_t nbig = (size_t)B * H * N * D * es, nq = (size_t)H * M * D * es;
  if (overlaps(out, nbig, K, nbig) || overlaps(out, nbig, V, nbig) || overlaps(out, nbig, Q, nq))
    return FLAREPP_INVALID_ARGUMENT;
  const Plan p = make_plan(B, H, N, M, D, dtype);
  if (!own_ws) {
    if (!ws || ws_bytes < p.total) return FLAREPP_INVALID_ARGUMENT;
    if ((uintptr_t)ws & 255) return FLAREPP_MISALIGNED;
  }
  rc = check_device();
  if (rc != FLAREPP_OK) return rc;
  if (own_ws) {
    if (hipMallocAsync(&ws, p.total, st) != hipSuccess) {
      (void)hipGetLastError();
      return FLAREPP_OUT_OF_MEMORY;
    }
  }
  flarepp::QueryPrepArgs qa{};
  qa.Q = Q; qa.H = H; qa.M = M; qa.Mout = p.Mp32; qa.out = static_cast<char*>(ws) + p.off_q;
  if (run_kernel(5, st, [&] { return flarepp::launch_query_prep(qa, dtype, D, p.BH, st); }) != hipSuccess)
    rc = FLAREPP_LAUNCH_FAILED;
  else
    rc = enqueue_routing(K, V, N, M, D, dtype, out, nullptr, ws, p, st);
  if (own_ws) (void)hipFreeAsync(ws, st);
  return rc;
}

// Simplified FLARE++ (Appendix A.8, Eq. 20): the seeds as fixed queries of the encode engine over
// the caller's synthesis keys Sk and values Sv give Qd, which the gate merge (without Qf) emits as
// the routing queries; then encode, merge and decode as for the mixer.
int simplified_common(const void* K, const void* V, const void* Sk, const void* Sv, const void* Qseed, int B, int H,
                      int64_t N, int M, int D, int dtype, void* out, void* ws, size_t ws_bytes, bool own_ws,
                      hipStream_t st) {
  bool empty = false;
  int rc = validate_sizes(B, H, N, M, D, dtype, &empty);
  if (rc != FLAREPP_OK || empty) return rc;
  if (!K || !V || !Sk || !Sv || !Qseed || !out) return FLAREPP_INVALID_ARGUMENT;
  const void* ptrs[] = {K, V, Sk, Sv, Qseed, out};
  for (const void* p : ptrs)
    if ((uintptr_t)p & 15) return FLAREPP_MISALIGNED;
  const size_t es = dtype == FLAREPP_BF16 ? 2 : 4;
  const size_t nbig = (size_t)B * H * N * D * es, nq = (size_t)H * M * D * es;
  if (overlaps(out, nbig, K, nbig) || overlaps(out, nbig, V, nbig) || overlaps(out, nbig, Sk, nbig) ||
      overlaps(out, nbig, Sv, nbig) || overlaps(out, nbig, Qseed, nq))
    return FLAREPP_INVALID_ARGUMENT;
  const Plan p = make_plan(B, H, N, M, D, dtype);
  if (!own_ws) {
    if (!ws || ws_bytes < p.total) return FLAREPP_INVALID_ARGUMENT;
    if ((uintptr_t)ws & 255) return FLAREPP_MISALIGNED;
  }
  rc = check_device();
  if (rc != FLAREPP_OK) return rc;
  if (own_ws) {
    if (hipMallocAsync(&ws, p.total, st) != hipSuccess) {
      (void)hipGetLastError();
      return FLAREPP_OUT_OF_MEMORY;
    }
  }
  char* w = static_cast<char*>(ws);
  void* qbuf = w + p.off_q;
  float* acc = reinterpret_cast<float*>(w + p.off_acc);
  float* pl = reinterpret_cast<float*>(w + p.off_l);
  float* pm = reinterpret_cast<float*>(w + p.off_m);
  rc = FLAREPP_OK;
  flarepp::QueryPrepArgs qa{};
  qa.Q = Qseed; qa.H = H; qa.M = M; qa.Mout = p.Mp32; qa.out = qbuf;
  flarepp::PartialArgs pa{};
  pa.K = Sk; pa.V = Sv; pa.Q = qbuf; pa.H = H; pa.Mq = p.Mp32; pa.Mp = p.Mp16; pa.N = N;
  pa.chunk = p.chunk; pa.nchunk = p.nchunk; pa.nlg = p.nlg; pa.part_acc = acc;
  pa.force_exact = g_force_exact.load(); pa.part_l = pl; pa.part_m = pm;
  flarepp::MergeArgs ma{};
  ma.part_acc = acc; ma.part_l = pl; ma.part_m = pm; ma.nchunk = p.nchunk; ma.Mp = p.Mp16; ma.M = M;
  ma.Mout = p.Mp32; ma.H = H; ma.Qf = nullptr; ma.g = nullptr; ma.out = qbuf;
  if (run_kernel(5, st, [&] { return flarepp::launch_query_prep(qa, dtype, D, p.BH, st); }) != hipSuccess ||
      run_kernel(0, st, [&] { return flarepp::launch_partial(pa, dtype, D, false, p.part_plan, p.part_gx, p.BH, st); }) != hipSuccess ||
      run_kernel(1, st, [&] { return flarepp::launch_merge(ma, dtype, D, true, p.BH, st); }) != hipSuccess)
    rc = FLAREPP_LAUNCH_FAILED;
  else
    rc = enqueue_routing(K, V, N, M, D, dtype, out, nullptr, ws, p, st);
  if (own_ws) (void)hipFreeAsync(ws, st);
  return rc;
}

// ---- Backward pass
//
// The synthesis and encode calls are recomputed with hi/lo query logits (the backward kernels'
// logits) and hi/lo P.V products (the partial kernel's HILO instance) and their normalizers kept, Z is centered, and the decode kernel forms every token's
// statistics and the decode call's part of dK; then, per routing call in reverse order (Appendix
// B.5, Eq. 46-49): the latent-side partials and their reduction for the decode call (dZ, dQ_dec)
// and the encode call (dQ_enc, then the gate), the synthesis call (dQseed and the batch sums), and
// the token-side kernels of the encode call (dK, dV) and the synthesis call (dS).
struct BwdPlan {
  Plan f;
  int Mp = 0;
  int lat_nw = 4, lat_nlg = 1, lat_nchunk = 0, lat_gx = 0;
  int64_t lat_chunk = 0;
  int tok_gx = 0;
  int tok_nw = flarepp::kBwdTokenWavesWide;  // waves per workgroup of the token encode and synthesis kernels
  int tok_dec_nw = flarepp::kBwdTokenWaves;  // ... and of the token decode kernel
  int64_t tok_tpw = 0;
  size_t off_qd = 0, off_z32 = 0, off_lsyn = 0, off_lenc = 0, off_zc = 0, off_zc_lo = 0, off_ldec = 0;
  size_t off_cd = 0, off_dkdec = 0, off_p0 = 0, off_p1 = 0, off_dz32 = 0, off_dzop = 0, off_dzop_lo = 0;
  size_t off_tmax = 0;
  size_t off_ce = 0, off_dqdec = 0, off_dqf = 0, off_gop = 0, off_gop_lo = 0, off_cs = 0, off_rowdot = 0;
  size_t off_zmax = 0;
  size_t total = 0;
};

BwdPlan make_bwd_plan(int B, int H, int64_t N, int M, int D, int dtype) {
  BwdPlan p;
  p.f = make_plan(B, H, N, M, D, dtype, true);
  const int BH = p.f.BH;
  p.Mp = p.f.Mp32;
  // Latent side: one wave per 32 latents, groups of 4 or 8 waves; about 512 workgroups over the token
  // chunks (a sweep of 256-4096 at the four bf16 workloads: 512 was within 2% of the best at each;
  // more chunks cost the latent kernels and their reductions more than they gain in occupancy).
  p.lat_nw = flarepp::bwd_latent_waves(p.Mp);

  p.lat_nlg = (int)ceil_div(p.Mp, 32 * p.lat_nw);
  const int64_t target = env_int("FLAREPP_BWD_LATENT_WORKGROUPS", 512);
  int64_t nchunk = ceil_div(target, (int64_t)BH * p.lat_nlg);
  const int64_t stage = flarepp::bwd_stage(dtype, p.lat_nw);
  const int64_t max_chunks = ceil_div(N, stage);
  if (nchunk > max_chunks) nchunk = max_chunks;
  if (nchunk < 1) nchunk = 1;
  p.lat_chunk = ceil_div(ceil_div(N, nchunk), stage) * stage;
  p.lat_nchunk = (int)ceil_div(N, p.lat_chunk);
  p.lat_gx = p.lat_nlg == 1 ? p.lat_nchunk : (int)(ceil_div(p.lat_nchunk, 8) * 8 * p.lat_nlg);
  // Token side: 256 or 512 workgroups, 32-token blocks. The latent tensors in LDS leave room for one
  // workgroup per CU: 12 waves (3 per SIMD) for encode and synthesis, and for the decode kernel
  // where its registers allow (bwd_decode_waves).
  const int tok_env = env_int("FLAREPP_BWD_TOKEN_WAVES", 0);
  if (tok_env == 8 || tok_env == 12) p.tok_nw = tok_env;
  p.tok_dec_nw = flarepp::bwd_decode_waves(dtype);
  const int dec_env = env_int("FLAREPP_BWD_DECODE_WAVES", 0);
  if (dec_env == 8 || (dec_env == 12 && dtype == FLAREPP_BF16)) p.tok_dec_nw = dec_env;
  // One workgroup per CU (256) unless each (b, h) has more than 2^27 token-latent pairs; there two
  // rounds of 512 ran 2-4% faster (a sweep of 128-1024 at the four bf16 workloads).
  const int64_t tok_target =
      env_int("FLAREPP_BWD_TOKEN_WORKGROUPS", N * (int64_t)p.Mp > ((int64_t)1 << 27) ? 512 : 256);
  int64_t gx = ceil_div(tok_target, (int64_t)BH);
  const int64_t max_gx = ceil_div(N, (int64_t)32 * flarepp::kBwdTokenWaves);
  if (gx > max_gx) gx = max_gx;
  if (gx < 1) gx = 1;
  p.tok_tpw = ceil_div(ceil_div(N, gx), (int64_t)32) * 32;
  p.tok_gx = (int)ceil_div(N, p.tok_tpw);

  const size_t es = dtype == FLAREPP_BF16 ? 2 : 4;
  const size_t lat = (size_t)BH * p.Mp;  // latent rows
  size_t off = p.f.total;
  p.off_qd = off;     off = align256(off + (size_t)BH * M * D * 4);
  p.off_z32 = off;    off = align256(off + (size_t)BH * M * D * 4);
  p.off_lsyn = off;   off = align256(off + lat * 4);
  p.off_lenc = off;   off = align256(off + lat * 4);
  p.off_zc = off;     off = align256(off + lat * D * es);
  p.off_zc_lo = off;  off = align256(off + lat * D * es);
  p.off_ldec = off;   off = align256(off + (size_t)BH * N * 4);
  p.off_cd = off;     off = align256(off + (size_t)BH * N * 4);
  // The decode call's part of dK in fp32 (fp32 runs keep it in dK itself).
  p.off_dkdec = off;  off = align256(off + (dtype == FLAREPP_BF16 ? (size_t)BH * N * D * 4 : 0));
  p.off_p0 = off;     off = align256(off + (size_t)BH * p.lat_nchunk * p.Mp * D * 4);
  p.off_p1 = off;     off = align256(off + (size_t)BH * p.lat_nchunk * p.Mp * D * 4);
  p.off_dz32 = off;   off = align256(off + lat * D * 4);
  p.off_dzop = off;   off = align256(off + lat * D * es);
  p.off_dzop_lo = off; off = align256(off + lat * D * es);
  p.off_ce = off;     off = align256(off + lat * 4);
  p.off_dqdec = off;  off = align256(off + lat * D * 4);
  p.off_dqf = off;    off = align256(off + lat * D * 4);
  p.off_gop = off;    off = align256(off + lat * D * es);
  p.off_gop_lo = off; off = align256(off + lat * D * es);
  p.off_cs = off;     off = align256(off + lat * 4);
  p.off_rowdot = off; off = align256(off + lat * 4);
  p.off_zmax = off;   off = align256(off + (size_t)BH * 4);
  p.off_tmax = off;   off = align256(off + (size_t)BH * p.tok_gx * p.tok_dec_nw * 2 * 4);
  p.total = off;
  return p;
}

// Sizes the backward kernels support beyond the forward's: the token-side kernels keep the latent
// tensors of one (batch, head) in LDS (160 KiB).
int validate_bwd_sizes(int B, int H, int64_t N, int M, int D, int dtype, bool* empty) {
  int rc = validate_sizes(B, H, N, M, D, dtype, empty);
  if (rc != FLAREPP_OK) return rc;
  const int Mp = (M + 31) / 32 * 32;
  for (int kind : {flarepp::kBwdTokDecode, flarepp::kBwdTokEncode, flarepp::kBwdTokSynthesis})
    if (flarepp::bwd_token_lds_bytes(dtype, D, Mp, kind) > 160 * 1024) return FLAREPP_UNSUPPORTED;
  return FLAREPP_OK;
}

// The forward state the backward starts from (Appendix B.3 and B.5: the forward keeps each routing
// call's log-normalizer and output): the synthesis and encode partials with hi/lo query logits and
// hi/lo P.V products, merged into the routing-query rows, Z and Qd in fp32 and both calls'
// per-latent log2 normalizers, all in the backward workspace. With `out` the decode runs too and
// writes the mixer's output.
int enqueue_saved_forward(const void* K, const void* V, const void* S, const void* Qseed, const void* Qf,
                          const float* g, int B, int H, int64_t N, int M, int D, int dtype, void* out, void* ws,
                          const BwdPlan& p, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  auto F = [&](size_t off) { return reinterpret_cast<float*>(w + off); };
  Saved sv;
  sv.lsyn = F(p.off_lsyn);
  sv.lenc = F(p.off_lenc);
  sv.hilo = true;
  sv.no_decode = out == nullptr;
  return enqueue(K, V, S, Qseed, Qf, g, B, H, N, M, D, dtype, out, F(p.off_qd), nullptr, F(p.off_z32), ws, p.f, st,
                 sv);
}

// The backward proper, from the state enqueue_saved_forward left in the workspace.
int enqueue_backward_from_saved(const void* K, const void* V, const void* S, const void* Qseed, const void* Qf,
                                const float* g, const void* dY, int B, int H, int64_t N, int M, int D, int dtype,
                                void* dK, void* dV, void* dS, void* dQseed, void* dQf, float* dg, void* ws,
                                const BwdPlan& p, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  auto F = [&](size_t off) { return reinterpret_cast<float*>(w + off); };
  const int BH = p.f.BH;
  Saved sv;
  sv.lsyn = F(p.off_lsyn);
  sv.lenc = F(p.off_lenc);
  void* qrows = w + p.f.off_q;
  float* ldec = F(p.off_ldec);
  float* cd = F(p.off_cd);
  float* dkdec = dtype == FLAREPP_BF16 ? F(p.off_dkdec) : static_cast<float*>(dK);

  flarepp::BwdCenterArgs ca{};
  ca.Z32 = F(p.off_z32); ca.Zc = w + p.off_zc; ca.Zc_lo = w + p.off_zc_lo; ca.zmax = F(p.off_zmax); ca.M = M;
  ca.Mp = p.Mp;
  if (run_kernel(6, st, [&] { return flarepp::launch_bwd_center(ca, dtype, D, BH, st); }) != hipSuccess)
    return FLAREPP_LAUNCH_FAILED;

  flarepp::BwdTokenArgs ta{};
  ta.K = K; ta.V = V; ta.dY = dY; ta.S = S; ta.tl = ldec; ta.tc = cd; ta.dKdec = dkdec; ta.Qrows = qrows;
  ta.Zc = w + p.off_zc; ta.Zc_lo = w + p.off_zc_lo; ta.zmax = F(p.off_zmax); ta.tmax = F(p.off_tmax); ta.dZop = w + p.off_dzop; ta.dZ_lo = w + p.off_dzop_lo;
  ta.lenc = sv.lenc; ta.ce = F(p.off_ce); ta.dZ32 = F(p.off_dz32); ta.Z32 = F(p.off_z32); ta.Qseed = Qseed; ta.Gop = w + p.off_gop; ta.G_lo = w + p.off_gop_lo;
  ta.lsyn = sv.lsyn; ta.cs = F(p.off_cs); ta.dK = dK; ta.dV = dV; ta.dS = dS; ta.N = N;
  ta.tokens_per_wg = p.tok_tpw; ta.M = M; ta.Mp = p.Mp; ta.H = H; ta.force_exact = g_force_exact.load() ? 1 : 0;
  if (run_kernel(7, st, [&] { return flarepp::launch_bwd_token(ta, dtype, D, flarepp::kBwdTokDecode, p.tok_dec_nw, p.tok_gx, BH, st); }) != hipSuccess)
    return FLAREPP_LAUNCH_FAILED;

  flarepp::BwdLatentArgs la{};
  la.N = N; la.chunk = p.lat_chunk; la.nchunk = p.lat_nchunk; la.nlg = p.lat_nlg; la.M = M; la.Mp = p.Mp; la.H = H;
  la.part0 = F(p.off_p0); la.part1 = F(p.off_p1);
  la.tmax = F(p.off_tmax); la.zmax = F(p.off_zmax); la.ntmax = p.tok_gx * p.tok_dec_nw;
  flarepp::BwdReduceArgs ra{};
  ra.part0 = la.part0; ra.part1 = la.part1; ra.nchunk = p.lat_nchunk; ra.M = M; ra.Mp = p.Mp; ra.H = H; ra.B = B;
  ra.Z32 = F(p.off_z32); ra.dZ32 = F(p.off_dz32); ra.dZop = w + p.off_dzop; ra.dZop_lo = w + p.off_dzop_lo;
  ra.ce = F(p.off_ce); ra.dQdec = F(p.off_dqdec); ra.Qf = Qf; ra.g = g; ra.Qd32 = F(p.off_qd);
  ra.dQf_bh = F(p.off_dqf); ra.Gop = w + p.off_gop; ra.Gop_lo = w + p.off_gop_lo; ra.cs = F(p.off_cs);
  ra.rowdot = F(p.off_rowdot); ra.dQseed = dQseed; ra.dQf = dQf; ra.dg = dg;

  // Decode call: dZ and dQ_dec.
  la.X = K; la.W = dY; la.tl = ldec; la.tc = cd; la.Qr = qrows; la.Wr = w + p.off_zc; la.Wr_lo = w + p.off_zc_lo;
  la.ll = nullptr; la.lc = nullptr;
  if (run_kernel(8, st, [&] { return flarepp::launch_bwd_latent(la, dtype, D, flarepp::kBwdDecode, p.lat_nw, p.lat_gx, BH, st); }) != hipSuccess)
    return FLAREPP_LAUNCH_FAILED;
  if (run_kernel(9, st, [&] { return flarepp::launch_bwd_reduce(ra, dtype, D, flarepp::kBwdDecode, BH, st); }) != hipSuccess)
    return FLAREPP_LAUNCH_FAILED;
  // Encode call: dQ_enc, then the gate.
  la.X = K; la.W = V; la.tl = nullptr; la.tc = nullptr; la.Qr = qrows; la.Wr = w + p.off_dzop;
  la.Wr_lo = w + p.off_dzop_lo; la.ll = sv.lenc; la.lc = F(p.off_ce);
  if (run_kernel(10, st, [&] { return flarepp::launch_bwd_latent(la, dtype, D, flarepp::kBwdEncode, p.lat_nw, p.lat_gx, BH, st); }) != hipSuccess)
    return FLAREPP_LAUNCH_FAILED;
  if (run_kernel(11, st, [&] { return flarepp::launch_bwd_reduce(ra, dtype, D, flarepp::kBwdEncode, BH, st); }) != hipSuccess)
    return FLAREPP_LAUNCH_FAILED;
  // Synthesis call: dQseed, and the batch sums of the shared parameters.
  la.X = S; la.W = nullptr; la.Qr = Qseed; la.Wr = w + p.off_gop; la.Wr_lo = w + p.off_gop_lo; la.ll = sv.lsyn;
  la.lc = F(p.off_cs);
  if (run_kernel(12, st, [&] { return flarepp::launch_bwd_latent(la, dtype, D, flarepp::kBwdSynthesis, p.lat_nw, p.lat_gx, BH, st); }) != hipSuccess)
    return FLAREPP_LAUNCH_FAILED;
  if (run_kernel(13, st, [&] { return flarepp::launch_bwd_reduce(ra, dtype, D, flarepp::kBwdSynthesis, BH, st); }) != hipSuccess)
    return FLAREPP_LAUNCH_FAILED;

  if (run_kernel(14, st, [&] { return flarepp::launch_bwd_token(ta, dtype, D, flarepp::kBwdTokEncode, p.tok_nw, p.tok_gx, BH, st); }) != hipSuccess)
    return FLAREPP_LAUNCH_FAILED;
  if (run_kernel(15, st, [&] { return flarepp::launch_bwd_token(ta, dtype, D, flarepp::kBwdTokSynthesis, p.tok_nw, p.tok_gx, BH, st); }) != hipSuccess)
    return FLAREPP_LAUNCH_FAILED;
  return FLAREPP_OK;
}

int enqueue_backward(const void* K, const void* V, const void* S, const void* Qseed, const void* Qf,
                     const float* g, const void* dY, int B, int H, int64_t N, int M, int D, int dtype, void* dK,
                     void* dV, void* dS, void* dQseed, void* dQf, float* dg, void* ws, const BwdPlan& p,
                     hipStream_t st) {
  const int rc = enqueue_saved_forward(K, V, S, Qseed, Qf, g, B, H, N, M, D, dtype, nullptr, ws, p, st);
  if (rc != FLAREPP_OK) return rc;
  return enqueue_backward_from_saved(K, V, S, Qseed, Qf, g, dY, B, H, N, M, D, dtype, dK, dV, dS, dQseed, dQf, dg,
                                     ws, p, st);
}

// from_saved: the workspace holds the state of flarepp_mix_forward_saved for the same inputs, and the
// backward starts from it instead of recomputing it.
int backward_common(const void* K, const void* V, const void* S, const void* Qseed, const void* Qf, const float* g,
                    const void* dY, int B, int H, int64_t N, int M, int D, int dtype, void* dK, void* dV, void* dS,
                    void* dQseed, void* dQf, float* dg, void* ws, size_t ws_bytes, bool own_ws, hipStream_t st,
                    bool from_saved = false) {
  bool empty = false;
  int rc = validate_bwd_sizes(B, H, N, M, D, dtype, &empty);
  if (rc != FLAREPP_OK) return rc;
  const size_t es = dtype == FLAREPP_BF16 ? 2 : 4;
  const size_t nbig = (size_t)B * H * N * D * es, nq = (size_t)H * M * D * es, ng = (size_t)H * sizeof(float);
  struct Buf { const void* p; size_t n; bool out; };
  const Buf bufs[] = {{K, nbig, false}, {V, nbig, false}, {S, nbig, false}, {Qseed, nq, false}, {Qf, nq, false},
                      {g, ng, false}, {dY, nbig, false}, {dK, nbig, true}, {dV, nbig, true}, {dS, nbig, true},
                      {dQseed, nq, true}, {dQf, nq, true}, {dg, ng, true}};
  for (const Buf& b : bufs) {
    if (!b.p && b.n) return FLAREPP_INVALID_ARGUMENT;
    if ((uintptr_t)b.p & 15) return FLAREPP_MISALIGNED;
  }
  // Every output is disjoint from every other buffer.
  for (const Buf& a : bufs)
    for (const Buf& b : bufs)
      if (&a != &b && (a.out || b.out) && a.n && b.n && overlaps(a.p, a.n, b.p, b.n)) return FLAREPP_INVALID_ARGUMENT;
  if (empty) {
    // No token reaches an output: the shared parameters' cotangents are zero.
    if (nq == 0) return FLAREPP_OK;
    rc = check_device();
    if (rc != FLAREPP_OK) return rc;
    if (flarepp::launch_bwd_zero(dQseed, nq, st) != hipSuccess || flarepp::launch_bwd_zero(dQf, nq, st) != hipSuccess ||
        flarepp::launch_bwd_zero(dg, ng, st) != hipSuccess)
      return FLAREPP_LAUNCH_FAILED;
    return FLAREPP_OK;
  }
  const BwdPlan p = make_bwd_plan(B, H, N, M, D, dtype);
  if (!own_ws) {
    if (!ws || ws_bytes < p.total) return FLAREPP_INVALID_ARGUMENT;
    if ((uintptr_t)ws & 255) return FLAREPP_MISALIGNED;
  }
  rc = check_device();
  if (rc != FLAREPP_OK) return rc;
  if (own_ws) {
    if (hipMallocAsync(&ws, p.total, st) != hipSuccess) {
      (void)hipGetLastError();
      return FLAREPP_OUT_OF_MEMORY;
    }
  }
  rc = from_saved ? enqueue_backward_from_saved(K, V, S, Qseed, Qf, g, dY, B, H, N, M, D, dtype, dK, dV, dS, dQseed,
                                                dQf, dg, ws, p, st)
                  : enqueue_backward(K, V, S, Qseed, Qf, g, dY, B, H, N, M, D, dtype, dK, dV, dS, dQseed, dQf, dg,
                                     ws, p, st);
  if (own_ws) (void)hipFreeAsync(ws, st);
  return rc;
}

// The forward that keeps the state the backward starts from (flarepp_mix_forward_saved).
int forward_saved_common(const void* K, const void* V, const void* S, const void* Qseed, const void* Qf,
                         const float* g, int B, int H, int64_t N, int M, int D, int dtype, void* out, void* ws,
                         size_t ws_bytes, hipStream_t st) {
  bool empty = false;
  int rc = validate_bwd_sizes(B, H, N, M, D, dtype, &empty);
  if (rc != FLAREPP_OK || empty) return rc;
  rc = validate_pointers(K, V, S, Qseed, Qf, g, B, H, N, M, D, dtype, out);
  if (rc != FLAREPP_OK) return rc;
  const BwdPlan p = make_bwd_plan(B, H, N, M, D, dtype);
  if (!ws || ws_bytes < p.total) return FLAREPP_INVALID_ARGUMENT;
  if ((uintptr_t)ws & 255) return FLAREPP_MISALIGNED;
  rc = check_device();
  if (rc != FLAREPP_OK) return rc;
  return enqueue_saved_forward(K, V, S, Qseed, Qf, g, B, H, N, M, D, dtype, out, ws, p, st);
}

// ---- Projections around the mixer and the whole block --------------------------------------

// Largest channel width C = H * D whose weight rows fit the projection kernel's registers.
int proj_max_channels(int dtype) { return dtype == FLAREPP_BF16 ? 512 : 256; }

int validate_proj_sizes(int B, int H, int64_t N, int D, int dtype, bool* empty) {
  *empty = false;
  if (dtype != FLAREPP_FP32 && dtype != FLAREPP_BF16) return FLAREPP_UNSUPPORTED;
  if (B < 0 || H < 0 || N < 0) return FLAREPP_INVALID_ARGUMENT;
  if (D != 16 && D != 32) return FLAREPP_UNSUPPORTED;
  if ((int64_t)H * D > proj_max_channels(dtype)) return FLAREPP_UNSUPPORTED;
  // Token tiles are counted in int; elements in int64.
  if (N > ((int64_t)1 << 35) || B > 65535) return FLAREPP_INVALID_ARGUMENT;
  if ((int64_t)B * H * N == 0) *empty = true;
  return FLAREPP_OK;
}

struct ProjPlan {
  flarepp::ProjArgs a{};
  int grid = 0;
};

ProjPlan make_proj_plan(int B, int H, int64_t N, int D, int dtype, int nproj) {
  ProjPlan p;
  const int C = H * D;
  const int64_t groups = ceil_div((int64_t)nproj * C, 32);
  const int64_t ngb = ceil_div(groups, (int64_t)flarepp::proj_waves(dtype, C));
  const int64_t ntiles = ceil_div(N, flarepp::kProjTile);
  // About 2048 workgroups (one per CU at a time, eight rounds: shorter token ranges even out the
  // finish); at least 8 tiles each so that a workgroup's weight loads stay small against its token
  // work.
  const int64_t target = env_int("FLAREPP_PROJECT_WORKGROUPS", 2048);
  int64_t tpw = ceil_div((int64_t)B * ntiles * ngb, target);
  if (tpw < 8) tpw = 8;
  const int64_t nranges = ceil_div(ntiles, tpw);
  p.a.H = H;
  p.a.C = C;
  p.a.nproj = nproj;
  p.a.ngb = (int)ngb;
  p.a.N = N;
  p.a.ntiles = (int)ntiles;
  p.a.tiles_per_wg = (int)tpw;
  p.a.nranges = (int)nranges;
  p.a.nwg = (int)(B * nranges * ngb);
  p.grid = (int)(ceil_div(p.a.nwg, 8) * 8);
  return p;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int enqueue_project(const void* X, const void* const W[3], const void* const bias[3], const void* scale,
                    void* const outs[3], int B, int H, int64_t N, int D, int dtype, bool front, hipStream_t st) {
  ProjPlan p = make_proj_plan(B, H, N, D, dtype, front ? 3 : 1);
  p.a.X = X;
  for (int i = 0; i < 3; i++) {
    p.a.W[i] = W[i];
    p.a.bias[i] = bias[i];
    p.a.out[i] = outs[i];
  }
  p.a.scale = scale;
  if (run_kernel(front ? 16 : 17, st, [&] { return flarepp::launch_project(p.a, dtype, D, front, p.grid, st); }) != hipSuccess)
    return FLAREPP_LAUNCH_FAILED;
  return FLAREPP_OK;
}

// Pointer checks shared by the projection entry points: the listed tensors non-null where required
// and 16-byte aligned (optional ones: element-aligned), outputs disjoint from every input and from
// each other.
struct Span {
  const void* p;
  size_t n;
};
bool any_overlap(const Span* outs, int no, const Span* ins, int ni) {
  for (int i = 0; i < no; i++) {
    for (int j = 0; j < ni; j++)
      if (ins[j].p && overlaps(outs[i].p, outs[i].n, ins[j].p, ins[j].n)) return true;
    for (int j = i + 1; j < no; j++)
      if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return true;
  }
  return false;
}

int project_common(const void* X, const void* Wk, const void* Wv, const void* Ws, const void* bk, const void* bv,
                   const void* bs, const void* nk, int B, int H, int64_t N, int D, int dtype, void* K, void* V,
                   void* S, hipStream_t st) {
  bool empty = false;
  int rc = validate_proj_sizes(B, H, N, D, dtype, &empty);
  if (rc != FLAREPP_OK || empty) return rc;
  if (!X || !Wk || !Wv || !Ws || !K || !V || !S) return FLAREPP_INVALID_ARGUMENT;
  const size_t es = dtype == FLAREPP_BF16 ? 2 : 4;
  for (const void* q : {X, Wk, Wv, Ws, (const void*)K, (const void*)V, (const void*)S})
    if (!aligned(q, 16)) return FLAREPP_MISALIGNED;
  for (const void* q : {bk, bv, bs, nk})
    if (q && !aligned(q, es)) return FLAREPP_MISALIGNED;
  const size_t C = (size_t)H * D, big = (size_t)B * N * C * es;
  const Span outs[] = {{K, big}, {V, big}, {S, big}};
  const Span ins[] = {{X, big}, {Wk, C * C * es}, {Wv, C * C * es}, {Ws, C * C * es},
                      {bk, C * es}, {bv, C * es}, {bs, C * es}, {nk, D * es}};
  if (any_overlap(outs, 3, ins, 8)) return FLAREPP_INVALID_ARGUMENT;
  rc = check_device();
  if (rc != FLAREPP_OK) return rc;
  const void* W[3] = {Wk, Wv, Ws};
  const void* bias[3] = {bk, bv, bs};
  void* o[3] = {K, V, S};
  return enqueue_project(X, W, bias, nk, o, B, H, N, D, dtype, true, st);
}

int out_project_common(const void* Y, const void* Wo, const void* bo, int B, int H, int64_t N, int D, int dtype,
                       void* out, hipStream_t st) {
  bool empty = false;
  int rc = validate_proj_sizes(B, H, N, D, dtype, &empty);
  if (rc != FLAREPP_OK || empty) return rc;
  if (!Y || !Wo || !out) return FLAREPP_INVALID_ARGUMENT;
  const size_t es = dtype == FLAREPP_BF16 ? 2 : 4;
  for (const void* q : {Y, Wo, (const void*)out})
    if (!aligned(q, 16)) return FLAREPP_MISALIGNED;
  if (bo && !aligned(bo, es)) return FLAREPP_MISALIGNED;
  const size_t C = (size_t)H * D, big = (size_t)B * N * C * es;
  const Span outs[] = {{out, big}};
  const Span ins[] = {{Y, big}, {Wo, C * C * es}, {bo, C * es}};
  if (any_overlap(outs, 1, ins, 3)) return FLAREPP_INVALID_ARGUMENT;
  rc = check_device();
  if (rc != FLAREPP_OK) return rc;
  const void* W[3] = {Wo, nullptr, nullptr};
  const void* bias[3] = {bo, nullptr, nullptr};
  void* o[3] = {out, nullptr, nullptr};
  return enqueue_project(Y, W, bias, nullptr, o, B, H, N, D, dtype, false, st);
}

// Workspace of the block: the mixer's own, then K, V, S, Y [B][H][N][D], the normalized seeds
// [H][M][D] and the gates [H].
struct BlockPlan {
  Plan mix;
  size_t off_k = 0, off_v = 0, off_s = 0, off_y = 0, off_qs = 0, off_g = 0, total = 0;
};

BlockPlan make_block_plan(int B, int H, int64_t N, int M, int D, int dtype) {
  BlockPlan bp;
  bp.mix = make_plan(B, H, N, M, D, dtype);
  const size_t es = dtype == FLAREPP_BF16 ? 2 : 4;
  const size_t big = (size_t)B * H * N * D * es;
  size_t off = align256(bp.mix.total);
  bp.off_k = off; off = align256(off + big);
  bp.off_v = off; off = align256(off + big);
  bp.off_s = off; off = align256(off + big);
  bp.off_y = off; off = align256(off + big);
  bp.off_qs = off; off = align256(off + (size_t)H * M * D * es);
  bp.off_g = off; off = align256(off + (size_t)H * sizeof(float));
  bp.total = off;
  return bp;
}

int validate_block_sizes(int B, int H, int64_t N, int M, int D, int dtype, bool* empty) {
  int rc = validate_sizes(B, H, N, M, D, dtype, empty);
  if (rc != FLAREPP_OK) return rc;
  bool e2 = false;
  return validate_proj_sizes(B, H, N, D, dtype, &e2);
}

int block_common(const void* X, const void* Wk, const void* Wv, const void* Ws, const void* Wo, const void* bk,
                 const void* bv, const void* bs, const void* bo, const void* Qseed, const void* Qf,
                 const float* gamma, const void* nq, const void* nk, int B, int H, int64_t N, int M, int D,
                 int dtype, void* out, void* ws, size_t ws_bytes, bool own_ws, hipStream_t st) {
  bool empty = false;
  int rc = validate_block_sizes(B, H, N, M, D, dtype, &empty);
  if (rc != FLAREPP_OK || empty) return rc;
  if (!X || !Wk || !Wv || !Ws || !Wo || !Qseed || !Qf || !gamma || !out) return FLAREPP_INVALID_ARGUMENT;
  const size_t es = dtype == FLAREPP_BF16 ? 2 : 4;
  for (const void* q : {X, Wk, Wv, Ws, Wo, Qseed, Qf, (const void*)gamma, (const void*)out})
    if (!aligned(q, 16)) return FLAREPP_MISALIGNED;
  for (const void* q : {bk, bv, bs, bo, nq, nk})
    if (q && !aligned(q, es)) return FLAREPP_MISALIGNED;
  const size_t C = (size_t)H * D, big = (size_t)B * N * C * es, ww = C * C * es, nqs = (size_t)H * M * D * es;
  const Span outs[] = {{out, big}};
  const Span ins[] = {{X, big},    {Wk, ww},     {Wv, ww},     {Ws, ww},        {Wo, ww},
                      {bk, C * es}, {bv, C * es}, {bs, C * es}, {bo, C * es},    {Qseed, nqs},
                      {Qf, nqs},   {gamma, H * sizeof(float)}, {nq, D * es}, {nk, D * es}};
  if (any_overlap(outs, 1, ins, 14)) return FLAREPP_INVALID_ARGUMENT;
  const BlockPlan bp = make_block_plan(B, H, N, M, D, dtype);
  if (!own_ws) {
    if (!ws || ws_bytes < bp.total) return FLAREPP_INVALID_ARGUMENT;
    if (!aligned(ws, 256)) return FLAREPP_MISALIGNED;
  }
  rc = check_device();
  if (rc != FLAREPP_OK) return rc;
  if (own_ws) {
    if (hipMallocAsync(&ws, bp.total, st) != hipSuccess) {
      (void)hipGetLastError();
      return FLAREPP_OUT_OF_MEMORY;
    }
  }
  char* w = static_cast<char*>(ws);
  void *K = w + bp.off_k, *V = w + bp.off_v, *S = w + bp.off_s, *Y = w + bp.off_y, *Qs = w + bp.off_qs;
  float* g = reinterpret_cast<float*>(w + bp.off_g);
  flarepp::BlockParamArgs pa{Qseed, nq, gamma, Qs, g, H, M};
  const void* W[3] = {Wk, Wv, Ws};
  const void* bias[3] = {bk, bv, bs};
  void* kvs[3] = {K, V, S};
  const void* Wout[3] = {Wo, nullptr, nullptr};
  const void* bout[3] = {bo, nullptr, nullptr};
  void* o[3] = {out, nullptr, nullptr};
  rc = FLAREPP_OK;
  if (run_kernel(18, st, [&] { return flarepp::launch_block_params(pa, dtype, D, st); }) != hipSuccess)
    rc = FLAREPP_LAUNCH_FAILED;
  if (rc == FLAREPP_OK) rc = enqueue_project(X, W, bias, nk, kvs, B, H, N, D, dtype, true, st);
  if (rc == FLAREPP_OK)
    rc = enqueue(K, V, S, Qs, Qf, g, B, H, N, M, D, dtype, Y, nullptr, nullptr, nullptr, ws, bp.mix, st);
  if (rc == FLAREPP_OK) rc = enqueue_project(Y, Wout, bout, nullptr, o, B, H, N, D, dtype, false, st);
  if (own_ws) (void)hipFreeAsync(ws, st);
  return rc;
}

}  // namespace

extern "C" {

int flarepp_flare(const void* K, const void* V, const void* Q, int B, int H, int64_t N, int M, int D, int dtype,
                  void* out, hipStream_t stream) {
  return flare_common(K, V, Q, B, H, N, M, D, dtype, out, nullptr, 0, true, stream);
}

int flarepp_flare_ws(const void* K, const void* V, const void* Q, int B, int H, int64_t N, int M, int D,
                     int dtype, void* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return flare_common(K, V, Q, B, H, N, M, D, dtype, out, workspace, workspace_bytes, false, stream);
}

int flarepp_mix(const void* K, const void* V, const void* S, const void* Qseed, const void* Qf, const float* g,
                int B, int H, int64_t N, int M, int D, int dtype, void* out, hipStream_t stream) {
  return mix_common(K, V, S, Qseed, Qf, g, B, H, N, M, D, dtype, out, nullptr, nullptr, nullptr, nullptr, 0,
                    true, stream);
}

int flarepp_mix_noalloc(const void* K, const void* V, const void* S, const void* Qseed, const void* Qf,
                        const float* g, int B, int H, int64_t N, int M, int D, int dtype, void* out,
                        hipStream_t stream) {
  return mix_noalloc_common(K, V, S, Qseed, Qf, g, B, H, N, M, D, dtype, out, stream);
}

size_t flarepp_workspace_bytes(int B, int H, int64_t N, int M, int D, int dtype) {
  bool empty = false;
  if (validate_sizes(B, H, N, M, D, dtype, &empty) != FLAREPP_OK || empty) return 0;
  return make_plan(B, H, N, M, D, dtype).total;
}

int flarepp_mix_ws(const void* K, const void* V, const void* S, const void* Qseed, const void* Qf, const float* g,
                   int B, int H, int64_t N, int M, int D, int dtype, void* out, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  return mix_common(K, V, S, Qseed, Qf, g, B, H, N, M, D, dtype, out, nullptr, nullptr, nullptr, workspace,
                    workspace_bytes, false, stream);
}

int flarepp_mix_debug(const void* K, const void* V, const void* S, const void* Qseed, const void* Qf,
                      const float* g, int B, int H, int64_t N, int M, int D, int dtype, void* out, float* Qd,
                      float* Q, float* Z, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const void* dbg[] = {Qd, Q, Z};
  for (const void* p : dbg)
    if ((uintptr_t)p & 15) return FLAREPP_MISALIGNED;
  return mix_common(K, V, S, Qseed, Qf, g, B, H, N, M, D, dtype, out, Qd, Q, Z, workspace, workspace_bytes,
                    false, stream);
}

int flarepp_mix_simplified(const void* K, const void* V, const void* Sk, const void* Sv, const void* Qseed, int B,
                           int H, int64_t N, int M, int D, int dtype, void* out, hipStream_t stream) {
  return simplified_common(K, V, Sk, Sv, Qseed, B, H, N, M, D, dtype, out, nullptr, 0, true, stream);
}

int flarepp_mix_simplified_ws(const void* K, const void* V, const void* Sk, const void* Sv, const void* Qseed,
                              int B, int H, int64_t N, int M, int D, int dtype, void* out, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  return simplified_common(K, V, Sk, Sv, Qseed, B, H, N, M, D, dtype, out, workspace, workspace_bytes, false,
                           stream);
}

size_t flarepp_backward_workspace_bytes(int B, int H, int64_t N, int M, int D, int dtype) {
  bool empty = false;
  if (validate_bwd_sizes(B, H, N, M, D, dtype, &empty) != FLAREPP_OK || empty) return 0;
  return make_bwd_plan(B, H, N, M, D, dtype).total;
}

int flarepp_mix_backward(const void* K, const void* V, const void* S, const void* Qseed, const void* Qf,
                         const float* g, const void* dY, int B, int H, int64_t N, int M, int D, int dtype, void* dK,
                         void* dV, void* dS, void* dQseed, void* dQf, float* dg, hipStream_t stream) {
  return backward_common(K, V, S, Qseed, Qf, g, dY, B, H, N, M, D, dtype, dK, dV, dS, dQseed, dQf, dg, nullptr, 0,
                         true, stream);
}

int flarepp_mix_backward_ws(const void* K, const void* V, const void* S, const void* Qseed, const void* Qf,
                            const float* g, const void* dY, int B, int H, int64_t N, int M, int D, int dtype,
                            void* dK, void* dV, void* dS, void* dQseed, void* dQf, float* dg, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  return backward_common(K, V, S, Qseed, Qf, g, dY, B, H, N, M, D, dtype, dK, dV, dS, dQseed, dQf, dg, workspace,
                         workspace_bytes, false, stream);
}

int flarepp_mix_forward_saved(const void* K, const void* V, const void* S, const void* Qseed, const void* Qf,
                              const float* g, int B, int H, int64_t N, int M, int D, int dtype, void* out,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return forward_saved_common(K, V, S, Qseed, Qf, g, B, H, N, M, D, dtype, out, workspace, workspace_bytes, stream);
}

int flarepp_mix_backward_saved(const void* K, const void* V, const void* S, const void* Qseed, const void* Qf,
                               const float* g, const void* dY, int B, int H, int64_t N, int M, int D, int dtype,
                               void* dK, void* dV, void* dS, void* dQseed, void* dQf, float* dg, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  return backward_common(K, V, S, Qseed, Qf, g, dY, B, H, N, M, D, dtype, dK, dV, dS, dQseed, dQf, dg, workspace,
                         workspace_bytes, false, stream, true);
}

int flarepp_project(const void* X, const void* Wk, const void* Wv, const void* Ws, const void* bk, const void* bv,
                    const void* bs, const void* nk, int B, int H, int64_t N, int D, int dtype, void* K, void* V,
                    void* S, hipStream_t stream) {
  return project_common(X, Wk, Wv, Ws, bk, bv, bs, nk, B, H, N, D, dtype, K, V, S, stream);
}

int flarepp_out_project(const void* Y, const void* Wo, const void* bo, int B, int H, int64_t N, int D, int dtype,
                        void* out, hipStream_t stream) {
  return out_project_common(Y, Wo, bo, B, H, N, D, dtype, out, stream);
}

size_t flarepp_block_workspace_bytes(int B, int H, int64_t N, int M, int D, int dtype) {
  bool empty = false;
  if (validate_block_sizes(B, H, N, M, D, dtype, &empty) != FLAREPP_OK || empty) return 0;
  return make_block_plan(B, H, N, M, D, dtype).total;
}

int flarepp_block(const void* X, const void* Wk, const void* Wv, const void* Ws, const void* Wo, const void* bk,
                  const void* bv, const void* bs, const void* bo, const void* Qseed, const void* Qf,
                  const float* gamma, const void* nq, const void* nk, int B, int H, int64_t N, int M, int D,
                  int dtype, void* out, hipStream_t stream) {
  return block_common(X, Wk, Wv, Ws, Wo, bk, bv, bs, bo, Qseed, Qf, gamma, nq, nk, B, H, N, M, D, dtype, out,
                      nullptr, 0, true, stream);
}

int flarepp_block_ws(const void* X, const void* Wk, const void* Wv, const void* Ws, const void* Wo, const void* bk,
                     const void* bv, const void* bs, const void* bo, const void* Qseed, const void* Qf,
                     const float* gamma, const void* nq, const void* nk, int B, int H, int64_t N, int M, int D,
                     int dtype, void* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return block_common(X, Wk, Wv, Ws, Wo, bk, bv, bs, bo, Qseed, Qf, gamma, nq, nk, B, H, N, M, D, dtype, out,
                      workspace, workspace_bytes, false, stream);
}

int flarepp_debug_force_exact(int enable) { return g_force_exact.exchange(enable != 0); }

int flarepp_timing_enable(int enable) {
  Timing& t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  t.enabled = enable != 0;
  return FLAREPP_OK;
}

int flarepp_timing_read(double* ms, long long* counts, int n) {
  Timing& t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  int rc = FLAREPP_OK;
  for (auto& r : t.pending) {
    float e = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&e, r.a, r.b) != hipSuccess) {
      rc = FLAREPP_DEVICE_ERROR;
    } else if (r.kind < n) {
      if (ms) ms[r.kind] += e;
      if (counts) counts[r.kind] += 1;
    }
    t.pool.push_back(r.a);
    t.pool.push_back(r.b);
  }
  t.pending.clear();
  return rc == FLAREPP_OK ? kNumKinds : -rc;
}

const char* flarepp_kernel_name(int i) { return (i >= 0 && i < kNumKinds) ? kKindNames[i] : nullptr; }

const char* flarepp_strerror(int status) {
  switch (status) {
    case FLAREPP_OK: return "ok";
    case FLAREPP_INVALID_ARGUMENT: return "invalid argument";
    case FLAREPP_UNSUPPORTED: return "unsupported shape, dtype or device";
    case FLAREPP_MISALIGNED: return "tensor pointer not 16-byte aligned (workspace: 256-byte)";
    case FLAREPP_OUT_OF_MEMORY: return "workspace allocation failed";
    case FLAREPP_LAUNCH_FAILED: return "kernel launch failed";
    case FLAREPP_DEVICE_ERROR: return "HIP runtime error while querying the device";
    case FLAREPP_SCRATCH_TOO_SMALL:
      return "the problem's workspace exceeds the static scratch of flarepp_mix_noalloc "
             "(FLAREPP_NOALLOC_SCRATCH_BYTES); use flarepp_mix_ws";
    default: return "unknown status";
  }
}

int flarepp_version(void) { return kVersion; }

}  // extern "C"
