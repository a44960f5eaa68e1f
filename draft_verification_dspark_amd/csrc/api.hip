// C ABI entry points: synchronous argument checks, workspace carving and
// kernel launches on the caller's stream.  No allocation, no synchronisation.
#include <hip/hip_runtime.h>

#include <mutex>

#include "args.hpp"
#include "schedule_args.hpp"
#include "calib_args.hpp"
#include "markov_args.hpp"

namespace dspark {

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxB = 1 << 24;
constexpr int kMaxK = 64;

size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct VerifyLayout {
  size_t sync, part1, part2, total;
};

// The sync block (two 128-byte lines per request) first, then the chunk
// summaries and the residual quarter sums.
VerifyLayout verify_layout(int B, int K, int V) {
  VerifyLayout L;
  if (B > kLaunchBatch) B = kLaunchBatch;  // sub-batches reuse the workspace
  const size_t G = (size_t)chunks_per_row_max(V);
  size_t off = 0;
  L.sync = off;  off += up(sync_bytes(B));
  L.part1 = off; off += up(sizeof(Partial) * (size_t)B * (K + 1) * 2 * G);
  L.part2 = off; off += up(sizeof(ResidualChunk) * (size_t)B * 4 * G);
  L.total = off;
  return L;
}

struct ScheduleLayout {
  size_t surv, lthr, total;
};

ScheduleLayout schedule_layout(int B, int K) {
  ScheduleLayout L;
  size_t off = 0;
  L.surv = off; off += up(sizeof(float) * (size_t)B * K);
  L.lthr = off; off += up(sizeof(int32_t) * (size_t)B);
  L.total = off;
  return L;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int kPhaseAll = kPhaseStream | kPhaseFinish;

}  // namespace

// Compute units of the current device (cached per device; 256 if the query
// fails).
int compute_units() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    return 256;
  if (dev < 64) cache[dev] = cus;
  return cus;
}

}  // namespace dspark

using namespace dspark;

extern "C" {

size_t dspark_workspace_bytes(int op, int B, int K, int V) {
  if (B < 1 || K < 1 || B > kMaxB) return 0;
  if (op == DSPARK_OP_SCHEDULE) return schedule_layout(B, K).total;
  if (op == DSPARK_OP_MARKOV_DRAFT) {
    if (V < 1) return 0;
    const size_t tiles = ((size_t)V + kMarkovRows - 1) / kMarkovRows;
    return up(sizeof(Partial) * (size_t)B * tiles);
  }
  if (op == DSPARK_OP_VERIFY || op == DSPARK_OP_VERIFY_GREEDY) {
    if (V < 1 || K > kMaxK) return 0;
    return verify_layout(B, K, V).total;
  }
  if (op == DSPARK_OP_SCHEDULE_VERIFY) {
    if (V < 1 || K > kMaxK) return 0;
    return up(verify_layout(B, K, V).total) + schedule_layout(B, K).total;
  }
  return 0;
}

const char* dspark_status_string(int status) {
  switch (status) {
    case DSPARK_OK: return "ok";
    case DSPARK_ERR_NULL: return "a required pointer is NULL";
    case DSPARK_ERR_SHAPE: return "B, K or V out of range";
    case DSPARK_ERR_DTYPE: return "unknown logits dtype";
    case DSPARK_ERR_BUDGET: return "budget below B*min_len or min_len outside [0,K]";
    case DSPARK_ERR_WORKSPACE: return "workspace too small or misaligned";
    case DSPARK_ERR_LAUNCH: return "kernel launch failed";
    case DSPARK_ERR_PARAM: return "parameter out of range or misaligned";
    case DSPARK_ERR_SCRATCH:
      return "the sizes need more workspace than the library's built-in scratch "
             "(DSPARK_SCRATCH_BYTES); use the call with a caller workspace";
    default: return "unknown status";
  }
}

static int schedule_common(ScheduleArgs& a, const float* conf, int B, int K, float threshold,
                           int budget, int min_len, int32_t* lengths, uint8_t* mask,
                           float* survival, int32_t* dev_status, void* workspace,
                           size_t ws_bytes) {
  if (!conf || !lengths || !dev_status || !workspace) return DSPARK_ERR_NULL;
  if (B < 1 || K < 1 || B > kMaxB || (long long)B * K > (1LL << 30)) return DSPARK_ERR_SHAPE;
  if (min_len < 0 || min_len > K) return DSPARK_ERR_BUDGET;
  if (budget >= 0 && (long long)budget < (long long)B * min_len) return DSPARK_ERR_BUDGET;
  const ScheduleLayout L = schedule_layout(B, K);
  if (ws_bytes < L.total || !aligned(workspace, kAlign)) return DSPARK_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  a = ScheduleArgs{};
  a.conf = conf;
  a.B = B;
  a.K = K;
  a.tau = threshold;
  a.budget = budget;
  a.min_len = min_len;
  a.lengths = lengths;
  a.mask = mask;
  a.surv = survival ? survival : reinterpret_cast<float*>(ws + L.surv);
  a.lthr = reinterpret_cast<int32_t*>(ws + L.lthr);
  a.dev_status = dev_status;
  a.vec4 = (K % 4 == 0) && aligned(conf, 16) && aligned(a.surv, 16);
  return DSPARK_OK;
}

int dspark_schedule(const float* conf, int B, int K, float threshold, int budget, int min_len,
                    int32_t* lengths, uint8_t* mask, float* survival, int32_t* dev_status,
                    void* workspace, size_t ws_bytes, void* stream) {
  ScheduleArgs a;
  const int st = schedule_common(a, conf, B, K, threshold, budget, min_len, lengths, mask,
                                 survival, dev_status, workspace, ws_bytes);
  if (st != DSPARK_OK) return st;
  return launch_schedule(a, static_cast<hipStream_t>(stream));
}

static bool finite_f(float x) { return x == x && x - x == 0.f; }

int dspark_schedule_load_aware(const float* conf, int B, int K, const float* load, float q_max,
                               float m_max, float tau_min, float tau_max, const float* curve,
                               int n_curve, float slot_cost, int min_len, int32_t* lengths,
                               uint8_t* mask, float* survival, float* tau_out,
                               int32_t* budget_out, int32_t* dev_status, void* workspace,
                               size_t ws_bytes, void* stream) {
  ScheduleArgs a;
  const int st = schedule_common(a, conf, B, K, 0.f, -1, min_len, lengths, mask, survival,
                                 dev_status, workspace, ws_bytes);
  if (st != DSPARK_OK) return st;
  if (!load) return DSPARK_ERR_NULL;
  if (!(finite_f(q_max) && q_max > 0.f && finite_f(m_max) && m_max > 0.f)) return DSPARK_ERR_PARAM;
  if (!(finite_f(tau_min) && finite_f(tau_max) && tau_min >= 0.f && tau_min <= tau_max))
    return DSPARK_ERR_PARAM;
  if (n_curve < 0 || n_curve > 64 || (n_curve > 0 && !curve) || !finite_f(slot_cost))
    return DSPARK_ERR_PARAM;
  a.load = load;
  a.q_max = q_max;
  a.m_max = m_max;
  a.tau_min = tau_min;
  a.tau_max = tau_max;
  a.curve = curve;
  a.n_curve = n_curve;
  a.slot_cost = slot_cost;
  a.tau_out = tau_out;
  a.budget_out = budget_out;
  return launch_schedule(a, static_cast<hipStream_t>(stream));
}

static int verify_common(const void* target, const void* draft, int dtype, int B, int K, int V,
                         const int32_t* drafted, const int32_t* lengths, const float* temperature,
                         const float* uniforms, int32_t* accepted, int32_t* tokens, float* p_tok,
                         float* q_tok, int32_t* dev_status, void* workspace, size_t ws_bytes,
                         void* stream, int greedy_only, int phases, bool dry = false,
                         const ScheduleArgs* fused = nullptr) {
  if (!target || !drafted || !accepted || !tokens || !dev_status || !workspace)
    return DSPARK_ERR_NULL;
  if (!greedy_only && (!draft || !temperature || !uniforms)) return DSPARK_ERR_NULL;
  if (B < 1 || K < 1 || V < 1 || K > kMaxK || B > kMaxB || V > (1 << 30)) return DSPARK_ERR_SHAPE;
  if (dtype != DSPARK_F32 && dtype != DSPARK_BF16) return DSPARK_ERR_DTYPE;
  // a call split into its phases keeps one launch batch's state in the workspace
  if (phases != kPhaseAll && (phases < 1 || phases > kPhaseAll)) return DSPARK_ERR_PARAM;
  if (phases != kPhaseAll && B > kLaunchBatch) return DSPARK_ERR_SHAPE;
  const VerifyLayout L = verify_layout(B, K, V);
  if (ws_bytes < L.total || !aligned(workspace, kAlign)) return DSPARK_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  VerifyArgs a;
  a.target = target;
  a.draft = greedy_only ? nullptr : draft;
  a.drafted = drafted;
  a.lengths = lengths;
  a.temperature = temperature;
  a.uniforms = uniforms;
  a.accepted = accepted;
  a.tokens = tokens;
  a.p_tok = greedy_only ? nullptr : p_tok;
  a.q_tok = greedy_only ? nullptr : q_tok;
  a.dev_status = dev_status;
  a.sync = ws + L.sync;
  a.part1 = reinterpret_cast<Partial*>(ws + L.part1);
  a.part2 = reinterpret_cast<ResidualChunk*>(ws + L.part2);
  a.K = K;
  a.V = V;
  const int per_vec = dtype == DSPARK_BF16 ? 8 : 4;
  a.G = dtype == DSPARK_BF16 ? chunks_per_row<DSPARK_BF16>(V) : chunks_per_row<DSPARK_F32>(V);
  // one quarter task per quarter chunk that holds part of the row: the last
  // chunk's quarters past the row's end would be empty tasks
  const int quarter =
      (dtype == DSPARK_BF16 ? item_elems<DSPARK_BF16>() : item_elems<DSPARK_F32>()) / 4;
  a.QT = (V + quarter - 1) / quarter;
  a.greedy_only = greedy_only;
  a.vec_ok = (V % per_vec == 0) && aligned(target, 16) && (greedy_only || aligned(draft, 16));
  if (dry) return DSPARK_OK;  // arguments checked, nothing launched
  // consecutive sub-batches of at most kLaunchBatch requests on one stream
  const size_t s = dtype == DSPARK_BF16 ? 2 : 4;
  for (int b0 = 0; b0 < B; b0 += kLaunchBatch) {
    VerifyArgs sub = a;
    const int nb = B - b0 < kLaunchBatch ? B - b0 : kLaunchBatch;
    sub.B = nb;
    sub.target = static_cast<const char*>(target) + (size_t)b0 * (K + 1) * V * s;
    sub.draft = greedy_only ? nullptr : static_cast<const char*>(draft) + (size_t)b0 * K * V * s;
    sub.drafted = drafted + (size_t)b0 * K;
    sub.lengths = lengths ? lengths + b0 : nullptr;
    sub.temperature = greedy_only ? nullptr : temperature + b0;
    sub.uniforms = greedy_only ? nullptr : uniforms + (size_t)b0 * (K + 1);
    sub.accepted = accepted + b0;
    sub.tokens = tokens + (size_t)b0 * (K + 1);
    sub.p_tok = a.p_tok ? a.p_tok + (size_t)b0 * K : nullptr;
    sub.q_tok = a.q_tok ? a.q_tok + (size_t)b0 * K : nullptr;
    const int st = launch_verify(sub, dtype, static_cast<hipStream_t>(stream), phases,
                                 b0 == 0 ? fused : nullptr);
    if (st != DSPARK_OK) return st;
  }
  return DSPARK_OK;
}

int dspark_verify_phase(int phases, const void* target_logits, const void* draft_logits,
                        int dtype, int B, int K, int V, const int32_t* drafted,
                        const int32_t* lengths, const float* temperature, const float* uniforms,
                        int32_t* accepted, int32_t* tokens, float* p_tok, float* q_tok,
                        int32_t* dev_status, void* workspace, size_t ws_bytes, void* stream) {
  return verify_common(target_logits, draft_logits, dtype, B, K, V, drafted, lengths, temperature,
                       uniforms, accepted, tokens, p_tok, q_tok, dev_status, workspace, ws_bytes,
                       stream, 0, phases);
}

int dspark_verify(const void* target_logits, const void* draft_logits, int dtype, int B, int K,
                  int V, const int32_t* drafted, const int32_t* lengths,
                  const float* temperature, const float* uniforms, int32_t* accepted,
                  int32_t* tokens, float* p_tok, float* q_tok, int32_t* dev_status,
                  void* workspace, size_t ws_bytes, void* stream) {
  return dspark_verify_phase(kPhaseAll, target_logits, draft_logits, dtype, B, K, V, drafted,
                             lengths, temperature, uniforms, accepted, tokens, p_tok, q_tok,
                             dev_status, workspace, ws_bytes, stream);
}

int dspark_verify_greedy_phase(int phases, const void* target_logits, int dtype, int B, int K,
                               int V, const int32_t* drafted, const int32_t* lengths,
                               int32_t* accepted, int32_t* tokens, int32_t* dev_status,
                               void* workspace, size_t ws_bytes, void* stream) {
  return verify_common(target_logits, nullptr, dtype, B, K, V, drafted, lengths, nullptr, nullptr,
                       accepted, tokens, nullptr, nullptr, dev_status, workspace, ws_bytes, stream,
                       1, phases);
}

int dspark_verify_greedy(const void* target_logits, int dtype, int B, int K, int V,
                         const int32_t* drafted, const int32_t* lengths, int32_t* accepted,
                         int32_t* tokens, int32_t* dev_status, void* workspace, size_t ws_bytes,
                         void* stream) {
  return dspark_verify_greedy_phase(kPhaseAll, target_logits, dtype, B, K, V, drafted, lengths,
                                    accepted, tokens, dev_status, workspace, ws_bytes, stream);
}

int dspark_calibrate(const float* raw, const float* theta, int B, int K, float* calibrated,
                     int32_t* dev_status, void* stream) {
  if (!raw || !theta || !calibrated || !dev_status) return DSPARK_ERR_NULL;
  if (B < 1 || K < 1 || K > kCalibMax || B > kMaxB) return DSPARK_ERR_SHAPE;
  CalibArgs a{};
  a.raw = raw;
  a.theta = const_cast<float*>(theta);
  a.B = B;
  a.K = K;
  a.calibrated_out = calibrated;
  a.dev_status = dev_status;
  return launch_calibrate(a, static_cast<hipStream_t>(stream));
}

size_t dspark_calib_state_bytes(int K, int n_bins) {
  if (K < 1 || K > kCalibMax || n_bins < 1 || n_bins > kCalibMax) return 0;
  return sizeof(long long) * (1 + 3 * (size_t)K + 3 * (size_t)n_bins);
}

int dspark_calib_observe(const float* calibrated, const int32_t* lengths, const int32_t* accepted,
                         int B, int K, float* theta, float lr, float theta_min, int window,
                         int n_bins, void* state, size_t state_bytes, float* ece_out,
                         int32_t* dev_status, void* stream) {
  if (!calibrated || !accepted || !theta || !state || !dev_status) return DSPARK_ERR_NULL;
  if (B < 1 || K < 1 || K > kCalibMax || B > kMaxB) return DSPARK_ERR_SHAPE;
  if (!(finite_f(lr) && finite_f(theta_min) && theta_min > 0.f) || window < 1 || n_bins < 1 ||
      n_bins > kCalibMax)
    return DSPARK_ERR_PARAM;
  if (state_bytes < dspark_calib_state_bytes(K, n_bins) || !aligned(state, 8))
    return DSPARK_ERR_WORKSPACE;
  CalibArgs a{};
  a.calibrated = calibrated;
  a.lengths = lengths;
  a.accepted = accepted;
  a.theta = theta;
  a.B = B;
  a.K = K;
  a.lr = lr;
  a.theta_min = theta_min;
  a.window = window;
  a.n_bins = n_bins;
  a.state = state;
  a.ece_out = ece_out;
  a.dev_status = dev_status;
  return launch_calib_observe(a, static_cast<hipStream_t>(stream));
}

int dspark_markov_draft(const void* base, int dtype, int B, int K, int V, const uint16_t* U,
                        const uint16_t* Vm, int r, float scale, const int32_t* y0,
                        const float* temperature, const float* uniforms, void* corrected,
                        int32_t* drafted, float* q_tok, int32_t* dev_status, void* workspace,
                        size_t ws_bytes, void* stream) {
  if (!base || !U || !Vm || !y0 || !temperature || !uniforms || !corrected || !drafted ||
      !dev_status || !workspace)
    return DSPARK_ERR_NULL;
  if (B < 1 || K < 1 || V < 1 || B > kMaxB || V > (1 << 30) ||
      (long long)B * ((V + kMarkovRows - 1) / kMarkovRows) > (1LL << 31))
    return DSPARK_ERR_SHAPE;
  if (r < 16 || r > kMarkovMaxRank || r % 16 != 0) return DSPARK_ERR_SHAPE;
  if (dtype != DSPARK_F32 && dtype != DSPARK_BF16) return DSPARK_ERR_DTYPE;
  if (!aligned(U, 16) || !aligned(Vm, 16)) return DSPARK_ERR_PARAM;
  if (ws_bytes < dspark_workspace_bytes(DSPARK_OP_MARKOV_DRAFT, B, K, V) ||
      !aligned(workspace, kAlign))
    return DSPARK_ERR_WORKSPACE;
  MarkovArgs a{};
  a.base = base;
  a.U = U;
  a.Vm = Vm;
  a.r = r;
  a.scale = scale;
  a.y0 = y0;
  a.temperature = temperature;
  a.uniforms = uniforms;
  a.corrected = corrected;
  a.drafted = drafted;
  a.q_tok = q_tok;
  a.dev_status = dev_status;
  a.part = static_cast<Partial*>(workspace);
  a.B = B;
  a.K = K;
  a.V = V;
  a.tiles = (V + kMarkovRows - 1) / kMarkovRows;
  return launch_markov(a, dtype, static_cast<hipStream_t>(stream));
}

int dspark_schedule_verify_phase(int phases, const float* conf, float threshold, int budget,
                                 int min_len, int32_t* lengths, uint8_t* mask, float* survival,
                                 const void* target_logits, const void* draft_logits, int dtype,
                                 int B, int K, int V, const int32_t* drafted,
                                 const float* temperature, const float* uniforms,
                                 int32_t* accepted, int32_t* tokens, float* p_tok, float* q_tok,
                                 int32_t* dev_status, void* workspace, size_t ws_bytes,
                                 void* stream) {
  if (!workspace) return DSPARK_ERR_NULL;
  if (B < 1 || K < 1 || V < 1 || K > kMaxK || B > kMaxB || V > (1 << 30)) return DSPARK_ERR_SHAPE;
  // workspace: the verify layout, then the schedule layout
  const size_t vbytes = up(verify_layout(B, K, V).total);
  if (ws_bytes < vbytes || !aligned(workspace, kAlign)) return DSPARK_ERR_WORKSPACE;
  ScheduleArgs sa;
  int st = schedule_common(sa, conf, B, K, threshold, budget, min_len, lengths, mask, survival,
                           dev_status, static_cast<char*>(workspace) + vbytes, ws_bytes - vbytes);
  if (st != DSPARK_OK) return st;
  st = verify_common(target_logits, draft_logits, dtype, B, K, V, drafted, lengths, temperature,
                     uniforms, accepted, tokens, p_tok, q_tok, dev_status, workspace, vbytes,
                     stream, 0, phases, true);
  if (st != DSPARK_OK) return st;
  const bool fuse = B <= kFusedMaxB && K <= kFusedMaxK && (long long)B * K <= kFusedMaxPositions;
  if (!fuse && (phases & kPhaseStream)) {
    st = launch_schedule(sa, static_cast<hipStream_t>(stream));
    if (st != DSPARK_OK) return st;
  }
  return verify_common(target_logits, draft_logits, dtype, B, K, V, drafted, lengths, temperature,
                       uniforms, accepted, tokens, p_tok, q_tok, dev_status, workspace, vbytes,
                       stream, 0, phases, false, fuse ? &sa : nullptr);
}

// The built-in scratch of dspark_schedule_verify_noalloc: one array per GPU,
// kept until the process ends.  Host code never uses the array's name as an
// address: the device address comes from hipGetSymbolAddress, once per
// device (with that device current), on the first call there.
static __device__ __align__(256) unsigned char scratch[DSPARK_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// device address of this device's scratch, or nullptr if it cannot be had
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}
}  // namespace

int dspark_schedule_verify_noalloc(const float* conf, float threshold, int budget, int min_len,
                                   int32_t* lengths, uint8_t* mask, float* survival,
                                   const void* target_logits, const void* draft_logits,
                                   int dtype, int B, int K, int V, const int32_t* drafted,
                                   const float* temperature, const float* uniforms,
                                   int32_t* accepted, int32_t* tokens, float* p_tok,
                                   float* q_tok, int32_t* dev_status, void* stream) {
  const size_t need = dspark_workspace_bytes(DSPARK_OP_SCHEDULE_VERIFY, B, K, V);
  if (need == 0) return DSPARK_ERR_SHAPE;
  if (need > (size_t)DSPARK_SCRATCH_BYTES) return DSPARK_ERR_SCRATCH;
  void* ws = scratch_ptr();
  if (!ws) return DSPARK_ERR_LAUNCH;
  return dspark_schedule_verify_phase(kPhaseAll, conf, threshold, budget, min_len, lengths, mask,
                                      survival, target_logits, draft_logits, dtype, B, K, V,
                                      drafted, temperature, uniforms, accepted, tokens, p_tok,
                                      q_tok, dev_status, ws, DSPARK_SCRATCH_BYTES, stream);
}

int dspark_schedule_verify(const float* conf, float threshold, int budget, int min_len,
                           int32_t* lengths, uint8_t* mask, float* survival,
                           const void* target_logits, const void* draft_logits, int dtype, int B,
                           int K, int V, const int32_t* drafted, const float* temperature,
                           const float* uniforms, int32_t* accepted, int32_t* tokens,
                           float* p_tok, float* q_tok, int32_t* dev_status, void* workspace,
                           size_t ws_bytes, void* stream) {
  return dspark_schedule_verify_phase(kPhaseAll, conf, threshold, budget, min_len, lengths, mask,
                                      survival, target_logits, draft_logits, dtype, B, K, V,
                                      drafted, temperature, uniforms, accepted, tokens, p_tok,
                                      q_tok, dev_status, workspace, ws_bytes, stream);
}

}  // extern "C"
