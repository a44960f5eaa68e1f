// Batched block verification on gfx950.
//
// What is computed (DSpark Deep Dive, "Speculative Decoding From First
// Principles" and "The Verification Phase"; DSpark Guide, "1. The Mathematics
// of Suffix Decay"): for each request, temperature softmaxes of the scheduled
// target and draft rows, the accept test u < min(1, p(y)/q(y)) at every
// scheduled position, the first rejection, and one more token drawn either
// from the normalised residual max(0, p - q) at the rejected position or,
// when everything was accepted, from the target row after the last draft.
// Requests with temperature 0 use the greedy rule (accept while the draft
// equals the target argmax).  Rows past the scheduled length are never read
// (DSpark Deep Dive, "GPU-Resident Scheduling": maximum-length buffers,
// variable lengths by masking).
//
// Kernels, all enqueued on the caller's stream with launch shapes fixed by
// (B, K, V):
//   k_plan      one workgroup: clamps lengths, picks each request's rule and
//               lists the rows to stream, in request order.
//   k_pass1     persistent grid: one wave per (row, 4096-token chunk) item,
//               16-byte loads, chunk max, then sum of 2^(x*c - k) with an
//               integer shift k (softmax rows) or (max, lowest index)
//               (greedy rows).
//   k_finalize  one wave per request: merges chunk summaries per row, forms
//               p(y), q(y), alpha, the accept ballot, the first rejection,
//               the emitted prefix, and the greedy token.
//   k_pass2     persistent grid over (rejected request, chunk): residual mass
//               per chunk; lanes holding normalised mass >= 2^-12 are redone
//               in fp64.
//   k_sample    one wave per request: locates the chunk of the draw from the
//               chunk masses, re-reads that chunk and scans it in token order.
#include <hip/hip_runtime.h>

#include "args.hpp"

namespace dspark {

__device__ __forceinline__ const char* target_row(const VerifyArgs& a, int b, int j, int s) {
  return static_cast<const char*>(a.target) + ((size_t)b * (a.K + 1) + j) * (size_t)a.V * s;
}
__device__ __forceinline__ const char* draft_row(const VerifyArgs& a, int b, int j, int s) {
  return static_cast<const char*>(a.draft) + ((size_t)b * a.K + j) * (size_t)a.V * s;
}

// ------------------------------------------------------------------ plan

__global__ void __launch_bounds__(1024) k_plan(VerifyArgs a) {
  __shared__ int scan[1024];
  __shared__ int carry;
  const int tid = threadIdx.x;
  const int R = 2 * a.K + 1;
  if (tid == 0) carry = 0;
  __syncthreads();
  int bad = 0;
  for (int base = 0; base < a.B; base += 1024) {
    const int b = base + tid;
    int cnt = 0, L = 0, kind = kKindSkip;
    float c = 0.f;
    if (b < a.B) {
      L = a.lengths ? a.lengths[b] : a.K;
      if (L < 0 || L > a.K) {
        bad |= DSPARK_DEV_BAD_LENGTH;
        L = L < 0 ? 0 : a.K;
      }
      if (a.greedy_only) {
        kind = kKindGreedy;
      } else {
        const float T = a.temperature[b];
        if (!(T >= 0.f)) {
          bad |= DSPARK_DEV_BAD_TEMP;
          kind = kKindSkip;
        } else if (T == 0.f) {
          kind = kKindGreedy;
        } else {
          kind = kKindSoftmax;
          c = (float)(1.4426950408889634 / (double)T);
        }
      }
      cnt = kind == kKindSoftmax ? 2 * L + 1 : (kind == kKindGreedy ? L + 1 : 0);
      ReqState& r = a.req[b];
      r.L = L;
      r.kind = kind;
      r.c = c;
      r.a = 0;
      r.mode = kModeNone;
    }
    // exclusive scan of cnt over the tile
    scan[tid] = cnt;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      int t = tid >= o ? scan[tid - o] : 0;
      __syncthreads();
      scan[tid] += t;
      __syncthreads();
    }
    const int off = carry + scan[tid] - cnt;
    if (b < a.B && cnt) {
      int* out = a.rows + off;
      // target rows 0..L, then (softmax) draft rows 0..L-1
      for (int j = 0; j <= L; ++j) out[j] = b * R + j;
      if (kind == kKindSoftmax)
        for (int j = 0; j < L; ++j) out[L + 1 + j] = b * R + a.K + 1 + j;
    }
    __syncthreads();
    if (tid == 1023) carry += scan[1023];
    __syncthreads();
  }
  if (tid == 0) *a.n_rows = carry;
  if (bad) flag(a.dev_status, bad);
}

// ------------------------------------------------------------------ pass 1

template <int DT>
__device__ void softmax_item(const VerifyArgs& a, const char* chunk, int n, float c, Partial* out) {
  Tile<DT> t;
  t.load(chunk, n, a.vec_ok);
  constexpr int P = Elem<DT>::kPerVec;
  float mx = -INFINITY;
#pragma unroll
  for (int v = 0; v < kUnroll; ++v)
#pragma unroll
    for (int e = 0; e < P; ++e) mx = fmaxf(mx, t.at(v, e));
  const float m = wave_max(mx);
  double s = 0.0;
  float k = -INFINITY;
  int bad = 0;
  if (m == -INFINITY) {
    // every element is -inf (or NaN): no mass; NaN is still reported
    int nan = 0;
#pragma unroll
    for (int v = 0; v < kUnroll; ++v)
#pragma unroll
      for (int e = 0; e < P; ++e) nan |= (t.at(v, e) != t.at(v, e));
    if (wave_or(nan)) bad = DSPARK_DEV_NONFINITE;
  } else {
    // integer shift: the chunk maximum maps into (-1, 0], so no element can
    // overflow, and chunks merge by exact powers of two
    k = ceilf(m * c);
    const float nk = -k;
    double acc = 0.0;
#pragma unroll
    for (int v = 0; v < kUnroll; ++v) {
      float p[P];
#pragma unroll
      for (int e = 0; e < P; ++e) p[e] = fast_exp2(fmaf(t.at(v, e), c, nk));
      float s4 = (p[0] + p[1]) + (p[2] + p[3]);
      if constexpr (P == 8) s4 += (p[4] + p[5]) + (p[6] + p[7]);
      acc += (double)s4;
    }
    s = wave_sum(acc);
    if (!(s < INFINITY) || m == INFINITY) bad = DSPARK_DEV_NONFINITE;  // NaN or +inf
  }
  if (lane_id() == 0) {
    out->k = k;
    out->idx = 0;
    out->s = s;
    if (bad) flag(a.dev_status, bad);
  }
}

template <int DT>
__device__ void argmax_item(const VerifyArgs& a, const char* chunk, int n, int first, Partial* out) {
  Tile<DT> t;
  t.load(chunk, n, a.vec_ok);
  constexpr int P = Elem<DT>::kPerVec;
  const int l = lane_id();
  float best = -INFINITY;
  int bi = 0x7fffffff;
  int nan = 0;
#pragma unroll
  for (int v = 0; v < kUnroll; ++v)
#pragma unroll
    for (int e = 0; e < P; ++e) {
      const float x = t.at(v, e);
      nan |= (x != x);
      if (x > best) {
        best = x;
        bi = first + (v * kWave + l) * P + e;
      }
    }
  wave_argmax(best, bi);
  nan = wave_or(nan);
  if (l == 0) {
    out->k = best;
    out->idx = bi;
    out->s = 0.0;
    if (nan || best == INFINITY) flag(a.dev_status, DSPARK_DEV_NONFINITE);
  }
}

template <int DT>
__global__ void __launch_bounds__(kBlock) k_pass1(VerifyArgs a) {
  constexpr int S = Elem<DT>::kBytes;
  constexpr int E = item_elems<DT>();
  const int R = 2 * a.K + 1;
  const int G = a.G;
  const long n_items = (long)(*a.n_rows) * G;
  const long wave0 = (long)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  const long stride = (long)gridDim.x * kWavesPerBlock;
  for (long it = wave0; it < n_items; it += stride) {
    const int rid = a.rows[it / G];
    const int c = (int)(it % G);
    const int b = rid / R;
    const int slot = rid % R;
    const char* row = slot <= a.K ? target_row(a, b, slot, S) : draft_row(a, b, slot - a.K - 1, S);
    const int e0 = c * E;
    const int n = min(E, a.V - e0);
    Partial* out = a.part1 + (size_t)rid * G + c;
    const ReqState& r = a.req[b];
    if (r.kind == kKindSoftmax)
      softmax_item<DT>(a, row + (size_t)e0 * S, n, r.c, out);
    else
      argmax_item<DT>(a, row + (size_t)e0 * S, n, e0, out);
  }
}

// ------------------------------------------------------------------ finalize

// merge the chunk summaries of one softmax row: shift K* = max k_c and
// S = sum_c s_c * 2^(k_c - K*) (exact scaling)
__device__ __forceinline__ void merge_softmax_row(const Partial* p, int G, float& kmax, double& S) {
  float km = -INFINITY;
  for (int c = 0; c < G; ++c)
    if (p[c].s > 0.0) km = fmaxf(km, p[c].k);
  double s = 0.0;
  if (km > -INFINITY) {
    for (int c = 0; c < G; ++c) {
      const double sc = p[c].s;
      if (sc > 0.0) {
        const float d = p[c].k - km;  // integer valued, <= 0
        s += ldexp(sc, d < -2000.f ? -2000 : (int)d);
      }
    }
  }
  kmax = km;
  S = s;
}

__device__ __forceinline__ void merge_argmax_row(const Partial* p, int G, float& best, int& bi) {
  best = -INFINITY;
  bi = 0x7fffffff;
  for (int c = 0; c < G; ++c) argmax_merge(best, bi, p[c].k, p[c].idx);
  if (bi == 0x7fffffff) bi = 0;  // no element above -inf: lowest index
}

// probability of x under a merged row: 2^(x*c - K*) / S, in fp64
__device__ __forceinline__ double row_prob(float x, float c, float kmax, double S) {
  if (!(S > 0.0)) return 0.0;
  const double arg = (double)x * (double)c - (double)kmax;
  return exp2(arg) / S;
}

template <int DT>
__global__ void __launch_bounds__(kBlock) k_finalize(VerifyArgs a) {
  constexpr int S = Elem<DT>::kBytes;
  const int b = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  if (b >= a.B) return;
  const int l = lane_id();
  const int R = 2 * a.K + 1;
  const int G = a.G;
  const int K = a.K;
  ReqState& rs = a.req[b];
  const int L = rs.L;
  const int kind = rs.kind;
  const Partial* pb = a.part1 + (size_t)b * R * G;
  int32_t* tok = a.tokens + (size_t)b * (K + 1);

  // drafted ids of the scheduled positions
  int y = 0;
  int bad = 0;
  if (l < L) {
    y = a.drafted[(size_t)b * K + l];
    if (y < 0 || y >= a.V) bad = DSPARK_DEV_BAD_TOKEN;
  }
  bad = wave_or(bad);
  if (kind == kKindSkip || (bad & DSPARK_DEV_BAD_TOKEN)) {
    for (int i = l; i <= K; i += kWave) tok[i] = -1;
    if (l < K) {
      if (a.p_tok) a.p_tok[(size_t)b * K + l] = 0.f;
      if (a.q_tok) a.q_tok[(size_t)b * K + l] = 0.f;
    }
    if (l == 0) {
      a.accepted[b] = 0;
      rs.mode = kModeNone;
      if (bad) flag(a.dev_status, bad);
    }
    return;
  }

  if (kind == kKindGreedy) {
    // lane j merges target row j (j <= L); row 64 (L = K = 64) by lane 0 later
    float g_best = 0.f;
    int g = 0;
    if (l <= L) {
      merge_argmax_row(pb + (size_t)l * G, G, g_best, g);
      if (g_best == -INFINITY) bad |= DSPARK_DEV_NONFINITE;  // no finite logit
    }
    const bool acc = l < L && y == g;
    const uint64_t m = __ballot(acc);
    const uint64_t want = L >= 64 ? ~0ull : ((1ull << L) - 1ull);
    const uint64_t rej = ~m & want;
    const int acc_n = rej ? __builtin_ctzll(rej) : L;
    int ga = __shfl(g, acc_n & 63);
    if (L == 64 && l == 0) {
      float b64;
      int g64;
      merge_argmax_row(pb + (size_t)64 * G, G, b64, g64);
      if (b64 == -INFINITY) bad |= DSPARK_DEV_NONFINITE;
      if (acc_n == 64) ga = g64;
    }
    if (acc_n == 64) ga = __shfl(ga, 0);  // lane 0 merged row 64
    bad = wave_or(bad);
    for (int i = l; i <= K; i += kWave) tok[i] = i < acc_n ? a.drafted[(size_t)b * K + i] : (i == acc_n ? ga : -1);
    if (l < K) {
      if (a.p_tok) a.p_tok[(size_t)b * K + l] = 0.f;
      if (a.q_tok) a.q_tok[(size_t)b * K + l] = 0.f;
    }
    if (l == 0) {
      a.accepted[b] = acc_n;
      rs.a = acc_n;
      rs.mode = kModeDone;
      if (bad) flag(a.dev_status, bad);
    }
    return;
  }

  // softmax rule
  const float c = rs.c;
  float kt = -INFINITY, kd = -INFINITY;
  double St = 0.0, Sd = 0.0;
  bool acc = false;
  float pf = 0.f, qf = 0.f;
  if (l < L) {
    merge_softmax_row(pb + (size_t)l * G, G, kt, St);
    merge_softmax_row(pb + (size_t)(K + 1 + l) * G, G, kd, Sd);
    if (!(St > 0.0) || !(Sd > 0.0)) bad |= DSPARK_DEV_NONFINITE;  // no finite logit
    const float xt = load_elem<DT>(target_row(a, b, l, S), y);
    const float xd = load_elem<DT>(draft_row(a, b, l, S), y);
    const double p = row_prob(xt, c, kt, St);
    const double q = row_prob(xd, c, kd, Sd);
    double alpha;
    if (p == 0.0) alpha = 0.0;
    else if (q == 0.0) alpha = 1.0;
    else alpha = fmin(1.0, p / q);
    const float u = a.uniforms[(size_t)b * (K + 1) + l];
    if (!(u >= 0.f && u < 1.f)) bad |= DSPARK_DEV_BAD_UNIFORM;
    acc = (double)u < alpha;
    pf = (float)p;
    qf = (float)q;
  }
  if (l < K) {
    if (a.p_tok) a.p_tok[(size_t)b * K + l] = pf;
    if (a.q_tok) a.q_tok[(size_t)b * K + l] = qf;
  }
  const uint64_t m = __ballot(acc);
  const uint64_t want = L >= 64 ? ~0ull : ((1ull << L) - 1ull);
  const uint64_t rej = ~m & want;
  const int acc_n = rej ? __builtin_ctzll(rej) : L;
  for (int i = l; i <= K; i += kWave)
    tok[i] = i < acc_n ? a.drafted[(size_t)b * K + i] : -1;
  if (acc_n < L) {
    // residual at the rejected position: lane acc_n holds both row merges
    if (l == acc_n) {
      rs.mode = kModeResidual;
      rs.row = acc_n;
      rs.kt = kt;
      rs.kd = kd;
      rs.st = St;
      rs.sd = Sd;
    }
  }
  if (l == 0) {
    // the bonus row is read whatever happens, so it is always checked
    float kb;
    double Sb;
    merge_softmax_row(pb + (size_t)L * G, G, kb, Sb);
    if (!(Sb > 0.0)) bad |= DSPARK_DEV_NONFINITE;
    if (acc_n == L) {
      rs.mode = kModeDrawP;
      rs.row = L;
      rs.kt = kb;
      rs.st = Sb;
    }
    const float uf = a.uniforms[(size_t)b * (K + 1) + K];
    if (!(uf >= 0.f && uf < 1.f)) bad |= DSPARK_DEV_BAD_UNIFORM;
    a.accepted[b] = acc_n;
    rs.a = acc_n;
  }
  bad = wave_or(bad);
  if (l == 0 && bad) flag(a.dev_status, bad);
}

// ------------------------------------------------------------------ pass 2

// Normalised-probability shifts of a residual row pair: p(v) ~ 2^(x*c + nbt),
// q(v) ~ 2^(x*c + nbd) in fp32 arithmetic.
struct ResidualRows {
  const char* tchunk;
  const char* dchunk;
  float c, nbt, nbd;
  float kt, kd;
  double st, sd;
  __device__ ResidualRows(const char* t, const char* d, float c_, float kt_, double st_, float kd_,
                          double sd_)
      : tchunk(t), dchunk(d), c(c_), kt(kt_), kd(kd_), st(st_), sd(sd_) {
    nbt = (float)(-(double)kt - log2(st));
    nbd = (float)(-(double)kd - log2(sd));
  }
  // exact residual of one element (fp64 exponent, fp64 exp2)
  template <int DT> __device__ double exact(int idx) const {
    const double p = exp2((double)load_elem<DT>(tchunk, idx) * (double)c - (double)kt) / st;
    const double q = exp2((double)load_elem<DT>(dchunk, idx) * (double)c - (double)kd) / sd;
    return fmax(p - q, 0.0);
  }
  // fp32 residual and the larger of the two normalised probabilities
  __device__ float fast(float xt, float xd, float& big) const {
    const float p = fast_exp2(fmaf(xt, c, nbt));
    const float q = fast_exp2(fmaf(xd, c, nbd));
    big = fmaxf(p, q);
    return fmaxf(p - q, 0.f);
  }
};

// element index (within the chunk) of lane l's i-th element, i = v*P + e
template <int P> __device__ __forceinline__ int lane_elem(int l, int i) {
  return ((i / P) * kWave + l) * P + (i % P);
}

// Residual mass of one work item, summed per lane.  fp32 everywhere, except
// lanes whose largest normalised p or q reaches 2^-12: those lanes are redone
// in fp64 (the cancellation in p - q makes their fp32 error visible once the
// residual is divided by its total mass).  Sets `heavy` for such lanes.
template <int DT>
__device__ double residual_lane_sum(const ResidualRows& rr, int n, bool vec_ok, bool& heavy) {
  Tile<DT> tt, td;
  tt.load(rr.tchunk, n, vec_ok);
  td.load(rr.dchunk, n, vec_ok);
  constexpr int P = Elem<DT>::kPerVec;
  float lane = 0.f, hv = 0.f;
#pragma unroll
  for (int v = 0; v < kUnroll; ++v) {
    float r[P];
#pragma unroll
    for (int e = 0; e < P; ++e) {
      float big;
      r[e] = rr.fast(tt.at(v, e), td.at(v, e), big);
      hv = fmaxf(hv, big);
    }
    float s4 = (r[0] + r[1]) + (r[2] + r[3]);
    if constexpr (P == 8) s4 += (r[4] + r[5]) + (r[6] + r[7]);
    lane += s4;
  }
  heavy = hv >= kHeavy;
  double lane64 = (double)lane;
  if (heavy) {
    const int l = lane_id();
    double acc = 0.0;
#pragma unroll 1
    for (int i = 0; i < kUnroll * P; ++i) {
      const int idx = lane_elem<P>(l, i);
      if (idx < n) acc += rr.template exact<DT>(idx);
    }
    lane64 = acc;
  }
  return lane64;
}

template <int DT>
__global__ void __launch_bounds__(kBlock) k_pass2(VerifyArgs a) {
  constexpr int S = Elem<DT>::kBytes;
  constexpr int E = item_elems<DT>();
  const int G = a.G;
  const long n_items = (long)a.B * G;
  const long wave0 = (long)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  const long stride = (long)gridDim.x * kWavesPerBlock;
  for (long it = wave0; it < n_items; it += stride) {
    const int b = (int)(it / G);
    const int c = (int)(it % G);
    const ReqState& rs = a.req[b];
    if (rs.mode != kModeResidual) continue;
    const int e0 = c * E;
    const int n = min(E, a.V - e0);
    const ResidualRows rr(target_row(a, b, rs.row, S) + (size_t)e0 * S,
                          draft_row(a, b, rs.row, S) + (size_t)e0 * S, rs.c, rs.kt, rs.st, rs.kd,
                          rs.sd);
    bool heavy;
    const double z = wave_sum(residual_lane_sum<DT>(rr, n, a.vec_ok, heavy));
    if (lane_id() == 0) a.part2[(size_t)b * G + c] = z;
  }
}

// ------------------------------------------------------------------ sample

// Scan one chunk in token order and return the index (within the chunk) of
// the first element whose running mass exceeds `target`, or, if none does,
// the last element with positive mass (or -1 when the chunk has none).
// `mass(idx)` gives the mass of chunk element idx as this lane computes it;
// lane l owns the elements lane_elem<P>(l, .).
template <int P, typename MassFn>
__device__ int scan_chunk(MassFn mass, int n, double target) {
  const int l = lane_id();
  double base = 0.0;
  int last_pos = -1;
#pragma unroll 1
  for (int v = 0; v < kUnroll; ++v) {
    double w[P];
    double ls = 0.0;
    int lp = -1;
#pragma unroll
    for (int e = 0; e < P; ++e) {
      const int idx = (v * kWave + l) * P + e;
      w[e] = idx < n ? mass(idx) : 0.0;
      ls += w[e];
      if (w[e] > 0.0) lp = idx;
    }
    for (int o = 32; o > 0; o >>= 1) lp = max(lp, __shfl_xor(lp, o));
    if (lp >= 0) last_pos = lp;
    const double incl = wave_incl_scan(ls);
    const double row_total = __shfl(incl, kWave - 1);
    if (base + row_total > target) {
      int cand = -1;
      if (base + incl > target) {
        double run = base + incl - ls;
#pragma unroll
        for (int e = 0; e < P; ++e) {
          run += w[e];
          if (cand < 0 && run > target && w[e] > 0.0) cand = (v * kWave + l) * P + e;
        }
      }
      const uint64_t has = __ballot(cand >= 0);
      if (has) return __shfl(cand, __builtin_ctzll(has));
    }
    base += row_total;
  }
  return last_pos;
}

template <int DT>
__global__ void __launch_bounds__(kBlock) k_sample(VerifyArgs a) {
  constexpr int S = Elem<DT>::kBytes;
  constexpr int E = item_elems<DT>();
  constexpr int P = Elem<DT>::kPerVec;
  const int b = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  if (b >= a.B) return;
  ReqState& rs = a.req[b];
  int mode = rs.mode;
  if (mode != kModeResidual && mode != kModeDrawP) return;
  const int l = lane_id();
  const int G = a.G;
  const int K = a.K;
  const float c = rs.c;
  const double u = (double)a.uniforms[(size_t)b * (K + 1) + K];
  const int R = 2 * K + 1;

  float kp = rs.kt;
  if (mode == kModeResidual) {
    double Z = 0.0;
    for (int c0 = 0; c0 < G; c0 += kWave) {
      const int ci = c0 + l;
      Z += wave_sum(ci < G ? a.part2[(size_t)b * G + ci] : 0.0);
    }
    if (!(Z > 0.0)) {
      // no residual mass: draw from p at the rejected position
      mode = kModeDrawP;
      double s2;
      merge_softmax_row(a.part1 + ((size_t)b * R + rs.row) * G, G, kp, s2);
    }
  }
  const Partial* prow = a.part1 + ((size_t)b * R + rs.row) * G;

  // chunk masses, in chunk order (p-mode: scaled to the row shift kp)
  auto chunk_mass = [&](int ci) -> double {
    if (ci >= G) return 0.0;
    if (mode == kModeResidual) return a.part2[(size_t)b * G + ci];
    const Partial& p = prow[ci];
    if (!(p.s > 0.0)) return 0.0;
    const float d = p.k - kp;
    return ldexp(p.s, d < -2000.f ? -2000 : (int)d);
  };
  double total = 0.0;
  for (int c0 = 0; c0 < G; c0 += kWave) total += wave_sum(chunk_mass(c0 + l));
  const double target = u * total;

  // chunk holding the draw: first chunk whose inclusive prefix exceeds target
  int cstar = -1, clast = -1;
  double base = 0.0;
  for (int c0 = 0; c0 < G && cstar < 0; c0 += kWave) {
    const double w = chunk_mass(c0 + l);
    const double incl = wave_incl_scan(w);
    const uint64_t hit = __ballot(base + incl > target && w > 0.0);
    const uint64_t pos = __ballot(w > 0.0);
    if (pos) clast = c0 + 63 - __builtin_clzll(pos);
    if (hit) {
      const int hl = __builtin_ctzll(hit);
      cstar = c0 + hl;
      base += __shfl(incl - w, hl);
    } else {
      base += __shfl(incl, kWave - 1);
    }
  }
  // rounding pushed the target past the end: take the last chunk with mass
  // and, inside it, the last token with mass
  const bool past_end = cstar < 0;
  if (past_end) cstar = clast;
  int tokv = 0;
  if (cstar >= 0) {
    const int e0 = cstar * E;
    const int n = min(E, a.V - e0);
    const double ctarget = past_end ? INFINITY : target - base;
    int f;
    if (mode == kModeResidual) {
      const ResidualRows rr(target_row(a, b, rs.row, S) + (size_t)e0 * S,
                            draft_row(a, b, rs.row, S) + (size_t)e0 * S, c, rs.kt, rs.st, rs.kd,
                            rs.sd);
      // same lane classification as the residual pass
      float hv = 0.f;
#pragma unroll 1
      for (int i = 0; i < kUnroll * P; ++i) {
        const int idx = lane_elem<P>(l, i);
        if (idx < n) {
          float big;
          rr.fast(load_elem<DT>(rr.tchunk, idx), load_elem<DT>(rr.dchunk, idx), big);
          hv = fmaxf(hv, big);
        }
      }
      const bool heavy = hv >= kHeavy;
      f = scan_chunk<P>(
          [&](int idx) -> double {
            if (heavy) return rr.template exact<DT>(idx);
            float big;
            return (double)rr.fast(load_elem<DT>(rr.tchunk, idx), load_elem<DT>(rr.dchunk, idx), big);
          },
          n, ctarget);
    } else {
      const char* tc = target_row(a, b, rs.row, S) + (size_t)e0 * S;
      const float nk = -prow[cstar].k;
      const float d = prow[cstar].k - kp;
      const int sh = d < -2000.f ? -2000 : (int)d;
      f = scan_chunk<P>(
          [&](int idx) -> double {
            return ldexp((double)fast_exp2(fmaf(load_elem<DT>(tc, idx), c, nk)), sh);
          },
          n, ctarget);
    }
    tokv = e0 + (f >= 0 ? f : 0);
  }
  if (l == 0) a.tokens[(size_t)b * (K + 1) + rs.a] = tokv;
}

// ------------------------------------------------------------------ launch

static int grid_for(long items) {
  long g = (items + kWavesPerBlock - 1) / kWavesPerBlock;
  const long cap = 256L * 8;  // 8 workgroups per CU on 256 CUs
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return (int)g;
}

template <int DT>
static int launch_verify_t(VerifyArgs& a, hipStream_t st) {
  const int R = 2 * a.K + 1;
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(1024), 0, st, a);
  hipLaunchKernelGGL(k_pass1<DT>, dim3(grid_for((long)a.B * R * a.G)), dim3(kBlock), 0, st, a);
  const int gb = (a.B + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL(k_finalize<DT>, dim3(gb), dim3(kBlock), 0, st, a);
  if (!a.greedy_only) {
    hipLaunchKernelGGL(k_pass2<DT>, dim3(grid_for((long)a.B * a.G)), dim3(kBlock), 0, st, a);
    hipLaunchKernelGGL(k_sample<DT>, dim3(gb), dim3(kBlock), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_ERR_LAUNCH;
}

int launch_verify(VerifyArgs& a, int dtype, hipStream_t st) {
  return dtype == DSPARK_BF16 ? launch_verify_t<DSPARK_BF16>(a, st)
                              : launch_verify_t<DSPARK_F32>(a, st);
}

}  // namespace dspark
