// Semi-autoregressive drafting with the Markov logit bias (DSpark Guide, the
// Markov logit-bias head and its code listing): for positions k = 1..K in
// order,
//   corrected[b,k] = base[b,k] + scale * U . Vm[y_{k-1}]^T   (U, Vm: V x r)
//   y_k ~ softmax(corrected[b,k] / T_b)  (inverse CDF at uniforms[b,k-1];
//         the lowest-index maximum at T = 0),  y_0 = the last target token.
// Two launches per position:
//   k_markov_bias  an MFMA contraction: persistent workgroups (three per
//                  compute unit) stage the previous tokens' rows of Vm for 64
//                  requests in LDS once and loop over 64-row tiles of U; four
//                  waves of 16 rows run v_mfma_f32_16x16x32_bf16 over the
//                  rank (one 16x16x16 step for a 16-entry remainder). A
//                  tile's rows of U and base logits are requested one tile
//                  ahead, and every global access has four lanes on 64
//                  contiguous bytes of a row. The bias tile goes through LDS
//                  to [request][row], and each lane finishes 16 rows of one
//                  request: adds the scaled bias to the base logits, stores
//                  the corrected logits in the base dtype (16-byte accesses)
//                  and summarises the tile per request over the four lanes
//                  that share it (integer shift k = ceil(max * c) and the sum
//                  of 2^(x*c - k) over the stored values, or (max, lowest
//                  index) at T = 0);
//   k_markov_draw  one workgroup per request: each thread reads a
//                  contiguous run of tile summaries once, the block merges
//                  them (exact power-of-two rescaling) and scans the runs to
//                  the tile holding u * S, and wave 0 finds the token inside
//                  it by a scan of its 64 stored logits.
// The bias is an fp32 sum (MFMA accumulation), scaled and added in fp32,
// and the draw reads the stored logits, so the draft distribution is exactly
// what the verifier reads back.
#include <hip/hip_runtime.h>

#include <cfloat>

#include "markov_args.hpp"

namespace dspark {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

namespace {

__device__ __forceinline__ float temp_c(float T) {
  return (float)(1.4426950408889634 / (double)T);  // log2(e) / T, as the verifier
}

// previous token of request b before position a.step (checked)
__device__ __forceinline__ int prev_token(const MarkovArgs& a, int b, int& bad) {
  const int y = a.step == 1 ? a.y0[b] : a.drafted[(size_t)b * a.K + a.step - 2];
  if (y < 0 || y >= a.V) {
    bad |= DSPARK_DEV_BAD_TOKEN;
    return 0;
  }
  return y;
}

// round to the storage dtype (bf16: nearest even) and back
template <int DT>
__device__ __forceinline__ float store_elem(void* row, int v, float x) {
  if constexpr (DT == DSPARK_BF16) {
    const uint32_t u = __float_as_uint(x);
    uint16_t h;
    if (x != x) h = 0x7fc0;
    else h = (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
    static_cast<uint16_t*>(row)[v] = h;
    return __uint_as_float((uint32_t)h << 16);
  } else {
    static_cast<float*>(row)[v] = x;
    return x;
  }
}

}  // namespace

static_assert(kMarkovBatch * 4 == 256, "four staging threads per request");

template <int DT>
__global__ void __launch_bounds__(256) k_markov_bias(MarkovArgs a) {
  constexpr int kLds = kMarkovMaxRank + 8;  // padded row of a staged Vm row (bf16)
  __shared__ __align__(16) uint16_t s_w[kMarkovBatch][kLds];
  // one tile's bias, [request][row] (rows padded to 68 floats: 16-byte aligned)
  __shared__ __align__(16) float s_c[kMarkovBatch][kMarkovRows + 4];
  const int b0 = blockIdx.y * kMarkovBatch;
  const int w = threadIdx.x / kWave, l = lane_id();
  const int r = a.r, K = a.K, V = a.V, k = a.step;
  const int r32 = r / 32;               // 16x16x32 steps over the rank
  const bool tail16 = (r & 31) != 0;    // and one 16x16x16 step on the last 16 entries
  int bad = 0;
  // lane l: row l % 16 of its wave's 16 rows and rank slice q = l / 16 in the
  // contraction; request 16w + l/4 and quarter part = l % 4 of the tile's
  // rows in the epilogue
  const int row16 = l & 15, q = l >> 4, ri = l >> 2, part = l & 3;
  const int bl = b0 + w * 16 + ri;
  const bool bok = bl < a.B;
  const int bb = bok ? bl : a.B - 1;
  const float Tl = a.temperature[bb];
  const bool greedy = Tl == 0.f;
  const float cl = greedy ? 0.f : temp_c(Tl);
  const size_t roff = ((size_t)bb * K + (k - 1)) * (size_t)V;
  const char* brow = static_cast<const char*>(a.base) + roff * Elem<DT>::kBytes;
  char* crow = static_cast<char*>(a.corrected) + roff * Elem<DT>::kBytes;
  // 16-byte vector accesses when rows start on 16-byte boundaries
  constexpr int kVecElems = 16 / Elem<DT>::kBytes;
  constexpr int kPieces = 16 / kVecElems;
  const bool vec = (V % kVecElems) == 0 &&
                   ((uintptr_t)a.base % 16) == 0 && ((uintptr_t)a.corrected % 16) == 0;
  // element i of this lane's 16 rows: 16-byte piece i / kVecElems sits at
  // rows 4 kVecElems (i / kVecElems) + kVecElems part .. + kVecElems - 1, so
  // the four lanes of a request cover 64 contiguous bytes per piece
  auto row_of = [&](int i) {
    return (i / kVecElems) * 4 * kVecElems + part * kVecElems + (i % kVecElems);
  };
  // A tile's operands, requested one tile ahead so that they arrive during
  // the current tile's MFMAs and epilogue:
  //   U row (tile row 16w + l % 16; rows past V re-read row V-1 and are
  //   dropped): rank entries 32 i + 8 q .. + 7 for step i (the 16-entry tail:
  //   32 i + 4 q .. + 3), so a quarter-wave reads 64 contiguous bytes of
  //   each of its 16 rows per load;
  //   the 16 base logits as raw words (whole vector tiles; a ragged tile
  //   reads them element by element in the epilogue)
  constexpr int kAw = kMarkovMaxRank / 8;
  constexpr int kXw = 16 * Elem<DT>::kBytes / 4;
  uint32_t areg[kAw], anext[kAw], xraw[kXw], xnext[kXw];
  auto load_a = [&](int tile, uint32_t (&dst)[kAw]) {
    const int vrow = min(tile * kMarkovRows + w * 16 + row16, V - 1);
    const uint16_t* up = a.U + (size_t)vrow * r;
#pragma unroll
    for (int i = 0; i < kMarkovMaxRank / 32; ++i) {
      if (i < r32) {
        const uint4 v = *reinterpret_cast<const uint4*>(up + 32 * i + 8 * q);
        dst[4 * i] = v.x;
        dst[4 * i + 1] = v.y;
        dst[4 * i + 2] = v.z;
        dst[4 * i + 3] = v.w;
      } else if (i == r32 && tail16) {
        const uint2 v = *reinterpret_cast<const uint2*>(up + 32 * i + 4 * q);
        dst[4 * i] = v.x;
        dst[4 * i + 1] = v.y;
        dst[4 * i + 2] = dst[4 * i + 3] = 0u;
      } else {
        dst[4 * i] = dst[4 * i + 1] = dst[4 * i + 2] = dst[4 * i + 3] = 0u;
      }
    }
  };
  auto load_base = [&](int tile, uint32_t (&dst)[kXw]) {
    const int vt = tile * kMarkovRows;
    if (vec && vt + kMarkovRows <= V) {
#pragma unroll
      for (int g = 0; g < kPieces; ++g) {
        const uint4 v = *reinterpret_cast<const uint4*>(
            brow + (size_t)(vt + g * 4 * kVecElems + part * kVecElems) * Elem<DT>::kBytes);
        dst[4 * g] = v.x;
        dst[4 * g + 1] = v.y;
        dst[4 * g + 2] = v.z;
        dst[4 * g + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kXw; ++i) dst[i] = 0u;
    }
  };
  if (blockIdx.x < a.tiles) {
    load_a(blockIdx.x, areg);
    load_base(blockIdx.x, xraw);
  }
  // the previous tokens' rows of Vm (zero rows past B), staged once for all
  // the tiles this workgroup takes: four threads per request, each with one
  // token load and then all its 16-byte pieces in flight at once (the four
  // threads cover 64 contiguous bytes per step)
  {
    const int i = threadIdx.x >> 2, sub = threadIdx.x & 3;
    const int b = b0 + i;
    const int pieces = r / 8;
    const uint16_t* vrow = nullptr;
    if (b < a.B) vrow = a.Vm + (size_t)prev_token(a, b, bad) * r;
    uint4 v[kMarkovMaxRank / 32];
#pragma unroll
    for (int j = 0; j < kMarkovMaxRank / 32; ++j) {
      const int piece = 4 * j + sub;
      v[j] = uint4{0u, 0u, 0u, 0u};
      if (vrow && piece < pieces) v[j] = *reinterpret_cast<const uint4*>(vrow + piece * 8);
    }
#pragma unroll
    for (int j = 0; j < kMarkovMaxRank / 32; ++j) {
      const int piece = 4 * j + sub;
      if (piece < pieces) *reinterpret_cast<uint4*>(&s_w[i][piece * 8]) = v[j];
    }
  }
  __syncthreads();
  for (int tile = blockIdx.x; tile < a.tiles; tile += gridDim.x) {
    const int nxt = tile + (int)gridDim.x;
    if (nxt < a.tiles) {
      load_a(nxt, anext);
      load_base(nxt, xnext);
    }
    const int vt = tile * kMarkovRows;
    const bool full = vec && vt + kMarkovRows <= V;
    // D[row][request] = sum over the rank of U[row][j] * Vm[prev][j]: A and
    // B take the same rank entries in every lane and step, so each product
    // enters the sum once
    float4_t acc[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[nb] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kMarkovMaxRank / 32; ++ks) {
      if (ks < r32) {
        const uint4 aw = {areg[4 * ks], areg[4 * ks + 1], areg[4 * ks + 2], areg[4 * ks + 3]};
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, aw);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const bf16x8_t bv =
              *reinterpret_cast<const bf16x8_t*>(&s_w[nb * 16 + row16][32 * ks + 8 * q]);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[nb], 0, 0, 0);
        }
      } else if (ks == r32 && tail16) {
        short4_t av;
        av[0] = (short)(areg[4 * ks] & 0xffffu);
        av[1] = (short)(areg[4 * ks] >> 16);
        av[2] = (short)(areg[4 * ks + 1] & 0xffffu);
        av[3] = (short)(areg[4 * ks + 1] >> 16);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const short4_t bv =
              *reinterpret_cast<const short4_t*>(&s_w[nb * 16 + row16][32 * ks + 4 * q]);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, acc[nb], 0, 0, 0);
        }
      }
    }
    // lane l holds rows 16w + 4q + j of requests 16 nb + l % 16: through
    // LDS to [request][row]
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j) s_c[nb * 16 + row16][w * 16 + 4 * q + j] = acc[nb][j];
    __syncthreads();
    // epilogue: corrected logits of this lane's 16 rows, stored, and the
    // tile's summary per request over the four lanes that share it
    float xb[16];
    if (full) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (DT == DSPARK_BF16)
          xb[i] = __uint_as_float((i & 1) ? (xraw[i >> 1] & 0xffff0000u) : (xraw[i >> 1] << 16));
        else
          xb[i] = __uint_as_float(xraw[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) xb[i] = load_elem<DT>(brow, min(vt + row_of(i), V - 1));
    }
    float xs[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float x = xb[i] + a.scale * s_c[w * 16 + ri][row_of(i)];
      // rounded to the storage dtype (bf16: nearest even; a NaN here is
      // flagged below, and the request's outputs are then unspecified)
      if constexpr (DT == DSPARK_BF16) {
        const uint32_t u = __float_as_uint(x);
        xs[i] = __uint_as_float((u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u);
      } else {
        xs[i] = x;
      }
    }
    // rows past V (ragged last tile) and lanes past B take no part
    if (!full || !bok) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (!bok || vt + row_of(i) >= V) xs[i] = -INFINITY;
    }
    if (bok) {
      if (full) {
#pragma unroll
        for (int g = 0; g < kPieces; ++g) {
          uint32_t wd[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (DT == DSPARK_BF16)
              wd[e] = (__float_as_uint(xs[g * 8 + 2 * e]) >> 16) |
                      (__float_as_uint(xs[g * 8 + 2 * e + 1]) & 0xffff0000u);
            else
              wd[e] = __float_as_uint(xs[g * 4 + e]);
          }
          *reinterpret_cast<uint4*>(
              crow + (size_t)(vt + g * 4 * kVecElems + part * kVecElems) * Elem<DT>::kBytes) =
              uint4{wd[0], wd[1], wd[2], wd[3]};
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (vt + row_of(i) < V) store_elem<DT>(crow, vt + row_of(i), xs[i]);
      }
    }
    float m = xs[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) m = fmaxf(m, xs[i]);
    // NaN or +inf among the values: a scaled sum (no overflow from finite
    // values) is NaN or +inf exactly then; -inf alone leaves it -inf
    float fin = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) fin = fmaf(xs[i], 0x1p-8f, fin);
    if (fin != fin || fin == INFINITY) bad |= DSPARK_DEV_NONFINITE;
    m = fmaxf(m, dpp<kQuadXor1>(m));
    m = fmaxf(m, dpp<kQuadXor2>(m));
    Partial pt;
    if (greedy) {
      int at = 0x7fffffff;
#pragma unroll
      for (int i = 15; i >= 0; --i)  // rows increase with i
        if (xs[i] == m && vt + row_of(i) < V) at = vt + row_of(i);
      at = min(at, dpp<kQuadXor1>(at));
      at = min(at, dpp<kQuadXor2>(at));
      pt.k = m;
      pt.idx = at;
      pt.s = 0.0;
    } else {
      const bool none = m == -INFINITY;
      const float kk = ceilf(m * cl);
      const float nk = none ? 0.f : -kk;
      float e[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) e[i] = fast_exp2(fmaf(xs[i], cl, nk));
      float s8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) s8[i] = e[2 * i] + e[2 * i + 1];
      const float s16 = ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
      double sd = (double)s16;
      sd += dpp<kQuadXor1>(sd);
      sd += dpp<kQuadXor2>(sd);
      pt.k = none ? -INFINITY : kk;
      pt.idx = 0;
      pt.s = sd;
    }
    if (bok && part == 0) a.part[(size_t)bl * a.tiles + tile] = pt;
    __syncthreads();  // s_c is rewritten by the next tile
#pragma unroll
    for (int i = 0; i < kAw; ++i) areg[i] = anext[i];
#pragma unroll
    for (int i = 0; i < kXw; ++i) xraw[i] = xnext[i];
  }
  if (bad) flag(a.dev_status, bad);
}

// block-wide helpers of k_markov_draw (256 threads, 4 waves)
constexpr int kRun = 16;  // tile summaries a draw thread keeps in registers
struct DrawLds {
  double w[4];
  float f[4];
  int i[4];
  int tile;
  double base;
};

template <int DT>
__global__ void __launch_bounds__(256) k_markov_draw(MarkovArgs a) {
  __shared__ DrawLds sh;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, w = tid / kWave, l = lane_id();
  const int K = a.K, V = a.V, k = a.step, nt = a.tiles;
  const Partial* pr = a.part + (size_t)b * nt;
  const size_t roff = ((size_t)b * K + (k - 1)) * (size_t)V;
  const void* crow = static_cast<const char*>(a.corrected) + roff * Elem<DT>::kBytes;
  // each thread owns a contiguous run of tiles; the first kRun summaries are
  // read into registers at once, together with the temperature and the
  // uniform (runs are longer only past 2^18 tokens: the rest is re-read)
  const int per = (nt + 255) / 256;
  const int t0 = min(tid * per, nt), t1 = min(t0 + per, nt);
  float rk[kRun];
  int rx[kRun];
  double rs[kRun];
#pragma unroll
  for (int j = 0; j < kRun; ++j) {
    rk[j] = -INFINITY;
    rx[j] = 0x7fffffff;
    rs[j] = 0.0;
    if (t0 + j < t1) {
      const Partial p = pr[t0 + j];
      rk[j] = p.k;
      rx[j] = p.idx;
      rs[j] = p.s;
    }
  }
  const float T = a.temperature[b];
  const double u = (double)a.uniforms[(size_t)b * K + (k - 1)];
  int y = 0;
  double qy = 1.0;
  if (!(T >= 0.f)) {
    if (tid == 0) flag(a.dev_status, DSPARK_DEV_BAD_TEMP);
  } else if (T == 0.f) {
    // the lowest-index maximum over the tiles
    float m = -INFINITY;
    int mi = 0x7fffffff;
    auto take = [&](float pk, int pi) {
      if (pk > m || (pk == m && pi < mi)) {
        m = pk;
        mi = pi;
      }
    };
#pragma unroll
    for (int j = 0; j < kRun; ++j) take(rk[j], rx[j]);
    for (int t = t0 + kRun; t < t1; ++t) {
      const Partial p = pr[t];
      take(p.k, p.idx);
    }
    // wave, then block
    for (int o = 32; o > 0; o >>= 1) take(__shfl_xor(m, o), __shfl_xor(mi, o));
    if (l == 0) {
      sh.f[w] = m;
      sh.i[w] = mi;
    }
    __syncthreads();
    m = sh.f[0];
    mi = sh.i[0];
    for (int ww = 1; ww < 4; ++ww) take(sh.f[ww], sh.i[ww]);
    y = mi < V ? mi : 0;
  } else {
    const float c = temp_c(T);
    float km = -INFINITY;
#pragma unroll
    for (int j = 0; j < kRun; ++j) km = fmaxf(km, rk[j]);
    for (int t = t0 + kRun; t < t1; ++t) km = fmaxf(km, pr[t].k);
    // shift of the row: the largest tile shift
    km = wave_max(km);
    if (l == 0) sh.f[w] = km;
    __syncthreads();
    km = fmaxf(fmaxf(sh.f[0], sh.f[1]), fmaxf(sh.f[2], sh.f[3]));
    auto scaled = [&](float pk, double ps) -> double {
      return ps > 0.0 ? ldexp(ps, shift_amount(pk - km)) : 0.0;
    };
    // the run's mass, then a block scan
    double own = 0.0;
    int lastpos = -1;
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
      const double mt = scaled(rk[j], rs[j]);
      own += mt;
      if (mt > 0.0) lastpos = t0 + j;
    }
    for (int t = t0 + kRun; t < t1; ++t) {
      const Partial p = pr[t];
      const double mt = scaled(p.k, p.s);
      own += mt;
      if (mt > 0.0) lastpos = t;
    }
    const double incl = wave_incl_scan(own);
    const int lastw = wave_max_i(lastpos);
    if (l == kWave - 1) {
      sh.w[w] = incl;
      sh.i[w] = lastw;
    }
    __syncthreads();
    double pre = 0.0, S = 0.0;
    int last = -1;
    for (int ww = 0; ww < 4; ++ww) {
      if (ww < w) pre += sh.w[ww];
      S += sh.w[ww];
      last = max(last, sh.i[ww]);
    }
    const double target = u * S;
    // a run's bounds: the previous lane's inclusive sum and its own, so that
    // consecutive runs meet exactly and one run holds the target
    double excl = __shfl_up(incl, 1);
    if (l == 0) excl = 0.0;
    const double before_me = pre + excl;
    const double after_me = pre + incl;
    const bool mine = own > 0.0 && after_me > target && before_me <= target;
    if (tid == 0) {
      sh.tile = last;  // rounding left no crossing: the last tile with mass
      sh.base = -1.0;
    }
    __syncthreads();
    if (mine) {
      // first tile of this run whose running mass passes the target
      double run = before_me;
      int tt = -1;
      double tb = 0.0;
#pragma unroll
      for (int j = 0; j < kRun; ++j) {
        const double mt = scaled(rk[j], rs[j]);
        if (tt < 0 && mt > 0.0 && run + mt > target) {
          tt = t0 + j;
          tb = run;
        }
        run += mt;
      }
      for (int t = t0 + kRun; t < t1 && tt < 0; ++t) {
        const Partial p = pr[t];
        const double mt = scaled(p.k, p.s);
        if (mt > 0.0 && run + mt > target) {
          tt = t;
          tb = run;
        }
        run += mt;
      }
      if (tt >= 0) {
        sh.tile = tt;
        sh.base = tb;
      }
    }
    __syncthreads();
    // the tile's 64 tokens, one per lane of wave 0, which also stores the
    // result
    if (w != 0) return;
    const int tile = max(sh.tile, 0);
    const double base = sh.base;
    const Partial p = pr[tile];
    const int v = tile * kMarkovRows + l;
    const float x = v < V ? load_elem<DT>(crow, v) : -INFINITY;
    const double m = v < V ? ldexp((double)fast_exp2(fmaf(x, c, p.k == -INFINITY ? 0.f : -p.k)),
                                   shift_amount(p.k - km))
                           : 0.0;
    const double inc = wave_incl_scan(m);
    const bool past = base < 0.0;  // no crossing: the last token with mass
    const uint64_t hit = __ballot(!past && m > 0.0 && base + inc > target);
    const int lastm = wave_max_i(m > 0.0 ? l : -1);
    const int pick = hit ? __builtin_ctzll(hit) : (lastm >= 0 ? lastm : 0);
    const float xp = __shfl(x, pick);
    y = tile * kMarkovRows + pick;
    qy = row_prob(xp, c, km, S);
  }
  if (tid == 0) {
    a.drafted[(size_t)b * K + (k - 1)] = y;
    if (a.q_tok) a.q_tok[(size_t)b * K + (k - 1)] = (float)qy;
  }
}

template <int DT>
static int launch_markov_t(MarkovArgs& a, hipStream_t st) {
  // persistent workgroups over the vocabulary tiles, three per compute unit
  // (51 KB of LDS each)
  const int wgs = min(a.tiles, 3 * compute_units());
  const dim3 gb((unsigned)wgs, (unsigned)((a.B + kMarkovBatch - 1) / kMarkovBatch));
  for (int k = 1; k <= a.K; ++k) {
    a.step = k;
    hipLaunchKernelGGL(k_markov_bias<DT>, gb, dim3(256), 0, st, a);
    hipLaunchKernelGGL(k_markov_draw<DT>, dim3((unsigned)a.B), dim3(256), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_ERR_LAUNCH;
}

int launch_markov(MarkovArgs& a, int dtype, hipStream_t st) {
  return dtype == DSPARK_BF16 ? launch_markov_t<DSPARK_BF16>(a, st)
                              : launch_markov_t<DSPARK_F32>(a, st);
}

}  // namespace dspark
