"""CPU oracle for confidence-scheduled block verification (test infrastructure).

This package is TEST INFRASTRUCTURE.  Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import it.  The HIP library never calls it
and it shares no code with the library: it is a plain, slow, direct transcript
of what the path computes, written so that it can be checked against the pages
by eye.  Floating point is fp64 except where the schedule must reproduce a
fixed fp32 decision (see ``schedule``).

Sources (page title, then section):

* "DSpark Deep Dive: How DeepSeek Squeezed an 85% Speedup Out of Inference
  Without Touching a Single Model Weight" (the Deep Dive):
  "Speculative Decoding From First Principles" (draft, verify, accept with
  probability min(1, p/q), resample a rejection from the normalised positive
  part of p - q); "Variable-Length Drafts" (verify from position 1 until the
  cumulative confidence drops below a threshold); "The Full Scheduling
  Pipeline" (1 <= L <= K; tokens past L are discarded); "The Optimization
  Logic" (a verify slot is better spent on a higher-confidence token of
  another request); "GPU-Resident Scheduling" (maximum-length buffers plus
  masking).
* "DSpark Guide: Confidence Speculative Decoding in LLMs" (the Guide):
  "1. The Mathematics of Suffix Decay" (alpha_k = min(1, P/Q_k);
  P(accepted length >= L) = prod_{k<=L} alpha_k); "2. Confidence-Scheduled
  Dynamic Verification" (C_k = prod_{i<=k} p_i; K* = max{k : C_k >= tau},
  truncate at the first k with C_k < tau; the tutorial code keeps at least one).
* "DSpark shows why fast AI inference is a scheduling problem, not a model
  trick": the prefix survival probability, truncated below a threshold.
* Markov logit-bias drafting: the Guide, the Markov logit-bias head (the
  corrected logits of position k are the parallel logits plus
  U . V[y_{k-1}]^T, U and V both vocabulary x rank) and its code listing
  (the bias is scaled by a learnable scalar; the first position's previous
  token is the last target token; positions are drafted in order).
* Online calibration: the Deep Dive, "Online Calibration" ("Sequential
  Temperature Scaling": per-position temperature on the logit of the score;
  "Online Adaptation" and "The Calibration Loop in Practice": per-position
  mean predicted confidence and acceptance fraction over a window of rounds,
  temperature += learning rate * (predicted - actual); ECE as the gap between
  predicted confidence and observed acceptance).
* Load-aware scheduling: the Guide, "Dynamic Verification Scheduling
  Algorithm" (load factor from queue depth and GPU memory in use, threshold
  rising with its square; the code listing's threshold line) and the Deep
  Dive, "The Throughput Curve", "The Optimization Logic" and "GPU-Resident
  Scheduling" (a pre-measured curve of tokens/s against tokens per forward
  pass, kept in GPU memory; a slot is worth adding while its marginal gain
  covers its cost).

Readings where the pages are silent (each also listed in the design notes):
the bonus token on full acceptance is drawn from target row L_b; a zero
residual (p == q) falls back to p; inverse-CDF draws walk token ids in
ascending order and take the first id whose cumulative mass exceeds u * Z
(fallback: the last id with positive mass); uniforms are laid out
``u[b, k-1]`` for position k's accept test and ``u[b, K]`` for the single final
draw; draft and target share the request's temperature and T = 0 selects the
greedy rule; greedy ties go to the lowest id; the budget counts drafted
positions only and is filled by (C desc, b asc, k asc) after reserving
``min_len`` positions per request.

Array conventions: target logits [B, K+1, V], draft logits [B, K, V], either
float32 or bf16 given as uint16 bit patterns; drafted int32 [B, K]; lengths
int32 [B]; temperature float32 [B]; uniforms float32 [B, K+1].

Parity status: every function here is pinned by the CPU tests (closed forms,
brute force, textbook special cases, hand-worked fixtures); no function is
"parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

BOUNDARY = 1e-6  # uniforms this close to a decision edge may legitimately differ

# device-status bits, same meaning as the library's (values fixed by the ABI)
DEV_BAD_TOKEN = 1
DEV_NONFINITE = 2
DEV_BAD_TEMP = 4
DEV_BAD_UNIFORM = 8
DEV_BAD_CONF = 16
DEV_BAD_LENGTH = 32
DEV_BAD_LOAD = 64
DEV_BAD_CURVE = 128


def widen(a) -> np.ndarray:
    """Exact widening to float64: bf16 bit patterns (uint16) or float32."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# Schedule: survival product, threshold truncation, global verify budget
# ----------------------------------------------------------------------------

def survival(conf) -> np.ndarray:
    """C[b,k] = C[b,k-1] * c[b,k] in fp32, left to right (Guide, "2.
    Confidence-Scheduled Dynamic Verification", C_k = prod_{i<=k} p_i).

    The product is kept in fp32 with one correctly rounded multiply per step so
    that the truncation decision below is reproducible bit for bit."""
    conf = np.asarray(conf, dtype=np.float32)
    C = np.empty_like(conf)
    if conf.shape[1] == 0:
        return C
    C[:, 0] = conf[:, 0]
    for k in range(1, conf.shape[1]):
        C[:, k] = C[:, k - 1] * conf[:, k]          # float32 * float32 -> float32
    return C


def threshold_lengths(C, threshold, min_len) -> np.ndarray:
    """L_thr[b] = number of leading positions with C >= tau (stop at the first
    C < tau), floored at min_len (Guide, "Dynamic Verification Scheduling
    Algorithm", step 3; Deep Dive, "The Full Scheduling Pipeline", 1 <= L)."""
    tau = np.float32(threshold)
    B, K = C.shape
    out = np.empty(B, dtype=np.int32)
    for b in range(B):
        n = 0
        while n < K and C[b, n] >= tau:
            n += 1
        out[b] = max(int(min_len), n)
    return out


def schedule(conf, threshold, budget, min_len=1):
    """Return (lengths int32[B], mask uint8[B,K], survival float32[B,K]).

    With ``budget >= 0`` and sum(L_thr) > budget, every request keeps
    ``min_len`` positions and the remaining ``budget - B*min_len`` slots go to
    the candidates (b, k), min_len < k <= L_thr[b], in order of C descending,
    then b ascending, then k ascending (Deep Dive, "The Optimization Logic":
    a slot goes to the most confident token in the batch).  L[b] is min_len
    plus the number of row-b candidates taken."""
    conf = np.asarray(conf, dtype=np.float32)
    B, K = conf.shape
    C = survival(conf)
    L = threshold_lengths(C, threshold, min_len)
    if budget >= 0 and int(L.sum()) > budget:
        cands = [(b, k) for b in range(B) for k in range(min_len + 1, int(L[b]) + 1)]
        # float comparison: -0.0 and +0.0 are the same key
        cands.sort(key=lambda t: (-float(C[t[0], t[1] - 1]), t[0], t[1]))
        take = budget - B * min_len
        L = np.full(B, min_len, dtype=np.int32)
        for (b, _k) in cands[:take]:
            L[b] += 1
    mask = (np.arange(1, K + 1)[None, :] <= L[:, None]).astype(np.uint8)
    return L.astype(np.int32), mask, C


# ----------------------------------------------------------------------------
# Load-aware threshold and throughput-curve budget
# ----------------------------------------------------------------------------

MAX_CURVE = 64  # curve points the library accepts


def load_factor(q, q_max, m, m_max):
    """Return (LF float32, flags).  LF = 0.6 * Q/Q_max + 0.4 * M/M_max, kept
    in [0, 1] (Guide, "Dynamic Verification Scheduling Algorithm", step 1:
    queue depth Q, GPU memory in use M).

    Readings: the computation is fp32 in this order (the two ratios, the two
    products, the sum), then clamped to [0, 1], which the page states as the
    range; a queue depth or memory figure that is NaN, infinite or negative is
    flagged and read as full load (LF = 1, the conservative end)."""
    f32 = np.float32
    q, m = f32(q), f32(m)
    if not (np.isfinite(q) and np.isfinite(m) and q >= 0 and m >= 0):
        return f32(1.0), DEV_BAD_LOAD
    lf = f32(0.6) * (q / f32(q_max)) + f32(0.4) * (m / f32(m_max))
    return f32(min(max(lf, f32(0.0)), f32(1.0))), 0


def load_threshold(lf, tau_min, tau_max):
    """tau = tau_min + (tau_max - tau_min) * LF^2 (Guide, "Dynamic
    Verification Scheduling Algorithm", step 2; the Guide's code listing has
    the same form with 0.25 and 0.50).  fp32 in this order: the difference,
    the square, their product, the sum.  The pages give tau_min as 0.20 in
    the prose and 0.25 in the code, so both ends are arguments."""
    f32 = np.float32
    lf = f32(lf)
    return f32(f32(tau_min) + (f32(tau_max) - f32(tau_min)) * (lf * lf))


def curve_budget(curve, slot_cost, B, min_len):
    """Return (budget int, flags): the verify-token budget from a throughput
    curve (Deep Dive, "The Throughput Curve": tokens/s measured at a range of
    batch sizes; "The Optimization Logic": keep adding tokens while the
    marginal gain of one more covers its cost).

    ``curve`` is [n, 2]: (x_i tokens per target forward pass, T_i tokens/s),
    x strictly ascending whole numbers >= 1.  Readings: between x_{i-1} and
    x_i every added token gains the segment's slope
    g_i = (T_i - T_{i-1}) / (x_i - x_{i-1}) (fp64); the pass grows up to x_j,
    where segment j+1 is the first whose gain is below ``slot_cost`` (the last
    point if none is); a forward pass carries one position per request that
    is not a drafted token, so the budget on drafted positions is x* - B,
    floored at B * min_len.  No curve (n = 0) means no budget (-1); a curve
    that breaks the rules above is flagged and also means no budget."""
    curve = np.asarray(curve, dtype=np.float32).reshape(-1, 2)
    n = curve.shape[0]
    if n == 0:
        return -1, 0
    x = curve[:, 0].astype(np.float64)
    t = curve[:, 1].astype(np.float64)
    ok = n <= MAX_CURVE and np.all(np.isfinite(x)) and np.all(np.isfinite(t))
    ok = ok and np.all(x >= 1) and np.all(x <= 2.0 ** 24) and np.all(np.floor(x) == x)
    ok = ok and np.all(np.diff(x) > 0)
    if not ok:
        return -1, DEV_BAD_CURVE
    cost = float(np.float32(slot_cost))
    xstar = x[-1]
    for i in range(1, n):
        g = (t[i] - t[i - 1]) / (x[i] - x[i - 1])
        if g < cost:
            xstar = x[i - 1]
            break
    return max(int(B) * int(min_len), int(xstar) - int(B)), 0


def schedule_load_aware(conf, load, q_max, m_max, tau_min, tau_max, curve, slot_cost,
                        min_len=1):
    """The schedule with its threshold and budget set from the load and the
    throughput curve (Deep Dive, "GPU-Resident Scheduling": the scheduler
    reads the confidences and the stored curve and writes one length per
    request).  Returns (lengths, mask, survival, tau, budget, flags)."""
    conf = np.asarray(conf, dtype=np.float32)
    B = conf.shape[0]
    lf, f1 = load_factor(load[0], q_max, load[1], m_max)
    tau = load_threshold(lf, tau_min, tau_max)
    budget, f2 = curve_budget(curve, slot_cost, B, min_len)
    L, mask, C = schedule(conf, tau, budget, min_len)
    return L, mask, C, tau, budget, f1 | f2


# ----------------------------------------------------------------------------
# Markov logit-bias drafting
# ----------------------------------------------------------------------------

def bf16_round(x32) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even; NaN stays
    a quiet NaN."""
    x = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x32, dtype=np.float32))
    r = ((x + 0x7FFF + ((x >> 16) & 1)) >> 16).astype(np.uint16)
    return np.where(nan, np.uint16(0x7FC0), r)


def markov_bias(U64, V64, prev):
    """bias[v] = sum_j U[v, j] * Vm[prev, j] (Guide, the Markov logit-bias
    head: U . V[y_{k-1}]^T), U and Vm already widened to fp64; one matrix-
    vector product.  Products of bf16 values are exact in fp64; the sum is
    exact too whenever the terms are multiples of a common power of two
    within 53 bits of each other, as for the fixed-point test weights."""
    return U64 @ V64[int(prev)]


def markov_draft(base, U, Vm, scale, y0, temperature, uniforms, requests=None):
    """Semi-autoregressive drafting with the Markov logit bias (Guide, the
    Markov logit-bias head and the drafting loop of its code listing).

    base [B, K, V] parallel logits (bf16 as uint16, or float32); U, Vm
    [V, r] bf16 (uint16); scale the listing's scalar on the bias; y0 [B] the
    token before the block (the last target token); temperature [B]; uniforms
    [B, K].  For k = 1..K, in order:
      corrected_k = base_k + scale * U . Vm[y_{k-1}]   stored in the base dtype
      y_k = the inverse-CDF draw at uniforms[b, k-1] from softmax(corrected_k / T)
            (T = 0: the lowest-index maximum)
    Readings: the bias is a sum in fp32 (here its exact value, then one
    rounding; the two agree whenever that sum is exact in fp32, which the
    fixed-point test weights ensure), scaled and added to the widened base
    logit in fp32, and stored rounded to nearest even; the draw uses the
    stored logits, so that the draft distribution is exactly the one the
    verifier reads back; the listing's greedy/top-p choice is read as the
    verifier's own rule: sampling at the request's temperature, greedy at
    T = 0.  Returns (corrected like base, drafted int32[B,K], q float64[B,K],
    boundary float64[B,K]: distance of each draw from a decision edge, inf
    for greedy; q is 1 for greedy draws).  ``requests`` limits the work to
    those rows (the others are left zero)."""
    base = np.asarray(base)
    B, K, V = base.shape
    bf = base.dtype == np.uint16
    f32 = np.float32
    corrected = np.empty_like(base)
    drafted = np.zeros((B, K), dtype=np.int32)
    q = np.zeros((B, K))
    dist = np.full((B, K), np.inf)
    U64, V64 = widen(U), widen(Vm)
    for b in (range(B) if requests is None else requests):
        prev = int(y0[b])
        T = float(np.float32(temperature[b]))
        for k in range(K):
            bias32 = markov_bias(U64, V64, prev).astype(np.float32)
            row32 = widen(base[b, k]).astype(np.float32)
            c32 = (row32 + (f32(scale) * bias32).astype(np.float32)).astype(np.float32)
            stored = bf16_round(c32) if bf else c32
            corrected[b, k] = stored
            x = widen(stored)
            if T == 0.0:
                y = int(np.argmax(x))
                qy = 1.0
            else:
                p = softmax_T(x, T)
                y, d = inverse_cdf(p, float(np.float32(uniforms[b, k])))
                qy = float(p[y])
                dist[b, k] = d
            drafted[b, k] = y
            q[b, k] = qy
            prev = y
    return corrected, drafted, q, dist


# ----------------------------------------------------------------------------
# Online calibration of the confidences
# ----------------------------------------------------------------------------

def calibrate(raw, theta):
    """Return (calibrated float64[B,K], flags): per-position temperature
    scaling, sigmoid(logit(raw[b,k]) / theta[k]) (Deep Dive, "Online
    Calibration", "Sequential Temperature Scaling").  fp64.

    Readings: scores 0 and 1 stay 0 and 1 (logit -inf and +inf); a score that
    is NaN or outside [0, 1] is flagged and passed through unchanged; a
    temperature that is NaN, infinite or not positive is flagged and that
    position is passed through unchanged."""
    raw = np.asarray(raw, dtype=np.float32).astype(np.float64)
    theta = np.asarray(theta, dtype=np.float32).astype(np.float64)
    out = raw.copy()
    flags = 0
    B, K = raw.shape
    for k in range(K):
        t = theta[k]
        if not (np.isfinite(t) and t > 0):
            flags |= DEV_BAD_CONF
            continue
        for b in range(B):
            x = raw[b, k]
            if not (0.0 <= x <= 1.0):
                flags |= DEV_BAD_CONF
                continue
            if x == 0.0 or x == 1.0:
                continue
            z = (math.log(x) - math.log1p(-x)) / t
            out[b, k] = 1.0 / (1.0 + math.exp(-z))
    return out, flags


def evaluated_positions(lengths, accepted, K):
    """The positions whose accept test ran in a round, and their outcomes:
    position k (1-based) of request b ran if k <= lengths[b] and
    k <= accepted[b] + 1 (the test stops at the first rejection; Deep Dive,
    "Speculative Decoding From First Principles"), and was accepted if
    k <= accepted[b].  Returns (ran bool[B,K], ok bool[B,K])."""
    L = np.asarray(lengths).reshape(-1, 1)
    a = np.asarray(accepted).reshape(-1, 1)
    k = np.arange(1, K + 1)[None, :]
    ran = (k <= L) & (k <= a + 1)
    return ran, ran & (k <= a)


class CalibrationWindow:
    """Per-position window statistics and binned calibration counts, updated
    once per round (Deep Dive, "The Calibration Loop in Practice": every N
    rounds, per position, the mean calibrated score and the fraction of
    tokens accepted over the window; temperature[i] += learning_rate *
    (predicted - actual)).

    Readings: the window covers the positions whose accept test ran (see
    ``evaluated_positions``); a position with no such token in the window
    keeps its temperature; temperatures are floored at ``theta_min`` (the
    pages give no bound, and the formula needs a positive temperature); ECE
    is the usual binned expected calibration error over the window's
    (score, outcome) pairs, bins of equal width on [0, 1], a score s in bin
    min(floor(s * n_bins), n_bins - 1)."""

    def __init__(self, K, n_bins=10):
        self.K, self.n_bins = K, n_bins
        self.reset()

    def reset(self):
        K, M = self.K, self.n_bins
        self.rounds = 0
        self.n = np.zeros(K, dtype=np.int64)        # tokens whose test ran
        self.acc = np.zeros(K, dtype=np.int64)      # of them accepted
        self.pred = np.zeros(K, dtype=np.float64)   # sum of their scores
        self.bn = np.zeros(M, dtype=np.int64)
        self.bconf = np.zeros(M, dtype=np.float64)
        self.bacc = np.zeros(M, dtype=np.int64)

    def observe(self, calibrated, lengths, accepted):
        """Add one round; returns the flags: lengths outside [0, K] or
        accepted counts outside [0, length] (then clamped), scores outside
        [0, 1]."""
        c = np.asarray(calibrated, dtype=np.float32).astype(np.float64)
        L = np.asarray(lengths, dtype=np.int64)
        a = np.asarray(accepted, dtype=np.int64)
        flags = 0
        if np.any((L < 0) | (L > self.K) | (a < 0) | (a > L)):
            flags |= DEV_BAD_LENGTH
        L = np.clip(L, 0, self.K)
        a = np.clip(a, 0, L)
        ran, ok = evaluated_positions(L, a, self.K)
        if np.any(ran & ~((c >= 0) & (c <= 1))):
            flags |= DEV_BAD_CONF
        self.n += ran.sum(axis=0)
        self.acc += ok.sum(axis=0)
        for k in range(self.K):
            self.pred[k] += sum(float(c[b, k]) for b in range(c.shape[0]) if ran[b, k])
        for b, k in zip(*np.nonzero(ran)):
            m = min(int(math.floor(c[b, k] * self.n_bins)), self.n_bins - 1)
            self.bn[m] += 1
            self.bconf[m] += c[b, k]
            self.bacc[m] += int(ok[b, k])
        self.rounds += 1
        return flags

    def ece(self):
        N = int(self.bn.sum())
        if N == 0:
            return 0.0
        return float(sum(abs(float(self.bacc[m]) - self.bconf[m]) for m in range(self.n_bins)) / N)

    def update(self, theta, lr, theta_min):
        """The temperature step; returns the new temperatures (float64)."""
        th = np.asarray(theta, dtype=np.float32).astype(np.float64).copy()
        for k in range(self.K):
            if self.n[k] > 0:
                err = self.pred[k] / self.n[k] - self.acc[k] / self.n[k]
                th[k] = max(float(np.float32(theta_min)), th[k] + float(np.float32(lr)) * err)
        return th


def calib_observe(win, theta, calibrated, lengths, accepted, lr, theta_min, window):
    """One round into the window; at the window's end the temperature step,
    the window's ECE and a fresh window.  Returns (theta, ece or None)."""
    win.observe(calibrated, lengths, accepted)
    if win.rounds < window:
        return np.asarray(theta, dtype=np.float64), None
    ece = win.ece()
    th = win.update(theta, lr, theta_min)
    win.reset()
    return th, ece


# ----------------------------------------------------------------------------
# Verification
# ----------------------------------------------------------------------------

def softmax_T(logits64: np.ndarray, T: float) -> np.ndarray:
    """p(v) = exp((l_v - M)/T) / sum_w exp((l_w - M)/T), M = max l, in fp64."""
    M = np.max(logits64)
    e = np.exp((logits64 - M) / T)
    return e / np.sum(e)


def inverse_cdf(mass: np.ndarray, u: float):
    """First token id whose cumulative mass exceeds u * Z, Z = total mass.

    Returns (token, distance) where distance = min(|u - F(t-1)|, |u - F(t)|)
    on the normalised CDF F (F(-1) = 0).  If rounding leaves no qualifying id,
    the last id with positive mass is returned."""
    cdf = np.cumsum(mass)
    Z = cdf[-1]
    hit = np.nonzero(cdf > u * Z)[0]
    if hit.size:
        t = int(hit[0])
    else:
        t = int(np.nonzero(mass > 0)[0][-1])
    F_t = cdf[t] / Z
    F_prev = cdf[t - 1] / Z if t > 0 else 0.0
    return t, min(abs(u - F_prev), abs(u - F_t))


def _row_flags(row64) -> int:
    """A row that is read must hold no NaN and no +Inf, and at least one
    finite logit (-Inf alone is a legal, masked logit)."""
    bad = np.isnan(row64).any() or np.isposinf(row64).any() or not np.isfinite(row64).any()
    return DEV_NONFINITE if bad else 0


def verify_request(target_b, draft_b, drafted_b, L, T, u_b):
    """Verify one request.

    target_b [K+1, V], draft_b [K, V] (raw arrays), drafted_b [K], L in 0..K,
    T float32 value, u_b [K+1].  Returns a dict with accepted, tokens [K+1],
    p_tok [K], q_tok [K], dist (smallest distance of any evaluated decision to
    its edge; inf when nothing was drawn), flags."""
    K = target_b.shape[0] - 1
    V = target_b.shape[1]
    T = float(np.float32(T))
    tokens = np.full(K + 1, -1, dtype=np.int32)
    p_tok = np.zeros(K, dtype=np.float64)
    q_tok = np.zeros(K, dtype=np.float64)
    flags = 0
    y = [int(v) for v in drafted_b[:L]]
    if any(v < 0 or v >= V for v in y):
        flags |= DEV_BAD_TOKEN
    if not (T >= 0.0):                        # negative or NaN: nothing is read
        return dict(accepted=0, tokens=tokens, p_tok=p_tok, q_tok=q_tok,
                    dist=np.inf, flags=flags | DEV_BAD_TEMP)
    # every row that the rule reads is checked, whatever the drafted ids are
    n_target = L + 1
    n_draft = L if T > 0.0 else 0
    for j in range(n_target):
        flags |= _row_flags(widen(target_b[j]))
    for j in range(n_draft):
        flags |= _row_flags(widen(draft_b[j]))
    if flags & (DEV_BAD_TOKEN | DEV_NONFINITE):
        # outputs of a flagged request are unspecified
        return dict(accepted=0, tokens=tokens, p_tok=p_tok, q_tok=q_tok,
                    dist=np.inf, flags=flags)

    if T == 0.0:
        # greedy rule (T = 0): accept y_k iff it is the lowest-index argmax of
        # target row k-1; emit the argmax at the first mismatch (or row L).
        g = []
        for j in range(L + 1):
            row = widen(target_b[j])
            g.append(int(np.argmax(row)))      # first maximal index
        a = L
        for k in range(1, L + 1):
            if y[k - 1] != g[k - 1]:
                a = k - 1
                break
        tokens[:a] = y[:a]
        tokens[a] = g[a]
        return dict(accepted=a, tokens=tokens, p_tok=p_tok, q_tok=q_tok,
                    dist=np.inf, flags=flags)

    u = np.asarray(u_b, dtype=np.float32).astype(np.float64)
    used_u = list(range(L)) + [K]
    if any(not (0.0 <= u[i] < 1.0) for i in used_u):
        flags |= DEV_BAD_UNIFORM

    # temperature softmaxes of every scheduled row (Deep Dive, "Speculative
    # Decoding From First Principles"; both distributions at the request's T)
    P = [softmax_T(widen(target_b[j]), T) for j in range(L + 1)]
    Q = [softmax_T(widen(draft_b[j]), T) for j in range(L)]

    alpha = np.zeros(L)
    for k in range(1, L + 1):
        py = P[k - 1][y[k - 1]]
        qy = Q[k - 1][y[k - 1]]
        p_tok[k - 1] = py
        q_tok[k - 1] = qy
        # alpha_k = min(1, p/q) (Guide, "1. The Mathematics of Suffix Decay")
        if py == 0.0:
            alpha[k - 1] = 0.0
        elif qy == 0.0:
            alpha[k - 1] = 1.0
        else:
            alpha[k - 1] = min(1.0, py / qy)

    # first rejection: accept position k iff u[k-1] < alpha_k
    a = L
    for k in range(1, L + 1):
        if not (u[k - 1] < alpha[k - 1]):
            a = k - 1
            break
    dist = np.inf
    for k in range(1, min(a + 1, L) + 1):
        dist = min(dist, abs(u[k - 1] - alpha[k - 1]))

    if a < L:
        # residual max(0, p - q) at the rejected position, normalised;
        # an all-zero residual falls back to p
        r = np.maximum(0.0, P[a] - Q[a])
        mass = r if np.sum(r) > 0.0 else P[a]
    else:
        # full acceptance: bonus token from the row after the last draft
        mass = P[L]
    t, d = inverse_cdf(mass, u[K])
    dist = min(dist, d)
    tokens[:a] = y[:a]
    tokens[a] = t
    return dict(accepted=a, tokens=tokens, p_tok=p_tok, q_tok=q_tok, dist=dist,
                flags=flags)


def verify(target, draft, drafted, lengths, temperature, uniforms, requests=None):
    """Batched verification.  ``lengths=None`` verifies all K positions.
    ``requests`` restricts the work to a subset of request indices (the other
    rows of the outputs stay at their fill values).

    Returns dict(accepted int32[B], tokens int32[B,K+1], p_tok float64[B,K],
    q_tok float64[B,K], dist float64[B], flags int (OR over requests),
    req_flags int32[B]).  Outputs of a request with flags are unspecified."""
    B, K1, V = target.shape
    K = K1 - 1
    accepted = np.zeros(B, dtype=np.int32)
    tokens = np.full((B, K + 1), -1, dtype=np.int32)
    p_tok = np.zeros((B, K))
    q_tok = np.zeros((B, K))
    dist = np.full(B, np.inf)
    req_flags = np.zeros(B, dtype=np.int32)
    flags = 0
    idx = range(B) if requests is None else requests
    for b in idx:
        L = K if lengths is None else int(lengths[b])
        r = verify_request(target[b], draft[b], drafted[b], L, temperature[b], uniforms[b])
        accepted[b] = r["accepted"]
        tokens[b] = r["tokens"]
        p_tok[b] = r["p_tok"]
        q_tok[b] = r["q_tok"]
        dist[b] = r["dist"]
        req_flags[b] = r["flags"]
        flags |= r["flags"]
    return dict(accepted=accepted, tokens=tokens, p_tok=p_tok, q_tok=q_tok,
                dist=dist, flags=flags, req_flags=req_flags)


def verify_greedy(target, drafted, lengths, requests=None):
    """Greedy (T = 0) verification of every request: returns
    dict(accepted, tokens, flags)."""
    B, K1, V = target.shape
    K = K1 - 1
    temp = np.zeros(B, dtype=np.float32)
    u = np.zeros((B, K + 1), dtype=np.float32)
    # at T = 0 the draft rows are never read; pass the target rows as a stand-in
    r = verify(target, target[:, :K], drafted, lengths, temp, u, requests=requests)
    return dict(accepted=r["accepted"], tokens=r["tokens"], flags=r["flags"])
