"""Plain fp64 CPU oracle for the CONF-KV decode step.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the tests, the package smoke check and the
benchmark's CPU-baseline leg use it. It shares no code with the HIP library;
its inputs come from the seeded generators in ``synth`` or from a snapshot of
device state, never from the HIP path's own arithmetic.

Sources (the pages describing CONF-KV, cited by page and section):
  [S]  "CONF-KV: Confidence-Aware KV Cache Eviction with Mixed-Precision
       Storage for Long-Horizon LLM", gist.science technical summary,
       section "Methodik: CONF-KV" (confidence score, budget gate, ranking,
       protected window, mixed-precision storage, compact layout).
  [R1] Same paper, paper.rainbus.top structured review, section "前置知识"
       (prerequisites): blockwise online softmax is exact; the EMA rule
       a_i <- lambda*a_i + (1-lambda)*Abar_i with lambda = 0.9.
  [R2] Same review, section "核心方法" (core method): H^ = H(p)/log V,
       m = log p(1) - log p(2), weights (0.4, 0.3, 0.3), c >= tau picks
       N_high, rank s_i = alpha*a^_i + (1-alpha)*r^_i, alpha = 0.65,
       newest P tokens always protected.
  [R3] Same review, section "方法步骤详情" (method step details,
       Algorithm 1): forward -> confidence -> budget -> per layer: EMA
       update, evict lowest-ranked unprotected tokens if |C_l| > N,
       compact survivors, quantise retained tokens outside the newest W to
       INT8 -> append the new K/V in FP16.
  [R4] Same review, section "复现评估" (reproduction): tau = 0.7,
       P = 32, alpha = 0.65, W = 128, block B = 128.

Where the pages are silent the oracle takes one reading; every reading is
named in a comment as "Reading:" and listed with the design notes.

Precision: everything is fp64 except the INT8 quantiser, whose scale and
quotient are IEEE fp32 by definition of the stored format (reading R16).
"""
from dataclasses import dataclass, field
import math

import numpy as np

# ---------------------------------------------------------------------------
# Confidence and budget  ([S] Konfidenzschaetzung; [R2]; [R3] steps 3-4)
# ---------------------------------------------------------------------------

STATUS_NONFINITE_LOGITS = 1


def confidence(logits, w_h=0.4, w_m=0.3, w_p=0.3):
    """Scalar confidence c = w_H(1 - H^) + w_m*sigmoid(m) + w_p*p(1) of one logit row.

    p = softmax(logits); H^ = H(p)/ln V (natural log; the base cancels);
    m = ln p(1) - ln p(2) for the two largest probabilities of the multiset
    (a duplicated maximum gives m = 0); p(1) the largest probability.
    Reading: -inf logits are allowed (probability 0, 0*ln 0 = 0); NaN, +inf,
    all -inf or V < 2 give c = NaN and the non-finite status bit.
    Returns (c, status, parts) with parts = dict(H_hat, m, sig, p1).
    """
    z = np.asarray(logits, dtype=np.float64)
    V = z.shape[0]
    if V < 2 or np.isnan(z).any() or np.isposinf(z).any() or np.isneginf(z).all():
        return float("nan"), STATUS_NONFINITE_LOGITS, None
    M = z.max()
    e = np.exp(z - M)
    S = e.sum()
    p = e / S
    nz = p > 0
    H = -np.sum(p[nz] * np.log(p[nz]))
    H_hat = H / math.log(V)
    top = np.sort(z)[::-1][:2]
    m = top[0] - top[1]            # ln p(1) - ln p(2); +inf when p(2) = 0
    sig = 1.0 / (1.0 + math.exp(-m)) if np.isfinite(m) else 1.0
    p1 = p.max()
    c = w_h * (1.0 - H_hat) + w_m * sig + w_p * p1
    return float(c), 0, dict(H_hat=float(H_hat), m=float(m), sig=float(sig), p1=float(p1))


def next_token(logits, temperature=0.0, u=0.0):
    """Next token x_{t+1} (review Algorithm 1, step 13).

    temperature 0: greedy, the smallest index among the largest logits.
    temperature > 0: sampling from softmax(z / temperature) by inversion with
    the uniform draw u in [0, 1): the smallest index i (index order) whose
    cumulative probability sum_{j<=i} p_j exceeds u. Reading: the pages name
    the sampling step without fixing a rule; inversion in index order with a
    caller-supplied uniform is the plain reading that makes the draw
    reproducible. Returns -1 for flagged rows (as the confidence does).
    """
    z = np.asarray(logits, dtype=np.float64)
    if z.shape[0] < 2 or np.isnan(z).any() or np.isposinf(z).any() or np.isneginf(z).all():
        return -1
    if temperature == 0:
        return int(np.flatnonzero(z == z.max())[0])
    w = np.exp((z - z.max()) / temperature)
    cdf = np.cumsum(w / w.sum())
    return int(min(np.searchsorted(cdf, u, side="right"), z.shape[0] - 1))


def token_interval(logits, temperature, i):
    """Cumulative probability before and through token i under
    softmax(z / temperature): a draw u picks i exactly when lo <= u < hi."""
    z = np.asarray(logits, dtype=np.float64)
    w = np.exp((z - z.max()) / temperature)
    p = w / w.sum()
    return float(p[:i].sum()), float(p[: i + 1].sum())


def budget(c, tau, n_high, n_low):
    """Tight budget N_high when c >= tau (confident), loose N_low otherwise ([S]; [R2]).

    Reading: a NaN confidence (flagged logits) takes the loose budget.
    """
    return int(n_high) if (c == c and c >= tau) else int(n_low)


# ---------------------------------------------------------------------------
# Per-(layer, sequence) cache state
# ---------------------------------------------------------------------------

@dataclass
class SeqCache:
    """Retained tokens of one (layer, sequence), in slot order: the INT8
    entries first, then the FP16 ones in ascending position (the INT8 part is
    in ascending position too unless compact(..., fill=True) reordered it).

    Each token is either FP16 (k16/v16 hold its values) or INT8 (k8/v8 hold
    its codes, dequantised with the per-(kv-head, channel) scales ks/vs).
    """
    pos: np.ndarray            # int64 [n]
    is8: np.ndarray            # bool [n]
    k16: np.ndarray            # float16 [n, Hkv, d]
    v16: np.ndarray
    k8: np.ndarray             # int8 [n, Hkv, d]
    v8: np.ndarray
    ema: np.ndarray            # float64 [n]
    ks: np.ndarray             # float32 [Hkv, d]
    vs: np.ndarray
    calibrated: bool = False
    saturated: int = 0         # codes clamped at +-127 so far

    @property
    def n(self):
        return int(self.pos.shape[0])

    def copy(self):
        return SeqCache(self.pos.copy(), self.is8.copy(), self.k16.copy(), self.v16.copy(),
                        self.k8.copy(), self.v8.copy(), self.ema.copy(), self.ks.copy(),
                        self.vs.copy(), self.calibrated, self.saturated)


def empty_cache(hkv, d):
    return SeqCache(np.zeros(0, np.int64), np.zeros(0, bool),
                    np.zeros((0, hkv, d), np.float16), np.zeros((0, hkv, d), np.float16),
                    np.zeros((0, hkv, d), np.int8), np.zeros((0, hkv, d), np.int8),
                    np.zeros(0, np.float64), np.zeros((hkv, d), np.float32),
                    np.zeros((hkv, d), np.float32), False, 0)


def dequant_rows(cache):
    """fp64 K^ and V^ [n, Hkv, d]: FP16 values as stored, INT8 codes times their scale."""
    k = cache.k16.astype(np.float64)
    v = cache.v16.astype(np.float64)
    k8 = cache.k8.astype(np.float64) * cache.ks.astype(np.float64)[None]
    v8 = cache.v8.astype(np.float64) * cache.vs.astype(np.float64)[None]
    m = cache.is8[:, None, None]
    return np.where(m, k8, k), np.where(m, v8, v)


# ---------------------------------------------------------------------------
# Attention and per-key mass  ([R1] blockwise online softmax is exact;
# [R3] steps 1-2; [S] Implementierung: dequantisation fused into block reads)
# ---------------------------------------------------------------------------

def attention(q, cache, k_new, v_new):
    """Decode attention of one (layer, sequence) over C plus the new token.

    q [Hq, d]; k_new, v_new [Hkv, d]. Query head h reads kv head h // (Hq/Hkv).
    Reading: scale 1/sqrt(d), no mask, the new token attends to itself.
    The blockwise recurrence of the kernel is exact, so the oracle uses the
    naive full softmax. Returns o [Hq, d] and the per-key mass
    Abar [n+1] = mean over query heads of the softmax rows (index n is the
    new token); reading: the attention mass of a token is that head-mean.
    """
    q = np.asarray(q, np.float64)
    Hq, d = q.shape
    kh, vh = dequant_rows(cache)
    K = np.concatenate([kh, np.asarray(k_new, np.float64)[None]], axis=0)   # [n+1, Hkv, d]
    Vv = np.concatenate([vh, np.asarray(v_new, np.float64)[None]], axis=0)
    Hkv = K.shape[1]
    g = Hq // Hkv
    o = np.zeros((Hq, d))
    mass = np.zeros(K.shape[0])
    for h in range(Hq):
        j = h // g
        u = K[:, j, :] @ q[h] / math.sqrt(d)
        e = np.exp(u - u.max())
        P = e / e.sum()
        o[h] = P @ Vv[:, j, :]
        mass += P
    return o, mass / Hq


# ---------------------------------------------------------------------------
# EMA metadata and rank score  ([R1] EMA; [R2] s_i)
# ---------------------------------------------------------------------------

def ema_update(ema, mass, lam):
    """a_i <- lam*a_i + (1-lam)*Abar_i for the cached tokens; the new token
    starts from a zero prior under the same rule (reading R8).
    Returns (a' [n], a_new)."""
    ema = np.asarray(ema, np.float64)
    n = ema.shape[0]
    a = lam * ema + (1.0 - lam) * mass[:n]
    return a, (1.0 - lam) * mass[n]


def rank_scores(a, pos, alpha):
    """s_i = alpha*a^_i + (1-alpha)*r^_i over the cached tokens.

    Reading: a^ = a / max a (0 when the max is 0); r^ is the min-max
    normalised position over the cached tokens (1 when only one token).
    """
    a = np.asarray(a, np.float64)
    pos = np.asarray(pos, np.float64)
    if a.shape[0] == 0:
        return np.zeros(0)
    amax = a.max()
    ah = a / amax if amax > 0 else np.zeros_like(a)
    lo, hi = pos.min(), pos.max()
    rh = (pos - lo) / (hi - lo) if hi > lo else np.ones_like(pos)
    return alpha * ah + (1.0 - alpha) * rh


# ---------------------------------------------------------------------------
# Eviction and compaction  ([S] Token-Ranking und Eviktion; [R3] steps 5-11)
# ---------------------------------------------------------------------------

def select_keep(s, pos, N, P, block=0):
    """Keep mask after budget eviction of one (layer, sequence).

    If n <= N nothing is evicted. Otherwise exactly k = n - N tokens are
    evicted: those with the smallest (s, pos) among all tokens except the P
    newest positions, which are always kept. Reading: equal scores evict the
    older token first.

    block = B > 0 is the coarse variant that the review's sections on
    limitations ("局限与改进", "独立分析的弱点") name for paged layouts:
    whole blocks of B position-consecutive candidates leave. Reading: the
    candidates are cut into blocks from the oldest, a trailing partial block
    stays, a block's score is the largest score among its tokens, and
    min(full blocks, ceil(k / B)) blocks with the smallest (block score,
    block order) leave, so the kept count may fall below N by less than B
    (or stay above it when too few full blocks exist).
    """
    n = len(s)
    if N < P:
        raise ValueError("budget below the protected window")
    if block < 0:
        raise ValueError("negative block size")
    keep = np.ones(n, dtype=bool)
    if n <= N:
        return keep
    k = n - N
    order_by_pos = np.argsort(pos, kind="stable")
    cand = order_by_pos[: max(0, n - P)]
    if block > 0:
        blocks = [cand[j * block:(j + 1) * block] for j in range(len(cand) // block)]
        kb = min(len(blocks), -(-k // block))
        ranked = sorted(range(len(blocks)),
                        key=lambda j: (max(float(s[i]) for i in blocks[j]), j))
        for j in ranked[:kb]:
            keep[blocks[j]] = False
        return keep
    key = sorted(cand.tolist(), key=lambda i: (float(s[i]), int(pos[i])))
    keep[np.asarray(key[:k], dtype=np.int64)] = False
    return keep


def compact(cache, keep, fill=False):
    """Survivors packed densely; the INT8 entries stay ahead of the FP16 ones.

    The pages ask for a contiguous layout without indirection tables; the
    default, fill=False, is the stable gather: survivors keep slot order, so
    a cache in position order stays in position order. fill=True (reading
    R24, the hole-filling option of token eviction): in the INT8 part, the
    survivors that lie at
    or beyond its new end m take the holes below m, the j-th such survivor
    (in slot order) the j-th hole; every other survivor keeps its slot. The
    FP16 part is always stable, so it stays in position order.
    """
    keep = np.asarray(keep, bool)
    n8 = int(cache.is8.sum())
    assert cache.is8[:n8].all() and not cache.is8[n8:].any(), "INT8 entries first"
    if fill:
        k8 = keep[:n8]
        m = int(k8.sum())
        order8 = np.arange(m)
        holes = np.flatnonzero(~k8[:m])
        tails = m + np.flatnonzero(k8[m:])
        assert len(holes) == len(tails)
        order8[holes] = tails
        idx = np.concatenate([order8, n8 + np.flatnonzero(keep[n8:])]).astype(np.int64)
    else:
        idx = np.flatnonzero(keep)
    c = cache.copy()
    for name in ("pos", "is8", "k16", "v16", "k8", "v8", "ema"):
        setattr(c, name, getattr(cache, name)[idx].copy())
    return c


def append(cache, k_new, v_new, t, a_new):
    """Add token t at the end as FP16 with EMA a_new ([R3] step 13)."""
    c = cache.copy()
    Hkv, d = np.asarray(k_new).shape
    c.pos = np.append(cache.pos, np.int64(t))
    c.is8 = np.append(cache.is8, False)
    c.k16 = np.concatenate([cache.k16, np.asarray(k_new, np.float16)[None]])
    c.v16 = np.concatenate([cache.v16, np.asarray(v_new, np.float16)[None]])
    c.k8 = np.concatenate([cache.k8, np.zeros((1, Hkv, d), np.int8)])
    c.v8 = np.concatenate([cache.v8, np.zeros((1, Hkv, d), np.int8)])
    c.ema = np.append(cache.ema, float(a_new))
    return c


# ---------------------------------------------------------------------------
# INT8 storage  ([S] gemischte Praezisionsspeicherung: newest W tokens FP16,
# older retained tokens INT8 per head and per channel; [R3] step 10)
# ---------------------------------------------------------------------------

def absmax_scale(x):
    """Per-(kv-head, channel) symmetric scale of rows x [m, Hkv, d].

    Reading R16: scale = fp32(absmax) / 127 with the IEEE fp32 quotient.
    """
    amax = np.abs(np.asarray(x, np.float32)).max(axis=0)
    return (amax.astype(np.float32) / np.float32(127.0)).astype(np.float32)


def quantize_rows(x, scale):
    """INT8 codes of rows x [m, Hkv, d] (fp16) under scale [Hkv, d].

    code = clamp(round_half_even(fp32(x) / scale), -127, 127), the quotient
    being the IEEE fp32 one; a zero scale gives code 0.
    Returns (codes int8, number of clamped elements).
    """
    xf = np.asarray(x, np.float32)
    s = np.broadcast_to(np.asarray(scale, np.float32), xf.shape)
    with np.errstate(divide="ignore", invalid="ignore"):
        qf = np.where(s > 0, xf / np.where(s > 0, s, np.float32(1)), np.float32(0)).astype(np.float32)
    r = np.rint(qf)
    sat = int(np.count_nonzero(np.abs(r) > 127))
    return np.clip(r, -127, 127).astype(np.int8), sat


def calibrate(cache):
    """Reading R17: scales are set once per (layer, sequence, K|V, kv-head,
    channel) when the INT8 region is first populated, over every token then
    in the cache (all FP16 at that moment), and frozen afterwards."""
    c = cache.copy()
    if cache.n > 0:
        c.ks = absmax_scale(cache.k16.astype(np.float32))
        c.vs = absmax_scale(cache.v16.astype(np.float32))
    c.calibrated = True
    return c


def quantize_window(cache, t, W):
    """Move retained FP16 tokens that left the FP16 window to INT8.

    Reading R15: after step t the FP16 window is positions t-W+1 .. t, so
    every FP16 token with pos <= t - W is quantised (at most one per step in
    steady state, exactly once per token).
    """
    c = cache
    move = (~c.is8) & (c.pos <= t - W)
    if not move.any():
        return c
    if not c.calibrated:
        c = calibrate(c)
    c = c.copy()
    idx = np.flatnonzero(move)
    k8, sk = quantize_rows(c.k16[idx], c.ks)
    v8, sv = quantize_rows(c.v16[idx], c.vs)
    c.k8[idx], c.v8[idx] = k8, v8
    c.k16[idx] = 0
    c.v16[idx] = 0
    c.is8[idx] = True
    c.saturated += sk + sv
    return c


def prefill(k, v, W):
    """Cache after a prefill of L0 tokens: positions 0..L0-1, EMA 0, scales
    calibrated over all L0 tokens when any token is older than the window,
    INT8 for pos <= L0-1-W and FP16 for the newest W (readings R17, R15).

    k, v: [Hkv, L0, d] fp16 for one (layer, sequence).
    """
    k = np.asarray(k, np.float16).transpose(1, 0, 2)
    v = np.asarray(v, np.float16).transpose(1, 0, 2)
    L0, Hkv, d = k.shape
    c = empty_cache(Hkv, d)
    c.pos = np.arange(L0, dtype=np.int64)
    c.is8 = np.zeros(L0, bool)
    c.k16, c.v16 = k.copy(), v.copy()
    c.k8 = np.zeros((L0, Hkv, d), np.int8)
    c.v8 = np.zeros((L0, Hkv, d), np.int8)
    c.ema = np.zeros(L0)
    return quantize_window(c, L0 - 1, W)


# ---------------------------------------------------------------------------
# One decode step  ([R3] Algorithm 1)
# ---------------------------------------------------------------------------

@dataclass
class StepOut:
    c: np.ndarray              # [B]
    status: np.ndarray         # [B]
    budget: np.ndarray         # [L, B]
    o: np.ndarray              # [L, B, Hq, d]
    mass: list                 # [L][B] -> [n+1]
    ema: list                  # [L][B] -> [n] updated EMA of the cached tokens
    a_new: np.ndarray          # [L, B]
    score: list                # [L][B] -> [n]
    keep: list                 # [L][B] -> bool [n]
    caches: list               # [L][B] -> SeqCache after the step


def step_one(cache, q, k_new, v_new, t, pol, N, score_given=None):
    """Steps 1-2 and 5-13 of Algorithm 1 for one (layer, sequence) with budget N.

    Returns dict(o, mass, ema, a_new, score, keep, cache) where ema is the
    updated EMA of the cached tokens and cache the state after the step.
    Order (reading R18): attention over C plus the new token; EMA update;
    rank; evict and compact; append the new token; quantise tokens that left
    the FP16 window. score_given replaces the computed scores in the
    selection (lock-step comparison on identical inputs).
    """
    o, m = attention(q, cache, k_new, v_new)
    a, a_new = ema_update(cache.ema, m, pol.lam)
    s = rank_scores(a, cache.pos, pol.alpha)
    s_sel = s if score_given is None else np.asarray(score_given, np.float64)
    kp = select_keep(s_sel, cache.pos, N, pol.protect, getattr(pol, "block", 0))
    c1 = cache.copy()
    c1.ema = a
    # Survivors keep position order (the review's Algorithm 1 compacts the
    # survivors of C_l; the summary's "Implementierung" asks for a dense layout
    # without indirection tables). Reading R24: order 1 is the hole-filling
    # option of token eviction; block eviction always packs stably.
    fill = getattr(pol, "block", 0) == 0 and getattr(pol, "order", 0) == 1
    c1 = compact(c1, kp, fill=fill)
    c1 = append(c1, k_new, v_new, t, a_new)
    c1 = quantize_window(c1, t, pol.window)
    return dict(o=o, mass=m, ema=a, a_new=a_new, score=s, keep=kp, cache=c1)


def step(caches, logits, q, k_new, v_new, t, pol, layer_budgets=None,
         c_given=None, score_given=None):
    """One CONF-KV decode step over every (layer, sequence).

    caches[l][b]: SeqCache before the step; logits [B, V]; q [L, B, Hq, d];
    k_new/v_new [L, B, Hkv, d]; t: position of the new token; pol: policy
    with tau, alpha, lam, w_h, w_m, w_p, n_high, n_low, protect, window.
    layer_budgets: optional (n_low[L], n_high[L]) for per-layer budgets.

    Lock-step hooks: c_given [B] replaces the computed confidence in the
    budget decision and score_given[l][b] replaces the computed scores in the
    selection (so that integer decisions are compared on identical inputs).
    """
    L, B = len(caches), len(caches[0])
    cs = np.zeros(B)
    st = np.zeros(B, np.int64)
    for b in range(B):
        cs[b], st[b], _ = confidence(logits[b], pol.w_h, pol.w_m, pol.w_p)
    cdec = cs if c_given is None else np.asarray(c_given, np.float64)
    budgets = np.zeros((L, B), np.int64)
    o = np.zeros(q.shape, np.float64)
    mass, ema, score, keep, new = [], [], [], [], []
    a_news = np.zeros((L, B))
    for l in range(L):
        nh, nl = pol.n_high, pol.n_low
        if layer_budgets is not None:
            nl, nh = layer_budgets[0][l], layer_budgets[1][l]
        row = [[], [], [], [], []]
        for b in range(B):
            N = budget(cdec[b], pol.tau, nh, nl)
            budgets[l, b] = N
            sg = None if score_given is None else score_given[l][b]
            r = step_one(caches[l][b], q[l, b], k_new[l, b], v_new[l, b], t, pol, N, sg)
            o[l, b] = r["o"]
            a_news[l, b] = r["a_new"]
            for lst, key in zip(row, ("mass", "ema", "score", "keep", "cache")):
                lst.append(r[key])
        mass.append(row[0]); ema.append(row[1]); score.append(row[2]); keep.append(row[3]); new.append(row[4])
    return StepOut(cs, st, budgets, o, mass, ema, a_news, score, keep, new)
