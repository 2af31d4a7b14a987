"""Pins of the fp64 oracle against what the pages and mathematics fix.

Every test here runs on the CPU. Expected values come from closed forms,
invariants, brute force on tiny inputs, or independent library routines
(scipy entropy/softmax, torch scaled-dot-product attention), never from the
oracle's own formula re-typed.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

from oracle import confk_oracle as O
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- confidence

@pytest.mark.parametrize("V", [2, 7, 50257, 152064])
def test_confidence_uniform_closed_form(V):
    # uniform p: H^ = 1, m = 0 (sigma = 1/2), p(1) = 1/V
    c, st, _ = O.confidence(np.full(V, 3.25, np.float32))
    assert st == 0
    assert abs(c - (0.15 + 0.3 / V)) < 1e-13


@pytest.mark.parametrize("V", [2, 1000, 50257])
def test_confidence_one_hot_is_one(V):
    z = np.full(V, -np.inf, np.float32)
    z[V // 3] = 1.5
    c, st, parts = O.confidence(z)
    assert st == 0 and c == 1.0
    assert parts["H_hat"] == 0.0 and parts["sig"] == 1.0 and parts["p1"] == 1.0


@pytest.mark.parametrize("k,V", [(2, 10), (3, 50257), (7, 152064)])
def test_confidence_k_way_tie_closed_form(k, V):
    # k equal maxima, rest -inf: H = ln k, m = 0, p(1) = 1/k
    z = np.full(V, -np.inf, np.float32)
    z[np.arange(k) * 5] = 0.75
    c, _, _ = O.confidence(z)
    want = 0.4 * (1 - math.log(k) / math.log(V)) + 0.3 * 0.5 + 0.3 / k
    assert abs(c - want) < 1e-13


@pytest.mark.parametrize("a", [0.1, 1.0, 4.0, 20.0])
def test_confidence_two_level_closed_form(a):
    # one logit a, V-1 logits 0: p1 = e^a/(e^a+V-1), rest (1-p1)/(V-1), margin m = a
    V = 1000
    z = np.zeros(V, np.float64)
    z[17] = a
    p1 = math.exp(a) / (math.exp(a) + V - 1)
    pr = (1 - p1) / (V - 1)
    H = -p1 * math.log(p1) - (V - 1) * pr * math.log(pr)
    want = 0.4 * (1 - H / math.log(V)) + 0.3 / (1 + math.exp(-a)) + 0.3 * p1
    c, _, parts = O.confidence(z)
    assert abs(c - want) < 1e-12
    assert abs(parts["m"] - a) < 1e-12


def test_confidence_against_scipy():
    rng = np.random.default_rng(5)
    for s in (0.5, 2.0, 8.0):
        z = (rng.standard_normal(4096) * s).astype(np.float32)
        p = scipy.special.softmax(z.astype(np.float64))
        H = scipy.stats.entropy(p)
        ps = np.sort(p)[::-1]
        m = math.log(ps[0]) - math.log(ps[1])
        want = 0.4 * (1 - H / math.log(4096)) + 0.3 * scipy.special.expit(m) + 0.3 * ps[0]
        c, _, _ = O.confidence(z)
        assert abs(c - want) < 1e-12


def test_confidence_shift_and_permutation_invariant():
    rng = np.random.default_rng(6)
    z = rng.standard_normal(999) * 3
    c0, _, _ = O.confidence(z)
    c1, _, _ = O.confidence(z + 123.0)
    c2, _, _ = O.confidence(rng.permutation(z))
    assert abs(c0 - c1) < 1e-12 and abs(c0 - c2) < 1e-12


def test_confidence_duplicate_max_gives_zero_margin():
    z = np.array([2.0, 5.0, 5.0, 1.0])
    _, _, parts = O.confidence(z)
    assert parts["m"] == 0.0 and parts["sig"] == 0.5


@pytest.mark.parametrize("bad", [np.nan, np.inf])
def test_confidence_flags_nonfinite(bad):
    z = np.zeros(10)
    z[3] = bad
    c, st, _ = O.confidence(z)
    assert st == O.STATUS_NONFINITE_LOGITS and c != c
    assert O.budget(c, 0.7, 256, 512) == 512


def test_confidence_flags_all_neg_inf_and_short_vocab():
    assert O.confidence(np.full(5, -np.inf))[1] == O.STATUS_NONFINITE_LOGITS
    assert O.confidence(np.zeros(1))[1] == O.STATUS_NONFINITE_LOGITS


def test_budget_gate_inclusive():
    assert O.budget(0.7, 0.7, 100, 200) == 100          # c >= tau is confident
    assert O.budget(np.nextafter(0.7, 0), 0.7, 100, 200) == 200
    # tau <= min c -> always tight; tau > 1 -> always loose (c <= 1)
    assert O.budget(0.150001, 0.15, 1, 2) == 1
    assert O.budget(1.0, 1.0000001, 1, 2) == 2


def test_pages_hyperparameters_match_defaults():
    g = json.load(open(os.path.join(GOLD, "pages_hyperparameters.json")))
    p = synth.Policy()
    assert [p.w_h, p.w_m, p.w_p] == g["confidence_weights"]["value"]
    assert p.tau == g["tau"]["value"] and p.alpha == g["alpha"]["value"] and p.lam == g["lambda"]["value"]
    # the oracle's default weights are the pages' weights
    z = np.array([0.0, 1.0, 3.0])
    assert O.confidence(z)[0] == O.confidence(z, *g["confidence_weights"]["value"])[0]


# ------------------------------------------------------------------ attention

def _cache_from_fp16(k, v):
    """SeqCache of FP16 tokens; k, v [n, Hkv, d]."""
    n, H, d = k.shape
    c = O.empty_cache(H, d)
    c.pos = np.arange(n, dtype=np.int64)
    c.is8 = np.zeros(n, bool)
    c.k16, c.v16 = k.astype(np.float16), v.astype(np.float16)
    c.k8 = np.zeros((n, H, d), np.int8)
    c.v8 = np.zeros((n, H, d), np.int8)
    c.ema = np.zeros(n)
    return c


def test_attention_single_token_returns_its_value():
    H, d = 3, 8
    rng = np.random.default_rng(1)
    c = O.empty_cache(H, d)
    q = rng.standard_normal((6, d)).astype(np.float16)
    kn = rng.standard_normal((H, d)).astype(np.float16)
    vn = rng.standard_normal((H, d)).astype(np.float16)
    o, mass = O.attention(q, c, kn, vn)
    assert np.array_equal(mass, [1.0])
    for h in range(6):
        assert np.allclose(o[h], vn[h // 2].astype(np.float64), atol=0, rtol=0)


def test_attention_equal_keys_average_values():
    H, d, n = 2, 16, 9
    rng = np.random.default_rng(2)
    k = np.repeat(rng.standard_normal((1, H, d)), n, 0)
    v = rng.standard_normal((n, H, d))
    c = _cache_from_fp16(k, v)
    q = rng.standard_normal((4, d)).astype(np.float16)
    o, mass = O.attention(q, c, k[0].astype(np.float16), v[0].astype(np.float16))
    allv = np.concatenate([c.v16.astype(np.float64), v[:1].astype(np.float16).astype(np.float64)])
    for h in range(4):
        assert np.allclose(o[h], allv[:, h // 2].mean(0), atol=1e-14)
    assert np.allclose(mass, 1.0 / (n + 1), atol=1e-15)


def test_attention_two_keys_ln3_weights():
    # scores differ by exactly ln 3 -> weights 1/4 and 3/4
    d = 4
    q = np.zeros((1, d)); q[0, 0] = 1.0
    k = np.zeros((1, 1, d))
    kn = np.zeros((1, d)); kn[0, 0] = math.log(3.0) * math.sqrt(d)
    v = np.zeros((1, 1, d)); v[0, 0, 1] = 1.0
    vn = np.zeros((1, d)); vn[0, 2] = 1.0
    c = _cache_from_fp16(k, v)
    # kn is not exactly representable in fp16; use the fp16 value in the expectation
    u2 = float(np.float16(kn[0, 0])) / math.sqrt(d)
    w2 = math.exp(u2) / (1 + math.exp(u2))
    o, mass = O.attention(q.astype(np.float16), c, kn.astype(np.float16), vn.astype(np.float16))
    assert abs(o[0, 1] - (1 - w2)) < 1e-15 and abs(o[0, 2] - w2) < 1e-15
    assert abs(w2 - 0.75) < 2e-3


def test_attention_matches_torch_sdpa_gqa():
    rng = np.random.default_rng(3)
    Hq, H, d, n = 10, 2, 32, 57
    k = rng.standard_normal((n, H, d)).astype(np.float16)
    v = rng.standard_normal((n, H, d)).astype(np.float16)
    c = _cache_from_fp16(k, v)
    # a few INT8 tokens with arbitrary scales
    c.is8[:20] = True
    c.k8[:20] = rng.integers(-127, 128, (20, H, d)).astype(np.int8)
    c.v8[:20] = rng.integers(-127, 128, (20, H, d)).astype(np.int8)
    c.ks = (rng.random((H, d)) * 0.05).astype(np.float32)
    c.vs = (rng.random((H, d)) * 0.05).astype(np.float32)
    q = rng.standard_normal((Hq, d)).astype(np.float16)
    kn = rng.standard_normal((H, d)).astype(np.float16)
    vn = rng.standard_normal((H, d)).astype(np.float16)
    o, mass = O.attention(q, c, kn, vn)
    # independent route: explicit dequantisation and torch SDPA in fp64
    K = np.where(c.is8[:, None, None], c.k8.astype(np.float64) * c.ks.astype(np.float64), k.astype(np.float64))
    Vv = np.where(c.is8[:, None, None], c.v8.astype(np.float64) * c.vs.astype(np.float64), v.astype(np.float64))
    K = np.concatenate([K, kn[None].astype(np.float64)])
    Vv = np.concatenate([Vv, vn[None].astype(np.float64)])
    g = Hq // H
    Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(g, 0)[None]
    Vt = torch.from_numpy(Vv).permute(1, 0, 2).repeat_interleave(g, 0)[None]
    Qt = torch.from_numpy(q.astype(np.float64))[None, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt)[0, :, 0].numpy()
    assert np.abs(o - ref).max() < 1e-12
    W = torch.softmax((Qt @ Kt.transpose(-1, -2)) / math.sqrt(d), -1)[0, :, 0].numpy()
    assert np.abs(mass - W.mean(0)).max() < 1e-14
    assert abs(mass.sum() - 1) < 1e-13 and (mass >= 0).all()


def test_attention_gqa_head_mapping():
    # kv head j holds constant value j+1 -> query head h must return (h // g) + 1
    H, d, n, g = 4, 8, 5, 3
    rng = np.random.default_rng(4)
    k = rng.standard_normal((n, H, d))
    v = np.broadcast_to((np.arange(H) + 1.0)[None, :, None], (n, H, d)).copy()
    c = _cache_from_fp16(k, v)
    q = rng.standard_normal((H * g, d)).astype(np.float16)
    o, _ = O.attention(q, c, k[0].astype(np.float16), v[0].astype(np.float16))
    for h in range(H * g):
        assert np.allclose(o[h], h // g + 1.0)


def test_int8_dequant_in_scores():
    # one INT8 token: code 10 at channel 3 with scale 0.5 means k = 5
    H, d = 1, 4
    c = O.empty_cache(H, d)
    c.pos = np.array([0]); c.is8 = np.array([True]); c.ema = np.zeros(1)
    c.k16 = np.zeros((1, H, d), np.float16); c.v16 = np.zeros((1, H, d), np.float16)
    c.k8 = np.zeros((1, H, d), np.int8); c.k8[0, 0, 3] = 10
    c.v8 = np.zeros((1, H, d), np.int8); c.v8[0, 0, 1] = -4
    c.ks = np.full((H, d), 0.5, np.float32); c.vs = np.full((H, d), 0.25, np.float32)
    q = np.zeros((1, d), np.float16); q[0, 3] = 1.0
    kn = np.zeros((H, d), np.float16); vn = np.zeros((H, d), np.float16)
    o, mass = O.attention(q, c, kn, vn)
    # u = [5/2, 0] -> w = [e^2.5, 1]/(e^2.5+1); v^ of the INT8 token is -1 at channel 1
    w = math.exp(2.5) / (math.exp(2.5) + 1)
    assert abs(o[0, 1] + w) < 1e-15 and abs(mass[0] - w) < 1e-15


# ------------------------------------------------------------------------ EMA

def test_ema_constant_mass_closed_form():
    lam, Abar, T = 0.9, 0.37, 25
    a = np.zeros(1)
    for _ in range(T):
        a, _ = O.ema_update(a, np.array([Abar, 0.0]), lam)
    assert abs(a[0] - Abar * (1 - lam ** T)) < 1e-15


def test_ema_lambda_zero_and_new_token():
    m = np.array([0.2, 0.3, 0.5])
    a, a_new = O.ema_update(np.array([0.9, 0.1]), m, 0.0)
    assert np.array_equal(a, m[:2]) and a_new == 0.5
    a, a_new = O.ema_update(np.array([0.9, 0.1]), m, 0.9)
    assert abs(a_new - 0.05) < 1e-16
    assert abs(a[0] - (0.81 + 0.02)) < 1e-15


# ----------------------------------------------------------------------- rank

def test_rank_hand_example():
    # a^ = [0.5, 1, 0.25]; r^ = [0, 0.5, 1]
    s = O.rank_scores(np.array([0.2, 0.4, 0.1]), np.array([0, 5, 10]), 0.65)
    assert np.allclose(s, [0.325, 0.825, 0.5125], atol=1e-15)


def test_rank_extremes():
    pos = np.array([3, 4, 9, 20])
    a = np.array([0.1, 0.0, 0.4, 0.2])
    assert np.allclose(O.rank_scores(a, pos, 0.0), (pos - 3) / 17)
    assert np.allclose(O.rank_scores(a, pos, 1.0), a / 0.4)
    assert np.allclose(O.rank_scores(np.zeros(4), pos, 1.0), 0)
    assert np.array_equal(O.rank_scores(np.array([0.3]), np.array([7]), 0.5), [0.5 * 1 + 0.5 * 1])


# ------------------------------------------------------------------ selection

def _brute_force_evict(s, pos, N, P):
    n = len(s)
    if n <= N:
        return set()
    k = n - N
    newest = set(np.argsort(pos)[n - P:].tolist()) if P > 0 else set()
    cand = [i for i in range(n) if i not in newest]
    found = []
    for E in itertools.combinations(cand, k):
        rest = [i for i in cand if i not in E]
        if all((s[e], pos[e]) < (s[r], pos[r]) for e in E for r in rest):
            found.append(set(E))
    assert len(found) == 1
    return found[0]


def test_select_exhaustive_small():
    rng = np.random.default_rng(7)
    for trial in range(300):
        n = int(rng.integers(1, 9))
        P = int(rng.integers(0, n + 1))
        N = int(rng.integers(P, n + 2)) if P <= n else n
        N = max(N, P)
        s = rng.integers(0, 4, n) / 4.0            # many ties
        pos = np.sort(rng.choice(50, n, replace=False))
        keep = O.select_keep(s, pos, N, P)
        assert set(np.flatnonzero(~keep).tolist()) == _brute_force_evict(s, pos, N, P)


def test_select_counts_and_protection():
    rng = np.random.default_rng(8)
    n, N, P = 300, 120, 32
    s = rng.random(n)
    pos = np.sort(rng.choice(10_000, n, replace=False))
    keep = O.select_keep(s, pos, N, P)
    assert keep.sum() == N and keep[-P:].all()
    assert O.select_keep(s, pos, n, P).all()       # n <= N is a no-op
    with pytest.raises(ValueError):
        O.select_keep(s, pos, 10, 32)


def test_select_sliding_window_and_topN():
    rng = np.random.default_rng(9)
    n, N = 200, 64
    pos = np.sort(rng.choice(5000, n, replace=False))
    a = rng.random(n)
    keep = O.select_keep(O.rank_scores(a, pos, 0.0), pos, N, 16)
    assert np.array_equal(np.flatnonzero(keep), np.arange(n - N, n))   # newest N survive
    keep = O.select_keep(O.rank_scores(a, pos, 1.0), pos, N, 0)
    assert set(np.flatnonzero(keep)) == set(np.argsort(-a)[:N].tolist())


def test_select_all_equal_evicts_oldest():
    pos = np.arange(10, 50)
    keep = O.select_keep(np.full(40, 0.5), pos, 30, 4)
    assert np.array_equal(np.flatnonzero(~keep), np.arange(10))


# ---- block eviction (the review's limitation sections: coarse eviction for
# paged layouts). Block grouping and the block score are readings; the pins
# below fix them by hand-worked cases, reduction to token eviction and a
# brute-force characterisation.

def test_select_block_hand_worked():
    # 12 tokens, P = 2 protected, B = 3: full candidate blocks {0,1,2},
    # {3,4,5}, {6,7,8}; token 9 is a partial block and stays. N = 7 -> k = 5
    # -> ceil(5/3) = 2 blocks leave. Block maxima 0.9, 0.5, 0.4: the last two
    # leave (a mean would drop block 0 instead of block 1, a min blocks 0, 2).
    s = np.array([0.1, 0.9, 0.1, 0.5, 0.5, 0.5, 0.2, 0.3, 0.4, 0.0, 0.0, 0.0])
    pos = np.arange(100, 112)
    keep = O.select_keep(s, pos, 7, 2, block=3)
    assert np.flatnonzero(~keep).tolist() == [3, 4, 5, 6, 7, 8]
    # equal block maxima: the older block leaves first
    s2 = np.array([0.5, 0.2, 0.1, 0.5, 0.1, 0.1, 0.7, 0.7, 0.7, 0.0, 0.0, 0.0])
    keep = O.select_keep(s2, pos, 9, 2, block=3)        # k = 3 -> one block
    assert np.flatnonzero(~keep).tolist() == [0, 1, 2]
    # too few full blocks: every full block leaves, the count stays above N
    keep = O.select_keep(s, pos, 2, 2, block=3)         # k = 10 -> 4 blocks wanted, 3 exist
    assert np.flatnonzero(keep).tolist() == [9, 10, 11]


def test_select_block_of_one_is_token_eviction():
    rng = np.random.default_rng(21)
    for _ in range(200):
        n = int(rng.integers(1, 60))
        P = int(rng.integers(0, n + 1))
        N = int(rng.integers(P, n + 3))
        s = rng.integers(0, 5, n) / 4.0                  # many ties
        pos = np.sort(rng.choice(1000, n, replace=False))
        perm = rng.permutation(n)                        # order must not matter
        a = O.select_keep(s[perm], pos[perm], N, P, block=1)
        b = O.select_keep(s[perm], pos[perm], N, P)
        assert np.array_equal(a, b)


def _brute_force_block_evict(s, pos, N, P, B):
    n = len(s)
    if n <= N:
        return set()
    rank = np.empty(n, np.int64)
    rank[np.argsort(pos)] = np.arange(n)                 # 0 = oldest
    nfull = (n - P) // B
    members = {j: [i for i in range(n) if rank[i] // B == j] for j in range(nfull)}
    score = {j: max(s[i] for i in members[j]) for j in members}
    kb = min(nfull, (n - N + B - 1) // B)
    found = []
    for E in itertools.combinations(range(nfull), kb):
        rest = [j for j in range(nfull) if j not in E]
        if all((score[e], e) < (score[r], r) for e in E for r in rest):
            found.append({i for e in E for i in members[e]})
    assert len(found) == 1
    return found[0]


def test_select_block_brute_force():
    rng = np.random.default_rng(22)
    for _ in range(300):
        B = int(rng.integers(1, 5))
        n = int(rng.integers(1, 25))
        P = int(rng.integers(0, n + 1))
        N = int(rng.integers(P, n + 2))
        s = rng.integers(0, 4, n) / 4.0
        pos = rng.choice(500, n, replace=False)          # unsorted positions
        keep = O.select_keep(s, pos, N, P, block=B)
        assert set(np.flatnonzero(~keep).tolist()) == _brute_force_block_evict(s, pos, N, P, B)


def test_select_block_recency_and_counts():
    rng = np.random.default_rng(23)
    n, P, B = 700, 32, 16
    pos = np.sort(rng.choice(50_000, n, replace=False))
    for N in (100, 333, 600, 668, 699):
        k = n - N
        nfull = (n - P) // B
        kb = min(nfull, -(-k // B))
        # recency scores (alpha = 0): the oldest kb blocks leave
        keep = O.select_keep(O.rank_scores(rng.random(n), pos, 0.0), pos, N, P, block=B)
        assert np.array_equal(np.flatnonzero(~keep), np.arange(kb * B))
        keep = O.select_keep(rng.random(n), pos, N, P, block=B)
        assert (~keep).sum() == kb * B and keep[-P:].all()
        assert N - B < keep.sum() <= N
        assert keep[nfull * B:].all()                    # partial block and protected stay
        ev = np.flatnonzero(~keep)
        assert np.all(ev.reshape(-1, B) % B == np.arange(B)) and np.all(np.diff(ev.reshape(-1, B)) == 1)


def test_compact_and_append_preserve_rows():
    rng = np.random.default_rng(10)
    k = rng.standard_normal((12, 2, 4)); v = rng.standard_normal((12, 2, 4))
    c = _cache_from_fp16(k, v)
    c.ema = rng.random(12)
    keep = rng.random(12) < 0.5
    c2 = O.compact(c, keep)
    idx = np.flatnonzero(keep)
    assert np.array_equal(c2.pos, c.pos[idx]) and np.array_equal(c2.k16, c.k16[idx])
    assert np.array_equal(c2.ema, c.ema[idx]) and (np.diff(c2.pos) > 0).all()
    c3 = O.append(c2, k[0], v[0], 99, 0.125)
    assert c3.pos[-1] == 99 and c3.ema[-1] == 0.125 and not c3.is8[-1]


def _int8_cache(n8, n16, rng):
    k = rng.standard_normal((n8 + n16, 2, 4)); v = rng.standard_normal((n8 + n16, 2, 4))
    c = _cache_from_fp16(k, v)
    c.is8 = np.arange(n8 + n16) < n8
    c.ema = rng.random(n8 + n16)
    return c


def test_compact_fill_hand_worked():
    # INT8 part of 8 entries keeps [0, 2, 3, 5, 6]: new INT8 length 5, holes
    # below it at slots 1 and 4, surviving tail entries 5 and 6 -> 5 fills
    # slot 1 and 6 fills slot 4; the FP16 part (slots 8-10) stays in order.
    c = _int8_cache(8, 3, np.random.default_rng(12))
    keep = np.array([1, 0, 1, 1, 0, 1, 1, 0, 1, 0, 1], bool)
    c2 = O.compact(c, keep, fill=True)
    assert c2.pos.tolist() == [c.pos[i] for i in (0, 5, 2, 3, 6, 8, 10)]
    assert np.array_equal(c2.is8, [1, 1, 1, 1, 1, 0, 0])
    assert np.array_equal(O.compact(c, keep).pos, c.pos[np.flatnonzero(keep)])  # stable form


def test_compact_fill_invariants():
    rng = np.random.default_rng(13)
    for _ in range(300):
        n8, n16 = int(rng.integers(0, 40)), int(rng.integers(1, 12))
        c = _int8_cache(n8, n16, rng)
        keep = rng.random(n8 + n16) < rng.random()
        f, st = O.compact(c, keep, fill=True), O.compact(c, keep)
        m = int(keep[:n8].sum())
        # same survivors with the same rows, INT8 first, FP16 part identical
        assert sorted(f.pos.tolist()) == sorted(st.pos.tolist())
        assert np.array_equal(f.is8, st.is8) and np.array_equal(f.pos[m:], st.pos[m:])
        for name in ("k16", "v16", "k8", "v8", "ema"):
            got = dict(zip(f.pos.tolist(), getattr(f, name)))
            want = dict(zip(c.pos.tolist(), getattr(c, name)))
            assert all(np.array_equal(got[p], want[p]) for p in got)
        # INT8 survivors below the new end keep their slot; the others move,
        # fewer than the evicted INT8 entries, and in slot order
        stay = [i for i in range(m) if keep[i]]
        assert all(f.pos[i] == c.pos[i] for i in stay)
        moved = [i for i in range(m) if not keep[i]]
        src = [int(np.flatnonzero(c.pos == f.pos[i])[0]) for i in moved]
        assert src == sorted(src) and all(s_ >= m for s_ in src)
        assert len(moved) <= n8 - m
        # evictions only at the INT8 tail move nothing
        tail_only = keep.copy(); tail_only[:n8] = np.arange(n8) < m
        assert np.array_equal(O.compact(c, tail_only, fill=True).pos, O.compact(c, tail_only).pos)


# --------------------------------------------------------------- quantisation

def test_quantize_round_trip_bound_and_absmax():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((500, 3, 16)).astype(np.float16)
    s = O.absmax_scale(x)
    codes, sat = O.quantize_rows(x, s)
    assert sat == 0
    err = np.abs(x.astype(np.float64) - codes.astype(np.float64) * s.astype(np.float64))
    assert (err <= s.astype(np.float64) / 2 * (1 + 2 ** -23 * 128)).all()
    am = np.abs(x.astype(np.float32)).argmax(0)
    for h in range(3):
        for ch in range(16):
            assert abs(int(codes[am[h, ch], h, ch])) == 127


def test_quantize_zero_channel_and_half_even():
    x = np.zeros((4, 1, 3), np.float16)
    x[:, 0, 1] = [127.0, 2.5, 3.5, -2.5]            # scale exactly 1.0
    s = O.absmax_scale(x)
    assert s[0, 0] == 0 and s[0, 1] == 1.0
    codes, _ = O.quantize_rows(x, s)
    assert list(codes[:, 0, 1]) == [127, 2, 4, -2]  # round half to even
    assert (codes[:, 0, 0] == 0).all()


def test_quantize_saturation_counted():
    s = np.full((1, 2), 0.01, np.float32)
    x = np.array([[[2.0, -0.5]]], np.float16)
    codes, sat = O.quantize_rows(x, s)
    assert list(codes[0, 0]) == [127, -50] and sat == 1


def _empty_start_steps(rows_k, rows_v, W):
    """Runs the oracle from an empty cache over len(rows_k) steps (one kv head,
    no eviction), appending the given K/V rows; returns the caches after each step."""
    from types import SimpleNamespace
    pol = SimpleNamespace(lam=0.9, alpha=0.65, protect=0, window=W, block=0, order=0)
    d = len(rows_k[0])
    c = O.empty_cache(1, d)
    out = []
    q = np.ones((1, d))
    for t, (k, v) in enumerate(zip(rows_k, rows_v)):
        r = O.step_one(c, q, np.asarray([k], np.float16), np.asarray([v], np.float16), t, pol, N=100)
        c = r["cache"]
        out.append(c)
    return out


def test_first_calibration_from_an_empty_cache_hand_worked():
    """Readings R17 + R18 from an empty cache with W = 2: the first token
    leaves the FP16 window at step t = 2, after the append, so the scales are
    set over the three tokens then cached (positions 0, 1, 2): the exiting
    token, the middle one and the token just appended. Hand-worked rows put
    each channel's absolute maximum on a different token, so leaving out the
    appended token (channel 2) or the exiting one (channel 0 of K, channel 1
    of V) changes a scale and the codes."""
    K = [[3.0, -1.0, 0.5], [1.0, -5.0, 2.0], [-0.25, 4.0, -7.0]]
    V = [[0.5, 6.0, -2.0], [-4.0, 1.0, 1.0], [1.0, -0.5, 2.5]]
    c0, c1, c2 = _empty_start_steps(K, V, W=2)
    # steps 0 and 1: nothing has left the window, no scales yet
    for c in (c0, c1):
        assert not c.calibrated and not c.is8.any()
    # step 2: scales = fp32(absmax over positions 0, 1, 2) / 127, per channel
    f = np.float32
    want_ks = np.array([[f(3) / f(127), f(5) / f(127), f(7) / f(127)]], np.float32)
    want_vs = np.array([[f(4) / f(127), f(6) / f(127), f(2.5) / f(127)]], np.float32)
    assert c2.calibrated
    assert np.array_equal(c2.ks.view(np.uint32), want_ks.view(np.uint32))
    assert np.array_equal(c2.vs.view(np.uint32), want_vs.view(np.uint32))
    # token 0 (and only it) is INT8 now: K 3/(3/127) = 127, -1/(5/127) = -25.4,
    # 0.5/(7/127) = 9.07; V 0.5/(4/127) = 15.9, 6/(6/127) = 127, -2/(2.5/127) = -101.6
    assert c2.pos.tolist() == [0, 1, 2] and c2.is8.tolist() == [True, False, False]
    assert c2.k8[0, 0].tolist() == [127, -25, 9]
    assert c2.v8[0, 0].tolist() == [16, 127, -102]
    assert c2.saturated == 0


def test_prefill_layout():
    rng = np.random.default_rng(12)
    H, L0, d, W = 2, 40, 8, 16
    k = rng.standard_normal((H, L0, d)).astype(np.float16)
    v = rng.standard_normal((H, L0, d)).astype(np.float16)
    c = O.prefill(k, v, W)
    assert c.calibrated and c.n == L0
    assert (c.is8 == (c.pos <= L0 - 1 - W)).all()
    assert np.array_equal(c.ks, (np.abs(k.astype(np.float32)).max(1) / np.float32(127)).astype(np.float32))
    short = O.prefill(k[:, :10], v[:, :10], W)
    assert not short.calibrated and not short.is8.any()


# ----------------------------------------------------------------- end to end

def _small_cfg():
    pol = synth.Policy(n_high=24, n_low=48, protect=8, window=16)
    return synth.Config(name="tiny", layers=2, batch=2, hq=4, hkv=2, d=16, vocab=64,
                        prefill=40, steps=60, policy=pol)


@pytest.mark.parametrize("order", [0, 1])
def test_end_to_end_invariants(order):
    """Over a free run: lengths, counts, protection, the FP16 window, EMA range
    and mass. The default, stable order (0) keeps every position ascending
    after every step, the new token last (the compacted survivors in their
    original order); the hole-filling option (1, reading R24) reorders the
    INT8 part at some step."""
    from dataclasses import replace
    cfg = _small_cfg()
    pol = replace(cfg.policy, order=order)
    kp, vp = synth.prefill_kv(cfg, seed=0)
    caches = [[O.prefill(kp[l, b], vp[l, b], pol.window) for b in range(cfg.batch)] for l in range(cfg.layers)]
    lengths = []
    reordered = False
    for i in range(cfg.steps):
        t = cfg.prefill + i
        logits = synth.logits_for_step(cfg, 0, i)
        q, kn, vn = synth.decode_inputs(cfg, 0, i)
        out = O.step(caches, logits, q, kn, vn, t, pol)
        for l in range(cfg.layers):
            for b in range(cfg.batch):
                c0, c1 = caches[l][b], out.caches[l][b]
                N = out.budget[l, b]
                assert c1.n <= max(c0.n, N) + 1 and c1.n <= max(N, c0.n) + 1
                if c0.n > N:
                    assert c1.n == N + 1
                    assert (~out.keep[l][b]).sum() == c0.n - N
                # new token last, positions unique, the FP16 part in ascending order
                n8 = int(c1.is8.sum())
                assert c1.pos[-1] == t and len(set(c1.pos.tolist())) == c1.n
                assert c1.is8[:n8].all() and (np.diff(c1.pos[n8:]) > 0).all()
                reordered |= bool((np.diff(c1.pos[:n8]) < 0).any())
                if order == 0:
                    assert (np.diff(c1.pos) > 0).all()
                assert (c1.is8 == (c1.pos <= t - pol.window)).all()      # FP16 = window positions
                # protected newest P of the pre-step cache survive
                assert set(np.sort(c0.pos)[-pol.protect:].tolist()) <= set(c1.pos.tolist())
                assert ((c1.ema >= 0) & (c1.ema <= 1)).all()
                assert abs(out.mass[l][b].sum() - 1) < 1e-12
        lengths.append(out.caches[0][0].n)
        caches = out.caches
    # sawtooth: the cache both shrinks (confident steps) and regrows
    d = np.diff(lengths)
    assert (d < 0).any() and (d > 0).any()
    assert reordered == (order == 1)  # the INT8 hole filling took place (fill order only)


def test_ema_of_retained_token_follows_closed_recurrence():
    # a slot's EMA equals sum_k (1-lam) lam^(t-k) Abar_k over the steps it has seen
    cfg = _small_cfg()
    pol = cfg.policy
    kp, vp = synth.prefill_kv(cfg, seed=1)
    caches = [[O.prefill(kp[l, b], vp[l, b], pol.window) for b in range(cfg.batch)] for l in range(cfg.layers)]
    hist = []
    tracked = cfg.prefill - 1          # protected for the first steps
    for i in range(6):
        q, kn, vn = synth.decode_inputs(cfg, 1, i)
        out = O.step(caches, synth.logits_for_step(cfg, 1, i), q, kn, vn, cfg.prefill + i, pol)
        j = int(np.flatnonzero(caches[0][0].pos == tracked)[0])
        hist.append(out.mass[0][0][j])
        caches = out.caches
    j = int(np.flatnonzero(caches[0][0].pos == tracked)[0])
    want = sum((1 - pol.lam) * pol.lam ** (len(hist) - 1 - k) * hist[k] for k in range(len(hist)))
    assert abs(caches[0][0].ema[j] - want) < 1e-15


# ---------------------------------------------------------------- next token

def test_next_token_greedy_smallest_index_among_ties():
    z = np.array([0.5, 2.0, -1.0, 2.0, 1.9], np.float32)
    assert O.next_token(z, 0.0) == 1
    z2 = np.array([-np.inf, 3.0, 3.0], np.float32)
    assert O.next_token(z2, 0.0) == 1
    assert O.next_token(np.array([np.nan, 1.0], np.float32), 0.0) == -1


def test_next_token_two_level_closed_form():
    # p = (1/4, 3/4) at temperature 1; (1, sqrt 3)/(1 + sqrt 3) at temperature 2
    z = np.array([0.0, np.log(3.0)])
    assert O.next_token(z, 1.0, 0.0) == 0
    assert O.next_token(z, 1.0, 0.2499) == 0
    assert O.next_token(z, 1.0, 0.2501) == 1
    p0 = 1.0 / (1.0 + np.sqrt(3.0))
    assert O.next_token(z, 2.0, p0 - 1e-6) == 0
    assert O.next_token(z, 2.0, p0 + 1e-6) == 1
    lo, hi = O.token_interval(z, 2.0, 1)
    assert abs(lo - p0) < 1e-12 and abs(hi - 1.0) < 1e-12


def test_next_token_frequencies_match_tempered_softmax():
    rng = np.random.default_rng(17)
    z = rng.standard_normal(12) * 1.5
    z[4] = -np.inf                       # never drawn
    T = 0.7
    p = np.exp((z - z.max()) / T)
    p /= p.sum()
    us = rng.random(20000)
    counts = np.bincount([O.next_token(z, T, u) for u in us], minlength=12)
    assert counts[4] == 0
    sd = np.sqrt(p * (1 - p) / len(us))
    assert np.all(np.abs(counts / len(us) - p) <= 4.5 * sd + 1e-12)


def test_next_token_low_temperature_approaches_greedy():
    rng = np.random.default_rng(5)
    z = rng.standard_normal(50)
    g = O.next_token(z, 0.0)
    for u in (0.01, 0.5, 0.99):
        assert O.next_token(z, 1e-3, u) == g
