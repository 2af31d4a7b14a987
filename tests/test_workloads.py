"""CPU pins of the synthetic workload recipe: the pyramid budgets of the
long-context variant (reading R14), the cache capacity rule, and the shape of
the throughput workload bench.py times."""
from fractions import Fraction

import synth
from synth.configs import _PYR_HI, _PYR_LO


def test_pyramid_budgets_follow_the_linear_reading():
    # N_low,l = round(4096 - 3072 l / 63), N_high,l = floor(N_low,l / 2),
    # computed exactly; no layer falls on a half-way case
    for l in range(64):
        x = Fraction(4096) - Fraction(3072 * l, 63)
        frac = x - (x.numerator // x.denominator)
        assert frac != Fraction(1, 2)
        want = int(x + Fraction(1, 2)) if frac else int(x)
        assert _PYR_LO[l] == want, l
        assert _PYR_HI[l] == _PYR_LO[l] // 2
    assert _PYR_LO[0] == 4096 and _PYR_LO[-1] == 1024
    assert all(a >= b for a, b in zip(_PYR_LO, _PYR_LO[1:]))


def test_capacity_holds_the_prefill_or_a_full_budget_plus_the_new_token():
    for name in ("gpt2_layer", "gpt2_stack", "qwen14b", "qwen32b", "qwen32b_niah"):
        cfg = synth.get_config(name)
        n_low = max(cfg.layer_n_low) if cfg.layer_n_low else cfg.policy.n_low
        assert cfg.cap == max(cfg.prefill, n_low + 1) + 1, name


def test_throughput_workload_shape():
    # Qwen-32B shape, batch 8, 4096 generated tokens on a 2048-token prefill
    cfg = synth.get_config("qwen32b")
    assert (cfg.layers, cfg.batch, cfg.hq, cfg.hkv, cfg.d, cfg.vocab) == (64, 8, 40, 8, 128, 152064)
    assert (cfg.prefill, cfg.steps) == (2048, 4096)
    p = cfg.policy
    assert (p.n_high, p.n_low, p.protect, p.window, p.block, p.order) == (1024, 2048, 64, 256, 0, 0)
    assert (p.tau, p.alpha, p.lam) == (0.7, 0.65, 0.9)
