"""GPU parity: every C-ABI call against the fp64 oracle on seeded inputs.

Protocol: the oracle runs free. It builds its own cache from the same seeded
prefill, computes its own confidence, attention, EMA and scores in fp64, and
takes its own decisions; the device runs the five calls on the same inputs.
After every step the two are compared:
  - budget choice, survivor positions and order, INT8 codes, scales and
    FP16 rows: bit-exact. A confidence within 1e-5 of tau lies in the
    rounding band where both budgets are correct; such steps (counted, and
    expected to be rare) follow the device's choice.
  - attention output: max |o - o_ref| <= 2e-3 * max |o_ref| per (layer, seq).
  - confidence, per-key mass, EMA and rank scores: absolute error <= 1e-5.
Selection compares fp32 device scores with fp64 oracle scores; a mismatch is
reported with the score gap at the eviction boundary.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import confk_oracle as O
from tests.helpers import assert_state_equal, rel_maxabs

pytestmark = pytest.mark.gpu

ATOL = 1e-5
OTOL = 2e-3


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mixed_precision_attention_amd as M
    M.load()  # raises if the HIP library is missing
    return torch.device("cuda")


def _cfg(name, layers, batch, hq, hkv, d, vocab, prefill, n_high, n_low, protect, window, **kw):
    pol = synth.Policy(n_high=n_high, n_low=n_low, protect=protect, window=window)
    return synth.Config(name=name, layers=layers, batch=batch, hq=hq, hkv=hkv, d=d, vocab=vocab,
                        prefill=prefill, steps=0, policy=pol, **kw)


# Small shapes spanning several 16-key tiles with ragged tails.
TINY = {
    "g5_d128": _cfg("g5_d128", 2, 3, 10, 2, 128, 1000, 300, 96, 200, 16, 64),
    "mha_d64": _cfg("mha_d64", 2, 2, 4, 4, 64, 777, 150, 40, 80, 8, 32),
    "g3_d64_empty": _cfg("g3_d64_empty", 1, 2, 6, 2, 64, 333, 0, 24, 48, 8, 16, sinks=2),
    "g16_d128": _cfg("g16_d128", 1, 2, 16, 1, 128, 500, 90, 40, 70, 4, 20),
}


def _nosplit_ws(eng, nlayers):
    """The engine's attention workspace cut to its part without the split
    exchange area (None when that part is empty), for launches over
    `nlayers` layers that must run one workgroup per kv head."""
    import mixed_precision_attention_amd as M
    nb = M.engine.workspace_bytes(M._lib.WS_ATTENTION_NOSPLIT, eng.cache, nlayers=nlayers)
    return eng.attn_ws[:nb] if nb else None


def _t(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def _inputs(cfg, seed, i):
    logits = synth.logits_for_step(cfg, seed, i)
    q, kn, vn = synth.decode_inputs(cfg, seed, i)
    t = cfg.prefill + i
    if cfg.sinks:
        kn = synth.gen.apply_sinks(cfg, seed, t, kn)
    return logits, q, kn, vn, t


class Run:
    """Device engine plus the oracle states of the checked (layer, seq) pairs."""

    def __init__(self, cfg, seed, pairs=None, device_prefill=False, split_keys=True, per_layer=False):
        import mixed_precision_attention_amd as M
        self.dev = _dev()
        self.cfg, self.seed = cfg, seed
        self.per_layer = per_layer  # attention as one launch per layer
        self.pairs = pairs or [(l, b) for l in range(cfg.layers) for b in range(cfg.batch)]
        self.eng = M.DecodeEngine(cfg, self.dev, split_keys=split_keys)
        self.band = 0
        W = cfg.policy.window
        if cfg.prefill == 0:
            self.eng.prefill(None, None)
            self.orc = {p: O.empty_cache(cfg.hkv, cfg.d) for p in self.pairs}
        elif device_prefill:
            kp, vp = synth.gen.prefill_kv_device(cfg, seed, self.dev)
            self.eng.prefill(kp, vp)
            self.orc = {(l, b): O.prefill(kp[l, b].cpu().numpy(), vp[l, b].cpu().numpy(), W)
                        for (l, b) in self.pairs}
            del kp, vp
        else:
            kp, vp = synth.prefill_kv(cfg, seed)
            self.eng.prefill(_t(kp, self.dev), _t(vp, self.dev))
            self.orc = {(l, b): O.prefill(kp[l, b], vp[l, b], W) for (l, b) in self.pairs}
        torch.cuda.synchronize()
        for (l, b) in self.pairs:
            assert_state_equal(self.eng.cache.snapshot(l, b), self.orc[(l, b)],
                               what=f"prefill l={l} b={b}")

    def budgets(self, l):
        cfg = self.cfg
        if cfg.layer_n_low is not None:
            return cfg.layer_n_low[l], cfg.layer_n_high[l]
        return cfg.policy.n_low, cfg.policy.n_high

    def step(self, i, scores=None):
        """One step on both sides; `scores` optionally replaces the rank scores
        (same array on both sides) to exercise selection with crafted ties."""
        cfg, eng, dev, pol = self.cfg, self.eng, self.dev, self.cfg.policy
        logits, q, kn, vn, t = _inputs(cfg, self.seed, i)
        lg, qd, kd, vd = _t(logits, dev), _t(q, dev), _t(kn, dev), _t(vn, dev)
        eng.step_confidence(lg)
        c_dev = eng.c.cpu().numpy().astype(np.float64)
        bud_dev = eng.budget.cpu().numpy()
        if self.per_layer:
            eng.step_attention_layerwise(qd, kd, vd)
        else:
            eng.step_attention(qd, kd, vd)
        out = eng.out.float().cpu().numpy()
        mass = eng.mass.cpu().numpy()
        rows = eng.cache.mass_rows()
        eng.step_ema_rank(t)
        ema = eng.cache.ema.cpu().numpy()
        if scores is not None:
            eng.score.copy_(_t(scores, dev))
        score = eng.score.cpu().numpy()
        eng.step_compact(kd, vd)
        eng.step_quantize(t)
        torch.cuda.synchronize()
        assert int(eng.cache.status.cpu()[0]) == 0, "device status set"
        evicted = eng.evicted.cpu().numpy()
        events = 0
        c_ref = np.zeros(cfg.batch)
        for b in range(cfg.batch):
            c_ref[b] = O.confidence(logits[b])[0]
            assert abs(c_dev[b] - c_ref[b]) <= ATOL, f"step {i} b={b}: confidence {c_dev[b]} vs {c_ref[b]}"
        for (l, b) in self.pairs:
            w = f"step {i} l={l} b={b}"
            nl, nh = self.budgets(l)
            N = O.budget(c_ref[b], pol.tau, nh, nl)
            got_N = int(bud_dev[l if bud_dev.shape[0] > 1 else 0, b])
            if got_N != N:
                assert abs(c_ref[b] - pol.tau) <= ATOL, f"{w}: budget {got_N} vs {N}, c={c_ref[b]}"
                self.band += 1
                N = got_N
            pre = self.orc[(l, b)]
            n = pre.n
            sg = None if scores is None else scores[l, b, :n]
            r = O.step_one(pre, q[l, b], kn[l, b], vn[l, b], t, pol, N, score_given=sg)
            assert rel_maxabs(out[l, b], r["o"]) <= OTOL, f"{w}: attention output"
            m = mass[l, b, : rows[l, b], : n + 1].sum(0) / cfg.hq
            assert np.abs(m - r["mass"]).max() <= ATOL, f"{w}: mass"
            assert np.abs(ema[l, b, :n] - r["ema"]).max(initial=0) <= ATOL, f"{w}: EMA"
            assert abs(ema[l, b, n] - r["a_new"]) <= ATOL, f"{w}: new-token EMA"
            if scores is None:
                assert np.abs(score[l, b, :n] - r["score"]).max(initial=0) <= ATOL, f"{w}: score"
            snap = eng.cache.snapshot(l, b)
            want_pos = r["cache"].pos
            if not np.array_equal(snap["pos"].astype(np.int64), want_pos):
                s = r["score"] if sg is None else sg
                ev = np.sort(s[~r["keep"]])
                kp = np.sort(s[: max(0, n - pol.protect)][r["keep"][: max(0, n - pol.protect)]])
                gap = (kp[0] - ev[-1]) if len(ev) and len(kp) else float("nan")
                raise AssertionError(f"{w}: survivors differ (boundary score gap {gap:.3e})")
            assert evicted[l, b] == int((~r["keep"]).sum()), f"{w}: evicted count"
            assert_state_equal(snap, r["cache"], what=w)
            self.orc[(l, b)] = r["cache"]
            events += int(evicted[l, b] > 0)
        return events


@pytest.mark.parametrize("split_keys", [True, False], ids=["split", "nosplit"])
@pytest.mark.parametrize("name", list(TINY))
def test_parity_tiny(name, split_keys):
    """The small shapes fill few of the GPU's workgroup slots, so attention
    splits each unit's keys over several workgroups unless the workspace
    leaves out the exchange area (nosplit): both forms against the oracle."""
    cfg = TINY[name]
    steps = 70 if cfg.prefill == 0 else 24
    print(f"[parity] {name} steps={steps} split_keys={split_keys}", flush=True)
    run = Run(cfg, seed=11, split_keys=split_keys)
    events = sum(run.step(i) for i in range(steps))
    assert events > 0
    assert run.band <= 1


def test_parity_gpt2_layer_workload():
    """The GPT-2 single-layer workload as configured (a 1024-token cache, the
    newest 64 FP16, 64 decode steps), free-running against the oracle."""
    cfg = synth.get_config("gpt2_layer")
    print(f"[parity] gpt2_layer steps={cfg.steps}", flush=True)
    run = Run(cfg, seed=0)
    events = sum(run.step(i) for i in range(cfg.steps))
    assert events > 0
    assert run.band <= 1


def test_parity_gpt2_stack_from_empty():
    """The GPT-2 stack workload as configured: 12 layers from an empty cache
    with four sink keys, all 2048 generated steps, every layer compared with
    the oracle after every step (past the first calibration at step W and
    through repeated evictions at both budgets)."""
    cfg = synth.get_config("gpt2_stack")
    steps = cfg.steps
    print(f"[parity] gpt2_stack steps={steps} layers={cfg.layers}", flush=True)
    run = Run(cfg, seed=0)
    events = 0
    for i in range(steps):
        events += run.step(i)
        if i % 256 == 255:
            print(f"[parity] gpt2_stack step {i + 1}: {events} eviction events", flush=True)
    n, n8 = run.eng.cache.lengths()
    assert events > 0
    assert (n8 > 0).all()  # the INT8 region was calibrated and populated
    assert run.band <= 4


SPLIT_CASES = {
    # one unit over 50001 keys: 16 pieces of about 3100 keys, whose scores
    # spill past the LDS budget; later steps (about 1200 keys) split in 2
    "g5_d128_spill": _cfg("split_spill", 1, 1, 5, 1, 128, 700, 50000, 600, 1200, 16, 64),
    # four MHA units (g = 1, d = 64): 5 pieces each at first, ragged INT8 tails
    "mha_d64": _cfg("split_mha", 1, 1, 4, 4, 64, 700, 2997, 1500, 2500, 8, 32),
    # sixteen query heads per kv head: the largest output partials
    "g16_d128": _cfg("split_g16", 1, 2, 16, 1, 128, 700, 2501, 900, 1900, 16, 48),
}


@pytest.mark.parametrize("case", list(SPLIT_CASES))
def test_parity_split_keys(case):
    """Launches of a few units split each unit's keys over up to eight
    workgroups that exchange their softmax maxima and normalisers (and
    output partials) through the workspace; output, per-key mass and the
    rest of the step against the oracle, with the status word clear (no
    split gave up waiting)."""
    cfg = SPLIT_CASES[case]
    print(f"[parity] split keys {case}", flush=True)
    run = Run(cfg, seed=21)
    for i in range(4):
        run.step(i)


def test_parity_split_keys_per_layer_pyramid():
    """Attention issued one layer at a time at batch 1 (as a forward pass
    issues it): each launch has eight units of 1200-2400 keys, which split
    into 2-4 pieces, with per-layer budgets falling from 2400 to 1200;
    every layer against the oracle after every step."""
    lo = (2400, 2000, 1600, 1200)
    hi = tuple(x // 2 for x in lo)
    cfg = _cfg("pyr_split", 4, 1, 40, 8, 128, 900, 2600, max(hi), max(lo), 64, 256,
               layer_n_low=lo, layer_n_high=hi)
    print("[parity] per-layer split pyramid", flush=True)
    run = Run(cfg, seed=13, per_layer=True)
    for i in range(5):
        run.step(i)


def test_split_keys_graph_replay():
    """A split-key attention launch captured in a HIP graph and replayed
    several times, with the program's own eager launches (unsplit) and
    synchronisations between the replays: every replay gives the eager
    launch's output and mass bit for bit (the exchange words carry a
    per-unit epoch that each launch advances, so a replay never reads a
    word of an earlier one; no memory-set node is recorded)."""
    import mixed_precision_attention_amd as M
    dev = _dev()
    cfg = SPLIT_CASES["mha_d64"]
    eng = M.DecodeEngine(cfg, dev)
    kp, vp = synth.prefill_kv(cfg, 21)
    eng.prefill(_t(kp, dev), _t(vp, dev))
    _, q, kn, vn, _ = _inputs(cfg, 21, 0)
    qd, kd, vd = _t(q, dev), _t(kn, dev), _t(vn, dev)
    print("[parity] split keys under graph replay", flush=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capture (the library's device queries)
        for _ in range(2):
            M.engine.attn_decode(eng.cache, qd, kd, vd, eng.out, eng.mass, eng.attn_ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    out0, mass0 = eng.out.clone(), eng.mass.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        M.engine.attn_decode(eng.cache, qd, kd, vd, eng.out, eng.mass, eng.attn_ws)
    nospl = _nosplit_ws(eng, cfg.layers)
    for rep in range(4):
        eng.out.zero_()
        eng.mass.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(eng.out, out0), f"replay {rep}: output"
        assert torch.equal(eng.mass, mass0), f"replay {rep}: mass"
        assert int(eng.cache.status.cpu()[0]) == 0, f"replay {rep}: status"
        # eager work between replays: an unsplit launch over the same cache
        M.engine.attn_decode(eng.cache, qd, kd, vd, eng.out, eng.mass, nospl)
        torch.cuda.synchronize()
        assert rel_maxabs(eng.out.float().cpu().numpy(), out0.float().cpu().numpy()) <= OTOL / 2


def test_parity_pyramid_budgets():
    lo = (60, 52, 44)
    hi = tuple(x // 2 for x in lo)
    cfg = _cfg("pyr", 3, 2, 10, 2, 128, 600, 120, max(hi), max(lo), 8, 24,
               layer_n_low=lo, layer_n_high=hi)
    print("[parity] pyramid", flush=True)
    run = Run(cfg, seed=5)
    for i in range(12):
        run.step(i)
    n, _ = run.eng.cache.lengths()
    for l in range(3):
        assert (n[l] <= lo[l] + 1).all()


def test_parity_long_cache_path():
    """Capacity above 4096 tokens: compaction re-reads scores from memory and
    stages metadata; the first step evicts thousands of tokens."""
    cfg = _cfg("long", 1, 2, 5, 1, 128, 900, 5000, 600, 1200, 16, 64)
    assert cfg.cap > 4096
    print("[parity] long cache", flush=True)
    run = Run(cfg, seed=8)
    events = sum(run.step(i) for i in range(6))
    assert events > 0


def test_parity_plan_and_move_kernels_path():
    """Capacity between the single-kernel limit (2560 slots) and 4096: the
    plan kernel selects from registers and a second kernel moves the rows."""
    cfg = _cfg("mid", 1, 2, 5, 1, 128, 700, 3000, 500, 1000, 16, 64)
    assert 2560 < cfg.cap <= 4096
    print("[parity] plan + move kernels", flush=True)
    run = Run(cfg, seed=6)
    events = sum(run.step(i) for i in range(6))
    assert events > 0


@pytest.mark.parametrize("case", ["regs", "long", "long_block"])
def test_selection_with_tied_scores(case):
    """Crafted scores with heavy ties (same array on both sides), so that the
    k-th key falls inside a large group of equal scores and the position
    tie-break decides. The long cases (capacity above 4096: the plan rewrites
    the metadata in place after staging it) put the tie boundary below the
    kept count, where the rewritten slots are destinations of survivors."""
    if case == "regs":
        cfg = TINY["g5_d128"]
    elif case == "long":
        cfg = _cfg("tie_long", 1, 2, 5, 1, 128, 900, 5000, 600, 1200, 16, 64)
    else:
        cfg = _block_cfg(_cfg("tie_long", 1, 2, 5, 1, 128, 900, 5000, 600, 1200, 16, 64), 32)
    print(f"[parity] tied scores {case}", flush=True)
    run = Run(cfg, seed=4)
    rng = np.random.default_rng(9)
    for i in range(8):
        s = (rng.integers(0, 3, size=(cfg.layers, cfg.batch, cfg.cap)) / 2.0).astype(np.float32)
        run.step(i, scores=s)


def _fill_cfg(cfg, **pol):
    from dataclasses import replace
    return cfg.with_(name=f"{cfg.name}_fill", policy=replace(cfg.policy, order=1, **pol))


@pytest.mark.parametrize("case", ["regs", "long"])
def test_parity_token_eviction_fill_order(case):
    """Token eviction with the hole-filling option (pol.order = 1): the INT8
    holes below the new INT8 length take the INT8 tail in slot order; every
    cache byte against the oracle's fill compaction."""
    if case == "regs":
        cfg = _fill_cfg(TINY["g5_d128"])
        steps = 24
    else:
        cfg = _fill_cfg(_cfg("fl_long", 1, 2, 5, 1, 128, 900, 5000, 600, 1200, 16, 64))
        assert cfg.cap > 4096
        steps = 8
    print(f"[parity] fill order {case} cap={cfg.cap}", flush=True)
    run = Run(cfg, seed=17)
    events = sum(run.step(i) for i in range(steps))
    assert events > 0
    assert run.band <= 1


@pytest.mark.parametrize("case", ["long", "protect_above_window"])
def test_parity_stable_order_positions_ascending(case):
    """The default, stable survivor order: both parts keep position order
    after every step (checked on every (layer, sequence), beside the
    byte-for-byte comparison with the oracle); also with a protected window
    larger than the FP16 window, which only this order accepts, and on a
    cache above 4096 slots (long-form plan, lists in the workspace)."""
    if case == "long":
        cfg = _cfg("st_long", 1, 2, 5, 1, 128, 900, 5000, 600, 1200, 16, 64)
        assert cfg.cap > 4096
        steps = 8
    else:
        cfg = _cfg("st_pw", 2, 2, 4, 2, 64, 500, 200, 60, 120, 24, 16)
        steps = 40
    print(f"[parity] stable order {case} cap={cfg.cap}", flush=True)
    run = Run(cfg, seed=17)
    events = 0
    for i in range(steps):
        events += run.step(i)
        for (l, b) in run.pairs:
            p = run.eng.cache.snapshot(l, b)["pos"]
            assert (np.diff(p) > 0).all(), (i, l, b)
    assert events > 0
    assert run.band <= 1


def _block_cfg(cfg, block):
    from dataclasses import replace
    return cfg.with_(name=f"{cfg.name}_block{block}", policy=replace(cfg.policy, block=block))


@pytest.mark.parametrize("case", ["regs", "long"])
def test_parity_block_eviction(case):
    """Whole blocks leave (block eviction): survivors, counts and every cache
    byte against the oracle, on the register-held plan path and on the long
    cache path (capacity above 4096)."""
    if case == "regs":
        cfg = _block_cfg(_cfg("blk", 2, 2, 10, 2, 128, 700, 400, 96, 200, 16, 48), 16)
        steps = 40
    else:
        cfg = _block_cfg(_cfg("blk_long", 1, 2, 5, 1, 128, 900, 5000, 600, 1200, 16, 64), 32)
        assert cfg.cap > 4096
        steps = 40
    print(f"[parity] {cfg.name} steps={steps}", flush=True)
    run = Run(cfg, seed=12)
    events = sum(run.step(i) for i in range(steps))
    ev = run.eng.evicted.cpu().numpy()
    assert events > 2 and np.all(ev % cfg.policy.block == 0)


def test_block_eviction_with_tied_block_maxima():
    """Crafted scores whose block maxima tie across blocks (same array on both
    sides): the older block leaves first, bit-exactly as in the oracle."""
    cfg = _block_cfg(TINY["g5_d128"], 16)
    print("[parity] tied block maxima", flush=True)
    run = Run(cfg, seed=4)
    rng = np.random.default_rng(19)
    nblk = cfg.cap // 16 + 1
    for i in range(24):
        top = rng.integers(0, 3, size=(cfg.layers, cfg.batch, nblk)) / 2.0
        s = np.repeat(top, 16, axis=2)[:, :, : cfg.cap]
        s = s - 0.25 * rng.integers(0, 2, size=s.shape)   # most blocks keep their top value
        run.step(i, scores=s.astype(np.float32))


@pytest.mark.parametrize("prefill", [4095, 4096])
def test_parity_register_and_long_plan_boundary(prefill):
    """Capacity 4096 (the last one whose plan keeps keys in registers) and
    4097 (the first on the long-cache path)."""
    cfg = _cfg(f"cap_edge_{prefill}", 1, 2, 5, 1, 128, 600, prefill, 400, 800, 16, 64)
    assert cfg.cap == prefill + 1
    print(f"[parity] plan path edge cap={cfg.cap}", flush=True)
    run = Run(cfg, seed=21)
    events = sum(run.step(i) for i in range(4))
    assert events > 0


def test_parity_protect_equals_window():
    """P = W, the largest protected window token eviction accepts."""
    cfg = _cfg("p_eq_w", 2, 2, 10, 2, 128, 500, 300, 64, 120, 32, 32)
    print("[parity] protect == window", flush=True)
    run = Run(cfg, seed=22)
    events = sum(run.step(i) for i in range(30))
    assert events > 0


def test_parity_block_eviction_d64():
    cfg = _block_cfg(_cfg("blk64", 2, 2, 4, 4, 64, 700, 400, 96, 200, 16, 48), 16)
    print("[parity] block eviction d64", flush=True)
    run = Run(cfg, seed=23)
    events = sum(run.step(i) for i in range(30))
    assert events > 2


def test_no_free_slot_sets_status_and_leaves_the_sequence_alone():
    """A (layer, sequence) whose metadata leaves no slot for the new token
    (forced from the host: n = cap) is flagged with CONFK_STATUS_CAPACITY by
    every call and left as it is; the other sequences step normally."""
    import mixed_precision_attention_amd as M
    dev = _dev()
    cfg = TINY["g5_d128"]
    kp, vp = synth.prefill_kv(cfg, 5)
    eng = M.DecodeEngine(cfg, dev)
    eng.prefill(_t(kp, dev), _t(vp, dev))
    twin = M.DecodeEngine(cfg, dev)
    twin.prefill(_t(kp, dev), _t(vp, dev))
    for i in range(3):
        logits, q, kn, vn, t = _inputs(cfg, 5, i)
        for e in (eng, twin):
            e.step(_t(logits, dev), _t(q, dev), _t(kn, dev), _t(vn, dev), t)
    torch.cuda.synchronize()
    bad = eng.cache.meta[1, 0].clone()
    bad[M.META_N], bad[M.META_N8] = cfg.cap, 0
    eng.cache.meta[1, 0] = bad
    print("[capacity] forced n = cap on (1, 0)", flush=True)
    logits, q, kn, vn, t = _inputs(cfg, 5, 3)
    for e in (eng, twin):
        e.step(_t(logits, dev), _t(q, dev), _t(kn, dev), _t(vn, dev), t)
    torch.cuda.synchronize()
    assert int(eng.cache.status.cpu()[0]) & M.STATUS_CAPACITY
    assert int(twin.cache.status.cpu()[0]) == 0
    after = eng.cache.meta[1, 0].cpu().numpy()
    for w in (M.META_N, M.META_N8, M.META_BASE8, M.META_BASE16):
        assert after[w] == bad.cpu().numpy()[w]
    # every other (layer, sequence) matches the twin that never saw the fault
    for l in range(cfg.layers):
        for b in range(cfg.batch):
            if (l, b) != (1, 0):
                assert torch.equal(eng.cache.meta[l, b], twin.cache.meta[l, b])
                assert torch.equal(eng.cache.pos[l, b], twin.cache.pos[l, b])
                assert torch.equal(eng.cache.k8[l, b], twin.cache.k8[l, b])
                assert torch.equal(eng.cache.k16[l, b], twin.cache.k16[l, b])


def test_confidence_closed_forms_and_flags():
    import mixed_precision_attention_amd as M
    dev = _dev()
    V, B = 152064, 8
    rng = np.random.default_rng(3)
    z = np.zeros((B, V), np.float32)
    z[0] = 1.25                                          # uniform
    z[1] = -np.inf; z[1, 777] = 3.0                       # one-hot
    z[2] = -np.inf; z[2, [5, 9, 100]] = 0.5               # 3-way tie
    z[3] = rng.standard_normal(V) * 8
    z[4] = rng.standard_normal(V) * 0.5
    z[5] = rng.standard_normal(V); z[5, 17] = np.nan      # flagged
    z[6] = -np.inf                                        # flagged
    z[7] = rng.standard_normal(V); z[7, 3] = np.inf       # flagged
    pol = M.make_policy(synth.Policy(n_high=1024, n_low=2048))
    c = torch.zeros(B, device=dev)
    bud = torch.zeros((1, B), dtype=torch.int32, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = torch.zeros(M.engine.workspace_bytes(M._lib.WS_CONFIDENCE, batch=B, vocab=V),
                     dtype=torch.uint8, device=dev)
    M.confidence(_t(z, dev), pol, c, bud, st, ws)
    torch.cuda.synchronize()
    c = c.cpu().numpy()
    bud = bud.cpu().numpy()[0]
    assert abs(c[0] - (0.15 + 0.3 / V)) <= ATOL
    assert abs(c[1] - 1.0) <= ATOL
    assert abs(c[2] - (0.4 * (1 - np.log(3) / np.log(V)) + 0.15 + 0.1)) <= ATOL
    for b in (3, 4):
        assert abs(c[b] - O.confidence(z[b])[0]) <= ATOL
    assert np.isnan(c[5:]).all() and (bud[5:] == 2048).all()
    assert int(st.cpu()[0]) & M.STATUS_NONFINITE_LOGITS
    for b in range(5):
        assert bud[b] == O.budget(O.confidence(z[b])[0], 0.7, 1024, 2048)


@pytest.mark.parametrize("V", [7, 4096, 4097, 50257])
def test_confidence_ragged_vocab(V):
    import mixed_precision_attention_amd as M
    dev = _dev()
    B = 5
    rng = np.random.default_rng(V)
    z = (rng.standard_normal((B, V + 3)) * rng.choice([0.5, 2, 8], size=(B, 1))).astype(np.float32)
    pol = M.make_policy(synth.Policy())
    c = torch.zeros(B, device=dev)
    bud = torch.zeros((1, B), dtype=torch.int32, device=dev)
    ws = torch.zeros(M.engine.workspace_bytes(M._lib.WS_CONFIDENCE, batch=B, vocab=V),
                     dtype=torch.uint8, device=dev)
    zt = _t(z, dev)[:, :V]   # row stride V+3 (ld > vocab)
    M.confidence(zt, pol, c, bud, None, ws)
    torch.cuda.synchronize()
    for b in range(B):
        assert abs(float(c[b]) - O.confidence(z[b, :V])[0]) <= ATOL


def test_qwen32b_shape_two_layers():
    cfg = synth.get_config("qwen32b").with_(layers=2)
    print(f"[parity] qwen32b 2 layers cap={cfg.cap}", flush=True)
    run = Run(cfg, seed=1, pairs=[(0, 0), (0, 5), (1, 3), (1, 7)], device_prefill=True)
    for i in range(3):
        run.step(i)


@pytest.mark.parametrize("name", ["qwen32b", "qwen32b_fill", "qwen32b_block128", "qwen32b_pyramid",
                                  "qwen32b_sw512", "qwen14b"])
def test_full_launch_sampled(name):
    """Every layer of a benchmarked workload in the benchmark's launch
    configuration: the Qwen-32B shape at batch 8 (token eviction with either
    survivor order, 128-token block eviction, the recency-only sliding
    window of 512), the long-context pyramid at batch 1 after a 32768-token
    prefill (the first step evicts down to the per-layer budgets), and the
    Qwen-14B shape after an 8192-token prefill (scores spill past shared
    memory); three (layer, sequence) pairs checked against the oracle."""
    cfg = synth.get_config(name)
    L, B = cfg.layers, cfg.batch
    print(f"[parity] {name} full cap={cfg.cap} block={cfg.policy.block} order={cfg.policy.order}", flush=True)
    run = Run(cfg, seed=2, pairs=[(0, 0), (L // 2, min(4, B - 1)), (L - 1, B - 1)], device_prefill=True)
    for i in range(4):
        run.step(i)


@pytest.mark.parametrize("name,steps", [("qwen32b_pyramid", 96), ("qwen14b", 48)])
def test_long_prefill_workloads_longer_runs(name, steps):
    """The long-prefill workloads at full size over more decode steps: the
    batch-1 pyramid (64 layers, per-layer budgets, 32768-token prefill) and
    the Qwen-14B shape (48 layers x batch 8, 8192-token prefill), three
    (layer, sequence) pairs followed by the oracle after every step, past
    the first large eviction into steady one-token steps."""
    cfg = synth.get_config(name)
    L, B = cfg.layers, cfg.batch
    print(f"[parity] {name} full size, {steps} steps", flush=True)
    run = Run(cfg, seed=4, pairs=[(0, 0), (L // 2, B // 2), (L - 1, B - 1)], device_prefill=True)
    events = 0
    for i in range(steps):
        events += run.step(i)
    assert events > 0


def test_qwen32b_full_size_free_run():
    """The throughput workload at full size (64 layers x batch 8) over its
    first 160 decode steps after the prefill (the window the short benchmark
    measures, with first evictions of about 1000 tokens, then one token per
    step with stable packing into the steady state), five (layer, sequence)
    pairs followed by the oracle after every step."""
    cfg = synth.get_config("qwen32b")
    L, B = cfg.layers, cfg.batch
    print(f"[parity] qwen32b full size, 160 steps", flush=True)
    run = Run(cfg, seed=9, pairs=[(0, 0), (13, 3), (31, 7), (48, 1), (L - 1, B - 3)], device_prefill=True)
    events = sum(run.step(i) for i in range(160))
    assert events > 0
    assert run.band <= 2


def test_full_kv_comparison_run_sampled():
    """The full FP16 comparison run at its size (64 layers x batch 8, a
    2048-token prefill, window and budget 6144 for its 4096 generated
    tokens): attention without the per-key mass over an all-FP16 cache, the
    rank call without mass (the new token's metadata slot only), then the
    append; nothing is evicted or quantised. Three (layer, sequence) pairs
    checked against the oracle, every cache byte, positions and the EMA (zero
    throughout: no mass is accumulated in this run)."""
    import mixed_precision_attention_amd as M
    dev = _dev()
    cfg = synth.get_config("qwen32b_fullkv")
    L, B = cfg.layers, cfg.batch
    print(f"[parity] qwen32b_fullkv full cap={cfg.cap}", flush=True)
    eng = M.DecodeEngine(cfg, dev)
    kp, vp = synth.gen.prefill_kv_device(cfg, 4, dev)
    eng.prefill(kp, vp)
    pairs = [(0, 0), (L // 2, 4), (L - 1, B - 1)]
    orc = {(l, b): O.prefill(kp[l, b].cpu().numpy(), vp[l, b].cpu().numpy(), cfg.policy.window)
           for (l, b) in pairs}
    del kp, vp
    for i in range(4):
        logits, q, kn, vn, t = _inputs(cfg, 4, i)
        eng.step(_t(logits, dev), _t(q, dev), _t(kn, dev), _t(vn, dev), t)
        torch.cuda.synchronize()
        assert int(eng.cache.status.cpu()[0]) == 0, "device status set"
        out = eng.out.float().cpu().numpy()
        for (l, b) in pairs:
            w = f"step {i} l={l} b={b}"
            o, _ = O.attention(q[l, b], orc[(l, b)], kn[l, b], vn[l, b])
            assert rel_maxabs(out[l, b], o) <= OTOL, f"{w}: attention output"
            orc[(l, b)] = O.append(orc[(l, b)], kn[l, b], vn[l, b], t, 0.0)
            assert not orc[(l, b)].is8.any()
            assert_state_equal(eng.cache.snapshot(l, b), orc[(l, b)], what=w)


def test_parity_many_heads_multi_round_moves():
    """16 kv heads of d128 and a large first eviction: the compaction moves
    take several rounds of the single-kernel path."""
    cfg = _cfg("h16_d128", 1, 2, 16, 16, 128, 400, 600, 96, 200, 16, 48)
    print("[parity] h16_d128 multi-round moves", flush=True)
    run = Run(cfg, seed=5)
    events = sum(run.step(i) for i in range(6))
    assert events > 0


@pytest.mark.parametrize("d", [64, 128])
def test_many_movers_in_both_rings(d):
    """Crafted uniform scores scatter the evictions over the whole cache, so
    the first step fills about 250 INT8 holes (several passes of the fill
    loop) and packs about a hundred FP16 rows per ring (several rounds)."""
    import mixed_precision_attention_amd as M
    hq, hkv = (4, 4) if d == 64 else (10, 2)
    cfg = _cfg(f"many_movers_d{d}", 1, 2, hq, hkv, d, 500, 1200, 600, 900, 16, 200)
    print(f"[parity] many movers d{d}", flush=True)
    run = Run(cfg, seed=13)
    rng = np.random.default_rng(31)
    for i in range(3):
        s = rng.random((cfg.layers, cfg.batch, cfg.cap)).astype(np.float32)
        run.step(i, scores=s)
        if i == 0:
            meta = run.eng.cache.meta.cpu().numpy()
            moved8, moved16 = meta[..., M.META_MOVED].max(), meta[..., M.META_MOVED16].max()
            assert moved8 > 200 and moved16 > 64, (moved8, moved16)


FUSED_CASES = {
    # the default, stable order: select, pack, move, append and window step in one kernel
    "g5_d128": lambda: TINY["g5_d128"],
    # empty start: the window step calibrates the scales inside the fused kernel
    "g3_d64_empty": lambda: TINY["g3_d64_empty"],
    # block eviction: the window step is a third launch after the move kernel
    "g5_d128_block16": lambda: _block_cfg(TINY["g5_d128"], 16),
    # token eviction in the hole-filling order (one kernel too)
    "g5_d128_fill": lambda: _fill_cfg(TINY["g5_d128"]),
    # more than 4096 slots: the long-cache plan form
    "long_cache": lambda: _cfg("long_cache", 1, 2, 4, 2, 64, 300, 4200, 1500, 3000, 16, 64),
}


def _assert_same_state(a, b):
    """Two engines hold the same cache and step outputs, bit for bit. EMA and
    position slots past the new length (evicted tokens) are not part of the
    state: the fused call leaves them."""
    import mixed_precision_attention_amd as M
    for name in ("meta", "k8", "v8", "k16", "v16", "kscale", "vscale", "status"):
        assert torch.equal(getattr(a.cache, name), getattr(b.cache, name)), name
    nlen = a.cache.meta[..., M.META_N].cpu().numpy()
    for l in range(nlen.shape[0]):
        for bb in range(nlen.shape[1]):
            n = int(nlen[l, bb])
            for name in ("ema", "pos"):
                x, y = getattr(a.cache, name)[l, bb, :n], getattr(b.cache, name)[l, bb, :n]
                assert torch.equal(x, y), (name, l, bb)
    for name in ("c", "budget", "out", "mass", "score"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name


def _split_step(e, lg, q, kn, vn, t):
    """The five calls in sequence; returns how many sequences the window step
    moved a token for."""
    import mixed_precision_attention_amd as M
    e.step_confidence(lg)
    e.step_attention(q, kn, vn)
    e.step_ema_rank(t)
    e.step_compact(kn, vn)
    n8 = e.cache.meta[..., M.META_N8].clone()
    e.step_quantize(t)
    return int((e.cache.meta[..., M.META_N8] > n8).sum())


def test_qwen32b_full_launch_fused_matches_split():
    """DecodeEngine.step (the whole-step call on one stream as bench.py times
    it: the confidence pass inside the attention launch, the merge and the
    budgets in the fused EMA + compaction + window-step launch; and with the
    confidence on a second stream) against
    the five calls issued one after another, bit for bit, at the full
    64-layer, batch-8 size (the split calls themselves are checked against
    the oracle at this size above)."""
    import mixed_precision_attention_amd as M
    dev = _dev()
    cfg = synth.get_config("qwen32b")
    print(f"[parity] qwen32b full fused vs split cap={cfg.cap}", flush=True)
    engs = [M.DecodeEngine(cfg, dev), M.DecodeEngine(cfg, dev, overlap=True), M.DecodeEngine(cfg, dev)]
    kp, vp = synth.gen.prefill_kv_device(cfg, 2, dev)
    for e in engs:
        e.prefill(kp, vp)
    del kp, vp
    quantised = 0
    for i in range(8):
        lg = synth.gen.logits_device(cfg, 2, i, dev)
        q, kn, vn = synth.gen.decode_inputs_device(cfg, 2, i, dev)
        t = cfg.prefill + i
        engs[0].step(lg, q, kn, vn, t)
        engs[1].step(lg, q, kn, vn, t)
        quantised += _split_step(engs[2], lg, q, kn, vn, t)
    torch.cuda.synchronize()
    assert quantised > 0
    _assert_same_state(engs[0], engs[2])
    _assert_same_state(engs[1], engs[2])


@pytest.mark.parametrize("case", list(FUSED_CASES))
def test_overlapped_step_matches_serial(case):
    """DecodeEngine.step (confidence on a second stream, EMA, compaction and
    the window step in one fused call) leaves exactly the state of the five
    calls issued one after another on one stream. EMA and position slots past
    the new length (evicted tokens) are not part of the state: the fused call
    leaves them."""
    import mixed_precision_attention_amd as M
    dev = _dev()
    cfg = FUSED_CASES[case]()
    engs = [M.DecodeEngine(cfg, dev, overlap=True), M.DecodeEngine(cfg, dev, overlap=False)]
    if cfg.prefill:
        kp, vp = synth.prefill_kv(cfg, 3)
        for e in engs:
            e.prefill(_t(kp, dev), _t(vp, dev))
    else:
        for e in engs:
            e.prefill(None, None)
    steps = 20 if cfg.prefill else cfg.policy.window + 24  # past the first calibration
    quantised = 0
    for i in range(steps):
        logits, q, kn, vn, t = _inputs(cfg, 3, i)
        lg, qd, kd, vd = _t(logits, dev), _t(q, dev), _t(kn, dev), _t(vn, dev)
        engs[0].step(lg, qd, kd, vd, t)
        quantised += _split_step(engs[1], lg, qd, kd, vd, t)
    torch.cuda.synchronize()
    assert quantised > 0  # the window step moved tokens
    _assert_same_state(*engs)


def test_attention_without_mass_gives_the_same_output():
    """mass = NULL (no score store, no mass pass) gives the same output to the
    attention tolerance (the compiler may order the arithmetic differently)."""
    import mixed_precision_attention_amd as M
    dev = _dev()
    cfg = TINY["g5_d128"]
    kp, vp = synth.prefill_kv(cfg, 3)
    eng = M.DecodeEngine(cfg, dev)
    eng.prefill(_t(kp, dev), _t(vp, dev))
    for i in range(3):
        logits, q, kn, vn, t = _inputs(cfg, 3, i)
        lg, qd, kd, vd = _t(logits, dev), _t(q, dev), _t(kn, dev), _t(vn, dev)
        eng.step_confidence(lg)
        eng.step_attention(qd, kd, vd)
        with_mass = eng.out.clone()
        M.engine.attn_decode(eng.cache, qd, kd, vd, eng.out, None, None)
        torch.cuda.synchronize()
        for l in range(cfg.layers):
            for b in range(cfg.batch):
                got = eng.out[l, b].float().cpu().numpy()
                ref = with_mass[l, b].float().cpu().numpy()
                assert rel_maxabs(got, ref) <= OTOL / 2, f"step {i} l={l} b={b}"
        eng.step_ema_rank(t)
        eng.step_compact(kd, vd)
        eng.step_quantize(t)


def test_two_kv_heads_per_workgroup_mass_rows():
    """At the Qwen-32B shape and batch 8 the launch's 4096 units fill more
    than two rounds of resident workgroups, so attention runs two kv heads
    per workgroup and sums their mass in one row, except in the workgroups
    of the last round of dispatch, which run one kv head each (so the launch
    drains sooner). A (layer, sequence)'s R rows (its metadata word, between
    hkv / 2 and hkv) are sums over consecutive runs of one or two of its kv
    heads, in head order. A launch over one layer (64 units) writes one row
    per kv head. Each row equals the sum of its heads' rows to fp32
    rounding, and the output is the same."""
    import mixed_precision_attention_amd as M
    dev = _dev()
    cfg = synth.get_config("qwen32b")
    H = cfg.hkv
    eng = M.DecodeEngine(cfg, dev)
    kp, vp = synth.gen.prefill_kv_device(cfg, 5, dev)
    eng.prefill(kp, vp)
    del kp, vp
    for s in range(3):  # mixed lengths: the first steps evict to either budget
        lg = synth.gen.logits_device(cfg, 5, s, dev)
        q, kn, vn = synth.gen.decode_inputs_device(cfg, 5, s, dev)
        eng.step(lg, q, kn, vn, cfg.prefill + s)
    q, kn, vn = synth.gen.decode_inputs_device(cfg, 5, 3, dev)
    M.engine.attn_decode(eng.cache, q, kn, vn, eng.out, eng.mass, eng.attn_ws)
    torch.cuda.synchronize()
    rows = eng.cache.mass_rows()
    assert rows.min() >= H // 2 and rows.max() <= H
    assert (rows == H // 2).mean() > 0.5, "most (layer, sequence) pairs run two kv heads per workgroup"
    out_all, mass_all = eng.out.clone(), eng.mass.clone()
    n = eng.cache.lengths()[0]
    for l in (0, 37, cfg.layers - 1):
        # the workspace without the split exchange area: one workgroup per
        # kv head, no split keys
        M.engine.attn_decode(eng.cache, q[l:], kn[l:], vn[l:], eng.out[l:], eng.mass[l:], _nosplit_ws(eng, 1),
                             layer0=l, nlayers=1)
        torch.cuda.synchronize()
        assert (eng.cache.mass_rows()[l] == H).all()
        for b in range(cfg.batch):
            k = int(n[l, b]) + 1
            R = int(rows[l, b])
            per_head = eng.mass[l, b, :, :k].double().cpu().numpy()
            summed = mass_all[l, b, :R, :k].double().cpu().numpy()
            tol = 1e-6 * max(1.0, np.abs(per_head).sum(axis=0).max())
            j = 0  # next kv head: each row is head j alone or heads j and j + 1
            for r in range(R):
                if j < H and np.abs(summed[r] - per_head[j]).max() <= tol:
                    j += 1
                elif j + 1 < H and np.abs(summed[r] - per_head[j] - per_head[j + 1]).max() <= tol:
                    j += 2
                else:
                    raise AssertionError(f"l={l} b={b}: row {r} is not kv head {j} or heads {j}, {j + 1}")
            assert j == H, f"l={l} b={b}: rows cover {j} of {H} kv heads"
            got = out_all[l, b].float().cpu().numpy()
            ref = eng.out[l, b].float().cpu().numpy()
            assert rel_maxabs(got, ref) <= OTOL / 2, f"l={l} b={b}: output"
    print(f"mass rows per (layer, sequence): {np.bincount(rows.reshape(-1), minlength=H + 1)[H // 2:].tolist()} "
          f"for R = {H // 2}..{H}")


def test_two_kv_heads_per_workgroup_wide_groups():
    """Sixteen query heads per kv head (d = 128): a unit's output (2048
    halves) is too large to be held in registers until the second unit's tile
    loops are done, so the first unit of a two-head workgroup stores it
    directly. 24 layers x batch 8 x 8 kv heads fill two rounds of resident
    workgroups, so the launch runs two kv heads per workgroup; its output
    equals the one-layer launches' (one kv head per workgroup) bit for bit,
    and its mass rows are sums of runs of one or two kv heads' rows."""
    import mixed_precision_attention_amd as M
    dev = _dev()
    cfg = _cfg("g16_pairs", 24, 8, 128, 8, 128, 1000, 300, 96, 200, 16, 64)
    H = cfg.hkv
    eng = M.DecodeEngine(cfg, dev)
    kp, vp = synth.gen.prefill_kv_device(cfg, 3, dev)
    eng.prefill(kp, vp)
    del kp, vp
    for s in range(2):
        lg = synth.gen.logits_device(cfg, 3, s, dev)
        q, kn, vn = synth.gen.decode_inputs_device(cfg, 3, s, dev)
        eng.step(lg, q, kn, vn, cfg.prefill + s)
    q, kn, vn = synth.gen.decode_inputs_device(cfg, 3, 2, dev)
    print(f"[parity] g16 pairs: {cfg.layers * cfg.batch * H} units", flush=True)
    M.engine.attn_decode(eng.cache, q, kn, vn, eng.out, eng.mass, eng.attn_ws)
    torch.cuda.synchronize()
    rows = eng.cache.mass_rows()
    assert rows.min() >= H // 2 and (rows < H).any(), "the launch runs two kv heads per workgroup"
    out_all, mass_all = eng.out.clone(), eng.mass.clone()
    n = eng.cache.lengths()[0]
    for l in (0, 11, cfg.layers - 1):
        # the workspace without the split exchange area: one workgroup per
        # kv head, no split keys
        M.engine.attn_decode(eng.cache, q[l:], kn[l:], vn[l:], eng.out[l:], eng.mass[l:], _nosplit_ws(eng, 1),
                             layer0=l, nlayers=1)
        torch.cuda.synchronize()
        assert torch.equal(out_all[l], eng.out[l]), f"l={l}: output"
        for b in range(cfg.batch):
            k = int(n[l, b]) + 1
            per_head = eng.mass[l, b, :, :k].double().cpu().numpy()
            summed = mass_all[l, b, :int(rows[l, b]), :k].double().cpu().numpy()
            tol = 1e-6 * max(1.0, np.abs(per_head).sum(axis=0).max())
            j = 0
            for r in range(summed.shape[0]):
                for m in (1, 2):
                    if j + m <= H and np.abs(summed[r] - per_head[j:j + m].sum(axis=0)).max() <= tol:
                        j += m
                        break
                else:
                    raise AssertionError(f"l={l} b={b}: row {r} is no run of 1 or 2 kv heads from {j}")
            assert j == H, f"l={l} b={b}: rows cover {j} of {H} kv heads"


@pytest.mark.parametrize("choice", ["none", "greedy", "sample"])
def test_fused_confidence_attention_matches_split(choice):
    """confk_confidence_attn_decode (the confidence merge inside the attention
    launch; with sampling the confidence call's own final kernel) against
    confk_confidence then confk_attn_decode, bit for bit: c, budgets, the
    next token, the output and the mass, at the Qwen-32B shape with two
    layers and at a small shape with a ragged vocabulary."""
    import mixed_precision_attention_amd as M
    dev = _dev()
    # (the last shape's launches split keys: the merge workgroups lead the split units)
    for cfg in (synth.get_config("qwen32b").with_(layers=2), TINY["g5_d128"], SPLIT_CASES["g16_d128"]):
        engs = [M.DecodeEngine(cfg, dev), M.DecodeEngine(cfg, dev)]
        kp, vp = synth.prefill_kv(cfg, 6)
        for e in engs:
            e.prefill(_t(kp, dev), _t(vp, dev))
        for i in range(3):
            logits, q, kn, vn, t = _inputs(cfg, 6, i)
            lg, qd, kd, vd = _t(logits, dev), _t(q, dev), _t(kn, dev), _t(vn, dev)
            temp = None if choice == "none" else (0.0 if choice == "greedy" else 0.8)
            u = torch.rand(cfg.batch, generator=torch.Generator().manual_seed(i)).to(dev)
            engs[0].step_confidence(lg, temperature=temp, uniform=u)
            engs[0].step_attention(qd, kd, vd)
            engs[1].step_confidence_attention(lg, qd, kd, vd, temperature=temp, uniform=u)
            torch.cuda.synchronize()
            for name in ("c", "budget", "out", "mass"):
                assert torch.equal(getattr(engs[0], name), getattr(engs[1], name)), (cfg.name, i, name)
            if temp is not None:
                assert torch.equal(engs[0].token, engs[1].token), (cfg.name, i, "token")
            assert torch.equal(engs[0].cache.meta, engs[1].cache.meta)
            for e in engs:
                e.step_ema_compact(t, kd, vd, fuse_quantize=True)


@pytest.mark.parametrize("choice", ["none", "greedy", "sample"])
def test_decode_step_matches_split(choice):
    """confk_decode_step (the confidence pass in the attention launch's last
    workgroups, the merge and the budget in the plan kernel; with sampling
    the confidence call's own kernels) against the five calls one after
    another, bit for bit over several steps: the whole cache, c, budgets, the
    next token, output, mass and scores. Shapes: the Qwen-32B shape with two
    layers, a small ragged one from an empty cache (the window step
    calibrates), per-layer (pyramid) budgets, and a launch that splits keys
    (the confidence pass's workgroups follow the split units)."""
    import mixed_precision_attention_amd as M
    dev = _dev()
    lo = (60, 52, 44)
    cases = (synth.get_config("qwen32b").with_(layers=2), TINY["g3_d64_empty"],
             _cfg("pyr", 3, 2, 10, 2, 128, 600, 120, max(lo) // 2, max(lo), 8, 24,
                  layer_n_low=lo, layer_n_high=tuple(x // 2 for x in lo)),
             SPLIT_CASES["mha_d64"])
    for cfg in cases:
        engs = [M.DecodeEngine(cfg, dev), M.DecodeEngine(cfg, dev)]
        if cfg.prefill:
            kp, vp = synth.prefill_kv(cfg, 7)
            for e in engs:
                e.prefill(_t(kp, dev), _t(vp, dev))
        temp = None if choice == "none" else (0.0 if choice == "greedy" else 0.8)
        steps = 8 if cfg.prefill else 40
        for i in range(steps):
            logits, q, kn, vn, t = _inputs(cfg, 7, i)
            lg, qd, kd, vd = _t(logits, dev), _t(q, dev), _t(kn, dev), _t(vn, dev)
            u = torch.rand(cfg.batch, generator=torch.Generator().manual_seed(i)).to(dev)
            e = engs[0]
            e.step_confidence(lg, temperature=temp, uniform=u)
            e.step_attention(qd, kd, vd)
            e.step_ema_rank(t)
            e.step_compact(kd, vd)
            e.step_quantize(t)
            f = engs[1]
            M.engine.decode_step(lg, f.pol, f.c, f.budget, f.cache, t, qd, kd, vd, f.out, f.mass, f.score,
                                 f.conf_ws, f.attn_ws, f.compact_ws, f.layer_n_high, f.layer_n_low,
                                 token_out=None if temp is None else f.token,
                                 temperature=0.0 if temp is None else temp, uniform=u, evicted=f.evicted)
            torch.cuda.synchronize()
            if temp is not None:
                assert torch.equal(e.token, f.token), (cfg.name, i, "token")
        _assert_same_state(engs[0], engs[1])
        assert int(engs[1].cache.status.cpu()[0]) == 0


def test_long_context_pyramid_retains_planted_keys():
    """Long-context pyramid at the Qwen-32B layer shape: a 32768-token prefill,
    the budgets of the first and last layer (4096 and 1024 loose), one planted
    key per sequence at 10/30/50/70/90 % depth that the decode queries align
    with. Sampled pairs follow the oracle; every planted key is kept."""
    base = synth.get_config("qwen32b_niah")
    cfg = base.with_(layers=2, layer_n_low=(base.layer_n_low[0], base.layer_n_low[-1]),
                     layer_n_high=(base.layer_n_high[0], base.layer_n_high[-1]))
    print(f"[parity] long-context pyramid cap={cfg.cap}", flush=True)
    run = Run(cfg, seed=3, pairs=[(0, 0), (1, 2), (1, 4)])
    planted = synth.gen.plant_positions(cfg)
    for i in range(3):
        run.step(i)
        pos = run.eng.cache.pos.cpu().numpy()
        n, _ = run.eng.cache.lengths()
        for l in range(cfg.layers):
            assert (n[l] <= cfg.layer_n_low[l] + 1).all()
            for b in range(cfg.batch):
                assert planted[b] in pos[l, b, : n[l, b]], f"step {i} l={l} b={b}: planted key evicted"


def _conf_buffers(dev, B, V):
    import mixed_precision_attention_amd as M
    pol = M.engine.make_policy(synth.Policy(n_high=1024, n_low=2048))
    c = torch.zeros(B, dtype=torch.float32, device=dev)
    bud = torch.zeros((1, B), dtype=torch.int32, device=dev)
    tok = torch.zeros(B, dtype=torch.int32, device=dev)
    ws = torch.zeros(M.engine.workspace_bytes(M._lib.WS_CONFIDENCE, batch=B, vocab=V), dtype=torch.uint8,
                     device=dev)
    return pol, c, bud, tok, ws


def test_next_token_greedy_and_sampled():
    """Step-13 choice fused into the confidence pass: greedy equals the
    oracle's (smallest index among the largest logits, ties crafted); a
    tempered draw is a token whose cumulative-probability interval holds u
    (to fp32 summation error)."""
    import mixed_precision_attention_amd as M
    dev = _dev()
    for V, ld in ((152064, 152064), (5003, 5008), (1000, 1003)):
        B = 8
        rng = np.random.default_rng(V)
        z = np.zeros((B, ld), np.float32)
        z[:, :V] = rng.standard_normal((B, V)).astype(np.float32) * np.array([0.5, 2, 8, 8, 2, 0.5, 8, 8])[:, None]
        z[3, [7, V - 2]] = z[3, :V].max() + 1.0        # tied maxima: the smaller index wins
        z[6, : V // 2] = -np.inf                        # a block of impossible tokens
        zt = _t(z, dev)[:, :V]
        pol, c, bud, tok, ws = _conf_buffers(dev, B, V)
        M.confidence(zt, pol, c, bud, None, ws, token_out=tok, temperature=0.0)
        torch.cuda.synchronize()
        for b in range(B):
            assert int(tok[b]) == O.next_token(z[b, :V], 0.0), f"V={V} b={b} greedy"
        for T in (0.5, 1.0, 2.0):
            u = rng.random(B).astype(np.float32)
            M.confidence(zt, pol, c, bud, None, ws, token_out=tok, temperature=T, uniform=_t(u, dev))
            torch.cuda.synchronize()
            for b in range(B):
                i = int(tok[b])
                assert 0 <= i < V and np.isfinite(z[b, i]), f"V={V} T={T} b={b}: token {i}"
                lo, hi = O.token_interval(z[b, :V], T, i)
                assert lo - 5e-5 <= float(u[b]) <= hi + 5e-5, f"V={V} T={T} b={b}: u={u[b]} not in [{lo}, {hi}]"
                assert abs(float(c[b]) - O.confidence(z[b, :V])[0]) <= ATOL


def test_next_token_temperature_sweep():
    """The confidence is computed on the untempered distribution; the higher
    the sampling temperature, the less often a confident step emits the token
    the confidence describes (its argmax). Rows follow the workload's logit
    mix (scales 0.5 / 2 / 8)."""
    import mixed_precision_attention_amd as M
    dev = _dev()
    cfg = synth.get_config("gpt2_layer")
    V, B, steps = cfg.vocab, cfg.batch, 96
    pol, c, bud, tok, ws = _conf_buffers(dev, B, V)
    rng = np.random.default_rng(23)
    rates = {}
    for T in (0.0, 0.5, 1.0, 1.5):
        hit = n = 0
        for s in range(steps):
            z = synth.logits_for_step(cfg, 31, s)
            u = rng.random(B).astype(np.float32)
            M.confidence(_t(z, dev), pol, c, bud, None, ws, token_out=tok, temperature=T, uniform=_t(u, dev))
            torch.cuda.synchronize()
            for b in range(B):
                if float(c[b]) >= 0.7:
                    n += 1
                    hit += int(tok[b]) == O.next_token(z[b], 0.0)
        rates[T] = hit / max(n, 1)
    print("[sweep] argmax rate of confident steps by temperature:", rates, flush=True)
    assert rates[0.0] == 1.0
    assert rates[0.5] >= rates[1.0] >= rates[1.5]
    assert rates[1.5] < 0.9
