#!/usr/bin/env python3
"""Throughput of the CONF-KV decode step on one MI355X.

One step = the whole hot path over one batch: confidence + budget, decode
attention with fused INT8 dequantisation and per-key mass, EMA + rank,
eviction + compaction + append, FP16 -> INT8 window quantisation, for every
layer and sequence. Workload: Qwen-32B shape (64 layers, 40 query / 8 KV
heads, d 128), batch 8, 2048-token prefill, V = 152064, N_high/N_low =
1024/2048, P = 64, W = 256; seeded synthetic inputs resident in HBM before
the timed region.

Byte accounting: the steps are deterministic, so an untimed pass from the
same prefill records every step's cache lengths and row moves; the timed
pass replays the same steps. Bytes are the algorithmic bytes of the method
(INT8 codes 2*Hkv*d per token, FP16 rows 4*Hkv*d, scales, q/o, mass,
metadata 16 B/token, moved rows read+write, quantised rows, logits).

Prints one JSON line.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "attn_decode_qwen32b_b8_traffic.md")


def code_sha256(path):
    """SHA-256 of a source file's code: line comments, trailing blanks and
    empty lines dropped, so that a change to the comments alone keeps it."""
    import hashlib
    import re
    lines = []
    for line in open(path, encoding="utf-8"):
        line = re.sub(r"//.*", "", line).rstrip()
        if line:
            lines.append(line)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def counted_traffic(workload):
    """HBM bytes per attention launch from the committed counter summary, or
    None when the summary is missing, covers another workload, or the
    attention code has changed since the counters were taken."""
    try:
        line = [l for l in open(TRAFFIC_SUMMARY) if l.startswith("traffic-json:")][-1]
        rec = json.loads(line.split(":", 1)[1])
        sha = code_sha256(os.path.join(ROOT, rec["source"]))
    except (OSError, IndexError, ValueError, KeyError):
        return None
    if sha != rec.get("source_code_sha256") or rec.get("workload") != workload:
        return None
    return int(rec["traffic_bytes_per_launch"])


def attn_kernel_name(cfg, eng, full, nl=None):
    """Instance of the attention kernel the timed launches ran: spill store
    (the workspace has a spill area), per-key mass (not in the full-cache
    run), the two-kv-heads-per-workgroup mass sum (fewer mass rows than kv
    heads), and split keys (the workspace holds the exchange area, the
    launch has at most 64 units and fills at most 1/32 of the GPU's resident
    workgroup slots, three per compute unit at this kernel's register count,
    and its capacity allows units of at least three 32-tile pieces)."""
    import torch

    import mixed_precision_attention_amd as M
    spill = not full and M.engine.workspace_bytes(M._lib.WS_ATTENTION_NOSPLIT, eng.cache, nlayers=cfg.layers) > 0
    acc = not full and bool((eng.cache.mass_rows() < cfg.hkv).any())
    nl = cfg.layers if nl is None else nl  # layers per attention launch
    units = nl * cfg.batch * cfg.hkv
    slots = 3 * torch.cuda.get_device_properties(0).multi_processor_count
    xchg = eng.attn_ws is not None and M.engine.workspace_bytes(
        M._lib.WS_ATTENTION, eng.cache, nlayers=cfg.layers) > M.engine.workspace_bytes(
        M._lib.WS_ATTENTION_NOSPLIT, eng.cache, nlayers=cfg.layers)
    wmax = (eng.cache.cap + 15) // 16 + 2 * ((eng.cache.cap16 + 15) // 16)  # INT8-tile weight bound of a unit
    split = not full and xchg and units <= 64 and 32 * units <= slots and wmax >= 96
    b = lambda x: "true" if x else "false"  # noqa: E731
    name = f"attn_decode_kernel<{cfg.d}, {b(spill)}, {b(not full)}, {b(acc)}"
    return name + (", true>" if split else ">")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: the workload's generated tokens minus the warmup)")
    ap.add_argument("--warmup", type=int, default=48)
    ap.add_argument("--config", default="qwen32b")
    ap.add_argument("--no-split-keys", action="store_true",
                    help="size the attention workspace without the split exchange area, so every "
                         "attention launch runs one workgroup per unit")
    ap.add_argument("--graph", action="store_true",
                    help="with --per-layer: replay the step's one-layer attention launches as one HIP graph "
                         "(each step's q, k_new, v_new copied into the graph's buffers first)")
    ap.add_argument("--per-layer", action="store_true",
                    help="issue attention as one launch per layer, as a model's forward pass does, instead "
                         "of one launch over all layers (then the confidence pass and the fused EMA + "
                         "compaction + window step launch on their own)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU time budget of the oracle baseline sample (0 disables it)")
    ap.add_argument("--read-ceiling-mib", type=int, default=2048,
                    help="buffer size of the streaming-read ceiling measurement (0 disables it)")
    ap.add_argument("--cpu-full", action="store_true",
                    help="time the oracle over every step of the run instead of a first-step sample "
                         "(small configs)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the run, one plain device copy of this size (counter scaling)")
    return ap.parse_args()


def step_bytes(cfg, n, n8, moved8, moved16, quantised):
    """Algorithmic bytes of one step from the pre-step lengths [L, B]. The
    full-cache comparison run moves K/V, q/o and the appended row only."""
    H, d, Hq = cfg.hkv, cfg.d, cfg.hq
    f = n - n8
    full = cfg.mode == "full_kv"
    attn = (H * d * (2 * n8 + 4 * (f + 1)) + 8 * H * d * (n8 > 0) + 4 * Hq * d + (0 if full else 4 * (n + 1))).sum()
    meta = 0 if full else (16 * n).sum()
    comp = (2 * (moved8 * 2 * H * d + moved16 * 4 * H * d)).sum() + 8 * H * d * n.size
    quant = 6 * H * d * quantised.sum()
    conf = 0 if full else 4 * cfg.batch * cfg.vocab
    return dict(attn=int(attn), meta=int(meta), compact=int(comp), quant=int(quant), conf=int(conf),
                total=int(attn + meta + comp + quant + conf))


def cpu_baseline(cfg, kp, vp, logits0, q0, kn0, vn0, budget_s):
    """Oracle (fp64 numpy) on the first decode step after the prefill, over
    as many (layer, sequence) pairs as fit the time budget; extrapolated to
    the whole step."""
    import numpy as np
    from oracle import confk_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    pol = cfg.policy
    t0 = time.perf_counter()
    cs = [O.confidence(logits0[b])[0] for b in range(cfg.batch)]
    t_conf = time.perf_counter() - t0
    # (layer, sequence) pairs in a seeded order, as many as the budget allows
    order = np.random.default_rng(0).permutation(cfg.layers * cfg.batch)
    pairs = [(int(i) // cfg.batch, int(i) % cfg.batch) for i in order]
    done, t_pairs = 0, 0.0
    for (l, b) in pairs:
        c = O.prefill(kp[l, b].cpu().numpy(), vp[l, b].cpu().numpy(), pol.window)
        N = O.budget(cs[b], pol.tau, pol.n_high, pol.n_low)
        t1 = time.perf_counter()
        O.step_one(c, q0[l, b], kn0[l, b], vn0[l, b], cfg.prefill, pol, N)
        t_pairs += time.perf_counter() - t1
        done += 1
        if t_pairs + t_conf >= budget_s:
            break
    per_step = t_conf + t_pairs / done * cfg.layers * cfg.batch
    return dict(per_step_s=per_step, pairs=done, threads=threads)


def cpu_full(cfg, kp, vp, inputs):
    """Oracle (fp64 numpy) over every step of the run from the prefill, on the
    same inputs (for the small configs, where it finishes in seconds). Host
    copies of the inputs are made before the clock starts."""
    import numpy as np
    from oracle import confk_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    pol = cfg.policy
    host = [(lg.cpu().numpy(), q.cpu().numpy(), kn.cpu().numpy(), vn.cpu().numpy(), t)
            for lg, q, kn, vn, t in inputs]
    lb = (np.asarray(cfg.layer_n_low), np.asarray(cfg.layer_n_high)) if cfg.layer_n_low else None
    caches = [[O.prefill(kp[l, b].cpu().numpy(), vp[l, b].cpu().numpy(), pol.window) if cfg.prefill
               else O.empty_cache(cfg.hkv, cfg.d) for b in range(cfg.batch)] for l in range(cfg.layers)]
    t0 = time.perf_counter()
    for lg, q, kn, vn, t in host:
        caches = O.step(caches, lg, q, kn, vn, t, pol, layer_budgets=lb).caches
    return dict(seconds=time.perf_counter() - t0, threads=threads)


def read_ceiling(dev, mib=2048, reps=10):
    """Streaming-read ceiling: GB/s of the library's read probe (the attention
    kernel's 16-byte streaming loads, whole lines per instruction) over a
    seeded random buffer, untimed warm-up then `reps` launches between two
    events. Outside the timed step loop."""
    import torch
    from mixed_precision_attention_amd import engine as E
    nbytes = mib << 20
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    buf = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=dev, generator=gen)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(2):
        E.read_probe(buf, sink)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    a.record(stream)
    for _ in range(reps):
        E.read_probe(buf, sink)
    b.record(stream)
    torch.cuda.synchronize()
    gbs = nbytes / (a.elapsed_time(b) / reps * 1e-3) / 1e9
    del buf
    return {"value": round(gbs, 1), "unit": "GB/s", "bytes": nbytes, "kernel": "read_probe_kernel",
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus N > 1 is not supported",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import mixed_precision_attention_amd as M
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    cfg = synth.get_config(args.config)
    pol = cfg.policy
    if args.per_layer and cfg.mode == "full_kv":
        print(json.dumps({"error": "--per-layer applies to the method's step, not the full-cache run"}), flush=True)
        sys.exit(2)
    layerwise = args.per_layer
    Wm = args.warmup
    K = args.steps if args.steps is not None else max(1, cfg.steps - Wm)
    S = K + Wm

    # one stream, in a model's order of dependence (the engine can also run the
    # confidence beside the attention on a second stream, which a model whose
    # logits come out of the same step's forward pass could not)
    eng = M.DecodeEngine(cfg, dev, split_keys=not args.no_split_keys)
    kp, vp = synth.gen.prefill_kv_device(cfg, args.seed, dev)
    inputs = []
    for s in range(S):
        lg = synth.gen.logits_device(cfg, args.seed, s, dev)
        q, kn, vn = synth.gen.decode_inputs_device(cfg, args.seed, s, dev)
        inputs.append((lg, q, kn, vn, cfg.prefill + s))
    torch.cuda.synchronize()

    # ---- untimed pass: per-step lengths and moves for the byte count
    eng.prefill(kp, vp)
    per_step = []
    evict_frac = []
    moved_rows = []
    full = cfg.mode == "full_kv"
    for s in range(S):
        lg, q, kn, vn, t = inputs[s]
        m0 = eng.cache.meta.cpu().numpy()
        if full:
            eng.step(lg, q, kn, vn, t)
            m1 = m2 = eng.cache.meta.cpu().numpy()
        else:
            eng.step_confidence(lg)
            eng.step_attention(q, kn, vn)
            eng.step_ema_rank(t)
            eng.step_compact(kn, vn)
            m1 = eng.cache.meta.cpu().numpy()
            eng.step_quantize(t)
            m2 = eng.cache.meta.cpu().numpy()
        evict_frac.append(float((m1[..., M.META_EVICTED] > 0).mean()))
        if s >= Wm:
            ev_mask = m1[..., M.META_EVICTED] > 0
            moved_rows.extend((m1[..., M.META_MOVED] + m1[..., M.META_MOVED16])[ev_mask].tolist())
        per_step.append(step_bytes(
            cfg, m0[..., M.META_N].astype(np.int64), m0[..., M.META_N8].astype(np.int64),
            m1[..., M.META_MOVED].astype(np.int64), m1[..., M.META_MOVED16].astype(np.int64),
            (m2[..., M.META_N8] - m1[..., M.META_N8]).astype(np.int64)))
    torch.cuda.synchronize()
    status = int(eng.cache.status.cpu()[0])
    n_end = eng.cache.meta[..., M.META_N].float()
    len_mean = float(n_end.mean())

    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    stream = torch.cuda.current_stream()

    run_step = eng.step_layerwise if layerwise else eng.step
    graph = None
    if layerwise and args.graph:
        qb, kb, vb = (x.clone() for x in inputs[0][1:4])

        def run_step(lg, q, kn, vn, t):  # noqa: F811  (the graph-replay form of step_layerwise)
            eng.step_confidence(lg)
            qb.copy_(q)
            kb.copy_(kn)
            vb.copy_(vn)
            graph.replay()
            eng.step_ema_compact(t, kn, vn, fuse_quantize=True)

    def replay_to_warm():
        eng.prefill(kp, vp)
        for s in range(Wm):
            lg, q, kn, vn, t = inputs[s]
            run_step(lg, q, kn, vn, t)
        torch.cuda.synchronize()

    # ---- timed pass: the K steps back to back, same steps from the same prefill
    if layerwise and args.graph:  # captured after one eager step (the library's device queries)
        eng.prefill(kp, vp)
        eng.step_layerwise(*inputs[0])
        torch.cuda.synchronize()
        graph = eng.capture_attention_layerwise(qb, kb, vb)
    replay_to_warm()
    start, stop = E(), E()
    start.record(stream)
    for i in range(K):
        lg, q, kn, vn, t = inputs[Wm + i]
        run_step(lg, q, kn, vn, t)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)

    # ---- per-kernel pass: the same steps again, with HIP events around the
    # attention and compaction launches (events between launches add idle gaps,
    # so this pass is not used for the step rate)
    replay_to_warm()
    ev = [(E(), E(), E(), E()) for _ in range(K)]
    lev = [[(E(), E()) for _ in range(cfg.layers)] for _ in range(K)] if layerwise else None
    for i in range(K):
        lg, q, kn, vn, t = inputs[Wm + i]
        a0, a1, c0, c1 = ev[i]
        if not full:
            eng.step_confidence(lg)
        a0.record(stream)
        if full:
            M.engine.attn_decode(eng.cache, q, kn, vn, eng.out, None, None)
        elif layerwise:  # events around each layer's launch
            for l in range(cfg.layers):
                lev[i][l][0].record(stream)
                M.engine.attn_decode(eng.cache, q[l:], kn[l:], vn[l:], eng.out[l:], eng.mass[l:], eng.attn_ws,
                                     layer0=l, nlayers=1)
                lev[i][l][1].record(stream)
        else:
            eng.step_attention(q, kn, vn)
        a1.record(stream)
        if not full:
            eng.step_ema_rank(t)
        else:  # the comparison run's step: the new token's metadata slot only
            M.engine.ema_rank(eng.cache, None, eng.pol, t, eng.score)
        c0.record(stream)
        eng.step_compact(kn, vn)
        c1.record(stream)
        if not full:
            eng.step_quantize(t)
    torch.cuda.synchronize()
    if layerwise:  # the launches' own durations, without the gaps between them
        attn_ms = [sum(x[0].elapsed_time(x[1]) for x in lev[i]) for i in range(K)]
    else:
        attn_ms = [e[0].elapsed_time(e[1]) for e in ev]
    comp_ms = [e[2].elapsed_time(e[3]) for e in ev]

    retention = None
    if cfg.plant_depths:  # planted keys still cached after the timed steps, per depth
        planted = synth.gen.plant_positions(cfg)
        pos = eng.cache.pos.cpu().numpy()
        nlen = eng.cache.meta[..., M.META_N].cpu().numpy()
        kept = np.array([[planted[b] in pos[l, b, : nlen[l, b]] for b in range(cfg.batch)]
                         for l in range(cfg.layers)])
        retention = {"depths": list(cfg.plant_depths), "positions": planted.tolist(),
                     "kept_layers_per_depth": kept.sum(axis=0).tolist(), "layers": cfg.layers,
                     "all_kept": bool(kept.all())}

    ceiling = read_ceiling(dev, args.read_ceiling_mib) if args.read_ceiling_mib else None

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    timed = per_step[Wm:]
    bytes_total = sum(p["total"] for p in timed)
    attn_bytes = sum(p["attn"] for p in timed) / K
    ms_per_step = total_ms / K
    value = bytes_total / (total_ms * 1e-3) / 1e9
    attn_avg_ms = sum(attn_ms) / K
    achieved = attn_bytes / (attn_avg_ms * 1e-3) / 1e9
    comp_avg_ms = sum(comp_ms) / K

    out = {
        "metric": "decode-step KV GB/s (% HBM peak) + steps/s, Qwen-32B-shape batch 8",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8+f16 (f32 accumulate)",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {cfg.layers} layers, {cfg.hq}/{cfg.hkv} heads, d{cfg.d}, "
                        f"batch {cfg.batch}, {cfg.prefill}-token prefill, V={cfg.vocab}, "
                        f"N_high/N_low={pol.n_high}/{pol.n_low}, P={pol.protect}, W={pol.window}, "
                        f"alpha={pol.alpha}" + (", full FP16 cache (comparison run)" if full else "")
                        + (f", block eviction B={pol.block}" if pol.block else "")
                        + (", stable survivor order" if getattr(pol, "order", 0) and not pol.block else ""),
            "layers": cfg.layers, "batch": cfg.batch, "hq": cfg.hq, "hkv": cfg.hkv, "d": cfg.d,
            "prefill": cfg.prefill, "vocab": cfg.vocab, "parallelism": "single GPU",
            "attention_launches": ("one per layer" + (", replayed as one HIP graph" if args.graph else "")
                                   if layerwise else "one over all layers"),
            "split_keys": not args.no_split_keys,
        },
        "steps_per_s": round(1000.0 / ms_per_step, 2),
        "hbm_frac_step": round(value / HBM_PEAK_GBS, 4),
        "bytes_per_step": int(bytes_total / K),
        "attn_ms": round(attn_avg_ms, 5),
        "compact_ms": round(comp_avg_ms, 5),
        "compact_share": round(comp_avg_ms / ms_per_step, 4),
        "mean_len_end": round(len_mean, 1),
        "eviction_frac": round(sum(evict_frac[Wm:]) / K, 4),
        "moved_rows_per_event": (round(float(np.mean(moved_rows)), 1) if moved_rows else 0.0),
        "moved_rows_p90": (int(np.percentile(moved_rows, 90)) if moved_rows else 0),
        "status": status,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": counted_traffic(cfg.name),
            "traffic_source": ("counted HBM bytes per launch (FETCH_SIZE x 2 + WRITE_SIZE) from the committed "
                               "counter summary profiles/attn_decode_qwen32b_b8_traffic.md, taken on this "
                               "attention source and workload, not in this run"
                               if counted_traffic(cfg.name) is not None else
                               "none: no counter summary matches this attention source and workload"),
            "kernel": attn_kernel_name(cfg, eng, full, 1 if layerwise else None),
            "bytes_per_launch": int(attn_bytes / (cfg.layers if layerwise else 1)),
        },
    }
    if ceiling is not None:
        out["read_ceiling"] = ceiling
        out["roofline"]["frac_of_read_ceiling"] = round(achieved / ceiling["value"], 4)
    if retention is not None:
        out["retention"] = retention
    if args.cpu_full:
        cf = cpu_full(cfg, kp, vp, inputs)
        out["cpu_baseline"] = {
            "value": round(sum(p["total"] for p in per_step) / cf["seconds"] / 1e9, 4),
            "unit": "GB/s",
            "cores": cf["threads"],
            "host_cpus": os.cpu_count(),
            "blas_threads": cf["threads"],
            "kind": "oracle",
            "sample": f"all {len(inputs)} steps of the run from the prefill, every (layer, sequence)",
            "steps_per_s": round(len(inputs) / cf["seconds"], 3),
        }
    elif args.cpu_seconds > 0:
        lg0, q0, kn0, vn0, _ = inputs[0]
        cb = cpu_baseline(cfg, kp, vp, lg0.cpu().numpy(), q0.cpu().numpy(), kn0.cpu().numpy(),
                          vn0.cpu().numpy(), args.cpu_seconds)
        step0 = per_step[0]["total"]
        out["cpu_baseline"] = {
            "value": round(step0 / cb["per_step_s"] / 1e9, 4),
            "unit": "GB/s",
            "cores": cb["threads"],
            "host_cpus": os.cpu_count(),
            "blas_threads": cb["threads"],
            "kind": "oracle",
            "sample": (f"the whole first decode step after the prefill: confidence of all {cfg.batch} rows "
                       f"and all {cb['pairs']} (layer, sequence) pairs"
                       if cb["pairs"] == cfg.layers * cfg.batch else
                       f"first decode step after the prefill: confidence of all {cfg.batch} rows plus "
                       f"{cb['pairs']} of {cfg.layers * cfg.batch} (layer, sequence) pairs, "
                       f"extrapolated to the whole step"),
            "steps_per_s": round(1.0 / cb["per_step_s"], 5),
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
