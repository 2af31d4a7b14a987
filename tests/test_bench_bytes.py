"""CPU pin of bench.py's algorithmic byte count (what `value` and the
attention roofline divide by), on a hand-worked two-sequence step."""
import importlib.util
import os

import numpy as np

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_step_bytes_hand_worked():
    b = _bench()
    pol = synth.Policy(n_high=8, n_low=16, protect=2, window=8)
    cfg = synth.Config(name="t", layers=1, batch=2, hq=4, hkv=2, d=64, vocab=100, prefill=0, steps=0, policy=pol)
    # sequence 0: 10 tokens, 4 INT8 (6 FP16); sequence 1: 20 tokens, all FP16
    n, n8 = np.array([[10, 20]]), np.array([[4, 0]])
    got = b.step_bytes(cfg, n, n8, np.array([[1, 0]]), np.array([[0, 2]]), np.array([[1, 0]]))
    # attention, per sequence: INT8 rows 2*H*d each, FP16 rows and the new one
    # 4*H*d each, K and V scales 8*H*d when INT8 rows exist, q and o 4*Hq*d,
    # the per-key mass 4 per cached token and the new one
    a0 = 2 * 64 * (2 * 4 + 4 * 7) + 8 * 2 * 64 + 4 * 4 * 64 + 4 * 11
    a1 = 2 * 64 * (4 * 21) + 4 * 4 * 64 + 4 * 21
    assert (a0, a1) == (6700, 11860)
    assert got["attn"] == a0 + a1
    assert got["meta"] == 16 * 30                      # EMA read + write, position, score
    # moved rows read and written (INT8 row 2*H*d, FP16 row 4*H*d) and the
    # new row read and written (8*H*d) for every sequence
    assert got["compact"] == 2 * (1 * 2 * 2 * 64) + 2 * (2 * 4 * 2 * 64) + 2 * 8 * 2 * 64
    assert got["quant"] == 6 * 2 * 64                  # FP16 row read, INT8 row written
    assert got["conf"] == 4 * 2 * 100                  # the logits
    assert got["total"] == 18560 + 480 + 4608 + 768 + 800


def test_step_bytes_full_cache_run_counts_kv_and_q_only():
    b = _bench()
    pol = synth.Policy(n_high=64, n_low=64, protect=2, window=64)
    cfg = synth.Config(name="t", layers=1, batch=1, hq=4, hkv=2, d=64, vocab=100, prefill=0, steps=0,
                       policy=pol, mode="full_kv")
    got = b.step_bytes(cfg, np.array([[10]]), np.array([[0]]), np.zeros((1, 1), int), np.zeros((1, 1), int),
                       np.zeros((1, 1), int))
    assert got["attn"] == 2 * 64 * 4 * 11 + 4 * 4 * 64
    assert got["meta"] == 0 and got["conf"] == 0 and got["quant"] == 0
    assert got["total"] == got["attn"] + 8 * 2 * 64


def test_bench_refuses_more_than_one_gpu():
    """The library runs on one GPU: bench.py --gpus 2 exits with a message
    that says so, before touching a device."""
    import json
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"] and msg["n_gpus"] == 2


def test_traffic_summary_hash_follows_the_code(tmp_path):
    """The counted traffic in bench.py's roofline line is tied to the attention
    code by a hash that ignores line comments and blank lines: a comment edit
    keeps it, a code edit voids it, and a summary never serves another
    workload."""
    b = _bench()
    src = tmp_path / "k.hip"
    src.write_text("// header\nint f(int x) {\n  return x + 1;  // one\n}\n\n")
    h0 = b.code_sha256(str(src))
    src.write_text("// another header\n\nint f(int x) {\n  return x + 1;   // changed note\n}\n")
    assert b.code_sha256(str(src)) == h0
    src.write_text("// header\nint f(int x) {\n  return x + 2;  // one\n}\n")
    assert b.code_sha256(str(src)) != h0
    assert b.counted_traffic("qwen14b") is None
