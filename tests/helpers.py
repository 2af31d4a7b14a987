"""Test helpers: device-state snapshots as oracle caches, and comparisons.

Conversions only; no method arithmetic lives here.
"""
import numpy as np

from oracle import confk_oracle as O


def oracle_cache(snap, hkv, d):
    """SeqCache (oracle state) holding exactly the device state of one (layer, sequence)."""
    n, n8 = snap["n"], snap["n8"]
    c = O.empty_cache(hkv, d)
    c.pos = snap["pos"].astype(np.int64)
    c.is8 = np.arange(n) < n8
    c.k16 = np.zeros((n, hkv, d), np.float16)
    c.v16 = np.zeros((n, hkv, d), np.float16)
    c.k16[n8:] = snap["k16"]
    c.v16[n8:] = snap["v16"]
    c.k8 = np.zeros((n, hkv, d), np.int8)
    c.v8 = np.zeros((n, hkv, d), np.int8)
    c.k8[:n8] = snap["k8"]
    c.v8[:n8] = snap["v8"]
    c.ema = snap["ema"].astype(np.float64)
    c.ks = snap["ks"].copy()
    c.vs = snap["vs"].copy()
    c.calibrated = snap["calibrated"]
    c.saturated = snap["saturated"]
    return c


def assert_state_equal(snap, oc, ema_tol=1e-5, what=""):
    """Device state vs oracle state: integer and byte content exactly, EMA to ema_tol."""
    n8 = int(oc.is8.sum())
    assert snap["n"] == oc.n, f"{what}: n {snap['n']} != {oc.n}"
    assert snap["n8"] == n8, f"{what}: n8 {snap['n8']} != {n8}"
    assert (oc.is8 == (np.arange(oc.n) < n8)).all(), f"{what}: INT8 tokens are not the oldest"
    assert np.array_equal(snap["pos"].astype(np.int64), oc.pos), f"{what}: positions differ"
    assert snap["calibrated"] == oc.calibrated, f"{what}: calibration flag"
    if oc.calibrated:
        assert np.array_equal(snap["ks"].view(np.uint32), oc.ks.view(np.uint32)), f"{what}: K scales"
        assert np.array_equal(snap["vs"].view(np.uint32), oc.vs.view(np.uint32)), f"{what}: V scales"
    assert np.array_equal(snap["k8"], oc.k8[:n8]), f"{what}: K codes"
    assert np.array_equal(snap["v8"], oc.v8[:n8]), f"{what}: V codes"
    assert np.array_equal(snap["k16"].view(np.uint16), oc.k16[n8:].view(np.uint16)), f"{what}: K fp16"
    assert np.array_equal(snap["v16"].view(np.uint16), oc.v16[n8:].view(np.uint16)), f"{what}: V fp16"
    assert snap["saturated"] == oc.saturated, f"{what}: saturation count"
    if oc.n:
        err = np.abs(snap["ema"].astype(np.float64) - oc.ema).max()
        assert err <= ema_tol, f"{what}: EMA error {err}"


def rel_maxabs(x, ref):
    """max |x - ref| / max(max |ref|, 1e-6)."""
    ref = np.asarray(ref, np.float64)
    return float(np.abs(np.asarray(x, np.float64) - ref).max() / max(np.abs(ref).max(), 1e-6))
