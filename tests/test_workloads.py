"""The seeded generators are deterministic, shaped as described, and their
schedules are valid."""
import json
import os

import numpy as np

import workloads as wl
from oracle.schedule import validate

HERE = os.path.dirname(__file__)


def test_fingerprints_are_stable():
    import importlib.util
    spec = importlib.util.spec_from_file_location("mkfp", os.path.join(HERE, "golden", "make_fingerprints.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    want = json.load(open(os.path.join(HERE, "golden", "fingerprints.json")))
    assert mod.fingerprints() == want


def test_seed_changes_inputs():
    a = wl.CONFIGS["tiny_ag"]["make"](0)
    b = wl.CONFIGS["tiny_ag"]["make"](1)
    assert wl.fingerprint(a.B) != wl.fingerprint(b.B)


def test_tiny_ag_shape_and_range():
    w = wl.CONFIGS["tiny_ag"]["make"]()
    assert (w.R, w.m_shard, w.K, w.N, w.unit_rows) == (4, 64, 128, 96, 64)
    from oracle.numerics import bf16_to_f64
    v = bf16_to_f64(np.vstack(w.shards))
    assert v.min() >= -1 and v.max() <= 1
    validate(w.order, w.delay_ns, 4)


def test_ag_schedule_shape_without_large_tensors():
    w = wl.make_ag(8, 128, 8, 8, seed=0, unit_rows=16, max_delay_ns=20000)
    assert w.order.shape == (64,)
    validate(w.order, w.delay_ns, 64)
    assert w.delay_ns.max() <= 20000 and w.delay_ns.dtype == np.uint32


def test_normal_variance_reading():
    # N(0, 1/K) means variance 1/K
    w = wl.make_ag(1, 4, 4096, 64, seed=3)
    from oracle.numerics import bf16_to_f64
    var = bf16_to_f64(w.B).var()
    assert abs(var * 4096 - 1.0) < 0.05


def test_moe_blocks_and_logits():
    m = wl.make_moe(64, 16, 32, 4, 8, 8, seed=0, block_tokens=16)
    assert m.order.shape == (4,) and sorted(m.order.tolist()) == [0, 1, 2, 3]
    assert m.logits.dtype == np.float32 and np.all(np.isfinite(m.logits))


def test_ring_schedule_is_step_major_permutation():
    w = wl.make_ring(5, 8, 16, 4, seed=9, step_delay_ns=1500)
    n = (w.R - 1) * w.H
    validate(w.order, w.delay_ns, n)
    # every unit of step s arrives before any unit of step s + 1
    steps = w.order // w.H
    assert np.all(np.diff(steps) >= 0)
    assert np.array_equal(w.delay_ns, (np.arange(n) // w.H * 1500).astype(np.uint32))
    assert (w.H, w.S, w.D, w.R) == (5, 8, 16, 4) and len(w.K) == len(w.V) == 4
    one = wl.make_ring(2, 8, 16, 1, seed=9)
    assert one.order.shape == (0,) and one.delay_ns.shape == (0,)
