"""Host logic of bench.py that needs no GPU: the parity verdict its CPU
baseline leg gives for the first step, and the lookup of the committed LDS
counters."""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from decode_attention_kv_05_amd import workloads as W  # noqa: E402
from oracle import decode_step  # noqa: E402


def _bf16(x):
    """fp64 -> fp32 -> bf16 (truncated here; any rounding within 2^-8 does) -> fp64."""
    return (np.asarray(x, np.float32).view(np.uint32) & 0xffff0000).view(np.float32).astype(np.float64)


@pytest.fixture(scope="module")
def tiny_step():
    wl = W.WORKLOADS["tiny"]
    batch = [0]
    k, v, m = W.initial_cache(wl, batch)
    q, nk, nv = W.step_inputs(wl, 0, batch)
    ref = decode_step(q, k, v, m, nk, nv, W.first_prev_slot(wl, batch), wl.scale)
    gpu = {"out": _bf16(ref[0]), "scores": ref[1].copy(), "evict": ref[2].copy()}
    return wl, m, gpu, ref


def test_parity_verdict_passes_outputs_within_the_rule(tiny_step):
    wl, m, gpu, ref = tiny_step
    v = bench.parity_verdict(wl, m, gpu, ref)
    assert v["verdict"] == "pass" and v["pairs"] == v["pairs_passed"] == wl.B * wl.Hkv
    assert v["evict_exact"] == wl.B * wl.Hkv and v["score_max_rel_err"] == 0.0


@pytest.mark.parametrize("what", ["scores", "o", "evict", "masked"])
def test_parity_verdict_fails_outputs_outside_the_rule(tiny_step, what):
    wl, m, gpu, ref = tiny_step
    bad = {key: val.copy() for key, val in gpu.items()}
    valid = np.flatnonzero(m[0])
    if what == "scores":  # one valid score 2e-3 off (the rule allows 1e-3)
        bad["scores"][0, 0, valid[3]] *= 1 + 2e-3
    elif what == "o":  # one output 0.1 off (the rule allows 1e-2 + 1e-2 |ref|)
        bad["out"][0, 0, 5] += 0.1 + 1e-2 * abs(bad["out"][0, 0, 5])
    elif what == "evict":  # a valid slot far from the minimum
        s = ref[1][0, 0, valid]
        bad["evict"][0, 0] = valid[np.argmax(s)]
    else:  # a masked slot's score not +inf
        bad["scores"][0, 0, np.flatnonzero(m[0] == 0)[0]] = 1.0
    assert bench.parity_verdict(wl, m, bad, ref)["verdict"] == "fail"


def test_parity_verdict_accepts_a_near_tie(tiny_step):
    """Two smallest oracle scores within 1e-4 relative: either slot is accepted."""
    wl, m, gpu, ref = tiny_step
    o, s, e = (x.copy() for x in ref)
    valid = np.flatnonzero(m[0])
    best = int(e[0, 0])
    other = int(valid[valid != best][0])
    s[0, 0, other] = s[0, 0, best] * (1 + 5e-5)
    g = {"out": gpu["out"], "scores": s.copy(), "evict": np.full_like(e, other)}
    v = bench.parity_verdict(wl, m, g, (o, s, e))
    assert v["verdict"] == "pass" and v["evict_exact"] == 0
    s[0, 0, other] = s[0, 0, best] * (1 + 5e-4)  # no longer a near-tie
    g["scores"] = s.copy()
    assert bench.parity_verdict(wl, m, g, (o, s, e))["verdict"] == "fail"


def test_measured_lds_reads_the_committed_counters():
    """Every workload with a counter profile on the current decode sources
    gives its bank-conflict figures; a workload without one gives None."""
    from decode_attention_kv_05_amd.build import source_hash
    for name in ("qwen3_8b", "long_reasoning", "ragged", "llama8b_budget"):
        path = os.path.join(ROOT, "profiles", f"longflow_decode_{name}_counters.txt")
        with open(path) as f:
            current = f"kernel sources (decode): {source_hash('decode')}" in f.read()
        rec = bench.measured_lds(name)
        if not current:
            assert rec is None
            continue
        assert rec["source"] == f"profiles/longflow_decode_{name}_counters.txt"
        assert 0.0 <= rec["bank_conflict_frac_of_lds_active"] < 1.0
        assert rec["bank_conflict_cycles_per_dispatch"] >= 0.0
    assert bench.measured_lds("no_such_workload") is None
