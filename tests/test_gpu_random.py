"""Randomised parity cases for the operator, the fill step and the k-slot
selection.

The cases are drawn once from a fixed seed, so every run checks the same
list; they combine what the hand-written cases vary one at a time: group size
(1..8, padded ones included), head count, d, slot counts from 1 to a few
thousand, the workload kinds, masks with scattered holes and explicit split
counts.  Holed masks go over the caches of the kinds without a valid-length
prefix (every slot holds finite data), and the K/V of their free slots are
poisoned with NaN.  Each decode case runs three steps in lockstep with the
oracle and checks the written cache rows; each fill case fills its caches
through to eviction in lockstep, the mask and every free-slot choice exact;
each selection case compares the k slots bit for bit.  Acceptance is the
operator's (tests/gpu_util.py)."""

import numpy as np
import pytest
import torch

from decode_attention_kv_05_amd import workloads as W
from gpu_util import FillLockstep, Lockstep, log, lowest_free
from oracle import evict_topk

pytestmark = pytest.mark.gpu


def _decode_cases():
    rng = np.random.default_rng(20261202)
    cases = []
    for i in range(48):
        G = int(rng.integers(1, 9))
        Hkv = int(rng.integers(1, 4))
        d = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 5))
        S = max(1, int(np.exp(rng.uniform(0.0, np.log(2500.0)))))
        kind = str(rng.choice(W.KINDS))
        holes = float(rng.choice([0.0, 0.0, 0.5, 0.9, 0.02]))  # 0: the kind's own mask
        if holes and kind == "ragged":
            kind = "plain"  # the ragged kind's cache is NaN past each valid length
        ns = int(rng.choice([0, 1, 2, 3, 5, 8]))
        nsplit = min(ns, S) if ns else None  # None: the library's plan
        cases.append((i, B, G, Hkv, d, S, kind, holes, nsplit))
    return cases


def _fill_cases():
    rng = np.random.default_rng(20261204)
    cases = []
    for i in range(16):
        G = int(rng.integers(1, 9))
        Hkv = int(rng.integers(1, 4))
        d = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 4))
        S = int(rng.integers(2, 600))
        free = int(rng.integers(1, min(S, 30) + 1))  # free slots per sequence, about
        ns = int(rng.choice([0, 1, 2, 3, 5]))
        nsplit = min(ns, S) if ns else None
        cases.append((i, B, G, Hkv, d, S, free, nsplit))
    return cases


def _topk_cases():
    rng = np.random.default_rng(20261203)
    cases = []
    for i in range(32):
        B = int(rng.integers(1, 4))
        Hkv = int(rng.integers(1, 5))
        S = max(1, int(np.exp(rng.uniform(0.0, np.log(20000.0)))))
        k = int(rng.integers(1, S + 1))
        kind = str(rng.choice(["ties", "spread", "special"]))
        frac = float(rng.choice([1.0, 0.7, 0.1, 0.0]))
        cases.append((i, B, Hkv, S, k, kind, frac))
    return cases


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    from decode_attention_kv_05_amd import longflow  # noqa: F401  (fails loudly if not built)
    yield


@pytest.mark.parametrize("case", _decode_cases(), ids=lambda c: f"r{c[0]}")
def test_random_decode_lockstep(case):
    i, B, G, Hkv, d, S, kind, holes, nsplit = case
    log(f"random decode {i}: B={B} G={G} Hkv={Hkv} d={d} S={S} {kind} holes={holes} nsplit={nsplit}")
    wl = W.Workload(f"rand{i}", B=B, Hq=G * Hkv, Hkv=Hkv, d=d, S=S, steps=3, kind=kind, seed=31000 + i,
                    len_lo=min(S, 1 + S // 4))
    k, v, mask = W.initial_cache(wl)
    if holes:
        mask = W.holed_mask(wl, 1.0 - holes)
        if B > 1:
            mask[B - 1] = 0  # a sequence with no valid slot
        W.poison_free(k, v, mask)
    ls = Lockstep(wl, nsplit=nsplit, state=(k, v, mask))
    for _ in range(wl.steps):
        ls.step()
    ls.check_full_cache()


@pytest.mark.parametrize("case", _fill_cases(), ids=lambda c: f"f{c[0]}")
def test_random_fill_lockstep(case):
    """Free slots scattered through the cache (the first sequence may start
    with nothing to write); fill steps until every cache is full, then two
    more, in lockstep with the oracle."""
    i, B, G, Hkv, d, S, free, nsplit = case
    log(f"random fill {i}: B={B} G={G} Hkv={Hkv} d={d} S={S} free~{free} nsplit={nsplit}")
    wl = W.Workload(f"rfill{i}", B=B, Hq=G * Hkv, Hkv=Hkv, d=d, S=S, steps=1, kind="plain", seed=34000 + i)
    k, v, _ = W.initial_cache(wl)
    mask = W.holed_mask(wl, 1.0 - free / S)
    W.poison_free(k, v, mask)
    prev = np.repeat(lowest_free(mask)[:, None], Hkv, axis=1)
    prev[0] = -1 if i % 2 else prev[0]
    ls = FillLockstep(wl, k, v, mask, prev, nsplit=nsplit)
    for _ in range(int((mask == 0).sum(axis=1).max()) + 3):
        ls.step()
    assert ls.mask.all()
    ls.finish()


@pytest.mark.parametrize("case", _topk_cases(), ids=lambda c: f"t{c[0]}")
def test_random_topk_exact(case):
    i, B, Hkv, S, k, kind, frac = case
    log(f"random top-k {i}: B={B} Hkv={Hkv} S={S} k={k} {kind} valid={frac}")
    from decode_attention_kv_05_amd import longflow as lf
    scores = W.synthetic_scores(B, Hkv, S, seed=32000 + i, kind=kind)
    mask = (np.random.default_rng(33000 + i).random((B, S)) < frac).astype(np.uint8)
    got = lf.longflow_evict_topk(torch.from_numpy(scores).cuda(), torch.from_numpy(mask).cuda(), k)
    torch.cuda.synchronize()
    want = evict_topk(scores, (mask != 0)[:, None, :], k)  # [B, Hkv, k]
    assert np.array_equal(got.cpu().numpy(), np.moveaxis(want, -1, 0))


def _path_cases():
    rng = np.random.default_rng(20261205)
    cases = []
    for i in range(24):
        G = int(rng.integers(1, 9))
        Hkv = int(rng.integers(1, 9))
        d = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 40))
        S = max(2, int(np.exp(rng.uniform(np.log(2.0), np.log(20000.0)))))
        nsplit = int(min(S, rng.choice([2, 3, 4, 6, 9, 17, 64])))
        kind = str(rng.choice(W.KINDS))
        holes = float(rng.choice([0.0, 0.0, 0.5, 0.02]))
        if holes and kind == "ragged":
            kind = "plain"
        cases.append((i, B, G, Hkv, d, S, nsplit, kind, holes))
    return cases


@pytest.mark.parametrize("case", _path_cases(), ids=lambda c: f"p{c[0]}")
def test_random_team_equals_combine(case):
    """The team and the combine path on the same random inputs: scores and
    evicted slots bit for bit, O within the O tolerance of each other, the
    written cache rows equal, no device status bit.  Batch sizes up to 39
    with up to 8 KV heads and up to 64 splits give more teams than the
    device holds at once."""
    from decode_attention_kv_05_amd import longflow as lf
    from gpu_util import bf16_dev, bf16_host, bf16_value
    i, B, G, Hkv, d, S, nsplit, kind, holes = case
    log(f"random paths {i}: B={B} G={G} Hkv={Hkv} d={d} S={S} nsplit={nsplit} {kind} holes={holes}")
    wl = W.Workload(f"rpath{i}", B=B, Hq=G * Hkv, Hkv=Hkv, d=d, S=S, steps=1, kind=kind, seed=35000 + i,
                    len_lo=min(S, 1 + S // 4))
    k, v, mask = W.initial_cache(wl)
    if holes:
        mask = W.holed_mask(wl, 1.0 - holes)
        W.poison_free(k, v, mask)
    q, nk, nv = W.step_inputs(wl, 0)
    rng = np.random.default_rng(36000 + i)
    prev = np.where(rng.random((B, Hkv)) < 0.8, rng.integers(0, S, (B, Hkv)), -1).astype(np.int32)
    prev[mask[np.arange(B)[:, None], np.maximum(prev, 0)] == 0] = -1  # written slots are valid ones
    res = {}
    for path in ("team", "combine"):
        ws = lf.new_workspace(B, wl.Hq, Hkv, d, S, nsplit)
        dk, dv = bf16_dev(k), bf16_dev(v)
        out, sc, ev = lf.longflow_decode(bf16_dev(q), dk, dv, torch.from_numpy(mask).cuda(), bf16_dev(nk),
                                         bf16_dev(nv), torch.from_numpy(prev).cuda(), scale=float(wl.scale),
                                         workspace=ws, nsplit=nsplit, split_path=path)
        torch.cuda.synchronize()
        assert lf.lf_read_device_status(ws) == 0
        res[path] = (bf16_value(bf16_host(out)), sc.cpu().numpy(), ev.cpu().numpy(), bf16_host(dk), bf16_host(dv))
    (ot, st, et, kt, vt), (oc, scb, ec, kc, vc) = res["team"], res["combine"]
    assert np.array_equal(st.view(np.uint32), scb.view(np.uint32)), "scores differ between the paths"
    assert np.array_equal(et, ec)
    assert np.array_equal(kt, kc) and np.array_equal(vt, vc)
    fin = np.isfinite(oc)
    assert np.array_equal(fin, np.isfinite(ot))
    assert np.all(np.abs(ot[fin] - oc[fin]) <= 1e-2 + 1e-2 * np.abs(oc[fin]))
