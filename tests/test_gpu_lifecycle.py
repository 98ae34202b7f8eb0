"""The cache lifecycle on the GPU against the oracle: the fill phase
(longflow_decode_fill), several-slot eviction (longflow_evict_topk) and a
periodic cadence built from the two.

Acceptance is that of tests/test_gpu_parity.py for O, scores and a chosen
eviction; the updated mask and every slot taken from the mask alone (the
lowest free slot) must match exactly; top-k selections on identical fp32
scores must match exactly; a top-k selection made from the GPU's own scores
may differ from the oracle's only among slots whose oracle scores lie within
1e-4 relative of the k-th smallest.
"""

import numpy as np
import pytest
import torch

from decode_attention_kv_05_amd import workloads as W
from gpu_util import (TIE_RTOL, FillLockstep, all_outputs_written, bf16_dev, bf16_host, bf16_value, compare_pair,
                      fill_sentinels, log, lowest_free, oracle_fill_every_seq,
                      split_variants)
from oracle import decode_step, decode_step_fill, evict_topk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    from decode_attention_kv_05_amd import longflow  # noqa: F401  (fails loudly if not built)
    yield


def _lf():
    from decode_attention_kv_05_amd import longflow as lf
    return lf


@pytest.mark.parametrize("nsplit,path", split_variants([1, 3]))
def test_fill_from_empty(nsplit, path):
    """Empty caches: sequence 0 starts writing at slot 0, sequence 1 starts
    with nothing to write; both fill up and then evict."""
    wl = W.Workload("fill_empty", B=2, Hq=8, Hkv=2, d=64, S=24, steps=30, kind="plain", seed=9400)
    k, v, _ = W.initial_cache(wl)
    mask = np.zeros((wl.B, wl.S), dtype=np.uint8)
    W.poison_free(k, v, mask)
    prev = np.zeros((wl.B, wl.Hkv), dtype=np.int32)
    prev[1] = -1
    log(f"fill from empty nsplit={nsplit} path={path}")
    ls = FillLockstep(wl, k, v, mask, prev, nsplit=nsplit, split_path=path)
    for _ in range(wl.steps):
        ls.step()
    assert ls.mask.all()
    ls.finish()


@pytest.mark.parametrize("G", [1, 4, 8])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nsplit,path", split_variants([1, 4]))
def test_fill_ragged_to_full(G, d, nsplit, path):
    """Ragged valid prefixes with up to 30 free slots, through the step where
    each cache becomes full and on into eviction."""
    wl = W.Workload(f"fill_ragged_g{G}_d{d}", B=3, Hq=2 * G, Hkv=2, d=d, S=300, steps=36, kind="ragged",
                    seed=9500 + G, len_lo=270)
    k, v, mask = W.initial_cache(wl)
    prev = np.repeat(lowest_free(mask)[:, None], wl.Hkv, axis=1)
    log(f"fill ragged G={G} d={d} nsplit={nsplit} path={path}")
    ls = FillLockstep(wl, k, v, mask, prev, nsplit=nsplit, split_path=path)
    for _ in range(wl.steps):
        ls.step()
    assert ls.mask.all()
    ls.finish()


@pytest.mark.parametrize("S,nsplit,path", [(500, 1, None), (500, 2, "team"), (500, 2, "combine"),
                                            (500, 5, "team"), (500, 5, "combine"), (5000, 3, "team"),
                                            (5000, 3, "combine"), (5000, 11, "team"), (5000, 11, "combine")])
def test_fill_holes(S, nsplit, path):
    """Free slots scattered through the cache; with 5000 slots the combine
    runs over three chunks, so the lowest free slot is taken across chunks."""
    wl = W.Workload(f"fill_holes_{S}", B=2, Hq=16, Hkv=4, d=128, S=S, steps=24, kind="plain", seed=9600 + S)
    k, v, _ = W.initial_cache(wl)
    mask = W.holed_mask(wl, 1.0 - 12.0 / S)
    W.poison_free(k, v, mask)
    prev = np.repeat(lowest_free(mask)[:, None], wl.Hkv, axis=1)
    log(f"fill holes S={S} nsplit={nsplit} path={path} free={[(m == 0).sum() for m in mask]}")
    ls = FillLockstep(wl, k, v, mask, prev, nsplit=nsplit, split_path=path)
    for _ in range(wl.steps):
        ls.step()
    ls.finish()


@pytest.mark.parametrize("nsplit,path", split_variants([1, 2]))
def test_fill_divergent_heads_flagged(nsplit, path):
    """KV heads of one sequence writing different free slots (or one writing
    none) is a caller error that the step records in the workspace."""
    lf = _lf()
    wl = W.Workload("fill_diverge", B=2, Hq=4, Hkv=2, d=64, S=64, steps=1, kind="plain", seed=9700, valid=32)
    for bad in ([32, 33], [32, -1]):
        k, v, mask = W.initial_cache(wl)
        prev = np.array([[40, 40], bad], dtype=np.int32)
        ws = lf.new_workspace(wl.B, wl.Hq, wl.Hkv, wl.d, wl.S, nsplit)
        q, nk, nv = W.step_inputs(wl, 0)
        dm = torch.from_numpy(mask).cuda()
        lf.longflow_decode_fill(bf16_dev(q), bf16_dev(k), bf16_dev(v), dm, bf16_dev(nk), bf16_dev(nv),
                                torch.from_numpy(prev).cuda(), workspace=ws, nsplit=nsplit, split_path=path)
        assert lf.lf_read_device_status(ws) & lf.LF_DEV_FILL_DIVERGED
        m = dm.cpu().numpy()
        assert m[0, 40] == 1 and m[1, 32] == 1
        lf.lf_workspace_init(ws)
        assert lf.lf_read_device_status(ws) == 0
    log("divergent fill heads flagged")


def test_fill_on_full_cache_is_decode():
    """With no free slot the fill entry point gives bit-identical results to
    longflow_decode."""
    lf = _lf()
    wl = W.Workload("fill_full", B=3, Hq=16, Hkv=4, d=128, S=700, steps=1, kind="sinks", seed=9800)
    k, v, mask = W.initial_cache(wl)
    q, nk, nv = W.step_inputs(wl, 0)
    prev = np.arange(wl.B * wl.Hkv, dtype=np.int32).reshape(wl.B, wl.Hkv) * 7
    res = []
    for entry in (lf.longflow_decode, lf.longflow_decode_fill):
        dk, dv, dm = bf16_dev(k), bf16_dev(v), torch.from_numpy(mask).cuda()
        out, sc, ev = entry(bf16_dev(q), dk, dv, dm, bf16_dev(nk), bf16_dev(nv), torch.from_numpy(prev).cuda())
        torch.cuda.synchronize()
        res.append([bf16_host(out), sc.cpu().numpy(), ev.cpu().numpy(), bf16_host(dk), dm.cpu().numpy()])
    for a, b in zip(*res):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


# ---------------------------------------------------------------- top-k

TOPK_CASES = [(1, 1, 1, 1), (2, 3, 7, 3), (1, 2, 255, 100), (2, 2, 256, 256), (1, 1, 257, 1), (3, 2, 100, 100),
              (2, 4, 3200, 128), (1, 1, 16384, 16384), (1, 1, 16385, 3), (2, 1, 20000, 5000)]


@pytest.mark.parametrize("B,Hkv,S,k", TOPK_CASES)
@pytest.mark.parametrize("kind", ["ties", "spread", "special"])
def test_topk_exact(B, Hkv, S, k, kind):
    """Same fp32 scores on both sides: the selections must be identical
    (rows with 16385 or more slots take the kernel's unstaged path)."""
    lf = _lf()
    scores = W.synthetic_scores(B, Hkv, S, seed=9900 + S + k, kind=kind)
    rng = np.random.default_rng(S * 7 + k)
    frac = rng.choice([1.0, 0.9, 0.3])
    mask = (rng.random((B, S)) < frac).astype(np.uint8)
    if B > 1:
        mask[1] = 0  # a sequence with no valid slot
    got = lf.longflow_evict_topk(torch.from_numpy(scores).cuda(), torch.from_numpy(mask).cuda(), k)
    torch.cuda.synchronize()
    want = evict_topk(scores, (mask != 0)[:, None, :], k)  # [B, Hkv, k]
    assert np.array_equal(got.cpu().numpy(), np.moveaxis(want, -1, 0)), f"B={B} Hkv={Hkv} S={S} k={k} {kind}"


def test_topk_headline_shape():
    """Batch 128, 8 KV heads, 3200 slots, k = 128, full and ragged masks."""
    lf = _lf()
    B, Hkv, S, k = 128, 8, 3200, 128
    for kind, seed in (("ties", 1), ("special", 2)):
        scores = W.synthetic_scores(B, Hkv, S, seed=10000 + seed, kind=kind)
        mask = np.ones((B, S), dtype=np.uint8)
        if seed == 2:
            lens = np.random.default_rng(5).integers(100, S + 1, size=B)
            mask = (np.arange(S)[None, :] < lens[:, None]).astype(np.uint8)
        got = lf.longflow_evict_topk(torch.from_numpy(scores).cuda(), torch.from_numpy(mask).cuda(), k)
        want = evict_topk(scores, (mask != 0)[:, None, :], k)
        assert np.array_equal(got.cpu().numpy(), np.moveaxis(want, -1, 0)), kind
    log("top-k at batch 128 x 8 heads x 3200 slots exact")


def topk_acceptable(gpu_set, ref_scores, valid, k):
    """The GPU's k slots, chosen from its own scores, against the oracle's
    scores: same size, all valid, every slot clearly below the oracle's k-th
    smallest score included and none clearly above it."""
    g = [int(x) for x in gpu_set if x >= 0]
    n = int(valid.sum())
    if len(g) != min(k, n) or any(not valid[x] for x in g) or len(set(g)) != len(g):
        return False
    if n <= k:
        return True
    vals = np.sort(ref_scores[valid])
    T = vals[k - 1]
    lo, hi = T * (1 - TIE_RTOL), T * (1 + TIE_RTOL)
    must = set(np.flatnonzero(valid & (ref_scores < lo)).tolist())
    return must <= set(g) and all(ref_scores[x] <= hi for x in g)


@pytest.mark.parametrize("nsplit,path", split_variants([1, 3]))
def test_periodic_cadence(nsplit, path):
    """Fill to full, then every N = 8 steps pick N slots with top-k from that
    step's scores and overwrite them one per step over the next N steps."""
    lf = _lf()
    N = 8
    wl = W.Workload("cadence", B=3, Hq=8, Hkv=2, d=128, S=200, steps=0, kind="ragged", seed=10100, len_lo=190)
    k, v, mask = W.initial_cache(wl)
    prev = np.repeat(lowest_free(mask)[:, None], wl.Hkv, axis=1)
    ls = FillLockstep(wl, k, v, mask, prev, nsplit=nsplit, split_path=path)
    while not ls.mask.all():
        ls.step()
    log(f"cadence: full after {ls.t} steps")
    exact_sets = 0
    for rnd in range(3):
        sc_gpu, s_ref = ls.last
        q_gpu = lf.longflow_evict_topk(sc_gpu, ls.dm, N)
        torch.cuda.synchronize()
        queue = q_gpu.cpu().numpy()                      # [N, B, Hkv]
        ref = evict_topk(s_ref, (ls.mask != 0)[:, None, :], N)
        for b in range(wl.B):
            for j in range(wl.Hkv):
                assert topk_acceptable(queue[:, b, j], s_ref[b, j], ls.mask[b] != 0, N), (rnd, b, j)
                exact_sets += np.array_equal(queue[:, b, j], ref[b, j])
        for t in range(N):
            ls.prev = queue[t].astype(np.int32)
            ls.dprev = q_gpu[t].clone()
            ls.step(use_fill=False)
    ls.finish()
    log(f"cadence nsplit={nsplit}: exact top-k sets {exact_sets}/{3 * wl.B * wl.Hkv}")


# ---------------------------------------------------------------- full size

@pytest.mark.parametrize("name,len_lo", [("qwen3_8b", 3000), ("long_reasoning", 16000)])
def test_fill_step_full_size(name, len_lo):
    """One fill step at full size (the device's split plan) with up to a few
    hundred free slots per sequence: every (sequence, KV head) pair against
    the oracle (a thread pool over the host's cores), outputs preset to
    sentinels so that an unwritten pair fails, and the mask update and every
    free-slot choice exact."""
    lf = _lf()
    base = W.WORKLOADS[name]
    wl = base.replace(name=name + "_fill", kind="ragged", len_lo=len_lo)
    log(f"full-size fill {wl.name}: generating")
    k, v, mask = W.initial_cache(wl)
    prev = np.repeat(lowest_free(mask)[:, None], wl.Hkv, axis=1)
    q, nk, nv = W.step_inputs(wl, 0)
    dk, dv, dm = bf16_dev(k), bf16_dev(v), torch.from_numpy(mask).cuda()
    ws = lf.new_workspace(wl.B, wl.Hq, wl.Hkv, wl.d, wl.S)
    out = torch.empty((wl.B, wl.Hq, wl.d), dtype=torch.bfloat16, device="cuda")
    sc = torch.empty((wl.B, wl.Hkv, wl.S), dtype=torch.float32, device="cuda")
    nx = torch.empty((wl.B, wl.Hkv), dtype=torch.int32, device="cuda")
    fill_sentinels(out, sc, nx)
    lf.longflow_decode_fill(bf16_dev(q), dk, dv, dm, bf16_dev(nk), bf16_dev(nv), torch.from_numpy(prev).cuda(),
                            scale=float(wl.scale), out=out, scores=sc, next_slot=nx, workspace=ws)
    torch.cuda.synchronize()
    assert lf.lf_read_device_status(ws) == 0
    all_outputs_written(out, sc, nx)
    want_mask = mask.copy()
    for b in range(wl.B):
        if prev[b, 0] >= 0:
            want_mask[b, prev[b, 0]] = 1
    assert np.array_equal(dm.cpu().numpy(), want_mask)
    n_gpu = nx.cpu().numpy()
    want_next = lowest_free(want_mask)
    full = want_next < 0
    assert np.array_equal(n_gpu[~full], np.repeat(want_next[~full, None], wl.Hkv, axis=1))
    log(f"  {wl.name}: oracle over all {wl.B} sequences")
    o_ref, s_ref, n_ref, m_ref = oracle_fill_every_seq(q, k, v, mask, nk, nv, prev, wl.scale)
    assert np.array_equal(m_ref, want_mask)
    o_gpu = bf16_value(bf16_host(out))
    s_all = sc.cpu().numpy().astype(np.float64)
    for b in range(wl.B):
        for j in range(wl.Hkv):
            heads = slice(j * wl.G, (j + 1) * wl.G)
            compare_pair(o_gpu[b, heads], s_all[b, j], n_gpu[b, j], o_ref[b, heads], s_ref[b, j], n_ref[b, j],
                         m_ref[b] != 0, f"{wl.name} b={b} j={j}")
    log(f"  {wl.name}: every pair matches; mask and free-slot choices exact")


@pytest.mark.parametrize("path", ["team", "combine"])
def test_fill_more_teams_than_the_device_holds(path):
    """160 pairs with 17 splits each: more teams than the device holds at
    once (about 30), so the KV heads of a sequence run at different times
    while its mask fills; lockstep with the oracle from scattered free slots
    to full and on into eviction."""
    wl = W.Workload("fill_many_teams", B=40, Hq=16, Hkv=4, d=64, S=600, steps=1, kind="plain", seed=9800)
    k, v, _ = W.initial_cache(wl)
    mask = W.holed_mask(wl, 1.0 - 6.0 / 600)
    W.poison_free(k, v, mask)
    prev = np.repeat(lowest_free(mask)[:, None], wl.Hkv, axis=1)
    log(f"fill with more teams than the device holds, path={path}, free={[(m == 0).sum() for m in mask][:8]}...")
    ls = FillLockstep(wl, k, v, mask, prev, nsplit=17, split_path=path)
    for _ in range(int((mask == 0).sum(axis=1).max()) + 2):
        ls.step()
    assert ls.mask.all()
    ls.finish()
