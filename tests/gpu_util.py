"""Helpers for the GPU parity tests: device upload of bf16 bit patterns, the
acceptance rule against the oracle, and a lockstep driver that runs the HIP
operator and the oracle on the same seeded inputs step after step."""

import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from decode_attention_kv_05_amd import workloads as W
from oracle import decode_step, decode_step_fill, write_slot

# Acceptance against the fp64 oracle (bf16 inputs, fp32 accumulation):
O_ATOL = 1e-2
O_RTOL = 1e-2
SCORE_RTOL = 1e-3
TIE_RTOL = 1e-4


def split_variants(counts):
    """(nsplit, split_path) cases: one per count of 1 (or None, the plan),
    both finishing paths for every count above 1."""
    out = []
    for n in counts:
        if n is None or n == 1:
            out.append((n, None))
        else:
            out += [(n, "team"), (n, "combine")]
    return out


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_dev(bits, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def bf16_host(t):
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_value(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def evict_acceptable(gpu_slot, ref_scores, valid, ref_slot):
    """Exact match, or a near-tie: the oracle's two smallest valid scores differ
    by less than TIE_RTOL relative and the GPU's slot is within that band."""
    if gpu_slot == ref_slot:
        return True
    if ref_slot < 0 or gpu_slot < 0 or gpu_slot >= len(valid) or not valid[gpu_slot]:
        return False
    vals = np.sort(ref_scores[valid])
    s1 = vals[0]
    s2 = vals[1] if vals.size > 1 else np.inf
    if s1 == 0:
        return ref_scores[gpu_slot] == 0
    return (s2 - s1) / s1 < TIE_RTOL and ref_scores[gpu_slot] <= s1 * (1 + TIE_RTOL)


def compare_pair(o_gpu, s_gpu, e_gpu, o_ref, s_ref, e_ref, valid, where):
    """Assert the acceptance rule for one (b, j); returns True at an exact evict match."""
    err = np.abs(o_gpu - o_ref)
    tol = O_ATOL + O_RTOL * np.abs(o_ref)
    assert np.all(err <= tol), f"{where}: O max err {err.max():.3e} (tol {tol.flat[np.argmax(err - tol)]:.3e})"
    assert np.all(np.isposinf(s_gpu[~valid])), f"{where}: masked scores not +inf"
    sv, rv = s_gpu[valid], s_ref[valid]
    rel = np.abs(sv - rv) / np.maximum(rv, 1e-300)
    assert np.all(rel <= SCORE_RTOL), f"{where}: score max rel err {rel.max():.3e} at slot {np.flatnonzero(valid)[np.argmax(rel)]}"
    assert evict_acceptable(int(e_gpu), s_ref, valid, int(e_ref)), \
        f"{where}: evict gpu {e_gpu} ref {e_ref} (ref scores {s_ref[e_gpu] if 0 <= e_gpu < len(s_ref) else None} vs {s_ref[e_ref] if e_ref >= 0 else None})"
    return int(e_gpu) == int(e_ref)


def oracle_workers():
    """Host threads for the oracle: the process's CPU share, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_every_pair(q, k, v, mask, nk, nv, prev, scale):
    """decode_step over every (sequence, KV head), one sequence per task on a
    thread pool (numpy releases the GIL in the array work); the caches are
    written in place as by one decode_step call over the whole batch."""
    from threadpoolctl import threadpool_limits
    B = q.shape[0]

    def one(b):
        return decode_step(q[b:b + 1], k[b:b + 1], v[b:b + 1], mask[b:b + 1], nk[b:b + 1], nv[b:b + 1],
                           prev[b:b + 1], scale)

    with threadpool_limits(limits=1), ThreadPoolExecutor(oracle_workers()) as ex:
        res = list(ex.map(one, range(B)))
    return (np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res]),
            np.concatenate([r[2] for r in res]))


def oracle_fill_every_seq(q, k, v, mask, nk, nv, prev, scale):
    """decode_step_fill over every sequence, one sequence per task on a
    thread pool; returns (O, scores, next slot, updated mask) as one
    decode_step_fill call over the whole batch would (the host arrays are
    not modified)."""
    from threadpoolctl import threadpool_limits
    B = q.shape[0]

    def one(b):
        sl = slice(b, b + 1)
        return decode_step_fill(q[sl], k[sl].copy(), v[sl].copy(), mask[sl].copy(), nk[sl], nv[sl], prev[sl], scale)

    with threadpool_limits(limits=1), ThreadPoolExecutor(oracle_workers()) as ex:
        res = list(ex.map(one, range(B)))
    return tuple(np.concatenate([r[i] for r in res]) for i in range(4))


def fill_sentinels(out, scores, evict):
    """Outputs a step must overwrite: NaN O and scores, -2 slots, so that a
    pair the step leaves unwritten fails every later check."""
    out.view(torch.int16).fill_(0x7FC0)
    scores.fill_(float("nan"))
    evict.fill_(-2)


def all_outputs_written(out, sc, ev):
    """No sentinel left: O finite everywhere, no NaN score, no -2 slot
    (the workloads hold finite inputs only)."""
    assert bool(torch.isfinite(out.float()).all()), "O not written (or not finite) for some pair"
    assert not bool(torch.isnan(sc).any()), "scores not written for some pair"
    assert bool((ev >= -1).all()), "evicted slot not written for some pair"


class Lockstep:
    """Runs `steps` decode steps of workload `wl` on the GPU and, for the pairs
    in `pairs` (None = all), on the oracle; both sides continue from the GPU's
    accepted eviction.  The oracle's cache takes every pair's write each step,
    so a step can be checked over every pair (step(all_pairs=True)) and the
    whole cache compared at the end.  Outputs are preset to sentinels before
    each step."""

    def __init__(self, wl, pairs=None, nsplit=None, device="cuda", state=None, split_path=None):
        from decode_attention_kv_05_amd import longflow as lf
        self.lf = lf
        self.wl = wl
        self.nsplit = nsplit
        self.split_path = split_path
        self.device = device
        if state is None:
            k, v, mask = W.initial_cache(wl)
        else:
            k, v, mask = state
        self.mask = mask
        self.pairs = pairs if pairs is not None else [(b, j) for b in range(wl.B) for j in range(wl.Hkv)]
        # the oracle's own copy of the cache (the host arrays, uploaded once)
        self.k_ref = k
        self.v_ref = v
        self.dk = bf16_dev(k, device)
        self.dv = bf16_dev(v, device)
        self.dm = torch.from_numpy(mask).to(device)
        self.prev = W.first_prev_slot(wl)
        self.dprev = torch.from_numpy(self.prev).to(device)
        self.ws = lf.new_workspace(wl.B, wl.Hq, wl.Hkv, wl.d, wl.S, nsplit, device)
        self.out = torch.empty((wl.B, wl.Hq, wl.d), dtype=torch.bfloat16, device=device)
        self.sc = torch.empty((wl.B, wl.Hkv, wl.S), dtype=torch.float32, device=device)
        self.evs = [torch.empty((wl.B, wl.Hkv), dtype=torch.int32, device=device) for _ in range(2)]
        self.t = 0
        self.exact = 0
        self.total = 0

    def gpu_step(self, t):
        q, nk, nv = W.step_inputs(self.wl, t)
        ev = self.evs[t % 2]
        fill_sentinels(self.out, self.sc, ev)
        out, sc, ev = self.lf.longflow_decode(
            bf16_dev(q, self.device), self.dk, self.dv, self.dm, bf16_dev(nk, self.device),
            bf16_dev(nv, self.device), self.dprev, scale=float(self.wl.scale), out=self.out, scores=self.sc,
            evict_slot=ev, workspace=self.ws, nsplit=self.nsplit, split_path=self.split_path)
        torch.cuda.synchronize()
        return (q, nk, nv), out, sc, ev

    def step(self, check=True, check_cache=True, all_pairs=False):
        """One lockstep step.  check: compare the sampled pairs (all_pairs:
        every pair) with the oracle; every pair's cache write is applied to
        the oracle's copy either way."""
        wl, t = self.wl, self.t
        (q, nk, nv), out, sc, ev = self.gpu_step(t)
        o_gpu = bf16_value(bf16_host(out))
        e_gpu = ev.cpu().numpy()
        pairs = [(b, j) for b in range(wl.B) for j in range(wl.Hkv)] if all_pairs else self.pairs
        checked = set(pairs) if check else set()
        # the writes of the pairs the oracle does not run this step
        for b in range(wl.B):
            for j in range(wl.Hkv):
                if (b, j) not in checked:
                    write_slot(self.k_ref[b, j], self.v_ref[b, j], nk[b, j], nv[b, j], self.prev[b, j])
        if check:
            if all_pairs:
                o_ref, s_ref, e_ref = oracle_every_pair(q, self.k_ref, self.v_ref, self.mask, nk, nv, self.prev,
                                                        wl.scale)
                s_all = sc.cpu().numpy().astype(np.float64)
                s_gpu = {b: s_all[b] for b in range(wl.B)}
            else:
                s_gpu = {b: sc[b].cpu().numpy().astype(np.float64) for b in sorted({b for b, _ in pairs})}
                o_ref, s_ref, e_ref = decode_step(q, self.k_ref, self.v_ref, self.mask, nk, nv, self.prev,
                                                  wl.scale, pairs=pairs)
            for b, j in pairs:
                heads = slice(j * wl.G, (j + 1) * wl.G)
                valid = self.mask[b] != 0
                self.exact += compare_pair(o_gpu[b, heads], s_gpu[b][j], e_gpu[b, j], o_ref[b, heads],
                                           s_ref[b, j], e_ref[b, j], valid, f"{wl.name} t={t} b={b} j={j}")
                self.total += 1
            if check_cache:
                for b, j in self.pairs:
                    p = int(self.prev[b, j])
                    if p >= 0:
                        assert np.array_equal(bf16_host(self.dk[b, j, p]), nk[b, j])
                        assert np.array_equal(bf16_host(self.dv[b, j, p]), nv[b, j])
                        assert np.array_equal(self.k_ref[b, j, p], nk[b, j])
        self.prev = e_gpu.astype(np.int32)
        self.dprev = ev.clone()
        self.t += 1
        return out, sc, ev

    def check_full_cache(self):
        """The GPU cache equals the oracle's cache bitwise for every pair
        (every step's write landed in its slot and nothing else changed), and
        no step set a device status bit (bad or masked prev_slot, diverged
        fill, team wait out of budget)."""
        assert self.lf.lf_read_device_status(self.ws) == 0
        for b in range(self.wl.B):
            assert np.array_equal(bf16_host(self.dk[b]), self.k_ref[b]), f"K cache of sequence {b}"
            assert np.array_equal(bf16_host(self.dv[b]), self.v_ref[b]), f"V cache of sequence {b}"


def global_properties(sc, ev, dm):
    """Checks over every pair, from the GPU's own outputs: masked slots +inf,
    the evicted slot is valid, holds the minimum valid score and is the lowest
    index among slots with exactly that score; -1 only for empty rows."""
    B, Hkv, S = sc.shape
    valid = (dm != 0)[:, None, :].expand(B, Hkv, S)
    assert bool(torch.isposinf(sc[~valid]).all()), "masked score not +inf"
    any_valid = valid.any(dim=-1)
    assert bool(((ev >= 0) == any_valid).all()), "evict -1 iff no valid slot"
    e = ev.clamp(min=0).long()
    chosen = sc.gather(-1, e[..., None])[..., 0]
    smin = torch.where(valid, sc, torch.full_like(sc, float("inf"))).min(dim=-1).values
    ok = (chosen == smin) | ~any_valid
    assert bool(ok.all()), "evicted slot does not hold the minimum score"
    idx = torch.arange(S, device=sc.device).expand(B, Hkv, S)
    first = torch.where(valid & (sc == smin[..., None]), idx, torch.full_like(idx, S)).min(dim=-1).values
    assert bool(((first == e) | ~any_valid).all()), "tie not broken toward the lowest index"
    vg = torch.gather(valid, -1, e[..., None])[..., 0]
    assert bool((vg | ~any_valid).all())


class Timer:
    def __init__(self, label):
        self.label = label

    def __enter__(self):
        self.t = time.time()
        return self

    def __exit__(self, *a):
        log(f"  {self.label}: {time.time() - self.t:.1f}s")


def lowest_free(mask):
    """First free slot of each sequence, -1 for a full one."""
    free = mask == 0
    return np.where(free.any(axis=1), free.argmax(axis=1), -1).astype(np.int32)


class FillLockstep:
    """Fill steps on the GPU and in the oracle from the same state; both sides
    continue from the GPU's next slot once it has been accepted."""

    def __init__(self, wl, k, v, mask, prev, nsplit=None, split_path=None):
        from decode_attention_kv_05_amd import longflow as lf
        self.lf, self.wl, self.nsplit, self.split_path = lf, wl, nsplit, split_path
        self.k_ref, self.v_ref, self.mask = k, v, mask.copy()
        self.dk, self.dv = bf16_dev(k), bf16_dev(v)
        self.dm = torch.from_numpy(mask.copy()).cuda()
        self.prev = prev.astype(np.int32)
        self.dprev = torch.from_numpy(self.prev.copy()).cuda()
        self.ws = lf.new_workspace(wl.B, wl.Hq, wl.Hkv, wl.d, wl.S, nsplit)
        self.t = 0
        self.exact = self.total = 0
        self.last = None

    def step(self, use_fill=True):
        wl, t = self.wl, self.t
        q, nk, nv = W.step_inputs(wl, t)
        entry = self.lf.longflow_decode_fill if use_fill else self.lf.longflow_decode
        out, sc, nx = entry(bf16_dev(q), self.dk, self.dv, self.dm, bf16_dev(nk), bf16_dev(nv), self.dprev,
                            scale=float(wl.scale), workspace=self.ws, nsplit=self.nsplit,
                            split_path=self.split_path)
        torch.cuda.synchronize()
        if use_fill:
            o_ref, s_ref, n_ref, m_ref = decode_step_fill(q, self.k_ref, self.v_ref, self.mask, nk, nv,
                                                          self.prev, wl.scale)
        else:
            o_ref, s_ref, n_ref = decode_step(q, self.k_ref, self.v_ref, self.mask, nk, nv, self.prev, wl.scale)
            m_ref = self.mask
        m_gpu = self.dm.cpu().numpy()
        assert np.array_equal(m_gpu, m_ref), f"{wl.name} t={t}: mask differs"
        o_gpu = bf16_value(bf16_host(out))
        s_gpu = sc.cpu().numpy().astype(np.float64)
        n_gpu = nx.cpu().numpy()
        for b in range(wl.B):
            has_free = bool((m_ref[b] == 0).any())
            valid = m_ref[b] != 0
            for j in range(wl.Hkv):
                where = f"{wl.name} t={t} b={b} j={j}"
                if use_fill and has_free:
                    assert n_gpu[b, j] == n_ref[b, j], f"{where}: next slot {n_gpu[b, j]} != {n_ref[b, j]}"
                heads = slice(j * wl.G, (j + 1) * wl.G)
                self.exact += compare_pair(o_gpu[b, heads], s_gpu[b, j], n_gpu[b, j], o_ref[b, heads],
                                           s_ref[b, j], n_ref[b, j], valid, where)
                self.total += 1
                p = int(self.prev[b, j])
                if p >= 0:
                    assert np.array_equal(bf16_host(self.dk[b, j, p]), nk[b, j]), where
                    assert np.array_equal(bf16_host(self.dv[b, j, p]), nv[b, j]), where
        self.mask = m_ref.copy()
        self.prev = n_gpu.astype(np.int32)
        self.dprev = nx.clone()
        self.last = (sc, s_ref)
        self.t += 1
        return out, sc, nx

    def finish(self):
        assert self.lf.lf_read_device_status(self.ws) == 0
        for b in range(self.wl.B):
            for j in range(self.wl.Hkv):
                valid = self.mask[b] != 0
                assert np.array_equal(bf16_host(self.dk[b, j])[valid], self.k_ref[b, j][valid])
                assert np.array_equal(bf16_host(self.dv[b, j])[valid], self.v_ref[b, j][valid])
        log(f"  {self.wl.name}: {self.t} steps, next slot exact {self.exact}/{self.total}")
