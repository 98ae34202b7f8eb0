"""Pins for the CPU oracle: checks against facts other than the oracle itself.

Each pin takes the implementation under test as an argument so the same pins
run against the oracle (they must all pass) and against deliberately wrong
variants of it (each variant must fail at least one pin).

Two signatures are used:
  pair(q, k, v, valid, scale) -> (O [Gq, d], scores [S], evict)   float64 inputs
  step(q_bits, k_bits, v_bits, mask, new_k_bits, new_v_bits, prev, scale)
       -> (O [B, Hq, d], scores [B, Hkv, S], evict [B, Hkv]), cache updated in place

What pins what (source: LongFlow, arXiv 2603.11504, Figure 2 caption):
  decimal brute force   softmax without max-subtraction in 50-digit arithmetic
  torch SDPA (fp64)     O, including GQA head grouping (library routine)
  q = 0                 uniform softmax: O = mean of valid v, score = G |v|_1 / n
  single valid slot     O = v, score = G |v|_1, that slot is evicted
  V >= 0                sum_i score_i = sum_h |O_h|_1 (equality case of the
                        triangle inequality)
  V -> 2V               O and scores double, eviction unchanged
  two slots             closed-form sigmoid weights
  golden fixtures       hand-derived rational examples (tests/golden)
  GQA grouping          constant-V groups give constant outputs per group
  write-before-attend   the written token attends to itself, cache bits
  mask poison           masked slot contents cannot change any result
  permutation           relabelling slots relabels scores and the eviction
  empty row             O = 0, scores +inf, evict -1
  bad prev_slot         rejected
"""

import glob
import json
import math
import os
import struct
from decimal import Decimal, getcontext

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")


def _bf16(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    u = x.view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def _bits_value(b):
    return struct.unpack("<f", struct.pack("<I", int(b) << 16))[0]


def _decode(bits):
    """bf16 bits -> float64 via struct, independent of the oracle's decoder."""
    flat = [_bits_value(b) for b in np.asarray(bits).ravel()]
    return np.array(flat, dtype=np.float64).reshape(np.asarray(bits).shape)


def _close(a, b, rtol, atol=0.0):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    fin = np.isfinite(b)
    assert np.array_equal(np.isinf(a), np.isinf(b)), "inf pattern differs"
    err = np.abs(a[fin] - b[fin])
    tol = atol + rtol * np.abs(b[fin])
    assert np.all(err <= tol), f"max err {err.max() if err.size else 0} (rtol {rtol}, atol {atol})"


# ---------------------------------------------------------------- pair level

def decimal_reference(q_bits, k_bits, v_bits, valid, scale, digits=50):
    """50-digit brute force: logits, exp without max subtraction, normalise,
    G, O, scores, and the lowest-index argmin by sorting (score, index)."""
    getcontext().prec = digits
    Q = [[Decimal(_bits_value(x)) for x in row] for row in q_bits]
    idx = [i for i in range(len(valid)) if valid[i]]
    K = {i: [Decimal(_bits_value(x)) for x in k_bits[i]] for i in idx}
    V = {i: [Decimal(_bits_value(x)) for x in v_bits[i]] for i in idx}
    sc = Decimal(float(scale))
    d = len(Q[0])
    out = []
    score = {i: Decimal(0) for i in idx}
    for qh in Q:
        e = {i: (sc * sum(qh[c] * K[i][c] for c in range(d))).exp() for i in idx}
        z = sum(e.values())
        o = [Decimal(0)] * d
        for i in idx:
            p = e[i] / z
            g = [p * V[i][c] for c in range(d)]
            o = [o[c] + g[c] for c in range(d)]
            score[i] += sum(abs(x) for x in g)
        out.append([float(x) for x in o])
    scores = np.full(len(valid), np.inf)
    for i in idx:
        scores[i] = float(score[i])
    evict = sorted((score[i], i) for i in idx)[0][1] if idx else -1
    return np.array(out), scores, evict


def pin_decimal_bruteforce(pair, seed=11, G=4, d=64, S=256, n_valid=200):
    """The tiny workload's shape: 4 heads on 1 KV head, d 64, 256 slots, 200 valid."""
    rng = np.random.default_rng(seed)
    qb, kb, vb = _bf16(rng, (G, d)), _bf16(rng, (S, d)), _bf16(rng, (S, d))
    valid = np.zeros(S, dtype=bool)
    valid[:n_valid] = True
    scale = np.float32(1.0 / math.sqrt(d))
    o_ref, s_ref, e_ref = decimal_reference(qb, kb, vb, valid, scale)
    o, s, e = pair(_decode(qb), _decode(kb), _decode(vb), valid, float(scale))
    _close(o, o_ref, rtol=1e-12, atol=1e-13)
    _close(s, s_ref, rtol=1e-12)
    assert e == e_ref, (e, e_ref)


def pin_q_zero(pair, seed=12, G=4, d=16, S=40):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((S, d))
    v = rng.standard_normal((S, d))
    valid = rng.random(S) < 0.7
    valid[[3, 9]] = True
    # slot 9 duplicates slot 3 and both carry the smallest |v|_1
    v[3] = 0.01 * rng.standard_normal(d)
    v[9] = v[3]
    v[5] = v[3] * 0.5
    valid[5] = False  # smaller still, but masked
    q = np.zeros((G, d))
    o, s, e = pair(q, k, v, valid, 0.25)
    n = valid.sum()
    l1 = np.abs(v).sum(axis=1)
    _close(o, np.tile(v[valid].mean(axis=0), (G, 1)), rtol=1e-12, atol=1e-14)
    want = np.where(valid, G * l1 / n, np.inf)
    _close(s, want, rtol=1e-12)
    assert e == 3, e


def pin_single_valid(pair, G=2, d=8, S=12, slot=7, seed=13):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((G, d))
    k = rng.standard_normal((S, d))
    v = rng.standard_normal((S, d))
    valid = np.zeros(S, dtype=bool)
    valid[slot] = True
    o, s, e = pair(q, k, v, valid, 0.3)
    _close(o, np.tile(v[slot], (G, 1)), rtol=1e-14, atol=0)
    want = np.full(S, np.inf)
    want[slot] = G * np.abs(v[slot]).sum()
    _close(s, want, rtol=1e-14)
    assert e == slot


def pin_empty(pair, G=3, d=4, S=5):
    q = np.ones((G, d))
    k = np.full((S, d), np.nan)
    v = np.full((S, d), np.nan)
    o, s, e = pair(q, k, v, np.zeros(S, dtype=bool), 1.0)
    assert np.array_equal(o, np.zeros((G, d)))
    assert np.all(np.isposinf(s))
    assert e == -1


def pin_nonneg_equality(pair, seed=14, G=4, d=32, S=100):
    """With v >= 0 every G entry is >= 0, so |O_h|_1 = sum_i |G_hi|_1 and the
    scores of a group add up to the L1 norms of the group's outputs.  With
    signed v the sum is strictly larger (triangle inequality)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((G, d))
    k = rng.standard_normal((S, d))
    valid = rng.random(S) < 0.8
    v = np.abs(rng.standard_normal((S, d)))
    o, s, _ = pair(q, k, v, valid, 0.2)
    total = np.abs(o).sum()
    assert abs(s[valid].sum() - total) <= 1e-12 * total
    o2, s2, _ = pair(q, k, v - 0.5, valid, 0.2)
    assert s2[valid].sum() > np.abs(o2).sum() * (1 + 1e-6)


def pin_v_scaling(pair, seed=15, G=4, d=16, S=64):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((G, d))
    k = rng.standard_normal((S, d))
    v = rng.standard_normal((S, d))
    valid = rng.random(S) < 0.9
    o, s, e = pair(q, k, v, valid, 0.25)
    o2, s2, e2 = pair(q, k, 2.0 * v, valid, 0.25)
    _close(o2, 2.0 * o, rtol=1e-15, atol=0)
    _close(s2, 2.0 * s, rtol=1e-15)
    assert e2 == e


def pin_two_slots(pair):
    """Two valid slots, scalar keys: p_1 = 1 / (1 + exp(scale q (k2 - k1)))."""
    scale = 0.5
    q = np.array([[1.5], [-0.75]])
    k = np.array([[2.0], [-1.0], [np.nan]])
    v = np.array([[3.0], [-4.0], [np.nan]])
    valid = np.array([True, True, False])
    p1 = np.array([1.0 / (1.0 + math.exp(scale * qh * (k[1, 0] - k[0, 0]))) for qh in q[:, 0]])
    p2 = 1.0 - p1
    o, s, e = pair(q, k, v, valid, scale)
    _close(o[:, 0], p1 * 3.0 + p2 * -4.0, rtol=1e-14, atol=1e-15)
    want = np.array([3.0 * p1.sum(), 4.0 * p2.sum(), np.inf])
    _close(s, want, rtol=1e-14)
    assert e == int(np.argmin(want[:2]))


def load_golden():
    cases = []
    for path in sorted(glob.glob(os.path.join(GOLDEN, "*.json"))):
        with open(path) as f:
            cases.append((os.path.basename(path), json.load(f)))
    return cases


def pin_golden(pair):
    cases = load_golden()
    assert cases, "no golden fixtures"
    for name, c in cases:
        f = lambda m: np.array([[float(x) for x in row] for row in m])
        q, k, v = f(c["q"]), f(c["k"]), f(c["v"])
        valid = np.array(c["valid"], dtype=bool)
        o, s, e = pair(q, k, v, valid, float(c["scale"]))
        exp = c["expect"]
        _close(o, f(exp["O"]), rtol=1e-14, atol=1e-14)
        _close(s, np.array([float(x) for x in exp["scores"]]), rtol=1e-14)
        assert e == exp["evict"], (name, e)


def pin_permutation(pair, seed=16, G=4, d=16, S=48):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((G, d))
    k = rng.standard_normal((S, d))
    v = rng.standard_normal((S, d))
    valid = rng.random(S) < 0.75
    perm = rng.permutation(S)
    o, s, e = pair(q, k, v, valid, 0.25)
    o2, s2, e2 = pair(q, k[perm], v[perm], valid[perm], 0.25)
    _close(o2, o, rtol=1e-12, atol=1e-14)
    _close(s2, s[perm], rtol=1e-12)
    assert perm[e2] == e


def pin_sdpa_pair(pair, seed=17, G=8, d=32, S=90):
    """O against torch's scaled_dot_product_attention in float64 (library routine)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((G, d))
    k = rng.standard_normal((S, d))
    v = rng.standard_normal((S, d))
    valid = rng.random(S) < 0.6
    o, _, _ = pair(q, k, v, valid, 0.125)
    kz = np.where(valid[:, None], k, 0.0)
    vz = np.where(valid[:, None], v, 0.0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :],
        torch.from_numpy(kz)[None, None].expand(1, G, S, d).contiguous(),
        torch.from_numpy(vz)[None, None].expand(1, G, S, d).contiguous(),
        attn_mask=torch.from_numpy(valid)[None, None, None, :],
        scale=0.125,
    )[0, :, 0, :].numpy()
    _close(o, ref, rtol=1e-12, atol=1e-13)


PAIR_PINS = [pin_decimal_bruteforce, pin_q_zero, pin_single_valid, pin_empty,
             pin_nonneg_equality, pin_v_scaling, pin_two_slots, pin_golden,
             pin_permutation, pin_sdpa_pair]


# ---------------------------------------------------------------- step level

def _random_state(seed, B, Hq, Hkv, d, S, valid_frac=0.8):
    rng = np.random.default_rng(seed)
    q = _bf16(rng, (B, Hq, d))
    k = _bf16(rng, (B, Hkv, S, d))
    v = _bf16(rng, (B, Hkv, S, d))
    mask = (rng.random((B, S)) < valid_frac).astype(np.uint8)
    mask[:, 0] = 1
    nk = _bf16(rng, (B, Hkv, d))
    nv = _bf16(rng, (B, Hkv, d))
    return rng, q, k, v, mask, nk, nv


def pin_sdpa_step(step, seed=21, B=2, Hq=8, Hkv=2, d=32, S=70):
    """Whole step against SDPA with enable_gqa (torch maps query head h to KV
    head h // (Hq // Hkv)); the write is applied to the reference's copy first."""
    rng, q, k, v, mask, nk, nv = _random_state(seed, B, Hq, Hkv, d, S)
    prev = rng.integers(0, S, size=(B, Hkv)).astype(np.int32)
    kr, vr = _decode(k), _decode(v)
    for b in range(B):
        for j in range(Hkv):
            kr[b, j, prev[b, j]] = _decode(nk[b, j])
            vr[b, j, prev[b, j]] = _decode(nv[b, j])
    scale = np.float32(1.0 / math.sqrt(d))
    o, _, _ = step(q, k.copy(), v.copy(), mask, nk, nv, prev, scale)
    valid = mask != 0
    kr = np.where(valid[:, None, :, None], kr, 0.0)
    vr = np.where(valid[:, None, :, None], vr, 0.0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(_decode(q))[:, :, None, :], torch.from_numpy(kr), torch.from_numpy(vr),
        attn_mask=torch.from_numpy(valid)[:, None, None, :], scale=float(scale), enable_gqa=True,
    )[:, :, 0, :].numpy()
    _close(o, ref, rtol=1e-12, atol=1e-13)


def pin_gqa_groups(step, seed=22, B=1, Hq=6, Hkv=3, d=8, S=20):
    """KV head j holds the same value row c_j in every slot, so every query
    head of group j must output exactly c_j whatever its softmax, and the
    group's scores must add up to G |c_j|_1."""
    rng, q, k, v, mask, nk, nv = _random_state(seed, B, Hq, Hkv, d, S, valid_frac=0.9)
    G = Hq // Hkv
    rows = [np.full(d, 0x3F80 + 0x80 * j, dtype=np.uint16) for j in range(Hkv)]  # 1, 2, 4
    for j in range(Hkv):
        v[0, j, :, :] = rows[j]
        nv[0, j] = rows[j]
    prev = np.full((B, Hkv), -1, dtype=np.int32)
    o, s, _ = step(q, k.copy(), v.copy(), mask, nk, nv, prev, np.float32(0.3))
    for h in range(Hq):
        c = _decode(rows[h // G])
        _close(o[0, h], c, rtol=1e-13, atol=0)
    for j in range(Hkv):
        total = s[0, j][mask[0] != 0].sum()
        want = G * np.abs(_decode(rows[j])).sum()
        assert abs(total - want) <= 1e-12 * want, (j, total, want)


def pin_write_then_attend(step, seed=23, B=1, Hq=4, Hkv=1, d=64, S=32):
    """The new token lands in prev_slot before attention: with its key along
    the queries (logit 512 vs at most ~40 elsewhere) the output is its value.
    The cache must hold the new bits at prev_slot and be unchanged elsewhere."""
    rng, q, k, v, mask, nk, nv = _random_state(seed, B, Hq, Hkv, d, S, valid_frac=1.0)
    q[:] = 0
    q[:, :, 0] = 0x4280  # 64.0
    nk[:] = 0
    nk[:, :, 0] = 0x4280
    prev = np.array([[5]], dtype=np.int32)
    k0, v0 = k.copy(), v.copy()
    o, _, _ = step(q, k, v, mask, nk, nv, prev, np.float32(0.125))
    _close(o[0], np.tile(_decode(nv[0, 0]), (Hq, 1)), rtol=1e-12, atol=1e-14)
    assert np.array_equal(k[0, 0, 5], nk[0, 0]) and np.array_equal(v[0, 0, 5], nv[0, 0])
    others = np.arange(S) != 5
    assert np.array_equal(k[0, 0, others], k0[0, 0, others])
    assert np.array_equal(v[0, 0, others], v0[0, 0, others])


def pin_mask_poison(step, seed=24, B=2, Hq=4, Hkv=2, d=16, S=50):
    """NaN in masked slots and random bits in masked slots give bitwise the
    same O, scores and evict."""
    rng, q, k, v, mask, nk, nv = _random_state(seed, B, Hq, Hkv, d, S, valid_frac=0.6)
    prev = np.full((B, Hkv), -1, dtype=np.int32)
    bad = mask[:, None, :, None] == 0
    ka = np.where(bad, np.uint16(0x7FC0), k)
    va = np.where(bad, np.uint16(0x7FC0), v)
    kb = np.where(bad, rng.integers(0, 1 << 16, size=k.shape).astype(np.uint16), k)
    vb = np.where(bad, rng.integers(0, 1 << 16, size=v.shape).astype(np.uint16), v)
    r1 = step(q, ka, va, mask, nk, nv, prev, np.float32(0.25))
    r2 = step(q, kb, vb, mask, nk, nv, prev, np.float32(0.25))
    for a, b in zip(r1, r2):
        assert np.array_equal(a, b, equal_nan=True) if np.asarray(a).dtype.kind == "f" else np.array_equal(a, b)
    assert np.all(np.isposinf(r1[1][np.broadcast_to(mask[:, None, :] == 0, r1[1].shape)]))


def pin_bad_prev(step, B=1, Hq=2, Hkv=1, d=8, S=10):
    _, q, k, v, mask, nk, nv = _random_state(25, B, Hq, Hkv, d, S)
    for bad in (S, -2):
        try:
            step(q, k, v, mask, nk, nv, np.array([[bad]], dtype=np.int32), np.float32(1.0))
        except ValueError:
            continue
        raise AssertionError(f"prev_slot {bad} accepted")


STEP_PINS = [pin_sdpa_step, pin_gqa_groups, pin_write_then_attend, pin_mask_poison, pin_bad_prev]
