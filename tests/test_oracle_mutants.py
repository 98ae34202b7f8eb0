"""The pins are not vacuous: plausible mistakes planted in copies of the
oracle (on the CPU) must each break at least one pin."""

import numpy as np
import pytest

import pins
from oracle import attend_pair, bf16_bits_to_f64, write_slot


def _mutant_pair(kind):
    def pair(q, k, v, valid, scale):
        q = np.asarray(q, dtype=np.float64)
        S = k.shape[0]
        idx = np.flatnonzero(valid)
        if kind == "masked_in_softmax":
            idx = np.arange(S)
            k = np.where(np.isfinite(k), k, 0.0)
            v = np.where(np.isfinite(v), v, 0.0)
        scores = np.full(S, np.inf)
        if idx.size == 0:
            return np.zeros((q.shape[0], k.shape[1])), scores, -1
        kv, vv = k[idx], v[idx]
        sc = 1.0 if kind == "no_scale" else scale
        s = sc * (q @ kv.T)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        if kind != "unnormalised":
            p = p / p.sum(axis=1, keepdims=True)
        g = p[:, :, None] * vv[None]
        o = g.sum(axis=1)
        if kind == "no_abs":
            per = np.abs(g.sum(axis=2)).sum(axis=0)
        elif kind == "l2":
            per = np.sqrt((g ** 2).sum(axis=2)).sum(axis=0)
        elif kind == "max_over_heads":
            per = np.abs(g).sum(axis=2).max(axis=0)
        elif kind == "prob_only":
            per = p.sum(axis=0)
        else:
            per = np.abs(g).sum(axis=2).sum(axis=0)
        scores[idx] = per
        if kind == "highest_index_tie":
            sub = scores[idx]
            e = int(idx[len(sub) - 1 - np.argmin(sub[::-1])])
        elif kind == "argmax":
            e = int(idx[np.argmax(scores[idx])])
        else:
            e = int(idx[np.argmin(scores[idx])])
        return o, scores, e
    return pair


def _mutant_step(kind):
    def step(q_bits, k_bits, v_bits, mask, nk, nv, prev, scale):
        B, Hq, d = q_bits.shape
        _, Hkv, S, _ = k_bits.shape
        G = Hq // Hkv
        out = np.zeros((B, Hq, d))
        scores = np.zeros((B, Hkv, S))
        evict = np.zeros((B, Hkv), dtype=np.int32)
        for b in range(B):
            for j in range(Hkv):
                if kind != "write_after":
                    write_slot(k_bits[b, j], v_bits[b, j], nk[b, j], nv[b, j], prev[b, j])
                if kind == "modulo_groups":
                    heads = np.arange(j, Hq, Hkv)
                else:
                    heads = np.arange(j * G, (j + 1) * G)
                valid = mask[b] != 0
                k = np.zeros((S, d))
                v = np.zeros((S, d))
                k[valid] = bf16_bits_to_f64(k_bits[b, j][valid])
                v[valid] = bf16_bits_to_f64(v_bits[b, j][valid])
                o, s, e = attend_pair(bf16_bits_to_f64(q_bits[b, heads]), k, v, valid, float(scale))
                out[b, heads] = o
                scores[b, j] = s
                evict[b, j] = e
                if kind == "write_after":
                    write_slot(k_bits[b, j], v_bits[b, j], nk[b, j], nv[b, j], prev[b, j])
        return out, scores, evict
    return step


PAIR_MUTANTS = ["masked_in_softmax", "no_scale", "unnormalised", "no_abs", "l2",
                "max_over_heads", "prob_only", "highest_index_tie", "argmax"]
STEP_MUTANTS = ["write_after", "modulo_groups"]


def _fails(pin, impl):
    try:
        pin(impl)
    except (AssertionError, ValueError, IndexError, FloatingPointError):
        return True
    return False


@pytest.mark.parametrize("kind", PAIR_MUTANTS)
def test_pair_mutant_is_caught(kind):
    impl = _mutant_pair(kind)
    caught = [p.__name__ for p in pins.PAIR_PINS if _fails(p, impl)]
    assert caught, f"mutant {kind} passes every pin"


@pytest.mark.parametrize("kind", STEP_MUTANTS)
def test_step_mutant_is_caught(kind):
    impl = _mutant_step(kind)
    caught = [p.__name__ for p in pins.STEP_PINS if _fails(p, impl)]
    assert caught, f"mutant {kind} passes every pin"
