"""The oracle's fill phase and several-slot eviction against their pins, and
planted mistakes (CPU copies of the oracle) that the pins must catch."""

import numpy as np
import pytest

import pins_lifecycle as PL
from oracle import attend_pair, bf16_bits_to_f64, decode_step_fill, evict_topk, write_slot


@pytest.mark.parametrize("pin", PL.FILL_PINS, ids=lambda f: f.__name__)
def test_fill_pin(pin):
    pin(decode_step_fill)


@pytest.mark.parametrize("pin", PL.TOPK_PINS, ids=lambda f: f.__name__)
def test_topk_pin(pin):
    pin(evict_topk)


def _mutant_fill(kind):
    def fill(q_bits, k_bits, v_bits, mask_in, nk, nv, prev, scale):
        B, Hq, d = q_bits.shape
        _, Hkv, S, _ = k_bits.shape
        G = Hq // Hkv
        mask_out = (np.asarray(mask_in) != 0).astype(np.uint8)
        out = np.zeros((B, Hq, d))
        scores = np.full((B, Hkv, S), np.inf)
        nxt = np.full((B, Hkv), -1, dtype=np.int32)
        for b in range(B):
            for j in range(Hkv):
                written = write_slot(k_bits[b, j], v_bits[b, j], nk[b, j], nv[b, j], prev[b, j])
                valid = (np.asarray(mask_in[b]) != 0).copy()
                if written:
                    if kind != "written_invisible":
                        valid[int(prev[b, j])] = True
                    if kind != "no_mask_update":
                        mask_out[b, int(prev[b, j])] = 1
                kk = np.zeros((S, d))
                vv = np.zeros((S, d))
                kk[valid] = bf16_bits_to_f64(k_bits[b, j][valid])
                vv[valid] = bf16_bits_to_f64(v_bits[b, j][valid])
                o, s, e = attend_pair(bf16_bits_to_f64(q_bits[b, j * G:(j + 1) * G]), kk, vv, valid, scale)
                out[b, j * G:(j + 1) * G] = o
                scores[b, j] = s
                nxt[b, j] = e
        if kind != "always_evict":
            for b in range(B):
                src = mask_in[b] if kind == "free_from_input" else mask_out[b]
                free = np.flatnonzero(np.asarray(src) == 0)
                if free.size:
                    nxt[b, :] = free[-1] if kind == "highest_free" else free[0]
        return out, scores, nxt, mask_out
    return fill


FILL_MUTANTS = ["written_invisible", "no_mask_update", "always_evict", "free_from_input", "highest_free"]


@pytest.mark.parametrize("kind", FILL_MUTANTS)
def test_fill_mutant_caught(kind):
    f = _mutant_fill(kind)
    failed = []
    for pin in PL.FILL_PINS:
        try:
            pin(f)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin catches the fill mutant {kind}"


def _mutant_topk(kind):
    def topk(scores, valid, k):
        scores = np.asarray(scores, dtype=np.float64)
        valid = np.asarray(valid, dtype=bool)
        lead = scores.shape[:-1]
        S = scores.shape[-1]
        fs = scores.reshape(-1, S)
        fv = np.broadcast_to(valid, scores.shape).reshape(-1, S)
        kk = k - 1 if kind == "one_short" else k
        out = np.full((fs.shape[0], k), -1, dtype=np.int32)
        for r in range(fs.shape[0]):
            idx = np.arange(S) if kind == "masked_too" else np.flatnonzero(fv[r])
            key = fs[r, idx]
            if kind == "nan_first":
                key = np.where(np.isnan(key), -np.inf, key)
            if kind == "high_slot_ties":
                order = idx[::-1][np.argsort(key[::-1], kind="stable")]
            else:
                order = idx[np.argsort(key, kind="stable")]
            take = order[:kk]
            if kind != "score_order":
                take = np.sort(take)
            out[r, :take.size] = take
        return out.reshape(*lead, k)
    return topk


TOPK_MUTANTS = ["one_short", "masked_too", "nan_first", "high_slot_ties", "score_order"]


@pytest.mark.parametrize("kind", TOPK_MUTANTS)
def test_topk_mutant_caught(kind):
    f = _mutant_topk(kind)
    failed = []
    for pin in PL.TOPK_PINS:
        try:
            pin(f)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin catches the top-k mutant {kind}"
