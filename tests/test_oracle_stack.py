"""The multi-layer step oracle against its pins, and planted mistakes in CPU
copies of its parts that the pins must catch."""

import numpy as np
import pytest

import pins_stack as PS
from oracle import stack_oracle as SO


def test_bf16_rounding():
    PS.pin_bf16_rounding(SO.f64_to_bf16_bits)


def test_rope():
    PS.pin_rope(SO.rope)


def test_projection():
    PS.pin_projection(SO.project)


@pytest.mark.parametrize("pin", PS.STACK_PINS, ids=lambda f: f.__name__)
def test_stack(pin):
    pin(SO.stack_step)


def _rope_interleaved(x, pos, base):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    inv = float(base) ** (-2.0 * np.arange(d // 2) / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * np.cos(ang) - b * np.sin(ang)
    out[..., 1::2] = b * np.cos(ang) + a * np.sin(ang)
    return out


_ROPE = SO.rope


def _rope_sign(x, pos, base):
    return _ROPE(x, -np.asarray(pos, dtype=np.float64), base)


def _rope_freq(x, pos, base):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    inv = float(base) ** (-1.0 * np.arange(half) / d)  # exponent halved
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * np.cos(ang) - b * np.sin(ang), b * np.cos(ang) + a * np.sin(ang)], axis=-1)


def test_rope_frequency_mutant_fails_the_rope_pin_alone():
    """The frequency schedule is pinned by pin_rope on its own (hand-derived
    angles of pairs i > 0), not only through the assembled layer."""
    with pytest.raises(AssertionError):
        PS.pin_rope(_rope_freq)


@pytest.mark.parametrize("mutant", [_rope_interleaved, _rope_sign, _rope_freq], ids=lambda f: f.__name__)
def test_rope_mutants_caught(mutant, monkeypatch):
    """Wrong pair layout, wrong direction or wrong frequencies break a RoPE
    pin or the hand-assembled layer."""
    failed = False
    try:
        PS.pin_rope(mutant)
    except AssertionError:
        failed = True
    monkeypatch.setattr(SO, "rope", mutant)
    try:
        PS.pin_one_layer(SO.stack_step)
    except AssertionError:
        failed = True
    assert failed


def _stack_no_residual(x_bits, pos, layers, Hq, Hkv, d, scale, base):
    orig = SO.bf16_bits_to_f64
    x = x_bits
    for lay in layers:
        o, _ = SO.stack_step(x, pos, [lay], Hq, Hkv, d, scale, base)
        x = SO.f64_to_bf16_bits(orig(o) - orig(x))
    return x, []


def _stack_pos_shift(x_bits, pos, layers, Hq, Hkv, d, scale, base):
    return SO.stack_step(x_bits, np.asarray(pos) + 1, layers, Hq, Hkv, d, scale, base)


def _stack_slot_kept(x_bits, pos, layers, Hq, Hkv, d, scale, base):
    saved = [lay["slot"].copy() for lay in layers]
    out = SO.stack_step(x_bits, pos, layers, Hq, Hkv, d, scale, base)
    for lay, s in zip(layers, saved):
        lay["slot"][...] = s
    return out


@pytest.mark.parametrize("mutant", [_stack_no_residual, _stack_pos_shift, _stack_slot_kept],
                         ids=lambda f: f.__name__)
def test_stack_mutants_caught(mutant):
    failed = []
    for pin in PS.STACK_PINS:
        try:
            pin(mutant)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed
