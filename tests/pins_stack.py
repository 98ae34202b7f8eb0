"""Pins for the multi-layer step oracle (oracle/stack_oracle.py): checks
against facts other than its own code.  Each pin takes the functions under
test, so planted mistakes can be run through the same pins.

  bf16 rounding       equals torch's float32 -> bfloat16 cast (library routine)
  RoPE                pos 0 is the identity; every pair keeps its norm;
                      rotations compose (a then b = a + b); a 2-dim head at
                      position p turns (1, 0) into (cos p, sin p) (math.cos);
                      pairs i > 0 turn at hand-derived rates (d 4, base 100:
                      pair 1 by p / 10; d 8, base 10^4: pair i by p / 10^i);
                      <R(m) q, R(n) k> depends only on m - n
  projection          identity and one-hot weights select inputs exactly
  residual            W_o = 0 leaves x unchanged
  one layer           reduces to the pinned decode step on the rotated
                      projections (checked against an independent assembly)
"""

import math

import numpy as np
import torch


def _rng(seed):
    return np.random.default_rng(seed)


def pin_bf16_rounding(f64_to_bf16_bits, seed=51):
    x = _rng(seed).standard_normal(4096) * np.exp(_rng(seed + 1).uniform(-20, 20, 4096))
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f64_to_bf16_bits(x), want)


def pin_rope(rope, seed=52):
    rng = _rng(seed)
    x = rng.standard_normal((3, 5, 16))
    assert np.allclose(rope(x, np.zeros((3, 1)), 1e4), x, atol=0, rtol=0)
    y = rope(x, rng.integers(0, 5000, size=(3, 1)), 1e4)
    n_x = x[..., :8] ** 2 + x[..., 8:] ** 2
    n_y = y[..., :8] ** 2 + y[..., 8:] ** 2
    assert np.allclose(n_x, n_y, rtol=1e-12, atol=0)
    a, b = 37.0, 1234.0
    assert np.allclose(rope(rope(x, a, 1e6), b, 1e6), rope(x, a + b, 1e6), rtol=1e-9, atol=1e-12)
    p = 3.25
    r = rope(np.array([1.0, 0.0]), p, 10.0)
    assert abs(r[0] - math.cos(p)) < 1e-15 and abs(r[1] - math.sin(p)) < 1e-15
    # Pairs beyond the first, at angles derived by hand: with d = 4 and base
    # 100 the two pairs turn at 100^0 = 1 and 100^(-2/4) = 1/10 radian per
    # position; with d = 8 and base 10^4, pair i turns at (10^4)^(-2i/8) =
    # 10^-i.  Pair i couples coordinates i and i + d/2.
    for p in (1.0, 7.0, 31.25):
        r = rope(np.array([0.0, 1.0, 0.0, 0.0]), p, 100.0)
        assert abs(r[1] - math.cos(p / 10)) < 1e-15 and abs(r[3] - math.sin(p / 10)) < 1e-15
        assert r[0] == 0.0 and r[2] == 0.0
        r = rope(np.array([1.0, 0.0, 0.0, 0.0]), p, 100.0)
        assert abs(r[0] - math.cos(p)) < 1e-15 and abs(r[2] - math.sin(p)) < 1e-15
        for i in range(4):
            x8 = np.zeros(8)
            x8[i] = 1.0
            r = rope(x8, p, 1e4)
            assert abs(r[i] - math.cos(p / 10 ** i)) < 1e-15 and abs(r[i + 4] - math.sin(p / 10 ** i)) < 1e-15
            assert np.count_nonzero(r) <= 2
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for m, n in ((100, 40), (1060, 1000), (60, 0)):
        assert abs(np.dot(rope(q, m, 1e6), rope(k, n, 1e6)) - np.dot(rope(q, m - n, 1e6), k)) < 1e-9


def pin_projection(project, seed=53):
    rng = _rng(seed)
    x = (rng.integers(-64, 64, size=(4, 32)) * 16).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)  # exact in bf16
    eye = (np.eye(32, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(project(xb, eye), x.astype(np.float64))
    w = np.zeros((3, 32), dtype=np.float32)
    w[0, 5] = 1.0
    w[1, 0] = 2.0
    w[2, 31] = -0.5
    wb = (w.view(np.uint32) >> 16).astype(np.uint16)
    want = np.stack([x[:, 5], 2 * x[:, 0], -0.5 * x[:, 31]], axis=1)
    assert np.array_equal(project(xb, wb), want.astype(np.float64))


def _layers(seed, L, B, H, Hq, Hkv, d, S, zero_wo=False):
    from decode_attention_kv_05_amd import workloads as W
    rng = _rng(seed)
    out = []
    for _ in range(L):
        wq = W.f32_to_bf16_bits((rng.standard_normal(((Hq + 2 * Hkv) * d, H)) / np.sqrt(H)).astype(np.float32))
        wo = W.f32_to_bf16_bits((rng.standard_normal((H, Hq * d)) / np.sqrt(Hq * d)).astype(np.float32))
        if zero_wo:
            wo[:] = 0
        k = W.f32_to_bf16_bits(rng.standard_normal((B, Hkv, S, d)).astype(np.float32))
        v = W.f32_to_bf16_bits(rng.standard_normal((B, Hkv, S, d)).astype(np.float32))
        mask = (rng.random((B, S)) < 0.9).astype(np.uint8)
        slot = np.full((B, Hkv), -1, dtype=np.int32)
        out.append({"w_qkv": wq, "w_o": wo, "k": k, "v": v, "mask": mask, "slot": slot})
    return out


def pin_residual(stack_step, seed=54):
    from decode_attention_kv_05_amd import workloads as W
    B, H, Hq, Hkv, d, S = 2, 32, 4, 2, 8, 12
    layers = _layers(seed, 3, B, H, Hq, Hkv, d, S, zero_wo=True)
    x = W.f32_to_bf16_bits(_rng(seed).standard_normal((B, H)).astype(np.float32))
    out, _ = stack_step(x, np.array([3, 9]), layers, Hq, Hkv, d, 1 / np.sqrt(d), 1e6)
    assert np.array_equal(out, x)


def pin_one_layer(stack_step, seed=55):
    """One layer assembled by hand from numpy and the pinned decode step."""
    from decode_attention_kv_05_amd import workloads as W
    from oracle import bf16_bits_to_f64, decode_step
    B, H, Hq, Hkv, d, S = 2, 48, 4, 2, 16, 20
    base, scale = 1e4, 0.25
    lay = _layers(seed, 1, B, H, Hq, Hkv, d, S)
    ref = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in lay[0].items()}
    x = W.f32_to_bf16_bits(_rng(seed).standard_normal((B, H)).astype(np.float32))
    pos = np.array([5, 17])
    out, trace = stack_step(x, pos, lay, Hq, Hkv, d, scale, base)

    def to_bits(a):
        return W.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))

    qkv = to_bits(bf16_bits_to_f64(x) @ bf16_bits_to_f64(ref["w_qkv"]).T)
    f = bf16_bits_to_f64(qkv)
    half = d // 2
    ang = pos[:, None, None] * (base ** (-np.arange(half) / half))[None, None, :]

    def rot(t):
        return np.concatenate([t[..., :half] * np.cos(ang) - t[..., half:] * np.sin(ang),
                               t[..., half:] * np.cos(ang) + t[..., :half] * np.sin(ang)], axis=-1)
    q = to_bits(rot(f[:, :Hq * d].reshape(B, Hq, d)))
    kn = to_bits(rot(f[:, Hq * d:(Hq + Hkv) * d].reshape(B, Hkv, d)))
    vn = qkv[:, (Hq + Hkv) * d:].reshape(B, Hkv, d)
    o, s, e = decode_step(q, ref["k"], ref["v"], ref["mask"], kn, vn, ref["slot"], scale)
    ob = to_bits(o.reshape(B, Hq * d))
    want = to_bits(bf16_bits_to_f64(x) + bf16_bits_to_f64(ob) @ bf16_bits_to_f64(ref["w_o"]).T)
    assert np.array_equal(out, want)
    assert np.array_equal(trace[0][1], q) and np.array_equal(trace[0][2], kn)
    assert np.array_equal(lay[0]["slot"], e)
    assert np.array_equal(lay[0]["k"], ref["k"])


STACK_PINS = [pin_residual, pin_one_layer]
