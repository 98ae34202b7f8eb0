"""Seeded input generators: rounding, determinism and the structure each
workload kind promises (CPU only, reduced batch sizes)."""

import numpy as np
import torch

from decode_attention_kv_05_amd import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 7,
        # exact halfway cases: 1 + 2^-8 rounds to 1 (even), 1 + 3*2^-8 rounds up
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3.0e38, 1e-40], dtype=np.float32),
    ])
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_named_workloads_have_the_stated_shapes():
    t = W.WORKLOADS
    assert (t["tiny"].B, t["tiny"].Hq, t["tiny"].Hkv, t["tiny"].d, t["tiny"].S, t["tiny"].valid, t["tiny"].steps) == (1, 4, 1, 64, 256, 200, 16)
    assert (t["qwen3_8b"].B, t["qwen3_8b"].G, t["qwen3_8b"].d, t["qwen3_8b"].S, t["qwen3_8b"].steps) == (128, 4, 128, 3200, 32)
    assert (t["llama8b_budget"].B, t["llama8b_budget"].S, t["llama8b_budget"].steps) == (64, 2400, 512)
    assert (t["long_reasoning"].B, t["long_reasoning"].G, t["long_reasoning"].S) == (16, 8, 16384)
    assert (t["ragged"].B, t["ragged"].S, t["ragged"].steps) == (256, 8192, 32)
    assert t["qwen3_8b"].scale == np.float32(1 / np.sqrt(128))


def test_generation_is_deterministic_and_sequence_keyed():
    wl = W.WORKLOADS["qwen3_8b"].replace(B=6, S=96)
    k1, v1, m1 = W.initial_cache(wl)
    k2, v2, m2 = W.initial_cache(wl, batch=[4, 1])
    assert np.array_equal(k1[[4, 1]], k2) and np.array_equal(v1[[4, 1]], v2) and np.array_equal(m1[[4, 1]], m2)
    q1, nk1, nv1 = W.step_inputs(wl, 3)
    q2, nk2, nv2 = W.step_inputs(wl, 3, batch=[5])
    assert np.array_equal(q1[5], q2[0]) and np.array_equal(nk1[5], nk2[0]) and np.array_equal(nv1[5], nv2[0])
    q3, _, _ = W.step_inputs(wl, 4)
    assert not np.array_equal(q1, q3)


def _f(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_tiny_mask_and_poison():
    wl = W.WORKLOADS["tiny"]
    k, v, m = W.initial_cache(wl)
    assert m.shape == (1, 256) and m[0, :200].all() and not m[0, 200:].any()
    assert np.all(k[0, 0, 200:] == W.BF16_NAN) and np.all(v[0, 0, 200:] == W.BF16_NAN)
    kf = _f(k[0, 0, :200])
    assert abs(kf.mean()) < 0.05 and abs(kf.std() - 1) < 0.05


def test_sinks_structure():
    wl = W.WORKLOADS["llama8b_budget"].replace(B=2)
    k, v, m = W.initial_cache(wl)
    q, _, _ = W.step_inputs(wl, 0)
    kf = _f(k[0, 0])
    norms = np.linalg.norm(kf, axis=1)
    u = kf[0] / norms[0]
    cos = kf @ u / norms
    assert np.all(cos[:4] > 0.999)
    planted = np.flatnonzero((cos > 0.75) & (cos < 0.85))
    assert len(planted) == 24  # 1% of 2400
    assert np.all(np.abs(norms[planted] / np.sqrt(128) - 1) < 0.01)
    # the queries of group 0 lean along u: E[q.u] = sqrt(d / 2)
    qf = _f(q[0, :4])
    assert np.all(qf @ u > 3)


def test_lognormal_v_structure():
    wl = W.WORKLOADS["long_reasoning"].replace(B=1, S=4096)
    _, v, _ = W.initial_cache(wl)
    n = np.linalg.norm(_f(v[0]).reshape(-1, 128), axis=1) / np.sqrt(128)
    assert abs(np.log(n).std() - 0.5) < 0.03


def test_ragged_structure():
    wl = W.WORKLOADS["ragged"].replace(B=6)
    k, v, m = W.initial_cache(wl)
    for b in range(wl.B):
        L = int(m[b].sum())
        assert 256 <= L <= 8192 and m[b, :L].all()
        assert np.all(k[b, :, L:] == W.BF16_NAN)
        rows = k[b, 0, :L].view(np.dtype((np.void, 256)))
        _, counts = np.unique(rows, return_counts=True)
        exact = int((counts - 1).sum())
        n_twin = int(round(0.02 * L))
        # even twins are exact copies of their source
        assert exact == (n_twin + 1) // 2
