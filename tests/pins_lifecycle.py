"""Pins for the oracle's cache-lifecycle functions: the fill phase
(decode_step_fill) and several-slot eviction (evict_topk).

As in pins.py, each pin takes the implementation under test as an argument,
so the same pins run against the oracle (all must pass) and against planted
mistakes (each must fail at least one).

Signatures:
  fill(q_bits, k_bits, v_bits, mask, new_k_bits, new_v_bits, prev, scale)
      -> (O [B, Hq, d], scores [B, Hkv, S], next [B, Hkv], mask_out [B, S])
  topk(scores [..., S], valid [..., S], k) -> int32 [..., k]

What pins what (source: LongFlow, arXiv 2603.11504, Figure 2 caption, Left
panel: write the chosen slot, attend, return the next slot):
  causal fill           filling an empty cache slot by slot is plain causal
                        decode attention: O equals torch SDPA over the tokens
                        written so far, scores equal |v|_1 times the summed
                        softmax weights (torch softmax), next = t + 1
  holes                 hand-worked mask with gaps: lowest free slot first
  written visible       a one-slot cache filled in one step returns v
  full cache            with no free slot the step is decode_step, which has
                        pins of its own
  free-slot poison      contents of free slots cannot change any result
  topk hand examples    hand-worked sets, NaN after +inf, -0 equal to +0
  topk separation       brute force over all pairs: every chosen (score, slot)
                        precedes every valid slot left out
  topk vs torch.topk    set equality on distinct scores (library routine)
  topk k = 1            the textbook first argmin
"""

import numpy as np
import torch

from pins import _bf16, _close, _decode


def _gqa_sdpa(q, k, v, G):
    """fp64 attention of one query per head, q [Hq, d], over k, v [Hkv, n, d],
    consecutive query heads sharing a KV head (torch SDPA)."""
    qt = torch.from_numpy(q)[None, :, None, :]
    kt = torch.from_numpy(k).repeat_interleave(G, dim=0)[None]
    vt = torch.from_numpy(v).repeat_interleave(G, dim=0)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=None)
    return o[0, :, 0].numpy()


def pin_fill_causal(fill, seed=31, B=2, Hq=8, Hkv=2, d=16, S=10, extra=3):
    """An empty cache filled one token per step, starting at slot 0."""
    rng = np.random.default_rng(seed)
    G = Hq // Hkv
    k = np.full((B, Hkv, S, d), 0x7FC0, dtype=np.uint16)  # free slots hold NaN
    v = np.full((B, Hkv, S, d), 0x7FC0, dtype=np.uint16)
    mask = np.zeros((B, S), dtype=np.uint8)
    prev = np.zeros((B, Hkv), dtype=np.int32)
    scale = 1.0 / np.sqrt(d)
    hist_k, hist_v = [], []
    for t in range(S + extra):
        q = _bf16(rng, (B, Hq, d))
        nk = _bf16(rng, (B, Hkv, d))
        nv = _bf16(rng, (B, Hkv, d))
        out, scores, nxt, mask_out = fill(q, k, v, mask, nk, nv, prev, scale)
        if t < S:
            hist_k.append(_decode(nk))
            hist_v.append(_decode(nv))
            kk = np.stack(hist_k, axis=2)  # [B, Hkv, t+1, d]
            vv = np.stack(hist_v, axis=2)
            assert np.array_equal(mask_out, (np.arange(S)[None, :] <= t).astype(np.uint8).repeat(B, 0))
            for b in range(B):
                qd = _decode(q[b])
                _close(out[b], _gqa_sdpa(qd, kk[b], vv[b], G), rtol=1e-12, atol=1e-13)
                logits = torch.from_numpy(qd.reshape(Hkv, G, d)) @ torch.from_numpy(kk[b]).transpose(1, 2)
                p = torch.softmax(logits * scale, dim=-1).numpy()  # [Hkv, G, t+1]
                want = np.abs(vv[b]).sum(axis=2) * p.sum(axis=1)      # [Hkv, t+1]
                _close(scores[b, :, :t + 1], want, rtol=1e-12)
                assert np.all(np.isinf(scores[b, :, t + 1:]))
            if t + 1 < S:
                assert np.array_equal(nxt, np.full((B, Hkv), t + 1))
            else:
                # full: the first argmin of each head's scores
                assert np.array_equal(nxt, np.argmin(scores, axis=2))
        else:
            assert np.array_equal(mask_out, mask)
            assert np.array_equal(nxt, np.argmin(scores, axis=2))
        mask = mask_out
        prev = nxt.astype(np.int32)


def pin_fill_holes(fill, seed=32):
    """Mask 1 0 1 0 0 1 with one KV head: the free slots 1, 3, 4 fill in that
    order, then eviction takes over."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, d, S = 1, 2, 1, 8, 6
    k = _bf16(rng, (B, Hkv, S, d))
    v = _bf16(rng, (B, Hkv, S, d))
    mask = np.array([[1, 0, 1, 0, 0, 1]], dtype=np.uint8)
    prev = np.full((B, Hkv), -1, dtype=np.int32)
    expect_next = [1, 3, 4]
    expect_mask = [[1, 0, 1, 0, 0, 1], [1, 1, 1, 0, 0, 1], [1, 1, 1, 1, 0, 1], [1, 1, 1, 1, 1, 1]]
    for t in range(4):
        q = _bf16(rng, (B, Hq, d))
        out, scores, nxt, mask_out = fill(q, k, v, mask, _bf16(rng, (B, Hkv, d)), _bf16(rng, (B, Hkv, d)),
                                          prev, 0.3)
        assert mask_out.tolist() == [expect_mask[t]], (t, mask_out)
        assert np.all(np.isinf(scores[0, 0][mask_out[0] == 0]))
        assert np.all(np.isfinite(scores[0, 0][mask_out[0] != 0]))
        if t < 3:
            assert int(nxt[0, 0]) == expect_next[t]
        else:
            assert int(nxt[0, 0]) == int(np.argmin(scores[0, 0]))
        mask, prev = mask_out, nxt.astype(np.int32)


def pin_fill_written_visible(fill, seed=33, G=3, d=8):
    """One slot, free: the step writes the token there and attends to it
    alone, so O = v and the score is G |v|_1; the cache is then full and the
    only slot is the next one."""
    rng = np.random.default_rng(seed)
    k = np.full((1, 1, 1, d), 0x7FC0, dtype=np.uint16)
    v = np.full((1, 1, 1, d), 0x7FC0, dtype=np.uint16)
    nk, nv = _bf16(rng, (1, 1, d)), _bf16(rng, (1, 1, d))
    out, scores, nxt, mask_out = fill(_bf16(rng, (1, G, d)), k, v, np.zeros((1, 1), np.uint8), nk, nv,
                                      np.zeros((1, 1), np.int32), 0.5)
    vd = _decode(nv[0, 0])
    _close(out[0], np.tile(vd, (G, 1)), rtol=1e-15)
    _close(scores[0, 0], [G * np.abs(vd).sum()], rtol=1e-15)
    assert int(nxt[0, 0]) == 0 and mask_out.tolist() == [[1]]
    assert np.array_equal(k[0, 0, 0], nk[0, 0]) and np.array_equal(v[0, 0, 0], nv[0, 0])


def pin_fill_full_is_decode(fill, seed=34, B=2, Hq=8, Hkv=4, d=16, S=30):
    """With every slot valid the fill step is the plain decode step."""
    from oracle import decode_step
    rng = np.random.default_rng(seed)
    k = _bf16(rng, (B, Hkv, S, d))
    v = _bf16(rng, (B, Hkv, S, d))
    mask = np.ones((B, S), dtype=np.uint8)
    q, nk, nv = _bf16(rng, (B, Hq, d)), _bf16(rng, (B, Hkv, d)), _bf16(rng, (B, Hkv, d))
    prev = rng.integers(0, S, size=(B, Hkv)).astype(np.int32)
    k2, v2 = k.copy(), v.copy()
    o1, s1, e1 = decode_step(q, k, v, mask, nk, nv, prev, 0.25)
    o2, s2, n2, m2 = fill(q, k2, v2, mask, nk, nv, prev, 0.25)
    assert np.array_equal(k, k2) and np.array_equal(v, v2)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2) and np.array_equal(e1, n2)
    assert np.array_equal(m2, mask)


def pin_fill_free_poison(fill, seed=35, B=2, Hq=4, Hkv=2, d=16, S=24):
    """Free-slot contents cannot change O, the scores or the next slot."""
    rng = np.random.default_rng(seed)
    mask = (rng.random((B, S)) < 0.6).astype(np.uint8)
    k = _bf16(rng, (B, Hkv, S, d))
    v = _bf16(rng, (B, Hkv, S, d))
    free = np.flatnonzero(mask[0] == 0)
    prev = np.full((B, Hkv), -1, dtype=np.int32)
    prev[0, :] = free[0]
    q, nk, nv = _bf16(rng, (B, Hq, d)), _bf16(rng, (B, Hkv, d)), _bf16(rng, (B, Hkv, d))
    k2, v2 = k.copy(), v.copy()
    for b in range(B):
        for j in range(Hkv):
            k2[b, j][mask[b] == 0] = 0x7FC0
            v2[b, j][mask[b] == 0] = 0xFF80
    r1 = fill(q, k, v, mask, nk, nv, prev, 0.25)
    r2 = fill(q, k2, v2, mask, nk, nv, prev, 0.25)
    for a, b in zip(r1, r2):
        assert np.array_equal(a, b)


FILL_PINS = [pin_fill_causal, pin_fill_holes, pin_fill_written_visible, pin_fill_full_is_decode,
             pin_fill_free_poison]


# ---------------------------------------------------------------- top-k

def pin_topk_hand(topk):
    inf, nan = np.inf, np.nan
    s = np.array([0.5, 0.25, 0.75, 0.25, inf, 2.0, -0.0, 0.0])
    m = np.array([1, 1, 1, 1, 1, 1, 1, 1], dtype=bool)
    assert topk(s, m, 1).tolist() == [6]            # -0 and +0 tie: lower slot
    assert topk(s, m, 2).tolist() == [6, 7]
    assert topk(s, m, 3).tolist() == [1, 6, 7]
    assert topk(s, m, 5).tolist() == [0, 1, 3, 6, 7]
    assert topk(s, m, 7).tolist() == [0, 1, 2, 3, 5, 6, 7]
    m2 = m.copy()
    m2[[1, 6]] = False
    assert topk(s, m2, 3).tolist() == [0, 3, 7]
    s3 = np.array([nan, inf, 1.0, nan])
    assert topk(s3, np.ones(4, bool), 2).tolist() == [1, 2]   # NaN after +inf
    assert topk(s3, np.ones(4, bool), 3).tolist() == [0, 1, 2]
    assert topk(s3, np.array([1, 0, 0, 1], bool), 4).tolist() == [0, 3, -1, -1]
    assert topk(s3, np.zeros(4, bool), 2).tolist() == [-1, -1]


def pin_topk_separation(topk, seed=41):
    """Random scores with many exact ties: the chosen set has min(k, n_valid)
    valid slots in ascending order, and each chosen (score, slot) precedes
    every unchosen valid one (brute force over all pairs)."""
    rng = np.random.default_rng(seed)
    for trial in range(40):
        S = int(rng.integers(1, 40))
        s = rng.integers(0, 5, size=S).astype(np.float64) * 0.5
        valid = rng.random(S) < 0.7
        k = int(rng.integers(1, S + 1))
        r = topk(s, valid, k)
        n = int(valid.sum())
        chosen = [int(x) for x in r if x >= 0]
        assert len(chosen) == min(k, n) and np.all(r[len(chosen):] == -1)
        assert chosen == sorted(chosen) and all(valid[c] for c in chosen)
        rest = [u for u in range(S) if valid[u] and u not in chosen]
        for c in chosen:
            for u in rest:
                assert (s[c], c) < (s[u], u), (trial, c, u)


def pin_topk_torch(topk, seed=42):
    """Distinct scores: the same set as torch.topk of the negated scores."""
    rng = np.random.default_rng(seed)
    for _ in range(10):
        S = int(rng.integers(5, 300))
        s = rng.permutation(S).astype(np.float64) + rng.random(S) * 0.5
        valid = rng.random(S) < 0.8
        idx = np.flatnonzero(valid)
        k = int(rng.integers(1, idx.size + 1))
        ref = idx[torch.topk(-torch.from_numpy(s[idx]), k).indices.numpy()]
        assert topk(s, valid, k).tolist() == sorted(ref.tolist())


def pin_topk_first_argmin(topk, seed=43):
    rng = np.random.default_rng(seed)
    s = rng.integers(0, 3, size=(6, 20)).astype(np.float64)
    valid = np.ones((6, 20), dtype=bool)
    r = topk(s, valid, 1)
    assert r.shape == (6, 1)
    assert np.array_equal(r[:, 0], np.argmin(s, axis=1))


TOPK_PINS = [pin_topk_hand, pin_topk_separation, pin_topk_torch, pin_topk_first_argmin]
