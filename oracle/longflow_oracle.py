"""Plain fp64 CPU oracle for LongFlow's fused decode step.

TEST INFRASTRUCTURE ONLY.  This module is imported by the tests, by the smoke
check and by the CPU-baseline leg of the benchmark, never by the library's
product path.  It shares no code with the HIP implementation: it neither
imports the package nor is imported by it.

Source: "LongFlow: Efficient KV Cache Compression for Reasoning Models"
(arXiv 2603.11504; card page and metadata page).

What one decode step computes, in the order the pages give it:

* Figure 2 caption, Left panel: the key/value of the current token overwrite
  the slot that the previous step selected; the static KV cache, the mask and
  the query then go through the operator, which returns the attention output
  and the slot to overwrite at the next step.
* Figure 2 caption, Right panel: attention is computed as logits S,
  probabilities P, and the product of P and V is split in two: first an
  intermediate G, then the output O from G.  The importance score
  (LongFlowScore, "I") is derived from G.
* Abstract: the score uses only the current query and keeps no state across
  steps; the operator fuses attention, importance estimation and eviction.

The pages do not spell out the form of G or of the score.  Readings taken
here (each one is also listed with the design notes of this repository):

* G[h, i, :] = p[h, i] * v[i, :] -- slot i's contribution to the output of
  query head h, so that O[h] = sum_i G[h, i, :].
* score[j, i] = sum over the query heads h of KV group j of ||G[h, i, :]||_1.
* query head h reads KV head j = h // (Hq // Hkv) (consecutive query heads
  share a KV head).
* mask[b, i] != 0 marks slot i of sequence b as valid; masked slots take no
  part in the softmax, get score +inf and are never chosen.
* evict[b, j] is the lowest index among the valid slots of minimum score;
  -1 when sequence b has no valid slot (then O = 0 and every score is +inf).
* prev_slot = -1 means "no write" (first step); any other value outside
  [0, S) is an error.
* The written slot is visible to the same step's attention (it is written
  before attention) and may itself be chosen for eviction.

Everything is float64.  bf16 inputs are decoded exactly (a bf16 value is the
upper half of an IEEE binary32).  Parity against the pages' own kernel is
unpinned: the pages print no operator values.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """Exact value of bf16 bit patterns (uint16) as float64.

    A bf16 number is the high 16 bits of an IEEE-754 binary32, so shifting the
    pattern into the top half of a 32-bit word gives the same number as a
    binary32, which float64 represents exactly.
    """
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def attend_pair(q, k, v, valid, scale, return_intermediates=False):
    """Attention, G, LongFlowScore and eviction for one (sequence, KV head).

    Figure 2 caption (Right panel): logits S, probabilities P, the split
    product P.V -> G -> O, and the score I derived from G; eviction per the
    Left panel.

    q:     float64 [Gq, d]  queries of the heads that share this KV head
    k, v:  float64 [S, d]   the whole static cache of this KV head
    valid: bool    [S]      slot validity (the mask)
    scale: float            logit scale
    Returns O [Gq, d], scores [S] (+inf at masked slots), evict (int).
    Masked rows of k and v are never read, so their contents cannot matter.
    """
    q = np.asarray(q, dtype=np.float64)
    n_slots = k.shape[0]
    idx = np.flatnonzero(np.asarray(valid, dtype=bool))
    scores = np.full(n_slots, np.inf)
    if idx.size == 0:
        out = np.zeros((q.shape[0], k.shape[1]))
        if return_intermediates:
            return out, scores, -1, None
        return out, scores, -1

    k_valid = np.asarray(k[idx], dtype=np.float64)   # [n, d]
    v_valid = np.asarray(v[idx], dtype=np.float64)   # [n, d]

    # S: one logit per (query head, valid slot).
    s = scale * (q @ k_valid.T)                      # [Gq, n]
    # P: softmax over the valid slots of each head.
    e = np.exp(s - s.max(axis=1, keepdims=True))
    p = e / e.sum(axis=1, keepdims=True)             # [Gq, n]
    # G: each slot's weighted value, per head.
    g = p[:, :, None] * v_valid[None, :, :]          # [Gq, n, d]
    # O: the sum of G over the slots.
    out = g.sum(axis=1)                              # [Gq, d]
    # I: L1 norm of G per (head, slot), summed over the heads of the group.
    scores[idx] = np.abs(g).sum(axis=2).sum(axis=0)
    # Eviction: np.argmin returns the first minimum, and idx is ascending,
    # so ties go to the lowest slot index.
    evict = int(idx[np.argmin(scores[idx])])
    if return_intermediates:
        return out, scores, evict, {"idx": idx, "s": s, "p": p, "g": g}
    return out, scores, evict


def write_slot(k_bits, v_bits, new_k_bits, new_v_bits, prev):
    """Overwrite the slot chosen at the previous step (Figure 2, Left panel).

    k_bits, v_bits: uint16 [S, d] cache of one (sequence, KV head), modified in
    place.  prev = -1 means there is nothing to write.  Returns True when a
    slot was written.
    """
    prev = int(prev)
    if prev == -1:
        return False
    if not 0 <= prev < k_bits.shape[0]:
        raise ValueError(f"prev_slot {prev} outside [0, {k_bits.shape[0]})")
    k_bits[prev] = new_k_bits
    v_bits[prev] = new_v_bits
    return True


def decode_step(q_bits, k_bits, v_bits, mask, new_k_bits, new_v_bits, prev_slot,
                scale, pairs=None):
    """One LongFlow decode step over a batch, following Figure 2 (Left panel).

    q_bits:     uint16 [B, Hq, d]        bf16 queries
    k_bits:     uint16 [B, Hkv, S, d]    bf16 key cache, updated in place
    v_bits:     uint16 [B, Hkv, S, d]    bf16 value cache, updated in place
    mask:       [B, S]                   nonzero = valid slot
    new_k_bits: uint16 [B, Hkv, d]       current token's key
    new_v_bits: uint16 [B, Hkv, d]       current token's value
    prev_slot:  int    [B, Hkv]          slot chosen at the previous step, -1 = none
    scale:      float                    logit scale (the caller's fp32 value)
    pairs:      optional iterable of (b, j) to compute; others are left as NaN
                (O), NaN (scores) and -2 (evict).  The cache writes are still
                applied only for the listed pairs.

    Returns (O float64 [B, Hq, d], scores float64 [B, Hkv, S], evict int32 [B, Hkv]).
    """
    B, Hq, d = q_bits.shape
    _, Hkv, S, _ = k_bits.shape
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    gsize = Hq // Hkv
    if pairs is None:
        pairs = [(b, j) for b in range(B) for j in range(Hkv)]
    out = np.full((B, Hq, d), np.nan)
    scores = np.full((B, Hkv, S), np.nan)
    evict = np.full((B, Hkv), -2, dtype=np.int32)
    for b, j in pairs:
        # 1. the current token's K/V go into the slot chosen last step.
        write_slot(k_bits[b, j], v_bits[b, j], new_k_bits[b, j], new_v_bits[b, j],
                   prev_slot[b, j])
        valid = np.asarray(mask[b]) != 0
        heads = slice(j * gsize, (j + 1) * gsize)
        q = bf16_bits_to_f64(q_bits[b, heads])
        # 2. attention + score + eviction over the updated static cache.
        #    Only the valid rows are decoded; attend_pair reads no others.
        k = np.zeros((S, d))
        v = np.zeros((S, d))
        k[valid] = bf16_bits_to_f64(k_bits[b, j][valid])
        v[valid] = bf16_bits_to_f64(v_bits[b, j][valid])
        o_j, s_j, e_j = attend_pair(q, k, v, valid, float(scale))
        out[b, heads] = o_j
        scores[b, j] = s_j
        evict[b, j] = e_j
    return out, scores, evict


def decode_step_fill(q_bits, k_bits, v_bits, mask_in, new_k_bits, new_v_bits, prev_slot, scale):
    """One decode step over a static cache that may still have free slots.

    The cache lifecycle of Figure 2 (Left panel), read with its mask: slots
    whose mask bit is 0 are free.  The current token is written into
    prev_slot as in decode_step, and that slot counts as valid for the same
    step whether or not its mask bit was set.  The returned mask_out is
    mask_in with every written slot set.  The slot for the next token is the
    lowest free slot of mask_out when the sequence still has one (the cache
    fills up before anything is evicted); once the cache is full it is the
    evicted slot of decode_step.  Every KV head of a sequence writes the
    same slot while the sequence is filling, so mask_out is well defined.

    Returns (O float64 [B,Hq,d], scores float64 [B,Hkv,S], next_slot int32
    [B,Hkv], mask_out uint8 [B,S]); k_bits/v_bits are updated in place.
    """
    B, Hq, d = q_bits.shape
    _, Hkv, S, _ = k_bits.shape
    gsize = Hq // Hkv
    mask_in = np.asarray(mask_in)
    mask_out = (mask_in != 0).astype(np.uint8)
    out = np.zeros((B, Hq, d))
    scores = np.full((B, Hkv, S), np.inf)
    nxt = np.full((B, Hkv), -1, dtype=np.int32)
    for b in range(B):
        for j in range(Hkv):
            written = write_slot(k_bits[b, j], v_bits[b, j], new_k_bits[b, j], new_v_bits[b, j],
                                 prev_slot[b, j])
            valid = mask_in[b] != 0
            if written:
                valid = valid.copy()
                valid[int(prev_slot[b, j])] = True
                mask_out[b, int(prev_slot[b, j])] = 1
            heads = slice(j * gsize, (j + 1) * gsize)
            k = np.zeros((S, d))
            v = np.zeros((S, d))
            k[valid] = bf16_bits_to_f64(k_bits[b, j][valid])
            v[valid] = bf16_bits_to_f64(v_bits[b, j][valid])
            o_j, s_j, e_j = attend_pair(bf16_bits_to_f64(q_bits[b, heads]), k, v, valid, float(scale))
            out[b, heads] = o_j
            scores[b, j] = s_j
            nxt[b, j] = e_j
    for b in range(B):
        free = np.flatnonzero(mask_out[b] == 0)
        if free.size:
            nxt[b, :] = free[0]
    return out, scores, nxt, mask_out


def evict_topk(scores, valid, k):
    """Several slots evicted at once (periodic compression): the set of the k
    valid slots that come first in (score, slot) order, listed in ascending
    slot order and padded with -1 when fewer than k slots are valid.  With
    k = 1 this is decode_step's eviction rule.

    Scores compare by value (so -0 equals +0 and the slot decides); NaN
    scores come after every number, +inf included.

    scores: [..., S] float; valid: [..., S] bool; returns int32 [..., k].
    """
    scores = np.asarray(scores, dtype=np.float64)
    valid = np.asarray(valid, dtype=bool)
    lead = scores.shape[:-1]
    S = scores.shape[-1]
    flat_s = scores.reshape(-1, S)
    flat_v = np.broadcast_to(valid, scores.shape).reshape(-1, S)
    out = np.full((flat_s.shape[0], k), -1, dtype=np.int32)
    for r in range(flat_s.shape[0]):
        idx = np.flatnonzero(flat_v[r])
        # (score, slot) order: a stable sort of the ascending slots by score;
        # numpy's sort places NaN after every number.
        order = idx[np.argsort(flat_s[r, idx], kind="stable")]
        take = np.sort(order[:k])
        out[r, :take.size] = take
    return out.reshape(*lead, k)
