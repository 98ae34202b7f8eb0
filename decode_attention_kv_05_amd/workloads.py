"""Seeded synthetic inputs for the LongFlow decode step.

This module only draws random numbers and lays them out; it holds none of the
attention, scoring or eviction arithmetic.  Both the HIP path (benchmark,
tests) and the CPU oracle (tests) take their inputs from here.

Every random slice comes from its own PCG64 stream keyed by
``SeedSequence([workload_seed, purpose, step, b])``, so any one sequence ``b``
of any step can be regenerated on its own (that is how the full-size tests
check sampled pairs against the oracle without building the oracle's copy of
the whole batch).  Samples are float32 normals rounded to bf16 with
round-to-nearest-even; masked slots are filled with a bf16 NaN so that a
kernel that reads them shows it.

The five named workloads follow the shapes of the source's experiments:
Figure 1 (Qwen3-8B, batch 128, length 3200, one eviction per attention call),
Table 1 (DeepSeek-R1-Distill-Llama-8B at a budget of 2400 slots) and the
abstract's 80% compression of long reasoning outputs.
"""

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BF16_NAN = 0x7FC0

# Purpose codes of the keyed streams.
_K, _V, _Q, _NEWK, _NEWV, _DIR, _PLANT, _TWIN, _LEN, _VNORM, _NEWVNORM, _HOLES, _SCORES, _WQKV, _WO, _X = range(1, 17)

KINDS = ("plain", "sinks", "lognormal_v", "ragged")


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and structure of one synthetic decode workload.

    kind:
      plain        Q/K/V ~ N(0, 1).
      sinks        4 sink slots (0..3) and 1% planted slots whose keys point
                   along a per-(sequence, KV head) query direction u (cosine
                   1 and 0.8); queries are (z + sqrt(d) u) / sqrt(2).
      lognormal_v  V rows are N(0, I) times exp(0.5 xi), xi ~ N(0, 1).
      ragged       valid length L_b ~ U{len_lo..S} per sequence (mask = first
                   L_b slots), plus 2% twin slots: even twins copy another
                   slot's K/V exactly, odd twins differ by one bf16 ulp in one
                   key coordinate.
    valid: number of leading valid slots for the non-ragged kinds (0 = all).
    """

    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    S: int
    steps: int
    kind: str = "plain"
    seed: int = 0
    valid: int = 0
    len_lo: int = 256

    def __post_init__(self):
        if self.kind not in KINDS:
            raise ValueError(f"unknown workload kind {self.kind!r}")
        if self.Hq % self.Hkv:
            raise ValueError("Hq must be a multiple of Hkv")

    @property
    def G(self):
        return self.Hq // self.Hkv

    @property
    def scale(self):
        """The 1/sqrt(d) logit scale as the float32 value handed to the operator."""
        return np.float32(1.0 / np.sqrt(np.float64(self.d)))

    def replace(self, **kw):
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # batch 1, 4 query heads on 1 KV head, d 64, 256 slots of which 200 valid.
    "tiny": Workload("tiny", 1, 4, 1, 64, 256, 16, "plain", 1000, valid=200),
    # Qwen3-8B-shaped layer: the Figure 1 shape (batch 128, length 3200).
    "qwen3_8b": Workload("qwen3_8b", 128, 32, 8, 128, 3200, 32, "plain", 2000),
    # Llama-8B-shaped budget cache of 2400 slots with sinks and planted keys.
    "llama8b_budget": Workload("llama8b_budget", 64, 32, 8, 128, 2400, 512, "sinks", 3000),
    # GQA-8 long reasoning cache: 16384 slots = 20% of 81920 generated tokens.
    "long_reasoning": Workload("long_reasoning", 16, 64, 8, 128, 16384, 64, "lognormal_v", 4000),
    # Ragged batch with near-duplicate keys.
    "ragged": Workload("ragged", 256, 32, 8, 128, 8192, 32, "ragged", 5000),
}

HEADLINE = "qwen3_8b"


def _rng(wl, purpose, step, b):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, purpose, step, b])))


def f32_to_bf16_bits(x):
    """Round finite float32 values to bf16 bit patterns, nearest-even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def _batch_list(wl, batch):
    if batch is None:
        return list(range(wl.B))
    out = [int(b) for b in batch]
    for b in out:
        if not 0 <= b < wl.B:
            raise ValueError(f"sequence {b} outside [0, {wl.B})")
    return out


def _workers(n):
    return max(1, min(n, 16, len(os.sched_getaffinity(0))))


def valid_length(wl, b):
    """Number of leading valid slots of sequence b."""
    if wl.kind == "ragged":
        lo = min(wl.len_lo, wl.S)
        return int(_rng(wl, _LEN, 0, b).integers(lo, wl.S + 1))
    return wl.valid if wl.valid else wl.S


def mask_for(wl, batch=None):
    """uint8 [nb, S]: 1 for the first valid_length(b) slots, 0 after."""
    bl = _batch_list(wl, batch)
    m = np.zeros((len(bl), wl.S), dtype=np.uint8)
    for r, b in enumerate(bl):
        m[r, :valid_length(wl, b)] = 1
    return m


def _direction(wl, b):
    """Per-KV-head unit query direction u [Hkv, d] (float64) of the sinks kind."""
    u = _rng(wl, _DIR, 0, b).standard_normal((wl.Hkv, wl.d))
    return u / np.linalg.norm(u, axis=1, keepdims=True)


def _cache_for_sequence(wl, b):
    Hkv, S, d = wl.Hkv, wl.S, wl.d
    kf = _rng(wl, _K, 0, b).standard_normal((Hkv, S, d), dtype=np.float32)
    vf = _rng(wl, _V, 0, b).standard_normal((Hkv, S, d), dtype=np.float32)
    if wl.kind == "sinks":
        u = _direction(wl, b)
        rp = _rng(wl, _PLANT, 0, b)
        n_plant = int(round(0.01 * S))
        root_d = np.sqrt(d)
        for j in range(Hkv):
            kf[j, :min(4, S)] = (root_d * u[j]).astype(np.float32)
            if S > 4 and n_plant:
                slots = rp.choice(np.arange(4, S), size=min(n_plant, S - 4), replace=False)
                w = rp.standard_normal((slots.size, d))
                w -= (w @ u[j])[:, None] * u[j][None, :]
                w /= np.linalg.norm(w, axis=1, keepdims=True)
                kf[j, slots] = (root_d * (0.8 * u[j][None, :] + 0.6 * w)).astype(np.float32)
    if wl.kind == "lognormal_v":
        xi = _rng(wl, _VNORM, 0, b).standard_normal((Hkv, S))
        vf *= np.exp(0.5 * xi).astype(np.float32)[:, :, None]
    kb = f32_to_bf16_bits(kf)
    vb = f32_to_bf16_bits(vf)
    del kf, vf
    n_valid = valid_length(wl, b)
    if wl.kind == "ragged":
        rt = _rng(wl, _TWIN, 0, b)
        n_twin = int(round(0.02 * n_valid))
        for j in range(Hkv):
            if n_twin == 0 or 2 * n_twin > n_valid:
                continue
            picks = rt.choice(n_valid, size=2 * n_twin, replace=False)
            src, dst = picks[:n_twin], picks[n_twin:]
            coord = rt.integers(0, d, size=n_twin)
            kb[j, dst] = kb[j, src]
            vb[j, dst] = vb[j, src]
            odd = np.arange(n_twin) % 2 == 1
            # one bf16 ulp away from the source in one key coordinate
            kb[j, dst[odd], coord[odd]] += np.uint16(1)
    kb[:, n_valid:] = BF16_NAN
    vb[:, n_valid:] = BF16_NAN
    return kb, vb


def initial_cache(wl, batch=None):
    """Initial state: (k_bits, v_bits) uint16 [nb, Hkv, S, d] and mask uint8 [nb, S]."""
    bl = _batch_list(wl, batch)
    k = np.empty((len(bl), wl.Hkv, wl.S, wl.d), dtype=np.uint16)
    v = np.empty_like(k)

    def fill(r):
        k[r], v[r] = _cache_for_sequence(wl, bl[r])

    with ThreadPoolExecutor(_workers(len(bl))) as ex:
        list(ex.map(fill, range(len(bl))))
    return k, v, mask_for(wl, bl)


def step_inputs(wl, t, batch=None):
    """Inputs of decode step t: q_bits [nb, Hq, d], new_k_bits and new_v_bits [nb, Hkv, d]."""
    bl = _batch_list(wl, batch)
    q = np.empty((len(bl), wl.Hq, wl.d), dtype=np.uint16)
    nk = np.empty((len(bl), wl.Hkv, wl.d), dtype=np.uint16)
    nv = np.empty_like(nk)
    for r, b in enumerate(bl):
        z = _rng(wl, _Q, t, b).standard_normal((wl.Hq, wl.d), dtype=np.float32)
        if wl.kind == "sinks":
            u = _direction(wl, b)
            heads = np.arange(wl.Hq) // wl.G
            z = ((z + np.sqrt(wl.d) * u[heads]) / np.sqrt(2.0)).astype(np.float32)
        q[r] = f32_to_bf16_bits(z)
        nk[r] = f32_to_bf16_bits(_rng(wl, _NEWK, t, b).standard_normal((wl.Hkv, wl.d), dtype=np.float32))
        nvf = _rng(wl, _NEWV, t, b).standard_normal((wl.Hkv, wl.d), dtype=np.float32)
        if wl.kind == "lognormal_v":
            xi = _rng(wl, _NEWVNORM, t, b).standard_normal(wl.Hkv)
            nvf *= np.exp(0.5 * xi).astype(np.float32)[:, None]
        nv[r] = f32_to_bf16_bits(nvf)
    return q, nk, nv


def first_prev_slot(wl, batch=None):
    """prev_slot of step 0: -1 everywhere (no slot was chosen before the first step)."""
    return np.full((len(_batch_list(wl, batch)), wl.Hkv), -1, dtype=np.int32)



def holed_mask(wl, frac_valid, batch=None):
    """uint8 [nb, S]: each slot valid with probability frac_valid, drawn per
    sequence (free slots scattered through the cache)."""
    bl = _batch_list(wl, batch)
    m = np.zeros((len(bl), wl.S), dtype=np.uint8)
    for r, b in enumerate(bl):
        m[r] = _rng(wl, _HOLES, 0, b).random(wl.S) < frac_valid
    return m


def poison_free(k, v, mask):
    """Fill the K/V rows of every slot whose mask byte is 0 with a bf16 NaN."""
    free = mask == 0
    for j in range(k.shape[1]):
        k[:, j][free] = BF16_NAN
        v[:, j][free] = BF16_NAN


def synthetic_scores(B, Hkv, S, seed, kind="ties"):
    """float32 [B, Hkv, S] stand-ins for the operator's scores, for testing
    slot selection on its own.  Drawn per sequence b.
      ties     multiples of 1/8 in [0, 2): many exact ties
      spread   log-normal values, distinct almost surely
      special  ties plus about 2% each of +0/-0, +inf, NaN and negative values
    """
    out = np.empty((B, Hkv, S), dtype=np.float32)
    for b in range(B):
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _SCORES, 0, b])))
        if kind == "spread":
            out[b] = np.exp(g.standard_normal((Hkv, S))).astype(np.float32)
            continue
        x = (g.integers(0, 16, size=(Hkv, S)) / 8.0).astype(np.float32)
        if kind == "special":
            u = g.random((Hkv, S))
            x[u < 0.02] = np.float32(0.0)
            x[(u >= 0.02) & (u < 0.04)] = np.float32(-0.0)
            x[(u >= 0.04) & (u < 0.06)] = np.float32(np.inf)
            x[(u >= 0.06) & (u < 0.08)] = np.float32(np.nan)
            x[(u >= 0.08) & (u < 0.10)] *= np.float32(-1.0)
        elif kind != "ties":
            raise ValueError(f"unknown score kind {kind!r}")
        out[b] = x
    return out


def layer_weights(seed, layer, H, Hq, Hkv, d):
    """Synthetic projection weights of one attention layer (bf16 bits):
    w_qkv [(Hq + 2 Hkv) d, H] ~ N(0, 1/H) and w_o [H, Hq d] ~ N(0, 1/(Hq d)),
    so that activations keep unit scale from layer to layer."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _WQKV, layer, 0])))
    wq = g.standard_normal(((Hq + 2 * Hkv) * d, H), dtype=np.float32) * np.float32(1.0 / np.sqrt(H))
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _WO, layer, 0])))
    wo = g.standard_normal((H, Hq * d), dtype=np.float32) * np.float32(1.0 / np.sqrt(Hq * d))
    return f32_to_bf16_bits(wq), f32_to_bf16_bits(wo)


def token_activations(seed, step, B, H):
    """bf16 bits [B, H] ~ N(0, 1): the new token's input to the first layer."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _X, step, 0])))
    return f32_to_bf16_bits(g.standard_normal((B, H), dtype=np.float32))
