"""The multi-layer decode step (include/longflow_stack.h) on the GPU against
the fp64 oracle (oracle/stack_oracle.py), and its HIP-graph replay against
eager launches.

Two checks, both every step:

Per layer, at the operator's own tolerances.  A twin of the state steps
through the same layers one at a time (one-layer calls, which run the same
kernels as the fused step; the twin must equal the fused step bit for bit),
and after each layer the stages are checked against the oracle fed the
GPU's own inputs of that stage:
  projection + RoPE  q, k_new, v_new from the GPU's x_l: every element
                     within one bf16 rounding of the oracle's (the GPU sums
                     in fp32, the oracle in fp64; a sum close to a bf16
                     rounding boundary can round to the neighbour), at most
                     1% of them not equal
  the operator       the oracle's decode step on the GPU's q, k_new, v_new
                     and the layer's cache: O within 1e-2 + 1e-2 |O_ref|,
                     scores within 1e-3 relative, masked +inf, the evicted
                     slot exact or within the oracle's 1e-4 near-tie band,
                     written cache rows bit-exact
  O projection +     x_{l+1} from the GPU's O and x_l: as for the projection
  residual
End to end.  The oracle runs the whole step from the token's activations
alone.  Its stages round to bf16 from fp64 where the GPU's round from fp32,
so one-ulp differences enter the residual stream at every layer and the gap
grows like a random walk, about as the square root of the depth (measured
at the Qwen3-8B shape: score differences of 5e-7 at layer 0, 7e-3 at layer
4, 1.4e-2 at layer 16 and at most 1.9e-2 by layer 36).  This check therefore
takes a depth-scaled bound, with g(l) = max(1, sqrt(l / 4)) for layer l and
G = max(1, sqrt(L / 8)) for the whole stack:
  x_out     |x - x_ref| <= G (3e-2 + 3e-2 |x_ref|) per element, mean <= G 3e-3
  scores    valid slots within g(l) 1e-2 relative, masked slots exactly +inf
  evict     equal, or within the oracle's near-tie band widened to g(l) 1e-2
            relative; both sides then continue from the GPU's choice
Eager and graph launches run the same kernels in the same order and must
agree bit for bit.
"""

import numpy as np
import pytest
import torch

from decode_attention_kv_05_amd import workloads as W
from gpu_util import bf16_dev, bf16_host, bf16_value, compare_pair, log, oracle_every_pair
from oracle import bf16_bits_to_f64
from oracle.stack_oracle import f64_to_bf16_bits, project, rope, stack_step

pytestmark = pytest.mark.gpu

X_ATOL = 3e-2
X_RTOL = 3e-2
X_MEAN = 3e-3
SCORE_RTOL = 1e-2
TIE_RTOL = 1e-2
BASE = 1e6


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    from decode_attention_kv_05_amd import longflow  # noqa: F401  (fails loudly if not built)
    yield


def depth_scale(n, per):
    return max(1.0, float(np.sqrt(n / per)))


def evict_ok(gpu, ref_scores, valid, ref, tie):
    if gpu == ref:
        return True
    if ref < 0 or gpu < 0 or not valid[gpu]:
        return False
    vals = np.sort(ref_scores[valid])
    return ref_scores[gpu] <= vals[0] * (1 + tie)


class StackCase:
    """One multi-layer state on the GPU and its oracle copy (host arrays)."""

    def __init__(self, L, B, H, Hq, Hkv, d, S, seed, kind="plain", len_lo=1, nsplit=None, shared_cache=False,
                 sample=None, chain=True):
        from decode_attention_kv_05_amd import longflow as lf
        self.lf = lf
        self.L, self.B, self.H, self.Hq, self.Hkv, self.d, self.S = L, B, H, Hq, Hkv, d, S
        self.G = Hq // Hkv
        self.seed = seed
        self.sample = list(range(B)) if sample is None else list(sample)
        wl = W.Workload(f"stack{seed}", B=B, Hq=Hq, Hkv=Hkv, d=d, S=S, steps=1, kind=kind, seed=seed,
                        len_lo=len_lo)
        self.scale = np.float32(1.0 / np.sqrt(d))
        dev = "cuda"
        self.layers_ref = []
        wq, wo, kc, vc, mk, sl, sc = [], [], [], [], [], [], []
        base_cache = W.initial_cache(wl) if shared_cache else None
        self.shared_cache = shared_cache
        chain_ref = []
        for l in range(L):
            k, v, mask = base_cache if shared_cache else W.initial_cache(wl.replace(seed=seed + 17 * l))
            w1, w2 = W.layer_weights(seed, l, H, Hq, Hkv, d)
            wq.append(bf16_dev(w1))
            wo.append(bf16_dev(w2))
            kc.append(bf16_dev(k))
            vc.append(bf16_dev(v))
            mk.append(torch.from_numpy(mask).to(dev))
            sl.append(torch.full((B, Hkv), -1, dtype=torch.int32, device=dev))
            sc.append(torch.empty((B, Hkv, S), dtype=torch.float32, device=dev))
            sb = self.sample
            self.layers_ref.append({"w_qkv": w1, "w_o": w2, "k": k[sb].copy(), "v": v[sb].copy(),
                                    "mask": mask[sb].copy(), "slot": np.full((len(sb), Hkv), -1, np.int32)})
            # the per-layer checks' oracle cache: every sequence (one shared host copy when every layer
            # starts from the same cache, which holds while no step has written to it)
            chain_ref.append({"w_qkv": w1, "w_o": w2, "k": k if shared_cache else k.copy(),
                              "v": v if shared_cache else v.copy(), "mask": mask})
        self.pos_ref = np.array([int(W.valid_length(wl, b)) for b in self.sample], dtype=np.int64)
        pos_all = np.array([int(W.valid_length(wl, b)) for b in range(B)], dtype=np.int32)
        self.x_in = torch.empty((B, H), dtype=torch.bfloat16, device=dev)
        self.x_out = torch.empty((B, H), dtype=torch.bfloat16, device=dev)
        self.pos = torch.from_numpy(pos_all).to(dev)
        self.scores = sc
        self.stack = lf.Stack(self.x_in, self.x_out, self.pos, wq, wo, kc, vc, mk, sl, sc, Hq=Hq,
                              scale=float(self.scale), rope_base=BASE, nsplit=nsplit)
        self.chain = LayerChain(self, chain_ref) if chain else None
        self.t = 0

    def load_token(self, t):
        x = W.token_activations(self.seed, t, self.B, self.H)
        self.x_in.copy_(bf16_dev(x))
        return x

    def check(self, x, where):
        """Oracle step on the sampled sequences and comparison; lockstep on evict."""
        sb = self.sample
        x_ref, trace = stack_step(x[sb], self.pos_ref, self.layers_ref, self.Hq, self.Hkv, self.d, self.scale,
                                  BASE)
        xo = bf16_value(bf16_host(self.x_out))[sb]
        xr = bf16_value(x_ref)
        err = np.abs(xo - xr)
        G = depth_scale(self.L, 8)
        assert np.all(err <= G * (X_ATOL + X_RTOL * np.abs(xr))), f"{where}: x_out max err {err.max():.3e}"
        assert err.mean() <= G * X_MEAN, f"{where}: x_out mean err {err.mean():.3e}"
        worst = 0.0
        exact = total = 0
        for l in range(self.L):
            s_gpu = self.scores[l].cpu().numpy().astype(np.float64)[sb]
            slots = self.stack.tensors["slot"][l].cpu().numpy()[sb]
            s_ref, e_ref = trace[l][5], trace[l][6]
            g = depth_scale(l, 4)
            for r in range(len(sb)):
                valid = self.layers_ref[l]["mask"][r] != 0
                for j in range(self.Hkv):
                    assert np.all(np.isposinf(s_gpu[r, j][~valid])), f"{where} l={l}: masked score"
                    rel = np.abs(s_gpu[r, j][valid] - s_ref[r, j][valid]) / s_ref[r, j][valid]
                    m = float(rel.max()) if rel.size else 0.0
                    worst = max(worst, m)
                    assert np.all(rel <= g * SCORE_RTOL), f"{where} l={l} b={sb[r]} j={j}: score rel {m:.3e}"
                    assert evict_ok(int(slots[r, j]), s_ref[r, j], valid, int(e_ref[r, j]), g * TIE_RTOL), \
                        f"{where} l={l} b={sb[r]} j={j}: evict {slots[r, j]} vs {e_ref[r, j]}"
                    exact += int(slots[r, j]) == int(e_ref[r, j])
                    total += 1
            self.layers_ref[l]["slot"][...] = slots  # lockstep on the accepted choice
        self.pos_ref += 1
        assert np.array_equal(self.pos.cpu().numpy()[sb], self.pos_ref)
        log(f"  {where}: x max err {err.max():.2e} mean {err.mean():.2e}; worst score rel {worst:.2e}; "
            f"evict exact {exact}/{total}")

    def run(self, steps, graph=None):
        if self.shared_cache and self.chain is not None:
            assert self.t + steps <= 1, "the per-layer checks share one host cache across layers for one step only"
        for _ in range(steps):
            x = self.load_token(self.t)
            if graph is None:
                self.stack.step()
            else:
                graph.launch()
            torch.cuda.synchronize()
            if self.chain is not None:
                self.chain.step(x, f"step {self.t}")
                self.chain.same_as(self, f"step {self.t}")
            self.check(x, f"step {self.t}")
            self.t += 1


def bf16_close(g_bits, r_bits, where, max_frac=0.01, mixed=None):
    """GPU and oracle bf16 results of one stage from the same inputs: every
    element within one bf16 rounding at its magnitude (2^-7 relative, plus
    1e-6 for values that cancel to near zero), at most max_frac of them not
    equal.  mixed: for a rotation, the magnitude of the pair each element
    came from; the two sides' unrotated values may already differ by one
    rounding at that magnitude, and the rotation carries it into both
    elements of the pair, so one more rounding at that magnitude is allowed."""
    g, r = bf16_value(np.asarray(g_bits)), bf16_value(np.asarray(r_bits))
    err = np.abs(g - r)
    tol = 2.0 ** -7 * np.maximum(np.abs(g), np.abs(r)) + 1e-6
    if mixed is not None:
        tol = tol + 2.0 ** -7 * mixed
    assert np.all(err <= tol), f"{where}: off by more than one rounding (max err {err.max():.3e})"
    ne = int(np.count_nonzero(np.asarray(g_bits) != np.asarray(r_bits)))
    assert ne <= max_frac * g.size + 1, f"{where}: {ne} of {g.size} elements differ"
    return ne


class LayerChain:
    """A twin of a StackCase's state stepped with one-layer calls, whose every
    stage is checked after each layer against the oracle fed the GPU's own
    inputs of that stage (the layer's x, then its q, k_new and v_new, then its
    O), at the operator's tolerances."""

    def __init__(self, case, ref):
        lf = case.lf
        L, B, H, Hq, Hkv, d, S = case.L, case.B, case.H, case.Hq, case.Hkv, case.d, case.S
        t = case.stack.tensors
        self.case, self.ref = case, ref
        self.xs = [torch.empty((B, H), dtype=torch.bfloat16, device="cuda") for _ in range(L + 1)]
        self.pos = t["pos"].clone()
        self.kc = [x.clone() for x in t["k_cache"]]
        self.vc = [x.clone() for x in t["v_cache"]]
        self.slot = [torch.full((B, Hkv), -1, dtype=torch.int32, device="cuda") for _ in range(L)]
        self.scores = [torch.empty((B, Hkv, S), dtype=torch.float32, device="cuda") for _ in range(L)]
        self.prev = [np.full((B, Hkv), -1, np.int32) for _ in range(L)]
        ws = torch.zeros(lf.lf_stack_workspace_size(1, B, H, Hq, Hkv, d, S, case.stack.nsplit), dtype=torch.uint8,
                         device="cuda")
        self.stacks = [lf.Stack(self.xs[l], self.xs[l + 1], self.pos, [t["w_qkv"][l]], [t["w_o"][l]], [self.kc[l]],
                                [self.vc[l]], [t["mask"][l]], [self.slot[l]], [self.scores[l]], Hq=Hq,
                                scale=case.stack.scale, rope_base=case.stack.rope_base, advance_pos=False,
                                nsplit=case.stack.nsplit, workspace=ws) for l in range(L)]

    def step(self, x_bits, where):
        c = self.case
        B, Hq, Hkv, d = c.B, c.Hq, c.Hkv, c.d
        self.xs[0].copy_(bf16_dev(x_bits))
        pos = self.pos.cpu().numpy().astype(np.float64)[:, None]
        flips = exact = 0
        for l in range(c.L):
            here = f"{where} layer {l}"
            self.stacks[l].step()
            torch.cuda.synchronize()
            im = {k: bf16_host(v) for k, v in self.stacks[l].intermediates().items()}
            x_l, x_n = bf16_host(self.xs[l]), bf16_host(self.xs[l + 1])
            ref = self.ref[l]
            # projection and RoPE, from the GPU's x_l
            qkv = f64_to_bf16_bits(project(x_l, ref["w_qkv"]))
            q_ref = f64_to_bf16_bits(rope(bf16_bits_to_f64(qkv[:, :Hq * d].reshape(B, Hq, d)), pos, BASE))
            k_ref = f64_to_bf16_bits(rope(bf16_bits_to_f64(qkv[:, Hq * d:(Hq + Hkv) * d].reshape(B, Hkv, d)), pos,
                                          BASE))
            v_ref = qkv[:, (Hq + Hkv) * d:].reshape(B, Hkv, d)

            def pair_mag(x):  # max(|x_i|, |x_{i+d/2}|) for both elements of each rotated pair
                a = np.abs(bf16_bits_to_f64(x))
                m = np.maximum(a[..., :d // 2], a[..., d // 2:])
                return np.concatenate([m, m], axis=-1)
            flips += bf16_close(im["q"], q_ref, f"{here}: q", mixed=pair_mag(qkv[:, :Hq * d].reshape(B, Hq, d)))
            flips += bf16_close(im["k_new"], k_ref, f"{here}: k_new",
                                mixed=pair_mag(qkv[:, Hq * d:(Hq + Hkv) * d].reshape(B, Hkv, d)))
            flips += bf16_close(im["v_new"], v_ref, f"{here}: v_new")
            # the operator, from the GPU's q, k_new and v_new, every pair
            o_ref, s_ref, e_ref = oracle_every_pair(im["q"], ref["k"], ref["v"], ref["mask"], im["k_new"],
                                                    im["v_new"], self.prev[l], c.scale)
            o_gpu = bf16_value(im["o"]).reshape(B, Hq, d)
            s_gpu = self.scores[l].cpu().numpy().astype(np.float64)
            e_gpu = self.slot[l].cpu().numpy()
            for b in range(B):
                valid = ref["mask"][b] != 0
                for j in range(Hkv):
                    heads = slice(j * c.G, (j + 1) * c.G)
                    exact += compare_pair(o_gpu[b, heads], s_gpu[b, j], e_gpu[b, j], o_ref[b, heads], s_ref[b, j],
                                          e_ref[b, j], valid, f"{here} b={b} j={j}")
                    p = int(self.prev[l][b, j])
                    if p >= 0:
                        assert np.array_equal(bf16_host(self.kc[l][b, j, p]), im["k_new"][b, j]), here
                        assert np.array_equal(bf16_host(self.vc[l][b, j, p]), im["v_new"][b, j]), here
            self.prev[l] = e_gpu.astype(np.int32)  # lockstep on the accepted slot
            # output projection and residual, from the GPU's O and x_l
            x_ref = f64_to_bf16_bits(bf16_bits_to_f64(x_l) + project(im["o"], ref["w_o"]))
            flips += bf16_close(x_n, x_ref, f"{here}: x_out")
        self.pos += 1
        log(f"  {where}: every layer's stages within the operator's tolerances on their GPU inputs "
            f"({flips} one-rounding differences in the projections, evict exact {exact}/{c.L * B * Hkv})")

    def same_as(self, case, where):
        """The one-layer calls equal the fused step bit for bit."""
        t = case.stack.tensors
        assert torch.equal(self.xs[-1].view(torch.int16), case.x_out.view(torch.int16)), f"{where}: x_out"
        assert torch.equal(self.pos, case.pos), f"{where}: pos"
        for l in range(case.L):
            assert torch.equal(self.slot[l], t["slot"][l]), f"{where} layer {l}: slots"
            assert torch.equal(self.scores[l].view(torch.int32), case.scores[l].view(torch.int32)), \
                f"{where} layer {l}: scores"
            assert torch.equal(self.kc[l].view(torch.int16), t["k_cache"][l].view(torch.int16)), f"{where}: K"
            assert torch.equal(self.vc[l].view(torch.int16), t["v_cache"][l].view(torch.int16)), f"{where}: V"


@pytest.mark.parametrize("nsplit", [1, 3])
def test_stack_small_multistep(nsplit):
    log(f"stack L=3 B=3 H=256 nsplit={nsplit}")
    case = StackCase(L=3, B=3, H=256, Hq=4, Hkv=2, d=64, S=80, seed=12000, kind="ragged", len_lo=40,
                     nsplit=nsplit)
    case.run(4)
    assert case.lf.lf_read_device_status(case.stack.tensors["workspace"]) == 0


@pytest.mark.parametrize("B", [1, 17, 40, 100, 200])
def test_stack_batch_sizes(B):
    """Batch sizes that select each row-tile instantiation of the projection
    kernel (2, 4 and 8 tiles of 16 rows) and, at 200, two 128-row blocks."""
    log(f"stack L=2 B={B}")
    case = StackCase(L=2, B=B, H=256, Hq=8, Hkv=2, d=128, S=48, seed=12100 + B,
                     sample=sorted({0, B // 2, B - 1}))
    case.run(2)


# Shapes whose two projections between them select every K-slice length the
# projection kernel is unrolled for (2 .. 16 chunks of 128): (QKV, O) =
# (6, 16), (10, 2), (12, 8), (14, 4) chunks; tests/test_abi_host.py checks
# the mapping.
SLICE_SHAPES = [(8448, 32, 8), (1280, 48, 8), (3072, 72, 9), (3584, 32, 8)]


@pytest.mark.parametrize("H,Hq,Hkv", SLICE_SHAPES)
def test_stack_projection_slice_lengths(H, Hq, Hkv):
    log(f"stack H={H} Hq={Hq} Hkv={Hkv}")
    case = StackCase(L=1, B=3, H=H, Hq=Hq, Hkv=Hkv, d=128, S=64, seed=12500 + H)
    case.run(2)


def _random_stack_cases():
    rng = np.random.default_rng(20261205)
    cases = []
    while len(cases) < 8:
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.integers(1, 9))
        Hq = G * Hkv
        if (Hq * d) % 256:
            continue
        H = 256 * int(rng.integers(1, 10))
        B = int(rng.integers(1, 41))
        S = int(rng.integers(16, 401))
        L = int(rng.integers(1, 3))
        ns = int(rng.choice([0, 1, 2, 3]))
        cases.append((len(cases), L, B, H, Hq, Hkv, d, S, ns or None))
    return cases


@pytest.mark.parametrize("case", _random_stack_cases(), ids=lambda c: f"s{c[0]}")
def test_stack_random_shapes(case):
    """Shapes drawn once from a fixed seed: hidden width, head counts, d,
    batch, slots, depth and split count together (two steps each)."""
    i, L, B, H, Hq, Hkv, d, S, nsplit = case
    log(f"random stack {i}: L={L} B={B} H={H} Hq={Hq} Hkv={Hkv} d={d} S={S} nsplit={nsplit}")
    case = StackCase(L=L, B=B, H=H, Hq=Hq, Hkv=Hkv, d=d, S=S, seed=12600 + i, kind="ragged",
                     len_lo=max(1, S // 2), nsplit=nsplit, sample=sorted({0, B - 1}))
    case.run(2)


def test_stack_gqa8_d64():
    log("stack GQA 8, d 64")
    case = StackCase(L=2, B=4, H=512, Hq=16, Hkv=2, d=64, S=300, seed=12200, kind="sinks")
    case.run(3)


def _state(case):
    t = case.stack.tensors
    out = [bf16_host(case.x_out), case.pos.cpu().numpy()]
    for l in range(case.L):
        out += [bf16_host(t["k_cache"][l]), bf16_host(t["v_cache"][l]), t["slot"][l].cpu().numpy(),
                case.scores[l].cpu().numpy()]
    return out


def test_stack_graph_replays_match_eager():
    """Twin states: one stepped with eager launches (and checked against the
    oracle every step), the other by replaying a graph recorded once, with the
    new activations copied in between replays; every replay must equal the
    eager step bit for bit."""
    log("stack graph vs eager")
    kw = dict(L=3, B=5, H=256, Hq=8, Hkv=4, d=64, S=120, seed=12300, kind="ragged", len_lo=60, nsplit=2, chain=False)
    eager, replay = StackCase(**kw), StackCase(**kw)
    g = replay.stack.graph()
    try:
        for t in range(5):
            x = eager.load_token(t)
            eager.stack.step()
            torch.cuda.synchronize()
            eager.check(x, f"eager step {t}")
            replay.load_token(t)
            g.launch()
            torch.cuda.synchronize()
            for a, b in zip(_state(eager), _state(replay)):
                assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"replay {t} differs"
    finally:
        g.close()


def test_stack_full_size_qwen3_8b():
    """36 layers of the Qwen3-8B shape (batch 128, 32/8 heads, d 128, 3200
    slots, hidden 4096), one step as a graph: every layer's stages for every
    (sequence, KV head) against the oracle on their GPU inputs, the one-layer
    twin bit for bit equal to the graph, and two sequences end to end."""
    log("stack full size: generating")
    case = StackCase(L=36, B=128, H=4096, Hq=32, Hkv=8, d=128, S=3200, seed=12400, shared_cache=True,
                     sample=[0, 77])
    g = case.stack.graph()
    try:
        case.run(1, graph=g)
    finally:
        g.close()
