"""The five named workloads at full size, in the launch configuration the
benchmark times (the library's own split plan), for every decode step.

The oracle checks every (sequence, KV head) pair of the first and of the
last step, and a sample of pairs (the extremes of the batch, the shortest
and longest ragged sequences) in every step between, in lockstep: both sides
continue from the GPU's accepted slot.  Outputs are preset to sentinels
before each step, and every pair of every step is checked for being written
and for the properties that hold at any size (masked scores +inf, the
evicted slot is valid, holds the minimum score and is the lowest index among
exact ties).  At the end the whole cache equals the oracle's bit for bit."""

import pytest
import torch

from decode_attention_kv_05_amd import workloads as W
from gpu_util import Lockstep, Timer, all_outputs_written, global_properties, log, oracle_workers

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    yield


def sample_pairs(wl):
    B, H = wl.B, wl.Hkv
    pairs = {(0, 0), (B - 1, H - 1), (B // 2, H // 2), (B // 3, max(0, H - 2)), (min(1, B - 1), min(1, H - 1))}
    if wl.kind == "ragged":
        lens = [W.valid_length(wl, b) for b in range(B)]
        pairs |= {(lens.index(min(lens)), 0), (lens.index(max(lens)), H - 1)}
    return sorted(pairs)


@pytest.mark.parametrize("name", ["tiny", "qwen3_8b", "llama8b_budget", "long_reasoning", "ragged"])
def test_full_workload(name):
    wl = W.WORKLOADS[name]
    pairs = sample_pairs(wl)
    log(f"{name}: B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} d={wl.d} S={wl.S} steps={wl.steps} pairs={pairs}")
    with Timer("generate + upload"):
        ls = Lockstep(wl, pairs=pairs)
    with Timer(f"{wl.steps} lockstep steps (every pair at steps 0 and {wl.steps - 1}, "
               f"{oracle_workers()} oracle threads)"):
        for t in range(wl.steps):
            every = t in (0, wl.steps - 1)
            out, sc, ev = ls.step(all_pairs=every)
            all_outputs_written(out, sc, ev)
            global_properties(sc, ev, ls.dm)
            if every or t % 64 == 0:
                log(f"  step {t} ok ({'every pair' if every else f'{len(pairs)} pairs'} against the oracle)")
    with Timer("whole cache against the oracle's"):
        ls.check_full_cache()
    log(f"  evictions exactly equal to the oracle's: {ls.exact}/{ls.total}")


def test_full_long_reasoning_combine_path():
    """The long-reasoning cache at full size through the other way of
    finishing its split steps (logits through the workspace, combine and
    finalize kernels), for 8 steps."""
    wl = W.WORKLOADS["long_reasoning"].replace(steps=8)
    pairs = sample_pairs(wl)
    log(f"long_reasoning, combine path, {wl.steps} steps, pairs={pairs}")
    ls = Lockstep(wl, pairs=pairs, nsplit=4, split_path="combine")
    for t in range(wl.steps):
        out, sc, ev = ls.step(all_pairs=t == wl.steps - 1)
        all_outputs_written(out, sc, ev)
        global_properties(sc, ev, ls.dm)
    ls.check_full_cache()
