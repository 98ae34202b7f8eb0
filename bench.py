"""Benchmark of the fused LongFlow decode step (attention + LongFlowScore +
eviction) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload qwen3_8b]
                    [--mode decode|fill|topk|cadence]

A step is one call of the operator: the KV-slot write of the previous choice,
attention over the static cache with its mask, the per-slot scores and the
next evicted slot for every (sequence, KV head), all in one kernel launch.
The default workload is the Qwen3-8B-shaped layer (batch 128, 32 query / 8
KV heads, d 128, 3200 slots, bf16 K/V).  Inputs of every step are generated
and uploaded before timing; the evicted slots go from step to step on the
device.  After at least W warm-up steps and at least one second of them
(clocks ramp up over the first milliseconds), K steps are timed between one
pair of events, five times over; the median of the five is the reported
time per step.  K further steps, each between its own pair of events, give
per-launch durations as a second figure, and plain device copy and read
probes on the same GPU give its practical HBM rates.  Prints one JSON
line.

Other modes measure the cache-lifecycle entry points on the same shape:
  fill     longflow_decode_fill: every timed pass starts from caches K slots
           short of full (the mask and the first slot restored before each
           pass) and reaches full at its last step (the mask grows by one
           slot per sequence and step)
  topk     longflow_evict_topk choosing --topk-k slots from synthetic scores
  cadence  longflow_decode with the written slots taken from a top-k queue
           refreshed every --cadence steps (periodic compression)
  stack    the attention module of a Qwen3-8B-shaped model: --layers layers
           (default 36) of QKV projection, RoPE, the LongFlow step and the
           output projection with residual, replayed as one HIP graph per
           token (synthetic weights; every layer's cache starts as a copy of
           the workload's cache)
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused decode-attn+evict: KV GB/s (% HBM peak), steps/s at B=128, 3200 slots"
HBM_PEAK_GBPS = 8000.0
REPEATS = 5            # timed repeats of K steps; the median is reported
WARMUP_MIN_S = 1.0     # warm-up lasts at least this long, whatever W says
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def valid_slots(mask):
    return int(np.count_nonzero(mask))


def kv_bytes(wl, mask):
    """Valid K and V rows read per step (bf16)."""
    return valid_slots(mask) * wl.Hkv * wl.d * 2 * 2


def algorithmic_bytes(wl, mask):
    """Bytes one step must move: valid K/V, the mask, Q, the new K/V read and
    written, O, fp32 scores of every slot, prev and evict slot indices."""
    B, Hq, Hkv, d, S = wl.B, wl.Hq, wl.Hkv, wl.d, wl.S
    return (kv_bytes(wl, mask) + B * S + B * Hq * d * 2 + 4 * B * Hkv * d * 2 + B * Hq * d * 2
            + B * Hkv * S * 4 + 2 * B * Hkv * 4)


def topk_bytes(B, Hkv, S, k):
    """Bytes one top-k launch must move: fp32 scores, the mask, the int32 list."""
    return B * Hkv * S * 4 + B * S + k * B * Hkv * 4


def measured_traffic(tag):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current sources of the kernel family of this tag
    (workload/split, or topk/workload/k)."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(tag)
    except (OSError, ValueError):
        return None
    from decode_attention_kv_05_amd.build import source_hash
    family = "topk" if tag.startswith("topk/") else "decode"
    if not rec or rec.get("kernel_hash") != source_hash(family):
        return None
    return rec.get("bytes_per_launch")


def measured_lds(name):
    """LDS bank conflicts of the decode kernel on this workload from the
    committed rocprofv3 counter run (profiles/longflow_decode_<name>_counters.txt),
    if it was taken on the current decode sources; else None."""
    path = os.path.join(PROFILES, f"longflow_decode_{name}_counters.txt")
    try:
        with open(path) as f:
            text = f.read()
    except OSError:
        return None
    from decode_attention_kv_05_amd.build import source_hash
    if f"kernel sources (decode): {source_hash('decode')}" not in text:
        return None
    rec = {"source": os.path.relpath(path, os.path.dirname(os.path.abspath(__file__)))}
    for line in text.splitlines():
        if line.startswith("SQ_LDS_BANK_CONFLICT"):
            rec["bank_conflict_cycles_per_dispatch"] = float(line.split()[1])
        elif line.startswith("LDS bank-conflict cycles / LDS active cycles"):
            rec["bank_conflict_frac_of_lds_active"] = float(line.split()[-1])
    return rec if len(rec) == 3 else None


def host_cores():
    """Threads the CPU baseline may use: the process's CPU share, at most 16
    (the host share of one GPU)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def host_info():
    """CPU model and the BLAS library numpy runs on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info() if i.get("user_api") == "blas"]
        blas = ", ".join(libs) or "none found"
    except Exception:
        pass
    return model, blas


def _per_sequence(fn, nb, workers):
    """fn(b) for b < nb on `workers` threads (numpy releases the GIL in its
    array work); BLAS limited to one thread per worker."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1), ThreadPoolExecutor(workers) as ex:
        return list(ex.map(fn, range(nb)))


def cpu_baseline_sequences(wl, max_pairs):
    """Sequences the decode CPU baseline runs: the first ceil(max_pairs / Hkv)."""
    return max(1, min(wl.B, -(-max_pairs // wl.Hkv)))


def parity_verdict(wl, mask, gpu, ref):
    """The GPU's first step against the oracle's on the sampled sequences, by
    the acceptance rule of the parity tests: O within 1e-2 + 1e-2 |O_ref|,
    valid scores within 1e-3 relative and masked ones +inf, the evicted slot
    exact or inside a near-tie band of 1e-4 relative."""
    o_ref, s_ref, e_ref = ref
    G = wl.Hq // wl.Hkv
    n = len(e_ref)
    passed = exact = 0
    o_err = s_rel = 0.0
    for b in range(n):
        valid = mask[b] != 0
        for j in range(wl.Hkv):
            og, orf = gpu["out"][b, j * G:(j + 1) * G], o_ref[b, j * G:(j + 1) * G]
            err = np.abs(og - orf)
            ok = bool(np.all(err <= 1e-2 + 1e-2 * np.abs(orf)))
            o_err = max(o_err, float(err.max()))
            sg, sr = gpu["scores"][b, j], s_ref[b, j]
            ok &= bool(np.all(np.isposinf(sg[~valid])))
            if valid.any():
                rel = np.abs(sg[valid] - sr[valid]) / np.maximum(sr[valid], 1e-300)
                s_rel = max(s_rel, float(rel.max()))
                ok &= bool(np.all(rel <= 1e-3))
            eg, er = int(gpu["evict"][b, j]), int(e_ref[b, j])
            if eg == er:
                exact += 1
            elif er >= 0 and 0 <= eg < wl.S and valid[eg]:
                vals = np.sort(sr[valid])
                s1, s2 = vals[0], (vals[1] if vals.size > 1 else np.inf)
                ok &= bool((sr[eg] == 0) if s1 == 0 else ((s2 - s1) / s1 < 1e-4 and sr[eg] <= s1 * (1 + 1e-4)))
            else:
                ok = False
            passed += ok
    pairs = n * wl.Hkv
    return {"verdict": "pass" if passed == pairs else "fail", "pairs": pairs, "pairs_passed": passed,
            "step": 0, "evict_exact": exact, "o_max_abs_err": o_err, "score_max_rel_err": s_rel,
            "rule": "O 1e-2 + 1e-2|ref|; scores 1e-3 rel, masked +inf; evict exact or 1e-4 near-tie"}


def cpu_baseline(wl, mask, max_pairs, min_seconds=10.0, gpu_step0=None):
    """The fp64 oracle on the host cores, on a bounded sample of the same
    workload: up to `max_pairs` (sequence, KV head) pairs per step, one
    sequence per task on a thread pool, over consecutive steps until
    `min_seconds` of wall time, scaled by valid K/V bytes to whole steps.
    With gpu_step0 (the GPU's outputs of step 0 on the same sequences), the
    oracle's first step also gives a parity verdict (returned under
    "parity")."""
    from decode_attention_kv_05_amd import workloads as W
    from oracle import decode_step

    nb = cpu_baseline_sequences(wl, max_pairs)
    batch = list(range(nb))
    k, v, m = W.initial_cache(wl, batch)
    prev = W.first_prev_slot(wl, batch)
    cores = host_cores()
    steps, busy = 0, 0.0
    parity = None
    while busy < min_seconds and steps < wl.steps:
        q, nk, nv = W.step_inputs(wl, steps, batch)
        t0 = time.perf_counter()
        res = _per_sequence(lambda b: decode_step(q[b:b + 1], k[b:b + 1], v[b:b + 1], m[b:b + 1], nk[b:b + 1],
                                                  nv[b:b + 1], prev[b:b + 1], wl.scale), nb, cores)
        busy += time.perf_counter() - t0
        prev = np.concatenate([r[2] for r in res])
        if steps == 0 and gpu_step0 is not None:
            parity = parity_verdict(wl, m, gpu_step0, tuple(np.concatenate([r[i] for r in res]) for i in range(3)))
        steps += 1
    frac = valid_slots(m) / max(1, valid_slots(mask))
    s_per_step = busy / steps / frac
    model, blas = host_info()
    return {
        "value": round(kv_bytes(wl, mask) / s_per_step / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{nb * wl.Hkv} of {wl.B * wl.Hkv} (sequence, KV head) pairs over {steps} decode steps "
                  f"({busy:.1f} s wall), scaled by valid K/V bytes; numpy fp64, one sequence per task on "
                  f"{cores} threads, BLAS 1 thread each",
        "steps_per_s": round(1.0 / s_per_step, 6),
        "s_per_step": round(s_per_step, 3),
        "cpu_model": model,
        "blas": blas,
        **({"parity": parity} if parity is not None else {}),
    }


def cpu_baseline_topk(B, Hkv, S, k, min_seconds=3.0):
    """The oracle's k-slot selection on one host thread (its per-row Python
    work holds the interpreter lock, so a thread pool ran slower), whole
    launches over the same synthetic scores until `min_seconds`."""
    from decode_attention_kv_05_amd import workloads as W
    from oracle import evict_topk

    scores = W.synthetic_scores(B, Hkv, S, seed=11000, kind="ties")
    valid = np.ones((Hkv, S), dtype=bool)
    launches, busy = 0, 0.0
    while busy < min_seconds:
        t0 = time.perf_counter()
        for b in range(B):
            evict_topk(scores[b], valid, k)
        busy += time.perf_counter() - t0
        launches += 1
    s_per_launch = busy / launches
    model, blas = host_info()
    return {
        "value": round(topk_bytes(B, Hkv, S, k) / s_per_launch / 1e9, 6),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{launches} whole launches of {B * Hkv} rows ({busy:.1f} s); numpy sort, 1 thread",
        "s_per_launch": round(s_per_launch, 4),
        "cpu_model": model,
        "blas": blas,
    }


def cpu_baseline_fill(wl, max_pairs, fill_from, min_seconds=10.0):
    """The oracle's fill step on the host cores (one sequence per task), on
    the first sequences of the fill workload (same start state), consecutive
    steps until `min_seconds` of wall time, as valid K/V bytes per second."""
    from decode_attention_kv_05_amd import workloads as W
    from oracle import decode_step_fill

    nb = max(1, min(wl.B, -(-max_pairs // wl.Hkv)))
    batch = list(range(nb))
    k, v, _ = W.initial_cache(wl, batch)
    m = (np.arange(wl.S)[None, :] < fill_from).astype(np.uint8).repeat(nb, 0)
    W.poison_free(k, v, m)
    prev = np.full((nb, wl.Hkv), min(fill_from, wl.S - 1), dtype=np.int32)
    cores = host_cores()
    steps, busy, rows = 0, 0.0, 0
    while busy < min_seconds and steps < wl.steps:
        q, nk, nv = W.step_inputs(wl, steps, batch)
        t0 = time.perf_counter()
        res = _per_sequence(lambda b: decode_step_fill(q[b:b + 1], k[b:b + 1], v[b:b + 1], m[b:b + 1],
                                                       nk[b:b + 1], nv[b:b + 1], prev[b:b + 1], wl.scale),
                            nb, cores)
        busy += time.perf_counter() - t0
        prev = np.concatenate([r[2] for r in res])
        m = np.concatenate([r[3] for r in res])
        rows += int(np.count_nonzero(m))
        steps += 1
    kv_per_row = wl.Hkv * wl.d * 2 * 2
    rate = rows * kv_per_row / busy
    model, blas = host_info()
    return {
        "value": round(rate / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{nb * wl.Hkv} of {wl.B * wl.Hkv} (sequence, KV head) pairs over {steps} fill steps "
                  f"({busy:.1f} s wall), valid K/V bytes per second; numpy fp64, one sequence per task on "
                  f"{cores} threads, BLAS 1 thread each",
        "cpu_model": model,
        "blas": blas,
    }


def timed(step, K, Wm, stream, dev, reset=None, warmup_s=WARMUP_MIN_S):
    """Warm up with at least Wm steps and at least WARMUP_MIN_S seconds of
    them; then REPEATS times: K steps between one pair of events on the
    launch stream, synchronized on both sides.  Then K steps, untimed as a
    whole, with an event pair around each for the per-launch durations
    (events recorded between launches hold the next launch back by a few
    microseconds, so they stay out of the timed repeats).  Steps are numbered
    on from the warm-up; reset(t), if given, restores the start state before
    every repeat and before the per-launch pass (untimed).  Returns (ms per
    step of each repeat, per-launch ms, wall seconds of the timed repeats,
    warm-up steps run)."""
    import torch
    t = 0
    w0 = time.perf_counter()
    while t < Wm or time.perf_counter() - w0 < warmup_s:
        for _ in range(max(1, Wm)):
            step(t)
            t += 1
        torch.cuda.synchronize(dev)
    warm = t
    reps, wall = [], 0.0
    for _ in range(REPEATS):
        if reset is not None:
            reset(t)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(dev)
        wall0 = time.perf_counter()
        start.record(stream)
        for _ in range(K):
            step(t)
            t += 1
        end.record(stream)
        torch.cuda.synchronize(dev)
        wall += time.perf_counter() - wall0
        reps.append(start.elapsed_time(end) / K)
    if reset is not None:
        reset(t)
        torch.cuda.synchronize(dev)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    for i in range(K):
        starts[i].record(stream)
        step(t)
        t += 1
        ends[i].record(stream)
    torch.cuda.synchronize(dev)
    per_launch = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    return np.array(reps), per_launch, wall, warm


def hbm_probes(dev, k_cache=None, v_cache=None, reps=5):
    """The GPU's practical HBM read rates, measured in the same
    run by plain read kernels (libhbm_probe.so, not the library): the whole
    grid reading in address order, and the decode's own pattern without its
    arithmetic (K then V of each (sequence, KV head) pair, one workgroup per
    pair) over the run's caches; plus a torch device-to-device copy (read +
    write bytes).  Median of `reps` event-timed runs each, GB/s."""
    import ctypes

    import torch

    from decode_attention_kv_05_amd.build import PROBE_PATH
    lib = ctypes.CDLL(PROBE_PATH)
    lib.lf_probe_read_interleaved.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    lib.lf_probe_read_pairs.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p]
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    nbytes = 1 << 30
    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)

    def rate(fn, moved):
        fn()
        torch.cuda.synchronize(dev)
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize(dev)
            ts.append(a.elapsed_time(b) / 1e3)
        return round(moved / float(np.median(ts)) / 1e9, 1)

    def call(rc):
        if rc != 0:
            raise RuntimeError("probe launch failed")

    out = {"read_interleaved_GBps": rate(lambda: call(lib.lf_probe_read_interleaved(src.data_ptr(), nbytes,
                                                                                     sink.data_ptr(), stream)), nbytes),
           "copy_GBps": rate(lambda: dst.copy_(src), 2 * nbytes)}
    if k_cache is not None:
        B, Hkv, S, d = k_cache.shape
        pb = S * d * 2
        out["read_pairs_GBps"] = rate(lambda: call(lib.lf_probe_read_pairs(k_cache.data_ptr(), v_cache.data_ptr(),
                                                                           B * Hkv, pb, sink.data_ptr(), stream)),
                                      2 * B * Hkv * pb)
    out["how"] = ("read_interleaved: 1 GiB read by the whole grid in address order; read_pairs: the run's K then V "
                  "caches, one 8-wave workgroup per pair, the decode's loads without its arithmetic; copy: torch "
                  "copy_ of 1 GiB (read + write); median of 5")
    del src, dst
    return out


def roofline(alg_bytes_per_launch, step_ms, per_launch_ms, kernel, traffic):
    """HBM roofline of the dominant kernel.  achieved: algorithmic bytes per
    step over the median timed step (one decode launch per step);
    achieved_per_launch: the same bytes over the mean event-timed launch."""
    step_s = float(step_ms) / 1e3
    launch_s = float(per_launch_ms.mean()) / 1e3
    achieved = alg_bytes_per_launch / step_s / 1e9
    per_launch = alg_bytes_per_launch / launch_s / 1e9
    return {
        "bound": "hbm",
        "achieved": round(achieved, 2),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": traffic,
        "kernel": kernel,
        "step_us_median": round(step_s * 1e6, 2),
        "achieved_per_launch": round(per_launch, 2),
        "frac_per_launch": round(per_launch / HBM_PEAK_GBPS, 4),
        "launch_us_mean": round(launch_s * 1e6, 2),
        "launch_us_p50": round(float(np.median(per_launch_ms)) * 1e3, 2),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qwen3_8b")
    ap.add_argument("--nsplit", type=int, default=None, help="slot splits per pair (default: library plan)")
    ap.add_argument("--cpu-pairs", type=int, default=1024, help="oracle sample: pairs per step for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", choices=("decode", "fill", "topk", "cadence", "stack"), default="decode")
    ap.add_argument("--layers", type=int, default=36, help="layers in stack mode")
    ap.add_argument("--hidden", type=int, default=4096, help="model width in stack mode")
    ap.add_argument("--topk-k", type=int, default=128, help="slots chosen per pair in topk mode")
    ap.add_argument("--cadence", type=int, default=128, help="steps between top-k refreshes in cadence mode")
    ap.add_argument("--warmup-seconds", type=float, default=WARMUP_MIN_S,
                    help="the warm-up lasts at least this long (counter runs under a profiler pass 0)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes 5 times "
                         "(calibrates HBM byte counters) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the operator shards by sequence or KV head with no exchange, see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    if os.environ.get("WORLD_SIZE", "1") not in ("", "1"):
        print("bench.py runs as a single process on one GPU", file=sys.stderr)
        sys.exit(2)

    import torch

    from decode_attention_kv_05_amd.build import ensure_built
    ensure_built()
    from decode_attention_kv_05_amd import longflow as lf
    from decode_attention_kv_05_amd import workloads as W

    if not torch.cuda.is_available():
        raise RuntimeError("no HIP device visible")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        src = torch.full((args.copy_probe,), 7, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize(dev)
        print(json.dumps({"copy_probe_bytes": args.copy_probe, "launches": 5}), flush=True)
        return
    props = torch.cuda.get_device_properties(dev)
    wl = W.WORKLOADS[args.workload]
    K, Wm = args.steps, args.warmup
    log(f"device {props.name} ({props.multi_processor_count} CUs, {props.total_memory / 2**30:.0f} GiB); "
        f"workload {wl}; mode {args.mode}")
    if args.mode == "topk":
        return bench_topk(args, wl, lf, W, dev)
    if args.mode == "stack":
        return bench_stack(args, wl, lf, W, dev)

    t0 = time.time()
    k, v, mask = W.initial_cache(wl)
    fill_from = None
    if args.mode == "fill":
        # every timed pass starts from the same state, every sequence K slots short
        # of full, and fills up at its last step (the mask is restored between passes)
        fill_from = max(1, wl.S - K)
        mask = (np.arange(wl.S)[None, :] < fill_from).astype(np.uint8).repeat(wl.B, 0)
        W.poison_free(k, v, mask)
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    dk, dv = to_dev(k), to_dev(v)
    del k, v
    dm = torch.from_numpy(mask).to(dev)
    n_inputs = max(1, min(wl.steps, K + Wm))
    qs, nks, nvs = [], [], []
    for t in range(n_inputs):
        q, nk, nv = W.step_inputs(wl, t)
        qs.append(to_dev(q))
        nks.append(to_dev(nk))
        nvs.append(to_dev(nv))
    log(f"inputs generated and resident in HBM in {time.time() - t0:.1f} s ({n_inputs} distinct steps)")

    nsplit = args.nsplit or lf.plan_nsplit(wl.B, wl.Hq, wl.Hkv, wl.d, wl.S)
    ws = lf.new_workspace(wl.B, wl.Hq, wl.Hkv, wl.d, wl.S, nsplit, dev)
    out = torch.empty((wl.B, wl.Hq, wl.d), dtype=torch.bfloat16, device=dev)
    scores = torch.empty((wl.B, wl.Hkv, wl.S), dtype=torch.float32, device=dev)
    slots = [torch.full((wl.B, wl.Hkv), -1, dtype=torch.int32, device=dev),
             torch.empty((wl.B, wl.Hkv), dtype=torch.int32, device=dev)]
    stream = torch.cuda.current_stream(dev)
    N = args.cadence
    queue = torch.full((N, wl.B, wl.Hkv), -1, dtype=torch.int32, device=dev)

    if args.mode == "fill":
        slots[0].fill_(fill_from if fill_from < wl.S else -1)

    def step(t):
        i = t % n_inputs
        if args.mode == "decode":
            lf.longflow_decode(qs[i], dk, dv, dm, nks[i], nvs[i], slots[t % 2], scale=float(wl.scale),
                               out=out, scores=scores, evict_slot=slots[(t + 1) % 2], workspace=ws,
                               nsplit=nsplit, stream=stream)
        elif args.mode == "fill":
            lf.longflow_decode_fill(qs[i], dk, dv, dm, nks[i], nvs[i], slots[t % 2], scale=float(wl.scale),
                                    out=out, scores=scores, next_slot=slots[(t + 1) % 2], workspace=ws,
                                    nsplit=nsplit, stream=stream)
        else:  # cadence: the written slot comes from the queue of the last refresh
            lf.longflow_decode(qs[i], dk, dv, dm, nks[i], nvs[i], queue[t % N], scale=float(wl.scale),
                               out=out, scores=scores, evict_slot=slots[0], workspace=ws,
                               nsplit=nsplit, stream=stream)
            if (t + 1) % N == 0:
                lf.longflow_evict_topk(scores, dm, N, out=queue, stream=stream)

    reset = None
    if args.mode == "fill":
        dm0 = dm.clone()

        def reset(t):
            dm.copy_(dm0)
            slots[t % 2].fill_(fill_from if fill_from < wl.S else -1)

    # The first step once more before the timing, for the parity verdict of
    # the CPU baseline leg: it writes no cache row (prev_slot -1) and only
    # sets slots[1], so the timed run starts from the same state.
    gpu_step0 = None
    if args.mode == "decode" and not args.no_cpu_baseline:
        nb = cpu_baseline_sequences(wl, args.cpu_pairs)
        step(0)
        torch.cuda.synchronize(dev)
        gpu_step0 = {"out": out[:nb].float().cpu().numpy().astype(np.float64),
                     "scores": scores[:nb].cpu().numpy().astype(np.float64),
                     "evict": slots[1][:nb].cpu().numpy()}

    reps, per_launch, wall, warm = timed(step, K, Wm, stream, dev, reset, args.warmup_seconds)
    ms_per_step = float(np.median(reps))
    status = lf.lf_read_device_status(ws)
    if status:
        raise RuntimeError(f"device status flags set during the run: {status:#x}")

    if args.mode == "fill":
        # valid rows of the t-th step of a pass: the prefix plus the t + 1 written slots
        rows = sum(min(wl.S, fill_from + t + 1) for t in range(K)) / K
        kvb = int(rows * wl.B * wl.Hkv * wl.d * 2 * 2)
        algb = algb_launch = kvb + algorithmic_bytes(wl, np.zeros_like(mask)) + wl.B
        if not dm.cpu().numpy().all():
            raise RuntimeError("fill pass ended with free slots left")
    else:
        kvb = kv_bytes(wl, mask)
        algb = algb_launch = algorithmic_bytes(wl, mask)
    # step index of the per-launch durations: warm + REPEATS * K + t
    first_launch = warm + REPEATS * K
    if args.mode == "cadence":
        # decode launches only: top-k launches are timed inside the steps that run them
        dec = np.array([x for t, x in enumerate(per_launch) if (first_launch + t + 1) % N != 0])
        rl = roofline(algb, ms_per_step, dec if dec.size else per_launch, "longflow_decode_kernel", None)
    else:
        rl = roofline(algb_launch, ms_per_step, per_launch, "longflow_decode_kernel",
                      measured_traffic(f"{wl.name}/nsplit{nsplit}" + ("/fill" if args.mode == "fill" else "")))
    metric = {
        "decode": METRIC,
        "fill": "fill-phase decode-attn+next slot: KV GB/s, steps/s at B=128, 3200 slots",
        "cadence": f"decode-attn with top-k eviction every {N} steps: KV GB/s, steps/s at B=128, 3200 slots",
    }[args.mode]
    result = {
        "metric": metric,
        "value": round(kvb / (ms_per_step / 1e3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "batch": wl.B, "q_heads": wl.Hq, "kv_heads": wl.Hkv,
            "head_dim": wl.d, "slots": wl.S, "valid_slots": valid_slots(mask), "nsplit": nsplit,
            "kv_dtype": "bf16", "accumulate": "f32",
        },
        "steps_per_s": round(1e3 / ms_per_step, 2),
        "kv_GBps": round(kvb / (ms_per_step / 1e3) / 1e9, 2),
        "alg_GBps": round(algb / (ms_per_step / 1e3) / 1e9, 2),
        "pct_hbm_peak": round(100 * algb / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBPS, 2),
        "alg_bytes_per_step": algb,
        "roofline": rl,
        "timing": {"repeats": REPEATS, "steps_per_repeat": K, "statistic": "median",
                   "ms_per_step_repeats": [round(float(x), 5) for x in reps],
                   "warmup_steps_run": warm, "warmup_min_s": args.warmup_seconds},
        "wall_s_timed": round(wall, 3),
    }
    result["hbm_probe"] = hbm_probes(dev, dk, dv)
    if args.mode != "cadence":
        result["lds"] = measured_lds(wl.name if args.mode == "decode" else f"fill_{wl.name}")
    if args.mode == "fill":
        result["config"].update({"mode": "fill", "start_valid_slots": fill_from})
    if args.mode == "cadence":
        result["config"].update({"mode": "cadence", "cadence": N})
        refresh = [x for t, x in enumerate(per_launch) if (first_launch + t + 1) % N == 0]
        if refresh:
            result["refresh_step_us_mean"] = round(float(np.mean(refresh)) * 1e3, 2)
    if not args.no_cpu_baseline and args.mode != "cadence":
        t0 = time.time()
        if args.mode == "fill":
            result["cpu_baseline"] = cpu_baseline_fill(wl, args.cpu_pairs, fill_from)
        else:
            result["cpu_baseline"] = cpu_baseline(wl, mask, args.cpu_pairs, gpu_step0=gpu_step0)
            parity = result["cpu_baseline"].pop("parity", None)
            if parity is not None:
                result["parity"] = parity
        log(f"cpu baseline took {time.time() - t0:.1f} s")
    print(json.dumps(result), flush=True)


def bench_topk(args, wl, lf, W, dev):
    """k-slot selection over synthetic scores of the workload's shape."""
    import torch
    B, Hkv, S, k = wl.B, wl.Hkv, wl.S, args.topk_k
    K, Wm = args.steps, args.warmup
    scores = torch.from_numpy(W.synthetic_scores(B, Hkv, S, seed=11000, kind="ties")).to(dev)
    mask = torch.ones((B, S), dtype=torch.uint8, device=dev)
    out = torch.empty((k, B, Hkv), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(t):
        lf.longflow_evict_topk(scores, mask, k, out=out, stream=stream)

    reps, per_launch, wall, warm = timed(step, K, Wm, stream, dev, warmup_s=args.warmup_seconds)
    ms = float(np.median(reps))
    algb = topk_bytes(B, Hkv, S, k)
    result = {
        "metric": f"k-slot eviction (k={k}): scores GB/s, launches/s at B={B}, {S} slots",
        "value": round(algb / (ms / 1e3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "mode": "topk", "batch": B, "kv_heads": Hkv, "slots": S, "k": k,
                   "scores": "ties"},
        "steps_per_s": round(1e3 / ms, 2),
        "alg_bytes_per_step": algb,
        "roofline": roofline(algb, ms, per_launch, "evict_topk_kernel", measured_traffic(f"topk/{wl.name}/k{k}")),
        "timing": {"repeats": REPEATS, "steps_per_repeat": K, "statistic": "median",
                   "ms_per_step_repeats": [round(float(x), 5) for x in reps], "warmup_steps_run": warm},
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_topk(B, Hkv, S, k)
    print(json.dumps(result), flush=True)



def stack_weight_bytes(L, H, Hq, Hkv, d):
    return L * ((Hq + 2 * Hkv) * d * H + H * Hq * d) * 2


def cpu_baseline_stack(wl, L, H, min_seconds=10.0):
    """The oracle's multi-layer step on the host cores, one sequence per task
    (sequences are independent), a round of as many sequences as threads at
    a time until `min_seconds` of wall time, scaled to the batch."""
    from decode_attention_kv_05_amd import workloads as W
    from oracle.stack_oracle import stack_step

    weights = [W.layer_weights(wl.seed, l, H, wl.Hq, wl.Hkv, wl.d) for l in range(L)]
    xs = W.token_activations(wl.seed, 0, wl.B, H)
    cores = host_cores()
    done, busy = 0, 0.0
    while busy < min_seconds and done < wl.B:
        jobs = []
        for b in range(done, min(wl.B, done + cores)):
            k, v, m = W.initial_cache(wl, [b])
            layers = [{"w_qkv": wq, "w_o": wo, "k": k.copy(), "v": v.copy(), "mask": m,
                       "slot": np.full((1, wl.Hkv), -1, np.int32)} for wq, wo in weights]
            jobs.append((xs[b:b + 1], layers))
        t0 = time.perf_counter()
        _per_sequence(lambda i: stack_step(jobs[i][0], np.array([wl.S]), jobs[i][1], wl.Hq, wl.Hkv, wl.d,
                                           wl.scale, 1e6), len(jobs), cores)
        busy += time.perf_counter() - t0
        done += len(jobs)
        del jobs
    s_per_step = busy / done * wl.B
    kvb = kv_bytes(wl, np.ones((wl.B, wl.S), np.uint8)) * L
    model, blas = host_info()
    return {
        "value": round(kvb / s_per_step / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{done} of {wl.B} sequences through all {L} layers ({busy:.1f} s wall), scaled to the batch; "
                  f"numpy fp64, one sequence per task on {cores} threads, BLAS 1 thread each",
        "s_per_step": round(s_per_step, 2),
        "cpu_model": model,
        "blas": blas,
    }


def bench_stack(args, wl, lf, W, dev):
    """--layers layers of the attention module around the operator, replayed
    as one HIP graph per token."""
    import torch
    L, H = args.layers, args.hidden
    K, Wm = args.steps, args.warmup
    t0 = time.time()
    k, v, mask = W.initial_cache(wl)
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    dk0, dv0 = to_dev(k), to_dev(v)
    del k, v
    dm = torch.from_numpy(mask).to(dev)
    kc = [dk0] + [dk0.clone() for _ in range(L - 1)]
    vc = [dv0] + [dv0.clone() for _ in range(L - 1)]
    wq, wo = [], []
    for l in range(L):
        a, b = W.layer_weights(wl.seed, l, H, wl.Hq, wl.Hkv, wl.d)
        wq.append(to_dev(a))
        wo.append(to_dev(b))
    n_inputs = max(1, min(16, K + Wm))
    xs = [to_dev(W.token_activations(wl.seed, t, wl.B, H)) for t in range(n_inputs)]
    x_in = torch.empty((wl.B, H), dtype=torch.bfloat16, device=dev)
    x_out = torch.empty_like(x_in)
    pos = torch.full((wl.B,), wl.S, dtype=torch.int32, device=dev)
    slots = [torch.full((wl.B, wl.Hkv), -1, dtype=torch.int32, device=dev) for _ in range(L)]
    nsplit = args.nsplit or lf.plan_nsplit(wl.B, wl.Hq, wl.Hkv, wl.d, wl.S)
    stack = lf.Stack(x_in, x_out, pos, wq, wo, kc, vc, [dm] * L, slots, None, Hq=wl.Hq,
                     scale=float(wl.scale), rope_base=1e6, nsplit=nsplit)
    graph = stack.graph()
    log(f"{L} layers set up in {time.time() - t0:.1f} s")
    stream = torch.cuda.current_stream(dev)

    def step(t):
        x_in.copy_(xs[t % n_inputs], non_blocking=True)
        graph.launch(stream)

    reps, per_launch, wall, warm = timed(step, K, Wm, stream, dev, warmup_s=args.warmup_seconds)
    ms = float(np.median(reps))
    status = lf.lf_read_device_status(stack.tensors["workspace"])
    graph.close()
    if status:
        raise RuntimeError(f"device status flags set during the run: {status:#x}")
    kvb = kv_bytes(wl, mask) * L
    wb = stack_weight_bytes(L, H, wl.Hq, wl.Hkv, wl.d)
    algb = algorithmic_bytes(wl, mask) * L + wb + 2 * wl.B * H * 2
    result = {
        "metric": f"{L}-layer attention module (QKV proj + RoPE + LongFlow step + O proj): KV GB/s, "
                  f"tokens/s at B={wl.B}, {wl.S} slots",
        "value": round(kvb / (ms / 1e3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "mode": "stack", "layers": L, "hidden": H, "batch": wl.B,
                   "q_heads": wl.Hq, "kv_heads": wl.Hkv, "head_dim": wl.d, "slots": wl.S, "nsplit": nsplit,
                   "weights": "synthetic N(0, 1/fan_in)", "launch": "one HIP graph per token"},
        "tokens_per_s": round(wl.B * 1e3 / ms, 1),
        "steps_per_s": round(1e3 / ms, 2),
        "alg_bytes_per_step": algb,
        "weight_bytes_per_step": wb,
        "roofline": roofline(algb, ms, per_launch, f"{L}-layer step (graph)", None),
        "timing": {"repeats": REPEATS, "steps_per_repeat": K, "statistic": "median",
                   "ms_per_step_repeats": [round(float(x), 5) for x in reps], "warmup_steps_run": warm},
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_stack(wl, L, H)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
