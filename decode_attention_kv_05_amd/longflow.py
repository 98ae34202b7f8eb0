"""ctypes binding of liblongflow.so (see include/longflow.h).

Argument marshalling only: torch tensors are checked for device, dtype,
shape and contiguity and handed over as raw pointers together with torch's
current HIP stream.  Every step of the decode runs in the library's HIP
kernels.  Importing this module fails if the library has not been built.
"""

import ctypes
import os

import torch

from .build import LIB_PATH, source_hash

LF_OK = 0
LF_E_NULL = -1
LF_E_SHAPE = -2
LF_E_ALIGN = -3
LF_E_ALIAS = -4
LF_E_WORKSPACE = -5
LF_E_HIP = -6
LF_E_NSPLIT = -7
LF_E_VALUE = -8
LF_E_SCRATCH = -9

LF_DEV_BAD_PREV = 0x1
LF_DEV_WRITE_MASKED = 0x2
LF_DEV_FILL_DIVERGED = 0x4
LF_DEV_TEAM_TIMEOUT = 0x8

LF_SPLIT_AUTO, LF_SPLIT_COMBINE, LF_SPLIT_TEAM = 0, 1, 2
SPLIT_PATHS = {"auto": LF_SPLIT_AUTO, "combine": LF_SPLIT_COMBINE, "team": LF_SPLIT_TEAM}

EXPORTED = (
    "lf_version", "lf_source_hash", "lf_strerror", "lf_check_shape", "lf_plan_nsplit", "lf_workspace_size",
    "lf_device_num_cus", "lf_workspace_init", "lf_validate", "longflow_decode",
    "longflow_decode_nsplit", "longflow_decode_fill", "longflow_decode_ex", "longflow_evict_topk",
    "lf_read_device_status", "longflow_decode_noalloc",
    "lf_stack_workspace_size", "lf_stack_workspace_offsets", "longflow_stack_step", "lf_stack_graph_create", "lf_graph_launch",
    "lf_graph_destroy",
)

_i, _f, _p, _sz = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m decode_attention_kv_05_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "lf_version": ([], _i),
        "lf_source_hash": ([], ctypes.c_char_p),
        "lf_strerror": ([_i], ctypes.c_char_p),
        "lf_check_shape": ([_i] * 5, _i),
        "lf_plan_nsplit": ([_i] * 6 + [ctypes.POINTER(_i)], _i),
        "lf_workspace_size": ([_i] * 6 + [ctypes.POINTER(_sz)], _i),
        "lf_device_num_cus": ([ctypes.POINTER(_i)], _i),
        "lf_workspace_init": ([_p, _sz, _p], _i),
        "lf_validate": ([_i] * 5 + [_f] + [_p] * 11 + [_sz, _i], _i),
        "longflow_decode": ([_i] * 5 + [_f] + [_p] * 11 + [_sz, _p], _i),
        "longflow_decode_nsplit": ([_i] * 5 + [_f] + [_p] * 11 + [_sz, _i, _p], _i),
        "longflow_decode_fill": ([_i] * 5 + [_f] + [_p] * 11 + [_sz, _i, _p], _i),
        "longflow_decode_ex": ([_i] * 5 + [_f] + [_p] * 4 + [_i] + [_p] * 7 + [_sz, _i, _i, _p], _i),
        "longflow_evict_topk": ([_i] * 4 + [_p] * 3 + [_p], _i),
        "lf_read_device_status": ([_p, _p, ctypes.POINTER(ctypes.c_uint32)], _i),
        "longflow_decode_noalloc": ([_i] * 5 + [_f] + [_p] * 10 + [_p], _i),
        "lf_stack_workspace_size": ([_i] * 8 + [ctypes.POINTER(_sz)], _i),
        "lf_stack_workspace_offsets": ([_i] * 7 + [ctypes.POINTER(_sz)], _i),
        "longflow_stack_step": ([_i] * 7 + [_f, _f] + [_p] * 3 + [_i] + [_p] * 8 + [_sz, _i, _p], _i),
        "lf_stack_graph_create": ([_i] * 7 + [_f, _f] + [_p] * 3 + [_i] + [_p] * 8 + [_sz, _i,
                                                                             ctypes.POINTER(_p)], _i),
        "lf_graph_launch": ([_p, _p], _i),
        "lf_graph_destroy": ([_p], _i),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    built, want = lib.lf_source_hash().decode(), source_hash()
    if built != want:
        raise ImportError(f"{LIB_PATH} was built from other sources ({built}) than the current ones ({want}): "
                          "run `python -m decode_attention_kv_05_amd.build`")
    return lib


_lib = _load()


class LongflowError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__(f"{where}: {lf_strerror(code)} (code {code})")


def _check(rc, where):
    if rc != LF_OK:
        if rc in (LF_E_SHAPE, LF_E_ALIGN, LF_E_ALIAS, LF_E_NULL, LF_E_NSPLIT, LF_E_VALUE, LF_E_WORKSPACE,
                  LF_E_SCRATCH):
            raise ValueError(f"{where}: {lf_strerror(rc)} (code {rc})")
        raise LongflowError(rc, where)


def lf_version():
    return _lib.lf_version()


def lf_source_hash():
    return _lib.lf_source_hash().decode()


def lf_strerror(code):
    return _lib.lf_strerror(code).decode()


def lf_check_shape(B, Hq, Hkv, d, S):
    return _lib.lf_check_shape(B, Hq, Hkv, d, S)


def lf_plan_nsplit(B, Hq, Hkv, d, S, num_cus):
    out = _i(0)
    _check(_lib.lf_plan_nsplit(B, Hq, Hkv, d, S, num_cus, ctypes.byref(out)), "lf_plan_nsplit")
    return out.value


def lf_workspace_size(B, Hq, Hkv, d, S, nsplit):
    out = _sz(0)
    _check(_lib.lf_workspace_size(B, Hq, Hkv, d, S, nsplit, ctypes.byref(out)), "lf_workspace_size")
    return out.value


def lf_device_num_cus():
    out = _i(0)
    _check(_lib.lf_device_num_cus(ctypes.byref(out)), "lf_device_num_cus")
    return out.value


def _stream_ptr(stream, device):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def lf_workspace_init(workspace, stream=None):
    _check(_lib.lf_workspace_init(ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
                                  _stream_ptr(stream, workspace.device)), "lf_workspace_init")


def lf_validate(B, Hq, Hkv, d, S, scale, q, k_cache, v_cache, mask, new_k, new_v, prev_slot,
                out, scores, evict_slot, workspace, workspace_bytes, nsplit):
    """Host-only check on raw addresses (ints); returns the lf_status code."""
    ptrs = [ctypes.c_void_p(x) for x in (q, k_cache, v_cache, mask, new_k, new_v, prev_slot,
                                          out, scores, evict_slot, workspace)]
    return _lib.lf_validate(B, Hq, Hkv, d, S, float(scale), *ptrs, workspace_bytes, nsplit)


def plan_nsplit(B, Hq, Hkv, d, S):
    """Split count the library picks on the current device."""
    return lf_plan_nsplit(B, Hq, Hkv, d, S, lf_device_num_cus())


def new_workspace(B, Hq, Hkv, d, S, nsplit=None, device=None):
    """Zeroed device workspace sized for (shape, nsplit); nsplit None = the device plan."""
    if nsplit is None:
        nsplit = plan_nsplit(B, Hq, Hkv, d, S)
    n = lf_workspace_size(B, Hq, Hkv, d, S, nsplit)
    return torch.zeros(n, dtype=torch.uint8, device=device or "cuda")


def _need(t, name, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class DeviceStatusError(RuntimeError):
    """LF_DEV_* bits found in a workspace after a step (see check=True)."""

    def __init__(self, flags):
        self.flags = flags
        names = [n for n, bit in (("LF_DEV_BAD_PREV", LF_DEV_BAD_PREV), ("LF_DEV_WRITE_MASKED", LF_DEV_WRITE_MASKED),
                                  ("LF_DEV_FILL_DIVERGED", LF_DEV_FILL_DIVERGED),
                                  ("LF_DEV_TEAM_TIMEOUT", LF_DEV_TEAM_TIMEOUT)) if flags & bit]
        super().__init__(f"device status {flags:#x}: {', '.join(names) or 'unknown bits'}")


def _step(entry, q, k_cache, v_cache, mask, new_k, new_v, prev_slot, scale, out, scores, evict_slot,
          workspace, nsplit, stream, split_path=None, check=False):
    B, Hq, d = q.shape
    Hkv, S = k_cache.shape[1], k_cache.shape[2]
    dev = q.device
    _need(q, "q", torch.bfloat16, (B, Hq, d), dev)
    _need(k_cache, "k_cache", torch.bfloat16, (B, Hkv, S, d), dev)
    _need(v_cache, "v_cache", torch.bfloat16, (B, Hkv, S, d), dev)
    _need(mask, "mask", (torch.uint8, torch.bool), (B, S), dev)
    _need(new_k, "new_k", torch.bfloat16, (B, Hkv, d), dev)
    _need(new_v, "new_v", torch.bfloat16, (B, Hkv, d), dev)
    _need(prev_slot, "prev_slot", torch.int32, (B, Hkv), dev)
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    if nsplit is None:
        nsplit = plan_nsplit(B, Hq, Hkv, d, S) if B > 0 else 1
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=dev)
    if scores is None:
        scores = torch.empty((B, Hkv, S), dtype=torch.float32, device=dev)
    if evict_slot is None:
        evict_slot = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    _need(out, "out", torch.bfloat16, (B, Hq, d), dev)
    _need(scores, "scores", torch.float32, (B, Hkv, S), dev)
    _need(evict_slot, "evict_slot", torch.int32, (B, Hkv), dev)
    if workspace is None:
        workspace = new_workspace(B, Hq, Hkv, d, S, nsplit, dev) if B > 0 else torch.zeros(256, dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the device of q")
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    if split_path is None:
        rc = getattr(_lib, entry)(
            B, Hq, Hkv, d, S, float(scale), ptr(q), ptr(k_cache), ptr(v_cache), ptr(mask),
            ptr(new_k), ptr(new_v), ptr(prev_slot), ptr(out), ptr(scores), ptr(evict_slot),
            ptr(workspace), workspace.numel() * workspace.element_size(), int(nsplit),
            _stream_ptr(stream, dev))
    else:
        if split_path not in SPLIT_PATHS:
            raise ValueError(f"split_path must be one of {sorted(SPLIT_PATHS)}, got {split_path!r}")
        fill = 1 if entry == "longflow_decode_fill" else 0
        entry = "longflow_decode_ex"
        rc = _lib.longflow_decode_ex(
            B, Hq, Hkv, d, S, float(scale), ptr(q), ptr(k_cache), ptr(v_cache), ptr(mask), fill, ptr(new_k), ptr(new_v), ptr(prev_slot), ptr(out), ptr(scores),
            ptr(evict_slot), ptr(workspace), workspace.numel() * workspace.element_size(), int(nsplit),
            SPLIT_PATHS[split_path], _stream_ptr(stream, dev))
    _check(rc, entry)
    if check:
        flags = lf_read_device_status(workspace, stream)
        if flags:
            raise DeviceStatusError(flags)
    return out, scores, evict_slot


def longflow_decode(q, k_cache, v_cache, mask, new_k, new_v, prev_slot, *, scale=None,
                    out=None, scores=None, evict_slot=None, workspace=None, nsplit=None,
                    stream=None, split_path=None, check=False):
    """One fused decode step; returns (out, scores, evict_slot).

    q [B, Hq, d] bf16; k_cache, v_cache [B, Hkv, S, d] bf16 (updated in place);
    mask [B, S] uint8 or bool; new_k, new_v [B, Hkv, d] bf16; prev_slot
    [B, Hkv] int32.  Outputs are allocated when not given: out [B, Hq, d]
    bf16, scores [B, Hkv, S] float32, evict_slot [B, Hkv] int32.  scale
    defaults to 1/sqrt(d).  nsplit None uses the library's plan for the
    device.  The work is enqueued on `stream` (default: torch's current
    stream) and not waited for.  split_path ("auto", "combine", "team"; None
    = "auto") chooses how a step with several splits is finished
    (longflow_decode_ex).  check=True waits for the step and raises
    DeviceStatusError if the workspace holds any LF_DEV_* bit, among them
    LF_DEV_TEAM_TIMEOUT (a team-path step whose results are unspecified
    because another process kept some of its workgroups from running).
    """
    return _step("longflow_decode_nsplit", q, k_cache, v_cache, mask, new_k, new_v, prev_slot, scale, out,
                 scores, evict_slot, workspace, nsplit, stream, split_path, check)


def longflow_decode_fill(q, k_cache, v_cache, mask, new_k, new_v, prev_slot, *, scale=None,
                         out=None, scores=None, next_slot=None, workspace=None, nsplit=None,
                         stream=None, split_path=None, check=False):
    """One decode step of the fill phase; returns (out, scores, next_slot).

    As longflow_decode, except that `mask` is updated in place (the written
    slot becomes valid) and next_slot is the lowest free slot of the updated
    mask while the sequence has one, else the evicted slot.
    """
    return _step("longflow_decode_fill", q, k_cache, v_cache, mask, new_k, new_v, prev_slot, scale, out,
                 scores, next_slot, workspace, nsplit, stream, split_path, check)


def longflow_decode_noalloc(q, k_cache, v_cache, mask, new_k, new_v, prev_slot, out, scores, evict_slot, *,
                            scale=None, stream=None):
    """longflow_decode with the library's static scratch array as its
    workspace (include/longflow.h): the caller passes every output, nothing
    is allocated.  Calls on one GPU must not overlap in time."""
    B, Hq, d = q.shape
    Hkv, S = k_cache.shape[1], k_cache.shape[2]
    dev = q.device
    for t, name, dt, shape in ((q, "q", torch.bfloat16, (B, Hq, d)), (k_cache, "k_cache", torch.bfloat16, (B, Hkv, S, d)),
                               (v_cache, "v_cache", torch.bfloat16, (B, Hkv, S, d)),
                               (mask, "mask", (torch.uint8, torch.bool), (B, S)),
                               (new_k, "new_k", torch.bfloat16, (B, Hkv, d)), (new_v, "new_v", torch.bfloat16, (B, Hkv, d)),
                               (prev_slot, "prev_slot", torch.int32, (B, Hkv)), (out, "out", torch.bfloat16, (B, Hq, d)),
                               (scores, "scores", torch.float32, (B, Hkv, S)),
                               (evict_slot, "evict_slot", torch.int32, (B, Hkv))):
        _need(t, name, dt, shape, dev)
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = _lib.longflow_decode_noalloc(B, Hq, Hkv, d, S, float(scale), ptr(q), ptr(k_cache), ptr(v_cache), ptr(mask),
                                      ptr(new_k), ptr(new_v), ptr(prev_slot), ptr(out), ptr(scores), ptr(evict_slot),
                                      _stream_ptr(stream, dev))
    _check(rc, "longflow_decode_noalloc")
    return out, scores, evict_slot


def longflow_evict_topk(scores, mask, k, *, out=None, stream=None):
    """The k valid slots first in (score, slot) order for every (b, j), in
    ascending slot order, -1 padded: int32 [k, B, Hkv] (entry t is a
    prev_slot array for the t-th following step)."""
    B, Hkv, S = scores.shape
    dev = scores.device
    _need(scores, "scores", torch.float32, (B, Hkv, S), dev)
    _need(mask, "mask", (torch.uint8, torch.bool), (B, S), dev)
    if out is None:
        out = torch.empty((k, B, Hkv), dtype=torch.int32, device=dev)
    _need(out, "out", torch.int32, (k, B, Hkv), dev)
    rc = _lib.longflow_evict_topk(B, Hkv, S, int(k), ctypes.c_void_p(scores.data_ptr()),
                                  ctypes.c_void_p(mask.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                  _stream_ptr(stream, dev))
    _check(rc, "longflow_evict_topk")
    return out


def lf_read_device_status(workspace, stream=None):
    """LF_DEV_* bits recorded in the workspace (synchronises the stream)."""
    flags = ctypes.c_uint32(0)
    _check(_lib.lf_read_device_status(ctypes.c_void_p(workspace.data_ptr()), _stream_ptr(stream, workspace.device),
                                      ctypes.byref(flags)), "lf_read_device_status")
    return flags.value


def lf_stack_workspace_size(L, B, H, Hq, Hkv, d, S, nsplit):
    out = _sz(0)
    _check(_lib.lf_stack_workspace_size(L, B, H, Hq, Hkv, d, S, nsplit, ctypes.byref(out)),
           "lf_stack_workspace_size")
    return out.value


def lf_stack_workspace_offsets(B, H, Hq, Hkv, d, S, nsplit):
    """Byte offsets of the last layer's q, k_new, v_new and O in a stack workspace."""
    out = (_sz * 4)()
    _check(_lib.lf_stack_workspace_offsets(B, H, Hq, Hkv, d, S, nsplit, out), "lf_stack_workspace_offsets")
    return tuple(out)


class Stack:
    """Argument marshalling for the multi-layer step (include/longflow_stack.h).

    Holds the per-layer device tensors and the host pointer arrays built from
    them; `step()` enqueues one eager step, `graph()` records one into a HIP
    graph (a StackGraph).  Tensors: x_in, x_out [B, H] bf16; pos [B] int32;
    per layer w_qkv [(Hq + 2 Hkv) d, H], w_o [H, Hq d] bf16, k_cache,
    v_cache [B, Hkv, S, d] bf16, mask [B, S] uint8, slot [B, Hkv] int32,
    scores [B, Hkv, S] float32 or None.
    """

    def __init__(self, x_in, x_out, pos, w_qkv, w_o, k_cache, v_cache, mask, slot, scores=None, *,
                 Hq, scale=None, rope_base=1e6, advance_pos=True, nsplit=None, workspace=None):
        L = len(w_qkv)
        B, H = x_in.shape
        Hkv, S, d = k_cache[0].shape[1], k_cache[0].shape[2], k_cache[0].shape[3]
        dev = x_in.device
        _need(x_in, "x_in", torch.bfloat16, (B, H), dev)
        _need(x_out, "x_out", torch.bfloat16, (B, H), dev)
        _need(pos, "pos", torch.int32, (B,), dev)
        for name, lst in (("w_qkv", w_qkv), ("w_o", w_o), ("k_cache", k_cache), ("v_cache", v_cache),
                          ("mask", mask), ("slot", slot)):
            if len(lst) != L:
                raise ValueError(f"{name} has {len(lst)} entries, expected {L}")
        for l in range(L):
            _need(w_qkv[l], "w_qkv", torch.bfloat16, ((Hq + 2 * Hkv) * d, H), dev)
            _need(w_o[l], "w_o", torch.bfloat16, (H, Hq * d), dev)
            _need(k_cache[l], "k_cache", torch.bfloat16, (B, Hkv, S, d), dev)
            _need(v_cache[l], "v_cache", torch.bfloat16, (B, Hkv, S, d), dev)
            _need(mask[l], "mask", (torch.uint8, torch.bool), (B, S), dev)
            _need(slot[l], "slot", torch.int32, (B, Hkv), dev)
            if scores is not None and scores[l] is not None:
                _need(scores[l], "scores", torch.float32, (B, Hkv, S), dev)
        if nsplit is None:
            nsplit = plan_nsplit(B, Hq, Hkv, d, S)
        if workspace is None:
            workspace = torch.zeros(lf_stack_workspace_size(L, B, H, Hq, Hkv, d, S, nsplit), dtype=torch.uint8,
                                    device=dev)
        self.dims = (L, B, H, Hq, Hkv, d, S)
        self.scale = float(scale if scale is not None else 1.0 / float(d) ** 0.5)
        self.rope_base = float(rope_base)
        self.advance_pos = 1 if advance_pos else 0
        self.nsplit = int(nsplit)
        self.tensors = dict(x_in=x_in, x_out=x_out, pos=pos, w_qkv=list(w_qkv), w_o=list(w_o),
                            k_cache=list(k_cache), v_cache=list(v_cache), mask=list(mask), slot=list(slot),
                            scores=list(scores) if scores is not None else None, workspace=workspace)
        arr = lambda ts: (_p * L)(*[t.data_ptr() if t is not None else None for t in ts])
        self._arrays = [arr(w_qkv), arr(w_o), arr(k_cache), arr(v_cache), arr(mask), arr(slot),
                        arr(scores) if scores is not None else None]

    def _args(self):
        t = self.tensors
        P = lambda x: ctypes.c_void_p(x.data_ptr())
        a = self._arrays
        return (*self.dims, self.scale, self.rope_base, P(t["x_in"]), P(t["x_out"]), P(t["pos"]),
                self.advance_pos, a[0], a[1], a[2], a[3], a[4], a[5], a[6], P(t["workspace"]),
                t["workspace"].numel(), self.nsplit)

    def step(self, stream=None):
        _check(_lib.longflow_stack_step(*self._args(), _stream_ptr(stream, self.tensors["x_in"].device)),
               "longflow_stack_step")

    def intermediates(self):
        """Views into the workspace of the last layer's q [B, Hq, d], k_new and
        v_new [B, Hkv, d] and O [B, Hq d] (bf16), valid after a step until the
        next one."""
        L, B, H, Hq, Hkv, d, S = self.dims
        offs = lf_stack_workspace_offsets(B, H, Hq, Hkv, d, S, self.nsplit)
        ws = self.tensors["workspace"]
        view = lambda off, shape: ws[off:off + 2 * int(torch.tensor(shape).prod())].view(torch.bfloat16).view(shape)
        return {"q": view(offs[0], (B, Hq, d)), "k_new": view(offs[1], (B, Hkv, d)),
                "v_new": view(offs[2], (B, Hkv, d)), "o": view(offs[3], (B, Hq * d))}

    def graph(self):
        return StackGraph(self)


class StackGraph:
    """A recorded step (lf_stack_graph_create); launch() replays it."""

    def __init__(self, stack):
        self.stack = stack  # keeps every tensor the graph points at alive
        h = _p(0)
        _check(_lib.lf_stack_graph_create(*stack._args(), ctypes.byref(h)), "lf_stack_graph_create")
        self.handle = h

    def launch(self, stream=None):
        _check(_lib.lf_graph_launch(self.handle, _stream_ptr(stream, self.stack.tensors["x_in"].device)),
               "lf_graph_launch")

    def close(self):
        if self.handle:
            torch.cuda.synchronize()
            _check(_lib.lf_graph_destroy(self.handle), "lf_graph_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
