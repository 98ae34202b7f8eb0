"""The C ABI on the CPU: the library loads, exports every function the header
declares, and its host-only entry points (shape check, planner, workspace
size, argument validation) behave as documented.  No kernel is launched."""

import ctypes
import glob
import os
import re

import pytest

from decode_attention_kv_05_amd.build import INCLUDE, ensure_built

ensure_built()
from decode_attention_kv_05_amd import longflow as lf  # noqa: E402

HEADER = os.path.join(INCLUDE, "longflow.h")


def declared_functions():
    """Every function declared by any header under include/."""
    names = set()
    for path in sorted(glob.glob(os.path.join(INCLUDE, "*.h"))):
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert "longflow_decode" in names and "lf_validate" in names
    lib = ctypes.CDLL(lf.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(lf.EXPORTED)


def test_version_and_errors():
    m = re.search(r"#define LF_ABI_VERSION (\d+)", open(HEADER).read())
    assert lf.lf_version() == int(m.group(1))
    for code in range(0, -9, -1):
        assert lf.lf_strerror(code) and "unknown" not in lf.lf_strerror(code)
    assert "unknown" in lf.lf_strerror(-99)


@pytest.mark.parametrize("shape,ok", [
    ((1, 4, 1, 64, 256), True), ((128, 32, 8, 128, 3200), True), ((0, 32, 8, 128, 10), True),
    ((1, 64, 8, 128, 16384), True), ((1, 3, 1, 128, 5), True),
    ((1, 4, 3, 128, 10), False), ((1, 32, 2, 128, 10), False), ((1, 4, 1, 96, 10), False),
    ((1, 4, 1, 256, 10), False), ((1, 4, 1, 128, 0), False), ((-1, 4, 1, 128, 5), False),
    ((1, 0, 1, 128, 5), False),
])
def test_check_shape(shape, ok):
    assert (lf.lf_check_shape(*shape) == lf.LF_OK) == ok


def _gp(g):
    p = 1
    while p < g:
        p *= 2
    return p


@pytest.mark.parametrize("shape", [
    (1, 4, 1, 64, 256), (128, 32, 8, 128, 3200), (64, 32, 8, 128, 2400),
    (16, 64, 8, 128, 16384), (256, 32, 8, 128, 8192), (1, 8, 1, 128, 200000), (3, 6, 2, 64, 333),
])
def test_plan_fits_lds_and_sizes_workspace(shape):
    B, Hq, Hkv, d, S = shape
    n = lf.lf_plan_nsplit(B, Hq, Hkv, d, S, 256)
    assert 1 <= n <= S
    length = -(-S // n)
    assert -(-S // length) == n  # no empty split
    assert length * _gp(Hq // Hkv) * 4 <= 136 * 1024
    ws = lf.lf_workspace_size(B, Hq, Hkv, d, S, n)
    assert ws % 256 == 0 and ws >= 256
    if n > 1:
        assert ws >= B * Hkv * S * (_gp(Hq // Hkv) + 1) * 4


def test_plan_for_the_named_workloads():
    assert lf.lf_plan_nsplit(128, 32, 8, 128, 3200, 256) == 1
    assert lf.lf_plan_nsplit(16, 64, 8, 128, 16384, 256) >= 4
    assert lf.lf_plan_nsplit(256, 32, 8, 128, 8192, 256) == 1
    # few pairs: split to give every compute unit work
    assert lf.lf_plan_nsplit(1, 32, 8, 128, 3000, 256) > 1


class Fake:
    """Distinct, aligned, non-overlapping fake device addresses (never dereferenced)."""

    def __init__(self, B=2, Hq=8, Hkv=2, d=128, S=100, nsplit=1):
        self.shape = (B, Hq, Hkv, d, S)
        self.nsplit = nsplit
        names = ["q", "k", "v", "mask", "nk", "nv", "prev", "out", "scores", "evict", "ws"]
        self.addr = {n: (1 << 40) + i * (1 << 34) for i, n in enumerate(names)}
        self.ws_bytes = lf.lf_workspace_size(B, Hq, Hkv, d, S, nsplit)

    def call(self, scale=0.1, ws_bytes=None, nsplit=None, shape=None, **over):
        a = dict(self.addr, **over)
        return lf.lf_validate(*(shape or self.shape), scale, a["q"], a["k"], a["v"], a["mask"], a["nk"], a["nv"],
                              a["prev"], a["out"], a["scores"], a["evict"], a["ws"],
                              self.ws_bytes if ws_bytes is None else ws_bytes,
                              self.nsplit if nsplit is None else nsplit)


def test_validate_accepts_good_arguments():
    assert Fake().call() == lf.LF_OK
    f = Fake(nsplit=3)
    assert f.call() == lf.LF_OK


@pytest.mark.parametrize("name", ["q", "k", "v", "mask", "nk", "nv", "prev", "out", "scores", "evict", "ws"])
def test_validate_null(name):
    assert Fake().call(**{name: 0}) == lf.LF_E_NULL


@pytest.mark.parametrize("name,offset", [("q", 8), ("k", 2), ("v", 4), ("nk", 8), ("nv", 8), ("out", 2),
                                         ("scores", 2), ("prev", 1), ("evict", 2), ("ws", 128)])
def test_validate_alignment(name, offset):
    f = Fake()
    assert f.call(**{name: f.addr[name] + offset}) == lf.LF_E_ALIGN


def test_validate_mask_needs_no_alignment():
    f = Fake()
    assert f.call(mask=f.addr["mask"] + 1) == lf.LF_OK


@pytest.mark.parametrize("a,b,off", [("out", "q", 0), ("evict", "prev", 0), ("k", "v", 256),
                                     ("scores", "k", 1024), ("ws", "out", 0), ("v", "mask", 0)])
def test_validate_alias(a, b, off):
    f = Fake()
    assert f.call(**{a: f.addr[b] + off}) == lf.LF_E_ALIAS


def test_read_only_inputs_may_share_memory():
    f = Fake()
    assert f.call(nv=f.addr["nk"]) == lf.LF_OK


def test_validate_workspace_and_split():
    f = Fake()
    assert f.call(ws_bytes=f.ws_bytes - 1) == lf.LF_E_WORKSPACE
    assert f.call(nsplit=0) == lf.LF_E_NSPLIT
    assert f.call(nsplit=101) == lf.LF_E_NSPLIT
    big = Fake(B=1, Hq=8, Hkv=1, S=10000, nsplit=1)
    assert big.call() == lf.LF_E_NSPLIT  # 10000 slots x 8 heads of logits exceed the LDS budget
    assert big.call(nsplit=3, ws_bytes=lf.lf_workspace_size(1, 8, 1, 128, 10000, 3)) == lf.LF_OK
    f3 = Fake(nsplit=3)
    assert f3.call(ws_bytes=lf.lf_workspace_size(2, 8, 2, 128, 100, 1)) == lf.LF_E_WORKSPACE


def test_validate_scale_and_empty_batch():
    f = Fake()
    assert f.call(scale=float("nan")) == lf.LF_E_VALUE
    assert f.call(scale=float("inf")) == lf.LF_E_VALUE
    zeros = {n: 0 for n in f.addr}
    assert f.call(shape=(0, 8, 2, 128, 100), **zeros) == lf.LF_OK
    assert f.call(shape=(2, 8, 3, 128, 100)) == lf.LF_E_SHAPE


def _fill_call(f, nsplit=1, ws_bytes=None, scale=0.1, shape=None, **over):
    """longflow_decode_fill on fake addresses; only argument errors are asked
    for, which return before anything is enqueued."""
    a = dict(f.addr, **over)
    P = lambda x: ctypes.c_void_p(x)
    return lf._lib.longflow_decode_fill(
        *(shape or f.shape), scale, P(a["q"]), P(a["k"]), P(a["v"]), P(a["mask"]), P(a["nk"]), P(a["nv"]),
        P(a["prev"]), P(a["out"]), P(a["scores"]), P(a["evict"]), P(a["ws"]),
        f.ws_bytes if ws_bytes is None else ws_bytes, nsplit, None)


def test_fill_argument_errors():
    f = Fake()
    assert _fill_call(f, nsplit=-1) == lf.LF_E_NSPLIT
    assert _fill_call(f, nsplit=101) == lf.LF_E_NSPLIT
    assert _fill_call(f, q=0) == lf.LF_E_NULL
    assert _fill_call(f, out=f.addr["out"] + 2) == lf.LF_E_ALIGN
    assert _fill_call(f, ws_bytes=f.ws_bytes - 1) == lf.LF_E_WORKSPACE
    assert _fill_call(f, scale=float("nan")) == lf.LF_E_VALUE
    assert _fill_call(f, shape=(2, 8, 3, 128, 100)) == lf.LF_E_SHAPE
    zeros = {n: 0 for n in f.addr}
    assert _fill_call(f, shape=(0, 8, 2, 128, 100), **zeros) == lf.LF_OK


@pytest.mark.parametrize("a,b", [("mask", "q"), ("mask", "nk"), ("mask", "prev"), ("prev", "mask")])
def test_fill_mask_is_written(a, b):
    """The fill step writes the mask, so it may not share memory with any
    input; the plain step only reads it."""
    f = Fake()
    assert _fill_call(f, **{a: f.addr[b]}) == lf.LF_E_ALIAS
    assert f.call(**{a: f.addr[b]}) == lf.LF_OK


def _ex_call(f, fill=0, nsplit=1, split_path=0, shape=None, **over):
    """longflow_decode_ex on fake addresses (argument errors only)."""
    a = dict(f.addr, **over)
    P = lambda x: ctypes.c_void_p(x)
    return lf._lib.longflow_decode_ex(
        *(shape or f.shape), 0.1, P(a["q"]), P(a["k"]), P(a["v"]), P(a["mask"]), fill, P(a["nk"]), P(a["nv"]),
        P(a["prev"]), P(a["out"]), P(a["scores"]), P(a["evict"]), P(a["ws"]), f.ws_bytes, nsplit, split_path, None)


def test_general_entry_argument_errors():
    """longflow_decode_ex: the split path must be one of the three, the split
    count non-negative; with fill = 1 the mask is written (so it may not share
    memory with an input), with fill = 0 it is only read."""
    f = Fake()
    assert (lf.LF_SPLIT_AUTO, lf.LF_SPLIT_COMBINE, lf.LF_SPLIT_TEAM) == (0, 1, 2)
    assert _ex_call(f, split_path=3) == lf.LF_E_NSPLIT
    assert _ex_call(f, split_path=-1) == lf.LF_E_NSPLIT
    assert _ex_call(f, nsplit=-1) == lf.LF_E_NSPLIT
    assert _ex_call(f, nsplit=101) == lf.LF_E_NSPLIT
    assert _ex_call(f, q=0) == lf.LF_E_NULL
    assert _ex_call(f, fill=1, mask=f.addr["q"]) == lf.LF_E_ALIAS
    assert _ex_call(f, shape=(2, 8, 3, 128, 100)) == lf.LF_E_SHAPE
    zeros = {n: 0 for n in f.addr}
    assert _ex_call(f, shape=(0, 8, 2, 128, 100), split_path=2, **zeros) == lf.LF_OK


# The one-split pair schedule after the 256-byte header: for up to 4096
# pairs, a 32-bit valid extent each and two 32-bit pair-order buffers.
ORDER_REGION = 3 * 4096 * 4


def test_fill_workspace_has_free_slot_minima():
    """Every workspace holds the 256-byte header and the one-split pair
    schedule; split workspaces then hold one 32-bit lowest-free-slot word per combine chunk,
    then the team path's exchange region: per split of a pair 64-bit words for
    its (max, sum) per padded head, its three results and its O accumulators,
    one 32-bit counter per pair and eight 32-bit ticket counters."""
    B, Hq, Hkv, d, S = 4, 16, 2, 128, 5000
    one = lf.lf_workspace_size(B, Hq, Hkv, d, S, 1)
    assert one == 256 + ORDER_REGION
    chunks = -(-S // 2048)
    pairs = B * Hkv
    gp = 8
    split = 3
    expect = 256 + ORDER_REGION
    for n in (pairs * split * gp * 2 * 4, pairs * split * gp * d * 4, pairs * S * gp * 4, pairs * S * 4,
              pairs * chunks * 8, pairs * chunks * 4, pairs * split * (gp * 2 + 3 + gp * d) * 8 + pairs * 4 + 8 * 4):
        expect += -(-n // 256) * 256
    assert lf.lf_workspace_size(B, Hq, Hkv, d, S, split) == expect


def _topk_call(B=2, Hkv=3, S=50, k=5, scores=1 << 40, mask=(1 << 40) + (1 << 34), out=(1 << 40) + (2 << 34)):
    P = lambda x: ctypes.c_void_p(x)
    return lf._lib.longflow_evict_topk(B, Hkv, S, k, P(scores), P(mask), P(out), None)


def test_topk_argument_errors():
    assert _topk_call(k=0) == lf.LF_E_SHAPE
    assert _topk_call(k=51) == lf.LF_E_SHAPE
    assert _topk_call(Hkv=0) == lf.LF_E_SHAPE
    assert _topk_call(S=0, k=1) == lf.LF_E_SHAPE
    assert _topk_call(B=-1) == lf.LF_E_SHAPE
    assert _topk_call(scores=0) == lf.LF_E_NULL
    assert _topk_call(mask=0) == lf.LF_E_NULL
    assert _topk_call(out=0) == lf.LF_E_NULL
    assert _topk_call(scores=(1 << 40) + 2) == lf.LF_E_ALIGN
    assert _topk_call(out=(1 << 40) + (2 << 34) + 1) == lf.LF_E_ALIGN
    assert _topk_call(out=(1 << 40) + 1024) == lf.LF_E_ALIAS            # inside scores
    assert _topk_call(out=(1 << 40) + (1 << 34) + 8) == lf.LF_E_ALIAS   # inside the mask
    assert _topk_call(B=0, scores=0, mask=0, out=0) == lf.LF_OK


def _stack_call(L=2, B=2, H=256, Hq=4, Hkv=2, d=64, S=40, nsplit=1, ws_bytes=None, x_out=None, k1=None,
                x_in=None, scale=0.125):
    """longflow_stack_step on fake addresses; only argument errors are asked
    for, which return before anything is enqueued."""
    base = 1 << 40
    step = 1 << 34
    addr = iter(base + i * step for i in range(64))
    x_in = next(addr) if x_in is None else x_in
    xo = next(addr) if x_out is None else x_out
    pos, ws = next(addr), next(addr)
    per = {n: [next(addr) for _ in range(L)] for n in ("wq", "wo", "k", "v", "m", "s")}
    if k1 is not None:
        per["k"][1] = k1
    arr = lambda xs: (ctypes.c_void_p * L)(*xs)
    if ws_bytes is None:
        ws_bytes = lf.lf_stack_workspace_size(L, B, H, Hq, Hkv, d, S, max(nsplit, 1))
    P = ctypes.c_void_p
    return lf._lib.longflow_stack_step(L, B, H, Hq, Hkv, d, S, scale, 1e6, P(x_in), P(xo), P(pos), 1,
                                       arr(per["wq"]), arr(per["wo"]), arr(per["k"]), arr(per["v"]),
                                       arr(per["m"]), arr(per["s"]), None, P(ws), ws_bytes, nsplit, None), per


def test_stack_argument_errors():
    for kw in ({"L": 0}, {"B": 0}, {"B": 257}, {"H": 96}, {"H": 128}, {"H": 384}, {"Hq": 6, "Hkv": 4}, {"d": 96},
               {"Hq": 2, "Hkv": 1}):
        args = dict(kw)
        assert lf._lib.longflow_stack_step(
            args.get("L", 2), args.get("B", 2), args.get("H", 256), args.get("Hq", 4), args.get("Hkv", 2),
            args.get("d", 64), 40, 0.1, 1e6, *([None] * 3), 1, *([None] * 7), None, 0, 1, None) == lf.LF_E_SHAPE, kw
    assert _stack_call(x_in=0)[0] == lf.LF_E_NULL
    assert _stack_call(x_in=(1 << 40) + 2)[0] == lf.LF_E_ALIGN
    assert _stack_call(scale=float("nan"))[0] == lf.LF_E_VALUE
    assert _stack_call(nsplit=-1)[0] == lf.LF_E_NSPLIT
    assert _stack_call(ws_bytes=256)[0] == lf.LF_E_WORKSPACE


def test_stack_alias_errors():
    assert _stack_call(x_out=1 << 40)[0] == lf.LF_E_ALIAS            # x_out on x_in
    rc, per = _stack_call(k1=(1 << 40) + 6 * (1 << 34) + 512)       # layer 1's K inside layer 0's K
    assert rc == lf.LF_E_ALIAS


def test_stack_workspace_size():
    """The decode workspace first, then q, k, v, O, two activation buffers, a
    scores buffer, the step's RoPE table (B x d/2 (cos, sin) pairs) and the
    projections' split-K partials (fp32, the larger of the two projections),
    each rounded up to 256 bytes."""
    up = lambda n: -(-n // 256) * 256

    def ksplit(N, K):  # the projection's K slices: whole 256-deep pieces, at most 8 per slice,
        blocks, pieces = -(-N // 128), K // 256  # then as many as about 256 workgroups of 128 columns allow
        ks = min(c for c in range(1, pieces + 1) if pieces % c == 0 and pieces // c <= 8)
        return max(c for c in range(ks, pieces + 1) if pieces % c == 0 and (c == ks or blocks * c <= 256))

    for L, B, H, Hq, Hkv, d, S in ((3, 5, 256, 8, 2, 64, 300), (36, 128, 4096, 32, 8, 128, 3200),
                                   (2, 200, 5120, 40, 8, 128, 64), (1, 7, 2304, 18, 3, 128, 40)):
        nq = (Hq + 2 * Hkv) * d
        part = max(ksplit(nq, H) * B * nq * 4, ksplit(H, Hq * d) * B * H * 4)
        for ns in (1, 3):
            dec = lf.lf_workspace_size(B, Hq, Hkv, d, S, ns)
            want = up(dec) + up(B * Hq * d * 2) + 2 * up(B * Hkv * d * 2) \
                + up(B * Hq * d * 2) + 2 * up(B * H * 2) + up(B * Hkv * S * 4) + up(B * (d // 2) * 8) + up(part)
            assert lf.lf_stack_workspace_size(L, B, H, Hq, Hkv, d, S, ns) == want
    assert ksplit(6144, 4096) == 4 and ksplit(4096, 4096) == 8
    assert ksplit(7168, 5120) == 4 and ksplit(5120, 5120) == 5 and ksplit(256, 2304) == 9
    # the GPU stack tests' shapes reach every unrolled slice length (chunks of 128)
    chunks = set()
    for H, Hq, Hkv in ((8448, 32, 8), (1280, 48, 8), (3072, 72, 9), (3584, 32, 8), (4096, 32, 8), (256, 4, 2)):
        nq = (Hq + 2 * Hkv) * 128
        chunks |= {2 * (H // 256) // ksplit(nq, H), 2 * (Hq * 128 // 256) // ksplit(H, Hq * 128)}
    assert chunks == {2, 4, 6, 8, 10, 12, 14, 16}


_LAYOUT_CHECK = r"""
#include <cstdio>
#include <cstdlib>
#include "layout.h"
// Every workspace region of a split step lies inside the workspace, is
// aligned for its element type and overlaps no other region (the one-split
// schedule region included); the team region holds exactly its words and
// the fill of zero_words covers it.
int main() {
  int bad = 0, cases = 0;
  const int Bs[] = {1, 2, 3, 16, 128, 257}, Hkvs[] = {1, 2, 8}, gs[] = {1, 2, 3, 4, 8}, ds[] = {64, 128};
  const int Ss[] = {1, 7, 256, 777, 3200, 16384, 65536}, ns[] = {2, 3, 4, 5, 16, 64, 1024};
  for (int B : Bs) for (int Hkv : Hkvs) for (int g : gs) for (int d : ds) for (int S : Ss) for (int n : ns) {
    if (n > S) continue;
    int len, eff;
    lf::split_geometry(S, n, &len, &eff);
    if (eff < 2) continue;
    const int gp = lf::padded_group(g);
    const lf::WorkspaceLayout w = lf::workspace_layout(B, Hkv, d, S, gp, eff);
    const lf::TeamLayout t = lf::team_layout(w, B, Hkv, d, gp, eff);
    const size_t pairs = (size_t)B * Hkv;
    struct R { size_t off, bytes, align; } r[] = {
      {w.part_ml, pairs * eff * gp * 2 * 4, 4}, {w.part_o, pairs * eff * gp * (size_t)d * 4, 4},
      {w.logit, pairs * (size_t)S * gp * 4, 16}, {w.vnorm, pairs * (size_t)S * 4, 4},
      {w.cand, pairs * (size_t)lf::combine_chunks(S) * 8, 8}, {w.ffree, pairs * (size_t)lf::combine_chunks(S) * 4, 4},
      {w.team, lf::team_region_bytes(pairs, eff, gp, d), 8}, {w.order, lf::kOrderRegionBytes, 4}};
    const int nr = sizeof(r) / sizeof(r[0]);
    ++cases;
    // the schedule region sits at the same place in one-split layouts, and
    // a team step's share of the workspace reaches past its team words
    const lf::WorkspaceLayout w1 = lf::workspace_layout(B, Hkv, d, S, gp, 1);
    if (w1.order != 256 || w1.total != 256 + lf::kOrderRegionBytes || w.order != w1.order) ++bad;
    if (lf::team_workspace_bytes(B, Hkv, d, gp, eff) < w.team + lf::team_region_bytes(pairs, eff, gp, d)) ++bad;
    for (int i = 0; i < nr; ++i) {
      if (r[i].off < 256 || r[i].off + r[i].bytes > w.total || r[i].off % r[i].align) ++bad;
      for (int k = i + 1; k < nr; ++k)
        if (r[i].off < r[k].off + r[k].bytes && r[k].off < r[i].off + r[i].bytes) ++bad;
    }
    if (t.xstat != w.team || t.xfin != t.xstat + pairs * eff * gp * 16 || t.xo != t.xfin + pairs * eff * 24 ||
        t.xcnt != t.xo + pairs * eff * gp * (size_t)d * 8 || t.xticket != t.xcnt + pairs * 4 ||
        t.xticket + 4 * lf::kTicketRanges != w.team + t.zero_words * 4 || t.xo % 8 || t.xcnt % 4 ||
        t.zero_words * 4 != lf::team_region_bytes(pairs, eff, gp, d))
      ++bad;
  }
  for (int pairs = 1; pairs < 3000; pairs += 7) {
    for (int rg = 1; rg <= lf::kTicketRanges; rg *= 2) {
      if (lf::ticket_range_first_pair(pairs, 0, rg) != 0 || lf::ticket_range_first_pair(pairs, rg, rg) != pairs) ++bad;
      for (int r = 0; r < rg; ++r)
        if (lf::ticket_range_first_pair(pairs, r + 1, rg) < lf::ticket_range_first_pair(pairs, r, rg)) ++bad;
    }
  }
  printf("%d %d\n", cases, bad);
  return 0;
}
"""


def test_workspace_regions_fit_and_do_not_overlap(tmp_path):
    """Host C++ check of the workspace layout of split steps (schedule,
    combine and team regions) over a grid of shapes and split counts."""
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    src = tmp_path / "layout_check.cpp"
    src.write_text(_LAYOUT_CHECK)
    exe = tmp_path / "layout_check"
    csrc = os.path.join(os.path.dirname(INCLUDE), "decode_attention_kv_05_amd", "csrc")
    subprocess.run([gxx, "-std=c++17", "-O1", "-I", csrc, str(src), "-o", str(exe)], check=True)
    cases, bad = map(int, subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split())
    assert cases > 1000 and bad == 0, (cases, bad)


def test_stack_workspace_offsets():
    """The last layer's q, k_new, v_new and O sit in the stack workspace's
    activation regions: after the decode workspace, 256-byte aligned,
    disjoint and inside the size lf_stack_workspace_size reports."""
    for B, H, Hq, Hkv, d, S, ns in ((3, 256, 8, 2, 64, 300, 1), (128, 4096, 32, 8, 128, 3200, 1),
                                    (7, 2304, 18, 3, 128, 40, 3)):
        offs = lf.lf_stack_workspace_offsets(B, H, Hq, Hkv, d, S, ns)
        sizes = (B * Hq * d * 2, B * Hkv * d * 2, B * Hkv * d * 2, B * Hq * d * 2)
        total = lf.lf_stack_workspace_size(1, B, H, Hq, Hkv, d, S, ns)
        dec = lf.lf_workspace_size(B, Hq, Hkv, d, S, ns)
        spans = sorted(zip(offs, sizes))
        assert spans[0][0] >= dec and all(o % 256 == 0 for o in offs)
        for (o1, n1), (o2, _) in zip(spans, spans[1:]):
            assert o1 + n1 <= o2
        assert spans[-1][0] + spans[-1][1] <= total
    with pytest.raises(ValueError):
        lf.lf_stack_workspace_offsets(3, 256, 8, 2, 64, 300, 0)


def test_workspace_size_for_the_device_plan_needs_a_device():
    """nsplit = 0 sizes the workspace for the device's own plan; with no
    usable device the call reports LF_E_HIP (and an explicit count never
    touches the device)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present; the GPU tests cover nsplit = 0")
    out = ctypes.c_size_t(0)
    rc = lf._lib.lf_workspace_size(128, 32, 8, 128, 3200, 0, ctypes.byref(out))
    assert rc == lf.LF_E_HIP
    assert lf.lf_workspace_size(128, 32, 8, 128, 3200, 1) == 256 + ORDER_REGION


def test_library_records_its_source_hash():
    """The built library carries the hash of the sources it was built from,
    both as an export and as a tag in the file that the build script reads
    without loading it; ensure_built rebuilds when they differ."""
    from decode_attention_kv_05_amd.build import built_hash, source_hash
    assert lf.lf_source_hash() == source_hash() == built_hash()
    assert len(lf.lf_source_hash()) == 16
