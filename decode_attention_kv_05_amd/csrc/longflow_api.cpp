// Host side of liblongflow.so: argument checks, split planning, workspace
// layout and the stream-ordered launch.  Declarations and the operator's
// definition are in include/longflow.h.

#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "launch.h"
#include "layout.h"
#include "longflow.h"


#ifndef LF_SOURCE_HASH
#define LF_SOURCE_HASH "unknown"
#endif

namespace {

// The hash of the sources this library was built from, behind a tag that
// the build script can find in the file without loading it.
const char kSourceHashTag[] = "lf-source-hash:" LF_SOURCE_HASH;
constexpr size_t kSourceHashTagLen = sizeof("lf-source-hash:") - 1;

constexpr int kMaxDevices = 64;
std::atomic<int> g_num_cus[kMaxDevices];

bool misaligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) != 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}


}  // namespace

extern "C" {

int lf_version(void) { return LF_ABI_VERSION; }

const char* lf_source_hash(void) { return kSourceHashTag + kSourceHashTagLen; }

const char* lf_strerror(int code) {
  switch (code) {
    case LF_OK: return "ok";
    case LF_E_NULL: return "a required pointer is NULL";
    case LF_E_SHAPE: return "unsupported or inconsistent sizes";
    case LF_E_ALIGN: return "a pointer misses its required alignment";
    case LF_E_ALIAS: return "an output overlaps an input or another output";
    case LF_E_WORKSPACE: return "workspace too small";
    case LF_E_HIP: return "HIP runtime call or kernel launch failed";
    case LF_E_NSPLIT: return "slot split count not usable for this shape";
    case LF_E_VALUE: return "non-finite scale";
    case LF_E_SCRATCH: return "the step needs more scratch memory than the library's static buffer holds";
    default: return "unknown longflow status code";
  }
}

int lf_check_shape(int B, int Hq, int Hkv, int d, int S) {
  if (B < 0 || Hq < 1 || Hkv < 1 || S < 1) return LF_E_SHAPE;
  if (d != 64 && d != 128) return LF_E_SHAPE;
  if (Hq % Hkv != 0) return LF_E_SHAPE;
  if (Hq / Hkv > lf::kMaxGroup) return LF_E_SHAPE;
  if ((int64_t)B * Hkv > INT_MAX || (int64_t)B * Hq > INT_MAX) return LF_E_SHAPE;
  return LF_OK;
}

int lf_plan_nsplit(int B, int Hq, int Hkv, int d, int S, int num_cus, int* nsplit) {
  if (!nsplit) return LF_E_NULL;
  int rc = lf_check_shape(B, Hq, Hkv, d, S);
  if (rc != LF_OK) return rc;
  if (num_cus < 1) num_cus = 1;
  const int gp = lf::padded_group(Hq / Hkv);
  const int64_t pairs = (int64_t)B * Hkv > 0 ? (int64_t)B * Hkv : 1;
  // The logits of a split must fit the LDS budget.
  const int64_t need = ((int64_t)S + lf::max_split_len(d, gp) - 1) / lf::max_split_len(d, gp);
  int64_t n = need;
  // One workgroup per pair keeps the whole step in one workgroup (no
  // exchange between splits); use it when there are enough pairs to give
  // every compute unit work.  Otherwise split the slots until there are
  // about two workgroups per compute unit, but not below 256 slots a split.
  // (Smaller splits that let two workgroups share a CU measured slower for
  // the 16384-slot GQA-8 cache on both split paths: team 261 us with 8
  // splits against 243 us with 4, combine 284 against 270.)
  if (!(need == 1 && pairs >= num_cus)) {
    const int64_t target = (2LL * num_cus + pairs - 1) / pairs;
    const int64_t cap = ((int64_t)S + 255) / 256;
    if (target > n) n = target < cap ? target : cap;
    if (n < need) n = need;
    // Splits short enough for the team path, which also keeps |v|_1 per row.
    const int team_len = lf::max_split_len(d, gp, true);
    const int64_t team_need = ((int64_t)S + team_len - 1) / team_len;
    if (n > 1 && n < team_need) n = team_need;
  }
  if (n < 1) n = 1;
  if (n > lf::kMaxSplits) return LF_E_SHAPE;
  int len, eff;
  lf::split_geometry(S, (int)n, &len, &eff);
  *nsplit = eff;
  return LF_OK;
}

int lf_workspace_size(int B, int Hq, int Hkv, int d, int S, int nsplit, size_t* bytes) {
  if (!bytes) return LF_E_NULL;
  int rc = lf_check_shape(B, Hq, Hkv, d, S);
  if (rc != LF_OK) return rc;
  if (nsplit == 0) {
    // The count longflow_decode plans for the current device.
    int cus = 0;
    if ((rc = lf_device_num_cus(&cus)) != LF_OK) return rc;
    if ((rc = lf_plan_nsplit(B, Hq, Hkv, d, S, cus, &nsplit)) != LF_OK) return rc;
  }
  if (nsplit < 1 || nsplit > S || nsplit > lf::kMaxSplits) return LF_E_NSPLIT;
  int len, eff;
  lf::split_geometry(S, nsplit, &len, &eff);
  *bytes = lf::workspace_layout(B, Hkv, d, S, lf::padded_group(Hq / Hkv), eff).total;
  return LF_OK;
}

int lf_device_num_cus(int* num_cus) {
  if (!num_cus) return LF_E_NULL;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LF_E_HIP;
  if (dev >= 0 && dev < kMaxDevices) {
    const int cached = g_num_cus[dev].load(std::memory_order_relaxed);
    if (cached > 0) {
      *num_cus = cached;
      return LF_OK;
    }
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return LF_E_HIP;
  if (dev >= 0 && dev < kMaxDevices) g_num_cus[dev].store(n, std::memory_order_relaxed);
  *num_cus = n;
  return LF_OK;
}

int lf_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return LF_E_NULL;
  if (misaligned(workspace, 256)) return LF_E_ALIGN;
  if (workspace_bytes < 256 || workspace_bytes % 4 != 0) return LF_E_WORKSPACE;
  return lf::launch_fill_u32(static_cast<uint32_t*>(workspace), workspace_bytes / 4, 0u,
                             static_cast<hipStream_t>(stream)) == hipSuccess
             ? LF_OK
             : LF_E_HIP;
}

}  // extern "C"

namespace {

// The checks of lf_validate; `mask_written` marks the fill step, which
// updates the mask in place (so it must not overlap any other buffer).
// `team_only`: the workspace need only hold what a team-path step touches.
int validate_step(int B, int Hq, int Hkv, int d, int S, float scale, const void* q,
                  const void* k_cache, const void* v_cache, const uint8_t* mask, const void* new_k,
                  const void* new_v, const int32_t* prev_slot, const void* out, const float* scores,
                  const int32_t* evict_slot, const void* workspace, size_t workspace_bytes,
                  int nsplit, bool mask_written, bool team_only = false) {
  int rc = lf_check_shape(B, Hq, Hkv, d, S);
  if (rc != LF_OK) return rc;
  if (!std::isfinite(scale)) return LF_E_VALUE;
  if (B == 0) return LF_OK;
  if (!q || !k_cache || !v_cache || !mask || !new_k || !new_v || !prev_slot || !out || !scores ||
      !evict_slot || !workspace)
    return LF_E_NULL;
  if (misaligned(q, 16) || misaligned(k_cache, 16) || misaligned(v_cache, 16) ||
      misaligned(new_k, 16) || misaligned(new_v, 16) || misaligned(out, 16) ||
      misaligned(scores, 4) || misaligned(prev_slot, 4) || misaligned(evict_slot, 4) ||
      misaligned(workspace, 256))
    return LF_E_ALIGN;
  if (nsplit < 1 || nsplit > S || nsplit > lf::kMaxSplits) return LF_E_NSPLIT;
  const int gp = lf::padded_group(Hq / Hkv);
  int len, eff;
  lf::split_geometry(S, nsplit, &len, &eff);
  if (len > lf::max_split_len(d, gp)) return LF_E_NSPLIT;
  if ((int64_t)B * Hkv * eff > INT_MAX) return LF_E_NSPLIT;

  const size_t pairs = (size_t)B * Hkv;
  const size_t q_bytes = (size_t)B * Hq * d * 2;
  const size_t cache_bytes = pairs * S * d * 2;
  const size_t mask_bytes = (size_t)B * S;
  const size_t row_bytes = pairs * d * 2;
  const size_t idx_bytes = pairs * 4;
  const size_t score_bytes = pairs * S * 4;
  const size_t ws_need = team_only ? lf::team_workspace_bytes(B, Hkv, d, gp, eff)
                                   : lf::workspace_layout(B, Hkv, d, S, gp, eff).total;

  struct Buf {
    const void* p;
    size_t n;
    bool written;
  };
  const Buf bufs[] = {
      {q, q_bytes, false},           {mask, mask_bytes, mask_written}, {new_k, row_bytes, false},
      {new_v, row_bytes, false},     {prev_slot, idx_bytes, false}, {k_cache, cache_bytes, true},
      {v_cache, cache_bytes, true},  {out, q_bytes, true},        {scores, score_bytes, true},
      {evict_slot, idx_bytes, true}, {workspace, ws_need, true},
  };
  const int nb = (int)(sizeof(bufs) / sizeof(bufs[0]));
  for (int i = 0; i < nb; ++i)
    for (int k = i + 1; k < nb; ++k)
      if ((bufs[i].written || bufs[k].written) &&
          overlaps(bufs[i].p, bufs[i].n, bufs[k].p, bufs[k].n))
        return LF_E_ALIAS;
  if (workspace_bytes < ws_need) return LF_E_WORKSPACE;
  return LF_OK;
}

}  // namespace

namespace lf {

// Ticket ranges for a team launch, or 0 when the team path cannot be taken.
// Its workgroups take (pair, split) tickets in the order they start, so in
// each range every team but the one holding the newest ticket is already
// running, and at most ranges * (nsplit - 1) workgroups ever wait for
// teammates that have not started.  Workgroups are dealt to the XCDs in
// turn and dispatched in block order, each waiting for room on its own XCD,
// and the waiting ones may all sit on one XCD; the next workgroup bound for
// it then starts only if that XCD also holds a workgroup that is not
// waiting.  So one XCD must hold more workgroups at once than can ever be
// waiting; the most ranges (of 8, 4, 2, 1) for which it does are used.
// (Counting the whole device instead let 64-split steps on 256 CUs stall
// until the waits' deadline now and then.)
static int team_ticket_ranges(int d, int gp, int nw, size_t lds, int nsplit_eff) {
  if (nsplit_eff < 2 || nsplit_eff > lf::kMaxTeamSplits) return 0;
  int per_cu = 0, cus = 0;
  if (lf_device_num_cus(&cus) != LF_OK) return 0;
  if (lf::decode_blocks_per_cu(true, d, gp, nw, lds, &per_cu) != hipSuccess || per_cu < 1) return 0;
  const int64_t per_xcd = (int64_t)per_cu * (cus >= lf::kXcds ? cus / lf::kXcds : cus);
  for (int r = lf::kTicketRanges; r >= 1; r /= 2)
    if (per_xcd > (int64_t)r * (nsplit_eff - 1)) return r;
  return 0;
}

// Enqueue one step after validation: the decode kernel, and for several
// splits either the team launch or the combine and finalize kernels.
int enqueue_decode_step(int B, int Hq, int Hkv, int d, int S, float scale, const void* q, void* k_cache,
                 void* v_cache, const uint8_t* mask, uint8_t* mask_w, const void* new_k,
                 const void* new_v, const int32_t* prev_slot, void* out, float* scores,
                 int32_t* evict_slot, void* workspace, int nsplit, int split_path, void* stream,
                 bool team_only, bool schedule) {
  const int G = Hq / Hkv;
  const int gp = lf::padded_group(G);
  int len, eff;
  lf::split_geometry(S, nsplit, &len, &eff);
  const lf::WorkspaceLayout wl = lf::workspace_layout(B, Hkv, d, S, gp, eff);
  unsigned char* ws = static_cast<unsigned char*>(workspace);

  lf::DecodeParams prm{};
  prm.q = static_cast<const uint16_t*>(q);
  prm.k = static_cast<uint16_t*>(k_cache);
  prm.v = static_cast<uint16_t*>(v_cache);
  prm.mask = mask;
  prm.mask_w = mask_w;
  prm.fill = mask_w != nullptr;
  prm.new_k = static_cast<const uint16_t*>(new_k);
  prm.new_v = static_cast<const uint16_t*>(new_v);
  prm.prev = prev_slot;
  prm.out = static_cast<uint16_t*>(out);
  prm.scores = scores;
  prm.evict = evict_slot;
  prm.status = reinterpret_cast<uint32_t*>(ws + wl.status);
  prm.queue = reinterpret_cast<uint32_t*>(ws + wl.queue);
  prm.part_ml = reinterpret_cast<float*>(ws + wl.part_ml);
  prm.part_o = reinterpret_cast<float*>(ws + wl.part_o);
  prm.ws_logit = reinterpret_cast<float*>(ws + wl.logit);
  prm.ws_vnorm = reinterpret_cast<float*>(ws + wl.vnorm);
  prm.cand = reinterpret_cast<uint64_t*>(ws + wl.cand);
  prm.ffree = reinterpret_cast<uint32_t*>(ws + wl.ffree);
  if (team_only) {
    // The workspace ends after the team region: the combine path's arrays
    // are not there (the team path and the one-split step never use them).
    prm.part_ml = prm.part_o = prm.ws_logit = prm.ws_vnorm = nullptr;
    prm.cand = nullptr;
    prm.ffree = nullptr;
    if (eff > 1) split_path = LF_SPLIT_TEAM;
  }
  prm.Hq = Hq;
  prm.Hkv = Hkv;
  prm.G = G;
  prm.S = S;
  prm.nsplit = eff;
  prm.split_len = len;
  // Logits are kept in the log2 domain: exp(scale * x) = exp2(scale * log2(e) * x).
  prm.qscale = scale * 1.4426950408889634f;

  const int nblocks = B * Hkv * eff;
  int nw = lf::decode_waves(gp, len);
  size_t lds = lf::lds_layout(d, gp, len, nw).total;
  prm.pairs = B * Hkv;
  int team_grid = 0;
  if (eff > 1 && split_path != LF_SPLIT_COMBINE) {
    const lf::TeamLayout tl = lf::team_layout(wl, B, Hkv, d, gp, eff);
    const int nw_team = lf::decode_waves(gp, len, true);
    const size_t lds_team = lf::lds_layout(d, gp, len, nw_team, true).total;
    const int ranges = lds_team <= lf::kMaxLdsBytes ? team_ticket_ranges(d, gp, nw_team, lds_team, eff) : 0;
    team_grid = ranges > 0 ? nblocks : 0;
    if (team_grid == 0 && split_path == LF_SPLIT_TEAM) return LF_E_NSPLIT;
    if (team_grid > 0) {
      nw = nw_team;
      lds = lds_team;
      prm.ticket_ranges = ranges;
    }
    prm.xstat = reinterpret_cast<uint64_t*>(ws + tl.xstat);
    prm.xfin = reinterpret_cast<uint64_t*>(ws + tl.xfin);
    prm.xo = reinterpret_cast<uint64_t*>(ws + tl.xo);
    prm.xcnt = reinterpret_cast<uint32_t*>(ws + tl.xcnt);
    prm.xticket = reinterpret_cast<uint32_t*>(ws + tl.xticket);
  }
  // One split: as many persistent workgroups as the device holds at once
  // (fewer when there are fewer pairs); they take the pairs from the
  // work-item counter.
  int grid = 0;
  if (eff == 1) {
    int per_cu = 0, cus = 0;
    if (lf_device_num_cus(&cus) != LF_OK) return LF_E_HIP;
    if (lf::decode_blocks_per_cu(false, d, gp, nw, lds, &per_cu) != hipSuccess || per_cu < 1) return LF_E_HIP;
    const int64_t resident = (int64_t)per_cu * cus;
    grid = (int)(resident < nblocks ? resident : nblocks);
    // With more pairs than workgroups, the workgroups take the pairs in the
    // order of the previous step's valid extents, longest first, so that
    // short pairs fill the end of the step (one-split steps of one pair count
    // sharing the workspace also share the order; it is only a schedule).
    if (schedule && grid < nblocks && nblocks <= lf::kOrderMaxPairs) {
      prm.lens = reinterpret_cast<uint32_t*>(ws + wl.order);
      prm.order = prm.lens + lf::kOrderMaxPairs;
    }
  }
  return lf::launch_decode(prm, d, gp, nw, nblocks, lds, team_grid, grid, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? LF_OK
             : LF_E_HIP;
}

}  // namespace lf

extern "C" {

int lf_validate(int B, int Hq, int Hkv, int d, int S, float scale, const void* q,
                const void* k_cache, const void* v_cache, const uint8_t* mask, const void* new_k,
                const void* new_v, const int32_t* prev_slot, const void* out, const float* scores,
                const int32_t* evict_slot, const void* workspace, size_t workspace_bytes,
                int nsplit) {
  return validate_step(B, Hq, Hkv, d, S, scale, q, k_cache, v_cache, mask, new_k, new_v, prev_slot,
                       out, scores, evict_slot, workspace, workspace_bytes, nsplit, false);
}

int longflow_decode_nsplit(int B, int Hq, int Hkv, int d, int S, float scale, const void* q,
                           void* k_cache, void* v_cache, const uint8_t* mask, const void* new_k,
                           const void* new_v, const int32_t* prev_slot, void* out, float* scores,
                           int32_t* evict_slot, void* workspace, size_t workspace_bytes,
                           int nsplit, void* stream) {
  int rc = lf_validate(B, Hq, Hkv, d, S, scale, q, k_cache, v_cache, mask, new_k, new_v,
                       prev_slot, out, scores, evict_slot, workspace, workspace_bytes, nsplit);
  if (rc != LF_OK) return rc;
  if (B == 0) return LF_OK;
  return lf::enqueue_decode_step(B, Hq, Hkv, d, S, scale, q, k_cache, v_cache, mask, nullptr, new_k, new_v,
                      prev_slot, out, scores, evict_slot, workspace, nsplit, LF_SPLIT_AUTO, stream);
}

int longflow_decode(int B, int Hq, int Hkv, int d, int S, float scale, const void* q,
                    void* k_cache, void* v_cache, const uint8_t* mask, const void* new_k,
                    const void* new_v, const int32_t* prev_slot, void* out, float* scores,
                    int32_t* evict_slot, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = lf_check_shape(B, Hq, Hkv, d, S);
  if (rc != LF_OK) return rc;
  if (B == 0) return std::isfinite(scale) ? LF_OK : LF_E_VALUE;
  int cus = 0;
  rc = lf_device_num_cus(&cus);
  if (rc != LF_OK) return rc;
  int nsplit = 1;
  rc = lf_plan_nsplit(B, Hq, Hkv, d, S, cus, &nsplit);
  if (rc != LF_OK) return rc;
  return longflow_decode_nsplit(B, Hq, Hkv, d, S, scale, q, k_cache, v_cache, mask, new_k, new_v,
                                prev_slot, out, scores, evict_slot, workspace, workspace_bytes,
                                nsplit, stream);
}

int longflow_decode_fill(int B, int Hq, int Hkv, int d, int S, float scale, const void* q,
                         void* k_cache, void* v_cache, uint8_t* mask, const void* new_k,
                         const void* new_v, const int32_t* prev_slot, void* out, float* scores,
                         int32_t* next_slot, void* workspace, size_t workspace_bytes, int nsplit,
                         void* stream) {
  int rc = lf_check_shape(B, Hq, Hkv, d, S);
  if (rc != LF_OK) return rc;
  if (nsplit < 0) return LF_E_NSPLIT;
  if (B == 0) return std::isfinite(scale) ? LF_OK : LF_E_VALUE;
  if (nsplit == 0) {
    int cus = 0;
    rc = lf_device_num_cus(&cus);
    if (rc != LF_OK) return rc;
    rc = lf_plan_nsplit(B, Hq, Hkv, d, S, cus, &nsplit);
    if (rc != LF_OK) return rc;
  }
  rc = validate_step(B, Hq, Hkv, d, S, scale, q, k_cache, v_cache, mask, new_k, new_v, prev_slot,
                     out, scores, next_slot, workspace, workspace_bytes, nsplit, true);
  if (rc != LF_OK) return rc;
  return lf::enqueue_decode_step(B, Hq, Hkv, d, S, scale, q, k_cache, v_cache, mask, mask, new_k, new_v,
                      prev_slot, out, scores, next_slot, workspace, nsplit, LF_SPLIT_AUTO, stream);
}

int longflow_decode_ex(int B, int Hq, int Hkv, int d, int S, float scale, const void* q,
                       void* k_cache, void* v_cache, uint8_t* mask, int fill, const void* new_k,
                       const void* new_v, const int32_t* prev_slot, void* out, float* scores,
                       int32_t* evict_slot, void* workspace, size_t workspace_bytes, int nsplit,
                       int split_path, void* stream) {
  int rc = lf_check_shape(B, Hq, Hkv, d, S);
  if (rc != LF_OK) return rc;
  if (nsplit < 0 || split_path < LF_SPLIT_AUTO || split_path > LF_SPLIT_TEAM) return LF_E_NSPLIT;
  if (B == 0) return std::isfinite(scale) ? LF_OK : LF_E_VALUE;
  if (nsplit == 0) {
    int cus = 0;
    rc = lf_device_num_cus(&cus);
    if (rc != LF_OK) return rc;
    rc = lf_plan_nsplit(B, Hq, Hkv, d, S, cus, &nsplit);
    if (rc != LF_OK) return rc;
  }
  rc = validate_step(B, Hq, Hkv, d, S, scale, q, k_cache, v_cache, mask, new_k, new_v, prev_slot,
                     out, scores, evict_slot, workspace, workspace_bytes, nsplit, fill != 0);
  if (rc != LF_OK) return rc;
  return lf::enqueue_decode_step(B, Hq, Hkv, d, S, scale, q, k_cache, v_cache, mask,
                                 fill ? mask : nullptr, new_k, new_v, prev_slot, out, scores,
                                 evict_slot, workspace, nsplit, split_path, stream);
}

int longflow_evict_topk(int B, int Hkv, int S, int k, const float* scores, const uint8_t* mask,
                        int32_t* evict_slots, void* stream) {
  if (B < 0 || Hkv < 1 || S < 1 || k < 1 || k > S) return LF_E_SHAPE;
  if ((int64_t)B * Hkv > INT_MAX || (int64_t)B * Hkv * k > INT_MAX) return LF_E_SHAPE;
  if (B == 0) return LF_OK;
  if (!scores || !mask || !evict_slots) return LF_E_NULL;
  if (misaligned(scores, 4) || misaligned(evict_slots, 4)) return LF_E_ALIGN;
  const size_t pairs = (size_t)B * Hkv;
  const size_t out_bytes = pairs * k * 4;
  if (overlaps(evict_slots, out_bytes, scores, pairs * S * 4) ||
      overlaps(evict_slots, out_bytes, mask, (size_t)B * S))
    return LF_E_ALIAS;
  lf::TopkParams prm{};
  prm.scores = scores;
  prm.mask = mask;
  prm.out = evict_slots;
  prm.Hkv = Hkv;
  prm.S = S;
  prm.k = k;
  prm.pairs = (int)pairs;
  return lf::launch_topk(prm, static_cast<hipStream_t>(stream)) == hipSuccess ? LF_OK : LF_E_HIP;
}

int lf_read_device_status(const void* workspace, void* stream, uint32_t* flags) {
  if (!workspace || !flags) return LF_E_NULL;
  if (misaligned(workspace, 256)) return LF_E_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  if (hipMemcpyAsync(&v, workspace, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess)
    return LF_E_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return LF_E_HIP;
  *flags = v;
  return LF_OK;
}

}  // extern "C"

// ------------------------------------------------------------------ no-allocation entry point
//
// longflow_decode_noalloc keeps its workspace in `scratch`, a device array of
// the library: one per GPU the library runs on, alive until the process
// ends.  In host code `scratch` names a host-side stand-in, not device
// memory, so its device address is looked up once per device (with that
// device current) and only that address is used.

namespace {

static __device__ __align__(256) unsigned char scratch[LF_STATIC_SCRATCH_BYTES];

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device, or null.
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess) g_scratch_ptr[dev] = ptr;
  });
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int longflow_decode_noalloc(int B, int Hq, int Hkv, int d, int S, float scale, const void* q,
                                       void* k_cache, void* v_cache, const uint8_t* mask, const void* new_k,
                                       const void* new_v, const int32_t* prev_slot, void* out, float* scores,
                                       int32_t* evict_slot, void* stream) {
  int rc = lf_check_shape(B, Hq, Hkv, d, S);
  if (rc != LF_OK) return rc;
  if (B == 0) return std::isfinite(scale) ? LF_OK : LF_E_VALUE;
  int cus = 0, nsplit = 1;
  if ((rc = lf_device_num_cus(&cus)) != LF_OK) return rc;
  if ((rc = lf_plan_nsplit(B, Hq, Hkv, d, S, cus, &nsplit)) != LF_OK) return rc;
  // What the step touches: the header with one split; the header and the
  // team region on the team path; else the whole combine layout.
  const int gp = lf::padded_group(Hq / Hkv);
  int len, eff;
  lf::split_geometry(S, nsplit, &len, &eff);
  bool team_only = false;
  size_t need = 256;
  if (eff > 1) {
    const int nw = lf::decode_waves(gp, len, true);
    const size_t lds = lf::lds_layout(d, gp, len, nw, true).total;
    team_only = lds <= lf::kMaxLdsBytes && lf::team_ticket_ranges(d, gp, nw, lds, eff) > 0;
    need = team_only ? lf::team_workspace_bytes(B, Hkv, d, gp, eff)
                     : lf::workspace_layout(B, Hkv, d, S, gp, eff).total;
  }
  if (need > (size_t)LF_STATIC_SCRATCH_BYTES) return LF_E_SCRATCH;
  void* ws = scratch_on_current_device();
  if (!ws) return LF_E_HIP;
  rc = validate_step(B, Hq, Hkv, d, S, scale, q, k_cache, v_cache, mask, new_k, new_v, prev_slot, out, scores,
                     evict_slot, ws, (size_t)LF_STATIC_SCRATCH_BYTES, nsplit, false, team_only);
  if (rc != LF_OK) return rc;
  // The previous call on this device left its status bits here, and, had
  // one of its team waits run out, set exchange words: this call's header
  // and team region start from zero (a fill kernel, so the call can be
  // recorded into a graph; its caller cannot zero a workspace it never sees).
  // So no pair schedule carries over between calls: a one-split step takes
  // its pairs in index order and leaves the schedule region alone.
  const size_t clear = team_only ? need : 256;
  if (lf::launch_fill_u32(static_cast<uint32_t*>(ws), clear / 4, 0u, static_cast<hipStream_t>(stream)) != hipSuccess)
    return LF_E_HIP;
  return lf::enqueue_decode_step(B, Hq, Hkv, d, S, scale, q, k_cache, v_cache, mask, nullptr, new_k, new_v,
                                 prev_slot, out, scores, evict_slot, ws, nsplit, LF_SPLIT_AUTO, stream, team_only,
                                 false);
}
