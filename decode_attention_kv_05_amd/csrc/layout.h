// Workspace and LDS layout shared by the host planner and the kernels of
// liblongflow.so.  No HIP types.
#pragma once

#include <stddef.h>
#include <stdint.h>

// Callable from host code and, when compiled by hipcc, from kernels.
#if defined(__HIPCC__)
#define LF_HD __host__ __device__
#else
#define LF_HD
#endif

namespace lf {

constexpr int kMaxGroup = 8;          // query heads per KV head supported
constexpr int kWavesSmallLds = 8;   // wavefronts per workgroup when two workgroups fit a CU's LDS
constexpr int kWavesLargeLds = 16;  // wavefronts per workgroup when one workgroup fills the LDS
constexpr int kUnroll = 4;          // 16-byte row loads per lane per batch
// Occupancy hint given to the register allocator, by padded group size:
// waves per SIMD the kernel must fit (512 VGPRs per lane / waves).
constexpr int kWavesPerEuSmall = 5;  // groups of up to 4 query heads
constexpr int kWavesPerEuLarge = 4;  // groups of 8

constexpr int kMaxWaves = kWavesLargeLds > kWavesSmallLds ? kWavesLargeLds : kWavesSmallLds;
constexpr int kMaxSplits = 1024;      // slot splits per (sequence, KV head)
// Largest split count the team path takes: every split of a team reads the
// (max, sum) words of all the others, so the exchange grows with the square
// of the count; beyond this the combine path finishes the step.
constexpr int kMaxTeamSplits = 64;
// Ticket counters of the team path: a launch uses `ranges` of them (1 to
// kTicketRanges), range r holding pairs [ticket_range_first_pair(pairs, r,
// ranges), ticket_range_first_pair(pairs, r + 1, ranges)).
constexpr int kTicketRanges = 8;
LF_HD inline int ticket_range_first_pair(int pairs, int r, int ranges) {
  return (int)((long long)pairs * r / ranges);
}
// XCDs of an MI355X: a launch's workgroups are dealt to them in turn, in
// block order, and each waits for room on its own XCD.
constexpr int kXcds = 8;
// LDS bytes a workgroup may spend on the logits of its slot range.
constexpr size_t kLogitLdsBudget = (size_t)136 * 1024;

LF_HD inline int padded_group(int g) {
  int p = 1;
  while (p < g) p <<= 1;
  return p;
}

LF_HD inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Slots per split and the number of non-empty splits for a requested count.
LF_HD inline void split_geometry(int S, int nsplit, int* split_len, int* nsplit_eff) {
  int len = (S + nsplit - 1) / nsplit;
  *split_len = len;
  *nsplit_eff = (S + len - 1) / len;
}

// Pairs of a one-split step that the persistent workgroups take longest
// first; a step with more pairs takes them in index order.
constexpr int kOrderMaxPairs = 4096;
// Valid-extent words and the two pair-order buffers of that schedule.
constexpr size_t kOrderRegionBytes = (size_t)3 * kOrderMaxPairs * 4;
// The schedule's words, from queue word kSchedWord on (128 bytes into the
// header, a cache line away from the counters every claim updates): [0]
// the order buffer the next one-split step reads (0 or 1; each such step
// flips it), [1 + buffer] the launch that buffer's order is for,
// pairs << 16 | workgroups (0: none, or every pair alike).
constexpr int kSchedWord = 28;

// Byte offsets inside the caller's workspace.
struct WorkspaceLayout {
  size_t status;    // uint32: LF_DEV_* bits
  size_t queue;     // uint32 [3]: [0] single-split work-item counter, [1] finished-workgroup
                    // count, [2] team launch's claimed-workgroup count (all zero
                    // between launches: each launch's last workgroup resets them);
                    // then, at word kSchedWord, the one-split schedule's words
                    // (see kSchedWord)
  size_t order;     // uint32 [3][kOrderMaxPairs]: one past the last valid slot of each
                    // pair at its latest step, then two buffers of the pair indices
                    // that the work-item counter hands out, longest first; written by
                    // one-split steps only
  size_t part_ml;   // float [pairs][nsplit][GP][2]: split max and sum of exp2
  size_t part_o;    // float [pairs][nsplit][GP][d]: split output accumulators
  size_t logit;     // float [pairs][S][GP]: log2-domain logits
  size_t vnorm;     // float [pairs][S]: |v|_1 per slot
  size_t cand;      // uint64 [pairs][combine chunks]: per-chunk (score, slot) minima
  size_t ffree;     // uint32 [pairs][combine chunks]: per-chunk lowest free slot (fill step)
  size_t team;      // team exchange region (see TeamLayout)
  size_t total;
};

// Exchange region of the team path.  Every word is a 64-bit (ready bit,
// 32-bit payload) pair written once per step, so the region is zeroed before
// each team launch; the counters (one per pair, then the ticket counters)
// come last.
LF_HD inline size_t team_region_bytes(size_t pairs, int nsplit_eff, int gp, int d) {
  return pairs * nsplit_eff * ((size_t)gp * 2 + 3 + (size_t)gp * d) * 8 + pairs * 4 + kTicketRanges * 4;
}

// Slots per workgroup of the split combine.
constexpr int kCombineSlots = 2048;
LF_HD inline int combine_chunks(int S) { return (S + kCombineSlots - 1) / kCombineSlots; }

// The status word and the work-item counters first, then the one-split
// schedule, then (several splits) the team exchange region and the combine
// path's arrays: a team-path step touches only the first
// team_workspace_bytes of the workspace.  The schedule region has the same
// place and size for every shape, so what one-split steps leave there never
// lies under another step's team words, whatever shapes share the workspace.
LF_HD inline WorkspaceLayout workspace_layout(int B, int Hkv, int d, int S, int gp, int nsplit_eff) {
  WorkspaceLayout w{};
  const size_t pairs = (size_t)B * (size_t)Hkv;
  w.status = 0;
  w.queue = 16;
  w.order = 256;
  size_t off = 256 + kOrderRegionBytes;
  if (nsplit_eff > 1) {
    w.team = off;
    off = align_up(off + team_region_bytes(pairs, nsplit_eff, gp, d), 256);
    w.part_ml = off;
    off = align_up(off + pairs * nsplit_eff * gp * 2 * 4, 256);
    w.part_o = off;
    off = align_up(off + pairs * nsplit_eff * gp * (size_t)d * 4, 256);
    w.logit = off;
    off = align_up(off + pairs * (size_t)S * gp * 4, 256);
    w.vnorm = off;
    off = align_up(off + pairs * (size_t)S * 4, 256);
    w.cand = off;
    off = align_up(off + pairs * (size_t)combine_chunks(S) * 8, 256);
    w.ffree = off;
    off = align_up(off + pairs * (size_t)combine_chunks(S) * 4, 256);
  } else {
    w.part_ml = w.part_o = w.logit = w.vnorm = w.cand = w.ffree = w.team = off;
  }
  w.total = off;
  return w;
}

// Bytes of the workspace a step touches on the team path (up to the end of
// the team region), or with one split and no schedule (header only).
LF_HD inline size_t team_workspace_bytes(int B, int Hkv, int d, int gp, int nsplit_eff) {
  if (nsplit_eff < 2) return 256;
  return align_up(256 + kOrderRegionBytes + team_region_bytes((size_t)B * (size_t)Hkv, nsplit_eff, gp, d), 256);
}

// Words of the team region, in this order: published split (max, sum) per
// head, published split results (minimum candidate high and low words, lowest
// free slot), published split O accumulators, the arrival counters, and the
// ticket counters that hand out (pair, split) work items.
struct TeamLayout {
  size_t xstat;   // uint64 [pairs][nsplit][GP][2]
  size_t xfin;    // uint64 [pairs][nsplit][3]
  size_t xo;      // uint64 [pairs][nsplit][GP][d]
  size_t xcnt;    // uint32 [pairs]
  size_t xticket; // uint32 [kTicketRanges]
  size_t zero_words;  // uint32 words of the whole region
};

LF_HD inline TeamLayout team_layout(const WorkspaceLayout& w, int B, int Hkv, int d, int gp, int nsplit_eff) {
  TeamLayout t{};
  const size_t pairs = (size_t)B * (size_t)Hkv;
  const size_t per = pairs * nsplit_eff;
  t.xstat = w.team;
  t.xfin = t.xstat + per * gp * 2 * 8;
  t.xo = t.xfin + per * 3 * 8;
  t.xcnt = t.xo + per * gp * (size_t)d * 8;
  t.xticket = t.xcnt + pairs * 4;
  t.zero_words = team_region_bytes(pairs, nsplit_eff, gp, d) / 4;
  return t;
}

// LDS layout of one workgroup, in bytes from the start of dynamic LDS.
struct LdsLayout {
  size_t logits;  // float [split_len + kRowPad][GP]; reused for the cross-wave O reduction
  size_t mask;    // uint8 [split_len + kRowPad], zero past the split
  size_t vnorm;   // team: float [split_len + kRowPad], |v|_1 per row (empty otherwise)
  size_t scratch; // reductions and broadcast values
  size_t total;
};

constexpr size_t kScratchBytes = 1024;
// Offsets in the scratch area of the work-item ticket, of the counter that
// hands phase-K batches to the waves and of the pair a ticket stands for;
// the decode body's reductions use the bytes below them.
constexpr size_t kTicketSlot = kScratchBytes - 16;
constexpr size_t kBatchSlot = kScratchBytes - 12;
constexpr size_t kPairSlot = kScratchBytes - 8;
// Rows past the end of a split that a wave batch may touch (a batch is 16
// rows at d = 128, 32 at d = 64, and the last one may run past the split by
// all but one of its rows); the mask and logit arrays are padded by this
// much so those accesses need no bounds check.
constexpr int kRowPad = 32;

// LDS a workgroup may use so that two of them share a compute unit.
constexpr size_t kHalfLdsBytes = 80 * 1024;

LF_HD inline LdsLayout lds_layout(int d, int gp, int split_len, int nw, bool team = false) {
  LdsLayout l{};
  size_t logits = align_up((size_t)(split_len + kRowPad) * gp * 4, 16);
  size_t ored = (size_t)nw * gp * d * 4;
  l.logits = 0;
  size_t off = logits > ored ? logits : ored;
  l.mask = off;
  off = align_up(off + split_len + kRowPad, 16);
  l.vnorm = off;
  if (team) off = align_up(off + (size_t)(split_len + kRowPad) * 4, 16);
  l.scratch = off;
  l.total = off + kScratchBytes;
  return l;
}

// Wavefronts per decode workgroup for a split: a workgroup whose logits
// leave room for a second one on the CU gets fewer waves, so that two of
// them (which reach their barriers independently) share the CU.
LF_HD inline int decode_waves(int gp, int split_len, bool team = false) {
  const size_t rows = (size_t)(split_len + kRowPad);
  return rows * gp * 4 + rows + kScratchBytes + (team ? rows * 4 : 0) > kHalfLdsBytes ? kWavesLargeLds
                                                                                      : kWavesSmallLds;
}

// LDS of one compute unit on gfx950; a workgroup may use all of it.
constexpr size_t kMaxLdsBytes = 160 * 1024;

// Longest split whose logits fit the budget and whose whole LDS layout fits
// the compute unit (on the team path, with its |v|_1 row as well).
LF_HD inline int max_split_len(int d, int gp, bool team = false) {
  int len = (int)(kLogitLdsBudget / ((size_t)gp * 4));
  while (len > 0 && lds_layout(d, gp, len, kMaxWaves, team).total > kMaxLdsBytes) len -= 64;
  return len;
}

}  // namespace lf
