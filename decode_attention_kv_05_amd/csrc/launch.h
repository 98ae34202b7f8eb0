// Kernel parameter block and launch entry points shared by the host API
// (longflow_api.cpp) and the kernels (longflow_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lf {

struct DecodeParams {
  const uint16_t* q;      // bf16 [B][Hq][d]
  uint16_t* k;            // bf16 [B][Hkv][S][d]
  uint16_t* v;            // bf16 [B][Hkv][S][d]
  const uint8_t* mask;    // [B][S]
  const uint16_t* new_k;  // bf16 [B][Hkv][d]
  const uint16_t* new_v;  // bf16 [B][Hkv][d]
  const int32_t* prev;    // [B][Hkv]
  uint16_t* out;          // bf16 [B][Hq][d]
  float* scores;          // [B][Hkv][S]
  int32_t* evict;         // [B][Hkv]
  uint32_t* status;       // workspace: LF_DEV_* bits
  uint32_t* queue;        // workspace: [3] single-split work-item counter, finished workgroups; team
                          // claims; the schedule's words from word kSchedWord on
  float* part_ml;         // workspace: [pairs][nsplit][GP][2]
  float* part_o;          // workspace: [pairs][nsplit][GP][d]
  float* ws_logit;        // workspace: [pairs][S][GP]
  float* ws_vnorm;        // workspace: [pairs][S]
  uint64_t* cand;         // workspace: [pairs][chunks] packed (score, slot) minima
  uint32_t* ffree;        // workspace: [pairs][chunks] lowest free slot (fill step)
  uint8_t* mask_w;        // fill step: the same mask, updated in place; else null
  uint64_t* xstat;        // team: [pairs][nsplit][GP][2] published (max, sum)
  uint64_t* xfin;         // team: [pairs][nsplit][3] published minimum (high, low word), lowest free slot
  uint64_t* xo;           // team: [pairs][nsplit][GP][d] published O accumulators
  uint32_t* xcnt;         // team: [pairs] splits finished
  uint32_t* xticket;      // team: [kTicketRanges] work items handed out per range (ticket_ranges used)
  uint32_t* lens;         // one split, longest-first schedule: [pairs] one past each pair's last
                          // valid slot; null without the schedule
  uint32_t* order;        // [2][kOrderMaxPairs] pair orders (one read, the other rebuilt)
  int pairs;              // B * Hkv
  int Hq, Hkv, G, S, nsplit, split_len;
  int fill;               // 1: fill step (next slot = lowest free slot while any)
  int ticket_ranges;      // team: ticket ranges in use, 1 .. kTicketRanges
  float qscale;           // logit scale times log2(e)
};

struct TopkParams {
  const float* scores;    // [B][Hkv][S]
  const uint8_t* mask;    // [B][S]
  int32_t* out;           // [k][B][Hkv]
  int Hkv, S, k, pairs;
};

// team_grid > 0: one launch of the team kernel with one workgroup per
// (pair, split), nblocks in all;
// otherwise, with one split, `grid` persistent workgroups of the
// single-split kernel that take the nblocks pairs from the work-item counter,
// or, with several, nblocks workgroups of the split kernel followed by the
// combine and finalize kernels.
hipError_t launch_decode(const DecodeParams& prm, int d, int gp, int nw, int nblocks, size_t lds,
                         int team_grid, int grid, hipStream_t stream);
// Workgroups of the team kernel (team = true) or of the single-split kernel
// for (d, gp, nw, lds) that one compute unit holds at once.
hipError_t decode_blocks_per_cu(bool team, int d, int gp, int nw, size_t lds, int* blocks);

// One decode step after validation (the decode kernel and, for several
// splits, the combine and finalize kernels).  mask_w non-null selects the
// fill step.  evict_slot may equal prev_slot outside the fill step: every
// split reads its pair's prev_slot before the pair's evicted slot is
// written (by the same workgroup at its end, or by the finalize kernel).
// team_only: the workspace holds only what a team-path step touches (a
// split step then takes the team path or fails with LF_E_NSPLIT).
// schedule: a one-split step keeps its longest-first pair order in the
// workspace for the next step (off: pairs in index order, the schedule
// region untouched).
int enqueue_decode_step(int B, int Hq, int Hkv, int d, int S, float scale, const void* q,
                        void* k_cache, void* v_cache, const uint8_t* mask, uint8_t* mask_w,
                        const void* new_k, const void* new_v, const int32_t* prev_slot, void* out,
                        float* scores, int32_t* evict_slot, void* workspace, int nsplit,
                        int split_path, void* stream, bool team_only = false, bool schedule = true);
hipError_t launch_topk(const TopkParams& prm, hipStream_t stream);
hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t value, hipStream_t stream);

}  // namespace lf
