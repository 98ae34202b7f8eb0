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
// Tuning knobs of the decode kernel; the defaults are the shipped choice.
#ifndef LF_WAVES
#define LF_WAVES 8  // wavefronts per workgroup
#endif
#ifndef LF_UNROLL
#define LF_UNROLL 8  // 16-byte row loads per lane per batch (halved for groups of 8)
#endif
#ifndef LF_WAVES_PER_EU
#define LF_WAVES_PER_EU 4  // occupancy hint given to the register allocator
#endif

constexpr int kWaves = LF_WAVES;      // wavefronts per workgroup
constexpr int kThreads = kWaves * 64; // threads per workgroup
constexpr int kMaxSplits = 1024;      // slot splits per (sequence, KV head)
// LDS bytes a workgroup may spend on the logits of its slot range.
constexpr size_t kLogitLdsBudget = 56 * 1024;

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

// Byte offsets inside the caller's workspace.
struct WorkspaceLayout {
  size_t status;    // uint32: LF_DEV_* bits
  size_t part_ml;   // float [pairs][nsplit][GP][2]: split max and sum of exp2
  size_t part_o;    // float [pairs][nsplit][GP][d]: split output accumulators
  size_t logit;     // float [pairs][S][GP]: log2-domain logits
  size_t vnorm;     // float [pairs][S]: |v|_1 per slot
  size_t total;
};

LF_HD inline WorkspaceLayout workspace_layout(int B, int Hkv, int d, int S, int gp, int nsplit_eff) {
  WorkspaceLayout w{};
  const size_t pairs = (size_t)B * (size_t)Hkv;
  size_t off = 256;
  w.status = 0;
  if (nsplit_eff > 1) {
    w.part_ml = off;
    off = align_up(off + pairs * nsplit_eff * gp * 2 * 4, 256);
    w.part_o = off;
    off = align_up(off + pairs * nsplit_eff * gp * (size_t)d * 4, 256);
    w.logit = off;
    off = align_up(off + pairs * (size_t)S * gp * 4, 256);
    w.vnorm = off;
    off = align_up(off + pairs * (size_t)S * 4, 256);
  } else {
    w.part_ml = w.part_o = w.logit = w.vnorm = off;
  }
  w.total = off;
  return w;
}

// LDS layout of one workgroup, in bytes from the start of dynamic LDS.
struct LdsLayout {
  size_t logits;  // float [split_len + kRowPad][GP]; reused for the cross-wave O reduction
  size_t mask;    // uint8 [split_len + kRowPad], zero past the split
  size_t scratch; // reductions and broadcast values
  size_t total;
};

constexpr size_t kScratchBytes = 1024;
// Rows past the end of a split that a wave batch may touch; the mask and
// logit arrays are padded by this much so those reads need no bounds check.
constexpr int kRowPad = 128;

LF_HD inline LdsLayout lds_layout(int d, int gp, int split_len) {
  LdsLayout l{};
  size_t logits = align_up((size_t)(split_len + kRowPad) * gp * 4, 16);
  size_t ored = (size_t)kWaves * gp * d * 4;
  l.logits = 0;
  size_t off = logits > ored ? logits : ored;
  l.mask = off;
  off = align_up(off + split_len + kRowPad, 16);
  l.scratch = off;
  l.total = off + kScratchBytes;
  return l;
}

}  // namespace lf
