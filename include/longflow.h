/*
 * longflow.h -- C ABI of liblongflow.so, LongFlow's fused decode operator for
 * AMD Instinct MI355X (gfx950).
 *
 * Source: "LongFlow: Efficient KV Cache Compression for Reasoning Models"
 * (arXiv 2603.11504).  The abstract describes one operator that fuses
 * attention, importance estimation and token eviction; the Figure 2 caption
 * gives its data flow:
 *   Left   the current token's K/V overwrite the slot chosen at the previous
 *          step; the static KV cache, the mask and the query then yield the
 *          attention output and the slot to overwrite at the next step;
 *   Middle K/V and mask are streamed from HBM into on-chip memory by block;
 *   Right  the product of P and V is split in two steps, an intermediate G and
 *          then O, and the importance score (LongFlowScore) comes from G.
 *
 * What the operator computes (the pages leave the exact form of G and of the
 * score open; this library fixes it as follows):
 *   for every sequence b and KV head j, with G = Hq / Hkv query heads
 *   h = j*G .. j*G+G-1 sharing KV head j and V_b = { i : mask[b][i] != 0 }:
 *     1. if prev_slot[b][j] != -1:  K[b][j][prev] = new_k[b][j],
 *                                   V[b][j][prev] = new_v[b][j]
 *     2. s[h][i] = scale * <q[b][h], K[b][j][i]>           for i in V_b
 *     3. p[h][i] = softmax over V_b of s[h][.]
 *     4. G[h][i] = p[h][i] * V[b][j][i]     (never materialised: the L1 norm
 *                                             of p*v is p * |v|_1 since p >= 0)
 *     5. out[b][h] = sum_i G[h][i]
 *     6. scores[b][j][i] = sum_h |G[h][i]|_1 for i in V_b, +inf otherwise
 *     7. evict_slot[b][j] = lowest i in V_b with minimum score; -1 if V_b is
 *        empty (then out = 0 and every score is +inf)
 *   The slot written in step 1 is part of the same step's attention.
 *
 * Data types and layouts (all row-major, contiguous, device memory):
 *   bf16 tensors are passed as raw 16-bit patterns (uint16_t / void*).
 *   q          bf16  [B][Hq][d]
 *   k_cache    bf16  [B][Hkv][S][d]   read, one row per (b, j) overwritten
 *   v_cache    bf16  [B][Hkv][S][d]   read, one row per (b, j) overwritten
 *   mask       uint8 [B][S]           nonzero = valid slot; shared by the KV heads
 *   new_k      bf16  [B][Hkv][d]
 *   new_v      bf16  [B][Hkv][d]
 *   prev_slot  int32 [B][Hkv]         -1 = nothing to write
 *   out        bf16  [B][Hq][d]       written (fp32 accumulate, round to nearest even)
 *   scores     fp32  [B][Hkv][S]      written
 *   evict_slot int32 [B][Hkv]         written
 * Supported shapes: B >= 0 (B = 0 is a no-op), Hq >= 1, Hkv >= 1,
 * Hq % Hkv == 0, 1 <= Hq / Hkv <= 8, d in {64, 128}, S >= 1.
 * Alignment: q, k_cache, v_cache, new_k, new_v, out on 16 bytes; scores,
 * prev_slot, evict_slot on 4 bytes; workspace on 256 bytes.
 *
 * Ownership and concurrency: the caller owns every buffer; the library keeps
 * no pointer after a call returns and holds no global state besides a cached
 * per-device compute-unit count.  Compute calls are asynchronous: they
 * enqueue work on `stream` (a hipStream_t; NULL = the default stream) and
 * return; results are valid once the stream has reached that point.  No call
 * synchronises, allocates device memory or copies to the host except
 * lf_read_device_status.  Two calls that share a workspace must be ordered on
 * one stream.
 *
 * Workspace: zero-filled before its first use (lf_workspace_init, or any
 * zeroing of the memory).  It holds the device status word, the work-item
 * counters of the one-split step and the team path's exchange words, which
 * every completed call leaves at zero for the next, and the one-split step's
 * pair schedule: each such step with more (sequence, KV head) pairs than
 * the device holds workgroups at once (and at most 4096 of them) records
 * every pair's valid extent there, and the next one of the same pair count
 * hands out its pairs longest first.  The schedule only orders work:
 * results do not depend on it, and any calls that keep their workspace may
 * share it.  Everything else in the workspace is scratch for the duration
 * of a call.  After a step that reports LF_DEV_TEAM_TIMEOUT, zero it again
 * before its next use.
 *
 * Errors: every entry point returns LF_OK (0) or a negative lf_status code
 * from host-side checks made before anything is enqueued; nothing is enqueued
 * on error.  Conditions that depend on device-resident values (prev_slot)
 * cannot be checked on the host without a synchronisation: they are recorded
 * as LF_DEV_* bits in a status word inside the workspace (see
 * lf_read_device_status).  NaN or Inf in valid slots propagate unchecked;
 * the contents of masked slots are never read.
 */
#ifndef LONGFLOW_H
#define LONGFLOW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LF_ABI_VERSION 1

typedef enum lf_status {
  LF_OK = 0,
  LF_E_NULL = -1,       /* a required pointer is NULL                          */
  LF_E_SHAPE = -2,      /* unsupported or inconsistent sizes                   */
  LF_E_ALIGN = -3,      /* a pointer misses its required alignment             */
  LF_E_ALIAS = -4,      /* an output overlaps an input or another output       */
  LF_E_WORKSPACE = -5,  /* workspace too small                                 */
  LF_E_HIP = -6,        /* a HIP runtime call or kernel launch failed          */
  LF_E_NSPLIT = -7,     /* requested slot split count not usable for the shape */
  LF_E_VALUE = -8,      /* non-finite scale                                    */
  LF_E_SCRATCH = -9     /* longflow_decode_noalloc: the step needs more than
                           LF_STATIC_SCRATCH_BYTES of scratch                  */
} lf_status;

/* Device status bits, accumulated in the workspace across calls until cleared. */
#define LF_DEV_BAD_PREV 0x1u     /* prev_slot outside {-1} U [0, S): write skipped */
#define LF_DEV_WRITE_MASKED 0x2u /* prev_slot named a masked slot: written, unused */
#define LF_DEV_FILL_DIVERGED 0x4u /* fill step: the KV heads of a sequence did not all
                                     write the same free slot (see longflow_decode_fill) */
#define LF_DEV_TEAM_TIMEOUT 0x8u  /* team path: a split waited more than 0.2 s for
                                     the other splits of its pair, which happens only
                                     when they were kept from running (another
                                     process holding compute units); that step's
                                     results are unspecified, and the workspace
                                     must be zeroed before its next use */

/* How a step with several slot splits per (b, j) pair is finished. */
#define LF_SPLIT_AUTO 0    /* LF_SPLIT_TEAM for up to 64 splits when the device
                              can hold a team, else LF_SPLIT_COMBINE */
#define LF_SPLIT_COMBINE 1 /* each split writes its logits, |v|_1 and partial
                              softmax statistics to the workspace; a combine and
                              a finalize kernel rescale them to the true softmax */
#define LF_SPLIT_TEAM 2    /* the splits of a pair run together as a team of
                              workgroups, exchange their (max, sum) through the
                              workspace, and score their slots against
                              the pair's softmax with the logits kept on chip
                              (the statistics are read after each split has
                              streamed its whole slot range);
                              the last split of a pair to finish writes O and
                              the evicted slot.  Workgroups take (pair, split)
                              tickets in the order they start, from R ticket
                              ranges, so the step completes whenever one XCD
                              holds more than R * (nsplit - 1) of them at once;
                              the library picks R (8, 4, 2 or 1) from the
                              occupancy query, else takes the combine path */

/* ABI version (LF_ABI_VERSION). */
int lf_version(void);

/* Hash of the source files the library was built from (16 hex digits, or
 * "unknown" for a build that did not record it); never NULL. */
const char* lf_source_hash(void);

/* Static description of an lf_status code; never NULL. */
const char* lf_strerror(int code);

/* Host-only shape check; returns LF_OK or LF_E_SHAPE.  Touches no device. */
int lf_check_shape(int B, int Hq, int Hkv, int d, int S);

/* Host-only choice of the number of slot splits per (sequence, KV head) for
 * a device with `num_cus` compute units.  Writes the count to *nsplit.  A
 * split count of 1 keeps the whole step of a (b, j) pair in one workgroup;
 * larger counts split the slots (flash-decoding), and the partial softmax
 * statistics are rescaled to the true softmax either inside the step (team
 * path) or by a combine kernel (see longflow_decode_ex). */
int lf_plan_nsplit(int B, int Hq, int Hkv, int d, int S, int num_cus, int* nsplit);

/* Workspace size in bytes for a step with `nsplit` slot splits (>= 1), or,
 * with nsplit = 0, for the count lf_plan_nsplit chooses for the current
 * device: the size longflow_decode needs.  Host-only for nsplit >= 1; with
 * nsplit = 0 it reads the current device's compute-unit count (LF_E_HIP
 * when no device is usable). */
int lf_workspace_size(int B, int Hq, int Hkv, int d, int S, int nsplit, size_t* bytes);

/* Compute units of the current HIP device (cached per device). */
int lf_device_num_cus(int* num_cus);

/* Zero the workspace (its status word included) with a fill kernel enqueued
 * on `stream`: before the first use of a workspace that was not allocated
 * zeroed, and to clear recorded LF_DEV_* bits. */
int lf_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* Host-only argument validation, exactly the checks longflow_decode_nsplit
 * makes before enqueuing anything.  Pointers are compared, never dereferenced. */
int lf_validate(int B, int Hq, int Hkv, int d, int S, float scale,
                const void* q, const void* k_cache, const void* v_cache,
                const uint8_t* mask, const void* new_k, const void* new_v,
                const int32_t* prev_slot, const void* out, const float* scores,
                const int32_t* evict_slot, const void* workspace,
                size_t workspace_bytes, int nsplit);

/* One fused decode step (Figure 2, Left panel: write the previous choice,
 * attend, score, choose the next slot), with the split count chosen by
 * lf_plan_nsplit for the current device.  The workspace must hold at least
 * lf_workspace_size(..., 0, &bytes) bytes (the size for that count). */
int longflow_decode(int B, int Hq, int Hkv, int d, int S, float scale,
                    const void* q, void* k_cache, void* v_cache,
                    const uint8_t* mask, const void* new_k, const void* new_v,
                    const int32_t* prev_slot, void* out, float* scores,
                    int32_t* evict_slot, void* workspace, size_t workspace_bytes,
                    void* stream);

/* The same step with an explicit split count (1 <= nsplit <= S). */
int longflow_decode_nsplit(int B, int Hq, int Hkv, int d, int S, float scale,
                           const void* q, void* k_cache, void* v_cache,
                           const uint8_t* mask, const void* new_k, const void* new_v,
                           const int32_t* prev_slot, void* out, float* scores,
                           int32_t* evict_slot, void* workspace, size_t workspace_bytes,
                           int nsplit, void* stream);

/* One decode step of the cache's fill phase: the static cache still has free
 * slots (mask 0), which are used up before anything is evicted.  Same
 * arguments, shapes and workspace as longflow_decode_nsplit, except:
 *   mask       uint8 [B][S]   read and updated in place: the slot written for
 *                             a sequence becomes valid (mask 1)
 *   next_slot  int32 [B][Hkv] the slot for the next step's token: the lowest
 *                             free slot of the updated mask while the
 *                             sequence has one, otherwise the evicted slot
 *                             of longflow_decode
 *   nsplit     0 = the count lf_plan_nsplit chooses for the current device
 * The written slot takes part in the same step's attention whether or not it
 * was free (Figure 2, Left panel: the current token is written, then
 * attended), so a sequence that starts empty with prev_slot = 0 gets plain
 * causal decode attention until its cache is full; after that the step is
 * exactly longflow_decode.  Writing a free slot sets no LF_DEV_WRITE_MASKED.
 * The mask is shared by the KV heads, so while a sequence has free slots all
 * of its KV heads must write the same slot (or none); otherwise
 * LF_DEV_FILL_DIVERGED is set and that sequence's results are unspecified
 * (every access stays in bounds).  The next_slot values this entry point
 * returns always satisfy that rule. */
int longflow_decode_fill(int B, int Hq, int Hkv, int d, int S, float scale,
                         const void* q, void* k_cache, void* v_cache, uint8_t* mask,
                         const void* new_k, const void* new_v, const int32_t* prev_slot,
                         void* out, float* scores, int32_t* next_slot, void* workspace,
                         size_t workspace_bytes, int nsplit, void* stream);

/* The general form of longflow_decode_nsplit and longflow_decode_fill:
 *   fill        0: mask is read only (longflow_decode_nsplit);
 *               1: fill step, mask updated in place (longflow_decode_fill)
 *   nsplit      0 = the count lf_plan_nsplit chooses for the current device
 *   split_path  LF_SPLIT_AUTO, LF_SPLIT_COMBINE or LF_SPLIT_TEAM: how a step
 *               with nsplit > 1 is finished (ignored when nsplit = 1).
 *               LF_SPLIT_TEAM returns LF_E_NSPLIT for more than 64 splits
 *               or when the device cannot hold more than 8 * (nsplit - 1)
 *               of its workgroups at once.
 * Both paths compute the same operator (Figure 2: the split is the
 * flash-decoding form of one attention pass; abstract: attention, scoring and
 * eviction fused in one operator).  The team path reads K and V once and
 * keeps the logits on chip; the scores are those of the combine path, O may
 * differ by rounding.  A team's splits wait for each other mid-step (at
 * most 0.2 s, else LF_DEV_TEAM_TIMEOUT); where another process may hold
 * compute units for that long, use LF_SPLIT_COMBINE.  Same workspace size as
 * longflow_decode_nsplit. */
int longflow_decode_ex(int B, int Hq, int Hkv, int d, int S, float scale,
                       const void* q, void* k_cache, void* v_cache, uint8_t* mask,
                       int fill, const void* new_k, const void* new_v,
                       const int32_t* prev_slot, void* out, float* scores,
                       int32_t* evict_slot, void* workspace, size_t workspace_bytes,
                       int nsplit, int split_path, void* stream);

/* Several slots evicted at once, for a periodic cadence (compress every N
 * steps instead of every step).  For every (b, j): the set of the k valid
 * slots (mask[b][i] != 0) that come first in (score, slot) order, written in
 * ascending slot order; when fewer than k slots are valid the set is all of
 * them and the rest of the list is -1.  Scores compare by value (-0 equals
 * +0, so the slot decides) and NaN comes after every number; with k = 1 this
 * is longflow_decode's eviction rule.
 *   scores       fp32  [B][Hkv][S]  read (typically longflow_decode's output)
 *   mask         uint8 [B][S]       read
 *   evict_slots  int32 [k][B][Hkv]  written; entry t is laid out like a
 *                                   prev_slot array, so `evict_slots + t*B*Hkv`
 *                                   can be passed as prev_slot of the t-th
 *                                   following step (a write queue: the listed
 *                                   slots stay valid and are attended until
 *                                   their turn to be overwritten comes)
 * Sizes: B >= 0 (0 = no-op), Hkv >= 1, S >= 1, 1 <= k <= S.  Alignment:
 * scores and evict_slots on 4 bytes.  evict_slots must not overlap scores or
 * mask.  Asynchronous on `stream`, no workspace, no allocation. */
int longflow_evict_topk(int B, int Hkv, int S, int k, const float* scores,
                        const uint8_t* mask, int32_t* evict_slots, void* stream);

/* Copy the workspace's LF_DEV_* bits to *flags.  Synchronises `stream`. */
int lf_read_device_status(const void* workspace, void* stream, uint32_t* flags);

/* Size of the device array that longflow_decode_noalloc uses as its
 * workspace: 16 MiB, one array per GPU the library runs on, held until the
 * process ends. */
#define LF_STATIC_SCRATCH_BYTES (16u << 20)

/* longflow_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops that
 * may not call hipMalloc, harnesses that forbid allocation.  Same operator,
 * arguments, shapes, plan and results as longflow_decode (the same kernels);
 * the workspace is the library's own LF_STATIC_SCRATCH_BYTES device array,
 * whose header (and, on the team path, exchange region) a fill kernel on
 * `stream` clears at the start of every call; so it keeps no pair schedule
 * between calls (a one-split step takes its pairs in index order).  The
 * call allocates nothing and makes no allocating library call; the array's
 * device address is looked up on the first call on each device.
 * A step that needs more scratch than the array holds returns LF_E_SCRATCH
 * before anything is enqueued: a one-split step needs 256 bytes; a split step
 * on the team path 48.25 KB plus its exchange region (about 8.3 KB per
 * (sequence, KV head) and split at 8 query heads per KV head and d = 128:
 * 4.3 MB for 16 x 8 pairs in 4 splits); a split step that cannot take the
 * team path, its whole combine workspace (lf_workspace_size).
 * All calls on one GPU share the array: calls that overlap in time on one
 * GPU (other streams, other threads of the process) race and give
 * unspecified results; order them on one stream.  The device status bits
 * are not reported (use longflow_decode with a workspace to read them). */
int longflow_decode_noalloc(int B, int Hq, int Hkv, int d, int S, float scale,
                            const void* q, void* k_cache, void* v_cache,
                            const uint8_t* mask, const void* new_k, const void* new_v,
                            const int32_t* prev_slot, void* out, float* scores,
                            int32_t* evict_slot, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LONGFLOW_H */
