/*
 * longflow_stack.h -- C ABI of the multi-layer decode step of liblongflow.so:
 * the LongFlow operator (include/longflow.h) inside the attention module of
 * a Qwen3-8B-shaped model, for AMD Instinct MI355X (gfx950).
 *
 * Source: "LongFlow: Efficient KV Cache Compression for Reasoning Models"
 * (arXiv 2603.11504).  Figure 1 caption: the attention module of Qwen3-8B
 * at decode (batch 128, length 3200), one eviction per attention call.
 * Figure 2 caption: one fused operator per attention call.  The layers
 * around the operator are not described on the pages; they are the ordinary
 * ones of such a module (normalisation and MLP are outside it).
 *
 * One step, for every layer l = 0 .. L-1 in order (x_0 = x_in, x_L = x_out):
 *   1. qkv = x_l W_qkv[l]^T       bf16 [B][(Hq + 2 Hkv) d], fp32 accumulation
 *   2. q, k_new = RoPE of qkv's q and k heads at pos; v_new = qkv's v heads.
 *      RoPE rotates the pairs (i, i + d/2), i < d/2, of every head by the
 *      angle pos[b] * rope_base^(-2i/d) (angle in fp64, rotation in fp32).
 *   3. the step of longflow_decode on (q, k_new, v_new) with layer l's cache
 *      and mask and slot[l] as prev_slot; slot[l] then receives the evicted
 *      slot, i.e. the prev_slot of the next step (read before written, so
 *      one array serves both).
 *   4. x_{l+1} = x_l + O W_o[l]^T  bf16 [B][H], fp32 accumulation; O is the
 *      query heads' outputs laid end to end, [B][Hq d].
 * Then, if advance_pos is nonzero, pos[b] += 1 for every sequence.
 *
 * Layouts (row-major, contiguous, device memory; bf16 as raw 16-bit words):
 *   x_in, x_out  bf16  [B][H]               x_out must not overlap x_in
 *   pos          int32 [B]                  token position of each sequence
 *   w_qkv[l]     bf16  [(Hq + 2 Hkv) d][H]  row n = output feature n: the Hq
 *                                           query heads, then Hkv key heads,
 *                                           then Hkv value heads, d each
 *   w_o[l]       bf16  [H][Hq d]
 *   k_cache[l], v_cache[l], mask[l]          as in longflow_decode
 *   slot[l]      int32 [B][Hkv]             in: previous choice (-1 = none);
 *                                           out: this step's evicted slot
 *   scores[l]    fp32  [B][Hkv][S] or NULL  NULL: kept in the workspace and
 *                                           overwritten by the next layer
 * The per-layer arguments are host arrays of L device pointers, read during
 * the call only.  Layers may share read-only buffers (weights, masks).
 * Sizes: L >= 1, 1 <= B <= 256, H >= 256 with H % 256 == 0, Hq d % 256 == 0;
 * Hq, Hkv, d, S as for longflow_decode.  Alignment: 16 bytes for bf16 arrays, 4 bytes for
 * pos, slot and scores, 256 bytes for the workspace.
 * nsplit: slot splits of the decode step; 0 = lf_plan_nsplit's count for the
 * current device.  The workspace must hold lf_stack_workspace_size(...,
 * nsplit, ...) bytes for the count used.  Its first bytes are the decode
 * step's workspace, so lf_read_device_status works on it unchanged.
 *
 * Ownership, asynchrony and errors follow include/longflow.h: host checks
 * return a negative lf_status before anything is enqueued (a buffer the step
 * writes that overlaps any other buffer gives LF_E_ALIAS); no call allocates
 * device memory or synchronises.
 */
#ifndef LONGFLOW_STACK_H
#define LONGFLOW_STACK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Host-only workspace size for an explicit split count (>= 1). */
int lf_stack_workspace_size(int L, int B, int H, int Hq, int Hkv, int d, int S, int nsplit,
                            size_t* bytes);

/* Where a step leaves the intermediates of its last layer inside the
 * workspace (sized by lf_stack_workspace_size for the same sizes and split
 * count; nsplit >= 1): byte offsets from the workspace start of
 *   offsets[0]  q after RoPE          bf16 [B][Hq][d]
 *   offsets[1]  k_new after RoPE      bf16 [B][Hkv][d]
 *   offsets[2]  v_new                 bf16 [B][Hkv][d]
 *   offsets[3]  O, the operator's output, laid end to end  bf16 [B][Hq d]
 * They hold the last layer's values from the end of a step until the next
 * step on that workspace, so a step of one layer (L = 1) exposes every stage
 * of that layer for inspection.  Host-only. */
int lf_stack_workspace_offsets(int B, int H, int Hq, int Hkv, int d, int S, int nsplit,
                               size_t* offsets);

/* One decode step through all L layers, enqueued on `stream`. */
int longflow_stack_step(int L, int B, int H, int Hq, int Hkv, int d, int S, float scale,
                        float rope_base, const void* x_in, void* x_out, int32_t* pos,
                        int advance_pos, const void* const* w_qkv, const void* const* w_o,
                        void* const* k_cache, void* const* v_cache, const uint8_t* const* mask,
                        int32_t* const* slot, float* const* scores, void* workspace,
                        size_t workspace_bytes, int nsplit, void* stream);

/* The same step recorded once into a HIP graph (every launch of every layer)
 * for replay with lf_graph_launch.  The graph keeps the pointers it was made
 * with: to run the next step, write the new token's activations into the same
 * x_in and launch it again (slot[l] and, with advance_pos, pos move on inside
 * the graph).  *graph receives an opaque handle that the caller owns and
 * releases with lf_graph_destroy; creating it allocates host-side graph
 * objects only.  Made and checked like longflow_stack_step (nsplit 0 is
 * resolved at creation). */
int lf_stack_graph_create(int L, int B, int H, int Hq, int Hkv, int d, int S, float scale,
                          float rope_base, const void* x_in, void* x_out, int32_t* pos,
                          int advance_pos, const void* const* w_qkv, const void* const* w_o,
                          void* const* k_cache, void* const* v_cache, const uint8_t* const* mask,
                          int32_t* const* slot, float* const* scores, void* workspace,
                          size_t workspace_bytes, int nsplit, void** graph);

/* Enqueue one replay of a graph on `stream`. */
int lf_graph_launch(void* graph, void* stream);

/* Release a graph handle (after the work it launched has finished). */
int lf_graph_destroy(void* graph);

#ifdef __cplusplus
}
#endif

#endif /* LONGFLOW_STACK_H */
