// Several-slot eviction for gfx950: for every (sequence b, KV head j) the k
// valid slots that come first in (score, slot) order, written in ascending
// slot order into a [k][B][Hkv] list.
//
// Source: "LongFlow: Efficient KV Cache Compression for Reasoning Models"
// (arXiv 2603.11504), Figure 2 caption (Left panel: the score decides which
// cache slot the coming token overwrites); several slots at once serve a
// periodic compression cadence.
//
// One 256-thread workgroup per (b, j) row:
//   keys    each score becomes a 32-bit key whose unsigned order is the
//           order of the values (-0 folded onto +0, every NaN one key above
//           +inf); masked slots get the key 0xffffffff and are never chosen.
//           Rows of up to kStageSlots slots keep their keys in LDS.
//   select  four 8-bit radix passes (LDS histogram, block prefix sum) find
//           the key T of the k-th smallest valid slot and how many slots with
//           key T are still needed ("need").
//   compact one ordered pass over the row: slots with key < T, plus the
//           first `need` slots with key T, get consecutive positions from
//           wave ballots and a block prefix sum; the list is padded with -1.
// Equal keys are resolved by slot index throughout, so the result is unique
// and equals the ordering rule of the single-slot eviction for k = 1.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace lf {

constexpr int kTopkThreads = 256;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kStageSlots = 16384;  // keys staged in LDS (64 KB) up to this row length
constexpr uint32_t kInvalidKey = 0xffffffffu;

__device__ __forceinline__ uint32_t order_key(float s, bool valid) {
  if (!valid) return kInvalidKey;
  uint32_t u = __float_as_uint(s);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0xfffffffeu;  // NaN, above +inf
  if (u == 0x80000000u) u = 0u;                              // -0 ranks with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Block-wide exclusive prefix of one count per thread; returns the block total.
__device__ __forceinline__ uint32_t block_exclusive(uint32_t x, uint32_t* wtot, uint32_t& excl) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    before += w < wave ? wtot[w] : 0u;
    total += wtot[w];
  }
  __syncthreads();  // wtot may be reused right away
  excl = before + incl - x;
  return total;
}

template <bool STAGE>
__global__ __launch_bounds__(kTopkThreads) void evict_topk_kernel(TopkParams p) {
  extern __shared__ uint32_t keys[];  // [S] when STAGE
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wtot[kTopkWaves];
  __shared__ uint32_t wtot2[kTopkWaves];
  __shared__ uint32_t pick[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int pair = blockIdx.x;
  const int b = pair / p.Hkv;
  const int S = p.S;
  const float* srow = p.scores + (size_t)pair * S;
  const uint8_t* mrow = p.mask + (size_t)b * S;
  auto key_at = [&](int i) -> uint32_t {
    if (STAGE) return keys[i];
    return order_key(srow[i], mrow[i] != 0);
  };

  // ---- keys, valid count and the histogram of the top byte
  hist[tid] = 0;
  __syncthreads();
  uint32_t nvalid = 0;
  for (int i = tid; i < S; i += kTopkThreads) {
    const uint32_t key = order_key(srow[i], mrow[i] != 0);
    if (STAGE) keys[i] = key;
    if (key != kInvalidKey) {
      ++nvalid;
      atomicAdd(&hist[key >> 24], 1u);
    }
  }
  uint32_t dummy;
  nvalid = block_exclusive(nvalid, wtot, dummy);  // also orders the histogram and keys

  uint32_t T = 0xfffffffeu;  // every valid key is <= T
  uint32_t need = (uint32_t)p.k;
  if (nvalid > (uint32_t)p.k) {
    uint32_t prefix = 0, krem = (uint32_t)p.k;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      if (pass > 0) {
        hist[tid] = 0;
        __syncthreads();
        const uint32_t hi_mask = ~0u << (shift + 8);
        for (int i = tid; i < S; i += kTopkThreads) {
          const uint32_t key = key_at(i);
          if (key != kInvalidKey && (key & hi_mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
      }
      // the digit whose bin holds the krem-th smallest of the remaining keys
      const uint32_t h = hist[tid];
      uint32_t excl;
      block_exclusive(h, wtot, excl);
      if (excl < krem && krem <= excl + h) {
        pick[0] = (uint32_t)tid;
        pick[1] = krem - excl;
      }
      __syncthreads();
      prefix |= pick[0] << shift;
      krem = pick[1];
      __syncthreads();  // pick and hist are rewritten by the next pass
    }
    T = prefix;
    need = krem;
  }

  // ---- ordered compaction
  int32_t* out = p.out;
  const size_t stride = (size_t)p.pairs;
  uint32_t base_sel = 0, base_eq = 0;
  for (int c0 = 0; c0 < S; c0 += kTopkThreads) {
    const int i = c0 + tid;
    const uint32_t key = i < S ? key_at(i) : kInvalidKey;
    const bool lt = key < T;
    const bool eq = key == T;
    // ranks among this chunk's equal keys, then among its selected slots
    const uint64_t below = (1ull << lane) - 1ull;
    const uint64_t beq = __ballot(eq);
    if (lane == 0) wtot[wave] = (uint32_t)__popcll(beq);
    __syncthreads();
    uint32_t eq_before = 0, eq_total = 0;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) {
      eq_before += w < wave ? wtot[w] : 0u;
      eq_total += wtot[w];
    }
    const uint32_t eq_rank = base_eq + eq_before + (uint32_t)__popcll(beq & below);
    const bool sel = lt || (eq && eq_rank < need);
    const uint64_t bsel = __ballot(sel);
    if (lane == 0) wtot2[wave] = (uint32_t)__popcll(bsel);
    __syncthreads();
    uint32_t sel_before = 0, sel_total = 0;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) {
      sel_before += w < wave ? wtot2[w] : 0u;
      sel_total += wtot2[w];
    }
    if (sel) {
      const uint32_t pos = base_sel + sel_before + (uint32_t)__popcll(bsel & below);
      out[(size_t)pos * stride + pair] = i;
    }
    base_sel += sel_total;
    base_eq += eq_total;
    __syncthreads();  // wtot and wtot2 are rewritten by the next chunk
  }
  for (uint32_t pos = base_sel + tid; pos < (uint32_t)p.k; pos += kTopkThreads)
    out[(size_t)pos * stride + pair] = -1;
}

hipError_t launch_topk(const TopkParams& prm, hipStream_t stream) {
  if (prm.pairs == 0) return hipSuccess;
  if (prm.S <= kStageSlots) {
    hipLaunchKernelGGL(evict_topk_kernel<true>, dim3(prm.pairs), dim3(kTopkThreads),
                       (size_t)prm.S * 4, stream, prm);
  } else {
    hipLaunchKernelGGL(evict_topk_kernel<false>, dim3(prm.pairs), dim3(kTopkThreads), 0, stream, prm);
  }
  return hipGetLastError();
}

}  // namespace lf
