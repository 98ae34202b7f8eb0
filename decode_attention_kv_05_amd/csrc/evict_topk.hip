// Several-slot eviction for gfx950: for every (sequence b, KV head j) the k
// valid slots that come first in (score, slot) order, written in ascending
// slot order into a [k][B][Hkv] list.
//
// Source: "LongFlow: Efficient KV Cache Compression for Reasoning Models"
// (arXiv 2603.11504), Figure 2 caption (Left panel: the score decides which
// cache slot the coming token overwrites); several slots at once serve a
// periodic compression cadence.
//
// Each score becomes a 32-bit key whose unsigned order is the order of the
// values (-0 folded onto +0, every NaN one key above +inf); masked slots get
// the key 0xffffffff and are never chosen.  Equal keys are resolved by slot
// index throughout, so the result is unique and equals the single-slot
// eviction rule for k = 1.
//
// One 256-thread workgroup per (b, j) row:
//   keys    scores and mask bytes are loaded eight per thread at a time, all
//           issued before any is used; rows of up to kStageSlots slots keep
//           their keys in LDS, longer rows re-read them from memory.
//   select  three radix passes over 11, 11 and 10 key bits (LDS histogram,
//           block prefix sum) find the key T of the k-th smallest valid slot
//           and how many slots with key T are still needed ("need").  Scores
//           cluster in a few exponents, so an 8-bit top digit would send most
//           atomics of the first pass to a handful of bins.
//   compact each wave owns a contiguous, 64-aligned run of slots: a counting
//           pass gives every wave its output offset (one barrier), then each
//           wave places its slots with key < T, and the first `need` slots
//           with key T overall, from wave ballots in slot order.
// Workgroups of one sequence's KV heads are placed on one XCD, so the mask
// row they share is fetched from HBM once.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace lf {

constexpr int kTopkThreads = 256;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTopkBatch = 8;       // slots loaded per thread before use
constexpr int kStageSlots = 16384;  // keys staged in LDS (64 KB) up to this row length
constexpr uint32_t kInvalidKey = 0xffffffffu;
constexpr int kRadixPasses = 3;
constexpr int kBinsMax = 2048;  // 11-bit digits
__host__ __device__ constexpr int radix_bits(int pass) { return pass < 2 ? 11 : 10; }
__host__ __device__ constexpr int radix_shift(int pass) { return pass == 0 ? 21 : pass == 1 ? 10 : 0; }

__device__ __forceinline__ uint32_t value_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;  // -0 ranks with +0
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (u & 0x7fffffffu) > 0x7f800000u ? 0xfffffffeu : k;  // NaN, above +inf
}

// Keys of slots base + u * kTopkThreads + tid, u < kTopkBatch (invalid past S).
// Every load is issued (at a clamped slot) before any key is formed.
__device__ __forceinline__ void load_keys(const float* srow, const uint8_t* mrow, int S, int base,
                                          uint32_t (&key)[kTopkBatch]) {
  float sv[kTopkBatch];
  uint8_t mv[kTopkBatch];
#pragma unroll
  for (int u = 0; u < kTopkBatch; ++u) {
    const int i = min(base + u * kTopkThreads + (int)threadIdx.x, S - 1);
    sv[u] = srow[i];
    mv[u] = mrow[i];
  }
#pragma unroll
  for (int u = 0; u < kTopkBatch; ++u) {
    const int i = base + u * kTopkThreads + (int)threadIdx.x;
    key[u] = (i < S && mv[u] != 0) ? value_key(sv[u]) : kInvalidKey;
  }
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
  __shared__ uint32_t hist[kBinsMax];
  __shared__ uint32_t wtot[kTopkWaves];
  __shared__ uint32_t wcount[2][kTopkWaves];
  __shared__ uint32_t pick[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  // The KV heads of a sequence are consecutive rows; give each XCD a
  // contiguous run of rows (workgroups are dispatched round-robin over 8).
  const int nblk = gridDim.x;
  const int xcd = blockIdx.x & 7;
  const int per = nblk >> 3, rem = nblk & 7;
  const int pair = xcd * per + (xcd < rem ? xcd : rem) + (blockIdx.x >> 3);
  const int b = pair / p.Hkv;
  const int S = p.S;
  const float* srow = p.scores + (size_t)pair * S;
  const uint8_t* mrow = p.mask + (size_t)b * S;

  // ---- keys, valid count and the histogram of the top 11 bits
  for (int i = tid; i < kBinsMax; i += kTopkThreads) hist[i] = 0;
  __syncthreads();
  uint32_t nvalid = 0;
  for (int base = 0; base < S; base += kTopkBatch * kTopkThreads) {
    uint32_t key[kTopkBatch];
    load_keys(srow, mrow, S, base, key);
#pragma unroll
    for (int u = 0; u < kTopkBatch; ++u) {
      const int i = base + u * kTopkThreads + tid;
      if (STAGE && i < S) keys[i] = key[u];
      if (key[u] != kInvalidKey) {
        ++nvalid;
        atomicAdd(&hist[key[u] >> radix_shift(0)], 1u);
      }
    }
  }
  uint32_t dummy;
  nvalid = block_exclusive(nvalid, wtot, dummy);  // its barriers also publish keys and histogram

  uint32_t T = 0xfffffffeu;  // fewer than k valid slots: every valid key is <= T
  uint32_t need = (uint32_t)p.k;
  if (nvalid > (uint32_t)p.k) {
    uint32_t prefix = 0, krem = (uint32_t)p.k;
    for (int pass = 0; pass < kRadixPasses; ++pass) {
      const int shift = radix_shift(pass);
      const int nb = 1 << radix_bits(pass);
      if (pass > 0) {
        for (int i = tid; i < kBinsMax; i += kTopkThreads) hist[i] = 0;
        __syncthreads();
        const uint32_t hi_mask = ~0u << (shift + radix_bits(pass));
        const uint32_t dmask = (uint32_t)nb - 1u;
        if (STAGE) {
          // eight LDS reads in flight before the first update
          for (int base = 0; base < S; base += kTopkBatch * kTopkThreads) {
            uint32_t key[kTopkBatch];
#pragma unroll
            for (int u = 0; u < kTopkBatch; ++u) {
              const int i = base + u * kTopkThreads + tid;
              key[u] = i < S ? keys[i] : kInvalidKey;
            }
#pragma unroll
            for (int u = 0; u < kTopkBatch; ++u)
              if (key[u] != kInvalidKey && (key[u] & hi_mask) == prefix)
                atomicAdd(&hist[(key[u] >> shift) & dmask], 1u);
          }
        } else {
          for (int base = 0; base < S; base += kTopkBatch * kTopkThreads) {
            uint32_t key[kTopkBatch];
            load_keys(srow, mrow, S, base, key);
#pragma unroll
            for (int u = 0; u < kTopkBatch; ++u)
              if (key[u] != kInvalidKey && (key[u] & hi_mask) == prefix)
                atomicAdd(&hist[(key[u] >> shift) & dmask], 1u);
          }
        }
        __syncthreads();
      }
      // the digit whose bin holds the krem-th smallest of the remaining keys:
      // thread t owns nb / 256 consecutive bins
      const int per = nb / kTopkThreads;
      uint32_t h[kBinsMax / kTopkThreads];
      uint32_t mine = 0;
#pragma unroll
      for (int q = 0; q < kBinsMax / kTopkThreads; ++q) {
        h[q] = q < per ? hist[tid * per + q] : 0u;
        mine += h[q];
      }
      uint32_t excl;
      block_exclusive(mine, wtot, excl);
#pragma unroll
      for (int q = 0; q < kBinsMax / kTopkThreads; ++q) {
        if (q < per && excl < krem && krem <= excl + h[q]) {
          pick[0] = (uint32_t)(tid * per + q);
          pick[1] = krem - excl;
        }
        if (q < per) excl += h[q];
      }
      __syncthreads();
      prefix |= pick[0] << shift;
      krem = pick[1];
      __syncthreads();  // pick and hist are rewritten by the next pass
    }
    T = prefix;
    need = krem;
  }

  // ---- compaction: wave w owns slots [lo, hi), a 64-aligned quarter of the row
  const int span = (S + kTopkWaves * 64 - 1) / (kTopkWaves * 64) * 64;
  const int lo = wave * span;
  const int hi = min(S, lo + span);
  const uint64_t below = (1ull << lane) - 1ull;
  auto key_at = [&](int i) -> uint32_t {
    if (i >= hi) return kInvalidKey;
    if (STAGE) return keys[i];
    const float sv = srow[i];
    const uint8_t mv = mrow[i];
    return mv != 0 ? value_key(sv) : kInvalidKey;
  };
  constexpr int C = 4;  // 64-slot chunks whose keys are read before use
  uint32_t n_lt = 0, n_eq = 0;
  for (int c0 = lo; c0 < hi; c0 += C * 64) {
    uint32_t key[C];
#pragma unroll
    for (int u = 0; u < C; ++u) key[u] = key_at(c0 + u * 64 + lane);
#pragma unroll
    for (int u = 0; u < C; ++u) {
      n_lt += (uint32_t)__popcll(__ballot(key[u] < T));
      n_eq += (uint32_t)__popcll(__ballot(key[u] == T));
    }
  }
  if (lane == 0) {
    wcount[0][wave] = n_lt;
    wcount[1][wave] = n_eq;
  }
  __syncthreads();
  uint32_t lt_before = 0, eq_before = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    lt_before += w < wave ? wcount[0][w] : 0u;
    eq_before += w < wave ? wcount[1][w] : 0u;
  }
  uint32_t base_eq = eq_before;
  uint32_t base_sel = lt_before + min(eq_before, need);
  int32_t* out = p.out;
  const size_t stride = (size_t)p.pairs;
  for (int c0 = lo; c0 < hi; c0 += C * 64) {
    uint32_t key[C];
#pragma unroll
    for (int u = 0; u < C; ++u) key[u] = key_at(c0 + u * 64 + lane);
#pragma unroll
    for (int u = 0; u < C; ++u) {
      const int i = c0 + u * 64 + lane;
      const bool lt = key[u] < T;
      const bool eq = key[u] == T;
      const uint64_t beq = __ballot(eq);
      const uint32_t eq_rank = base_eq + (uint32_t)__popcll(beq & below);
      const bool sel = lt || (eq && eq_rank < need);
      const uint64_t bsel = __ballot(sel);
      if (sel) out[(size_t)(base_sel + (uint32_t)__popcll(bsel & below)) * stride + pair] = i;
      base_eq += (uint32_t)__popcll(beq);
      base_sel += (uint32_t)__popcll(bsel);
    }
  }
  // the last wave ends with the row's total; it pads the list
  if (wave == kTopkWaves - 1)
    for (uint32_t pos = base_sel + lane; pos < (uint32_t)p.k; pos += 64) out[(size_t)pos * stride + pair] = -1;
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
