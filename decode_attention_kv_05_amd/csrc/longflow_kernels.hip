// HIP kernels of LongFlow's fused decode step for gfx950 (MI355X).
//
// Source: "LongFlow: Efficient KV Cache Compression for Reasoning Models"
// (arXiv 2603.11504): abstract (one operator fusing attention, importance
// estimation and eviction) and Figure 2 caption (Left: write the previous
// choice, attend, return the next slot; Middle: K/V and mask streamed from HBM
// by block; Right: P.V split into G then O, score from G).
//
// One launch per decode step.  Workgroup (256 threads) = one slot range
// ("split") of one (sequence b, KV head j) pair.
//
//   setup    the split that owns prev_slot copies new_k/new_v into the cache
//            row and reads that row from new_k/new_v for the rest of the step;
//            the mask of the split is staged in LDS.
//   phase K  K rows stream from HBM in 16-byte lane loads (a 256-byte row
//            = 16 lanes).  Each lane dots its 8 columns with the G queries of
//            the group; a DPP reduce-scatter across the 16 lanes leaves one
//            head's full logit per lane group.  Logits (log2 domain: the scale
//            is pre-multiplied by log2 e) go to LDS.
//   softmax  block max M_h and sum L_h of exp2(s - M_h); LDS logits become
//            e = exp2(s - M_h) in place.
//   phase V  V rows stream the same way.  Each lane accumulates e*v for its 8
//            columns and G heads (G = p*v is never stored: only O = sum G and
//            |G|_1 = p*|v|_1 are needed, since p >= 0), and |v|_1 per row.
//   finish   (single split) score_i = |v_i|_1 * sum_h e_hi / L_h is written in
//            phase V, O = acc / L, argmin over (score bits, slot) pairs.
//            (several splits) each split stores its (M, L, acc) partials, the
//            logits and |v|_1; the last split of the pair to finish (atomic
//            counter) rescales the partials to the true softmax, writes O,
//            every score and the evicted slot, and resets the counter.
//
// The per-slot arithmetic is the same instruction sequence for every slot, so
// two slots with identical K/V rows get bit-identical scores and the argmin's
// lowest-index rule decides exact ties.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "launch.h"
#include "layout.h"
#include "longflow.h"

namespace lf {

// ------------------------------------------------------------ lane helpers

__device__ __forceinline__ void bf16x8_to_f32(const uint4& x, float (&f)[8]) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Value of the partner lane for step BIT of a reduction inside a 16-lane DPP
// row.  The partner has the opposite value of lane bit BIT and the same
// value of every higher lane bit, which is all a butterfly needs:
//   8: row_ror:8 (lane ^ 8)        4: row_half_mirror (lane ^ 7)
//   2: quad_perm 2,3,0,1 (lane ^ 2) 1: quad_perm 1,0,3,2 (lane ^ 1)
template <int BIT>
__device__ __forceinline__ float partner(float x) {
  if constexpr (BIT == 8) return dpp_mov<0x128>(x);
  else if constexpr (BIT == 4) return dpp_mov<0x141>(x);
  else if constexpr (BIT == 2) return dpp_mov<0x4E>(x);
  else if constexpr (BIT == 1) return dpp_mov<0xB1>(x);
  else return __shfl_xor(x, BIT);
}

// Reduce-scatter of N per-lane partial sums over the lanes of one row group.
// While N > 1 each step keeps half of the values (upper half if the lane's
// BIT is set) and adds the partner's copy of that half; once one value is
// left the steps are plain butterfly adds.
template <int BIT, int N>
__device__ __forceinline__ void reduce_scatter(float* a, int c) {
  if constexpr (BIT >= 1) {
    if constexpr (N > 1) {
      constexpr int H = N / 2;
      const bool upper = (c & BIT) != 0;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const float send = upper ? a[i] : a[H + i];
        const float keep = upper ? a[H + i] : a[i];
        a[i] = keep + partner<BIT>(send);
      }
      reduce_scatter<BIT / 2, H>(a, c);
    } else {
      a[0] += partner<BIT>(a[0]);
      reduce_scatter<BIT / 2, 1>(a, c);
    }
  }
}

template <int BIT>
__device__ __forceinline__ float allreduce_sum(float x) {
  if constexpr (BIT >= 1) {
    x += partner<BIT>(x);
    return allreduce_sum<BIT / 2>(x);
  } else {
    return x;
  }
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)x, m);
  const uint32_t hi = __shfl_xor((uint32_t)(x >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_min_u64(uint64_t x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const uint64_t y = shfl_xor_u64(x, m);
    x = y < x ? y : x;
  }
  return x;
}

// (score, slot) packed so that unsigned order = score order, then slot order.
// Scores are >= +0, and non-negative IEEE floats order like their bit patterns.
__device__ __forceinline__ uint64_t pack_candidate(float score, int slot) {
  return ((uint64_t)__float_as_uint(score) << 32) | (uint32_t)slot;
}

constexpr uint64_t kNoCandidate = ~0ull;

// ------------------------------------------------------------------ kernel

template <int D, int GP, bool SPLIT>
__global__ __launch_bounds__(kThreads) void longflow_decode_kernel(DecodeParams p) {
  constexpr int LPR = D / 8;                           // lanes per 16-byte-chunked row
  constexpr int RPW = 64 / LPR;                        // rows per wave load
  constexpr int U = 8;                                 // wave loads in flight per batch
  constexpr int ROWS_PER_BATCH = RPW * U;
  constexpr int HPL = GP > LPR ? GP / LPR : 1;         // heads per lane after reduce-scatter
  constexpr int LPH = GP < LPR ? LPR / GP : 1;         // lanes holding each head
  constexpr float kNegInf = -__builtin_huge_valf();
  constexpr float kInf = __builtin_huge_valf();

  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = lane % LPR;   // 16-byte column chunk of the row
  const int rg = lane / LPR;  // row within the wave load

  // Blocks are dispatched round-robin over the 8 XCDs; give each XCD a
  // contiguous run of work items so the splits of a pair share an L2.
  const int nblk = gridDim.x;
  const int xcd = blockIdx.x & 7;
  const int per = nblk >> 3, rem = nblk & 7;
  const int item = xcd * per + (xcd < rem ? xcd : rem) + (blockIdx.x >> 3);

  const int nsplit = SPLIT ? p.nsplit : 1;
  const int pair = item / nsplit;
  const int sp = item - pair * nsplit;
  const int b = pair / p.Hkv;
  const int j = pair - b * p.Hkv;
  const int s0 = sp * p.split_len;
  const int n = min(p.S, s0 + p.split_len) - s0;

  const LdsLayout L = lds_layout(D, GP, p.split_len);
  float* lg = reinterpret_cast<float*>(smem + L.logits);
  uint8_t* mk = smem + L.mask;
  float* red = reinterpret_cast<float*>(smem + L.scratch);  // [kWaves][GP]
  float* stat_m = red + kWaves * GP;                          // [GP]
  float* stat_il = stat_m + GP;                               // [GP] 1 / L
  uint64_t* best_w = reinterpret_cast<uint64_t*>(stat_il + GP);  // [kWaves], 8-byte aligned
  int* flag = reinterpret_cast<int*>(best_w + kWaves);

  const size_t row0 = (size_t)pair * p.S;  // first cache row of this pair
  const uint16_t* kp = p.k + row0 * D;
  const uint16_t* vp = p.v + row0 * D;
  const uint8_t* mrow = p.mask + (size_t)b * p.S;
  const uint16_t* nk = p.new_k + (size_t)pair * D;
  const uint16_t* nv = p.new_v + (size_t)pair * D;

  // ---- setup: slot write (Figure 2, Left panel) and mask staging
  int prev = p.prev[pair];
  int prev_local = -1;  // split-relative row served from new_k/new_v
  if (prev != -1) {
    if (prev < 0 || prev >= p.S) {
      if (sp == 0 && tid == 0) atomicOr(p.status, LF_DEV_BAD_PREV);
    } else if (prev >= s0 && prev < s0 + n) {
      prev_local = prev - s0;
      if (tid < D / 8) {
        const uint4 kx = reinterpret_cast<const uint4*>(nk)[tid];
        const uint4 vx = reinterpret_cast<const uint4*>(nv)[tid];
        reinterpret_cast<uint4*>(p.k + (row0 + prev) * D)[tid] = kx;
        reinterpret_cast<uint4*>(p.v + (row0 + prev) * D)[tid] = vx;
      }
      if (tid == 0 && mrow[prev] == 0) atomicOr(p.status, LF_DEV_WRITE_MASKED);
    }
  }
  {
    const uint8_t* src = mrow + s0;
    for (int base = 0; base < n; base += kThreads * 8) {
      uint8_t t8[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * kThreads + tid;
        t8[u] = i < n ? src[i] : 0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * kThreads + tid;
        if (i < n) mk[i] = t8[u];
      }
    }
  }

  // Queries of the group, pre-scaled into the log2 domain.  Padded heads
  // (h >= G) get q = 0; their results are never stored.
  float qf[GP][8];
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    if (h < p.G) {
      const uint4 x = reinterpret_cast<const uint4*>(
          p.q + ((size_t)b * p.Hq + (size_t)j * p.G + h) * D)[c];
      bf16x8_to_f32(x, qf[h]);
#pragma unroll
      for (int k = 0; k < 8; ++k) qf[h][k] *= p.qscale;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) qf[h][k] = 0.f;
    }
  }
  __syncthreads();

  // ---- phase K: logits into LDS
  const int hbase = GP <= LPR ? c / LPH : c * HPL;
  const bool writer = (c % LPH) == 0;
  float mx[HPL];
#pragma unroll
  for (int i = 0; i < HPL; ++i) mx[i] = kNegInf;

  for (int r0 = wave * ROWS_PER_BATCH; r0 < n; r0 += kWaves * ROWS_PER_BATCH) {
    uint4 kx[U];
    bool ok[U];
    bool any = false;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u * RPW + rg;
      ok[u] = r < n && mk[r] != 0;
      any |= ok[u];
    }
    if (__ballot(any) == 0) {  // every row of this batch is masked or past the end
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = r0 + u * RPW + rg;
        if (writer && r < n) {
#pragma unroll
          for (int i = 0; i < HPL; ++i) lg[r * GP + hbase + i] = kNegInf;
        }
      }
      continue;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u * RPW + rg;
      const uint16_t* src = (r == prev_local) ? nk : kp + (size_t)(s0 + r) * D;
      kx[u] = ok[u] ? reinterpret_cast<const uint4*>(src)[c] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[8];
      bf16x8_to_f32(kx[u], kf);
      float a[GP];
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) s = fmaf(qf[h][k], kf[k], s);
        a[h] = s;
      }
      reduce_scatter<LPR / 2, GP>(a, c);
      const int r = r0 + u * RPW + rg;
      if (writer && r < n) {
#pragma unroll
        for (int i = 0; i < HPL; ++i) {
          const float val = ok[u] ? a[i] : kNegInf;
          lg[r * GP + hbase + i] = val;
          mx[i] = fmaxf(mx[i], val);
        }
      }
    }
  }

  // ---- softmax statistics of this split
  // Lanes with equal c hold the same heads; fold the row groups, then waves.
#pragma unroll
  for (int i = 0; i < HPL; ++i) {
#pragma unroll
    for (int m = LPR; m < 64; m <<= 1) mx[i] = fmaxf(mx[i], __shfl_xor(mx[i], m));
  }
  if (rg == 0 && writer) {
#pragma unroll
    for (int i = 0; i < HPL; ++i) red[wave * GP + hbase + i] = mx[i];
  }
  __syncthreads();
  if (tid < GP) {
    float m = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) m = fmaxf(m, red[w * GP + tid]);
    stat_m[tid] = m;
  }
  __syncthreads();

  {
    // thread -> (head tid % GP, rows tid / GP + k * kThreads / GP):
    // consecutive threads touch consecutive LDS words and workspace floats.
    const int h = tid % GP;
    const float mh = stat_m[h];
    float lsum = 0.f;
    float* wl = SPLIT ? p.ws_logit + (row0 + s0) * GP : nullptr;
    for (int r = tid / GP; r < n; r += kThreads / GP) {
      const float s = lg[r * GP + h];
      const float e = (s == kNegInf) ? 0.f : exp2f(s - mh);
      lg[r * GP + h] = e;
      lsum += e;
      if (SPLIT) wl[r * GP + h] = s;
    }
#pragma unroll
    for (int m = GP; m < 64; m <<= 1) lsum += __shfl_xor(lsum, m);
    __syncthreads();  // every wave is done reading `red` (maxima)
    if (lane < GP) red[wave * GP + lane] = lsum;
    __syncthreads();
    if (tid < GP) {
      float l = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) l += red[w * GP + tid];
      stat_il[tid] = l > 0.f ? 1.0f / l : 0.f;
      if (SPLIT) {
        float* ml = p.part_ml + (((size_t)pair * nsplit + sp) * GP + tid) * 2;
        ml[0] = stat_m[tid];
        ml[1] = l;
      }
    }
    __syncthreads();
  }

  // ---- phase V: O accumulators, |v|_1, and (single split) scores
  float il[GP];
#pragma unroll
  for (int h = 0; h < GP; ++h) il[h] = stat_il[h];
  float acc[GP][8];
#pragma unroll
  for (int h = 0; h < GP; ++h)
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[h][k] = 0.f;
  uint64_t best = kNoCandidate;
  float* score_row = p.scores + row0 + s0;
  float* vn_row = SPLIT ? p.ws_vnorm + row0 + s0 : nullptr;

  for (int r0 = wave * ROWS_PER_BATCH; r0 < n; r0 += kWaves * ROWS_PER_BATCH) {
    uint4 vx[U];
    bool ok[U];
    bool any = false;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u * RPW + rg;
      ok[u] = r < n && mk[r] != 0;
      any |= ok[u];
    }
    if (__ballot(any) == 0) {
      if (!SPLIT) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int r = r0 + u * RPW + rg;
          if (c == 0 && r < n) score_row[r] = kInf;
        }
      }
      continue;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u * RPW + rg;
      const uint16_t* src = (r == prev_local) ? nv : vp + (size_t)(s0 + r) * D;
      vx[u] = ok[u] ? reinterpret_cast<const uint4*>(src)[c] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u * RPW + rg;
      float vf[8];
      bf16x8_to_f32(vx[u], vf);
      float e[GP];
#pragma unroll
      for (int h = 0; h < GP; ++h) e[h] = ok[u] ? lg[r * GP + h] : 0.f;
#pragma unroll
      for (int h = 0; h < GP; ++h)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[h][k] = fmaf(e[h], vf[k], acc[h][k]);
      float vn = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) vn += fabsf(vf[k]);
      vn = allreduce_sum<LPR / 2>(vn);
      if (c == 0 && r < n) {
        if (SPLIT) {
          if (ok[u]) vn_row[r] = vn;
        } else {
          float sc = kInf;
          if (ok[u]) {
            float ps = 0.f;
#pragma unroll
            for (int h = 0; h < GP; ++h)
              if (h < p.G) ps = fmaf(e[h], il[h], ps);
            sc = vn * ps;
            const uint64_t cand = pack_candidate(sc, s0 + r);
            best = cand < best ? cand : best;
          }
          score_row[r] = sc;
        }
      }
    }
  }

  // ---- O: fold the row groups of each wave, then the waves through LDS
#pragma unroll
  for (int h = 0; h < GP; ++h)
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int m = LPR; m < 64; m <<= 1) acc[h][k] += __shfl_xor(acc[h][k], m);
  __syncthreads();  // logits region is reused below
  float* ored = lg;  // [kWaves][GP][D]
  if (rg == 0) {
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
      for (int k = 0; k < 8; ++k) ored[(wave * GP + h) * D + c * 8 + k] = acc[h][k];
  }
  if (!SPLIT) {
    best = wave_min_u64(best);
    if (lane == 0) best_w[wave] = best;
  }
  __syncthreads();

  if (!SPLIT) {
    for (int idx = tid; idx < GP * D; idx += kThreads) {
      const int h = idx / D;
      if (h >= p.G) continue;
      float o = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) o += ored[w * GP * D + idx];
      p.out[((size_t)b * p.Hq + (size_t)j * p.G + h) * D + (idx - h * D)] =
          f32_to_bf16_rne(o * stat_il[h]);
    }
    if (tid == 0) {
      uint64_t m = best_w[0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) m = best_w[w] < m ? best_w[w] : m;
      p.evict[pair] = m == kNoCandidate ? -1 : (int32_t)(uint32_t)m;
    }
    return;
  }

  // ---- several splits: publish partials, the last split combines
  {
    float* po = p.part_o + ((size_t)pair * nsplit + sp) * GP * D;
    for (int idx = tid; idx < GP * D; idx += kThreads) {
      float o = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) o += ored[w * GP * D + idx];
      po[idx] = o;
    }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t done = atomicAdd(p.counters + pair, 1u);
    *flag = (done == (uint32_t)(nsplit - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (*flag == 0) return;
  __threadfence();

  // Global softmax statistics of the pair from the split partials.
  if (tid < GP) {
    const float* ml = p.part_ml + (size_t)pair * nsplit * GP * 2;
    float m = kNegInf;
    for (int s = 0; s < nsplit; ++s) m = fmaxf(m, ml[(s * GP + tid) * 2]);
    float l = 0.f;
    if (m != kNegInf) {
      for (int s = 0; s < nsplit; ++s) {
        const float ms = ml[(s * GP + tid) * 2];
        if (ms != kNegInf) l += ml[(s * GP + tid) * 2 + 1] * exp2f(ms - m);
      }
    }
    stat_m[tid] = m;
    stat_il[tid] = l > 0.f ? 1.0f / l : 0.f;
  }
  __syncthreads();

  {
    const float* ml = p.part_ml + (size_t)pair * nsplit * GP * 2;
    const float* po = p.part_o + (size_t)pair * nsplit * GP * D;
    for (int idx = tid; idx < GP * D; idx += kThreads) {
      const int h = idx / D;
      if (h >= p.G) continue;
      const float m = stat_m[h];
      float o = 0.f;
      if (m != kNegInf) {
        for (int s = 0; s < nsplit; ++s) {
          const float ms = ml[(s * GP + h) * 2];
          if (ms != kNegInf) o += po[(size_t)s * GP * D + idx] * exp2f(ms - m);
        }
      }
      p.out[((size_t)b * p.Hq + (size_t)j * p.G + h) * D + (idx - h * D)] =
          f32_to_bf16_rne(o * stat_il[h]);
    }
  }

  float gm[GP], gil[GP];
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    gm[h] = stat_m[h];
    gil[h] = stat_il[h];
  }
  best = kNoCandidate;
  const float* wl = p.ws_logit + row0 * GP;
  const float* wv = p.ws_vnorm + row0;
  float* sr = p.scores + row0;
  for (int r = tid; r < p.S; r += kThreads) {
    float sc = kInf;
    if (mrow[r] != 0) {
      float ps = 0.f;
#pragma unroll
      for (int h = 0; h < GP; ++h)
        if (h < p.G) ps = fmaf(exp2f(wl[(size_t)r * GP + h] - gm[h]), gil[h], ps);
      sc = wv[r] * ps;
      const uint64_t cand = pack_candidate(sc, r);
      best = cand < best ? cand : best;
    }
    sr[r] = sc;
  }
  best = wave_min_u64(best);
  if (lane == 0) best_w[wave] = best;
  __syncthreads();
  if (tid == 0) {
    uint64_t m = best_w[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = best_w[w] < m ? best_w[w] : m;
    p.evict[pair] = m == kNoCandidate ? -1 : (int32_t)(uint32_t)m;
    p.counters[pair] = 0;  // ready for the next call
  }
}

__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t value) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = value;
}

// ------------------------------------------------------------------ launch

template <int D, int GP>
hipError_t launch_dg(const DecodeParams& prm, int nblocks, size_t lds, hipStream_t stream) {
  if (prm.nsplit > 1)
    hipLaunchKernelGGL((longflow_decode_kernel<D, GP, true>), dim3(nblocks), dim3(kThreads), lds,
                       stream, prm);
  else
    hipLaunchKernelGGL((longflow_decode_kernel<D, GP, false>), dim3(nblocks), dim3(kThreads), lds,
                       stream, prm);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeParams& prm, int gp, int nblocks, size_t lds, hipStream_t stream) {
  switch (gp) {
    case 1: return launch_dg<D, 1>(prm, nblocks, lds, stream);
    case 2: return launch_dg<D, 2>(prm, nblocks, lds, stream);
    case 4: return launch_dg<D, 4>(prm, nblocks, lds, stream);
    case 8: return launch_dg<D, 8>(prm, nblocks, lds, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeParams& prm, int d, int gp, int nblocks, size_t lds,
                         hipStream_t stream) {
  switch (d) {
    case 64: return launch_d<64>(prm, gp, nblocks, lds, stream);
    case 128: return launch_d<128>(prm, gp, nblocks, lds, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t value, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n, value);
  return hipGetLastError();
}

}  // namespace lf
