// HIP kernels of LongFlow's fused decode step for gfx950 (MI355X).
//
// Source: "LongFlow: Efficient KV Cache Compression for Reasoning Models"
// (arXiv 2603.11504): abstract (one operator fusing attention, importance
// estimation and eviction) and Figure 2 caption (Left: write the previous
// choice, attend, return the next slot; Middle: K/V and mask streamed from HBM
// by block; Right: P.V split into G then O, score from G).
//
// decode kernel: one workgroup (8 or 16 waves) per slot range ("split") of
// one (sequence b, KV head j) pair.
//
//   setup    the split that owns prev_slot copies new_k/new_v into that cache
//            row before the workgroup barrier that follows the mask staging,
//            so the rest of the step reads the new row from the cache.
//   phase K  K rows stream from HBM in 16-byte lane loads (a d = 128 row is
//            16 lanes), two batches in flight per wave.  Each lane dots its 8
//            columns with the group's G queries; a DPP reduce-scatter over
//            the row's lanes leaves each head's full logit in one lane group.
//            Logits (log2 domain: the scale is pre-multiplied by log2 e) go
//            to LDS.
//   softmax  split max M_h and sum L_h of exp2(s - M_h); the LDS logits turn
//            into e = exp2(s - M_h) in place.
//   phase V  V rows stream the same way.  Each lane accumulates e * v for its
//            8 columns and G heads, and |v|_1 per row.  G = p * v is never
//            stored: O needs only sum_i e_i v_i / L and |G_hi|_1 = p_hi |v_i|_1
//            because p >= 0.
//   finish   single split: score_i = |v_i|_1 * sum_h e_hi / L_h is written in
//            phase V, O = acc / L, and the argmin over packed (score bits,
//            slot) words gives the evicted slot.
//            team (several splits, the default): the splits of a pair run
//            at once; between the softmax pass and phase V they exchange
//            their (M, L) through the workspace, so e, the scores and the
//            argmin candidates are formed against the pair's softmax as with
//            one split, and the last split of the pair to finish sums the
//            O accumulators and takes the minimum.
//            combine (several splits): each split writes its (M, L, acc)
//            partials, the logits and |v|_1 to the workspace; the combine and
//            finalize kernels launched right after on the same stream rescale
//            them to the true softmax.  The kernel boundary orders the two,
//            so no cross-workgroup fences are needed.
//
// Every slot goes through the same instruction sequence, so two slots with
// identical K/V rows get bit-identical scores and the lowest-index rule
// decides exact ties.

#include <hip/hip_runtime.h>

#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "launch.h"
#include "layout.h"
#include "longflow.h"

namespace lf {

// ------------------------------------------------------------ lane helpers

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Buffer resource over `bytes` bytes at `base` (raw, stride 0).  A load whose
// offset is not below `bytes` returns zero without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

constexpr uint32_t kOutOfRange = 0x80000000u;

// Cache policy of the K/V stream: rows are read once per step, so they are
// marked non-temporal (nt, policy bit 1) to leave the caches to everything
// else (about 6% faster than the default policy).
constexpr int kStreamPolicy = 2;

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t offset) {
  const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)offset, 0, kStreamPolicy);
  return make_uint4(x.x, x.y, x.z, x.w);
}

// fp32 sum of the 8 products of two rows of 8 bf16 values, plus `acc`
// (bf16 x bf16 products are exact in fp32).
__device__ __forceinline__ float dot8_bf16(const uint4& a, const uint4& b, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x), __builtin_bit_cast(bf16x2_t, b.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y), __builtin_bit_cast(bf16x2_t, b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z), __builtin_bit_cast(bf16x2_t, b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w), __builtin_bit_cast(bf16x2_t, b.w), acc, false);
  return acc;
}

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
//   8: row_ror:8 (lane ^ 8)         4: row_half_mirror (lane ^ 7)
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
// While N > 1 each step keeps half of the values (the upper half if the
// lane's BIT is set) and adds the partner's copy of that half; once one value
// is left the remaining steps are plain butterfly adds.
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

// Sum of each of N = GP * 8 accumulators over the row groups of a wave
// (the lanes that share a column chunk: lane bits 5, 4 and, for 8-lane rows,
// 3), left scattered: afterwards the first N / RG entries of a (RG = 64 /
// LPR row groups) hold the sums of entries fold_base(lane) .. + N / RG - 1.
// Bits 5 and 4 go through gfx950's lane swaps in the VALU: after
// permlane32_swap(x, y), lanes 0-31 hold (x_l, x_{l+32}) and lanes 32-63
// (y_{l-32}, y_l), so adding the pair leaves x's sum in the lower half and
// y's in the upper half; permlane16_swap does the same within each half.
template <int LPR, int GP>
__device__ __forceinline__ void fold_row_groups(float (&a)[GP][8], int lane) {
  constexpr int N = GP * 8;
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const int j = N / 2 + i;
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a[i / 8][i % 8]), __float_as_uint(a[j / 8][j % 8]),
                                                    false, false);
    a[i / 8][i % 8] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    const int j = N / 4 + i;
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[i / 8][i % 8]), __float_as_uint(a[j / 8][j % 8]),
                                                    false, false);
    a[i / 8][i % 8] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if constexpr (LPR == 8) {
    const bool upper = (lane & 8) != 0;
#pragma unroll
    for (int i = 0; i < N / 8; ++i) {
      const int j = N / 8 + i;
      // select values, not array elements: a select of two element
      // addresses keeps the compiler from holding the array in registers
      const float lo = a[i / 8][i % 8], hi = a[j / 8][j % 8];
      const float send = upper ? lo : hi;
      const float keep = upper ? hi : lo;
      a[i / 8][i % 8] = keep + partner<8>(send);
    }
  }
}

template <int LPR, int GP>
__device__ __forceinline__ int fold_base(int lane) {
  constexpr int N = GP * 8;
  int base = (lane >> 5) * (N / 2) + ((lane >> 4) & 1) * (N / 4);
  if constexpr (LPR == 8) base += ((lane >> 3) & 1) * (N / 8);
  return base;
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

// Keeps the scheduler from hoisting the LDS reads and conversions of later
// rows of a batch above the current one, which would multiply the live
// registers per wave (and so cut the waves per CU that keep loads in flight).
#define LF_ROW_FENCE() __builtin_amdgcn_sched_barrier(0)

// Ties 8 accumulators to this point of the program (an empty asm that reads
// and writes them), so the compiler cannot gather the FMAs of all rows of a
// batch at its end and keep every row's converted values live meanwhile.
__device__ __forceinline__ void pin8(float (&a)[8]) {
  asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]),
               "+v"(a[6]), "+v"(a[7]));
}
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kInf = __builtin_huge_valf();

// ------------------------------------------------------------ decode kernel

// Stagger of the streaming order in the split and team modes: each wave
// starts at batch (workgroup index * kRotate) mod (its batch count).
// Splits of a power-of-two number of rows otherwise stream in lockstep from
// addresses a power of two apart (batch 16, 64/8 heads, 16384 slots in 4
// splits: 269.8 -> 248.6 us/step); the single-split kernel measured no
// better staggered (the ragged batch of 256 sequences 3% slower),
// so it streams in order.
constexpr int kRotate = 5;

constexpr int waves_per_eu(int gp) { return gp >= 8 ? kWavesPerEuLarge : kWavesPerEuSmall; }

template <int D, int GP>
struct Shape {
  static constexpr int LPR = D / 8;                     // lanes per row (16 bytes each)
  static constexpr int RPW = 64 / LPR;                  // rows per wave load
  static constexpr int U = kUnroll;                   // wave loads per batch
  static constexpr int ROWS = RPW * U;                  // rows per wave batch
  static constexpr int HPL = GP > LPR ? GP / LPR : 1;   // heads per lane after reduce-scatter
  static constexpr int LPH = GP < LPR ? LPR / GP : 1;   // lanes holding each head
};

// One batch of U rows of a cache tensor: each lane reads its 16-byte chunk
// of rows r0 + u * RPW + rg.  Rows past the split or masked get an offset
// outside the buffer resource and come back as zero without a memory access;
// bit u of the result says whether row u is valid.
template <int D, int U, int RPW>
__device__ __forceinline__ uint32_t load_batch(uint4 (&buf)[U], __amdgpu_buffer_rsrc_t rows,
                                               const uint8_t* mk, int r0, int rg, int c) {
  uint32_t ok = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int r = r0 + u * RPW + rg;
    const bool v = mk[r] != 0;  // zero past the split
    const uint32_t off = v ? (uint32_t)r * (D * 2) + (uint32_t)c * 16 : kOutOfRange;
    buf[u] = load16(rows, off);
    ok |= (uint32_t)v << u;
  }
  return ok;
}

// How the workgroups of a launch share the pairs.
constexpr int kModeSingle = 0;  // one workgroup per pair, the whole step on chip
constexpr int kModeSplit = 1;   // one workgroup per split; combine kernels finish the step
constexpr int kModeTeam = 2;    // a team of workgroups per pair (one per split), all
                                // resident at once, exchanges softmax statistics mid-step

// Time a thread may spend on all of its team waits of one pair before it
// stops waiting and sets LF_DEV_TEAM_TIMEOUT: 0.2 s of the constant-rate
// real-time counter (100 MHz).  A wait lasts about one split's phase K, or
// for a team whose last members have not started, until some running
// workgroup ends; it runs out only if a member is kept from running, and
// then the step still ends, flagged.
constexpr uint64_t kTeamWaitTicks = 20000000ull;
constexpr uint64_t kReady = 1ull << 32;

// Publishes a float as a 64-bit word whose upper half marks it written.
__device__ __forceinline__ void team_publish(uint64_t* w, float x) {
  __hip_atomic_store(w, kReady | __float_as_uint(x), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits for a word published by another workgroup of the team until the
// thread's deadline; past it, it returns NaN at once.
__device__ __forceinline__ float team_wait(const uint64_t* w, uint32_t* status, uint64_t deadline) {
  for (;;) {
    const uint64_t v = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v & kReady) return __uint_as_float((uint32_t)v);
    if (__builtin_amdgcn_s_memrealtime() > deadline) break;
    __builtin_amdgcn_s_sleep(2);
  }
  atomicOr(status, LF_DEV_TEAM_TIMEOUT);
  return __builtin_nanf("");
}

// Up to 8 published words from each of K arrays, w[k][i * stride[k]] for
// i < n, with all their loads in flight at once (one round trip to memory
// where word-by-word waits took one each); words not yet ready are then
// waited for one by one.  out[k][i] for i >= n is unspecified.
template <int K>
__device__ __forceinline__ void team_read8(const uint64_t* const (&w)[K], const size_t (&stride)[K], int n,
                                           float (&out)[K][8], uint32_t* status, uint64_t deadline) {
  uint64_t v[K][8];
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      v[k][i] = i < n ? __hip_atomic_load(w[k] + i * stride[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : kReady;
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      out[k][i] = (v[k][i] & kReady) ? __uint_as_float((uint32_t)v[k][i])
                                     : team_wait(w[k] + i * stride[k], status, deadline);
}

// One (pair, split) of a decode step.
template <int D, int GP, int NW, int MODE>
__device__ __forceinline__ void decode_pair(const DecodeParams& p, int item, int pair, int sp, int nsplit) {
  constexpr bool SPLIT = MODE == kModeSplit;
  constexpr bool TEAM = MODE == kModeTeam;
  using SH = Shape<D, GP>;
  constexpr int LPR = SH::LPR, RPW = SH::RPW, U = SH::U, ROWS = SH::ROWS;
  constexpr int HPL = SH::HPL, LPH = SH::LPH;
  constexpr int kThreads = NW * 64;
  static_assert(ROWS <= kRowPad, "a wave batch may run past the split by at most kRowPad rows");

  extern __shared__ __align__(16) unsigned char smem[];

  // (opaque to the compiler, so that what derives from the thread index is
  // computed for each pair and not kept live across the persistent loop)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = lane % LPR;   // 16-byte column chunk of the row
  const int rg = lane / LPR;  // row within the wave load

  const int b = pair / p.Hkv;
  const int j = pair - b * p.Hkv;
  const int s0 = sp * p.split_len;
  const int n = min(p.S, s0 + p.split_len) - s0;

  const LdsLayout L = lds_layout(D, GP, p.split_len, NW, TEAM);
  float* lg = reinterpret_cast<float*>(smem + L.logits);
  uint8_t* mk = smem + L.mask;
  float* vnl = reinterpret_cast<float*>(smem + L.vnorm);         // team: |v|_1 per row
  float* red = reinterpret_cast<float*>(smem + L.scratch);     // [NW][GP]
  float* stat_m = red + NW * GP;                                 // [GP] split max (team: then the pair's)
  float* stat_il = stat_m + GP;                                  // [GP] 1 / L (team: the pair's)
  float* stat_c = stat_il + GP;                                  // [GP] team: e_split -> p factor
  uint64_t* best_w = reinterpret_cast<uint64_t*>(stat_c + GP);   // [NW]
  int* red_i = reinterpret_cast<int*>(best_w + NW);              // [NW]
  int* red_f = red_i + NW;                                       // [NW] fill step
  int* last = red_f + NW;                                        // team: last to finish the pair
  static_assert(NW * GP * 4 + GP * 12 + NW * 8 + NW * 8 + 4 <= kTicketSlot,
                "the reductions must stay below the team ticket in the scratch area");

  const size_t row0 = (size_t)pair * p.S;  // first cache row of this pair
  const uint16_t* krows = p.k + (row0 + s0) * D;
  const uint16_t* vrows = p.v + (row0 + s0) * D;
  const uint8_t* mrow = p.mask + (size_t)b * p.S;
  const uint16_t* nk = p.new_k + (size_t)pair * D;
  const uint16_t* nv = p.new_v + (size_t)pair * D;

  // ---- setup: queries, slot write (Figure 2, Left panel), mask staging
  // The group's queries stay packed bf16; the logit scale (times log2 e) is
  // applied to the reduced dot products.  Padded heads (h >= G) get q = 0 and
  // their results are never stored.
  uint4 qx[GP];
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    const int hh = h < p.G ? h : 0;
    const uint4 x = reinterpret_cast<const uint4*>(p.q + ((size_t)b * p.Hq + (size_t)j * p.G + hh) * D)[c];
    qx[h] = h < p.G ? x : make_uint4(0, 0, 0, 0);
  }
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(krows, (uint32_t)n * D * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vrows, (uint32_t)n * D * 2);

  // The split that owns prev_slot overwrites that cache row before anything
  // reads it: the barrier after the mask staging makes the workgroup's global
  // writes visible to all of its threads, so the row is then streamed like any
  // other (no other workgroup reads it during this step).  The new row, the
  // slot and the first block of the split's mask are all requested before
  // the row is written: the mask loads could not move above those stores
  // (a byte load may alias them), and one round trip to memory then covers
  // what took three.
  const int prev = p.prev[pair];
  const uint8_t* src = mrow + s0;
  uint8_t m0[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int i = u * kThreads + tid;
    m0[u] = i < n ? src[i] : 0;
  }
  uint4 kx = make_uint4(0, 0, 0, 0), vx = kx;
  if (tid < D / 8) {
    kx = reinterpret_cast<const uint4*>(nk)[tid];
    vx = reinterpret_cast<const uint4*>(nv)[tid];
  }
  const bool owns_prev = prev >= s0 && prev < s0 + n;
  if (prev != -1) {
    if (prev < 0 || prev >= p.S) {
      if (sp == 0 && tid == 0) atomicOr(p.status, LF_DEV_BAD_PREV);
    } else if (owns_prev) {
      if (tid < D / 8) {
        reinterpret_cast<uint4*>(p.k + (row0 + prev) * D)[tid] = kx;
        reinterpret_cast<uint4*>(p.v + (row0 + prev) * D)[tid] = vx;
      }
      if (p.fill && tid == 0 && mrow[prev] == 0) {
        // A free slot: it joins the mask.  The mask is shared by the KV
        // heads, so all of them must be writing this same slot.
        p.mask_w[(size_t)b * p.S + prev] = 1;
        for (int jj = 0; jj < p.Hkv; ++jj)
          if (p.prev[(size_t)b * p.Hkv + jj] != prev) {
            atomicOr(p.status, LF_DEV_FILL_DIVERGED);
            break;
          }
      }
    }
  }
  // Mask of the split into LDS, zero-padded past its end; n_eff = one past
  // the last valid row, so trailing masked rows are never streamed.  A fill
  // step also counts the slot it wrote as valid (whatever the mask byte
  // reads while other workgroups update it) and finds the lowest free slot.
  int* kq = reinterpret_cast<int*>(smem + L.scratch + kBatchSlot);  // next phase-K batch
  if (tid == 0) *kq = 0;
  int last_valid = -1;
  int first_free = INT_MAX;
  const int own = (p.fill && owns_prev) ? prev - s0 : -1;
  {
    const int npad = n + kRowPad;
    for (int base = 0; base < npad; base += kThreads * 8) {
      uint8_t t8[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * kThreads + tid;
        const uint8_t raw = base == 0 ? m0[u] : (i < n ? src[i] : 0);
        t8[u] = i < n ? (uint8_t)(raw | (i == own)) : 0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * kThreads + tid;
        if (i < npad) mk[i] = t8[u];
        if (t8[u] != 0) last_valid = i;
        if (!SPLIT && i < n && t8[u] == 0) first_free = min(first_free, i);
      }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) last_valid = max(last_valid, __shfl_xor(last_valid, m));
    if (lane == 0) red_i[wave] = last_valid;
    if (!SPLIT && p.fill) {
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) first_free = min(first_free, __shfl_xor(first_free, m));
      if (lane == 0) red_f[wave] = first_free;
    }
  }
  __syncthreads();
  // A write into a masked slot (outside the fill step) is flagged from the
  // staged mask.
  if (!p.fill && owns_prev && tid == 0 && mk[prev - s0] == 0) atomicOr(p.status, LF_DEV_WRITE_MASKED);
  int n_eff = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) n_eff = max(n_eff, red_i[w] + 1);

  const int stride = NW * ROWS;

  // ---- phase K: logits into LDS (rows past n_eff within the last batch get -inf)
  // Every lane of a head's lane group holds the same reduced logit, so all of
  // them store it (same value, same address): no branch in the loop body.
  const int hbase = GP <= LPR ? c / LPH : c * HPL;
  float mx[HPL];
#pragma unroll
  for (int i = 0; i < HPL; ++i) mx[i] = kNegInf;
  // Phase K takes batches of ROWS rows in the order the waves ask for them
  // (an LDS counter), so the waves of a workgroup finish it together (with
  // a fixed share each, the last wave of a 16-wave team split finished
  // 12 us after the first); each logit lands in its row's LDS word and the
  // maximum does not depend on the order.  The split and team modes start
  // from a per-workgroup batch, so that workgroups streaming at the same
  // pace read addresses that differ by more than the power-of-two spacing
  // of their cache rows.
  const int nbk = (n_eff + ROWS - 1) / ROWS;
  const int rotk = MODE != kModeSingle && nbk > 0 ? (int)(((unsigned)item * kRotate) % (unsigned)nbk) : 0;
  int next = 0;
  if (lane == 0) next = atomicAdd(kq, 1);
  next = __builtin_amdgcn_readfirstlane(next);
  while (next < nbk) {
    const int bk = next + rotk < nbk ? next + rotk : next + rotk - nbk;
    const int r0 = bk * ROWS;
    uint4 buf[U];
    const uint32_t ok = load_batch<D, U, RPW>(buf, krs, mk, r0, rg, c);
    int claim = 0;
    if (lane == 0) claim = atomicAdd(kq, 1);
    float* lrow = lg + (r0 + rg) * GP + hbase;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float a[GP];
#pragma unroll
      for (int h = 0; h < GP; ++h) a[h] = dot8_bf16(buf[u], qx[h], 0.f);
      reduce_scatter<LPR / 2, GP>(a, c);
      const bool valid = (ok >> u) & 1u;
#pragma unroll
      for (int i = 0; i < HPL; ++i) {
        const float val = valid ? a[i] * p.qscale : kNegInf;
        lrow[u * RPW * GP + i] = val;
        mx[i] = fmaxf(mx[i], val);
      }
      LF_ROW_FENCE();
    }
    next = __builtin_amdgcn_readfirstlane(claim);
  }
  // Phase V keeps a fixed share of rows per wave (rows wave * ROWS + k *
  // stride), so each lane's O accumulators sum the same rows in the same
  // order every time and O is the same bit for bit from run to run.
  //
  // A SIMD serves its waves oldest first, and waves w, w + 4, w + 8, w + 12
  // share one, so with equal shares the later waves end phase V last (on
  // the 16-wave team kernel waves 12-15 ended about 8.5 us after waves 0-3).
  // The team kernel therefore gives the last eighth of the batches to the
  // older half of the waves only: batch b < nbv - tailn goes to wave
  // b % NW, batch nbv - tailn + t to wave t % (NW / 2).  The shares stay a
  // fixed function of the wave and the row count.
  constexpr bool kSkew = MODE == kModeTeam && NW == 16;
  int nbatch, nmain = 0, mainn = 0, wv = 0;
  if constexpr (kSkew) {
    wv = __builtin_amdgcn_readfirstlane(wave);
    const int nbv = (n_eff + ROWS - 1) / ROWS;
    const int tailn = nbv / 8;
    mainn = nbv - tailn;
    nmain = wv < mainn ? (mainn - wv + NW - 1) / NW : 0;
    const int ntail = wv < NW / 2 && wv < tailn ? (tailn - wv + NW / 2 - 1) / (NW / 2) : 0;
    nbatch = nmain + ntail;
  } else {
    nbatch = wave * ROWS < n_eff ? (n_eff - wave * ROWS + stride - 1) / stride : 0;
    nmain = nbatch;
  }
  const int rot = MODE != kModeSingle && nmain > 0 ? (int)(((unsigned)item * kRotate) % (unsigned)nmain) : 0;

  // ---- softmax statistics of this split
  // Lanes with equal c hold the same heads; fold the row groups, then waves.
#pragma unroll
  for (int i = 0; i < HPL; ++i) {
#pragma unroll
    for (int m = LPR; m < 64; m <<= 1) mx[i] = fmaxf(mx[i], __shfl_xor(mx[i], m));
  }
  if (rg == 0 && (c % LPH) == 0) {
#pragma unroll
    for (int i = 0; i < HPL; ++i) red[wave * GP + hbase + i] = mx[i];
  }
  __syncthreads();
  if (tid < GP) {
    float m = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) m = fmaxf(m, red[w * GP + tid]);
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
    // Rows up to the end of the last batch (all written in phase K, -inf
    // when invalid) become e = exp2(s - split max); invalid ones become
    // exactly 0, so phase V needs no per-row select.
    // Four rows per thread at a time, their LDS reads issued together (one
    // row at a time, each read waited for the previous row's write); the
    // sum still adds the rows in the same order.
    const int covered = (n_eff + ROWS - 1) / ROWS * ROWS;
    constexpr int kStride = kThreads / GP;
    int r = tid / GP;
    for (; r + 3 * kStride < covered; r += 4 * kStride) {
      float sv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) sv[q] = lg[(r + q * kStride) * GP + h];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rq = r + q * kStride;
        const float e = (sv[q] == kNegInf) ? 0.f : exp2f(sv[q] - mh);
        lg[rq * GP + h] = e;
        lsum += e;
        if (SPLIT && rq < n_eff) wl[rq * GP + h] = e;
      }
    }
    for (; r < covered; r += kStride) {
      const float s = lg[r * GP + h];
      const float e = (s == kNegInf) ? 0.f : exp2f(s - mh);
      lg[r * GP + h] = e;
      lsum += e;
      if (SPLIT && r < n_eff) wl[r * GP + h] = e;
    }
#pragma unroll
    for (int m = GP; m < 64; m <<= 1) lsum += __shfl_xor(lsum, m);
    __syncthreads();  // every wave is done with the maxima in `red`
    if (lane < GP) red[wave * GP + lane] = lsum;
    __syncthreads();
    if (tid < GP) {
      float l = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) l += red[w * GP + tid];
      stat_il[tid] = (l > 0.f || l != l) ? 1.0f / l : 0.f;  // NaN logits make every p NaN
      if (SPLIT) {
        float* ml = p.part_ml + (((size_t)pair * nsplit + sp) * GP + tid) * 2;
        ml[0] = stat_m[tid];
        ml[1] = l;
      }
      if (TEAM) {
        // Publish this split's (max, sum) and go on to phase V at once; the
        // pair's statistics are read after it, when every split of the
        // team has long passed this point.
        uint64_t* xs = p.xstat + (size_t)pair * nsplit * GP * 2;
        team_publish(xs + (sp * GP + tid) * 2, stat_m[tid]);
        team_publish(xs + (sp * GP + tid) * 2 + 1, l);
      }
    }
    __syncthreads();
  }

  // ---- phase V: O accumulators, |v|_1, and (single split) scores
  float il[GP];
#pragma unroll
  for (int h = 0; h < GP; ++h) il[h] = (h < p.G) ? stat_il[h] : 0.f;
  float acc[GP][8];
#pragma unroll
  for (int h = 0; h < GP; ++h)
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[h][k] = 0.f;
  uint64_t best = kNoCandidate;

  // Each row's score (single split) or |v|_1 (combine path) goes into the
  // LDS word that held the row's first logit, written by all lanes of the row
  // group (same value), and leaves for HBM in one coalesced pass afterwards;
  // a team split keeps |v|_1 in its own row of LDS for the scores it forms
  // once the pair's statistics are known.
  auto finish_row = [&](float* slot, float vn, const float (&e)[GP], bool valid, int r) {
    vn = allreduce_sum<LPR / 2>(vn);
    if (SPLIT) {
      *slot = vn;
    } else if (TEAM) {
      vnl[r] = vn;
    } else {
      float ps = 0.f;
#pragma unroll
      for (int h = 0; h < GP; ++h) ps = fmaf(e[h], il[h], ps);
      const float sc = valid ? vn * ps : kInf;
      const uint64_t cand = valid ? pack_candidate(sc, s0 + r) : kNoCandidate;
      best = cand < best ? cand : best;
      *slot = sc;
    }
  };
  for (int bi = 0; bi < nbatch; ++bi) {
    int r0;
    if constexpr (kSkew) {
      r0 = (bi < nmain ? wv + (bi + rot < nmain ? bi + rot : bi + rot - nmain) * NW
                       : mainn + wv + (bi - nmain) * (NW / 2)) * ROWS;
    } else {
      r0 = wave * ROWS + (bi + rot < nbatch ? bi + rot : bi + rot - nbatch) * stride;
    }
    uint4 vbuf[U];
    const uint32_t vok = load_batch<D, U, RPW>(vbuf, vrs, mk, r0, rg, c);
    float* lrow = lg + (r0 + rg) * GP;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool valid = (vok >> u) & 1u;
      float vf[8];
      bf16x8_to_f32(vbuf[u], vf);
      float e[GP];  // exactly 0 for invalid rows (see the softmax pass)
#pragma unroll
      for (int h = 0; h < GP; ++h) e[h] = lrow[u * RPW * GP + h];
#pragma unroll
      for (int h = 0; h < GP; ++h) {
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[h][k] = fmaf(e[h], vf[k], acc[h][k]);
        pin8(acc[h]);
      }
      float vn = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) vn += fabsf(vf[k]);
      finish_row(lrow + u * RPW * GP, vn, e, valid, r0 + u * RPW + rg);
      LF_ROW_FENCE();
    }
  }
  __syncthreads();
  if constexpr (TEAM) {
    // The pair's statistics, rebuilt as the combine kernel does: max over
    // the splits, then the rescaled sums in split order (a split without a
    // finite logit adds its sum as it is: 0 when it has no valid slot, NaN
    // when its logits are NaN).  c turns this split's e into probabilities:
    // p = e * exp2(split max - pair max) / L.
    if (tid < GP) {
      // this head's (max, sum) words: split q's at xs + q * GP * 2
      const uint64_t* xs = p.xstat + (size_t)pair * nsplit * GP * 2 + tid * 2;
      const size_t st2[2] = {(size_t)GP * 2, (size_t)GP * 2};
      const uint64_t deadline = __builtin_amdgcn_s_memrealtime() + kTeamWaitTicks;
      float gm = kNegInf;
      float gl = 0.f;
      if (nsplit <= 8) {  // every word in one batch
        float ml[2][8];
        const uint64_t* w2[2] = {xs, xs + 1};
        team_read8<2>(w2, st2, nsplit, ml, p.status, deadline);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (i < nsplit) gm = fmaxf(gm, ml[0][i]);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (i < nsplit) gl = ml[0][i] != kNegInf ? fmaf(ml[1][i], exp2f(ml[0][i] - gm), gl) : gl + ml[1][i];
      } else {  // the maxima 8 splits at a time, then the sums
        for (int q0 = 0; q0 < nsplit; q0 += 8) {
          float m[1][8];
          const uint64_t* w1[1] = {xs + (size_t)q0 * GP * 2};
          const size_t st1[1] = {(size_t)GP * 2};
          team_read8<1>(w1, st1, nsplit - q0, m, p.status, deadline);
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (q0 + i < nsplit) gm = fmaxf(gm, m[0][i]);
        }
        for (int q0 = 0; q0 < nsplit; q0 += 8) {
          float ml[2][8];
          const uint64_t* w2[2] = {xs + (size_t)q0 * GP * 2, xs + (size_t)q0 * GP * 2 + 1};
          team_read8<2>(w2, st2, nsplit - q0, ml, p.status, deadline);
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (q0 + i < nsplit)
              gl = ml[0][i] != kNegInf ? fmaf(ml[1][i], exp2f(ml[0][i] - gm), gl) : gl + ml[1][i];
        }
      }
      const float gil = (gl > 0.f || gl != gl) ? 1.0f / gl : 0.f;
      const float ms = stat_m[tid];
      stat_c[tid] = ms != kNegInf ? exp2f(ms - gm) * gil : 0.f;
      stat_m[tid] = gm;
      stat_il[tid] = gil;
    }
    __syncthreads();
    // Scores of the split's rows, written in one coalesced pass, and the
    // split's lowest (score, slot).
    float cc[GP];
#pragma unroll
    for (int h = 0; h < GP; ++h) cc[h] = h < p.G ? stat_c[h] : 0.f;
    for (int r = tid; r < n; r += kThreads) {
      float sc = kInf;
      if (r < n_eff && mk[r] != 0) {
        float ps = 0.f;
#pragma unroll
        for (int h = 0; h < GP; ++h) ps = fmaf(lg[r * GP + h], cc[h], ps);
        sc = vnl[r] * ps;
        const uint64_t cand = pack_candidate(sc, s0 + r);
        best = cand < best ? cand : best;
      }
      p.scores[row0 + s0 + r] = sc;
    }
  } else {
    // Rows at or past n_eff are all masked: score +inf, no |v|_1 needed.
    float* dst = SPLIT ? p.ws_vnorm + row0 + s0 : p.scores + row0 + s0;
    const int lim = SPLIT ? n_eff : n;
    int r = tid;
    for (; r + 3 * kThreads < lim; r += 4 * kThreads) {
      float sv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) sv[q] = lg[(r + q * kThreads) * GP];
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[r + q * kThreads] = r + q * kThreads < n_eff ? sv[q] : kInf;
    }
    for (; r < lim; r += kThreads) dst[r] = r < n_eff ? lg[r * GP] : kInf;
  }

  // ---- O: fold the row groups of each wave, then the waves through LDS
  static_assert(LPR == 16 || LPR == 8, "row groups of 16 or 8 lanes");
  fold_row_groups<LPR, GP>(acc, lane);
  if (!SPLIT) {
    best = wave_min_u64(best);
    if (lane == 0) best_w[wave] = best;
  }
  __syncthreads();  // the logits region is reused below
  float* ored = lg;  // [NW][GP][D]
  {
    constexpr int PER = GP * 8 / (64 / LPR);  // sums each lane holds
    const int fb = fold_base<LPR, GP>(lane);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int g = fb + i;
      ored[(wave * GP + g / 8) * D + c * 8 + (g & 7)] = acc[i / 8][i % 8];
    }
  }
  __syncthreads();

  if (MODE == kModeSingle) {
    for (int idx = tid; idx < GP * D; idx += kThreads) {
      const int h = idx / D;
      if (h >= p.G) continue;
      float o = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) o += ored[w * GP * D + idx];
      p.out[((size_t)b * p.Hq + (size_t)j * p.G + h) * D + (idx - h * D)] =
          f32_to_bf16_rne(o * stat_il[h]);
    }
    if (tid == 0) {
      uint64_t m = best_w[0];
#pragma unroll
      for (int w = 1; w < NW; ++w) m = best_w[w] < m ? best_w[w] : m;
      int32_t next = m == kNoCandidate ? -1 : (int32_t)(uint32_t)m;
      if (p.fill) {
        // while the sequence has a free slot, the next token goes there
        int ff = INT_MAX;
#pragma unroll
        for (int w = 0; w < NW; ++w) ff = min(ff, red_f[w]);
        if (ff != INT_MAX) next = ff;
      }
      p.evict[pair] = next;
      // the pair's valid extent, for the next step's longest-first schedule
      if (p.lens) __hip_atomic_store(p.lens + pair, (uint32_t)n_eff, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else if (SPLIT) {
    // The split's O accumulators, against the split's own max.
    float* po = p.part_o + ((size_t)pair * nsplit + sp) * GP * D;
    for (int idx = tid; idx < GP * D; idx += kThreads) {
      float o = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) o += ored[w * GP * D + idx];
      po[idx] = o;
    }
  }
  if (TEAM) {
    // Publish this split's O accumulators and results, count it in; the
    // team's last split to arrive waits for the others' words, sums them in
    // split order and writes O and the slot.  Every word carries its own
    // ready bit, so no fence orders them against the count.
    uint64_t* xo = p.xo + ((size_t)pair * nsplit + sp) * GP * D;
    for (int idx = tid; idx < GP * D; idx += kThreads) {
      float o = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) o += ored[w * GP * D + idx];
      team_publish(xo + idx, o);
    }
    if (tid == 0) {
      uint64_t m = best_w[0];
#pragma unroll
      for (int w = 1; w < NW; ++w) m = best_w[w] < m ? best_w[w] : m;
      int ff = INT_MAX;
#pragma unroll
      for (int w = 0; w < NW; ++w) ff = min(ff, red_f[w]);
      uint64_t* xf = p.xfin + ((size_t)pair * nsplit + sp) * 3;
      team_publish(xf, __uint_as_float((uint32_t)(m >> 32)));
      team_publish(xf + 1, __uint_as_float((uint32_t)m));
      team_publish(xf + 2, __uint_as_float(p.fill && ff != INT_MAX ? (uint32_t)(s0 + ff) : (uint32_t)INT_MAX));
    }
    __syncthreads();
    if (tid == 0) *last = atomicAdd(p.xcnt + pair, 1u) == (unsigned)(nsplit - 1);
    __syncthreads();
    if (*last) {
      // O = sum over the splits of acc * exp2(split max - pair max), in split
      // order, divided by L: the combine kernel's expression.
      const uint64_t deadline = __builtin_amdgcn_s_memrealtime() + kTeamWaitTicks;
      const uint64_t* xa = p.xo + (size_t)pair * nsplit * GP * D;
      const uint64_t* xs = p.xstat + (size_t)pair * nsplit * GP * 2;
      for (int idx = tid; idx < GP * D; idx += kThreads) {
        const int h = idx / D;
        if (h >= p.G) continue;
        const float gm = stat_m[h];
        float o = 0.f;
        if (gm != kNegInf) {
          for (int q0 = 0; q0 < nsplit; q0 += 8) {  // 8 splits' words per batch
            float mp[2][8];
            const uint64_t* w2[2] = {xs + ((size_t)q0 * GP + h) * 2, xa + (size_t)q0 * GP * D + idx};
            const size_t st2[2] = {(size_t)GP * 2, (size_t)GP * D};
            team_read8<2>(w2, st2, nsplit - q0, mp, p.status, deadline);
#pragma unroll
            for (int i = 0; i < 8; ++i)
              if (q0 + i < nsplit && mp[0][i] != kNegInf) o = fmaf(mp[1][i], exp2f(mp[0][i] - gm), o);
          }
        }
        p.out[((size_t)b * p.Hq + (size_t)j * p.G + h) * D + (idx - h * D)] = f32_to_bf16_rne(o * stat_il[h]);
      }
      if (tid == 0) {
        uint64_t m = kNoCandidate;
        uint32_t ff = (uint32_t)INT_MAX;
        for (int q0 = 0; q0 < nsplit; q0 += 8) {
          const uint64_t* xf = p.xfin + ((size_t)pair * nsplit + q0) * 3;
          float r[3][8];
          const uint64_t* w3[3] = {xf, xf + 1, xf + 2};
          const size_t st3[3] = {3, 3, 3};
          team_read8<3>(w3, st3, nsplit - q0, r, p.status, deadline);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            if (q0 + i >= nsplit) break;
            const uint64_t cq = (uint64_t)__float_as_uint(r[0][i]) << 32 | __float_as_uint(r[1][i]);
            m = cq < m ? cq : m;
            ff = min(ff, __float_as_uint(r[2][i]));
          }
        }
        int32_t next = m == kNoCandidate ? -1 : (int32_t)(uint32_t)m;
        if (p.fill && ff != (uint32_t)INT_MAX) next = (int32_t)ff;
        p.evict[pair] = next;
      }
      // Leave the pair's words at zero for the next step.  Every split has
      // read all it needs from them: each reads the statistics before it
      // publishes and counts itself in, and this last split has read the rest.
      __syncthreads();
      uint64_t* zo = p.xo + (size_t)pair * nsplit * GP * D;
      for (int i = tid; i < nsplit * GP * D; i += kThreads)
        __hip_atomic_store(zo + i, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      uint64_t* zs = p.xstat + (size_t)pair * nsplit * GP * 2;
      for (int i = tid; i < nsplit * GP * 2; i += kThreads)
        __hip_atomic_store(zs + i, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      uint64_t* zf = p.xfin + (size_t)pair * nsplit * 3;
      for (int i = tid; i < nsplit * 3; i += kThreads)
        __hip_atomic_store(zf + i, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (tid == 0) __hip_atomic_store(p.xcnt + pair, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Pair indices [first, pairs) into `dst`, sorted by the valid extents in
// p.lens, longest first (a counting sort over kOrderBins extent classes; the
// order inside a class is arbitrary).  Each extent is read once, so `dst`
// is a permutation whatever the words hold: the pairs of this step still
// running have not written theirs yet, and their previous value (or zero)
// stands in.
// Returns false, and writes nothing, when all of them fall in one class (an
// order would then only cost its lookups).  Uses the first kOrderBins + 1
// words of LDS; the caller is done with them.
constexpr int kOrderBins = 512;

template <int NT>
__device__ __forceinline__ bool build_pair_order(const DecodeParams& p, int first, uint32_t* dst) {
  static_assert(kOrderMaxPairs % NT == 0 && kOrderBins % 64 == 0, "");
  constexpr int kPer = kOrderMaxPairs / NT;
  constexpr int kBinsPerLane = kOrderBins / 64;
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* hist = reinterpret_cast<uint32_t*>(smem);
  uint32_t* spread = hist + kOrderBins;  // non-empty classes
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  for (int i = tid; i < kOrderBins; i += NT) hist[i] = 0;
  int shift = 0;
  while (((p.S - 1) >> shift) >= kOrderBins) ++shift;
  __syncthreads();
  uint32_t bin[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = first + u * NT + tid;
    if (i < p.pairs) {
      const uint32_t len = __hip_atomic_load(p.lens + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      bin[u] = (uint32_t)(kOrderBins - 1) - min(len >> shift, (uint32_t)(kOrderBins - 1));
      atomicAdd(hist + bin[u], 1u);
    }
  }
  __syncthreads();
  if (tid < 64) {  // exclusive prefix sum of the class counts
    uint32_t c[kBinsPerLane], sum = 0, used = 0;
#pragma unroll
    for (int r = 0; r < kBinsPerLane; ++r) {
      c[r] = hist[lane * kBinsPerLane + r];
      sum += c[r];
      used += c[r] != 0;
    }
    uint32_t incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
      used += __shfl_xor(used, o);
    }
    uint32_t at = incl - sum;
#pragma unroll
    for (int r = 0; r < kBinsPerLane; ++r) {
      hist[lane * kBinsPerLane + r] = at;
      at += c[r];
    }
    if (lane == 0) *spread = used;
  }
  __syncthreads();
  if (*spread < 2) return false;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = first + u * NT + tid;
    if (i < p.pairs) dst[atomicAdd(hist + bin[u], 1u)] = (uint32_t)i;
  }
  return true;
}

// The kernel's parameter block read from the kernarg segment through a
// pointer the compiler cannot follow (so the loads are not hoisted out of a
// loop around the call).
__device__ __forceinline__ DecodeParams reload_params() {
  static_assert(sizeof(DecodeParams) % 4 == 0, "copied as 32-bit words");
  auto pk = (const __attribute__((address_space(4))) uint32_t*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(pk));
  DecodeParams q;
  uint32_t* dst = reinterpret_cast<uint32_t*>(&q);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(DecodeParams) / 4); ++i) dst[i] = pk[i];
  return q;
}

template <int D, int GP, int NW, int MODE>
__global__ __launch_bounds__(NW * 64, waves_per_eu(GP)) void longflow_decode_kernel(DecodeParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  int* tk = reinterpret_cast<int*>(smem + lds_layout(D, GP, p.split_len, NW, MODE == kModeTeam).scratch + kTicketSlot);
  if constexpr (MODE == kModeSingle) {
    // Persistent workgroups: workgroup w takes pair w first, then further
    // pairs from the work-item counter (tickets gridDim.x, gridDim.x + 1, ...)
    // until none is left, so a compute unit that streams faster takes more
    // pairs.  (The dispatcher deals workgroups to the 8 XCDs in turn, and the
    // XCDs stream at different rates: with one workgroup per pair, the first
    // pairs of batch 128 x 8 KV heads x 3200 slots took 105 us on the fastest
    // XCDs and 140 us on the slowest,
    // and the ragged batch's long sequences ended the step on slow XCDs.  The
    // first pair goes by block index because 512 workgroups starting on one
    // counter at once spread their starts over 5 us.)
    //
    // The parameters are read again for every pair through a pointer the
    // compiler cannot follow across iterations; otherwise it keeps every
    // parameter and everything derived from it live across the loop, and
    // the registers the pair needs spill.
    // With at least as many workgroups as pairs the counter is not used.
    //
    // Ticket t hands out pair order[t - gridDim.x] when the workspace holds
    // an order for this launch (pair count and workgroups): the pairs past
    // the first gridDim.x sorted by their valid extent at the previous step,
    // longest first, so that short pairs fill the end of the step instead of
    // a long pair starting last (the ragged batch, 256 sequences of 256..8192
    // valid slots: 727 us instead of 767).  The first pair stays the block
    // index, so no workgroup waits for the schedule words to start.  The
    // workgroup that draws ticket `pairs` (the first to find the queue
    // empty) builds the next order into the other buffer while the rest
    // finish their last pairs, and the last workgroup to leave switches
    // buffers: every claim of this launch has read the switch word by then.
    // Each buffer has a word of its own naming the launch its order is for
    // (0: none, or all pairs alike), so the builder can set it at once.
    const bool dynamic = gridDim.x < (unsigned)p.pairs;
    const uint32_t key = (uint32_t)p.pairs << 16 | gridDim.x;
    int* tp = tk + (int)((kPairSlot - kTicketSlot) / 4);
    unsigned t = blockIdx.x;
    int pair = (int)t;
    while (t < (unsigned)p.pairs) {
      const DecodeParams pp = reload_params();
      decode_pair<D, GP, NW, MODE>(pp, pair, pair, 0, 1);
      if (!dynamic) break;
      __syncthreads();  // the pair is done with the LDS
      if (threadIdx.x == 0) {
        // the schedule words travel with the claim (no wait of their own)
        uint32_t st = 0, k0 = 0, k1 = 0;
        if (p.order) {
          const uint32_t* sw = p.queue + kSchedWord;
          st = sw[0] & 1u;
          k0 = sw[1];
          k1 = sw[2];
        }
        const unsigned nt = gridDim.x + atomicAdd(p.queue, 1u);
        unsigned np = nt;
        if (nt < (unsigned)p.pairs && (st ? k1 : k0) == key)
          np = p.order[(size_t)st * kOrderMaxPairs + (nt - gridDim.x)];
        *tk = (int)nt;
        *tp = (int)np;
      }
      __syncthreads();
      t = (unsigned)*tk;
      pair = *tp;
    }
    if (dynamic && p.order && t == (unsigned)p.pairs) {
      const uint32_t nb = (p.queue[kSchedWord] & 1u) ^ 1u;  // the buffer this launch does not read
      const bool built = build_pair_order<NW * 64>(p, (int)gridDim.x, p.order + (size_t)nb * kOrderMaxPairs);
      if (threadIdx.x == 0) atomicExch(p.queue + kSchedWord + 1 + nb, built ? key : 0u);
    }
    // Every workgroup has made its last claim once all have counted
    // themselves out, so the last one can leave the counters at zero for the
    // next launch (and flip the schedule's switch word without reading it).
    if (dynamic && threadIdx.x == 0 && atomicAdd(p.queue + 1, 1u) == gridDim.x - 1) {
      atomicExch(p.queue, 0u);
      atomicExch(p.queue + 1, 0u);
      if (p.order) atomicXor(p.queue + kSchedWord, 1u);
    }
  } else if constexpr (MODE == kModeTeam) {
    // Work items go out by tickets in the order workgroups start, not by
    // block index.  The pairs form p.ticket_ranges ranges of whole teams,
    // each with its own counter (left at zero by the previous launch); a
    // workgroup claims from range (block index mod ranges) first and from the
    // next ranges once that one is used up.  There are as many workgroups as
    // items, so every claim succeeds.  Within a range tickets go out in start
    // order, so every team of a range except the one holding its newest
    // ticket has all its members running: at most ranges * (nsplit - 1)
    // workgroups ever wait for members that have not started, and only until
    // some running workgroup ends.  The host picks the number of ranges so
    // that one XCD holds more workgroups at once than that, since a
    // workgroup waits for room on the XCD it is dealt to.  (One counter for
    // all made 256 workgroups queue on one atomic as a wave of them started:
    // 3-4% slower, so the most ranges that fit are used.)
    const int nsplit = p.nsplit;
    const int ranges = p.ticket_ranges;
    if (threadIdx.x == 0) {
      int claimed = -1;
      for (int k = 0; k < ranges && claimed < 0; ++k) {
        const int r = (int)((blockIdx.x + k) % ranges);
        const int lo = ticket_range_first_pair(p.pairs, r, ranges) * nsplit;
        const int hi = ticket_range_first_pair(p.pairs, r + 1, ranges) * nsplit;
        if (lo == hi) continue;
        const unsigned t = atomicAdd(p.xticket + r, 1u);
        if (t < (unsigned)(hi - lo)) claimed = lo + (int)t;
      }
      *tk = claimed;
      // Every workgroup has made its last claim once all have counted
      // themselves in here (each counts after its claims have returned): the
      // last one zeroes the ticket counters and this count for the next launch.
      if (atomicAdd(p.queue + 2, 1u) == gridDim.x - 1) {
        for (int r = 0; r < kTicketRanges; ++r) atomicExch(p.xticket + r, 0u);
        atomicExch(p.queue + 2, 0u);
      }
    }
    __syncthreads();
    const int t = *tk;
    if (t < 0) return;  // not reached: one workgroup per item
    decode_pair<D, GP, NW, MODE>(p, t, t / nsplit, t % nsplit, nsplit);
  } else {
    // The split mode gives each XCD (workgroups are dealt to the 8 XCDs in
    // turn) a contiguous run of work items, so the splits of a pair share an
    // L2.
    const int nblk = gridDim.x;
    const int xcd = blockIdx.x & 7;
    const int per = nblk >> 3, rem = nblk & 7;
    const int item = xcd * per + (xcd < rem ? xcd : rem) + (blockIdx.x >> 3);
    decode_pair<D, GP, NW, MODE>(p, item, item / p.nsplit, item % p.nsplit, p.nsplit);
  }
}

// ------------------------------------------------------------ combine kernels
//
// After a split decode.  longflow_combine_kernel: one workgroup per (pair,
// chunk of kCombineRows slots).  It rebuilds the pair's global max M_h and sum
// L_h from the split partials, and for every split q the factor c_qh =
// exp2(m_qh - M_h) / L_h that turns the split's e = exp2(s - m_qh) into
// probabilities.  It writes score_i = |v_i|_1 * sum_h e_hi c_qh for the valid
// slots of its chunk (+inf elsewhere) and the chunk's lowest-index minimum;
// chunk 0 also writes O = sum_q acc_q exp2(m_q - M_h) / L_h.
// longflow_finalize_kernel then takes the minimum over the chunks of each
// pair.  The team path forms its scores and O with the same expressions in
// the same order, so the two paths give the same scores bit for bit.

constexpr int kCombineThreads = 256;
constexpr int kCombineRowsPerThread = 8;
constexpr int kCombineRows = kCombineThreads * kCombineRowsPerThread;
static_assert(kCombineRows == kCombineSlots, "combine chunking must match the workspace layout");

template <int D, int GP>
__global__ __launch_bounds__(kCombineThreads) void longflow_combine_kernel(DecodeParams p, int nchunk) {
  constexpr int NWC = kCombineThreads / 64;
  constexpr int R = kCombineRowsPerThread;
  __shared__ float stat_m[GP], stat_il[GP];
  __shared__ float cs[kMaxSplits * GP];  // [split][head] e -> p factors
  __shared__ uint64_t best_w[NWC];
  __shared__ int free_w[NWC];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int pair = blockIdx.x / nchunk;
  const int chunk = blockIdx.x - pair * nchunk;
  const int b = pair / p.Hkv;
  const int j = pair - b * p.Hkv;
  const int nsplit = p.nsplit;
  const float* ml = p.part_ml + (size_t)pair * nsplit * GP * 2;

  const size_t row0 = (size_t)pair * p.S;
  const float* wl = p.ws_logit + row0 * GP;
  const float* wv = p.ws_vnorm + row0;
  const uint8_t* mrow = p.mask + (size_t)b * p.S;
  float* sr = p.scores + row0;
  const int base = chunk * kCombineRows;
  // Every load is issued, mask, e and |v|_1 together, before any is used
  // (rows past S read row S - 1); the mask only decides what the values are
  // used for.  A masked row's workspace entry may be stale and is never
  // used.
  bool valid[R];
  uint8_t mk[R];
  float vn[R];
  float s[R][GP];
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int r = min(base + u * kCombineThreads + tid, p.S - 1);
    mk[u] = mrow[r];
    vn[u] = wv[r];
    if constexpr (GP >= 4) {
#pragma unroll
      for (int h4 = 0; h4 < GP; h4 += 4) {
        const float4 x = reinterpret_cast<const float4*>(wl + (size_t)r * GP + h4)[0];
        s[u][h4] = x.x;
        s[u][h4 + 1] = x.y;
        s[u][h4 + 2] = x.z;
        s[u][h4 + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int h = 0; h < GP; ++h) s[u][h] = wl[(size_t)r * GP + h];
    }
  }
  // The pair's global max M_h and sum L_h over the splits, split partials
  // read eight at a time (the order of the sums is the split order).
  if (tid < GP) {
    constexpr int SB = 8;
    float m = kNegInf;
    for (int s0 = 0; s0 < nsplit; s0 += SB) {
      float ms[SB];
#pragma unroll
      for (int u = 0; u < SB; ++u) ms[u] = ml[(min(s0 + u, nsplit - 1) * GP + tid) * 2];
#pragma unroll
      for (int u = 0; u < SB; ++u) m = s0 + u < nsplit ? fmaxf(m, ms[u]) : m;
    }
    // A split without a finite logit adds its sum as it is: 0 when it has no
    // valid slot, NaN when its valid logits are NaN, which then reaches O and
    // the scores as it does with one split.
    float l = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += SB) {
      float ms[SB], ls[SB];
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        const int sc = min(s0 + u, nsplit - 1);
        ms[u] = ml[(sc * GP + tid) * 2];
        ls[u] = ml[(sc * GP + tid) * 2 + 1];
      }
#pragma unroll
      for (int u = 0; u < SB; ++u)
        if (s0 + u < nsplit) l = ms[u] != kNegInf ? fmaf(ls[u], exp2f(ms[u] - m), l) : l + ls[u];
    }
    stat_m[tid] = m;
    stat_il[tid] = (l > 0.f || l != l) ? 1.0f / l : 0.f;
  }
  __syncthreads();
  // e -> p factor of every (split, head); zero for padded heads.
  for (int i = tid; i < nsplit * GP; i += kCombineThreads) {
    const int q = i / GP, h = i - q * GP;
    const float mq = ml[(q * GP + h) * 2];
    const float gil = h < p.G ? stat_il[h] : 0.f;
    cs[i] = mq != kNegInf ? exp2f(mq - stat_m[h]) * gil : 0.f;
  }
  __syncthreads();

  if (chunk == 0) {
    const float* po = p.part_o + (size_t)pair * nsplit * GP * D;
    constexpr int SB = 4;
    for (int idx = tid; idx < GP * D; idx += kCombineThreads) {
      const int h = idx / D;
      if (h >= p.G) continue;
      const float m = stat_m[h];
      float o = 0.f;
      if (m != kNegInf) {
        for (int s0 = 0; s0 < nsplit; s0 += SB) {
          float pv[SB], ms[SB];
#pragma unroll
          for (int u = 0; u < SB; ++u) {
            const int sc = min(s0 + u, nsplit - 1);
            pv[u] = po[(size_t)sc * GP * D + idx];
            ms[u] = ml[(sc * GP + h) * 2];
          }
#pragma unroll
          for (int u = 0; u < SB; ++u)
            if (s0 + u < nsplit && ms[u] != kNegInf) o = fmaf(pv[u], exp2f(ms[u] - m), o);
        }
      }
      p.out[((size_t)b * p.Hq + (size_t)j * p.G + h) * D + (idx - h * D)] =
          f32_to_bf16_rne(o * stat_il[h]);
    }
  }

#pragma unroll
  for (int u = 0; u < R; ++u) valid[u] = base + u * kCombineThreads + tid < p.S && mk[u] != 0;
  // Fill step: the lowest free slot of the chunk.  The decode kernel has
  // already added the written slots to the mask.
  if (p.fill) {
    int ff = INT_MAX;
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int r = base + u * kCombineThreads + tid;
      if (r < p.S && !valid[u]) ff = min(ff, r);
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) ff = min(ff, __shfl_xor(ff, m));
    if (lane == 0) free_w[wave] = ff;
  }
  uint64_t best = kNoCandidate;
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int r = base + u * kCombineThreads + tid;
    float sc = kInf;
    if (valid[u]) {
      const float* cq = cs + (r / p.split_len) * GP;
      float ps = 0.f;
#pragma unroll
      for (int h = 0; h < GP; ++h) ps = fmaf(s[u][h], cq[h], ps);
      sc = vn[u] * ps;
      const uint64_t cand = pack_candidate(sc, r);
      best = cand < best ? cand : best;
    }
    if (r < p.S) sr[r] = sc;
  }
  best = wave_min_u64(best);
  if (lane == 0) best_w[wave] = best;
  __syncthreads();
  if (tid == 0) {
    uint64_t m = best_w[0];
#pragma unroll
    for (int w = 1; w < NWC; ++w) m = best_w[w] < m ? best_w[w] : m;
    p.cand[(size_t)pair * nchunk + chunk] = m;
    if (p.fill) {
      int ff = free_w[0];
#pragma unroll
      for (int w = 1; w < NWC; ++w) ff = min(ff, free_w[w]);
      p.ffree[(size_t)pair * nchunk + chunk] = (uint32_t)ff;
    }
  }
}

__global__ void longflow_finalize_kernel(DecodeParams p, int pairs, int nchunk) {
  const int pair = blockIdx.x * blockDim.x + threadIdx.x;
  if (pair >= pairs) return;
  const uint64_t* c = p.cand + (size_t)pair * nchunk;
  uint64_t m = kNoCandidate;
  for (int i = 0; i < nchunk; ++i) m = c[i] < m ? c[i] : m;
  int32_t next = m == kNoCandidate ? -1 : (int32_t)(uint32_t)m;
  if (p.fill) {
    uint32_t ff = (uint32_t)INT_MAX;
    for (int i = 0; i < nchunk; ++i) ff = min(ff, p.ffree[(size_t)pair * nchunk + i]);
    if (ff != (uint32_t)INT_MAX) next = (int32_t)ff;
  }
  p.evict[pair] = next;
}

__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t value) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = value;
}

// ------------------------------------------------------------------ launch

template <int D, int GP, int NW>
hipError_t launch_dgw(const DecodeParams& prm, int nblocks, size_t lds, int team_grid, int grid, hipStream_t stream) {
  if (team_grid > 0) {
    // The exchange region is all zero: from the workspace's first zero fill,
    // and after every team launch (each team zeroes its words and the last
    // workgroup the counters).  One plain launch of every (pair, split): the ticket order (see the
    // kernel) needs no co-residency promise, so no cooperative launch (which
    // cost 11-19 us more per launch) and no rounds.
    hipLaunchKernelGGL((longflow_decode_kernel<D, GP, NW, kModeTeam>), dim3(team_grid), dim3(NW * 64), lds,
                       stream, prm);
    return hipGetLastError();
  }
  if (prm.nsplit > 1) {
    hipLaunchKernelGGL((longflow_decode_kernel<D, GP, NW, kModeSplit>), dim3(nblocks), dim3(NW * 64), lds,
                       stream, prm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int pairs = nblocks / prm.nsplit;
    const int nchunk = combine_chunks(prm.S);
    hipLaunchKernelGGL((longflow_combine_kernel<D, GP>), dim3(pairs * nchunk), dim3(kCombineThreads),
                       0, stream, prm, nchunk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(longflow_finalize_kernel, dim3((pairs + 255) / 256), dim3(256), 0, stream,
                       prm, pairs, nchunk);
  } else {
    hipLaunchKernelGGL((longflow_decode_kernel<D, GP, NW, kModeSingle>), dim3(grid), dim3(NW * 64), lds,
                       stream, prm);
  }
  return hipGetLastError();
}

template <int D, int GP>
hipError_t launch_dg(const DecodeParams& prm, int nw, int nblocks, size_t lds, int team_grid, int grid,
                     hipStream_t stream) {
  if (nw == kWavesLargeLds) return launch_dgw<D, GP, kWavesLargeLds>(prm, nblocks, lds, team_grid, grid, stream);
  if (nw == kWavesSmallLds) return launch_dgw<D, GP, kWavesSmallLds>(prm, nblocks, lds, team_grid, grid, stream);
  return hipErrorInvalidValue;
}

template <int D, int GP, int NW>
hipError_t occupancy_dgw(bool team, size_t lds, int* blocks) {
  const void* f = team ? reinterpret_cast<const void*>(&longflow_decode_kernel<D, GP, NW, kModeTeam>)
                       : reinterpret_cast<const void*>(&longflow_decode_kernel<D, GP, NW, kModeSingle>);
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, f, NW * 64, lds);
}

template <int D, int GP>
hipError_t occupancy_dg(bool team, int nw, size_t lds, int* blocks) {
  if (nw == kWavesLargeLds) return occupancy_dgw<D, GP, kWavesLargeLds>(team, lds, blocks);
  if (nw == kWavesSmallLds) return occupancy_dgw<D, GP, kWavesSmallLds>(team, lds, blocks);
  return hipErrorInvalidValue;
}

template <int D>
hipError_t occupancy_d(bool team, int gp, int nw, size_t lds, int* blocks) {
  switch (gp) {
    case 1: return occupancy_dg<D, 1>(team, nw, lds, blocks);
    case 2: return occupancy_dg<D, 2>(team, nw, lds, blocks);
    case 4: return occupancy_dg<D, 4>(team, nw, lds, blocks);
    case 8: return occupancy_dg<D, 8>(team, nw, lds, blocks);
    default: return hipErrorInvalidValue;
  }
}

static hipError_t query_blocks_per_cu(bool team, int d, int gp, int nw, size_t lds, int* blocks) {
  switch (d) {
    case 64: return occupancy_d<64>(team, gp, nw, lds, blocks);
    case 128: return occupancy_d<128>(team, gp, nw, lds, blocks);
    default: return hipErrorInvalidValue;
  }
}

// The occupancy query costs several microseconds of host time, as much as a
// small step's whole launch, and its answer depends only on the device and
// the kernel configuration: answers are kept per (device, configuration).
hipError_t decode_blocks_per_cu(bool team, int d, int gp, int nw, size_t lds, int* blocks) {
  struct Entry {
    int dev, team, d, gp, nw, blocks;
    size_t lds;
  };
  static std::mutex mu;
  static Entry cache[64];
  static int used = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i) {
      const Entry& c = cache[i];
      if (c.dev == dev && c.team == (int)team && c.d == d && c.gp == gp && c.nw == nw && c.lds == lds) {
        *blocks = c.blocks;
        return hipSuccess;
      }
    }
  }
  e = query_blocks_per_cu(team, d, gp, nw, lds, blocks);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if (used < 64) cache[used++] = Entry{dev, (int)team, d, gp, nw, *blocks, lds};
  return hipSuccess;
}

template <int D>
hipError_t launch_d(const DecodeParams& prm, int gp, int nw, int nblocks, size_t lds, int team_grid, int grid,
                    hipStream_t stream) {
  switch (gp) {
    case 1: return launch_dg<D, 1>(prm, nw, nblocks, lds, team_grid, grid, stream);
    case 2: return launch_dg<D, 2>(prm, nw, nblocks, lds, team_grid, grid, stream);
    case 4: return launch_dg<D, 4>(prm, nw, nblocks, lds, team_grid, grid, stream);
    case 8: return launch_dg<D, 8>(prm, nw, nblocks, lds, team_grid, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeParams& prm, int d, int gp, int nw, int nblocks, size_t lds,
                         int team_grid, int grid, hipStream_t stream) {
  switch (d) {
    case 64: return launch_d<64>(prm, gp, nw, nblocks, lds, team_grid, grid, stream);
    case 128: return launch_d<128>(prm, gp, nw, nblocks, lds, team_grid, grid, stream);
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
