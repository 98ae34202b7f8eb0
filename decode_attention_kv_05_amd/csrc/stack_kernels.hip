// Kernels of the multi-layer decode step around the LongFlow operator, for
// gfx950 (MI355X): the projections on the matrix cores, RoPE, and the step's
// position update.
//
// Source for the operator: "LongFlow: Efficient KV Cache Compression for
// Reasoning Models" (arXiv 2603.11504), Figure 1 caption (the attention
// module of a Qwen3-8B-shaped model at decode) and Figure 2 caption (one
// fused operator per attention call).  The layers around it are the
// ordinary ones of such a module: QKV projection, rotary position embedding
// of q and the new k, output projection with the residual.
//
// gemm_bf16_kernel<MT, NCH> + gemm_epilogue_kernel: C[M][N] = A[M][K] W[N][K]^T
// (+ R[M][N]), bf16 in and out, fp32 accumulation.  At decode M is the batch
// (up to 128 rows per workgroup; more rows take further row blocks) and the
// weights are the stream.  A workgroup of 4 wavefronts (one per SIMD) owns
// 128 columns, two 16-column tiles per wave, and one K slice of NCH 128-deep
// chunks; the slices (split-K) give about one workgroup per compute unit.
// v_mfma_f32_16x16x32_bf16 takes, in lane l, row (or column) l % 16 and the
// 8 k values 8 (l / 16) .. + 7 of each operand's 32-deep step and returns
// column l % 16, rows 4 (l / 16) .. + 3 of the 16 x 16 result.  The slices'
// fp32 partials go to a workspace; the epilogue kernel sums them, adds R and
// rounds to bf16.
//
// gemm_rope_epilogue_kernel takes the epilogue's place after the QKV
// projection: it splits each sequence's qkv row into q [Hq][d], k [Hkv][d]
// and v [Hkv][d] and rotates the q and k pairs (i, i + d/2) by
// pos * base^(-2i/d) (angle in fp64, rotation in fp32); rope_table_kernel
// computes the angles' cosines and sines once per step.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "launch.h"
#include "stack_launch.h"

namespace lf {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

constexpr int kGemmWaves = 4;                         // one per SIMD
constexpr int kGemmNT = 2;                            // 16-column tiles per wave
constexpr int kGemmCols = kGemmWaves * kGemmNT * 16;  // columns of a workgroup (128)
constexpr int kGemmChunk = 128;                       // k values per pipeline stage
constexpr int kGemmSteps = kGemmChunk / 32;           // 32-deep MFMA steps per stage
static_assert(kGemmSteps == kGemmWaves, "each wave stages one A fragment per row tile");

// Partial products of one K slice: P[ks][m][n] = sum over k in slice ks of
// A[m][k] W[n][k], for the workgroup's 128 columns and rows m0 .. m0 + 16 MT.
//
// A stage is one 128-deep chunk of A (all rows), staged in LDS in MFMA
// fragment order: fragment f = mt * 4 + s (row tile mt, 32-deep step s) is
// 64 lanes x 16 bytes, lane l holding A[16 mt + l % 16][32 s + 8 (l / 16)
// .. + 7].  A wave reads or writes a fragment as 1 KB of consecutive LDS,
// so no access has bank conflicts; each wave stages MT of the stage's 4 MT
// fragments.  Each wave owns two 16-column tiles, streams their weights
// from HBM two stages ahead of use, reads the next step's A fragments while
// the current step multiplies, and reuses every A fragment for both tiles.
//
// Per stage j: the loads of A chunk j + 1 and of the weights of chunk j + 2
// are issued first, then chunk j is multiplied, then A chunk j + 1 goes from
// registers to LDS; one barrier per stage.  Loads complete in issue order,
// so that last step waits for A chunk j + 1 and the loads before it (the
// weights of chunk j + 1, needed next) and leaves the weights of chunk j + 2
// in flight.  Every load is unconditional and the chunk loop is unrolled (NCH
// chunks per slice), so the compiler counts outstanding loads exactly and
// waits for no more than a step needs.
template <int MT, int NCH>
__global__ __launch_bounds__(kGemmWaves * 64) void gemm_bf16_kernel(GemmParams p) {
  __shared__ __align__(16) bf16x8_t frag[2][MT * kGemmSteps][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * kGemmCols + wave * (kGemmNT * 16);
  const int col = lane & 15;
  const int kq = (lane >> 4) * 8;
  const int k_begin = blockIdx.y * (NCH * kGemmChunk);
  const int m0 = blockIdx.z * (MT * 16);  // first row of this row block

  // Columns past N read row N - 1 and rows past M repeat row M - 1; their
  // products are dropped.
  const uint16_t* wrow[kGemmNT];
#pragma unroll
  for (int nt = 0; nt < kGemmNT; ++nt)
    wrow[nt] = p.w + (size_t)min(n0 + nt * 16 + col, p.N - 1) * p.K + k_begin + kq;
  // the A fragments this wave stages: f = wave + 4 i, i < MT
  const uint16_t* arow[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int f = wave + kGemmWaves * i;
    const int r = min(m0 + (f / kGemmSteps) * 16 + col, p.M - 1);
    arow[i] = p.a + (size_t)r * p.K + k_begin + (f % kGemmSteps) * 32 + kq;
  }

  bf16x8_t w[3][kGemmNT][kGemmSteps];  // chunk c's weights live in w[c % 3]
  bf16x8_t ar[MT];                      // A fragments of the next chunk
  auto load_w = [&](int c) {
#pragma unroll
    for (int nt = 0; nt < kGemmNT; ++nt)
#pragma unroll
      for (int s = 0; s < kGemmSteps; ++s)
        w[c % 3][nt][s] = *reinterpret_cast<const bf16x8_t*>(wrow[nt] + c * kGemmChunk + s * 32);
  };
  auto load_a = [&](int c) {
#pragma unroll
    for (int i = 0; i < MT; ++i) ar[i] = *reinterpret_cast<const bf16x8_t*>(arow[i] + c * kGemmChunk);
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < MT; ++i) frag[buf][wave + kGemmWaves * i][lane] = ar[i];
  };

  f32x4_t acc[MT][kGemmNT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < kGemmNT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  load_a(0);
  load_w(0);
  if (NCH > 1) load_w(1);
  store_a(0);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    // the next stage's loads go out before any arithmetic of this one
    if (j + 1 < NCH) load_a(j + 1);
    if (j + 2 < NCH) load_w(j + 2);
    __builtin_amdgcn_sched_barrier(0);
    const int buf = j & 1;
    bf16x8_t af[2][MT];  // A fragments of steps s and s + 1
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) af[0][mt] = frag[buf][mt * kGemmSteps][lane];
#pragma unroll
    for (int s = 0; s < kGemmSteps; ++s) {
      if (s + 1 < kGemmSteps) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) af[(s + 1) & 1][mt] = frag[buf][mt * kGemmSteps + s + 1][lane];
      }
      __builtin_amdgcn_sched_barrier(0);  // keep those reads ahead of this step's products
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < kGemmNT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s & 1][mt], w[j % 3][nt][s], acc[mt][nt], 0, 0, 0);
    }
    if (j + 1 < NCH) {
      store_a(buf ^ 1);
      __syncthreads();
    }
  }

  float* part = p.part + (size_t)blockIdx.y * p.M * p.N;
#pragma unroll
  for (int nt = 0; nt < kGemmNT; ++nt) {
    const int n = n0 + nt * 16 + col;
    if (n >= p.N) continue;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + mt * 16 + (lane >> 4) * 4 + r;
        if (m < p.M) part[(size_t)m * p.N + n] = acc[mt][nt][r];
      }
    }
  }
}

// C = bf16(sum of the K-slice partials (+ R)), four columns per thread.
__global__ void gemm_epilogue_kernel(GemmParams p) {
  const size_t n4 = (size_t)p.M * p.N / 4;
  const size_t plane = (size_t)p.M * p.N;
  for (size_t t = blockIdx.x * (size_t)blockDim.x + threadIdx.x; t < n4; t += (size_t)gridDim.x * blockDim.x) {
    float4 s = reinterpret_cast<const float4*>(p.part)[t];
    for (int ks = 1; ks < p.ksplit; ++ks) {
      const float4 x = reinterpret_cast<const float4*>(p.part + ks * plane)[t];
      s.x += x.x;
      s.y += x.y;
      s.z += x.z;
      s.w += x.w;
    }
    if (p.r) {
      const uint2 r = reinterpret_cast<const uint2*>(p.r)[t];
      s.x += bf16_to_f32((uint16_t)(r.x & 0xffffu));
      s.y += bf16_to_f32((uint16_t)(r.x >> 16));
      s.z += bf16_to_f32((uint16_t)(r.y & 0xffffu));
      s.w += bf16_to_f32((uint16_t)(r.y >> 16));
    }
    uint2 o;
    o.x = (uint32_t)f32_to_bf16_rne(s.x) | ((uint32_t)f32_to_bf16_rne(s.y) << 16);
    o.y = (uint32_t)f32_to_bf16_rne(s.z) | ((uint32_t)f32_to_bf16_rne(s.w) << 16);
    reinterpret_cast<uint2*>(p.c)[t] = o;
  }
}

// The step's rotations: table[b][i] = (cos, sin) of pos[b] * base^(-2i/d),
// angle in fp64, rounded to fp32.
__global__ void rope_table_kernel(RopeParams p) {
  const int half = p.d / 2;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= p.B * half) return;
  const int b = t / half, i = t - b * half;
  const double ang = (double)p.pos[b] * exp2(-(2.0 * i / p.d) * p.log2_base);
  double sn, cs;
  sincos(ang, &sn, &cs);
  p.table[t] = make_float2((float)cs, (float)sn);
}

// The QKV projection's epilogue: sums the K-slice partials of columns
// h d + i and h d + i + d/2 of head h (i < d/2), four values of i per
// thread, rounds them to bf16 (the projection's output precision), rotates
// the pairs of query and key heads by the step's table (in fp32) and writes
// q, k and v head by head.
__global__ void gemm_rope_epilogue_kernel(GemmParams g, RopeParams p) {
  const int half = p.d / 2, quads = half / 4;
  const int heads = p.Hq + 2 * p.Hkv;
  const size_t plane = (size_t)g.M * g.N;
  const size_t total = (size_t)p.B * heads * quads;
  for (size_t t = blockIdx.x * (size_t)blockDim.x + threadIdx.x; t < total;
       t += (size_t)gridDim.x * blockDim.x) {
    const int i = (int)(t % quads) * 4;
    const size_t bh = t / quads;
    const int h = (int)(bh % heads);
    const int b = (int)(bh / heads);
    const float* src = g.part + (size_t)b * g.N + (size_t)h * p.d + i;
    float4 s0 = *reinterpret_cast<const float4*>(src), s1 = *reinterpret_cast<const float4*>(src + half);
    for (int ks = 1; ks < g.ksplit; ++ks) {
      const float4 x0 = *reinterpret_cast<const float4*>(src + ks * plane);
      const float4 x1 = *reinterpret_cast<const float4*>(src + ks * plane + half);
      s0.x += x0.x;
      s0.y += x0.y;
      s0.z += x0.z;
      s0.w += x0.w;
      s1.x += x1.x;
      s1.y += x1.y;
      s1.z += x1.z;
      s1.w += x1.w;
    }
    uint16_t x0[4] = {f32_to_bf16_rne(s0.x), f32_to_bf16_rne(s0.y), f32_to_bf16_rne(s0.z), f32_to_bf16_rne(s0.w)};
    uint16_t x1[4] = {f32_to_bf16_rne(s1.x), f32_to_bf16_rne(s1.y), f32_to_bf16_rne(s1.z), f32_to_bf16_rne(s1.w)};
    uint16_t* dst;
    if (h < p.Hq) {
      dst = p.q + ((size_t)b * p.Hq + h) * p.d;
    } else if (h < p.Hq + p.Hkv) {
      dst = p.k + ((size_t)b * p.Hkv + (h - p.Hq)) * p.d;
    } else {
      dst = p.v + ((size_t)b * p.Hkv + (h - p.Hq - p.Hkv)) * p.d;
    }
    if (h < p.Hq + p.Hkv) {
      const float4* tab = reinterpret_cast<const float4*>(p.table + (size_t)b * half + i);
      const float4 c01 = tab[0], c23 = tab[1];
      const float cf[4] = {c01.x, c01.z, c23.x, c23.z}, sf[4] = {c01.y, c01.w, c23.y, c23.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = bf16_to_f32(x0[j]), bb = bf16_to_f32(x1[j]);
        x0[j] = f32_to_bf16_rne(a * cf[j] - bb * sf[j]);
        x1[j] = f32_to_bf16_rne(bb * cf[j] + a * sf[j]);
      }
    }
    *reinterpret_cast<uint2*>(dst + i) = make_uint2(x0[0] | ((uint32_t)x0[1] << 16), x0[2] | ((uint32_t)x0[3] << 16));
    *reinterpret_cast<uint2*>(dst + i + half) =
        make_uint2(x1[0] | ((uint32_t)x1[1] << 16), x1[2] | ((uint32_t)x1[3] << 16));
  }
}

__global__ void advance_pos_kernel(int32_t* pos, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) pos[i] += 1;
}

// Workgroups the K slices aim for (a 256-CU device); more slices keep more
// compute units streaming weights but add fp32 partials to write and read.
constexpr int kGemmTargetWorkgroups = 256;

int gemm_ksplit(int N, int K) {
  const int blocks = (N + kGemmCols - 1) / kGemmCols;
  const int pieces = K / (2 * kGemmChunk);  // 256-deep pieces; a slice is a whole number of them
  // the fewest slices of at most 8 pieces (16 chunks, the longest unrolled slice) ...
  int ks = 1;
  while (pieces / ks > 8 || pieces % ks != 0) ++ks;
  // ... then more slices while the grid stays within the workgroup target
  for (int c = ks + 1; c <= pieces && blocks * c <= kGemmTargetWorkgroups; ++c)
    if (pieces % c == 0) ks = c;
  return ks;
}

size_t gemm_partial_bytes(int M, int N, int K) { return (size_t)gemm_ksplit(N, K) * M * N * 4; }

hipError_t launch_gemm(const GemmParams& in, hipStream_t stream, const RopeParams* rope) {
  GemmParams prm = in;
  prm.ksplit = gemm_ksplit(prm.N, prm.K);
  prm.kslice = prm.K / prm.ksplit;
  // Up to 128 rows per workgroup; more rows take further row blocks (grid z),
  // each of which streams the weights again.
  const int tiles = (prm.M + 15) / 16;
  const int mt = tiles <= 2 ? 2 : tiles <= 4 ? 4 : 8;
  const dim3 grid((prm.N + kGemmCols - 1) / kGemmCols, prm.ksplit, (tiles + mt - 1) / mt);
  const dim3 block(kGemmWaves * 64);
  if (prm.M < 1 || grid.z > 65535) return hipErrorInvalidValue;
  const int nch = prm.kslice / kGemmChunk;  // even, 2 .. 16
  if (prm.K != prm.ksplit * prm.kslice || nch < 2 || nch > 16 || nch % 2 != 0) return hipErrorInvalidValue;
#define LF_GEMM_LAUNCH(MT_, NCH_) \
  case NCH_: hipLaunchKernelGGL((gemm_bf16_kernel<MT_, NCH_>), grid, block, 0, stream, prm); break;
#define LF_GEMM_BY_NCH(MT_)                                                                  \
  switch (nch) {                                                                             \
    LF_GEMM_LAUNCH(MT_, 2) LF_GEMM_LAUNCH(MT_, 4) LF_GEMM_LAUNCH(MT_, 6) LF_GEMM_LAUNCH(MT_, 8) \
    LF_GEMM_LAUNCH(MT_, 10) LF_GEMM_LAUNCH(MT_, 12) LF_GEMM_LAUNCH(MT_, 14)                    \
    LF_GEMM_LAUNCH(MT_, 16)                                                                  \
  }
  if (mt == 2) {
    LF_GEMM_BY_NCH(2)
  } else if (mt == 4) {
    LF_GEMM_BY_NCH(4)
  } else {
    LF_GEMM_BY_NCH(8)
  }
#undef LF_GEMM_BY_NCH
#undef LF_GEMM_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (rope) {
    const size_t total = (size_t)rope->B * (rope->Hq + 2 * rope->Hkv) * (rope->d / 8);
    size_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(gemm_rope_epilogue_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, prm, *rope);
    return hipGetLastError();
  }
  size_t blocks = ((size_t)prm.M * prm.N / 4 + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(gemm_epilogue_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, prm);
  return hipGetLastError();
}

hipError_t launch_rope_table(const RopeParams& rope, hipStream_t stream) {
  const int n = rope.B * (rope.d / 2);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, rope);
  return hipGetLastError();
}

hipError_t launch_advance_pos(int32_t* pos, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(advance_pos_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, pos, n);
  return hipGetLastError();
}

}  // namespace lf
