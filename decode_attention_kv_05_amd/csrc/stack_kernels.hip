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
// gemm_bf16_kernel<MT> + gemm_epilogue_kernel: C[M][N] = A[M][K] W[N][K]^T
// (+ R[M][N]), bf16 in and out, fp32 accumulation.  At decode M is the batch
// (at most 16 * MT rows) and the weights are the stream.  A workgroup of 8
// wavefronts owns 128 columns (a 16-column slab per wave) and one K slice;
// the slices (split-K, whole 256-deep super-chunks) give about one
// workgroup per compute unit.  Each 128-deep chunk of A (all rows) is staged
// once in LDS, double-buffered, and shared by the 8 waves; each wave streams
// its slab's weights from HBM a 256-deep super-chunk ahead of their use and
// runs v_mfma_f32_16x16x32_bf16 per 32-deep step and 16-row tile.  Lane l
// supplies row (or column) l % 16 and the 8 k-values 8 * (l / 16) .. + 7 of
// both operands and receives column l % 16, rows 4 * (l / 16) .. + 3 of the
// 16 x 16 result.  The slices' fp32 partials go to a workspace; the epilogue
// kernel sums them, adds R and rounds to bf16.
//
// rope_split_kernel: splits each sequence's qkv row into q [Hq][d],
// k [Hkv][d] and v [Hkv][d]; q and k pairs (i, i + d/2) are rotated by
// pos * base^(-2i/d) (angle in fp64, rotation in fp32).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "launch.h"

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

#ifndef LF_GEMM_WAVES
#define LF_GEMM_WAVES 8
#endif
constexpr int kGemmWaves = LF_GEMM_WAVES;  // one 16-column slab each
constexpr int kGemmCols = kGemmWaves * 16;  // columns of a workgroup
constexpr int kGemmChunk = 128;             // k values of A staged per round
#ifndef LF_GEMM_PAD
#define LF_GEMM_PAD 8
#endif
constexpr int kGemmPad = LF_GEMM_PAD;       // bf16 padding of an LDS row

// Partial products of one K slice: P[ks][m][n] = sum over k in slice ks of
// A[m][k] W[n][k], for the workgroup's 128 columns and every row of A.
template <int MT>
__global__ __launch_bounds__(kGemmWaves * 64) void gemm_bf16_kernel(GemmParams p) {
  __shared__ __align__(16) uint16_t as[2][MT * 16][kGemmChunk + kGemmPad];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n0 = blockIdx.x * kGemmCols + wave * 16;
  const bool live = n0 < p.N;  // dead waves still stage A and meet the barriers
  const int col = lane & 15;
  const int kq = (lane >> 4) * 8;
  const int k_begin = blockIdx.y * p.kslice;
  const uint16_t* wrow = p.w + (size_t)(live ? n0 + col : 0) * p.K + kq;

  // staging map: thread -> (row, 8 k values) of a 128-deep chunk of A, in
  // MT * 16 / 32 passes of 32 rows
  constexpr int kRowsPerPass = kGemmWaves * 64 / (kGemmChunk / 8);  // 32
  auto stage = [&](int buf, int k0) {
#pragma unroll
    for (int r0 = 0; r0 < MT * 16; r0 += kRowsPerPass) {
      const int r = r0 + tid / (kGemmChunk / 8);
      const int c8 = (tid % (kGemmChunk / 8)) * 8;
      const uint16_t* src = p.a + (size_t)min(r, p.M - 1) * p.K + k0 + c8;
      *reinterpret_cast<uint4*>(&as[buf][r][c8]) = *reinterpret_cast<const uint4*>(src);
    }
  };
  constexpr int SPC = kGemmChunk / 32;  // 32-deep steps per A chunk
  // Weights are loaded a super-chunk (two A chunks, 256 k) at a time: eight
  // 16-byte loads per lane, issued a whole super-chunk ahead of their use.
  auto load_w = [&](bf16x8_t (&b)[2 * SPC], int k0) {
#pragma unroll
    for (int s = 0; s < 2 * SPC; ++s)
      b[s] = live ? *reinterpret_cast<const bf16x8_t*>(wrow + k0 + s * 32) : bf16x8_t{};
  };

  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // products of one A chunk (LDS buffer `buf`) with weights b[half * SPC ..]
  auto compute = [&](const bf16x8_t (&b)[2 * SPC], int half, int buf) {
#pragma unroll
    for (int s = 0; s < SPC; ++s) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&as[buf][mt * 16 + col][s * 32 + kq]);
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[half * SPC + s], acc[mt], 0, 0, 0);
      }
    }
  };

  // A chunk j of the slice lives in LDS buffer j & 1 and is staged while
  // chunk j - 1 is multiplied.  Super-chunks alternate between two weight
  // register sets (the loop is unrolled by two super-chunks).
  constexpr int KS = 2 * kGemmChunk;
  const int nsuper = p.kslice / KS;
  bf16x8_t b0[2 * SPC], b1[2 * SPC];
  load_w(b0, k_begin);
  stage(0, k_begin);
  __syncthreads();
  for (int sc = 0; sc < nsuper; sc += 2) {
    const int k0 = k_begin + sc * KS;
    const bool next = sc + 1 < nsuper;
    if (next) load_w(b1, k0 + KS);
    stage(1, k0 + kGemmChunk);
    compute(b0, 0, 0);
    __syncthreads();
    if (next) stage(0, k0 + KS);
    compute(b0, 1, 1);
    __syncthreads();
    if (!next) break;
    const bool next2 = sc + 2 < nsuper;
    if (next2) load_w(b0, k0 + 2 * KS);
    stage(1, k0 + KS + kGemmChunk);
    compute(b1, 0, 0);
    __syncthreads();
    if (next2) stage(0, k0 + 2 * KS);
    compute(b1, 1, 1);
    __syncthreads();
  }
  if (!live) return;
  float* part = p.part + (size_t)blockIdx.y * p.M * p.N;
  const int n = n0 + col;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = mt * 16 + (lane >> 4) * 4 + r;
      if (m < p.M) part[(size_t)m * p.N + n] = acc[mt][r];
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

__global__ void rope_split_kernel(RopeParams p) {
  const int half = p.d / 2;
  const int heads = p.Hq + 2 * p.Hkv;
  const size_t total = (size_t)p.B * heads * half;
  for (size_t t = blockIdx.x * (size_t)blockDim.x + threadIdx.x; t < total;
       t += (size_t)gridDim.x * blockDim.x) {
    const int i = (int)(t % half);
    const size_t bh = t / half;
    const int h = (int)(bh % heads);
    const int b = (int)(bh / heads);
    const uint16_t* src = p.qkv + ((size_t)b * heads + h) * p.d;
    const uint16_t x0 = src[i], x1 = src[i + half];
    if (h >= p.Hq + p.Hkv) {
      uint16_t* dst = p.v + ((size_t)b * p.Hkv + (h - p.Hq - p.Hkv)) * p.d;
      dst[i] = x0;
      dst[i + half] = x1;
      continue;
    }
    const double ang = (double)p.pos[b] * exp2(-(2.0 * i / p.d) * p.log2_base);
    double s, c;
    sincos(ang, &s, &c);
    const float cf = (float)c, sf = (float)s;
    const float a = bf16_to_f32(x0), bb = bf16_to_f32(x1);
    uint16_t* dst = h < p.Hq ? p.q + ((size_t)b * p.Hq + h) * p.d
                             : p.k + ((size_t)b * p.Hkv + (h - p.Hq)) * p.d;
    dst[i] = f32_to_bf16_rne(a * cf - bb * sf);
    dst[i + half] = f32_to_bf16_rne(bb * cf + a * sf);
  }
}

__global__ void advance_pos_kernel(int32_t* pos, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) pos[i] += 1;
}

// Workgroups the K slices aim for (a 256-CU device); more slices keep more
// compute units streaming weights but add fp32 partials to write and read.
#ifndef LF_GEMM_TARGET_WG
#define LF_GEMM_TARGET_WG 256
#endif

int gemm_ksplit(int N, int K) {
  const int blocks = (N + kGemmCols - 1) / kGemmCols;
  const int chunks = K / (2 * kGemmChunk);  // slices are whole 256-deep super-chunks
  int ks = 1;
  while (ks * 2 <= chunks && chunks % (ks * 2) == 0 && blocks * ks * 2 <= LF_GEMM_TARGET_WG) ks *= 2;
  return ks;
}

size_t gemm_partial_bytes(int M, int N, int K) { return (size_t)gemm_ksplit(N, K) * M * N * 4; }

hipError_t launch_gemm(const GemmParams& in, hipStream_t stream) {
  GemmParams prm = in;
  prm.ksplit = gemm_ksplit(prm.N, prm.K);
  prm.kslice = prm.K / prm.ksplit;
  const dim3 grid((prm.N + kGemmCols - 1) / kGemmCols, prm.ksplit), block(kGemmWaves * 64);
  const int tiles = (prm.M + 15) / 16;
  if (tiles <= 2) hipLaunchKernelGGL(gemm_bf16_kernel<2>, grid, block, 0, stream, prm);
  else if (tiles <= 4) hipLaunchKernelGGL(gemm_bf16_kernel<4>, grid, block, 0, stream, prm);
  else if (tiles <= 8) hipLaunchKernelGGL(gemm_bf16_kernel<8>, grid, block, 0, stream, prm);
  else if (tiles <= 16) hipLaunchKernelGGL(gemm_bf16_kernel<16>, grid, block, 0, stream, prm);
  else return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  size_t blocks = ((size_t)prm.M * prm.N / 4 + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(gemm_epilogue_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, prm);
  return hipGetLastError();
}

hipError_t launch_rope_split(const RopeParams& prm, hipStream_t stream) {
  const size_t total = (size_t)prm.B * (prm.Hq + 2 * prm.Hkv) * (prm.d / 2);
  if (total == 0) return hipSuccess;
  size_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(rope_split_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, prm);
  return hipGetLastError();
}

hipError_t launch_advance_pos(int32_t* pos, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(advance_pos_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, pos, n);
  return hipGetLastError();
}

}  // namespace lf
