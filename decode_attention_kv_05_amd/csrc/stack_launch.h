// Parameter blocks and launch entry points of the kernels around the
// operator in the multi-layer decode step (stack_kernels.hip), used by its
// host side (stack_api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lf {

// C[M][N] = A[M][K] W[N][K]^T (+ R[M][N] when r is set), all bf16; part is
// an fp32 workspace of gemm_partial_bytes(M, N, K) bytes.  K % 256 == 0;
// any M >= 1 and N >= 1 (rows go in blocks of 128, columns in blocks of 128).
struct GemmParams {
  const uint16_t* a;
  const uint16_t* w;
  const uint16_t* r;
  uint16_t* c;
  float* part;
  int M, N, K;
  int ksplit, kslice;  // set by launch_gemm
};
int gemm_ksplit(int N, int K);
size_t gemm_partial_bytes(int M, int N, int K);

// The QKV projection's output [B][(Hq + 2 Hkv) d] as q [B][Hq][d], k, v
// [B][Hkv][d], with q and k rotated (RoPE at pos): table[b][i] holds the
// (cos, sin) of pos[b] * base^(-2i/d), i < d/2, filled by launch_rope_table
// once per step (the positions hold for every layer of a step).
struct RopeParams {
  const int32_t* pos;
  float2* table;
  uint16_t* q;
  uint16_t* k;
  uint16_t* v;
  int B, Hq, Hkv, d;
  double log2_base;
};

// rope set: the epilogue writes q, k, v as RopeParams describes instead of C.
hipError_t launch_gemm(const GemmParams& prm, hipStream_t stream, const RopeParams* rope = nullptr);
hipError_t launch_rope_table(const RopeParams& rope, hipStream_t stream);
hipError_t launch_advance_pos(int32_t* pos, int n, hipStream_t stream);

}  // namespace lf
