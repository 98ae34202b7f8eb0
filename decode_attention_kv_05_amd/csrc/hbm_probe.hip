// Read-bandwidth probes for the benchmark (measurement only; not part of
// liblongflow.so).  Built into libhbm_probe.so; called through ctypes.
//
//   int lf_probe_read_interleaved(const void* p, size_t bytes, uint32_t* sink, void* stream)
//       the whole grid walks [p, p + bytes) in address order: 256 workgroups
//       of 256 threads, 8 non-temporal 16-byte loads in flight per thread,
//       consecutive threads on consecutive 16-byte chunks (the best pattern
//       of a sweep over workgroup size, count and loads in flight).
//   int lf_probe_read_pairs(const void* k, const void* v, int pairs, int pair_bytes,
//                           uint32_t* sink, void* stream)
//       the decode's pattern without its arithmetic: one workgroup of 8 waves
//       per (sequence, KV head) pair, streaming the pair's K rows, then its V
//       rows, in 4 KB wave batches (4 x 1 KB loads), with the same LDS
//       footprint per workgroup as the one-split decode kernel at 3200 slots
//       and 4 query heads per KV head, so two workgroups share a compute unit.
// Both return 0, or -1 when the launch fails.  `sink` (>= 4 KB of device
// memory) receives a word only if the data XOR to a marker, which keeps the
// loads from being removed.  bytes and pair_bytes must be multiples of 16;
// every buffer stays below 2^31 bytes per buffer resource.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr uint32_t kMarker = 0x9e3779b9u;
constexpr int kPolicyNt = 2;

__global__ __launch_bounds__(256) void read_interleaved(const uint4* __restrict__ p, size_t n16, uint32_t* sink) {
  constexpr int U = 8;
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  // The buffer resource covers at most 2^31 - 1 bytes; the host splits
  // larger reads.
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)p, 0, (int)(n16 * 16), 0x00020000);
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4_t x[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      x[u] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)((i + u * stride) * 16), 0, kPolicyNt);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 x = p[i];
    acc ^= x.x ^ x.y ^ x.z ^ x.w;
  }
  if (acc == kMarker) sink[blockIdx.x & 1023] = acc;
}

__global__ __launch_bounds__(512) void read_pairs(const char* __restrict__ k, const char* __restrict__ v,
                                                  int pair_bytes, uint32_t* sink) {
  constexpr int U = 4;
  extern __shared__ char lds[];
  const int nw = blockDim.x / 64, w = threadIdx.x / 64, lane = threadIdx.x & 63;
  uint32_t acc = 0;
  for (int pass = 0; pass < 2; ++pass) {
    const char* base = (pass ? v : k) + (size_t)blockIdx.x * pair_bytes;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, pair_bytes, 0x00020000);
    const int nbatch = (pair_bytes + nw * U * 1024 - 1) / (nw * U * 1024);
    for (int bi = 0; bi < nbatch; ++bi) {
      u32x4_t x[U];
      const int off0 = (bi * nw + w) * U * 1024 + lane * 16;  // past the end: zero, no access
#pragma unroll
      for (int u = 0; u < U; ++u) x[u] = __builtin_amdgcn_raw_buffer_load_b128(r, off0 + u * 1024, 0, kPolicyNt);
#pragma unroll
      for (int u = 0; u < U; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
    }
    if (threadIdx.x == 0) lds[0] = (char)acc;
    __syncthreads();
  }
  if (acc == kMarker) sink[blockIdx.x & 1023] = acc + (uint32_t)lds[1];
}

}  // namespace

extern "C" int lf_probe_read_interleaved(const void* p, size_t bytes, uint32_t* sink, void* stream) {
  const size_t chunk = (size_t)1 << 30;  // per launch, within one buffer resource
  for (size_t off = 0; off < bytes; off += chunk) {
    const size_t n = bytes - off < chunk ? bytes - off : chunk;
    hipLaunchKernelGGL(read_interleaved, dim3(256), dim3(256), 0, static_cast<hipStream_t>(stream),
                       reinterpret_cast<const uint4*>(static_cast<const char*>(p) + off), n / 16, sink);
    if (hipGetLastError() != hipSuccess) return -1;
  }
  return 0;
}

extern "C" int lf_probe_read_pairs(const void* k, const void* v, int pairs, int pair_bytes, uint32_t* sink,
                                   void* stream) {
  // the one-split decode kernel's LDS at 3200 slots and 4 query heads per KV head
  const size_t lds = (size_t)(3200 + 128) * 4 * 4 + (3200 + 128) + 1024;
  hipLaunchKernelGGL(read_pairs, dim3(pairs), dim3(512), lds, static_cast<hipStream_t>(stream),
                     static_cast<const char*>(k), static_cast<const char*>(v), pair_bytes, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
