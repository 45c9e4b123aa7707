// Read-bandwidth probe for gfx950 (benchmark context only; not part of the
// quantized-matmul library).  Every thread streams 16-byte loads over its
// share of a buffer with a grid-stride loop, several loads in flight, and
// folds them with XOR so the loads cannot be removed; one word per
// workgroup is written.  The bytes read per launch over the launch time is
// what plain streaming reads reach on this GPU, the figure beside the 8 TB/s
// peak.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kProbeThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void k_read_probe(const uint4* __restrict__ src,
                                                              int64_t n16, uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[kProbeThreads / 64];
  for (int d = 32; d > 0; d >>= 1) acc ^= __shfl_xor(acc, d, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    for (int k = 0; k < kProbeThreads / 64; ++k) a ^= red[k];
    out[blockIdx.x] = a;
  }
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) at src (16-byte aligned) with `workgroups`
// workgroups of 256 threads; writes one word per workgroup to out.  Returns
// 0, or the HIP error code of the launch.
int msq_probe_read(const void* src, int64_t bytes, uint32_t* out, int workgroups,
                   hipStream_t stream) {
  if (!src || !out || bytes <= 0 || bytes % 16 != 0 || workgroups <= 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15) != 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_read_probe, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, stream,
                     reinterpret_cast<const uint4*>(src), bytes / 16, out);
  return (int)hipGetLastError();
}

}  // extern "C"
