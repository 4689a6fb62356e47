// Measurement helper, not a step of the layer: a plain streaming read of a
// device buffer.  Timed over a buffer far larger than the 256 MiB last-level
// cache, it gives the practical HBM read rate of the device, which the decode
// step's bandwidth is set against beside the 8 TB/s peak.
#include <hip/hip_runtime.h>

#include "../../include/moe.h"

namespace {

constexpr int PR_THREADS = 256;
constexpr int PR_UNROLL = 4;         // 16-byte loads in flight per thread per round
constexpr int PR_BLOCKS_PER_CU = 2;   // measured best of 1-16 with 256-1024 threads and 2-16 loads per thread

// Grid-stride rounds of PR_UNROLL loads per thread; the XOR of every 32-bit
// word keeps the loads live, one atomic per wave adds it to *sink.
__global__ __launch_bounds__(PR_THREADS) void hbm_read_kernel(const uint4* src, size_t n16, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * PR_THREADS;
  size_t i = (size_t)blockIdx.x * PR_THREADS + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + (PR_UNROLL - 1) * stride < n16; i += PR_UNROLL * stride) {
    uint4 v[PR_UNROLL];
#pragma unroll
    for (int u = 0; u < PR_UNROLL; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < PR_UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  if ((threadIdx.x & 63) == 0 && acc != 0u) atomicXor(sink, acc);
}

}  // namespace

extern "C" moe_status_t moe_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink) return MOE_E_NULLPTR;
  if (((uintptr_t)src & 15u) || (bytes & 15u) || ((uintptr_t)sink & 3u)) return MOE_E_ALIGN;
  if (bytes == 0) return MOE_OK;
  (void)hipGetLastError();
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return MOE_E_HIP;
  const size_t n16 = bytes / 16;
  size_t blocks = (n16 + (size_t)PR_THREADS * PR_UNROLL - 1) / ((size_t)PR_THREADS * PR_UNROLL);
  if (blocks > (size_t)cus * PR_BLOCKS_PER_CU) blocks = (size_t)cus * PR_BLOCKS_PER_CU;
  hipLaunchKernelGGL(hbm_read_kernel, dim3((unsigned)blocks), dim3(PR_THREADS), 0, (hipStream_t)stream,
                     (const uint4*)src, n16, sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
}
