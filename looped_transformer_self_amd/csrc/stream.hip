// Streaming-read reference: the achievable HBM read rate of the loads the layer kernel's
// producer waves issue (16-byte direct-to-LDS loads, non-temporal, 1 KB per wave
// instruction, 16 in flight per wave, two waves per workgroup, one workgroup per CU), with
// no consumers.  A measurement aid for the roofline of ls_loop_step; nothing in the decode
// path calls it.
#include <hip/hip_runtime.h>

#include "../../include/loopspec.h"

namespace ls {
namespace {

constexpr int SW_WAVES = 2, SW_DEPTH = 16, SW_CHUNK = 1024;

template <int N>
__device__ __forceinline__ void sw_wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup b reads bytes [b * per_wg, (b + 1) * per_wg) of src, its two waves each half of
// that, 1 KB per instruction into a 16 KB LDS ring per wave; the ring is never read.
__global__ __launch_bounds__(64 * SW_WAVES) void k_stream_read(const char* __restrict__ src, long long per_wg) {
  __shared__ __attribute__((aligned(16))) char ring[SW_WAVES][SW_DEPTH][SW_CHUNK];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long long per_wave = per_wg / SW_WAVES;
  const char* p = src + (long long)blockIdx.x * per_wg + (long long)w * per_wave + lane * 16;
  const long long n = per_wave / SW_CHUNK;
  for (long long i = 0; i < n; ++i) {
    __builtin_amdgcn_global_load_lds(p + i * SW_CHUNK, (__attribute__((address_space(3))) void*)&ring[w][i & (SW_DEPTH - 1)][0],
                                     16, 0, 2);
    if (i >= SW_DEPTH) sw_wait_vm<SW_DEPTH>();
  }
  sw_wait_vm<0>();
}

}  // namespace
}  // namespace ls

extern "C" ls_status ls_measure_stream_read(const void* src, size_t bytes, int n_workgroups, hipStream_t stream) {
  const size_t unit = (size_t)n_workgroups * ls::SW_WAVES * ls::SW_CHUNK;
  if (!src || n_workgroups <= 0 || bytes == 0 || bytes % unit)
    return LS_ERR_INVALID;
  hipLaunchKernelGGL(ls::k_stream_read, dim3(n_workgroups), dim3(64 * ls::SW_WAVES), 0, stream, (const char*)src,
                     (long long)(bytes / n_workgroups));
  return hipGetLastError() == hipSuccess ? LS_OK : LS_ERR_HIP;
}
