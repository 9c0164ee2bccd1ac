// Small helper kernel: fills.
#include "common.h"
#include "kernels.h"

namespace ls {

__global__ void k_fill_i32(int32_t* p, int n, int v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

void launch_fill_i32(int32_t* p, int n, int v, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_i32, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v);
}

}  // namespace ls
