// Small helper kernels: fills and row validation.
#include "common.h"
#include "kernels.h"

namespace ls {

// Validates row descriptors: rows whose slot, depth, ancestor range or position is out of
// contract get slot -1 in the checked copy (every kernel skips such rows) and raise the
// error word.  dep_lo..dep_hi is the legal depth range (dep may be NULL).
__global__ void k_validate(int n, const int32_t* slot, const int32_t* dep, int dep_lo, int dep_hi, const int32_t* pos,
                           const int32_t* anc_off, int n_fin, int max_anc, long long S, int32_t* slot_ok,
                           int32_t* dep_ok, int32_t* row_ok, int* err) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int sl = slot[i];
  const int dp = dep ? dep[i] : dep_lo;
  const int a0 = anc_off[i], a1 = anc_off[i + 1];
  bool ok = sl >= 0 && sl < S && dp >= dep_lo && dp <= dep_hi && a0 >= 0 && a1 >= a0 && a1 - a0 <= max_anc;
  if (ok && pos) ok = pos[i] == n_fin + (a1 - a0);
  if (!ok) ls_flag(err, 1);
  slot_ok[i] = ok ? sl : -1;
  dep_ok[i] = ok ? dp : dep_lo;
  row_ok[i] = ok ? i : -1;
}

__global__ void k_fill_i32(int32_t* p, int n, int v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

void launch_fill_i32(int32_t* p, int n, int v, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_i32, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v);
}

void launch_validate(int n, const int32_t* slot, const int32_t* dep, int dep_lo, int dep_hi, const int32_t* pos,
                     const int32_t* anc_off, int n_fin, int max_anc, long long S, int32_t* slot_ok, int32_t* dep_ok,
                     int32_t* row_ok, int* err, hipStream_t s) {
  hipLaunchKernelGGL(k_validate, dim3((n + 127) / 128), dim3(128), 0, s, n, slot, dep, dep_lo, dep_hi, pos, anc_off, n_fin,
                     max_anc, S, slot_ok, dep_ok, row_ok, err);
}

}  // namespace ls
