// Embedding gather (the prelude P of Ouro-like models, LoopSpec page section 2.1) and row
// gathers of the hidden states.
#include "common.h"
#include "kernels.h"

namespace ls {

template <typename T>
__global__ __launch_bounds__(256) void k_embed(const T* emb, const int32_t* tokens, const int32_t* slot, int V, int d,
                                               long long S, float* H, int* err) {
  const int m = blockIdx.x;
  const int tok = tokens[m], sl = slot[m];
  if (sl < 0) return;                             // row rejected by validation
  if (tok < 0 || tok >= V || sl >= S) {
    if (threadIdx.x == 0) ls_flag(err, 1);
    return;
  }
  for (int i = threadIdx.x; i < d; i += 256) H[(size_t)sl * d + i] = Elem<T>::load(emb + (size_t)tok * d + i);
}

void launch_embed(bool bf16, const void* emb, const int32_t* tokens, const int32_t* slot, int M, int V, int d,
                  long long S, float* H, int* err, hipStream_t s) {
  if (bf16) hipLaunchKernelGGL(k_embed<uint16_t>, dim3(M), dim3(256), 0, s, (const uint16_t*)emb, tokens, slot, V, d, S, H, err);
  else hipLaunchKernelGGL(k_embed<float>, dim3(M), dim3(256), 0, s, (const float*)emb, tokens, slot, V, d, S, H, err);
}

__global__ __launch_bounds__(256) void k_gather(const float* H, const int32_t* slot, int d, long long S, float* out, int* err) {
  const int m = blockIdx.x;
  const int sl = slot[m];
  if (sl < 0 || sl >= S) {
    if (threadIdx.x == 0) ls_flag(err, 1);
    for (int i = threadIdx.x; i < d; i += 256) out[(size_t)m * d + i] = 0.f;
    return;
  }
  for (int i = threadIdx.x; i < d; i += 256) out[(size_t)m * d + i] = H[(size_t)sl * d + i];
}

void launch_gather(const float* H, const int32_t* slot, int M, int d, long long S, float* out, int* err, hipStream_t s) {
  hipLaunchKernelGGL(k_gather, dim3(M), dim3(256), 0, s, H, slot, d, S, out, err);
}

}  // namespace ls

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
