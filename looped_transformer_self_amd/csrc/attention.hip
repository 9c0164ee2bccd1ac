// Branch-masked decode attention over the paged, depth-indexed KV cache.
//
// Row i attends, at its own loop depth, to the finished prefix, its speculative ancestors
// (the branch mask) and itself (LoopSpec page, section 2.2 and 2.4: per-branch, per-depth KV,
// children reuse the parent's prefix by index).  Work is split over (key chunk, head, row);
// each chunk produces (max, sum, unnormalised output) and a second kernel merges the chunks
// with the log-sum-exp rule.  Within a chunk, 16 lanes share one key: lane group kk = lane/16
// takes a key, lane e = lane%16 holds 8 consecutive head dimensions, so every load instruction
// reads four whole key (or value) vectors; dot products reduce over the 16 lanes with shuffles.
#include "common.h"
#include "kernels.h"

namespace ls {

template <typename T>
LS_DEV void load8(const T* p, float* v);
template <>
LS_DEV void load8<uint16_t>(const uint16_t* p, float* v) {
  const u32x4_t x = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(x[i] << 16);
    v[2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u);
  }
}
template <>
LS_DEV void load8<float>(const float* p, float* v) {
  const u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(p);
  const u32x4_t x1 = *reinterpret_cast<const u32x4_t*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = __uint_as_float(x0[i]); v[4 + i] = __uint_as_float(x1[i]); }
}

template <typename T>
__global__ __launch_bounds__(256) void k_attn_chunk(AttnArgs a) {
  const int c = blockIdx.x, h = blockIdx.y, i = blockIdx.z;
  if (a.slot[i] < 0) return;                    // row rejected by validation
  const int n_anc = a.anc_off[i + 1] - a.anc_off[i];
  const int nk = a.n_fin + n_anc + 1;
  const int k0 = c * ATTN_CHUNK;
  if (k0 >= nk) return;
  const int kn = min(ATTN_CHUNK, nk - k0);
  const int self = a.slot[i];
  const int a0 = a.anc_off[i];
  const int blk = (a.kv.dep ? a.kv.dep[i] + a.kv.dep_off : 0) * a.kv.blk_mul + a.kv.layer;
  const T* cache = (const T*)a.kv.base + (size_t)blk * a.kv.S * 2 * a.d;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int kk = lane >> 4, e = lane & 15;
  const bool dim_ok = 8 * e < a.hd;
  const float scale = 1.0f / sqrtf((float)a.hd);

  __shared__ float s_p[ATTN_CHUNK];
  __shared__ int s_slot[ATTN_CHUNK];
  __shared__ float red[4];
  __shared__ float s_acc[4][128];

  for (int j = threadIdx.x; j < kn; j += 256) {
    int sl = key_slot(k0 + j, a.n_fin, a.fin, a.anc, a0, n_anc, self);
    if (sl < 0 || sl >= a.kv.S) { ls_flag(a.err, 1); sl = -1; }
    s_slot[j] = sl;
  }
  float q[8];
  if (dim_ok) {
#pragma unroll
    for (int t = 0; t < 8; ++t) q[t] = a.q[(size_t)i * a.d + h * a.hd + 8 * e + t] * scale;
  }
  __syncthreads();

  // scores: wave wv handles keys wv*4 + kk, +16, ...
  float mloc = -INFINITY;
  for (int j = wv * 4 + kk; j < kn; j += 16) {
    const int sl = s_slot[j];
    float part = 0.f;
    if (dim_ok && sl >= 0) {
      float kv8[8];
      load8<T>(cache + (size_t)sl * 2 * a.d + h * a.hd + 8 * e, kv8);
#pragma unroll
      for (int t = 0; t < 8; ++t) part += q[t] * kv8[t];
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
    const float sc = sl >= 0 ? part : -INFINITY;
    if (e == 0) s_p[j] = sc;
    mloc = fmaxf(mloc, sc);
  }
  const float mx = block_max(mloc, red);
  float lsum = 0.f;
  for (int j = threadIdx.x; j < kn; j += 256) {
    const float p = s_p[j] == -INFINITY ? 0.f : __expf(s_p[j] - mx);
    s_p[j] = p;
    lsum += p;
  }
  const float l = block_sum(lsum, red);   // block_sum syncs, so s_p is complete below

  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int j = wv * 4 + kk; j < kn; j += 16) {
    const int sl = s_slot[j];
    if (!dim_ok || sl < 0) continue;
    const float p = s_p[j];
    float v8[8];
    load8<T>(cache + (size_t)sl * 2 * a.d + a.d + h * a.hd + 8 * e, v8);
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] += p * v8[t];
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    acc[t] += __shfl_xor(acc[t], 16, 64);
    acc[t] += __shfl_xor(acc[t], 32, 64);
  }
  if (kk == 0 && dim_ok) {
#pragma unroll
    for (int t = 0; t < 8; ++t) s_acc[wv][8 * e + t] = acc[t];
  }
  __syncthreads();
  float* out = a.part + (((size_t)i * a.n_heads + h) * a.max_chunks + c) * (a.hd + 2);
  for (int dd = threadIdx.x; dd < a.hd; dd += 256) out[2 + dd] = s_acc[0][dd] + s_acc[1][dd] + s_acc[2][dd] + s_acc[3][dd];
  if (threadIdx.x == 0) { out[0] = mx; out[1] = l; }
}

template <typename T>
__global__ __launch_bounds__(128) void k_attn_combine(AttnArgs a) {
  const int h = blockIdx.x, i = blockIdx.y;
  if (a.slot[i] < 0) {
    for (int dd = threadIdx.x; dd < a.hd; dd += blockDim.x) Elem<T>::store((T*)a.o + (size_t)i * a.d + h * a.hd + dd, 0.f);
    return;
  }
  const int nk = a.n_fin + (a.anc_off[i + 1] - a.anc_off[i]) + 1;
  const int nc = (nk + ATTN_CHUNK - 1) / ATTN_CHUNK;
  const float* base = a.part + ((size_t)i * a.n_heads + h) * a.max_chunks * (a.hd + 2);
  float mx = -INFINITY;
  for (int c = 0; c < nc; ++c) mx = fmaxf(mx, base[c * (a.hd + 2)]);
  for (int dd = threadIdx.x; dd < a.hd; dd += blockDim.x) {
    float num = 0.f, den = 0.f;
    for (int c = 0; c < nc; ++c) {
      const float* pc = base + c * (a.hd + 2);
      const float w = pc[0] == -INFINITY ? 0.f : __expf(pc[0] - mx);
      den += w * pc[1];
      num += w * pc[2 + dd];
    }
    Elem<T>::store((T*)a.o + (size_t)i * a.d + h * a.hd + dd, den > 0.f ? num / den : 0.f);
  }
}

void launch_attention(bool bf16, const AttnArgs& a, hipStream_t s) {
  dim3 g1(a.grid_chunks, a.n_heads, a.M), g2(a.n_heads, a.M);
  if (bf16) {
    hipLaunchKernelGGL(k_attn_chunk<uint16_t>, g1, dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_attn_combine<uint16_t>, g2, dim3(128), 0, s, a);
  } else {
    hipLaunchKernelGGL(k_attn_chunk<float>, g1, dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_attn_combine<float>, g2, dim3(128), 0, s, a);
  }
}

}  // namespace ls
