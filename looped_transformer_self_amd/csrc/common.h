// Device helpers shared by the libloopspec kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define LS_DEV __device__ __forceinline__

typedef short bf16x8_t __attribute__((__vector_size__(8 * sizeof(short))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// bf16 <-> fp32 (bf16 held as uint16 bit patterns).
LS_DEV float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
LS_DEV uint16_t f2bf(float f) {   // round to nearest even; inputs are finite
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Storage element of the model: bf16 (uint16_t) or fp32 (float).
template <typename T> struct Elem;
template <> struct Elem<uint16_t> {
  static constexpr int per16 = 8;           // elements per 16-byte vector
  LS_DEV static float load(const uint16_t* p) { return bf2f(*p); }
  LS_DEV static void store(uint16_t* p, float v) { *p = f2bf(v); }
  LS_DEV static float round(float v) { return bf2f(f2bf(v)); }
};
template <> struct Elem<float> {
  static constexpr int per16 = 4;
  LS_DEV static float load(const float* p) { return *p; }
  LS_DEV static void store(float* p, float v) { *p = v; }
  LS_DEV static float round(float v) { return v; }
};

LS_DEV float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
LS_DEV float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Block-wide reductions through LDS; every thread gets the result.  `red` must hold
// blockDim.x / 64 floats; callers separate successive uses with __syncthreads().
LS_DEV float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = warp_sum(v);
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  __syncthreads();
  return t;
}
LS_DEV float block_max(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = warp_max(v);
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = red[0];
  for (int i = 1; i < nw; ++i) t = fmaxf(t, red[i]);
  __syncthreads();
  return t;
}

// Device error word (first error wins).
LS_DEV void ls_flag(int* err, int code) { atomicCAS(err, 0, code); }

// Attention key j of row i: finished prefix, then the row's ancestors, then itself.
LS_DEV int key_slot(int j, int n_fin, const int32_t* fin, const int32_t* anc, int a0, int na, int self) {
  return j < n_fin ? fin[j] : (j < n_fin + na ? anc[a0 + (j - n_fin)] : self);
}
