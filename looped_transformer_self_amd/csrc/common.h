// Device helpers shared by the libloopspec kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define LS_DEV __device__ __forceinline__

typedef short bf16x8_t __attribute__((__vector_size__(8 * sizeof(short))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

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

// Reductions with every lane of the wave active, on DPP lane moves instead of LDS-crossbar
// shuffles.  Within each 16-lane row: swap neighbours, swap pairs, mirror halves of 8, mirror
// halves of 16 (every lane of the row ends with the row's result); across the four rows the
// row results are read out to scalars, so the wave-wide result is wave-uniform.
template <int CTRL>
LS_DEV float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
LS_DEV float lane_f(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
LS_DEV float row_sum16(float v) {
  v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);   // row_half_mirror
  v += dpp_f<0x140>(v);   // row_mirror
  return v;
}
LS_DEV float row_max16(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return v;
}
// v already uniform within each row: combine the four rows.
LS_DEV float rows_sum(float v) { return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48)); }
LS_DEV float rows_max(float v) { return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48))); }
LS_DEV float wave_sum(float v) { return rows_sum(row_sum16(v)); }
LS_DEV float wave_max(float v) { return rows_max(row_max16(v)); }

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

// NaN in its canonical (positive, quiet) encoding, other values unchanged.  Buffers whose
// readers poll for the disappearance of an all-ones fill pattern store through this, so a NaN
// carried in from a caller's input (which may keep its payload through arithmetic) can never
// look like the fill.
LS_DEV float canon_nan(float v) { return v == v ? v : __uint_as_float(0x7fc00000u); }

// Device error word (first error wins).
LS_DEV void ls_flag(int* err, int code) { atomicCAS(err, 0, code); }

// Attention key j of row i: finished prefix, then the row's ancestors, then itself.
LS_DEV int key_slot(int j, int n_fin, const int32_t* fin, const int32_t* anc, int a0, int na, int self) {
  return j < n_fin ? fin[j] : (j < n_fin + na ? anc[a0 + (j - n_fin)] : self);
}

// The row check (VA is the launchers' ValidateArgs): a row whose slot, depth, ancestor range or
// position is out of contract has checked slot -1.  row_slot only reads; check_row also writes
// the checked copies and raises the error word.
template <typename VA>
LS_DEV int row_slot(const VA& v, int i) {
  const int sl = v.slot[i];
  const int dp = v.dep ? v.dep[i] : v.dep_lo;
  const int a0 = v.anc_off[i], a1 = v.anc_off[i + 1];
  bool ok = sl >= 0 && sl < v.S && dp >= v.dep_lo && dp <= v.dep_hi && a0 >= 0 && a1 >= a0 && a1 - a0 <= v.max_anc;
  if (ok && v.pos) ok = v.pos[i] == v.n_fin + (a1 - a0);
  return ok ? sl : -1;
}
template <typename VA>
LS_DEV int check_row(const VA& v, int i) {
  const int sl = row_slot(v, i);
  if (sl < 0) ls_flag(v.err, 1);
  v.slot_ok[i] = sl;
  v.dep_ok[i] = sl >= 0 && v.dep ? v.dep[i] : v.dep_lo;
  v.row_ok[i] = sl >= 0 ? i : -1;
  return sl;
}
