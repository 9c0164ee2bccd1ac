// Readout distribution of C: temperature, softmax, top-p truncation, normalisation (LoopSpec
// page, section 2.1: every intermediate readout applies the same processing as the target).
//
// One 1024-thread workgroup per row; the row lives in registers (thread t holds ids
// t, t + 1024, t + 2048, ...: coalesced loads and stores, one read of the logits and one write
// of the distribution).  Top-p keeps the tokens ordered by probability (then id) up to and
// including the one at which the kept mass reaches top_p.  The crossing token's key (the
// float32 bit pattern of its probability, monotone for non-negative floats) is found by a
// radix select over the occupied key range, accumulating mass in 32-bit fixed point
// (floor(p * 2^31)), so the selection is exact for those masses and independent of summation
// order.  Ties at the crossing key are kept in id order.  The kept tokens are renormalised by
// their kept mass (the 31-bit masses plus the fractions they dropped).
#include "common.h"
#include "kernels.h"

namespace ls {

constexpr int DIST_THREADS = 1024;
constexpr int DIST_PT_MAX = 64;           // ids per thread: V <= 65536
constexpr int DIST_BINS = 2048;

LS_DEV unsigned block_sum_u32(unsigned v, unsigned* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) red[w] = v;
  __syncthreads();
  unsigned t = 0;
  for (int i = 0; i < nw; ++i) t += red[i];
  __syncthreads();
  return t;
}
LS_DEV unsigned block_min_u32(unsigned v, unsigned* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, (unsigned)__shfl_xor(v, o, 64));
  if (lane == 0) red[w] = v;
  __syncthreads();
  unsigned t = red[0];
  for (int i = 1; i < nw; ++i) t = min(t, red[i]);
  __syncthreads();
  return t;
}
LS_DEV unsigned block_max_u32(unsigned v, unsigned* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (unsigned)__shfl_xor(v, o, 64));
  if (lane == 0) red[w] = v;
  __syncthreads();
  unsigned t = red[0];
  for (int i = 1; i < nw; ++i) t = max(t, red[i]);
  __syncthreads();
  return t;
}

// Row access through a buffer descriptor: id j*DIST_THREADS + tid is at vector offset tid*4 and
// scalar offset j*DIST_THREADS*4, so the unrolled loops need no per-element address registers;
// stores past the row end fall outside the descriptor's range and are dropped.
LS_DEV __amdgpu_buffer_rsrc_t row_rsrc(const float* base, int n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, n * 4, 0x00020000);
}
LS_DEV float row_ld(__amdgpu_buffer_rsrc_t r, int j) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)threadIdx.x * 4, j * DIST_THREADS * 4, 0));
}
LS_DEV void row_st(__amdgpu_buffer_rsrc_t r, int j, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)threadIdx.x * 4, j * DIST_THREADS * 4, 0);
}

LS_DEV unsigned mass31(float p) { return (unsigned)(p * 2147483648.0f); }   // exact floor(p * 2^31), p in [0, 1]
// The same value recomputed where it is needed: the radix rounds would otherwise keep all
// PT masses live next to the probabilities (the compiler hoists them out of the rounds
// loop), which spills.  Volatile assembly is not hoisted; v_cvt_u32_f32 truncates like the
// conversion above.
LS_DEV unsigned mass31_here(float p) {
  unsigned r;
  asm volatile("v_mul_f32 %0, 0x4f000000, %1\n\tv_cvt_u32_f32 %0, %0" : "=v"(r) : "v"(p));
  return r;
}

// PT ids per thread (PT * DIST_THREADS >= V): the smallest multiple of 16 that covers the row,
// so a vocabulary below 65536 runs no padding columns.
template <int PT>
__global__ __launch_bounds__(DIST_THREADS) void k_dist(const float* logits, int V, int greedy, float T, float top_p,
                                                      float* probs, const int32_t* out_rows, int n_prob_rows,
                                                      int32_t* argmax, int* err) {
  const int m = blockIdx.x;
  const float* z = logits + (size_t)m * V;
  const int orow = out_rows ? out_rows[m] : m;
  const int tid = threadIdx.x;
  __shared__ float redf[16];
  __shared__ int redi[16];
  __shared__ unsigned redu[16];
  __shared__ unsigned hist[DIST_BINS];
  __shared__ unsigned s_sel[2];

  // ids past V hold -inf logits: probability 0, mass 0, never kept
  float x[PT];
  {
    const __amdgpu_buffer_rsrc_t Rz = row_rsrc(z, V);
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const float v = row_ld(Rz, j);
      x[j] = tid + DIST_THREADS * j < V ? v : -INFINITY;
    }
  }
  // argmax, lowest id on ties (a thread's ids increase with j)
  float best = -INFINITY;
  int bi = 0x7fffffff;
#pragma unroll
  for (int j = 0; j < PT; ++j)
    if (x[j] > best) { best = x[j]; bi = tid + DIST_THREADS * j; }
  for (int o = 32; o > 0; o >>= 1) {
    const float ob = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
  }
  if ((tid & 63) == 0) { redf[tid >> 6] = best; redi[tid >> 6] = bi; }
  __syncthreads();
  best = redf[0]; bi = redi[0];
  for (int w = 1; w < DIST_THREADS / 64; ++w)
    if (redf[w] > best || (redf[w] == best && redi[w] < bi)) { best = redf[w]; bi = redi[w]; }
  __syncthreads();
  if (argmax && tid == 0) argmax[m] = bi;
  if (orow == -1) return;                       // distribution not requested for this row
  if (orow < 0 || orow >= n_prob_rows) {
    if (tid == 0) ls_flag(err, 1);
    return;
  }
  float* p = probs + (size_t)orow * V;
  const __amdgpu_buffer_rsrc_t Rp = row_rsrc(p, V);
  if (greedy) {
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const int v = tid + DIST_THREADS * j;
      row_st(Rp, j, v == bi ? 1.0f : 0.0f);
    }
    return;
  }

  // softmax of z / T
  const float mx = best / T;
  float sacc = 0.f;
#pragma unroll
  for (int j = 0; j < PT; ++j) {
    x[j] = __expf(x[j] / T - mx);
    sacc += x[j];
  }
  const float inv = 1.0f / block_sum(sacc, redf);
#pragma unroll
  for (int j = 0; j < PT; ++j) x[j] *= inv;
  if (!(top_p < 1.0f)) {
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const int v = tid + DIST_THREADS * j;
      row_st(Rp, j, x[j]);
    }
    return;
  }

  // fixed-point masses and the top-p target
  unsigned zl = 0, kmin = 0xffffffffu, kmax = 0;
#pragma unroll
  for (int j = 0; j < PT; ++j) {
    zl += mass31(x[j]);
    const unsigned k = __float_as_uint(x[j]);
    kmin = min(kmin, k);
    kmax = max(kmax, k);
  }
  const unsigned Z = block_sum_u32(zl, redu);
  const unsigned TP = (unsigned)ceil((double)top_p * (double)Z);
  kmin = block_min_u32(kmin, redu);
  kmax = block_max_u32(kmax, redu);

  // radix select over keys in [lo, lo + 2^width): find the key at which the mass of larger
  // keys reaches TP; `above` is the mass of keys above the current range
  unsigned lo = kmin;
  int width = 32 - __clz(kmax - kmin);          // bits needed for (key - lo)
  unsigned above = 0;
  while (true) {
    const int shift = width > 11 ? width - 11 : 0;
    const int nb = min(DIST_BINS, ((int)((1ull << width) - 1) >> shift) + 1);
    for (int b = tid; b < nb; b += DIST_THREADS) hist[b] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const unsigned off = __float_as_uint(x[j]) - lo;       // keys below lo wrap to large offsets
      const unsigned ms = mass31_here(x[j]);
      if (ms && (width >= 32 || off < (1u << width))) atomicAdd(&hist[off >> shift], ms);   // zero masses add nothing
    }
    __syncthreads();
    {
      // descending inclusive scan over the bins: thread t takes BPT consecutive bins from the top
      constexpr int BPT = DIST_BINS / DIST_THREADS;
      unsigned hv[BPT], tot = 0;
#pragma unroll
      for (int q = 0; q < BPT; ++q) {
        const int b = nb - 1 - (BPT * tid + q);
        hv[q] = b >= 0 ? hist[b] : 0u;
        tot += hv[q];
      }
      unsigned inc = tot;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned y = __shfl_up(inc, o, 64);
        if ((tid & 63) >= o) inc += y;
      }
      if ((tid & 63) == 63) redu[tid >> 6] = inc;
      __syncthreads();
      unsigned run = above + inc - tot;             // mass of the bins above this thread's first
      for (int w = 0; w < (tid >> 6); ++w) run += redu[w];
      // the crossing bin: the first (highest) where the running mass reaches TP
#pragma unroll
      for (int q = 0; q < BPT; ++q) {
        const int b = nb - 1 - (BPT * tid + q);
        if (b >= 0 && run < TP && run + hv[q] >= TP) { s_sel[0] = (unsigned)b; s_sel[1] = run; }
        run += hv[q];
      }
    }
    __syncthreads();
    const unsigned sel = s_sel[0];
    above = s_sel[1];
    lo += sel << shift;
    width = shift;
    __syncthreads();
    if (shift == 0) break;
  }
  const unsigned kstar = lo;
  const unsigned Pk = mass31(__uint_as_float(kstar));
  // tokens at kstar kept: enough of them (in id order) to reach TP; at least one
  unsigned n_keep = Pk > 0 ? (TP - above + Pk - 1) / Pk : 0xffffffffu;
  if (n_keep == 0) n_keep = 1;
  // ties at kstar, and the kept mass for the renormalisation.  The radix select left the exact
  // 31-bit mass of the tokens above kstar in `above`; what floor(p * 2^31) dropped from each of
  // them is the fraction of p * 2^31 (exact in float32), summed here, so the kept mass is known
  // to float32 rounding of that small correction rather than off by up to V * 2^-31 relative
  unsigned nt_local = 0;
  float fl = 0.f;
#pragma unroll
  for (int j = 0; j < PT; ++j) {
    const unsigned k = __float_as_uint(x[j]);
    nt_local += k == kstar;
    fl += k > kstar ? __builtin_amdgcn_fractf(x[j] * 2147483648.0f) : 0.f;
  }
  const unsigned n_ties = block_sum_u32(nt_local, redu);
  const unsigned kept_ties = min(n_keep, n_ties);
  const double kept = ((double)above + (double)block_sum(fl, redf)) * 0x1p-31 +
                      (double)kept_ties * (double)__uint_as_float(kstar);
  const float scale = (float)(1.0 / kept);
  if (n_keep >= n_ties) {
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const int v = tid + DIST_THREADS * j;
      row_st(Rp, j, __float_as_uint(x[j]) >= kstar ? x[j] * scale : 0.0f);
    }
    return;
  }
  // rare: more ties at kstar than are kept.  The row goes to the output first, then the ties
  // are ranked by id (column j, then thread) reading it back.
#pragma unroll
  for (int j = 0; j < PT; ++j)
    if (tid + DIST_THREADS * j < V) p[tid + DIST_THREADS * j] = x[j];
  __syncthreads();
  unsigned before = 0;                          // ties with smaller ids in earlier columns
  for (int j = 0; j < PT; ++j) {
    const int v = tid + DIST_THREADS * j;
    const float pv = v < V ? p[v] : 0.f;
    const bool tie = v < V && __float_as_uint(pv) == kstar;
    const unsigned long long bal = __ballot(tie);
    const unsigned in_wave = __popcll(bal & ((1ull << (tid & 63)) - 1ull));
    if ((tid & 63) == 0) redu[tid >> 6] = __popcll(bal);
    __syncthreads();
    unsigned wave_off = 0, col = 0;
    for (int w = 0; w < DIST_THREADS / 64; ++w) {
      if (w < (tid >> 6)) wave_off += redu[w];
      col += redu[w];
    }
    __syncthreads();
    const unsigned rank = before + wave_off + in_wave;
    if (v < V) {
      const bool keep = __float_as_uint(pv) > kstar || (tie && rank < n_keep);
      p[v] = keep ? pv * scale : 0.0f;
    }
    before += col;
  }
}

// ---- LM head without coda layers: logits[m][n] = RMSNorm(H[slot of row m]) . E[n] ------------
// A plain streaming kernel (no persistent workgroups): one wave per 16 vocabulary rows, 4 waves
// per workgroup, many workgroups per CU, so the 16-row weight tiles of the whole vocabulary
// are in flight at once.  Each workgroup first normalises the M <= 16 rows (final RMSNorm,
// gains g) into LDS, rounded to bf16 like every GEMM input; a wave then runs
// v_mfma_f32_16x16x32_bf16 with A = 16 embedding rows read straight from memory (lane l:
// row l%16, 8 columns at 8*(l/16)) and B = the normalised rows from LDS, its loads issued
// eight k-steps ahead of the multiplies.
constexpr int HEAD_WAVES = 4;

__global__ __launch_bounds__(64 * HEAD_WAVES) void k_head(const float* H, ValidateArgs rc, int i0, int M, int d, int V,
                                                         const uint16_t* emb, const float* g, float eps,
                                                         float* logits, int ldo) {
  extern __shared__ __attribute__((aligned(16))) char hsm[];
  const int xs = d + 8;                                   // LDS row stride (elements)
  uint16_t* X = reinterpret_cast<uint16_t*>(hsm);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // normalised rows: wave w takes rows w, w + 4, ...; each workgroup checks the rows itself
  // (workgroup 0 records the check), rejected rows are zero
  for (int m = w; m < M; m += HEAD_WAVES) {
    uint16_t* xr = X + (size_t)m * xs;
    const int hr = row_slot(rc, i0 + m);
    if (blockIdx.x == 0 && lane == 0) check_row(rc, i0 + m);
    if (hr < 0) {
      for (int k = 8 * lane; k < d; k += 512) *reinterpret_cast<uint4*>(xr + k) = make_uint4(0, 0, 0, 0);
      continue;
    }
    const float* row = H + (size_t)hr * d;
    float ss = 0.f;
    for (int k = 4 * lane; k < d; k += 256) {
      const float4 v = *reinterpret_cast<const float4*>(row + k);
      ss += (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
    }
    const float ri = 1.0f / sqrtf(wave_sum(ss) / (float)d + eps);
    for (int k = 4 * lane; k < d; k += 256) {
      const float4 v = *reinterpret_cast<const float4*>(row + k);
      const float4 gg = *reinterpret_cast<const float4*>(g + k);
      const unsigned lo = (unsigned)f2bf(v.x * ri * gg.x) | ((unsigned)f2bf(v.y * ri * gg.y) << 16);
      const unsigned hi = (unsigned)f2bf(v.z * ri * gg.z) | ((unsigned)f2bf(v.w * ri * gg.w) << 16);
      *reinterpret_cast<uint2*>(xr + k) = make_uint2(lo, hi);
    }
  }
  __syncthreads();
  const int tile = blockIdx.x * HEAD_WAVES + w;
  const int n0 = tile * 16;
  if (n0 >= V) return;
  const int r = lane & 15, kq = lane >> 4;
  const uint16_t* arow = emb + (size_t)min(n0 + r, V - 1) * d + 8 * kq;   // rows past V: any valid row
  const uint16_t* brow = X + (size_t)min(r, M - 1) * xs + 8 * kq;   // rows m >= M multiply zeros
  const bool live = r < M;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int B8 = 8;                                   // k-steps of 32 per batch
  u32x4_t wa[B8], wb[B8];
#pragma unroll
  for (int u = 0; u < B8; ++u) wa[u] = *reinterpret_cast<const u32x4_t*>(arow + 32 * u);
  for (int kb = 0; kb < d; kb += 64 * B8) {
    const bool more = kb + 32 * B8 < d;
#pragma unroll
    for (int u = 0; u < B8; ++u)
      if (more) wb[u] = *reinterpret_cast<const u32x4_t*>(arow + kb + 32 * (B8 + u));
#pragma unroll
    for (int u = 0; u < B8; ++u) {
      u32x4_t xv = *reinterpret_cast<const u32x4_t*>(brow + kb + 32 * u);
      if (!live) xv = u32x4_t{0u, 0u, 0u, 0u};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wa[u]), __builtin_bit_cast(bf16x8_t, xv),
                                                    acc, 0, 0, 0);
    }
    if (!more) break;
    const bool more2 = kb + 64 * B8 < d;
#pragma unroll
    for (int u = 0; u < B8; ++u)
      if (more2) wa[u] = *reinterpret_cast<const u32x4_t*>(arow + kb + 64 * B8 + 32 * u);
#pragma unroll
    for (int u = 0; u < B8; ++u) {
      u32x4_t xv = *reinterpret_cast<const u32x4_t*>(brow + kb + 32 * (B8 + u));
      if (!live) xv = u32x4_t{0u, 0u, 0u, 0u};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wb[u]), __builtin_bit_cast(bf16x8_t, xv),
                                                    acc, 0, 0, 0);
    }
  }
  // lane l holds rows n = 4*(l/16) + j of the tile for activation row m = l%16
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + 4 * kq + j;
    if (r < M && n < V) logits[(size_t)r * ldo + n] = acc[j];
  }
}

size_t head_smem_bytes(int M, int d) { return (size_t)M * (d + 8) * 2; }

void launch_head(const float* H, const ValidateArgs& v, int i0, int M, int d, int V, const void* emb, const float* g,
                 float eps, float* logits, int ldo, hipStream_t s) {
  const int tiles = (V + 15) / 16;
  hipLaunchKernelGGL(k_head, dim3((tiles + HEAD_WAVES - 1) / HEAD_WAVES), dim3(64 * HEAD_WAVES), head_smem_bytes(M, d), s,
                     H, v, i0, M, d, V, static_cast<const uint16_t*>(emb), g, eps, logits, ldo);
}

void launch_dist(const float* logits, int M, int V, int greedy, float T, float top_p, float* probs,
                 const int32_t* out_rows, int n_prob_rows, int32_t* argmax, int* err, hipStream_t s) {
  const int cols = (V + DIST_THREADS - 1) / DIST_THREADS;
  auto k = cols <= 16 ? k_dist<16> : cols <= 32 ? k_dist<32> : cols <= 48 ? k_dist<48> : k_dist<DIST_PT_MAX>;
  hipLaunchKernelGGL(k, dim3(M), dim3(DIST_THREADS), 0, s, logits, V, greedy, T, top_p, probs, out_rows, n_prob_rows,
                     argmax, err);
}

}  // namespace ls
