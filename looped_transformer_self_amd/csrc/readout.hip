// Readout distribution of C: temperature, softmax, top-p truncation, normalisation (LoopSpec
// page, section 2.1: every intermediate readout applies the same processing as the target).
//
// One 1024-thread workgroup per row; thread t owns a contiguous id range, so "lowest id first"
// orderings reduce to prefix scans over threads.  Top-p keeps the tokens ordered by
// probability (then id) up to and including the one at which the kept mass reaches top_p.
// The crossing token is found by an MSB-first radix select over the float32 bit patterns of
// the probabilities (monotone for non-negative floats), accumulating mass in integer fixed
// point (floor(p * 2^40)), so the selection is exact and independent of summation order.
#include "common.h"
#include "kernels.h"

namespace ls {

constexpr int DIST_THREADS = 1024;

LS_DEV unsigned long long shfl_xor_u64(unsigned long long v, int o) {
  unsigned lo = (unsigned)v, hi = (unsigned)(v >> 32);
  lo = __shfl_xor(lo, o, 64);
  hi = __shfl_xor(hi, o, 64);
  return ((unsigned long long)hi << 32) | lo;
}

LS_DEV unsigned long long block_sum_u64(unsigned long long v, unsigned long long* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += shfl_xor_u64(v, o);
  if (lane == 0) red[w] = v;
  __syncthreads();
  unsigned long long t = 0;
  for (int i = 0; i < nw; ++i) t += red[i];
  __syncthreads();
  return t;
}

// Exclusive prefix sum of one int per thread (thread order).
LS_DEV int block_excl_scan(int v, int* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) red[w] = incl;
  __syncthreads();
  int off = 0;
  for (int i = 0; i < w; ++i) off += red[i];
  (void)nw;
  __syncthreads();
  return off + incl - v;
}

__global__ __launch_bounds__(DIST_THREADS) void k_dist(const float* logits, int V, int greedy, float T, float top_p,
                                                      float* probs, const int32_t* out_rows, int n_prob_rows,
                                                      int32_t* argmax, int* err) {
  const int m = blockIdx.x;
  const float* z = logits + (size_t)m * V;
  const int orow = out_rows ? out_rows[m] : m;
  if (orow == -1) return;                       // distribution not requested for this row
  if (orow < 0 || orow >= n_prob_rows) {
    if (threadIdx.x == 0) ls_flag(err, 1);
    return;
  }
  float* p = probs + (size_t)orow * V;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int per = (V + nt - 1) / nt;
  const int v0 = min(V, tid * per), v1 = min(V, v0 + per);

  __shared__ float redf[16];
  __shared__ int redi[16];
  __shared__ unsigned long long redu[16];
  __shared__ unsigned long long hist[256];
  __shared__ unsigned s_prefix;
  __shared__ unsigned long long s_base;

  // argmax, lowest id on ties
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int v = v0; v < v1; ++v) {
    const float x = z[v];
    if (x > best) { best = x; bi = v; }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float ob = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
  }
  if ((tid & 63) == 0) { redf[tid >> 6] = best; redi[tid >> 6] = bi; }
  __syncthreads();
  best = redf[0]; bi = redi[0];
  for (int w = 1; w < nt / 64; ++w)
    if (redf[w] > best || (redf[w] == best && redi[w] < bi)) { best = redf[w]; bi = redi[w]; }
  __syncthreads();
  if (argmax && tid == 0) argmax[m] = bi;
  if (greedy) {
    for (int v = v0; v < v1; ++v) p[v] = v == bi ? 1.0f : 0.0f;
    return;
  }

  // softmax of z / T
  const float mx = best / T;
  float s = 0.f;
  for (int v = v0; v < v1; ++v) s += expf(z[v] / T - mx);
  s = block_sum(s, redf);
  const float inv = 1.0f / s;
  for (int v = v0; v < v1; ++v) p[v] = expf(z[v] / T - mx) * inv;
  if (!(top_p < 1.0f)) return;

  // fixed-point masses and the top-p target
  const double ONE = 1099511627776.0;   // 2^40
  unsigned long long zs = 0;
  for (int v = v0; v < v1; ++v) zs += (unsigned long long)((double)p[v] * ONE);
  const unsigned long long Z = block_sum_u64(zs, redu);
  const unsigned long long TP = (unsigned long long)ceil((double)top_p * (double)Z);

  // radix select: the key of the token at which the descending cumulative mass reaches TP
  unsigned prefix = 0, pmask = 0;
  unsigned long long base = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int b = tid; b < 256; b += nt) hist[b] = 0;
    __syncthreads();
    for (int v = v0; v < v1; ++v) {
      const float pv = p[v];
      const unsigned key = __float_as_uint(pv);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], (unsigned long long)((double)pv * ONE));
    }
    __syncthreads();
    if (tid == 0) {
      unsigned long long cum = base;
      int sel = 0;
      for (int dg = 255; dg >= 0; --dg) {
        if (cum + hist[dg] >= TP) { sel = dg; break; }
        cum += hist[dg];
      }
      s_prefix = prefix | ((unsigned)sel << shift);
      s_base = cum;
    }
    __syncthreads();
    prefix = s_prefix;
    base = s_base;
    pmask |= 255u << shift;
    __syncthreads();
  }
  const unsigned kstar = prefix;
  const unsigned long long Pk = (unsigned long long)((double)__uint_as_float(kstar) * ONE);
  const unsigned long long n_keep = (TP - base + Pk - 1) / Pk;

  // ties at kstar are kept in id order
  int nt_local = 0;
  for (int v = v0; v < v1; ++v) nt_local += __float_as_uint(p[v]) == kstar;
  const int tie0 = block_excl_scan(nt_local, redi);
  const int n_ties = (int)block_sum((float)nt_local, redf);
  const unsigned long long kept_ties = n_keep < (unsigned long long)n_ties ? n_keep : (unsigned long long)n_ties;
  const unsigned long long Zk = base + kept_ties * Pk;
  const float scale = (float)(ONE / (double)Zk);
  int tr = tie0;
  for (int v = v0; v < v1; ++v) {
    const unsigned key = __float_as_uint(p[v]);
    bool keep = key > kstar;
    if (key == kstar) { keep = (unsigned long long)tr < n_keep; ++tr; }
    p[v] = keep ? p[v] * scale : 0.0f;
  }
}

void launch_dist(const float* logits, int M, int V, int greedy, float T, float top_p, float* probs,
                 const int32_t* out_rows, int n_prob_rows, int32_t* argmax, int* err, hipStream_t s) {
  hipLaunchKernelGGL(k_dist, dim3(M), dim3(DIST_THREADS), 0, s, logits, V, greedy, T, top_p, probs, out_rows, n_prob_rows,
                     argmax, err);
}

}  // namespace ls
