// Lossless verification (LoopSpec page, section 2.2-2.3): residual operator (eq. 2), single
// candidate rejection (eq. 3-4), gate and residual second proposal (eq. 5-6; or p_d2 with the
// first candidate masked, the non-residual form of the ablation in Table 3, section 3.4),
// cascade, the shallow screening of copied candidates (CopyLoop page) and the point-mass
// cascade that verifies them.  Probabilities enter as the fixed-point
// integers A(v) = floor(p(v) * 2^40); every decision is exact integer arithmetic (u64/u128),
// so identical inputs give identical outputs whatever the thread schedule.  One 1024-thread
// workgroup per job; thread t owns a contiguous id range; one pass over the vocabulary per
// reduction, sums in u64 (u128 only for the second residual of the cascade).
#include "common.h"
#include "kernels.h"
#include "../../include/loopspec.h"

namespace ls {

typedef unsigned __int128 u128;
typedef unsigned long long u64;
constexpr int VT = 1024;
constexpr int NW = VT / 64;

LS_DEV u64 fixp(float p) { return (u64)((double)p * 1099511627776.0); }

LS_DEV u64 shfl_xor64(u64 v, int o) {
  return ((u64)(unsigned)__shfl_xor((int)(v >> 32), o, 64) << 32) | (unsigned)__shfl_xor((int)v, o, 64);
}
LS_DEV u64 shfl_up64(u64 v, int o) {
  return ((u64)(unsigned)__shfl_up((int)(v >> 32), o, 64) << 32) | (unsigned)__shfl_up((int)v, o, 64);
}

struct Scratch {
  u64 w64[NW];
  u128 w128[NW];
  int res;
};

// Thread t owns the contiguous ids [v0, v1) (thread order = id order, so prefix sums over
// threads are prefix sums over ids).
struct Range {
  int v0, v1;
  LS_DEV Range(int V) {
    const int per = (V + VT - 1) / VT;
    v0 = min(V, (int)threadIdx.x * per);
    v1 = min(V, v0 + per);
  }
};

// Sum over the block of u64 values (every thread gets it).
LS_DEV u64 bsum64(u64 v, Scratch& sc) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += shfl_xor64(v, o);
  if ((threadIdx.x & 63) == 0) sc.w64[threadIdx.x >> 6] = v;
  __syncthreads();
  u64 t = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) t += sc.w64[i];
  __syncthreads();
  return t;
}
// Exclusive scan over threads of u64 values.
LS_DEV u64 bscan64(u64 v, Scratch& sc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  u64 inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const u64 y = shfl_up64(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) sc.w64[w] = inc;
  __syncthreads();
  u64 off = 0;
  for (int i = 0; i < w; ++i) off += sc.w64[i];
  __syncthreads();
  return off + inc - v;
}
LS_DEV u128 bsum128(u128 v, Scratch& sc) {
  // per-wave partials in LDS, summed in fixed order
  for (int o = 32; o > 0; o >>= 1) {
    const u64 hi = shfl_xor64((u64)(v >> 64), o), lo = shfl_xor64((u64)v, o);
    v += ((u128)hi << 64) | lo;
  }
  if ((threadIdx.x & 63) == 0) sc.w128[threadIdx.x >> 6] = v;
  __syncthreads();
  u128 t = 0;
  for (int i = 0; i < NW; ++i) t += sc.w128[i];
  __syncthreads();
  return t;
}
LS_DEV u128 bscan128(u128 v, Scratch& sc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  u128 inc = v;
  for (int o = 1; o < 64; o <<= 1) {
    const u64 hi = shfl_up64((u64)(inc >> 64), o), lo = shfl_up64((u64)inc, o);
    if (lane >= o) inc += ((u128)hi << 64) | lo;
  }
  if (lane == 63) sc.w128[w] = inc;
  __syncthreads();
  u128 off = 0;
  for (int i = 0; i < w; ++i) off += sc.w128[i];
  __syncthreads();
  return off + inc - v;
}

// floor(U * Z / 2^32) without overflow for Z < 2^120.
LS_DEV u128 scale_u(uint32_t U, u128 Z) {
  const u64 zh = (u64)(Z >> 64), zl = (u64)Z;
  return (((u128)U * zh) << 32) + (((u128)U * zl) >> 32);
}

// Block total of a mass function (u64 masses whose sum stays below 2^64).
// Range sums issue their loads sixteen at a time (a plain loop would wait for each load).
template <class F>
LS_DEV u64 range_sum64(F A, const Range& r) {
  u64 loc = 0;
  int v = r.v0;
  for (; v + 16 <= r.v1; v += 16) {
    u64 t[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) t[k] = A(v + k);
#pragma unroll
    for (int k = 0; k < 16; ++k) loc += t[k];
  }
  for (; v < r.v1; ++v) loc += A(v);
  return loc;
}
template <class F>
LS_DEV u128 range_sum128(F A, const Range& r) {
  u128 loc = 0;
  int v = r.v0;
  for (; v + 8 <= r.v1; v += 8) {
    u128 t[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) t[k] = A(v + k);
#pragma unroll
    for (int k = 0; k < 8; ++k) loc += t[k];
  }
  for (; v < r.v1; ++v) loc += A(v);
  return loc;
}

template <class F>
LS_DEV u64 total64(F A, const Range& r, Scratch& sc) {
  return bsum64(range_sum64(A, r), sc);
}
template <class F>
LS_DEV u128 total128(F A, const Range& r, Scratch& sc) {
  return bsum128(range_sum128(A, r), sc);
}

// SAMPLE(A, U): smallest v whose prefix sum of A exceeds floor(U * Z / 2^32); -1 if Z = 0.
template <class F>
LS_DEV int sample64(F A, const Range& r, uint32_t U, Scratch& sc) {
  const u64 loc = range_sum64(A, r);
  const u64 ex = bscan64(loc, sc);
  const u64 Z = bsum64(loc, sc);
  if (threadIdx.x == 0) sc.res = -1;
  __syncthreads();
  if (Z > 0) {
    const u64 thr = (u64)scale_u(U, Z);
    if (loc > 0 && ex <= thr && thr < ex + loc) {
      u64 c = ex;
      for (int v = r.v0; v < r.v1; ++v) {
        c += A(v);
        if (c > thr) { sc.res = v; break; }
      }
    }
  }
  __syncthreads();
  const int res = sc.res;
  __syncthreads();
  return res;
}
template <class F>
LS_DEV int sample128(F A, const Range& r, uint32_t U, Scratch& sc) {
  const u128 loc = range_sum128(A, r);
  const u128 ex = bscan128(loc, sc);
  const u128 Z = bsum128(loc, sc);
  if (threadIdx.x == 0) sc.res = -1;
  __syncthreads();
  if (Z > 0) {
    const u128 thr = scale_u(U, Z);
    if (loc > 0 && ex <= thr && thr < ex + loc) {
      u128 c = ex;
      for (int v = r.v0; v < r.v1; ++v) {
        c += A(v);
        if (c > thr) { sc.res = v; break; }
      }
    }
  }
  __syncthreads();
  const int res = sc.res;
  __syncthreads();
  return res;
}

__global__ __launch_bounds__(VT) void k_verify(const ls_verify_job* jobs, const float* probs, int V, int n_rows,
                                              int32_t* cands, int n_cands, const uint32_t* uniforms,
                                              ls_verify_out* out, int* err) {
  __shared__ Scratch sc;
  // the job and its uniforms are read once, into LDS (they may live in pinned host memory,
  // where every access crosses the bus)
  __shared__ int32_t s_job[sizeof(ls_verify_job) / 4];
  __shared__ uint32_t s_u[LS_UNIFORMS_PER_JOB];
  if (threadIdx.x < sizeof(ls_verify_job) / 4)
    s_job[threadIdx.x] = reinterpret_cast<const int32_t*>(jobs + blockIdx.x)[threadIdx.x];
  else if (threadIdx.x >= 64 && threadIdx.x < 64 + LS_UNIFORMS_PER_JOB)
    s_u[threadIdx.x - 64] = uniforms[(size_t)blockIdx.x * LS_UNIFORMS_PER_JOB + threadIdx.x - 64];
  __syncthreads();
  const ls_verify_job jb = *reinterpret_cast<const ls_verify_job*>(s_job);
  const uint32_t* u = s_u;
  ls_verify_out o = {-1, 0, 0, -1};
  const Range rg(V);

  auto row_ok = [&](int r) { return r >= 0 && r < n_rows; };
  auto tok_ok = [&](int x) { return x >= 0 && x < V; };
  const float* pR = probs + (size_t)(row_ok(jb.p_row) ? jb.p_row : 0) * V;
  const float* q1 = probs + (size_t)(row_ok(jb.q1_row) ? jb.q1_row : 0) * V;
  const float* q2 = probs + (size_t)(row_ok(jb.q2_row) ? jb.q2_row : 0) * V;
  const u64 LIM = (u64)1 << 41;         // a probability row sums to at most ~1 (< 2 in fixed point)
  bool bad = false;
  auto P = [&](int v) { return fixp(pR[v]); };
  auto Q1 = [&](int v) { return fixp(q1[v]); };
  auto Q2 = [&](int v) { return fixp(q2[v]); };
  // second proposal: residual q2 (-) q1 (eq. 5), or q2 with x1 masked (non-residual ablation)
  const bool nonres = (jb.flags & LS_JOB_NON_RESIDUAL) != 0;
  const int x1m = jb.x1;
  auto r2 = [&](int v) {
    const u64 a = fixp(q2[v]);
    if (nonres) return v == x1m ? (u64)0 : a;
    const u64 b = fixp(q1[v]);
    return a > b ? a - b : (u64)0;
  };

  if (jb.op == LS_JOB_SAMPLE) {
    if (!row_ok(jb.p_row) || total64(P, rg, sc) >= LIM) bad = true;
    else { o.token = sample64(P, rg, u[5], sc); o.outcome = LS_OUT_DRAWN; }
  } else if (jb.op == LS_JOB_DRAW1) {
    if (!row_ok(jb.q1_row) || total64(Q1, rg, sc) >= LIM) bad = true;
    else { o.token = sample64(Q1, rg, u[0], sc); o.outcome = LS_OUT_DRAWN; }
  } else if (jb.op == LS_JOB_DRAW2) {
    if (!row_ok(jb.q1_row) || !row_ok(jb.q2_row) || !tok_ok(jb.x1)) bad = true;
    else {
      const u64 Z2 = total64(r2, rg, sc);
      const bool open = Z2 > 0 && (!jb.gate || Q2(jb.x1) < Q1(jb.x1));
      o.outcome = LS_OUT_DRAWN;
      if (Z2 >= LIM) bad = true;
      else if (open) { o.gate = 1; o.token = sample64(r2, rg, u[1], sc); }
    }
  } else if (jb.op == LS_JOB_VERIFY) {
    if (!row_ok(jb.p_row) || !row_ok(jb.q1_row) || !tok_ok(jb.x1) || (jb.gate && (!row_ok(jb.q2_row) || !tok_ok(jb.x2)))) {
      bad = true;
    } else if (total64(P, rg, sc) >= LIM) {
      bad = true;
    } else {
      const u64 Px = P(jb.x1), Qx = Q1(jb.x1);
      if ((u128)u[2] * Qx < ((u128)Px << 32)) {
        o.token = jb.x1; o.outcome = LS_OUT_ACC1;
      } else {
        auto r1raw = [&](int v) { const u64 a = fixp(pR[v]), b = fixp(q1[v]); return a > b ? a - b : (u64)0; };
        u64 Z1 = total64(r1raw, rg, sc);
        const bool fb1 = Z1 == 0;                              // residual vanished: fall back to p_R
        auto r1 = [&](int v) { return fb1 ? fixp(pR[v]) : r1raw(v); };
        if (fb1) Z1 = total64(r1, rg, sc);
        if (!jb.gate) {
          o.token = sample64(r1, rg, u[4], sc); o.outcome = LS_OUT_RESAMPLED;
        } else {
          const u64 Z2 = total64(r2, rg, sc);
          if (Z2 >= LIM) bad = true;
          else if ((u128)u[3] * Z1 * r2(jb.x2) < (((u128)r1(jb.x2) * Z2) << 32)) {
            o.token = jb.x2; o.outcome = LS_OUT_ACC2;
          } else {
            auto r3 = [&](int v) { const u128 a = (u128)r1(v) * Z2, b = (u128)r2(v) * Z1; return a > b ? a - b : (u128)0; };
            const u128 Z3 = total128(r3, rg, sc);
            if (Z3 == 0) o.token = sample64(r1, rg, u[4], sc);
            else o.token = sample128(r3, rg, u[4], sc);
            o.outcome = LS_OUT_RESAMPLED;
          }
        }
      }
    }
  } else if (jb.op == LS_JOB_VERIFY_COPY) {
    __shared__ int cs[16];
    __shared__ int s_tok, s_j;
    if (!row_ok(jb.p_row) || jb.n_cand < 0 || jb.n_cand > 16 || jb.cand_off < 0 ||
        jb.cand_off + jb.n_cand > n_cands)
      bad = true;
    else {
      for (int j = threadIdx.x; j < jb.n_cand; j += VT) cs[j] = cands[jb.cand_off + j];
      __syncthreads();
      for (int j = 0; j < jb.n_cand; ++j) bad |= !tok_ok(cs[j]);
      const u64 Z0 = bad ? 0 : total64(P, rg, sc);
      if (Z0 >= LIM) bad = true;
      if (!bad) {
        if (threadIdx.x == 0) {
          u64 Z = Z0;
          s_tok = -1; s_j = -1;
          for (int j = 0; j < jb.n_cand; ++j) {
            const int c = cs[j];
            bool removed = false;
            for (int k = 0; k < j; ++k) removed |= cs[k] == c;
            const u64 rho = removed ? 0 : P(c);
            if ((u128)u[8 + j] * Z < ((u128)rho << 32)) { s_tok = c; s_j = j; break; }
            Z -= rho;
          }
        }
        __syncthreads();
        if (s_j >= 0) {
          o.token = s_tok; o.outcome = LS_OUT_ACC_COPY; o.aux = s_j;
        } else {
          const int nc = jb.n_cand;
          auto rho = [&](int v) {
            for (int k = 0; k < nc; ++k) if (cs[k] == v) return (u64)0;
            return fixp(pR[v]);
          };
          o.token = sample64(rho, rg, u[4], sc); o.outcome = LS_OUT_RESAMPLED;
        }
      }
    }
  } else if (jb.op == LS_JOB_SCREEN) {
    // shallow screening of copied candidates: keep c when P(c) >= thr (thr = x1 | x2 << 32),
    // survivors ordered by P descending then id, written back to the front of the job's
    // candidate range; with no survivor, one proposal x ~ p_row (first-draw uniform)
    __shared__ int cs[16];
    __shared__ int s_ns;
    if (!row_ok(jb.p_row) || jb.n_cand < 0 || jb.n_cand > 16 || jb.cand_off < 0 ||
        jb.cand_off + jb.n_cand > n_cands)
      bad = true;
    else {
      for (int j = threadIdx.x; j < jb.n_cand; j += VT) cs[j] = cands[jb.cand_off + j];
      __syncthreads();
      for (int j = 0; j < jb.n_cand; ++j) bad |= !tok_ok(cs[j]);
      if (!bad && total64(P, rg, sc) >= LIM) bad = true;
      if (!bad) {
        if (threadIdx.x == 0) {
          const u64 thr = (u64)(uint32_t)jb.x1 | ((u64)(uint32_t)jb.x2 << 32);
          int keep[16];
          u64 mass[16];
          int ns = 0;
          for (int j = 0; j < jb.n_cand; ++j) {
            const u64 m = P(cs[j]);
            if (m < thr) continue;
            int k = ns++;
            while (k > 0 && (mass[k - 1] < m || (mass[k - 1] == m && keep[k - 1] > cs[j]))) {
              keep[k] = keep[k - 1]; mass[k] = mass[k - 1]; --k;
            }
            keep[k] = cs[j]; mass[k] = m;
          }
          int w = 0;
          for (int k = 0; k < ns; ++k) cands[jb.cand_off + w++] = keep[k];
          for (int j = 0; j < jb.n_cand; ++j)
            if (P(cs[j]) < thr) cands[jb.cand_off + w++] = cs[j];
          s_ns = ns;
        }
        __syncthreads();
        o.aux = s_ns;
        if (s_ns > 0) {
          o.outcome = LS_OUT_SCREENED;
        } else {
          o.token = sample64(P, rg, u[0], sc);
          o.outcome = LS_OUT_DRAWN;
        }
      }
    }
  } else {
    bad = true;
  }
  if (threadIdx.x == 0) {
    if (bad) { ls_flag(err, 1); o.token = -1; o.outcome = 0; }
    out[blockIdx.x] = o;
  }
}

void launch_verify(const void* jobs, int n_jobs, const float* probs, int V, int n_rows, int32_t* cands, int n_cands,
                   const uint32_t* uniforms, void* out, int* err, hipStream_t s) {
  hipLaunchKernelGGL(k_verify, dim3(n_jobs), dim3(VT), 0, s, (const ls_verify_job*)jobs, probs, V, n_rows, cands, n_cands,
                     uniforms, (ls_verify_out*)out, err);
}

}  // namespace ls
