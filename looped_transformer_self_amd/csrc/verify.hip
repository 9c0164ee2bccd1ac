// Lossless verification (LoopSpec page, section 2.2-2.3): residual operator (eq. 2), single
// candidate rejection (eq. 3-4), gate and residual second proposal (eq. 5-6), cascade, and the
// point-mass cascade used for copied candidates.  Probabilities enter as the fixed-point
// integers A(v) = floor(p(v) * 2^40); every decision is exact integer arithmetic (u64/u128),
// so identical inputs give identical outputs whatever the thread schedule.  One 256-thread
// workgroup per job, one pass over the vocabulary per reduction.
#include "common.h"
#include "kernels.h"
#include "../../include/loopspec.h"

namespace ls {

typedef unsigned __int128 u128;
typedef unsigned long long u64;
constexpr int VT = 256;

LS_DEV u64 fixp(float p) { return (u64)((double)p * 1099511627776.0); }

// Sum over the block (every thread gets it).
LS_DEV u128 bsum128(u128 v, u128* s) {
  s[threadIdx.x] = v;
  __syncthreads();
  for (int off = VT / 2; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) s[threadIdx.x] += s[threadIdx.x + off];
    __syncthreads();
  }
  const u128 t = s[0];
  __syncthreads();
  return t;
}

// Exclusive scan over threads; also returns the total.
LS_DEV u128 bscan128(u128 v, u128* s, u128* s2, u128& total) {
  s[threadIdx.x] = v;
  __syncthreads();
  u128* a = s;
  u128* b = s2;
  for (int off = 1; off < VT; off <<= 1) {
    b[threadIdx.x] = a[threadIdx.x] + ((int)threadIdx.x >= off ? a[threadIdx.x - off] : (u128)0);
    __syncthreads();
    u128* t = a; a = b; b = t;
  }
  const u128 incl = a[threadIdx.x];
  total = a[VT - 1];
  __syncthreads();
  return incl - v;
}

// floor(U * Z / 2^32) without overflow for Z < 2^120.
LS_DEV u128 scale_u(uint32_t U, u128 Z) {
  const u64 zh = (u64)(Z >> 64), zl = (u64)Z;
  return (((u128)U * zh) << 32) + (((u128)U * zl) >> 32);
}

// SAMPLE(A, U): smallest v whose prefix sum of A exceeds floor(U * Z / 2^32).
template <class F>
LS_DEV int block_sample(F A, int V, uint32_t U, u128* s, u128* s2, int* res) {
  const int per = (V + VT - 1) / VT;
  const int v0 = min(V, (int)threadIdx.x * per), v1 = min(V, v0 + per);
  u128 loc = 0;
  for (int v = v0; v < v1; ++v) loc += A(v);
  u128 Z;
  const u128 ex = bscan128(loc, s, s2, Z);
  if (threadIdx.x == 0) *res = -1;
  __syncthreads();
  if (Z > 0) {
    const u128 thr = scale_u(U, Z);
    if (loc > 0 && ex <= thr && thr < ex + loc) {
      u128 c = ex;
      for (int v = v0; v < v1; ++v) {
        c += A(v);
        if (c > thr) { *res = v; break; }
      }
    }
  }
  __syncthreads();
  const int r = *res;
  __syncthreads();
  return r;
}

template <class F>
LS_DEV u128 block_total(F A, int V, u128* s) {
  const int per = (V + VT - 1) / VT;
  const int v0 = min(V, (int)threadIdx.x * per), v1 = min(V, v0 + per);
  u128 loc = 0;
  for (int v = v0; v < v1; ++v) loc += A(v);
  return bsum128(loc, s);
}

__global__ __launch_bounds__(VT) void k_verify(const ls_verify_job* jobs, const float* probs, int V, int n_rows,
                                              const int32_t* cands, int n_cands, const uint32_t* uniforms,
                                              ls_verify_out* out, int* err) {
  __shared__ u128 s[VT], s2[VT];
  __shared__ int res;
  const ls_verify_job jb = jobs[blockIdx.x];
  const uint32_t* u = uniforms + (size_t)blockIdx.x * LS_UNIFORMS_PER_JOB;
  ls_verify_out o = {-1, 0, 0, -1};

  auto row_ok = [&](int r) { return r >= 0 && r < n_rows; };
  auto tok_ok = [&](int x) { return x >= 0 && x < V; };
  const float* pR = probs + (size_t)(row_ok(jb.p_row) ? jb.p_row : 0) * V;
  const float* q1 = probs + (size_t)(row_ok(jb.q1_row) ? jb.q1_row : 0) * V;
  const float* q2 = probs + (size_t)(row_ok(jb.q2_row) ? jb.q2_row : 0) * V;
  const u128 LIM = (u128)1 << 41;       // a probability row sums to at most ~1 (< 2 in fixed point)
  bool bad = false;

  if (jb.op == LS_JOB_SAMPLE) {
    if (!row_ok(jb.p_row)) bad = true;
    else if (block_total([&](int v) { return (u128)fixp(pR[v]); }, V, s) >= LIM) bad = true;
    else { o.token = block_sample([&](int v) { return (u128)fixp(pR[v]); }, V, u[5], s, s2, &res); o.outcome = LS_OUT_DRAWN; }
  } else if (jb.op == LS_JOB_DRAW1) {
    if (!row_ok(jb.q1_row)) bad = true;
    else if (block_total([&](int v) { return (u128)fixp(q1[v]); }, V, s) >= LIM) bad = true;
    else { o.token = block_sample([&](int v) { return (u128)fixp(q1[v]); }, V, u[0], s, s2, &res); o.outcome = LS_OUT_DRAWN; }
  } else if (jb.op == LS_JOB_DRAW2) {
    if (!row_ok(jb.q1_row) || !row_ok(jb.q2_row) || !tok_ok(jb.x1)) bad = true;
    else {
      auto r2 = [&](int v) { const u64 a = fixp(q2[v]), b = fixp(q1[v]); return (u128)(a > b ? a - b : 0); };
      const u128 Z2 = block_total(r2, V, s);
      const bool open = Z2 > 0 && (!jb.gate || fixp(q2[jb.x1]) < fixp(q1[jb.x1]));
      o.outcome = LS_OUT_DRAWN;
      if (Z2 >= LIM) bad = true;
      else if (open) { o.gate = 1; o.token = block_sample(r2, V, u[1], s, s2, &res); }
    }
  } else if (jb.op == LS_JOB_VERIFY) {
    if (!row_ok(jb.p_row) || !row_ok(jb.q1_row) || !tok_ok(jb.x1) || (jb.gate && (!row_ok(jb.q2_row) || !tok_ok(jb.x2)))) {
      bad = true;
    } else if (block_total([&](int v) { return (u128)fixp(pR[v]); }, V, s) >= LIM) {
      bad = true;
    } else {
      const u64 Px = fixp(pR[jb.x1]), Qx = fixp(q1[jb.x1]);
      if ((u128)u[2] * Qx < ((u128)Px << 32)) {
        o.token = jb.x1; o.outcome = LS_OUT_ACC1;
      } else {
        auto r1raw = [&](int v) { const u64 a = fixp(pR[v]), b = fixp(q1[v]); return (u128)(a > b ? a - b : 0); };
        u128 Z1 = block_total(r1raw, V, s);
        const bool fb1 = Z1 == 0;                              // residual vanished: fall back to p_R
        auto r1 = [&](int v) { return fb1 ? (u128)fixp(pR[v]) : r1raw(v); };
        if (fb1) Z1 = block_total(r1, V, s);
        if (!jb.gate) {
          o.token = block_sample(r1, V, u[4], s, s2, &res); o.outcome = LS_OUT_RESAMPLED;
        } else {
          auto r2 = [&](int v) { const u64 a = fixp(q2[v]), b = fixp(q1[v]); return (u128)(a > b ? a - b : 0); };
          const u128 Z2 = block_total(r2, V, s);
          if (Z2 >= LIM) bad = true;
          else if ((u128)u[3] * Z1 * r2(jb.x2) < ((r1(jb.x2) * Z2) << 32)) {
            o.token = jb.x2; o.outcome = LS_OUT_ACC2;
          } else {
            auto r3raw = [&](int v) { const u128 a = r1(v) * Z2, b = r2(v) * Z1; return a > b ? a - b : (u128)0; };
            const u128 Z3 = block_total(r3raw, V, s);
            if (Z3 == 0) o.token = block_sample(r1, V, u[4], s, s2, &res);
            else o.token = block_sample(r3raw, V, u[4], s, s2, &res);
            o.outcome = LS_OUT_RESAMPLED;
          }
        }
      }
    }
  } else if (jb.op == LS_JOB_VERIFY_COPY) {
    __shared__ int sc[16];
    __shared__ int s_tok, s_j;
    if (!row_ok(jb.p_row) || jb.n_cand < 0 || jb.n_cand > 16 || jb.cand_off < 0 ||
        jb.cand_off + jb.n_cand > n_cands)
      bad = true;
    else {
      for (int j = threadIdx.x; j < jb.n_cand; j += VT) sc[j] = cands[jb.cand_off + j];
      __syncthreads();
      for (int j = 0; j < jb.n_cand; ++j) bad |= !tok_ok(sc[j]);
      const u128 Z0 = bad ? 0 : block_total([&](int v) { return (u128)fixp(pR[v]); }, V, s);
      if (Z0 >= LIM) bad = true;
      if (!bad) {
        if (threadIdx.x == 0) {
          u128 Z = Z0;
          s_tok = -1; s_j = -1;
          for (int j = 0; j < jb.n_cand; ++j) {
            const int c = sc[j];
            bool removed = false;
            for (int k = 0; k < j; ++k) removed |= sc[k] == c;
            const u128 rho = removed ? 0 : (u128)fixp(pR[c]);
            if ((u128)u[8 + j] * Z < (rho << 32)) { s_tok = c; s_j = j; break; }
            Z -= rho;
          }
        }
        __syncthreads();
        if (s_j >= 0) {
          o.token = s_tok; o.outcome = LS_OUT_ACC_COPY; o.aux = s_j;
        } else {
          const int nc = jb.n_cand;
          auto rho = [&](int v) {
            for (int k = 0; k < nc; ++k) if (sc[k] == v) return (u128)0;
            return (u128)fixp(pR[v]);
          };
          o.token = block_sample(rho, V, u[4], s, s2, &res); o.outcome = LS_OUT_RESAMPLED;
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

void launch_verify(const void* jobs, int n_jobs, const float* probs, int V, int n_rows, const int32_t* cands, int n_cands,
                   const uint32_t* uniforms, void* out, int* err, hipStream_t s) {
  hipLaunchKernelGGL(k_verify, dim3(n_jobs), dim3(VT), 0, s, (const ls_verify_job*)jobs, probs, V, n_rows, cands, n_cands,
                     uniforms, (ls_verify_out*)out, err);
}

}  // namespace ls
