// Prefill of a chunk of prompt positions as large-M matrix products.
//
// The prompt runs through P, every loop iteration 1..R of B and the coda layers at the
// readout depths before decoding starts (LoopSpec page, section 2.1, eq. 1: the same P/B/C
// map, applied to all prompt positions at once; section 2.4: prelude, loop and coda caches
// indexed by depth; section 3.1 leaves prefill out of the decode timing).  A chunk of n
// consecutive positions follows the n_fin committed ones; each layer of each depth is
//   RMSNorm -> [q k v] = a W^T -> RoPE, K/V into the depth's cache -> causal attention over
//   the committed prefix and the chunk -> h += o Wo^T -> RMSNorm -> silu(b Wg^T) * (b Wu^T)
//   -> h += act Wd^T,
// with the chunk's rows as the M dimension of every product, so the weights are streamed
// once per layer for the whole chunk and the products run on the matrix cores.
//
// Storage precision is the decode path's: weights, normalised activations, attention
// outputs, SwiGLU outputs and the K/V cache in the model dtype; residual stream, queries,
// scores and softmax in fp32 (the matrix-core attention of bf16 models feeds the fp32 query
// and softmax weights to bf16 MFMAs as hi + lo pairs, ~16 significant bits, and accumulates in
// fp32).
#include <math.h>

#include <utility>

#include "common.h"
#include "kernels.h"

namespace ls {

namespace {

// ---- matrix product C = X W^T over 256 x 128 tiles -------------------------------------------
// X: activation rows [M][K] (model dtype); W: weight rows [N][K].  A workgroup computes 256
// weight rows x 128 activation rows.  Three producer waves stream the operands into a ring of
// GNST LDS stages with direct-to-LDS 16-byte loads (each producer 128 of the stage's 384 rows,
// weight rows first; 128 bytes of K per row per stage), keeping GNST - 1 stages in flight;
// four consumer waves multiply: consumer (wn, wx) a 128 x 64 part as 8 x 4 MFMA blocks of
// 16 x 16 (A = 16 weight rows, B = 16 activation rows; lane l holds weight rows 4*(l/16) + j
// of activation row l%16 of a block), so a k-step reads 12 operand fragments from LDS for 32
// MFMAs.  A stage holds each tile as rows of eight 16-byte chunks, chunk c of row r at
// c ^ (r & 7) (the producers pick each lane's source chunk so the loads land that way), so the
// 16 rows an MFMA operand read touches fall on distinct banks.  One workgroup barrier per
// stage: a producer passes it once its loads of that stage have landed, and issues the stage
// GNST - 1 ahead only after it, when every consumer is done with the buffer that stage reuses.
#ifndef LS_PF_WTILE
#define LS_PF_WTILE 256
#endif
constexpr int GWT = LS_PF_WTILE;     // weight rows per tile (128 or 256)
constexpr int GT = 128;              // activation rows per tile
constexpr int GCH = 8;               // 16-byte chunks per tile row per stage
constexpr int GWB = GWT / 32;        // 16-row weight blocks per consumer wave
#ifndef LS_PF_STAGES
#define LS_PF_STAGES (GWT == 128 ? 4 : 3)
#endif
constexpr int GNST = LS_PF_STAGES;   // LDS stages
constexpr int GLOADS = 16;           // load instructions per producer wave per stage (8 rows each)
constexpr int GCONS = 4, GPROD = (GWT + GT) / (8 * GLOADS);
constexpr int GTHREADS = 64 * (GCONS + GPROD);
constexpr int GSTAGE = (GWT + GT) * GCH * 16;   // bytes of one stage: weight tile, then activation tile

enum PfMode { PF_STORE = 0, PF_ADD = 1, PF_SWIGLU = 2 };

struct GemmArgs {
  const void* X;                     // [M][K], row stride K
  int M, K;
  const void* W[3];                  // nmat weight matrices [Nb][K]; SWIGLU: W[0] = gate, W[1] = up
  int Nb, nmat;
  int n_wt, n_xt;                    // weight tiles (over all matrices), activation tiles
  float* out;                        // STORE: out[m][mat*Nb + n]; ADD: out[m][n] += (row stride ldo)
  int ldo;
  void* act;                         // SWIGLU: act[m][n] (model dtype, row stride Nb)
};

template <typename T> struct PfMma;
template <> struct PfMma<uint16_t> {
  LS_DEV static void run(f32x4_t& c, const u32x4_t& a, const u32x4_t& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0,
                                                0, 0);
  }
};
template <> struct PfMma<float> {
  LS_DEV static void run(f32x4_t& c, const u32x4_t& a, const u32x4_t& b) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[e]), __uint_as_float(b[e]), c, 0, 0, 0);
  }
};

// Wait until at most N vector memory instructions of this wave are outstanding.
template <int N>
LS_DEV void vm_wait() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <typename T, int MODE>
__global__ __launch_bounds__(GTHREADS) void k_pf_gemm(GemmArgs g) {
  extern __shared__ __attribute__((aligned(16))) char gsm[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // tile of this workgroup: workgroups are placed on the 8 XCDs round-robin; consecutive tile
  // numbers (which share a weight tile) go to one XCD so its L2 serves their weight reads
  const int nt = g.n_wt * g.n_xt, gid = blockIdx.x;
  const int q8 = nt >> 3, r8 = nt & 7, x8 = gid & 7;
  const int t = x8 * q8 + min(x8, r8) + (gid >> 3);
  const int wt = t / g.n_xt, xt = t - wt * g.n_xt;
  const int rb = g.K * (int)sizeof(T);                                  // bytes per row
  const int nst = (rb + 16 * GCH - 1) / (16 * GCH);                     // stages
  const bool tail = rb % (16 * GCH) != 0;                               // last stage: one 64-byte k-step

  if (w >= GCONS) {
    // ------------------------------ producer waves ------------------------------
    // producer p loads stage rows [128p, 128p + 128): weight rows first, then activation rows
    const int p = w - GCONS, pos = lane & 7;
    const char* src[GLOADS];
    int cb[GLOADS];                                                     // byte offset of the lane's chunk
#pragma unroll
    for (int i = 0; i < GLOADS; ++i) {
      const int r = 128 * p + 8 * i + (lane >> 3);                      // row within the stage
      cb[i] = 16 * (pos ^ (r & 7));
      if (r < GWT) {
        int mat, n;
        if (MODE == PF_SWIGLU) {                                        // 16-row blocks alternate gate / up
          const int blk = r >> 4;
          mat = blk & 1;
          n = wt * (GWT / 2) + (blk >> 1) * 16 + (r & 15);
        } else {
          const int tpm = (g.Nb + GWT - 1) / GWT;
          mat = wt / tpm;
          n = (wt - mat * tpm) * GWT + r;
        }
        src[i] = static_cast<const char*>(g.W[mat]) + (size_t)min(n, g.Nb - 1) * rb;   // rows past Nb: never stored
      } else {
        src[i] = static_cast<const char*>(g.X) + (size_t)min(xt * GT + r - GWT, g.M - 1) * rb;  // rows past M: never stored
      }
    }
    auto issue = [&](int st) {
      char* dst = gsm + (st % GNST) * GSTAGE + p * (128 * GCH * 16);
      const int off = st * 16 * GCH;
#pragma unroll
      for (int i = 0; i < GLOADS; ++i) {
        // a chunk past the row end (second half of a ragged last stage, never multiplied):
        // load the row's first chunk instead, so every address stays inside the row
        const int o = off + cb[i] < rb ? off + cb[i] : 0;
        __builtin_amdgcn_global_load_lds(src[i] + o, (__attribute__((address_space(3))) void*)(dst + i * 1024), 16, 0, 0);
      }
    };
    for (int st = 0; st < GNST - 1 && st < nst; ++st) issue(st);
    for (int st = 0; st < nst; ++st) {
      const int newer = min(nst, st + GNST - 1) - st - 1;               // stages issued after st
      if (newer >= 2) vm_wait<2 * GLOADS>();
      else if (newer == 1) vm_wait<GLOADS>();
      else vm_wait<0>();
      asm volatile("s_barrier" ::: "memory");                           // stage st is in LDS
      if (st + GNST - 1 < nst) issue(st + GNST - 1);
    }
    return;
  }

  // ------------------------------ consumer waves ------------------------------
  const int wn = w & 1, wx = w >> 1;
  f32x4_t acc[GWB][4];
#pragma unroll
  for (int a = 0; a < GWB; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int fr = lane & 15, fq = lane >> 4;
  for (int st = 0; st < nst; ++st) {
    __syncthreads();
    const u32x4_t* const Ws = reinterpret_cast<const u32x4_t*>(gsm + (st % GNST) * GSTAGE);
    const u32x4_t* const Xs = Ws + GWT * GCH;
    const int nk = tail && st == nst - 1 ? 1 : 2;
    for (int s = 0; s < nk; ++s) {
      u32x4_t af[GWB], bf[4];
#pragma unroll
      for (int a = 0; a < GWB; ++a) {
        const int r = wn * (GWT / 2) + a * 16 + fr;
        af[a] = Ws[r * GCH + ((s * 4 + fq) ^ (r & 7))];
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int r = wx * 64 + b * 16 + fr;
        bf[b] = Xs[r * GCH + ((s * 4 + fq) ^ (r & 7))];
      }
#pragma unroll
      for (int a = 0; a < GWB; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) PfMma<T>::run(acc[a][b], af[a], bf[b]);
    }
  }

  // epilogue: block (a, b) holds weight rows wn*GWT/2 + a*16 + 4*fq + j of activation row
  // wx*64 + b*16 + fr
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int m = xt * GT + wx * 64 + b * 16 + fr;
    if (m >= g.M) continue;
    if (MODE == PF_SWIGLU) {
#pragma unroll
      for (int p = 0; p < GWB / 2; ++p) {
        const int f = wt * (GWT / 2) + (wn * GWB / 2 + p) * 16 + 4 * fq;
        if (f >= g.Nb) continue;
        T* dst = static_cast<T*>(g.act) + (size_t)m * g.Nb + f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float gt = acc[2 * p][b][j], up = acc[2 * p + 1][b][j];
          Elem<T>::store(dst + j, gt / (1.0f + expf(-gt)) * up);
        }
      }
    } else {
      const int tpm = (g.Nb + GWT - 1) / GWT;
      const int mat = wt / tpm, n0 = (wt - mat * tpm) * GWT;
#pragma unroll
      for (int a = 0; a < GWB; ++a) {
        const int n = n0 + wn * (GWT / 2) + a * 16 + 4 * fq;
        if (n >= g.Nb) continue;
        float4* dst = reinterpret_cast<float4*>(g.out + (size_t)m * g.ldo + (size_t)mat * g.Nb + n);
        float4 v = make_float4(acc[a][b][0], acc[a][b][1], acc[a][b][2], acc[a][b][3]);
        if (MODE == PF_ADD) {
          const float4 h = *dst;
          v = make_float4(h.x + v.x, h.y + v.y, h.z + v.z, h.w + v.w);
        }
        *dst = v;
      }
    }
  }
}

template <typename T, int MODE>
void gemm(const void* X, int M, int K, const void* W0, const void* W1, const void* W2, int Nb, int nmat, float* out,
          int ldo, void* act, hipStream_t s) {
  GemmArgs g{};
  g.X = X; g.M = M; g.K = K;
  g.W[0] = W0; g.W[1] = W1; g.W[2] = W2;
  g.Nb = Nb; g.nmat = nmat;
  g.n_wt = MODE == PF_SWIGLU ? (Nb + GWT / 2 - 1) / (GWT / 2) : nmat * ((Nb + GWT - 1) / GWT);
  g.n_xt = (M + GT - 1) / GT;
  g.out = out; g.ldo = ldo; g.act = act;
  hipLaunchKernelGGL((k_pf_gemm<T, MODE>), dim3(g.n_wt * g.n_xt), dim3(GTHREADS), (size_t)GNST * GSTAGE, s, g);
}

// ---- row kernels --------------------------------------------------------------------------------
// Row check and embedding gather: X[i] = E[tokens[i]] (P without prelude layers, the first
// step of P with them).  Tokens outside [0, V), slots outside [0, S) and committed-prefix
// slots outside [0, S) raise the error word; such a row's embedding is zero.
template <typename T>
__global__ void k_pf_embed(const int32_t* tokens, const int32_t* slots, int n, const int32_t* fin, int n_fin, long long S,
                           const T* emb, int V, int d, float* X, int* err) {
  const int i = blockIdx.x;
  if (i < n) {
    const int tok = tokens[i], sl = slots[i];
    const bool ok = tok >= 0 && tok < V;
    if (threadIdx.x == 0 && (!ok || sl < 0 || sl >= S)) ls_flag(err, 1);
    const T* e = emb + (size_t)(ok ? tok : 0) * d;
    for (int k = threadIdx.x; k < d; k += blockDim.x) X[(size_t)i * d + k] = ok ? Elem<T>::load(e + k) : 0.f;
  }
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < n_fin; j += gridDim.x * blockDim.x)
    if (fin[j] < 0 || fin[j] >= S) ls_flag(err, 1);
}

// A[i] = RMSNorm(X[i]) * g in the model dtype (one workgroup per row).
template <typename T>
__global__ __launch_bounds__(256) void k_pf_norm(const float* X, const float* g, T* A, int d, float eps) {
  __shared__ float red[4];
  const float* x = X + (size_t)blockIdx.x * d;
  float ss = 0.f;
  for (int k = threadIdx.x; k < d; k += 256) ss += x[k] * x[k];
  const float ri = 1.0f / sqrtf(block_sum(ss, red) / (float)d + eps);
  T* a = A + (size_t)blockIdx.x * d;
  for (int k = threadIdx.x; k < d; k += 256) Elem<T>::store(a + k, x[k] * ri * g[k]);
}

// Rotary embedding of q and k (rotate-half pairs (f, f + hd/2) of every head, angle
// pos * theta^(-2f/hd) evaluated in double), q kept in fp32 in place, k and v stored into the
// cache entry of the row's slot (rows with an invalid slot store nothing).
template <typename T>
__global__ void k_pf_rope(float* QKV, int n, int d, int hd, int pos0, const double* invf, const int32_t* slots,
                          long long S, T* kv) {
  const int i = blockIdx.x, half = hd / 2;
  float* row = QKV + (size_t)i * 3 * d;
  const int sl = slots[i];
  const bool st = sl >= 0 && sl < S;
  T* ent = kv + (size_t)(st ? sl : 0) * 2 * d;
  for (int p = threadIdx.x; p < d / 2; p += blockDim.x) {
    const int h = p / half, f = p - h * half;
    const int c0 = h * hd + f, c1 = c0 + half;
    double sd, cd;
    sincos((double)(pos0 + i) * invf[f], &sd, &cd);
    const float c = (float)cd, s = (float)sd;
    const float q0 = row[c0], q1 = row[c1];
    row[c0] = q0 * c - q1 * s;
    row[c1] = q1 * c + q0 * s;
    const float k0 = row[d + c0], k1 = row[d + c1];
    if (st) {
      Elem<T>::store(ent + c0, k0 * c - k1 * s);
      Elem<T>::store(ent + c1, k1 * c + k0 * s);
      Elem<T>::store(ent + d + c0, row[2 * d + c0]);
      Elem<T>::store(ent + d + c1, row[2 * d + c1]);
    }
  }
}

// H[slots[i]] = X[i] (rows with an invalid slot are skipped).
__global__ void k_pf_scatter(const float* X, const int32_t* slots, long long S, int d, float* H) {
  const int sl = slots[blockIdx.x];
  if (sl < 0 || sl >= S) return;
  for (int k = threadIdx.x; k < d; k += blockDim.x) H[(size_t)sl * d + k] = X[(size_t)blockIdx.x * d + k];
}

// ---- causal attention of the chunk ----------------------------------------------------------
// Workgroup (query block of 64 rows, head): keys of the committed prefix (slots fin[0..n_fin))
// and of the chunk (slots[0..n)) in blocks of 64, row i seeing keys t <= n_fin + i; online
// softmax in fp32.  Thread t: queries 4*(t/16) + i (i < 4); scores of keys t%16 + 16 j (j < 4);
// output dims (t%16)*HD/16 + e.  Q, the key block's K and V (converted to fp32) and the
// probabilities sit in LDS.
constexpr int AQ = 64;

template <int HD> struct AttLds {
  static constexpr int ST = HD + 4;                                      // row stride (floats)
  static constexpr size_t bytes = (size_t)(3 * AQ * ST + AQ * (AQ + 4)) * 4 + AQ * 4;
};

template <typename T, int HD>
__global__ __launch_bounds__(256) void k_pf_attn(const float* Q, int ldq, int n, int n_fin, const int32_t* fin,
                                                 const int32_t* slots, long long S, const T* kv, int d, T* O,
                                                 float scale) {
  extern __shared__ __attribute__((aligned(16))) char asm_[];
  constexpr int ST = AttLds<HD>::ST, DPT = HD / 16;
  float* const Qs = reinterpret_cast<float*>(asm_);
  float* const Ks = Qs + AQ * ST;
  float* const Vs = Ks + AQ * ST;
  float* const Ps = Vs + AQ * ST;                                       // [AQ][AQ + 4]
  int* const ksl = reinterpret_cast<int*>(Ps + AQ * (AQ + 4));
  const int tid = threadIdx.x, qg = tid >> 4, kg = tid & 15;
  const int q0 = blockIdx.x * AQ, h = blockIdx.y;
  const int qlast = min(q0 + AQ, n) - 1;
  const int tmax = n_fin + qlast;                                        // last key any row sees

  for (int e = tid; e < AQ * HD; e += 256) {
    const int r = e / HD, c = e - r * HD;
    Qs[r * ST + c] = q0 + r < n ? Q[(size_t)(q0 + r) * ldq + h * HD + c] * scale : 0.f;
  }
  float mrun[4], lsum[4], acc[4][DPT];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mrun[i] = -INFINITY;
    lsum[i] = 0.f;
#pragma unroll
    for (int e = 0; e < DPT; ++e) acc[i][e] = 0.f;
  }

  for (int k0 = 0; k0 <= tmax; k0 += AQ) {
    __syncthreads();                                                     // previous block's reads done
    if (tid < AQ) {
      const int t = k0 + tid;
      int sl = t < n_fin ? fin[t] : (t < n_fin + n ? slots[t - n_fin] : 0);
      ksl[tid] = sl >= 0 && sl < S ? sl : 0;
    }
    __syncthreads();
    for (int e = tid; e < AQ * HD; e += 256) {
      const int r = e / HD, c = e - r * HD;
      const T* ent = kv + (size_t)ksl[r] * 2 * d + h * HD + c;
      Ks[r * ST + c] = Elem<T>::load(ent);
      Vs[r * ST + c] = Elem<T>::load(ent + d);
    }
    __syncthreads();
    float sc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[i][j] = 0.f;
    for (int c = 0; c < HD; c += 4) {
      float4 qv[4], kk[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) qv[i] = *reinterpret_cast<const float4*>(Qs + (4 * qg + i) * ST + c);
#pragma unroll
      for (int j = 0; j < 4; ++j) kk[j] = *reinterpret_cast<const float4*>(Ks + (kg + 16 * j) * ST + c);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sc[i][j] += qv[i].x * kk[j].x + qv[i].y * kk[j].y + qv[i].z * kk[j].z + qv[i].w * kk[j].w;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = n_fin + q0 + 4 * qg + i;                             // this query's position
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = k0 + kg + 16 * j;
        if (t > p || t >= n_fin + n) sc[i][j] = -INFINITY;
        mx = fmaxf(mx, sc[i][j]);
      }
      mx = row_max16(mx);
      const float mnew = fmaxf(mrun[i], mx);                             // finite: key 0 <= p
      const float al = expf(mrun[i] - mnew);
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float e = expf(sc[i][j] - mnew);
        Ps[(4 * qg + i) * (AQ + 4) + kg + 16 * j] = e;
        ps += e;
      }
      lsum[i] = lsum[i] * al + row_sum16(ps);
      mrun[i] = mnew;
#pragma unroll
      for (int e = 0; e < DPT; ++e) acc[i][e] *= al;
    }
    __syncthreads();
    for (int kk = 0; kk < AQ; kk += 4) {
      float4 pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[i] = *reinterpret_cast<const float4*>(Ps + (4 * qg + i) * (AQ + 4) + kk);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float vv[DPT];
#pragma unroll
        for (int e = 0; e < DPT; ++e) vv[e] = Vs[(kk + u) * ST + kg * DPT + e];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pw = u == 0 ? pv[i].x : (u == 1 ? pv[i].y : (u == 2 ? pv[i].z : pv[i].w));
#pragma unroll
          for (int e = 0; e < DPT; ++e) acc[i][e] += pw * vv[e];
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = q0 + 4 * qg + i;
    if (r >= n) continue;
    const float inv = 1.0f / lsum[i];
#pragma unroll
    for (int e = 0; e < DPT; ++e) Elem<T>::store(O + (size_t)r * d + h * HD + kg * DPT + e, acc[i][e] * inv);
  }
}

// ---- causal attention of the chunk on the matrix cores (bf16 caches) -------------------------
// Workgroup (query block of 64 rows, head); wave w takes queries 16w .. 16w + 15 of the block.
// Keys arrive in blocks of 64: K rows [key][hd] and V transposed [hd][key] in LDS (bf16, as
// cached).  Scores S = K q^T come out of v_mfma_f32_16x16x32_bf16 with A = 16 keys x 32 dims
// of K and B = 32 dims x 16 queries; the fp32 query (scaled by 1/sqrt(hd)) enters as two bf16
// terms, q = hi + lo with lo the rounding residual, so the products keep ~16 significant
// bits of q (the key is exactly bf16) and accumulate in fp32.  Lane l then holds the scores
// of query l%16 for keys 16b + 4(l/16) + j; the four lanes of a query meet by shuffles for the
// online-softmax maximum and sum (fp32).  The same lane's eight weights of keys
// {32c + 4(l/16) + j, 32c + 16 + 4(l/16) + j} are its B operand of O^T += V^T P^T (again as
// hi + lo bf16 terms), with A = 16 dims x those 8 keys read from the transposed V: no
// exchange of weights between lanes.  Lane l accumulates dims 16e + 4(l/16) + j of query l%16.
constexpr int AKB = 64;                                  // keys per block

template <int HD> struct MAttLds {
  static constexpr int KS = HD + 8;                      // K row stride (elements)
  static constexpr int VS = AKB + 4;                     // V^T row stride (elements)
  static constexpr size_t bytes = (size_t)(AKB * KS + HD * VS) * 2;
};

LS_DEV void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = f2bf(x);
  lo = f2bf(x - bf2f(hi));
}

template <int HD>
__global__ __launch_bounds__(256) void k_pf_attn_mfma(const float* Q, int ldq, int n, int n_fin, const int32_t* fin,
                                                      const int32_t* slots, long long S, const uint16_t* kv, int d,
                                                      uint16_t* O, float scale) {
  constexpr int NC = HD / 32, NE = HD / 16, CPR = HD / 8;   // dim chunks, dim blocks, 16-byte chunks per row
  constexpr int LPT = (AKB * CPR + 255) / 256;               // 16-byte loads per thread per operand
  extern __shared__ __attribute__((aligned(16))) char msm[];
  uint16_t* const Ks = reinterpret_cast<uint16_t*>(msm);
  uint16_t* const Vt = Ks + AKB * MAttLds<HD>::KS;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int qn = lane & 15, g = lane >> 4;
  const int q0 = blockIdx.x * AKB, h = blockIdx.y;
  const int qlast = min(q0 + AKB, n) - 1;
  const int tmax = n_fin + qlast;
  const int qrow = q0 + 16 * w + qn;                          // this lane's query (chunk row)
  const int qpos = n_fin + qrow;                              // its position

  // the query's B fragments: dims 32c + 8g .. +7, hi and lo terms
  u32x4_t qh[NC], ql[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    uint16_t hv[8], lv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = qrow < n ? Q[(size_t)qrow * ldq + h * HD + 32 * c + 8 * g + i] * scale : 0.f;
      split_bf16(x, hv[i], lv[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qh[c][i] = (unsigned)hv[2 * i] | ((unsigned)hv[2 * i + 1] << 16);
      ql[c][i] = (unsigned)lv[2 * i] | ((unsigned)lv[2 * i + 1] << 16);
    }
  }
  f32x4_t acc[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) acc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lsum = 0.f;

  // this thread's 16-byte pieces of a key block: key r = idx / CPR, chunk idx % CPR
  u32x4_t kr[LPT], vr[LPT];
  auto gload = [&](int k0) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int idx = tid + 256 * u;
      if (idx < AKB * CPR) {
        const int r = idx / CPR, ch = idx - r * CPR;
        const int t = k0 + r;
        int sl = t < n_fin ? fin[t] : (t < n_fin + n ? slots[t - n_fin] : 0);
        sl = sl >= 0 && sl < S ? sl : 0;
        const uint16_t* ent = kv + (size_t)sl * 2 * d + h * HD + 8 * ch;
        kr[u] = *reinterpret_cast<const u32x4_t*>(ent);
        vr[u] = *reinterpret_cast<const u32x4_t*>(ent + d);
      }
    }
  };
  gload(0);
  for (int k0 = 0; k0 <= tmax; k0 += AKB) {
    __syncthreads();                                            // previous block's reads done
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int idx = tid + 256 * u;
      if (idx < AKB * CPR) {
        const int r = idx / CPR, ch = idx - r * CPR;
        *reinterpret_cast<u32x4_t*>(Ks + r * MAttLds<HD>::KS + 8 * ch) = kr[u];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Vt[(8 * ch + 2 * i) * MAttLds<HD>::VS + r] = (uint16_t)(vr[u][i] & 0xffffu);
          Vt[(8 * ch + 2 * i + 1) * MAttLds<HD>::VS + r] = (uint16_t)(vr[u][i] >> 16);
        }
      }
    }
    __syncthreads();
    if (k0 + AKB <= tmax) gload(k0 + AKB);                      // next block in flight meanwhile

    // scores of this lane's query for keys k0 + 16b + 4g + j
    f32x4_t sc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      sc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const u32x4_t ka = *reinterpret_cast<const u32x4_t*>(Ks + (16 * b + qn) * MAttLds<HD>::KS + 32 * c + 8 * g);
        PfMma<uint16_t>::run(sc[b], ka, qh[c]);
        PfMma<uint16_t>::run(sc[b], ka, ql[c]);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = k0 + 16 * b + 4 * g + j;
        if (t > qpos || t >= n_fin + n) sc[b][j] = -INFINITY;
        mx = fmaxf(mx, sc[b][j]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(mrun, mx);                         // finite: key 0 <= every position
    const float al = expf(mrun - mnew);
    float ps = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sc[b][j] = expf(sc[b][j] - mnew);
        ps += sc[b][j];
      }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    lsum = lsum * al + ps;
    mrun = mnew;
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[e][j] *= al;
    // O^T += V^T P^T over the two 32-key chunks
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint16_t ph[8], pl[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        split_bf16(sc[2 * c][j], ph[j], pl[j]);
        split_bf16(sc[2 * c + 1][j], ph[4 + j], pl[4 + j]);
      }
      u32x4_t pbh, pbl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pbh[i] = (unsigned)ph[2 * i] | ((unsigned)ph[2 * i + 1] << 16);
        pbl[i] = (unsigned)pl[2 * i] | ((unsigned)pl[2 * i + 1] << 16);
      }
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const uint16_t* vrow = Vt + (16 * e + qn) * MAttLds<HD>::VS + 32 * c + 4 * g;
        const u32x2_t v0 = *reinterpret_cast<const u32x2_t*>(vrow);
        const u32x2_t v1 = *reinterpret_cast<const u32x2_t*>(vrow + 16);
        const u32x4_t va = u32x4_t{v0.x, v0.y, v1.x, v1.y};
        PfMma<uint16_t>::run(acc[e], va, pbh);
        PfMma<uint16_t>::run(acc[e], va, pbl);
      }
    }
  }
  if (qrow < n) {
    const float inv = 1.0f / lsum;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      uint16_t* dst = O + (size_t)qrow * d + h * HD + 16 * e + 4 * g;
      const unsigned lo = (unsigned)f2bf(acc[e][0] * inv) | ((unsigned)f2bf(acc[e][1] * inv) << 16);
      const unsigned hi = (unsigned)f2bf(acc[e][2] * inv) | ((unsigned)f2bf(acc[e][3] * inv) << 16);
      *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{lo, hi};
    }
  }
}

template <typename T, int HD>
void attn_hd(const float* Q, int n, int n_fin, const int32_t* fin, const int32_t* slots, long long S, const T* kv, int d,
             int nh, T* O, hipStream_t s) {
  hipLaunchKernelGGL((k_pf_attn<T, HD>), dim3((n + AQ - 1) / AQ, nh), dim3(256), AttLds<HD>::bytes, s, Q, 3 * d, n,
                     n_fin, fin, slots, S, kv, d, O, 1.0f / sqrtf((float)HD));
}

template <int HD>
void attn_mfma(const float* Q, int n, int n_fin, const int32_t* fin, const int32_t* slots, long long S,
               const uint16_t* kv, int d, int nh, uint16_t* O, hipStream_t s) {
  hipLaunchKernelGGL((k_pf_attn_mfma<HD>), dim3((n + AKB - 1) / AKB, nh), dim3(256), MAttLds<HD>::bytes, s, Q, 3 * d,
                     n, n_fin, fin, slots, S, kv, d, O, 1.0f / sqrtf((float)HD));
}

template <typename T>
void attn(int hd, const float* Q, int n, int n_fin, const int32_t* fin, const int32_t* slots, long long S, const T* kv,
          int d, int nh, T* O, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    // bf16 caches: the matrix-core kernel for head dims it tiles (multiples of 32)
    const uint16_t* k16 = reinterpret_cast<const uint16_t*>(kv);
    uint16_t* o16 = reinterpret_cast<uint16_t*>(O);
    switch (hd) {
      case 32: return attn_mfma<32>(Q, n, n_fin, fin, slots, S, k16, d, nh, o16, s);
      case 64: return attn_mfma<64>(Q, n, n_fin, fin, slots, S, k16, d, nh, o16, s);
      case 96: return attn_mfma<96>(Q, n, n_fin, fin, slots, S, k16, d, nh, o16, s);
      case 128: return attn_mfma<128>(Q, n, n_fin, fin, slots, S, k16, d, nh, o16, s);
      default: break;
    }
  }
  switch (hd) {
    case 16: attn_hd<T, 16>(Q, n, n_fin, fin, slots, S, kv, d, nh, O, s); break;
    case 32: attn_hd<T, 32>(Q, n, n_fin, fin, slots, S, kv, d, nh, O, s); break;
    case 48: attn_hd<T, 48>(Q, n, n_fin, fin, slots, S, kv, d, nh, O, s); break;
    case 64: attn_hd<T, 64>(Q, n, n_fin, fin, slots, S, kv, d, nh, O, s); break;
    case 80: attn_hd<T, 80>(Q, n, n_fin, fin, slots, S, kv, d, nh, O, s); break;
    case 96: attn_hd<T, 96>(Q, n, n_fin, fin, slots, S, kv, d, nh, O, s); break;
    case 112: attn_hd<T, 112>(Q, n, n_fin, fin, slots, S, kv, d, nh, O, s); break;
    default: attn_hd<T, 128>(Q, n, n_fin, fin, slots, S, kv, d, nh, O, s); break;
  }
}

// One pre-norm layer on the chunk: X (fp32 [n][d]) updated in place; K/V of the chunk stored
// into kv (the layer's cache block [S][2][d]).  kv_only: stop after the K/V store (the last
// coda layer, whose output no later computation reads during prefill).
template <typename T>
void layer(const PrefillArgs& a, const LayerW& lw, T* kv, bool kv_only, hipStream_t s) {
  const int n = a.n, d = a.d, F = a.F;
  const PrefillBufs& b = a.b;
  T* A = static_cast<T*>(b.A);
  hipLaunchKernelGGL(k_pf_norm<T>, dim3(n), dim3(256), 0, s, b.X, lw.g1, A, d, a.eps);
  gemm<T, PF_STORE>(A, n, d, lw.Wq, lw.Wk, lw.Wv, d, 3, b.QKV, 3 * d, nullptr, s);
  hipLaunchKernelGGL(k_pf_rope<T>, dim3(n), dim3(256), 0, s, b.QKV, n, d, a.hd, a.n_fin, a.invf, a.slots, a.S, kv);
  if (kv_only) return;
  attn<T>(a.hd, b.QKV, n, a.n_fin, a.fin, a.slots, a.S, kv, d, a.nh, static_cast<T*>(b.O), s);
  gemm<T, PF_ADD>(b.O, n, d, lw.Wo, nullptr, nullptr, d, 1, b.X, d, nullptr, s);
  hipLaunchKernelGGL(k_pf_norm<T>, dim3(n), dim3(256), 0, s, b.X, lw.g2, A, d, a.eps);
  gemm<T, PF_SWIGLU>(A, n, d, lw.Wg, lw.Wu, nullptr, F, 2, nullptr, 0, b.ACT, s);
  gemm<T, PF_ADD>(b.ACT, n, F, lw.Wd, nullptr, nullptr, d, 1, b.X, d, nullptr, s);
}

template <typename T>
hipError_t run(const PrefillArgs& a, hipStream_t s) {
  const size_t ent = (size_t)2 * a.d;                                    // elements per cache entry
  const size_t blk = (size_t)a.S * ent;                                  // elements per cache block
  hipLaunchKernelGGL(k_pf_embed<T>, dim3(a.n), dim3(256), 0, s, a.tokens, a.slots, a.n, a.fin, a.n_fin, a.S,
                     static_cast<const T*>(a.emb), a.V, a.d, a.b.X, a.err);
  for (int l = 0; l < a.L_pre; ++l)
    layer<T>(a, a.pre[l], static_cast<T*>(a.kv_pre) + l * blk, false, s);
  for (int k = 1; k <= a.R; ++k) {
    for (int l = 0; l < a.L; ++l)
      layer<T>(a, a.core[l], static_cast<T*>(a.kv_core) + ((size_t)(k - 1) * a.L + l) * blk, false, s);
    // coda caches at readout depth k (index ri): the coda layers on a copy of H^(k)
    int ri = -1;
    for (int j = 0; j < a.n_readout; ++j)
      if (a.readout_depths[j] == k) ri = j;
    if (ri >= 0 && a.L_coda && (a.coda_mask >> ri & 1)) {
      const hipError_t e = hipMemcpyAsync(a.b.Xc, a.b.X, (size_t)a.n * a.d * 4, hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return e;
      PrefillArgs c = a;
      std::swap(c.b.X, c.b.Xc);
      for (int l = 0; l < a.L_coda; ++l)
        layer<T>(c, a.coda[l], static_cast<T*>(a.kv_coda) + ((size_t)ri * a.L_coda + l) * blk,
                 l == a.L_coda - 1, s);
    }
  }
  hipLaunchKernelGGL(k_pf_scatter, dim3(a.n), dim3(256), 0, s, a.b.X, a.slots, a.S, a.d, a.H);
  return hipGetLastError();
}

}  // namespace

size_t prefill_bytes(int n, int d, int F, bool bf16) {
  const size_t es = bf16 ? 2 : 4;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return al((size_t)n * d * 4) * 2                                       // X, Xc
         + al((size_t)n * d * es)                                         // A
         + al((size_t)n * 3 * d * 4)                                      // QKV
         + al((size_t)n * d * es)                                         // O
         + al((size_t)n * F * es);                                        // ACT
}

PrefillBufs prefill_carve(void* base, int n, int d, int F, bool bf16) {
  const size_t es = bf16 ? 2 : 4;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  char* p = static_cast<char*>(base);
  PrefillBufs b;
  b.X = reinterpret_cast<float*>(p); p += al((size_t)n * d * 4);
  b.Xc = reinterpret_cast<float*>(p); p += al((size_t)n * d * 4);
  b.A = p; p += al((size_t)n * d * es);
  b.QKV = reinterpret_cast<float*>(p); p += al((size_t)n * 3 * d * 4);
  b.O = p; p += al((size_t)n * d * es);
  b.ACT = p;
  return b;
}

hipError_t launch_prefill(bool bf16, const PrefillArgs& a, hipStream_t s) {
  return bf16 ? run<uint16_t>(a, s) : run<float>(a, s);
}

}  // namespace ls
