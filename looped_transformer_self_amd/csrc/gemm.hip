// Skinny weight-streaming GEMM: Y[M][N] = X[M][K] * W[N][K]^T for the few branch rows of a
// pipeline step (M <= 128), with fp32 accumulation on MFMA.
//
// Each workgroup owns a tile of 16 output features and streams those 16 weight rows over the
// full K exactly once; its four waves split K, each lane loading 16-byte vectors of a row (the
// MFMA A operand) and of the activation rows (the B operand, read from L2).  Because the
// reduction is a sum, the k index assigned to each (lane group, vector element) only has to
// agree between A and B; lanes load long contiguous runs of a weight row.  The wave partials
// are reduced through LDS and a fused epilogue writes the result:
//   EP_STORE  - plain fp32 store (LM-head logits);
//   EP_RESID  - residual add into the fp32 hidden rows (attention output / MLP down);
//   EP_SWIGLU - tile rows 0-7 are gate rows j..j+7, rows 8-15 the matching up rows, so
//               silu(g) * u is formed in-tile and stored in the model dtype;
//   EP_QKV    - tile rows pair element i with i + hd/2 of one head, so the rotary embedding
//               (rotate-half) is applied in-tile; q goes to the workspace (fp32), k and v
//               to the row's KV slot at its loop depth (model dtype).
#include "common.h"
#include "kernels.h"

namespace ls {

template <typename T> struct MfmaOp;

// bf16: one 16-byte vector = 8 k-values = one 16x16x32 MFMA operand per lane.
template <> struct MfmaOp<uint16_t> {
  LS_DEV static void mma(f32x4_t& c, const u32x4_t& a, const u32x4_t& b) {
    bf16x8_t av = __builtin_bit_cast(bf16x8_t, a);
    bf16x8_t bv = __builtin_bit_cast(bf16x8_t, b);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
  }
};
// fp32: one 16-byte vector = 4 k-values = four 16x16x4 MFMAs.
template <> struct MfmaOp<float> {
  LS_DEV static void mma(f32x4_t& c, const u32x4_t& a, const u32x4_t& b) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[e]), __uint_as_float(b[e]), c, 0, 0, 0);
  }
};

LS_DEV u32x4_t ldg16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// Weight row (in elements from the matrix start) for tile row r of tile t.
template <int EP>
LS_DEV const void* tile_row(const GemmArgs& a, int t, int r, int esz, bool& valid) {
  valid = true;
  if (EP == EP_SWIGLU) {
    const int j = 8 * t + (r & 7);
    return (const char*)(r < 8 ? a.W0 : a.W1) + (size_t)j * a.K * esz;
  } else if (EP == EP_QKV) {
    const int tiles_per_mat = a.d / 16, tph = a.hd / 16;
    const int mat = t / tiles_per_mat, tl = t % tiles_per_mat;
    const int h = tl / tph, jj = tl % tph;
    const int n = h * a.hd + 8 * jj + (r & 7) + (r < 8 ? 0 : a.hd / 2);
    const void* W = mat == 0 ? a.W0 : (mat == 1 ? a.W1 : a.W2);
    return (const char*)W + (size_t)n * a.K * esz;
  } else {
    int n = 16 * t + r;
    if (n >= a.N) { valid = false; n = a.N - 1; }
    return (const char*)a.W0 + (size_t)n * a.K * esz;
  }
}

template <typename T, int EP, int MT>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs a) {
  constexpr int E = Elem<T>::per16;          // elements per 16-byte vector
  constexpr int U = 4;                        // vectors per lane per group (64 contiguous bytes)
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  bool row_ok;
  const char* wrow = (const char*)tile_row<EP>(a, t, r, (int)sizeof(T), row_ok);
  const char* X = (const char*)a.X;
  const size_t xstride = (size_t)a.K * sizeof(T);

  // k-blocks of 4E elements (64 bytes per row); wave wv owns blocks [b0, b1).
  const int nblk = a.K / (4 * E);
  const int b0 = (wv * nblk) / 4, b1 = ((wv + 1) * nblk) / 4;

  f32x4_t acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  int b = b0;
  // Main groups: U consecutive blocks; lane group g covers U*E contiguous elements.
  for (; b + U <= b1; b += U) {
    const size_t kb = (size_t)b * 4 * E + (size_t)g * U * E;     // element offset of this lane's run
    u32x4_t w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = ldg16(wrow + (kb + u * E) * sizeof(T));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + r;
      u32x4_t x[U];
      if (m < a.M) {
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = ldg16(X + m * xstride + (kb + u * E) * sizeof(T));
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) MfmaOp<T>::mma(acc[mt], w[u], x[u]);
    }
  }
  // Tail: single blocks; lane group g covers E elements of each block.
  for (; b < b1; ++b) {
    const size_t kb = (size_t)b * 4 * E + (size_t)g * E;
    u32x4_t w = ldg16(wrow + kb * sizeof(T));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + r;
      u32x4_t x = m < a.M ? ldg16(X + m * xstride + kb * sizeof(T)) : u32x4_t{0u, 0u, 0u, 0u};
      MfmaOp<T>::mma(acc[mt], w, x);
    }
  }

  // Cross-wave reduction.  Lane (r, g) holds D[n = 4g + j][m = mt*16 + r].
  __shared__ float red[4][MT][16][17];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) red[wv][mt][4 * g + j][r] = acc[mt][j];
  __syncthreads();
  __shared__ float tile[MT * 16][17];        // tile[m][n_local]
  for (int idx = threadIdx.x; idx < MT * 256; idx += 256) {
    const int mt = idx >> 8, nl = (idx >> 4) & 15, mr = idx & 15;
    tile[mt * 16 + mr][nl] = red[0][mt][nl][mr] + red[1][mt][nl][mr] + red[2][mt][nl][mr] + red[3][mt][nl][mr];
  }
  __syncthreads();

  if (EP == EP_STORE || EP == EP_RESID) {
    for (int idx = threadIdx.x; idx < a.M * 16; idx += 256) {
      const int m = idx >> 4, nl = idx & 15, n = 16 * t + nl;
      if (n >= a.N) continue;
      const float y = tile[m][nl];
      if (EP == EP_STORE) {
        a.out[(size_t)m * a.ldo + n] = y;
      } else {
        const int hr = a.hidx ? a.hidx[m] : m;
        if (hr >= 0) a.H[(size_t)hr * a.ldh + n] += y;
      }
    }
  } else if (EP == EP_SWIGLU) {
    T* act = (T*)a.act;
    for (int idx = threadIdx.x; idx < a.M * 8; idx += 256) {
      const int m = idx >> 3, p = idx & 7;
      const float gv = tile[m][p], uv = tile[m][p + 8];
      const float s = gv / (1.0f + expf(-gv));
      Elem<T>::store(act + (size_t)m * a.F + 8 * t + p, s * uv);
    }
  } else {  // EP_QKV
    const int tiles_per_mat = a.d / 16, tph = a.hd / 16;
    const int mat = t / tiles_per_mat, tl = t % tiles_per_mat;
    const int h = tl / tph, jj = tl % tph;
    for (int idx = threadIdx.x; idx < a.M * 8; idx += 256) {
      const int m = idx >> 3, p = idx & 7;
      const int i = 8 * jj + p;                         // index in the first half of the head
      const int e0 = h * a.hd + i, e1 = e0 + a.hd / 2;
      float y0 = tile[m][p], y1 = tile[m][p + 8];
      if (mat < 2) {
        const double inv = pow((double)a.theta, -2.0 * (double)i / (double)a.hd);
        const double ang = (double)a.pos[m] * inv;
        const float c = (float)cos(ang), sn = (float)sin(ang);
        const float r0 = y0 * c - y1 * sn, r1 = y1 * c + y0 * sn;
        y0 = r0; y1 = r1;
      }
      if (mat == 0) {
        a.q[(size_t)m * a.d + e0] = y0;
        a.q[(size_t)m * a.d + e1] = y1;
      } else {
        const int sl = a.slot[m];
        if (sl < 0 || sl >= a.kv.S) { ls_flag(a.err, 1); continue; }
        const int blk = (a.kv.dep ? a.kv.dep[m] + a.kv.dep_off : 0) * a.kv.blk_mul + a.kv.layer;
        T* ent = (T*)a.kv.base + ((size_t)blk * a.kv.S + sl) * 2 * a.d + (mat == 2 ? a.d : 0);
        Elem<T>::store(ent + e0, y0);
        Elem<T>::store(ent + e1, y1);
      }
    }
  }
}

template <typename T, int EP>
static void launch_t(const GemmArgs& a, hipStream_t s) {
  int tiles;
  if (EP == EP_SWIGLU) tiles = a.F / 8;
  else if (EP == EP_QKV) tiles = 3 * (a.d / 16);
  else tiles = (a.N + 15) / 16;
  const int mt = (a.M + 15) / 16;
  if (mt <= 1) hipLaunchKernelGGL((k_gemm<T, EP, 1>), dim3(tiles), dim3(256), 0, s, a);
  else if (mt <= 2) hipLaunchKernelGGL((k_gemm<T, EP, 2>), dim3(tiles), dim3(256), 0, s, a);
  else if (mt <= 4) hipLaunchKernelGGL((k_gemm<T, EP, 4>), dim3(tiles), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_gemm<T, EP, 8>), dim3(tiles), dim3(256), 0, s, a);
}

void launch_gemm(bool bf16, int ep, const GemmArgs& a, hipStream_t s) {
  if (bf16) {
    switch (ep) {
      case EP_STORE: launch_t<uint16_t, EP_STORE>(a, s); break;
      case EP_RESID: launch_t<uint16_t, EP_RESID>(a, s); break;
      case EP_SWIGLU: launch_t<uint16_t, EP_SWIGLU>(a, s); break;
      default: launch_t<uint16_t, EP_QKV>(a, s); break;
    }
  } else {
    switch (ep) {
      case EP_STORE: launch_t<float, EP_STORE>(a, s); break;
      case EP_RESID: launch_t<float, EP_RESID>(a, s); break;
      case EP_SWIGLU: launch_t<float, EP_SWIGLU>(a, s); break;
      default: launch_t<float, EP_QKV>(a, s); break;
    }
  }
}

// X[m][:] = RMSNorm(H[hidx[m]]) * g, stored in the model dtype (the GEMM operand).
template <typename T>
__global__ __launch_bounds__(256) void k_rmsnorm(const float* H, const int32_t* hidx, int ldh, const float* g,
                                                 int d, float eps, T* X) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  const int hr = hidx ? hidx[m] : m;
  if (hr < 0) {                         // rejected row: feed zeros
    for (int i = threadIdx.x; i < d; i += 256) Elem<T>::store(X + (size_t)m * d + i, 0.f);
    return;
  }
  const float* h = H + (size_t)hr * ldh;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += 256) ss += h[i] * h[i];
  ss = block_sum(ss, red);
  const float rinv = 1.0f / sqrtf(ss / (float)d + eps);
  for (int i = threadIdx.x; i < d; i += 256) Elem<T>::store(X + (size_t)m * d + i, h[i] * rinv * g[i]);
}

void launch_rmsnorm(bool bf16, const float* H, const int32_t* hidx, int ldh, const float* g, int M, int d,
                    float eps, void* X, hipStream_t s) {
  if (bf16) hipLaunchKernelGGL(k_rmsnorm<uint16_t>, dim3(M), dim3(256), 0, s, H, hidx, ldh, g, d, eps, (uint16_t*)X);
  else hipLaunchKernelGGL(k_rmsnorm<float>, dim3(M), dim3(256), 0, s, H, hidx, ldh, g, d, eps, (float*)X);
}

}  // namespace ls
