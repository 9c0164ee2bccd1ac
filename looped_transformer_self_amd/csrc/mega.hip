// Persistent producer/consumer kernel for the transformer layers of one call (ls_loop_step:
// the shared block B applied once to every branch row; ls_prelude: embedding + prelude
// layers; ls_readout: coda layers + final norm + LM head).
//
// One cooperative launch, one 512-thread workgroup per CU, all resident.  Each workgroup owns
// a static share of every projection's 16-output-feature tiles (dealt round-robin across the
// phases of the call, so every workgroup streams about the same bytes) and of the attention
// chunks.  Its waves are specialised:
//   * 4 producer waves walk the workgroup's weight-slab sequence (slab = 16 rows x 512 bytes)
//     across all phases and layers and copy slabs straight into an LDS ring with
//     global_load_lds_dwordx4.  Weights never depend on activations, so producers never wait
//     on other workgroups: HBM keeps streaming while consumers wait on dependencies.
//   * 4 consumer waves wait on the dependency counters of exactly the producers they need,
//     stage the activation columns (RMSNorm applied on the fly) in LDS, run 16x16 MFMAs
//     from the ring (A = weights) and the staged activations (B), reduce the four consumer
//     partials of each tile in fixed order, apply the fused epilogue (rotary embedding + KV
//     write, residual add + per-tile sum of squares, SwiGLU, or a plain store) and bump the
//     counters their consumers poll.  They also run the attention chunks, merged with the
//     log-sum-exp rule by the last chunk to finish.
// Every tile is reduced over its full K inside one workgroup, so there are no cross-workgroup
// partial sums on the weight path.  Progress is guaranteed because work only waits on earlier
// phases and all workgroups are co-resident.
//
// Cross-XCD visibility without L2 maintenance: values handed between workgroups are stored and
// loaded with agent-scope coherent accesses; a producer of such values drains its stores
// before bumping a counter, and consumers load them only after observing the counter.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace ls {

enum Phase { PH_INIT = 0, PH_QKV = 1, PH_ATT = 2, PH_O = 3, PH_GU = 4, PH_DOWN = 5, PH_HEAD = 6 };
constexpr int ATT_CH = 64;              // keys per attention unit
constexpr int NCONS = 4, NPROD = 4;
constexpr int MEGA_THREADS = 64 * (NCONS + NPROD);
constexpr int SLAB = 8192;              // bytes: 16 rows x 512 bytes
constexpr int PADC = 64;                // counters that are polled get their own 256-byte line

// ---- coherent (agent-scope) accesses ---------------------------------------------------------
LS_DEV void drain() { __builtin_amdgcn_s_waitcnt(0); }
LS_DEV int ld_acq(const int* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
LS_DEV float ldc(const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
LS_DEV void stc(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
LS_DEV uint16_t ldc(const uint16_t* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
LS_DEV void stc(uint16_t* p, uint16_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
LS_DEV unsigned long long ldc64(const void* p) {
  return __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T> struct Coh;
template <> struct Coh<uint16_t> {
  LS_DEV static void store(uint16_t* p, float v) { stc(p, f2bf(v)); }
  LS_DEV static uint16_t raw(const uint16_t* p) { return ldc(p); }
};
template <> struct Coh<float> {
  LS_DEV static void store(float* p, float v) { stc(p, v); }
  LS_DEV static float raw(const float* p) { return ldc(p); }
};

// Every wait below is bounded: after SPIN_LIMIT polls (about a second) the wait gives up and
// records LS_TIMEOUT in the error word, so a broken dependency ends the kernel with an error
// instead of hanging the device.
constexpr int SPIN_LIMIT = 1 << 25;
constexpr int LS_TIMEOUT = 5;

// ---- LDS synchronisation among the consumer waves only -----------------------------------------
LS_DEV int lds_ld(const int* p) { return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP); }
LS_DEV void lds_add(int* p, int v) { __hip_atomic_fetch_add(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP); }

struct ConsBar {
  int* ctr;
  int gen;
  int* err;
  LS_DEV void sync() {
    gen += NCONS;
    if ((threadIdx.x & 63) == 0) {
      lds_add(ctr, 1);
      int n = 0;
      while (lds_ld(ctr) < gen) {
        __builtin_amdgcn_s_sleep(0);
        if (++n > SPIN_LIMIT) { ls_flag(err, LS_TIMEOUT); break; }
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
};

// Consumer-side wait until *c >= target (one lane polls), then all consumer waves proceed.
LS_DEV void wait_ge(const int* c, int target, ConsBar& cb) {
  if (threadIdx.x == 0) {
    int n = 0;
    while (ld_acq(c) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (++n > SPIN_LIMIT) { ls_flag(cb.err, LS_TIMEOUT); break; }
    }
  }
  cb.sync();
}

// ---- counter layout -----------------------------------------------------------------------------
struct CntLayout {
  int per_layer, nchF;
  int o_qkvh, o_att, o_o, o_gu, o_down, o_fa;
  int o_init, total;
};

__host__ __device__ inline CntLayout cnt_layout(int M, int F, int nh, int XC, int n_layers) {
  CntLayout c;
  c.nchF = (F + XC - 1) / XC;
  int o = 0;
  c.o_qkvh = o; o += nh * PADC;
  c.o_att = o; o += nh * PADC;
  c.o_o = o; o += PADC;
  c.o_gu = o; o += c.nchF * PADC;
  c.o_down = o; o += PADC;
  c.o_fa = o; o += M * nh;
  o = (o + PADC - 1) / PADC * PADC;
  c.per_layer = o;
  c.o_init = n_layers * o;
  c.total = c.o_init + PADC;
  return c;
}

// LDS plan by row count and element size: ring depth, activation columns staged per chunk
// (a multiple of every slab width), and single/double buffering of the tile reduction.
struct LdsPlan {
  int NS, XC, nred;
};
__host__ __device__ inline size_t lds_bytes_for(int M, int esz, int NS, int XC, int nred) {
  size_t off = (size_t)NS * SLAB;
  off = (off + (size_t)M * (XC + 16 / esz) * esz + 15) & ~(size_t)15;
  off = (off + (size_t)nred * NCONS * M * 16 * 4 + 15) & ~(size_t)15;
  off = (off + (size_t)M * 4 + 15) & ~(size_t)15;
  off = (off + (4 * 128 + 64) * 4 + 15) & ~(size_t)15;
  off += (2 * NS + 8) * 4;
  return off;
}
__host__ __device__ inline LdsPlan lds_plan(int M, int esz) {
  LdsPlan p;
  p.NS = M <= 16 ? 12 : 6;
  p.nred = M <= 64 ? 2 : 1;
  const int sk = 512 / esz;
  p.XC = 2048;
  while (p.XC > sk && lds_bytes_for(M, esz, p.NS, p.XC, p.nred) > 160 * 1024 - 512) p.XC /= 2;
  return p;
}
__host__ __device__ inline int x_chunk_for(int M, int esz) { return lds_plan(M, esz).XC; }

// accumulators of this many tiles stay in registers per consumer wave
template <int MT> struct TileBatch { static constexpr int value = MT == 1 ? 16 : (MT == 2 ? 4 : (MT == 4 ? 2 : 1)); };

size_t mega_counter_ints(int M, int d, int F, int nh, int V, int KU, int n_layers) {
  (void)V; (void)KU; (void)d;
  size_t worst = 0;
  for (int m = 1; m <= M; ++m)
    for (int esz = 2; esz <= 4; esz += 2)
      worst = std::max(worst, (size_t)cnt_layout(m, F, nh, x_chunk_for(m, esz), n_layers).total);
  return worst;
}

// ---- LDS layout -----------------------------------------------------------------------------------
struct Lds {
  char* ring;        // NS slabs
  char* X;           // M x (XC + pad) elements
  float* red;        // nred x NCONS x M x 16: per-tile partials of the consumer waves
  float* rinv;       // M
  float* scr;        // attention scratch: 4*128 + 64 floats
  int* ints;         // [0..NS) full, [NS..2NS) empty, [2NS] consumer barrier, [2NS+1..] flags
  int xstride;       // elements
  int NS, XC, nred;
};

LS_DEV size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

template <typename T>
LS_DEV Lds lds_carve(char* base, int M) {
  Lds s;
  const LdsPlan pl = lds_plan(M, (int)sizeof(T));
  s.NS = pl.NS;
  s.XC = pl.XC;
  s.nred = pl.nred;
  s.xstride = s.XC + 16 / (int)sizeof(T);
  size_t off = 0;
  s.ring = base; off += (size_t)s.NS * SLAB;
  s.X = base + off; off = align16(off + (size_t)M * s.xstride * sizeof(T));
  s.red = (float*)(base + off); off = align16(off + (size_t)s.nred * NCONS * M * 16 * 4);
  s.rinv = (float*)(base + off); off = align16(off + (size_t)M * 4);
  s.scr = (float*)(base + off); off = align16(off + (4 * 128 + 64) * 4);
  s.ints = (int*)(base + off);
  return s;
}

size_t mega_smem_bytes(bool bf16, int M, int KU) {
  (void)KU;
  const int esz = bf16 ? 2 : 4;
  const LdsPlan p = lds_plan(M, esz);
  return lds_bytes_for(M, esz, p.NS, p.XC, p.nred);
}

// ---- phase geometry -------------------------------------------------------------------------------
struct PhaseGeo {
  int n_tiles, K;
  int sk;                  // elements per slab row (512 bytes)
};

template <typename T>
LS_DEV PhaseGeo phase_geo(const MegaArgs& a, int ph) {
  PhaseGeo g;
  g.sk = 512 / (int)sizeof(T);
  if (ph == PH_QKV) { g.n_tiles = 3 * a.d / 16; g.K = a.d; }
  else if (ph == PH_GU) { g.n_tiles = a.F / 8; g.K = a.d; }
  else if (ph == PH_HEAD) { g.n_tiles = (a.V + 15) / 16; g.K = a.d; }
  else if (ph == PH_DOWN) { g.n_tiles = a.d / 16; g.K = a.F; }
  else { g.n_tiles = a.d / 16; g.K = a.d; }
  return g;
}

// Weight row r (0..15) of tile t: byte pointer of the row start.
template <typename T>
LS_DEV const char* wrow(const MegaArgs& a, const LayerW& lw, int ph, int t, int r, int K) {
  const size_t rb = (size_t)K * sizeof(T);
  if (ph == PH_QKV) {
    const int tpm = a.d / 16, tph = a.hd / 16;
    const int mat = t / tpm, tl = t % tpm;
    const int h = tl / tph, jj = tl % tph;
    const int n = h * a.hd + 8 * jj + (r & 7) + (r < 8 ? 0 : a.hd / 2);
    const void* W = mat == 0 ? lw.Wq : (mat == 1 ? lw.Wk : lw.Wv);
    return (const char*)W + (size_t)n * rb;
  }
  if (ph == PH_GU) return (const char*)(r < 8 ? lw.Wg : lw.Wu) + (size_t)(8 * t + (r & 7)) * rb;
  const void* W = ph == PH_O ? lw.Wo : (ph == PH_DOWN ? lw.Wd : a.emb);
  const int N = ph == PH_HEAD ? a.V : a.d;
  const int n = min(16 * t + r, N - 1);
  return (const char*)W + (size_t)n * rb;
}

template <typename T> struct Mma;
template <> struct Mma<uint16_t> {
  LS_DEV static void run(f32x4_t& c, const u32x4_t& a, const u32x4_t& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  LS_DEV static void run(f32x4_t& c, const u32x4_t& a, const u32x4_t& b) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[e]), __uint_as_float(b[e]), c, 0, 0, 0);
  }
};

// The workgroup's tiles of a phase are t = first + i*G for i < count (round-robin dealing that
// continues from phase to phase so every workgroup gets about the same bytes per call).
struct Share {
  int first, count;
};
LS_DEV Share share_of(int n, int deal, int G, int b) {
  Share s;
  s.first = ((b - deal) % G + G) % G;
  s.count = s.first < n ? (n - 1 - s.first) / G + 1 : 0;
  return s;
}

// vmcnt-only wait with a compile-time count (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt[5:4] << 14; expcnt/lgkmcnt at their maxima = no wait).
template <int N>
LS_DEV void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// =========================================== producer ===========================================
template <typename T, int DP>
struct Producer {
  const MegaArgs& a;
  const Lds& s;
  int p;           // producer index 0..3
  int lane;
  int j = 0;       // slabs issued
  int pub = 0;     // slabs published

  LS_DEV Producer(const MegaArgs& a_, const Lds& s_, int p_) : a(a_), s(s_), p(p_), lane(threadIdx.x & 63) {}

  LS_DEV void publish_one() {
    if (lane == 0) lds_add(s.ints + (pub % s.NS), 1);
    ++pub;
  }

  // Copy slab (t, k) of phase ph into the next ring slot: this producer's four rows, as two
  // 1 KB direct-to-LDS loads.  Lane l of a load carries 16 bytes of row 4p + 2i + l/32; the
  // 16-byte chunk index is XOR-swizzled with the row so consumers read conflict-free.
  LS_DEV void issue(const LayerW& lw, int ph, int t, int k, const PhaseGeo& g) {
    const int slot = j % s.NS, use = j / s.NS;
    if (use > 0) {
      if (lane == 0) {
        int n = 0;
        while (lds_ld(s.ints + s.NS + slot) < use) {
          __builtin_amdgcn_s_sleep(0);
          if (++n > SPIN_LIMIT) { ls_flag(a.err, LS_TIMEOUT); break; }
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
    const int k0 = k * g.sk;
    const int kn = min(g.sk, g.K - k0);
    constexpr int E = 16 / (int)sizeof(T);
    const int nch = kn / E;                         // valid 16-byte chunks in each row
    char* dst = s.ring + (size_t)slot * SLAB;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int rho = 4 * p + 2 * i + (lane >> 5);
      const int pos = lane & 31;
      int ch = pos ^ (rho & 31);
      if (ch >= nch) ch = 0;
      const char* src = wrow<T>(a, lw, ph, t, rho, g.K) + ((size_t)k0 + (size_t)ch * E) * sizeof(T);
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(dst + (4 * p + 2 * i) * 512),
                                       16, 0, 0);
    }
    ++j;
    if (j - pub > DP) {
      wait_vm<2 * DP>();
      publish_one();
    }
  }

  LS_DEV void finish() {
    wait_vm<0>();
    while (pub < j) publish_one();
  }
};

// =========================================== consumer ===========================================
template <typename T, int MT>
struct Consumer {
  const MegaArgs& a;
  const Lds& s;
  ConsBar& cb;
  int c;            // consumer index 0..3
  int lane;
  int j = 0;        // slabs passed in the sequence
  int rinv_tag = -1;

  LS_DEV Consumer(const MegaArgs& a_, const Lds& s_, ConsBar& cb_, int c_)
      : a(a_), s(s_), cb(cb_), c(c_), lane(threadIdx.x & 63) {}

  // RMSNorm factors for all rows, once per (layer, phase).
  LS_DEV void compute_rinv(const float* ssq, const float* Hsrc, bool via_hidx, int tag) {
    if (rinv_tag == tag) return;
    const int nt = a.d / 16;
    for (int m = c; m < a.M; m += NCONS) {
      float acc = 0.f;
      if (ssq) {
        for (int t = lane; t < nt; t += 64) acc += ldc(ssq + (size_t)t * a.M + m);
      } else {
        const int hr = via_hidx ? (a.hidx ? a.hidx[m] : m) : m;
        if (hr >= 0)
          for (int k = lane; k < a.d; k += 64) {
            const float x = ldc(Hsrc + (size_t)hr * a.d + k);
            acc += x * x;
          }
      }
      acc = warp_sum(acc);
      if (lane == 0) s.rinv[m] = 1.0f / sqrtf(acc / (float)a.d + a.eps);
    }
    rinv_tag = tag;
    cb.sync();
  }

  // Stage activation columns [x0, x0 + xn) of phase ph into LDS.
  LS_DEV void stage_x(int ph, const LayerW& lw, int x0, int xn, int K) {
    T* X = (T*)s.X;
    const int tid = threadIdx.x;          // consumers are threads 0..255
    if (ph == PH_QKV || ph == PH_GU || ph == PH_HEAD) {
      const float* gain = ph == PH_QKV ? lw.g1 : (ph == PH_GU ? lw.g2 : a.g_final);
      for (int idx = tid; idx < a.M * xn; idx += 64 * NCONS) {
        const int m = idx / xn, kk = idx - m * xn;
        float x;
        if (ph == PH_GU) {
          x = ldc(a.Hb + (size_t)m * a.d + x0 + kk);
        } else {
          const int hr = a.hidx ? a.hidx[m] : m;
          x = hr >= 0 ? ldc(a.H + (size_t)hr * a.d + x0 + kk) : 0.f;
        }
        Elem<T>::store(X + (size_t)m * s.xstride + kk, x * s.rinv[m] * gain[x0 + kk]);
      }
    } else {
      const T* src = (const T*)(ph == PH_O ? a.o : a.act);
      for (int idx = tid; idx < a.M * xn; idx += 64 * NCONS) {
        const int m = idx / xn, kk = idx - m * xn;
        X[(size_t)m * s.xstride + kk] = Coh<T>::raw(src + (size_t)m * K + x0 + kk);
      }
    }
    cb.sync();
  }

  // Pass one slab of the sequence; if it is this consumer's (q mod 4 == c), multiply it.
  LS_DEV void slab(int q, int kn, f32x4_t* acc) {
    const int slot = j % s.NS, use = j / s.NS;
    ++j;
    if (q % NCONS != c) return;
    if (lane == 0) {
      int n = 0;
      while (lds_ld(s.ints + slot) < (use + 1) * NPROD) {
        __builtin_amdgcn_s_sleep(0);
        if (++n > SPIN_LIMIT) { ls_flag(a.err, LS_TIMEOUT); break; }
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    constexpr int E = 16 / (int)sizeof(T);
    const int r = lane & 15, g = lane >> 4;
    const char* base = s.ring + (size_t)slot * SLAB + r * 512;
    const int nst = kn / (4 * E);
    const int xoff = q * (512 / (int)sizeof(T));     // element offset of this slab in the staged chunk
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      if (v < nst) {
        const int ch = 4 * v + g;
        const u32x4_t w = *reinterpret_cast<const u32x4_t*>(base + ((ch ^ (r & 31)) * 16));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int m = mt * 16 + r;
          u32x4_t x = u32x4_t{0u, 0u, 0u, 0u};
          if (m < a.M)
            x = *reinterpret_cast<const u32x4_t*>((const T*)s.X + (size_t)m * s.xstride + xoff + ch * E);
          Mma<T>::run(acc[mt], w, x);
        }
      }
    }
    // ring reads are complete (their values fed the MFMAs) before the slot is released
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (lane == 0) lds_add(s.ints + s.NS + slot, 1);
  }
};

// Epilogue of one finished tile (its sum over the four consumers is in Ts[m*16 + n]).
template <typename T>
LS_DEV void epilogue(const MegaArgs& a, const CntLayout& cl, int ph, int l, int t, const float* Ts, int lane) {
  int* C = a.cnt + (size_t)l * cl.per_layer;
  if (ph == PH_QKV) {
    const int tpm = a.d / 16, tph = a.hd / 16;
    const int mat = t / tpm, tl = t % tpm;
    const int h = tl / tph, jj = tl % tph;
    for (int idx = lane; idx < a.M * 8; idx += 64) {
      const int m = idx >> 3, p = idx & 7;
      const int i = 8 * jj + p;
      const int e0 = h * a.hd + i, e1 = e0 + a.hd / 2;
      float y0 = Ts[m * 16 + p], y1 = Ts[m * 16 + p + 8];
      if (mat < 2) {
        const double ang = (double)a.pos[m] * a.inv_freq[i];
        const float cs = (float)cos(ang), sn = (float)sin(ang);
        const float r0 = y0 * cs - y1 * sn, r1 = y1 * cs + y0 * sn;
        y0 = r0; y1 = r1;
      }
      if (mat == 0) {
        stc(a.q + (size_t)m * a.d + e0, y0);
        stc(a.q + (size_t)m * a.d + e1, y1);
      } else {
        const int sl = a.slot[m];
        if (sl < 0) continue;
        const int blk = (a.dep ? a.dep[m] + a.dep_off : 0) * a.blk_mul + a.layer0 + l;
        T* ent = (T*)a.kv + ((size_t)blk * a.S + sl) * 2 * a.d + (mat == 2 ? a.d : 0);
        Coh<T>::store(ent + e0, y0);
        Coh<T>::store(ent + e1, y1);
      }
    }
    drain();
    if (lane == 0) atomicAdd(C + cl.o_qkvh + h * PADC, 1);
  } else if (ph == PH_O || ph == PH_DOWN) {
    float* ssq = a.ssq + ((size_t)l * 2 + (ph == PH_DOWN)) * (a.d / 16) * a.M;
    for (int m = lane; m < a.M; m += 64) {
      const int hr = a.hidx ? a.hidx[m] : m;
      float sq = 0.f;
      for (int nl = 0; nl < 16; ++nl) {
        const int n = 16 * t + nl;
        const float y = Ts[m * 16 + nl];
        float nv = 0.f;
        if (hr >= 0) {
          if (ph == PH_O) {
            nv = ldc(a.H + (size_t)hr * a.d + n) + y;
            stc(a.Hb + (size_t)m * a.d + n, nv);
          } else {
            nv = ldc(a.Hb + (size_t)m * a.d + n) + y;
            stc(a.H + (size_t)hr * a.d + n, nv);
          }
        } else if (ph == PH_O) {
          stc(a.Hb + (size_t)m * a.d + n, 0.f);
        }
        sq += nv * nv;
      }
      stc(ssq + (size_t)t * a.M + m, sq);
    }
    drain();
    if (lane == 0) atomicAdd(C + (ph == PH_O ? cl.o_o : cl.o_down), 1);
  } else if (ph == PH_GU) {
    T* act = (T*)a.act;
    for (int idx = lane; idx < a.M * 8; idx += 64) {
      const int m = idx >> 3, p = idx & 7;
      const float gv = Ts[m * 16 + p], uv = Ts[m * 16 + p + 8];
      Coh<T>::store(act + (size_t)m * a.F + 8 * t + p, gv / (1.0f + expf(-gv)) * uv);
    }
    drain();
    if (lane == 0) atomicAdd(C + cl.o_gu + ((8 * t) / x_chunk_for(a.M, (int)sizeof(T))) * PADC, 1);
  } else {  // PH_HEAD
    for (int idx = lane; idx < a.M * 16; idx += 64) {
      const int m = idx >> 4, nl = idx & 15, n = 16 * t + nl;
      if (n < a.V) a.logits[(size_t)m * a.ldo + n] = Ts[idx];
    }
  }
}

// ---- attention unit (consumer waves) -----------------------------------------------------------------
template <typename T>
LS_DEV void load8f(const T* p, float* v);
template <>
LS_DEV void load8f<uint16_t>(const uint16_t* p, float* v) {
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const unsigned long long x = ldc64(p + 4 * h2);
    const unsigned lo = (unsigned)x, hi = (unsigned)(x >> 32);
    v[4 * h2 + 0] = __uint_as_float(lo << 16);
    v[4 * h2 + 1] = __uint_as_float(lo & 0xffff0000u);
    v[4 * h2 + 2] = __uint_as_float(hi << 16);
    v[4 * h2 + 3] = __uint_as_float(hi & 0xffff0000u);
  }
}
template <>
LS_DEV void load8f<float>(const float* p, float* v) {
#pragma unroll
  for (int h2 = 0; h2 < 4; ++h2) {
    const unsigned long long x = ldc64(p + 2 * h2);
    v[2 * h2] = __uint_as_float((unsigned)x);
    v[2 * h2 + 1] = __uint_as_float((unsigned)(x >> 32));
  }
}

template <typename T>
LS_DEV void att_unit(const MegaArgs& a, const Lds& s, const CntLayout& cl, ConsBar& cb, int l, int i, int h, int c) {
  int* C = a.cnt + (size_t)l * cl.per_layer;
  const int self = a.slot[i];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;     // wv = consumer 0..3
  const int kk = lane >> 4, e = lane & 15;
  if (self < 0) {                               // rejected row: zero output, still counted
    if (c == 0) {
      wait_ge(C + cl.o_qkvh + h * PADC, 3 * (a.hd / 16), cb);
      for (int dd = threadIdx.x; dd < a.hd; dd += 64 * NCONS)
        Coh<T>::store((T*)a.o + (size_t)i * a.d + h * a.hd + dd, 0.f);
      drain();
      cb.sync();
      if (threadIdx.x == 0) atomicAdd(C + cl.o_att + h * PADC, 1);
    }
    return;
  }
  const int a0 = a.anc_off[i], na = a.anc_off[i + 1] - a0;
  const int nk = a.n_fin + na + 1;
  const int nc = (nk + ATT_CH - 1) / ATT_CH;
  if (c >= nc) return;
  const int k0 = c * ATT_CH;
  const int kn = min(ATT_CH, nk - k0);
  const int blk = (a.dep ? a.dep[i] + a.dep_off : 0) * a.blk_mul + a.layer0 + l;
  const T* cache = (const T*)a.kv + (size_t)blk * a.S * 2 * a.d;
  const bool dim_ok = 8 * e < a.hd;

  int sl[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int jk = wv * 16 + kk + 4 * rr;
    sl[rr] = -1;
    if (jk < kn) {
      const int x = key_slot(k0 + jk, a.n_fin, a.fin, a.anc, a0, na, self);
      sl[rr] = (x >= 0 && x < a.S) ? x : -1;
      if (x < 0 || x >= a.S) ls_flag(a.err, 1);
    }
  }
  float kf[4][8], vf[4][8];
  const bool early = k0 + kn <= a.n_fin;     // keys written by earlier calls only
  auto load_kv = [&]() {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      if (sl[rr] >= 0 && dim_ok) {
        load8f<T>(cache + (size_t)sl[rr] * 2 * a.d + h * a.hd + 8 * e, kf[rr]);
        load8f<T>(cache + (size_t)sl[rr] * 2 * a.d + a.d + h * a.hd + 8 * e, vf[rr]);
      }
  };
  if (early) load_kv();
  wait_ge(C + cl.o_qkvh + h * PADC, 3 * (a.hd / 16), cb);
  if (!early) load_kv();
  float q[8];
  const float scale = 1.0f / sqrtf((float)a.hd);
#pragma unroll
  for (int t = 0; t < 8; ++t) q[t] = dim_ok ? ldc(a.q + (size_t)i * a.d + h * a.hd + 8 * e + t) * scale : 0.f;
  float sc[4];
  float mloc = -INFINITY;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    float part = 0.f;
    if (sl[rr] >= 0 && dim_ok) {
#pragma unroll
      for (int t = 0; t < 8; ++t) part += q[t] * kf[rr][t];
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
    sc[rr] = sl[rr] >= 0 ? part : -INFINITY;
    mloc = fmaxf(mloc, sc[rr]);
  }
  float* red = s.scr + 4 * 128;
  mloc = warp_max(mloc);
  if (lane == 0) red[wv] = mloc;
  cb.sync();
  const float mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float lsum = 0.f;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const float p = sc[rr] == -INFINITY ? 0.f : __expf(sc[rr] - mx);
    if (e == 0) lsum += p;
    if (sl[rr] >= 0 && dim_ok) {
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] += p * vf[rr][t];
    }
  }
  lsum = warp_sum(lsum);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    acc[t] += __shfl_xor(acc[t], 16, 64);
    acc[t] += __shfl_xor(acc[t], 32, 64);
  }
  cb.sync();                                    // red[] reuse
  if (lane == 0) red[4 + wv] = lsum;
  if (kk == 0 && dim_ok) {
#pragma unroll
    for (int t = 0; t < 8; ++t) s.scr[wv * 128 + 8 * e + t] = acc[t];
  }
  cb.sync();
  float* out = a.patt + (((size_t)i * a.nh + h) * a.att_chunks + c) * (a.hd + 2);
  for (int dd = threadIdx.x; dd < a.hd; dd += 64 * NCONS)
    stc(out + 2 + dd, s.scr[dd] + s.scr[128 + dd] + s.scr[256 + dd] + s.scr[384 + dd]);
  if (threadIdx.x == 0) { stc(out, mx); stc(out + 1, red[4] + red[5] + red[6] + red[7]); }
  drain();
  cb.sync();
  int* flag = s.ints + 2 * s.NS + 1;
  if (threadIdx.x == 0) *flag = atomicAdd(C + cl.o_fa + i * a.nh + h, 1);
  cb.sync();
  const int arrived = *flag;
  cb.sync();
  if (arrived != nc - 1) return;
  // the last chunk merges all chunks of (row, head) in chunk order; the per-chunk maxima and
  // sums are staged in LDS first so every output loads its partials independently
  const float* base = a.patt + ((size_t)i * a.nh + h) * a.att_chunks * (a.hd + 2);
  float* cmx = (float*)s.X;                          // the activation stage is free during attention
  for (int cc = threadIdx.x; cc < nc; cc += 64 * NCONS) {
    cmx[cc] = ldc(base + (size_t)cc * (a.hd + 2));
    cmx[a.att_chunks + cc] = ldc(base + (size_t)cc * (a.hd + 2) + 1);
  }
  cb.sync();
  float M_ = -INFINITY;
  for (int cc = 0; cc < nc; ++cc) M_ = fmaxf(M_, cmx[cc]);
  float den = 0.f;
  for (int cc = 0; cc < nc; ++cc) den += (cmx[cc] == -INFINITY ? 0.f : __expf(cmx[cc] - M_)) * cmx[a.att_chunks + cc];
  for (int dd = threadIdx.x; dd < a.hd; dd += 64 * NCONS) {
    float num = 0.f;
    for (int cc = 0; cc < nc; ++cc) {
      const float wgt = cmx[cc] == -INFINITY ? 0.f : __expf(cmx[cc] - M_);
      num += wgt * ldc(base + (size_t)cc * (a.hd + 2) + 2 + dd);
    }
    Coh<T>::store((T*)a.o + (size_t)i * a.d + h * a.hd + dd, den > 0.f ? num / den : 0.f);
  }
  drain();
  cb.sync();
  if (threadIdx.x == 0) atomicAdd(C + cl.o_att + h * PADC, 1);
}

// ---- init unit: embedding row or gathered hidden row into the working rows ---------------------------
template <typename T>
LS_DEV void init_unit(const MegaArgs& a, const CntLayout& cl, ConsBar& cb, int m) {
  const int hr = a.hidx ? a.hidx[m] : m;
  if (hr >= 0) {
    if (a.init_mode == 1) {
      const int tok = a.tokens[m];
      if (tok >= 0 && tok < a.V) {
        for (int k = threadIdx.x; k < a.d; k += 64 * NCONS)
          stc(a.H + (size_t)hr * a.d + k, Elem<T>::load((const T*)a.emb + (size_t)tok * a.d + k));
      } else if (threadIdx.x == 0) {
        ls_flag(a.err, 1);
      }
    } else {
      const int src = a.gather[m];
      for (int k = threadIdx.x; k < a.d; k += 64 * NCONS)
        stc(a.H + (size_t)hr * a.d + k, src >= 0 ? a.Hg[(size_t)src * a.d + k] : 0.f);
    }
  }
  drain();
  cb.sync();
  if (threadIdx.x == 0) atomicAdd(a.cnt + cl.o_init, 1);
}

// ---- the walk: the same slab sequence for producers and consumers ----------------------------------
// Phase ph of layer l: the workgroup's tiles in batches of TB; within a batch, activation chunk
// by chunk (XC columns); within a chunk, tile by tile, slab by slab.
template <typename T, int MT, int DP, bool PROD>
LS_DEV void walk_gemm(const MegaArgs& a, const Lds& s, const CntLayout& cl, int ph, int l, int& deal,
                      Producer<T, DP>* pr, Consumer<T, MT>* co, ConsBar* cb) {
  const int G = gridDim.x, b = blockIdx.x;
  const PhaseGeo g = phase_geo<T>(a, ph);
  const Share sh = share_of(g.n_tiles, deal, G, b);
  deal = (deal + g.n_tiles) % G;
  if (sh.count == 0) return;
  const LayerW lw = ph == PH_HEAD ? LayerW{} : a.layers[l];
  const int nchunk = (g.K + s.XC - 1) / s.XC;

  if (!PROD) {
    // dependencies of the normalised phases (full rows are needed for the RMSNorm factor)
    const int* C = a.cnt + (size_t)l * cl.per_layer;
    if (ph == PH_QKV) {
      if (l > 0) wait_ge(a.cnt + (size_t)(l - 1) * cl.per_layer + cl.o_down, a.d / 16, *cb);
      else if (a.init_mode) wait_ge(a.cnt + cl.o_init, a.M, *cb);
      const float* ssq = l > 0 ? a.ssq + ((size_t)(l - 1) * 2 + 1) * (a.d / 16) * a.M : nullptr;
      co->compute_rinv(ssq, a.H, true, l * 8 + ph);
    } else if (ph == PH_GU) {
      wait_ge(C + cl.o_o, a.d / 16, *cb);
      co->compute_rinv(a.ssq + ((size_t)l * 2) * (a.d / 16) * a.M, a.Hb, false, l * 8 + ph);
    } else if (ph == PH_HEAD) {
      if (a.n_layers > 0) wait_ge(a.cnt + (size_t)(a.n_layers - 1) * cl.per_layer + cl.o_down, a.d / 16, *cb);
      else if (a.init_mode) wait_ge(a.cnt + cl.o_init, a.M, *cb);
      const float* ssq = a.n_layers > 0 ? a.ssq + ((size_t)(a.n_layers - 1) * 2 + 1) * (a.d / 16) * a.M : nullptr;
      co->compute_rinv(ssq, a.H, true, l * 8 + ph);
    }
  }

  constexpr int TBM = TileBatch<MT>::value;
  for (int b0 = 0; b0 < sh.count; b0 += TBM) {
    const int nb = min(TBM, sh.count - b0);
    f32x4_t acc[TBM][MT];
    if (!PROD) {
#pragma unroll
      for (int tb = 0; tb < TBM; ++tb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[tb][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    for (int ch = 0; ch < nchunk; ++ch) {
      const int x0 = ch * s.XC;
      const int xn = min(s.XC, g.K - x0);
      if (!PROD) {
        const int* C = a.cnt + (size_t)l * cl.per_layer;
        if (ph == PH_O) {
          for (int h = x0 / a.hd; h <= (x0 + xn - 1) / a.hd; ++h) wait_ge(C + cl.o_att + h * PADC, a.M, *cb);
        } else if (ph == PH_DOWN) {
          wait_ge(C + cl.o_gu + ch * PADC, xn / 8, *cb);
        } else {
          cb->sync();                     // previous chunk's readers are done with X
        }
        co->stage_x(ph, lw, x0, xn, g.K);
      }
      const int k_first = x0 / g.sk;
      const int k_last = (x0 + xn + g.sk - 1) / g.sk;
      for (int tb = 0; tb < nb; ++tb) {
        const int t = sh.first + (b0 + tb) * G;
        for (int k = k_first; k < k_last; ++k) {
          if (PROD) {
            pr->issue(lw, ph, t, k, g);
          } else {
            const int kn = min(g.sk, g.K - k * g.sk);
            // constant-index accumulator selection keeps acc in registers
#pragma unroll
            for (int tt = 0; tt < TBM; ++tt)
              if (tt == tb) co->slab(k - k_first, kn, acc[tt]);
          }
        }
      }
    }
    if (!PROD) {
      // per tile: the four consumer partials meet in LDS and are summed in consumer order by
      // consumer (tile mod 4), which then runs the epilogue
      const int lane = threadIdx.x & 63, r = lane & 15, gq = lane >> 4;
      for (int tb = 0; tb < nb; ++tb) {
        float* buf = s.red + (size_t)(tb % s.nred) * NCONS * a.M * 16;
#pragma unroll
        for (int tt = 0; tt < TBM; ++tt) {
          if (tt == tb) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              const int m = mt * 16 + r;
              if (m < a.M) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) buf[((size_t)co->c * a.M + m) * 16 + 4 * gq + jj] = acc[tt][mt][jj];
              }
            }
          }
        }
        cb->sync();
        if (tb % NCONS == co->c) {
          for (int idx = lane; idx < a.M * 16; idx += 64) {
            float y = 0.f;
#pragma unroll
            for (int cc = 0; cc < NCONS; ++cc) y += buf[(size_t)cc * a.M * 16 + idx];
            buf[idx] = y;                 // consumer 0's slot now holds the tile sum
          }
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
          epilogue<T>(a, cl, ph, l, sh.first + (b0 + tb) * G, buf, lane);
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
        }
        if (s.nred == 1) cb->sync();      // single buffer: the sum is read before the next tile
      }
      cb->sync();                         // reduction buffers reusable
    }
  }
}

template <typename T, int MT, int DP>
__global__ __launch_bounds__(MEGA_THREADS) void k_mega(MegaArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  const Lds s = lds_carve<T>(smem_raw, a.M);
  const CntLayout cl = cnt_layout(a.M, a.F, a.nh, x_chunk_for(a.M, (int)sizeof(T)), a.n_layers);
  const int G = gridDim.x, b = blockIdx.x;
  const int wv = threadIdx.x >> 6;
  // ring counters and the consumer barrier start at zero
  for (int i = threadIdx.x; i < 2 * s.NS + 8; i += MEGA_THREADS) s.ints[i] = 0;
  __syncthreads();
  int deal = 0;
  if (wv >= NCONS) {
    // ------------------------------ producer waves ------------------------------
    Producer<T, DP> pr(a, s, wv - NCONS);
    for (int l = 0; l < a.n_layers; ++l) {
      walk_gemm<T, MT, DP, true>(a, s, cl, PH_QKV, l, deal, &pr, nullptr, nullptr);
      walk_gemm<T, MT, DP, true>(a, s, cl, PH_O, l, deal, &pr, nullptr, nullptr);
      walk_gemm<T, MT, DP, true>(a, s, cl, PH_GU, l, deal, &pr, nullptr, nullptr);
      walk_gemm<T, MT, DP, true>(a, s, cl, PH_DOWN, l, deal, &pr, nullptr, nullptr);
    }
    if (a.do_head) walk_gemm<T, MT, DP, true>(a, s, cl, PH_HEAD, a.n_layers, deal, &pr, nullptr, nullptr);
    pr.finish();
    return;
  }
  // ------------------------------ consumer waves ------------------------------
  ConsBar cb{s.ints + 2 * s.NS, 0, a.err};
  Consumer<T, MT> co(a, s, cb, wv);
  auto stamp = [&](int l, int ph, int e) {
    if (a.trace && l < 4 && threadIdx.x == 0) a.trace[(((size_t)b * 4 + l) * 6 + ph) * 2 + e] = wall_clock64();
  };
  if (a.init_mode)
    for (int u = b; u < a.M; u += G) init_unit<T>(a, cl, cb, u);
  int att_deal = 0;
  for (int l = 0; l < a.n_layers; ++l) {
    stamp(l, 1, 0);
    walk_gemm<T, MT, DP, false>(a, s, cl, PH_QKV, l, deal, nullptr, &co, &cb);
    stamp(l, 1, 1);
    stamp(l, 2, 0);
    const int natt = a.M * a.nh * a.att_chunks;
    const Share sa = share_of(natt, att_deal, G, b);
    att_deal = (att_deal + natt) % G;
    for (int k = 0; k < sa.count; ++k) {
      const int u = sa.first + k * G;
      const int cch = u % a.att_chunks, ih = u / a.att_chunks;
      att_unit<T>(a, s, cl, cb, l, ih / a.nh, ih % a.nh, cch);
    }
    stamp(l, 2, 1);
    stamp(l, 3, 0);
    walk_gemm<T, MT, DP, false>(a, s, cl, PH_O, l, deal, nullptr, &co, &cb);
    stamp(l, 3, 1);
    stamp(l, 4, 0);
    walk_gemm<T, MT, DP, false>(a, s, cl, PH_GU, l, deal, nullptr, &co, &cb);
    stamp(l, 4, 1);
    stamp(l, 5, 0);
    walk_gemm<T, MT, DP, false>(a, s, cl, PH_DOWN, l, deal, nullptr, &co, &cb);
    stamp(l, 5, 1);
  }
  if (a.do_head) walk_gemm<T, MT, DP, false>(a, s, cl, PH_HEAD, a.n_layers, deal, nullptr, &co, &cb);
}

__global__ void k_zero_i32(int* p, long long n) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    p[i] = 0;
}

template <typename T>
static const void* pick_t(int mt) {
  if (mt <= 1) return reinterpret_cast<const void*>(&k_mega<T, 1, 8>);
  if (mt <= 2) return reinterpret_cast<const void*>(&k_mega<T, 2, 4>);
  if (mt <= 4) return reinterpret_cast<const void*>(&k_mega<T, 4, 4>);
  return reinterpret_cast<const void*>(&k_mega<T, 8, 4>);
}

static const void* pick(bool bf16, int M) {
  const int mt = (M + 15) / 16;
  return bf16 ? pick_t<uint16_t>(mt) : pick_t<float>(mt);
}

int mega_occupancy(bool bf16, int M, int KU) {
  const size_t smem = mega_smem_bytes(bf16, M, KU);
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, pick(bf16, M), MEGA_THREADS, smem) != hipSuccess) return 0;
  return n;
}

hipError_t launch_mega(bool bf16, const MegaArgs& a, int G, hipStream_t s) {
  const CntLayout cl = cnt_layout(a.M, a.F, a.nh, x_chunk_for(a.M, bf16 ? 2 : 4), a.n_layers);
  hipLaunchKernelGGL(k_zero_i32, dim3(std::min(1024, (cl.total + 255) / 256)), dim3(256), 0, s, a.cnt,
                     (long long)cl.total);
  const size_t smem = mega_smem_bytes(bf16, a.M, a.KU);
  void* args[] = {(void*)&a};
  return hipLaunchCooperativeKernel(pick(bf16, a.M), dim3(G), dim3(MEGA_THREADS), args, (unsigned)smem, s);
}

}  // namespace ls
