// Persistent producer/consumer kernel for the transformer layers of one call (ls_loop_step:
// the shared block B applied once to every branch row; ls_prelude: embedding + prelude
// layers; ls_readout: coda layers + final norm + LM head).
//
// One cooperative launch of resident 448-thread workgroups (one per CU for the model shapes
// here).  Each workgroup owns a static share of every projection's 16-output-feature tiles
// (dealt round-robin across the phases of the call, so every workgroup streams about the same
// bytes) and of the attention units.  Its seven waves are specialised:
//   * 2 producer waves walk the workgroup's weight-slab sequence (slab = 16 rows x 512 bytes)
//     across all phases and layers and copy whole slabs straight into an LDS ring with
//     global_load_lds_dwordx4.  Weights never depend on activations, so producers never wait
//     on other workgroups: HBM keeps streaming while consumers wait on dependencies.
//   * 4 consumer waves wait for their inputs (polling the data itself where it is filled
//     with a NaN pattern beforehand, else the producing tiles' counters), stage the
//     activation columns (RMSNorm applied on the fly) in LDS, run 16x16 MFMAs from the ring
//     (A = weights) and the staged activations (B), and post their partial tile sums to LDS.
//     Between the QKV and O projections they run attention: one wave per (depth group, head,
//     unit of the shared prefix's keys), with the rows of one depth group sharing the prefix
//     keys; the last unit of a (group, head) to finish merges the partials with the
//     log-sum-exp rule.
//   * 1 epilogue wave sums each tile's four partials in fixed order and applies the fused
//     epilogue (rotary embedding + q and KV stores, residual add + per-tile sum of squares,
//     SwiGLU, or the logits store), then signals the tile where its readers use counters.
// Every tile is reduced over its full K inside one workgroup, so there are no cross-workgroup
// partial sums on the weight path.  Progress is guaranteed because work only waits on earlier
// phases and all workgroups are co-resident; every wait is bounded.
//
// Cross-XCD visibility without L2 maintenance: values handed between workgroups are stored and
// loaded with agent-scope coherent accesses; a producer of counted values drains its stores
// before bumping a counter, and consumers load them only after observing the counter.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace ls {

enum Phase { PH_INIT = 0, PH_QKV = 1, PH_ATT = 2, PH_O = 3, PH_GU = 4, PH_DOWN = 5, PH_HEAD = 6 };
constexpr int NCONS = 4, NPROD = 2, NEPI = 1;
constexpr int MEGA_THREADS = 64 * (NCONS + NPROD + NEPI);
constexpr int EPI_WAVE = NCONS + NPROD;  // wave index of the epilogue wave
constexpr int SLAB = 8192;              // bytes: 16 rows x 512 bytes
constexpr int PADC = 64;                // counters that are polled get their own 256-byte line

// Wave index within the workgroup, known to the compiler to be wave-uniform (kept in SGPRs;
// values derived from threadIdx.x are otherwise treated as divergent, which turns the walk's
// bookkeeping into VGPR arithmetic under exec masks).
LS_DEV int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

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

// 16-byte coherent loads through a buffer descriptor: the SC1 cache-policy bit makes them the
// same agent-coherent access as the atomic loads above, four words at a time.  A descriptor
// covers n_bytes from base; the hardware range check returns zeros beyond it, so ragged row
// ends and absent rows (n_bytes = 0) need no branches.
constexpr int CPOL_SC1 = 16;
LS_DEV __amdgpu_buffer_rsrc_t rsrc_of(const void* base, int n_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n_bytes, 0x00020000);
}
LS_DEV u32x4_t ldc128(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, CPOL_SC1);
}
// Plain (cached) 16-byte load.  Used for activations that every workgroup reads: each is
// written exactly once per launch (per-layer buffers) and read only after its producers'
// counters, so no cache can hold an older copy of it, and the workgroups of one XCD share
// one L2 fill instead of each going to memory.
LS_DEV u32x4_t ld128(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

// Layer inputs Xs[l] (l >= 1) and post-attention rows Ys[l] start every launch filled with
// SENT32 (a NaN bit pattern that arithmetic does not produce: generated NaNs are the
// positive canonical one, and no input element converts to it).  Their readers poll the data
// itself with agent-coherent loads instead of a completion counter: a row is complete when no
// element still holds SENT32.  The epilogues still count their tiles for the other readers.
// The attention outputs o[l] are polled the same way by the O phase (all-ones words: 0xFFFF
// halves in bf16, also a NaN pattern no merge stores), so the merge signals nothing.
constexpr unsigned SENT32 = 0xFFFFFFFFu;
// Rows up to this many columns are staged, normalised and (for Xs / Ys) polled in one pass.
constexpr int FUSE_MAX_K = 2048;

// Per-layer activation buffers of one launch (rows m < M):
//   layer input   l == 0: H[hidx[m]] (the caller's hidden rows), l > 0: Xs[l][m]
//   after attention residual: Ys[l][m];  attention output o[l][m];  SwiGLU output act[l][m]
// The last layer's output goes to H[hidx[m]] and, when the LM head follows, to Xs[n_layers].
LS_DEV const float* layer_in(const MegaArgs& a, int l) { return l == 0 ? a.H : a.Xs + (size_t)l * a.M * a.d; }
LS_DEV float* ys_of(const MegaArgs& a, int l) { return a.Ys + (size_t)l * a.M * a.d; }
template <typename T> LS_DEV T* o_of(const MegaArgs& a, int l) { return (T*)a.o + (size_t)l * a.M * a.d; }
template <typename T> LS_DEV T* act_of(const MegaArgs& a, int l) { return (T*)a.act + (size_t)l * a.M * a.F; }

template <typename T> struct Coh;
template <> struct Coh<uint16_t> {
  LS_DEV static void store(uint16_t* p, float v) { stc(p, f2bf(v)); }
  LS_DEV static uint16_t raw(const uint16_t* p) { return ldc(p); }
};
template <> struct Coh<float> {
  LS_DEV static void store(float* p, float v) { stc(p, v); }
  LS_DEV static float raw(const float* p) { return ldc(p); }
};
// A 32-bit word of the polled attention output that still holds (part of) the fill pattern.
template <typename T> LS_DEV bool holds_fill(unsigned w);
template <> LS_DEV bool holds_fill<uint16_t>(unsigned w) { return (w & 0xffffu) == 0xffffu || (w >> 16) == 0xffffu; }
template <> LS_DEV bool holds_fill<float>(unsigned w) { return w == 0xffffffffu; }

// Every wait below is bounded: after SPIN_LIMIT polls (about a second) the wait gives up and
// records LS_TIMEOUT in the error word, so a broken dependency ends the kernel with an error
// instead of hanging the device.
constexpr int SPIN_LIMIT = 1 << 25;
// Global counters are polled by up to every workgroup at once; each poll is a memory access
// to the same line, so polls are spaced (s_sleep units of 64 cycles) to leave that line's
// bandwidth to the atomics that move the counter.
#ifndef LS_POLL_SLEEP
#define LS_POLL_SLEEP 8
#endif
constexpr int POLL_SLEEP = LS_POLL_SLEEP;
constexpr int LS_TIMEOUT = 5;

// ---- LDS synchronisation among the consumer waves only -----------------------------------------

// LDS signalling from inline assembly.  A compiler-visible LDS access after direct-to-LDS
// loads (producers) gets a conservative wait for every one still in flight, and release or
// acquire orderings make a wave wait for all of its outstanding global stores (consumers);
// neither is needed for LDS-to-LDS signalling, where a wave's LDS operations complete in order.
LS_DEV int lds_peek(const int* p) {
  const unsigned addr = (unsigned)(size_t)(__attribute__((address_space(3))) const int*)p;
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return __builtin_amdgcn_readfirstlane(v);      // every lane read the same word
}
LS_DEV void lds_bump(int* p) {
  const unsigned addr = (unsigned)(size_t)(__attribute__((address_space(3))) int*)p;
  asm volatile("s_waitcnt lgkmcnt(0)\n\tds_add_u32 %0, %1" : : "v"(addr), "v"(1) : "memory");
}

// Barrier among the consumer waves (an LDS counter; the producer waves never take part).  It
// orders LDS accesses only: global stores that other waves must see are drained explicitly.
struct ConsBar {
  int* ctr;
  int gen;
  int* err;
  LS_DEV void sync() {
    gen += NCONS;
    if ((threadIdx.x & 63) == 0) {
      lds_bump(ctr);
      int n = 0;
      while (lds_peek(ctr) < gen) {
        __builtin_amdgcn_s_sleep(0);
        if (++n > SPIN_LIMIT) { ls_flag(err, LS_TIMEOUT); break; }
      }
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("" : : : "memory");
  }
};

// Consumer-side wait until *c >= target (one lane polls), then all consumer waves proceed.
LS_DEV void wait_ge(const int* c, int target, ConsBar& cb) {
  if (threadIdx.x == 0) {
    int n = 0;
    while (ld_acq(c) < target) {
      __builtin_amdgcn_s_sleep(POLL_SLEEP);
      if (++n > SPIN_LIMIT) { ls_flag(cb.err, LS_TIMEOUT); break; }
    }
  }
  cb.sync();
}

// Consumer-side wait until base[i * stride] >= target for all i < n (n <= 64): lanes of the
// first consumer wave poll one counter each, so n counters cost one round trip, not n.
LS_DEV void wait_all_ge(const int* base, int stride, int n, int target, ConsBar& cb) {
  if (threadIdx.x < 64) {
    const int i = threadIdx.x;
    int n_polls = 0;
    bool done = i >= n;
    while (true) {
      if (!done) done = ld_acq(base + (size_t)i * stride) >= target;
      if (__all(done)) break;
      __builtin_amdgcn_s_sleep(POLL_SLEEP);
      if (++n_polls > SPIN_LIMIT) { if (i == 0) ls_flag(cb.err, LS_TIMEOUT); break; }
    }
  }
  cb.sync();
}

// Completion counts of the O, GU and DOWN tiles are spread over NSPREAD counters (tile t bumps
// counter t mod NSPREAD, each on a line of its own): a phase's tiles finish within a few
// microseconds of each other, and atomics on one address would queue behind each other and
// behind the polls of every workgroup.
constexpr int NSPREAD = 64;

// Tiles t in [lo, hi) with t mod NSPREAD == k.
__host__ __device__ inline int spread_count(int lo, int hi, int k) {
  auto fdiv = [](int x) { return x >= 0 ? x / NSPREAD : -((-x + NSPREAD - 1) / NSPREAD); };
  return hi > lo ? fdiv(hi - 1 - k) - fdiv(lo - 1 - k) : 0;
}

// Consumer-side wait until the tiles [lo, hi) have all been counted on the spread counters at
// base (counter k at base + k * PADC): lane k of the first consumer wave polls counter k.
LS_DEV void wait_spread(const int* base, int lo, int hi, ConsBar& cb) {
  if (threadIdx.x < 64) {
    const int k = threadIdx.x;
    const int target = k < NSPREAD ? spread_count(lo, hi, k) : 0;
    int n_polls = 0;
    bool done = k >= NSPREAD || target == 0;
    while (true) {
      if (!done) done = ld_acq(base + (size_t)k * PADC) >= target;
      if (__all(done)) break;
      __builtin_amdgcn_s_sleep(POLL_SLEEP);
      if (++n_polls > SPIN_LIMIT) { if (k == 0) ls_flag(cb.err, LS_TIMEOUT); break; }
    }
  }
  cb.sync();
}

// ---- counter layout -----------------------------------------------------------------------------
struct CntLayout {
  int per_layer, nchF;
  int o_qkvh, o_o, o_gu, o_down, o_fa;
  int o_init, total;
};

// QKV tiles each set a flag of their own (o_qkvh + t * PADC, t head-major), so the attention
// units of a head wait on its 3 * hd / 16 flags, one per lane, without a shared counter.
__host__ __device__ inline CntLayout cnt_layout(int M, int d, int F, int nh, int XC, int n_layers) {
  CntLayout c;
  c.nchF = (F + XC - 1) / XC;
  int o = 0;
  c.o_qkvh = o; o += 3 * (d / 16) * PADC;
  c.o_o = o; o += NSPREAD * PADC;
  c.o_gu = o; o += c.nchF * NSPREAD * PADC;
  c.o_down = o; o += NSPREAD * PADC;
  c.o_fa = o; o += M * nh;
  o = (o + PADC - 1) / PADC * PADC;
  c.per_layer = o;
  c.o_init = n_layers * o;
  c.total = c.o_init + PADC;
  return c;
}

// LDS plan by row count, element size and width d: ring depth, activation columns staged per
// chunk (a multiple of every slab width; the whole row when it fits, so the normalised phases
// need one staging pass) and how many tiles' partials the reduction holds at once.
struct LdsPlan {
  int NS, XC, nred;
};
constexpr int LDS_BUDGET = 160 * 1024 - 512;
#ifndef LS_GU_AVOID
#define LS_GU_AVOID 1
#endif
__host__ __device__ inline size_t x_region_bytes(int M, int esz, int XC) { return (size_t)M * (XC + 16 / esz) * esz; }
// Per-launch row tables in LDS: rows by group [M], depth histogram [64], group offsets and
// count [65], and copies of the rows' slot [M], depth [M] and ancestor offsets [M + 1].
__host__ __device__ inline int row_table_ints(int M) { return M + 64 + 65 + M + M + M + 1; }
__host__ __device__ inline size_t lds_bytes_for(int M, int esz, int NS, int XC, int nred) {
  size_t off = (size_t)NS * SLAB;
  off = (off + x_region_bytes(M, esz, XC) + 15) & ~(size_t)15;
  off = (off + (size_t)row_table_ints(M) * 4 + 15) & ~(size_t)15;
  off = (off + (size_t)nred * NCONS * M * 16 * 4 + 15) & ~(size_t)15;
  off = (off + (size_t)M * 4 + 15) & ~(size_t)15;
  off = (off + (size_t)M * 4 + 15) & ~(size_t)15;
  off += (2 * NS + 8) * 4;
  return off;
}
__host__ __device__ inline LdsPlan lds_plan(int M, int esz, int d) {
  const int sk = 512 / esz;
  const int xfull = (d + sk - 1) / sk * sk;
  const int ns_opts[5] = {16, 14, 12, 10, 8};
  for (int i = 0; i < 5; ++i)
    if (lds_bytes_for(M, esz, ns_opts[i], xfull, 2) <= LDS_BUDGET) return LdsPlan{ns_opts[i], xfull, 2};
  // many rows: narrower activation chunks first, then a shallower ring (down to 4 slabs, one
  // per consumer), so every row count up to the workspace maximum fits
  LdsPlan p{8, xfull, M <= 64 ? 2 : 1};
  while (p.XC > sk && lds_bytes_for(M, esz, p.NS, p.XC, p.nred) > LDS_BUDGET) p.XC = (p.XC / 2 + sk - 1) / sk * sk;
  while (p.NS > NCONS && lds_bytes_for(M, esz, p.NS, p.XC, p.nred) > LDS_BUDGET) p.NS -= 2;
  return p;
}
__host__ __device__ inline int x_chunk_for(int M, int esz, int d) { return lds_plan(M, esz, d).XC; }


size_t mega_counter_ints(int M, int d, int F, int nh, int n_layers) {
  size_t worst = 0;
  for (int m = 1; m <= M; ++m)
    for (int esz = 2; esz <= 4; esz += 2)
      worst = std::max(worst, (size_t)cnt_layout(m, d, F, nh, x_chunk_for(m, esz, d), n_layers).total);
  return worst;
}

// ---- LDS layout -----------------------------------------------------------------------------------
struct Lds {
  char* ring;        // NS slabs
  char* X;           // M x (XC + pad) elements
  float* red;        // nred x NCONS x M x 16: per-tile partials of the consumer waves
  float* rinv;       // M
  int* hx;           // M: hidden-state row of each working row (-1: none)
  int* grow;         // M: rows ordered by KV depth group (attention shares a group's keys)
  int* goff;         // group g's rows: grow[goff[g] .. goff[g+1]); goff[64] = group count
  int *rslot, *rdep, *raoff;   // the rows' validated slot, depth (0 without depths), ancestor offsets
  int* ints;         // [0..NS) full, [NS..2NS) empty, [2NS] consumer barrier, [2NS+1+b] partials
                     // posted to partial buffer b (4 per tile, b < nred <= 2), [2NS+3] tiles whose
                     // partial buffer the epilogue wave has released
  int xstride;       // elements
  int NS, XC, nred;
};

LS_DEV size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

template <typename T>
LS_DEV Lds lds_carve(char* base, int M, int d) {
  Lds s;
  const LdsPlan pl = lds_plan(M, (int)sizeof(T), d);
  s.NS = pl.NS;
  s.XC = pl.XC;
  s.nred = pl.nred;
  s.xstride = s.XC + 16 / (int)sizeof(T);
  size_t off = 0;
  s.ring = base; off += (size_t)s.NS * SLAB;
  s.X = base + off; off = align16(off + x_region_bytes(M, (int)sizeof(T), s.XC));
  s.grow = (int*)(base + off);
  s.goff = s.grow + M + 64;
  s.rslot = s.goff + 65;
  s.rdep = s.rslot + M;
  s.raoff = s.rdep + M;
  off = align16(off + (size_t)row_table_ints(M) * 4);
  s.red = (float*)(base + off); off = align16(off + (size_t)s.nred * NCONS * M * 16 * 4);
  s.rinv = (float*)(base + off); off = align16(off + (size_t)M * 4);
  s.hx = (int*)(base + off); off = align16(off + (size_t)M * 4);
  s.ints = (int*)(base + off);
  return s;
}

size_t mega_smem_bytes(bool bf16, int M, int d) {
  const int esz = bf16 ? 2 : 4;
  const LdsPlan p = lds_plan(M, esz, d);
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

// QKV tiles are numbered head-major: tile t holds 16 output features (8 rotary pairs) of matrix
// mat (0 Q, 1 K, 2 V) of head h, pair block jj.  With round-robin dealing the first round of
// tiles then completes whole heads, whose attention can start while later rounds run.
struct QkvTile {
  int mat, h, jj;
};
LS_DEV QkvTile qkv_tile(const MegaArgs& a, int t) {
  const int tph = a.hd / 16;
  const int h = t / (3 * tph), r = t % (3 * tph);
  return QkvTile{r / tph, h, r % tph};
}

// Weight row r (0..15) of tile t: byte pointer of the row start.
template <typename T>
LS_DEV const char* wrow(const MegaArgs& a, const LayerW& lw, int ph, int t, int r, int K) {
  const size_t rb = (size_t)K * sizeof(T);
  if (ph == PH_QKV) {
    const QkvTile q = qkv_tile(a, t);
    const int mat = q.mat;
    const int n = q.h * a.hd + 8 * q.jj + (r & 7) + (r < 8 ? 0 : a.hd / 2);
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

// A phase's tiles for workgroup b, in order.  Round-robin (tile first + i*G), except that the
// gate/up phase deals its tiles beyond the last full round only to workgroups that will own
// no down-projection tile (the down phase is dealt next, from deal + n): otherwise a quarter of
// the workgroups would stream three gate/up tiles and then a 2.8x larger down tile while
// others sit idle.
struct PhaseShare {
  int first, count;   // round-robin part: tiles first + i*G, i < rounds
  int rounds;
  int rem0, nN, kN;   // extra tiles rem0 + kN + m*nN (m >= 0) of a workgroup outside the down set
  LS_DEV int tile(int i, int G) const { return i < rounds ? first + i * G : rem0 + kN + (i - rounds) * nN; }
};
LS_DEV PhaseShare phase_share(const MegaArgs& a, int ph, int n, int deal, int G, int b) {
  PhaseShare p;
  const Share s = share_of(n, deal, G, b);
  p.first = s.first;
  p.count = s.count;
  p.rounds = s.count;
  p.rem0 = 0; p.nN = 1; p.kN = 0;
  const int nd = a.d / 16;                                  // down-projection tiles
  if (LS_GU_AVOID && ph == PH_GU && nd < G && n % G != 0) {
    const int full = n / G;                                 // complete rounds for everyone
    const int jd = ((s.first - n) % G + G) % G;             // this workgroup's index in the down deal
    p.rounds = full;
    p.rem0 = full * G;
    p.nN = G - nd;
    p.kN = jd - nd;
    const int rem = n - full * G;
    p.count = full + (jd >= nd && p.kN < rem ? (rem - 1 - p.kN) / p.nN + 1 : 0);
  }
  return p;
}

// Wait for this wave's LDS (and scalar memory) operations only.
LS_DEV void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// vmcnt-only wait with a compile-time count (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt[5:4] << 14; expcnt/lgkmcnt at their maxima = no wait).
template <int N>
LS_DEV void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until at most n (a multiple of 8, run time) vector memory operations of this wave are in
// flight.
template <int N>
LS_DEV void wait_vm_le8_impl(int n) {
  if constexpr (N <= 0) {
    wait_vm<0>();
  } else {
    if (n >= N) wait_vm<N>();
    else wait_vm_le8_impl<N - 8>(n);
  }
}
LS_DEV void wait_vm_le8(int n) { wait_vm_le8_impl<56>(__builtin_amdgcn_readfirstlane(n)); }

// =========================================== producer ===========================================
// Every producer wave walks the workgroup's whole slab sequence and issues every NPROD-th slab
// (slab j belongs to wave j mod NPROD) as eight 1 KB direct-to-LDS loads; a wave keeps at most
// PFL of its slabs in flight.  A GCN/CDNA wave issues at most one instruction per four cycles,
// so the per-slab instruction count is what bounds a wave's streaming rate: row addresses are
// computed once per tile, and a slab costs a compare, eight address adds and eight loads.
constexpr int PFL = 2;

template <typename T>
struct Producer {
  const MegaArgs& a;
  const Lds& s;
  int p;              // producer index 0..NPROD-1
  int lane;
  int j = 0;          // position in the workgroup's slab sequence
  int mine = 0;       // slabs issued by this wave (sequence positions p, p + NPROD, ...)
  int pub = 0;        // of which published
  int slot = 0, use = 0;          // ring slot and use count of this wave's next slab
  int pslot = 0;                  // ring slot of this wave's oldest unpublished slab
  const char* rp[8];  // this lane's source in load i of the current tile: row 2i + lane/32, swizzled chunk
  int co[8];          // the swizzled chunk's byte offset within the 512-byte row segment

  LS_DEV Producer(const MegaArgs& a_, const Lds& s_, int p_)
      : a(a_), s(s_), p(p_), lane(threadIdx.x & 63), slot(p_), pslot(p_) {}

  // Callers have waited (vmcnt retires in order) for the slab's loads to land in LDS.  The
  // count is bumped by a non-returning ds_add issued from inline assembly: any compiler-visible
  // LDS access here would get a conservative wait for every direct-to-LDS load still in flight,
  // i.e. drain the prefetch pipeline at each slab.
  LS_DEV void publish_one() {
    if (lane == 0) lds_bump(s.ints + pslot);
    ++pub;
    pslot += NPROD;
    if (pslot >= s.NS) pslot -= s.NS;
  }

  // Row addresses of tile t of phase ph for this lane's eight loads.
  LS_DEV void begin_tile(const LayerW& lw, int ph, int t, const PhaseGeo& g) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rho = 2 * i + (lane >> 5);
      co[i] = ((lane & 31) ^ rho) * 16;
      rp[i] = wrow<T>(a, lw, ph, t, rho, g.K) + co[i];
    }
  }

  // Slab k (512-byte column segment k) of the current tile.
  LS_DEV void issue(int k, const PhaseGeo& g) {
    const int jj = j++;
    if ((jj & (NPROD - 1)) != p) return;
    if (use > 0) {
      // Wait for the consumers to release the slot.  Meanwhile publish, oldest first, every
      // issued slab whose loads have landed, so a full ring never holds back ready slabs.
      int n = 0;
      while (lds_peek(s.ints + s.NS + slot) < use) {
        if (pub < mine) {
          wait_vm_le8(8 * (mine - pub - 1));
          publish_one();
        } else {
          __builtin_amdgcn_s_sleep(0);
          if (++n > SPIN_LIMIT) {
            if (lane == 0) ls_flag(a.err, LS_TIMEOUT);
            break;
          }
        }
      }
    }
    while (mine - pub >= PFL) {
      wait_vm_le8(8 * (mine - pub - 1));
      publish_one();
    }
    char* dst = s.ring + (size_t)slot * SLAB;
    const int kb = k * 512;                           // byte offset of the segment in each row
    const int vb = (g.K - k * g.sk) * (int)sizeof(T); // valid bytes of the segment (< 512: ragged tail)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const char* src = rp[i] + kb;
      if (vb < 512 && co[i] >= vb) src -= co[i];      // chunk past the row end: any valid chunk will do
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(dst + i * 1024), 16, 0, 0);
    }
    ++mine;
    slot += NPROD;
    if (slot >= s.NS) { slot -= s.NS; ++use; }
  }

  LS_DEV void finish() {
    wait_vm<0>();
    while (pub < mine) publish_one();
  }
};

// Debug time stamps (wall clock, 100 MHz) of the first four layers: [grid][4][8 phases][8 events].
LS_DEV void tstamp(const MegaArgs& a, int l, int ph, int e) {
  if (a.trace && l < 4) a.trace[(((size_t)blockIdx.x * 4 + l) * 8 + ph) * 8 + e] = wall_clock64();
}
// Finer stamps of the first layer's QKV phase by thread 0, after the phase stamps: [grid][32].
LS_DEV void dstamp(const MegaArgs& a, bool on, int e) {
  if (on && a.trace && threadIdx.x == 0)
    a.trace[(size_t)gridDim.x * 4 * 8 * 8 + (size_t)blockIdx.x * 32 + e] = wall_clock64();
}

// =========================================== consumer ===========================================
template <typename T, int MT>
struct Consumer {
  const MegaArgs& a;
  const Lds& s;
  ConsBar& cb;
  int c;            // consumer index 0..3
  int lane;
  int cslot = 0, cuse = 0;   // ring slot and use count of the next slab in the sequence
  int seq = 0;               // GEMM tiles of the launch whose partials this consumer has posted
  bool dbg = false; // fine stamps on (first layer's QKV phase)

  LS_DEV Consumer(const MegaArgs& a_, const Lds& s_, ConsBar& cb_, int c_)
      : a(a_), s(s_), cb(cb_), c(c_), lane(threadIdx.x & 63) {}

  // RMSNorm factor of every row from the per-tile sums of squares that the residual epilogues
  // left (row m's d/16 tile sums are contiguous); one wave per row.
  LS_DEV void rinv_from_ssq(const float* ssq) {
    const int nt = a.d / 16;
    for (int m = c; m < a.M; m += NCONS) {
      const __amdgpu_buffer_rsrc_t R = rsrc_of(ssq + (size_t)m * nt, nt * 4);
      float acc = 0.f;
      for (int p0 = 0; p0 < nt; p0 += 256) {
        const u32x4_t v = ld128(R, (p0 + 4 * lane) * 4);
        acc += (__uint_as_float(v.x) + __uint_as_float(v.y)) + (__uint_as_float(v.z) + __uint_as_float(v.w));
      }
      acc = wave_sum(acc);
      if (lane == 0) s.rinv[m] = 1.0f / sqrtf(acc / (float)a.d + a.eps);
    }
    cb.sync();
  }

  // RMSNorm factor of every row straight from the hidden rows (first layer of a call, where no
  // residual epilogue has left tile sums).
  LS_DEV void rinv_from_rows(const float* src) {
    constexpr int NV = 8;
    for (int m = c; m < a.M; m += NCONS) {
      const int hr = __builtin_amdgcn_readfirstlane(s.hx[m]);
      const __amdgpu_buffer_rsrc_t R = rsrc_of(src + (size_t)(hr >= 0 ? hr : 0) * a.d, hr >= 0 ? a.d * 4 : 0);
      float acc = 0.f;
      for (int p0 = 0; p0 < a.d; p0 += 256 * NV) {
        u32x4_t v[NV];
#pragma unroll
        for (int u = 0; u < NV; ++u) v[u] = ld128(R, (p0 + 4 * (lane + 64 * u)) * 4);
#pragma unroll
        for (int u = 0; u < NV; ++u) {
          const float f0 = __uint_as_float(v[u].x), f1 = __uint_as_float(v[u].y);
          const float f2 = __uint_as_float(v[u].z), f3 = __uint_as_float(v[u].w);
          acc += (f0 * f0 + f1 * f1) + (f2 * f2 + f3 * f3);
        }
      }
      acc = wave_sum(acc);
      if (lane == 0) s.rinv[m] = 1.0f / sqrtf(acc / (float)a.d + a.eps);
    }
    cb.sync();
  }

  // Stage columns [x0, x0 + xn) of the normalised rows, T(x * rinv * gain), into LDS; one
  // wave per row, every load of a row pass in flight at once.  With fuse (the chunk is the
  // whole row, d <= 64*4*NVF) the RMSNorm factor comes from the same loads.
  static constexpr int NVF = 8;
  static_assert(64 * 4 * NVF == FUSE_MAX_K, "fused staging covers FUSE_MAX_K columns");
  LS_DEV void stage_norm(const float* src, bool via_hidx, const float* gain, int x0, int xn, bool fuse,
                         bool poll) {
    T* X = (T*)s.X;
    const __amdgpu_buffer_rsrc_t Rg = rsrc_of(gain + x0, xn * 4);
    for (int m = c; m < a.M; m += NCONS) {
      const int hv = __builtin_amdgcn_readfirstlane(s.hx[m]);   // negative: rejected row, stages zeros
      const int hr = via_hidx ? hv : m;
      const float* row = src + (size_t)(hv >= 0 ? hr : 0) * a.d + x0;
      const __amdgpu_buffer_rsrc_t R = rsrc_of(row, hv >= 0 ? xn * 4 : 0);
      T* xr = X + (size_t)m * s.xstride;
      // row values and gains of a pass are all requested before any is used
      if (fuse) {
        u32x4_t v[NVF], gv[NVF];
        dstamp(a, dbg && m == 0, 0);
#pragma unroll
        for (int u = 0; u < NVF; ++u) gv[u] = ld128(Rg, (4 * (lane + 64 * u)) * 4);
        if (poll) {
          // the row is complete once no element holds the fill pattern
          int n = 0;
          while (true) {
#pragma unroll
            for (int u = 0; u < NVF; ++u) v[u] = ldc128(R, (4 * (lane + 64 * u)) * 4);
            bool ok = true;
#pragma unroll
            for (int u = 0; u < NVF; ++u) ok = ok && v[u].x != SENT32 && v[u].y != SENT32 && v[u].z != SENT32 && v[u].w != SENT32;
            if (__all(ok)) break;
            __builtin_amdgcn_s_sleep(POLL_SLEEP);
            if (++n > SPIN_LIMIT) { if (lane == 0) ls_flag(a.err, LS_TIMEOUT); break; }
          }
        } else {
#pragma unroll
          for (int u = 0; u < NVF; ++u) v[u] = ld128(R, (4 * (lane + 64 * u)) * 4);
        }
        dstamp(a, dbg && m == 0, 1);
        float ss = 0.f;
#pragma unroll
        for (int u = 0; u < NVF; ++u) {
          const float f0 = __uint_as_float(v[u].x), f1 = __uint_as_float(v[u].y);
          const float f2 = __uint_as_float(v[u].z), f3 = __uint_as_float(v[u].w);
          ss += (f0 * f0 + f1 * f1) + (f2 * f2 + f3 * f3);
        }
        ss = wave_sum(ss);
        dstamp(a, dbg && m == 0, 2);
        const float ri = 1.0f / sqrtf(ss / (float)a.d + a.eps);
#pragma unroll
        for (int u = 0; u < NVF; ++u) {
          const int k = 4 * (lane + 64 * u);
          if (k < xn) put4(xr + k, v[u], ri, gv[u]);
        }
        dstamp(a, dbg && m == 0, 3);
      } else {
        const float ri = s.rinv[m];
        constexpr int NV = 8;
        for (int p0 = 0; p0 < xn; p0 += 256 * NV) {
          u32x4_t v[NV], gv[NV];
#pragma unroll
          for (int u = 0; u < NV; ++u) v[u] = ld128(R, (p0 + 4 * (lane + 64 * u)) * 4);
#pragma unroll
          for (int u = 0; u < NV; ++u) gv[u] = ld128(Rg, (p0 + 4 * (lane + 64 * u)) * 4);
#pragma unroll
          for (int u = 0; u < NV; ++u) {
            const int k = p0 + 4 * (lane + 64 * u);
            if (k < xn) put4(xr + k, v[u], ri, gv[u]);
          }
        }
      }
    }
    cb.sync();
  }

  LS_DEV static void put4(T* dst, const u32x4_t& v, float ri, const u32x4_t& g) {
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = __uint_as_float(v[e]) * ri * __uint_as_float(g[e]);
    if constexpr (sizeof(T) == 2) {
      const unsigned lo = (unsigned)f2bf(y[0]) | ((unsigned)f2bf(y[1]) << 16);
      const unsigned hi = (unsigned)f2bf(y[2]) | ((unsigned)f2bf(y[3]) << 16);
      *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
    } else {
      *reinterpret_cast<float4*>(dst) = make_float4(y[0], y[1], y[2], y[3]);
    }
  }

  // Stage columns [x0, x0 + xn) of rows already in GEMM-input precision (attention output or
  // SwiGLU activations, row stride K) into LDS, 16 bytes per lane.  The chunk is cut into
  // pieces of 2 x 64 x 16 bytes dealt over the consumer waves; with `poll` (attention output) a
  // piece is re-read until none of its elements holds the fill pattern.
  LS_DEV void stage_raw(const T* src, int K, int x0, int xn, bool poll) {
    constexpr int E = 16 / (int)sizeof(T);
    constexpr int PIECE = 2 * 64 * E;                    // elements per piece
    const int npc = (xn + PIECE - 1) / PIECE;
    for (int it = c; it < a.M * npc; it += NCONS) {
      const int m = it / npc, p0 = (it - m * npc) * PIECE;
      const __amdgpu_buffer_rsrc_t R = rsrc_of(src + (size_t)m * K + x0, xn * (int)sizeof(T));
      char* xr = (char*)((T*)s.X + (size_t)m * s.xstride);
      const int o0 = (p0 + E * lane) * (int)sizeof(T), o1 = (p0 + E * (lane + 64)) * (int)sizeof(T);
      u32x4_t v0, v1;
      if (poll) {
        int n = 0;
        while (true) {
          v0 = ldc128(R, o0);
          v1 = ldc128(R, o1);
          bool ok = true;
#pragma unroll
          for (int j = 0; j < 4; ++j) ok = ok && !holds_fill<T>(v0[j]) && !holds_fill<T>(v1[j]);
          if (__all(ok)) break;
          __builtin_amdgcn_s_sleep(POLL_SLEEP);
          if (++n > SPIN_LIMIT) { if (lane == 0) ls_flag(a.err, LS_TIMEOUT); break; }
        }
      } else {
        v0 = ld128(R, o0);
        v1 = ld128(R, o1);
      }
      if (p0 + E * lane < xn) *reinterpret_cast<u32x4_t*>(xr + o0) = v0;
      if (p0 + E * (lane + 64) < xn) *reinterpret_cast<u32x4_t*>(xr + o1) = v1;
    }
    cb.sync();
  }

  // Pass one slab of the sequence; if it is this consumer's (q mod 4 == c), multiply it.
  LS_DEV void slab(int q, int kn, f32x4_t* acc) {
    const int slot = cslot, use = cuse;
    if (++cslot == s.NS) { cslot = 0; ++cuse; }
    if ((q & (NCONS - 1)) != c) return;
    if (lane == 0) {
      int n = 0;
      while (lds_peek(s.ints + slot) < use + 1) {
        __builtin_amdgcn_s_sleep(0);
        if (++n > SPIN_LIMIT) { ls_flag(a.err, LS_TIMEOUT); break; }
      }
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("" : : : "memory");
    if (dbg && a.trace && threadIdx.x == 0 && a.trace[(size_t)gridDim.x * 256 + (size_t)blockIdx.x * 32 + 6] == 0) dstamp(a, true, 6);
    dstamp(a, dbg, 7);
    constexpr int E = 16 / (int)sizeof(T);
    const int r = lane & 15, g = lane >> 4;
    const char* base = s.ring + (size_t)slot * SLAB + r * 512;
    const int nst = kn / (4 * E);                    // 64-byte steps holding data (8 but for a ragged tail)
    const int xoff = q * (512 / (int)sizeof(T));     // element offset of this slab in the staged chunk
    // Straight-line LDS traffic: every ring and activation read of a group is issued before the
    // first MFMA consumes one, so a slab costs one LDS round trip per group rather than one per
    // step.  Rows m >= M and steps past a ragged tail multiply zeros (their ring bytes are
    // finite weights, their activation reads stay inside the row's staged chunk).
    constexpr int VG = MT == 1 ? 8 : (MT == 2 ? 4 : (MT == 4 ? 2 : 1));
    const T* xrow[MT];
    bool mok[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + r;
      mok[mt] = m < a.M;
      xrow[mt] = (const T*)s.X + (size_t)(mok[mt] ? m : 0) * s.xstride + xoff;
    }
#pragma unroll
    for (int v0 = 0; v0 < 8; v0 += VG) {
      u32x4_t w[VG], x[VG][MT];
#pragma unroll
      for (int u = 0; u < VG; ++u) {
        const int ch = 4 * (v0 + u) + g;
        w[u] = *reinterpret_cast<const u32x4_t*>(base + ((ch ^ r) * 16));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) x[u][mt] = *reinterpret_cast<const u32x4_t*>(xrow[mt] + ch * E);
      }
#pragma unroll
      for (int u = 0; u < VG; ++u) {
        const bool live = v0 + u < nst;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const u32x4_t xv = (live && mok[mt]) ? x[u][mt] : u32x4_t{0u, 0u, 0u, 0u};
          Mma<T>::run(acc[mt], w[u], xv);
        }
      }
    }
    // ring reads are complete (their values fed the MFMAs) before the slot is released
    if (lane == 0) lds_bump(s.ints + s.NS + slot);
    dstamp(a, dbg, 8);
  }
};

// Residual inputs of a tile's epilogue (O: the layer input, DOWN: the post-attention rows):
// res[u] for row m0 + 4u + lane/16, column 16t + lane%16, through one descriptor; absent rows
// read as zero (offset beyond the descriptor's range).  Every load is issued before any is used.
LS_DEV void residual_load(const MegaArgs& a, const Lds& s, int ph, int l, int t, int m0, int lane, float* res) {
  const __amdgpu_buffer_rsrc_t Rr = rsrc_of(ph == PH_O ? layer_in(a, l) : ys_of(a, l), 0x7fffffff);
  const int n = 16 * t + (lane & 15);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int m = m0 + 4 * u + (lane >> 4);
    const int hr = m < a.M ? s.hx[m] : -1;
    const int row = ph == PH_O && l == 0 ? hr : m;
    const int off = hr >= 0 ? (row * a.d + n) * 4 : 0x7fffffff;
    res[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(Rr, off, 0, CPOL_SC1));
  }
}

// Epilogue of one finished tile (its sum over the four consumers is in Ts[m*16 + n]).  With
// have_pre, pre holds the residual inputs of rows 0..15 (O and DOWN), loaded ahead.
template <typename T>
LS_DEV void epilogue(const MegaArgs& a, const CntLayout& cl, const Lds& s, int ph, int l, int t, const float* Ts,
                     int lane, bool have_pre, const float (&pre)[4]) {
  (void)cl;
  if (ph == PH_QKV) {
    const QkvTile qt = qkv_tile(a, t);
    const int mat = qt.mat, h = qt.h, jj = qt.jj;
    for (int idx = lane; idx < a.M * 8; idx += 64) {
      const int m = idx >> 3, p = idx & 7;
      const int i = 8 * jj + p;
      const int e0 = h * a.hd + i, e1 = e0 + a.hd / 2;
      float y0 = Ts[m * 16 + p], y1 = Ts[m * 16 + p + 8];
      if (mat < 2) {
        const float cs = a.rope[((size_t)m * (a.hd / 2) + i) * 2], sn = a.rope[((size_t)m * (a.hd / 2) + i) * 2 + 1];
        const float r0 = y0 * cs - y1 * sn, r1 = y1 * cs + y0 * sn;
        y0 = r0; y1 = r1;
      }
      if (mat == 0) {
        stc(a.q + (size_t)m * a.d + e0, y0);
        stc(a.q + (size_t)m * a.d + e1, y1);
      } else {
        const int sl = s.rslot[m];
        if (sl < 0) continue;
        const int blk = (a.dep ? s.rdep[m] + a.dep_off : 0) * a.blk_mul + a.layer0 + l;
        T* ent = (T*)a.kv + ((size_t)blk * a.S + sl) * 2 * a.d + (mat == 2 ? a.d : 0);
        Coh<T>::store(ent + e0, y0);
        Coh<T>::store(ent + e1, y1);
      }
    }
  } else if (ph == PH_O || ph == PH_DOWN) {
    // residual add: lane = (row group, column); the residual loads of up to 16 rows are in
    // flight together, and the tile's sum of squares per row is reduced over its 16 lanes
    const int nt = a.d / 16;
    float* ssq = a.ssq + ((size_t)l * 2 + (ph == PH_DOWN)) * nt * a.M;
    const int nl = lane & 15, n = 16 * t + nl;
    float* yl = ys_of(a, l);
    const bool last = l == a.n_layers - 1;
    float* xout = (!last || a.do_head) ? a.Xs + (size_t)(l + 1) * a.M * a.d : nullptr;
    for (int m0 = 0; m0 < a.M; m0 += 16) {
      float res[4];
      if (have_pre && m0 == 0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) res[u] = pre[u];
      } else {
        residual_load(a, s, ph, l, t, m0, lane, res);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int m = m0 + 4 * u + (lane >> 4);
        const int hr = m < a.M ? s.hx[m] : -1;
        const float nv = hr >= 0 ? res[u] + Ts[m * 16 + nl] : 0.f;
        if (m < a.M) {
          if (ph == PH_O) {
            stc(yl + (size_t)m * a.d + n, nv);
          } else {
            if (xout) stc(xout + (size_t)m * a.d + n, nv);
            if (last && hr >= 0) stc(a.H + (size_t)hr * a.d + n, nv);
          }
        }
        const float sq = row_sum16(nv * nv);
        if (nl == 0 && m < a.M) stc(ssq + (size_t)m * nt + t, sq);
      }
    }
  } else if (ph == PH_GU) {
    T* act = act_of<T>(a, l);
    for (int idx = lane; idx < a.M * 8; idx += 64) {
      const int m = idx >> 3, p = idx & 7;
      const float gv = Ts[m * 16 + p], uv = Ts[m * 16 + p + 8];
      Coh<T>::store(act + (size_t)m * a.F + 8 * t + p, gv / (1.0f + expf(-gv)) * uv);
    }
  } else {  // PH_HEAD
    for (int idx = lane; idx < a.M * 16; idx += 64) {
      const int m = idx >> 4, nl = idx & 15, n = 16 * t + nl;
      if (n < a.V) a.logits[(size_t)m * a.ldo + n] = Ts[idx];
    }
  }
}

// Counter bump of a finished tile; the caller has drained the tile's stores.
LS_DEV void tile_signal(const MegaArgs& a, const CntLayout& cl, int ph, int l, int t, int XC) {
  int* C = a.cnt + (size_t)l * cl.per_layer;
  if (ph == PH_QKV) {
    atomicAdd(C + cl.o_qkvh + t * PADC, 1);
  } else if (ph == PH_O || ph == PH_DOWN) {
    atomicAdd(C + (ph == PH_O ? cl.o_o : cl.o_down) + (t % NSPREAD) * PADC, 1);
  } else if (ph == PH_GU) {
    atomicAdd(C + cl.o_gu + (((8 * t) / XC) * NSPREAD + t % NSPREAD) * PADC, 1);
  }
}

// ---- attention (consumer waves) -------------------------------------------------------------------
// Causal decode attention of layer l, split over keys and merged with the log-sum-exp rule.
// Rows are grouped by KV depth (a row at loop iteration k reads the depth-k cache, LoopSpec
// section 2.1 and 2.4), and rows of one group share the finished prefix's keys:
//  1. unit (group g, head h, chunk c): the prefix keys [64c, 64c + 64), for every row of the
//     group at once, so those keys are read once per unit.  Wave w takes keys 16w..16w+15;
//     lane = (key kk + 4rr, dims 8e..8e+7).  Partial (max, sum, acc[hd]) per row.
//  2. the workgroup that finishes the group's last unit of head h merges, per row, those
//     partials with the row's own keys (its speculative ancestors and itself, written by this
//     launch) and stores o[l][row][h].

template <typename T>
LS_DEV void load8_plain(const T* p, float* v);
template <>
LS_DEV void load8_plain<uint16_t>(const uint16_t* p, float* v) {
  const uint4 x = *reinterpret_cast<const uint4*>(p);
  const unsigned w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
LS_DEV void load8_plain<float>(const float* p, float* v) {
  const float4 x0 = *reinterpret_cast<const float4*>(p), x1 = *reinterpret_cast<const float4*>(p + 4);
  v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
  v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
}

// Two adjacent elements of a K/V entry written by this launch (agent-coherent load).
template <typename T>
LS_DEV float2 load2_coh(const T* p);
template <>
LS_DEV float2 load2_coh<uint16_t>(const uint16_t* p) {
  const unsigned w = __hip_atomic_load(reinterpret_cast<const unsigned*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}
template <>
LS_DEV float2 load2_coh<float>(const float* p) {
  const unsigned long long w = ldc64(p);
  return make_float2(__uint_as_float((unsigned)w), __uint_as_float((unsigned)(w >> 32)));
}
template <typename T>
LS_DEV void store2_coh(T* p, float x, float y);
template <>
LS_DEV void store2_coh<uint16_t>(uint16_t* p, float x, float y) {
  const unsigned w = (unsigned)f2bf(x) | ((unsigned)f2bf(y) << 16);
  __hip_atomic_store(reinterpret_cast<unsigned*>(p), w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <>
LS_DEV void store2_coh<float>(float* p, float x, float y) {
  const unsigned long long w = (unsigned long long)__float_as_uint(x) | ((unsigned long long)__float_as_uint(y) << 32);
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Group the call's rows by KV depth (at kernel start, all threads).  Depth values index a
// 64-bin histogram; rows with no depth array form one group.
LS_DEV void group_rows(const MegaArgs& a, const Lds& s) {
  int* hist = s.grow + a.M;
  for (int i = threadIdx.x; i < 64; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  for (int m = threadIdx.x; m < a.M; m += blockDim.x) {
    const int dv = min(max(s.rdep[m], 0), 63);
    atomicAdd(hist + dv, 1);
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int cnt = hist[lane];
    // exclusive prefix of the counts and of the non-empty bins, in bin order
    int pre = cnt, ne = cnt > 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int x = __shfl_up(pre, o, 64), y = __shfl_up(ne, o, 64);
      if (lane >= o) { pre += x; ne += y; }
    }
    const int start = pre - cnt, gidx = ne - (cnt > 0);
    if (cnt > 0) s.goff[gidx] = start;
    if (lane == 63) { s.goff[ne] = pre; s.goff[64] = ne; }
    hist[lane] = start;                          // fill cursor of the bin
  }
  __syncthreads();
  for (int m = threadIdx.x; m < a.M; m += blockDim.x) {
    const int dv = min(max(s.rdep[m], 0), 63);
    s.grow[atomicAdd(hist + dv, 1)] = m;         // order inside a group does not affect results
  }
  __syncthreads();
}

// Keys of the finished prefix one attention unit covers: NPASS passes, each giving every lane
// RR keys (for its 8 head dims); lanes hold one pass in registers while the next is in flight.
template <typename T>
struct AttUnit {
  static constexpr int RR = sizeof(T) == 2 ? 2 : 1;     // keys per lane per pass
  static constexpr int NPASS = 8;
  static constexpr int KEYS = 4 * RR * NPASS;             // 64 (bf16) / 32 (fp32)
};
int att_unit_keys(bool bf16) { return bf16 ? AttUnit<uint16_t>::KEYS : AttUnit<float>::KEYS; }

// 8 consecutive elements of a K or V entry as raw storage words.
template <typename T>
struct Raw8 {
  u32x4_t w[sizeof(T) / 2];
  LS_DEV void load(const T* p) {
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 2); ++i) w[i] = *reinterpret_cast<const u32x4_t*>(p + i * (16 / sizeof(T)));
  }
  LS_DEV void zero() {
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 2); ++i) w[i] = u32x4_t{0u, 0u, 0u, 0u};
  }
  LS_DEV void unpack(float* f) const {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[0][i] << 16);
        f[2 * i + 1] = __uint_as_float(w[0][i] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[i] = __uint_as_float(w[0][i]);
        f[4 + i] = __uint_as_float(w[1][i]);
      }
    }
  }
};

template <typename T>
LS_DEV void att_merge(const MegaArgs& a, const Lds& s, const CntLayout& cl, int l, int g, int h, int nu);

// One wave processes unit (g, h, c): prefix keys [KEYS*c, KEYS*c + KEYS) for every row of
// group g, with no workgroup synchronisation.  Lane = (key kk of each group of four, dims
// 8e..8e+7); key j of pass p = 4*RR*p + kk + 4*rr.  Online log-sum-exp over the passes;
// partial (max, sum, acc[hd]) per row to the partial buffer; the wave that completes the last
// unit of (g, h) merges.
template <typename T>
LS_DEV void att_unit_wave(const MegaArgs& a, const Lds& s, const CntLayout& cl, int l, int g, int h, int c, int nu) {
  constexpr int RR = AttUnit<T>::RR, NPASS = AttUnit<T>::NPASS, KEYS = AttUnit<T>::KEYS;
  int* C = a.cnt + (size_t)l * cl.per_layer;
  const int lane = threadIdx.x & 63;
  const int kk = lane >> 4, e = lane & 15;
  const int hd = a.hd;
  const bool dim_ok = 8 * e < hd;
  const int g0 = s.goff[g], ng = s.goff[g + 1] - g0;
  const int rep = s.grow[g0];
  const int blk = (a.dep ? s.rdep[rep] + a.dep_off : 0) * a.blk_mul + a.layer0 + l;
  const T* cache = (const T*)a.kv + (size_t)blk * a.S * 2 * a.d + h * hd + 8 * e;
  const int k0 = c * KEYS;
  const int kn = max(0, min(KEYS, a.n_fin - k0));

  // slots of this lane's keys (prefix keys were written by earlier launches: plain loads)
  int sl[NPASS * RR];
#pragma unroll
  for (int q = 0; q < NPASS * RR; ++q) {
    const int j = (q / RR) * 4 * RR + kk + 4 * (q % RR);
    sl[q] = j < kn ? a.fin[k0 + min(j, kn - 1)] : -1;
  }
  bool bad = false;
#pragma unroll
  for (int q = 0; q < NPASS * RR; ++q) {
    const int j = (q / RR) * 4 * RR + kk + 4 * (q % RR);
    if (j < kn && (sl[q] < 0 || sl[q] >= a.S)) { bad = true; sl[q] = -1; }
  }
  if (bad) ls_flag(a.err, 1);
  auto load_pass = [&](int p, Raw8<T>* kr, Raw8<T>* vr) {
#pragma unroll
    for (int rr = 0; rr < RR; ++rr) {
      const int x = sl[p * RR + rr];
      kr[rr].zero();
      vr[rr].zero();
      if (x >= 0 && dim_ok) {
        kr[rr].load(cache + (size_t)x * 2 * a.d);
        vr[rr].load(cache + (size_t)x * 2 * a.d + a.d);
      }
    }
  };
  // The first NPF passes of prefix keys and values are requested before the wait (they were
  // written by earlier launches, so their latency overlaps the QKV phase); pass p + NPF reuses
  // the registers of pass p, requested as soon as pass p is consumed.
  constexpr int NPF = NPASS / 2;
  Raw8<T> kr[NPF][RR], vr[NPF][RR];
#pragma unroll
  for (int p = 0; p < NPF; ++p) load_pass(p, kr[p], vr[p]);
  // queries of this head are complete once the head's q/k/v tiles have all signalled
  {
    const int nf = 3 * (hd / 16);                         // the head's QKV tiles: flags h * nf .. + nf
    bool done = lane >= nf;
    int n = 0;
    while (true) {
      if (!done) done = ld_acq(C + cl.o_qkvh + (h * nf + lane) * PADC) >= 1;
      if (__all(done)) break;
      __builtin_amdgcn_s_sleep(POLL_SLEEP);
      if (++n > SPIN_LIMIT) { if (lane == 0) ls_flag(a.err, LS_TIMEOUT); break; }
    }
  }
  __builtin_amdgcn_wave_barrier();
  asm volatile("" : : : "memory");

  const float scale = 1.0f / sqrtf((float)hd);
  const __amdgpu_buffer_rsrc_t Rq = rsrc_of(a.q, a.M * a.d * 4);
  for (int r = 0; r < ng; ++r) {
    const int i = s.grow[g0 + r];
    const int qoff = (i * a.d + h * hd + 8 * e) * 4;
    const u32x4_t qa = ldc128(Rq, dim_ok ? qoff : 0x7fffff00), qb = ldc128(Rq, dim_ok ? qoff + 16 : 0x7fffff00);
    if (r > 0) {                                          // a later row re-reads the keys (cached)
#pragma unroll
      for (int p = 0; p < NPF; ++p) load_pass(p, kr[p], vr[p]);
    }
    float q8[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      q8[t] = __uint_as_float(qa[t]) * scale;
      q8[4 + t] = __uint_as_float(qb[t]) * scale;
    }
    float run_m = -INFINITY, lsum = 0.f, acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    auto consume = [&](int p, const Raw8<T>* kp, const Raw8<T>* vp) {
      float sc[RR];
      float pm = -INFINITY;
#pragma unroll
      for (int rr = 0; rr < RR; ++rr) {
        float kf[8];
        kp[rr].unpack(kf);
        float part = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) part += q8[t] * kf[t];
        part = row_sum16(part);             // the key's score in every lane of its row
        sc[rr] = sl[p * RR + rr] >= 0 ? part : -INFINITY;
        pm = fmaxf(pm, sc[rr]);
      }
      pm = rows_max(pm);
      const float nm = fmaxf(run_m, pm);
      if (nm == -INFINITY) return;                        // no key so far
      const float rs = run_m == -INFINITY ? 0.f : __expf(run_m - nm);
      lsum *= rs;
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] *= rs;
      run_m = nm;
#pragma unroll
      for (int rr = 0; rr < RR; ++rr) {
        const float pw = sl[p * RR + rr] >= 0 ? __expf(sc[rr] - nm) : 0.f;
        lsum += pw;
        float vf[8];
        vp[rr].unpack(vf);
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[t] += pw * vf[t];
      }
    };
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      consume(p, kr[p % NPF], vr[p % NPF]);
      __builtin_amdgcn_sched_barrier(0);
      if (p + NPF < NPASS) load_pass(p + NPF, kr[p % NPF], vr[p % NPF]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // per-lane sums cover the lane's keys; combine the four key groups
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      acc[t] += __shfl_xor(acc[t], 16, 64);
      acc[t] += __shfl_xor(acc[t], 32, 64);
    }
    float* out = a.patt + (((size_t)i * a.nh + h) * a.att_chunks + c) * (hd + 2);
    if (lane == 0) { stc(out, run_m); stc(out + 1, lsum); }
    if (kk == 0 && dim_ok) {
#pragma unroll
      for (int t = 0; t < 8; ++t) stc(out + 2 + 8 * e + t, acc[t]);
    }
  }
  drain();
  int arrived = 0;
  if (lane == 0) arrived = atomicAdd(C + cl.o_fa + g * a.nh + h, 1);
  arrived = __shfl(arrived, 0, 64);
  if (arrived == nu - 1) att_merge<T>(a, s, cl, l, g, h, nu);
}

// Long prefixes (att_sub > 1): one wave processes unit (g, h, c): prefix keys [span*c,
// span*c + span), span = KEYS *
// att_sub, for every row of group g, with no workgroup synchronisation.  The unit walks its
// att_sub sub-units of KEYS keys in order; lane = (key kk of each group of four, dims
// 8e..8e+7); key j of a sub-unit's pass p = 4*RR*p + kk + 4*rr.  Online log-sum-exp over all
// passes; partial (max, sum, acc[hd]) per row to the partial buffer; the wave that completes
// the last unit of (g, h) merges.  Long prefixes use several sub-units per unit (fewer
// partials to merge, and the key loads run on from one sub-unit into the next).
template <typename T>
LS_DEV void att_unit_wave_long(const MegaArgs& a, const Lds& s, const CntLayout& cl, int l, int g, int h, int c, int nu) {
  constexpr int RR = AttUnit<T>::RR, NPASS = AttUnit<T>::NPASS, KEYS = AttUnit<T>::KEYS;
  int* C = a.cnt + (size_t)l * cl.per_layer;
  const int lane = threadIdx.x & 63;
  const int kk = lane >> 4, e = lane & 15;
  const int hd = a.hd;
  const bool dim_ok = 8 * e < hd;
  const int g0 = s.goff[g], ng = s.goff[g + 1] - g0;
  const int rep = s.grow[g0];
  const int blk = (a.dep ? s.rdep[rep] + a.dep_off : 0) * a.blk_mul + a.layer0 + l;
  const T* cache = (const T*)a.kv + (size_t)blk * a.S * 2 * a.d + h * hd + 8 * e;
  const int k0 = c * KEYS * a.att_sub;
  const int nsub = max(1, min(a.att_sub, (a.n_fin - k0 + KEYS - 1) / KEYS));   // sub-units holding keys

  // slots of this lane's keys in the sub-unit starting at key kb (prefix keys were written by
  // earlier launches: plain loads); out-of-range slots raise the error word and are skipped
  auto fill_sl = [&](int kb, int* sl) {
    const int kn = max(0, min(KEYS, a.n_fin - kb));
#pragma unroll
    for (int q = 0; q < NPASS * RR; ++q) {
      const int j = (q / RR) * 4 * RR + kk + 4 * (q % RR);
      sl[q] = j < kn ? a.fin[kb + min(j, kn - 1)] : -1;
    }
    bool bad = false;
#pragma unroll
    for (int q = 0; q < NPASS * RR; ++q) {
      const int j = (q / RR) * 4 * RR + kk + 4 * (q % RR);
      if (j < kn && (sl[q] < 0 || sl[q] >= a.S)) { bad = true; sl[q] = -1; }
    }
    if (bad) ls_flag(a.err, 1);
  };
  auto load_pass = [&](const int* sl, int p, Raw8<T>* kr, Raw8<T>* vr) {
#pragma unroll
    for (int rr = 0; rr < RR; ++rr) {
      const int x = sl[p * RR + rr];
      kr[rr].zero();
      vr[rr].zero();
      if (x >= 0 && dim_ok) {
        kr[rr].load(cache + (size_t)x * 2 * a.d);
        vr[rr].load(cache + (size_t)x * 2 * a.d + a.d);
      }
    }
  };
  // The first NPF passes of prefix keys and values are requested before the wait (they were
  // written by earlier launches, so their latency overlaps the QKV phase); pass p + NPF reuses
  // the registers of pass p, requested as soon as pass p is consumed (from the next sub-unit
  // once the current one has no further pass).
  constexpr int NPF = NPASS / 2;
  int sl[NPASS * RR], sn[NPASS * RR];
  fill_sl(k0, sl);
  Raw8<T> kr[NPF][RR], vr[NPF][RR];
#pragma unroll
  for (int p = 0; p < NPF; ++p) load_pass(sl, p, kr[p], vr[p]);
  // queries of this head are complete once the head's q/k/v tiles have all signalled
  {
    const int nf = 3 * (hd / 16);                         // the head's QKV tiles: flags h * nf .. + nf
    bool done = lane >= nf;
    int n = 0;
    while (true) {
      if (!done) done = ld_acq(C + cl.o_qkvh + (h * nf + lane) * PADC) >= 1;
      if (__all(done)) break;
      __builtin_amdgcn_s_sleep(POLL_SLEEP);
      if (++n > SPIN_LIMIT) { if (lane == 0) ls_flag(a.err, LS_TIMEOUT); break; }
    }
  }
  __builtin_amdgcn_wave_barrier();
  asm volatile("" : : : "memory");

  const float scale = 1.0f / sqrtf((float)hd);
  const __amdgpu_buffer_rsrc_t Rq = rsrc_of(a.q, a.M * a.d * 4);
  for (int r = 0; r < ng; ++r) {
    const int i = s.grow[g0 + r];
    const int qoff = (i * a.d + h * hd + 8 * e) * 4;
    const u32x4_t qa = ldc128(Rq, dim_ok ? qoff : 0x7fffff00), qb = ldc128(Rq, dim_ok ? qoff + 16 : 0x7fffff00);
    if (r > 0) {                                          // a later row re-reads the keys (cached)
      if (nsub > 1) fill_sl(k0, sl);
#pragma unroll
      for (int p = 0; p < NPF; ++p) load_pass(sl, p, kr[p], vr[p]);
    }
    float q8[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      q8[t] = __uint_as_float(qa[t]) * scale;
      q8[4 + t] = __uint_as_float(qb[t]) * scale;
    }
    float run_m = -INFINITY, lsum = 0.f, acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    auto consume = [&](int p, const Raw8<T>* kp, const Raw8<T>* vp) {
      float sc[RR];
      float pm = -INFINITY;
#pragma unroll
      for (int rr = 0; rr < RR; ++rr) {
        float kf[8];
        kp[rr].unpack(kf);
        float part = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) part += q8[t] * kf[t];
        part = row_sum16(part);             // the key's score in every lane of its row
        sc[rr] = sl[p * RR + rr] >= 0 ? part : -INFINITY;
        pm = fmaxf(pm, sc[rr]);
      }
      pm = rows_max(pm);
      const float nm = fmaxf(run_m, pm);
      if (nm == -INFINITY) return;                        // no key so far
      const float rs = run_m == -INFINITY ? 0.f : __expf(run_m - nm);
      lsum *= rs;
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] *= rs;
      run_m = nm;
#pragma unroll
      for (int rr = 0; rr < RR; ++rr) {
        const float pw = sl[p * RR + rr] >= 0 ? __expf(sc[rr] - nm) : 0.f;
        lsum += pw;
        float vf[8];
        vp[rr].unpack(vf);
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[t] += pw * vf[t];
      }
    };
    for (int j = 0; j < nsub; ++j) {
      const bool more = j + 1 < nsub;
      if (more) fill_sl(k0 + (j + 1) * KEYS, sn);        // next sub-unit's slots, in flight meanwhile
#pragma unroll
      for (int p = 0; p < NPASS; ++p) {
        consume(p, kr[p % NPF], vr[p % NPF]);
        __builtin_amdgcn_sched_barrier(0);
        if (p + NPF < NPASS) load_pass(sl, p + NPF, kr[p % NPF], vr[p % NPF]);
        else if (more) load_pass(sn, p + NPF - NPASS, kr[p % NPF], vr[p % NPF]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (more) {
#pragma unroll
        for (int q = 0; q < NPASS * RR; ++q) sl[q] = sn[q];
      }
    }
    // per-lane sums cover the lane's keys; combine the four key groups
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      acc[t] += __shfl_xor(acc[t], 16, 64);
      acc[t] += __shfl_xor(acc[t], 32, 64);
    }
    float* out = a.patt + (((size_t)i * a.nh + h) * a.att_chunks + c) * (hd + 2);
    if (lane == 0) { stc(out, run_m); stc(out + 1, lsum); }
    if (kk == 0 && dim_ok) {
#pragma unroll
      for (int t = 0; t < 8; ++t) stc(out + 2 + 8 * e + t, acc[t]);
    }
  }
  drain();
  int arrived = 0;
  if (lane == 0) arrived = atomicAdd(C + cl.o_fa + g * a.nh + h, 1);
  arrived = __shfl(arrived, 0, 64);
  if (arrived == nu - 1) att_merge<T>(a, s, cl, l, g, h, nu);
}

// Merge of head h for the rows of group g, by one wave, row by row; lane = dims 2*lane, 2*lane + 1.
// Online log-sum-exp over batches of (16 prefix-chunk partials, 8 own keys); every load of a
// batch is issued before any is used, so a batch costs one memory round trip.
template <typename T>
LS_DEV void att_merge(const MegaArgs& a, const Lds& s, const CntLayout& cl, int l, int g, int h, int nu) {
  const int lane = threadIdx.x & 63;
  const int hd = a.hd;
  const bool dok = 2 * lane < hd;
  const int g0 = s.goff[g], ng = s.goff[g + 1] - g0;
  const int rep = s.grow[g0];
  const int blk = (a.dep ? s.rdep[rep] + a.dep_off : 0) * a.blk_mul + a.layer0 + l;
  const T* cache = (const T*)a.kv + (size_t)blk * a.S * 2 * a.d;
  const float scale = 1.0f / sqrtf((float)hd);
  for (int r = 0; r < ng; ++r) {
    const int i = s.grow[g0 + r];
    T* orow = o_of<T>(a, l) + (size_t)i * a.d + h * hd;
    const int self = s.rslot[i];
    if (self < 0) {                                  // rejected row: zero output
      if (dok) store2_coh<T>(orow + 2 * lane, 0.f, 0.f);
      continue;
    }
    const int a0 = s.raoff[i], na = s.raoff[i + 1] - a0;
    const int nt = na + 1;                           // the row's own keys: ancestors, then itself
    const float* base = a.patt + ((size_t)i * a.nh + h) * a.att_chunks * (hd + 2);
    // the query joins the first batch's loads (it is converted where the scores are formed)
    const unsigned long long qw = dok ? ldc64(a.q + (size_t)i * a.d + h * hd + 2 * lane) : 0ull;
    float run_m = -INFINITY, den = 0.f, num0 = 0.f, num1 = 0.f;
    const int nbat = max((nu + 15) / 16, (nt + 7) / 8);
    for (int bt = 0; bt < nbat; ++bt) {
      const int c0 = bt * 16, j0 = bt * 8;
      // ---- issue the batch's loads
      const int cl_ = c0 + lane;                     // chunk whose statistics this lane holds
      float mxc = -INFINITY, smc = 0.f;
      if (lane < 16 && cl_ < nu) {
        mxc = ldc(base + (size_t)cl_ * (hd + 2));
        smc = ldc(base + (size_t)cl_ * (hd + 2) + 1);
      }
      float2 ac[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int cc = min(c0 + u, nu - 1);
        ac[u] = make_float2(0.f, 0.f);
        if (dok && c0 + u < nu) {
          const unsigned long long w = ldc64(base + (size_t)cc * (hd + 2) + 2 + 2 * lane);
          ac[u] = make_float2(__uint_as_float((unsigned)w), __uint_as_float((unsigned)(w >> 32)));
        }
      }
      float2 k2[8], v2[8];
      int xs[8];
      bool bad = false;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = min(j0 + u, nt - 1);
        xs[u] = j < na ? a.anc[a0 + j] : self;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (xs[u] < 0 || xs[u] >= a.S) { bad = bad || j0 + u < nt; xs[u] = self; }
        const T* ent = cache + (size_t)xs[u] * 2 * a.d + h * hd + 2 * lane;
        k2[u] = v2[u] = make_float2(0.f, 0.f);
        if (dok && j0 + u < nt) {
          k2[u] = load2_coh<T>(ent);
          v2[u] = load2_coh<T>(ent + a.d);
        }
      }
      if (bad) ls_flag(a.err, 1);
      // ---- the batch's scores and its maximum
      const float q0 = __uint_as_float((unsigned)qw) * scale, q1 = __uint_as_float((unsigned)(qw >> 32)) * scale;
      float sc[8];
      float bm = wave_max(mxc);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        sc[u] = wave_sum(q0 * k2[u].x + q1 * k2[u].y);
        if (j0 + u < nt) bm = fmaxf(bm, sc[u]);
      }
      const float nm = fmaxf(run_m, bm);
      if (nm == -INFINITY) continue;                 // nothing in this batch or before
      const float rs = run_m == -INFINITY ? 0.f : __expf(run_m - nm);
      den *= rs; num0 *= rs; num1 *= rs;
      run_m = nm;
      // prefix chunks: weight w_c = exp(mx_c - m) held by lane c - c0
      const float wl = mxc == -INFINITY ? 0.f : __expf(mxc - nm);
      den += wave_sum(wl * smc);
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const float w = lane_f(wl, u);
        num0 += w * ac[u].x;
        num1 += w * ac[u].y;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float w = j0 + u < nt ? __expf(sc[u] - nm) : 0.f;
        den += w;
        num0 += w * v2[u].x;
        num1 += w * v2[u].y;
      }
    }
    if (dok) store2_coh<T>(orow + 2 * lane, den > 0.f ? num0 / den : 0.f, den > 0.f ? num1 / den : 0.f);
  }
}

// ---- init unit: embedding row or gathered hidden row into the working rows ---------------------------
template <typename T>
LS_DEV void init_unit(const MegaArgs& a, const CntLayout& cl, ConsBar& cb, int m) {
  const int hr = a.hidx ? a.hidx[m] : m;
  if (hr >= 0) {
    if (a.init_mode == 1) {
      const int tok = a.tokens[m];
      if (tok >= 0 && tok < a.V) {
#pragma unroll 8
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

// Phase stamps: consumer wave 0: 0 phase begin, 1 phase end, 2 dependencies met, 3 first chunk
// staged, 4 first tile batch multiplied.  Producer wave 0: 5 first slab issued, 6 last issued.

// ---- the walk: the same slab sequence for producers and consumers ----------------------------------
// Phase ph of layer l: the workgroup's tiles one by one; within a tile, activation chunk by
// chunk (XC columns), slab by slab.
template <typename T, int MT, bool PROD>
LS_DEV void walk_gemm(const MegaArgs& a, const Lds& s, const CntLayout& cl, int ph, int l, int& deal,
                      Producer<T>* pr, Consumer<T, MT>* co, ConsBar* cb) {
  const int G = gridDim.x, b = blockIdx.x;
  const PhaseGeo g = phase_geo<T>(a, ph);
  const PhaseShare sh = phase_share(a, ph, g.n_tiles, deal, G, b);
  deal = (deal + g.n_tiles) % G;
  if (sh.count == 0) return;
  const LayerW lw = ph == PH_HEAD ? LayerW{} : a.layers[l];
  const int nchunk = (g.K + s.XC - 1) / s.XC;

  // normalised phases (QKV, GU, HEAD) read a whole row when one activation chunk covers it and
  // then take the RMSNorm factor from the same loads; otherwise from the per-tile sums of squares
  const bool fuse = nchunk == 1 && g.K <= FUSE_MAX_K;
  const int lin = ph == PH_HEAD ? a.n_layers : l;              // layer whose input a normalised phase reads
  const float* nsrc = ph == PH_GU ? ys_of(a, l) : layer_in(a, lin);
  const bool nvia = ph != PH_GU && lin == 0;                   // rows addressed through hidx
  const float* gain = ph == PH_QKV ? lw.g1 : (ph == PH_GU ? lw.g2 : a.g_final);
  // fused normalised phases whose input was written in this launch read it by polling
  const bool poll = fuse && (ph == PH_GU || lin > 0);
  if (!PROD) {
    co->dbg = l == 0 && ph == PH_QKV;
    dstamp(a, co->dbg, 4);
    const int* C = a.cnt + (size_t)l * cl.per_layer;
    const int nt = a.d / 16;
    const float* ssq = nullptr;
    if (ph == PH_QKV || ph == PH_HEAD) {
      const int lp = ph == PH_QKV ? l - 1 : a.n_layers - 1;    // layer whose output feeds this phase
      if (lp >= 0) {
        if (!poll) wait_spread(a.cnt + (size_t)lp * cl.per_layer + cl.o_down, 0, nt, *cb);
        ssq = a.ssq + ((size_t)lp * 2 + 1) * nt * a.M;
      } else if (a.init_mode) {
        wait_ge(a.cnt + cl.o_init, a.M, *cb);
      }
      if (!fuse) {
        if (ssq) co->rinv_from_ssq(ssq);
        else co->rinv_from_rows(a.H);            // first layer of the call: the caller's rows
      }
    } else if (ph == PH_GU) {
      if (!poll) wait_spread(C + cl.o_o, 0, nt, *cb);
      if (!fuse) co->rinv_from_ssq(a.ssq + ((size_t)l * 2) * nt * a.M);
    }
    if (threadIdx.x == 0) tstamp(a, l, ph, 2);
  }

  // One tile at a time.  With one activation chunk (the usual case) the chunk is staged once
  // for all of the workgroup's tiles; with several, every tile re-stages its chunks.
  const bool restage = nchunk > 1;
  for (int i = 0; i < sh.count; ++i) {
    const int t = sh.tile(i, G);
    f32x4_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int ch = 0; ch < nchunk; ++ch) {
      const int x0 = ch * s.XC;
      const int xn = min(s.XC, g.K - x0);
      if (!PROD && (restage || i == 0)) {
        const int* C = a.cnt + (size_t)l * cl.per_layer;
        if (ph == PH_DOWN) {
          wait_spread(C + cl.o_gu + ch * NSPREAD * PADC, x0 / 8, (x0 + xn) / 8, *cb);
        } else {
          cb->sync();                     // earlier readers of the stage are done
        }
        dstamp(a, co->dbg, 5);
        if (ph == PH_O || ph == PH_DOWN) co->stage_raw(ph == PH_O ? o_of<T>(a, l) : act_of<T>(a, l), g.K, x0, xn, ph == PH_O);
        else co->stage_norm(nsrc, nvia, gain, x0, xn, fuse, poll);
        if (threadIdx.x == 0 && i == 0 && ch == 0) tstamp(a, l, ph, 3);
      }
      const int k_first = x0 / g.sk;
      const int k_last = (x0 + xn + g.sk - 1) / g.sk;
      if (PROD && ch == 0) pr->begin_tile(lw, ph, t, g);
      for (int k = k_first; k < k_last; ++k) {
        if (PROD) {
          if (threadIdx.x == 64 * NCONS && i == 0 && ch == 0 && k == k_first) tstamp(a, l, ph, 5);
          pr->issue(k, g);
        } else {
          co->slab(k - k_first, min(g.sk, g.K - k * g.sk), acc);
        }
      }
    }
    if (!PROD) {
      if (threadIdx.x == 0 && i == 0) tstamp(a, l, ph, 4);
      // The four consumer partials meet in LDS (s.nred rotating buffers) and the epilogue wave
      // takes the tile from there: consumers never wait for the epilogue's stores to drain.
      const int lane = threadIdx.x & 63, r = lane & 15, gq = lane >> 4;
      const int q = co->seq++;
      float* buf = s.red + (size_t)(q % s.nred) * NCONS * a.M * 16;
      if (q >= s.nred && lane == 0) {      // the epilogue wave is done with this buffer's last tile
        int n = 0;
        while (lds_peek(s.ints + 2 * s.NS + 3) < q - s.nred + 1) {
          __builtin_amdgcn_s_sleep(0);
          if (++n > SPIN_LIMIT) { ls_flag(a.err, LS_TIMEOUT); break; }
        }
      }
      __builtin_amdgcn_wave_barrier();
      asm volatile("" : : : "memory");
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + r;
        if (m < a.M) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) buf[((size_t)co->c * a.M + m) * 16 + 4 * gq + jj] = acc[mt][jj];
        }
      }
      // Counted per buffer: a consumer may run a tile ahead of the others, but never onto a
      // buffer the epilogue wave has not released, so buffer b's count covers one tile at a time.
      if (lane == 0) lds_bump(s.ints + 2 * s.NS + 1 + q % s.nred);   // after this wave's partial writes complete
    }
    if (PROD && threadIdx.x == 64 * NCONS && i == sh.count - 1) tstamp(a, l, ph, 6);
  }
}

// The epilogue wave's part of a GEMM phase: for each of the workgroup's tiles (in the
// consumers' order) wait for the four consumer partials, sum them in consumer order, run the
// epilogue and release the partial buffer.  Stores are drained, and the tiles' counters
// bumped, once no further tile of the phase is ready, so a burst of tiles costs one drain.
//
// Residual inputs of the first O / DOWN tile are loaded when the walk starts if the workgroup
// had tiles in the phase before (QKV / GU): their partials having arrived means the consumers
// passed that phase's dependency wait, which implies the residual rows are complete (the
// previous layer for O, the O phase for DOWN).  The loads then overlap the consumers' work.
template <typename T>
LS_DEV void epi_walk(const MegaArgs& a, const Lds& s, const CntLayout& cl, int ph, int l, int& deal, int& seq,
                     bool& had_tiles) {
  const int G = gridDim.x, b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const PhaseGeo g = phase_geo<T>(a, ph);
  const PhaseShare sh = phase_share(a, ph, g.n_tiles, deal, G, b);
  deal = (deal + g.n_tiles) % G;
  const bool pref = (ph == PH_O || ph == PH_DOWN) && had_tiles && sh.count > 0 && a.M <= 16;
  // O / DOWN counts are waited for only when the next normalised phase cannot poll its input
  // (its row does not fit one fused staging pass); otherwise their drain and bump are skipped.
  const bool next_polls = a.d <= s.XC && a.d <= FUSE_MAX_K;
  const bool signals = ph != PH_HEAD && !((ph == PH_O || ph == PH_DOWN) && next_polls);
  float pre[4] = {0.f, 0.f, 0.f, 0.f};
  if (pref) residual_load(a, s, ph, l, sh.tile(0, G), 0, lane, pre);
  had_tiles = sh.count > 0;
  int pend = 0;                            // first of this phase's tiles not yet signalled
  for (int i = 0; i < sh.count; ++i) {
    const int t = sh.tile(i, G);
    const int q = seq++;
    float* buf = s.red + (size_t)(q % s.nred) * NCONS * a.M * 16;
    if (lane == 0) {
      int n = 0;
      while (lds_peek(s.ints + 2 * s.NS + 1 + q % s.nred) < NCONS * (q / s.nred + 1)) {
        __builtin_amdgcn_s_sleep(0);
        if (++n > SPIN_LIMIT) { ls_flag(a.err, LS_TIMEOUT); break; }
      }
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("" : : : "memory");
    for (int idx = lane; idx < a.M * 16; idx += 64) {
      float y = 0.f;
#pragma unroll
      for (int cc = 0; cc < NCONS; ++cc) y += buf[(size_t)cc * a.M * 16 + idx];
      buf[idx] = y;                        // consumer 0's slot now holds the tile sum
    }
    __builtin_amdgcn_wave_barrier();
    wait_lgkm0();                          // the sums are visible to every lane
    epilogue<T>(a, cl, s, ph, l, t, buf, lane, pref && i == 0, pre);
    wait_lgkm0();                          // the epilogue's reads of the buffer are complete
    if (lane == 0) lds_bump(s.ints + 2 * s.NS + 3);
    if (!signals) continue;
    const bool next_ready =
        i + 1 < sh.count && lds_peek(s.ints + 2 * s.NS + 1 + (q + 1) % s.nred) >= NCONS * ((q + 1) / s.nred + 1);
    if (!next_ready) {
      drain();
      if (lane == 0)
        for (int k = pend; k <= i; ++k) tile_signal(a, cl, ph, l, sh.tile(k, G), s.XC);
      pend = i + 1;
    }
  }
}

// Step st of a call's phase sequence: per layer QKV, attention, O, GU, DOWN; then the LM head.
struct Step {
  int ph, l;
};
LS_DEV Step step_of(const MegaArgs& a, int st) {
  if (st >= 5 * a.n_layers) return Step{PH_HEAD, a.n_layers};
  const int k = st % 5;
  return Step{k == 0 ? PH_QKV : (k == 1 ? PH_ATT : (k == 2 ? PH_O : (k == 3 ? PH_GU : PH_DOWN))), st / 5};
}

template <typename T, int MT, bool LONG>
LS_DEV void mega_body(const MegaArgs& a) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  const Lds s = lds_carve<T>(smem_raw, a.M, a.d);
  const CntLayout cl = cnt_layout(a.M, a.d, a.F, a.nh, x_chunk_for(a.M, (int)sizeof(T), a.d), a.n_layers);
  const int G = gridDim.x, b = blockIdx.x;
  const int wv = wave_id();
  // ring counters and the consumer barrier start at zero
  for (int i = threadIdx.x; i < 2 * s.NS + 8; i += MEGA_THREADS) s.ints[i] = 0;
  for (int i = threadIdx.x; i < a.M; i += MEGA_THREADS) {
    s.hx[i] = a.hidx ? a.hidx[i] : i;
    s.rslot[i] = a.slot[i];
    s.rdep[i] = a.dep ? a.dep[i] : 0;
  }
  for (int i = threadIdx.x; i <= a.M; i += MEGA_THREADS) s.raoff[i] = a.anc_off ? a.anc_off[i] : 0;
  __syncthreads();
  group_rows(a, s);
  __syncthreads();
  int deal = 0;
  const int n_steps = 5 * a.n_layers + (a.do_head ? 1 : 0);
  if (wv == EPI_WAVE) {
    // ------------------------------ epilogue wave ------------------------------
    int seq = 0;
    bool had_tiles = false;
#pragma unroll 1
    for (int st = 0; st < n_steps; ++st) {
      const Step sp = step_of(a, st);
      if (sp.ph != PH_ATT) epi_walk<T>(a, s, cl, sp.ph, sp.l, deal, seq, had_tiles);
    }
    return;
  }
  if (wv >= NCONS) {
    // ------------------------------ producer waves ------------------------------
    Producer<T> pr(a, s, wv - NCONS);
#pragma unroll 1
    for (int st = 0; st < n_steps; ++st) {
      const Step sp = step_of(a, st);
      if (sp.ph != PH_ATT) walk_gemm<T, MT, true>(a, s, cl, sp.ph, sp.l, deal, &pr, nullptr, nullptr);
    }
    pr.finish();
    return;
  }
  // ------------------------------ consumer waves ------------------------------
  ConsBar cb{s.ints + 2 * s.NS, 0, a.err};
  Consumer<T, MT> co(a, s, cb, wv);
  if (a.init_mode)
    for (int u = b; u < a.M; u += G) init_unit<T>(a, cl, cb, u);
  int att_deal = 0;
#pragma unroll 1
  for (int st = 0; st < n_steps; ++st) {
    const Step sp = step_of(a, st);
    if (threadIdx.x == 0) tstamp(a, sp.l, sp.ph, 0);
    if (sp.ph == PH_ATT) {
      const int nu = a.att_chunks;                 // prefix chunks per (group, head), >= 1
      const int natt = s.goff[64] * a.nh * nu;
      const Share sa = share_of(natt, att_deal, G, b);
      att_deal = (att_deal + natt) % G;
      // unit u runs on workgroup (u + att_deal) mod G, wave (u / G) mod 4: every unit gets a
      // wave of its own before any wave takes a second one
      for (int k = co.c; k < sa.count; k += NCONS) {
        const int u = sa.first + k * G;
        const int cch = u % nu, gh = u / nu;
        if constexpr (LONG) att_unit_wave_long<T>(a, s, cl, sp.l, gh / a.nh, gh % a.nh, cch, nu);
        else att_unit_wave<T>(a, s, cl, sp.l, gh / a.nh, gh % a.nh, cch, nu);
      }
    } else {
      walk_gemm<T, MT, false>(a, s, cl, sp.ph, sp.l, deal, nullptr, &co, &cb);
    }
    if (threadIdx.x == 0) tstamp(a, sp.l, sp.ph, 1);
  }
}

// Two entry symbols over the same body, so that profiles tell the loop block's launches
// (ls_loop_step) apart from the prelude, coda and LM-head launches.
// LONG: attention units of several sub-units (long prefixes), compiled separately so that the
// short-prefix kernels keep their code size.
template <typename T, int MT, bool LONG>
__global__ __launch_bounds__(MEGA_THREADS) void k_mega(MegaArgs a) { mega_body<T, MT, LONG>(a); }
template <typename T, int MT, bool LONG>
__global__ __launch_bounds__(MEGA_THREADS) void k_mega_aux(MegaArgs a) { mega_body<T, MT, LONG>(a); }

// P of a model without prelude layers (LoopSpec page, section 2.1, eq. 1; here P is the
// embedding row alone): one workgroup per row checks the row and copies its token's embedding
// into H[slot] in fp32.
template <typename T>
__global__ __launch_bounds__(256) void k_embed(ValidateArgs v, const int32_t* tokens, const T* emb, int V, int d,
                                               float* H) {
  __shared__ int s_slot;
  const int i = blockIdx.x;
  if (threadIdx.x == 0) s_slot = check_row(v, i);
  __syncthreads();
  const int hr = s_slot;
  if (hr < 0) return;
  const int tok = tokens[i];
  if (tok < 0 || tok >= V) {
    if (threadIdx.x == 0) ls_flag(v.err, 1);
    return;
  }
  for (int k = threadIdx.x; k < d; k += blockDim.x) H[(size_t)hr * d + k] = Elem<T>::load(emb + (size_t)tok * d + k);
}

hipError_t launch_embed(bool bf16, const ValidateArgs& v, const int32_t* tokens, const void* emb, int V, int d, float* H,
                        hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(k_embed<uint16_t>, dim3(v.n), dim3(256), 0, s, v, tokens, (const uint16_t*)emb, V, d, H);
  else
    hipLaunchKernelGGL(k_embed<float>, dim3(v.n), dim3(256), 0, s, v, tokens, (const float*)emb, V, d, H);
  return hipGetLastError();
}

// Set-up of one launch: counters to zero, this launch's polled buffers to SENT32, rotary
// cos/sin of the rows' positions, and (first launch of a call) the row-descriptor check.
__global__ void k_prep(int* cnt, long long n, float* rope, const int32_t* pos, const double* inv_freq, int M, int half,
                       unsigned* xs_fill, long long n_xs, unsigned* ys_fill, long long n_ys, unsigned* o_fill,
                       long long n_o, ValidateArgs v) {
  const long long tid = (long long)blockIdx.x * blockDim.x + threadIdx.x, str = (long long)gridDim.x * blockDim.x;
  for (long long i = tid; i < v.n; i += str) check_row(v, (int)i);
  for (long long i = tid; i < n; i += str) cnt[i] = 0;
  for (long long i = tid; i < n_xs; i += str) xs_fill[i] = SENT32;
  for (long long i = tid; i < n_ys; i += str) ys_fill[i] = SENT32;
  for (long long i = tid; i < n_o; i += str) o_fill[i] = 0xffffffffu;
  for (long long i = tid; i < (long long)M * half; i += str) {
    const int m = (int)(i / half), f = (int)(i % half);
    double sn, cs;
    sincos((double)pos[m] * inv_freq[f], &sn, &cs);
    rope[2 * i] = (float)cs;
    rope[2 * i + 1] = (float)sn;
  }
}

template <typename T, bool LONG>
static const void* pick_tl(int mt, bool loop) {
  if (loop) {
    if (mt <= 1) return reinterpret_cast<const void*>(&k_mega<T, 1, LONG>);
    if (mt <= 2) return reinterpret_cast<const void*>(&k_mega<T, 2, LONG>);
    if (mt <= 4) return reinterpret_cast<const void*>(&k_mega<T, 4, LONG>);
    return reinterpret_cast<const void*>(&k_mega<T, 8, LONG>);
  }
  if (mt <= 1) return reinterpret_cast<const void*>(&k_mega_aux<T, 1, LONG>);
  if (mt <= 2) return reinterpret_cast<const void*>(&k_mega_aux<T, 2, LONG>);
  if (mt <= 4) return reinterpret_cast<const void*>(&k_mega_aux<T, 4, LONG>);
  return reinterpret_cast<const void*>(&k_mega_aux<T, 8, LONG>);
}

static const void* pick(bool bf16, int M, bool loop = true, bool lng = false) {
  const int mt = (M + 15) / 16;
  if (lng) return bf16 ? pick_tl<uint16_t, true>(mt, loop) : pick_tl<float, true>(mt, loop);
  return bf16 ? pick_tl<uint16_t, false>(mt, loop) : pick_tl<float, false>(mt, loop);
}

int mega_occupancy(bool bf16, int M, int d) {
  const size_t smem = mega_smem_bytes(bf16, M, d);
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, pick(bf16, M), MEGA_THREADS, smem) != hipSuccess) return 0;
  return n;
}

hipError_t launch_mega(bool bf16, const MegaArgs& a, int G, hipStream_t s, bool loop_block, const ValidateArgs& v) {
  const CntLayout cl = cnt_layout(a.M, a.d, a.F, a.nh, x_chunk_for(a.M, bf16 ? 2 : 4, a.d), a.n_layers);
  const long long n_prep = std::max<long long>(std::max<long long>(cl.total, (long long)a.M * (a.hd / 2)), v.n);
  const long long rows = (long long)a.M * a.d;   // one layer slice of Xs / Ys
  hipLaunchKernelGGL(k_prep, dim3((unsigned)std::min<long long>(1024, (n_prep + 255) / 256)), dim3(256), 0, s, a.cnt,
                     (long long)cl.total, a.rope, a.pos, a.inv_freq, a.M, a.hd / 2,
                     reinterpret_cast<unsigned*>(a.Xs + rows), (long long)a.n_layers * rows,
                     reinterpret_cast<unsigned*>(a.Ys), (long long)a.n_layers * rows,
                     reinterpret_cast<unsigned*>(a.o), (long long)a.n_layers * rows * (bf16 ? 2 : 4) / 4, v);
  const size_t smem = mega_smem_bytes(bf16, a.M, a.d);
  void* args[] = {(void*)&a};
  return hipLaunchCooperativeKernel(pick(bf16, a.M, loop_block, a.att_sub > 1), dim3(G), dim3(MEGA_THREADS), args,
                                    (unsigned)smem, s);
}

}  // namespace ls
