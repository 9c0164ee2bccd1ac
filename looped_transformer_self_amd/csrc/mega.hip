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
// Rows up to this many columns are staged, normalised and (for Xs / Ys) polled in one pass of
// one wave; rows up to NCONS times as wide in one pass of the consumer waves together.
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

// Every wait below is bounded by one deadline per launch on the constant-rate wall clock: each
// workgroup sets it when it starts (MegaArgs::wait_ticks later; every workgroup of a cooperative
// launch starts together), and a wait checks it on its first poll and every WAIT_CHECK polls
// after that.  A wait still unmet at the deadline records LS_TIMEOUT in the error word and gives
// up; since the deadline is shared, every later wait of the launch gives up after one poll too,
// so a broken dependency ends the whole launch shortly after the deadline (the remaining work
// runs on unchecked data) instead of each wait spending a budget of its own.  Only the clock is
// read in the loops: an error-word load there would delay the wake-up of waits in tight LDS
// spin loops.
__shared__ long long ls_wait_deadline;
constexpr int WAIT_CHECK = 256;
LS_DEV void set_deadline(long long ticks) {
  if (threadIdx.x == 0) ls_wait_deadline = (long long)wall_clock64() + ticks;
}
// Global counters are polled by up to every workgroup at once; each poll is a memory access
// to the same line, so polls are spaced (s_sleep units of 64 cycles) to leave that line's
// bandwidth to the atomics that move the counter.
#ifndef LS_POLL_SLEEP
#define LS_POLL_SLEEP 8
#endif
constexpr int POLL_SLEEP = LS_POLL_SLEEP;
constexpr int LS_TIMEOUT = 5;

// Poll count n of a wait: true (after recording LS_TIMEOUT) once the launch's deadline passed.
LS_DEV bool give_up(int& n, int* err) {
  if ((++n & (WAIT_CHECK - 1)) != 1) return false;
  if ((long long)wall_clock64() < ls_wait_deadline) return false;
  ls_flag(err, LS_TIMEOUT);
  return true;
}

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
LS_DEV void lds_add(int* p, int v) {
  const unsigned addr = (unsigned)(size_t)(__attribute__((address_space(3))) int*)p;
  asm volatile("s_waitcnt lgkmcnt(0)\n\tds_add_u32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}
LS_DEV void lds_bump(int* p) { lds_add(p, 1); }
// Per-lane read of an LDS word (every lane its own address).
LS_DEV int lds_read_lane(const int* p) {
  const unsigned addr = (unsigned)(size_t)(__attribute__((address_space(3))) const int*)p;
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
// The producers' bump: their LDS operations complete in order and nothing they read from LDS
// is pending, so no wait is needed (which leaves scalar loads of key slots in flight).
LS_DEV void lds_bump_nw(int* p) {
  const unsigned addr = (unsigned)(size_t)(__attribute__((address_space(3))) int*)p;
  asm volatile("ds_add_u32 %0, %1" : : "v"(addr), "v"(1) : "memory");
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
        if (give_up(n, err)) break;
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
      if (give_up(n, cb.err)) break;
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
      if (give_up(n_polls, cb.err)) break;
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
      if (give_up(n_polls, cb.err)) break;
    }
  }
  cb.sync();
}

// ---- counter layout -----------------------------------------------------------------------------
struct CntLayout {
  int per_layer, nchF;
  int o_qkvh, o_o, o_gu, o_down, o_split;
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
  c.o_split = o; o += 2 * (d / 16);        // arrivals at the split O and DOWN tiles
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
// Rows of the attention phase's virtual groups (see the attention section).
constexpr int NRA = 1;
// The attention phase reuses the activation region for the consumer waves' softmax states:
// consumers 1..3 x NRA rows x (a head block's accumulators, HB * hd <= min(2048 / esz, d)
// floats, and the block's maxima and sums, 2 x HB <= 16).
__host__ __device__ inline size_t att_cmb_bytes(int esz, int d) {
  const int hbhd = 2048 / esz < d ? 2048 / esz : d;
  return (size_t)(NCONS - 1) * NRA * (hbhd + 16) * 4;
}
__host__ __device__ inline size_t x_region_bytes(int M, int esz, int XC, int d) {
  const size_t x = (size_t)M * (XC + 16 / esz) * esz, c = att_cmb_bytes(esz, d);
  return x > c ? x : c;
}
// Per-launch row tables in LDS: rows by group [M], depth histogram [64], group offsets and
// count [65], copies of the rows' slot [M], depth [M] and ancestor offsets [M + 1], and the
// virtual groups of the attention phase [M + 1].
__host__ __device__ inline int row_table_ints(int M) { return M + 64 + 65 + M + M + M + 1 + M + 1; }
// Key-slot windows of the producer waves (ATT_WPW slots each).
constexpr int ATT_WPW = 256;
constexpr int ATT_WIN = 2 * ATT_WPW;
// Row-normalisation scratch: the factor of each row, or (staging of rows split over the
// consumer waves) two buffers of up to SRG rows' NCONS quarter sums of squares.
constexpr int SRG = 2;
__host__ __device__ inline int norm_floats(int M) {
  const int g = M < SRG ? M : SRG;
  return 2 * g * NCONS > M ? 2 * g * NCONS : M;
}
__host__ __device__ inline size_t lds_bytes_for(int M, int esz, int NS, int XC, int nred, int d) {
  size_t off = (size_t)NS * SLAB + ATT_WIN * 4;
  off = (off + x_region_bytes(M, esz, XC, d) + 15) & ~(size_t)15;
  off = (off + (size_t)row_table_ints(M) * 4 + 15) & ~(size_t)15;
  off = (off + (size_t)nred * NCONS * M * 16 * 4 + 15) & ~(size_t)15;
  off = (off + (size_t)norm_floats(M) * 4 + 15) & ~(size_t)15;
  off = (off + (size_t)M * 4 + 15) & ~(size_t)15;
  off += (2 * NS + 8) * 4;
  return off;
}
__host__ __device__ inline LdsPlan lds_plan(int M, int esz, int d) {
  const int sk = 512 / esz;
  const int xfull = (d + sk - 1) / sk * sk;
#ifndef LS_NS_MAX
#define LS_NS_MAX 18
#endif
  const int ns_opts[6] = {LS_NS_MAX, LS_NS_MAX - 2, LS_NS_MAX - 4, LS_NS_MAX - 6, LS_NS_MAX - 8, 8};
  for (int i = 0; i < 6; ++i)
    if (lds_bytes_for(M, esz, ns_opts[i], xfull, 2, d) <= LDS_BUDGET) return LdsPlan{ns_opts[i], xfull, 2};
  // many rows: narrower activation chunks first, then a shallower ring (down to 4 slabs, one
  // per consumer), so every row count up to the workspace maximum fits
  LdsPlan p{8, xfull, M <= 64 ? 2 : 1};
  while (p.XC > sk && lds_bytes_for(M, esz, p.NS, p.XC, p.nred, d) > LDS_BUDGET) p.XC = (p.XC / 2 + sk - 1) / sk * sk;
  while (p.NS > NCONS && lds_bytes_for(M, esz, p.NS, p.XC, p.nred, d) > LDS_BUDGET) p.NS -= 2;
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
  int* win;          // key-slot windows of the producer waves, ATT_WPW each
  char* X;           // M x (XC + pad) elements
  float* red;        // nred x NCONS x M x 16: per-tile partials of the consumer waves
  float* rinv;       // norm_floats(M): row factors, or the split staging's quarter sums
  int* hx;           // M: hidden-state row of each working row (-1: none)
  int* grow;         // M: rows ordered by KV depth group (attention shares a group's keys)
  int* goff;         // group g's rows: grow[goff[g] .. goff[g+1]); goff[64] = group count
  int *rslot, *rdep, *raoff;   // the rows' validated slot, depth (0 without depths), ancestor offsets
  int* vgt;          // virtual groups (attention): g + 64 * first row within group g; [M] = count
  int* ints;         // [0..NS) full, [NS..2NS) empty (NCONS per release), [2NS] consumer barrier, [2NS+1+b] partials
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
  s.win = (int*)(base + off); off += ATT_WIN * 4;
  s.X = base + off; off = align16(off + x_region_bytes(M, (int)sizeof(T), s.XC, d));
  s.grow = (int*)(base + off);
  s.goff = s.grow + M + 64;
  s.rslot = s.goff + 65;
  s.rdep = s.rslot + M;
  s.raoff = s.rdep + M;
  s.vgt = s.raoff + M + 1;
  off = align16(off + (size_t)row_table_ints(M) * 4);
  s.red = (float*)(base + off); off = align16(off + (size_t)s.nred * NCONS * M * 16 * 4);
  s.rinv = (float*)(base + off); off = align16(off + (size_t)norm_floats(M) * 4);
  s.hx = (int*)(base + off); off = align16(off + (size_t)M * 4);
  s.ints = (int*)(base + off);
  return s;
}

size_t mega_smem_bytes(bool bf16, int M, int d) {
  const int esz = bf16 ? 2 : 4;
  const LdsPlan p = lds_plan(M, esz, d);
  return lds_bytes_for(M, esz, p.NS, p.XC, p.nred, d);
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

// A phase's tiles for workgroup b, in order: tile first + i*G, i < count (round-robin).
struct PhaseShare {
  int first, count;
  LS_DEV int tile(int i, int G) const { return first + i * G; }
};
LS_DEV PhaseShare phase_share(int n, int deal, int G, int b) {
  const Share sh = share_of(n, deal, G, b);
  return PhaseShare{sh.first, sh.count};
}

// The residual phases (O, DOWN) have only d/16 tiles, often between one and two per workgroup,
// so when there are more tiles than workgroups they are dealt by slabs (stream-K; with at most
// one tile per workgroup whole tiles are balanced already and need no combining of partial
// sums): workgroup b < Gs = min(G, n * nk) takes the phase's slabs
// [b * n * nk / Gs, (b + 1) * n * nk / Gs) in tile-major order, as units (tile, slabs
// [k0, k1)).  A tile whose slabs span several (consecutive) workgroups is split: each leaves
// its partial sum, and the last to arrive adds them in workgroup order and runs the epilogue.
// Other phases deal whole tiles round-robin.
LS_DEV bool split_phase(int ph) { return ph == PH_O || ph == PH_DOWN; }
struct Units {
  bool split;
  PhaseShare sh;
  int nk;                    // slabs per tile
  int S0, S1, total, Gs;     // split phases: this workgroup's slabs, all slabs, workgroups used
  LS_DEV int count() const {
    if (!split) return sh.count;
    return S1 > S0 ? (S1 - 1) / nk - S0 / nk + 1 : 0;
  }
  LS_DEV void get(int i, int G, int& t, int& k0, int& k1) const {
    if (!split) { t = sh.tile(i, G); k0 = 0; k1 = nk; return; }
    t = S0 / nk + i;
    k0 = max(S0 - t * nk, 0);
    k1 = min(S1 - t * nk, nk);
  }
  LS_DEV int owner(int sl) const { return (int)(((long long)(sl + 1) * Gs - 1) / total); }
  LS_DEV int first_tile(int b) const { return (int)((long long)b * total / Gs) / nk; }
  // the partial slot of workgroup b for split tile t: 0 for its first unit, 1 for its last
  LS_DEV int pslot(int b, int t) const { return t == first_tile(b) ? 0 : 1; }
};
LS_DEV Units units_of(int ph, int n_tiles, int nk, int deal, int G, int b) {
  Units u;
  u.split = split_phase(ph) && n_tiles > G;   // at most one tile per workgroup: whole tiles
  u.nk = nk;
  u.sh = PhaseShare{0, 0};
  u.S0 = u.S1 = 0;
  u.total = n_tiles * nk;
  u.Gs = min(G, u.total);
  if (!u.split) {
    u.sh = phase_share(n_tiles, deal, G, b);
  } else if (b < u.Gs) {
    u.S0 = (int)((long long)b * u.total / u.Gs);
    u.S1 = (int)((long long)(b + 1) * u.total / u.Gs);
  }
  return u;
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
#ifndef LS_PFL
#define LS_PFL 4
#endif
constexpr int PFL = LS_PFL;
// Cache policy of the weight loads: non-temporal.  Every weight byte is read once per call, by
// one workgroup; marked as streaming, the loads sustain ~7.0 TB/s on MI355X where the default
// policy sustains ~6.1 (a 16-row x 512-byte slab pattern read straight into LDS, 256
// workgroups of two loading waves, measured on the device).
#ifndef LS_WEIGHT_CPOL
#define LS_WEIGHT_CPOL 2
#endif
constexpr int WEIGHT_CPOL = LS_WEIGHT_CPOL;

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
    if (lane == 0) lds_bump_nw(s.ints + pslot);
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

  // Row addresses of an attention tile: row 2i (lanes 0-31) is key i's K piece, row 2i + 1
  // (lanes 32-63) its V piece, `hoff` bytes into the cache entries of slots sl[0..7] of the
  // cache block at `cache`.  Unlike weight rows these are not swizzled: the attention
  // consumers read a row's 8-byte units at consecutive addresses.
  LS_DEV void begin_kv_tile(const char* cache, const int (&sl)[8], int hoff) {
    const size_t ent = (size_t)2 * a.d * sizeof(T);
    const int vo = (lane >> 5) * a.d * (int)sizeof(T) + hoff;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      co[i] = (lane & 31) * 16;
      rp[i] = cache + (size_t)sl[i] * ent + vo + co[i];
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
      while (lds_peek(s.ints + s.NS + slot) < NCONS * use) {
        if (pub < mine) {
          wait_vm_le8(8 * (mine - pub - 1));
          publish_one();
        } else if (give_up(n, a.err)) {
          break;
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
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(dst + i * 1024), 16, 0, WEIGHT_CPOL);
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
    if (fuse && xn > FUSE_MAX_K) {
      // a quarter of qw <= FUSE_MAX_K columns is ceil(qw / 256) float4 per lane
      const int qw = (xn + 4 * NCONS - 1) / (4 * NCONS) * 4;
      stage_split_nv<8>((qw + 255) / 256, src, via_hidx, gain, xn, poll);
      return;
    }
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
            if (give_up(n, a.err)) break;
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

  // Whole rows wider than one wave's fused pass (FUSE_MAX_K < xn <= NCONS * FUSE_MAX_K): consumer
  // wave c takes quarter c of every row, NV float4 per lane.  Rows go SRG at a time: the waves
  // load (or poll) their quarters of the group's rows and the gains at once, leave each
  // quarter's sum of squares in LDS, meet, and normalise from registers; the row's factor adds
  // the four quarter sums in wave order.
  template <int NV>
  LS_DEV void stage_norm_split(const float* src, bool via_hidx, const float* gain, int xn, bool poll) {
    T* X = (T*)s.X;
    const int qw = (xn + 4 * NCONS - 1) / (4 * NCONS) * 4;     // columns per quarter
    const int q0 = min(c * qw, xn), qn = min(qw, xn - q0);
    const __amdgpu_buffer_rsrc_t Rg = rsrc_of(gain + q0, qn * 4);
    u32x4_t gv[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) gv[u] = ld128(Rg, (4 * (lane + 64 * u)) * 4);
    const int gmax = min(SRG, a.M);
    int grp = 0;
    for (int m0 = 0; m0 < a.M; m0 += SRG, ++grp) {
      const int gn = min(SRG, a.M - m0);
      __amdgpu_buffer_rsrc_t R[SRG];
#pragma unroll
      for (int r = 0; r < SRG; ++r) {
        const int m = m0 + min(r, gn - 1);
        const int hv = __builtin_amdgcn_readfirstlane(s.hx[m]);   // negative: rejected row, stages zeros
        const int hr = via_hidx ? hv : m;
        R[r] = rsrc_of(src + (size_t)(hv >= 0 ? hr : 0) * a.d + q0, r < gn && hv >= 0 ? qn * 4 : 0);
      }
      u32x4_t v[SRG][NV];
      if (poll) {
        // a quarter is complete once none of its elements holds the fill pattern
        int n = 0;
        while (true) {
#pragma unroll
          for (int r = 0; r < SRG; ++r)
#pragma unroll
            for (int u = 0; u < NV; ++u) v[r][u] = ldc128(R[r], (4 * (lane + 64 * u)) * 4);
          bool ok = true;
#pragma unroll
          for (int r = 0; r < SRG; ++r)
#pragma unroll
            for (int u = 0; u < NV; ++u)
              ok = ok && v[r][u].x != SENT32 && v[r][u].y != SENT32 && v[r][u].z != SENT32 && v[r][u].w != SENT32;
          if (__all(ok)) break;
          __builtin_amdgcn_s_sleep(POLL_SLEEP);
          if (give_up(n, a.err)) break;
        }
      } else {
#pragma unroll
        for (int r = 0; r < SRG; ++r)
#pragma unroll
          for (int u = 0; u < NV; ++u) v[r][u] = ld128(R[r], (4 * (lane + 64 * u)) * 4);
      }
      float* sp = s.rinv + (grp & 1) * gmax * NCONS;   // alternate buffers: one meeting per group
#pragma unroll
      for (int r = 0; r < SRG; ++r) {
        float ss = 0.f;
#pragma unroll
        for (int u = 0; u < NV; ++u) {
          const float f0 = __uint_as_float(v[r][u].x), f1 = __uint_as_float(v[r][u].y);
          const float f2 = __uint_as_float(v[r][u].z), f3 = __uint_as_float(v[r][u].w);
          ss += (f0 * f0 + f1 * f1) + (f2 * f2 + f3 * f3);
        }
        ss = wave_sum(ss);
        if (lane == 0 && r < gn) sp[r * NCONS + c] = ss;
      }
      cb.sync();
#pragma unroll
      for (int r = 0; r < SRG; ++r) {
        if (r >= gn) break;
        const float tot = (sp[r * NCONS] + sp[r * NCONS + 1]) + (sp[r * NCONS + 2] + sp[r * NCONS + 3]);
        const float ri = 1.0f / sqrtf(tot / (float)a.d + a.eps);
        T* xr = X + (size_t)(m0 + r) * s.xstride + q0;
#pragma unroll
        for (int u = 0; u < NV; ++u) {
          const int k = 4 * (lane + 64 * u);
          if (k < qn) put4(xr + k, v[r][u], ri, gv[u]);
        }
      }
    }
    cb.sync();
  }
  // stage_norm_split with NV = nv (3 <= nv <= NVMAX: quarters wider than FUSE_MAX_K / NCONS)
  template <int NVMAX>
  LS_DEV void stage_split_nv(int nv, const float* src, bool via_hidx, const float* gain, int xn, bool poll) {
    if constexpr (NVMAX > 3) {
      if (nv < NVMAX) {
        stage_split_nv<NVMAX - 1>(nv, src, via_hidx, gain, xn, poll);
        return;
      }
    }
    stage_norm_split<NVMAX>(src, via_hidx, gain, xn, poll);
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
          if (give_up(n, a.err)) break;
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

  // Pass one slab of the sequence; if it is this consumer's, multiply it (q: the slab's index in
  // the staged activation chunk).
  LS_DEV void slab(int q, int kn, f32x4_t* acc) {
    const int slot = cslot, use = cuse;
    if (++cslot == s.NS) { cslot = 0; ++cuse; }
    // slabs are dealt to the consumers by position in the workgroup's whole sequence, so the
    // four share every phase's slabs evenly whatever the slabs per tile
    if (((use * s.NS + slot) & (NCONS - 1)) != c) return;
    if (lane == 0) {
      int n = 0;
      while (lds_peek(s.ints + slot) < use + 1)     // tight poll: the slab is usually close
        if (give_up(n, a.err)) break;
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
    if (lane == 0) lds_add(s.ints + s.NS + slot, NCONS);
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
        const float nv = hr >= 0 ? canon_nan(res[u] + Ts[m * 16 + nl]) : 0.f;
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

// ---- attention -------------------------------------------------------------------------------------
// Causal decode attention of layer l, split over keys and merged with the log-sum-exp rule.
// Rows are grouped by KV depth (a row at loop iteration k reads the depth-k cache, LoopSpec
// section 2.1 and 2.4); rows of one group share the finished prefix's keys and are taken NRA at
// a time (a virtual group), so that each key is read once per virtual group.  The prefix keys
// stream through the producers' ring like weights:
//  1. tile (vg, hb, kt): keys [8kt, 8kt + 8) x heads [hb*HB, hb*HB + HB) of virtual group vg;
//     its 16 rows are the keys' K pieces (rows 2i) and V pieces (rows 2i + 1) of HB * hd
//     elements.  The consumers of a workgroup update a partial softmax state per (row, head)
//     from the ring; a (vg, hb) pair is a segment, and each workgroup that holds tiles of it
//     leaves one partial (max, sum, acc[hd]) per (row, head).
//  2. the last workgroup of a segment to finish merges, per (row, head), those partials with
//     the row's own keys (its speculative ancestors and itself, written by this launch) and
//     stores o[l][row][h].
struct AttGeo {
  int HB, n_hb, n_kt, n_vg;
  int N;                    // tiles: (vg * n_hb + hb) * n_kt + kt
};
template <typename T>
LS_DEV AttGeo att_geo(const MegaArgs& a, int n_vg) {
  AttGeo g;
  g.HB = att_heads_per_block(a.nh, a.hd, (int)sizeof(T));
  g.n_hb = (a.nh + g.HB - 1) / g.HB;
  g.n_kt = max(1, (a.n_fin + 7) / 8);
  g.n_vg = n_vg;
  g.N = n_vg * g.n_hb * g.n_kt;
  return g;
}
// Workgroup b < Ga = att_workgroups(G, N) takes tiles [b*N/Ga, (b+1)*N/Ga) (a share of at least
// one tile, so that the workgroups holding a segment's tiles are consecutive); the owner of tile t.
LS_DEV int att_grid(int N) { return att_workgroups((int)gridDim.x, N); }
LS_DEV int att_owner(int t, int N, int Ga) { return (int)(((long long)(t + 1) * Ga - 1) / N); }

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
// 64-bin histogram; rows with no depth array form one group.  Then the virtual groups of the
// attention phase: each group's rows, NRA at a time.
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
  // rows of a group in row order: every workgroup must split a group into the same virtual
  // groups, whose partial results other workgroups merge
  for (int m = threadIdx.x; m < a.M; m += blockDim.x) {
    const int dv = min(max(s.rdep[m], 0), 63);
    int rank = 0;
    for (int m2 = 0; m2 < m; ++m2) rank += min(max(s.rdep[m2], 0), 63) == dv;
    s.grow[hist[dv] + rank] = m;
  }
  __syncthreads();
  // virtual groups: each group's rows NRA at a time
  if (threadIdx.x == 0) {
    int nv = 0;
    for (int g = 0; g < s.goff[64]; ++g)
      for (int r0 = 0; r0 < s.goff[g + 1] - s.goff[g]; r0 += NRA) s.vgt[nv++] = g + 64 * r0;
    s.vgt[a.M] = nv;
  }
}

// A producer wave's window of key slots in LDS: slots of keys [base, base + ATT_WPW), keys past
// the prefix and out-of-range slots stored as slot 0 (the prep kernel reports the latter; the
// consumers mask keys past the prefix), so a tile's eight slots are two 16-byte LDS reads.  A
// workgroup's attention share is the same in every layer and its tiles' keys are consecutive
// within a segment, so the window is refilled only when a tile falls outside it.
struct AttWindow {
  int base = -(1 << 30);
  int* tab = nullptr;
  LS_DEV void fill(const MegaArgs& a, int kb) {
    base = kb;
    const int lane = threadIdx.x & 63;
    const unsigned S32 = (unsigned)a.S;
    int v[ATT_WPW / 64];
#pragma unroll
    for (int j = 0; j < ATT_WPW / 64; ++j) {
      const int k = kb + 64 * j + lane;
      const int x = k < a.n_fin ? a.fin[k] : 0;
      v[j] = (unsigned)x < S32 ? x : 0;
    }
    // (the compiler waits for the loads before the writes: a refill drains this wave's loads)
#pragma unroll
    for (int j = 0; j < ATT_WPW / 64; ++j) {
      const unsigned addr = (unsigned)(size_t)(__attribute__((address_space(3))) int*)(tab + 64 * j + lane);
      asm volatile("ds_write_b32 %0, %1" : : "v"(addr), "v"(v[j]) : "memory");
    }
  }
  // Slots of tile kt's eight keys.
  LS_DEV void slots(const MegaArgs& a, int kt, int (&sl)[8]) {
    const int k0 = 8 * kt;
    if (k0 < base || k0 + 8 > base + ATT_WPW) fill(a, k0);
    const unsigned addr = (unsigned)(size_t)(__attribute__((address_space(3))) int*)(tab + (k0 - base));
    u32x4_t x0, x1;
    // early-clobber outputs: the first read's destination must not share a register with the
    // address the second read still needs
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:16\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(x0), "=&v"(x1) : "v"(addr) : "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sl[i] = __builtin_amdgcn_readfirstlane((int)x0[i]);
      sl[4 + i] = __builtin_amdgcn_readfirstlane((int)x1[i]);
    }
  }
};

// The producer waves' part of the attention phase: the workgroup's tiles in order, each as
// ceil(HB * hd * esz / 512) slabs of its 16 rows (key i's K piece is row 2i, its V piece row
// 2i + 1).
template <typename T>
LS_DEV void walk_att_prod(const MegaArgs& a, const Lds& s, int l, Producer<T>& pr, AttWindow& win) {
  const AttGeo ag = att_geo<T>(a, lds_peek(s.vgt + a.M));
  const int G = att_grid(ag.N), b = blockIdx.x;
  if (b >= G) return;
  const int T0 = (int)((long long)b * ag.N / G), T1 = (int)((long long)(b + 1) * ag.N / G);
  constexpr int esz = (int)sizeof(T);
  int seg = T0 / ag.n_kt, kt = T0 - seg * ag.n_kt;
  int vg = seg / ag.n_hb, hb = seg - vg * ag.n_hb;
  int cur[8];
  int cur_vg = -1;
  const char* cache = nullptr;
  for (int t = T0; t < T1; ++t) {
    win.slots(a, kt, cur);
    if (vg != cur_vg) {
      cur_vg = vg;
      const int g = lds_peek(s.vgt + vg) & 63;
      const int rep = lds_peek(s.grow + lds_peek(s.goff + g));
      const int blk = (a.dep ? lds_peek(s.rdep + rep) + a.dep_off : 0) * a.blk_mul + a.layer0 + l;
      cache = (const char*)a.kv + (size_t)blk * a.S * 2 * a.d * esz;
    }
    const int h0 = hb * ag.HB;
    PhaseGeo g;
    g.n_tiles = 0;
    g.K = min(ag.HB, a.nh - h0) * a.hd;
    g.sk = 512 / esz;
    if (threadIdx.x == 64 * NCONS && t == T0) tstamp(a, l, PH_ATT, 5);
    pr.begin_kv_tile(cache, cur, h0 * a.hd * esz);
    const int ns = (g.K + g.sk - 1) / g.sk;
    for (int k = 0; k < ns; ++k) pr.issue(k, g);
    if (++kt == ag.n_kt) {
      kt = 0;
      if (++hb == ag.n_hb) { hb = 0; ++vg; }
    }
  }
  if (threadIdx.x == 64 * NCONS) tstamp(a, l, PH_ATT, 6);
}

// Partial records of the attention phase: acc[hd], then max and sum (16-byte aligned rows);
// layer l's records [row][head][partial] of a launch.  Each layer has records of its own: they
// carry no completion signal, so a reader tells this layer's records from an earlier layer's
// only by the fill pattern they start the launch with.
LS_DEV int att_rec(int hd) { return hd + 4; }
LS_DEV float* patt_of(const MegaArgs& a, int l) { return a.patt + (size_t)l * a.M * a.nh * a.att_pmax * att_rec(a.hd); }

// Four elements of a K / V entry written by this launch (agent-coherent load).
template <typename T> LS_DEV void load4_coh(const T* p, float* f);
template <> LS_DEV void load4_coh<uint16_t>(const uint16_t* p, float* f) {
  const unsigned long long w = ldc64(p);
  const unsigned lo = (unsigned)w, hi = (unsigned)(w >> 32);
  f[0] = __uint_as_float(lo << 16); f[1] = __uint_as_float(lo & 0xffff0000u);
  f[2] = __uint_as_float(hi << 16); f[3] = __uint_as_float(hi & 0xffff0000u);
}
template <> LS_DEV void load4_coh<float>(const float* p, float* f) {
  const unsigned long long w0 = ldc64(p), w1 = ldc64(p + 2);
  f[0] = __uint_as_float((unsigned)w0); f[1] = __uint_as_float((unsigned)(w0 >> 32));
  f[2] = __uint_as_float((unsigned)w1); f[3] = __uint_as_float((unsigned)(w1 >> 32));
}

// Sum / maximum over the 32 lanes of each half of the wave (every lane gets its half's result).
LS_DEV float half_sum(float v) {
  v = row_sum16(v);
  const float h0 = lane_f(v, 0) + lane_f(v, 16), h1 = lane_f(v, 32) + lane_f(v, 48);
  return (threadIdx.x & 32) ? h1 : h0;
}
LS_DEV float half_max(float v) {
  v = row_max16(v);
  const float h0 = fmaxf(lane_f(v, 0), lane_f(v, 16)), h1 = fmaxf(lane_f(v, 32), lane_f(v, 48));
  return (threadIdx.x & 32) ? h1 : h0;
}

// Merge of heads hA (lanes 0-31) and hB (lanes 32-63; hB < 0: none) for row i, by one wave;
// lane = 4 dims of its half's head: the np prefix partials of the row's segment and the row's
// own keys (its speculative ancestors, then itself, written by this launch), online
// log-sum-exp over batches of (16 partials, 4 own keys); every load of a batch is issued before
// any is used, so a batch costs one memory round trip.  The partial records start the launch
// filled with SENT32 and are written without a completion signal, so a batch is re-read until
// none of its words holds the fill pattern.
template <typename T>
LS_DEV void att_merge2(const MegaArgs& a, const Lds& s, int l, int blk, int i, int hA, int hB, int np) {
  const int lane = threadIdx.x & 63, half = lane >> 5, hl = lane & 31;
  const int hd = a.hd, rec = att_rec(hd);
  const int h = half ? hB : hA;
  const bool hok = h >= 0;
  const int hh = hok ? h : hA;
  const bool dok = hok && 4 * hl < hd;
  const int d0 = 4 * min(hl, hd / 4 - 1);           // this lane's dims (lanes past the head repeat)
  const T* cache = (const T*)a.kv + (size_t)blk * a.S * 2 * a.d + hh * hd + d0;
  const float scale = 1.0f / sqrtf((float)hd);
  T* orow = o_of<T>(a, l) + (size_t)i * a.d + hh * hd + d0;
  const int self = s.rslot[i];
  if (self < 0) {                                    // rejected row: zero output
    if (dok) { store2_coh<T>(orow, 0.f, 0.f); store2_coh<T>(orow + 2, 0.f, 0.f); }
    return;
  }
  const int a0 = s.raoff[i], na = s.raoff[i + 1] - a0;
  const int nt = na + 1;                             // the row's own keys: ancestors, then itself
  const float* const prow = patt_of(a, l) + (size_t)i * a.nh * a.att_pmax * rec;
  const __amdgpu_buffer_rsrc_t Rp = rsrc_of(prow, a.nh * a.att_pmax * rec * 4);
  const int pbase = hh * a.att_pmax * rec;           // this half's head: its first partial record
  float q[4];
  {
    const u32x4_t w = ldc128(rsrc_of(a.q, a.M * a.d * 4), (i * a.d + hh * hd + d0) * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) q[e] = __uint_as_float(w[e]) * scale;
  }
  float run_m = -INFINITY, den = 0.f, num[4] = {0.f, 0.f, 0.f, 0.f};
  constexpr int NK = 4;                             // own keys per batch
#ifndef LS_ATT_NPB
#define LS_ATT_NPB 16
#endif
  constexpr int NPB = LS_ATT_NPB;                   // prefix partials per batch (at most 32)
  const int nbat = max((np + NPB - 1) / NPB, (nt + NK - 1) / NK);
  for (int bt = 0; bt < nbat; ++bt) {
    const int c0 = bt * NPB, j0 = bt * NK;
    // ---- the batch's own keys, then its partials, re-read until none holds the fill pattern
    float kf[NK][4], vf[NK][4];
    bool bad = false;
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      const int j = min(j0 + u, nt - 1);
      int x = j < na ? a.anc[a0 + j] : self;
      if (x < 0 || x >= a.S) { bad = bad || j0 + u < nt; x = self; }
      load4_coh<T>(cache + (size_t)x * 2 * a.d, kf[u]);
      load4_coh<T>(cache + (size_t)x * 2 * a.d + a.d, vf[u]);
    }
    float mxc, smc;                                  // statistics of partial c0 + hl (hl < NPB)
    u32x4_t ac[NPB];
    for (int n = 0;;) {
      mxc = -INFINITY;
      smc = 0.f;
      if (hok && hl < NPB && c0 + hl < np) {
        mxc = ldc(prow + pbase + (size_t)(c0 + hl) * rec + hd);
        smc = ldc(prow + pbase + (size_t)(c0 + hl) * rec + hd + 1);
      }
#pragma unroll
      for (int u = 0; u < NPB; ++u)
        ac[u] = ldc128(Rp, hok && c0 + u < np ? (pbase + (c0 + u) * rec + d0) * 4 : 0x7fffff00);
      bool ok = __float_as_uint(mxc) != SENT32 && __float_as_uint(smc) != SENT32;
#pragma unroll
      for (int u = 0; u < NPB; ++u) ok = ok && ac[u].x != SENT32 && ac[u].y != SENT32 && ac[u].z != SENT32 && ac[u].w != SENT32;
      if (__all(ok)) break;
      __builtin_amdgcn_s_sleep(POLL_SLEEP);
      if (give_up(n, a.err)) break;
    }
    if (bad) ls_flag(a.err, 1);
    // ---- the batch's scores and its maximum
    float sc[NK];
    float bm = half_max(mxc);
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      const float part = dok ? (q[0] * kf[u][0] + q[1] * kf[u][1]) + (q[2] * kf[u][2] + q[3] * kf[u][3]) : 0.f;
      sc[u] = half_sum(part);
      if (j0 + u < nt) bm = fmaxf(bm, sc[u]);
    }
    const float nm = fmaxf(run_m, bm);
    if (__all(nm == -INFINITY)) continue;            // nothing in this batch or before
    const float rs = run_m == -INFINITY ? 0.f : __expf(run_m - nm);
    den *= rs;
#pragma unroll
    for (int e = 0; e < 4; ++e) num[e] *= rs;
    run_m = nm;
    // prefix partials: weight w_c = exp(mx_c - m) held by lane c - c0 of the half
    const float wl = mxc == -INFINITY ? 0.f : __expf(mxc - nm);
    den += half_sum(wl * smc);
#pragma unroll
    for (int u = 0; u < NPB; ++u) {
      const float w = half ? lane_f(wl, 32 + u) : lane_f(wl, u);
#pragma unroll
      for (int e = 0; e < 4; ++e) num[e] += w * __uint_as_float(ac[u][e]);
    }
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      const float w = j0 + u < nt ? __expf(sc[u] - nm) : 0.f;
      den += w;
#pragma unroll
      for (int e = 0; e < 4; ++e) num[e] += w * vf[u][e];
    }
  }
  if (dok) {
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = den > 0.f ? canon_nan(num[e] / den) : 0.f;
    store2_coh<T>(orow, y[0], y[1]);
    store2_coh<T>(orow + 2, y[2], y[3]);
  }
}

// 8 bytes of LDS at byte address addr.
LS_DEV u32x2_t lds_ld64(unsigned addr) {
  return *(const __attribute__((address_space(3))) u32x2_t*)(size_t)addr;
}

// Agent-coherent stores of 16 / 8 bytes through a buffer descriptor (the store side of ldc128).
LS_DEV void stc128(__amdgpu_buffer_rsrc_t r, int byte_off, const u32x4_t& v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, CPOL_SC1);
}

// A lane's share of a head's K or V piece in the attention phase: 8-byte units u = g, g + 8,
// ... (g: the lane's place among the head's eight lanes), D elements each.  UMAX units cover a
// 128-dim head; KG keys' K units are held in registers at once.
template <typename T> struct AttUnit;
template <> struct AttUnit<uint16_t> {
  static constexpr int D = 4, UMAX = 4, KG = 4;
  LS_DEV static void unpack(const u32x2_t& w, float* f) {
    f[0] = __uint_as_float(w[0] << 16);
    f[1] = __uint_as_float(w[0] & 0xffff0000u);
    f[2] = __uint_as_float(w[1] << 16);
    f[3] = __uint_as_float(w[1] & 0xffff0000u);
  }
  // D fp32 elements at byte offset off of r (zeros out of range)
  LS_DEV static void load(__amdgpu_buffer_rsrc_t r, int off, float* f) {
    const u32x4_t w = ldc128(r, off);
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(w[e]);
  }
  LS_DEV static void store(__amdgpu_buffer_rsrc_t r, int off, const float* f) {
    stc128(r, off, u32x4_t{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])});
  }
};
template <> struct AttUnit<float> {
  static constexpr int D = 2, UMAX = 8, KG = 2;
  LS_DEV static void unpack(const u32x2_t& w, float* f) {
    f[0] = __uint_as_float(w[0]);
    f[1] = __uint_as_float(w[1]);
  }
  LS_DEV static void load(__amdgpu_buffer_rsrc_t r, int off, float* f) {
    const u32x2_t w = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, CPOL_SC1);
    f[0] = __uint_as_float(w[0]);
    f[1] = __uint_as_float(w[1]);
  }
  LS_DEV static void store(__amdgpu_buffer_rsrc_t r, int off, const float* f) {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{__float_as_uint(f[0]), __float_as_uint(f[1])}, r, off, 0, CPOL_SC1);
  }
};

// Rows (up to NRA), cache block and head block of attention segment sg of layer l.
LS_DEV void att_segment(const MegaArgs& a, const Lds& s, const AttGeo& ag, int l, int sg, int (&rows)[NRA], int& nr,
                        int& blk, int& h0, int& hbn) {
  const int vg = sg / ag.n_hb, hb = sg - vg * ag.n_hb;
  const int vt = s.vgt[vg], gr = vt & 63, r0 = vt >> 6;
  const int g0 = s.goff[gr];
  nr = min(NRA, s.goff[gr + 1] - g0 - r0);
#pragma unroll
  for (int r = 0; r < NRA; ++r) rows[r] = s.grow[g0 + r0 + min(r, nr - 1)];
  blk = (a.dep ? s.rdep[s.grow[g0]] + a.dep_off : 0) * a.blk_mul + a.layer0 + l;
  h0 = hb * ag.HB;
  hbn = min(ag.HB, a.nh - h0);
}

// Release of a tile's ns ring slots from slot first on (a whole release per slab: the tile's
// consumer is its only reader).
struct SlotRelease {
  int* empty;
  int first, ns, NS;
  LS_DEV void operator()() const {
    const int lane = threadIdx.x & 63;
    if (lane < ns) {
      int sl = first + lane;
      if (sl >= NS) sl -= NS;
      lds_add(empty + sl, NCONS);
    }
  }
};

// One tile for one consumer: the eight keys' K units (LDS addresses ua[j] + 1024 i, V units
// 512 further) against the lane's query elements, the scores summed over the head's eight lanes,
// the online-softmax update of the state, and the weighted V units into the accumulators.  JN
// units per lane (a compile-time count, so the loops carry no guards); kn valid keys.  With
// bf16 pieces all of the tile's units are read into registers first and the slots released
// (`release`) before any arithmetic, so that a consumer holds ring slots only for the reads;
// fp32 pieces (twice the registers) are read KG keys at a time and released at the end.
template <typename T, int JN, typename Rel>
LS_DEV void att_tile(const unsigned (&ua)[AttUnit<T>::UMAX], float (&q)[NRA][AttUnit<T>::UMAX * AttUnit<T>::D],
                     float (&acc)[NRA][AttUnit<T>::UMAX * AttUnit<T>::D], float (&mrun)[NRA], float (&lsum)[NRA],
                     int kn, const Rel& release) {
  using U = AttUnit<T>;
  constexpr int D = U::D;
  constexpr bool EARLY = sizeof(T) == 2 && JN <= 3;
  constexpr int KG = EARLY ? 8 : U::KG;
  u32x2_t ke[EARLY ? 8 : 1][JN], vw[EARLY ? 8 : 1][JN];
  if constexpr (EARLY) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < JN; ++j) {
        ke[i][j] = lds_ld64(ua[j] + 1024 * i);
        vw[i][j] = lds_ld64(ua[j] + 1024 * i + 512);
      }
    release();
  }
  float sc[NRA][8];
#pragma unroll
  for (int k0 = 0; k0 < 8; k0 += KG) {
    u32x2_t kw[KG][JN];
#pragma unroll
    for (int i = 0; i < KG; ++i)
#pragma unroll
      for (int j = 0; j < JN; ++j) {
        if constexpr (EARLY) kw[i][j] = ke[k0 + i][j];
        else kw[i][j] = lds_ld64(ua[j] + 1024 * (k0 + i));
      }
#pragma unroll
    for (int i = 0; i < KG; ++i) {
#pragma unroll
      for (int r = 0; r < NRA; ++r) sc[r][k0 + i] = 0.f;
#pragma unroll
      for (int j = 0; j < JN; ++j) {
        float f[D];
        U::unpack(kw[i][j], f);
#pragma unroll
        for (int r = 0; r < NRA; ++r)
#pragma unroll
          for (int e = 0; e < D; ++e) sc[r][k0 + i] += q[r][j * D + e] * f[e];
      }
    }
  }
  float p[NRA][8];
#pragma unroll
  for (int r = 0; r < NRA; ++r) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float x = sc[r][i];
      x += dpp_f<0xB1>(x);                          // the head's eight lanes: quads, then halves
      x += dpp_f<0x4E>(x);
      x += dpp_f<0x141>(x);
      sc[r][i] = i < kn ? x : -INFINITY;
      mx = fmaxf(mx, sc[r][i]);
    }
    // the state is rescaled only when the running maximum grows
    const bool up = mx > mrun[r];
    if (__any(up)) {
      const float al = !up ? 1.f : (mrun[r] == -INFINITY ? 0.f : __expf(mrun[r] - mx));
      lsum[r] *= al;
#pragma unroll
      for (int x2 = 0; x2 < JN * D; ++x2) acc[r][x2] *= al;
      if (up) mrun[r] = mx;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[r][i] = sc[r][i] == -INFINITY ? 0.f : __expf(sc[r][i] - mrun[r]);
      lsum[r] += p[r][i];
    }
  }
#pragma unroll
  for (int k0 = 0; k0 < 8; k0 += KG) {
    u32x2_t vg[KG][JN];
#pragma unroll
    for (int i = 0; i < KG; ++i)
#pragma unroll
      for (int j = 0; j < JN; ++j) {
        if constexpr (EARLY) vg[i][j] = vw[k0 + i][j];
        else vg[i][j] = lds_ld64(ua[j] + 1024 * (k0 + i) + 512);
      }
#pragma unroll
    for (int i = 0; i < KG; ++i) {
#pragma unroll
      for (int j = 0; j < JN; ++j) {
        float f[D];
        U::unpack(vg[i][j], f);
#pragma unroll
        for (int r = 0; r < NRA; ++r)
#pragma unroll
          for (int e = 0; e < D; ++e) acc[r][j * D + e] += p[r][k0 + i] * f[e];
      }
    }
  }
  if constexpr (!EARLY) release();
}
// att_tile with JN = jn (1 <= jn <= JMAX)
template <typename T, int JMAX, typename Rel>
LS_DEV void att_tile_jn(int jn, const unsigned (&ua)[AttUnit<T>::UMAX],
                        float (&q)[NRA][AttUnit<T>::UMAX * AttUnit<T>::D],
                        float (&acc)[NRA][AttUnit<T>::UMAX * AttUnit<T>::D], float (&mrun)[NRA], float (&lsum)[NRA],
                        int kn, const Rel& release) {
  if constexpr (JMAX > 1) {
    if (jn < JMAX) {
      att_tile_jn<T, JMAX - 1>(jn, ua, q, acc, mrun, lsum, kn, release);
      return;
    }
  }
  att_tile<T, JMAX>(ua, q, acc, mrun, lsum, kn, release);
}

// The consumer waves' part of the attention phase.  The workgroup's tiles are dealt to the four
// consumers in turn (tile i of the share to consumer i mod 4), and a consumer reads its tiles'
// slabs alone.  Lane = (head hi of the block, place g among the head's eight lanes): the lane
// holds units g, g + 8, ... of the head's K and V pieces, so a key's score is a partial dot
// product per lane that three DPP steps sum over the head's lanes; every lane of the head then
// holds the tile's eight scores, its maximum and the weights.  Per row (up to NRA, the rows of
// the segment's virtual group) a lane keeps its query elements and a softmax state over its
// consumer's keys: running maximum and sum (equal on the head's lanes) and the accumulator of
// its elements.  At the end of its part of a segment the workgroup combines the four consumers'
// states in LDS, consumer 0 leaves one partial per (row, head), and the last workgroup of the
// segment merges.
template <typename T, int MT>
LS_DEV void att_phase(const MegaArgs& a, const Lds& s, const CntLayout& cl, int l, Consumer<T, MT>& co,
                      ConsBar& cb) {
  using U = AttUnit<T>;
  constexpr int D = U::D, UMAX = U::UMAX, KG = U::KG, QN = UMAX * D;
  const AttGeo ag = att_geo<T>(a, s.vgt[a.M]);
  const int G = att_grid(ag.N), b = blockIdx.x;
  if (b >= G) return;
  const int T0 = (int)((long long)b * ag.N / G), T1 = (int)((long long)(b + 1) * ag.N / G);
  int* C = a.cnt + (size_t)l * cl.per_layer;
  const int lane = threadIdx.x & 63, hi = lane >> 3, g = lane & 7;
  const int c = co.c;
  const int hd = a.hd;
  constexpr int esz = (int)sizeof(T);
  const int nu = hd * esz / 8;                      // units of one head's piece
  const int jn = (nu + 7) / 8;                      // units per lane (the last ones ragged)
  const float scale = 1.0f / sqrtf((float)hd);
  const __amdgpu_buffer_rsrc_t Rq = rsrc_of(a.q, a.M * a.d * 4);
  // softmax states of consumers 1..3: [consumer][row][HB x hd accumulators, HB maxima, HB sums]
  float* const cmb = (float*)s.X;
  const int cst = ag.HB * (hd + 2);
  float q[NRA][QN], acc[NRA][QN], mrun[NRA], lsum[NRA];
  int rows[NRA];
  int nr = 0, hbn = 0, h0 = 0, blk = 0;
  bool hv = false;
  int seg = T0 / ag.n_kt, kt = T0 - seg * ag.n_kt;
  int cur_seg = -1;

  // end of this workgroup's part of segment sg: one partial per (row, head), written without a
  // completion signal (the segment's merger polls the records)
  auto flush = [&](int sg) {
    const int o0 = att_owner(sg * ag.n_kt, ag.N, G);
    if (c > 0 && hv) {
#pragma unroll
      for (int r = 0; r < NRA; ++r) {
        if (r >= nr) break;
        float* cs = cmb + (size_t)((c - 1) * NRA + r) * cst;
#pragma unroll
        for (int j = 0; j < UMAX; ++j) {
          const int u = g + 8 * j;
          if (j < jn && u < nu) {
#pragma unroll
            for (int e = 0; e < D; ++e) cs[hi * hd + D * u + e] = acc[r][j * D + e];
          }
        }
        if (g == 0) {
          cs[ag.HB * hd + hi] = mrun[r];
          cs[ag.HB * hd + ag.HB + hi] = lsum[r];
        }
      }
    }
    cb.sync();
    if (c == 0) {
      if (hv) {
#pragma unroll
        for (int r = 0; r < NRA; ++r) {
          if (r >= nr) break;
          float mo[NCONS - 1], so[NCONS - 1];
          float mx = mrun[r];
#pragma unroll
          for (int k = 0; k < NCONS - 1; ++k) {
            const float* cs = cmb + (size_t)(k * NRA + r) * cst;
            mo[k] = cs[ag.HB * hd + hi];
            so[k] = cs[ag.HB * hd + ag.HB + hi];
            mx = fmaxf(mx, mo[k]);
          }
          float wk[NCONS - 1];
          const float w0 = mrun[r] == -INFINITY ? 0.f : __expf(mrun[r] - mx);
          float sum = w0 * lsum[r];
#pragma unroll
          for (int k = 0; k < NCONS - 1; ++k) {
            wk[k] = mo[k] == -INFINITY ? 0.f : __expf(mo[k] - mx);
            sum += wk[k] * so[k];
          }
          // partial record of (row, head h0 + hi) from this workgroup
          float* const prow = patt_of(a, l) + (size_t)rows[r] * a.nh * a.att_pmax * att_rec(hd);
          const __amdgpu_buffer_rsrc_t Rp = rsrc_of(prow, a.nh * a.att_pmax * att_rec(hd) * 4);
          const int rec0 = ((h0 + hi) * a.att_pmax + (b - o0)) * att_rec(hd);
#pragma unroll
          for (int j = 0; j < UMAX; ++j) {
            const int u = g + 8 * j;
            if (j < jn && u < nu) {
              float y[D];
#pragma unroll
              for (int e = 0; e < D; ++e) {
                y[e] = w0 * acc[r][j * D + e];
#pragma unroll
                for (int k = 0; k < NCONS - 1; ++k)
                  y[e] += wk[k] * cmb[(size_t)(k * NRA + r) * cst + hi * hd + D * u + e];
              }
              U::store(Rp, (rec0 + D * u) * 4, y);
            }
          }
          if (g == 0) {
            stc(prow + rec0 + hd, mx);
            stc(prow + rec0 + hd + 1, sum);
          }
        }
      }
    }
    // consumers 1..3 write the next segment's states only after the sync of its set-up, which
    // consumer 0 reaches once it has read these
  };

  const unsigned ring0 = (unsigned)(size_t)(__attribute__((address_space(3))) char*)s.ring;
  for (int t = T0; t < T1; ++t) {
    if (seg != cur_seg) {
      if (cur_seg >= 0) flush(cur_seg);
      cur_seg = seg;
      att_segment(a, s, ag, l, seg, rows, nr, blk, h0, hbn);
      hv = hi < hbn;
      // queries of the block's heads are complete once their q/k/v tiles have signalled:
      // consumer c waits for heads c and c + 4 (whose merge it may run), then all four meet
      {
        const int nf = 3 * (hd / 16);
        bool done = true;
        int fi = 0;
        if (lane < nf) { done = c >= hbn; fi = (h0 + c) * nf + lane; }
        else if (lane < 2 * nf) { done = c + 4 >= hbn; fi = (h0 + c + 4) * nf + lane - nf; }
        int n = 0;
        while (true) {
          if (!done) done = ld_acq(C + cl.o_qkvh + (size_t)fi * PADC) >= 1;
          if (__all(done)) break;
          __builtin_amdgcn_s_sleep(POLL_SLEEP);
          if (give_up(n, a.err)) break;
        }
      }
      cb.sync();
#pragma unroll
      for (int r = 0; r < NRA; ++r) {
#pragma unroll
        for (int j = 0; j < UMAX; ++j) {
          const int u = g + 8 * j;
          const bool ok = hv && r < nr && j < jn && u < nu;
          U::load(Rq, ok ? (rows[r] * a.d + (h0 + hi) * hd + D * u) * 4 : 0x7fffff00, q[r] + j * D);
#pragma unroll
          for (int e = 0; e < D; ++e) q[r][j * D + e] *= scale;
        }
        mrun[r] = -INFINITY;
        lsum[r] = 0.f;
#pragma unroll
        for (int x = 0; x < QN; ++x) acc[r][x] = 0.f;
      }
    }
    const int ns = (hbn * hd * esz + 511) / 512;
    if (((t - T0) & (NCONS - 1)) == c) {
      // ---- one tile of this consumer: keys [8kt, 8kt + 8)
      {
        // lane k < ns watches the tile's slab k
        const int k = lane < ns ? lane : 0;
        int sl = co.cslot + k, us = co.cuse;
        if (sl >= s.NS) { sl -= s.NS; ++us; }
        int n = 0;
        while (!__all(lds_read_lane(s.ints + sl) >= us + 1))   // tight poll: the slabs are usually close
          if (give_up(n, a.err)) break;
      }
      __builtin_amdgcn_wave_barrier();
      asm volatile("" : : : "memory");
      // LDS address of each unit in key 0's K row; key i's K row is 1024 i further, its V row
      // 512 beyond that.  Units past the head (and lanes past the block) read the head's (the
      // block's) first unit, finite data whose query elements are zero.
      unsigned ua[UMAX];
#pragma unroll
      for (int j = 0; j < UMAX; ++j) {
        const int u = g + 8 * j;
        const int off = hv ? hi * hd * esz + (u < nu ? 8 * u : 0) : 0;
        int sl = co.cslot + (off >> 9);
        if (sl >= s.NS) sl -= s.NS;
        ua[j] = ring0 + (unsigned)(sl * SLAB + (off & 511));
      }
      att_tile_jn<T, UMAX>(jn, ua, q, acc, mrun, lsum, a.n_fin - 8 * kt, SlotRelease{s.ints + s.NS, co.cslot, ns, s.NS});
    }
    co.cslot += ns;
    while (co.cslot >= s.NS) { co.cslot -= s.NS; ++co.cuse; }
    if (++kt == ag.n_kt) { kt = 0; ++seg; }
  }
  flush(cur_seg);
  // Merges of the segments whose last tile this workgroup holds, after all of its own tiles:
  // consumer c takes heads c and c + 4 (it waited for their QKV tiles at the segment's set-up)
  // and polls the other workgroups' partials.
  for (int sg = T0 / ag.n_kt; sg <= (T1 - 1) / ag.n_kt; ++sg) {
    const int last = sg * ag.n_kt + ag.n_kt - 1;
    if (att_owner(last, ag.N, G) != b) continue;
    const int np = b - att_owner(sg * ag.n_kt, ag.N, G) + 1;
    att_segment(a, s, ag, l, sg, rows, nr, blk, h0, hbn);
    for (int r = 0; r < nr; ++r)
      if (c < hbn) att_merge2<T>(a, s, l, blk, rows[r], h0 + c, c + 4 < hbn ? h0 + c + 4 : -1, np);
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
// Phase ph of layer l: the workgroup's units (whole tiles, or slab ranges of tiles in the
// residual phases) one by one; within a unit, activation chunk by chunk (XC columns), slab by
// slab.
template <typename T, int MT, bool PROD>
LS_DEV void walk_gemm(const MegaArgs& a, const Lds& s, const CntLayout& cl, int ph, int l, int& deal,
                      Producer<T>* pr, Consumer<T, MT>* co, ConsBar* cb) {
  const int G = gridDim.x, b = blockIdx.x;
  const PhaseGeo g = phase_geo<T>(a, ph);
  const Units un = units_of(ph, g.n_tiles, (g.K + g.sk - 1) / g.sk, deal, G, b);
  deal = (deal + g.n_tiles) % G;
  const int nun = un.count();
  if (nun == 0) return;
  const LayerW lw = ph == PH_HEAD ? LayerW{} : a.layers[l];
  const int nchunk = (g.K + s.XC - 1) / s.XC;

  // normalised phases (QKV, GU, HEAD) read a whole row when one activation chunk covers it and
  // then take the RMSNorm factor from the same loads; otherwise from the per-tile sums of squares
  const bool fuse = nchunk == 1 && g.K <= NCONS * FUSE_MAX_K;
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

  // One unit at a time.  With one activation chunk (the usual case) the chunk is staged once
  // for all of the workgroup's units; with several, every unit re-stages the chunks it covers.
  const bool restage = nchunk > 1;
  for (int i = 0; i < nun; ++i) {
    int t, k0, k1;
    un.get(i, G, t, k0, k1);
    f32x4_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    bool began = false;
    for (int ch = 0; ch < nchunk; ++ch) {
      const int x0 = ch * s.XC;
      const int xn = min(s.XC, g.K - x0);
      const int k_first = x0 / g.sk;
      const int k_last = (x0 + xn + g.sk - 1) / g.sk;
      const int ka = max(k_first, k0), kb = min(k_last, k1);
      if (ka >= kb) continue;                 // the unit has no slab in this chunk
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
      if (PROD && !began) {
        pr->begin_tile(lw, ph, t, g);
        if (threadIdx.x == 64 * NCONS && i == 0) tstamp(a, l, ph, 5);
      }
      began = true;
      for (int k = ka; k < kb; ++k) {
        if (PROD) pr->issue(k, g);
        else co->slab(k - k_first, min(g.sk, g.K - k * g.sk), acc);
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
          if (give_up(n, a.err)) break;
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
    if (PROD && threadIdx.x == 64 * NCONS && i == nun - 1) tstamp(a, l, ph, 6);
  }
}

// The epilogue wave's part of a GEMM phase: for each of the workgroup's tiles (in the
// consumers' order) wait for the four consumer partials, sum them in consumer order, run the
// epilogue and release the partial buffer.  Stores are drained, and the tiles' counters
// bumped, once no further tile of the phase is ready, so a burst of tiles costs one drain.
//
// Residual inputs of the first O / DOWN unit, when it is a whole tile, are loaded when the walk
// starts if the workgroup had tiles in the phase before (QKV / GU): their partials having
// arrived means the consumers passed that phase's dependency wait, which implies the residual
// rows are complete (the previous layer for O, the O phase for DOWN).  The loads then overlap
// the consumers' work.
//
// A unit that covers only part of a split tile stores its sum to the workgroup's partial slot
// (spart: [workgroup][first / last unit][M x 16]) and counts itself on the tile's counter; the
// last of the tile's workgroups adds every partial in workgroup order (its own from LDS) and
// runs the epilogue.  The slots are reused from phase to phase: a residual phase starts only
// after the previous one's tiles are complete.
template <typename T>
LS_DEV void epi_walk(const MegaArgs& a, const Lds& s, const CntLayout& cl, int ph, int l, int& deal, int& seq,
                     bool& had_tiles) {
  const int G = gridDim.x, b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const PhaseGeo g = phase_geo<T>(a, ph);
  const Units un = units_of(ph, g.n_tiles, (g.K + g.sk - 1) / g.sk, deal, G, b);
  deal = (deal + g.n_tiles) % G;
  const int nun = un.count();
  int t0 = 0, k00 = 0, k10 = 0;
  if (nun > 0) un.get(0, G, t0, k00, k10);
  const bool pref = (ph == PH_O || ph == PH_DOWN) && had_tiles && nun > 0 && k00 == 0 && k10 == un.nk && a.M <= 16;
  // O / DOWN counts are waited for only when the next normalised phase cannot poll its input
  // (its row does not fit one fused staging pass); otherwise their drain and bump are skipped.
  const bool next_polls = a.d <= s.XC && a.d <= NCONS * FUSE_MAX_K;
  const bool signals = ph != PH_HEAD && !((ph == PH_O || ph == PH_DOWN) && next_polls);
  float pre[4] = {0.f, 0.f, 0.f, 0.f};
  if (pref) residual_load(a, s, ph, l, t0, 0, lane, pre);
  had_tiles = nun > 0;
  int* C = a.cnt + (size_t)l * cl.per_layer;
  const int MS = a.M * 16;
  constexpr int NPEND = 8;
  int pend[NPEND];                         // finished tiles not yet signalled
  int npend = 0;
  for (int i = 0; i < nun; ++i) {
    int t, k0, k1;
    un.get(i, G, t, k0, k1);
    const int q = seq++;
    float* buf = s.red + (size_t)(q % s.nred) * NCONS * MS;
    if (lane == 0) {
      int n = 0;
      while (lds_peek(s.ints + 2 * s.NS + 1 + q % s.nred) < NCONS * (q / s.nred + 1)) {
        __builtin_amdgcn_s_sleep(0);
        if (give_up(n, a.err)) break;
      }
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("" : : : "memory");
    for (int idx = lane; idx < MS; idx += 64) {
      float y = 0.f;
#pragma unroll
      for (int cc = 0; cc < NCONS; ++cc) y += buf[(size_t)cc * MS + idx];
      buf[idx] = y;                        // consumer 0's slot now holds the unit's sum
    }
    __builtin_amdgcn_wave_barrier();
    wait_lgkm0();                          // the sums are visible to every lane
    bool run = k0 == 0 && k1 == un.nk;     // the unit is the whole tile
    if (!run) {
      float* mine = a.spart + ((size_t)b * 2 + un.pslot(b, t)) * MS;
      for (int idx = lane; idx < MS; idx += 64) stc(mine + idx, buf[idx]);
      drain();
      int old = 0;
      if (lane == 0) old = atomicAdd(C + cl.o_split + (ph == PH_DOWN ? g.n_tiles : 0) + t, 1);
      old = __shfl(old, 0, 64);
      const int o0 = un.owner(t * un.nk), o1 = un.owner(t * un.nk + un.nk - 1);
      if (old == o1 - o0) {                // every other part has arrived: sum in workgroup order
        for (int idx = lane; idx < MS; idx += 64) {
          float y = 0.f;
          for (int bb = o0; bb <= o1; ++bb)
            y += bb == b ? buf[idx] : ldc(a.spart + ((size_t)bb * 2 + un.pslot(bb, t)) * MS + idx);
          buf[idx] = y;
        }
        __builtin_amdgcn_wave_barrier();
        wait_lgkm0();
        run = true;
      }
    }
    if (run) epilogue<T>(a, cl, s, ph, l, t, buf, lane, pref && i == 0, pre);
    wait_lgkm0();                          // the epilogue's reads of the buffer are complete
    if (lane == 0) lds_bump(s.ints + 2 * s.NS + 3);
    if (!signals) continue;
    if (run) pend[npend++] = t;
    const bool next_ready =
        i + 1 < nun && lds_peek(s.ints + 2 * s.NS + 1 + (q + 1) % s.nred) >= NCONS * ((q + 1) / s.nred + 1);
    if (npend > 0 && (!next_ready || npend == NPEND)) {
      drain();
      if (lane == 0)
        for (int k = 0; k < npend; ++k) tile_signal(a, cl, ph, l, pend[k], s.XC);
      npend = 0;
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

template <typename T, int MT>
LS_DEV void mega_body(const MegaArgs& a) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  const Lds s = lds_carve<T>(smem_raw, a.M, a.d);
  const CntLayout cl = cnt_layout(a.M, a.d, a.F, a.nh, x_chunk_for(a.M, (int)sizeof(T), a.d), a.n_layers);
  const int G = gridDim.x, b = blockIdx.x;
  const int wv = wave_id();
  // ring counters and the consumer barrier start at zero
  for (int i = threadIdx.x; i < 2 * s.NS + 8; i += MEGA_THREADS) s.ints[i] = 0;
  set_deadline(a.wait_ticks);
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
    AttWindow win;
    win.tab = s.win + (wv - NCONS) * ATT_WPW;
#pragma unroll 1
    for (int st = 0; st < n_steps; ++st) {
      const Step sp = step_of(a, st);
      if (sp.ph == PH_ATT) walk_att_prod<T>(a, s, sp.l, pr, win);
      else walk_gemm<T, MT, true>(a, s, cl, sp.ph, sp.l, deal, &pr, nullptr, nullptr);
    }
    pr.finish();
    return;
  }
  // ------------------------------ consumer waves ------------------------------
  ConsBar cb{s.ints + 2 * s.NS, 0, a.err};
  Consumer<T, MT> co(a, s, cb, wv);
  if (a.init_mode)
    for (int u = b; u < a.M; u += G) init_unit<T>(a, cl, cb, u);
#pragma unroll 1
  for (int st = 0; st < n_steps; ++st) {
    const Step sp = step_of(a, st);
    if (threadIdx.x == 0) tstamp(a, sp.l, sp.ph, 0);
    if (sp.ph == PH_ATT) {
      att_phase<T, MT>(a, s, cl, sp.l, co, cb);
    } else {
      walk_gemm<T, MT, false>(a, s, cl, sp.ph, sp.l, deal, nullptr, &co, &cb);
    }
    if (threadIdx.x == 0) tstamp(a, sp.l, sp.ph, 1);
  }
}

// Two entry symbols over the same body, so that profiles tell the loop block's launches
// (ls_loop_step) apart from the prelude, coda and LM-head launches.
template <typename T, int MT>
__global__ __launch_bounds__(MEGA_THREADS) void k_mega(MegaArgs a) { mega_body<T, MT>(a); }
template <typename T, int MT>
__global__ __launch_bounds__(MEGA_THREADS) void k_mega_aux(MegaArgs a) { mega_body<T, MT>(a); }

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
// cos/sin of the rows' positions, the check of the finished prefix's slots (the attention
// phase reads keys at slot 0 in place of an out-of-range slot), and (first launch of a call)
// the row-descriptor check.
__global__ void k_prep(int* cnt, long long n, float* rope, const int32_t* pos, const double* inv_freq, int M, int half,
                       unsigned* xs_fill, long long n_xs, unsigned* ys_fill, long long n_ys, unsigned* o_fill,
                       long long n_o, unsigned* p_fill, int p_rows, int p_max, int p_n, int p_rec, ValidateArgs v,
                       const int32_t* fin, int n_fin, long long S, int* err) {
  const long long tid = (long long)blockIdx.x * blockDim.x + threadIdx.x, str = (long long)gridDim.x * blockDim.x;
  for (long long i = tid; i < v.n; i += str) check_row(v, (int)i);
  for (long long i = tid; i < n_fin; i += str)
    if (fin[i] < 0 || fin[i] >= S) ls_flag(err, 1);
  for (long long i = tid; i < n; i += str) cnt[i] = 0;
  for (long long i = tid; i < n_xs; i += str) xs_fill[i] = SENT32;
  for (long long i = tid; i < n_ys; i += str) ys_fill[i] = SENT32;
  for (long long i = tid; i < n_o; i += str) o_fill[i] = 0xffffffffu;
  // the first p_n partial records of each of p_rows (layer, row, head) triples
  const long long per = (long long)p_n * p_rec;
  for (long long i = tid; i < (long long)p_rows * per; i += str) {
    const long long rh = i / per, k = i - rh * per;
    p_fill[rh * p_max * p_rec + k] = SENT32;
  }
  for (long long i = tid; i < (long long)M * half; i += str) {
    const int m = (int)(i / half), f = (int)(i % half);
    double sn, cs;
    sincos((double)pos[m] * inv_freq[f], &sn, &cs);
    rope[2 * i] = (float)cs;
    rope[2 * i + 1] = (float)sn;
  }
}

template <typename T>
static const void* pick_tl(int mt, bool loop) {
  if (loop) {
    if (mt <= 1) return reinterpret_cast<const void*>(&k_mega<T, 1>);
    if (mt <= 2) return reinterpret_cast<const void*>(&k_mega<T, 2>);
    if (mt <= 4) return reinterpret_cast<const void*>(&k_mega<T, 4>);
    return reinterpret_cast<const void*>(&k_mega<T, 8>);
  }
  if (mt <= 1) return reinterpret_cast<const void*>(&k_mega_aux<T, 1>);
  if (mt <= 2) return reinterpret_cast<const void*>(&k_mega_aux<T, 2>);
  if (mt <= 4) return reinterpret_cast<const void*>(&k_mega_aux<T, 4>);
  return reinterpret_cast<const void*>(&k_mega_aux<T, 8>);
}

static const void* pick(bool bf16, int M, bool loop = true) {
  const int mt = (M + 15) / 16;
  return bf16 ? pick_tl<uint16_t>(mt, loop) : pick_tl<float>(mt, loop);
}

int mega_occupancy(bool bf16, int M, int d, bool loop_block) {
  const size_t smem = mega_smem_bytes(bf16, M, d);
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, pick(bf16, M, loop_block), MEGA_THREADS, smem) !=
      hipSuccess)
    return 0;
  return n;
}

hipError_t launch_mega(bool bf16, const MegaArgs& a, int G, hipStream_t s, bool loop_block, const ValidateArgs& v) {
  const CntLayout cl = cnt_layout(a.M, a.d, a.F, a.nh, x_chunk_for(a.M, bf16 ? 2 : 4, a.d), a.n_layers);
  const long long n_patt = (long long)a.n_layers * a.M * a.nh * a.att_npf * (a.hd + 4);
  const long long n_prep = std::max<long long>(std::max<long long>(std::max<long long>(cl.total, (long long)a.M * (a.hd / 2)),
                                                                   std::max<long long>(v.n, a.n_fin)),
                                               n_patt);
  const long long rows = (long long)a.M * a.d;   // one layer slice of Xs / Ys
  hipLaunchKernelGGL(k_prep, dim3((unsigned)std::min<long long>(1024, (n_prep + 255) / 256)), dim3(256), 0, s, a.cnt,
                     (long long)cl.total, a.rope, a.pos, a.inv_freq, a.M, a.hd / 2,
                     reinterpret_cast<unsigned*>(a.Xs + rows), (long long)a.n_layers * rows,
                     reinterpret_cast<unsigned*>(a.Ys), (long long)a.n_layers * rows,
                     reinterpret_cast<unsigned*>(a.o), (long long)a.n_layers * rows * (bf16 ? 2 : 4) / 4,
                     reinterpret_cast<unsigned*>(a.patt), a.n_layers * a.M * a.nh, a.att_pmax, a.att_npf, a.hd + 4, v, a.fin,
                     a.n_fin, a.S, a.err);
  const size_t smem = mega_smem_bytes(bf16, a.M, a.d);
  void* args[] = {(void*)&a};
  return hipLaunchCooperativeKernel(pick(bf16, a.M, loop_block), dim3(G), dim3(MEGA_THREADS), args,
                                    (unsigned)smem, s);
}

}  // namespace ls
