// C ABI of libloopspec: argument validation, workspace carving and kernel orchestration for
// ls_prelude / ls_loop_step / ls_readout / ls_verify (see include/loopspec.h).
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <mutex>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/loopspec.h"
#include "kernels.h"

using namespace ls;

namespace {

thread_local char g_err[512] = "";
std::atomic<unsigned long long> g_model_ids{0};   // ids of created models

ls_status fail(ls_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// Device buffers of one workspace (a caller's, bound by ls_bind_workspace, or the library's
// static scratch for ls_loop_step_static): plain pointers into it.
struct Workspace {
  char* base = nullptr;
  int max_rows = 0, max_keys = 0, max_jobs = 0;
  int* err = nullptr;
  int32_t *slot_ok = nullptr, *dep_ok = nullptr, *row_ok = nullptr;
  float *q = nullptr, *hc = nullptr, *logits = nullptr;
  // persistent-kernel buffers: per-layer activations, rotary tables, attention partials,
  // per-tile sums of squares, dependency counters
  float *Xs = nullptr, *Ys = nullptr;
  void *o = nullptr, *act = nullptr;
  double* invf = nullptr;
  float* rope = nullptr;
  float *patt = nullptr, *ssq = nullptr, *spart = nullptr;
  int att_pmax = 0;                 // attention partials per (row, head) in patt
  int* cnt = nullptr;
  LayerW *tab_pre = nullptr, *tab_core = nullptr, *tab_coda = nullptr;
};

struct ls_model {
  ls_model_desc d;
  unsigned long long id = 0;        // unique per created model
  const void* emb = nullptr;
  const float* g_final = nullptr;
  std::vector<ls_layer_ptrs> pre, core, coda;
  std::vector<LayerW> host_tab;     // device layer table contents (prelude, core, coda)
  std::vector<double> host_invf;    // rotary frequencies theta^(-2i/hd)
  Workspace w;                      // the bound workspace
  int n_cu = 0;
  // resident workgroups per CU of the persistent kernel, by [loop-block symbol][long-prefix
  // attention][rows per launch] (each variant is a separately compiled kernel)
  int occ[2][LS_MAX_ROWS + 1] = {};
  long long clock_khz = 100000;     // wall-clock rate of the device
  double wait_seconds = 2.0;        // bound on every dependency wait inside a launch
  long long* trace = nullptr;   // optional phase timestamps of the next ls_loop_step
  int last_grid = 0;
  bool bf16() const { return d.dtype == LS_BF16; }
  size_t esz() const { return bf16() ? 2 : 4; }
  size_t entry() const { return (size_t)2 * d.d * esz(); }   // bytes of one KV entry
};

namespace {

struct Carve {
  int max_rows, max_keys, max_jobs, att_pmax;
  size_t off_err, off_slot, off_dep, off_row, off_q, off_o, off_act, off_hc, off_logits;
  size_t off_Xs, off_Ys, off_invf, off_rope, off_patt, off_ssq, off_spart, off_cnt, off_tab, total;
};

// Elements of one layer's slice of a per-layer activation buffer: rows x width, rounded up so
// that slices of different layers never share a 256-byte span (and hence a cache line).
size_t layer_slice(size_t rows, size_t width) { return (rows * width + 127) / 128 * 128; }

Carve carve(const ls_model* m, int max_rows, int max_keys, int max_jobs) {
  Carve c{};
  c.max_rows = max_rows;
  c.max_keys = max_keys;
  c.max_jobs = max_jobs;
  const ls_model_desc& d = m->d;
  const size_t R = (size_t)max_rows;
  const size_t es = d.dtype == LS_BF16 ? 2 : 4;
  const size_t nl = (size_t)std::max(d.L, std::max(d.L_pre, d.L_coda));   // most layers in one launch
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  c.off_err = take(256);
  c.off_slot = take(R * 4);
  c.off_dep = take(R * 4);
  c.off_row = take(R * 4);
  c.off_q = take(R * d.d * 4);
  c.off_hc = take(R * d.d * 4);
  c.off_logits = take(R * (size_t)d.V * 4);
  // per-layer activations of one launch (each written once per launch)
  c.off_Xs = take((nl + 1) * layer_slice(R, d.d) * 4);
  c.off_Ys = take(nl * layer_slice(R, d.d) * 4);
  c.off_o = take(nl * layer_slice(R, d.d) * es);
  c.off_act = take(nl * layer_slice(R, d.F) * es);
  c.off_invf = take((size_t)d.head_dim / 2 * 8);
  c.off_rope = take(R * (size_t)d.head_dim * 4);
  c.att_pmax = att_pmax_for(max_keys, d.n_heads, d.head_dim, (int)es);
  c.off_patt = take(nl * R * d.n_heads * (size_t)c.att_pmax * (d.head_dim + 4) * 4);   // per layer: the records are polled
  c.off_ssq = take(nl * 2 * (d.d / 16) * R * 4);
  c.off_spart = take((size_t)MEGA_MAX_GRID * 2 * R * 16 * 4);
  c.off_cnt = take(mega_counter_ints(max_rows, d.d, d.F, d.n_heads, (int)nl) * 4);
  c.off_tab = take((size_t)(d.L + d.L_pre + d.L_coda) * sizeof(LayerW));
  c.total = off;
  return c;
}

// Pointers of a workspace laid out by `c` from `b`.
Workspace carve_into(const Carve& c, char* b) {
  Workspace w;
  w.base = b;
  w.max_rows = c.max_rows; w.max_keys = c.max_keys; w.max_jobs = c.max_jobs;
  w.err = (int*)(b + c.off_err);
  w.slot_ok = (int32_t*)(b + c.off_slot);
  w.dep_ok = (int32_t*)(b + c.off_dep);
  w.row_ok = (int32_t*)(b + c.off_row);
  w.q = (float*)(b + c.off_q);
  w.hc = (float*)(b + c.off_hc);
  w.logits = (float*)(b + c.off_logits);
  w.Xs = (float*)(b + c.off_Xs);
  w.Ys = (float*)(b + c.off_Ys);
  w.o = b + c.off_o;
  w.act = b + c.off_act;
  w.invf = (double*)(b + c.off_invf);
  w.rope = (float*)(b + c.off_rope);
  w.patt = (float*)(b + c.off_patt);
  w.att_pmax = c.att_pmax;
  w.ssq = (float*)(b + c.off_ssq);
  w.spart = (float*)(b + c.off_spart);
  w.cnt = (int*)(b + c.off_cnt);
  return w;
}

ls_status check_hip(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(LS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return LS_OK;
}

// The model's layer table (into w.tab_*) and rotary frequencies (w.invf) go to the device
// (stream-ordered copies from the host vectors built at model creation).
ls_status upload_tables(ls_model* m, Workspace& w, hipStream_t stream, const char* who);

// Where the layer table and the rotary frequencies live in workspace w.
void set_tables(const ls_model* m, Workspace& w, LayerW* tab, double* invf) {
  w.tab_pre = tab;
  w.tab_core = tab + m->pre.size();
  w.tab_coda = tab + m->pre.size() + m->core.size();
  w.invf = invf;
}

// Device attributes the launches need (multiprocessor count, wall-clock rate), once per bind.
ls_status device_setup(ls_model* m) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&m->n_cu, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess || m->n_cu <= 0)
    return fail(LS_ERR_HIP, "no usable current device");
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess && khz > 0) m->clock_khz = khz;
  for (auto& x : m->occ)
    for (int& o : x) o = 0;
  return LS_OK;
}

ls_status check_rows(const ls_model* m, const ls_rows* r, const char* who) {
  if (!m || !r) return fail(LS_ERR_INVALID, "%s: null model or rows", who);
  if (!m->w.base) return fail(LS_ERR_INVALID, "%s: no workspace bound", who);
  if (r->n < 0 || r->n_fin < 0 || r->max_anc < 0) return fail(LS_ERR_INVALID, "%s: negative sizes", who);
  if (r->n > m->w.max_rows) return fail(LS_ERR_CAPACITY, "%s: %d rows > workspace max_rows %d", who, r->n, m->w.max_rows);
  if ((long long)r->n_fin + r->max_anc + 1 > m->w.max_keys)
    return fail(LS_ERR_CAPACITY, "%s: n_fin + max_anc + 1 = %lld > workspace max_keys %d", who,
                (long long)r->n_fin + r->max_anc + 1, m->w.max_keys);
  if (r->n > 0 && (!r->slot || !r->pos || !r->anc_off)) return fail(LS_ERR_INVALID, "%s: null row array", who);
  if (r->n_fin > 0 && !r->fin_slots) return fail(LS_ERR_INVALID, "%s: null fin_slots", who);
  if (r->max_anc > 0 && !r->anc_slots) return fail(LS_ERR_INVALID, "%s: null anc_slots", who);
  return LS_OK;
}

ls_status upload_tables(ls_model* m, Workspace& w, hipStream_t stream, const char* who) {
  hipError_t e = hipMemcpyAsync(w.invf, m->host_invf.data(), m->host_invf.size() * sizeof(double),
                                hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return fail(LS_ERR_HIP, "%s: rotary table upload: %s", who, hipGetErrorString(e));
  if (!m->host_tab.empty()) {
    e = hipMemcpyAsync(w.tab_pre, m->host_tab.data(), m->host_tab.size() * sizeof(LayerW), hipMemcpyHostToDevice,
                       stream);
    if (e != hipSuccess) return fail(LS_ERR_HIP, "%s: layer table upload: %s", who, hipGetErrorString(e));
  }
  return LS_OK;
}

}  // namespace

extern "C" {

const char* ls_last_error(void) { return g_err; }

ls_status ls_model_create(const ls_model_desc* desc, const ls_weight_ptrs* w, ls_model** out) {
  if (!desc || !w || !out) return fail(LS_ERR_INVALID, "ls_model_create: null argument");
  const ls_model_desc& d = *desc;
  if (d.V <= 0 || d.d <= 0 || d.n_heads <= 0 || d.head_dim <= 0 || d.F <= 0 || d.L <= 0 || d.R <= 0 ||
      d.L_pre < 0 || d.L_coda < 0 || d.slot_capacity <= 0)
    return fail(LS_ERR_INVALID, "ls_model_create: non-positive shape");
  if (d.n_heads * d.head_dim != d.d) return fail(LS_ERR_INVALID, "ls_model_create: n_heads * head_dim != d");
  if (d.dtype != LS_F32 && d.dtype != LS_BF16) return fail(LS_ERR_INVALID, "ls_model_create: bad dtype");
  if (d.head_dim % 16 || d.head_dim > 128) return fail(LS_ERR_UNSUPPORTED, "head_dim must be a multiple of 16, <= 128");
  if (d.V > 65536) return fail(LS_ERR_UNSUPPORTED, "V must be <= 65536 (the readout keeps a row in one workgroup's registers)");
  const int kmul = d.dtype == LS_BF16 ? 32 : 16;
  if (d.d % kmul || d.F % kmul) return fail(LS_ERR_UNSUPPORTED, "d and F must be multiples of %d", kmul);
  if (d.n_readout < 1 || d.n_readout > LS_MAX_READOUT_DEPTHS) return fail(LS_ERR_INVALID, "bad n_readout");
  for (int i = 0; i < d.n_readout; ++i) {
    if (d.readout_depths[i] < 1 || d.readout_depths[i] > d.R || (i && d.readout_depths[i] <= d.readout_depths[i - 1]))
      return fail(LS_ERR_INVALID, "readout depths must be ascending within [1, R]");
  }
  if (d.readout_depths[d.n_readout - 1] != d.R) return fail(LS_ERR_INVALID, "last readout depth must be R");
  if (!w->emb || !w->g_final || (d.L && !w->core) || (d.L_pre && !w->pre) || (d.L_coda && !w->coda))
    return fail(LS_ERR_INVALID, "ls_model_create: null weight pointer");
  auto check_layers = [&](const ls_layer_ptrs* p, int n) {
    for (int i = 0; i < n; ++i)
      if (!p[i].Wq || !p[i].Wk || !p[i].Wv || !p[i].Wo || !p[i].Wg || !p[i].Wu || !p[i].Wd || !p[i].g1 || !p[i].g2)
        return false;
    return true;
  };
  if (!check_layers(w->core, d.L) || !check_layers(w->pre, d.L_pre) || !check_layers(w->coda, d.L_coda))
    return fail(LS_ERR_INVALID, "ls_model_create: null layer weight");
  ls_model* m = new ls_model();
  m->d = d;
  m->id = ++g_model_ids;
  m->emb = w->emb;
  m->g_final = w->g_final;
  m->core.assign(w->core, w->core + d.L);
  if (d.L_pre) m->pre.assign(w->pre, w->pre + d.L_pre);
  if (d.L_coda) m->coda.assign(w->coda, w->coda + d.L_coda);
  auto add = [&](const std::vector<ls_layer_ptrs>& v) {
    for (const auto& p : v) m->host_tab.push_back(LayerW{p.Wq, p.Wk, p.Wv, p.Wo, p.Wg, p.Wu, p.Wd, p.g1, p.g2});
  };
  add(m->pre); add(m->core); add(m->coda);
  m->host_invf.resize(d.head_dim / 2);
  for (int i = 0; i < d.head_dim / 2; ++i)
    m->host_invf[i] = std::pow((double)d.rope_theta, -2.0 * (double)i / (double)d.head_dim);
  *out = m;
  return LS_OK;
}

void ls_model_destroy(ls_model* m) { delete m; }

size_t ls_workspace_bytes(const ls_model* m, int max_rows, int max_keys, int max_jobs) {
  if (!m || max_rows <= 0 || max_keys <= 0 || max_jobs < 0) return 0;
  return carve(m, max_rows, max_keys, max_jobs).total;
}

ls_status ls_bind_workspace(ls_model* m, void* ws, int max_rows, int max_keys, int max_jobs, hipStream_t stream) {
  if (!m || !ws) return fail(LS_ERR_INVALID, "ls_bind_workspace: null argument");
  if (max_rows <= 0 || max_rows > LS_MAX_ROWS || max_keys <= 0 || max_jobs < 0)
    return fail(LS_ERR_INVALID, "ls_bind_workspace: bad capacities (rows 1..%d)", LS_MAX_ROWS);
  if ((uintptr_t)ws % 256) return fail(LS_ERR_INVALID, "ls_bind_workspace: workspace not 256-byte aligned");
  const Carve c = carve(m, max_rows, max_keys, max_jobs);
  char* b = (char*)ws;
  m->w = carve_into(c, b);
  set_tables(m, m->w, (LayerW*)(b + c.off_tab), (double*)(b + c.off_invf));
  ls_status st = upload_tables(m, m->w, stream, "ls_bind_workspace");
  if (st) return st;
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(LS_ERR_HIP, "ls_bind_workspace: %s", hipGetErrorString(e));
  st = device_setup(m);
  if (st) return st;
  launch_fill_i32(m->w.err, 1, 0, stream);
  return check_hip("ls_bind_workspace");
}

}  // extern "C"

namespace {

#ifndef LS_HEAD_KERNEL
#define LS_HEAD_KERNEL 1
#endif

// The row check of a call over `r` (depth range dep_lo..dep_hi; dep NULL: no depths).
ValidateArgs validate_args(ls_model* m, const ls_rows* r, const int32_t* dep, int dep_lo, int dep_hi) {
  ValidateArgs v;
  v.n = r->n; v.slot = r->slot; v.dep = dep; v.pos = r->pos; v.anc_off = r->anc_off;
  v.dep_lo = dep_lo; v.dep_hi = dep_hi; v.n_fin = r->n_fin; v.max_anc = r->max_anc; v.S = m->d.slot_capacity;
  v.slot_ok = m->w.slot_ok; v.dep_ok = m->w.dep_ok; v.row_ok = m->w.row_ok; v.err = m->w.err;
  return v;
}

// One launch of the persistent layer kernel over rows [i0, i0 + mc) of `r`; its prep kernel
// runs the row check `v` first (the call's first launch; later launches pass an empty one).
ls_status run_mega(ls_model* m, const ls_rows* r, int i0, int mc, float* H, const int32_t* hidx, const LayerW* tab,
                   int n_layers, void* kv, const int32_t* dep, int dep_off, int blk_mul, int init_mode,
                   const int32_t* tokens, const int32_t* gather, const float* Hg, float* logits, hipStream_t s,
                   const ValidateArgs& v, bool loop_block = false) {
  const ls_model_desc& d = m->d;
  MegaArgs a{};
  a.M = mc; a.d = d.d; a.F = d.F; a.hd = d.head_dim; a.nh = d.n_heads; a.V = d.V;
  a.theta = d.rope_theta; a.eps = d.norm_eps;
  a.layers = tab; a.n_layers = n_layers;
  a.g_final = m->g_final; a.emb = m->emb;
  a.H = H; a.hidx = hidx ? hidx + i0 : nullptr; a.Xs = m->w.Xs; a.Ys = m->w.Ys;
  a.slot = m->w.slot_ok + i0; a.pos = r->pos + i0; a.dep = dep ? dep + i0 : nullptr;
  a.fin = r->fin_slots; a.anc_off = r->anc_off + i0; a.anc = r->anc_slots;
  a.tokens = tokens ? tokens + i0 : nullptr;
  a.n_fin = r->n_fin;
  a.kv = kv; a.dep_off = dep_off; a.blk_mul = blk_mul; a.layer0 = 0; a.S = d.slot_capacity;
  a.q = m->w.q; a.o = m->w.o; a.act = m->w.act;
  a.logits = logits; a.ldo = d.V;
  a.inv_freq = m->w.invf;
  a.rope = m->w.rope;
  a.patt = m->w.patt; a.ssq = m->w.ssq; a.spart = m->w.spart;
  a.cnt = m->w.cnt; a.err = m->w.err;
  a.init_mode = init_mode; a.gather = gather ? gather + i0 : nullptr; a.Hg = Hg;
  a.do_head = logits != nullptr;
  // resident workgroups per CU of the kernel variant that is launched (cached per variant)
  int& occ = m->occ[loop_block ? 1 : 0][mc];
  if (!occ) occ = std::min(mega_occupancy(m->bf16(), mc, d.d, loop_block), 4);
  if (occ <= 0) return fail(LS_ERR_HIP, "persistent kernel: no resident workgroup fits (M=%d)", mc);
  const int G = occ * m->n_cu;
  // attention partials per (row, head): at most the workgroups one segment's tiles span
  {
    const int esz = m->bf16() ? 2 : 4;
    const int hb = att_heads_per_block(d.n_heads, d.head_dim, esz);
    const int n_hb = (d.n_heads + hb - 1) / hb;
    const int n_kt = std::max(1, (r->n_fin + 7) / 8);
    const int need = std::min(n_kt, (G + n_hb - 1) / n_hb + 1);
    if (G > MEGA_MAX_GRID || need > m->w.att_pmax)
      return fail(LS_ERR_UNSUPPORTED, "persistent kernel: %d workgroups need %d attention partials, workspace holds %d",
                  G, need, m->w.att_pmax);
    // partials of the launch's segments (one row per virtual group): the workgroups that hold
    // tiles of a segment, by the same contiguous deal as the kernel's
    const long long N = (long long)mc * n_hb * n_kt, Ga = att_workgroups(G, (int)N);
    auto owner = [&](long long t) { return ((t + 1) * Ga - 1) / N; };
    int npf = 1;
    for (long long sg = 0; sg < (long long)mc * n_hb; ++sg)
      npf = std::max(npf, (int)(owner(sg * n_kt + n_kt - 1) - owner(sg * n_kt) + 1));
    if (npf > m->w.att_pmax)
      return fail(LS_ERR_UNSUPPORTED, "persistent kernel: %d attention partials per head, workspace holds %d", npf,
                  m->w.att_pmax);
    a.att_npf = npf;
  }
  a.att_pmax = m->w.att_pmax;
  a.wait_ticks = (long long)(m->wait_seconds * 1e3 * (double)m->clock_khz);
  a.trace = m->trace;
  m->last_grid = G;
  hipError_t e = launch_mega(m->bf16(), a, G, s, loop_block, v);
  if (e != hipSuccess) return fail(LS_ERR_HIP, "persistent kernel launch: %s", hipGetErrorString(e));
  return LS_OK;
}

}  // namespace

extern "C" {

ls_status ls_prelude(ls_model* m, const ls_rows* r, const int32_t* tokens, float* H, const ls_kv* kv, hipStream_t s) {
  ls_status st = check_rows(m, r, "ls_prelude");
  if (st) return st;
  if (!H || !kv || (r->n && !tokens)) return fail(LS_ERR_INVALID, "ls_prelude: null argument");
  if (m->d.L_pre && !kv->pre) return fail(LS_ERR_INVALID, "ls_prelude: prelude layers need kv->pre");
  if (r->n == 0) return LS_OK;
  const ls_model_desc& d = m->d;
  if (!d.L_pre) {                                    // embedding rows only: one small kernel
    hipError_t e = launch_embed(m->bf16(), validate_args(m, r, nullptr, 0, 0), tokens, m->emb, d.V, d.d, H, s);
    if (e != hipSuccess) return fail(LS_ERR_HIP, "ls_prelude: embedding launch: %s", hipGetErrorString(e));
    return LS_OK;
  }
  st = run_mega(m, r, 0, r->n, H, m->w.slot_ok, m->w.tab_pre, d.L_pre, kv->pre, nullptr, 0, 0, 1, tokens, nullptr, nullptr,
                nullptr, s, validate_args(m, r, nullptr, 0, 0));
  if (st) return st;
  return check_hip("ls_prelude");
}

ls_status ls_loop_step(ls_model* m, const ls_rows* r, float* H, const ls_kv* kv, hipStream_t s) {
  ls_status st = check_rows(m, r, "ls_loop_step");
  if (st) return st;
  if (!H || !kv || !kv->core) return fail(LS_ERR_INVALID, "ls_loop_step: null argument");
  if (r->n && !r->depth) return fail(LS_ERR_INVALID, "ls_loop_step: null depth");
  if (r->n == 0) return LS_OK;
  const ls_model_desc& d = m->d;
  st = run_mega(m, r, 0, r->n, H, m->w.slot_ok, m->w.tab_core, d.L, kv->core, m->w.dep_ok, -1, d.L, 0, nullptr, nullptr,
                nullptr, nullptr, s, validate_args(m, r, r->depth, 1, d.R), true);
  if (st) return st;
  return check_hip("ls_loop_step");
}

}  // extern "C"

// ---- the loop step without a caller workspace -----------------------------------------------
// The device memory of ls_loop_step_static is this file-scope array: one copy per GPU, held
// until the process ends.  It starts with a header (error word, rotary frequencies, layer
// table) followed by the loop step's buffers laid out as in a workspace.  Host code never uses
// the array's name as an address: each device's address comes from hipGetSymbolAddress at the
// first call on that device, with that device current.
static __device__ __align__(256) char scratch[LS_STATIC_SCRATCH_BYTES];

namespace {

constexpr size_t STATIC_INVF = 256, STATIC_TAB = 1280, STATIC_HDR = 72 * 1024;
constexpr int MAX_DEVICES = 64;
struct StaticScratch {
  char* ptr = nullptr;          // device address of `scratch` on this device
  unsigned long long owner = 0; // model whose tables the header holds
};
StaticScratch g_static[MAX_DEVICES];
std::mutex g_static_mu;

}  // namespace

extern "C" {

ls_status ls_loop_step_static(ls_model* m, const ls_rows* r, float* H, const ls_kv* kv, int* err_out, hipStream_t s) {
  if (!m || !r || !H || !kv || !kv->core) return fail(LS_ERR_INVALID, "ls_loop_step_static: null argument");
  if (r->n < 0 || r->n_fin < 0 || r->max_anc < 0) return fail(LS_ERR_INVALID, "ls_loop_step_static: negative sizes");
  if (r->n > LS_MAX_ROWS) return fail(LS_ERR_CAPACITY, "ls_loop_step_static: %d rows > %d", r->n, LS_MAX_ROWS);
  if (r->n > 0 && (!r->slot || !r->pos || !r->anc_off || !r->depth))
    return fail(LS_ERR_INVALID, "ls_loop_step_static: null row array");
  if (r->n_fin > 0 && !r->fin_slots) return fail(LS_ERR_INVALID, "ls_loop_step_static: null fin_slots");
  if (r->max_anc > 0 && !r->anc_slots) return fail(LS_ERR_INVALID, "ls_loop_step_static: null anc_slots");
  if (r->n == 0) return LS_OK;
  const long long keys = (long long)r->n_fin + r->max_anc + 1;
  if (keys > (1LL << 30)) return fail(LS_ERR_CAPACITY, "ls_loop_step_static: %lld keys", keys);
  const Carve c = carve(m, r->n, (int)keys, 0);
  if (STATIC_HDR + c.total > (size_t)LS_STATIC_SCRATCH_BYTES)
    return fail(LS_ERR_CAPACITY, "ls_loop_step_static: %d rows with %lld keys need %zu bytes of scratch, the static "
                "scratch holds %zu", r->n, keys, STATIC_HDR + c.total, (size_t)LS_STATIC_SCRATCH_BYTES);
  if (STATIC_TAB + m->host_tab.size() * sizeof(LayerW) > STATIC_HDR || m->host_invf.size() * sizeof(double) > STATIC_TAB - STATIC_INVF)
    return fail(LS_ERR_UNSUPPORTED, "ls_loop_step_static: too many layers for the scratch header");
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES)
    return fail(LS_ERR_HIP, "ls_loop_step_static: no usable current device");
  std::lock_guard<std::mutex> lock(g_static_mu);
  StaticScratch& ss = g_static[dev];
  if (!ss.ptr) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(LS_ERR_HIP, "ls_loop_step_static: scratch address: %s", hipGetErrorString(e));
    ss.ptr = (char*)p;
  }
  if (!m->n_cu) {
    ls_status st = device_setup(m);
    if (st) return st;
  }
  Workspace w = carve_into(c, ss.ptr + STATIC_HDR);
  set_tables(m, w, (LayerW*)(ss.ptr + STATIC_TAB), (double*)(ss.ptr + STATIC_INVF));
  w.err = err_out ? err_out : (int*)ss.ptr;
  if (ss.owner != m->id) {
    ls_status st = upload_tables(m, w, s, "ls_loop_step_static");
    if (st) return st;
    ss.owner = m->id;
  }
  if (!err_out) launch_fill_i32(w.err, 1, 0, s);
  const Workspace saved = m->w;
  m->w = w;
  const ls_model_desc& d = m->d;
  ls_status st = run_mega(m, r, 0, r->n, H, m->w.slot_ok, m->w.tab_core, d.L, kv->core, m->w.dep_ok, -1, d.L, 0, nullptr,
                          nullptr, nullptr, nullptr, s, validate_args(m, r, r->depth, 1, d.R), true);
  m->w = saved;
  if (st) return st;
  return check_hip("ls_loop_step_static");
}

ls_status ls_readout(ls_model* m, const ls_rows* r, const float* H, const ls_sampling* smp, float* probs,
                     const int32_t* out_rows, int n_prob_rows, int32_t* argmax, float* logits, const ls_kv* kv,
                     hipStream_t s) {
  ls_status st = check_rows(m, r, "ls_readout");
  if (st) return st;
  if (!H || !smp || !probs || !kv) return fail(LS_ERR_INVALID, "ls_readout: null argument");
  if (r->n && !r->depth) return fail(LS_ERR_INVALID, "ls_readout: null depth");
  if (!smp->greedy && !(smp->temperature > 0.f)) return fail(LS_ERR_INVALID, "ls_readout: temperature must be > 0");
  if (!smp->greedy && !(smp->top_p > 0.f)) return fail(LS_ERR_INVALID, "ls_readout: top_p must be > 0");
  if (m->d.L_coda && !kv->coda) return fail(LS_ERR_INVALID, "ls_readout: coda layers need kv->coda");
  if (!out_rows && n_prob_rows < r->n) return fail(LS_ERR_INVALID, "ls_readout: n_prob_rows < rows");
  if (r->n == 0) return LS_OK;
  const ls_model_desc& d = m->d;
  float* lg = logits ? logits : m->w.logits;
  const ValidateArgs v = validate_args(m, r, r->depth, 0, d.n_readout - 1), none{};
  if (!d.L_coda && m->bf16() && d.d % 256 == 0 && LS_HEAD_KERNEL) {
    // no coda layers: the streaming head kernel per 16 rows, which checks its rows itself
    for (int i0 = 0; i0 < r->n; i0 += 16) {
      const int mc = std::min(16, r->n - i0);
      launch_head(H, v, i0, mc, d.d, d.V, m->emb, m->g_final, d.norm_eps, lg + (size_t)i0 * d.V, d.V, s);
    }
    launch_dist(lg, r->n, d.V, smp->greedy, smp->temperature, smp->top_p, probs, out_rows, n_prob_rows, argmax, m->w.err, s);
    return check_hip("ls_readout");
  }
  for (int i0 = 0; i0 < r->n; i0 += 16) {
    const int mc = std::min(16, r->n - i0);
    if (d.L_coda)
      st = run_mega(m, r, i0, mc, m->w.hc, m->w.row_ok, m->w.tab_coda, d.L_coda, kv->coda, m->w.dep_ok, 0, d.L_coda, 2,
                    nullptr, m->w.slot_ok, H, lg + (size_t)i0 * d.V, s, i0 == 0 ? v : none);
    else
      st = run_mega(m, r, i0, mc, (float*)H, m->w.slot_ok, nullptr, 0, nullptr, nullptr, 0, 0, 0, nullptr, nullptr,
                    nullptr, lg + (size_t)i0 * d.V, s, i0 == 0 ? v : none);
    if (st) return st;
  }
  launch_dist(lg, r->n, d.V, smp->greedy, smp->temperature, smp->top_p, probs, out_rows, n_prob_rows, argmax, m->w.err, s);
  return check_hip("ls_readout");
}

size_t ls_prefill_workspace_bytes(const ls_model* m, int max_n) {
  if (!m || max_n < 0) return 0;
  return prefill_bytes(max_n, m->d.d, m->d.F, m->bf16());
}

ls_status ls_prefill(ls_model* m, const int32_t* tokens, const int32_t* slots, int n, const int32_t* fin_slots, int n_fin,
                     unsigned coda_mask, float* H, const ls_kv* kv, void* pws, size_t pws_bytes, hipStream_t s) {
  if (!m || !m->w.base) return fail(LS_ERR_INVALID, "ls_prefill: null model or no workspace bound");
  if (n < 0 || n_fin < 0) return fail(LS_ERR_INVALID, "ls_prefill: negative sizes");
  if (n == 0) return LS_OK;
  const ls_model_desc& d = m->d;
  if (!tokens || !slots || !H || !kv || !kv->core || !pws || (n_fin && !fin_slots))
    return fail(LS_ERR_INVALID, "ls_prefill: null argument");
  if (d.L_pre && !kv->pre) return fail(LS_ERR_INVALID, "ls_prefill: prelude layers need kv->pre");
  const unsigned mask = coda_mask & ((1u << d.n_readout) - 1u);
  if (d.L_coda && mask && !kv->coda) return fail(LS_ERR_INVALID, "ls_prefill: coda layers need kv->coda");
  if ((long long)n_fin + n > 0x7fffffffLL) return fail(LS_ERR_INVALID, "ls_prefill: positions overflow");
  const size_t need = prefill_bytes(n, d.d, d.F, m->bf16());
  if (pws_bytes < need)
    return fail(LS_ERR_CAPACITY, "ls_prefill: %d rows need %zu workspace bytes, %zu given", n, need, pws_bytes);
  if ((uintptr_t)pws % 256) return fail(LS_ERR_INVALID, "ls_prefill: workspace must be 256-byte aligned");
  PrefillArgs a{};
  a.n = n; a.n_fin = n_fin; a.d = d.d; a.F = d.F; a.hd = d.head_dim; a.nh = d.n_heads; a.V = d.V;
  a.L = d.L; a.L_pre = d.L_pre; a.L_coda = d.L_coda; a.R = d.R; a.n_readout = d.n_readout;
  for (int i = 0; i < d.n_readout; ++i) a.readout_depths[i] = d.readout_depths[i];
  a.coda_mask = mask;
  a.eps = d.norm_eps;
  a.S = d.slot_capacity;
  a.tokens = tokens; a.slots = slots; a.fin = fin_slots;
  a.emb = m->emb;
  a.pre = m->host_tab.data();
  a.core = a.pre + m->pre.size();
  a.coda = a.core + m->core.size();
  a.kv_pre = kv->pre; a.kv_core = kv->core; a.kv_coda = kv->coda;
  a.invf = m->w.invf;
  a.H = H;
  a.err = m->w.err;
  a.b = prefill_carve(pws, n, d.d, d.F, m->bf16());
  hipError_t e = launch_prefill(m->bf16(), a, s);
  if (e != hipSuccess) return fail(LS_ERR_HIP, "ls_prefill: launch: %s", hipGetErrorString(e));
  return LS_OK;
}

ls_status ls_verify(ls_model* m, const ls_verify_job* jobs, int n_jobs, const float* probs, int n_prob_rows,
                    int32_t* cands, int n_cands, const uint32_t* uniforms, ls_verify_out* out, hipStream_t s) {
  if (!m || !m->w.base) return fail(LS_ERR_INVALID, "ls_verify: null model or no workspace");
  if (n_jobs < 0 || n_prob_rows < 0) return fail(LS_ERR_INVALID, "ls_verify: negative count");
  if (n_jobs == 0) return LS_OK;
  if (n_jobs > m->w.max_jobs) return fail(LS_ERR_CAPACITY, "ls_verify: %d jobs > workspace max_jobs %d", n_jobs, m->w.max_jobs);
  if (!jobs || !probs || !uniforms || !out) return fail(LS_ERR_INVALID, "ls_verify: null argument");
  if (n_cands < 0 || (n_cands > 0 && !cands)) return fail(LS_ERR_INVALID, "ls_verify: bad candidate array");
  launch_verify(jobs, n_jobs, probs, m->d.V, n_prob_rows, cands, n_cands, uniforms, out, m->w.err, s);
  return check_hip("ls_verify");
}

ls_status ls_sync_status(ls_model* m, hipStream_t s) {
  if (!m || !m->w.err) return fail(LS_ERR_INVALID, "ls_sync_status: no workspace bound");
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(LS_ERR_HIP, "stream: %s", hipGetErrorString(e));
  int h = 0;
  e = hipMemcpy(&h, m->w.err, sizeof(int), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(LS_ERR_HIP, "error word: %s", hipGetErrorString(e));
  if (h == 5) return fail(LS_ERR_HIP, "a device-side dependency wait timed out (error word 5)");
  if (h) return fail((ls_status)h, "a kernel rejected a descriptor (device error word %d)", h);
  return LS_OK;
}

ls_status ls_set_wait_limit(ls_model* m, double seconds) {
  if (!m) return fail(LS_ERR_INVALID, "ls_set_wait_limit: null model");
  if (!(seconds >= 0.0) || seconds > 3600.0) return fail(LS_ERR_INVALID, "ls_set_wait_limit: seconds must be in [0, 3600]");
  m->wait_seconds = seconds;
  return LS_OK;
}

ls_status ls_debug_trace(ls_model* m, long long* dev_buf, int* grid_out) {
  if (!m) return fail(LS_ERR_INVALID, "ls_debug_trace: null model");
  m->trace = dev_buf;
  if (grid_out) *grid_out = m->last_grid;
  return LS_OK;
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of
// (c0,c1,c2,c3) -> (hi(M1*c2)^c1^k0, lo(M1*c2), hi(M0*c0)^c3^k1, lo(M0*c0)), key bumped by the
// Weyl constants between rounds.
void ls_philox_uniforms(uint64_t seed, int64_t pos, const int32_t* purposes, int n, uint32_t* out) {
  for (int i = 0; i < n; ++i) {
    uint32_t c0 = (uint32_t)pos, c1 = (uint32_t)purposes[i], c2 = 0, c3 = 0;
    uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    for (int rnd = 0; rnd < 10; ++rnd) {
      if (rnd) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
      const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
      const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n1 = (uint32_t)p1;
      const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1, n3 = (uint32_t)p0;
      c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[i] = c0;
  }
}

}  // extern "C"
