// Internal launchers of the libloopspec kernels (host side; not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ls {

// Weight pointers of one layer (device table entry).
struct LayerW {
  const void *Wq, *Wk, *Wv, *Wo, *Wg, *Wu, *Wd;
  const float *g1, *g2;
};

// Arguments of the persistent layer kernel (mega.hip).
// Row-descriptor check of one call, run by the prep kernel of the call's first launch: rows
// whose slot, depth, ancestor range or position is out of contract get slot -1 in the checked
// copy (every kernel skips such rows) and raise the error word.  dep_lo..dep_hi is the legal
// depth range (dep may be NULL); n == 0 means nothing to check.
struct ValidateArgs {
  int n = 0;
  const int32_t *slot = nullptr, *dep = nullptr, *pos = nullptr, *anc_off = nullptr;
  int dep_lo = 0, dep_hi = 0, n_fin = 0, max_anc = 0;
  long long S = 0;
  int32_t *slot_ok = nullptr, *dep_ok = nullptr, *row_ok = nullptr;
  int* err = nullptr;
};

struct MegaArgs {
  int M, d, F, hd, nh, V;
  float theta, eps;
  const LayerW* layers;         // device table of this call's layers
  int n_layers;
  const float* g_final;
  const void* emb;
  float* H;                     // working hidden rows H[hidx[m]] (stride d)
  const int32_t* hidx;          // NULL: row m; negative: rejected row
  float* Xs;                    // per-layer inputs, layer l > 0 at Xs + l*M*d (see layer_in)
  float* Ys;                    // per-layer attention-residual outputs at Ys + l*M*d
  const int32_t *slot, *pos, *dep, *fin, *anc_off, *anc, *tokens;
  int n_fin;
  int att_pmax;                 // attention partials per (row, head) that patt holds (att_pmax_for)
  int att_npf;                  // partial records per (row, head) this launch fills and its mergers poll
  void* kv;                     // cache tensor; block(i, l) = (dep[i] + dep_off) * blk_mul + layer0 + l
  int dep_off, blk_mul, layer0;
  long long S;
  const double* inv_freq;       // rotary frequencies theta^(-2i/hd), i < hd/2
  float* rope;                  // [M][hd/2][2]: cos, sin of pos[m] * inv_freq[i], filled before the launch
  float* q;
  void *o, *act;                // per-layer attention outputs (l*M*d) and SwiGLU outputs (l*M*F)
  float* logits;
  int ldo;
  float *patt, *ssq;
  float* spart;                 // partial sums of split residual tiles: [workgroup][2][M][16]
  int* cnt;
  int* err;
  int init_mode;                // 0 none, 1 embedding rows of tokens, 2 gather Hg[gather[m]]
  const int32_t* gather;
  const float* Hg;
  int do_head;
  long long* trace;             // optional: per-workgroup phase timestamps (wall clock)
  long long wait_ticks;         // bound on every dependency wait, wall-clock ticks from launch start
};

size_t mega_counter_ints(int M, int d, int F, int nh, int n_layers);
size_t mega_smem_bytes(bool bf16, int M, int d);
// resident workgroups per CU of the variant launch_mega picks for (M, loop_block)
int mega_occupancy(bool bf16, int M, int d, bool loop_block);

// Attention tiles of the layer kernel: 8 prefix keys x a block of heads, the block at most 8
// heads and at most 2048 bytes of one key's K piece (so a tile is at most 4 ring slabs).
__host__ __device__ inline int att_heads_per_block(int nh, int hd, int esz) {
  int h = 2048 / (hd * esz);
  h = h < 1 ? 1 : (h > 8 ? 8 : h);
  return h < nh ? h : nh;
}
// Workgroups of a G-workgroup launch that take the N attention tiles of a layer: each takes at
// least LS_ATT_TMIN tiles (a segment's partials are merged by one workgroup, a memory round trip
// per 16 of them, so spreading few tiles over many workgroups lengthens the merge).
#ifndef LS_ATT_TMIN
#define LS_ATT_TMIN 3
#endif
__host__ __device__ inline int att_workgroups(int G, int N) {
  int g = N / LS_ATT_TMIN;
  g = g < 1 ? 1 : g;
  return g < G ? g : G;
}
// Most workgroups a launch of the layer kernel uses (4 per CU on 256 CUs).
constexpr int MEGA_MAX_GRID = 1024;
// Partials per (row, head) that a workspace for keys up to max_keys holds: the workgroups that
// share one segment (one head block of one row group) of the contiguous tile deal, at most
// ceil(G / n_hb) + 1, and never more than the segment's 8-key tiles.
inline int att_pmax_for(int max_keys, int nh, int hd, int esz) {
  const int n_hb = (nh + att_heads_per_block(nh, hd, esz) - 1) / att_heads_per_block(nh, hd, esz);
  const int kt = max_keys > 8 ? (max_keys + 7) / 8 : 1;
  const int g = (MEGA_MAX_GRID + n_hb - 1) / n_hb + 1;
  return kt < g ? kt : g;
}
// loop_block: launch under the k_mega symbol (shared block B) rather than k_mega_aux
hipError_t launch_mega(bool bf16, const MegaArgs& a, int G, hipStream_t s, bool loop_block, const ValidateArgs& v);

void launch_fill_i32(int32_t* p, int n, int v, hipStream_t s);
// LM head without coda layers (bf16 models): logits of rows i0 .. i0+M-1 (1 <= M <= 16) of the
// call, H at their checked slots, d a multiple of 256; the kernel runs the row check itself.
void launch_head(const float* H, const ValidateArgs& v, int i0, int M, int d, int V, const void* emb, const float* g,
                 float eps, float* logits, int ldo, hipStream_t s);
// P without prelude layers: row check and embedding gather into H[slot] (one kernel).
hipError_t launch_embed(bool bf16, const ValidateArgs& v, const int32_t* tokens, const void* emb, int V, int d, float* H,
                        hipStream_t s);
void launch_dist(const float* logits, int M, int V, int greedy, float T, float top_p, float* probs,
                 const int32_t* out_rows, int n_prob_rows, int32_t* argmax, int* err, hipStream_t s);
void launch_verify(const void* jobs, int n_jobs, const float* probs, int V, int n_rows, int32_t* cands, int n_cands,
                   const uint32_t* uniforms, void* out, int* err, hipStream_t s);

// Prefill of a chunk of prompt positions (prefill.hip): buffers carved from the caller's
// prefill workspace, n rows each.
struct PrefillBufs {
  float *X = nullptr, *Xc = nullptr;   // residual stream of the chunk and its coda copy [n][d]
  void* A = nullptr;                   // normalised rows [n][d] (model dtype)
  float* QKV = nullptr;                // q | k | v [n][3d]; q rotated in place
  void *O = nullptr, *ACT = nullptr;   // attention outputs [n][d], SwiGLU outputs [n][F]
};
struct PrefillArgs {
  int n, n_fin, d, F, hd, nh, V, L, L_pre, L_coda, R, n_readout;
  int readout_depths[8];
  unsigned coda_mask;                  // bit j: fill the coda caches of readout depth index j
  float eps;
  long long S;
  const int32_t *tokens, *slots, *fin;
  const void* emb;
  const LayerW *pre, *core, *coda;     // host arrays of device weight pointers
  void *kv_pre, *kv_core, *kv_coda;
  const double* invf;                  // device rotary frequencies
  float* H;
  int* err;
  PrefillBufs b;
};
size_t prefill_bytes(int n, int d, int F, bool bf16);
PrefillBufs prefill_carve(void* base, int n, int d, int F, bool bf16);
hipError_t launch_prefill(bool bf16, const PrefillArgs& a, hipStream_t s);

}  // namespace ls
