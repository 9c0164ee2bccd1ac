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
  int att_chunks;               // attention units per (group, head): ceil(n_fin / (att_unit_keys * att_sub)), >= 1
  int att_sub;                  // sub-units of att_unit_keys keys per attention unit, >= 1
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
  int* cnt;
  int* err;
  int init_mode;                // 0 none, 1 embedding rows of tokens, 2 gather Hg[gather[m]]
  const int32_t* gather;
  const float* Hg;
  int do_head;
  long long* trace;             // optional: per-workgroup phase timestamps (wall clock)
};

size_t mega_counter_ints(int M, int d, int F, int nh, int n_layers);
size_t mega_smem_bytes(bool bf16, int M, int d);
int mega_occupancy(bool bf16, int M, int d);
int att_unit_keys(bool bf16);   // prefix keys per attention unit
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
void launch_verify(const void* jobs, int n_jobs, const float* probs, int V, int n_rows, const int32_t* cands, int n_cands,
                   const uint32_t* uniforms, void* out, int* err, hipStream_t s);

}  // namespace ls
