// Internal launchers of the libloopspec kernels (host side; not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ls {

enum Epilogue { EP_STORE = 0, EP_RESID = 1, EP_SWIGLU = 2, EP_QKV = 3 };

// Which rows of which KV block a kernel touches: block(i) = (dep ? dep[i] + dep_off : 0) * blk_mul + layer.
struct KvSel {
  void* base;               // first entry of the cache tensor
  const int32_t* dep;       // per-row depth or readout index (NULL: 0)
  int dep_off, blk_mul, layer;
  long long S;              // slots per block
};

struct GemmArgs {
  const void *W0, *W1, *W2;   // plain: W0; SwiGLU: gate W0, up W1; QKV: Wq W0, Wk W1, Wv W2
  int N, K;                   // output features (plain / per matrix for QKV), reduction dim
  const void* X;              // operand rows [M][K], model dtype
  int M;
  float* out; int ldo;        // EP_STORE
  float* H; const int32_t* hidx; int ldh;   // EP_RESID: H[(hidx ? hidx[m] : m) * ldh + n]
  void* act; int F;           // EP_SWIGLU: act[m * F + j]
  float* q; KvSel kv; const int32_t* slot; const int32_t* pos;  // EP_QKV
  int d, hd; float theta;
  int* err;
};

struct AttnArgs {
  const float* q;             // [M][d] fp32 after RoPE
  KvSel kv;
  const int32_t *slot, *pos, *fin, *anc_off, *anc;
  int n_fin, M, d, n_heads, hd;
  float* part;                // [M][n_heads][max_chunks][hd + 2]
  int max_chunks;             // chunk stride of `part`
  int grid_chunks;            // chunks launched: ceil((n_fin + max_anc + 1) / ATTN_CHUNK)
  void* o;                    // [M][d] model dtype
  int* err;
};

constexpr int ATTN_CHUNK = 256;

struct LayerW {
  const void *Wq, *Wk, *Wv, *Wo, *Wg, *Wu, *Wd;
  const float *g1, *g2;
};

// Arguments of the persistent layer kernel (mega.hip).
struct MegaArgs {
  int M, d, F, hd, nh, V;
  int KU;                       // reduction columns per weight unit
  float theta, eps;
  const LayerW* layers;         // device table of this call's layers
  int n_layers;
  const float* g_final;
  const void* emb;
  float* H;                     // working hidden rows H[hidx[m]] (stride d)
  const int32_t* hidx;          // NULL: row m; negative: rejected row
  float* Hb;                    // [M][d] second residual buffer
  const int32_t *slot, *pos, *dep, *fin, *anc_off, *anc, *tokens;
  int n_fin;
  int att_chunks;               // 64-key chunks per (row, head)
  void* kv;                     // cache tensor; block(i, l) = (dep[i] + dep_off) * blk_mul + layer0 + l
  int dep_off, blk_mul, layer0;
  long long S;
  const double* inv_freq;       // rotary frequencies theta^(-2i/hd), i < hd/2
  float* q;
  void *o, *act;
  float* logits;
  int ldo;
  float *pq, *po, *pgu, *pdown, *phead, *patt, *ssq;
  int* cnt;
  int* err;
  int init_mode;                // 0 none, 1 embedding rows of tokens, 2 gather Hg[gather[m]]
  const int32_t* gather;
  const float* Hg;
  int do_head;
  long long* trace;             // optional: per-workgroup phase timestamps (wall clock)
};

size_t mega_counter_ints(int M, int d, int F, int nh, int V, int KU, int n_layers);
size_t mega_smem_bytes(bool bf16, int M, int KU);
int mega_occupancy(bool bf16, int M, int KU);
hipError_t launch_mega(bool bf16, const MegaArgs& a, int G, hipStream_t s);

void launch_gemm(bool bf16, int ep, const GemmArgs& a, hipStream_t s);
void launch_rmsnorm(bool bf16, const float* H, const int32_t* hidx, int ldh, const float* g, int M, int d,
                    float eps, void* X, hipStream_t s);
void launch_attention(bool bf16, const AttnArgs& a, hipStream_t s);
void launch_embed(bool bf16, const void* emb, const int32_t* tokens, const int32_t* slot, int M, int V, int d,
                  long long S, float* H, int* err, hipStream_t s);
void launch_validate(int n, const int32_t* slot, const int32_t* dep, int dep_lo, int dep_hi, const int32_t* pos,
                     const int32_t* anc_off, int n_fin, int max_anc, long long S, int32_t* slot_ok, int32_t* dep_ok,
                     int32_t* row_ok, int* err, hipStream_t s);
void launch_fill_i32(int32_t* p, int n, int v, hipStream_t s);
void launch_gather(const float* H, const int32_t* slot, int M, int d, long long S, float* out, int* err,
                   hipStream_t s);
void launch_dist(const float* logits, int M, int V, int greedy, float T, float top_p, float* probs,
                 const int32_t* out_rows, int n_prob_rows, int32_t* argmax, int* err, hipStream_t s);
void launch_verify(const void* jobs, int n_jobs, const float* probs, int V, int n_rows, const int32_t* cands, int n_cands,
                   const uint32_t* uniforms, void* out, int* err, hipStream_t s);

}  // namespace ls
