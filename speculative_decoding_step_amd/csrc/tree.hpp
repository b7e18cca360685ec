// Device-side state of the draft tree builder and its launch wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace e3 {

constexpr int TREE_CMAX = 1024;  // candidates per sequence: k + (D-1) k^2

struct TreeState {
  int batch, topk, cmax, emax;  // cmax: candidate capacity, emax = (D-1) k expansion rows
  int* tok;                     // [B][cmax] candidate token
  int* par;                     // [B][cmax] parent's creation index, -1 = root
  int* dep;                     // [B][cmax] depth (root's children: 1)
  float* score;                 // [B][cmax] cumulative draft log-prob
  int* erow;                    // [B][cmax] expansion row of the candidate, -1 if not expanded
  int* front;                   // [B][k] frontier (creation indices, rank order)
  uint64_t* emask;              // [B][emax] draft tail mask of each expansion row
};

// Inputs of the draft rows of one expansion (or chain) pass.
struct DraftRows {
  int batch;
  int* tok;        // [rows] token whose embedding forms e
  int* src;        // [rows] where x comes from: >= 0 row of a_rows, -1-b the catch-up row of b
  int* seq;        // RowMeta fields, see kernels.hpp
  int* pos;
  int* slot;
  int* lim;
  int* tail0;
  uint64_t* mask;
};

// The children of one draft tree level, recorded by the slice merge of that level's LM head: rows are the
// level's expansion rows (depth_new == 1: one root row per sequence), their k best ids (through d2t when set)
// and fp32 log-probabilities value - lse become candidates of depth depth_new.
struct TreeKids {
  TreeState ts;
  int depth_new;
  const int* d2t;
  int Vd;
};

struct TreeOut {
  int* tokens;
  int* parents;
  int* depth;
  int* pos;
  uint64_t* mask;
  float* score;
};

void tree_children(const TreeState& ts, int depth_new, const int* ids, const float* vals, const float* lse, int kk,
                   hipStream_t st);
void tree_frontier(const TreeState& ts, int d, const int* seq_lens, const DraftRows& dr, int S_cap, int* status,
                   hipStream_t st);
void tree_finalize(const TreeState& ts, int n_cand, int n_nodes, const int* roots, const int* seq_lens,
                   const TreeOut& out, int* status, hipStream_t st);
// Chain draw j for every sequence: logits rows of Vd entries (the draft vocabulary), q rows of V (the target's;
// scattered through d2t when the draft vocabulary is reduced, d2t NULL otherwise).
void chain_draw(int j, int K, const float* logits, int ld, int Vd, int V, float temperature, const double* lse64,
                const int* top1, const float* uniforms, int draft_greedy, float* q_out, int* chain_tok, int batch,
                unsigned long long* wsum, const int* d2t, hipStream_t st);
// ids[i] <- d2t[ids[i]] for i < n, ids outside [0, Vd) -> -1 (no-op when d2t is NULL).
void map_draft_ids(int* ids, int n, const int* d2t, int Vd, hipStream_t st);
// Raises BAD_TOKEN unless d2t[0..Vd) is strictly ascending within [0, V).
void check_d2t(const int* d2t, int Vd, int V, int* status, hipStream_t st);
void sample_rows(int n, const float* logits, int V, float temperature, const double* lse64, const int* top1,
                 const float* uniforms, int* tokens, unsigned long long* wsum, hipStream_t st);
void chain_rows(int j, int K, const int* chain_tok, const int* seq_lens, int emax, const DraftRows& dr, int S_cap,
                hipStream_t st);
void chain_finalize(int K, const int* roots, const int* seq_lens, int* chain_tok, const TreeOut& out, int batch,
                    hipStream_t st);

// ------------------------------------------------------------ accept/compact
// ndraft (nullable, [batch]): per-request draft lengths; only a request's first ndraft[b] nodes (plus the root)
// take part, the chain's final draw keeps uniforms[b, K].
void accept_greedy(int batch, int n_rows, int depth, const int* tokens, const int* parents, const int* argmax,
                   int* path, int* path_len, int* next_root, int* emitted, const int* ndraft, int* status,
                   hipStream_t st);
// Tree rejection sampling: slice sums of the integer weights of every row (wsum holds
// rows * sampler_slices(V) values), then one 1024-thread block per sequence walks the
// tree (n_rows, topk <= 64).
void accept_tree(int batch, int n_rows, int V, int topk, int depth, const int* tokens, const int* parents,
                 const float* logits, const double* lse64, unsigned long long* wsum, float temperature,
                 const float* uniforms, int* path, int* path_len, int* next_root, int* emitted, const int* ndraft,
                 int* status, hipStream_t st);
// Chain acceptance: sel [batch] ints and wsum [2 * batch * sampler_slices(V)] are scratch.
void accept_chain(int batch, int K, int V, const int* tokens, const float* logits, const double* lse64,
                  float temperature, const float* q, const float* uniforms, int* path, int* path_len, int* next_root,
                  int* emitted, int* sel, unsigned long long* wsum, const int* ndraft, hipStream_t st);
// kv: n_layers x (K, V) arrays of layer_elems elements each, addressed as in KvPages.
void compact_kv(bool bf16, int batch, const int* seq_lens, const int* path, const int* path_len, int maxp,
                int n_rows, void* kv, int n_layers, size_t layer_elems, size_t unit_stride, size_t head_stride,
                const KvPages& pg, int Hkv, int S_cap, int hd, int* status, hipStream_t st);
void compact_finish(bool bf16, int batch, int* seq_lens, int n_rows, int maxp, const int* path, const int* path_len,
                    const int* tokens, const int* next_root, const void* aux_tree, int aux_w, void* aux_new,
                    int* next_tok, int* new_len, int* src_dst, hipStream_t st);

}  // namespace e3
