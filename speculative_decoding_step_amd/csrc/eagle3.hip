// C ABI of the EAGLE-3 step: context, workspace layout and the launch
// sequences of draft_tree / verify_tree / accept / compact_kv (see eagle3.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/eagle3.h"
#include "common.hpp"
#include "kernels.hpp"
#include "sampler.hpp"
#include "tree.hpp"

using namespace e3;

namespace {

constexpr int KMAX = 16;  // largest top-k the vocabulary kernels keep
constexpr int ATT_CHUNK = 256;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Carver {
  char* base;
  size_t off = 0;
  template <typename P>
  P* take(size_t count) {
    off = align_up(off, 256);
    P* p = base ? (P*)(base + off) : nullptr;
    off += count * sizeof(P);
    return p;
  }
};

struct ProfRec {
  int kernel;
  hipEvent_t a, b;
  double bytes, flops;
};

}  // namespace

struct eagle3_ctx {
  eagle3_shape sh;
  eagle3_spec_cfg cfg;
  eagle3_target_weights tw;
  std::vector<eagle3_layer_weights> layers;
  eagle3_head_weights hw;
  int Vd;                  // draft vocabulary (the target's when the head is shared)
  const void* dhead;       // the draft's LM head: its own [Vd, d], or the target's
  const int* d2t;          // draft id -> target id (NULL when the head is shared)
  int B, R, S_cap;
  bool bf16;
  size_t esz;
  hipStream_t st;
  char* kv_t;
  char* kv_d;
  KvPages pg;                   // block table of a paged cache (pg.bt null: contiguous)
  size_t kv_us, kv_hs, kv_le;   // unit stride, head stride, elements per layer's K (or V) array
  const int* ndraft = nullptr;  // per-request draft lengths (device, [max_batch]) or null
  float* dl_out = nullptr;      // draft logits table [max_batch, tab_rows, Vd] (parity output) or null
  float* hid_out = nullptr;     // verify residual streams [n_layers + 1, R, d] (parity output) or null
  // workspace
  int* status;
  double* inv_freq;
  float *xres, *dx, *part;
  size_t part_elems;
  void *hbuf, *abuf, *qbuf, *gbuf;
  float *o_part, *ml_part;
  int att_splits;
  int* att_plan;  // work order of the attention launches over several sequences
  float* logits;
  float *tk_pv, *tk_pmax, *tk_vals, *tk_lse;
  int *tk_pi, *tk_ids;
  double *tk_psum, *tk_lse64;
  SliceTopk tf;  // candidates of the LM-head GEMMs with the top-k in their epilogue
  int tf_k = 0;  // the largest k they are sized for
  unsigned long long* tk_wsum;  // per-row slice sums of integer sampling weights
  int* acc_sel;                 // chain acceptance: drafts accepted per sequence
  RowMeta rm;
  int *rtok, *gidx, *roots;
  float *a_last, *a_rows;
  DraftRows dr;
  TreeState ts;
  int* chain_tok;
  int emax, n_cand;
  int tab_rows;  // rows per sequence of a draft-logits table: the root row + (depth - 1) * topk expansions
  // profiling
  bool prof = false;
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
  size_t pool_used = 0;
};

namespace {

size_t carve(eagle3_ctx* c, char* base) {
  const eagle3_shape& s = c->sh;
  const int R = c->R, B = c->B, d = s.d_model, V = s.vocab;
  const int qdim = s.n_heads * s.head_dim, kvdim = s.n_kv_heads * s.head_dim;
  const size_t es = c->esz;
  Carver cv{base};
  c->status = cv.take<int>(64);
  c->inv_freq = cv.take<double>(s.head_dim / 2);
  c->xres = cv.take<float>((size_t)R * d);
  c->dx = cv.take<float>((size_t)R * d);
  const int nmax = std::max({qdim + 2 * kvdim, 2 * s.ffn, d});
  const size_t prow = std::max(R, 512);
  c->part_elems = prow * nmax;
  c->part = cv.take<float>(c->part_elems);
  // GEMM inputs (hbuf, abuf, gbuf) are stored in column slabs of 32 in passes of more than 64 rows (sized for
  // rows padded to 16)
  const size_t R16 = (size_t)(R + 15) / 16 * 16;
  c->hbuf = cv.take<char>(R16 * 2 * d * es);
  c->abuf = cv.take<char>(R16 * std::max(qdim, s.ffn) * es);
  c->qbuf = cv.take<char>((size_t)R * qdim * es);
  c->gbuf = cv.take<char>(R16 * d * es);
  c->att_splits = std::max(1, (c->S_cap + ATT_CHUNK - 1) / ATT_CHUNK);
  c->o_part = cv.take<float>((size_t)c->att_splits * R * qdim);
  c->ml_part = cv.take<float>((size_t)c->att_splits * R * s.n_heads * 2);
  c->att_plan = cv.take<int>(ATT_PLAN_CAP);
  c->logits = cv.take<float>((size_t)R * V);
  const int ns = topk_slices(V);
  c->tk_pv = cv.take<float>((size_t)R * ns * KMAX);
  c->tk_pi = cv.take<int>((size_t)R * ns * KMAX);
  c->tk_pmax = cv.take<float>((size_t)R * ns);
  c->tk_psum = cv.take<double>((size_t)R * ns);
  c->tk_ids = cv.take<int>((size_t)R * KMAX);
  c->tk_vals = cv.take<float>((size_t)R * KMAX);
  c->tk_lse = cv.take<float>(R);
  c->tk_lse64 = cv.take<double>(R);
  {  // fused LM-head top-k: up to R rows, k up to the tree's top-k (2 for the verify's argmax and margin)
    const size_t nsf = (size_t)(V + TOPK_SLICE - 1) / TOPK_SLICE;
    c->tf_k = std::max(2, c->cfg.topk);
    c->tf.pv = cv.take<float>((size_t)R * nsf * c->tf_k);
    c->tf.pi = cv.take<int>((size_t)R * nsf * c->tf_k);
    c->tf.pmax = cv.take<float>((size_t)R * nsf);
    c->tf.psum = cv.take<double>((size_t)R * nsf);
  }
  c->tk_wsum = cv.take<unsigned long long>((size_t)R * sampler_slices(V));
  c->acc_sel = cv.take<int>(B);
  c->rm.seq = cv.take<int>(R);
  c->rm.pos = cv.take<int>(R);
  c->rm.slot = cv.take<int>(R);
  c->rm.lim = cv.take<int>(R);
  c->rm.tail0 = cv.take<int>(R);
  c->rm.mask = cv.take<uint64_t>(R);
  c->rtok = cv.take<int>(R);
  c->gidx = cv.take<int>(R);
  c->roots = cv.take<int>(B);
  const int D = c->cfg.depth, k = c->cfg.topk;
  c->emax = std::max(1, (D - 1) * k);  // scratch row count, at least one so depth 1 carves no empty arrays
  c->tab_rows = 1 + (D - 1) * k;
  c->n_cand = c->cfg.mode != EAGLE3_SAMPLE_CHAIN ? k + (D - 1) * k * k : D;
  c->a_last = cv.take<float>((size_t)B * d);
  c->a_rows = cv.take<float>((size_t)B * c->emax * d);
  c->dr.batch = B;
  c->dr.tok = cv.take<int>(R);
  c->dr.src = cv.take<int>(R);
  c->dr.seq = cv.take<int>(R);
  c->dr.pos = cv.take<int>(R);
  c->dr.slot = cv.take<int>(R);
  c->dr.lim = cv.take<int>(R);
  c->dr.tail0 = cv.take<int>(R);
  c->dr.mask = cv.take<uint64_t>(R);
  const int cmax = std::max(c->n_cand, 1);
  c->ts.batch = B;
  c->ts.topk = k;
  c->ts.cmax = cmax;
  c->ts.emax = c->emax;
  c->ts.tok = cv.take<int>((size_t)B * cmax);
  c->ts.par = cv.take<int>((size_t)B * cmax);
  c->ts.dep = cv.take<int>((size_t)B * cmax);
  c->ts.score = cv.take<float>((size_t)B * cmax);
  c->ts.erow = cv.take<int>((size_t)B * cmax);
  c->ts.front = cv.take<int>((size_t)B * k);
  c->ts.emask = cv.take<uint64_t>((size_t)B * c->emax);
  c->chain_tok = cv.take<int>((size_t)B * (D + 1));
  return align_up(cv.off, 256);
}

eagle3_status check_shape(const eagle3_shape* s, const eagle3_spec_cfg* c) {
  if (!s || !c) return EAGLE3_EINVAL;
  if (s->n_layers < 1 || s->d_model < 1 || s->n_heads < 1 || s->n_kv_heads < 1 || s->head_dim < 2 ||
      s->ffn < 1 || s->vocab < 2)
    return EAGLE3_EINVAL;
  if (s->n_heads % s->n_kv_heads || s->head_dim % 4 || s->head_dim > 256) return EAGLE3_EINVAL;
  if (s->dtype != EAGLE3_F32 && s->dtype != EAGLE3_BF16) return EAGLE3_EINVAL;
  for (int i = 0; i < 3; ++i)
    if (s->taps[i] < 0 || s->taps[i] >= s->n_layers) return EAGLE3_EINVAL;
  if (s->dtype == EAGLE3_BF16) {
    const int qdim = s->n_heads * s->head_dim;
    if (s->d_model % 256 || qdim % 256 || s->ffn % 256) return EAGLE3_EUNSUPPORTED;
  }
  if (s->vocab > 64 * 4096) return EAGLE3_EUNSUPPORTED;
  if (s->draft_vocab < 0 || s->draft_vocab > s->vocab) return EAGLE3_EINVAL;
  const int Vd = s->draft_vocab > 0 ? s->draft_vocab : s->vocab;
  if (c->depth < 1 || c->topk < 1 || c->topk > KMAX || c->n_nodes < 1 || c->topk > Vd) return EAGLE3_EINVAL;
  if (c->n_nodes + 1 > 64 || (c->depth - 1) * c->topk > 64) return EAGLE3_EUNSUPPORTED;
  if (c->mode == EAGLE3_GREEDY_TREE || c->mode == EAGLE3_SAMPLE_TREE) {
    const int nc = c->topk + (c->depth - 1) * c->topk * c->topk;
    if (nc < c->n_nodes) return EAGLE3_EINVAL;  // more nodes than the tree has candidates
    if (nc > TREE_CMAX) return EAGLE3_EUNSUPPORTED;
    if (c->mode == EAGLE3_SAMPLE_TREE && !(c->temperature > 0.f)) return EAGLE3_EINVAL;
  } else if (c->mode == EAGLE3_SAMPLE_CHAIN) {
    if (c->topk != 1 || c->n_nodes != c->depth || !(c->temperature > 0.f)) return EAGLE3_EINVAL;
  } else {
    return EAGLE3_EINVAL;
  }
  return EAGLE3_OK;
}

// ------------------------------------------------------------- small kernels

__global__ void k_verify_meta(int batch, int seq_begin, int n_rows, const int* __restrict__ seq_lens,
                              const int* __restrict__ tokens, const int* __restrict__ pos_in,
                              const uint64_t* __restrict__ mask_in, int S_cap, const int* __restrict__ ndraft,
                              RowMeta rm, int* __restrict__ rtok, int* __restrict__ gidx, int* status) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= batch * n_rows) return;
  const int b = r / n_rows, i = r % n_rows;
  const int P = seq_lens[b];
  const int slot = P + i;
  // with per-request draft lengths, rows of a draft (a masked verify) past the request's first ndraft nodes take
  // no part (no K/V, no keys); a prefill (no mask) keeps every row
  const int nr = ndraft && mask_in ? min(max(ndraft[seq_begin + b], 0), n_rows - 1) + 1 : n_rows;
  const bool ok = P >= 0 && P + nr <= S_cap;
  if (!ok && i == 0) raise_flag(status, E3_DEV_KV_OVERFLOW);
  rm.seq[r] = ok && i < nr ? seq_begin + b : -1;
  rm.pos[r] = pos_in ? pos_in[r] : slot;
  rm.slot[r] = slot;
  rm.lim[r] = mask_in ? P : slot + 1;
  rm.tail0[r] = P;
  rm.mask[r] = mask_in ? mask_in[r] : 0ull;
  rtok[r] = tokens[r];
  if (i == n_rows - 1) gidx[b] = r;
}

// Catch-up rows of the draft: row b*(D+1)+j is position P_b - c_b + j.
__global__ void k_catchup_meta(int batch, int W, const int* __restrict__ seq_lens, const int* __restrict__ new_len,
                               const int* __restrict__ next_tok, int S_cap, RowMeta rm, int* __restrict__ rtok,
                               int* __restrict__ gidx, int* __restrict__ roots, int* status) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= batch * W) return;
  const int b = r / W, j = r % W;
  const int P = seq_lens[b], c = new_len[b];
  const bool cok = c >= 1 && c <= W && P - c >= 0 && P <= S_cap;
  const bool valid = cok && j < c;
  const int pos = P - c + j;
  if (!cok && j == 0) raise_flag(status, E3_DEV_BAD_PATH);
  rm.seq[r] = valid && pos < S_cap ? b : -1;
  rm.pos[r] = valid ? pos : 0;
  rm.slot[r] = valid ? pos : 0;
  rm.lim[r] = valid ? pos + 1 : 0;
  rm.tail0[r] = 0;
  rm.mask[r] = 0ull;
  rtok[r] = valid ? next_tok[r] : -1;
  if (j == 0) {
    const int last = cok ? c - 1 : 0;
    gidx[b] = b * W + last;
    roots[b] = next_tok[b * W + last];
  }
}

__global__ void k_prefill_meta(int batch, int seq_begin, int n_rows, const int* __restrict__ start,
                               const int* __restrict__ next_tok, int S_cap, RowMeta rm, int* __restrict__ rtok,
                               int* status) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= batch * n_rows) return;
  const int b = r / n_rows, j = r % n_rows;
  const int pos = start[b] + j;
  const bool ok = pos >= 0 && pos < S_cap;
  if (!ok) raise_flag(status, E3_DEV_KV_OVERFLOW);
  rm.seq[r] = ok ? seq_begin + b : -1;
  rm.pos[r] = pos;
  rm.slot[r] = ok ? pos : 0;
  rm.lim[r] = pos + 1;
  rm.tail0[r] = 0;
  rm.mask[r] = 0ull;
  rtok[r] = next_tok[r];
}

template <typename T>
__global__ void k_store_tap(const float* __restrict__ x, int d, T* __restrict__ aux, int aux_ld, int col0) {
  const int r = blockIdx.x;
  for (int i = threadIdx.x; i < d; i += blockDim.x) st<T>(aux, (size_t)r * aux_ld + col0 + i, x[(size_t)r * d + i]);
}

__global__ void k_argmax_margin(int n, const int* __restrict__ ids, const float* __restrict__ vals, int kk,
                                int* __restrict__ am, float* __restrict__ mg) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n) return;
  if (am) am[r] = ids[(size_t)r * kk];
  if (mg) mg[r] = kk > 1 ? vals[(size_t)r * kk] - vals[(size_t)r * kk + 1] : 0.f;
}

__global__ void k_seq_roots(int batch, int K1, const int* __restrict__ roots_in, int* __restrict__ roots) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch) roots[b] = roots_in[b];
  (void)K1;
}

inline unsigned nb(size_t n, int b) { return (unsigned)((n + b - 1) / b); }

// n floats src -> dst (n % 4 == 0), 256 threads, one float4 per thread.
__global__ void k_copy_f32x4(const float* __restrict__ src, float* __restrict__ dst, size_t n4) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) ((float4*)dst)[i] = ((const float4*)src)[i];
}

// Draft logits table output: rows [b * per, (b + 1) * per) of src (Vd floats
// each) go to rows row0 .. row0 + per - 1 of sequence b's table block.
// grid (ceil(Vd / 1024), batch * per), 256 threads, float4 when Vd % 4 == 0.
__global__ void k_copy_logit_rows(const float* __restrict__ src, int per, int Vd, float* __restrict__ dst,
                                  size_t seq_stride, int row0) {
  const int r = blockIdx.y, b = r / per, i = r % per;
  const float* s = src + (size_t)r * Vd;
  float* d = dst + (size_t)b * seq_stride + (size_t)(row0 + i) * Vd;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if ((Vd & 3) == 0) {
    if (c < Vd) *(float4*)(d + c) = *(const float4*)(s + c);
  } else {
    for (int j = c; j < min(c + 4, Vd); ++j) d[j] = s[j];
  }
}

// ------------------------------------------------------------ profiling
// With record = false the caller hands the event pair to a launch that records
// it itself (at the kernel's start and end).
void prof_begin(eagle3_ctx* c, int kernel, double bytes, double flops, ProfRec* rec, bool record = true) {
  if (!c->prof) return;
  if (c->pool_used + 2 > c->pool.size()) {
    for (int i = 0; i < 256; ++i) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) break;
      c->pool.push_back(e);
    }
  }
  if (c->pool_used + 2 > c->pool.size()) return;
  rec->kernel = kernel;
  rec->a = c->pool[c->pool_used++];
  rec->b = c->pool[c->pool_used++];
  rec->bytes = bytes;
  rec->flops = flops;
  if (record) (void)hipEventRecord(rec->a, c->st);
}
void prof_end(eagle3_ctx* c, ProfRec* rec, bool record = true) {
  if (!c->prof || !rec->a) return;
  if (record) (void)hipEventRecord(rec->b, c->st);
  c->recs.push_back(*rec);
}

// ----------------------------------------------------------------- GEMM plan
int plan_splits(eagle3_ctx* c, int M, int N, int K, int m_tile) {
  if (!c->bf16) return 1;
  const int rows = gemm_rows_per_tile(true, m_tile);
  const int tiles = ((N + rows - 1) / rows) * ((M + m_tile - 1) / m_tile);
  // Skinny kernels: about 256 eight-wave (M <= 64) or 512 four-wave (M <= 16)
  // workgroups.  Large-M kernel (two workgroups per CU): the most splits that
  // still fit one round of 512 workgroups, since a partial second round costs
  // more than the split saves (measured at M = 1088).  At most 8 splits: every
  // split adds M x N fp32 partials that the consumer kernel reads back.
  int S;
  if (m_tile > 64)
    S = std::max(1, 512 / tiles);
  else
    S = ((m_tile == 64 ? 256 : 512) + tiles / 2) / tiles;
  S = std::max(1, std::min(8, S));
  const int mpad = (M + m_tile - 1) / m_tile * m_tile;
  while (S > 1 && (size_t)S * mpad * N > c->part_elems) --S;
  return gemm_splits(true, K, S, m_tile);
}

// Whether a pass of M rows keeps its bf16 GEMM inputs (the norm outputs, the draft input, the attention output,
// SiLU(g)*u) in column slabs of 32 (slab32_index): the large-M GEMM reads them as contiguous fragments.
inline bool packed_inputs(const eagle3_ctx* c, int M) { return c->bf16 && M > 64; }

// X [M, K] of T times the stacked weights; returns the number of splits in c->part.  X is in column slabs of 32
// when packed_inputs(M), except for a row-major input (x_rowmajor: the fusion FC's tap rows).
int run_gemm(eagle3_ctx* c, const void* X, int M, int K, const GemmSegs& sg, float* out_direct = nullptr,
             bool x_rowmajor = false) {
  const int N = gemm_ntot(sg);
  const int m_tile = M <= 16 ? 16 : (M <= 64 ? 64 : 128);
  const int S = out_direct ? 1 : plan_splits(c, M, N, K, m_tile);
  ProfRec rec{};
  const double bytes = (double)N * K * c->esz + (double)M * K * c->esz + (double)M * N * 4.0;
  const int kid = m_tile == 16 ? EAGLE3_PROF_GEMM_M16 : (m_tile == 64 ? EAGLE3_PROF_GEMM_M64 : EAGLE3_PROF_GEMM_BIG);
  // the bf16 kernels record the pair at their own start and end
  prof_begin(c, kid, bytes, 2.0 * M * N * K, &rec, !c->bf16);
  const int used = gemm(c->bf16, X, M, K, sg, out_direct ? out_direct : c->part, (size_t)M * N, S, m_tile, c->st,
                        c->bf16 ? rec.a : nullptr, c->bf16 ? rec.b : nullptr, packed_inputs(c, M) && !x_rowmajor);
  prof_end(c, &rec, !c->bf16);
  return used;
}

// LM head over n rows of X (bf16) with the top-k of every row taken in the GEMM's epilogue
// (per 128-id slice) and merged by one more kernel: logits [n, V] as run_gemm writes them (none when logits
// is null), the k best (id,
// value) of each row in tk_ids / tk_vals, and the log-sum-exp of logits / temperature in tk_lse / tk_lse64
// when lse.  Returns false, launching nothing, for shapes the fused kernel does not cover.
bool run_lm_topk(eagle3_ctx* c, const void* X, int n, const void* W, int V, float* logits, int k, float temperature,
                 bool lse, const TreeKids* kids = nullptr, bool* kids_done = nullptr) {
  const int d = c->sh.d_model;
  if (!c->bf16 || n <= 0 || n > c->R || k > c->tf_k) return false;
  SliceTopk tk = c->tf;
  tk.k = k;
  tk.ns = (V + TOPK_SLICE - 1) / TOPK_SLICE;
  tk.temp = (double)temperature;
  if (!lse) {
    tk.pmax = nullptr;
    tk.psum = nullptr;
  }
  ProfRec rec{};
  const double bytes = (double)V * d * c->esz + (double)n * d * c->esz + (double)n * V * 4.0;
  prof_begin(c, n <= 16 ? EAGLE3_PROF_GEMM_M16 : (n <= 64 ? EAGLE3_PROF_GEMM_M64 : EAGLE3_PROF_GEMM_BIG), bytes,
             2.0 * n * V * d, &rec, false);
  const bool ok = gemm_lm_topk(X, n, d, W, V, logits, V, tk, c->st, rec.a, rec.b);
  prof_end(c, &rec, false);
  if (!ok) return false;
  const bool kd = topk_merge_slices(n, tk, c->tk_ids, c->tk_vals, lse ? c->tk_lse : nullptr,
                                    lse ? c->tk_lse64 : nullptr, c->st, kids);
  if (kids_done) *kids_done = kd;
  return true;
}

// abuf = T(silu(X w_gate^T) * (X w_up^T)) for X [M, K]: fused into the GEMM's
// epilogue for bf16 when the fused launch has enough workgroups without a K
// split (M > 64, or F / 64 >= 128 column groups), else GEMM partials +
// silu_mul.
void run_gateup(eagle3_ctx* c, const void* X, int M, int K, const void* w_gate, const void* w_up, int F) {
  if (c->bf16 && (M > 64 || F / 64 >= 128)) {
    ProfRec rec{};
    const double bytes = 2.0 * F * K * c->esz + (double)M * K * c->esz + (double)M * F * c->esz;
    const int kid = M > 64 ? EAGLE3_PROF_GEMM_BIG : (M > 16 ? EAGLE3_PROF_GEMM_M64 : EAGLE3_PROF_GEMM_M16);
    prof_begin(c, kid, bytes, 4.0 * M * F * K, &rec, false);
    if (M > 64)
      gemm_big_silu(X, M, K, w_gate, w_up, F, c->abuf, c->st, rec.a, rec.b);
    else
      gemm_silu(X, M, K, w_gate, w_up, F, c->abuf, c->st, rec.a, rec.b);
    prof_end(c, &rec, false);
    return;
  }
  const int S = run_gemm(c, X, M, K, make_segs(w_gate, F, w_up, F));
  silu_mul(c->bf16, c->abuf, c->part, S, (size_t)M * 2 * F, M, F, 2 * F, c->st);
}

// Orders the work of the attention launches over rm that follow (every layer of one pass); false when they
// take no order.
bool plan_attention(eagle3_ctx* c, const RowMeta& rm, int R, int rps) {
  const eagle3_shape& s = c->sh;
  return attention_plan(c->bf16, c->pg, rm, R, rps, s.n_heads, s.n_kv_heads, s.head_dim, c->S_cap,
                        c->att_splits, c->att_plan, c->ml_part, c->st);
}

// planned: plan_attention returned true for these rows since their metadata last changed.
void run_attention(eagle3_ctx* c, const void* kc, const void* vc, const RowMeta& rm, int R, int rps,
                   bool planned) {
  const eagle3_shape& s = c->sh;
  ProfRec rec{};
  prof_begin(c, EAGLE3_PROF_ATTN, 0.0, 0.0, &rec);
  attention(c->bf16, c->qbuf, kc, vc, c->kv_us, c->kv_hs, c->pg, rm, R, rps, s.n_heads, s.n_kv_heads, s.head_dim,
            c->S_cap, c->o_part, c->ml_part, c->att_splits, c->abuf, c->st, packed_inputs(c, R),
            planned ? c->att_plan : nullptr);
  prof_end(c, &rec);
}

// K (which = 0) or V (1) array of layer l: kv_le elements each, in layer order.
char* kv_layer(eagle3_ctx* c, char* base, int l, int which) {
  return base + ((size_t)l * 2 + which) * c->kv_le * c->esz;
}

// Target pass over R rows whose metadata is in c->rm and tokens in c->rtok.
// lm: EAGLE3_LM_ALL (rows 0..R-1), LM_LAST (rows c->gidx[0..nlast)), LM_NONE.
void target_forward(eagle3_ctx* c, int R, int rps, void* aux, int lm, int nlast, float* logits, int* argmax,
                    float* margin) {
  const eagle3_shape& s = c->sh;
  const int d = s.d_model, qdim = s.n_heads * s.head_dim, kvdim = s.n_kv_heads * s.head_dim;
  const bool bf = c->bf16;
  const bool pk = packed_inputs(c, R);
  hipStream_t st = c->st;
  auto record = [&](int l) {  // parity output: the residual entering layer l (l = n_layers: leaving the last)
    if (!c->hid_out) return;
    const size_t n = (size_t)R * d;
    if (n % 4 == 0)
      k_copy_f32x4<<<nb(n / 4, 256), 256, 0, st>>>(c->xres, c->hid_out + (size_t)l * n, n / 4);
    else
      (void)hipMemcpyAsync(c->hid_out + (size_t)l * n, c->xres, n * sizeof(float), hipMemcpyDeviceToDevice, st);
  };
  embed_rows(bf, c->tw.embed, c->rtok, c->xres, R, d, s.vocab, c->status, st);
  record(0);
  // Residual entering layer l (after adding S partials of the previous GEMM, if
  // any): captured into the aux columns of every tap equal to l and normalised
  // with w into out.
  auto enter = [&](int l, int S, const void* w, void* out) {
    int first = -1;
    for (int t = 0; t < 3; ++t)
      if (aux && s.taps[t] == l && first < 0) first = t;
    void* tap = first < 0 ? nullptr : (char*)aux + (size_t)first * d * c->esz;
    add_rmsnorm(bf, c->xres, S ? c->part : nullptr, S, (size_t)R * d, d, w, out, d, R, d, s.rms_eps, tap, 3 * d, st,
                pk);
    for (int t = first + 1; first >= 0 && t < 3; ++t)
      if (s.taps[t] == l) {
        if (bf)
          k_store_tap<bf16_t><<<R, 256, 0, st>>>(c->xres, d, (bf16_t*)aux, 3 * d, t * d);
        else
          k_store_tap<float><<<R, 256, 0, st>>>(c->xres, d, (float*)aux, 3 * d, t * d);
      }
  };
  enter(0, 0, c->layers[0].attn_norm, c->hbuf);
  const bool planned = plan_attention(c, c->rm, R, rps);
  bool final_normed = false;
  for (int l = 0; l < s.n_layers; ++l) {
    const eagle3_layer_weights& L = c->layers[l];
    const GemmSegs qkv = make_segs(L.wq, qdim, L.wk, kvdim, L.wv, kvdim);
    int S = run_gemm(c, c->hbuf, R, d, qkv);
    char* kc = kv_layer(c, c->kv_t, l, 0);
    char* vc = kv_layer(c, c->kv_t, l, 1);
    rope_kv(bf, c->part, S, (size_t)R * gemm_ntot(qkv), R, c->rm, c->inv_freq, c->qbuf, kc, vc,
            c->kv_us, c->kv_hs, c->pg, s.n_heads, s.n_kv_heads, s.head_dim, c->status, st);
    run_attention(c, kc, vc, c->rm, R, rps, planned);
    S = run_gemm(c, c->abuf, R, qdim, make_segs(L.wo, d));
    add_rmsnorm(bf, c->xres, c->part, S, (size_t)R * d, d, L.ffn_norm, c->hbuf, d, R, d, s.rms_eps, nullptr, 0, st,
                pk);
    run_gateup(c, c->hbuf, R, d, L.w_gate, L.w_up, s.ffn);
    S = run_gemm(c, c->abuf, R, s.ffn, make_segs(L.w_down, d));
    if (l + 1 < s.n_layers) {
      enter(l + 1, S, c->layers[l + 1].attn_norm, c->hbuf);
    } else if (lm == EAGLE3_LM_ALL) {
      add_rmsnorm(bf, c->xres, c->part, S, (size_t)R * d, d, c->tw.final_norm, c->gbuf, d, R, d, s.rms_eps, nullptr,
                  0, st, pk);
      final_normed = true;
    } else {
      resid_add(c->xres, c->part, S, (size_t)R * d, R, d, d, st);
    }
    record(l + 1);
  }
  if (lm == EAGLE3_LM_NONE) return;
  int n = R;
  const float* fin = c->xres;
  if (lm == EAGLE3_LM_LAST) {
    gather_rows_f32(c->dx, c->xres, c->gidx, nlast, d, st);
    fin = c->dx;
    n = nlast;
  }
  if (!final_normed) rmsnorm(bf, fin, c->tw.final_norm, c->gbuf, d, n, d, s.rms_eps, nullptr, 0, st, packed_inputs(c, n));
  float* lg = logits ? logits : c->logits;
  // the fused head writes the logits only when the caller asked for them
  if ((argmax || margin) && run_lm_topk(c, c->gbuf, n, c->tw.lm_head, s.vocab, logits, 2, 1.f, false)) {
    k_argmax_margin<<<nb(n, 128), 128, 0, st>>>(n, c->tk_ids, c->tk_vals, 2, argmax, margin);
    return;
  }
  run_gemm(c, c->gbuf, n, d, make_segs(c->tw.lm_head, s.vocab), lg);
  if (argmax || margin) {
    topk_lse(lg, n, s.vocab, s.vocab, 2, 1.f, c->tk_pv, c->tk_pi, c->tk_pmax, c->tk_psum, c->tk_ids, c->tk_vals,
             nullptr, nullptr, st);
    k_argmax_margin<<<nb(n, 128), 128, 0, st>>>(n, c->tk_ids, c->tk_vals, 2, argmax, margin);
  }
}

// The draft decoder layer over R rows: x (fp32 [R, d]) is g or a on entry and
// a on exit; tokens in tok; row metadata rm (draft KV cache).  fc_splits > 0:
// x is formed on entry from that many fusion-FC split partials in c->part
// (g = W_fc [l; m; h]) by the same kernel that builds the layer's input.
// io (optional): the layer's input rows gathered from their parents' outputs by the kernel that builds the
// layer's input (src / a_rows / a_last, as draft_input takes them), and, with norm_out, the layer's last
// kernel also forms the draft LM head's input (x += partials; gbuf = T(rmsnorm(x) * final_norm)) and copies
// the rows to the tree's expansion-row store (keep).
struct DraftIo {
  const int* src = nullptr;
  const float* a_rows = nullptr;
  const float* a_last = nullptr;
  bool norm_out = false;
  RowCopy keep;
};

void draft_layer(eagle3_ctx* c, int R, int rps, const int* tok, float* x, const RowMeta& rm, int fc_splits = 0,
                 const DraftIo* io = nullptr) {
  const eagle3_shape& s = c->sh;
  const eagle3_head_weights& H = c->hw;
  const int d = s.d_model, qdim = s.n_heads * s.head_dim, kvdim = s.n_kv_heads * s.head_dim;
  const bool bf = c->bf16;
  hipStream_t st = c->st;
  const bool pk = packed_inputs(c, R);
  draft_input(bf, c->tw.embed, tok, x, fc_splits ? c->part : nullptr, fc_splits, (size_t)R * d, H.input_norm,
              H.hidden_norm, c->hbuf, R, d, s.vocab, s.rms_eps, c->status, st, pk, io ? io->src : nullptr,
              io ? io->a_rows : nullptr, io ? io->a_last : nullptr);
  const GemmSegs qkv = make_segs(H.wq, qdim, H.wk, kvdim, H.wv, kvdim);
  int S = run_gemm(c, c->hbuf, R, 2 * d, qkv);
  char* kc = kv_layer(c, c->kv_d, 0, 0);
  char* vc = kv_layer(c, c->kv_d, 0, 1);
  rope_kv(bf, c->part, S, (size_t)R * gemm_ntot(qkv), R, rm, c->inv_freq, c->qbuf, kc, vc,
          c->kv_us, c->kv_hs, c->pg, s.n_heads, s.n_kv_heads, s.head_dim, c->status, st);
  run_attention(c, kc, vc, rm, R, rps, plan_attention(c, rm, R, rps));
  S = run_gemm(c, c->abuf, R, qdim, make_segs(H.wo, d));
  add_rmsnorm(bf, x, c->part, S, (size_t)R * d, d, H.post_norm, c->hbuf, d, R, d, s.rms_eps, nullptr, 0, st, pk);
  run_gateup(c, c->hbuf, R, d, H.w_gate, H.w_up, s.ffn);
  S = run_gemm(c, c->abuf, R, s.ffn, make_segs(H.w_down, d));
  if (io && io->norm_out)
    add_rmsnorm(bf, x, c->part, S, (size_t)R * d, d, H.final_norm, c->gbuf, d, R, d, s.rms_eps, nullptr, 0, st, pk,
                io->keep);
  else
    resid_add(x, c->part, S, (size_t)R * d, R, d, d, st);
}

// Draft logits of n rows of a (fp32 [n, d]) -> c->logits; top-K + lse, ids
// through d2t.  With a draft logits table set, the n rows (per rows of each of
// n / per sequences) are also copied to table rows row0 .. row0 + per - 1.
// normed: the head's input (the rows' final norm, in c->gbuf) is already
// there.  kids_depth > 0: the rows are a tree level whose children have depth
// kids_depth; returns true when the head's merge has recorded them (else the
// caller runs tree_children).
bool draft_lm(eagle3_ctx* c, int n, const float* a, int K, float temperature, int per, int row0, bool normed = false,
              int kids_depth = 0) {
  const eagle3_shape& s = c->sh;
  if (!normed)
    rmsnorm(c->bf16, a, c->hw.final_norm, c->gbuf, s.d_model, n, s.d_model, s.rms_eps, nullptr, 0, c->st,
            packed_inputs(c, n));
  // the logits themselves are read only by the chain sampler and the draft-logits table
  const bool keep = c->dl_out || c->cfg.mode == EAGLE3_SAMPLE_CHAIN;
  TreeKids kids{c->ts, kids_depth, c->d2t, c->Vd};
  bool kids_done = false;
  const bool fused = run_lm_topk(c, c->gbuf, n, c->dhead, c->Vd, keep ? c->logits : nullptr, K, temperature, true,
                                 kids_depth > 0 ? &kids : nullptr, &kids_done);
  if (!fused) run_gemm(c, c->gbuf, n, s.d_model, make_segs(c->dhead, c->Vd), c->logits);
  if (c->dl_out && n > 0)
    k_copy_logit_rows<<<dim3(nb(c->Vd, 1024), n), 256, 0, c->st>>>(c->logits, per, c->Vd, c->dl_out,
                                                                   (size_t)c->tab_rows * c->Vd, row0);
  if (!fused)
    topk_lse(c->logits, n, c->Vd, c->Vd, K, temperature, c->tk_pv, c->tk_pi, c->tk_pmax, c->tk_psum, c->tk_ids,
             c->tk_vals, c->tk_lse, c->tk_lse64, c->st);
  if (!fused || kids_depth <= 0) map_draft_ids(c->tk_ids, n * K, c->d2t, c->Vd, c->st);  // else the merge mapped them
  return kids_done;
}

RowMeta dr_meta(eagle3_ctx* c) {
  RowMeta m;
  m.seq = c->dr.seq;
  m.pos = c->dr.pos;
  m.slot = c->dr.slot;
  m.lim = c->dr.lim;
  m.tail0 = c->dr.tail0;
  m.mask = c->dr.mask;
  return m;
}

// Tree / chain construction after the root's draft row is in c->logits
// (top-k in c->tk_*).  table != null: rows come from the table instead of
// the draft model.
eagle3_status build_tree(eagle3_ctx* c, int batch, const int* seq_lens, const float* table, const float* uniforms,
                         const TreeOut& out, float* q, bool root_kids_done = false) {
  const eagle3_shape& s = c->sh;
  const int D = c->cfg.depth, k = c->cfg.topk, V = s.vocab, Vd = c->Vd, d = s.d_model;
  hipStream_t st = c->st;
  TreeState ts = c->ts;
  ts.batch = batch;
  DraftRows dr = c->dr;
  dr.batch = batch;
  const size_t tstride = (size_t)c->tab_rows * Vd;  // table row stride between sequences
  if (c->cfg.mode != EAGLE3_SAMPLE_CHAIN) {  // trees (greedy or sampled acceptance alike)
    if (!root_kids_done) tree_children(ts, 1, c->tk_ids, c->tk_vals, c->tk_lse, k, st);
    for (int dd = 1; dd < D; ++dd) {
      const int n = batch * k;
      tree_frontier(ts, dd, seq_lens, dr, c->S_cap, c->status, st);
      bool kids_done = false;
      if (table) {
        // expansion rows (dd-1)k .. dd k - 1 of each sequence
        for (int b = 0; b < batch; ++b)
          topk_lse(table + b * tstride + (size_t)(1 + (dd - 1) * k) * Vd, k, Vd, Vd, k, 1.f,
                   c->tk_pv + (size_t)b * k * topk_slices(Vd) * KMAX, c->tk_pi + (size_t)b * k * topk_slices(Vd) * KMAX,
                   c->tk_pmax + (size_t)b * k * topk_slices(Vd), c->tk_psum + (size_t)b * k * topk_slices(Vd),
                   c->tk_ids + (size_t)b * k * k, c->tk_vals + (size_t)b * k * k, c->tk_lse + b * k,
                   c->tk_lse64 + b * k, st);
        map_draft_ids(c->tk_ids, batch * k * k, c->d2t, c->Vd, st);
      } else {
        // the rows' inputs gathered from their parents inside the layer's first kernel; its last kernel forms the
        // head's input and keeps the rows for their children
        DraftIo io;
        io.src = dr.src;
        io.a_rows = c->a_rows;
        io.a_last = c->a_last;
        io.norm_out = true;
        if (dd + 1 < D) io.keep = RowCopy{c->a_rows, dr.slot, seq_lens, k, c->emax};
        draft_layer(c, n, k, dr.tok, c->dx, dr_meta(c), 0, &io);
        kids_done = draft_lm(c, n, c->dx, k, 1.f, k, 1 + (dd - 1) * k, true, dd + 1);
      }
      if (!kids_done) tree_children(ts, dd + 1, c->tk_ids, c->tk_vals, c->tk_lse, k, st);
    }
    tree_finalize(ts, c->n_cand, c->cfg.n_nodes, c->roots, seq_lens, out, c->status, st);
  } else {
    const int K = D;
    const float T = c->cfg.temperature;
    const float* z0 = table ? table : c->logits;
    const int ld0 = table ? (int)tstride : Vd;
    chain_draw(0, K, z0, ld0, Vd, V, T, c->tk_lse64, c->tk_ids, uniforms, c->cfg.draft_greedy, q, c->chain_tok,
               batch, c->tk_wsum, c->d2t, st);
    for (int j = 1; j < K; ++j) {
      if (table) {
        const float* zj = table + (size_t)j * Vd;
        for (int b = 0; b < batch; ++b)
          topk_lse(zj + b * tstride, 1, Vd, Vd, 1, T, c->tk_pv, c->tk_pi, c->tk_pmax, c->tk_psum, c->tk_ids + b,
                   c->tk_vals + b, c->tk_lse + b, c->tk_lse64 + b, st);
        map_draft_ids(c->tk_ids, batch, c->d2t, c->Vd, st);
        chain_draw(j, K, zj, (int)tstride, Vd, V, T, c->tk_lse64, c->tk_ids, uniforms, c->cfg.draft_greedy, q,
                   c->chain_tok, batch, c->tk_wsum, c->d2t, st);
      } else {
        chain_rows(j - 1, K, c->chain_tok, seq_lens, c->emax, dr, c->S_cap, st);
        DraftIo io;
        io.src = dr.src;
        io.a_rows = c->a_rows;
        io.a_last = c->a_last;
        io.norm_out = true;
        if (j + 1 < K) io.keep = RowCopy{c->a_rows, dr.slot, seq_lens, 1, c->emax};
        draft_layer(c, batch, 1, dr.tok, c->dx, dr_meta(c), 0, &io);
        draft_lm(c, batch, c->dx, 1, T, 1, j, true);
        chain_draw(j, K, c->logits, Vd, Vd, V, T, c->tk_lse64, c->tk_ids, uniforms, c->cfg.draft_greedy, q,
                   c->chain_tok, batch, c->tk_wsum, c->d2t, st);
      }
    }
    chain_finalize(K, c->roots, seq_lens, c->chain_tok, out, batch, st);
  }
  return EAGLE3_OK;
}

eagle3_status last_error() { return hipGetLastError() == hipSuccess ? EAGLE3_OK : EAGLE3_EHIP; }

}  // namespace

// =================================================================== C ABI
extern "C" {

const char* eagle3_status_string(eagle3_status s) {
  switch (s) {
    case EAGLE3_OK: return "ok";
    case EAGLE3_EINVAL: return "invalid argument";
    case EAGLE3_ECAPACITY: return "capacity exceeded";
    case EAGLE3_EUNSUPPORTED: return "unsupported";
    case EAGLE3_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

eagle3_status eagle3_kv_bytes(const eagle3_shape* s, int32_t max_batch, int32_t max_seq, size_t* tb, size_t* db) {
  if (!s || !tb || !db || max_batch < 1 || max_seq < 1) return EAGLE3_EINVAL;
  const size_t es = s->dtype == EAGLE3_BF16 ? 2 : 4;
  const size_t per = (size_t)max_batch * s->n_kv_heads * max_seq * s->head_dim * es;
  *tb = (size_t)s->n_layers * 2 * per;
  *db = 2 * per;
  return EAGLE3_OK;
}

eagle3_status eagle3_workspace_bytes(const eagle3_shape* s, const eagle3_spec_cfg* cfg, int32_t max_batch,
                                     int32_t max_rows, int32_t max_seq, size_t* bytes) {
  eagle3_status e = check_shape(s, cfg);
  if (e) return e;
  if (!bytes || max_batch < 1 || max_rows < 1 || max_seq < 1) return EAGLE3_EINVAL;
  eagle3_ctx tmp;
  tmp.sh = *s;
  tmp.cfg = *cfg;
  tmp.B = max_batch;
  tmp.R = max_rows;
  tmp.S_cap = max_seq;
  tmp.bf16 = s->dtype == EAGLE3_BF16;
  tmp.esz = tmp.bf16 ? 2 : 4;
  *bytes = carve(&tmp, nullptr);
  return EAGLE3_OK;
}

eagle3_status eagle3_paged_kv_bytes(const eagle3_shape* s, int32_t block_size, int32_t n_blocks, size_t* tb,
                                    size_t* db) {
  if (!s || !tb || !db || block_size < 64 || (block_size & (block_size - 1)) || n_blocks < 1) return EAGLE3_EINVAL;
  const size_t es = s->dtype == EAGLE3_BF16 ? 2 : 4;
  const size_t per = (size_t)n_blocks * s->n_kv_heads * block_size * s->head_dim * es;
  *tb = (size_t)s->n_layers * 2 * per;
  *db = 2 * per;
  return EAGLE3_OK;
}

namespace {

eagle3_status create_impl(const eagle3_shape* s, const eagle3_spec_cfg* cfg, const eagle3_target_weights* tw,
                          const eagle3_head_weights* hw, int32_t max_batch, int32_t max_rows, int32_t max_seq,
                          const eagle3_kv_pages* pages, void* ws, size_t ws_bytes, void* kv_t, void* kv_d,
                          void* stream, eagle3_ctx** out) {
  eagle3_status e = check_shape(s, cfg);
  if (e) return e;
  if (!tw || !hw || !out || !ws || !kv_t || !kv_d || !tw->layers || max_batch < 1 || max_rows < 1 || max_seq < 1)
    return EAGLE3_EINVAL;
  const int W = cfg->depth + 1;
  if (max_batch * W > max_rows || max_batch * cfg->topk > max_rows) return EAGLE3_ECAPACITY;
  if (!tw->embed || !tw->final_norm || !tw->lm_head) return EAGLE3_EINVAL;
  for (int l = 0; l < s->n_layers; ++l) {
    const eagle3_layer_weights& L = tw->layers[l];
    if (!L.attn_norm || !L.wq || !L.wk || !L.wv || !L.wo || !L.ffn_norm || !L.w_gate || !L.w_up || !L.w_down)
      return EAGLE3_EINVAL;
  }
  if (!hw->fc || !hw->input_norm || !hw->hidden_norm || !hw->wq || !hw->wk || !hw->wv || !hw->wo || !hw->post_norm ||
      !hw->w_gate || !hw->w_up || !hw->w_down || !hw->final_norm)
    return EAGLE3_EINVAL;
  if (s->draft_vocab > 0 && (!hw->lm_head || !hw->d2t)) return EAGLE3_EINVAL;
  eagle3_ctx* c = new (std::nothrow) eagle3_ctx();
  if (!c) return EAGLE3_EINVAL;
  c->sh = *s;
  c->cfg = *cfg;
  c->tw = *tw;
  c->layers.assign(tw->layers, tw->layers + s->n_layers);
  c->tw.layers = nullptr;
  c->hw = *hw;
  c->Vd = s->draft_vocab > 0 ? s->draft_vocab : s->vocab;
  c->dhead = s->draft_vocab > 0 ? hw->lm_head : tw->lm_head;
  c->d2t = s->draft_vocab > 0 ? hw->d2t : nullptr;
  c->B = max_batch;
  c->R = max_rows;
  c->S_cap = max_seq;
  c->bf16 = s->dtype == EAGLE3_BF16;
  c->esz = c->bf16 ? 2 : 4;
  c->st = (hipStream_t)stream;
  c->kv_t = (char*)kv_t;
  c->kv_d = (char*)kv_d;
  const size_t hd = s->head_dim, Hkv = s->n_kv_heads;
  if (pages) {
    int lbs = 0;
    while ((1 << lbs) < pages->block_size) ++lbs;
    c->pg = KvPages{pages->block_table, pages->blocks_per_seq, lbs, pages->n_blocks};
    c->kv_us = Hkv * pages->block_size * hd;
    c->kv_hs = (size_t)pages->block_size * hd;
    c->kv_le = (size_t)pages->n_blocks * c->kv_us;
  } else {
    c->kv_us = Hkv * max_seq * hd;
    c->kv_hs = (size_t)max_seq * hd;
    c->kv_le = (size_t)max_batch * c->kv_us;
  }
  const size_t need = carve(c, (char*)ws);
  if (ws_bytes < need) {
    delete c;
    return EAGLE3_ECAPACITY;
  }
  if (hipMemsetAsync(c->status, 0, 64 * sizeof(int), c->st) != hipSuccess) {
    delete c;
    return EAGLE3_EHIP;
  }
  if (c->d2t) check_d2t(c->d2t, c->Vd, s->vocab, c->status, c->st);  // a bad map raises BAD_TOKEN
  {
    // rotary inverse frequencies theta^(-2i/hd) in double
    std::vector<double> inv(s->head_dim / 2);
    for (int i = 0; i < s->head_dim / 2; ++i)
      inv[i] = std::pow((double)s->rope_theta, -2.0 * (double)i / (double)s->head_dim);
    if (hipMemcpyAsync(c->inv_freq, inv.data(), inv.size() * sizeof(double), hipMemcpyHostToDevice, c->st) !=
            hipSuccess ||
        hipStreamSynchronize(c->st) != hipSuccess) {
      delete c;
      return EAGLE3_EHIP;
    }
  }
  *out = c;
  return EAGLE3_OK;
}

}  // namespace

eagle3_status eagle3_create(const eagle3_shape* s, const eagle3_spec_cfg* cfg, const eagle3_target_weights* tw,
                            const eagle3_head_weights* hw, int32_t max_batch, int32_t max_rows, int32_t max_seq,
                            void* ws, size_t ws_bytes, void* kv_t, void* kv_d, void* stream, eagle3_ctx** out) {
  return create_impl(s, cfg, tw, hw, max_batch, max_rows, max_seq, nullptr, ws, ws_bytes, kv_t, kv_d, stream, out);
}

eagle3_status eagle3_create_paged(const eagle3_shape* s, const eagle3_spec_cfg* cfg, const eagle3_target_weights* tw,
                                  const eagle3_head_weights* hw, int32_t max_batch, int32_t max_rows,
                                  const eagle3_kv_pages* pages, void* ws, size_t ws_bytes, void* kv_t, void* kv_d,
                                  void* stream, eagle3_ctx** out) {
  if (!pages || !pages->block_table || pages->block_size < 64 || (pages->block_size & (pages->block_size - 1)) ||
      pages->n_blocks < 1 || pages->blocks_per_seq < 1)
    return EAGLE3_EINVAL;
  const long long cap = (long long)pages->blocks_per_seq * pages->block_size;
  if (cap > (1ll << 30)) return EAGLE3_EUNSUPPORTED;
  return create_impl(s, cfg, tw, hw, max_batch, max_rows, (int32_t)cap, pages, ws, ws_bytes, kv_t, kv_d, stream, out);
}

eagle3_status eagle3_set_hidden_out(eagle3_ctx* c, float* buf) {
  if (!c) return EAGLE3_EINVAL;
  c->hid_out = buf;
  return EAGLE3_OK;
}

eagle3_status eagle3_set_draft_logits_out(eagle3_ctx* c, float* table) {
  if (!c) return EAGLE3_EINVAL;
  c->dl_out = table;
  return EAGLE3_OK;
}

eagle3_status eagle3_set_draft_lengths(eagle3_ctx* c, const int32_t* n_draft) {
  if (!c) return EAGLE3_EINVAL;
  c->ndraft = n_draft;
  return EAGLE3_OK;
}

// One workgroup: request b's drafts nd' = nd clamped into [0, scheduled - 1]; an exclusive scan of nd' over the
// batch (in chunks of the block, carrying the running total) places every request's entries.
__global__ __launch_bounds__(1024) void k_spec_meta(int batch, int max_drafts, const int* __restrict__ cu,
                                                    const int* __restrict__ nd_in, const int* __restrict__ ids,
                                                    int* __restrict__ cu_nd, int* __restrict__ li, int* __restrict__ tli,
                                                    int* __restrict__ bli, int* __restrict__ dti, int* __restrict__ err) {
  __shared__ int scan[1024];
  __shared__ int s_carry, s_bad;
  const int tid = threadIdx.x;
  const int total = cu[batch - 1];  // flat positions (input_ids entries)
  if (tid == 0) {
    s_carry = 0;
    s_bad = 0;
  }
  for (int base = 0; base < batch; base += 1024) {
    __syncthreads();
    const int b = base + tid;
    int nd = 0, end = 0;
    bool bad = false;
    if (b < batch) {
      end = cu[b];
      const int sched = end - (b ? cu[b - 1] : 0);
      const int want = nd_in[b];
      nd = max(0, min(want, sched - 1));
      bad = nd != want || sched < 1;
    }
    scan[tid] = nd;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {  // inclusive scan
      const int v = tid >= o ? scan[tid - o] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int carry = s_carry;
    if (b < batch) {
      const int incl = carry + scan[tid], excl = incl - nd;
      const int first = excl + b;  // entries of logits_indices before request b
      cu_nd[b] = incl;
      bli[b] = first + nd;
      for (int t = 0; t <= nd; ++t)
        if (first + t < batch + max_drafts) li[first + t] = end - nd - 1 + t;
      for (int t = 0; t < nd; ++t)
        if (excl + t < max_drafts) {
          tli[excl + t] = first + t;
          const int src = end - nd + t;  // inside [0, total) unless cu is not increasing (flagged)
          if (dti) dti[excl + t] = src >= 0 && src < total ? ids[src] : -1;
        }
      bad = bad || incl > max_drafts;
    }
    if (bad) s_bad = 1;  // every writer stores the same value
    __syncthreads();
    if (tid == 1023) s_carry = carry + scan[1023];
  }
  __syncthreads();
  if (tid == 0 && err) err[0] = s_bad;
}

eagle3_status eagle3_spec_decode_metadata(int32_t batch, int32_t max_drafts, const int32_t* cu, const int32_t* nd,
                                          const int32_t* ids, int32_t* cu_nd, int32_t* li, int32_t* tli, int32_t* bli,
                                          int32_t* dti, int32_t* err, void* stream) {
  if (batch < 1 || max_drafts < 0 || !cu || !nd || !cu_nd || !li || !bli || (max_drafts > 0 && !tli) ||
      (dti && !ids))
    return EAGLE3_EINVAL;
  k_spec_meta<<<1, 1024, 0, (hipStream_t)stream>>>(batch, max_drafts, cu, nd, ids, cu_nd, li, tli, bli, dti, err);
  return hipGetLastError() == hipSuccess ? EAGLE3_OK : EAGLE3_EHIP;
}

eagle3_status eagle3_pack_linear(int32_t dtype, const void* src, void* dst, int32_t rows, int32_t cols,
                                 void* stream) {
  if (!src || !dst || rows < 1 || cols < 1) return EAGLE3_EINVAL;
  if (dtype != EAGLE3_F32 && dtype != EAGLE3_BF16) return EAGLE3_EINVAL;
  const bool bf = dtype == EAGLE3_BF16;
  const size_t sbytes = (size_t)rows * cols * (bf ? 2 : 4);
  const size_t dbytes = bf ? (size_t)(rows + 15) / 16 * 16 * cols * 2 : sbytes;
  const char *s0 = (const char*)src, *d0 = (const char*)dst;
  if (s0 < d0 + dbytes && d0 < s0 + sbytes) return EAGLE3_EINVAL;  // overlapping buffers
  const hipStream_t st = (hipStream_t)stream;
  if (!bf)
    return hipMemcpyAsync(dst, src, sbytes, hipMemcpyDeviceToDevice, st) == hipSuccess ? EAGLE3_OK : EAGLE3_EHIP;
  if (cols % PACK_KB) return EAGLE3_EUNSUPPORTED;
  pack_linear(src, dst, rows, cols, st);
  return hipGetLastError() == hipSuccess ? EAGLE3_OK : EAGLE3_EHIP;
}

eagle3_status eagle3_destroy(eagle3_ctx* c) {
  if (!c) return EAGLE3_EINVAL;
  for (hipEvent_t ev : c->pool) (void)hipEventDestroy(ev);
  delete c;
  return EAGLE3_OK;
}

eagle3_status eagle3_verify_tree(eagle3_ctx* c, int32_t seq_begin, int32_t batch, const int32_t* seq_lens,
                                 int32_t n_rows, const int32_t* tokens, const int32_t* pos, const uint64_t* mask,
                                 int32_t lm_mode, float* logits, int32_t* argmax, float* margin, void* aux) {
  if (!c || !seq_lens || !tokens || batch < 1 || n_rows < 1) return EAGLE3_EINVAL;
  if (seq_begin < 0 || seq_begin + batch > c->B) return EAGLE3_ECAPACITY;
  if ((size_t)batch * n_rows > (size_t)c->R) return EAGLE3_ECAPACITY;
  if (mask && n_rows > 64) return EAGLE3_EUNSUPPORTED;
  if (lm_mode < EAGLE3_LM_ALL || lm_mode > EAGLE3_LM_NONE) return EAGLE3_EINVAL;
  const int R = batch * n_rows;
  k_verify_meta<<<nb(R, 128), 128, 0, c->st>>>(batch, seq_begin, n_rows, seq_lens, tokens, pos, mask, c->S_cap,
                                                c->ndraft, c->rm, c->rtok, c->gidx, c->status);
  target_forward(c, R, n_rows, aux, lm_mode, batch, logits, argmax, margin);
  return last_error();
}

eagle3_status eagle3_draft_prefill(eagle3_ctx* c, int32_t seq_begin, int32_t batch, const int32_t* start,
                                   int32_t n_rows, const void* aux, const int32_t* next_tok) {
  if (!c || !start || !aux || !next_tok || batch < 1 || n_rows < 1) return EAGLE3_EINVAL;
  if (seq_begin < 0 || seq_begin + batch > c->B) return EAGLE3_ECAPACITY;
  if ((size_t)batch * n_rows > (size_t)c->R) return EAGLE3_ECAPACITY;
  const int R = batch * n_rows, d = c->sh.d_model;
  k_prefill_meta<<<nb(R, 128), 128, 0, c->st>>>(batch, seq_begin, n_rows, start, next_tok, c->S_cap, c->rm, c->rtok,
                                                 c->status);
  const int S = run_gemm(c, aux, R, 3 * d, make_segs(c->hw.fc, d), nullptr, true);
  draft_layer(c, R, n_rows, c->rtok, c->dx, c->rm, S);
  return last_error();
}

eagle3_status eagle3_draft_tree(eagle3_ctx* c, int32_t batch, const int32_t* seq_lens, const int32_t* new_len,
                                const void* aux_new, const int32_t* next_tok, const float* uniforms, int32_t* tokens,
                                int32_t* parents, int32_t* depth, int32_t* pos, uint64_t* mask, float* score,
                                float* q) {
  if (!c || !seq_lens || !new_len || !aux_new || !next_tok || !tokens || !parents || !depth || !pos || !mask || !score)
    return EAGLE3_EINVAL;
  if (batch < 1 || batch > c->B) return EAGLE3_ECAPACITY;
  const bool chain = c->cfg.mode == EAGLE3_SAMPLE_CHAIN;
  if (chain && ((!uniforms && !c->cfg.draft_greedy) || !q)) return EAGLE3_EINVAL;
  const eagle3_shape& s = c->sh;
  const int W = c->cfg.depth + 1, d = s.d_model;
  const int Rc = batch * W;
  hipStream_t st = c->st;
  k_catchup_meta<<<nb(Rc, 128), 128, 0, st>>>(batch, W, seq_lens, new_len, next_tok, c->S_cap, c->rm, c->rtok,
                                               c->gidx, c->roots, c->status);
  const int S = run_gemm(c, aux_new, Rc, 3 * d, make_segs(c->hw.fc, d), nullptr, true);
  draft_layer(c, Rc, W, c->rtok, c->dx, c->rm, S);
  gather_rows_f32(c->a_last, c->dx, c->gidx, batch, d, st);
  const bool kids = draft_lm(c, batch, c->a_last, chain ? 1 : c->cfg.topk, chain ? c->cfg.temperature : 1.f, 1, 0,
                             false, chain ? 0 : 1);
  TreeOut out{tokens, parents, depth, pos, mask, score};
  build_tree(c, batch, seq_lens, nullptr, uniforms, out, q, kids);
  return last_error();
}

eagle3_status eagle3_tree_from_logits(eagle3_ctx* c, int32_t batch, const int32_t* roots, const int32_t* seq_lens,
                                      const float* table, const float* uniforms, int32_t* tokens, int32_t* parents,
                                      int32_t* depth, int32_t* pos, uint64_t* mask, float* score, float* q) {
  if (!c || !roots || !seq_lens || !table || !tokens || !parents || !depth || !pos || !mask || !score)
    return EAGLE3_EINVAL;
  if (batch < 1 || batch > c->B) return EAGLE3_ECAPACITY;
  const bool chain = c->cfg.mode == EAGLE3_SAMPLE_CHAIN;
  if (chain && ((!uniforms && !c->cfg.draft_greedy) || !q)) return EAGLE3_EINVAL;
  const int Vd = c->Vd;
  const size_t tstride = (size_t)c->tab_rows * Vd;
  k_seq_roots<<<nb(batch, 64), 64, 0, c->st>>>(batch, 0, roots, c->roots);
  const int K = chain ? 1 : c->cfg.topk;
  const float T = chain ? c->cfg.temperature : 1.f;
  topk_lse(table, batch, Vd, (int)tstride, K, T, c->tk_pv, c->tk_pi, c->tk_pmax, c->tk_psum, c->tk_ids, c->tk_vals,
           c->tk_lse, c->tk_lse64, c->st);
  map_draft_ids(c->tk_ids, batch * K, c->d2t, c->Vd, c->st);
  TreeOut out{tokens, parents, depth, pos, mask, score};
  build_tree(c, batch, seq_lens, table, uniforms, out, q);
  return last_error();
}

eagle3_status eagle3_accept(eagle3_ctx* c, int32_t batch, int32_t n_rows, const int32_t* tokens,
                            const int32_t* parents, const int32_t* argmax, const float* logits, const float* q,
                            const float* uniforms, int32_t* path, int32_t* path_len, int32_t* next_root,
                            int32_t* emitted) {
  if (!c || !tokens || !path || !path_len || !next_root || batch < 1 || n_rows < 1) return EAGLE3_EINVAL;
  if (batch > c->B || n_rows > 64) return EAGLE3_ECAPACITY;
  if (c->cfg.mode == EAGLE3_GREEDY_TREE) {
    if (!parents || !argmax) return EAGLE3_EINVAL;
    accept_greedy(batch, n_rows, c->cfg.depth, tokens, parents, argmax, path, path_len, next_root, emitted, c->ndraft,
                  c->status, c->st);
  } else if (c->cfg.mode == EAGLE3_SAMPLE_TREE) {
    if (!parents || !logits || !uniforms) return EAGLE3_EINVAL;
    if ((size_t)batch * n_rows > (size_t)c->R) return EAGLE3_ECAPACITY;
    const int V = c->sh.vocab;
    topk_lse(logits, batch * n_rows, V, V, 1, c->cfg.temperature, c->tk_pv, c->tk_pi, c->tk_pmax, c->tk_psum,
             c->tk_ids, c->tk_vals, c->tk_lse, c->tk_lse64, c->st);
    accept_tree(batch, n_rows, V, c->cfg.topk, c->cfg.depth, tokens, parents, logits, c->tk_lse64, c->tk_wsum,
                c->cfg.temperature, uniforms, path, path_len, next_root, emitted, c->ndraft, c->status, c->st);
  } else {
    const int K = c->cfg.depth;
    if (n_rows != K + 1 || !logits || !q || !uniforms) return EAGLE3_EINVAL;
    if ((size_t)batch * n_rows > (size_t)c->R) return EAGLE3_ECAPACITY;
    const int V = c->sh.vocab;
    topk_lse(logits, batch * n_rows, V, V, 1, c->cfg.temperature, c->tk_pv, c->tk_pi, c->tk_pmax, c->tk_psum,
             c->tk_ids, c->tk_vals, c->tk_lse, c->tk_lse64, c->st);
    accept_chain(batch, K, V, tokens, logits, c->tk_lse64, c->cfg.temperature, q, uniforms, path, path_len, next_root,
                 emitted, c->acc_sel, c->tk_wsum, c->ndraft, c->st);
  }
  return last_error();
}

eagle3_status eagle3_compact_kv(eagle3_ctx* c, int32_t batch, int32_t* seq_lens, int32_t n_rows, const int32_t* path,
                                const int32_t* path_len, const int32_t* tokens, const int32_t* next_root,
                                const void* aux_tree, void* aux_new, int32_t* next_tok, int32_t* new_len,
                                int32_t* src_dst) {
  if (!c || !seq_lens || !path || !path_len || !tokens || !next_root || !aux_tree || !aux_new || !next_tok || !new_len)
    return EAGLE3_EINVAL;
  if (batch < 1 || batch > c->B || n_rows < 1 || n_rows > 64) return EAGLE3_ECAPACITY;
  const eagle3_shape& s = c->sh;
  const int maxp = c->cfg.depth + 1;
  compact_kv(c->bf16, batch, seq_lens, path, path_len, maxp, n_rows, c->kv_t, s.n_layers, c->kv_le, c->kv_us, c->kv_hs,
             c->pg, s.n_kv_heads, c->S_cap, s.head_dim, c->status, c->st);
  compact_finish(c->bf16, batch, seq_lens, n_rows, maxp, path, path_len, tokens, next_root, aux_tree, 3 * s.d_model,
                 aux_new, next_tok, new_len, src_dst, c->st);
  return last_error();
}

eagle3_status eagle3_sample(eagle3_ctx* c, int32_t n, const float* logits, float temperature, const float* uniforms,
                            int32_t* tokens) {
  if (!c || !logits || !tokens || n < 1 || temperature < 0.f) return EAGLE3_EINVAL;
  if (temperature > 0.f && !uniforms) return EAGLE3_EINVAL;
  if (n > c->R) return EAGLE3_ECAPACITY;
  const int V = c->sh.vocab;
  topk_lse(logits, n, V, V, 1, temperature > 0.f ? temperature : 1.f, c->tk_pv, c->tk_pi, c->tk_pmax, c->tk_psum,
           c->tk_ids, c->tk_vals, c->tk_lse, c->tk_lse64, c->st);
  sample_rows(n, logits, V, temperature, c->tk_lse64, c->tk_ids, uniforms, tokens, c->tk_wsum, c->st);
  return last_error();
}

eagle3_status eagle3_ttt_workspace_bytes(int32_t T, int32_t n_heads, int32_t head_dim, size_t* bytes) {
  if (!bytes || T < 1 || n_heads < 1 || head_dim < 4 || head_dim > 256 || head_dim % 4) return EAGLE3_EINVAL;
  *bytes = ttt_workspace_bytes(T, n_heads, head_dim);
  return EAGLE3_OK;
}

eagle3_status eagle3_ttt_attention(int32_t dtype, int32_t T, int32_t S, int32_t n_heads, int32_t n_kv_heads,
                                   int32_t head_dim, const void* q, const void* k0, const void* v0, const void* ks,
                                   const void* vs, void* out, void* ws, size_t ws_bytes, void* stream) {
  if (dtype != EAGLE3_F32 && dtype != EAGLE3_BF16) return EAGLE3_EINVAL;
  if (T < 1 || S < 0 || n_heads < 1 || n_kv_heads < 1 || n_heads % n_kv_heads || head_dim < 4 || head_dim > 256 ||
      head_dim % 4)
    return EAGLE3_EINVAL;
  if (!q || !k0 || !v0 || !out || !ws || (S > 0 && (!ks || !vs)) || ((uintptr_t)ws & 255)) return EAGLE3_EINVAL;
  if (ws_bytes < ttt_workspace_bytes(T, n_heads, head_dim)) return EAGLE3_ECAPACITY;
  ttt_attention(dtype == EAGLE3_BF16, T, S, n_heads, n_kv_heads, head_dim, q, k0, v0, ks, vs, out, ws,
                (hipStream_t)stream);
  return last_error();
}

eagle3_status eagle3_ttt_attention_static(int32_t dtype, int32_t T, int32_t S, int32_t n_heads, int32_t n_kv_heads,
                                          int32_t head_dim, const void* q, const void* k0, const void* v0,
                                          const void* ks, const void* vs, void* out, void* stream) {
  static_assert(EAGLE3_TTT_STATIC_SCRATCH_BYTES == TTT_STATIC_SCRATCH, "header and library agree on the limit");
  if (dtype != EAGLE3_F32 && dtype != EAGLE3_BF16) return EAGLE3_EINVAL;
  if (T < 1 || S < 0 || n_heads < 1 || n_kv_heads < 1 || n_heads % n_kv_heads || head_dim < 4 || head_dim > 256 ||
      head_dim % 4)
    return EAGLE3_EINVAL;
  if (!q || !k0 || !v0 || !out || (S > 0 && (!ks || !vs))) return EAGLE3_EINVAL;
  const bool bf = dtype == EAGLE3_BF16;
  if (ttt_scratch_bytes(bf, T, n_heads, head_dim) > TTT_STATIC_SCRATCH) return EAGLE3_ECAPACITY;
  void* ws = nullptr;
  if (ttt_static_scratch(&ws) != hipSuccess) return EAGLE3_EHIP;
  ttt_attention(bf, T, S, n_heads, n_kv_heads, head_dim, q, k0, v0, ks, vs, out, ws, (hipStream_t)stream);
  return last_error();
}

eagle3_status eagle3_set_stream(eagle3_ctx* c, void* stream) {
  if (!c) return EAGLE3_EINVAL;
  c->st = (hipStream_t)stream;
  return EAGLE3_OK;
}

eagle3_status eagle3_device_status(eagle3_ctx* c, int32_t* flags) {
  if (!c || !flags) return EAGLE3_EINVAL;
  int v = 0;
  if (hipMemcpyAsync(&v, c->status, sizeof(int), hipMemcpyDeviceToHost, c->st) != hipSuccess) return EAGLE3_EHIP;
  if (hipStreamSynchronize(c->st) != hipSuccess) return EAGLE3_EHIP;
  if (hipMemsetAsync(c->status, 0, sizeof(int), c->st) != hipSuccess) return EAGLE3_EHIP;
  *flags = v;
  return EAGLE3_OK;
}

eagle3_status eagle3_profile(eagle3_ctx* c, int32_t enable) {
  if (!c) return EAGLE3_EINVAL;
  if (hipStreamSynchronize(c->st) != hipSuccess) return EAGLE3_EHIP;
  c->recs.clear();
  c->pool_used = 0;
  c->prof = enable != 0;
  return EAGLE3_OK;
}

eagle3_status eagle3_profile_read(eagle3_ctx* c, int32_t kernel, int64_t* launches, double* total_ms, double* bytes,
                                  double* flops) {
  if (!c || !launches || !total_ms || !bytes || !flops || kernel < 0 || kernel >= EAGLE3_PROF_COUNT)
    return EAGLE3_EINVAL;
  if (hipStreamSynchronize(c->st) != hipSuccess) return EAGLE3_EHIP;
  int64_t n = 0;
  double ms = 0, by = 0, fl = 0;
  for (const ProfRec& r : c->recs) {
    if (r.kernel != kernel) continue;
    float t = 0.f;
    if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) return EAGLE3_EHIP;
    ++n;
    ms += t;
    by += r.bytes;
    fl += r.flops;
  }
  *launches = n;
  *total_ms = ms;
  *bytes = by;
  *flops = fl;
  return EAGLE3_OK;
}

}  // extern "C"
