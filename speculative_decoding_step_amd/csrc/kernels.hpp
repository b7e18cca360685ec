// Host-side launch wrappers of the EAGLE-3 step kernels (all on one hipStream_t).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace e3 {

// bf16 linear weights are stored in the packed slab layout read by every bf16
// GEMM kernel (k_gemm.hip): W [N, K] with K % PACK_KB == 0, rows padded with
// zeros to N16 = 16 ceil(N / 16), element (n, k) at
// ((k / 128 * (N16 / 16) + n / 16) * 4 + (k % 128) / 32) * 512
// + ((n % 16) + 16 * ((k % 32) / 8)) * 8 + k % 8.  fp32 weights stay row-major.
constexpr int PACK_KB = 128;
// dst (N16 x K elements) = the packed form of the row-major bf16 matrix src [N, K] (no overlap).
void pack_linear(const void* src, void* dst, int N, int K, hipStream_t st);

// Up to three weight matrices stacked along N (e.g. Wq;Wk;Wv), each [rows, K]
// (packed for bf16); output column of segment i starts at col0[i].
struct GemmSegs {
  const void* w[3];
  int rows[3];
  int col0[3];
  int tiles0[4];  // prefix of 64-row N tiles per segment
  int nseg;
};

// Per-slice top-k of an LM-head GEMM's logits, taken in the GEMM's epilogue:
// every workgroup owns 128 consecutive vocabulary ids (one slice) of every
// row, and writes for each row its k best (value, id) pairs to
// pv / pi [row][slice][k] and, when pmax is non-null, the slice's largest
// logit and sum of exp(z / temp - max / temp) (in double) to pmax / psum
// [row][slice].  topk_merge_slices combines the slices of each row.
struct SliceTopk {
  int k = 0;  // 0: no top-k epilogue
  int ns = 0;  // slices per row (vocabulary / 128, rounded up)
  double temp = 1.0;
  float* pv = nullptr;
  int* pi = nullptr;
  float* pmax = nullptr;
  double* psum = nullptr;
};
constexpr int TOPK_SLICE = 128;  // vocabulary ids per slice of the fused LM-head top-k

GemmSegs make_segs(const void* w0, int r0, const void* w1 = nullptr, int r1 = 0,
                   const void* w2 = nullptr, int r2 = 0);

// out[s][m][n] (split s of the K reduction) = sum_k X[m][k] W[n][k].
// Returns the number of splits used; out must hold splits * split_stride floats.
// m_tile is 16 or 64 (skinny bf16 MFMA tiles) or 128 (the large-M bf16
// kernel); ignored for float.  When
// ev_start/ev_stop are given, the bf16 launch records them at the kernel's own
// start and end (profiling).
// a_packed: X is stored in column slabs of 32 (slab32_index), which the
// large-M kernel (m_tile 128) reads; the skinny kernels read X row-major.
int gemm(bool bf16, const void* X, int M, int K, const GemmSegs& segs, float* out,
         size_t split_stride, int splits, int m_tile, hipStream_t st,
         hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr, bool a_packed = false);
// LM head with its top-k taken in the epilogue (bf16, W [V, K] packed; X
// row-major for M <= 64 rows, in column slabs of 32 above, as the large-M GEMM
// reads it): logits [M, ldo] fp32 as gemm() writes them (not written when
// logits is null), plus the per-slice candidates of tk (tk.ns = ceil(V /
// TOPK_SLICE)).  Returns false, launching nothing, when the shape is not
// covered (K not a multiple of 128, tk.k outside 1..16, more than 1024 slices).
bool gemm_lm_topk(const void* X, int M, int K, const void* W, int V, float* logits, int ldo, const SliceTopk& tk,
                  hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop);
// Merge the slices of gemm_lm_topk: the k best (value, id) of every row in
// (value desc, id asc) order, and its log-sum-exp of z / temp when pmax was
// written (lse32 / lse64 may be null).
// With kids (a draft tree level, tree.hpp) the merge also maps the ids through
// d2t (when set) and, when it computes the log-sum-exp and tk.k is the tree's
// top-k, records each row's k children as tree candidates, as tree_children
// does; returns whether it recorded them.
struct TreeKids;
bool topk_merge_slices(int R, const SliceTopk& tk, int* out_ids, float* out_vals, float* lse32, double* lse64,
                       hipStream_t st, const TreeKids* kids = nullptr);
// The large-M form of gemm_lm_topk (M > 64, X in column slabs of 32).
void gemm_big_lm_topk(const void* X, int M, int K, const void* W, int V, float* logits, int ldo, const SliceTopk& tk,
                      hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop);
// The large-M kernel behind gemm() for m_tile 128: weight rows per tile and
// K step (K must be a multiple of it); returns the number of splits used.
constexpr int GEMM_BIG_ROWS = 256, GEMM_BIG_KSTEP = 32;
int gemm_big(const void* X, int M, int K, const GemmSegs& segs, float* out, size_t split_stride, int splits,
             hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop, bool a_packed = false);
// act[m][n] = bf16(silu(X w_gate^T) * (X w_up^T)) in one GEMM launch, no partials:
// gemm_silu for bf16 with M <= 64 (skinny kernels, X and act row-major),
// gemm_big_silu for M > 64 (X and act in column slabs of 32).
void gemm_silu(const void* X, int M, int K, const void* w_gate, const void* w_up, int F, void* act, hipStream_t st,
               hipEvent_t ev_start, hipEvent_t ev_stop);
void gemm_big_silu(const void* X, int M, int K, const void* w_gate, const void* w_up, int F, void* act,
                   hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop);
// Number of K splits gemm() will actually use for a requested count.
int gemm_splits(bool bf16, int K, int splits, int m_tile);
// Weight rows per workgroup of the kernel gemm() picks.
int gemm_rows_per_tile(bool bf16, int m_tile);
int gemm_ntot(const GemmSegs& s);

// Consumers of split partials part[s][m][ldp].
void resid_add(float* x, const float* part, int S, size_t sstride, int M, int N, int ldp, hipStream_t st);
void silu_mul(bool bf16, void* out, const float* part, int S, size_t sstride, int M, int F, int ldp,
              hipStream_t st);

// Embedding rows (T) -> fp32 residual rows; invalid token -> zeros + flag.
void embed_rows(bool bf16, const void* table, const int* tokens, float* x, int R, int d, int V,
                int* status, hipStream_t st);
// out[r] = T(x[r] * rsqrt(mean(x^2)+eps) * w); if tap != null also tap[r*tap_ld] = T(x[r]).
// add_rmsnorm first adds the S split partials part[s][r][0..d) (row stride ldp) into x.
// packed: out is written in column slabs of 32 of an [R, d] matrix (a large-M GEMM input) instead of
// row-major with stride out_ld; tap is always row-major.
// rc: when rc.dst is set, each row's updated x[r] is also copied (fp32) to row
// (r / rc.k) * rc.emax + rc.slot[r] - rc.seq_lens[r / rc.k] of rc.dst (the draft
// tree's expansion rows, kept as their children's inputs).
struct RowCopy {
  float* dst = nullptr;
  const int* slot = nullptr;
  const int* seq_lens = nullptr;
  int k = 1;
  int emax = 0;
};
void add_rmsnorm(bool bf16, float* x, const float* part, int S, size_t sstride, int ldp, const void* w, void* out,
                 int out_ld, int R, int d, float eps, void* tap, int tap_ld, hipStream_t st, bool packed = false,
                 const RowCopy& rc = RowCopy{});
void rmsnorm(bool bf16, const float* x, const void* w, void* out, int out_ld, int R, int d, float eps,
             void* tap, int tap_ld, hipStream_t st, bool packed = false);
// Draft input: out[r] = [T(rms(embed[tok[r]]) * w_in) ; T(rms(x[r]) * w_hid)], [R, 2d].  With part != null
// x[r] is first set to the sum of the S split partials part[s][r][0..d) (split stride sstride): the fusion
// FC's reduction in the same pass.
// packed: out ([R, 2d]) in column slabs of 32.
// With src != null (and no partials) x[r] is first gathered from row src[r] of a_rows, or from row -1 - src[r] of
// a_last when src[r] < 0 (the tree's expansion rows take their parent's output).
void draft_input(bool bf16, const void* embed, const int* tokens, float* x, const float* part, int S,
                 size_t sstride, const void* w_in, const void* w_hid, void* out, int R, int d, int V, float eps,
                 int* status, hipStream_t st, bool packed = false, const int* src = nullptr,
                 const float* a_rows = nullptr, const float* a_last = nullptr);

// KV cache addressing of one layer's K (or V) array: element (unit u, KV head
// g, row r, dim i) sits at u * unit_stride + g * head_stride + r * hd + i.
// Contiguous ([sequences][Hkv][S_cap][hd]): position pos of sequence b is unit
// b, row pos.  Paged ([blocks][Hkv][2^lbs][hd]): it is unit bt[b * stride +
// (pos >> lbs)], row pos & (2^lbs - 1) -- the block table's slot mapping.
// Blocks hold at least 64 positions, so an attention key tile never straddles
// two blocks.  Table entries outside [0, nblk) are never dereferenced: writers
// drop the row and raise E3_DEV_KV_OVERFLOW, readers clamp (and read a wrong
// but existing block).
struct KvPages {
  const int* bt = nullptr;  // block table [sequences, stride] (device); null = contiguous
  int stride = 0;           // table entries per sequence
  int lbs = 0;              // log2 of the block size (>= 6)
  int nblk = 0;             // blocks in each pool
};
struct KvLoc {
  int unit, row;
};
// Reader's view: entries clamped into the pool.
__device__ __forceinline__ KvLoc kv_loc(const KvPages& pg, int seq, int pos) {
  if (!pg.bt) return KvLoc{seq, pos};
  const int e = pg.bt[(size_t)seq * pg.stride + (pos >> pg.lbs)];
  return KvLoc{min(max(e, 0), pg.nblk - 1), pos & ((1 << pg.lbs) - 1)};
}
// Writer's view: unit -1 when the table entry is outside the pool.
__device__ __forceinline__ KvLoc kv_loc_w(const KvPages& pg, int seq, int pos) {
  if (!pg.bt) return KvLoc{seq, pos};
  const int e = pg.bt[(size_t)seq * pg.stride + (pos >> pg.lbs)];
  return KvLoc{e >= 0 && e < pg.nblk ? e : -1, pos & ((1 << pg.lbs) - 1)};
}

// Row metadata of one forward pass.
struct RowMeta {
  int* seq;        // cache slot (sequence) of the row, -1 = padding row
  int* pos;        // RoPE position
  int* slot;       // KV slot this row writes
  int* lim;        // keys [0, lim) visible
  int* tail0;      // first slot addressed by mask bit 0
  uint64_t* mask;  // extra visible slots tail0 + j for set bits j
};

// Rotary embedding + KV write from the QKV partials [S][R][(Hq+2Hkv)*hd].
// inv_freq: [hd/2] doubles theta^(-2i/hd).  K/V of row r go to position
// rm.slot[r] of sequence rm.seq[r] through pg (unit_stride / head_stride as in
// KvPages); status receives E3_DEV_KV_OVERFLOW for a row whose block is invalid.
void rope_kv(bool bf16, const float* part, int S, size_t sstride, int R, const RowMeta& rm,
             const double* inv_freq, void* q_out, void* kc, void* vc, size_t unit_stride, size_t head_stride,
             const KvPages& pg, int Hq, int Hkv, int hd, int* status, hipStream_t st);

// Attention of rows over their visible keys, split over key chunks, then combined.
// rps: rows per sequence (rows of one sequence are consecutive; R % rps == 0).
struct AttnSplits {
  int ns, chunk;  // key chunks written, keys per chunk
  bool direct;    // one chunk: the output was written by the attention kernel (dout), no partials
};
AttnSplits attention_partials(bool bf16, const void* q, const void* kc, const void* vc, size_t unit_stride,
                              size_t head_stride, const KvPages& pg, const RowMeta& rm, int R, int rps, int Hq, int Hkv, int hd,
                              int key_bound, float* o_part, float* ml_part, int max_splits, hipStream_t st,
                              int chunk_override,  // > 0: keys per chunk (else the size policy)
                              // training-time test (bf16, hd 64 or 128, one chunk covering every key): the
                              // diagonal keys dk / dv [nstep][Hkv][R][hd] join each row's softmax and the output
                              // is written to tout [R][Hq][hd]; no partials
                              const void* dk = nullptr, const void* dv = nullptr, int nstep = 0,
                              void* tout = nullptr, const int* plan = nullptr,
                              // bf16 [R, Hq * hd] (column slabs of 32 when dpacked): output written directly
                              // when a planned launch covers every key in one chunk (AttnSplits::direct)
                              void* dout = nullptr, bool dpacked = false);
// Work order for the attention launches over rows rm (same sizes, until the row metadata changes) when they
// cover several sequences in more than one round of workgroups: writes the order to plan (ATT_PLAN_CAP ints)
// and marks the partials of work items without keys as empty in ml_part; returns false (nothing launched)
// when such launches take no plan.  Launches given the plan must follow on the same stream.
constexpr int ATT_PLAN_CHUNK = 3072;       // keys per chunk of planned launches that need several chunks
constexpr int ATT_MAX_TILES = 128;         // 64-key tiles per chunk at most (paged caches)
constexpr int ATT_PLAN_MAX_WORK = 16384;   // work items a plan orders
constexpr int ATT_PLAN_MAX_BLOCKS = 2048;  // query blocks (sequences x query blocks per sequence)
constexpr int ATT_PLAN_BINS = ATT_MAX_TILES + 1;  // key tiles per work item: 0..128
constexpr int ATT_PLAN_CAP = ATT_PLAN_MAX_WORK + 8;
bool attention_plan(bool bf16, const KvPages& pg, const RowMeta& rm, int R, int rps, int Hq, int Hkv, int hd,
                    int key_bound, int max_splits, int* plan, float* ml_part, hipStream_t st);
// Training-time-test attention: q, out [T, Hq, hd]; k0, v0 [Hkv, T, hd]; ks, vs [S, Hkv, T, hd]; ws of
// ttt_workspace_bytes(T, Hq, hd) bytes.
size_t ttt_workspace_bytes(int T, int Hq, int hd);
// Bytes of that workspace a call with these sizes actually uses (0 on the fused bf16 path).
size_t ttt_scratch_bytes(bool bf16, int T, int Hq, int hd);
// The allocation-free call's scratch: a fixed per-device array of TTT_STATIC_SCRATCH bytes; *out receives its
// device address on the current device (looked up once per device).
constexpr size_t TTT_STATIC_SCRATCH = (size_t)32 << 20;
hipError_t ttt_static_scratch(void** out);
void ttt_attention(bool bf16, int T, int S, int Hq, int Hkv, int hd, const void* q, const void* k0, const void* v0,
                   const void* ks, const void* vs, void* out, void* ws, hipStream_t st);
// out [R, Hq * hd] of T, row-major, or in column slabs of 32 when packed.
void attention(bool bf16, const void* q, const void* kc, const void* vc, size_t unit_stride,
               size_t head_stride, const KvPages& pg, const RowMeta& rm, int R, int rps, int Hq, int Hkv, int hd, int key_bound,
               float* o_part, float* ml_part, int max_splits, void* out, hipStream_t st, bool packed = false,
               const int* plan = nullptr);

// Row-wise top-k + log-sum-exp over fp32 logits [R, ld] (first V columns).
// z = logits / temperature (in double); ids/vals are of the raw logits.
void topk_lse(const float* logits, int R, int V, int ld, int K, float temperature, float* pv, int* pi,
              float* pmax, double* psum, int* out_ids, float* out_vals, float* lse32, double* lse64,
              hipStream_t st);
int topk_slices(int V);

// Gather rows: dst[i] = src[idx[i]] (fp32 rows of d) with idx < 0 -> zeros.
void gather_rows_f32(float* dst, const float* src, const int* idx, int n, int d, hipStream_t st);

}  // namespace e3
