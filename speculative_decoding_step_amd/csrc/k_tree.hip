// Draft-tree construction: candidates, frontier selection, final re-rank and
// the ancestry masks ("Advanced speculative decoding: tree drafts and EAGLE",
// Why trees and Implementation; EAGLE-2's dynamic tree as summarised in
// "EAGLE-3: Engineering Implementation of LLM Inference Acceleration", VI.7).
//
// Reading implemented (per sequence, k = topk, D = depth):
//   score(root) = 0, score(child) = fl32(score(parent) + fl32(logit - lse)),
//   children = the top-k logits of the expanded row (value desc, id asc);
//   the frontier of depth d is the k best depth-d candidates by (score desc,
//   creation index asc); after depth D the N best of all candidates are kept
//   and numbered root first, then by (depth, creation index).
// Candidate c (creation index) lives at cand[b][c]; depth-1 candidates are
// 0..k-1, those created at depth d >= 2 are k + (d-2) k^2 + rank*k + child.
// Expansion row e = (d-1) k + rank is the draft row that expanded the rank-th
// frontier node of depth d; its draft K/V sits at slot P_b + e and its tail
// mask (bits of the expansion rows on its ancestor chain and itself) is
// emask[b][e].
#include "common.hpp"
#include "sampler.hpp"
#include "tree.hpp"

namespace e3 {

static inline unsigned nblk(size_t n, int b) { return (unsigned)((n + b - 1) / b); }

// Children of the rows just expanded.  depth_new = depth of the children.
// Rows: depth_new == 1 -> one root row per sequence (row b); else k rows per
// sequence (row b*k + rank).
__global__ void k_tree_children(TreeState ts, int depth_new, const int* __restrict__ ids,
                                const float* __restrict__ vals, const float* __restrict__ lse, int kk) {
  const int k = ts.topk;
  const int per = depth_new == 1 ? k : k * k;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= ts.batch * per) return;
  const int b = i / per, j = i % per;
  const int rank = j / k, child = j % k;
  const int row = depth_new == 1 ? b : b * k + rank;
  const int base = depth_new == 1 ? 0 : k + (depth_new - 2) * k * k;
  const int c = base + j;
  const float lp = vals[(size_t)row * kk + child] - lse[row];
  float ps = 0.f;
  int par = -1;
  if (depth_new > 1) {
    par = ts.front[b * k + rank];
    ps = ts.score[(size_t)b * ts.cmax + par];
  }
  const size_t o = (size_t)b * ts.cmax + c;
  ts.tok[o] = ids[(size_t)row * kk + child];
  ts.par[o] = par;
  ts.dep[o] = depth_new;
  ts.score[o] = ps + lp;
  ts.erow[o] = -1;
}

E3_DEV bool cand_better(float sa, int ca, float sb, int cb) { return sa > sb || (sa == sb && ca < cb); }

// Frontier of depth d (the k best candidates of that depth), one block per
// sequence.  Also fills the expansion rows' draft inputs: token, parent row,
// RoPE position P + d - 1, KV slot P + e, and the tail mask.
__global__ __launch_bounds__(256) void k_tree_frontier(TreeState ts, int d, const int* __restrict__ seq_lens,
                                                       DraftRows dr, int S_cap, int* status) {
  __shared__ float sc_s[256];  // k * k <= 256 (k <= 16)
  __shared__ int tok_s[256], par_s[256], front_s[16];
  const int b = blockIdx.x, k = ts.topk;
  const int c0 = d == 1 ? 0 : k + (d - 2) * k * k;
  const int n = d == 1 ? k : k * k;
  const size_t base = (size_t)b * ts.cmax;
  const int P = seq_lens[b];
  for (int c = threadIdx.x; c < n; c += blockDim.x) {  // the level's candidates, read once
    sc_s[c] = ts.score[base + c0 + c];
    tok_s[c] = ts.tok[base + c0 + c];
    par_s[c] = ts.par[base + c0 + c];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < n; c += blockDim.x) {
    const float sc = sc_s[c];
    int rank = 0;
    for (int o = 0; o < n; ++o) rank += cand_better(sc_s[o], c0 + o, sc, c0 + c);
    if (rank < k) {
      ts.front[b * k + rank] = c0 + c;
      front_s[rank] = c;
    }
  }
  __syncthreads();
  for (int rank = threadIdx.x; rank < k; rank += blockDim.x) {
    const int cl = front_s[rank], c = c0 + cl;
    const int e = (d - 1) * k + rank;
    ts.erow[base + c] = e;
    const int par = par_s[cl];
    const int pe = par < 0 ? -1 : ts.erow[base + par];
    const uint64_t pm = pe < 0 ? 0ull : ts.emask[(size_t)b * ts.emax + pe];
    const uint64_t m = pm | (1ull << e);
    ts.emask[(size_t)b * ts.emax + e] = m;
    const int r = b * k + rank;
    const bool fits = P >= 0 && P + e < S_cap;
    if (!fits) raise_flag(status, E3_DEV_KV_OVERFLOW);
    dr.tok[r] = tok_s[cl];
    dr.src[r] = pe < 0 ? -1 - b : b * ts.emax + pe;  // -1-b: the catch-up row's a
    dr.seq[r] = fits ? b : -1;
    dr.pos[r] = P + d - 1;
    dr.slot[r] = P + e;
    dr.lim[r] = P;
    dr.tail0[r] = P;
    dr.mask[r] = m;
  }
}

// Final selection, numbering and masks, one block (512 threads) per sequence.
// The candidates are sorted in LDS (bitonic, by score descending then creation
// index ascending, as one 64-bit key); the first n_nodes are kept and numbered
// by (depth, creation index).
E3_DEV unsigned long long cand_key(float score, int c) {
  const uint32_t u = __float_as_uint(score + 0.0f);  // -0 -> +0: equal scores get equal keys
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // ascending in score
  return ((unsigned long long)(~ord) << 32) | (uint32_t)c;           // descending score, ascending index
}

__global__ __launch_bounds__(512) void k_tree_finalize(TreeState ts, int n_cand, int n_nodes,
                                                       const int* __restrict__ roots, const int* __restrict__ seq_lens,
                                                       TreeOut out, int* status) {
  __shared__ int node_of[TREE_CMAX];  // creation index -> node index (0 = not kept)
  __shared__ unsigned long long keys[TREE_CMAX];
  __shared__ int c_tok[TREE_CMAX], c_par[TREE_CMAX], c_dep[TREE_CMAX];  // the candidates, read once
  __shared__ float c_score[TREE_CMAX];
  __shared__ int pidx[65];
  const int b = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const size_t base = (size_t)b * ts.cmax;
  const int rows = n_nodes + 1;
  const int P = seq_lens[b], root = roots[b];
  int np = 1;
  while (np < n_cand) np <<= 1;  // n_cand <= TREE_CMAX (checked on the host)
  for (int c = tid; c < np; c += nt) {
    if (c < n_cand) {
      const float sc = ts.score[base + c];
      c_score[c] = sc;
      c_tok[c] = ts.tok[base + c];
      c_par[c] = ts.par[base + c];
      c_dep[c] = ts.dep[base + c];
      keys[c] = cand_key(sc, c);
    } else {
      keys[c] = ~0ull;
    }
    node_of[c] = 0;
  }
  __syncthreads();
  if (np <= nt) {
    // Bitonic sort with one key per thread: partners in the same wave (distance < 64) are exchanged by
    // shuffles, farther ones through LDS; the thread keeps the smaller key when its position and the block
    // direction agree, else the larger.
    unsigned long long key = tid < np ? keys[tid] : ~0ull;
    for (int k = 2; k <= np; k <<= 1)
      for (int j = k >> 1; j > 0; j >>= 1) {
        unsigned long long other;
        if (j >= 64) {
          __syncthreads();  // the previous exchange's reads are done
          if (tid < np) keys[tid] = key;
          __syncthreads();
          other = tid < np ? keys[tid ^ j] : key;
        } else {
          other = __shfl_xor(key, j, 64);
        }
        const bool keep_min = ((tid & j) == 0) == ((tid & k) == 0);
        key = keep_min ? (other < key ? other : key) : (other > key ? other : key);
      }
    __syncthreads();
    if (tid < np) keys[tid] = key;
    __syncthreads();
  } else {
    for (int k = 2; k <= np; k <<= 1)
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < np; i += nt) {
          const int l = i ^ j;
          if (l > i) {
            const unsigned long long x = keys[i], y = keys[l];
            if ((x > y) == ((i & k) == 0)) {
              keys[i] = y;
              keys[l] = x;
            }
          }
        }
        __syncthreads();
      }
  }
  const int nk = min(n_nodes, n_cand);  // <= 63: the kept candidates fit one wave
  if (tid < 64) {  // BFS number of kept candidate c: 1 + the kept candidates before it in (depth, creation) order
    const int c = tid < nk ? (int)(uint32_t)keys[tid] : 0;
    const int mine = tid < nk ? c_dep[c] * TREE_CMAX + c : INT_MAX;
    int pos = 1;
    for (int o = 0; o < nk; ++o) pos += __builtin_amdgcn_readlane(mine, o) < mine;
    if (tid < nk) node_of[c] = pos;
  }
  __syncthreads();
  const size_t ob = (size_t)b * rows;
  if (tid == 0) {
    out.tokens[ob] = root;
    out.parents[ob] = -1;
    out.depth[ob] = 0;
    out.pos[ob] = P;
    out.score[ob] = 0.f;
    pidx[0] = -1;
  }
  for (int c = tid; c < n_cand; c += blockDim.x) {
    const int i = node_of[c];
    if (i <= 0) continue;
    const int pc = c_par[c];
    const int pi = pc < 0 ? 0 : node_of[pc];
    if (pc >= 0 && pi <= 0) raise_flag(status, E3_DEV_BAD_TREE);
    out.tokens[ob + i] = c_tok[c];
    out.parents[ob + i] = pi;
    out.depth[ob + i] = c_dep[c];
    out.pos[ob + i] = P + c_dep[c];
    out.score[ob + i] = c_score[c];
    pidx[i] = pi;
  }
  __syncthreads();
  for (int i = tid; i < rows; i += blockDim.x) {
    uint64_t m = 0ull;
    int j = i, guard = 0;
    while (j >= 0 && guard++ <= 64) {
      m |= 1ull << j;
      j = pidx[j];
    }
    out.mask[ob + i] = m;
  }
}

// ---------------------------------------------------------------- sampled chain
// Draws one token per row from q = softmax(logits / T), in two launches.
// Logit rows are V entries long (the draft vocabulary); q rows are Vq long
// (the target vocabulary): with a reduced draft vocabulary q(v) lands at
// target id d2t[v] (the rest of the row is zeroed beforehand) and the drawn
// draft id is mapped through d2t.  Since d2t is ascending, this is the draw
// over the scattered q.
// k_draw_slices, grid (slices, rows): q(v) = fl32(exp(z_v / T - lse)) (stored
// when q_out is given) and the slice's sum of integer weights floor(q * 2^48);
// greedy rows (draft_greedy, or temperature 0) store the one-hot q of top1
// (a target id) over the Vq-long row.
// k_draw_pick, one 1024-thread block per row: r = floor(u * S) from the slice
// sums, the slice holding r, and the first entry of that slice whose prefix
// exceeds r (greedy rows: top1).
__global__ __launch_bounds__(256) void k_draw_slices(const float* __restrict__ logits, int ld, int V, int Vq,
                                                     double temp, const double* __restrict__ lse64,
                                                     const int* __restrict__ top1, int greedy,
                                                     float* __restrict__ q_out, size_t q_stride,
                                                     const int* __restrict__ d2t, int ns,
                                                     unsigned long long* __restrict__ wsum) {
  __shared__ unsigned long long red[256];
  const int sl = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  float* q = q_out ? q_out + (size_t)b * q_stride : nullptr;
  if (greedy) {
    if (q) {
      const int t = top1[b];
      const int w1 = min(Vq, (sl + 1) * SAMPLE_SLICE);
      for (int v = sl * SAMPLE_SLICE + tid; v < w1; v += 256) q[v] = v == t ? 1.f : 0.f;
    }
    return;
  }
  const int v0 = sl * SAMPLE_SLICE, v1 = min(V, v0 + SAMPLE_SLICE);
  const float* z = logits + (size_t)b * ld;
  const double l = lse64[b];
  unsigned long long acc = 0ull;
  for (int v = v0 + tid; v < v1; v += 256) {
    const float qv = sample_prob(z, v, temp, l);
    if (q) q[d2t ? d2t[v] : v] = qv;
    acc += int_weight_of(qv);
  }
  const unsigned long long tot = block_sum256(red, acc);
  if (tid == 0) wsum[(size_t)b * ns + sl] = tot;
}

__global__ __launch_bounds__(1024) void k_draw_pick(const float* __restrict__ logits, int ld, int V, double temp,
                                                    const double* __restrict__ lse64, const int* __restrict__ top1,
                                                    const float* __restrict__ uniforms, int u_stride, int greedy,
                                                    int ns, const unsigned long long* __restrict__ wsum,
                                                    const int* __restrict__ d2t, int* __restrict__ out_tok,
                                                    int tok_stride) {
  __shared__ unsigned long long scan[1024];
  __shared__ unsigned long long s_rin;
  __shared__ int s_slice, pick;
  const int b = blockIdx.x, tid = threadIdx.x;
  if (greedy) {
    if (tid == 0) out_tok[(size_t)b * tok_stride] = top1[b];
    return;
  }
  if (tid == 0) {
    unsigned long long S = 0ull;
    for (int j = 0; j < ns; ++j) S += wsum[(size_t)b * ns + j];
    const unsigned long long r = floor_u_times(S, uniform24(uniforms[(size_t)b * u_stride]));
    int slice = -1;
    unsigned long long cum = 0ull;
    for (int j = 0; j < ns && S > 0ull; ++j) {
      const unsigned long long sj = wsum[(size_t)b * ns + j];
      if (r < cum + sj) {
        slice = j;
        break;
      }
      cum += sj;
    }
    s_slice = slice;
    s_rin = r - cum;
    pick = -1;
  }
  __syncthreads();
  const int slice = s_slice;
  if (slice >= 0) {
    const float* z = logits + (size_t)b * ld;
    const double l = lse64[b];
    constexpr int PER = SAMPLE_SLICE / 1024;
    const int v0 = slice * SAMPLE_SLICE + tid * PER, v1 = min(V, v0 + PER);
    unsigned long long mine = 0ull;
    for (int v = v0; v < v1; ++v) mine += int_weight(z, v, temp, l);
    block_prefix(scan, mine);
    const unsigned long long r = s_rin, lo = tid ? scan[tid - 1] : 0ull;
    if (r >= lo && r < scan[tid]) {  // exactly one thread's range holds the pick
      unsigned long long acc = lo;
      for (int v = v0; v < v1; ++v) {
        acc += int_weight(z, v, temp, l);
        if (acc > r) {
          pick = v;
          break;
        }
      }
    }
  }
  __syncthreads();
  if (tid == 0) out_tok[(size_t)b * tok_stride] = (d2t && pick >= 0) ? d2t[pick] : pick;
}

// ids[i] <- d2t[ids[i]] (draft ids to target ids; an id outside [0, Vd) becomes -1)
__global__ void k_map_ids(int* __restrict__ ids, int n, const int* __restrict__ d2t, int Vd) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    const int id = ids[i];
    ids[i] = (id >= 0 && id < Vd) ? d2t[id] : -1;
  }
}

// d2t must hold strictly ascending ids in [0, V)
__global__ void k_check_d2t(const int* __restrict__ d2t, int Vd, int V, int* status) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= Vd) return;
  const int t = d2t[i];
  if (t < 0 || t >= V || (i > 0 && d2t[i - 1] >= t)) raise_flag(status, E3_DEV_BAD_TOKEN);
}

// rows [n] of length V at stride ld set to zero
__global__ void k_zero_rows(float* __restrict__ p, size_t ld, int V) {
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v < V) p[(size_t)blockIdx.y * ld + v] = 0.f;
}

// Chain expansion row j (0-based) of sequence b expands draft d_{j+1}.
__global__ void k_chain_rows(int j, int K, const int* __restrict__ chain_tok, const int* __restrict__ seq_lens,
                             int emax, DraftRows dr, int S_cap) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= dr.batch) return;
  const int P = seq_lens[b];
  dr.tok[b] = chain_tok[b * (K + 1) + 1 + j];
  dr.src[b] = j == 0 ? -1 - b : b * emax + (j - 1);
  dr.seq[b] = (P >= 0 && P + j < S_cap) ? b : -1;
  dr.pos[b] = P + j;
  dr.slot[b] = P + j;
  dr.lim[b] = P;
  dr.tail0[b] = P;
  dr.mask[b] = (j + 1 >= 64) ? ~0ull : ((1ull << (j + 1)) - 1ull);
}

__global__ void k_chain_finalize(int K, const int* __restrict__ roots, const int* __restrict__ seq_lens,
                                 int* __restrict__ chain_tok, TreeOut out, int batch) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= batch * (K + 1)) return;
  const int b = i / (K + 1), n = i % (K + 1);
  const int t = n == 0 ? roots[b] : chain_tok[i];
  out.tokens[i] = t;
  out.parents[i] = n - 1;
  out.depth[i] = n;
  out.pos[i] = seq_lens[b] + n;
  out.mask[i] = (n + 1 >= 64) ? ~0ull : ((1ull << (n + 1)) - 1ull);
  out.score[i] = 0.f;
}

// ------------------------------------------------------------------- launches
void tree_children(const TreeState& ts, int depth_new, const int* ids, const float* vals, const float* lse, int kk,
                   hipStream_t st) {
  const int per = depth_new == 1 ? ts.topk : ts.topk * ts.topk;
  k_tree_children<<<nblk((size_t)ts.batch * per, 128), 128, 0, st>>>(ts, depth_new, ids, vals, lse, kk);
}
void tree_frontier(const TreeState& ts, int d, const int* seq_lens, const DraftRows& dr, int S_cap, int* status,
                   hipStream_t st) {
  k_tree_frontier<<<ts.batch, 256, 0, st>>>(ts, d, seq_lens, dr, S_cap, status);
}
void tree_finalize(const TreeState& ts, int n_cand, int n_nodes, const int* roots, const int* seq_lens,
                   const TreeOut& out, int* status, hipStream_t st) {
  k_tree_finalize<<<ts.batch, 512, 0, st>>>(ts, n_cand, n_nodes, roots, seq_lens, out, status);
}
void chain_draw(int j, int K, const float* logits, int ld, int Vd, int V, float temperature, const double* lse64,
                const int* top1, const float* uniforms, int draft_greedy, float* q_out, int* chain_tok, int batch,
                unsigned long long* wsum, const int* d2t, hipStream_t st) {
  const int ns = sampler_slices(Vd);
  float* qj = q_out + (size_t)j * V;
  if (draft_greedy) {
    k_draw_slices<<<dim3(sampler_slices(V), batch), 256, 0, st>>>(logits, ld, Vd, V, (double)temperature, lse64, top1,
                                                                  1, qj, (size_t)K * V, d2t, ns, wsum);
  } else {
    if (d2t) k_zero_rows<<<dim3(nblk(V, 256), batch), 256, 0, st>>>(qj, (size_t)K * V, V);
    k_draw_slices<<<dim3(ns, batch), 256, 0, st>>>(logits, ld, Vd, V, (double)temperature, lse64, top1, 0, qj,
                                                   (size_t)K * V, d2t, ns, wsum);
  }
  k_draw_pick<<<batch, 1024, 0, st>>>(logits, ld, Vd, (double)temperature, lse64, top1, uniforms ? uniforms + j : nullptr,
                                      K, draft_greedy, ns, wsum, d2t, chain_tok + 1 + j, K + 1);
}
void sample_rows(int n, const float* logits, int V, float temperature, const double* lse64, const int* top1,
                 const float* uniforms, int* tokens, unsigned long long* wsum, hipStream_t st) {
  const int ns = sampler_slices(V), greedy = temperature == 0.f;
  if (!greedy)
    k_draw_slices<<<dim3(ns, n), 256, 0, st>>>(logits, V, V, V, (double)temperature, lse64, top1, 0, nullptr, 0,
                                               nullptr, ns, wsum);
  k_draw_pick<<<n, 1024, 0, st>>>(logits, V, V, (double)temperature, lse64, top1, uniforms, 1, greedy, ns, wsum,
                                  nullptr, tokens, 1);
}
void map_draft_ids(int* ids, int n, const int* d2t, int Vd, hipStream_t st) {
  if (d2t && n > 0) k_map_ids<<<nblk(n, 256), 256, 0, st>>>(ids, n, d2t, Vd);
}
void check_d2t(const int* d2t, int Vd, int V, int* status, hipStream_t st) {
  k_check_d2t<<<nblk(Vd, 256), 256, 0, st>>>(d2t, Vd, V, status);
}
void chain_rows(int j, int K, const int* chain_tok, const int* seq_lens, int emax, const DraftRows& dr, int S_cap,
                hipStream_t st) {
  k_chain_rows<<<nblk(dr.batch, 64), 64, 0, st>>>(j, K, chain_tok, seq_lens, emax, dr, S_cap);
}
void chain_finalize(int K, const int* roots, const int* seq_lens, int* chain_tok, const TreeOut& out, int batch,
                    hipStream_t st) {
  k_chain_finalize<<<nblk((size_t)batch * (K + 1), 128), 128, 0, st>>>(K, roots, seq_lens, chain_tok, out, batch);
}

}  // namespace e3
