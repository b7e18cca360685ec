// Acceptance and KV compaction.
//
// Greedy: from the root follow the child whose token equals the target's
// argmax at the current node, until none does ("Advanced speculative
// decoding: tree drafts and EAGLE", Implementation).
// Sampling (chains): accept d_i iff u_i < p_i(d_i) / q_i(d_i); at the first
// rejection draw from max(0, p_i - q_i), else draw a bonus from p_K
// ("EAGLE-3: Engineering Implementation of LLM Inference Acceleration",
// III.5, X.3-X.6).  Draws use the integer inverse CDF over
// W_v = floor(w_v * 2^48) with r = floor(u * sum W), so the pick does not
// depend on summation order.
// Sampling (trees): level by level, a node's children are tested in row
// order; each was chosen by the draft's top-k, so its draft distribution is
// the point mass at its token and it is accepted iff u < p'(x) with p' the
// node's residual; a rejection removes x's mass (norm(max(0, p' - q))); when
// every child is rejected, or the node has none, one token is drawn from the
// final residual ("Advanced speculative decoding: tree drafts and EAGLE",
// Exercises, trees under sampling).  In the same fixed point: child i is
// accepted iff floor(u * S_i) < W_x, S_i the integer mass not yet removed.
// Compaction: the accepted nodes' K/V move to consecutive slots after the
// committed prefix (the page's note on compacting KV slots).
#include "common.hpp"
#include "sampler.hpp"
#include "tree.hpp"

namespace e3 {

static inline unsigned nblk(size_t n, int b) { return (unsigned)((n + b - 1) / b); }

// Rows of sequence b's tree that take part in acceptance: the root and its
// first n_draft[b] nodes (all n_rows without per-request draft lengths).
E3_DEV int draft_rows(const int* ndraft, int b, int n_rows) {
  return ndraft ? min(max(ndraft[b], 0), n_rows - 1) + 1 : n_rows;
}

// One wave per sequence, lane i holding tree row i (n_rows <= 64): the walk
// reads the current node's argmax as a scalar and finds the matching child
// with a ballot (the lowest such index).
__global__ __launch_bounds__(64) void k_accept_greedy(int batch, int n_rows, int maxp, const int* __restrict__ tokens,
                                                      const int* __restrict__ parents, const int* __restrict__ argmax,
                                                      int* __restrict__ path, int* __restrict__ path_len,
                                                      int* __restrict__ next_root, int* __restrict__ emitted,
                                                      const int* __restrict__ ndraft, int* status) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const bool in = lane < draft_rows(ndraft, b, n_rows);
  const size_t rb = (size_t)b * n_rows;
  const int tk = in ? tokens[rb + lane] : -1;
  const int pa = in ? parents[rb + lane] : -2;
  const int am = in ? argmax[rb + lane] : -1;
  const bool bad = in && lane >= 1 && (pa < 0 || pa >= lane);
  if (__ballot(bad) != 0ull && lane == 0) raise_flag(status, E3_DEV_BAD_TREE);
  int node = 0, len = 1, mine = lane == 0 ? 0 : -1;  // lane j holds path[j]
  while (true) {
    const int pred = __builtin_amdgcn_readlane(am, node);
    const unsigned long long hit = __ballot(in && pa == node && tk == pred);
    if (hit == 0ull) break;
    if (len >= maxp) {
      if (lane == 0) raise_flag(status, E3_DEV_BAD_PATH);
      break;
    }
    const int child = __ffsll((long long)hit) - 1;
    if (lane == len) mine = child;
    ++len;
    node = child;
  }
  const int tok_mine = __shfl(tk, mine < 0 ? 0 : mine, 64);
  if (lane == 0) {
    next_root[b] = __builtin_amdgcn_readlane(am, node);
    path_len[b] = len;
  }
  for (int j = lane; j < maxp; j += 64) {
    path[(size_t)b * maxp + j] = j < len ? mine : -1;
    if (emitted) emitted[(size_t)b * maxp + j] = j < len ? tok_mine : -1;
  }
}

// Chain acceptance in three launches.  lse64[b*(K+1)+i] = log-sum-exp of row
// i's logits / T in double; p_i(v) = fl32(exp(z / T - lse)).
// k_chain_decide (one wave per sequence): the K ratio tests front to back,
// sel[b] = the number accepted.  k_chain_slices, grid (slices, B): at row
// n = sel[b], the slice sums of floor(p_n * 2^48) and, when n < K, of
// floor(max(0, p_n - q_n) * 2^48).  k_chain_pick (one 1024-thread block per
// sequence): the bonus (n = K) draws from p_K; a rejection draws from the
// residual, or from p_n when the residual is all zero in fp32; the pick comes
// from the slice sums and one slice's scan.
__global__ __launch_bounds__(64) void k_chain_decide(int K, int V, const int* __restrict__ tokens,
                                                     const float* __restrict__ logits,
                                                     const double* __restrict__ lse64, double temp,
                                                     const float* __restrict__ q, const float* __restrict__ uniforms,
                                                     const int* __restrict__ ndraft, int* __restrict__ sel) {
  const int b = blockIdx.x;
  if (threadIdx.x != 0) return;
  const int rows = K + 1, Kb = draft_rows(ndraft, b, rows) - 1;  // this request's drafts
  const int* tk = tokens + (size_t)b * rows;
  const float* u = uniforms + (size_t)b * rows;
  int n = Kb;
  for (int i = 0; i < Kb; ++i) {
    const int t = tk[i + 1];
    const float p = sample_prob(logits + ((size_t)b * rows + i) * V, t, temp, lse64[(size_t)b * rows + i]);
    const float qq = q[((size_t)b * K + i) * V + t];
    const float ratio = p / qq;
    if (!(u[i] < ratio)) {
      n = i;
      break;
    }
  }
  sel[b] = n;
}

__global__ __launch_bounds__(256) void k_chain_slices(int K, int V, const float* __restrict__ logits,
                                                      const double* __restrict__ lse64, double temp,
                                                      const float* __restrict__ q, const int* __restrict__ sel, int ns,
                                                      const int* __restrict__ ndraft,
                                                      unsigned long long* __restrict__ wsum_p,
                                                      unsigned long long* __restrict__ wsum_r) {
  __shared__ unsigned long long red[256];
  const int sl = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int rows = K + 1, n = sel[b], Kb = draft_rows(ndraft, b, rows) - 1;
  const float* z = logits + ((size_t)b * rows + n) * V;
  const double l = lse64[(size_t)b * rows + n];
  const float* qr = n < Kb ? q + ((size_t)b * K + n) * V : nullptr;  // a rejection: the residual's sums too
  const int v1 = min(V, (sl + 1) * SAMPLE_SLICE);
  unsigned long long ap = 0ull, ar = 0ull;
  for (int v = sl * SAMPLE_SLICE + tid; v < v1; v += 256) {
    const float p = sample_prob(z, v, temp, l);
    ap += int_weight_of(p);
    if (qr) ar += int_weight_of(fmaxf(p - qr[v], 0.f));
  }
  const unsigned long long tp = block_sum256(red, ap);
  const unsigned long long tr = block_sum256(red, ar);
  if (tid == 0) {
    wsum_p[(size_t)b * ns + sl] = tp;
    wsum_r[(size_t)b * ns + sl] = tr;
  }
}

__global__ __launch_bounds__(1024) void k_chain_pick(int K, int V, const int* __restrict__ tokens,
                                                     const float* __restrict__ logits,
                                                     const double* __restrict__ lse64, double temp,
                                                     const float* __restrict__ q, const float* __restrict__ uniforms,
                                                     const int* __restrict__ sel, int ns, const int* __restrict__ ndraft,
                                                     const unsigned long long* __restrict__ wsum_p,
                                                     const unsigned long long* __restrict__ wsum_r,
                                                     int* __restrict__ path, int* __restrict__ path_len,
                                                     int* __restrict__ next_root, int* __restrict__ emitted) {
  __shared__ unsigned long long scan[1024];
  __shared__ unsigned long long s_rin;
  __shared__ int s_slice, s_usep, pick;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int rows = K + 1, n = sel[b], Kb = draft_rows(ndraft, b, rows) - 1;
  const int* tk = tokens + (size_t)b * rows;
  if (tid == 0) {
    unsigned long long Sp = 0ull, Sr = 0ull;
    for (int j = 0; j < ns; ++j) {
      Sp += wsum_p[(size_t)b * ns + j];
      Sr += wsum_r[(size_t)b * ns + j];
    }
    const bool use_p = n == Kb || Sr == 0ull;  // the bonus, or a residual that is all zero in fp32
    const unsigned long long* ws = (use_p ? wsum_p : wsum_r) + (size_t)b * ns;
    const unsigned long long S = use_p ? Sp : Sr;
    const unsigned long long r = floor_u_times(S, uniform24(uniforms[(size_t)b * rows + K]));
    int slice = -1;
    unsigned long long cum = 0ull;
    for (int j = 0; j < ns && S > 0ull; ++j) {
      if (r < cum + ws[j]) {
        slice = j;
        break;
      }
      cum += ws[j];
    }
    s_slice = slice;
    s_rin = r - cum;
    s_usep = use_p;
    pick = -1;
  }
  __syncthreads();
  const int slice = s_slice;
  if (slice >= 0) {
    const float* z = logits + ((size_t)b * rows + n) * V;
    const double l = lse64[(size_t)b * rows + n];
    const float* qr = s_usep ? nullptr : q + ((size_t)b * K + n) * V;
    auto w = [&](int v) -> unsigned long long {
      const float p = sample_prob(z, v, temp, l);
      return int_weight_of(qr ? fmaxf(p - qr[v], 0.f) : p);
    };
    constexpr int PER = SAMPLE_SLICE / 1024;
    const int v0 = slice * SAMPLE_SLICE + tid * PER, v1 = min(V, v0 + PER);
    unsigned long long mine = 0ull;
    for (int v = v0; v < v1; ++v) mine += w(v);
    block_prefix(scan, mine);
    const unsigned long long r = s_rin, lo = tid ? scan[tid - 1] : 0ull;
    if (r >= lo && r < scan[tid]) {  // exactly one thread's range holds the pick
      unsigned long long acc = lo;
      for (int v = v0; v < v1; ++v) {
        acc += w(v);
        if (acc > r) {
          pick = v;
          break;
        }
      }
    }
  }
  __syncthreads();
  if (tid < rows) {
    path[(size_t)b * rows + tid] = tid <= n ? tid : -1;
    if (emitted) emitted[(size_t)b * rows + tid] = tid <= n ? tk[tid] : -1;
  }
  if (tid == 0) {
    path_len[b] = n + 1;
    next_root[b] = pick;
  }
}

// grid (slices, rows), 256 threads: wsum[row * ns + s] = sum of the integer
// weights floor(p(v) * 2^48) over slice s of the row (exact, order-free).
__global__ __launch_bounds__(256) void k_row_wsum(int V, int ns, const float* __restrict__ logits,
                                                  const double* __restrict__ lse64, double temp,
                                                  unsigned long long* __restrict__ wsum) {
  __shared__ unsigned long long red[256];
  const int s = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  const float* z = logits + (size_t)row * V;
  const double l = lse64[row];
  const int v1 = min(V, (s + 1) * SAMPLE_SLICE);
  unsigned long long acc = 0ull;
  for (int v = s * SAMPLE_SLICE + tid; v < v1; v += 256) acc += int_weight(z, v, temp, l);
  const unsigned long long tot = block_sum256(red, acc);
  if (tid == 0) wsum[(size_t)row * ns + s] = tot;
}

// One block of 1024 threads per sequence, n_rows <= 64, topk <= 64, ns <= 64,
// depth * topk + 1 <= 1024.  lse64[b*n_rows + i] = log-sum-exp of row i's logits / T in double; wsum
// [b*n_rows + i][ns] the rows' slice sums of integer weights (k_row_wsum).
// uniforms [B, maxd*topk + 1]: child i of the node at depth d uses
// uniforms[d*topk + i], the final draw uses uniforms[maxd*topk].  A visited
// node costs one weight per child; the final draw finds the slice holding
// r = floor(u * S) from the slice sums (less the rejected tokens' weights)
// and scans that slice only, so the pick is the full inverse CDF's.
__global__ __launch_bounds__(1024) void k_accept_tree(int n_rows, int V, int topk, int maxd, int ns,
                                                      const int* __restrict__ tokens, const int* __restrict__ parents,
                                                      const float* __restrict__ logits,
                                                      const double* __restrict__ lse64,
                                                      const unsigned long long* __restrict__ wsum, double temp,
                                                      const float* __restrict__ uniforms, int* __restrict__ path,
                                                      int* __restrict__ path_len, int* __restrict__ next_root,
                                                      int* __restrict__ emitted, const int* __restrict__ ndraft,
                                                      int* status) {
  __shared__ unsigned long long scan[1024];
  __shared__ unsigned long long wkid[64], wsl[64];
  __shared__ int kid[64], rej[64], pathv[64], tk[64], pa[64];
  __shared__ float u[1024];
  __shared__ unsigned long long s_rem, s_rin;
  __shared__ int s_node, s_len, s_nk, s_nrej, s_go, s_pick, s_slice;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int maxp = maxd + 1, nu = maxd * topk + 1;
  const int nr = draft_rows(ndraft, b, n_rows);  // rows of this request's draft
  // the sequence's tree and uniforms, staged once (the walk below is sequential)
  if (tid < nr) {
    const int t = tokens[(size_t)b * n_rows + tid], p = parents[(size_t)b * n_rows + tid];
    tk[tid] = t;
    pa[tid] = p;
    if (tid >= 1 && (p < 0 || p >= tid)) raise_flag(status, E3_DEV_BAD_TREE);
    if (t < 0 || t >= V) raise_flag(status, E3_DEV_BAD_TOKEN);
  }
  for (int i = tid; i < nu; i += 1024) u[i] = uniforms[(size_t)b * nu + i];
  if (tid == 0) {
    s_node = 0;
    s_len = 1;
    pathv[0] = 0;
    s_pick = -1;
  }
  while (true) {
    __syncthreads();
    const int node = s_node, len = s_len, d = len - 1;
    // the node's children in row order (only later rows, so the walk always ends); depth-maxd nodes are leaves
    if (tid == 0) {
      int nk = 0;
      if (d < maxd)
        for (int j = node + 1; j < nr; ++j)
          if (pa[j] == node) {
            if (nk < topk) kid[nk] = j;
            ++nk;
          }
      if (nk > topk) raise_flag(status, E3_DEV_BAD_TREE);
      s_nk = min(nk, topk);
    }
    __syncthreads();
    const int nk = s_nk;
    const size_t rrow = (size_t)b * n_rows + node;
    if (tid < nk) {
      const int x = tk[kid[tid]];
      wkid[tid] = (x >= 0 && x < V) ? int_weight(logits + rrow * V, x, temp, lse64[rrow]) : 0ull;
    }
    if (tid < ns) wsl[tid] = wsum[rrow * ns + tid];
    __syncthreads();
    if (tid == 0) {
      unsigned long long rem = 0ull;  // the node's integer mass, less the rejected candidates'
      for (int j = 0; j < ns; ++j) rem += wsl[j];
      int acc = -1, i = 0;
      for (; i < nk; ++i) {
        const int x = tk[kid[i]];
        bool dup = false;
        for (int j = 0; j < i; ++j) dup |= rej[j] == x;
        const unsigned long long wx = dup ? 0ull : wkid[i];
        const unsigned long long r = floor_u_times(rem, uniform24(u[d * topk + i]));
        if (r < wx) {
          acc = kid[i];
          break;
        }
        rem -= wx;
        rej[i] = x;
      }
      if (acc >= 0) {
        pathv[len] = acc;
        s_len = len + 1;
        s_node = acc;
        s_go = 1;
      } else {
        s_nrej = i;
        s_rem = rem;
        s_go = 0;
      }
    }
    __syncthreads();
    if (!s_go) break;
  }
  // final draw from the residual at the last node: its p with the rejected candidates removed
  const int node = s_node, nrej = s_nrej;
  const size_t rrow = (size_t)b * n_rows + node;
  const float* z = logits + rrow * V;
  const double l = lse64[rrow];
  if (tid == 0) {
    const unsigned long long S = s_rem;
    const unsigned long long r = floor_u_times(S, uniform24(u[(size_t)maxd * topk]));
    // remove each distinct rejected token's weight from its slice, then find the slice holding r
    for (int i = 0; i < nrej; ++i) {
      bool dup = false;
      for (int k = 0; k < i; ++k) dup |= rej[k] == rej[i];
      if (!dup && rej[i] >= 0 && rej[i] < V) wsl[rej[i] / SAMPLE_SLICE] -= wkid[i];
    }
    int slice = -1;
    unsigned long long cum = 0ull;
    for (int j = 0; j < ns && S > 0ull; ++j) {
      if (r < cum + wsl[j]) {
        slice = j;
        break;
      }
      cum += wsl[j];
    }
    s_slice = slice;
    s_rin = r - cum;
  }
  __syncthreads();
  const int slice = s_slice;
  if (slice >= 0) {
    constexpr int PER = SAMPLE_SLICE / 1024;
    const int v0 = slice * SAMPLE_SLICE + tid * PER, v1 = min(V, v0 + PER);
    auto w_res = [&](int v) -> unsigned long long {
      for (int j = 0; j < nrej; ++j)
        if (rej[j] == v) return 0ull;
      return int_weight(z, v, temp, l);
    };
    unsigned long long mine = 0ull;
    for (int v = v0; v < v1; ++v) mine += w_res(v);
    block_prefix(scan, mine);
    const unsigned long long r = s_rin, lo = tid ? scan[tid - 1] : 0ull;
    if (r >= lo && r < scan[tid]) {  // exactly one thread's range holds the pick
      unsigned long long acc = lo;
      for (int v = v0; v < v1; ++v) {
        acc += w_res(v);
        if (acc > r) {
          s_pick = v;
          break;
        }
      }
    }
  }
  __syncthreads();
  const int len = s_len;
  if (tid < maxp) {
    const int row = tid < len ? pathv[tid] : -1;
    path[(size_t)b * maxp + tid] = row;
    if (emitted) emitted[(size_t)b * maxp + tid] = row >= 0 ? tk[row] : -1;
  }
  if (tid == 0) {
    path_len[b] = len;
    next_root[b] = s_pick;
  }
}

// grid (B, L*2*Hkv): per (sequence, layer, K|V, head) move path rows to positions P..P+n-1 (through the
// block table when the cache is paged; every source row is read before any is written).
template <typename E>
__global__ __launch_bounds__(128) void k_compact_kv(const int* __restrict__ seq_lens, const int* __restrict__ path,
                                                    const int* __restrict__ path_len, int maxp, int n_rows,
                                                    E* __restrict__ kv, size_t layer_elems, size_t unit_stride,
                                                    size_t head_stride, KvPages pg, int Hkv, int S_cap, int hd,
                                                    int* status) {
  extern __shared__ unsigned char smem[];
  E* buf = (E*)smem;
  const int b = blockIdx.x, lh = blockIdx.y;
  const int lkv = lh / Hkv, g = lh % Hkv;  // lkv = layer*2 + (0 K | 1 V)
  const int P = seq_lens[b], n = path_len[b];
  const int* pb = path + (size_t)b * maxp;
  bool ok = n >= 1 && n <= maxp && pb[0] == 0;
  for (int j = 1; ok && j < n; ++j) ok = pb[j] > pb[j - 1] && pb[j] < n_rows;
  if (!ok) {
    if (threadIdx.x == 0 && lh == 0) raise_flag(status, E3_DEV_BAD_PATH);
    return;
  }
  if (P < 0 || P + pb[n - 1] >= S_cap) {
    if (threadIdx.x == 0 && lh == 0) raise_flag(status, E3_DEV_KV_OVERFLOW);
    return;
  }
  E* lay = kv + (size_t)lkv * layer_elems + (size_t)g * head_stride;
  for (int idx = threadIdx.x; idx < n * hd; idx += blockDim.x) {
    const int j = idx / hd, i = idx % hd;
    const KvLoc a = kv_loc(pg, b, P + pb[j]);
    buf[idx] = lay[(size_t)a.unit * unit_stride + (size_t)a.row * hd + i];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < n * hd; idx += blockDim.x) {
    const int j = idx / hd, i = idx % hd;
    const KvLoc a = kv_loc_w(pg, b, P + j);
    if (a.unit >= 0)
      lay[(size_t)a.unit * unit_stride + (size_t)a.row * hd + i] = buf[idx];
    else if (i == 0 && lh == 0)
      raise_flag(status, E3_DEV_KV_OVERFLOW);
  }
}

// grid (B, maxp): block (b, j) copies the aux row of path node j (if j < n)
// in 16-byte chunks; block (b, 0) also writes next_tok, new_len, the move list
// src_dst (if given) and seq_lens.
template <typename E>
__global__ __launch_bounds__(256) void k_compact_finish(int* __restrict__ seq_lens, int n_rows, int maxp,
                                                        const int* __restrict__ path, const int* __restrict__ path_len,
                                                        const int* __restrict__ tokens, const int* __restrict__ next_root,
                                                        const E* __restrict__ aux_tree, int aux_w, E* __restrict__ aux_new,
                                                        int* __restrict__ next_tok, int* __restrict__ new_len,
                                                        int* __restrict__ src_dst) {
  const int b = blockIdx.x, jrow = blockIdx.y;
  const int n = path_len[b];
  const int P = seq_lens[b];  // read by every thread before thread 0 of block (b, 0) advances it
  const int* pb = path + (size_t)b * maxp;
  bool ok = n >= 1 && n <= maxp && pb[0] == 0;
  for (int j = 1; ok && j < n; ++j) ok = pb[j] > pb[j - 1] && pb[j] < n_rows;
  if (!ok) {
    if (jrow == 0 && src_dst)
      for (int j = threadIdx.x; j < 2 * maxp; j += blockDim.x) src_dst[(size_t)b * maxp * 2 + j] = -1;
    return;
  }
  if (jrow < n) {
    const E* src = aux_tree + ((size_t)b * n_rows + pb[jrow]) * aux_w;
    E* dst = aux_new + ((size_t)b * maxp + jrow) * aux_w;
    const int bytes = aux_w * (int)sizeof(E);
    if ((bytes & 15) == 0) {
      const int n16 = bytes >> 4;
      for (int c0 = threadIdx.x; c0 < n16; c0 += 8 * blockDim.x) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int c = c0 + u * blockDim.x;
          if (c < n16) v[u] = ((const uint4*)src)[c];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int c = c0 + u * blockDim.x;
          if (c < n16) ((uint4*)dst)[c] = v[u];
        }
      }
    } else {
      for (int i = threadIdx.x; i < aux_w; i += blockDim.x) dst[i] = src[i];
    }
  }
  if (jrow != 0) return;
  for (int j = threadIdx.x; j < maxp; j += blockDim.x) {
    next_tok[(size_t)b * maxp + j] =
        j < n ? (j + 1 < n ? tokens[(size_t)b * n_rows + pb[j + 1]] : next_root[b]) : -1;
    if (src_dst) {
      src_dst[((size_t)b * maxp + j) * 2] = j < n ? P + pb[j] : -1;
      src_dst[((size_t)b * maxp + j) * 2 + 1] = j < n ? P + j : -1;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    new_len[b] = n;
    seq_lens[b] = P + n;
  }
}

void accept_greedy(int batch, int n_rows, int depth, const int* tokens, const int* parents, const int* argmax,
                   int* path, int* path_len, int* next_root, int* emitted, const int* ndraft, int* status,
                   hipStream_t st) {
  k_accept_greedy<<<batch, 64, 0, st>>>(batch, n_rows, depth + 1, tokens, parents, argmax, path, path_len, next_root,
                                        emitted, ndraft, status);
}

void accept_tree(int batch, int n_rows, int V, int topk, int depth, const int* tokens, const int* parents,
                 const float* logits, const double* lse64, unsigned long long* wsum, float temperature,
                 const float* uniforms, int* path, int* path_len, int* next_root, int* emitted, const int* ndraft,
                 int* status, hipStream_t st) {
  const int ns = sampler_slices(V);
  k_row_wsum<<<dim3(ns, batch * n_rows), 256, 0, st>>>(V, ns, logits, lse64, (double)temperature, wsum);
  k_accept_tree<<<batch, 1024, 0, st>>>(n_rows, V, topk, depth, ns, tokens, parents, logits, lse64, wsum,
                                        (double)temperature, uniforms, path, path_len, next_root, emitted, ndraft,
                                        status);
}

void accept_chain(int batch, int K, int V, const int* tokens, const float* logits, const double* lse64,
                  float temperature, const float* q, const float* uniforms, int* path, int* path_len, int* next_root,
                  int* emitted, int* sel, unsigned long long* wsum, const int* ndraft, hipStream_t st) {
  const int ns = sampler_slices(V);
  const double T = temperature;
  k_chain_decide<<<batch, 64, 0, st>>>(K, V, tokens, logits, lse64, T, q, uniforms, ndraft, sel);
  k_chain_slices<<<dim3(ns, batch), 256, 0, st>>>(K, V, logits, lse64, T, q, sel, ns, ndraft, wsum,
                                                  wsum + (size_t)batch * ns);
  k_chain_pick<<<batch, 1024, 0, st>>>(K, V, tokens, logits, lse64, T, q, uniforms, sel, ns, ndraft, wsum,
                                       wsum + (size_t)batch * ns, path, path_len, next_root, emitted);
}

void compact_kv(bool bf16, int batch, const int* seq_lens, const int* path, const int* path_len, int maxp, int n_rows,
                void* kv, int n_layers, size_t layer_elems, size_t unit_stride, size_t head_stride, const KvPages& pg,
                int Hkv, int S_cap, int hd, int* status, hipStream_t st) {
  dim3 grid(batch, n_layers * 2 * Hkv);
  if (bf16)
    k_compact_kv<uint16_t><<<grid, 128, maxp * hd * 2, st>>>(seq_lens, path, path_len, maxp, n_rows, (uint16_t*)kv,
                                                             layer_elems, unit_stride, head_stride, pg, Hkv, S_cap,
                                                             hd, status);
  else
    k_compact_kv<uint32_t><<<grid, 128, maxp * hd * 4, st>>>(seq_lens, path, path_len, maxp, n_rows, (uint32_t*)kv,
                                                             layer_elems, unit_stride, head_stride, pg, Hkv, S_cap,
                                                             hd, status);
}

void compact_finish(bool bf16, int batch, int* seq_lens, int n_rows, int maxp, const int* path, const int* path_len,
                    const int* tokens, const int* next_root, const void* aux_tree, int aux_w, void* aux_new,
                    int* next_tok, int* new_len, int* src_dst, hipStream_t st) {
  if (bf16)
    k_compact_finish<uint16_t><<<dim3(batch, maxp), 256, 0, st>>>(seq_lens, n_rows, maxp, path, path_len, tokens, next_root,
                                                      (const uint16_t*)aux_tree, aux_w, (uint16_t*)aux_new, next_tok,
                                                      new_len, src_dst);
  else
    k_compact_finish<uint32_t><<<dim3(batch, maxp), 256, 0, st>>>(seq_lens, n_rows, maxp, path, path_len, tokens, next_root,
                                                      (const uint32_t*)aux_tree, aux_w, (uint32_t*)aux_new, next_tok,
                                                      new_len, src_dst);
}

}  // namespace e3
