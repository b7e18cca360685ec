// Tree-masked grouped-query attention over the KV cache.
//
// A row r of sequence b sees the committed keys [0, lim[r]) plus the slots
// tail0[r] + j whose bit j is set in mask[r] (its tree ancestors and itself,
// "Advanced speculative decoding: tree drafts and EAGLE", Why trees:
// prefix + ancestors + self).  Query head h reads KV head h / (Hq / Hkv).
// Keys are split into chunks processed by separate workgroups; each writes an
// online-softmax partial (max, sum, unnormalised output) and the combine
// kernel merges them in chunk order.  Masked keys are skipped, not added as
// -inf.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace e3 {

constexpr int ATT_CHUNK = 256;

E3_DEV int key_end(int lim, int t0, uint64_t mask) {
  return mask ? max(lim, t0 + 64 - __clzll(mask)) : lim;
}

E3_DEV bool visible(int j, int lim, int t0, uint64_t mask) {
  return j < lim || (j >= t0 && j - t0 < 64 && ((mask >> (j - t0)) & 1ull));
}

template <typename T>
__global__ __launch_bounds__(64) void k_attn_partial(const T* __restrict__ q, const T* __restrict__ kc,
                                                     const T* __restrict__ vc, size_t seq_stride, size_t head_stride,
                                                     const int* __restrict__ rseq, const int* __restrict__ rlim,
                                                     const int* __restrict__ rt0, const uint64_t* __restrict__ rmask,
                                                     int R, int Hq, int Hkv, int hd, int S_cap, float scale,
                                                     float* __restrict__ o_part, float* __restrict__ ml_part) {
  __shared__ float qs[256];
  __shared__ float ps[ATT_CHUNK];
  const int r = blockIdx.x, h = blockIdx.y, s = blockIdx.z, lane = threadIdx.x;
  const int b = rseq[r], lim = rlim[r], t0 = rt0[r];
  const uint64_t mask = rmask[r];
  const int kend = min(key_end(lim, t0, mask), S_cap);  // never past the cache
  const int c0 = s * ATT_CHUNK, c1 = min(c0 + ATT_CHUNK, kend);
  const size_t oi = ((size_t)s * R + r) * Hq + h;
  float* op = o_part + oi * hd;
  if (b < 0 || c0 >= c1) {
    for (int i = lane; i < hd; i += 64) op[i] = 0.f;
    if (lane == 0) {
      ml_part[2 * oi] = -INFINITY;
      ml_part[2 * oi + 1] = 0.f;
    }
    return;
  }
  for (int i = lane; i < hd; i += 64) qs[i] = ld<T>(q, ((size_t)r * Hq + h) * hd + i);
  __syncthreads();
  const int g = h / (Hq / Hkv);
  const T* kb = kc + (size_t)b * seq_stride + (size_t)g * head_stride;
  const T* vb = vc + (size_t)b * seq_stride + (size_t)g * head_stride;
  float mloc = -INFINITY;
  for (int j = c0 + lane; j < c1; j += 64) {
    float sc = -INFINITY;
    if (visible(j, lim, t0, mask)) {
      float acc = 0.f;
      const T* kr = kb + (size_t)j * hd;
      for (int i = 0; i < hd; ++i) acc += qs[i] * ld<T>(kr, i);
      sc = acc * scale;
    }
    ps[j - c0] = sc;
    mloc = fmaxf(mloc, sc);
  }
  const float m = wave_max(mloc);
  float lsum = 0.f;
  for (int j = c0 + lane; j < c1; j += 64) {
    const float sc = ps[j - c0];
    const float p = (sc == -INFINITY) ? 0.f : expf(sc - m);
    ps[j - c0] = p;
    lsum += p;
  }
  const float l = wave_sum(lsum);
  __syncthreads();
  for (int i = lane; i < hd; i += 64) {
    float acc = 0.f;
    for (int j = c0; j < c1; ++j) acc += ps[j - c0] * ld<T>(vb, (size_t)j * hd + i);
    op[i] = acc;
  }
  if (lane == 0) {
    ml_part[2 * oi] = m;
    ml_part[2 * oi + 1] = l;
  }
}

// Merge the chunk partials of each (row, head): out = sum_s e_s o_s / sum_s e_s l_s
// with e_s = exp(m_s - M), M = max_s m_s, summed in chunk order.  Only the
// chunks that can hold a key the row sees are read (the row's key end comes
// from its metadata).  A workgroup covers 256 / (hd / 4) heads of one row and
// a thread one 4-dim slice of one head; the (m, l) pairs and output slices of
// up to CMB_BATCH chunks are loaded together, so a row costs two dependent
// memory round trips (metadata, then partials).  Past CMB_BATCH chunks the
// running sums are rescaled when a later batch raises the maximum.
constexpr int CMB_BATCH = 16;
template <typename T>
__global__ __launch_bounds__(256) void k_attn_combine(const float* __restrict__ o_part,
                                                      const float* __restrict__ ml_part, int ns, int R, int Hq,
                                                      int hd, const int* __restrict__ rseq,
                                                      const int* __restrict__ rlim, const int* __restrict__ rt0,
                                                      const uint64_t* __restrict__ rmask, int S_cap, int chunk,
                                                      T* __restrict__ out) {
  const int r = blockIdx.x;
  const int tph = hd >> 2;  // threads per head
  const int h = blockIdx.y * (blockDim.x / tph) + threadIdx.x / tph, d4 = threadIdx.x % tph;
  if (h >= Hq) return;  // no barrier below
  const size_t sstride = (size_t)R * Hq;  // (row, head) entries per chunk
  const size_t oi0 = (size_t)r * Hq + h;
  int nsr = 0;
  if (rseq[r] >= 0) {
    const int kend = min(key_end(rlim[r], rt0[r], rmask[r]), S_cap);
    nsr = min(ns, (kend + chunk - 1) / chunk);
  }
  const float2* ml = (const float2*)ml_part;
  const float4* o4 = (const float4*)o_part;
  float M = -INFINITY, den = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < nsr; s0 += CMB_BATCH) {
    float2 v[CMB_BATCH];
    float4 o[CMB_BATCH];
#pragma unroll
    for (int j = 0; j < CMB_BATCH; ++j) {
      const bool in = s0 + j < nsr;
      v[j] = in ? ml[(s0 + j) * sstride + oi0] : make_float2(-INFINITY, 0.f);
      o[j] = in ? o4[((s0 + j) * sstride + oi0) * tph + d4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float Mb = M;
#pragma unroll
    for (int j = 0; j < CMB_BATCH; ++j) Mb = fmaxf(Mb, v[j].x);
    if (Mb > M) {
      if (M != -INFINITY) {
        const float c = expf(M - Mb);
        den *= c;
        acc.x *= c, acc.y *= c, acc.z *= c, acc.w *= c;
      }
      M = Mb;
    }
#pragma unroll
    for (int j = 0; j < CMB_BATCH; ++j)
      if (v[j].x != -INFINITY) {
        const float e = expf(v[j].x - M);
        den += v[j].y * e;
        acc.x += o[j].x * e, acc.y += o[j].y * e, acc.z += o[j].z * e, acc.w += o[j].w * e;
      }
  }
  const size_t ob = oi0 * hd + 4 * d4;
  st<T>(out, ob, den > 0.f ? acc.x / den : 0.f);
  st<T>(out, ob + 1, den > 0.f ? acc.y / den : 0.f);
  st<T>(out, ob + 2, den > 0.f ? acc.z / den : 0.f);
  st<T>(out, ob + 3, den > 0.f ? acc.w / den : 0.f);
}

template <typename T>
void combine(const float* o_part, const float* ml_part, int ns, int R, int Hq, int hd, const RowMeta& rm,
             int key_bound, int chunk, T* out, hipStream_t st) {
  const int hpb = 256 / (hd / 4);
  k_attn_combine<T><<<dim3(R, (Hq + hpb - 1) / hpb), 256, 0, st>>>(o_part, ml_part, ns, R, Hq, hd, rm.seq, rm.lim,
                                                                   rm.tail0, rm.mask, key_bound, chunk, out);
}

// ---------------------------------------------------------------- MFMA path
// bf16 flash-decoding with grouped queries.  A workgroup of NW waves (4..8)
// owns one sequence, one KV head g, 16 NW query vectors (row i, query head
// g*G + hl, numbered i*G + hl, 16 per wave) and one chunk of keys.  Key tiles
// of 64 are staged in LDS (K row-major, V transposed) and shared by the waves;
// the next tile is loaded into registers while the current one is used.  A
// workgroup whose chunk starts past every key its rows see exits without
// writing: the combine step reads only chunks below each row's key end.
//
// Scores are computed transposed, S^T = K Q^T (v_mfma_f32_16x16x32_bf16,
// A = 16 keys, B = the wave's 16 queries), so that a lane holds four keys of
// its own query.  Those accumulator registers are then, unchanged in place,
// the B operand of O^T += V^T P^T: one 32-key MFMA step takes keys
// 4*lg + e and 16 + 4*lg + e (e = 0..3) in lane group lg, and the V^T operand
// is read from LDS in the same key order.  P enters as two bf16 terms
// (hi + lo, two MFMAs), keeping about 16 significant bits.
//
// Online softmax in base 2 with a lazy maximum: the running maximum m of a
// query is raised (and O, l rescaled) only when a tile's scaled maximum
// exceeds it by more than 8, so p = exp2(s * c - m) <= 256 (c = log2(e) /
// sqrt(hd)).  Exact in real arithmetic.  m starts at -1e30 rather than -inf so
// that masked scores (-inf) give p = 0 without a test; the partial maximum is
// stored in natural-log units (-inf when the row saw no key in the chunk).
//
// Work items (query block fastest, then KV head, key chunk, sequence) are
// dealt to the 8 XCDs in contiguous runs, so the query blocks that read the
// same K/V chunk share one L2.
constexpr int AKT = 64;  // keys per LDS tile
constexpr int VPAD = 8;  // bf16 padding per transposed-V row
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float LAZY = 8.f;     // log2 headroom before the running maximum moves
constexpr float M_EMPTY = -1e30f;

// LDS position of V(key, dim) in the transposed tile: groups of 8 keys are
// XOR-swizzled by the dimension's 8-group so that the transposing stores of
// one wave spread over the banks while 8 consecutive keys stay contiguous.
E3_DEV int vt_index(int dim, int key) {
  return dim * (AKT + VPAD) + ((((key >> 3) ^ (dim >> 3)) & 7) << 3) + (key & 7);
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int HD>
__global__ __launch_bounds__(512) void k_attn_mfma(const bf16_t* __restrict__ q, const bf16_t* __restrict__ kc,
                                                   const bf16_t* __restrict__ vc, size_t seq_stride,
                                                   size_t head_stride, const int* __restrict__ rseq,
                                                   const int* __restrict__ rlim, const int* __restrict__ rt0,
                                                   const uint64_t* __restrict__ rmask, int R, int rps, int qblocks,
                                                   int Hq, int Hkv, int ns, int nwork, int S_cap, float scale,
                                                   int chunk, float* __restrict__ o_part, float* __restrict__ ml_part) {
  __shared__ __attribute__((aligned(16))) bf16_t ks[AKT][HD + 8];
  __shared__ __attribute__((aligned(16))) bf16_t vt[HD * (AKT + VPAD)];
  __shared__ int red_end[8], red_seq[8];
  const int per = (nwork + 7) >> 3;
  const int lam = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (lam >= nwork) return;
  const int NW = blockDim.x >> 6, QB = 16 * NW;
  const int qb = lam % qblocks;
  int t = lam / qblocks;
  const int g = t % Hkv;
  t /= Hkv;
  const int sp = t % ns, bs = t / ns;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int nq = rps * G;

  // the lane's query vector: 16w + lr of the block
  const int v = qb * QB + 16 * w + lr;
  bool ok = v < nq;
  const int row = bs * rps + (ok ? v / G : 0), h = g * G + (ok ? v % G : 0);
  const int sq = ok ? rseq[row] : -1;
  ok = ok && sq >= 0;
  const int lim = rlim[row], t0 = rt0[row];
  const uint64_t mask = rmask[row];
  int my_end = ok ? min(key_end(lim, t0, mask), S_cap) : 0;
  int my_seq = ok ? sq : -1;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    my_end = max(my_end, __shfl_xor(my_end, o, 64));
    my_seq = max(my_seq, __shfl_xor(my_seq, o, 64));
  }
  if (lane == 0) {
    red_end[w] = my_end;
    red_seq[w] = my_seq;
  }
  __syncthreads();
  int kend = 0, cs = -1;
  for (int i = 0; i < NW; ++i) {
    kend = max(kend, red_end[i]);
    cs = max(cs, red_seq[i]);
  }
  const int c0 = sp * chunk, c1 = min(c0 + chunk, kend);
  if (cs < 0 || c0 >= c1) return;  // no row of the block sees a key of this chunk
  const int vis_all = ok ? min(lim, c1) : -1;  // keys below this are visible to the lane's query

  float m = M_EMPTY, lsum = 0.f;  // running maximum (log2 units) and the lane's share of the sum
  f32x4 O[HD / 16];               // O^T: dims 16b + 4lg + r of the lane's query
#pragma unroll
  for (int b = 0; b < HD / 16; ++b) O[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const float qscale = scale * LOG2E;
  u32x4 qf[HD / 32];  // B operand: the lane's query, dims 32kk + 8lg .. +7
  {
    const bf16_t* qp = q + ((size_t)row * Hq + h) * HD + 8 * lg;
#pragma unroll
    for (int kk = 0; kk < HD / 32; ++kk) qf[kk] = ok ? *(const u32x4*)(qp + 32 * kk) : u32x4{0u, 0u, 0u, 0u};
  }
  const bf16_t* kb = kc + (size_t)cs * seq_stride + (size_t)g * head_stride;
  const bf16_t* vb = vc + (size_t)cs * seq_stride + (size_t)g * head_stride;
  constexpr int CPK = HD / 8;             // 16-byte chunks per key row
  constexpr int MAXCH = AKT * CPK / 256;  // chunks per thread at 4 waves (the fewest)
  const int nt = blockDim.x;
  u32x4 kr[MAXCH], vr[MAXCH];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < MAXCH; ++i) {
      const int c = tid + nt * i, key = c / CPK, d8 = (c % CPK) * 8;
      const int j = kt + key;
      if (c < AKT * CPK && j < c1) {
        kr[i] = *(const u32x4*)(kb + (size_t)j * HD + d8);
        vr[i] = *(const u32x4*)(vb + (size_t)j * HD + d8);
      } else {
        kr[i] = u32x4{0u, 0u, 0u, 0u};
        vr[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  load_tile(c0);
  for (int kt = c0; kt < c1; kt += AKT) {
    __syncthreads();  // every wave is done with the previous tile
#pragma unroll
    for (int i = 0; i < MAXCH; ++i) {
      const int c = tid + nt * i, key = c / CPK, d8 = (c % CPK) * 8;
      if (c < AKT * CPK) {
        *(u32x4*)&ks[key][d8] = kr[i];
        const bf16_t* ve = (const bf16_t*)&vr[i];
#pragma unroll
        for (int e = 0; e < 8; ++e) vt[vt_index(d8 + e, key)] = ve[e];
      }
    }
    __syncthreads();
    if (kt + AKT < c1) load_tile(kt + AKT);  // in flight during this tile's math
    // S^T blocks: S[kb4][r] = raw score(key kt + 16 kb4 + 4 lg + r, the lane's query)
    f32x4 S[4];
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4) {
      S[kb4] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < HD / 32; ++kk) {
        const bf16x8 ak = __builtin_bit_cast(bf16x8, *(const u32x4*)&ks[16 * kb4 + lr][32 * kk + 8 * lg]);
        S[kb4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, __builtin_bit_cast(bf16x8, qf[kk]), S[kb4], 0, 0, 0);
      }
    }
    if (kt + AKT > vis_all) {  // tile reaches past the committed keys (or the lane has no query)
#pragma unroll
      for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = kt + 16 * kb4 + 4 * lg + r;
          if (!(ok && j < c1 && visible(j, lim, t0, mask))) S[kb4][r] = -INFINITY;
        }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4)
      tmax = fmaxf(tmax, fmaxf(fmaxf(S[kb4][0], S[kb4][1]), fmaxf(S[kb4][2], S[kb4][3])));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float tm = tmax * qscale;  // -inf when the tile is fully masked
    if (tm > m + LAZY) {             // same decision in the four lanes of a query
      const float alpha = __builtin_amdgcn_exp2f(m - tm);  // 0 while m is M_EMPTY
      m = tm;
      lsum *= alpha;
#pragma unroll
      for (int b = 0; b < HD / 16; ++b) O[b] *= alpha;
    }
    bf16x8 ph[2], pl[2];
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const f32x2 p{__builtin_amdgcn_exp2f(fmaf(S[kb4][r], qscale, -m)),
                      __builtin_amdgcn_exp2f(fmaf(S[kb4][r + 1], qscale, -m))};
        lsum += p[0] + p[1];
        const bf16x2 hi = __builtin_convertvector(p, bf16x2);
        const f32x2 rest = p - __builtin_convertvector(hi, f32x2);
        const bf16x2 lo = __builtin_convertvector(rest, bf16x2);
        ph[kb4 >> 1][4 * (kb4 & 1) + r] = hi[0];
        ph[kb4 >> 1][4 * (kb4 & 1) + r + 1] = hi[1];
        pl[kb4 >> 1][4 * (kb4 & 1) + r] = lo[0];
        pl[kb4 >> 1][4 * (kb4 & 1) + r + 1] = lo[1];
      }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int b = 0; b < HD / 16; ++b) {
        const int dim = 16 * b + lr;
        const u32x2 v0 = *(const u32x2*)&vt[vt_index(dim, 32 * k2 + 4 * lg)];
        const u32x2 v1 = *(const u32x2*)&vt[vt_index(dim, 32 * k2 + 16 + 4 * lg)];
        const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{v0[0], v0[1], v1[0], v1[1]});
        O[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, ph[k2], O[b], 0, 0, 0);
        O[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pl[k2], O[b], 0, 0, 0);
      }
  }
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (v < nq) {
    const size_t oi = ((size_t)sp * R + row) * Hq + h;
#pragma unroll
    for (int b = 0; b < HD / 16; ++b)
      *(f32x4*)&o_part[oi * HD + 16 * b + 4 * lg] = O[b];
    if (lg == 0) {
      ml_part[2 * oi] = m == M_EMPTY ? -INFINITY : m * LN2;
      ml_part[2 * oi + 1] = lsum;
    }
  }
}

void attention(bool bf16, const void* q, const void* kc, const void* vc, size_t seq_stride, size_t head_stride,
               const RowMeta& rm, int R, int rps, int Hq, int Hkv, int hd, int key_bound, float* o_part,
               float* ml_part, int max_splits, void* out, hipStream_t st) {
  if (R <= 0) return;
  int ns = (key_bound + ATT_CHUNK - 1) / ATT_CHUNK;
  if (ns < 1) ns = 1;
  if (ns > max_splits) ns = max_splits;  // the workspace holds ceil(max_seq / chunk) splits
  const float scale = 1.f / sqrtf((float)hd);
  if (bf16 && (hd == 64 || hd == 128) && rps > 0 && R % rps == 0) {
    const int G = Hq / Hkv;
    const int nq = rps * G;
    const int nw = std::min(8, std::max(4, (nq + 15) / 16));  // waves: 16 queries each
    const int qblocks = (nq + 16 * nw - 1) / (16 * nw);
    // Longer key chunks when the launch has work to spare: fewer partials to
    // write and merge, and each workgroup's set-up spread over more tiles.
    const long tiles256 = (long)(R / rps) * qblocks * Hkv * ns;
    const int chunk = tiles256 >= 4096 ? 3 * ATT_CHUNK : (tiles256 >= 2048 ? 2 * ATT_CHUNK : ATT_CHUNK);
    ns = (key_bound + chunk - 1) / chunk;
    const int nwork = (R / rps) * qblocks * Hkv * ns;
    const int nblocks = (nwork + 7) / 8 * 8;
    if (hd == 128)
      k_attn_mfma<128><<<nblocks, 64 * nw, 0, st>>>((const bf16_t*)q, (const bf16_t*)kc, (const bf16_t*)vc,
                                                     seq_stride, head_stride, rm.seq, rm.lim, rm.tail0, rm.mask, R,
                                                     rps, qblocks, Hq, Hkv, ns, nwork, key_bound, scale, chunk,
                                                     o_part, ml_part);
    else
      k_attn_mfma<64><<<nblocks, 64 * nw, 0, st>>>((const bf16_t*)q, (const bf16_t*)kc, (const bf16_t*)vc,
                                                    seq_stride, head_stride, rm.seq, rm.lim, rm.tail0, rm.mask, R,
                                                    rps, qblocks, Hq, Hkv, ns, nwork, key_bound, scale, chunk,
                                                    o_part, ml_part);
    combine<bf16_t>(o_part, ml_part, ns, R, Hq, hd, rm, key_bound, chunk, (bf16_t*)out, st);
    return;
  }
  dim3 grid(R, Hq, ns);
  if (bf16) {
    k_attn_partial<bf16_t><<<grid, 64, 0, st>>>((const bf16_t*)q, (const bf16_t*)kc, (const bf16_t*)vc, seq_stride,
                                                head_stride, rm.seq, rm.lim, rm.tail0, rm.mask, R, Hq, Hkv, hd,
                                                key_bound, scale, o_part, ml_part);
    combine<bf16_t>(o_part, ml_part, ns, R, Hq, hd, rm, key_bound, ATT_CHUNK, (bf16_t*)out, st);
  } else {
    k_attn_partial<float><<<grid, 64, 0, st>>>((const float*)q, (const float*)kc, (const float*)vc, seq_stride,
                                               head_stride, rm.seq, rm.lim, rm.tail0, rm.mask, R, Hq, Hkv, hd, key_bound,
                                               scale, o_part, ml_part);
    combine<float>(o_part, ml_part, ns, R, Hq, hd, rm, key_bound, ATT_CHUNK, (float*)out, st);
  }
}

}  // namespace e3
