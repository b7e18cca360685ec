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
#include <climits>
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace e3 {

constexpr int ATT_CHUNK = 256;

E3_DEV int key_end(int lim, int t0, uint64_t mask) {
  return mask ? max(lim, t0 + 64 - __clzll(mask)) : lim;
}

// Bitwise form (no short-circuit): callers select on the result, and the
// select must not turn into nested divergent branches (written with || and &&
// inside a divergent branch, the masked writes were lost in generated code).
E3_DEV bool visible(int j, int lim, int t0, uint64_t mask) {
  const unsigned dt = (unsigned)(j - t0);
  return (j < lim) | ((dt < 64u) & (((mask >> (dt & 63u)) & 1ull) != 0ull));
}

template <typename T>
__global__ __launch_bounds__(64) void k_attn_partial(const T* __restrict__ q, const T* __restrict__ kc,
                                                     const T* __restrict__ vc, size_t unit_stride, size_t head_stride,
                                                     KvPages pg, const int* __restrict__ rseq, const int* __restrict__ rlim,
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
  const T* kb = kc + (size_t)g * head_stride;
  const T* vb = vc + (size_t)g * head_stride;
  auto krow = [&](int j) {  // element offset of key j of sequence b
    const KvLoc at = kv_loc(pg, b, j);
    return (size_t)at.unit * unit_stride + (size_t)at.row * hd;
  };
  float mloc = -INFINITY;
  for (int j = c0 + lane; j < c1; j += 64) {
    float sc = -INFINITY;
    if (visible(j, lim, t0, mask)) {
      float acc = 0.f;
      const T* kr = kb + krow(j);
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
    for (int j = c0; j < c1; ++j) acc += ps[j - c0] * ld<T>(vb, krow(j) + i);
    op[i] = acc;
  }
  if (lane == 0) {
    ml_part[2 * oi] = m;
    ml_part[2 * oi + 1] = l;
  }
}

// Merge the chunk partials of each (row, head): out = sum_s e_s o_s / sum_s e_s l_s
// with e_s = exp(m_s - M), M = max_s m_s, summed in chunk order.  Every chunk
// has an entry for every (row, head): a chunk without keys for the row holds
// m = -inf (written by the attention kernel, also for workgroups that had no
// key at all), and its output slice is then not used.  A workgroup covers
// 256 / (hd / 4) heads of one row and a thread one 4-dim slice of one head;
// the (m, l) pairs and output slices of up to CMB_BATCH chunks are loaded
// together.  EAGER: the output slices are loaded with the (m, l) pairs, empty
// chunks included (one memory round trip per row: launches of few rows, where
// latency decides); otherwise only the non-empty chunks' slices, after the
// pairs (two round trips, no bytes spent on empty chunks: many rows of ragged
// lengths).  Past CMB_BATCH chunks the running sums are rescaled when a later
// batch raises the maximum.
constexpr int CMB_BATCH = 16;
template <typename T, bool EAGER>
__global__ __launch_bounds__(256) void k_attn_combine(const float* __restrict__ o_part,
                                                      const float* __restrict__ ml_part, int ns, int R, int Hq,
                                                      int hd, int extra, T* __restrict__ out, bool packed) {
  const int r = blockIdx.x;
  const int tph = hd >> 2;  // threads per head
  const int h = blockIdx.y * (blockDim.x / tph) + threadIdx.x / tph, d4 = threadIdx.x % tph;
  if (h >= Hq) return;  // no barrier below
  const size_t sstride = (size_t)R * Hq;  // (row, head) entries per chunk
  const size_t oi0 = (size_t)r * Hq + h;
  const float2* ml = (const float2*)ml_part;
  const float4* o4 = (const float4*)o_part;
  float M = -INFINITY, den = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < ns; s0 += CMB_BATCH) {
    float2 v[CMB_BATCH];
    float4 o[CMB_BATCH];
#pragma unroll
    for (int j = 0; j < CMB_BATCH; ++j) v[j] = s0 + j < ns ? ml[(s0 + j) * sstride + oi0] : make_float2(-INFINITY, 0.f);
#pragma unroll
    for (int j = 0; j < CMB_BATCH; ++j)
      o[j] = s0 + j < ns && (EAGER || v[j].x != -INFINITY) ? o4[((s0 + j) * sstride + oi0) * tph + d4]
                                                             : make_float4(0.f, 0.f, 0.f, 0.f);
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
      if (v[j].x != -INFINITY) {  // an empty chunk's output slice is never used (it may hold older data)
        const float e = expf(v[j].x - M);
        den += v[j].y * e;
        acc.x += o[j].x * e, acc.y += o[j].y * e, acc.z += o[j].z * e, acc.w += o[j].w * e;
      }
  }
  if (extra >= 0) {  // one more partial merged for every row (not tied to the key chunks)
    const float2 ve = ml[(size_t)extra * sstride + oi0];
    if (ve.x != -INFINITY) {
      const float4 oe = o4[((size_t)extra * sstride + oi0) * tph + d4];
      if (ve.x > M) {
        if (M != -INFINITY) {
          const float c = expf(M - ve.x);
          den *= c;
          acc.x *= c, acc.y *= c, acc.z *= c, acc.w *= c;
        }
        M = ve.x;
      }
      const float e = expf(ve.x - M);
      den += ve.y * e;
      acc.x += oe.x * e, acc.y += oe.y * e, acc.z += oe.z * e, acc.w += oe.w * e;
    }
  }
  // row r, columns h hd + 4 d4 .. + 3 of the [R, Hq hd] output: row-major, or column slabs of 32 of a
  // large-M GEMM input (the 4 columns stay inside one slab)
  const size_t ob = packed ? slab32_index(r, h * hd + 4 * d4, R) : oi0 * hd + 4 * d4;
  const float id = den > 0.f ? 1.f / den : 0.f;
  st4<T>(out, ob, make_float4(acc.x * id, acc.y * id, acc.z * id, acc.w * id));
}

template <typename T>
void combine(const float* o_part, const float* ml_part, int ns, int R, int Hq, int hd, int extra, T* out,
             hipStream_t st, bool packed = false) {
  const int hpb = 256 / (hd / 4);
  const dim3 grid(R, (Hq + hpb - 1) / hpb);
  if (R <= 256)
    k_attn_combine<T, true><<<grid, 256, 0, st>>>(o_part, ml_part, ns, R, Hq, hd, extra, out, packed);
  else
    k_attn_combine<T, false><<<grid, 256, 0, st>>>(o_part, ml_part, ns, R, Hq, hd, extra, out, packed);
}

// ---------------------------------------------------------------- MFMA path
// bf16 flash-decoding with grouped queries.  A workgroup of NW waves (4..8)
// owns one sequence, one KV head g, 16 NW query vectors (row i, query head
// g*G + hl, numbered i*G + hl, 16 per wave) and one chunk of keys.  Key tiles
// of 64 are shared by the waves through LDS.  A workgroup whose chunk starts
// past every key its rows see exits without writing: the combine step reads
// only chunks below each row's key end.
//
// Staging: every tile is copied from the KV cache straight into LDS
// (global_load_lds, 16 bytes per lane, landing in lane order), NST - 1 tiles
// ahead (four stages: the copies of tile t + 3 are issued while tile t is
// used; 128 KiB of LDS at head_dim 128), with one barrier per tile and no
// staging registers.  A copy's source is a wave-uniform base in scalar
// registers (K or V of the sequence and head, advanced a whole tile at a
// time) plus a fixed per-lane offset.  K lands in the order of the
// score product's A fragments (16 keys x 32 dims, lane l: key l % 16, dims
// 8 (l / 16) .. + 7).  V lands in blocks of 4 keys x 16 dims (128 bytes,
// keys outer); the PV product reads its transposed operand from them with
// ds_read_b64_tr_b16: when lane j of a 16-lane group points at key j / 4,
// dims 4 (j % 4) .. + 3 of a block, lane q receives the 4 keys of dim q.
// In the chunk's last tile, source rows past the chunk end are clamped to
// its last key (finite data; those keys are masked out of the scores, and a
// non-finite V row would turn the zero weight into NaN).  The copies are
// issued from inline asm and waited for explicitly: each wave issues PW
// copies per tile (indices past the tile's count repeat its last copy, an
// identical write), so the vmcnt at the top of tile t leaves exactly the
// later tiles' copies in flight.
//
// Scores are computed transposed, S^T = K Q^T (v_mfma_f32_16x16x32_bf16,
// A = 16 keys, B = the wave's 16 queries), so that a lane holds four keys of
// its own query.  Those accumulator registers are then, unchanged in place,
// the B operand of O^T += V^T P^T: one 32-key MFMA step takes keys
// 4*lg + e and 16 + 4*lg + e (e = 0..3) in lane group lg, and the V^T operand
// is read in the same key order.  P enters as two bf16 terms (hi + lo, two
// MFMAs), keeping about 16 significant bits.
//
// Masking costs nothing on tiles that every query of the wave sees whole (a
// wave-uniform test against the smallest committed length); other tiles build
// a 64-bit visibility word per query (committed prefix | shifted tree mask,
// cut at the chunk end) and select -inf per score from it.
//
// Online softmax in base 2 with a lazy maximum: the running maximum m of a
// query is raised (and O, l rescaled) only when a tile's scaled maximum
// exceeds it by more than 8, so p = exp2(s * c - m) <= 256 (c = log2(e) /
// sqrt(hd)).  Exact in real arithmetic.  The rescale runs as a wave-uniform
// branch when any query of the wave raises its maximum.  m starts at -1e30
// rather than -inf so that masked scores (-inf) give p = 0 without a test;
// the partial maximum is stored in natural-log units (-inf when the row saw
// no key in the chunk).
//
// Work items (query block fastest, then KV head, key chunk, sequence) are
// dealt to the 8 XCDs in contiguous runs, so the query blocks that read the
// same K/V chunk share one L2.
constexpr int AKT = 64;  // keys per LDS tile
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float LAZY = 8.f;     // log2 headroom before the running maximum moves
constexpr float M_EMPTY = -1e30f;

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* attn_lds_t;

// 16 bytes per lane from sbase + voff (sbase wave-uniform, voff a per-lane byte
// offset) into LDS at l + 16 * lane (l wave-uniform).
E3_DEV void attn_copy16(const void* sbase, unsigned voff, void* l) {
  const unsigned base = (unsigned)(size_t)(attn_lds_t)l;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(__builtin_amdgcn_readfirstlane(base)),
               "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// TTT: training-time test.  The rows are the positions of one sequence; after the native keys, the S simulated
// steps' diagonal keys of each row (dk / dv [S][Hkv][R][HD]) join the same softmax in the epilogue, and the
// normalised output goes straight to tout [R][Hq][HD] (the launch must cover all keys in one chunk; no partials).
template <int HD, int NW, int NST, bool TTT>
__global__ __launch_bounds__(64 * NW) void k_attn_mfma(const bf16_t* __restrict__ q, const bf16_t* __restrict__ kc,
                                                       const bf16_t* __restrict__ vc, size_t unit_stride,
                                                       size_t head_stride, KvPages pg, const int* __restrict__ rseq,
                                                       const int* __restrict__ rlim, const int* __restrict__ rt0,
                                                       const uint64_t* __restrict__ rmask, int R, int rps,
                                                       int qblocks, int Hq, int Hkv, int ns, int nwork, int S_cap,
                                                       float scale, int chunk, float* __restrict__ o_part,
                                                       float* __restrict__ ml_part, const bf16_t* __restrict__ dk,
                                                       const bf16_t* __restrict__ dv, int nstep,
                                                       bf16_t* __restrict__ tout, const int* __restrict__ plan,
                                                       bf16_t* __restrict__ dout, int dpacked) {
  constexpr int TILE = AKT * HD;               // bf16 elements of one K (or V) tile
  constexpr int NCP = 2 * TILE / 512;          // 1 KiB copies per tile: K fragments, then V block groups
  constexpr int PW = (NCP + NW - 1) / NW;      // copies per wave and tile
  constexpr int KF = HD / 32;                  // K fragments per 16-key block
  constexpr int VB = HD / 16;                  // V blocks per 4-key group
  // V: one 4-key group (VB blocks of 4 keys x 16 dims) every VGS elements.  At HD 128 a group is 1 KiB and
  // gets 128 bytes of padding, so the four 16-lane parts of a transposed read (groups 1 KiB apart otherwise)
  // fall on alternate halves of the LDS banks.  (At HD 64 one copy fills two groups back to back.)
  constexpr int VGS = VB * 64 + (HD == 128 ? 64 : 0);
  constexpr int STG = TILE + (AKT / 4) * VGS;  // elements per stage: K, then V
  __shared__ __attribute__((aligned(1024))) bf16_t stg[NST][STG];
  __shared__ int red_end[8], red_seq[8];
  const int per = (nwork + 7) >> 3;
  const int lam = plan ? plan[blockIdx.x] : (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (lam < 0 || lam >= nwork) return;
  constexpr int QB = 16 * NW;
  const int qb = qblocks - 1 - lam % qblocks;  // later query rows first: under a causal mask they see the most keys
  int t = lam / qblocks;
  const int g = t % Hkv;
  t /= Hkv;
  const int sp = t % ns, bs = t / ns;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in scalar registers
  const int nq = rps * G;

  // the lane's query vector: 16w + lr of the block
  const int v = qb * QB + 16 * w + lr;
  bool ok = v < nq;
  const int row = bs * rps + (ok ? v / G : 0), h = g * G + (ok ? v % G : 0);
  // training-time test: one sequence, row i sees native keys 0..i (no metadata arrays to read)
  const int sq = ok ? (TTT ? 0 : rseq[row]) : -1;
  ok = ok && sq >= 0;
  const int lim = TTT ? row + 1 : rlim[row], t0 = TTT ? 0 : rt0[row];
  const uint64_t mask = TTT ? 0ull : rmask[row];
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
  kend = __builtin_amdgcn_readfirstlane(kend);
  cs = __builtin_amdgcn_readfirstlane(cs);
  const int c0 = sp * chunk, c1 = min(c0 + chunk, kend);
  if (cs < 0 || c0 >= c1) {  // no row of the block sees a key of this chunk: an empty partial for each row
    if (!TTT && dout && v < nq) {  // one chunk per row: the row's output is zero
#pragma unroll
      for (int b = 0; b < HD / 16; ++b) {
        const int col = h * HD + 16 * b + 4 * lg;
        *(uint2*)(dout + (dpacked ? slab32_index(row, col, R) : (size_t)row * Hq * HD + col)) = make_uint2(0u, 0u);
      }
    } else if (!TTT && v < nq && lg == 0) {
      const size_t oi = ((size_t)sp * R + row) * Hq + h;
      ml_part[2 * oi] = -INFINITY;
      ml_part[2 * oi + 1] = 0.f;
    }
    return;
  }
  // Keys below vis_min are visible to every query of the wave, so tiles below it need no mask (a wave-uniform
  // test).  Lanes without a query vector never force masking (their results are not stored); rows without a
  // sequence see no key.
  int vis_min = v >= nq ? INT_MAX : (ok ? min(lim, c1) : -1);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) vis_min = min(vis_min, __shfl_xor(vis_min, o, 64));
  vis_min = __builtin_amdgcn_readfirstlane(vis_min);

  // Tile kt's keys start at kb/vb + tile_off(kt): contiguous, the sequence's unit advanced by kt rows; paged, the
  // block the table gives for kt (a block holds whole 64-key tiles).  The chunk's block ids are loaded once, lane i
  // holding tile i's and tile 64 + i's (a chunk has at most 128 tiles), and each tile reads its id with readlane:
  // no memory wait in the copy ring.
  const bool paged = pg.bt != nullptr;
  const size_t seq0 = paged ? 0 : (size_t)cs * unit_stride;
  const bf16_t* kb = kc + seq0 + (size_t)g * head_stride;
  const bf16_t* vb = vc + seq0 + (size_t)g * head_stride;
  int vblk = 0, vblk_hi = 0;
  if (paged) {
    const int nt = (c1 - c0 + AKT - 1) >> 6;
    if (lane < nt) vblk = min(max(pg.bt[(size_t)cs * pg.stride + ((c0 + AKT * lane) >> pg.lbs)], 0), pg.nblk - 1);
    if (lane + 64 < nt)
      vblk_hi = min(max(pg.bt[(size_t)cs * pg.stride + ((c0 + AKT * (lane + 64)) >> pg.lbs)], 0), pg.nblk - 1);
  }
  auto tile_off = [&](int kt) -> size_t {
    if (!paged) return (size_t)kt * HD;
    const int i = (kt - c0) >> 6;  // wave-uniform
    const int e = i < 64 ? __builtin_amdgcn_readlane(vblk, i) : __builtin_amdgcn_readlane(vblk_hi, i - 64);
    return (size_t)e * unit_stride + (size_t)(kt & ((1 << pg.lbs) - 1)) * HD;
  };
  // this wave's copies of a tile: index f = w + NW i (i < PW), clamped to the last one; the source is a
  // wave-uniform base (K or V of this sequence and head, advanced by whole tiles) plus a per-lane offset
  const bf16_t* cbase[PW];
  unsigned voff[PW];
  int dst[PW], ckey[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int f = min(w + NW * i, NCP - 1);
    int key, d0;
    if (f < NCP / 2) {  // K fragment (16-key block kb4, dims 32 kk ..): lane: key lr, dims 8 lg ..
      const int kb4 = f / KF, kk = f % KF;
      key = 16 * kb4 + lr;
      d0 = 32 * kk + 8 * lg;
      dst[i] = f * 512;
    } else {  // V blocks 8 (f - NCP / 2) .. + 7: lane: block + l / 8, key 2-chunk (l % 8) / 2, dim half l % 2
      const int bi = 8 * (f - NCP / 2) + (lane >> 3), c = lane & 7;
      key = 4 * (bi / VB) + (c >> 1);
      d0 = 16 * (bi % VB) + 8 * (c & 1);
      dst[i] = TILE + (f - NCP / 2) * (512 / (VB * 64)) * VGS;
    }
    ckey[i] = key;  // key within the tile
    cbase[i] = f < NCP / 2 ? kb : vb;
    voff[i] = (unsigned)(key * HD + d0) * 2u;
  }
  auto issue = [&](bf16_t* stgp, int kt) {
    const size_t to = tile_off(kt);
    if (kt + AKT <= c1) {  // whole tile inside the chunk
#pragma unroll
      for (int i = 0; i < PW; ++i) attn_copy16(cbase[i] + to, voff[i], stgp + dst[i]);
    } else {  // the chunk's last tile: rows past its end repeat its last key (finite data, masked out)
#pragma unroll
      for (int i = 0; i < PW; ++i) {
        const int back = kt + ckey[i] - min(kt + ckey[i], c1 - 1);  // rows moved back, >= 0
        attn_copy16(cbase[i] + to, voff[i] - (unsigned)(back * HD * 2), stgp + dst[i]);
      }
    }
  };

  // The first NST - 1 tiles' copies go out before the query loads, so their latencies overlap (the query
  // must be complete before the first tile, which waits for everything issued so far anyway).
  const int ntl = (c1 - c0 + AKT - 1) / AKT;
  for (int t = 0; t < NST - 1 && t < ntl; ++t) issue(stg[t], c0 + t * AKT);

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
  // Complete the query loads (and the first tiles' copies issued above) here, visibly to the compiler: its own
  // wait for them would otherwise land inside the tile loop, where (not seeing the asm copies) it would drain
  // every tile in flight.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  auto tile = [&](const bf16_t* stgp, int kt) {
    const bf16_t* ks = stgp + 8 * lane;                                 // + constant fragment offsets
    const bf16_t* vs = stgp + TILE + lg * VGS + 4 * lr;                // + constant block offsets
    // S^T blocks: S[kb4][r] = raw score(key kt + 16 kb4 + 4 lg + r, the lane's query)
    f32x4 S[4];
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4) {
      S[kb4] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KF; ++kk) {
        const bf16x8 ak = __builtin_bit_cast(bf16x8, *(const u32x4*)(ks + (kb4 * KF + kk) * 512));
        S[kb4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, __builtin_bit_cast(bf16x8, qf[kk]), S[kb4], 0, 0, 0);
      }
    }
    if (kt + AKT > vis_min) {  // some query of the wave does not see every key of the tile (wave-uniform)
      // visibility of keys kt .. kt + 63 for the lane's query, one bit per key: the committed prefix, the
      // tree slots t0 + j (bit j of mask), cut at the chunk end.  Every select below is branch-free.
      const int np = lim - kt, d = t0 - kt, ne = c1 - kt;  // ne >= 1
      const uint64_t pre = np >= 64 ? ~0ull : (np <= 0 ? 0ull : (1ull << np) - 1ull);
      const uint64_t tr = (d >= 64 || d <= -64) ? 0ull : (d >= 0 ? mask << d : mask >> -d);
      const uint64_t end = ne >= 64 ? ~0ull : (1ull << ne) - 1ull;
      uint64_t vis = (pre | tr) & end;
      vis = v >= nq ? ~0ull : (ok ? vis : 0ull);
      const uint64_t vl = vis >> (4 * lg);  // bit 16 kb4 + r: key kt + 16 kb4 + 4 lg + r
#pragma unroll
      for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[kb4][r] = ((vl >> (16 * kb4 + r)) & 1ull) ? S[kb4][r] : -INFINITY;
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4)
      tmax = fmaxf(tmax, fmaxf(fmaxf(S[kb4][0], S[kb4][1]), fmaxf(S[kb4][2], S[kb4][3])));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float tm = tmax * qscale;  // -inf when the tile is fully masked
    const bool raise = tm > m + LAZY;  // same decision in the four lanes of a query
    if (__builtin_amdgcn_ballot_w64(raise)) {  // wave-uniform: rare once the maxima have settled
      const float mn = raise ? tm : m;
      const float alpha = __builtin_amdgcn_exp2f(m - mn);  // 1 where the maximum stays, 0 while m is M_EMPTY
      m = mn;
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
        ph[kb4 >> 1][4 * (kb4 & 1) + r] = hi[0];
        ph[kb4 >> 1][4 * (kb4 & 1) + r + 1] = hi[1];
        if constexpr (!TTT) {  // the verify path keeps P's low half too (two MFMAs, ~16 significant bits)
          const f32x2 rest = p - __builtin_convertvector(hi, f32x2);
          const bf16x2 lo = __builtin_convertvector(rest, bf16x2);
          pl[kb4 >> 1][4 * (kb4 & 1) + r] = lo[0];
          pl[kb4 >> 1][4 * (kb4 & 1) + r + 1] = lo[1];
        }
      }
    // V^T operand of dim block b, keys {32 k2 + 4 lg + e} then {32 k2 + 16 + 4 lg + e}: the 4-key groups
    // 8 k2 + lg and 8 k2 + 4 + lg, read transposed (lane lr points at 4 lr elements into the block; the
    // lane's part of the address is in vs)
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int b = 0; b < HD / 16; ++b) {
        const bf16_t* b0 = vs + 8 * k2 * VGS + b * 64;
        const bf16_t* b1 = vs + (8 * k2 + 4) * VGS + b * 64;
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(attn_lds_t)b0);
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(attn_lds_t)b1);
        const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{__builtin_bit_cast(u32x2, v0)[0], __builtin_bit_cast(u32x2, v0)[1],
                                                           __builtin_bit_cast(u32x2, v1)[0], __builtin_bit_cast(u32x2, v1)[1]});
        O[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, ph[k2], O[b], 0, 0, 0);
        if constexpr (!TTT) O[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pl[k2], O[b], 0, 0, 0);
      }
  };

  // NST-stage ring: tile t lives in stage t % NST and its copies are issued NST - 1 tiles ahead.  At the top
  // of tile t this wave has issued the copies of tiles 0 .. min(ntl - 1, t + NST - 2), PW per tile, in order,
  // so vmcnt(PW * a) with a = min(NST - 2, ntl - 1 - t) tiles issued after t means tile t has landed.  The
  // barrier then publishes every wave's copies of tile t and guarantees that all waves finished tile t - 1,
  // whose stage the copies of tile t + NST - 1 refill.
  static_assert(NST >= 2 && NST <= 4, "the wait below covers at most two tiles in flight after the current one");
  static_assert(PW * (NST - 2) <= 63, "copies in flight exceed the vmcnt range");
  for (int t = 0; t < ntl; ++t) {
    const int after = min(NST - 2, ntl - 1 - t);
    if (after >= 2)
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * PW) : "memory");
    else if (after == 1)
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(PW) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (t + NST - 1 < ntl) issue(stg[(t + NST - 1) % NST], c0 + (t + NST - 1) * AKT);
    tile(stg[t % NST], c0 + t * AKT);
  }

  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if constexpr (TTT) {
    // Each simulated step's diagonal key of the lane's position: the score from the lane's quarter of the query
    // (the B operand: dims 32 kk + 8 lg ..) summed over the query's four lanes, then an online-softmax update of
    // (m, lsum, O) with the matching value (the lane's output dims 16 b + 4 lg + r).  All lanes take part in
    // the exchanges; lanes without a query read row `row` (a valid one) and store nothing.
    for (int js = 0; js < nstep; ++js) {
      const size_t base = (((size_t)js * Hkv + g) * R + row) * HD;
      const bf16_t* kp = dk + base + 8 * lg;
      float dot = 0.f;
#pragma unroll
      for (int kk = 0; kk < HD / 32; ++kk) {
        const u32x4 kv = *(const u32x4*)(kp + 32 * kk);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dot = fmaf(__uint_as_float(qf[kk][e] << 16), __uint_as_float(kv[e] << 16), dot);
          dot = fmaf(__uint_as_float(qf[kk][e] & 0xffff0000u), __uint_as_float(kv[e] & 0xffff0000u), dot);
        }
      }
      dot += __shfl_xor(dot, 16, 64);
      dot += __shfl_xor(dot, 32, 64);
      const float sc = dot * qscale;  // log2 units, like m
      const float mn = fmaxf(m, sc);
      const float alpha = __builtin_amdgcn_exp2f(m - mn), p = __builtin_amdgcn_exp2f(sc - mn);
      m = mn;
      lsum = fmaf(lsum, alpha, p);
      const bf16_t* vp = dv + base + 4 * lg;
#pragma unroll
      for (int b = 0; b < HD / 16; ++b) {
        const uint2 raw = *(const uint2*)(vp + 16 * b);
        O[b][0] = fmaf(O[b][0], alpha, p * __uint_as_float(raw.x << 16));
        O[b][1] = fmaf(O[b][1], alpha, p * __uint_as_float(raw.x & 0xffff0000u));
        O[b][2] = fmaf(O[b][2], alpha, p * __uint_as_float(raw.y << 16));
        O[b][3] = fmaf(O[b][3], alpha, p * __uint_as_float(raw.y & 0xffff0000u));
      }
    }
    if (v < nq && ok) {
      const float inv = 1.f / lsum;
      bf16_t* op = tout + ((size_t)row * Hq + h) * HD + 4 * lg;
#pragma unroll
      for (int b = 0; b < HD / 16; ++b) {
        uint2 w;
        w.x = (uint32_t)f2bf(O[b][0] * inv) | ((uint32_t)f2bf(O[b][1] * inv) << 16);
        w.y = (uint32_t)f2bf(O[b][2] * inv) | ((uint32_t)f2bf(O[b][3] * inv) << 16);
        *(uint2*)(op + 16 * b) = w;
      }
    }
    return;
  }
  if (dout) {  // one chunk covers every key: the normalised output (zero for a row that sees no key)
    if (v < nq) {
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
      for (int b = 0; b < HD / 16; ++b) {
        const int col = h * HD + 16 * b + 4 * lg;
        uint2 w;
        w.x = (uint32_t)f2bf(O[b][0] * inv) | ((uint32_t)f2bf(O[b][1] * inv) << 16);
        w.y = (uint32_t)f2bf(O[b][2] * inv) | ((uint32_t)f2bf(O[b][3] * inv) << 16);
        *(uint2*)(dout + (dpacked ? slab32_index(row, col, R) : (size_t)row * Hq * HD + col)) = w;
      }
    }
    return;
  }
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

template <int HD, int NST, bool TTT>
void launch_attn(int nw, unsigned nblocks, hipStream_t st, const bf16_t* q, const bf16_t* kc, const bf16_t* vc,
                 size_t unit_stride, size_t head_stride, const KvPages& pg, const RowMeta& rm, int R, int rps,
                 int qblocks, int Hq, int Hkv, int ns, int nwork, int key_bound, float scale, int chunk,
                 float* o_part, float* ml_part, const bf16_t* dk, const bf16_t* dv, int nstep, bf16_t* tout,
                 const int* plan, bf16_t* dout, int dpacked) {
#define E3_ATTN_LAUNCH(N)                                                                                             \
  k_attn_mfma<HD, N, NST, TTT><<<nblocks, 64 * N, 0, st>>>(q, kc, vc, unit_stride, head_stride, pg, rm.seq, rm.lim,   \
                                                      rm.tail0, rm.mask, R, rps, qblocks, Hq, Hkv, ns, nwork,       \
                                                      key_bound, scale, chunk, o_part, ml_part, dk, dv, nstep, tout, \
                                                      plan, dout, dpacked)
  switch (nw) {
    case 4: E3_ATTN_LAUNCH(4); break;
    case 5: E3_ATTN_LAUNCH(5); break;
    case 6: E3_ATTN_LAUNCH(6); break;
    case 7: E3_ATTN_LAUNCH(7); break;
    default: E3_ATTN_LAUNCH(8); break;
  }
#undef E3_ATTN_LAUNCH
}

// Launch geometry of the MFMA path: waves per workgroup, query blocks per
// sequence, keys per chunk, chunk slots and work items.  mfma false: the
// scalar kernel runs (ns chunks of ATT_CHUNK).
struct AttnGeom {
  bool mfma = false, planned = false, direct = false;
  int nw = 0, qblocks = 0, chunk = ATT_CHUNK, ns = 1, nwork = 0;
  unsigned nblocks = 0;
};

AttnGeom attn_geom(bool bf16, const KvPages& pg, int R, int rps, int Hq, int Hkv, int hd, int key_bound,
                   int max_splits, int chunk_override, bool ttt, bool can_direct) {
  AttnGeom g;
  g.ns = std::min(std::max(1, (key_bound + ATT_CHUNK - 1) / ATT_CHUNK), max_splits);
  if (!(bf16 && (hd == 64 || hd == 128) && rps > 0 && R % rps == 0)) return g;
  g.mfma = true;
  const int G = Hq / Hkv, nq = rps * G, nseq = R / rps;
  g.nw = std::min(8, std::max(4, (nq + 15) / 16));  // waves: 16 queries each
  g.qblocks = (nq + 16 * g.nw - 1) / (16 * g.nw);
  // Longer key chunks when the launch has work to spare: fewer partials to
  // write and merge, and each workgroup's set-up spread over more tiles.
  const long tiles256 = (long)nseq * g.qblocks * Hkv * g.ns;
  int chunk = chunk_override > 0 ? chunk_override
              : tiles256 >= 8192 ? 6 * ATT_CHUNK
              : tiles256 >= 4096 ? 3 * ATT_CHUNK
              : tiles256 >= 2048 ? 2 * ATT_CHUNK
                                 : ATT_CHUNK;
  if (pg.bt && chunk > ATT_MAX_TILES * AKT) chunk = ATT_MAX_TILES * AKT;  // paged: block ids in two registers
  // Several sequences over more than one round of workgroups: their lengths
  // differ, so the work is ordered by a plan (largest items first, spread over
  // the XCDs).  When one chunk per (query block, KV head) still gives a full
  // round of work items and covers every key, each item writes its rows'
  // normalised output itself (no partials, no merge); otherwise chunks of
  // ATT_PLAN_CHUNK keys.
  if (chunk_override <= 0 && !ttt && nseq > 1 && tiles256 >= 2048 && (long)nseq * g.qblocks <= ATT_PLAN_MAX_BLOCKS) {
    const int one = (key_bound + AKT - 1) / AKT * AKT;
    const long w1 = (long)nseq * g.qblocks * Hkv;
    const int pc = can_direct && one <= ATT_MAX_TILES * AKT && w1 >= 512 ? one : ATT_PLAN_CHUNK;
    const int pns = (key_bound + pc - 1) / pc;
    const long pwork = w1 * pns;
    if (pwork >= 512 && pwork <= ATT_PLAN_MAX_WORK && pns <= max_splits) {
      g.planned = true;
      g.direct = pns == 1 && can_direct;
      chunk = pc;
    }
  }
  g.chunk = chunk;
  g.ns = (key_bound + chunk - 1) / chunk;
  g.nwork = nseq * g.qblocks * Hkv * g.ns;
  g.nblocks = (unsigned)((g.nwork + 7) / 8 * 8);
  return g;
}

// Work order of the tree-attention launches over several sequences
// (blockIdx.x > 0: one query block each; blockIdx.x = 0: the order).
//
// A work item (query block, KV head, key chunk) costs about its number of key
// tiles.  The order sorts the non-empty items by tile count, largest first
// (equal counts in item order), and deals rank i to XCD x(i) in a serpentine
// over the 8 XCDs (x = i mod 8, reversed on odd rounds), at position i / 8 of
// that XCD's queue: workgroup 8 (i / 8) + x(i) runs it, since workgroup j runs
// on XCD j mod 8.  Each XCD gets nearly the same tiles and, within it, its
// largest items first.  Unused positions hold -1 (the workgroup exits).
//
// Items with no key (chunks past the end of a query block's keys) are left
// out of the order; their partials are marked empty here (m = -inf, l = 0),
// once for every launch over the same rows, so the combine skips them: every
// (row, head, chunk) entry is written either here or by its one work item.
// Both sides compute a query block's key end and sequence exactly as the
// attention kernel does.
//
// keep_empty (one chunk per item, each writing its rows' output): the items
// without keys stay in the order, after all others, since they write zeros.
__global__ __launch_bounds__(1024) void k_attn_plan(const int* __restrict__ rseq, const int* __restrict__ rlim,
                                                    const int* __restrict__ rt0, const uint64_t* __restrict__ rmask,
                                                    int R, int rps, int qblocks, int QB, int G, int Hq, int Hkv,
                                                    int ns, int nwork, int S_cap, int chunk, int nblocks,
                                                    int keep_empty, int* __restrict__ plan,
                                                    float* __restrict__ ml_part) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nq = rps * G, nbq = (R / rps) * qblocks;
  // key end and sequence of query block b (largest over its query vectors, as the attention kernel takes them)
  auto vec_end = [&](int b, int i, int* end, int* seq) {
    const int bs = b / qblocks, qb = b % qblocks, v = qb * QB + i;
    *end = 0;
    *seq = -1;
    if (i >= QB || v >= nq) return;
    const int row = bs * rps + v / G;
    const int sq = rseq[row], lim = rlim[row], t0 = rt0[row];  // loaded together: one memory round trip
    const uint64_t mk = rmask[row];
    if (sq < 0) return;
    *end = min(key_end(lim, t0, mk), S_cap);
    *seq = sq;
  };
  if (blockIdx.x > 0) {  // the empty partials of query block b
    __shared__ int b_end, b_seq;
    const int b = blockIdx.x - 1;
    if (tid == 0) {
      b_end = 0;
      b_seq = -1;
    }
    __syncthreads();
    for (int i = tid; i < QB; i += blockDim.x) {
      int e, sq;
      vec_end(b, i, &e, &sq);
      if (sq >= 0) {
        atomicMax(&b_end, e);
        atomicMax(&b_seq, sq);
      }
    }
    __syncthreads();
    const int kend = b_end, bs = b / qblocks, qb = b % qblocks;
    const int sp0 = b_seq < 0 ? 0 : min(ns, (kend + chunk - 1) / chunk);  // chunks sp0.. have no key
    const int nv = min(QB, nq - qb * QB);
    const int total = (ns - sp0) * Hkv * nv;
    for (int i = tid; i < total; i += blockDim.x) {
      const int vi = i % nv, t = i / nv, g = t % Hkv, sp = sp0 + t / Hkv;
      const int v = qb * QB + vi, row = bs * rps + v / G, h = g * G + v % G;
      const size_t oi = ((size_t)sp * R + row) * Hq + h;
      *(float2*)&ml_part[2 * oi] = make_float2(-INFINITY, 0.f);
    }
    return;
  }
  __shared__ int s_end[ATT_PLAN_MAX_BLOCKS], s_seq[ATT_PLAN_MAX_BLOCKS];
  __shared__ unsigned char s_tiles[ATT_PLAN_MAX_WORK];
  __shared__ int s_cnt[ATT_PLAN_BINS], s_start[ATT_PLAN_BINS], s_run[ATT_PLAN_BINS];
  __shared__ int s_wcnt[16][ATT_PLAN_BINS];
  __shared__ int s_nreal;
  for (int b = tid; b < nbq; b += blockDim.x) {
    s_end[b] = 0;
    s_seq[b] = -1;
  }
  for (int i = tid; i < ATT_PLAN_BINS; i += blockDim.x) {
    s_cnt[i] = 0;
    s_run[i] = 0;
  }
  for (int i = tid; i < 16 * ATT_PLAN_BINS; i += blockDim.x) s_wcnt[i / ATT_PLAN_BINS][i % ATT_PLAN_BINS] = 0;
  __syncthreads();
  // per row (its G query vectors lie in one or two query blocks of its sequence)
  for (int r = tid; r < R; r += blockDim.x) {
    const int sq = rseq[r], lim = rlim[r], t0 = rt0[r];
    const uint64_t mk = rmask[r];
    if (sq < 0) continue;
    const int e = min(key_end(lim, t0, mk), S_cap), bs = r / rps, v0 = (r - bs * rps) * G;
    for (int qb = v0 / QB; qb <= (v0 + G - 1) / QB; ++qb) {
      atomicMax(&s_end[bs * qblocks + qb], e);
      atomicMax(&s_seq[bs * qblocks + qb], sq);
    }
  }
  __syncthreads();
  // tiles of item lam, decoded as the attention kernel decodes it
  for (int lam = tid; lam < nwork; lam += blockDim.x) {
    const int qb = qblocks - 1 - lam % qblocks;
    const int t = lam / qblocks / Hkv;
    const int sp = t % ns, bs = t / ns, b = bs * qblocks + qb;
    const int c0 = sp * chunk, c1 = min(c0 + chunk, s_end[b]);
    const int tiles = (s_seq[b] < 0 || c0 >= c1) ? 0 : min((c1 - c0 + AKT - 1) / AKT, ATT_PLAN_BINS - 1);
    s_tiles[lam] = (unsigned char)tiles;
    if (tiles || keep_empty) atomicAdd(&s_cnt[tiles], 1);
  }
  __syncthreads();
  if (w == 0) {  // bin starts, largest tile count first: an exclusive scan over the bins in descending order
    static_assert(3 * 64 >= ATT_PLAN_BINS, "three bins per lane");
    int v[3], sum = 0;
#pragma unroll
    for (int e = 0; e < 3; ++e) {
      const int t = ATT_PLAN_BINS - 1 - (3 * lane + e);
      v[e] = t >= 0 ? s_cnt[t] : 0;
      sum += v[e];
    }
    int inc = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    int ex = inc - sum;
#pragma unroll
    for (int e = 0; e < 3; ++e) {
      const int t = ATT_PLAN_BINS - 1 - (3 * lane + e);
      if (t >= 0) s_start[t] = ex;
      ex += v[e];
    }
    if (lane == 63) s_nreal = inc;
  }
  __syncthreads();
  auto slot = [](int i) {
    const int r = i >> 3, j = i & 7;
    return 8 * r + ((r & 1) ? 7 - j : j);
  };
  // ranks: bin start + items of the same tile count before this one (earlier passes, earlier waves, lower lanes)
  for (int base = 0; base < nwork; base += blockDim.x) {
    const int lam = base + tid;
    int t = lam < nwork ? s_tiles[lam] : -1;
    if (t == 0 && !keep_empty) t = -1;  // left out of the order
    unsigned long long todo = __ballot(t >= 0);
    int rank = 0;
    while (todo) {  // one round per distinct tile count in the wave
      const int leader = __ffsll((long long)todo) - 1;
      const int tk = __shfl(t, leader, 64);
      const unsigned long long m = __ballot(t == tk);
      if (t == tk) rank = __popcll(m & ((1ull << lane) - 1ull));
      if (lane == leader) s_wcnt[w][tk] = __popcll(m);
      todo &= ~m;
    }
    __syncthreads();
    if (t >= 0) {
      int off = s_run[t];
      for (int u = 0; u < w; ++u) off += s_wcnt[u][t];
      plan[slot(s_start[t] + off + rank)] = lam;
    }
    __syncthreads();
    if (tid < ATT_PLAN_BINS) {
      int sum = 0;
      for (int u = 0; u < 16; ++u) {
        sum += s_wcnt[u][tid];
        s_wcnt[u][tid] = 0;
      }
      s_run[tid] += sum;
    }
    __syncthreads();
  }
  for (int i = s_nreal + tid; i < nblocks; i += blockDim.x) plan[slot(i)] = -1;
}

bool attention_plan(bool bf16, const KvPages& pg, const RowMeta& rm, int R, int rps, int Hq, int Hkv, int hd,
                    int key_bound, int max_splits, int* plan, float* ml_part, hipStream_t st) {
  if (R <= 0 || !plan) return false;
  const AttnGeom g = attn_geom(bf16, pg, R, rps, Hq, Hkv, hd, key_bound, max_splits, 0, false, true);
  if (!g.planned) return false;
  const int nbq = (R / rps) * g.qblocks;
  // direct output: no partials to mark, every item stays in the order
  k_attn_plan<<<g.direct ? 1 : 1 + nbq, 1024, 0, st>>>(rm.seq, rm.lim, rm.tail0, rm.mask, R, rps, g.qblocks,
                                                       16 * g.nw, Hq / Hkv, Hq, Hkv, g.ns, g.nwork, key_bound, g.chunk,
                                                       (int)g.nblocks, g.direct ? 1 : 0, plan, ml_part);
  return true;
}

// The chunk partials of tree-masked attention (o_part / ml_part, chunk-major);
// returns the number of key chunks written and their length.
AttnSplits attention_partials(bool bf16, const void* q, const void* kc, const void* vc, size_t unit_stride,
                              size_t head_stride, const KvPages& pg, const RowMeta& rm, int R, int rps, int Hq, int Hkv,
                              int hd,
                              int key_bound, float* o_part, float* ml_part, int max_splits, hipStream_t st,
                              int chunk_override, const void* dk, const void* dv, int nstep, void* tout,
                              const int* plan, void* dout, bool dpacked) {
  const AttnGeom g = attn_geom(bf16, pg, R, rps, Hq, Hkv, hd, key_bound, max_splits, chunk_override, tout != nullptr,
                               dout != nullptr);
  const float scale = 1.f / sqrtf((float)hd);
  if (g.mfma) {
    const int nw = g.nw, qblocks = g.qblocks, ns = g.ns, nwork = g.nwork, chunk = g.chunk;
    const unsigned nblocks = g.nblocks;
    const int* pl = g.planned ? plan : nullptr;  // a plan made for this geometry (attention_plan) or none
    bf16_t* dot = g.direct ? (bf16_t*)dout : nullptr;
#define E3_ATTN_ARGS                                                                                                \
  nw, nblocks, st, (const bf16_t*)q, (const bf16_t*)kc, (const bf16_t*)vc, unit_stride, head_stride, pg, rm, R, rps,   \
      qblocks, Hq, Hkv, ns, nwork, key_bound, scale, chunk, o_part, ml_part, (const bf16_t*)dk, (const bf16_t*)dv,      \
      nstep, (bf16_t*)tout, pl, dot, dpacked ? 1 : 0
    if (tout) {  // training-time test: diagonal keys merged in the epilogue, output written directly
      if (hd == 128)
        launch_attn<128, 4, true>(E3_ATTN_ARGS);
      else
        launch_attn<64, 4, true>(E3_ATTN_ARGS);
    } else if (hd == 128 && nwork >= 512) {
      // More than one round of workgroups: two stages (68 KiB) let two workgroups share a CU, whose waves then
      // spread over the SIMDs more evenly than one workgroup's (5 waves on 4 SIMDs at 68 queries per tile)
      launch_attn<128, 2, false>(E3_ATTN_ARGS);
    } else if (hd == 128) {
      launch_attn<128, 4, false>(E3_ATTN_ARGS);
    } else {
      launch_attn<64, 4, false>(E3_ATTN_ARGS);
    }
#undef E3_ATTN_ARGS
    return AttnSplits{ns, chunk, g.direct};
  }
  const int ns = g.ns;
  dim3 grid(R, Hq, ns);
  if (bf16)
    k_attn_partial<bf16_t><<<grid, 64, 0, st>>>((const bf16_t*)q, (const bf16_t*)kc, (const bf16_t*)vc, unit_stride,
                                                head_stride, pg, rm.seq, rm.lim, rm.tail0, rm.mask, R, Hq, Hkv, hd,
                                                key_bound, scale, o_part, ml_part);
  else
    k_attn_partial<float><<<grid, 64, 0, st>>>((const float*)q, (const float*)kc, (const float*)vc, unit_stride,
                                               head_stride, pg, rm.seq, rm.lim, rm.tail0, rm.mask, R, Hq, Hkv, hd, key_bound,
                                               scale, o_part, ml_part);
  return AttnSplits{ns, ATT_CHUNK};
}

void attention(bool bf16, const void* q, const void* kc, const void* vc, size_t unit_stride, size_t head_stride,
               const KvPages& pg, const RowMeta& rm, int R, int rps, int Hq, int Hkv, int hd, int key_bound,
               float* o_part, float* ml_part, int max_splits, void* out, hipStream_t st, bool packed,
               const int* plan) {
  if (R <= 0) return;
  const AttnSplits sp = attention_partials(bf16, q, kc, vc, unit_stride, head_stride, pg, rm, R, rps, Hq, Hkv, hd,
                                           key_bound, o_part, ml_part, max_splits, st, 0, nullptr, nullptr, 0,
                                           nullptr, plan, bf16 ? out : nullptr, packed);
  if (sp.direct) return;  // the attention kernel wrote the output
  if (bf16)
    combine<bf16_t>(o_part, ml_part, sp.ns, R, Hq, hd, -1, (bf16_t*)out, st, packed);
  else
    combine<float>(o_part, ml_part, sp.ns, R, Hq, hd, -1, (float*)out, st, packed);
}

// ------------------------------------------------------ training-time test
// Attention of the draft layer during training-time test ("EAGLE-3:
// Engineering Implementation of LLM Inference Acceleration", VII.5 and the
// draft layer's forward_ttt): the native step's keys are attended causally,
// each simulated step adds one key per position that only the query at that
// position sees.  The causal part is the tree-masked attention above with row
// i seeing keys [0, i] (lim = i + 1, no tree part).  For bf16 at head sizes 64
// and 128 one key chunk covers every native key and the attention kernel's
// epilogue folds in the S diagonal keys (TTT = true).  Otherwise the S
// diagonal scores of every (position, head) form one more online-softmax
// partial (k_ttt_diag), merged by the combine kernel with the chunk partials.

// rows i < T: one sequence, causal over the native keys
__global__ void k_ttt_meta(int T, RowMeta rm) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T) return;
  rm.seq[i] = 0;
  rm.pos[i] = i;
  rm.slot[i] = i;
  rm.lim[i] = i + 1;
  rm.tail0[i] = 0;
  rm.mask[i] = 0ull;
}

// One wave per (position i, query head h): scores s_j = scale * q . ks[j][g][i]
// for j < S, partial (m = max s_j, l = sum exp(s_j - m), o = sum exp(s_j - m) vs[j][g][i])
// written as split `split` of o_part / ml_part (m = -inf, l = 0 when S = 0).
template <typename T>
__global__ __launch_bounds__(64) void k_ttt_diag(int Tn, int S, int Hq, int Hkv, int hd, float scale,
                                                 const T* __restrict__ q, const T* __restrict__ ks,
                                                 const T* __restrict__ vs, int split, float* __restrict__ o_part,
                                                 float* __restrict__ ml_part) {
  const int i = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int g = h / (Hq / Hkv);
  const size_t oi = ((size_t)split * Tn + i) * Hq + h;
  const T* qp = q + ((size_t)i * Hq + h) * hd;
  float m = -INFINITY;
  for (int j = 0; j < S; ++j) {  // pass 1: the maximum
    const T* kp = ks + (((size_t)j * Hkv + g) * Tn + i) * hd;
    float d = 0.f;
    for (int e = lane; e < hd; e += 64) d += ld<T>(qp, e) * ld<T>(kp, e);
    m = fmaxf(m, wave_sum(d) * scale);
  }
  float l = 0.f;
  float o[4] = {0.f, 0.f, 0.f, 0.f};  // dims lane, lane + 64, ... (hd <= 256)
  for (int j = 0; j < S; ++j) {  // pass 2: weights and the weighted values
    const T* kp = ks + (((size_t)j * Hkv + g) * Tn + i) * hd;
    const T* vp = vs + (((size_t)j * Hkv + g) * Tn + i) * hd;
    float d = 0.f;
    for (int e = lane; e < hd; e += 64) d += ld<T>(qp, e) * ld<T>(kp, e);
    const float p = expf(wave_sum(d) * scale - m);
    l += p;
    for (int c = 0; c * 64 + lane < hd; ++c) o[c] += p * ld<T>(vp, c * 64 + lane);
  }
  for (int c = 0; c * 64 + lane < hd; ++c) o_part[oi * hd + c * 64 + lane] = o[c];
  if (lane == 0) {
    ml_part[2 * oi] = m;
    ml_part[2 * oi + 1] = l;
  }
}

// Workspace the call really touches: none on the fused path (bf16 at head size 64 or 128, where the attention
// kernel derives the rows' metadata itself and writes the output without partials), else the general path's.
size_t ttt_scratch_bytes(bool bf16, int T, int Hq, int hd) {
  return bf16 && (hd == 64 || hd == 128) ? 0 : ttt_workspace_bytes(T, Hq, hd);
}

size_t ttt_workspace_bytes(int T, int Hq, int hd) {
  const size_t splits = (size_t)(T + ATT_CHUNK - 1) / ATT_CHUNK + 1;  // the key chunks + the diagonal partial
  size_t b = 0;
  b += splits * T * Hq * hd * sizeof(float);      // o_part
  b += splits * T * Hq * 2 * sizeof(float);       // ml_part
  b += (size_t)T * (5 * sizeof(int) + sizeof(uint64_t));  // row metadata
  return b + 8 * 256;                                      // each of the 8 arrays starts 256-aligned
}

void ttt_attention(bool bf16, int T, int S, int Hq, int Hkv, int hd, const void* q, const void* k0, const void* v0,
                   const void* ks, const void* vs, void* out, void* ws, hipStream_t st) {
  const int max_splits = (T + ATT_CHUNK - 1) / ATT_CHUNK;
  char* p = (char*)ws;
  auto take = [&](size_t bytes) {
    char* r = p;
    p += (bytes + 255) / 256 * 256;
    return r;
  };
  float* o_part = (float*)take((size_t)(max_splits + 1) * T * Hq * hd * sizeof(float));
  float* ml_part = (float*)take((size_t)(max_splits + 1) * T * Hq * 2 * sizeof(float));
  RowMeta rm{};
  rm.seq = (int*)take(T * sizeof(int));
  rm.pos = (int*)take(T * sizeof(int));
  rm.slot = (int*)take(T * sizeof(int));
  rm.lim = (int*)take(T * sizeof(int));
  rm.tail0 = (int*)take(T * sizeof(int));
  rm.mask = (uint64_t*)take(T * sizeof(uint64_t));
  const float scale = 1.f / sqrtf((float)hd);
  if (bf16 && (hd == 64 || hd == 128)) {  // (the kernel derives each row's metadata itself)
    // one key chunk spans all T native keys (the T rows already fill the chip); the diagonal keys are merged in
    // the attention kernel's epilogue, which writes the output
    const int chunk = (T + 63) / 64 * 64;
    attention_partials(true, q, k0, v0, (size_t)Hkv * T * hd, (size_t)T * hd, KvPages{}, rm, T, T, Hq, Hkv, hd, T,
                       o_part, ml_part, max_splits, st, chunk, ks, vs, S, out);
    return;
  }
  k_ttt_meta<<<(T + 255) / 256, 256, 0, st>>>(T, rm);
  // native keys [Hkv][T][hd]: one "sequence" of T slots
  const AttnSplits sp = attention_partials(bf16, q, k0, v0, (size_t)Hkv * T * hd, (size_t)T * hd, KvPages{}, rm, T, T, Hq, Hkv,
                                           hd, T, o_part, ml_part, max_splits, st, 0);
  const int extra = max_splits;  // a split index no key chunk uses
  if (bf16) {
    k_ttt_diag<bf16_t><<<dim3(T, Hq), 64, 0, st>>>(T, S, Hq, Hkv, hd, scale, (const bf16_t*)q, (const bf16_t*)ks,
                                                   (const bf16_t*)vs, extra, o_part, ml_part);
    combine<bf16_t>(o_part, ml_part, sp.ns, T, Hq, hd, extra, (bf16_t*)out, st);
  } else {
    k_ttt_diag<float><<<dim3(T, Hq), 64, 0, st>>>(T, S, Hq, Hkv, hd, scale, (const float*)q, (const float*)ks,
                                                  (const float*)vs, extra, o_part, ml_part);
    combine<float>(o_part, ml_part, sp.ns, T, Hq, hd, extra, (float*)out, st);
  }
}

// ---------------------------------------------- allocation-free entry point
// The training-time-test call for callers that cannot allocate: its scratch is
// this fixed per-device array (every GPU the library runs on holds its own
// copy until the process ends).  Host code never uses the array's name as an
// address: on the first call on a device its device address is looked up once
// (with that device current) and kept per device.
}  // namespace e3

static __device__ __align__(256) unsigned char scratch[e3::TTT_STATIC_SCRATCH];

namespace e3 {
namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};  // per device ordinal: the array's device address
}  // namespace

hipError_t ttt_static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace e3
