// Weight-streaming GEMM for the step's linear layers: out = X W^T.
//
// X [M, K] activations (rows of one verify / draft pass); W [N, K] is a bf16
// weight in the packed layout below (fp32 weights stay row-major).  At the
// batch-1 shapes M is 1..64 and every weight byte is read once per pass, so
// the kernel is HBM-bound: each wave streams its 16-row weight blocks
// straight from global memory into MFMA operand registers with nontemporal
// 16-byte loads (one fully used 1 KiB fragment per wave instruction), two K
// steps ahead of the multiply, and the activation tile is staged in LDS and
// shared by the waves.  K is optionally split across workgroups (fp32
// partials, summed in a fixed order by the consumer kernel), which keeps
// enough workgroups in flight on 256 CUs when N is small.
//
// Packed weight layout ("slab" layout): K is cut into 128-wide slabs and the
// slabs are stored one after the other; inside slab t come the 16-row blocks
// rb = 0 .. N/16 - 1 in order, each as four MFMA fragments (K 32f .. 32f + 31
// of the slab, f = 0..3) of 64 lanes x 8 consecutive bf16: lane l holds row
// 16 rb + l % 16 and K 8 (l / 16) .. + 7 of the fragment.  All workgroups
// work through the K slabs at roughly the same pace, so at any moment the
// whole chip reads one contiguous region of each weight (good DRAM page
// locality), and every fragment load is a contiguous 1 KiB.
//
// MFMA v_mfma_f32_16x16x32_bf16: A (16x32) and B (32x16) fragments hold, in
// lane l, row/column (l % 16) and K elements 8*(l/16) .. 8*(l/16)+7; the
// 16x16 fp32 result holds rows 4*(l/16)+r (r = 0..3), column l % 16.
#include <hip/hip_ext.h>

#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace e3 {

GemmSegs make_segs(const void* w0, int r0, const void* w1, int r1, const void* w2, int r2) {
  GemmSegs s{};
  const void* w[3] = {w0, w1, w2};
  int r[3] = {r0, r1, r2};
  s.nseg = 0;
  s.tiles0[0] = 0;
  int col = 0;
  for (int i = 0; i < 3; ++i) {
    if (!w[i] || r[i] <= 0) break;
    s.w[i] = w[i];
    s.rows[i] = r[i];
    s.col0[i] = col;
    col += r[i];
    s.tiles0[i + 1] = s.tiles0[i] + (r[i] + 63) / 64;
    s.nseg = i + 1;
  }
  for (int i = s.nseg; i < 3; ++i) s.tiles0[i + 1] = s.tiles0[i];
  return s;
}

int gemm_ntot(const GemmSegs& s) { return s.nseg ? s.col0[s.nseg - 1] + s.rows[s.nseg - 1] : 0; }

__device__ __forceinline__ void seg_of(const GemmSegs& s, int tile, int& seg, int& n0) {
  seg = 0;
  while (seg + 1 < s.nseg && tile >= s.tiles0[seg + 1]) ++seg;
  n0 = (tile - s.tiles0[seg]) * 64;
}

constexpr int XPAD = 8;  // bf16 elements of padding per LDS row

// Tile prefix over the stacked segments for a given tile height.
struct TileMap {
  int tiles0[4];
};

__host__ TileMap tile_map(const GemmSegs& s, int rows_per_tile) {
  TileMap t;
  t.tiles0[0] = 0;
  for (int i = 0; i < 3; ++i)
    t.tiles0[i + 1] = t.tiles0[i] + (i < s.nseg ? (s.rows[i] + rows_per_tile - 1) / rows_per_tile : 0);
  return t;
}

// Packing: one thread per 16-byte destination chunk (a coalesced store; the
// source reads are 16-byte gathers).  Rows N .. 16 ceil(N / 16) - 1 of the
// last block are zeros.
__global__ void k_pack_linear(const bf16_t* __restrict__ src, bf16_t* __restrict__ dst, int N, int K) {
  const int nb16 = (N + 15) >> 4;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)nb16 * 16 * K / 8) return;
  const int lane = (int)(i & 63);
  size_t f = i >> 6;
  const int fi = (int)(f & 3);
  f >>= 2;
  const size_t rb = f % nb16, t = f / nb16;
  const size_t n = rb * 16 + (lane & 15);
  const size_t k = t * PACK_KB + 32 * fi + 8 * (lane >> 4);
  *(u32x4*)(dst + i * 8) = n < (size_t)N ? *(const u32x4*)(src + n * K + k) : u32x4{0u, 0u, 0u, 0u};
}

void pack_linear(const void* src, void* dst, int N, int K, hipStream_t st) {
  const size_t chunks = (size_t)((N + 15) / 16) * 16 * K / 8;
  if (chunks == 0) return;
  k_pack_linear<<<(unsigned)((chunks + 255) / 256), 256, 0, st>>>((const bf16_t*)src, (bf16_t*)dst, N, K);
}

// Skinny GEMM: MB 16-row activation blocks (M <= 16 MB per workgroup); each
// of the NW waves owns NB 16-row weight blocks; K in steps of one 128-wide
// slab.  Work item lam = (m-tile, K split, N tile), m-tile fastest.
// Workgroups are dispatched round-robin over the 8 XCDs, so workgroup L runs
// item (L % 8) * per + L / 8: the m-tiles of one weight tile land on the
// same XCD back to back and re-read that tile from its L2 rather than HBM.
//
// FUSE (NB = 2, no K split): the two segments are the gate and up
// projections (F rows each); wave w's block 0 is gate rows and block 1 the up
// rows of the same 16 columns, and the epilogue writes
// act[m][n] = bf16(silu(g) * u) straight from the accumulators.
//
// TOPK (one segment, no K split, 128 columns per workgroup): after storing
// its logits the workgroup stages them in LDS and takes, for each of its
// rows, the tk.k best (value, id) pairs of its 128 ids with tk.k rounds of a
// wave-wide argmax (one wave per row, two ids per lane; taken ids drop out),
// plus the slice's maximum and sum of exponentials for the log-sum-exp.
template <int MB, int NB, int NW, bool FUSE, bool TOPK = false>
__global__ __launch_bounds__(64 * NW) void k_gemm_bf16(const bf16_t* __restrict__ X, int M, int K, GemmSegs segs,
                                                   TileMap tm, float* __restrict__ out, int ldo, size_t split_stride,
                                                   int kchunk, int mtiles, int S, int nwork,
                                                   bf16_t* __restrict__ act, SliceTopk tk) {
  static_assert(!FUSE || NB == 2, "the fused gate/up epilogue pairs a gate and an up block in each wave");
  static_assert(!TOPK || (!FUSE && 16 * NB * NW == TOPK_SLICE), "a top-k workgroup owns one 128-id slice");
  constexpr int KT = PACK_KB;               // K per step: one slab
  constexpr int KS = KT / 32;               // fragments per block and step
  constexpr int NT = 64 * NW;               // threads
  constexpr int ROWS = FUSE ? 16 * NW : 16 * NB * NW;  // output columns per workgroup
  constexpr int CPR = KT / 8;               // 16-byte chunks per activation row
  constexpr int XCH = 16 * MB * CPR / NT;   // chunks per thread
  constexpr int D = 3;                      // register ring depth (steps)
  static_assert(XCH * NT == 16 * MB * CPR, "activation tile splits evenly over the threads");
  __shared__ __attribute__((aligned(16))) bf16_t xs[2][16 * MB][KT + XPAD];
  const int per = (nwork + 7) >> 3;
  const int lam = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (lam >= nwork) return;
  const int mt = lam % mtiles, rest = lam / mtiles;
  const int split = rest % S, ntile = rest / S;
  int seg = 0;
  while (!FUSE && seg + 1 < segs.nseg && ntile >= tm.tiles0[seg + 1]) ++seg;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n0 = FUSE ? ntile * ROWS : (ntile - tm.tiles0[seg]) * ROWS;
  const int nrows = segs.rows[seg];  // FUSE: F, the rows of each of the two matrices
  const size_t slab = (size_t)((nrows + 15) >> 4) * (4 * 512);  // elements per K slab
  const int m0 = mt * 16 * MB;
  const int kb = split * kchunk;
  const int ke = min(K, kb + kchunk);
  const int lr = lane & 15, lg = lane >> 4;

  // The wave's weight blocks: lane's 16 bytes of fragment 0 of slab 0.  A
  // block past the segment reads block 0 instead, the padding rows of a
  // partial last block are zeros (neither result is stored), and activation
  // rows past M repeat row M - 1, so every load is unconditional.
  const bf16_t* wp[NB];
  bool wok[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int r0 = FUSE ? n0 + 16 * wv : n0 + 16 * (NB * wv + nb);
    wok[nb] = r0 < nrows;
    const bf16_t* W = (const bf16_t*)segs.w[FUSE ? nb : seg];
    wp[nb] = W + (size_t)(wok[nb] ? r0 >> 4 : 0) * (4 * 512) + 8 * lane;
  }
  const bf16_t* xp[XCH];
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int c = tid + NT * i, row = c / CPR, col = (c % CPR) * 8;
    xp[i] = X + (size_t)min(m0 + row, M - 1) * K + col;
  }
  u32x4 xr[D][XCH];
  u32x4 wr[D][NB][KS];
  f32x4 acc[NB][MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < MB; ++i) acc[nb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto load = [&](int slot, int kt) {  // kt: first K of the step (a slab boundary)
#pragma unroll
    for (int i = 0; i < XCH; ++i) xr[slot][i] = *(const u32x4*)(xp[i] + kt);
    const size_t off = (size_t)(kt / KT) * slab;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int s = 0; s < KS; ++s)
        wr[slot][nb][s] = __builtin_nontemporal_load((const u32x4*)(wp[nb] + off + 512 * s));
  };
  auto store_x = [&](int slot, int buf) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = tid + NT * i, row = c / CPR, col = (c % CPR) * 8;
      *(u32x4*)&xs[buf][row][col] = xr[slot][i];
    }
  };
  auto mul = [&](int slot, int buf) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      bf16x8 a[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        a[mb] = __builtin_bit_cast(bf16x8, *(const u32x4*)&xs[buf][16 * mb + lr][32 * s + 8 * lg]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, wr[slot][nb][s]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb], b, acc[nb][mb], 0, 0, 0);
      }
    }
  };
  // Pipeline over K steps: a ring of D register slots holds the loads of
  // steps i .. i + D - 1 (weights and activations alike).  Step i (slot
  // j = i % D) first issues the loads of step i + D - 1 into the slot step
  // i - 1 freed, multiplies slot j against LDS tile i & 1, then writes the
  // activations of step i + 1 (loaded D - 2 steps earlier) to the other LDS
  // tile; one barrier per step publishes that tile and retires the one just
  // read.  Past the last step the loads repeat the last step's addresses.
  const int nsteps = (ke - kb) / KT;
  const int klast = kb + (nsteps - 1) * KT;
  auto step = [&](int i, int j) {
    load((j + D - 1) % D, min(kb + (i + D - 1) * KT, klast));
    __builtin_amdgcn_sched_barrier(0);  // issue the loads before the multiplies
    mul(j, i & 1);
    store_x((j + 1) % D, (i + 1) & 1);
    __syncthreads();
  };
  if (nsteps > 0) {
#pragma unroll
    for (int j = 0; j < D - 1; ++j) load(j, min(kb + j * KT, klast));
    store_x(0, 0);
    __syncthreads();
    int i = 0;
    for (; i + D <= nsteps; i += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) step(i + j, j);
    }
#pragma unroll
    for (int j = 0; j < D - 1; ++j)
      if (i + j < nsteps) step(i + j, j);
  }
  if (FUSE) {
    const int n = n0 + 16 * wv + lr;
    if (n >= nrows) return;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * mb + 4 * lg + r;
        const float g = acc[0][mb][r], u = acc[1][mb][r];
        if (m < M) act[(size_t)m * nrows + n] = f2bf(g / (1.f + expf(-g)) * u);
      }
    return;
  }
  // result: acc[nb][mb][r] = out[m0 + 16 mb + 4 lg + r][n0 + 16 (NB wv + nb) + lr]  (TOPK: out may be null)
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if ((TOPK && !out) || n0 + 16 * (NB * wv + nb) + lr >= nrows) continue;
    float* o = out + split * split_stride + segs.col0[seg] + n0 + 16 * (NB * wv + nb) + lr;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * mb + 4 * lg + r;
        if (m < M) o[(size_t)m * ldo] = acc[nb][mb][r];
      }
  }
  if constexpr (TOPK) {
    // The tile goes to LDS, over the activation buffers (free: the K loop ended with a barrier); ids past the
    // vocabulary are -inf and marked taken.  Each 16-lane row of a wave then owns one tile row: a lane holds 8
    // of its 128 values, and each of the tk.k rounds takes the row's best (value, id) with four DPP steps.
    static_assert(sizeof(xs) >= sizeof(float) * 16 * MB * (TOPK_SLICE + 1), "the logit tile fits the LDS buffers");
    float(*tt)[TOPK_SLICE + 1] = reinterpret_cast<float(*)[TOPK_SLICE + 1]>(&xs[0][0][0]);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int c = 16 * (NB * wv + nb) + lr;
      const bool in = n0 + c < nrows;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) tt[16 * mb + 4 * lg + r][c] = in ? acc[nb][mb][r] : -INFINITY;
    }
    __syncthreads();
    const int rows = min(16 * MB, M - m0);
    const int slice = ntile;
    for (int rb = 4 * wv; rb < rows; rb += 4 * NW) {  // wave-uniform; row rb + lg in lane row lg
      const int rr = rb + lg;
      const bool live = rr < rows;  // uniform within the lane row
      float x[8];
      int id[8];
      unsigned taken = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = lr + 16 * j;
        x[j] = live ? tt[rr][c] : -INFINITY;
        id[j] = n0 + c;
        if (!live || id[j] >= nrows) taken |= 1u << j;
      }
      const size_t o = (size_t)(m0 + rr) * tk.ns + slice;
      float top = -INFINITY;
      for (int k = 0; k < tk.k; ++k) {
        VI b{-INFINITY, 0x7fffffff};
        int bj = -1;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bool take = !((taken >> j) & 1u) & better(x[j], id[j], b.v, b.i);
          b = take ? VI{x[j], id[j]} : b;
          bj = take ? j : bj;
        }
        const VI rbst = row16_best(b);
        if (bj >= 0 && b.i == rbst.i && b.v == rbst.v) taken |= 1u << bj;
        if (k == 0) top = rbst.v;
        if (live && lr == 0) {
          tk.pv[o * tk.k + k] = rbst.v;
          tk.pi[o * tk.k + k] = rbst.i;
        }
      }
      if (tk.pmax) {  // the slice's maximum and sum of exp(z / T - max / T) in double, as the separate pass takes them
        const double mt = (double)top / tk.temp;
        double sum = 0.0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (live && id[j] < nrows) sum += exp((double)x[j] / tk.temp - mt);
        sum = row16_sum_d(sum);
        if (live && lr == 0) {
          tk.pmax[o] = top;
          tk.psum[o] = sum;
        }
      }
    }
  }
}

// The skinny variants: M <= 16: <MB 1, NB 2, 4 waves>; M <= 64: <MB 4, NB 1,
// 8 waves>; both cover 128 weight rows per workgroup.  Fused gate/up: 4 waves
// of one gate + one up block, 64 output columns per workgroup.
constexpr int ROWS16 = 16 * 2 * 4, ROWS64 = 16 * 1 * 8, ROWS64N = 16 * 1 * 4, SILU_COLS = 16 * 4;

// fp32 GEMM (the tiny fp32 workload): 32 x 64 output tile per workgroup, each
// thread 2 x 4 outputs, K tiles of 32 staged in LDS for both operands.
__global__ __launch_bounds__(256) void k_gemm_f32(const float* __restrict__ X, int M, int K, GemmSegs segs,
                                                  float* __restrict__ out, int ldo, size_t split_stride,
                                                  int kchunk) {
  __shared__ float xs[32][33];
  __shared__ float ws[64][33];
  int seg, n0;
  seg_of(segs, blockIdx.x, seg, n0);
  const float* __restrict__ W = (const float*)segs.w[seg];
  const int nrows = segs.rows[seg];
  const int m0 = blockIdx.z * 32;
  const int kb = blockIdx.y * kchunk, ke = min(K, kb + kchunk);
  const int tid = threadIdx.x, tn = tid & 15, tm = tid >> 4;  // 16 x 16 threads
  float acc[2][4] = {};
  for (int kt = kb; kt < ke; kt += 32) {
    for (int i = tid; i < 32 * 32; i += 256) {
      const int r = i >> 5, c = i & 31, m = m0 + r, k = kt + c;
      xs[r][c] = (m < M && k < ke) ? X[(size_t)m * K + k] : 0.f;
    }
    for (int i = tid; i < 64 * 32; i += 256) {
      const int r = i >> 5, c = i & 31, n = n0 + r, k = kt + c;
      ws[r][c] = (n < nrows && k < ke) ? W[(size_t)n * K + k] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < 32; ++c) {
      float a0 = xs[tm * 2][c], a1 = xs[tm * 2 + 1][c];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float b = ws[tn + 16 * j][c];
        acc[0][j] += a0 * b;
        acc[1][j] += a1 * b;
      }
    }
    __syncthreads();
  }
  float* o = out + blockIdx.y * split_stride + segs.col0[seg];
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + tm * 2 + i, n = n0 + tn + 16 * j;
      if (m < M && n < nrows) o[(size_t)m * ldo + n] = acc[i][j];
    }
}

int gemm_splits(bool bf16, int K, int splits, int m_tile) {
  const int unit = !bf16 ? 32 : (m_tile <= 64 ? PACK_KB : GEMM_BIG_KSTEP);
  const int kt = (K + unit - 1) / unit;
  if (splits < 1) splits = 1;
  if (splits > kt) splits = kt;
  const int per = (kt + splits - 1) / splits;
  return (kt + per - 1) / per;
}

void gemm_silu(const void* X, int M, int K, const void* w_gate, const void* w_up, int F, void* act, hipStream_t st,
               hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (M <= 0) return;
  const GemmSegs segs = make_segs(w_gate, F, w_up, F);
  const TileMap tm{};
  const int nwork = (F + SILU_COLS - 1) / SILU_COLS;
  const unsigned grid = 8u * (unsigned)((nwork + 7) / 8);
  if (M <= 16)
    hipExtLaunchKernelGGL((k_gemm_bf16<1, 2, 4, true>), dim3(grid), dim3(256), 0, st, ev_start, ev_stop, 0,
                          (const bf16_t*)X, M, K, segs, tm, (float*)nullptr, 0, (size_t)0, K, 1, 1, nwork,
                          (bf16_t*)act, SliceTopk{});
  else
    hipExtLaunchKernelGGL((k_gemm_bf16<4, 2, 4, true>), dim3(grid), dim3(256), 0, st, ev_start, ev_stop, 0,
                          (const bf16_t*)X, M, K, segs, tm, (float*)nullptr, 0, (size_t)0, K, 1, 1, nwork,
                          (bf16_t*)act, SliceTopk{});
}

bool gemm_lm_topk(const void* X, int M, int K, const void* W, int V, float* logits, int ldo, const SliceTopk& tk,
                  hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const int ns = (V + TOPK_SLICE - 1) / TOPK_SLICE;
  if (M <= 0 || K <= 0 || K % PACK_KB || V <= 0 || tk.k < 1 || tk.k > 16 || tk.ns != ns || ns > 1024 || !tk.pv ||
      !tk.pi || (tk.pmax && !tk.psum))
    return false;
  if (M > 64) {
    gemm_big_lm_topk(X, M, K, W, V, logits, ldo, tk, st, ev_start, ev_stop);
    return true;
  }
  const GemmSegs segs = make_segs(W, V);
  const TileMap tm = tile_map(segs, TOPK_SLICE);
  const int nwork = tm.tiles0[1];  // one workgroup per slice, no K split
  const unsigned grid = 8u * (unsigned)((nwork + 7) / 8);
  if (M <= 16)
    hipExtLaunchKernelGGL((k_gemm_bf16<1, 2, 4, false, true>), dim3(grid), dim3(256), 0, st, ev_start, ev_stop, 0,
                          (const bf16_t*)X, M, K, segs, tm, logits, ldo, (size_t)0, K, 1, 1, nwork, (bf16_t*)nullptr,
                          tk);
  else
    hipExtLaunchKernelGGL((k_gemm_bf16<4, 1, 8, false, true>), dim3(grid), dim3(512), 0, st, ev_start, ev_stop, 0,
                          (const bf16_t*)X, M, K, segs, tm, logits, ldo, (size_t)0, K, 1, 1, nwork, (bf16_t*)nullptr,
                          tk);
  return true;
}

int gemm_rows_per_tile(bool bf16, int m_tile) {
  if (!bf16) return 64;
  return m_tile == 16 ? ROWS16 : (m_tile == 64 ? ROWS64 : GEMM_BIG_ROWS);
}

int gemm(bool bf16, const void* X, int M, int K, const GemmSegs& segs, float* out, size_t split_stride,
         int splits, int m_tile, hipStream_t st, hipEvent_t ev_start,
         hipEvent_t ev_stop, bool a_packed) {
  if (bf16 && m_tile > 64)
    return gemm_big(X, M, K, segs, out, split_stride, splits, st, ev_start, ev_stop, a_packed);
  const int ldo = gemm_ntot(segs);
  // 64-row tiles on matrices of at most 8192 rows: four-wave workgroups of 64 weight rows with half the K
  // splits (the same number of workgroups, each streaming twice the K; half the partials to read back)
  const bool narrow = bf16 && m_tile <= 64 && ldo <= 8192;
  if (narrow) splits = std::max(1, splits / 2);
  splits = gemm_splits(bf16, K, splits, m_tile);
  if (M <= 0) return splits;
  if (bf16) {
    const int ktiles = K / PACK_KB;
    const int per = (ktiles + splits - 1) / splits;
    const int kchunk = per * PACK_KB;
    const int S = (ktiles + per - 1) / per;
    const TileMap tm = tile_map(segs, narrow ? ROWS64N : (m_tile == 16 ? ROWS16 : ROWS64));
    const int ntiles = tm.tiles0[segs.nseg];
    const int mtiles = (M + m_tile - 1) / m_tile;
    const int nwork = mtiles * S * ntiles;
    const unsigned grid = 8u * (unsigned)((nwork + 7) / 8);
    if (m_tile == 16 && narrow)
      hipExtLaunchKernelGGL((k_gemm_bf16<1, 1, 4, false>), dim3(grid), dim3(256), 0, st, ev_start, ev_stop, 0,
                            (const bf16_t*)X, M, K, segs, tm, out, ldo, split_stride, kchunk, mtiles, S, nwork,
                            (bf16_t*)nullptr, SliceTopk{});
    else if (m_tile == 16)
      hipExtLaunchKernelGGL((k_gemm_bf16<1, 2, 4, false>), dim3(grid), dim3(256), 0, st, ev_start, ev_stop, 0,
                            (const bf16_t*)X, M, K, segs, tm, out, ldo, split_stride, kchunk, mtiles, S, nwork,
                            (bf16_t*)nullptr, SliceTopk{});
    else if (narrow)
      hipExtLaunchKernelGGL((k_gemm_bf16<4, 1, 4, false>), dim3(grid), dim3(256), 0, st, ev_start, ev_stop, 0,
                            (const bf16_t*)X, M, K, segs, tm, out, ldo, split_stride, kchunk, mtiles, S, nwork,
                            (bf16_t*)nullptr, SliceTopk{});
    else
      hipExtLaunchKernelGGL((k_gemm_bf16<4, 1, 8, false>), dim3(grid), dim3(512), 0, st, ev_start, ev_stop, 0,
                            (const bf16_t*)X, M, K, segs, tm, out, ldo, split_stride, kchunk, mtiles, S, nwork,
                            (bf16_t*)nullptr, SliceTopk{});
  } else {
    const int ntiles = segs.tiles0[segs.nseg];
    const int per = ((K + 31) / 32 + splits - 1) / splits;
    const int kchunk = per * 32;
    const int S = (K + kchunk - 1) / kchunk;
    dim3 grid(ntiles, S, (M + 31) / 32);
    k_gemm_f32<<<grid, 256, 0, st>>>((const float*)X, M, K, segs, out, ldo, split_stride, kchunk);
  }
  return splits;
}

// ------------------------------------------------------------- partial consumers

__global__ void k_resid_add(float* __restrict__ x, const float* __restrict__ part, int S, size_t sstride,
                            int M, int N, int ldp) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)M * N) return;
  const int m = i / N, n = i % N;
  x[i] += sum_splits(part + (size_t)m * ldp + n, S, sstride);
}

template <typename T>
__global__ void k_silu_mul(T* __restrict__ out, const float* __restrict__ part, int S, size_t sstride, int M,
                           int F, int ldp) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)M * F) return;
  const int m = i / F, n = i % F;
  const float g = sum_splits(part + (size_t)m * ldp + n, S, sstride);
  const float u = sum_splits(part + (size_t)m * ldp + F + n, S, sstride);
  st<T>(out, i, g / (1.f + expf(-g)) * u);
}

static inline unsigned nblk(size_t n, int b) { return (unsigned)((n + b - 1) / b); }

void resid_add(float* x, const float* part, int S, size_t sstride, int M, int N, int ldp, hipStream_t st) {
  if (M <= 0) return;
  k_resid_add<<<nblk((size_t)M * N, 256), 256, 0, st>>>(x, part, S, sstride, M, N, ldp);
}
void silu_mul(bool bf16, void* out, const float* part, int S, size_t sstride, int M, int F, int ldp,
              hipStream_t st) {
  if (M <= 0) return;
  if (bf16)
    k_silu_mul<bf16_t><<<nblk((size_t)M * F, 256), 256, 0, st>>>((bf16_t*)out, part, S, sstride, M, F, ldp);
  else
    k_silu_mul<float><<<nblk((size_t)M * F, 256), 256, 0, st>>>((float*)out, part, S, sstride, M, F, ldp);
}

}  // namespace e3
