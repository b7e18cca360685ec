// Weight-streaming GEMM for the step's linear layers: out = X W^T.
//
// X [M, K] activations (rows of one verify / draft pass), W [N, K] weights in
// nn.Linear layout.  At the batch-1 shapes M is 1..64 and every weight byte is
// read once per pass, so the kernel is HBM-bound: each wave streams 16 weight
// rows straight from global memory into MFMA operand registers (16-byte loads
// along K, next K-tile prefetched while the current one is multiplied), and
// the activation tile is staged once per workgroup in LDS and shared by the
// four waves.  K is optionally split across workgroups (fp32 partials, summed
// in a fixed order by the consumer kernel), which keeps enough workgroups in
// flight on 256 CUs when N is small.
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

// Skinny GEMM: MB 16-row activation blocks (M <= 16 MB per workgroup), each of
// the NW waves owns NB 16-row weight blocks, K in LDS tiles of KTT.  K must be
// a multiple of KTT (the shapes are checked on the host).
// Work item lam = (m-tile, K split, N tile), m-tile fastest.  Workgroups are
// dispatched round-robin over the 8 XCDs, so workgroup L runs item
// (L % 8) * per + L / 8: the m-tiles of one weight tile land on the same XCD
// back to back and re-read that tile from its L2 rather than from HBM.
//
// FUSE (NB = 1, no K split): the two segments are the gate and up projections
// (F rows each); waves 0 .. NW/2 - 1 own gate rows and waves NW/2 .. NW - 1 the
// up rows of the same 16 NW / 2 columns, and the epilogue exchanges the up
// values through LDS and writes act[m][n] = bf16(silu(g) * u).
template <int MB, int NB, int KTT, int NW, bool FUSE = false>
__global__ __launch_bounds__(64 * NW) void k_gemm_bf16(const bf16_t* __restrict__ X, int M, int K, GemmSegs segs,
                                                   TileMap tm, float* __restrict__ out, int ldo, size_t split_stride,
                                                   int kchunk, int mtiles, int S, int nwork,
                                                   bf16_t* __restrict__ act) {
  static_assert(!FUSE || NB == 1, "the fused gate/up epilogue pairs single-block waves");
  constexpr int KS = KTT / 32;
  constexpr int NT = 64 * NW;               // threads
  constexpr int ROWS = 16 * NB * NW;        // weight rows per workgroup
  constexpr int CPR = KTT / 8;              // 16-byte chunks per activation row
  constexpr int XCH = 16 * MB * CPR / NT;   // chunks per thread
  static_assert(XCH * NT == 16 * MB * CPR, "activation tile splits evenly over the threads");
  __shared__ __attribute__((aligned(16))) bf16_t xs[2][16 * MB][KTT + XPAD];
  const int per = (nwork + 7) >> 3;
  const int lam = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (lam >= nwork) return;
  const int mt = lam % mtiles, rest = lam / mtiles;
  const int split = rest % S, ntile = rest / S;
  int seg = 0;
  while (!FUSE && seg + 1 < segs.nseg && ntile >= tm.tiles0[seg + 1]) ++seg;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const bool up_wave = FUSE && wv >= NW / 2;
  const int n0 = FUSE ? ntile * (ROWS / 2) : (ntile - tm.tiles0[seg]) * ROWS;
  const bf16_t* __restrict__ W = (const bf16_t*)segs.w[FUSE ? (up_wave ? 1 : 0) : seg];
  const int nrows = segs.rows[seg];
  const int m0 = mt * 16 * MB;
  const int kb = split * kchunk;
  const int ke = min(K, kb + kchunk);
  const int lr = lane & 15, lg = lane >> 4;

  // weight fragment sources: rows n0 + 16 (NB wv + nb) + lr, K offset 8 lg in each 32-step.
  // Rows past the segment read row 0 instead (their results are not stored),
  // and activation rows past M repeat row M - 1, so every load is unconditional.
  const bf16_t* wp[NB];
  bool wok[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int r = FUSE ? n0 + 16 * (wv % (NW / 2)) + lr : n0 + 16 * (NB * wv + nb) + lr;
    wok[nb] = r < nrows;
    wp[nb] = W + (size_t)(wok[nb] ? r : 0) * K + 8 * lg;
  }
  const bf16_t* xp[XCH];
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int c = tid + NT * i, row = c / CPR, col = (c % CPR) * 8;
    xp[i] = X + (size_t)min(m0 + row, M - 1) * K + col;
  }
  u32x4 x0[XCH], x1[XCH];
  u32x4 w0[NB][KS], w1[NB][KS], w2[NB][KS];
  f32x4 acc[NB][MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < MB; ++i) acc[nb][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load_w = [&](u32x4 (&dst)[NB][KS], int kt) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int s = 0; s < KS; ++s) dst[nb][s] = *(const u32x4*)(wp[nb] + kt + 32 * s);
  };
  auto load_x = [&](u32x4 (&dst)[XCH], int kt) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) dst[i] = *(const u32x4*)(xp[i] + kt);
  };
  auto store_x = [&](const u32x4 (&src)[XCH], int buf) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = tid + NT * i, row = c / CPR, col = (c % CPR) * 8;
      *(u32x4*)&xs[buf][row][col] = src[i];
    }
  };
  auto mul = [&](const u32x4 (&wc)[NB][KS], int buf) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      bf16x8 a[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        a[mb] = __builtin_bit_cast(bf16x8, *(const u32x4*)&xs[buf][16 * mb + lr][32 * s + 8 * lg]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, wc[nb][s]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb], b, acc[nb][mb], 0, 0, 0);
      }
    }
  };
  // Pipeline over K steps of KTT.  Weights: three register buffers, so while
  // step i is multiplied, steps i + 1 and i + 2 are in flight.  Activations:
  // two register buffers and two LDS tiles; the tile of step i + 1 is written
  // to LDS at the end of step i (its loads were issued a step earlier), and one
  // barrier per step both publishes it and retires the tile just read.  Past
  // the last step the loads repeat the last step's addresses.
  const int nsteps = (ke - kb) / KTT;
  const int klast = kb + (nsteps - 1) * KTT;
  auto step = [&](int i, const u32x4 (&cur)[NB][KS], u32x4 (&ahead)[NB][KS], const u32x4 (&xnext)[XCH],
                  u32x4 (&xafter)[XCH]) {
    // xnext holds the activations of step i + 1; xafter receives those of step i + 2
    load_x(xafter, min(kb + (i + 2) * KTT, klast));
    load_w(ahead, min(kb + (i + 2) * KTT, klast));
    __builtin_amdgcn_sched_barrier(0);  // issue the loads before the multiplies
    mul(cur, i & 1);
    store_x(xnext, (i + 1) & 1);
    __syncthreads();
  };
  if (nsteps > 0) {
    load_x(x0, kb);
    load_x(x1, min(kb + KTT, klast));
    load_w(w0, kb);
    load_w(w1, min(kb + KTT, klast));
    store_x(x0, 0);
    __syncthreads();
    int i = 0;
    for (; i + 6 <= nsteps; i += 6) {
      step(i, w0, w2, x1, x0);
      step(i + 1, w1, w0, x0, x1);
      step(i + 2, w2, w1, x1, x0);
      step(i + 3, w0, w2, x0, x1);
      step(i + 4, w1, w0, x1, x0);
      step(i + 5, w2, w1, x0, x1);
    }
    // remaining steps: the buffer roles continue from i (a multiple of 6)
    if (i < nsteps) step(i, w0, w2, x1, x0);
    if (i + 1 < nsteps) step(i + 1, w1, w0, x0, x1);
    if (i + 2 < nsteps) step(i + 2, w2, w1, x1, x0);
    if (i + 3 < nsteps) step(i + 3, w0, w2, x0, x1);
    if (i + 4 < nsteps) step(i + 4, w1, w0, x1, x0);
  }
  if (FUSE) {
    __shared__ float ub[NW / 2][16 * MB][17];  // up values: [wave pair][row][column]
    if (up_wave) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) ub[wv - NW / 2][16 * mb + 4 * lg + r][lr] = acc[0][mb][r];
    }
    __syncthreads();
    if (!up_wave && wok[0]) {
      const int n = n0 + 16 * wv + lr;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ml = 16 * mb + 4 * lg + r, m = m0 + ml;
          const float g = acc[0][mb][r], u = ub[wv][ml][lr];
          if (m < M) act[(size_t)m * nrows + n] = f2bf(g / (1.f + expf(-g)) * u);
        }
    }
    return;
  }
  // result: acc[nb][mb][r] = out[m0 + 16 mb + 4 lg + r][n0 + 16 (NB wv + nb) + lr]
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if (!wok[nb]) continue;
    float* o = out + split * split_stride + segs.col0[seg] + n0 + 16 * (NB * wv + nb) + lr;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * mb + 4 * lg + r;
        if (m < M) o[(size_t)m * ldo] = acc[nb][mb][r];
      }
  }
}

// K tile and weight rows per workgroup of the two skinny variants:
// M <= 16: <MB 1, NB 2, KTT 256, 4 waves>; M <= 64: <MB 4, NB 1, KTT 128, 8 waves>.
constexpr int KT16 = 256, KT64 = 128;
constexpr int ROWS16 = 16 * 2 * 4, ROWS64 = 16 * 1 * 8;

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
  const int unit = !bf16 ? 32 : (m_tile == 16 ? KT16 : (m_tile == 64 ? KT64 : GEMM_BIG_KSTEP));
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
  constexpr int COLS = ROWS64 / 2;  // output columns per workgroup
  const int nwork = (F + COLS - 1) / COLS;
  const unsigned grid = 8u * (unsigned)((nwork + 7) / 8);
  hipExtLaunchKernelGGL((k_gemm_bf16<4, 1, KT64, 8, true>), dim3(grid), dim3(512), 0, st, ev_start, ev_stop, 0,
                        (const bf16_t*)X, M, K, segs, tm, (float*)nullptr, 0, (size_t)0, K, 1, 1, nwork,
                        (bf16_t*)act);
}

int gemm_rows_per_tile(bool bf16, int m_tile) {
  if (!bf16) return 64;
  return m_tile == 16 ? ROWS16 : (m_tile == 64 ? ROWS64 : GEMM_BIG_ROWS);
}

int gemm(bool bf16, const void* X, int M, int K, const GemmSegs& segs, float* out, size_t split_stride,
         int splits, int m_tile, hipStream_t st, hipEvent_t ev_start,
         hipEvent_t ev_stop) {
  if (bf16 && m_tile > 64)
    return gemm_big(X, M, K, segs, out, split_stride, splits, st, ev_start, ev_stop);
  splits = gemm_splits(bf16, K, splits, m_tile);
  if (M <= 0) return splits;
  const int ldo = gemm_ntot(segs);
  if (bf16) {
    const int unit = m_tile == 16 ? KT16 : KT64;
    const int ktiles = K / unit;
    const int per = (ktiles + splits - 1) / splits;
    const int kchunk = per * unit;
    const int S = (ktiles + per - 1) / per;
    const TileMap tm = tile_map(segs, m_tile == 16 ? ROWS16 : ROWS64);
    const int ntiles = tm.tiles0[segs.nseg];
    const int mtiles = (M + m_tile - 1) / m_tile;
    const int nwork = mtiles * S * ntiles;
    const unsigned grid = 8u * (unsigned)((nwork + 7) / 8);
    if (m_tile == 16)
      hipExtLaunchKernelGGL((k_gemm_bf16<1, 2, KT16, 4>), dim3(grid), dim3(256), 0, st, ev_start, ev_stop, 0,
                            (const bf16_t*)X, M, K, segs, tm, out, ldo, split_stride, kchunk, mtiles, S, nwork, nullptr);
    else
      hipExtLaunchKernelGGL((k_gemm_bf16<4, 1, KT64, 8>), dim3(grid), dim3(512), 0, st, ev_start, ev_stop, 0,
                            (const bf16_t*)X, M, K, segs, tm, out, ldo, split_stride, kchunk, mtiles, S, nwork, nullptr);
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

__global__ void k_sum_store(float* __restrict__ out, const float* __restrict__ part, int S, size_t sstride,
                            int M, int N, int ldp) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)M * N) return;
  const int m = i / N, n = i % N;
  const float s = sum_splits(part + (size_t)m * ldp + n, S, sstride);
  out[i] = s;
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
void sum_store(float* out, const float* part, int S, size_t sstride, int M, int N, int ldp, hipStream_t st) {
  if (M <= 0) return;
  k_sum_store<<<nblk((size_t)M * N, 256), 256, 0, st>>>(out, part, S, sstride, M, N, ldp);
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
