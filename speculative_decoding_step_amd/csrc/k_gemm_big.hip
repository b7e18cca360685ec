// Large-M bf16 GEMM (prefill chunks, batch-64 verify): out = X W^T with
// X [M, K] row-major and W [N, K] in the packed slab layout, fp32 partials
// per K split.
#include <hip/hip_ext.h>

#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace e3 {

// Large-M GEMM (prefill chunks, batch-64 verify): 128 (M) x 256 (N) output
// tile per workgroup, K in steps of 32 through double-buffered LDS for both
// operands; a step's weight tile is one packed fragment (1 KiB, contiguous)
// of each of the tile's sixteen 16-row blocks.  Four waves in a 2 x 2 arrangement each own a 64 x 128 sub-tile
// (4 x 8 MFMA blocks of 16 x 16), so every operand fragment read from LDS
// feeds 4 or 8 MFMAs.  LDS rows are 64 bytes (four 16-byte chunks) with the
// chunk index XOR-swizzled by (row / 2) % 4: any eight consecutive lanes of
// a fragment read (eight rows, one chunk) or of a staging store (two rows)
// then touch distinct banks.  Global loads run two
// K steps ahead through two register buffers.  Tile
// order: m-tile fastest, dealt round-robin over the 8 XCDs as in the skinny
// kernel, so the m-tiles that share a weight tile read it from the same L2.
constexpr int BM = 128, BN = GEMM_BIG_ROWS, BKK = GEMM_BIG_KSTEP;

struct BigTiles {
  int tiles0[4];  // prefix of BN-row N tiles per segment
};

E3_DEV int swz(int row, int chunk) { return row * 4 + (chunk ^ ((row >> 1) & 3)); }  // in 16-byte chunks

// FUSE: the two segments are the gate and up projections (F rows each); a
// tile covers 128 output columns n0 .. n0 + 127 of both, arranged so that in
// each wave the 16-column blocks alternate gate, up, gate, up ... over the
// same columns, and the epilogue writes act[m][n] = bf16(silu(g) * u)
// directly (no K split).
template <bool FUSE>
__global__ __launch_bounds__(256, 2) void k_gemm_bf16_big(const bf16_t* __restrict__ X, int M, int K, GemmSegs segs,
                                                          BigTiles bt, float* __restrict__ out, int ldo,
                                                          size_t split_stride, int kchunk, int S, int mtiles,
                                                          int nwork, bf16_t* __restrict__ act, int F) {
  __shared__ __attribute__((aligned(16))) u32x4 as[2][BM * 4];
  __shared__ __attribute__((aligned(16))) u32x4 bs[2][BN * 4];
  const int per = (nwork + 7) >> 3;
  const int lam = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (lam >= nwork) return;
  const int mt = lam % mtiles, rest = lam / mtiles;
  const int split = rest % S, ntile = rest / S;
  int seg = 0;
  while (seg + 1 < segs.nseg && ntile >= bt.tiles0[seg + 1]) ++seg;
  const int n0 = (ntile - bt.tiles0[seg]) * BN;
  const int kb = split * kchunk, ke = min(K, kb + kchunk);
  const bf16_t* __restrict__ W = (const bf16_t*)segs.w[seg];
  const int nrows = segs.rows[seg];
  const int m0 = mt * BM;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int wm = (wv & 1) * 64, wn = (wv >> 1) * 128;
  // staging: A chunk c = tid + 256 i (i < 2): row c / 4, K chunk c % 4.  B
  // chunk c = tid + 256 i (i < 4): lane c % 64 of the fragment of tile block
  // c / 64, i.e. tile row 16 (c / 64) + c % 16, K chunk (c % 64) / 16.  Rows
  // past M read row M - 1 and blocks past the segment read block 0; their
  // results are not stored.
  const bf16_t* ap[2];
  const bf16_t* bp[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i;
    ap[i] = X + (size_t)min(m0 + (c >> 2), M - 1) * K + (c & 3) * 8;
  }
  const int bn = FUSE ? F : nrows;  // rows of the packed matrix (both FUSE matrices have F)
  const size_t slab = (size_t)((bn + 15) >> 4) * (4 * 512);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i, jj = c >> 6, l = c & 63;
    int rb;
    const bf16_t* Wb;
    if (FUSE) {  // tile block jj: half h = jj / 8, block j = jj % 8 of it; odd blocks are up rows
      const int h = jj >> 3, j = jj & 7;
      rb = ntile * 8 + 4 * h + (j >> 1);
      Wb = (const bf16_t*)segs.w[j & 1];
    } else {
      rb = (n0 >> 4) + jj;
      Wb = W;
    }
    bp[i] = Wb + (size_t)(16 * rb < bn ? rb : 0) * (4 * 512) + 8 * l;
  }
  u32x4 ar0[2], br0[4], ar1[2], br1[4];
  auto fetch = [&](u32x4 (&ar)[2], u32x4 (&br)[4], int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) ar[i] = *(const u32x4*)(ap[i] + k0);
    const size_t off = (size_t)(k0 / PACK_KB) * slab + ((k0 % PACK_KB) / 32) * 512;
#pragma unroll
    for (int i = 0; i < 4; ++i) br[i] = *(const u32x4*)(bp[i] + off);
  };
  auto stash = [&](const u32x4 (&ar)[2], const u32x4 (&br)[4], int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      as[buf][swz(c >> 2, c & 3)] = ar[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, l = c & 63;
      bs[buf][swz(16 * (c >> 6) + (l & 15), l >> 4)] = br[i];
    }
  };
  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mul = [&](int buf) {
    bf16x8 a[4], b[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = __builtin_bit_cast(bf16x8, as[buf][swz(wm + 16 * i + lr, lg)]);
#pragma unroll
    for (int j = 0; j < 8; ++j) b[j] = __builtin_bit_cast(bf16x8, bs[buf][swz(wn + 16 * j + lr, lg)]);
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  };
  // LDS holds K step s (double-buffered), registers hold step s + 1, and the
  // loads of step s + 2 are issued before step s is multiplied, so every load
  // has two multiply phases to arrive.  Past the last step the loads repeat
  // the last step's addresses.
  const int nsteps = (ke - kb) / BKK, klast = ke - BKK;
  auto step = [&](int s, const u32x4 (&anext)[2], const u32x4 (&bnext)[4], u32x4 (&aafter)[2], u32x4 (&bafter)[4]) {
    fetch(aafter, bafter, min(kb + (s + 2) * BKK, klast));
    __builtin_amdgcn_sched_barrier(0);
    mul(s & 1);
    stash(anext, bnext, (s + 1) & 1);
    __syncthreads();
  };
  fetch(ar0, br0, kb);
  fetch(ar1, br1, min(kb + BKK, klast));
  stash(ar0, br0, 0);
  __syncthreads();
  int s = 0;
  for (; s + 2 <= nsteps; s += 2) {
    step(s, ar1, br1, ar0, br0);
    step(s + 1, ar0, br0, ar1, br1);
  }
  if (s < nsteps) step(s, ar1, br1, ar0, br0);
  if (FUSE) {  // acc[i][2t] = gate, acc[i][2t + 1] = up at column ntile*128 + wn/2 + 16 t + lr
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int n = ntile * 128 + (wn >> 1) + 16 * t + lr;
      if (n >= F) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm + 16 * i + 4 * lg + r;
          const float g = acc[i][2 * t][r], u = acc[i][2 * t + 1][r];
          if (m < M) act[(size_t)m * F + n] = f2bf(g / (1.f + expf(-g)) * u);
        }
    }
    return;
  }
  // acc[i][j][r] = out[m0 + wm + 16 i + 4 lg + r][n0 + wn + 16 j + lr]
  float* o = out + split * split_stride + segs.col0[seg];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int n = n0 + wn + 16 * j + lr;
    if (n >= nrows) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm + 16 * i + 4 * lg + r;
        if (m < M) o[(size_t)m * ldo + n] = acc[i][j][r];
      }
  }
}

int gemm_big(const void* X, int M, int K, const GemmSegs& segs, float* out, size_t split_stride, int splits,
             hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop) {
  BigTiles bt;
  bt.tiles0[0] = 0;
  for (int i = 0; i < 3; ++i) bt.tiles0[i + 1] = bt.tiles0[i] + (i < segs.nseg ? (segs.rows[i] + BN - 1) / BN : 0);
  const int ktiles = K / BKK;
  const int per = (ktiles + std::max(1, splits) - 1) / std::max(1, splits);
  const int kchunk = per * BKK;
  const int S = (ktiles + per - 1) / per;
  const int mtiles = (M + BM - 1) / BM;
  const int nwork = mtiles * S * bt.tiles0[segs.nseg];
  const unsigned grid = 8u * (unsigned)((nwork + 7) / 8);
  if (M > 0)
    hipExtLaunchKernelGGL(k_gemm_bf16_big<false>, dim3(grid), dim3(256), 0, st, ev_start, ev_stop, 0,
                          (const bf16_t*)X, M, K, segs, bt, out, gemm_ntot(segs), split_stride, kchunk, S, mtiles,
                          nwork, (bf16_t*)nullptr, 0);
  return S;
}

void gemm_big_silu(const void* X, int M, int K, const void* w_gate, const void* w_up, int F, void* act,
                   hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (M <= 0) return;
  const GemmSegs segs = make_segs(w_gate, F, w_up, F);
  BigTiles bt{};
  const int mtiles = (M + BM - 1) / BM;
  const int nwork = mtiles * ((F + 127) / 128);
  const unsigned grid = 8u * (unsigned)((nwork + 7) / 8);
  hipExtLaunchKernelGGL(k_gemm_bf16_big<true>, dim3(grid), dim3(256), 0, st, ev_start, ev_stop, 0, (const bf16_t*)X,
                        M, K, segs, bt, (float*)nullptr, 0, (size_t)0, K, 1, mtiles, nwork, (bf16_t*)act, F);
}

}  // namespace e3
