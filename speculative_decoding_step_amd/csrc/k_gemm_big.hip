// Large-M bf16 GEMM (prefill chunks, batch-64 verify): out = X W^T with
// X [M, K] row-major (or in column slabs of 32) and W [N, K] in the packed slab layout, fp32 partials
// per K split.
#include <hip/hip_ext.h>

#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace e3 {

// Large-M GEMM (prefill chunks, batch-64 verify): 128 (M) x 256 (N) output
// tile per workgroup, K in steps of 32.  Four waves in a 2 x 2 arrangement
// each own a 64 x 128 sub-tile (4 x 8 MFMA blocks of 16 x 16), so every
// operand fragment read from LDS feeds 4 or 8 MFMAs.
//
// Operand tiles go from global memory straight into LDS (global_load_lds,
// 16 bytes per lane, landing in lane order) already in MFMA fragment order:
// a step's A tile is 8 fragments (16 activation rows x 32 K each, lane l
// fetching row l % 16, K 8 (l / 16) .. + 7 of row-major X) and its B tile 16
// fragments, each one contiguous 1 KiB of the packed weight.  Fragment reads
// are then plain lane-order 16-byte LDS reads (conflict-free), and staging
// costs no registers and no LDS store instructions.  Three LDS stages: the
// copies of step s + 2 are issued during step s, and one barrier per step
// both publishes step s and retires the stage that is refilled next.  The
// copies are issued from inline asm and the wait for them (vmcnt) is explicit:
// the compiler's own wait insertion cannot tell the stages apart and would
// otherwise drain all of them at every step.
//
// Tile order: m-tile fastest, dealt round-robin over the 8 XCDs as in the
// skinny kernel, so the m-tiles that share a weight tile read it from the
// same L2.
constexpr int BM = 128, BN = GEMM_BIG_ROWS, BKK = GEMM_BIG_KSTEP;
constexpr int AFR = BM / 16, BFR = BN / 16;  // fragments per stage

struct BigTiles {
  int tiles0[4];  // prefix of BN-row N tiles per segment
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 16 bytes per lane from g into LDS at l + 16 * lane (l wave-uniform).
E3_DEV void lds_copy16(const void* g, void* l) {
  const unsigned base = (unsigned)(size_t)(lds_ptr_t)l;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(__builtin_amdgcn_readfirstlane(base)),
               "v"(g)
               : "memory", "m0");
}

// FUSE: the two segments are the gate and up projections (F rows each); a
// tile covers 128 output columns n0 .. n0 + 127 of both, arranged so that in
// each wave the 16-column blocks alternate gate, up, gate, up ... over the
// same columns, and the epilogue writes act[m][n] = bf16(silu(g) * u)
// directly (no K split), in column slabs of 32 when APACK.
//
// APACK: X is stored in column slabs of 32 (slab32_index), as the kernels
// that produce this GEMM's input write it for passes of more than 64 rows: an
// A fragment (16 rows x 32 K) is then one contiguous KiB, like a weight
// fragment, instead of 16 row pieces of 64 bytes, and a producer writing one
// row still writes whole 64-byte pieces.
//
// TOPK (an LM head: one segment, no K split): each wave's 64 x 128 sub-tile
// is one 128-id slice of 64 rows.  Row 64 wm + 16 i + 4 lg + r of it lives
// in the 16 lanes of lane row lg, 8 values per lane (acc[i][0..7][r]), so
// each of tk.k rounds takes the row's best (value, id) pair with four DPP
// steps, straight from the accumulators; then the slice's maximum and sum of
// exponentials for the log-sum-exp.  The fp32 logits are stored only when out
// is non-null.
template <bool FUSE, bool APACK, bool TOPK = false>
__global__ __launch_bounds__(256, 2) void k_gemm_bf16_big(const bf16_t* __restrict__ X, int M, int K, GemmSegs segs,
                                                          BigTiles bt, float* __restrict__ out, int ldo,
                                                          size_t split_stride, int kchunk, int S, int mtiles,
                                                          int nwork, bf16_t* __restrict__ act, int F, SliceTopk tk) {
  static_assert(!TOPK || (!FUSE && BN == 2 * TOPK_SLICE), "a top-k wave owns one 128-id slice");
  __shared__ __attribute__((aligned(1024))) bf16_t sa0[AFR * 512], sa1[AFR * 512], sa2[AFR * 512];
  __shared__ __attribute__((aligned(1024))) bf16_t sb0[BFR * 512], sb1[BFR * 512], sb2[BFR * 512];
  const int per = (nwork + 7) >> 3;
  const int lam = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (lam >= nwork) return;
  const int mt = lam % mtiles, rest = lam / mtiles;
  const int split = rest % S, ntile = rest / S;
  int seg = 0;
  while (!FUSE && seg + 1 < segs.nseg && ntile >= bt.tiles0[seg + 1]) ++seg;
  const int n0 = (ntile - bt.tiles0[seg]) * BN;
  const int kb = split * kchunk, ke = min(K, kb + kchunk);
  const int nrows = FUSE ? F : segs.rows[seg];  // rows of the packed matrix (both FUSE matrices have F)
  const size_t slab = (size_t)((nrows + 15) >> 4) * (4 * 512);
  const int m0 = mt * BM;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int wm = wv & 1, wn = wv >> 1;
  // this wave's copies: A fragments 2 wv, 2 wv + 1 and B fragments 4 wv .. 4 wv + 3 of every stage.
  // Rows past M read row M - 1 and blocks past the segment read block 0; their results are not stored.
  const bf16_t* ap[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    ap[i] = X + (size_t)min(m0 + 16 * (2 * wv + i) + lr, M - 1) * (APACK ? 32 : K) + 8 * lg;
  const bf16_t* bp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int jj = 4 * wv + i;  // tile block
    int rb;
    const bf16_t* Wb;
    if (FUSE) {  // tile block jj: half h = jj / 8, block j = jj % 8 of it; odd blocks are up rows
      const int h = jj >> 3, j = jj & 7;
      rb = ntile * 8 + 4 * h + (j >> 1);
      Wb = (const bf16_t*)segs.w[j & 1];
    } else {
      rb = (n0 >> 4) + jj;
      Wb = (const bf16_t*)segs.w[seg];
    }
    bp[i] = Wb + (size_t)(16 * rb < nrows ? rb : 0) * (4 * 512) + 8 * lane;
  }
  auto issue = [&](bf16_t* sa, bf16_t* sb, int k0) {
    const size_t aoff = APACK ? (size_t)(k0 >> 5) * M * 32 : (size_t)k0;  // slab k0 / 32, or column k0
#pragma unroll
    for (int i = 0; i < 2; ++i) lds_copy16(ap[i] + aoff, sa + (2 * wv + i) * 512);
    const size_t off = (size_t)(k0 / PACK_KB) * slab + ((k0 % PACK_KB) / 32) * 512;
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_copy16(bp[i] + off, sb + (4 * wv + i) * 512);
  };
  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mul = [&](const bf16_t* sa, const bf16_t* sb) {
    bf16x8 a[4], b[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = __builtin_bit_cast(bf16x8, *(const u32x4*)(sa + (4 * wm + i) * 512 + 8 * lane));
#pragma unroll
    for (int j = 0; j < 8; ++j) b[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)(sb + (8 * wn + j) * 512 + 8 * lane));
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  };
  // Step s: this wave's 6 copies of step s were issued two steps earlier and
  // only the 6 of step s + 1 were issued after them, so vmcnt(6) means step s
  // has landed; the barrier makes every wave's copies visible and guarantees
  // that all waves finished reading the stage the copies of step s + 2 refill
  // (it was read in step s - 1).  Past the last step the copies repeat the
  // last step's addresses into stages nobody reads again.
  const int nsteps = (ke - kb) / BKK, klast = ke - BKK;
  auto step = [&](int s, const bf16_t* ca, const bf16_t* cb, bf16_t* na, bf16_t* nb) {
    asm volatile("s_waitcnt vmcnt(6)\n\ts_barrier" ::: "memory");
    issue(na, nb, min(kb + (s + 2) * BKK, klast));
    mul(ca, cb);
  };
  issue(sa0, sb0, kb);
  issue(sa1, sb1, min(kb + BKK, klast));
  int s = 0;
  for (; s + 3 <= nsteps; s += 3) {
    step(s, sa0, sb0, sa2, sb2);
    step(s + 1, sa1, sb1, sa0, sb0);
    step(s + 2, sa2, sb2, sa1, sb1);
  }
  if (s < nsteps) step(s, sa0, sb0, sa2, sb2);
  if (s + 1 < nsteps) step(s + 1, sa1, sb1, sa0, sb0);
  __builtin_amdgcn_s_waitcnt(0);  // the trailing copies land before the workgroup's LDS is released
  if (FUSE) {  // acc[i][2t] = gate, acc[i][2t + 1] = up at column ntile*128 + wn*64 + 16 t + lr
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int n = ntile * 128 + 64 * wn + 16 * t + lr;
      if (n >= F) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + 64 * wm + 16 * i + 4 * lg + r;
          const float g = acc[i][2 * t][r], u = acc[i][2 * t + 1][r];
          if (m < M) act[APACK ? slab32_index(m, n, M) : (size_t)m * F + n] = f2bf(g / (1.f + expf(-g)) * u);
        }
    }
    return;
  }
  // acc[i][j][r] = out[m0 + 64 wm + 16 i + 4 lg + r][n0 + 128 wn + 16 j + lr]
  if (!TOPK || out) {
    float* o = out + split * split_stride + segs.col0[seg];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = n0 + 128 * wn + 16 * j + lr;
      if (n >= nrows) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + 64 * wm + 16 * i + 4 * lg + r;
          if (m < M) o[(size_t)m * ldo + n] = acc[i][j][r];
        }
    }
  }
  if constexpr (TOPK) {
    const int slice = (n0 >> 7) + wn;
    int id[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) id[j] = n0 + 128 * wn + 16 * j + lr;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 64 * wm + 16 * i + 4 * lg + r;
        const bool live = m < M;  // uniform within the lane row
        unsigned taken = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (!live || id[j] >= nrows) taken |= 1u << j;
        const size_t o = (size_t)m * tk.ns + slice;
        float top = -INFINITY;
        for (int k = 0; k < tk.k; ++k) {
          VI b{-INFINITY, 0x7fffffff};
          int bj = -1;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const bool take = !((taken >> j) & 1u) & better(acc[i][j][r], id[j], b.v, b.i);
            b = take ? VI{acc[i][j][r], id[j]} : b;
            bj = take ? j : bj;
          }
          const VI rb = row16_best(b);
          if (bj >= 0 && b.i == rb.i && b.v == rb.v) taken |= 1u << bj;
          if (k == 0) top = rb.v;
          if (live && lr == 0) {
            tk.pv[o * tk.k + k] = rb.v;
            tk.pi[o * tk.k + k] = rb.i;
          }
        }
        if (tk.pmax) {  // the slice's maximum and sum of exp(z / T - max / T) in double
          const double mt = (double)top / tk.temp;
          double sum = 0.0;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (live && id[j] < nrows) sum += exp((double)acc[i][j][r] / tk.temp - mt);
          sum = row16_sum_d(sum);
          if (live && lr == 0) {
            tk.pmax[o] = top;
            tk.psum[o] = sum;
          }
        }
      }
  }
}

int gemm_big(const void* X, int M, int K, const GemmSegs& segs, float* out, size_t split_stride, int splits,
             hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop, bool a_packed) {
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
  if (M > 0) {
    if (a_packed)
      hipExtLaunchKernelGGL((k_gemm_bf16_big<false, true>), dim3(grid), dim3(256), 0, st, ev_start, ev_stop, 0,
                            (const bf16_t*)X, M, K, segs, bt, out, gemm_ntot(segs), split_stride, kchunk, S, mtiles,
                            nwork, (bf16_t*)nullptr, 0, SliceTopk{});
    else
      hipExtLaunchKernelGGL((k_gemm_bf16_big<false, false>), dim3(grid), dim3(256), 0, st, ev_start, ev_stop, 0,
                            (const bf16_t*)X, M, K, segs, bt, out, gemm_ntot(segs), split_stride, kchunk, S, mtiles,
                            nwork, (bf16_t*)nullptr, 0, SliceTopk{});
  }
  return S;
}

void gemm_big_lm_topk(const void* X, int M, int K, const void* W, int V, float* logits, int ldo, const SliceTopk& tk,
                      hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const GemmSegs segs = make_segs(W, V);
  BigTiles bt;
  bt.tiles0[0] = 0;
  bt.tiles0[1] = bt.tiles0[2] = bt.tiles0[3] = (V + BN - 1) / BN;
  const int mtiles = (M + BM - 1) / BM;
  const int nwork = mtiles * bt.tiles0[1];
  const unsigned grid = 8u * (unsigned)((nwork + 7) / 8);
  hipExtLaunchKernelGGL((k_gemm_bf16_big<false, true, true>), dim3(grid), dim3(256), 0, st, ev_start, ev_stop, 0,
                        (const bf16_t*)X, M, K, segs, bt, logits, ldo, (size_t)0, K, 1, mtiles, nwork,
                        (bf16_t*)nullptr, 0, tk);
}

void gemm_big_silu(const void* X, int M, int K, const void* w_gate, const void* w_up, int F, void* act,
                   hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (M <= 0) return;
  const GemmSegs segs = make_segs(w_gate, F, w_up, F);
  BigTiles bt{};
  const int mtiles = (M + BM - 1) / BM;
  const int nwork = mtiles * ((F + 127) / 128);
  const unsigned grid = 8u * (unsigned)((nwork + 7) / 8);
  // passes of more than 64 rows read and write column slabs of 32 (the input from the RMSNorm, the output for
  // the down projection)
  hipExtLaunchKernelGGL((k_gemm_bf16_big<true, true>), dim3(grid), dim3(256), 0, st, ev_start, ev_stop, 0,
                        (const bf16_t*)X, M, K, segs, bt, (float*)nullptr, 0, (size_t)0, K, 1, mtiles, nwork,
                        (bf16_t*)act, F, SliceTopk{});
}

}  // namespace e3
