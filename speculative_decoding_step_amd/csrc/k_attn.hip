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

template <typename T>
__global__ __launch_bounds__(128) void k_attn_combine(const float* __restrict__ o_part,
                                                      const float* __restrict__ ml_part, int ns, int R, int Hq,
                                                      int hd, T* __restrict__ out) {
  const int r = blockIdx.x, h = blockIdx.y;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, ml_part[2 * (((size_t)s * R + r) * Hq + h)]);
  float den = 0.f;
  for (int s = 0; s < ns; ++s) {
    const size_t oi = ((size_t)s * R + r) * Hq + h;
    if (ml_part[2 * oi] != -INFINITY) den += ml_part[2 * oi + 1] * expf(ml_part[2 * oi] - M);
  }
  for (int i = threadIdx.x; i < hd; i += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < ns; ++s) {
      const size_t oi = ((size_t)s * R + r) * Hq + h;
      if (ml_part[2 * oi] != -INFINITY) acc += o_part[oi * hd + i] * expf(ml_part[2 * oi] - M);
    }
    st<T>(out, ((size_t)r * Hq + h) * hd + i, den > 0.f ? acc / den : 0.f);
  }
}

// ---------------------------------------------------------------- MFMA path
// bf16 flash-decoding with grouped queries.  A workgroup (4 waves) owns one
// sequence, one KV head g, 64 query vectors (row i, query head g*G + hl,
// numbered i*G + hl, 16 per wave) and one chunk of keys; key tiles of 64 are
// staged in LDS (K row-major, V transposed) and shared by the four waves.
// S = Q K^T and O += P V run on v_mfma_f32_16x16x32_bf16; the online softmax
// (max, sum) stays in fp32, and P enters the PV product as two bf16 terms
// (P = hi + lo, two MFMAs) so it keeps about 16 significant bits.
constexpr int AKT = 64;  // keys per LDS tile

template <int HD>
__global__ __launch_bounds__(256) void k_attn_mfma(const bf16_t* __restrict__ q, const bf16_t* __restrict__ kc,
                                                   const bf16_t* __restrict__ vc, size_t seq_stride,
                                                   size_t head_stride, const int* __restrict__ rseq,
                                                   const int* __restrict__ rlim, const int* __restrict__ rt0,
                                                   const uint64_t* __restrict__ rmask, int R, int rps, int qblocks,
                                                   int Hq, int Hkv, int S_cap, float scale, int chunk,
                                                   float* __restrict__ o_part, float* __restrict__ ml_part) {
  __shared__ __attribute__((aligned(16))) bf16_t ks[AKT][HD + 8];
  __shared__ __attribute__((aligned(16))) bf16_t vt[HD][AKT + 8];
  __shared__ __attribute__((aligned(16))) bf16_t ps[2][4][16][AKT + 8];  // [hi|lo][wave][query][key]
  __shared__ int red_end[4], red_seq[4];
  const int G = Hq / Hkv;
  const int bs = blockIdx.x / qblocks, qb = blockIdx.x % qblocks;
  const int g = blockIdx.y, sp = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int nq = rps * G;

  // output-row metadata: this lane accumulates query vectors 16w + 4lg + r
  int o_row[4], o_h[4], o_lim[4], o_t0[4];
  uint64_t o_mask[4];
  bool o_ok[4];
  int my_end = 0, my_seq = -1;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int v = qb * 64 + 16 * w + 4 * lg + r;
    o_ok[r] = v < nq;
    o_row[r] = bs * rps + (o_ok[r] ? v / G : 0);
    o_h[r] = g * G + (o_ok[r] ? v % G : 0);
    const int sq = o_ok[r] ? rseq[o_row[r]] : -1;
    o_ok[r] = o_ok[r] && sq >= 0;
    o_lim[r] = rlim[o_row[r]];
    o_t0[r] = rt0[o_row[r]];
    o_mask[r] = rmask[o_row[r]];
    if (o_ok[r]) {
      my_end = max(my_end, min(key_end(o_lim[r], o_t0[r], o_mask[r]), S_cap));
      my_seq = max(my_seq, sq);
    }
  }
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
  const int kend = max(max(red_end[0], red_end[1]), max(red_end[2], red_end[3]));
  const int cs = max(max(red_seq[0], red_seq[1]), max(red_seq[2], red_seq[3]));
  const int c0 = sp * chunk, c1 = min(c0 + chunk, kend);

  float m[4], l[4];
  f32x4 O[HD / 16];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
  }
#pragma unroll
  for (int b = 0; b < HD / 16; ++b) O[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (cs >= 0 && c0 < c1) {
    // Q fragment of the lane's A row: query vector 16w + lr
    u32x4 qf[HD / 32];
    {
      const int v = qb * 64 + 16 * w + lr;
      const bool ok = v < nq;
      const int row = bs * rps + (ok ? v / G : 0), h = g * G + (ok ? v % G : 0);
      const bf16_t* qp = q + ((size_t)row * Hq + h) * HD + 8 * lg;
#pragma unroll
      for (int kk = 0; kk < HD / 32; ++kk) qf[kk] = ok ? *(const u32x4*)(qp + 32 * kk) : u32x4{0u, 0u, 0u, 0u};
    }
    const bf16_t* kb = kc + (size_t)cs * seq_stride + (size_t)g * head_stride;
    const bf16_t* vb = vc + (size_t)cs * seq_stride + (size_t)g * head_stride;
    constexpr int CH = AKT * HD / 8;  // 16-byte chunks per tile
    for (int kt = c0; kt < c1; kt += AKT) {
      __syncthreads();
      for (int c = tid; c < CH; c += 256) {
        const int key = c / (HD / 8), d8 = (c % (HD / 8)) * 8;
        const int j = kt + key;
        u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
        if (j < c1) {
          kv = *(const u32x4*)(kb + (size_t)j * HD + d8);
          vv = *(const u32x4*)(vb + (size_t)j * HD + d8);
        }
        *(u32x4*)&ks[key][d8] = kv;
        const bf16_t* ve = (const bf16_t*)&vv;
#pragma unroll
        for (int e = 0; e < 8; ++e) vt[d8 + e][key] = ve[e];
      }
      __syncthreads();
      f32x4 S[4];
#pragma unroll
      for (int kb4 = 0; kb4 < 4; ++kb4) {
        S[kb4] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < HD / 32; ++kk) {
          const bf16x8 bk = __builtin_bit_cast(bf16x8, *(const u32x4*)&ks[16 * kb4 + lr][32 * kk + 8 * lg]);
          S[kb4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qf[kk]), bk, S[kb4], 0, 0, 0);
        }
      }
      // S[kb4][r] = score(query 16w + 4lg + r, key kt + 16 kb4 + lr)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float tmax = -INFINITY;
#pragma unroll
        for (int kb4 = 0; kb4 < 4; ++kb4) {
          const int j = kt + 16 * kb4 + lr;
          const bool vis = o_ok[r] && j < c1 && visible(j, o_lim[r], o_t0[r], o_mask[r]);
          const float x = vis ? S[kb4][r] * scale : -INFINITY;
          S[kb4][r] = x;
          tmax = fmaxf(tmax, x);
        }
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o, 64));
        const float mn = fmaxf(m[r], tmax);
        const float alpha = (mn == -INFINITY) ? 1.f : expf(m[r] - mn);
        float psum = 0.f;
#pragma unroll
        for (int kb4 = 0; kb4 < 4; ++kb4) {
          const float p = (S[kb4][r] == -INFINITY) ? 0.f : expf(S[kb4][r] - mn);
          S[kb4][r] = p;
          psum += p;
        }
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) psum += __shfl_xor(psum, o, 64);
        l[r] = l[r] * alpha + psum;
        m[r] = mn;
#pragma unroll
        for (int b = 0; b < HD / 16; ++b) O[b][r] *= alpha;
#pragma unroll
        for (int kb4 = 0; kb4 < 4; ++kb4) {
          const bf16_t hi = f2bf(S[kb4][r]);
          ps[0][w][4 * lg + r][16 * kb4 + lr] = hi;
          ps[1][w][4 * lg + r][16 * kb4 + lr] = f2bf(S[kb4][r] - bf2f(hi));
        }
      }
      __syncthreads();
#pragma unroll
      for (int k2 = 0; k2 < AKT / 32; ++k2) {
        const bf16x8 ph = __builtin_bit_cast(bf16x8, *(const u32x4*)&ps[0][w][lr][32 * k2 + 8 * lg]);
        const bf16x8 pl = __builtin_bit_cast(bf16x8, *(const u32x4*)&ps[1][w][lr][32 * k2 + 8 * lg]);
#pragma unroll
        for (int b = 0; b < HD / 16; ++b) {
          const bf16x8 vbf = __builtin_bit_cast(bf16x8, *(const u32x4*)&vt[16 * b + lr][32 * k2 + 8 * lg]);
          O[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vbf, O[b], 0, 0, 0);
          O[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vbf, O[b], 0, 0, 0);
        }
      }
    }
  }
  // partials of the lane's four query vectors
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int v = qb * 64 + 16 * w + 4 * lg + r;
    if (v >= nq) continue;
    const size_t oi = ((size_t)sp * R + o_row[r]) * Hq + o_h[r];
#pragma unroll
    for (int b = 0; b < HD / 16; ++b) o_part[oi * HD + 16 * b + lr] = O[b][r];
    if (lr == 0) {
      ml_part[2 * oi] = m[r];
      ml_part[2 * oi + 1] = l[r];
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
    const int qblocks = (rps * G + 63) / 64;
    dim3 grid((R / rps) * qblocks, Hkv, ns);
    if (hd == 128)
      k_attn_mfma<128><<<grid, 256, 0, st>>>((const bf16_t*)q, (const bf16_t*)kc, (const bf16_t*)vc, seq_stride,
                                             head_stride, rm.seq, rm.lim, rm.tail0, rm.mask, R, rps, qblocks, Hq, Hkv,
                                             key_bound, scale, ATT_CHUNK, o_part, ml_part);
    else
      k_attn_mfma<64><<<grid, 256, 0, st>>>((const bf16_t*)q, (const bf16_t*)kc, (const bf16_t*)vc, seq_stride,
                                            head_stride, rm.seq, rm.lim, rm.tail0, rm.mask, R, rps, qblocks, Hq, Hkv,
                                            key_bound, scale, ATT_CHUNK, o_part, ml_part);
    k_attn_combine<bf16_t><<<dim3(R, Hq), 128, 0, st>>>(o_part, ml_part, ns, R, Hq, hd, (bf16_t*)out);
    return;
  }
  dim3 grid(R, Hq, ns);
  if (bf16) {
    k_attn_partial<bf16_t><<<grid, 64, 0, st>>>((const bf16_t*)q, (const bf16_t*)kc, (const bf16_t*)vc, seq_stride,
                                                head_stride, rm.seq, rm.lim, rm.tail0, rm.mask, R, Hq, Hkv, hd,
                                                key_bound, scale, o_part, ml_part);
    k_attn_combine<bf16_t><<<dim3(R, Hq), 128, 0, st>>>(o_part, ml_part, ns, R, Hq, hd, (bf16_t*)out);
  } else {
    k_attn_partial<float><<<grid, 64, 0, st>>>((const float*)q, (const float*)kc, (const float*)vc, seq_stride,
                                               head_stride, rm.seq, rm.lim, rm.tail0, rm.mask, R, Hq, Hkv, hd, key_bound,
                                               scale, o_part, ml_part);
    k_attn_combine<float><<<dim3(R, Hq), 128, 0, st>>>(o_part, ml_part, ns, R, Hq, hd, (float*)out);
  }
}

}  // namespace e3
