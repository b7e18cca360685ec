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

void attention(bool bf16, const void* q, const void* kc, const void* vc, size_t seq_stride, size_t head_stride,
               const RowMeta& rm, int R, int Hq, int Hkv, int hd, int key_bound, float* o_part, float* ml_part,
               int max_splits, void* out, hipStream_t st) {
  if (R <= 0) return;
  int ns = (key_bound + ATT_CHUNK - 1) / ATT_CHUNK;
  if (ns < 1) ns = 1;
  if (ns > max_splits) ns = max_splits;  // the workspace holds ceil(max_seq / chunk) splits
  const float scale = 1.f / sqrtf((float)hd);
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
