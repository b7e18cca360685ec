// Row-wise kernels of the step: embedding gather, RMSNorm (+ aux tap capture),
// the draft head's [input_norm(e) ; hidden_norm(x)] input, rotary embedding
// with the KV-cache write, and the vocabulary top-k / log-sum-exp.
#include "common.hpp"
#include "kernels.hpp"
#include "tree.hpp"

namespace e3 {

static inline unsigned nblk(size_t n, int b) { return (unsigned)((n + b - 1) / b); }

// ------------------------------------------------------------------ embedding
template <typename T>
__global__ void k_embed(const T* __restrict__ table, const int* __restrict__ tokens, float* __restrict__ x,
                        int d, int V, int* status) {
  const int r = blockIdx.x;
  int t = tokens[r];
  float* xr = x + (size_t)r * d;
  if (t < 0 || t >= V) {
    if (threadIdx.x == 0 && t != -1) raise_flag(status, E3_DEV_BAD_TOKEN);
    for (int i = threadIdx.x; i < d; i += blockDim.x) xr[i] = 0.f;
    return;
  }
  const T* er = table + (size_t)t * d;
  if ((d & 3) == 0) {
    const int d4 = d >> 2;
    for (int c0 = threadIdx.x; c0 < d4; c0 += 4 * blockDim.x) {
      float4 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = c0 + j * blockDim.x;
        if (c < d4) v[j] = ld4<T>(er, 4 * c);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = c0 + j * blockDim.x;
        if (c < d4) ((float4*)xr)[c] = v[j];
      }
    }
  } else {
    for (int i = threadIdx.x; i < d; i += blockDim.x) xr[i] = ld<T>(er, i);
  }
}

void embed_rows(bool bf16, const void* table, const int* tokens, float* x, int R, int d, int V, int* status,
                hipStream_t st) {
  if (R <= 0) return;
  if (bf16)
    k_embed<bf16_t><<<R, 256, 0, st>>>((const bf16_t*)table, tokens, x, d, V, status);
  else
    k_embed<float><<<R, 256, 0, st>>>((const float*)table, tokens, x, d, V, status);
}

// -------------------------------------------------------------------- rmsnorm
// One block per row, one float4 column group per thread (NV groups when the
// row is wider than 4 * blockDim), so the whole row and all its split
// partials are loaded at once.  Optional steps, in order:
//   x[r] += sum_s part[s][r]   (the split-K partials of the preceding GEMM)
//   tap[r] = T(x[r])           (the aux feature capture)
//   out[r] = T(x[r] * rsqrt(mean(x^2) + eps) * w)
template <typename T, int NV>
__global__ __launch_bounds__(1024) void k_add_rmsnorm(float* __restrict__ x, const float* __restrict__ part, int S,
                                                      size_t sstride, int ldp, const T* __restrict__ w,
                                                      T* __restrict__ out, int out_ld, int d, float eps,
                                                      T* __restrict__ tap, int tap_ld, bool packed, RowCopy rc) {
  __shared__ float red[16];
  const int r = blockIdx.x, tid = threadIdx.x, nt = blockDim.x, d4 = d >> 2;
  float4* xr = (float4*)(x + (size_t)r * d);
  float4* cr = nullptr;
  if (rc.dst) {
    const int b = r / rc.k;
    cr = (float4*)(rc.dst + ((size_t)b * rc.emax + rc.slot[r] - rc.seq_lens[b]) * d);
  }
  float4 v[NV];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = tid + nt * i;
    if (c < d4) {
      v[i] = xr[c];
      if (part) {
        const float4 a = sum_splits4((const float4*)(part + (size_t)r * ldp) + c, S, sstride >> 2);
        v[i].x += a.x; v[i].y += a.y; v[i].z += a.z; v[i].w += a.w;
        xr[c] = v[i];
      }
      if (cr) cr[c] = v[i];
      ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
      if (tap) st4<T>(tap, (size_t)r * tap_ld + 4 * c, v[i]);
    }
  }
  ss = block_sum(ss, red);
  const float inv = 1.f / sqrtf(ss / (float)d + eps);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = tid + nt * i;
    if (c < d4) {
      const int e = 4 * c;  // the 4 columns stay inside one 32-column slab
      const float4 wv = ld4<T>(w, e);
      st4<T>(out, packed ? slab32_index(r, e, gridDim.x) : (size_t)r * out_ld + e,
             make_float4(v[i].x * inv * wv.x, v[i].y * inv * wv.y, v[i].z * inv * wv.z, v[i].w * inv * wv.w));
    }
  }
}

// Rows whose width is not a multiple of 4 (or wider than 8192): element loop.
template <typename T>
__global__ __launch_bounds__(256) void k_add_rmsnorm_any(float* __restrict__ x, const float* __restrict__ part,
                                                         int S, size_t sstride, int ldp, const T* __restrict__ w,
                                                         T* __restrict__ out, int out_ld, int d, float eps,
                                                         T* __restrict__ tap, int tap_ld, bool packed, RowCopy rc) {
  __shared__ float red[16];
  const int r = blockIdx.x, tid = threadIdx.x;
  float* xr = x + (size_t)r * d;
  float* cr = nullptr;
  if (rc.dst) {
    const int b = r / rc.k;
    cr = rc.dst + ((size_t)b * rc.emax + rc.slot[r] - rc.seq_lens[b]) * d;
  }
  float ss = 0.f;
  for (int i = tid; i < d; i += 256) {
    float v = xr[i];
    if (part) {
      v += sum_splits(part + (size_t)r * ldp + i, S, sstride);
      xr[i] = v;
    }
    if (cr) cr[i] = v;
    ss += v * v;
    if (tap) st<T>(tap, (size_t)r * tap_ld + i, v);
  }
  ss = block_sum(ss, red);
  const float inv = 1.f / sqrtf(ss / (float)d + eps);
  for (int i = tid; i < d; i += 256)
    st<T>(out, packed ? slab32_index(r, i, gridDim.x) : (size_t)r * out_ld + i, xr[i] * inv * ld<T>(w, i));
}

template <typename T>
static void launch_add_rmsnorm(float* x, const float* part, int S, size_t sstride, int ldp, const T* w, T* out,
                               int out_ld, int R, int d, float eps, T* tap, int tap_ld, hipStream_t st, bool pk,
                               const RowCopy& rc) {
  const int d4 = d / 4;
  // the float4 kernel moves 4 elements at a time: every row start must be aligned to 4 of them
  const size_t al = 4 * sizeof(T);
  const bool aligned = (size_t)out % al == 0 && (size_t)w % al == 0 && out_ld % 4 == 0 &&
                       (!tap || ((size_t)tap % al == 0 && tap_ld % 4 == 0)) && (size_t)rc.dst % 16 == 0;
  if (d % 4 == 0 && d4 <= 2048 && aligned) {
    const int nt = std::min(1024, (d4 + 63) / 64 * 64);
    if (d4 <= nt)
      k_add_rmsnorm<T, 1><<<R, nt, 0, st>>>(x, part, S, sstride, ldp, w, out, out_ld, d, eps, tap, tap_ld, pk, rc);
    else
      k_add_rmsnorm<T, 2><<<R, nt, 0, st>>>(x, part, S, sstride, ldp, w, out, out_ld, d, eps, tap, tap_ld, pk, rc);
  } else {
    k_add_rmsnorm_any<T><<<R, 256, 0, st>>>(x, part, S, sstride, ldp, w, out, out_ld, d, eps, tap, tap_ld, pk, rc);
  }
}

void add_rmsnorm(bool bf16, float* x, const float* part, int S, size_t sstride, int ldp, const void* w, void* out,
                 int out_ld, int R, int d, float eps, void* tap, int tap_ld, hipStream_t st, bool packed,
                 const RowCopy& rc) {
  if (R <= 0) return;
  if (bf16)
    launch_add_rmsnorm<bf16_t>(x, part, S, sstride, ldp, (const bf16_t*)w, (bf16_t*)out, out_ld, R, d, eps,
                               (bf16_t*)tap, tap_ld, st, packed, rc);
  else
    launch_add_rmsnorm<float>(x, part, S, sstride, ldp, (const float*)w, (float*)out, out_ld, R, d, eps,
                              (float*)tap, tap_ld, st, packed, rc);
}

void rmsnorm(bool bf16, const float* x, const void* w, void* out, int out_ld, int R, int d, float eps, void* tap,
             int tap_ld, hipStream_t st, bool packed) {
  add_rmsnorm(bf16, (float*)x, nullptr, 0, 0, 0, w, out, out_ld, R, d, eps, tap, tap_ld, st, packed);
}

// Where a draft-input row's features come from: x[r] itself, or (src != null) row src[r] of a_rows, row
// -1 - src[r] of a_last when src[r] < 0.
struct RowSrc {
  const int* src = nullptr;
  const float* a_rows = nullptr;
  const float* a_last = nullptr;
  E3_DEV const float* row(int r, const float* xr, int d) const {
    if (!src) return xr;
    const int s = src[r];
    return s < 0 ? a_last + (size_t)(-1 - s) * d : a_rows + (size_t)s * d;
  }
};

// ---------------------------------------------------------------- draft input
// One block per row, one float4 column group per thread (NV groups when the
// row is wider): out[r] = [input_norm(embed[token]) ; hidden_norm(x[r])].
// With split partials (part != null, the fusion FC's K splits) the feature row
// is first formed from them, x[r] = sum of the S splits in split order, and
// stored as the layer's residual stream: the FC's reduction, the two norms
// and the concatenation are one pass.  Rows whose width is not a multiple of 4
// use the element loop.
template <typename T, int NV>
__global__ __launch_bounds__(1024) void k_draft_input(const T* __restrict__ embed, const int* __restrict__ tokens,
                                                      float* __restrict__ x, const float* __restrict__ part, int S,
                                                      size_t sstride, const T* __restrict__ w_in,
                                                      const T* __restrict__ w_hid, T* __restrict__ out, int d,
                                                      int V, float eps, int* status, bool packed, RowSrc gs) {
  __shared__ float red[16];
  const int r = blockIdx.x, tid = threadIdx.x, nt = blockDim.x, d4 = d >> 2;
  int t = tokens[r];
  const bool ok = t >= 0 && t < V;
  if (!ok && tid == 0 && t != -1) raise_flag(status, E3_DEV_BAD_TOKEN);
  if (!ok) t = 0;
  float* xr = x + (size_t)r * d;
  const float* hr = gs.row(r, xr, d);  // the feature row: x[r] itself, or the gathered source row
  const T* er = embed + (size_t)t * d;
  float4 e[NV], h[NV];
  float se = 0.f, sx = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = tid + nt * i;
    if (c < d4) {
      e[i] = ok ? ld4<T>(er, 4 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
      if (part) {
        h[i] = sum_splits4((const float4*)(part + (size_t)r * d) + c, S, sstride >> 2);
        *(float4*)(xr + 4 * c) = h[i];
      } else {
        h[i] = *(const float4*)(hr + 4 * c);
        if (gs.src) *(float4*)(xr + 4 * c) = h[i];
      }
      se += e[i].x * e[i].x + e[i].y * e[i].y + e[i].z * e[i].z + e[i].w * e[i].w;
      sx += h[i].x * h[i].x + h[i].y * h[i].y + h[i].z * h[i].z + h[i].w * h[i].w;
    }
  }
  se = block_sum(se, red);
  sx = block_sum(sx, red);
  const float ie = 1.f / sqrtf(se / (float)d + eps), ix = 1.f / sqrtf(sx / (float)d + eps);
  // column c of the row: row-major, or column slabs of 32 of an [R, 2d] matrix
  auto at = [&](int col) { return packed ? slab32_index(r, col, gridDim.x) : (size_t)r * 2 * d + col; };
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = tid + nt * i;
    if (c < d4) {
      const float4 wi = ld4<T>(w_in, 4 * c), wh = ld4<T>(w_hid, 4 * c);
      st4<T>(out, at(4 * c),
             make_float4(e[i].x * ie * wi.x, e[i].y * ie * wi.y, e[i].z * ie * wi.z, e[i].w * ie * wi.w));
      st4<T>(out, at(d + 4 * c),
             make_float4(h[i].x * ix * wh.x, h[i].y * ix * wh.y, h[i].z * ix * wh.z, h[i].w * ix * wh.w));
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_draft_input_any(const T* __restrict__ embed, const int* __restrict__ tokens,
                                                         float* __restrict__ x, const float* __restrict__ part, int S,
                                                         size_t sstride, const T* __restrict__ w_in,
                                                         const T* __restrict__ w_hid, T* __restrict__ out, int d,
                                                         int V, float eps, int* status, bool packed, RowSrc gs) {
  __shared__ float red[16];
  const int r = blockIdx.x;
  int t = tokens[r];
  const bool ok = t >= 0 && t < V;
  if (!ok && threadIdx.x == 0 && t != -1) raise_flag(status, E3_DEV_BAD_TOKEN);
  if (!ok) t = 0;
  float* xr = x + (size_t)r * d;
  const float* hr = gs.row(r, xr, d);
  float se = 0.f, sx = 0.f;
  for (int i = threadIdx.x; i < d; i += blockDim.x) {
    const float e = ok ? ld<T>(embed, (size_t)t * d + i) : 0.f;
    if (part) xr[i] = sum_splits(part + (size_t)r * d + i, S, sstride);
    else if (gs.src) xr[i] = hr[i];
    se += e * e;
    sx += xr[i] * xr[i];
  }
  se = block_sum(se, red);
  sx = block_sum(sx, red);
  const float ie = 1.f / sqrtf(se / (float)d + eps), ix = 1.f / sqrtf(sx / (float)d + eps);
  auto at = [&](int col) { return packed ? slab32_index(r, col, gridDim.x) : (size_t)r * 2 * d + col; };
  for (int i = threadIdx.x; i < d; i += blockDim.x) {
    const float e = ok ? ld<T>(embed, (size_t)t * d + i) : 0.f;
    st<T>(out, at(i), e * ie * ld<T>(w_in, i));
    st<T>(out, at(d + i), xr[i] * ix * ld<T>(w_hid, i));
  }
}

template <typename T>
static void launch_draft_input(const T* embed, const int* tokens, float* x, const float* part, int S, size_t sstride,
                               const T* w_in, const T* w_hid, T* out, int R, int d, int V, float eps, int* status,
                               hipStream_t st, bool pk, const RowSrc& gs) {
  const int d4 = d / 4;
  // the float4 kernel moves 4 elements at a time: every row start must be aligned to 4 of them
  const size_t al = 4 * sizeof(T);
  const bool aligned = (size_t)out % al == 0 && (size_t)embed % al == 0 && (size_t)w_in % al == 0 &&
                       (size_t)w_hid % al == 0;
  if (d % 4 == 0 && d4 <= 2048 && aligned) {
    const int nt = std::min(1024, (d4 + 63) / 64 * 64);
    if (d4 <= nt)
      k_draft_input<T, 1><<<R, nt, 0, st>>>(embed, tokens, x, part, S, sstride, w_in, w_hid, out, d, V, eps, status,
                                            pk, gs);
    else
      k_draft_input<T, 2><<<R, nt, 0, st>>>(embed, tokens, x, part, S, sstride, w_in, w_hid, out, d, V, eps, status,
                                            pk, gs);
  } else {
    k_draft_input_any<T><<<R, 256, 0, st>>>(embed, tokens, x, part, S, sstride, w_in, w_hid, out, d, V, eps, status,
                                            pk, gs);
  }
}

void draft_input(bool bf16, const void* embed, const int* tokens, float* x, const float* part, int S,
                 size_t sstride, const void* w_in, const void* w_hid, void* out, int R, int d, int V, float eps,
                 int* status, hipStream_t st, bool packed, const int* src, const float* a_rows,
                 const float* a_last) {
  if (R <= 0) return;
  RowSrc gs;
  gs.src = src;
  gs.a_rows = a_rows;
  gs.a_last = a_last;
  if (bf16)
    launch_draft_input<bf16_t>((const bf16_t*)embed, tokens, x, part, S, sstride, (const bf16_t*)w_in,
                               (const bf16_t*)w_hid, (bf16_t*)out, R, d, V, eps, status, st, packed, gs);
  else
    launch_draft_input<float>((const float*)embed, tokens, x, part, S, sstride, (const float*)w_in,
                              (const float*)w_hid, (float*)out, R, d, V, eps, status, st, packed, gs);
}

// ----------------------------------------------------------- rope + KV write
// One block per (row, head) over QKV partial columns [q heads | k heads | v heads].
// The angle pos * inv_freq[i] (inv_freq = theta^(-2i/hd), tabulated in double
// on the host) is formed and reduced modulo 2 pi in double; cos/sin of the
// reduced angle are then taken in float.
template <typename T>
__global__ __launch_bounds__(64) void k_rope_kv(const float* __restrict__ part, int S, size_t sstride,
                                                const int* __restrict__ rseq, const int* __restrict__ rpos,
                                                const int* __restrict__ rslot, const double* __restrict__ inv_freq,
                                                T* __restrict__ q_out, T* __restrict__ kc, T* __restrict__ vc,
                                                size_t unit_stride, size_t head_stride, KvPages pg, int Hq, int Hkv,
                                                int hd, int* status) {
  const int r = blockIdx.x, h = blockIdx.y;
  int b = rseq[r];
  KvLoc at{0, 0};
  if (h >= Hq && b >= 0) {  // K or V head: where the row's position lives
    at = kv_loc_w(pg, b, rslot[r]);
    if (at.unit < 0) {
      if (threadIdx.x == 0 && h == Hq) raise_flag(status, E3_DEV_KV_OVERFLOW);
      b = -1;
    }
  }
  const int ncol = (Hq + 2 * Hkv) * hd;
  const int half = hd / 2;
  const float* pr = part + (size_t)r * ncol + (size_t)h * hd;
  auto val = [&](int c) { return sum_splits(pr + c, S, sstride); };
  if (h >= Hq + Hkv) {  // V: copy
    if (b < 0) return;
    T* vp = vc + (size_t)at.unit * unit_stride + (size_t)(h - Hq - Hkv) * head_stride + (size_t)at.row * hd;
    for (int i = threadIdx.x; i < hd; i += blockDim.x) st<T>(vp, i, val(i));
    return;
  }
  if (h >= Hq && b < 0) return;
  const double pos = (double)rpos[r];
  constexpr double TWO_PI = 6.283185307179586476925286766559;
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    const float x1 = val(i), x2 = val(i + half);
    const double ang = pos * inv_freq[i];
    const float red = (float)(ang - TWO_PI * rint(ang / TWO_PI));
    float sn, cs;
    sincosf(red, &sn, &cs);
    const float y1 = x1 * cs - x2 * sn, y2 = x2 * cs + x1 * sn;
    if (h < Hq) {
      T* qp = q_out + ((size_t)r * Hq + h) * hd;
      st<T>(qp, i, y1);
      st<T>(qp, i + half, y2);
    } else {
      T* kp = kc + (size_t)at.unit * unit_stride + (size_t)(h - Hq) * head_stride + (size_t)at.row * hd;
      st<T>(kp, i, y1);
      st<T>(kp, i + half, y2);
    }
  }
}

// The same, four rotation pairs per thread (float4 partial loads, 4-wide stores): a block covers 256 / (hd / 8)
// heads of one row, and the row's cos/sin of each pair index are formed once per block into LDS.  Same
// arithmetic and summation order as k_rope_kv.  Needs hd % 8 == 0, hd <= 128 and 256 % (hd / 8) == 0.
template <typename T>
__global__ __launch_bounds__(256) void k_rope_kv4(const float* __restrict__ part, int S, size_t sstride,
                                                  const int* __restrict__ rseq, const int* __restrict__ rpos,
                                                  const int* __restrict__ rslot, const double* __restrict__ inv_freq,
                                                  T* __restrict__ q_out, T* __restrict__ kc, T* __restrict__ vc,
                                                  size_t unit_stride, size_t head_stride, KvPages pg, int Hq, int Hkv,
                                                  int hd, int* status) {
  __shared__ __attribute__((aligned(16))) float cs_l[64], sn_l[64];
  const int r = blockIdx.x, tph = hd >> 3, half = hd >> 1;
  const int h = blockIdx.y * (256 / tph) + threadIdx.x / tph, j = threadIdx.x % tph;
  // the partial loads go out first; the row's cos/sin are formed while they are in flight
  int b = rseq[r];
  KvLoc at{0, 0};
  if (h >= Hq && h < Hq + 2 * Hkv && b >= 0) {  // K or V head: where the row's position lives
    at = kv_loc_w(pg, b, rslot[r]);
    if (at.unit < 0) {
      if (j == 0 && h == Hq) raise_flag(status, E3_DEV_KV_OVERFLOW);
      b = -1;
    }
  }
  const bool live = h < Hq || (h < Hq + 2 * Hkv && b >= 0);
  float4 x1 = make_float4(0.f, 0.f, 0.f, 0.f), x2 = x1;
  if (live) {
    const int ncol = (Hq + 2 * Hkv) * hd;
    const float* pr = part + (size_t)r * ncol + (size_t)h * hd + 4 * j;
    x1 = sum_splits4((const float4*)pr, S, sstride / 4);
    x2 = sum_splits4((const float4*)(pr + half), S, sstride / 4);
  }
  constexpr double TWO_PI = 6.283185307179586476925286766559;
  const double pos = (double)rpos[r];
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    const double ang = pos * inv_freq[i];
    const float red = (float)(ang - TWO_PI * rint(ang / TWO_PI));
    float sn, cs;
    sincosf(red, &sn, &cs);
    cs_l[i] = cs;
    sn_l[i] = sn;
  }
  __syncthreads();
  if (!live) return;
  T* dst = h < Hq ? q_out + ((size_t)r * Hq + h) * hd
                  : (h < Hq + Hkv ? kc : vc) + (size_t)at.unit * unit_stride +
                        (size_t)(h < Hq + Hkv ? h - Hq : h - Hq - Hkv) * head_stride + (size_t)at.row * hd;
  if (h >= Hq + Hkv) {  // V: copy
    st4<T>(dst, 4 * j, x1);
    st4<T>(dst, half + 4 * j, x2);
    return;
  }
  const float4 c = *(const float4*)&cs_l[4 * j], sn = *(const float4*)&sn_l[4 * j];
  st4<T>(dst, 4 * j,
         make_float4(x1.x * c.x - x2.x * sn.x, x1.y * c.y - x2.y * sn.y, x1.z * c.z - x2.z * sn.z,
                     x1.w * c.w - x2.w * sn.w));
  st4<T>(dst, half + 4 * j,
         make_float4(x2.x * c.x + x1.x * sn.x, x2.y * c.y + x1.y * sn.y, x2.z * c.z + x1.z * sn.z,
                     x2.w * c.w + x1.w * sn.w));
}

void rope_kv(bool bf16, const float* part, int S, size_t sstride, int R, const RowMeta& rm, const double* inv_freq,
             void* q_out, void* kc, void* vc, size_t unit_stride, size_t head_stride, const KvPages& pg, int Hq,
             int Hkv, int hd, int* status, hipStream_t st) {
  if (R <= 0) return;
  const int tph = hd / 8;
  if (hd % 8 == 0 && hd <= 128 && 256 % tph == 0) {
    const dim3 grid4(R, (Hq + 2 * Hkv + 256 / tph - 1) / (256 / tph));
    if (bf16)
      k_rope_kv4<bf16_t><<<grid4, 256, 0, st>>>(part, S, sstride, rm.seq, rm.pos, rm.slot, inv_freq,
                                                (bf16_t*)q_out, (bf16_t*)kc, (bf16_t*)vc, unit_stride, head_stride,
                                                pg, Hq, Hkv, hd, status);
    else
      k_rope_kv4<float><<<grid4, 256, 0, st>>>(part, S, sstride, rm.seq, rm.pos, rm.slot, inv_freq, (float*)q_out,
                                               (float*)kc, (float*)vc, unit_stride, head_stride, pg, Hq, Hkv, hd,
                                               status);
    return;
  }
  dim3 grid(R, Hq + 2 * Hkv);
  if (bf16)
    k_rope_kv<bf16_t><<<grid, 64, 0, st>>>(part, S, sstride, rm.seq, rm.pos, rm.slot, inv_freq, (bf16_t*)q_out,
                                           (bf16_t*)kc, (bf16_t*)vc, unit_stride, head_stride, pg, Hq, Hkv, hd,
                                           status);
  else
    k_rope_kv<float><<<grid, 64, 0, st>>>(part, S, sstride, rm.seq, rm.pos, rm.slot, inv_freq, (float*)q_out,
                                          (float*)kc, (float*)vc, unit_stride, head_stride, pg, Hq, Hkv, hd, status);
}

// ------------------------------------------------------------- top-k + lse
constexpr int TK_SLICE = 4096;  // vocabulary entries per partial block
constexpr int TK_KMAX = 16;

int topk_slices(int V) { return (V + TK_SLICE - 1) / TK_SLICE; }

// grid (R, nslices), block 256.  Per slice: the K best (value, index) and,
// when LSE, the slice's max and sum of exp(z - max) in double, with z = logit /
// temperature.  The slice is held in registers (16 values per thread, loaded
// at once).  Each wave first finds the K best of its own 1024 entries in K
// rounds with no barrier (a lane marks its winner in a 16-bit mask), then
// wave 0 merges the four waves' lists (4K <= 64 candidates, one per lane) in
// K more rounds.  The (value, index) order is total, so the result does not
// depend on how the entries are split.
constexpr int TK_PER = TK_SLICE / 256;  // values per thread

template <bool LSE>
__global__ __launch_bounds__(256) void k_topk_partial(const float* __restrict__ logits, int V, int ld, int K,
                                                      double temp, float* __restrict__ pv, int* __restrict__ pi,
                                                      float* __restrict__ pmax, double* __restrict__ psum) {
  __shared__ VI cand[4][TK_KMAX];
  __shared__ double dred[4];
  const int r = blockIdx.x, sl = blockIdx.y, ns = gridDim.y;
  const int v0 = sl * TK_SLICE, n = min(TK_SLICE, V - v0);
  const float* row = logits + (size_t)r * ld + v0;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float v[TK_PER];
#pragma unroll
  for (int j = 0; j < TK_PER; ++j) {
    const int i = tid + 256 * j;  // coalesced: consecutive threads, consecutive entries
    v[j] = i < n ? row[i] : -INFINITY;
  }
  unsigned taken = 0;
#pragma unroll
  for (int j = 0; j < TK_PER; ++j)
    if (tid + 256 * j >= n) taken |= 1u << j;
  auto local_best = [&]() {  // taken entries become (-inf, INT_MAX), which never wins
    VI b{-INFINITY, 0x7fffffff};
#pragma unroll
    for (int j = 0; j < TK_PER; ++j) {
      const bool tk = (taken >> j) & 1u;
      b = vi_best(b, VI{tk ? -INFINITY : v[j], tk ? 0x7fffffff : v0 + tid + 256 * j});
    }
    return b;
  };
  for (int k = 0; k < K; ++k) {
    const VI b = wave_best(local_best());
    if (lane == 0) cand[w][k] = b;
    const int li = b.i - v0;
    if (li >= 0 && li < n && (li & 255) == tid) taken |= 1u << (li >> 8);
  }
  __syncthreads();
  const size_t o = (size_t)r * ns + sl;
  if (LSE) {
    const float top = fmaxf(fmaxf(cand[0][0].v, cand[1][0].v), fmaxf(cand[2][0].v, cand[3][0].v));
    const double m = (double)top / temp;
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < TK_PER; ++j)
      if (tid + 256 * j < n) s += exp((double)v[j] / temp - m);
    s = wave_sum_d(s);
    if (lane == 0) dred[w] = s;
    if (tid == 0) pmax[o] = top;
  }
  if (w == 0) {
    VI mine = lane < 4 * K ? cand[lane / K][lane % K] : VI{-INFINITY, 0x7fffffff};
    for (int k = 0; k < K; ++k) {
      const VI b = wave_best(mine);
      if (lane == 0) {
        pv[o * K + k] = b.v;
        pi[o * K + k] = b.i;
      }
      if (mine.i == b.i && mine.v == b.v) mine = VI{-INFINITY, 0x7fffffff};
    }
  }
  if (LSE) {
    __syncthreads();
    if (tid == 0) psum[o] = dred[0] + dred[1] + dred[2] + dred[3];
  }
}

// grid (R), block 64: merge the slices' candidates (held in registers) and
// combine the slices' sums.
constexpr int TK_MERGE_PER = 16;  // candidates per lane: ns * K <= 64 * TK_KMAX

__global__ __launch_bounds__(64) void k_topk_merge(int ns, int K, double temp, const float* __restrict__ pv,
                                                   const int* __restrict__ pi, const float* __restrict__ pmax,
                                                   const double* __restrict__ psum, int* __restrict__ out_ids,
                                                   float* __restrict__ out_vals, float* __restrict__ lse32,
                                                   double* __restrict__ lse64) {
  const int r = blockIdx.x, tid = threadIdx.x;
  const int nc = ns * K;
  const float* cv = pv + (size_t)r * nc;
  const int* ci = pi + (size_t)r * nc;
  float v[TK_MERGE_PER];
  int id[TK_MERGE_PER];
  unsigned taken = 0;
#pragma unroll
  for (int j = 0; j < TK_MERGE_PER; ++j) {
    const int c = tid + 64 * j;
    v[j] = c < nc ? cv[c] : -INFINITY;
    id[j] = c < nc ? ci[c] : 0x7fffffff;
    if (c >= nc) taken |= 1u << j;
  }
  // slice maxima and sums: lane s holds slice s (ns <= 64 for V <= 64 * 4096)
  const float pm = pmax && tid < ns ? pmax[(size_t)r * ns + tid] : -INFINITY;
  const double ps = pmax && tid < ns ? psum[(size_t)r * ns + tid] : 0.0;
  for (int k = 0; k < K; ++k) {
    VI b{-INFINITY, 0x7fffffff};
    int bj = -1;
#pragma unroll
    for (int j = 0; j < TK_MERGE_PER; ++j) {
      const bool take = !((taken >> j) & 1u) & better(v[j], id[j], b.v, b.i);
      b = take ? VI{v[j], id[j]} : b;
      bj = take ? j : bj;
    }
    const VI wb = wave_best(b);
    if (bj >= 0 && b.i == wb.i && b.v == wb.v) taken |= 1u << bj;
    if (tid == 0) {
      out_ids[(size_t)r * K + k] = wb.i;
      out_vals[(size_t)r * K + k] = wb.v;
    }
  }
  if (!pmax) return;  // no log-sum-exp asked for
  const float mx = wave_max(pm);
  const double M = (double)mx / temp;
  const double S = wave_sum_d(tid < ns ? ps * exp((double)pm / temp - M) : 0.0);
  if (tid == 0) {
    const double l = M + log(S);
    if (lse64) lse64[r] = l;
    if (lse32) lse32[r] = (float)l;
  }
}

void topk_lse(const float* logits, int R, int V, int ld, int K, float temperature, float* pv, int* pi, float* pmax,
              double* psum, int* out_ids, float* out_vals, float* lse32, double* lse64, hipStream_t st) {
  if (R <= 0) return;
  const int ns = topk_slices(V);
  const double t = (double)temperature;
  const bool lse = lse32 || lse64;  // the argmax / top-2 of a verify needs no log-sum-exp
  if (lse)
    k_topk_partial<true><<<dim3(R, ns), 256, 0, st>>>(logits, V, ld, K, t, pv, pi, pmax, psum);
  else
    k_topk_partial<false><<<dim3(R, ns), 256, 0, st>>>(logits, V, ld, K, t, pv, pi, pmax, psum);
  k_topk_merge<<<R, 64, 0, st>>>(ns, K, t, pv, pi, lse ? pmax : nullptr, psum, out_ids, out_vals, lse32, lse64);
}

// A (value, index) pair as a 64-bit key ordered as better() orders pairs (a
// larger key is better): the value's bits mapped monotonically, -0.0 as +0.0
// (the two compare equal), then the complemented index.  Values are not NaN.
// One unsigned compare then decides what better() decides with three.
E3_DEV uint64_t pair_key(float v, int i) {
  unsigned u = __float_as_uint(v);
  u = u == 0x80000000u ? 0u : u;
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint64_t)~(unsigned)i;
}
E3_DEV int pair_key_index(uint64_t k) { return (int)~(unsigned)k; }
template <int CTRL>
E3_DEV uint64_t key_dpp_max(uint64_t a) {
  const unsigned lo = __builtin_amdgcn_update_dpp(0u, (unsigned)a, CTRL, 0xF, 0xF, false);
  const unsigned hi = __builtin_amdgcn_update_dpp(0u, (unsigned)(a >> 32), CTRL, 0xF, 0xF, false);
  const uint64_t b = ((uint64_t)hi << 32) | lo;
  return a > b ? a : b;
}
E3_DEV uint64_t key_swap_max(uint64_t a, bool wide) {
  const unsigned lo = (unsigned)a, hi = (unsigned)(a >> 32);
  const auto l = wide ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false)
                      : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const auto h = wide ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false)
                      : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  const uint64_t x = ((uint64_t)h[0] << 32) | l[0], y = ((uint64_t)h[1] << 32) | l[1];
  return x > y ? x : y;
}
// The wave's largest key, to every lane: the exchanges of wave_best on keys.
E3_DEV uint64_t wave_max_key(uint64_t x) {
  x = key_dpp_max<0xB1>(x);
  x = key_dpp_max<0x4E>(x);
  x = key_dpp_max<0x141>(x);
  x = key_dpp_max<0x140>(x);
  return key_swap_max(key_swap_max(x, false), true);
}
// Keys among the n (non-increasing) at p that are larger than x.
E3_DEV int keys_above(const uint64_t* p, int n, uint64_t x) {
  int lo = 0, hi = n;  // p[0, lo) > x >= p[hi, n)
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (p[mid] > x)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

// grid (R), block 256: merge the 128-id slices of the fused LM-head top-k.
// The k best of a row lie in the k slices whose own best (value, id) pairs
// rank highest: a pair among the k best has its slice's best at or above it,
// and k slices ranked above that slice would hold k pairs above it.  So the
// kernel first picks those k slices: a thread holds the best of up to 4
// slices and each wave takes its k best in k rounds (one wave-wide maximum of
// 64-bit keys per round); a candidate's rank among the four waves' lists is
// its place in its own list plus the keys above it in the other three.  Then
// the k x k candidates of those slices, one per thread, are ranked the same
// way (each slice's list is in order), and the k with ranks below k are the
// row's k best in rank order.  Keys are distinct (distinct ids) except for
// the (-inf, INT_MAX) filler of slots without a candidate, which never ranks
// among real pairs.  The log-sum-exp combines the slices' maxima and sums as
// the separate merge does.
__global__ __launch_bounds__(256) void k_topk_merge_slices(SliceTopk tk, int* __restrict__ out_ids,
                                                           float* __restrict__ out_vals, float* __restrict__ lse32,
                                                           double* __restrict__ lse64, TreeKids kids) {
  __shared__ uint64_t wk[4][TK_KMAX];         // each wave's k best slice maxima, in order
  __shared__ uint64_t gk[TK_KMAX * TK_KMAX];  // the chosen slices' candidates, slice-major (0: no slice)
  __shared__ VI best[TK_KMAX];
  __shared__ int sel[TK_KMAX];
  __shared__ float fred[4];
  __shared__ double dred[4];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int K = tk.k, ns = tk.ns;
  const float* cv = tk.pv + (size_t)r * ns * K;
  const int* ci = tk.pi + (size_t)r * ns * K;
  const uint64_t FILL = pair_key(-INFINITY, 0x7fffffff);
  // the slices' log-sum-exp partials, loaded first so that their latency hides under the selection
  float pm[4];
  double ps[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int sl = tid + 256 * j;
    pm[j] = tk.pmax && sl < ns ? tk.pmax[(size_t)r * ns + sl] : -INFINITY;
    ps[j] = tk.pmax && sl < ns ? tk.psum[(size_t)r * ns + sl] : 0.0;
  }
  // the parent of this row's children (the previous level's output), loaded now rather than after the merge
  int kpar = -1;
  float kps = 0.f;
  if (tid == 0 && kids.depth_new > 1) {
    const int k = kids.ts.topk, b = r / k, rank = r % k;
    kpar = kids.ts.front[b * k + rank];
    kps = kids.ts.score[(size_t)b * kids.ts.cmax + kpar];
  }
  uint64_t key[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // slice s = tid + 256 j: its best pair is its candidate 0
    const int sl = tid + 256 * j;
    key[j] = sl < ns ? pair_key(cv[(size_t)sl * K], ci[(size_t)sl * K]) : FILL;
  }
  if (tid < TK_KMAX) sel[tid] = -1;
  for (int k = 0; k < K; ++k) {  // a lane's taken keys become 0; one with nothing left offers the filler
    uint64_t b = FILL;
    int bj = -1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool take = key[j] > b;
      b = take ? key[j] : b;
      bj = take ? j : bj;
    }
    const uint64_t wb = wave_max_key(b);
    if (bj >= 0 && b == wb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) key[j] = bj == j ? 0ull : key[j];
    }
    if (lane == 0) wk[w][k] = wb;
  }
  if (tk.pmax) {  // the wave's largest slice maximum, for the log-sum-exp (published by the barrier below)
    float mloc = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) mloc = fmaxf(mloc, pm[j]);
    const float wm = wave_max_reg(mloc);
    if (lane == 0) fred[w] = wm;
  }
  __syncthreads();
  if (w == 0 && lane < 4 * K) {  // the k best slices (a slice is known by its best id: ids of slice s are s * 128 ..)
    const int lw = lane / K, lp = lane % K;
    const uint64_t x = wk[lw][lp];
    int rank = lp;
#pragma unroll
    for (int o = 1; o < 4; ++o) rank += keys_above(wk[(lw + o) & 3], K, x);
    if (rank < K && x != FILL) sel[rank] = pair_key_index(x) / TOPK_SLICE;
  }
  double sloc = 0.0, M = 0.0;
  if (tk.pmax) {  // this thread's share of the log-sum-exp
    const float mx = fmaxf(fmaxf(fred[0], fred[1]), fmaxf(fred[2], fred[3]));
    M = (double)mx / tk.temp;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (tid + 256 * j < ns) sloc += ps[j] * exp((double)pm[j] / tk.temp - M);
  }
  __syncthreads();
  // the chosen slices' k x k candidates, one per thread
  const int li = tid / K, lp = tid % K;
  const int sl = tid < K * K ? sel[li] : -1;
  float cval = -INFINITY;
  int cid = 0x7fffffff;
  if (sl >= 0) {
    cval = cv[(size_t)sl * K + lp];
    cid = ci[(size_t)sl * K + lp];
  }
  const uint64_t x = sl >= 0 ? pair_key(cval, cid) : 0ull;
  if (tid < K * K) gk[tid] = x;
  __syncthreads();
  if (sl >= 0) {
    int rank = lp;
    for (int o = 0; o < K; ++o)
      if (o != li) rank += keys_above(gk + o * K, K, x);
    if (rank < K) {
      const int id = kids.d2t ? (cid >= 0 && cid < kids.Vd ? kids.d2t[cid] : -1) : cid;
      out_ids[(size_t)r * K + rank] = id;
      out_vals[(size_t)r * K + rank] = cval;
      best[rank] = VI{cval, id};
    }
  }
  if (!tk.pmax) return;  // uniform: no log-sum-exp asked for
  const double sw = wave_sum_d_reg(sloc);
  if (lane == 0) dred[w] = sw;
  __syncthreads();
  if (tid == 0) {
    const double l = M + log(dred[0] + dred[1] + dred[2] + dred[3]);
    if (lse64) lse64[r] = l;
    if (lse32) lse32[r] = (float)l;
    if (kids.depth_new > 0) {  // the row's children: candidates of depth depth_new, log-prob value - (float)lse
      const TreeState& ts = kids.ts;
      const int k = ts.topk, dn = kids.depth_new;
      const int b = dn == 1 ? r : r / k, rank = dn == 1 ? 0 : r % k;
      const int c0 = (dn == 1 ? 0 : k + (dn - 2) * k * k) + rank * k;
      const int par = dn > 1 ? kpar : -1;
      const float ps0 = dn > 1 ? kps : 0.f;
      const float l32 = (float)l;
      for (int ch = 0; ch < k; ++ch) {
        const size_t o = (size_t)b * ts.cmax + c0 + ch;
        ts.tok[o] = best[ch].i;
        ts.par[o] = par;
        ts.dep[o] = dn;
        ts.score[o] = ps0 + (best[ch].v - l32);
        ts.erow[o] = -1;
      }
    }
  }
}

bool topk_merge_slices(int R, const SliceTopk& tk, int* out_ids, float* out_vals, float* lse32, double* lse64,
                       hipStream_t st, const TreeKids* kids) {
  if (R <= 0) return false;
  SliceTopk t = tk;
  if (!lse32 && !lse64) t.pmax = nullptr;
  TreeKids kd{};
  if (kids) kd = *kids;
  if (kd.depth_new > 0 && (!t.pmax || t.k != kd.ts.topk)) kd.depth_new = 0;  // children need the row's k and lse
  k_topk_merge_slices<<<R, 256, 0, st>>>(t, out_ids, out_vals, lse32, lse64, kd);
  return kd.depth_new > 0;
}

// -------------------------------------------------------------- row gather
__global__ void k_gather_rows_f32(float* __restrict__ dst, const float* __restrict__ src,
                                  const int* __restrict__ idx, int d) {
  const int r = blockIdx.x, s = idx[r];
  for (int i = threadIdx.x; i < d; i += blockDim.x) dst[(size_t)r * d + i] = s >= 0 ? src[(size_t)s * d + i] : 0.f;
}

void gather_rows_f32(float* dst, const float* src, const int* idx, int n, int d, hipStream_t st) {
  if (n <= 0) return;
  k_gather_rows_f32<<<n, 256, 0, st>>>(dst, src, idx, d);
}

}  // namespace e3
